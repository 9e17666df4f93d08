/*
 * scope.h - C ABI of the SCOPE sparse-attention hot path for video DiTs,
 * built for AMD Instinct MI355X (gfx950).
 *
 * Method: "SCOPE: Subspace Clustering with Online Per-Head Top-K Estimation
 * for Sparse Video Attention" (arXiv 2608.12780).  The abstract fixes the
 * pipeline (3D-RoPE-aligned key subspace clustering, LUT proxy scores,
 * hybrid Top-p with an online per-head Top-k, exact attention over the
 * selected original keys and values); the pith.science review of the paper
 * quotes Eq. (3), (6)-(10) and (27) and the hyper-parameters.
 *
 * One attention layer is split into two calls:
 *   scope_plan   - per (batch, head): 3D RoPE on Q/K; k-means of the queries
 *                  (Cq clusters) and of the key T/H/W channel subspaces (Cm
 *                  centroids each; Eq. (3)); lookup tables of query-centroid .
 *                  key-subspace-centroid dot products; proxy logits (Eq. (6));
 *                  Top-p counts t_c (Eq. (7)), base counts b_c (Eq. (8)),
 *                  k_head (Eq. (9)), final counts r_c (Eq. (10)) and the
 *                  selected key sets S_c.
 *   scope_attend - o_i = softmax over j in S_c(i) of <q'_i, k'_j>/sqrt(d),
 *                  times v_j, on the original post-RoPE keys and values.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers; the caller allocates and owns
 *     every buffer (the library never allocates, frees or keeps state).
 *   - Q, K, V, Q', K' and O are [B][H][N][d] contiguous, N = T*Hg*Wg, token
 *     n = (t*Hg + h)*Wg + w; element type per scope_params.dtype (bf16 as
 *     raw uint16 bit patterns, or fp32).  Base pointers must be 256-byte
 *     aligned.
 *   - Work is enqueued on `stream` (a hipStream_t); no call synchronises the
 *     host.  Results become visible in stream order.
 *   - Parameter errors are reported synchronously, before any launch.  No
 *     C++ exception crosses the ABI.  SCOPE_ERR_INVALID: a size below 1, an
 *     odd or non-positive channel range, d_t+d_h+d_w != d, Cq or Cm above N,
 *     iters outside 0..1000, rope_base <= 1, rho outside (0, 1], alpha
 *     outside [0, 1], an unknown dtype or flag, a null or misaligned pointer.
 *     SCOPE_ERR_UNSUPPORTED: d not in {64, 128}, N > 262144, Cq or Cm above
 *     1024, B*H > 65535, and in bf16 runs a centroid table larger than the
 *     160 KB LDS of a CU: ceil32(C) * (ceil16(d_m) + 8) * 2 + ceil32(C) * 4
 *     + 4096 bytes for any clustering (C = Cq with d_m = d for the queries,
 *     C = Cm with the subspace width, or d with SCOPE_FULL_DIM_KEYS, for the
 *     keys); at d = 128 that allows up to 576 centroids.
 *   - Calls that overlap in time must use distinct workspaces and plans.
 */
#ifndef SCOPE_H
#define SCOPE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SCOPE_OK = 0,
  SCOPE_ERR_INVALID = 1,      /* bad parameter, null or misaligned pointer */
  SCOPE_ERR_UNSUPPORTED = 2,  /* valid but not implemented (d not in {64, 128}) */
  SCOPE_ERR_WORKSPACE = 3,    /* workspace smaller than scope_workspace_size() */
  SCOPE_ERR_CAPACITY = 4,     /* plan buffer smaller than the sizes below */
  SCOPE_ERR_HIP = 5           /* a HIP launch or runtime call failed */
} scope_status;

typedef enum { SCOPE_F32 = 0, SCOPE_BF16 = 1 } scope_dtype;

/* scope_params.flags */
#define SCOPE_USE_INIT_CENTROIDS 0x1u /* start Lloyd from plan->q_centroids / k_centroids
                                         instead of seeded k-means++ */
#define SCOPE_PERMUTE_CHANNELS 0x2u   /* proxy subspaces from channel_perm instead of the
                                         3D-RoPE ranges (the partition ablation, Table 3 of
                                         the SCOPE paper's experiments): see channel_perm */
#define SCOPE_FIXED_TOPK_ONLY 0x4u    /* r_c = b_c (Eq. 8) for non-empty clusters: the hybrid
                                         Top-p / fixed Top-k selection without the online
                                         per-head Top-k extension of Eq. (10) (the Fig. 7
                                         ablation); k_head is still computed and written */
#define SCOPE_FULL_DIM_KEYS 0x10u     /* the cluster-level ablation proxy (forward implications of
                                         the SCOPE review: clustering whole key vectors instead of
                                         the 3D-RoPE subspaces): one key codebook of Cm centroids
                                         over all d channels (k-means++ draws of clustering 1), the
                                         proxy P[c][z_j] / sqrt(d) with a one-term table; the other
                                         two codes are 0 and their table rows zero.  Not with
                                         SCOPE_PERMUTE_CHANNELS or SCOPE_DENSE */
#define SCOPE_DENSE 0x8u              /* dense attention (the dense prefix of the SCOPE paper's
                                         schedule: the first layer at every step and the first
                                         denoising steps run dense): scope_plan applies RoPE and
                                         writes a plan in which every query attends to all N keys
                                         (cluster 0 holds all queries in token order, r_0 = t_0 =
                                         b_0 = k_head = N, S_0 = 0..N-1, the other clusters are
                                         empty); no k-means, scoring or selection runs, and the
                                         optional debug buffers are not written.  Not combinable
                                         with the other flags. */

typedef struct {
  int32_t B, H;            /* batch and heads; every (b, h) is independent; B*H <= 65535 */
  int32_t T, Hg, Wg;       /* latent grid; N = T*Hg*Wg tokens, N <= 262144 */
  int32_t d;               /* head dim, 64 or 128 */
  int32_t d_t, d_h, d_w;   /* 3D-RoPE channel ranges [T | H | W], each even, sum d */
  int32_t Cq;              /* query clusters, 1..N and at most 1024 */
  int32_t Cm;              /* centroids per key subspace (CT = CH = CW), 1..N and at most 1024 */
  int32_t iters;           /* Lloyd iterations after seeding, 0..1000 */
  double rope_base;        /* RoPE base, > 1 (10000) */
  double rho;              /* Top-p threshold of Eq. (7), 0 < rho <= 1 */
  double alpha;            /* fixed Top-k floor of Eq. (8) as a fraction of N, 0..1 */
  uint64_t seed;           /* k-means++ draws: SplitMix64 outputs */
  int32_t dtype;           /* scope_dtype */
  uint32_t flags;          /* SCOPE_USE_INIT_CENTROIDS | SCOPE_PERMUTE_CHANNELS | SCOPE_FIXED_TOPK_ONLY |
                              SCOPE_FULL_DIM_KEYS, or SCOPE_DENSE alone */
  /* With SCOPE_PERMUTE_CHANNELS: entries 0..d-1 are a permutation of
   * 0..d-1 (else SCOPE_ERR_INVALID); the query clustering, the three key
   * codebooks, the centroids and the LUT then work on the RoPE'd rows with
   * their channels in this order (position i holds channel channel_perm[i]),
   * so key subspace 0 is channels channel_perm[0 .. d_t), 1 the next d_h and
   * 2 the last d_w.  q_rope / k_rope and the attention are unchanged (a
   * common reordering of Q and K channels leaves every q.k); the workspace
   * then holds one reordered copy of q_rope and of k_rope.  Ignored without
   * the flag; entries d..127 are never read. */
  uint8_t channel_perm[128];
} scope_params;

/* Device buffers of one plan (all caller-allocated; sizes in elements).
 * Required by scope_plan and scope_attend: perm_q .. status.
 * Optional (may be NULL; when set, scope_plan writes the intermediate there,
 * and SCOPE_USE_INIT_CENTROIDS reads initial centroids from there):
 * q_centroids .. lut. */
typedef struct {
  int32_t* perm_q;       /* [B*H][N]: tokens grouped by query cluster, ascending inside a cluster */
  int32_t* q_off;        /* [B*H][Cq+1]: cluster c of head bh is perm_q[bh][q_off[c] .. q_off[c+1]) */
  int32_t* counts_t;     /* [B*H][Cq]: Top-p counts t_c (Eq. 7) */
  int32_t* counts_b;     /* [B*H][Cq]: base counts b_c = max(t_c, ceil(alpha*N)) (Eq. 8) */
  int32_t* counts_r;     /* [B*H][Cq]: final counts r_c (Eq. 10); 0 for empty clusters */
  int32_t* k_head;       /* [B*H]: ceil(sum n_c b_c / sum n_c) (Eq. 9) */
  int64_t* sel_off;      /* [B*H*Cq + 1]: CSR offsets into sel_idx, cluster-major over all heads */
  int32_t* sel_idx;      /* [sel_capacity]: key indices of S_c, ascending inside each cluster */
  int64_t sel_capacity;  /* elements of sel_idx; B*H*Cq*N always suffices */
  int32_t* work;         /* [2*work_capacity]: attention work items (built by scope_plan) */
  int64_t work_capacity; /* items; from scope_workspace_size */
  int32_t* status;       /* [4]: [0] work items, [1] set if sum r_c > sel_capacity,
                            [2] set if the workgroups that share one k-means++
                            clustering (large N, bf16) stopped waiting on each other
                            (not expected: they are launched cooperatively; the
                            plan's clusters are then not valid),
                            [3] bf16 runs: set if some element of q_rope / k_rope is
                            neither 0 nor of magnitude in [2^-47, 2^9); inside that
                            range the centroid sums of the Lloyd updates are exact
                            (the centroids are then the exact means rounded once to
                            fp32, independent of scheduling); outside it they are
                            ordinary fp64 sums (the plan is still valid) */
  float* q_centroids;    /* [B*H][Cq][d] final query centroids (fp32) */
  float* k_centroids;    /* [B*H][Cm][d] key centroids, row z = (mu^T_z | mu^H_z | mu^W_z)
                            (SCOPE_FULL_DIM_KEYS: mu_z over all d channels) */
  int32_t* q_labels;     /* [B*H][N] query cluster of each token */
  uint16_t* k_codes;     /* [B*H][N][4] (z^T, z^H, z^W, 0) key subspace codes */
  int32_t* seeds;        /* [B*H][4][max(Cq,Cm)] k-means++ centre indices (Q, T, H, W) */
  double* lut;           /* [B*H][Cq][3][Cm] lookup tables P^m[c][z] (fp64) */
  float* k_norm_max;     /* [B*H] optional: an upper bound of ||k'_j|| over the keys of each head,
                            written by scope_plan.  scope_attend uses it to bound the logits of a
                            query (|<q', k'>| <= ||q'|| ||k'||) and then drops the running maximum
                            of the online softmax when that bound is tight enough; NULL: the
                            maximum is always tracked.  It must belong to the k_rope that is
                            passed to scope_attend (scope_plan_finalize does not write it). */
} scope_plan_t;

/* Sizes for a parameter set: workspace bytes for scope_plan, the worst-case
 * sel_idx capacity (B*H*Cq*N) and the attention work-list capacity.
 * Any output pointer may be NULL.  Returns SCOPE_ERR_INVALID /
 * SCOPE_ERR_UNSUPPORTED for bad parameters. */
scope_status scope_workspace_size(const scope_params* p, size_t* ws_bytes,
                                  int64_t* sel_capacity_worst, int64_t* work_capacity);

/* Stages RoPE .. selection.  q, k: pre-RoPE [B][H][N][d]; q_rope, k_rope:
 * outputs of the same shape (the rotated Q'/K' that scope_attend reads).
 * ws: device workspace of at least scope_workspace_size() bytes, 256-byte
 * aligned; its contents are scratch.  If sum_c r_c exceeds
 * plan->sel_capacity, plan->status[1] is set on the device, sel_idx is left
 * incomplete and scope_attend skips every head. */
scope_status scope_plan(const scope_params* p, const void* q, const void* k, void* q_rope,
                        void* k_rope, scope_plan_t* plan, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* scope_plan, recording stage_events[i] (caller-created HIP events, i <
 * n_events, 1 <= n_events <= 5) on `stream` right after stage i has been
 * enqueued: 0 RoPE (S1), 1 k-means++ seeding (S2a), 2 Lloyd assignments and
 * centroid updates (S2b, S2c), 3 query-cluster permutation and lookup tables
 * (S3), 4 proxy scoring, Top-p, k_head, final selection and the attention work
 * list (S4, S5; scoring is fused into the selection passes).  An event
 * recorded before the call marks the start; elapsed times between the events
 * are the stage times.  Results are identical to scope_plan's.
 * SCOPE_ERR_INVALID also for a null event array or event, or n_events out of
 * range. */
scope_status scope_plan_timed(const scope_params* p, const void* q, const void* k, void* q_rope,
                              void* k_rope, scope_plan_t* plan, void* ws, size_t ws_bytes,
                              const hipEvent_t* stage_events, int n_events, hipStream_t stream);

/* scope_plan without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Its scratch memory is one fixed array of
 * SCOPE_NOALLOC_MAX_WORKSPACE bytes inside the library, one per GPU (each GPU
 * the library runs on holds it until the process ends); no call allocates or
 * frees memory.  Same arguments, results and errors as scope_plan, plus
 * SCOPE_ERR_WORKSPACE (before any launch) when scope_workspace_size() of the
 * parameters exceeds SCOPE_NOALLOC_MAX_WORKSPACE.  Every call on one GPU
 * shares that GPU's array, so calls that overlap in time on one GPU (other
 * streams, other threads) race and must not be issued; calls in stream order
 * are fine (each call initialises what it reads). */
#define SCOPE_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
scope_status scope_plan_noalloc(const scope_params* p, const void* q, const void* k, void* q_rope,
                                void* k_rope, scope_plan_t* plan, hipStream_t stream);

/* Rebuilds plan->work and plan->status[0] from perm_q/q_off/counts_r/sel_off
 * for a plan whose CSR was written by the caller (for instance copied from
 * another implementation).  scope_plan already does this. */
scope_status scope_plan_finalize(const scope_params* p, scope_plan_t* plan, hipStream_t stream);

/* Stage attention: out[bh][i] = sum_{j in S_c(i)} softmax_j(<q'_i, k'_j>/sqrt(d)) v[bh][j].
 * One kernel launch; needs no workspace. */
scope_status scope_attend(const scope_params* p, const scope_plan_t* plan, const void* q_rope,
                          const void* k_rope, const void* v, void* out, hipStream_t stream);

/* Static string for a status code. */
const char* scope_status_string(scope_status s);

#ifdef __cplusplus
}
#endif
#endif /* SCOPE_H */
