// Internal host/device interface of the SCOPE library: derived sizes, the
// workspace carve-up and the kernel launchers.  Not part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/scope.h"

namespace scope {

constexpr int ATT_BM = 128;     // queries per attention work item (fp32 storage; bf16 with d = 64: 4 waves x 32)
constexpr int ATT_BM128 = 256;  // queries per attention work item, bf16 with d = 128 (8 waves x 32)
constexpr int ATT_NW64 = 4;     // waves per attention workgroup, bf16 with d = 64
constexpr int ATT_NW128 = 8;    // waves per attention workgroup, bf16 with d = 128
constexpr int SEL_NB = 2048;    // histogram bins per level in the selection kernels
constexpr int SEL_CAP = 1024;   // boundary candidates sorted in LDS (more fall back to a walk over distinct logits)
constexpr int MAX_C = 1024;     // largest Cq / Cm supported
// per-clustering exchange area of the k-means++ kernel when one clustering
// spans several workgroups: counter, drawn index, 2 x 32 partial sums, MAX_C minima
constexpr int SEED_SYNC_BYTES = 8 + 2 * 8 * 32 + 4 * MAX_C;
constexpr size_t MAX_ASSIGN_LDS = 160 * 1024;   // LDS of one CU: holds a clustering's bf16 centroid table
constexpr int MAX_N = 1 << 18;  // largest token count supported (16 groups of 16 rounds of 1024)

// Geometry of the four clusterings of a head: 0 = queries (full d),
// 1..3 = key channel ranges T, H, W.
struct Geo {
  int BH, N, d, T, Hg, Wg;
  int Cq, Cm, iters;
  int off[4], dm[4], C[4], Cpad[4], dpad[4];   // channel offset / width, centroids, padded sizes per clustering
  int rdm[3];                   // 3D-RoPE channel ranges (d_t, d_h, d_w), whatever the clustering geometry
  int Cmax, CmaxPad, DPmax;
  int nk;                       // key clusterings: 3 (T, H, W subspaces) or 1 (all d channels,
                                // SCOPE_FULL_DIM_KEYS); clusterings 0 .. nk are active
  int bf16;                     // 1: bf16 storage, 0: fp32
  int permute;                  // 1: clustering on channel-reordered copies of q_rope / k_rope
  int online_khead;             // 1: r_c = max(b_c, k_head) (Eq. 10); 0: r_c = b_c
  uint64_t seed;
};

// Channel order of the proxy subspaces (kernel argument of the reordering kernel).
struct ChanPerm {
  uint8_t p[128];
};

// Per-cluster state of the selection kernels.
struct ClusterSel {
  double smax, smin, scale1;    // proxy-logit range and level-1 bin scale
  double tau;                   // logit at the Top-p boundary
  int32_t m;                    // keys with logit == tau that are taken (lowest indices)
  int32_t t;                    // Top-p count t_c
  int32_t all;                  // 1: every key selected
  int32_t pad;
  uint64_t zfx;                 // fixed-point softmax mass of all keys
  double pad2;
};

struct Workspace {
  double2* rope_tab;            // cos/sin per (range, position, pair)
  int rope_off[3];
  double* d2;                   // [BH][4][N] k-means++ squared distance to the nearest centre
  int32_t* nearest;             // [BH][4][N] uint16: index of that centre (bit 15: point is a centre)
  int32_t* seeds;               // [BH][4][Cmax]
  float* qcent;                 // [BH][Cq][d]
  float* kcent;                 // [BH][Cm][d]
  uint16_t* cbf;                // [BH][4][CmaxPad][DPmax] bf16 centroids, zero padded
  float* cnorm;                 // [BH][4][CmaxPad] ||bf16 centroid||^2 (FLT_MAX on padding)
  int32_t* labels;              // [BH][4][N] (labels of the last assignment)
  int32_t* labels_alt;          // [BH][4][N] (assignments alternate between the two arrays)
  double* psum;                 // [BH][4][acc_slices][acc_parts][Cmax][acc_sw] partial centroid sums
  int32_t* pcnt;                // [BH][4][acc_parts][Cmax] partial cluster sizes
  double* stot;                 // [BH][4][Cmax][d] per-cluster sums of the values of magnitude >= 2^-19
  double* ssm;                  // [BH][4][Cmax][d] per-cluster sums of the smaller nonzero values (bf16 data)
  int32_t* ntot;                // [BH][4][Cmax] cluster sizes of the last update
  uint16_t* codes;              // [BH][N][4]
  int32_t* qlab;                // [BH][N] (final query labels)
  double* lut;                  // [BH][Cq][3][Cm]
  ClusterSel* csel;             // [BH][Cq]
  int64_t* htot;                // [BH] per-head total of r_c, then the head's offset in sel_idx
  int32_t* hist1;               // [BH][Cq][SEL_NB] level-1 key counts of the Top-p pass (reused by the final selection)
  char* seed_sync;              // [BH][4] k-means++ exchange areas (SEED_SYNC_BYTES) when a clustering spans workgroups
  int4* amb;                    // [BH * 4 * N] near-tie points of one Lloyd assignment: (bh * 4 + m, point, block marks)
  int32_t* amb_cnt;             // [iters + 1] entries of amb per assignment (zeroed before the first)
  void* qperm;                  // [BH][N][d] q_rope with reordered channels (SCOPE_PERMUTE_CHANNELS only)
  void* kperm;                  // [BH][N][d] k_rope likewise
  size_t bytes;
};

// Queries per attention work item (every kernel: 128).
inline int att_chunk(const Geo& g) { return g.bf16 && g.d == 128 ? ATT_BM128 : ATT_BM; }
// Lloyd update layout: channel slices of acc_sw channels, acc_parts point
// ranges per (head, clustering).  Slices are 32 channels wide unless the
// per-cluster sums of that width (Cmax x 32 fp64 plus the counts, beside the
// 16 KB of lists of the delta update) would not fit in the 160 KB LDS.
inline int acc_sw(const Geo& g) { return g.Cmax <= 544 ? 32 : 16; }
inline int acc_slices(const Geo& g) { return (g.d + acc_sw(g) - 1) / acc_sw(g); }
inline int acc_parts(const Geo& g) {
  const int p = (g.N + 4095) / 4096;
  return p < 1 ? 1 : (p > 8 ? 8 : p);
}

// Elements of the small-value centroid sums (Workspace::ssm).
inline size_t ssm_elems(const Geo& g) { return (size_t)g.BH * 4 * g.Cmax * g.d; }

Geo make_geo(const scope_params& p);
// Lays the workspace out from `base` (nullptr: only computes .bytes).
Workspace carve(const Geo& g, const scope_plan_t* plan, char* base);

// ---- launchers (return hipGetLastError()) ---------------------------------
hipError_t launch_rope(const Geo& g, const scope_params& p, const void* q, const void* k, void* qo,
                       void* ko, const Workspace& w, float* k_norm_max, int32_t* range_flag, hipStream_t s);
hipError_t launch_permute(const Geo& g, const ChanPerm& perm, const void* qr, const void* kr, const Workspace& w,
                          hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s);
hipError_t launch_seed(const Geo& g, const void* qr, const void* kr, const Workspace& w, int32_t* status,
                       hipStream_t s);
hipError_t launch_prep(const Geo& g, const Workspace& w, hipStream_t s);
hipError_t launch_assign(const Geo& g, const void* qr, const void* kr, const Workspace& w, int iter,
                         hipStream_t s);
// Lloyd update `it` (1 .. iters) from the labels of assignment it - 1.
hipError_t launch_update(const Geo& g, const void* qr, const void* kr, const Workspace& w, int it, hipStream_t s);
hipError_t launch_pack(const Geo& g, const Workspace& w, int32_t* q_labels_out, hipStream_t s);
hipError_t launch_perm(const Geo& g, const Workspace& w, int32_t* perm_q, int32_t* q_off, hipStream_t s);
hipError_t launch_lut(const Geo& g, const Workspace& w, hipStream_t s);
hipError_t launch_topp(const Geo& g, const scope_params& p, const Workspace& w, int32_t* ct, int32_t* cb,
                       hipStream_t s);
hipError_t launch_khead(const Geo& g, const scope_plan_t& plan, const Workspace& w, hipStream_t s);
hipError_t launch_final_select(const Geo& g, const scope_params& p, const Workspace& w,
                               const scope_plan_t& plan, hipStream_t s);
hipError_t launch_worklist(const Geo& g, const scope_plan_t& plan, hipStream_t s);
// The plan of dense attention (SCOPE_DENSE): cluster 0 holds every query and all N keys.
hipError_t launch_dense_plan(const Geo& g, const scope_plan_t& plan, hipStream_t s);
hipError_t launch_attend(const Geo& g, const scope_plan_t& plan, const void* qr, const void* kr,
                         const void* v, void* out, hipStream_t s);

}  // namespace scope
