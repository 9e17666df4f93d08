// Stage 2: k-means of the post-RoPE queries (Cq clusters, full d) and of the
// post-RoPE keys restricted to each 3D-RoPE channel range T, H, W (Cm
// centroids each), the per-subspace clustering of SCOPE's Eq. (3) (Euclidean
// reconstruction objective; pith.science review of arXiv 2608.12780).
// Procedure: seeded k-means++ followed by Lloyd rounds
//   labels_0 = assign(init); for it in 1..iters: mu = mean(labels); labels = assign(mu).
//
// Reproducibility.  The centroid sums of bf16 data are exact (split by
// magnitude, see accum_kernel), so the order of their atomics does not matter
// and each mean is the exact sum / n rounded once.  The k-means++ squared
// distances and their running sums are ordinary fp64 arithmetic evaluated in
// a fixed order (no floating-point atomics), so every run gives the same
// draws; a draw can differ from an index-order scan in exact arithmetic only
// where the target lies within the sums' rounding error of a running-sum
// boundary (a near tie).  The MFMA assignment is a filter whose near-ties are
// re-decided with fp64 distances.
#include <float.h>
#include <type_traits>

#include "scope_device.hpp"
#include "scope_internal.hpp"

namespace scope {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int CENTRE_MARK = 1 << 30;   // `nearest` bit: the point is a chosen centre

template <typename T>
__device__ __forceinline__ double sqdist_row(const T* __restrict__ x, const double* __restrict__ c, int dm) {
  double acc = 0.0;
  for (int ch = 0; ch < dm; ++ch) {
    const double df = Elem<T>::ld(x + ch) - c[ch];
    acc += df * df;
  }
  return acc;
}

// ---------------------------------------------------------------------------
// k-means++ seeding (Arthur and Vassilvitskii 2007): one workgroup of 1024
// threads per (head, clustering).  Centre 0 = floor(u_0 N); centre s = the
// smallest i whose running sum of D^2 (index order) exceeds u_s * sum(D^2),
// D^2 being the squared distance to the nearest centre chosen so far (fp64,
// summed in a fixed order).
// The points form groups of 8192; inside a group, wave w owns the 512
// consecutive points starting at 512 w, one 64-point round per step of its
// 8 rounds (lane = point mod 64).  So (group, wave, round, lane) is the index
// order, and the running sum is taken over (group, wave) sums, then over the
// rounds of the crossing (group, wave), then over its lanes.
// The D^2 update skips a point whose current centre a has
// ||c_s - a||^2 >= 4 D^2 (triangle inequality, Elkan ICML 2003): then
// ||x - c_s|| >= D(x), so the result equals the unpruned update.  Each wave
// compacts the points that still need a distance into an LDS list and
// computes it with all 64 lanes, so the work is balanced across lanes.
// State: with RESIDENT, one group covers every point and D^2 / the nearest
// centre id stay in registers across steps; otherwise every group is loaded
// from and written back to global memory each step (coalesced).
// Points beyond N carry D^2 = 0 and the centre mark, so they are never drawn.
// ---------------------------------------------------------------------------
constexpr int SEED_NT = 1024;
constexpr int SEED_NW = SEED_NT / 64;
constexpr int SEED_RG = 8;                 // rounds per group
constexpr int SEED_MAX_GROUPS = 32;        // N <= 2^18
constexpr int SEED_LIST = 512;             // list entries per wave
// the chosen centres' rows are kept in LDS when they fit beside the lists and
// the kernel's static arrays (cvec, cvs, cc, chosen, wsum, gscr, scalars)
constexpr int SEED_CACHE_BYTES = 40 * 1024;
constexpr int SEED_STATIC_LDS = 8 * 128 + 8 * 136 + 12 * MAX_C + 8 * SEED_MAX_GROUPS * (SEED_NT / 64) +
                                8 * SEED_RG * 64 + 64;
static_assert((SEED_NT / 64) * SEED_LIST * 12 + SEED_CACHE_BYTES + SEED_STATIC_LDS <= 160 * 1024,
              "k-means++ LDS of one workgroup");
constexpr uint32_t NR_MARK = 0x8000u;      // point is a chosen centre
constexpr uint32_t NR_ID = 0x7FFFu;

template <typename T>
__device__ __forceinline__ double sqdist_g(const T* __restrict__ x, const double* __restrict__ c, int dm);
template <>
__device__ __forceinline__ double sqdist_g<uint16_t>(const uint16_t* __restrict__ x, const double* __restrict__ c,
                                                      int dm) {
  // dm even and x 4-byte aligned: channel pairs
  double acc = 0.0;
  const uint32_t* x2 = reinterpret_cast<const uint32_t*>(x);
#pragma unroll 8
  for (int i = 0; i < dm / 2; ++i) {
    const uint32_t u = x2[i];
    const double d0 = (double)__uint_as_float(u << 16) - c[2 * i];
    const double d1 = (double)__uint_as_float(u & 0xFFFF0000u) - c[2 * i + 1];
    acc = fma(d0, d0, acc);
    acc = fma(d1, d1, acc);
  }
  return acc;
}
template <>
__device__ __forceinline__ double sqdist_g<float>(const float* __restrict__ x, const double* __restrict__ c, int dm) {
  double acc = 0.0;
#pragma unroll 8
  for (int i = 0; i < dm; ++i) {
    const double df = (double)x[i] - c[i];
    acc = fma(df, df, acc);
  }
  return acc;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Exchange area of one clustering when W workgroups share its points
// (SeedSync::W[m] > 1, a cooperative launch: all of them are resident at once).
// Each workgroup owns a contiguous run of groups; per draw it publishes the
// sum of its D^2, waits for the others, and the workgroup holding the
// crossing publishes the drawn index, tagged with the draw, which the others
// poll for.
static_assert(SEED_SYNC_BYTES == 8 + 2 * 8 * SEED_MAX_GROUPS + 4 * MAX_C, "exchange area layout");
constexpr uint32_t SEED_SPIN_LIMIT = 1u << 18;   // polls before giving up: well over a second, far above one draw
struct SeedSync {
  char* base;        // [BH][4] areas of SEED_SYNC_BYTES: counter, drawn index, part[2][32], lowest[MAX_C]
  int32_t* abort;    // set when a wait ran out (every later wait is then skipped)
  int W[4];          // workgroups per clustering m of a head (all 1: no exchange)
  int flat;          // 1: blockIdx.x enumerates the nbh*W[0] query workgroups, then per head
                     // the W[1] + .. + W[nk] key workgroups (m ascending), heads bh0 ..
                     // bh0+nbh-1; 0: grid (BH, 1+nk) with one each
  int bh0, nbh;      // heads of this launch (flat)
};

// (m, head, workgroup within the clustering) of this workgroup
__device__ __forceinline__ void seed_block(const SeedSync& sy, int nk, int& m, int& bh, int& wg) {
  m = blockIdx.y; bh = blockIdx.x; wg = 0;
  if (!sy.flat) return;
  const int b = blockIdx.x, w0 = sy.W[0], nq = sy.nbh * w0;
  if (b < nq) {
    m = 0; bh = b / w0; wg = b - bh * w0;
  } else {
    const int w1 = sy.W[1], w2 = nk >= 2 ? sy.W[2] : 0, w3 = nk >= 3 ? sy.W[3] : 0;
    const int kw = w1 + w2 + w3, r0 = b - nq;
    bh = r0 / kw;
    const int r = r0 - bh * kw;
    m = r < w1 ? 1 : (r < w1 + w2 ? 2 : 3);
    wg = r - (m == 1 ? 0 : (m == 2 ? w1 : w1 + w2));
  }
  bh += sy.bh0;
}

__global__ void seed_sync_init_kernel(char* base, int chains, int32_t* abort) {
  const int c = blockIdx.x;
  int32_t* a = reinterpret_cast<int32_t*>(base + (size_t)c * SEED_SYNC_BYTES);
  int32_t* lo = reinterpret_cast<int32_t*>(base + (size_t)c * SEED_SYNC_BYTES + 8 + 2 * 8 * SEED_MAX_GROUPS);
  if (threadIdx.x == 0) { a[0] = 0; a[1] = 0; }
  for (int i = threadIdx.x; i < MAX_C; i += blockDim.x) lo[i] = 0x7FFFFFFF;
  if (c == 0 && threadIdx.x == 0) *abort = 0;
}

template <typename T, bool RESIDENT>
__global__ __launch_bounds__(SEED_NT) void seed_kernel(const T* __restrict__ qr, const T* __restrict__ kr, Geo g,
                                                       double* __restrict__ d2all, uint16_t* __restrict__ nearall,
                                                       int32_t* __restrict__ seeds, float* __restrict__ qcent,
                                                       float* __restrict__ kcent, SeedSync sy) {
  int m, bh, wg;
  seed_block(sy, g.nk, m, bh, wg);
  const int W = m == 0 ? sy.W[0] : (m == 1 ? sy.W[1] : (m == 2 ? sy.W[2] : sy.W[3]));
  const int N = g.N, d = g.d, dm = g.dm[m], off = g.off[m], C = g.C[m];
  const T* X = (m == 0 ? qr : kr) + (size_t)bh * N * d + off;
  double* D2g = d2all + ((size_t)bh * 4 + m) * N;
  uint16_t* NRg = nearall + ((size_t)bh * 4 + m) * N;
  int32_t* sd = seeds + ((size_t)bh * 4 + m) * g.Cmax;

  __shared__ double cvec[128];
  __shared__ double cvs[136];   // centre row shifted right by sh channels, zero outside the subspace
  __shared__ double cc[MAX_C];
  __shared__ int32_t chosen[MAX_C];
  __shared__ double wsum[SEED_MAX_GROUPS * SEED_NW];
  __shared__ double gscr[SEED_RG * 64];
  __shared__ double sh_excl, sh_target;
  __shared__ int32_t sh_grp, sh_wave, sh_mode, sh_lo, sh_hi, sh_own, sh_ci;
  extern __shared__ __align__(16) unsigned char seed_smem[];
  int32_t* lp = reinterpret_cast<int32_t*>(seed_smem) + (threadIdx.x >> 6) * SEED_LIST;
  double* ldist = reinterpret_cast<double*>(seed_smem + SEED_NW * SEED_LIST * 4) + (threadIdx.x >> 6) * SEED_LIST;
  T* cache = reinterpret_cast<T*>(seed_smem + SEED_NW * SEED_LIST * 12);   // chosen centres [C][cld]
  const int cld = dm + 2;   // padded row: consecutive rows start in different LDS banks
  const bool cached = (size_t)C * cld * sizeof(T) <= SEED_CACHE_BYTES;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int R = (N + SEED_NT - 1) / SEED_NT;
  const int G = (R + SEED_RG - 1) / SEED_RG;
  // 16-byte row loads: the aligned 8-channel pieces that cover the subspace,
  // starting sh = off mod 8 channels before it (even: RoPE pairs), all inside
  // the row.  Channel pair j of piece p is subspace channel 8 p + 2 j - sh;
  // pairs outside 0 .. dm - 1 are zeroed in the loaded word and meet a zero
  // in cvs, so they add exact zeros and the loop needs no per-channel branch.
  const int sh = off & 7;
  const bool vec16 = sizeof(T) == 2 && ((d * 2) % 16 == 0) && (sh % 2 == 0) && (dm % 2 == 0) &&
                     off - sh + ((dm + sh + 7) & ~7) <= d;
  int lpr = 1;   // lanes per row: power of two covering ceil((dm + sh) / 8) 16-byte pieces
  while (lpr * 8 < dm + sh) lpr <<= 1;
  const uint64_t stream = ((uint64_t)bh * 4 + m) << 20;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  // point of round k of the group starting at round r0 held by this thread:
  // each wave owns SEED_RG*64 consecutive points of its group, so the order
  // (group, wave, round, lane) is the index order
  auto pidx = [&](int r0, int k) -> int { return r0 * SEED_NT + wv * (SEED_RG * 64) + k * 64 + lane; };

  // group state: D^2 and packed 16-bit centre ids of this thread's 8 points of the group
  double gd2[SEED_RG];
  uint32_t gnr[SEED_RG / 2];
  auto nr_get = [&](int k) -> uint32_t { return (gnr[k >> 1] >> (16 * (k & 1))) & 0xFFFFu; };
  auto nr_set = [&](int k, uint32_t v) {
    gnr[k >> 1] = (gnr[k >> 1] & ~(0xFFFFu << (16 * (k & 1)))) | (v << (16 * (k & 1)));
  };
  auto valid_mask = [&](int r0) {
    uint32_t vm = 0;
    for (int k = 0; k < SEED_RG; ++k) vm |= (uint32_t)(pidx(r0, k) < N) << k;
    return vm;
  };
  auto load_group = [&](int r0, uint32_t vm) {
#pragma unroll
    for (int k = 0; k < SEED_RG; ++k) {
      const int p = pidx(r0, k);
      const bool ok = (vm >> k) & 1u;
      gd2[k] = ok ? D2g[p] : 0.0;
      nr_set(k, ok ? (uint32_t)NRg[p] : NR_MARK);
    }
  };
#pragma unroll
  for (int k = 0; k < SEED_RG; ++k) { gd2[k] = 0.0; nr_set(k, NR_MARK); }

  // this workgroup's groups [gi0, gi1) of the clustering
  const int gi0 = (int)((int64_t)wg * G / W), gi1 = (int)((int64_t)(wg + 1) * G / W);
  char* xs = sy.base + ((size_t)bh * 4 + m) * SEED_SYNC_BYTES;
  int32_t* x_ctr = reinterpret_cast<int32_t*>(xs);
  int32_t* x_ci = x_ctr + 1;
  unsigned long long* x_part = reinterpret_cast<unsigned long long*>(xs + 8);
  // partial sums by draw parity: a workgroup may publish draw s + 1's while a
  // slower one still reads draw s's (it cannot get two draws ahead)
  int32_t* x_lo = reinterpret_cast<int32_t*>(xs + 8 + 2 * 8 * SEED_MAX_GROUPS);
  // the crossing wave (ww) of group gg: rounds of its group, then lanes of
  // the crossing round; sh_excl is the sum of D^2 before the wave's points
  auto cross_wave = [&](int gg, int ww) __attribute__((always_inline)) {
    const int r0 = gg * SEED_RG;
    if (RESIDENT) {
#pragma unroll
      for (int k = 0; k < SEED_RG; ++k) gscr[k * 64 + lane] = gd2[k];
    } else {
      for (int k = 0; k < SEED_RG; ++k) {
        const int p = pidx(r0, k);
        gscr[k * 64 + lane] = p < N ? D2g[p] : 0.0;
      }
    }
    wave_sync_lds();
    double excl = sh_excl;
    const double target = sh_target;
    int ksel = -1, klast = -1;
    for (int k = 0; k < SEED_RG; ++k) {
      const double rs = wave_sum_dpp(gscr[k * 64 + lane]);
      if (rs > 0.0) klast = k;
      if (ksel < 0) { if (excl + rs > target) ksel = k; else excl += rs; }
    }
    if (ksel < 0) ksel = klast;   // rounding: the group's last round with weight
    const double v = gscr[ksel * 64 + lane];
    const double inc = excl + wave_incl_scan(v);
    const uint64_t hit = __ballot(inc > target);
    const uint64_t pos = __ballot(v > 0.0);
    const int L = hit ? __ffsll((unsigned long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
    if (lane == 0) sh_lo = r0 * SEED_NT + ww * (SEED_RG * 64) + ksel * 64 + L;
    wave_sync_lds();
  };
  int nwait = 0;
  // every workgroup of the clustering reaches this point (bounded polling).
  // heavy: a device-wide fence on both sides (data written by any thread);
  // light: only thread 0's own agent-scope atomic stores are published
  // (waited for before the counter moves), so no cache write-back is needed.
  auto chain_wait = [&](bool heavy) __attribute__((always_inline)) {
    __syncthreads();
    ++nwait;
    if (tid == 0) {
      if (heavy) __threadfence();
      else __builtin_amdgcn_s_waitcnt(0);
      atomicAdd(x_ctr, 1);
      const int want = W * nwait;
      uint32_t spins = 0;
      while (__hip_atomic_load(x_ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want) {
        if (__hip_atomic_load(sy.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
        if (++spins > SEED_SPIN_LIMIT) { atomicExch(sy.abort, 1); break; }
        __builtin_amdgcn_s_sleep(2);
      }
      if (heavy) __threadfence();
    }
    __syncthreads();
  };
  // the drawn index of draw s, published by its owner as (s << 20) | index
  auto wait_ci = [&](int s) __attribute__((always_inline)) -> int {
    if (tid == 0) {
      uint32_t spins = 0;
      int v = __hip_atomic_load(x_ci, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      while ((v >> 20) != s) {
        if (__hip_atomic_load(sy.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
        if (++spins > SEED_SPIN_LIMIT) { atomicExch(sy.abort, 1); break; }
        __builtin_amdgcn_s_sleep(1);
        v = __hip_atomic_load(x_ci, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      sh_ci = v & 0xFFFFF;
    }
    __syncthreads();
    return sh_ci;
  };
  int ci = 0;
  for (int s = 0; s < C; ++s) {
    // ---- centre s ----------------------------------------------------------------
    if (s == 0) {
      const uint64_t k0 = splitmix64(g.seed, stream) >> 11;
      const uint64_t lo = k0 * (uint64_t)N, hi = __umul64hi(k0, (uint64_t)N);
      ci = (int)((hi << 11) | (lo >> 53));
    } else if (W > 1) {
      // ---- the workgroups of the clustering together ----------------------------
      if (wv == 0) {
        const int n0 = gi0 * SEED_NW, n1 = gi1 * SEED_NW;
        double run = 0.0;
        for (int c0 = n0; c0 < n1; c0 += 64) {
          const double v = c0 + lane < n1 ? wsum[c0 + lane] : 0.0;
          run += __shfl(wave_incl_scan(v), 63);
        }
        if (lane == 0)
          __hip_atomic_store(x_part + (s & 1) * SEED_MAX_GROUPS + wg, (unsigned long long)__double_as_longlong(run),
                             __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      chain_wait(false);
      if (wv == 0) {
        // every workgroup: the same sums in the same order, so the same owner
        const double v = lane < W ? __longlong_as_double((long long)__hip_atomic_load(
                                        x_part + (s & 1) * SEED_MAX_GROUPS + lane, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT))
                                  : 0.0;
        const double inc = wave_incl_scan(v);
        const double total = __shfl(inc, 63);
        int mode = 2, owner = 0;
        double excl = 0.0, target = 0.0;
        if (total > 0.0) {
          const uint64_t ku = splitmix64(g.seed, stream + (uint64_t)s) >> 11;
          target = ((double)ku * 0x1p-53) * total;
          const uint64_t hit = __ballot(lane < W && inc > target);
          if (hit) {
            mode = 0;
            owner = __ffsll((unsigned long long)hit) - 1;
            excl = __shfl(inc - v, owner);
          } else {
            mode = 1;
            const uint64_t pos = __ballot(lane < W && v > 0.0);
            owner = 63 - __clzll((long long)pos);
          }
        }
        int gg = -1, ww = -1;
        if (mode == 0 && wg == owner) {
          // the owner walks its (group, wave) sums from the sum before it
          const int n0 = gi0 * SEED_NW, n1 = gi1 * SEED_NW;
          double run = excl;
          for (int c0 = n0; c0 < n1; c0 += 64) {
            const bool in = c0 + lane < n1;
            const double u = in ? wsum[c0 + lane] : 0.0;
            const double ic = wave_incl_scan(u);
            const uint64_t h = __ballot(in && run + ic > target);
            if (h) {
              const int L = __ffsll((unsigned long long)h) - 1;
              const double prev = __shfl(ic, L > 0 ? L - 1 : 0);
              excl = run + (L > 0 ? prev : 0.0);
              gg = (c0 + L) / SEED_NW;
              ww = (c0 + L) % SEED_NW;
              break;
            }
            run += __shfl(ic, 63);
          }
          if (gg < 0) { gg = gi1 - 1; ww = SEED_NW - 1; }   // not reached: the owner's sums cross
        }
        if (lane == 0) {
          sh_grp = gg; sh_wave = ww; sh_excl = excl; sh_target = target;
          sh_mode = mode; sh_own = owner;
          sh_lo = 0x7FFFFFFF; sh_hi = -1;
        }
      }
      __syncthreads();
      const int mode = sh_mode, owner = sh_own;
      if (mode == 2) {
        for (int gi = gi0; gi < gi1; ++gi) {
          const int r0 = gi * SEED_RG;
          const uint32_t vm = valid_mask(r0);
          if (!RESIDENT) load_group(r0, vm);
          uint32_t free_ = 0;
#pragma unroll
          for (int k = 0; k < SEED_RG; ++k) free_ |= (uint32_t)!(nr_get(k) & NR_MARK) << k;
          free_ &= vm;
          if (free_) {
            atomicMin(x_lo + s, pidx(r0, __ffs(free_) - 1));
            __builtin_amdgcn_s_waitcnt(0);   // performed before the wait below publishes it
            break;
          }
        }
      } else if (wg == owner) {
        if (mode == 1) {
          for (int gi = gi1 - 1; gi >= gi0; --gi) {
            const int r0 = gi * SEED_RG;
            const uint32_t vm = valid_mask(r0);
            if (!RESIDENT) load_group(r0, vm);
            uint32_t posm = 0;
#pragma unroll
            for (int k = 0; k < SEED_RG; ++k) posm |= (uint32_t)(gd2[k] > 0.0) << k;
            posm &= vm;
            if (posm) { atomicMax(&sh_hi, pidx(r0, 31 - __clz(posm))); break; }
          }
        } else if (wv == sh_wave) {
          cross_wave(sh_grp, sh_wave);
        }
        __syncthreads();
        if (tid == 0) {
          const int own = sh_lo != 0x7FFFFFFF ? sh_lo : sh_hi;
          __hip_atomic_store(x_ci, (s << 20) | (own & 0xFFFFF), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (mode == 2) {
        chain_wait(true);
        ci = __hip_atomic_load(x_lo + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        ci = wait_ci(s);
      }
      if (ci < 0 || ci >= N) ci = 0;
    } else {
      if (wv == 0) {
        // wave 0 walks the (group, wave) sums in index order
        const int n = G * SEED_NW;
        double run = 0.0;
        for (int c0 = 0; c0 < n; c0 += 64) {
          const double v = c0 + lane < n ? wsum[c0 + lane] : 0.0;
          run += __shfl(wave_incl_scan(v), 63);
        }
        const double total = run;
        int gg = -1, ww = -1;
        double excl = 0.0, target = 0.0;
        if (total > 0.0) {
          const uint64_t ku = splitmix64(g.seed, stream + (uint64_t)s) >> 11;
          target = ((double)ku * 0x1p-53) * total;
          run = 0.0;
          for (int c0 = 0; c0 < n; c0 += 64) {
            const bool in = c0 + lane < n;
            const double v = in ? wsum[c0 + lane] : 0.0;
            const double inc = wave_incl_scan(v);
            const uint64_t hit = __ballot(in && run + inc > target);
            if (hit) {
              const int L = __ffsll((unsigned long long)hit) - 1;
              const double prev = __shfl(inc, L > 0 ? L - 1 : 0);
              excl = run + (L > 0 ? prev : 0.0);
              gg = (c0 + L) / SEED_NW;
              ww = (c0 + L) % SEED_NW;
              break;
            }
            run += __shfl(inc, 63);
          }
        }
        if (lane == 0) {
          sh_grp = gg; sh_wave = ww; sh_excl = excl; sh_target = target;
          sh_mode = total > 0.0 ? (gg >= 0 ? 0 : 1) : 2;   // 0 draw, 1 rounding at the end, 2 all zero
          sh_lo = 0x7FFFFFFF; sh_hi = -1;
        }
      }
      __syncthreads();
      const int gg = sh_grp, ww = sh_wave, mode = sh_mode;
      if (mode == 2) {
        // every remaining point coincides with a centre: lowest index not chosen yet
        for (int gi = 0; gi < G; ++gi) {
          const int r0 = gi * SEED_RG;
          const uint32_t vm = valid_mask(r0);
          if (!RESIDENT) load_group(r0, vm);
          uint32_t free_ = 0;
#pragma unroll
          for (int k = 0; k < SEED_RG; ++k) free_ |= (uint32_t)!(nr_get(k) & NR_MARK) << k;
          free_ &= vm;
          if (free_) { atomicMin(&sh_lo, pidx(r0, __ffs(free_) - 1)); break; }
        }
      } else if (mode == 1) {
        // rounding left the target at the very end: the last point with positive weight
        for (int gi = G - 1; gi >= 0; --gi) {
          const int r0 = gi * SEED_RG;
          const uint32_t vm = valid_mask(r0);
          if (!RESIDENT) load_group(r0, vm);
          uint32_t posm = 0;
#pragma unroll
          for (int k = 0; k < SEED_RG; ++k) posm |= (uint32_t)(gd2[k] > 0.0) << k;
          posm &= vm;
          if (posm) { atomicMax(&sh_hi, pidx(r0, 31 - __clz(posm))); break; }
        }
      } else if (wv == ww) {
        cross_wave(gg, ww);
      }
      __syncthreads();
      ci = sh_lo != 0x7FFFFFFF ? sh_lo : sh_hi;
      if (ci < 0 || ci >= N) ci = 0;
    }
    // ---- centre vector, cache row and distances to the previous centres -----------
    if (tid == 0) { chosen[s] = ci; if (wg == 0) sd[s] = ci; }
    if (tid < dm) {
      const T xv = X[(size_t)ci * d + tid];
      cvec[tid] = Elem<T>::ld(&xv);
      if (cached) cache[(size_t)s * cld + tid] = xv;
    }
    if (tid < 136) {
      const int ch = tid - sh;
      cvs[tid] = ch >= 0 && ch < dm ? Elem<T>::ld(X + (size_t)ci * d + ch) : 0.0;
    }
    __syncthreads();
    for (int a = tid; a < s; a += SEED_NT) {
      double acc = 0.0;
      if (cached) {
        const T* row = cache + (size_t)a * cld;
        for (int ch = 0; ch < dm; ++ch) { const double df = Elem<T>::ld(row + ch) - cvec[ch]; acc = fma(df, df, acc); }
      } else {
        acc = sqdist_g<T>(X + (size_t)chosen[a] * d, cvec, dm);
      }
      cc[a] = acc;
    }
    __syncthreads();
    // ---- D^2 update, group by group; (group, wave) sums for the next draw ----------
    for (int gi = gi0; gi < gi1; ++gi) {
      const int r0 = gi * SEED_RG;
      const uint32_t vm = valid_mask(r0);
      if (!RESIDENT) {
        if (s > 0) {
          load_group(r0, vm);
        } else {
          // first pass: no stored state yet; points past N must not keep the
          // previous group's values (they enter the wave sums below)
#pragma unroll
          for (int k = 0; k < SEED_RG; ++k) { gd2[k] = 0.0; nr_set(k, NR_MARK); }
        }
      }
      uint32_t mask = vm;
      if (s > 0) {
        mask = 0;   // points past N carry D^2 = 0, so the test prunes them
#pragma unroll
        for (int k = 0; k < SEED_RG; ++k)
          mask |= (uint32_t)!(cc[nr_get(k) & NR_ID] * (1.0 - 1e-9) >= 4.0 * gd2[k]) << k;
      }
      uint32_t chg = 0;
      // wave-wide compaction: lane offsets by an exclusive scan of the popcounts
      const int cnt = __popc(mask);
      int incl_c = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) { const int u = __shfl_up(incl_c, o, 64); if (lane >= o) incl_c += u; }
      const int offs = incl_c - cnt, total = __shfl(incl_c, 63, 64);
      for (int base = 0; base < total; base += SEED_LIST) {
        uint32_t mm = mask;
        int kk = offs;
        while (mm) {
          const int k = __ffs(mm) - 1;
          mm &= mm - 1;
          if (kk >= base && kk < base + SEED_LIST) lp[kk - base] = pidx(r0, k);
          ++kk;
        }
        wave_sync_lds();
        const int nl = min(SEED_LIST, total - base);
        if constexpr (sizeof(T) == 2) {
          if (vec16) {
            // lpr lanes share one row, 8 channels (16 bytes) each; partial sums
            // are combined inside the lane group (DPP, no LDS)
            const int rpi = 64 / lpr, sub = lane & (lpr - 1), slot = lane / lpr;
            for (int e0 = 0; e0 < nl; e0 += 4 * rpi) {
              uint4 b[4];
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * rpi + slot;
                b[u] = e < nl && sub * 8 < dm + sh
                           ? *reinterpret_cast<const uint4*>(X - sh + (size_t)lp[e] * d + sub * 8)
                           : make_uint4(0, 0, 0, 0);
              }
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const uint32_t w[4] = {b[u].x, b[u].y, b[u].z, b[u].w};
                double acc = 0.0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const uint32_t wj = (uint32_t)(sub * 8 + 2 * j - sh) < (uint32_t)dm ? w[j] : 0u;
                  const double p0 = (double)__uint_as_float(wj << 16) - cvs[sub * 8 + 2 * j];
                  const double p1 = (double)__uint_as_float(wj & 0xFFFF0000u) - cvs[sub * 8 + 2 * j + 1];
                  acc = fma(p0, p0, acc);
                  acc = fma(p1, p1, acc);
                }
                acc = group_sum_dpp(acc, lpr);
                const int e = e0 + u * rpi + slot;
                if (sub == 0 && e < nl) ldist[e] = acc;
              }
            }
          } else {
            for (int e = lane; e < nl; e += 64) ldist[e] = sqdist_g<T>(X + (size_t)lp[e] * d, cvec, dm);
          }
        } else {
          for (int e = lane; e < nl; e += 64) ldist[e] = sqdist_g<T>(X + (size_t)lp[e] * d, cvec, dm);
        }
        wave_sync_lds();
#pragma unroll
        for (int q = 0; q < SEED_RG; ++q) {
          if ((mask >> q) & 1u) {
            const int kq = offs + __popc(mask & ((1u << q) - 1u));
            if (kq >= base && kq < base + SEED_LIST) {
              const double dist = ldist[kq - base];
              if (s == 0 || dist < gd2[q]) {
                gd2[q] = dist;
                nr_set(q, s == 0 ? 0u : ((uint32_t)s | (nr_get(q) & NR_MARK)));
                chg |= 1u << q;
              }
            }
          }
        }
        wave_sync_lds();
      }
      if (ci / (SEED_RG * SEED_NT) == gi && tid == ((ci >> 9) & (SEED_NW - 1)) * 64 + (ci & 63)) {
        const int kc = (ci >> 6) & (SEED_RG - 1);
#pragma unroll
        for (int k = 0; k < SEED_RG; ++k) if (k == kc) { nr_set(k, nr_get(k) | NR_MARK); chg |= 1u << k; }
      }
      if (!RESIDENT) {
        chg &= vm;
#pragma unroll
        for (int k = 0; k < SEED_RG; ++k) {
          if ((chg >> k) & 1u) {
            const int p = pidx(r0, k);
            D2g[p] = gd2[k];
            NRg[p] = (uint16_t)nr_get(k);
          }
        }
      }
      double loc = 0.0;
#pragma unroll
      for (int k = 0; k < SEED_RG; ++k) loc += gd2[k];
      const double t = wave_sum_dpp(loc);
      if (lane == 0) wsum[gi * SEED_NW + wv] = t;
    }
    __syncthreads();
  }
  // ---- initial centroids = the chosen points ----------------------------------------
  for (int idx = wg == 0 ? tid : C * dm; idx < C * dm; idx += SEED_NT) {
    const int c = idx / dm, ch = idx % dm;
    const float val = Elem<T>::ldf(X + (size_t)chosen[c] * d + ch);
    if (m == 0) qcent[((size_t)bh * g.Cq + c) * d + ch] = val;
    else kcent[((size_t)bh * g.Cm + c) * d + off + ch] = val;
  }
}

// ---------------------------------------------------------------------------
// k-means++ seeding with the point state in registers (N <= SR_NT * SR_PMAX).
// Same draw rule as seed_kernel (index-order running sum of D^2).
// Thread t owns the P consecutive points t P .. t P + P - 1, so (thread, slot)
// is the index order.  Per draw:
//   1. a block scan of the per-thread D^2 sums finds the crossing thread,
//      which walks its own slots to the point;
//   2. the centre row is staged in LDS; 3. its distances to the earlier
//      centres are computed by all waves (lanes = channels);
//   4. the Elkan test (||c_s - a||^2 >= 4 D^2 means no change) leaves the
//      points whose distance is needed; a block scan of the per-thread counts
//      orders them into one list, all threads compute the distances (lpr lanes
//      per row, 8 row loads in flight per lane), and the owners apply them.
// ---------------------------------------------------------------------------
constexpr int SR_NT = 512;
constexpr int SR_PMAX = 36;          // points per thread held in registers
constexpr int SR_LIST = 4096;        // list entries per compute round
constexpr int SR_CACHE_BYTES = 48 * 1024;

// squared distance over 8 channels c0 .. c0+7 of a row (channels >= dm count 0)
template <typename T>
__device__ __forceinline__ double sqdist8(const T* __restrict__ row, const double* __restrict__ c, int c0, int dm) {
  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (c0 + j < dm) {
      const double df = Elem<T>::ld(row + c0 + j) - c[c0 + j];
      acc = fma(df, df, acc);
    }
  }
  return acc;
}
__device__ __forceinline__ double sqdist8v(u32x4_t u, const double* __restrict__ c) {
  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double d0 = (double)__uint_as_float(u[j] << 16) - c[2 * j];
    const double d1 = (double)__uint_as_float(u[j] & 0xFFFF0000u) - c[2 * j + 1];
    acc = fma(d0, d0, acc);
    acc = fma(d1, d1, acc);
  }
  return acc;
}

template <typename T, int PM>
__global__ __launch_bounds__(SR_NT) void seedr_kernel(const T* __restrict__ qr, const T* __restrict__ kr, Geo g,
                                                      int32_t* __restrict__ seeds, float* __restrict__ qcent,
                                                      float* __restrict__ kcent) {
  const int m = blockIdx.y, bh = blockIdx.x;
  const int N = g.N, d = g.d, dm = g.dm[m], off = g.off[m], C = g.C[m];
  const T* X = (m == 0 ? qr : kr) + (size_t)bh * N * d + off;
  int32_t* sd = seeds + ((size_t)bh * 4 + m) * g.Cmax;

  __shared__ double cvec[128];
  __shared__ double cc[MAX_C];
  __shared__ int32_t chosen[MAX_C];
  __shared__ double dtmp[SR_NT / 64 + 1];
  __shared__ int32_t itmp[SR_NT / 64 + 1];
  __shared__ int32_t sh_ci, sh_lo, sh_hi;
  extern __shared__ __align__(16) unsigned char seedr_smem[];
  int32_t* list = reinterpret_cast<int32_t*>(seedr_smem);                                // [SR_LIST]
  double* ldist = reinterpret_cast<double*>(seedr_smem + SR_LIST * 4);                    // [SR_LIST]
  T* cache = reinterpret_cast<T*>(seedr_smem + SR_LIST * 12);                             // [C][cld]
  const int cld = dm + 2;
  const bool cached = (size_t)C * cld * sizeof(T) <= SR_CACHE_BYTES;

  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = (N + SR_NT - 1) / SR_NT;          // slots per thread (<= PM)
  // 16-byte row pieces: bf16 rows 16-byte aligned and the range a multiple of 8 channels
  const bool vecrow = sizeof(T) == 2 && ((off * 2) % 16 == 0) && ((d * 2) % 16 == 0) && (dm % 8 == 0);
  int lpr = 1;
  while (lpr * 8 < dm) lpr <<= 1;
  const uint64_t stream = ((uint64_t)bh * 4 + m) << 20;

  double d2[PM];
  // nearest centre of slot k (bits 0..14) | 0x8000 if the point is a chosen centre; two ids per word
  uint32_t nrw[(PM + 1) / 2];
#pragma unroll
  for (int k = 0; k < PM; ++k) d2[k] = 0.0;
#pragma unroll
  for (int k = 0; k < (PM + 1) / 2; ++k) nrw[k] = NR_MARK | (NR_MARK << 16);
  auto nr_get = [&](int k) -> uint32_t { return (nrw[k >> 1] >> (16 * (k & 1))) & 0xFFFFu; };
  auto nr_set = [&](int k, uint32_t v) {
    nrw[k >> 1] = (nrw[k >> 1] & ~(0xFFFFu << (16 * (k & 1)))) | (v << (16 * (k & 1)));
  };
  const int p0 = tid * P;
  auto valid = [&](int k) { return k < P && p0 + k < N; };

  int ci = 0;
  for (int s = 0; s < C; ++s) {
    // ---- 1. centre s -------------------------------------------------------------
    if (s == 0) {
      const uint64_t k0 = splitmix64(g.seed, stream) >> 11;
      const uint64_t lo = k0 * (uint64_t)N, hi = __umul64hi(k0, (uint64_t)N);
      ci = (int)((hi << 11) | (lo >> 53));
    } else {
      double loc = 0.0;
#pragma unroll
      for (int k = 0; k < PM; ++k) loc += valid(k) ? d2[k] : 0.0;
      double total;
      const double incl = block_incl_scan<double, SR_NT>(loc, dtmp, &total);
      const uint64_t ku = splitmix64(g.seed, stream + (uint64_t)s) >> 11;
      const double target = ((double)ku * 0x1p-53) * total;
      const int mode = total > 0.0 ? 0 : 2;   // 0 draw, 1 rounding at the end, 2 all zero
      if (tid == 0) { sh_ci = -1; sh_lo = 0x7FFFFFFF; sh_hi = -1; }
      __syncthreads();
      if (mode == 0) {
        const double excl = incl - loc;
        if (excl <= target && incl > target) {   // exactly one thread, unless rounding left no crossing
          double run = excl;
          int pick = -1;
#pragma unroll
          for (int k = 0; k < PM; ++k) {
            if (pick < 0 && valid(k)) { run += d2[k]; if (run > target) pick = k; }
          }
          if (pick < 0) {   // rounding inside the thread: its last slot with weight
#pragma unroll
            for (int k = 0; k < PM; ++k) if (valid(k) && d2[k] > 0.0) pick = k;
          }
          sh_ci = p0 + max(pick, 0);
        }
      } else {
        int low = 0x7FFFFFFF;
#pragma unroll
        for (int k = PM - 1; k >= 0; --k) if (valid(k) && !(nr_get(k) & NR_MARK)) low = p0 + k;
        if (low != 0x7FFFFFFF) atomicMin(&sh_lo, low);
      }
      __syncthreads();
      if (mode == 0 && sh_ci < 0) {
        // no crossing (u * total rounded up to total): the last point with D^2 > 0
        int best = -1;
#pragma unroll
        for (int k = 0; k < PM; ++k) if (valid(k) && d2[k] > 0.0) best = p0 + k;
        if (best >= 0) atomicMax(&sh_hi, best);
        __syncthreads();
        ci = sh_hi;
      } else {
        ci = mode == 0 ? sh_ci : sh_lo;
      }
      if (ci < 0 || ci >= N) ci = 0;
    }
    // ---- 2. centre row ---------------------------------------------------------------
    if (tid == 0) { chosen[s] = ci; sd[s] = ci; }
    if (tid < dm) {
      const T xv = X[(size_t)ci * d + tid];
      cvec[tid] = Elem<T>::ld(&xv);
      if (cached) cache[(size_t)s * cld + tid] = xv;
    }
    __syncthreads();
    // ---- 3. distances to the earlier centres (one centre per wave step, lanes = channels)
    for (int a = wv; a < s; a += SR_NT / 64) {
      double t = 0.0;
      for (int ch = lane; ch < dm; ch += 64) {
        const double xa = cached ? Elem<T>::ld(cache + (size_t)a * cld + ch) : Elem<T>::ld(X + (size_t)chosen[a] * d + ch);
        const double df = xa - cvec[ch];
        t = fma(df, df, t);
      }
      t = wave_sum_dpp(t);
      if (lane == 0) cc[a] = t;
    }
    __syncthreads();
    // ---- 4. points whose D^2 may change ------------------------------------------------
    static_assert(PM <= 64, "one need bit per slot");
    uint64_t need = 0;
#pragma unroll
    for (int k = 0; k < PM; ++k) {
      const bool nd = valid(k) && (s == 0 || !(cc[nr_get(k) & NR_ID] * (1.0 - 1e-9) >= 4.0 * d2[k]));
      need |= (uint64_t)nd << k;
    }
    const int cnt = __popcll(need);
    int K;
    const int o_t = block_incl_scan<int, SR_NT>(cnt, itmp, &K) - cnt;   // first list position of this thread
    for (int base = 0; base < K; base += SR_LIST) {
      if (o_t + cnt > base && o_t < base + SR_LIST) {
#pragma unroll
        for (int k = 0; k < PM; ++k) {
          if ((need >> k) & 1ull) {
            const int pos = o_t + __popcll(need & ((1ull << k) - 1ull));
            if (pos >= base && pos < base + SR_LIST) list[pos - base] = p0 + k;
          }
        }
      }
      __syncthreads();
      const int nl = min(SR_LIST, K - base);
      {
        const int sub = tid & (lpr - 1), slot = tid / lpr, nslot = SR_NT / lpr;
        const bool lv = sub * 8 < dm;
        const int c0 = lv ? sub * 8 : 0;
        for (int e0 = slot; e0 < nl; e0 += 8 * nslot) {
          double acc[8];
          if (vecrow) {
            u32x4_t b[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const int e = min(e0 + u * nslot, nl - 1);
              b[u] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(X) + (size_t)list[e] * d + c0);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[u] = sqdist8v(b[u], cvec + c0);
          } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const int e = min(e0 + u * nslot, nl - 1);
              acc[u] = sqdist8<T>(X + (size_t)list[e] * d, cvec, c0, dm);
            }
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const double a2 = group_sum_dpp(lv ? acc[u] : 0.0, lpr);
            const int e = e0 + u * nslot;
            if (sub == 0 && e < nl) ldist[e] = a2;
          }
        }
      }
      __syncthreads();
      if (o_t + cnt > base && o_t < base + SR_LIST) {
#pragma unroll
        for (int k = 0; k < PM; ++k) {
          if ((need >> k) & 1ull) {
            const int pos = o_t + __popcll(need & ((1ull << k) - 1ull));
            if (pos >= base && pos < base + SR_LIST) {
              const double dist = ldist[pos - base];
              if (s == 0 || dist < d2[k]) {
                d2[k] = dist;
                nr_set(k, s == 0 ? 0u : ((uint32_t)s | (nr_get(k) & NR_MARK)));
              }
            }
          }
        }
      }
      if (base + SR_LIST < K) __syncthreads();   // the list is rewritten in the next round
    }
    // the chosen point is a centre
    if (ci >= p0 && ci < p0 + P) {
#pragma unroll
      for (int k = 0; k < PM; ++k) if (p0 + k == ci) nr_set(k, nr_get(k) | NR_MARK);
    }
    __syncthreads();
  }
  for (int idx = tid; idx < C * dm; idx += SR_NT) {
    const int c = idx / dm, ch = idx % dm;
    const float val = Elem<T>::ldf(X + (size_t)chosen[c] * d + ch);
    if (m == 0) qcent[((size_t)bh * g.Cq + c) * d + ch] = val;
    else kcent[((size_t)bh * g.Cm + c) * d + off + ch] = val;
  }
}

// ---------------------------------------------------------------------------
// k-means++ seeding for bf16 data with the point state in LDS (1024 threads).
// Same draw rule as seed_kernel.  Thread t owns the P consecutive points
// t P .. t P + P - 1 ((thread, slot) is the index order).  The fp64 D^2 of
// every point lives in global memory; LDS holds, per point, one 32-bit word
// with D^2 rounded up to bf16 (high half) and ||x|| rounded to bf16 (low half)
// for the pruning tests, the 16-bit nearest centre ids, and each thread's fp64
// D^2 sum.  Per draw: a block scan of the per-thread sums finds the crossing
// thread, which reads its fp64 values to find the point; the centre's
// distances to the earlier centres are computed by all waves; the points that
// neither the Elkan test (||c_s - a||^2 >= 4 D^2, a the nearest centre) nor the
// norm test ((||x|| - ||c_s||)^2 >= D^2) rules out are listed in index order (a
// scan of per-thread counts) and all threads compute their fp64 distances;
// the thread that computes a distance applies it: it replaces the fp64 D^2
// (global) when smaller, refreshes the LDS copies and flags the owner, which
// then sums its P values afresh in slot order (no floating-point atomics, so
// the sums do not depend on timing).
// ---------------------------------------------------------------------------
constexpr int SL_NT = 1024;

// x >= 0 rounded to fp32 towards +infinity (for a non-negative finite float
// the next float up has the bit pattern plus one)
__device__ __forceinline__ float f32_up(double x) {
  const float f = (float)x;
  return (double)f < x ? __uint_as_float(__float_as_uint(f) + 1u) : f;
}
// bf16 bits of x >= 0 rounded up (an upper bound of x)
__device__ __forceinline__ uint32_t bf16_up_bits(double x) {
  const uint32_t b = __float_as_uint(f32_up(x));
  return (b >> 16) + ((b & 0xFFFFu) != 0u);
}
// bf16 bits of x >= 0 rounded to nearest (ties to even)
__device__ __forceinline__ uint32_t bf16_rn_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}
// squared norm of a 16-byte bf16 row piece, fp32 (only rounded to bf16 later)
__device__ __forceinline__ float sqnorm8v(u32x4_t u) {
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // through a scalar: this compiler turns a bit_cast of the vector element
    // u[j] itself into a cast of u[0]
    const uint32_t wj = u[j];
    const bf16x2_t pr = __builtin_bit_cast(bf16x2_t, wj);
    a = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, a, false);
  }
  return a;
}
__device__ __forceinline__ float sqnorm8(const uint16_t* __restrict__ row, int c0, int dm) {
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (c0 + j < dm) { const float x = bf16_to_f32(row[c0 + j]); a = fmaf(x, x, a); }
  return a;
}
constexpr int SL_LIST = 4096;
constexpr int SL_U = 8;          // rows in flight per lane group in the distance phase
constexpr int SL_LDS_LIMIT = 160 * 1024;

struct SeedLLayout {
  size_t d2s, nrs, list, tsum, tflag, cc, chosen, cache, bytes;
  bool cached;
};
__host__ __device__ inline SeedLLayout seedl_layout(int N, int C, int dm) {
  SeedLLayout L;
  const int P = (N + SL_NT - 1) / SL_NT;
  size_t o = 0;
  auto take = [&](size_t b) { const size_t r = o; o += (b + 15) & ~(size_t)15; return r; };
  L.d2s = take((size_t)4 * SL_NT * P);
  L.nrs = take((size_t)2 * SL_NT * P);
  L.list = take((size_t)4 * (SL_LIST + 1));
  L.tsum = take((size_t)8 * SL_NT);
  L.tflag = take((size_t)SL_NT);
  L.cc = take((size_t)8 * C);
  L.chosen = take((size_t)4 * C);
  const size_t base = o;
  L.cache = take((size_t)2 * C * (dm + 2));
  L.cached = o <= (size_t)SL_LDS_LIMIT - 2048;   // room left for the static LDS
  if (!L.cached) o = base;
  L.bytes = o;
  return L;
}

// VEC: every clustering reads its rows as aligned 16-byte pieces (offsets and
// widths are multiples of 8 channels); the host checks this.
template <bool VEC>
__global__ __launch_bounds__(SL_NT) void seedl_kernel(const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr,
                                                      Geo g, double* __restrict__ d2all, int32_t* __restrict__ seeds,
                                                      float* __restrict__ qcent, float* __restrict__ kcent, SeedSync sy) {
  int m, bh, wg;
  seed_block(sy, g.nk, m, bh, wg);
  // W workgroups share the clustering: this one owns the points
  // [pbase, pbase + N) (local indices below; drawn centres are global)
  const int W = m == 0 ? sy.W[0] : (m == 1 ? sy.W[1] : (m == 2 ? sy.W[2] : sy.W[3]));
  const int Nall = g.N;
  const int pbase = (int)((int64_t)wg * Nall / W);
  const int N = (int)((int64_t)(wg + 1) * Nall / W) - pbase;
  const int d = g.d, dm = g.dm[m], off = g.off[m], C = g.C[m];
  const uint16_t* Xh = (m == 0 ? qr : kr) + (size_t)bh * Nall * d + off;
  const uint16_t* X = Xh + (size_t)pbase * d;
  double* D2g = d2all + ((size_t)bh * 4 + m) * Nall + pbase;
  char* xs = sy.base + ((size_t)bh * 4 + m) * SEED_SYNC_BYTES;
  int32_t* x_ctr = reinterpret_cast<int32_t*>(xs);
  int32_t* x_ci = x_ctr + 1;
  unsigned long long* x_part = reinterpret_cast<unsigned long long*>(xs + 8);
  int32_t* x_lo = reinterpret_cast<int32_t*>(xs + 8 + 2 * 8 * SEED_MAX_GROUPS);
  int32_t* sd = seeds + ((size_t)bh * 4 + m) * g.Cmax;
  const SeedLLayout L = seedl_layout(N, C, dm);
  extern __shared__ __align__(16) unsigned char seedl_smem[];
  uint32_t* d2s = reinterpret_cast<uint32_t*>(seedl_smem + L.d2s);     // [P][NT] slot-major: D^2 up | norm
  uint16_t* nrs = reinterpret_cast<uint16_t*>(seedl_smem + L.nrs);     // [P][NT]
  int32_t* list = reinterpret_cast<int32_t*>(seedl_smem + L.list);     // [SL_LIST + 1]
  double* tsum = reinterpret_cast<double*>(seedl_smem + L.tsum);       // [NT]
  uint8_t* tflag = reinterpret_cast<uint8_t*>(seedl_smem + L.tflag);   // [NT] a point of the thread changed
  double* cc = reinterpret_cast<double*>(seedl_smem + L.cc);           // [C]
  int32_t* chosen = reinterpret_cast<int32_t*>(seedl_smem + L.chosen); // [C]
  uint16_t* cache = reinterpret_cast<uint16_t*>(seedl_smem + L.cache); // [C][cld]
  __shared__ double cvec[128];
  __shared__ double dtmp[SL_NT / 64 + 1];
  __shared__ int32_t itmp[SL_NT / 64 + 1];
  __shared__ int32_t sh_ci, sh_lo, sh_hi, sh_mode, sh_own;
  __shared__ double sh_pre, sh_tgt, sh_cn;
  const int cld = dm + 2;
  const bool cached = L.cached;

  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int P = (N + SL_NT - 1) / SL_NT;
  int lpr = 1;
  while (lpr * 8 < dm) lpr <<= 1;
  const uint64_t stream = ((uint64_t)bh * 4 + m) << 20;

  for (int i = threadIdx.x; i < SL_NT * P; i += SL_NT) { d2s[i] = 0u; nrs[i] = (uint16_t)NR_MARK; }
  tsum[threadIdx.x] = 0.0;
  tflag[threadIdx.x] = 0;
  __syncthreads();

  int nwait = 0;
  // all W workgroups of the clustering reach this point (bounded polling);
  // heavy: a device-wide fence on both sides, light: thread 0's own
  // agent-scope atomic stores only
  auto chain_wait = [&](bool heavy) __attribute__((always_inline)) {
    __syncthreads();
    ++nwait;
    if (threadIdx.x == 0) {
      if (heavy) __threadfence();
      else __builtin_amdgcn_s_waitcnt(0);
      atomicAdd(x_ctr, 1);
      const int want = W * nwait;
      uint32_t spins = 0;
      while (__hip_atomic_load(x_ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want) {
        if (__hip_atomic_load(sy.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
        if (++spins > SEED_SPIN_LIMIT) { atomicExch(sy.abort, 1); break; }
        __builtin_amdgcn_s_sleep(2);
      }
      if (heavy) __threadfence();
    }
    __syncthreads();
  };

  int ci = 0;
  for (int s = 0; s < C; ++s) {
    // the thread index is made opaque once per draw, so that values derived
    // from it are recomputed here instead of being kept live (and spilled)
    // across the whole loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int p0 = tid * P;
    // bit k: point p0 + k exists
    const int nk = max(0, min(P, N - p0));
    const uint32_t vmask = nk >= 32 ? 0xFFFFFFFFu : ((1u << nk) - 1u);
    // ---- 1. centre s -------------------------------------------------------------
    if (s == 0) {
      const uint64_t k0 = splitmix64(g.seed, stream) >> 11;
      const uint64_t lo = k0 * (uint64_t)Nall, hi = __umul64hi(k0, (uint64_t)Nall);
      ci = (int)((hi << 11) | (lo >> 53));
    } else if (W > 1) {
      // ---- the workgroups of the clustering together ------------------------------
      const double loc = tsum[tid];
      double total;   // this workgroup's
      const double incl = block_incl_scan_dpp<double, SL_NT>(loc, dtmp, &total);
      if (tid == 0)
        __hip_atomic_store(x_part + (s & 1) * SEED_MAX_GROUPS + wg, (unsigned long long)__double_as_longlong(total),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      chain_wait(false);
      if (wv == 0) {
        // every workgroup: the same sums in the same order, so the same owner
        const double v = lane < W ? __longlong_as_double((long long)__hip_atomic_load(
                                        x_part + (s & 1) * SEED_MAX_GROUPS + lane, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT))
                                  : 0.0;
        const double inc = wave_incl_scan(v);
        const double gtot = __shfl(inc, 63);
        int mode = 2, owner = 0;
        double pre = 0.0, tgt = 0.0;
        if (gtot > 0.0) {
          const uint64_t ku = splitmix64(g.seed, stream + (uint64_t)s) >> 11;
          tgt = ((double)ku * 0x1p-53) * gtot;
          const uint64_t hit = __ballot(lane < W && inc > tgt);
          if (hit) {
            mode = 0;
            owner = __ffsll((unsigned long long)hit) - 1;
            pre = __shfl(inc - v, owner);
          } else {
            mode = 1;
            owner = 63 - __clzll((long long)__ballot(lane < W && v > 0.0));
          }
        }
        if (lane == 0) {
          sh_mode = mode; sh_own = owner; sh_pre = pre; sh_tgt = tgt;
          sh_ci = -1; sh_lo = 0x7FFFFFFF; sh_hi = -1;
        }
      }
      __syncthreads();
      const int mode = sh_mode;
      if (mode == 2) {
        // every point coincides with a centre: the lowest index not chosen yet
        int low = 0x7FFFFFFF;
        for (int k = P - 1; k >= 0; --k) {
          const int p = p0 + k;
          if (p < N && !(nrs[k * SL_NT + tid] & NR_MARK)) low = p;
        }
        if (low != 0x7FFFFFFF) {
          atomicMin(x_lo + s, pbase + low);
          __builtin_amdgcn_s_waitcnt(0);   // performed before the wait below publishes it
        }
        chain_wait(true);
        ci = __hip_atomic_load(x_lo + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        if (wg == sh_own) {
          const double pre = sh_pre, target = sh_tgt;
          int lci = -1;
          if (mode == 0) {
            const double excl = pre + (incl - loc), inc2 = pre + incl;
            const uint64_t cross = __ballot(excl <= target && inc2 > target);
            if (cross) {
              const int L = __ffsll((unsigned long long)cross) - 1;
              const double ex = __shfl(excl, L);
              const int q0 = (wv * 64 + L) * P;
              const int p = q0 + lane;
              const double v = (lane < P && p < N) ? D2g[p] : 0.0;
              const double inc = ex + wave_incl_scan_dpp(v);
              const uint64_t hit = __ballot(lane < P && p < N && inc > target);
              const uint64_t pos = __ballot(v > 0.0);
              const int k = hit ? __ffsll((unsigned long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
              if (lane == 0) sh_ci = q0 + k;
            }
            __syncthreads();
            lci = sh_ci;
          }
          if (lci < 0) {
            // the last point with D^2 > 0 (rounding left the target at the end)
            int best = -1;
            for (int k = 0; k < P; ++k) { const int p = p0 + k; if (p < N && D2g[p] > 0.0) best = p; }
            if (best >= 0) atomicMax(&sh_hi, best);
            __syncthreads();
            lci = sh_hi;
          }
          if (tid == 0)
            __hip_atomic_store(x_ci, (s << 20) | ((pbase + max(lci, 0)) & 0xFFFFF), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        // the drawn index, published by its owner as (s << 20) | index
        if (tid == 0) {
          uint32_t spins = 0;
          int v = __hip_atomic_load(x_ci, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          while ((v >> 20) != s) {
            if (__hip_atomic_load(sy.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
            if (++spins > SEED_SPIN_LIMIT) { atomicExch(sy.abort, 1); break; }
            __builtin_amdgcn_s_sleep(1);
            v = __hip_atomic_load(x_ci, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          sh_lo = v & 0xFFFFF;
        }
        __syncthreads();
        ci = sh_lo;
      }
      if (ci < 0 || ci >= Nall) ci = 0;
    } else {
      const double loc = tsum[tid];
      double total;
      const double incl = block_incl_scan_dpp<double, SL_NT>(loc, dtmp, &total);
      const uint64_t ku = splitmix64(g.seed, stream + (uint64_t)s) >> 11;
      const double target = ((double)ku * 0x1p-53) * total;
      if (tid == 0) { sh_ci = -1; sh_lo = 0x7FFFFFFF; sh_hi = -1; }
      __syncthreads();
      if (total > 0.0) {
        const double excl = incl - loc;
        // the crossing thread's wave reads its P fp64 values (one per lane) and scans them
        const uint64_t cross = __ballot(excl <= target && incl > target);
        if (cross) {
          const int L = __ffsll((unsigned long long)cross) - 1;
          const double ex = __shfl(excl, L);
          const int q0 = (wv * 64 + L) * P;
          const int p = q0 + lane;
          const double v = (lane < P && p < N) ? D2g[p] : 0.0;
          const double inc = ex + wave_incl_scan_dpp(v);
          const uint64_t hit = __ballot(lane < P && p < N && inc > target);
          const uint64_t pos = __ballot(v > 0.0);
          const int k = hit ? __ffsll((unsigned long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
          if (lane == 0) sh_ci = q0 + k;
        }
        __syncthreads();
        if (sh_ci < 0) {
          // no crossing (u * total rounded up to total): the last point with D^2 > 0
          int best = -1;
          for (int k = 0; k < P; ++k) { const int p = p0 + k; if (p < N && D2g[p] > 0.0) best = p; }
          if (best >= 0) atomicMax(&sh_hi, best);
          __syncthreads();
          ci = sh_hi;
        } else {
          ci = sh_ci;
        }
      } else {
        // every point coincides with a centre: the lowest index not chosen yet
        int low = 0x7FFFFFFF;
        for (int k = P - 1; k >= 0; --k) {
          const int p = p0 + k;
          if (p < N && !(nrs[k * SL_NT + tid] & NR_MARK)) low = p;
        }
        if (low != 0x7FFFFFFF) atomicMin(&sh_lo, low);
        __syncthreads();
        ci = sh_lo;
      }
      if (ci < 0 || ci >= N) ci = 0;
    }
    // ---- 2. centre row ---------------------------------------------------------------
    if (tid == 0) { chosen[s] = ci; if (wg == 0) sd[s] = ci; }
    if (tid < dm) {
      const uint16_t xv = Xh[(size_t)ci * d + tid];
      cvec[tid] = (double)bf16_to_f32(xv);
      if (cached) cache[(size_t)s * cld + tid] = xv;
    }
    __syncthreads();
    if (W > 1 && wv == 0) {
      // squared norm of the centre (for its bf16 norm when it is another workgroup's point)
      double t = 0.0;
      for (int ch = lane; ch < dm; ch += 64) t = fma(cvec[ch], cvec[ch], t);
      t = wave_sum_dpp(t);
      if (lane == 0) sh_cn = t;
    }
    // ---- 3. distances to the earlier centres (lanes = channels) -------------------------
    for (int a = wv; a < s; a += SL_NT / 64) {
      double t = 0.0;
      for (int ch = lane; ch < dm; ch += 64) {
        const double xa = (double)bf16_to_f32(cached ? cache[(size_t)a * cld + ch] : Xh[(size_t)chosen[a] * d + ch]);
        const double df = xa - cvec[ch];
        t = fma(df, df, t);
      }
      t = wave_sum_dpp(t);
      if (lane == 0) cc[a] = t;
    }
    __syncthreads();
    // ---- 4. points whose D^2 may change ------------------------------------------------
    // dv (the high half) is the exact D^2 rounded up, so both tests only skip
    // points whose distance cannot drop:
    //   Elkan: ||c_s - a||^2 >= 4 dv (the factor 4.000004 covers the product's
    //     rounding);
    //   norm: | ||x|| - ||c_s|| | >= |xb - cb| - 2^-7 (xb + cb) =: g, with xb, cb
    //     the bf16 norms (relative error <= 2^-9 each, plus fp32 rounding), so
    //     g > 0 and g^2 >= 1.0001 dv imply ||x - c_s||^2 >= D^2.
    uint32_t need = vmask;
    if (s > 0) {
      // the centre's bf16 norm: from its slot when the centre is this
      // workgroup's point, else from its row (any bf16 rounding of the norm
      // keeps the test's bound)
      const int lc = ci - pbase;
      float cb;
      if (lc >= 0 && lc < N) {
        const uint32_t cw = d2s[(lc - (lc / P) * P) * SL_NT + lc / P];
        cb = __uint_as_float(cw << 16);
      } else {
        cb = __uint_as_float(bf16_rn_bits(sqrtf((float)sh_cn)) << 16);
      }
      need = 0;
      for (int k0 = 0; k0 < P; k0 += 8) {
        // eight slots at a time: their LDS reads issue together
        uint32_t nv[8], wv8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int k = min(k0 + u, P - 1);
          nv[u] = nrs[k * SL_NT + tid];
          wv8[u] = d2s[k * SL_NT + tid];
        }
        double ca[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) ca[u] = cc[nv[u] & NR_ID];
        uint32_t bits = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float dv = __uint_as_float(wv8[u] & 0xFFFF0000u), xb = __uint_as_float(wv8[u] << 16);
          const float gap = fabsf(xb - cb) - 0x1p-7f * (xb + cb);
          const bool skip = ca[u] >= 4.000004 * (double)dv || (gap > 0.f && gap * gap >= dv * 1.0001f);
          bits |= (uint32_t)!skip << u;
        }
        need |= bits << k0;
      }
      need &= vmask;
    }
    const int cnt = __popc(need);
    int K;
    const int o_t = block_incl_scan_dpp<int, SL_NT>(cnt, itmp, &K) - cnt;
    for (int base = 0; base < K; base += SL_LIST) {
      if (o_t + cnt > base && o_t < base + SL_LIST) {
        int pos = o_t;
        for (uint32_t mm = need; mm != 0u; mm &= mm - 1u, ++pos)
          if (pos >= base && pos < base + SL_LIST) list[pos - base] = p0 + __ffs(mm) - 1;
      }
      __syncthreads();
      const int nl = min(SL_LIST, K - base);
      {
        const int sub = tid & (lpr - 1), slot = tid / lpr, nslot = SL_NT / lpr;
        const bool lv = sub * 8 < dm;
        const int c0 = lv ? sub * 8 : 0;
        for (int e0 = slot; e0 < nl; e0 += SL_U * nslot) {
          double acc[SL_U];
          float xx[SL_U];   // squared norms (first draw only)
          int pp[SL_U];
#pragma unroll
          for (int u = 0; u < SL_U; ++u) pp[u] = list[min(e0 + u * nslot, nl - 1)];
          if constexpr (VEC) {
            // 32-bit byte offsets from the uniform row base (N d <= 2^25)
            const char* Xb = reinterpret_cast<const char*>(X);
            u32x4_t b[SL_U];
#pragma unroll
            for (int u = 0; u < SL_U; ++u)
              b[u] = *reinterpret_cast<const u32x4_t*>(Xb + ((uint32_t)pp[u] * (uint32_t)(2 * d) + (uint32_t)(2 * c0)));
#pragma unroll
            for (int u = 0; u < SL_U; ++u) acc[u] = sqdist8v(b[u], cvec + c0);
            if (s == 0) {
#pragma unroll
              for (int u = 0; u < SL_U; ++u) xx[u] = lv ? sqnorm8v(b[u]) : 0.f;
            }
          } else {
#pragma unroll
            for (int u = 0; u < SL_U; ++u) acc[u] = sqdist8<uint16_t>(X + (size_t)pp[u] * d, cvec, c0, dm);
            if (s == 0) {
#pragma unroll
              for (int u = 0; u < SL_U; ++u) xx[u] = lv ? sqnorm8(X + (size_t)pp[u] * d, c0, dm) : 0.f;
            }
          }
          double old[SL_U];
#pragma unroll
          for (int u = 0; u < SL_U; ++u)
            old[u] = (sub == 0 && s > 0)
                         ? *reinterpret_cast<const double*>(reinterpret_cast<const char*>(D2g) + (uint32_t)pp[u] * 8u)
                         : 0.0;
#pragma unroll
          for (int u = 0; u < SL_U; ++u) {
            const double dist = group_sum_dpp(lv ? acc[u] : 0.0, lpr);
            // norm of the row (first draw): fp32 partial sums, rounded to bf16
            const float xn = s == 0 ? sqrtf((float)group_sum_dpp((double)xx[u], lpr)) : 0.f;
            const int e = e0 + u * nslot;
            if (sub == 0 && e < nl && (s == 0 || dist < old[u])) {
              const int p = pp[u];
              const int t = p / P, k = p - t * P;
              const int li = k * SL_NT + t;
              D2g[p] = dist;
              d2s[li] = (bf16_up_bits(dist) << 16) | (s == 0 ? bf16_rn_bits(xn) : (d2s[li] & 0xFFFFu));
              nrs[li] = s == 0 ? (uint16_t)0 : (uint16_t)(s | (nrs[li] & NR_MARK));
              tflag[t] = 1;
            }
          }
        }
      }
      __syncthreads();
    }
    // the D^2 sum of each thread whose points changed, afresh in slot order
    // (a fixed order, so the sums, and with them every draw, are the same on
    // every run)
    if (tflag[tid]) {
      double acc = 0.0;
      for (int k0 = 0; k0 < nk; k0 += 8) {
        double v[8];   // eight loads in flight, added in slot order
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = k0 + u < nk ? D2g[p0 + k0 + u] : 0.0;
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
      }
      tsum[tid] = acc;
      tflag[tid] = 0;
    }
    if (tid == 0 && ci - pbase >= 0 && ci - pbase < N) {
      const int lc = ci - pbase;
      const int t = lc / P, k = lc - t * P;
      nrs[k * SL_NT + t] |= (uint16_t)NR_MARK;
    }
    __syncthreads();
  }
  for (int idx = wg == 0 ? (int)threadIdx.x : C * dm; idx < C * dm; idx += SL_NT) {
    const int c = idx / dm, ch = idx % dm;
    const float val = bf16_to_f32(Xh[(size_t)chosen[c] * d + ch]);
    if (m == 0) qcent[((size_t)bh * g.Cq + c) * d + ch] = val;
    else kcent[((size_t)bh * g.Cm + c) * d + off + ch] = val;
  }
}

// ---------------------------------------------------------------------------
// bf16 copies of the fp32 centroids (zero padded to [Cpad][dpad]) and their
// squared norms (FLT_MAX on padding rows, so padding never wins).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void centroid_kernel(Geo g, const float* __restrict__ qcent,
                                                       const float* __restrict__ kcent, uint16_t* __restrict__ cbf,
                                                       float* __restrict__ cnorm) {
  const int m = blockIdx.x, bh = blockIdx.y;
  const int d = g.d, dm = g.dm[m], off = g.off[m], C = g.C[m], Cpad = g.Cpad[m], dpad = g.dpad[m];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint16_t* cb = cbf + ((size_t)bh * 4 + m) * g.CmaxPad * g.DPmax;
  float* cn = cnorm + ((size_t)bh * 4 + m) * g.CmaxPad;
  for (int c = wv; c < Cpad; c += 4) {
    const float* row =
        c < C ? (m == 0 ? qcent + ((size_t)bh * g.Cq + c) * d : kcent + ((size_t)bh * g.Cm + c) * d + off) : nullptr;
    double nrm = 0.0;
    for (int ch = lane; ch < dpad; ch += 64) {
      uint16_t b = 0;
      if (c < C && ch < dm) {
        b = f32_to_bf16(row[ch]);
        const double bv = (double)bf16_to_f32(b);
        nrm += bv * bv;
      }
      cb[(size_t)c * g.DPmax + ch] = b;
    }
    nrm = wave_sum(nrm);
    if (lane == 0) cn[c] = c < C ? (float)nrm : FLT_MAX;
  }
}

// Assignment, fp32 storage: exact fp64 distances to the fp32 centroids.
__global__ __launch_bounds__(256) void assign_exact_f32_kernel(const float* __restrict__ qr, const float* __restrict__ kr,
                                                               Geo g, const float* __restrict__ qcent,
                                                               const float* __restrict__ kcent,
                                                               int32_t* __restrict__ labels) {
  const int m = blockIdx.y, bh = blockIdx.z;
  const int N = g.N, d = g.d, dm = g.dm[m], off = g.off[m], C = g.C[m];
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= N) return;
  const float* x = (m == 0 ? qr : kr) + ((size_t)bh * N + p) * d + off;
  double best = __builtin_inf();
  int bi = 0;
  for (int c = 0; c < C; ++c) {
    const float* mu = m == 0 ? qcent + ((size_t)bh * g.Cq + c) * d : kcent + ((size_t)bh * g.Cm + c) * d + off;
    double acc = 0.0;
    for (int ch = 0; ch < dm; ++ch) {
      const double df = (double)x[ch] - (double)mu[ch];
      acc += df * df;
    }
    if (acc < best) { best = acc; bi = c; }
  }
  labels[((size_t)bh * 4 + m) * N + p] = bi;
}

// ---------------------------------------------------------------------------
// Stable counting sort of the labels of one clustering (one workgroup of 16
// waves per (clustering, head)): perm lists the points cluster by cluster in
// ascending index order, off[c] .. off[c+1] delimits cluster c.  Each wave
// owns a contiguous segment; inside a 64-point chunk, lanes with equal labels
// are ranked with a ballot per distinct label, so the order is deterministic.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void sort_kernel(Geo g, const int32_t* __restrict__ labels, int mlo,
                                                    int32_t* __restrict__ perm, int64_t perm_bh, int64_t perm_m,
                                                    int32_t* __restrict__ off, int64_t off_bh, int64_t off_m) {
  const int m = mlo + blockIdx.x, bh = blockIdx.y;
  const int N = g.N, C = g.C[m];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  __shared__ int32_t hist[16][MAX_C];
  __shared__ int32_t base[MAX_C + 1];
  __shared__ int32_t tmp[17];
  const int32_t* lab = labels + ((size_t)bh * 4 + m) * N;
  int32_t* pm = perm + bh * perm_bh + m * perm_m;
  int32_t* of = off + bh * off_bh + m * off_m;
  for (int i = tid; i < 16 * MAX_C; i += 1024) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int seg = (N + 15) / 16, s0 = min(N, wv * seg), s1 = min(N, s0 + seg);
  for (int c0 = s0; c0 < s1; c0 += 256) {
    int l4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) { const int p = c0 + u * 64 + lane; l4[u] = p < s1 ? lab[p] : -1; }
#pragma unroll
    for (int u = 0; u < 4; ++u) if (l4[u] >= 0) atomicAdd(&hist[wv][l4[u]], 1);
  }
  __syncthreads();
  // cluster totals, exclusive scan over clusters, per-wave cursors
  int run = 0;
  const int per = (C + 1023) / 1024;
  for (int k = 0; k < per; ++k) {
    const int c = tid * per + k;
    if (c < C) for (int w = 0; w < 16; ++w) run += hist[w][c];
  }
  int total;
  const int incl = block_incl_scan<int, 1024>(run, tmp, &total);
  int cur = incl - run;
  for (int k = 0; k < per; ++k) {
    const int c = tid * per + k;
    if (c < C) {
      base[c] = cur;
      for (int w = 0; w < 16; ++w) { const int h = hist[w][c]; hist[w][c] = cur; cur += h; }
    }
  }
  if (tid == 0) base[C] = N;
  __syncthreads();
  for (int c = tid; c <= C; c += 1024) of[c] = base[c];
  // stable scatter
  int Lnext = s0 + lane < s1 ? lab[s0 + lane] : -1;
  for (int c0 = s0; c0 < s1; c0 += 64) {
    const int p = c0 + lane;
    const int L = Lnext;
    Lnext = c0 + 64 + lane < s1 ? lab[c0 + 64 + lane] : -1;   // prefetch the next chunk
    uint64_t active = __ballot(p < s1);
    while (active) {
      const int first = __ffsll((unsigned long long)active) - 1;
      const int Lf = __shfl(L, first);
      const uint64_t mask = __ballot(L == Lf && p < s1);
      if (L == Lf && p < s1) {
        const int rank = __popcll(mask & ((1ull << lane) - 1ull));
        pm[hist[wv][Lf] + rank] = p;
      }
      __builtin_amdgcn_wave_barrier();
      if (lane == first) hist[wv][Lf] += __popcll(mask);
      __builtin_amdgcn_wave_barrier();
      active &= ~mask;
    }
  }
}

// ---------------------------------------------------------------------------
// Lloyd update, in two passes that replace a sort by label:
//  accum_kernel: one workgroup per (point range, channel slice, clustering,
//    head) streams its points in index order and adds every channel value, in
//    fp64, to an LDS table sums[label][channel] (lanes = channels, 64/SW points
//    per instruction, so no two lanes of one instruction share an address
//    unless two points share a label); slice 0 also counts the points per
//    label.  The table is written out as one partial per workgroup.
//  finalize_kernel: one wave per centroid adds the partials in a fixed order,
//    divides by the count, rounds to fp32 (an empty cluster keeps its
//    centroid), and refreshes the bf16 copy and its squared norm.
// For bf16 data the sums are exact (split by magnitude, below), so the LDS
// atomic order does not change the result: the mean equals exact sum / n
// rounded once.  fp32 data is summed in rounded fp64 (no delta updates).
// ---------------------------------------------------------------------------
constexpr int ACC_NT = 512;

// Centroid sums of bf16 data are kept in two parts, split by magnitude at
// 2^-19.  A bf16 value of magnitude >= 2^-19 is a multiple of 2^-26, so while
// every |x| < 2^9 and N <= 2^18 any sum of such values is below 2^27, a
// multiple of 2^-26, and exact in fp64 (53 bits).  The smaller nonzero values
// (rare: about 1.6e-6 of unit-variance data) are added with fp64 atomics to a
// global table; each is a multiple of 2^-54 when |x| >= 2^-47, and their sums
// stay below 2^-1, so these sums are exact as well.  Both parts are therefore
// independent of the order of the atomics, and big + small, rounded once, is
// the correctly rounded exact sum.  The RoPE kernel flags data outside
// {0} u [2^-47, 2^9) (plan status[3]).
__device__ __forceinline__ bool is_small_value(float v) { return v != 0.f && fabsf(v) < 0x1p-19f; }

template <typename T, int SW>
__global__ __launch_bounds__(ACC_NT) void accum_kernel(const T* __restrict__ qr, const T* __restrict__ kr, Geo g,
                                                       const int32_t* __restrict__ labels, double* __restrict__ psum,
                                                       int32_t* __restrict__ pcnt, int nslices, int parts,
                                                       double* __restrict__ ssm) {
  const int part = blockIdx.x, bh = blockIdx.z;
  // blockIdx.y enumerates the (clustering, slice) pairs
  int m = 0, sl = blockIdx.y;
  while (m < 3 && sl >= (g.dm[m] + SW - 1) / SW) { sl -= (g.dm[m] + SW - 1) / SW; ++m; }
  const int N = g.N, d = g.d, dm = g.dm[m], C = g.C[m];
  const int s0 = sl * SW, sw = min(SW, dm - s0);
  if (sw <= 0) return;
  extern __shared__ __align__(16) unsigned char acc_smem[];
  double* S = reinterpret_cast<double*>(acc_smem);                         // [C][SW]
  int32_t* cnt = reinterpret_cast<int32_t*>(acc_smem + (size_t)C * SW * 8);  // [C]
  // the wave index is uniform; readfirstlane lets the compiler keep wave-level values in SGPRs
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < C * SW; i += ACC_NT) S[i] = 0.0;
  for (int i = tid; i < C; i += ACC_NT) cnt[i] = 0;
  __syncthreads();

  const int per = (N + parts - 1) / parts;
  const int p0 = min(N, part * per), p1 = min(N, p0 + per);
  const int32_t* lab = labels + ((size_t)bh * 4 + m) * N;
  const T* X = (m == 0 ? qr : kr) + (size_t)bh * N * d + g.off[m] + s0;
  // A wave takes 64 points at a time.  Instruction k covers the G points
  // k + j*ST (j = lane / SW), which lie ST tokens apart and so rarely share a
  // label (an LDS address).  Loads use clamped addresses and adds are
  // unconditional, so the loop has no branches.
  constexpr int G = 64 / SW, ST = SW;
  const int ch = lane % SW, sub = lane / SW;
  const bool chv = ch < sw;
  const int chc = min(ch, sw - 1);
  int c0 = p0 + wv * 64;
  int Lnext = lab[min(c0 + lane, N - 1)];
  for (; c0 < p1; c0 += ACC_NT) {
    const int pl = c0 + lane;
    const int L = min(max(Lnext, 0), C - 1);
    const int np = min(64, p1 - c0);
    float v[ST];   // exact copies of the stored values (bf16 or fp32)
    const char* xc = reinterpret_cast<const char*>(X + (size_t)c0 * d);   // uniform base, 32-bit byte offsets
#pragma unroll
    for (int k = 0; k < ST; ++k)
      v[k] = Elem<T>::ldf(reinterpret_cast<const T*>(xc + (uint32_t)((min(k + sub * ST, np - 1) * d + chc) * sizeof(T))));
    // labels of the next chunk, in flight during this chunk's adds
    Lnext = lab[min(c0 + ACC_NT + lane, N - 1)];
    if (sl == 0 && pl < p1) atomicAdd(&cnt[L], 1);
#pragma unroll
    for (int k = 0; k < ST; ++k) {
      const int q = k + sub * ST;
      const int lk = __shfl(L, q, 64);
      const bool in = chv && q < np;
      // bf16: values below the split go to the global small-value sums (rare)
      const bool sm = sizeof(T) == 2 && in && is_small_value(v[k]);
      // lanes without a point add -0.0, which leaves every sum unchanged
      atomicAdd(&S[lk * SW + ch], (in && !sm) ? (double)v[k] : -0.0);
      if (sm) atomicAdd(&ssm[(((size_t)bh * 4 + m) * g.Cmax + lk) * d + s0 + ch], (double)v[k]);
    }
  }
  __syncthreads();
  double* out = psum + ((((size_t)bh * 4 + m) * nslices + sl) * parts + part) * (size_t)g.Cmax * SW;
  for (int i = tid; i < C * SW; i += ACC_NT) out[i] = S[i];
  if (sl == 0) {
    int32_t* oc = pcnt + (((size_t)bh * 4 + m) * parts + part) * g.Cmax;
    for (int i = tid; i < C; i += ACC_NT) oc[i] = cnt[i];
  }
}

// Changes of the sums: every point whose label differs from the previous
// assignment's adds its channel values (fp64, exact) to its new cluster and
// subtracts them from its old one; the sizes change by one each.  Same grid
// and LDS table as accum_kernel; the nonzero entries of the table are then
// added to the totals in global memory (fp64 atomics; exact, so in any
// order).  The workgroup takes its points in segments of PPT per thread (all
// labels of a segment in flight at once), lists the changed ones in LDS (after
// the table: 8 PPT bytes per thread) and then loads their rows in batches of
// 8 instructions per wave (64 / SW points each: lanes = channels) before
// adding them.  The launch takes the largest PPT of 16, 8, 4 whose lists fit
// next to the table: the segments of a workgroup are a chain of dependent
// label loads.
template <int SW, int PPT>
__global__ __launch_bounds__(ACC_NT) void accum_delta_kernel(const uint16_t* __restrict__ qr,
                                                             const uint16_t* __restrict__ kr, Geo g,
                                                             const int32_t* __restrict__ labels,
                                                             const int32_t* __restrict__ prev,
                                                             double* __restrict__ stot, int32_t* __restrict__ ntot,
                                                             int parts, double* __restrict__ ssm) {
  const int part = blockIdx.x, bh = blockIdx.z;
  int m = 0, sl = blockIdx.y;
  while (m < 3 && sl >= (g.dm[m] + SW - 1) / SW) { sl -= (g.dm[m] + SW - 1) / SW; ++m; }
  const int N = g.N, d = g.d, dm = g.dm[m], C = g.C[m];
  const int s0 = sl * SW, sw = min(SW, dm - s0);
  if (sw <= 0) return;
  extern __shared__ __align__(16) unsigned char acc_smem[];
  constexpr int SEG = ACC_NT * PPT;
  double* S = reinterpret_cast<double*>(acc_smem);                         // [C][SW]
  int32_t* cnt = reinterpret_cast<int32_t*>(acc_smem + (size_t)C * SW * 8);  // [C]
  int32_t* dpt = cnt + ((g.Cmax + 3) & ~3);   // [SEG] changed points of a segment
  int32_t* dlab = dpt + SEG;                  // [SEG] their new label | old label << 16
  __shared__ int32_t dcount;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < C * SW; i += ACC_NT) S[i] = 0.0;
  for (int i = tid; i < C; i += ACC_NT) cnt[i] = 0;
  __syncthreads();
  const int per = (N + parts - 1) / parts;
  const int p0 = min(N, part * per), p1 = min(N, p0 + per);
  const int32_t* lab = labels + ((size_t)bh * 4 + m) * N;
  const int32_t* prv = prev + ((size_t)bh * 4 + m) * N;
  const uint16_t* X = (m == 0 ? qr : kr) + (size_t)bh * N * d + g.off[m] + s0;
  constexpr int G = 64 / SW, U = 8;
  const int j = lane / SW, ch = lane % SW;
  const bool chv = ch < sw;
  // Segments of PPT points per thread: every thread loads its labels at
  // once, the changed points go to an LDS list (point, new | old << 16), and
  // then all waves add their rows (G points per instruction, U instructions
  // in flight).  The list order depends on timing, but the sums are exact.
  for (int seg = p0; seg < p1; seg += SEG) {
    if (tid == 0) dcount = 0;
    __syncthreads();
    int Ln[PPT], Lp[PPT];
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int p = seg + u * ACC_NT + tid;
      const bool ok = p < p1;
      Ln[u] = ok ? lab[p] : 0;
      Lp[u] = ok ? prv[p] : 0;
    }
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int p = seg + u * ACC_NT + tid;
      const bool c = p < p1 && Ln[u] != Lp[u];
      const uint64_t mk = __ballot(c);
      if (mk == 0) continue;
      int base = 0;
      if (lane == 0) base = atomicAdd(&dcount, (int)__popcll(mk));
      base = __shfl(base, 0);
      if (c) {
        const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
        dpt[pos] = p;
        dlab[pos] = min(max(Ln[u], 0), C - 1) | (min(max(Lp[u], 0), C - 1) << 16);
      }
    }
    __syncthreads();
    const int nchg = dcount;
    for (int b = wv * U * G; b < nchg; b += (ACC_NT / 64) * U * G) {
      float xv[U];
      int ln[U], lo[U];
      bool vv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = b + u * G + j;
        vv[u] = idx < nchg;
        const int pt = vv[u] ? dpt[idx] : 0;
        const int lb = vv[u] ? dlab[idx] : 0;
        ln[u] = lb & 0xFFFF;
        lo[u] = lb >> 16;
        xv[u] = (vv[u] && chv) ? bf16_to_f32(X[(size_t)pt * d + ch]) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (vv[u] && chv) {
          if (!is_small_value(xv[u])) {
            atomicAdd(&S[ln[u] * SW + ch], (double)xv[u]);
            atomicAdd(&S[lo[u] * SW + ch], -(double)xv[u]);
          } else {
            double* sr = ssm + ((size_t)bh * 4 + m) * g.Cmax * d + s0 + ch;
            atomicAdd(&sr[(size_t)ln[u] * d], (double)xv[u]);
            atomicAdd(&sr[(size_t)lo[u] * d], -(double)xv[u]);
          }
        }
        if (vv[u] && sl == 0 && ch == 0) {
          atomicAdd(&cnt[ln[u]], 1);
          atomicAdd(&cnt[lo[u]], -1);
        }
      }
    }
    __syncthreads();   // the list is rewritten by the next segment
  }
  __syncthreads();
  double* st = stot + ((size_t)bh * 4 + m) * g.Cmax * d + s0;
  for (int i = tid; i < C * SW; i += ACC_NT) {
    const double v = S[i];
    if (v != 0.0) atomicAdd(&st[(size_t)(i / SW) * d + i % SW], v);
  }
  if (sl == 0) {
    int32_t* nt = ntot + ((size_t)bh * 4 + m) * g.Cmax;
    for (int i = tid; i < C; i += ACC_NT)
      if (cnt[i] != 0) atomicAdd(&nt[i], cnt[i]);
  }
}

__global__ __launch_bounds__(256) void finalize_kernel(Geo g, const double* __restrict__ psum,
                                                       const int32_t* __restrict__ pcnt, int SW, int nslices,
                                                       int parts, int delta, double* __restrict__ stot,
                                                       const double* __restrict__ ssm,
                                                       int32_t* __restrict__ ntot, float* __restrict__ qcent,
                                                       float* __restrict__ kcent, uint16_t* __restrict__ cbf,
                                                       float* __restrict__ cnorm) {
  const int m = blockIdx.y, bh = blockIdx.z;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c >= g.C[m]) return;
  const int d = g.d, dm = g.dm[m], lane = threadIdx.x & 63;
  // totals: the sum of the partials, kept for the next update; with `delta`
  // the totals were updated in place by accum_delta_kernel
  int32_t* nt = ntot + ((size_t)bh * 4 + m) * g.Cmax + c;
  double* st = stot + (((size_t)bh * 4 + m) * g.Cmax + c) * d;
  int n = 0;
  if (delta) {
    n = *nt;
  } else {
    const int32_t* pc = pcnt + ((size_t)bh * 4 + m) * parts * g.Cmax + c;
    for (int q = 0; q < parts; ++q) n += pc[(size_t)q * g.Cmax];
  }
  float* row = m == 0 ? qcent + ((size_t)bh * g.Cq + c) * d : kcent + ((size_t)bh * g.Cm + c) * d + g.off[m];
  for (int ch = lane; ch < dm; ch += 64) {
    double sum = 0.0;
    if (delta) {
      sum = st[ch];
    } else {
      const int sl = ch / SW, j = ch % SW;
      const double* ps = psum + (((size_t)bh * 4 + m) * nslices + sl) * parts * (size_t)g.Cmax * SW + (size_t)c * SW + j;
      for (int q = 0; q < parts; ++q) sum += ps[(size_t)q * g.Cmax * SW];
      st[ch] = sum;
    }
    // big + small part: one rounding of the exact sum (bf16; ssm is zero for fp32)
    if (n > 0) row[ch] = (float)((sum + ssm[(((size_t)bh * 4 + m) * g.Cmax + c) * d + ch]) / (double)n);
  }
  if (lane == 0 && !delta) *nt = n;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // bf16 copy and squared norm of the (possibly unchanged) centroid
  uint16_t* cb = cbf + (((size_t)bh * 4 + m) * g.CmaxPad + c) * g.DPmax;
  double nrm = 0.0;
  for (int ch = lane; ch < dm; ch += 64) {
    const uint16_t bv = f32_to_bf16(row[ch]);
    cb[ch] = bv;
    const double f = (double)bf16_to_f32(bv);
    nrm += f * f;
  }
  nrm = wave_sum_dpp(nrm);
  if (lane == 0) cnorm[((size_t)bh * 4 + m) * g.CmaxPad + c] = (float)nrm;
}

// Final labels -> packed key codes [N][4] (uint16) and query labels.
__global__ void pack_kernel(Geo g, const int32_t* __restrict__ labels, uint16_t* __restrict__ codes,
                            int32_t* __restrict__ qlab, int32_t* __restrict__ qlab_out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)g.BH * g.N) return;
  const int bh = (int)(i / g.N), n = (int)(i % g.N);
  const int32_t* l = labels + (size_t)bh * 4 * g.N + n;
  ushort4 c;
  c.x = (uint16_t)l[g.N];
  // one key codebook (SCOPE_FULL_DIM_KEYS): the other two codes are 0, and
  // their lookup-table rows are all zero
  c.y = g.nk > 1 ? (uint16_t)l[2 * (size_t)g.N] : (uint16_t)0;
  c.z = g.nk > 2 ? (uint16_t)l[3 * (size_t)g.N] : (uint16_t)0;
  c.w = 0;
  reinterpret_cast<ushort4*>(codes)[i] = c;
  qlab[i] = l[0];
  if (qlab_out) qlab_out[i] = l[0];
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
// Lloyd assignment, bf16 data: persistent workgroups per (clustering, head),
// each wave taking 64-point tiles (two 32-point MFMA column tiles).
// The centroids sit in LDS as -2*mu (exact in bf16), so MFMA output + ||mu||^2
// is ||x - mu||^2 - ||x||^2.  Each lane holds 16 candidates (centroid rows) of
// one point per 32-centroid block; their element number 0..15 is written into
// the low 4 mantissa bits, so min3 / med3 give the block's best and second best
// together with the position of the best, and the block of the running best is
// kept apart.
// Error of a candidate value against the exact distance (up to the common
// ||x||^2), M = max ||mu||, with every addition (inside the MFMA and after it)
// off by at most one ulp, i.e. 2^-23 relative (faithful rounding, which
// covers rounding toward zero): accumulation of the dpad products
// <= (dpad + 16) 2^-23 * 2 |x| M; rounding of ||mu||^2 and of the sum
// <= 2^-22 (M^2 + 2 |x| M).  EPS is the sum of the two; the two values
// compared carry at most 2 EPS between them, and the packed bits move a value
// v by < 2^-19 |v| (charged at 2^-18 on each).  A point whose best two
// candidates lie within that window is re-decided with fp64 distances (ties
// to the lowest index), so the labels equal the fp64 argmin.
// ---------------------------------------------------------------------------
constexpr int ASG_WAVES = 12288;   // waves of one assignment, over all heads and clusterings

__device__ __forceinline__ float pack_pos(float x, int v) {
  return __uint_as_float((__float_as_uint(x) & ~0xFu) | (uint32_t)v);
}

// 8 bf16 channels c0 .. c0+7 of a row (channels >= dm read as zero; dm even)
__device__ __forceinline__ bf16x8_t load_row8(const uint16_t* __restrict__ row, int c0, int dm, bool vec16) {
  u32x4_t u = {0u, 0u, 0u, 0u};
  if (vec16 && c0 + 8 <= dm) {
    u = *reinterpret_cast<const u32x4_t*>(row + c0);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (c0 + 2 * j < dm) u[j] = *reinterpret_cast<const uint32_t*>(row + c0 + 2 * j);
  }
  return __builtin_bit_cast(bf16x8_t, u);
}

template <int KB>
__device__ __forceinline__ void assign_tiles(const uint16_t* __restrict__ X, int N, int d, int dm, int C, int Cpad,
                                             bool vec16, const uint16_t* __restrict__ sc, int ldc,
                                             const float* __restrict__ scn, float M, int32_t* __restrict__ lab,
                                             int gw, int gstride, int4* __restrict__ amb,
                                             int32_t* __restrict__ amb_ctr, int bhm) {
  const int lane = threadIdx.x & 63, hi = lane >> 5, col = lane & 31;
  const int ncb = Cpad / 32;
  const float gamma = (float)(KB * 16 + 16) * 0x1p-23f;
  const int ntiles = (N + 63) / 64;
  for (int tile = gw; tile < ntiles; tile += gstride) {
    bf16x8_t b[2][KB];
    float xn2[2] = {0.f, 0.f};
    int pts[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pts[t] = tile * 64 + t * 32 + col;
      const uint16_t* row = X + (size_t)min(pts[t], N - 1) * d;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        b[t][kb] = load_row8(row, kb * 16 + hi * 8, dm, vec16);
        const u32x4_t u = __builtin_bit_cast(u32x4_t, b[t][kb]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // through a scalar: a bit_cast of the vector element u[j] itself is
          // compiled as a cast of u[0]
          const uint32_t wj = u[j];
          const bf16x2_t pr = __builtin_bit_cast(bf16x2_t, wj);
          xn2[t] = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, xn2[t], false);
        }
      }
    }
    float best[2] = {FLT_MAX, FLT_MAX}, second[2] = {FLT_MAX, FLT_MAX};
    int bcb[2] = {0, 0};
    // Blocks that may hold the least exact distance: a block is marked when its
    // best value lies within wmark of the running best (a bound of the final
    // window, set before the final best and second are known: |v| <= |x|^2 +
    // 2 |x| M + M^2), so the marks cover every block with a value within the
    // window of the final best.  The re-decision only visits marked blocks.
    uint32_t live[2] = {0u, 0u};
    float wmark[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float xn = sqrtf(xn2[t] + __shfl_xor(xn2[t], 32)) * 1.0001f;
      const float eps = gamma * 2.f * xn * M + 0x1p-22f * (M * M + 2.f * xn * M);
      wmark[t] = 2.f * eps + 0x1p-17f * (xn * xn + 2.f * xn * M + M * M);
    }
    for (int cb = 0; cb < ncb; ++cb) {
      f32x16_t cn;   // ||mu||^2 of rows cb*32 + 8*(v/4) + 4*hi + v%4
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 q = *reinterpret_cast<const float4*>(scn + cb * 32 + 8 * g4 + 4 * hi);
        cn[4 * g4] = q.x; cn[4 * g4 + 1] = q.y; cn[4 * g4 + 2] = q.z; cn[4 * g4 + 3] = q.w;
      }
      const uint16_t* arow = sc + (cb * 32 + col) * ldc + hi * 8;
      f32x16_t acc[2];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(arow + kb * 16);
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[t][kb], kb == 0 ? f32x16_t{} : acc[t], 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float kb1 = FLT_MAX, ks1 = FLT_MAX;
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const float x = pack_pos(acc[t][v] + cn[v], v), y = pack_pos(acc[t][v + 1] + cn[v + 1], v + 1);
          ks1 = fminf(ks1, __builtin_amdgcn_fmed3f(kb1, x, y));
          kb1 = fminf(kb1, fminf(x, y));
        }
        second[t] = fminf(fminf(second[t], ks1), fmaxf(best[t], kb1));
        if (kb1 < best[t]) { best[t] = kb1; bcb[t] = cb; }
        if (kb1 <= best[t] + wmark[t]) live[t] |= 1u << cb;
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int v = (int)(__float_as_uint(best[t]) & 0xFu);
      const int idx = bcb[t] * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
      // merge the two half-waves holding the same point
      const float ob = __shfl_xor(best[t], 32), os = __shfl_xor(second[t], 32);
      const int oi = __shfl_xor(idx, 32);
      const bool mine = best[t] < ob || (best[t] == ob && idx < oi);
      const int ii = mine ? idx : oi;
      const float bb = fminf(best[t], ob);
      const float ss = fminf(fminf(second[t], os), fmaxf(best[t], ob));
      const float xn = sqrtf(xn2[t] + __shfl_xor(xn2[t], 32)) * 1.0001f;
      const float eps = gamma * 2.f * xn * M + 0x1p-22f * (M * M + 2.f * xn * M);
      const float window = 2.f * eps + 0x1p-18f * (fabsf(bb) + fabsf(ss));
      const uint32_t lvm = live[t] | __shfl_xor(live[t], 32);
      const int p = pts[t];
      if (hi == 0 && p < N) lab[p] = ii;
      // near ties: appended to the assignment's list with their marked
      // blocks; asg_exact_kernel re-decides them, spread over the whole chip
      const bool near = hi == 0 && p < N && ss - bb <= window;
      const uint64_t nm = __ballot(near);
      if (nm) {
        int base = 0;
        if (lane == 0) base = atomicAdd(amb_ctr, __popcll(nm));
        base = __shfl(base, 0);
        if (near)
          amb[base + __popcll(nm & ((1ull << lane) - 1ull))] = make_int4(bhm, p, (int)lvm, 0);
      }
    }
  }
}

// Exact re-decision of the near ties of one assignment (the list written by
// assign2_kernel; every entry is one point, so the order of the list does
// not matter): fp64 distances to the centroids of the marked blocks, in
// channel order, ties to the lowest index; the label is overwritten.  One
// wave per entry, two marked blocks at a time (lanes 0-31 the first, 32-63
// the second; lane col takes row col of its block).  The bf16 centroid rows
// are read from global memory, a whole row (zero padded to dpad) in flight
// at once in 16-byte pieces.
constexpr int AEX_NT = 256;
__global__ __launch_bounds__(AEX_NT) void asg_exact_kernel(const uint16_t* __restrict__ qr,
                                                            const uint16_t* __restrict__ kr, Geo g,
                                                            const uint16_t* __restrict__ cbf,
                                                            const int4* __restrict__ amb,
                                                            const int32_t* __restrict__ amb_ctr,
                                                            int32_t* __restrict__ labels) {
  __shared__ double xsh[AEX_NT / 64][128];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, hi = lane >> 5, col = lane & 31;
  double* xs = xsh[wv];
  const int n = *amb_ctr;
  for (int e = blockIdx.x * (AEX_NT / 64) + wv; e < n; e += gridDim.x * (AEX_NT / 64)) {
    const int4 en = amb[e];
    const int m = en.x & 3, bh = en.x >> 2, pp = en.y;
    uint32_t mm = (uint32_t)en.z;
    const int dm = g.dm[m], C = g.C[m], dp = g.dpad[m];
    const uint16_t* X = (m == 0 ? qr : kr) + ((size_t)bh * g.N + pp) * g.d + g.off[m];
    // the point's channels, zero up to the padded width (the centroid rows
    // are zero there too)
    for (int ch = lane; ch < dp; ch += 64) xs[ch] = ch < dm ? (double)bf16_to_f32(X[ch]) : 0.0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint16_t* gc = cbf + ((size_t)bh * 4 + m) * g.CmaxPad * g.DPmax;
    double bd = __builtin_inf();
    int bc = 0x7FFFFFFF;
    while (mm) {
      const int cb0 = __ffs(mm) - 1;
      mm &= mm - 1;
      const int cb1 = mm ? __ffs(mm) - 1 : -1;
      if (mm) mm &= mm - 1;
      const int cbl = hi ? cb1 : cb0;
      const int c = cbl * 32 + col;
      if (cbl < 0 || c >= C) continue;
      const uint16_t* row = gc + (size_t)c * g.DPmax;
      // the whole row in flight at once (up to 16 pieces of 8 channels), then
      // the products in channel order
      u32x4_t ur[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        ur[i] = i * 8 < dp ? *reinterpret_cast<const u32x4_t*>(row + i * 8) : u32x4_t{0u, 0u, 0u, 0u};
      double accd = 0.0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i * 8 < dp) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t wj = ur[i][j];
            const double d0 = xs[i * 8 + 2 * j] - (double)__uint_as_float(wj << 16);
            const double d1 = xs[i * 8 + 2 * j + 1] - (double)__uint_as_float(wj & 0xFFFF0000u);
            accd = fma(d0, d0, accd);
            accd = fma(d1, d1, accd);
          }
        }
      }
      if (accd < bd) { bd = accd; bc = c; }
    }
#pragma unroll
    for (int o2 = 32; o2 >= 1; o2 >>= 1) {
      const double od = __shfl_xor(bd, o2);
      const int oc = __shfl_xor(bc, o2);
      if (od < bd || (od == bd && oc < bc)) { bd = od; bc = oc; }
    }
    if (lane == 0 && bc != 0x7FFFFFFF) labels[((size_t)bh * 4 + m) * g.N + pp] = bc;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// KBMAX: the largest dpad / 16 of the launch; the kernel's register budget is
// that of its widest instantiated tile loop, so narrow heads get a narrow kernel.
// Workgroups of one head: split.start[m] .. split.start[m + 1] - 1 serve
// clustering m (counts proportional to its estimated work).
struct AsgSplit {
  int start[5];
};
// NT threads (NT / 64 waves) share one centroid table in LDS: a launch whose
// table is large takes more waves per workgroup, so that the SIMDs still hold
// two or three waves each.
template <int KBMAX, int NT>
__global__ __launch_bounds__(NT) void assign2_kernel(const uint16_t* __restrict__ qr,
                                                         const uint16_t* __restrict__ kr, Geo g,
                                                         const uint16_t* __restrict__ cbf,
                                                         const float* __restrict__ cnorm,
                                                         int32_t* __restrict__ labels, AsgSplit split,
                                                         int4* __restrict__ amb, int32_t* __restrict__ amb_ctr) {
  const int bx = blockIdx.x, bh = blockIdx.z;
  const int m = bx < split.start[1] ? 0 : (bx < split.start[2] ? 1 : (bx < split.start[3] ? 2 : 3));
  const int part = bx - (m == 0 ? 0 : (m == 1 ? split.start[1] : (m == 2 ? split.start[2] : split.start[3])));
  const int nparts = (m == 0 ? split.start[1] : (m == 1 ? split.start[2] : (m == 2 ? split.start[3] : split.start[4]))) -
                     (m == 0 ? 0 : (m == 1 ? split.start[1] : (m == 2 ? split.start[2] : split.start[3])));
  const int N = g.N, d = g.d, dm = g.dm[m], off = g.off[m], C = g.C[m], Cpad = g.Cpad[m], dpad = g.dpad[m];
  const int ldc = dpad + 8;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint16_t* sc = reinterpret_cast<uint16_t*>(smem_raw);                               // [Cpad][ldc] -2 mu
  float* scn = reinterpret_cast<float*>(smem_raw + (size_t)Cpad * ldc * 2);           // [Cpad] ||mu||^2
  __shared__ float red[NT / 64];
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint16_t* gc = cbf + ((size_t)bh * 4 + m) * g.CmaxPad * g.DPmax;
  for (int idx = tid; idx < Cpad * (dpad / 2); idx += NT) {
    const int r = idx / (dpad / 2), c2 = idx % (dpad / 2);
    const uint32_t u = *reinterpret_cast<const uint32_t*>(gc + (size_t)r * g.DPmax + 2 * c2);
    const float f0 = -2.f * __uint_as_float(u << 16), f1 = -2.f * __uint_as_float(u & 0xFFFF0000u);
    // x -2 is exact in bf16: the fp32 products keep 8 significant bits
    *reinterpret_cast<uint32_t*>(sc + r * ldc + 2 * c2) = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
  }
  const float* gcn = cnorm + ((size_t)bh * 4 + m) * g.CmaxPad;
  float mx = 0.f;
  for (int idx = tid; idx < Cpad; idx += NT) {
    const float v = gcn[idx];
    scn[idx] = v;
    if (idx < C) mx = fmaxf(mx, v);
  }
  mx = block_max<float, NT>(mx, red);   // also orders the LDS fills above
  const float M = sqrtf(mx) * 1.0001f;
  const uint16_t* X = (m == 0 ? qr : kr) + (size_t)bh * N * d + off;
  const bool vec16 = ((off * 2) % 16 == 0) && ((d * 2) % 16 == 0);
  int32_t* lab = labels + ((size_t)bh * 4 + m) * N;
  const int gw = part * (NT / 64) + wv, gstride = nparts * (NT / 64);
  const int kbn = dpad / 16;
  auto run = [&](auto kb) {
    constexpr int KB = decltype(kb)::value;
    if constexpr (KB <= KBMAX)
      if (kbn == KB)
        assign_tiles<KB>(X, N, d, dm, C, Cpad, vec16, sc, ldc, scn, M, lab, gw, gstride, amb, amb_ctr, bh * 4 + m);
  };
  run(std::integral_constant<int, 1>{});
  run(std::integral_constant<int, 2>{});
  run(std::integral_constant<int, 3>{});
  run(std::integral_constant<int, 4>{});
  run(std::integral_constant<int, 5>{});
  run(std::integral_constant<int, 6>{});
  run(std::integral_constant<int, 7>{});
  run(std::integral_constant<int, 8>{});
}

// ---- launchers --------------------------------------------------------------

hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s) {
  if (n) fill_i32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, v, n);
  return hipGetLastError();
}

template <typename T>
static void seed_launch(const Geo& g, const T* qr, const T* kr, const Workspace& w, int32_t* status, hipStream_t s) {
  const int ncl = 1 + g.nk;   // active clusterings
  dim3 grid(g.BH, ncl);
  size_t cache = 0;
  for (int m = 0; m < ncl; ++m) {
    const size_t b = (size_t)g.C[m] * (g.dm[m] + 2) * sizeof(T);
    if (b <= (size_t)SEED_CACHE_BYTES && b > cache) cache = b;
  }
  if (sizeof(T) == 2) {
    size_t need = 0;
    bool fits = (g.N + SL_NT - 1) / SL_NT <= 32;
    for (int m = 0; m < ncl; ++m) {
      const SeedLLayout L = seedl_layout(g.N, g.C[m], g.dm[m]);
      need = L.bytes > need ? L.bytes : need;
    }
    fits = fits && need + 2048 <= (size_t)SL_LDS_LIMIT;
    if (fits) {
      bool vec = g.d % 8 == 0;
      for (int m = 0; m < ncl; ++m) vec = vec && g.off[m] % 8 == 0 && g.dm[m] % 8 == 0;
      const void* fn = vec ? (const void*)seedl_kernel<true> : (const void*)seedl_kernel<false>;
      (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)need);
      // Resident slots left over after one workgroup per clustering go to the
      // query clusterings (the widest rows), at least 4 points per thread each.
      const int chains = g.BH * ncl;
      const int wmax = max(1, g.N / (4 * SL_NT));
      int Wq = 1, Wk = 1, dev = 0, ncu = 0, coop = 0, per_cu = 0;
      if (hipGetDevice(&dev) == hipSuccess &&
          hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
          hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess && coop &&
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, SL_NT, need) == hipSuccess) {
        const int cap = ncu * per_cu;
        Wk = max(1, min(wmax, cap / chains));
        Wq = max(Wk, min(wmax, (cap - g.nk * g.BH * Wk) / g.BH));
      }
      seed_sync_init_kernel<<<g.BH * 4, 256, 0, s>>>(w.seed_sync, g.BH * 4, status + 2);   // areas (bh, m) for all 4 m
      SeedSync sy;
      sy.base = w.seed_sync;
      sy.abort = status + 2;
      sy.W[0] = Wq;
      sy.W[1] = sy.W[2] = sy.W[3] = Wk;
      sy.flat = 1;
      sy.bh0 = 0;
      sy.nbh = g.BH;
      const uint16_t* q16 = (const uint16_t*)qr;
      const uint16_t* k16 = (const uint16_t*)kr;
      double* d2 = w.d2;
      int32_t* sd = w.seeds;
      float* qc = w.qcent;
      float* kc = w.kcent;
      if (Wq > 1 || Wk > 1) {
        void* args[] = {(void*)&q16, (void*)&k16, (void*)&g, (void*)&d2, (void*)&sd, (void*)&qc, (void*)&kc,
                        (void*)&sy};
        const unsigned nblk = (unsigned)(g.BH * Wq + g.nk * g.BH * Wk);
        if (hipLaunchCooperativeKernel(fn, dim3(nblk), dim3(SL_NT), args, (unsigned)need, s) == hipSuccess) return;
        (void)hipGetLastError();
      }
      sy.W[0] = sy.W[1] = sy.W[2] = sy.W[3] = 1;
      sy.flat = 0;
      if (vec)
        seedl_kernel<true><<<grid, SL_NT, need, s>>>(q16, k16, g, d2, sd, qc, kc, sy);
      else
        seedl_kernel<false><<<grid, SL_NT, need, s>>>(q16, k16, g, d2, sd, qc, kc, sy);
      return;
    }
  }
  const int P = (g.N + SR_NT - 1) / SR_NT;
  if (P <= SR_PMAX) {
    size_t rcache = 0;
    for (int m = 0; m < ncl; ++m) {
      const size_t b = (size_t)g.C[m] * (g.dm[m] + 2) * sizeof(T);
      if (b <= (size_t)SR_CACHE_BYTES && b > rcache) rcache = b;
    }
    const size_t rlds = (size_t)SR_LIST * 12 + rcache;
    auto gor = [&](auto kern) {
      (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)rlds);
      kern<<<grid, SR_NT, rlds, s>>>(qr, kr, g, w.seeds, w.qcent, w.kcent);
    };
    if (P <= 8) gor(seedr_kernel<T, 8>);
    else if (P <= 16) gor(seedr_kernel<T, 16>);
    else if (P <= 24) gor(seedr_kernel<T, 24>);
    else gor(seedr_kernel<T, SR_PMAX>);
    return;
  }
  const size_t lds = (size_t)SEED_NW * SEED_LIST * 12 + cache;
  const int chains = g.BH * ncl;
  const int G = ((g.N + SEED_NT - 1) / SEED_NT + SEED_RG - 1) / SEED_RG;
  seed_sync_init_kernel<<<g.BH * 4, 256, 0, s>>>(w.seed_sync, g.BH * 4, status + 2);   // areas (bh, m) for all 4 m
  double* d2 = w.d2;
  uint16_t* nr = reinterpret_cast<uint16_t*>(w.nearest);
  int32_t* sd = w.seeds;
  float* qc = w.qcent;
  float* kc = w.kcent;
  int dev = 0, ncu = 0, coop = 0;
  const bool can_coop = sizeof(T) == 2 && hipGetDevice(&dev) == hipSuccess &&
                        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess && coop;
  SeedSync sy;
  sy.base = w.seed_sync;
  sy.abort = status + 2;
  // bf16 data only (fp32 data keeps one workgroup per clustering): the running
  // sum then adds the workgroups' partial sums in range order, a fixed order,
  // so the draws are reproducible; only the rounding of the sums changes.
  //
  // Several workgroups per clustering when the chip holds them all at once
  // (a cooperative launch guarantees that, or fails and one is used), with
  // the point state in global memory.  A draw of clustering m costs about
  // ceil(G / W[m]) groups times (16 + d_m) (the state of every point, the
  // rows of the points that may move): the resident slots go, a head's
  // worth at a time, to the clustering with the largest such cost, each step
  // lowering its groups per workgroup by one; slots left at the end go to
  // the query clusterings (the widest rows).  (One workgroup per
  // 8192-point group with the state in registers, in launches of a few heads
  // whose rows stay in the Infinity Cache, measured 103.7 ms instead of
  // 56.8 ms at the Hunyuan-like size: the exchange among 15 workgroups per
  // draw and the six sequential launches cost more than the state traffic.)
  const auto kern = seed_kernel<T, false>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  int Wm[4] = {1, 1, 1, 1}, per_cu = 0;
  if (can_coop && hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, SEED_NT, lds) == hipSuccess &&
      chains <= ncu * per_cu) {
    const int cap = ncu * per_cu;
    int used = chains;
    auto groups = [&](int m) { return (G + Wm[m] - 1) / Wm[m]; };
    // one step for clustering m: the fewest workgroups with one group less each
    auto step = [&](int m) -> bool {
      const int k = groups(m) - 1;
      if (k < 1) return false;
      const int wn = (G + k - 1) / k;
      if (used + (wn - Wm[m]) * g.BH > cap) return false;
      used += (wn - Wm[m]) * g.BH;
      Wm[m] = wn;
      return true;
    };
    for (;;) {
      int mx = -1;
      double cmax = 0.0;
      for (int m = 0; m < ncl; ++m) {
        const double c = (double)groups(m) * (16 + g.dm[m]);
        if (groups(m) > 1 && c > cmax) { cmax = c; mx = m; }
      }
      if (mx < 0 || !step(mx)) break;
    }
    while (step(0)) {}
  }
  for (int m = 0; m < 4; ++m) sy.W[m] = m < ncl ? Wm[m] : 1;
  sy.flat = 1;
  sy.bh0 = 0;
  sy.nbh = g.BH;
  int nblk = 0;
  for (int m = 0; m < ncl; ++m) nblk += g.BH * Wm[m];
  if (nblk > chains) {
    void* args[] = {(void*)&qr, (void*)&kr, (void*)&g, (void*)&d2, (void*)&nr, (void*)&sd, (void*)&qc, (void*)&kc,
                    (void*)&sy};
    if (hipLaunchCooperativeKernel((const void*)kern, dim3((unsigned)nblk), dim3(SEED_NT), args, (unsigned)lds, s) ==
        hipSuccess)
      return;
    (void)hipGetLastError();
  }
  sy.W[0] = sy.W[1] = sy.W[2] = sy.W[3] = 1;
  sy.flat = 0;
  kern<<<grid, SEED_NT, lds, s>>>(qr, kr, g, d2, nr, sd, qc, kc, sy);
}

hipError_t launch_seed(const Geo& g, const void* qr, const void* kr, const Workspace& w, int32_t* status,
                       hipStream_t s) {
  if (g.bf16) seed_launch<uint16_t>(g, (const uint16_t*)qr, (const uint16_t*)kr, w, status, s);
  else seed_launch<float>(g, (const float*)qr, (const float*)kr, w, status, s);
  return hipGetLastError();
}

hipError_t launch_prep(const Geo& g, const Workspace& w, hipStream_t s) {
  centroid_kernel<<<dim3(1 + g.nk, g.BH), 256, 0, s>>>(g, w.qcent, w.kcent, w.cbf, w.cnorm);
  return hipGetLastError();
}

// Assignment i writes w.labels when iters - i is even, else w.labels_alt, so
// the last one (i = iters) always lands in w.labels.
static int32_t* labels_of(const Geo& g, const Workspace& w, int i) {
  return ((g.iters - i) % 2 == 0) ? w.labels : w.labels_alt;
}

hipError_t launch_assign(const Geo& g, const void* qr, const void* kr, const Workspace& w, int iter,
                         hipStream_t s) {
  int32_t* out = labels_of(g, w, iter);
  if (g.bf16) {
    if (iter == 0) fill_i32_kernel<<<(g.iters + 256) / 256, 256, 0, s>>>(w.amb_cnt, 0, (size_t)g.iters + 1);
    // ASG_WAVES waves in all, shared among the clusterings of a head in
    // proportion to Cpad (dpad / 16 + 1) (MFMA blocks plus the per-candidate
    // selection work; equal shares left the query clustering, with the widest
    // rows, as the last to finish), at most one wave per 64-point tile
    const int ntiles = (g.N + 63) / 64;
    double wsum = 0.0, wm[4];
    for (int m = 0; m < 4; ++m) { wm[m] = (double)g.Cpad[m] * (g.dpad[m] / 16 + 1); wsum += wm[m]; }
    const double per_head = (double)(ASG_WAVES + g.BH - 1) / g.BH;
    int waves[4];
    for (int m = 0; m < 4; ++m) {
      const int wv = (int)(per_head * wm[m] / wsum + 0.5);
      waves[m] = m <= g.nk ? max(1, min(wv, ntiles)) : 0;   // inactive clusterings get no waves
    }
    auto table_of = [&](int m) { return g.Cpad[m] * (g.dpad[m] + 8) * 2 + g.Cpad[m] * 4; };
    constexpr int kLdsCU = 160 * 1024;   // LDS of one CU
    // one launch for clusterings [lo_m, hi_m): the workgroup size that gives
    // the most waves per SIMD (LDS per CU and the kernel's registers), the
    // smaller one on ties
    auto launch = [&](int lo_m, int hi_m) {
      int table = 0, kb = 1;
      for (int m = lo_m; m < hi_m; ++m) { table = max(table, table_of(m)); kb = max(kb, g.dpad[m] / 16); }
      const int kbmax = kb <= 2 ? 2 : (kb <= 4 ? 4 : 8);
      const int vgpr_waves = kbmax <= 4 ? 4 : 3;   // waves per SIMD the kernel's registers allow
      int nt = 256, best = 0;
      for (int cand = 256; cand <= 768; cand += 256) {
        const int per_simd = min((kLdsCU / (table + 1024)) * (cand / 256), vgpr_waves);
        if (per_simd > best) { best = per_simd; nt = cand; }
      }
      const int bytes = table;
      AsgSplit sp;
      sp.start[0] = 0;
      for (int m = 0; m < 4; ++m) {
        const int wg = (m >= lo_m && m < hi_m) ? max(1, (waves[m] + nt / 64 - 1) / (nt / 64)) : 0;
        sp.start[m + 1] = sp.start[m] + wg;
      }
      const dim3 grid(sp.start[4], 1, g.BH);
      auto go = [&](auto kern) {
        if (bytes > 64 * 1024)
          (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        kern<<<grid, nt, bytes, s>>>((const uint16_t*)qr, (const uint16_t*)kr, g, w.cbf, w.cnorm, out, sp, w.amb,
                                     w.amb_cnt + iter);
      };
      if (kbmax == 2) {
        if (nt == 256) go(assign2_kernel<2, 256>); else if (nt == 512) go(assign2_kernel<2, 512>);
        else go(assign2_kernel<2, 768>);
      } else if (kbmax == 4) {
        if (nt == 256) go(assign2_kernel<4, 256>); else if (nt == 512) go(assign2_kernel<4, 512>);
        else go(assign2_kernel<4, 768>);
      } else {
        if (nt == 256) go(assign2_kernel<8, 256>); else if (nt == 512) go(assign2_kernel<8, 512>);
        else go(assign2_kernel<8, 768>);
      }
    };
    int table_k = 0;
    for (int m = 1; m <= g.nk; ++m) table_k = max(table_k, table_of(m));
    if (table_of(0) > 64 * 1024 && table_k < table_of(0)) {
      // The query clustering's centroid table is large: the key clusterings
      // get a launch of their own with their smaller tables.
      launch(0, 1);
      launch(1, 1 + g.nk);
    } else {
      launch(0, 1 + g.nk);
    }
    // the near ties of this assignment, over the whole chip
    asg_exact_kernel<<<1024, AEX_NT, 0, s>>>((const uint16_t*)qr, (const uint16_t*)kr, g, w.cbf, w.amb,
                                             w.amb_cnt + iter, out);
  } else {
    dim3 grid((g.N + 255) / 256, 1 + g.nk, g.BH);
    assign_exact_f32_kernel<<<grid, 256, 0, s>>>((const float*)qr, (const float*)kr, g, w.qcent, w.kcent, out);
  }
  return hipGetLastError();
}

hipError_t launch_update(const Geo& g, const void* qr, const void* kr, const Workspace& w, int it, hipStream_t s) {
  const int SW = acc_sw(g), ns = acc_slices(g);
  const int32_t* cur = labels_of(g, w, it - 1);
  // bf16 data from the second update on: only the points whose label changed
  // since the previous assignment move between the exact sums (fp32 data is
  // summed afresh every time)
  const bool delta = g.bf16 && it >= 2;
  const int parts = acc_parts(g);
  int ypairs = 0;
  for (int m = 0; m <= g.nk; ++m) ypairs += (g.dm[m] + SW - 1) / SW;
  const size_t lds = (size_t)g.Cmax * SW * 8 + (size_t)g.Cmax * 4;
  dim3 grid(parts, ypairs, g.BH);
  auto go = [&](auto kern, const auto* q, const auto* k) {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    kern<<<grid, ACC_NT, lds, s>>>(q, k, g, cur, w.psum, w.pcnt, ns, parts, w.ssm);
  };
  // the delta update's LDS: the table, then the two lists of PPT entries per
  // thread (the largest PPT that fits one CU, leaving 1 KB for the rest)
  const size_t tbl = (size_t)g.Cmax * SW * 8 + (size_t)((g.Cmax + 3) & ~3) * 4;
  auto dlds = [&](int ppt) { return tbl + (size_t)2 * ACC_NT * ppt * 4; };
  const int ppt = dlds(16) + 1024 <= MAX_ASSIGN_LDS ? 16 : (dlds(8) + 1024 <= MAX_ASSIGN_LDS ? 8 : 4);
  auto god = [&](auto kern) {
    const size_t dl = dlds(ppt);
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dl);
    kern<<<grid, ACC_NT, dl, s>>>((const uint16_t*)qr, (const uint16_t*)kr, g, cur, labels_of(g, w, it - 2), w.stot,
                                 w.ntot, parts, w.ssm);
  };
  const uint16_t *qb = (const uint16_t*)qr, *kb = (const uint16_t*)kr;
  const float *qf = (const float*)qr, *kf = (const float*)kr;
  if (it == 1) {
    // small-value sums start at zero (a fill kernel: no memset node in a captured graph)
    const hipError_t e = launch_fill_i32(reinterpret_cast<int32_t*>(w.ssm), 0, ssm_elems(g) * 2, s);
    if (e != hipSuccess) return e;
  }
  if (delta) {
    if (SW == 32) {
      if (ppt == 16) god(accum_delta_kernel<32, 16>);
      else if (ppt == 8) god(accum_delta_kernel<32, 8>);
      else god(accum_delta_kernel<32, 4>);
    } else {
      if (ppt == 16) god(accum_delta_kernel<16, 16>);
      else if (ppt == 8) god(accum_delta_kernel<16, 8>);
      else god(accum_delta_kernel<16, 4>);
    }
  } else if (g.bf16) {
    if (SW == 32) go(accum_kernel<uint16_t, 32>, qb, kb); else go(accum_kernel<uint16_t, 16>, qb, kb);
  } else {
    if (SW == 32) go(accum_kernel<float, 32>, qf, kf); else go(accum_kernel<float, 16>, qf, kf);
  }
  finalize_kernel<<<dim3((g.Cmax + 3) / 4, 1 + g.nk, g.BH), 256, 0, s>>>(g, w.psum, w.pcnt, SW, ns, parts, delta ? 1 : 0,
                                                                  w.stot, w.ssm, w.ntot, w.qcent, w.kcent, w.cbf, w.cnorm);
  return hipGetLastError();
}

hipError_t launch_perm(const Geo& g, const Workspace& w, int32_t* perm_q, int32_t* q_off, hipStream_t s) {
  sort_kernel<<<dim3(1, g.BH), 1024, 0, s>>>(g, w.labels, 0, perm_q, g.N, 0, q_off, g.Cq + 1, 0);
  return hipGetLastError();
}

hipError_t launch_pack(const Geo& g, const Workspace& w, int32_t* q_labels_out, hipStream_t s) {
  const int64_t n = (int64_t)g.BH * g.N;
  pack_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(g, w.labels, w.codes, w.qlab, q_labels_out);
  return hipGetLastError();
}

}  // namespace scope
