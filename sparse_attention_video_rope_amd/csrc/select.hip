// Stages 3-5 of SCOPE (arXiv 2608.12780; equations as quoted on the
// pith.science review page):
//   LUT      P^m[c][z] = <qbar_c on range m, mu^m_z>, m in {T, H, W}
//   proxy    s[c][j] = (1/sqrt(d)) (P^T[c][zT_j] + P^H[c][zH_j] + P^W[c][zW_j])   (Eq. 6)
//   Top-p    t_c = smallest t whose first t keys, ordered by (s desc, j asc),
//            hold softmax mass >= rho                                          (Eq. 7)
//   base     b_c = max(t_c, ceil(alpha N))                                     (Eq. 8)
//   k_head   ceil(sum_c n_c b_c / sum_c n_c)                                   (Eq. 9)
//   final    r_c = max(b_c, k_head) for non-empty clusters, 0 otherwise; S_c =
//            the first r_c keys in the same order, stored ascending          (Eq. 10)
//
// Selection never materialises the Cq x N score matrix: one workgroup per
// query cluster streams the packed key codes (8 B per key) and recomputes each
// logit from the cluster's three LUT rows in LDS.  The boundary key is found
// with two levels of 2048 linear bins over [s_min, s_max] carrying exact
// counts and fixed-point softmax mass (integer adds, so the result does not
// depend on the order of the LDS atomics), followed by an exact sort of the
// boundary bin by (s desc, j asc).  The softmax weight of key j is
// exp(s_j - s_max), formed as the product of three per-subspace factors
// exp(P^m/sqrt(d) - A_m) and exp(sum_m A_m - s_max).
#include <float.h>

#include "scope_device.hpp"
#include "scope_internal.hpp"

namespace scope {

// ---------------------------------------------------------------------------
// Stage 3: lookup tables, fp64 dot products of fp32 centroids.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lut_kernel(Geo g, const float* __restrict__ qcent,
                                                  const float* __restrict__ kcent, double* __restrict__ lut) {
  const int c = blockIdx.x, bh = blockIdx.y, d = g.d, Cm = g.Cm;
  __shared__ double qs[128];
  if (threadIdx.x < d) qs[threadIdx.x] = (double)qcent[((size_t)bh * g.Cq + c) * d + threadIdx.x];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 3 * Cm; idx += 256) {
    const int mm = idx / Cm, z = idx % Cm, o = g.off[mm + 1], dmm = g.dm[mm + 1];
    const float* kr = kcent + ((size_t)bh * Cm + z) * d + o;
    double acc = 0.0;
    for (int ch = 0; ch < dmm; ++ch) acc += qs[o + ch] * (double)kr[ch];
    lut[(((size_t)bh * g.Cq + c) * 3 + mm) * Cm + z] = acc;
  }
}

// ---------------------------------------------------------------------------
// Shared machinery of the selection kernels
// ---------------------------------------------------------------------------
constexpr int NT = 512;
constexpr int BPT = SEL_NB / NT;      // histogram bins per thread in a walk

struct SelArgs {
  int N, Cq, Cm;
  double inv_sqrt_d;                  // 1/sqrt(d), rounded once
  double rho;
  double fx_scale;                    // 2^S: fixed-point scale of softmax weights
  int floor_a;                        // ceil(alpha N)
};

struct Sel {
  const double *P0, *P1, *P2;         // LUT rows of the cluster
  const double *E0, *E1, *E2;         // exp(P^m/sqrt(d) - A_m)
  double F;                           // exp(sum_m A_m - s_max)
  double inv_sqrt_d, fx;
  double smax, scale1;
  const ushort4* codes;               // [N] packed (zT, zH, zW, 0)
  int N;
};

// No fused multiply-adds in the logit and the bin position: every pass must put
// a key in the same bin, whichever pass the compiler inlines them into.
__device__ __forceinline__ double logit(const Sel& S, ushort4 z) {
#pragma clang fp contract(off)
  return ((S.P0[z.x] + S.P1[z.y]) + S.P2[z.z]) * S.inv_sqrt_d;
}
__device__ __forceinline__ uint64_t weight_fx(const Sel& S, ushort4 z) {
  return (uint64_t)__double2ull_rn(((S.E0[z.x] * S.E1[z.y]) * S.E2[z.z]) * S.F * S.fx);
}
__device__ __forceinline__ double bin_x(const Sel& S, double s) {
#pragma clang fp contract(off)
  return (S.smax - s) * S.scale1;
}
__device__ __forceinline__ int bin1_of(double x) { return min(max((int)x, 0), SEL_NB - 1); }
__device__ __forceinline__ int bin2_of(double x, int b1) {
#pragma clang fp contract(off)
  return min(max((int)((x - (double)b1) * SEL_NB), 0), SEL_NB - 1);
}

// f(j, codes[j]) for the keys j = threadIdx.x + k NT, four code loads in flight
template <typename F>
__device__ __forceinline__ void each_key(const Sel& S, F&& f) {
  const int N = S.N;
  int j = threadIdx.x;
  for (; j + 3 * NT < N; j += 4 * NT) {
    const ushort4 z0 = S.codes[j], z1 = S.codes[j + NT], z2 = S.codes[j + 2 * NT], z3 = S.codes[j + 3 * NT];
    f(j, z0); f(j + NT, z1); f(j + 2 * NT, z2); f(j + 3 * NT, z3);
  }
  for (; j < N; j += NT) f(j, S.codes[j]);
}

struct SelSmem {
  int32_t* hc;       // [SEL_NB] counts
  uint64_t* hm;      // [SEL_NB] fixed-point mass
  double* cs;        // [SEL_CAP] candidate logits
  int32_t* cj;       // [SEL_CAP] candidate key indices
  uint64_t* cw;      // [SEL_CAP] candidate weights
  uint64_t* u64tmp;  // [NT/64 + 1]
  int64_t* i64tmp;   // [NT/64 + 1]
  double* dtmp;      // [NT/64]
  int32_t* misc;     // [8]
};

// Walk a histogram: first bin whose inclusive running weight (mass or count,
// starting at the given bases) reaches `tgt`.  Returns the bin and the
// running mass / count before it.
__device__ int hist_walk(const SelSmem& sm, bool by_mass, uint64_t tgt, uint64_t baseM, int64_t baseC,
                         uint64_t* beforeM, int64_t* beforeC) {
  const int tid = threadIdx.x;
  uint64_t lm = 0;
  int64_t lc = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) { lm += sm.hm[tid * BPT + i]; lc += sm.hc[tid * BPT + i]; }
  uint64_t totM;
  int64_t totC;
  const uint64_t exM = block_incl_scan<uint64_t, NT>(lm, sm.u64tmp, &totM) - lm;
  const int64_t exC = block_incl_scan<int64_t, NT>(lc, sm.i64tmp, &totC) - lc;
  uint64_t cm = baseM + exM;
  int64_t cc = baseC + exC;
  if (tid == NT - 1) {
    // default (target beyond the total): the last bin
    sm.misc[0] = SEL_NB - 1;
    sm.u64tmp[NT / 64] = baseM + totM - sm.hm[SEL_NB - 1];
    sm.i64tmp[NT / 64] = baseC + totC - sm.hc[SEL_NB - 1];
  }
  __syncthreads();
  const bool mine = by_mass ? (cm < tgt && cm + lm >= tgt) : ((uint64_t)cc < tgt && (uint64_t)(cc + lc) >= tgt);
  if (mine) {
    for (int i = 0; i < BPT; ++i) {
      const int b = tid * BPT + i;
      const uint64_t nm = cm + sm.hm[b];
      const int64_t nc = cc + sm.hc[b];
      if (by_mass ? nm >= tgt : (uint64_t)nc >= tgt) {
        sm.misc[0] = b;
        sm.u64tmp[NT / 64] = cm;   // slot past the scan's per-wave area
        sm.i64tmp[NT / 64] = cc;
        break;
      }
      cm = nm;
      cc = nc;
    }
  }
  __syncthreads();
  const int b = sm.misc[0];
  *beforeM = sm.u64tmp[NT / 64];
  *beforeC = sm.i64tmp[NT / 64];
  __syncthreads();
  return b;
}

// Boundary of the first `tgt` weight (mass or count) in the (s desc, j asc)
// order: the logit tau of the boundary key, how many keys with logit tau are
// taken (the lowest-indexed ones), and the total number of keys taken.
struct Boundary {
  double tau;
  int m;
  int count;
};

// Exact resolution of a boundary bin holding at most 64 keys (candidates already
// in sm.cs / cj / cw, n of them) by one wave: a bitonic sort across the lanes
// by (s desc, j asc), then the first position whose running weight reaches
// tgt (mass) or position tgt - before_count - 1 (count).
__device__ Boundary resolve_small_bin(const SelSmem& sm, int n, bool by_mass, uint64_t tgt, uint64_t bm, int64_t bc) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    double s = tid < n ? sm.cs[tid] : -__builtin_inf();
    int j = tid < n ? sm.cj[tid] : 0x7FFFFFFF - tid;   // distinct sentinels after every key
    uint64_t w = tid < n ? sm.cw[tid] : 0;
    for (int size = 2; size <= 64; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        const double so = __shfl_xor(s, stride);
        const int jo = __shfl_xor(j, stride);
        const uint64_t wo = __shfl_xor(w, stride);
        const bool other_first = so > s || (so == s && jo < j);
        const bool lower = (tid & stride) == 0, asc = (tid & size) == 0;
        if (lower == asc ? other_first : !other_first) { s = so; j = jo; w = wo; }
      }
    }
    int kb;
    if (by_mass) {
      const uint64_t run = bm + wave_incl_scan(w);
      const uint64_t hit = __ballot(tid < n && run >= tgt);
      kb = hit ? __ffsll((unsigned long long)hit) - 1 : n - 1;
    } else {
      kb = min(max((int)((int64_t)tgt - bc - 1), 0), n - 1);
    }
    const double tau = __shfl(s, kb);
    const uint64_t same = __ballot(s == tau);
    const int k0 = __ffsll((unsigned long long)same) - 1;
    if (tid == 0) {
      sm.dtmp[0] = tau;
      sm.misc[4] = kb - k0 + 1;
      sm.misc[5] = (int)bc + kb + 1;
    }
  }
  __syncthreads();
  Boundary r;
  r.tau = sm.dtmp[0];
  r.m = sm.misc[4];
  r.count = sm.misc[5];
  __syncthreads();
  return r;
}

// Exact resolution of a boundary bin of at most SEL_CAP keys (candidates already
// in sm.cs / cj / cw, ncand of them, bin bases bm / bc): a bitonic sort in LDS
// by (s desc, j asc), then the first position whose running weight reaches tgt
// (mass) or position tgt - bc - 1 (count).
__device__ Boundary resolve_lds_bin(const SelSmem& sm, int ncand, bool by_mass, uint64_t tgt, uint64_t bm,
                                    int64_t bc) {
  const int tid = threadIdx.x;
  Boundary r;
  int P2 = 1;
  while (P2 < ncand) P2 <<= 1;
  for (int k = ncand + tid; k < P2; k += NT) { sm.cs[k] = -__builtin_inf(); sm.cj[k] = 0x7FFFFFFF; sm.cw[k] = 0; }
  __syncthreads();
  for (int size = 2; size <= P2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P2 / 2; i += NT) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const bool up = (lo & size) == 0;
        const double s0 = sm.cs[lo], s1 = sm.cs[hi];
        const int j0 = sm.cj[lo], j1 = sm.cj[hi];
        const bool hi_first = s1 > s0 || (s1 == s0 && j1 < j0);
        if (hi_first == up) {
          sm.cs[lo] = s1; sm.cs[hi] = s0;
          sm.cj[lo] = j1; sm.cj[hi] = j0;
          const uint64_t w0 = sm.cw[lo];
          sm.cw[lo] = sm.cw[hi]; sm.cw[hi] = w0;
        }
      }
      __syncthreads();
    }
  }
  int kb;
  if (by_mass) {
    // running mass over the sorted candidates; first position reaching tgt
    constexpr int PER = SEL_CAP / NT;
    uint64_t lw = 0;
    for (int i = 0; i < PER; ++i) { const int k = tid * PER + i; if (k < ncand) lw += sm.cw[k]; }
    uint64_t tot;
    uint64_t run = bm + block_incl_scan<uint64_t, NT>(lw, sm.u64tmp, &tot) - lw;
    if (tid == 0) sm.misc[2] = ncand - 1;
    __syncthreads();
    for (int i = 0; i < PER; ++i) {
      const int k = tid * PER + i;
      if (k >= ncand) break;
      if (run < tgt && run + sm.cw[k] >= tgt) { sm.misc[2] = k; break; }
      run += sm.cw[k];
    }
    __syncthreads();
    kb = sm.misc[2];
  } else {
    kb = (int)((int64_t)tgt - bc - 1);
  }
  r.tau = sm.cs[kb];
  int k0 = kb;
  while (k0 > 0 && sm.cs[k0 - 1] == r.tau) --k0;
  r.m = kb - k0 + 1;
  r.count = (int)bc + kb + 1;
  __syncthreads();
  return r;
}

// by_mass with rho > 0: the target is ceil(rho * total mass), the total (returned
// in *zmass) taken from the level-1 histogram (integer sums, exact).
// pre_hc: level-1 key counts of the same bins, computed earlier (count mode
// only; replaces the level-1 pass).  save_hc: where to store the level-1 counts.
__device__ Boundary find_boundary(const Sel& S, const SelSmem& sm, bool by_mass, uint64_t tgt, double rho = 0.0,
                                  uint64_t* zmass = nullptr, const int32_t* pre_hc = nullptr,
                                  int32_t* save_hc = nullptr) {
  const int tid = threadIdx.x, N = S.N;
  // ---- level 1 ------------------------------------------------------------
  if (pre_hc) {
    for (int b = tid; b < SEL_NB; b += NT) { sm.hc[b] = pre_hc[b]; sm.hm[b] = 0; }
    __syncthreads();
  } else {
    for (int b = tid; b < SEL_NB; b += NT) { sm.hc[b] = 0; sm.hm[b] = 0; }
    __syncthreads();
    each_key(S, [&](int, ushort4 z) {
      const int b1 = bin1_of(bin_x(S, logit(S, z)));
      atomicAdd(&sm.hc[b1], 1);
      if (by_mass) atomicAdd((unsigned long long*)&sm.hm[b1], (unsigned long long)weight_fx(S, z));
    });
    __syncthreads();
    if (save_hc)
      for (int b = tid; b < SEL_NB; b += NT) save_hc[b] = sm.hc[b];
  }
  if (by_mass && rho > 0.0) {
    uint64_t zl = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) zl += sm.hm[tid * BPT + i];
    const uint64_t z = block_sum<uint64_t, NT>(zl, sm.u64tmp);
    tgt = (uint64_t)ceil(rho * (double)z);
    tgt = tgt > z ? z : (tgt < 1 ? 1 : tgt);
    if (zmass) *zmass = z;
  }
  uint64_t bm;
  int64_t bc;
  const int B1 = hist_walk(sm, by_mass, tgt, 0, 0, &bm, &bc);
  const int n1 = sm.hc[B1];
  if (n1 > 0 && n1 <= 64) {
    // ---- few keys in the boundary bin: sort them directly ----------------
    if (tid == 0) sm.misc[1] = 0;
    __syncthreads();
    each_key(S, [&](int j, ushort4 z) {
      const double s = logit(S, z);
      if (bin1_of(bin_x(S, s)) != B1) return;
      const int k = atomicAdd(&sm.misc[1], 1);
      sm.cs[k] = s;
      sm.cj[k] = j;
      sm.cw[k] = by_mass ? weight_fx(S, z) : 0;
    });
    __syncthreads();
    return resolve_small_bin(sm, n1, by_mass, tgt, bm, bc);
  }
  if (n1 > 64 && n1 <= SEL_CAP) {
    // ---- at most SEL_CAP keys in the boundary bin: sort them in LDS (no level-2 pass)
    if (tid == 0) sm.misc[1] = 0;
    __syncthreads();
    each_key(S, [&](int j, ushort4 z) {
      const double s = logit(S, z);
      if (bin1_of(bin_x(S, s)) != B1) return;
      const int k = atomicAdd(&sm.misc[1], 1);
      sm.cs[k] = s;
      sm.cj[k] = j;
      sm.cw[k] = by_mass ? weight_fx(S, z) : 0;
    });
    __syncthreads();
    return resolve_lds_bin(sm, n1, by_mass, tgt, bm, bc);
  }
  // ---- level 2 ------------------------------------------------------------
  for (int b = tid; b < SEL_NB; b += NT) { sm.hc[b] = 0; sm.hm[b] = 0; }
  __syncthreads();
  each_key(S, [&](int, ushort4 z) {
    const double x = bin_x(S, logit(S, z));
    if (bin1_of(x) != B1) return;
    const int b2 = bin2_of(x, B1);
    atomicAdd(&sm.hc[b2], 1);
    if (by_mass) atomicAdd((unsigned long long*)&sm.hm[b2], (unsigned long long)weight_fx(S, z));
  });
  __syncthreads();
  const int B2 = hist_walk(sm, by_mass, tgt, bm, bc, &bm, &bc);
  const int ncand = sm.hc[B2];
  Boundary r;
  if (ncand <= SEL_CAP) {
    // ---- exact resolution: sort the boundary bin by (s desc, j asc) --------
    if (tid == 0) sm.misc[1] = 0;
    __syncthreads();
    each_key(S, [&](int j, ushort4 z) {
      const double s = logit(S, z);
      const double x = bin_x(S, s);
      if (bin1_of(x) != B1 || bin2_of(x, B1) != B2) return;
      const int k = atomicAdd(&sm.misc[1], 1);
      sm.cs[k] = s;
      sm.cj[k] = j;
      sm.cw[k] = by_mass ? weight_fx(S, z) : 0;
    });
    __syncthreads();
    r = resolve_lds_bin(sm, ncand, by_mass, tgt, bm, bc);
  } else {
    // ---- many keys in one fine bin (ties): walk its distinct logits --------
    double hi = __builtin_inf();
    for (;;) {
      double mx = -__builtin_inf();
      for (int j = tid; j < N; j += NT) {
        const double s = logit(S, S.codes[j]);
        const double x = bin_x(S, s);
        if (bin1_of(x) == B1 && bin2_of(x, B1) == B2 && s < hi) mx = fmax(mx, s);
      }
      const double g = block_max<double, NT>(mx, sm.dtmp);
      if (!(g > -__builtin_inf())) {
        // no logit left below `hi` (only if the histogram walk was inconsistent):
        // close at the previous group
        r.tau = hi;
        r.m = 0;
        r.count = (int)bc;
        break;
      }
      uint64_t gm = 0;
      int64_t gc = 0;
      for (int j = tid; j < N; j += NT) {
        const ushort4 z = S.codes[j];
        if (logit(S, z) == g) { ++gc; if (by_mass) gm += weight_fx(S, z); }
      }
      gc = block_sum<int64_t, NT>(gc, sm.i64tmp);
      gm = block_sum<uint64_t, NT>(gm, sm.u64tmp);
      const bool here = by_mass ? bm + gm >= tgt : (uint64_t)(bc + gc) >= tgt;
      if (!here) { bm += gm; bc += gc; hi = g; continue; }
      r.tau = g;
      if (!by_mass) {
        r.m = (int)((int64_t)tgt - bc);
      } else {
        // ordered walk over the keys with logit g, in index order
        int64_t rank = 0;
        uint64_t run = bm;
        int found = -1;
        for (int j0 = 0; j0 < N && found < 0; j0 += NT * 8) {
          uint64_t lw = 0;
          int64_t lc = 0;
          for (int i = 0; i < 8; ++i) {
            const int j = j0 + tid * 8 + i;
            if (j < N) { const ushort4 z = S.codes[j]; if (logit(S, z) == g) { lw += weight_fx(S, z); ++lc; } }
          }
          uint64_t totw;
          int64_t totc;
          uint64_t ew = run + block_incl_scan<uint64_t, NT>(lw, sm.u64tmp, &totw) - lw;
          int64_t ec = rank + block_incl_scan<int64_t, NT>(lc, sm.i64tmp, &totc) - lc;
          if (tid == 0) sm.misc[3] = -1;
          __syncthreads();
          if (ew < tgt && ew + lw >= tgt) {
            for (int i = 0; i < 8; ++i) {
              const int j = j0 + tid * 8 + i;
              const ushort4 z = S.codes[j];
              if (logit(S, z) != g) continue;
              ew += weight_fx(S, z);
              ++ec;
              if (ew >= tgt) { sm.misc[3] = (int)ec; break; }
            }
          }
          __syncthreads();
          found = sm.misc[3];
          run += totw;
          rank += totc;
          __syncthreads();
        }
        r.m = found > 0 ? found : (int)gc;
      }
      r.count = (int)bc + r.m;
      break;
    }
  }
  return r;
}

// Loads the cluster's LUT rows (and, for mass selection, the exp factors)
// and computes s_min / s_max over the N keys.
__device__ void setup_cluster(Sel& S, const SelArgs& a, const double* lutrow, const ushort4* codes, double* Pl,
                              double* El, bool with_mass, const SelSmem& sm) {
  const int tid = threadIdx.x, Cm = a.Cm;
  for (int i = tid; i < 3 * Cm; i += NT) Pl[i] = lutrow[i];
  __syncthreads();
  S.P0 = Pl; S.P1 = Pl + Cm; S.P2 = Pl + 2 * Cm;
  S.codes = codes;
  S.N = a.N;
  S.inv_sqrt_d = a.inv_sqrt_d;
  S.fx = a.fx_scale;
  double smax = -__builtin_inf(), smin = __builtin_inf();
  each_key(S, [&](int, ushort4 z) {
    const double s = logit(S, z);
    smax = fmax(smax, s);
    smin = fmin(smin, s);
  });
  S.smax = block_max<double, NT>(smax, sm.dtmp);
  const double lo = block_min<double, NT>(smin, sm.dtmp);
  S.scale1 = S.smax > lo ? (double)SEL_NB / (S.smax - lo) : 0.0;
  if (with_mass) {
    double A[3];
    for (int mm = 0; mm < 3; ++mm) {
      double mx = -__builtin_inf();
      for (int z = tid; z < Cm; z += NT) mx = fmax(mx, Pl[mm * Cm + z] * a.inv_sqrt_d);
      A[mm] = block_max<double, NT>(mx, sm.dtmp);
    }
    for (int i = tid; i < 3 * Cm; i += NT) El[i] = exp(Pl[i] * a.inv_sqrt_d - A[i / Cm]);
    S.E0 = El; S.E1 = El + Cm; S.E2 = El + 2 * Cm;
    S.F = exp(((A[0] + A[1]) + A[2]) - S.smax);
    __syncthreads();
  }
}

__device__ SelSmem carve_sel(unsigned char* base, int Cm, double** Pl, double** El) {
  SelSmem sm;
  size_t o = 0;
  auto take = [&](size_t bytes) { unsigned char* p = base + o; o += (bytes + 15) & ~(size_t)15; return p; };
  *Pl = reinterpret_cast<double*>(take(sizeof(double) * 3 * Cm));
  *El = reinterpret_cast<double*>(take(sizeof(double) * 3 * Cm));
  sm.hc = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * SEL_NB));
  sm.hm = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * SEL_NB));
  sm.cs = reinterpret_cast<double*>(take(sizeof(double) * SEL_CAP));
  sm.cj = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * SEL_CAP));
  sm.cw = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * SEL_CAP));
  sm.u64tmp = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * (NT / 64 + 2)));
  sm.i64tmp = reinterpret_cast<int64_t*>(take(sizeof(int64_t) * (NT / 64 + 2)));
  sm.dtmp = reinterpret_cast<double*>(take(sizeof(double) * (NT / 64 + 2)));
  sm.misc = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * 8));
  return sm;
}

static size_t sel_smem_bytes(int Cm) {
  auto r = [](size_t b) { return (b + 15) & ~(size_t)15; };
  return 2 * r(sizeof(double) * 3 * Cm) + r(4 * SEL_NB) + r(8 * SEL_NB) + r(8 * SEL_CAP) + r(4 * SEL_CAP) +
         r(8 * SEL_CAP) + 3 * r(8 * (NT / 64 + 2)) + r(32);
}

// ---------------------------------------------------------------------------
// Stage 5a: Top-p count t_c and base count b_c per (cluster, head).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void topp_kernel(SelArgs a, const double* __restrict__ lut,
                                                  const ushort4* __restrict__ codes, ClusterSel* __restrict__ csel,
                                                  int32_t* __restrict__ ct, int32_t* __restrict__ cb,
                                                  int32_t* __restrict__ hist1) {
  const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  double *Pl, *El;
  const SelSmem sm = carve_sel(smem_raw, a.Cm, &Pl, &El);
  Sel S;
  const bool take_all = a.rho >= 1.0;
  setup_cluster(S, a, lut + ((size_t)bh * a.Cq + c) * 3 * a.Cm, codes + (size_t)bh * a.N, Pl, El, !take_all, sm);
  ClusterSel st;
  st.smax = S.smax;
  st.scale1 = S.scale1;
  st.smin = 0.0;
  st.pad = 0;
  st.pad2 = 0.0;
  int t;
  if (take_all) {
    t = a.N;
    st.all = 1;
    st.tau = -__builtin_inf();
    st.m = 0;
    st.zfx = 0;
  } else {
    uint64_t z = 0;
    const Boundary b = find_boundary(S, sm, true, 0, a.rho, &z, nullptr,
                                     hist1 + ((size_t)bh * a.Cq + c) * SEL_NB);
    t = b.count;
    st.all = t >= a.N;
    st.tau = b.tau;
    st.m = b.m;
    st.zfx = z;
  }
  st.t = t;
  if (tid == 0) {
    const size_t i = (size_t)bh * a.Cq + c;
    csel[i] = st;
    ct[i] = t;
    cb[i] = max(t, a.floor_a);
  }
}

// ---------------------------------------------------------------------------
// Stage 5b: k_head (Eq. 9), r_c (Eq. 10) and the CSR offsets (r_c = b_c when
// the online per-head Top-k is switched off: the hybrid Top-p / fixed Top-k
// selection SCOPE builds on).
// khead_kernel (one workgroup per head) writes k_head, r_c, the head-local
// prefix of r_c into sel_off and the head total; seloff_scan_kernel turns the
// head totals into head offsets (and flags a capacity overflow);
// seloff_add_kernel adds them to sel_off.
// ---------------------------------------------------------------------------
constexpr int KH_NT = 256;

__global__ __launch_bounds__(KH_NT) void khead_kernel(int Cq, int N, int online, const int32_t* __restrict__ q_off,
                                                      const int32_t* __restrict__ cb, int32_t* __restrict__ cr,
                                                      int32_t* __restrict__ khead, int64_t* __restrict__ sel_off,
                                                      int64_t* __restrict__ htot) {
  __shared__ int64_t tmp[KH_NT / 64 + 1];
  const int tid = threadIdx.x, bh = blockIdx.x;
  const int32_t* qo = q_off + (size_t)bh * (Cq + 1);
  int64_t num = 0, den = 0;
  for (int c = tid; c < Cq; c += KH_NT) {
    const int64_t n = qo[c + 1] - qo[c];
    num += n * cb[(size_t)bh * Cq + c];
    den += n;
  }
  num = block_sum<int64_t, KH_NT>(num, tmp);
  den = block_sum<int64_t, KH_NT>(den, tmp);
  const int64_t kh = den > 0 ? (num + den - 1) / den : 0;
  if (tid == 0) khead[bh] = (int32_t)kh;
  int64_t base = 0;
  for (int c0 = 0; c0 < Cq; c0 += KH_NT) {
    const int c = c0 + tid;
    int64_t r = 0;
    if (c < Cq) {
      const int64_t n = qo[c + 1] - qo[c];
      const int64_t b = cb[(size_t)bh * Cq + c];
      r = n > 0 ? ((online && kh > b) ? kh : b) : 0;
      if (r > N) r = N;
      cr[(size_t)bh * Cq + c] = (int32_t)r;
    }
    int64_t tot;
    const int64_t inc = block_incl_scan<int64_t, KH_NT>(r, tmp, &tot);
    if (c < Cq) sel_off[(size_t)bh * Cq + c] = base + inc - r;
    base += tot;
  }
  if (tid == 0) htot[bh] = base;
}

__global__ __launch_bounds__(1024) void seloff_scan_kernel(int BH, int Cq, int64_t* __restrict__ htot,
                                                           int64_t* __restrict__ sel_off, int64_t capacity,
                                                           int32_t* __restrict__ status) {
  __shared__ int64_t tmp[17];
  const int tid = threadIdx.x;
  int64_t base = 0;
  for (int h0 = 0; h0 < BH; h0 += 1024) {
    const int h = h0 + tid;
    const int64_t v = h < BH ? htot[h] : 0;
    int64_t tot;
    const int64_t inc = block_incl_scan<int64_t, 1024>(v, tmp, &tot);
    if (h < BH) htot[h] = base + inc - v;   // offset of head h
    base += tot;
  }
  if (tid == 0) {
    sel_off[(size_t)BH * Cq] = base;
    status[1] = base > capacity ? 1 : 0;
  }
}

__global__ __launch_bounds__(256) void seloff_add_kernel(int Cq, const int64_t* __restrict__ htot,
                                                         int64_t* __restrict__ sel_off) {
  const int c = blockIdx.x * 256 + threadIdx.x, bh = blockIdx.y;
  if (c < Cq) sel_off[(size_t)bh * Cq + c] += htot[bh];
}

// ---------------------------------------------------------------------------
// Stage 5c: S_c = first r_c keys in (s desc, j asc) order, written in
// ascending index order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void final_select_kernel(SelArgs a, const double* __restrict__ lut,
                                                          const ushort4* __restrict__ codes,
                                                          const ClusterSel* __restrict__ csel,
                                                          const int32_t* __restrict__ cr,
                                                          const int64_t* __restrict__ sel_off,
                                                          int32_t* __restrict__ sel_idx,
                                                          const int32_t* __restrict__ status,
                                                          const int32_t* __restrict__ hist1) {
  const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const size_t ci = (size_t)bh * a.Cq + c;
  const int r = cr[ci];
  if (r == 0 || status[1]) return;
  int32_t* out = sel_idx + sel_off[ci];
  const ClusterSel st = csel[ci];
  if (st.all || r >= a.N) {
    for (int j = tid; j < a.N; j += NT) out[j] = j;
    return;
  }
  extern __shared__ __align__(16) unsigned char smem_raw[];
  double *Pl, *El;
  const SelSmem sm = carve_sel(smem_raw, a.Cm, &Pl, &El);
  const int Cm = a.Cm;
  for (int i = tid; i < 3 * Cm; i += NT) Pl[i] = lut[ci * 3 * Cm + i];
  __syncthreads();
  Sel S;
  S.P0 = Pl; S.P1 = Pl + Cm; S.P2 = Pl + 2 * Cm;
  S.codes = codes + (size_t)bh * a.N;
  S.N = a.N;
  S.inv_sqrt_d = a.inv_sqrt_d;
  S.fx = a.fx_scale;
  S.smax = st.smax;
  S.scale1 = st.scale1;
  double tau;
  int m;
  if (r == st.t) {
    tau = st.tau;
    m = st.m;
  } else {
    // same bins as the Top-p pass (smax, scale1 from csel): its level-1 counts are reused
    const Boundary b = find_boundary(S, sm, false, (uint64_t)r, 0.0, nullptr, hist1 + ci * SEL_NB);
    tau = b.tau;
    m = b.m;
  }
  // ordered compaction over chunks of NT * 8 keys: wave w takes keys
  // j0 + 512 w + 64 i + lane (i = 0..7), so the chunk's order is (wave, i,
  // lane) = index order and every store instruction writes consecutive
  // positions.  Per chunk: the ties (s == tau) before each wave, then the
  // selected keys before each wave, from per-wave counts in LDS.
  constexpr int KI = 8;
  const int lane = tid & 63, wv = tid >> 6;
  int32_t* wcnt = sm.misc;   // [NT / 64] per-wave counts (misc has room for 8)
  static_assert(NT / 64 <= 8, "per-wave counts fit sm.misc");
  int64_t selBase = 0, tieBase = 0;
  __syncthreads();   // the boundary search's results in sm.misc are read by every thread
  for (int j0 = 0; j0 < a.N; j0 += NT * KI) {
    uint64_t gtm[KI], eqm[KI];
    int wgt = 0, weq = 0;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int j = j0 + wv * 64 * KI + i * 64 + lane;
      bool g = false, e = false;
      if (j < a.N) {
        const double sj = logit(S, S.codes[j]);
        g = sj > tau;
        e = sj == tau;
      }
      gtm[i] = __ballot(g);
      eqm[i] = __ballot(e);
      wgt += __popcll(gtm[i]);
      weq += __popcll(eqm[i]);
    }
    // ties before this wave
    if (lane == 0) wcnt[wv] = weq;
    __syncthreads();
    int64_t exTie = tieBase, totTie = 0;
    for (int w2 = 0; w2 < NT / 64; ++w2) {
      const int v = wcnt[w2];
      if (w2 < wv) exTie += v;
      totTie += v;
    }
    __syncthreads();
    int64_t take = (int64_t)m - exTie;
    take = take < 0 ? 0 : (take > weq ? weq : take);
    // selected keys before this wave
    if (lane == 0) wcnt[wv] = wgt + (int)take;
    __syncthreads();
    int64_t pos = selBase, totSel = 0;
    for (int w2 = 0; w2 < NT / 64; ++w2) {
      const int v = wcnt[w2];
      if (w2 < wv) pos += v;
      totSel += v;
    }
    __syncthreads();
    int64_t tr = exTie;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const uint64_t below = (1ull << lane) - 1ull;
      const bool e = (eqm[i] >> lane) & 1ull;
      const bool take1 = ((gtm[i] >> lane) & 1ull) || (e && tr + __popcll(eqm[i] & below) < m);
      const uint64_t sm1 = __ballot(take1);
      const int64_t p = pos + __popcll(sm1 & below);
      if (take1 && p < r) out[p] = j0 + wv * 64 * KI + i * 64 + lane;
      pos += __popcll(sm1);
      tr += __popcll(eqm[i]);
    }
    selBase += totSel;
    tieBase += totTie;
  }
}

// ---------------------------------------------------------------------------
// Attention work list: one item per (cluster, 128-query chunk), cluster-major
// in (head, cluster) order; one workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void worklist_kernel(int BH, int Cq, int chunk, const int32_t* __restrict__ q_off,
                                                        const int32_t* __restrict__ cr, int32_t* __restrict__ work,
                                                        int64_t cap, int32_t* __restrict__ status) {
  __shared__ int64_t tmp[17];
  const int tid = threadIdx.x;
  const int64_t total = (int64_t)BH * Cq;
  int64_t base = 0;
  for (int64_t i0 = 0; i0 < total; i0 += 1024) {
    const int64_t i = i0 + tid;
    int64_t items = 0;
    if (i < total) {
      const int bh = (int)(i / Cq), c = (int)(i % Cq);
      const int n = q_off[(size_t)bh * (Cq + 1) + c + 1] - q_off[(size_t)bh * (Cq + 1) + c];
      items = (cr[i] > 0 && n > 0) ? (n + chunk - 1) / chunk : 0;
    }
    int64_t tot;
    int64_t pos = base + block_incl_scan<int64_t, 1024>(items, tmp, &tot) - items;
    for (int64_t k = 0; k < items && pos + k < cap; ++k) {
      work[2 * (pos + k)] = (int32_t)i;
      work[2 * (pos + k) + 1] = (int32_t)k;
    }
    base += tot;
  }
  if (tid == 0) status[0] = (int32_t)(base < cap ? base : cap);
}

// ---------------------------------------------------------------------------
// Dense attention (SCOPE_DENSE): the plan in which every query attends to all
// keys of its head.  Cluster 0 of each head holds the N queries in token
// order and the key set 0..N-1 (r_0 = t_0 = b_0 = k_head = N); the other
// clusters are empty.  Grid (ceil(N / 256), BH).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dense_plan_kernel(int BH, int N, int Cq, int32_t* __restrict__ perm_q,
                                                         int32_t* __restrict__ q_off, int32_t* __restrict__ ct,
                                                         int32_t* __restrict__ cb, int32_t* __restrict__ cr,
                                                         int32_t* __restrict__ khead, int64_t* __restrict__ sel_off,
                                                         int32_t* __restrict__ sel_idx, int64_t capacity,
                                                         int32_t* __restrict__ status) {
  const int bh = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  const bool fits = (int64_t)BH * N <= capacity;
  if (i < N) {
    perm_q[(size_t)bh * N + i] = i;
    if (fits) sel_idx[(size_t)bh * N + i] = i;
  }
  if (blockIdx.x == 0) {
    for (int c = threadIdx.x; c <= Cq; c += 256) q_off[(size_t)bh * (Cq + 1) + c] = c == 0 ? 0 : N;
    for (int c = threadIdx.x; c < Cq; c += 256) {
      const int v = c == 0 ? N : 0;
      ct[(size_t)bh * Cq + c] = v;
      cb[(size_t)bh * Cq + c] = v;
      cr[(size_t)bh * Cq + c] = v;
      sel_off[(size_t)bh * Cq + c] = (int64_t)bh * N + (c == 0 ? 0 : N);
    }
    if (threadIdx.x == 0) {
      khead[bh] = N;
      if (bh == BH - 1) {
        sel_off[(size_t)BH * Cq] = (int64_t)BH * N;
        status[1] = fits ? 0 : 1;
        status[2] = 0;
      }
    }
  }
}

// ---- launchers ----------------------------------------------------------------

hipError_t launch_dense_plan(const Geo& g, const scope_plan_t& plan, hipStream_t s) {
  dense_plan_kernel<<<dim3((g.N + 255) / 256, g.BH), 256, 0, s>>>(
      g.BH, g.N, g.Cq, plan.perm_q, plan.q_off, plan.counts_t, plan.counts_b, plan.counts_r, plan.k_head,
      plan.sel_off, plan.sel_idx, plan.sel_capacity, plan.status);
  return hipGetLastError();
}

static SelArgs sel_args(const Geo& g, const scope_params& p) {
  SelArgs a;
  a.N = g.N; a.Cq = g.Cq; a.Cm = g.Cm;
  a.inv_sqrt_d = 1.0 / sqrt((double)g.d);
  a.rho = p.rho;
  int lg = 0;
  while ((1ll << lg) < (int64_t)g.N + 1) ++lg;
  a.fx_scale = ldexp(1.0, 62 - lg);
  a.floor_a = (int)ceil(p.alpha * (double)g.N);
  return a;
}

static void allow_big_lds(const void* fn, size_t bytes) {
  if (bytes > 64 * 1024) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_lut(const Geo& g, const Workspace& w, hipStream_t s) {
  lut_kernel<<<dim3(g.Cq, g.BH), 256, 0, s>>>(g, w.qcent, w.kcent, w.lut);
  return hipGetLastError();
}

hipError_t launch_topp(const Geo& g, const scope_params& p, const Workspace& w, int32_t* ct, int32_t* cb,
                       hipStream_t s) {
  const size_t lds = sel_smem_bytes(g.Cm);
  allow_big_lds((const void*)topp_kernel, lds);
  topp_kernel<<<dim3(g.Cq, g.BH), NT, lds, s>>>(sel_args(g, p), w.lut, (const ushort4*)w.codes, w.csel, ct, cb,
                                                 w.hist1);
  return hipGetLastError();
}

hipError_t launch_khead(const Geo& g, const scope_plan_t& plan, const Workspace& w, hipStream_t s) {
  khead_kernel<<<g.BH, KH_NT, 0, s>>>(g.Cq, g.N, g.online_khead, plan.q_off, plan.counts_b, plan.counts_r, plan.k_head, plan.sel_off,
                                      w.htot);
  seloff_scan_kernel<<<1, 1024, 0, s>>>(g.BH, g.Cq, w.htot, plan.sel_off, plan.sel_capacity, plan.status);
  seloff_add_kernel<<<dim3((g.Cq + 255) / 256, g.BH), 256, 0, s>>>(g.Cq, w.htot, plan.sel_off);
  return hipGetLastError();
}

hipError_t launch_final_select(const Geo& g, const scope_params& p, const Workspace& w,
                               const scope_plan_t& plan, hipStream_t s) {
  const size_t lds = sel_smem_bytes(g.Cm);
  allow_big_lds((const void*)final_select_kernel, lds);
  final_select_kernel<<<dim3(g.Cq, g.BH), NT, lds, s>>>(sel_args(g, p), w.lut, (const ushort4*)w.codes, w.csel,
                                                        plan.counts_r, plan.sel_off, plan.sel_idx, plan.status,
                                                        w.hist1);
  return hipGetLastError();
}

hipError_t launch_worklist(const Geo& g, const scope_plan_t& plan, hipStream_t s) {
  worklist_kernel<<<1, 1024, 0, s>>>(g.BH, g.Cq, att_chunk(g), plan.q_off, plan.counts_r, plan.work, plan.work_capacity,
                                      plan.status);
  return hipGetLastError();
}

}  // namespace scope
