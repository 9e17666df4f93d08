// Stage 2: k-means of the post-RoPE queries (Cq clusters, full d) and of the
// post-RoPE keys restricted to each 3D-RoPE channel range T, H, W (Cm
// centroids each), the per-subspace clustering of SCOPE's Eq. (3) (Euclidean
// reconstruction objective; pith.science review of arXiv 2608.12780).
// Procedure: seeded k-means++ followed by Lloyd rounds
//   labels_0 = assign(init); for it in 1..iters: mu = mean(labels); labels = assign(mu).
//
// Exactness.  bf16 data makes every k-means++ squared distance and every
// centroid sum exactly representable in fp64 for data of ordinary range, so
// the fp64 arithmetic below is order-independent; the MFMA assignment is a
// filter whose near-ties are re-decided with exact fp64 distances.
#include <float.h>

#include "scope_device.hpp"
#include "scope_internal.hpp"

namespace scope {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

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

// First index of a length-n sequence whose running sum (starting at `base`)
// exceeds `target`; executed by one whole wave.  Returns -1 if none, and the
// running sum before that index in *excl.
template <typename F>
__device__ int wave_crossing(F val, int n, double base, double target, double* excl) {
  const int lane = threadIdx.x & 63;
  double run = base;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const bool in = c0 + lane < n;
    const double v = in ? val(c0 + lane) : 0.0;
    const double inc = wave_incl_scan(v);
    const uint64_t hit = __ballot(in && run + inc > target);
    if (hit) {
      const int L = __ffsll((unsigned long long)hit) - 1;
      const double prev = __shfl(inc, L > 0 ? L - 1 : 0);
      *excl = run + (L > 0 ? prev : 0.0);
      return c0 + L;
    }
    run += __shfl(inc, 63);
  }
  *excl = run;
  return -1;
}

// Last index of a length-n sequence with a positive value (one wave), or -1.
template <typename F>
__device__ int wave_last_positive(F val, int n) {
  const int lane = threadIdx.x & 63;
  for (int c0 = ((n - 1) / 64) * 64; c0 >= 0; c0 -= 64) {
    const bool in = c0 + lane < n;
    const uint64_t hit = __ballot(in && val(c0 + lane) > 0.0);
    if (hit) return c0 + 63 - __clzll((long long)hit);
  }
  return -1;
}

// ---------------------------------------------------------------------------
// k-means++ seeding (Arthur and Vassilvitskii 2007): one workgroup per
// (head, clustering).  Centre 0 = floor(u_0 N); centre s = smallest i whose
// running sum of D^2 exceeds u_s * sum(D^2).  Running sums are taken over
// 64-point blocks and 64-block super-blocks.  The D^2 update skips a point x
// when its current centre a and the new centre c satisfy
// ||c - a||^2 >= 4 D^2(x) (triangle inequality, Elkan ICML 2003): then
// ||x - c|| >= D(x) and D^2(x) cannot change, so the result equals the
// unpruned update.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(1024) void seed_kernel(const T* __restrict__ qr, const T* __restrict__ kr, Geo g,
                                                    double* __restrict__ d2all, int32_t* __restrict__ nearall,
                                                    double* __restrict__ bsumall, int32_t* __restrict__ seeds,
                                                    float* __restrict__ qcent, float* __restrict__ kcent) {
  const int m = blockIdx.y, bh = blockIdx.x;
  const int N = g.N, d = g.d, dm = g.dm[m], off = g.off[m], C = g.C[m];
  const int NB = (N + 63) / 64, NS = (NB + 63) / 64;
  const T* X = (m == 0 ? qr : kr) + (size_t)bh * N * d + off;
  double* D2 = d2all + ((size_t)bh * 4 + m) * N;
  int32_t* nearest = nearall + ((size_t)bh * 4 + m) * N;
  double* bsum = bsumall + ((size_t)bh * 4 + m) * NB;
  int32_t* sd = seeds + ((size_t)bh * 4 + m) * g.Cmax;

  __shared__ double cvec[128];
  __shared__ double cc[MAX_C];
  __shared__ int32_t chosen[MAX_C];
  __shared__ double sbs[256];
  __shared__ int sh_i;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint64_t stream = ((uint64_t)bh * 4 + m) << 20;

  for (int s = 0; s < C; ++s) {
    // ---- choose centre s -------------------------------------------------
    if (wv == 0) {
      int pick = -1;
      if (s == 0) {
        const uint64_t k0 = splitmix64(g.seed, stream) >> 11;
        const uint64_t lo = k0 * (uint64_t)N, hi = __umul64hi(k0, (uint64_t)N);
        pick = (int)((hi << 11) | (lo >> 53));
      } else {
        double total;
        wave_crossing([&](int k) { return sbs[k]; }, NS, 0.0, __builtin_inf(), &total);
        if (total == 0.0) {
          // every remaining point coincides with a centre: lowest index not chosen yet
          for (int c0 = 0; c0 < N && pick < 0; c0 += 64) {
            const uint64_t free_ = __ballot(c0 + lane < N && !(nearest[c0 + lane] & CENTRE_MARK));
            if (free_) pick = c0 + __ffsll((unsigned long long)free_) - 1;
          }
        } else {
          const uint64_t ku = splitmix64(g.seed, stream + (uint64_t)s) >> 11;
          const double target = ((double)ku * 0x1p-53) * total;
          double e2, e1, e0;
          const int K = wave_crossing([&](int k) { return sbs[k]; }, NS, 0.0, target, &e2);
          if (K >= 0) {
            const int nb = min(64, NB - K * 64);
            // rounding may leave the crossing just past a group: then take the
            // group's last point with positive weight
            int B = wave_crossing([&](int k) { return bsum[K * 64 + k]; }, nb, e2, target, &e1);
            const bool lastb = B < 0;
            if (lastb) B = wave_last_positive([&](int k) { return bsum[K * 64 + k]; }, nb);
            B += K * 64;
            const int np = min(64, N - B * 64);
            int i = lastb ? -1 : wave_crossing([&](int k) { return D2[B * 64 + k]; }, np, e1, target, &e0);
            if (i < 0) i = wave_last_positive([&](int k) { return D2[B * 64 + k]; }, np);
            pick = B * 64 + i;
          } else {
            pick = wave_last_positive([&](int k) { return D2[k]; }, N);
          }
        }
      }
      if (lane == 0) sh_i = pick < 0 ? 0 : (pick >= N ? N - 1 : pick);
    }
    __syncthreads();
    const int ci = sh_i;
    if (tid == 0) { chosen[s] = ci; sd[s] = ci; }
    if (tid < dm) cvec[tid] = Elem<T>::ld(X + (size_t)ci * d + tid);
    __syncthreads();
    // ---- squared distances from the new centre to the previous ones ------
    for (int a = tid; a < s; a += 1024) cc[a] = sqdist_row(X + (size_t)chosen[a] * d, cvec, dm);
    __syncthreads();
    // ---- D^2 update, one 64-point block per wave --------------------------
    for (int b = wv; b < NB; b += 16) {
      const int p = b * 64 + lane;
      double v = 0.0;
      if (p < N) {
        if (s == 0) {
          v = sqdist_row(X + (size_t)p * d, cvec, dm);
          D2[p] = v;
          nearest[p] = 0;
        } else {
          v = D2[p];
          const int a = nearest[p] & 0xFFFF;
          if (!(cc[a] * (1.0 - 1e-9) >= 4.0 * v)) {
            const double dist = sqdist_row(X + (size_t)p * d, cvec, dm);
            if (dist < v) {
              v = dist;
              D2[p] = dist;
              nearest[p] = s;
            }
          }
        }
      }
      v = wave_sum(v);
      if (lane == 0) bsum[b] = v;
    }
    __syncthreads();
    if (tid == 0) nearest[ci] |= CENTRE_MARK;
    for (int K = wv; K < NS; K += 16) {
      const double v = K * 64 + lane < NB ? bsum[K * 64 + lane] : 0.0;
      const double t = wave_sum(v);
      if (lane == 0) sbs[K] = t;
    }
    __syncthreads();
  }
  // ---- initial centroids = the chosen points ------------------------------
  for (int idx = tid; idx < C * dm; idx += 1024) {
    const int c = idx / dm, ch = idx % dm;
    const float val = Elem<T>::ldf(X + (size_t)chosen[c] * d + ch);
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

// ---------------------------------------------------------------------------
// Assignment, bf16: MFMA filter + fp64 refinement.
// Each wave takes 64 points as two 32-column tiles; the WG's 256 points share
// the clustering's centroids in LDS.  v_mfma_f32_32x32x16_bf16 gives
// dot(x, mu~_c) for 32 centroids x 32 points; dhat_c = ||mu~_c||^2 - 2 dot.
// If the two smallest dhat of a point lie within the worst-case rounding
// window of each other, the point is queued for exact fp64 refinement.
// ---------------------------------------------------------------------------
constexpr int ASG_PTS = 256;

__global__ __launch_bounds__(256) void assign_bf16_kernel(const uint16_t* __restrict__ qr,
                                                          const uint16_t* __restrict__ kr, Geo g,
                                                          const uint16_t* __restrict__ cbf,
                                                          const float* __restrict__ cnorm,
                                                          int32_t* __restrict__ labels, int32_t* __restrict__ rlist,
                                                          int32_t* __restrict__ rcnt) {
  const int m = blockIdx.y, bh = blockIdx.z;
  const int N = g.N, d = g.d, dm = g.dm[m], off = g.off[m], C = g.C[m], Cpad = g.Cpad[m], dpad = g.dpad[m];
  const int KB = dpad / 16, ldc = dpad + 8;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint16_t* sc = reinterpret_cast<uint16_t*>(smem_raw);
  float* scn = reinterpret_cast<float*>(smem_raw + (size_t)Cpad * ldc * 2);
  __shared__ float red[8];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hi = lane >> 5, col = lane & 31;
  const uint16_t* gc = cbf + ((size_t)bh * 4 + m) * g.CmaxPad * g.DPmax;
  for (int idx = tid; idx < Cpad * (dpad / 8); idx += 256) {
    const int r = idx / (dpad / 8), c8 = idx % (dpad / 8);
    *reinterpret_cast<uint4*>(sc + r * ldc + c8 * 8) =
        *reinterpret_cast<const uint4*>(gc + (size_t)r * g.DPmax + c8 * 8);
  }
  const float* gcn = cnorm + ((size_t)bh * 4 + m) * g.CmaxPad;
  float mx = 0.f;
  for (int idx = tid; idx < Cpad; idx += 256) {
    const float v = gcn[idx];
    scn[idx] = v;
    if (idx < C) mx = fmaxf(mx, v);
  }
  mx = block_max<float, 256>(mx, red);   // also orders the LDS fills above
  const float M = sqrtf(mx) * 1.0001f;

  // point operands: tile t, k-block kb -> 8 bf16 channels kb*16 + hi*8 + 0..7
  const uint16_t* X = (m == 0 ? qr : kr) + (size_t)bh * N * d + off;
  bf16x8_t b[2][8];
  float xn2[2] = {0.f, 0.f};
  int pts[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int p = blockIdx.x * ASG_PTS + wv * 64 + t * 32 + col;
    pts[t] = p;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      uint16_t e[8];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const int ch = kb * 16 + hi * 8 + j;
        uint32_t two = 0;
        if (kb < KB && p < N && ch < dm) two = *reinterpret_cast<const uint32_t*>(X + (size_t)p * d + ch);
        e[j] = (uint16_t)(two & 0xFFFF);
        e[j + 1] = (uint16_t)(two >> 16);
        const float f0 = bf16_to_f32(e[j]), f1 = bf16_to_f32(e[j + 1]);
        xn2[t] += f0 * f0 + f1 * f1;
      }
      b[t][kb] = *reinterpret_cast<bf16x8_t*>(e);
    }
  }

  float best[2] = {FLT_MAX, FLT_MAX}, second[2] = {FLT_MAX, FLT_MAX};
  int bi[2] = {0, 0};
  for (int cb = 0; cb < Cpad / 32; ++cb) {
    f32x16_t acc0 = {}, acc1 = {};
    const uint16_t* arow = sc + (cb * 32 + col) * ldc + hi * 8;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      if (kb < KB) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(arow + kb * 16);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[0][kb], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[1][kb], acc1, 0, 0, 0);
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int c = cb * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
      const float cn = scn[c];
      const float d0 = fmaf(-2.f, acc0[v], cn), d1 = fmaf(-2.f, acc1[v], cn);
      if (d0 < best[0]) { second[0] = best[0]; best[0] = d0; bi[0] = c; }
      else if (d0 < second[0]) second[0] = d0;
      if (d1 < best[1]) { second[1] = best[1]; best[1] = d1; bi[1] = c; }
      else if (d1 < second[1]) second[1] = d1;
    }
  }
  const float gamma = (float)(dpad + 16) * 0x1p-23f;
  int32_t* lab = labels + ((size_t)bh * 4 + m) * N;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    // merge the two half-waves holding the same point
    const float ob = __shfl_xor(best[t], 32), os = __shfl_xor(second[t], 32);
    const int oi = __shfl_xor(bi[t], 32);
    float bb, ss;
    int ii;
    if (best[t] < ob || (best[t] == ob && bi[t] < oi)) { bb = best[t]; ii = bi[t]; ss = fminf(second[t], ob); }
    else { bb = ob; ii = oi; ss = fminf(os, best[t]); }
    const float xn = sqrtf(xn2[t] + __shfl_xor(xn2[t], 32)) * 1.0001f;
    const float eps = gamma * 2.f * xn * M + 0x1p-22f * (M * M + 2.f * xn * M);
    const int p = pts[t];
    if (hi == 0 && p < N) {
      lab[p] = ii;
      if (ss - bb <= 4.f * eps) {
        const int slot = atomicAdd(&rcnt[bh * 4 + m], 1);
        rlist[((size_t)bh * 4 + m) * N + slot] = p;
      }
    }
  }
}

// Exact fp64 re-decision of queued points: one wave per point, lanes over
// centroids, ||x - mu~_c||^2 in difference form, ties to the lowest c.
__global__ __launch_bounds__(256) void refine_kernel(const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr,
                                                     Geo g, const uint16_t* __restrict__ cbf,
                                                     int32_t* __restrict__ labels, const int32_t* __restrict__ rlist,
                                                     const int32_t* __restrict__ rcnt) {
  const int m = blockIdx.y, bh = blockIdx.z;
  const int N = g.N, d = g.d, dm = g.dm[m], off = g.off[m], C = g.C[m];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __shared__ double xs[4][128];
  const int cnt = rcnt[bh * 4 + m];
  const uint16_t* X = (m == 0 ? qr : kr) + (size_t)bh * N * d + off;
  const uint16_t* cb = cbf + ((size_t)bh * 4 + m) * g.CmaxPad * g.DPmax;
  for (int e = blockIdx.x * 4 + wv; e < cnt; e += gridDim.x * 4) {
    const int p = rlist[((size_t)bh * 4 + m) * N + e];
    for (int ch = lane; ch < dm; ch += 64) xs[wv][ch] = (double)bf16_to_f32(X[(size_t)p * d + ch]);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    double best = __builtin_inf();
    int bi = 0x7FFFFFFF;
    for (int c = lane; c < C; c += 64) {
      double acc = 0.0;
      const uint16_t* row = cb + (size_t)c * g.DPmax;
      for (int ch = 0; ch < dm; ++ch) {
        const double df = xs[wv][ch] - (double)bf16_to_f32(row[ch]);
        acc += df * df;
      }
      if (acc < best) { best = acc; bi = c; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const double ob = __shfl_xor(best, o);
      const int oi = __shfl_xor(bi, o);
      if (ob < best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
    if (lane == 0) labels[((size_t)bh * 4 + m) * N + p] = bi;
    __builtin_amdgcn_wave_barrier();
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
  for (int p = s0 + lane; p < s1; p += 64) atomicAdd(&hist[wv][lab[p]], 1);
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
  for (int c0 = s0; c0 < s1; c0 += 64) {
    const int p = c0 + lane;
    const int L = p < s1 ? lab[p] : -1;
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
// Lloyd update: one workgroup per (cluster, clustering, head) sums its
// members' rows (in the order of the stable sort), divides by the count in
// fp64, rounds to fp32, and refreshes the bf16 copy and its squared norm.
// Thread (group, octet) accumulates channels octet*8 .. +7 of members
// group, group + G, ...; groups are combined in a fixed order.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void segsum_kernel(const T* __restrict__ qr, const T* __restrict__ kr, Geo g,
                                                     const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ off, float* __restrict__ qcent,
                                                     float* __restrict__ kcent, uint16_t* __restrict__ cbf,
                                                     float* __restrict__ cnorm) {
  const int c = blockIdx.x, m = blockIdx.y, bh = blockIdx.z;
  if (c >= g.C[m]) return;
  const int N = g.N, d = g.d, dm = g.dm[m], doff = g.off[m], dpad = g.dpad[m];
  const int OCT = dpad / 8, G = 256 / OCT;
  const int tid = threadIdx.x, oct = tid % OCT, grp = tid / OCT;
  __shared__ double part[256 * 8];
  __shared__ double nrm_s[4];
  const int32_t* of = off + ((size_t)bh * 4 + m) * (g.Cmax + 1);
  const int a = of[c], b = of[c + 1], cnt = b - a;
  float* row = m == 0 ? qcent + ((size_t)bh * g.Cq + c) * d : kcent + ((size_t)bh * g.Cm + c) * d + doff;
  if (cnt > 0) {
    const int32_t* pm = perm + ((size_t)bh * 4 + m) * N + a;
    const T* X = (m == 0 ? qr : kr) + (size_t)bh * N * d + doff + oct * 8;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (grp < G) {
      for (int k = grp; k < cnt; k += G) {
        const T* x = X + (size_t)pm[k] * d;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (oct * 8 + j < dm) acc[j] += Elem<T>::ld(x + j);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) part[tid * 8 + j] = acc[j];
    __syncthreads();
    for (int ch = tid; ch < dm; ch += 256) {
      const int o = ch / 8, j = ch % 8;
      double s = 0.0;
      for (int gg = 0; gg < G; ++gg) s += part[(gg * OCT + o) * 8 + j];
      row[ch] = (float)(s / (double)cnt);
    }
    __syncthreads();
  }
  // bf16 copy and squared norm of the (possibly unchanged) centroid
  uint16_t* cb = cbf + (((size_t)bh * 4 + m) * g.CmaxPad + c) * g.DPmax;
  double nrm = 0.0;
  for (int ch = tid; ch < dm; ch += 256) {
    const uint16_t bv = f32_to_bf16(row[ch]);
    cb[ch] = bv;
    const double f = (double)bf16_to_f32(bv);
    nrm += f * f;
  }
  nrm = block_sum<double, 256>(nrm, nrm_s);
  if (tid == 0) cnorm[((size_t)bh * 4 + m) * g.CmaxPad + c] = (float)nrm;
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
  c.y = (uint16_t)l[2 * (size_t)g.N];
  c.z = (uint16_t)l[3 * (size_t)g.N];
  c.w = 0;
  reinterpret_cast<ushort4*>(codes)[i] = c;
  qlab[i] = l[0];
  if (qlab_out) qlab_out[i] = l[0];
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---- launchers --------------------------------------------------------------

hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s) {
  if (n) fill_i32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, v, n);
  return hipGetLastError();
}

hipError_t launch_seed(const Geo& g, const void* qr, const void* kr, const Workspace& w, hipStream_t s) {
  dim3 grid(g.BH, 4);
  if (g.bf16)
    seed_kernel<uint16_t><<<grid, 1024, 0, s>>>((const uint16_t*)qr, (const uint16_t*)kr, g, w.d2, w.nearest,
                                                w.bsum, w.seeds, w.qcent, w.kcent);
  else
    seed_kernel<float><<<grid, 1024, 0, s>>>((const float*)qr, (const float*)kr, g, w.d2, w.nearest, w.bsum,
                                             w.seeds, w.qcent, w.kcent);
  return hipGetLastError();
}

hipError_t launch_prep(const Geo& g, const Workspace& w, hipStream_t s) {
  centroid_kernel<<<dim3(4, g.BH), 256, 0, s>>>(g, w.qcent, w.kcent, w.cbf, w.cnorm);
  return hipGetLastError();
}

hipError_t launch_assign(const Geo& g, const void* qr, const void* kr, const Workspace& w, int iter,
                         hipStream_t s) {
  int32_t* rcnt = w.rcnt + (size_t)iter * g.BH * 4;
  if (g.bf16) {
    int maxpad = 0;
    for (int m = 0; m < 4; ++m) maxpad = max(maxpad, g.Cpad[m] * (g.dpad[m] + 8) * 2 + g.Cpad[m] * 4);
    dim3 grid((g.N + ASG_PTS - 1) / ASG_PTS, 4, g.BH);
    if (maxpad > 64 * 1024)
      (void)hipFuncSetAttribute((const void*)assign_bf16_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, maxpad);
    assign_bf16_kernel<<<grid, 256, maxpad, s>>>((const uint16_t*)qr, (const uint16_t*)kr, g, w.cbf, w.cnorm,
                                                w.labels, w.rlist, rcnt);
    refine_kernel<<<dim3(64, 4, g.BH), 256, 0, s>>>((const uint16_t*)qr, (const uint16_t*)kr, g, w.cbf, w.labels,
                                                    w.rlist, rcnt);
  } else {
    dim3 grid((g.N + 255) / 256, 4, g.BH);
    assign_exact_f32_kernel<<<grid, 256, 0, s>>>((const float*)qr, (const float*)kr, g, w.qcent, w.kcent, w.labels);
  }
  return hipGetLastError();
}

hipError_t launch_sort(const Geo& g, const Workspace& w, hipStream_t s) {
  sort_kernel<<<dim3(4, g.BH), 1024, 0, s>>>(g, w.labels, 0, w.perm, (int64_t)4 * g.N, g.N, w.off,
                                             (int64_t)4 * (g.Cmax + 1), g.Cmax + 1);
  return hipGetLastError();
}

hipError_t launch_update(const Geo& g, const void* qr, const void* kr, const Workspace& w, hipStream_t s) {
  hipError_t e = launch_sort(g, w, s);
  if (e != hipSuccess) return e;
  dim3 grid(g.Cmax, 4, g.BH);
  if (g.bf16)
    segsum_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)qr, (const uint16_t*)kr, g, w.perm, w.off,
                                                 w.qcent, w.kcent, w.cbf, w.cnorm);
  else
    segsum_kernel<float><<<grid, 256, 0, s>>>((const float*)qr, (const float*)kr, g, w.perm, w.off, w.qcent,
                                              w.kcent, w.cbf, w.cnorm);
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
