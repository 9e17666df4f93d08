// Stage 1: 3D rotary position embedding of Q and K, fused with the cast to the
// storage type.  The head channels are the concatenation of the temporal,
// height and width ranges of 3D RoPE (the ranges SCOPE's key subspaces follow,
// per the SCOPE abstract); inside a range of width d_m at offset o, channel
// pair (o+2i, o+2i+1) of token (t, h, w) rotates by p * base^(-2i/d_m), with
// p the token's t, h or w index.  The rotation is evaluated in fp64 and
// rounded once to bf16 or fp32.  HBM-bound: 2 tensors x (read + write).
#include "scope_device.hpp"
#include "scope_internal.hpp"

namespace scope {

struct RopeArgs {
  int BH, N, d, Hg, Wg;
  int off1, off2;               // start of the H and W ranges
  int dm[3], toff[3];
  uint64_t mhw, mw;             // ceil(2^32 / (Hg Wg)), ceil(2^32 / Wg): n / x = (n * m) >> 32 for n x < 2^32
  int magic;                    // the token count allows that division
};

__global__ void rope_table_kernel(double2* tab, int n0, int n1, int n2, int dm0, int dm1, int dm2,
                                  double base, int32_t* range_flag) {
  int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx == 0) *range_flag = 0;   // set again below by rope_kernel if needed
  if (idx >= n0 + n1 + n2) return;
  int r = idx, dm = dm0;
  if (r >= n0) { r -= n0; dm = dm1; if (r >= n1) { r -= n1; dm = dm2; } }
  const int half = dm / 2, p = r / half, i = r % half;
  const double theta = pow(base, -(2.0 * i) / dm);
  double sn, cs;
  sincos((double)p * theta, &sn, &cs);
  tab[idx] = make_double2(cs, sn);
}

template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {
  uint16_t v[8];
  __device__ void load(const uint16_t* p) { *reinterpret_cast<uint4*>(v) = *reinterpret_cast<const uint4*>(p); }
  __device__ void store(uint16_t* p) const { *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(v); }
};
template <> struct Vec8<float> {
  float v[8];
  __device__ void load(const float* p) {
    *reinterpret_cast<float4*>(v) = *reinterpret_cast<const float4*>(p);
    *reinterpret_cast<float4*>(v + 4) = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ void store(float* p) const {
    *reinterpret_cast<float4*>(p) = *reinterpret_cast<const float4*>(v);
    *reinterpret_cast<float4*>(p + 4) = *reinterpret_cast<const float4*>(v + 4);
  }
};

// Round the 8 fp64 results to the storage type.  bf16: round to nearest even
// at mantissa bit 45 of the fp64 value (then exact as fp32), which is correct
// for every result of magnitude >= 2^-126 or zero; a wave with any other
// result takes the general conversion for all its values.
__device__ __forceinline__ void store_rounded(Vec8<float>& x, const double (&y)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) x.v[i] = (float)y[i];
}
__device__ __forceinline__ void store_rounded(Vec8<uint16_t>& x, const double (&y)[8]) {
  bool odd = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint64_t u = (uint64_t)__double_as_longlong(y[i]);
    u += 0x0FFFFFFFFFFFull + ((u >> 45) & 1ull);
    u &= ~0x1FFFFFFFFFFFull;
    x.v[i] = (uint16_t)(__float_as_uint((float)__longlong_as_double((long long)u)) >> 16);
    odd |= !(fabs(y[i]) >= 0x1p-126) && y[i] != 0.0;
  }
  if (__ballot(odd)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x.v[i] = f64_to_bf16(y[i]);
  }
}

// One thread rotates 8 consecutive channels (4 pairs) of one token of Q or K,
// for ROPE_R chunks: sub-block k of the workgroup's ROPE_R * 256 chunks; the
// loads of all ROPE_R chunks are issued before any is processed.
// Grid: x over the tokens x (d/8) chunks of one head, y over heads, z over Q / K, so
// all index arithmetic is 32-bit (d/8 is 8 or 16: a shift).  For K, knm (if set)
// receives an upper bound of the head's largest ||k'|| over the stored
// (rounded) rows: the fp32 norm times 1 + 2^-12 (which covers the rounding of
// the fp32 sum and the square root), as float bits via atomicMax (zeroed
// beforehand; non-negative floats order like their bits).
constexpr int ROPE_R = 4;
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   T* __restrict__ qo, T* __restrict__ ko,
                                                   const double2* __restrict__ tab, RopeArgs a,
                                                   uint32_t* __restrict__ knm, int32_t* __restrict__ range_flag) {
  __shared__ float red[256 / 64];
  const int cshift = a.d == 128 ? 4 : 3;
  const int sel = blockIdx.z, bh = blockIdx.y;
  const int hw = a.Hg * a.Wg;
  const int nchunk = a.N << cshift;
  Vec8<T> x[ROPE_R];
  size_t base[ROPE_R];
  int rr[ROPE_R];
#pragma unroll
  for (int kk = 0; kk < ROPE_R; ++kk) {
    const int r0 = (blockIdx.x * ROPE_R + kk) * 256 + threadIdx.x;   // token * (d/8) + chunk
    rr[kk] = r0 < nchunk ? r0 : -1;
    const int r = r0 < nchunk ? r0 : 0;
    base[kk] = ((size_t)bh * a.N + (r >> cshift)) * a.d + (r & ((1 << cshift) - 1)) * 8;
    x[kk].load((sel ? k : q) + base[kk]);
  }
  float mx = 0.f;
#pragma unroll
  for (int kk = 0; kk < ROPE_R; ++kk) {
    const bool valid = rr[kk] >= 0;
    const int r = valid ? rr[kk] : 0;
    const int chunk = r & ((1 << cshift) - 1);
    const int n = r >> cshift;
    int t, hh;
    if (a.magic) {
      t = (int)(((uint64_t)(uint32_t)n * a.mhw) >> 32);
      hh = (int)(((uint64_t)(uint32_t)(n - t * hw) * a.mw) >> 32);
    } else {
      t = n / hw;
      hh = (n - t * hw) / a.Wg;
    }
    const int rem = n - t * hw, ww = rem - hh * a.Wg;
    double y[8];
#pragma unroll
    for (int pi = 0; pi < 4; ++pi) {
      const int ch = chunk * 8 + 2 * pi;
      // range of the pair, by selects (a runtime index into the argument
      // struct would load it from memory)
      const bool in0 = ch < a.off1, in1 = ch < a.off2;
      const int o = in0 ? 0 : (in1 ? a.off1 : a.off2);
      const int tof = in0 ? a.toff[0] : (in1 ? a.toff[1] : a.toff[2]);
      const int hd = in0 ? a.dm[0] / 2 : (in1 ? a.dm[1] / 2 : a.dm[2] / 2);
      const int ps = in0 ? t : (in1 ? hh : ww);
      const double2 cs = tab[tof + ps * hd + (ch - o) / 2];
      const double x0 = Elem<T>::ld(&x[kk].v[2 * pi]), x1 = Elem<T>::ld(&x[kk].v[2 * pi + 1]);
      {
#pragma clang fp contract(off)
        y[2 * pi] = x0 * cs.x - x1 * cs.y;
        y[2 * pi + 1] = x0 * cs.y + x1 * cs.x;
      }
    }
    store_rounded(x[kk], y);
    if (valid) x[kk].store((sel ? ko : qo) + base[kk]);
    if constexpr (sizeof(T) == 2) {
      // exact-sum range of the clustering: every stored value 0 or of
      // magnitude in [2^-47, 2^9) (bf16 bit patterns 0x2800 .. 0x43FF)
      bool out = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t mag = (uint32_t)x[kk].v[i] & 0x7FFFu;
        out |= valid && mag != 0u && (mag < 0x2800u || mag >= 0x4400u);
      }
      if (__ballot(out) && (threadIdx.x & 63) == 0) atomicOr(range_flag, 1);
    }
    if (sel && knm) {
      // squared norm of the token: its d/8 threads are consecutive lanes
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) { const float e = (float)Elem<T>::ld(&x[kk].v[i]); ss = fmaf(e, e, ss); }
      ss = (float)group_sum_dpp(valid ? (double)ss : 0.0, 1 << cshift);
      mx = fmaxf(mx, ss);
    }
  }
  if (sel && knm) {
    mx = block_max<float, 256>(mx, red);
    if (threadIdx.x == 0) atomicMax(&knm[bh], __float_as_uint(sqrtf(mx) * (1.0f + 0x1p-12f)));
  }
}

hipError_t launch_rope(const Geo& g, const scope_params& p, const void* q, const void* k, void* qo,
                       void* ko, const Workspace& w, float* k_norm_max, int32_t* range_flag, hipStream_t s) {
  // the rotation follows the 3D-RoPE ranges (g.rdm), not the clustering geometry
  const int n0 = g.T * g.rdm[0] / 2, n1 = g.Hg * g.rdm[1] / 2, n2 = g.Wg * g.rdm[2] / 2;
  rope_table_kernel<<<(n0 + n1 + n2 + 255) / 256, 256, 0, s>>>(w.rope_tab, n0, n1, n2, g.rdm[0], g.rdm[1],
                                                               g.rdm[2], p.rope_base, range_flag);
  RopeArgs a;
  a.BH = g.BH; a.N = g.N; a.d = g.d; a.Hg = g.Hg; a.Wg = g.Wg;
  a.off1 = g.rdm[0]; a.off2 = g.rdm[0] + g.rdm[1];
  a.dm[0] = g.rdm[0]; a.dm[1] = g.rdm[1]; a.dm[2] = g.rdm[2];
  a.toff[0] = 0; a.toff[1] = n0; a.toff[2] = n0 + n1;
  const uint64_t hw = (uint64_t)g.Hg * g.Wg;
  a.mhw = ((1ull << 32) + hw - 1) / hw;
  a.mw = ((1ull << 32) + g.Wg - 1) / (uint64_t)g.Wg;
  a.magic = (uint64_t)g.N * hw < (1ull << 32) ? 1 : 0;
  const dim3 blocks((unsigned)((g.N * (g.d / 8) + 256 * ROPE_R - 1) / (256 * ROPE_R)), (unsigned)g.BH, 2);
  uint32_t* knm = reinterpret_cast<uint32_t*>(k_norm_max);
  if (knm) {
    const hipError_t e = launch_fill_i32(reinterpret_cast<int32_t*>(knm), 0, (size_t)g.BH, s);
    if (e != hipSuccess) return e;
  }
  if (g.bf16)
    rope_kernel<uint16_t><<<blocks, 256, 0, s>>>((const uint16_t*)q, (const uint16_t*)k, (uint16_t*)qo,
                                                 (uint16_t*)ko, w.rope_tab, a, knm, range_flag);
  else
    rope_kernel<float><<<blocks, 256, 0, s>>>((const float*)q, (const float*)k, (float*)qo, (float*)ko,
                                              w.rope_tab, a, knm, range_flag);
  return hipGetLastError();
}

// Reordered copy of the RoPE'd rows for the partition ablation:
// out[row][i] = in[row][perm[i]].  One thread per output element (coalesced
// stores; the gathered loads stay inside one row of d elements).
template <typename T>
__global__ void __launch_bounds__(256) permute_kernel(const T* __restrict__ qi, const T* __restrict__ ki,
                                                      T* __restrict__ qo, T* __restrict__ ko, ChanPerm perm,
                                                      int d, size_t total) {
  __shared__ uint8_t pl[128];
  if (threadIdx.x < 128) pl[threadIdx.x] = perm.p[threadIdx.x];
  __syncthreads();
  const T* in = blockIdx.y ? ki : qi;
  T* out = blockIdx.y ? ko : qo;
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const size_t row = e / (size_t)d;
  const int i = (int)(e - row * (size_t)d);
  out[e] = in[row * (size_t)d + pl[i]];
}

hipError_t launch_permute(const Geo& g, const ChanPerm& perm, const void* qr, const void* kr, const Workspace& w,
                          hipStream_t s) {
  const size_t total = (size_t)g.BH * g.N * g.d;
  const dim3 blocks((unsigned)((total + 255) / 256), 2);
  if (g.bf16)
    permute_kernel<uint16_t><<<blocks, 256, 0, s>>>((const uint16_t*)qr, (const uint16_t*)kr, (uint16_t*)w.qperm,
                                                   (uint16_t*)w.kperm, perm, g.d, total);
  else
    permute_kernel<float><<<blocks, 256, 0, s>>>((const float*)qr, (const float*)kr, (float*)w.qperm,
                                                (float*)w.kperm, perm, g.d, total);
  return hipGetLastError();
}

}  // namespace scope
