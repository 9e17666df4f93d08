// Device helpers shared by the SCOPE kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace scope {

constexpr int WAVE = 64;

// ---- number formats -------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> bf16 with a single round-to-nearest-even from the fp64 value.
// Normal range: keep the top 7 of the 52 explicit mantissa bits (carry may
// move into the exponent; beyond the bf16 range the fp32 conversion gives
// inf).  Below 2^-126: round to a multiple of the bf16 subnormal spacing.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  if (!(fabs(x) >= 0x1p-126)) {
    double r = rint(x * 0x1p133) * 0x1p-133;
    return (uint16_t)(__float_as_uint((float)r) >> 16);
  }
  uint64_t u = (uint64_t)__double_as_longlong(x);
  u += 0x0FFFFFFFFFFFull + ((u >> 45) & 1ull);
  u &= ~0x1FFFFFFFFFFFull;
  return (uint16_t)(__float_as_uint((float)__longlong_as_double((long long)u)) >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ double ld(const uint16_t* p) { return (double)bf16_to_f32(*p); }
  static __device__ __forceinline__ float ldf(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void st(uint16_t* p, double x) { *p = f64_to_bf16(x); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ double ld(const float* p) { return (double)*p; }
  static __device__ __forceinline__ float ldf(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, double x) { *p = (float)x; }
};

// ---- wave / block reductions ----------------------------------------------

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) { T u = __shfl_xor(v, o, WAVE); v = u > v ? u : v; }
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_min(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) { T u = __shfl_xor(v, o, WAVE); v = u < v ? u : v; }
  return v;
}

// The DPP builtins are not convergent operations for the compiler, so a DPP
// reduction whose result is only used inside a branch may be sunk into that
// branch, where the disabled lanes read as 0.  Every DPP helper below ends by
// passing its result through an empty volatile asm, which keeps the whole
// reduction where the helper is called.
template <typename T>
__device__ __forceinline__ T dpp_pin(T v) {
  asm volatile("" : "+v"(v));
  return v;
}

// DPP lane move of an fp64 value (both 32-bit halves; lanes outside the pattern read 0).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, true);
  return __hiloint2double(hi, lo);
}

// Sum over the 64 lanes of a wave, in a fixed order, without LDS: quad_perm
// xor-1 / xor-2, row_half_mirror and row_mirror leave every lane of a 16-lane
// row holding the row sum; the four row sums are then read from lanes 0, 16,
// 32 and 48.  All 64 lanes must be active.
__device__ __forceinline__ double wave_sum_dpp(double v) {
  v += dpp_f64<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);   // row_half_mirror
  v += dpp_f64<0x140>(v);   // row_mirror
  v = dpp_pin(v);
  auto rl = [&](int l) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
  };
  return (rl(0) + rl(16)) + (rl(32) + rl(48));
}

// Sum inside aligned groups of `n` lanes (n in {1, 2, 4, 8, 16}); every lane of
// a group receives the group sum.  Fixed order, no LDS.
__device__ __forceinline__ double group_sum_dpp(double v, int n) {
  if (n >= 2) v += dpp_f64<0xB1>(v);    // xor 1
  if (n >= 4) v += dpp_f64<0x4E>(v);    // xor 2
  if (n >= 8) v += dpp_f64<0x141>(v);   // i <-> 7-i within 8
  if (n >= 16) v += dpp_f64<0x140>(v);  // i <-> 15-i within 16
  return dpp_pin(v);
}

// Inclusive prefix sum over the 64 lanes of a wave (fixed order).
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T u = __shfl_up(v, o, WAVE);
    if (lane >= o) v += u;
  }
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves only (no
// LDS, no lane-address registers): a Hillis-Steele scan inside each 16-lane
// row (row_shr 1, 2, 4, 8), then row 0's total is added to row 1 and row 2's
// to row 3 (row_bcast:15), then lane 31's running total to rows 2 and 3
// (row_bcast:31).  The addition order differs from wave_incl_scan, so use it
// for integers or for fp64 values whose partial sums are exact.  All 64 lanes
// must be active.
template <int CTRL, int RM>
__device__ __forceinline__ int dpp_row_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, RM, 0xF, false);
}
template <int CTRL, int RM>
__device__ __forceinline__ double dpp_row_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, RM, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, RM, 0xF, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
  v += dpp_row_i32<0x111, 0xF>(v);
  v += dpp_row_i32<0x112, 0xF>(v);
  v += dpp_row_i32<0x114, 0xF>(v);
  v += dpp_row_i32<0x118, 0xF>(v);
  v += dpp_row_i32<0x142, 0xA>(v);
  v += dpp_row_i32<0x143, 0xC>(v);
  return dpp_pin(v);
}
__device__ __forceinline__ double wave_incl_scan_dpp(double v) {
  v += dpp_row_f64<0x111, 0xF>(v);
  v += dpp_row_f64<0x112, 0xF>(v);
  v += dpp_row_f64<0x114, 0xF>(v);
  v += dpp_row_f64<0x118, 0xF>(v);
  v += dpp_row_f64<0x142, 0xA>(v);
  v += dpp_row_f64<0x143, 0xC>(v);
  return dpp_pin(v);
}

// Block-wide inclusive scan built on wave_incl_scan_dpp (same caveat on the
// order); `tmp` holds NT/64 + 1 values.  All threads must call.
template <typename T, int NT>
__device__ __forceinline__ T block_incl_scan_dpp(T v, T* tmp, T* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  T inc = wave_incl_scan_dpp(v);
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    T x = lane < NW ? tmp[lane] : T(0);
    T xs = wave_incl_scan_dpp(x);
    if (lane < NW) tmp[lane] = xs - x;   // exclusive wave offsets
    if (lane == NW - 1) tmp[NW] = xs;
  }
  __syncthreads();
  T r = inc + tmp[w];
  if (total) *total = tmp[NW];
  __syncthreads();
  return r;
}

// Block-wide inclusive scan; `tmp` holds one T per wave.  All threads must call.
template <typename T, int NT>
__device__ __forceinline__ T block_incl_scan(T v, T* tmp, T* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  T inc = wave_incl_scan(v);
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    T x = lane < NW ? tmp[lane] : T(0);
    T xs = wave_incl_scan(x);
    if (lane < NW) tmp[lane] = xs - x;   // exclusive wave offsets
    if (lane == NW - 1) tmp[NW] = xs;
  }
  __syncthreads();
  T r = inc + tmp[w];
  if (total) *total = tmp[NW];
  __syncthreads();
  return r;
}

template <typename T, int NT>
__device__ __forceinline__ T block_sum(T v, T* tmp) {
  constexpr int NW = NT / 64;
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  T r = tmp[0];
  for (int i = 1; i < NW; ++i) r += tmp[i];
  __syncthreads();
  return r;
}

template <typename T, int NT>
__device__ __forceinline__ T block_max(T v, T* tmp) {
  constexpr int NW = NT / 64;
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  T r = tmp[0];
  for (int i = 1; i < NW; ++i) r = tmp[i] > r ? tmp[i] : r;
  __syncthreads();
  return r;
}

template <typename T, int NT>
__device__ __forceinline__ T block_min(T v, T* tmp) {
  constexpr int NW = NT / 64;
  v = wave_min(v);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  T r = tmp[0];
  for (int i = 1; i < NW; ++i) r = tmp[i] < r ? tmp[i] : r;
  __syncthreads();
  return r;
}

// ---- SplitMix64 (Steele, Lea and Flood, OOPSLA 2014), counter form ---------
// Output number i of the generator seeded with `seed`.
__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace scope
