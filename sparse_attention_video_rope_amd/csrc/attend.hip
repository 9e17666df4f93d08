// Stage 6: exact attention of every query over its cluster's selected keys,
// with the original post-RoPE keys and values ("sparse attention is then
// computed over the selected original keys and values", SCOPE abstract):
//   o_i = sum_{j in S_c(i)} softmax_j(<q'_i, k'_j> / sqrt(d)) v_j.
//
// bf16 path (gfx950, wave64): one workgroup of 4 waves per (cluster, 128-query
// chunk) work item; each wave owns 32 queries whose Q rows stay in registers
// as MFMA operands.  The selected keys' K and V rows are gathered 64 at a time
// straight into LDS (row-major, double buffered).  Per 32-key subtile the wave
// computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so each lane holds 16
// logits of one query: the online-softmax max and sum need one cross-lane
// exchange, and the probabilities are already laid out as the B operand of
// O^T += V^T P^T, whose V^T operand comes from transposing LDS reads.
#include <float.h>

#include "scope_device.hpp"
#include "scope_internal.hpp"

namespace scope {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// 16-byte row piece; a native vector (not the uint4 struct, whose whole-object
// copies become memcpy through private memory)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Work item of this workgroup, or -1 (items past the device-side count exit).
__device__ __forceinline__ int att_item(int n_work) {
  const int item = blockIdx.x;
  return item < n_work ? item : -1;
}

struct AttArgs {
  int N, Cq;
  float scale_log2;   // log2(e) / sqrt(d)
  float scale;        // 1 / sqrt(d)
};

// bf16 path with the K / V rows gathered straight into LDS
// (global_load_lds_dwordx4: lane l of a wave writes 16 bytes at the wave's LDS
// base + 16 l), so the gathers hold no registers and need no stash code.  Both
// tiles are row-major [64 keys][D] with the 16-byte pieces of a row permuted
// by an XOR so that the operand reads meet the LDS's 64 four-byte banks
// (256 bytes per cycle) without conflicts:
//   K: piece c of key j sits at c ^ kswz(j); a ds_read_b128 serves 16 lanes
//      (16 consecutive keys, one piece) per cycle, so those 16 pieces must
//      cover all 64 banks: with D = 64 two rows share a bank cycle and
//      kswz(j) = (j >> 1) & 7, with D = 128 kswz(j) = j & 15;
//   V: piece c of key j sits at c ^ (D / 32) (j & 3); the V^T operand of the
//      P V product is read with ds_read_b64_tr_b16 (in each 16-lane group lane
//      i receives 4 consecutive keys of dim i), 32 lanes per cycle read 4
//      rows x 64 bytes, and the XOR puts the 4 rows on disjoint banks.
// The two buffers of each tile are separate LDS arrays, so the compiler can
// see that the loads in flight never alias the buffer being read.
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
typedef __attribute__((address_space(1))) const char gbl_char;

// gfx950-only builtins behind device functions (the kernel template itself
// is also compiled by the host pass, which does not know them)
__device__ __forceinline__ void lds_load16(gbl_char* src, lds_u16* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}
__device__ __forceinline__ s16x4_t lds_read_tr16(const lds_u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

template <int D, int WPE, int BN = 64>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE))) void attend_bf16_lds_kernel(
    AttArgs a, const int32_t* __restrict__ work, const int32_t* __restrict__ status,
    const int32_t* __restrict__ perm_q, const int32_t* __restrict__ q_off, const int32_t* __restrict__ cr,
    const int64_t* __restrict__ sel_off, const int32_t* __restrict__ sel_idx, const float* __restrict__ knm,
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr, const uint16_t* __restrict__ vv,
    uint16_t* __restrict__ out) {
  constexpr int NW = 4;
  constexpr int BM = 32 * NW;
  static_assert(BM == ATT_BM, "queries per workgroup must equal the work-list chunk");
  constexpr int NST = BN / 32;               // 32-key MFMA row blocks per chunk
  constexpr int PR = D / 8;                  // 16-byte pieces per row
  constexpr int TILE = BN * D;               // elements per tile
  constexpr int BLK = TILE / 512;            // 1 KB blocks per tile
  constexpr int IPW = BLK / NW;              // blocks per wave per tile
  constexpr int RPB = 64 / PR;               // rows per block
  static_assert(IPW * NW == BLK, "gather split");
  constexpr float RESCALE_LOG2 = 8.f;
  __shared__ __align__(1024) uint16_t Ks0[TILE];
  __shared__ __align__(1024) uint16_t Ks1[TILE];
  __shared__ __align__(1024) uint16_t Vs0[TILE];
  __shared__ __align__(1024) uint16_t Vs1[TILE];

  if (status[1]) return;
  const int item = att_item(status[0]);
  if (item < 0) return;
  const int cid = work[2 * item], chunk = work[2 * item + 1];
  const int bh = cid / a.Cq, c = cid % a.Cq;
  const int32_t* qo = q_off + (size_t)bh * (a.Cq + 1);
  const int q0 = qo[c] + chunk * BM;
  const int nq = min(BM, qo[c + 1] - q0);
  const int r = cr[cid];
  const char* keyb = reinterpret_cast<const char*>(sel_idx + sel_off[cid]);
  const size_t hb = (size_t)bh * a.N;
  gbl_char* kbase = (gbl_char*)(kr + hb * D);
  gbl_char* vbase = (gbl_char*)(vv + hb * D);

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hi = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool active = wv * 32 < nq;
  const int qi = wv * 32 + col;
  const bool qvalid = qi < nq;
  const int tok = qvalid ? min(max(perm_q[hb + q0 + qi], 0), a.N - 1) : 0;
  bf16x8_t qb[D / 16];
  {
    const uint16_t* qrow = qr + (hb + tok) * D + hi * 8;
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      u32x4_t u = qvalid ? *reinterpret_cast<const u32x4_t*>(qrow + kb * 16) : u32x4_t{0, 0, 0, 0};
      qb[kb] = __builtin_bit_cast(bf16x8_t, u);
    }
  }
  // Q scaled by log2(e) / sqrt(d) (rounded to bf16), so the QK^T product gives
  // the logits in log2 units and the softmax weight of a logit t is exp2(t -
  // mref); the MFMA accumulator starts at -mref, so the product yields
  // t - mref directly
  const float cs = a.scale_log2;
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) {
    const u32x4_t u = __builtin_bit_cast(u32x4_t, qb[kb]);
    u32x4_t w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t wj = u[j];   // through a scalar (a bit_cast of u[j] compiles as u[0])
      const f32x2_t f = __builtin_convertvector(__builtin_bit_cast(bf16x2_t, wj), f32x2_t) * cs;
      w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
    }
    qb[kb] = __builtin_bit_cast(bf16x8_t, w);
  }
  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16_t{};
  float mref = 0.f, lsum = 0.f;    // reference (log2 units); set from the first chunk
  f32x16_t cneg = {};              // -mref in every element: the QK^T accumulator's start
  const int nchunks = (r + BN - 1) / BN;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  // upper bound of this query's scaled logits <q'', k'_j> (q'' the scaled bf16
  // row): ||q''|| (fp32 sum of exact bf16 squares) times the head's key-norm
  // bound, with a factor 1 + 2^-12 for the roundings; negative when there is
  // no bound
  float bound = -1.f;
  {
    float qn2 = 0.f;
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      const u32x4_t u = __builtin_bit_cast(u32x4_t, qb[kb]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t wj = u[j];   // through a scalar (a bit_cast of u[j] compiles as u[0])
        const bf16x2_t pr = __builtin_bit_cast(bf16x2_t, wj);
        qn2 = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, qn2, false);
      }
    }
    qn2 += __shfl_xor(qn2, 32);
    const float kb_ = knm ? knm[bh] : -1.f;
    if (kb_ > 0.f) bound = sqrtf(qn2) * kb_ * (1.f + 0x1p-12f);
  }

  auto kswz = [](int j) { return D == 64 ? (j >> 1) & 7 : j & (PR - 1); };
  auto vswz = [](int j) { return (D / 32) * (j & 3); };
  // gather role of this lane: block wv*IPW + i of each tile, row grow(i), piece
  // slot lane % PR, holding logical K piece slot ^ kswz(row) and V piece
  // slot ^ vswz(row)
  auto grow = [&](int i) { return (wv * IPW + i) * RPB + lane / PR; };
  uint32_t koff[IPW], voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int row = grow(i), slot = lane % PR;
    koff[i] = (uint32_t)((slot ^ kswz(row)) * 16);
    voff[i] = (uint32_t)((slot ^ vswz(row)) * 16);
  }
  // raw key indices of the next chunk's rows (loaded a chunk ahead)
  int kidx[IPW];
  auto load_idx = [&](int kc) {
#pragma unroll
    for (int i = 0; i < IPW; ++i)
      kidx[i] = *reinterpret_cast<const int*>(keyb + (uint32_t)min(kc * BN + grow(i), r - 1) * 4u);
  };
  auto gather = [&](lds_u16* Kd, lds_u16* Vd) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const uint32_t ro = min((uint32_t)kidx[i], (uint32_t)(a.N - 1)) * (uint32_t)(D * 2);
      lds_load16(kbase + (ro + koff[i]), Kd + (wv * IPW + i) * 512);
      lds_load16(vbase + (ro + voff[i]), Vd + (wv * IPW + i) * 512);
    }
  };
  // operand read offsets (elements): K rows st*32 + col, logical piece 2 kb + hi;
  // V^T for dims dt*32 + col: this lane, as a source of the transposing read,
  // reads key row (lane & 15) >> 2 of its 4-key group at dims
  // dt*32 + 16*((lane >> 4) & 1) + 4*(lane & 3)
  uint32_t kro[D / 16], vro[D / 32];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) kro[kb] = (uint32_t)(col * D + (((2 * kb) | hi) ^ kswz(col)) * 8);
  {
    const int i16 = lane & 15, ra = i16 >> 2, b = i16 & 3, gl = (lane >> 4) & 1;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int lp = dt * 4 + 2 * gl + (b >> 1);
      vro[dt] = (uint32_t)((4 * hi + ra) * D + ((lp ^ vswz(ra)) * 8) + (b & 1) * 4);
    }
  }

  // fixed (wave-uniform): the softmax reference mref is final, no running
  // maximum is kept; see the switch after the first chunk below
  bool fixed = false;
  auto step = [&](int kc, lds_u16* Kc, lds_u16* Vc, lds_u16* Kn, lds_u16* Vn) {
    if (kc + 1 < nchunks) {
      gather(Kn, Vn);                              // rows of chunk kc+1
      load_idx(min(kc + 2, nchunks - 1));          // indices of chunk kc+2
    }
    if (active) {
      f32x16_t s[NST];
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        bf16x8_t ak[D / 16];
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) ak[kb] = *(const lds_bf16x8*)(Kc + kro[kb] + st * 32 * D);
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[0], qb[0], cneg, 0, 0, 0);
#pragma unroll
        for (int kb = 1; kb < D / 16; ++kb) s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[kb], qb[kb], s[st], 0, 0, 0);
      }
      const int kleft = r - kc * BN;
      if (kleft < BN) {
        // key offset of this lane's rows, made opaque here so that the 32 key
        // positions are formed in this (last-chunk) branch instead of being
        // kept live in registers across the loop
        int k4 = 4 * hi;
        asm volatile("" : "+v"(k4));
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (st * 32 + 8 * (v >> 2) + (v & 3) + k4 >= kleft) s[st][v] = -__builtin_inff();
      }
      if (!fixed) {
        // running maximum: s holds logits minus mref; the first chunk sets
        // the reference to its maximum, a later one raises it when its
        // maximum exceeds it by more than RESCALE_LOG2
        float mloc = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int e = 2; e < NST * 16; e += 2) mloc = fmaxf(fmaxf(mloc, s[e >> 4][e & 15]), s[e >> 4][(e + 1) & 15]);
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const bool first = kc == 0;
        const bool grow_m = first || mloc > RESCALE_LOG2;
        if (__ballot(grow_m)) {
          const float dm = grow_m ? mloc : 0.f;
          const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(-dm);
          lsum *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
#pragma unroll
          for (int st = 0; st < NST; ++st)
#pragma unroll
            for (int v = 0; v < 16; ++v) s[st][v] -= dm;
          mref += dm;
#pragma unroll
          for (int v = 0; v < 16; ++v) cneg[v] = -mref;
        }
      }
#pragma unroll
      for (int st = 0; st < NST; ++st) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x2_t pk[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = __builtin_amdgcn_exp2f(s[st][half * 8 + 2 * i]);
            const float p1 = __builtin_amdgcn_exp2f(s[st][half * 8 + 2 * i + 1]);
            pk[i] = __builtin_convertvector((f32x2_t){p0, p1}, bf16x2_t);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(pk[i], ones, lsum, false);
          }
          const bf16x8_t bp = __builtin_bit_cast(bf16x8_t, pk);
          const int kofs = (st * 32 + half * 16) * D;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const s16x4_t v0 = lds_read_tr16(Vc + vro[dt] + kofs);
            const s16x4_t v1 = lds_read_tr16(Vc + vro[dt] + kofs + 8 * D);
            const bf16x8_t av = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bp, o[dt], 0, 0, 0);
          }
        }
      }
    }
    // this chunk's reads are done and the next chunk's rows have landed
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  lds_u16* K0 = (lds_u16*)&Ks0[0];
  lds_u16* K1 = (lds_u16*)&Ks1[0];
  lds_u16* V0 = (lds_u16*)&Vs0[0];
  lds_u16* V1 = (lds_u16*)&Vs1[0];
  if (nchunks > 0) {
    load_idx(0);
    __builtin_amdgcn_s_waitcnt(0);
    gather(K0, V0);
    if (nchunks > 1) load_idx(1);
  }
  // Q rows, the first chunk and the next indices are complete here on every
  // path, so the loop starts with no loads outstanding
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // After the first chunk mref is its maximum m0 <= max_j t_j <= bound (t the
  // scaled logits).  If bound - m0 <= 124 for every query of the wave, the
  // reference becomes mref = max(m0, bound - 60) for the rest of the item:
  // every later weight is exp2(t - mref) <= 2^60 (no overflow), and the
  // largest one is >= 2^-64 (the fp32 / bf16 exponent range keeps every weight
  // that is not negligible next to it), so the chunk maximum is no longer
  // needed.
  auto decide = [&]() {
    if (nchunks < 2 || !active) return;
    const bool ok = !qvalid || (bound >= mref && bound - mref <= 124.f);
    // the decision is wave-uniform; it is handed over in a VGPR the compiler
    // cannot see through, so the branches on it compile as exec-masked
    // regions that update O in place (as a uniform branch, the accumulators
    // were copied between register sets on every chunk)
    int fv = __ballot(!ok) == 0 ? 1 : 0;
    asm volatile("" : "+v"(fv));
    fixed = fv != 0;
    if (fixed) {
      const float mnew = qvalid ? fmaxf(mref, bound - 60.f) : mref;
      const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
      mref = mnew;
#pragma unroll
      for (int v = 0; v < 16; ++v) cneg[v] = -mref;
    }
  };
  for (int kc = 0; kc < nchunks; kc += 2) {
    step(kc, K0, V0, K1, V1);
    if (kc == 0) decide();
    if (kc + 1 < nchunks) step(kc + 1, K1, V1, K0, V0);
  }
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (!qvalid) return;
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  uint16_t* orow = out + (hb + tok) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x2_t e[2];
      e[0] = __builtin_convertvector((f32x2_t){o[dt][g4 * 4] * inv, o[dt][g4 * 4 + 1] * inv}, bf16x2_t);
      e[1] = __builtin_convertvector((f32x2_t){o[dt][g4 * 4 + 2] * inv, o[dt][g4 * 4 + 3] * inv}, bf16x2_t);
      *reinterpret_cast<uint2*>(orow + dt * 32 + 8 * g4 + 4 * hi) = *reinterpret_cast<uint2*>(e);
    }
  }
}

// fp32 storage: one thread per query, fp32 online softmax over the selected keys.
template <int D>
__global__ __launch_bounds__(ATT_BM) void attend_f32_kernel(AttArgs a, const int32_t* __restrict__ work,
                                                            const int32_t* __restrict__ status,
                                                            const int32_t* __restrict__ perm_q,
                                                            const int32_t* __restrict__ q_off,
                                                            const int32_t* __restrict__ cr,
                                                            const int64_t* __restrict__ sel_off,
                                                            const int32_t* __restrict__ sel_idx,
                                                            const float* __restrict__ /*knm: unused*/,
                                                            const float* __restrict__ qr, const float* __restrict__ kr,
                                                            const float* __restrict__ vv, float* __restrict__ out) {
  if (status[1]) return;
  const int item = att_item(status[0]);
  if (item < 0) return;
  const int cid = work[2 * item], chunk = work[2 * item + 1];
  const int bh = cid / a.Cq, c = cid % a.Cq;
  const int32_t* qo = q_off + (size_t)bh * (a.Cq + 1);
  const int q0 = qo[c] + chunk * ATT_BM;
  const int nq = min(ATT_BM, qo[c + 1] - q0);
  if ((int)threadIdx.x >= nq) return;
  const size_t hb = (size_t)bh * a.N;
  const int tok = min(max(perm_q[hb + q0 + threadIdx.x], 0), a.N - 1);
  const int r = cr[cid];
  const int32_t* keys = sel_idx + sel_off[cid];
  float q[D], o[D];
  for (int i = 0; i < D; ++i) { q[i] = qr[(hb + tok) * D + i]; o[i] = 0.f; }
  float mrun = -FLT_MAX, l = 0.f;
  for (int k = 0; k < r; ++k) {
    const size_t kj = hb + min(max(keys[k], 0), a.N - 1);
    float s = 0.f;
    for (int i = 0; i < D; ++i) s = fmaf(q[i], kr[kj * D + i], s);
    s *= a.scale;
    const float mnew = fmaxf(mrun, s);
    const float alpha = expf(mrun - mnew), p = expf(s - mnew);
    l = l * alpha + p;
    for (int i = 0; i < D; ++i) o[i] = o[i] * alpha + p * vv[kj * D + i];
    mrun = mnew;
  }
  for (int i = 0; i < D; ++i) out[(hb + tok) * D + i] = o[i] / l;
}

hipError_t launch_attend(const Geo& g, const scope_plan_t& plan, const void* qr, const void* kr, const void* v,
                         void* out, hipStream_t s) {
  AttArgs a;
  a.N = g.N;
  a.Cq = g.Cq;
  a.scale = (float)(1.0 / sqrt((double)g.d));
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)g.d));
  if (plan.work_capacity == 0) return hipSuccess;
  const unsigned grid = (unsigned)plan.work_capacity;
#define SCOPE_ATT_ARGS \
  a, plan.work, plan.status, plan.perm_q, plan.q_off, plan.counts_r, plan.sel_off, plan.sel_idx, plan.k_norm_max
  if (g.bf16) {
    // 4 waves x 32 queries; 3 (d = 64) or 2 (d = 128) waves per SIMD
    if (g.d == 64)
      attend_bf16_lds_kernel<64, 3><<<grid, 256, 0, s>>>(SCOPE_ATT_ARGS, (const uint16_t*)qr, (const uint16_t*)kr,
                                                         (const uint16_t*)v, (uint16_t*)out);
    else
      attend_bf16_lds_kernel<128, 2><<<grid, 256, 0, s>>>(SCOPE_ATT_ARGS, (const uint16_t*)qr, (const uint16_t*)kr,
                                                          (const uint16_t*)v, (uint16_t*)out);
  } else {
    if (g.d == 64)
      attend_f32_kernel<64><<<grid, ATT_BM, 0, s>>>(SCOPE_ATT_ARGS, (const float*)qr, (const float*)kr,
                                                    (const float*)v, (float*)out);
    else
      attend_f32_kernel<128><<<grid, ATT_BM, 0, s>>>(SCOPE_ATT_ARGS, (const float*)qr, (const float*)kr,
                                                     (const float*)v, (float*)out);
  }
#undef SCOPE_ATT_ARGS
  return hipGetLastError();
}

}  // namespace scope
