// Stage 6: exact attention of every query over its cluster's selected keys,
// with the original post-RoPE keys and values ("sparse attention is then
// computed over the selected original keys and values", SCOPE abstract):
//   o_i = sum_{j in S_c(i)} softmax_j(<q'_i, k'_j> / sqrt(d)) v_j.
//
// bf16 path (gfx950, wave64): one workgroup per (cluster, query chunk) work
// item; each wave owns 32 (head dim 128) or 64 (head dim 64) queries whose Q
// rows stay in registers as MFMA operands.  Selected keys are gathered 64 at a time into LDS (K row-major,
// V transposed), double buffered.  Per 32-key subtile the wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so each lane holds 16 logits of
// one query: the online-softmax max and sum need one cross-lane exchange, and
// the probabilities are already laid out as the B operand of O^T += V^T P^T.
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

// bf16 path with TT 32-query column tiles per wave (NW waves, 32*TT*NW queries
// per workgroup): every K / V^T operand read from LDS feeds TT MFMAs, and the
// key indices of chunk kc+2 are loaded while chunk kc is computed.  Gathers
// are unconditional: indices past r_c repeat the last selected key (those
// logits are masked to -inf), so no lane needs a branch or a zero fill.  The
// row sum is taken over the bf16-rounded probabilities that feed the P V
// product (dot2 with (1, 1)), so the normalisation matches the weights used.
template <int D, int NW, int TT, int WPE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE))) void attend_bf16_tiles_kernel(
    AttArgs a, const int32_t* __restrict__ work, const int32_t* __restrict__ status,
    const int32_t* __restrict__ perm_q, const int32_t* __restrict__ q_off, const int32_t* __restrict__ cr,
    const int64_t* __restrict__ sel_off, const int32_t* __restrict__ sel_idx, const uint16_t* __restrict__ qr,
    const uint16_t* __restrict__ kr, const uint16_t* __restrict__ vv, uint16_t* __restrict__ out) {
  constexpr int NTH = 64 * NW;
  constexpr int BM = 32 * TT * NW;
  static_assert(BM == ATT_BM, "queries per workgroup must equal the work-list chunk");
  constexpr int BN = 64;
  constexpr int KLD = D + 8;
  constexpr int VLD = BN + 4;
  constexpr int KPT = BN * D / 8 / NTH;            // K 16-byte pieces per thread
  constexpr int VPIECES = (BN / 2) * (D / 8);       // V key-pair pieces per chunk
  constexpr int VPT = (VPIECES + NTH - 1) / NTH;     // per thread (the last round may be partial)
  static_assert(KPT * NTH == BN * D / 8, "gather split");
  static_assert(VPIECES % 64 == 0, "V pieces per wave");
  constexpr int NIDX = KPT + 2 * VPT;              // key indices per thread per chunk
  constexpr float RESCALE_LOG2 = 8.f;
  __shared__ __align__(16) uint16_t Ks[2][BN * KLD];
  __shared__ __align__(16) uint16_t Vt[2][D * VLD];

  if (status[1]) return;
  const int item = att_item(status[0]);
  if (item < 0) return;
  const int cid = work[2 * item], chunk = work[2 * item + 1];
  const int bh = cid / a.Cq, c = cid % a.Cq;
  const int32_t* qo = q_off + (size_t)bh * (a.Cq + 1);
  const int q0 = qo[c] + chunk * BM;
  const int nq = min(BM, qo[c + 1] - q0);
  const int r = cr[cid];
  const int32_t* keys = sel_idx + sel_off[cid];
  const size_t hb = (size_t)bh * a.N;
  const char* kbase = reinterpret_cast<const char*>(kr + hb * D);
  const char* vbase = reinterpret_cast<const char*>(vv + hb * D);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, col = lane & 31, hi = lane >> 5;
  const bool active = wv * 32 * TT < nq;
  int tok[TT];
  bool qvalid[TT];
  bf16x8_t qb[TT][D / 16];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int qi = wv * 32 * TT + t * 32 + col;
    qvalid[t] = qi < nq;
    tok[t] = qvalid[t] ? min(max(perm_q[hb + q0 + qi], 0), a.N - 1) : 0;
    const uint16_t* qrow = qr + (hb + tok[t]) * D + hi * 8;
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      uint4 u = qvalid[t] ? *reinterpret_cast<const uint4*>(qrow + kb * 16) : make_uint4(0, 0, 0, 0);
      qb[t][kb] = *reinterpret_cast<bf16x8_t*>(&u);
    }
  }
  f32x16_t o[TT][D / 32];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[t][dt] = f32x16_t{};
  float mref[TT], lsum[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) { mref[t] = -__builtin_inff(); lsum[t] = 0.f; }
  const float cs = a.scale_log2;
  const int nchunks = (r + BN - 1) / BN;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // rows this thread gathers: K pieces i -> row (tid + i*NTH) / (D/8); V pairs i -> rows 2kp, 2kp+1
  auto row_of = [&](int i) -> int {
    if (i < KPT) return (tid + i * NTH) / (D / 8);
    const int j = (i - KPT) >> 1, piece = min(tid + j * NTH, VPIECES - 1);
    return 2 * (piece % (BN / 2)) + ((i - KPT) & 1);
  };
  // Raw key indices of a chunk, loaded one chunk ahead of their gather and left
  // untouched until then: vmcnt retires loads in order, so any arithmetic on
  // them here would make the wave wait for the row gathers issued before them.
  int kidx[NIDX];
  const char* keyb = reinterpret_cast<const char*>(keys);   // uniform base, 32-bit byte offsets
  auto load_idx = [&](int kc, int* dst) {
#pragma unroll
    for (int i = 0; i < NIDX; ++i)
      dst[i] = *reinterpret_cast<const int*>(keyb + (uint32_t)min(kc * BN + row_of(i), r - 1) * 4u);
  };
  // byte offset of a gathered row inside the head (index clamped to [0, N))
  auto row_off = [&](int j) -> uint32_t { return (uint32_t)min(max(j, 0), a.N - 1) * (uint32_t)(D * 2); };
  u32x4_t kbuf[KPT], vb0[VPT], vb1[VPT];
  auto gather = [&](const int* ix) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c8 = (tid + i * NTH) % (D / 8);
      kbuf[i] = *reinterpret_cast<const u32x4_t*>(kbase + (row_off(ix[i]) + (uint32_t)(c8 * 16)));
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int oc = min(tid + i * NTH, VPIECES - 1) / (BN / 2);
      vb0[i] = *reinterpret_cast<const u32x4_t*>(vbase + (row_off(ix[KPT + 2 * i]) + (uint32_t)(oc * 16)));
      vb1[i] = *reinterpret_cast<const u32x4_t*>(vbase + (row_off(ix[KPT + 2 * i + 1]) + (uint32_t)(oc * 16)));
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int piece = tid + i * NTH;
      const int row = piece / (D / 8), c8 = piece % (D / 8);
      *reinterpret_cast<u32x4_t*>(&Ks[buf][row * KLD + c8 * 8]) = kbuf[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int piece = tid + i * NTH;
      if (VPIECES % NTH != 0 && piece >= VPIECES) break;   // wave-uniform
      const int kp = piece % (BN / 2), oc = piece / (BN / 2);
      const uint32_t w0[4] = {vb0[i].x, vb0[i].y, vb0[i].z, vb0[i].w};
      const uint32_t w1[4] = {vb1[i].x, vb1[i].y, vb1[i].z, vb1[i].w};
      uint32_t* dst = reinterpret_cast<uint32_t*>(&Vt[buf][(oc * 8) * VLD + 2 * kp]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dst[(2 * j) * (VLD / 2)] = __builtin_amdgcn_perm(w1[j], w0[j], 0x05040100u);
        dst[(2 * j + 1) * (VLD / 2)] = __builtin_amdgcn_perm(w1[j], w0[j], 0x07060302u);
      }
    }
  };

  if (nchunks > 0) {
    load_idx(0, kidx);
    gather(kidx);
    stash(0);
  }
  // Q rows, the first chunk and its indices are complete here: the loop then
  // carries only its own loads, whose waits sit at their first use
  __builtin_amdgcn_s_waitcnt(0);
  if (nchunks > 1) load_idx(1, kidx);
  __syncthreads();
  for (int kc = 0; kc < nchunks; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nchunks) {
      gather(kidx);                                // rows of chunk kc+1
      // indices of chunk kc+2 (kidx is free again); issued unconditionally
      // (clamped to the last chunk) so the wait before the stash below counts
      // exactly these loads
      load_idx(min(kc + 2, nchunks - 1), kidx);
    }
    if (active) {
      f32x16_t s[TT][2];   // [query tile][key subtile]
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint16_t* arow = &Ks[buf][(st * 32 + col) * KLD + hi * 8];
        bf16x8_t ak[D / 16];
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) ak[kb] = *reinterpret_cast<const bf16x8_t*>(arow + kb * 16);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          s[t][st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[0], qb[t][0], f32x16_t{}, 0, 0, 0);
#pragma unroll
          for (int kb = 1; kb < D / 16; ++kb)
            s[t][st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[kb], qb[t][kb], s[t][st], 0, 0, 0);
        }
      }
      const int kleft = r - kc * BN;
      if (kleft < BN) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (st * 32 + 8 * (v >> 2) + 4 * hi + (v & 3) >= kleft) s[t][st][v] = -__builtin_inff();
      }
      float mc[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        // max3 chain over the 32 logits of this lane
        float mloc = fmaxf(s[t][0][0], s[t][0][1]);
#pragma unroll
        for (int e = 2; e < 32; e += 2)
          mloc = fmaxf(fmaxf(mloc, s[t][e >> 4][e & 15]), s[t][e >> 4][(e + 1) & 15]);
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const bool grow = (mloc - mref[t]) * cs > RESCALE_LOG2;
        if (__ballot(grow)) {
          const float mnew = grow ? mloc : mref[t];
          const float alpha = __builtin_amdgcn_exp2f((mref[t] - mnew) * cs);
          lsum[t] *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[t][dt][v] *= alpha;
          mref[t] = mnew;
        }
        mc[t] = mref[t] * cs;
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8_t bp[TT];
#pragma unroll
          for (int t = 0; t < TT; ++t) {
            bf16x2_t pk[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float p0 = __builtin_amdgcn_exp2f(fmaf(s[t][st][half * 8 + 2 * i], cs, -mc[t]));
              const float p1 = __builtin_amdgcn_exp2f(fmaf(s[t][st][half * 8 + 2 * i + 1], cs, -mc[t]));
              pk[i] = __builtin_convertvector((f32x2_t){p0, p1}, bf16x2_t);
              lsum[t] = __builtin_amdgcn_fdot2_f32_bf16(pk[i], ones, lsum[t], false);
            }
            bp[t] = *reinterpret_cast<bf16x8_t*>(pk);
          }
          const int base = st * 32 + half * 16 + 4 * hi;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const uint16_t* vrow = &Vt[buf][(dt * 32 + col) * VLD + base];
            uint2 av[2];
            av[0] = *reinterpret_cast<const uint2*>(vrow);
            av[1] = *reinterpret_cast<const uint2*>(vrow + 8);
            const bf16x8_t avv = *reinterpret_cast<bf16x8_t*>(av);
#pragma unroll
            for (int t = 0; t < TT; ++t)
              o[t][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(avv, bp[t], o[t][dt], 0, 0, 0);
          }
        }
      }
    }
    if (kc + 1 < nchunks) stash(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float ltot = lsum[t] + __shfl_xor(lsum[t], 32);
    if (!qvalid[t]) continue;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    uint16_t* orow = out + (hb + tok[t]) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x2_t e[2];
        e[0] = __builtin_convertvector((f32x2_t){o[t][dt][g4 * 4] * inv, o[t][dt][g4 * 4 + 1] * inv}, bf16x2_t);
        e[1] = __builtin_convertvector((f32x2_t){o[t][dt][g4 * 4 + 2] * inv, o[t][dt][g4 * 4 + 3] * inv}, bf16x2_t);
        *reinterpret_cast<uint2*>(orow + dt * 32 + 8 * g4 + 4 * hi) = *reinterpret_cast<uint2*>(e);
      }
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
#define SCOPE_ATT_ARGS a, plan.work, plan.status, plan.perm_q, plan.q_off, plan.counts_r, plan.sel_off, plan.sel_idx
  if (g.bf16) {
    // 4 waves x 32 queries; head dim 64 fits 128 VGPRs (4 waves per SIMD)
    if (g.d == 64)
      attend_bf16_tiles_kernel<64, 4, 1, 4><<<grid, 256, 0, s>>>(SCOPE_ATT_ARGS, (const uint16_t*)qr,
                                                                 (const uint16_t*)kr, (const uint16_t*)v,
                                                                 (uint16_t*)out);
    else
      attend_bf16_tiles_kernel<128, 4, 1, 2><<<grid, 256, 0, s>>>(SCOPE_ATT_ARGS, (const uint16_t*)qr,
                                                                  (const uint16_t*)kr, (const uint16_t*)v,
                                                                  (uint16_t*)out);
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
