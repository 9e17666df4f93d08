// Stage 6: exact attention of every query over its cluster's selected keys,
// with the original post-RoPE keys and values ("sparse attention is then
// computed over the selected original keys and values", SCOPE abstract):
//   o_i = sum_{j in S_c(i)} softmax_j(<q'_i, k'_j> / sqrt(d)) v_j.
//
// bf16 path (gfx950, wave64): one workgroup per (cluster, 128-query chunk);
// each of the 4 waves owns 32 queries whose Q rows stay in registers as MFMA
// operands.  Selected keys are gathered 64 at a time into LDS (K row-major,
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

struct AttArgs {
  int N, Cq;
  float scale_log2;   // log2(e) / sqrt(d)
  float scale;        // 1 / sqrt(d)
};

template <int D>
__global__ __launch_bounds__(256) void attend_bf16_kernel(AttArgs a, const int32_t* __restrict__ work,
                                                          const int32_t* __restrict__ status,
                                                          const int32_t* __restrict__ perm_q,
                                                          const int32_t* __restrict__ q_off,
                                                          const int32_t* __restrict__ cr,
                                                          const int64_t* __restrict__ sel_off,
                                                          const int32_t* __restrict__ sel_idx,
                                                          const uint16_t* __restrict__ qr,
                                                          const uint16_t* __restrict__ kr,
                                                          const uint16_t* __restrict__ vv,
                                                          uint16_t* __restrict__ out) {
  constexpr int BN = 64;                 // keys per chunk
  constexpr int KLD = D + 8;             // K tile row stride (elements)
  constexpr int VLD = BN + 4;            // V^T tile row stride (elements, 8-byte aligned rows)
  constexpr int PIECES = BN * D / 8;     // 16-byte pieces per tile
  constexpr int PPT = PIECES / 256;      // pieces per thread
  __shared__ __align__(16) uint16_t Ks[2][BN * KLD];
  __shared__ __align__(16) uint16_t Vt[2][D * VLD];

  if (status[1]) return;
  const int item = blockIdx.x;
  if (item >= status[0]) return;
  const int cid = work[2 * item], chunk = work[2 * item + 1];
  const int bh = cid / a.Cq, c = cid % a.Cq;
  const int32_t* qo = q_off + (size_t)bh * (a.Cq + 1);
  const int q0 = qo[c] + chunk * ATT_BM;
  const int nq = min(ATT_BM, qo[c + 1] - q0);
  const int r = cr[cid];
  const int32_t* keys = sel_idx + sel_off[cid];
  const size_t hb = (size_t)bh * a.N;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, col = lane & 31, hi = lane >> 5;
  const bool active = wv * 32 < nq;
  const int qi = wv * 32 + col;
  const bool qvalid = qi < nq;
  const int tok = qvalid ? min(max(perm_q[hb + q0 + qi], 0), a.N - 1) : 0;

  bf16x8_t qb[D / 16];
  {
    const uint16_t* qrow = qr + (hb + tok) * D + hi * 8;
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      uint4 u = qvalid ? *reinterpret_cast<const uint4*>(qrow + kb * 16) : make_uint4(0, 0, 0, 0);
      qb[kb] = *reinterpret_cast<bf16x8_t*>(&u);
    }
  }
  f32x16_t o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) o[t] = f32x16_t{};
  float mrun = -FLT_MAX, lsum = 0.f;

  const int nchunks = (r + BN - 1) / BN;
  // key indices come from the plan; clamp so a malformed plan cannot read out of bounds
  auto key_at = [&](int i) -> size_t { const int j = keys[i]; return (size_t)min(max(j, 0), a.N - 1); };
  uint4 kbuf[PPT], vbuf[PPT];
  auto gather = [&](int kc) {
    const int nk = min(BN, r - kc * BN);
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      // K: 16 lanes per row (row-major tile); V: one lane per row, so the
      // transposed LDS writes of a wave hit consecutive addresses
      const int piece = tid + i * 256;
      const int krow = piece / (D / 8), kc8 = piece % (D / 8);
      const int vrow = piece % BN, vc8 = piece / BN;
      kbuf[i] = krow < nk ? *reinterpret_cast<const uint4*>(kr + (hb + key_at(kc * BN + krow)) * D + kc8 * 8)
                          : make_uint4(0, 0, 0, 0);
      vbuf[i] = vrow < nk ? *reinterpret_cast<const uint4*>(vv + (hb + key_at(kc * BN + vrow)) * D + vc8 * 8)
                          : make_uint4(0, 0, 0, 0);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int piece = tid + i * 256;
      const int krow = piece / (D / 8), kc8 = piece % (D / 8);
      const int vrow = piece % BN, vc8 = piece / BN;
      *reinterpret_cast<uint4*>(&Ks[buf][krow * KLD + kc8 * 8]) = kbuf[i];
      const uint16_t* e = reinterpret_cast<const uint16_t*>(&vbuf[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) Vt[buf][(vc8 * 8 + j) * VLD + vrow] = e[j];
    }
  };

  if (nchunks > 0) { gather(0); stash(0); }
  __syncthreads();
  for (int kc = 0; kc < nchunks; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nchunks) gather(kc + 1);
    if (active) {
      f32x16_t s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        s[st] = f32x16_t{};
        const uint16_t* arow = &Ks[buf][(st * 32 + col) * KLD + hi * 8];
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) {
          const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(arow + kb * 16);
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qb[kb], s[st], 0, 0, 0);
        }
      }
      const int kleft = r - kc * BN;
      float mloc = -FLT_MAX;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = st * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
          const float x = key < kleft ? s[st][v] * a.scale_log2 : -FLT_MAX;
          s[st][v] = x;
          mloc = fmaxf(mloc, x);
        }
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float mnew = fmaxf(mrun, mloc);
      if (mnew > mrun) {
        const float alpha = exp2f(mrun - mnew);
        lsum *= alpha;
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[t][v] *= alpha;
        mrun = mnew;
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint16_t pb[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float x = s[st][half * 8 + i];
            const float p = x == -FLT_MAX ? 0.f : exp2f(x - mrun);
            pb[i] = f32_to_bf16(p);
            lsum += bf16_to_f32(pb[i]);   // normalise by what the MFMA multiplies
          }
          const bf16x8_t bp = *reinterpret_cast<bf16x8_t*>(pb);
          const int base = st * 32 + half * 16 + 4 * hi;
#pragma unroll
          for (int t = 0; t < D / 32; ++t) {
            const uint16_t* vrow = &Vt[buf][(t * 32 + col) * VLD + base];
            uint16_t av[8];
            *reinterpret_cast<uint2*>(av) = *reinterpret_cast<const uint2*>(vrow);
            *reinterpret_cast<uint2*>(av + 4) = *reinterpret_cast<const uint2*>(vrow + 8);
            o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<bf16x8_t*>(av), bp, o[t], 0, 0, 0);
          }
        }
      }
    }
    if (kc + 1 < nchunks) stash(buf ^ 1);
    __syncthreads();
  }
  if (!qvalid) return;
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  uint16_t* orow = out + (hb + tok) * D;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      uint16_t e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = f32_to_bf16(o[t][g4 * 4 + i] * inv);
      *reinterpret_cast<uint2*>(orow + t * 32 + 8 * g4 + 4 * hi) = *reinterpret_cast<uint2*>(e);
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
  const int item = blockIdx.x;
  if (item >= status[0]) return;
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
  const unsigned grid = (unsigned)plan.work_capacity;
  if (grid == 0) return hipSuccess;
#define SCOPE_ATT_ARGS a, plan.work, plan.status, plan.perm_q, plan.q_off, plan.counts_r, plan.sel_off, plan.sel_idx
  if (g.bf16) {
    if (g.d == 64)
      attend_bf16_kernel<64><<<grid, 256, 0, s>>>(SCOPE_ATT_ARGS, (const uint16_t*)qr, (const uint16_t*)kr,
                                                  (const uint16_t*)v, (uint16_t*)out);
    else
      attend_bf16_kernel<128><<<grid, 256, 0, s>>>(SCOPE_ATT_ARGS, (const uint16_t*)qr, (const uint16_t*)kr,
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
