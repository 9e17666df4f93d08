// Stage 6: exact attention of every query over its cluster's selected keys,
// on the post-RoPE keys and original values themselves rather than their
// proxies (SCOPE abstract):
//   o_i = sum_{j in S_c(i)} softmax_j(<q'_i, k'_j> / sqrt(d)) v_j.
//
// bf16 path (gfx950, wave64): one workgroup of NW waves per (cluster, 32 NW-query
// chunk) work item (NW = 8 at head dim 128, 4 at 64); each wave owns a block of
// 32 queries whose Q rows stay in registers as MFMA operands (in a small item,
// two waves share a block, one 32-key subtile each).  The selected keys' K and
// V rows are gathered 64 at a time straight into LDS (row-major, three
// buffers, gathered two chunks ahead).  Per 32-key subtile the wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so each lane holds 16 logits of
// one query: the online-softmax max and sum need one cross-lane exchange, and
// the probabilities are already laid out as the B operand of O^T += V^T P^T,
// whose V^T operand comes from transposing LDS reads.
#include <float.h>

#include <type_traits>

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
// Workgroups are dispatched to the 8 XCDs round-robin by block index; each
// XCD has its own L2, and the 256 MB Infinity Cache behind them is shared.
// The work list runs in (head, cluster, chunk) order and is cut into runs of
// ATT_RUN consecutive items; the runs go to the XCDs in turn, and XCD x takes
// its runs in list order (block b: k = b / 8 on XCD b mod 8, item
// (k / ATT_RUN * 8 + x) * ATT_RUN + k mod ATT_RUN).  So all XCDs work on the
// same stretch of the list, whose K / V rows (one head, 61 MB at the
// Hunyuan-like size) stay in the Infinity Cache, and the items of one cluster
// (same key set, adjacent in the list) mostly start together on one XCD and
// share its L2.  Giving each XCD one contiguous eighth of the list instead
// puts eight heads' K / V in flight at once; at the Hunyuan-like size that
// launch took 149 ms instead of 136 ms.  The grid is a multiple of 8 ATT_RUN.
constexpr int ATT_RUN = 8;
__device__ __forceinline__ int att_item(int n_work) {
  const int b = blockIdx.x, x = b & 7, k = b >> 3;
  const int item = ((k / ATT_RUN) * 8 + x) * ATT_RUN + k % ATT_RUN;
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
// The three buffers of each tile are separate LDS arrays, so the compiler can
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
// s_waitcnt immediate that waits until at most n vector memory operations are
// outstanding and leaves the other counters alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
__device__ __forceinline__ s16x4_t lds_read_tr16(const lds_u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

template <int D, int WPE, int NW, int BN = 64>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE))) void attend_bf16_lds_kernel(
    AttArgs a, const int32_t* __restrict__ work, const int32_t* __restrict__ status,
    const int32_t* __restrict__ perm_q, const int32_t* __restrict__ q_off, const int32_t* __restrict__ cr,
    const int64_t* __restrict__ sel_off, const int32_t* __restrict__ sel_idx, const float* __restrict__ knm,
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr, const uint16_t* __restrict__ vv,
    uint16_t* __restrict__ out) {
  constexpr int BM = 32 * NW;                // queries per work item (the work-list chunk)
  constexpr int NST = BN / 32;               // 32-key MFMA row blocks per chunk
  constexpr int PR = D / 8;                  // 16-byte pieces per row
  constexpr int TILE = BN * D;               // elements per tile
  constexpr int BLK = TILE / 512;            // 1 KB blocks per tile
  constexpr int IPW = BLK / NW;              // blocks per wave per tile
  constexpr int RPB = 64 / PR;               // rows per block
  static_assert(IPW * NW == BLK, "gather split");
  constexpr float RESCALE_LOG2 = 8.f;
  // three buffers per tile: chunk c lives in buffer c mod 3, and its rows are
  // gathered two chunks ahead
  __shared__ __align__(1024) uint16_t Ks0[TILE];
  __shared__ __align__(1024) uint16_t Ks1[TILE];
  __shared__ __align__(1024) uint16_t Ks2[TILE];
  __shared__ __align__(1024) uint16_t Vs0[TILE];
  __shared__ __align__(1024) uint16_t Vs1[TILE];
  __shared__ __align__(1024) uint16_t Vs2[TILE];
  // key indices of chunk c in slot c mod 3 (one row of 64 per wave), loaded
  // four chunks ahead
  __shared__ __align__(256) int32_t Is0[NW * BN];
  __shared__ __align__(256) int32_t Is1[NW * BN];
  __shared__ __align__(256) int32_t Is2[NW * BN];
  static_assert(BN == 64, "one 64-lane dword load per chunk of indices");

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
  // Split items.  An item of nb <= 3 NW / 4 query blocks (a cluster's last
  // item, often) would leave waves idle, and with 8 waves SIMDs with one busy
  // wave beside SIMDs with two (waves w and w + 4 share a SIMD).  Instead
  // some query blocks run on two waves, each taking one 32-key subtile of
  // every chunk, and the two partial softmax states are merged at the end
  // (H = NW / 2):
  //   nb <= H: block w on waves w and w + H (subtiles 0 and 1);
  //   H < nb <= 3H/2: blocks 0 .. H-1 whole on waves 0 .. H-1, block H + j on
  //   waves H + j and H + H/2 + j.
  constexpr int H = NW / 2;
  static_assert(NW % 4 == 0 && H <= 4, "split pairs and their merge buffers");
  const int nb = (nq + 31) / 32;
  const bool split = 2 * nb <= 3 * H;                // some blocks split (workgroup-uniform)
  const bool half = split && (nb <= H || wv >= H);   // this wave takes one subtile
  // query block of the wave, first key of its subtile in a chunk, and the
  // merge slot of its pair
  const int qw = !half ? wv : (nb <= H ? wv % H : H + (wv - H) % (H / 2));
  const int stb = !half ? 0 : (nb <= H ? wv / H : (wv - H) / (H / 2)) * 32;
  const int mslot = !half ? 0 : (nb <= H ? qw : qw - H);
  const bool active = qw * 32 < nq;
  const int qi = qw * 32 + col;
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
  // Q stays the exact bf16 row: the QK^T product is the logit in natural units,
  // scaled by cs = log2(e) / sqrt(d) in fp32 right after the MFMA chain, so
  // that the softmax weight of a scaled logit t is exp2(t - mref).  The MFMA
  // accumulator starts at -mref / cs, so the scaled product is t - mref
  // (up to fp32 rounding).  (A Q operand scaled by cs and rounded to bf16
  // would add an error of up to 2^-9 sum_i |q_i k_i| cs to every scaled
  // logit: an error in the exponent that grows with the logits.)
  const float cs = a.scale_log2, inv_cs = 1.f / a.scale_log2;
  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16_t{};
  float mref = 0.f, lsum = 0.f;    // reference (log2 units); set from the first chunk
  f32x16_t cneg = {};              // -mref / cs in every element: the QK^T accumulator's start
  const int nchunks = (r + BN - 1) / BN;
  // upper bound of this query's scaled logits cs <q', k'_j>: ||q'|| (fp32 sum
  // of exact bf16 squares) times the head's key-norm bound times cs, with a
  // factor 1 + 2^-12 for the roundings; negative when there is no bound
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
    if (kb_ > 0.f) bound = sqrtf(qn2) * kb_ * cs * (1.f + 0x1p-12f);
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
  // Key indices travel through LDS: each wave copies the 64 indices of a
  // chunk into its own row of the chunk's slot with one dword load to LDS
  // (lane l: key c BN + l, clamped to the last one) and reads its rows'
  // indices from there.  No register is loaded from global memory inside the
  // loop, so the compiler inserts no vector-memory wait of its own for them,
  // and the rows gathered ahead stay in flight until the explicit wait at the
  // end of each step.  The three slots are separate arrays, so that the
  // compiler can see that a slot being read is not the one being loaded.
  typedef __attribute__((address_space(3))) int32_t lds_i32;
  lds_i32* I0 = (lds_i32*)&Is0[0];
  lds_i32* I1 = (lds_i32*)&Is1[0];
  lds_i32* I2 = (lds_i32*)&Is2[0];
  int kidx[IPW];
  auto load_idx = [&](int c, lds_i32* slot) {
    __builtin_amdgcn_global_load_lds((gbl_char*)(keyb + (uint32_t)min(c * BN + lane, r - 1) * 4u),
                                     (__attribute__((address_space(3))) void*)(slot + wv * BN), 4, 0, 0);
  };
  auto take_idx = [&](const lds_i32* slot) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) kidx[i] = slot[wv * BN + grow(i)];
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
  for (int kb = 0; kb < D / 16; ++kb) kro[kb] = (uint32_t)((stb + col) * D + (((2 * kb) | hi) ^ kswz(col)) * 8);
  {
    const int i16 = lane & 15, ra = i16 >> 2, b = i16 & 3, gl = (lane >> 4) & 1;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int lp = dt * 4 + 2 * gl + (b >> 1);
      vro[dt] = (uint32_t)((stb + 4 * hi + ra) * D + ((lp ^ vswz(ra)) * 8) + (b & 1) * 4);
    }
  }

  // fixed (wave-uniform): the softmax reference mref is final, no running
  // maximum is kept; see the switch after the first chunk below
  bool fixed = false;
  // FAST: a chunk that is neither the first nor the last, on a wave whose
  // softmax reference is fixed: no key mask, no running maximum, the next
  // chunk exists.  Without the branches of the general step, the compiler can
  // interleave the exponentials of one 32-key subtile with the QK^T MFMAs of
  // the other.
  // Step of chunk kc (rows in Kc / Vc): gathers chunk kc + 2 into Kg / Vg
  // (the buffer of chunk kc - 1, free since the last barrier) with the
  // indices in slot It, and loads the indices of chunk kc + 4 into slot Il
  // (the slot of chunk kc + 1, whose indices were used in the last step).
  auto step = [&](auto fast_c, auto nst_c, int kc, lds_u16* Kc, lds_u16* Vc, lds_u16* Kg, lds_u16* Vg,
                  lds_i32* It, lds_i32* Il) __attribute__((always_inline)) {
    constexpr bool FAST = decltype(fast_c)::value;
    constexpr int NSTW = decltype(nst_c)::value;   // subtiles of the chunk this wave takes
    const bool more = FAST || kc + 2 < nchunks;
    if (more) {
      take_idx(It);                                // indices of chunk kc+2 (landed by the last step's wait)
      load_idx(min(kc + 4, nchunks - 1), Il);      // indices of chunk kc+4
      gather(Kg, Vg);                              // rows of chunk kc+2
    }
    if (active) {
      f32x16_t s[NSTW];
#pragma unroll
      for (int st = 0; st < NSTW; ++st) {
        bf16x8_t ak[D / 16];
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) ak[kb] = *(const lds_bf16x8*)(Kc + kro[kb] + st * 32 * D);
        // keep the subtile's K reads above its MFMA chain: issued together,
        // only the first read's latency is waited for
        __builtin_amdgcn_sched_barrier(0);
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[0], qb[0], cneg, 0, 0, 0);
#pragma unroll
        for (int kb = 1; kb < D / 16; ++kb) s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[kb], qb[kb], s[st], 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 16; ++v) s[st][v] *= cs;
      }
      const int kleft = r - kc * BN;
      if (!FAST && kleft < BN) {
        // key offset of this lane's rows, made opaque here so that the 32 key
        // positions are formed in this (last-chunk) branch instead of being
        // kept live in registers across the loop
        int k4 = 4 * hi + stb;
        asm volatile("" : "+v"(k4));
#pragma unroll
        for (int st = 0; st < NSTW; ++st)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (st * 32 + 8 * (v >> 2) + (v & 3) + k4 >= kleft) s[st][v] = -__builtin_inff();
      }
      if (!FAST && !fixed) {
        // running maximum: s holds logits minus mref; the first chunk sets
        // the reference to its maximum, a later one raises it when its
        // maximum exceeds it by more than RESCALE_LOG2
        float mloc = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int e = 2; e < NSTW * 16; e += 2) mloc = fmaxf(fmaxf(mloc, s[e >> 4][e & 15]), s[e >> 4][(e + 1) & 15]);
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const bool first = kc == 0;
        const bool grow_m = first || mloc > RESCALE_LOG2;
        if (__ballot(grow_m)) {
          // a split wave's subtile can be empty in the only chunk (r <= 32):
          // its reference stays 0 and its weights 0
          const float dm = grow_m && mloc != -__builtin_inff() ? mloc : 0.f;
          const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(-dm);
          lsum *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
#pragma unroll
          for (int st = 0; st < NSTW; ++st)
#pragma unroll
            for (int v = 0; v < 16; ++v) s[st][v] -= dm;
          mref += dm;
#pragma unroll
          for (int v = 0; v < 16; ++v) cneg[v] = -mref * inv_cs;
        }
      }
      // the chunk's share of the row sum, in four fp32 partial sums of the
      // weights before their bf16 rounding: plain adds overlap the other
      // wave's MFMAs, where a bf16 dot2 on the packed weights stalls them
      float csum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NSTW; ++st) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x2_t pk[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = __builtin_amdgcn_exp2f(s[st][half * 8 + 2 * i]);
            const float p1 = __builtin_amdgcn_exp2f(s[st][half * 8 + 2 * i + 1]);
            pk[i] = __builtin_convertvector((f32x2_t){p0, p1}, bf16x2_t);
            csum[i] += p0 + p1;
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
      lsum += (csum[0] + csum[1]) + (csum[2] + csum[3]);
    }
    // this chunk's reads are done, and the next chunk's rows (gathered in the
    // previous step) and the indices of chunk kc + 3 (loaded before them) have
    // landed: only this step's loads (one index load and 2 IPW row loads) may
    // still be in flight
    if (more) __builtin_amdgcn_s_waitcnt(waitcnt_vm(1 + 2 * IPW));
    else __builtin_amdgcn_s_waitcnt(0);
    // a bare barrier: __syncthreads() adds a workgroup fence, whose release
    // waits for every outstanding load, the prefetched chunk's too.  Every LDS
    // read of this step has completed (its values are MFMA operands) and the
    // explicit wait above covers this wave's part of the next chunk; the
    // memory clobber keeps the compiler from moving LDS accesses across it.
    asm volatile("s_barrier" ::: "memory");
  };

  lds_u16* K0 = (lds_u16*)&Ks0[0];
  lds_u16* K1 = (lds_u16*)&Ks1[0];
  lds_u16* K2 = (lds_u16*)&Ks2[0];
  lds_u16* V0 = (lds_u16*)&Vs0[0];
  lds_u16* V1 = (lds_u16*)&Vs1[0];
  lds_u16* V2 = (lds_u16*)&Vs2[0];
  if (nchunks > 0) {
    // indices of chunks 0 .. 3 (clamped to the last chunk), then rows of
    // chunks 0 and 1
    load_idx(0, I0);
    load_idx(min(1, nchunks - 1), I1);
    load_idx(min(2, nchunks - 1), I2);
    __builtin_amdgcn_s_waitcnt(0);
    take_idx(I0);
    gather(K0, V0);
    if (nchunks > 1) {
      take_idx(I1);
      gather(K1, V1);
    }
    load_idx(min(3, nchunks - 1), I0);
  }
  // Q rows, the first two chunks and the indices of chunks 2 and 3 are
  // complete here on every path, so the loop starts with no loads outstanding
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // After the first chunk mref is its maximum m0 <= max_j t_j <= bound (t the
  // scaled logits).  If bound - m0 <= 124 for every query of the wave, the
  // reference becomes mref = max(m0, bound - 60) for the rest of the item:
  // every later weight is exp2(t - mref) <= 2^60 (no overflow), and the
  // largest one is >= 2^-64 (the fp32 / bf16 exponent range keeps every weight
  // that is not negligible next to it), so the chunk maximum is no longer
  // needed.
  auto decide = [&]() __attribute__((always_inline)) {
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
      for (int v = 0; v < 16; ++v) cneg[v] = -mref * inv_cs;
    }
  };
  const std::false_type general{};
  const std::true_type fast{};
  auto run = [&](auto nst_c) __attribute__((always_inline)) {
    int kc = 1;
    if (nchunks > 0) {
      step(general, nst_c, 0, K0, V0, K2, V2, I2, I1);
      decide();
      // middle chunks, three per iteration (kc = 1 mod 3: chunk kc in buffer 1,
      // kc + 1 in 2, kc + 2 in 0); each gathers the chunk two ahead, so the
      // loop runs while kc + 4 < nchunks.  A wave-uniform choice, made once.
      if (fixed && __builtin_amdgcn_readfirstlane((int)fixed)) {
        for (; kc + 4 < nchunks; kc += 3) {
          step(fast, nst_c, kc, K1, V1, K0, V0, I0, I2);
          step(fast, nst_c, kc + 1, K2, V2, K1, V1, I1, I0);
          step(fast, nst_c, kc + 2, K0, V0, K2, V2, I2, I1);
        }
      }
      // the rest (the last chunk may be partial), and every chunk of a wave
      // that keeps the running maximum: kc = 1 mod 3 here as well, so the
      // buffers stay compile-time choices (selected at run time, they became
      // a table in scratch memory)
      for (; kc < nchunks; kc += 3) {
        step(general, nst_c, kc, K1, V1, K0, V0, I0, I2);
        if (kc + 1 >= nchunks) break;
        step(general, nst_c, kc + 1, K2, V2, K1, V1, I1, I0);
        if (kc + 2 >= nchunks) break;
        step(general, nst_c, kc + 2, K0, V0, K2, V2, I2, I1);
      }
    }
  };
  if (half) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, NST>{});
  float ltot = lsum + __shfl_xor(lsum, 32);
  if (split) {
    // the waves of the second subtile hand their state to their partners
    // through the K / V buffers (free: every step ended with a barrier after
    // its reads, and the last one waited for all gathers): O lane-major in
    // one buffer (64 x D bf16 = 32 D floats per lane) per split block, the
    // references and row sums in V1
    typedef __attribute__((address_space(3))) float lds_f32;
    lds_f32* const xo = (lds_f32*)(mslot == 0 ? K0 : (mslot == 1 ? K1 : (mslot == 2 ? K2 : V0)));
    lds_f32* const xm = (lds_f32*)V1 + mslot * 128;
    if (half && stb) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) xo[(dt * 16 + v) * 64 + lane] = o[dt][v];
      xm[lane] = mref;
      xm[64 + lane] = lsum;
    }
    __syncthreads();
    if (half && stb) return;
    if (half) {
      const float m2 = xm[lane], l2 = xm[64 + lane];
      const float t1 = ltot, t2 = l2 + __shfl_xor(l2, 32);
      // merge: both sides rescaled to the larger reference; a side without
      // weight (an empty subtile) takes no part
      float a1 = 1.f, a2 = 0.f;
      if (t2 > 0.f) {
        if (t1 > 0.f) {
          const float mm = fmaxf(mref, m2);
          a1 = __builtin_amdgcn_exp2f(mref - mm);
          a2 = __builtin_amdgcn_exp2f(m2 - mm);
        } else {
          a1 = 0.f;
          a2 = 1.f;
        }
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][v] = o[dt][v] * a1 + xo[(dt * 16 + v) * 64 + lane] * a2;
      ltot = t1 * a1 + t2 * a2;
    }
  }
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
  const unsigned grid = (unsigned)((plan.work_capacity + 8 * ATT_RUN - 1) / (8 * ATT_RUN) * (8 * ATT_RUN));
#define SCOPE_ATT_ARGS \
  a, plan.work, plan.status, plan.perm_q, plan.q_off, plan.counts_r, plan.sel_off, plan.sel_idx, plan.k_norm_max
  if (g.bf16) {
    // d = 64: 4 waves x 32 queries, 3 waves per SIMD (three workgroups per
    // CU); d = 128: 8 waves x 32 queries, 2 waves per SIMD (one workgroup per
    // CU), so that each K / V chunk gathered into LDS serves 256 queries
    static_assert(32 * ATT_NW64 == ATT_BM && 32 * ATT_NW128 == ATT_BM128, "work-list chunks");
    if (g.d == 64)
      attend_bf16_lds_kernel<64, 3, ATT_NW64><<<grid, 64 * ATT_NW64, 0, s>>>(
          SCOPE_ATT_ARGS, (const uint16_t*)qr, (const uint16_t*)kr, (const uint16_t*)v, (uint16_t*)out);
    else
      attend_bf16_lds_kernel<128, 2, ATT_NW128><<<grid, 64 * ATT_NW128, 0, s>>>(
          SCOPE_ATT_ARGS, (const uint16_t*)qr, (const uint16_t*)kr, (const uint16_t*)v, (uint16_t*)out);
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
