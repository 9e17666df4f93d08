// C ABI of the SCOPE hot path: parameter validation, workspace layout and the
// stage sequence of scope_plan / scope_attend (declared in include/scope.h).
#include <math.h>
#include <string.h>

#include <mutex>

#include "scope_internal.hpp"

namespace scope {

static inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

Geo make_geo(const scope_params& p) {
  Geo g;
  memset(&g, 0, sizeof(g));
  g.BH = p.B * p.H;
  g.T = p.T; g.Hg = p.Hg; g.Wg = p.Wg;
  g.N = p.T * p.Hg * p.Wg;
  g.d = p.d;
  g.Cq = p.Cq; g.Cm = p.Cm; g.iters = p.iters;
  g.off[0] = 0; g.dm[0] = p.d; g.C[0] = p.Cq;
  g.off[1] = 0; g.dm[1] = p.d_t;
  g.off[2] = p.d_t; g.dm[2] = p.d_h;
  g.off[3] = p.d_t + p.d_h; g.dm[3] = p.d_w;
  g.rdm[0] = p.d_t; g.rdm[1] = p.d_h; g.rdm[2] = p.d_w;
  g.nk = 3;
  if (p.flags & SCOPE_FULL_DIM_KEYS) {
    // one key codebook over all d channels; clusterings 2 and 3 unused
    g.nk = 1;
    g.dm[1] = p.d;
    g.off[2] = g.off[3] = 0;
    g.dm[2] = g.dm[3] = 0;
  }
  g.Cmax = p.Cq > p.Cm ? p.Cq : p.Cm;
  g.DPmax = 0; g.CmaxPad = 0;
  for (int m = 0; m < 4; ++m) {
    if (m > 0) g.C[m] = m <= g.nk ? p.Cm : 0;
    g.Cpad[m] = round_up(g.C[m], 32);
    g.dpad[m] = round_up(g.dm[m], 16);
    if (g.dpad[m] > g.DPmax) g.DPmax = g.dpad[m];
    if (g.Cpad[m] > g.CmaxPad) g.CmaxPad = g.Cpad[m];
  }
  g.bf16 = p.dtype == SCOPE_BF16;
  g.permute = (p.flags & SCOPE_PERMUTE_CHANNELS) ? 1 : 0;
  g.online_khead = (p.flags & SCOPE_FIXED_TOPK_ONLY) ? 0 : 1;
  g.seed = p.seed;
  return g;
}

Workspace carve(const Geo& g, const scope_plan_t* plan, char* base) {
  Workspace w;
  memset(&w, 0, sizeof(w));
  size_t o = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + o : nullptr;
    o += (bytes + 255) & ~(size_t)255;
    return p;
  };
  const size_t BH = g.BH, N = g.N;
  const int nrope = g.T * g.rdm[0] / 2 + g.Hg * g.rdm[1] / 2 + g.Wg * g.rdm[2] / 2;
  w.rope_tab = (double2*)take(sizeof(double2) * nrope);
  w.d2 = (double*)take(8 * BH * 4 * N);
  w.nearest = (int32_t*)take(4 * BH * 4 * N);
  w.seeds = (int32_t*)take(4 * BH * 4 * g.Cmax);
  w.qcent = (float*)take(4 * BH * g.Cq * g.d);
  w.kcent = (float*)take(4 * BH * g.Cm * g.d);
  w.cbf = (uint16_t*)take(2 * BH * 4 * g.CmaxPad * g.DPmax);
  w.cnorm = (float*)take(4 * BH * 4 * g.CmaxPad);
  w.labels = (int32_t*)take(4 * BH * 4 * N);
  w.labels_alt = (int32_t*)take(4 * BH * 4 * N);
  w.psum = (double*)take(8 * BH * 4 * (size_t)acc_slices(g) * acc_parts(g) * g.Cmax * acc_sw(g));
  w.pcnt = (int32_t*)take(4 * BH * 4 * (size_t)acc_parts(g) * g.Cmax);
  w.stot = (double*)take(8 * BH * 4 * (size_t)g.Cmax * g.d);
  w.ssm = (double*)take(8 * ssm_elems(g));
  w.ntot = (int32_t*)take(4 * BH * 4 * (size_t)g.Cmax);
  w.codes = (uint16_t*)take(8 * BH * N);
  w.qlab = (int32_t*)take(4 * BH * N);
  w.lut = (double*)take(8 * BH * g.Cq * 3 * g.Cm);
  w.csel = (ClusterSel*)take(sizeof(ClusterSel) * BH * g.Cq);
  w.htot = (int64_t*)take(8 * BH);
  w.hist1 = (int32_t*)take(4 * BH * g.Cq * (size_t)SEL_NB);
  w.seed_sync = (char*)take((size_t)SEED_SYNC_BYTES * BH * 4);
  w.amb = (int4*)take(16 * BH * 4 * N);
  w.amb_cnt = (int32_t*)take(4 * (size_t)(g.iters + 1));
  if (g.permute) {
    const size_t rows = (size_t)(g.bf16 ? 2 : 4) * BH * N * g.d;
    w.qperm = take(rows);
    w.kperm = take(rows);
  }
  w.bytes = o;
  if (plan) {
    if (plan->seeds) w.seeds = plan->seeds;
    if (plan->q_centroids) w.qcent = plan->q_centroids;
    if (plan->k_centroids) w.kcent = plan->k_centroids;
    if (plan->k_codes) w.codes = plan->k_codes;
    if (plan->lut) w.lut = plan->lut;
  }
  return w;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static scope_status validate(const scope_params* p) {
  if (!p) return SCOPE_ERR_INVALID;
  if (p->B < 1 || p->H < 1 || p->T < 1 || p->Hg < 1 || p->Wg < 1) return SCOPE_ERR_INVALID;
  if ((int64_t)p->B * p->H > 65535) return SCOPE_ERR_UNSUPPORTED;
  const int64_t N = (int64_t)p->T * p->Hg * p->Wg;
  if (N > MAX_N) return SCOPE_ERR_UNSUPPORTED;
  if (p->d_t < 2 || p->d_h < 2 || p->d_w < 2 || (p->d_t | p->d_h | p->d_w) & 1) return SCOPE_ERR_INVALID;
  if (p->d_t + p->d_h + p->d_w != p->d) return SCOPE_ERR_INVALID;
  if (p->d != 64 && p->d != 128) return SCOPE_ERR_UNSUPPORTED;
  if (p->Cq < 1 || p->Cm < 1 || p->Cq > N || p->Cm > N) return SCOPE_ERR_INVALID;
  if (p->Cq > MAX_C || p->Cm > MAX_C) return SCOPE_ERR_UNSUPPORTED;
  if (p->iters < 0 || p->iters > 1000) return SCOPE_ERR_INVALID;
  if (!(p->rope_base > 1.0) || !isfinite(p->rope_base)) return SCOPE_ERR_INVALID;
  if (!(p->rho > 0.0 && p->rho <= 1.0)) return SCOPE_ERR_INVALID;
  if (!(p->alpha >= 0.0 && p->alpha <= 1.0)) return SCOPE_ERR_INVALID;
  if (p->dtype != SCOPE_F32 && p->dtype != SCOPE_BF16) return SCOPE_ERR_INVALID;
  if (p->flags &
      ~(SCOPE_USE_INIT_CENTROIDS | SCOPE_PERMUTE_CHANNELS | SCOPE_FIXED_TOPK_ONLY | SCOPE_DENSE | SCOPE_FULL_DIM_KEYS))
    return SCOPE_ERR_INVALID;
  if ((p->flags & SCOPE_DENSE) && p->flags != SCOPE_DENSE) return SCOPE_ERR_INVALID;
  if ((p->flags & SCOPE_FULL_DIM_KEYS) && (p->flags & SCOPE_PERMUTE_CHANNELS)) return SCOPE_ERR_INVALID;
  if (p->dtype == SCOPE_BF16 && !(p->flags & SCOPE_DENSE)) {
    // the bf16 assignment keeps a clustering's whole centroid table in the
    // LDS of one CU (bf16 rows padded to 16 channels + 8, fp32 norms, and the
    // kernel's own 4 KB)
    const Geo g = make_geo(*p);
    for (int m = 0; m <= g.nk; ++m)
      if ((size_t)g.Cpad[m] * (g.dpad[m] + 8) * 2 + (size_t)g.Cpad[m] * 4 + 4 * 1024 > MAX_ASSIGN_LDS)
        return SCOPE_ERR_UNSUPPORTED;
  }
  if (p->flags & SCOPE_PERMUTE_CHANNELS) {
    bool seen[128] = {};
    for (int i = 0; i < p->d; ++i) {
      const int c = p->channel_perm[i];
      if (c >= p->d || seen[c]) return SCOPE_ERR_INVALID;
      seen[c] = true;
    }
  }
  return SCOPE_OK;
}

static int64_t work_cap(const Geo& g) {
  const int bm = att_chunk(g);
  return (int64_t)g.BH * (g.Cq + (g.N + bm - 1) / bm);
}

static scope_status check_plan_core(const scope_plan_t* pl) {
  if (!pl) return SCOPE_ERR_INVALID;
  if (!pl->perm_q || !pl->q_off || !pl->counts_t || !pl->counts_b || !pl->counts_r || !pl->k_head ||
      !pl->sel_off || !pl->sel_idx || !pl->work || !pl->status)
    return SCOPE_ERR_INVALID;
  if (!aligned(pl->sel_off, 8) || !aligned(pl->perm_q, 4) || !aligned(pl->q_off, 4) || !aligned(pl->sel_idx, 4) ||
      !aligned(pl->counts_t, 4) || !aligned(pl->counts_b, 4) || !aligned(pl->counts_r, 4) ||
      !aligned(pl->k_head, 4) || !aligned(pl->work, 8) || !aligned(pl->status, 4))
    return SCOPE_ERR_INVALID;
  if (pl->sel_capacity < 0 || pl->work_capacity < 0) return SCOPE_ERR_INVALID;
  return SCOPE_OK;
}

static scope_status hip_status(hipError_t e) { return e == hipSuccess ? SCOPE_OK : SCOPE_ERR_HIP; }

}  // namespace scope

using namespace scope;

extern "C" {

const char* scope_status_string(scope_status s) {
  switch (s) {
    case SCOPE_OK: return "ok";
    case SCOPE_ERR_INVALID: return "invalid argument";
    case SCOPE_ERR_UNSUPPORTED: return "unsupported configuration";
    case SCOPE_ERR_WORKSPACE: return "workspace too small";
    case SCOPE_ERR_CAPACITY: return "plan buffer too small";
    case SCOPE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

scope_status scope_workspace_size(const scope_params* p, size_t* ws_bytes, int64_t* sel_capacity_worst,
                                  int64_t* work_capacity) {
  const scope_status st = validate(p);
  if (st != SCOPE_OK) return st;
  const Geo g = make_geo(*p);
  if (ws_bytes) *ws_bytes = carve(g, nullptr, nullptr).bytes;
  if (sel_capacity_worst) *sel_capacity_worst = (int64_t)g.BH * g.Cq * g.N;
  if (work_capacity) *work_capacity = work_cap(g);
  return SCOPE_OK;
}

}  // extern "C"

namespace scope {

// scope_plan with optional stage events: ev[i] (if ev and i < nev) is
// recorded on the stream after stage i: 0 RoPE, 1 k-means++, 2 Lloyd,
// 3 cluster permutation + LUT, 4 scoring + selection + work list.
static scope_status plan_impl(const scope_params* p, const void* q, const void* k, void* q_rope, void* k_rope,
                              scope_plan_t* plan, void* ws, size_t ws_bytes, const hipEvent_t* ev, int nev,
                              hipStream_t stream) {
  scope_status st = validate(p);
  if (st != SCOPE_OK) return st;
  st = check_plan_core(plan);
  if (st != SCOPE_OK) return st;
  if (!q || !k || !q_rope || !k_rope || !ws) return SCOPE_ERR_INVALID;
  if (!aligned(q, 256) || !aligned(k, 256) || !aligned(q_rope, 256) || !aligned(k_rope, 256) || !aligned(ws, 256))
    return SCOPE_ERR_INVALID;
  const void* opt[] = {plan->q_centroids, plan->k_centroids, plan->q_labels, plan->k_codes, plan->seeds, plan->lut};
  for (const void* o : opt)
    if (o && !aligned(o, 8)) return SCOPE_ERR_INVALID;
  if (plan->k_norm_max && !aligned(plan->k_norm_max, 4)) return SCOPE_ERR_INVALID;
  if ((p->flags & SCOPE_USE_INIT_CENTROIDS) && (!plan->q_centroids || !plan->k_centroids)) return SCOPE_ERR_INVALID;
  const Geo g = make_geo(*p);
  if (plan->work_capacity < work_cap(g)) return SCOPE_ERR_CAPACITY;
  const Workspace w = carve(g, plan, (char*)ws);
  if (ws_bytes < w.bytes) return SCOPE_ERR_WORKSPACE;

  if (ev && nev > 0)
    for (int i = 0; i < nev && i < 5; ++i)
      if (!ev[i]) return SCOPE_ERR_INVALID;
  hipError_t e = hipSuccess;
#define STEP(x) do { e = (x); if (e != hipSuccess) return hip_status(e); } while (0)
  auto mark = [&](int i) -> hipError_t { return (ev && i < nev) ? hipEventRecord(ev[i], stream) : hipSuccess; };
  STEP(launch_rope(g, *p, q, k, q_rope, k_rope, w, plan->k_norm_max, plan->status + 3, stream));
  STEP(mark(0));
  if (p->flags & SCOPE_DENSE) {
    // dense attention: every query of a head attends to all of its keys
    STEP(launch_dense_plan(g, *plan, stream));
    STEP(launch_worklist(g, *plan, stream));
    for (int i = 1; i < 5; ++i) STEP(mark(i));
    return SCOPE_OK;
  }
  // the clustering reads the rows in proxy channel order
  const void* qc = q_rope;
  const void* kc = k_rope;
  if (g.permute) {
    ChanPerm cp;
    memcpy(cp.p, p->channel_perm, sizeof(cp.p));
    STEP(launch_permute(g, cp, q_rope, k_rope, w, stream));
    qc = w.qperm;
    kc = w.kperm;
  }
  if (!(p->flags & SCOPE_USE_INIT_CENTROIDS)) STEP(launch_seed(g, qc, kc, w, plan->status, stream));
  STEP(mark(1));
  STEP(launch_prep(g, w, stream));
  STEP(launch_assign(g, qc, kc, w, 0, stream));
  for (int it = 1; it <= g.iters; ++it) {
    STEP(launch_update(g, qc, kc, w, it, stream));
    STEP(launch_assign(g, qc, kc, w, it, stream));
  }
  STEP(mark(2));
  STEP(launch_pack(g, w, plan->q_labels, stream));
  STEP(launch_perm(g, w, plan->perm_q, plan->q_off, stream));
  STEP(launch_lut(g, w, stream));
  STEP(mark(3));
  STEP(launch_topp(g, *p, w, plan->counts_t, plan->counts_b, stream));
  STEP(launch_khead(g, *plan, w, stream));
  STEP(launch_final_select(g, *p, w, *plan, stream));
  STEP(launch_worklist(g, *plan, stream));
  STEP(mark(4));
#undef STEP
  return SCOPE_OK;
}

// ---- workspace of the no-allocation entry point ------------------------------
// One fixed array per GPU, in the library's code object (each device that
// loads the library holds its own copy until the process ends).  Host code
// never uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static_assert(SCOPE_NOALLOC_MAX_WORKSPACE % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[SCOPE_NOALLOC_MAX_WORKSPACE];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static scope_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SCOPE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SCOPE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SCOPE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SCOPE_OK;
}

}  // namespace scope

extern "C" {

scope_status scope_plan_noalloc(const scope_params* p, const void* q, const void* k, void* q_rope, void* k_rope,
                                scope_plan_t* plan, hipStream_t stream) {
  const scope_status st = validate(p);
  if (st != SCOPE_OK) return st;
  if (carve(make_geo(*p), nullptr, nullptr).bytes > SCOPE_NOALLOC_MAX_WORKSPACE) return SCOPE_ERR_WORKSPACE;
  void* ws = nullptr;
  const scope_status sst = scratch_of_current_device(&ws);
  if (sst != SCOPE_OK) return sst;
  return plan_impl(p, q, k, q_rope, k_rope, plan, ws, SCOPE_NOALLOC_MAX_WORKSPACE, nullptr, 0, stream);
}

scope_status scope_plan(const scope_params* p, const void* q, const void* k, void* q_rope, void* k_rope,
                        scope_plan_t* plan, void* ws, size_t ws_bytes, hipStream_t stream) {
  return plan_impl(p, q, k, q_rope, k_rope, plan, ws, ws_bytes, nullptr, 0, stream);
}

scope_status scope_plan_timed(const scope_params* p, const void* q, const void* k, void* q_rope, void* k_rope,
                              scope_plan_t* plan, void* ws, size_t ws_bytes, const hipEvent_t* stage_events,
                              int n_events, hipStream_t stream) {
  if (!stage_events || n_events < 1 || n_events > 5) return SCOPE_ERR_INVALID;
  return plan_impl(p, q, k, q_rope, k_rope, plan, ws, ws_bytes, stage_events, n_events, stream);
}

scope_status scope_plan_finalize(const scope_params* p, scope_plan_t* plan, hipStream_t stream) {
  scope_status st = validate(p);
  if (st != SCOPE_OK) return st;
  st = check_plan_core(plan);
  if (st != SCOPE_OK) return st;
  const Geo g = make_geo(*p);
  if (plan->work_capacity < work_cap(g)) return SCOPE_ERR_CAPACITY;
  return hip_status(launch_worklist(g, *plan, stream));
}

scope_status scope_attend(const scope_params* p, const scope_plan_t* plan, const void* q_rope, const void* k_rope,
                          const void* v, void* out, hipStream_t stream) {
  scope_status st = validate(p);
  if (st != SCOPE_OK) return st;
  st = check_plan_core(plan);
  if (st != SCOPE_OK) return st;
  if (!q_rope || !k_rope || !v || !out) return SCOPE_ERR_INVALID;
  if (!aligned(q_rope, 256) || !aligned(k_rope, 256) || !aligned(v, 256) || !aligned(out, 256))
    return SCOPE_ERR_INVALID;
  const Geo g = make_geo(*p);
  if (plan->work_capacity < work_cap(g)) return SCOPE_ERR_CAPACITY;
  return hip_status(launch_attend(g, *plan, q_rope, k_rope, v, out, stream));
}

}  // extern "C"
