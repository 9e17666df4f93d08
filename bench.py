"""Benchmark of the SCOPE hot path (plan + attend) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config hunyuan_720p] [--rho 0.9]

One step = scope_plan (3D RoPE, k-means++ and Lloyd on queries and the three
key subspaces, LUT, proxy scoring, hybrid Top-p / k_head selection) plus
scope_attend (gathered exact attention), on every head of one batch of
synthetic inputs resident in HBM.  Prints one JSON line.

  value      effective TFLOP/s on selected keys over the whole step:
             4 d sum_c n_c r_c / (t_plan + t_attend)
  roofline   the attention kernel (bf16 MFMA): its algorithmic flops per
             launch / its average launch time, HIP events on its stream
  cpu_baseline  the CPU oracle on one head of the same workload
  --fidelity instead: the proxy-fidelity sweep (recall of each sampled query's
             true top-10% keys by its cluster's key set, softmax mass on that
             set, rank correlation of the Eq. (6) proxy with the exact logits,
             error against dense attention) over rho in {0.5 .. 0.99} at
             alpha = 0.1, three input seeds; one JSON line
  warm_start the same step on a later denoising step's inputs (the workload's
             step-1 stand-in), with Lloyd started from the step-0 plan's
             centroids (SCOPE_USE_INIT_CENTROIDS, no k-means++) and fewer
             iterations; timed and compared with a full plan of those inputs
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    # the largest workload (HunyuanVideo-like 720p, 129 frames), the setting of the SCOPE abstract's headline
    ap.add_argument("--config", default="hunyuan_720p")
    ap.add_argument("--rho", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fidelity", action="store_true", help="run the proxy-fidelity sweep instead of the bench")
    ap.add_argument("--fidelity-rows", type=int, default=32, help="sampled query rows per head for --fidelity")
    ap.add_argument("--partition", choices=("rope", "random", "full"), default="rope",
                    help="--fidelity: proxy subspaces from the 3D-RoPE ranges, from a seeded random channel order, "
                         "or no partition: one key codebook over all d channels (the cluster-level proxy) with "
                         "--full-cm centroids")
    ap.add_argument("--full-cm", type=int, default=None,
                    help="--partition full: key centroids of the one codebook (default 3 Cm, the centroid budget "
                         "of the three subspace codebooks, lowered to the largest the library supports: its "
                         "bf16 table must fit in one CU's LDS)")
    ap.add_argument("--heads", type=int, default=None,
                    help="--fidelity: run only the first H heads of the workload (sampled heads at the 720p sizes)")
    ap.add_argument("--selection", choices=("scope", "fixed-topk"), default="scope",
                    help="--fidelity: the full selection, or Top-p / fixed Top-k without the online per-head Top-k "
                         "at a rho matched to the full selection's density")
    ap.add_argument("--layers", type=int, default=40,
                    help="attention layers per denoising step of the dense-prefix schedule (the pages fix only "
                         "that the first layer is dense at every step; the count is a stand-in)")
    ap.add_argument("--dense-steps", type=float, default=None,
                    help="fraction of denoising steps run dense (default: 0.2 for the Wan-like workloads, "
                         "0.1 otherwise, as the pages give for Wan and HunyuanVideo)")
    ap.add_argument("--no-dense-prefix", action="store_true", help="leave out the dense-prefix measurement")
    ap.add_argument("--warm-iters", type=int, default=2,
                    help="Lloyd iterations of the warm-started plan (negative: skip the warm-start measurement)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "attend_traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters (used if present and current)")
    ap.add_argument("--profile-pass", action="store_true",
                    help="one plan, 3 attention launches and 3 plain 256 MiB streaming copies (torch.neg), for "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the counter CSVs of two --profile-pass runs into --traffic-json")
    return ap.parse_args()


COPY_BYTES = 256 << 20


def profile_pass(a):
    """Launches whose FETCH_SIZE / WRITE_SIZE counters give the attention kernel's HBM traffic.

    The copy (torch.neg on 256 MiB of fp32) reads and writes COPY_BYTES each: the
    ratio of its counters to COPY_BYTES calibrates the counters' unit."""
    import torch
    import sparse_attention_video_rope_amd as sav
    import workloads
    w = workloads.CONFIGS[a.config]
    rho = w.rho if a.rho is None else a.rho
    p = sav.params_for(w, rho=rho)
    q, k, v = workloads.generate(w)
    dev = torch.device("cuda:0")
    to = lambda x: torch.from_numpy(x.reshape(-1)).to(torch.bfloat16 if w.dtype == "bf16" else torch.float32).to(dev)
    qd, kd, vd = to(q), to(k), to(v)
    pl = sav.Plan(p, device=dev, debug=False)
    qr, kr = torch.empty_like(qd), torch.empty_like(kd)
    out = torch.empty_like(vd)
    sav.plan(p, qd, kd, pl, qr, kr)
    for _ in range(3):
        sav.attend(p, pl, qr, kr, vd, out)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"profile_pass": w.name, "rho": rho}), flush=True)


def traffic_from(a):
    """Per-launch HBM bytes of the attention kernel from two rocprofv3 counter CSVs."""
    import csv
    import workloads

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    out = {}
    for counter, path in (("FETCH_SIZE", a.traffic_from[0]), ("WRITE_SIZE", a.traffic_from[1])):
        vals = per_kernel(path, counter)
        att = [v for n, v in vals.items() if "attend_" in n]
        cp = [v for n, v in vals.items() if "neg" in n]
        if len(att) != 1 or len(cp) != 1:
            raise SystemExit(f"{counter}: expected one attention and one copy kernel in {path}")
        kib_att, kib_cp = float(np.mean(att[0])), float(np.mean(cp[0]))
        factor = COPY_BYTES / (kib_cp * 1024.0)
        out[counter] = {"attend_kib_per_launch": kib_att, "copy_kib_per_launch": kib_cp,
                        "copy_bytes": COPY_BYTES, "factor": factor,
                        "attend_bytes_per_launch": kib_att * 1024.0 * factor}
    w = workloads.CONFIGS[a.config]
    rho = w.rho if a.rho is None else a.rho
    doc = {"workload": w.name, "rho": rho, "kernel_source_sha": _attend_sha(),
           "bytes_per_launch": out["FETCH_SIZE"]["attend_bytes_per_launch"] +
                               out["WRITE_SIZE"]["attend_bytes_per_launch"],
           "counters": out}
    with open(a.traffic_json, "w") as f:
        json.dump(doc, f, indent=1)
    print(json.dumps(doc))


def cpu_baseline(w, rho, pairs_head0):
    """The oracle as it stands, timed stage by stage on head 0 of the workload.

    A whole 720p head takes the oracle over ten minutes, so each stage runs on
    a bounded sample and its time is scaled to the full head (the stage costs
    follow the sample sizes linearly):
      S1   RoPE of Q and K: the whole head;
      S2a  k-means++: the first SEED_DRAWS draws of each of the four
           clusterings (every draw is one pass over the N points), x C / draws;
      S2bc Lloyd: one assignment of LLOYD_PTS points of each clustering,
           x (N / points) x (iters + 1), and one centroid mean over all N
           points (seeded labels), x iters;
      S3-5 lookup tables, Eq. (6) proxy logits and the hybrid selection of
           SEL_CLUSTERS query clusters, x Cq / clusters;
      S6   exact attention of ATT_CLUSTERS clusters of N / Cq queries over
           r keys each, r the head's mean selected-key count, x Cq / clusters.
    The inputs of S3-S6 (centroids, codes, labels, key sets) only need the
    right shapes, so they are taken from the head's rows and a seeded
    generator.  value = 4 d sum_c n_c r_c of head 0 (the GPU plan's selected
    pairs, the flops the metric counts) / the scaled oracle time."""
    import workloads
    from oracle import scope_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    SEED_DRAWS, LLOYD_PTS, SEL_CLUSTERS, ATT_CLUSTERS = 8, 4096, 8, 4
    q, k, v = workloads.generate(w, [0])
    q, k, v = q[0], k[0], v[0]
    N, d, grid = w.N, w.d, (w.T, w.Hg, w.Wg)
    rng = np.random.default_rng([w.index, 99])
    st = {}
    t0 = time.perf_counter()
    qr = O.round_storage(O.rope_3d(q, grid, w.split, w.rope_base), w.dtype)
    kr = O.round_storage(O.rope_3d(k, grid, w.split, w.rope_base), w.dtype)
    st["S1"] = time.perf_counter() - t0
    offs = O.subspace_offsets(w.split)
    sets = [(qr, w.Cq)] + [(kr[:, o:o + dm], w.Cm) for o, dm in zip(offs, w.split)]
    st["S2a"] = st["S2bc"] = 0.0
    pts = min(N, LLOYD_PTS)
    for m, (X, C) in enumerate(sets):
        X = np.ascontiguousarray(X)
        t0 = time.perf_counter()
        O.kmeanspp_seeds(X, min(SEED_DRAWS, C), w.kmeans_seed, 0, m)
        st["S2a"] += (time.perf_counter() - t0) * C / min(SEED_DRAWS, C)
        M = X[rng.choice(N, C, replace=False)]
        t0 = time.perf_counter()
        O.assign(X[:pts], O.round_bf16(M) if w.dtype == "bf16" else M)
        t1 = time.perf_counter()
        O.centroid_means(X, rng.integers(0, C, N), M)
        t2 = time.perf_counter()
        st["S2bc"] += (t1 - t0) * (w.iters + 1) * N / pts + (t2 - t1) * w.iters
    qc = qr[rng.choice(N, w.Cq, replace=False)]
    kc = kr[rng.choice(N, w.Cm, replace=False)]
    codes = rng.integers(0, w.Cm, (N, 3))
    n_c = np.bincount(rng.integers(0, w.Cq, N), minlength=w.Cq)
    nsel = min(SEL_CLUSTERS, w.Cq)
    t0 = time.perf_counter()
    P = O.lookup_tables(qc, kc, w.split)
    s = O.proxy_logits(P[:, :nsel], codes, d)
    O.hybrid_select(s, n_c[:nsel], rho, w.alpha)
    st["S3-5"] = (time.perf_counter() - t0) * w.Cq / nsel
    r_mean = int(round(pairs_head0 / N))
    na = min(ATT_CLUSTERS, w.Cq)
    nq = N // w.Cq
    labels = np.full(N, na, dtype=np.int64)
    labels[:na * nq] = np.repeat(np.arange(na), nq)
    sel = [np.sort(rng.choice(N, r_mean, replace=False)) for _ in range(na)]
    t0 = time.perf_counter()
    O.sparse_attention(qr, kr, v, labels, sel)
    st["S6"] = (time.perf_counter() - t0) * w.Cq / na
    total = sum(st.values())
    flops = 4.0 * w.d * pairs_head0
    return {"value": flops / total / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"head 0 of {w.BH} ({w.name}), oracle stages on bounded samples scaled to the head: RoPE "
                      f"whole; k-means++ {SEED_DRAWS} draws per clustering; Lloyd assignment {pts} points, means all; "
                      f"LUT + proxy + "
                      f"selection {nsel} clusters; attention {na} clusters of {nq} queries x {r_mean} keys",
            "seconds_scaled": {k_: round(v_, 2) for k_, v_ in st.items()}, "seconds_head": round(total, 2),
            "host_cpus": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def _min_dist_sum(x, c):
    """sum over rows of x of the squared distance to the nearest row of c (per head, fp32)."""
    import torch
    tot = 0.0
    for h in range(x.shape[0]):
        tot += float(torch.cdist(x[h], c[h]).pow(2).min(dim=1).values.double().sum())
    return tot


def _inertia(w, qr, kr, pl):
    """k-means objective of the plan's query centroids and of its three key subspace codebooks."""
    import torch
    BH, N, d = w.BH, w.N, w.d
    q = qr.view(BH, N, d).float()
    k = kr.view(BH, N, d).float()
    cq = pl.q_centroids.view(BH, w.Cq, d)
    ck = pl.k_centroids.view(BH, w.Cm, d)
    kin, o = 0.0, 0
    for dm in w.split:
        kin += _min_dist_sum(k[:, :, o:o + dm].contiguous(), ck[:, :, o:o + dm].contiguous())
        o += dm
    return _min_dist_sum(q, cq), kin


def _dense_rel_l2(w, qr, kr, vd, outs, torch):
    """||out - dense attention|| / ||dense attention|| for each of outs (fp32, head by head)."""
    BH, N, d = w.BH, w.N, w.d
    q, k, v = (t.view(BH, N, d) for t in (qr, kr, vd))
    num = [0.0] * len(outs)
    den = 0.0
    rows = 4096                                   # query rows per block (bounded memory at any N)
    for h in range(BH):
        kt, vh = k[h].float().t().contiguous(), v[h].float()
        for r0 in range(0, N, rows):
            qh = q[h, r0:r0 + rows].float()
            ref = torch.softmax((qh @ kt) / float(np.sqrt(d)), dim=1) @ vh
            den += float(ref.double().pow(2).sum())
            for i, o in enumerate(outs):
                num[i] += float((o.view(BH, N, d)[h, r0:r0 + rows].float() - ref).double().pow(2).sum())
    return [float(np.sqrt(x / den)) for x in num]


def warm_start(a, w, rho, qd, kd, vd, sav, torch):
    """Codebook reuse across denoising steps on the workload's step-1 stand-in inputs."""
    import workloads
    dev = qd.device
    p_cold = sav.params_for(w, rho=rho)
    p_warm = sav.params_for(w, rho=rho, iters=a.warm_iters, init_centroids=True)
    to = lambda x: torch.from_numpy(x.reshape(-1)).to(qd.dtype).to(dev)
    q1, k1, _ = workloads.generate(w, step=1)
    q1d, k1d = to(q1), to(k1)
    del q1, k1
    qr, kr = torch.empty_like(qd), torch.empty_like(kd)
    pl0 = sav.Plan(p_cold, device=dev, debug=False, centroids=True)
    sav.plan(p_cold, qd, kd, pl0, qr, kr)                      # step 0: full plan
    # step 1, full plan: the reference the warm start is compared with
    plc = sav.Plan(p_cold, device=dev, debug=False, centroids=True)
    sav.plan(p_cold, q1d, k1d, plc, qr, kr)
    out_c = sav.attend(p_cold, plc, qr, kr, vd)
    inert_c = _inertia(w, qr, kr, plc)
    plw = sav.Plan(p_warm, device=dev, debug=False, centroids=True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.warmup + a.steps)]
    out_w = torch.empty_like(vd)
    for e0, e1, e2 in ev:
        plw.q_centroids.copy_(pl0.q_centroids)
        plw.k_centroids.copy_(pl0.k_centroids)
        e0.record()
        sav.plan(p_warm, q1d, k1d, plw, qr, kr)
        e1.record()
        sav.attend(p_warm, plw, qr, kr, vd, out_w)
        e2.record()
    torch.cuda.synchronize()
    ev = ev[a.warmup:]
    plan_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1, _ in ev]))
    step_ms = float(np.mean([e0.elapsed_time(e2) for e0, _, e2 in ev]))
    inert_w = _inertia(w, qr, kr, plw)

    def density(pl):
        n = (pl.q_off.view(w.BH, w.Cq + 1)[:, 1:] - pl.q_off.view(w.BH, w.Cq + 1)[:, :-1]).double()
        return float((n * pl.counts_r.view(w.BH, w.Cq).double()).sum()) / (w.BH * float(w.N) ** 2)

    dc, dw = out_c.float(), out_w.float()
    err_w, err_c = _dense_rel_l2(w, qr, kr, vd, [out_w, out_c], torch)
    return {"inputs": "step-1 stand-in (every Gaussian draw of Q and K rotated 0.05 rad towards a fresh one)",
            "init": "centroids of the full plan of the step-0 inputs", "lloyd_iters": a.warm_iters,
            "plan_ms": round(plan_ms, 4), "step_ms": round(step_ms, 4),
            "q_inertia_vs_full": round(inert_w[0] / inert_c[0], 5),
            "k_inertia_vs_full": round(inert_w[1] / inert_c[1], 5),
            "density": round(density(plw), 4), "density_full": round(density(plc), 4),
            "out_rel_l2_vs_full": float(torch.linalg.vector_norm(dw - dc) / torch.linalg.vector_norm(dc)),
            "out_rel_l2_vs_dense": err_w, "out_rel_l2_vs_dense_full": err_c}


def _avg_ranks(x):
    """Ranks 0..n-1 of a 1-D tensor, equal values sharing the mean of their ranks (fp64)."""
    import torch
    srt, order = torch.sort(x)
    _, inv, cnt = torch.unique_consecutive(srt, return_inverse=True, return_counts=True)
    start = torch.cumsum(cnt, 0) - cnt
    r = torch.empty_like(x, dtype=torch.float64)
    r[order] = (start.double() + (cnt.double() - 1.0) / 2.0)[inv]
    return r


def proxy_fidelity_rows(qr, kr, v, labels, lut, codes, sets, out, rows, top_frac=0.1):
    """Proxy fidelity at sampled query rows of one head (fp64 throughout).

    qr, kr, v, out [N, d]; labels [N] query clusters; lut [Cq, 3, Cm] = P^m[c][z]
    (no 1/sqrt(d)); codes [N, 3] key codes; sets(c) -> key indices of S_c;
    rows: the query rows.  Per row i with cluster c: recall of the true top
    ceil(top_frac N) keys by exact logit within S_c, softmax mass on S_c,
    Spearman correlation (mean ranks for ties) of the Eq. (6) proxy s[c, :]
    with the exact logits q_i . k_j / sqrt(d).  Also the squared error of the
    output rows against dense attention and the squared norm of the latter."""
    import math
    import torch
    N, d = kr.shape
    lg = (qr[rows].double() @ kr.double().t()) / math.sqrt(d)
    cs = labels[rows].long()
    cd = codes.long()
    lt = lut.double()
    prox = (lt[cs, 0][:, cd[:, 0]] + lt[cs, 1][:, cd[:, 1]] + lt[cs, 2][:, cd[:, 2]]) / math.sqrt(d)
    member = torch.zeros(len(rows), N, dtype=torch.bool, device=kr.device)
    for i, c in enumerate(cs.tolist()):
        member[i, sets(c).long()] = True
    kt = math.ceil(top_frac * N)
    top = lg.topk(kt, dim=1).indices
    recall = member.gather(1, top).double().mean(1)
    p = torch.softmax(lg, dim=1)
    mass = (p * member.double()).sum(1)
    rho_s = []
    for i in range(len(rows)):
        a, b = _avg_ranks(prox[i]), _avg_ranks(lg[i])
        a, b = a - a.mean(), b - b.mean()
        rho_s.append(float((a * b).sum() / torch.sqrt((a * a).sum() * (b * b).sum())))
    dense = p @ v.double()
    err2 = float((out[rows].double() - dense).pow(2).sum())
    return {"recall": recall.cpu().numpy(), "mass": mass.cpu().numpy(), "spearman": np.array(rho_s),
            "err2": err2, "ref2": float(dense.pow(2).sum())}


FID_RHOS = (0.5, 0.7, 0.9, 0.95, 0.99)
FID_ALPHA = 0.1
FID_REPS = 3


def _density(w, pl):
    n = (pl.q_off.view(w.BH, w.Cq + 1)[:, 1:] - pl.q_off.view(w.BH, w.Cq + 1)[:, :-1]).double()
    return float((n * pl.counts_r.view(w.BH, w.Cq).double()).sum()) / (w.BH * float(w.N) ** 2)


def _fidelity_of_plan(a, w, p, pl, qd, kd, vd, rng):
    """Plan + attend with p, then the proxy_fidelity_rows measures over every head."""
    import torch
    import sparse_attention_video_rope_amd as sav
    qr, kr, _ = sav.plan(p, qd, kd, pl)
    out = sav.attend(p, pl, qr, kr, vd)
    torch.cuda.synchronize()
    assert int(pl.status[1]) == 0, "selected-key capacity overflow"
    N, d, Cq, Cm = w.N, w.d, w.Cq, w.Cm
    sel_off = pl.sel_off.cpu().numpy()
    acc = {"recall": [], "mass": [], "spearman": [], "err2": 0.0, "ref2": 0.0}
    for bh in range(w.BH):
        hs = slice(bh * N * d, (bh + 1) * N * d)
        rows = torch.from_numpy(np.sort(rng.choice(N, a.fidelity_rows, replace=False))).to(qd.device)
        base = bh * Cq
        sets = lambda c, base=base: pl.sel_idx[int(sel_off[base + c]):int(sel_off[base + c + 1])]
        r = proxy_fidelity_rows(
            qr[hs].view(N, d), kr[hs].view(N, d), vd[hs].view(N, d), pl.q_labels[bh * N:(bh + 1) * N],
            pl.lut[bh * Cq * 3 * Cm:(bh + 1) * Cq * 3 * Cm].view(Cq, 3, Cm),
            pl.k_codes[bh * N * 4:(bh + 1) * N * 4].view(N, 4)[:, :3].int() & 0xFFFF, sets,
            out[hs].view(N, d), rows)
        for key in ("recall", "mass", "spearman"):
            acc[key].append(r[key])
        acc["err2"] += r["err2"]
        acc["ref2"] += r["ref2"]
    res = {key: float(np.mean(np.concatenate(acc[key]))) for key in ("recall", "mass", "spearman")}
    res["density"] = _density(w, pl)
    res["err"] = float(np.sqrt(acc["err2"] / acc["ref2"]))
    return res


def _matched_rho(w, sav, qd, kd, pl, target, lo, perm, extra=None, steps=14):
    """rho of the fixed-Top-k-only selection whose realised density is closest to target (bisection;
    the density is nondecreasing in rho)."""
    import torch
    best = (float("inf"), 1.0)
    hi = 1.0
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        p = sav.params_for(w, rho=mid, channel_perm=perm, online_khead=False, **(extra or {}))
        sav.plan(p, qd, kd, pl)
        torch.cuda.synchronize()
        dens = _density(w, pl)
        best = min(best, (abs(dens - target), mid))
        if dens < target:
            lo = mid
        else:
            hi = mid
    return best[1]


def fidelity(a):
    """Proxy-fidelity sweep on the GPU plans of the workload (three input seeds).

    --selection fixed-topk: at every rho, the selection without the online
    per-head Top-k (r_c = b_c), with its own rho' set so that its realised
    density matches the full method's at rho (the Fig. 7 comparison)."""
    import torch
    import sparse_attention_video_rope_amd as sav
    import workloads
    w0 = workloads.CONFIGS[a.config]
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w0.dtype == "bf16" else torch.float32
    keys = ("recall", "mass", "spearman", "density", "err", "rho_used")
    res = {rho: {k: [] for k in keys} for rho in FID_RHOS}
    extra = {}
    if a.partition == "full":
        extra = {"full_dim_keys": True}
        cm = a.full_cm or min(1024, 3 * w0.Cm)
        while cm > 32:     # the largest supported codebook up to the request (LDS holds its table)
            try:
                sav.sizes(sav.params_for(w0.with_(Cm=cm), **extra))
                break
            except sav.ScopeError:
                cm -= 32 if cm % 32 == 0 else cm % 32
        w0 = w0.with_(Cm=cm)
    if a.heads:
        w0 = w0.with_(H=min(a.heads, w0.H))
    for rep in range(FID_REPS):
        w = w0.with_(index=w0.index + 1000 * rep, alpha=FID_ALPHA)
        q, k, v = workloads.generate(w)
        qd, kd, vd = (torch.from_numpy(x.reshape(-1)).to(dt).to(dev) for x in (q, k, v))
        del q, k, v
        perm = None
        if a.partition == "random":
            perm = np.random.default_rng([w.index, 11]).permutation(w.d).tolist()
        pl = sav.Plan(sav.params_for(w, channel_perm=perm, **extra), device=dev, debug=True)
        for rho in FID_RHOS:
            rng = np.random.default_rng([w.index, 77])     # the same sampled rows at every rho
            p = sav.params_for(w, rho=rho, channel_perm=perm, **extra)
            rho_used = rho
            if a.selection == "fixed-topk":
                sav.plan(p, qd, kd, pl)
                torch.cuda.synchronize()
                rho_used = _matched_rho(w, sav, qd, kd, pl, _density(w, pl), rho, perm, extra)
                p = sav.params_for(w, rho=rho_used, channel_perm=perm, online_khead=False, **extra)
            r = _fidelity_of_plan(a, w, p, pl, qd, kd, vd, rng)
            r["rho_used"] = rho_used
            for key in keys:
                res[rho][key].append(r[key])
            print(json.dumps({"rep": rep, "rho": rho, **{k_: round(r[k_], 5) for k_ in keys}}), flush=True)
        del pl
    summary = {rho: {key: {"mean": float(np.mean(vals)), "std": float(np.std(vals, ddof=1))}
                     for key, vals in e.items()} for rho, e in res.items()}
    print(json.dumps({"fidelity": w0.name, "partition": a.partition, "key_centroids": w0.Cm, "heads": w0.BH,
                      "selection": a.selection, "alpha": FID_ALPHA,
                      "reps": FID_REPS, "rows_per_head": a.fidelity_rows, "top_frac": 0.1,
                      "by_rho": {str(r): v for r, v in summary.items()}}), flush=True)


def main():
    a = parse()
    if a.traffic_from:
        return traffic_from(a)
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 (heads shard across GPUs, "
                                   "see the design notes)"}))
        sys.exit(2)
    if a.profile_pass:
        return profile_pass(a)
    if a.fidelity:
        return fidelity(a)
    import torch
    import sparse_attention_video_rope_amd as sav
    import workloads

    w = workloads.CONFIGS[a.config]
    rho = w.rho if a.rho is None else a.rho
    p = sav.params_for(w, rho=rho)
    q, k, v = workloads.generate(w)
    dev = torch.device("cuda:0")
    to = lambda x: torch.from_numpy(x.reshape(-1)).to(torch.bfloat16 if w.dtype == "bf16" else torch.float32).to(dev)
    qd, kd, vd = to(q), to(k), to(v)
    del q, k, v
    pl = sav.Plan(p, device=dev, debug=False)
    qr, kr = torch.empty_like(qd), torch.empty_like(kd)
    out = torch.empty_like(vd)

    def step():
        sav.plan(p, qd, kd, pl, qr, kr)
        sav.attend(p, pl, qr, kr, vd, out)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for e0, e1, e2 in ev:
        e0.record()
        sav.plan(p, qd, kd, pl, qr, kr)
        e1.record()
        sav.attend(p, pl, qr, kr, vd, out)
        e2.record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / a.steps
    plan_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1, _ in ev]))
    att_ms = float(np.mean([e1.elapsed_time(e2) for _, e1, e2 in ev]))

    n = (pl.q_off.view(w.BH, w.Cq + 1)[:, 1:] - pl.q_off.view(w.BH, w.Cq + 1)[:, :-1]).double()
    r = pl.counts_r.view(w.BH, w.Cq).double()
    pairs = float((n * r).sum())
    flops = 4.0 * w.d * pairs
    density = pairs / (w.BH * float(w.N) ** 2)
    kh = pl.k_head.cpu().numpy()
    status = pl.status.cpu().numpy()
    assert status[1] == 0, "selected-key capacity overflow"
    assert status[2] == 0, "k-means++ workgroups stopped waiting on each other"

    traffic = None
    if os.path.exists(a.traffic_json):
        try:
            t = json.load(open(a.traffic_json))
            if t.get("workload") == w.name and abs(t.get("rho", -1) - rho) < 1e-12 and \
                    t.get("kernel_source_sha") == _attend_sha():
                traffic = t.get("bytes_per_launch")
        except Exception:
            traffic = None
    achieved = flops / (att_ms * 1e-3) / 1e12
    stages = stage_breakdown(w, p, sav, pl, qd, kd, vd, qr, kr, out, torch, pairs)
    line = {
        "metric": "SCOPE attention layer latency (ms) + effective TFLOP/s on selected keys, 1 GPU",
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded smooth-field Q/K + noise, V ~ N(0,1))",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "tokens": w.N,
                   "grid": [w.T, w.Hg, w.Wg], "head_dim": w.d, "rope_split": list(w.split), "Cq": w.Cq,
                   "Cm": w.Cm, "lloyd_iters": w.iters, "rho": rho, "alpha": w.alpha},
        "latency_ms": {"step": round(ms, 4), "plan": round(plan_ms, 4), "attend": round(att_ms, 4)},
        "stages": stages,
        "attend_tflops": round(achieved, 2),
        "density": round(density, 4),
        "k_head": {"min": int(kh.min()), "mean": float(kh.mean()), "max": int(kh.max())},
        "roofline": {"kernel": "attend_bf16_lds_kernel" if w.dtype == "bf16" else "attend_f32_kernel",
                     "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "wall_s": round(wall, 3),
    }
    if not a.no_dense_prefix:
        line["dense_prefix"] = dense_prefix(a, w, qd, kd, vd, sav, torch, ms)
    if a.warm_iters >= 0:
        line["warm_start"] = warm_start(a, w, rho, qd, kd, vd, sav, torch)
    if not a.no_cpu_baseline:
        nh0 = (pl.q_off[1:w.Cq + 1] - pl.q_off[:w.Cq]).double()
        line["cpu_baseline"] = cpu_baseline(w, rho, float((nh0 * pl.counts_r[:w.Cq].double()).sum()))
    print(json.dumps(line), flush=True)


def stage_breakdown(w, p, sav, pl, qd, kd, vd, qr, kr, out, torch, pairs, reps=3):
    """Per-stage times of the step (medians of `reps` extra plans with stage
    events, scope_plan_timed, plus the attention launch) and, for the
    bandwidth-bound stages, GB/s on their algorithmic bytes: S1 reads Q, K and
    writes Q', K' (8 N d bytes per head in bf16); S4+S5 per head, with the
    Cq x N fp32 score matrix written once and read once, 6 N bytes of key
    codes, the three Cq x Cm LUTs and 4 bytes per selected index:
    8 Cq N + 6 N + 12 Cq Cm + 4 sum_c r_c (this build recomputes the scores
    from the codes and never stores them, so it moves fewer bytes)."""
    runs = []
    for _ in range(reps):
        ms = sav.plan_timed(p, qd, kd, pl, qr, kr)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sav.attend(p, pl, qr, kr, vd, out)
        e1.record()
        e1.synchronize()
        ms["attend"] = e0.elapsed_time(e1)
        runs.append(ms)
    med = {k: float(np.median([r[k] for r in runs])) for k in runs[0]}
    names = {"rope": "S1_rope", "kmeanspp": "S2a_kmeanspp", "lloyd": "S2bc_lloyd", "perm_lut": "S3_perm_lut",
             "score_select": "S4S5_score_select", "attend": "S6_attend"}
    out_ms = {names[k]: round(v, 4) for k, v in med.items()}
    esz = 2 if w.dtype == "bf16" else 4
    sum_r = float(pl.counts_r.double().sum())
    b_rope = 4.0 * esz * w.BH * w.N * w.d
    b_sel = w.BH * (8.0 * w.Cq * w.N + 6.0 * w.N + 12.0 * w.Cq * w.Cm) + 4.0 * sum_r
    gbs = lambda b, ms: round(b / (ms * 1e-3) / 1e9, 1)
    return {"ms": out_ms,
            "S1_rope": {"bound": "hbm", "bytes": b_rope, "GB/s": gbs(b_rope, med["rope"]),
                        "frac": round(b_rope / (med["rope"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "S4S5_score_select": {"bound": "hbm", "bytes": b_sel, "GB/s": gbs(b_sel, med["score_select"]),
                                  "frac": round(b_sel / (med["score_select"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "S6_attend": {"bound": "mfma", "TFLOP/s": round(4.0 * w.d * pairs / (med["attend"] * 1e-3) / 1e12, 2)}}


def dense_prefix(a, w, qd, kd, vd, sav, torch, scope_ms):
    """The dense-prefix schedule of the SCOPE paper (referee report, major
    comment 3): the first attention layer is dense at every denoising step and
    the first 20% (Wan) or 10% (HunyuanVideo) of the steps are dense
    throughout.  Measures one dense layer (SCOPE_DENSE: RoPE, the all-keys
    plan and the same attention kernel) and blends it with the sparse step:
    share of dense layer-steps f = 1/L + (1 - 1/L) p, blended = f t_dense +
    (1 - f) t_scope per layer-step."""
    p_dense = sav.params_for(w, dense=True)
    pl = sav.Plan(p_dense, device=qd.device, debug=False)
    qr, kr, out = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(a.warmup + a.steps)]
    for e0, e1 in ev:
        e0.record()
        sav.plan(p_dense, qd, kd, pl, qr, kr)
        sav.attend(p_dense, pl, qr, kr, vd, out)
        e1.record()
    torch.cuda.synchronize()
    dense_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev[a.warmup:]]))
    frac = a.dense_steps if a.dense_steps is not None else (0.2 if w.name.startswith("wan") else 0.1)
    L = max(1, a.layers)
    f = 1.0 / L + (1.0 - 1.0 / L) * frac
    blended = f * dense_ms + (1.0 - f) * scope_ms
    dense_flops = 4.0 * w.d * float(w.N) ** 2 * w.BH
    return {"dense_step_ms": round(dense_ms, 4), "dense_tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 2),
            "layers": L, "dense_step_fraction": frac, "dense_share": round(f, 5),
            "blended_ms_per_layer_step": round(blended, 4),
            "attention_speedup_vs_all_dense": round(dense_ms / blended, 4)}


def _attend_sha():
    import hashlib
    src = os.path.join(ROOT, "sparse_attention_video_rope_amd", "csrc", "attend.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


if __name__ == "__main__":
    main()
