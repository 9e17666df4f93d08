"""The proxy-fidelity measurement (bench.py --fidelity) on the GPU path,
against the same measures computed in fp64 on the CPU from the oracle's plan
(the oracle run live on the same inputs): recall of each sampled query's true
top-10% keys by its cluster's key set, softmax mass on that set, Spearman
correlation of the Eq. (6) proxy with the exact logits, and the relative error
of the output rows against dense attention."""
import types

import numpy as np
import pytest
import torch

import bench
import sparse_attention_video_rope_amd as sav
import workloads
from oracle import scope_oracle as O
from tests.scope_gpu import say, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    (workloads.small("fid64", 5, 12, 14, 64, (16, 24, 24), "bf16", 12, 20, H=2, index=130, alpha=0.1), {}),
    (workloads.small("fid128", 4, 11, 15, 128, (16, 56, 56), "bf16", 10, 16, H=2, index=131, alpha=0.1), {}),
    (workloads.small("fidfull", 4, 11, 15, 128, (44, 42, 42), "bf16", 10, 48, H=1, index=132, alpha=0.1),
     {"full_dim_keys": True}),
]


@pytest.mark.parametrize("w,extra", CASES, ids=[c[0].name for c in CASES])
@pytest.mark.parametrize("rho", [0.5, 0.9])
def test_fidelity_measures_match_the_oracle_plan(w, extra, rho):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sav.load()
    say("fidelity", w.name, rho, extra)
    q, k, v = workloads.generate(w)
    qd, kd, vd = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)
    p = sav.params_for(w, rho=rho, **extra)
    pl = sav.Plan(p, debug=True)
    a = types.SimpleNamespace(fidelity_rows=24)
    got = bench._fidelity_of_plan(a, w, p, pl, qd, kd, vd, np.random.default_rng([w.index, 77]))
    # the same rows, measured on the oracle's plan in fp64 on the CPU
    rng = np.random.default_rng([w.index, 77])
    acc = {"recall": [], "mass": [], "spearman": [], "err2": 0.0, "ref2": 0.0}
    dens = 0.0
    for bh in range(w.BH):
        o = O.workload_head(w, bh, q[bh], k[bh], v[bh], rho=rho, **extra)
        rows = torch.from_numpy(np.sort(rng.choice(w.N, a.fidelity_rows, replace=False)))
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
        r = bench.proxy_fidelity_rows(t(o["q_rope"]), t(o["k_rope"]), t(v[bh]), t(o["q_labels"]),
                                      t(np.transpose(o["lut"], (1, 0, 2))), t(o["k_codes"]),
                                      lambda c, o=o: t(o["sel"][c]), t(o["out"]), rows)
        for key in ("recall", "mass", "spearman"):
            acc[key].append(r[key])
        acc["err2"] += r["err2"]
        acc["ref2"] += r["ref2"]
        dens += float(np.sum(o["n"] * o["r"])) / w.N ** 2 / w.BH
    want = {key: float(np.mean(np.concatenate(acc[key]))) for key in ("recall", "mass", "spearman")}
    want["err"] = float(np.sqrt(acc["err2"] / acc["ref2"]))
    say(f"  gpu {got}\n  oracle {want} density {dens:.4f}")
    assert abs(got["density"] - dens) < 1e-12
    assert abs(got["recall"] - want["recall"]) < 1e-12
    assert abs(got["mass"] - want["mass"]) < 1e-9
    assert abs(got["spearman"] - want["spearman"]) < 1e-9
    # the GPU output is bf16 attention, the oracle's fp64: by the triangle
    # inequality the two errors differ by at most ||out_gpu - out_oracle|| /
    # ||dense||, a few 1e-3 for bf16 outputs
    assert abs(got["err"] - want["err"]) < 0.01
