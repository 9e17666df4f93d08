"""Writes the full-size parity fixtures full_<workload>_h<bh>_rho<rho>.json.

Runs only the CPU oracle (oracle/scope_oracle.py) on sampled heads of the
full workloads; each fixture holds what the GPU test compares: the k-means++
seeds, hashes of the labels, codes and centroids, the counts t_c, b_c, r_c,
k_head, a hash of every selected key set, the logit gap at every selection
boundary, and the attention output of 16 sampled query rows.

    python tests/golden/make_full_golden.py wan13b_480p 0 [rho ...]
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads  # noqa: E402
from oracle import scope_oracle as O  # noqa: E402


def sha(a, dtype):
    return hashlib.sha256(np.ascontiguousarray(a, dtype=dtype).tobytes()).hexdigest()


def main():
    name, bh = sys.argv[1], int(sys.argv[2])
    w = workloads.CONFIGS[name]
    rhos = [float(x) for x in sys.argv[3:]] or list(w.rhos)
    q, k, v = workloads.generate(w, [bh])
    q, k, v = q[0], k[0], v[0]
    t0 = time.time()
    base = O.workload_head(w, bh, q, k, v, rho=rhos[0], with_attention=False)
    n = base["n"]
    rows = np.sort(np.random.default_rng([20260813, bh, w.index]).choice(w.N, 16, replace=False))
    for rho in rhos:
        t, b, kh, r, sel = O.hybrid_select(base["scores"], n, rho, w.alpha)
        gaps = []
        for c in range(w.Cq):
            if r[c] == 0 or r[c] >= w.N:
                gaps.append(None)
                continue
            srow = base["scores"][c]
            order = O.key_order(srow)
            gaps.append(float(srow[order[r[c] - 1]] - srow[order[r[c]]]))
        out = O.sparse_attention(base["q_rope"], base["k_rope"], v, base["q_labels"], sel, only_rows=rows)
        doc = {
            "source": "oracle/scope_oracle.py via tests/golden/make_full_golden.py",
            "workload": name, "head": bh, "rho": rho,
            "q_seeds": [int(x) for x in base["q_seeds"]],
            "k_seeds": [[int(x) for x in s] for s in base["k_seeds"]],
            "q_labels_sha256": sha(base["q_labels"], np.int32),
            "k_codes_sha256": sha(base["k_codes"], np.int32),
            "q_centroids_sha256": sha(base["q_centroids"], np.float32),
            "k_centroids_sha256": sha(base["k_centroids"], np.float32),
            "n": [int(x) for x in n], "t": [int(x) for x in t], "b": [int(x) for x in b],
            "k_head": int(kh), "r": [int(x) for x in r],
            "sel_sha256": [sha(s, np.int32) for s in sel],
            "boundary_gap": gaps,
            "rows": [int(x) for x in rows],
            "out_rows": [[float(x) for x in out[i]] for i in rows],
            "oracle_seconds": round(time.time() - t0, 1),
        }
        path = os.path.join(HERE, f"full_{name}_h{bh}_rho{rho}.json")
        with open(path, "w") as f:
            json.dump(doc, f, separators=(",", ":"))
        print("wrote", path, round(time.time() - t0, 1), "s", flush=True)


if __name__ == "__main__":
    main()
