"""The seeded input generators: the later-step stand-in keeps V and moves Q
and K by the stated angle."""
import numpy as np

import workloads


def test_later_step_inputs_rotate_the_draws():
    w = workloads.small("wstep", 3, 8, 9, 64, (16, 24, 24), "f32", 4, 6, index=120, H=1)
    q0, k0, v0 = workloads.generate(w)
    q1, k1, v1 = workloads.generate(w, step=1)
    q2, _, _ = workloads.generate(w, step=2)
    assert np.array_equal(v0, v1)
    assert np.array_equal(q0, workloads.generate(w, step=0)[0])
    # the noise term alone: ||0.1 (n1 - n0)|| ~ 0.1 * 2 sin(a / 2) per element; the
    # field adds a change of the same relative size at unit RMS
    for x0, x1 in ((q0, q1), (k0, k1)):
        rel = np.sqrt(np.mean((x1 - x0) ** 2) / np.mean(x0 ** 2))
        assert 0.02 < rel < 0.1, rel
    rel2 = np.sqrt(np.mean((q2 - q0) ** 2) / np.mean(q0 ** 2))
    assert rel2 > 1.5 * np.sqrt(np.mean((q1 - q0) ** 2) / np.mean(q0 ** 2))
