"""The parity tests' per-frame diagnostics find a difference planted in one frame."""
import numpy as np

from tests.helpers import frame_diagnostics


def test_frame_diagnostics_finds_the_planted_frame():
    rng = np.random.default_rng(3)
    B, T, P, H, d = 2, 5, 7, 3, 4
    r = rng.standard_normal((B, T * P, H, d))
    g = r.copy()
    g[1, 3 * P + 2, 1, 0] += 0.25          # one value of frame 3
    g[0, 1 * P + 4, 2, 3] -= 0.01          # a smaller one in frame 1
    f, e, m = frame_diagnostics(g, r, P)
    assert f == 3
    fr = slice(3 * P, 4 * P)
    assert np.isclose(e, np.linalg.norm((g - r)[:, fr]) / np.linalg.norm(r[:, fr]))
    assert np.isclose(m, 0.25)
    assert frame_diagnostics(r, r, P)[1:] == (0.0, 0.0)
