"""The pins must catch plausible slips: plant each slip in the oracle (CPU only,
via monkeypatch) and check that the pin battery rejects it."""

import glob
import json
import os

import numpy as np
import pytest

from oracle import squad_oracle as so
from tests import bruteforce as bf
from tests.test_oracle_pins import GOLDEN, rand_qkv, sdpa64


def battery():
    """Runs the core pins; raises AssertionError if any fails."""
    for path in sorted(glob.glob(os.path.join(GOLDEN, "closed_form_*.json"))):
        fx = json.load(open(path))
        q, k, v = (np.array(fx[c], np.float64)[None, :, None, :] for c in "qkv")
        out = so.squad_forward(q, k, v, fx["grid"], fx["tile"], fx["scale"])
        np.testing.assert_allclose(out[0, :, 0, :], np.array(fx["out"]), atol=1e-12)
    for grid, tile in [((2, 4, 6), (2, 2, 3)), ((4, 8, 8), (1, 4, 4))]:
        q, k, v = rand_qkv(grid, 1, 2, 8, 0)
        ref, _ = bf.squad_bruteforce(q, k, v, grid, tile, 0.37)
        np.testing.assert_allclose(so.squad_forward(q, k, v, grid, tile, 0.37), ref, atol=1e-12)
    q, k, v = rand_qkv((2, 3, 5), 1, 2, 16, 1)
    np.testing.assert_allclose(so.squad_forward(q, k, v, (2, 3, 5), (2, 3, 5)), sdpa64(q, k, v, 0.25), atol=1e-12)


def _swap_axes_softmax(q, k, v, scale):
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    logits = float(scale) * np.matmul(q, np.swapaxes(k, -1, -2))
    w = np.exp(logits - logits.max(axis=-2, keepdims=True))
    return np.matmul(w / w.sum(axis=-2, keepdims=True), v)


MUTANTS = {
    "global pass grouped by window": lambda mp: mp.setattr(
        so, "global_pass", lambda q, k, v, g, t, s=None: so.local_pass(q, k, v, g, t, s)),
    "global pass fed v instead of the local output": lambda mp: mp.setattr(
        so, "squad_forward", lambda q, k, v, g, t, s=None: so.global_pass(q, k, v, g, t, s)),
    "q and k swapped in the global pass": lambda mp: mp.setattr(
        so, "global_pass", (lambda f: (lambda q, k, v, g, t, s=None: f(k, q, v, g, t, s)))(so.global_pass)),
    "local pass skipped": lambda mp: mp.setattr(
        so, "local_pass", lambda q, k, v, g, t, s=None: np.asarray(v, np.float64)),
    "softmax over the query axis": lambda mp: mp.setattr(so, "softmax_attention", _swap_axes_softmax),
    "scale dropped": lambda mp: mp.setattr(
        so, "softmax_attention", (lambda f: (lambda q, k, v, s: f(q, k, v, 1.0)))(so.softmax_attention)),
    "windows and offsets swapped": lambda mp: mp.setattr(
        so, "window_index", (lambda f: (lambda g, t: f(g, t).T.copy()))(so.window_index)),
    "token order flattened (w, h, t)": lambda mp: mp.setattr(
        so, "window_index", (lambda f: (lambda g, t: (lambda idx, G: (idx % G[2]) * G[0] * G[1]
                                                      + ((idx // G[2]) % G[1]) * G[0] + idx // (G[1] * G[2]))(
            f(g, t), g)))(so.window_index)),
}


def test_battery_passes_on_the_real_oracle():
    battery()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_battery_rejects_mutant(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    with pytest.raises(AssertionError):
        battery()
