"""CPU checks of the planted-key inputs used by the reference-move parity
tests: on unplanted N(0, 1) inputs without a window the prefill kernels'
reference never moves (so those inputs cannot test the rescale; under a
window a row whose keys start after the tile's first block moves the other
rows of its wave when it sets its own reference), while the planted ones move
it in every wave that has room for a planted jump."""
from __future__ import annotations

import pytest

import fmha_synth as fs
import rescale_plant as rp


@pytest.mark.parametrize("dtype,d,bn", [("f16", 128, 32), ("bf16", 64, 64), ("fp8_e4m3", 192, 64)])
@pytest.mark.parametrize("mask", ["none", "causal", "window"])
def test_planted_keys_move_the_reference(dtype, d, bn, mask):
    kw = dict(causal=(mask == "causal"), window=(128, 0) if mask == "window" else (-1, -1))
    lens_q, lens_k = [300, 129, 70], [300, 129, 70]
    dv = 128 if dtype == "fp8_e4m3" else d
    prob, planted = rp.planted_problem("m", dtype=dtype, lens_q=lens_q, lens_k=lens_k, hq=8,
                                       hkv=2, dqk=d, dv=dv, seed=31, rows_per_tile=128,
                                       key_block=bn, **kw)
    sim = rp.simulate(prob, rows_per_tile=128, key_block=bn)
    eligible = {k: v for k, v in planted.items() if v > 0}
    assert len(eligible) >= len(sim) // 2
    for (b, h, w0), jumps in eligible.items():
        assert sim[(b, h, 0, w0)][0] >= jumps
    assert max(v[1] for v in sim.values()) >= 0.25
    base = fs.make_problem("m", dtype=dtype, lens_q=lens_q, lens_k=lens_k, hq=8, hkv=2, dqk=d,
                           dv=dv, seed=31, varlen_q=True, varlen_k=True, **kw)
    if mask != "window":
        assert sum(v[0] for v in rp.simulate(base, rows_per_tile=128, key_block=bn).values()) == 0


def test_planted_heights():
    # the keys planted for a row with a long key range sit, relative to the
    # row's first-block max, at limit - MID_BELOW (twice), limit + JUMP_ABOVE,
    # then the same three again above that jump
    import math

    import numpy as np
    import torch
    lens = [256]

    prob, planted = rp.planted_problem("h", dtype="f16", lens_q=lens, lens_k=lens, hq=1, hkv=1,
                                       dqk=128, dv=128, seed=5, rows_per_tile=128, key_block=32)
    q = prob.q.to(torch.float64).numpy()[:, 0]
    k = prob.k.to(torch.float64).numpy()[:, 0]
    s = (q @ k.T) / math.sqrt(128) / math.log(2.0)
    # last row of the first wave group (row 31) under no mask: first block = keys 0..31
    m0 = s[31, :32].max()
    above = s[31, 32:] - m0
    assert planted[(0, 0, 0)] == 2
    top = np.sort(above)[-6:]
    L, mid, jump = rp.LIMIT_LOG2["f16"], -rp.MID_BELOW, rp.JUMP_ABOVE
    want = np.sort([L + mid, L + mid, L + jump, 2 * L + jump + mid, 2 * L + jump + mid,
                    2 * (L + jump)])
    assert np.abs(top - want).max() < 0.2, (top, want)
    # every other key of the row stays within the ordinary N(0, 1) range
    assert np.sort(above)[-7] < 4
