"""GPU parity of the prefill kernels' reference move (the rescale of a
non-zero O and l by alpha in (0, 1)) against the CPU oracle.

Inputs: keys planted at chosen score heights (tests/rescale_plant.py) so that,
by a host model of the kernels' decisions, every wave group that has enough
key blocks moves its reference at least once per planted jump.  Both the
f16/bf16 prefill kernel (head dims 64, 128, 256; no mask, bottom-right causal,
window (128, 0)) and the fp8 one (Dqk 128 and 192, 96- and 128-row tiles) are
compared element by element with the oracle at the usual tolerances, with one
split and with several.
"""
from __future__ import annotations

import pytest
import torch

import rescale_plant as rp
from gpu_helpers import upload
from test_gpu_parity import announce, check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fmha():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import split_kv_flash_fmha_amd as m
    return m


def _plan(fmha, prob, splits):
    dev = upload(prob)
    args = fmha.make_args(dev["q"], dev["k"], dev["v"], cu_seqlens_q=dev.get("cu_seqlens_q"),
                          cu_seqlens_k=dev.get("cu_seqlens_k"),
                          max_seqlen_q=dev.get("max_seqlen_q"),
                          max_seqlen_k=dev.get("max_seqlen_k"), causal=prob.causal,
                          window=prob.window, num_kv_splits=splits,
                          q_descale=dev.get("q_descale"), k_descale=dev.get("k_descale"),
                          v_descale=dev.get("v_descale"), num_cus=fmha.device_num_cus())
    ws = torch.empty(max(fmha.workspace_size(args), 256), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    return fmha.plan(args)


def _run(fmha, oracle, name, *, dtype, lens_q, lens_k, hq, hkv, dqk, dv, seed, mask,
         expect_rows):
    kw = dict(causal=(mask == "causal"), window=(128, 0) if mask == "window" else (-1, -1))
    shape = dict(dtype=dtype, lens_q=lens_q, lens_k=lens_k, hq=hq, hkv=hkv, dqk=dqk, dv=dv,
                 seed=seed, **kw)
    # the tiling of the launch (row tile, key block) from the library's plan
    probe, _ = rp.planted_problem(name, rows_per_tile=128, key_block=32, **shape)
    pl = _plan(fmha, probe, 1)
    assert pl.kernel_id % 1000 >= 200, f"not a prefill kernel: {pl.kernel_id}"
    assert pl.rows_per_tile == expect_rows, pl.rows_per_tile
    rpt, bn = pl.rows_per_tile, pl.key_block
    prob, planted = rp.planted_problem(name, rows_per_tile=rpt, key_block=bn, **shape)
    # by the model, every wave with a planted jump moves its reference, and
    # some move keeps a large share of old mass (alpha well inside (0, 1))
    sim = rp.simulate(prob, rows_per_tile=rpt, key_block=bn)
    eligible = {k: v for k, v in planted.items() if v > 0}
    assert eligible, "no wave has room for a planted jump"
    for (b, h, w0), jumps in eligible.items():
        assert sim[(b, h, 0, w0)][0] >= jumps, (b, h, w0, sim[(b, h, 0, w0)], jumps)
    assert max(v[1] for v in sim.values()) >= 0.25
    moves = sum(v[0] for v in sim.values())
    pl3 = _plan(fmha, prob, 3)
    sim3 = rp.simulate(prob, rows_per_tile=rpt, key_block=bn, split_chunk=pl3.split_chunk)
    moves3 = sum(v[0] for v in sim3.values())
    assert moves3 > 0
    announce(f"{name}: {len(eligible)} waves with planted jumps, {moves} reference moves "
             f"(1 split), {moves3} (3 splits of {pl3.split_chunk} keys)")
    check(fmha, oracle, prob, splits=(1, 3), label=f"planted {mask}")


@pytest.mark.parametrize("mask", ["none", "causal", "window"])
@pytest.mark.parametrize("dtype,d", [("f16", 64), ("f16", 128), ("f16", 256),
                                     ("bf16", 64), ("bf16", 128), ("bf16", 256)])
def test_prefill_reference_move(fmha, oracle, dtype, d, mask):
    # GQA 8:2 (4 query heads per kv head packed into the rows), lengths over
    # several 128-row tiles with ragged tails
    lens = [300, 129, 257, 70]
    _run(fmha, oracle, f"move_{dtype}_{d}_{mask}", dtype=dtype, lens_q=lens, lens_k=lens, hq=8,
         hkv=2, dqk=d, dv=d, seed=21, mask=mask, expect_rows=128)


@pytest.mark.parametrize("mask", ["none", "causal", "window"])
@pytest.mark.parametrize("dqk", [128, 192])
@pytest.mark.parametrize("hq,hkv,lens_q,rows", [(12, 4, [70, 33, 96], 128), (4, 4, [70, 45, 17], 96)])
def test_prefill8_reference_move(fmha, oracle, dqk, mask, hq, hkv, lens_q, rows):
    _run(fmha, oracle, f"move_fp8_{dqk}_{mask}_{rows}", dtype="fp8_e4m3", lens_q=lens_q,
         lens_k=[1000, 300, 517], hq=hq, hkv=hkv, dqk=dqk, dv=128, seed=22, mask=mask,
         expect_rows=rows)
