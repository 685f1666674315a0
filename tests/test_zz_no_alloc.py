"""fmha_fwd_no_alloc (split partials in the library's per-GPU scratch) against
fmha_fwd (caller's workspace) and the oracle, through the C ABI: two calls in
a row, the second smaller, plus a plan too large for the scratch."""
from __future__ import annotations

import ctypes
import sys

import pytest
import torch

import fmha_synth as fs
from fmha_synth import make_problem
from gpu_helpers import SENTINEL_LSE, SENTINEL_O, alloc_outputs, compare, run_oracle, to_packed, upload

pytestmark = pytest.mark.gpu


def announce(msg):
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module")
def fmha():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import split_kv_flash_fmha_amd as m
    return m


def _args(fmha, prob, dev, out, lse, splits):
    return fmha.make_args(dev["q"], dev["k"], dev["v"], out=out, lse=lse,
                          cu_seqlens_q=dev.get("cu_seqlens_q"),
                          cu_seqlens_k=dev.get("cu_seqlens_k"),
                          max_seqlen_q=dev.get("max_seqlen_q"),
                          max_seqlen_k=dev.get("max_seqlen_k"), causal=prob.causal,
                          window=prob.window, num_kv_splits=splits,
                          q_descale=dev.get("q_descale"), k_descale=dev.get("k_descale"),
                          v_descale=dev.get("v_descale"), num_cus=fmha.device_num_cus())


def _no_alloc_matches(fmha, oracle, prob, splits, combine_mode_b=0):
    dev = upload(prob)
    stream = torch.cuda.current_stream().cuda_stream
    # fmha_fwd with the caller's workspace
    out_a, lse_a = alloc_outputs(prob, dev)
    args = _args(fmha, prob, dev, out_a, lse_a, splits)
    nbytes = fmha.workspace_size(args)
    assert 0 < nbytes <= fmha.NO_ALLOC_SCRATCH_BYTES, nbytes
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), nbytes
    assert fmha.lib.fmha_fwd(ctypes.byref(args), ctypes.c_void_p(stream)) == 0
    # fmha_fwd_no_alloc on the same inputs (its workspace argument is ignored)
    out_b, lse_b = alloc_outputs(prob, dev)
    args_b = _args(fmha, prob, dev, out_b, lse_b, splits)
    args_b.workspace, args_b.workspace_bytes = None, 0
    args_b.combine_mode = combine_mode_b
    assert fmha.lib.fmha_fwd_no_alloc(ctypes.byref(args_b), ctypes.c_void_p(stream)) == 0
    torch.cuda.synchronize()
    # same kernels, same plan: identical bits; and the oracle's tolerance
    assert torch.equal(out_a.view(torch.int16 if out_a.element_size() == 2 else torch.int32),
                       out_b.view(torch.int16 if out_b.element_size() == 2 else torch.int32))
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32))
    go, gl = to_packed(prob, out_b, lse_b)
    return compare(prob, go, gl, *run_oracle(oracle, prob), what=f"no_alloc {prob.name}")


def test_no_alloc_two_calls_second_smaller(fmha, oracle):
    # GQA decode with automatic splits (a workspace of several MB), then a
    # smaller problem whose partials overwrite only part of what the first
    # left in the scratch
    lens_k = [30000, 1200, 17777, 4096, 25000, 9000, 1, 31000]
    big = make_problem("no_alloc_big", dtype="bf16", lens_q=[1] * 8, lens_k=lens_k, hq=32,
                       hkv=8, dqk=128, dv=128, seed=41, varlen_q=False, varlen_k=True)
    announce("no_alloc: GQA decode, 8 sequences, auto splits")
    _no_alloc_matches(fmha, oracle, big, 0)
    small = make_problem("no_alloc_small", dtype="bf16", lens_q=[1, 3, 2], lens_k=[700, 129, 0],
                         hq=8, hkv=2, dqk=128, dv=128, seed=42, varlen_q=True, varlen_k=True,
                         causal=True)
    announce("no_alloc: small varlen decode, 5 splits")
    _no_alloc_matches(fmha, oracle, small, 5)


def test_no_alloc_fp8_short_prefix(fmha, oracle):
    prob = fs.fp8_prefix(11008)
    announce("no_alloc: fp8 short prefix, auto splits")
    _no_alloc_matches(fmha, oracle, prob, 0)


def test_no_alloc_ignores_the_in_launch_combine(fmha, oracle):
    # the fp8 prefix is a plan the in-launch combine serves (combine_mode 1 with
    # a zeroed workspace); on the scratch, which the GQA decode call before it
    # leaves full of partials, no_alloc must take the two-launch path: the bits
    # of fmha_fwd's default call, not NaN rows from a dirty counter block
    lens_k = [30000, 1200, 17777, 4096, 25000, 9000, 1, 31000]
    big = make_problem("no_alloc_dirty", dtype="bf16", lens_q=[1] * 8, lens_k=lens_k, hq=32,
                       hkv=8, dqk=128, dv=128, seed=44, varlen_q=False, varlen_k=True)
    announce("no_alloc: GQA decode leaves the scratch dirty")
    _no_alloc_matches(fmha, oracle, big, 0)
    prob = fs.fp8_prefix(11008)
    announce("no_alloc: fp8 short prefix asking for the in-launch combine")
    _no_alloc_matches(fmha, oracle, prob, 0, combine_mode_b=1)


def test_no_alloc_refuses_plans_beyond_the_scratch(fmha):
    # 256 splits of 64 query rows x 8 heads x Dv 128 need 64 MiB of partials
    prob = make_problem("no_alloc_too_big", dtype="bf16", lens_q=[64], lens_k=[65536], hq=8,
                        hkv=8, dqk=128, dv=128, seed=43)
    dev = upload(prob)
    out, lse = alloc_outputs(prob, dev)
    args = _args(fmha, prob, dev, out, lse, 256)
    assert fmha.workspace_size(args) > fmha.NO_ALLOC_SCRATCH_BYTES
    stream = torch.cuda.current_stream().cuda_stream
    assert fmha.lib.fmha_fwd_no_alloc(ctypes.byref(args), ctypes.c_void_p(stream)) == 3
    with pytest.raises(ValueError):
        fmha.fwd_no_alloc(dev["q"], dev["k"], dev["v"], out=out, lse=lse, num_kv_splits=256)
    torch.cuda.synchronize()
    assert (out.float() == SENTINEL_O).all() and (lse == SENTINEL_LSE).all()
