"""Shared plumbing for the GPU parity tests: upload a fmha_synth.Problem, run
the HIP path through the C ABI binding, run the oracle on the same bits, and
compare element by element.

Tolerances (max abs error): O <= 2e-2 for f32/f16/bf16 and <= 0.13 for fp8;
LSE <= 1e-3 for every dtype, with equal -inf patterns required.  Rows of
sequences with no keys must keep the sentinel bit pattern.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from fmha_synth import raw_bits

TOL_O = {"f32": 2e-2, "f16": 2e-2, "bf16": 2e-2, "fp8_e4m3": 0.13}
TOL_LSE = 1e-3
SENTINEL_O = 3.140625        # exactly representable in bf16/f16/f32
SENTINEL_LSE = -12345.0


def out_dtype(prob):
    return torch.bfloat16 if prob.dtype == "fp8_e4m3" else prob.q.dtype


def upload(prob, device="cuda"):
    """Device tensors in the API layout (fixed-length sides as [B, S, H, D])."""
    B = prob.batch
    d = {}
    if prob.varlen_q:
        d["q"] = prob.q.to(device)
        d["cu_seqlens_q"] = torch.from_numpy(prob.cu_q).to(device)
        d["max_seqlen_q"] = prob.max_seqlen_q
    else:
        d["q"] = prob.q.reshape(B, -1, prob.hq, prob.dqk).to(device)
    if prob.varlen_k:
        d["k"] = prob.k.to(device)
        d["v"] = prob.v.to(device)
        d["cu_seqlens_k"] = torch.from_numpy(prob.cu_k).to(device)
        d["max_seqlen_k"] = prob.max_seqlen_k
    else:
        d["k"] = prob.k.reshape(B, -1, prob.hkv, prob.dqk).to(device)
        d["v"] = prob.v.reshape(B, -1, prob.hkv, prob.dv).to(device)
    if prob.dtype == "fp8_e4m3":
        for n, val in (("q_descale", prob.q_descale), ("k_descale", prob.k_descale),
                       ("v_descale", prob.v_descale)):
            d[n] = torch.tensor([val], dtype=torch.float32, device=device)
    return d


def alloc_outputs(prob, dev):
    """Sentinel-filled out / lse in the API layout."""
    od = out_dtype(prob)
    tq = sum(prob.lens_q)
    if prob.varlen_q:
        out = torch.full((tq, prob.hq, prob.dv), SENTINEL_O, dtype=od, device="cuda")
        lse = torch.full((prob.hq, tq), SENTINEL_LSE, dtype=torch.float32, device="cuda")
    else:
        B, S = prob.batch, prob.lens_q[0]
        out = torch.full((B, S, prob.hq, prob.dv), SENTINEL_O, dtype=od, device="cuda")
        lse = torch.full((B, prob.hq, S), SENTINEL_LSE, dtype=torch.float32, device="cuda")
    return out, lse


def to_packed(prob, out, lse):
    """GPU outputs -> fp64 numpy in the oracle layout out [Tq,Hq,Dv], lse [Hq,Tq]."""
    tq = sum(prob.lens_q)
    o = out.detach().to(torch.float64).cpu().reshape(tq, prob.hq, prob.dv).numpy()
    if prob.varlen_q:
        l = lse.detach().cpu().to(torch.float64).numpy()
    else:
        l = lse.detach().cpu().to(torch.float64).permute(1, 0, 2).reshape(prob.hq, tq).numpy()
    return o, l


def run_gpu(fmha, prob, *, num_kv_splits=0, softmax_scale=0.0, dev=None, out=None,
            lse=None, **extra):
    dev = dev or upload(prob)
    if out is None:
        out, lse = alloc_outputs(prob, dev)
    fmha.fwd(dev["q"], dev["k"], dev["v"], cu_seqlens_q=dev.get("cu_seqlens_q"),
             cu_seqlens_k=dev.get("cu_seqlens_k"), max_seqlen_q=dev.get("max_seqlen_q"),
             max_seqlen_k=dev.get("max_seqlen_k"), softmax_scale=softmax_scale,
             causal=prob.causal, window=prob.window, num_kv_splits=num_kv_splits,
             q_descale=dev.get("q_descale"), k_descale=dev.get("k_descale"),
             v_descale=dev.get("v_descale"), out=out, lse=lse, **extra)
    torch.cuda.synchronize()
    return out, lse


def run_oracle(oracle, prob, scale=None):
    scale = 1.0 / math.sqrt(prob.dqk) if scale is None else scale
    return oracle.attention(
        raw_bits(prob.q), raw_bits(prob.k), raw_bits(prob.v), prob.dtype,
        cu_q=prob.cu_q, cu_k=prob.cu_k, batch=prob.batch, scale=scale,
        q_descale=prob.q_descale, k_descale=prob.k_descale, v_descale=prob.v_descale,
        causal=prob.causal, window=prob.window)


def rows_with_keys(prob):
    m = []
    for sq, sk in zip(prob.lens_q, prob.lens_k):
        m += [sk > 0] * sq
    return np.array(m, dtype=bool)


def compare(prob, gpu_o, gpu_l, ref_o, ref_l, what=""):
    """Element-wise parity plus sentinel checks; returns (err_o, err_lse)."""
    written = rows_with_keys(prob)
    tol_o = TOL_O[prob.dtype]
    # untouched rows keep the sentinel exactly
    if (~written).any():
        assert (gpu_o[~written] == SENTINEL_O).all(), f"{what}: a no-key row of O was written"
        assert (gpu_l[:, ~written] == SENTINEL_LSE).all(), f"{what}: a no-key LSE was written"
    go, ro = gpu_o[written], ref_o[written]
    gl, rl = gpu_l[:, written], ref_l[:, written]
    assert not np.isnan(go).any(), f"{what}: NaN in O"
    assert not np.isnan(gl).any(), f"{what}: NaN in LSE"
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), f"{what}: -inf LSE pattern differs"
    fin = ~np.isneginf(rl)
    err_o = float(np.max(np.abs(go - ro))) if go.size else 0.0
    err_l = float(np.max(np.abs(gl[fin] - rl[fin]))) if fin.any() else 0.0
    assert err_o <= tol_o, f"{what}: max |O - oracle| = {err_o:.3e} > {tol_o}"
    assert err_l <= TOL_LSE, f"{what}: max |LSE - oracle| = {err_l:.3e} > {TOL_LSE}"
    return err_o, err_l
