"""The battery of checks that pins the CPU oracle to something other than itself.

Each ``check_*`` takes an ``Oracle`` handle and raises AssertionError on a
mismatch.  tests/test_oracle_pins.py runs them against the real oracle (all
must pass) and against planted-mistake builds of it (each build must fail at
least one), so that a dropped term, a wrong sign or index or a transposed
operand anywhere in the oracle cannot go unnoticed.

What the checks compare against:
  * brute force in 50-digit arithmetic with torch's own dtype decoding
    (tests/bruteforce.py);
  * torch's fp64 scaled_dot_product_attention with an explicit boolean mask
    and enable_gqa (a library routine), plus torch.logsumexp;
  * closed forms: one key, two keys, all-equal scores, constant V, V = I;
  * invariants: split + combine == unsplit, GQA == MHA on repeated K/V,
    joint key permutation, packed == separate calls, special mask cases;
  * torch's own fp16 / bf16 / fp8-e4m3fn -> fp64 casts for the decoders.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import bruteforce
from fmha_synth import make_problem, raw_bits

TOL_BRUTE = 1e-12


def run(o, prob, *, scale=None, causal=None, window=None, fill=np.nan):
    """Oracle forward on a fmha_synth.Problem (packed layout)."""
    if scale is None:
        scale = 1.0 / math.sqrt(prob.dqk)
    return o.attention(
        raw_bits(prob.q), raw_bits(prob.k), raw_bits(prob.v), prob.dtype,
        cu_q=prob.cu_q, cu_k=prob.cu_k, batch=prob.batch, scale=scale,
        q_descale=prob.q_descale, k_descale=prob.k_descale,
        v_descale=prob.v_descale,
        causal=prob.causal if causal is None else causal,
        window=prob.window if window is None else window, fill=fill)


def rows_written(prob):
    """Boolean [Tq] mask of query tokens whose sequence has at least one key."""
    out = []
    for sq, sk in zip(prob.lens_q, prob.lens_k):
        out += [sk > 0] * sq
    return np.array(out, dtype=bool)


def assert_close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    inf_a, inf_b = np.isneginf(a), np.isneginf(b)
    assert np.array_equal(inf_a, inf_b), f"{what}: -inf pattern differs"
    fin = ~inf_a
    assert not np.isnan(a[fin]).any(), f"{what}: NaN in first operand"
    assert not np.isnan(b[fin]).any(), f"{what}: NaN in second operand"
    if fin.any():
        err = float(np.max(np.abs(a[fin] - b[fin])))
        assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ---- tiny problems for the brute force -------------------------------------

TINY_CASES = [
    # name, dtype, lens_q, lens_k, hq, hkv, d, dv, causal, window, varlen
    ("mha_nomask_sk0", "f32", [3, 1, 4], [5, 0, 7], 4, 4, 8, 6, False, (-1, -1), True),
    ("mha_causal_sk0", "f32", [3, 1, 4], [5, 0, 7], 4, 4, 8, 6, True, (-1, -1), True),
    ("gqa42_window20", "bf16", [4, 2], [4, 6], 4, 2, 5, 3, False, (2, 0), True),
    ("gqa41_window11", "f16", [6], [9], 4, 1, 8, 4, False, (1, 1), False),
    ("fp8_causal_sq_gt_sk", "fp8_e4m3", [7, 3], [2, 9], 2, 1, 8, 5, True, (-1, -1), True),
    ("fixed_len_b2", "bf16", [3, 3], [5, 5], 2, 2, 4, 4, True, (3, -1), False),
]


def tiny_problem(case, seed):
    name, dtype, lq, lk, hq, hkv, d, dv, causal, window, varlen = case
    return make_problem(name, dtype=dtype, lens_q=lq, lens_k=lk, hq=hq, hkv=hkv,
                        dqk=d, dv=dv, seed=seed, varlen_q=varlen, varlen_k=varlen,
                        causal=causal, window=window)


_BRUTE_CACHE: dict = {}


def brute(prob, scale):
    key = (prob.name, scale, prob.causal, prob.window)
    if key not in _BRUTE_CACHE:
        _BRUTE_CACHE[key] = bruteforce.attention(
            prob.q, prob.k, prob.v, prob.lens_q, prob.lens_k, scale=scale,
            qs=prob.q_descale, ks=prob.k_descale, vs=prob.v_descale,
            causal=prob.causal, window=prob.window)
    return _BRUTE_CACHE[key]


def check_bruteforce(o):
    for n, case in enumerate(TINY_CASES):
        prob = tiny_problem(case, seed=100 + n)
        scale = 1.0 / math.sqrt(prob.dqk)
        out, lse = run(o, prob, scale=scale)
        ref = brute(prob, scale)
        written = rows_written(prob)
        for t in range(out.shape[0]):
            for h in range(prob.hq):
                if not written[t]:
                    assert np.isnan(out[t, h]).all() and np.isnan(lse[h, t]), \
                        f"{prob.name}: row {t} of a sequence with no keys was written"
                    continue
                o_ref, l_ref = ref[(t, h)]
                o_ref = np.array([float(x) for x in o_ref])
                assert_close(out[t, h], o_ref, TOL_BRUTE, f"{prob.name} O[{t},{h}]")
                assert_close([lse[h, t]], [float(l_ref)], TOL_BRUTE,
                             f"{prob.name} LSE[{h},{t}]")


# ---- library routine: torch fp64 SDPA with an explicit mask ---------------

def explicit_mask(sq, sk, causal, window):
    i = torch.arange(sq).unsqueeze(1)
    j = torch.arange(sk).unsqueeze(0)
    d0 = i + sk - sq
    m = torch.ones(sq, sk, dtype=torch.bool)
    wl, wr = window
    if causal:
        m &= j <= d0
    if wl >= 0:
        m &= j >= d0 - wl
    if wr >= 0:
        m &= j <= d0 + wr
    return m


def check_sdpa(o):
    cases = [
        ("sdpa_gqa", "bf16", [33, 17, 40], [50, 17, 9], 8, 2, 32, 16, True, (-1, -1)),
        ("sdpa_win", "f16", [20, 64], [70, 64], 4, 4, 16, 24, False, (7, 3)),
        ("sdpa_mqa", "f32", [12], [31], 6, 1, 12, 8, False, (-1, -1)),
    ]
    for n, (name, dt, lq, lk, hq, hkv, d, dv, causal, window) in enumerate(cases):
        prob = make_problem(name, dtype=dt, lens_q=lq, lens_k=lk, hq=hq, hkv=hkv,
                            dqk=d, dv=dv, seed=200 + n, varlen_q=True,
                            varlen_k=True, causal=causal, window=window)
        scale = 0.37
        out, lse = run(o, prob, scale=scale)
        q = prob.q.to(torch.float64)
        k = prob.k.to(torch.float64)
        v = prob.v.to(torch.float64)
        q0 = k0 = 0
        for sq, sk in zip(lq, lk):
            qs = q[q0:q0 + sq].permute(1, 0, 2).unsqueeze(0)
            ks = k[k0:k0 + sk].permute(1, 0, 2).unsqueeze(0)
            vs = v[k0:k0 + sk].permute(1, 0, 2).unsqueeze(0)
            mask = explicit_mask(sq, sk, causal, window)
            full = mask.any(dim=1)
            ref = torch.nn.functional.scaled_dot_product_attention(
                qs, ks, vs, attn_mask=mask, scale=scale, enable_gqa=True)[0]
            ref = ref.permute(1, 0, 2).numpy()
            g = hq // hkv
            kr = ks.repeat_interleave(g, dim=1)
            sc = (qs @ kr.transpose(-1, -2)) * scale
            sc = sc.masked_fill(~mask, -math.inf)
            ref_lse = torch.logsumexp(sc, dim=-1)[0].numpy()
            got = out[q0:q0 + sq]
            got_lse = lse[:, q0:q0 + sq]
            fm = full.numpy()
            assert_close(got[fm], ref[fm], 1e-12, f"{name} O vs SDPA")
            assert_close(got_lse[:, fm], ref_lse[:, fm], 1e-12, f"{name} LSE vs logsumexp")
            if (~fm).any():
                assert (got[~fm] == 0).all(), f"{name}: fully masked rows must be 0"
                assert np.isneginf(got_lse[:, ~fm]).all(), f"{name}: masked LSE must be -inf"
            q0 += sq
            k0 += sk


# ---- closed forms ----------------------------------------------------------

def _f32_problem(q, k, v, lens_q, lens_k, name="closed"):
    """Problem from explicit fp32 arrays [T,H,D]."""
    from fmha_synth import Problem
    q = torch.tensor(q, dtype=torch.float32)
    k = torch.tensor(k, dtype=torch.float32)
    v = torch.tensor(v, dtype=torch.float32)
    return Problem(name, "f32", q, k, v, 1.0, 1.0, 1.0, list(lens_q), list(lens_k),
                   True, True, q.shape[1], k.shape[1], q.shape[2], v.shape[2])


def check_closed_forms(o):
    rng = np.random.default_rng(7)
    # One key: O = v, LSE = scale * q.k
    q = rng.standard_normal((1, 1, 8)).astype(np.float32)
    k = rng.standard_normal((1, 1, 8)).astype(np.float32)
    v = rng.standard_normal((1, 1, 5)).astype(np.float32)
    p = _f32_problem(q, k, v, [1], [1])
    out, lse = run(o, p, scale=0.3)
    dot = float(np.dot(q[0, 0].astype(np.float64), k[0, 0].astype(np.float64)))
    assert_close(out[0, 0], v[0, 0], 1e-15, "one key O")
    assert_close([lse[0, 0]], [0.3 * dot], 1e-15, "one key LSE")
    # Two keys: O = sigma(a-b) v1 + sigma(b-a) v2, LSE = ln(e^a + e^b)
    k2 = rng.standard_normal((2, 1, 8)).astype(np.float32)
    v2 = rng.standard_normal((2, 1, 5)).astype(np.float32)
    p = _f32_problem(q, k2, v2, [1], [2])
    out, lse = run(o, p, scale=0.7)
    a = 0.7 * float(np.dot(q[0, 0].astype(np.float64), k2[0, 0].astype(np.float64)))
    b = 0.7 * float(np.dot(q[0, 0].astype(np.float64), k2[1, 0].astype(np.float64)))
    sa = 1.0 / (1.0 + math.exp(b - a))
    exp_o = sa * v2[0, 0].astype(np.float64) + (1 - sa) * v2[1, 0].astype(np.float64)
    assert_close(out[0, 0], exp_o, 1e-14, "two keys O")
    assert_close([lse[0, 0]], [max(a, b) + math.log1p(math.exp(-abs(a - b)))], 1e-14,
                 "two keys LSE")
    # All-equal scores (Q = 0): O = mean of V over allowed keys, LSE = ln|A|
    sq, sk = 5, 11
    qz = np.zeros((sq, 2, 4), np.float32)
    kk = rng.standard_normal((sk, 2, 4)).astype(np.float32)
    vv = rng.standard_normal((sk, 2, 3)).astype(np.float32)
    for causal, window in ((False, (-1, -1)), (True, (-1, -1)), (False, (2, 1))):
        p = _f32_problem(qz, kk, vv, [sq], [sk])
        out, lse = run(o, p, scale=1.0, causal=causal, window=window)
        mask = explicit_mask(sq, sk, causal, window).numpy()
        for i in range(sq):
            for h in range(2):
                sel = mask[i]
                if not sel.any():
                    continue
                mean = vv[sel, h].astype(np.float64).mean(axis=0)
                assert_close(out[i, h], mean, 1e-14, f"equal scores O (causal={causal})")
                assert_close([lse[h, i]], [math.log(sel.sum())], 1e-14,
                             f"equal scores LSE (causal={causal})")
    # V constant: O = c
    vc = np.full((sk, 2, 3), 1.75, np.float32)
    qq = rng.standard_normal((sq, 2, 4)).astype(np.float32)
    p = _f32_problem(qq, kk, vc, [sq], [sk])
    out, _ = run(o, p, scale=0.5, causal=True)
    assert_close(out, np.full_like(out, 1.75), 1e-14, "constant V")
    # V = I (sk <= Dv): O rows are the probability rows, non-negative, sum 1,
    # and causal sq == sk gives row i exactly i + 1 non-zero probabilities.
    n = 6
    vi = np.zeros((n, 1, n), np.float32)
    for j in range(n):
        vi[j, 0, j] = 1.0
    qq = rng.standard_normal((n, 1, 4)).astype(np.float32)
    kk = rng.standard_normal((n, 1, 4)).astype(np.float32)
    p = _f32_problem(qq, kk, vi, [n], [n])
    out, lse = run(o, p, scale=0.9, causal=True)
    assert (out >= 0).all(), "probabilities must be non-negative"
    assert_close(out.sum(axis=2), np.ones((n, 1)), 1e-14, "softmax rows sum to 1")
    for i in range(n):
        assert (out[i, 0, :i + 1] > 0).all() and (out[i, 0, i + 1:] == 0).all(), \
            f"causal row {i} must see exactly {i + 1} keys"
        # the probability row is exp(s_ij - LSE_i)
        s = 0.9 * (kk[:i + 1, 0].astype(np.float64) @ qq[i, 0].astype(np.float64))
        assert_close(out[i, 0, :i + 1], np.exp(s - lse[0, i]), 1e-14, "P = exp(s - LSE)")


# ---- split + combine -------------------------------------------------------

def check_split_combine(o):
    cases = [
        ("split_fixed", "bf16", [1], [257], 4, 4, 16, 16, False, (-1, -1)),
        ("split_varlen_gqa", "f16", [2, 1, 3], [100, 0, 37], 4, 2, 8, 8, False, (-1, -1)),
        ("split_causal", "f32", [5, 9], [40, 9], 2, 2, 8, 8, True, (-1, -1)),
        ("split_window", "bf16", [6], [90], 2, 1, 8, 4, False, (10, 0)),
    ]
    for n, (name, dt, lq, lk, hq, hkv, d, dv, causal, window) in enumerate(cases):
        prob = make_problem(name, dtype=dt, lens_q=lq, lens_k=lk, hq=hq, hkv=hkv,
                            dqk=d, dv=dv, seed=300 + n, varlen_q=True,
                            varlen_k=True, causal=causal, window=window)
        scale = 1.0 / math.sqrt(d)
        ref_o, ref_l = run(o, prob, scale=scale)
        written = rows_written(prob)
        args = dict(cu_q=prob.cu_q, cu_k=prob.cu_k, scale=scale, causal=causal,
                    window=window)
        for chunk in (1, 7, 16, 33, max(lk)):
            nsplit = -(-max(lk) // chunk)
            co, cl = o.split_then_combine(
                raw_bits(prob.q), raw_bits(prob.k), raw_bits(prob.v), dt,
                num_splits=nsplit, chunk=chunk, **args)
            assert_close(co[written], ref_o[written], 1e-12, f"{name} chunk={chunk} O")
            assert_close(cl[:, written], ref_l[:, written], 1e-12, f"{name} chunk={chunk} LSE")
            assert np.isnan(co[~written]).all(), f"{name}: combine wrote a no-key row"


def check_combine_edge(o):
    # All partials -inf -> O = 0, LSE = -inf, never NaN.
    o_part = np.random.default_rng(0).standard_normal((3, 2, 1, 4))
    lse_part = np.full((3, 1, 2), -np.inf)
    lse_part[1, 0, 1] = 0.25  # row 1 has one real split
    out, lse = o.combine(o_part, lse_part, chunk=4, batch=2, seqlen_q=1, seqlen_k=12)
    assert (out[0] == 0).all() and np.isneginf(lse[0, 0])
    assert_close(out[1, 0], o_part[1, 1, 0], 1e-15, "single live split passes through")
    assert_close([lse[0, 1]], [0.25], 1e-15, "single live split LSE")
    # Weighted sum by hand for two splits.
    o_part = np.random.default_rng(1).standard_normal((2, 1, 1, 3))
    lse_part = np.array([[[0.5]], [[-1.25]]])
    out, lse = o.combine(o_part, lse_part, chunk=8, batch=1, seqlen_q=1, seqlen_k=16)
    tot = math.log(math.exp(0.5) + math.exp(-1.25))
    exp_o = math.exp(0.5 - tot) * o_part[0, 0, 0] + math.exp(-1.25 - tot) * o_part[1, 0, 0]
    assert_close(out[0, 0], exp_o, 1e-15, "two-split combine O")
    assert_close([lse[0, 0]], [tot], 1e-15, "two-split combine LSE")


# ---- invariants ----------------------------------------------------------

def check_invariants(o):
    # GQA == MHA on repeat-interleaved K/V
    p = make_problem("gqa", dtype="bf16", lens_q=[3, 5], lens_k=[9, 4], hq=6, hkv=2,
                     dqk=8, dv=8, seed=400, varlen_q=True, varlen_k=True, causal=True)
    out_g, lse_g = run(o, p)
    from fmha_synth import Problem
    m = Problem("mha", p.dtype, p.q, p.k.repeat_interleave(3, dim=1),
                p.v.repeat_interleave(3, dim=1), 1.0, 1.0, 1.0, p.lens_q, p.lens_k,
                True, True, 6, 6, 8, 8, True)
    out_m, lse_m = run(o, m)
    assert_close(out_g, out_m, 0.0, "GQA == MHA(repeat) O")
    assert_close(lse_g, lse_m, 0.0, "GQA == MHA(repeat) LSE")
    # Joint key permutation leaves unmasked attention unchanged
    p = make_problem("perm", dtype="f16", lens_q=[4], lens_k=[23], hq=2, hkv=2,
                     dqk=8, dv=8, seed=401)
    out_a, lse_a = run(o, p)
    perm = torch.randperm(23, generator=torch.Generator().manual_seed(1))
    pp = Problem("perm2", p.dtype, p.q, p.k[perm], p.v[perm], 1.0, 1.0, 1.0,
                 p.lens_q, p.lens_k, False, False, 2, 2, 8, 8)
    out_b, lse_b = run(o, pp)
    assert_close(out_a, out_b, 1e-13, "key permutation O")
    assert_close(lse_a, lse_b, 1e-13, "key permutation LSE")
    # Packed == separate per-sequence calls (varlen Q and K)
    p = make_problem("packed", dtype="bf16", lens_q=[3, 1, 6], lens_k=[7, 12, 5], hq=2,
                     hkv=1, dqk=8, dv=4, seed=402, varlen_q=True, varlen_k=True,
                     causal=True)
    out_p, lse_p = run(o, p)
    q0 = k0 = 0
    for sq, sk in zip(p.lens_q, p.lens_k):
        s = Problem("one", p.dtype, p.q[q0:q0 + sq], p.k[k0:k0 + sk], p.v[k0:k0 + sk],
                    1.0, 1.0, 1.0, [sq], [sk], False, False, 2, 1, 8, 4, True)
        out_s, lse_s = run(o, s)
        assert_close(out_p[q0:q0 + sq], out_s, 0.0, "packed == separate O")
        assert_close(lse_p[:, q0:q0 + sq], lse_s, 0.0, "packed == separate LSE")
        q0 += sq
        k0 += sk
    # Q-only varlen and K-only varlen == fixed-length equivalents
    base = make_problem("fixed", dtype="f32", lens_q=[4, 4], lens_k=[6, 6], hq=2, hkv=2,
                        dqk=8, dv=8, seed=403, varlen_q=False, varlen_k=False,
                        causal=True)
    out_f, lse_f = run(o, base)
    for vq, vk in ((True, False), (False, True)):
        b2 = Problem("vq", base.dtype, base.q, base.k, base.v, 1.0, 1.0, 1.0,
                     base.lens_q, base.lens_k, vq, vk, 2, 2, 8, 8, True)
        out_v, lse_v = run(o, b2)
        assert_close(out_v, out_f, 0.0, f"varlen q={vq} k={vk} == fixed O")
        assert_close(lse_v, lse_f, 0.0, f"varlen q={vq} k={vk} == fixed LSE")
    # Mask special cases
    p = make_problem("masks", dtype="bf16", lens_q=[1, 7, 12], lens_k=[9, 7, 30], hq=2,
                     hkv=2, dqk=8, dv=8, seed=404, varlen_q=True, varlen_k=True)
    none_o, none_l = run(o, p)
    cau_o, cau_l = run(o, p, causal=True)
    # causal with sq == 1 is no mask
    assert_close(cau_o[0], none_o[0], 0.0, "causal sq=1 == no mask")
    # window (-1, 0) == causal
    w_o, w_l = run(o, p, window=(-1, 0))
    assert_close(w_o, cau_o, 0.0, "window(-1,0) == causal O")
    assert_close(w_l, cau_l, 0.0, "window(-1,0) == causal LSE")
    # window (>= sk, >= sk) == no mask
    big_o, big_l = run(o, p, window=(30, 30))
    assert_close(big_o, none_o, 0.0, "window(sk,sk) == no mask O")
    assert_close(big_l, none_l, 0.0, "window(sk,sk) == no mask LSE")
    # causal + window (wl, 5) == causal + window (wl, 0)
    a_o, _ = run(o, p, causal=True, window=(3, 5))
    b_o, _ = run(o, p, causal=False, window=(3, 0))
    assert_close(a_o, b_o, 0.0, "causal clamps the right window bound to 0")


# ---- decoders --------------------------------------------------------------

def check_decoders(o):
    codes16 = np.arange(65536, dtype=np.uint16)
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        got = o.decode(codes16, dt)
        ref = torch.from_numpy(codes16.view(np.int16)).view(tdt).to(torch.float64).numpy()
        same = (got == ref) | (np.isnan(got) & np.isnan(ref))
        assert same.all(), f"{dt} decoder differs at {np.flatnonzero(~same)[:5]}"
    codes8 = np.arange(256, dtype=np.uint8)
    got = o.decode(codes8, "fp8_e4m3")
    ref = torch.from_numpy(codes8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), f"e4m3 decoder differs at {np.flatnonzero(~same)[:5]}"
    # format facts: e4m3fn max 448, min normal 2^-6, min subnormal 2^-9
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def check_rows_driver(o):
    # The sampled-rows driver locates (sequence, position) from the packed
    # token index itself: it must reproduce the full result row for row,
    # leave no-key rows alone, and the full result is pinned above.
    p = make_problem("rows", dtype="bf16", lens_q=[3, 0, 4, 2], lens_k=[5, 3, 0, 9],
                     hq=4, hkv=2, dqk=8, dv=8, seed=500, varlen_q=True, varlen_k=True,
                     causal=True, window=(2, -1))
    full_o, full_l = run(o, p)
    tq = sum(p.lens_q)
    rt = [t for t in range(tq) for h in range(4)]
    rh = [h for t in range(tq) for h in range(4)]
    ro, rl = o.attention_rows(raw_bits(p.q), raw_bits(p.k), raw_bits(p.v), p.dtype,
                              rt, rh, cu_q=p.cu_q, cu_k=p.cu_k, scale=1 / math.sqrt(8),
                              causal=True, window=(2, -1))
    for n, (t, h) in enumerate(zip(rt, rh)):
        if np.isnan(full_l[h, t]):
            assert np.isnan(rl[n]) and np.isnan(ro[n]).all(), "no-key row written"
        else:
            assert_close(ro[n], full_o[t, h], 0.0, f"rows driver O[{t},{h}]")
            assert_close([rl[n]], [full_l[h, t]], 0.0, f"rows driver LSE[{h},{t}]")


ALL_CHECKS = [check_decoders, check_closed_forms, check_bruteforce, check_sdpa,
              check_split_combine, check_combine_edge, check_invariants,
              check_rows_driver]
