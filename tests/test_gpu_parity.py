"""GPU parity: the HIP path (through the C ABI binding) against the CPU oracle,
element by element, on seeded synthetic inputs of every workload shape.

Tolerances are in tests/gpu_helpers.py.  Full-size prefill is checked on
sampled rows the oracle computes one by one; everything else is checked on
every output element.
"""
from __future__ import annotations

import ctypes
import math
import sys

import numpy as np
import pytest
import torch

import fmha_synth as fs
from fmha_synth import make_problem, raw_bits
from gpu_helpers import (SENTINEL_LSE, SENTINEL_O, TOL_LSE, TOL_O, alloc_outputs,
                         compare, out_dtype, run_gpu, run_oracle, to_packed, upload)

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


def check(fmha, oracle, prob, splits=(0,), ref=None, label=""):
    ref = ref or run_oracle(oracle, prob)
    dev = upload(prob)
    errs = {}
    for s in splits:
        announce(f"{prob.name} {label} splits={s} dtype={prob.dtype} lens_q={prob.lens_q[:8]} "
                 f"lens_k={prob.lens_k[:8]} hq={prob.hq} hkv={prob.hkv} d={prob.dqk}/{prob.dv}")
        out, lse = run_gpu(fmha, prob, num_kv_splits=s, dev=dev)
        go, gl = to_packed(prob, out, lse)
        errs[s] = compare(prob, go, gl, *ref, what=f"{prob.name} {label} splits={s}")
    return errs


# ---- tiny: fp32 and bf16, splits {1, 4} -----------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny(fmha, oracle, dtype):
    prob = fs.tiny(dtype)
    check(fmha, oracle, prob, splits=(1, 4, 0))


# ---- long-context decode: full size, split sweep ----------------------------

def test_long_decode_split_sweep(fmha, oracle):
    prob = fs.long_decode()
    check(fmha, oracle, prob, splits=(0, 1, 2, 4, 8, 16, 32, 64, 128))


# ---- GQA batched decode: varlen K, full size ------------------------------

def test_gqa_decode(fmha, oracle):
    prob = fs.gqa_decode()
    check(fmha, oracle, prob, splits=(0, 1, 4))


# ---- fp8 short cached-prefix prefill ---------------------------------------

@pytest.mark.parametrize("seqlen_k", [11008, 16384])
def test_fp8_prefix(fmha, oracle, seqlen_k):
    prob = fs.fp8_prefix(seqlen_k)
    check(fmha, oracle, prob, splits=(0, 1, 4, 8, 16))


def test_fp8_prefix_causal_split(fmha, oracle):
    # the combination the fp8 split-K page refuses (causal, Sq=70, Skv=16384,
    # 4 splits) is computed exactly here: split == oracle
    prob = fs.fp8_prefix(16384)
    prob.causal = True
    check(fmha, oracle, prob, splits=(4, 1, 0), label="causal")


@pytest.mark.parametrize("dqk,lens_q", [(192, [70, 17, 33, 96, 1]), (192, [20, 5, 31, 1, 9]),
                                         (128, [70, 17, 33, 96, 1]), (128, [20, 5, 31, 1, 9])])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_varlen_prefix(fmha, oracle, dqk, lens_q, causal):
    # packed fp8 (Dv=128) with key offsets that are not multiples of 16 (the
    # unaligned varlen case) and query counts around the 32-row tiles; GQA 3:1
    # gives at most 288 rows (the 128-row kernel) or 93 (the 96-row one)
    prob = make_problem("fp8_varlen", dtype="fp8_e4m3", lens_q=lens_q,
                        lens_k=[1000, 77, 1301, 515, 9], hq=12, hkv=4, dqk=dqk, dv=128,
                        seed=13, varlen_q=True, varlen_k=True, causal=causal)
    dev = upload(prob)
    pl = fmha.plan(fmha.make_args(dev["q"], dev["k"], dev["v"], cu_seqlens_q=dev["cu_seqlens_q"],
                                  cu_seqlens_k=dev["cu_seqlens_k"],
                                  max_seqlen_q=dev["max_seqlen_q"],
                                  max_seqlen_k=dev["max_seqlen_k"], causal=causal,
                                  num_kv_splits=1, q_descale=dev.get("q_descale"),
                                  k_descale=dev.get("k_descale"),
                                  v_descale=dev.get("v_descale")))
    assert pl.rows_per_tile == (128 if max(lens_q) * 3 > 96 else 96), pl.rows_per_tile
    check(fmha, oracle, prob, splits=(0, 1, 3), label=f"d={dqk} causal={causal}")


# ---- varlen prefill ------------------------------------------------------

SMALL_SKEWED = [256, 32, 192, 64, 160, 96, 128, 96]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lengths", ["skewed", "equal"])
def test_varlen_prefill_small(fmha, oracle, lengths, causal):
    lens = SMALL_SKEWED if lengths == "skewed" else [128] * 8
    prob = make_problem(f"varlen_small_{lengths}", dtype="f16", lens_q=lens, lens_k=lens,
                        hq=16, hkv=16, dqk=128, dv=128, seed=4, varlen_q=True,
                        varlen_k=True, causal=causal)
    check(fmha, oracle, prob, splits=(0,))


@pytest.mark.parametrize("sq,sk", [(300, 200), (200, 500), (257, 257)])
def test_fixed_length_causal_prefill(fmha, oracle, sq, sk):
    # fixed-length (batched, no cu_seqlens) causal prefill in the longest-first
    # tile order; q > k leaves rows before the first key (O = 0, LSE = -inf)
    prob = make_problem("fixed_causal", dtype="bf16", lens_q=[sq] * 3, lens_k=[sk] * 3, hq=8,
                        hkv=4, dqk=128, dv=128, seed=13, varlen_q=False, varlen_k=False,
                        causal=True)
    check(fmha, oracle, prob, splits=(1, 0), label=f"{sq}x{sk}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_d256(fmha, oracle, dtype, causal):
    # head dim 256 (one wave per SIMD, 512-byte K/V rows): skewed lengths over
    # several 128-row tiles and 32-key blocks, ragged tails, GQA 8:2
    lens = [300, 33, 129, 1, 257]
    prob = make_problem("prefill_d256", dtype=dtype, lens_q=lens, lens_k=lens, hq=8, hkv=2,
                        dqk=256, dv=256, seed=12, varlen_q=True, varlen_k=True, causal=causal)
    check(fmha, oracle, prob, splits=(1,))


def sample_rows(prob, n_random=768, seed=0):
    """Token/head pairs: the first, last and tile-edge rows of every sequence
    at every query head, plus random (token, head) pairs."""
    rng = np.random.default_rng(seed)
    pairs = set()
    t0 = 0
    for sq in prob.lens_q:
        for i in (0, 1, 15, 16, 31, 32, 63, 64, 127, 128, sq // 2, sq - 2, sq - 1):
            if 0 <= i < sq:
                pairs |= {(t0 + i, h) for h in range(prob.hq)}
        t0 += sq
    tq = t0
    pairs |= set(zip((int(x) for x in rng.integers(0, tq, size=n_random)),
                     (int(x) for x in rng.integers(0, prob.hq, size=n_random))))
    pairs = sorted(pairs)
    return np.array([p[0] for p in pairs]), np.array([p[1] for p in pairs])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lengths", ["skewed", "equal"])
def test_varlen_prefill_full_sampled(fmha, oracle, lengths, causal):
    prob = fs.varlen_prefill(lengths, causal)
    announce(f"{prob.name} causal={causal} full size, sampled rows")
    out, lse = run_gpu(fmha, prob)
    go, gl = to_packed(prob, out, lse)
    rt, rh = sample_rows(prob)
    assert set(rh.tolist()) == set(range(prob.hq))
    ro, rl = oracle.attention_rows(raw_bits(prob.q), raw_bits(prob.k), raw_bits(prob.v),
                                   prob.dtype, rt, rh, cu_q=prob.cu_q, cu_k=prob.cu_k,
                                   scale=1 / math.sqrt(prob.dqk), causal=causal)
    err_o = float(np.max(np.abs(go[rt, rh] - ro)))
    err_l = float(np.max(np.abs(gl[rh, rt] - rl)))
    assert err_o <= TOL_O[prob.dtype], err_o
    assert err_l <= TOL_LSE, err_l
    # properties at every row: finite, |O| bounded by max |V| of the sequence
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    assert np.abs(go).max() <= float(prob.v.abs().max()) + 1e-3
    # every row has a key here: every LSE is written (no tile left out)
    assert (gl != SENTINEL_LSE).all()


# ---- tile orders: many sequences of mixed lengths --------------------------

WINDOWS = {"none": (-1, -1), "causal": (-1, -1), "right_window": (-1, 40),
           "left_window": (40, -1), "sliding": (128, 0)}


def _tile_table_model(prob, rows_per_tile, key_block):
    """(sequence, tile) -> cost of every existing tile (the key blocks its
    first and last rows span, + 1), for checking the device's table."""
    G = prob.hq // prob.hkv
    wl, wr = prob.window
    if prob.causal:
        wr = 0
    out = {}
    for b, (sq, sk) in enumerate(zip(prob.lens_q, prob.lens_k)):
        if sq == 0 or sk == 0:
            continue
        rows = sq * G
        for t in range(-(-rows // rows_per_tile)):
            i_lo, i_hi = t * rows_per_tile // G, (min(t * rows_per_tile + rows_per_tile, rows) - 1) // G
            lo = max(i_lo + sk - sq - wl, 0) if wl >= 0 else 0
            hi = min(i_hi + sk - sq + wr, sk - 1) if wr >= 0 else sk - 1
            jb = lo // key_block * key_block
            out[(b, t)] = (-(-(hi + 1 - jb) // key_block) if hi + 1 > jb else 0) + 1
    return out


@pytest.mark.parametrize("batch", [64, 65, 130, 200])
@pytest.mark.parametrize("mask", ["none", "causal", "right_window", "left_window", "sliding"])
def test_tile_order_many_sequences(fmha, oracle, batch, mask):
    # causal or a right-only window: up to 64 sequences take the in-kernel
    # longest-first order, more sequences and left windows the device-sorted
    # table; no mask the grouped order.  The lengths mix empty sequences,
    # q > k and k > q (rows before the first key)
    rng = np.random.default_rng(batch)
    choices = [0, 1, 31, 32, 33, 95, 128, 129, 200, 257, 300]
    lens_q = [int(x) for x in rng.choice(choices, size=batch)]
    lens_k = [int(x) for x in rng.choice(choices, size=batch)]
    lens_q[0], lens_k[0] = 300, 300
    prob = make_problem(f"tile_order_b{batch}", dtype="bf16" if mask == "none" else "f16",
                        lens_q=lens_q, lens_k=lens_k, hq=8, hkv=2, dqk=128, dv=128,
                        seed=11, varlen_q=True, varlen_k=True, causal=(mask == "causal"),
                        window=WINDOWS[mask])
    dev = upload(prob)
    args = fmha.make_args(dev["q"], dev["k"], dev["v"], cu_seqlens_q=dev["cu_seqlens_q"],
                          cu_seqlens_k=dev["cu_seqlens_k"], max_seqlen_q=dev["max_seqlen_q"],
                          max_seqlen_k=dev["max_seqlen_k"], causal=prob.causal,
                          window=prob.window, num_kv_splits=1)
    ws = torch.zeros(max(fmha.workspace_size(args), 256), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    pl = fmha.plan(args)
    expect = 0 if mask == "none" else (1 if batch <= 64 and mask in ("causal", "right_window")
                                       else 4)
    assert pl.tile_order == expect, (pl.tile_order, expect)
    check(fmha, oracle, prob, splits=(1,), label=mask)
    if expect == 4:
        _check_table(fmha, prob, dev, args, ws, pl, monotone=(mask != "sliding"), balanced=True)


def _check_table(fmha, prob, dev, args, ws, pl, *, monotone, balanced):
    """The table the schedule kernel wrote: every existing (tile, kv head)
    once, lists without holes, a group's items costliest first where tile
    costs are monotone along a sequence; optionally XCD loads balanced."""
    out, lse = alloc_outputs(prob, dev)
    args.out, args.lse = out.data_ptr(), lse.data_ptr()
    stream = torch.cuda.current_stream().cuda_stream
    assert fmha.lib.fmha_fwd(ctypes.byref(args), ctypes.c_void_p(stream)) == 0
    torch.cuda.synchronize()
    tab = ws[pl.sched_offset:].view(torch.int32).cpu().numpy()
    n = int(tab[0])
    assert n == pl.sched_items == pl.grid_main
    model = _tile_table_model(prob, pl.rows_per_tile, pl.key_block)
    H = prob.hkv
    # position 8 j + x: item j of XCD x's list; lists have no holes
    lists = [[] for _ in range(8)]
    for pos in range(n):
        b = int(tab[16 + 2 * pos])
        e = int(tab[17 + 2 * pos])
        lists[pos % 8].append(None if b < 0 else (b, e >> 20, e & 0xFFFFF))
    got = []
    for lst in lists:
        k = next((i for i, e in enumerate(lst) if e is None), len(lst))
        assert all(e is None for e in lst[k:]), "an XCD list has a hole"
        got += lst[:k]
        # a group's items within one list: contiguous, costliest tile first
        groups = []
        for e in lst[:k]:
            if not groups or groups[-1][0] != e[:2]:
                groups.append((e[:2], []))
            groups[-1][1].append(model[(e[0], e[2])])
        assert len({g[0] for g in groups}) == len(groups), "a group split within a list"
        if monotone:
            for _, costs in groups:
                assert all(a >= b for a, b in zip(costs, costs[1:])), "group not costliest first"
    want = sorted((b, h, t) for (b, t) in model for h in range(H))
    assert sorted(got) == want, "table is not every (tile, kv head) once"
    if balanced:
        # groups longest first: XCD loads within two groups' cost of each other
        load = [sum(model[(e[0], e[2])] for e in lst if e) for lst in lists]
        gmax = max(sum(model[(b, t)] for (bb, t) in model if bb == b) for b in {b for b, _ in model})
        assert max(load) - min(load) <= 2 * gmax
    return lists


def test_tile_table_list_overflow(fmha, oracle):
    # Dealing groups by cost does not bound an XCD list's tile count: here every
    # sequence costs 17 key-block units (causal, GQA 4:1, 128-row tiles of 32-key
    # blocks), but "M" sequences (512 queries, 8 keys: 15 keyless tiles + 1) have
    # 16 tiles and "F" sequences (32 queries, 512 keys) one.  Equal costs rank by
    # index, and the pattern M F F F F F F M puts both kv heads of every M on XCDs
    # 0 and 1: 32 tiles per 8 sequences there against 2 elsewhere, far past a
    # list's room (1/8 of the tile bound plus one sequence's tiles).  The
    # schedule moves the excess to the other lists; every row must be written
    # (the keyless ones as O = 0, LSE = -inf) and every tile listed once.
    pattern = "MFFFFFFM" * 9
    lens_q = [512 if c == "M" else 32 for c in pattern]
    lens_k = [8 if c == "M" else 512 for c in pattern]
    prob = make_problem("tile_table_overflow", dtype="f16", lens_q=lens_q, lens_k=lens_k,
                        hq=8, hkv=2, dqk=128, dv=128, seed=14, varlen_q=True, varlen_k=True,
                        causal=True)
    model = _tile_table_model(prob, 128, 32)
    costs = {b: sum(c for (bb, _), c in model.items() if bb == b) for b in range(len(pattern))}
    assert set(costs.values()) == {17}, costs
    dev = upload(prob)
    args = fmha.make_args(dev["q"], dev["k"], dev["v"], cu_seqlens_q=dev["cu_seqlens_q"],
                          cu_seqlens_k=dev["cu_seqlens_k"], max_seqlen_q=dev["max_seqlen_q"],
                          max_seqlen_k=dev["max_seqlen_k"], causal=True, num_kv_splits=1)
    ws = torch.zeros(max(fmha.workspace_size(args), 256), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    pl = fmha.plan(args)
    assert pl.tile_order == 4 and pl.rows_per_tile == 128 and pl.key_block == 32, pl
    room = pl.sched_items // 8
    m_tiles = 16 * pattern.count("M")  # dealt to XCD 0: one kv head of every M sequence
    assert m_tiles > room, (m_tiles, room)
    announce(f"tile table overflow: {len(pattern)} sequences, XCD 0 dealt {m_tiles} tiles, room {room}")
    check(fmha, oracle, prob, splits=(1,), label="causal")
    lists = _check_table(fmha, prob, dev, args, ws, pl, monotone=True, balanced=False)
    assert max(sum(e is not None for e in lst) for lst in lists) <= room
    # the persistent grid claims the moved items at the ends of the other lists
    ref = run_oracle(oracle, prob)
    out, lse = run_gpu(fmha, prob, num_kv_splits=1, dev=dev, persistent=True)
    go, gl = to_packed(prob, out, lse)
    compare(prob, go, gl, *ref, what="tile table overflow, persistent")


@pytest.mark.parametrize("seed", range(6))
def test_longest_first_random_mixes(fmha, oracle, seed):
    # the in-kernel longest-first order (up to 64 sequences, causal or a right
    # window) on seeded length mixes with keyless tiles (many queries, few
    # keys), keyless sequences and long ones: every row as the oracle
    menu = [(0, 7), (5, 0), (1, 900), (32, 512), (512, 8), (300, 300), (129, 1000), (1000, 40),
            (64, 64), (700, 1)]
    rng = np.random.default_rng(2000 + seed)
    batch = int(rng.integers(2, 65))
    picks = rng.integers(0, len(menu), batch)
    lens_q = [menu[i][0] for i in picks]
    lens_k = [menu[i][1] for i in picks]
    lens_q[0], lens_k[0] = 300, 300
    mask = ("causal", "right_window")[seed % 2]
    prob = make_problem(f"lf_mix_{seed}", dtype=("f16", "bf16")[seed % 2], lens_q=lens_q,
                        lens_k=lens_k, hq=8, hkv=2, dqk=(64, 128, 256)[seed % 3],
                        dv=(64, 128, 256)[seed % 3], seed=seed, varlen_q=True, varlen_k=True,
                        causal=(mask == "causal"), window=WINDOWS[mask])
    dev = upload(prob)
    args = fmha.make_args(dev["q"], dev["k"], dev["v"], cu_seqlens_q=dev["cu_seqlens_q"],
                          cu_seqlens_k=dev["cu_seqlens_k"], max_seqlen_q=dev["max_seqlen_q"],
                          max_seqlen_k=dev["max_seqlen_k"], causal=prob.causal,
                          window=prob.window, num_kv_splits=1)
    assert fmha.plan(args).tile_order == 1
    check(fmha, oracle, prob, splits=(1,), label=mask)


@pytest.mark.parametrize("seed", range(6))
def test_heads_together_random(fmha, oracle, seed):
    # one query tile per sequence and several splits put the kv heads of one
    # (sequence, split) together on an XCD (tile order 3, a last partial round
    # in head pairs): odd and even kv-head counts, GQA, varlen q and k with
    # empty and short sequences, explicit splits
    rng = np.random.default_rng(3000 + seed)
    hkv = (1, 3, 5, 12, 7, 2)[seed]
    g = (1, 2, 1, 1, 4, 8)[seed]
    dtype = ("fp8_e4m3", "f16", "bf16")[seed % 3]
    d = 128 if dtype != "fp8_e4m3" else (128, 192)[seed % 2]
    rows = 96 if dtype == "fp8_e4m3" else 128  # one query tile: q * g rows at most
    batch = int(rng.integers(1, 6))
    lens_q = [int(x) for x in rng.integers(rows // (2 * g), rows // g + 1, batch)]
    lens_k = [int(x) for x in rng.choice([0, 1, 700, 3000, 5000], size=batch)]
    lens_k[0] = 4096
    prob = make_problem(f"heads_together_{seed}", dtype=dtype, lens_q=lens_q, lens_k=lens_k,
                        hq=hkv * g, hkv=hkv, dqk=d, dv=128, seed=seed, varlen_q=True,
                        varlen_k=True)
    dev = upload(prob)
    splits = (3, 7, 16)[seed % 3]
    args = fmha.make_args(dev["q"], dev["k"], dev["v"], cu_seqlens_q=dev["cu_seqlens_q"],
                          cu_seqlens_k=dev["cu_seqlens_k"], max_seqlen_q=dev["max_seqlen_q"],
                          max_seqlen_k=dev["max_seqlen_k"], num_kv_splits=splits,
                          q_descale=dev.get("q_descale"), k_descale=dev.get("k_descale"),
                          v_descale=dev.get("v_descale"))
    ws = torch.zeros(max(fmha.workspace_size(args), 256), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    pl = fmha.plan(args)
    assert pl.num_q_tiles == 1 and pl.num_splits == splits and pl.tile_order == 3, pl
    check(fmha, oracle, prob, splits=(splits,), label=f"hkv={hkv} g={g}")


def test_tile_table_random_mixes(fmha):
    # the device schedule on many seeded length mixes (tables only, no oracle):
    # sequences with many queries and few keys (cheap but many tiles), the
    # reverse, empty ones and long ones, 65..300 sequences, three masks, GQA
    # 4:1 and 1:1, head dims 64 and 128; every table must list every (tile, kv
    # head) once, without holes, each group costliest first where costs are
    # monotone
    menu = [(0, 7), (5, 0), (1, 900), (32, 512), (512, 8), (300, 300), (129, 2000), (2000, 40),
            (64, 64), (700, 1)]
    cases = 0
    for seed in range(24):
        rng = np.random.default_rng(1000 + seed)
        batch = int(rng.integers(65, 301))
        picks = rng.integers(0, len(menu), batch)
        lens_q = [menu[i][0] for i in picks]
        lens_k = [menu[i][1] for i in picks]
        lens_q[0], lens_k[0] = 300, 300
        mask = ("causal", "left_window", "sliding")[seed % 3]
        hq, hkv = ((8, 2), (4, 4))[seed % 2]
        d = (64, 128)[(seed // 2) % 2]  # 64- and 32-key blocks
        prob = make_problem(f"tile_mix_{seed}", dtype="f16", lens_q=lens_q, lens_k=lens_k, hq=hq,
                            hkv=hkv, dqk=d, dv=d, seed=seed, varlen_q=True, varlen_k=True,
                            causal=(mask == "causal"), window=WINDOWS[mask])
        dev = upload(prob)
        args = fmha.make_args(dev["q"], dev["k"], dev["v"], cu_seqlens_q=dev["cu_seqlens_q"],
                              cu_seqlens_k=dev["cu_seqlens_k"], max_seqlen_q=dev["max_seqlen_q"],
                              max_seqlen_k=dev["max_seqlen_k"], causal=prob.causal,
                              window=prob.window, num_kv_splits=1)
        ws = torch.zeros(max(fmha.workspace_size(args), 256), dtype=torch.uint8, device="cuda")
        args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
        pl = fmha.plan(args)
        assert pl.tile_order == 4, (seed, pl.tile_order)
        announce(f"tile table mix {seed}: {batch} sequences, {mask}, GQA {hq}:{hkv}")
        _check_table(fmha, prob, dev, args, ws, pl, monotone=(mask != "sliding"), balanced=False)
        cases += 1
    assert cases == 24


@pytest.mark.parametrize("batch", [64, 65])
def test_decode_split_order_many_sequences(fmha, oracle, batch):
    # decode with splits: 64 sequences take the full-first split order, 65 the
    # plain one; the key lengths mix empty sequences, exact multiples of the
    # 96-key chunk (7 splits of max 672 keys) and partial last splits, the query
    # lengths 0..4 rows per sequence (GQA 4:1 packs them into one 16-row tile)
    rng = np.random.default_rng(100 + batch)
    lens_q = [int(x) for x in rng.choice([0, 1, 1, 1, 2, 4], size=batch)]
    lens_k = [int(x) for x in rng.choice([0, 1, 31, 96, 97, 192, 300, 480, 671, 672], size=batch)]
    lens_q[0], lens_k[0] = 1, 672
    prob = make_problem(f"decode_order_b{batch}", dtype="bf16", lens_q=lens_q, lens_k=lens_k,
                        hq=8, hkv=2, dqk=128, dv=128, seed=12, varlen_q=True, varlen_k=True)
    dev = upload(prob)
    pl = fmha.plan(fmha.make_args(dev["q"], dev["k"], dev["v"], cu_seqlens_q=dev["cu_seqlens_q"],
                                  cu_seqlens_k=dev["cu_seqlens_k"],
                                  max_seqlen_q=dev["max_seqlen_q"],
                                  max_seqlen_k=dev["max_seqlen_k"], num_kv_splits=7,
                                  workspace=torch.zeros(16 << 20, dtype=torch.uint8,
                                                        device="cuda")))
    assert pl.split_chunk == 96 and pl.tile_order == (2 if batch <= 64 else 0)
    check(fmha, oracle, prob, splits=(7, 0), label=f"decode order b{batch}")


@pytest.mark.parametrize("dtype,d,dv", [("f16", 64, 64), ("f16", 128, 128), ("bf16", 64, 64),
                                        ("fp8_e4m3", 128, 128), ("fp8_e4m3", 192, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_kernels(fmha, oracle, dtype, d, dv, causal):
    # every decode instance (<= 16 rows per (sequence, kv head): 1..4 queries x
    # 4 q heads per kv head), packed keys of mixed lengths including an empty
    # sequence and one shorter than its queries
    prob = make_problem(f"decode_{dtype}_{d}", dtype=dtype, lens_q=[1, 4, 2, 1, 3],
                        lens_k=[3000, 517, 0, 33, 2], hq=8, hkv=2, dqk=d, dv=dv, seed=14,
                        varlen_q=True, varlen_k=True, causal=causal)
    dev = upload(prob)
    pl = fmha.plan(fmha.make_args(dev["q"], dev["k"], dev["v"], cu_seqlens_q=dev["cu_seqlens_q"],
                                  cu_seqlens_k=dev["cu_seqlens_k"],
                                  max_seqlen_q=dev["max_seqlen_q"],
                                  max_seqlen_k=dev["max_seqlen_k"], causal=causal,
                                  num_kv_splits=1, q_descale=dev.get("q_descale"),
                                  k_descale=dev.get("k_descale"),
                                  v_descale=dev.get("v_descale")))
    assert pl.kernel_id % 1000 in (100, 101), pl.kernel_id  # a decode instance
    check(fmha, oracle, prob, splits=(0, 1, 5), label=f"causal={causal}")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("max_q,nwm", [(1, 1), (6, 2), (12, 4), (20, 5)])
def test_generic_kernel_tiles(fmha, oracle, dtype, d, max_q, nwm):
    # the 16-row-tile kernel at each of its tile heights: GQA 4:1 packs
    # max_q queries into 4 * max_q rows (f16/bf16 use it from 17 to 80 rows and,
    # for head dims without a decode instance, below; f32 throughout)
    if dtype != "f32" and nwm == 1 and d != 256:
        pytest.skip("served by the decode kernel")
    if dtype == "f32" and d == 256:
        pytest.skip("no f32 instance at D = 256 (UNSUPPORTED)")
    prob = make_problem(f"generic_{dtype}_{d}_{max_q}", dtype=dtype, lens_q=[max_q, max_q // 2 + 1, 1],
                        lens_k=[300, 77, 40], hq=8, hkv=2, dqk=d, dv=d, seed=15, varlen_q=True,
                        varlen_k=True, causal=True)
    dev = upload(prob)
    pl = fmha.plan(fmha.make_args(dev["q"], dev["k"], dev["v"], cu_seqlens_q=dev["cu_seqlens_q"],
                                  cu_seqlens_k=dev["cu_seqlens_k"],
                                  max_seqlen_q=dev["max_seqlen_q"],
                                  max_seqlen_k=dev["max_seqlen_k"], causal=True,
                                  num_kv_splits=1))
    assert pl.rows_per_tile == 16 * nwm, pl.rows_per_tile
    check(fmha, oracle, prob, splits=(0, 1, 3), label=f"nwm={nwm}")


# ---- edge set: lengths [1,0,63,64,65,128,129,700], GQA 8:2, bf16 ----------

@pytest.mark.parametrize("mask", ["window", "none", "causal"])
def test_edge_set(fmha, oracle, mask):
    prob = fs.edge_set(causal=(mask == "causal"),
                       window=(128, 0) if mask == "window" else (-1, -1))
    check(fmha, oracle, prob, splits=(0, 1, 3), label=mask)


@pytest.mark.parametrize("hkv", [8, 2, 1])
@pytest.mark.parametrize("mask", ["none", "causal", "window"])
def test_edge_set_gqa_matrix(fmha, oracle, hkv, mask):
    prob = make_problem("edge_gqa", dtype="bf16", lens_q=fs.EDGE_LENGTHS,
                        lens_k=fs.EDGE_LENGTHS, hq=8, hkv=hkv, dqk=128, dv=128, seed=5,
                        varlen_q=True, varlen_k=True, causal=(mask == "causal"),
                        window=(128, 0) if mask == "window" else (-1, -1))
    check(fmha, oracle, prob, splits=(0,), label=f"{mask} 8:{hkv}")


@pytest.mark.parametrize("causal", [False, True])
def test_different_q_k_lengths(fmha, oracle, causal):
    # q "3,(1,129,700),8,128"  k "3,(65,300,700),2,128"
    prob = make_problem("qk_lengths", dtype="bf16", lens_q=[1, 129, 700],
                        lens_k=[65, 300, 700], hq=8, hkv=2, dqk=128, dv=128, seed=6,
                        varlen_q=True, varlen_k=True, causal=causal)
    check(fmha, oracle, prob, splits=(0, 1, 2, 5), label=f"causal={causal}")


@pytest.mark.parametrize("side", ["q", "k"])
def test_varlen_one_side(fmha, oracle, side):
    lens_q = [37, 37, 37] if side == "k" else [5, 90, 33]
    lens_k = [200, 13, 77] if side == "k" else [150, 150, 150]
    prob = make_problem(f"varlen_{side}_only", dtype="f16", lens_q=lens_q, lens_k=lens_k,
                        hq=4, hkv=2, dqk=128, dv=128, seed=7, varlen_q=(side == "q"),
                        varlen_k=(side == "k"), causal=True)
    check(fmha, oracle, prob, splits=(0, 1, 3))


@pytest.mark.parametrize("dtype,d,dv", [("bf16", 64, 64), ("bf16", 256, 256),
                                        ("f16", 64, 64), ("f16", 256, 256),
                                        ("f32", 128, 128), ("fp8_e4m3", 128, 128)])
def test_head_dims(fmha, oracle, dtype, d, dv):
    prob = make_problem(f"dims_{dtype}_{d}", dtype=dtype, lens_q=[1, 67, 130],
                        lens_k=[300, 67, 513], hq=4, hkv=2, dqk=d, dv=dv, seed=8,
                        varlen_q=True, varlen_k=True, causal=True)
    check(fmha, oracle, prob, splits=(0, 1, 2))


def test_queries_without_keys_complete(fmha):
    # a sequence with queries but no keys: completes, rows untouched
    prob = make_problem("no_keys", dtype="bf16", lens_q=[4, 9], lens_k=[0, 0], hq=2,
                        hkv=2, dqk=64, dv=64, seed=9, varlen_q=True, varlen_k=True)
    out, lse = run_gpu(fmha, prob, num_kv_splits=2)
    assert (out.float() == SENTINEL_O).all() and (lse == SENTINEL_LSE).all()


# ---- split partials and the combine --------------------------------------

def test_partials_match_oracle_splits(fmha, oracle):
    prob = make_problem("partials", dtype="bf16", lens_q=[1, 3, 2], lens_k=[700, 129, 0],
                        hq=8, hkv=2, dqk=128, dv=128, seed=10, varlen_q=True,
                        varlen_k=True, causal=True)
    dev = upload(prob)
    announce("partials vs oracle split partials")
    o_part, lse_part, pl = fmha.splitkv_partials(
        dev["q"], dev["k"], dev["v"], num_kv_splits=5, cu_seqlens_q=dev["cu_seqlens_q"],
        cu_seqlens_k=dev["cu_seqlens_k"], max_seqlen_q=dev["max_seqlen_q"],
        max_seqlen_k=dev["max_seqlen_k"], causal=True)
    torch.cuda.synchronize()
    chunk = pl.split_chunk
    assert pl.num_splits == 5 and chunk % pl.key_block == 0
    scale = 1 / math.sqrt(128)
    for s in range(5):
        ro, rl = oracle.split_attention(raw_bits(prob.q), raw_bits(prob.k), raw_bits(prob.v),
                                        "bf16", chunk=chunk, split=s, cu_q=prob.cu_q,
                                        cu_k=prob.cu_k, scale=scale, causal=True)
        go = o_part[s].double().cpu().numpy()
        gl = lse_part[s].double().cpu().numpy()
        t0 = 0
        for sq, sk in zip(prob.lens_q, prob.lens_k):
            if s < -(-sk // chunk):  # written splits only
                sl = slice(t0, t0 + sq)
                assert np.array_equal(np.isneginf(gl[:, sl]), np.isneginf(rl[:, sl]))
                fin = ~np.isneginf(rl[:, sl])
                assert np.abs(go[sl] - ro[sl]).max() <= TOL_O["bf16"]
                if fin.any():
                    assert np.abs(gl[:, sl][fin] - rl[:, sl][fin]).max() <= TOL_LSE
            t0 += sq


def test_combine_kernel_on_oracle_partials(fmha, oracle):
    # partials computed by the oracle alone, rounded to fp32, combined on the GPU
    prob = make_problem("combine", dtype="f32", lens_q=[2, 1, 3], lens_k=[90, 0, 33],
                        hq=4, hkv=4, dqk=64, dv=64, seed=11, varlen_q=True, varlen_k=True,
                        causal=True)
    chunk, S = 16, 6
    scale = 0.125
    parts = [oracle.split_attention(raw_bits(prob.q), raw_bits(prob.k), raw_bits(prob.v),
                                    "f32", chunk=chunk, split=s, cu_q=prob.cu_q,
                                    cu_k=prob.cu_k, scale=scale, causal=True)
             for s in range(S)]
    o_part = np.stack([p[0] for p in parts]).astype(np.float32)
    l_part = np.stack([p[1] for p in parts]).astype(np.float32)
    ref_o, ref_l = oracle.combine(o_part.astype(np.float64), l_part.astype(np.float64),
                                  chunk=chunk, cu_q=prob.cu_q, cu_k=prob.cu_k)
    dev = upload(prob)
    out, lse = alloc_outputs(prob, dev)
    op = torch.from_numpy(np.nan_to_num(o_part, nan=0.0)).cuda()
    lp = torch.from_numpy(np.nan_to_num(l_part, nan=-np.inf)).cuda()
    announce("combine kernel on oracle partials")
    fmha.splitkv_combine(op, lp, split_chunk=chunk, out=out, lse=lse,
                         cu_seqlens_q=dev["cu_seqlens_q"], cu_seqlens_k=dev["cu_seqlens_k"],
                         max_seqlen_q=dev["max_seqlen_q"])
    torch.cuda.synchronize()
    go, gl = to_packed(prob, out, lse)
    compare(prob, go, gl, ref_o, ref_l, what="combine")
    assert np.abs(go[~np.isnan(ref_o)] - ref_o[~np.isnan(ref_o)]).max() < 1e-5


@pytest.mark.parametrize("num_splits,dv,lens_q", [
    (6, 64, [2, 1]),        # few rows: narrowest column groups, one partial row per thread
    (100, 128, [3, 2]),     # few rows, many splits: several partial rows per thread
    (256, 128, [40, 30]),   # many rows: widest groups capped so a thread owns <= 16 rows
    (256, 256, [2, 1]),     # widest Dv, most splits
    (37, 256, [40, 30]),
    # many rows, few partials: one wave per row
    (20, 128, [40, 30]),
    (6, 64, [40, 30]),
    (16, 256, [40, 30]),
    (3, 128, [70]),
])
def test_combine_shapes(fmha, oracle, num_splits, dv, lens_q):
    # the combine's grid shapes (column-group width, partial rows per thread)
    # on oracle partials: every split of every row, fp32
    chunk = 4
    lens_k = [num_splits * chunk - 3, (num_splits * chunk) // 3][:len(lens_q)]
    prob = make_problem(f"combine_{num_splits}_{dv}", dtype="f32", lens_q=lens_q, lens_k=lens_k,
                        hq=4, hkv=4, dqk=dv, dv=dv, seed=12, varlen_q=True, varlen_k=True)
    scale = 1 / math.sqrt(dv)
    parts = [oracle.split_attention(raw_bits(prob.q), raw_bits(prob.k), raw_bits(prob.v),
                                    "f32", chunk=chunk, split=s, cu_q=prob.cu_q,
                                    cu_k=prob.cu_k, scale=scale)
             for s in range(num_splits)]
    o_part = np.stack([p[0] for p in parts]).astype(np.float32)
    l_part = np.stack([p[1] for p in parts]).astype(np.float32)
    ref_o, ref_l = oracle.combine(o_part.astype(np.float64), l_part.astype(np.float64),
                                  chunk=chunk, cu_q=prob.cu_q, cu_k=prob.cu_k)
    dev = upload(prob)
    out, lse = alloc_outputs(prob, dev)
    op = torch.from_numpy(np.nan_to_num(o_part, nan=0.0)).cuda()
    lp = torch.from_numpy(np.nan_to_num(l_part, nan=-np.inf)).cuda()
    announce(f"combine shapes S={num_splits} dv={dv} lens_q={lens_q}")
    fmha.splitkv_combine(op, lp, split_chunk=chunk, out=out, lse=lse,
                         cu_seqlens_q=dev["cu_seqlens_q"], cu_seqlens_k=dev["cu_seqlens_k"],
                         max_seqlen_q=dev["max_seqlen_q"])
    torch.cuda.synchronize()
    go, gl = to_packed(prob, out, lse)
    compare(prob, go, gl, ref_o, ref_l, what=f"combine S={num_splits} dv={dv}")
    assert np.abs(go - ref_o).max() < 1e-5


# ---- determinism, graph replay, guard bands, errors -------------------------

def test_determinism(fmha):
    prob = fs.edge_set()
    dev = upload(prob)
    announce("determinism")
    a = run_gpu(fmha, prob, dev=dev, num_kv_splits=3)
    b = run_gpu(fmha, prob, dev=dev, num_kv_splits=3)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_graph_capture_replay(fmha):
    prob = fs.fp8_prefix(11008)
    dev = upload(prob)
    out, lse = alloc_outputs(prob, dev)
    kw = dict(cu_seqlens_q=None, cu_seqlens_k=None, num_kv_splits=8,
              q_descale=dev["q_descale"], k_descale=dev["k_descale"],
              v_descale=dev["v_descale"], out=out, lse=lse)
    ws_args = fmha.make_args(dev["q"], dev["k"], dev["v"], num_kv_splits=8,
                             num_cus=fmha.device_num_cus(), out=out, lse=lse)
    ws = torch.zeros(fmha.workspace_size(ws_args), dtype=torch.uint8, device="cuda")
    announce("graph capture + replay")
    fmha.fwd(dev["q"], dev["k"], dev["v"], workspace=ws, **kw)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    out.fill_(0)
    lse.fill_(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fmha.fwd(dev["q"], dev["k"], dev["v"], workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        out.fill_(0)
        lse.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep} O"
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), f"replay {rep} LSE"
        _ = (dev["q"].float().sum() + 1).item()  # unrelated eager work between replays


def test_guard_bands(fmha):
    prob = make_problem("guards", dtype="bf16", lens_q=[3, 65, 1], lens_k=[129, 65, 40],
                        hq=8, hkv=2, dqk=128, dv=128, seed=12, varlen_q=True, varlen_k=True,
                        causal=True)
    dev = upload(prob)
    tq = sum(prob.lens_q)
    pad = 4096
    ob = torch.full((pad + tq * 8 * 128 + pad,), SENTINEL_O, dtype=torch.bfloat16, device="cuda")
    lb = torch.full((pad + 8 * tq + pad,), SENTINEL_LSE, dtype=torch.float32, device="cuda")
    out = ob[pad:pad + tq * 8 * 128].view(tq, 8, 128)
    lse = lb[pad:pad + 8 * tq].view(8, tq)
    for s in (1, 4):
        announce(f"guard bands splits={s}")
        run_gpu(fmha, prob, dev=dev, out=out, lse=lse, num_kv_splits=s)
        assert (ob[:pad].float() == SENTINEL_O).all() and (ob[-pad:].float() == SENTINEL_O).all()
        assert (lb[:pad] == SENTINEL_LSE).all() and (lb[-pad:] == SENTINEL_LSE).all()


def test_errors_write_nothing(fmha):
    prob = fs.tiny("bf16")
    dev = upload(prob)
    out, lse = alloc_outputs(prob, dev)
    q, k, v = dev["q"], dev["k"], dev["v"]
    bad = [
        dict(softmax_scale=-1.0),
        dict(window=(-2, 0)),
        dict(num_kv_splits=257),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            fmha.fwd(q, k, v, out=out, lse=lse, **kw)
    with pytest.raises(ValueError):  # Hq % Hkv != 0
        fmha.fwd(q[:, :, :3], k, v, out=out[:, :, :3], lse=lse[:, :3])
    with pytest.raises(ValueError):  # no kernel for head dim 48
        fmha.fwd(q[..., :48], k[..., :48], v, out=out, lse=lse)
    with pytest.raises(ValueError):  # workspace too small
        fmha.fwd(q, k, v, out=out, lse=lse, num_kv_splits=4,
                 workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert (out.float() == SENTINEL_O).all() and (lse == SENTINEL_LSE).all()


def test_binding_rejects_mismatched_tensors(fmha):
    # the binding checks dtype, device and shape before the library sees a
    # pointer: an int64 cu_seqlens, an out of another dtype or shape, a short
    # lse or a non-fp32 descale would otherwise be read or written wrongly
    prob = fs.edge_set()
    dev = upload(prob)
    out, lse = alloc_outputs(prob, dev)
    kw = dict(cu_seqlens_q=dev["cu_seqlens_q"], cu_seqlens_k=dev["cu_seqlens_k"],
              max_seqlen_q=dev["max_seqlen_q"], max_seqlen_k=dev["max_seqlen_k"])
    q, k, v = dev["q"], dev["k"], dev["v"]
    bad = [
        dict(kw, cu_seqlens_q=dev["cu_seqlens_q"].long()),
        dict(kw, cu_seqlens_k=dev["cu_seqlens_k"].cpu()),
        dict(kw, out=out.float(), lse=lse),
        dict(kw, out=out[:-1], lse=lse),
        dict(kw, out=out, lse=lse[:, :-1]),
        dict(kw, out=out, lse=lse.double()),
    ]
    for b in bad:
        with pytest.raises(ValueError):
            fmha.fwd(q, k, v, **b)
    with pytest.raises(ValueError):  # a host tensor among device ones
        fmha.fwd(q, k.cpu(), v, out=out, lse=lse, **kw)
    f8 = fs.fp8_prefix(11008)
    d8 = upload(f8)
    with pytest.raises(ValueError):
        fmha.fwd(d8["q"], d8["k"], d8["v"], q_descale=d8["q_descale"].half(),
                 k_descale=d8["k_descale"], v_descale=d8["v_descale"])
    torch.cuda.synchronize()
    assert (out.float() == SENTINEL_O).all() and (lse == SENTINEL_LSE).all()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_o_unbiased(fmha, oracle, dtype):
    # P is rounded to nearest even before the PV MFMA while the row sum adds
    # the unrounded p, so O carries no systematic scale error: the least-squares
    # slope of (O_gpu - O_oracle) on O_oracle stays far below one P rounding
    # step (2^-11 relative for f16: a one-sided rounding would show a slope of
    # about -2^-12); the max error stays within the usual tolerance
    lens = [512] * 8
    prob = make_problem(f"bias_{dtype}", dtype=dtype, lens_q=lens, lens_k=lens, hq=8, hkv=8,
                        dqk=128, dv=128, seed=17, varlen_q=True, varlen_k=True)
    ro, rl = run_oracle(oracle, prob)
    announce(f"signed O error {dtype}")
    out, lse = run_gpu(fmha, prob, num_kv_splits=1)
    go, gl = to_packed(prob, out, lse)
    compare(prob, go, gl, ro, rl, what="bias")
    # the output rounding (to the input dtype, nearest even) is unbiased too;
    # remove it from the comparison by rounding the oracle the same way
    rr = torch.from_numpy(ro).to(fs.TORCH_DTYPE[dtype]).double().numpy()
    slope = float(((go - rr) * rr).sum() / (rr * rr).sum())
    announce(f"{dtype} prefill: O error slope {slope:.3e}")
    assert abs(slope) < 2.0 ** -15, slope


# ---- split combine inside the attention launch ------------------------------

def _f8_args(fmha, dev, out, lse, splits, ws=None):
    a = fmha.make_args(dev["q"], dev["k"], dev["v"], out=out, lse=lse, num_kv_splits=splits,
                       q_descale=dev["q_descale"], k_descale=dev["k_descale"],
                       v_descale=dev["v_descale"], num_cus=fmha.device_num_cus(),
                       combine_in_kernel=True)
    if ws is not None:
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    return a


@pytest.mark.parametrize("seed", range(4))
def test_in_kernel_combine_random(fmha, oracle, seed):
    # the in-launch combine beyond the fp8 prefix: f16/bf16/fp8 multi-row
    # kernels, varlen q and k (empty and short sequences, splits that some
    # sequences do not reach), GQA, 2-12 kv heads, 2-20 splits, causal or not
    rng = np.random.default_rng(4000 + seed)
    dtype = ("f16", "bf16", "fp8_e4m3", "f16")[seed]
    hkv, g = ((2, 4), (5, 1), (3, 2), (12, 1))[seed]
    splits = (2, 7, 20, 9)[seed]
    d = 128
    rows = 96 if dtype == "fp8_e4m3" else 128
    batch = int(rng.integers(1, 4))
    # more than 80 query rows per (sequence, kv head) for the f16/bf16 multi-row
    # kernel (fewer take the 16-row kernel, which has no in-launch combine)
    lens_q = [int(x) for x in rng.integers(2 * rows // (3 * g) + 1, rows // g + 1, batch)]
    lens_k = [int(x) for x in rng.choice([0, 1, 900, 2500], size=batch)]
    lens_k[0] = 3000
    causal = seed % 2 == 1
    splits = min(splits, fmha.device_num_cus() // (batch * hkv))  # the grid must be resident
    prob = make_problem(f"in_kernel_combine_{seed}", dtype=dtype, lens_q=lens_q, lens_k=lens_k,
                        hq=hkv * g, hkv=hkv, dqk=d, dv=d, seed=seed, varlen_q=True,
                        varlen_k=True, causal=causal)
    dev = upload(prob)
    out, lse = alloc_outputs(prob, dev)
    args = fmha.make_args(dev["q"], dev["k"], dev["v"], out=out, lse=lse,
                          cu_seqlens_q=dev["cu_seqlens_q"],
                          cu_seqlens_k=dev["cu_seqlens_k"], max_seqlen_q=dev["max_seqlen_q"],
                          max_seqlen_k=dev["max_seqlen_k"], causal=causal, num_kv_splits=splits,
                          q_descale=dev.get("q_descale"), k_descale=dev.get("k_descale"),
                          v_descale=dev.get("v_descale"), num_cus=fmha.device_num_cus(),
                          combine_in_kernel=True)
    ws = torch.zeros(max(fmha.workspace_size(args), 256), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    pl = fmha.plan(args)
    assert pl.combine_in_kernel == 1 and pl.num_splits == splits, pl
    ref = run_oracle(oracle, prob)
    for rep in range(2):  # the counters are zero again after each launch
        announce(f"in-kernel combine {dtype} hkv={hkv} g={g} S={splits} causal={causal} rep {rep}")
        out, lse = alloc_outputs(prob, dev)
        args.out, args.lse = out.data_ptr(), lse.data_ptr()
        stream = torch.cuda.current_stream().cuda_stream
        assert fmha.lib.fmha_fwd(ctypes.byref(args), ctypes.c_void_p(stream)) == 0
        torch.cuda.synchronize()
        go, gl = to_packed(prob, out, lse)
        compare(prob, go, gl, *ref, what=f"in-kernel combine random {seed} rep {rep}")
    cb = ws[pl.counter_offset:pl.counter_offset + pl.counter_bytes]
    assert int(cb.count_nonzero()) == 0


def test_in_kernel_combine_matches_two_launches(fmha, oracle):
    # fp8 short prefix (12 kv heads, one query tile): with one round of split
    # workgroups fmha_fwd combines inside the attention launch; the result
    # matches the partials launch + combine launch of the same plan and the
    # oracle, and the counter block is zero again afterwards
    prob = fs.fp8_prefix(11008)
    ref = run_oracle(oracle, prob)
    dev = upload(prob)
    for splits in (0, 4, 16):
        out, lse = alloc_outputs(prob, dev)
        args = _f8_args(fmha, dev, out, lse, splits)
        ws = torch.zeros(fmha.workspace_size(args), dtype=torch.uint8, device="cuda")
        args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
        pl = fmha.plan(args)
        assert pl.num_splits > 1 and pl.combine_in_kernel == 1 and pl.grid_combine == 0
        announce(f"in-kernel combine, fp8 prefix 11008, {pl.num_splits} splits")
        stream = torch.cuda.current_stream().cuda_stream
        assert fmha.lib.fmha_fwd(ctypes.byref(args), ctypes.c_void_p(stream)) == 0
        torch.cuda.synchronize()
        cb = ws[pl.counter_offset:pl.counter_offset + pl.counter_bytes]
        assert int(cb.count_nonzero()) == 0, "counter block not left zero"
        go, gl = to_packed(prob, out, lse)
        compare(prob, go, gl, *ref, what=f"in-kernel combine S={pl.num_splits}")
        # the same plan as two launches: partials, then the combine kernel
        o2, l2 = alloc_outputs(prob, dev)
        o_part, lse_part, pl2 = fmha.splitkv_partials(
            dev["q"], dev["k"], dev["v"], num_kv_splits=splits, q_descale=dev["q_descale"],
            k_descale=dev["k_descale"], v_descale=dev["v_descale"])
        assert pl2.combine_in_kernel == 0 and pl2.split_chunk == pl.split_chunk
        fmha.splitkv_combine(o_part, lse_part, split_chunk=pl2.split_chunk, out=o2, lse=l2,
                             seqlen_k=prob.lens_k[0])
        torch.cuda.synchronize()
        g2, gl2 = to_packed(prob, o2, l2)
        assert np.abs(go - g2).max() <= 2 ** -7 * max(1.0, np.abs(g2).max())
        assert np.abs(gl - gl2).max() <= 1e-5
    # graph replays: the counters return to zero after every launch, so each
    # replay gives the eager result bit for bit
    ref_o, ref_l = out.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            assert fmha.lib.fmha_fwd(ctypes.byref(args), ctypes.c_void_p(side.cuda_stream)) == 0
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        out.fill_(0)
        lse.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep}"
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), f"replay {rep}"
        _ = (dev["q"].float().sum() + 1).item()


def test_in_kernel_combine_with_dirty_counters_recovers(fmha, oracle):
    # a counter block that was not zeroed (an arrival count far past the
    # split count) makes the tile's workgroups write NaN at once instead of
    # waiting; the call still leaves the block zero, and the next call is right
    prob = fs.fp8_prefix(11008)
    dev = upload(prob)
    out, lse = alloc_outputs(prob, dev)
    args = _f8_args(fmha, dev, out, lse, 8)
    ws = torch.zeros(fmha.workspace_size(args), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    pl = fmha.plan(args)
    assert pl.combine_in_kernel == 1
    counters = ws[pl.counter_offset:pl.counter_offset + pl.counter_bytes].view(torch.int32)
    counters[0] = 1000  # arrival counter of (sequence 0, kv head 0, tile 0)
    stream = torch.cuda.current_stream().cuda_stream
    announce("in-kernel combine with a dirty counter block")
    assert fmha.lib.fmha_fwd(ctypes.byref(args), ctypes.c_void_p(stream)) == 0
    torch.cuda.synchronize()
    assert int(counters.count_nonzero()) == 0
    o = out.float()
    assert torch.isnan(o[0, :, 0]).all()          # head 0 of the one sequence: NaN
    assert not torch.isnan(o[0, :, 1:]).any()     # the other heads: combined normally
    assert fmha.lib.fmha_fwd(ctypes.byref(args), ctypes.c_void_p(stream)) == 0
    torch.cuda.synchronize()
    go, gl = to_packed(prob, out, lse)
    compare(prob, go, gl, *run_oracle(oracle, prob), what="after a dirty counter block")


@pytest.mark.parametrize("dtype,d,mask,batch", [("f16", 128, "causal", 130), ("bf16", 128, "sliding", 65),
                                                ("f16", 256, "causal", 80), ("bf16", 64, "left_window", 20)])
def test_persistent_table_order(fmha, oracle, dtype, d, mask, batch):
    # a persistent grid (one round of workgroups) taking tiles from the
    # device-sorted table, own XCD's list first: every row as the oracle
    rng = np.random.default_rng(300 + batch)
    choices = [0, 1, 31, 33, 95, 128, 129, 200, 257, 300, 511]
    lens_q = [int(x) for x in rng.choice(choices, size=batch)]
    lens_k = [int(x) for x in rng.choice(choices, size=batch)]
    lens_q[0], lens_k[0] = 511, 511
    prob = make_problem(f"persistent_{dtype}_{d}_{mask}", dtype=dtype, lens_q=lens_q,
                        lens_k=lens_k, hq=8, hkv=2, dqk=d, dv=d, seed=17, varlen_q=True,
                        varlen_k=True, causal=(mask == "causal"), window=WINDOWS[mask])
    dev = upload(prob)
    args = fmha.make_args(dev["q"], dev["k"], dev["v"], cu_seqlens_q=dev["cu_seqlens_q"],
                          cu_seqlens_k=dev["cu_seqlens_k"], max_seqlen_q=dev["max_seqlen_q"],
                          max_seqlen_k=dev["max_seqlen_k"], causal=prob.causal,
                          window=prob.window, num_kv_splits=1, persistent=True,
                          num_cus=fmha.device_num_cus())
    ws = torch.zeros(max(fmha.workspace_size(args), 256), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    pl = fmha.plan(args)
    assert pl.tile_order == 4 and pl.persistent == 1
    assert pl.grid_main == min(pl.sched_items, fmha.device_num_cus() * (1 if d == 256 else 3))
    ref = run_oracle(oracle, prob)
    for rep in range(2):
        announce(f"persistent table order {dtype} d={d} {mask} b={batch} rep {rep}")
        out, lse = run_gpu(fmha, prob, num_kv_splits=1, dev=dev, persistent=True)
        go, gl = to_packed(prob, out, lse)
        compare(prob, go, gl, *ref, what=f"persistent {mask} rep {rep}")
