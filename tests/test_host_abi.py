"""CPU-only tests of the C ABI's host logic: the library loads, exports every
symbol include/fmha.h declares, and validates / resolves arguments (default
scale, windows, split count, workspace size, error codes) without a GPU.
No compute call is made here.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import numpy as np
import pytest

import split_kv_flash_fmha_amd as fmha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x7F0000000000  # 16-byte aligned stand-in device address (never dereferenced)


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fmha.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fmha_\w+)\s*\(", src, re.M)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 8, names
    for n in names:
        assert hasattr(fmha.lib, n), f"{n} declared in include/fmha.h but not exported"


def test_check_seqlens_argument_errors():
    # rejected on the host before any launch (no GPU needed)
    f = fmha.lib.fmha_check_seqlens
    assert f(None, 2, 10, 10, FAKE, None) == INVALID
    assert f(FAKE, 2, 10, 10, None, None) == INVALID
    for batch, total, mx in ((-1, 0, 0), (1, -1, 0), (1, 0, -1)):
        assert f(FAKE, batch, total, mx, FAKE, None) == INVALID


def make(*, dtype=2, out_dtype=None, batch=1, sq=1, sk=1024, hq=4, hkv=4, dqk=64, dv=64,
         varlen_q=False, varlen_k=False, max_q=None, max_k=None, total_q=None, total_k=None,
         scale=0.0, causal=False, window=(-1, -1), splits=1, num_cus=256, lse=True,
         workspace=None, workspace_bytes=0):
    a = fmha.FwdArgs()
    a.q = a.k = a.v = a.out = FAKE
    a.lse = FAKE if lse else None
    a.batch = batch
    if varlen_q:
        a.cu_seqlens_q = FAKE
        a.total_q = total_q if total_q is not None else batch * sq
        a.max_seqlen_q = max_q if max_q is not None else sq
    else:
        a.seqlen_q = sq
    if varlen_k:
        a.cu_seqlens_k = FAKE
        a.total_k = total_k if total_k is not None else batch * sk
        a.max_seqlen_k = max_k if max_k is not None else sk
    else:
        a.seqlen_k = sk
    a.num_heads_q, a.num_heads_kv, a.head_dim_qk, a.head_dim_v = hq, hkv, dqk, dv
    a.q_stride_head, a.q_stride_tok, a.q_stride_batch = dqk, hq * dqk, sq * hq * dqk
    a.k_stride_head, a.k_stride_tok, a.k_stride_batch = dqk, hkv * dqk, sk * hkv * dqk
    a.v_stride_head, a.v_stride_tok, a.v_stride_batch = dv, hkv * dv, sk * hkv * dv
    a.o_stride_head, a.o_stride_tok, a.o_stride_batch = dv, hq * dv, sq * hq * dv
    a.lse_stride_head, a.lse_stride_batch = sq, hq * sq
    a.in_dtype = dtype
    a.out_dtype = out_dtype if out_dtype is not None else (2 if dtype == 3 else dtype)
    a.softmax_scale = scale
    a.causal = int(causal)
    a.window_left, a.window_right = window
    a.num_kv_splits = splits
    a.num_cus = num_cus
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace, workspace_bytes
    return a


def check(a):
    p = fmha.Plan()
    st = fmha.lib.fmha_fwd_check(ctypes.byref(a), ctypes.byref(p))
    return st, p


# ---- default softmax scale (pinned for non-square shapes) ---------------------

@pytest.mark.parametrize("varlen,sq,d", [(True, 129, 64), (False, 700, 64), (True, 129, 128),
                                         (False, 129, 128)])
def test_default_scale_uses_head_dim(varlen, sq, d):
    a = make(varlen_q=varlen, sq=sq, dqk=d, dv=d, sk=sq, varlen_k=varlen, splits=1)
    st, p = check(a)
    assert st == OK
    assert p.softmax_scale == np.float32(1.0 / math.sqrt(d))
    assert p.softmax_scale != np.float32(1.0 / math.sqrt(sq))


def test_explicit_scale_passes_through():
    st, p = check(make(scale=0.3))
    assert st == OK and p.softmax_scale == np.float32(0.3)


def test_fp8_default_scale_is_qk_head_dim():
    st, p = check(make(dtype=3, dqk=192, dv=128, sq=70, sk=16384, hq=12, hkv=12))
    assert st == OK and p.softmax_scale == np.float32(1 / math.sqrt(192))


# ---- masks --------------------------------------------------------------------

@pytest.mark.parametrize("window,causal,expect", [((-1, -1), True, (-1, 0)), ((128, 0), False, (128, 0)),
                                                  ((5, 7), True, (5, 0)), ((3, -1), False, (3, -1))])
def test_window_resolution(window, causal, expect):
    st, p = check(make(window=window, causal=causal, sq=64, sk=64))
    assert st == OK and (p.window_left, p.window_right) == expect


# ---- errors -------------------------------------------------------------------

@pytest.mark.parametrize("kw,code", [
    (dict(hq=6, hkv=4), INVALID),
    (dict(hq=0), INVALID),
    (dict(window=(-2, 0)), INVALID),
    (dict(window=(0, -5)), INVALID),
    (dict(scale=-0.5), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(splits=-1), INVALID),
    (dict(splits=257), INVALID),
    (dict(dtype=7), INVALID),
    (dict(dqk=48, dv=48), UNSUPPORTED),
    (dict(dqk=128, dv=64), UNSUPPORTED),
    (dict(dtype=2, out_dtype=1), UNSUPPORTED),
    (dict(dtype=3, out_dtype=3), INVALID),
    (dict(dtype=3, out_dtype=1, dqk=128, dv=128), UNSUPPORTED),
    (dict(varlen_q=True, max_q=10, total_q=5), INVALID),
    (dict(sq=-1), INVALID),
    (dict(splits=4), WORKSPACE),
])
def test_rejections(kw, code):
    st, _ = check(make(**kw))
    assert st == code, (kw, st)


def test_misaligned_pointer_and_stride():
    a = make()
    a.q = FAKE + 2
    assert check(a)[0] == INVALID
    a = make()
    a.k_stride_tok = 4 * 64 + 1  # not a multiple of 16 bytes
    assert check(a)[0] == INVALID


def test_null_pointers_rejected_unless_empty():
    a = make()
    a.q = None
    assert check(a)[0] == INVALID
    a = make(splits=1)
    a.out = None  # partials-only check: accepted only with a split
    assert check(a)[0] == OK
    assert fmha.lib.fmha_fwd_splitkv_partials(ctypes.byref(a), None) == INVALID
    a = make(batch=0)
    a.out = a.q = a.k = a.v = None
    assert check(a)[0] == OK


def test_status_strings():
    for s in range(5):
        assert fmha.lib.fmha_status_str(s)
    assert b"unknown" in fmha.lib.fmha_status_str(99)


# ---- splits and workspace -------------------------------------------------------

def test_explicit_splits_and_workspace_size():
    a = make(sk=1024, splits=4, hq=4, hkv=4, dv=64)
    n = ctypes.c_int32()
    assert fmha.lib.fmha_num_splits(ctypes.byref(a), ctypes.byref(n)) == OK and n.value == 4
    sz = ctypes.c_size_t()
    assert fmha.lib.fmha_fwd_workspace_size(ctypes.byref(a), ctypes.byref(sz)) == OK
    tq, hq, dv, S = 1, 4, 64, 4
    al = lambda x: (x + 255) // 256 * 256
    # partials O, partials LSE, then a 128-byte line of arrival counters per
    # (sequence, kv head, query tile), each part 256-byte aligned
    assert sz.value == al(S * tq * hq * dv * 4) + al(S * hq * tq * 4) + al(1 * 4 * 1 * 128)
    a.workspace, a.workspace_bytes = FAKE, sz.value
    st, p = check(a)
    assert st == OK and p.num_splits == 4 and p.split_chunk * 4 >= 1024
    assert p.split_chunk % p.key_block == 0
    assert p.lse_part_offset >= S * tq * hq * dv * 4 and p.lse_part_offset % 256 == 0
    assert p.counter_offset == p.lse_part_offset + al(S * hq * tq * 4) and p.counter_bytes == 512
    assert p.combine_in_kernel == 0  # a decode-kernel plan: the separate combine
    a.workspace_bytes = sz.value - 1
    assert check(a)[0] == WORKSPACE
    a.workspace_bytes = sz.value
    a.workspace = FAKE + 16  # not 256-byte aligned
    assert check(a)[0] == WORKSPACE


def test_many_splits_beyond_key_blocks_are_honoured():
    a = make(sk=100, splits=64)
    n = ctypes.c_int32()
    assert fmha.lib.fmha_num_splits(ctypes.byref(a), ctypes.byref(n)) == OK
    assert n.value == 64


def test_auto_splits_long_decode_fills_device():
    a = make(sq=1, sk=131072, hq=32, hkv=32, dqk=128, dv=128, splits=0)
    n = ctypes.c_int32()
    assert fmha.lib.fmha_num_splits(ctypes.byref(a), ctypes.byref(n)) == OK
    assert 8 <= n.value <= 128
    # units x splits cover the device several times over
    assert n.value * 32 >= 2 * 256


def test_auto_splits_avoid_power_of_two_chunks():
    # a power-of-two number of 32-key blocks per split aligns every split's
    # stream (measured slower); the automatic count steps past such chunks
    for sk, hq in ((131072, 32), (65536, 32), (16384, 8)):
        st, p = check(make(sq=1, sk=sk, hq=hq, hkv=hq, dqk=128, dv=128, splits=0,
                           workspace=FAKE, workspace_bytes=1 << 40))
        assert st == OK and p.num_splits > 1
        nb = p.split_chunk // p.key_block
        assert not (nb >= 4 and nb & (nb - 1) == 0), (sk, p.num_splits, p.split_chunk)
    # long decode: 127 splits of 1056 keys instead of 128 of 1024
    st, p = check(make(sq=1, sk=131072, hq=32, hkv=32, dqk=128, dv=128, splits=0,
                       workspace=FAKE, workspace_bytes=1 << 40))
    assert (p.num_splits, p.split_chunk) == (127, 1056)


def test_auto_splits_decode_prefers_long_splits():
    # batched GQA decode (16 x 8 kv heads, keys ~ U[1024, 32768]): splits of
    # ~1024 keys while each CU still sees >= 8 workgroups -- 31 splits of 1056
    # keys (1024 is a power-of-two block count), not 60 of 544
    st, p = check(make(batch=16, sq=1, sk=32542, hq=32, hkv=8, dqk=128, dv=128, varlen_k=True,
                       total_k=266241, splits=0, workspace=FAKE, workspace_bytes=1 << 40))
    assert st == OK and (p.num_splits, p.split_chunk) == (31, 1056)
    # too little work for 8 per CU at 1024 keys: the chunk shrinks with it
    st, p = check(make(batch=1, sq=1, sk=65536, hq=8, hkv=8, dqk=128, dv=128, splits=0,
                       workspace=FAKE, workspace_bytes=1 << 40))
    assert st == OK and p.split_chunk < 1024 and p.num_splits * 8 >= 8 * 256 // 2
    # the same shape through the 16-row streaming kernel (fp32): 16 per CU
    st, p = check(make(dtype=0, batch=16, sq=1, sk=32542, hq=32, hkv=8, dqk=128, dv=128,
                       varlen_k=True, total_k=266241, splits=0, workspace=FAKE,
                       workspace_bytes=1 << 40))
    assert st == OK and p.split_chunk < 1024


def test_auto_splits_scale_with_cu_count():
    base = dict(sq=1, sk=131072, hq=32, hkv=32, dqk=128, dv=128)
    s = []
    for cus in (64, 256):
        a = make(num_cus=cus, splits=0, **base)
        n = ctypes.c_int32()
        fmha.lib.fmha_num_splits(ctypes.byref(a), ctypes.byref(n))
        s.append(n.value)
    assert s[0] < s[1]


def test_auto_splits_off_for_prefill():
    a = make(varlen_q=True, varlen_k=True, batch=8, sq=2048, sk=2048, hq=16, hkv=16, dqk=128,
             dv=128, dtype=1, max_q=4096, max_k=4096, total_q=16384, total_k=16384, splits=0)
    n = ctypes.c_int32()
    assert fmha.lib.fmha_num_splits(ctypes.byref(a), ctypes.byref(n)) == OK and n.value == 1


def test_auto_splits_short_prefix_fp8():
    # multi-row kernel: one round of workgroups, 12 (sequence, head) units
    for sk in (16384, 11008):
        a = make(dtype=3, sq=70, sk=sk, hq=12, hkv=12, dqk=192, dv=128, splits=0)
        n = ctypes.c_int32()
        assert fmha.lib.fmha_num_splits(ctypes.byref(a), ctypes.byref(n)) == OK
        assert 16 <= n.value and n.value * 12 <= 256


def test_gqa_rows_packed_into_one_tile():
    # 4 query heads per kv head, one query token: a single 16-row tile
    st, p = check(make(sq=1, sk=4096, hq=32, hkv=8, dqk=128, dv=128, splits=1))
    assert st == OK and p.num_q_tiles == 1 and p.rows_per_tile == 16
    assert p.grid_main == 8  # batch 1 x 8 kv heads x 1 tile x 1 split


def test_combine_rejections():
    c = fmha.CombineArgs()
    c.o_part = c.lse_part = c.out = FAKE
    c.batch, c.seqlen_q, c.seqlen_k = 1, 1, 64
    c.num_heads_q, c.head_dim_v, c.num_splits, c.split_chunk = 4, 64, 2, 32
    c.o_stride_head, c.o_stride_tok, c.o_stride_batch = 64, 256, 256
    c.out_dtype = 2
    c.num_splits = 0
    assert fmha.lib.fmha_splitkv_combine(ctypes.byref(c), None) == INVALID
    c.num_splits, c.split_chunk = 2, 0
    assert fmha.lib.fmha_splitkv_combine(ctypes.byref(c), None) == INVALID
    c.split_chunk, c.out_dtype = 32, 3
    assert fmha.lib.fmha_splitkv_combine(ctypes.byref(c), None) == INVALID


def test_tile_order_and_grid():
    # 32-row-tile prefill, one split, causal or a right-only window, <= 64
    # sequences: all tiles longest first, the grid bounded by the packed query
    # count
    lens = [4096, 512, 3072, 1024, 2560, 1536, 2048, 1536]
    for kw in (dict(causal=True), dict(window=(-1, 0)), dict(window=(-1, 300))):
        st, p = check(make(dtype=1, batch=8, sq=4096, sk=4096, hq=16, hkv=16, dqk=128,
                           dv=128, varlen_q=True, varlen_k=True, total_q=sum(lens),
                           total_k=sum(lens), splits=1, **kw))
        assert st == OK and p.tile_order == 1 and p.rows_per_tile == 128, kw
        # sum over sequences of ceil(len / 128) <= (16384 + 8 * 127) // 128 = 135 < 8 * 32
        assert p.grid_main == 16 * 135
    # fixed length: exact tile count
    st, p = check(make(dtype=1, batch=8, sq=2048, sk=2048, hq=16, hkv=16, dqk=128, dv=128,
                       causal=True, splits=1))
    assert st == OK and p.tile_order == 1 and p.grid_main == 16 * 8 * 16
    # no mask, a left window, more than 64 sequences, a split, or a decode
    # shape: grouped
    for kw in (dict(causal=False), dict(window=(128, 0)), dict(batch=65),
               dict(splits=2, workspace=FAKE, workspace_bytes=1 << 40)):
        args = dict(dtype=1, batch=8, sq=512, sk=512, hq=16, hkv=16, dqk=128, dv=128,
                    splits=1, causal=True)
        args.update(kw)
        st, p = check(make(**args))
        assert st == OK and p.tile_order == 0, kw
        assert p.grid_main == args["batch"] * 16 * p.num_q_tiles * p.num_splits
    st, p = check(make(dtype=1, batch=2, sq=1, sk=4096, hq=16, hkv=16, dqk=128, dv=128,
                       splits=1, causal=True))
    assert st == OK and p.tile_order == 0


def test_decode_split_order():
    # the decode kernel with more than one split and <= 64 sequences: full
    # splits first, then the partial ones (order 2); the grid keeps its
    # (sequence, kv head, split) size
    for dtype in (1, 2, 3):
        for batch in (1, 16, 64):
            st, p = check(make(dtype=dtype, batch=batch, sq=1, sk=20000, hq=32, hkv=8, dqk=128,
                               dv=128, varlen_k=True, total_k=max(20000, batch * 9000), splits=0,
                               workspace=FAKE, workspace_bytes=1 << 40))
            assert st == OK and p.num_splits > 1 and p.tile_order == 2, (dtype, batch)
            assert p.grid_main == batch * 8 * p.num_splits
    # 65 sequences, one split, or fp32 (no decode kernel): the plain order
    for kw in (dict(batch=65), dict(splits=1), dict(dtype=0)):
        args = dict(dtype=2, batch=16, sq=1, sk=20000, hq=32, hkv=8, dqk=128, dv=128,
                    varlen_k=True, splits=4, workspace=FAKE, workspace_bytes=1 << 40)
        args.update(kw)
        st, p = check(make(**args))
        assert st == OK and p.tile_order == 0, kw


def test_prefill_token_strides_that_would_wrap_are_unsupported():
    # the prefill kernels address the rows of one key block with 32-bit buffer
    # offsets: a token stride whose key-block span reaches 2^31 bytes is refused
    # up front (decode shapes use 64-bit addresses and are not limited)
    big = (1 << 31) // (32 * 2)  # elements: 32-key block x 2-byte rows reaches 2^31 bytes
    big -= big % 8
    a = make(dtype=1, batch=1, sq=256, sk=256, hq=4, hkv=4, dqk=128, dv=128, splits=1)
    st, p = check(a)
    assert st == OK and p.kernel_id % 1000 >= 200  # a prefill kernel
    a.k_stride_tok = big
    assert check(a)[0] == UNSUPPORTED
    a.k_stride_tok, a.v_stride_tok = 4 * 128, big
    assert check(a)[0] == UNSUPPORTED
    a.v_stride_tok = big // 2 - 4096  # half the span: fits
    assert check(a)[0] == OK
    d = make(dtype=2, batch=1, sq=1, sk=256, hq=4, hkv=4, dqk=128, dv=128, splits=1)
    d.k_stride_tok = d.v_stride_tok = big
    st, p = check(d)
    assert st == OK and 100 <= p.kernel_id % 1000 < 200  # the decode kernel


def test_combine_rejects_total_q_beyond_int32():
    c = fmha.CombineArgs()
    c.o_part = c.lse_part = c.out = FAKE
    c.batch, c.seqlen_q, c.seqlen_k = 1 << 16, 1 << 15, 64
    c.num_heads_q, c.head_dim_v, c.num_splits, c.split_chunk = 1, 64, 2, 32
    c.o_stride_head, c.o_stride_tok, c.o_stride_batch = 64, 64, 64 << 15
    c.out_dtype = 2
    assert fmha.lib.fmha_splitkv_combine(ctypes.byref(c), None) == INVALID


def test_check_seqlens_rejects_batch_near_int32_max():
    f = fmha.lib.fmha_check_seqlens
    assert f(FAKE, 2**31 - 1, 10, 10, FAKE, None) == INVALID
    assert f(FAKE, 2**31 - 256, 10, 10, FAKE, None) == INVALID


def test_binding_refuses_host_tensors():
    # every pointer the library receives is dereferenced on the GPU: the
    # binding refuses tensors that are not on one GPU before calling it
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="must be a tensor on"):
        fmha.make_args(q, k, k)
    cu = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError):
        fmha.check_seqlens(cu, 0, 0)


def test_heads_together_order_for_split_short_prefix():
    # one query tile per sequence and several splits (the fp8 short cached
    # prefix): the kv heads of one split go together (tile order 3); with
    # several query tiles the grouped order stays (0)
    st, p = check(make(dtype=3, batch=1, sq=70, sk=16384, hq=12, hkv=12, dqk=192, dv=128,
                       splits=0, workspace=FAKE, workspace_bytes=1 << 30))
    assert st == OK and p.num_splits > 1 and p.num_q_tiles == 1 and p.tile_order == 3
    st, p = check(make(dtype=1, batch=1, sq=600, sk=16384, hq=4, hkv=4, dqk=128, dv=128,
                       splits=4, workspace=FAKE, workspace_bytes=1 << 30))
    assert st == OK and p.num_q_tiles > 1 and p.tile_order == 0


def test_combine_in_kernel_only_for_resident_split_grids():
    # fp8 short prefix: 12 kv heads x S splits on one round of workgroups ->
    # with combine_mode 1 the combine runs inside the attention launch; not
    # by default, not when the grid exceeds the compute units, nor for a
    # partials-only check (out = NULL)
    kw = dict(dtype=3, batch=1, sq=70, sk=16384, hq=12, hkv=12, dqk=192, dv=128,
              workspace=FAKE, workspace_bytes=1 << 30)

    def fused(**k):
        a = make(**kw, **k)
        a.combine_mode = 1
        return a
    st, p = check(make(splits=16, num_cus=256, **kw))
    assert st == OK and p.combine_in_kernel == 0 and p.grid_combine > 0  # default: two launches
    st, p = check(fused(splits=16, num_cus=256))
    assert st == OK and p.grid_main == 192 and p.combine_in_kernel == 1 and p.grid_combine == 0
    st, p = check(fused(splits=16, num_cus=128))
    assert st == OK and p.combine_in_kernel == 0 and p.grid_combine > 0
    st, p = check(fused(splits=0, num_cus=256))
    assert st == OK and p.grid_main <= 256 and p.combine_in_kernel == 1
    a = fused(splits=16, num_cus=256)
    a.out = None
    st, p = check(a)
    assert st == OK and p.combine_in_kernel == 0
    a = fused(splits=16, num_cus=256)
    a.combine_mode = 2
    assert check(a)[0] == INVALID


def test_table_order_for_many_sequences_and_left_windows():
    # masked prefill beyond the in-kernel longest-first search (more than 64
    # sequences, or a left window) sorts its tiles on the device into a table
    # in the workspace (tile order 4); without a workspace the grouped order
    # stays (0)
    al = lambda x: (x + 255) // 256 * 256

    def plan(batch, causal, window, ws):
        a = make(dtype=1, batch=batch, sq=300, sk=300, hq=8, hkv=2, dqk=128, dv=128, varlen_q=True,
                 varlen_k=True, causal=causal, window=window, splits=1)
        if ws:
            a.workspace, a.workspace_bytes = FAKE, 1 << 30
        return check(a)
    st, p = plan(64, True, (-1, -1), True)
    assert st == OK and p.tile_order == 1 and p.workspace_bytes == 0
    st, p = plan(65, True, (-1, -1), True)
    tiles = 65 * 10  # ceil(300 * 4 / 128) = 10 tiles per sequence
    positions = 8 * ((2 * tiles + 7) // 8 + 10)  # 2 kv heads; + the longest sequence's tiles
    assert st == OK and p.tile_order == 4 and p.sched_items == positions
    assert p.grid_main == positions and p.workspace_bytes == al((16 + 2 * positions) * 4)
    st, p = plan(65, True, (-1, -1), False)
    assert st == OK and p.tile_order == 0
    st, p = plan(8, False, (128, 0), True)
    assert st == OK and p.tile_order == 4
    st, p = plan(8, False, (40, -1), True)
    assert st == OK and p.tile_order == 4
    st, p = plan(200, False, (-1, -1), True)
    assert st == OK and p.tile_order == 0  # no mask: grouped
    a = make(dtype=1, batch=65, sq=300, sk=300, hq=8, hkv=2, dqk=128, dv=128, varlen_q=True,
             varlen_k=True, causal=True, splits=1)
    sz = ctypes.c_size_t()
    assert fmha.lib.fmha_fwd_workspace_size(ctypes.byref(a), ctypes.byref(sz)) == OK
    assert sz.value == al((16 + 2 * positions) * 4)
    st, p = plan(1025, True, (-1, -1), True)
    assert st == OK and p.tile_order == 0  # beyond the schedule kernel's sequences
    a.workspace, a.workspace_bytes = FAKE, sz.value - 4
    assert check(a)[0] == WORKSPACE
    # a table entry packs the query tile in 20 bits: a sequence of 2^20 or more
    # 128-row tiles keeps the grouped order (a valid call, not an error)
    for max_q, order in ((((1 << 20) - 1) * 32, 4), ((1 << 20) * 32, 0)):
        a = make(dtype=1, batch=65, sq=300, sk=300, hq=8, hkv=2, dqk=128, dv=128, varlen_q=True,
                 varlen_k=True, causal=True, splits=1, max_q=max_q, total_q=max_q + 64 * 300)
        a.workspace, a.workspace_bytes = FAKE, 1 << 40
        st, p = check(a)
        assert st == OK and p.tile_order == order, (max_q, st, p.tile_order)


def test_persistent_table_order_grid():
    # persistent: one round of workgroups (two per CU; one at head dim 256)
    # takes the table's positions; only with the table order, not for fp8
    def plan(d, dtype=1, persistent=1, batch=130):
        a = make(dtype=dtype, batch=batch, sq=300, sk=300, hq=8, hkv=2, dqk=d, dv=128 if dtype == 3 else d,
                 varlen_q=True, varlen_k=True, causal=True, splits=1, num_cus=256)
        a.workspace, a.workspace_bytes = FAKE, 1 << 30
        a.persistent = persistent
        return check(a)
    st, p = plan(128)
    assert st == OK and p.tile_order == 4 and p.persistent == 1 and p.grid_main == 768
    st, p = plan(256)
    assert st == OK and p.persistent == 1 and p.grid_main == 256
    st, p = plan(128, persistent=0)
    assert st == OK and p.persistent == 0 and p.grid_main == p.sched_items
    st, p = plan(192, dtype=3)
    assert st == OK and p.tile_order == 4 and p.persistent == 0
    st, p = plan(128, batch=8)  # in-kernel longest-first order: not persistent
    assert st == OK and p.tile_order == 1 and p.persistent == 0
    a = make(dtype=1, batch=8, sq=300, sk=300, hq=8, hkv=2, dqk=128, dv=128, causal=True, splits=1)
    a.persistent = 2
    assert check(a)[0] == INVALID
