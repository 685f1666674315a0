"""Python binding of libfmha.so: attention forward with split-KV and varlen.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI (include/fmha.h); torch supplies device memory and
the current stream.  There is no fallback: if libfmha.so is missing the import
fails, and every non-zero status from the library raises ValueError.

Layouts (last dimension contiguous):
  fixed length : q [B, Sq, Hq, Dqk], k [B, Sk, Hkv, Dqk], v [B, Sk, Hkv, Dv],
                 out [B, Sq, Hq, Dv], lse [B, Hq, Sq] (fp32)
  varlen       : q [total_q, Hq, Dqk] with cu_seqlens_q int32 [B+1] (device),
                 likewise k / v with cu_seqlens_k; lse [Hq, total_q]
Q and K may be variable-length independently.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "fwd", "fwd_no_alloc", "splitkv_partials", "splitkv_combine", "plan", "num_splits",
    "workspace_size", "device_num_cus", "FwdArgs", "CombineArgs", "Plan",
    "lib", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfmha.so")

DTYPE_CODE = {
    torch.float32: 0,
    torch.float16: 1,
    torch.bfloat16: 2,
    torch.float8_e4m3fn: 3,
}
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "hip"}
NO_ALLOC_SCRATCH_BYTES = 32 << 20  # FMHA_NO_ALLOC_SCRATCH_BYTES

_i32, _i64, _f32, _vp, _sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_void_p, ctypes.c_size_t)


class FwdArgs(ctypes.Structure):
    _fields_ = [
        ("q", _vp), ("k", _vp), ("v", _vp), ("out", _vp), ("lse", _vp),
        ("cu_seqlens_q", _vp), ("cu_seqlens_k", _vp),
        ("batch", _i32), ("seqlen_q", _i32), ("seqlen_k", _i32),
        ("max_seqlen_q", _i32), ("max_seqlen_k", _i32),
        ("total_q", _i32), ("total_k", _i32),
        ("num_heads_q", _i32), ("num_heads_kv", _i32),
        ("head_dim_qk", _i32), ("head_dim_v", _i32),
        ("q_stride_batch", _i64), ("q_stride_tok", _i64), ("q_stride_head", _i64),
        ("k_stride_batch", _i64), ("k_stride_tok", _i64), ("k_stride_head", _i64),
        ("v_stride_batch", _i64), ("v_stride_tok", _i64), ("v_stride_head", _i64),
        ("o_stride_batch", _i64), ("o_stride_tok", _i64), ("o_stride_head", _i64),
        ("lse_stride_batch", _i64), ("lse_stride_head", _i64),
        ("in_dtype", _i32), ("out_dtype", _i32),
        ("q_descale", _vp), ("k_descale", _vp), ("v_descale", _vp),
        ("softmax_scale", _f32), ("causal", _i32),
        ("window_left", _i32), ("window_right", _i32),
        ("num_kv_splits", _i32),
        ("workspace", _vp), ("workspace_bytes", _sz),
        ("num_cus", _i32), ("combine_mode", _i32), ("persistent", _i32),
    ]


class Plan(ctypes.Structure):
    _fields_ = [
        ("softmax_scale", _f32), ("window_left", _i32), ("window_right", _i32),
        ("num_splits", _i32), ("split_chunk", _i32), ("rows_per_tile", _i32),
        ("num_q_tiles", _i32), ("key_block", _i32), ("kernel_id", _i32),
        ("grid_main", _i64), ("grid_combine", _i64),
        ("workspace_bytes", _sz), ("o_part_offset", _sz), ("lse_part_offset", _sz),
        ("counter_offset", _sz), ("counter_bytes", _sz), ("combine_in_kernel", _i32),
        ("sched_offset", _sz), ("sched_items", _i32), ("persistent", _i32),
        ("tile_order", _i32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class CombineArgs(ctypes.Structure):
    _fields_ = [
        ("o_part", _vp), ("lse_part", _vp), ("out", _vp), ("lse", _vp),
        ("cu_seqlens_q", _vp), ("cu_seqlens_k", _vp),
        ("batch", _i32), ("seqlen_q", _i32), ("seqlen_k", _i32),
        ("max_seqlen_q", _i32), ("total_q", _i32),
        ("num_heads_q", _i32), ("head_dim_v", _i32),
        ("num_splits", _i32), ("split_chunk", _i32),
        ("o_stride_batch", _i64), ("o_stride_tok", _i64), ("o_stride_head", _i64),
        ("lse_stride_batch", _i64), ("lse_stride_head", _i64),
        ("out_dtype", _i32),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first "
            "(python split_kv_flash_fmha_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.fmha_fwd_check.argtypes = [P(FwdArgs), P(Plan)]
    L.fmha_num_splits.argtypes = [P(FwdArgs), P(_i32)]
    L.fmha_fwd_workspace_size.argtypes = [P(FwdArgs), P(_sz)]
    L.fmha_fwd.argtypes = [P(FwdArgs), _vp]
    L.fmha_fwd_no_alloc.argtypes = [P(FwdArgs), _vp]
    L.fmha_fwd_splitkv_partials.argtypes = [P(FwdArgs), _vp]
    L.fmha_splitkv_combine.argtypes = [P(CombineArgs), _vp]
    L.fmha_status_str.argtypes = [ctypes.c_int]
    L.fmha_status_str.restype = ctypes.c_char_p
    L.fmha_device_num_cus.argtypes = [P(_i32)]
    L.fmha_check_seqlens.argtypes = [_vp, _i32, _i32, _i32, _vp, _vp]
    for f in ("fmha_fwd_check", "fmha_num_splits", "fmha_fwd_workspace_size",
              "fmha_fwd", "fmha_fwd_no_alloc", "fmha_fwd_splitkv_partials",
              "fmha_splitkv_combine",
              "fmha_device_num_cus", "fmha_check_seqlens"):
        getattr(L, f).restype = ctypes.c_int
    return L


lib = _load()


def _raise(status: int, what: str):
    if status != 0:
        msg = lib.fmha_status_str(status).decode()
        raise ValueError(f"{what}: {msg} (status {status})")


_NUM_CUS: dict = {}


def device_num_cus() -> int:
    """Compute units of the current HIP device (cached per device)."""
    dev = torch.cuda.current_device()
    if dev not in _NUM_CUS:
        n = _i32(0)
        _raise(lib.fmha_device_num_cus(ctypes.byref(n)), "fmha_device_num_cus")
        _NUM_CUS[dev] = int(n.value)
    return _NUM_CUS[dev]


def check_seqlens(cu_seqlens, total: int, max_seqlen: int) -> int:
    """fmha_check_seqlens: check a device cu_seqlens array (int32, batch + 1
    entries) against the varlen contract.  Returns 0 if it holds, else 1 + the
    first failing index.  Synchronises the current stream to read the result."""
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 device tensor")
    for name, val in (("total", total), ("max_seqlen", max_seqlen)):
        if not 0 <= int(val) < 2**31:
            raise ValueError(f"{name} must be in [0, 2**31), got {val}")
    cu = cu_seqlens.contiguous()
    res = torch.empty(1, dtype=torch.int32, device=cu.device)
    stream = torch.cuda.current_stream(cu.device).cuda_stream
    _raise(lib.fmha_check_seqlens(cu.data_ptr(), cu.numel() - 1, int(total), int(max_seqlen),
                                  res.data_ptr(), stream), "fmha_check_seqlens")
    return int(res.item())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check_tensor(name, t, ndim):
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")


def _check_device(name, t, device, dtype=None):
    """t must live on the GPU `device` (and have `dtype` when given): the
    library dereferences every pointer on the device."""
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a tensor on {device}, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _check_cu_seqlens(name, cu, device):
    _check_device(name, cu, device, torch.int32)
    if cu.dim() != 1 or cu.numel() < 1 or cu.stride(0) != 1:
        raise ValueError(f"{name} must be a contiguous 1-D int32 tensor of batch + 1 entries")


def _check_shape(name, t, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def make_args(q, k, v, *, out=None, lse=None, cu_seqlens_q=None, cu_seqlens_k=None,
              max_seqlen_q=None, max_seqlen_k=None, softmax_scale=0.0, causal=False,
              window=(-1, -1), num_kv_splits=0, q_descale=None, k_descale=None,
              v_descale=None, out_dtype=None, num_cus=None, workspace=None,
              combine_in_kernel=False, persistent=False):
    """Fill an FwdArgs from tensors (metadata only, nothing is launched).

    combine_in_kernel: combine split partials inside the attention launch
    where the plan allows it (combine_mode 1) instead of a second launch.
    persistent: with a device-sorted tile table (tile order 4), one round of
    workgroups takes the tiles from it instead of one workgroup per tile."""
    if q.dtype not in DTYPE_CODE:
        raise ValueError(f"unsupported input dtype {q.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_device(name, t, dev)
    vq, vk = cu_seqlens_q is not None, cu_seqlens_k is not None
    _check_tensor("q", q, 3 if vq else 4)
    _check_tensor("k", k, 3 if vk else 4)
    _check_tensor("v", v, 3 if vk else 4)
    if vq:
        _check_cu_seqlens("cu_seqlens_q", cu_seqlens_q, dev)
    if vk:
        _check_cu_seqlens("cu_seqlens_k", cu_seqlens_k, dev)
    expect_out = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    if out_dtype is not None and out_dtype != expect_out:
        raise ValueError(f"out_dtype must be {expect_out} for {q.dtype} inputs")
    if q.dtype == torch.float8_e4m3fn:
        for name, t in (("q_descale", q_descale), ("k_descale", k_descale),
                        ("v_descale", v_descale)):
            if t is not None:
                _check_device(name, t, dev, torch.float32)
                if t.numel() < 1:
                    raise ValueError(f"{name} must hold one fp32 value")
    if workspace is not None:
        _check_device("workspace", workspace, dev)
    a = FwdArgs()
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.out, a.lse = _ptr(out), _ptr(lse)
    if vq and vk:
        batch = cu_seqlens_q.numel() - 1
        if cu_seqlens_k.numel() - 1 != batch:
            raise ValueError("cu_seqlens_q and cu_seqlens_k disagree on the batch size")
    elif vq:
        batch = cu_seqlens_q.numel() - 1
        if k.shape[0] != batch:
            raise ValueError("fixed-length k batch differs from cu_seqlens_q")
    elif vk:
        batch = cu_seqlens_k.numel() - 1
        if q.shape[0] != batch:
            raise ValueError("fixed-length q batch differs from cu_seqlens_k")
    else:
        batch = q.shape[0]
        if k.shape[0] != batch or v.shape[0] != batch:
            raise ValueError("q, k, v batch sizes differ")
    a.batch = batch
    a.cu_seqlens_q = _ptr(cu_seqlens_q)
    a.cu_seqlens_k = _ptr(cu_seqlens_k)
    hq, dqk = q.shape[-2], q.shape[-1]
    hkv, dv = v.shape[-2], v.shape[-1]
    if k.shape[-2] != hkv or k.shape[-1] != dqk:
        raise ValueError("k shape does not match q / v")
    a.num_heads_q, a.num_heads_kv, a.head_dim_qk, a.head_dim_v = hq, hkv, dqk, dv
    if vq:
        a.total_q = q.shape[0]
        if max_seqlen_q is None:
            raise ValueError("max_seqlen_q is required with cu_seqlens_q")
        a.max_seqlen_q = int(max_seqlen_q)
        a.q_stride_tok, a.q_stride_head = q.stride(0), q.stride(1)
    else:
        a.seqlen_q = q.shape[1]
        a.q_stride_batch, a.q_stride_tok, a.q_stride_head = q.stride(0), q.stride(1), q.stride(2)
    if vk:
        a.total_k = k.shape[0]
        if max_seqlen_k is None:
            raise ValueError("max_seqlen_k is required with cu_seqlens_k")
        a.max_seqlen_k = int(max_seqlen_k)
        a.k_stride_tok, a.k_stride_head = k.stride(0), k.stride(1)
        a.v_stride_tok, a.v_stride_head = v.stride(0), v.stride(1)
        if v.shape[0] != k.shape[0]:
            raise ValueError("k and v token counts differ")
    else:
        a.seqlen_k = k.shape[1]
        if v.shape[1] != k.shape[1]:
            raise ValueError("k and v sequence lengths differ")
        a.k_stride_batch, a.k_stride_tok, a.k_stride_head = k.stride(0), k.stride(1), k.stride(2)
        a.v_stride_batch, a.v_stride_tok, a.v_stride_head = v.stride(0), v.stride(1), v.stride(2)
    if out is not None:
        _check_device("out", out, dev, expect_out)
        _check_tensor("out", out, q.dim())
        _check_shape("out", out, (*q.shape[:-1], dv))
        if vq:
            a.o_stride_tok, a.o_stride_head = out.stride(0), out.stride(1)
        else:
            a.o_stride_batch, a.o_stride_tok, a.o_stride_head = out.stride(0), out.stride(1), out.stride(2)
    if lse is not None:
        _check_device("lse", lse, dev, torch.float32)
        _check_shape("lse", lse, (hq, q.shape[0]) if vq else (q.shape[0], hq, q.shape[1]))
        if vq:
            a.lse_stride_head = lse.stride(0)
            if lse.stride(1) != 1:
                raise ValueError("lse token dimension must be contiguous")
        else:
            a.lse_stride_batch, a.lse_stride_head = lse.stride(0), lse.stride(1)
            if lse.stride(2) != 1:
                raise ValueError("lse token dimension must be contiguous")
    a.in_dtype = DTYPE_CODE[q.dtype]
    a.out_dtype = DTYPE_CODE[expect_out]
    a.q_descale, a.k_descale, a.v_descale = _ptr(q_descale), _ptr(k_descale), _ptr(v_descale)
    a.softmax_scale = float(softmax_scale or 0.0)
    a.causal = int(bool(causal))
    a.window_left, a.window_right = int(window[0]), int(window[1])
    a.num_kv_splits = int(num_kv_splits)
    a.num_cus = int(num_cus) if num_cus is not None else 0
    a.combine_mode = 1 if combine_in_kernel else 0
    a.persistent = 1 if persistent else 0
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return a


def plan(args: FwdArgs) -> Plan:
    """fmha_fwd_check: validate and resolve (host only)."""
    p = Plan()
    _raise(lib.fmha_fwd_check(ctypes.byref(args), ctypes.byref(p)), "fmha_fwd_check")
    return p


def num_splits(args: FwdArgs) -> int:
    n = _i32(0)
    _raise(lib.fmha_num_splits(ctypes.byref(args), ctypes.byref(n)), "fmha_num_splits")
    return int(n.value)


def workspace_size(args: FwdArgs) -> int:
    n = _sz(0)
    _raise(lib.fmha_fwd_workspace_size(ctypes.byref(args), ctypes.byref(n)),
           "fmha_fwd_workspace_size")
    return int(n.value)


def _alloc_outputs(q, v, vq, out_dtype, return_lse):
    dv = v.shape[-1]
    out = torch.empty((*q.shape[:-1], dv), dtype=out_dtype, device=q.device)
    lse = None
    if return_lse:
        if vq:
            lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
        else:
            lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32,
                              device=q.device)
    return out, lse


def _workspace(args, device):
    """A workspace for `args`, zeroed (its arrival-counter block must start at
    zero; every call leaves it zero, so a caller may reuse it)."""
    nbytes = workspace_size(args)
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def fwd(q, k, v, *, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
        max_seqlen_k=None, softmax_scale=0.0, causal=False, window=(-1, -1),
        num_kv_splits=0, q_descale=None, k_descale=None, v_descale=None,
        out=None, lse=None, return_lse=True, workspace=None, combine_in_kernel=False,
        persistent=False):
    """Attention forward.  Returns (out, lse); lse is None if return_lse=False.

    softmax_scale 0 means 1/sqrt(head_dim_qk); causal is bottom-right aligned;
    window=(left, right) with -1 unbounded; num_kv_splits 0 = automatic.
    FP8 (float8_e4m3fn) inputs take per-tensor fp32 device descales and give
    bf16 out.  Rows of a sequence with no keys are left as they were in
    ``out`` / ``lse`` (allocated uninitialised when not given).
    """
    out_dtype = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    vq = cu_seqlens_q is not None
    if out is None:
        o2, l2 = _alloc_outputs(q, v, vq, out_dtype, return_lse and lse is None)
        out = o2
        if lse is None:
            lse = l2
    kw = dict(out=out, lse=lse, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k,
              max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k,
              softmax_scale=softmax_scale, causal=causal, window=window,
              num_kv_splits=num_kv_splits, q_descale=q_descale, k_descale=k_descale,
              v_descale=v_descale, num_cus=device_num_cus(),
              combine_in_kernel=combine_in_kernel, persistent=persistent)
    args = make_args(q, k, v, **kw)
    if workspace is None:
        workspace = _workspace(args, q.device)
    if workspace is not None:
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel() * workspace.element_size()
    _raise(lib.fmha_fwd(ctypes.byref(args), _stream()), "fmha_fwd")
    return out, lse


def fwd_no_alloc(q, k, v, *, out, lse=None, cu_seqlens_q=None, cu_seqlens_k=None,
                 max_seqlen_q=None, max_seqlen_k=None, softmax_scale=0.0, causal=False,
                 window=(-1, -1), num_kv_splits=0, q_descale=None, k_descale=None,
                 v_descale=None, num_cus=None):
    """fmha_fwd_no_alloc: the forward with the split partials in the
    library's per-GPU scratch (nothing allocated, here or in the library).

    ``out`` (and ``lse`` if wanted) must be given.  Calls that overlap on one
    GPU share the scratch and must be ordered by the caller.
    """
    args = make_args(q, k, v, out=out, lse=lse, cu_seqlens_q=cu_seqlens_q,
                     cu_seqlens_k=cu_seqlens_k, max_seqlen_q=max_seqlen_q,
                     max_seqlen_k=max_seqlen_k, softmax_scale=softmax_scale, causal=causal,
                     window=window, num_kv_splits=num_kv_splits, q_descale=q_descale,
                     k_descale=k_descale, v_descale=v_descale,
                     num_cus=device_num_cus() if num_cus is None else num_cus)
    _raise(lib.fmha_fwd_no_alloc(ctypes.byref(args), _stream()), "fmha_fwd_no_alloc")
    return out, lse


def splitkv_partials(q, k, v, *, num_kv_splits, workspace=None, **kw):
    """Attention launch of a split forward only.

    Returns (o_part [S, total_q, Hq, Dv], lse_part [S, Hq, total_q], plan) as
    views into the fp32 workspace.
    """
    args = make_args(q, k, v, num_kv_splits=num_kv_splits, num_cus=device_num_cus(), **kw)
    nbytes = workspace_size(args)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    args.workspace = workspace.data_ptr()
    args.workspace_bytes = workspace.numel() * workspace.element_size()
    pl = plan(args)
    _raise(lib.fmha_fwd_splitkv_partials(ctypes.byref(args), _stream()),
           "fmha_fwd_splitkv_partials")
    S = pl.num_splits
    hq, dv = args.num_heads_q, args.head_dim_v
    tq = args.total_q if kw.get("cu_seqlens_q") is not None else args.batch * args.seqlen_q
    ws = workspace.view(torch.uint8)
    o_part = ws[pl.o_part_offset:pl.o_part_offset + S * tq * hq * dv * 4].view(
        torch.float32).view(S, tq, hq, dv)
    lse_part = ws[pl.lse_part_offset:pl.lse_part_offset + S * hq * tq * 4].view(
        torch.float32).view(S, hq, tq)
    return o_part, lse_part, pl


def splitkv_combine(o_part, lse_part, *, split_chunk, out, lse=None, cu_seqlens_q=None,
                    cu_seqlens_k=None, max_seqlen_q=None, seqlen_k=None):
    """LSE-weighted combine of fp32 partials into out (and lse).

    o_part [S, total_q, Hq, Dv], lse_part [S, Hq, total_q] (fp32, contiguous).
    out / lse follow the fixed-length or varlen layout of cu_seqlens_q.
    """
    dev = o_part.device
    _check_device("o_part", o_part, dev, torch.float32)
    _check_device("lse_part", lse_part, dev, torch.float32)
    if o_part.dim() != 4 or not o_part.is_contiguous() or not lse_part.is_contiguous():
        raise ValueError("partials must be contiguous fp32 [S, total_q, Hq, Dv] / [S, Hq, total_q]")
    S, tq, hq, dv = o_part.shape
    _check_shape("lse_part", lse_part, (S, hq, tq))
    if out.dtype not in (torch.float32, torch.float16, torch.bfloat16):
        raise ValueError(f"unsupported out dtype {out.dtype}")
    _check_device("out", out, dev)
    if out.stride(-1) != 1:
        raise ValueError("out: last dimension must be contiguous")
    vq = cu_seqlens_q is not None
    if vq:
        _check_cu_seqlens("cu_seqlens_q", cu_seqlens_q, dev)
        _check_shape("out", out, (tq, hq, dv))
        if lse is not None:
            _check_device("lse", lse, dev, torch.float32)
            _check_shape("lse", lse, (hq, tq))
    else:
        if out.dim() != 4 or out.shape[0] * out.shape[1] != tq:
            raise ValueError(f"out must be [B, Sq, Hq, Dv] with B * Sq = {tq}")
        _check_shape("out", out, (out.shape[0], out.shape[1], hq, dv))
        if lse is not None:
            _check_device("lse", lse, dev, torch.float32)
            _check_shape("lse", lse, (out.shape[0], hq, out.shape[1]))
    if cu_seqlens_k is not None:
        _check_cu_seqlens("cu_seqlens_k", cu_seqlens_k, dev)
    a = CombineArgs()
    a.o_part, a.lse_part, a.out, a.lse = _ptr(o_part), _ptr(lse_part), _ptr(out), _ptr(lse)
    a.cu_seqlens_q, a.cu_seqlens_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k)
    if vq:
        a.batch = cu_seqlens_q.numel() - 1
        a.max_seqlen_q = int(max_seqlen_q)
        a.total_q = tq
        a.o_stride_tok, a.o_stride_head = out.stride(0), out.stride(1)
        if lse is not None:
            a.lse_stride_head = lse.stride(0)
    else:
        a.batch = out.shape[0]
        a.seqlen_q = out.shape[1]
        a.o_stride_batch, a.o_stride_tok, a.o_stride_head = out.stride(0), out.stride(1), out.stride(2)
        if lse is not None:
            a.lse_stride_batch, a.lse_stride_head = lse.stride(0), lse.stride(1)
    if cu_seqlens_k is not None:
        if cu_seqlens_k.numel() - 1 != a.batch:
            raise ValueError("cu_seqlens_k batch differs")
    else:
        if seqlen_k is None:
            raise ValueError("seqlen_k is required without cu_seqlens_k")
        a.seqlen_k = int(seqlen_k)
    a.num_heads_q, a.head_dim_v = hq, dv
    a.num_splits, a.split_chunk = S, int(split_chunk)
    a.out_dtype = DTYPE_CODE[out.dtype]
    _raise(lib.fmha_splitkv_combine(ctypes.byref(a), _stream()), "fmha_splitkv_combine")
    return out, lse

