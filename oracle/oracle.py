"""Python handle on the plain fp64 CPU attention reference (fmha_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It does not import the
HIP package and the HIP package does not import it.

The C file holds the arithmetic; this module only compiles it with gcc and
marshals numpy arrays.  Inputs are raw element bits in their storage dtype
(``float32``, ``uint16`` for fp16/bf16, ``uint8`` for fp8 e4m3fn), contiguous
in the packed layouts q [Tq, Hq, Dqk], k [Tk, Hkv, Dqk], v [Tk, Hkv, Dv].
Outputs are fp64: out [Tq, Hq, Dv] and lse [Hq, Tq].  Rows of a sequence with
no keys are left as the caller's ``fill`` value (NaN by default), so a test can
check that they stay untouched.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fmha_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8_e4m3": 3}

_lock = threading.Lock()
_lib = None


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile the oracle into a shared library with gcc (plain C, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    c_void_p, c_int, c_double = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    lib.oracle_attention.restype = c_int
    lib.oracle_attention.argtypes = [
        c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_int, c_int,
        c_int, c_int, c_int, c_int, c_int, c_double, c_double, c_double,
        c_double, c_int, c_int, c_int, c_void_p, c_void_p]
    lib.oracle_split_attention.restype = c_int
    lib.oracle_split_attention.argtypes = [
        c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_int, c_int,
        c_int, c_int, c_int, c_int, c_int, c_double, c_double, c_double,
        c_double, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p]
    lib.oracle_combine.restype = c_int
    lib.oracle_combine.argtypes = [
        c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p, c_int, c_int,
        c_int, c_int, c_int, c_void_p, c_void_p]
    lib.oracle_attention_rows.restype = c_int
    lib.oracle_attention_rows.argtypes = [
        c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_int, c_int,
        c_int, c_int, c_int, c_int, c_int, c_double, c_double, c_double,
        c_double, c_int, c_int, c_int, c_void_p, c_void_p, c_int, c_void_p,
        c_void_p]
    lib.oracle_decode.restype = None
    lib.oracle_decode.argtypes = [c_void_p, c_int, ctypes.c_int64, c_void_p]
    lib.oracle_num_threads.restype = c_int
    lib.oracle_set_num_threads.argtypes = [c_int]
    return lib


def load(path: str | None = None):
    """Load (building first if needed) the oracle library.

    With ``path`` given, load that file (used to load planted-mistake builds in
    the pin tests); otherwise the default in-tree build.
    """
    global _lib
    if path is not None:
        return Oracle(_bind(ctypes.CDLL(path)))
    with _lock:
        if _lib is None:
            if (not os.path.exists(LIB)
                    or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
                build()
            _lib = Oracle(_bind(ctypes.CDLL(LIB)))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _cu(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class Oracle:
    """Thin marshalling wrapper; every number is computed by the C library."""

    def __init__(self, lib):
        self.lib = lib

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))

    def decode(self, raw: np.ndarray, dtype: str) -> np.ndarray:
        raw = np.ascontiguousarray(raw)
        out = np.empty(raw.size, dtype=np.float64)
        self.lib.oracle_decode(_ptr(raw), DTYPE_CODE[dtype], raw.size, _ptr(out))
        return out.reshape(raw.shape)

    @staticmethod
    def _geometry(q, k, v, cu_q, cu_k, batch, seqlen_q, seqlen_k):
        tq, hq, dqk = q.shape
        tk, hkv, _ = k.shape
        dv = v.shape[2]
        if cu_q is not None:
            batch = len(cu_q) - 1
        elif cu_k is not None:
            batch = len(cu_k) - 1
        if cu_q is None:
            seqlen_q = tq // batch if batch else 0
        if cu_k is None:
            seqlen_k = tk // batch if batch else 0
        return tq, hq, dqk, hkv, dv, batch, seqlen_q, seqlen_k

    def attention(self, q, k, v, dtype, *, cu_q=None, cu_k=None, batch=1,
                  scale, q_descale=1.0, k_descale=1.0, v_descale=1.0,
                  causal=False, window=(-1, -1), fill=np.nan):
        """Full forward.  Returns (out [Tq,Hq,Dv], lse [Hq,Tq]) in fp64."""
        q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
        cu_q, cu_k = _cu(cu_q), _cu(cu_k)
        tq, hq, dqk, hkv, dv, batch, sq, sk = self._geometry(
            q, k, v, cu_q, cu_k, batch, 0, 0)
        out = np.full((tq, hq, dv), fill, dtype=np.float64)
        lse = np.full((hq, tq), fill, dtype=np.float64)
        rc = self.lib.oracle_attention(
            _ptr(q), _ptr(k), _ptr(v), DTYPE_CODE[dtype], _ptr(cu_q), _ptr(cu_k),
            batch, sq, sk, hq, hkv, dqk, dv, float(scale), float(q_descale),
            float(k_descale), float(v_descale), int(bool(causal)),
            int(window[0]), int(window[1]), _ptr(out), _ptr(lse))
        if rc != 0:
            raise ValueError(f"oracle_attention rejected its arguments ({rc})")
        return out, lse

    def attention_rows(self, q, k, v, dtype, rows_t, rows_h, *, cu_q=None,
                       cu_k=None, batch=1, scale, q_descale=1.0, k_descale=1.0,
                       v_descale=1.0, causal=False, window=(-1, -1), fill=np.nan):
        """Selected rows (token rows_t[n], head rows_h[n]) -> (out [n,Dv], lse [n])."""
        q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
        cu_q, cu_k = _cu(cu_q), _cu(cu_k)
        tq, hq, dqk, hkv, dv, batch, sq, sk = self._geometry(
            q, k, v, cu_q, cu_k, batch, 0, 0)
        rt = np.ascontiguousarray(np.asarray(rows_t, dtype=np.int32))
        rh = np.ascontiguousarray(np.asarray(rows_h, dtype=np.int32))
        n = len(rt)
        out = np.full((n, dv), fill, dtype=np.float64)
        lse = np.full((n,), fill, dtype=np.float64)
        rc = self.lib.oracle_attention_rows(
            _ptr(q), _ptr(k), _ptr(v), DTYPE_CODE[dtype], _ptr(cu_q), _ptr(cu_k),
            batch, sq, sk, hq, hkv, dqk, dv, float(scale), float(q_descale),
            float(k_descale), float(v_descale), int(bool(causal)),
            int(window[0]), int(window[1]), _ptr(rt), _ptr(rh), n, _ptr(out),
            _ptr(lse))
        if rc != 0:
            raise ValueError(f"oracle_attention_rows rejected its arguments ({rc})")
        return out, lse

    def split_attention(self, q, k, v, dtype, *, chunk, split, cu_q=None,
                        cu_k=None, batch=1, scale, q_descale=1.0, k_descale=1.0,
                        v_descale=1.0, causal=False, window=(-1, -1),
                        fill=np.nan):
        """Partial (out, lse) of keys [split*chunk, (split+1)*chunk) per sequence."""
        q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
        cu_q, cu_k = _cu(cu_q), _cu(cu_k)
        tq, hq, dqk, hkv, dv, batch, sq, sk = self._geometry(
            q, k, v, cu_q, cu_k, batch, 0, 0)
        out = np.full((tq, hq, dv), fill, dtype=np.float64)
        lse = np.full((hq, tq), fill, dtype=np.float64)
        rc = self.lib.oracle_split_attention(
            _ptr(q), _ptr(k), _ptr(v), DTYPE_CODE[dtype], _ptr(cu_q), _ptr(cu_k),
            batch, sq, sk, hq, hkv, dqk, dv, float(scale), float(q_descale),
            float(k_descale), float(v_descale), int(bool(causal)),
            int(window[0]), int(window[1]), int(chunk), int(split), _ptr(out),
            _ptr(lse))
        if rc != 0:
            raise ValueError(f"oracle_split_attention rejected its arguments ({rc})")
        return out, lse

    def combine(self, o_part, lse_part, *, chunk, cu_q=None, cu_k=None,
                batch=1, seqlen_q=0, seqlen_k=0, fill=np.nan):
        """Combine partials o_part [S,Tq,Hq,Dv], lse_part [S,Hq,Tq] (fp64)."""
        o_part = np.ascontiguousarray(o_part, dtype=np.float64)
        lse_part = np.ascontiguousarray(lse_part, dtype=np.float64)
        cu_q, cu_k = _cu(cu_q), _cu(cu_k)
        s, tq, hq, dv = o_part.shape
        if cu_q is not None:
            batch = len(cu_q) - 1
        elif cu_k is not None:
            batch = len(cu_k) - 1
        out = np.full((tq, hq, dv), fill, dtype=np.float64)
        lse = np.full((hq, tq), fill, dtype=np.float64)
        rc = self.lib.oracle_combine(
            _ptr(o_part), _ptr(lse_part), s, int(chunk), _ptr(cu_q), _ptr(cu_k),
            batch, int(seqlen_q), int(seqlen_k), hq, dv, _ptr(out), _ptr(lse))
        if rc != 0:
            raise ValueError(f"oracle_combine rejected its arguments ({rc})")
        return out, lse

    def split_then_combine(self, q, k, v, dtype, *, num_splits, chunk, **kw):
        """Partials of every split followed by the combine (for the invariant)."""
        parts = [self.split_attention(q, k, v, dtype, chunk=chunk, split=s, **kw)
                 for s in range(num_splits)]
        o_part = np.stack([p[0] for p in parts])
        lse_part = np.stack([p[1] for p in parts])
        ckw = {x: kw[x] for x in ("cu_q", "cu_k", "batch") if x in kw}
        tq = q.shape[0]
        tk = k.shape[0]
        b = ckw.get("batch", 1)
        if kw.get("cu_q") is not None:
            b = len(kw["cu_q"]) - 1
        elif kw.get("cu_k") is not None:
            b = len(kw["cu_k"]) - 1
        ckw["batch"] = b
        return self.combine(o_part, lse_part, chunk=chunk,
                            seqlen_q=tq // b if b else 0,
                            seqlen_k=tk // b if b else 0, **ckw)
