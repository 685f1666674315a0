"""Brute-force attention in 50-digit arithmetic, for pinning the CPU oracle.

Independent of the oracle's code: inputs are decoded by torch's own dtype
casts, the mask is an explicit predicate over every (query, key) pair, and the
softmax is materialised without subtracting a maximum:

    P_ij = exp(s_ij) / sum_{j' in A_i} exp(s_ij'),   O_i = sum_j P_ij v_j,
    LSE_i = ln sum_{j in A_i} exp(s_ij).

Only for tiny problems (pure-Python loops).
"""
from __future__ import annotations

import math

import mpmath
import numpy as np
import torch

mpmath.mp.dps = 50


def decode(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a tensor of any supported storage dtype."""
    return t.detach().cpu().to(torch.float64).numpy()


def attention(q, k, v, lens_q, lens_k, *, scale, qs=1.0, ks=1.0, vs=1.0,
              causal=False, window=(-1, -1)):
    """q [Tq,Hq,D], k [Tk,Hkv,D], v [Tk,Hkv,Dv] torch tensors (any dtype).

    Returns dict {(t, h): (O list of mpf, LSE mpf or -inf)} for every row of
    every sequence with at least one key; rows of sequences with no keys are
    absent (they must stay untouched).
    """
    qd, kd, vd = decode(q), decode(k), decode(v)
    hq, hkv = qd.shape[1], kd.shape[1]
    g = hq // hkv
    wl, wr = window
    res = {}
    q0 = k0 = 0
    for sq, sk in zip(lens_q, lens_k):
        for h in range(hq):
            hk = h // g
            for i in range(sq):
                if sk == 0:
                    continue
                d0 = i + sk - sq
                allowed = []
                for j in range(sk):
                    ok = True
                    if causal and j > d0:
                        ok = False
                    if wl >= 0 and j < d0 - wl:
                        ok = False
                    if wr >= 0 and j > d0 + wr:
                        ok = False
                    if ok:
                        allowed.append(j)
                dv = vd.shape[2]
                if not allowed:
                    res[(q0 + i, h)] = ([mpmath.mpf(0)] * dv, -math.inf)
                    continue
                s = []
                for j in allowed:
                    dot = mpmath.mpf(0)
                    for d in range(qd.shape[2]):
                        dot += mpmath.mpf(qd[q0 + i, h, d]) * mpmath.mpf(kd[k0 + j, hk, d])
                    s.append(mpmath.mpf(scale) * mpmath.mpf(qs) * mpmath.mpf(ks) * dot)
                e = [mpmath.exp(x) for x in s]
                z = mpmath.fsum(e)
                o = []
                for c in range(dv):
                    acc = mpmath.mpf(0)
                    for w, j in zip(e, allowed):
                        acc += w / z * mpmath.mpf(vs) * mpmath.mpf(vd[k0 + j, hk, c])
                    o.append(acc)
                res[(q0 + i, h)] = (o, mpmath.log(z))
        q0 += sq
        k0 += sk
    return res
