"""Inputs that move the prefill kernels' lazily kept softmax reference, and a
host model of when the kernels move it.

Test infrastructure only (used by tests/test_rescale_parity.py and
tests/test_rescale_model.py).

How the prefill kernels keep the running max (online softmax of flash
attention; "[Cute,Fwd,Sm100] Support q_stage=1 for inference", description:
running row max and sum): a wave owns 32 query rows of a row tile and walks the
tile's key range in blocks of BN keys.  The first block sets each row's
reference m (scores in log2 units) from its max; later blocks take
p = 2^(s - m) with no max and check afterwards whether, for some lane, the sum
of p over its half of the block exceeds a limit (lane half h holds the keys
whose in-block offset has bit 2 equal to h; limit 2^12 for f16/bf16, and 448
on the stored 8p, i.e. 56 on p, for fp8), or whether a row with keys in the
block still has no reference.  When either holds anywhere in the wave, every
row of the wave takes m' = max(m, block max), scales its O and l by
alpha = 2^(m - m') and recomputes the block's p.

With N(0, 1) inputs a later block almost never beats the first by 12 log2
units, so the rescale of a non-zero accumulator by alpha in (0, 1) is not
reached.  ``planted_problem`` writes, for the last row of every 32-row wave
group, keys at chosen heights above that row's first-block max: keys 2 log2
units below the limit in the next blocks (mass that does not move the
reference) and then one 2.5 above it (a move whose alpha multiplies that
mass), and, where the row has keys left, the same pattern again above the
moved reference.  A planted key is k_j = c * q_i with c chosen so that
scale * q_i . k_j hits the height; other rows see it as an ordinary key.

``simulate`` replays the kernels' decisions on the final (rounded) inputs in
fp64 and reports, per wave, how many times a row with a finite reference and
a non-zero sum had its reference moved up, and the largest share the old
mass (alpha * l) keeps after such a move.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import fmha_synth as fs

LOG2E = 1.0 / math.log(2.0)
ROWS_PER_WAVE = 32

# limit on a lane's half-block sum of p, in log2 units
LIMIT_LOG2 = {"f16": 12.0, "bf16": 12.0, "fp8_e4m3": math.log2(448.0 / 8.0)}
MID_BELOW = 2.0    # mid keys sit this far below the limit (no move)
JUMP_ABOVE = 2.5   # a jump key sits this far above it (a move)


def _rounded(x32: torch.Tensor, dtype: str) -> np.ndarray:
    """The values the kernels and the oracle see, as fp64 (dequantised)."""
    t, d = fs.cast(x32, dtype)
    return t.to(torch.float64).numpy() * d


class Geometry:
    """Row tiles, waves and key ranges of one prefill launch."""

    def __init__(self, lens_q, lens_k, hq, hkv, *, causal, window, rows_per_tile, key_block,
                 split_chunk=None):
        self.lens_q, self.lens_k = list(lens_q), list(lens_k)
        self.hq, self.hkv, self.G = hq, hkv, hq // hkv
        self.wl = window[0]
        self.wr = 0 if causal else window[1]
        self.rows_per_tile, self.bn = rows_per_tile, key_block
        self.chunk = split_chunk
        self.q_off = np.concatenate([[0], np.cumsum(self.lens_q)]).astype(int)
        self.k_off = np.concatenate([[0], np.cumsum(self.lens_k)]).astype(int)

    def splits(self, sk):
        if not self.chunk:
            return [(0, sk)]
        return [(kb, min(kb + self.chunk, sk)) for kb in range(0, sk, self.chunk)]

    def key_range(self, i, sq, sk, kb, ke):
        """Allowed keys [lo, hi] of query i within the split [kb, ke)."""
        shift = sk - sq
        lo = max(i + shift - self.wl, 0) if self.wl >= 0 else 0
        hi = min(i + shift + self.wr, sk - 1) if self.wr >= 0 else sk - 1
        return max(kb, lo), min(ke - 1, hi)

    def waves(self):
        """(b, hkv, split (kb, ke), tile rows [row0, row1), wave rows [w0, w1), j_begin, n_iter)."""
        for b, (sq, sk) in enumerate(zip(self.lens_q, self.lens_k)):
            rows = sq * self.G
            if rows == 0 or sk == 0:
                continue
            for kb, ke in self.splits(sk):
                for row0 in range(0, rows, self.rows_per_tile):
                    last = min(row0 + self.rows_per_tile, rows) - 1
                    t_lo = self.key_range(row0 // self.G, sq, sk, kb, ke)[0]
                    t_hi = self.key_range(last // self.G, sq, sk, kb, ke)[1]
                    j_begin = (t_lo // self.bn) * self.bn
                    n_iter = -(-(t_hi + 1 - j_begin) // self.bn) if t_hi + 1 > j_begin else 0
                    for hkv in range(self.hkv):
                        for w0 in range(row0, last + 1, ROWS_PER_WAVE):
                            w1 = min(w0 + ROWS_PER_WAVE, last + 1)
                            yield b, hkv, (kb, ke), (row0, last + 1), (w0, w1), j_begin, n_iter


def planted_problem(name, *, dtype, lens_q, lens_k, hq, hkv, dqk, dv, seed, causal=False,
                    window=(-1, -1), rows_per_tile=128, key_block=32, varlen=True):
    """make_problem with keys planted for the last row of every wave group.

    Returns (problem, planted) where planted maps (b, hkv, w0) -> the number
    of jump keys planted for that wave (0, 1 or 2).  The plan assumes one
    split (the key range of a tile is the whole sequence).
    """
    geo = Geometry(lens_q, lens_k, hq, hkv, causal=causal, window=window,
                   rows_per_tile=rows_per_tile, key_block=key_block)
    scale_log2 = LOG2E / math.sqrt(dqk)
    limit = LIMIT_LOG2[dtype]
    planted = {}
    rng = np.random.default_rng(seed + 1000)

    def shape(q32, k32, v32):
        qr = _rounded(q32, dtype)
        kr = _rounded(k32, dtype)
        used = set()
        for b, h, (kb, ke), (row0, row1), (w0, w1), j_begin, n_iter in geo.waves():
            sq, sk = geo.lens_q[b], geo.lens_k[b]
            r = w1 - 1
            i, hqi = r // geo.G, h * geo.G + r % geo.G
            lo, hi = geo.key_range(i, sq, sk, kb, ke)
            if lo > hi:
                continue
            qi = qr[geo.q_off[b] + i, hqi]
            n0, nlast = lo // geo.bn, hi // geo.bn
            blk0 = np.arange(max(lo, n0 * geo.bn), min(hi, n0 * geo.bn + geo.bn - 1) + 1)
            s0 = scale_log2 * (kr[geo.k_off[b] + blk0, h] @ qi)
            m = float(s0.max())
            later = nlast - n0
            if later >= 3:
                plan = [(1, -MID_BELOW), (2, -MID_BELOW), (3, JUMP_ABOVE)]
                if later >= 6:
                    plan += [(4, -MID_BELOW), (5, -MID_BELOW), (6, JUMP_ABOVE)]
            elif later == 2:
                plan = [(1, -MID_BELOW), (2, JUMP_ABOVE)]
            elif later == 1:
                plan = [(1, JUMP_ABOVE)]
            else:
                plan = []
            jumps = 0
            qq = float(qi @ qi)
            for dn, off in plan:
                n = n0 + dn
                cand = [j for j in range(max(lo, n * geo.bn), min(hi, n * geo.bn + geo.bn - 1) + 1)
                        if (b, h, j) not in used]
                if not cand or qq <= 0:
                    break
                j = int(rng.choice(cand))
                used.add((b, h, j))
                height = m + limit + off
                c = height / (scale_log2 * qq)
                k32[geo.k_off[b] + j, h] = torch.from_numpy(c * qi).to(torch.float32)
                kr[geo.k_off[b] + j, h] = c * qi
                if off > 0:
                    jumps += 1
                    m = height
            planted[(b, h, w0)] = jumps

    prob = fs.make_problem(name, dtype=dtype, lens_q=lens_q, lens_k=lens_k, hq=hq, hkv=hkv,
                           dqk=dqk, dv=dv, seed=seed, varlen_q=varlen, varlen_k=varlen,
                           causal=causal, window=window, shape_draws=shape)
    return prob, planted


def simulate(prob, *, rows_per_tile, key_block, split_chunk=None):
    """Replay the prefill kernels' reference decisions on prob's inputs.

    Returns {(b, hkv, kb, w0): (moves, best_old_share)}: moves counts rows
    (over the wave's blocks) whose finite reference moved up while their sum
    was non-zero; best_old_share is the largest alpha*l / (alpha*l + block
    sum) after such a move (0 if none).
    """
    geo = Geometry(prob.lens_q, prob.lens_k, prob.hq, prob.hkv, causal=prob.causal,
                   window=prob.window, rows_per_tile=rows_per_tile, key_block=key_block,
                   split_chunk=split_chunk)
    dt = prob.dtype
    qr = prob.q.to(torch.float64).numpy() * prob.q_descale
    kr = prob.k.to(torch.float64).numpy() * prob.k_descale
    scale_log2 = LOG2E / math.sqrt(prob.dqk)
    pscale, limit = (8.0, 448.0) if dt == "fp8_e4m3" else (1.0, 4096.0)
    half = (np.arange(geo.bn) >> 2) & 1
    out = {}
    for b, h, (kb, ke), _tile, (w0, w1), j_begin, n_iter in geo.waves():
        sq, sk = geo.lens_q[b], geo.lens_k[b]
        rows = np.arange(w0, w1)
        iq = rows // geo.G
        hqs = h * geo.G + rows % geo.G
        rng_ = np.array([geo.key_range(int(i), sq, sk, kb, ke) for i in iq])
        my_lo, my_hi = rng_[:, 0], rng_[:, 1]
        keys = np.arange(j_begin, j_begin + n_iter * geo.bn)
        kk = np.clip(keys, 0, sk - 1)
        s = scale_log2 * np.einsum("rd,kd->rk", qr[geo.q_off[b] + iq, hqs],
                                   kr[geo.k_off[b] + kk, h])
        allowed = (keys[None, :] >= my_lo[:, None]) & (keys[None, :] <= my_hi[:, None])
        s = np.where(allowed, s, -np.inf)
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        moves, best = 0, 0.0
        for it in range(n_iter):
            j0 = j_begin + it * geo.bn
            blk = s[:, it * geo.bn:(it + 1) * geo.bn]
            bmax = blk.max(axis=1)
            if it == 0:
                m = bmax.copy()

            def exps(ref):
                base = np.where(np.isneginf(ref), 0.0, ref)
                return np.exp2(blk - base[:, None])

            p = exps(m)
            rs = np.stack([p[:, half == 0].sum(1), p[:, half == 1].sum(1)]) * pscale
            has_keys = (my_lo <= j0 + geo.bn - 1) & (my_hi >= j0) & (my_lo <= my_hi)
            if (rs > limit).any() or (np.isneginf(m) & has_keys).any():
                m_new = np.maximum(m, bmax)
                base = np.where(np.isneginf(m_new), 0.0, m_new)
                alpha = np.exp2(m - base)
                moved = np.isfinite(m) & (m_new > m) & (l > 0)
                p = exps(m_new)
                if moved.any():
                    moves += int(moved.sum())
                    old = alpha * l
                    share = old / (old + p.sum(1))
                    best = max(best, float(share[moved].max()))
                l = l * alpha
                m = m_new
            l = l + p.sum(1)
        out[(b, h, kb, w0)] = (moves, best)
    return out
