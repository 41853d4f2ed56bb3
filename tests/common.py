"""Glue between the seeded inputs, the CPU oracle and the HIP binding (tests only)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle as O
from sparse_kv_cache_block_amd.inputs import DecodeInputs, raw_bytes


def oracle_problem(inp: DecodeInputs, k_max: int | None = None) -> O.Problem:
    wl = inp.wl
    return O.problem(wl.batch, wl.n_q_tokens, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                     wl.block_size, wl.max_blocks, inp.n_pool_blocks, inp.pool_stride_block,
                     inp.pool_stride_head, wl.window, k_max if k_max is not None else inp.k_max,
                     wl.q_dtype, wl.kv_dtype, wl.landmark_dtype)


class HostArrays:
    """Host copies of one decode step's input bytes."""

    def __init__(self, inp: DecodeInputs):
        self.q = raw_bytes(inp.q)
        self.landmarks = raw_bytes(inp.landmarks)
        self.k_pool = raw_bytes(inp.k_pool)
        self.v_pool = raw_bytes(inp.v_pool)
        self.k_scales = raw_bytes(inp.k_scales)
        self.v_scales = raw_bytes(inp.v_scales)
        self.block_table = raw_bytes(inp.block_table)
        self.seq_lens = raw_bytes(inp.seq_lens)
        self.k_per_seq = raw_bytes(inp.k_per_seq)

    def pools(self):
        return self.k_pool, self.v_pool, self.k_scales, self.v_scales


def oracle_decode(inp: DecodeInputs, h: HostArrays | None = None) -> dict:
    h = h or HostArrays(inp)
    pr = oracle_problem(inp)
    return O.decode_step(pr, h.q, h.landmarks, h.k_pool, h.v_pool, h.k_scales, h.v_scales,
                         h.block_table, h.seq_lens, h.k_per_seq)


def exempt_set(oracle_row: np.ndarray, k: int, rel: float = 1e-5) -> set:
    """Candidates whose fp32 score lies within rel of the oracle's k-th score.

    oracle_row: fp64 scores of the candidates of one (b, t, g)."""
    if k == 0:
        return set()
    order = sorted(range(len(oracle_row)), key=lambda j: (-oracle_row[j], j))
    sk = np.float32(oracle_row[order[k - 1]])
    s32 = oracle_row.astype(np.float32)
    gap = np.abs(s32.astype(np.float64) - np.float64(sk))
    tol = rel * max(abs(float(sk)), 1e-30)
    return set(int(j) for j in np.nonzero(gap < tol)[0])


def check_indices(gpu_idx, gpu_nsel, orc_idx, orc_nsel, orc_scores, seq_lens, window, blk) -> int:
    """Compare GPU and oracle selections under the 1e-5 exemption rule.

    Returns the number of rows where an exempt swap was observed; raises on a
    real mismatch."""
    B, T, Hkv, kmax = orc_idx.shape
    swaps = 0
    for b in range(B):
        L = int(seq_lens[b])
        nc = -(-max(0, L - window) // blk)
        for t in range(T):
            for g in range(Hkv):
                n = int(orc_nsel[b, t, g])
                assert int(gpu_nsel[b, t, g]) == n, (b, t, g, int(gpu_nsel[b, t, g]), n)
                gi = [int(x) for x in gpu_idx[b, t, g]]
                oi = [int(x) for x in orc_idx[b, t, g]]
                assert gi[n:] == [-1] * (kmax - n), ("padding", b, t, g)
                assert gi[:n] == sorted(gi[:n]) and len(set(gi[:n])) == n, ("order", b, t, g)
                if gi == oi:
                    continue
                assert all(0 <= j < nc for j in gi[:n]), ("range", b, t, g)
                E = exempt_set(orc_scores[b, t, g, :nc], n)
                gs, os_ = set(gi[:n]) - E, set(oi[:n]) - E
                assert gs == os_, ("mismatch outside exemption", b, t, g, sorted(gs ^ os_))
                swaps += 1
    return swaps
