"""Workload shapes for the sparse-KV decode step.

Each workload is one decode step of one attention layer over a paged KV cache:
score every historical block's landmark against the query, keep the top-k
blocks per KV head, attend them plus a dense recent window, and fuse the two
partial results by log-sum-exp.  The shapes follow the five synthetic
workloads this library is measured on (tiny fp32 reference, a Llama-3-8B-shaped
32k layer, a ragged batch, host-resident KV, and dual-query lookahead).

The pages that describe the method (PulseInfer, "SoloHead sparse selection" and
the gather-scatter I/O engine, section 2; DualDecoder, core claim and the
two-layer ping-pong buffer of Fig. 11; Beyond, abstract: dense recent window
plus per-head sparse attention fused by log-sum-exp) fix no shapes; the
numbers below are the workload definitions themselves.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Optional

DTYPES = ("fp32", "bf16", "fp8")
ELEM_BYTES = {"fp32": 4, "bf16": 2, "fp8": 1}


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    context: int                  # L for fixed-length batches; max L for ragged
    top_k: int                    # k (fixed), or 0 for the ragged rule
    window: int                   # W
    kv_dtype: str = "bf16"
    q_dtype: str = "bf16"
    landmark_dtype: str = "bf16"
    n_q_tokens: int = 1           # 2 = real + speculative token
    pool: str = "device"          # "device" (HBM pool) or "host" (pinned host pool)
    ragged_min: int = 0           # ragged: lengths uniform in [ragged_min, context]
    ragged_topk_frac: float = 0.0  # ragged: k_b = max(ragged_topk_min, floor(frac * nb_b))
    ragged_topk_min: int = 0
    occupancy: float = 1.0        # fraction of pool blocks in use
    shuffle_table: bool = True    # block table = seeded permutation (else identity)
    outlier_channels: int = 0     # key channels scaled x outlier_scale
    outlier_scale: float = 10.0
    salient_frac: float = 0.0     # host: fraction of blocks per head aligned with q
    salient_alpha: float = 2.0
    spec_noise: float = 0.0       # dual: speculative = real + N(0, spec_noise)
    n_layers: int = 1             # host: layer-steps sharing one pool (ping-pong)
    poison: bool = False          # NaN-fill free blocks and tail rows

    # ---- derived shapes -------------------------------------------------
    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_blocks(self) -> int:
        return -(-self.context // self.block_size)

    def scaled(self, **kw) -> "Workload":
        """A copy with some fields replaced (smaller parity cases)."""
        return dataclasses.replace(self, **kw)


TINY = Workload(
    name="tiny", seed=0, batch=1, n_q_heads=8, n_kv_heads=2, head_dim=64,
    block_size=16, context=4096, top_k=16, window=64,
    kv_dtype="fp32", q_dtype="fp32", landmark_dtype="fp32",
    shuffle_table=False)

LLAMA32K = Workload(
    name="llama32k", seed=1, batch=32, n_q_heads=32, n_kv_heads=8, head_dim=128,
    block_size=32, context=32768, top_k=64, window=512,
    outlier_channels=4, outlier_scale=10.0)

RAGGED = Workload(
    name="ragged", seed=2, batch=64, n_q_heads=32, n_kv_heads=8, head_dim=128,
    block_size=32, context=65536, top_k=0, window=256,
    ragged_min=4096, ragged_topk_frac=0.02, ragged_topk_min=8,
    occupancy=0.9, poison=True)

HOST = Workload(
    name="host", seed=3, batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128,
    block_size=64, context=131072, top_k=32, window=512,
    pool="host", shuffle_table=False, salient_frac=0.05, salient_alpha=2.0,
    n_layers=4)

DUAL = Workload(
    name="dual", seed=4, batch=4, n_q_heads=64, n_kv_heads=8, head_dim=128,
    block_size=64, context=262144, top_k=128, window=1024,
    kv_dtype="fp8", n_q_tokens=2, spec_noise=0.3)

WORKLOADS = {w.name: w for w in (TINY, LLAMA32K, RAGGED, HOST, DUAL)}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def n_candidates(L: int, window: int, blk: int) -> int:
    """Blocks holding at least one position before the recent window."""
    ws = max(0, L - window)
    return -(-ws // blk)


def algorithmic_bytes(wl: Workload, seq_lens, k_per_seq) -> int:
    """Bytes the decode step must move: landmarks of every candidate block,
    the selected K/V blocks (plus fp8 scales), the window's K/V, the queries
    and the fp32 output and lse.  Scratch and split partials are excluded."""
    d, blk = wl.head_dim, wl.block_size
    e_kv = ELEM_BYTES[wl.kv_dtype]
    e_l = ELEM_BYTES[wl.landmark_dtype]
    e_q = ELEM_BYTES[wl.q_dtype]
    e_scale = 8 if wl.kv_dtype == "fp8" else 0
    total = 0
    for L, k in zip(seq_lens, k_per_seq):
        L = int(L)
        k = int(k)
        nc = n_candidates(L, wl.window, blk)
        nsel = min(k, nc)
        per_head = nc * d * e_l + nsel * (2 * blk * d * e_kv + e_scale) \
            + min(wl.window, L) * 2 * d * e_kv
        total += wl.n_kv_heads * per_head
    total += wl.batch * wl.n_q_tokens * wl.n_q_heads * d * e_q
    total += wl.batch * wl.n_q_heads * (d + 1) * 4
    return total


def host_link_bytes(wl: Workload, seq_lens, k_per_seq) -> int:
    """Bytes the host-resident path pulls over the host link per layer-step."""
    e_kv = ELEM_BYTES[wl.kv_dtype]
    total = 0
    for L, k in zip(seq_lens, k_per_seq):
        nc = n_candidates(int(L), wl.window, wl.block_size)
        total += wl.n_kv_heads * min(int(k), nc) * 2 * wl.block_size * wl.head_dim * e_kv
    return total


def ragged_top_k(wl: Workload, L: int) -> int:
    nb = -(-L // wl.block_size)
    return max(wl.ragged_topk_min, int(math.floor(wl.ragged_topk_frac * nb)))
