"""Seeded synthetic inputs for the sparse-KV decode step.

This module only draws and encodes data: queries, a paged K/V pool, block
tables, per-block landmarks (the mean of a block's stored keys, which a serving
system builds once when the block is filled and keeps resident on the GPU, as
DualDecoder's core claim describes), sequence lengths and per-sequence k.  It
contains none of the decode step's arithmetic (scoring, selection, gathering,
attention or the merge), and both the HIP path and the CPU oracle consume the
very same bytes it produces.

Random numbers come from torch generators on the device that will hold the
data, seeded from ``numpy.random.SeedSequence([workload.seed, instance])``
spawned into eight streams in a fixed order: q, K, V, block-table permutation,
outlier channels / lengths, salience, speculative noise, spare.  A given
(workload, instance, device type) always yields the same bytes.

Encodings:
  * bf16: round-to-nearest-even from fp32 (torch's cast).
  * fp8: OCP e4m3fn, one fp32 scale per (pool block, KV head) and tensor equal
    to amax/448 (1.0 for an all-zero chunk); values are divided by the scale,
    clamped to +-448 and rounded to nearest even (torch's cast).
  * NaN poison (free pool blocks, rows past a sequence's end): bf16 0x7FC0,
    fp8 0x7F, fp32 quiet NaN.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

from .configs import Workload, n_candidates, ragged_top_k

_TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}
FP8_MAX = 448.0

STREAM_Q, STREAM_K, STREAM_V, STREAM_TABLE, STREAM_SHAPE, STREAM_SALIENCE, STREAM_SPEC, STREAM_SPARE = range(8)


def _generators(wl: Workload, instance: int, device) -> list:
    states = np.random.SeedSequence([wl.seed, instance]).spawn(8)
    gens = []
    for s in states:
        g = torch.Generator(device=device)
        g.manual_seed(int(s.generate_state(1, np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF)))
        gens.append(g)
    return gens


@dataclass
class DecodeInputs:
    """One decode step's inputs; every tensor lives on ``device``."""
    wl: Workload
    q: torch.Tensor            # [B][T][Hq][d] q dtype
    landmarks: torch.Tensor    # [B][Hkv][max_blocks][d] landmark dtype
    k_pool: torch.Tensor       # pool layout (see pool_layout), kv dtype
    v_pool: torch.Tensor
    k_scales: Optional[torch.Tensor]   # [P][Hkv] fp32 (fp8 only)
    v_scales: Optional[torch.Tensor]
    block_table: torch.Tensor  # [B][max_blocks] int32 (unused entries 0)
    seq_lens: torch.Tensor     # [B] int32
    k_per_seq: torch.Tensor    # [B] int32
    n_pool_blocks: int
    pool_layout: str           # "block_major" [P][Hkv][blk][d] or "head_major" [Hkv][P][blk][d]
    window_k: Optional[torch.Tensor] = None   # [B][Hkv][W][d] (host pool only)
    window_v: Optional[torch.Tensor] = None
    window_k_scales: Optional[torch.Tensor] = None   # [B][Hkv][W] fp32 (host pool, fp8 only)
    window_v_scales: Optional[torch.Tensor] = None
    extras: dict = field(default_factory=dict)

    @property
    def pool_stride_block(self) -> int:
        wl = self.wl
        if self.pool_layout == "block_major":
            return wl.n_kv_heads * wl.block_size * wl.head_dim
        return wl.block_size * wl.head_dim

    @property
    def pool_stride_head(self) -> int:
        wl = self.wl
        if self.pool_layout == "block_major":
            return wl.block_size * wl.head_dim
        return self.n_pool_blocks * wl.block_size * wl.head_dim

    @property
    def k_max(self) -> int:
        return int(self.k_per_seq.max().item())

    def to(self, device) -> "DecodeInputs":
        def mv(t):
            return None if t is None else t.to(device)
        return DecodeInputs(
            wl=self.wl, q=mv(self.q), landmarks=mv(self.landmarks), k_pool=mv(self.k_pool),
            v_pool=mv(self.v_pool), k_scales=mv(self.k_scales), v_scales=mv(self.v_scales),
            block_table=mv(self.block_table), seq_lens=mv(self.seq_lens),
            k_per_seq=mv(self.k_per_seq), n_pool_blocks=self.n_pool_blocks,
            pool_layout=self.pool_layout, window_k=mv(self.window_k), window_v=mv(self.window_v),
            window_k_scales=mv(self.window_k_scales), window_v_scales=mv(self.window_v_scales),
            extras=dict(self.extras))


def _quantize_fp8(x: torch.Tensor):
    """x: [..., blk, d] fp32 chunks -> (codes e4m3fn, scale fp32 per chunk)."""
    amax = x.abs().amax(dim=(-2, -1))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    y = (x / scale[..., None, None]).clamp_(-FP8_MAX, FP8_MAX)
    return y.to(torch.float8_e4m3fn), scale.to(torch.float32)


def _encode(x: torch.Tensor, dtype: str):
    if dtype == "fp8":
        return _quantize_fp8(x)
    return x.to(_TORCH_DTYPE[dtype]), None


def _decode64(codes: torch.Tensor, scales: Optional[torch.Tensor]) -> torch.Tensor:
    """Stored values as fp64 (used only to build landmarks)."""
    x = codes.to(torch.float64)
    if scales is not None:
        x = x * scales.to(torch.float64)[..., None, None]
    return x


def make_inputs(wl: Workload, device="cpu", instance: int = 0,
                seq_lens: Optional[list] = None) -> DecodeInputs:
    """Draw one decode step's inputs for ``wl`` on ``device``.

    ``seq_lens`` overrides the drawn lengths (edge-case tests)."""
    device = torch.device(device)
    g = _generators(wl, instance, device)
    B, T, Hq, Hkv, d, blk = wl.batch, wl.n_q_tokens, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.block_size
    G = Hq // Hkv
    max_blocks = wl.max_blocks

    # ---- lengths and k --------------------------------------------------
    if seq_lens is not None:
        lens = torch.tensor(seq_lens, dtype=torch.int64)
        assert lens.numel() == B
    elif wl.ragged_min:
        lens = torch.randint(wl.ragged_min, wl.context + 1, (B,), generator=g[STREAM_SHAPE],
                             device=device).cpu()
    else:
        lens = torch.full((B,), wl.context, dtype=torch.int64)
    lens_list = [int(x) for x in lens]
    assert all(0 <= L <= wl.context for L in lens_list)
    nbs = [-(-L // blk) for L in lens_list]
    if wl.ragged_topk_frac:
        ks = [ragged_top_k(wl, L) for L in lens_list]
    else:
        ks = [wl.top_k] * B

    # ---- pool size and block tables --------------------------------------
    total_blocks = sum(nbs)
    if wl.occupancy < 1.0:
        P = max(1, math.ceil(total_blocks / wl.occupancy))
    else:
        P = max(1, B * max_blocks)
    block_table = torch.zeros((B, max_blocks), dtype=torch.int64)
    if wl.shuffle_table:
        perm = torch.randperm(P, generator=g[STREAM_TABLE], device=device).cpu()
    else:
        perm = torch.arange(P)
    off = 0
    for b in range(B):
        if wl.occupancy < 1.0:
            block_table[b, :nbs[b]] = perm[off:off + nbs[b]]
            off += nbs[b]
        else:
            block_table[b, :nbs[b]] = perm[b * max_blocks: b * max_blocks + nbs[b]]
    used = torch.zeros(P, dtype=torch.bool)
    for b in range(B):
        used[block_table[b, :nbs[b]]] = True

    # ---- queries ----------------------------------------------------------
    q32 = torch.empty((B, T, Hq, d), dtype=torch.float32, device=device)
    q32[:, 0].normal_(generator=g[STREAM_Q])
    if T == 2:
        noise = torch.empty((B, Hq, d), dtype=torch.float32, device=device).normal_(generator=g[STREAM_SPEC])
        q32[:, 1] = q32[:, 0] + wl.spec_noise * noise
    q = q32.to(_TORCH_DTYPE[wl.q_dtype])

    # ---- keys and values in physical (pool) order --------------------------
    head_major = wl.pool == "host"
    shape = (Hkv, P, blk, d) if head_major else (P, Hkv, blk, d)
    k32 = torch.empty(shape, dtype=torch.float32, device=device).normal_(generator=g[STREAM_K])
    if wl.outlier_channels:
        ch = torch.randperm(d, generator=g[STREAM_SHAPE], device=device)[:wl.outlier_channels]
        k32[..., ch] *= wl.outlier_scale
    salient = None
    if wl.salient_frac > 0:
        # Per (b, g): u = normalize(sum of the group's real-token queries + eps);
        # a seeded subset of ceil(frac * nb) logical blocks gets keys N(0,1) + alpha*u.
        salient = torch.zeros((B, Hkv, max_blocks), dtype=torch.bool)
        qsum = q32[:, 0].view(B, Hkv, G, d).sum(dim=2)
        eps = torch.empty((B, Hkv, d), dtype=torch.float32, device=device).normal_(generator=g[STREAM_SALIENCE])
        u = qsum + eps
        u = u / u.norm(dim=-1, keepdim=True)
        for b in range(B):
            n_sal = math.ceil(wl.salient_frac * nbs[b])
            for h in range(Hkv):
                js = torch.randperm(nbs[b], generator=g[STREAM_SALIENCE], device=device)[:n_sal].cpu()
                salient[b, h, js] = True
                phys = block_table[b, js].to(device)
                if head_major:
                    k32[h, phys] += wl.salient_alpha * u[b, h]
                else:
                    k32[phys, h] += wl.salient_alpha * u[b, h]
    v32 = torch.empty(shape, dtype=torch.float32, device=device).normal_(generator=g[STREAM_V])

    k_codes, k_scales = _encode(k32, wl.kv_dtype)
    v_codes, v_scales = _encode(v32, wl.kv_dtype)
    del v32
    if head_major and k_scales is not None:
        k_scales = k_scales.transpose(0, 1).contiguous()
        v_scales = v_scales.transpose(0, 1).contiguous()

    # ---- landmarks: mean of each logical block's stored keys over its valid rows
    lm = torch.zeros((B, Hkv, max_blocks, d), dtype=torch.float64, device=device)
    for b in range(B):
        nb = nbs[b]
        if nb == 0:
            continue
        phys = block_table[b, :nb].to(device)
        if head_major:
            kb = k_codes[:, phys]                      # [Hkv][nb][blk][d]
            sc = None if k_scales is None else k_scales[phys].transpose(0, 1)
        else:
            kb = k_codes[phys].transpose(0, 1)         # [Hkv][nb][blk][d]
            sc = None if k_scales is None else k_scales[phys].transpose(0, 1)
        kd = _decode64(kb, sc)
        rows = torch.clamp(lens_list[b] - torch.arange(nb, device=device) * blk, max=blk)  # valid rows per block
        mask = (torch.arange(blk, device=device)[None, :] < rows[:, None]).to(torch.float64)
        s = (kd * mask[None, :, :, None]).sum(dim=2)
        lm[b, :, :nb] = s / rows.to(torch.float64)[None, :, None]
    landmarks = lm.to(torch.float32).to(_TORCH_DTYPE[wl.landmark_dtype])
    del lm

    # ---- poison free blocks and rows past each sequence's end ---------------
    if wl.poison:
        nan_code = _nan_code(wl.kv_dtype)
        free = (~used).nonzero().flatten().to(device)
        for codes in (k_codes, v_codes):
            if free.numel():
                _fill_code(codes, (slice(None), free) if head_major else (free,), nan_code)
        for b in range(B):
            L, nb = lens_list[b], nbs[b]
            if nb == 0 or L % blk == 0:
                continue
            p_last = int(block_table[b, nb - 1])
            r0 = L - (nb - 1) * blk
            for codes in (k_codes, v_codes):
                idx = (slice(None), p_last, slice(r0, None)) if head_major else (p_last, slice(None), slice(r0, None))
                _fill_code(codes, idx, nan_code)

    # ---- recent-window buffers for the host-resident pool ----------------
    # Row r of pair (b, g) holds position ws_b + r; fp8 rows keep their pool
    # block's scales, one per row.  Rows past the window's end are unused:
    # zero, or with poison on, NaN codes and NaN scales.
    window_k = window_v = window_ks = window_vs = None
    if head_major:
        W = wl.window
        window_k = torch.zeros((B, Hkv, W, d), dtype=k_codes.dtype, device=device)
        window_v = torch.zeros((B, Hkv, W, d), dtype=v_codes.dtype, device=device)
        if k_scales is not None:
            window_ks = torch.ones((B, Hkv, W), dtype=torch.float32, device=device)
            window_vs = torch.ones((B, Hkv, W), dtype=torch.float32, device=device)
        for b in range(B):
            L = lens_list[b]
            ws = max(0, L - W)
            pos = torch.arange(ws, L, device=device)
            n = pos.numel()
            if wl.poison and n < W:
                for codes in (window_k, window_v):
                    _fill_code(codes, (b, slice(None), slice(n, None)), _nan_code(wl.kv_dtype))
                if window_ks is not None:
                    window_ks[b, :, n:] = float("nan")
                    window_vs[b, :, n:] = float("nan")
            if n == 0:
                continue
            phys = block_table[b].to(device)[pos // blk]
            rows = pos % blk
            window_k[b, :, :n] = k_codes[:, phys, rows].reshape(Hkv, -1, d)
            window_v[b, :, :n] = v_codes[:, phys, rows].reshape(Hkv, -1, d)
            if window_ks is not None:
                window_ks[b, :, :n] = k_scales[phys].transpose(0, 1)
                window_vs[b, :, :n] = v_scales[phys].transpose(0, 1)

    extras = {}
    if salient is not None:
        extras["salient"] = salient
    return DecodeInputs(
        wl=wl, q=q, landmarks=landmarks, k_pool=k_codes, v_pool=v_codes,
        k_scales=k_scales, v_scales=v_scales,
        block_table=block_table.to(torch.int32).to(device),
        seq_lens=torch.tensor(lens_list, dtype=torch.int32, device=device),
        k_per_seq=torch.tensor(ks, dtype=torch.int32, device=device),
        n_pool_blocks=P, pool_layout="head_major" if head_major else "block_major",
        window_k=window_k, window_v=window_v, window_k_scales=window_ks, window_v_scales=window_vs,
        extras=extras)


def _nan_code(dtype: str) -> int:
    return {"bf16": 0x7FC0, "fp8": 0x7F, "fp32": 0x7FC00000}[dtype]


def _fill_code(base: torch.Tensor, index, code: int) -> None:
    """Write the raw NaN bit pattern into base[index]."""
    int_dtype = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[base.element_size()]
    raw = base.view(int_dtype)
    if int_dtype == torch.int16 and code >= 0x8000:
        code -= 0x10000
    raw[index] = code


def raw_bytes(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Host numpy view of a tensor's bytes (uint16 for bf16, uint8 for fp8)."""
    if t is None:
        return None
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()
