"""The seeded input generator: determinism, the encoders and the workload
structure the parity tests and the bench rely on (CPU only)."""
import math

import numpy as np
import pytest
import torch

from sparse_kv_cache_block_amd import configs
from sparse_kv_cache_block_amd.inputs import FP8_MAX, _quantize_fp8, make_inputs, raw_bytes

FIELDS = ("q", "landmarks", "k_pool", "v_pool", "k_scales", "v_scales", "block_table", "seq_lens",
          "k_per_seq")


def _bytes(inp):
    return {f: raw_bytes(getattr(inp, f)) for f in FIELDS}


@pytest.mark.parametrize("wl", [configs.TINY, configs.LLAMA32K.scaled(batch=2, context=2048),
                                configs.DUAL.scaled(batch=1, context=4096),
                                configs.RAGGED.scaled(batch=4, context=4096, ragged_min=100)])
def test_same_seed_same_bytes_other_instance_other_bytes(wl):
    a, b, c = make_inputs(wl), make_inputs(wl), make_inputs(wl, instance=1)
    ba, bb, bc = _bytes(a), _bytes(b), _bytes(c)
    for f in FIELDS:
        if ba[f] is None:
            continue
        assert np.array_equal(ba[f].view(np.uint8), bb[f].view(np.uint8)), f
    assert not np.array_equal(ba["q"].view(np.uint8), bc["q"].view(np.uint8))


def _rne_bf16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of fp32 values to bf16 bit patterns, from the bits."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def test_bf16_encoding_is_round_to_nearest_even():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(1 << 16, generator=g) * torch.exp2(torch.randint(-20, 20, (1 << 16,), generator=g).float())
    # exact ties: the 16 dropped bits are 0x8000
    ties = (torch.arange(1, 1025, dtype=torch.int32) << 16 | 0x8000).view(torch.float32)
    x = torch.cat([x, ties, -ties])
    got = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, _rne_bf16(x.numpy()))


def _e4m3_value(code: int) -> float:
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def test_fp8_quantization_scale_and_rounding():
    g = torch.Generator().manual_seed(6)
    x = torch.randn(6, 3, 64, 128, generator=g) * torch.tensor([1e-3, 1.0, 50.0])[None, :, None, None]
    x[0, 0] = 0.0                                   # an all-zero chunk
    codes, scale = _quantize_fp8(x)
    amax = x.abs().amax(dim=(-2, -1))
    assert torch.equal(scale[0, 0], torch.tensor(1.0))
    nz = amax > 0
    assert torch.allclose(scale[nz], amax[nz] / FP8_MAX, rtol=0, atol=0)
    table = np.array([_e4m3_value(c) for c in range(256)])
    c = codes.view(torch.uint8).numpy().astype(np.int64)
    assert not np.isnan(table[c]).any()
    y = (x / scale[..., None, None]).numpy().astype(np.float64)
    dec = table[c]
    # nearest representable: no e4m3 value lies closer to y than the chosen one
    finite = table[~np.isnan(table)]
    sample = np.random.default_rng(0).choice(y.size, 4000, replace=False)
    for i in sample:
        yy, dd = y.flat[i], dec.flat[i]
        assert abs(dd - yy) <= np.min(np.abs(finite - yy)) + 1e-12
    assert np.abs(dec).max() <= FP8_MAX


def test_workload_structure():
    # llama32k: the block table is a permutation of the pool, the pool is fully used
    wl = configs.LLAMA32K.scaled(batch=2, context=2048)
    inp = make_inputs(wl)
    bt = inp.block_table.numpy()
    assert sorted(bt.ravel().tolist()) == list(range(inp.n_pool_blocks))
    # landmarks are the rounded mean of a block's stored keys
    g, b, j = 1, 1, 5
    blk = wl.block_size
    keys = inp.k_pool[bt[b, j], g].double().numpy()
    lm = inp.landmarks[b, g, j].double().numpy()
    mean = torch.tensor(keys.mean(axis=0), dtype=torch.float64).to(torch.float32).to(torch.bfloat16).double().numpy()
    assert keys.shape == (blk, wl.head_dim) and np.array_equal(lm, mean)
    # ragged: rows past each sequence's end and the free blocks hold NaN
    wr = configs.RAGGED.scaled(batch=3, context=4096, ragged_min=100)
    ri = make_inputs(wr, seq_lens=[4096, 1000, 37])
    kp = ri.k_pool.float().numpy()
    rt = ri.block_table.numpy()
    last = rt[2, 37 // wr.block_size]
    assert np.isnan(kp[last, :, 37 % wr.block_size:]).all()
    assert not np.isnan(kp[last, :, :37 % wr.block_size]).any()
    used = set(rt[0, :4096 // wr.block_size]) | set(rt[1, :-(-1000 // wr.block_size)]) | set(rt[2, :2])
    free = [p for p in range(ri.n_pool_blocks) if p not in used]
    assert free and np.isnan(kp[free]).all()
