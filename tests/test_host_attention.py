"""The host part of the hybrid step (sparsekv_host_attention) against the
oracle's sparse partial, on the CPU: no GPU is needed for this entry point.

The oracle's attention returns each part (sparse, window) separately; the
host part must equal the sparse one on the same selection, to fp32 rounding.
"""
import numpy as np
import pytest

from oracle import oracle as O
from sparse_kv_cache_block_amd import binding as B
from sparse_kv_cache_block_amd import configs
from sparse_kv_cache_block_amd.inputs import make_inputs
from sparse_kv_cache_block_amd.step import problem_for
from tests.common import HostArrays, oracle_problem


def _ptr(a):
    return None if a is None else a.ctypes.data


@pytest.mark.parametrize("kw,lens,threads", [
    (dict(batch=2, context=4096), None, 0),                                   # bf16, G = 4, blk 64
    (dict(batch=3, context=4096, top_k=20), [4096, 700, 0], 2),               # ragged, an empty sequence
    (dict(batch=2, context=2048, head_dim=64, block_size=32, n_q_heads=64), None, 1),   # d 64, G = 8
    (dict(batch=2, context=2048, window=0, kv_dtype="fp8"), None, 0),
    (dict(batch=1, context=1024, kv_dtype="fp32", q_dtype="fp32", landmark_dtype="fp32", block_size=16,
          window=64), None, 0),
])
def test_host_attention_equals_oracle_sparse_part(kw, lens, threads):
    wl = configs.HOST.scaled(**kw)
    inp = make_inputs(wl, device="cpu", seq_lens=lens)
    h = HostArrays(inp)
    opr = oracle_problem(inp)
    r = O.decode_step(opr, h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens, h.k_per_seq)
    idx, nsel = r["indices"], r["n_sel"]
    _, _, po, pl = O.attend(opr, h.q, *h.pools(), h.block_table, h.seq_lens, idx, nsel, want_parts=True)
    o = np.full((wl.batch, wl.n_q_heads, wl.head_dim), np.nan, dtype=np.float32)
    lse = np.full((wl.batch, wl.n_q_heads), np.nan, dtype=np.float32)
    q = np.ascontiguousarray(h.q)
    sl = np.ascontiguousarray(h.seq_lens, dtype=np.int32)
    bt = np.ascontiguousarray(h.block_table, dtype=np.int32)
    idx32 = np.ascontiguousarray(idx, dtype=np.int32)
    nsel32 = np.ascontiguousarray(nsel, dtype=np.int32)
    kp, vp = np.ascontiguousarray(h.k_pool), np.ascontiguousarray(h.v_pool)
    ks = None if h.k_scales is None else np.ascontiguousarray(h.k_scales, dtype=np.float32)
    vs = None if h.v_scales is None else np.ascontiguousarray(h.v_scales, dtype=np.float32)
    part = B.HostPart(_ptr(kp), _ptr(vp), threads, _ptr(q), _ptr(sl), _ptr(bt), _ptr(idx32), _ptr(nsel32),
                      _ptr(ks), _ptr(vs), _ptr(o), _ptr(lse))
    B.sparsekv_host_attention(problem_for(inp), part)
    ref_o, ref_lse = po[:, :, 0, :], pl[:, :, 0]
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.all(lse[~fin] == -np.inf) and np.all(o[~fin] == 0.0)
    tol = {"fp32": 1e-5, "bf16": 2e-3, "fp8": 8e-3}[wl.kv_dtype]
    err = float(np.max(np.abs(o.astype(np.float64) - ref_o)))
    assert err <= tol, err
    if fin.any():
        assert float(np.max(np.abs(lse[fin] - ref_lse[fin]))) <= 1e-4
    # fp32 arithmetic on exactly decoded inputs: far inside the bound
    assert err <= 1e-5


def test_host_attention_rejects_device_pools():
    wl = configs.HOST.scaled(batch=1, context=4096)
    inp = make_inputs(wl, device="cpu")
    pr = problem_for(inp)
    d = 0x1000
    assert B.lib().sparsekv_host_attention(pr, None) == B.SKV_E_NULL
    pr.pool_location = B.SKV_POOL_DEVICE
    part = B.HostPart(d, d, 0, d, d, d, d, d, None, None, d, d)
    assert B.lib().sparsekv_host_attention(pr, part) == B.SKV_E_UNSUPPORTED
