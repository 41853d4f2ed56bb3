"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a hand-worked fixture, a closed form, an
invariant, an independent library computation or brute force, chosen so that a
plausible slip (a dropped head in the group sum, a transposed operand, a wrong
window boundary, a missing 1/sqrt(d), a wrong tie-break) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_kv_cache_block_amd import configs
from sparse_kv_cache_block_amd.inputs import make_inputs
from tests.common import HostArrays, oracle_problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------- decoders
def test_bf16_decode_all_codes_vs_torch():
    codes = np.arange(1 << 16, dtype=np.uint32)
    ref = torch.from_numpy(codes.astype(np.uint16).view(np.int16)).view(torch.bfloat16).float().numpy()
    got = np.array([O.bf16_value(int(c)) for c in codes], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan].astype(np.float64))


def test_e4m3fn_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([O.e4m3fn_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan].astype(np.float64))


def test_e4m3fn_decode_golden_points():
    with open(os.path.join(GOLDEN, "e4m3fn_points.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            code, value = line.split()
            got = O.e4m3fn_value(int(code, 16))
            if value == "nan":
                assert math.isnan(got)
            else:
                assert got == float(value) and math.copysign(1, got) == math.copysign(1, float(value)), code


# --------------------------------------------------------------- hand-worked step
def _small_problem(fx, k):
    B, Hq, Hkv, d, blk, L, W = (fx[x] for x in ("B", "Hq", "Hkv", "d", "blk", "L", "W"))
    nb = len(fx["landmarks"])
    pr = O.problem(B, 1, Hq, Hkv, d, blk, nb, nb, Hkv * blk * d, blk * d, W, max(k, 1),
                   "fp32", "fp32", "fp32")
    q = np.array(fx["q"], dtype=np.float32).reshape(B, 1, Hq, d)
    lm = np.array(fx["landmarks"], dtype=np.float32).reshape(B, Hkv, nb, d)
    kpool = np.zeros((nb, Hkv, blk, d), dtype=np.float32)
    vpool = np.zeros((nb, Hkv, blk, d), dtype=np.float32)
    for p in range(nb * blk):
        vpool[p // blk, 0, p % blk] = [p, 1.0]
    bt = np.arange(nb, dtype=np.int32).reshape(1, nb)
    return pr, q, lm, kpool, vpool, bt, np.array([L], np.int32), np.array([k], np.int32)


def test_small_step_golden():
    with open(os.path.join(GOLDEN, "small_step.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        pr, q, lm, kp, vp, bt, sl, kk = _small_problem(fx, case["k"])
        r = O.decode_step(pr, q, lm, kp, vp, None, None, bt, sl, kk)
        exp_scores = [float(x) for x in fx["expected_scores"]]
        assert list(r["scores"][0, 0, 0]) == exp_scores
        n = len(case["indices"])
        assert int(r["n_sel"][0, 0, 0]) == n
        assert list(r["indices"][0, 0, 0, :n]) == case["indices"]
        assert all(x == -1 for x in r["indices"][0, 0, 0, n:])
        for h in range(2):
            assert r["out"][0, h, 0] == pytest.approx(case["sum_p"] / case["count"], abs=1e-12)
            assert r["out"][0, h, 1] == pytest.approx(1.0, abs=1e-12)
            assert r["lse"][0, h] == pytest.approx(math.log(case["count"]), abs=1e-12)


# --------------------------------------------------------------- scoring
def _tiny(**kw):
    return configs.TINY.scaled(**kw)


def _decoded(t: torch.Tensor, scales=None, head_major=False) -> np.ndarray:
    x = t.to(torch.float64)
    if scales is not None:
        s = scales.to(torch.float64)
        if head_major:
            s = s.transpose(0, 1)
        x = x * s[..., None, None]
    return x.numpy()


@pytest.mark.parametrize("wl", [
    _tiny(context=512),
    configs.LLAMA32K.scaled(batch=2, context=1024, n_q_heads=8, n_kv_heads=2),
    configs.DUAL.scaled(batch=1, context=2048, n_q_heads=16, n_kv_heads=2),
])
def test_scores_vs_einsum(wl):
    inp = make_inputs(wl)
    h = HostArrays(inp)
    pr = oracle_problem(inp)
    got = O.scores(pr, h.q, h.landmarks, h.seq_lens)
    q = inp.q.to(torch.float64).numpy()
    lm = inp.landmarks.to(torch.float64).numpy()
    B, T, Hq, d = q.shape
    G = wl.group
    qg = q.reshape(B, T, wl.n_kv_heads, G, d)
    ref = np.einsum("btgxd,bgjd->btgj", qg, lm)
    for b in range(B):
        nc = configs.n_candidates(int(h.seq_lens[b]), wl.window, wl.block_size)
        assert np.all(np.isneginf(got[b, :, :, nc:]))
        np.testing.assert_allclose(got[b, :, :, :nc], ref[b, :, :, :nc], rtol=1e-12, atol=1e-9)


def test_scores_basis_landmarks_closed_form():
    # Landmark j = unit vector e_(j mod d) => score = sum over the group's heads of q_h[j mod d].
    wl = _tiny(context=1024, n_q_heads=6, n_kv_heads=2)
    inp = make_inputs(wl)
    d = wl.head_dim
    lm = torch.zeros_like(inp.landmarks)
    for j in range(wl.max_blocks):
        lm[:, :, j, j % d] = 1.0
    inp.landmarks = lm
    h = HostArrays(inp)
    got = O.scores(oracle_problem(inp), h.q, h.landmarks, h.seq_lens)
    q = inp.q.double().numpy()
    nc = configs.n_candidates(wl.context, wl.window, wl.block_size)
    for g in range(2):
        for j in range(nc):
            assert got[0, 0, g, j] == pytest.approx(q[0, 0, 3 * g:3 * g + 3, j % d].sum(), abs=1e-12)


def test_scores_linear_in_block_keys():
    # The landmark is the mean of the block's keys, and the score is linear in it:
    # score(j) = mean over the block's rows of sum_h q_h . k_row.
    wl = _tiny(context=1000)
    inp = make_inputs(wl)
    h = HostArrays(inp)
    got = O.scores(oracle_problem(inp), h.q, h.landmarks, h.seq_lens)
    q = inp.q.double().numpy()[0, 0]
    K = inp.k_pool.double().numpy()
    bt = h.block_table[0]
    blk, L = wl.block_size, wl.context
    nc = configs.n_candidates(L, wl.window, blk)
    for g in range(wl.n_kv_heads):
        qs = q[g * wl.group:(g + 1) * wl.group].sum(0)
        for j in range(nc):
            rows = min(blk, L - j * blk)
            keys = K[bt[j], g, :rows]
            exact = float(np.mean(keys @ qs))
            # landmarks are stored in fp32, so agreement is to fp32 rounding of the mean
            assert got[0, 0, g, j] == pytest.approx(exact, rel=1e-5, abs=1e-5)


# --------------------------------------------------------------- selection
def test_select_vs_lexsort():
    rng = np.random.default_rng(7)
    wl = _tiny(context=4096, batch=3)
    inp = make_inputs(wl, seq_lens=[4096, 700, 33])
    pr = oracle_problem(inp, k_max=40)
    sc = rng.standard_normal((3, 1, 2, wl.max_blocks))
    sc[..., ::7] = 0.25   # ties
    ks = np.array([40, 5, 3], np.int32)
    idx, nsel = O.select(pr, sc, [4096, 700, 33], ks)
    for b, L in enumerate([4096, 700, 33]):
        nc = configs.n_candidates(L, wl.window, wl.block_size)
        for g in range(2):
            row = sc[b, 0, g, :nc]
            order = np.lexsort((np.arange(nc), -row))
            k = min(int(ks[b]), nc)
            assert nsel[b, 0, g] == k
            assert list(idx[b, 0, g, :k]) == sorted(order[:k].tolist())
            assert all(idx[b, 0, g, k:] == -1)


def test_select_zero_query_picks_lowest_ids():
    wl = _tiny(context=2048)
    inp = make_inputs(wl)
    inp.q.zero_()
    h = HostArrays(inp)
    r = O.decode_step(oracle_problem(inp), h.q, h.landmarks, *h.pools(), h.block_table,
                      h.seq_lens, h.k_per_seq)
    assert np.all(r["scores"][0, 0, :, :100] == 0.0)
    assert list(r["indices"][0, 0, 0]) == list(range(wl.top_k))
    # q = 0 => every logit is 0 => o is the plain mean of v over sparse + window positions
    V = inp.v_pool.double().numpy()
    ws = wl.context - wl.window
    pos = [j * 16 + r_ for j in range(wl.top_k) for r_ in range(16) if j * 16 + r_ < ws] + list(range(ws, wl.context))
    for g in range(2):
        vals = np.stack([V[p // 16, g, p % 16] for p in pos])
        for hq in range(g * 4, g * 4 + 4):
            np.testing.assert_allclose(r["out"][0, hq], vals.mean(0), atol=1e-12)
            assert r["lse"][0, hq] == pytest.approx(math.log(len(pos)), abs=1e-12)


def test_select_all_when_k_exceeds_candidates():
    wl = _tiny(context=512, top_k=1000)
    inp = make_inputs(wl)
    h = HostArrays(inp)
    pr = oracle_problem(inp)
    sc = O.scores(pr, h.q, h.landmarks, h.seq_lens)
    idx, nsel = O.select(pr, sc, h.seq_lens, h.k_per_seq)
    nc = configs.n_candidates(512, wl.window, wl.block_size)
    assert int(nsel[0, 0, 0]) == nc
    assert list(idx[0, 0, 0, :nc]) == list(range(nc))


# --------------------------------------------------------------- gather
def test_gather_equals_fancy_indexing_and_round_trips():
    for wl in (configs.LLAMA32K.scaled(batch=2, context=2048, n_q_heads=8, n_kv_heads=2),
               configs.DUAL.scaled(batch=2, context=2048, n_q_heads=16, n_kv_heads=2)):
        inp = make_inputs(wl)
        h = HostArrays(inp)
        pr = oracle_problem(inp)
        sc = O.scores(pr, h.q, h.landmarks, h.seq_lens)
        idx, nsel = O.select(pr, sc, h.seq_lens, h.k_per_seq)
        ks, vs, kss, vss = O.gather(pr, *h.pools(), h.block_table, idx, nsel)
        kz = np.zeros_like(h.k_pool)
        for b in range(wl.batch):
            for g in range(wl.n_kv_heads):
                n = int(nsel[b, 0, g])
                phys = h.block_table[b, idx[b, 0, g, :n]]
                assert np.array_equal(ks[b, g, :n].view(np.uint8), h.k_pool[phys, g].view(np.uint8))
                assert np.array_equal(vs[b, g, :n].view(np.uint8), h.v_pool[phys, g].view(np.uint8))
                if h.k_scales is not None:
                    assert np.array_equal(kss[b, g, :n], h.k_scales[phys, g])
                    assert np.array_equal(vss[b, g, :n], h.v_scales[phys, g])
                kz[phys, g] = ks[b, g, :n]          # scatter back
                touched = np.zeros(h.k_pool.shape[0], bool)
                touched[phys] = True
                assert np.array_equal(kz[touched, g].view(np.uint8), h.k_pool[touched, g].view(np.uint8))


# --------------------------------------------------------------- attention
def _numpy_dense(inp, b, hq, positions, t=0):
    """Independent brute force: softmax(q.k/sqrt(d)) v over positions, numpy fp64
    (query token t)."""
    wl = inp.wl
    blk = wl.block_size
    g = hq // wl.group
    K = _decoded(inp.k_pool, inp.k_scales, inp.pool_layout == "head_major")
    V = _decoded(inp.v_pool, inp.v_scales, inp.pool_layout == "head_major")
    bt = inp.block_table.numpy()
    phys = bt[b, np.asarray(positions) // blk]
    rows = np.asarray(positions) % blk
    if inp.pool_layout == "head_major":
        kk, vv = K[g, phys, rows], V[g, phys, rows]
    else:
        kk, vv = K[phys, g, rows], V[phys, g, rows]
    q = inp.q.double().numpy()[b, t, hq]
    z = kk @ q / math.sqrt(wl.head_dim)
    m = z.max()
    w = np.exp(z - m)
    return (w[:, None] * vv).sum(0) / w.sum(), m + math.log(w.sum())


@pytest.mark.parametrize("wl", [
    _tiny(context=1000),
    configs.LLAMA32K.scaled(batch=2, context=1500, n_q_heads=8, n_kv_heads=2),
    configs.DUAL.scaled(batch=1, context=1200, n_q_heads=16, n_kv_heads=2, window=100),
    configs.HOST.scaled(batch=2, context=1100, window=70),
])
def test_k_all_equals_dense(wl):
    wl = wl.scaled(top_k=10_000)
    inp = make_inputs(wl)
    h = HostArrays(inp)
    pr = oracle_problem(inp)
    r = O.decode_step(pr, h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens, h.k_per_seq)
    dense_o, dense_lse = O.dense(pr, h.q, *h.pools(), h.block_table, h.seq_lens)
    np.testing.assert_allclose(r["out"], dense_o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(r["lse"], dense_lse, atol=1e-12, rtol=0)
    for b in range(wl.batch):
        L = int(h.seq_lens[b])
        for hq in (0, wl.n_q_heads - 1):
            o, lse = _numpy_dense(inp, b, hq, np.arange(L))
            np.testing.assert_allclose(r["out"][b, hq], o, atol=1e-12, rtol=0)
            assert r["lse"][b, hq] == pytest.approx(lse, abs=1e-12)


def test_sparse_step_vs_numpy_brute_force():
    wl = configs.LLAMA32K.scaled(batch=2, context=2000, n_q_heads=8, n_kv_heads=2, top_k=7)
    inp = make_inputs(wl)
    h = HostArrays(inp)
    pr = oracle_problem(inp)
    r = O.decode_step(pr, h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens, h.k_per_seq)
    ws = wl.context - wl.window
    for b in range(2):
        for hq in range(8):
            sel = r["indices"][b, 0, hq // 4, :int(r["n_sel"][b, 0, hq // 4])]
            pos = [j * 32 + x for j in sel for x in range(32) if j * 32 + x < ws] + list(range(ws, wl.context))
            o, lse = _numpy_dense(inp, b, hq, np.array(pos))
            np.testing.assert_allclose(r["out"][b, hq], o, atol=1e-12)
            assert r["lse"][b, hq] == pytest.approx(lse, abs=1e-12)


def test_merge_of_disjoint_partitions_is_attention_over_union():
    wl = configs.LLAMA32K.scaled(batch=1, context=900, n_q_heads=8, n_kv_heads=2)
    inp = make_inputs(wl)
    h = HostArrays(inp)
    pr = oracle_problem(inp)
    rng = np.random.default_rng(3)
    for trial in range(4):
        perm = rng.permutation(900)
        cuts = sorted(rng.choice(np.arange(1, 900), size=3, replace=False))
        parts = np.split(perm, cuts)
        hq = int(rng.integers(8))
        ps = [O.partial(pr, h.q, *h.pools(), h.block_table, 0, hq, np.sort(p)) for p in parts]
        o, lse = O.merge(np.stack([p[0] for p in ps]), np.array([p[1] for p in ps]))
        ou, lseu = O.partial(pr, h.q, *h.pools(), h.block_table, 0, hq, np.arange(900))
        np.testing.assert_allclose(o, ou, atol=1e-12)
        assert lse == pytest.approx(lseu, abs=1e-12)
        # two-way then two-way equals four-way
        o01, l01 = O.merge(np.stack([ps[0][0], ps[1][0]]), np.array([ps[0][1], ps[1][1]]))
        o23, l23 = O.merge(np.stack([ps[2][0], ps[3][0]]), np.array([ps[2][1], ps[3][1]]))
        o2, l2 = O.merge(np.stack([o01, o23]), np.array([l01, l23]))
        np.testing.assert_allclose(o2, ou, atol=1e-12)
        # merging an empty part is the identity
        oe, le = O.merge(np.stack([ou, np.zeros_like(ou)]), np.array([lseu, -np.inf]))
        np.testing.assert_array_equal(oe, ou)
        assert le == lseu


def test_attention_closed_forms():
    wl = _tiny(context=300, window=40)
    inp = make_inputs(wl)
    h = HostArrays(inp)
    pr = oracle_problem(inp)
    V = inp.v_pool.double().numpy()
    # a single attended position => o = v at that position, lse = its logit
    o, lse = O.partial(pr, h.q, *h.pools(), h.block_table, 0, 5, [123])
    np.testing.assert_array_equal(o, V[123 // 16, 1, 123 % 16])
    z = float(inp.q.double()[0, 0, 5] @ inp.k_pool.double()[123 // 16, 1, 123 % 16]) / 8.0
    assert lse == pytest.approx(z, abs=1e-12)
    # identical keys => uniform weights => o = mean of v
    inp.k_pool[:] = inp.k_pool[0, 0, 0]
    h2 = HostArrays(inp)
    pos = np.array([3, 50, 51, 200, 299])
    o, lse = O.partial(pr, h2.q, *h2.pools(), h2.block_table, 0, 2, pos)
    np.testing.assert_allclose(o, np.stack([V[p // 16, 0, p % 16] for p in pos]).mean(0), atol=1e-12)
    # an empty set => lse = -inf, o = 0
    o, lse = O.partial(pr, h.q, *h.pools(), h.block_table, 0, 0, [])
    assert lse == -math.inf and not o.any()


def test_window_edge_cases():
    # W = 0: no window part; L < W: no candidates; L = 0: empty everything.
    for W, lens in ((0, [700, 16]), (64, [40, 64, 65]), (64, [0, 5, 100])):
        wl = _tiny(context=768, window=W, batch=len(lens), top_k=4)
        inp = make_inputs(wl, seq_lens=lens)
        h = HostArrays(inp)
        pr = oracle_problem(inp)
        r = O.decode_step(pr, h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens, h.k_per_seq)
        for b, L in enumerate(lens):
            nc = configs.n_candidates(L, W, 16)
            assert int(r["n_sel"][b, 0, 0]) == min(4, nc)
            if L == 0:
                assert np.all(np.isneginf(r["lse"][b])) and not r["out"][b].any()
                continue
            ws = max(0, L - W)
            sel = r["indices"][b, 0, 0, :int(r["n_sel"][b, 0, 0])]
            pos = [j * 16 + x for j in sel for x in range(16) if j * 16 + x < ws] + list(range(ws, L))
            o, lse = _numpy_dense(inp, b, 1, np.array(pos))
            np.testing.assert_allclose(r["out"][b, 1], o, atol=1e-12)


def test_permuting_pool_and_table_changes_nothing():
    wl = configs.LLAMA32K.scaled(batch=2, context=1024, n_q_heads=8, n_kv_heads=2, top_k=5)
    inp = make_inputs(wl)
    h = HostArrays(inp)
    pr = oracle_problem(inp)
    r1 = O.decode_step(pr, h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens, h.k_per_seq)
    perm = np.random.default_rng(1).permutation(inp.n_pool_blocks)
    inv = np.argsort(perm)
    kp = np.ascontiguousarray(h.k_pool[perm])     # new block n holds old block perm[n]
    vp = np.ascontiguousarray(h.v_pool[perm])
    bt = inv[h.block_table].astype(np.int32)
    r2 = O.decode_step(pr, h.q, h.landmarks, kp, vp, None, None, bt, h.seq_lens, h.k_per_seq)
    assert np.array_equal(r1["indices"], r2["indices"])
    assert np.array_equal(r1["out"], r2["out"]) and np.array_equal(r1["lse"], r2["lse"])


def test_fp8_scale_is_applied_to_keys_and_values():
    wl = configs.DUAL.scaled(batch=1, context=700, n_q_heads=16, n_kv_heads=2, window=64, top_k=3)
    inp = make_inputs(wl)
    h = HostArrays(inp)
    pr = oracle_problem(inp)
    r = O.decode_step(pr, h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens, h.k_per_seq)
    ws = 700 - 64
    for hq in (0, 9):
        g = hq // 8
        sel = r["indices"][0, 0, g, :int(r["n_sel"][0, 0, g])]
        pos = [j * 64 + x for j in sel for x in range(64) if j * 64 + x < ws] + list(range(ws, 700))
        o, lse = _numpy_dense(inp, 0, hq, np.array(pos))
        np.testing.assert_allclose(r["out"][0, hq], o, atol=1e-12)


def test_overlap_identical_and_disjoint():
    wl = configs.DUAL.scaled(batch=2, context=4096, n_q_heads=16, n_kv_heads=2, top_k=10)
    inp = make_inputs(wl)
    inp.q[:, 1] = inp.q[:, 0]
    h = HostArrays(inp)
    pr = oracle_problem(inp)
    r = O.decode_step(pr, h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens, h.k_per_seq)
    assert np.all(r["overlap"] == 1.0)
    # speculative query = -real query reverses the ranking: disjoint top-10 of 48 candidates
    inp.q[:, 1] = -inp.q[:, 0]
    h = HostArrays(inp)
    r = O.decode_step(pr, h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens, h.k_per_seq)
    assert np.all(r["overlap"] == 0.0)
    # hand count on a partial overlap
    idx = np.full((1, 2, 1, 4), -1, np.int32)
    idx[0, 0, 0] = [1, 4, 6, 9]
    idx[0, 1, 0] = [4, 5, 9, -1]
    pr1 = O.problem(1, 2, 1, 1, 1, 1, 16, 16, 1, 1, 0, 4, "bf16", "bf16", "bf16")
    ov = O.overlap(pr1, idx, np.array([[[4], [3]]], np.int32))
    assert ov[0, 0] == 0.5


# --------------------------------------------------------------- both query tokens
def _dual_small(**kw):
    return configs.DUAL.scaled(batch=2, context=1500, n_q_heads=16, n_kv_heads=2, window=100, top_k=6, **kw)


def test_attend_tokens_vs_numpy_brute_force():
    # each token attends its own selection plus the window (co-batched attention)
    wl = _dual_small()
    inp = make_inputs(wl)
    h = HostArrays(inp)
    pr = oracle_problem(inp)
    r = O.decode_step(pr, h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens, h.k_per_seq)
    out, lse = O.attend_tokens(pr, h.q, *h.pools(), h.block_table, h.seq_lens, r["indices"], r["n_sel"])
    assert not np.array_equal(r["indices"][:, 0], r["indices"][:, 1])
    blk, G = wl.block_size, wl.group
    for b in range(wl.batch):
        L = int(h.seq_lens[b])
        ws = max(0, L - wl.window)
        for t in range(2):
            for hq in (0, 7, 8, 15):
                sel = r["indices"][b, t, hq // G, :int(r["n_sel"][b, t, hq // G])]
                pos = [j * blk + x for j in sel for x in range(blk) if j * blk + x < ws] + list(range(ws, L))
                o, ls = _numpy_dense(inp, b, hq, np.array(pos), t=t)
                np.testing.assert_allclose(out[b, t, hq], o, atol=1e-12, rtol=0)
                assert lse[b, t, hq] == pytest.approx(ls, abs=1e-12)


def test_attend_tokens_swapping_tokens_swaps_results():
    wl = _dual_small()
    inp = make_inputs(wl)
    h = HostArrays(inp)
    pr = oracle_problem(inp)
    r = O.decode_step(pr, h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens, h.k_per_seq)
    out, lse = O.attend_tokens(pr, h.q, *h.pools(), h.block_table, h.seq_lens, r["indices"], r["n_sel"])
    q_sw = np.ascontiguousarray(h.q[:, ::-1])
    idx_sw = np.ascontiguousarray(r["indices"][:, ::-1])
    nsel_sw = np.ascontiguousarray(r["n_sel"][:, ::-1])
    out_sw, lse_sw = O.attend_tokens(pr, q_sw, *h.pools(), h.block_table, h.seq_lens, idx_sw, nsel_sw)
    assert np.array_equal(out_sw[:, 0], out[:, 1]) and np.array_equal(out_sw[:, 1], out[:, 0])
    assert np.array_equal(lse_sw[:, ::-1], lse)
    assert not np.allclose(out[:, 0], out[:, 1])
