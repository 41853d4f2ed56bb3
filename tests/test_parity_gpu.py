"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Gates (selected indices bit-exact outside the 1e-5 relative exemption band of
the k-th score; gathered bytes exact; attention output max-abs 2e-3 for bf16
K/V, 8e-3 for fp8, and 1e-4 for the fp32 reference shape) on seeded inputs.
Attention is compared against the oracle evaluated on the GPU's own index set,
so an exempt near-tie swap is never counted as an attention error.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_kv_cache_block_amd import binding as B
from sparse_kv_cache_block_amd import configs
from sparse_kv_cache_block_amd.inputs import make_inputs
from sparse_kv_cache_block_amd.step import DecodeStep, to_device_for
from tests.common import HostArrays, check_indices, oracle_problem

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-3, "fp8": 8e-3}


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _np(t):
    return t.detach().cpu().numpy()


def compare_attention(inp, h, gpu_idx, gpu_nsel, gpu_out, gpu_lse, tol):
    pr = oracle_problem(inp, k_max=gpu_idx.shape[-1])
    o_out, o_lse = O.attend(pr, h.q, *h.pools(), h.block_table, h.seq_lens, gpu_idx, gpu_nsel)
    err = float(np.max(np.abs(gpu_out.astype(np.float64) - o_out))) if o_out.size else 0.0
    assert err <= tol, f"attention max-abs error {err} > {tol}"
    fin = np.isfinite(o_lse)
    assert np.array_equal(fin, np.isfinite(gpu_lse)), "lse finiteness differs"
    if fin.any():
        lerr = float(np.max(np.abs(gpu_lse[fin] - o_lse[fin])))
        assert lerr <= tol, f"lse error {lerr} > {tol}"
    assert np.all(gpu_lse[~fin] == -np.inf)
    return err


def run_step(wl, seq_lens=None, gen_device="cpu", mutate=None, k_max=None):
    inp = make_inputs(wl, device=gen_device, seq_lens=seq_lens)
    if mutate:
        mutate(inp)
    inp = inp.to("cpu") if gen_device != "cpu" else inp
    dev = to_device_for(inp)
    st = DecodeStep(dev, k_max=k_max)
    st.run()
    torch.cuda.synchronize()
    return inp, st


def check_step(wl, seq_lens=None, gen_device="cpu", mutate=None):
    announce(f"decode_step {wl.name} B={wl.batch} L={wl.context} kv={wl.kv_dtype} T={wl.n_q_tokens} "
             f"pool={wl.pool} seq_lens={seq_lens}")
    inp, st = run_step(wl, seq_lens, gen_device, mutate)
    h = HostArrays(inp)
    pr = oracle_problem(inp)
    orc = O.decode_step(pr, h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens, h.k_per_seq)
    gi, gn = _np(st.indices), _np(st.n_sel)
    swaps = check_indices(gi, gn, orc["indices"], orc["n_sel"], orc["scores"], h.seq_lens,
                          wl.window, wl.block_size)
    err = compare_attention(inp, h, gi, gn, _np(st.out), _np(st.lse), TOL[wl.kv_dtype])
    if wl.n_q_tokens == 2:
        ov = O.overlap(pr, gi, gn)
        np.testing.assert_allclose(_np(st.overlap), ov, rtol=0, atol=1e-6)
    if swaps == 0:
        # same selection: the end-to-end result matches the oracle's own decode step
        assert float(np.max(np.abs(_np(st.out) - orc["out"]))) <= TOL[wl.kv_dtype]
    print(f"[case] ok: max-abs err {err:.3g}, exempt swaps {swaps}", flush=True)
    return inp, st


# ------------------------------------------------------------ small shapes
def test_tiny_reference_config():
    check_step(configs.TINY)


def test_llama32k_shape_small_context():
    check_step(configs.LLAMA32K.scaled(batch=2, context=4096))


def test_llama32k_shape_mixed_lengths():
    check_step(configs.LLAMA32K.scaled(batch=4, context=4096), seq_lens=[4096, 1000, 513, 37])


def test_ragged_small_poisoned():
    check_step(configs.RAGGED.scaled(batch=6, context=8192, ragged_min=100))


def test_dual_fp8_small():
    check_step(configs.DUAL.scaled(batch=2, context=16384, window=1024))


def test_host_pool_small():
    check_step(configs.HOST.scaled(batch=2, context=8192))


# fp8 window buffers of a host pool: each row carries the K and V scales of
# the pool block its position lives in.  With poison on, the rows past each
# window's end hold NaN codes and NaN scales, and free blocks NaN codes.
FP8_WIN = configs.HOST.scaled(batch=3, context=8192, kv_dtype="fp8", poison=True)


@pytest.mark.parametrize("wl,lens", [
    (FP8_WIN, [8192, 300, 0]),                # a window shorter than W, an empty sequence
    (FP8_WIN.scaled(block_size=16, window=256, head_dim=64), [8192, 5000, 200]),
    (FP8_WIN.scaled(block_size=32, n_q_tokens=2, spec_noise=0.3), [8192, 4100, 1500]),
])
def test_host_pool_fp8_window(wl, lens):
    check_step(wl, seq_lens=lens)


@pytest.mark.parametrize("kw", [
    dict(window=0),
    dict(top_k=90),
    dict(head_dim=64),
    dict(block_size=16),
    dict(block_size=64),
    dict(n_q_heads=16, n_kv_heads=8),
    dict(n_q_heads=8, n_kv_heads=1),
])
def test_bf16_variants(kw):
    args = dict(batch=2, context=3000, top_k=24)
    args.update(kw)
    check_step(configs.LLAMA32K.scaled(**args), seq_lens=[3000, 2100])


@pytest.mark.parametrize("kw", [dict(block_size=16), dict(block_size=32), dict(head_dim=64)])
def test_fp8_variants(kw):
    check_step(configs.DUAL.scaled(batch=2, context=4096, window=256, top_k=20, **kw))


@pytest.mark.parametrize("blk", [32, 64])
def test_fp32_variants(blk):
    # fp32 K/V at d = 128 attends 16-token slices (a 32-token one would not fit a wave's registers)
    check_step(configs.TINY.scaled(batch=2, head_dim=128, block_size=blk), seq_lens=[4096, 777])


def test_zero_query_ties_go_to_lowest_ids():
    def zero_q(inp):
        inp.q.zero_()
    inp, st = check_step(configs.LLAMA32K.scaled(batch=2, context=4096), mutate=zero_q)
    gi = _np(st.indices)
    assert np.all(gi[:, 0, :, :] == np.arange(64)[None, None, :])


def test_duplicated_landmarks_exact_ties():
    def dup(inp):
        inp.landmarks[:, :, 1::2] = inp.landmarks[:, :, 0::2]
    check_step(configs.LLAMA32K.scaled(batch=2, context=4096, top_k=13), mutate=dup)


def test_empty_and_window_only_sequences():
    check_step(configs.LLAMA32K.scaled(batch=4, context=2048), seq_lens=[0, 1, 512, 513])


def test_dual_identical_tokens_overlap_one():
    def same(inp):
        inp.q[:, 1] = inp.q[:, 0]
    inp, st = check_step(configs.DUAL.scaled(batch=2, context=8192), mutate=same)
    assert np.all(_np(st.overlap) == 1.0)


def test_two_tokens_many_candidates_few_pairs():
    """Two tokens, 2 (sequence, KV head) pairs and 9996 candidates each: the
    scoring rows are split over many workgroups, and the selecting workgroup's
    candidate ids (2 x 9996 words) do not fit in its LDS next to the keys, so
    the selected ids are read back from the workspace."""
    wl = configs.DUAL.scaled(batch=1, n_q_heads=16, n_kv_heads=2, block_size=16, context=160000,
                             window=64, top_k=64)
    check_step(wl, gen_device="cuda")


@pytest.mark.parametrize("k", [200, 16], ids=["one_level", "two_levels"])
def test_two_tokens_at_the_block_limit(k):
    """16384 blocks per sequence (the most the library takes), two tokens, 2
    pairs, 16380 candidates.  k 200 exceeds a chunk's 128 rows, so the last
    workgroup selects over all 2 x 16380 published scores in LDS (about 135 KB);
    k 16 takes two levels with the candidates' ids read back from the workspace."""
    wl = configs.DUAL.scaled(batch=1, n_q_heads=16, n_kv_heads=2, block_size=16, context=262144,
                             window=64, top_k=k)
    assert wl.max_blocks == 16384
    check_step(wl, gen_device="cuda")


# 2 sequences x 2 KV heads, 4080 candidates, k 16: each of 64 scoring workgroups
# per pair keeps its own top 16 (1024 candidates) and the last one selects
TWO_LEVEL = configs.LLAMA32K.scaled(batch=2, n_q_heads=8, n_kv_heads=2, context=131072, top_k=16)


@pytest.mark.parametrize("wl", [TWO_LEVEL, TWO_LEVEL.scaled(n_q_tokens=2, spec_noise=0.3)],
                         ids=["one_token", "two_tokens"])
def test_two_level_selection_ragged(wl):
    """Chunk counts differ per sequence: the second has 1221 candidates, 19 full
    chunks of 64 and a last one of 5 rows, which keeps fewer than k."""
    check_step(wl, seq_lens=[131072, 39584], gen_device="cuda")


# The split step (two-level selection on a device pool): every attention split
# selects from the chunks' candidates.  An empty sequence (no candidates, no
# window), one whose 6 candidates fit one chunk and are all selected, no window
# at all, and the dual fp8 shape with NaN-poisoned free blocks and tail rows.
@pytest.mark.parametrize("wl,lens", [
    (TWO_LEVEL.scaled(n_q_tokens=2, spec_noise=0.3), [0, 131072]),
    (TWO_LEVEL, [700, 131072]),
    (TWO_LEVEL.scaled(window=0), [131072, 39584]),
    (configs.DUAL.scaled(poison=True), [262144, 100000, 1500, 0]),
    (configs.DUAL.scaled(batch=2, block_size=32), None),                       # fp8, blocks of 32, 16 chunks
    (TWO_LEVEL.scaled(block_size=64, context=262144), [262144, 150000]),       # bf16, blocks of 64
    (configs.RAGGED.scaled(batch=4, context=131072), None),                    # k = 2% of each sequence's blocks
], ids=["empty_sequence", "all_candidates_selected", "no_window", "dual_poisoned_ragged", "fp8_block32",
        "bf16_block64", "ragged_k"])
def test_split_step_edge_cases(wl, lens):
    check_step(wl, seq_lens=lens, gen_device="cuda")


def test_two_level_selection_ties_go_to_lowest_ids():
    def zero_q(inp):
        inp.q.zero_()
    inp, st = check_step(TWO_LEVEL.scaled(n_q_tokens=2), mutate=zero_q, gen_device="cuda")
    gi = _np(st.indices)
    assert np.all(gi == np.arange(16)[None, None, None, :])


# More two-level shapes: one token over 32 chunks of 256 rows; two tokens over
# 4 chunks of 1024 rows; k = 100 (not a power of two) over 8 chunks of 512.
@pytest.mark.parametrize("wl", [
    configs.LLAMA32K.scaled(batch=1, context=262144),
    configs.DUAL.scaled(batch=8),
    configs.DUAL.scaled(top_k=100),
], ids=["one_token_32_chunks", "two_tokens_1024_rows", "k_100"])
def test_two_level_selection_shapes(wl):
    check_step(wl, gen_device="cuda")


def _random_split_shapes(n, seed=11):
    """Seeded random few-pair shapes whose device step takes the split step."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        hkv = int(rng.choice([1, 2, 4, 8]))
        wl = configs.LLAMA32K.scaled(
            name=f"split{len(out)}", batch=int(rng.integers(1, 4)), n_kv_heads=hkv,
            n_q_heads=hkv * int(rng.choice([1, 2, 4, 8])), block_size=int(rng.choice([32, 64])),
            context=int(rng.choice([98304, 131072, 196608])), top_k=int(rng.integers(1, 200)),
            window=int(rng.choice([0, 64, 256, 1024])), n_q_tokens=int(rng.choice([1, 2])),
            kv_dtype=str(rng.choice(["bf16", "fp8"])), spec_noise=0.3, outlier_channels=0,
            seed=int(rng.integers(0, 1 << 16)))
        if wl.batch * wl.n_kv_heads >= 128 or wl.top_k > wl.max_blocks:
            continue
        pr = B.make_problem(wl.batch, wl.n_q_tokens, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.block_size,
                            wl.max_blocks, wl.batch * wl.max_blocks, wl.n_kv_heads * wl.block_size * wl.head_dim,
                            wl.block_size * wl.head_dim, wl.window, wl.top_k, wl.q_dtype, wl.kv_dtype,
                            wl.landmark_dtype)
        if B.sparsekv_decode_step_kernel(pr, 1) != "split_step_kernel":
            continue
        lens = [int(x) for x in rng.integers(0, wl.context + 1, size=wl.batch)]
        lens[0] = wl.context
        out.append((wl, lens))
    return out


@pytest.mark.parametrize("wl,lens", _random_split_shapes(8), ids=lambda v: getattr(v, "name", None))
def test_split_step_random_shapes(wl, lens):
    """Seeded random few-pair shapes (batch, heads, group size, block size,
    context, k, window, tokens, K/V type, lengths) that the plan sends to the
    split step, against the oracle."""
    check_step(wl, seq_lens=lens, gen_device="cuda")


# ------------------------------------------------ single-launch step (>= 128 pairs)
# 16 sequences x 8 KV heads: decode_step runs as one launch, one workgroup per pair
MIXED16 = [4096, 1000, 513, 37, 0, 1, 512, 513, 4000, 2048, 3333, 4095, 64, 700, 2500, 4096]


def check_single_launch(wl, **kw):
    inp, st = check_step(wl, **kw)
    assert B.sparsekv_decode_step_launches(st.pr) == 1
    return inp, st


@pytest.mark.parametrize("kw,lens", [
    (dict(), MIXED16),
    (dict(window=0), None),                 # no window slice comes first in any wave
    (dict(top_k=120), MIXED16),             # k beyond every sequence's candidates
    (dict(block_size=64), MIXED16),
    (dict(n_q_heads=16), None),             # G = 2
    (dict(n_q_heads=64), None),             # G = 8
])
def test_single_launch_bf16(kw, lens):
    args = dict(batch=16, context=4096)
    args.update(kw)
    check_single_launch(configs.LLAMA32K.scaled(**args), seq_lens=lens)


def test_single_launch_full_waves():
    # 17 window slices over the 7 waves that do not select (3 in the first)
    # and 488 selected blocks over all 8 (61 each): the first window wave
    # holds 64 items, one per lane, the most a wave takes
    wl = configs.LLAMA32K.scaled(batch=16, context=32768, top_k=488)
    check_single_launch(wl)


def test_many_blocks_fall_back_to_two_launches():
    # 600 selected blocks + 17 window blocks exceed one step workgroup's 512 item slots
    wl = configs.LLAMA32K.scaled(batch=16, context=32768, top_k=600)
    inp, st = check_step(wl)
    assert B.sparsekv_decode_step_launches(st.pr) == 2


def test_single_launch_longest_first():
    # 40 x 8 = 320 pairs, more than the compute units: the step visits the
    # sequences longest first; every output row must still be its own sequence's
    lens = [int(x) for x in np.random.default_rng(7).integers(0, 2049, size=40)]
    lens[3] = lens[4] = 2048   # equal lengths keep index order
    check_single_launch(configs.LLAMA32K.scaled(batch=40, context=2048, top_k=24), seq_lens=lens)


def test_single_launch_ragged_poisoned():
    check_single_launch(configs.RAGGED.scaled(batch=16, context=8192, ragged_min=100))


# 64 sequences x 8 KV heads = 512 pairs, twice the compute units: two rounds
# of step workgroups, longest sequences first
LENS64 = [int(x) for x in np.random.default_rng(11).integers(0, 3073, size=64)]
LENS64[:6] = [0, 1, 256, 257, 3072, 3072]


@pytest.mark.parametrize("wl", [
    configs.RAGGED.scaled(batch=64, context=3072, ragged_min=0),
    configs.LLAMA32K.scaled(batch=64, context=3072, top_k=24),
    configs.LLAMA32K.scaled(batch=64, context=3072, top_k=24, block_size=64, window=0),
    configs.DUAL.scaled(batch=64, context=3072, window=256, top_k=20),
], ids=["ragged_poisoned", "bf16", "bf16_blk64_no_window", "dual_fp8"])
def test_single_launch_two_rounds_of_pairs(wl):
    lens = None if wl.name == "ragged" else LENS64
    check_single_launch(wl, seq_lens=lens)


@pytest.mark.parametrize("kw", [dict(), dict(block_size=32, context=4096, window=256, top_k=20)])
def test_single_launch_dual_fp8(kw):
    args = dict(batch=16, context=8192, top_k=30)
    args.update(kw)
    check_single_launch(configs.DUAL.scaled(**args))


def test_single_launch_ties():
    def zero_q(inp):
        inp.q.zero_()
    inp, st = check_single_launch(configs.LLAMA32K.scaled(batch=16, context=4096), mutate=zero_q)
    assert np.all(_np(st.indices)[:, 0, :, :] == np.arange(64)[None, None, :])

    def dup(inp):
        inp.landmarks[:, :, 1::2] = inp.landmarks[:, :, 0::2]
    check_single_launch(configs.LLAMA32K.scaled(batch=16, context=4096, top_k=13), mutate=dup)


# ------------------------------------------------------------ separate entry points
def test_score_and_topk_entry_points():
    wl = configs.DUAL.scaled(batch=2, context=8192, top_k=40)
    announce("sparsekv_score + sparsekv_topk on the dual shape")
    inp = make_inputs(wl, seq_lens=[8192, 5000])
    dev = to_device_for(inp)
    from sparse_kv_cache_block_amd.step import problem_for
    pr = problem_for(dev)
    scores = torch.empty((2, 2, wl.n_kv_heads, wl.max_blocks), dtype=torch.float32, device="cuda")
    B.sparsekv_score(pr, dev.q, dev.landmarks, dev.seq_lens, scores)
    idx = torch.empty((2, 2, wl.n_kv_heads, pr.k_max), dtype=torch.int32, device="cuda")
    nsel = torch.empty((2, 2, wl.n_kv_heads), dtype=torch.int32, device="cuda")
    ov = torch.empty((2, wl.n_kv_heads), dtype=torch.float32, device="cuda")
    B.sparsekv_topk(pr, scores, dev.seq_lens, dev.k_per_seq, idx, nsel, ov)
    torch.cuda.synchronize()
    h = HostArrays(inp)
    opr = oracle_problem(inp)
    osc = O.scores(opr, h.q, h.landmarks, h.seq_lens)
    gsc = _np(scores).astype(np.float64)
    fin = np.isfinite(osc)
    assert np.array_equal(fin, np.isfinite(gsc))
    rel = np.abs(gsc[fin] - osc[fin]) / np.maximum(np.abs(osc[fin]), 1.0)
    assert rel.max() < 1e-5, rel.max()
    # top-k of the GPU's own fp32 scores must equal the oracle's selection on them, bit for bit
    oi, on = O.select(opr, gsc, h.seq_lens, h.k_per_seq)
    assert np.array_equal(_np(idx), oi) and np.array_equal(_np(nsel), on)
    np.testing.assert_allclose(_np(ov), O.overlap(opr, oi, on), atol=1e-6)


def test_gather_and_attend_entry_points():
    for wl in (configs.LLAMA32K.scaled(batch=2, context=4096),
               configs.DUAL.scaled(batch=2, context=8192, top_k=30)):
        announce(f"sparsekv_gather + sparsekv_attend ({wl.name})")
        inp, st = run_step(wl)
        dev = st.inp
        pr = st.pr
        Bn, Hkv, km = wl.batch, wl.n_kv_heads, pr.k_max
        shape = (Bn, Hkv, km, wl.block_size, wl.head_dim)
        ks = torch.zeros(shape, dtype=dev.k_pool.dtype, device="cuda")
        vs = torch.zeros(shape, dtype=dev.v_pool.dtype, device="cuda")
        kss = vss = None
        if dev.k_scales is not None:
            kss = torch.zeros((Bn, Hkv, km), dtype=torch.float32, device="cuda")
            vss = torch.zeros((Bn, Hkv, km), dtype=torch.float32, device="cuda")
        B.sparsekv_gather(pr, dev.k_pool, dev.v_pool, dev.k_scales, dev.v_scales, dev.block_table,
                          st.indices, st.n_sel, ks, vs, kss, vss)
        torch.cuda.synchronize()
        h = HostArrays(inp)
        opr = oracle_problem(inp, k_max=km)
        oks, ovs, okss, ovss = O.gather(opr, *h.pools(), h.block_table, _np(st.indices), _np(st.n_sel))
        nsel = _np(st.n_sel)
        from sparse_kv_cache_block_amd.inputs import raw_bytes
        gks, gvs = raw_bytes(ks), raw_bytes(vs)
        for b in range(Bn):
            for g in range(Hkv):
                n = int(nsel[b, 0, g])
                assert np.array_equal(gks[b, g, :n].view(np.uint8), oks[b, g, :n].view(np.uint8))
                assert np.array_equal(gvs[b, g, :n].view(np.uint8), ovs[b, g, :n].view(np.uint8))
                if kss is not None:
                    assert np.array_equal(_np(kss)[b, g, :n], okss[b, g, :n])
                    assert np.array_equal(_np(vss)[b, g, :n], ovss[b, g, :n])
        # attention from the staged copy equals attention straight from the pool;
        # the decode step runs as one launch with its own split layout, so the
        # two agree up to the order of fp32 sums
        out2 = torch.empty_like(st.out)
        lse2 = torch.empty_like(st.lse)
        sparse = B.kv_source(B.SKV_SRC_STAGED, ks, vs, kss, vss)
        window = B.kv_source(B.SKV_SRC_PAGED, dev.k_pool, dev.v_pool, dev.k_scales, dev.v_scales,
                             dev.block_table)
        B.sparsekv_attend(pr, dev.q, sparse, st.indices, st.n_sel, window, dev.seq_lens, out2, lse2, st.ws)
        torch.cuda.synchronize()
        assert (out2 - st.out).abs().max().item() <= 2e-5
        assert (lse2 - st.lse).abs().max().item() <= 2e-5


# ------------------------------------------------ co-batched two-token attention
def _two_token_attention(st):
    """Co-batched attention of both tokens, and the two single-token launches
    it replaces (token 1 through views that start at its rows)."""
    dev, pr = st.inp, st.pr
    Bn, Hq, D = dev.q.shape[0], dev.q.shape[2], dev.q.shape[3]
    out = torch.full((Bn, 2, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((Bn, 2, Hq), float("nan"), dtype=torch.float32, device="cuda")
    src = B.kv_source(B.SKV_SRC_PAGED, dev.k_pool, dev.v_pool, dev.k_scales, dev.v_scales, dev.block_table)
    B.sparsekv_attend_cobatched(pr, dev.q, src, st.indices, st.n_sel, src, dev.seq_lens, out, lse, st.ws)
    sep_out = torch.empty_like(out)
    sep_lse = torch.empty_like(lse)
    for t in range(2):
        o_t = torch.empty((Bn, Hq, D), dtype=torch.float32, device="cuda")
        l_t = torch.empty((Bn, Hq), dtype=torch.float32, device="cuda")
        B.sparsekv_attend(pr, dev.q[:, t:], src, st.indices[:, t:], st.n_sel[:, t:], src, dev.seq_lens,
                          o_t, l_t, st.ws)
        sep_out[:, t] = o_t
        sep_lse[:, t] = l_t
    torch.cuda.synchronize()
    return out, lse, sep_out, sep_lse


def check_cobatched(wl, seq_lens=None, mutate=None):
    announce(f"attend_cobatched {wl.name} B={wl.batch} L={wl.context} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} "
             f"d={wl.head_dim} blk={wl.block_size} k={wl.top_k} W={wl.window} kv={wl.kv_dtype} "
             f"seq_lens={seq_lens}")
    inp, st = run_step(wl, seq_lens=seq_lens, mutate=mutate)
    out, lse, sep_out, sep_lse = _two_token_attention(st)
    h = HostArrays(inp)
    gi, gn = _np(st.indices), _np(st.n_sel)
    pr = oracle_problem(inp, k_max=gi.shape[-1])
    o_out, o_lse = O.attend_tokens(pr, h.q, *h.pools(), h.block_table, h.seq_lens, gi, gn)
    tol = TOL[wl.kv_dtype]
    g_out, g_lse = _np(out), _np(lse)
    err = float(np.max(np.abs(g_out.astype(np.float64) - o_out)))
    assert err <= tol, f"co-batched attention max-abs error {err} > {tol}"
    fin = np.isfinite(o_lse)
    assert np.array_equal(fin, np.isfinite(g_lse))
    assert np.all(g_lse[~fin] == -np.inf)
    if fin.any():
        assert float(np.max(np.abs(g_lse[fin] - o_lse[fin]))) <= tol
    # the same values as one launch per token, and as the decode step's real token
    assert (out - sep_out).abs().max().item() <= 2e-5
    if fin.any():
        fin_t = torch.from_numpy(fin).cuda()
        assert (lse[fin_t] - sep_lse[fin_t]).abs().max().item() <= 2e-5
    assert (out[:, 0] - st.out).abs().max().item() <= 2e-5
    union = sum(len(set(gi[b, 0, g, :gn[b, 0, g]]) | set(gi[b, 1, g, :gn[b, 1, g]]))
                for b in range(gi.shape[0]) for g in range(gi.shape[2]))
    print(f"[case] ok: max-abs err {err:.3g}, union blocks {union}", flush=True)
    return out, st


@pytest.mark.parametrize("wl,lens", [
    (configs.DUAL.scaled(batch=2, context=8192, top_k=30), None),                  # G = 8 fp8, 16 columns
    (configs.DUAL.scaled(batch=3, context=4096, block_size=32, top_k=20, window=256), [4096, 700, 0]),
    (configs.LLAMA32K.scaled(batch=2, context=4096, n_q_tokens=2, spec_noise=0.3), None),   # G = 4 bf16
    (configs.LLAMA32K.scaled(batch=2, context=3000, n_q_tokens=2, spec_noise=0.3, block_size=16,
                             head_dim=64, window=0), [3000, 1]),
    (configs.TINY.scaled(n_q_tokens=2, spec_noise=0.3), None),                      # fp32
    (configs.TINY.scaled(n_q_tokens=2, spec_noise=0.3, head_dim=128, block_size=32), None),  # fp32, 16-token slices
])
def test_cobatched_attention(wl, lens):
    check_cobatched(wl, seq_lens=lens)


def test_cobatched_identical_and_disjoint_tokens():
    wl = configs.DUAL.scaled(batch=2, context=8192, top_k=30)

    def same(inp):
        inp.q[:, 1] = inp.q[:, 0]
    out, st = check_cobatched(wl, mutate=same)
    assert (out[:, 0] - out[:, 1]).abs().max().item() <= 1e-6

    def opposite(inp):
        inp.q[:, 1] = -inp.q[:, 0]
    # reversed ranking: the union holds 2k blocks per (sequence, KV head)
    check_cobatched(wl, mutate=opposite)
    # k beyond the candidates: both tokens select every candidate
    check_cobatched(wl.scaled(top_k=120))


def test_cobatched_full_size_dual():
    check_cobatched(configs.DUAL)


def test_cobatched_rejects_staged_and_host():
    wl = configs.DUAL.scaled(batch=2, context=4096, top_k=10)
    inp, st = run_step(wl)
    dev, pr = st.inp, st.pr
    src = B.kv_source(B.SKV_SRC_STAGED, dev.k_pool, dev.v_pool, dev.k_scales, dev.v_scales)
    win = B.kv_source(B.SKV_SRC_PAGED, dev.k_pool, dev.v_pool, dev.k_scales, dev.v_scales, dev.block_table)
    out = torch.empty((2, 2, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="paged"):
        B.sparsekv_attend_cobatched(pr, dev.q, src, st.indices, st.n_sel, win, dev.seq_lens, out, None, st.ws)


@pytest.mark.parametrize("wl", [configs.DUAL.scaled(batch=2, context=8192, top_k=30),
                                configs.HOST.scaled(batch=2, context=8192, n_q_tokens=2, spec_noise=0.3)])
def test_speculative_gather_correction(wl):
    # stage the speculative token's selection, then correct it to the real
    # token's: the result must be the real selection's gather, byte for byte
    announce(f"sparsekv_gather_correct ({wl.name}, pool={wl.pool})")
    inp, st = run_step(wl)
    dev, pr = st.inp, st.pr
    Bn, Hkv, km = wl.batch, wl.n_kv_heads, pr.k_max
    shape = (Bn, Hkv, km, wl.block_size, wl.head_dim)
    fp8 = dev.k_scales is not None

    def stage():
        k = torch.zeros(shape, dtype=dev.k_pool.dtype, device="cuda")
        v = torch.zeros(shape, dtype=dev.v_pool.dtype, device="cuda")
        ks = torch.zeros((Bn, Hkv, km), dtype=torch.float32, device="cuda") if fp8 else None
        vs = torch.zeros((Bn, Hkv, km), dtype=torch.float32, device="cuda") if fp8 else None
        return k, v, ks, vs

    pools = (dev.k_pool, dev.v_pool, dev.k_scales, dev.v_scales, dev.block_table)
    none_n = torch.zeros_like(st.n_sel)
    spare, spec, out, ref = stage(), stage(), stage(), stage()
    miss_spec = torch.full((Bn, Hkv), -1, dtype=torch.int32, device="cuda")
    miss = torch.full((Bn, Hkv), -1, dtype=torch.int32, device="cuda")
    # an empty speculative row: every block of token 1 is a miss
    B.sparsekv_gather_correct(pr, *pools, st.indices, none_n, 0, spare[0], spare[1], spare[2], spare[3],
                              st.indices, st.n_sel, 1, *spec, misses=miss_spec)
    # the correction from token 1's stage to token 0's selection
    B.sparsekv_gather_correct(pr, *pools, st.indices, st.n_sel, 1, *spec, st.indices, st.n_sel, 0, *out,
                              misses=miss)
    B.sparsekv_gather(pr, *pools, st.indices, st.n_sel, *ref)
    torch.cuda.synchronize()

    from sparse_kv_cache_block_amd.inputs import raw_bytes
    idx, nsel = _np(st.indices), _np(st.n_sel)
    h = HostArrays(inp)
    oks, ovs, okss, ovss = O.gather(oracle_problem(inp, k_max=km), *h.pools(), h.block_table, idx, nsel)
    for b in range(Bn):
        for g in range(Hkv):
            n0, n1 = int(nsel[b, 0, g]), int(nsel[b, 1, g])
            common = len(set(idx[b, 0, g, :n0].tolist()) & set(idx[b, 1, g, :n1].tolist()))
            assert int(miss[b, g]) == n0 - common
            assert int(miss_spec[b, g]) == n1
            for a, r in ((out[0], ref[0]), (out[1], ref[1])):
                assert np.array_equal(raw_bytes(a)[b, g, :n0].view(np.uint8), raw_bytes(r)[b, g, :n0].view(np.uint8))
            assert np.array_equal(raw_bytes(out[0])[b, g, :n0].view(np.uint8), oks[b, g, :n0].view(np.uint8))
            assert np.array_equal(raw_bytes(out[1])[b, g, :n0].view(np.uint8), ovs[b, g, :n0].view(np.uint8))
            if fp8:
                assert np.array_equal(_np(out[2])[b, g, :n0], okss[b, g, :n0])
                assert np.array_equal(_np(out[3])[b, g, :n0], ovss[b, g, :n0])
    # a wrong prediction: every real id moved up by one (inside the candidates),
    # so hits fall at arbitrary slots and most blocks are misses
    L = _np(dev.seq_lens)
    bad = np.full_like(idx, -1)
    bad_n = np.zeros_like(nsel)
    for b in range(Bn):
        nc = -(-max(0, int(L[b]) - wl.window) // wl.block_size)
        for g in range(Hkv):
            ids = sorted({int(j) + 1 for j in idx[b, 0, g, :int(nsel[b, 0, g])] if int(j) + 1 < nc})
            bad[b, 0, g, :len(ids)] = ids
            bad_n[b, 0, g] = len(ids)
    bad_t, bad_nt = torch.from_numpy(bad).cuda(), torch.from_numpy(bad_n).cuda()
    wrong = stage()
    B.sparsekv_gather(pr, *pools, bad_t, bad_nt, *wrong)
    fixed = stage()
    B.sparsekv_gather_correct(pr, *pools, bad_t, bad_nt, 0, *wrong, st.indices, st.n_sel, 0, *fixed, misses=miss)
    torch.cuda.synchronize()
    for b in range(Bn):
        for g in range(Hkv):
            n0 = int(nsel[b, 0, g])
            hits = len(set(idx[b, 0, g, :n0].tolist()) & set(bad[b, 0, g, :int(bad_n[b, 0, g])].tolist()))
            assert int(miss[b, g]) == n0 - hits
            for a, r in zip(fixed, ref):
                if a is not None:
                    assert torch.equal(a[b, g, :n0], r[b, g, :n0])
    # identical selections: nothing is missed, the stage is moved as it is
    B.sparsekv_gather_correct(pr, *pools, st.indices, st.n_sel, 0, *ref, st.indices, st.n_sel, 0, *spare,
                              misses=miss)
    torch.cuda.synchronize()
    assert int(miss.abs().sum()) == 0
    for b in range(Bn):
        for g in range(Hkv):
            n0 = int(nsel[b, 0, g])
            assert torch.equal(spare[0][b, g, :n0], ref[0][b, g, :n0])


# ------------------------------------------------ hybrid CPU-GPU step
def check_hybrid(wl, seq_lens=None, n_threads=0):
    announce(f"decode_step_hybrid {wl.name} B={wl.batch} L={wl.context} kv={wl.kv_dtype} T={wl.n_q_tokens} "
             f"W={wl.window} seq_lens={seq_lens} threads={n_threads}")
    from sparse_kv_cache_block_amd.step import HybridHost
    inp, st = run_step(wl, seq_lens=seq_lens)   # the GPU host-pool step: gather, then attention
    ref_out, ref_lse, ref_idx = st.out.clone(), st.lse.clone(), st.indices.clone()
    host = HybridHost(st, n_threads)
    st.out.fill_(float("nan"))
    st.lse.fill_(float("nan"))
    st.run_hybrid(host)
    torch.cuda.synchronize()
    assert torch.equal(st.indices, ref_idx)
    # the same values as the all-GPU step (fp32 rounding apart) ...
    fin = torch.isfinite(ref_lse)
    assert torch.equal(fin, torch.isfinite(st.lse))
    assert bool(torch.all(st.lse[~fin] == -float("inf")))
    assert (st.out - ref_out).abs().max().item() <= 1e-4
    if fin.any():
        assert (st.lse[fin] - ref_lse[fin]).abs().max().item() <= 1e-4
    # ... and as the oracle on the same selection
    h = HostArrays(inp)
    err = compare_attention(inp, h, _np(st.indices), _np(st.n_sel), _np(st.out), _np(st.lse), TOL[wl.kv_dtype])
    print(f"[case] ok: max-abs err {err:.3g}", flush=True)


@pytest.mark.parametrize("wl,lens,threads", [
    (configs.HOST.scaled(batch=2, context=8192), None, 0),
    (configs.HOST.scaled(batch=3, context=8192, top_k=40), [8192, 700, 0], 3),
    (configs.HOST.scaled(batch=2, context=4096, window=0), None, 0),
    (configs.HOST.scaled(batch=2, context=4096, window=0, kv_dtype="fp8"), None, 0),
    (FP8_WIN, [8192, 300, 0], 0),
    (FP8_WIN.scaled(block_size=16, window=256), None, 2),
    (configs.HOST.scaled(batch=2, context=8192, n_q_tokens=2, spec_noise=0.3), None, 0),
    (configs.HOST.scaled(batch=2, context=4096, head_dim=64, block_size=32, n_q_heads=64), None, 2),
    (configs.HOST.scaled(batch=2, context=4096, n_q_heads=24, top_k=60), None, 0),       # G = 3, k > candidates
    (configs.HOST.scaled(batch=1, context=2048, kv_dtype="fp32", q_dtype="fp32", landmark_dtype="fp32",
                         block_size=16, window=64), None, 0),
])
def test_hybrid_step(wl, lens, threads):
    check_hybrid(wl, seq_lens=lens, n_threads=threads)


def test_hybrid_step_full_host_workload():
    check_hybrid(configs.HOST)


# ------------------------------------------------ host-pool layer pipelines
# Every layer gets its own input set (query, pinned pool, landmarks, table and
# window of another instance), so layers select different blocks and stage
# different bytes.  Both staging slots (and the predicted pipeline's stage) are
# filled with NaN before every call: a gather that ran late, a slot mix-up or
# an attention that did not wait for its gather reads NaN or another layer's
# blocks, and fails the per-layer comparison with the oracle.
_LAYER_INPUTS = {}


def layer_inputs(wl, n_layers):
    """Host copies and device placements of n_layers independent input sets."""
    key = (wl, n_layers)
    if key not in _LAYER_INPUTS:
        _LAYER_INPUTS.clear()
        host = [make_inputs(wl, device="cpu", instance=l) for l in range(n_layers)]
        _LAYER_INPUTS[key] = (host, [to_device_for(h) for h in host])
    return _LAYER_INPUTS[key]


def poison(tensors):
    """Fill with NaN: bf16 0x7FC0, fp8 e4m3fn 0x7F, fp32 NaN."""
    for t in tensors:
        if t.dtype == torch.bfloat16:
            t.view(torch.int16).fill_(0x7FC0)
        elif t.element_size() == 1:
            t.view(torch.uint8).fill_(0x7F)
        else:
            t.fill_(float("nan"))


def check_layers_against_oracle(wl, host, outs):
    """Each layer's selection, output and lse against the oracle's decode step on
    that layer's own inputs."""
    for l, (inp, o) in enumerate(zip(host, outs)):
        h = HostArrays(inp)
        orc = O.decode_step(oracle_problem(inp), h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens,
                            h.k_per_seq)
        gi, gn = _np(o["indices"]), _np(o["n_sel"])
        check_indices(gi, gn, orc["indices"], orc["n_sel"], orc["scores"], h.seq_lens, wl.window, wl.block_size)
        compare_attention(inp, h, gi, gn, _np(o["out"]), _np(o["lse"]), TOL[wl.kv_dtype])
    # the layers really differ (otherwise a slot mix-up could go unseen)
    if len(outs) > 1:
        assert not torch.equal(outs[0]["indices"], outs[1]["indices"])
        assert not torch.equal(outs[0]["out"], outs[1]["out"])


PIPE_WL = configs.HOST.scaled(batch=2, context=8192)


@pytest.mark.parametrize("n_layers", [2, 4, 8])
def test_host_layer_pipeline_per_layer_oracle(n_layers):
    announce(f"sparsekv_decode_layers, {n_layers} layers with their own inputs, poisoned slots")
    from sparse_kv_cache_block_amd.step import LayerPipeline
    host, dev = layer_inputs(PIPE_WL, 8)
    pipe = LayerPipeline(dev[:n_layers])
    poison(pipe.staging_buffers())
    pipe.run(copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    check_layers_against_oracle(PIPE_WL, host[:n_layers], pipe.outs)


def test_host_layer_pipeline_delayed_copy_stream():
    # the copy stream held up by a bounded spin kernel queued ahead of the
    # gathers, with NaN in both slots: every attention must still wait for its
    # own layer's gather (the events order them) and give the undelayed result
    announce("sparsekv_decode_layers, 5 layers, poisoned slots, delayed copy stream")
    from sparse_kv_cache_block_amd.step import LayerPipeline
    host, dev = layer_inputs(PIPE_WL, 8)
    pipe = LayerPipeline(dev[:5])
    poison(pipe.staging_buffers())
    pipe.run(copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    ref = [(o["out"].clone(), o["lse"].clone(), o["indices"].clone()) for o in pipe.outs]
    check_layers_against_oracle(PIPE_WL, host[:5], pipe.outs)
    for o in pipe.outs:
        o["out"].fill_(0)
    poison(pipe.staging_buffers())
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        torch.cuda._sleep(200_000_000)   # a bounded spin kernel, tens of ms
    pipe.run(copy_stream=cs)
    torch.cuda.synchronize()
    for o, (out, lse, idx) in zip(pipe.outs, ref):
        assert torch.equal(o["indices"], idx)
        assert torch.equal(o["out"], out) and torch.equal(o["lse"], lse)


def test_host_layer_pipeline_fp8_odd_layers():
    wl = configs.HOST.scaled(batch=2, context=4096, window=0, kv_dtype="fp8")
    announce("sparsekv_decode_layers, fp8 pool, 3 layers, poisoned slots and stage scales")
    from sparse_kv_cache_block_amd.step import LayerPipeline
    host, dev = layer_inputs(wl, 3)
    pipe = LayerPipeline(dev)
    poison(pipe.staging_buffers())
    pipe.run(copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    check_layers_against_oracle(wl, host, pipe.outs)


def test_host_layer_pipeline_fp8_window():
    wl = FP8_WIN.scaled(batch=2)
    announce("sparsekv_decode_layers, fp8 pool and window buffers, 3 layers, poisoned slots")
    from sparse_kv_cache_block_amd.step import LayerPipeline
    host, dev = layer_inputs(wl, 3)
    pipe = LayerPipeline(dev)
    poison(pipe.staging_buffers())
    pipe.run(copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    check_layers_against_oracle(wl, host, pipe.outs)


PRED_WL = configs.HOST.scaled(batch=2, context=8192, n_q_tokens=2, spec_noise=0.3)


def _expected_misses(real_idx, real_n, pred_idx, pred_n, token):
    Bn, _, Hkv, _ = real_idx.shape
    m = np.zeros((Bn, Hkv), dtype=np.int64)
    for b in range(Bn):
        for g in range(Hkv):
            r = set(real_idx[b, 0, g, :real_n[b, 0, g]].tolist())
            q = set(pred_idx[b, token, g, :pred_n[b, token, g]].tolist())
            m[b, g] = len(r - q)
    return m


def _run_predicted(pipe, preds, copy_stream):
    pipe.alloc_stage()
    poison(pipe.staging_buffers())
    for o in pipe.outs:
        o["misses"].fill_(-1)
        o["out"].fill_(0)
    pipe.run_predicted(preds, copy_stream=copy_stream)
    torch.cuda.synchronize()


@pytest.mark.parametrize("kind", ["speculative", "empty", "exact", "other_layer"])
def test_predicted_layer_pipeline(kind):
    # The prediction of layer l: the speculative token's selection of a
    # previous step on the same layer ("speculative"); nothing (every block a
    # miss); the real selection itself (no miss); another layer's selection
    # (hits only by chance).  Whatever it is, each layer's stage must hold the
    # real selection's gather, so results equal the plain pipeline's bit for
    # bit and the oracle's at the dtype's bound; misses match the set difference.
    n = 4
    announce(f"sparsekv_decode_layers_predicted, {n} layers, prediction = {kind}")
    from sparse_kv_cache_block_amd.step import LayerPipeline
    host, dev = layer_inputs(PRED_WL, n)
    plain = LayerPipeline(dev)
    poison(plain.staging_buffers())
    plain.run(copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    check_layers_against_oracle(PRED_WL, host, plain.outs)
    prev = [(o["indices"].clone(), o["n_sel"].clone()) for o in plain.outs]
    if kind == "speculative":
        preds = [(idx, nsel, 1) for idx, nsel in prev]
    elif kind == "empty":
        preds = [(idx, torch.zeros_like(nsel), 1) for idx, nsel in prev]
    elif kind == "exact":
        preds = [(idx, nsel, 0) for idx, nsel in prev]
    else:
        preds = [(prev[(l + 1) % n][0], prev[(l + 1) % n][1], 0) for l in range(n)]
    pipe = LayerPipeline(dev)
    _run_predicted(pipe, preds, torch.cuda.Stream())
    check_layers_against_oracle(PRED_WL, host, pipe.outs)
    total = 0
    for l, (o, p) in enumerate(zip(pipe.outs, plain.outs)):
        assert torch.equal(o["indices"], p["indices"]) and torch.equal(o["n_sel"], p["n_sel"])
        assert torch.equal(o["out"], p["out"]) and torch.equal(o["lse"], p["lse"])
        exp = _expected_misses(_np(o["indices"]), _np(o["n_sel"]), _np(preds[l][0]), _np(preds[l][1]), preds[l][2])
        assert np.array_equal(_np(o["misses"]), exp), (l, _np(o["misses"]), exp)
        total += int(exp.sum())
    nsel0 = sum(int(o["n_sel"][:, 0].sum()) for o in pipe.outs)
    if kind == "empty":
        assert total == nsel0
    elif kind == "exact":
        assert total == 0
    elif kind == "speculative":
        assert 0 < total < nsel0
    print(f"[case] ok: {total} of {nsel0} selected blocks missed", flush=True)


def test_predicted_layer_pipeline_delayed_copy_stream():
    # prefetches held up behind a bounded spin kernel, slots poisoned: each
    # correction must wait for its layer's prefetch (a hit read early would be NaN)
    announce("sparsekv_decode_layers_predicted, 5 layers, delayed copy stream, poisoned slots")
    from sparse_kv_cache_block_amd.step import LayerPipeline
    host, dev = layer_inputs(PRED_WL, 5)
    plain = LayerPipeline(dev)
    plain.run(copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    preds = [(o["indices"].clone(), o["n_sel"].clone(), 1) for o in plain.outs]
    pipe = LayerPipeline(dev)
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        torch.cuda._sleep(200_000_000)
    _run_predicted(pipe, preds, cs)
    check_layers_against_oracle(PRED_WL, host, pipe.outs)
    for o, p in zip(pipe.outs, plain.outs):
        assert torch.equal(o["out"], p["out"]) and torch.equal(o["lse"], p["lse"])


def test_predicted_layer_pipeline_fp8():
    wl = configs.HOST.scaled(batch=2, context=4096, window=0, kv_dtype="fp8", n_q_tokens=2, spec_noise=0.3)
    announce("sparsekv_decode_layers_predicted, fp8 pool, 3 layers")
    from sparse_kv_cache_block_amd.step import LayerPipeline
    host, dev = layer_inputs(wl, 3)
    plain = LayerPipeline(dev)
    plain.run(copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    preds = [(o["indices"].clone(), o["n_sel"].clone(), 1) for o in plain.outs]
    pipe = LayerPipeline(dev)
    _run_predicted(pipe, preds, torch.cuda.Stream())
    check_layers_against_oracle(wl, host, pipe.outs)
    for o, p in zip(pipe.outs, plain.outs):
        assert torch.equal(o["out"], p["out"]) and torch.equal(o["lse"], p["lse"])


def test_predicted_layer_pipeline_fp8_window():
    wl = FP8_WIN.scaled(batch=2, n_q_tokens=2, spec_noise=0.3)
    announce("sparsekv_decode_layers_predicted, fp8 pool and window buffers, 3 layers")
    from sparse_kv_cache_block_amd.step import LayerPipeline
    host, dev = layer_inputs(wl, 3)
    plain = LayerPipeline(dev)
    plain.run(copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    preds = [(o["indices"].clone(), o["n_sel"].clone(), 1) for o in plain.outs]
    pipe = LayerPipeline(dev)
    _run_predicted(pipe, preds, torch.cuda.Stream())
    check_layers_against_oracle(wl, host, pipe.outs)
    for o, p in zip(pipe.outs, plain.outs):
        assert torch.equal(o["out"], p["out"]) and torch.equal(o["lse"], p["lse"])


def test_repeated_calls_reuse_workspace():
    wl = configs.LLAMA32K.scaled(batch=2, context=4096)
    announce("repeated decode steps on one workspace")
    inp, st = run_step(wl)
    first = st.out.clone()
    for _ in range(3):
        st.run()
    torch.cuda.synchronize()
    assert torch.equal(first, st.out)


def test_alternating_inputs_share_one_workspace():
    # the single-launch step leaves its ticket counter, ready flags and merge
    # counters at zero; a stale flag would let a later call read the previous
    # call's selection, so two input sets alternate on one workspace
    for wl in (configs.LLAMA32K.scaled(batch=2, context=4096),
               configs.DUAL.scaled(batch=2, context=8192, top_k=30)):
        announce(f"alternating inputs on one workspace ({wl.name})")
        steps = [DecodeStep(to_device_for(make_inputs(wl, device="cpu", instance=i))) for i in range(2)]
        fresh = []
        for st in steps:
            st.run()
            torch.cuda.synchronize()
            fresh.append((st.indices.clone(), st.out.clone(), st.lse.clone()))
        steps[1].ws = steps[0].ws
        for _ in range(3):
            for st, (idx, out, lse) in zip(steps, fresh):
                st.run()
                torch.cuda.synchronize()
                assert torch.equal(st.indices, idx)
                assert torch.equal(st.out, out) and torch.equal(st.lse, lse)


# ------------------------------------------------------------ graph capture
@pytest.mark.parametrize("wl", [configs.LLAMA32K.scaled(batch=16, context=4096),          # one launch
                                configs.DUAL.scaled(batch=2, context=8192, top_k=30),      # two launches
                                TWO_LEVEL.scaled(n_q_tokens=2, spec_noise=0.3)])           # split step
def test_graph_replays_match_eager(wl):
    # the step enqueues no memset and its kernels return their counters to
    # zero, so a captured step replays exactly; eager work runs between replays
    announce(f"graph capture of decode_step {wl.name} B={wl.batch} L={wl.context}")
    inp, st = run_step(wl)
    ref = (st.out.clone(), st.lse.clone(), st.indices.clone(), st.n_sel.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.run()
    for _ in range(3):
        st.out.fill_(float("nan"))
        st.lse.fill_(float("nan"))
        st.indices.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        got = (st.out, st.lse, st.indices, st.n_sel)
        assert all(torch.equal(a, b) for a, b in zip(got, ref))
        st.run()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(got, ref))


@pytest.mark.parametrize("wl,names", [
    (configs.LLAMA32K.scaled(batch=16, context=4096), ["pair_step_kernel"]),
    (TWO_LEVEL.scaled(n_q_tokens=2, spec_noise=0.3), ["score_kernel", "split_step_kernel"]),
    (configs.DUAL.scaled(batch=2, context=8192, top_k=30), ["score_kernel", "attend_kernel"]),
], ids=["single_launch", "split_step", "two_launches"])
def test_launch_times_run_the_step(wl, names):
    """The per-launch timing entry point runs the very step: its outputs equal
    a plain decode step's bit for bit, and it reports one positive time per
    launch of the kernels the plan names."""
    announce(f"launch times {wl.name}")
    inp, st = run_step(wl, gen_device="cuda")
    ref = [_np(t).copy() for t in (st.indices, st.n_sel, st.out, st.lse)]
    for t in (st.indices, st.n_sel, st.out, st.lse):
        t.fill_(-7)
    us = B.sparsekv_decode_step_launch_times(st.pr, st.inputs, st.outputs, st.ws, 5)
    torch.cuda.synchronize()
    assert [B.sparsekv_decode_step_kernel(st.pr, i) for i in range(len(us))] == names
    assert len(us) == len(names) and all(u > 0 for u in us)
    for a, t in zip(ref, (st.indices, st.n_sel, st.out, st.lse)):
        assert np.array_equal(a, _np(t))


def test_concurrent_streams_keep_results():
    # the library keeps no state outside the caller's workspace: two steps with
    # their own workspaces, enqueued on two streams at once, give each one's
    # stand-alone result (one single-launch, one two-launch shape)
    announce("two decode steps on two streams at once")
    _, a = run_step(configs.LLAMA32K.scaled(batch=16, context=4096))
    _, b = run_step(configs.DUAL.scaled(batch=2, context=8192, top_k=30))
    ref = [(st.out.clone(), st.indices.clone()) for st in (a, b)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(5):
        for st in (a, b):
            st.out.fill_(float("nan"))
        torch.cuda.synchronize()
        for st, sm in zip((a, b), streams):
            st.run(stream=sm.cuda_stream)
        torch.cuda.synchronize()
        for st, (o, i) in zip((a, b), ref):
            assert torch.equal(st.out, o) and torch.equal(st.indices, i)


# ------------------------------------------------------------ full-size workloads
def test_stream_read_writes_nothing():
    """The read-ceiling probe reads a buffer (a ragged size: several grid
    strides plus a tail) and leaves its sink untouched."""
    announce("stream_read 3 MiB + 48 B")
    buf = torch.ones((3 << 20) + 48, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    B.sparsekv_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum().item()) == 0


@pytest.mark.parametrize("name", ["llama32k", "dual", "ragged", "host"])
def test_full_size_workload(name):
    wl = configs.get(name)
    check_step(wl, gen_device="cuda")
