"""The C-ABI library loads and exports every entry point its header declares,
and its host-side validation rejects bad arguments before any launch.
No GPU work is issued here."""
import ctypes as C
import os
import re

import pytest

from sparse_kv_cache_block_amd import binding as B
from sparse_kv_cache_block_amd import build as skv_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparsekv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        skv_build.build()
    return B.lib()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparsekv_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for name in ("sparsekv_score", "sparsekv_topk", "sparsekv_gather", "sparsekv_attend",
                 "sparsekv_decode_step"):
        assert name in syms
    assert set(syms) == set(B.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def _good_problem(**kw):
    base = dict(B=2, T=1, Hq=8, Hkv=2, d=128, blk=32, max_blocks=64, n_pool_blocks=128,
                stride_block=2 * 32 * 128, stride_head=32 * 128, window=64, k_max=8,
                q_dtype="bf16", kv_dtype="bf16", landmark_dtype="bf16")
    base.update(kw)
    return B.make_problem(base["B"], base["T"], base["Hq"], base["Hkv"], base["d"], base["blk"],
                          base["max_blocks"], base["n_pool_blocks"], base["stride_block"],
                          base["stride_head"], base["window"], base["k_max"], base["q_dtype"],
                          base["kv_dtype"], base["landmark_dtype"])


def test_workspace_size_is_host_only(lib):
    n = B.sparsekv_workspace_size(_good_problem())
    assert n > 0 and n % 256 == 0
    assert B.sparsekv_version().count(".") == 2


def test_decode_step_launch_count(lib):
    # one launch for the 32k Llama-shaped layer (256 pairs), two when the
    # pairs are too few to fill the chip or the shape has no step kernel,
    # three for a host pool
    big = dict(B=32, Hq=32, Hkv=8, max_blocks=1024, n_pool_blocks=32 * 1024, window=512, k_max=64)
    assert B.sparsekv_decode_step_launches(_good_problem(**big)) == 1
    assert B.sparsekv_decode_step_launches(_good_problem(**dict(big, kv_dtype="fp8"))) == 1
    assert B.sparsekv_decode_step_launches(_good_problem()) == 2
    assert B.sparsekv_decode_step_launches(_good_problem(**dict(big, d=64))) == 2
    assert B.sparsekv_decode_step_launches(_good_problem(**dict(big, blk=16))) == 2
    # a wave holds at most 64 items (one descriptor per lane): 17 window slices
    # over the 7 waves that do not select (3 in the first) plus ceil(k_max / 8)
    # selected ones; k_max 488 fills 64, 489 would need 65
    assert B.sparsekv_decode_step_launches(_good_problem(**dict(big, k_max=488))) == 1
    assert B.sparsekv_decode_step_launches(_good_problem(**dict(big, k_max=489))) == 2
    # two tokens: 6 window waves, still 3 slices in the first
    assert B.sparsekv_decode_step_launches(_good_problem(**dict(big, T=2, k_max=488))) == 1
    assert B.sparsekv_decode_step_launches(_good_problem(**dict(big, T=2, k_max=489))) == 2
    # a wider window: 129 slices over 7 waves (19 in the first) leave 45 for
    # the selected blocks, so k_max 360 still plans one launch and 361 two
    wide = dict(big, window=4096, max_blocks=1024)
    assert B.sparsekv_decode_step_launches(_good_problem(**dict(wide, k_max=360))) == 1
    assert B.sparsekv_decode_step_launches(_good_problem(**dict(wide, k_max=361))) == 2
    host = B.make_problem(32, 1, 32, 8, 128, 32, 1024, 32 * 1024, 8 * 32 * 128, 32 * 128, 512, 64,
                          "bf16", "bf16", "bf16", pool_location=B.SKV_POOL_HOST)
    assert B.sparsekv_decode_step_launches(host) == 3


def test_decode_step_kernel_names(lib):
    big = dict(B=32, Hq=32, Hkv=8, max_blocks=1024, n_pool_blocks=32 * 1024, window=512, k_max=64)
    assert B.sparsekv_decode_step_kernel(_good_problem(**big), 0) == "pair_step_kernel"
    # 4 pairs, 2 x 64 candidates: one chunk per pair, the scoring launch selects
    small = _good_problem()
    assert [B.sparsekv_decode_step_kernel(small, i) for i in range(2)] == ["score_kernel", "attend_kernel"]
    # the dual shape: 32 pairs, 4080 candidates in 8 chunks of 512, k 128: the
    # chunks keep their own top 128 and the attention launch selects
    dual = _good_problem(B=4, T=2, Hq=64, Hkv=8, blk=64, max_blocks=4096, n_pool_blocks=4 * 4096,
                         stride_block=8 * 64 * 128, stride_head=64 * 128, window=1024, k_max=128,
                         kv_dtype="fp8")
    assert B.sparsekv_decode_step_launches(dual) == 2
    assert [B.sparsekv_decode_step_kernel(dual, i) for i in range(2)] == ["score_kernel", "split_step_kernel"]
    host = B.make_problem(32, 1, 32, 8, 128, 32, 1024, 32 * 1024, 8 * 32 * 128, 32 * 128, 512, 64,
                          "bf16", "bf16", "bf16", pool_location=B.SKV_POOL_HOST)
    assert [B.sparsekv_decode_step_kernel(host, i) for i in range(3)] == \
        ["score_kernel", "gather_kernel", "attend_kernel"]
    for pr, bad in ((small, 2), (small, -1), (host, 3)):
        with pytest.raises(B.SkvError) as e:
            B.sparsekv_decode_step_kernel(pr, bad)
        assert e.value.status == B.SKV_E_SHAPE


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=6, Hkv=4), B.SKV_E_SHAPE),
    (dict(T=3), B.SKV_E_SHAPE),
    (dict(k_max=0), B.SKV_E_SHAPE),
    (dict(k_max=65), B.SKV_E_SHAPE),
    (dict(window=-1), B.SKV_E_SHAPE),
    (dict(d=96), B.SKV_E_UNSUPPORTED),
    (dict(blk=8), B.SKV_E_UNSUPPORTED),
    (dict(Hq=32, Hkv=2), B.SKV_E_UNSUPPORTED),
    (dict(kv_dtype="fp32"), B.SKV_E_UNSUPPORTED),
    (dict(q_dtype=7), B.SKV_E_DTYPE),
    (dict(max_blocks=20000, k_max=8), B.SKV_E_UNSUPPORTED),
])
def test_validation_rejects_before_launch(lib, kw, status):
    pr = _good_problem(**kw)
    n = C.c_size_t(0)
    assert lib.sparsekv_workspace_size(C.byref(pr), C.byref(n)) == status
    # a compute entry point with dummy (never dereferenced) pointers fails the same way
    dummy = 0x1000
    assert lib.sparsekv_score(C.byref(pr), dummy, dummy, dummy, dummy, None) == status
    assert len(B.sparsekv_last_error()) > 0


def test_null_pointers_rejected(lib):
    pr = _good_problem()
    assert lib.sparsekv_score(C.byref(pr), None, 0x1000, 0x1000, 0x1000, None) == B.SKV_E_NULL
    assert lib.sparsekv_topk(C.byref(pr), 0x1000, 0x1000, 0x1000, None, 0x1000, None, None) == B.SKV_E_NULL
    assert lib.sparsekv_score(None, 0x1000, 0x1000, 0x1000, 0x1000, None) == B.SKV_E_NULL


def test_workspace_too_small_rejected(lib):
    pr = _good_problem()
    src = B.KvSource(B.SKV_SRC_PAGED, 0x1000, 0x1000, None, None, 0x1000)
    st = lib.sparsekv_attend(C.byref(pr), 0x1000, C.byref(src), 0x1000, 0x1000, C.byref(src), 0x1000,
                             0x1000, None, 0x1000, 16, None)
    assert st == B.SKV_E_WORKSPACE


def test_window_buffer_needs_aligned_window(lib):
    pr = _good_problem(window=48)
    n = B.sparsekv_workspace_size(pr)
    src = B.KvSource(B.SKV_SRC_PAGED, 0x1000, 0x1000, None, None, 0x1000)
    win = B.KvSource(B.SKV_SRC_WINDOW, 0x1000, 0x1000, None, None, None)
    st = lib.sparsekv_attend(C.byref(pr), 0x1000, C.byref(src), 0x1000, 0x1000, C.byref(win), 0x1000,
                             0x1000, None, 0x1000, n, None)
    assert st == B.SKV_E_SHAPE


def test_fp8_needs_scales(lib):
    pr = _good_problem(kv_dtype="fp8")
    n = B.sparsekv_workspace_size(pr)
    src = B.KvSource(B.SKV_SRC_PAGED, 0x1000, 0x1000, None, None, 0x1000)
    st = lib.sparsekv_attend(C.byref(pr), 0x1000, C.byref(src), 0x1000, 0x1000, C.byref(src), 0x1000,
                             0x1000, None, 0x1000, n, None)
    assert st == B.SKV_E_NULL


def _gather_correct(lib, pr, spec_token=0, real_token=0, spec_indices=0x1000, spec_stage=0x200000,
                    out_stage=0x100000000, scales=None):
    d = 0x1000
    return lib.sparsekv_gather_correct(C.byref(pr), d, d, scales, scales, d, spec_indices, d, spec_token,
                                       spec_stage, spec_stage, scales, scales, d, d, real_token,
                                       out_stage, out_stage, scales, scales, None, None)


def test_gather_correct_validation(lib):
    pr = _good_problem(T=2)
    # every check runs on the host, before any launch
    assert _gather_correct(lib, pr, spec_indices=None) == B.SKV_E_NULL
    assert _gather_correct(lib, pr, spec_token=2) == B.SKV_E_SHAPE
    assert _gather_correct(lib, pr, real_token=-1) == B.SKV_E_SHAPE
    # stage bytes: B * Hkv * k_max * blk * d * 2 = 2*2*8*32*128*2 = 256 KiB: overlapping ranges
    assert _gather_correct(lib, pr, spec_stage=0x200000, out_stage=0x200000 + 0x1000) == B.SKV_E_SHAPE
    assert _gather_correct(lib, _good_problem(T=2, kv_dtype="fp8")) == B.SKV_E_NULL
    assert "gather_correct" in B.sparsekv_last_error()


def _attend_cobatched(lib, pr, kind=None, ws_bytes=None):
    d = 0x1000
    src = B.KvSource(B.SKV_SRC_PAGED if kind is None else kind, d, d, d, d, d)
    n = ws_bytes if ws_bytes is not None else B.sparsekv_workspace_size(pr)
    return lib.sparsekv_attend_cobatched(C.byref(pr), d, C.byref(src), d, d, C.byref(src), d, d, None, d, n,
                                         None)


def test_attend_cobatched_validation(lib):
    pr = _good_problem(T=2)
    # every check runs on the host, before any launch
    assert _attend_cobatched(lib, pr, kind=B.SKV_SRC_STAGED) == B.SKV_E_UNSUPPORTED
    assert "paged" in B.sparsekv_last_error()
    assert _attend_cobatched(lib, pr, ws_bytes=16) == B.SKV_E_WORKSPACE
    host = B.make_problem(2, 2, 8, 2, 128, 32, 64, 128, 2 * 32 * 128, 32 * 128, 64, 8, "bf16", "bf16", "bf16",
                          pool_location=B.SKV_POOL_HOST)
    assert _attend_cobatched(lib, host) == B.SKV_E_UNSUPPORTED
    # the largest selections plan without error (stopped at the workspace
    # check: no launch is issued here)
    big = _good_problem(T=2, Hq=16, Hkv=2, d=64, blk=64, max_blocks=16384, n_pool_blocks=16384,
                        stride_block=2 * 64 * 64, stride_head=64 * 64, k_max=16384)
    assert B.sparsekv_workspace_size(big) > 0
    assert _attend_cobatched(lib, big, ws_bytes=16) == B.SKV_E_WORKSPACE


def test_workspace_covers_cobatched_partials(lib):
    one = B.sparsekv_workspace_size(_good_problem(T=1, Hq=16, Hkv=2))
    two = B.sparsekv_workspace_size(_good_problem(T=2, Hq=16, Hkv=2))
    assert two > one


def test_hybrid_step_validation(lib):
    # every check runs on the host, before any GPU call
    d = 0x1000
    ins = B.StepInputs(d, d, d, d, d, d, d, d, d, d, d)
    outs = B.StepOutputs(d, d, d, d, None)
    host = B.HostPart(d, d, 0, d, d, d, d, d, None, None, d, d)
    dev = _good_problem()
    n = B.sparsekv_workspace_size(dev)
    assert lib.sparsekv_decode_step_hybrid(C.byref(dev), C.byref(ins), C.byref(outs), C.byref(host), d, n,
                                           None) == B.SKV_E_UNSUPPORTED
    hp = B.make_problem(2, 1, 8, 2, 128, 32, 64, 128, 2 * 32 * 128, 32 * 128, 64, 8, "bf16", "bf16", "bf16",
                        pool_location=B.SKV_POOL_HOST)
    n = B.sparsekv_workspace_size(hp)
    assert lib.sparsekv_decode_step_hybrid(C.byref(hp), C.byref(ins), C.byref(outs), None, d, n,
                                           None) == B.SKV_E_NULL
    no_o = B.HostPart(d, d, 0, d, d, d, d, d, None, None, None, d)
    assert lib.sparsekv_decode_step_hybrid(C.byref(hp), C.byref(ins), C.byref(outs), C.byref(no_o), d, n,
                                           None) == B.SKV_E_NULL
    fp8 = B.make_problem(2, 1, 8, 2, 128, 32, 64, 128, 2 * 32 * 128, 32 * 128, 64, 8, "bf16", "fp8", "bf16",
                         pool_location=B.SKV_POOL_HOST)
    host8 = B.HostPart(d, d, 0, d, d, d, d, d, d, d, d, d)
    # fp8 window buffers need their per-row scales, 16-byte aligned
    assert lib.sparsekv_decode_step_hybrid(C.byref(fp8), C.byref(ins), C.byref(outs), C.byref(host8), d,
                                           B.sparsekv_workspace_size(fp8), None) == B.SKV_E_NULL
    assert "per-row scales" in B.sparsekv_last_error()
    ins8 = B.StepInputs(d, d, d, d, d, d, d, d, d, d, d, d, d + 4)
    assert lib.sparsekv_decode_step_hybrid(C.byref(fp8), C.byref(ins8), C.byref(outs), C.byref(host8), d,
                                           B.sparsekv_workspace_size(fp8), None) == B.SKV_E_SHAPE
    assert "aligned" in B.sparsekv_last_error()
    assert lib.sparsekv_decode_step_hybrid(C.byref(hp), C.byref(ins), C.byref(outs), C.byref(host), d, 16,
                                           None) == B.SKV_E_WORKSPACE


def test_stream_read_validates_before_launch(lib):
    vp = C.c_void_p
    lib.sparsekv_stream_read.argtypes = [vp, C.c_size_t, vp, C.c_size_t, vp]
    assert lib.sparsekv_stream_read(None, 16, 0x1000, 4, None) == B.SKV_E_NULL
    assert lib.sparsekv_stream_read(0x1000, 16, None, 4, None) == B.SKV_E_NULL
    assert lib.sparsekv_stream_read(0x1000, 15, 0x1000, 4, None) == B.SKV_E_SHAPE
    assert lib.sparsekv_stream_read(0x1008, 16, 0x1000, 4, None) == B.SKV_E_SHAPE
    assert lib.sparsekv_stream_read(0x1000, 16, 0x1000, 2, None) == B.SKV_E_SHAPE
    assert len(B.sparsekv_last_error()) > 0


# ---------------------------------------------------------------- LDS limits
# The selection keeps a pair's keys in one workgroup's 160 KiB of LDS; shapes
# beyond it fail with SKV_E_UNSUPPORTED before any launch.  Each case probes
# both sides of the limit: just inside it, the call gets past the LDS check
# and stops at the (too small) workspace or at a NULL pointer instead.
D = 0x1000


def _step_args():
    ins = B.StepInputs(D, D, D, D, D, D, D, D, D, None, None)
    outs = B.StepOutputs(D, D, D, D, D)
    return ins, outs


def _decode_step(lib, pr, ws_bytes=16):
    ins, outs = _step_args()
    return lib.sparsekv_decode_step(C.byref(pr), C.byref(ins), C.byref(outs), D, D, None, None, D, ws_bytes,
                                    None, None)


def test_launch_times_checks_before_any_gpu_work(lib):
    """The timing aid rejects its bad arguments on the host (no GPU here)."""
    ins, outs = _step_args()
    pr = _good_problem()
    ws = B.sparsekv_workspace_size(pr)
    us = (C.c_float * 2)()

    def call(p, n_steps=5, out=us, ws_bytes=ws):
        return lib.sparsekv_decode_step_launch_times(C.byref(p), C.byref(ins), C.byref(outs), D, ws_bytes,
                                                     None, n_steps, out)
    assert call(pr, out=None) == B.SKV_E_NULL
    assert call(pr, n_steps=0) == B.SKV_E_SHAPE and call(pr, n_steps=4097) == B.SKV_E_SHAPE
    assert call(pr, ws_bytes=16) == B.SKV_E_WORKSPACE
    host = B.make_problem(2, 1, 8, 2, 128, 32, 64, 128, 2 * 32 * 128, 32 * 128, 64, 8, "bf16", "bf16", "bf16",
                          pool_location=B.SKV_POOL_HOST)
    assert call(host) == B.SKV_E_UNSUPPORTED


def _limit_problem(T, k_max, B_=1, **kw):
    # 16384 blocks of 64 tokens, window 256: 16380 candidates per sequence
    base = dict(B=B_, T=T, Hq=32, Hkv=8, blk=64, max_blocks=16384, n_pool_blocks=16384 * B_,
                stride_block=8 * 64 * 128, stride_head=64 * 128, window=256, k_max=k_max)
    base.update(kw)
    return _good_problem(**base)


@pytest.mark.parametrize("T,k_ok,k_bad", [(2, 3187, 3188), (1, 11441, 11442)])
def test_selection_lds_limit_two_launch_step(lib, T, k_ok, k_bad):
    # 8 pairs: the two-launch step, whose scoring workgroups select
    assert _decode_step(lib, _limit_problem(T, k_ok)) == B.SKV_E_WORKSPACE
    assert _decode_step(lib, _limit_problem(T, k_bad)) == B.SKV_E_UNSUPPORTED
    assert "LDS" in B.sparsekv_last_error()


def test_selection_lds_limit_many_pairs(lib):
    # T = 2 with 16380 candidates and k_max 4096 at 256 pairs: too big for the
    # single-launch step, and its two-launch selection does not fit either
    pr = _limit_problem(2, 4096, B_=32)
    assert B.sparsekv_decode_step_launches(pr) == 2
    assert _decode_step(lib, pr) == B.SKV_E_UNSUPPORTED
    # the single-launch step keeps its own LDS check: a fitting shape plans
    assert B.sparsekv_decode_step_launches(_limit_problem(1, 64, B_=32, blk=32, max_blocks=1024,
                                                          stride_block=8 * 32 * 128, stride_head=32 * 128,
                                                          window=512)) == 1


def test_topk_lds_limit(lib):
    ok = _good_problem(max_blocks=16384, n_pool_blocks=16384, k_max=11759)
    bad = _good_problem(max_blocks=16384, n_pool_blocks=16384, k_max=11760)
    # inside the limit the call reaches the pointer checks; beyond it, it stops first
    assert lib.sparsekv_topk(C.byref(ok), D, D, D, None, D, None, None) == B.SKV_E_NULL
    assert lib.sparsekv_topk(C.byref(bad), D, D, D, None, D, None, None) == B.SKV_E_UNSUPPORTED
    bad12k = _good_problem(max_blocks=16384, n_pool_blocks=16384, k_max=12000)
    assert lib.sparsekv_topk(C.byref(bad12k), D, D, D, D, D, None, None) == B.SKV_E_UNSUPPORTED


def test_hybrid_and_layers_check_selection_lds(lib):
    pr = _limit_problem(2, 4096)
    pr.pool_location = B.SKV_POOL_HOST
    ins = B.StepInputs(D, D, D, D, D, D, D, D, D, D, D)
    outs = B.StepOutputs(D, D, D, D, D)
    host = B.HostPart(D, D, 0, D, D, D, D, D, None, None, D, D)
    assert lib.sparsekv_decode_step_hybrid(C.byref(pr), C.byref(ins), C.byref(outs), C.byref(host), D, 16,
                                           None) == B.SKV_E_UNSUPPORTED
    slots = (C.c_void_p * 2)(D, D)
    assert lib.sparsekv_decode_layers(C.byref(pr), 1, C.byref(ins), C.byref(outs), slots, slots, None, None,
                                      D, 16, None, None) == B.SKV_E_UNSUPPORTED


# ------------------------------------------------ host-pool checks before enqueue
def _host_problem(**kw):
    base = dict(B=2, T=1, Hq=8, Hkv=2, d=128, blk=32, max_blocks=64, n_pool_blocks=128, window=64, k_max=8,
                kv_dtype="bf16")
    base.update(kw)
    return B.make_problem(base["B"], base["T"], base["Hq"], base["Hkv"], base["d"], base["blk"],
                          base["max_blocks"], base["n_pool_blocks"], base["blk"] * base["d"],
                          base["n_pool_blocks"] * base["blk"] * base["d"], base["window"], base["k_max"],
                          "bf16", base["kv_dtype"], "bf16", pool_location=B.SKV_POOL_HOST)


@pytest.mark.parametrize("kw,scales,status,text", [
    (dict(kv_dtype="fp8"), (None, None), B.SKV_E_NULL, "per-row scales"),
    (dict(kv_dtype="fp8"), (D, None), B.SKV_E_NULL, "per-row scales"),
    (dict(kv_dtype="fp8"), (D, D + 8), B.SKV_E_SHAPE, "aligned"),
    (dict(window=48), (None, None), B.SKV_E_SHAPE, "window"),
])
def test_host_pool_window_checked_before_any_launch(lib, kw, scales, status, text):
    # the window-source checks run before the scoring launch (dummy pointers:
    # a launch would fail here with SKV_E_HIP, not with these statuses)
    pr = _host_problem(**kw)
    n = B.sparsekv_workspace_size(pr)
    ins = B.StepInputs(D, D, D, D, D, D, D, D, D, D, D, *scales)
    outs = B.StepOutputs(D, D, D, D, None)
    assert lib.sparsekv_decode_step(C.byref(pr), C.byref(ins), C.byref(outs), D, D, D, D, D, n, None,
                                    None) == status
    assert text in B.sparsekv_last_error()
    slots = (C.c_void_p * 2)(D, D)
    ins3 = (B.StepInputs * 3)(ins, ins, ins)
    outs3 = (B.StepOutputs * 3)(outs, outs, outs)
    assert lib.sparsekv_decode_layers(C.byref(pr), 3, ins3, outs3, slots, slots, slots, slots, D, n, None,
                                      None) == status
    preds = (B.LayerPrediction * 3)(*[B.LayerPrediction(D, D, 0, None)] * 3)
    assert lib.sparsekv_decode_layers_predicted(C.byref(pr), 3, ins3, outs3, preds, slots, slots, slots, slots,
                                                0x10000000, 0x20000000, D, D, D, n, None, None) == status


def test_fp8_window_buffers_rejected_for_device_pools(lib):
    # the device pool's fused step reads the window from the pool itself
    pr = _good_problem(kv_dtype="fp8")
    n = B.sparsekv_workspace_size(pr)
    ins = B.StepInputs(D, D, D, D, D, D, D, D, D, D, D, D, D)
    outs = B.StepOutputs(D, D, D, D, None)
    assert lib.sparsekv_decode_step(C.byref(pr), C.byref(ins), C.byref(outs), None, None, None, None, D, n,
                                    None, None) == B.SKV_E_UNSUPPORTED
    assert "host pools only" in B.sparsekv_last_error()
    assert lib.sparsekv_decode_step_noalloc(C.byref(pr), C.byref(ins), C.byref(outs), None) == B.SKV_E_UNSUPPORTED


def test_host_pool_staging_checked_before_any_launch(lib):
    pr = _host_problem()
    n = B.sparsekv_workspace_size(pr)
    ins = B.StepInputs(D, D, D, D, D, D, D, D, D, D, D)
    outs = B.StepOutputs(D, D, D, D, None)
    assert lib.sparsekv_decode_step(C.byref(pr), C.byref(ins), C.byref(outs), None, D, None, None, D, n, None,
                                    None) == B.SKV_E_NULL
    assert lib.sparsekv_decode_step(C.byref(pr), C.byref(ins), C.byref(outs), 0x1008, D, None, None, D, n,
                                    None, None) == B.SKV_E_SHAPE
    assert "aligned" in B.sparsekv_last_error()


def test_predicted_layers_validation(lib):
    pr = _host_problem(T=2)
    n = B.sparsekv_workspace_size(pr)
    ins = B.StepInputs(D, D, D, D, D, D, D, D, D, D, D)
    outs = B.StepOutputs(D, D, D, D, None)
    ins2 = (B.StepInputs * 2)(ins, ins)
    outs2 = (B.StepOutputs * 2)(outs, outs)
    slots = (C.c_void_p * 2)(0x1000000, 0x2000000)

    def call(preds, stage=0x30000000, problem=pr, ws=n):
        arr = (B.LayerPrediction * 2)(*preds)
        return lib.sparsekv_decode_layers_predicted(C.byref(problem), 2, ins2, outs2, arr, slots, slots, None,
                                                    None, stage, stage, None, None, D, ws, None, None)

    good = B.LayerPrediction(D, D, 1, None)
    assert call([good, B.LayerPrediction(None, D, 1, None)]) == B.SKV_E_NULL
    assert call([good, B.LayerPrediction(D, D, 2, None)]) == B.SKV_E_SHAPE
    # the real stage may not overlap a prefetch slot (a hit reads one while the stage is written)
    assert call([good, good], stage=0x2000000 + 0x100) == B.SKV_E_SHAPE
    assert "overlaps" in B.sparsekv_last_error()
    assert call([good, good], ws=16) == B.SKV_E_WORKSPACE
    dev = _good_problem(T=2)
    assert call([good, good], problem=dev) == B.SKV_E_UNSUPPORTED


# ---------------------------------------------------------------- alignment
def test_pool_strides_must_be_16_byte_multiples(lib):
    # bf16 elements: a stride of 4 elements is 8 bytes
    n = C.c_size_t(0)
    pr = _good_problem(stride_block=2 * 32 * 128 + 4)
    assert lib.sparsekv_workspace_size(C.byref(pr), C.byref(n)) == B.SKV_E_SHAPE
    pr = _good_problem(kv_dtype="fp8", stride_head=32 * 128 + 8)
    assert lib.sparsekv_workspace_size(C.byref(pr), C.byref(n)) == B.SKV_E_SHAPE
    assert lib.sparsekv_workspace_size(C.byref(_good_problem(kv_dtype="fp8", stride_head=32 * 128 + 16)),
                                       C.byref(n)) == B.SKV_OK


def test_vector_buffers_must_be_16_byte_aligned(lib):
    pr = _good_problem()
    assert lib.sparsekv_score(C.byref(pr), 0x1008, D, D, D, None) == B.SKV_E_SHAPE
    assert lib.sparsekv_score(C.byref(pr), D, 0x1004, D, D, None) == B.SKV_E_SHAPE
    assert lib.sparsekv_gather(C.byref(pr), D, 0x1002, None, None, D, D, D, D, D, None, None, None) == B.SKV_E_SHAPE
    n = B.sparsekv_workspace_size(pr)
    src = B.KvSource(B.SKV_SRC_PAGED, 0x1010, 0x1008, None, None, D)
    ok = B.KvSource(B.SKV_SRC_PAGED, D, D, None, None, D)
    assert lib.sparsekv_attend(C.byref(pr), D, C.byref(src), D, D, C.byref(ok), D, D, None, D, n,
                               None) == B.SKV_E_SHAPE
    assert lib.sparsekv_attend(C.byref(pr), 0x1001, C.byref(ok), D, D, C.byref(ok), D, D, None, D, n,
                               None) == B.SKV_E_SHAPE
    ins = B.StepInputs(D, D, 0x1004, D, None, None, D, D, D, None, None)
    outs = B.StepOutputs(D, D, D, D, None)
    assert lib.sparsekv_decode_step(C.byref(pr), C.byref(ins), C.byref(outs), None, None, None, None, D, n,
                                    None, None) == B.SKV_E_SHAPE


def test_noalloc_step_rejects_host_pools_and_oversized_problems(lib):
    # both checks run on the host before any HIP call
    ins = B.StepInputs(D, D, D, D, D, D, D, D, D, D, D)
    outs = B.StepOutputs(D, D, D, D, None)
    assert lib.sparsekv_decode_step_noalloc(C.byref(_host_problem()), C.byref(ins), C.byref(outs),
                                            None) == B.SKV_E_UNSUPPORTED
    # 512 pairs x 2 tokens x 16380 candidates of score staging: beyond the 32 MiB array
    big = _limit_problem(2, 16, B_=64, Hq=64)
    assert B.sparsekv_workspace_size(big) > 32 << 20
    assert lib.sparsekv_decode_step_noalloc(C.byref(big), C.byref(ins), C.byref(outs), None) == B.SKV_E_WORKSPACE
    assert "workspace" in B.sparsekv_last_error()
    # a problem that fits gets past every check (stopped here by a NULL output)
    no_out = B.StepOutputs(D, D, None, D, None)
    assert lib.sparsekv_decode_step_noalloc(C.byref(_good_problem()), C.byref(ins), C.byref(no_out),
                                            None) == B.SKV_E_NULL
