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
    # more items per (sequence, KV head) than one workgroup's 8 x 64 descriptors
    assert B.sparsekv_decode_step_launches(_good_problem(**dict(big, k_max=495))) == 1
    assert B.sparsekv_decode_step_launches(_good_problem(**dict(big, k_max=496))) == 2
    host = B.make_problem(32, 1, 32, 8, 128, 32, 1024, 32 * 1024, 8 * 32 * 128, 32 * 128, 512, 64,
                          "bf16", "bf16", "bf16", pool_location=B.SKV_POOL_HOST)
    assert B.sparsekv_decode_step_launches(host) == 3


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
    assert lib.sparsekv_decode_step_hybrid(C.byref(fp8), C.byref(ins), C.byref(outs), C.byref(host8), d,
                                           B.sparsekv_workspace_size(fp8), None) == B.SKV_E_UNSUPPORTED
    assert "fp8 window" in B.sparsekv_last_error()
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
