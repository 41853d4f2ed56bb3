"""ctypes wrapper of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg may use it; the product path never does.
It imports nothing from the HIP package.  Arrays in and out are numpy; raw
encodings are passed as their bit patterns (bf16 as uint16, fp8 as uint8).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
DTYPE_CODE = {"fp32": 0, "bf16": 1, "fp8": 2}
# Host AddressSanitizer + UndefinedBehaviorSanitizer build (clang, LLVM OpenMP),
# selected with SKV_ORACLE_LIB for a sanitized CPU test run.
SAN_LIB = os.path.join(_HERE, "_asan", "liboracle.so")


def build_sanitized() -> str:
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    subprocess.check_call(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-fno-omit-frame-pointer", "-fsanitize=address", "-fsanitize=undefined",
                           "-fno-sanitize-recover=undefined", "-o", SAN_LIB, os.path.join(_HERE, "oracle.c"),
                           "-lm", "-L/opt/rocm/llvm/lib", "-Wl,-rpath,/opt/rocm/llvm/lib"])
    return SAN_LIB


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP over (b, g))."""
    if os.environ.get("SKV_ORACLE_LIB"):
        return os.environ["SKV_ORACLE_LIB"]
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < max(
            os.path.getmtime(src), os.path.getmtime(os.path.join(_HERE, "oracle.h"))):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, src, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class Problem(C.Structure):
    _fields_ = [("B", C.c_int32), ("T", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32),
                ("d", C.c_int32), ("blk", C.c_int32), ("max_blocks", C.c_int32),
                ("n_pool_blocks", C.c_int32), ("stride_block", C.c_int64),
                ("stride_head", C.c_int64), ("window", C.c_int32), ("k_max", C.c_int32),
                ("q_dtype", C.c_int32), ("kv_dtype", C.c_int32), ("lm_dtype", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        L = C.CDLL(build())
        L.orc_bf16_value.restype = C.c_double
        L.orc_bf16_value.argtypes = [C.c_uint16]
        L.orc_e4m3fn_value.restype = C.c_double
        L.orc_e4m3fn_value.argtypes = [C.c_uint8]
        L.orc_max_threads.restype = C.c_int
        L.orc_set_threads.argtypes = [C.c_int]
        L.orc_partial.argtypes = [C.POINTER(Problem)] + [C.c_void_p] * 6 + [
            C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]
        L.orc_merge.argtypes = [C.c_int, C.c_int] + [C.c_void_p] * 4
        _lib = L
    return _lib


def problem(B, T, Hq, Hkv, d, blk, max_blocks, n_pool_blocks, stride_block, stride_head,
            window, k_max, q_dtype, kv_dtype, lm_dtype) -> Problem:
    return Problem(B, T, Hq, Hkv, d, blk, max_blocks, n_pool_blocks, stride_block, stride_head,
                   window, k_max, DTYPE_CODE[q_dtype], DTYPE_CODE[kv_dtype], DTYPE_CODE[lm_dtype])


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def bf16_value(code: int) -> float:
    return lib().orc_bf16_value(int(code))


def e4m3fn_value(code: int) -> float:
    return lib().orc_e4m3fn_value(int(code))


def n_candidates(pr: Problem, L: int) -> int:
    return lib().orc_n_candidates(C.byref(pr), int(L))


def scores(pr: Problem, q, landmarks, seq_lens) -> np.ndarray:
    out = np.empty((pr.B, pr.T, pr.Hkv, pr.max_blocks), dtype=np.float64)
    sl = _i32(seq_lens)
    lib().orc_scores(C.byref(pr), _p(q), _p(landmarks), _p(sl), _p(out))
    return out


def select(pr: Problem, sc: np.ndarray, seq_lens, k_per_seq):
    idx = np.empty((pr.B, pr.T, pr.Hkv, pr.k_max), dtype=np.int32)
    nsel = np.empty((pr.B, pr.T, pr.Hkv), dtype=np.int32)
    sc = np.ascontiguousarray(sc, dtype=np.float64)
    sl, kp = _i32(seq_lens), _i32(k_per_seq)
    lib().orc_select(C.byref(pr), _p(sc), _p(sl), _p(kp), _p(idx), _p(nsel))
    return idx, nsel


def overlap(pr: Problem, idx, nsel) -> np.ndarray:
    out = np.empty((pr.B, pr.Hkv), dtype=np.float64)
    idx, nsel = _i32(idx), _i32(nsel)
    lib().orc_overlap(C.byref(pr), _p(idx), _p(nsel), _p(out))
    return out


def gather(pr: Problem, k_pool, v_pool, k_scales, v_scales, block_table, idx, nsel):
    shape = (pr.B, pr.Hkv, pr.k_max, pr.blk, pr.d)
    ks = np.zeros(shape, dtype=k_pool.dtype)
    vs = np.zeros(shape, dtype=v_pool.dtype)
    kss = np.zeros((pr.B, pr.Hkv, pr.k_max), dtype=np.float32)
    vss = np.zeros((pr.B, pr.Hkv, pr.k_max), dtype=np.float32)
    bt, idx, nsel = _i32(block_table), _i32(idx), _i32(nsel)
    lib().orc_gather(C.byref(pr), _p(k_pool), _p(v_pool), _p(k_scales), _p(v_scales), _p(bt),
                     _p(idx), _p(nsel), _p(ks), _p(vs), _p(kss), _p(vss))
    return ks, vs, kss, vss


def partial(pr: Problem, q, k_pool, v_pool, k_scales, v_scales, block_table, b, h, positions):
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    o = np.empty(pr.d, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    bt = _i32(block_table)
    lib().orc_partial(C.byref(pr), _p(q), _p(k_pool), _p(v_pool), _p(k_scales), _p(v_scales),
                      _p(bt), int(b), int(h), _p(pos), int(pos.size), _p(o), _p(lse))
    return o, float(lse[0])


def merge(o_parts, lse_parts):
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n, d = o_parts.shape
    o = np.empty(d, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    lib().orc_merge(int(n), int(d), _p(o_parts), _p(lse_parts), _p(o), _p(lse))
    return o, float(lse[0])


def attend(pr: Problem, q, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens, idx, nsel,
           want_parts: bool = False):
    out = np.empty((pr.B, pr.Hq, pr.d), dtype=np.float64)
    lse = np.empty((pr.B, pr.Hq), dtype=np.float64)
    po = np.empty((pr.B, pr.Hq, 2, pr.d), dtype=np.float64) if want_parts else None
    pl = np.empty((pr.B, pr.Hq, 2), dtype=np.float64) if want_parts else None
    bt, sl, idx, nsel = _i32(block_table), _i32(seq_lens), _i32(idx), _i32(nsel)
    lib().orc_attend(C.byref(pr), _p(q), _p(k_pool), _p(v_pool), _p(k_scales), _p(v_scales),
                     _p(bt), _p(sl), _p(idx), _p(nsel), _p(out), _p(lse), _p(po), _p(pl))
    if want_parts:
        return out, lse, po, pl
    return out, lse


def attend_tokens(pr: Problem, q, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens, idx, nsel):
    """Every query token over its own selection plus the window: out [B][T][Hq][d], lse [B][T][Hq]."""
    out = np.empty((pr.B, pr.T, pr.Hq, pr.d), dtype=np.float64)
    lse = np.empty((pr.B, pr.T, pr.Hq), dtype=np.float64)
    bt, sl, idx, nsel = _i32(block_table), _i32(seq_lens), _i32(idx), _i32(nsel)
    lib().orc_attend_tokens(C.byref(pr), _p(q), _p(k_pool), _p(v_pool), _p(k_scales), _p(v_scales),
                            _p(bt), _p(sl), _p(idx), _p(nsel), _p(out), _p(lse))
    return out, lse


def dense(pr: Problem, q, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens):
    out = np.empty((pr.B, pr.Hq, pr.d), dtype=np.float64)
    lse = np.empty((pr.B, pr.Hq), dtype=np.float64)
    bt, sl = _i32(block_table), _i32(seq_lens)
    lib().orc_dense(C.byref(pr), _p(q), _p(k_pool), _p(v_pool), _p(k_scales), _p(v_scales),
                    _p(bt), _p(sl), _p(out), _p(lse))
    return out, lse


def decode_step(pr: Problem, q, landmarks, k_pool, v_pool, k_scales, v_scales, block_table,
                seq_lens, k_per_seq) -> dict:
    sc = np.empty((pr.B, pr.T, pr.Hkv, pr.max_blocks), dtype=np.float64)
    idx = np.empty((pr.B, pr.T, pr.Hkv, pr.k_max), dtype=np.int32)
    nsel = np.empty((pr.B, pr.T, pr.Hkv), dtype=np.int32)
    out = np.empty((pr.B, pr.Hq, pr.d), dtype=np.float64)
    lse = np.empty((pr.B, pr.Hq), dtype=np.float64)
    ov = np.empty((pr.B, pr.Hkv), dtype=np.float64) if pr.T == 2 else None
    bt, sl, kp = _i32(block_table), _i32(seq_lens), _i32(k_per_seq)
    lib().orc_decode_step(C.byref(pr), _p(q), _p(landmarks), _p(k_pool), _p(v_pool),
                          _p(k_scales), _p(v_scales), _p(bt), _p(sl), _p(kp), _p(sc), _p(idx),
                          _p(nsel), _p(out), _p(lse), _p(ov))
    return {"scores": sc, "indices": idx, "n_sel": nsel, "out": out, "lse": lse, "overlap": ov}


def max_threads() -> int:
    return lib().orc_max_threads()


def set_threads(n: int) -> None:
    lib().orc_set_threads(n)
