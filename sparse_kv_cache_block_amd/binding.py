"""ctypes binding of libsparsekv.so (the C ABI in include/sparsekv.h).

Argument marshalling only: every function below forwards to the C entry point
of the same name; all arithmetic runs in the HIP kernels.  Tensors are passed
by their data pointers; streams default to torch's current stream.  There is
no CPU fallback: loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SKV_LIB selects another build of the library (the host-sanitized one under _asan/)
LIB_PATH = os.environ.get("SKV_LIB") or os.path.join(_HERE, "libsparsekv.so")

SKV_OK, SKV_E_NULL, SKV_E_SHAPE, SKV_E_DTYPE, SKV_E_UNSUPPORTED, SKV_E_WORKSPACE, SKV_E_HIP = range(7)
SKV_F32, SKV_BF16, SKV_FP8_E4M3FN = range(3)
SKV_POOL_DEVICE, SKV_POOL_HOST = range(2)
SKV_SRC_PAGED, SKV_SRC_STAGED, SKV_SRC_WINDOW = range(3)
DTYPE_CODE = {"fp32": SKV_F32, "bf16": SKV_BF16, "fp8": SKV_FP8_E4M3FN}

EXPORTED = ("sparsekv_status_string", "sparsekv_last_error", "sparsekv_version",
            "sparsekv_workspace_size", "sparsekv_workspace_init", "sparsekv_score",
            "sparsekv_topk", "sparsekv_gather", "sparsekv_attend", "sparsekv_decode_step",
            "sparsekv_decode_layers", "sparsekv_decode_step_launches", "sparsekv_gather_correct",
            "sparsekv_attend_cobatched", "sparsekv_decode_step_hybrid", "sparsekv_host_attention",
            "sparsekv_stream_read", "sparsekv_decode_layers_predicted", "sparsekv_decode_step_noalloc",
            "sparsekv_decode_step_kernel", "sparsekv_decode_step_launch_times")


class SkvError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class Problem(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_tokens", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("block_size", C.c_int32),
                ("max_blocks_per_seq", C.c_int32), ("n_pool_blocks", C.c_int32),
                ("pool_stride_block", C.c_int64), ("pool_stride_head", C.c_int64),
                ("window", C.c_int32), ("k_max", C.c_int32), ("q_dtype", C.c_int32),
                ("kv_dtype", C.c_int32), ("landmark_dtype", C.c_int32),
                ("pool_location", C.c_int32)]


class KvSource(C.Structure):
    _fields_ = [("kind", C.c_int32), ("k", C.c_void_p), ("v", C.c_void_p),
                ("k_scales", C.c_void_p), ("v_scales", C.c_void_p), ("block_table", C.c_void_p)]


class StepInputs(C.Structure):
    _fields_ = [("q", C.c_void_p), ("landmarks", C.c_void_p), ("k_pool", C.c_void_p),
                ("v_pool", C.c_void_p), ("k_scales", C.c_void_p), ("v_scales", C.c_void_p),
                ("block_table", C.c_void_p), ("seq_lens", C.c_void_p), ("k_per_seq", C.c_void_p),
                ("window_k", C.c_void_p), ("window_v", C.c_void_p),
                ("window_k_scales", C.c_void_p), ("window_v_scales", C.c_void_p)]


class StepOutputs(C.Structure):
    _fields_ = [("indices", C.c_void_p), ("n_sel", C.c_void_p), ("out", C.c_void_p),
                ("lse", C.c_void_p), ("overlap", C.c_void_p)]


class HostPart(C.Structure):
    _fields_ = [("k_pool", C.c_void_p), ("v_pool", C.c_void_p), ("n_threads", C.c_int32),
                ("q", C.c_void_p), ("seq_lens", C.c_void_p), ("block_table", C.c_void_p),
                ("indices", C.c_void_p), ("n_sel", C.c_void_p), ("k_scales", C.c_void_p),
                ("v_scales", C.c_void_p), ("o", C.c_void_p), ("lse", C.c_void_p)]


class LayerPrediction(C.Structure):
    _fields_ = [("indices", C.c_void_p), ("n_sel", C.c_void_p), ("token", C.c_int32),
                ("misses", C.c_void_p)]


_lib = None


def lib() -> C.CDLL:
    """Load libsparsekv.so once; raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(there is no CPU fallback)")
        L = C.CDLL(LIB_PATH)
        vp, sz = C.c_void_p, C.c_size_t
        P = C.POINTER(Problem)
        sig = {
            "sparsekv_status_string": (C.c_char_p, [C.c_int]),
            "sparsekv_last_error": (C.c_char_p, []),
            "sparsekv_version": (C.c_char_p, []),
            "sparsekv_workspace_size": (C.c_int, [P, C.POINTER(sz)]),
            "sparsekv_workspace_init": (C.c_int, [vp, sz, vp]),
            "sparsekv_stream_read": (C.c_int, [vp, sz, vp, sz, vp]),
            "sparsekv_score": (C.c_int, [P, vp, vp, vp, vp, vp]),
            "sparsekv_topk": (C.c_int, [P, vp, vp, vp, vp, vp, vp, vp]),
            "sparsekv_gather": (C.c_int, [P] + [vp] * 12),
            "sparsekv_gather_correct": (C.c_int, [P] + [vp] * 7 + [C.c_int32] + [vp] * 6 + [C.c_int32]
                                        + [vp] * 6),
            "sparsekv_decode_step_launches": (C.c_int, [P, C.POINTER(C.c_int32)]),
            "sparsekv_decode_step_kernel": (C.c_int, [P, C.c_int32, C.POINTER(C.c_char_p)]),
            "sparsekv_decode_step_launch_times": (C.c_int, [P, C.POINTER(StepInputs), C.POINTER(StepOutputs),
                                                            vp, sz, vp, C.c_int32, C.POINTER(C.c_float)]),
            "sparsekv_attend": (C.c_int, [P, vp, C.POINTER(KvSource), vp, vp, C.POINTER(KvSource),
                                          vp, vp, vp, vp, sz, vp]),
            "sparsekv_attend_cobatched": (C.c_int, [P, vp, C.POINTER(KvSource), vp, vp,
                                                    C.POINTER(KvSource), vp, vp, vp, vp, sz, vp]),
            "sparsekv_decode_step_hybrid": (C.c_int, [P, C.POINTER(StepInputs), C.POINTER(StepOutputs),
                                                      C.POINTER(HostPart), vp, sz, vp]),
            "sparsekv_host_attention": (C.c_int, [P, C.POINTER(HostPart)]),
            "sparsekv_decode_step": (C.c_int, [P, C.POINTER(StepInputs), C.POINTER(StepOutputs),
                                               vp, vp, vp, vp, vp, sz, vp, vp]),
            "sparsekv_decode_step_noalloc": (C.c_int, [P, C.POINTER(StepInputs), C.POINTER(StepOutputs), vp]),
            "sparsekv_decode_layers": (C.c_int, [P, C.c_int32, C.POINTER(StepInputs),
                                                 C.POINTER(StepOutputs), C.POINTER(vp), C.POINTER(vp),
                                                 C.POINTER(vp), C.POINTER(vp), vp, sz, vp, vp]),
            "sparsekv_decode_layers_predicted": (C.c_int, [P, C.c_int32, C.POINTER(StepInputs),
                                                           C.POINTER(StepOutputs), C.POINTER(LayerPrediction),
                                                           C.POINTER(vp), C.POINTER(vp), C.POINTER(vp),
                                                           C.POINTER(vp), vp, vp, vp, vp, vp, sz, vp, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != SKV_OK:
        L = lib()
        raise SkvError(status, where, f"{L.sparsekv_status_string(status).decode()}: "
                                      f"{L.sparsekv_last_error().decode()}")


# ---------------------------------------------------------------- entry points
def sparsekv_status_string(status: int) -> str:
    return lib().sparsekv_status_string(status).decode()


def sparsekv_last_error() -> str:
    return lib().sparsekv_last_error().decode()


def sparsekv_version() -> str:
    return lib().sparsekv_version().decode()


def sparsekv_workspace_size(pr: Problem) -> int:
    n = C.c_size_t(0)
    _check(lib().sparsekv_workspace_size(C.byref(pr), C.byref(n)), "sparsekv_workspace_size")
    return int(n.value)


def sparsekv_decode_step_launches(pr: Problem) -> int:
    n = C.c_int32(0)
    _check(lib().sparsekv_decode_step_launches(C.byref(pr), C.byref(n)), "sparsekv_decode_step_launches")
    return int(n.value)


def sparsekv_decode_step_kernel(pr: Problem, launch: int) -> str:
    name = C.c_char_p()
    _check(lib().sparsekv_decode_step_kernel(C.byref(pr), launch, C.byref(name)), "sparsekv_decode_step_kernel")
    return name.value.decode()


def sparsekv_decode_step_launch_times(pr: Problem, inputs: StepInputs, outputs: StepOutputs,
                                      workspace: torch.Tensor, n_steps: int, stream=None) -> list:
    n = sparsekv_decode_step_launches(pr)
    us = (C.c_float * n)()
    _check(lib().sparsekv_decode_step_launch_times(C.byref(pr), C.byref(inputs), C.byref(outputs),
                                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                   _stream(stream), n_steps, us),
           "sparsekv_decode_step_launch_times")
    return [float(x) for x in us]


def sparsekv_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    _check(lib().sparsekv_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream(stream)), "sparsekv_workspace_init")


def sparsekv_stream_read(buffer: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    _check(lib().sparsekv_stream_read(_ptr(buffer), buffer.numel() * buffer.element_size(), _ptr(sink),
                                      sink.numel() * sink.element_size(), _stream(stream)),
           "sparsekv_stream_read")


def sparsekv_score(pr: Problem, q, landmarks, seq_lens, scores, stream=None) -> None:
    _check(lib().sparsekv_score(C.byref(pr), _ptr(q), _ptr(landmarks), _ptr(seq_lens), _ptr(scores),
                                _stream(stream)), "sparsekv_score")


def sparsekv_topk(pr: Problem, scores, seq_lens, k_per_seq, indices, n_sel, overlap=None,
                  stream=None) -> None:
    _check(lib().sparsekv_topk(C.byref(pr), _ptr(scores), _ptr(seq_lens), _ptr(k_per_seq),
                               _ptr(indices), _ptr(n_sel), _ptr(overlap), _stream(stream)),
           "sparsekv_topk")


def sparsekv_gather(pr: Problem, k_pool, v_pool, k_scales, v_scales, block_table, indices, n_sel,
                    k_stage, v_stage, k_stage_scales=None, v_stage_scales=None, stream=None) -> None:
    _check(lib().sparsekv_gather(C.byref(pr), _ptr(k_pool), _ptr(v_pool), _ptr(k_scales),
                                 _ptr(v_scales), _ptr(block_table), _ptr(indices), _ptr(n_sel),
                                 _ptr(k_stage), _ptr(v_stage), _ptr(k_stage_scales),
                                 _ptr(v_stage_scales), _stream(stream)), "sparsekv_gather")


def sparsekv_gather_correct(pr: Problem, k_pool, v_pool, k_scales, v_scales, block_table,
                            spec_indices, spec_n_sel, spec_token: int, spec_k_stage, spec_v_stage,
                            spec_k_scales, spec_v_scales, real_indices, real_n_sel, real_token: int,
                            k_stage, v_stage, k_stage_scales=None, v_stage_scales=None, misses=None,
                            stream=None) -> None:
    _check(lib().sparsekv_gather_correct(
        C.byref(pr), _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales), _ptr(block_table),
        _ptr(spec_indices), _ptr(spec_n_sel), int(spec_token), _ptr(spec_k_stage), _ptr(spec_v_stage),
        _ptr(spec_k_scales), _ptr(spec_v_scales), _ptr(real_indices), _ptr(real_n_sel), int(real_token),
        _ptr(k_stage), _ptr(v_stage), _ptr(k_stage_scales), _ptr(v_stage_scales), _ptr(misses),
        _stream(stream)), "sparsekv_gather_correct")


def kv_source(kind: int, k, v, k_scales=None, v_scales=None, block_table=None) -> KvSource:
    return KvSource(kind, _ptr(k), _ptr(v), _ptr(k_scales), _ptr(v_scales), _ptr(block_table))


def sparsekv_attend(pr: Problem, q, sparse: KvSource, indices, n_sel, window: Optional[KvSource],
                    seq_lens, out, lse, workspace: torch.Tensor, stream=None) -> None:
    _check(lib().sparsekv_attend(C.byref(pr), _ptr(q), C.byref(sparse), _ptr(indices), _ptr(n_sel),
                                 C.byref(window) if window is not None else None, _ptr(seq_lens),
                                 _ptr(out), _ptr(lse), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "sparsekv_attend")


def sparsekv_attend_cobatched(pr: Problem, q, sparse: KvSource, indices, n_sel, window: Optional[KvSource],
                              seq_lens, out, lse, workspace: torch.Tensor, stream=None) -> None:
    _check(lib().sparsekv_attend_cobatched(
        C.byref(pr), _ptr(q), C.byref(sparse), _ptr(indices), _ptr(n_sel),
        C.byref(window) if window is not None else None, _ptr(seq_lens), _ptr(out), _ptr(lse),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
        "sparsekv_attend_cobatched")


def step_inputs(q, landmarks, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens, k_per_seq,
                window_k=None, window_v=None, window_k_scales=None, window_v_scales=None) -> StepInputs:
    return StepInputs(*(_ptr(x) for x in (q, landmarks, k_pool, v_pool, k_scales, v_scales,
                                          block_table, seq_lens, k_per_seq, window_k, window_v,
                                          window_k_scales, window_v_scales)))


def step_outputs(indices, n_sel, out, lse=None, overlap=None) -> StepOutputs:
    return StepOutputs(*(_ptr(x) for x in (indices, n_sel, out, lse, overlap)))


def sparsekv_decode_step(pr: Problem, inputs: StepInputs, outputs: StepOutputs, workspace: torch.Tensor,
                         k_stage=None, v_stage=None, k_stage_scales=None, v_stage_scales=None,
                         stream=None, copy_stream=None) -> None:
    cs = None if copy_stream is None else _stream(copy_stream)
    _check(lib().sparsekv_decode_step(C.byref(pr), C.byref(inputs), C.byref(outputs), _ptr(k_stage),
                                      _ptr(v_stage), _ptr(k_stage_scales), _ptr(v_stage_scales),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream), cs), "sparsekv_decode_step")


def sparsekv_decode_step_noalloc(pr: Problem, inputs: StepInputs, outputs: StepOutputs, stream=None) -> None:
    _check(lib().sparsekv_decode_step_noalloc(C.byref(pr), C.byref(inputs), C.byref(outputs), _stream(stream)),
           "sparsekv_decode_step_noalloc")


def sparsekv_decode_step_hybrid(pr: Problem, inputs: StepInputs, outputs: StepOutputs, host: HostPart,
                                workspace: torch.Tensor, stream=None) -> None:
    _check(lib().sparsekv_decode_step_hybrid(C.byref(pr), C.byref(inputs), C.byref(outputs), C.byref(host),
                                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                                             _stream(stream)), "sparsekv_decode_step_hybrid")


def sparsekv_host_attention(pr: Problem, host: HostPart) -> None:
    _check(lib().sparsekv_host_attention(C.byref(pr), C.byref(host)), "sparsekv_host_attention")


def sparsekv_decode_layers(pr: Problem, inputs: Sequence[StepInputs], outputs: Sequence[StepOutputs],
                           k_stage: Sequence, v_stage: Sequence, workspace: torch.Tensor,
                           k_stage_scales: Optional[Sequence] = None,
                           v_stage_scales: Optional[Sequence] = None,
                           stream=None, copy_stream=None) -> None:
    n = len(inputs)
    InArr, OutArr, PtrArr = StepInputs * n, StepOutputs * n, C.c_void_p * 2
    ks = PtrArr(*(_ptr(x) for x in k_stage))
    vs = PtrArr(*(_ptr(x) for x in v_stage))
    kss = PtrArr(*(_ptr(x) for x in k_stage_scales)) if k_stage_scales else None
    vss = PtrArr(*(_ptr(x) for x in v_stage_scales)) if v_stage_scales else None
    cs = None if copy_stream is None else _stream(copy_stream)
    _check(lib().sparsekv_decode_layers(C.byref(pr), n, InArr(*inputs), OutArr(*outputs), ks, vs,
                                        kss, vss, _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream), cs), "sparsekv_decode_layers")


def layer_prediction(indices, n_sel, token: int, misses=None) -> LayerPrediction:
    return LayerPrediction(_ptr(indices), _ptr(n_sel), int(token), _ptr(misses))


def sparsekv_decode_layers_predicted(pr: Problem, inputs: Sequence[StepInputs], outputs: Sequence[StepOutputs],
                                     predictions: Sequence[LayerPrediction], pref_k: Sequence, pref_v: Sequence,
                                     k_stage, v_stage, workspace: torch.Tensor,
                                     pref_k_scales: Optional[Sequence] = None,
                                     pref_v_scales: Optional[Sequence] = None, k_stage_scales=None,
                                     v_stage_scales=None, stream=None, copy_stream=None) -> None:
    n = len(inputs)
    InArr, OutArr, PredArr, PtrArr = StepInputs * n, StepOutputs * n, LayerPrediction * n, C.c_void_p * 2
    pk = PtrArr(*(_ptr(x) for x in pref_k))
    pv = PtrArr(*(_ptr(x) for x in pref_v))
    pks = PtrArr(*(_ptr(x) for x in pref_k_scales)) if pref_k_scales else None
    pvs = PtrArr(*(_ptr(x) for x in pref_v_scales)) if pref_v_scales else None
    cs = None if copy_stream is None else _stream(copy_stream)
    _check(lib().sparsekv_decode_layers_predicted(
        C.byref(pr), n, InArr(*inputs), OutArr(*outputs), PredArr(*predictions), pk, pv, pks, pvs,
        _ptr(k_stage), _ptr(v_stage), _ptr(k_stage_scales), _ptr(v_stage_scales), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream), cs), "sparsekv_decode_layers_predicted")


# ---------------------------------------------------------------- helpers
def make_problem(B, T, Hq, Hkv, d, blk, max_blocks, n_pool_blocks, stride_block, stride_head,
                 window, k_max, q_dtype, kv_dtype, landmark_dtype, pool_location=SKV_POOL_DEVICE) -> Problem:
    def code(x):
        return DTYPE_CODE[x] if isinstance(x, str) else int(x)
    return Problem(B, T, Hq, Hkv, d, blk, max_blocks, n_pool_blocks, stride_block, stride_head,
                   window, k_max, code(q_dtype), code(kv_dtype), code(landmark_dtype), pool_location)


def alloc_workspace(pr: Problem, device="cuda", stream=None) -> torch.Tensor:
    """Allocate (torch) and clear (library fill kernel) a workspace for pr."""
    n = sparsekv_workspace_size(pr)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    sparsekv_workspace_init(ws, stream)
    return ws
