"""Device-side setup for one decode step: problem description, output and
workspace allocation (torch device memory), and the calls into the C ABI.

Nothing here computes any part of the step; it only allocates and forwards.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as B
from .configs import Workload
from .inputs import DecodeInputs


def problem_for(inp: DecodeInputs, k_max: Optional[int] = None) -> B.Problem:
    wl = inp.wl
    loc = B.SKV_POOL_HOST if wl.pool == "host" else B.SKV_POOL_DEVICE
    return B.make_problem(wl.batch, wl.n_q_tokens, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                          wl.block_size, wl.max_blocks, inp.n_pool_blocks, inp.pool_stride_block,
                          inp.pool_stride_head, wl.window, k_max or inp.k_max, wl.q_dtype,
                          wl.kv_dtype, wl.landmark_dtype, loc)


class DecodeStep:
    """Outputs, workspace and staging for repeated decode steps on one input set.

    ``inp`` must already live where the library reads it: device tensors for a
    device pool; for a host pool, k_pool / v_pool in pinned host memory and
    everything else on the device."""

    def __init__(self, inp: DecodeInputs, k_max: Optional[int] = None, device="cuda"):
        self.inp = inp
        wl: Workload = inp.wl
        self.pr = problem_for(inp, k_max)
        km = self.pr.k_max
        Bn, T, Hq, Hkv, d, blk = wl.batch, wl.n_q_tokens, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.block_size
        self.device = device
        self.ws = B.alloc_workspace(self.pr, device)
        self.indices = torch.empty((Bn, T, Hkv, km), dtype=torch.int32, device=device)
        self.n_sel = torch.empty((Bn, T, Hkv), dtype=torch.int32, device=device)
        self.out = torch.empty((Bn, Hq, d), dtype=torch.float32, device=device)
        self.lse = torch.empty((Bn, Hq), dtype=torch.float32, device=device)
        self.overlap = torch.empty((Bn, Hkv), dtype=torch.float32, device=device) if T == 2 else None
        self.k_stage = self.v_stage = self.k_stage_scales = self.v_stage_scales = None
        if wl.pool == "host":
            shape = (Bn, Hkv, km, blk, d)
            self.k_stage = [torch.empty(shape, dtype=inp.k_pool.dtype, device=device) for _ in range(2)]
            self.v_stage = [torch.empty(shape, dtype=inp.v_pool.dtype, device=device) for _ in range(2)]
            if inp.k_scales is not None:
                self.k_stage_scales = [torch.empty((Bn, Hkv, km), dtype=torch.float32, device=device)
                                       for _ in range(2)]
                self.v_stage_scales = [torch.empty((Bn, Hkv, km), dtype=torch.float32, device=device)
                                       for _ in range(2)]
        self.inputs = B.step_inputs(inp.q, inp.landmarks, inp.k_pool, inp.v_pool, inp.k_scales,
                                    inp.v_scales, inp.block_table, inp.seq_lens, inp.k_per_seq,
                                    inp.window_k, inp.window_v,
                                    inp.window_k_scales, inp.window_v_scales)
        self.outputs = B.step_outputs(self.indices, self.n_sel, self.out, self.lse, self.overlap)

    def run(self, stream=None, copy_stream=None, slot: int = 0) -> None:
        ks = self.k_stage[slot] if self.k_stage else None
        vs = self.v_stage[slot] if self.v_stage else None
        kss = self.k_stage_scales[slot] if self.k_stage_scales else None
        vss = self.v_stage_scales[slot] if self.v_stage_scales else None
        B.sparsekv_decode_step(self.pr, self.inputs, self.outputs, self.ws, ks, vs, kss, vss,
                               stream=stream, copy_stream=copy_stream)

    def run_hybrid(self, host: "HybridHost", stream=None) -> None:
        """Host pool: the hybrid step (window on the GPU, selected blocks on the host)."""
        B.sparsekv_decode_step_hybrid(self.pr, self.inputs, self.outputs, host.part, self.ws, stream)


def _stage_slots(inp: DecodeInputs, km: int, n: int, device) -> tuple:
    """n staging buffers [B][Hkv][k_max][blk][d] for K and V (and fp8 scales)."""
    wl = inp.wl
    shape = (wl.batch, wl.n_kv_heads, km, wl.block_size, wl.head_dim)
    k = [torch.empty(shape, dtype=inp.k_pool.dtype, device=device) for _ in range(n)]
    v = [torch.empty(shape, dtype=inp.v_pool.dtype, device=device) for _ in range(n)]
    ks = vs = None
    if inp.k_scales is not None:
        ks = [torch.empty(shape[:3], dtype=torch.float32, device=device) for _ in range(n)]
        vs = [torch.empty(shape[:3], dtype=torch.float32, device=device) for _ in range(n)]
    return k, v, ks, vs


class LayerPipeline:
    """The host-pool layer pipelines over one input set per layer (each with
    its own query, landmarks, pinned pool, table and window, all of one
    problem shape): per-layer outputs, one shared workspace, two staging slots
    and, for the predicted pipeline, the stage the correction writes.
    Allocation and forwarding only."""

    def __init__(self, layers: list, k_max: Optional[int] = None, device="cuda"):
        self.layers = layers
        self.pr = problem_for(layers[0], k_max)
        for inp in layers[1:]:
            other = problem_for(inp, k_max)
            for f, _ in B.Problem._fields_:
                if getattr(other, f) != getattr(self.pr, f):
                    raise ValueError(f"layer inputs differ in problem field {f}")
        wl = layers[0].wl
        km = self.pr.k_max
        Bn, T, Hq, Hkv, d = wl.batch, wl.n_q_tokens, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
        self.device = device
        self.ws = B.alloc_workspace(self.pr, device)
        self.outs = []
        for _ in layers:
            o = dict(indices=torch.empty((Bn, T, Hkv, km), dtype=torch.int32, device=device),
                     n_sel=torch.empty((Bn, T, Hkv), dtype=torch.int32, device=device),
                     out=torch.empty((Bn, Hq, d), dtype=torch.float32, device=device),
                     lse=torch.empty((Bn, Hq), dtype=torch.float32, device=device),
                     overlap=torch.empty((Bn, Hkv), dtype=torch.float32, device=device) if T == 2 else None,
                     misses=torch.empty((Bn, Hkv), dtype=torch.int32, device=device))
            o["struct"] = B.step_outputs(o["indices"], o["n_sel"], o["out"], o["lse"], o["overlap"])
            self.outs.append(o)
        self.inputs = [B.step_inputs(inp.q, inp.landmarks, inp.k_pool, inp.v_pool, inp.k_scales, inp.v_scales,
                                     inp.block_table, inp.seq_lens, inp.k_per_seq, inp.window_k, inp.window_v,
                                    inp.window_k_scales, inp.window_v_scales)
                       for inp in layers]
        self.k_slots, self.v_slots, self.k_slot_scales, self.v_slot_scales = _stage_slots(layers[0], km, 2, device)
        self.stage = None

    def staging_buffers(self) -> list:
        """Every staging tensor the pipelines write (slots, then the predicted stage)."""
        bufs = list(self.k_slots) + list(self.v_slots)
        for extra in (self.k_slot_scales, self.v_slot_scales):
            bufs += list(extra or [])
        if self.stage is not None:
            bufs += [t for t in self.stage if t is not None]
        return bufs

    def run(self, stream=None, copy_stream=None) -> list:
        """sparsekv_decode_layers: every layer's selection, then gathers into
        slot l % 2 on the copy stream and attention on `stream`."""
        B.sparsekv_decode_layers(self.pr, self.inputs, [o["struct"] for o in self.outs], self.k_slots,
                                 self.v_slots, self.ws, self.k_slot_scales, self.v_slot_scales,
                                 stream=stream, copy_stream=copy_stream)
        return self.outs

    def alloc_stage(self) -> None:
        """The stage the predicted pipeline's corrections write (allocated once)."""
        if self.stage is None:
            k, v, ks, vs = _stage_slots(self.layers[0], self.pr.k_max, 1, self.device)
            self.stage = (k[0], v[0], ks[0] if ks else None, vs[0] if vs else None)

    def run_predicted(self, predictions: list, stream=None, copy_stream=None) -> list:
        """sparsekv_decode_layers_predicted.  predictions[l] = (indices, n_sel,
        token): layer l's predicted selection (row `token` of an earlier
        selection); the per-layer miss counts land in outs[l]["misses"]."""
        self.alloc_stage()
        preds = [B.layer_prediction(idx, nsel, tok, o["misses"])
                 for (idx, nsel, tok), o in zip(predictions, self.outs)]
        k, v, ks, vs = self.stage
        B.sparsekv_decode_layers_predicted(self.pr, self.inputs, [o["struct"] for o in self.outs], preds,
                                           self.k_slots, self.v_slots, k, v, self.ws, self.k_slot_scales,
                                           self.v_slot_scales, ks, vs, stream=stream, copy_stream=copy_stream)
        return self.outs


def device_pointer_of_pinned(t: torch.Tensor) -> int:
    """Device address of a pinned host tensor (hipHostGetDevicePointer)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    dptr = ctypes.c_void_p(0)
    err = hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(t.data_ptr()), 0)
    if err != 0 or not dptr.value:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({err}); pool is not mapped pinned memory")
    return int(dptr.value)


class PinnedPool:
    """A pinned host tensor plus its device-visible address (what the library reads)."""

    def __init__(self, t: torch.Tensor):
        self.tensor = t if t.is_pinned() else t.cpu().pin_memory()
        self.dptr = device_pointer_of_pinned(self.tensor)
        self.dtype = self.tensor.dtype

    def data_ptr(self) -> int:
        return self.dptr


class HybridHost:
    """Pinned host buffers of the hybrid step for one input set (allocation only)."""

    def __init__(self, st: "DecodeStep", n_threads: int = 0):
        inp, pr = st.inp, st.pr
        wl = inp.wl
        if not isinstance(inp.k_pool, PinnedPool):
            raise ValueError("the hybrid step reads a pinned host pool")
        Bn, T, Hq, Hkv, d = wl.batch, wl.n_q_tokens, wl.n_q_heads, wl.n_kv_heads, wl.head_dim

        def pinned(shape, dtype):
            return torch.empty(shape, dtype=dtype, pin_memory=True)

        self.q = pinned(tuple(inp.q.shape), inp.q.dtype)
        self.seq_lens = pinned((Bn,), torch.int32)
        self.block_table = pinned((Bn, wl.max_blocks), torch.int32)
        self.indices = pinned((Bn, T, Hkv, pr.k_max), torch.int32)
        self.n_sel = pinned((Bn, T, Hkv), torch.int32)
        self.k_scales = self.v_scales = None
        if inp.k_scales is not None:
            self.k_scales = pinned(tuple(inp.k_scales.shape), torch.float32)
            self.v_scales = pinned(tuple(inp.v_scales.shape), torch.float32)
        self.o = pinned((Bn, Hq, d), torch.float32)
        self.lse = pinned((Bn, Hq), torch.float32)
        self.part = B.HostPart(inp.k_pool.tensor.data_ptr(), inp.v_pool.tensor.data_ptr(), int(n_threads),
                               self.q.data_ptr(), self.seq_lens.data_ptr(), self.block_table.data_ptr(),
                               self.indices.data_ptr(), self.n_sel.data_ptr(),
                               self.k_scales.data_ptr() if self.k_scales is not None else None,
                               self.v_scales.data_ptr() if self.v_scales is not None else None,
                               self.o.data_ptr(), self.lse.data_ptr())


def to_device_for(inp: DecodeInputs, device="cuda") -> DecodeInputs:
    """Place inputs where the library reads them (host pools go to pinned memory)."""
    pools = (inp.k_pool, inp.v_pool)
    if inp.wl.pool == "host":
        inp.k_pool = inp.v_pool = None
    dev = inp.to(device)
    inp.k_pool, inp.v_pool = pools
    if inp.wl.pool == "host":
        dev.k_pool = PinnedPool(pools[0])
        dev.v_pool = PinnedPool(pools[1])
    else:
        dev.k_pool, dev.v_pool = pools[0].to(device), pools[1].to(device)
    return dev
