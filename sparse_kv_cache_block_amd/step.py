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
                                    inp.window_k, inp.window_v)
        self.outputs = B.step_outputs(self.indices, self.n_sel, self.out, self.lse, self.overlap)

    def run(self, stream=None, copy_stream=None, slot: int = 0) -> None:
        ks = self.k_stage[slot] if self.k_stage else None
        vs = self.v_stage[slot] if self.v_stage else None
        kss = self.k_stage_scales[slot] if self.k_stage_scales else None
        vss = self.v_stage_scales[slot] if self.v_stage_scales else None
        B.sparsekv_decode_step(self.pr, self.inputs, self.outputs, self.ws, ks, vs, kss, vss,
                               stream=stream, copy_stream=copy_stream)

    def layer_outputs(self, n_layers: int) -> list:
        """Per-layer output buffers (indices, n_sel, out, lse) for run_layers."""
        if len(getattr(self, "_layer_bufs", [])) != n_layers:
            self._layer_bufs = []
            for _ in range(n_layers):
                bufs = dict(indices=torch.empty_like(self.indices), n_sel=torch.empty_like(self.n_sel),
                            out=torch.empty_like(self.out), lse=torch.empty_like(self.lse),
                            overlap=None if self.overlap is None else torch.empty_like(self.overlap))
                bufs["struct"] = B.step_outputs(bufs["indices"], bufs["n_sel"], bufs["out"],
                                                bufs["lse"], bufs["overlap"])
                self._layer_bufs.append(bufs)
        return self._layer_bufs

    def run_hybrid(self, host: "HybridHost", stream=None) -> None:
        """Host pool: the hybrid step (window on the GPU, selected blocks on the host)."""
        B.sparsekv_decode_step_hybrid(self.pr, self.inputs, self.outputs, host.part, self.ws, stream)

    def run_layers(self, n_layers: int, stream=None, copy_stream=None) -> list:
        """Host pool: n_layers layer-steps over the same inputs through the
        two-slot staging pipeline; returns the per-layer output buffers."""
        outs = self.layer_outputs(n_layers)
        B.sparsekv_decode_layers(self.pr, [self.inputs] * n_layers, [o["struct"] for o in outs],
                                 self.k_stage, self.v_stage, self.ws, self.k_stage_scales,
                                 self.v_stage_scales, stream=stream, copy_stream=copy_stream)
        return outs


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
