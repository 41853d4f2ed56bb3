#!/usr/bin/env python3
"""Benchmark of the sparse-KV decode step on one MI355X.

A step is one pass of the whole hot path -- landmark scoring, per-KV-head
top-k, the paged gather fused into the attention loads, attention over the
selected blocks plus the recent window, and the log-sum-exp merge -- over one
batch of seeded synthetic inputs already resident in HBM.  Steps rotate over
several independent input instances so that neither the landmarks nor the K/V
blocks can be served from the 256 MB last-level cache between steps.

Prints one JSON line: tokens/s (real query tokens per second), the dominant
kernel's roofline (algorithmic HBM bytes per launch over its mean launch time
from HIP events on the launch stream: the single-launch step kernel where the
step is one launch, else the attention launch timed alone), that rate against
the streaming-read ceiling of a plain read with the same loads on the same box,
and the CPU oracle timed on a bounded sample of the same workload.  After the
headline workload the same process times the other workloads (--others) and
adds their step times, per-kernel figures and fractions of peak to the line as
other_workloads; the headline's own fields are unaffected.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Kernel arguments in device memory (read before the HIP runtime starts).  The
# kernels take their parameters by value and every workgroup reads them
# first; from host memory that costs a link round trip per launch (32k step
# 69.7 us with HIP_FORCE_DEV_KERNARG=0 against 66.4 us with 1 on one box).
os.environ.setdefault("HIP_FORCE_DEV_KERNARG", "1")

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attention_bytes(wl, seq_lens, nsel_real) -> int:
    """Algorithmic bytes of one attention launch: the selected K/V chunks (and
    fp8 scales), the window's K/V, the real-token queries, the fp32 output and
    lse."""
    from sparse_kv_cache_block_amd.configs import ELEM_BYTES
    d, blk = wl.head_dim, wl.block_size
    e_kv = ELEM_BYTES[wl.kv_dtype]
    e_scale = 8 if wl.kv_dtype == "fp8" else 0
    total = int(nsel_real.sum()) * (2 * blk * d * e_kv + e_scale)
    for L in seq_lens:
        total += wl.n_kv_heads * min(wl.window, int(L)) * 2 * d * e_kv
    total += wl.batch * wl.n_q_heads * d * ELEM_BYTES[wl.q_dtype]
    total += wl.batch * wl.n_q_heads * (d + 1) * 4
    return total


KERNEL_SOURCES = {
    "pair_step_kernel": ("step.hip", "attend_dev.h", "select_dev.h", "skv_device.h", "skv_internal.h"),
    "attend_kernel": ("attend.hip", "attend_dev.h", "select_dev.h", "skv_device.h", "skv_internal.h"),
    "attend_cobatched_kernel": ("attend.hip", "attend_dev.h", "select_dev.h", "skv_device.h", "skv_internal.h"),
    "split_step_kernel": ("split_step.hip", "attend_dev.h", "select_dev.h", "skv_device.h", "skv_internal.h"),
}


def _code_only(text: str) -> str:
    """Source text without comments, trailing blanks or empty lines."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def kernel_source_digest(kernel: str) -> str:
    """sha256 over a kernel's sources, comments aside (counter results go stale
    when the code changes)."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sparse_kv_cache_block_amd", "csrc", name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def recorded_traffic(kernel: str, workload: str):
    """Per-launch HBM bytes of a kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if "```json" not in text:
        return None
    rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    if rec.get("source_sha256") != kernel_source_digest(kernel):
        return None
    return rec


def copy_probe(mib: int, reps: int) -> int:
    """A plain device-to-device copy of known size (counter calibration)."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "reps": reps}))
    return 0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_ceiling_gbps(gib: int = 2, reps: int = 20) -> float:
    """Streaming-read rate of sparsekv_stream_read (the kernels' own 16-byte
    non-temporal loads) over a buffer far larger than the last-level cache."""
    import torch
    from sparse_kv_cache_block_amd import binding as B
    buf = torch.ones(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    for _ in range(3):
        B.sparsekv_stream_read(buf, sink)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        B.sparsekv_stream_read(buf, sink)
    e1.record(stream)
    e1.synchronize()
    rate = buf.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    return rate


def h2d_ceiling_gbps(mib: int = 64, reps: int = 20) -> float:
    """Contiguous host-to-device copy rate from pinned memory (hipMemcpyAsync
    through torch), the reference for the host-link rate of the gather."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, pin_memory=True).fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    e1.record()
    e1.synchronize()
    return n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def gather_correct_probe(reps: int) -> int:
    """Host-pool workload with a speculative second query token (real + N(0, 0.3)):
    the full gather of the real token's selection against the correction of a
    stage already holding the speculative token's selection."""
    import numpy as np
    import torch

    from sparse_kv_cache_block_amd import binding as B
    from sparse_kv_cache_block_amd import configs
    from sparse_kv_cache_block_amd.inputs import make_inputs
    from sparse_kv_cache_block_amd.step import DecodeStep, LayerPipeline, to_device_for

    wl = configs.HOST.scaled(n_q_tokens=2, spec_noise=0.3)
    torch.cuda.set_device(0)
    st = DecodeStep(to_device_for(make_inputs(wl, device="cuda", instance=0)))
    st.run()
    torch.cuda.synchronize()
    d, pr = st.inp, st.pr
    shape = (wl.batch, wl.n_kv_heads, pr.k_max, wl.block_size, wl.head_dim)
    stages = [(torch.empty(shape, dtype=d.k_pool.dtype, device="cuda"),
               torch.empty(shape, dtype=d.v_pool.dtype, device="cuda")) for _ in range(3)]
    pools = (d.k_pool, d.v_pool, d.k_scales, d.v_scales, d.block_table)
    misses = torch.empty((wl.batch, wl.n_kv_heads), dtype=torch.int32, device="cuda")
    spec, out, full = stages
    none_n = torch.zeros_like(st.n_sel)
    B.sparsekv_gather_correct(pr, *pools, st.indices, none_n, 0, *full, None, None, st.indices, st.n_sel, 1,
                              *spec)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn) -> float:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        ev[1].synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / reps

    t_full = timed(lambda: B.sparsekv_gather(pr, *pools, st.indices, st.n_sel, *full))
    t_corr = timed(lambda: B.sparsekv_gather_correct(pr, *pools, st.indices, st.n_sel, 1, *spec, None, None,
                                                     st.indices, st.n_sel, 0, *out, misses=misses))
    chunk = 2 * wl.block_size * wl.head_dim * 2
    n_real = int(st.n_sel[:, 0].sum())
    n_miss = int(misses.sum())
    print(json.dumps({
        "probe": "gather_correct", "workload": "host, 2 query tokens, speculative = real + N(0, 0.3)",
        "reps": reps, "full_gather_us": round(t_full, 1), "correction_us": round(t_corr, 1),
        "speedup": round(t_full / t_corr, 2), "selected_chunks": n_real, "misses": n_miss,
        "miss_fraction": round(n_miss / max(1, n_real), 4),
        "host_link_bytes_full": n_real * chunk, "host_link_bytes_correction": n_miss * chunk,
        "overlap_mean": round(float(np.mean(st.overlap.cpu().numpy())), 4)}), flush=True)
    return 0


def predicted_layers_probe(reps: int, n_layers: int = 4) -> int:
    """Host-pool workload with a speculative second query token (real +
    N(0, 0.3)) over n_layers layer-steps: the plain two-slot pipeline (each
    layer's selected blocks gathered over the host link after its selection)
    against the predicted one (each layer's blocks prefetched by the previous
    step's speculative selection, then only the misses fetched after the real
    selection).  Reports both pipelines' time per layer and host-link bytes
    per layer, and the per-layer critical path after a layer's selection: the
    full gather against the correction of an already staged prediction."""
    import torch

    from sparse_kv_cache_block_amd import binding as B
    from sparse_kv_cache_block_amd import configs
    from sparse_kv_cache_block_amd.inputs import make_inputs
    from sparse_kv_cache_block_amd.step import LayerPipeline, to_device_for

    wl = configs.HOST.scaled(n_q_tokens=2, spec_noise=0.3)
    torch.cuda.set_device(0)
    layers = [to_device_for(make_inputs(wl, device="cuda", instance=l)) for l in range(n_layers)]
    pipe = LayerPipeline(layers)
    cs = torch.cuda.Stream()
    pipe.run(copy_stream=cs)
    torch.cuda.synchronize()
    # the previous step's selections: the speculative token's rows predict this step's
    preds = [(o["indices"].clone(), o["n_sel"].clone(), 1) for o in pipe.outs]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn) -> float:
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        ev[1].synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / reps

    t_plain = timed(lambda: pipe.run(copy_stream=cs))
    t_pred = timed(lambda: pipe.run_predicted(preds, copy_stream=cs))
    chunk = 2 * wl.block_size * wl.head_dim * configs.ELEM_BYTES[wl.kv_dtype]
    real = sum(int(o["n_sel"][:, 0].sum()) for o in pipe.outs)
    pref = sum(int(p[1][:, 1].sum()) for p in preds)
    miss = sum(int(o["misses"].sum()) for o in pipe.outs)

    # critical path of one layer after its selection: gather + attention
    # (plain) against correction + attention (predicted, prefetch staged)
    st_in, o0 = layers[0], pipe.outs[0]
    pools = (st_in.k_pool, st_in.v_pool, st_in.k_scales, st_in.v_scales, st_in.block_table)
    pk, pv = pipe.k_slots[0], pipe.v_slots[0]
    k_st, v_st = pipe.stage[0], pipe.stage[1]
    B.sparsekv_gather(pipe.pr, *pools, preds[0][0][:, 1:], preds[0][1][:, 1:], pk, pv, None, None)
    sp = B.kv_source(B.SKV_SRC_STAGED, k_st, v_st, pipe.stage[2], pipe.stage[3])
    win = B.kv_source(B.SKV_SRC_WINDOW, st_in.window_k, st_in.window_v, st_in.window_k_scales,
                      st_in.window_v_scales)
    out = torch.empty_like(o0["out"])
    lse = torch.empty_like(o0["lse"])

    def plain_path():
        B.sparsekv_gather(pipe.pr, *pools, o0["indices"], o0["n_sel"], k_st, v_st, None, None)
        B.sparsekv_attend(pipe.pr, st_in.q, sp, o0["indices"], o0["n_sel"], win, st_in.seq_lens, out, lse, pipe.ws)

    def pred_path():
        B.sparsekv_gather_correct(pipe.pr, *pools, preds[0][0], preds[0][1], 1, pk, pv, None, None,
                                  o0["indices"], o0["n_sel"], 0, k_st, v_st)
        B.sparsekv_attend(pipe.pr, st_in.q, sp, o0["indices"], o0["n_sel"], win, st_in.seq_lens, out, lse, pipe.ws)
    t_cp_plain = timed(plain_path)
    t_cp_pred = timed(pred_path)
    print(json.dumps({
        "probe": "predicted_layers",
        "workload": f"host, 2 query tokens (speculative = real + N(0, 0.3)), {n_layers} layers with their own inputs",
        "reps": reps,
        "plain_us_per_layer": round(t_plain / n_layers, 1),
        "predicted_us_per_layer": round(t_pred / n_layers, 1),
        "link_bytes_per_layer_plain": real * chunk // n_layers,
        "link_bytes_per_layer_predicted": (pref + miss) * chunk // n_layers,
        "link_bytes_per_layer_after_selection_predicted": miss * chunk // n_layers,
        "miss_fraction": round(miss / max(1, real), 4),
        "critical_path_us_plain": round(t_cp_plain, 1),
        "critical_path_us_predicted": round(t_cp_pred, 1),
        "note": "per-layer times cover the whole call (prefetches included); the critical path is one "
                "layer's work after its selection, with the prediction already staged"}), flush=True)
    return 0


def hbm_gather_probe(reps: int, instances: int) -> int:
    """llama32k workload: the stand-alone gather of the selected K/V chunks from
    the HBM pool into staging buffers (in the decode step this gather is fused
    into the attention's loads and never copied).  Rotates over `instances`
    input sets, each with its own stage."""
    import torch

    from sparse_kv_cache_block_amd import binding as B
    from sparse_kv_cache_block_amd import configs
    from sparse_kv_cache_block_amd.inputs import make_inputs
    from sparse_kv_cache_block_amd.step import DecodeStep

    wl = configs.LLAMA32K
    torch.cuda.set_device(0)
    sets = []
    for i in range(instances):
        st = DecodeStep(make_inputs(wl, device="cuda", instance=i))
        st.run()
        shape = (wl.batch, wl.n_kv_heads, st.pr.k_max, wl.block_size, wl.head_dim)
        sets.append((st, torch.empty(shape, dtype=st.inp.k_pool.dtype, device="cuda"),
                     torch.empty(shape, dtype=st.inp.v_pool.dtype, device="cuda")))
    torch.cuda.synchronize()

    def gather(k: int) -> None:
        st, ks, vs = sets[k % len(sets)]
        d = st.inp
        B.sparsekv_gather(st.pr, d.k_pool, d.v_pool, d.k_scales, d.v_scales, d.block_table, st.indices,
                          st.n_sel, ks, vs, None, None)

    for k in range(5):
        gather(k)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for k in range(reps):
        gather(k)
    ev[1].record()
    ev[1].synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
    chunks = int(sets[0][0].n_sel[:, 0].sum())
    moved = chunks * 2 * wl.block_size * wl.head_dim * 2   # K and V chunks, bf16
    print(json.dumps({
        "probe": "hbm_gather", "workload": "llama32k (B32, 8 KV heads, k64, blk32, bf16, HBM pool)",
        "reps": reps, "instances": instances, "us_per_gather": round(us, 2), "chunks": chunks,
        "bytes_read": moved, "bytes_written": moved,
        "read_gbps": round(moved / (us * 1e-6) / 1e9, 1),
        "read_plus_write_gbps": round(2 * moved / (us * 1e-6) / 1e9, 1)}), flush=True)
    return 0


def cobatched_probe(reps: int, instances: int) -> int:
    """Dual workload: both query tokens attended by one co-batched launch over
    the union of their selections, against one attention launch per token."""
    import torch

    from sparse_kv_cache_block_amd import binding as B
    from sparse_kv_cache_block_amd import configs
    from sparse_kv_cache_block_amd.configs import ELEM_BYTES
    from sparse_kv_cache_block_amd.inputs import make_inputs
    from sparse_kv_cache_block_amd.step import DecodeStep

    wl = configs.DUAL
    torch.cuda.set_device(0)
    runs = []
    for i in range(instances):
        st = DecodeStep(make_inputs(wl, device="cuda", instance=i))
        st.run()
        d = st.inp
        src = B.kv_source(B.SKV_SRC_PAGED, d.k_pool, d.v_pool, d.k_scales, d.v_scales, d.block_table)
        Bn, Hq, D = d.q.shape[0], d.q.shape[2], d.q.shape[3]
        out2 = torch.empty((Bn, 2, Hq, D), dtype=torch.float32, device="cuda")
        lse2 = torch.empty((Bn, 2, Hq), dtype=torch.float32, device="cuda")
        outs = [torch.empty((Bn, Hq, D), dtype=torch.float32, device="cuda") for _ in range(2)]
        lses = [torch.empty((Bn, Hq), dtype=torch.float32, device="cuda") for _ in range(2)]
        runs.append((st, src, out2, lse2, outs, lses))
    torch.cuda.synchronize()

    def two_launches(k):
        st, src, _, _, outs, lses = runs[k % len(runs)]
        d = st.inp
        for t in range(2):
            B.sparsekv_attend(st.pr, d.q[:, t:], src, st.indices[:, t:], st.n_sel[:, t:], src, d.seq_lens,
                              outs[t], lses[t], st.ws)

    def cobatched(k):
        st, src, out2, lse2, _, _ = runs[k % len(runs)]
        d = st.inp
        B.sparsekv_attend_cobatched(st.pr, d.q, src, st.indices, st.n_sel, src, d.seq_lens, out2, lse2, st.ws)

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn) -> float:
        for k in range(5):
            fn(k)
        torch.cuda.synchronize()
        ev[0].record()
        for k in range(reps):
            fn(k)
        ev[1].record()
        ev[1].synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / reps

    # interleave the two so that both see the same clocks
    t_two, t_cob = [], []
    for _ in range(3):
        t_two.append(timed(two_launches))
        t_cob.append(timed(cobatched))
    t_two, t_cob = statistics.median(t_two), statistics.median(t_cob)
    # the two outputs agree (same values up to fp32 summation order)
    st, _, out2, lse2, outs, lses = runs[0]
    two_launches(0)
    cobatched(0)
    torch.cuda.synchronize()
    diff = max((out2[:, t] - outs[t]).abs().max().item() for t in range(2))

    chunk = 2 * wl.block_size * wl.head_dim * ELEM_BYTES[wl.kv_dtype] + 8
    idx, nsel = st.indices.cpu().numpy(), st.n_sel.cpu().numpy()
    union = sel = 0
    for b in range(wl.batch):
        for g in range(wl.n_kv_heads):
            a0 = set(idx[b, 0, g, :nsel[b, 0, g]].tolist())
            a1 = set(idx[b, 1, g, :nsel[b, 1, g]].tolist())
            union += len(a0 | a1)
            sel += len(a0) + len(a1)
    lens = st.inp.seq_lens.cpu().numpy()
    win = sum(wl.n_kv_heads * min(wl.window, int(L)) * 2 * wl.head_dim * ELEM_BYTES[wl.kv_dtype] for L in lens)
    qo = wl.batch * 2 * wl.n_q_heads * (wl.head_dim * 2 + (wl.head_dim + 1) * 4)
    cob_bytes = union * chunk + win + qo
    print(json.dumps({
        "probe": "cobatched_attention", "workload": "dual (B4, L262144, Hq64/Hkv8, blk64, k128, W1024, fp8)",
        "reps": reps, "instances": instances,
        "two_launches_us": round(t_two, 2), "cobatched_us": round(t_cob, 2),
        "saving": round(1 - t_cob / t_two, 3), "max_abs_diff": diff,
        "selected_blocks_two_tokens": sel, "union_blocks": union,
        "cobatched_bytes": cob_bytes, "cobatched_gbps": round(cob_bytes / (t_cob * 1e-6) / 1e9, 1),
        "two_launch_bytes": sel * chunk + 2 * win + qo}), flush=True)
    return 0


def hybrid_probe(reps: int) -> int:
    """Host workload, one layer-step: the hybrid step (selected blocks attended
    by the host in place, window on the GPU, LSE fusion) against the all-GPU
    host-pool step (selected blocks gathered over the host link, then attended
    on the GPU).  Wall time per call, the device synchronised after each batch."""
    import torch

    from sparse_kv_cache_block_amd import configs
    from sparse_kv_cache_block_amd.configs import ELEM_BYTES
    from sparse_kv_cache_block_amd.inputs import make_inputs
    from sparse_kv_cache_block_amd.step import DecodeStep, HybridHost, to_device_for

    wl = configs.HOST
    torch.cuda.set_device(0)
    st = DecodeStep(to_device_for(make_inputs(wl, device="cuda", instance=0)))
    host = HybridHost(st)
    for _ in range(3):
        st.run()
        st.run_hybrid(host)
    torch.cuda.synchronize()

    def timed(fn) -> float:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / reps

    t_gpu, t_hyb = [], []
    for _ in range(3):
        t_gpu.append(timed(st.run))
        t_hyb.append(timed(lambda: st.run_hybrid(host)))
    t_gpu, t_hyb = statistics.median(t_gpu), statistics.median(t_hyb)
    nsel = int(st.n_sel[:, 0].sum())
    kv_bytes = nsel * 2 * wl.block_size * wl.head_dim * ELEM_BYTES[wl.kv_dtype]
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    print(json.dumps({
        "probe": "hybrid_step", "workload": "host (B8, L131072, Hq32/Hkv8, blk64, k32, W512, bf16, pinned pool)",
        "reps": reps, "gpu_host_path_us": round(t_gpu, 1), "hybrid_us": round(t_hyb, 1),
        "speedup": round(t_gpu / t_hyb, 3), "selected_kv_bytes": kv_bytes,
        "gpu_path_link_gbps": round(kv_bytes / (t_gpu * 1e-6) / 1e9, 1),
        "hybrid_host_gbps": round(kv_bytes / (t_hyb * 1e-6) / 1e9, 1), "host_threads": threads}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama32k",
                    help="llama32k (default), ragged, host, dual or tiny")
    ap.add_argument("--instances", type=int, default=3)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 disables it)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--gather-correct", action="store_true",
                    help="only compare the full host gather with the speculative correction and exit")
    ap.add_argument("--hybrid", action="store_true",
                    help="only compare the hybrid CPU-GPU step with the all-GPU host-pool step and exit")
    ap.add_argument("--gather", action="store_true",
                    help="only time the stand-alone gather from the HBM pool (llama32k) and exit")
    ap.add_argument("--cobatched", action="store_true",
                    help="only compare co-batched two-token attention with one launch per token and exit")
    ap.add_argument("--layers-predicted", action="store_true",
                    help="only compare the predicted-prefetch layer pipeline with the plain one and exit")
    ap.add_argument("--others", default="ragged,dual,host,tiny",
                    help="after the headline workload, time these workloads in the same process and add "
                         "their figures to the line as other_workloads ('none': skip)")
    args = ap.parse_args()
    if args.copy_probe:
        return copy_probe(args.copy_probe, max(1, args.steps))
    if args.gather_correct:
        return gather_correct_probe(max(1, min(args.steps, 50)))
    if args.cobatched:
        return cobatched_probe(max(1, args.steps), max(1, args.instances))
    if args.gather:
        return hbm_gather_probe(max(1, args.steps), max(1, args.instances))
    if args.hybrid:
        return hybrid_probe(max(1, min(args.steps, 50)))
    if args.layers_predicted:
        return predicted_layers_probe(max(1, min(args.steps, 30)))

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs the single-GPU decode step only; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported: each (sequence, KV head) pair is "
              "independent, so more GPUs would each run this same kernel on their own share.",
              file=sys.stderr)
        return 2

    import gc

    import torch

    line = run_workload(args, args.workload, args.cpu_budget)
    others = [w for w in args.others.split(",") if w and w != "none" and w != args.workload]
    if others:
        line["other_workloads"] = []
        for name in others:
            gc.collect()
            torch.cuda.empty_cache()
            o = run_workload(args, name, 0.0)
            keep = ("ms_per_step", "value", "unit", "step_bytes", "step_gbps", "step_frac_of_peak",
                    "step_us_p10_p50_p90", "launches_per_step", "kernels", "overlap_mean", "host_link")
            entry = {"workload": name, "config": o["config"]}
            entry.update({k: o[k] for k in keep if k in o})
            if o.get("roofline"):
                entry["roofline_frac"] = o["roofline"]["frac"]
                entry["frac_of_read_ceiling"] = o["roofline"]["frac_of_read_ceiling"]
            line["other_workloads"].append(entry)
    print(json.dumps(line), flush=True)
    return 0


def run_workload(args, name: str, cpu_budget: float) -> dict:
    """Times one workload's decode step (args.warmup untimed, args.steps timed
    over args.instances input sets) and returns its bench line."""
    import numpy as np
    import torch

    from sparse_kv_cache_block_amd import binding as B
    from sparse_kv_cache_block_amd import configs
    from sparse_kv_cache_block_amd.inputs import make_inputs
    from sparse_kv_cache_block_amd.step import DecodeStep, LayerPipeline, to_device_for

    wl = configs.get(name)
    torch.cuda.set_device(0)
    B.lib()
    log(f"workload {name}")

    # ---- inputs: independent instances generated on the GPU
    steps = []
    host_inputs = None
    for i in range(args.instances):
        t0 = time.perf_counter()
        inp = make_inputs(wl, device="cuda", instance=i)
        if i == 0 and cpu_budget > 0:
            host_inputs = inp.to("cpu")
        if wl.pool == "host":
            inp = to_device_for(inp)   # the K/V pool moves to pinned host memory
        st = DecodeStep(inp)
        steps.append(st)
        torch.cuda.synchronize()
        log(f"instance {i} ready in {time.perf_counter() - t0:.1f}s")

    n_layers = wl.n_layers if wl.pool == "host" else 1
    copy_stream = torch.cuda.Stream() if wl.pool == "host" else None
    # host pool: n_layers layer-steps sharing the instance's pool, landmarks and
    # query, through the two-slot staging pipeline
    pipes = [LayerPipeline([st.inp] * n_layers) for st in steps] if wl.pool == "host" else None

    def one_step(k: int) -> None:
        if pipes:
            pipes[k % len(pipes)].run(copy_stream=copy_stream)
        else:
            steps[k % len(steps)].run()

    for k in range(args.warmup):
        one_step(k)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for k in range(args.steps):
        one_step(k)
    ev1.record(stream)
    ev1.synchronize()
    wall1 = time.perf_counter()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    wall_ms = (wall1 - wall0) * 1e3 / args.steps
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (wall {wall_ms * 1e3:.1f} us)")

    # per-step spread: a separate pass with an event after every step (the
    # events sit between launches and add about 2 us per step, so this pass
    # gives the spread, not the rate)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for k in range(args.steps):
        one_step(k)
        evs[k + 1].record(stream)
    evs[-1].synchronize()
    per_step = sorted(evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(args.steps))

    def pct(q: float) -> float:
        return round(per_step[min(len(per_step) - 1, int(q * len(per_step)))], 2)

    # the steps rotate over the instances, whose lengths differ for ragged
    # batches: a step moves the mean of their algorithmic bytes
    shapes = [(st.inp.seq_lens.cpu().numpy(), st.inp.k_per_seq.cpu().numpy()) for st in steps]
    bytes_per_instance = [configs.algorithmic_bytes(wl, L, K) for L, K in shapes]
    step_bytes = statistics.mean(bytes_per_instance)
    tokens_per_s = wl.batch * n_layers / (ms_per_step * 1e-3)

    # ---- per-kernel figures.  One launch: the step kernel is the step.  Two
    # launches (device pool): each launch of the step is timed between events
    # recorded around it (sparsekv_decode_step_launch_times), over the same
    # instances; the kernels are the ones the plan names (the scoring launch,
    # then the attention or the split step's selection + attention).  Host
    # pool: the gather (pinned pool -> stage, over the host link) and the
    # attention of the staged blocks are each timed alone.
    launches = B.sparsekv_decode_step_launches(steps[0].pr)

    def timed_us(fn) -> float:
        for k in range(args.warmup):
            fn(k)
        torch.cuda.synchronize()
        ev0.record(stream)
        for k in range(args.steps):
            fn(k)
        ev1.record(stream)
        ev1.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / args.steps

    def entry(name, nbytes, us, bound="hbm", note=None):
        gbps = nbytes / (us * 1e-6) / 1e9
        e = {"kernel": name, "bytes_per_launch": int(nbytes), "us_per_launch": round(us, 2),
             "gbps": round(gbps, 1), "bound": bound}
        if bound == "hbm":
            e["frac_of_peak"] = round(gbps / HBM_PEAK_GBS, 4)
        if note:
            e["note"] = note
        return e

    # each instance's selection: the decode step's outputs, or for a host
    # pool those of layer 0 of its pipeline (every layer has the same inputs,
    # so the staging slots hold this selection's blocks)
    sels = [(p.outs[0]["indices"], p.outs[0]["n_sel"]) for p in pipes] if pipes else \
        [(st.indices, st.n_sel) for st in steps]

    def staged_attend_us() -> float:
        """The host pool's attention launch alone: staged blocks plus the HBM window."""
        srcs = []
        for i, st in enumerate(steps):
            d = st.inp
            pipe = pipes[i]
            sp = B.kv_source(B.SKV_SRC_STAGED, pipe.k_slots[0], pipe.v_slots[0],
                             pipe.k_slot_scales[0] if pipe.k_slot_scales else None,
                             pipe.v_slot_scales[0] if pipe.v_slot_scales else None)
            win = B.kv_source(B.SKV_SRC_WINDOW, d.window_k, d.window_v, d.window_k_scales,
                              d.window_v_scales) if wl.window else None
            srcs.append((st, sp, win, sels[i]))

        def one(k):
            st, sp, win, (idx, nsel) = srcs[k % len(srcs)]
            B.sparsekv_attend(st.pr, st.inp.q, sp, idx, nsel, win, st.inp.seq_lens, st.out, st.lse, st.ws)
        return timed_us(one)

    attn_bytes = statistics.mean(attention_bytes(wl, s.inp.seq_lens.cpu().numpy(), sel[1][:, 0].cpu().numpy())
                                 for s, sel in zip(steps, sels))
    e_l = configs.ELEM_BYTES[wl.landmark_dtype]
    score_bytes = statistics.mean(
        wl.n_kv_heads * sum(configs.n_candidates(int(L), wl.window, wl.block_size) for L in s.inp.seq_lens.cpu())
        * wl.head_dim * e_l + wl.batch * wl.n_q_tokens * wl.n_q_heads * wl.head_dim * configs.ELEM_BYTES[wl.q_dtype]
        for s in steps)
    kernels = []
    kernel = k_ms = k_bytes = None
    if launches == 1:
        kernel, k_ms, k_bytes = "pair_step_kernel", ms_per_step, step_bytes
        kernels.append(entry(kernel, k_bytes, k_ms * 1e3))
    elif wl.pool != "host":
        names = [B.sparsekv_decode_step_kernel(steps[0].pr, i) for i in range(launches)]
        reps = max(1, args.steps // len(steps))
        per = [B.sparsekv_decode_step_launch_times(st.pr, st.inputs, st.outputs, st.ws, reps) for st in steps]
        l_us = [statistics.mean(p[i] for p in per) for i in range(launches)]
        log("launches: " + ", ".join(f"{n} {u:.1f} us" for n, u in zip(names, l_us)))
        split = names[1] == "split_step_kernel"
        kernels.append(entry(names[0], score_bytes, l_us[0],
                             note="scoring with each chunk's own top-k' (its candidates published)" if split
                             else "scoring with the fused top-k"))
        kernels.append(entry(names[1], attn_bytes, l_us[1],
                             note="final top-k from the chunks' candidates, then attention" if split
                             else "attention of the selected blocks and the window"))
        kernel, k_ms, k_bytes = names[1], l_us[1] * 1e-3, attn_bytes
    else:
        a_us = staged_attend_us()
        kernels.append(entry("attend_kernel", attn_bytes, a_us,
                             note="staged blocks plus the HBM window, timed alone"))
        link = statistics.mean(configs.host_link_bytes(wl, s.inp.seq_lens.cpu(), s.inp.k_per_seq.cpu())
                               for s in steps)

        def gather(k):
            i = k % len(steps)
            st, pipe, (idx, nsel) = steps[i], pipes[i], sels[i]
            d = st.inp
            B.sparsekv_gather(st.pr, d.k_pool, d.v_pool, d.k_scales, d.v_scales, d.block_table, idx, nsel,
                              pipe.k_slots[0], pipe.v_slots[0], pipe.k_slot_scales and pipe.k_slot_scales[0],
                              pipe.v_slot_scales and pipe.v_slot_scales[0])
        g_us = timed_us(gather)
        kernels.append(entry("gather_kernel", link, g_us, bound="host_link",
                             note="selected K/V read over the host link (and written to the HBM stage), "
                                  "timed alone"))

    roofline = None
    if kernel:
        ceiling = read_ceiling_gbps()
        log(f"streaming-read ceiling: {ceiling:.0f} GB/s")
        achieved = k_bytes / (k_ms * 1e-3) / 1e9
        rec = recorded_traffic(kernel, wl.name)
        traffic = None
        if rec is not None:
            traffic = int(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])
        roofline = {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "bytes_per_launch": int(k_bytes),
                    "us_per_launch": round(k_ms * 1e3, 2),
                    "read_ceiling_gbps": round(ceiling, 1),
                    "frac_of_read_ceiling": round(achieved / ceiling, 4)}

    # ---- CPU oracle on a bounded sample of instance 0
    cpu = None
    if cpu_budget > 0 and host_inputs is not None:
        from oracle import oracle as O
        from tests.common import HostArrays, oracle_problem
        h = HostArrays(host_inputs)
        pr = oracle_problem(host_inputs)
        log("timing the CPU oracle")
        times = []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            O.decode_step(pr, h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens, h.k_per_seq)
            times.append(time.perf_counter() - t0)
            spent = time.perf_counter() - t_start
            if len(times) >= 100 or (len(times) >= 3 and spent > cpu_budget):
                break
        t = statistics.median(times)
        threads = O.max_threads()
        # the same steps on one thread (3, about the multi-thread sample's cost again)
        O.set_threads(1)
        t1 = []
        for _ in range(3):
            t0 = time.perf_counter()
            O.decode_step(pr, h.q, h.landmarks, *h.pools(), h.block_table, h.seq_lens, h.k_per_seq)
            t1.append(time.perf_counter() - t0)
        O.set_threads(threads)
        t1 = statistics.median(t1)
        cpu = {"value": round(wl.batch / t, 2), "unit": "tokens/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{len(times)} full {wl.name} decode steps (B={wl.batch}) on instance 0, "
                         f"fp64, median {t * 1e3:.1f} ms; 3 more on one thread, median {t1 * 1e3:.1f} ms",
               "gbps": round(bytes_per_instance[0] / t / 1e9, 3),
               "value_1_thread": round(wl.batch / t1, 2),
               "cpu_model": cpu_model()}

    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    cfg = {"workload": wl.name, "batch": wl.batch, "context": wl.context, "n_q_heads": wl.n_q_heads,
           "n_kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "block_size": wl.block_size,
           "top_k": wl.top_k, "window": wl.window, "kv_dtype": wl.kv_dtype,
           "n_q_tokens": wl.n_q_tokens, "pool": wl.pool, "instances": args.instances,
           "seed": wl.seed, "instance_ids": list(range(args.instances)),
           "generator": "numpy SeedSequence([seed, instance]).spawn(8) seeding torch cuda generators"}
    if n_layers > 1:
        cfg["layers_per_step"] = n_layers
    line = {
        "metric": "sparse decode steps: tokens/s and achieved HBM GB/s (% roofline) at 32k context",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp32": "f32", "bf16": "bf16", "fp8": "fp8e4m3"}[wl.kv_dtype],
        "data": "synthetic",
        "config": cfg,
        "step_bytes": int(step_bytes),
        "step_bytes_per_instance": [int(x) for x in bytes_per_instance],
        "step_gbps": round(step_gbps, 1),
        "step_frac_of_peak": round(step_gbps / HBM_PEAK_GBS, 4),
        "wall_ms_per_step": round(wall_ms, 5),
        "step_us_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "launches_per_step": launches,
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    if wl.n_q_tokens == 2:
        ov = pipes[0].outs[0]["overlap"] if pipes else steps[0].overlap
        line["overlap_mean"] = round(float(ov.mean().item()), 4)
    if wl.pool == "host":
        # the gather's pull over the host link, against a contiguous pinned copy
        link_bytes = n_layers * statistics.mean(configs.host_link_bytes(wl, L, K) for L, K in shapes)
        link_gbps = link_bytes / (ms_per_step * 1e-3) / 1e9
        ceiling = h2d_ceiling_gbps()
        line["host_link"] = {"bytes_per_step": int(link_bytes), "gbps": round(link_gbps, 2),
                             "h2d_ceiling_gbps": round(ceiling, 2), "frac": round(link_gbps / ceiling, 4),
                             "note": "whole-step time (scoring and attention included) over the "
                                     "gathered K/V bytes; ceiling = 64 MiB pinned hipMemcpyAsync"}
    return line


if __name__ == "__main__":
    sys.exit(main())
