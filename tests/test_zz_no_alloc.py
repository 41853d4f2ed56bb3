"""The allocation-free decode step (its workspace a fixed device array of the
library) against sparsekv_decode_step with a caller's workspace, through the
C ABI, on consecutive calls of different sizes."""
import pytest
import torch

from sparse_kv_cache_block_amd import binding as B
from sparse_kv_cache_block_amd import configs
from sparse_kv_cache_block_amd.inputs import make_inputs
from sparse_kv_cache_block_amd.step import DecodeStep, to_device_for

pytestmark = pytest.mark.gpu


def _case(wl, instance=0):
    """A decode step with its own workspace, and output buffers for the no-alloc call."""
    st = DecodeStep(to_device_for(make_inputs(wl, device="cpu", instance=instance)))
    st.run()
    bufs = dict(indices=torch.full_like(st.indices, -7), n_sel=torch.full_like(st.n_sel, -7),
                out=torch.full_like(st.out, float("nan")), lse=torch.full_like(st.lse, float("nan")),
                overlap=None if st.overlap is None else torch.full_like(st.overlap, float("nan")))
    outs = B.step_outputs(bufs["indices"], bufs["n_sel"], bufs["out"], bufs["lse"], bufs["overlap"])
    return st, bufs, outs


def _check(st, bufs):
    # the same kernels on the same inputs: identical results
    assert torch.equal(bufs["indices"], st.indices)
    assert torch.equal(bufs["n_sel"], st.n_sel)
    assert torch.equal(bufs["out"], st.out)
    assert torch.equal(bufs["lse"], st.lse)
    if st.overlap is not None:
        assert torch.equal(bufs["overlap"], st.overlap)


CASES = [
    configs.LLAMA32K.scaled(batch=16, context=4096),                   # one launch, 128 pairs
    configs.LLAMA32K.scaled(batch=2, context=2048, top_k=8),           # smaller: two launches
    configs.DUAL.scaled(batch=2, context=16384, top_k=30),             # fp8, two tokens, split scoring rows
    configs.RAGGED.scaled(batch=40, context=8192),                     # one launch, 320 pairs, longest first
    configs.LLAMA32K.scaled(batch=2, n_q_heads=8, n_kv_heads=2, context=131072, top_k=16,
                            n_q_tokens=2, spec_noise=0.3),             # split step: chunks' candidates, then
                                                                       # selection and attention per split
]


def test_noalloc_matches_workspace_step_on_consecutive_calls():
    order = [0, 1, 2, 3, 4, 1, 0]   # each call after one of another size; the second is smaller than the first
    prepared = {}
    for i in order:
        wl = CASES[i]
        print(f"[case] decode_step_noalloc {wl.name} B={wl.batch} L={wl.context} kv={wl.kv_dtype} "
              f"T={wl.n_q_tokens}", flush=True)
        if i not in prepared:
            prepared[i] = _case(wl, instance=i)
            torch.cuda.synchronize()
        st, bufs, outs = prepared[i]
        for t in bufs.values():
            if t is not None:
                t.fill_(-7 if t.dtype == torch.int32 else float("nan"))
        B.sparsekv_decode_step_noalloc(st.pr, st.inputs, outs)
        torch.cuda.synchronize()
        _check(st, bufs)
