"""kda_chunk_prefill_noalloc (the prefill whose workspace is the library's fixed
device scratch, for callers that cannot allocate) against kda_chunk_prefill
with a caller workspace, through the C ABI: two calls in a row on one GPU,
the second with a smaller input, each equal to the workspace call bit for
bit (the same kernels; the segments only split T). The first case needs
several segments of the 64 MiB scratch; the second fits in one. Also the
scratch's contents left by the first call do not leak into the second, and
the workspace-size rejection happens before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as kda
import workloads
from tests.gpu_util import device, load_state, to_dev

pytestmark = pytest.mark.gpu


def _pair(inp, chunk, io):
    """(o, S, ring) from the workspace call and from the scratch call."""
    dev = device()
    B, T, H, dk, dv = inp.dims
    d = to_dev(inp, dev)
    outs = []
    for noalloc in (False, True):
        st = kda.KDAState(B, H, dk, dv, io=io, device=dev)
        load_state(st, inp)
        o = torch.full((B, T, H, dv), float("nan"), dtype=io, device=dev)
        if noalloc:
            kda.kda_chunk_prefill_noalloc(st.handle, T, d["q"], d["k"], d["v"], d["g"],
                                          d["beta"], d["conv_w"], o, chunk=chunk, io=io)
        else:
            nbytes = kda.kda_prefill_workspace_bytes(st.dims, T, chunk)
            ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            kda.kda_chunk_prefill(st.handle, T, d["q"], d["k"], d["v"], d["g"], d["beta"],
                                  d["conv_w"], o, chunk=chunk, workspace=ws, io=io)
        torch.cuda.synchronize()
        outs.append((o.clone(), st.S.clone(), st.ring.clone()))
    return outs


def _same(a, b):
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))


def test_noalloc_equals_workspace_call_twice():
    # 1) 4 sequences x 96 heads of 128 x 128, bf16: one chunk of all heads is
    #    28.5 MB, so the 64 MiB scratch holds two chunks and T = 300 (five
    #    chunks) takes three segments
    big = workloads.make("tiny", T=300, B=4, H=96, dk=128, dv=128, io="bf16",
                         s0_random=True, ring_random=True, seed=1201)
    per_chunk = kda.kda_prefill_workspace_bytes(kda.make_dims(4, 96, 128, 128, kda.KDA_BF16),
                                                64, 64)
    assert 2 * per_chunk <= kda.KDA_NOALLOC_SCRATCH_BYTES < 3 * per_chunk
    a, b = _pair(big, 64, torch.bfloat16)
    assert torch.isfinite(b[0].float()).all()
    _same(a, b)
    # 2) a smaller input right after it on the same GPU (the scratch still
    #    holds the first call's blocks): fp32, another shape and chunk
    small = workloads.make("tiny", T=77, B=2, H=3, dk=64, dv=32, io="f32", s0_random=True,
                           ring_random=True, seed=1202)
    a, b = _pair(small, 32, torch.float32)
    assert torch.isfinite(b[0]).all()
    _same(a, b)


def test_noalloc_rejects_too_many_heads_before_launch():
    dev = device()
    # 12 x 96 heads of 128 x 128 at chunk 64: 85.5 MB per chunk > 64 MiB
    st = kda.KDAState(12, 96, 128, 128, io=torch.bfloat16, device=dev)
    before = st.S.clone()
    x = torch.zeros(12, 64, 96, 128, dtype=torch.bfloat16, device=dev)
    g = torch.zeros(12, 64, 96, 128, device=dev)
    beta = torch.zeros(12, 64, 96, device=dev)
    w = torch.zeros(96 * 384, 4, device=dev)
    o = torch.zeros_like(x)
    with pytest.raises(kda.KDAError) as e:
        kda.kda_chunk_prefill_noalloc(st.handle, 64, x, x, x, g, beta, w, o, chunk=64)
    assert e.value.status == -2 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(st.S, before)
