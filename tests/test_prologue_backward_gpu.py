"""GPU parity of kda_prologue_backward (the gradient of the conv, SiLU and L2
prologue) against the oracle's kdao_prologue_backward (pinned to central
finite differences of the oracle's forward prologue), and of the two
backward calls chained against the two oracle gradients chained.

Inputs: the seeded workloads of workloads.py (raw q, k, v, conv weights and
a random ring as the history), activation gradients from
workloads.draw_prologue_grads. Tolerance (max |gpu - oracle| / max |oracle|
per gradient tensor): 1e-4 for fp32 I/O, 2e-2 for bf16 I/O."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as kda
import workloads
from oracle import kda_oracle
from tests.gpu_util import channels, device, f64, rel_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def run(inp, dqh, dkh, dvh, with_ring=True, want_dring=True):
    dev = device()
    B, T, H, dk, dv = inp.dims
    io = inp.q.dtype
    dims = kda.make_dims(B, H, dk, dv, io)
    ctot = H * (2 * dk + dv)
    out = dict(dq=torch.empty(B, T, H, dk, dtype=io, device=dev),
               dk=torch.empty(B, T, H, dk, dtype=io, device=dev),
               dv=torch.empty(B, T, H, dv, dtype=io, device=dev),
               dw=torch.full((ctot, 4), float("nan"), device=dev),
               dring=torch.full((B, 3, ctot), float("nan"), device=dev) if want_dring else None)
    kda.kda_prologue_backward(
        dims, T, inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.conv_w.to(dev),
        inp.ring0.to(dev) if with_ring else None, dqh.to(dev), dkh.to(dev), dvh.to(dev),
        out["dq"], out["dk"], out["dv"], out["dw"], out["dring"])
    torch.cuda.synchronize()
    return out


def check(inp, io, with_ring=True, heads=None):
    B, T, H, dk, dv = inp.dims
    dqh, dkh, dvh = workloads.draw_prologue_grads(B, T, H, dk, dv, io=io, seed=inp.meta["seed"])
    got = run(inp, dqh, dkh, dvh, with_ring=with_ring)
    hs = list(range(H)) if heads is None else list(heads)
    ch = channels(H, dk, dv, hs)
    ring = inp.ring0 if with_ring else torch.zeros_like(inp.ring0)
    ref = kda_oracle.default().prologue_backward(
        inp.q[:, :, hs], inp.k[:, :, hs], inp.v[:, :, hs], inp.conv_w[ch], ring[:, :, ch],
        dqh[:, :, hs], dkh[:, :, hs], dvh[:, :, hs])
    errs = {
        "dq": rel_err(f64(got["dq"])[:, :, hs], ref[0]),
        "dk": rel_err(f64(got["dk"])[:, :, hs], ref[1]),
        "dv": rel_err(f64(got["dv"])[:, :, hs], ref[2]),
        "dconv_w": rel_err(f64(got["dw"])[ch], ref[3]),
        "dring": rel_err(f64(got["dring"])[:, :, ch], ref[4]) if with_ring else 0.0,
    }
    print(f"prologue backward {inp.dims} {io}: " +
          " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for name, e in errs.items():
        assert e <= TOL[io], (name, e)


def test_prologue_backward_tiny():
    check(workloads.make("tiny", ring_random=True), "f32")


@pytest.mark.parametrize("B,T,H,dk,dv", [
    (2, 130, 3, 32, 64),    # ragged last segment, two sequences
    (1, 2, 2, 16, 16),      # fewer tokens than the conv history
    (1, 67, 2, 128, 16),    # the segment halo reaches the end exactly
])
def test_prologue_backward_shapes_f32(B, T, H, dk, dv):
    check(workloads.draw(B, T, H, dk, dv, io="f32", seed=21, ring_random=True), "f32")


def test_prologue_backward_bf16():
    check(workloads.draw(1, 200, 2, 128, 128, io="bf16", seed=22, ring_random=True), "bf16")


def test_prologue_backward_without_ring():
    inp = workloads.draw(1, 50, 2, 64, 32, io="f32", seed=23, ring_random=True)
    check(inp, "f32", with_ring=False)


def test_prologue_backward_zero_tokens():
    dev = device()
    dims = kda.make_dims(2, 3, 16, 32, kda.KDA_F32)
    ctot = 3 * (2 * 16 + 32)
    dw = torch.full((ctot, 4), float("nan"), device=dev)
    dring = torch.full((2, 3, ctot), float("nan"), device=dev)
    kda.kda_prologue_backward(dims, 0, None, None, None, torch.zeros(ctot, 4, device=dev), None,
                              None, None, None, None, None, None, dw, dring)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw).item() == 0 and torch.count_nonzero(dring).item() == 0


def test_prologue_backward_full_size_prefill_4k():
    """The 4096-token, 96-head bf16 workload with a random ring; heads 0 and
    95 (their channels of every output) checked against the oracle."""
    check(workloads.make("prefill_4k", ring_random=True), "bf16", heads=[0, 95])


def test_training_gradient_chained():
    """kda_chunk_backward then kda_prologue_backward: the gradient of the whole
    forward (prologue and recurrence) with respect to the raw projections,
    the conv weights, the ring, g, beta and S0, against the two oracle
    gradients chained the same way."""
    dev = device()
    inp = workloads.draw(2, 100, 2, 32, 32, io="f32", seed=24, s0_random=True, ring_random=True)
    B, T, H, dk, dv = inp.dims
    dims = kda.make_dims(B, H, dk, dv, torch.float32)
    orc = kda_oracle.default()
    qh, kh, vh = orc.prologue(inp.q, inp.k, inp.v, inp.conv_w, inp.ring0)[:3]
    dO, dST = workloads.draw_backward_grads(B, T, H, dk, dv, io="f32", seed=24)
    ref_core = orc.core_backward(qh, kh, vh, inp.g, inp.beta, inp.S0, dO, dST)
    ref_pro = orc.prologue_backward(inp.q, inp.k, inp.v, inp.conv_w, inp.ring0, *ref_core[:3])
    # GPU: the activations from the library's own prologue, then both backward calls
    acts = [torch.empty(B, T, H, d, device=dev) for d in (dk, dk, dv)]
    ring = inp.ring0.to(dev)
    kda.kda_conv_prologue(dims, T, inp.q.to(dev), inp.k.to(dev), inp.v.to(dev),
                          inp.conv_w.to(dev), ring.clone(), *acts)
    g1 = [torch.empty_like(acts[0]), torch.empty_like(acts[1]), torch.empty_like(acts[2]),
          torch.empty(B, T, H, dk, device=dev), torch.empty(B, T, H, device=dev),
          torch.empty(B, H, dk, dv, device=dev)]
    kda.kda_chunk_backward(dims, T, *acts, inp.g.to(dev), inp.beta.to(dev), inp.S0.to(dev),
                           dO.to(dev), dST.to(dev), *g1, chunk=64)
    ctot = H * (2 * dk + dv)
    g2 = [torch.empty(B, T, H, dk, device=dev), torch.empty(B, T, H, dk, device=dev),
          torch.empty(B, T, H, dv, device=dev), torch.empty(ctot, 4, device=dev),
          torch.empty(B, 3, ctot, device=dev)]
    kda.kda_prologue_backward(dims, T, inp.q.to(dev), inp.k.to(dev), inp.v.to(dev),
                              inp.conv_w.to(dev), ring, g1[0], g1[1], g1[2], *g2)
    torch.cuda.synchronize()
    pairs = [("dq", g2[0], ref_pro[0]), ("dk", g2[1], ref_pro[1]), ("dv", g2[2], ref_pro[2]),
             ("dconv_w", g2[3], ref_pro[3]), ("dring", g2[4], ref_pro[4]),
             ("dg", g1[3], ref_core[3]), ("dbeta", g1[4], ref_core[4]),
             ("dS0", g1[5], ref_core[5])]
    errs = {n: rel_err(f64(a), b) for n, a, b in pairs}
    print("chained training gradient: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= 1e-4, (n, e)


def test_training_backward_in_captured_graph_matches_eager():
    """Both backward calls with caller workspaces launch only kernels, so they
    can be captured in one HIP graph: each replay (outputs overwritten with
    NaN by eager work in between) gives the eager gradients bit for bit."""
    dev = device()
    inp = workloads.draw(1, 150, 2, 128, 64, io="bf16", seed=25, s0_random=True,
                         ring_random=True)
    B, T, H, dk, dv = inp.dims
    bf = torch.bfloat16
    dims = kda.make_dims(B, H, dk, dv, bf)
    ctot = H * (2 * dk + dv)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    w, ring = inp.conv_w.to(dev), inp.ring0.to(dev)
    g, beta, S0 = inp.g.to(dev), inp.beta.to(dev), inp.S0.to(dev)
    acts = [torch.empty(B, T, H, d, device=dev) for d in (dk, dk, dv)]
    kda.kda_conv_prologue(dims, T, q, k, v, w, ring.clone(), *acts)
    qh, kh, vh = (x.to(bf) for x in acts)
    dO, dST = (x.to(dev) for x in workloads.draw_backward_grads(B, T, H, dk, dv, io="bf16",
                                                                  seed=25))
    ws1 = torch.empty(kda.kda_backward_workspace_bytes(dims, T, 64), dtype=torch.uint8,
                      device=dev)
    ws2 = torch.empty(kda.kda_prologue_backward_workspace_bytes(dims, T), dtype=torch.uint8,
                      device=dev)

    def outputs():
        return [torch.empty(B, T, H, dk, dtype=bf, device=dev),
                torch.empty(B, T, H, dk, dtype=bf, device=dev),
                torch.empty(B, T, H, dv, dtype=bf, device=dev),
                torch.empty(B, T, H, dk, device=dev), torch.empty(B, T, H, device=dev),
                torch.empty(B, H, dk, dv, device=dev),
                torch.empty(B, T, H, dk, dtype=bf, device=dev),
                torch.empty(B, T, H, dk, dtype=bf, device=dev),
                torch.empty(B, T, H, dv, dtype=bf, device=dev),
                torch.empty(ctot, 4, device=dev), torch.empty(B, 3, ctot, device=dev)]

    def call(o):
        kda.kda_chunk_backward(dims, T, qh, kh, vh, g, beta, S0, dO, dST, *o[:6], chunk=64,
                               workspace=ws1)
        kda.kda_prologue_backward(dims, T, q, k, v, w, ring, o[0], o[1], o[2], *o[6:],
                                  workspace=ws2)

    eager, cap = outputs(), outputs()
    call(cap)  # warm-up, eager
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        call(eager)
        torch.cuda.synchronize()
        for t in cap:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(cap, eager)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs"


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(a, b) for a in (16, 32, 64, 128) for b in (16, 32, 64, 128)])
def test_prologue_backward_every_shape(dk, dv, io):
    """Every supported (d_k, d_v, I/O type): 70 tokens (three segments, the
    last ragged), two sequences, a random ring."""
    check(workloads.draw(2, 70, 2, dk, dv, io=io, seed=32, ring_random=True), io)
