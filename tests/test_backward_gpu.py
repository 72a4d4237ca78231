"""GPU parity of kda_chunk_backward (the chunked gradient of the recurrence)
against the oracle's sequential fp64 gradient (kdao_core_backward, pinned to
central finite differences of the forward oracle).

Inputs: the seeded workloads of workloads.py; the activations q^, k^, v^ come
from the oracle's prologue (conv, SiLU, L2) of the raw draws, rounded to the
I/O type, and feed both sides; dO and dST from workloads.draw_backward_grads.
Tolerance (max |gpu - oracle| / max |oracle| per gradient tensor): 1e-4 for
fp32 I/O (fp32 arithmetic over chunk-length sums of products); 2e-2 for bf16
I/O (bf16 rounding of dq, dk, dv on output)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as kda
import workloads
from oracle import kda_oracle
from tests.gpu_util import device, f64, rel_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ["dq", "dk", "dv", "dg", "dbeta", "dS0"]


def activations(inp):
    """q^, k^, v^ from the oracle prologue, in the workload's I/O type."""
    qh, kh, vh = kda_oracle.prologue(inp.q, inp.k, inp.v, inp.conv_w, inp.ring0)[:3]
    tt = inp.q.dtype
    return [torch.from_numpy(np.ascontiguousarray(x)).to(tt) for x in (qh, kh, vh)]


def run_gpu(inp, qh, kh, vh, dO, dST, chunk, S0=True, want_dS0=True):
    dev = device()
    B, T, H, dk, dv = inp.dims
    io = inp.q.dtype
    dims = kda.make_dims(B, H, dk, dv, io)
    out = dict(dq=torch.empty(B, T, H, dk, dtype=io, device=dev),
               dk=torch.empty(B, T, H, dk, dtype=io, device=dev),
               dv=torch.empty(B, T, H, dv, dtype=io, device=dev),
               dg=torch.empty(B, T, H, dk, device=dev),
               dbeta=torch.empty(B, T, H, device=dev),
               dS0=torch.empty(B, H, dk, dv, device=dev) if want_dS0 else None)
    kda.kda_chunk_backward(
        dims, T, qh.to(dev), kh.to(dev), vh.to(dev), inp.g.to(dev), inp.beta.to(dev),
        inp.S0.to(dev) if S0 else None, dO.to(dev), dST.to(dev) if dST is not None else None,
        out["dq"], out["dk"], out["dv"], out["dg"], out["dbeta"], out["dS0"], chunk=chunk)
    torch.cuda.synchronize()
    return out


def check(inp, chunk, io, S0=True, use_dST=True, heads=None):
    B, T, H, dk, dv = inp.dims
    qh, kh, vh = activations(inp)
    dO, dST = workloads.draw_backward_grads(B, T, H, dk, dv, io=io, seed=inp.meta["seed"])
    got = run_gpu(inp, qh, kh, vh, dO, dST if use_dST else None, chunk, S0=S0)
    hs = list(range(H)) if heads is None else list(heads)
    S0r = inp.S0 if S0 else torch.zeros_like(inp.S0)
    dSTr = dST if use_dST else torch.zeros_like(dST)
    ref = kda_oracle.default().core_backward(
        qh[:, :, hs], kh[:, :, hs], vh[:, :, hs], inp.g[:, :, hs], inp.beta[:, :, hs],
        S0r[:, hs], dO[:, :, hs], dSTr[:, hs])
    errs = {}
    for name, r in zip(NAMES, ref):
        g = f64(got[name])
        g = g[:, hs] if name == "dS0" else g[:, :, hs]
        errs[name] = rel_err(g, r)
    print(f"backward {inp.dims} chunk={chunk} {io}: " +
          " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for name, e in errs.items():
        assert e <= TOL[io], (name, e)
    return errs


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_backward_tiny(chunk):
    inp = workloads.make("tiny", s0_random=True, ring_random=True)
    check(inp, chunk, "f32")


@pytest.mark.parametrize("B,T,H,dk,dv,chunk", [
    (2, 100, 3, 32, 64, 32),     # ragged last chunk, two sequences
    (1, 37, 2, 64, 16, 16),
    (1, 50, 2, 16, 128, 64),     # one partial chunk
    (1, 130, 2, 128, 128, 64),   # the K3 head shape, ragged
])
def test_backward_shapes_f32(B, T, H, dk, dv, chunk):
    inp = workloads.draw(B, T, H, dk, dv, io="f32", seed=11, s0_random=True,
                         ring_random=True)
    check(inp, chunk, "f32")


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 32)])
def test_backward_bf16(dk, dv):
    inp = workloads.draw(1, 130, 2, dk, dv, io="bf16", seed=12, s0_random=True,
                         ring_random=True, g_mu=2.0)
    check(inp, 64, "bf16")


def test_backward_zero_state_and_no_state_gradient():
    inp = workloads.draw(1, 70, 2, 32, 32, io="f32", seed=13)
    check(inp, 32, "f32", S0=False, use_dST=False)


def test_backward_strong_decay():
    # decays far below what the forward prefill accepts (the backward forms
    # every factor as the exponential of a non-positive difference)
    inp = workloads.draw(1, 96, 2, 32, 32, io="f32", seed=14, s0_random=True)
    inp.g = -torch.rand(inp.g.shape, generator=torch.Generator().manual_seed(1)) * 40.0
    check(inp, 64, "f32")


def test_backward_zero_tokens_passes_state_gradient_through():
    dev = device()
    dims = kda.make_dims(2, 3, 16, 32, kda.KDA_F32)
    dST = torch.randn(2, 3, 16, 32, device=dev)
    dS0 = torch.full_like(dST, float("nan"))
    kda.kda_chunk_backward(dims, 0, None, None, None, None, None, None, None, dST, None, None,
                           None, None, None, dS0, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(dS0, dST)
    kda.kda_chunk_backward(dims, 0, None, None, None, None, None, None, None, None, None, None,
                           None, None, None, dS0, chunk=64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dS0).item() == 0


def test_backward_full_size_prefill_4k():
    """The 4096-token, 96-head, 128 x 128 bf16 workload; heads 0 and 95
    checked in full against the oracle (heads are independent)."""
    inp = workloads.make("prefill_4k", s0_random=True)
    check(inp, 64, "bf16", heads=[0, 95])


def test_backward_ignores_workspace_contents_and_is_deterministic():
    """A workspace filled with NaN gives the same gradients, bit for bit, as a
    zeroed one (no stage reads scratch it has not written), and two calls in
    a row agree bitwise; ragged last chunk, two sequences, bf16."""
    dev = device()
    inp = workloads.draw(2, 150, 3, 64, 128, io="bf16", seed=15, s0_random=True,
                         ring_random=True)
    B, T, H, dk, dv = inp.dims
    qh, kh, vh = activations(inp)
    dO, dST = workloads.draw_backward_grads(B, T, H, dk, dv, io="bf16", seed=15)
    dims = kda.make_dims(B, H, dk, dv, torch.bfloat16)
    ws = torch.empty(kda.kda_backward_workspace_bytes(dims, T, 64), dtype=torch.uint8,
                     device=dev)
    ins = [x.to(dev) for x in (qh, kh, vh, inp.g, inp.beta, inp.S0, dO, dST)]

    def call(fill):
        if fill == "nan":
            ws.view(torch.float32).fill_(float("nan"))
        else:
            ws.zero_()
        out = [torch.empty(B, T, H, dk, dtype=torch.bfloat16, device=dev),
               torch.empty(B, T, H, dk, dtype=torch.bfloat16, device=dev),
               torch.empty(B, T, H, dv, dtype=torch.bfloat16, device=dev),
               torch.empty(B, T, H, dk, device=dev), torch.empty(B, T, H, device=dev),
               torch.empty(B, H, dk, dv, device=dev)]
        kda.kda_chunk_backward(dims, T, *ins, *out, chunk=64, workspace=ws)
        torch.cuda.synchronize()
        return out

    a, b, c = call("zero"), call("nan"), call("nan")
    for x, y, z in zip(a, b, c):
        assert torch.isfinite(x.float()).all()
        assert torch.equal(x, y) and torch.equal(y, z)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dk,dv", [(a, b) for a in (16, 32, 64, 128) for b in (16, 32, 64, 128)])
def test_backward_every_shape(dk, dv, chunk, io):
    """Every supported (d_k, d_v, chunk, I/O type): 70 tokens (a ragged last
    chunk for every chunk size), two sequences, random S0 and ring."""
    inp = workloads.draw(2, 70, 2, dk, dv, io=io, seed=31, s0_random=True, ring_random=True)
    check(inp, chunk, io)
