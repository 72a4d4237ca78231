"""Robustness of the boundary on the GPU.

- Caller workspaces are scratch: a call whose workspace is filled with NaN
  gives results bitwise equal to the same call on a zero-filled one (every
  workspace byte a kernel reads was written earlier in the same call), for
  the prefill (one-shot and segmented), the backward and the prologue's
  backward.
- The session state is S plus the 3-token conv ring ("KDA 递推公式先衰减再差分":
  the short convolution keeps the last tokens of the previous step): saving
  both (on the device or in host memory), resetting, running other work on
  the handle, and restoring them gives a decode bitwise equal to an
  uninterrupted one.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as kda
import workloads
from tests.gpu_util import device, f64, load_state, run_decode, to_dev
from tests.test_backward_gpu import activations

pytestmark = pytest.mark.gpu

NAN = float("nan")


def _ws(nbytes, fill, dev):
    """A workspace of nbytes (+ 16 spare) filled with float NaN or zeros."""
    w = torch.empty((nbytes + 16 + 3) // 4, dtype=torch.float32, device=dev)
    w.fill_(fill)
    return w


def _prefill(inp, dev, chunk, io, ws, flags=0):
    B, T, H, dk, dv = inp.dims
    d = to_dev(inp, dev)
    st = kda.KDAState(B, H, dk, dv, io=io, device=dev)
    load_state(st, inp)
    o = torch.empty(B, T, H, dv, dtype=io, device=dev)
    st.prefill(T, d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], o, chunk=chunk,
               workspace=ws, flags=flags)
    torch.cuda.synchronize()
    return st, o


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("chunk,segment_chunks", [(64, None), (16, None), (32, 3)])
@pytest.mark.parametrize("flags", [0, kda.KDA_F_SCALAR_G])
def test_prefill_nan_workspace_equals_zero_workspace(io, chunk, segment_chunks, flags):
    dev = device()
    scalar = bool(flags & kda.KDA_F_SCALAR_G)
    inp = workloads.make("tiny", T=203, B=2, H=3, dk=64, dv=64, io=io, s0_random=True,
                         ring_random=True, scalar_g=scalar, seed=1200 + chunk)
    B, T, H, dk, dv = inp.dims
    tio = torch.float32 if io == "f32" else torch.bfloat16
    dims = kda.make_dims(B, H, dk, dv, tio)
    if segment_chunks is None:
        nbytes = kda.kda_prefill_workspace_bytes(dims, T, chunk)
    else:
        nbytes = segment_chunks * kda.kda_prefill_workspace_bytes(dims, chunk, chunk)
    outs = []
    for fill in (0.0, NAN):
        st, o = _prefill(inp, dev, chunk, tio, _ws(nbytes, fill, dev), flags)
        outs.append((o, st.S.clone(), st.ring.clone()))
    (o0, S0, r0), (o1, S1, r1) = outs
    assert torch.isfinite(o0.float()).all() and torch.isfinite(S0).all()
    assert torch.equal(o0, o1) and torch.equal(S0, S1) and torch.equal(r0, r1)


def _backward(inp, ws, dev):
    B, T, H, dk, dv = inp.dims
    io = inp.q.dtype
    dims = kda.make_dims(B, H, dk, dv, io)
    dO, dST = workloads.draw_backward_grads(B, T, H, dk, dv, io="f32" if io == torch.float32
                                            else "bf16", seed=inp.meta["seed"])
    out = dict(dq=torch.empty(B, T, H, dk, dtype=io, device=dev),
               dk=torch.empty(B, T, H, dk, dtype=io, device=dev),
               dv=torch.empty(B, T, H, dv, dtype=io, device=dev),
               dg=torch.empty(B, T, H, dk, device=dev),
               dbeta=torch.empty(B, T, H, device=dev),
               dS0=torch.empty(B, H, dk, dv, device=dev))
    qh, kh, vh = activations(inp)
    kda.kda_chunk_backward(dims, T, qh.to(dev), kh.to(dev), vh.to(dev), inp.g.to(dev),
                           inp.beta.to(dev), inp.S0.to(dev), dO.to(dev), dST.to(dev),
                           out["dq"], out["dk"], out["dv"], out["dg"], out["dbeta"],
                           out["dS0"], chunk=64, workspace=ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_backward_nan_workspace_equals_zero_workspace(io):
    dev = device()
    inp = workloads.make("tiny", T=150, B=2, H=2, dk=64, dv=64, io=io, s0_random=True,
                         seed=1250)
    B, T, H, dk, dv = inp.dims
    nbytes = kda.kda_backward_workspace_bytes(kda.make_dims(B, H, dk, dv, inp.q.dtype), T, 64)
    zero = _backward(inp, _ws(nbytes, 0.0, dev), dev)
    nan = _backward(inp, _ws(nbytes, NAN, dev), dev)
    for name in zero:
        assert torch.isfinite(zero[name].float()).all(), name
        assert torch.equal(zero[name], nan[name]), name


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prologue_backward_nan_workspace_equals_zero_workspace(io):
    dev = device()
    tio = torch.float32 if io == "f32" else torch.bfloat16
    B, T, H, dk, dv = 2, 77, 2, 32, 64
    inp = workloads.make("tiny", T=T, B=B, H=H, dk=dk, dv=dv, io=io, ring_random=True,
                         seed=1260)
    dims = kda.make_dims(B, H, dk, dv, tio)
    gen = torch.Generator().manual_seed(1261)
    dqh = torch.randn(B, T, H, dk, generator=gen).to(tio)
    dkh = torch.randn(B, T, H, dk, generator=gen).to(tio)
    dvh = torch.randn(B, T, H, dv, generator=gen).to(tio)
    ctot = H * (2 * dk + dv)
    nbytes = kda.kda_prologue_backward_workspace_bytes(dims, T)
    res = []
    for fill in (0.0, NAN):
        outs = dict(dq=torch.empty(B, T, H, dk, dtype=tio, device=dev),
                    dk=torch.empty(B, T, H, dk, dtype=tio, device=dev),
                    dv=torch.empty(B, T, H, dv, dtype=tio, device=dev),
                    dw=torch.empty(ctot, 4, device=dev),
                    dring=torch.empty(B, 3, ctot, device=dev))
        kda.kda_prologue_backward(dims, T, inp.q.to(dev), inp.k.to(dev), inp.v.to(dev),
                                  inp.conv_w.to(dev), inp.ring0.to(dev, tio), dqh.to(dev),
                                  dkh.to(dev), dvh.to(dev), outs["dq"], outs["dk"], outs["dv"],
                                  outs["dw"], outs["dring"], workspace=_ws(nbytes, fill, dev))
        torch.cuda.synchronize()
        res.append(outs)
    for name in res[0]:
        assert torch.isfinite(res[0][name].float()).all(), name
        assert torch.equal(res[0][name], res[1][name]), name


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("where", ["device", "host"])
def test_save_reset_restore_decode(io, where):
    """prefill 70 tokens, decode 10, save (S, ring); reset and decode other
    tokens on the same handle; restore; decode the last 20: o and the final
    state are bitwise those of the run that never stopped."""
    dev = device()
    inp = workloads.make("tiny", T=100, B=3, H=2, dk=64, dv=32, s0_random=True,
                         ring_random=True, io="f32" if io == torch.float32 else "bf16",
                         seed=1300)
    B, T, H, dk, dv = inp.dims
    d = to_dev(inp, dev)
    sm = to_dev(inp, dev, step_major=True)
    noise = to_dev(workloads.make("tiny", T=9, B=B, H=H, dk=dk, dv=dv, seed=1301,
                                  io="f32" if io == torch.float32 else "bf16"), dev,
                   step_major=True)

    def steps(src, t0, n):
        part = {key: src[key][t0:t0 + n] for key in ("q", "k", "v", "g", "beta")}
        part["conv_w"] = d["conv_w"]
        return part

    def start():
        st = kda.KDAState(B, H, dk, dv, io=io, device=dev)
        load_state(st, inp)
        o = torch.empty(B, 70, H, dv, dtype=io, device=dev)
        part = {key: d[key][:, :70].contiguous() for key in ("q", "k", "v", "g", "beta")}
        st.prefill(70, part["q"], part["k"], part["v"], part["g"], part["beta"], d["conv_w"], o)
        o_a = run_decode(st, steps(sm, 70, 10), 10)
        return st, o_a

    # uninterrupted
    ref, _ = start()
    ref_o = run_decode(ref, steps(sm, 80, 20), 20)
    torch.cuda.synchronize()

    st, _ = start()
    target = "cpu" if where == "host" else dev
    saved_S, saved_ring = st.S.to(target, copy=True), st.ring.to(target, copy=True)
    torch.cuda.synchronize()
    st.reset()
    torch.cuda.synchronize()
    assert not st.S.any() and not st.ring.any()
    nz = {key: noise[key] for key in ("q", "k", "v", "g", "beta")}
    nz["conv_w"] = d["conv_w"]
    run_decode(st, nz, 9)  # other work on the handle in between
    torch.cuda.synchronize()
    assert st.S.abs().sum() > 0
    st.S.copy_(saved_S)
    st.ring.copy_(saved_ring)
    got_o = run_decode(st, steps(sm, 80, 20), 20)
    torch.cuda.synchronize()
    assert torch.equal(got_o, ref_o)
    assert torch.equal(st.S, ref.S) and torch.equal(st.ring, ref.ring)
    assert np.isfinite(f64(got_o)).all()
