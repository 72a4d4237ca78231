"""Degenerate inputs of the recurrence on the GPU, decode and prefill, against
the fp64 oracle: no update (beta = 0), full update with q = k (exact recall),
no decay (g = 0) over many chunks, a strong decay (-4.9 per token: 16-token
blocks decay by 73.5, past the factored diagonal tiles' limit, so those are
formed term by term), and all-zero q, k, v (the L2 step then divides 0 by
sqrt(eps)). Stronger and infinite decays: test_strong_decay_gpu.py.

Tolerances: fp32 max |err| <= 1e-4; bf16 max|err|/max|ref| <= 2e-2.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as kda
import workloads
from oracle import kda_oracle
from tests.gpu_util import abs_err, device, f64, load_state, rel_err, run_decode, to_dev

pytestmark = pytest.mark.gpu


def _case(kind, io, T):
    inp = workloads.make("tiny", T=T, B=2, H=2, dk=64, dv=64, io=io, s0_random=True,
                         ring_random=True, seed=700 + len(kind))
    dt = inp.q.dtype
    if kind == "beta0":
        inp.beta = torch.zeros_like(inp.beta)
    elif kind == "recall":
        inp.beta = torch.ones_like(inp.beta)
        # q gets k's raw inputs, conv weights and history, so q^ = k^ exactly
        hd = inp.q.shape[2] * inp.q.shape[3]
        inp.q = inp.k.clone()
        inp.conv_w[:hd] = inp.conv_w[hd:2 * hd]
        inp.ring0[:, :, :hd] = inp.ring0[:, :, hd:2 * hd]
    elif kind == "nodecay":
        inp.g = torch.zeros_like(inp.g)
    elif kind == "strong":
        inp.g = torch.full_like(inp.g, -4.9)
    elif kind == "zeros":
        inp.q, inp.k, inp.v = (torch.zeros_like(x) for x in (inp.q, inp.k, inp.v))
        inp.ring0 = torch.zeros_like(inp.ring0)
    assert inp.q.dtype == dt
    return inp


def _check(got_o, got_S, ref_o, ref_S, io):
    if io == "f32":
        eo, es = abs_err(got_o, ref_o), abs_err(got_S, ref_S)
        assert eo <= 1e-4 and es <= 1e-4, (eo, es)
    else:
        eo, es = rel_err(got_o, ref_o), rel_err(got_S, ref_S)
        assert eo <= 2e-2 and es <= 2e-2, (eo, es)


KINDS = ["beta0", "recall", "nodecay", "strong", "zeros"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("kind", KINDS)
def test_decode_degenerate(kind, io):
    dev = device()
    inp = _case(kind, io, T=12)
    B, T, H, dk, dv = inp.dims
    ref_o, ref_S, ref_ring = kda_oracle.forward(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                                inp.conv_w, inp.S0, inp.ring0)
    st = kda.KDAState(B, H, dk, dv, io=torch.float32 if io == "f32" else torch.bfloat16,
                      device=dev)
    load_state(st, inp)
    o = run_decode(st, to_dev(inp, dev, step_major=True), T)
    torch.cuda.synchronize()
    got_o = f64(o).transpose(1, 0, 2, 3)
    _check(got_o, f64(st.S), ref_o, ref_S, io)
    np.testing.assert_array_equal(f64(st.ring), ref_ring)
    if kind == "zeros":
        assert np.all(got_o == 0.0)
    if kind == "recall":  # o_t = v^_t: the readout recalls the value just written
        _, _, vh, _ = kda_oracle.prologue(inp.q, inp.k, inp.v, inp.conv_w, inp.ring0)
        assert abs_err(got_o, vh) <= (1e-4 if io == "f32" else 2e-2 * np.abs(vh).max())


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 64])
@pytest.mark.parametrize("kind", KINDS)
def test_prefill_degenerate(kind, chunk, io):
    dev = device()
    inp = _case(kind, io, T=203)
    B, T, H, dk, dv = inp.dims
    ref_o, ref_S, ref_ring = kda_oracle.forward(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                                inp.conv_w, inp.S0, inp.ring0)
    tio = torch.float32 if io == "f32" else torch.bfloat16
    d = to_dev(inp, dev)
    st = kda.KDAState(B, H, dk, dv, io=tio, device=dev)
    load_state(st, inp)
    o = torch.empty(B, T, H, dv, dtype=tio, device=dev)
    st.prefill(T, d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], o, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(st.S).all()
    _check(f64(o), f64(st.S), ref_o, ref_S, io)
    np.testing.assert_array_equal(f64(st.ring), ref_ring)
    if kind == "zeros":
        assert np.all(f64(o) == 0.0)
