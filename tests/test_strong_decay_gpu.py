"""Strong and infinite decay through kda_chunk_prefill (and decode), against the
fp64 oracle: the prefill accepts any g <= 0 that is not NaN, the way a decode
step does. A decay of 1 means alpha = e^{-1}; -10 and -40 per token (and
-inf) all but erase the state ("为什么 Kimi K3 敢把 KV Cache 扔掉？…", section 6:
alpha -> 0 clears the memory).

Kinds (the workload's mild decays g = logsigmoid(N(0, 1)) elsewhere):
  g10, g40   every token and channel decays by 10 / 40 (every 16-token block
             decays past 64: the diagonal tiles are formed term by term);
  g5, g6     -5 and -6 per token: blocks decay by 75 and 90 over their last 15
             tokens, just past the factored form's limit (16 x -6 = -96: where a
             factor e^{+90} of an unbounded in-block reference would overflow fp32);
  mixed      bands of -40 on half the channels, a 16-token run of -6, one
             token at -inf on one channel, one token at -1e30 on all, mild
             chunks in between (factored and explicit tiles in one call, and
             chunks that are mild after a strong one);
  edge       -4.2 per token: blocks decay by 63, just inside the factored
             form's limit.

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

RAW, SG = kda.KDA_F_RAW_GATES, kda.KDA_F_SCALAR_G


def _strong(g, kind):
    """g with the kind's decays written in (last axis: key channels, or none
    for a scalar decay)."""
    g = g.clone()
    per_channel = g.dim() == 4
    if kind == "g10":
        g.fill_(-10.0)
    elif kind == "g40":
        g.fill_(-40.0)
    elif kind == "g5":
        g.fill_(-5.0)
    elif kind == "g6":
        g.fill_(-6.0)
    elif kind == "edge":
        g.fill_(-4.2)
    elif kind == "mixed":
        T = g.shape[1]
        if per_channel:
            half = g.shape[-1] // 2
            g[:, 20:37, :, :half] = -40.0
            g[:, 70, :, 0] = float("-inf")
        else:
            g[:, 20:37] = -40.0
            g[:, 70, 0] = float("-inf")
        g[:, 100] = -1e30
        g[:, 130:146] = -6.0
        if T > 250:
            g[:, 250:260] = -25.0
    return g


def _oracle(inp):
    g = inp.g
    if g.dim() == 3:  # one decay per (token, head): repeat it over the key channels
        g = g.unsqueeze(-1).expand(*g.shape, inp.q.shape[-1]).contiguous()
    return kda_oracle.forward(inp.q, inp.k, inp.v, g, inp.beta, inp.conv_w, inp.S0, inp.ring0)


def _check(got_o, got_S, ref_o, ref_S, io):
    assert np.isfinite(got_o).all() and np.isfinite(got_S).all()
    if io == torch.float32:
        eo, es = abs_err(got_o, ref_o), abs_err(got_S, ref_S)
        assert eo <= 1e-4 and es <= 1e-4, (eo, es)
    else:
        eo, es = rel_err(got_o, ref_o), rel_err(got_S, ref_S)
        assert eo <= 2e-2 and es <= 2e-2, (eo, es)
    return eo, es


def _prefill(inp, chunk, io, flags=0):
    dev = device()
    B, T, H, dk, dv = inp.dims
    d = to_dev(inp, dev)
    st = kda.KDAState(B, H, dk, dv, io=io, device=dev)
    load_state(st, inp)
    o = torch.empty(B, T, H, dv, dtype=io, device=dev)
    st.prefill(T, d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], o, chunk=chunk,
               flags=flags)
    torch.cuda.synchronize()
    return st, o


KINDS = ["g10", "g40", "g5", "mixed", "edge", "g6"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("kind", KINDS)
def test_prefill_strong_decay(kind, chunk, io):
    inp = workloads.make("tiny", T=203, B=2, H=2, dk=64, dv=64, io=io, s0_random=True,
                         ring_random=True, seed=900 + KINDS.index(kind))
    inp.g = _strong(inp.g, kind)
    tio = torch.float32 if io == "f32" else torch.bfloat16
    ref_o, ref_S, ref_ring = _oracle(inp)
    st, o = _prefill(inp, chunk, tio)
    eo, es = _check(f64(o), f64(st.S), ref_o, ref_S, tio)
    print(f"prefill {kind} C={chunk} {io}: err o={eo:.2e} S={es:.2e}")
    np.testing.assert_array_equal(f64(st.ring), ref_ring)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["g40", "mixed", "edge"])
def test_prefill_strong_decay_d128(kind, io):
    """The 128 x 128 shape of the workloads (the bf16 kernel instantiation
    that the benchmark times), 300 tokens: five chunks of 64, ragged."""
    inp = workloads.make("tiny", T=300, B=1, H=2, dk=128, dv=128, io=io, s0_random=True,
                         ring_random=True, seed=950 + len(kind))
    inp.g = _strong(inp.g, kind)
    tio = torch.float32 if io == "f32" else torch.bfloat16
    ref_o, ref_S, _ = _oracle(inp)
    st, o = _prefill(inp, 64, tio)
    eo, es = _check(f64(o), f64(st.S), ref_o, ref_S, tio)
    print(f"prefill d128 {kind} {io}: err o={eo:.2e} S={es:.2e}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["g40", "mixed"])
def test_prefill_strong_scalar_decay(kind, io):
    inp = workloads.make("tiny", T=203, B=2, H=2, dk=64, dv=32, io=io, scalar_g=True,
                         s0_random=True, seed=970 + len(kind))
    inp.g = _strong(inp.g, kind)
    tio = torch.float32 if io == "f32" else torch.bfloat16
    ref_o, ref_S, _ = _oracle(inp)
    st, o = _prefill(inp, 64, tio, flags=SG)
    _check(f64(o), f64(st.S), ref_o, ref_S, tio)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_strong_raw_gates(io):
    """Raw decay projections a far below zero (g = log sigmoid(a) ~ a) and
    a = -inf (g = -inf) in the middle of mild ones."""
    inp = workloads.make("tiny", T=203, B=2, H=2, dk=64, dv=64, io=io, raw_gates=True,
                         s0_random=True, ring_random=True, seed=990)
    inp.g[:, 40:60] = -45.0
    inp.g[:, 120, :, 3] = float("-inf")
    inp.g[:, 150:170, :, ::2] = -7.0
    g, beta = kda_oracle.gates_from_raw(inp.g, inp.beta)
    tio = torch.float32 if io == "f32" else torch.bfloat16
    ref_o, ref_S, _ = kda_oracle.forward(inp.q, inp.k, inp.v, g, beta, inp.conv_w, inp.S0,
                                         inp.ring0)
    st, o = _prefill(inp, 64, tio, flags=RAW)
    _check(f64(o), f64(st.S), ref_o, ref_S, tio)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["g40", "mixed"])
def test_decode_strong_decay(kind, io):
    inp = workloads.make("tiny", T=140, B=2, H=2, dk=64, dv=64, io=io, s0_random=True,
                         ring_random=True, seed=930 + len(kind))
    inp.g = _strong(inp.g, kind)
    tio = torch.float32 if io == "f32" else torch.bfloat16
    ref_o, ref_S, _ = _oracle(inp)
    dev = device()
    B, T, H, dk, dv = inp.dims
    st = kda.KDAState(B, H, dk, dv, io=tio, device=dev)
    load_state(st, inp)
    o = run_decode(st, to_dev(inp, dev, step_major=True), T)
    torch.cuda.synchronize()
    _check(f64(o).transpose(1, 0, 2, 3), f64(st.S), ref_o, ref_S, tio)
