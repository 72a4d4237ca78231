"""kda_decode_step on the GPU against the fp64 oracle.

Tolerances (stated for the workloads): fp32 inputs, max |err| <= 1e-4 on o
and S; bf16 inputs with an fp32 state, max|err| / max|ref| <= 2e-2.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as kda
import workloads
from oracle import kda_oracle
from tests.gpu_util import (abs_err, device, f64, load_state, rel_err, run_decode, subset,
                            to_dev)

pytestmark = pytest.mark.gpu


def _oracle(inp):
    return kda_oracle.forward(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.conv_w, inp.S0,
                              inp.ring0)


@pytest.mark.parametrize("name,overrides", [
    ("tiny", {}),
    ("tiny", dict(dk=32, dv=64, H=3, B=2, T=20, s0_random=True, ring_random=True, seed=11)),
    ("tiny", dict(dk=128, dv=16, H=2, B=3, T=9, s0_random=True, ring_random=True, seed=12)),
    ("tiny", dict(dk=64, dv=128, H=1, B=2, T=7, s0_random=True, ring_random=True, seed=13)),
])
def test_decode_f32_sequence(name, overrides):
    dev = device()
    inp = workloads.make(name, **overrides)
    B, T, H, dk, dv = inp.dims
    ref_o, ref_S, ref_ring = _oracle(inp)
    st = kda.KDAState(B, H, dk, dv, io=torch.float32, device=dev)
    load_state(st, inp)
    o = run_decode(st, to_dev(inp, dev, step_major=True), T)
    torch.cuda.synchronize()
    eo = abs_err(f64(o).transpose(1, 0, 2, 3), ref_o)
    es = abs_err(f64(st.S), ref_S)
    print(f"{name} {overrides}: max|err| o={eo:.2e} S={es:.2e}")
    assert eo <= 1e-4 and es <= 1e-4
    np.testing.assert_array_equal(f64(st.ring), ref_ring)


def test_decode_k3_single_step():
    """One decode step at the K3 shape (96 heads, 128x128), fp32, random
    state and ring."""
    dev = device()
    inp = workloads.make("k3_decode1")
    B, T, H, dk, dv = inp.dims
    ref_o, ref_S, ref_ring = _oracle(inp)
    st = kda.KDAState(B, H, dk, dv, io=torch.float32, device=dev)
    load_state(st, inp)
    o = run_decode(st, to_dev(inp, dev, step_major=True), T)
    torch.cuda.synchronize()
    eo = abs_err(f64(o)[0], ref_o[:, 0])
    es = abs_err(f64(st.S), ref_S)
    print(f"k3_decode1: max|err| o={eo:.2e} S={es:.2e}")
    assert eo <= 1e-4 and es <= 1e-4
    np.testing.assert_array_equal(f64(st.ring), ref_ring)


def test_decode_batched_bf16_full_size():
    """64 sequences x 96 heads x 128x128, bf16 I/O, 256 consecutive steps, in
    the launch configuration the benchmark times; the oracle checks 9 sampled
    (sequence, head) pairs over all 256 steps, and the ring everywhere."""
    dev = device()
    inp = workloads.make("batched_decode")
    B, T, H, dk, dv = inp.dims
    d = to_dev(inp, dev, step_major=True)
    st = kda.KDAState(B, H, dk, dv, io=torch.bfloat16, device=dev)
    load_state(st, inp)
    o = run_decode(st, d, T)
    torch.cuda.synchronize()
    seqs, heads = [0, 17, 63], [0, 41, 95]
    sub = subset(inp, seqs, heads)
    ref_o, ref_S, _ = _oracle(sub)
    got_o = f64(o[:, seqs][:, :, heads]).transpose(1, 0, 2, 3)
    got_S = f64(st.S[seqs][:, heads])
    eo, es = rel_err(got_o, ref_o), rel_err(got_S, ref_S)
    print(f"batched_decode: rel err o={eo:.2e} S={es:.2e}")
    assert eo <= 2e-2 and es <= 2e-2
    # the ring holds exactly the last three raw tokens of every channel
    Hd = H * dk
    ring = st.ring.cpu()
    for p, x in enumerate((inp.q, inp.k, inp.v)):
        want = x[:, T - 3:].reshape(B, 3, -1)
        off = p * Hd
        assert torch.equal(ring[:, :, off:off + want.shape[-1]], want)


def test_decode_worked_example_flags():
    """The delta-rule worked example (key [1,3] written with value [2,4], then
    with [0,1]) embedded in 16-wide heads, conv skipped, L2 on, g = 0,
    beta = 1, q = k: the second read returns exactly the new value."""
    dev = device()
    d = 16
    k = torch.zeros(1, 1, d)
    k[0, 0, :2] = torch.tensor([1.0, 3.0])
    vs = [torch.zeros(1, 1, d), torch.zeros(1, 1, d)]
    vs[0][0, 0, :2] = torch.tensor([2.0, 4.0])
    vs[1][0, 0, :2] = torch.tensor([0.0, 1.0])
    st = kda.KDAState(1, 1, d, d, io=torch.float32, device=dev)
    st.reset()
    o = torch.empty(1, 1, d, device=dev)
    g = torch.zeros(1, 1, d, device=dev)
    beta = torch.ones(1, 1, device=dev)
    outs = []
    for v in vs:
        st.decode_step(k.to(dev), k.to(dev), v.to(dev), g, beta, None, o,
                       flags=kda.KDA_F_SKIP_CONV)
        outs.append(o.cpu().clone())
    np.testing.assert_allclose(outs[0][0, 0, :2].numpy(), [2.0, 4.0], atol=1e-5)
    np.testing.assert_allclose(outs[1][0, 0, :2].numpy(), [0.0, 1.0], atol=1e-5)
    S = st.S.cpu()[0, 0]
    np.testing.assert_allclose(S[:2, :2].numpy(), [[0, 10 ** -0.5], [0, 3 * 10 ** -0.5]],
                               atol=1e-6)


def test_decode_minus_inf_clears_and_reset_subset():
    dev = device()
    inp = workloads.make("tiny", B=3, T=6, H=2, dk=32, dv=32, s0_random=True,
                         ring_random=True, seed=21)
    B, T, H, dk, dv = inp.dims
    inp.g[:, 4] = -float("inf")            # token 4 clears every sequence's memory
    ref_o, ref_S, ref_ring = _oracle(inp)
    st = kda.KDAState(B, H, dk, dv, io=torch.float32, device=dev)
    load_state(st, inp)
    o = run_decode(st, to_dev(inp, dev, step_major=True), T)
    torch.cuda.synchronize()
    assert np.isfinite(f64(o)).all()
    assert abs_err(f64(o).transpose(1, 0, 2, 3), ref_o) <= 1e-4
    assert abs_err(f64(st.S), ref_S) <= 1e-4
    S_before = st.S.clone()
    st.reset([1])
    torch.cuda.synchronize()
    assert torch.count_nonzero(st.S[1]) == 0 and torch.count_nonzero(st.ring[1]) == 0
    assert torch.equal(st.S[0], S_before[0]) and torch.equal(st.S[2], S_before[2])


def test_decode_in_captured_graph_matches_eager():
    """Decode steps captured in a HIP graph: each replay (with eager work and
    synchronizations between replays) advances the state exactly as the same
    launches issued eagerly do."""
    dev = device()
    inp = workloads.make("tiny", T=4, B=3, H=4, dk=128, dv=64, io="bf16", s0_random=True,
                         ring_random=True, seed=81)
    B, T, H, dk, dv = inp.dims
    d = to_dev(inp, dev, step_major=True)
    eager = kda.KDAState(B, H, dk, dv, io=torch.bfloat16, device=dev)
    cap = kda.KDAState(B, H, dk, dv, io=torch.bfloat16, device=dev)
    for st in (eager, cap):
        load_state(st, inp)
    oe = torch.empty(T, B, H, dv, dtype=torch.bfloat16, device=dev)
    oc = torch.empty_like(oe)

    def steps(st, o):
        for t in range(T):
            st.decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t],
                           d["conv_w"], o[t])

    steps(cap, oc)                  # warm-up, as eager
    torch.cuda.synchronize()
    load_state(cap, inp)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps(cap, oc)
    load_state(cap, inp)            # capture does not run the launches
    torch.cuda.synchronize()
    for rep in range(4):
        steps(eager, oe)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(oc, oe), f"replay {rep}: o differs"
        assert torch.equal(cap.S, eager.S) and torch.equal(cap.ring, eager.ring), \
            f"replay {rep}: state differs"


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(a, b) for a in (16, 32, 64, 128) for b in (16, 32, 64, 128)])
def test_decode_every_shape(dk, dv, io):
    """Every supported (d_k, d_v, I/O type): 6 decode steps for 2 sequences x 2
    heads from a random state and ring, against the oracle."""
    dev = device()
    inp = workloads.make("tiny", T=6, B=2, H=2, dk=dk, dv=dv, io=io, s0_random=True,
                         ring_random=True, seed=2000 + dk + 7 * dv + (1 if io == "bf16" else 0))
    B, T, H, dk, dv = inp.dims
    ref_o, ref_S, ref_ring = _oracle(inp)
    st = kda.KDAState(B, H, dk, dv, io=torch.float32 if io == "f32" else torch.bfloat16,
                      device=dev)
    load_state(st, inp)
    o = run_decode(st, to_dev(inp, dev, step_major=True), T)
    torch.cuda.synchronize()
    got = f64(o).transpose(1, 0, 2, 3)
    if io == "f32":
        eo, es = abs_err(got, ref_o), abs_err(f64(st.S), ref_S)
        assert eo <= 1e-4 and es <= 1e-4, (eo, es)
    else:
        eo, es = rel_err(got, ref_o), rel_err(f64(st.S), ref_S)
        assert eo <= 2e-2 and es <= 2e-2, (eo, es)
    np.testing.assert_array_equal(f64(st.ring), ref_ring)
