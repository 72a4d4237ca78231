"""The output gate (gated RMSNorm of each head's readout) on the GPU against
the fp64 oracle: the standalone kda_gated_rmsnorm on any [B,T,H,d_v] tensor,
and kda_decode_step_gated with the gate fused into the readout.

Tolerances: fp32 max |err| <= 1e-4; bf16 max|err|/max|ref| <= 2e-2.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as kda
import workloads
from oracle import kda_oracle
from tests.gpu_util import abs_err, device, f64, load_state, rel_err, subset, to_dev

pytestmark = pytest.mark.gpu

TORCH_IO = {"f32": torch.float32, "bf16": torch.bfloat16}


def _check(got, ref, io):
    if io == "f32":
        err = abs_err(got, ref)
        assert err <= 1e-4, err
    else:
        err = rel_err(got, ref)
        assert err <= 2e-2, err
    return err


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_gated_rmsnorm_every_width(dv, io):
    """222 rows (2 x 37 tokens x 3 heads, not a multiple of a block's rows),
    row scales from 1e-2 to 1e2, against the oracle on the same inputs."""
    dev = device()
    B, T, H = 2, 37, 3
    gen = torch.Generator().manual_seed(900 + dv)
    scale = torch.logspace(-2, 2, B * T * H).reshape(B, T, H, 1)
    x = (torch.randn(B, T, H, dv, generator=gen) * scale).to(TORCH_IO[io])
    z, w, eps = workloads.draw_output_gate(B, T, H, dv, io, seed=dv)
    ref = kda_oracle.gated_rmsnorm(x, z, w, eps)
    dims = kda.make_dims(B, H, 16, dv, kda.KDA_F32 if io == "f32" else kda.KDA_BF16)
    xd, zd, wd = x.to(dev), z.to(dev), w.to(dev)
    out = torch.empty_like(xd)
    kda.kda_gated_rmsnorm(dims, T, xd, zd, wd, eps, out)
    torch.cuda.synchronize()
    err = _check(f64(out), ref, io)
    print(f"gated rmsnorm dv={dv} {io}: err {err:.2e}")
    # in place gives the same bits
    kda.kda_gated_rmsnorm(dims, T, xd, zd, wd, eps, xd)
    torch.cuda.synchronize()
    assert torch.equal(xd, out)
    # T = 0 does nothing
    kda.kda_gated_rmsnorm(dims, 0, xd, zd, wd, eps, xd)


def test_gated_rmsnorm_rejects_bad_arguments():
    dev = device()
    dims = kda.make_dims(1, 2, 16, 16, kda.KDA_F32)
    x = torch.zeros(1, 4, 2, 16, device=dev)
    z, w = torch.zeros_like(x), torch.ones(16, device=dev)
    for eps in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(kda.KDAError):
            kda.kda_gated_rmsnorm(dims, 4, x, z, w, eps, x)
    with pytest.raises(kda.KDAError):
        kda.kda_gated_rmsnorm(dims, 4, x, z, w, 1e-5, z)          # out overlaps the gate
    flat = torch.zeros(2 * 4 * 2 * 16, device=dev)
    with pytest.raises(kda.KDAError):                             # out partly overlaps x
        kda.kda_gated_rmsnorm(dims, 4, flat[:128], z, w, 1e-5, flat[64:192])


def _gated_decode(inp, z, w, eps, dev, io):
    B, T, H, dk, dv = inp.dims
    st = kda.KDAState(B, H, dk, dv, io=TORCH_IO[io], device=dev)
    load_state(st, inp)
    d = to_dev(inp, dev, step_major=True)
    zd = z.transpose(0, 1).contiguous().to(dev)
    wd = w.to(dev)
    o = torch.empty(T, B, H, dv, dtype=TORCH_IO[io], device=dev)
    for t in range(T):
        st.decode_step_gated(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t],
                             d["conv_w"], zd[t], wd, eps, o[t])
    torch.cuda.synchronize()
    return st, o


@pytest.mark.parametrize("dk,dv,io", [(16, 16, "f32"), (32, 64, "f32"), (128, 32, "f32"),
                                      (64, 128, "bf16"), (128, 128, "bf16"), (16, 64, "bf16")])
def test_decode_gated(dk, dv, io):
    """Fused gate against the oracle's readout passed through the oracle's
    gate; the state and ring are those of the plain step."""
    dev = device()
    inp = workloads.make("tiny", T=8, B=2, H=3, dk=dk, dv=dv, io=io, s0_random=True,
                         ring_random=True, seed=950 + dk + dv)
    B, T, H, dk, dv = inp.dims
    z, w, eps = workloads.draw_output_gate(B, T, H, dv, io, seed=950)
    ref_o, ref_S, ref_ring = kda_oracle.forward(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                                inp.conv_w, inp.S0, inp.ring0)
    ref_y = kda_oracle.gated_rmsnorm(ref_o, z, w, eps)
    st, o = _gated_decode(inp, z, w, eps, dev, io)
    ey = _check(f64(o).transpose(1, 0, 2, 3), ref_y, io)
    es = _check(f64(st.S), ref_S, io)
    print(f"decode gated dk={dk} dv={dv} {io}: err y={ey:.2e} S={es:.2e}")
    np.testing.assert_array_equal(f64(st.ring), ref_ring)


def test_decode_gated_batched_full_size():
    """64 sequences x 96 heads x 128x128, bf16, 256 steps with the fused gate
    (the launch the benchmark times); 4 sampled (sequence, head) pairs."""
    dev = device()
    inp = workloads.make("batched_decode")
    B, T, H, dk, dv = inp.dims
    z, w, eps = workloads.draw_output_gate(B, T, H, dv, "bf16", seed=2)
    st, o = _gated_decode(inp, z, w, eps, dev, "bf16")
    seqs, heads = [5, 60], [7, 88]
    sub = subset(inp, seqs, heads)
    ref_o, ref_S, _ = kda_oracle.forward(sub.q, sub.k, sub.v, sub.g, sub.beta, sub.conv_w,
                                         sub.S0, sub.ring0)
    ref_y = kda_oracle.gated_rmsnorm(ref_o, z[seqs][:, :, heads], w, eps)
    got = f64(o[:, seqs][:, :, heads]).transpose(1, 0, 2, 3)
    ey = _check(got, ref_y, "bf16")
    es = _check(f64(st.S[seqs][:, heads]), ref_S, "bf16")
    print(f"batched decode gated: rel err y={ey:.2e} S={es:.2e}")


def test_prefill_4k_then_gate_in_place():
    """The 4096-token prefill (96 heads, chunk 64, bf16) followed by the gate in
    place on its output; the oracle checks 6 sampled heads over all tokens."""
    dev = device()
    inp = workloads.make("prefill_4k")
    B, T, H, dk, dv = inp.dims
    z, w, eps = workloads.draw_output_gate(B, T, H, dv, "bf16", seed=3)
    d = to_dev(inp, dev)
    st = kda.KDAState(B, H, dk, dv, io=torch.bfloat16, device=dev)
    st.reset()
    o = torch.empty(B, T, H, dv, dtype=torch.bfloat16, device=dev)
    st.prefill(T, d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], o, chunk=64)
    st.gated_rmsnorm(T, o, z.to(dev), w.to(dev), eps, o)
    torch.cuda.synchronize()
    heads = [1, 20, 39, 58, 77, 94]
    sub = subset(inp, [0], heads)
    ref_o, _, _ = kda_oracle.forward(sub.q, sub.k, sub.v, sub.g, sub.beta, sub.conv_w, sub.S0,
                                     sub.ring0)
    ref_y = kda_oracle.gated_rmsnorm(ref_o, z[:, :, heads], w, eps)
    ey = _check(f64(o[:, :, heads]), ref_y, "bf16")
    print(f"prefill_4k + gate: rel err {ey:.2e}")


def test_gated_paths_in_captured_graph_match_eager():
    """Gated decode steps from raw gate projections, then the standalone gate
    kernel on their outputs, captured in one HIP graph: every replay (with
    eager work and synchronizations between replays) equals the same launches
    issued eagerly, bit for bit."""
    dev = device()
    inp = workloads.make("tiny", T=3, B=2, H=4, dk=64, dv=128, io="bf16", s0_random=True,
                         ring_random=True, raw_gates=True, seed=960)
    B, T, H, dk, dv = inp.dims
    z, w, eps = workloads.draw_output_gate(B, T, H, dv, "bf16", seed=960)
    d = to_dev(inp, dev, step_major=True)
    zd, wd = z.transpose(0, 1).contiguous().to(dev), w.to(dev)
    eager = kda.KDAState(B, H, dk, dv, io=torch.bfloat16, device=dev)
    cap = kda.KDAState(B, H, dk, dv, io=torch.bfloat16, device=dev)
    for st in (eager, cap):
        load_state(st, inp)
    oe = torch.empty(T, B, H, dv, dtype=torch.bfloat16, device=dev)
    oc, ye, yc = torch.empty_like(oe), torch.empty_like(oe), torch.empty_like(oe)
    raw = kda.KDA_F_RAW_GATES

    def run(st, o, y):
        for t in range(T):
            st.decode_step_gated(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t],
                                 d["conv_w"], zd[t], wd, eps, o[t], flags=raw)
        # the plain gate kernel over all T steps' outputs ([T*B] rows of H heads)
        kda.kda_gated_rmsnorm(kda.make_dims(T * B, H, dk, dv), 1, o, zd, wd, eps, y)

    run(cap, oc, yc)
    torch.cuda.synchronize()
    load_state(cap, inp)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(cap, oc, yc)
    load_state(cap, inp)
    torch.cuda.synchronize()
    for rep in range(3):
        run(eager, oe, ye)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(oc, oe) and torch.equal(yc, ye), f"replay {rep}: outputs differ"
        assert torch.equal(cap.S, eager.S) and torch.equal(cap.ring, eager.ring), \
            f"replay {rep}: state differs"
