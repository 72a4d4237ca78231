"""KDA_F_SCALAR_G (one decay per token and head, the scalar-alpha Gated
DeltaNet form) on the GPU.

Two checks per case: against the fp64 oracle run on g repeated over the key
channels (the oracle's scalar-decay case is pinned to the Gated DeltaNet
update by the P-b' pin), with the usual tolerances (fp32: max |err| <= 1e-4;
bf16: max|err|/max|ref| <= 2e-2); and bitwise against the per-channel call of
the library on that repeated g, since both calls feed the same decay values
to the same arithmetic.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as kda
import workloads
from oracle import kda_oracle
from tests.gpu_util import (abs_err, device, f64, load_state, per_channel_g, rel_err,
                            run_decode, subset, to_dev)

pytestmark = pytest.mark.gpu

SG = kda.KDA_F_SCALAR_G


def _oracle(inp, flags=0):
    full = per_channel_g(inp)
    return kda_oracle.forward(full.q, full.k, full.v, full.g, full.beta, full.conv_w, full.S0,
                              full.ring0, flags=flags)


def _torch_io(inp):
    return torch.float32 if inp.meta["io"] == "f32" else torch.bfloat16


def _check(got_o, got_S, ref_o, ref_S, io):
    if io == torch.float32:
        eo, es = abs_err(got_o, ref_o), abs_err(got_S, ref_S)
        assert eo <= 1e-4 and es <= 1e-4, (eo, es)
    else:
        eo, es = rel_err(got_o, ref_o), rel_err(got_S, ref_S)
        assert eo <= 2e-2 and es <= 2e-2, (eo, es)
    return eo, es


def _decode(inp, dev, flags):
    B, T, H, dk, dv = inp.dims
    st = kda.KDAState(B, H, dk, dv, io=_torch_io(inp), device=dev)
    load_state(st, inp)
    o = run_decode(st, to_dev(inp, dev, step_major=True), T, flags=flags)
    torch.cuda.synchronize()
    return st, o


@pytest.mark.parametrize("overrides", [
    dict(T=12, B=2, H=3, dk=32, dv=64, io="f32", seed=301),
    dict(T=7, B=1, H=2, dk=128, dv=128, io="f32", g_mu=-1.0, seed=302),
    dict(T=9, B=3, H=2, dk=16, dv=32, io="bf16", seed=303),
    dict(T=6, B=2, H=2, dk=128, dv=16, io="bf16", seed=304),
])
def test_decode_scalar_g(overrides):
    dev = device()
    inp = workloads.make("tiny", s0_random=True, ring_random=True, scalar_g=True, **overrides)
    io = _torch_io(inp)
    ref_o, ref_S, ref_ring = _oracle(inp)
    st, o = _decode(inp, dev, SG)
    eo, es = _check(f64(o).transpose(1, 0, 2, 3), f64(st.S), ref_o, ref_S, io)
    print(f"decode scalar g {overrides}: err o={eo:.2e} S={es:.2e}")
    np.testing.assert_array_equal(f64(st.ring), ref_ring)
    st2, o2 = _decode(per_channel_g(inp), dev, 0)
    assert torch.equal(o, o2) and torch.equal(st.S, st2.S)


def test_decode_scalar_g_batched_full_size():
    """64 sequences x 96 heads x 128x128, bf16, 256 steps with one decay per
    (token, head): the launch configuration the benchmark times; the oracle
    checks 6 sampled (sequence, head) pairs over all steps."""
    dev = device()
    inp = workloads.make("batched_decode_gdn")
    st, o = _decode(inp, dev, SG)
    seqs, heads = [0, 40], [3, 50, 95]
    ref_o, ref_S, _ = _oracle(subset(inp, seqs, heads))
    got_o = f64(o[:, seqs][:, :, heads]).transpose(1, 0, 2, 3)
    eo, es = _check(got_o, f64(st.S[seqs][:, heads]), ref_o, ref_S, torch.bfloat16)
    print(f"batched_decode_gdn: rel err o={eo:.2e} S={es:.2e}")


def _prefill(inp, dev, chunk, flags):
    B, T, H, dk, dv = inp.dims
    io = _torch_io(inp)
    d = to_dev(inp, dev)
    st = kda.KDAState(B, H, dk, dv, io=io, device=dev)
    load_state(st, inp)
    o = torch.empty(B, T, H, dv, dtype=io, device=dev)
    st.prefill(T, d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], o, chunk=chunk,
               flags=flags)
    torch.cuda.synchronize()
    return st, o


@pytest.mark.parametrize("chunk,overrides", [
    (64, dict(T=200, B=2, H=2, dk=128, dv=128, io="bf16", seed=311)),          # row kernel
    (32, dict(T=77, B=1, H=3, dk=64, dv=32, io="bf16", g_mu=2.0, seed=312)),   # row kernel
    (16, dict(T=40, B=2, H=2, dk=32, dv=16, io="bf16", seed=313)),             # general, bf16
    (64, dict(T=130, B=1, H=2, dk=16, dv=64, io="f32", seed=314)),             # general, fp32
    (32, dict(T=45, B=2, H=1, dk=128, dv=32, io="f32", seed=315)),
    (16, dict(T=3, B=1, H=2, dk=64, dv=64, io="f32", seed=316)),               # T < ring
])
def test_prefill_scalar_g(chunk, overrides):
    dev = device()
    inp = workloads.make("tiny", s0_random=True, ring_random=True, scalar_g=True, **overrides)
    io = _torch_io(inp)
    ref_o, ref_S, ref_ring = _oracle(inp)
    st, o = _prefill(inp, dev, chunk, SG)
    eo, es = _check(f64(o), f64(st.S), ref_o, ref_S, io)
    print(f"prefill scalar g C={chunk} {overrides}: err o={eo:.2e} S={es:.2e}")
    np.testing.assert_array_equal(f64(st.ring), ref_ring)
    st2, o2 = _prefill(per_channel_g(inp), dev, chunk, 0)
    assert torch.equal(o, o2) and torch.equal(st.S, st2.S)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_scalar_g_skip_conv(io):
    dev = device()
    inp = workloads.make("tiny", T=90, B=1, H=2, dk=64, dv=128, io=io, s0_random=True,
                         ring_random=True, scalar_g=True, seed=320)
    flags = SG | kda.KDA_F_SKIP_CONV
    ref_o, ref_S, _ = _oracle(inp, flags=kda.KDA_F_SKIP_CONV)
    st, o = _prefill(inp, dev, 64, flags)
    _check(f64(o), f64(st.S), ref_o, ref_S, _torch_io(inp))
    np.testing.assert_array_equal(f64(st.ring), f64(inp.ring0))


def test_prefill_scalar_g_4k_full_size():
    """T=4096, 96 heads of 128x128, chunk 64, bf16, one decay per (token,
    head): the launch the benchmark times; the oracle checks 6 sampled heads
    over all tokens and the final state."""
    dev = device()
    inp = workloads.make("prefill_4k_gdn")
    st, o = _prefill(inp, dev, 64, SG)
    heads = [0, 19, 38, 57, 76, 95]
    ref_o, ref_S, _ = _oracle(subset(inp, [0], heads))
    eo, es = _check(f64(o[:, :, heads]), f64(st.S[:, heads]), ref_o, ref_S, torch.bfloat16)
    print(f"prefill_4k_gdn: rel err o={eo:.2e} S={es:.2e}")
    assert np.isfinite(f64(o)).all()
