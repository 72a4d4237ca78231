"""kda_chunk_prefill (and kda_conv_prologue) on the GPU against the fp64
oracle: fp32 inputs max |err| <= 1e-4; bf16 inputs max|err|/max|ref| <= 2e-2."""
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


def _prefill(inp, dev, chunk, io, workspace=None, flags=0):
    B, T, H, dk, dv = inp.dims
    d = to_dev(inp, dev)
    st = kda.KDAState(B, H, dk, dv, io=io, device=dev)
    load_state(st, inp)
    o = torch.empty(B, T, H, dv, dtype=io, device=dev)
    st.prefill(T, d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], o, chunk=chunk,
               workspace=workspace, flags=flags)
    torch.cuda.synchronize()
    return st, o


CASES_F32 = [
    ("tiny", 64, {}),
    ("tiny", 16, {}),
    ("tiny", 32, {}),
    ("tiny", 16, dict(T=50, s0_random=True, ring_random=True, seed=31)),      # ragged tail
    ("tiny", 64, dict(T=2, s0_random=True, ring_random=True, seed=32)),       # T < ring
    ("tiny", 32, dict(T=1, s0_random=True, ring_random=True, seed=33)),
    ("tiny", 64, dict(T=130, B=2, H=3, dk=32, dv=64, s0_random=True, ring_random=True,
                      seed=34)),
    ("tiny", 32, dict(T=45, B=1, H=2, dk=128, dv=32, s0_random=True, seed=35)),
    ("tiny", 16, dict(T=40, B=2, H=1, dk=64, dv=16, ring_random=True, seed=36)),
]


@pytest.mark.parametrize("name,chunk,overrides", CASES_F32)
def test_prefill_f32(name, chunk, overrides):
    dev = device()
    inp = workloads.make(name, **overrides)
    ref_o, ref_S, ref_ring = _oracle(inp)
    st, o = _prefill(inp, dev, chunk, torch.float32)
    eo, es = abs_err(f64(o), ref_o), abs_err(f64(st.S), ref_S)
    print(f"prefill f32 C={chunk} {overrides}: max|err| o={eo:.2e} S={es:.2e}")
    assert eo <= 1e-4 and es <= 1e-4
    np.testing.assert_array_equal(f64(st.ring), ref_ring)


@pytest.mark.parametrize("chunk,overrides", [
    (64, dict(T=200, B=2, H=3, dk=128, dv=128, io="bf16", s0_random=True, ring_random=True,
              seed=41)),
    (32, dict(T=77, B=1, H=4, dk=64, dv=64, io="bf16", seed=42)),
    (16, dict(T=40, B=2, H=2, dk=16, dv=32, io="bf16", ring_random=True, seed=43)),
    (64, dict(T=300, B=1, H=2, dk=128, dv=128, io="bf16", g_mu=2.0, seed=44)),
])
def test_prefill_bf16_small(chunk, overrides):
    dev = device()
    inp = workloads.make("tiny", **overrides)
    ref_o, ref_S, ref_ring = _oracle(inp)
    st, o = _prefill(inp, dev, chunk, torch.bfloat16)
    eo, es = rel_err(f64(o), ref_o), rel_err(f64(st.S), ref_S)
    print(f"prefill bf16 C={chunk} {overrides}: rel err o={eo:.2e} S={es:.2e}")
    assert eo <= 2e-2 and es <= 2e-2
    np.testing.assert_array_equal(f64(st.ring), ref_ring)


@pytest.mark.parametrize("chunk,overrides", [
    (64, dict(T=150, B=2, H=2, dk=128, dv=32, io="bf16", s0_random=True, seed=45)),
    (32, dict(T=70, B=1, H=3, dk=32, dv=128, io="bf16", s0_random=True, ring_random=True,
              seed=46)),
    (64, dict(T=3, B=2, H=2, dk=64, dv=128, io="bf16", s0_random=True, ring_random=True,
              seed=47)),
    (32, dict(T=1, B=1, H=2, dk=128, dv=64, io="bf16", s0_random=True, ring_random=True,
              seed=48)),
    (64, dict(T=129, B=1, H=2, dk=32, dv=32, io="bf16", ring_random=True, seed=49)),
])
def test_prefill_bf16_row_layout_shapes(chunk, overrides):
    """bf16 shapes of the token-row preparation kernel: d_k != d_v, chunk 32
    and 64, ragged tails, T below the conv history (history from the ring)."""
    test_prefill_bf16_small(chunk, overrides)


@pytest.mark.parametrize("flags", [kda.KDA_F_SKIP_CONV, kda.KDA_F_SKIP_CONV | kda.KDA_F_SKIP_L2])
def test_prefill_bf16_flags(flags):
    """bf16 chunk 64, 128x128 with the conv (and the L2 step) skipped; for
    KDA_F_SKIP_L2 the inputs are unit-norm q, k rounded to bf16."""
    dev = device()
    inp = workloads.make("tiny", T=90, B=1, H=2, dk=128, dv=128, io="bf16", s0_random=True,
                         ring_random=True, seed=52)
    if flags & kda.KDA_F_SKIP_L2:
        for name in ("q", "k"):
            x = getattr(inp, name).double()
            x = x / x.pow(2).sum(-1, keepdim=True).sqrt()
            setattr(inp, name, x.to(getattr(inp, name).dtype))
    ref_o, ref_S, _ = kda_oracle.forward(inp.q, inp.k, inp.v, inp.g, inp.beta, None, inp.S0,
                                         inp.ring0, flags=flags)
    st, o = _prefill(inp, dev, 64, torch.bfloat16, flags=flags)
    eo, es = rel_err(f64(o), ref_o), rel_err(f64(st.S), ref_S)
    print(f"prefill bf16 flags={flags}: rel err o={eo:.2e} S={es:.2e}")
    assert eo <= 2e-2 and es <= 2e-2
    np.testing.assert_array_equal(f64(st.ring), f64(inp.ring0))


def test_prefill_4k_bf16_full_size():
    """T=4096, 96 heads of 128x128, chunk 64, bf16 I/O, slow decay: the full
    launch the benchmark times; the oracle checks 8 sampled heads over all
    4096 tokens and the final state."""
    dev = device()
    inp = workloads.make("prefill_4k")
    st, o = _prefill(inp, dev, 64, torch.bfloat16)
    heads = [0, 13, 27, 40, 55, 68, 81, 95]
    sub = subset(inp, [0], heads)
    ref_o, ref_S, ref_ring = _oracle(sub)
    eo = rel_err(f64(o[:, :, heads]), ref_o)
    es = rel_err(f64(st.S[:, heads]), ref_S)
    print(f"prefill_4k: rel err o={eo:.2e} S={es:.2e}")
    assert eo <= 2e-2 and es <= 2e-2
    assert np.isfinite(f64(o)).all() and np.isfinite(f64(st.S)).all()


def test_prefill_segmented_workspace_is_identical():
    dev = device()
    inp = workloads.make("tiny", T=300, B=2, H=2, dk=64, dv=64, io="bf16", seed=51)
    B, T, H, dk, dv = inp.dims
    st1, o1 = _prefill(inp, dev, 32, torch.bfloat16)
    per = kda.kda_prefill_workspace_bytes(st1.dims, 32, 32)       # one chunk
    ws = torch.empty(3 * per + 8, dtype=torch.uint8, device=dev)  # 3 chunks per segment
    st2, o2 = _prefill(inp, dev, 32, torch.bfloat16, workspace=ws)
    assert torch.equal(o1, o2) and torch.equal(st1.S, st2.S) and torch.equal(st1.ring, st2.ring)


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_split_calls_and_decode_handoff(io):
    """prefill(T1) + prefill(T2) + decode steps == the oracle on all tokens."""
    dev = device()
    inp = workloads.make("tiny", T=100, B=2, H=2, dk=32, dv=32, s0_random=True,
                         ring_random=True, io="f32" if io == torch.float32 else "bf16",
                         seed=61)
    B, T, H, dk, dv = inp.dims
    ref_o, ref_S, ref_ring = _oracle(inp)
    d = to_dev(inp, dev)
    st = kda.KDAState(B, H, dk, dv, io=io, device=dev)
    load_state(st, inp)
    pieces = []
    t = 0
    for n, chunk in ((37, 16), (2, 64), (41, 32)):
        sl = slice(t, t + n)
        part = {key: d[key][:, sl].contiguous() for key in ("q", "k", "v", "g", "beta")}
        o = torch.empty(B, n, H, dv, dtype=io, device=dev)
        st.prefill(n, part["q"], part["k"], part["v"], part["g"], part["beta"], d["conv_w"], o,
                   chunk=chunk)
        pieces.append(o)
        t += n
    rest = {key: d[key][:, t:].transpose(0, 1).contiguous()
            for key in ("q", "k", "v", "g", "beta")}
    rest["conv_w"] = d["conv_w"]
    od = run_decode(st, rest, T - t)
    torch.cuda.synchronize()
    got = np.concatenate([f64(p) for p in pieces] + [f64(od).transpose(1, 0, 2, 3)], axis=1)
    if io == torch.float32:
        assert abs_err(got, ref_o) <= 1e-4 and abs_err(f64(st.S), ref_S) <= 1e-4
    else:
        assert rel_err(got, ref_o) <= 2e-2 and rel_err(f64(st.S), ref_S) <= 2e-2
    np.testing.assert_array_equal(f64(st.ring), ref_ring)


def test_prefill_worked_example_flags():
    """Worked example through the chunked path: conv skipped, g = 0, beta = 1."""
    dev = device()
    d = 16
    q = torch.zeros(1, 2, 1, d)
    q[0, :, 0, :2] = torch.tensor([1.0, 3.0])
    v = torch.zeros(1, 2, 1, d)
    v[0, 0, 0, :2] = torch.tensor([2.0, 4.0])
    v[0, 1, 0, :2] = torch.tensor([0.0, 1.0])
    st = kda.KDAState(1, 1, d, d, io=torch.float32, device=dev)
    st.reset()
    o = torch.empty(1, 2, 1, d, device=dev)
    st.prefill(2, q.to(dev), q.to(dev), v.to(dev), torch.zeros(1, 2, 1, d, device=dev),
               torch.ones(1, 2, 1, device=dev), None, o, chunk=16, flags=kda.KDA_F_SKIP_CONV)
    torch.cuda.synchronize()
    o = o.cpu()
    np.testing.assert_allclose(o[0, 0, 0, :2].numpy(), [2.0, 4.0], atol=1e-5)
    np.testing.assert_allclose(o[0, 1, 0, :2].numpy(), [0.0, 1.0], atol=1e-5)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_prologue(io):
    dev = device()
    inp = workloads.make("tiny", T=9, B=2, H=3, dk=32, dv=64, ring_random=True, io=io,
                         seed=71)
    B, T, H, dk, dv = inp.dims
    qh, kh, vh, ring = kda_oracle.prologue(inp.q, inp.k, inp.v, inp.conv_w, inp.ring0)
    d = to_dev(inp, dev)
    dims = kda.make_dims(B, H, dk, dv, kda.KDA_F32 if io == "f32" else kda.KDA_BF16)
    ring_dev = inp.ring0.to(dev)
    qo = torch.empty(B, T, H, dk, device=dev)
    ko = torch.empty_like(qo)
    vo = torch.empty(B, T, H, dv, device=dev)
    kda.kda_conv_prologue(dims, T, d["q"], d["k"], d["v"], d["conv_w"], ring_dev, qo, ko, vo)
    torch.cuda.synchronize()
    tol = 1e-5
    assert abs_err(f64(qo), qh) <= tol and abs_err(f64(ko), kh) <= tol
    assert abs_err(f64(vo), vh) <= 1e-4 * max(1.0, np.abs(vh).max())
    np.testing.assert_array_equal(f64(ring_dev), ring)


def test_prefill_in_captured_graph_matches_eager():
    """A prefill call with a caller-provided workspace launches only kernels
    (preparation, chain, ring advance), so it can be captured in a HIP graph:
    each replay, with eager work and synchronizations between replays, gives
    the eager result bit for bit."""
    dev = device()
    inp = workloads.make("tiny", T=150, B=2, H=2, dk=128, dv=128, io="bf16", s0_random=True,
                         ring_random=True, seed=91)
    B, T, H, dk, dv = inp.dims
    d = to_dev(inp, dev)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(kda.make_dims(B, H, dk, dv, kda.KDA_BF16),
                                                     T, 64), dtype=torch.uint8, device=dev)
    eager = kda.KDAState(B, H, dk, dv, io=torch.bfloat16, device=dev)
    cap = kda.KDAState(B, H, dk, dv, io=torch.bfloat16, device=dev)
    oe = torch.empty(B, T, H, dv, dtype=torch.bfloat16, device=dev)
    oc = torch.empty_like(oe)

    def call(st, o):
        st.prefill(T, d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], o, chunk=64,
                   workspace=ws)

    load_state(cap, inp)
    call(cap, oc)                   # warm-up, eager
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(cap, oc)
    torch.cuda.synchronize()
    for rep in range(3):
        load_state(eager, inp)
        call(eager, oe)
        torch.cuda.synchronize()
        load_state(cap, inp)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(oc, oe), f"replay {rep}: o differs"
        assert torch.equal(cap.S, eager.S) and torch.equal(cap.ring, eager.ring), \
            f"replay {rep}: state differs"


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dk,dv", [(a, b) for a in (16, 32, 64, 128) for b in (16, 32, 64, 128)])
def test_prefill_every_shape(dk, dv, chunk, io):
    """Every supported (d_k, d_v, chunk, I/O type), 70 tokens from a random
    state and ring: each combination of preparation kernel (general or
    token-row) and chain kernel (generic or role-split) that the dispatch can
    choose, against the oracle."""
    dev = device()
    seed = 1000 + dk + 7 * dv + 13 * chunk + (1 if io == "bf16" else 0)
    inp = workloads.make("tiny", T=70, B=1, H=2, dk=dk, dv=dv, io=io, s0_random=True,
                         ring_random=True, seed=seed)
    ref_o, ref_S, ref_ring = _oracle(inp)
    tio = torch.float32 if io == "f32" else torch.bfloat16
    st, o = _prefill(inp, dev, chunk, tio)
    if io == "f32":
        eo, es = abs_err(f64(o), ref_o), abs_err(f64(st.S), ref_S)
        assert eo <= 1e-4 and es <= 1e-4, (eo, es)
    else:
        eo, es = rel_err(f64(o), ref_o), rel_err(f64(st.S), ref_S)
        assert eo <= 2e-2 and es <= 2e-2, (eo, es)
    np.testing.assert_array_equal(f64(st.ring), ref_ring)
