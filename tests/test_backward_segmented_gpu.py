"""kda_chunk_backward in a workspace smaller than the one-pass layout: the
chunks are taken in ranges (the state entering each range kept from a first
forward pass, the state gradient handed from range to range), and the
gradients are bitwise those of the one-pass call. At the size of a layer of
the 69-layer model's training step, 16 sequences of 32768 tokens with 96
heads of 128 x 128 (451 GB in one pass), the call runs in a workspace of a
few tens of GB; one sequence-head of it is checked against the fp64 oracle
and eight heads of one sequence bitwise against a one-pass call on them
alone (heads and sequences are independent).

The training recurrence is the chunkwise form of "为什么 Kimi K3 敢把 KV Cache
扔掉？…", section 5 (the state handed from chunk to chunk).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as kda
import workloads
from oracle import kda_oracle
from tests.gpu_util import device, f64, rel_err
from tests.test_backward_gpu import activations

pytestmark = pytest.mark.gpu


def _outputs(B, T, H, dk, dv, io, dev):
    return [torch.empty(B, T, H, dk, dtype=io, device=dev),
            torch.empty(B, T, H, dk, dtype=io, device=dev),
            torch.empty(B, T, H, dv, dtype=io, device=dev),
            torch.empty(B, T, H, dk, device=dev), torch.empty(B, T, H, device=dev),
            torch.empty(B, H, dk, dv, device=dev)]


def _call(dims, T, ins, chunk, ws_bytes, dev, want_dS0=True):
    B, H, dk, dv = dims.batch, dims.heads, dims.d_k, dims.d_v
    io = torch.bfloat16 if dims.io == kda.KDA_BF16 else torch.float32
    out = _outputs(B, T, H, dk, dv, io, dev)
    if not want_dS0:
        out[5] = None
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws.view(torch.float32)[: ws_bytes // 4].fill_(float("nan"))
    kda.kda_chunk_backward(dims, T, *ins, *out, chunk=chunk, workspace=ws)
    torch.cuda.synchronize()
    return out


def _ranges_of(dims, T, chunk, ws_bytes):
    """How many chunks one range takes for ws_bytes (the rule the call uses,
    from the sizes the library reports)."""
    nc = -(-T // chunk)
    full = kda.kda_backward_workspace_bytes(dims, T, chunk)
    if ws_bytes >= full:
        return nc
    per_chunk = full // nc
    state = dims.batch * dims.heads * dims.d_k * dims.d_v * 4
    for L in range(min(nc - 1, ws_bytes // per_chunk), 0, -1):
        if L * per_chunk + (-(-nc // L)) * state <= ws_bytes:
            return L
    return 0


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("state", ["S0+dST", "none"])
def test_segmented_backward_is_bitwise_one_pass(io, chunk, state):
    dev = device()
    inp = workloads.draw(2, 301, 3, 64, 32, io=io, seed=1400 + chunk, s0_random=True,
                         ring_random=True)
    B, T, H, dk, dv = inp.dims
    qh, kh, vh = activations(inp)
    dO, dST = workloads.draw_backward_grads(B, T, H, dk, dv, io=io, seed=1400 + chunk)
    with_state = state == "S0+dST"
    ins = [x.to(dev) if x is not None else None for x in
           (qh, kh, vh, inp.g, inp.beta, inp.S0 if with_state else None, dO,
            dST if with_state else None)]
    dims = kda.make_dims(B, H, dk, dv, inp.q.dtype)
    full = kda.kda_backward_workspace_bytes(dims, T, chunk)
    least = kda.kda_backward_workspace_min_bytes(dims, T, chunk)
    nc = -(-T // chunk)
    assert 0 < least < full
    ref = _call(dims, T, ins, chunk, full, dev)
    per_chunk = full // nc
    state_b = B * H * dk * dv * 4
    sizes = {least, least + 16, full - 16}
    for L in (1, 2, 3, nc // 2, nc - 1):  # a workspace that gives ranges of L chunks
        sizes.add(L * per_chunk + (-(-nc // L)) * state_b)
    seen = set()
    for nbytes in sorted(sizes):
        if nbytes < least:
            continue
        L = _ranges_of(dims, T, chunk, nbytes)
        seen.add(L)
        got = _call(dims, T, ins, chunk, nbytes, dev)
        for name, x, y in zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), ref, got):
            assert torch.isfinite(x.float()).all(), name
            assert torch.equal(x, y), (name, nbytes, L)
    assert 1 in seen and nc - 1 in seen and len(seen) >= 4, seen
    # dS0 not wanted: the other gradients are unchanged
    got = _call(dims, T, ins, chunk, least, dev, want_dS0=False)
    for x, y in zip(ref[:5], got[:5]):
        assert torch.equal(x, y)


def test_segmented_backward_rejects_a_smaller_workspace():
    dev = device()
    dims = kda.make_dims(1, 2, 32, 32, kda.KDA_F32)
    T = 200
    least = kda.kda_backward_workspace_min_bytes(dims, T, 64)
    ins = [torch.zeros(1, T, 2, 32, device=dev) for _ in range(3)]
    ins += [torch.zeros(1, T, 2, 32, device=dev), torch.zeros(1, T, 2, device=dev), None,
            torch.zeros(1, T, 2, 32, device=dev), None]
    with pytest.raises(kda.KDAError, match="workspace"):
        _call(dims, T, ins, 64, least - 16, dev)


def test_backward_layer_16x32768_in_bounded_workspace():
    dev = device()
    B, T, H, dk, dv = 16, 32768, 96, 128, 128
    dims = kda.make_dims(B, H, dk, dv, torch.bfloat16)
    ws_bytes = 24 << 30
    free, _ = torch.cuda.mem_get_info(dev)
    need = B * T * H * (dk * 2 * 2 + dv * 2 + dk * 4 + 4) * 2 + ws_bytes
    if free < need + (8 << 30):
        pytest.skip(f"needs about {need >> 30} GiB of device memory, {free >> 30} free")
    assert kda.kda_backward_workspace_bytes(dims, T, 64) > 400e9  # one pass would not fit
    assert kda.kda_backward_workspace_min_bytes(dims, T, 64) < ws_bytes
    L = _ranges_of(dims, T, 64, ws_bytes)
    print(f"ranges of {L} chunks, {-(-512 // L)} ranges", flush=True)
    ins = workloads.draw_layer_activations(B, T, H, dk, dv, dev, seed=1500)
    out = _outputs(B, T, H, dk, dv, torch.bfloat16, dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    kda.kda_chunk_backward(dims, T, *ins, *out, chunk=64, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    print(f"16 x 32768 x 96 heads: {e0.elapsed_time(e1):.1f} ms", flush=True)
    del ws
    for x in out:
        assert torch.isfinite(x.float()).all()
    # eight heads of sequence 5 alone, one pass: bitwise the same
    b, hs = 5, slice(40, 48)
    sub = [x[b:b + 1, :, hs].contiguous() for x in ins[:5]]
    sub += [ins[5][b:b + 1, hs].contiguous(), ins[6][b:b + 1, :, hs].contiguous(),
            ins[7][b:b + 1, hs].contiguous()]
    dsub = kda.make_dims(1, 8, dk, dv, torch.bfloat16)
    one = _call(dsub, T, sub, 64, kda.kda_backward_workspace_bytes(dsub, T, 64), dev)
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dbeta"), one[:5], out[:5]):
        assert torch.equal(x, y[b:b + 1, :, hs]), name
    assert torch.equal(one[5], out[5][b:b + 1, hs])
    # sequence 11, head 77 against the fp64 oracle
    b, h = 11, 77
    cut = [x[b:b + 1, :, h:h + 1].cpu() for x in (ins[0], ins[1], ins[2], ins[3], ins[4], ins[6])]
    S0 = ins[5][b:b + 1, h:h + 1].cpu()
    dST = ins[7][b:b + 1, h:h + 1].cpu()
    ref = kda_oracle.default().core_backward(cut[0], cut[1], cut[2], cut[3], cut[4], S0, cut[5],
                                             dST)
    got = [f64(out[0][b:b + 1, :, h:h + 1]), f64(out[1][b:b + 1, :, h:h + 1]),
           f64(out[2][b:b + 1, :, h:h + 1]), f64(out[3][b:b + 1, :, h:h + 1]),
           f64(out[4][b:b + 1, :, h:h + 1]), f64(out[5][b:b + 1, h:h + 1])]
    errs = [rel_err(x, r) for x, r in zip(got, ref)]
    print("oracle rel errs", ["%.2e" % e for e in errs], flush=True)
    assert max(errs) <= 2e-2
    assert np.isfinite(got[0]).all()
