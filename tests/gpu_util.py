"""Helpers shared by the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def f64(t):
    return t.detach().to("cpu").double().numpy()


def rel_err(got, ref):
    """max |got - ref| / max |ref| over the whole tensor."""
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def abs_err(got, ref):
    return float(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)).max())


def channels(H, dk, dv, heads):
    """Conv/ring channel indices of the given heads, in q | k | v order."""
    q = [h * dk + i for h in heads for i in range(dk)]
    k = [H * dk + h * dk + i for h in heads for i in range(dk)]
    v = [2 * H * dk + h * dv + j for h in heads for j in range(dv)]
    return np.array(q + k + v)


def subset(inp: workloads.Inputs, seqs, heads) -> workloads.Inputs:
    """The same workload restricted to some sequences and heads (heads are
    independent, so the oracle on the subset is exact for those heads)."""
    B, T, H, dk, dv = inp.dims
    seqs, heads = list(seqs), list(heads)
    ch = torch.from_numpy(channels(H, dk, dv, heads))
    sb = torch.tensor(seqs)
    hb = torch.tensor(heads)
    return workloads.Inputs(
        q=inp.q[sb][:, :, hb], k=inp.k[sb][:, :, hb], v=inp.v[sb][:, :, hb],
        g=inp.g[sb][:, :, hb], beta=inp.beta[sb][:, :, hb],
        conv_w=inp.conv_w[ch], S0=inp.S0[sb][:, hb], ring0=inp.ring0[sb][:, :, ch],
        meta=dict(inp.meta, seqs=seqs, heads=heads))


def per_channel_g(inp: workloads.Inputs) -> workloads.Inputs:
    """A scalar-decay workload (g [B, T, H]) with g repeated over the d_k key
    channels ([B, T, H, d_k]): the per-channel form the oracle and the
    per-channel library call take."""
    if inp.g.dim() == 4:
        return inp
    dk = inp.q.shape[-1]
    g = inp.g.unsqueeze(-1).expand(*inp.g.shape, dk).contiguous()
    return workloads.Inputs(q=inp.q, k=inp.k, v=inp.v, g=g, beta=inp.beta, conv_w=inp.conv_w,
                            S0=inp.S0, ring0=inp.ring0, meta=dict(inp.meta, scalar_g=False))


def to_dev(inp: workloads.Inputs, dev, step_major=False):
    """Device copies. step_major=True lays q, k, v, g, beta out as [T, B, ...]
    so that each decode step's inputs are contiguous."""
    def mv(x):
        if step_major:
            x = x.transpose(0, 1)
        return x.contiguous().to(dev)
    return dict(q=mv(inp.q), k=mv(inp.k), v=mv(inp.v), g=mv(inp.g), beta=mv(inp.beta),
                conv_w=inp.conv_w.contiguous().to(dev))


def load_state(st, inp: workloads.Inputs):
    """Copy S0 and the ring of a workload into a KDAState (a restore)."""
    st.S.copy_(inp.S0.to(st.S.device))
    st.ring.copy_(inp.ring0.to(st.ring.device, st.ring.dtype))


def run_decode(st, d, T, o_all=None, flags=0):
    """T decode steps from step-major device inputs; returns o [T, B, H, dv]."""
    B, H = d["q"].shape[1], d["q"].shape[2]
    dv = d["v"].shape[-1]
    if o_all is None:
        o_all = torch.empty(T, B, H, dv, dtype=st.io, device=d["q"].device)
    for t in range(T):
        st.decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t], d["conv_w"],
                       o_all[t], flags=flags)
    return o_all
