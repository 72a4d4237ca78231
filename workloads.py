"""Seeded synthetic inputs for the KDA workloads.

This module only draws random numbers. It holds none of the recurrence's
arithmetic, and both the GPU tests/benchmark and the CPU oracle take their
inputs from it.

Every workload is drawn on the CPU with one ``torch.Generator`` seeded per
workload, in a fixed order:

    q, k, v, g_raw, beta_raw, conv_w, S0 (if random), ring (if random)

with q, k, v ~ N(0, 1) of shape [B, T, H, d]; g = logsigmoid(g_mu + N(0, 1))
per key channel [B, T, H, dk] (with scalar_g, one per token and head:
[B, T, H], the scalar-alpha Gated DeltaNet form); beta = sigmoid(N(0, 1)) [B, T, H]
(with raw_gates, g and beta hold the pre-activations g_mu + N(0, 1) and
N(0, 1) themselves, drawn from the same stream); conv
weights ~ 0.5 * N(0, 1) of shape [H*(2dk+dv), 4]; S0 ~ 0.02 * N(0, 1) of
shape [B, H, dk, dv]; ring ~ N(0, 1) of shape [B, 3, H*(2dk+dv)]. For
bf16 workloads q, k, v and the ring are rounded to bf16 (round to nearest
even); g, beta, the conv weights and S0 stay fp32. "N(m, s)" means mean m,
standard deviation s.

For decode workloads T is the number of consecutive decode steps; step t
reads q[:, t], ... .
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

# name -> shape and distribution parameters (sizes follow the K3 KDA layer:
# 96 heads with a 128x128 state per head).
WORKLOADS = {
    # 1 layer, batch 1, 2 heads of 16x16, 64 tokens, fp32 throughout.
    "tiny": dict(B=1, T=64, H=2, dk=16, dv=16, io="f32", seed=0,
                 s0_random=False, ring_random=False, g_mu=0.0, chunk=64),
    # One decode step at the K3 shape, fp32, random state and ring.
    "k3_decode1": dict(B=1, T=1, H=96, dk=128, dv=128, io="f32", seed=1,
                       s0_random=True, ring_random=True, g_mu=0.0, chunk=64),
    # 64 independent sequences, 256 consecutive decode steps, bf16 I/O.
    "batched_decode": dict(B=64, T=256, H=96, dk=128, dv=128, io="bf16", seed=2,
                           s0_random=True, ring_random=True, g_mu=0.0, chunk=64),
    # Chunked prefill of 4096 tokens, chunk 64, slow decay, bf16 I/O.
    "prefill_4k": dict(B=1, T=4096, H=96, dk=128, dv=128, io="bf16", seed=3,
                       s0_random=False, ring_random=False, g_mu=2.0, chunk=64),
    # The same two workloads with one decay per token and head (scalar-alpha
    # Gated DeltaNet), g of shape [B, T, H].
    "batched_decode_gdn": dict(B=64, T=256, H=96, dk=128, dv=128, io="bf16", seed=5,
                               s0_random=True, ring_random=True, g_mu=0.0, chunk=64,
                               scalar_g=True),
    "prefill_4k_gdn": dict(B=1, T=4096, H=96, dk=128, dv=128, io="bf16", seed=6,
                           s0_random=False, ring_random=False, g_mu=2.0, chunk=64,
                           scalar_g=True),
}


@dataclass
class Inputs:
    """One workload's tensors, all on the CPU."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    conv_w: torch.Tensor
    S0: torch.Tensor
    ring0: torch.Tensor
    meta: dict = field(default_factory=dict)

    @property
    def dims(self):
        B, T, H, dk = self.q.shape
        return B, T, H, dk, self.v.shape[-1]


def draw(B, T, H, dk, dv, io="f32", seed=0, s0_random=False, ring_random=False,
         g_mu=0.0, scalar_g=False, raw_gates=False, **meta) -> Inputs:
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    ctot = H * (2 * dk + dv)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, dtype=torch.float32)

    q = randn(B, T, H, dk)
    k = randn(B, T, H, dk)
    v = randn(B, T, H, dv)
    g_shape = (B, T, H) if scalar_g else (B, T, H, dk)
    g = randn(*g_shape) + float(g_mu)
    beta = randn(B, T, H)
    if not raw_gates:  # with raw_gates g and beta stay the pre-activations
        g = torch.nn.functional.logsigmoid(g)
        beta = torch.sigmoid(beta)
    conv_w = 0.5 * randn(ctot, 4)
    S0 = 0.02 * randn(B, H, dk, dv) if s0_random else torch.zeros(B, H, dk, dv)
    ring0 = randn(B, 3, ctot) if ring_random else torch.zeros(B, 3, ctot)
    if io == "bf16":
        q, k, v, ring0 = (x.to(torch.bfloat16) for x in (q, k, v, ring0))
    elif io != "f32":
        raise ValueError(f"io must be 'f32' or 'bf16', not {io!r}")
    info = dict(B=B, T=T, H=H, dk=dk, dv=dv, io=io, seed=seed, g_mu=g_mu, scalar_g=scalar_g,
                raw_gates=raw_gates, **meta)
    return Inputs(q, k, v, g, beta, conv_w, S0, ring0, info)


def draw_output_gate(B, T, H, dv, io="f32", seed=0):
    """Inputs of the output gate that follows the readout, from a generator of
    their own (seed + 500,000, so the recurrence's draws are unchanged): gate
    pre-activations z ~ N(0, 1) [B, T, H, dv] (rounded to bf16 for bf16
    workloads) and a norm weight w = 1 + 0.1 * N(0, 1) [dv] (fp32), with
    eps = 1e-5. Returns (z, w, eps)."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed) + 500_000)
    z = torch.randn(B, T, H, dv, generator=gen, dtype=torch.float32)
    w = 1.0 + 0.1 * torch.randn(dv, generator=gen, dtype=torch.float32)
    if io == "bf16":
        z = z.to(torch.bfloat16)
    return z, w, 1e-5


def draw_backward_grads(B, T, H, dk, dv, io="f32", seed=0):
    """Loss gradients for a backward pass, from a generator of their own
    (seed + 600,000, so the forward draws are unchanged): dO ~ N(0, 1)
    [B, T, H, dv] (rounded to bf16 for bf16 workloads) and dST ~ N(0, 1)
    [B, H, dk, dv] (fp32). Returns (dO, dST)."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed) + 600_000)
    dO = torch.randn(B, T, H, dv, generator=gen, dtype=torch.float32)
    dST = torch.randn(B, H, dk, dv, generator=gen, dtype=torch.float32)
    if io == "bf16":
        dO = dO.to(torch.bfloat16)
    return dO, dST


def draw_prologue_grads(B, T, H, dk, dv, io="f32", seed=0):
    """Gradients of the activations q^, k^, v^ for a backward pass through
    the prologue, from a generator of their own (seed + 700,000): each
    ~ N(0, 1), rounded to bf16 for bf16 workloads. Returns (dqh, dkh, dvh)."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed) + 700_000)
    out = [torch.randn(B, T, H, d, generator=gen, dtype=torch.float32) for d in (dk, dk, dv)]
    if io == "bf16":
        out = [x.to(torch.bfloat16) for x in out]
    return tuple(out)


def make(name: str, **overrides) -> Inputs:
    """Draw the named workload; keyword overrides replace its parameters
    (e.g. a smaller T for a quick check)."""
    params = dict(WORKLOADS[name])
    params.update(overrides)
    inp = draw(**params)
    inp.meta["name"] = name
    return inp


# ---------------------------------------------------------------------------
# The stacked K3 KDA workload: 69 KDA layers, 16 sequences, 96 heads of
# 128x128; each (layer, sequence) has a 32768-token prefill from a zero state
# and zero ring, then 64 decode steps. It is far too large for host memory,
# so it is drawn on the device, one (layer, sequence) at a time, with a
# generator of that device seeded per (layer, sequence); the checked pairs
# are copied back to the host for the oracle.
STACK = dict(layers=69, B=16, T=32768, decode_steps=64, H=96, dk=128, dv=128)


def stack_seed(layer: int, seq: int) -> int:
    return 4_000_000 + 100 * layer + seq


def draw_stack_seq(layer: int, seq: int, T: int, H: int, dk: int, dv: int,
                   device) -> dict:
    """Tokens 0..T-1 of one (layer, sequence): q, k, v bf16 [1, T, H, d],
    g fp32 [1, T, H, dk], beta fp32 [1, T, H]; drawn in the order q, k, v,
    g_raw, beta_raw with the distributions of the module docstring (g_mu 0)."""
    gen = torch.Generator(device=device).manual_seed(stack_seed(layer, seq))

    def randn(*shape):
        return torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)

    q = randn(1, T, H, dk).to(torch.bfloat16)
    k = randn(1, T, H, dk).to(torch.bfloat16)
    v = randn(1, T, H, dv).to(torch.bfloat16)
    g = torch.nn.functional.logsigmoid(randn(1, T, H, dk))
    beta = torch.sigmoid(randn(1, T, H))
    return dict(q=q, k=k, v=v, g=g, beta=beta)


def draw_stack_conv_w(layer: int, H: int, dk: int, dv: int, device) -> torch.Tensor:
    """The conv weights of one layer, [H*(2dk+dv), 4] fp32 ~ 0.5 N(0, 1), from
    the generator seeded 4,000,000 + 100 layer + 99 (no sequence uses 99)."""
    gen = torch.Generator(device=device).manual_seed(4_000_000 + 100 * layer + 99)
    return 0.5 * torch.randn(H * (2 * dk + dv), 4, generator=gen, dtype=torch.float32,
                             device=device)


def draw_layer_activations(B: int, T: int, H: int, dk: int, dv: int, device,
                           seed: int) -> list:
    """Inputs of a backward call at the size of a training layer, drawn on the
    device one sequence at a time (no host copy of the ~150 GB they take at
    16 x 32768 x 96 heads): q^ and k^ unit vectors per head (bf16), v^ ~
    N(0, 1) (bf16), g = log sigmoid(N(0, 1)), beta = sigmoid(N(0, 1)),
    S0 ~ N(0, 1) / 4, dO ~ N(0, 1) (bf16), dST ~ N(0, 1).
    Returns [q, k, v, g, beta, S0, dO, dST]."""
    gen = torch.Generator(device=device).manual_seed(seed)
    bf = torch.bfloat16
    q = torch.empty(B, T, H, dk, dtype=bf, device=device)
    k = torch.empty_like(q)
    v = torch.empty(B, T, H, dv, dtype=bf, device=device)
    g = torch.empty(B, T, H, dk, device=device)
    dO = torch.empty(B, T, H, dv, dtype=bf, device=device)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)

    for b in range(B):
        for dst in (q[b], k[b]):
            dst.copy_(torch.nn.functional.normalize(randn(T, H, dk), dim=-1))
        v[b].copy_(randn(T, H, dv))
        g[b].copy_(torch.nn.functional.logsigmoid(randn(T, H, dk)))
        dO[b].copy_(randn(T, H, dv))
    beta = torch.sigmoid(randn(B, T, H))
    S0 = randn(B, H, dk, dv) * 0.25
    dST = randn(B, H, dk, dv)
    return [q, k, v, g, beta, S0, dO, dST]
