"""The stacked K3 KDA workload at full size on the GPU: 69 layers x 16
sequences x 96 heads of 128x128, a 32768-token chunked prefill per (layer,
sequence) from a zero state, then 64 decode steps taken token by token
through all 69 layers. The fp64 oracle checks two (layer, sequence) pairs
in full, (0, 0) and (68, 15): o of all 32832 tokens and the final S, to
max|err|/max|ref| <= 2e-2 (bf16 I/O, fp32 state)."""
import time

import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as kda
import workloads
from oracle import kda_oracle
from tests.gpu_util import device, f64, rel_err

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CHECKED = [(0, 0), (68, 15)]


def test_k3_stack_69_layers_prefill_then_decode():
    dev = device()
    cfg = workloads.STACK
    L, B, T, TD = cfg["layers"], cfg["B"], cfg["T"], cfg["decode_steps"]
    H, dk, dv = cfg["H"], cfg["dk"], cfg["dv"]
    bf = torch.bfloat16
    t0 = time.perf_counter()
    ws = torch.empty(2 << 30, dtype=torch.uint8, device=dev)  # shared prefill workspace
    states, dec, weights = [], [], []
    host_inputs, pre_o = {}, {}
    q = torch.empty(B, T, H, dk, dtype=bf, device=dev)
    k = torch.empty_like(q)
    v = torch.empty(B, T, H, dv, dtype=bf, device=dev)
    g = torch.empty(B, T, H, dk, device=dev)
    beta = torch.empty(B, T, H, device=dev)
    o = torch.empty(B, T, H, dv, dtype=bf, device=dev)
    for layer in range(L):
        w = workloads.draw_stack_conv_w(layer, H, dk, dv, dev)
        d = dict(q=torch.empty(TD, B, H, dk, dtype=bf, device=dev),
                 k=torch.empty(TD, B, H, dk, dtype=bf, device=dev),
                 v=torch.empty(TD, B, H, dv, dtype=bf, device=dev),
                 g=torch.empty(TD, B, H, dk, device=dev),
                 beta=torch.empty(TD, B, H, device=dev))
        for s in range(B):
            x = workloads.draw_stack_seq(layer, s, T + TD, H, dk, dv, dev)
            for name, buf in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
                buf[s].copy_(x[name][0, :T])
                d[name][:, s].copy_(x[name][0, T:])
            if (layer, s) in CHECKED:
                host_inputs[(layer, s)] = {name: t.cpu() for name, t in x.items()}
            del x
        st = kda.KDAState(B, H, dk, dv, io=bf, device=dev)
        st.reset()
        st.prefill(T, q, k, v, g, beta, w, o, chunk=64, workspace=ws)
        for (cl, cs) in CHECKED:
            if cl == layer:
                pre_o[(cl, cs)] = o[cs].cpu()
        states.append(st)
        dec.append(d)
        weights.append(w)
        if layer % 10 == 0 or layer == L - 1:
            torch.cuda.synchronize()
            print(f"layer {layer}: drawn and prefilled, {time.perf_counter() - t0:.1f} s",
                  flush=True)
    del q, k, v, g, beta, o, ws
    dec_o = {key: torch.empty(TD, H, dv, dtype=bf, device=dev) for key in CHECKED}
    ot = torch.empty(B, H, dv, dtype=bf, device=dev)
    for t in range(TD):
        for layer in range(L):
            d = dec[layer]
            states[layer].decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t],
                                      weights[layer], ot)
            for (cl, cs) in CHECKED:
                if cl == layer:
                    dec_o[(cl, cs)][t].copy_(ot[cs])
    torch.cuda.synchronize()
    print(f"64 decode steps through 69 layers done, {time.perf_counter() - t0:.1f} s",
          flush=True)
    assert all(torch.isfinite(st.S).all().item() for st in states)

    for (layer, s) in CHECKED:
        x = host_inputs[(layer, s)]
        ref_o, ref_S, ref_ring = kda_oracle.forward(
            x["q"], x["k"], x["v"], x["g"], x["beta"], weights[layer].cpu(),
            torch.zeros(1, H, dk, dv), torch.zeros(1, 3, H * (2 * dk + dv)))
        got = np.concatenate([f64(pre_o[(layer, s)])[None], f64(dec_o[(layer, s)])[None]],
                             axis=1)
        eo = rel_err(got, ref_o)
        es = rel_err(f64(states[layer].S[s:s + 1]), ref_S)
        print(f"stack (layer {layer}, seq {s}): rel err o={eo:.2e} S={es:.2e}, "
              f"{time.perf_counter() - t0:.1f} s", flush=True)
        assert eo <= 2e-2 and es <= 2e-2
        np.testing.assert_array_equal(f64(states[layer].ring[s:s + 1]), ref_ring)
