"""KDA benchmark on one MI355X: batched decode throughput (the headline), the
4096-token chunked prefill alongside it, roofline fractions, and the fp64 CPU
oracle timed on the host as a reported baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

A step is one decode token for each of 64 independent sequences of one KDA
layer (96 heads, 128x128 fp32 state per head, bf16 q/k/v/o, fp32 g/beta):
short conv + SiLU + L2, decay, delta, rank-1 write and readout, fused in one
kernel launch. Inputs for 256 consecutive steps are staged in HBM before the
timed region; step i uses staged step i % 256. The chunked prefill of 4096
tokens (batch 1, 96 heads, chunk 64, bf16) is timed separately in the same
run and reported under "prefill", and the 69-layer stack (16 sequences, one
decode token through all 69 layers as one captured HIP graph over 6.5 GiB of
state; one layer's 32768-token prefill of the 16 sequences) under "stack", and
the same decode and prefill workloads with one decay per token and head
(KDA_F_SCALAR_G, the scalar-alpha Gated DeltaNet form) under "scalar_decay",
the same with the gates formed in the kernels from raw projections
(KDA_F_RAW_GATES) under "raw_gates",
and the output gate (gated RMSNorm of the readout: fused into the decode step,
and as its own kernel on the prefill output) under "output_gate".
Beside them: the latency of one K3-shape decode step (batch 1, fp32, warm and
with the caches flushed) under "single_step", the practical bandwidth ceiling
of a state stream ("stream_ceiling": a non-temporal in-place read-modify-write
of 1 GiB, kda_stream_rmw; "roofline.frac_of_stream_ceiling"; a plain torch
copy beside it), and
the fp64 oracle timed on the host (all cores and one core on the decode
workload, all cores on the 4096-token prefill) under "cpu_baseline".
One JSON line is printed.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_DENSE_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_VECTOR_TFLOPS = 157.3      # MI355X fp32 vector (and fp32 MFMA)
METRIC = ("KDA tokens/s: decode (B×96h×128²) + prefill T=4K; "
          "HBM GB/s & MFMA % of peak")


def decode_bytes(B, H, dk, dv, io_bytes=2, scalar_g=False):
    """Algorithmic HBM bytes of one decode launch (all B sequences)."""
    ctot = H * (2 * dk + dv)
    state = 2 * B * H * dk * dv * 4                   # read + write of S
    tok_in = B * H * (2 * dk + dv) * io_bytes          # raw q, k, v
    gates = B * H * (1 if scalar_g else dk) * 4 + B * H * 4   # g, beta
    ring = 2 * B * 3 * ctot * io_bytes                 # ring read + write
    out = B * H * dv * io_bytes                        # o
    weights = ctot * 4 * 4                             # conv weights, once
    return state + tok_in + gates + ring + out + weights


def decode_flops(B, H, dk, dv):
    # decay (dk*dv), two column reductions (2*2*dk*dv), rank-1 write (2*dk*dv)
    return B * H * 7 * dk * dv


def prefill_bytes(B, T, H, dk, dv, io_bytes=2, scalar_g=False):
    """Compulsory HBM bytes of a T-token prefill: inputs, outputs, S in/out."""
    g_bytes = 4 if scalar_g else dk * 4
    return (B * T * H * ((2 * dk + dv) * io_bytes + g_bytes + 4 + dv * io_bytes)
            + 2 * B * H * dk * dv * 4)


def prefill_flops(B, T, H, dk, dv, C):
    """Algorithmic FLOPs of the chunked form per token-head, the count of the
    hot-path scope table: the three state contractions (W S or K~ S, Q~ S,
    K^T U: 6 d^2), the four triangular C x C by d products (A, P, T V or
    T K~, P U: 4 C d, half of each dense product) and the triangular inverse
    (C^2 / 3); d = dk = dv. 132,437 at d = 128, C = 64."""
    d = dk
    per = 6 * dk * dv + 4 * C * d + (C * C) // 3
    return B * T * H * per


def prefill_flops_as_built(B, T, H, dk, dv, C):
    """The count the kernels' own products add up to per token-head (a coarser
    average of the triangular products): 6 dk dv + 2 C dk (A, P) +
    C (dk + dv) (W, U') + C dv (P U) + C^2 / 3."""
    per = 6 * dk * dv + 2 * C * dk + C * (dk + dv) + C * dv + (C * C) // 3
    return B * T * H * per


def backward_flops(B, T, H, dk, dv, C):
    """Algorithmic FLOPs of the chunked backward per token-head, as its kernels
    compute it: the forward recomputed (A and P: 2 C dk; W and U': C (dk+dv);
    U = U' - W S and the state update: 4 dk dv; the inverse C^2/3), the
    reverse chain (P^T dO: C dv; K^d dS, Q~^T dO, W^T dU: 6 dk dv), the dense
    gradients (dO S0^T, dU S0^T, U dS1^T: 6 dk dv; dP: C dv), the solve
    gradients (X^T dW, X^T dU: C (dk+dv); dX: 2 C (dk+dv); T1 and dM: 2 C^2/3)
    and the decayed-Gram gradients (row and column side: 4 C dk)."""
    per = (2 * C * dk + C * (dk + dv) + 4 * dk * dv + (C * C) // 3 +
           C * dv + 6 * dk * dv +
           6 * dk * dv + C * dv +
           3 * C * (dk + dv) + 2 * (C * C) // 3 +
           4 * C * dk)
    return B * T * H * per


def backward_forward_flops(B, T, H, dk, dv, C):
    """The part of backward_flops that recomputes the forward (A and P, W and
    U', U and the state update, the inverse)."""
    per = 2 * C * dk + C * (dk + dv) + 4 * dk * dv + (C * C) // 3
    return B * T * H * per


def backward_bytes(B, T, H, dk, dv, io_bytes=2):
    """Compulsory bytes of one backward call: q^, k^, v^, dO and dq, dk, dv in
    the I/O type, g and dg fp32, beta and dbeta fp32, plus S0, dST and dS0."""
    per_tok = 2 * ((2 * dk + dv) + dv) * io_bytes + 2 * dk * 4 + 2 * 4
    return B * T * H * per_tok + 3 * B * H * dk * dv * 4


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_b64_h96_d128_bf16_traffic.json")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_t4096_h96_d128_bf16_traffic.json")
CSRC = "gated_delta_rule_83_amd/csrc/"
# (file, first marker, last marker): the digest covers only the text the
# kernel is built from; None markers = the whole file
COMMON_DECODE_PART = (CSRC + "kda_common.h", "namespace kda {",
                      "hipError_t launch_decode(")
DECODE_SOURCES = [(CSRC + "kda_decode.hip", None, None), COMMON_DECODE_PART]
PREFILL_SOURCES = [(CSRC + "kda_prep_rows.hip", None, None),
                   (CSRC + "kda_prefill.hip", None, None),
                   (CSRC + "kda_prefill.h", None, None),
                   (CSRC + "kda_common.h", "namespace kda {", "hipError_t launch_prefill(")]


def source_digest(parts):
    import hashlib

    h = hashlib.sha256()
    for rel, first, last in parts:
        with open(os.path.join(ROOT, rel), "rb") as f:
            text = f.read()
        if first is not None:
            a = text.index(first.encode())
            b = text.index(last.encode(), a) + len(last)
            text = text[a:b]
        h.update(text)
    return h.hexdigest()


def measured_traffic(path, parts):
    """The committed FETCH_SIZE/WRITE_SIZE record of a kernel, or None when
    its source changed since the counters were taken."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest(parts):
        return None
    return rec


def counter_means(csv_path, counter):
    """Mean per dispatch of one counter, per (kernel name, grid size), from a
    rocprofv3 counter-collection CSV (values of one dispatch summed over
    instances)."""
    import collections
    import csv

    per = collections.defaultdict(lambda: collections.defaultdict(float))
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            name = row.get("Kernel_Name") or row.get("Kernel-Name")
            disp = row.get("Dispatch_Id") or row.get("Dispatch-Id")
            per[(name, row.get("Grid_Size", ""))][disp] += float(row["Counter_Value"])
    return {key: (sum(d.values()) / len(d), len(d)) for key, d in per.items()}


def record_traffic(fetch_csv, write_csv, command):
    """Writes profiles/decode_b64_h96_d128_bf16_traffic.json and profiles/prefill_t4096_h96_d128_bf16_traffic.json
    from the FETCH_SIZE and WRITE_SIZE counter runs of this benchmark
    (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, each over
    `python bench.py ... --no-stack --no-gdn --no-backward`). The counters
    are scaled by what they read for kda_stream_rmw over 6 GiB in the same
    runs (the stream-ceiling leg: 6 GiB read, 6 GiB written per dispatch)."""
    fetch, write = counter_means(fetch_csv, "FETCH_SIZE"), counter_means(write_csv, "WRITE_SIZE")

    def pick(table, *parts, grid=None):
        hits = [(n, v) for (n, gs), v in table.items()
                if all(p in n for p in parts) and (grid is None or gs == str(grid))]
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel matching {parts}, found {[n for n, _ in hits]}")
        return hits[0]

    calib_bytes = 6 << 30  # one stream_rmw_kernel thread per 8 x 16 bytes
    calib_kib, calib_grid = float(calib_bytes >> 10), calib_bytes // (16 * 8)
    fscale = calib_kib / pick(fetch, "stream_rmw_kernel", grid=calib_grid)[1][0]
    wscale = calib_kib / pick(write, "stream_rmw_kernel", grid=calib_grid)[1][0]
    common = {"scale": "FETCH_SIZE x %.4f, WRITE_SIZE x %.4f (kda_stream_rmw over 6 GiB: "
                       "6 GiB read and 6 GiB written per dispatch)" % (fscale, wscale),
              "fetch_scale": fscale, "write_scale": wscale, "command": command}

    def traffic(parts, grid):
        (name, (f_kib, nf)) = pick(fetch, *parts, grid=grid)
        (_, (w_kib, _)) = pick(write, *parts, grid=grid)
        return name, nf, f_kib, w_kib, 1024 * (f_kib * fscale + w_kib * wscale)

    # the 64-sequence decode without the gate: 64 x 96 workgroups of 1024
    name, n, f_kib, w_kib, tb = traffic(("decode_step_kernel<128, 128, 1024",
                                         "false>(kda::DecodeAr"), 64 * 96 * 1024)
    algo = decode_bytes(64, 96, 128, 128)
    rec = dict(common, kernel=name, dispatches=n,
               workload="64 sequences x 96 heads x 128x128, bf16 I/O",
               source_files=[p_ for p_, _, _ in DECODE_SOURCES],
               source_digest=source_digest(DECODE_SOURCES),
               fetch_kib_per_dispatch=f_kib, write_kib_per_dispatch=w_kib,
               traffic_bytes_per_launch=tb, algorithmic_bytes_per_launch=algo,
               traffic_over_algorithmic=tb / algo)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    per_kernel, total = {}, 0.0
    for label, parts, grid in (
            ("prep", ("prefill_prep_rows_kernel<64, 128, 128, true, false, false>",),
             64 * 96 * 256),
            ("chain", ("prefill_chain_roles_kernel",), 2 * 96 * 512),
            ("ring_advance", ("ring_advance_kernel", "DF16b"), None)):
        if label == "ring_advance" and not any(all(p in n for p in parts) for n, _ in fetch):
            continue  # the bf16 chain advances the ring itself
        name, n, f_kib, w_kib, tb = traffic(parts, grid)
        per_kernel[label] = {"kernel": name, "dispatches": n, "fetch_kib_per_dispatch": f_kib,
                             "write_kib_per_dispatch": w_kib, "traffic_bytes": tb}
        total += tb
    palgo = prefill_bytes(1, 4096, 96, 128, 128)
    rec = dict(common, workload="prefill T=4096, batch 1, 96 heads of 128x128, chunk 64, bf16",
               source_files=[p_ for p_, _, _ in PREFILL_SOURCES],
               source_digest=source_digest(PREFILL_SOURCES), per_kernel=per_kernel,
               traffic_bytes_per_call=total, compulsory_bytes_per_call=palgo,
               traffic_over_compulsory=total / palgo)
    with open(PREFILL_TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    with open(TRAFFIC_FILE) as f:
        dec = json.load(f)
    print(json.dumps({"decode_traffic_over_algorithmic": dec["traffic_over_algorithmic"],
                      "prefill_traffic_over_compulsory": total / palgo,
                      "prefill_per_kernel_MB": {k: v["traffic_bytes"] / 1e6
                                                for k, v in per_kernel.items()}}))


def single_step_latency(kda, workloads, torch, dev, reps=20):
    """One decode step of the K3 shape (batch 1, 96 heads of 128x128, fp32
    I/O, 6 MiB of state): median latency of single launches, warm (state in
    the caches) and flushed (a 512 MiB buffer written between launches)."""
    inp = workloads.make("k3_decode1")
    B, T, H, dk, dv = inp.dims
    d = {name: getattr(inp, name)[:, 0].contiguous().to(dev)
         for name in ("q", "k", "v", "g", "beta")}
    w = inp.conv_w.to(dev)
    st = kda.KDAState(B, H, dk, dv, io=torch.float32, device=dev)
    st.S.copy_(inp.S0.to(dev))
    st.ring.copy_(inp.ring0.to(dev))
    o = torch.empty(B, H, dv, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def once(flushed):
        if flushed:
            flush.fill_(1)
        torch.cuda.synchronize()
        ev0.record()
        st.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], w, o)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e3

    for _ in range(5):
        once(False)
    warm = sorted(once(False) for _ in range(reps))[reps // 2]
    cold = sorted(once(True) for _ in range(reps))[reps // 2]
    del flush
    # consecutive steps issued back to back (one token after another of the
    # same sequence, no event between them)
    n = 200
    b2b = back_to_back_ms(
        torch, lambda: st.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], w, o), n) * 1e3
    return {"workload": "one decode step, batch 1, 96 heads of 128x128 fp32 state (6 MiB), "
                        "fp32 q/k/v/o; median of single launches",
            "latency_us_warm": warm, "latency_us_flushed": cold,
            "tokens_per_s_warm": 1e6 / warm, "tokens_per_s_flushed": 1e6 / cold,
            "us_per_step_back_to_back": b2b}


def stack_bench(kda, workloads, torch, dev, args):
    """The 69-layer stack of the K3 KDA layers (16 sequences, 96 heads of
    128x128 per layer): one decode token through all layers, the 69 launches
    captured in one HIP graph and replayed (each replay advances every
    layer's state and ring); and one layer's 32768-token chunked prefill of
    the 16 sequences. Inputs are drawn on the device with the stack recipe
    and are resident before timing."""
    cfg = workloads.STACK
    L, B, T, H, dk, dv = (cfg[x] for x in ("layers", "B", "T", "H", "dk", "dv"))
    bf = torch.bfloat16
    gen = torch.Generator(device=dev).manual_seed(5)
    states, xs, ws_ = [], [], []
    for layer in range(L):
        st = kda.KDAState(B, H, dk, dv, io=bf, device=dev)
        st.S.normal_(0.0, 0.02, generator=gen)
        st.ring.zero_()
        states.append(st)
        # one decode token per sequence: tokens 0..B-1 of the layer's draw
        x = workloads.draw_stack_seq(layer, 0, B, H, dk, dv, dev)
        xs.append({name: t[0].contiguous() for name, t in x.items()})
        ws_.append(workloads.draw_stack_conv_w(layer, H, dk, dv, dev))
    o = torch.empty(L, B, H, dv, dtype=bf, device=dev)

    def stack_step():
        for layer in range(L):
            x = xs[layer]
            states[layer].decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], ws_[layer],
                                      o[layer])

    stack_step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stack_step()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.stack_reps):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    step_s = ev0.elapsed_time(ev1) / 1e3 / args.stack_reps
    assert all(torch.isfinite(st.S).all().item() for st in states)
    dbytes = L * decode_bytes(B, H, dk, dv)
    del graph, states, xs, o

    # one layer's prefill of the 16 sequences, T = 32768
    q = torch.empty(B, T, H, dk, dtype=bf, device=dev)
    k = torch.empty_like(q)
    v = torch.empty(B, T, H, dv, dtype=bf, device=dev)
    g = torch.empty(B, T, H, dk, device=dev)
    beta = torch.empty(B, T, H, device=dev)
    for s_ in range(B):
        x = workloads.draw_stack_seq(0, s_, T, H, dk, dv, dev)
        for name, buf in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
            buf[s_].copy_(x[name][0])
        del x
    o = torch.empty(B, T, H, dv, dtype=bf, device=dev)
    ws = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    pst = kda.KDAState(B, H, dk, dv, io=bf, device=dev)

    pst.reset()

    def prefill():
        pst.prefill(T, q, k, v, g, beta, ws_[0], o, chunk=64, workspace=ws)

    for _ in range(2):
        prefill()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(5)]
    for e0, e1 in evs:
        e0.record()
        prefill()
        e1.record()
    torch.cuda.synchronize()
    pre_s = sorted(e0.elapsed_time(e1) for e0, e1 in evs)[len(evs) // 2] / 1e3
    assert torch.isfinite(pst.S).all().item()
    pbytes = prefill_bytes(B, T, H, dk, dv)
    del q, k, v, g, beta, o, ws, pst
    torch.cuda.empty_cache()
    return {
        "workload": "69 KDA layers x 16 sequences x 96 heads of 128x128 fp32 state "
                    "(6.5 GiB), bf16 I/O; decode: one token through all layers (69 launches "
                    "in one HIP graph); prefill: one layer, 32768 tokens per sequence, chunk 64",
        "decode_stack_tokens_per_s": B / step_s, "decode_ms_per_stack_step": step_s * 1e3,
        "decode_bytes_per_stack_step": dbytes, "decode_GBps": dbytes / step_s / 1e9,
        "decode_hbm_frac": dbytes / step_s / 1e9 / HBM_PEAK_GBPS,
        "prefill_layer_tokens_per_s": B * T / pre_s, "prefill_layer_ms": pre_s * 1e3,
        "prefill_hbm_GBps": pbytes / pre_s / 1e9,
        "prefill_stack_tokens_per_s": B * T / (L * pre_s),
    }


def backward_bench(kda, workloads, torch, dev, args):
    """The chunked backward on the 4096-token, 96-head, 128x128 bf16 workload
    (random entering state): q^, k^, v^ made on the device by kda_conv_prologue
    from the raw draws (rounded to bf16), dO and dST from
    workloads.draw_backward_grads; median of event-bracketed calls after
    warm-up calls."""
    inp = workloads.make("prefill_4k", s0_random=True)
    B, T, H, dk, dv = inp.dims
    dims = kda.make_dims(B, H, dk, dv, torch.bfloat16)
    conv_w = inp.conv_w.to(dev)
    ring = torch.zeros(B, 3, H * (2 * dk + dv), dtype=torch.bfloat16, device=dev)
    acts = [torch.empty(B, T, H, d, device=dev) for d in (dk, dk, dv)]
    kda.kda_conv_prologue(dims, T, inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), conv_w, ring,
                          *acts)
    qh, kh, vh = (x.to(torch.bfloat16) for x in acts)
    del acts
    g, beta, S0 = inp.g.to(dev), inp.beta.to(dev), inp.S0.to(dev)
    dO, dST = workloads.draw_backward_grads(B, T, H, dk, dv, io="bf16", seed=3)
    dO, dST = dO.to(dev), dST.to(dev)
    out = [torch.empty(B, T, H, dk, dtype=torch.bfloat16, device=dev),
           torch.empty(B, T, H, dk, dtype=torch.bfloat16, device=dev),
           torch.empty(B, T, H, dv, dtype=torch.bfloat16, device=dev),
           torch.empty(B, T, H, dk, device=dev), torch.empty(B, T, H, device=dev),
           torch.empty(B, H, dk, dv, device=dev)]
    ws = torch.empty(kda.kda_backward_workspace_bytes(dims, T, 64), dtype=torch.uint8,
                     device=dev)

    def call():
        kda.kda_chunk_backward(dims, T, qh, kh, vh, g, beta, S0, dO, dST, *out, chunk=64,
                               workspace=ws)

    for _ in range(args.backward_warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.backward_reps)]
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    med = ms[len(ms) // 2]
    assert all(torch.isfinite(t.float()).all().item() for t in out)
    # the prologue's gradient from the activation gradients just computed
    ctot = H * (2 * dk + dv)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    ring0 = torch.zeros(B, 3, ctot, dtype=torch.bfloat16, device=dev)
    pout = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
            torch.empty(ctot, 4, device=dev), torch.empty(B, 3, ctot, device=dev)]
    pws = torch.empty(kda.kda_prologue_backward_workspace_bytes(dims, T), dtype=torch.uint8,
                      device=dev)

    def pcall():
        kda.kda_prologue_backward(dims, T, q, k, v, conv_w, ring0, out[0], out[1], out[2],
                                  *pout, workspace=pws)

    for _ in range(args.backward_warmup):
        pcall()
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        pcall()
        e1.record()
    torch.cuda.synchronize()
    pms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    pmed = pms[len(pms) // 2]
    assert all(torch.isfinite(t.float()).all().item() for t in pout)
    # raw q, k, v and the three activation gradients read, three raw gradients
    # written (bf16), plus the conv weights and their gradient
    pbytes = B * T * H * (2 * dk + dv) * 2 * 3 + ctot * 4 * 4 * 2
    flops = backward_flops(B, T, H, dk, dv, 64)
    fwd_flops = backward_forward_flops(B, T, H, dk, dv, 64)
    nbytes = backward_bytes(B, T, H, dk, dv)
    res = {"workload": "chunked backward (gradients of q^, k^, v^, g, beta, S0) of the "
                       "4096-token prefill, batch 1, 96 heads of 128x128, chunk 64, bf16 I/O, "
                       "fp32 arithmetic",
           "tokens_per_s": B * T / (med / 1e3), "ms": med, "ms_min": ms[0], "ms_max": ms[-1],
           "calls": len(ms), "flops": flops, "tflops": flops / (med / 1e3) / 1e12,
           "fp32_frac": flops / (med / 1e3) / 1e12 / FP32_VECTOR_TFLOPS,
           "flops_note": "flops includes the forward the call recomputes; flops_gradient "
                         "excludes it",
           "flops_gradient": flops - fwd_flops,
           "fp32_frac_gradient": (flops - fwd_flops) / (med / 1e3) / 1e12 / FP32_VECTOR_TFLOPS,
           "compulsory_bytes": nbytes, "hbm_GBps": nbytes / (med / 1e3) / 1e9,
           "hbm_frac": nbytes / (med / 1e3) / 1e9 / HBM_PEAK_GBPS,
           "workspace_bytes": ws.numel(),
           "prologue": {"what": "kda_prologue_backward: gradients of the raw q, k, v, the conv "
                                "weights and the ring history from those of q^, k^, v^",
                        "ms": pmed, "ms_min": pms[0], "ms_max": pms[-1],
                        "compulsory_bytes": pbytes,
                        "hbm_GBps": pbytes / (pmed / 1e3) / 1e9,
                        "hbm_frac": pbytes / (pmed / 1e3) / 1e9 / HBM_PEAK_GBPS},
           "training_backward_ms": med + pmed,
           "training_backward_tokens_per_s": B * T / ((med + pmed) / 1e3)}
    del ws, out, pws, pout, qh, kh, vh, g, beta, S0, dO, dST, q, k, v
    torch.cuda.empty_cache()
    if not args.no_backward_layer:
        # about 150 GB of inputs and outputs plus the 24 GiB workspace: run it
        # only where the device has the room, and never lose the line to it
        free, _ = torch.cuda.mem_get_info(dev)
        need = 16 * 32768 * 96 * (128 * 2 * 2 + 128 * 2 + 128 * 4 + 4) * 2 + (24 << 30)
        if free < need + (8 << 30):
            res["layer_16x32768"] = {"skipped": f"needs about {need >> 30} GiB of device memory, "
                                                f"{free >> 30} GiB free"}
        else:
            try:
                res["layer_16x32768"] = backward_layer_bench(kda, workloads, torch, dev, args)
            except torch.cuda.OutOfMemoryError as e:
                torch.cuda.empty_cache()
                res["layer_16x32768"] = {"skipped": f"out of device memory: {e}"[:300]}
    return res


def backward_layer_bench(kda, workloads, torch, dev, args):
    """The backward of one training layer of the stack's shape (16 sequences
    of 32768 tokens, 96 heads of 128 x 128, bf16 I/O), whose one-pass
    workspace (451 GB) exceeds the device: the call takes its chunks in
    ranges within a 24 GiB workspace. Inputs drawn on the device
    (workloads.draw_layer_activations); one warm-up call, then the median of
    event-bracketed calls."""
    B, T, H, dk, dv = 16, 32768, 96, 128, 128
    ws_bytes = 24 << 30
    dims = kda.make_dims(B, H, dk, dv, torch.bfloat16)
    ins = workloads.draw_layer_activations(B, T, H, dk, dv, dev, seed=1500)
    out = [torch.empty(B, T, H, dk, dtype=torch.bfloat16, device=dev),
           torch.empty(B, T, H, dk, dtype=torch.bfloat16, device=dev),
           torch.empty(B, T, H, dv, dtype=torch.bfloat16, device=dev),
           torch.empty(B, T, H, dk, device=dev), torch.empty(B, T, H, device=dev),
           torch.empty(B, H, dk, dv, device=dev)]
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def call():
        kda.kda_chunk_backward(dims, T, *ins, *out, chunk=64, workspace=ws)

    call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.backward_layer_reps)]
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    med = ms[len(ms) // 2]
    assert all(torch.isfinite(t.float()).all().item() for t in out)
    nc = -(-T // 64)
    full = kda.kda_backward_workspace_bytes(dims, T, 64)
    per_chunk, state = full // nc, B * H * dk * dv * 4
    L = next(n for n in range(min(nc - 1, ws_bytes // per_chunk), 0, -1)
             if n * per_chunk + (-(-nc // n)) * state <= ws_bytes)
    flops = backward_flops(B, T, H, dk, dv, 64)
    res = {"workload": "chunked backward of one layer of the training step: 16 sequences x "
                       "32768 tokens, 96 heads of 128x128, chunk 64, bf16 I/O",
           "workspace_bytes": ws_bytes, "one_pass_workspace_bytes": full,
           "min_workspace_bytes": kda.kda_backward_workspace_min_bytes(dims, T, 64),
           "chunks_per_range": L, "ranges": -(-nc // L),
           "ms": med, "ms_min": ms[0], "ms_max": ms[-1], "calls": len(ms),
           "tokens_per_s": B * T / (med / 1e3),
           "tflops": flops / (med / 1e3) / 1e12}
    del ins, out, ws
    torch.cuda.empty_cache()
    return res


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=16)
    p.add_argument("--prefill-reps", type=int, default=20)
    p.add_argument("--prefill-warmup", type=int, default=100,
                   help="untimed prefill calls before the timed ones")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--calib-copy", action="store_true",
                   help="(kept for old command lines; the copy ceiling is always measured)")
    p.add_argument("--no-stack", action="store_true",
                   help="skip the 69-layer stack measurements")
    p.add_argument("--stack-reps", type=int, default=20)
    p.add_argument("--no-backward", action="store_true",
                   help="skip the chunked backward measurement")
    p.add_argument("--backward-reps", type=int, default=10)
    p.add_argument("--backward-warmup", type=int, default=5)
    p.add_argument("--no-backward-layer", action="store_true",
                   help="skip the backward of the 16 x 32768-token layer (ranges in 24 GiB)")
    p.add_argument("--backward-layer-reps", type=int, default=3)
    p.add_argument("--no-gdn", action="store_true",
                   help="skip the flag variants (KDA_F_SCALAR_G, KDA_F_RAW_GATES)")
    p.add_argument("--record-traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"),
                   help="(no GPU) write the committed counter records from two rocprofv3 "
                        "counter CSVs of this benchmark, and the command that made them")
    return p.parse_args()


def back_to_back_ms(torch, call, n):
    """Average duration of n calls issued back to back between one pair of
    events (steady-state throughput: no event between the calls)."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def variant_bench(kda, workloads, torch, dev, args, decode_name, prefill_name, flags, what,
                  **overrides):
    """A flag variant on the two workloads of the headline: 64 sequences x 96
    heads x 128x128 bf16 decode (same step count and warm-up as the headline)
    and the 4096-token chunk-64 prefill (median of event-bracketed calls after
    the warm-up calls)."""
    scalar_g = bool(flags & kda.KDA_F_SCALAR_G)
    inp = workloads.make(decode_name, **overrides)
    B, T, H, dk, dv = inp.dims
    stg = {name: getattr(inp, name).transpose(0, 1).contiguous().to(dev)
           for name in ("q", "k", "v", "g", "beta")}
    conv_w = inp.conv_w.to(dev)
    st = kda.KDAState(B, H, dk, dv, io=torch.bfloat16, device=dev)
    st.S.copy_(inp.S0.to(dev))
    st.ring.copy_(inp.ring0.to(dev))
    o = torch.empty(B, H, dv, dtype=torch.bfloat16, device=dev)

    def step(i):
        j = i % T
        st.decode_step(stg["q"][j], stg["k"][j], stg["v"][j], stg["g"][j], stg["beta"][j],
                       conv_w, o, flags=flags)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record()
    torch.cuda.synchronize()
    per_launch = ev0.elapsed_time(ev1) / 1e3 / args.steps
    assert torch.isfinite(st.S).all().item() and torch.isfinite(o.float()).all().item()
    dbytes = decode_bytes(B, H, dk, dv, scalar_g=scalar_g)
    st.close()
    del stg, st

    pin = workloads.make(prefill_name, **overrides)
    pB, pT, pH, pdk, pdv = pin.dims
    pd = {name: getattr(pin, name).contiguous().to(dev) for name in ("q", "k", "v", "g", "beta")}
    pw = pin.conv_w.to(dev)
    pst = kda.KDAState(pB, pH, pdk, pdv, io=torch.bfloat16, device=dev)
    pst.reset()
    po = torch.empty(pB, pT, pH, pdv, dtype=torch.bfloat16, device=dev)

    def prefill():
        pst.prefill(pT, pd["q"], pd["k"], pd["v"], pd["g"], pd["beta"], pw, po, chunk=64,
                    flags=flags)

    for _ in range(args.prefill_warmup):
        prefill()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.prefill_reps)]
    for e0, e1 in evs:
        e0.record()
        prefill()
        e1.record()
    torch.cuda.synchronize()
    calls_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    pre_ms = calls_ms[len(calls_ms) // 2]
    b2b_ms = back_to_back_ms(torch, prefill, args.prefill_reps)
    assert torch.isfinite(pst.S).all().item()
    pbytes = prefill_bytes(pB, pT, pH, pdk, pdv, scalar_g=scalar_g)
    pst.close()
    return {
        "workload": what,
        "decode": {"tokens_per_s": B / per_launch, "avg_launch_us": per_launch * 1e6,
                   "bytes_per_launch": dbytes, "hbm_GBps": dbytes / per_launch / 1e9,
                   "hbm_frac": dbytes / per_launch / 1e9 / HBM_PEAK_GBPS},
        "prefill": {"tokens_per_s": pT * pB / (pre_ms / 1e3), "ms": pre_ms,
                    "ms_min": calls_ms[0], "ms_max": calls_ms[-1], "calls": len(calls_ms),
                    "ms_back_to_back": b2b_ms,
                    "tokens_per_s_back_to_back": pT * pB / (b2b_ms / 1e3),
                    "compulsory_bytes": pbytes,
                    "hbm_GBps": pbytes / (pre_ms / 1e3) / 1e9,
                    "hbm_frac": pbytes / (pre_ms / 1e3) / 1e9 / HBM_PEAK_GBPS},
    }


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the KDA state of every (sequence, head) is "
              "independent, so more GPUs would each run this same kernel on their own "
              "share; this benchmark runs on one GPU only.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_83_amd as kda
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------- decode: 64 sequences x 96 heads, bf16 I/O -------------
    inp = workloads.make("batched_decode")
    B, T, H, dk, dv = inp.dims
    stg = {name: getattr(inp, name).transpose(0, 1).contiguous().to(dev)
           for name in ("q", "k", "v", "g", "beta")}           # [T, B, ...] per step
    conv_w = inp.conv_w.to(dev)
    st = kda.KDAState(B, H, dk, dv, io=torch.bfloat16, device=dev)
    st.S.copy_(inp.S0.to(dev))
    st.ring.copy_(inp.ring0.to(dev))
    o = torch.empty(B, H, dv, dtype=torch.bfloat16, device=dev)

    def step(i):
        j = i % T
        st.decode_step(stg["q"][j], stg["k"][j], stg["v"][j], stg["g"][j], stg["beta"][j],
                       conv_w, o)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    dec_ms = ev0.elapsed_time(ev1)                   # HIP events on the launch stream
    per_launch_s = dec_ms / 1e3 / args.steps         # one kernel launch per step
    tok_s = B * args.steps / (dec_ms / 1e3)
    dbytes = decode_bytes(B, H, dk, dv)
    achieved = dbytes / per_launch_s / 1e9
    assert torch.isfinite(st.S).all().item() and torch.isfinite(o.float()).all().item()

    # the same steps with the output gate fused into the readout (continuing
    # from the state the timed steps left)
    gz, gw, geps = workloads.draw_output_gate(B, T, H, dv, "bf16", seed=2)
    gz = gz.transpose(0, 1).contiguous().to(dev)
    gw = gw.to(dev)

    def gated_step(i):
        j = i % T
        st.decode_step_gated(stg["q"][j], stg["k"][j], stg["v"][j], stg["g"][j],
                             stg["beta"][j], conv_w, gz[j], gw, geps, o)

    for i in range(args.warmup):
        gated_step(i)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(args.steps):
        gated_step(args.warmup + i)
    ev1.record()
    torch.cuda.synchronize()
    gated_launch_s = ev0.elapsed_time(ev1) / 1e3 / args.steps
    gated_bytes = dbytes + B * H * dv * 2 + dv * 4     # + the gate inputs and weights
    assert torch.isfinite(o.float()).all().item()
    del gz

    # ---------------- prefill: T=4096, 96 heads, chunk 64, bf16 ------------
    pin = workloads.make("prefill_4k")
    pB, pT, pH, pdk, pdv = pin.dims
    pd = {name: getattr(pin, name).contiguous().to(dev)
          for name in ("q", "k", "v", "g", "beta")}
    pw = pin.conv_w.to(dev)
    pst = kda.KDAState(pB, pH, pdk, pdv, io=torch.bfloat16, device=dev)
    pst.reset()
    po = torch.empty(pB, pT, pH, pdv, dtype=torch.bfloat16, device=dev)

    def prefill():
        pst.prefill(pT, pd["q"], pd["k"], pd["v"], pd["g"], pd["beta"], pw, po, chunk=64)

    # the first calls, each bracketed by events (the first one allocates the
    # handle's workspace), then warm-up calls (the prefill kernels take 60-80
    # calls, about 25 ms of sustained load, to settle: the first calls run up
    # to 25 % longer), then calls bracketed one by one by events on the
    # launch stream (back to back, no host synchronization between them); the
    # median call is reported
    first_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(10)]
    for e0, e1 in first_evs:
        e0.record()
        prefill()
        e1.record()
    torch.cuda.synchronize()
    first_ms = [e0.elapsed_time(e1) for e0, e1 in first_evs]
    for _ in range(args.prefill_warmup):
        prefill()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.prefill_reps)]
    for e0, e1 in evs:
        e0.record()
        prefill()
        e1.record()
    torch.cuda.synchronize()
    calls_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    pre_ms = calls_ms[len(calls_ms) // 2]
    b2b_ms = back_to_back_ms(torch, prefill, args.prefill_reps)
    pbytes = prefill_bytes(pB, pT, pH, pdk, pdv)
    pflops = prefill_flops(pB, pT, pH, pdk, pdv, 64)
    pflops_built = prefill_flops_as_built(pB, pT, pH, pdk, pdv, 64)
    assert torch.isfinite(pst.S).all().item()

    # the output gate as its own kernel on the prefill's output (one read of
    # o and of the gate, one write; out of place so every call sees the same
    # input)
    pz, pwn, peps = workloads.draw_output_gate(pB, pT, pH, pdv, "bf16", seed=3)
    pz, pwn = pz.to(dev), pwn.to(dev)
    py = torch.empty_like(po)
    for _ in range(10):
        pst.gated_rmsnorm(pT, po, pz, pwn, peps, py)
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        pst.gated_rmsnorm(pT, po, pz, pwn, peps, py)
        e1.record()
    torch.cuda.synchronize()
    gate_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    gate_med = gate_ms[len(gate_ms) // 2]
    gate_bytes = 3 * pB * pT * pH * pdv * 2 + pdv * 4
    assert torch.isfinite(py.float()).all().item()
    del pz, py

    stack = None if args.no_stack else stack_bench(kda, workloads, torch, dev, args)
    gdn = None if args.no_gdn else variant_bench(
        kda, workloads, torch, dev, args, "batched_decode_gdn", "prefill_4k_gdn",
        kda.KDA_F_SCALAR_G, "KDA_F_SCALAR_G (one decay per token and head): the decode and "
        "prefill workloads above with g [B,T,H]")
    raw = None if args.no_gdn else variant_bench(
        kda, workloads, torch, dev, args, "batched_decode", "prefill_4k", kda.KDA_F_RAW_GATES,
        "KDA_F_RAW_GATES (the decay and beta formed in the kernels from raw projections): the "
        "decode and prefill workloads above drawn as pre-activations", raw_gates=True)

    bwd = None if args.no_backward else backward_bench(kda, workloads, torch, dev, args)
    dtraffic = measured_traffic(TRAFFIC_FILE, DECODE_SOURCES)
    ptraffic = measured_traffic(PREFILL_TRAFFIC_FILE, PREFILL_SOURCES)

    # ---------------- one K3-shape decode step: latency, warm and flushed ---
    single = single_step_latency(kda, workloads, torch, dev)

    # ---------------- practical HBM ceiling of a state stream --------------
    # a non-temporal in-place read-modify-write (the decode's access pattern,
    # kda_stream_rmw) over the headline's state size (384 MiB) and the
    # stack's (6 GiB), and a plain torch device copy of 1 GiB beside it
    stream_gbps = {}
    for label, nbytes in (("384MiB", 384 << 20), ("6GiB", 6 << 30)):
        buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        kda.kda_stream_rmw(buf, 1.0)
        torch.cuda.synchronize()
        best = 0.0
        for _ in range(3):
            ev0.record()
            for _ in range(5):
                kda.kda_stream_rmw(buf, 1.0)
            ev1.record()
            torch.cuda.synchronize()
            best = max(best, 2 * nbytes * 5 / (ev0.elapsed_time(ev1) / 1e3) / 1e9)
        stream_gbps[label] = best
        del buf
    torch.cuda.empty_cache()
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(5):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * n * 5 / (ev0.elapsed_time(ev1) / 1e3) / 1e9
    del src, dst

    # ---------------- CPU baseline: the fp64 oracle on a bounded sample -----
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import kda_oracle

        def run_oracle(nsteps):
            # steps cycle through the staged ones, as on the GPU; the state and
            # the ring carry over from one pass to the next
            t0 = time.perf_counter()
            S, ring, done = inp.S0, inp.ring0, 0
            while done < nsteps:
                m = min(T, nsteps - done)
                sl = slice(0, m)
                _, S, ring = kda_oracle.forward(inp.q[:, sl], inp.k[:, sl], inp.v[:, sl],
                                                inp.g[:, sl], inp.beta[:, sl], inp.conv_w, S,
                                                ring)
                done += m
            return time.perf_counter() - t0

        n, tn = 4, run_oracle(4)
        while tn < 0.5 * args.cpu_seconds and n < 16 * T:
            n = int(min(16 * T, max(n + 1, n * args.cpu_seconds / max(tn, 1e-3))))
            tn = run_oracle(n)
        cpu = {"value": B * n / tn, "unit": "tokens/s", "cores": kda_oracle.max_threads(),
               "kind": "oracle",
               "sample": f"fp64 sequential oracle, {n} decode steps cycling through the {T} "
                         f"staged ones, for all {B} sequences x {H} heads ({tn:.1f} s); "
                         f"includes the conversion of the inputs to float64"}
        # the same oracle on one core (a short sample of the same workload)
        n1 = 2
        t1 = time.perf_counter()
        kda_oracle.forward(inp.q[:, :n1], inp.k[:, :n1], inp.v[:, :n1], inp.g[:, :n1],
                           inp.beta[:, :n1], inp.conv_w, inp.S0, inp.ring0, threads=1)
        t1 = time.perf_counter() - t1
        cpu["one_core"] = {"value": B * n1 / t1, "unit": "tokens/s", "cores": 1,
                           "sample": f"first {n1} decode steps, {B} sequences x {H} heads "
                                     f"({t1:.1f} s)"}
        # the gradient oracle (sequential fp64, one thread) on one head of the
        # 4096-token workload, scaled to its 96 heads
        bq = workloads.make("prefill_4k", s0_random=True)
        qb, kb, vb = kda_oracle.prologue(bq.q, bq.k, bq.v, bq.conv_w, bq.ring0)[:3]
        dOb, dSTb = workloads.draw_backward_grads(1, pT, pH, pdk, pdv, io="bf16", seed=3)
        tb = time.perf_counter()
        kda_oracle.default().core_backward(qb[:, :, :1], kb[:, :, :1], vb[:, :, :1],
                                           bq.g[:, :, :1], bq.beta[:, :, :1], bq.S0[:, :1],
                                           dOb[:, :, :1], dSTb[:, :1])
        tb = time.perf_counter() - tb
        cpu["backward"] = {"value": pT / (tb * pH), "unit": "tokens/s", "cores": 1,
                           "sample": f"gradient of the recurrence for head 0 of the "
                                     f"4096-token workload ({tb:.1f} s), scaled to 96 heads"}
        del bq, qb, kb, vb, dOb, dSTb
        # and on the 4096-token prefill workload, all of it
        tp0 = time.perf_counter()
        kda_oracle.forward(pin.q, pin.k, pin.v, pin.g, pin.beta, pin.conv_w, pin.S0, pin.ring0)
        tp0 = time.perf_counter() - tp0
        cpu["prefill"] = {"value": pT * pB / tp0, "unit": "tokens/s",
                          "cores": kda_oracle.max_threads(),
                          "sample": f"the whole 4096-token prefill workload, 96 heads, "
                                    f"sequentially per head ({tp0:.1f} s)"}

    line = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; shapes of the K3 KDA layer)",
        "config": {"workload": "batched KDA decode: 64 sequences x 96 heads x 128x128 fp32 "
                               "state, bf16 q/k/v/o, one token per sequence per step "
                               "(inputs of 256 consecutive steps staged in HBM)",
                   "batch": B, "heads": H, "d_k": dk, "d_v": dv, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": dtraffic["traffic_bytes_per_launch"] if dtraffic else None,
                     "kernel": "decode_step_kernel<128,128,1024,bf16,nontemporal>",
                     "bytes_per_launch": dbytes, "avg_launch_us": per_launch_s * 1e6},
        "prefill": {"workload": "chunked prefill T=4096, batch 1, 96 heads, chunk 64, bf16",
                    "tokens_per_s": pT * pB / (pre_ms / 1e3), "ms": pre_ms,
                    "ms_min": calls_ms[0], "ms_max": calls_ms[-1], "calls": len(calls_ms),
                    "ms_back_to_back": b2b_ms,
                    "tokens_per_s_back_to_back": pT * pB / (b2b_ms / 1e3),
                    "hbm_GBps": pbytes / (pre_ms / 1e3) / 1e9,
                    "hbm_frac": pbytes / (pre_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
                    "ms_first_call": first_ms[0], "ms_first_10_calls": first_ms,
                    "tflops": pflops / (pre_ms / 1e3) / 1e12,
                    "mfma_frac": pflops / (pre_ms / 1e3) / 1e12 / BF16_DENSE_TFLOPS,
                    "compulsory_bytes": pbytes, "flops": pflops,
                    "flops_per_token_head": pflops // (pB * pT * pH),
                    "flops_as_built": pflops_built,
                    "mfma_frac_as_built": pflops_built / (pre_ms / 1e3) / 1e12 / BF16_DENSE_TFLOPS,
                    "traffic": ptraffic["traffic_bytes_per_call"] if ptraffic else None,
                    "traffic_per_kernel": ptraffic["per_kernel"] if ptraffic else None},
        "stack": stack,
        "backward": bwd,
        "scalar_decay": gdn,
        "raw_gates": raw,
        "output_gate": {
            "workload": "gated RMSNorm of each head's readout (sigmoid gate, shared weight, "
                        "eps 1e-5): fused into the decode step (64 sequences, same steps), "
                        "and as its own kernel on the 4096-token prefill output",
            "decode_tokens_per_s": B / gated_launch_s,
            "decode_avg_launch_us": gated_launch_s * 1e6,
            "decode_hbm_frac": gated_bytes / gated_launch_s / 1e9 / HBM_PEAK_GBPS,
            "epilogue_kernel": "gated_rmsnorm_kernel<128,bf16>",
            "epilogue_us": gate_med * 1e3, "epilogue_us_min": gate_ms[0] * 1e3,
            "epilogue_bytes": gate_bytes,
            "epilogue_GBps": gate_bytes / (gate_med / 1e3) / 1e9,
            "epilogue_hbm_frac": gate_bytes / (gate_med / 1e3) / 1e9 / HBM_PEAK_GBPS,
            "prefill_with_gate_tokens_per_s": pT * pB / ((pre_ms + gate_med) / 1e3),
        },
        "decode_flops_per_step": decode_flops(B, H, dk, dv),
        "wall_s_timed_region": wall,
        "cpu_baseline": cpu,
    }
    line["stream_ceiling"] = {
        "what": "kda_stream_rmw: non-temporal in-place read-modify-write, 16-byte accesses "
                "(the state stream's pattern), best of 3 x 5 calls, on the headline's state "
                "size and the stack's; torch copy_ of 1 GiB beside it",
        "GBps_384MiB": stream_gbps["384MiB"], "GBps_6GiB": stream_gbps["6GiB"],
        "frac_of_peak_384MiB": stream_gbps["384MiB"] / HBM_PEAK_GBPS,
        "torch_copy_GBps": copy_gbps}
    line["roofline"]["frac_of_stream_ceiling"] = achieved / stream_gbps["384MiB"]
    if stack is not None:
        stack["decode_frac_of_stream_ceiling"] = stack["decode_GBps"] / stream_gbps["6GiB"]
    line["single_step"] = single
    print(json.dumps(line))


if __name__ == "__main__":
    main()
