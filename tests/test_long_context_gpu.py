"""The bf16 prefill's error against the fp64 oracle as the context grows.

The bf16 path rounds the state to bf16 for its products in every chunk, so
the error could in principle build up with the number of chunks. With the
workloads' decays (g = log sigmoid of a standard normal per token and
channel: most channels forget within tens of tokens) the state is held by
the recent tokens, and the error should level off rather than grow with T.
Checked at 8192, 32768 and 131072 tokens (two heads of 128 x 128, one
sequence, random S0 and ring), each in full against the oracle, with the
same bound as every bf16 parity test: max|err| / max|ref| <= 2e-2 on o and
on the final S.
("为什么 Kimi K3 敢把 KV Cache 扔掉？…", section 5: the chunked form; section 6:
the per-channel forgetting.)
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as kda
import workloads
from oracle import kda_oracle
from tests.gpu_util import device, f64, load_state, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [8192, 32768, 131072])
def test_bf16_prefill_error_with_context(T):
    dev = device()
    inp = workloads.make("tiny", T=T, B=1, H=2, dk=128, dv=128, io="bf16", s0_random=True,
                         ring_random=True, seed=1600 + T % 97)
    B, _, H, dk, dv = inp.dims
    d = to_dev(inp, dev)
    st = kda.KDAState(B, H, dk, dv, io=torch.bfloat16, device=dev)
    load_state(st, inp)
    o = torch.empty(B, T, H, dv, dtype=torch.bfloat16, device=dev)
    st.prefill(T, d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], o, chunk=64)
    torch.cuda.synchronize()
    ref_o, ref_S, ref_ring = kda_oracle.forward(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                                inp.conv_w, inp.S0, inp.ring0)
    got_o, got_S = f64(o), f64(st.S)
    eo, es = rel_err(got_o, ref_o), rel_err(got_S, ref_S)
    # the error over the last 4096 tokens alone, against that window's largest value
    tail = slice(T - 4096, T)
    et = rel_err(got_o[:, tail], ref_o[:, tail])
    print(f"bf16 prefill T={T}: rel err o={eo:.2e} (last 4096 tokens {et:.2e}) S={es:.2e}")
    assert np.isfinite(got_o).all() and np.isfinite(got_S).all()
    assert eo <= 2e-2 and es <= 2e-2 and et <= 2e-2
    np.testing.assert_array_equal(f64(st.ring), ref_ring)
