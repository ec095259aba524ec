"""GPU parity on a seeded sweep of random layer shapes, through the fused
entry point: hidden and expert widths (multiples of 64 up to 1536), 2 to 32
experts, k from 1 to 4, optional logit bias (skewed routing), and batch sizes
on both sides of the kernel-family switches (few rows per expert: streaming
kernels; many: 128-row and 256x256-row tile kernels, the latter with either
XCD mapping and with or without a K split of the down projection). Each case
runs standard-layout and fragment-order weights (bit-identical) and int8
weights, against the float64 oracle on every token, or on a sample of tokens
for the larger batches."""
import numpy as np
import pytest
import torch

import gen
import oracle
from parity import OUT_TOL, check_routing, expected_output, host, rel_err, to_device

pytestmark = pytest.mark.gpu

N_CASES = 16


def _case(i):
    """Shape of sweep case i (deterministic)."""
    rng = np.random.default_rng(9000 + i)
    E = int(rng.choice([2, 4, 8, 8, 16, 32]))
    k = int(rng.choice([1, 2, 2, min(4, E)]))
    d = 64 * int(rng.integers(1, 25))
    ffn = 64 * int(rng.integers(1, 21))
    regime = i % 3      # 0: few rows per expert, 1: middle, 2: many
    if regime == 2 and i % 6 != 5:  # widths the 256x256-tile kernels take (down: d % 256)
        d = 256 * int(rng.integers(1, 9))
        ffn = 128 * int(rng.integers(1, 17))
    per_expert = [int(rng.integers(1, 32)), int(rng.integers(40, 500)),
                  int(rng.integers(520, 1400))][regime]
    T = max(1, per_expert * E // k)
    bias = None
    if rng.random() < 0.3:
        bias = [float(b) for b in rng.normal(0.0, 1.5, E)]
    return dict(T=T, d=d, ffn=ffn, E=E, k=k, dtype=gen.BF16, seed=9100 + i, bias=bias)


@pytest.fixture(scope="module")
def m():
    import sparse_mixture_experts_06_amd as lib
    yield lib


def _dequantized(inp):
    return {n: oracle.dequantize_int8(*oracle.quantize_int8(inp[n])) for n in ("w1", "w3", "w2")}


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep(m, i):
    cfg = _case(i)
    print(f"[sweep] case {i}: {cfg}", flush=True)
    inp = gen.make_inputs(**cfg)
    dev = to_device(inp)
    T, E, k = inp["T"], inp["E"], inp["k"]
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    out = m.moe_forward(dev["x"], dev["router"], dev["w1"], dev["w3"], dev["w2"], k,
                        logit_bias=dev["bias"], out_dtype=torch.float32, topk_idx_out=idx,
                        topk_w_out=w)
    pw = m.PackedWeights(dev["w1"], dev["w3"], dev["w2"])
    out_p = m.moe_forward(dev["x"], dev["router"], pw.w1, pw.w3, pw.w2, k,
                          logit_bias=dev["bias"], out_dtype=torch.float32, packed=True)
    qw = m.QuantizedWeights(dev["w1"], dev["w3"], dev["w2"])
    out_q = m.moe_forward(dev["x"], dev["router"], qw.w1, qw.w3, qw.w2, k,
                          logit_bias=dev["bias"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out)

    logits64 = oracle.router_logits(inp["x"], inp["router"], inp["bias"])
    idx_g = host(idx)
    check_routing(logits64, k, idx_g, host(w))
    if T <= 2048:
        tokens = np.arange(T)
    else:
        rng = np.random.default_rng(9200 + i)
        tokens = np.unique(np.concatenate([rng.choice(T, size=256, replace=False), [0, T - 1]]))
    ref = expected_output(inp, idx_g, None, tokens, logits64)
    err = rel_err(host(out)[tokens], ref)
    deq = _dequantized(inp)
    ref_q = expected_output(dict(inp, **deq), idx_g, None, tokens, logits64)
    err_q = rel_err(host(out_q)[tokens], ref_q)
    print(f"[sweep] case {i}: A={T * k} max|err|/rms bf16 {err:.2e} int8 {err_q:.2e}", flush=True)
    assert err <= OUT_TOL[gen.BF16]
    assert err_q <= OUT_TOL[gen.BF16]
