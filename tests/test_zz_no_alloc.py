"""moe_forward_noalloc (the entry point for callers that cannot allocate)
against moe_forward on the same inputs: two calls in a row, the second on a
smaller batch (the scratch keeps the first call's contents), bit-identical
outputs and routing, and both within the bf16 / fp32 bar of the oracle; sizes
beyond the built-in scratch are refused before anything runs."""
import numpy as np
import pytest
import torch

import gen
import oracle
from parity import OUT_TOL, host, rel_err, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import sparse_mixture_experts_06_amd as lib
    yield lib


def _both(m, inp, dev, packed=False, pw=None, variant=0):
    T, E, k = inp["T"], inp["E"], inp["k"]
    w1, w3, w2 = (pw.w1, pw.w3, pw.w2) if packed else (dev["w1"], dev["w3"], dev["w2"])
    res = {}
    for name, fn in (("ws", m.moe_forward), ("noalloc", m.moe_forward_noalloc)):
        idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
        w = torch.full((T, k), -1.0, dtype=torch.float32, device="cuda")
        counts = torch.full((E,), -1, dtype=torch.int32, device="cuda")
        out = fn(dev["x"], dev["router"], w1, w3, w2, k, logit_bias=dev["bias"],
                 out_dtype=torch.float32, topk_idx_out=idx, topk_w_out=w, counts_out=counts,
                 packed=packed, variant=variant)
        res[name] = (out, idx, w, counts)
    torch.cuda.synchronize()
    return res


def _check(inp, res):
    a, b = res["ws"], res["noalloc"]
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    T, k = inp["T"], inp["k"]
    logits64 = oracle.router_logits(inp["x"], inp["router"], inp["bias"])
    idx_ref = oracle.select_topk(logits64, k)
    near, _ = oracle.certify(logits64, k)
    idx_use = idx_ref.copy()
    idx_use[near] = host(b[1])[near]
    w_use = oracle.renormalised_weights_for(logits64, idx_use)
    ref = oracle.tokens_output(inp["x"], inp["w1"], inp["w3"], inp["w2"], idx_use, w_use,
                               np.arange(T))
    err = rel_err(host(b[0]), ref)
    print(f"[noalloc] T={T} d={inp['d']} ffn={inp['ffn']} {inp['dtype']}: max|err|/rms {err:.2e}",
          flush=True)
    assert err <= OUT_TOL[inp["dtype"]]


@pytest.mark.parametrize("cfgs", [
    # tiled kernels (400 assignments), then a smaller batch on the streaming ones
    [dict(T=200, d=512, ffn=1024, E=8, k=2, dtype=gen.BF16, seed=301),
     dict(T=33, d=512, ffn=1024, E=8, k=2, dtype=gen.BF16, seed=302)],
    # float32 path, a ragged shape, then fewer tokens
    [dict(T=150, d=70, ffn=50, E=8, k=2, dtype=gen.F32, seed=303),
     dict(T=7, d=70, ffn=50, E=8, k=2, dtype=gen.F32, seed=304)],
    # the 256x256-tile kernels with a skewed routing, then a decode-size batch
    [dict(T=1200, d=256, ffn=256, E=8, k=2, dtype=gen.BF16, seed=305,
          bias=[3, 1, 0, 0, 0, 0, -1, -2]),
     dict(T=32, d=256, ffn=256, E=8, k=2, dtype=gen.BF16, seed=306)],
])
def test_noalloc_matches_forward_twice(m, cfgs):
    for cfg in cfgs:
        print(f"[noalloc] case {cfg}", flush=True)
        inp = gen.make_inputs(**cfg)
        dev = to_device(inp)
        _check(inp, _both(m, inp, dev))
        if inp["dtype"] == gen.BF16:
            pw = m.PackedWeights(dev["w1"], dev["w3"], dev["w2"])
            _check(inp, _both(m, inp, dev, packed=True, pw=pw, variant=1))


def test_noalloc_decode_8x7b_shape(m):
    """The Mixtral-8x7B decode shape (the batch size this entry point is for),
    fragment-order weights, then a smaller batch on the same weights."""
    inp = gen.make_config("decode_8x7b")
    dev = to_device(inp)
    pw = m.PackedWeights(dev["w1"], dev["w3"], dev["w2"])
    for T in (32, 8):
        sub = dict(inp, T=T, x=inp["x"][:T])
        sdev = dict(dev, x=dev["x"][:T])
        print(f"[noalloc] decode_8x7b T={T}", flush=True)
        res = _both(m, sub, sdev, packed=True, pw=pw)
        a, b = res["ws"], res["noalloc"]
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_noalloc_refuses_sizes_beyond_the_scratch(m):
    T, d, ffn, E, k = 600, 4096, 14336, 8, 2
    assert m.moe_workspace_bytes(T, d, ffn, E, k, torch.bfloat16) > m.MOE_NOALLOC_SCRATCH_BYTES
    assert m.moe_workspace_bytes(545, d, ffn, E, k, torch.bfloat16) <= m.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(T, d, dtype=torch.bfloat16, device="cuda")
    r = torch.zeros(E, d, dtype=torch.float32, device="cuda")
    w1 = torch.zeros(E, ffn, d, dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros(E, d, ffn, dtype=torch.bfloat16, device="cuda")
    out = torch.full((T, d), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MoeError) as err:
        m.moe_forward_noalloc(x, r, w1, w1, w2, k, out=out)
    assert err.value.status == m.MOE_EWORKSPACE
    torch.cuda.synchronize()
    assert (out == 3.0).all()   # nothing ran
