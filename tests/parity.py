"""Helpers shared by the GPU parity tests: upload the generator's arrays,
and compare the HIP results with the oracle's under the stated rules.

Rules (derived in the design notes):
* routing indices, counts, offsets and the permutation are compared exactly;
  a token whose oracle (float64) gap between its k-th and (k+1)-th logit is
  below 1e-5 is "certified" and its indices are not compared; a token whose
  selected logits are within 1e-5 of each other has its indices compared as
  a set. The permutation is always checked bit-exactly against the oracle
  run on the GPU's own indices.
* routing weights: |w_gpu - w_oracle| <= 1e-5.
* outputs: max|out_gpu - out_oracle| <= tol * rms(out_oracle) with
  tol = 1e-4 (float32 inputs) or 2e-2 (bfloat16 inputs); certified tokens
  are compared with the oracle output under the GPU's routing.
"""
from __future__ import annotations

import numpy as np
import torch

import gen
import oracle

W_TOL = 1e-5
OUT_TOL = {gen.F32: 1e-4, gen.BF16: 2e-2}


def to_device(inp: dict, device="cuda") -> dict:
    """Upload one input dict; bf16 bit patterns become torch.bfloat16 tensors."""
    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    out = {k: up(inp[k]) for k in ("x", "router", "w1", "w3", "w2", "bias")}
    return out


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return oracle.widen(t.view(torch.int16).cpu().numpy())
    return t.cpu().numpy()


def check_routing(logits64, k, idx_gpu, w_gpu):
    """Returns (certified mask, number of tokens compared as sets)."""
    idx_ref = oracle.select_topk(logits64, k)
    w_ref = oracle.renormalise(oracle.softmax(logits64), idx_ref)
    near, order = oracle.certify(logits64, k)
    idx_gpu = np.asarray(idx_gpu)
    w_gpu = np.asarray(w_gpu, dtype=np.float64)
    exact = ~near & ~order
    bad = np.nonzero(exact & (idx_gpu != idx_ref).any(1))[0]
    assert bad.size == 0, f"routing differs on tokens {bad[:10]}: gpu {idx_gpu[bad[:3]]} ref {idx_ref[bad[:3]]}"
    sets = ~near & order
    for t in np.nonzero(sets)[0]:
        assert sorted(idx_gpu[t]) == sorted(idx_ref[t]), t
    ok = exact
    err = np.abs(w_gpu[ok] - w_ref[ok]).max(initial=0.0)
    assert err <= W_TOL, f"routing weight error {err}"
    if sets.any():
        ws = np.sort(w_gpu[sets], axis=1)
        wr = np.sort(w_ref[sets], axis=1)
        assert np.abs(ws - wr).max() <= W_TOL
    # every token: distinct experts in range, weights positive and summing to one
    assert ((idx_gpu >= 0) & (idx_gpu < logits64.shape[1])).all()
    for j in range(1, k):
        assert (idx_gpu[:, j:] != idx_gpu[:, j - 1:j]).all()
    assert np.abs(w_gpu.sum(1) - 1.0).max() <= 4e-7 * k
    assert (np.diff(w_gpu, axis=1) <= 0).all()
    return near, int(sets.sum())


def check_permutation(idx_gpu, E, counts, offsets, sorted_asg, asg_pos):
    c, o, s, p = oracle.permute(np.asarray(idx_gpu), E)
    assert np.array_equal(np.asarray(counts), c)
    assert np.array_equal(np.asarray(offsets), o)
    assert np.array_equal(np.asarray(sorted_asg), s)
    assert np.array_equal(np.asarray(asg_pos), p)


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)) / rms)


def bf16_half_ulp(ref) -> np.ndarray:
    """Half a bfloat16 unit in the last place of each reference value."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def expected_output(inp, idx_gpu, w_gpu_unused, tokens, logits64):
    """Oracle output rows for ``tokens``: the oracle's routing, except on
    certified near-tie tokens, where the GPU's experts are used with weights
    the oracle computes for them."""
    k = inp["k"]
    idx_ref = oracle.select_topk(logits64, k)
    near, _ = oracle.certify(logits64, k)
    idx_use = idx_ref.copy()
    idx_use[near] = np.asarray(idx_gpu)[near]
    w_use = oracle.renormalised_weights_for(logits64, idx_use)
    return oracle.tokens_output(inp["x"], inp["w1"], inp["w3"], inp["w2"], idx_use, w_use, tokens)
