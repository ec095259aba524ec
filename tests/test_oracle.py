"""Pins for the CPU oracle: each test checks it against something other than
itself -- brute force, closed forms, library routines, invariants the pages
assert, and a hand-derived worked example. No GPU is used."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import gen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def tiny():
    return gen.make_config("tiny")


def _fwd(inp):
    return oracle.forward(inp["x"], inp["router"], inp["w1"], inp["w3"], inp["w2"], inp["k"],
                          inp["bias"])


# ----------------------------------------------------------------- inputs --
def test_generator_is_deterministic_and_scaled(tiny):
    again = gen.make_config("tiny")
    for name in ("x", "router", "w1", "w3", "w2"):
        assert np.array_equal(tiny[name], again[name])
    other = gen.make_config("tiny", seed=7)
    assert not np.array_equal(tiny["w1"], other["w1"])
    d, ffn = tiny["d"], tiny["ffn"]
    assert abs(tiny["w1"].std() * math.sqrt(d) - 1) < 0.05
    assert abs(tiny["w2"].std() * math.sqrt(ffn) - 1) < 0.05
    assert abs(tiny["x"].std() - 1) < 0.05


def test_bf16_encoding_round_trip():
    # bit patterns fixed by the bfloat16 format: sign, 8 exponent bits, 7 mantissa bits
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x4049], np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0, 3.140625]
    assert oracle.widen(bits).tolist() == want
    # round to nearest even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1 (even)
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -2.0 - 2.0 ** -6],
                    np.float32)
    got = oracle.widen(gen.f32_to_bf16_bits(vals)).tolist()
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> 1 + 2^-6;
    # -2 - 2^-6 is exactly representable (step 2^-6 above 2)
    assert got == [1.0, 1.0 + 2.0 ** -6, 1.0, -2.0 - 2.0 ** -6]


def test_page_shapes_match_workloads():
    with open(os.path.join(GOLDEN, "mixtral_shapes.json")) as f:
        g = json.load(f)
    a, b = g["mixtral_8x7b"], g["mixtral_8x22b"]
    for name in ("decode_8x7b", "prefill_8x7b", "skew_8x7b"):
        c = gen.CONFIGS[name]
        assert (c["d"], c["ffn"], c["E"], c["k"]) == (
            a["hidden_size"], a["intermediate_size"], a["num_local_experts"],
            a["num_experts_per_tok"])
    c = gen.CONFIGS["prefill_8x22b"]
    assert c["d"] == b["num_attention_heads"] * b["head_dim"]
    assert c["ffn"] == b["intermediate_size"]
    # expert parameters of 8x7B from these sizes: 32 layers x 8 experts x 3 matrices
    experts = a["num_hidden_layers"] * a["num_local_experts"] * 3 * a["hidden_size"] * \
        a["intermediate_size"]
    assert round(experts / 1e9) == g["total_parameters_billion_printed"]


# ---------------------------------------------------------------- routing --
def test_logits_brute_force(tiny):
    bias = np.array([0.5, -1.0, 0, 0, 2.0, 0, 0, -0.25], np.float32)
    logits = oracle.router_logits(tiny["x"], tiny["router"], bias)
    for t in (0, 5, 63):
        for e in range(tiny["E"]):
            s = math.fsum(float(tiny["x"][t, i]) * float(tiny["router"][e, i])
                          for i in range(tiny["d"])) + float(bias[e])
            assert abs(logits[t, e] - s) <= 1e-12 * max(1.0, abs(s))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topk_pairs_brute_force(seed):
    inp = gen.make_config("tiny", seed=seed)
    logits, idx, w = oracle.route(inp["x"], inp["router"], 2)
    probs = scipy.special.softmax(logits, axis=1)
    for t in range(logits.shape[0]):
        best = max(itertools.combinations(range(8), 2), key=lambda p: probs[t, p[0]] + probs[t, p[1]])
        assert set(idx[t].tolist()) == set(best)
        assert probs[t, idx[t, 0]] >= probs[t, idx[t, 1]]


def test_topk_subsets_brute_force_k3():
    inp = gen.make_inputs(T=40, d=64, ffn=64, E=6, k=3, dtype=gen.F32, seed=11)
    logits, idx, _ = oracle.route(inp["x"], inp["router"], 3)
    for t in range(40):
        best = max(itertools.combinations(range(6), 3), key=lambda s: sum(logits[t, list(s)]))
        assert set(idx[t].tolist()) == set(best)
        assert list(idx[t]) == sorted(idx[t], key=lambda e: -logits[t, e])


def test_exact_ties_go_to_lower_index():
    inp = gen.make_inputs(T=16, d=32, ffn=64, E=8, k=2, dtype=gen.F32, seed=3)
    r = inp["router"].copy()
    r[5] = r[2]  # experts 2 and 5 give bit-identical logits
    bias = np.zeros(8, np.float32)
    bias[[2, 5]] = 100.0  # and are the top two for every token
    _, idx, w = oracle.route(inp["x"], r, 2, bias)
    assert (idx[:, 0] == 2).all() and (idx[:, 1] == 5).all()
    assert np.all(w == 0.5)
    r2 = inp["router"].copy()
    r2[3] = r2[1]
    r2[6] = r2[1]
    b2 = np.zeros(8, np.float32)
    b2[[1, 3, 6]] = 100.0  # three-way tie: the two lowest indices win
    _, idx2, _ = oracle.route(inp["x"], r2, 2, b2)
    assert (idx2[:, 0] == 1).all() and (idx2[:, 1] == 3).all()


def test_weights_closed_form(tiny):
    logits, idx, w = oracle.route(tiny["x"], tiny["router"], 2)
    for t in range(logits.shape[0]):
        la, lb = logits[t, idx[t, 0]], logits[t, idx[t, 1]]
        w0 = 1.0 / (1.0 + math.exp(lb - la))  # the softmax denominator cancels
        assert abs(w[t, 0] - w0) < 1e-14
        assert abs(w[t, 1] - (1.0 - w0)) < 1e-14
        assert w[t, 0] >= w[t, 1]
    assert np.all(np.abs(w.sum(1) - 1.0) < 1e-14)


def test_k1_and_k_equals_E(tiny):
    logits, idx1, w1 = oracle.route(tiny["x"], tiny["router"], 1)
    assert np.all(w1 == 1.0)
    assert np.array_equal(idx1[:, 0], np.argmax(logits, axis=1))
    _, idxE, wE = oracle.route(tiny["x"], tiny["router"], 8)
    sm = scipy.special.softmax(logits, axis=1)
    assert np.allclose(wE, np.take_along_axis(sm, idxE.astype(np.int64), 1), rtol=0, atol=1e-15)
    assert np.array_equal(idxE, np.argsort(-logits, axis=1, kind="stable"))


def test_certify_flags_only_close_gaps():
    logits = np.array([[3.0, 2.0, 2.0 - 5e-6, 0.0],     # 2nd/3rd gap below 1e-5
                       [3.0, 2.0, 1.0, 0.0],            # clear
                       [3.0, 3.0 - 2e-6, 1.0, 0.0]])    # slot order uncertain only
    near, order = oracle.certify(logits, 2)
    assert near.tolist() == [True, False, False]
    assert order.tolist() == [False, False, True]


# ------------------------------------------------------------ permutation --
@pytest.mark.parametrize("T,E,k,seed", [(64, 8, 2, 0), (257, 8, 2, 1), (100, 16, 4, 2),
                                        (33, 5, 1, 3)])
def test_permute_against_library(T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, sorted_asg, asg_pos = oracle.permute(idx, E)
    flat = idx.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert counts.sum() == k * T
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(sorted_asg, np.argsort(flat, kind="stable"))
    assert np.array_equal(asg_pos[sorted_asg], np.arange(T * k))


def test_permute_degenerate():
    c, o, s, p = oracle.permute(np.zeros((0, 2), np.int32), 8)
    assert c.tolist() == [0] * 8 and o.tolist() == [0] * 9 and s.size == 0 and p.size == 0
    idx = np.tile(np.array([[3, 6]], np.int32), (5, 1))  # everyone on experts 3 and 6
    c, o, s, p = oracle.permute(idx, 8)
    assert c.tolist() == [0, 0, 0, 5, 0, 0, 5, 0]
    assert s.tolist() == [0, 2, 4, 6, 8, 1, 3, 5, 7, 9]
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 8]], np.int32), 8)


# ------------------------------------------------------- experts, combine --
def test_silu_values():
    z = np.array([0.0, 1.0, -1.0, 40.0, -800.0])
    got = oracle.silu(z)
    assert got[0] == 0.0
    assert abs(got[1] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(got[2] + 1.0 / (1.0 + math.e)) < 1e-16
    assert abs(got[3] - 40.0) < 1e-12 and got[4] == 0.0
    assert np.allclose(got, F.silu(torch.tensor(z)).numpy(), rtol=1e-15, atol=0)


def test_dense_masked_agrees(tiny):
    ref = _fwd(tiny)
    dense = oracle.dense_masked(tiny["x"], tiny["router"], tiny["w1"], tiny["w3"], tiny["w2"], 2)
    scale = np.sqrt(np.mean(ref["out"] ** 2))
    assert np.max(np.abs(ref["out"] - dense)) <= 1e-12 * scale


def test_dense_masked_agrees_bf16_with_bias():
    inp = gen.make_inputs(T=48, d=64, ffn=192, E=8, k=2, dtype=gen.BF16, seed=5,
                          bias=[3, 1, 0, 0, 0, 0, -1, -2])
    ref = _fwd(inp)
    dense = oracle.dense_masked(inp["x"], inp["router"], inp["w1"], inp["w3"], inp["w2"], 2,
                                inp["bias"])
    scale = np.sqrt(np.mean(ref["out"] ** 2))
    assert np.max(np.abs(ref["out"] - dense)) <= 1e-12 * scale
    sub = oracle.tokens_output(inp["x"], inp["w1"], inp["w3"], inp["w2"], ref["idx"], ref["w"],
                               [0, 7, 47])
    assert np.max(np.abs(sub - ref["out"][[0, 7, 47]])) <= 1e-12 * scale


def _torch_slots(inp, idx, w):
    """Per-slot weighted expert outputs with torch's own linear/silu (float64)."""
    x = torch.tensor(oracle.widen(inp["x"]))
    w1 = torch.tensor(oracle.widen(inp["w1"]))
    w3 = torch.tensor(oracle.widen(inp["w3"]))
    w2 = torch.tensor(oracle.widen(inp["w2"]))
    T, k = idx.shape
    slots = torch.zeros(T, k, x.shape[1], dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            hid = F.silu(F.linear(x[t], w1[e])) * F.linear(x[t], w3[e])
            slots[t, j] = float(w[t, j]) * F.linear(hid, w2[e])
    return slots.numpy()


def test_slot_sum_identity_with_library_ops(tiny):
    ref = _fwd(tiny)
    slots = _torch_slots(tiny, ref["idx"], ref["w"])
    scale = np.sqrt(np.mean(ref["out"] ** 2))
    assert np.max(np.abs(slots.sum(1) - ref["out"])) <= 1e-12 * scale


def test_identical_experts_reduce_to_one_swiglu(tiny):
    inp = dict(tiny)
    for name in ("w1", "w3", "w2"):
        inp[name] = np.repeat(tiny[name][:1], 8, axis=0)
    ref = _fwd(inp)
    x = torch.tensor(tiny["x"], dtype=torch.float64)
    mlp = F.linear(F.silu(F.linear(x, torch.tensor(tiny["w1"][0], dtype=torch.float64))) *
                   F.linear(x, torch.tensor(tiny["w3"][0], dtype=torch.float64)),
                   torch.tensor(tiny["w2"][0], dtype=torch.float64)).numpy()
    assert np.max(np.abs(ref["out"] - mlp)) <= 1e-12 * np.sqrt(np.mean(mlp ** 2))


def test_single_expert_is_textbook_swiglu():
    inp = gen.make_inputs(T=10, d=32, ffn=96, E=1, k=1, dtype=gen.F32, seed=9)
    ref = _fwd(inp)
    x = torch.tensor(inp["x"], dtype=torch.float64)
    mlp = F.linear(F.silu(F.linear(x, torch.tensor(inp["w1"][0], dtype=torch.float64))) *
                   F.linear(x, torch.tensor(inp["w3"][0], dtype=torch.float64)),
                   torch.tensor(inp["w2"][0], dtype=torch.float64)).numpy()
    assert np.all(ref["w"] == 1.0)
    assert np.max(np.abs(ref["out"] - mlp)) <= 1e-12 * np.sqrt(np.mean(mlp ** 2))


def test_convex_combination_bound(tiny):
    ref = _fwd(tiny)
    T = ref["out"].shape[0]
    pos = ref["asg_pos"].reshape(T, 2)
    ya, yb = ref["y"][pos[:, 0]], ref["y"][pos[:, 1]]
    lo, hi = np.minimum(ya, yb), np.maximum(ya, yb)
    eps = 1e-12 * np.abs(ref["out"]).max()
    assert np.all(ref["out"] >= lo - eps) and np.all(ref["out"] <= hi + eps)


@pytest.mark.parametrize("e", range(8))
def test_ablation_changes_exactly_the_tokens_that_chose_e(tiny, e):
    ref = _fwd(tiny)
    w_abl = np.where(ref["idx"] == e, 0.0, ref["w"])
    abl = oracle.combine(ref["y"], ref["asg_pos"], w_abl, 2)
    changed = (abl != ref["out"]).any(1)
    assert np.array_equal(changed, (ref["idx"] == e).any(1))


def test_worked_example_closed_form():
    """Hand-derived two-token example (d=2, ffn=3, E=4, k=2).

    Token 0 = [1, 0] has logits [2, 0, 1, -1] -> experts (0, 2), weights
    sigmoid(1), sigmoid(-1). Token 1 = [0, 1] has logits [0.5, 1.5, -2, 1]
    -> experts (1, 3), weights sigmoid(0.5), sigmoid(-0.5).
    With w1[e] = c_e [[1,0],[0,1],[1,1]], w3[e] = [[1,0],[0,2],[0,0]] and
    w2[e] = [[a,p,0],[b,q,0]]_e, expert e maps token 0 to silu(c_e) [a_e, b_e]
    and token 1 to 2 silu(c_e) [p_e, q_e].
    """
    def f32(v):  # the layer's inputs are float32: use the values they hold
        return [float(np.float32(u)) for u in v]

    c = f32([1.0, -0.5, 2.0, 0.25])
    a, b = f32([1.0, 2.0, 3.0, 4.0]), f32([-1.0, 0.5, 2.0, -3.0])
    p, q = f32([0.3, -1.2, 0.7, 2.5]), f32([1.1, 0.9, -0.4, 0.6])
    x = np.array([[1.0, 0.0], [0.0, 1.0]], np.float32)
    router = np.array([[2.0, 0.5], [0.0, 1.5], [1.0, -2.0], [-1.0, 1.0]], np.float32)
    w1 = np.stack([ce * np.array([[1, 0], [0, 1], [1, 1]], np.float32) for ce in c])
    w3 = np.stack([np.array([[1, 0], [0, 2], [0, 0]], np.float32)] * 4)
    w2 = np.stack([np.array([[a[e], p[e], 0], [b[e], q[e], 0]], np.float32) for e in range(4)])
    ref = oracle.forward(x, router, w1, w3, w2, 2)

    def sig(z):
        return 1.0 / (1.0 + math.exp(-z))

    def sl(z):
        return z * sig(z)

    want0 = [sig(1) * sl(c[0]) * a[0] + sig(-1) * sl(c[2]) * a[2],
             sig(1) * sl(c[0]) * b[0] + sig(-1) * sl(c[2]) * b[2]]
    want1 = [sig(0.5) * 2 * sl(c[1]) * p[1] + sig(-0.5) * 2 * sl(c[3]) * p[3],
             sig(0.5) * 2 * sl(c[1]) * q[1] + sig(-0.5) * 2 * sl(c[3]) * q[3]]
    assert ref["idx"].tolist() == [[0, 2], [1, 3]]
    assert np.allclose(ref["w"], [[sig(1), sig(-1)], [sig(0.5), sig(-0.5)]], rtol=0, atol=1e-15)
    assert ref["counts"].tolist() == [1, 1, 1, 1]
    assert ref["sorted_asg"].tolist() == [0, 2, 1, 3]
    assert np.allclose(ref["out"], [want0, want1], rtol=1e-14, atol=1e-15)


def test_skew_bias_concentrates_routing():
    inp = gen.make_inputs(T=2000, d=128, ffn=64, E=8, k=2, dtype=gen.F32, seed=4,
                          bias=gen.CONFIGS["skew_8x7b"]["bias"])
    _, idx, _ = oracle.route(inp["x"], inp["router"], 2, inp["bias"])
    counts, *_ = oracle.permute(idx, 8)
    frac0 = counts[0] / counts.sum()
    # at most one slot per token can be expert 0, so its share is at most 1/k
    assert 0.45 < frac0 <= 0.5
    assert counts[0] > counts[1] > counts[2] and counts[7] == counts.min()


# ------------------------------------------------- pre-norm and residual --
def test_rms_norm_worked_example():
    # row 0: mean square (9 + 16) / 2 = 25/2, rms 5/sqrt(2): [3, 4] -> [3, 4] * sqrt(2)/5,
    #        times gamma [1, 2] -> [3 sqrt(2)/5, 8 sqrt(2)/5]
    # row 1: mean square 1/4, rms 1/2: [1/2, -1/2] -> [1, -1], times gamma -> [1, -2]
    h = np.array([[3.0, 4.0], [0.5, -0.5]])
    g = np.array([1.0, 2.0])
    got = oracle.rms_norm(h, g, eps=0.0)
    r2 = math.sqrt(2.0)
    want = np.array([[3 * r2 / 5, 8 * r2 / 5], [1.0, -2.0]])
    assert np.allclose(got, want, rtol=1e-15, atol=0)
    # eps sits under the square root: a row of ones becomes 1 / sqrt(1 + eps)
    got = oracle.rms_norm(np.ones((1, 4)), np.ones(4), eps=1e-5)
    assert np.allclose(got, 1.0 / math.sqrt(1.0 + 1e-5), rtol=1e-15, atol=0)


def test_rms_norm_matches_library_routine():
    rng = np.random.default_rng(5)
    h = rng.standard_normal((7, 96)) * rng.uniform(0.1, 10.0, size=(7, 1))
    g = rng.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(h), (96,), torch.from_numpy(g), eps=1e-5).numpy()
    assert np.allclose(oracle.rms_norm(h, g, 1e-5), ref, rtol=1e-13, atol=1e-13)


def test_rms_norm_invariants():
    rng = np.random.default_rng(6)
    h = rng.standard_normal((5, 64))
    ones = np.ones(64)
    base = oracle.rms_norm(h, ones, eps=0.0)
    assert np.allclose(oracle.rms_norm(7.25 * h, ones, eps=0.0), base, rtol=1e-14, atol=0)
    assert np.array_equal(oracle.rms_norm(-h, ones, eps=0.0), -base)
    assert np.allclose(np.mean(base ** 2, axis=1), 1.0, rtol=1e-14, atol=0)


def test_block_is_residual_plus_layer_on_normed_rows(tiny):
    rng = np.random.default_rng(8)
    gamma = rng.uniform(0.5, 1.5, tiny["d"])
    b = oracle.block_forward(tiny["x"], gamma, tiny["router"], tiny["w1"], tiny["w3"], tiny["w2"],
                             tiny["k"], tiny["bias"])
    assert np.allclose(b["norm"], oracle.rms_norm(tiny["x"], gamma), rtol=1e-15, atol=0)
    # experts with a zero down projection add nothing: the block returns its input
    z = oracle.block_forward(tiny["x"], gamma, tiny["router"], tiny["w1"], tiny["w3"],
                             np.zeros_like(tiny["w2"]), tiny["k"], tiny["bias"])
    assert np.array_equal(z["out"], oracle.widen(tiny["x"]))
    # routing is decided on the normed rows: a per-token rescale of h changes nothing
    scaled = oracle.widen(tiny["x"]) * rng.uniform(0.5, 4.0, size=(tiny["T"], 1))
    s = oracle.block_forward(scaled, gamma, tiny["router"], tiny["w1"], tiny["w3"], tiny["w2"],
                             tiny["k"], tiny["bias"], eps=0.0)
    b0 = oracle.block_forward(tiny["x"], gamma, tiny["router"], tiny["w1"], tiny["w3"],
                              tiny["w2"], tiny["k"], tiny["bias"], eps=0.0)
    assert np.array_equal(s["idx"], b0["idx"])
    assert np.allclose(s["mlp"], b0["mlp"], rtol=1e-9, atol=1e-12)


# ------------------------------------------------------ int8 expert weights --
def test_quantize_int8_worked_example():
    # row 0: max |w| = 127 -> scale 1 exactly; -63.5 and 0.5 are halfway cases and go to even
    # row 1: max |w| = 127/4 -> scale 1/4; w / scale = [4, -2, 127, 1] exactly
    # row 2: all zero -> scale 0 and codes 0
    w = np.array([[[127.0, -63.5, 0.5, 1.0], [1.0, -0.5, 31.75, 0.25], [0.0, 0.0, 0.0, 0.0]]],
                 np.float32)
    q, s = oracle.quantize_int8(w)
    assert s.tolist() == [[1.0, 0.25, 0.0]]
    assert q.tolist() == [[[127, -64, 0, 1], [4, -2, 127, 1], [0, 0, 0, 0]]]
    assert q.dtype == np.int8 and s.dtype == np.float32


def test_quantize_int8_error_bound_and_symmetry():
    rng = np.random.default_rng(11)
    w = gen.f32_to_bf16_bits(rng.standard_normal((3, 32, 96)).astype(np.float32) * 0.05)
    q, s = oracle.quantize_int8(w)
    wd = oracle.widen(w)
    err = np.abs(wd - oracle.dequantize_int8(q, s))
    # round to nearest: within half a step, plus the float32 rounding of w / scale
    # (|w / scale| <= 127, so at most 127 * 2^-24 < 2^-16 of a step)
    assert (err <= s[..., None] * (0.5 + 2.0 ** -16)).all()
    assert err.max() > 0.45 * s.max()  # and the bound is not vacuous
    # the largest magnitude of each row becomes +-127
    assert (np.abs(q).max(axis=-1) == 127).all()
    q2, s2 = oracle.quantize_int8(gen.f32_to_bf16_bits(-gen.bf16_bits_to_f32(w)))
    assert np.array_equal(s2, s) and np.array_equal(q2, -q)


def test_quantize_int8_matches_library_rounding():
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((2, 16, 64)) * 0.02).astype(np.float32)
    q, s = oracle.quantize_int8(w)
    wt = torch.from_numpy(w)
    st = wt.abs().amax(dim=-1) / torch.tensor(127.0, dtype=torch.float32)
    qt = torch.clamp(torch.round(wt / st[..., None]), -127, 127).to(torch.int8)
    assert np.array_equal(s, st.numpy())
    assert np.array_equal(q, qt.numpy())
