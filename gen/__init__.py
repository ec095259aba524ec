"""Seeded synthetic inputs for the Mixtral sparse-MoE layer.

This module is shared by the CPU oracle, the tests and the benchmark. It draws
random arrays and encodes them (float32 -> bfloat16 bit patterns); it holds
none of the layer's arithmetic (no router, softmax, top-k, permutation, SwiGLU
or combine).

Shapes and distributions follow the layer sizes printed for Mixtral-8x7B and
Mixtral-8x22B ("MixtralConfig" on the Transformers Mixtral page; the "Config"
table on the nnterp Mixtral encyclopedia page): hidden 4096 / 6144,
intermediate 14336 / 16384, 8 local experts, 2 experts per token. No trained
weights exist here, so weights are random with std 1/sqrt(fan_in) and the
hidden states are standard normal.

Random streams: ``np.random.SeedSequence(seed).spawn(2 + 3*E)`` gives one child
per tensor slice, in the order x, router, w1[0..E-1], w3[0..E-1], w2[0..E-1];
each child seeds a PCG64 generator that draws float32 standard normals, which
are scaled by a float32 std and, for bf16 inputs, rounded to nearest-even.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32 = "f32"
BF16 = "bf16"

# Named workloads. ``T`` tokens, hidden ``d``, expert width ``ffn``, ``E``
# experts, ``k`` experts per token. ``bias`` is a per-expert logit offset
# (only the load-imbalanced workload has one).
CONFIGS = {
    # fp32 throughout, small enough for the oracle to run in well under a second
    "tiny": dict(T=64, d=128, ffn=256, E=8, k=2, dtype=F32, seed=0, bias=None),
    # Mixtral-8x7B shape, decode batch of 32 tokens: weight streaming dominates
    "decode_8x7b": dict(T=32, d=4096, ffn=14336, E=8, k=2, dtype=BF16, seed=1, bias=None),
    # Mixtral-8x7B shape, prefill of 8 sequences x 512 tokens flattened to 4096
    "prefill_8x7b": dict(T=4096, d=4096, ffn=14336, E=8, k=2, dtype=BF16, seed=2, bias=None),
    # Mixtral-8x7B shape with a per-expert logit bias that skews the routing
    "skew_8x7b": dict(T=8192, d=4096, ffn=14336, E=8, k=2, dtype=BF16, seed=3,
                      bias=[3.0, 1.0, 0.0, 0.0, 0.0, 0.0, -1.0, -2.0]),
    # Mixtral-8x22B shape
    "prefill_8x22b": dict(T=2048, d=6144, ffn=16384, E=8, k=2, dtype=BF16, seed=4, bias=None),
    # Mixtral-8x7B widths with other routing settings (MixtralConfig num_experts_per_tok and
    # num_local_experts): one expert per token, and 16 or 32 experts with two per token,
    # each at a decode batch (32 tokens) and a prefill batch (4096 tokens). A decode
    # batch's x is the first 32 rows of the prefill batch's (same seed, same weights).
    "decode_8x7b_k1": dict(T=32, d=4096, ffn=14336, E=8, k=1, dtype=BF16, seed=5, bias=None),
    "prefill_8x7b_k1": dict(T=4096, d=4096, ffn=14336, E=8, k=1, dtype=BF16, seed=5, bias=None),
    "decode_e16": dict(T=32, d=4096, ffn=14336, E=16, k=2, dtype=BF16, seed=6, bias=None),
    "prefill_e16": dict(T=4096, d=4096, ffn=14336, E=16, k=2, dtype=BF16, seed=6, bias=None),
    "decode_e32": dict(T=32, d=4096, ffn=14336, E=32, k=2, dtype=BF16, seed=7, bias=None),
    "prefill_e32": dict(T=4096, d=4096, ffn=14336, E=32, k=2, dtype=BF16, seed=7, bias=None),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as ``uint16``. NaN payloads are not preserved
    (the generators never produce NaN).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (for host-side use)."""
    return (np.ascontiguousarray(b).view(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(child: np.random.SeedSequence, shape, std: float, dtype: str) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(child))
    a = np.empty(shape, dtype=np.float32)
    g.standard_normal(dtype=np.float32, out=a)
    if std != 1.0:
        a *= np.float32(std)
    if dtype == BF16:
        return f32_to_bf16_bits(a)
    return a


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(T: int, d: int, ffn: int, E: int = 8, k: int = 2, dtype: str = BF16,
                seed: int = 0, bias=None, router_std: float | None = None,
                x_std: float = 1.0, **_ignored) -> dict:
    """Draw one layer's inputs.

    Returns a dict with
      ``x``      [T, d]       float32, or uint16 bf16 bits when dtype == "bf16"
      ``router`` [E, d]       float32 (the router stays fp32 for every dtype)
      ``w1``     [E, ffn, d]  gate projection per expert (same encoding as x)
      ``w3``     [E, ffn, d]  up projection per expert
      ``w2``     [E, d, ffn]  down projection per expert
      ``bias``   [E] float32 or None
    plus the scalar sizes.
    """
    if dtype not in (F32, BF16):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    children = np.random.SeedSequence(seed).spawn(2 + 3 * E)
    r_std = (1.0 / np.sqrt(d)) if router_std is None else router_std
    w_in_std = 1.0 / np.sqrt(d)
    w_out_std = 1.0 / np.sqrt(ffn)
    enc = np.uint16 if dtype == BF16 else np.float32
    w1 = np.empty((E, ffn, d), enc)
    w3 = np.empty((E, ffn, d), enc)
    w2 = np.empty((E, d, ffn), enc)

    jobs = [("x", None, children[0], (T, d), x_std, dtype),
            ("router", None, children[1], (E, d), r_std, F32)]
    for e in range(E):
        jobs.append(("w1", e, children[2 + e], (ffn, d), w_in_std, dtype))
        jobs.append(("w3", e, children[2 + E + e], (ffn, d), w_in_std, dtype))
        jobs.append(("w2", e, children[2 + 2 * E + e], (d, ffn), w_out_std, dtype))
    out = {}
    dst = {"w1": w1, "w3": w3, "w2": w2}

    def run(job):
        name, e, child, shape, std, dt = job
        a = _draw(child, shape, std, dt)
        if e is None:
            out[name] = a
        else:
            dst[name][e] = a

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, jobs))
    b = None if bias is None else np.asarray(bias, dtype=np.float32).reshape(E)
    return dict(x=out["x"], router=out["router"], w1=w1, w3=w3, w2=w2, bias=b,
                T=T, d=d, ffn=ffn, E=E, k=k, dtype=dtype, seed=seed)


def make_norm_weight(d: int, seed: int = 0) -> np.ndarray:
    """Weight [d] float32 of the RMS norm in front of the layer: 1 + 0.1 * N(0, 1)
    (no trained norm weights exist here; a norm's weight starts at one). Drawn
    from its own stream, SeedSequence([seed, 1]), so the layer's inputs for
    the same seed do not change."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1])))
    a = np.empty(d, dtype=np.float32)
    g.standard_normal(dtype=np.float32, out=a)
    return np.float32(1.0) + np.float32(0.1) * a


def make_config(name: str, seed: int | None = None, T: int | None = None) -> dict:
    """Inputs of a named workload; ``seed``/``T`` override the defaults."""
    cfg = dict(CONFIGS[name])
    if seed is not None:
        cfg["seed"] = seed
    if T is not None:
        cfg["T"] = T
    return make_inputs(**cfg)
