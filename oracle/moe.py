"""Plain float64 CPU definition of the Mixtral sparse-MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY. This module is the correctness oracle for the HIP
library. Only the tests, the package's ``smoke()`` check and the benchmark's
CPU-baseline leg may import it; the product path never does. It shares no code
with the GPU path (the seeded input generator in ``gen`` is the only common
module, and it holds none of the layer's arithmetic).

What the layer computes (sources are the five pages on Mixtral):

* Router: one logit per expert from a bias-free linear map of the token's
  hidden state (nnterp Mixtral page, "The API / support()": router_logits is
  the output of the router's F.linear; Transformers Mixtral page, MixtralConfig
  num_local_experts / num_experts_per_tok).
* Scoring: a softmax over the experts in float32, keep the top k (k = 2),
  divide the kept probabilities by their sum so each token's weights add to
  one; slot 0 holds the larger weight (nnterp page, Notes, "The router
  renormalizes its top 2, in float32").
* Dispatch: each token is sent to k experts ("dispatched twice (top 2
  routing)", Transformers page, "Architectural details").
* Experts: SwiGLU, down_proj(act(gate_proj x) * up_proj x) with act = SiLU
  (nnterp page, support() rows mlp_activation / mlp_neurons; MixtralConfig
  hidden_act = "silu"). Here w1 = gate, w3 = up, w2 = down.
* Combine: each slot's expert output is scaled by its weight and the slots
  are summed; there is no shared expert, so this sum is the layer output
  (nnterp page, Notes: "expert_outputs ... sums over its slot axis to
  routed_output" and "mlp_output is routed_output").

Readings where the pages leave a step open (all listed with the design notes):

* Top-k is taken on the logits. Softmax is strictly increasing, so this picks
  the same experts as top-k on probabilities; exactly equal logits go to the
  lower expert index.
* An optional per-expert logit bias is added before the softmax (used only by
  the load-imbalanced workload; the model itself has none).
* The gate weight is applied in the combine step; the per-expert outputs ``y``
  kept between steps are unweighted.
* Assignment ``a = t*k + j`` is token t's slot j. The grouping of assignments
  by expert is a stable counting sort: experts in increasing order and,
  within an expert, assignments in increasing order.

Inputs are the generator's arrays: float32, or bfloat16 bit patterns as
uint16, which are widened exactly to float64 here. Nothing is rounded to a
lower precision anywhere in this module.
"""
from __future__ import annotations

import numpy as np

NEAR_TIE_GAP = 1e-5


# --------------------------------------------------------------------------
# input decoding
# --------------------------------------------------------------------------
def widen(a) -> np.ndarray:
    """float32 -> float64, or bfloat16 bits (uint16/int16) -> float64, exactly."""
    a = np.asarray(a)
    if a.dtype in (np.uint16, np.int16):
        bits = a.view(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# --------------------------------------------------------------------------
# routing: logits -> softmax -> top-k -> renormalise
# --------------------------------------------------------------------------
def router_logits(x, router, bias=None) -> np.ndarray:
    """l[t, e] = sum_i x[t, i] * router[e, i] (+ bias[e]).

    nnterp Mixtral page, support(): router_logits [batch seq num_experts] is
    the output of the router's F.linear; the logit bias is this build's
    optional addition for the skewed workload.
    """
    logits = widen(x) @ widen(router).T
    if bias is not None:
        logits = logits + widen(bias)[None, :]
    return logits


def softmax(logits) -> np.ndarray:
    """Row softmax, max-subtracted (nnterp page, Notes: moe.SCORING is softmax)."""
    z = logits - logits.max(axis=-1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=-1, keepdims=True)


def select_topk(logits, k: int) -> np.ndarray:
    """Indices of the k largest logits per row, largest first.

    Repeated argmax over the experts not yet taken; numpy's argmax returns the
    first maximal position, so an exact tie goes to the lower expert index.
    (nnterp page, Notes: topk(moe.top_k) with slot 0 the larger weight.)
    """
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    idx = np.empty((T, k), dtype=np.int32)
    work = logits.copy()
    rows = np.arange(T)
    for j in range(k):
        sel = np.argmax(work, axis=1)
        idx[:, j] = sel
        work[rows, sel] = -np.inf
    return idx


def renormalise(probs, idx) -> np.ndarray:
    """w[t, j] = p[t, idx[t, j]] / sum_j' p[t, idx[t, j']] (nnterp page, Notes:
    the kept values divided by their sum; "there is no config flag for it")."""
    kept = np.take_along_axis(probs, idx.astype(np.int64), axis=1)
    return kept / kept.sum(axis=1, keepdims=True)


def route(x, router, k: int, bias=None):
    """Steps 1-4: returns (logits [T,E] f64, idx [T,k] int32, w [T,k] f64)."""
    logits = router_logits(x, router, bias)
    probs = softmax(logits)
    idx = select_topk(logits, k)
    w = renormalise(probs, idx)
    return logits, idx, w


def certify(logits, k: int, gap: float = NEAR_TIE_GAP):
    """Flag tokens whose routing a correctly rounded fp32 kernel may decide
    differently.

    Returns (near_tie [T] bool, order_tie [T] bool):
    near_tie  -- the gap between the k-th and (k+1)-th largest logit is below
                 ``gap``: the selected set itself is not certain;
    order_tie -- two of the k selected logits are closer than ``gap``: the set
                 is certain but the slot order is not.
    """
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    s = -np.sort(-logits, axis=1)
    near = np.zeros(T, bool)
    if k < E:
        near = (s[:, k - 1] - s[:, k]) < gap
    order = np.zeros(T, bool)
    for j in range(k - 1):
        order |= (s[:, j] - s[:, j + 1]) < gap
    return near, order


# --------------------------------------------------------------------------
# grouping of assignments by expert (counting sort)
# --------------------------------------------------------------------------
def permute(idx, E: int):
    """Stable counting sort of the assignments a = t*k + j by expert.

    Returns (counts [E], offsets [E+1], sorted_asg [A], asg_pos [A]) as int32:
    counts[e]   = number of assignments to expert e,
    offsets     = exclusive prefix sum of counts (offsets[E] = A),
    sorted_asg  = assignment ids grouped by expert, increasing within each,
    asg_pos[a]  = position of assignment a in sorted_asg.
    (Transformers page, "Architectural details": each token is dispatched to
    its k experts; nnterp page: the experts are one stacked module, so the
    rows each expert sees are gathered per expert.)
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    A = flat.size
    if A and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert index out of range")
    counts = np.zeros(E, dtype=np.int64)
    for e in range(E):
        counts[e] = int(np.count_nonzero(flat == e))
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E].copy()
    sorted_asg = np.empty(A, dtype=np.int64)
    asg_pos = np.empty(A, dtype=np.int64)
    for a in range(A):
        e = flat[a]
        p = cursor[e]
        sorted_asg[p] = a
        asg_pos[a] = p
        cursor[e] = p + 1
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_asg.astype(np.int32), asg_pos.astype(np.int32))


# --------------------------------------------------------------------------
# experts and combine
# --------------------------------------------------------------------------
def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)) (MixtralConfig hidden_act)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(rows, w1e, w3e, w2e):
    """One expert on a block of rows: w2 (silu(w1 x) * (w3 x)), row-wise.

    rows [M, d] f64; w1e, w3e [ffn, d] and w2e [d, ffn] (any encoding).
    nnterp page, support(): mlp_neurons = act(gate)*up is what the down
    projection receives.
    """
    g = rows @ widen(w1e).T
    u = rows @ widen(w3e).T
    h = silu(g) * u
    return h @ widen(w2e).T


def expert_ffn(x, w1, w3, w2, offsets, sorted_asg, k: int) -> np.ndarray:
    """y[p] = FFN_e(x[sorted_asg[p] // k]) for p in expert e's range.

    Output [A, d] f64, unweighted, in grouped (expert-major) order.
    """
    xd = widen(x)
    E = np.asarray(w1).shape[0]
    A = int(np.asarray(sorted_asg).size)
    y = np.zeros((A, xd.shape[1]), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        tokens = np.asarray(sorted_asg[lo:hi], dtype=np.int64) // k
        y[lo:hi] = swiglu(xd[tokens], w1[e], w3[e], w2[e])
    return y


def combine(y, asg_pos, w, k: int) -> np.ndarray:
    """out[t] = sum_j w[t, j] * y[asg_pos[t*k + j]], slots in order
    (nnterp page, Notes: expert_outputs are the weighted slot outputs and
    sum over the slot axis to routed_output)."""
    w = np.asarray(w, dtype=np.float64)
    T = w.shape[0]
    pos = np.asarray(asg_pos, dtype=np.int64).reshape(T, k)
    out = np.zeros((T, np.asarray(y).shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y[pos[:, j]]
    return out


def forward(x, router, w1, w3, w2, k: int, bias=None):
    """The whole layer. Returns a dict with every intermediate."""
    E = np.asarray(w1).shape[0]
    logits, idx, w = route(x, router, k, bias)
    counts, offsets, sorted_asg, asg_pos = permute(idx, E)
    y = expert_ffn(x, w1, w3, w2, offsets, sorted_asg, k)
    out = combine(y, asg_pos, w, k)
    return dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
                sorted_asg=sorted_asg, asg_pos=asg_pos, y=y, out=out)


# --------------------------------------------------------------------------
# the MLP half of the decoder block: pre-norm and residual around the layer
# --------------------------------------------------------------------------
def rms_norm(h, gamma, eps: float = 1e-5) -> np.ndarray:
    """n[t, i] = gamma[i] * h[t, i] / sqrt(mean_i h[t, i]^2 + eps).

    The MLP is called on post_attention_layernorm(h), a MixtralRMSNorm over
    hidden_size (nnterp Mixtral page, "The Notes", the block in order, and the
    module printout); eps is rms_norm_eps, 1e-5 (Transformers Mixtral page,
    MixtralConfig). The pages print no formula; this is root-mean-square
    normalisation over the hidden axis, scaled per channel by the norm's weight.
    """
    hd = widen(h)
    g = widen(gamma)
    ms = np.mean(hd * hd, axis=1, keepdims=True)
    return g[None, :] * (hd / np.sqrt(ms + eps))


def block_forward(h, gamma, router, w1, w3, w2, k: int, bias=None, eps: float = 1e-5):
    """out = h + layer(rms_norm(h)) (nnterp page, Notes: out = h +
    mlp(post_attention_layernorm(h)), and nothing norms the sublayer's output).
    Returns forward()'s dict for the normed rows, with ``norm`` = the normed
    rows, ``mlp`` = the layer's output and ``out`` = the block's."""
    n = rms_norm(h, gamma, eps)
    f = forward(n, router, w1, w3, w2, k, bias)
    f["norm"] = n
    f["mlp"] = f["out"]
    f["out"] = widen(h) + f["mlp"]
    return f


# --------------------------------------------------------------------------
# weight-only int8 expert weights
# --------------------------------------------------------------------------
def quantize_int8(w):
    """Per-output-row symmetric int8 codes of a weight [..., rows, cols].

    ZeroModels Mixtral page, "Lower memory": checkpoints may load weight-only
    quantized to int8 with bfloat16 activations. The pages give no scheme;
    the reading taken is one float32 scale per output row,
      scale = max_k |w[n, k]| / 127,  q[n, k] = round_half_even(w[n, k] / scale)
    (q = 0 for an all-zero row), clipped to [-127, 127]. The scale and the
    integer codes are decided in float32, as the quantizer on the device
    decides them (correctly rounded division), so the two agree exactly.
    Returns (q int8, scale float32 [..., rows]).
    """
    a = np.asarray(w)
    if a.dtype in (np.uint16, np.int16):  # bfloat16 bits -> float32, exactly
        wf = (a.view(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    else:
        wf = a.astype(np.float32)
    amax = np.abs(wf).max(axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(wf / scale[..., None])
    q = np.where(scale[..., None] > 0, q, 0.0)
    return np.clip(q, -127, 127).astype(np.int8), scale


def dequantize_int8(q, scale) -> np.ndarray:
    """The weights the int8 layer computes with: scale[n] * q[n, k], float64 (exact)."""
    return np.asarray(q, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[..., None]


# --------------------------------------------------------------------------
# second, independent formulations
# --------------------------------------------------------------------------
def gate_matrix(idx, w, E: int) -> np.ndarray:
    """m[t, e] = w[t, j] if idx[t, j] == e else 0."""
    T, k = np.asarray(idx).shape
    m = np.zeros((T, E), dtype=np.float64)
    for j in range(k):
        m[np.arange(T), np.asarray(idx)[:, j]] += np.asarray(w, dtype=np.float64)[:, j]
    return m


def dense_masked(x, router, w1, w3, w2, k: int, bias=None, idx=None, w=None):
    """Every expert on every token, masked by the renormalised gates:
    out[t] = sum_e m[t, e] * FFN_e(x[t]). No grouping, no gather."""
    xd = widen(x)
    E = np.asarray(w1).shape[0]
    if idx is None or w is None:
        _, idx, w = route(x, router, k, bias)
    m = gate_matrix(idx, w, E)
    out = np.zeros_like(xd)
    for e in range(E):
        out += m[:, e:e + 1] * swiglu(xd, w1[e], w3[e], w2[e])
    return out


def tokens_output(x, w1, w3, w2, idx, w, tokens) -> np.ndarray:
    """Layer output for a subset of tokens under a given routing (idx, w):
    out[t] = sum_j w[t, j] * FFN_{idx[t, j]}(x[t]) for t in ``tokens``.

    Experts are visited one at a time so only one expert's weights are held in
    float64 at once; used to check sampled rows of full-size workloads.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    idx = np.asarray(idx)[tokens]
    w = np.asarray(w, dtype=np.float64)[tokens]
    xs = widen(np.asarray(x)[tokens])
    out = np.zeros_like(xs)
    E = np.asarray(w1).shape[0]
    for e in range(E):
        sel_t, sel_j = np.nonzero(idx == e)
        if sel_t.size == 0:
            continue
        ye = swiglu(xs[sel_t], w1[e], w3[e], w2[e])
        for r in range(sel_t.size):
            out[sel_t[r]] += w[sel_t[r], sel_j[r]] * ye[r]
    return out


def renormalised_weights_for(logits, idx) -> np.ndarray:
    """Oracle weights (float64) for an externally chosen routing ``idx``."""
    return renormalise(softmax(np.asarray(logits, dtype=np.float64)), np.asarray(idx))
