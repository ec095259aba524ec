"""ctypes binding for libmoe.so (C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. PyTorch supplies device memory (tensors) and the current HIP stream.
The functions keep the C names; outputs that are not passed in are allocated
with torch on the input's device. There is no fallback: if libmoe.so is
missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_EWORKSPACE, MOE_EHIP = 0, 1, 2, 3, 4
MOE_F32, MOE_BF16, MOE_BF16_PACKED, MOE_INT8_PACKED = 0, 1, 2, 3
MOE_MAX_EXPERTS = 32
MOE_MAX_ASSIGNMENTS = 2 ** 31 - 1024
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_sz = ctypes.c_size_t
_vp = ctypes.c_void_p


class MoeOptions(ctypes.Structure):
    """struct moe_options (include/moe.h): per-call kernel family, stage events
    and down-projection K split."""
    _fields_ = [("ffn_variant", ctypes.c_int), ("stage_events", ctypes.POINTER(ctypes.c_void_p)),
                ("down_split", ctypes.c_int)]


_opts_p = ctypes.POINTER(MoeOptions)

_SIGNATURES = {
    "moe_strerror": (ctypes.c_char_p, [_c_int]),
    "moe_workspace_bytes": (_c_sz, [_c_i64, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "moe_route": (_c_int, [_vp, _c_int, _vp, _vp, _c_i64, _c_int, _c_int, _c_int, _vp, _vp, _vp,
                           _vp]),
    "moe_permute": (_c_int, [_vp, _c_i64, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _c_sz, _vp]),
    "moe_check_routing": (_c_int, [_vp, _c_i64, _c_int, _c_int, _vp, _vp]),
    "moe_expert_ffn": (_c_int, [_vp, _c_int, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_int, _c_int,
                                _c_int, _c_int, _vp, _vp, _c_sz, _vp, _opts_p]),
    "moe_combine": (_c_int, [_vp, _vp, _vp, _c_i64, _c_int, _c_int, _vp, _c_int, _vp]),
    "moe_forward": (_c_int, [_vp, _c_int, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_int, _c_int,
                             _c_int, _c_int, _vp, _c_int, _vp, _vp, _vp, _vp, _c_sz, _vp,
                             _opts_p]),
    "moe_forward_noalloc": (_c_int, [_vp, _c_int, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_int,
                                     _c_int, _c_int, _c_int, _vp, _c_int, _vp, _vp, _vp, _vp,
                                     _opts_p]),
    "moe_block_forward": (_c_int, [_vp, _c_int, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _c_i64, _c_int, _c_int, _c_int, _c_int, _vp, _c_int,
                                   _vp, _vp, _vp, _vp, _c_sz, _vp, _opts_p]),
    "moe_pack_weight": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp]),
    "moe_quantized_weight_bytes": (_c_sz, [_c_int, _c_int, _c_int]),
    "moe_quantize_weight": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp]),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({strerror(status)})")


def load() -> ctypes.CDLL:
    """Load libmoe.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_mixture_experts_06_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions include/moe.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def strerror(status: int) -> str:
    return load().moe_strerror(int(status)).decode()


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return MOE_F32
    if t == torch.bfloat16:
        return MOE_BF16
    raise ValueError(f"unsupported dtype {t} (float32 or bfloat16)")


def _weight_code(t: torch.dtype, packed: bool, w1, w3, w2) -> int:
    """The dtype code of the expert weights: all three int8 matrices
    (QuantizedMatrix), or all three tensors of the activations' dtype
    (fragment order when packed). A mix is refused before any library call."""
    code = _dtype_code(t)
    quant = [isinstance(w, QuantizedMatrix) for w in (w1, w3, w2)]
    if any(quant) and not all(quant):
        raise ValueError("w1, w3 and w2 must all be int8 (QuantizedMatrix) or all tensors")
    if all(quant):
        if code != MOE_BF16:
            raise ValueError("int8 weights take bfloat16 activations")
        if packed:
            raise ValueError("int8 weights have their own layout (packed=False)")
        return MOE_INT8_PACKED
    if packed:
        if code != MOE_BF16:
            raise ValueError("packed weights are bfloat16 only")
        return MOE_BF16_PACKED
    return code


def _options(variant: int = 0, events=None, down_split: int = 0):
    """A moe_options for one call (None when everything is at its default).
    The returned object keeps the event array alive for the call."""
    if not variant and not events and not down_split:
        return None
    opts = MoeOptions()
    opts.ffn_variant = int(variant)
    opts.down_split = int(down_split)
    if events:
        if len(events) != 6:
            raise ValueError("stage events: a sequence of 6 hipEvent_t handles")
        arr = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(int(e)) for e in events])
        opts.stage_events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        opts._keep = arr
    return ctypes.pointer(opts)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, QuantizedMatrix):
        t = t.blob
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape, device, code=None):
    """Checks dtype, shape and device. An int8 QuantizedMatrix passes only where
    the weight code is MOE_INT8_PACKED, and then on shape and device alone."""
    if isinstance(t, QuantizedMatrix):
        if code != MOE_INT8_PACKED:
            raise ValueError(f"{name}: an int8 matrix where {dtype} weights are expected")
        dtype = t.dtype
    elif code == MOE_INT8_PACKED:
        raise ValueError(f"{name}: a tensor where int8 weights (QuantizedMatrix) are expected")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


# ---------------------------------------------------------------------------
def moe_pack_weight(w, out=None):
    """Fragment-order copy of bf16 weights w [E, rows, cols] (see moe.h)."""
    if w.dtype != torch.bfloat16 or w.dim() != 3:
        raise ValueError("moe_pack_weight takes a bfloat16 tensor [E, rows, cols]")
    E, rows, cols = w.shape
    if out is None:
        out = torch.empty_like(w)
    _need(out, "out", torch.bfloat16, (E, rows, cols), w.device)
    st = load().moe_pack_weight(_ptr(w), MOE_BF16, E, rows, cols, _ptr(out), _stream(w.device))
    _check("moe_pack_weight", st)
    return out


class QuantizedMatrix:
    """Weight-only int8 matrix made by moe_quantize_weight: the uint8 blob the
    library reads (codes in 16 x 64 blocks, then float32 row scales) and the
    logical shape (E, rows, cols) of the matrix it stands for."""

    dtype = "int8-blob"

    def __init__(self, blob, shape):
        self.blob = blob
        self.shape = tuple(int(v) for v in shape)
        self.device = blob.device

    def codes(self) -> torch.Tensor:
        """The int8 codes in standard [E, rows, cols] order (a copy)."""
        E, rows, cols = self.shape
        q = self.blob[:E * rows * cols].view(torch.int8)
        q = q.view(E, rows // 16, cols // 64, 4, 16, 2, 8)  # e, rt, s, g, r, half, i
        return q.permute(0, 1, 4, 2, 5, 3, 6).reshape(E, rows, cols).contiguous()

    def scales(self) -> torch.Tensor:
        """float32 [E, rows]."""
        E, rows, cols = self.shape
        off = (E * rows * cols + 255) // 256 * 256
        return self.blob[off:off + E * rows * 4].view(torch.float32).view(E, rows)


def moe_quantize_weight(w, out=None) -> QuantizedMatrix:
    """Weight-only int8 copy of bf16 weights w [E, rows, cols] (see moe.h)."""
    if w.dtype != torch.bfloat16 or w.dim() != 3:
        raise ValueError("moe_quantize_weight takes a bfloat16 tensor [E, rows, cols]")
    E, rows, cols = w.shape
    n = int(load().moe_quantized_weight_bytes(E, rows, cols))
    if n == 0:
        raise ValueError("moe_quantize_weight needs rows % 16 == 0 and cols % 64 == 0")
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=w.device)
    if out.dtype != torch.uint8 or out.numel() < n or out.device != w.device:
        raise ValueError(f"out: a uint8 tensor of at least {n} bytes on {w.device}")
    st = load().moe_quantize_weight(_ptr(w), MOE_BF16, E, rows, cols, _ptr(out),
                                    _stream(w.device))
    _check("moe_quantize_weight", st)
    return QuantizedMatrix(out, (E, rows, cols))


class QuantizedWeights:
    """w1, w3, w2 as weight-only int8 matrices (moe_quantize_weight), for
    moe_forward / moe_expert_ffn / moe_block_forward in place of the bf16
    tensors."""

    def __init__(self, w1, w3, w2):
        self.w1 = moe_quantize_weight(w1)
        self.w3 = moe_quantize_weight(w3)
        self.w2 = moe_quantize_weight(w2)


class PackedWeights:
    """w1, w3, w2 in fragment order (moe_pack_weight), for moe_forward /
    moe_expert_ffn with packed=True. Shapes are those of the originals."""

    def __init__(self, w1, w3, w2):
        self.w1 = moe_pack_weight(w1)
        self.w3 = moe_pack_weight(w3)
        self.w2 = moe_pack_weight(w2)


def moe_workspace_bytes(T: int, d: int, ffn: int, E: int, k: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(load().moe_workspace_bytes(int(T), int(d), int(ffn), int(E), int(k), code))


def workspace(T: int, d: int, ffn: int, E: int, k: int, dtype, device) -> torch.Tensor:
    n = moe_workspace_bytes(T, d, ffn, E, k, dtype)
    if n == 0:
        raise ValueError("invalid sizes for moe_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_route(x, router, k: int, logit_bias=None, logits_out=None, topk_idx=None, topk_w=None):
    """Returns (topk_idx [T,k] int32, topk_w [T,k] float32); logits_out, if
    given ([T,E] float32), receives the pre-softmax logits."""
    T, d = x.shape
    E = router.shape[0]
    dev = x.device
    _need(router, "router", torch.float32, (E, d), dev)
    if logit_bias is not None:
        _need(logit_bias, "logit_bias", torch.float32, (E,), dev)
    if logits_out is not None:
        _need(logits_out, "logits_out", torch.float32, (T, E), dev)
    if topk_idx is None:
        topk_idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty(T, k, dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    st = load().moe_route(_ptr(x), _dtype_code(x.dtype), _ptr(router), _ptr(logit_bias), T, d, E,
                          k, _ptr(logits_out), _ptr(topk_idx), _ptr(topk_w), _stream(dev))
    _check("moe_route", st)
    return topk_idx, topk_w


def moe_permute(topk_idx, E: int, counts=None, offsets=None, sorted_asg=None, asg_pos=None):
    """Returns (counts [E], offsets [E+1], sorted_asg [T*k], asg_pos [T*k]), int32."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    A = T * k
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    sorted_asg = torch.empty(A, dtype=torch.int32, device=dev) if sorted_asg is None else sorted_asg
    asg_pos = torch.empty(A, dtype=torch.int32, device=dev) if asg_pos is None else asg_pos
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(counts, "counts", torch.int32, (E,), dev)
    _need(offsets, "offsets", torch.int32, (E + 1,), dev)
    _need(sorted_asg, "sorted_asg", torch.int32, (A,), dev)
    _need(asg_pos, "asg_pos", torch.int32, (A,), dev)
    st = load().moe_permute(_ptr(topk_idx), T, E, k, _ptr(counts), _ptr(offsets),
                            _ptr(sorted_asg), _ptr(asg_pos), None, 0, _stream(dev))
    _check("moe_permute", st)
    return counts, offsets, sorted_asg, asg_pos


def moe_check_routing(topk_idx, E: int, bad=None):
    """Returns bad [2] int32 on the device: tokens with an expert id outside
    [0, E), tokens with a repeated id."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    bad = torch.empty(2, dtype=torch.int32, device=dev) if bad is None else bad
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(bad, "bad", torch.int32, (2,), dev)
    st = load().moe_check_routing(_ptr(topk_idx), T, E, k, _ptr(bad), _stream(dev))
    _check("moe_check_routing", st)
    return bad


def moe_expert_ffn(x, w1, w3, w2, offsets, sorted_asg, k: int, y=None, ws=None, packed=False,
                   variant: int = 0, down_split: int = 0):
    """Returns y [T*k, d] float32 (unweighted expert outputs, grouped order).
    packed=True: w1/w3/w2 come from moe_pack_weight. variant: the expert-FFN
    kernel family (0 = by size, 1 = streaming, 2 = tiled). down_split: the
    down projection's K split where the 256x256-tile kernel runs (0 = chosen
    on the device, -1 = none, 8..13 = first part of that many sixteenths)."""
    T, d = x.shape
    E, ffn, _ = w1.shape
    dev = x.device
    code = _weight_code(x.dtype, packed, w1, w3, w2)
    for name, t, shp in (("w1", w1, (E, ffn, d)), ("w3", w3, (E, ffn, d)), ("w2", w2, (E, d, ffn))):
        _need(t, name, x.dtype, shp, dev, code)
    _need(offsets, "offsets", torch.int32, (E + 1,), dev)
    _need(sorted_asg, "sorted_asg", torch.int32, (T * k,), dev)
    if y is None:
        y = torch.empty(T * k, d, dtype=torch.float32, device=dev)
    _need(y, "y", torch.float32, (T * k, d), dev)
    if ws is None:
        ws = workspace(T, d, ffn, E, k, code, dev)
    st = load().moe_expert_ffn(_ptr(x), code, _ptr(w1), _ptr(w3), _ptr(w2),
                               _ptr(offsets), _ptr(sorted_asg), T, d, ffn, E, k, _ptr(y),
                               _ptr(ws), ws.numel(), _stream(dev),
                               _options(variant, down_split=down_split))
    _check("moe_expert_ffn", st)
    return y


def moe_combine(y, asg_pos, topk_w, out=None, out_dtype=torch.float32):
    """Returns out [T, d] = sum_j topk_w[t, j] * y[asg_pos[t*k + j]]."""
    T, k = topk_w.shape
    d = y.shape[1]
    dev = y.device
    _need(y, "y", torch.float32, (T * k, d), dev)
    _need(asg_pos, "asg_pos", torch.int32, (T * k,), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    if out is None:
        out = torch.empty(T, d, dtype=out_dtype, device=dev)
    _need(out, "out", out.dtype, (T, d), dev)
    st = load().moe_combine(_ptr(y), _ptr(asg_pos), _ptr(topk_w), T, d, k, _ptr(out),
                            _dtype_code(out.dtype), _stream(dev))
    _check("moe_combine", st)
    return out


def moe_forward(x, router, w1, w3, w2, k: int, logit_bias=None, out=None, out_dtype=None,
                ws=None, topk_idx_out=None, topk_w_out=None, counts_out=None, packed=False,
                variant: int = 0, events=None, down_split: int = 0):
    """The whole layer; returns out [T, d] (dtype out_dtype, default x.dtype).
    packed=True: w1/w3/w2 come from moe_pack_weight. variant: the expert-FFN
    kernel family; events: 6 hipEvent_t handles recorded between the stages;
    down_split: as for moe_expert_ffn."""
    T, d = x.shape
    E, ffn, _ = w1.shape
    dev = x.device
    code = _weight_code(x.dtype, packed, w1, w3, w2)
    _need(router, "router", torch.float32, (E, d), dev)
    for name, t, shp in (("w1", w1, (E, ffn, d)), ("w3", w3, (E, ffn, d)), ("w2", w2, (E, d, ffn))):
        _need(t, name, x.dtype, shp, dev, code)
    if logit_bias is not None:
        _need(logit_bias, "logit_bias", torch.float32, (E,), dev)
    if out is None:
        out = torch.empty(T, d, dtype=out_dtype or x.dtype, device=dev)
    _need(out, "out", out.dtype, (T, d), dev)
    if topk_idx_out is not None:
        _need(topk_idx_out, "topk_idx_out", torch.int32, (T, k), dev)
    if topk_w_out is not None:
        _need(topk_w_out, "topk_w_out", torch.float32, (T, k), dev)
    if counts_out is not None:
        _need(counts_out, "counts_out", torch.int32, (E,), dev)
    if ws is None:
        ws = workspace(T, d, ffn, E, k, code, dev)
    st = load().moe_forward(_ptr(x), code, _ptr(router), _ptr(logit_bias),
                            _ptr(w1), _ptr(w3), _ptr(w2), T, d, ffn, E, k, _ptr(out),
                            _dtype_code(out.dtype), _ptr(topk_idx_out), _ptr(topk_w_out),
                            _ptr(counts_out), _ptr(ws), ws.numel(), _stream(dev),
                            _options(variant, events, down_split))
    _check("moe_forward", st)
    return out


def moe_block_forward(hidden, norm_weight, router, w1, w3, w2, k: int, eps: float = 1e-5,
                      logit_bias=None, out=None, out_dtype=None, norm_out=None, ws=None,
                      topk_idx_out=None, topk_w_out=None, counts_out=None, packed=False,
                      variant: int = 0, events=None, down_split: int = 0):
    """out = hidden + layer(RMSNorm(hidden)); returns (out, norm_out).
    norm_weight [d] float32; norm_out [T, d] has hidden's dtype."""
    T, d = hidden.shape
    E, ffn, _ = w1.shape
    dev = hidden.device
    code = _weight_code(hidden.dtype, packed, w1, w3, w2)
    _need(norm_weight, "norm_weight", torch.float32, (d,), dev)
    _need(router, "router", torch.float32, (E, d), dev)
    for name, t, shp in (("w1", w1, (E, ffn, d)), ("w3", w3, (E, ffn, d)), ("w2", w2, (E, d, ffn))):
        _need(t, name, hidden.dtype, shp, dev, code)
    if logit_bias is not None:
        _need(logit_bias, "logit_bias", torch.float32, (E,), dev)
    if norm_out is None:
        norm_out = torch.empty(T, d, dtype=hidden.dtype, device=dev)
    _need(norm_out, "norm_out", hidden.dtype, (T, d), dev)
    if out is None:
        out = torch.empty(T, d, dtype=out_dtype or hidden.dtype, device=dev)
    _need(out, "out", out.dtype, (T, d), dev)
    if topk_idx_out is not None:
        _need(topk_idx_out, "topk_idx_out", torch.int32, (T, k), dev)
    if topk_w_out is not None:
        _need(topk_w_out, "topk_w_out", torch.float32, (T, k), dev)
    if counts_out is not None:
        _need(counts_out, "counts_out", torch.int32, (E,), dev)
    if ws is None:
        ws = workspace(T, d, ffn, E, k, code, dev)
    st = load().moe_block_forward(_ptr(hidden), code, _ptr(norm_weight), float(eps),
                                  _ptr(norm_out), _ptr(router), _ptr(logit_bias), _ptr(w1),
                                  _ptr(w3), _ptr(w2), T, d, ffn, E, k, _ptr(out),
                                  _dtype_code(out.dtype), _ptr(topk_idx_out), _ptr(topk_w_out),
                                  _ptr(counts_out), _ptr(ws), ws.numel(), _stream(dev),
                                  _options(variant, events, down_split))
    _check("moe_block_forward", st)
    return out, norm_out


def moe_forward_noalloc(x, router, w1, w3, w2, k: int, logit_bias=None, out=None, out_dtype=None,
                        topk_idx_out=None, topk_w_out=None, counts_out=None, packed=False,
                        variant: int = 0, events=None, down_split: int = 0):
    """moe_forward on the library's built-in scratch instead of a workspace (the
    C call allocates nothing; this wrapper allocates `out` only when it is not
    passed). Sizes needing more than MOE_NOALLOC_SCRATCH_BYTES raise MoeError
    (MOE_EWORKSPACE). Calls that overlap on one GPU race (one shared scratch)."""
    T, d = x.shape
    E, ffn, _ = w1.shape
    dev = x.device
    code = _weight_code(x.dtype, packed, w1, w3, w2)
    _need(router, "router", torch.float32, (E, d), dev)
    for name, t, shp in (("w1", w1, (E, ffn, d)), ("w3", w3, (E, ffn, d)), ("w2", w2, (E, d, ffn))):
        _need(t, name, x.dtype, shp, dev, code)
    if logit_bias is not None:
        _need(logit_bias, "logit_bias", torch.float32, (E,), dev)
    if out is None:
        out = torch.empty(T, d, dtype=out_dtype or x.dtype, device=dev)
    _need(out, "out", out.dtype, (T, d), dev)
    if topk_idx_out is not None:
        _need(topk_idx_out, "topk_idx_out", torch.int32, (T, k), dev)
    if topk_w_out is not None:
        _need(topk_w_out, "topk_w_out", torch.float32, (T, k), dev)
    if counts_out is not None:
        _need(counts_out, "counts_out", torch.int32, (E,), dev)
    st = load().moe_forward_noalloc(_ptr(x), code, _ptr(router), _ptr(logit_bias), _ptr(w1),
                                    _ptr(w3), _ptr(w2), T, d, ffn, E, k, _ptr(out),
                                    _dtype_code(out.dtype), _ptr(topk_idx_out),
                                    _ptr(topk_w_out), _ptr(counts_out), _stream(dev),
                                    _options(variant, events, down_split))
    _check("moe_forward_noalloc", st)
    return out
