// libmoe C ABI: argument checks, workspace carving and stream-ordered
// launches. Nothing here allocates, frees or synchronises, and nothing is
// kept between calls: the per-call choices (kernel family, profiling events)
// arrive in a moe_options argument.
#include "moe.h"

#include <string.h>

#include <mutex>

#include "common.h"

// Workspace of moe_forward_noalloc: one array per GPU (the code object's copy
// on each device), never passed to a kernel by this name: host code takes its
// device address from hipGetSymbolAddress once per device and uses that.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxAssignments = MOE_MAX_ASSIGNMENTS;
static_assert(kMaxAssignments + 1024 <= (int64_t(1) << 31), "the permutation's steps use int");

// a call's options, checked
struct Opts {
  int variant = 0;                     // expert-FFN kernel family (0 = by size)
  void* const* events = nullptr;       // 6 stage events, or none
  int down_split = 0;                  // down K split (0 = chosen on the device)
};

int read_options(const moe_options* o, Opts* out) {
  *out = Opts{};
  if (!o) return MOE_OK;
  if (o->ffn_variant < 0 || o->ffn_variant > 2) return MOE_EINVAL;
  if (!(o->down_split == 0 || o->down_split == -1 || (o->down_split >= 8 && o->down_split <= 13)))
    return MOE_EINVAL;
  if (o->stage_events)
    for (int i = 0; i < 6; ++i)
      if (!o->stage_events[i]) return MOE_EINVAL;
  out->variant = o->ffn_variant;
  out->events = o->stage_events;
  out->down_split = o->down_split;
  return MOE_OK;
}

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Device address of `scratch` on the current device, looked up on the first
// call there (with that device current) and kept per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

struct Layout {
  size_t idx, w, counts, offsets, sorted, pos, nsplit, h, y, wide, total;
};

// bfloat16 activations (x, h): bf16 weights in either layout, or int8 weights
inline bool is_bf16(int dtype) {
  return dtype == MOE_BF16 || dtype == MOE_BF16_PACKED || dtype == MOE_INT8_PACKED;
}

// float32 partial results the down projection may leave (split K); the most
// either kernel family may leave, so that the workspace does not depend on
// the variant (the direct-to-LDS kernel chooses within it on the device)
int ws_splits(int64_t A, int d, int ffn, int E, int dtype) {
  if (!is_bf16(dtype)) return 1;
  const int a = moe::down_splits(1, A, d, ffn, E), b = moe::down_splits(2, A, d, ffn, E);
  // int8: its tiled kernel also runs where bf16 would take the direct-to-LDS one
  const int c = dtype == MOE_INT8_PACKED ? moe::int8_down_splits(2, A, d, ffn, E) : 1;
  const int ab = a > b ? a : b;
  return ab > c ? ab : c;
}

Layout layout(int64_t T, int d, int ffn, int E, int k, int dtype) {
  const size_t A = static_cast<size_t>(T) * static_cast<size_t>(k);
  const size_t hb = is_bf16(dtype) ? 2 : 4;
  const size_t ns = static_cast<size_t>(ws_splits(static_cast<int64_t>(A), d, ffn, E, dtype));
  Layout L;
  size_t o = 0;
  L.idx = o;     o = align256(o + A * 4);
  L.w = o;       o = align256(o + A * 4);
  L.counts = o;  o = align256(o + static_cast<size_t>(E) * 4);
  L.offsets = o; o = align256(o + static_cast<size_t>(E + 1) * 4);
  L.sorted = o;  o = align256(o + A * 4);
  L.pos = o;     o = align256(o + A * 4);
  L.nsplit = o;  o = align256(o + 4);  // partial arrays the down kernel wrote
  L.h = o;       o = align256(o + A * static_cast<size_t>(ffn) * hb);
  L.y = o;       o = align256(o + ns * A * static_cast<size_t>(d) * 4);
  L.wide = o;
  if (dtype == MOE_INT8_PACKED)
    o = align256(o + moe::int8_wide_bytes(static_cast<int64_t>(A), k, d, ffn, E));
  L.total = o;
  return L;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline bool valid_dtype(int t) { return t == MOE_F32 || t == MOE_BF16; }
inline bool valid_weight_dtype(int t) {
  return valid_dtype(t) || t == MOE_BF16_PACKED || t == MOE_INT8_PACKED;
}

int check_sizes(int64_t T, int E, int k) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E) return MOE_EINVAL;
  if (T > kMaxAssignments / k) return MOE_EINVAL;
  return MOE_OK;
}

int check_ffn_shape(int64_t T, int d, int ffn, int E, int k, int dtype) {
  if (d < 1 || ffn < 1) return MOE_EINVAL;
  if (!valid_weight_dtype(dtype)) return MOE_EINVAL;
  const int64_t A = T * k;
  if (is_bf16(dtype)) {
    if (d % 64 != 0 || ffn % 64 != 0) return MOE_ENOTSUP;
    // worst-case tile grid of the tiled kernels must fit a 1-D launch
    const int64_t mt = (A + 127) / 128 + E;
    // (the down grid doubles when it splits K)
    const int64_t n = (ffn / 64 > 2 * ((d + 127) / 128)) ? ffn / 64 : 2 * ((d + 127) / 128);
    if (mt * n >= (int64_t(1) << 31)) return MOE_ENOTSUP;
  } else {
    const int64_t mt = (A + 15) / 16 + E;
    const int64_t n = ((ffn > d ? ffn : d) + 15) / 16;
    if (mt * n >= (int64_t(1) << 31)) return MOE_ENOTSUP;
  }
  return MOE_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

inline void stage(const Opts& o, int i, hipStream_t s) {
  if (o.events) (void)hipEventRecord(static_cast<hipEvent_t>(o.events[i]), s);
}

// gate/up then down; the down result is left as up to `nsplit_out` partial
// arrays at `part` (the caller sums them: the combine, or moe_expert_ffn).
// Where the direct-to-LDS down kernel runs it chooses the count on the device
// and writes it to `ns_word`; *ns_dev_out is then ns_word, else null. `wide`:
// the workspace region for int8 weights widened to bf16 (prefill sizes)
int run_ffn(const void* x, int dtype, const void* w1, const void* w3, const void* w2,
            const int32_t* offsets, const int32_t* sorted_asg, int64_t T, int d, int ffn, int E,
            int k, float* part, void* h, void* wide, int32_t* ns_word, hipStream_t s,
            const Opts& opt, bool with_events, int* nsplit_out, const int32_t** ns_dev_out,
            const moe::FusedPermute* fp = nullptr) {
  const int64_t A = T * k;
  const moe::DownSplit ds{opt.down_split, ns_word};
  *ns_dev_out = nullptr;
  hipError_t err;
  if (dtype == MOE_INT8_PACKED) {
    // int8 weights: the streaming kernels on the codes (few rows per expert),
    // the tiled kernel widening its operands in registers (more), or the
    // codes widened to bf16 in the workspace and the direct-to-LDS kernels
    // with row scales (many rows per expert)
    const int variant = moe::choose_int8_ffn_variant(opt.variant, A, E);
    const int dvariant = moe::choose_int8_down_variant(opt.variant, A, E);
    *nsplit_out = moe::int8_down_splits(dvariant, A, d, ffn, E);
    uint16_t* wb = static_cast<uint16_t*>(wide);
    if (variant != 1 && moe::int8_gate_up_dma(A, k, d, ffn, E)) {
      uint16_t* w3b = wb + static_cast<size_t>(E) * ffn * d;
      err = moe::launch_widen_int8(w1, E, ffn, d, wb, s);
      if (err == hipSuccess) err = moe::launch_widen_int8(w3, E, ffn, d, w3b, s);
      if (err == hipSuccess)
        err = moe::launch_gate_up_dma(true, static_cast<const uint16_t*>(x), wb, w3b, offsets,
                                      sorted_asg, A, d, ffn, E, k, static_cast<uint16_t*>(h), s,
                                      moe::int8_scales(w1, E, ffn, d),
                                      moe::int8_scales(w3, E, ffn, d));
    } else {
      err = moe::launch_gate_up_int8(variant, static_cast<const uint16_t*>(x), w1, w3, offsets,
                                     sorted_asg, A, d, ffn, E, k, static_cast<uint16_t*>(h), s);
    }
    if (err != hipSuccess) return MOE_EHIP;
    if (with_events) stage(opt, 3, s);
    if (dvariant != 1 && moe::int8_down_dma(A, d, ffn, E)) {
      // (stream order: gate/up has finished with the widened w1 and w3)
      err = moe::launch_widen_int8(w2, E, d, ffn, wb, s);
      if (err == hipSuccess)
        err = moe::launch_down_dma(true, static_cast<const uint16_t*>(h), wb, offsets, A, d, ffn,
                                   E, *nsplit_out, part, s, moe::int8_scales(w2, E, d, ffn), ds);
      *ns_dev_out = ns_word;
    } else {
      err = moe::launch_down_int8(dvariant, static_cast<const uint16_t*>(h), w2, offsets, A, d,
                                  ffn, E, *nsplit_out, part, s);
    }
  } else if (is_bf16(dtype)) {
    const int variant = moe::choose_ffn_variant(opt.variant, A, E);
    const int dvariant = moe::choose_down_variant(opt.variant, A, E);
    const bool packed = dtype == MOE_BF16_PACKED;
    *nsplit_out = moe::down_splits(dvariant, A, d, ffn, E);
    err = moe::launch_gate_up_bf16(variant, packed, static_cast<const uint16_t*>(x),
                                   static_cast<const uint16_t*>(w1),
                                   static_cast<const uint16_t*>(w3), offsets, sorted_asg, A, d,
                                   ffn, E, k, static_cast<uint16_t*>(h), s, fp);
    if (err != hipSuccess) return MOE_EHIP;
    if (with_events) stage(opt, 3, s);
    err = moe::launch_down_bf16(dvariant, packed, static_cast<const uint16_t*>(h),
                                static_cast<const uint16_t*>(w2), offsets, A, d, ffn, E, part, s,
                                ds);
    if (moe::down_dma_runs(dvariant, A, d, ffn, E)) *ns_dev_out = ns_word;
  } else {
    *nsplit_out = 1;
    err = moe::launch_gate_up_f32(static_cast<const float*>(x), static_cast<const float*>(w1),
                                  static_cast<const float*>(w3), offsets, sorted_asg, A, d, ffn,
                                  E, k, static_cast<float*>(h), s);
    if (err != hipSuccess) return MOE_EHIP;
    if (with_events) stage(opt, 3, s);
    err = moe::launch_down_f32(static_cast<const float*>(h), static_cast<const float*>(w2),
                               offsets, A, d, ffn, E, part, s);
  }
  return hip_status(err);
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "success";
    case MOE_EINVAL: return "invalid argument (pointer, size, dtype, k or E)";
    case MOE_ENOTSUP: return "unsupported shape or alignment (bf16 needs d, ffn % 64 == 0 and 16-byte aligned buffers)";
    case MOE_EWORKSPACE: return "workspace missing or smaller than moe_workspace_bytes() (moe_forward_noalloc: more than its built-in scratch)";
    case MOE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t moe_workspace_bytes(int64_t T, int d, int ffn, int E, int k, int dtype) {
  if (check_sizes(T, E, k) != MOE_OK || d < 1 || ffn < 1 || !valid_weight_dtype(dtype)) return 0;
  return layout(T, d, ffn, E, k, dtype).total;
}

int moe_route(const void* x, int x_dtype, const float* router, const float* logit_bias,
              int64_t T, int d, int E, int k, float* logits_out, int32_t* topk_idx,
              float* topk_w, void* stream) {
  int st = check_sizes(T, E, k);
  if (st != MOE_OK) return st;
  if (d < 1 || !valid_dtype(x_dtype)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !router || !topk_idx || !topk_w) return MOE_EINVAL;
  return hip_status(moe::launch_route(x, x_dtype == MOE_BF16, router, logit_bias, T, d, E, k,
                                      logits_out, topk_idx, topk_w,
                                      static_cast<hipStream_t>(stream)));
}

int moe_permute(const int32_t* topk_idx, int64_t T, int E, int k, int32_t* counts,
                int32_t* offsets, int32_t* sorted_asg, int32_t* asg_pos, void* ws,
                size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int st = check_sizes(T, E, k);
  if (st != MOE_OK) return st;
  if (!counts || !offsets) return MOE_EINVAL;
  if (T > 0 && (!topk_idx || !sorted_asg || !asg_pos)) return MOE_EINVAL;
  return hip_status(moe::launch_permute(topk_idx, T * k, E, counts, offsets, sorted_asg,
                                        asg_pos, static_cast<hipStream_t>(stream)));
}

int moe_check_routing(const int32_t* topk_idx, int64_t T, int E, int k, int32_t* bad_out,
                      void* stream) {
  const int st = check_sizes(T, E, k);
  if (st != MOE_OK) return st;
  if (!bad_out || (T > 0 && !topk_idx)) return MOE_EINVAL;
  return hip_status(moe::launch_check_routing(topk_idx, T, k, E, bad_out,
                                              static_cast<hipStream_t>(stream)));
}

int moe_expert_ffn(const void* x, int dtype, const void* w1, const void* w3, const void* w2,
                   const int32_t* offsets, const int32_t* sorted_asg, int64_t T, int d,
                   int ffn, int E, int k, float* y, void* ws, size_t ws_bytes, void* stream,
                   const moe_options* options) {
  Opts opt;
  int st = read_options(options, &opt);
  if (st != MOE_OK) return st;
  st = check_sizes(T, E, k);
  if (st != MOE_OK) return st;
  st = check_ffn_shape(T, d, ffn, E, k, dtype);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !w1 || !w3 || !w2 || !offsets || !sorted_asg || !y) return MOE_EINVAL;
  const Layout L = layout(T, d, ffn, E, k, dtype);
  if (!ws || ws_bytes < L.total) return MOE_EWORKSPACE;
  if (is_bf16(dtype) &&
      !(aligned16(x) && aligned16(w1) && aligned16(w3) && aligned16(w2) && aligned16(ws) &&
        aligned16(y)))
    return MOE_ENOTSUP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  const int64_t A = T * k;
  const int nsplit =
      dtype == MOE_INT8_PACKED
          ? moe::int8_down_splits(moe::choose_int8_down_variant(opt.variant, A, E), A, d, ffn, E)
      : is_bf16(dtype)
          ? moe::down_splits(moe::choose_down_variant(opt.variant, A, E), A, d, ffn, E)
          : 1;
  float* part = nsplit > 1 ? reinterpret_cast<float*>(base + L.y) : y;
  int used = 1;
  const int32_t* ns_dev = nullptr;
  st = run_ffn(x, dtype, w1, w3, w2, offsets, sorted_asg, T, d, ffn, E, k, part, base + L.h,
               base + L.wide, reinterpret_cast<int32_t*>(base + L.nsplit), s, opt, false, &used,
               &ns_dev);
  if (st != MOE_OK) return st;
  if (used > 1)
    return hip_status(
        moe::launch_sum_partials(part, used, A * static_cast<int64_t>(d), y, s, ns_dev));
  return MOE_OK;
}

int moe_combine(const float* y, const int32_t* asg_pos, const float* topk_w, int64_t T, int d,
                int k, void* out, int out_dtype, void* stream) {
  if (T < 0 || d < 1 || k < 1 || !valid_dtype(out_dtype)) return MOE_EINVAL;
  if (T > kMaxAssignments / k) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!y || !asg_pos || !topk_w || !out) return MOE_EINVAL;
  return hip_status(moe::launch_combine(y, 1, asg_pos, topk_w, T, d, k, out,
                                        out_dtype == MOE_BF16, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// the fused path; with gamma non-null the router and experts read the RMS-normed
// rows (written to norm_out) and the combine adds x back (the block's MLP half)
int forward_impl(const void* x, int dtype, const float* gamma, float eps, void* norm_out,
                 const float* router, const float* logit_bias, const void* w1, const void* w3,
                 const void* w2, int64_t T, int d, int ffn, int E, int k, void* out,
                 int out_dtype, int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                 void* ws, size_t ws_bytes, void* stream, const moe_options* options) {
  Opts opt;
  int st = read_options(options, &opt);
  if (st != MOE_OK) return st;
  st = check_sizes(T, E, k);
  if (st != MOE_OK) return st;
  st = check_ffn_shape(T, d, ffn, E, k, dtype);
  if (st != MOE_OK) return st;
  if (!valid_dtype(out_dtype)) return MOE_EINVAL;
  if (T > 0 && (!x || !router || !w1 || !w3 || !w2 || !out)) return MOE_EINVAL;
  const Layout L = layout(T, d, ffn, E, k, dtype);
  if (!ws || ws_bytes < L.total) return MOE_EWORKSPACE;
  if (is_bf16(dtype) && T > 0 &&
      !(aligned16(x) && aligned16(w1) && aligned16(w3) && aligned16(w2) && aligned16(ws) &&
        (!norm_out || aligned16(norm_out))))
    return MOE_ENOTSUP;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  int32_t* idx = topk_idx_out ? topk_idx_out : reinterpret_cast<int32_t*>(base + L.idx);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(base + L.w);
  int32_t* counts = counts_out ? counts_out : reinterpret_cast<int32_t*>(base + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* sorted_asg = reinterpret_cast<int32_t*>(base + L.sorted);
  int32_t* asg_pos = reinterpret_cast<int32_t*>(base + L.pos);
  void* h = base + L.h;
  float* y = reinterpret_cast<float*>(base + L.y);
  const void* xin = gamma ? norm_out : x;  // what the experts read

  // few assignments on the bf16 streaming kernels: the gate/up kernel does the
  // permutation itself (one launch less; the same arrays, bit for bit)
  const int64_t A = T * k;
  const bool fuse = T > 0 && (dtype == MOE_BF16 || dtype == MOE_BF16_PACKED) &&
                    moe::gate_up_fuses_permute(moe::choose_ffn_variant(opt.variant, A, E), A);
  const moe::FusedPermute fp{idx, counts, offsets, sorted_asg, asg_pos};

  stage(opt, 0, s);
  if (T > 0 && moe::launch_route(x, is_bf16(dtype), router, logit_bias, T, d, E, k, nullptr,
                                 idx, w, s, gamma, eps, norm_out) != hipSuccess)
    return MOE_EHIP;
  stage(opt, 1, s);
  if (!fuse &&
      moe::launch_permute(idx, A, E, counts, offsets, sorted_asg, asg_pos, s) != hipSuccess)
    return MOE_EHIP;
  stage(opt, 2, s);
  if (T == 0) {
    for (int i = 3; i < 6; ++i) stage(opt, i, s);
    return MOE_OK;
  }
  int nsplit = 1;
  const int32_t* ns_dev = nullptr;
  st = run_ffn(xin, dtype, w1, w3, w2, offsets, sorted_asg, T, d, ffn, E, k, y, h, base + L.wide,
               reinterpret_cast<int32_t*>(base + L.nsplit), s, opt, true, &nsplit, &ns_dev,
               fuse ? &fp : nullptr);
  if (st != MOE_OK) return st;
  stage(opt, 4, s);
  if (moe::launch_combine(y, nsplit, asg_pos, w, T, d, k, out, out_dtype == MOE_BF16, s,
                          gamma ? x : nullptr, is_bf16(dtype), ns_dev) != hipSuccess)
    return MOE_EHIP;
  stage(opt, 5, s);
  return MOE_OK;
}

inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const char* p = static_cast<const char*>(a);
  const char* q = static_cast<const char*>(b);
  return p < q + nb && q < p + na;
}

}  // namespace

extern "C" {

int moe_forward(const void* x, int dtype, const float* router, const float* logit_bias,
                const void* w1, const void* w3, const void* w2, int64_t T, int d, int ffn,
                int E, int k, void* out, int out_dtype, int32_t* topk_idx_out,
                float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                void* stream, const moe_options* options) {
  return forward_impl(x, dtype, nullptr, 0.0f, nullptr, router, logit_bias, w1, w3, w2, T, d,
                      ffn, E, k, out, out_dtype, topk_idx_out, topk_w_out, counts_out, ws,
                      ws_bytes, stream, options);
}

int moe_block_forward(const void* hidden, int dtype, const float* norm_weight, float eps,
                      void* norm_out, const float* router, const float* logit_bias,
                      const void* w1, const void* w3, const void* w2, int64_t T, int d, int ffn,
                      int E, int k, void* out, int out_dtype, int32_t* topk_idx_out,
                      float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                      void* stream, const moe_options* options) {
  if (!(eps >= 0.0f) || eps > 3.0e38f) return MOE_EINVAL;  // rejects NaN and infinity too
  if (T > 0) {
    if (!norm_weight || !norm_out || !hidden || !out) return MOE_EINVAL;
    if (!valid_weight_dtype(dtype) || !valid_dtype(out_dtype) || d < 1) return MOE_EINVAL;
    if (T > kMaxAssignments) return MOE_EINVAL;
    const size_t xb = is_bf16(dtype) ? 2 : 4;
    const size_t ob = out_dtype == MOE_BF16 ? 2 : 4;
    const size_t n = static_cast<size_t>(T) * static_cast<size_t>(d);
    if (overlap(norm_out, n * xb, hidden, n * xb) || overlap(out, n * ob, hidden, n * xb) ||
        overlap(out, n * ob, norm_out, n * xb))
      return MOE_EINVAL;
  }
  return forward_impl(hidden, dtype, norm_weight, eps, norm_out, router, logit_bias, w1, w3, w2,
                      T, d, ffn, E, k, out, out_dtype, topk_idx_out, topk_w_out, counts_out, ws,
                      ws_bytes, stream, options);
}

int moe_forward_noalloc(const void* x, int dtype, const float* router, const float* logit_bias,
                        const void* w1, const void* w3, const void* w2, int64_t T, int d, int ffn,
                        int E, int k, void* out, int out_dtype, int32_t* topk_idx_out,
                        float* topk_w_out, int32_t* counts_out, void* stream,
                        const moe_options* options) {
  // sizes beyond the scratch (or invalid ones) reach forward_impl without a
  // workspace, which reports them before anything is enqueued
  const size_t need = moe_workspace_bytes(T, d, ffn, E, k, dtype);
  void* ws = nullptr;
  if (need > 0 && need <= MOE_NOALLOC_SCRATCH_BYTES) {
    const int st = scratch_address(&ws);
    if (st != MOE_OK) return st;
  }
  return forward_impl(x, dtype, nullptr, 0.0f, nullptr, router, logit_bias, w1, w3, w2, T, d,
                      ffn, E, k, out, out_dtype, topk_idx_out, topk_w_out, counts_out, ws,
                      ws ? MOE_NOALLOC_SCRATCH_BYTES : 0, stream, options);
}

size_t moe_quantized_weight_bytes(int E, int rows, int cols) {
  if (E < 1 || E > MOE_MAX_EXPERTS || rows < 1 || cols < 1) return 0;
  if (rows % 16 != 0 || cols % 64 != 0) return 0;
  return moe::int8_weight_bytes(E, rows, cols);
}

int moe_quantize_weight(const void* w, int dtype, int E, int rows, int cols, void* out,
                        void* stream) {
  if (dtype != MOE_BF16) return MOE_EINVAL;
  if (E < 1 || E > MOE_MAX_EXPERTS || rows < 1 || cols < 1) return MOE_EINVAL;
  if (rows % 16 != 0 || cols % 64 != 0) return MOE_ENOTSUP;
  if (!w || !out) return MOE_EINVAL;
  if (!aligned16(w) || !aligned16(out)) return MOE_ENOTSUP;
  const size_t in_bytes = static_cast<size_t>(E) * rows * cols * 2;
  const size_t out_bytes = moe::int8_weight_bytes(E, rows, cols);
  const char* a = static_cast<const char*>(w);
  const char* b = static_cast<const char*>(out);
  if (a < b + out_bytes && b < a + in_bytes) return MOE_EINVAL;  // must not overlap
  return hip_status(moe::launch_quantize_int8(static_cast<const uint16_t*>(w), E, rows, cols, out,
                                              static_cast<hipStream_t>(stream)));
}

int moe_pack_weight(const void* w, int dtype, int E, int rows, int cols, void* out,
                    void* stream) {
  if (dtype != MOE_BF16) return MOE_EINVAL;
  if (E < 1 || E > MOE_MAX_EXPERTS || rows < 1 || cols < 1) return MOE_EINVAL;
  if (rows % 16 != 0 || cols % 32 != 0) return MOE_ENOTSUP;
  if (!w || !out) return MOE_EINVAL;
  if (!aligned16(w) || !aligned16(out)) return MOE_ENOTSUP;
  const size_t bytes = static_cast<size_t>(E) * rows * cols * 2;
  const char* a = static_cast<const char*>(w);
  const char* b = static_cast<const char*>(out);
  if (a < b + bytes && b < a + bytes) return MOE_EINVAL;  // must not overlap
  return hip_status(moe::launch_pack_bf16(static_cast<const uint16_t*>(w), E, rows, cols,
                                          static_cast<uint16_t*>(out),
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"
#pragma GCC visibility pop
