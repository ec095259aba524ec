// Router + scoring: logits = x . router^T (+bias), float32 softmax over the
// experts, top-k (largest first, exact ties to the lower expert index) and
// renormalisation of the kept probabilities (nnterp Mixtral page, "The Notes":
// the router renormalizes its top 2 in float32; support(): router_logits is
// the router's linear output, before the scoring).
//
// Work split: one wave handles kTokensPerWave tokens at once, so each router
// element fetched from L2 is used for several tokens. Lanes stride over the
// hidden dimension in 8-element chunks (16-byte loads for bf16), accumulate
// kTokensPerWave x E float32 partial dot products, and a butterfly reduction
// leaves every logit in every lane. Lane j then finishes token j.
#include "common.h"

namespace moe {
namespace {

constexpr int kTokensPerWave = 4;
constexpr int kWavesPerBlock = 4;

template <bool BF16>
__device__ __forceinline__ void load8(const void* x, int64_t row, int d, int i, float* v) {
  if constexpr (BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(x) + row * d + i;
    u32x4 q = ldg16(p);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[2 * h] = __uint_as_float(q[h] << 16);
      v[2 * h + 1] = __uint_as_float(q[h] & 0xFFFF0000u);
    }
  } else {
    const float* p = static_cast<const float*>(x) + row * d + i;
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* x, int64_t row, int d, int i) {
  if constexpr (BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(x)[row * d + i]);
  } else {
    return static_cast<const float*>(x)[row * d + i];
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// EM: compile-time upper bound on E (8 or 32). VEC: rows are 16-byte aligned
// and d % 8 == 0, so the 8-wide loads are legal.
template <bool BF16, int EM, bool VEC>
__global__ __launch_bounds__(kWave* kWavesPerBlock) void route_kernel(
    const void* __restrict__ x, const float* __restrict__ router, const float* __restrict__ bias,
    int64_t T, int d, int E, int k, float* __restrict__ logits_out, int32_t* __restrict__ idx,
    float* __restrict__ wout) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t t0 = (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave) * kTokensPerWave;

  float acc[kTokensPerWave][EM];
#pragma unroll
  for (int tt = 0; tt < kTokensPerWave; ++tt)
#pragma unroll
    for (int e = 0; e < EM; ++e) acc[tt][e] = 0.0f;

  int64_t rows[kTokensPerWave];
  bool live[kTokensPerWave];
#pragma unroll
  for (int tt = 0; tt < kTokensPerWave; ++tt) {
    live[tt] = (t0 + tt) < T;
    rows[tt] = live[tt] ? t0 + tt : 0;
  }

  int tail_start = 0;
  if constexpr (VEC) {
    const int nvec = d / 8;
    for (int c = lane; c < nvec; c += kWave) {
      const int i = c * 8;
      float xv[kTokensPerWave][8];
#pragma unroll
      for (int tt = 0; tt < kTokensPerWave; ++tt) {
        if (live[tt]) {
          load8<BF16>(x, rows[tt], d, i, xv[tt]);
        } else {
#pragma unroll
          for (int v = 0; v < 8; ++v) xv[tt][v] = 0.0f;
        }
      }
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        if (e < E) {
          const float* rp = router + static_cast<int64_t>(e) * d + i;
          float4 ra = *reinterpret_cast<const float4*>(rp);
          float4 rb = *reinterpret_cast<const float4*>(rp + 4);
          const float r8[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
#pragma unroll
          for (int tt = 0; tt < kTokensPerWave; ++tt)
#pragma unroll
            for (int v = 0; v < 8; ++v) acc[tt][e] = fmaf(xv[tt][v], r8[v], acc[tt][e]);
        }
      }
    }
    tail_start = nvec * 8;
  }
  for (int i = tail_start + lane; i < d; i += kWave) {
    float xs[kTokensPerWave];
#pragma unroll
    for (int tt = 0; tt < kTokensPerWave; ++tt) xs[tt] = live[tt] ? load1<BF16>(x, rows[tt], d, i) : 0.0f;
#pragma unroll
    for (int e = 0; e < EM; ++e) {
      if (e < E) {
        const float r = router[static_cast<int64_t>(e) * d + i];
#pragma unroll
        for (int tt = 0; tt < kTokensPerWave; ++tt) acc[tt][e] = fmaf(xs[tt], r, acc[tt][e]);
      }
    }
  }

#pragma unroll
  for (int tt = 0; tt < kTokensPerWave; ++tt)
#pragma unroll
    for (int e = 0; e < EM; ++e)
      if (e < E) acc[tt][e] = wave_sum(acc[tt][e]);

  // lane tt finishes token t0 + tt
  if (lane >= kTokensPerWave) return;
  float l[EM];
#pragma unroll
  for (int e = 0; e < EM; ++e) l[e] = 0.0f;
#pragma unroll
  for (int tt = 0; tt < kTokensPerWave; ++tt)
    if (lane == tt)
#pragma unroll
      for (int e = 0; e < EM; ++e) l[e] = acc[tt][e];
  const int64_t t = t0 + lane;
  if (t >= T) return;

  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    if (e < E) {
      if (bias) l[e] += bias[e];
      m = fmaxf(m, l[e]);
    }
  }
  if (logits_out) {
#pragma unroll
    for (int e = 0; e < EM; ++e)
      if (e < E) logits_out[t * E + e] = l[e];
  }
  // float32 softmax over the E experts
  float p[EM];
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    p[e] = (e < E) ? expf(l[e] - m) : 0.0f;
    s += p[e];
  }
#pragma unroll
  for (int e = 0; e < EM; ++e) p[e] = p[e] / s;

  // top-k on the logits: strict '>' keeps the lower index on an exact tie
  uint32_t taken = 0;
  float psum = 0.0f;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    float bl = 0.0f;
    float bp = 0.0f;
#pragma unroll
    for (int e = 0; e < EM; ++e) {
      if (e < E && !((taken >> e) & 1u) && (best < 0 || l[e] > bl)) {
        best = e;
        bl = l[e];
        bp = p[e];
      }
    }
    if (best < 0) {  // only with NaN logits: take the lowest free expert
#pragma unroll
      for (int e = EM - 1; e >= 0; --e)
        if (e < E && !((taken >> e) & 1u)) { best = e; bp = p[e]; }
    }
    taken |= 1u << best;
    idx[t * k + j] = best;
    psum += bp;
    wout[t * k + j] = bp;  // rescaled below
  }
  for (int j = 0; j < k; ++j) wout[t * k + j] = wout[t * k + j] / psum;
}

template <bool BF16, int EM>
hipError_t launch_em(const void* x, const float* router, const float* bias, int64_t T, int d,
                     int E, int k, float* logits_out, int32_t* idx, float* w, hipStream_t s) {
  const int64_t per_block = static_cast<int64_t>(kTokensPerWave) * kWavesPerBlock;
  const dim3 grid(static_cast<unsigned>((T + per_block - 1) / per_block));
  const dim3 block(kWave * kWavesPerBlock);
  const bool vec = (d % 8 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(router) & 15) == 0);
  if (vec)
    hipLaunchKernelGGL((route_kernel<BF16, EM, true>), grid, block, 0, s, x, router, bias, T, d,
                       E, k, logits_out, idx, w);
  else
    hipLaunchKernelGGL((route_kernel<BF16, EM, false>), grid, block, 0, s, x, router, bias, T,
                       d, E, k, logits_out, idx, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const void* x, int x_bf16, const float* router, const float* bias,
                        int64_t T, int d, int E, int k, float* logits_out, int32_t* idx,
                        float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (x_bf16) {
    if (E <= 8) return launch_em<true, 8>(x, router, bias, T, d, E, k, logits_out, idx, w, s);
    return launch_em<true, 32>(x, router, bias, T, d, E, k, logits_out, idx, w, s);
  }
  if (E <= 8) return launch_em<false, 8>(x, router, bias, T, d, E, k, logits_out, idx, w, s);
  return launch_em<false, 32>(x, router, bias, T, d, E, k, logits_out, idx, w, s);
}

}  // namespace moe
