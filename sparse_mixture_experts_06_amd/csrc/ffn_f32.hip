// Expert SwiGLU in float32 (the all-fp32 workloads): the same two grouped
// steps as the bf16 path, one thread per output element, float32 FMA
// accumulation, h kept in float32. Any d and ffn. When the rows are 16-byte
// aligned (K % 4 == 0 and aligned arrays) a thread reads them 4 floats at a
// time into 4 partial sums (the products of element i go to sum i % 4,
// added as (s0 + s1) + (s2 + s3) at the end), with several loads in flight:
// the dot products are short, so their time is load latency.
//   gate/up: h[p, n] = silu(x[r] . w1[e, n]) * (x[r] . w3[e, n]),  r = sorted_asg[p] / k
//   down:    y[p, n] = h[p] . w2[e, n]
// (nnterp Mixtral page, support(): act(gate) * up feeds the down projection.)
#include "common.h"

namespace moe {
namespace {

constexpr int TM = 16;  // rows per tile
constexpr int TN = 16;  // columns per tile

// tile b of a 1-D grid -> (expert, first row, first column); tiles are
// (expert, m-tile) major, n-tile minor, counted from the device offsets
__device__ __forceinline__ bool decode(const int32_t* __restrict__ offsets, int E, int ntn,
                                       int& e, int& beg, int& M, int& m0, int& n0) {
  int L = blockIdx.x / ntn;
  n0 = (blockIdx.x % ntn) * TN;
  for (int i = 0; i < E; ++i) {
    const int Mi = offsets[i + 1] - offsets[i];
    const int mt = (Mi + TM - 1) / TM;
    if (L < mt) {
      e = i;
      beg = offsets[i];
      M = Mi;
      m0 = L * TM;
      return true;
    }
    L -= mt;
  }
  return false;
}

// sum_i a[i] * b[i] over n floats: in order (VEC false) or with 16-byte
// loads into 4 partial sums (VEC: n % 4 == 0, both 16-byte aligned)
template <bool VEC>
__device__ __forceinline__ float dot_f32(const float* __restrict__ a, const float* __restrict__ b,
                                         int n) {
  if constexpr (VEC) {
    const float4* a4 = reinterpret_cast<const float4*>(a);
    const float4* b4 = reinterpret_cast<const float4*>(b);
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll 8
    for (int i = 0; i < n / 4; ++i) {
      const float4 u = a4[i], v = b4[i];
      s0 = fmaf(u.x, v.x, s0);
      s1 = fmaf(u.y, v.y, s1);
      s2 = fmaf(u.z, v.z, s2);
      s3 = fmaf(u.w, v.w, s3);
    }
    return (s0 + s1) + (s2 + s3);
  } else {
    float acc = 0.0f;
    for (int i = 0; i < n; ++i) acc = fmaf(a[i], b[i], acc);
    return acc;
  }
}

template <bool VEC>
__global__ __launch_bounds__(TM* TN) void gate_up_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w1, const float* __restrict__ w3,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_asg, int d, int ffn,
    int E, int k, float* __restrict__ h, int ntn) {
  int e, beg, M, m0, n0;
  if (!decode(offsets, E, ntn, e, beg, M, m0, n0)) return;
  const int m = m0 + static_cast<int>(threadIdx.x) / TN;
  const int n = n0 + static_cast<int>(threadIdx.x) % TN;
  if (m >= M || n >= ffn) return;
  const int64_t row = sorted_asg[beg + m] / k;
  const float* xr = x + row * d;
  const float* g1 = w1 + (static_cast<int64_t>(e) * ffn + n) * d;
  const float* g3 = w3 + (static_cast<int64_t>(e) * ffn + n) * d;
  const float g = dot_f32<VEC>(xr, g1, d);
  const float u = dot_f32<VEC>(xr, g3, d);
  h[static_cast<int64_t>(beg + m) * ffn + n] = g / (1.0f + expf(-g)) * u;
}

template <bool VEC>
__global__ __launch_bounds__(TM* TN) void down_f32_kernel(const float* __restrict__ h,
                                                         const float* __restrict__ w2,
                                                         const int32_t* __restrict__ offsets,
                                                         int d, int ffn, int E,
                                                         float* __restrict__ y, int ntn) {
  int e, beg, M, m0, n0;
  if (!decode(offsets, E, ntn, e, beg, M, m0, n0)) return;
  const int m = m0 + static_cast<int>(threadIdx.x) / TN;
  const int n = n0 + static_cast<int>(threadIdx.x) % TN;
  if (m >= M || n >= d) return;
  const float* hr = h + static_cast<int64_t>(beg + m) * ffn;
  const float* wr = w2 + (static_cast<int64_t>(e) * d + n) * ffn;
  y[static_cast<int64_t>(beg + m) * d + n] = dot_f32<VEC>(hr, wr, ffn);
}

inline unsigned grid_for(int64_t A, int E, int ntn) {
  return static_cast<unsigned>(((A + TM - 1) / TM + E) * ntn);
}

inline bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_gate_up_f32(const float* x, const float* w1, const float* w3,
                              const int32_t* offsets, const int32_t* sorted_asg, int64_t A,
                              int d, int ffn, int E, int k, float* h, hipStream_t s) {
  if (A == 0) return hipSuccess;
  const int ntn = (ffn + TN - 1) / TN;
  if (d % 4 == 0 && a16(x) && a16(w1) && a16(w3))
    hipLaunchKernelGGL(gate_up_f32_kernel<true>, dim3(grid_for(A, E, ntn)), dim3(TM * TN), 0, s,
                       x, w1, w3, offsets, sorted_asg, d, ffn, E, k, h, ntn);
  else
    hipLaunchKernelGGL(gate_up_f32_kernel<false>, dim3(grid_for(A, E, ntn)), dim3(TM * TN), 0, s,
                       x, w1, w3, offsets, sorted_asg, d, ffn, E, k, h, ntn);
  return hipGetLastError();
}

hipError_t launch_down_f32(const float* h, const float* w2, const int32_t* offsets, int64_t A,
                           int d, int ffn, int E, float* y, hipStream_t s) {
  if (A == 0) return hipSuccess;
  const int ntn = (d + TN - 1) / TN;
  // (h rows are ffn floats apart from an aligned workspace region)
  if (ffn % 4 == 0 && a16(h) && a16(w2))
    hipLaunchKernelGGL(down_f32_kernel<true>, dim3(grid_for(A, E, ntn)), dim3(TM * TN), 0, s, h,
                       w2, offsets, d, ffn, E, y, ntn);
  else
    hipLaunchKernelGGL(down_f32_kernel<false>, dim3(grid_for(A, E, ntn)), dim3(TM * TN), 0, s, h,
                       w2, offsets, d, ffn, E, y, ntn);
  return hipGetLastError();
}

}  // namespace moe
