// Gate-weighted sum back to token order (nnterp Mixtral page, "The Notes":
// each routing slot's weighted expert output, summed over the slots, is the
// layer output, and there is no shared expert):
//   out[t] = sum_{j<k} w[t*k+j] * y[asg_pos[t*k+j]]
// A gather, not a scatter: no atomics, float32 accumulation in slot order,
// so the result is deterministic and a token whose weights are unchanged
// gives bit-identical output. One workgroup per token row; 16-byte accesses
// when d % 4 == 0.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <bool OUT_BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ y,
                                                          const int32_t* __restrict__ asg_pos,
                                                          const float* __restrict__ w, int d,
                                                          int k, void* __restrict__ out) {
  const int64_t t = blockIdx.x;
  if constexpr (VEC) {
    for (int i = threadIdx.x * 4; i < d; i += kThreads * 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < k; ++j) {
        const int64_t p = asg_pos[t * k + j];
        const float wt = w[t * k + j];
        const f32x4 v = *reinterpret_cast<const f32x4*>(y + p * d + i);
        acc[0] = fmaf(wt, v[0], acc[0]);
        acc[1] = fmaf(wt, v[1], acc[1]);
        acc[2] = fmaf(wt, v[2], acc[2]);
        acc[3] = fmaf(wt, v[3], acc[3]);
      }
      if constexpr (OUT_BF16) {
        uint2 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + t * d + i) = o;
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + t * d + i) = acc;
      }
    }
  } else {
    for (int i = threadIdx.x; i < d; i += kThreads) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) {
        const int64_t p = asg_pos[t * k + j];
        acc = fmaf(w[t * k + j], y[p * d + i], acc);
      }
      if constexpr (OUT_BF16) {
        static_cast<uint16_t*>(out)[t * d + i] = f32_to_bf16(acc);
      } else {
        static_cast<float*>(out)[t * d + i] = acc;
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const float* y, const int32_t* asg_pos, const float* w, int64_t T,
                          int d, int k, void* out, int out_bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const bool vec = (d % 4 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(out) & (out_bf16 ? 7 : 15)) == 0);
  const dim3 grid(static_cast<unsigned>(T));
  if (out_bf16) {
    if (vec)
      hipLaunchKernelGGL((combine_kernel<true, true>), grid, dim3(kThreads), 0, s, y, asg_pos, w,
                         d, k, out);
    else
      hipLaunchKernelGGL((combine_kernel<true, false>), grid, dim3(kThreads), 0, s, y, asg_pos,
                         w, d, k, out);
  } else {
    if (vec)
      hipLaunchKernelGGL((combine_kernel<false, true>), grid, dim3(kThreads), 0, s, y, asg_pos,
                         w, d, k, out);
    else
      hipLaunchKernelGGL((combine_kernel<false, false>), grid, dim3(kThreads), 0, s, y, asg_pos,
                         w, d, k, out);
  }
  return hipGetLastError();
}

}  // namespace moe
