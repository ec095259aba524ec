// Gate-weighted sum back to token order (nnterp Mixtral page, "The Notes":
// each routing slot's weighted expert output, summed over the slots, is the
// layer output, and there is no shared expert):
//   out[t] = sum_{j<k} w[t*k+j] * y[asg_pos[t*k+j]]
// A gather, not a scatter: no atomics, float32 accumulation in slot order,
// so the result is deterministic and a token whose weights are unchanged
// gives bit-identical output. Workgroup (t, c) handles columns
// [c*1024, (c+1)*1024) of token t, 4 per thread with 16-byte accesses when
// d % 4 == 0, so all of a thread's k*nsplit loads are in flight together. When the down projection left its result as nsplit
// partial sums (split K), each y row is first summed over the splits in
// split order. With a residual (the block's input, nnterp Mixtral page,
// "The Notes": out = h + mlp(post_attention_layernorm(h))), it is added to
// the finished slot sum.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// RES: 0 none, 1 float32 residual, 2 bfloat16 residual
template <bool OUT_BF16, bool VEC, int RES>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ y,
                                                          int nsplit, int64_t pstride,
                                                          const int32_t* __restrict__ asg_pos,
                                                          const float* __restrict__ w, int d,
                                                          int k, void* __restrict__ out,
                                                          const void* __restrict__ res) {
  const int64_t t = blockIdx.x;
  const int col0 = blockIdx.y * kThreads * 4;
  const int col1 = min(d, col0 + kThreads * 4);
  if constexpr (VEC) {
    for (int i = col0 + threadIdx.x * 4; i < col1; i += kThreads * 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < k; ++j) {
        const int64_t p = asg_pos[t * k + j];
        const float wt = w[t * k + j];
        f32x4 v = *reinterpret_cast<const f32x4*>(y + p * d + i);
        for (int sp = 1; sp < nsplit; ++sp)
          v += *reinterpret_cast<const f32x4*>(y + sp * pstride + p * d + i);
        acc[0] = fmaf(wt, v[0], acc[0]);
        acc[1] = fmaf(wt, v[1], acc[1]);
        acc[2] = fmaf(wt, v[2], acc[2]);
        acc[3] = fmaf(wt, v[3], acc[3]);
      }
      if constexpr (RES == 1) {
        acc += *reinterpret_cast<const f32x4*>(static_cast<const float*>(res) + t * d + i);
      } else if constexpr (RES == 2) {
        const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(res) + t * d + i);
        acc[0] += __uint_as_float(r.x << 16);
        acc[1] += __uint_as_float(r.x & 0xFFFF0000u);
        acc[2] += __uint_as_float(r.y << 16);
        acc[3] += __uint_as_float(r.y & 0xFFFF0000u);
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
    for (int i = col0 + threadIdx.x; i < col1; i += kThreads) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) {
        const int64_t p = asg_pos[t * k + j];
        float v = y[p * d + i];
        for (int sp = 1; sp < nsplit; ++sp) v += y[sp * pstride + p * d + i];
        acc = fmaf(w[t * k + j], v, acc);
      }
      if constexpr (RES == 1) acc += static_cast<const float*>(res)[t * d + i];
      else if constexpr (RES == 2) acc += bf16_to_f32(static_cast<const uint16_t*>(res)[t * d + i]);
      if constexpr (OUT_BF16) {
        static_cast<uint16_t*>(out)[t * d + i] = f32_to_bf16(acc);
      } else {
        static_cast<float*>(out)[t * d + i] = acc;
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void sum_partials_kernel(const float* __restrict__ part,
                                                               int nsplit, int64_t n,
                                                               float* __restrict__ y) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kThreads) {
    float v = part[i];
    for (int sp = 1; sp < nsplit; ++sp) v += part[sp * n + i];
    y[i] = v;
  }
}

}  // namespace

namespace {
template <int RES>
void launch_combine_res(const float* y, int nsplit, int64_t pstride, const int32_t* asg_pos,
                        const float* w, int64_t T, int d, int k, void* out, int out_bf16,
                        bool vec, const void* res, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>((d + kThreads * 4 - 1) / (kThreads * 4)));
  if (out_bf16) {
    if (vec)
      hipLaunchKernelGGL((combine_kernel<true, true, RES>), grid, dim3(kThreads), 0, s, y, nsplit,
                         pstride, asg_pos, w, d, k, out, res);
    else
      hipLaunchKernelGGL((combine_kernel<true, false, RES>), grid, dim3(kThreads), 0, s, y, nsplit,
                         pstride, asg_pos, w, d, k, out, res);
  } else {
    if (vec)
      hipLaunchKernelGGL((combine_kernel<false, true, RES>), grid, dim3(kThreads), 0, s, y, nsplit,
                         pstride, asg_pos, w, d, k, out, res);
    else
      hipLaunchKernelGGL((combine_kernel<false, false, RES>), grid, dim3(kThreads), 0, s, y,
                         nsplit, pstride, asg_pos, w, d, k, out, res);
  }
}
}  // namespace

hipError_t launch_combine(const float* y, int nsplit, const int32_t* asg_pos, const float* w,
                          int64_t T, int d, int k, void* out, int out_bf16, hipStream_t s,
                          const void* residual, int res_bf16) {
  if (T == 0) return hipSuccess;
  const int64_t pstride = T * k * static_cast<int64_t>(d);
  const auto aligned = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
  const bool vec = (d % 4 == 0) && aligned(y, 16) && aligned(out, out_bf16 ? 8 : 16) &&
                   (!residual || aligned(residual, res_bf16 ? 8 : 16));
  if (!residual)
    launch_combine_res<0>(y, nsplit, pstride, asg_pos, w, T, d, k, out, out_bf16, vec, nullptr, s);
  else if (res_bf16)
    launch_combine_res<2>(y, nsplit, pstride, asg_pos, w, T, d, k, out, out_bf16, vec, residual, s);
  else
    launch_combine_res<1>(y, nsplit, pstride, asg_pos, w, T, d, k, out, out_bf16, vec, residual, s);
  return hipGetLastError();
}

hipError_t launch_sum_partials(const float* part, int nsplit, int64_t n, float* y, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t want = (n + kThreads - 1) / kThreads;
  const unsigned blocks = static_cast<unsigned>(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(sum_partials_kernel, dim3(blocks), dim3(kThreads), 0, s, part, nsplit, n, y);
  return hipGetLastError();
}

}  // namespace moe
