// Grouping of the T*k assignments by expert: per-expert counts, their
// exclusive prefix sum and a stable counting sort (each token is dispatched
// to its k experts: Transformers Mixtral page, "Architectural details").
//
// One workgroup of 1024 threads does the whole job, so there is no
// inter-workgroup synchronisation and the result is deterministic:
//   1. counts with LDS integer atomics (the sum is order-independent);
//   2. offsets = exclusive scan of counts;
//   3. the assignments are walked in steps of 1024 in increasing order; in a
//      step, wave ballots give each assignment its rank among the earlier
//      lanes of its wave with the same expert, the per-wave totals give the
//      rank across waves, and a per-expert cursor carries the position from
//      step to step.
// Expert ids outside [0, E) are ignored (no out-of-bounds access).
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

__global__ __launch_bounds__(kThreads) void permute_kernel(const int32_t* __restrict__ idx,
                                                           int A, int E,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_asg,
                                                           int32_t* __restrict__ asg_pos) {
  __shared__ int s_count[kMaxExperts];
  __shared__ int s_cursor[kMaxExperts];
  __shared__ int s_wave[kWaves][kMaxExperts];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  if (tid < kMaxExperts) s_count[tid] = 0;
  __syncthreads();

  for (int a = tid; a < A; a += kThreads) {
    const int e = idx[a];
    if (e >= 0 && e < E) atomicAdd(&s_count[e], 1);
  }
  __syncthreads();

  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      const int c = s_count[e];
      counts[e] = c;
      offsets[e] = run;
      s_cursor[e] = run;
      run += c;
    }
    offsets[E] = run;
  }
  __syncthreads();

  const uint64_t lower_lanes = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int base = 0; base < A; base += kThreads) {
    const int a = base + tid;
    int e = (a < A) ? idx[a] : -1;
    if (e < 0 || e >= E) e = -1;
    int rank = 0;
    for (int ee = 0; ee < E; ++ee) {
      const uint64_t mask = __ballot(e == ee);
      if (e == ee) rank = __popcll(mask & lower_lanes);
      if (lane == 0) s_wave[wave][ee] = __popcll(mask);
    }
    __syncthreads();
    if (e >= 0) {
      int pos = s_cursor[e] + rank;
      for (int w = 0; w < wave; ++w) pos += s_wave[w][e];
      sorted_asg[pos] = a;
      asg_pos[a] = pos;
    }
    __syncthreads();
    if (tid < E) {
      int tot = 0;
      for (int w = 0; w < kWaves; ++w) tot += s_wave[w][tid];
      s_cursor[tid] += tot;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_permute(const int32_t* idx, int64_t A, int E, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_asg, int32_t* asg_pos,
                          hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kThreads), 0, s, idx, static_cast<int>(A), E,
                     counts, offsets, sorted_asg, asg_pos);
  return hipGetLastError();
}

}  // namespace moe
