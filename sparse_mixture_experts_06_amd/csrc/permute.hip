// Grouping of the T*k assignments by expert: per-expert counts, their
// exclusive prefix sum and a stable counting sort (each token is dispatched
// to its k experts: Transformers Mixtral page, "Architectural details").
//
// One workgroup of 16 waves does the whole job, so there is no
// inter-workgroup synchronisation and the result is deterministic. Wave w
// owns the contiguous slice of assignments [w C, (w+1) C), C = A / 16
// rounded up to a multiple of 64, and walks it in steps of 64:
//   1. counts: per step one ballot per expert; lane e keeps expert e's count
//      of the slice, written to LDS;
//   2. one thread per expert sums the slices' counts in slice order: counts,
//      offsets (exclusive scan over experts) and each slice's first position
//      per expert (offsets[e] + the counts of the earlier slices);
//   3. each wave walks its slice again: an assignment's position is its
//      slice's first position for its expert, plus the expert's count in the
//      earlier steps of the slice, plus its rank among the earlier lanes of
//      its step with the same expert (a ballot).
// Each walk loads 8 steps of ids at a time, all in flight before the first
// is used (one memory latency per 512 ids, not per 64).
// Slices, steps and lanes are all in increasing assignment order, so within
// an expert the assignments keep their order (a stable sort). Two barriers.
// Expert ids outside [0, E) are ignored (no out-of-bounds access).
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kSteps = 8;  // steps of 64 expert ids a wave loads at once

__global__ __launch_bounds__(kThreads) void permute_kernel(const int32_t* __restrict__ idx,
                                                           int A, int E,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_asg,
                                                           int32_t* __restrict__ asg_pos) {
  __shared__ int s_cnt[kWaves][kMaxExperts];   // slice counts, then slice first positions
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  // slice of this wave, in whole steps of 64 (A <= 2^31 - 1024, so no overflow)
  const int per = ((A + kWaves - 1) / kWaves + kWave - 1) / kWave * kWave;
  const int lo = min(A, wave * per), hi = min(A, lo + per);

  // the slice's expert ids are loaded kSteps steps of 64 at a time, all in
  // flight together, before any is used
  int cnt = 0;  // lane e: expert e's count in this slice
  for (int c0 = lo; c0 < hi; c0 += kSteps * kWave) {
    int ev[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int a = c0 + u * kWave + lane;
      ev[u] = a < hi ? idx[a] : -1;
    }
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      for (int ee = 0; ee < E; ++ee) {
        const int c = __popcll(__ballot(ev[u] == ee));
        if (lane == ee) cnt += c;
      }
    }
  }
  if (lane < E) s_cnt[wave][lane] = cnt;
  __syncthreads();

  if (tid < E) {
    int before = 0;  // assignments of lower experts
    for (int e = 0; e < tid; ++e)
      for (int w = 0; w < kWaves; ++w) before += s_cnt[w][e];
    int run = before;
    for (int w = 0; w < kWaves; ++w) {
      const int c = s_cnt[w][tid];
      s_cnt[w][tid] = run;
      run += c;
    }
    counts[tid] = run - before;
    offsets[tid] = before;
    if (tid == E - 1) offsets[E] = run;
  }
  __syncthreads();

  const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  int next = lane < E ? s_cnt[wave][lane] : 0;  // lane e: next position of expert e
  for (int c0 = lo; c0 < hi; c0 += kSteps * kWave) {
    int ev[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int a = c0 + u * kWave + lane;
      const int e = a < hi ? idx[a] : -1;
      ev[u] = e < E ? e : -1;
    }
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int a = c0 + u * kWave + lane;
      int pos = 0;
      for (int ee = 0; ee < E; ++ee) {
        const uint64_t m = __ballot(ev[u] == ee);
        const int first = __builtin_amdgcn_readlane(next, ee);
        if (ev[u] == ee) pos = first + __popcll(m & lower);
        if (lane == ee) next += __popcll(m);
      }
      if (ev[u] >= 0) {
        sorted_asg[pos] = a;
        asg_pos[a] = pos;
      }
    }
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
