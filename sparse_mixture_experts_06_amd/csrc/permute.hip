// Grouping of the T*k assignments by expert: per-expert counts, their
// exclusive prefix sum and a stable counting sort (each token is dispatched
// to its k experts: Transformers Mixtral page, "Architectural details").
//
// One workgroup of 16 waves does the whole job, so there is no
// inter-workgroup synchronisation and the result is deterministic. Wave w
// owns the contiguous slice of assignments [w C, (w+1) C), C = A / 16
// rounded up to a multiple of 64, and walks it in steps of 64. In a step,
// each lane finds the lanes holding the same expert id as its own from one
// ballot per bit of the id (an id has at most 5 bits, E <= 32): the AND of
// the ballots its bits select; its rank in the step is the number of those
// lanes below it, and the lowest of them (rank 0) speaks for the group.
//   1. counts: the speaking lane of each group adds the group's size to its
//      expert's count of the slice in LDS;
//   2. one thread per expert sums the slices' counts in slice order: counts,
//      offsets (exclusive scan over experts) and each slice's first position
//      per expert (offsets[e] + the counts of the earlier slices), written to
//      an array of their own (the counts stay unchanged while other threads
//      read them);
//   3. each wave walks its slice again: an assignment's position is the
//      running position of its expert in the slice (its slice's first
//      position plus the expert's count in the earlier steps) plus its rank;
//      the speaking lane then advances the running position.
// Slices, steps and lanes are all in increasing assignment order, so within
// an expert the assignments keep their order (a stable sort). Each walk
// loads 8 steps of ids at a time, all in flight before the first is used;
// when a wave's slice is one such batch (A <= 8192), the second walk reuses
// the ids the first loaded.
// Two barriers (after zeroing the counts, one more). Expert ids outside
// [0, E) take no place in the grouping: they are not counted, and their
// asg_pos entry is -1 (which the combine skips), so a bad id never leads to
// an access out of bounds.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kSteps = 8;  // steps of 64 expert ids a wave loads at once

// lanes of the wave whose id equals this lane's (valid lanes only; nb = bits of
// an id): the AND, over the nb bits, of the ballot of lanes with that bit set
// or of its complement
__device__ __forceinline__ uint64_t same_id_lanes(int e, bool valid, int nb) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nb; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t set = __ballot(valid && bit);
    m &= bit ? set : ~set;
  }
  return m;
}

__global__ __launch_bounds__(kThreads) void permute_kernel(const int32_t* __restrict__ idx,
                                                           int A, int E,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_asg,
                                                           int32_t* __restrict__ asg_pos) {
  __shared__ int s_cnt[kWaves][kMaxExperts];  // count of each expert in each slice
  __shared__ int s_pos[kWaves][kMaxExperts];  // each slice's running position per expert
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  if (tid < kWaves * kMaxExperts) (&s_cnt[0][0])[tid] = 0;
  __syncthreads();
  int nb = 0;  // bits of the largest id
  while ((1 << nb) < E) ++nb;
  const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  // slice of this wave, in whole steps of 64 (A <= 2^31 - 1024, so no overflow)
  const int per = ((A + kWaves - 1) / kWaves + kWave - 1) / kWave * kWave;
  const int lo = min(A, wave * per), hi = min(A, lo + per);

  // a slice of at most one batch (A <= 8192) keeps its ids in registers for
  // the second walk
  const bool one_batch = hi - lo <= kSteps * kWave;
  int ev0[kSteps];
  for (int c0 = lo; c0 < hi; c0 += kSteps * kWave) {
    int ev[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int a = c0 + u * kWave + lane;
      ev[u] = a < hi ? idx[a] : -1;
      ev0[u] = ev[u];
    }
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const bool valid = ev[u] >= 0 && ev[u] < E;
      const uint64_t m = same_id_lanes(ev[u], valid, nb);
      if (valid && (m & lower) == 0) s_cnt[wave][ev[u]] += __popcll(m);
    }
  }
  __syncthreads();

  if (tid < E) {
    int before = 0;  // assignments of lower experts
    for (int e = 0; e < tid; ++e)
      for (int w = 0; w < kWaves; ++w) before += s_cnt[w][e];
    int run = before;
    for (int w = 0; w < kWaves; ++w) {
      s_pos[w][tid] = run;
      run += s_cnt[w][tid];
    }
    counts[tid] = run - before;
    offsets[tid] = before;
    if (tid == E - 1) offsets[E] = run;
  }
  __syncthreads();

  for (int c0 = lo; c0 < hi; c0 += kSteps * kWave) {
    int ev[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int a = c0 + u * kWave + lane;
      ev[u] = one_batch ? ev0[u] : a < hi ? idx[a] : -1;
    }
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int a = c0 + u * kWave + lane;
      const bool valid = ev[u] >= 0 && ev[u] < E;
      const uint64_t m = same_id_lanes(ev[u], valid, nb);
      if (valid) {
        const uint64_t below = m & lower;
        const int pos = s_pos[wave][ev[u]] + __popcll(below);
        sorted_asg[pos] = a;
        asg_pos[a] = pos;
        if (below == 0) s_pos[wave][ev[u]] = pos + __popcll(m);
      } else if (a < hi) {
        asg_pos[a] = -1;
      }
    }
  }
}

// Routing check (a debugging aid for callers that pass their own expert ids):
// bad[0] = tokens with an id outside [0, E), bad[1] = tokens whose ids repeat
// one (a token goes to k distinct experts). One workgroup strides over the
// tokens; the per-thread counts are summed in LDS, so the result is exact and
// needs no zeroed output.
__global__ __launch_bounds__(kThreads) void check_routing_kernel(const int32_t* __restrict__ idx,
                                                                 int64_t T, int k, int E,
                                                                 int32_t* __restrict__ bad) {
  __shared__ int s_bad[2][kWaves];
  const int tid = threadIdx.x;
  int out_of_range = 0, repeated = 0;
  for (int64_t t = tid; t < T; t += kThreads) {
    uint32_t seen = 0;
    bool oor = false, rep = false;
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e < 0 || e >= E) {
        oor = true;
      } else {
        rep = rep || ((seen >> e) & 1u);
        seen |= 1u << e;
      }
    }
    out_of_range += oor;
    repeated += rep;
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    out_of_range += __shfl_xor(out_of_range, o, kWave);
    repeated += __shfl_xor(repeated, o, kWave);
  }
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  if (lane == 0) {
    s_bad[0][wave] = out_of_range;
    s_bad[1][wave] = repeated;
  }
  __syncthreads();
  if (tid < 2) {
    int sum = 0;
    for (int w = 0; w < kWaves; ++w) sum += s_bad[tid][w];
    bad[tid] = sum;
  }
}

}  // namespace

hipError_t launch_check_routing(const int32_t* idx, int64_t T, int k, int E, int32_t* bad,
                                hipStream_t s) {
  hipLaunchKernelGGL(check_routing_kernel, dim3(1), dim3(kThreads), 0, s, idx, T, k, E, bad);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int64_t A, int E, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_asg, int32_t* asg_pos,
                          hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kThreads), 0, s, idx, static_cast<int>(A), E,
                     counts, offsets, sorted_asg, asg_pos);
  return hipGetLastError();
}

}  // namespace moe
