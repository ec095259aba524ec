// Expert SwiGLU on bf16 MFMA (nnterp Mixtral page, support(): the down
// projection receives act(gate) * up with act = SiLU; section "expert_outputs
// needs the default experts implementation": the 8 experts are one stacked
// module).
//
//   gate/up:  h[p, n] = silu(sum_i x[r,i] w1[e,n,i]) * (sum_i x[r,i] w3[e,n,i])
//             r = sorted_asg[p] / k,  p in expert e's grouped range; h is bf16
//   down:     y[p, n] = sum_f h[p,f] w2[e,n,f]                      y is f32
//
// Both are grouped GEMMs whose two operands are "row x K" with K contiguous
// (weight rows n, token rows m), so the weights are the MFMA A operand and the
// tokens the B operand: D[n][m] = W[n,:] . X[m,:]. With
// v_mfma_f32_16x16x32_bf16 a lane (r = lane % 16, g = lane / 16) holds the 8
// values k = 8g .. 8g+7 of row r of either operand, and the result rows
// 4g .. 4g+3 of token column r, which gives 8-byte (h) and 16-byte (y) stores.
//
// Weight layouts (template parameter PACKED):
//  * standard: w[e][n][k], k contiguous.
//  * fragment order (moe_pack_weight): the matrix is cut into 16-row x 32-k
//    fragments, each stored as 1 KiB in MFMA lane order (lane l's 8 values at
//    byte 16*l), fragments ordered (expert, row tile, k step). A wave's load
//    of one A fragment is then one contiguous KiB, the friendliest access for
//    HBM3E; the values are the same, only their order differs.
//
// Two kernel families:
//  * streaming (few rows per expert, decode): no LDS staging of weights.
//    gate/up: a workgroup owns RT 16-row tiles of w1 and w3; its 4 waves split
//    K and stream those rows once with 16-byte loads, each token fragment
//    serving 2*RT weight fragments; the partial sums meet in LDS.
//    down: every wave is independent: RT 16-row tiles of w2 over 1/nsplit of
//    K, written as a float32 partial; the partials are summed later in a
//    fixed order (by the combine, or by moe_expert_ffn before it returns).
//    With fragment-order weights the weight loads are non-temporal.
//  * tiled (many rows per expert, prefill). When experts average half a
//    256-row tile or more for gate/up (A >= 128 E) and a full one for down
//    (A >= 256 E; d and ffn multiples of 128, and for down d % 256 == 0) the
//    256x256-tile direct-to-LDS kernels of ffn_dma.hip run, for either
//    layout. Below that: with fragment-order weights wtiled_kernel (256
//    weight rows x 128 tokens, weights straight into registers), with
//    the standard layout tiled_kernel: 128 weight rows x 128 token rows x 64
//    K per step, double-buffered in LDS with an XOR swizzle of the 16-byte
//    chunks (conflict-free ds_read_b128 for the MFMA fragments); 4 waves each
//    own a 64x64 block of 4x4 MFMA tiles. Tiles are listed expert by expert,
//    n-tile by n-tile, m-tile by m-tile, and consecutive tiles go to the same
//    XCD so the m-tiles sharing a weight tile meet in that XCD's L2.
#include <type_traits>
#include <utility>

#include "common.h"

namespace moe {
namespace {

// elements between one lane's values of consecutive 32-wide k steps
template <bool PACKED>
constexpr int kStep32() { return PACKED ? 512 : 32; }

// 16-byte weight load; NT marks it non-temporal (streamed once, not kept)
template <bool NT>
__device__ __forceinline__ u32x4 ldw(const uint16_t* p) {
  if constexpr (NT) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  } else {
    return ldg16(p);
  }
}

// ----------------------------------------------------------------------------
// weight packing
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ w, int64_t chunks,
                                                   int R, int C, uint16_t* __restrict__ out) {
  const int nrt = R >> 4;
  const int S = C >> 5;
  for (int64_t o = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; o < chunks;
       o += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t f = o >> 6;
    const int lane = static_cast<int>(o & 63);
    const int s = static_cast<int>(f % S);
    const int64_t t = f / S;
    const int rt = static_cast<int>(t % nrt);
    const int64_t e = t / nrt;
    const uint16_t* src = w + (e * R + rt * 16 + (lane & 15)) * C + s * 32 + (lane >> 4) * 8;
    *reinterpret_cast<u32x4*>(out + o * 8) = ldg16(src);
  }
}

// ----------------------------------------------------------------------------
// streaming kernels
// ----------------------------------------------------------------------------
constexpr int kStreamWaves = 4;

// The grouping of the assignments by expert, from the expert ids alone, for
// few assignments (A <= kFusedPermuteMaxA): the same stable counting sort as
// permute.hip (assignments of an expert in increasing id order; ids outside
// [0, E) ignored), by wave ballots over the ids in steps of 64.
// count_expert: the first grouped row `beg` of expert e (assignments of lower
// experts) and its count M.
__device__ __forceinline__ void count_expert(const int32_t* __restrict__ idx, int A, int e,
                                             int lane, int& beg, int& M) {
  beg = 0;
  M = 0;
  for (int a0 = 0; a0 < A; a0 += kWave) {
    const int a = a0 + lane;
    const int ea = a < A ? idx[a] : -1;
    beg += __popcll(__ballot(ea >= 0 && ea < e));
    M += __popcll(__ballot(ea == e));
  }
}

// rank_expert: row(rank, a) for each assignment a of expert e, rank = its
// position among the expert's assignments
template <typename F>
__device__ __forceinline__ void rank_expert(const int32_t* __restrict__ idx, int A, int e, int lane,
                                            F&& row) {
  const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  int M = 0;
  for (int a0 = 0; a0 < A; a0 += kWave) {
    const int a = a0 + lane;
    const int ea = a < A ? idx[a] : -1;
    const uint64_t eq = __ballot(ea == e);
    if (ea == e) row(M + __popcll(eq & lower), a);
    M += __popcll(eq);
  }
}

// Start of a streaming gate/up workgroup that does the permutation itself:
// the waves of workgroup (0, 0) write counts, offsets, sorted_asg and
// asg_pos for the kernels that follow; in every workgroup wave 0 puts the
// token rows of expert e, in grouped order, into s_rows. Returns the expert's
// first grouped row and its row count (every wave; one barrier).
__device__ __forceinline__ void fused_permute(const FusedPermute& fp, int A, int E, int e,
                                              int ktop, int lane, int wave, int* s_rows,
                                              int* s_begm, int& beg, int& M) {
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int ee = wave; ee < E; ee += kStreamWaves) {
      int b, m;
      count_expert(fp.idx, A, ee, lane, b, m);
      rank_expert(fp.idx, A, ee, lane, [&](int rank, int a) {
        fp.sorted_asg[b + rank] = a;
        fp.asg_pos[a] = b + rank;
      });
      if (lane == 0) {
        fp.counts[ee] = m;
        fp.offsets[ee] = b;
        if (ee == E - 1) fp.offsets[E] = b + m;
      }
    }
  }
  if (wave == 0) {
    int b, m;
    count_expert(fp.idx, A, e, lane, b, m);
    rank_expert(fp.idx, A, e, lane, [&](int rank, int a) { s_rows[rank] = a / ktop; });
    if (lane == 0) {
      s_begm[0] = b;
      s_begm[1] = m;
    }
  }
  __syncthreads();
  beg = s_begm[0];
  M = s_begm[1];
}

// x [T, K=d] rows gathered through sorted_asg / ktop; w1, w3 [E, N=ffn, K];
// h bf16 [A, N]. Token rows go 32 at a time (two 16-row MFMA column tiles;
// the second is skipped when the rows run out).
// FUSED: the permutation is done here instead of by a kernel of its own (few
// assignments: the expert ids fp.idx [A] of E experts), by fused_permute;
// offsets and sorted_asg are not read then.
template <int RT, int U, bool PACKED, bool NT, bool FUSED>
__global__ __launch_bounds__(kWave* kStreamWaves) void gate_up_stream_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w1,
    const uint16_t* __restrict__ w3, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_asg, int K, int N, int ktop, uint16_t* __restrict__ h,
    FusedPermute fp, int A, int E) {
  const int e = blockIdx.y;
  const int n0 = blockIdx.x * (16 * RT);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  __shared__ int s_rows[FUSED ? kFusedPermuteMaxA : 1];
  __shared__ int s_begm[2];
  int beg, M;
  if constexpr (FUSED) {
    fused_permute(fp, A, E, e, ktop, lane, wave, s_rows, s_begm, beg, M);
  } else {
    beg = offsets[e];
    M = offsets[e + 1] - beg;
  }
  if (M <= 0) return;
  // token row of the expert's m-th assignment
  auto token = [&](int m) { return FUSED ? s_rows[m] : sorted_asg[beg + m] / ktop; };
  const int r = lane & 15;
  const int g = lane >> 4;
  const int S = K / 32;
  const int s_lo = (wave * S) / kStreamWaves;
  const int s_hi = ((wave + 1) * S) / kStreamWaves;
  constexpr int ST = kStep32<PACKED>();
  const uint16_t* pg[RT];
  const uint16_t* pu[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const size_t o = wofs<PACKED>(e, n0 + t * 16 + r, g * 8, N, K);
    pg[t] = w1 + o;
    pu[t] = w3 + o;
  }

  __shared__ f32x4 red[kStreamWaves - 1][2][RT][2][kWave];

  for (int mb = 0; mb < M; mb += 32) {
    const bool two = (M - mb) > 16;  // wave-uniform
    const int m0 = min(mb + r, M - 1);
    const int m1 = min(mb + 16 + r, M - 1);
    const uint16_t* px0 = x + static_cast<int64_t>(token(m0)) * K + g * 8;
    const uint16_t* px1 = x + static_cast<int64_t>(token(m1)) * K + g * 8;

    f32x4 ag[RT][2], au[RT][2];
#pragma unroll
    for (int t = 0; t < RT; ++t)
      ag[t][0] = ag[t][1] = au[t][0] = au[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    int s = s_lo;
    for (; s + U <= s_hi; s += U) {
      u32x4 G[U][RT], V[U][RT], B0[U], B1[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          G[u][t] = ldw<NT>(pg[t] + (s + u) * ST);
          V[u][t] = ldw<NT>(pu[t] + (s + u) * ST);
        }
        B0[u] = ldg16(px0 + (s + u) * 32);
        B1[u] = two ? ldg16(px1 + (s + u) * 32) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          ag[t][0] = mfma16x16x32(G[u][t], B0[u], ag[t][0]);
          au[t][0] = mfma16x16x32(V[u][t], B0[u], au[t][0]);
          if (two) {
            ag[t][1] = mfma16x16x32(G[u][t], B1[u], ag[t][1]);
            au[t][1] = mfma16x16x32(V[u][t], B1[u], au[t][1]);
          }
        }
      }
    }
    for (; s < s_hi; ++s) {
      const u32x4 b0 = ldg16(px0 + s * 32);
      const u32x4 b1 = two ? ldg16(px1 + s * 32) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const u32x4 gw = ldw<NT>(pg[t] + s * ST);
        const u32x4 uw = ldw<NT>(pu[t] + s * ST);
        ag[t][0] = mfma16x16x32(gw, b0, ag[t][0]);
        au[t][0] = mfma16x16x32(uw, b0, au[t][0]);
        if (two) {
          ag[t][1] = mfma16x16x32(gw, b1, ag[t][1]);
          au[t][1] = mfma16x16x32(uw, b1, au[t][1]);
        }
      }
    }

    if (wave > 0) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        red[wave - 1][0][t][0][lane] = ag[t][0];
        red[wave - 1][1][t][0][lane] = au[t][0];
        if (two) {
          red[wave - 1][0][t][1][lane] = ag[t][1];
          red[wave - 1][1][t][1][lane] = au[t][1];
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < kStreamWaves - 1; ++w)
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          ag[t][0] += red[w][0][t][0][lane];
          au[t][0] += red[w][1][t][0][lane];
          if (two) {
            ag[t][1] += red[w][0][t][1][lane];
            au[t][1] += red[w][1][t][1][lane];
          }
        }
      // lane holds token column r and weight rows 4g .. 4g+3 of each tile
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int m = mb + c * 16 + r;
        if (m < M) {
#pragma unroll
          for (int t = 0; t < RT; ++t) {
            const f32x4 gt = ag[t][c];
            const f32x4 up = au[t][c];
            uint2 v;
            v.x = pack_bf16x2(silu_f32(gt[0]) * up[0], silu_f32(gt[1]) * up[1]);
            v.y = pack_bf16x2(silu_f32(gt[2]) * up[2], silu_f32(gt[3]) * up[3]);
            *reinterpret_cast<uint2*>(h + static_cast<size_t>(beg + m) * N + n0 + t * 16 + 4 * g) =
                v;
          }
        }
      }
    }
    __syncthreads();
  }
}

// h [A, K=ffn] in grouped order; w2 [E, N=d, K]; part [nsplit, A, N] f32.
// Wave task = (row group of RT 16-row tiles, split sp); no barriers, so a
// wave with no task simply returns.
template <int RT, int U, bool PACKED, bool NT>
__global__ __launch_bounds__(kWave* kStreamWaves) void down_stream_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ offsets, int K, int N, int A, int nsplit,
    float* __restrict__ part) {
  const int e = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int task = blockIdx.x * kStreamWaves + static_cast<int>(threadIdx.x) / kWave;
  const int ngroups = N / (16 * RT);
  if (task >= ngroups * nsplit) return;
  const int sp = task % nsplit;
  const int n0 = (task / nsplit) * (16 * RT);
  const int beg = offsets[e];
  const int M = offsets[e + 1] - beg;
  if (M <= 0) return;

  const int r = lane & 15;
  const int g = lane >> 4;
  const int S = K / 32;
  const int s_lo = (sp * S) / nsplit;
  const int s_hi = ((sp + 1) * S) / nsplit;
  constexpr int ST = kStep32<PACKED>();
  const uint16_t* pw[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) pw[t] = w2 + wofs<PACKED>(e, n0 + t * 16 + r, g * 8, N, K);
  float* dst = part + static_cast<size_t>(sp) * A * N;

  for (int mb = 0; mb < M; mb += 32) {
    const bool two = (M - mb) > 16;
    const uint16_t* px0 = h + static_cast<int64_t>(beg + min(mb + r, M - 1)) * K + g * 8;
    const uint16_t* px1 = h + static_cast<int64_t>(beg + min(mb + 16 + r, M - 1)) * K + g * 8;
    f32x4 acc[RT][2];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t][0] = acc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    int s = s_lo;
    for (; s + U <= s_hi; s += U) {
      u32x4 W[U][RT], B0[U], B1[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int t = 0; t < RT; ++t) W[u][t] = ldw<NT>(pw[t] + (s + u) * ST);
        B0[u] = ldg16(px0 + (s + u) * 32);
        B1[u] = two ? ldg16(px1 + (s + u) * 32) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          acc[t][0] = mfma16x16x32(W[u][t], B0[u], acc[t][0]);
          if (two) acc[t][1] = mfma16x16x32(W[u][t], B1[u], acc[t][1]);
        }
    }
    for (; s < s_hi; ++s) {
      const u32x4 b0 = ldg16(px0 + s * 32);
      const u32x4 b1 = two ? ldg16(px1 + s * 32) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const u32x4 w = ldw<NT>(pw[t] + s * ST);
        acc[t][0] = mfma16x16x32(w, b0, acc[t][0]);
        if (two) acc[t][1] = mfma16x16x32(w, b1, acc[t][1]);
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int m = mb + c * 16 + r;
      if (m < M) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
          *reinterpret_cast<f32x4*>(dst + static_cast<size_t>(beg + m) * N + n0 + t * 16 + 4 * g) =
              acc[t][c];
      }
    }
  }
}

// ----------------------------------------------------------------------------
// streaming kernels for standard-layout weights, whole cache lines per load
// ----------------------------------------------------------------------------
// A weight fragment (16 rows x 32 k) read straight from the standard layout
// is 16 half cache lines (64 B of each row), and the other halves come with
// the next k step's load: measured on MI355X, that access streams at 6.2 TB/s
// with or without the non-temporal hint, while loads of whole 128-byte lines
// (8 rows x 128 B per wave load) reach 7.0 TB/s with it. These kernels load
// whole lines and rearrange them through a small LDS buffer of each wave:
// one 64-wide k block of 16 rows is two wave loads; lane l of the load for
// rows 8q .. 8q+7 takes row 8q + l/8 and 16-byte chunk (l % 8) ^ ((row / 2)
// % 8) of the block, and writes it to slot l of a 1 KiB LDS area (lane
// order); the MFMA operand of k step s (chunk 4s + g of row r for lane
// 16g + r) is then read from slot 8 (r % 8) + ((4s + g) ^ ((r / 2) % 8)) of
// area q = r / 8: the swizzle puts the 16 rows of a fragment read on 16
// different bank groups. The operands, and the MFMAs and their order, are
// those of the kernels above on fragment-order weights, so both layouts give
// the same bits. A wave's k range must be whole 64-wide blocks.
constexpr int kRmBlocks = 4;  // 64-wide k blocks in flight per wave (8 k steps)

// this lane's element offsets, within a 16-row tile, of its two line loads
// (rows 0-7 and 8-15) of k block 0
__device__ __forceinline__ void rm_load_offsets(int lane, int K, int (&off)[2]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 8 * q + (lane >> 3);
    off[q] = row * K + (((lane & 7) ^ ((row >> 1) & 7)) << 3);
  }
}

// byte offset in a wave's LDS buffer of this lane's operand for k step s of
// 16-row tile t (areas 2t and 2t + 1 hold its rows 0-7 and 8-15)
__device__ __forceinline__ int rm_read_offset(int lane, int t, int s) {
  const int r = lane & 15, g = lane >> 4;
  return ((2 * t + (r >> 3)) * 64 + 8 * (r & 7) + ((4 * s + g) ^ ((r >> 1) & 7))) * 16;
}

// gate/up as gate_up_stream_kernel (RT = 1: 16 rows of w1 and of w3 per
// workgroup, 4 waves splitting K = d; FUSED as there), standard-layout
// weights loaded in whole lines.
template <bool FUSED>
__global__ __launch_bounds__(kWave* kStreamWaves) void gate_up_stream_rm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w1,
    const uint16_t* __restrict__ w3, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_asg, int K, int N, int ktop, uint16_t* __restrict__ h,
    FusedPermute fp, int A, int E) {
  const int e = blockIdx.y;
  const int n0 = blockIdx.x * 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  __shared__ int s_rows[FUSED ? kFusedPermuteMaxA : 1];
  __shared__ int s_begm[2];
  __shared__ __attribute__((aligned(16))) uint8_t stg[kStreamWaves][4096];
  __shared__ f32x4 red[kStreamWaves - 1][2][2][kWave];
  int beg, M;
  if constexpr (FUSED) {
    fused_permute(fp, A, E, e, ktop, lane, wave, s_rows, s_begm, beg, M);
  } else {
    beg = offsets[e];
    M = offsets[e + 1] - beg;
  }
  if (M <= 0) return;
  auto token = [&](int m) { return FUSED ? s_rows[m] : sorted_asg[beg + m] / ktop; };

  const int r = lane & 15;
  const int g = lane >> 4;
  const int S = K / 32;
  const int b_lo = (wave * S) / kStreamWaves / 2;  // 64-wide k blocks of this wave
  const int b_hi = ((wave + 1) * S) / kStreamWaves / 2;
  int off[2];
  rm_load_offsets(lane, K, off);
  const uint16_t* pg = w1 + (static_cast<size_t>(e) * N + n0) * K;
  const uint16_t* pu = w3 + (static_cast<size_t>(e) * N + n0) * K;
  uint8_t* buf = stg[wave];
  const int rd0 = rm_read_offset(lane, 0, 0), rd1 = rm_read_offset(lane, 0, 1);

  for (int mb = 0; mb < M; mb += 32) {
    const bool two = (M - mb) > 16;  // wave-uniform
    const int m0 = min(mb + r, M - 1);
    const int m1 = min(mb + 16 + r, M - 1);
    const uint16_t* px0 = x + static_cast<int64_t>(token(m0)) * K + g * 8;
    const uint16_t* px1 = x + static_cast<int64_t>(token(m1)) * K + g * 8;
    f32x4 ag[2], au[2];
    ag[0] = ag[1] = au[0] = au[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // one 64-wide k block: the line loads (issued by the caller) into LDS,
    // its four operands back, and the MFMAs of its two k steps
    auto consume = [&](const u32x4 (&W)[4], const u32x4 (&B0)[2], const u32x4 (&B1)[2]) {
#pragma unroll
      for (int i = 0; i < 4; ++i)  // areas: w1 rows 0-7, 8-15, w3 rows 0-7, 8-15
        *reinterpret_cast<u32x4*>(buf + (i * 64 + lane) * 16) = W[i];
      const u32x4 G0 = *reinterpret_cast<const u32x4*>(buf + rd0);
      const u32x4 G1 = *reinterpret_cast<const u32x4*>(buf + rd1);
      const u32x4 V0 = *reinterpret_cast<const u32x4*>(buf + 2048 + rd0);
      const u32x4 V1 = *reinterpret_cast<const u32x4*>(buf + 2048 + rd1);
      ag[0] = mfma16x16x32(G0, B0[0], ag[0]);
      au[0] = mfma16x16x32(V0, B0[0], au[0]);
      if (two) {
        ag[1] = mfma16x16x32(G0, B1[0], ag[1]);
        au[1] = mfma16x16x32(V0, B1[0], au[1]);
      }
      ag[0] = mfma16x16x32(G1, B0[1], ag[0]);
      au[0] = mfma16x16x32(V1, B0[1], au[0]);
      if (two) {
        ag[1] = mfma16x16x32(G1, B1[1], ag[1]);
        au[1] = mfma16x16x32(V1, B1[1], au[1]);
      }
    };
    auto load = [&](int b, u32x4 (&W)[4], u32x4 (&B0)[2], u32x4 (&B1)[2]) {
      W[0] = ldw<true>(pg + off[0] + b * 64);
      W[1] = ldw<true>(pg + off[1] + b * 64);
      W[2] = ldw<true>(pu + off[0] + b * 64);
      W[3] = ldw<true>(pu + off[1] + b * 64);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        B0[s2] = ldg16(px0 + (2 * b + s2) * 32);
        B1[s2] = two ? ldg16(px1 + (2 * b + s2) * 32) : u32x4{0u, 0u, 0u, 0u};
      }
    };
    int b = b_lo;
    for (; b + kRmBlocks <= b_hi; b += kRmBlocks) {
      u32x4 W[kRmBlocks][4], B0[kRmBlocks][2], B1[kRmBlocks][2];
#pragma unroll
      for (int u = 0; u < kRmBlocks; ++u) load(b + u, W[u], B0[u], B1[u]);
#pragma unroll
      for (int u = 0; u < kRmBlocks; ++u) consume(W[u], B0[u], B1[u]);
    }
    for (; b < b_hi; ++b) {
      u32x4 W[4], B0[2], B1[2];
      load(b, W, B0, B1);
      consume(W, B0, B1);
    }

    if (wave > 0) {
      red[wave - 1][0][0][lane] = ag[0];
      red[wave - 1][1][0][lane] = au[0];
      if (two) {
        red[wave - 1][0][1][lane] = ag[1];
        red[wave - 1][1][1][lane] = au[1];
      }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < kStreamWaves - 1; ++w) {
        ag[0] += red[w][0][0][lane];
        au[0] += red[w][1][0][lane];
        if (two) {
          ag[1] += red[w][0][1][lane];
          au[1] += red[w][1][1][lane];
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int m = mb + c * 16 + r;
        if (m < M) {
          const f32x4 gt = ag[c];
          const f32x4 up = au[c];
          uint2 v;
          v.x = pack_bf16x2(silu_f32(gt[0]) * up[0], silu_f32(gt[1]) * up[1]);
          v.y = pack_bf16x2(silu_f32(gt[2]) * up[2], silu_f32(gt[3]) * up[3]);
          *reinterpret_cast<uint2*>(h + static_cast<size_t>(beg + m) * N + n0 + 4 * g) = v;
        }
      }
    }
    __syncthreads();
  }
}

// down as down_stream_kernel (RT = 2: 32 rows of w2 per wave, each wave its
// own task over 1/nsplit of K = ffn), standard-layout weights loaded in whole
// lines.
__global__ __launch_bounds__(kWave* kStreamWaves) void down_stream_rm_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ offsets, int K, int N, int A, int nsplit,
    float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t stg[kStreamWaves][4096];
  const int e = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = static_cast<int>(threadIdx.x) / kWave;
  const int task = blockIdx.x * kStreamWaves + wave;
  const int ngroups = N / 32;
  if (task >= ngroups * nsplit) return;
  const int sp = task % nsplit;
  const int n0 = (task / nsplit) * 32;
  const int beg = offsets[e];
  const int M = offsets[e + 1] - beg;
  if (M <= 0) return;

  const int r = lane & 15;
  const int g = lane >> 4;
  const int S = K / 32;
  const int b_lo = (sp * S) / nsplit / 2;
  const int b_hi = ((sp + 1) * S) / nsplit / 2;
  int off[2];
  rm_load_offsets(lane, K, off);
  const uint16_t* pw = w2 + (static_cast<size_t>(e) * N + n0) * K;
  const size_t tile1 = static_cast<size_t>(16) * K;  // rows 16-31
  uint8_t* buf = stg[wave];
  int rd[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) rd[t][s2] = rm_read_offset(lane, t, s2);
  float* dst = part + static_cast<size_t>(sp) * A * N;

  for (int mb = 0; mb < M; mb += 32) {
    const bool two = (M - mb) > 16;
    const uint16_t* px0 = h + static_cast<int64_t>(beg + min(mb + r, M - 1)) * K + g * 8;
    const uint16_t* px1 = h + static_cast<int64_t>(beg + min(mb + 16 + r, M - 1)) * K + g * 8;
    f32x4 acc[2][2];
    acc[0][0] = acc[0][1] = acc[1][0] = acc[1][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto consume = [&](const u32x4 (&W)[4], const u32x4 (&B0)[2], const u32x4 (&B1)[2]) {
#pragma unroll
      for (int i = 0; i < 4; ++i)  // areas: rows 0-7, 8-15, 16-23, 24-31
        *reinterpret_cast<u32x4*>(buf + (i * 64 + lane) * 16) = W[i];
      u32x4 F[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) F[t][s2] = *reinterpret_cast<const u32x4*>(buf + rd[t][s2]);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          acc[t][0] = mfma16x16x32(F[t][s2], B0[s2], acc[t][0]);
          if (two) acc[t][1] = mfma16x16x32(F[t][s2], B1[s2], acc[t][1]);
        }
    };
    auto load = [&](int b, u32x4 (&W)[4], u32x4 (&B0)[2], u32x4 (&B1)[2]) {
      W[0] = ldw<true>(pw + off[0] + b * 64);
      W[1] = ldw<true>(pw + off[1] + b * 64);
      W[2] = ldw<true>(pw + tile1 + off[0] + b * 64);
      W[3] = ldw<true>(pw + tile1 + off[1] + b * 64);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        B0[s2] = ldg16(px0 + (2 * b + s2) * 32);
        B1[s2] = two ? ldg16(px1 + (2 * b + s2) * 32) : u32x4{0u, 0u, 0u, 0u};
      }
    };
    int b = b_lo;
    for (; b + kRmBlocks <= b_hi; b += kRmBlocks) {
      u32x4 W[kRmBlocks][4], B0[kRmBlocks][2], B1[kRmBlocks][2];
#pragma unroll
      for (int u = 0; u < kRmBlocks; ++u) load(b + u, W[u], B0[u], B1[u]);
#pragma unroll
      for (int u = 0; u < kRmBlocks; ++u) consume(W[u], B0[u], B1[u]);
    }
    for (; b < b_hi; ++b) {
      u32x4 W[4], B0[2], B1[2];
      load(b, W, B0, B1);
      consume(W, B0, B1);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int m = mb + c * 16 + r;
      if (m < M) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
          *reinterpret_cast<f32x4*>(dst + static_cast<size_t>(beg + m) * N + n0 + t * 16 + 4 * g) =
              acc[t][c];
      }
    }
  }
}

// tuned on the Mixtral-8x7B decode shapes (weights streamed once per call)
constexpr int kGateUpRT = 1, kGateUpU = 8;
constexpr int kDownRT = 2, kDownU = 8;
// non-temporal weight loads pay off when each wave load is one contiguous KiB
// (fragment order); on the standard layout's 16 rows x 64 B pattern they cost
template <bool PACKED>
constexpr bool kStreamNT = PACKED;

// ----------------------------------------------------------------------------
// tiled kernels
// ----------------------------------------------------------------------------
constexpr int BM = 128;  // token rows per tile (MFMA B operand)
constexpr int BN = 128;  // weight rows per tile (MFMA A operand)
constexpr int BK = 64;   // K per LDS stage: 8 chunks of 16 bytes per row
constexpr int kTiledThreads = 256;

// Maps this workgroup to (expert, first token row, n-tile, K split). Tiles are counted
// from the device-side offsets, so no host synchronisation is needed; the
// grid is sized for the worst case and surplus workgroups return. Workgroup b
// runs on XCD b % 8, so XCD x is given the contiguous logical range
// [x*per, (x+1)*per).
__device__ __forceinline__ bool decode_tile(const int32_t* __restrict__ offsets, int E, int ntn,
                                            int nsplit, int& e, int& beg, int& M, int& m0,
                                            int& nt, int& sp) {
  int total = 0;
  for (int i = 0; i < E; ++i) {
    const int Mi = offsets[i + 1] - offsets[i];
    total += ((Mi + BM - 1) / BM) * ntn * nsplit;
  }
  const int per = (total + 7) / 8;
  const int q = blockIdx.x >> 3;
  if (q >= per) return false;
  int L = (blockIdx.x & 7) * per + q;
  if (L >= total) return false;
  for (int i = 0; i < E; ++i) {
    const int Mi = offsets[i + 1] - offsets[i];
    const int mt = (Mi + BM - 1) / BM;
    const int cnt = mt * ntn * nsplit;
    if (L < cnt) {
      e = i;
      beg = offsets[i];
      M = Mi;
      m0 = (L % mt) * BM;
      const int r = L / mt;
      nt = r % ntn;
      sp = r / ntn;
      return true;
    }
    L -= cnt;
  }
  return false;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

// GATE_UP: act = x (rows gathered), wa = w1, wb = w3, out = h bf16 [A, N=ffn];
// the 128 weight rows of a tile are w1 rows [n, n+32), w3 rows [n, n+32),
// w1 rows [n+32, n+64), w3 rows [n+32, n+64) with n = nt*64, so wave column
// wn holds gate and up for the same 32 h-columns.
// !GATE_UP: act = h (grouped rows), wa = w2, out = y f32 [A, N=d], or with
// nsplit > 1 partial sums over K ranges [sp K/nsplit, (sp+1) K/nsplit) in
// nsplit arrays pstride floats apart.
//
// Pipeline: the global loads of K stage s are issued two iterations before
// stage s is written to LDS (two register sets alternate), so each load has
// two stages of MFMA work to arrive; LDS is double-buffered and one barrier
// per stage separates the writes of stage s+1 from the reads of stage s. The
// barrier waits for LDS operations only (lds_barrier), never for the global
// loads in flight.
// Weight tile loading: standard layout, thread t moves 16-byte chunk t % 8 of
// rows t / 8 + 32 j; fragment order, wave w moves whole fragments w + 4 j
// (one contiguous KiB per load instruction).
template <bool GATE_UP, bool PACKED>
__global__ __launch_bounds__(kTiledThreads, 2) void tiled_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ wa,
    const uint16_t* __restrict__ wb, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_asg, int K, int N, int E, int ktop,
    void* __restrict__ out, int ntn, int nsplit, int64_t pstride) {
  int e, beg, M, m0, nt, sp;
  if (!decode_tile(offsets, E, ntn, nsplit, e, beg, M, m0, nt, sp)) return;
  // this tile's K range [k0, k0 + Kc); split K only for down (nsplit 1 for gate/up)
  const int Kc = K / nsplit;
  const int k0 = sp * Kc;

  __shared__ __attribute__((aligned(16))) uint16_t sW[2][BN * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][BM * BK];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wn = wave & 1;
  const int wm = wave >> 1;

  // weight row of LDS row R
  auto wrow = [&](int R) -> int {
    if constexpr (GATE_UP) {
      return nt * 64 + ((R >> 5) >> 1) * 32 + (R & 31);
    } else {
      return min(nt * BN + R, N - 1);
    }
  };
  auto wmat = [&](int R) -> const uint16_t* {
    if constexpr (GATE_UP) {
      return ((R >> 5) & 1) ? wb : wa;
    } else {
      return wa;
    }
  };

  constexpr int WSTEP = PACKED ? 1024 : BK;  // weight elements per BK advance
  const uint16_t* gw[4];
  const uint16_t* gx[4];
  int sow[4], sox[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // weight chunk j of this thread: LDS row Rw, 16-byte chunk cw (of 8 per row)
    int Rw, cw;
    if constexpr (PACKED) {
      const int F = wave + 4 * j;  // fragment: row tile F >> 1, k step F & 1
      Rw = (F >> 1) * 16 + (lane & 15);
      cw = (F & 1) * 4 + (lane >> 4);
    } else {
      Rw = (tid >> 3) + 32 * j;
      cw = tid & 7;
    }
    gw[j] = wmat(Rw) + wofs<PACKED>(e, wrow(Rw), k0 + cw * 8, N, K);
    sow[j] = swz(Rw, cw);
    // token chunk j: LDS row Rx, chunk cx
    const int Rx = (tid >> 3) + 32 * j;
    const int cx = tid & 7;
    const int mm = min(m0 + Rx, M - 1);
    int64_t row;
    if constexpr (GATE_UP) {
      row = sorted_asg[beg + mm] / ktop;
    } else {
      row = beg + mm;
    }
    gx[j] = act + row * K + k0 + cx * 8;
    sox[j] = swz(Rx, cx);
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = Kc / BK;
  u32x4 rw[2][4], rx[2][4];
  auto issue = [&](int set, int kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      rw[set][j] = ldg16(gw[j] + static_cast<size_t>(kb) * WSTEP);
      rx[set][j] = ldg16(gx[j] + kb * BK);
    }
  };
  auto stash = [&](int set, int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<u32x4*>(&sW[buf][sow[j]]) = rw[set][j];
      *reinterpret_cast<u32x4*>(&sX[buf][sox[j]]) = rx[set][j];
    }
  };

  // prologue: stage 0 -> LDS, stages 1 and 2 in flight. Stage indices past
  // the end are clamped to the last stage: the loop body has no branches
  // around its loads and stores (branches there make the compiler wait for
  // every load in flight), and the few extra loads hit in cache.
  const int last = nk - 1;
  issue(0, 0);
  issue(1, min(1, last));
  stash(0, 0);
  issue(0, min(2, last));
  lds_barrier();

  const int fr = lane & 15;
  const int fg = lane >> 4;
  // one K stage; P = kb & 1 is a compile-time constant so that the register
  // sets are fixed and no load result is copied (a copy would wait for it)
  auto stage_body = [&](auto par, int kb) {
    constexpr int P = decltype(par)::value;
    // an odd stage count leaves one past-the-end stage in the last pair: skip
    // its MFMA work (this branch holds no loads, so the wait counts of the
    // loads in flight stay exact)
    if (kb < nk) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = s * 4 + fg;
      u32x4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int R = wn * 64 + i * 16 + fr;
        a[i] = *reinterpret_cast<const u32x4*>(&sW[P][swz(R, c)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int R = wm * 64 + j * 16 + fr;
        b[j] = *reinterpret_cast<const u32x4*>(&sX[P][swz(R, c)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
    }
    }
    // stage kb+1 has been in register set 1-P since two stages ago (after the
    // last stage this writes a buffer nobody reads); kept after the MFMA work
    // so that its loads get two stages of compute to arrive
    __builtin_amdgcn_sched_barrier(0);
    stash(1 - P, 1 - P);
    lds_barrier();
    issue(1 - P, min(kb + 3, last));
  };
  for (int kb = 0; kb < nk; kb += 2) {
    stage_body(std::integral_constant<int, 0>{}, kb);
    stage_body(std::integral_constant<int, 1>{}, kb + 1);
  }

  // epilogue: lane holds token column fr of each 16x16 tile and weight rows
  // 4*fg .. 4*fg+3 of it
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 64 + j * 16 + fr;
    if (m >= M) continue;
    if constexpr (GATE_UP) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int n = nt * 64 + wn * 32 + i * 16 + 4 * fg;
        const f32x4 gt = acc[i][j];
        const f32x4 up = acc[i + 2][j];
        uint2 v;
        v.x = pack_bf16x2(silu_f32(gt[0]) * up[0], silu_f32(gt[1]) * up[1]);
        v.y = pack_bf16x2(silu_f32(gt[2]) * up[2], silu_f32(gt[3]) * up[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + static_cast<size_t>(beg + m) * N +
                                  n) = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = nt * BN + wn * 64 + i * 16 + 4 * fg;
        if (n < N)
          *reinterpret_cast<f32x4*>(static_cast<float*>(out) + sp * pstride +
                                    static_cast<size_t>(beg + m) * N + n) = acc[i][j];
      }
    }
  }
}

// Weights-in-registers tiled kernel (many rows per expert): a workgroup tile
// is 256 weight rows x 128 token rows; wave w owns weight rows 64w .. 64w+63
// and all 128 tokens (4 x 8 MFMA tiles). Each wave loads its own weight
// fragments straight into registers (never shared, so no LDS traffic for
// weights; with fragment-order weights every load is one contiguous KiB);
// only the token rows, shared by the four waves, are staged through LDS. Per
// 64-wide K stage that is 16 KiB of LDS writes and 64 KiB of reads for
// 4.2 MFLOP, against 32 + 64 KiB for 2.1 MFLOP when both operands go
// through LDS. Weights are fetched RING 32-wide K steps ahead, tokens XSETS
// stages ahead (register sets).
// GATE_UP: wave w's rows are w1 rows n+32w .. n+32w+31 then the same rows of
// w3 (n = nt*128), so gate and up of one h column sit in the same lane.
// Needs N % 256 == 0 (down) or ffn % 128 == 0 (gate/up). Used with
// fragment-order weights; with the standard layout each weight load would be
// 16 rows x 64 bytes, and staging both operands through LDS is faster there.
// W8: int8 weight codes in their 16-row x 64-k blocks (one 16-byte lane load
// per block holds the lane's operands of two 32-wide K steps), converted to
// bf16 operands in registers; the ring then holds RING/2 64-wide stages and
// the epilogue multiplies each row's sum by its scale (sa: w1 or w2, sb: w3).

constexpr int gcd_i(int a, int b) { return b == 0 ? a : gcd_i(b, a % b); }
constexpr int lcm_i(int a, int b) { return a / gcd_i(a, b) * b; }

template <bool GATE_UP, bool PACKED, bool W8, int RING, int OCC, int XSETS>
__global__ __launch_bounds__(kTiledThreads, OCC) void wtiled_kernel(
    const uint16_t* __restrict__ act, const void* __restrict__ wa, const void* __restrict__ wb,
    const float* __restrict__ sa, const float* __restrict__ sb,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_asg, int K, int N,
    int E, int ktop, void* __restrict__ out, int ntn, int nsplit, int64_t pstride) {
  int e, beg, M, m0, nt, sp;
  if (!decode_tile(offsets, E, ntn, nsplit, e, beg, M, m0, nt, sp)) return;
  // this tile's K range [k0, k0 + Kc) (split only for down; Kc % 64 == 0)
  const int Kc = K / nsplit;
  const int k0 = sp * Kc;

  __shared__ __attribute__((aligned(16))) uint16_t sX[2][BM * BK];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int fr = lane & 15;
  const int fg = lane >> 4;
  constexpr int ST = kStep32<PACKED>();

  // weight fragment addresses: a wave-uniform part per row tile (scalar
  // registers) plus one per-lane offset
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint16_t* wbase[4];
  const int8_t* qbase[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int row;
    const void* base;
    if constexpr (GATE_UP) {
      row = nt * 128 + wv * 32 + (i & 1) * 16;
      base = (i < 2) ? wa : wb;
    } else {
      row = nt * 256 + wv * 64 + i * 16;
      base = wa;
    }
    if constexpr (W8)
      qbase[i] = static_cast<const int8_t*>(base) +
                 ((static_cast<size_t>(e) * (N >> 4) + (row >> 4)) * static_cast<size_t>(K >> 6) +
                  (k0 >> 6)) * 1024 + lane * 16;
    else
      wbase[i] = static_cast<const uint16_t*>(base) + wofs<PACKED>(e, row, k0, N, K);
  }
  const int wlane = static_cast<int>(wofs<PACKED>(0, fr, fg * 8, N, K));

  // token chunk j of this thread: row (tid >> 3) + 32 j of the tile, 16-byte
  // chunk tid & 7; all four share one swizzled LDS column (rows differ by 32)
  int xrow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int mm = min(m0 + (tid >> 3) + 32 * j, M - 1);
    if constexpr (GATE_UP) {
      xrow[j] = sorted_asg[beg + mm] / ktop;
    } else {
      xrow[j] = beg + mm;
    }
  }
  const int xcol = (tid & 7) * 8;
  const int sox0 = swz(tid >> 3, tid & 7);

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = Kc / BK;
  const int last = nk - 1;
  const int nsteps = 2 * nk;  // 32-wide K steps
  // weights: a ring of RING K32 slots; the loads of step t+RING are issued
  // as soon as step t has used its slot ((RING-1)/2 stages of lead time).
  // W8: RING/2 slots of one 64-wide stage each, refilled when a stage is done.
  constexpr int WSLOTS = W8 ? RING / 2 : RING;
  u32x4 wr[WSLOTS][4];  // [slot][row tile]
  u32x4 rx[XSETS][4];   // token chunks in flight (XSETS stages)
  auto issue_w = [&](int slot, int t) {  // t: K32 step, or 64-wide stage (W8)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (W8)
        wr[slot][i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(qbase[i] + static_cast<size_t>(t) * 1024));
      else
        wr[slot][i] = ldw<PACKED>(wbase[i] + static_cast<size_t>(t) * ST + wlane);
    }
  };
  auto issue_x = [&](int set, int kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      rx[set][j] = ldg16(act + static_cast<int64_t>(xrow[j]) * K + k0 + kb * BK + xcol);
  };
  auto stash = [&](int set, int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(&sX[buf][sox0 + j * 32 * BK]) = rx[set][j];
  };

  // prologue: tokens of stage 0 in LDS, tokens of stages 1..XSETS and the
  // weights of steps 0..RING-1 in flight (indices past the end clamp to the
  // last one); token stage s lives in register set s mod XSETS
#pragma unroll
  for (int t = 0; t < WSLOTS; ++t) issue_w(t, min(t, (W8 ? nk : nsteps) - 1));
  issue_x(0, 0);
#pragma unroll
  for (int q = 1; q < XSETS; ++q) issue_x(q, min(q, last));
  stash(0, 0);
  issue_x(0, min(XSETS, last));
  lds_barrier();
  // W8: bf16 operands of steps t and t+1 (set t mod 2); each step converts
  // the next one's while its own MFMAs run
  u32x4 wcv[2][4];
  if constexpr (W8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) wcv[0][i] = i8_operand(wr[0][i], 0);
  }

  // K32 step t (T = t mod U, compile-time; U a multiple of 4, of RING and of
  // 2*XSETS): stage kb = t / 2 lives in LDS buffer kb mod 2, half t mod 2 of it
  constexpr int U = lcm_i(lcm_i(4, RING), 2 * XSETS);
  int t0 = 0;
  auto step_body = [&](auto tm) {
    constexpr int T = decltype(tm)::value;
    constexpr int SLOT = W8 ? (T >> 1) % WSLOTS : T % RING;
    constexpr int P = (T >> 1) & 1;  // LDS buffer of this stage
    constexpr int S = T & 1;         // which 32-wide half of the 64-wide stage
    constexpr int XN = ((T >> 1) + 1) % XSETS;  // token set of the next stage
    const int t = t0 + T;
    const int kb = t >> 1;
    if (t < nsteps) {
      const int c = S * 4 + fg;
      u32x4 wf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[i] = W8 ? wcv[T & 1][i] : wr[SLOT][i];
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {  // token fragments four at a time
        u32x4 b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          b[j] = *reinterpret_cast<const u32x4*>(&sX[P][swz((jh * 4 + j) * 16 + fr, c)]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][jh * 4 + j] = mfma16x16x32(wf[i], b[j], acc[i][jh * 4 + j]);
      }
      if constexpr (W8) {
        constexpr int TN = T + 1;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          wcv[TN & 1][i] = i8_operand(wr[(TN >> 1) % WSLOTS][i], TN & 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!W8)
      issue_w(SLOT, min(t + RING, nsteps - 1));
    else if constexpr (S == 1)
      issue_w(SLOT, min(kb + WSLOTS, last));
    if constexpr (S == 1) {
      // end of stage kb: tokens of stage kb+1 (in registers for XSETS stages)
      // go to the other buffer; tokens of stage kb+1+XSETS start loading
      stash(XN, 1 - P);
      lds_barrier();
      issue_x(XN, min(kb + 1 + XSETS, last));
    }
  };
  for (; t0 < nsteps; t0 += U) unrolled(step_body, std::make_integer_sequence<int, U>{});

  // epilogue: lane holds token column fr of each 16x16 tile and weight rows
  // 4*fg .. 4*fg+3 of it (W8: their scales, loaded once)
  f32x4 sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = f32x4{1.f, 1.f, 1.f, 1.f};
    if constexpr (W8) {
      const int n = GATE_UP ? nt * 128 + wave * 32 + (i & 1) * 16 + 4 * fg
                            : nt * 256 + wave * 64 + i * 16 + 4 * fg;
      sc[i] = *reinterpret_cast<const f32x4*>((GATE_UP && i >= 2 ? sb : sa) +
                                              static_cast<size_t>(e) * N + n);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = m0 + j * 16 + fr;
    if (m >= M) continue;
    if constexpr (GATE_UP) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int n = nt * 128 + wave * 32 + i * 16 + 4 * fg;
        f32x4 gt = acc[i][j];
        f32x4 up = acc[i + 2][j];
        if constexpr (W8) {
          gt *= sc[i];
          up *= sc[i + 2];
        }
        uint2 v;
        v.x = pack_bf16x2(silu_f32(gt[0]) * up[0], silu_f32(gt[1]) * up[1]);
        v.y = pack_bf16x2(silu_f32(gt[2]) * up[2], silu_f32(gt[3]) * up[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + static_cast<size_t>(beg + m) * N +
                                  n) = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = nt * 256 + wave * 64 + i * 16 + 4 * fg;
        f32x4 v = acc[i][j];
        if constexpr (W8) v *= sc[i];
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + sp * pstride +
                                  static_cast<size_t>(beg + m) * N + n) = v;
      }
    }
  }
}

// weight ring depth (32-wide K steps; int8 codes: RING/2 slots of 64),
// workgroups per CU and token stages in registers of wtiled_kernel. Down:
// one workgroup per CU with deep rings. Gate/up: two per CU with shallow ones
// (at most 256 registers, no spills), since a second workgroup's MFMAs cover
// this one's waits better than a deeper ring. Measured at 8x7B (gate/up us,
// one per CU -> two): bf16 T = 128 365 -> 325, 384 375 -> 353; int8 codes
// T = 512 443 -> 381, 1024 648 -> 539, 4096 2108 -> 1715; down kept one per CU
// (two: bf16 about the same, int8 T = 512 238 -> 295).
constexpr int kWRing = 8, kWOcc = 1, kWXSets = 2;
constexpr int kW8Ring = 8;
constexpr int kWGuRing = 4, kWGuOcc = 2, kWGuXSets = 1;

inline unsigned tiled_grid(int64_t A, int E, int ntn, int nsplit = 1) {
  const int64_t mt = (A + BM - 1) / BM + E;
  const int64_t tiles = mt * ntn * nsplit;
  return static_cast<unsigned>((tiles + 7) / 8 * 8);
}

template <bool PACKED, int RT, bool FUSED>
void launch_gate_up_stream(const uint16_t* x, const uint16_t* w1, const uint16_t* w3,
                           const int32_t* offsets, const int32_t* sorted_asg, int64_t A, int d,
                           int ffn, int E, int k, uint16_t* h, const FusedPermute& fp,
                           hipStream_t s) {
  hipLaunchKernelGGL((gate_up_stream_kernel<RT, kGateUpU, PACKED, kStreamNT<PACKED>, FUSED>),
                     dim3(ffn / (16 * RT), E), dim3(kWave * kStreamWaves), 0, s, x, w1, w3,
                     offsets, sorted_asg, d, ffn, k, h, fp, static_cast<int>(A), E);
}

template <bool PACKED>
hipError_t gate_up_impl(int variant, const uint16_t* x, const uint16_t* w1, const uint16_t* w3,
                        const int32_t* offsets, const int32_t* sorted_asg, int64_t A, int d,
                        int ffn, int E, int k, uint16_t* h, hipStream_t s,
                        const FusedPermute* fp) {
  if (variant == 1) {
    constexpr int rows = 16 * kGateUpRT;
    const FusedPermute none{};
    if (!PACKED && d % 256 == 0) {  // whole-line loads: each wave's k range whole 64-blocks
      const bool fused = fp && A <= kFusedPermuteMaxA;
      if (fused)
        hipLaunchKernelGGL(gate_up_stream_rm_kernel<true>, dim3(ffn / 16, E),
                           dim3(kWave * kStreamWaves), 0, s, x, w1, w3, offsets, sorted_asg, d,
                           ffn, k, h, *fp, static_cast<int>(A), E);
      else
        hipLaunchKernelGGL(gate_up_stream_rm_kernel<false>, dim3(ffn / 16, E),
                           dim3(kWave * kStreamWaves), 0, s, x, w1, w3, offsets, sorted_asg, d,
                           ffn, k, h, none, static_cast<int>(A), E);
    } else if (fp && A <= kFusedPermuteMaxA) {
      if (ffn % rows != 0)
        launch_gate_up_stream<PACKED, 1, true>(x, w1, w3, offsets, sorted_asg, A, d, ffn, E, k, h,
                                               *fp, s);
      else
        launch_gate_up_stream<PACKED, kGateUpRT, true>(x, w1, w3, offsets, sorted_asg, A, d, ffn,
                                                       E, k, h, *fp, s);
    } else if (ffn % rows != 0) {
      launch_gate_up_stream<PACKED, 1, false>(x, w1, w3, offsets, sorted_asg, A, d, ffn, E, k, h,
                                              none, s);
    } else {
      launch_gate_up_stream<PACKED, kGateUpRT, false>(x, w1, w3, offsets, sorted_asg, A, d, ffn,
                                                      E, k, h, none, s);
    }
  } else if (dma_gate_up_ok(A, k, d, ffn, E)) {
    return launch_gate_up_dma(PACKED, x, w1, w3, offsets, sorted_asg, A, d, ffn, E, k, h, s);
  } else if (PACKED && ffn % 128 == 0) {
    const int ntn = ffn / 128;
    hipLaunchKernelGGL((wtiled_kernel<true, PACKED, false, kWGuRing, kWGuOcc, kWGuXSets>),
                       dim3(tiled_grid(A, E, ntn)), dim3(kTiledThreads), 0, s, x, w1, w3,
                       static_cast<const float*>(nullptr), static_cast<const float*>(nullptr),
                       offsets, sorted_asg, d, ffn, E, k, static_cast<void*>(h), ntn, 1,
                       int64_t(0));
  } else {
    const int ntn = ffn / 64;
    hipLaunchKernelGGL((tiled_kernel<true, PACKED>), dim3(tiled_grid(A, E, ntn)),
                       dim3(kTiledThreads), 0, s, x, w1, w3, offsets, sorted_asg, d, ffn, E, k,
                       static_cast<void*>(h), ntn, 1, int64_t(0));
  }
  return hipGetLastError();
}

template <bool PACKED>
hipError_t down_impl(int variant, const uint16_t* h, const uint16_t* w2, const int32_t* offsets,
                     int64_t A, int d, int ffn, int E, float* part, hipStream_t s,
                     DownSplit ds) {
  const int nsplit = down_splits(variant, A, d, ffn, E);
  if (variant == 1) {
    constexpr int rows = 16 * kDownRT;
    if (!PACKED && d % 32 == 0 && (ffn / 32) % (2 * nsplit) == 0) {
      // whole-line loads: each wave's k range whole 64-blocks
      const unsigned blocks =
          static_cast<unsigned>((d / 32 * nsplit + kStreamWaves - 1) / kStreamWaves);
      hipLaunchKernelGGL(down_stream_rm_kernel, dim3(blocks, E), dim3(kWave * kStreamWaves), 0, s,
                         h, w2, offsets, ffn, d, static_cast<int>(A), nsplit, part);
    } else if (d % rows != 0) {
      const unsigned blocks =
          static_cast<unsigned>((d / 16 * nsplit + kStreamWaves - 1) / kStreamWaves);
      hipLaunchKernelGGL((down_stream_kernel<1, kDownU, PACKED, kStreamNT<PACKED>>), dim3(blocks, E),
                         dim3(kWave * kStreamWaves), 0, s, h, w2, offsets, ffn, d,
                         static_cast<int>(A), nsplit, part);
    } else {
      const unsigned blocks =
          static_cast<unsigned>((d / rows * nsplit + kStreamWaves - 1) / kStreamWaves);
      hipLaunchKernelGGL((down_stream_kernel<kDownRT, kDownU, PACKED, kStreamNT<PACKED>>), dim3(blocks, E),
                         dim3(kWave * kStreamWaves), 0, s, h, w2, offsets, ffn, d,
                         static_cast<int>(A), nsplit, part);
    }
  } else if (down_dma_runs(variant, A, d, ffn, E)) {
    return launch_down_dma(PACKED, h, w2, offsets, A, d, ffn, E, nsplit, part, s, nullptr, ds);
  } else if (PACKED && d % 256 == 0) {
    const int ntn = d / 256;
    hipLaunchKernelGGL((wtiled_kernel<false, PACKED, false, kWRing, kWOcc, kWXSets>),
                       dim3(tiled_grid(A, E, ntn, nsplit)), dim3(kTiledThreads), 0, s, h, w2, w2,
                       static_cast<const float*>(nullptr), static_cast<const float*>(nullptr),
                       offsets, static_cast<const int32_t*>(nullptr), ffn, d, E, 1,
                       static_cast<void*>(part), ntn, nsplit, A * d);
  } else {
    const int ntn = (d + BN - 1) / BN;
    hipLaunchKernelGGL((tiled_kernel<false, PACKED>), dim3(tiled_grid(A, E, ntn, nsplit)),
                       dim3(kTiledThreads), 0, s, h, w2, w2, offsets,
                       static_cast<const int32_t*>(nullptr), ffn, d, E, 1,
                       static_cast<void*>(part), ntn, nsplit, A * d);
  }
  return hipGetLastError();
}

}  // namespace

// Kernel family per projection when the caller does not force one: the
// streaming kernels while experts average few rows, the tiled ones beyond.
// Measured at the 8x7B shape (T tokens, k = 2, E = 8; us): gate/up 336 vs 323
// at 18 rows per expert, 320 vs 320 at 16; down 194 vs 225 at 26 rows per
// expert, 232 vs 218 at 28.
int choose_ffn_variant(int requested, int64_t A, int E) {
  if (requested == 1 || requested == 2) return requested;
  return (A <= static_cast<int64_t>(16) * E) ? 1 : 2;
}

int choose_down_variant(int requested, int64_t A, int E) {
  if (requested == 1 || requested == 2) return requested;
  return (A <= static_cast<int64_t>(27) * E) ? 1 : 2;
}

int tiled_down_splits(int64_t A, int d, int ffn, int E) {
  if (d % 256 != 0 || ffn % 128 != 0) return 1;
  const int64_t tiles = (A / BM + E) * (d / 256);  // at most this many 256-row tiles
  return tiles < 256 ? 2 : 1;
}

bool down_dma_runs(int variant, int64_t A, int d, int ffn, int E) {
  return variant != 1 && dma_down_ok(A, d, ffn, E);
}

int down_splits(int variant, int64_t A, int d, int ffn, int E) {
  // the streaming down kernel splits K two ways while its float32 partials
  // stay small; the direct-to-LDS kernel chooses its split on the device from
  // the expert counts (at most two parts), and below its sizes the tiled
  // kernels split K while the 256-row weights-in-registers tiles would not
  // give every CU one (all tiled kernels of a size follow the same rule, so y
  // does not depend on the weight layout)
  if (variant == 1) return A <= 4096 ? 2 : 1;
  if (dma_down_ok(A, d, ffn, E)) return dma_down_splits(A, d, ffn, E);
  return tiled_down_splits(A, d, ffn, E);
}

hipError_t launch_gate_up_w8_tiled(const uint16_t* x, const void* q1, const void* q3,
                                  const float* s1, const float* s3, const int32_t* offsets,
                                  const int32_t* sorted_asg, int64_t A, int d, int ffn, int E,
                                  int k, uint16_t* h, hipStream_t s) {
  const int ntn = ffn / 128;
  hipLaunchKernelGGL((wtiled_kernel<true, true, true, kWGuRing, kWGuOcc, kWGuXSets>),
                     dim3(tiled_grid(A, E, ntn)), dim3(kTiledThreads), 0, s, x, q1, q3, s1, s3,
                     offsets, sorted_asg, d, ffn, E, k, static_cast<void*>(h), ntn, 1, int64_t(0));
  return hipGetLastError();
}

hipError_t launch_down_w8_tiled(const uint16_t* h, const void* q2, const float* s2,
                               const int32_t* offsets, int64_t A, int d, int ffn, int E,
                               int nsplit, float* part, hipStream_t s) {
  const int ntn = d / 256;
  hipLaunchKernelGGL((wtiled_kernel<false, true, true, kW8Ring, kWOcc, kWXSets>),
                     dim3(tiled_grid(A, E, ntn, nsplit)), dim3(kTiledThreads), 0, s, h, q2, q2, s2,
                     static_cast<const float*>(nullptr), offsets,
                     static_cast<const int32_t*>(nullptr), ffn, d, E, 1, static_cast<void*>(part),
                     ntn, nsplit, A * d);
  return hipGetLastError();
}

hipError_t launch_pack_bf16(const uint16_t* w, int E, int R, int C, uint16_t* out, hipStream_t s) {
  const int64_t chunks = static_cast<int64_t>(E) * R * C / 8;
  if (chunks == 0) return hipSuccess;
  const int64_t want = (chunks + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(256), 0, s, w, chunks, R, C, out);
  return hipGetLastError();
}

hipError_t launch_gate_up_bf16(int variant, bool packed, const uint16_t* x, const uint16_t* w1,
                               const uint16_t* w3, const int32_t* offsets,
                               const int32_t* sorted_asg, int64_t A, int d, int ffn, int E,
                               int k, uint16_t* h, hipStream_t s, const FusedPermute* fp) {
  if (A == 0) return hipSuccess;
  if (fp && !gate_up_fuses_permute(variant, A)) return hipErrorInvalidValue;
  return packed ? gate_up_impl<true>(variant, x, w1, w3, offsets, sorted_asg, A, d, ffn, E, k, h, s, fp)
                : gate_up_impl<false>(variant, x, w1, w3, offsets, sorted_asg, A, d, ffn, E, k, h, s, fp);
}

bool gate_up_fuses_permute(int variant, int64_t A) {
  return variant == 1 && A > 0 && A <= kFusedPermuteMaxA;
}

hipError_t launch_down_bf16(int variant, bool packed, const uint16_t* h, const uint16_t* w2,
                            const int32_t* offsets, int64_t A, int d, int ffn, int E, float* part,
                            hipStream_t s, DownSplit ds) {
  if (A == 0) return hipSuccess;
  return packed ? down_impl<true>(variant, h, w2, offsets, A, d, ffn, E, part, s, ds)
                : down_impl<false>(variant, h, w2, offsets, A, d, ffn, E, part, s, ds);
}

}  // namespace moe
