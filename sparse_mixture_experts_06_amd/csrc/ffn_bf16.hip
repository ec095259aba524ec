// Expert SwiGLU on bf16 MFMA (nnterp Mixtral page, support(): the down
// projection receives act(gate) * up with act = SiLU; "expert_outputs needs
// the default experts implementation": the 8 experts are one stacked module).
//
//   gate/up:  h[p, n] = silu(sum_i x[r,i] w1[e,n,i]) * (sum_i x[r,i] w3[e,n,i])
//             r = sorted_asg[p] / k,  p in expert e's grouped range; h is bf16
//   down:     y[p, n] = sum_f h[p,f] w2[e,n,f]                      y is f32
//
// Both are grouped GEMMs whose two operands are "row x K" with K contiguous
// (weight rows n, token rows m), so the weights are the MFMA A operand and the
// tokens the B operand: D[n][m] = W[n,:] . X[m,:]. With
// v_mfma_f32_16x16x32_bf16 a lane holds 8 consecutive K values of one row for
// either operand, and four consecutive n of one token in the result, which
// gives 8-byte (h) and 16-byte (y) row stores.
//
// Two families:
//  * streaming (few rows per expert, decode): no LDS staging. A workgroup owns
//    16 weight rows (of w1 and w3 together for gate/up); its 4 waves split K
//    and stream those rows once from HBM with 16-byte loads, reusing each load
//    for up to 32 token rows; partial sums meet in LDS.
//  * tiled (many rows per expert, prefill): 128 weight rows x 128 token rows
//    x 64 K per step, double-buffered in LDS with an XOR swizzle of the
//    16-byte chunks (conflict-free ds_read_b128 for the MFMA fragments); 4
//    waves each own a 64x64 block of 4x4 MFMA tiles. Tiles are listed expert
//    by expert, n-tile by n-tile, m-tile by m-tile, and consecutive tiles go
//    to the same XCD so the m-tiles sharing a weight tile meet in that XCD's
//    L2.
#include "common.h"

namespace moe {
namespace {

// ----------------------------------------------------------------------------
// streaming kernels
// ----------------------------------------------------------------------------
constexpr int kStreamWaves = 4;
constexpr int kStreamUnroll = 4;

// GATE_UP: act = x [T, K=d] with rows gathered through sorted_asg / ktop,
//          wa = w1, wb = w3 (each [E, N=ffn, K]), out = h bf16 [A, N].
// !GATE_UP: act = h [A, K=ffn] in grouped order, wa = w2 [E, N=d, K],
//          out = y f32 [A, N].
template <bool GATE_UP>
__global__ __launch_bounds__(kWave* kStreamWaves) void stream_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ wa,
    const uint16_t* __restrict__ wb, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_asg, int K, int N, int ktop, void* __restrict__ out) {
  constexpr int NM = GATE_UP ? 2 : 1;
  const int e = blockIdx.y;
  const int n0 = blockIdx.x * 16;
  const int beg = offsets[e];
  const int M = offsets[e + 1] - beg;
  if (M <= 0) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int S = K / 32;
  const int s_lo = (wave * S) / kStreamWaves;
  const int s_hi = ((wave + 1) * S) / kStreamWaves;
  const size_t wrow = (static_cast<size_t>(e) * N + n0 + r) * K + g * 8;
  const uint16_t* pa = wa + wrow;
  const uint16_t* pb = GATE_UP ? wb + wrow : wa + wrow;

  __shared__ f32x4 red[kStreamWaves - 1][NM][2][kWave];

  for (int mb = 0; mb < M; mb += 32) {
    const bool two = (M - mb) > 16;  // wave-uniform
    const int m0 = min(mb + r, M - 1);
    const int m1 = min(mb + 16 + r, M - 1);
    int64_t row0, row1;
    if constexpr (GATE_UP) {
      row0 = sorted_asg[beg + m0] / ktop;
      row1 = sorted_asg[beg + m1] / ktop;
    } else {
      row0 = beg + m0;
      row1 = beg + m1;
    }
    const uint16_t* px0 = act + row0 * K + g * 8;
    const uint16_t* px1 = act + row1 * K + g * 8;

    f32x4 acc[NM][2];
#pragma unroll
    for (int a = 0; a < NM; ++a) acc[a][0] = acc[a][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    int s = s_lo;
    for (; s + kStreamUnroll <= s_hi; s += kStreamUnroll) {
      u32x4 A0[kStreamUnroll], A1[kStreamUnroll], B0[kStreamUnroll], B1[kStreamUnroll];
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const int off = (s + u) * 32;
        A0[u] = ldg16(pa + off);
        if constexpr (GATE_UP) A1[u] = ldg16(pb + off);
        B0[u] = ldg16(px0 + off);
        B1[u] = two ? ldg16(px1 + off) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        acc[0][0] = mfma16x16x32(A0[u], B0[u], acc[0][0]);
        if constexpr (GATE_UP) acc[1][0] = mfma16x16x32(A1[u], B0[u], acc[1][0]);
        if (two) {
          acc[0][1] = mfma16x16x32(A0[u], B1[u], acc[0][1]);
          if constexpr (GATE_UP) acc[1][1] = mfma16x16x32(A1[u], B1[u], acc[1][1]);
        }
      }
    }
    for (; s < s_hi; ++s) {
      const int off = s * 32;
      const u32x4 a0 = ldg16(pa + off);
      const u32x4 b0 = ldg16(px0 + off);
      acc[0][0] = mfma16x16x32(a0, b0, acc[0][0]);
      u32x4 a1 = a0;
      if constexpr (GATE_UP) {
        a1 = ldg16(pb + off);
        acc[1][0] = mfma16x16x32(a1, b0, acc[1][0]);
      }
      if (two) {
        const u32x4 b1 = ldg16(px1 + off);
        acc[0][1] = mfma16x16x32(a0, b1, acc[0][1]);
        if constexpr (GATE_UP) acc[1][1] = mfma16x16x32(a1, b1, acc[1][1]);
      }
    }

    if (wave > 0) {
#pragma unroll
      for (int a = 0; a < NM; ++a)
#pragma unroll
        for (int t = 0; t < 2; ++t) red[wave - 1][a][t][lane] = acc[a][t];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < kStreamWaves - 1; ++w)
#pragma unroll
        for (int a = 0; a < NM; ++a)
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[a][t] += red[w][a][t][lane];
      // lane holds token column r and weight rows n0 + 4g .. n0 + 4g + 3
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int m = mb + t * 16 + r;
        if (m < M) {
          const size_t o = static_cast<size_t>(beg + m) * N + n0 + 4 * g;
          if constexpr (GATE_UP) {
            const f32x4 gt = acc[0][t];
            const f32x4 up = acc[1][t];
            uint2 v;
            v.x = pack_bf16x2(silu_f32(gt[0]) * up[0], silu_f32(gt[1]) * up[1]);
            v.y = pack_bf16x2(silu_f32(gt[2]) * up[2], silu_f32(gt[3]) * up[3]);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) = v;
          } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(out) + o) = acc[0][t];
          }
        }
      }
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------
// tiled kernels
// ----------------------------------------------------------------------------
constexpr int BM = 128;  // token rows per tile (MFMA B operand)
constexpr int BN = 128;  // weight rows per tile (MFMA A operand)
constexpr int BK = 64;   // K per LDS stage: 8 chunks of 16 bytes per row
constexpr int kTiledThreads = 256;

// Maps this workgroup to (expert, first token row, n-tile). Tiles are counted
// from the device-side offsets, so no host synchronisation is needed; the
// grid is sized for the worst case and surplus workgroups return. Workgroup b
// runs on XCD b % 8, so XCD x is given the contiguous logical range
// [x*per, (x+1)*per).
__device__ __forceinline__ bool decode_tile(const int32_t* __restrict__ offsets, int E, int ntn,
                                            int& e, int& beg, int& M, int& m0, int& nt) {
  int total = 0;
  for (int i = 0; i < E; ++i) {
    const int Mi = offsets[i + 1] - offsets[i];
    total += ((Mi + BM - 1) / BM) * ntn;
  }
  const int per = (total + 7) / 8;
  const int q = blockIdx.x >> 3;
  if (q >= per) return false;
  int L = (blockIdx.x & 7) * per + q;
  if (L >= total) return false;
  for (int i = 0; i < E; ++i) {
    const int Mi = offsets[i + 1] - offsets[i];
    const int mt = (Mi + BM - 1) / BM;
    const int cnt = mt * ntn;
    if (L < cnt) {
      e = i;
      beg = offsets[i];
      M = Mi;
      nt = L / mt;
      m0 = (L % mt) * BM;
      return true;
    }
    L -= cnt;
  }
  return false;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

// GATE_UP: the 128 weight rows of a tile are w1 rows [n, n+32), w3 rows
// [n, n+32), w1 rows [n+32, n+64), w3 rows [n+32, n+64) with n = nt*64, so
// wave column wn holds gate and up for the same 32 h-columns.
template <bool GATE_UP>
__global__ __launch_bounds__(kTiledThreads, 2) void tiled_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ wa,
    const uint16_t* __restrict__ wb, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_asg, int K, int N, int E, int ktop,
    void* __restrict__ out, int ntn) {
  int e, beg, M, m0, nt;
  if (!decode_tile(offsets, E, ntn, e, beg, M, m0, nt)) return;

  __shared__ __attribute__((aligned(16))) uint16_t sW[2][BN * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][BM * BK];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wn = wave & 1;
  const int wm = wave >> 1;

  // this thread moves 16-byte chunk (tid & 7) of rows (tid >> 3) + 32 j, j < 4
  const int lrow = tid >> 3;
  const int lch = tid & 7;
  const uint16_t* gw[4];
  const uint16_t* gx[4];
  int so[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int R = lrow + 32 * j;
    int n;
    const uint16_t* base;
    if constexpr (GATE_UP) {
      base = (j & 1) ? wb : wa;
      n = nt * 64 + (j >> 1) * 32 + lrow;
    } else {
      base = wa;
      n = min(nt * BN + R, N - 1);
    }
    gw[j] = base + (static_cast<size_t>(e) * N + n) * K + lch * 8;
    const int mm = min(m0 + R, M - 1);
    int64_t row;
    if constexpr (GATE_UP) {
      row = sorted_asg[beg + mm] / ktop;
    } else {
      row = beg + mm;
    }
    gx[j] = act + row * K + lch * 8;
    so[j] = swz(R, lch);
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 rw[4], rx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    rw[j] = ldg16(gw[j]);
    rx[j] = ldg16(gx[j]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    *reinterpret_cast<u32x4*>(&sW[0][so[j]]) = rw[j];
    *reinterpret_cast<u32x4*>(&sX[0][so[j]]) = rx[j];
  }
  __syncthreads();

  const int nk = K / BK;
  const int fr = lane & 15;
  const int fg = lane >> 4;
  for (int kb = 0; kb < nk; ++kb) {
    const int cur = kb & 1;
    const bool more = (kb + 1) < nk;
    if (more) {
      const int off = (kb + 1) * BK;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rw[j] = ldg16(gw[j] + off);
        rx[j] = ldg16(gx[j] + off);
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = s * 4 + fg;
      u32x4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int R = wn * 64 + i * 16 + fr;
        a[i] = *reinterpret_cast<const u32x4*>(&sW[cur][swz(R, c)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int R = wm * 64 + j * 16 + fr;
        b[j] = *reinterpret_cast<const u32x4*>(&sX[cur][swz(R, c)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<u32x4*>(&sW[cur ^ 1][so[j]]) = rw[j];
        *reinterpret_cast<u32x4*>(&sX[cur ^ 1][so[j]]) = rx[j];
      }
    }
    __syncthreads();
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
          *reinterpret_cast<f32x4*>(static_cast<float*>(out) + static_cast<size_t>(beg + m) * N +
                                    n) = acc[i][j];
      }
    }
  }
}

inline unsigned tiled_grid(int64_t A, int E, int ntn) {
  const int64_t mt = (A + BM - 1) / BM + E;
  const int64_t tiles = mt * ntn;
  return static_cast<unsigned>((tiles + 7) / 8 * 8);
}

}  // namespace

int choose_ffn_variant(int requested, int64_t A, int E) {
  if (requested == 1 || requested == 2) return requested;
  // up to 32 rows per expert on average the weight stream dominates
  return (A <= static_cast<int64_t>(32) * E) ? 1 : 2;
}

hipError_t launch_gate_up_bf16(int variant, const uint16_t* x, const uint16_t* w1,
                               const uint16_t* w3, const int32_t* offsets,
                               const int32_t* sorted_asg, int64_t A, int d, int ffn, int E,
                               int k, uint16_t* h, hipStream_t s) {
  if (A == 0) return hipSuccess;
  if (choose_ffn_variant(variant, A, E) == 1) {
    hipLaunchKernelGGL(stream_kernel<true>, dim3(ffn / 16, E), dim3(kWave * kStreamWaves), 0, s,
                       x, w1, w3, offsets, sorted_asg, d, ffn, k, static_cast<void*>(h));
  } else {
    const int ntn = ffn / 64;
    hipLaunchKernelGGL(tiled_kernel<true>, dim3(tiled_grid(A, E, ntn)), dim3(kTiledThreads), 0,
                       s, x, w1, w3, offsets, sorted_asg, d, ffn, E, k, static_cast<void*>(h),
                       ntn);
  }
  return hipGetLastError();
}

hipError_t launch_down_bf16(int variant, const uint16_t* h, const uint16_t* w2,
                            const int32_t* offsets, int64_t A, int d, int ffn, int E, float* y,
                            hipStream_t s) {
  if (A == 0) return hipSuccess;
  if (choose_ffn_variant(variant, A, E) == 1) {
    hipLaunchKernelGGL(stream_kernel<false>, dim3(d / 16, E), dim3(kWave * kStreamWaves), 0, s,
                       h, w2, w2, offsets, static_cast<const int32_t*>(nullptr), ffn, d, 1,
                       static_cast<void*>(y));
  } else {
    const int ntn = (d + BN - 1) / BN;
    hipLaunchKernelGGL(tiled_kernel<false>, dim3(tiled_grid(A, E, ntn)), dim3(kTiledThreads), 0,
                       s, h, w2, w2, offsets, static_cast<const int32_t*>(nullptr), ffn, d, E, 1,
                       static_cast<void*>(y), ntn);
  }
  return hipGetLastError();
}

}  // namespace moe
