// Weight-only int8 experts for the decode path (ZeroModels Mixtral page,
// "Lower memory": checkpoints load weight-only quantized to int8 with
// bfloat16 activations). The layer is unchanged (nnterp Mixtral page,
// support(): the down projection receives act(gate) * up with act = SiLU);
// only the expert matrices are stored as int8 codes q with one float32 scale
// per output row, w[e][n][k] ~ scale[e][n] * q[e][n][k]:
//
//   scale[e][n] = max_k |w[e][n][k]| / 127                   (float32)
//   q[e][n][k]  = round_half_even(w[e][n][k] / scale[e][n])   (0 where scale is 0)
//
// The kernels multiply bf16 activations by the codes (|q| <= 127 is exact in
// bfloat16) on the same MFMA as the bf16 path, accumulate in float32 and apply
// the row's scale to the finished sum: g = scale * sum_k x_k q_k, which is
// sum_k x_k (scale q_k) up to float32 rounding.
//
// Quantized matrix (moe_quantize_weight), one allocation: the codes of [E,
// rows, cols] in 16-row x 64-column blocks of 1 KiB, each in MFMA lane order
// (lane l = 16 g + r holds row r, columns 64 s + 8 g .. + 7 in bytes 16 l ..
// 16 l + 7 and columns 64 s + 32 + 8 g .. + 7 in bytes 16 l + 8 .. 16 l + 15),
// blocks ordered (expert, row tile, 64-column step); then, at the next
// 256-byte boundary, the float32 scales [E, rows]. A wave's 16-byte load of one
// block is one contiguous KiB and feeds two 32-deep MFMA steps.
//
// More rows per expert: the weights-in-registers tile kernel of ffn_bf16.hip
// (template argument W8) reads the code blocks and converts them to bf16
// operands in registers. Large prefill batches: the codes are widened to
// bfloat16 (exact) in the fragment order of the bf16 path, into the caller's
// workspace, and the direct-to-LDS tile kernels run on them with the row
// scales applied to their finished sums. Block b of the codes holds exactly
// the bf16 fragments 2b (its bytes 0-7 in each lane) and 2b+1 (bytes 8-15),
// since both layouts order (expert, 16-row tile, K step) and put lane l's
// values in lane order.
//
// Kernels here: the streaming decode kernels of ffn_bf16.hip with int8
// weights.
// gate/up: a workgroup owns two 16-row tiles of w1 and w3, its 4 waves split
// K, partial sums meet in LDS, wave 0 scales, applies SiLU*mul and stores bf16
// h. down: each wave streams four 16-row tiles of w2 over 1/nsplit of K and
// writes a scaled float32 partial of y. Every 64-deep step also loads the
// token fragments (as many bytes as one weight block), so several row tiles
// share them.
#include "common.h"

namespace moe {
namespace {

constexpr int kW8Waves = 4;

__host__ __device__ constexpr size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// byte offset of block (e, row tile rt, 64-column step s) in the codes
__device__ __forceinline__ size_t w8_block(int e, int rt, int s, int rows, int cols) {
  return ((static_cast<size_t>(e) * (rows >> 4) + rt) * static_cast<size_t>(cols >> 6) + s) * 1024;
}

// 16 int8 codes -> two MFMA operands of 8 bf16 each (bytes 0-7 and 8-15)
__device__ __forceinline__ void cvt16(u32x4 q, u32x4& lo, u32x4& hi) {
  lo = i8_operand(q, 0);
  hi = i8_operand(q, 1);
}

__device__ __forceinline__ u32x4 ldw8(const int8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// One wave per row: absmax, scale, then the row's codes, 8 at a time into
// their block positions. w [E*rows, cols] bf16 (standard layout).
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ w,
                                                       int64_t nrows, int rows, int cols,
                                                       int8_t* __restrict__ codes,
                                                       float* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= nrows) return;
  const uint16_t* src = w + row * cols;
  float m = 0.0f;
  for (int c = lane; c < cols; c += kWave) m = fmaxf(m, fabsf(bf16_to_f32(src[c])));
  for (int o = kWave / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  const float scale = m / 127.0f;
  if (lane == 0) scales[row] = scale;
  const int e = static_cast<int>(row / rows);
  const int n = static_cast<int>(row % rows);
  const int r = n & 15;
  // 8-column groups: group j = columns 8j .. 8j+7
  for (int j = lane; j < cols / 8; j += kWave) {
    const int c0 = j * 8;
    const int s = c0 >> 6, within = c0 & 63, half = within >> 5, g = (within & 31) >> 3;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int q = 0;
      if (scale > 0.0f) {
        q = static_cast<int>(rintf(bf16_to_f32(src[c0 + i]) / scale));
        q = max(-127, min(127, q));
      }
      const uint32_t b = static_cast<uint32_t>(q) & 0xFFu;
      if (i < 4) lo |= b << (8 * i);
      else hi |= b << (8 * (i - 4));
    }
    int8_t* dst = codes + w8_block(e, n >> 4, s, rows, cols) + (16 * g + r) * 16 + half * 8;
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  }
}

// codes of nblocks blocks -> bf16 fragment order: one thread per (block, lane)
__global__ __launch_bounds__(256) void widen_kernel(const int8_t* __restrict__ codes,
                                                    int64_t nblocks, uint16_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= nblocks * kWave) return;
  const int64_t b = i / kWave;
  const int lane = static_cast<int>(i % kWave);
  u32x4 lo, hi;
  cvt16(ldw8(codes + b * 1024 + lane * 16), lo, hi);
  *reinterpret_cast<u32x4*>(out + (2 * b) * 512 + lane * 8) = lo;
  *reinterpret_cast<u32x4*>(out + (2 * b + 1) * 512 + lane * 8) = hi;
}

// x [T, K=d] bf16 rows gathered through sorted_asg / ktop; w1, w3 codes and
// scales [E, N=ffn]; h bf16 [A, N]. A workgroup owns RT 16-row tiles (each
// token fragment load serves 2*RT weight blocks). Token rows 32 at a time.
template <int RT, int U>
__global__ __launch_bounds__(kWave* kW8Waves) void gate_up_w8_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ w1, const float* __restrict__ s1,
    const int8_t* __restrict__ w3, const float* __restrict__ s3,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_asg, int K, int N,
    int ktop, uint16_t* __restrict__ h) {
  const int e = blockIdx.y;
  const int n0 = blockIdx.x * (16 * RT);
  const int beg = offsets[e];
  const int M = offsets[e + 1] - beg;
  if (M <= 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int S = K / 64;
  const int s_lo = (wave * S) / kW8Waves;
  const int s_hi = ((wave + 1) * S) / kW8Waves;
  const int8_t* pg[RT];
  const int8_t* pu[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    pg[t] = w1 + w8_block(e, (n0 >> 4) + t, 0, N, K) + lane * 16;
    pu[t] = w3 + w8_block(e, (n0 >> 4) + t, 0, N, K) + lane * 16;
  }
  __shared__ f32x4 red[kW8Waves - 1][2][RT][2][kWave];

  for (int mb = 0; mb < M; mb += 32) {
    const bool two = (M - mb) > 16;  // wave-uniform
    const uint16_t* px0 =
        x + static_cast<int64_t>(sorted_asg[beg + min(mb + r, M - 1)] / ktop) * K + g * 8;
    const uint16_t* px1 =
        x + static_cast<int64_t>(sorted_asg[beg + min(mb + 16 + r, M - 1)] / ktop) * K + g * 8;
    f32x4 ag[RT][2], au[RT][2];
#pragma unroll
    for (int t = 0; t < RT; ++t)
      ag[t][0] = ag[t][1] = au[t][0] = au[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto body = [&](const u32x4* G, const u32x4* V, u32x4 b0a, u32x4 b0b, u32x4 b1a, u32x4 b1b) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        u32x4 gl, gh, ul, uh;
        cvt16(G[t], gl, gh);
        cvt16(V[t], ul, uh);
        ag[t][0] = mfma16x16x32(gl, b0a, ag[t][0]);
        ag[t][0] = mfma16x16x32(gh, b0b, ag[t][0]);
        au[t][0] = mfma16x16x32(ul, b0a, au[t][0]);
        au[t][0] = mfma16x16x32(uh, b0b, au[t][0]);
        if (two) {
          ag[t][1] = mfma16x16x32(gl, b1a, ag[t][1]);
          ag[t][1] = mfma16x16x32(gh, b1b, ag[t][1]);
          au[t][1] = mfma16x16x32(ul, b1a, au[t][1]);
          au[t][1] = mfma16x16x32(uh, b1b, au[t][1]);
        }
      }
    };
    int s = s_lo;
    for (; s + U <= s_hi; s += U) {
      u32x4 G[U][RT], V[U][RT], B0a[U], B0b[U], B1a[U], B1b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          G[u][t] = ldw8(pg[t] + (s + u) * 1024);
          V[u][t] = ldw8(pu[t] + (s + u) * 1024);
        }
        B0a[u] = ldg16(px0 + (s + u) * 64);
        B0b[u] = ldg16(px0 + (s + u) * 64 + 32);
        B1a[u] = two ? ldg16(px1 + (s + u) * 64) : u32x4{0u, 0u, 0u, 0u};
        B1b[u] = two ? ldg16(px1 + (s + u) * 64 + 32) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) body(G[u], V[u], B0a[u], B0b[u], B1a[u], B1b[u]);
    }
    for (; s < s_hi; ++s) {
      const u32x4 b1a = two ? ldg16(px1 + s * 64) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 b1b = two ? ldg16(px1 + s * 64 + 32) : u32x4{0u, 0u, 0u, 0u};
      u32x4 G[RT], V[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        G[t] = ldw8(pg[t] + s * 1024);
        V[t] = ldw8(pu[t] + s * 1024);
      }
      body(G, V, ldg16(px0 + s * 64), ldg16(px0 + s * 64 + 32), b1a, b1b);
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
      for (int w = 0; w < kW8Waves - 1; ++w)
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          ag[t][0] += red[w][0][t][0][lane];
          au[t][0] += red[w][1][t][0][lane];
          if (two) {
            ag[t][1] += red[w][0][t][1][lane];
            au[t][1] += red[w][1][t][1][lane];
          }
        }
      // lane holds token column r and weight rows n0 + 16t + 4g .. + 3 of tile t
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const size_t srow = static_cast<size_t>(e) * N + n0 + 16 * t + 4 * g;
        const f32x4 sg = *reinterpret_cast<const f32x4*>(s1 + srow);
        const f32x4 su = *reinterpret_cast<const f32x4*>(s3 + srow);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int m = mb + c * 16 + r;
          if (m < M) {
            const f32x4 gt = ag[t][c] * sg;
            const f32x4 up = au[t][c] * su;
            uint2 v;
            v.x = pack_bf16x2(silu_f32(gt[0]) * up[0], silu_f32(gt[1]) * up[1]);
            v.y = pack_bf16x2(silu_f32(gt[2]) * up[2], silu_f32(gt[3]) * up[3]);
            *reinterpret_cast<uint2*>(h + static_cast<size_t>(beg + m) * N + n0 + 16 * t + 4 * g) = v;
          }
        }
      }
    }
    __syncthreads();
  }
}

// h [A, K=ffn] bf16 in grouped order; w2 codes and scales [E, N=d];
// part [nsplit, A, N] f32. Wave task = (RT 16-row tiles, split sp).
template <int RT, int U>
__global__ __launch_bounds__(kWave* kW8Waves) void down_w8_kernel(
    const uint16_t* __restrict__ h, const int8_t* __restrict__ w2, const float* __restrict__ s2,
    const int32_t* __restrict__ offsets, int K, int N, int A, int nsplit,
    float* __restrict__ part) {
  const int e = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int task = blockIdx.x * kW8Waves + static_cast<int>(threadIdx.x) / kWave;
  if (task >= (N / (16 * RT)) * nsplit) return;
  const int sp = task % nsplit;
  const int n0 = (task / nsplit) * (16 * RT);
  const int beg = offsets[e];
  const int M = offsets[e + 1] - beg;
  if (M <= 0) return;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int S = K / 64;
  const int s_lo = (sp * S) / nsplit;
  const int s_hi = ((sp + 1) * S) / nsplit;
  const int8_t* pw[RT];
  f32x4 sc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    pw[t] = w2 + w8_block(e, (n0 >> 4) + t, 0, N, K) + lane * 16;
    sc[t] = *reinterpret_cast<const f32x4*>(s2 + static_cast<size_t>(e) * N + n0 + 16 * t + 4 * g);
  }
  float* dst = part + static_cast<size_t>(sp) * A * N;
  for (int mb = 0; mb < M; mb += 32) {
    const bool two = (M - mb) > 16;
    const uint16_t* px0 = h + static_cast<int64_t>(beg + min(mb + r, M - 1)) * K + g * 8;
    const uint16_t* px1 = h + static_cast<int64_t>(beg + min(mb + 16 + r, M - 1)) * K + g * 8;
    f32x4 acc[RT][2];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t][0] = acc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto body = [&](const u32x4* W, u32x4 b0a, u32x4 b0b, u32x4 b1a, u32x4 b1b) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        u32x4 wl, wh;
        cvt16(W[t], wl, wh);
        acc[t][0] = mfma16x16x32(wl, b0a, acc[t][0]);
        acc[t][0] = mfma16x16x32(wh, b0b, acc[t][0]);
        if (two) {
          acc[t][1] = mfma16x16x32(wl, b1a, acc[t][1]);
          acc[t][1] = mfma16x16x32(wh, b1b, acc[t][1]);
        }
      }
    };
    int s = s_lo;
    for (; s + U <= s_hi; s += U) {
      u32x4 W[U][RT], B0a[U], B0b[U], B1a[U], B1b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int t = 0; t < RT; ++t) W[u][t] = ldw8(pw[t] + (s + u) * 1024);
        B0a[u] = ldg16(px0 + (s + u) * 64);
        B0b[u] = ldg16(px0 + (s + u) * 64 + 32);
        B1a[u] = two ? ldg16(px1 + (s + u) * 64) : u32x4{0u, 0u, 0u, 0u};
        B1b[u] = two ? ldg16(px1 + (s + u) * 64 + 32) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) body(W[u], B0a[u], B0b[u], B1a[u], B1b[u]);
    }
    for (; s < s_hi; ++s) {
      const u32x4 b1a = two ? ldg16(px1 + s * 64) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 b1b = two ? ldg16(px1 + s * 64 + 32) : u32x4{0u, 0u, 0u, 0u};
      u32x4 W[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) W[t] = ldw8(pw[t] + s * 1024);
      body(W, ldg16(px0 + s * 64), ldg16(px0 + s * 64 + 32), b1a, b1b);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int m = mb + c * 16 + r;
      if (m < M) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
          *reinterpret_cast<f32x4*>(dst + static_cast<size_t>(beg + m) * N + n0 + 16 * t + 4 * g) =
              acc[t][c] * sc[t];
      }
    }
  }
}

// 16-row tiles per workgroup (gate/up) or wave (down) and 64-wide K steps per
// wave in flight, from a sweep at the 8x7B decode shape (gate/up 2 x 3:
// 6.5 TB/s of codes; down 4 x 4: 6.0 TB/s)
#ifndef MOE_W8_GU_RT
#define MOE_W8_GU_RT 2
#endif
#ifndef MOE_W8_GU_U
#define MOE_W8_GU_U 3
#endif
#ifndef MOE_W8_DN_RT
#define MOE_W8_DN_RT 4
#endif
#ifndef MOE_W8_DN_U
#define MOE_W8_DN_U 4
#endif
constexpr int kW8GateUpRT = MOE_W8_GU_RT, kW8GateUpU = MOE_W8_GU_U;
constexpr int kW8DownRT = MOE_W8_DN_RT, kW8DownU = MOE_W8_DN_U;

}  // namespace

size_t int8_weight_bytes(int E, int rows, int cols) {
  return align256(static_cast<size_t>(E) * rows * cols) + static_cast<size_t>(E) * rows * 4;
}

const float* int8_scales(const void* w, int E, int rows, int cols) {
  return reinterpret_cast<const float*>(static_cast<const char*>(w) +
                                        align256(static_cast<size_t>(E) * rows * cols));
}

hipError_t launch_widen_int8(const void* w, int E, int rows, int cols, uint16_t* out,
                             hipStream_t s) {
  const int64_t nblocks = static_cast<int64_t>(E) * (rows / 16) * (cols / 64);
  const int64_t threads = nblocks * kWave;
  hipLaunchKernelGGL(widen_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256),
                     0, s, static_cast<const int8_t*>(w), nblocks, out);
  return hipGetLastError();
}

// Kernel family for int8 weights when the caller does not force one. The
// streaming kernels stay ahead of the tiled one longer than with bf16 weights
// (half the bytes per pass over the weights). Measured at the 8x7B shape
// (T tokens, k = 2, E = 8; us, streaming vs tiled): gate/up 242 vs 301 at 32
// rows per expert, 333 vs 293 at 40; down 192 vs 229 at 48, 249 vs 228 at 56.
int choose_int8_ffn_variant(int requested, int64_t A, int E) {
  if (requested == 1 || requested == 2) return requested;
  return (A <= static_cast<int64_t>(36) * E) ? 1 : 2;
}
int choose_int8_down_variant(int requested, int64_t A, int E) {
  if (requested == 1 || requested == 2) return requested;
  return (A <= static_cast<int64_t>(52) * E) ? 1 : 2;
}

// Widening the codes into the workspace and running the direct-to-LDS tiles
// overtakes the tiled kernel's in-register widening only for large batches,
// since the widening itself streams the codes and writes twice their bytes.
// Down (8x7B shape, us, tiled vs widened): 861 vs 869 at 768 rows per expert,
// 1053 vs 1042 at 1024, 1478 vs 1398 at 1536. Gate/up: the tiled kernel wins
// at every size measured (1536 rows per expert: 2463 vs 2782; 2048: 3271 vs
// 3495), being about 3% slower per row than the direct-to-LDS kernel while
// widening w1 and w3 costs about 0.47 ms per call; the two meet near 8192 rows
// per expert (extrapolated), where widening starts.
bool int8_gate_up_dma(int64_t A, int k, int d, int ffn, int E) {
  return A >= static_cast<int64_t>(8192) * E && dma_gate_up_ok(A, k, d, ffn, E);
}
bool int8_down_dma(int64_t A, int d, int ffn, int E) {
  return A >= static_cast<int64_t>(1024) * E && dma_down_ok(A, d, ffn, E);
}

int int8_down_splits(int variant, int64_t A, int d, int ffn, int E) {
  if (variant != 1 && int8_down_dma(A, d, ffn, E)) return dma_down_splits(A, d, ffn, E);
  if (variant != 1 && d % 256 == 0) return tiled_down_splits(A, d, ffn, E);
  return down_splits(1, A, d, ffn, E);
}

size_t int8_wide_bytes(int64_t A, int k, int d, int ffn, int E) {
  const size_t m = static_cast<size_t>(E) * ffn * d * 2;  // one widened matrix
  size_t b = 0;
  if (int8_gate_up_dma(A, k, d, ffn, E)) b = 2 * m;        // w1 and w3
  if (int8_down_dma(A, d, ffn, E) && m > b) b = m;          // w2, after gate/up is done
  return b;
}

hipError_t launch_quantize_int8(const uint16_t* w, int E, int rows, int cols, void* out,
                                hipStream_t s) {
  const int64_t nrows = static_cast<int64_t>(E) * rows;
  int8_t* codes = static_cast<int8_t*>(out);
  float* scales = reinterpret_cast<float*>(static_cast<char*>(out) +
                                           align256(static_cast<size_t>(E) * rows * cols));
  hipLaunchKernelGGL(quantize_kernel, dim3(static_cast<unsigned>((nrows + 3) / 4)), dim3(256), 0, s,
                     w, nrows, rows, cols, codes, scales);
  return hipGetLastError();
}

hipError_t launch_gate_up_int8(int variant, const uint16_t* x, const void* w1, const void* w3,
                               const int32_t* offsets, const int32_t* sorted_asg, int64_t A,
                               int d, int ffn, int E, int k, uint16_t* h, hipStream_t s) {
  const size_t cb = align256(static_cast<size_t>(E) * ffn * d);
  const int8_t* q1 = static_cast<const int8_t*>(w1);
  const int8_t* q3 = static_cast<const int8_t*>(w3);
  const float* s1 = reinterpret_cast<const float*>(static_cast<const char*>(w1) + cb);
  const float* s3 = reinterpret_cast<const float*>(static_cast<const char*>(w3) + cb);
  if (variant != 1 && ffn % 128 == 0)
    return launch_gate_up_w8_tiled(x, q1, q3, s1, s3, offsets, sorted_asg, A, d, ffn, E, k, h, s);
  if (ffn % (16 * kW8GateUpRT) != 0)
    hipLaunchKernelGGL((gate_up_w8_kernel<1, kW8GateUpU>), dim3(ffn / 16, E), dim3(kWave * kW8Waves),
                       0, s, x, q1, s1, q3, s3, offsets, sorted_asg, d, ffn, k, h);
  else
    hipLaunchKernelGGL((gate_up_w8_kernel<kW8GateUpRT, kW8GateUpU>), dim3(ffn / (16 * kW8GateUpRT), E),
                       dim3(kWave * kW8Waves), 0, s, x, q1, s1, q3, s3, offsets, sorted_asg, d, ffn,
                       k, h);
  return hipGetLastError();
}

hipError_t launch_down_int8(int variant, const uint16_t* h, const void* w2,
                            const int32_t* offsets, int64_t A, int d, int ffn, int E, int nsplit,
                            float* part, hipStream_t s) {
  const size_t cb = align256(static_cast<size_t>(E) * d * ffn);
  const int8_t* q2 = static_cast<const int8_t*>(w2);
  const float* s2 = reinterpret_cast<const float*>(static_cast<const char*>(w2) + cb);
  if (variant != 1 && d % 256 == 0)
    return launch_down_w8_tiled(h, q2, s2, offsets, A, d, ffn, E, nsplit, part, s);
  const int rt = (d % (16 * kW8DownRT) == 0) ? kW8DownRT : 1;
  const unsigned blocks = static_cast<unsigned>((d / (16 * rt) * nsplit + kW8Waves - 1) / kW8Waves);
  if (rt != kW8DownRT) {
    hipLaunchKernelGGL((down_w8_kernel<1, kW8DownU>), dim3(blocks, E), dim3(kWave * kW8Waves), 0,
                       s, h, q2, s2, offsets, ffn, d, static_cast<int>(A), nsplit, part);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((down_w8_kernel<kW8DownRT, kW8DownU>), dim3(blocks, E), dim3(kWave * kW8Waves), 0, s, h, q2,
                     s2, offsets, ffn, d, static_cast<int>(A), nsplit, part);
  return hipGetLastError();
}

}  // namespace moe
