// Router + scoring: logits = x . router^T (+bias), float32 softmax over the
// experts, top-k (largest first, exact ties to the lower expert index) and
// renormalisation of the kept probabilities (nnterp Mixtral page, "The Notes":
// the router renormalizes its top 2 in float32; support(): router_logits is
// the router's linear output, before the scoring).
//
// With a norm (NORM), the router and the experts read the normed stream
// instead of x (nnterp Mixtral page, "The Notes": the block calls the MLP on
// post_attention_layernorm(h), a MixtralRMSNorm with eps = rms_norm_eps,
// MixtralConfig): a first pass over the token rows sums their squares, and
// the second pass forms n[t,i] = (x[t,i] * r_t) * gamma[i] in float32 with
// r_t = 1 / sqrt(sum_i x[t,i]^2 / d + eps), rounds it once to the input's
// type, stores it to norm_out and feeds that stored value to the logits.
//
// Work split (latency first: a decode batch has only a few dozen tokens): a
// workgroup of 256 threads takes TB tokens and splits the hidden dimension
// across all its threads in 8-element chunks (16-byte loads), so every load
// of a token row and of the router is in flight at once. Each thread then
// holds TB x EM float32 partial sums (token x expert); a reduce-scatter
// across the wave (halving steps, then butterflies) leaves lane l with the
// wave's sum for value l, the four waves meet in LDS in a fixed order, and
// one thread per token finishes the scoring. TB = 1 for batches of up to 256
// tokens (one workgroup per token, the most CUs and the least arithmetic per
// workgroup), else 64 / EM (fewer re-reads of the router rows).
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kVals = 64;  // partial sums per thread at most: tokens per block x EM

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

// One halving step of the reduce-scatter: lanes with bit O set keep the
// upper half of the O*2 live values, the others the lower half, and each adds
// the half its partner (lane ^ O) gives away.
template <int O, int NV>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[NV], bool upper) {
#pragma unroll
  for (int i = 0; i < O; ++i) {
    const float keep = upper ? v[i + O] : v[i];
    const float give = upper ? v[i] : v[i + O];
    v[i] = keep + __shfl_xor(give, O, kWave);
  }
}

// v[0..NV-1] in every lane (NV a power of two <= 64) -> lane l returns the
// sum over the wave of v[l % NV]: halving steps while values remain, then
// butterflies between the lane groups that hold partial sums of one value.
template <int NV>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[NV], int lane) {
  if constexpr (NV > 32) reduce_scatter_step<32>(v, (lane & 32) != 0);
  if constexpr (NV > 16) reduce_scatter_step<16>(v, (lane & 16) != 0);
  if constexpr (NV > 8) reduce_scatter_step<8>(v, (lane & 8) != 0);
  if constexpr (NV > 4) reduce_scatter_step<4>(v, (lane & 4) != 0);
  if constexpr (NV > 2) reduce_scatter_step<2>(v, (lane & 2) != 0);
  if constexpr (NV > 1) reduce_scatter_step<1>(v, (lane & 1) != 0);
  float r = v[0];
#pragma unroll
  for (int o = NV; o < kWave; o <<= 1) r += __shfl_xor(r, o, kWave);
  return r;
}

// normed value of x (float32) at hidden index i, rounded to the stored type
template <bool BF16>
__device__ __forceinline__ float norm1(float x, float r, float g) {
  const float v = (x * r) * g;
  if constexpr (BF16) return bf16_to_f32(f32_to_bf16(v));
  return v;
}

template <bool BF16>
__device__ __forceinline__ void store8(void* out, int64_t row, int d, int i, const float* v) {
  if constexpr (BF16) {
    u32x4 q;
#pragma unroll
    for (int h = 0; h < 4; ++h) q[h] = pack_bf16x2(v[2 * h], v[2 * h + 1]);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + row * d + i) = q;
  } else {
    float* p = static_cast<float*>(out) + row * d + i;
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// Scoring of token t from its EM logits (entries e >= E unused): + bias,
// optional logits out, float32 softmax over the E experts, top-k on the
// logits (strict '>' keeps the lower index on an exact tie), renormalised
// weights.
template <int EM>
__device__ __forceinline__ void score_token(float (&l)[EM], const float* __restrict__ bias,
                                            int64_t t, int E, int k, float* __restrict__ logits_out,
                                            int32_t* __restrict__ idx, float* __restrict__ wout) {
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

// EM: compile-time bound on E (8 or 32); TB tokens per block (TB * EM <= 64).
// VEC: x, router, gamma and norm_out rows are 16-byte aligned and d % 8 == 0.
// NORM: route the RMS-normed rows (gamma [d] float32, eps) and store them.
template <bool BF16, int EM, int TB, bool VEC, bool NORM>
__global__ __launch_bounds__(kThreads, 1) void route_kernel(
    const void* __restrict__ x, const float* __restrict__ router, const float* __restrict__ bias,
    int64_t T, int d, int E, int k, float* __restrict__ logits_out, int32_t* __restrict__ idx,
    float* __restrict__ wout, const float* __restrict__ gamma, float eps,
    void* __restrict__ norm_out) {
  constexpr int NV = TB * EM;
  static_assert(NV <= kVals && (NV & (NV - 1)) == 0, "TB * EM: a power of two up to 64");
  __shared__ float s_part[kWavesPerBlock][NV];
  __shared__ float s_logit[NV];
  __shared__ float s_ss[kWavesPerBlock][TB];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TB;

  float acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.0f;

  int64_t rows[TB];
  bool live[TB];
#pragma unroll
  for (int tt = 0; tt < TB; ++tt) {
    live[tt] = (t0 + tt) < T;
    rows[tt] = live[tt] ? t0 + tt : 0;
  }

  // router rows e >= E (when E < EM) read row E-1: every load and FMA is
  // unconditional, so all loads of a chunk are in flight together; those
  // sums are never used
  const float* rrow[EM];
#pragma unroll
  for (int e = 0; e < EM; ++e) rrow[e] = router + static_cast<int64_t>(e < E ? e : E - 1) * d;

  // per-token factor r_t of the norm (first pass: sums of squares, reduced
  // over the wave by a butterfly and over the waves in LDS in a fixed order)
  float rs[TB];
#pragma unroll
  for (int tt = 0; tt < TB; ++tt) rs[tt] = 1.0f;
  if constexpr (NORM) {
    float ss[TB];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) ss[tt] = 0.0f;
    int i0 = 0;
    if constexpr (VEC) {
      for (int c = tid; c < d / 8; c += kThreads) {
        float xv[TB][8];
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) load8<BF16>(x, rows[tt], d, c * 8, xv[tt]);
#pragma unroll
        for (int tt = 0; tt < TB; ++tt)
#pragma unroll
          for (int v = 0; v < 8; ++v) ss[tt] = fmaf(xv[tt][v], xv[tt][v], ss[tt]);
      }
      i0 = d / 8 * 8;
    }
    for (int i = i0 + tid; i < d; i += kThreads) {
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        const float xs = load1<BF16>(x, rows[tt], d, i);
        ss[tt] = fmaf(xs, xs, ss[tt]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
      float v = ss[tt];
#pragma unroll
      for (int o = kWave / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
      if (lane == 0) s_ss[wave][tt] = v;
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
      float v = s_ss[0][tt];
#pragma unroll
      for (int w = 1; w < kWavesPerBlock; ++w) v += s_ss[w][tt];
      rs[tt] = 1.0f / sqrtf(v / static_cast<float>(d) + eps);
    }
  }

  int tail_start = 0;
  if constexpr (VEC) {
    const int nvec = d / 8;
    for (int c = tid; c < nvec; c += kThreads) {
      const int i = c * 8;
      float xv[TB][8];
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) load8<BF16>(x, rows[tt], d, i, xv[tt]);
      float g8[8];
      if constexpr (NORM) {
        const float4 ga = *reinterpret_cast<const float4*>(gamma + i);
        const float4 gb = *reinterpret_cast<const float4*>(gamma + i + 4);
        g8[0] = ga.x; g8[1] = ga.y; g8[2] = ga.z; g8[3] = ga.w;
        g8[4] = gb.x; g8[5] = gb.y; g8[6] = gb.z; g8[7] = gb.w;
      }
      float4 ra[EM], rb[EM];
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        ra[e] = *reinterpret_cast<const float4*>(rrow[e] + i);
        rb[e] = *reinterpret_cast<const float4*>(rrow[e] + i + 4);
      }
      // keep every load of the chunk ahead of the arithmetic (one round trip)
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NORM) {
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) {
#pragma unroll
          for (int v = 0; v < 8; ++v) xv[tt][v] = norm1<BF16>(xv[tt][v], rs[tt], g8[v]);
          if (live[tt]) store8<BF16>(norm_out, rows[tt], d, i, xv[tt]);
        }
      }
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        const float r8[8] = {ra[e].x, ra[e].y, ra[e].z, ra[e].w, rb[e].x, rb[e].y, rb[e].z, rb[e].w};
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) {
          float a = acc[tt * EM + e];
#pragma unroll
          for (int v = 0; v < 8; ++v) a = fmaf(live[tt] ? xv[tt][v] : 0.0f, r8[v], a);
          acc[tt * EM + e] = a;
        }
      }
    }
    tail_start = nvec * 8;
  }
  for (int i = tail_start + tid; i < d; i += kThreads) {
    float xs[TB];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) xs[tt] = live[tt] ? load1<BF16>(x, rows[tt], d, i) : 0.0f;
    if constexpr (NORM) {
      const float g = gamma[i];
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        xs[tt] = norm1<BF16>(xs[tt], rs[tt], g);
        if (live[tt]) {
          if constexpr (BF16) static_cast<uint16_t*>(norm_out)[rows[tt] * d + i] = f32_to_bf16(xs[tt]);
          else static_cast<float*>(norm_out)[rows[tt] * d + i] = xs[tt];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EM; ++e) {
      const float r = rrow[e][i];
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) acc[tt * EM + e] = fmaf(xs[tt], r, acc[tt * EM + e]);
    }
  }

  const float part = wave_reduce_scatter<NV>(acc, lane);
  if (lane < NV) s_part[wave][lane] = part;
  __syncthreads();
  if (tid < NV) {
    float sum = s_part[0][tid];
#pragma unroll
    for (int w = 1; w < kWavesPerBlock; ++w) sum += s_part[w][tid];
    s_logit[tid] = sum;
  }
  __syncthreads();
  if (tid >= TB) return;
  const int64_t t = t0 + tid;
  if (t >= T) return;

  float l[EM];
#pragma unroll
  for (int e = 0; e < EM; ++e) l[e] = s_logit[tid * EM + e];
  score_token<EM>(l, bias, t, E, k, logits_out, idx, wout);
}

// Large batches: the logits as a small GEMM on fp32 MFMA
// (v_mfma_f32_16x16x4_f32: 16 tokens x 4 k x 16 experts, float32 operands
// and accumulation). A workgroup takes 16 tokens and all E experts (one or two
// 16-expert tiles); its 8 waves split d into 8 slices, each walked in groups
// of 64 k. A group is loaded in whole cache lines (tokens: 8 rows x 128 bytes
// per load, lane l row l / 8, 16-byte chunk l % 8; router: 4 rows x 256 bytes,
// lane l row l / 16, chunk l % 16), the next group's loads in flight while the
// wave works on this one; the wave writes the group into its own LDS area
// (chunk c of row r at slot c ^ (r % 8) for tokens, c ^ (r % 16) for router
// rows; no barrier: only the wave reads it back, and a wave's LDS operations
// complete in order) and reads the MFMA operands from there: in a 32-k step
// lane (t, q) = (l % 16, l / 16) takes token t's 8 values 8q .. 8q+7 (16
// bytes of bf16, widened) and, per expert tile, expert (l % 16)'s router
// values at the same k (32 bytes); MFMA i of the step multiplies value i of
// both, so the 8 MFMAs cover the 32 k of the step. (Read straight from global
// memory in that operand layout, every load touched 16 rows 8 or 16 KiB apart:
// the same bytes as whole lines measured a fifth faster.) The router is read
// once per 16 tokens. The waves' partial sums meet in LDS in a fixed order;
// one thread per token then scores it. Needs d % 512 == 0 (whole groups per
// wave), x and router 16-byte aligned, E <= 32.
constexpr int kMfmaWaves = 8;
constexpr int kGroupK = 64;  // k of one group

template <int NT>  // expert tiles of 16
__global__ __launch_bounds__(kWave* kMfmaWaves, 1) void route_mfma_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ router,
    const float* __restrict__ bias, int64_t T, int d, int E, int k, float* __restrict__ logits_out,
    int32_t* __restrict__ idx, float* __restrict__ wout) {
  constexpr int EM = 16 * NT;
  constexpr int kXBytes = 16 * kGroupK * 2;   // 16 token rows x 64 k bf16 (2 KiB)
  constexpr int kRBytes = EM * kGroupK * 4;   // EM router rows x 64 k fp32
  constexpr int kRLoads = EM / 4;             // router loads per group (4 rows each)
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[kMfmaWaves][kXBytes + kRBytes];
  __shared__ f32x4 s_part[kMfmaWaves][NT][kWave];
  __shared__ float s_logit[16][EM];
  __shared__ float s_l[16][32];  // scoring: logits + bias, exponentials
  __shared__ float s_p[16][32];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int t = lane & 15, q = lane >> 4;
  uint8_t* xs = s_stage[wave];
  uint8_t* rs = s_stage[wave] + kXBytes;

  // global loads of a group (k0 = its first k): tokens rows 8i + l/8 (rows past
  // the batch read the last row), router rows 4i + l/16 (rows of experts >= E
  // load nothing: zeros, whose sums are unused)
  const int xr = lane >> 3, xc = lane & 7;
  const int rr = lane >> 4, rc = lane & 15;
  const uint16_t* xrow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) xrow[i] = x + min(t0 + 8 * i + xr, T - 1) * d + 8 * xc;
  auto load_group = [&](int k0, u32x4 (&xv)[2], float4 (&rv)[kRLoads]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) xv[i] = ldg16(xrow[i] + k0);
#pragma unroll
    for (int i = 0; i < kRLoads; ++i) {
      const int e = 4 * i + rr;
      rv[i] = e < E ? *reinterpret_cast<const float4*>(router + static_cast<int64_t>(e) * d + k0 + 4 * rc)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto use_group = [&](const u32x4 (&xv)[2], const float4 (&rv)[kRLoads]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * i + xr;
      *reinterpret_cast<u32x4*>(xs + r * 128 + ((xc ^ (r & 7)) * 16)) = xv[i];
    }
#pragma unroll
    for (int i = 0; i < kRLoads; ++i) {
      const int e = 4 * i + rr;
      *reinterpret_cast<float4*>(rs + e * 256 + ((rc ^ (e & 15)) * 16)) = rv[i];
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {  // 32-k steps of the group
      const int cx = 4 * s + q;    // token chunk: k 32s + 8q .. +7
      const u32x4 xw = *reinterpret_cast<const u32x4*>(xs + t * 128 + ((cx ^ (t & 7)) * 16));
      float xf[8];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        xf[2 * h] = __uint_as_float(xw[h] << 16);
        xf[2 * h + 1] = __uint_as_float(xw[h] & 0xFFFF0000u);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int e = 16 * nt + t;
        const int c0 = 8 * s + 2 * q;  // router chunks: k 32s + 8q .. +3, +4 .. +7
        const float4 a = *reinterpret_cast<const float4*>(rs + e * 256 + ((c0 ^ t) * 16));
        const float4 b = *reinterpret_cast<const float4*>(rs + e * 256 + (((c0 + 1) ^ t) * 16));
        const float rf[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xf[i], rf[i], acc[nt], 0, 0, 0);
      }
    }
  };
  // this wave's groups, two at a time (two register sets: the next group's
  // loads are in flight while this one is used)
  const int ng = d / kGroupK / kMfmaWaves;  // groups per wave (d % 512 == 0)
  const int kb = wave * ng * kGroupK;
  u32x4 xa[2], xb[2];
  float4 ra[kRLoads], rb[kRLoads];
  load_group(kb, xa, ra);
  for (int g = 0; g < ng; g += 2) {
    if (g + 1 < ng) load_group(kb + (g + 1) * kGroupK, xb, rb);
    use_group(xa, ra);
    if (g + 1 < ng) {
      if (g + 2 < ng) load_group(kb + (g + 2) * kGroupK, xa, ra);
      use_group(xb, rb);
    }
  }
  // lane l holds tokens 4 (l / 16) + i of expert 16 nt + l % 16
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) s_part[wave][nt][lane] = acc[nt];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 v = s_part[0][nt][lane];
#pragma unroll
      for (int w = 1; w < kMfmaWaves; ++w) v += s_part[w][nt][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) s_logit[4 * q + i][16 * nt + t] = v[i];
    }
  }
  __syncthreads();
  // scoring, as score_token computes it: 32 lanes per token (lane e: expert
  // e) add the bias, write the logits out, take the maximum (an exact
  // operation in any order) and their exponentials; the token's first lane
  // then sums the probabilities and selects the top k in expert order, with
  // the same operations on the same values as score_token
  {
    const int tt = tid >> 5, e = tid & 31;
    const int64_t tok = t0 + tt;
    const bool valid = e < E;
    float le = valid ? s_logit[tt][e] : -INFINITY;
    if (valid && bias) le += bias[e];
    if (valid && logits_out && tok < T) logits_out[tok * E + e] = le;
    float m = valid ? le : -INFINITY;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    s_l[tt][e] = le;
    s_p[tt][e] = valid ? expf(le - m) : 0.0f;
    // (the lanes of a token share a wave, whose LDS operations complete in order)
    if (e != 0 || tok >= T) return;
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < EM; ++j) sum += s_p[tt][j];
    uint32_t taken = 0;
    float psum = 0.0f;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      float bl = 0.0f;
#pragma unroll
      for (int x = 0; x < EM; ++x) {
        const float lx = s_l[tt][x];
        if (x < E && !((taken >> x) & 1u) && (best < 0 || lx > bl)) {
          best = x;
          bl = lx;
        }
      }
      if (best < 0) {  // only with NaN logits: take the lowest free expert
#pragma unroll
        for (int x = EM - 1; x >= 0; --x)
          if (x < E && !((taken >> x) & 1u)) best = x;
      }
      taken |= 1u << best;
      const float bp = s_p[tt][best] / sum;
      idx[tok * k + j] = best;
      psum += bp;
      wout[tok * k + j] = bp;  // rescaled below
    }
    for (int j = 0; j < k; ++j) wout[tok * k + j] = wout[tok * k + j] / psum;
  }
}

constexpr int64_t kSmallBatch = 256;

template <bool BF16, int EM, bool NORM>
hipError_t launch_em(const void* x, const float* router, const float* bias, int64_t T, int d,
                     int E, int k, float* logits_out, int32_t* idx, float* w,
                     const float* gamma, float eps, void* norm_out, hipStream_t s) {
  // one token per block while the batch leaves CUs free (a decode batch: each
  // block then does 1/TB of the arithmetic), else kVals / EM tokens per block
  // so that the router rows are read by fewer blocks
  constexpr int kBig = kVals / EM;
  const int64_t per_block = T <= kSmallBatch ? 1 : kBig;
  const dim3 grid(static_cast<unsigned>((T + per_block - 1) / per_block));
  const dim3 block(kThreads);
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec = (d % 8 == 0) && a16(x) && a16(router) && (!NORM || (a16(gamma) && a16(norm_out)));
  if (per_block == 1) {
    if (vec)
      hipLaunchKernelGGL((route_kernel<BF16, EM, 1, true, NORM>), grid, block, 0, s, x, router,
                         bias, T, d, E, k, logits_out, idx, w, gamma, eps, norm_out);
    else
      hipLaunchKernelGGL((route_kernel<BF16, EM, 1, false, NORM>), grid, block, 0, s, x, router,
                         bias, T, d, E, k, logits_out, idx, w, gamma, eps, norm_out);
  } else if (vec) {
    hipLaunchKernelGGL((route_kernel<BF16, EM, kBig, true, NORM>), grid, block, 0, s, x, router,
                       bias, T, d, E, k, logits_out, idx, w, gamma, eps, norm_out);
  } else {
    hipLaunchKernelGGL((route_kernel<BF16, EM, kBig, false, NORM>), grid, block, 0, s, x, router,
                       bias, T, d, E, k, logits_out, idx, w, gamma, eps, norm_out);
  }
  return hipGetLastError();
}

template <bool BF16, bool NORM>
hipError_t launch_bf(const void* x, const float* router, const float* bias, int64_t T, int d,
                     int E, int k, float* logits_out, int32_t* idx, float* w,
                     const float* gamma, float eps, void* norm_out, hipStream_t s) {
  if (E <= 8)
    return launch_em<BF16, 8, NORM>(x, router, bias, T, d, E, k, logits_out, idx, w, gamma, eps,
                                    norm_out, s);
  return launch_em<BF16, 32, NORM>(x, router, bias, T, d, E, k, logits_out, idx, w, gamma, eps,
                                   norm_out, s);
}

}  // namespace

hipError_t launch_route(const void* x, int x_bf16, const float* router, const float* bias,
                        int64_t T, int d, int E, int k, float* logits_out, int32_t* idx,
                        float* w, hipStream_t s, const float* gamma, float eps, void* norm_out) {
  if (T == 0) return hipSuccess;
  if (gamma) {
    if (x_bf16)
      return launch_bf<true, true>(x, router, bias, T, d, E, k, logits_out, idx, w, gamma, eps,
                                   norm_out, s);
    return launch_bf<false, true>(x, router, bias, T, d, E, k, logits_out, idx, w, gamma, eps,
                                  norm_out, s);
  }
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  // (measured at T = 4096, d = 4096, bench events: 32 experts 140 us scalar,
  // 49 us with the first MFMA kernel, whose loads each touched 16 rows and
  // whose 16 scoring threads each ran a 32-expert softmax, 36 us now; 16
  // experts 28 -> 23 us; with 8 experts the scalar kernel stays faster at
  // T = 4096, 21 vs 24 us, though not at 8192, 36 vs 27)
  if (x_bf16 && E > 8 && T > kSmallBatch && d % (kGroupK * kMfmaWaves) == 0 &&
      a16(x) && a16(router)) {
    const dim3 grid(static_cast<unsigned>((T + 15) / 16));
    if (E <= 16)
      hipLaunchKernelGGL(route_mfma_kernel<1>, grid, dim3(kWave * kMfmaWaves), 0, s,
                         static_cast<const uint16_t*>(x), router, bias, T, d, E, k, logits_out,
                         idx, w);
    else
      hipLaunchKernelGGL(route_mfma_kernel<2>, grid, dim3(kWave * kMfmaWaves), 0, s,
                         static_cast<const uint16_t*>(x), router, bias, T, d, E, k, logits_out,
                         idx, w);
    return hipGetLastError();
  }
  if (x_bf16)
    return launch_bf<true, false>(x, router, bias, T, d, E, k, logits_out, idx, w, nullptr, 0.0f,
                                  nullptr, s);
  return launch_bf<false, false>(x, router, bias, T, d, E, k, logits_out, idx, w, nullptr, 0.0f,
                                 nullptr, s);
}

}  // namespace moe
