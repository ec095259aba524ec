// Device helpers and internal launcher declarations shared by the libmoe
// translation units. gfx950 (CDNA4) only: wave64, bf16 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 32;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Two float32 -> bfloat16, round to nearest, ties to even, in one
// v_cvt_pk_bf16_f32 (lo in bits 0-15); for every non-NaN input the same bits
// as rounding the float32 bit pattern by hand (u + 0x7FFF + lsb, >> 16).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f));
}

// SiLU(z) = z / (1 + exp(-z)) in float32, the division as a multiply by the
// hardware reciprocal (v_rcp_f32, 1 ulp): the gate/up epilogues evaluate one
// per output, and h is rounded to bfloat16 right after. Limits: 1 + exp(-z)
// = inf for very negative z gives -0, as the division does.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// 16 bytes (8 bf16) as an MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D += A(16x32) * B(32x16); lane l holds A row (l%16), k-group (l/16) and the
// matching B column/k-group; D lane l holds column (l%16), rows 4*(l/16)+i.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// One 32-deep MFMA operand from a lane's 16 bytes of int8 weight codes: half
// 0 takes bytes 0-7, half 1 bytes 8-15. Each code is sign-extended to float32
// (v_cvt_f32_i32 with a byte select); a code is a small integer, so the top
// half of its float32 is its exact bfloat16 encoding, and v_perm_b32 joins
// two of those halves into one dword.
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t q, int b) {
  const float lo = static_cast<float>(static_cast<int32_t>(q << (24 - 8 * b)) >> 24);
  const float hi = static_cast<float>(static_cast<int32_t>(q << (16 - 8 * b)) >> 24);
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ __forceinline__ u32x4 i8_operand(u32x4 q, int half) {
  const uint32_t a = q[2 * half], b = q[2 * half + 1];
  return u32x4{i8x2_to_bf16x2(a, 0), i8x2_to_bf16x2(a, 2), i8x2_to_bf16x2(b, 0),
               i8x2_to_bf16x2(b, 2)};
}

// element offset of w[e][n][k] (k a multiple of 8) of an [E, N, K] weight in
// the standard layout (PACKED false) or in fragment order (PACKED true: 16-row
// x 32-k fragments of 1 KiB in MFMA lane order, ordered expert, row tile, k step)
template <bool PACKED>
__device__ __forceinline__ size_t wofs(int e, int n, int k, int N, int K) {
  if constexpr (PACKED) {
    return ((static_cast<size_t>(e) * (N >> 4) + (n >> 4)) * static_cast<size_t>(K >> 5) +
            (k >> 5)) * 512 + ((((k & 31) >> 3) << 4) + (n & 15)) * 8;
  } else {
    return (static_cast<size_t>(e) * N + n) * K + k;
  }
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// f(integral_constant<int, I>) for I in Is, in order: a loop unrolled with the
// index as a compile-time constant (fixed register sets, immediate offsets)
template <typename F, int... Is>
__device__ __forceinline__ void unrolled(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}

// Workgroup barrier for handing LDS data between waves. __syncthreads() also
// orders global memory, which here means waiting for every global load still
// in flight; a software pipeline that keeps loads in flight across the
// barrier only needs this wave's LDS operations finished (lgkmcnt = 0; vmcnt
// and expcnt left at their maxima, 63 and 7, in the gfx9 s_waitcnt encoding)
// and the hardware barrier. The signal fences stop the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------------------
// internal launchers (host side); each returns hipSuccess or the launch error
// ---------------------------------------------------------------------------
// with gamma non-null the router reads the RMS-normed rows (eps) and stores
// them, in x's type, to norm_out
hipError_t launch_route(const void* x, int x_bf16, const float* router, const float* bias,
                        int64_t T, int d, int E, int k, float* logits_out, int32_t* idx,
                        float* w, hipStream_t s, const float* gamma = nullptr, float eps = 0.0f,
                        void* norm_out = nullptr);

hipError_t launch_check_routing(const int32_t* idx, int64_t T, int k, int E, int32_t* bad,
                                hipStream_t s);
hipError_t launch_permute(const int32_t* idx, int64_t A, int E, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_asg, int32_t* asg_pos,
                          hipStream_t s);

// The permutation done by the streaming gate/up kernel itself (few
// assignments): the expert ids and the arrays moe_permute would write.
struct FusedPermute {
  const int32_t* idx;  // [A] expert ids (topk_idx)
  int32_t* counts;     // [E]
  int32_t* offsets;    // [E + 1]
  int32_t* sorted_asg; // [A]
  int32_t* asg_pos;    // [A]
};
constexpr int kFusedPermuteMaxA = 512;
// whether the bf16 gate/up kernel of this resolved family takes the
// permutation over for A assignments
bool gate_up_fuses_permute(int variant, int64_t A);
// bf16 experts: gate/up (+SiLU*mul) -> h [A, ffn] bf16, down -> y [A, d] f32.
// `variant` is resolved (1 streaming, 2 tiled); `packed` selects the
// fragment-order weight layout. The down kernel writes up to
// down_splits(variant, A, d, ffn, E) float32 partial results [nsplit, A, d]
// whose sum (in split order) is y; the count depends on the sizes (and, for
// the direct-to-LDS kernel, the expert counts), not on the layout, so both
// layouts give bit-identical y.
// fp non-null (only where gate_up_fuses_permute): offsets and sorted_asg
// are not read, the kernel writes fp's arrays
hipError_t launch_gate_up_bf16(int variant, bool packed, const uint16_t* x, const uint16_t* w1,
                               const uint16_t* w3, const int32_t* offsets,
                               const int32_t* sorted_asg, int64_t A, int d, int ffn, int E,
                               int k, uint16_t* h, hipStream_t s,
                               const FusedPermute* fp = nullptr);
// The direct-to-LDS down kernel's K split: the caller's choice (0 = made on
// the device from the expert counts, -1 = none, 8..13 = a first part of that
// many sixteenths of K) and a device int32 (or null) that receives the number
// of partial arrays it wrote (1 or 2; at most down_splits(...)).
struct DownSplit {
  int opt = 0;
  int32_t* word = nullptr;
};
hipError_t launch_down_bf16(int variant, bool packed, const uint16_t* h, const uint16_t* w2,
                            const int32_t* offsets, int64_t A, int d, int ffn, int E, float* part,
                            hipStream_t s, DownSplit ds = {});
// the most partial arrays the down kernel of this resolved family writes; for
// the direct-to-LDS kernel (down_dma_runs) the count it used goes to ds.word
int down_splits(int variant, int64_t A, int d, int ffn, int E);
bool down_dma_runs(int variant, int64_t A, int d, int ffn, int E);
// K split of the tiled down kernels below the direct-to-LDS sizes: 2 while
// the 256-row tiles would leave CUs idle (d % 256 == 0, ffn % 128 == 0), else 1
int tiled_down_splits(int64_t A, int d, int ffn, int E);
// int8 codes (16-row x 64-k blocks) with float32 row scales on the tiled
// weights-in-registers kernel, operands widened in registers: gate/up needs
// ffn % 128 == 0, down d % 256 == 0 and nsplit partials as tiled_down_splits
hipError_t launch_gate_up_w8_tiled(const uint16_t* x, const void* q1, const void* q3,
                                  const float* s1, const float* s3, const int32_t* offsets,
                                  const int32_t* sorted_asg, int64_t A, int d, int ffn, int E,
                                  int k, uint16_t* h, hipStream_t s);
hipError_t launch_down_w8_tiled(const uint16_t* h, const void* q2, const float* s2,
                               const int32_t* offsets, int64_t A, int d, int ffn, int E,
                               int nsplit, float* part, hipStream_t s);

// gate/up and down for many rows per expert with direct-to-LDS loads
// (ffn_dma.hip), for fragment-order (packed) or row-major weights: the sizes
// they are used for, the K split of the down projection (1 or 2) and the
// launchers; optional float32 row scales [E, rows] multiply the finished sums
// (int8 codes widened to bfloat16)
bool dma_gate_up_ok(int64_t A, int k, int d, int ffn, int E);
hipError_t launch_gate_up_dma(bool packed, const uint16_t* x, const uint16_t* w1,
                              const uint16_t* w3, const int32_t* offsets,
                              const int32_t* sorted_asg, int64_t A, int d, int ffn, int E, int k,
                              uint16_t* h, hipStream_t s, const float* s1 = nullptr,
                              const float* s3 = nullptr);
bool dma_down_ok(int64_t A, int d, int ffn, int E);
int dma_down_splits(int64_t A, int d, int ffn, int E);
hipError_t launch_down_dma(bool packed, const uint16_t* h, const uint16_t* w2,
                           const int32_t* offsets, int64_t A, int d, int ffn, int E,
                           int max_split, float* part, hipStream_t s, const float* s2,
                           DownSplit ds);
// weight-only int8 experts (ffn_int8.hip): bytes of one quantized matrix
// (codes, then float32 row scales at the next 256-byte boundary), the
// quantizer, and the gate/up and down launchers that read it (`variant`
// resolved as for bf16: 1 streaming, 2 tiled)
size_t int8_weight_bytes(int E, int rows, int cols);
// the row scales inside a quantized matrix; prefill: whether gate/up and down
// widen the codes and run the direct-to-LDS kernels, the down K split, and
// the workspace bytes the widened matrices take (0 when neither does)
const float* int8_scales(const void* w, int E, int rows, int cols);
hipError_t launch_widen_int8(const void* w, int E, int rows, int cols, uint16_t* out,
                             hipStream_t s);
int choose_int8_ffn_variant(int requested, int64_t A, int E);   // gate/up
int choose_int8_down_variant(int requested, int64_t A, int E);  // down
bool int8_gate_up_dma(int64_t A, int k, int d, int ffn, int E);
bool int8_down_dma(int64_t A, int d, int ffn, int E);
int int8_down_splits(int variant, int64_t A, int d, int ffn, int E);
size_t int8_wide_bytes(int64_t A, int k, int d, int ffn, int E);
hipError_t launch_quantize_int8(const uint16_t* w, int E, int rows, int cols, void* out,
                                hipStream_t s);
hipError_t launch_gate_up_int8(int variant, const uint16_t* x, const void* w1, const void* w3,
                               const int32_t* offsets, const int32_t* sorted_asg, int64_t A,
                               int d, int ffn, int E, int k, uint16_t* h, hipStream_t s);
hipError_t launch_down_int8(int variant, const uint16_t* h, const void* w2,
                            const int32_t* offsets, int64_t A, int d, int ffn, int E, int nsplit,
                            float* part, hipStream_t s);
// standard [E, R, C] bf16 -> fragment order (16-row x 32-column fragments)
hipError_t launch_pack_bf16(const uint16_t* w, int E, int R, int C, uint16_t* out, hipStream_t s);

// f32 experts: same steps in float32 (h stays float32)
hipError_t launch_gate_up_f32(const float* x, const float* w1, const float* w3,
                              const int32_t* offsets, const int32_t* sorted_asg, int64_t A,
                              int d, int ffn, int E, int k, float* h, hipStream_t s);
hipError_t launch_down_f32(const float* h, const float* w2, const int32_t* offsets, int64_t A,
                           int d, int ffn, int E, float* y, hipStream_t s);

// out[t] = sum_j w[t*k+j] * y[asg_pos[t*k+j]] (+ residual[t] when residual is
// non-null, added after the slot sum; bf16 or float32 per res_bf16), with y
// the split-order sum of nsplit partial arrays of A x d floats (A = T*k)
// starting at `part`
// (ns_dev non-null: a device int32 holding the count actually written, at
// most nsplit, read by the kernels)
hipError_t launch_combine(const float* part, int nsplit, const int32_t* asg_pos, const float* w,
                          int64_t T, int d, int k, void* out, int out_bf16, hipStream_t s,
                          const void* residual = nullptr, int res_bf16 = 0,
                          const int32_t* ns_dev = nullptr);
// y[i] = sum_s part[s*n + i] in split order (ns_dev as for the combine)
hipError_t launch_sum_partials(const float* part, int nsplit, int64_t n, float* y, hipStream_t s,
                               const int32_t* ns_dev = nullptr);

// Resolved expert-FFN kernel family for these sizes (1 streaming, 2 tiled).
int choose_ffn_variant(int requested, int64_t A, int E);   // gate/up
int choose_down_variant(int requested, int64_t A, int E);  // down

}  // namespace moe
