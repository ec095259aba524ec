/*
 * moe.h -- C ABI of libmoe, the Mixtral sparse-MoE feed-forward layer on one
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (nnterp Mixtral encyclopedia page, "The API / support()" and
 * "The Notes"; Transformers Mixtral page, "Architectural details" and
 * MixtralConfig):
 *   logits[t,e] = x[t,:] . router[e,:]               (+ optional bias[e])
 *   p[t,:]      = softmax(logits[t,:])                in float32
 *   idx[t,0..k) = the k largest, largest first; w = p[idx] / sum(p[idx])
 *   out[t]      = sum_j w[t,j] * w2[e] (silu(w1[e] x[t]) * (w3[e] x[t])),  e = idx[t,j]
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: every tensor pointer is a DEVICE pointer (memory the caller got
 *   from hipMalloc or a framework allocator on the current device). The
 *   library never allocates, frees or synchronises; the caller owns every
 *   buffer. Inputs are read-only. Outputs are fully overwritten (no
 *   accumulation into them).
 * Layout: dense, row-major, no padding:
 *   x       [T, d]        dtype (MOE_F32 or MOE_BF16)
 *   router  [E, d]        float32 for every dtype
 *   w1, w3  [E, ffn, d]   gate and up projections (each expert's
 *                         nn.Linear(d -> ffn).weight), same dtype as x
 *   w2      [E, d, ffn]   down projection (nn.Linear(ffn -> d).weight)
 *   topk_idx [T, k] int32, topk_w [T, k] float32: slot j of token t is
 *   assignment a = t*k + j.
 * Stream: `stream` is a hipStream_t (NULL = the null stream). All work is
 *   enqueued on it in order and the call returns without waiting. The
 *   library keeps no state between calls (per-call choices travel in a
 *   moe_options argument), so calls are re-entrant: two calls may run
 *   concurrently, from any threads, on different streams if they use
 *   distinct outputs and workspaces (moe_forward_noalloc is the exception:
 *   its calls on one GPU share one scratch area).
 * Sizes: 0 <= T, T*k <= MOE_MAX_ASSIGNMENTS; 1 <= k <= E <= MOE_MAX_EXPERTS;
 *   d, ffn >= 1.
 *   T == 0 is valid: nothing is computed, except that moe_permute (and
 *   moe_forward's counts_out) still write zero counts and offsets.
 *   MOE_BF16 additionally needs d % 64 == 0,
 *   ffn % 64 == 0 and 16-byte aligned x/w1/w3/w2/workspace pointers, else
 *   MOE_ENOTSUP.
 * Errors: every function returns MOE_OK or an error code; arguments are
 *   checked before anything is enqueued, so on MOE_EINVAL / MOE_ENOTSUP /
 *   MOE_EWORKSPACE nothing ran. MOE_EHIP means the HIP runtime rejected a
 *   launch (the stream state is then the runtime's). No C++ exception and no
 *   abort crosses this boundary.
 * Device-side preconditions: expert ids in [0, E) and distinct within a
 *   token (moe_check_routing counts the tokens that break either, on the
 *   device); offsets, sorted_asg and asg_pos exactly as moe_permute produces
 *   them for the same T, k and E. moe_permute leaves expert ids out of range
 *   out of the grouping (asg_pos -1, which moe_combine skips); a repeated id
 *   is grouped twice like any other. Arrays that moe_permute did not produce
 *   give unspecified results and may be read or written out of bounds.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = 1,     /* bad pointer, size, dtype or k/E */
  MOE_ENOTSUP = 2,    /* valid but not supported (shape/alignment for bf16) */
  MOE_EWORKSPACE = 3, /* workspace missing or smaller than moe_workspace_bytes */
  MOE_EHIP = 4        /* the HIP runtime reported an error */
};

/* Element types. MOE_BF16_PACKED and MOE_INT8_PACKED are accepted only as
 * the `dtype` of moe_expert_ffn, moe_forward and moe_block_forward: x is
 * bfloat16 as for MOE_BF16, and w1, w3 and w2 are, for MOE_BF16_PACKED, the
 * bfloat16 weights rearranged by moe_pack_weight (same values, fragment
 * order) and, for MOE_INT8_PACKED, weight-only int8 matrices made by
 * moe_quantize_weight (codes plus float32 row scales); everything else is
 * unchanged. */
enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_BF16_PACKED = 2, MOE_INT8_PACKED = 3 };

#define MOE_MAX_EXPERTS 32
/* Largest T*k: 2^31 - 1024, so that the permutation's 1024-wide steps over
 * the assignments stay within 32-bit indices. */
#define MOE_MAX_ASSIGNMENTS 2147482624

/* Per-call options of moe_expert_ffn, moe_forward, moe_block_forward and
 * moe_forward_noalloc; NULL means every field at its default (0 / NULL).
 * The struct is read during the call only and nothing of it is kept.
 *   ffn_variant   expert-FFN kernel family for bf16 and int8 weights (float32
 *                 ignores it): 0 = chosen by size, per projection and weight
 *                 format; 1 = weight-streaming kernels (meant for few rows per
 *                 expert); 2 = tiled MFMA kernels (meant for many; which tile
 *                 kernel, and for int8 whether the codes are widened, still
 *                 follows the size), for both projections. Any other value is
 *                 MOE_EINVAL. The results are correct for every choice.
 *   stage_events  NULL, or an array of 6 hipEvent_t the caller created, for
 *                 profiling: the fused calls record events[0] before the
 *                 router, events[1] after it, then events[2..5] after the
 *                 permutation, the gate/up step, the down step and the
 *                 combine, all on their stream (a NULL entry is MOE_EINVAL).
 *                 moe_expert_ffn ignores it.
 *   down_split    K split of the down projection where the 256x256-tile
 *                 kernel runs with room for two partial sums (bf16 and int8
 *                 weights at prefill sizes; other kernels ignore it): 0 =
 *                 chosen on the device from the expert counts (default), -1 =
 *                 never split, 8..13 = a first part of that many sixteenths
 *                 of K (rounded down to a multiple of 128 columns). Other
 *                 values are MOE_EINVAL. Every choice is correct; they differ
 *                 in speed and in float32 summation order. */
typedef struct moe_options {
  int ffn_variant;
  void* const* stage_events;
  int down_split;
} moe_options;

/* Static description of a status code. Never NULL. */
const char* moe_strerror(int status);

/* Bytes of device workspace that moe_forward needs for these sizes; the same
 * amount is always enough for moe_permute and moe_expert_ffn. Pure host
 * function. Returns 0 for invalid arguments. With MOE_INT8_PACKED at large
 * prefill sizes (d and ffn multiples of 128) it includes room for weights
 * widened to bfloat16 (see moe_quantize_weight): E*ffn*d*2 bytes for w2 from
 * T*k >= 1024*E (d % 256 == 0), 2*E*ffn*d*2 for w1 and w3 from T*k >= 8192*E. */
size_t moe_workspace_bytes(int64_t T, int d, int ffn, int E, int k, int dtype);

/* Router + scoring (nnterp page, Notes: softmax over the experts in float32,
 * keep the k largest, divide them by their sum; slot 0 is the larger).
 *   x          [T, d] of x_dtype
 *   router     [E, d] float32
 *   logit_bias [E] float32 or NULL; added to the logits before the softmax
 *   logits_out [T, E] float32 or NULL; receives the pre-softmax logits (+bias)
 *   topk_idx   [T, k] int32 out; experts by decreasing logit, an exact tie
 *              goes to the lower expert index
 *   topk_w     [T, k] float32 out; renormalised weights, sum to 1 per token
 * Logits accumulate in float32. */
int moe_route(const void* x, int x_dtype, const float* router, const float* logit_bias,
              int64_t T, int d, int E, int k, float* logits_out, int32_t* topk_idx,
              float* topk_w, void* stream);

/* Grouping of the T*k assignments by expert (each token is dispatched to its
 * k experts: Transformers page, "Architectural details"). Integer only,
 * deterministic. Outputs:
 *   counts     [E]    assignments per expert
 *   offsets    [E+1]  exclusive prefix sum of counts, offsets[E] = T*k
 *   sorted_asg [T*k]  assignment ids a = t*k + j grouped by expert; within an
 *                     expert in increasing a (a stable counting sort)
 *   asg_pos    [T*k]  inverse: sorted_asg[asg_pos[a]] == a
 * An expert id outside [0, E) is not counted and gets asg_pos -1; offsets[E]
 * is then the number of assignments grouped, and sorted_asg past it is left
 * as it was.
 * ws/ws_bytes: reserved scratch; the current kernel needs none, so NULL/0
 * is accepted (any buffer passed is left untouched). */
int moe_permute(const int32_t* topk_idx, int64_t T, int E, int k, int32_t* counts,
                int32_t* offsets, int32_t* sorted_asg, int32_t* asg_pos, void* ws,
                size_t ws_bytes, void* stream);

/* Routing check for callers that pass their own expert ids to moe_permute
 * (a debugging aid; the router's own ids always pass). On the stream, writes
 * bad_out[0] = the number of tokens with an id outside [0, E) and bad_out[1]
 * = the number of tokens with an id repeated (a token is dispatched to k
 * distinct experts: Transformers page, "Architectural details"). topk_idx
 * [T, k] int32 device; bad_out int32[2] device. Same size checks as
 * moe_permute; T == 0 writes zeros. */
int moe_check_routing(const int32_t* topk_idx, int64_t T, int E, int k, int32_t* bad_out,
                      void* stream);

/* The experts on their grouped rows (nnterp page, support(): the down
 * projection receives act(gate) * up, act = SiLU):
 *   y[p] = w2[e] (silu(w1[e] x[r]) * (w3[e] x[r])),  r = sorted_asg[p] / k,
 * for every p in [offsets[e], offsets[e+1]). y [T*k, d] float32, unweighted,
 * in grouped order. offsets/sorted_asg are device arrays as produced by
 * moe_permute. For MOE_BF16 / MOE_BF16_PACKED the gate/up products
 * accumulate in float32, the SwiGLU activation is rounded to bfloat16 (the
 * down projection's MFMA input) and the down projection accumulates in
 * float32 (on few rows per expert, and on many where it packs the tiles
 * better onto the GPU, it splits K two ways and adds the two float32 partial
 * sums in a fixed order; the split depends on T, d, ffn, E, k, the per-expert
 * row counts and options->down_split only, so MOE_BF16 and MOE_BF16_PACKED
 * give bit-identical y). ws must hold moe_workspace_bytes(T, d, ffn, E, k,
 * dtype) bytes. options: NULL or per-call options (kernel family, down
 * split). */
int moe_expert_ffn(const void* x, int dtype, const void* w1, const void* w3, const void* w2,
                   const int32_t* offsets, const int32_t* sorted_asg, int64_t T, int d,
                   int ffn, int E, int k, float* y, void* ws, size_t ws_bytes, void* stream,
                   const moe_options* options);

/* Gate-weighted sum back in token order (nnterp page, Notes: each slot's
 * weighted expert output, summed over the slots, is the layer output):
 *   out[t] = sum_{j=0..k-1} topk_w[t*k+j] * y[asg_pos[t*k+j]]
 * accumulated in float32 in slot order; out [T, d] float32 or bfloat16
 * (round to nearest even). topk_w may be any caller array (e.g. with a slot
 * zeroed to ablate an expert). Slots with asg_pos < 0 (ids moe_permute left
 * out) are skipped. */
int moe_combine(const float* y, const int32_t* asg_pos, const float* topk_w, int64_t T, int d,
                int k, void* out, int out_dtype, void* stream);

/* The whole layer: moe_route, moe_permute, moe_expert_ffn and moe_combine
 * in one call on one stream. topk_idx_out [T,k], topk_w_out [T,k] and
 * counts_out [E] are optional (NULL) copies of the routing; logit_bias may be
 * NULL. ws must hold moe_workspace_bytes(T, d, ffn, E, k, dtype) bytes.
 * options: NULL or per-call options (kernel family, stage events, down split). */
int moe_forward(const void* x, int dtype, const float* router, const float* logit_bias,
                const void* w1, const void* w3, const void* w2, int64_t T, int d, int ffn,
                int E, int k, void* out, int out_dtype, int32_t* topk_idx_out,
                float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                void* stream, const moe_options* options);

/* The MLP half of the decoder block around the layer (nnterp Mixtral page,
 * "The Notes", the block in order: out = h + mlp(post_attention_layernorm(h));
 * the norm is a MixtralRMSNorm over hidden_size with eps = rms_norm_eps,
 * 1e-5 in MixtralConfig):
 *   r_t         = 1 / sqrt(sum_i hidden[t,i]^2 / d + eps)          (float32)
 *   norm_out[t] = round((hidden[t,i] * r_t) * norm_weight[i])      (hidden's type)
 *   out[t]      = hidden[t] + moe_forward(norm_out)[t]              (float32, then out_dtype)
 * The router and the experts both read the stored norm_out, exactly as
 * moe_forward would read it as x (same kernels, same results bit for bit),
 * and the residual is added to the finished slot sum. hidden [T, d] and
 * norm_out [T, d] have the element type of dtype (float32 for MOE_F32,
 * bfloat16 for MOE_BF16 / MOE_BF16_PACKED); norm_weight [d] is float32;
 * eps must be finite and >= 0 (a zero row with eps = 0 gives NaN). norm_out
 * and out must not overlap hidden or each other (MOE_EINVAL). Every other
 * argument, alignment rule and the workspace are as for moe_forward. */
int moe_block_forward(const void* hidden, int dtype, const float* norm_weight, float eps,
                      void* norm_out, const float* router, const float* logit_bias,
                      const void* w1, const void* w3, const void* w2, int64_t T, int d, int ffn,
                      int E, int k, void* out, int out_dtype, int32_t* topk_idx_out,
                      float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                      void* stream, const moe_options* options);

/* moe_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The library calls no hipMalloc, hipFree
 * or allocating routine: the workspace is a scratch array built into the
 * library, MOE_NOALLOC_SCRATCH_BYTES bytes on each GPU it runs on, held from
 * its first use there until the process ends. Arguments, results and options
 * are those of moe_forward (the same kernels, bit-identical output); sizes
 * whose moe_workspace_bytes exceeds MOE_NOALLOC_SCRATCH_BYTES are refused with
 * MOE_EWORKSPACE before anything is enqueued (with bf16 or int8 weights at
 * k = 2 that admits batches of up to 545 tokens at the Mixtral-8x7B shape,
 * 409 at the 8x22B shape). Every call on a GPU
 * uses that GPU's one array and nothing in it needs to start at a particular
 * value, so calls that overlap on one GPU (concurrent streams, or threads
 * without ordering between their streams) race and give wrong results: order
 * them. The scratch of the current device is used; MOE_EHIP if its address
 * cannot be obtained. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_noalloc(const void* x, int dtype, const float* router, const float* logit_bias,
                        const void* w1, const void* w3, const void* w2, int64_t T, int d, int ffn,
                        int E, int k, void* out, int out_dtype, int32_t* topk_idx_out,
                        float* topk_w_out, int32_t* counts_out, void* stream,
                        const moe_options* options);

/* One-time weight preparation for the MOE_BF16_PACKED path: copies the
 * bfloat16 matrices w [E, rows, cols] (standard layout, cols contiguous) into
 * `out` (same size, E*rows*cols*2 bytes, must not overlap w) in fragment
 * order: 16-row x 32-column fragments, each 1 KiB in the lane order of a
 * 16x16x32 bf16 MFMA operand (value w[e][16*rt + r][32*s + 8*g + i] at
 * element ((e*rows/16 + rt)*cols/32 + s)*512 + (16*g + r)*8 + i). Pack w1 and
 * w3 with rows = ffn, cols = d, and w2 with rows = d, cols = ffn. Expert
 * weights do not change between calls, so this runs once when they are
 * loaded. dtype must be MOE_BF16; rows % 16 == 0 and cols % 32 == 0, and
 * both pointers 16-byte aligned, else MOE_ENOTSUP. */
int moe_pack_weight(const void* w, int dtype, int E, int rows, int cols, void* out,
                    void* stream);

/* Weight-only int8 quantization for the MOE_INT8_PACKED path (ZeroModels
 * Mixtral page, "Lower memory": weight-only int8 with bfloat16 activations).
 * For each output row n of w [E, rows, cols] (bfloat16, standard layout):
 *   scale[e][n] = max_k |w[e][n][k]| / 127                  (float32)
 *   q[e][n][k]  = round_half_even(w[e][n][k] / scale[e][n]) (int8, |q| <= 127;
 *                 0 for an all-zero row)
 * computed in float32 (the division correctly rounded). `out` receives
 * moe_quantized_weight_bytes(E, rows, cols) bytes: the codes in 16-row x
 * 64-column blocks of 1 KiB (block (e, row tile rt, column step s) at byte
 * ((e*rows/16 + rt)*cols/64 + s)*1024; in it, row r's columns 64s + 8g + i sit
 * at byte (16g + r)*16 + i and columns 64s + 32 + 8g + i at (16g + r)*16 + 8
 * + i, for g < 4, i < 8), then, from the next multiple of 256 bytes, the
 * float32 scales [E, rows]. Quantize w1 and w3 with rows = ffn, cols = d, and
 * w2 with rows = d, cols = ffn. The layer then computes with the weights
 * scale * q: each expert's products accumulate in float32 over bfloat16
 * activations and codes, and the row's scale multiplies the finished sum.
 * dtype must be MOE_BF16; rows % 16 == 0 and cols % 64 == 0 and 16-byte
 * aligned, non-overlapping buffers, else MOE_ENOTSUP / MOE_EINVAL. With int8
 * weights the streaming expert kernels read the codes directly when experts
 * get few rows (decode, where the weight bytes set the time); beyond that a
 * tiled MFMA kernel converts them to bfloat16 operands in registers (gate/up
 * when ffn % 128 == 0, down when d % 256 == 0); for large prefill batches
 * (T*k >= 8192*E for w1 and w3, >= 1024*E for w2) the codes are first widened
 * to bfloat16 (exact) in the workspace and the direct-to-LDS tile kernels of
 * the bf16 path run on them. Every kernel applies the row scales to its
 * finished sums. */
size_t moe_quantized_weight_bytes(int E, int rows, int cols);
int moe_quantize_weight(const void* w, int dtype, int E, int rows, int cols, void* out,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
