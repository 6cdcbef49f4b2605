/*
 * moe.h -- C ABI of the MoE expert feed-forward hot path on one AMD MI355X (gfx950).
 *
 * The path, as "Efficient MoE Training for Biological Foundation Models" describes
 * it (Challenge 1: Fragmented expert kernels; Challenge 3: Quantization overhead):
 * router top-k gating -> token permutation into per-expert groups (split_sizes) ->
 * grouped GEMM gate_up -> ScaledSwiGLU (routing probability folded in) -> grouped
 * GEMM down -> unpermute with combine; plus the matching backward and MXFP8 block
 * quantisation (one scale per 32 consecutive values, Challenge 2).
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers unless marked [host]. The caller owns all memory,
 *    including workspaces; the library keeps no pointer after a call returns.
 *  - Every call only enqueues work on `stream` (a hipStream_t passed as void*, NULL
 *    for the null stream) and returns: no host<->device synchronisation and no
 *    device allocation. Results are ready once the stream reaches them.
 *  - Tensors are row-major and densely packed. bf16 tensors are raw 16-bit patterns.
 *    Expert weights follow the [out_features, in_features] convention: gate_up is
 *    [2I, H] with the gate rows first ([0, I)) and the up rows after ([I, 2I));
 *    down is [H, I]. Each expert's weight is its own tensor, passed in a [host]
 *    array of E device pointers.
 *  - Arguments are checked before anything is launched. A bad argument returns
 *    MOE_ERR_INVALID_ARG, a shape the kernels do not implement MOE_ERR_UNSUPPORTED,
 *    a workspace that is too small MOE_ERR_WORKSPACE, and a failed launch
 *    MOE_ERR_LAUNCH; nothing is launched in the first three cases. moe_last_error()
 *    returns a description of the last failure on the calling thread. The library
 *    never aborts the process.
 *  - T = 0 and experts that receive no tokens are legal.
 *  - Results are deterministic: the same inputs give the same bits.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_LAUNCH = 4
} moe_status;

typedef enum {
  MOE_F32 = 0,   /* float32 */
  MOE_BF16 = 1,  /* bfloat16 bit patterns */
  MOE_MXFP8 = 2, /* E4M3 codes (uint8) + one E8M0 scale byte per 32 consecutive values */
  MOE_FP8 = 3    /* E4M3 codes (uint8) + one float32 scale for the whole tensor (value = code x scale) */
} moe_dtype;

/* Largest expert count the library accepts. */
#define MOE_MAX_EXPERTS 256

/*
 * Router top-k gating. Source: routing_weights of the Hugging Face per-expert loop
 * (Challenge 1). The pages show no router; the rule implemented is softmax over
 * the E logits, keep the k largest, and (renormalize != 0) rescale the kept
 * probabilities to sum to 1; with renormalize == 0 they are the full softmax's
 * entries. Selection compares the float32 logits: slot 0 holds the largest; on
 * equal logits the lower expert index comes first.
 *   logits    [T, E] float32
 *   topk_idx  [T, k] int32   (out) expert of each slot
 *   topk_prob [T, k] float32 (out) routing weight of each slot
 * Limits: 1 <= k <= E <= MOE_MAX_EXPERTS, k <= 16.
 */
moe_status moe_route_topk(const float* logits, int64_t T, int E, int k, int renormalize,
                          int32_t* topk_idx, float* topk_prob, void* stream);

/*
 * Router gate linear. Source: the router logits behind routing_weights of the
 * Hugging Face per-expert loop (Challenge 1). The pages show no router; the gate is
 * read as a bias-free linear map hidden -> E with an [E, H] weight (the [out, in]
 * layout of the pages' GroupedLinear weights):
 *   logits[t, e] = sum_h x[t, h] * w_router[e, h], bf16 products, float32 accumulation
 *   x        [T, H] bf16, 16-byte aligned
 *   w_router [E, H] bf16, 16-byte aligned
 *   logits   [T, E] float32 (out)
 * The four H quarters of each token are summed in a fixed order (deterministic).
 * Limits: 1 <= E <= MOE_MAX_EXPERTS, H % 64 == 0.
 */
moe_status moe_router_logits(const void* x, const void* w_router, int64_t T, int H, int E,
                             float* logits, void* stream);

/*
 * Backward of moe_route_topk (the selection is piecewise constant in the logits;
 * only the probabilities carry a gradient). With g = d_topk_prob and p = topk_prob:
 *   renormalize != 0: d_logits[t, idx[t, j]] = p[t, j] * (g[t, j] - sum_j' p[t, j'] g[t, j']),
 *                     every other expert 0; logits may be NULL;
 *   renormalize == 0: d_logits[t, e] = P[t, e] * (G[t, e] - sum_j p[t, j] g[t, j]) with P the
 *                     softmax of the logits row and G[t, e] = g[t, j] where e = idx[t, j], else 0.
 *   logits [T, E] float32 (renormalize == 0 only), topk_idx [T, k] int32,
 *   topk_prob, d_topk_prob [T, k] float32, d_logits [T, E] float32 (out, every entry written)
 * Limits: 1 <= k <= E <= MOE_MAX_EXPERTS, k <= 16.
 */
moe_status moe_route_topk_bwd(const float* logits, const int32_t* topk_idx, const float* topk_prob,
                              const float* d_topk_prob, int64_t T, int E, int k, int renormalize,
                              float* d_logits, void* stream);

/*
 * Backward of moe_router_logits:
 *   dx[t, h]        = dx_in[t, h] + sum_e d_logits[t, e] * w_router[e, h]   (bf16 out; dx_in
 *                     bf16 or NULL for 0, may equal dx: the expert path's input gradient
 *                     plus the router's)
 *   dw_router[e, h] = sum_t d_logits[t, e] * x[t, h]                        (float32 out)
 * float32 arithmetic; dw_router adds chunks of 64..1024 tokens (a function of T, H, E)
 * in order (deterministic).
 * workspace: moe_workspace_size(MOE_OP_ROUTER_BWD, desc with E and H, R ignored, T)
 * bytes (0 when one chunk covers T), 16-byte aligned, caller-owned. T == 0 writes
 * dw_router = 0.
 * Limits: 1 <= E <= MOE_MAX_EXPERTS, H % 8 == 0; x, w_router, dx, dx_in, dw_router
 * 16-byte aligned.
 */
moe_status moe_router_bwd(const void* x, const void* w_router, const float* d_logits, const void* dx_in,
                          int64_t T, int H, int E, void* dx, float* dw_router, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Token permutation into per-expert groups. Source: split_sizes of GroupedLinear
 * (Challenge 1) and the per-expert row gather of the baseline loop; token
 * permutation before the grouped GEMM is also named in the PyTorch-native MoE
 * library article (DeepEP dispatcher with permute/unpermute fusion).
 * The R = T*k (token, slot) pairs are grouped by expert in ascending expert
 * order; inside a group rows are in ascending token order. Row r of the result
 * holds x[src_token[r]].
 *   x            [T, H] in dtype dt (F32 or BF16; MXFP8: codes, with x_scale [T, H/32])
 *   topk_idx     [T, k] int32, topk_prob [T, k] float32 (may be NULL: prob_perm not written)
 *   x_perm       [R, H] (out), x_perm_scale [R, H/32] (out, MXFP8 only)
 *   prob_perm    [R] float32 (out, may be NULL) routing weight of each row
 *   split_sizes  [E] int32 (out) rows per expert; offsets [E+1] int32 (out) prefix sums
 *   row_id_map   [T*k] int32 (out) row of pair (t, j) at index t*k + j
 *   src_token    [R] int32 (out) token of each row
 * reuse_map != 0: the maps are INPUTS from an earlier call with the same routing;
 * only x is gathered into x_perm (used to gather the output gradient).
 * workspace: moe_workspace_size(MOE_OP_PERMUTE, ...) bytes, 256-byte aligned.
 * Input contract: each token's k expert ids are distinct and in [0, E), as
 * moe_route_topk produces them. A (token, slot) pair whose id is out of range, or
 * repeats the id of an earlier slot of the same token, is dropped: its row_id_map
 * entry is -1, split_sizes does not count it, and only the first offsets[E] rows of
 * x_perm, prob_perm and src_token are written (T*k - offsets[E] pairs were dropped).
 * moe_unpermute_combine skips -1 entries, so a dropped pair contributes nothing.
 */
moe_status moe_permute(const void* x, const uint8_t* x_scale, moe_dtype dt, int64_t T, int H,
                       int E, int k, const int32_t* topk_idx, const float* topk_prob,
                       int reuse_map, void* x_perm, uint8_t* x_perm_scale, float* prob_perm,
                       int32_t* split_sizes, int32_t* offsets, int32_t* row_id_map,
                       int32_t* src_token, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * moe_permute without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops or harnesses that forbid
 * hipMalloc). Same arguments (minus the workspace), semantics and outputs as
 * moe_permute. Its count/scan scratch is a static 8 MiB device array inside the
 * library: one per GPU, held until the process ends, its address looked up once per
 * device on the first call. Sizes whose scratch (moe_workspace_size(MOE_OP_PERMUTE,
 * ...)) exceeds 8 MiB return MOE_ERR_UNSUPPORTED before anything is launched (T*k up
 * to about two million pairs at E = 8). The call allocates nothing. Every call on one
 * GPU shares that GPU's array and no entry of it needs clearing (each call writes
 * what it reads); calls that overlap in time on one GPU (other streams or threads)
 * race on it and must be serialised by the caller.
 */
moe_status moe_permute_noalloc(const void* x, const uint8_t* x_scale, moe_dtype dt, int64_t T, int H,
                               int E, int k, const int32_t* topk_idx, const float* topk_prob,
                               int reuse_map, void* x_perm, uint8_t* x_perm_scale, float* prob_perm,
                               int32_t* split_sizes, int32_t* offsets, int32_t* row_id_map,
                               int32_t* src_token, void* stream);

/*
 * Unpermute with combine. Source: the index_add_ into final_hidden_states of the
 * baseline loop (Challenge 1).
 *   out[t] = sum over j = 0..k-1 (in that order, float32) of w[t, j] * y_perm[row_id_map[t*k + j]]
 * with w = weights [T, k] float32, or w = 1 when weights is NULL (the routing
 * probability already folded into ScaledSwiGLU). y_perm [T*k, H] and out [T, H]
 * are both dtype dt (F32 or BF16; bf16 output is rounded to nearest even).
 */
moe_status moe_unpermute_combine(const void* y_perm, moe_dtype dt, const int32_t* row_id_map,
                                 const float* weights, int64_t T, int H, int k, void* out,
                                 void* stream);

/*
 * MXFP8 block quantisation of a bf16 matrix along its rows. Source: Challenge 2
 * (one scaling factor per block of 32 consecutive values, 8-bit values) and
 * Challenge 3 (bf16 -> MXFP8 before the low-precision GEMM).
 * For each block of 32 consecutive elements of a row: s = the smallest integer
 * with max|block| <= 448 * 2^s, clamped to [-127, 127] (s = -127 for an all-zero
 * block); the scale byte is s + 127 (E8M0); each element becomes the OCP E4M3
 * code of x / 2^s, rounded to nearest with ties to even, keeping x's sign bit.
 *   in [rows, cols] bf16 (cols % 32 == 0), e4m3 [rows, cols] uint8 (out),
 *   e8m0 [rows, cols/32] uint8 (out).
 */
moe_status mxfp8_quantize(const void* in_bf16, int64_t rows, int64_t cols, uint8_t* e4m3,
                          uint8_t* e8m0, void* stream);

/*
 * Column-wise MXFP8 quantisation, expert by expert, along the token axis: the operand
 * layout of the weight-gradient GEMMs of an MXFP8 backward, whose reduction runs over
 * each expert's rows. Source: Challenge 2 (one scaling factor per 32 consecutive
 * values) with Challenge 3's matching backward taking its GEMM operands in MXFP8 along
 * each GEMM's own reduction axis (the pages show no layout; this is the reading).
 * Expert e owns rows [offsets[e], offsets[e+1]) of x; those rows, zero-padded to a
 * multiple of `pad`, become columns [kofs[e], kofs[e+1]) of the transposed output,
 * quantised in blocks of 32 along that axis by the rule of mxfp8_quantize (blocks that
 * are all padding get scale byte 0 and codes 0).
 *   x       [R, C] bf16 (16-byte aligned), offsets [E+1] int32 (device)
 *   e4m3_t  [C, kcap] uint8 (out, 16-byte aligned), e8m0_t [C, kcap/32] uint8 (out)
 *   kofs    [E+1] int32 (out, device): the padded column offsets; columns at and past
 *           kofs[E] are not written
 * Limits: C % 64 == 0, pad a positive multiple of 32, kcap a multiple of 32 with
 * kcap >= R + E * (pad - 1) (room for every expert's padding), 1 <= E <= MOE_MAX_EXPERTS.
 */
moe_status mxfp8_quantize_colwise(const void* x_bf16, int64_t R, int64_t C, int E, const int32_t* offsets, int pad,
                                  int64_t kcap, uint8_t* e4m3_t, uint8_t* e8m0_t, int32_t* kofs, void* stream);

/*
 * MXFP8 packing of one bf16 weight for moe_grouped_mlp_bwd (the MXFP8 backward's data
 * gradients take each weight quantised along the axis they reduce over: W2_e [H, I]
 * along H, W1_e [2I, H] along 2I). Source: Challenge 2 (32-value blocks) and Challenge 3
 * (quantisation as separate ops is the overhead the fused recipe removes: a training
 * loop packs each weight once per optimizer step instead of once per call).
 *   w [rows, cols] bf16 (16-byte aligned)
 *   packed (out, 16-byte aligned, rows * cols * 33 / 32 bytes): the E4M3 codes of the
 *     transpose, [cols][rows] (element (c, r) is w[r, c] quantised in blocks of 32
 *     along r by the rule of mxfp8_quantize), then at byte rows * cols the E8M0 scales,
 *     "step-major": the 4 scales of rows [128 k, 128 k + 128) of column c are one 32-bit
 *     word (lowest byte first) at word index k * cols + c.
 * Limits: rows % 128 == 0, cols % 64 == 0, rows * cols < 2^31.
 */
moe_status mxfp8_pack_weight_bwd(const void* w_bf16, int64_t rows, int64_t cols, void* packed, void* stream);

/*
 * Per-tensor FP8 quantisation of a bf16 tensor. Source: Challenge 2 (FP8 with one
 * scaling factor for a whole tensor, the contrast to MXFP8's factor per 32 values).
 * The pages give no scale rule; the one implemented ("current scaling"):
 *   amax = max |in| over the n elements; scale = amax / 448 (float32 division,
 *   rounded to nearest), or 1 when amax = 0;
 *   e4m3[i] = the OCP E4M3 code of the float32 quotient in[i] / scale (rounded to
 *   nearest even, saturating to +-448, sign kept).
 *   in [n] bf16 (16-byte aligned), e4m3 [n] uint8 (out, 8-byte aligned),
 *   scale: ONE float32 in device memory (out, 4-byte aligned; also used as the amax
 *   accumulator while the call's kernels run).
 * Limits: n % 8 == 0. n == 0 writes scale = 1.
 */
moe_status fp8_tensor_quantize(const void* in_bf16, int64_t n, uint8_t* e4m3, float* scale, void* stream);

/*
 * Per-tensor FP8 codes laid out along the token axis, expert by expert: the operand
 * layout of the weight-gradient GEMMs of the per-tensor FP8 backward. Source:
 * Challenge 2 (FP8: one scaling factor for a whole tensor). One factor for the whole
 * tensor means the codes are those of fp8_tensor_quantize on x, transposed: expert e's
 * rows [offsets[e], offsets[e+1]) of x, zero-padded to a multiple of `pad`, become
 * columns [kofs[e], kofs[e+1]) of the output (padding is code 0).
 *   x       [R, C] bf16 (16-byte aligned), offsets [E+1] int32 (device)
 *   e4m3_t  [C, kcap] uint8 (out, 16-byte aligned); columns at and past kofs[E] are
 *           not written
 *   scale   ONE float32 in device memory (out, 4-byte aligned): x's factor, by the rule
 *           of fp8_tensor_quantize (also the amax accumulator while the call runs)
 *   kofs    [E+1] int32 (out, device): the padded column offsets
 * Limits: C % 64 == 0, pad a positive multiple of 32, kcap a multiple of 32 with
 * kcap >= R + E * (pad - 1), 1 <= E <= MOE_MAX_EXPERTS, R < 2^31.
 */
moe_status fp8_tensor_quantize_colwise(const void* x_bf16, int64_t R, int64_t C, int E, const int32_t* offsets,
                                       int pad, int64_t kcap, uint8_t* e4m3_t, float* scale, int32_t* kofs,
                                       void* stream);

/*
 * Per-tensor FP8 packing of one bf16 weight for moe_grouped_mlp_bwd (the FP8 backward's
 * data gradients take each weight transposed, K-contiguous: W2_e [H, I] as [I, H], W1_e
 * [2I, H] as [H, 2I]). Source: Challenge 2 (FP8: one scaling factor for a whole tensor)
 * and Challenge 3 (quantisation as separate ops is the overhead the fused recipe
 * removes: a training loop packs each weight once per optimizer step).
 *   w [rows, cols] bf16 (16-byte aligned)
 *   packed (out, 16-byte aligned, rows * cols + 4 bytes): the E4M3 codes of the
 *     transpose, [cols][rows] (element (c, r) is the code of w[r, c] under the rule of
 *     fp8_tensor_quantize), then at byte rows * cols the tensor's float32 factor.
 * Limits: rows % 32 == 0, cols % 64 == 0, rows * cols < 2^31.
 */
moe_status fp8_tensor_pack_weight_bwd(const void* w_bf16, int64_t rows, int64_t cols, void* packed, void* stream);

/*
 * MXFP8 quantisation of n bf16 weights of one shape into both layouts a training step
 * takes, from one read of each weight. Source: Challenge 2 (32-value blocks) and
 * Challenge 3 (quantisation as separate ops is the overhead the fused recipe removes: a
 * step that updates its bf16 master weights needs the forward's and the backward's
 * operand once per step, and one pass over each weight makes both).
 * For weight i (w_bf16, e4m3, e8m0, packed: host arrays of n device pointers):
 *   w_bf16[i] [rows, cols] bf16 (16-byte aligned)
 *   e4m3[i] [rows, cols] uint8 (out, 8-byte aligned), e8m0[i] [rows, cols/32] uint8 (out):
 *     byte for byte the output of mxfp8_quantize on w_bf16[i] (the forward's operand,
 *     moe_grouped_mlp_fwd with wt = MXFP8)
 *   packed[i] (out, 16-byte aligned, rows * cols * 33 / 32 bytes): byte for byte the
 *     output of mxfp8_pack_weight_bwd on w_bf16[i] (the backward's operand)
 * Limits: 1 <= n <= MOE_MAX_EXPERTS and those of mxfp8_pack_weight_bwd (rows % 128 == 0,
 * cols % 64 == 0, rows * cols < 2^31). rows == 0 or cols == 0 is a no-op.
 */
moe_status mxfp8_quantize_weights(int n, const void* const* w_bf16, int64_t rows, int64_t cols, uint8_t* const* e4m3,
                                  uint8_t* const* e8m0, void* const* packed, void* stream);

/*
 * Per-tensor FP8 quantisation of n bf16 weights of one shape into both layouts a
 * training step takes: one pass for the maxima, one that writes both codes. Source:
 * Challenge 2 (FP8: one scaling factor for a whole tensor) and Challenge 3 (quantisation
 * as separate ops is the overhead the fused recipe removes).
 * For weight i (w_bf16, e4m3, packed: host arrays of n device pointers):
 *   w_bf16[i] [rows, cols] bf16 (16-byte aligned)
 *   e4m3[i] [rows, cols] uint8 (out, 8-byte aligned) and scale[i] (scale: a device array
 *     of n float32, out, 4-byte aligned): the codes and factor of fp8_tensor_quantize on
 *     w_bf16[i] (the forward's operand, moe_grouped_mlp_fwd with wt = FP8)
 *   packed[i] (out, 16-byte aligned, rows * cols + 4 bytes): byte for byte the output
 *     of fp8_tensor_pack_weight_bwd on w_bf16[i] (the backward's operand)
 * scale also holds the maxima while the call's kernels run. Limits: 1 <= n <=
 * MOE_MAX_EXPERTS, rows % 32 == 0, cols % 64 == 0, rows * cols < 2^31. rows == 0 or
 * cols == 0 writes only the factors (1, the factor of an empty tensor).
 */
moe_status fp8_tensor_quantize_weights(int n, const void* const* w_bf16, int64_t rows, int64_t cols,
                                       uint8_t* const* e4m3, float* scale, void* const* packed, void* stream);

/* Description of one grouped MLP layer (the experts' shapes and precisions). */
typedef struct {
  int E;             /* experts, 1..MOE_MAX_EXPERTS */
  int H;             /* hidden size (GEMM K of gate_up, N of down) */
  int I;             /* intermediate size (gate_up has 2I outputs) */
  moe_dtype compute; /* GEMM input precision: MOE_F32, MOE_BF16, MOE_MXFP8 or MOE_FP8 */
  moe_dtype act;     /* storage of x_perm: F32 (compute F32), BF16, or the compute dtype's
                        codes (MXFP8 / FP8: codes + x_perm_scale) */
  moe_dtype wt;      /* storage of weights: F32 (compute F32), BF16 (for MXFP8 / FP8 compute:
                        master weights quantised inside the call), or the compute dtype's
                        codes (codes + scale tables) */
  int save_for_bwd;  /* nonzero: write z_save and h_save for moe_grouped_mlp_bwd */
} moe_mlp_desc;

/*
 * Grouped MLP forward: GroupedLinear(gate_up) -> ScaledSwiGLU -> GroupedLinear(down)
 * over the permuted rows. Source: Challenge 3 (the Sequential of the three ops and
 * its fused forward: SwiGLU and probability scaling inside the grouped path, some
 * intermediates never materialised; with MXFP8, quantisation fused before the
 * down projection, Figure 4).
 * For expert e and its rows r in [offsets[e], offsets[e+1]):
 *   z = x_perm[r] W1_e^T  (2I values; float32 accumulation)
 *   h = silu(z[0:I]) * z[I:2I] * prob_perm[r]      (silu(g) = g / (1 + exp(-g)))
 *   y_perm[r] = h W2_e^T
 * With compute = MXFP8, x_perm (along H), W1_e (along H), h (along I) and W2_e
 * (along I) enter their GEMMs as MXFP8 (rule of mxfp8_quantize); h is quantised in
 * the gate_up epilogue from its float32 value. With compute = FP8, x_perm (one
 * tensor), each expert's W1_e and W2_e (one tensor each) and h (one tensor) enter their
 * GEMMs as per-tensor FP8 (rule of fp8_tensor_quantize); h is first stored in bf16,
 * since its scale needs the maximum over all of it, and quantised from those bf16
 * values; the GEMM products are scaled by the product of the two tensors' scales.
 * FP8 scale arguments are float32 scales in device memory reached through the same
 * parameters: x_perm_scale -> one float (act = FP8), w_gate_up_scale[e] / w_down_scale[e]
 * -> one float each (wt = FP8). Outputs: y_perm [R, H] (bf16, or
 * float32 when compute = F32). With save_for_bwd: z_save [R, 2I] and h_save [R, I]
 * (bf16, or float32 when compute = F32; with MXFP8, z is the gate_up product of the
 * MXFP8 operands and h its ScaledSwiGLU before quantisation, both rounded to bf16;
 * with FP8, z is the gate_up product of the FP8 operands times the two scales and h
 * the bf16 value that is then quantised); otherwise both may be NULL.
 *   w_gate_up [host] E pointers to [2I, H]; w_down [host] E pointers to [H, I]
 *   w_gate_up_scale / w_down_scale [host] E pointers to [2I, H/32] / [H, I/32]
 *       E8M0 scales, only when wt = MXFP8 (else NULL)
 *   offsets [E+1] int32 (device), prob_perm [R] float32
 * Shapes the GEMM kernels implement: BF16 needs H % 256 == 0 and I % 128 == 0;
 * MXFP8 and FP8 need H % 256 == 0, I % 256 == 0 and E <= 128; F32 needs H % 4 == 0.
 */
moe_status moe_grouped_mlp_fwd(const moe_mlp_desc* desc, int64_t R, const void* x_perm,
                               const uint8_t* x_perm_scale, const void* const* w_gate_up,
                               const void* const* w_down, const uint8_t* const* w_gate_up_scale,
                               const uint8_t* const* w_down_scale, const int32_t* offsets,
                               const float* prob_perm, void* y_perm, void* z_save, void* h_save,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped MLP backward (the "matching fused backward" of Challenge 3), compute
 * BF16, F32, MXFP8 or FP8. With dY = dy_perm (gradient of y_perm), G, U = the halves of z_save,
 * A = silu(G) * U, p = prob_perm, per expert e:
 *   dW2_e    = dY^T h_save                          -> dw_down[e]    [H, I]
 *   dH       = dY W2_e
 *   dprob[r] = sum_i dH[r, i] * A[r, i]             -> dprob_perm    [R] float32
 *   dA       = dH * p
 *   dG       = dA * U * sig(G) * (1 + G * (1 - sig(G))),  dU = dA * silu(G)
 *   dx_perm  = [dG, dU] W1_e                         -> dx_perm       [R, H]
 *   dW1_e    = [dG, dU]^T x_perm                     -> dw_gate_up[e] [2I, H]
 * Experts without rows get all-zero weight gradients. Weight gradients are bf16 (float32
 * with compute = F32) and are overwritten, not accumulated.
 * compute = MXFP8 (act BF16; wt BF16, or MXFP8 for weights packed by mxfp8_pack_weight_bwd:
 * w_gate_up[e] the packing of W1_e (rows 2I, cols H), w_down[e] that of W2_e (rows H,
 * cols I), bit-identical to quantising the bf16 weights in the call): each of the four
 * GEMMs takes both operands as MXFP8 along its own reduction axis (Challenge 2's
 * 32-value blocks, Challenge 3's recipe): dY and dZ = [dG, dU] by rows, W2_e along H,
 * W1_e along 2I, and dY, h_save, dZ, x_perm along each expert's rows (blocks starting
 * at the expert's first row, zero-padded). dH and dZ are rounded to bf16 before use, as
 * the recipe returns a low-precision GEMM's result to bf16. Needs H % 256 == 0,
 * I % 256 == 0, E <= 128. Its workspace (moe_workspace_size(MOE_OP_MLP_BWD, ...))
 * holds every quantised operand, the column-wise weight copies and dH in bf16 (dZ is
 * only stored quantised): about R (3.1 H + 7.3 I) + 3.1 E H I bytes (the last term only
 * for bf16 weights), plus (2H + 3I) bytes per padding row of the token-axis layouts
 * (2.5 GB at R = 8192, H = 4096, I = 14336, E = 8, bf16 weights). Calls sharing a
 * workspace must not overlap.
 * compute = FP8 (act BF16; wt BF16, or FP8 for weights packed by
 * fp8_tensor_pack_weight_bwd, laid out as for MXFP8 above): every GEMM operand is one
 * tensor quantised by the rule of fp8_tensor_quantize (Challenge 2's FP8: one factor per
 * tensor): dY, dZ, h_save and x_perm each over all R rows, W1_e and W2_e each per
 * expert; a product is scaled by its two tensors' factors. dH and dZ are rounded to
 * bf16 before use, as for MXFP8. Same shape limits; the workspace holds the same
 * operands with one code per element and no scales.
 */
moe_status moe_grouped_mlp_bwd(const moe_mlp_desc* desc, int64_t R, const void* dy_perm,
                               const void* x_perm, const void* z_save, const void* h_save,
                               const float* prob_perm, const void* const* w_gate_up,
                               const void* const* w_down, const int32_t* offsets,
                               void* dx_perm, void* const* dw_gate_up, void* const* dw_down,
                               float* dprob_perm, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * GroupedLinear: one grouped GEMM submission over all local experts. Source:
 * "Efficient MoE Training for Biological Foundation Models", Challenge 1 (GroupedLinear
 * applies each expert's linear map to that expert's rows in one call, with per-expert
 * token counts; bias=False).
 *   y[r] = x[r] W_e^T  for r in [offsets[e], offsets[e+1]), float32 accumulation
 *   x [R, K], W_e [N, K] ([host] array of E device pointers), y [R, N]; dt = F32 or BF16
 *   (bf16 output rounded to nearest even).
 * Shapes the kernels implement: BF16 needs N % 256 == 0 and K % 64 == 0.
 * workspace: NULL (workspace_bytes ignored), or at least
 *   moe_workspace_size(MOE_OP_GROUPED_GEMM, ...) bytes, 256-byte aligned, caller-owned,
 *   contents need no initialisation; with it, a last round of tiles that would leave
 *   most CUs idle is split along K into float32 partial tiles that a second kernel sums.
 *   The result is the same sum in another association order. Calls sharing a workspace
 *   must not overlap.
 */
moe_status moe_grouped_linear(int E, int64_t R, int K, int N, moe_dtype dt, const void* x,
                              const void* const* w, const int32_t* offsets, void* y, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * GroupedLinear(gate_up) fused with ScaledSwiGLU (the first kernel of the fused grouped
 * MLP, Challenge 3 and Figure 4). For the rows r of expert e:
 *   z = x[r] W_e^T (2I values),  h[r] = silu(z[0:I]) * z[I:2I] * prob[r]
 *   x [R, H], W_e [2I, H] ([host] array of E device pointers), prob [R] float32,
 *   h [R, I] (out), z_save [R, 2I] (out, may be NULL); dt = F32 or BF16.
 * With dt = MXFP8, x holds E4M3 codes with x_scale [R, H/32], W_e codes with
 * w_scale[e] [2I, H/32], and h is written as E4M3 codes with h_scale [R, I/32]
 * (quantised from the float32 value of h by the rule of mxfp8_quantize); z_save must
 * be NULL. Shapes: H % 256 == 0 and I % 128 == 0 (BF16, MXFP8).
 * workspace: as for moe_grouped_linear (used by BF16 only; NULL is always valid).
 */
moe_status moe_grouped_gate_up_swiglu(int E, int64_t R, int H, int I, moe_dtype dt, const void* x,
                                      const uint8_t* x_scale, const void* const* w,
                                      const uint8_t* const* w_scale, const int32_t* offsets,
                                      const float* prob, void* h, uint8_t* h_scale, void* z_save,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Operations for moe_workspace_size. */
typedef enum {
  MOE_OP_PERMUTE = 0,  /* T = token count, E, k used; desc may be NULL */
  MOE_OP_MLP_FWD = 1,  /* desc and R used */
  MOE_OP_MLP_BWD = 2,  /* desc and R used */
  MOE_OP_GROUPED_GEMM = 3, /* moe_grouped_linear / moe_grouped_gate_up_swiglu; no argument used */
  MOE_OP_ROUTER_BWD = 4    /* moe_router_bwd: desc (E, H) and T used */
} moe_op;

/* Workspace bytes an operation needs (0 is possible). bytes is a [host] pointer. */
moe_status moe_workspace_size(moe_op op, const moe_mlp_desc* desc, int64_t R, int64_t T, int E,
                              int k, size_t* bytes);

const char* moe_status_str(moe_status s);
/* Description of the last failure on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
