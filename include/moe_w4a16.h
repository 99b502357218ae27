/*
 * moe_w4a16.h - C ABI of the MI355X (gfx950) weight-only INT4 MoE layer.
 *
 * The layer is the one "The Throughput Lever: Quantifying the MoE GEMM and
 * Mapping the Road to B300" identifies as the throughput lever of its MoE
 * serving stack (section "Phase 3: The INT4 Marlin MoE Throughput Lever"):
 * an INT4, group-size-32 (section "Building the Benchmark"), weight-only
 * Mixture-of-Experts grouped GEMM run over a dense token batch of
 * M = streams x q_len tokens (section "What It Means for the Engine"), each
 * token routed to its top-k experts (section "The Result: Two Regimes").
 *
 * One layer call is two entry points on one stream:
 *   moe_route_align   top-k routing + per-expert grouping of the M*k
 *                     (token, slot) assignments, padded to the tile size;
 *   moe_w4a16_forward FC1 (gate/up) with SiLU(gate)*up, FC2, and the
 *                     routing-weighted sum of each token's k expert outputs.
 * Weights are converted once by moe_w4a16_repack from the canonical GPTQ-style
 * format into the device layout the kernels stream.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked "host". The caller allocates
 *     and frees every buffer; the library allocates nothing, keeps no pointer
 *     after returning and has no mutable global state.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work: no host synchronisation, no device-to-host
 *     copy, so a layer call can be captured in a HIP graph. Buffers must stay
 *     alive until the stream has executed the work.
 *   - Arguments are validated on the host before anything is launched; on an
 *     error nothing is launched and no output is touched. Launch failures
 *     return MOE_ERR_HIP. A device fault surfaces at the caller's next
 *     synchronisation. No C++ exception crosses this interface.
 *   - M = 0 is valid: the call returns MOE_OK and launches nothing.
 *   - bf16 and fp16 values travel as uint16_t bit patterns.
 *
 * Canonical weight format (input of moe_w4a16_repack, a reading of the
 * "GPTQ-format" INT4 weights of "Building the Benchmark"):
 *   qweight uint8 [E, N, K/2]: byte i of a row holds input channel 2i in its
 *           low nibble and 2i+1 in its high nibble; nibble u encodes q = u - 8.
 *   scales  fp16  [E, N, K/32]: W[e, n, c] = q[e, n, c] * scales[e, n, c/32].
 *   W13 (kind 0): N = 2*I, K = H; rows [0, I) gate, rows [I, 2I) up.
 *   W2  (kind 1): N = H,   K = I.
 *
 * Limits (MOE_ERR_UNSUPPORTED otherwise): 1 <= E <= 1024, 1 <= top_k <= min(E, 16),
 * H and I multiples of 128, block_m in {16, 32, 64, 128}, M*top_k*max(H, I) < 2^31,
 * and one expert's repacked W13 or W2 (moe_w4a16_packed_bytes with E = 1,
 * less its trailer) below 2^31 bytes (H*I below about 1.9e9; the repack and size
 * calls apply the same per-tensor limit, and -1 / MOE_ERR_UNSUPPORTED past it).
 *
 * MXFP4 expert weights (the moe_mxfp4_* entry points at the end): "From
 * 1,060 to 4,016 tok/s on one B300, and why it wasn't the kernels" serves a
 * MoE whose experts are MXFP4 (opening section; its MoE kernels are MXFP4,
 * section "Finding 2: the MoE autotuner only saw decode shapes"). The same
 * routing, grouping, layer structure and bf16 activations, with the weights
 * in the OCP Microscaling (MX) v1.0 MXFP4 format: FP4 e2m1 codes and one E8M0
 * scale per 32 input channels.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* null pointer, negative size, misaligned pointer */
    MOE_ERR_UNSUPPORTED = -2, /* a size outside the limits above */
    MOE_ERR_CAPACITY = -3,    /* cap smaller than moe_route_align_capacity() */
    MOE_ERR_WORKSPACE = -4,   /* workspace smaller than moe_w4a16_workspace_bytes() */
    MOE_ERR_HIP = -5,         /* a HIP launch failed */
    MOE_ERR_SCRATCH = -6      /* batch too large for moe_w4a16_layer_noalloc's static scratch */
};

/* Version of this interface (bumped on any signature or layout change). */
int32_t moe_w4a16_abi_version(void);

/* Static, human-readable text for a status code (host). */
const char* moe_w4a16_status_string(int status);

/*
 * moe_route_align_capacity (host): entries of sorted_token_ids a call with
 * these sizes may write, rounded up to a multiple of block_m:
 *   roundup(M*k + min(E, M*k)*(block_m - 1), block_m).
 * Every expert's list is padded to a multiple of block_m, so the padded total
 * never exceeds this. Returns -1 on invalid sizes.
 */
int64_t moe_route_align_capacity(int32_t M, int32_t E, int32_t top_k, int32_t block_m);

/*
 * moe_route_align: top-k routing and per-expert grouping of one token batch.
 *
 * Routing ("The Result: Two Regimes": each token activates its top-k
 * experts; softmax over the experts, keep the k largest, renormalise):
 *   logits        fp32 [M, E] row-major, finite.
 *   topk_ids      out int32 [M, top_k]: the k experts with the largest logits,
 *                 largest first; equal logits go to the lower expert index,
 *                 -0.0 equals +0.0.
 *   topk_weights  out fp32 [M, top_k]: exp(L_j - L_0) / sum_i exp(L_i - L_0)
 *                 over the kept logits (equal to softmax-then-renormalise).
 * Grouping (the grouped GEMM of "Phase 3: The INT4 Marlin MoE Throughput
 * Lever" runs each expert over the tokens routed to it). Assignment
 * f = t*top_k + j:
 *   expert_offsets     out int32 [E+1]: exclusive prefix sum of the per-expert
 *                      counts, each rounded up to a multiple of block_m.
 *   num_tokens_post_pad out int32 [1]: expert_offsets[E] (NPP).
 *   sorted_token_ids   out int32 [cap]: entries [off[e], off[e+1]) list the
 *                      assignments of expert e in ascending f, then the
 *                      sentinel M*top_k up to the end of the range. Entries at
 *                      positions >= NPP are unspecified.
 *   block_expert_ids   out int32 [cap/block_m]: expert of each block_m-row
 *                      block; entries >= NPP/block_m are unspecified.
 * cap must be >= moe_route_align_capacity(M, E, top_k, block_m) and a multiple
 * of block_m. The integer outputs are deterministic (identical on every call).
 */
int moe_route_align(const float* logits, int32_t M, int32_t E, int32_t top_k, int32_t block_m,
                    int32_t* topk_ids, float* topk_weights,
                    int32_t* sorted_token_ids, int32_t* block_expert_ids,
                    int32_t* expert_offsets, int32_t* num_tokens_post_pad,
                    int64_t cap, void* stream);

/*
 * moe_w4a16_packed_bytes (host): size of the repacked weights of E experts
 * of an [N, K] INT4 matrix with the given group size: E*N*K*9/16 (nibbles plus
 * fp16 scales) + E*N (one int8 exponent shift per weight row, derived from its
 * scales, used by the large-batch kernels). Returns -1 unless group == 32,
 * N % 32 == 0 and K % 128 == 0.
 */
int64_t moe_w4a16_packed_bytes(int32_t E, int32_t N, int32_t K, int32_t group);

/*
 * moe_w4a16_repack: canonical INT4 weights -> the device layout the forward
 * streams. This is the analogue of the one-time weight repack of "Building
 * the Benchmark" (there into the Marlin layout; here a gfx950 layout of
 * 16-row x 128-channel tiles, each 1 KiB of nibbles followed by its 128 B of
 * scales, ordered so one wave reads one tile with one 16-byte load per lane,
 * and for W13 with gate tile r followed by up tile r).
 *   qweight  uint8 [E, N, K/2], scales_f16 uint16 [E, N, K/32] (canonical).
 *   kind     0 = W13 (N = 2I, K = H), 1 = W2 (N = H, K = I).
 *   packed   out, moe_w4a16_packed_bytes(E, N, K, group) bytes, 16-byte aligned.
 * The map is a bijection: moe_w4a16_unpack inverts it exactly (the row
 * shifts after the tiles are derived data: sigma = clamp(floor(log2(max over
 * the row's groups of |scale|)) - 11, -15, 4), 0 for a row of zero scales).
 */
int moe_w4a16_repack(const uint8_t* qweight, const uint16_t* scales_f16,
                     int32_t E, int32_t N, int32_t K, int32_t group, int32_t kind,
                     void* packed, void* stream);

/* moe_w4a16_unpack: exact inverse of moe_w4a16_repack (used by tests). */
int moe_w4a16_unpack(const void* packed, int32_t E, int32_t N, int32_t K, int32_t group, int32_t kind,
                     uint8_t* qweight, uint16_t* scales_f16, void* stream);

/*
 * moe_w4a16_workspace_bytes (host): scratch the forward needs for M tokens:
 * an fp32 [M, H] accumulator, the bf16 [M*top_k, I] FC1 activations, and
 * the tile table of the tiled grouped GEMM (256 bytes + (2*M*top_k + 16) x
 * 8 bytes); from M*top_k >= 16*E on also fp16 copies of the A rows
 * (max(M*H, M*top_k*I) x 2 bytes) and their exponents (M*top_k x 4 bytes).
 * Each part is padded to 256 bytes. Returns -1 on invalid sizes.
 */
int64_t moe_w4a16_workspace_bytes(int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k);

/*
 * moe_w4a16_preferred_block_m (host): the block_m the forward runs best with
 * for this batch (a function of the expected tokens per expert, M*top_k/E).
 * It never returns 128: the kernels that take blocks take at most 64 rows,
 * so with block_m = 128 they run each block as its two 64-row halves (and
 * the tiled kernel as one tile). Measured on the 384-expert layer: as fast
 * as the preferred size from 16 assignments per expert (the tiled kernel),
 * 1.5-1.8x slower below (64-row blocks of mostly padding rows).
 */
int32_t moe_w4a16_preferred_block_m(int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k);

/*
 * moe_w4a16_forward: the expert MLPs and the weighted combine for one batch.
 * "The Throughput Lever: Quantifying the MoE GEMM and Mapping the Road to
 * B300", section "Phase 3: The INT4 Marlin MoE Throughput Lever": the MoE
 * layer's work is a grouped GEMM over the experts with INT4 weights fused into
 * it (there the fused Marlin MoE kernel), run over the dense token batch;
 * section "The Result: Two Regimes": each token's top-k expert outputs are
 * combined with its routing weights.
 * Equivalent to moe_w4a16_fc1 followed by moe_w4a16_fc2 on the same stream.
 *   x_bf16      bf16 [M, H] activations, 16-byte aligned.
 *   topk_weights, sorted_token_ids, block_expert_ids, expert_offsets,
 *   num_tokens_post_pad: the outputs of moe_route_align for the same M, E,
 *               top_k, block_m and cap (read on the device only).
 *   w13_packed  moe_w4a16_repack output of W13 (kind 0), w2_packed of W2 (kind 1).
 *   workspace   >= moe_w4a16_workspace_bytes(M, E, H, I, top_k) bytes,
 *               16-byte aligned; contents on entry do not matter.
 *   out_bf16    out bf16 [M, H]: out[t] = sum_j topk_weights[t, j] *
 *               FC2_e(SiLU(gate_e(x_t)) * up_e(x_t)), e = topk_ids[t, j],
 *               accumulated in fp32 and rounded once to bf16. The FC1
 *               activation is stored as bf16 between the two GEMMs.
 * Numerics by regime. While experts average fewer than 16 assignments
 * (M*top_k < 16*E) each group's partial product uses the exact weights
 * q*s (scale applied to the fp32 product). From 16 on ("The Result: Two
 * Regimes": the compute-heavy regime) the weights enter the matrix core as
 * fp16(q * s * 2^-sigma), one rounding of the exact product (relative error
 * <= 2^-11), and each activation row as an exact fp16 copy scaled by a power
 * of two; the shifts are undone exactly in fp32. Both stay within the
 * layer's error bound against a float64 reference.
 * Float results may differ in the last bits between calls (the k
 * contributions are added with fp32 atomics in arrival order).
 */
int moe_w4a16_forward(const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I,
                      int32_t top_k, int32_t block_m, const float* topk_weights,
                      const int32_t* sorted_token_ids, const int32_t* block_expert_ids,
                      const int32_t* expert_offsets, const int32_t* num_tokens_post_pad, int64_t cap,
                      const void* w13_packed, const void* w2_packed,
                      void* workspace, int64_t workspace_bytes, uint16_t* out_bf16, void* stream);

/*
 * moe_w4a16_fc1: first stage of moe_w4a16_forward. For every assignment f in
 * sorted_token_ids (expert e, token t = f / top_k) it computes
 * h = W13_e x_t, stores act_f = bf16(SiLU(h[0:I]) * h[I:2I]) in the
 * workspace, and clears the fp32 accumulator stage 2 uses.
 */
int moe_w4a16_fc1(const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I,
                  int32_t top_k, int32_t block_m,
                  const int32_t* sorted_token_ids, const int32_t* block_expert_ids,
                  const int32_t* num_tokens_post_pad, int64_t cap,
                  const void* w13_packed, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * moe_w4a16_fc2: second stage. y_f = W2_e act_f; acc[t] += topk_weights[f] * y_f
 * in fp32 (atomics), then out_bf16 = bf16(acc) in one rounding. Must follow
 * moe_w4a16_fc1 with the same workspace on the same stream.
 */
int moe_w4a16_fc2(int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, int32_t block_m,
                  const float* topk_weights, const int32_t* sorted_token_ids,
                  const int32_t* block_expert_ids, const int32_t* num_tokens_post_pad, int64_t cap,
                  const void* w2_packed, void* workspace, int64_t workspace_bytes,
                  uint16_t* out_bf16, void* stream);

/*
 * moe_w4a16_layer: one whole layer call, moe_route_align followed by
 * moe_w4a16_forward, with the same arguments, outputs and results (integer
 * outputs identical, out_bf16 within the same tolerance).
 *
 * "The Throughput Lever: Quantifying the MoE GEMM and Mapping the Road to
 * B300", section "The B300 Analysis: When the Bottleneck Flips": at decode
 * sizes fixed per-step costs such as kernel launches dominate once the GEMM
 * runs at HBM speed. Small batches therefore run two kernels instead of
 * four, with the routing and grouping inside the FC1 kernel (one of its
 * workgroups also writes the routing/grouping outputs):
 *   - M = 1: the decode path; every FC1 workgroup routes the
 *     batch, and FC2 is output-stationary (each output tile sums its token's
 *     top_k expert results in slot order in one workgroup: no atomics, and
 *     the bf16 output is then identical on every call);
 *   - M <= 16 and M*top_k <= 256 while few experts are touched and the
 *     batch's x rows fit in 128 KB of LDS (the grouped FC1 would fill at
 *     most 1.75 rounds of the device's CUs; on the 384-expert top-8 layer
 *     M = 2..7), and M = 2 or 3 wherever M*top_k <= 64: a persistent FC1
 *     kernel that routes once per workgroup and splits the work into small
 *     items (not when the tiled grouped GEMM below takes the batch);
 *   - else M = 4 with M*top_k <= 64: the decode path.
 * Up to 16 tokens the output-stationary FC2 follows the FC1 while the
 * M*top_k expert reads stay within 1.2x the expected number of distinct
 * experts (no accumulator and no finalize kernel); otherwise the grouped FC2
 * of moe_w4a16_forward.
 *   stage_events  NULL, or two hipEvent_t that receive the start and end
 *                 timestamps of the FC1-stage kernel itself (on the two-kernel
 *                 paths the routing is part of it), for timing that stage.
 */
int moe_w4a16_layer(const float* logits, const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I,
                    int32_t top_k, int32_t block_m, int32_t* topk_ids, float* topk_weights,
                    int32_t* sorted_token_ids, int32_t* block_expert_ids, int32_t* expert_offsets,
                    int32_t* num_tokens_post_pad, int64_t cap, const void* w13_packed, const void* w2_packed,
                    void* workspace, int64_t workspace_bytes, uint16_t* out_bf16, void* stream,
                    void* const* stage_events);

/*
 * moe_w4a16_layer_noalloc: moe_w4a16_layer without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). The workspace is a
 * static device array of MOE_W4A16_NOALLOC_SCRATCH_BYTES inside the library:
 * each GPU the library runs on holds its own copy from the first call on that
 * device until the process ends (the call resolves its address with
 * hipGetSymbolAddress on the current device; `stream` must belong to that
 * device). Arguments, outputs and results are those of moe_w4a16_layer (no
 * stage events). A batch whose moe_w4a16_workspace_bytes exceeds the scratch
 * size returns MOE_ERR_SCRATCH and launches nothing (48 MiB covers, e.g., up
 * to 512 tokens of the 384-expert layer: E = 384, H = 7168, I = 2048, top-8).
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine). Every call on a GPU shares that GPU's scratch, which keeps the
 * last call's contents (the kernels clear what must start at zero): calls
 * that overlap on one GPU (several streams, several threads) race and must
 * be serialised by the caller.
 */
#define MOE_W4A16_NOALLOC_SCRATCH_BYTES (48ll << 20)
int moe_w4a16_layer_noalloc(const float* logits, const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H,
                            int32_t I, int32_t top_k, int32_t block_m, int32_t* topk_ids, float* topk_weights,
                            int32_t* sorted_token_ids, int32_t* block_expert_ids, int32_t* expert_offsets,
                            int32_t* num_tokens_post_pad, int64_t cap, const void* w13_packed,
                            const void* w2_packed, uint16_t* out_bf16, void* stream);

/*
 * ---- MXFP4 weights --------------------------------------------------------
 * Canonical MXFP4 weight format (input of moe_mxfp4_repack):
 *   qweight     uint8 [E, N, K/2]: byte i of a row holds input channel 2i in
 *               its low nibble and 2i+1 in its high nibble; a nibble is an
 *               FP4 e2m1 code (bit 3 sign, bits 2..1 exponent with bias 1,
 *               bit 0 mantissa: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).
 *   scales_e8m0 uint8 [E, N, K/32]: s encodes 2^(s - 127) (255 = NaN).
 *   W[e, n, c] = fp4(qweight code) * 2^(scales_e8m0[e, n, c/32] - 127).
 *   W13 / W2 rows and shapes as for the INT4 format. Limits as above.
 * The device layout is the INT4 one with the codes in canonical byte order
 * and one scale byte per group: 0.53125 bytes per weight (INT4: 0.5625).
 * The kernels widen each code to the exact bf16 value code * 2^(s - 127)
 * (gfx950's FP4 conversion), so scales whose weights leave bf16's range
 * (s >= 253, or subnormal products) are outside the exact-result contract.
 */

/* Bytes of one repacked MXFP4 weight tensor (host); -1 for unsupported shapes. */
int64_t moe_mxfp4_packed_bytes(int32_t E, int32_t N, int32_t K);

/* moe_mxfp4_repack / moe_mxfp4_unpack: as moe_w4a16_repack / _unpack for the
 * MXFP4 format (kind 0 = W13, 1 = W2; 16-byte aligned buffers). */
int moe_mxfp4_repack(const uint8_t* qweight, const uint8_t* scales_e8m0, int32_t E, int32_t N, int32_t K,
                     int32_t kind, void* packed, void* stream);
int moe_mxfp4_unpack(const void* packed, int32_t E, int32_t N, int32_t K, int32_t kind, uint8_t* qweight,
                     uint8_t* scales_e8m0, void* stream);

/* moe_mxfp4_fc1, _fc2, _forward, _layer: the moe_w4a16_* entry points of the
 * same names (same arguments, workspace, routing buffers and semantics) with
 * moe_mxfp4_repack weights. */
int moe_mxfp4_fc1(const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k,
                  int32_t block_m, const int32_t* sorted_token_ids, const int32_t* block_expert_ids,
                  const int32_t* num_tokens_post_pad, int64_t cap, const void* w13_packed, void* workspace,
                  int64_t workspace_bytes, void* stream);
int moe_mxfp4_fc2(int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, int32_t block_m,
                  const float* topk_weights, const int32_t* sorted_token_ids, const int32_t* block_expert_ids,
                  const int32_t* num_tokens_post_pad, int64_t cap, const void* w2_packed, void* workspace,
                  int64_t workspace_bytes, uint16_t* out_bf16, void* stream);
int moe_mxfp4_forward(const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k,
                      int32_t block_m, const float* topk_weights, const int32_t* sorted_token_ids,
                      const int32_t* block_expert_ids, const int32_t* expert_offsets,
                      const int32_t* num_tokens_post_pad, int64_t cap, const void* w13_packed,
                      const void* w2_packed, void* workspace, int64_t workspace_bytes, uint16_t* out_bf16,
                      void* stream);
int moe_mxfp4_layer(const float* logits, const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I,
                    int32_t top_k, int32_t block_m, int32_t* topk_ids, float* topk_weights,
                    int32_t* sorted_token_ids, int32_t* block_expert_ids, int32_t* expert_offsets,
                    int32_t* num_tokens_post_pad, int64_t cap, const void* w13_packed, const void* w2_packed,
                    void* workspace, int64_t workspace_bytes, uint16_t* out_bf16, void* stream,
                    void* const* stage_events);

/* Measurement helpers (not part of the layer). They measure what this GPU
 * sustains, so that a layer kernel's rate can be stated as a fraction of the
 * attainable rate as well as of the published peaks ("The Throughput Lever",
 * section "The Result: Two Regimes", measures the layer as a fraction of the
 * memory bandwidth).
 *
 * moe_calib_read_granule (host): the byte multiple moe_calib_hbm_read reads
 *   (32768).
 * moe_calib_hbm_read: reads `bytes` of `buf` once (non-temporal 16-byte loads,
 *   `workgroups` workgroups of 256 threads; each thread writes the XOR of the
 *   32-bit words it read to sink[workgroup * 256 + thread], so the XOR of the
 *   whole sink is the XOR of every word of the buffer). bytes > 0, a multiple
 *   of the granule; buf 16-byte and sink 4-byte aligned; sink holds
 *   workgroups * 256 words; 1 <= workgroups <= 2^20. MOE_ERR_INVALID_ARG
 *   otherwise (nothing launched).
 * moe_calib_mfma_f16: `workgroups` workgroups of 4 waves each issue
 *   iters * 8 v_mfma_f32_16x16x32_f16 on register operands (16384 flops
 *   each; operand values are a fixed hash of lane, element and operand
 *   index). Each thread writes the sum of its accumulators to
 *   sink[workgroup * 256 + thread] (workgroups * 256 floats). iters >= 0;
 *   1 <= workgroups <= 2^20; sink 4-byte aligned. */
int64_t moe_calib_read_granule(void);
int moe_calib_hbm_read(const void* buf, int64_t bytes, int32_t workgroups, uint32_t* sink, void* stream);
int moe_calib_mfma_f16(int64_t iters, int32_t workgroups, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
