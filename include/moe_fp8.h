/*
 * moe_fp8.h -- C ABI of the routed FP8 Mixture-of-Experts expert step for AMD MI355X
 * (gfx950), one GPU, every expert local.
 *
 * The step (MindIE-SD "Fused MoE" page, section "执行流程" / execution flow:
 * select_experts -> dispatch -> mlp -> combine; metrale "fp8_grouped_tc_w8a8.rs",
 * module doc and run_fp8_grouped_w8a8: quantise the layer input, gate+up with quantised
 * SiLU products, down):
 *
 *   route            softmax / sigmoid top-k with optional group-limited selection and
 *                    routed_scaling_factor; optional RMSNorm + router gate prelude
 *                    (mlx-native "moe_gate.rs", module doc);
 *   dispatch         stable counting sort of the assignments by expert;
 *   quant_act        E4M3 per (row, 128 columns), UE8M0 power-of-two scales;
 *   grouped FFN      gate+up FP8 GEMM, SwiGLU, E4M3 re-quantisation, down FP8 GEMM;
 *   combine          weighted sum of each token's k expert outputs into bf16.
 *
 * Conventions for every entry point
 *   - All data pointers are DEVICE pointers owned by the caller, except the parameter
 *     structs themselves, which are host memory read during the call only.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.  Work is
 *     enqueued asynchronously; nothing synchronises with the host.  A device fault shows
 *     at the caller's next synchronisation.
 *   - All arguments are validated on the host before anything is launched; on an error
 *     nothing is launched (the guard of run_fp8_grouped_w8a8: launch nothing unless the
 *     shapes and buffers fit).  moe_last_error() then describes the failure.
 *   - Dtypes: bf16 values travel as uint16_t bit patterns; E4M3FN and UE8M0 as uint8_t;
 *     router logits, routing weights and the gate prelude tensors are float32; expert
 *     ids and permutation indices are int32.  Row-major throughout.
 *   - Reentrant; the library keeps no device memory of its own and allocates nothing:
 *     temporaries live in the caller's workspace (moe_workspace_size).
 *   - Size limits of the expert step (MOE_ERR_UNSUPPORTED beyond them): H and I multiples of
 *     128 and at most 32768; T * top_k < 2^29; T * H < 2^31 and 2 * I * H < 2^31 (the kernels
 *     address activation rows and one expert's weights with 32-bit offsets).
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------------------ */
#define MOE_OK               0
#define MOE_ERR_INVALID      1  /* a null pointer, a non-positive size, an inconsistent shape */
#define MOE_ERR_UNSUPPORTED  2  /* a valid shape the library does not handle (e.g. H % 128) */
#define MOE_ERR_WORKSPACE    3  /* workspace_bytes below what the call needs                */
#define MOE_ERR_HIP          4  /* a HIP runtime error while enqueuing                      */

/* ---- limits -------------------------------------------------------------------------- */
#define MOE_MAX_EXPERTS      1024
#define MOE_MAX_GROUPS       64

/* ---- routing ------------------------------------------------------------------------- */
#define MOE_SCORING_SOFTMAX  0
#define MOE_SCORING_SIGMOID  1

/* Routing parameters: the routing arguments of the "Fused MoE" parameter table
 * (num_experts, top_k, routing_method, renormalize, group_count, k_group,
 * group_select_mode, routed_scaling_factor) and section "路由选择" (routing).
 *   scoring            MOE_SCORING_SOFTMAX or MOE_SCORING_SIGMOID.
 *   renormalize        softmax only: divide the k selected weights by their sum.  Sigmoid
 *                      weights are always normalised over the k selected.
 *   group_count        G >= 1 contiguous expert groups (1 = ungrouped); E % G == 0.
 *   k_group            groups kept per token, 1 <= k_group <= G.
 *   group_select_mode  0: a group scores its largest score; 1: the sum of its two largest
 *                      scores (needs E/G >= 2).
 *   routed_scaling_factor  multiplies every selected weight, last.
 * The k selected experts of a token are listed by descending score; equal scores go to
 * the lower expert id, equal group scores to the lower group id.  Selection compares the
 * float32 logits themselves (softmax and sigmoid preserve their order), so it is exact;
 * only group_select_mode 1 and the gate prelude select on computed float32 values. */
typedef struct moe_route_params {
    int32_t num_experts;
    int32_t top_k;
    int32_t scoring;
    int32_t renormalize;
    int32_t group_count;
    int32_t k_group;
    int32_t group_select_mode;
    float   routed_scaling_factor;
} moe_route_params;

/* Gate prelude of the decode shape ("moe_gate.rs", moe_gate doc): per token
 * r = 1/sqrt(mean(x^2) + rms_eps), logits = (x * r * norm_weight) @ router_weight^T in
 * float32; top-k by logit; weights = softmax over the k selected logits, times
 * per_expert_scale[id] (NULL = 1), times routed_scaling_factor.  The hidden state given
 * to the experts is the un-normalised one. */
typedef struct moe_gate_prelude {
    const float* norm_weight;       /* [H]                                   */
    const float* router_weight;     /* [E, H]                                */
    const float* per_expert_scale;  /* [E] or NULL                           */
    float        rms_eps;
} moe_gate_prelude;

/* moe_route flags */
#define MOE_ROUTE_IDS_GIVEN  1  /* topk_ids / topk_weights are inputs: skip selection and
                                   only build the permutation (stands in for the page's
                                   custom_routing_function, which returns weights and ids) */

/* moe_route: selection (unless MOE_ROUTE_IDS_GIVEN) and the static dispatch ("Dispatcher
 * 策略": sort tokens by expert, count tokens per expert).
 *   T                 tokens, >= 1.  A = T * top_k assignments, flat index f = t*k + j.
 *   router_logits     [T, E] float32; NULL when `prelude` is given.
 *   hidden_states     [T, H] bf16; read only by the prelude (may be NULL otherwise).
 *   H                 hidden size, used only by the prelude (ignored otherwise).
 *   topk_ids          [T, k] int32 out (in with MOE_ROUTE_IDS_GIVEN; ids in [0, E)).
 *   topk_weights      [T, k] float32 out (in with MOE_ROUTE_IDS_GIVEN).
 *   expert_counts     [E] int32 out: assignments per expert.
 *   expert_offsets    [E+1] int32 out: exclusive prefix sum of expert_counts.
 *   sorted_assign     [A] int32 out: the flat index f at each expert-sorted slot; within
 *                     an expert the slots keep increasing f (a stable sort).
 *   assign_pos        [A] int32 out: the slot of each flat index (inverse permutation).
 *   workspace         >= moe_route_workspace_size(T, E, top_k, H, prelude != NULL) bytes,
 *                     256-byte aligned.
 * Returns MOE_OK or an error code.  All outputs are bit-exact functions of the inputs. */
int moe_route(const moe_route_params* p, int32_t T,
              const float* router_logits, const uint16_t* hidden_states, int32_t H,
              const moe_gate_prelude* prelude, int32_t flags,
              int32_t* topk_ids, float* topk_weights,
              int32_t* expert_counts, int32_t* expert_offsets,
              int32_t* sorted_assign, int32_t* assign_pos,
              void* workspace, size_t workspace_bytes, void* stream);

size_t moe_route_workspace_size(int32_t T, int32_t E, int32_t top_k, int32_t H, int32_t with_prelude);

/* moe_quant_act: per (row, 128-column group) E4M3 quantisation ("fp8_grouped_tc_w8a8.rs"
 * module doc: the layer input is quantised to E4M3 per (row, 128 group)).
 *   amax = max |x| over the group; e = the smallest integer with amax <= 448 * 2^e,
 *   clamped to [-127, 127] (e = 0 for an all-zero group); xq = E4M3FN(x / 2^e), rounded
 *   to nearest even, sign of zero kept; xs = e + 127 (UE8M0).
 *   x    [rows, ld] bf16, the first `cols` columns used; ld % 8 == 0, x 16-byte aligned.
 *   xq   [rows, cols] E4M3 out; xs [rows, cols/128] UE8M0 out.  cols % 128 == 0.
 * Bit-exact. */
int moe_quant_act(const uint16_t* x, int32_t rows, int32_t cols, int64_t ld,
                  uint8_t* xq, uint8_t* xs, void* stream);

/* ---- weights ------------------------------------------------------------------------- */
/* Expert weights are E4M3 with one UE8M0 scale per 128 x 128 block of (K, N):
 *   w13 logical [E, H, 2I]: K = H, N = 2I; gate projection in columns [0, I), up in
 *                [I, 2I) ("Fused MoE" parameter table: w13_weight is the fused gate/up
 *                projection [experts, hidden, 2*intermediate]);
 *   w2  logical [E, I, H]: K = I, N = H;
 *   w13_scale [E, H/128, 2I/128], w2_scale [E, I/128, H/128] uint8.
 * The GEMMs read the weights in a packed layout made once by moe_prepack_weights (the
 * one-time weight transform of the MATE Mega MoE "Typical Flow", step 2): per expert,
 * blocks of 16 columns x 128 rows of K, each block 2048 contiguous bytes in the order
 * the matrix cores consume them.  Scales keep the logical layout. */

/* moe_quant_weight_blocks: float32 [E, K, N] -> E4M3 [E, K, N] + UE8M0 [E, K/128, N/128]
 * with the same scale rule as moe_quant_act applied per 128 x 128 block.  K % 128 == 0,
 * N % 128 == 0.  Bit-exact.  An offline helper, not part of the timed step. */
int moe_quant_weight_blocks(const float* w, int32_t E, int32_t K, int32_t N,
                            uint8_t* q, uint8_t* scale, void* stream);

/* moe_prepack_weights: logical E4M3 [E, K, N] -> packed (same byte count, E*K*N).
 * Packed byte (e, n16, kb, h, lane, b) at ((e*(N/16) + n16)*(K/128) + kb)*2048
 * + h*1024 + lane*16 + b holds W[e][kb*128 + (lane/16)*32 + h*16 + b][n16*16 + lane%16].
 * K % 128 == 0, N % 16 == 0.  `packed` must not alias `w`. */
int moe_prepack_weights(const uint8_t* w, int32_t E, int32_t K, int32_t N,
                        uint8_t* packed, void* stream);

/* ---- micro-scaled schemes (one UE8M0 scale per 32 elements) ------------------------ */
/* Quantisation schemes of the grouped FFN (moe_ffn_args.quant, moe_fused_args.quant):
 *   MOE_QUANT_FP8_BLOCK128  E4M3 activations per (row, 128 columns), E4M3 weights per
 *                           128 x 128 block (the scheme above; the default, value 0).
 *   MOE_QUANT_MXFP8         E4M3 activations per (row, 32 columns), E4M3 weights per (32 rows
 *                           of K, one column) ("Fused MoE" page, section "MXFP8 dynamic quant
 *                           MoE": E4M3 weights whose MX scales run along K; the MATE Mega MoE
 *                           recipe (1, 1, 32)).
 *   MOE_QUANT_W4A8          the MXFP8 activations with E2M1 (FP4) weights per (32 x 1) (the
 *                           FP8 x FP4 path of the DeepGEMM Mega MoE pull request, whose W8A8
 *                           variant keeps its UE8M0 scale handling and switches the weights
 *                           from e2m1 to e4m3).
 * Every 32-element group uses the rule of moe_quant_act with the format's largest magnitude
 * M (448 for E4M3, 6 for E2M1): e = the smallest integer with amax <= M * 2^e, clamped to
 * [-127, 127], e = 0 for an all-zero group; codes = RNE(v / 2^e), ties to the even code, sign
 * of zero kept.  The SwiGLU output is re-quantised to E4M3 per (row, 32 columns) in both MX
 * schemes.  E2M1 is the OCP 4-bit float: sign, 2 exponent bits (bias 1), 1 mantissa bit,
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 *   MOE_QUANT_W8A16         weight-only: the E4M3 weights and 128 x 128 scales of
 *                           MOE_QUANT_FP8_BLOCK128 (same packing), bf16 activations (the
 *                           metrale grouped FP8 MoE page, module notes: the experts decode
 *                           W8A16 unless FP8 activations are published; the W8A8 step differs
 *                           only by the activation rounding).  gu = x @ dequant(w13) with x
 *                           the bf16 hidden state as is; h = silu(g) * u rounded once to bf16
 *                           (RNE); expert_out = h @ dequant(w2).  Float32 accumulation. */
#define MOE_QUANT_FP8_BLOCK128  0
#define MOE_QUANT_MXFP8         1
#define MOE_QUANT_W4A8          2
#define MOE_QUANT_W8A16         3
#define MOE_WFMT_E4M3           0
#define MOE_WFMT_E2M1           1

/* moe_quant_act_mx: E4M3 per (row, 32-column group), the MX activation quantisation.
 *   x [rows, ld] bf16 (first `cols` used; ld % 8 == 0, 16-byte aligned); xq [rows, cols]
 *   E4M3 out; xs [rows, cols/32] UE8M0 out.  cols % 32 == 0.  Bit-exact. */
int moe_quant_act_mx(const uint16_t* x, int32_t rows, int32_t cols, int64_t ld,
                     uint8_t* xq, uint8_t* xs, void* stream);

/* moe_quant_weight_mx: float32 [E, K, N] -> codes + UE8M0 scale [E, K/32, N], one scale per
 * (32 consecutive rows of K, one column).  wfmt MOE_WFMT_E4M3: codes [E, K, N], one byte
 * each; MOE_WFMT_E2M1: codes [E, K, N/2], column 2c in the low nibble of byte c.
 * K % 32 == 0, N % 2 == 0.  Bit-exact.  An offline helper, not part of the timed step. */
int moe_quant_weight_mx(const float* w, int32_t E, int32_t K, int32_t N, int32_t wfmt,
                        uint8_t* q, uint8_t* scale, void* stream);

/* moe_prepack_weights_mx: logical MX weights (as moe_quant_weight_mx writes them) -> the
 * packed layout the MX GEMMs read (the matrix-core instruction's K order, so that one
 * per-lane scale covers one 32-row group).
 *   E4M3: E*K*N bytes; byte ((e*(N/16) + n16)*(K/128) + kb)*2048 + h*1024 + lane*16 + b
 *         holds row kb*128 + h*64 + (lane/16)*16 + b of column n16*16 + lane%16.
 *   E2M1: E*K*N/2 bytes; byte ((e*(N/16) + n16)*(K/128) + kb)*1024 + lane*16 + b holds rows
 *         kb*128 + (lane/16)*32 + 2b (low nibble) and 2b + 1 (high nibble) of column
 *         n16*16 + lane%16.
 *   scales: E*K*N/32 bytes; byte ((e*(N/16) + n16)*(K/128) + kb)*64 + lane is the scale of
 *         rows kb*128 + (lane/16)*32 .. +31 of column n16*16 + lane%16.
 * K % 128 == 0, N % 16 == 0.  Outputs must not alias the inputs. */
int moe_prepack_weights_mx(const uint8_t* q, const uint8_t* scale, int32_t E, int32_t K, int32_t N,
                           int32_t wfmt, uint8_t* packed, uint8_t* packed_scale, void* stream);

/* ---- grouped expert FFN ------------------------------------------------------------ */
#define MOE_DTYPE_F32   0
#define MOE_DTYPE_BF16  1

/* moe_grouped_ffn: both expert GEMMs of every assignment, grouped by expert (the `mlp`
 * stage; run_fp8_grouped_w8a8's gate+up and down launches).  For each sorted slot s of
 * expert e holding assignment f (token t = f / k):
 *   gu = dequant(xq[t]) @ dequant(w13[e])                      (FP8 x FP8, fp32 accumulate)
 *   h  = silu(gu[:I]) * gu[I:]                                 (float32)
 *   hq, hs = quant per 128 columns of h                        (as moe_quant_act)
 *   expert_out[s] = dequant(hq, hs) @ dequant(w2[e])           (fp32, or bf16 RNE)
 * Arguments in moe_ffn_args:
 *   T, k, H, I, E     shapes; H % 128 == 0, I % 128 == 0.
 *   xq, xs            from moe_quant_act of the hidden states, [T, H] and [T, H/128].
 *   expert_counts, expert_offsets, sorted_assign   from moe_route.
 *   w13, w2           PACKED weights; w13_scale, w2_scale logical scales.
 *   expert_out        [T*k, H] in sorted-slot order, dtype out_dtype.
 *   workspace         >= moe_ffn_workspace_size(T, H, I, E, k) bytes, 256-byte aligned.
 * Accuracy: expert_out carries the float32 GEMMs' rounding and the rare E4M3 tie flips of
 * hq; compare with a tolerance, not bit for bit. */
typedef struct moe_ffn_args {
    int32_t T, k, H, I, E;
    const uint8_t* xq;
    const uint8_t* xs;
    const int32_t* expert_counts;
    const int32_t* expert_offsets;
    const int32_t* sorted_assign;
    const uint8_t* w13;
    const uint8_t* w13_scale;
    const uint8_t* w2;
    const uint8_t* w2_scale;
    void*          expert_out;
    int32_t        out_dtype;
    void*          workspace;
    size_t         workspace_bytes;
    void*          stream;
    int32_t        quant;       /* MOE_QUANT_*; the MX schemes take xs [T, H/32] from
                                   moe_quant_act_mx and the packed MX weights and scales of
                                   moe_prepack_weights_mx in w13 / w13_scale / w2 / w2_scale */
    const uint16_t* x;          /* MOE_QUANT_W8A16 only: the bf16 hidden states [T, H]
                                   (16-byte aligned); xq and xs are then unused and may be
                                   NULL.  Ignored by the other schemes. */
    /* Optional test outputs (NULL in production; all three NULL, or debug_h and debug_hq and,
     * except for MOE_QUANT_W8A16, debug_hs).  They expose the SwiGLU + re-quantisation step of
     * the gate+up epilogue (the "SiLU products are quantised to E4M3 per (row, 128 group)" of
     * the fp8_grouped_tc_w8a8.rs module doc) for a unit check, each [T*k, ...] in sorted-slot
     * order (row s = expert_offsets[e] + i):
     *   debug_h   float32 [T*k, I]: h = silu(g) * u as the epilogue computed it, before the
     *             re-quantisation;
     *   debug_hq  [T*k, I] the re-quantised h that the down GEMM reads, copied out of its
     *             operand layout: E4M3 codes, or bf16 (2 bytes each) for MOE_QUANT_W8A16;
     *   debug_hs  [T*k, I/128] its UE8M0 scales ([T*k, I/32] for the MX schemes).
     * The gate+up GEMM then runs a variant that also stores h, and one more kernel copies hq
     * and hs out; expert_out is the same as without them. */
    float*         debug_h;
    uint8_t*       debug_hq;
    uint8_t*       debug_hs;
    /* Optional per-expert biases (the w13_bias / w2_bias of the "Fused MoE" page's interface
     * table), float32 device memory, 4-byte aligned, NULL for none; rows indexed by expert:
     *   w13_bias [E, 2I]: gate columns then up columns, added to gu before SwiGLU;
     *   w2_bias  [E, H]:  added to expert_out (before the routing weight of moe_combine). */
    const float*   w13_bias;
    const float*   w2_bias;
} moe_ffn_args;

int moe_grouped_ffn(const moe_ffn_args* a);
/* covers every quantisation scheme */
size_t moe_ffn_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k);

/* moe_combine: y[t, c] = bf16_RNE( sum_{j<k} topk_weights[t, j] * expert_out[assign_pos[t*k+j], c] ),
 * the sum taken in float32 in increasing j (the `combine` stage: restore token order and
 * merge; the MATE page's contiguous bfloat16 output).  Deterministic.
 *   expert_out [T*k, H] of dtype MOE_DTYPE_F32 or MOE_DTYPE_BF16, 16-byte aligned;
 *   y [T, H] bf16, contiguous, 8-byte aligned.  H % 4 == 0; T * k < 2^29.
 *   assign_pos entries < 0 are skipped (dropped assignments). */
int moe_combine(const void* expert_out, int32_t dtype, const int32_t* assign_pos,
                const float* topk_weights, int32_t T, int32_t k, int32_t H,
                uint16_t* y, void* stream);

/* ---- the whole step -------------------------------------------------------------------- */
#define MOE_FUSED_EXPERT_OUT_BF16  1   /* keep the per-assignment expert outputs in bf16 */
/* One shared expert (the metrale grouped FP8 MoE page's shared gate/up/down, "GroupedExpertIo"
 * and the W8A8 gate_up / down launches that also take the shared projections): every token also
 * runs through expert E, whose weights follow the E routed experts' in w13..w2_scale (E + 1
 * experts, same H and I and packing), and its output is added to y with weight 1 (the routed
 * weights keep routed_scaling_factor).  It runs in the same grouped launches as an extra
 * expert with T rows: topk_ids / topk_weights then have k + 1 columns (column k = E, weight
 * 1.0) and expert_counts E + 1 entries.  moe_workspace_size takes the same flags. */
#define MOE_FUSED_SHARED_EXPERT    2

/* Stage boundaries of moe_fused, for timing: quant_act | route (incl. prelude) | dispatch
 * (incl. the GEMM tile list) | gate+up GEMM | down GEMM | combine.  The activation
 * quantisation runs inside the routing kernel, so its own stage is empty. */
#define MOE_STAGES 6

/* moe_fused: route, dispatch, quant_act, grouped FFN and combine in one call, with no host
 * synchronisation (the single entry point of the MATE page's fp8_fp8_mega_moe, restricted
 * to one GPU).  Output y [T, H] bf16 has the shape of hidden_states ("Fused MoE", return
 * value).
 *   route             routing parameters; route.num_experts = E.
 *   hidden_states     [T, H] bf16.
 *   router_logits     [T, E] float32, or NULL when prelude != NULL.
 *   w13..w2_scale     packed weights and logical scales as for moe_grouped_ffn.
 *   topk_ids, topk_weights, expert_counts   optional outputs ([T,k], [T,k], [E]; with
 *                     MOE_FUSED_SHARED_EXPERT [T,k+1], [T,k+1], [E+1]); NULL to skip.
 *   flags             MOE_FUSED_EXPERT_OUT_BF16 | MOE_FUSED_SHARED_EXPERT.
 *   workspace         >= moe_workspace_size(T, H, I, E, k, flags) bytes (covers the prelude).
 *   stage_events      NULL, or MOE_STAGES + 1 hipEvent_t (created by the caller; NULL entries
 *                     are skipped) recorded on `stream` before the first and after every stage.
 *   act_q, act_scales optional outputs (each NULL, or 16-byte aligned device memory that the
 *                     call writes and then reads): the activations quantised for the gate+up
 *                     GEMM go there instead of into the workspace.  act_q [T, H] E4M3FN codes
 *                     (all three activation-quantising schemes use E4M3); act_scales UE8M0,
 *                     [T, H/128] for MOE_QUANT_FP8, [T, H/32] for MOE_QUANT_MXFP8 and
 *                     MOE_QUANT_W4A8.  MOE_QUANT_W8A16 quantises no activations: both must be
 *                     NULL then. */
typedef struct moe_fused_args {
    int32_t T, H, I;
    moe_route_params route;
    const uint16_t* hidden_states;
    const float*    router_logits;
    const moe_gate_prelude* prelude;
    const uint8_t* w13;
    const uint8_t* w13_scale;
    const uint8_t* w2;
    const uint8_t* w2_scale;
    uint16_t*      y;
    int32_t*       topk_ids;
    float*         topk_weights;
    int32_t*       expert_counts;
    int32_t        flags;
    void*          workspace;
    size_t         workspace_bytes;
    void*          stream;
    void* const*   stage_events;
    int32_t        quant;       /* MOE_QUANT_*: packed weights and scales of that scheme */
    uint8_t*       act_q;       /* optional: the step's quantised activations go here */
    uint8_t*       act_scales;  /* optional: their UE8M0 scales */
    /* Optional per-expert biases as in moe_ffn_args (float32, NULL for none): w13_bias [E, 2I]
     * on the gate/up sums before SwiGLU, w2_bias [E, H] on each expert's output before its
     * routing weight; with MOE_FUSED_SHARED_EXPERT both have E + 1 rows (row E: the shared
     * expert's). */
    const float*   w13_bias;
    const float*   w2_bias;
} moe_fused_args;

int moe_fused(const moe_fused_args* a);
size_t moe_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t flags);

/* moe_fused_static: moe_fused for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The step's
 * temporaries live in a scratch array of MOE_STATIC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends; the call allocates nothing.  Arguments are
 * those of moe_fused except that workspace must be NULL and workspace_bytes 0; steps whose
 * moe_workspace_size(T, H, I, E, k, flags) exceeds MOE_STATIC_SCRATCH_BYTES are rejected
 * with MOE_ERR_UNSUPPORTED before anything is launched.  Every call on one GPU uses that
 * GPU's one array: calls that overlap on one GPU (other streams, other host threads) race
 * and must be serialised by the caller; the array keeps the last call's contents, and the
 * step needs none of them to start at zero.  The first call on a device looks the array's
 * address up with that device current. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
int moe_fused_static(const moe_fused_args* a);

/* Thread-local description of the last error returned on this thread ("" after success). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FP8_H */
