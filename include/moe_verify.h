/* moe_verify.h -- C ABI of the MoE verify-block library (gfx950 / CDNA4).
 *
 * The target model of a speculative decoder checks a whole draft block in one pass and keeps
 * only the tokens it would itself have produced ("Speculating on a Strix Halo", section
 * "Speculative decoding"). In a mixture-of-experts target each block token routes to its own
 * experts, so the block wakes the union of its tokens' experts plus the always-on shared expert
 * ("Speculating on a Strix Halo", sections "What the pieces cost" and "Spoilers"); the expert
 * work is grouped by expert, one grouped launch per projection ("Speculating on a Strix Halo",
 * section "The verify's own cost"). The verify cost tracks the expert bytes streamed
 * ("Speculating on a Strix Halo (part 2)", section "The verification cog").
 *
 * Two calls cover that pass, and a third prepares the weights they read:
 *   moe_verify_block -- one MoE layer over a block of k <= 16 tokens: fp32 router logits,
 *                       top-K with softmax renormalised over the K, woken-expert union, grouped
 *                       SwiGLU experts (bf16 or mxfp4 weights), weighted combine with the shared
 *                       expert, optional RMSNorm pre-norm and residual add; also the blocks of
 *                       many sequences verified together (up to 1024 tokens, bf16 or mxfp4
 *                       weights; mxfp4 experts on the scaled matrix-core instruction);
 *   accept_prefix    -- per-position target argmax and greedy longest-prefix acceptance;
 *   moe_pack_weights -- rearranges row-major expert matrices into the tiled layout the verify
 *                       block streams (done once, when the weights are loaded).
 *
 * Conventions (all calls):
 *   - Pointers are DEVICE memory owned by the caller unless stated otherwise; the library never
 *     allocates, frees or synchronises. Work is enqueued on `hip_stream` (a hipStream_t; NULL is
 *     the default stream) and the call returns; results are valid after the stream completes.
 *   - Only host-visible arguments are validated, all before any HIP call, so a failing status
 *     leaves the stream untouched. Device contents (ids, codes) are not validated.
 *   - Device pointers must be 16-byte aligned.
 *   - Results are deterministic: fixed reduction orders, no floating-point atomics.
 *   - Calls that share a workspace must not overlap in time (same stream is always safe).
 *   - Errors: a launch failure returns MOE_ERR_HIP and clears that error (hipGetLastError). If a
 *     HIP error from the caller's earlier work is already pending in the calling thread when a
 *     call starts, the call enqueues nothing, returns MOE_ERR_HIP and leaves that error pending,
 *     so the caller's own hipGetLastError still reports it.
 */
#ifndef MOE_VERIFY_H
#define MOE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,      /* a required pointer is NULL                                     */
  MOE_ERR_SHAPE = -2,     /* a size is outside the supported range (see each call)           */
  MOE_ERR_DTYPE = -3,     /* unknown weight format or layout, or mxfp4 without its scales   */
  MOE_ERR_ALIGN = -4,     /* a device pointer is not 16-byte aligned                         */
  MOE_ERR_WORKSPACE = -5, /* workspace smaller than the matching *_workspace_size()          */
  MOE_ERR_ALIAS = -6,     /* output overlaps an input it must not overlap                    */
  MOE_ERR_HIP = -7,       /* a launch failed, or an earlier HIP error was pending (device
                             faults surface at the next sync)                             */
  MOE_ERR_ARG = -8        /* unknown flag bits or a bad scalar argument                      */
};

/* Routed-expert weight formats. The shared expert is always bf16. */
enum {
  MOE_W_BF16 = 0,  /* bf16 bit patterns                                                       */
  MOE_W_MXFP4 = 1  /* OCP MX FP4: E2M1 codes, two per byte (element 2j in the low nibble of
                      byte j), one e8m0 scale byte 2^(s-127) per 32 consecutive values along the
                      reduction dimension. Target weights in mxfp4 cut the verify's HBM bytes
                      (DFlash-on-MI355X article, allbreaknews.com/?p=4397, section "Why Quantize
                      the Target Model on Top?"). Scale bytes 1..254 are supported; 0 only on a
                      block whose codes are all zero; 255 (NaN) is not supported. */
};

/* Weight layouts (moe_layer.layout). The verify block streams every woken expert's bytes once
 * per block ("Speculating on a Strix Halo (part 2)", section "The verification cog"), so the
 * expert matrices are stored in the order the kernels consume them: MFMA operand tiles, each
 * 16 rows x 32 reduction columns, 1 KiB contiguous, one 16-byte lane slice after another.
 *
 * MOE_LAYOUT_TILED, for a row-major matrix W[R][C] (R % 16 == 0, C % 128 == 0):
 *   bf16:  16-byte chunk ((rt * (C/32) + s) * 64 + l) holds W[16 rt + l%16][32 s + 8 (l/16) + i],
 *          i = 0..7 (rt < R/16, s < C/32, l < 64).
 *   mxfp4: 16-byte code chunk ((rt * (C/128) + w) * 64 + l) holds the 16 code bytes of 32-value
 *          block 4 w + l/16 of row 16 rt + l%16; scale byte of the same index holds that block's
 *          scale (w < C/128).
 * Each matrix of a stacked [n][R][C] array is tiled on its own (same byte size as row-major).
 * moe_pack_weights produces this layout from row-major arrays. */
enum {
  MOE_LAYOUT_TILED = 1
};

/* moe_verify_block flags: y = [x +] MoE([RMSNorm](x)). */
enum {
  MOE_PRE_RMSNORM = 1u, /* x_hat = x / sqrt(mean(x^2) + rms_eps) (unit gain) before the router
                           and the experts, as in a pre-norm stack of MoE layers              */
  MOE_RESIDUAL = 2u,    /* add the un-normalised input x to the MoE output                    */
  MOE_GATHER = 4u       /* use the gathered path (below) for any k; implied for k > 16         */
};

/* One MoE layer (a host struct, read only during the call; the arrays are device memory).
 * Shapes (router_w row-major; expert and shared-expert matrices in MOE_LAYOUT_TILED, each
 * [R][C] below tiled as a matrix of R rows and C reduction columns):
 *   router_w  fp32 [E][H]
 *   w_gate, w_up   bf16 [E][I][H]    | mxfp4 codes [E][I][H/2],  s_gate, s_up  [E][I][H/32]
 *   w_down         bf16 [E][H][I]    | mxfp4 codes [E][H][I/2],  s_down        [E][H][I/32]
 *   sh_gate, sh_up bf16 [Is][H];  sh_down bf16 [H][Is]    (NULL when shared_inter == 0)
 * Expert FFN: y_e = W_down (silu(W_gate x) * (W_up x)), silu(z) = z / (1 + e^-z).
 * Supported sizes: H a multiple of 128 in [128, 1024] or of 256 in [1280, 2048] (mxfp4: a
 * multiple of 256); I a multiple of 128 in [128, 1024]; Is a multiple of 128 in [128, 1024], or 0
 * for no shared expert; 1 <= top_k <= min(E, 16); E <= 512. Layers with I in {128, 256, 512, 1024}
 * and Is in {0, I} run blocks of up to 16 tokens on the single-block kernels; every other layer
 * takes the gathered path at every k (moe_verify_block). */
typedef struct moe_layer {
  int32_t hidden;       /* H */
  int32_t n_experts;    /* E */
  int32_t top_k;        /* K experts routed per token */
  int32_t inter;        /* I, routed expert intermediate size */
  int32_t shared_inter; /* Is, shared expert intermediate size; 0 = no shared expert */
  int32_t wdtype;       /* MOE_W_BF16 | MOE_W_MXFP4 */
  int32_t layout;       /* MOE_LAYOUT_TILED (anything else: MOE_ERR_DTYPE) */
  float rms_eps;        /* used with MOE_PRE_RMSNORM; must be finite and >= 0 */
  const float* router_w;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const uint8_t* s_gate; /* mxfp4 scales; NULL for bf16 */
  const uint8_t* s_up;
  const uint8_t* s_down;
  const void* sh_gate;
  const void* sh_up;
  const void* sh_down;
} moe_layer;

/* Bytes of device workspace moe_verify_block needs for calls of up to k_max tokens, on either
 * path, 1 <= k_max <= 1024 (0 if the layer description is invalid or k_max is out of range).
 * Host only. */
size_t moe_verify_workspace_size(const moe_layer* layer, int32_t k_max);

/* One MoE layer over a verify block.
 *   x        fp32 [k][H]  block hidden states (input; not modified)
 *   k        1 <= k <= 1024 tokens. One sequence's block carries 1 known token and up to 15
 *            drafted ones ("Speculating on a Strix Halo", section "Speculative decoding"); the
 *            blocks of several sequences may be stacked into one call, since every token routes
 *            on its own. With k > 16, MOE_GATHER, or a layer outside the single-block sizes
 *            (I not in {128, 256, 512, 1024}, or a shared expert of another size than I), the
 *            call takes the gathered path: the
 *            tokens are sorted by expert (a deterministic counting sort) and each woken expert
 *            is applied to its own tokens only, 32 token columns per weight pass. That is the
 *            regime of batched serving, where the verify step becomes compute-heavy
 *            (DFlash-on-MI355X article, section "Results: Throughput and Speedup"). With
 *            mxfp4 weights the routed experts run on the scaled matrix-core instruction there
 *            too (MX-fp8 hi/lo activations) and the shared expert in bf16.
 *   flags    MOE_PRE_RMSNORM | MOE_RESIDUAL | MOE_GATHER
 *   y        fp32 [k][H]  output; must not overlap x or the workspace
 *   topk_ids int32 [k][K] or NULL: each token's experts, descending router logit, equal logits
 *            to the lower expert index
 *   topk_w   fp32  [k][K] or NULL: the matching weights, softmax over the K selected logits
 *   n_woken  int32 [1]    or NULL: size of the union of the block's routed experts (shared
 *            expert not counted)
 *   workspace, ws_bytes: device scratch of at least moe_verify_workspace_size(layer, k) bytes
 *            (k_max = 1024 with bf16 weights: about 106 MB at H 2048, E 256, K 8, I 512);
 *            its contents need no initialisation and are overwritten.
 * The single-block path (k <= 16) runs its expert phases in one launch whose workgroups wait for
 * each other's phases through counters in the workspace, one workgroup per compute unit, so every
 * workgroup must be resident at once: a device with fewer compute units than the launch needs
 * (max(k H / 512, Is / 16, H / 64), at most 64 here) gets MOE_ERR_SHAPE. The waits are bounded: if
 * a phase is not complete within seconds (only possible when other work holds the GPU's compute
 * units that long), the call's outputs are invalid and *n_woken is set to -1. Two single-block
 * calls that run at the same time (on different streams) can each hold compute units the other's
 * waiting workgroups need, so both would reach that bound: order such calls on one stream (or
 * with events). The gathered path and the other entry points have no such waits.
 * Returns MOE_OK or an MOE_ERR_* code (nothing is enqueued on error). */
int moe_verify_block(const moe_layer* layer, const float* x, int32_t k, uint32_t flags, float* y,
                     int32_t* topk_ids, float* topk_w, int32_t* n_woken, void* workspace,
                     size_t ws_bytes, void* hip_stream);

/* moe_verify_block with per-kernel timing, for profiling: the same computation and launches;
 * additionally records events[i] (hipEvent_t created and owned by the caller; any entry may be
 * NULL) on hip_stream at the kernel boundaries: [0] before the router kernel, [1] after it
 * (gathered path: after the router, top-K and permutation kernels), [2] after the gate/up
 * phase, [3] after the down phase, [4] after the combine. On the single-block path (k <= 16)
 * gate/up, down and combine are one launch, so [2], [3] and [4] are all recorded after it. A
 * failing event record returns MOE_ERR_HIP. */
int moe_verify_block_timed(const moe_layer* layer, const float* x, int32_t k, uint32_t flags, float* y,
                           int32_t* topk_ids, float* topk_w, int32_t* n_woken, void* workspace,
                           size_t ws_bytes, void* hip_stream, void* const* events /* [5] */);

/* Bytes of the library's own device scratch used by moe_verify_block_noalloc (per GPU). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)24 << 20)

/* moe_verify_block for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Same computation, kernels and
 * results as moe_verify_block; the workspace is a fixed device array inside the library
 * (MOE_NOALLOC_SCRATCH_BYTES, one per GPU, kept until the process ends) instead of a caller
 * buffer, and the call allocates nothing. The caller passes inputs and outputs only.
 *   Covers every k <= 16 block of a supported layer (at most about 19 MB of workspace) and
 *   gathered calls whose moe_verify_workspace_size(layer, k) fits the scratch (about 200 tokens
 *   on the H 2048 / 256-expert / I 512 layer); larger calls return MOE_ERR_WORKSPACE.
 *   Every call on one GPU shares that GPU's scratch, which keeps the last call's contents (no
 *   call depends on them): calls that overlap in time on one GPU (different streams, threads)
 *   race and must be serialised by the caller; calls on one stream are always safe.
 *   The scratch's device address is looked up (hipGetSymbolAddress) on the first call on each
 *   device; a failed lookup returns MOE_ERR_HIP. Other statuses as moe_verify_block. */
int moe_verify_block_noalloc(const moe_layer* layer, const float* x, int32_t k, uint32_t flags, float* y,
                             int32_t* topk_ids, float* topk_w, int32_t* n_woken, void* hip_stream);

/* Largest number of layers one moe_verify_stack call takes. */
#define MOE_STACK_MAX_LAYERS 4096

/* Bytes of device workspace moe_verify_stack needs for blocks of up to k_max tokens of layers of
 * this shape (0 if the layer is invalid, k_max is outside 1..16, or the layer's sizes take the
 * gathered path: see moe_verify_block's supported sizes). Host only. */
size_t moe_verify_stack_workspace_size(const moe_layer* layer, int32_t k_max);

/* A stack of n_layers MoE layers over one block in one call: y = L_{n-1}(... L_1(L_0(x))), each
 * layer as moe_verify_block computes it with the same flags, so with MOE_PRE_RMSNORM |
 * MOE_RESIDUAL the layers form a pre-norm residual stream (the target's MoE layers run back to
 * back in a verify pass: "Speculating on a Strix Halo", section "The verify's own cost"). The
 * result equals, bit for bit, n_layers moe_verify_block calls chained through their outputs: the
 * same two launches per layer, with the intermediate rows in the workspace.
 *   layers    moe_layer [n_layers]: every layer of one shape (hidden, n_experts, top_k, inter,
 *             shared_inter, wdtype, layout); rms_eps and the weights may differ
 *   x, y      fp32 [k][H] input and output (must not overlap each other or the workspace)
 *   k         1..16; the layers' sizes must take the single-block path (I in {128, 256, 512,
 *             1024}, shared_inter 0 or I); other stacks are run with one moe_verify_block call
 *             per layer
 *   flags     MOE_PRE_RMSNORM | MOE_RESIDUAL (MOE_GATHER is not accepted)
 *   n_woken   int32 [n_layers] or NULL: each layer's woken-expert count (-1: that layer's wait
 *             ran past its bound, as in moe_verify_block)
 *   workspace, ws_bytes: at least moe_verify_stack_workspace_size(&layers[0], k) bytes, no
 *             initialisation needed
 * Limits: 1 <= n_layers <= MOE_STACK_MAX_LAYERS. x, y, n_woken and workspace 16-byte aligned.
 * Each layer's launches wait for each other as moe_verify_block's single-block launch does (every
 * workgroup resident; overlapping calls on two streams can exhaust the bound). Returns MOE_OK or
 * an MOE_ERR_* code (nothing is enqueued on an argument error). */
int moe_verify_stack(const moe_layer* layers, int32_t n_layers, const float* x, int32_t k, uint32_t flags, float* y,
                     int32_t* n_woken, void* workspace, size_t ws_bytes, void* hip_stream);

/* Rearranges n_mats row-major matrices of rows x cols into MOE_LAYOUT_TILED (a permutation of
 * 16-byte chunks and, for mxfp4, of scale bytes; output sizes equal input sizes).
 *   wdtype      MOE_W_BF16: src, dst bf16 [n_mats][rows][cols]
 *               MOE_W_MXFP4: src, dst codes [n_mats][rows][cols/2]; src_scales, dst_scales
 *               [n_mats][rows][cols/32] (NULL for bf16)
 *   rows, cols  multiples of 16 and 128 (cols is the reduction dimension: H for gate/up, I for
 *               down), each <= 2^20
 * Outputs must not overlap inputs. Enqueued on hip_stream. Returns MOE_OK, MOE_ERR_NULL,
 * MOE_ERR_DTYPE, MOE_ERR_SHAPE, MOE_ERR_ALIGN (src, dst), MOE_ERR_ALIAS or MOE_ERR_HIP. */
int moe_pack_weights(int32_t wdtype, int32_t n_mats, int32_t rows, int32_t cols, const void* src,
                     const uint8_t* src_scales, void* dst, uint8_t* dst_scales, void* hip_stream);

/* Bytes of device workspace accept_prefix needs (0 if the sizes are invalid). Host only. */
size_t accept_prefix_workspace_size(int32_t n_target, int32_t vocab);

/* Greedy acceptance of a draft block ("Speculating on a Strix Halo", section "Speculative
 * decoding": the target keeps the draft prefix it would itself produce, then adds its own next
 * token; the n-th draft counts only if the ones before it did: "Speculating on a Strix Halo
 * (part 2)", section "Why drafter performance doesn't really matter").
 *   logits     fp32 [n_target][vocab]: the target's logits at each block position
 *   draft_ids  int32 [n_draft] (may be NULL when n_draft == 0); draft i is compared with the
 *              target's choice at position i; ids outside [0, vocab) never match
 *   target_ids int32 [n_target] out: per-row argmax, equal values to the lowest index
 *   accepted   int32 [1] out: a = the longest prefix with draft_ids[i] == target_ids[i]; the
 *              committed tokens are draft_ids[0..a) followed by target_ids[a] when a < n_target
 * Limits: 1 <= n_target <= 64, 0 <= n_draft <= n_target, 1 <= vocab <= 2^24.
 * One launch: chunk workgroups publish their maxima as records tagged for this execution, and
 * the last workgroup reduces them once all are valid (the workspace needs no initialisation).
 * The tags mix a per-call value with a generation word in the workspace that every execution
 * advances, so the call may be captured in a HIP graph and replayed. That wait is bounded: past
 * it (seconds; only when other work holds the GPU that long) *accepted is set to -1 and
 * target_ids are invalid.
 * NaN logits give an unspecified argmax. Returns MOE_OK or an MOE_ERR_* code. */
int accept_prefix(const float* logits, int32_t n_target, int32_t vocab, const int32_t* draft_ids,
                  int32_t n_draft, int32_t* target_ids, int32_t* accepted, void* workspace,
                  size_t ws_bytes, void* hip_stream);

/* Bytes of device workspace accept_prefix_batch needs (0 if the sizes are invalid). Host only. */
size_t accept_prefix_batch_workspace_size(int32_t n_seq, int32_t n_target, int32_t vocab);

/* accept_prefix for many sequences verified together (the blocks of one moe_verify_block call
 * over several sequences): sequence s is judged exactly as accept_prefix judges one block, in
 * one launch for all of them. Draft counts may differ per sequence: a cycle need not draft a
 * full block ("Speculating on a Strix Halo (part 2)", section "llama curiosities").
 *   logits      fp32 [n_seq][n_target][vocab]
 *   draft_ids   int32 [n_seq][n_draft_max] (may be NULL when n_draft_max == 0)
 *   n_draft     int32 [n_seq] or NULL: sequence s compares its first n_draft[s] drafts (device
 *               values are clamped to [0, n_draft_max]); NULL: every sequence has n_draft_max
 *   target_ids  int32 [n_seq][n_target] out: per-row argmax, equal values to the lowest index
 *   accepted    int32 [n_seq] out: each sequence's accepted length
 * Limits: 1 <= n_seq <= 1024, 1 <= n_target <= 64, n_seq * n_target <= 65535,
 * 0 <= n_draft_max <= n_target, 1 <= vocab <= 2^24. One launch, as accept_prefix (a sequence
 * whose wait ran past its bound gets accepted[s] = -1). Returns MOE_OK or an MOE_ERR_* code. */
int accept_prefix_batch(const float* logits, int32_t n_seq, int32_t n_target, int32_t vocab,
                        const int32_t* draft_ids, int32_t n_draft_max, const int32_t* n_draft,
                        int32_t* target_ids, int32_t* accepted, void* workspace, size_t ws_bytes,
                        void* hip_stream);

/* Bytes of device workspace lm_head_accept needs (0 if the sizes are invalid). Host only. */
size_t lm_head_accept_workspace_size(int32_t n_target, int32_t hidden, int32_t vocab);

/* The target's output head with a fused argmax, then greedy acceptance. The head is a single
 * [V x H] matrix read once for the whole block ("Speculating on a Strix Halo", section "What the
 * pieces cost"); it is the hidden-by-vocabulary matrix whose streaming cost grows with V (same
 * page, section "Should we shrink the vocab?"). The logits are never written to memory.
 *   h          fp32 [n_target][hidden]: final hidden states of the block positions (taken as
 *              given, no final normalisation)
 *   w_head     bf16 head weights [V][hidden] in MOE_LAYOUT_TILED, produced by moe_pack_weights
 *              (wdtype MOE_W_BF16, n_mats 1, rows = V rounded up to a multiple of 16, cols =
 *              hidden); rows past V are never selected, whatever they hold
 *   layout     must be MOE_LAYOUT_TILED
 *   draft_ids, n_draft, target_ids, accepted: as in accept_prefix; target_ids[i] is the lowest
 *              row attaining the maximum of h[i] . W[v] over v < vocab
 * Limits: 1 <= n_target <= 16, 0 <= n_draft <= n_target, hidden a multiple of 128 in
 * [128, 2048], 1 <= vocab with round_up(vocab, 16) * hidden * 2 < 2^32. h, w_head, target_ids,
 * accepted, draft_ids and workspace 16-byte aligned; the outputs may not overlap the inputs or
 * the workspace. Non-finite inputs give unspecified ids. Returns MOE_OK or an MOE_ERR_* code;
 * the work is enqueued on hip_stream (NULL: the default stream). */
int lm_head_accept(const float* h, int32_t n_target, int32_t hidden, const void* w_head, int32_t vocab,
                   int32_t layout, const int32_t* draft_ids, int32_t n_draft, int32_t* target_ids,
                   int32_t* accepted, void* workspace, size_t ws_bytes, void* hip_stream);

/* Bytes of device workspace accept_sample needs (0 if the sizes are invalid). Host only. */
size_t accept_sample_workspace_size(int32_t n_target, int32_t n_draft, int32_t vocab);

/* Lossless acceptance at temperature T: the committed tokens are distributed exactly as the
 * target's own samples ("Speculating on a Strix Halo", section "Speculative decoding", which
 * cites Leviathan et al. for the rule). With p_i = softmax(target_logits[i] / T) and
 * q_i = softmax(draft_logits[i] / T), draft i is kept while u_accept[i] * q_i(d_i) < p_i(d_i);
 * at the first rejection a, the token is drawn from the renormalised residual max(0, p_a - q_a)
 * (from p_a if the residual has no mass) as the smallest index whose running weight exceeds
 * u_sample[a] times the total; if every draft is kept, from p_{n_draft} with u_sample[n_draft]
 * when n_target > n_draft, else no token.
 *   target_logits fp32 [n_target][vocab], draft_logits fp32 [n_draft][vocab] (the drafter's
 *                 logits at each draft position), draft_ids int32 [n_draft] (ids outside
 *                 [0, vocab) are rejected)
 *   u_accept fp32 [n_draft], u_sample fp32 [n_target]: uniforms in [0, 1) drawn by the caller
 *   accepted int32 [1] out: a; token int32 [1] out: the target's own token, or -1 when every
 *                 draft is kept and n_target == n_draft
 * draft_logits, draft_ids and u_accept may be NULL when n_draft == 0. Limits: 1 <= n_target <=
 * 64, 0 <= n_draft <= n_target, 1 <= vocab <= 2^24, 0 < temperature < inf. Logit arrays and the
 * workspace 16-byte aligned, the rest 4-byte aligned; outputs may not overlap inputs, each other
 * or the workspace. Logits must be finite except -inf entries (probability zero); u outside
 * [0, 1) and non-finite logits give unspecified results (the token is still an index of positive
 * weight when any exists). Computed in fp32 with base-2 exponents; decisions within fp32
 * rounding of a boundary may differ from exact arithmetic. Returns MOE_OK or an MOE_ERR_* code. */
int accept_sample(const float* target_logits, int32_t n_target, int32_t vocab, const float* draft_logits,
                  const int32_t* draft_ids, int32_t n_draft, float temperature, const float* u_accept,
                  const float* u_sample, int32_t* accepted, int32_t* token, void* workspace, size_t ws_bytes,
                  void* hip_stream);

/* Bytes of device workspace accept_sample_batch needs (0 if the sizes are invalid). Host only. */
size_t accept_sample_batch_workspace_size(int32_t n_seq, int32_t n_target, int32_t n_draft, int32_t vocab);

/* accept_sample for many sequences verified together, in three launches for all of them:
 * sequence s is judged exactly as accept_sample judges one block (same rule, same arithmetic, so
 * each sequence's result equals that call's).
 *   target_logits fp32 [n_seq][n_target][vocab]; draft_logits fp32 [n_seq][n_draft][vocab]
 *   draft_ids int32 [n_seq][n_draft]; u_accept fp32 [n_seq][n_draft]; u_sample fp32 [n_seq][n_target]
 *   accepted, token int32 [n_seq] out
 * Limits as accept_sample, and 1 <= n_seq <= 1024. Returns MOE_OK or an MOE_ERR_* code. */
int accept_sample_batch(const float* target_logits, int32_t n_seq, int32_t n_target, int32_t vocab,
                        const float* draft_logits, const int32_t* draft_ids, int32_t n_draft, float temperature,
                        const float* u_accept, const float* u_sample, int32_t* accepted, int32_t* token,
                        void* workspace, size_t ws_bytes, void* hip_stream);

/* Acceptance statistics over many cycles: the histogram of accepted lengths ("Speculating on a
 * Strix Halo (part 2)", section "Why drafter performance doesn't really matter", counts cycles
 * by accepted length) and the per-position marginal as counts (the DFlash-on-MI355X article
 * plots P(accept >= i + 1) per position).
 *   accepted int32 [n_cycles]; hist int64 [n_draft + 1] out: cycles that accepted exactly j;
 *   survival int64 [n_draft] out (may be NULL when n_draft == 0): cycles that accepted at least
 *   i + 1. Values outside [0, n_draft] are not counted. 0 <= n_draft <= 64, n_cycles >= 0;
 *   accepted 4-byte and the outputs 8-byte aligned, no overlaps. Returns MOE_OK or an
 *   MOE_ERR_* code. */
int accept_histogram(const int32_t* accepted, int32_t n_cycles, int32_t n_draft, int64_t* hist, int64_t* survival,
                     void* hip_stream);

/* Static description of a status code. Host only. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_VERIFY_H */
