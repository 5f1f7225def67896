/*
 * wan_attn.h -- C ABI of the Wan2.2 DiT self-attention hot path on AMD
 * Instinct MI355X (gfx950).
 *
 * One self-attention step of the Wan2.2 video diffusion transformer:
 *
 *   packed [Q|K|V] projection output (bf16, one allocation)
 *     -> wan_qknorm_rope : RMSNorm of Q and of K over the full model width,
 *                          x gamma, rounded to bf16, 3-D rotary embedding over
 *                          the (frame, row, column) token grid, rounded to bf16,
 *                          written back in place
 *     -> wan_attn_fwd    : bidirectional (unmasked) softmax attention of every
 *                          head over every token, read straight from the packed
 *                          buffer
 *   (before the norm, wan_qkv_proj can fill the packed buffer from the token
 *    activations; fp8 variant: wan_qkv_quant_fp8, then wan_attn_fwd_fp8; or
 *    wan_qknorm_rope_quant_fp8 in place of the first two steps)
 *
 * Sources (web pages on Wan2.2, cited by title and section):
 *   "Optimizing High-Quality Offline Video Generation" (AWS Neuron docs):
 *       "Grounding in an output spec" (the token grid and S), "Overview"
 *       (bidirectional DiT), "Tensor parallelism" (40 heads x 128), "Context
 *       parallelism" (K/V chunks and the per-chunk log-sum-exp merge).
 *   "[visual_gen] Optimize Wan2.2 Dataflow" (TensorRT-LLM pull request):
 *       change 1 (Q, K read as strided views of the fused QKV allocation and
 *       updated in place, [Q | K | V] preserved), "Fused Q/K Norm and RoPE"
 *       (fp32 norm -> bf16 -> fp32 RoPE -> bf16), the review comments (the
 *       norm spans num_heads * head_dim; weight index head * head_dim + dim),
 *       change 2 (amax -> E4M3 inverse scale -> quantise), "Fallback
 *       Behavior" (preconditions of the packed path).
 *   "Wan2.2 Text-to-Video" (vLLM-Omni recipe): head_dim == 128, and an
 *       unsupported configuration raises instead of degrading silently.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Layout. The packed buffer is row-major [B, S, 3*D] with D = heads *
 *    head_dim: token (b, s) owns the row at element offset (b*S + s)*3*D;
 *    Q of head h sits at +h*head_dim, K at +D + h*head_dim, V at +2*D +
 *    h*head_dim. Token s of a T x H x W grid is frame f = s / (H*W), row
 *    y = (s / W) % H, column x = s % W.
 *  * Pointers are device pointers (hipMalloc / torch CUDA tensors) unless a
 *    parameter says otherwise. The caller owns every pointer; the library never
 *    frees or retains caller memory. Buffers must be 16-byte aligned (4-byte for
 *    fp32 vectors).
 *  * stream is a hipStream_t (NULL = the default stream). Every entry point
 *    only enqueues work on it and returns; the caller synchronises. Device-side
 *    faults surface at that synchronisation, not in the return code.
 *  * Return value: WAN_OK (0) or a negative wan_status. Argument validation runs
 *    first, touches no memory and makes no HIP call; on any error nothing is
 *    written. There is no fallback path and no environment variable.
 *  * Empty input (B == 0 or S == 0) is a valid no-op that returns WAN_OK
 *    without looking at the pointers.
 *  * head_dim must be 128 (the only head width of the model and of its
 *    kernels); heads must be 1..256.
 *  * Calls are thread-safe; calls on different streams may overlap unless a
 *    function says otherwise.
 */
#ifndef WAN_ATTN_H
#define WAN_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WAN_ABI_VERSION 1

typedef enum {
  WAN_OK = 0,
  WAN_E_NULL = -1,        /* a required pointer is NULL */
  WAN_E_SHAPE = -2,       /* a size is negative, zero where it must not be, or inconsistent */
  WAN_E_UNSUPPORTED = -3, /* head_dim != 128 or heads outside 1..256 */
  WAN_E_ALIGN = -4,       /* a pointer is not aligned as required */
  WAN_E_ALIAS = -5,       /* an output overlaps an input it must not overlap */
  WAN_E_OVERFLOW = -6,    /* a size product overflows int64, or S exceeds 2^31-1 */
  WAN_E_HIP = -7,         /* a HIP runtime call or kernel launch failed */
  WAN_E_NOMEM = -8,       /* a library-owned table could not be allocated */
  WAN_E_VALUE = -9,       /* a scalar argument is out of range (eps, theta, scale) */
  WAN_E_LIMIT = -10       /* beyond the fixed capacity of an allocation-free entry point */
} wan_status;

/* Version of this ABI (WAN_ABI_VERSION of the built library). */
int wan_abi_version(void);

/* Static, human-readable text for a wan_status value. Never NULL. */
const char *wan_status_str(int status);

/*
 * wan_token_grid -- the DiT token grid of a clip ("Optimizing High-Quality
 * Offline Video Generation", Grounding in an output spec): the pipeline rounds
 * the frame's height and width down to a multiple of 16; the VAE compresses
 * space 8x and time 4x (latent frames = (num_frames - 1) / 4 + 1); the DiT
 * patchifies 2 x 2 in space. So
 *   T = (num_frames - 1) / 4 + 1,  H = (height / 16 * 16) / 16,  W = (width / 16 * 16) / 16,
 * and S = T * H * W tokens (832 x 480 at 81 frames: 21 x 30 x 52 = 32,760).
 *
 *   width, height  frame size in pixels, >= 0.
 *   num_frames     >= 1 and num_frames - 1 divisible by 4 (the 4x temporal
 *                  compression keeps the first frame).
 *   T, H, W        host int64_t outputs, written only on success.
 * Pure host arithmetic: no HIP call, no device memory.
 * Errors: WAN_E_NULL (an output pointer), WAN_E_SHAPE (negative size, or
 * num_frames not of the form 4k+1), WAN_E_OVERFLOW (T*H*W beyond int64).
 */
int wan_token_grid(int64_t width, int64_t height, int64_t num_frames, int64_t *T, int64_t *H, int64_t *W);

/*
 * wan_qkv_proj -- the QKV projection that fills the packed buffer: for every
 * token, [Q | K | V] = x W^T + bias. "Optimize Wan2.2 Dataflow", change 1: the
 * fused QKV projection produces Q, K and V in one shared allocation (the
 * buffer wan_qknorm_rope and wan_attn_fwd then read in place); "Optimizing
 * High-Quality Offline Video Generation", NKI kernels: qkv_cte is this
 * projection, fused there with the norm and RoPE -- wan_qkv_proj_norm_rope
 * below is that fused form; this one leaves the norm to wan_qknorm_rope).
 *
 *   x      bf16 [B, S, D] token activations, D = heads * head_dim.
 *   w_qkv  bf16 [3*D, D]: one row per output feature (features 0..D-1 are Q,
 *          D..2D-1 K, 2D..3D-1 V), i.e. the stacked weights of the three
 *          linear layers in their usual (out_features, in_features) layout.
 *   bias   bf16 [3*D] or NULL.
 *   qkv    bf16 [B, S, 3*D] output (the packed buffer); must not overlap an
 *          input.
 * Arithmetic: bf16 products accumulated in fp32 (gfx950 MFMA), bias added in
 * fp32, one round-to-nearest-even to bf16.
 * Launch: a persistent grid taking output tiles from a 32-byte block of
 * device counters (per-XCD tile queues when the 3*D output features form 57
 * to 64 tiles of 256, as at D = 5120; else one counter), one block per call
 * from a ring of 65,536 per device that the library allocates (2 MB) on the
 * first call on the device and keeps until the process ends.
 * Errors: WAN_E_NULL, WAN_E_SHAPE, WAN_E_UNSUPPORTED, WAN_E_ALIGN (16-byte),
 * WAN_E_ALIAS, WAN_E_OVERFLOW (also B*S above 2^31 - 257 token rows),
 * WAN_E_NOMEM (the counter), WAN_E_HIP.
 */
int wan_qkv_proj(const void *x, const void *w_qkv, const void *bias, void *qkv, int64_t B, int64_t S,
                 int64_t heads, int64_t head_dim, void *stream);

/*
 * wan_qknorm_rope -- in-place Q/K RMSNorm + bf16 rounding point + 3-D RoPE.
 *
 * For every token row and separately for Q and K ("Optimize Wan2.2 Dataflow":
 * change 1, "Fused Q/K Norm and RoPE", and the review comments):
 *   ms   = mean over all D channels of x^2        (fp32 accumulation)
 *   n_c  = bf16( x_c * (ms + eps)^-1/2 * gamma[c] ), c = h*head_dim + i
 *   RoPE on interleaved pairs (2j, 2j+1) of each head: pairs 0..21 rotate with
 *   the frame index, 22..42 with the row index, 43..63 with the column index
 *   (the 44/42/42 channel split of Wan2.2's 3-D rotary embedding); pair j' of an
 *   axis with d_a channels has angle pos * theta^(-2 j' / d_a);
 *   out = bf16( rotate(n) ), fp32 arithmetic, stored over Q and K in place.
 *
 *   qkv      bf16 [B, S, 3*D], S = T*H*W, in/out. Q and K are overwritten; V is
 *            never read or written.
 *   gamma_q  bf16 [D], RMSNorm weight of Q (norm_q); read only.
 *   gamma_k  bf16 [D], RMSNorm weight of K (norm_k); read only.
 *   B        batch (2 = the classifier-free-guidance pair), >= 0.
 *   T, H, W  token grid (frames, rows, columns), each >= 0.
 *   heads    number of heads (40 for Wan2.2-A14B); head_dim must be 128.
 *   eps      RMSNorm epsilon (1e-6), finite and >= 0.
 *   theta    RoPE base (10000), finite and > 0.
 *
 * The cos/sin tables of a (device, T, H, W, theta) are computed once by a
 * device kernel in double precision, rounded to fp32, and kept in a
 * library-owned device allocation for the life of the process (its first call
 * per shape therefore allocates and synchronises the stream once; later calls
 * only launch).
 * Errors: WAN_E_NULL, WAN_E_SHAPE, WAN_E_UNSUPPORTED, WAN_E_ALIGN (qkv, gammas
 * 16-byte), WAN_E_ALIAS (a gamma inside qkv), WAN_E_OVERFLOW, WAN_E_VALUE,
 * WAN_E_NOMEM, WAN_E_HIP.
 */
int wan_qknorm_rope(void *qkv, const void *gamma_q, const void *gamma_k,
                    int64_t B, int64_t T, int64_t H, int64_t W,
                    int64_t heads, int64_t head_dim,
                    float eps, float theta, void *stream);

/*
 * wan_qkv_proj_norm_rope -- the QKV projection with the Q/K RMSNorm and 3-D
 * RoPE in its epilogue ("Optimizing High-Quality Offline Video Generation",
 * NKI kernels: qkv_cte fuses the QKV projection, the distributed QK RMSNorm and
 * RoPE). Computes what wan_qkv_proj followed by wan_qknorm_rope computes:
 *   y   = bf16( x W^T + bias )                     (as wan_qkv_proj)
 *   Q,K = the norm + RoPE of wan_qknorm_rope applied to y, V = y,
 * without writing the unnormalised Q and K to memory. The mean square of a
 * token's Q (and K) is summed from per-head partial sums exchanged between the
 * output tiles of the token's block (the single-GPU counterpart of the pages'
 * norm distributed over tensor-parallel ranks), so its fp32 summation order
 * differs from wan_qknorm_rope's: an output can differ from the two-call
 * result where the bf16 rounding of n_c or of the rotation sits at a tie.
 *
 *   x, w_qkv, bias   as wan_qkv_proj (bias may be NULL).
 *   gamma_q, gamma_k, T, H, W, eps, theta   as wan_qknorm_rope (S = T*H*W).
 *   qkv        bf16 [B, S, 3*D] output; must not overlap an input.
 *   workspace  device memory of at least
 *              wan_qkv_proj_norm_rope_workspace_bytes(B, S, heads, head_dim)
 *              bytes, 16-byte aligned, caller-owned, overlapping no other
 *              argument; its contents on entry do not matter. After the call
 *              completes, the 32-bit word at byte offset 4 is nonzero if a
 *              token block's wait for its partial sums hit the kernel's spin
 *              limit (about a second: only when other work holds the device);
 *              the Q and K outputs of such blocks are then NaN. Calls that
 *              share a workspace must be ordered (same stream). The
 *              environment variable WAN_PROJ_NORM_SPIN_LIMIT, read at each
 *              call, lowers the wait bound (polls; tests force the time-out
 *              path with 0).
 * Launch: a persistent grid, one workgroup per CU slot, taking output tiles
 * from a counter in the workspace; requires room on the device for `heads`
 * workgroups at once (WAN_E_UNSUPPORTED otherwise).
 * Errors: as wan_qkv_proj and wan_qknorm_rope; WAN_E_NULL (workspace),
 * WAN_E_SHAPE (workspace_bytes too small), WAN_E_ALIGN, WAN_E_ALIAS (the
 * workspace or a gamma overlapping another buffer), WAN_E_UNSUPPORTED.
 */
int wan_qkv_proj_norm_rope(const void *x, const void *w_qkv, const void *bias,
                           const void *gamma_q, const void *gamma_k, void *qkv,
                           void *workspace, int64_t workspace_bytes,
                           int64_t B, int64_t T, int64_t H, int64_t W,
                           int64_t heads, int64_t head_dim,
                           float eps, float theta, void *stream);

/* Workspace bytes of wan_qkv_proj_norm_rope for B x S tokens (S = T*H*W):
 * 256 + 8 * ceil(B*S / 256) rounded up to 256, + B*S * 2*heads * 8;
 * -1 on invalid sizes or overflow. Pure host arithmetic. */
int64_t wan_qkv_proj_norm_rope_workspace_bytes(int64_t B, int64_t S, int64_t heads, int64_t head_dim);

/*
 * wan_attn_fwd -- bidirectional multi-head softmax attention on the packed
 * buffer (AWS page "Overview": the DiT denoiser is bidirectional; "Tensor
 * parallelism": 40 heads of 128).
 *
 *   out[b, s, h*128 + i] = sum_t p(s,t) V[b,t,h,i],
 *   p(s,t) = softmax_t( Q[b,s,h,:] . K[b,t,h,:] * softmax_scale )
 * over every key t < S; no mask, no dropout. QK^T and PV run on bf16 MFMA with
 * fp32 accumulation; the softmax is fp32; P is rounded to bf16 for PV. With
 * lse == NULL the row sum that normalises the output is the fp32 sum of those
 * bf16 weights; with an lse buffer it is the fp32 sum of the unrounded
 * probabilities, so that the returned log-sum-exp is that of the scores up to
 * fp32 rounding (the two differ in the output by at most 2^-9 relative).
 *
 *   qkv            bf16 [B, S, 3*D] packed buffer (normally after
 *                  wan_qknorm_rope); read only.
 *   out            bf16 [B, S, D], head h at channels h*128..; written fully.
 *                  Must not overlap qkv.
 *   lse            fp32 [B, heads, S] natural-log log-sum-exp of every score
 *                  row (m + ln sum exp(s - m)), or NULL to skip it. Must not
 *                  overlap qkv or out.
 *   softmax_scale  > 0 and finite (1/sqrt(128) for the model).
 * Errors: WAN_E_NULL, WAN_E_SHAPE, WAN_E_UNSUPPORTED, WAN_E_ALIGN, WAN_E_ALIAS,
 * WAN_E_OVERFLOW, WAN_E_VALUE, WAN_E_HIP.
 */
int wan_attn_fwd(const void *qkv, void *out, float *lse,
                 int64_t B, int64_t S, int64_t heads, int64_t head_dim,
                 float softmax_scale, void *stream);

/*
 * wan_attn_fwd_skip -- wan_attn_fwd with Skip-Softmax in threshold mode (the
 * vLLM-Omni recipe "Wan2.2 Text-to-Video", section "Accelerating with
 * TRTLLM_ATTN + Skip-Softmax", table "Skip-Softmax controls": `threshold` is a
 * direct skip threshold, finite and >= 0, calibration-free; the mode does not
 * apply to ring sequence parallelism, so there is no chunk variant).
 *
 * The page defines the knob, not the rule; the rule implemented: keys are
 * taken in blocks of WAN_SKIP_BLOCK_K consecutive keys in increasing order and
 * queries in blocks of WAN_SKIP_BLOCK_Q consecutive rows (from key 0 and row 0
 * of each (b, head)). For query row i and key block j, let m_j(i) be the
 * block's largest score and M_j(i) the largest score of all earlier blocks
 * (-inf for j = 0). Block j is skipped for a query block when
 *   exp(m_j(i) - M_j(i)) < threshold   for every row i of the query block;
 * a skipped block contributes neither to the softmax numerator nor to its
 * denominator. Block 0 is always kept; threshold = 0 is dense attention. The
 * scores of every block are computed; only the softmax and PV of a skipped
 * block are not.
 *
 *   qkv, out, lse, B, S, heads, head_dim, softmax_scale: as wan_attn_fwd
 *              (lse, when given, is over the kept keys).
 *   kept       uint8 [B, heads, ceil(S / WAN_SKIP_BLOCK_Q), ceil(S / WAN_SKIP_BLOCK_K)]
 *              decision map (1 = the block was kept for that query block), or
 *              NULL; size from wan_attn_skip_map_bytes(). Must not overlap
 *              the other buffers.
 *   threshold  finite, >= 0.
 * Errors: as wan_attn_fwd; WAN_E_VALUE also for a negative or non-finite
 * threshold.
 */
#define WAN_SKIP_BLOCK_Q 48
#define WAN_SKIP_BLOCK_K 64
int wan_attn_fwd_skip(const void *qkv, void *out, float *lse, uint8_t *kept,
                      int64_t B, int64_t S, int64_t heads, int64_t head_dim,
                      float softmax_scale, float threshold, void *stream);

/* Bytes of the decision map of wan_attn_fwd_skip; -1 on invalid sizes or
 * overflow. Pure host arithmetic. */
int64_t wan_attn_skip_map_bytes(int64_t B, int64_t S, int64_t heads, int64_t head_dim);

/*
 * wan_attn_fwd_chunk -- one round of ring attention on one device ("Optimizing
 * High-Quality Offline Video Generation", Context parallelism: each rank keeps
 * its S/CP queries and K/V chunks rotate around the ring so the local queries
 * attend the whole sequence). The local queries attend ONE chunk of keys and
 * values; the result is normalised within the chunk and returned with its
 * log-sum-exp, ready for wan_attn_merge.
 *
 *   q_src      bf16 [B, Sq, 3*D] packed buffer; its Q part holds the queries.
 *   kv_src     bf16 [B, Skv, 3*D] packed buffer; its K and V parts hold the
 *              chunk (may be q_src itself). Both read only.
 *   out        fp32 [B, Sq, D]: softmax over the chunk's keys times its values.
 *   lse        fp32 [B, heads, Sq]: natural log-sum-exp of the chunk's scores
 *              (required).
 * Sq == 0 or B == 0 is a no-op; Skv must be >= 1 when there are queries.
 * out and lse must not overlap the inputs or each other.
 * Errors: as wan_attn_fwd (WAN_E_SHAPE also for Skv == 0).
 */
int wan_attn_fwd_chunk(const void *q_src, int64_t Sq, const void *kv_src, int64_t Skv,
                       float *out, float *lse, int64_t B, int64_t heads, int64_t head_dim,
                       float softmax_scale, void *stream);

/*
 * wan_attn_merge -- fold a chunk result into an accumulator of earlier chunks
 * (disjoint key sets), in place:
 *   L = log(exp(acc_lse) + exp(chunk_lse));
 *   acc_out = exp(acc_lse - L) acc_out + exp(chunk_lse - L) chunk_out;  acc_lse = L
 * An accumulator row with acc_lse = -inf counts as empty.
 *   acc_out    fp32 [B, Sq, D] in/out;   acc_lse   fp32 [B, heads, Sq] in/out.
 *   chunk_out  fp32 [B, Sq, D];          chunk_lse fp32 [B, heads, Sq].
 *   out_bf16   bf16 [B, Sq, D] copy of the merged output, or NULL.
 * No two buffers may overlap. Errors: WAN_E_NULL, WAN_E_SHAPE,
 * WAN_E_UNSUPPORTED, WAN_E_ALIGN, WAN_E_ALIAS, WAN_E_OVERFLOW, WAN_E_HIP.
 */
int wan_attn_merge(float *acc_out, float *acc_lse, const float *chunk_out, const float *chunk_lse,
                   void *out_bf16, int64_t B, int64_t Sq, int64_t heads, int64_t head_dim,
                   void *stream);

/*
 * wan_attn_fwd_chunk_merge -- one ring round with the merge done in the
 * attention epilogue: the queries of q_src attend the chunk of kv_src, and the
 * result is folded straight into the accumulator with the wan_attn_merge
 * formula, bit-identical to wan_attn_fwd_chunk followed by wan_attn_merge (the
 * chunk's fp32 output is never written). Same sources as those two calls.
 *
 *   q_src, kv_src, Sq, Skv, B, heads, head_dim, softmax_scale: as
 *              wan_attn_fwd_chunk.
 *   acc_out    fp32 [B, Sq, D] in/out;  acc_lse  fp32 [B, heads, Sq] in/out
 *              (required; an LSE of -inf marks an empty row, whose acc_out is
 *              not read).
 *   out_bf16   bf16 [B, Sq, D] copy of the merged output, or NULL.
 * acc_out, acc_lse and out_bf16 must not overlap the inputs or each other.
 * Errors: as wan_attn_fwd_chunk, plus WAN_E_ALIAS / WAN_E_ALIGN for out_bf16.
 */
int wan_attn_fwd_chunk_merge(const void *q_src, int64_t Sq, const void *kv_src, int64_t Skv,
                             float *acc_out, float *acc_lse, void *out_bf16, int64_t B, int64_t heads,
                             int64_t head_dim, float softmax_scale, void *stream);

/*
 * wan_qkv_quant_fp8 -- per-tensor e4m3 quantisation of Q, K and V for the fp8
 * attention path (the amax -> E4M3 scale -> quantise recipe of "Optimize Wan2.2
 * Dataflow", change 2, applied to the attention inputs; the pull request's
 * 720p attention itself runs in FP8).
 *
 * For X in (Q, K, V), over all B*S*D elements of X:
 *   amax[X]   = max |x|
 *   scale[X]  = 448 / amax[X] in fp32 (IEEE division), or 1 if amax is 0
 *   x8        = e4m3( fl32(x * scale[X]) ), round to nearest even, saturated
 *               to +-448 (OCP E4M3, the gfx950 fp8 format; never NaN)
 *
 *   qkv     bf16 [B, S, 3*D] packed buffer (normally after wan_qknorm_rope);
 *           read only.
 *   qk8     e4m3 [B, S, 2*D] output: per token Q (all heads) then K.
 *   vt8     e4m3 [B, heads, 128, S_pad] output: V of each head transposed
 *           (channel-major, keys contiguous), S_pad = S rounded up to 128;
 *           positions S..S_pad-1 are written as 0. Size: wan_fp8_vt_bytes().
 *   scales  device float[3] output: scale of Q, K, V (x8 = x * scale).
 *   amax    device float[3] output: amax of Q, K, V (also used as the
 *           reduction target; cleared by the call itself).
 * Three kernels on `stream` (clear, amax, quantise). Outputs must not overlap
 * each other or qkv. Calls that share `amax` must not overlap in time.
 * Errors: WAN_E_NULL, WAN_E_SHAPE, WAN_E_UNSUPPORTED, WAN_E_ALIGN (16-byte
 * tensors, 4-byte scale vectors), WAN_E_ALIAS, WAN_E_OVERFLOW (also B > 65535),
 * WAN_E_HIP.
 */
int wan_qkv_quant_fp8(const void *qkv, void *qk8, void *vt8, float *scales, float *amax,
                      int64_t B, int64_t S, int64_t heads, int64_t head_dim, void *stream);

/*
 * wan_qknorm_rope_quant_fp8 -- wan_qknorm_rope followed by wan_qkv_quant_fp8 on
 * its result, with the amax step folded into the norm pass: while Q and K are
 * normalised, rotated and written back (bf16, in place), the same pass takes
 * max |x| of the values it writes and of V, so the quantisation needs no
 * separate pass over the buffer to find them ("Optimize Wan2.2 Dataflow":
 * change 2 fuses amax, E4M3 scale and quantisation into the producing kernel;
 * here the producer is the fused Q/K norm + RoPE of the same pull request).
 *
 * Every output is bit-identical to the two calls in sequence with the same
 * arguments: qkv (Q, K updated in place), qk8, vt8, scales and amax.
 * Arguments: those of wan_qknorm_rope (qkv, gamma_q, gamma_k, B, T, H, W,
 * heads, head_dim, eps, theta), then those of wan_qkv_quant_fp8 (qk8, vt8,
 * scales, amax; S = T*H*W), then the stream. Three kernels on `stream`
 * (clear amax, norm + RoPE + amax, quantise). Calls that share `amax` must
 * not overlap in time.
 * Errors: those of both calls; WAN_E_ALIAS also when a gamma overlaps an fp8
 * output.
 */
int wan_qknorm_rope_quant_fp8(void *qkv, const void *gamma_q, const void *gamma_k, int64_t B, int64_t T,
                              int64_t H, int64_t W, int64_t heads, int64_t head_dim, float eps, float theta,
                              void *qk8, void *vt8, float *scales, float *amax, void *stream);

/*
 * wan_qknorm_rope_noalloc -- wan_qknorm_rope for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, same output bit for bit. It never
 * allocates or frees: the rotary tables live in a fixed library-owned device
 * array of 65,536 (cos, sin) entries per device (512 KiB, held until the
 * process ends) and are rebuilt on `stream` by every call, so the grid must
 * satisfy T*22 + H*21 + W*21 <= 65,536 (else WAN_E_LIMIT, nothing launched).
 * Every call on a device shares that device's array: calls on one device that
 * overlap in time (different streams, or threads without ordering) race on it.
 * Errors: those of wan_qknorm_rope except WAN_E_NOMEM; WAN_E_LIMIT.
 */
int wan_qknorm_rope_noalloc(void *qkv, const void *gamma_q, const void *gamma_k,
                            int64_t B, int64_t T, int64_t H, int64_t W,
                            int64_t heads, int64_t head_dim,
                            float eps, float theta, void *stream);

/*
 * wan_qknorm_rope_quant_fp8_delayed -- the single-pass fp8 producer: the norm
 * + RoPE of wan_qknorm_rope and the e4m3 quantisation of wan_qkv_quant_fp8 in
 * one pass over Q and K and one over V, with DELAYED per-tensor scales
 * ("Optimize Wan2.2 Dataflow", change 2: amax, E4M3 scale and quantisation in
 * the producing kernel). One scale per tensor cannot come from the amax of
 * the tensor being written in a single pass, so each tensor's scale is taken
 * from the amax an earlier call reported (for the DiT: the previous layer or
 * step), and the call reports the amax of what it wrote for the next one:
 *   scale[X] = 448 / amax_prev[X] (fp32 IEEE division; 1 if amax_prev[X] is 0)
 *   x8       = e4m3( fl32(x * scale[X]) ), round to nearest even; a value with
 *              |x * scale| > 448 saturates to +-448
 *   amax[X]  = max |x| over the tensor quantised (the bf16 Q and K the norm +
 *              RoPE step produces -- bit-identical to wan_qknorm_rope's -- and V)
 * With amax_prev equal to the data's own amax, every output equals
 * wan_qknorm_rope followed by wan_qkv_quant_fp8 (the current-scale recipe).
 *
 *   qkv        bf16 [B, S, 3*D], S = T*H*W: READ ONLY (the bf16 result is not
 *              written back; Q and K reach attention as e4m3 only).
 *   gamma_q, gamma_k, B, T, H, W, heads, head_dim, eps, theta: as wan_qknorm_rope.
 *   amax_prev  device float[3] input: earlier amax of Q, K, V.
 *   qk8, vt8   e4m3 outputs, layouts as wan_qkv_quant_fp8.
 *   scales     device float[3] output: the scales used (what wan_attn_fwd_fp8
 *              takes).
 *   amax       device float[3] output: amax of this call's Q, K, V (cleared by
 *              the call; pass it as amax_prev to the next call, into a
 *              different buffer).
 * Reads 4*D + 2*D bytes and writes 3*D bytes per token (the two-call path
 * reads and writes the bf16 Q and K in place and reads Q, K, V once more).
 * Three kernels on `stream` (clear amax, norm + RoPE + e4m3 Q/K, e4m3 V^T).
 * Outputs must not overlap each other, qkv, the gammas or amax_prev. Calls
 * that share `amax` must not overlap in time.
 * Errors: those of wan_qknorm_rope_quant_fp8; WAN_E_NULL / WAN_E_ALIGN /
 * WAN_E_ALIAS also for amax_prev.
 */
int wan_qknorm_rope_quant_fp8_delayed(const void *qkv, const void *gamma_q, const void *gamma_k, int64_t B,
                                      int64_t T, int64_t H, int64_t W, int64_t heads, int64_t head_dim, float eps,
                                      float theta, const float *amax_prev, void *qk8, void *vt8, float *scales,
                                      float *amax, void *stream);

/* Bytes of the vt8 buffer for (B, S, heads, head_dim); -1 on invalid sizes or
 * overflow. Pure host arithmetic. */
int64_t wan_fp8_vt_bytes(int64_t B, int64_t S, int64_t heads, int64_t head_dim);

/*
 * wan_attn_fwd_fp8 -- bidirectional attention from the wan_qkv_quant_fp8
 * buffers on fp8 MFMA (16x16x128 e4m3, fp32 accumulation):
 *   s     = (q8 . k8) / (scale_q * scale_k) * softmax_scale      (fp32)
 *   p8    = e4m3(2^8 * exp(s - m)), m a running maximum (fp32 softmax, online)
 *   out   = sum_t p8 v8 / (scale_v * sum_t p8)
 *   lse   = m + ln(sum_t exp(s - m)), summed in fp32 before the e4m3 rounding
 *
 *   qk8, vt8, scales  as written by wan_qkv_quant_fp8 for the same sizes.
 *   out               bf16 [B, S, D]; must not overlap the inputs.
 *   lse               fp32 [B, heads, S] natural log-sum-exp of the scores, or NULL.
 * Errors: as wan_attn_fwd.
 */
int wan_attn_fwd_fp8(const void *qk8, const void *vt8, const float *scales, void *out, float *lse,
                     int64_t B, int64_t S, int64_t heads, int64_t head_dim, float softmax_scale,
                     void *stream);

#ifdef __cplusplus
}
#endif

#endif /* WAN_ATTN_H */
