/*
 * vsmooth.h -- C ABI of libvsmooth, FP8 (E4M3) FlashAttention-style forward
 * with attention-equivalent K/V smoothing, for AMD CDNA4 (gfx950).
 *
 * The method (sources cited per entry point):
 *   - K is centred by its per-head sequence mean in FP32 before E4M3
 *     quantization; softmax does not change (TeleFuser PR #40, "Changes").
 *   - V tokens may be grouped by k-means and K and V permuted together; the
 *     output does not change (VC-Attention summary, Key Contribution 1 and
 *     "Methodology in Plain English").
 *   - each 128-token block subtracts its V mean and quantizes the residual;
 *     the mean is restored inside the online-softmax recurrence as a
 *     rank-one term from the tile row sum (same sources).
 *   - the probability tile can be written as E4M3 straight from the
 *     log-domain score with one FMA (ExpCast-FP8, VC-Attention summary, Key
 *     Contribution 2).
 *   - output O and the log2 softmax normalizer (FastVideo PR #2048, "Test
 *     Results": output plus log2-LSE); inputs [B, S, H, D] (TeleFuser PR #40,
 *     "Smooth Attention Kernel Accuracy": live shape (1, 32626, 56, 128)).
 *   - options of the fused prologue and of the 4-bit path (VC-Attention
 *     summary, Key Contribution 3 and Main Findings): the gather by the
 *     permutation inside the quantizers, a static space-time cube grouping,
 *     a QK Hadamard rotation, and the V residual as MXFP4.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller (the one
 *     exception, vs_cube_permutation, is a host function on host memory).
 *     The library never allocates, frees or keeps device memory; scratch
 *     space is passed in as a workspace whose size a *_workspace_bytes query
 *     returns.
 *   - bf16 tensors are passed as raw 16-bit patterns (uint16_t).
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*,
 *     NULL = the null stream), stateless, and safe to call from several host
 *     threads on different streams.  Calls that share output or workspace
 *     buffers must be ordered by the caller.
 *   - Arguments are validated on the host before anything is launched; on
 *     any error nothing is launched and the outputs are left untouched.
 *     B, S or H equal to 0 is an empty problem: VS_OK, nothing launched.
 *   - Pointers must be 16-byte aligned (VS_ERR_UNSUPPORTED otherwise).
 *   - D must be 64 or 128 (VS_ERR_UNSUPPORTED otherwise).
 *   - Blocks are 128 consecutive tokens; nb = ceil(S / 128) and
 *     S_pad = 128 * nb.  The last block of a ragged sequence holds S mod 128
 *     valid tokens; its padding rows are encoded as 0 and masked.
 *   - No C++ exception crosses this interface.
 */
#ifndef VSMOOTH_H
#define VSMOOTH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define VS_OK               0
#define VS_ERR_INVALID_ARG  1   /* null pointer, negative size, bad mode   */
#define VS_ERR_UNSUPPORTED  2   /* D not in {64,128}, k > 256, misaligned   */
#define VS_ERR_WORKSPACE    3   /* workspace missing or too small           */
#define VS_ERR_HIP          4   /* a HIP launch or runtime call failed      */

/* token layouts of bf16 K / V inputs */
#define VS_LAYOUT_BSHD 0        /* [B, S, H, D], D contiguous                */
#define VS_LAYOUT_BHSD 1        /* [B, H, S, D], D contiguous                */

/* V mean modes */
#define VS_VMEAN_NONE  0        /* V quantized as is, nothing restored       */
#define VS_VMEAN_BLOCK 1        /* per-128-block mean, restored per tile     */
#define VS_VMEAN_SEQ   2        /* one sequence mean, restored at the end    */
#define VS_VMEAN_BLOCK_OUT 3    /* vs_quantize_residual only: forms the      */
                                /* per-block means itself and writes them;   */
                                /* attention then takes VS_VMEAN_BLOCK       */

/* vs_fp8_attn_fwd flags */
#define VS_EXPCAST 1u           /* ExpCast-FP8 probability cast              */

/* vs_quantize_residual_ex flags */
#define VS_QK_HADAMARD 1u       /* rotate Q and centred K by H_D first       */
/* vs_quantize_residual_ex and vs_fp8_attn_fwd flag */
#define VS_V_MXFP4 2u           /* V residual as MXFP4 (E2M1, E8M0 per 32)   */
/* vs_fp8_attn_fwd flag */
#define VS_OUT_BF16 4u          /* attention output in bf16 instead of f32   */
/* vs_quantize_residual_ex and vs_fp8_attn_fwd flag */
#define VS_BF16_MMA 8u           /* Q, K operands as scaled bf16; QK^T on the */
                                /* bf16 matrix core (FP32-accurate scores)   */
/* vs_quantize_residual_ex and vs_fp8_attn_fwd flag */
#define VS_P_MXFP4 16u          /* 4-bit probability tile (E2M1, E8M0 per 32 */
                                /* keys) and the V code order it reads       */

/* Human-readable name of a return code (static string, never NULL). */
const char* vs_status_string(int status);

/* Library version string, "major.minor.patch". */
const char* vs_version(void);

/*
 * vs_smooth_stats -- exact K/V statistics in one pass over K and V.
 * Source: TeleFuser PR #40, "Changes" (fuse exact K/V statistics into one
 * reduction; centre K in FP32; centre V and restore its mean) and
 * VC-Attention summary, Key Contribution 1 (per-block V mean).
 *
 *   k, v          bf16 [B,S,H,D] (layout VS_LAYOUT_BSHD) or [B,H,S,D]
 *                 (VS_LAYOUT_BHSD), e.g. the permuted K', V'.  v may be
 *                 NULL when both V outputs are NULL (then V is not read).
 *   k_mean        out f32 [B,H,D]: mean of K over the S tokens, or NULL.
 *   v_block_mean  out f32 [B,H,nb,D]: mean of V over each block's valid
 *                 tokens, or NULL.
 *   v_seq_mean    out f32 [B,H,D]: mean of V over the S tokens, or NULL.
 *   ws, ws_bytes  workspace of at least vs_smooth_stats_workspace_bytes().
 * Means are exact: float64 sums of the bf16 values, one float64 division,
 * one rounding to float32.  At least one output must be non-NULL.
 */
int vs_smooth_stats_workspace_bytes(int B, int S, int H, int D, size_t* bytes);
int vs_smooth_stats(const uint16_t* k, const uint16_t* v, int B, int S, int H,
                    int D, int layout, float* k_mean, float* v_block_mean,
                    float* v_seq_mean, void* ws, size_t ws_bytes, void* stream);

/*
 * vs_smooth_stats_ex -- vs_smooth_stats with the rotary embedding of K
 * fused in: k_mean is the mean of the rotated keys, and the rotated K is
 * never written.  Source: VC-Attention summary, Key Contribution 3 (the
 * fused prologue absorbs the rotary embedding together with the means).
 *
 *   rope_cos, rope_sin  f32 [S, D/2] each, or both NULL (then this is
 *                 vs_smooth_stats): row t holds the cosines and sines of
 *                 token t's D/2 rotation angles; channel pair
 *                 (2i, 2i+1) of token t turns by angle (t, i):
 *                   y0 = a cos - b sin,  y1 = a sin + b cos,
 *                 each product and difference / sum rounded to float32 in
 *                 that order (no fused multiply-add), the result rounded
 *                 to bf16 (nearest even) -- the rotation a model applies to
 *                 its bf16 activations.  Rows are indexed by the token's
 *                 position in k (not permuted here).  One table serves all
 *                 B and H.  Only one of the two NULL: VS_ERR_INVALID_ARG.
 *   all other arguments as vs_smooth_stats.  V is not rotated.
 */
int vs_smooth_stats_ex(const uint16_t* k, const uint16_t* v, int B, int S,
                       int H, int D, int layout, const float* rope_cos,
                       const float* rope_sin, float* k_mean,
                       float* v_block_mean, float* v_seq_mean, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * vs_smooth_stats_noalloc -- vs_smooth_stats for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  It calls no
 * allocating routine; its workspace is a statically sized array in the
 * library's device code, one per GPU, kept until the process ends.
 *
 *   arguments     as vs_smooth_stats, without ws / ws_bytes.
 *   limit         vs_smooth_stats_workspace_bytes(B, S, H, D) must not
 *                 exceed VS_NOALLOC_STATS_SCRATCH_BYTES (32 MiB: e.g.
 *                 B*H = 56 heads of S = 32626 at D = 128); larger problems
 *                 return VS_ERR_WORKSPACE before anything is launched.
 *   device        the current HIP device (the stream's); the array's
 *                 address on it is looked up on the first call there.
 *                 VS_ERR_HIP if that lookup fails.
 * Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (different streams or host threads without ordering) race and give
 * undefined results.  The kernels write every workspace entry they later
 * read, so no call depends on what an earlier one left there.  Results are
 * bit-identical to vs_smooth_stats.
 */
#define VS_NOALLOC_STATS_SCRATCH_BYTES (32u << 20)
int vs_smooth_stats_noalloc(const uint16_t* k, const uint16_t* v, int B, int S,
                            int H, int D, int layout, float* k_mean,
                            float* v_block_mean, float* v_seq_mean,
                            void* stream);

/*
 * vs_quantize_residual -- per-128-token-block E4M3 quantizers for Q, centred
 * K and residual V.  Source: TeleFuser PR #40, "Changes" (centre K in FP32
 * before E4M3) and VC-Attention summary, Key Contribution 1
 * (each hardware block subtracts its mean and quantizes only the residual);
 * scale set by the block's largest entry (VC-Attention abstract).
 *
 *   q             bf16 [B,S,H,D] (always BSHD).
 *   k, v          bf16 in `kv_layout` (VS_LAYOUT_BSHD or VS_LAYOUT_BHSD).
 *   softmax_scale the attention scale (1/sqrt(D) is the usual value): Q is
 *                 multiplied by c = softmax_scale * log2(e) in FP32 before
 *                 its quantization, and q_mu uses the same c.
 *   k_mean        f32 [B,H,D] from vs_smooth_stats, or NULL: no K centring.
 *   v_mean        f32 [B,H,nb,D] (VS_VMEAN_BLOCK) or [B,H,D] (VS_VMEAN_SEQ),
 *                 read; or out f32 [B,H,nb,D] (VS_VMEAN_BLOCK_OUT): each
 *                 block's mean over its valid tokens, formed here from the
 *                 same V the block quantizer reads, exactly as
 *                 vs_smooth_stats forms v_block_mean (bit-identical), which
 *                 saves that call's pass over V; NULL with VS_VMEAN_NONE.
 *   q8, k8        out u8 [B,H,S_pad,D]: E4M3 codes, row per token.
 *   v8            out u8 [B,H,nb,D,128]: E4M3 codes of the residual, per
 *                 block one row of 128 tokens per channel.  Within a block
 *                 the token of row position p (0..127) is
 *                   t(p) = 64*(p/64) + 32*((p%32)/16) + 8*((p%16)/4)
 *                          + 4*((p%64)/32) + p%4
 *                 (the order the attention kernel's FP8 MFMA consumes).
 *   q_scale, k_scale, v_scale  out f32 [B,H,nb]: dequantization scales,
 *                 each a power of two.
 *   q_mu          out f32 [B,H,S]: c * (q . k_mean) from the bf16 q;
 *                 required iff k_mean != NULL.
 * Per block: x = float32 input (Q times c, K minus its mean, V minus its
 * mean: one float32 operation), amax = max |x| over the valid tokens and D
 * channels, scale = 2^e with e the smallest integer >= -126 such that
 * amax <= 448 * 2^e (e = 0 when amax == 0), codes = E4M3(x * 2^-e), round to
 * nearest even: an E8M0 block scale that the FP8 matrix core applies exactly
 * in QK^T and PV.
 */
int vs_quantize_residual(const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, int kv_layout, int B, int S, int H,
                         int D, float softmax_scale, const float* k_mean,
                         float* v_mean, int vmean_mode, uint8_t* q8,
                         float* q_scale, uint8_t* k8, float* k_scale,
                         uint8_t* v8, float* v_scale, float* q_mu,
                         void* stream);

/*
 * vs_quantize_residual_perm -- vs_quantize_residual with the grouping's
 * gather fused in: the permuted K and V are never written.  Source:
 * VC-Attention summary, Key Contribution 3 (gather, means and quantizers in
 * one fused prologue) and Key Contribution 1 (keys and values permuted
 * together by the sorted cluster labels).
 *
 *   q, k, v       bf16 [B,S,H,D] (BSHD), the caller's tensors.
 *   perm          i32 [B,H,S] (vs_kmeans_permute's perm): position i of
 *                 head h takes K and V of token perm[b,h,i].  Must be a
 *                 permutation of 0..S-1 per head for the result to mean
 *                 anything; entries outside [0, S) are clamped (never read
 *                 out of bounds).  NULL is VS_ERR_INVALID_ARG.
 *   all other arguments as vs_quantize_residual (v_mean holds the block
 *   means of the permuted V; k_mean is permutation-invariant and may come
 *   from vs_smooth_stats over the unpermuted K).
 * Outputs are bit-identical to vs_quantize_residual on K[perm], V[perm] in
 * VS_LAYOUT_BHSD.  Q is not permuted.
 */
int vs_quantize_residual_perm(const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const int32_t* perm, int B,
                              int S, int H, int D, float softmax_scale,
                              const float* k_mean, float* v_mean,
                              int vmean_mode, uint8_t* q8, float* q_scale,
                              uint8_t* k8, float* k_scale, uint8_t* v8,
                              float* v_scale, float* q_mu, void* stream);

/*
 * vs_quantize_residual_ex -- the quantizers with every option: the rotary
 * embedding of Q and K, the grouping permutation (as
 * vs_quantize_residual_perm) and the QK Hadamard rotation.  Source:
 * VC-Attention summary, Key Contribution 3 (the fused prologue holds the
 * rotary embedding, the gather by the permutation and a QK Hadamard
 * rotation, so rotated and permuted tensors never reach HBM) and Main
 * Findings (rotating Q and K moves PSNR by at most 0.1-0.3 dB).
 *
 *   rope_cos, rope_sin  f32 [S, D/2] each, or both NULL: Q and K rows are
 *                 first rotated exactly as vs_smooth_stats_ex rotates K
 *                 (bf16 result), and everything below -- q_mu, the K
 *                 centring, the Hadamard rotation, the block scales --
 *                 works on the rotated rows.  K's table row is the source
 *                 token: position i of a permuted head uses row perm[i].
 *                 k_mean must then come from vs_smooth_stats_ex with the
 *                 same tables.  Only one of the two NULL:
 *                 VS_ERR_INVALID_ARG.
 *
 *   kv_layout     as vs_quantize_residual; must be VS_LAYOUT_BSHD when
 *                 perm != NULL.
 *   perm          i32 [B,H,S] or NULL (as vs_quantize_residual_perm).
 *   flags         0 or VS_QK_HADAMARD: each row of Q and of the centred K
 *                 is multiplied by the Sylvester Hadamard matrix H_D
 *                 (entries +-1) in float32 -- butterflies (a+b, a-b) over
 *                 channel bit 0, 1, ..., log2(D)-1 in that order, one
 *                 rounding each -- before quantization, and Q's factor
 *                 c = softmax_scale * log2(e) becomes c / D (exact), so the
 *                 codes' product is the same score: (Q H / D)(K H)^T = Q K^T.
 *                 q_mu and lse2 are unchanged (original logits).  V is not
 *                 rotated.  vs_fp8_attn_fwd takes the outputs as they are.
 *                 | VS_V_MXFP4: the V residual as OCP MX FP4 -- E2M1 codes
 *                 (0, 0.5, 1, 1.5, 2, 3, 4, 6, signed; nearest, ties to the
 *                 even code) with one E8M0 scale 2^e per channel and 32
 *                 consecutive tokens of a block (group g = tokens
 *                 32g..32g+31), e the smallest integer >= -127 with
 *                 amax <= 6 * 2^e (0 for an all-zero group).  v8 is then
 *                 u8 [B,H,nb,D,64]: channel row d of block j holds group g in
 *                 bytes 16g..16g+15, nibble q (low nibble first) = token
 *                 32g + 8*((q%16)/4) + 4*(q/16) + q%4 (the k order of
 *                 gfx950's 4-bit matrix-core A operand); v_scale is u8
 *                 [B,H,nb,D,4], byte g = e + 127.  Source: VC-Attention
 *                 summary (V-Smooth with 4-bit operands; the pages' NVFP4
 *                 read as gfx950's MX FP4).
 *                 | VS_P_MXFP4 (E4M3 V only): position p of each v8
 *                 channel row holds token p with bits 4 and 5 of p swapped
 *                 (tokens 0-15, 32-47, 16-31, 48-63 of each half-tile): the
 *                 k order in which vs_fp8_attn_fwd's 4-bit probability tile
 *                 meets V.
 *                 | VS_BF16_MMA: q8 and k8 receive, instead of the E4M3
 *                 bytes, each code's value times its block scale as bf16
 *                 (u16 [B,H,S_pad,D], twice the bytes): the same quantized
 *                 operands, for vs_fp8_attn_fwd's VS_BF16_MMA form.  Exact
 *                 while the smallest code times the scale is a bf16 number
 *                 (block scale >= 2^-124, i.e. block amax above ~1e-35).
 *                 q_scale and k_scale are still written.
 *   all other arguments as vs_quantize_residual.
 * With perm, rope_cos, rope_sin == NULL and flags == 0 this is
 * vs_quantize_residual.
 */
int vs_quantize_residual_ex(const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, int kv_layout,
                            const int32_t* perm, unsigned flags, int B, int S,
                            int H, int D, float softmax_scale,
                            const float* rope_cos, const float* rope_sin,
                            const float* k_mean, float* v_mean,
                            int vmean_mode, uint8_t* q8, float* q_scale,
                            uint8_t* k8, float* k_scale, uint8_t* v8,
                            float* v_scale, float* q_mu, void* stream);

/*
 * vs_fp8_attn_fwd -- FP8 attention forward with the in-recurrence V-mean
 * restore.  Source: VC-Attention summary, Key Contributions 1-2 and
 * "Methodology in Plain English"; abstract (low-bit matrix cores for QK^T
 * and PV, FP32 softmax between them); FastVideo PR #2048, "Test Results"
 * (output and log2-LSE).
 *
 *   q8, q_scale, k8, k_scale, v8, v_scale  from vs_quantize_residual (the
 *                 power-of-two block scales; q8 encodes c * Q, so the
 *                 product of the codes and scales is the score in log2
 *                 units -- the softmax scale was applied there).
 *   v_mean        the same mean buffer given to vs_quantize_residual
 *                 ([B,H,nb,D] for VS_VMEAN_BLOCK, [B,H,D] for VS_VMEAN_SEQ),
 *                 NULL with VS_VMEAN_NONE.
 *   q_mu          f32 [B,H,S] or NULL (then 0).
 *   flags         any of VS_EXPCAST, VS_V_MXFP4 (v8 and v_scale in the
 *                 MXFP4 layout of vs_quantize_residual_ex; the PV product
 *                 then takes 4-bit V codes with their per-lane group
 *                 scales), VS_OUT_BF16, VS_BF16_MMA (q8 and k8 are the bf16
 *                 operands vs_quantize_residual_ex writes with that flag;
 *                 q_scale and k_scale are then not read and may be NULL),
 *                 VS_P_MXFP4 (the 4-bit probability tile: per query row,
 *                 each group of 32 consecutive keys of a 128-key tile gets
 *                 the E8M0 exponent e of its largest 2^8 p -- the smallest
 *                 e >= -127 with max <= 6 * 2^e -- and E2M1 codes of
 *                 2^8 p 2^-e, nearest with ties to the even code, which
 *                 the FP8/FP4 matrix core multiplies with the E4M3 V codes
 *                 (v8 in the order vs_quantize_residual_ex writes with
 *                 VS_P_MXFP4); l still sums the float32 p.  Not with
 *                 VS_EXPCAST, VS_V_MXFP4 or VS_BF16_MMA: VS_ERR_INVALID_ARG.
 *                 Source: VC-Attention summary, Future Directions (a 4-bit
 *                 probability with its per-block scale on the softmax
 *                 path), read as gfx950's MXFP4).
 *   out           out f32 [B,S,H,D] (bf16 [B,S,H,D] with VS_OUT_BF16: the
 *                 float32 result rounded to nearest even): attention output
 *                 in the caller's query order.
 *   lse2          out f32 [B,H,S]: log2 sum_t 2^(c * score_t) of the
 *                 (uncentred) logits: m + log2(l) + q_mu.
 * Non-causal full attention; keys past S are masked.  Per 128-key tile, in
 * log2 units: s = the score (the codes' dot product times the block
 * scales), the running row maximum m' = max(m, max_t s_t);
 * p = 2^(s - m'), P = E4M3(p * 2^8) (float32 exp2, round to nearest even),
 * or with VS_EXPCAST the code rint(8 (s - m') + K0),
 * K0 = 120 - 4 (log2(1.5) - 1/2), codes < 8 -> 0; the tile row sum l_tile
 * is the sum of the float32 p (with VS_EXPCAST of the decoded codes times
 * 2^-8); l and O are rescaled by 2^(m - m') where the max grows, O
 * accumulates s_V * 2^-8 P.R~ + l_tile * mu_block, and O = acc / l.
 * QK^T runs on the FP8 matrix core from the E4M3 codes, which sums each
 * group of 8 products after truncating the small ones to about 13 bits
 * below the group's largest (scores then differ from the exact dot
 * product by ~1e-5 of their magnitude, which moves a few E4M3 probability
 * codes per thousand across a rounding boundary); with VS_BF16_MMA on the
 * bf16 matrix core, whose scores are float32-accurate.
 * Block scales must be powers of two (as vs_quantize_residual writes them).
 * S * D (rounded up to whole blocks) must stay below 2^31 per head
 * (VS_ERR_UNSUPPORTED otherwise).
 */
int vs_fp8_attn_fwd(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                    const float* k_scale, const uint8_t* v8,
                    const float* v_scale, const float* v_mean, int vmean_mode,
                    const float* q_mu, int B, int S, int H, int D,
                    unsigned flags, void* out, float* lse2, void* stream);

/*
 * vs_fp8_attn_fwd_pcodes -- vs_fp8_attn_fwd that also writes the E4M3
 * probability codes it multiplies V with, for every row_stride-th query
 * row: a diagnostic that lets a test count, code by code, where the
 * kernel's probabilities differ from a reference's.  Same source as
 * vs_fp8_attn_fwd.
 *
 *   p_codes       out u8 [B,H,ceil(S/row_stride),S_pad]: row r holds query
 *                 r * row_stride; column t the code of key t (in the order
 *                 K was given, i.e. permuted order after a grouping), each
 *                 relative to the running max of t's tile (2^8 p, or the
 *                 ExpCast code).  Padding columns of the last tile hold 0.
 *                 Must not be NULL for a non-empty problem.
 *   row_stride    >= 1 (VS_ERR_INVALID_ARG otherwise).
 *   all other arguments as vs_fp8_attn_fwd (out and lse2 are written as
 *   there); VS_V_MXFP4 and VS_P_MXFP4 are VS_ERR_UNSUPPORTED here.
 */
int vs_fp8_attn_fwd_pcodes(const uint8_t* q8, const float* q_scale,
                           const uint8_t* k8, const float* k_scale,
                           const uint8_t* v8, const float* v_scale,
                           const float* v_mean, int vmean_mode,
                           const float* q_mu, int B, int S, int H, int D,
                           unsigned flags, void* out, float* lse2,
                           uint8_t* p_codes, int row_stride, void* stream);

/*
 * vs_kmeans_permute -- V-Smooth grouping: integer k-means over each head's V
 * tokens, stable sort of the labels, K and V gathered by the permutation.
 * Source: VC-Attention summary, Key Contribution 1 and "Methodology in
 * Plain English" (lightweight online k-means on V; keys and values permuted
 * together by the sorted labels; attention unchanged).
 *
 *   k, v          bf16 [B,S,H,D] (BSHD).
 *   k_clusters    1..256;  iters >= 1 Lloyd passes.
 *   labels        out i32 [B,H,S]: cluster of each token (last assignment).
 *   perm          out i32 [B,H,S]: perm[i] = source token of position i,
 *                 ascending label, original order within a label.
 *   k_perm, v_perm out bf16 [B,H,S,D] (BHSD): K[perm], V[perm] per head;
 *                 both NULL: no gather (labels and perm only, for
 *                 vs_quantize_residual_perm, which reads K and V through
 *                 perm itself).  Exactly one NULL is VS_ERR_INVALID_ARG.
 *   ws, ws_bytes  workspace of at least vs_kmeans_workspace_bytes().
 * Integer definition (bit-exact on any implementation): codes =
 * rint(V * 2^-e) with 2^e the smallest power of two such that
 * max|V| <= 127 * 2^e (per head); init centroid j = codes of token
 * floor(j*S/k); assign argmin_j |c_j|^2 - 2 v.c_j (ties: lowest j);
 * update c_j = round-half-away(sum/count), empty clusters keep theirs.
 */
int vs_kmeans_workspace_bytes(int B, int S, int H, int D, int k_clusters,
                              size_t* bytes);
int vs_kmeans_permute(const uint16_t* k, const uint16_t* v, int B, int S,
                      int H, int D, int k_clusters, int iters, int32_t* labels,
                      int32_t* perm, uint16_t* k_perm, uint16_t* v_perm,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * vs_cube_permutation -- static spatiotemporal-cube grouping of a video
 * token grid, a zero-cost alternative to k-means grouping.  Source:
 * VC-Attention summary, Main Findings (block demeaning in sequence order,
 * under a static spatiotemporal cube, after k-means grouping) and Key
 * Contribution 3 (a grouping permutation reused across calls).
 *
 * HOST function: no GPU work, `perm` is host memory.
 *   S             tokens; the grid T x Hg x W (raster order, token s at
 *                 (t, y, x) with s = (t*Hg + y)*W + x) must hold them:
 *                 T*Hg*W >= S; positions s >= S are empty.
 *   ct, ch, cw    cube extent along t, y, x (>= 1).
 *   perm          out i32 [S]: perm[i] = token at position i: cubes in
 *                 raster order of the cube grid (the last cube along an
 *                 axis may be shorter), tokens of a cube in raster order.
 * To use it, broadcast it to [B,H,S] and pass it to
 * vs_quantize_residual_perm (K and V permuted together, Q not).
 * VS_ERR_INVALID_ARG for non-positive sizes, a grid smaller than S, or a
 * NULL perm with S > 0.
 */
int vs_cube_permutation(int S, int T, int Hg, int W, int ct, int ch, int cw,
                        int32_t* perm);

#ifdef __cplusplus
}
#endif

#endif /* VSMOOTH_H */
