/*
 * h3attn.h -- C ABI of the MI355X (gfx950) library for one Ulysses rank's
 * exact attention in MiniMax-H3, with its QK-RMSNorm + RoPE prologue.
 *
 * Where the operations come from:
 *   - "buqi-minimax-h3-multigpu" (README), How it works: every rank computes
 *     exact full attention over the full packed sequence for 56/world_size
 *     heads; On accuracy: nothing is approximated, masked or cached.
 *   - "Tensor parallelism for MiniMax-H3" (diffusers PR), PR description:
 *     QK-norms are head_dim-shaped and applied after the head split; the
 *     rotary embedding uses real sin/cos that broadcast over the head axis.
 *     whn09's comment (Bug: non-persistent buffers): rotary angles come from
 *     inv_freq and position ids.  whn09's Neuron FYI: the attention is packed
 *     full self-attention with no mask, and the real sequence length need not
 *     be a multiple of any tile size.
 *
 * Conventions for every call:
 *   - Tensors are row-major with batch 1: q, k, v, out are bf16 [H][L][D]
 *     (element (h, i, d) at offset (h*L + i)*D + d).  D must be 128 (MiniMax-
 *     H3's head_dim: inner width 7168 over 56 heads).
 *   - Pointers are device pointers on the current HIP device, owned by the
 *     caller.  The library allocates nothing and keeps no mutable state, so
 *     calls are thread-safe.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work; a return of H3_OK means "validated and launched".  Faults
 *     inside a kernel surface at the caller's next synchronisation.
 *   - Arguments are validated before anything is launched.  On error the call
 *     returns a negative h3_status, launches nothing, writes nothing and
 *     prints nothing.
 *   - Head splits: heads are independent, so a caller may pass pointers offset
 *     by h0*L*D with a smaller H.  Per-head results are bit-identical for any
 *     split and across repeated calls.
 */
#ifndef H3ATTN_H
#define H3ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

#define H3ATTN_ABI_VERSION 1
#define H3ATTN_HEAD_DIM 128
/* Longest sequence h3_attention takes: one head's K or V must stay below 2 GiB. */
#define H3ATTN_MAX_ATTENTION_L (1 << 23)

typedef enum {
  H3_OK = 0,
  H3_ERR_NULL = -1,        /* a required pointer is NULL                          */
  H3_ERR_SHAPE = -2,       /* H < 1, L < 1, a bad hidden size, or an overflow     */
  H3_ERR_UNSUPPORTED = -3, /* D != 128                                            */
  H3_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned             */
  H3_ERR_ALIAS = -5,       /* out overlaps q, k or v; q overlaps k; cos overlaps sin */
  H3_ERR_VALUE = -6,       /* eps <= 0 or not finite; scale <= 0, not finite, or  */
                           /* scale*log2(e) not finite; theta <= 1 or not finite  */
  H3_ERR_LAUNCH = -7       /* the HIP runtime refused the launch                  */
} h3_status;

/*
 * QK-RMSNorm followed by RoPE, applied to q and to k in place.
 *
 * For every head h and token i, with x = q[h][i][:] (gamma = gamma_q) and
 * again with x = k[h][i][:] (gamma = gamma_k):
 *   r     = 1 / sqrt(mean_d(x_d^2) + eps)
 *   y_d   = x_d * r * gamma_d
 *   x'_2j   = y_2j * cos[i][j] - y_2j+1 * sin[i][j]      j = 0 .. D/2-1
 *   x'_2j+1 = y_2j * sin[i][j] + y_2j+1 * cos[i][j]
 * computed in fp32 and rounded once to bf16 (round to nearest even), written
 * back over x.  The norm is the head_dim-shaped QK-norm after the head split;
 * the tables broadcast over heads (see the passages above).
 *
 *   q, k          bf16 [H][L][D], read and overwritten.  Must not overlap.
 *                 Finite values whose sum of squares per token stays finite
 *                 in fp32 (every |x_d| below about 2^63); larger rows are
 *                 out of contract.
 *   gamma_q/_k    fp32 [D], shared by all heads.
 *   cos, sin      fp32 [L][D/2]: entry (i, j) is cos/sin of token i's rotary
 *                 angle for pair j (h3_rope_tables builds them).
 *   H, L, D       heads, tokens, head_dim (== 128).
 *   eps           > 0, added to the mean of squares inside the square root.
 * All pointers must be 16-byte aligned.
 */
int h3_qknorm_rope(void *q, void *k, const float *gamma_q, const float *gamma_k,
                   const float *cos, const float *sin, int H, int L, int D,
                   float eps, void *stream);

/*
 * Exact, unmasked, non-causal attention per head:
 *   out[h][i][:] = sum_j softmax_j(scale * <q[h][i], k[h][j]>) * v[h][j][:]
 * over all L keys of head h.  This is what each Ulysses rank computes for its
 * 56/world_size heads over the whole packed sequence ("buqi-minimax-h3-
 * multigpu", How it works), exactly, with nothing approximated or masked
 * (the same README, On accuracy); the packed video+audio sequence takes no
 * mask and its real lengths are not tile multiples ("Tensor parallelism for
 * MiniMax-H3", whn09's FYI for anyone else on Neuron eager).
 * bf16 inputs, bf16 MFMA products with fp32 accumulation, online softmax in
 * fp32, output rounded once to bf16.  Any 1 <= L <= H3ATTN_MAX_ATTENTION_L is
 * accepted; a partial last tile is predicated, never padded.
 *
 *   q, k, v       bf16 [H][L][D], read only; finite values.
 *   out           bf16 [H][L][D], written; must not overlap q, k or v.
 *   scale         > 0 and finite, with scale * log2(e) finite in fp32
 *                 (H3_ERR_VALUE otherwise); MiniMax-H3 uses 1/sqrt(128).  The
 *                 caller keeps every scale * <q, k> finite in fp32.
 * All tensor pointers must be 16-byte aligned.
 */
int h3_attention(const void *q, const void *k, const void *v, void *out,
                 int H, int L, int D, float scale, void *stream);

/*
 * h3_attention with V given transposed: the same result, bit for bit, as
 * h3_attention on v[h][j][d] = vt[(h*D + d)*ldv + j].  Keys are contiguous in
 * this layout, so the kernel reads V tiles as plain 16-byte rows instead of
 * transposing them on the LDS read, which makes the call a few per cent
 * faster.  The layout is the one h3_qkv_proj_qknorm_rope_vt and its fp8 form
 * write.
 *
 *   q, k          bf16 [H][L][D], read only.
 *   vt            bf16 [H][D][ldv], read only: row (h, d) holds v[h][0..L-1][d]
 *                 in columns 0..L-1.  Columns from L up to the next multiple
 *                 of 8 are read and weighted by exact zeros, so they must be
 *                 finite (the projection writes zeros there); later columns are
 *                 never read.
 *   ldv           L <= ldv <= H3ATTN_MAX_ATTENTION_L, a multiple of 8
 *                 (H3_ERR_ALIGN otherwise).
 *   out           bf16 [H][L][D], written; must not overlap q, k or vt.
 *   L, scale      as for h3_attention.
 * All tensor pointers must be 16-byte aligned.  A head split offsets vt by
 * h0*D*ldv.
 */
int h3_attention_vt(const void *q, const void *k, const void *vt, void *out,
                    int H, int L, int ldv, int D, float scale, void *stream);

/*
 * Partial attention over a range of keys, with its log-sum-exp: the building
 * block for splitting the keys of one head across launches or devices
 * (context/ring parallelism, which "Tensor parallelism for MiniMax-H3" names,
 * in whn09's comments, as the next axis past the head-count cap on Ulysses).
 * For every head h and query row i:
 *   out[h][i][:] = sum_j softmax_j(scale * <q[h][i], k_h[j]>) * v_h[j][:]
 *   lse[h][i]    = ln sum_j exp(scale * <q[h][i], k_h[j]>)
 * over the Lk keys j of this range only, with out kept in fp32 (normalised
 * within the range) so that h3_attention_merge can combine ranges exactly.
 *
 *   q             bf16 [H][Lq][D].
 *   k, v          bf16; element (h, j, d) at h*kv_head_stride + j*D + d,
 *                 j < Lk.  A key range [j0, j0+Lk) of a [H][L][D] tensor is
 *                 k + j0*D with kv_head_stride = L*D.
 *   out           fp32 [H][Lq][D], written.      lse  fp32 [H][Lq], written.
 *   Lq, Lk        1 .. H3ATTN_MAX_ATTENTION_L;  kv_head_stride >= Lk*D and a
 *                 multiple of 8 elements.
 *   scale         as for h3_attention.
 * q, k, v, out must be 16-byte aligned; out and lse must not overlap the
 * inputs or each other.  Bit-identical per head for any head split.
 */
int h3_attention_lse(const void *q, const void *k, const void *v, float *out, float *lse,
                     int H, int Lq, int Lk, long long kv_head_stride, int D, float scale,
                     void *stream);

/*
 * Combines P partial results over disjoint key ranges of the same queries:
 *   lse = ln sum_p exp(lse_p),   out = sum_p exp(lse_p - lse) * out_p,
 * with out rounded once to bf16 (a part with lse_p = -inf contributes 0).
 *
 *   outs          fp32 [P][H][L][D] (h3_attention_lse outputs, stacked).
 *   lses          fp32 [P][H][L].
 *   out           bf16 [H][L][D], written.
 *   lse_out       fp32 [H][L], written; may be NULL.
 * outs and out must be 16-byte aligned, lses and lse_out 4-byte aligned;
 * outputs must not overlap inputs.
 */
int h3_attention_merge(const float *outs, const float *lses, int P, void *out, float *lse_out,
                       int H, int L, int D, void *stream);

/*
 * Rotary tables for h3_qknorm_rope:
 *   inv_freq_j = theta^(-2j/D),  angle = positions[i] * inv_freq_j,
 *   cos[i][j] = cos(angle), sin[i][j] = sin(angle),   j = 0 .. D/2-1,
 * computed in fp64 and rounded once to fp32.  The angle is position times
 * inv_freq ("Tensor parallelism for MiniMax-H3", whn09's comment on the
 * rotary inv_freq buffer); theta = 10000 for MiniMax-H3's synthetic layout.
 *
 *   positions     int32 [L], device memory: the rotary position of each
 *                 packed token (e.g. video 0..Lv-1 then audio restarting at 0).
 *   cos, sin      fp32 [L][D/2], written; must not overlap.
 *   theta         > 1 and finite.
 * cos and sin must be 16-byte aligned; positions 4-byte aligned.
 */
int h3_rope_tables(const int *positions, int L, int D, double theta,
                   float *cos, float *sin, void *stream);

/*
 * The rank's row-sliced qkv projection with QK-RMSNorm + RoPE fused behind
 * it.  A rank that holds the whole modulated hidden state projects it through
 * only its own heads' rows of qkv_proj; slicing rows is exact because the
 * weight's scale is per-tensor ("buqi-minimax-h3-multigpu", How it works: the
 * all_gather form used at small world sizes; H3's hidden size is 5376).  For
 * every head h, token t and d < D, with f = h*D + d:
 *   q~[h][t][d] = sum_c x[t][c] * wq[f][c]    (k~ and v~ likewise)
 *   q = h3_qknorm_rope's transform of q~ with gamma_q, k likewise with
 *   gamma_k, v = v~, each rounded once to bf16.
 * Products are bf16 x bf16 on the matrix cores with fp32 accumulation; the
 * norm and rotation use the fp32 accumulators directly (no bf16 rounding
 * before the norm).  No bias.
 *
 *   x             bf16 [L][hidden], read only (token-major hidden state).
 *   wq, wk, wv    bf16 [H*D][hidden] each, read only: the rank's rows of the
 *                 q, k and v blocks of qkv_proj (nn.Linear layout), e.g.
 *                 pointer offsets into the full weight.
 *   gamma_q/_k    fp32 [D];  cos, sin  fp32 [L][D/2] (as for h3_qknorm_rope).
 *   q, k, v       bf16 [H][L][D], written: the layout h3_attention reads.
 *                 They must not overlap each other or any input.
 *   hidden        a positive multiple of 32, at most 2^20.
 *   eps           > 0 and finite.
 * All pointers must be 16-byte aligned.
 */
int h3_qkv_proj_qknorm_rope(const void *x, const void *wq, const void *wk, const void *wv,
                            const float *gamma_q, const float *gamma_k, const float *cos,
                            const float *sin, void *q, void *k, void *v, int H, int L,
                            int hidden, int D, float eps, void *stream);

/*
 * The fp8 form of h3_qkv_proj_qknorm_rope.  The checkpoint the page
 * recommends stores fp8 weights with one scale per tensor, and its
 * transformer GEMMs run in fp8 ("buqi-minimax-h3-multigpu", VRAM & resolution
 * guidance and How it works).  Both operands are OCP e4m3 codes (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits):
 *   q~[h][t][d] = x_scale * w_scale * sum_c x[t][c] * wq[h*D+d][c]
 * (k~, v~ likewise), then the same norm, rotation and bf16 rounding as the
 * bf16 form.  Products on the matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4
 * with unit block scales), fp32 accumulation; the scales multiply the fp32
 * accumulator before the norm.
 *
 *   x             e4m3 [L][hidden];   x_scale  fp32 scalar in device memory.
 *   wq, wk, wv    e4m3 [H*D][hidden]: row slices of one weight tensor;
 *                 w_scale  its fp32 scale, a scalar in device memory.
 *   the rest      as for h3_qkv_proj_qknorm_rope; hidden a positive multiple
 *                 of 64, at most 2^20.
 * x, w*, gamma, cos, sin, q, k, v must be 16-byte aligned, the scales 4-byte
 * aligned.  Scales are read on the device, so the call needs no host sync.
 */
int h3_qkv_proj_fp8_qknorm_rope(const void *x, const float *x_scale, const void *wq, const void *wk,
                                const void *wv, const float *w_scale, const float *gamma_q,
                                const float *gamma_k, const float *cos, const float *sin, void *q,
                                void *k, void *v, int H, int L, int hidden, int D, float eps,
                                void *stream);

/*
 * h3_qkv_proj_qknorm_rope and h3_qkv_proj_fp8_qknorm_rope with v written
 * transposed, in the layout h3_attention_vt reads.  q and k are as in those
 * calls; v goes to
 *   vt[(h*D + d)*ldv + t] = v[h][t][d]     t < L,
 * and the columns from L up to the next multiple of 8 are set to zero (their
 * token rows of x read as zeros); later columns are left untouched.
 *
 *   vt            bf16 [H][D][ldv], written; must not overlap q, k or any input.
 *   ldv           L <= ldv <= H3ATTN_MAX_ATTENTION_L, a multiple of 8
 *                 (H3_ERR_ALIGN otherwise).
 *   the rest      as for the call without _vt.
 */
int h3_qkv_proj_qknorm_rope_vt(const void *x, const void *wq, const void *wk, const void *wv,
                               const float *gamma_q, const float *gamma_k, const float *cos,
                               const float *sin, void *q, void *k, void *vt, int H, int L, int ldv,
                               int hidden, int D, float eps, void *stream);
int h3_qkv_proj_fp8_qknorm_rope_vt(const void *x, const float *x_scale, const void *wq, const void *wk,
                                   const void *wv, const float *w_scale, const float *gamma_q,
                                   const float *gamma_k, const float *cos, const float *sin, void *q,
                                   void *k, void *vt, int H, int L, int ldv, int hidden, int D, float eps,
                                   void *stream);

/* A static, human-readable name for a status code (never NULL). */
const char *h3_status_string(int status);

/* H3ATTN_ABI_VERSION of the built library. */
int h3_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* H3ATTN_H */
