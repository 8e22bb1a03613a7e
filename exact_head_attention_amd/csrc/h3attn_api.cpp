// Host side of the C ABI in include/h3attn.h: argument validation, then one
// launch on the caller's stream.  Validation runs before any HIP call, so the
// error paths need no GPU.
#include "h3attn.h"

#include <cmath>
#include <cstdint>

#include "h3attn_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) overlap.
bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a);
  const uintptr_t y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// H*L*D elements must be addressable with 64-bit offsets and the row count
// must stay below 2^31 (grid and row indices are 32-bit).
bool shape_ok(int H, int L) {
  if (H < 1 || L < 1) return false;
  const int64_t rows = static_cast<int64_t>(H) * L;
  return rows < (int64_t{1} << 31);
}

// The attention kernels work in base 2 with scale * log2(e) folded into one
// fp32 factor; a scale whose factor overflows fp32 is rejected.
bool scale_ok(float scale) {
  return scale > 0.0f && std::isfinite(scale) && std::isfinite(scale * 1.4426950408889634f);
}

}  // namespace

extern "C" {

int h3_abi_version(void) { return H3ATTN_ABI_VERSION; }

const char *h3_status_string(int status) {
  switch (status) {
    case H3_OK: return "ok";
    case H3_ERR_NULL: return "a required pointer is NULL";
    case H3_ERR_SHAPE: return "a size is out of range (H, L >= 1, H*L < 2^31, hidden a multiple of the step)";
    case H3_ERR_UNSUPPORTED: return "only head_dim D == 128 is supported";
    case H3_ERR_ALIGN: return "tensor pointers must be 16-byte aligned";
    case H3_ERR_ALIAS: return "output and input buffers overlap";
    case H3_ERR_VALUE: return "eps, scale or theta is out of range or not finite";
    case H3_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
    default: return "unknown h3attn status";
  }
}

int h3_qknorm_rope(void *q, void *k, const float *gamma_q, const float *gamma_k,
                   const float *cos, const float *sin, int H, int L, int D,
                   float eps, void *stream) {
  if (!q || !k || !gamma_q || !gamma_k || !cos || !sin) return H3_ERR_NULL;
  if (!shape_ok(H, L)) return H3_ERR_SHAPE;
  if (D != H3ATTN_HEAD_DIM) return H3_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(gamma_q) || !aligned16(gamma_k) ||
      !aligned16(cos) || !aligned16(sin))
    return H3_ERR_ALIGN;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return H3_ERR_VALUE;
  const uint64_t tensor_bytes = static_cast<uint64_t>(H) * L * D * 2;
  const uint64_t table_bytes = static_cast<uint64_t>(L) * (D / 2) * 4;
  if (overlaps(q, tensor_bytes, k, tensor_bytes)) return H3_ERR_ALIAS;
  if (overlaps(cos, table_bytes, q, tensor_bytes) || overlaps(cos, table_bytes, k, tensor_bytes) ||
      overlaps(sin, table_bytes, q, tensor_bytes) || overlaps(sin, table_bytes, k, tensor_bytes) ||
      overlaps(gamma_q, D * 4u, q, tensor_bytes) || overlaps(gamma_q, D * 4u, k, tensor_bytes) ||
      overlaps(gamma_k, D * 4u, q, tensor_bytes) || overlaps(gamma_k, D * 4u, k, tensor_bytes))
    return H3_ERR_ALIAS;
  hipError_t e = h3::launch_qknorm_rope(static_cast<uint16_t *>(q), static_cast<uint16_t *>(k),
                                        gamma_q, gamma_k, cos, sin, H, L, eps,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? H3_OK : H3_ERR_LAUNCH;
}

int h3_attention(const void *q, const void *k, const void *v, void *out,
                 int H, int L, int D, float scale, void *stream) {
  if (!q || !k || !v || !out) return H3_ERR_NULL;
  if (!shape_ok(H, L) || L > H3ATTN_MAX_ATTENTION_L || h3::attention_grid(H, L) >= (int64_t{1} << 31))
    return H3_ERR_SHAPE;
  if (D != H3ATTN_HEAD_DIM) return H3_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return H3_ERR_ALIGN;
  if (!scale_ok(scale)) return H3_ERR_VALUE;
  const uint64_t bytes = static_cast<uint64_t>(H) * L * D * 2;
  if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes))
    return H3_ERR_ALIAS;
  hipError_t e = h3::launch_attention(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                                      static_cast<const uint16_t *>(v), static_cast<uint16_t *>(out),
                                      H, L, scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? H3_OK : H3_ERR_LAUNCH;
}

int h3_attention_vt(const void *q, const void *k, const void *vt, void *out, int H, int L, int ldv, int D,
                    float scale, void *stream) {
  if (!q || !k || !vt || !out) return H3_ERR_NULL;
  if (!shape_ok(H, L) || L > H3ATTN_MAX_ATTENTION_L || h3::attention_grid(H, L) >= (int64_t{1} << 31) ||
      ldv < L || ldv > H3ATTN_MAX_ATTENTION_L)
    return H3_ERR_SHAPE;
  if (D != H3ATTN_HEAD_DIM) return H3_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(out) || (ldv % 8) != 0) return H3_ERR_ALIGN;
  if (!scale_ok(scale)) return H3_ERR_VALUE;
  const uint64_t bytes = static_cast<uint64_t>(H) * L * D * 2;
  const uint64_t vt_bytes = static_cast<uint64_t>(H) * D * ldv * 2;
  if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, vt, vt_bytes))
    return H3_ERR_ALIAS;
  hipError_t e = h3::launch_attention_vt(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                                         static_cast<const uint16_t *>(vt), static_cast<uint16_t *>(out), H, L, ldv,
                                         scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? H3_OK : H3_ERR_LAUNCH;
}

int h3_attention_lse(const void *q, const void *k, const void *v, float *out, float *lse, int H, int Lq,
                     int Lk, long long kv_head_stride, int D, float scale, void *stream) {
  if (!q || !k || !v || !out || !lse) return H3_ERR_NULL;
  if (!shape_ok(H, Lq) || Lk < 1 || Lq > H3ATTN_MAX_ATTENTION_L || Lk > H3ATTN_MAX_ATTENTION_L ||
      h3::attention_grid(H, Lq) >= (int64_t{1} << 31) || kv_head_stride < static_cast<long long>(Lk) * D ||
      kv_head_stride > (int64_t{1} << 40))
    return H3_ERR_SHAPE;
  if (D != H3ATTN_HEAD_DIM) return H3_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned4(lse) ||
      (kv_head_stride % 8) != 0)
    return H3_ERR_ALIGN;
  if (!scale_ok(scale)) return H3_ERR_VALUE;
  const uint64_t q_bytes = static_cast<uint64_t>(H) * Lq * D * 2;
  const uint64_t kv_bytes = (static_cast<uint64_t>(H - 1) * kv_head_stride + static_cast<uint64_t>(Lk) * D) * 2;
  const uint64_t out_bytes = static_cast<uint64_t>(H) * Lq * D * 4;
  const uint64_t lse_bytes = static_cast<uint64_t>(H) * Lq * 4;
  if (overlaps(out, out_bytes, q, q_bytes) || overlaps(out, out_bytes, k, kv_bytes) ||
      overlaps(out, out_bytes, v, kv_bytes) || overlaps(lse, lse_bytes, q, q_bytes) ||
      overlaps(lse, lse_bytes, k, kv_bytes) || overlaps(lse, lse_bytes, v, kv_bytes) ||
      overlaps(lse, lse_bytes, out, out_bytes))
    return H3_ERR_ALIAS;
  hipError_t e = h3::launch_attention_lse(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                                          static_cast<const uint16_t *>(v), out, lse, H, Lq, Lk, kv_head_stride,
                                          scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? H3_OK : H3_ERR_LAUNCH;
}

int h3_attention_merge(const float *outs, const float *lses, int P, void *out, float *lse_out, int H, int L,
                       int D, void *stream) {
  if (!outs || !lses || !out) return H3_ERR_NULL;
  if (P < 1 || !shape_ok(H, L) || static_cast<int64_t>(P) * H * L >= (int64_t{1} << 40)) return H3_ERR_SHAPE;
  if (D != H3ATTN_HEAD_DIM) return H3_ERR_UNSUPPORTED;
  if (!aligned16(outs) || !aligned4(lses) || !aligned16(out) || (lse_out && !aligned4(lse_out)))
    return H3_ERR_ALIGN;
  const uint64_t rows = static_cast<uint64_t>(H) * L;
  const uint64_t outs_bytes = static_cast<uint64_t>(P) * rows * D * 4;
  const uint64_t lses_bytes = static_cast<uint64_t>(P) * rows * 4;
  const uint64_t out_bytes = rows * D * 2;
  if (overlaps(out, out_bytes, outs, outs_bytes) || overlaps(out, out_bytes, lses, lses_bytes)) return H3_ERR_ALIAS;
  if (lse_out && (overlaps(lse_out, rows * 4, outs, outs_bytes) || overlaps(lse_out, rows * 4, lses, lses_bytes) ||
                  overlaps(lse_out, rows * 4, out, out_bytes)))
    return H3_ERR_ALIAS;
  hipError_t e = h3::launch_attention_merge(outs, lses, P, static_cast<uint16_t *>(out), lse_out, H, L,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? H3_OK : H3_ERR_LAUNCH;
}

int h3_rope_tables(const int *positions, int L, int D, double theta,
                   float *cos, float *sin, void *stream) {
  if (!positions || !cos || !sin) return H3_ERR_NULL;
  if (L < 1) return H3_ERR_SHAPE;
  if (D != H3ATTN_HEAD_DIM) return H3_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(positions) & 3u) != 0 || !aligned16(cos) || !aligned16(sin))
    return H3_ERR_ALIGN;
  if (!(theta > 1.0) || !std::isfinite(theta)) return H3_ERR_VALUE;
  const uint64_t table_bytes = static_cast<uint64_t>(L) * (D / 2) * 4;
  if (overlaps(cos, table_bytes, sin, table_bytes) ||
      overlaps(positions, static_cast<uint64_t>(L) * 4, cos, table_bytes) ||
      overlaps(positions, static_cast<uint64_t>(L) * 4, sin, table_bytes))
    return H3_ERR_ALIAS;
  if (static_cast<int64_t>(L) * (D / 2) >= (int64_t{1} << 31)) return H3_ERR_SHAPE;
  hipError_t e = h3::launch_rope_tables(positions, L, D / 2, theta, cos, sin,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? H3_OK : H3_ERR_LAUNCH;
}

// Shared checks of the projection entry points (scales = the fp8 form's two
// device scalars, else null; ldv = 0 for v as [H][L][D], else v's row length
// as [H][D][ldv]).
static int check_qkv_proj(const void *x, const void *wq, const void *wk, const void *wv, const float *x_scale,
                          const float *w_scale, bool fp8, const float *gamma_q, const float *gamma_k,
                          const float *cos, const float *sin, void *q, void *k, void *v, int H, int L,
                          int hidden, int D, float eps, int ldv) {
  if (!x || !wq || !wk || !wv || !gamma_q || !gamma_k || !cos || !sin || !q || !k || !v) return H3_ERR_NULL;
  if (fp8 && (!x_scale || !w_scale)) return H3_ERR_NULL;
  const int step = fp8 ? 64 : 32;   // hidden elements per 64 bytes: half of the kernel's 128-byte step
  if (!shape_ok(H, L) || hidden < step || hidden % step != 0 || hidden > (1 << 20) ||
      h3::qkv_proj_grid(H, L) >= (int64_t{1} << 31) || (ldv != 0 && (ldv < L || ldv > H3ATTN_MAX_ATTENTION_L)))
    return H3_ERR_SHAPE;
  if (D != H3ATTN_HEAD_DIM) return H3_ERR_UNSUPPORTED;
  const void *ptrs[] = {x, wq, wk, wv, gamma_q, gamma_k, cos, sin, q, k, v};
  for (const void *p : ptrs)
    if (!aligned16(p)) return H3_ERR_ALIGN;
  if (fp8 && (!aligned4(x_scale) || !aligned4(w_scale))) return H3_ERR_ALIGN;
  if (ldv % 8 != 0) return H3_ERR_ALIGN;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return H3_ERR_VALUE;
  const uint64_t elem = fp8 ? 1 : 2;
  const uint64_t x_bytes = static_cast<uint64_t>(L) * hidden * elem;
  const uint64_t w_bytes = static_cast<uint64_t>(H) * D * hidden * elem;
  const uint64_t t_bytes = static_cast<uint64_t>(H) * L * D * 2;
  const uint64_t tab_bytes = static_cast<uint64_t>(L) * (D / 2) * 4;
  const void *outs[] = {q, k, v};
  const uint64_t out_bytes[] = {t_bytes, t_bytes, ldv ? static_cast<uint64_t>(H) * D * ldv * 2 : t_bytes};
  const struct { const void *p; uint64_t n; } ins[] = {
      {x, x_bytes}, {wq, w_bytes}, {wk, w_bytes}, {wv, w_bytes}, {gamma_q, D * 4u}, {gamma_k, D * 4u},
      {cos, tab_bytes}, {sin, tab_bytes}, {x_scale, fp8 ? 4u : 0u}, {w_scale, fp8 ? 4u : 0u}};
  for (int i = 0; i < 3; ++i) {
    for (const auto &in : ins)
      if (in.p && overlaps(outs[i], out_bytes[i], in.p, in.n)) return H3_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return H3_ERR_ALIAS;
  }
  return H3_OK;
}

static int qkv_proj_bf16(const void *x, const void *wq, const void *wk, const void *wv, const float *gamma_q,
                         const float *gamma_k, const float *cos, const float *sin, void *q, void *k, void *v, int H,
                         int L, int ldv, int hidden, int D, float eps, void *stream) {
  const int st = check_qkv_proj(x, wq, wk, wv, nullptr, nullptr, false, gamma_q, gamma_k, cos, sin, q, k, v, H,
                                L, hidden, D, eps, ldv);
  if (st != H3_OK) return st;
  hipError_t e = h3::launch_qkv_proj_qknorm_rope(
      static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(wq), static_cast<const uint16_t *>(wk),
      static_cast<const uint16_t *>(wv), gamma_q, gamma_k, cos, sin, static_cast<uint16_t *>(q),
      static_cast<uint16_t *>(k), static_cast<uint16_t *>(v), H, L, hidden, eps, ldv,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? H3_OK : H3_ERR_LAUNCH;
}

static int qkv_proj_fp8(const void *x, const float *x_scale, const void *wq, const void *wk, const void *wv,
                        const float *w_scale, const float *gamma_q, const float *gamma_k, const float *cos,
                        const float *sin, void *q, void *k, void *v, int H, int L, int ldv, int hidden, int D,
                        float eps, void *stream) {
  const int st = check_qkv_proj(x, wq, wk, wv, x_scale, w_scale, true, gamma_q, gamma_k, cos, sin, q, k, v, H,
                                L, hidden, D, eps, ldv);
  if (st != H3_OK) return st;
  hipError_t e = h3::launch_qkv_proj_fp8_qknorm_rope(
      static_cast<const uint8_t *>(x), x_scale, static_cast<const uint8_t *>(wq),
      static_cast<const uint8_t *>(wk), static_cast<const uint8_t *>(wv), w_scale, gamma_q, gamma_k, cos, sin,
      static_cast<uint16_t *>(q), static_cast<uint16_t *>(k), static_cast<uint16_t *>(v), H, L, hidden, eps, ldv,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? H3_OK : H3_ERR_LAUNCH;
}

int h3_qkv_proj_qknorm_rope(const void *x, const void *wq, const void *wk, const void *wv,
                            const float *gamma_q, const float *gamma_k, const float *cos,
                            const float *sin, void *q, void *k, void *v, int H, int L,
                            int hidden, int D, float eps, void *stream) {
  return qkv_proj_bf16(x, wq, wk, wv, gamma_q, gamma_k, cos, sin, q, k, v, H, L, 0, hidden, D, eps, stream);
}

int h3_qkv_proj_qknorm_rope_vt(const void *x, const void *wq, const void *wk, const void *wv,
                               const float *gamma_q, const float *gamma_k, const float *cos,
                               const float *sin, void *q, void *k, void *vt, int H, int L, int ldv,
                               int hidden, int D, float eps, void *stream) {
  if (ldv < 1) return H3_ERR_SHAPE;
  return qkv_proj_bf16(x, wq, wk, wv, gamma_q, gamma_k, cos, sin, q, k, vt, H, L, ldv, hidden, D, eps, stream);
}

int h3_qkv_proj_fp8_qknorm_rope(const void *x, const float *x_scale, const void *wq, const void *wk,
                                const void *wv, const float *w_scale, const float *gamma_q,
                                const float *gamma_k, const float *cos, const float *sin, void *q,
                                void *k, void *v, int H, int L, int hidden, int D, float eps,
                                void *stream) {
  return qkv_proj_fp8(x, x_scale, wq, wk, wv, w_scale, gamma_q, gamma_k, cos, sin, q, k, v, H, L, 0, hidden, D, eps,
                      stream);
}

int h3_qkv_proj_fp8_qknorm_rope_vt(const void *x, const float *x_scale, const void *wq, const void *wk,
                                   const void *wv, const float *w_scale, const float *gamma_q,
                                   const float *gamma_k, const float *cos, const float *sin, void *q,
                                   void *k, void *vt, int H, int L, int ldv, int hidden, int D, float eps,
                                   void *stream) {
  if (ldv < 1) return H3_ERR_SHAPE;
  return qkv_proj_fp8(x, x_scale, wq, wk, wv, w_scale, gamma_q, gamma_k, cos, sin, q, k, vt, H, L, ldv, hidden, D,
                      eps, stream);
}

}  // extern "C"
