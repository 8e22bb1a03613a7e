// Launchers shared between the host API (h3attn_api.cpp) and the kernels.
// Arguments reaching these have already been validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3 {

constexpr int kHeadDim = 128;

hipError_t launch_qknorm_rope(uint16_t *q, uint16_t *k, const float *gamma_q,
                              const float *gamma_k, const float *cos_t,
                              const float *sin_t, int H, int L, float eps,
                              hipStream_t stream);

hipError_t launch_rope_tables(const int *positions, int L, int half,
                              double theta, float *cos_t, float *sin_t,
                              hipStream_t stream);

// Number of 256-row work units (head, query tile) for H heads of L tokens.
int64_t attention_grid(int H, int L);

hipError_t launch_attention(const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, uint16_t *out, int H, int L,
                            float scale, hipStream_t stream);

// V given transposed: element (h, j, d) at (h*D + d)*ldv + j.
hipError_t launch_attention_vt(const uint16_t *q, const uint16_t *k, const uint16_t *vt, uint16_t *out, int H,
                               int L, int ldv, float scale, hipStream_t stream);

hipError_t launch_attention_lse(const uint16_t *q, const uint16_t *k, const uint16_t *v, float *out, float *lse,
                                int H, int Lq, int Lk, long long kv_stride, float scale, hipStream_t stream);

hipError_t launch_attention_merge(const float *outs, const float *lses, int P, uint16_t *out, float *lse_out,
                                  int H, int L, hipStream_t stream);

// Number of workgroups h3_qkv_proj_qknorm_rope launches.  The projection
// launchers write v as [H][L][128] when ldv == 0, else as [H][128][ldv].
int64_t qkv_proj_grid(int H, int L);

hipError_t launch_qkv_proj_qknorm_rope(const uint16_t *x, const uint16_t *wq, const uint16_t *wk,
                                       const uint16_t *wv, const float *gamma_q, const float *gamma_k,
                                       const float *cos_t, const float *sin_t, uint16_t *q, uint16_t *k,
                                       uint16_t *v, int H, int L, int C, float eps, int ldv, hipStream_t stream);

hipError_t launch_qkv_proj_fp8_qknorm_rope(const uint8_t *x, const float *x_scale, const uint8_t *wq,
                                           const uint8_t *wk, const uint8_t *wv, const float *w_scale,
                                           const float *gamma_q, const float *gamma_k, const float *cos_t,
                                           const float *sin_t, uint16_t *q, uint16_t *k, uint16_t *v, int H, int L,
                                           int C, float eps, int ldv, hipStream_t stream);

}  // namespace h3
