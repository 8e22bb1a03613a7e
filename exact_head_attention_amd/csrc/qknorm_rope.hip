// QK-RMSNorm + RoPE prologue and the rotary-table builder, for gfx950.
//
// The prologue is a streaming, HBM-bound kernel: every q and k row (128 bf16 =
// 256 B) is read once and written once, in place.  One 16-lane row of a wave
// owns one token: each lane holds 8 consecutive elements (one 16-byte load),
// i.e. four adjacent RoPE pairs, so the pair rotation is lane-local and only
// the sum of squares crosses lanes (a 16-lane DPP reduction).
//
// A workgroup is 16 tokens of one head.  Workgroups are numbered by token
// chunk (of at most 32768), then by head, then by token, so the whole chip streams
// through one head's share of q and k at a time: two long sequential streams,
// which DRAM serves better (45.5 us cold at H = 7, L = 32768, 5.5 TB/s) than
// every workgroup walking all H heads at once (50.4 us).  The cos/sin rows are
// re-read for every head; a chunk's rows fit the XCDs' L2, and a token block
// maps to the same XCD for every head, so HBM sees the tables about once
// (L = 37726: 51 us instead of 61 us; L = 131072: 168 us instead of 195 us).
// Non-temporal loads and stores measured best (plain ones: 52-53 us).
//
// Math follows "Tensor parallelism for MiniMax-H3", PR description (head_dim-
// shaped QK-norm after the head split; real cos/sin broadcast over heads):
// fp32 throughout, one round-to-nearest-even to bf16 at the store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3attn_internal.h"

namespace h3 {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// q and k rows are touched exactly once: stream them past the caches.
__device__ __forceinline__ uint4 load_stream(const uint16_t *p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)));
}
__device__ __forceinline__ void store_stream(uint16_t *p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(p));
}

constexpr int kTokensPerBlock = 16;   // 16 lanes per token

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest even) and pack them, lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = static_cast<__bf16>(lo);
  __bf16 b = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Sum over the 16 lanes of a DPP row, as a butterfly: lanes exchange with
// their partner at distance 1, 2 (quad_perm), then across the half-row
// (row_half_mirror) and across the row (row_mirror).  At every stage both
// partners add the same two values, and fp32 addition is commutative, so all
// 16 lanes end with the same bits: the whole token is normalised by one r.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));   // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));   // row_mirror
  return v;
}

// Normalise, scale by gamma and rotate one lane's 8 elements (4 pairs).
__device__ __forceinline__ uint4 norm_rope8(uint4 raw, const float g[8], const float c[4],
                                            const float s[4], float eps) {
  float x[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
  ss = row16_sum(ss);
  const float r = __builtin_amdgcn_rsqf(ss * (1.0f / kHeadDim) + eps);
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float y0 = x[2 * p] * r * g[2 * p];
    const float y1 = x[2 * p + 1] * r * g[2 * p + 1];
    const float o0 = y0 * c[p] - y1 * s[p];
    const float o1 = y0 * s[p] + y1 * c[p];
    w[p] = pack_bf16x2(o0, o1);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Token chunks: the grid walks chunk by chunk and, inside a chunk, head by
// head.  A chunk's cos/sin rows (up to 32768 x 512 B, 2 MB per XCD) stay in
// the XCDs' L2 while every head streams past them, and each chunk's block
// count per head is a multiple of the 8 XCDs, so a token block lands on the
// same XCD for every head.  A sequence is cut into ceil(L / 32768) chunks of
// equal size (rounded up to whole XCD rounds of blocks), so an odd length
// such as 37726 makes two chunks of about 18900 tokens rather than 32768
// plus a short tail.
constexpr int kMaxChunk = 32768;
constexpr int kXcds = 8;
constexpr int kChunkQuantum = kTokensPerBlock * kXcds;   // tokens per XCD round of blocks

__host__ __device__ inline int chunk_tokens(int L) {
  const int n = (L + kMaxChunk - 1) / kMaxChunk;
  const int c = (L + n - 1) / n;
  return (c + kChunkQuantum - 1) / kChunkQuantum * kChunkQuantum;
}

// Blocks per head for the last, partial chunk of rem tokens.
__host__ __device__ inline int tail_chunk_blocks(int rem) {
  return ((rem + kTokensPerBlock - 1) / kTokensPerBlock + kXcds - 1) / kXcds * kXcds;
}

__global__ __launch_bounds__(kTokensPerBlock * 16) void qknorm_rope_kernel(
    uint16_t *__restrict__ q, uint16_t *__restrict__ k, const float *__restrict__ gamma_q,
    const float *__restrict__ gamma_k, const float *__restrict__ cos_t,
    const float *__restrict__ sin_t, int H, int L, float eps) {
  const int chunk_len = chunk_tokens(L);
  const int chunk_blocks = chunk_len / kTokensPerBlock;
  const int full = L / chunk_len;
  const int full_blocks = full * H * chunk_blocks;
  int b = blockIdx.x, chunk, head, tb;
  if (b < full_blocks) {
    chunk = b / (H * chunk_blocks);
    b -= chunk * H * chunk_blocks;
    head = b / chunk_blocks;
    tb = b - head * chunk_blocks;
  } else {
    const int per_head = tail_chunk_blocks(L - full * chunk_len);
    b -= full_blocks;
    chunk = full;
    head = b / per_head;
    tb = b - head * per_head;
  }
  const int sub = threadIdx.x & 15;                       // lane within the 16-lane row
  const int tok = chunk * chunk_len + tb * kTokensPerBlock + (threadIdx.x >> 4);
  if (tok >= L) return;                                   // whole 16-lane rows exit together

  const size_t off = (static_cast<size_t>(head) * L + tok) * kHeadDim + 8 * sub;
  const uint4 rq = load_stream(q + off);
  const uint4 rk = load_stream(k + off);
  const float4 c4 = *reinterpret_cast<const float4 *>(cos_t + static_cast<size_t>(tok) * 64 + 4 * sub);
  const float4 s4 = *reinterpret_cast<const float4 *>(sin_t + static_cast<size_t>(tok) * 64 + 4 * sub);
  const float c[4] = {c4.x, c4.y, c4.z, c4.w};
  const float s[4] = {s4.x, s4.y, s4.z, s4.w};
  float gq[8], gk[8];
  {
    const float4 a = *reinterpret_cast<const float4 *>(gamma_q + 8 * sub);
    const float4 b = *reinterpret_cast<const float4 *>(gamma_q + 8 * sub + 4);
    const float4 e = *reinterpret_cast<const float4 *>(gamma_k + 8 * sub);
    const float4 f = *reinterpret_cast<const float4 *>(gamma_k + 8 * sub + 4);
    gq[0] = a.x; gq[1] = a.y; gq[2] = a.z; gq[3] = a.w; gq[4] = b.x; gq[5] = b.y; gq[6] = b.z; gq[7] = b.w;
    gk[0] = e.x; gk[1] = e.y; gk[2] = e.z; gk[3] = e.w; gk[4] = f.x; gk[5] = f.y; gk[6] = f.z; gk[7] = f.w;
  }
  store_stream(q + off, norm_rope8(rq, gq, c, s, eps));
  store_stream(k + off, norm_rope8(rk, gk, c, s, eps));
}

// cos/sin of positions[i] * theta^(-2j/D) in fp64, rounded once to fp32.
__global__ __launch_bounds__(256) void rope_tables_kernel(const int *__restrict__ positions, int L, int half,
                                                          double theta, float *__restrict__ cos_t,
                                                          float *__restrict__ sin_t) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= L * half) return;
  const int i = idx / half;
  const int j = idx - i * half;
  const double inv_freq = pow(theta, (-2.0 * j) / (2 * half));
  const double angle = static_cast<double>(positions[i]) * inv_freq;
  double sn, cs;
  sincos(angle, &sn, &cs);
  cos_t[idx] = static_cast<float>(cs);
  sin_t[idx] = static_cast<float>(sn);
}

}  // namespace

hipError_t launch_qknorm_rope(uint16_t *q, uint16_t *k, const float *gamma_q, const float *gamma_k,
                              const float *cos_t, const float *sin_t, int H, int L, float eps,
                              hipStream_t stream) {
  const int chunk_len = chunk_tokens(L);
  const int full = L / chunk_len, rem = L - full * chunk_len;
  // < 2^31: H*L < 2^31 is validated, and padding adds under 8 blocks per
  // head and chunk
  const int64_t blocks = static_cast<int64_t>(H) * (static_cast<int64_t>(full) * (chunk_len / kTokensPerBlock) +
                                                    (rem > 0 ? tail_chunk_blocks(rem) : 0));
  hipLaunchKernelGGL(qknorm_rope_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kTokensPerBlock * 16), 0, stream,
                     q, k, gamma_q, gamma_k, cos_t, sin_t, H, L, eps);
  return hipGetLastError();
}

hipError_t launch_rope_tables(const int *positions, int L, int half, double theta, float *cos_t,
                              float *sin_t, hipStream_t stream) {
  const int n = L * half;
  hipLaunchKernelGGL(rope_tables_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, positions, L, half,
                     theta, cos_t, sin_t);
  return hipGetLastError();
}

}  // namespace h3
