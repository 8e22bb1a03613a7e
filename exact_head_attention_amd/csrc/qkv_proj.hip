// Row-sliced qkv projection with QK-RMSNorm + RoPE in the epilogue, for gfx950.
//
// A rank that holds the whole (gathered) hidden state x [L][C] projects it
// through only its own heads' rows of qkv_proj: wq, wk, wv are [H*128][C]
// ("buqi-minimax-h3-multigpu", How it works: the all_gather form for small
// world sizes, where slicing rows of the weight is exact).  q and k then get
// the head_dim RMSNorm and the rotary embedding ("Tensor parallelism for
// MiniMax-H3", PR description), fused here into the GEMM epilogue so the
// projection never goes through HBM in between and is never rounded before
// the norm.  Outputs are [H][L][128] bf16, the layout the attention reads.
//
// Work decomposition
//   * Workgroup = (feature tile, token tile): two head slots (256 output
//     features; slot j of the 3H q, k, v heads) x 256 tokens; 4 waves, each
//     one head slot (128 features) x 128 tokens, with its 16 accumulator
//     tiles (256 registers) in AGPRs: one wave per SIMD.
//   * The product is computed transposed, C^T = W . X^T, with
//     v_mfma_f32_32x32x16_bf16: A = weight rows (features), B = hidden rows
//     (tokens).  Both operands are K-contiguous in memory, so every fragment
//     is one 16-byte LDS read.  The accumulator puts one token per lane
//     column and 16 features per lane, so a token's sum of squares over its
//     128 features is lane-local plus one lane-half exchange, and each RoPE
//     pair (2j, 2j+1) sits in one lane.
//   * The hidden dimension streams in steps of 128 bytes per row (64 bf16)
//     or 64 bytes (64 fp8) through double-buffered LDS (rows padded by 16
//     bytes: 8 consecutive rows hit 8 disjoint bank groups); global loads are
//     buffer loads one step ahead, so the last partial token tile reads zeros
//     and writes nothing past L.
//   * fp8 form: OCP e4m3 operands on v_mfma_scale_f32_32x32x64_f8f6f4 (unit
//     block scales), each lane's fragment 32 consecutive hidden elements of
//     its row for both operands; any fixed split of a step's elements over
//     lanes and registers pairs every element of A with the same element of
//     B, so the dot product is complete.  The two per-tensor scales multiply
//     the fp32 accumulator before the norm.
//   * Blocks are ordered so that the workgroups an XCD runs at once cover
//     8 token tiles x 4 feature tiles: each hidden-state tile and each weight
//     tile is then read by several concurrent workgroups through that XCD's
//     L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3attn_internal.h"

namespace h3 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int D = kHeadDim;          // features per head slot
constexpr int kSlots = 2;            // head slots (of the 3H q, k, v heads) per workgroup
constexpr int kTok = 256;            // tokens per workgroup
#ifndef H3_QKV_THREADS
#define H3_QKV_THREADS 512
#endif
constexpr int kThreads = H3_QKV_THREADS;   // waves (slot, token range): 2 slots x kThreads/128 token ranges
constexpr int kTS = 1024 / kThreads;       // 32-token sub-tiles per wave
constexpr int kRows = kSlots * D;    // weight rows per workgroup
constexpr int kGroupTiles = 8;       // token tiles per placement group
constexpr int kBufferFlags = 0x00020000;
constexpr int kE8M0One = 127;        // block-scale exponent of 1.0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes < 0 ? 0 : bytes, kBufferFlags);
}
__device__ __forceinline__ uint4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float lane_half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Contiguous logical ranges per XCD (the hardware deals blocks round-robin).
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = nblk >> 3, extra = nblk & 7;
  return xcd < extra ? xcd * (per + 1) + slot : extra * (per + 1) + (xcd - extra) * per + slot;
}

// kFp8 = false: bf16 operands.  kFp8 = true: e4m3 operands with per-tensor
// scales *x_scale and *w_scale (device scalars).  C counts hidden elements.
// Head slot j in [0, 3H) is q head j, k head j - H or v head j - 2H.
template <bool kFp8>
__global__ __launch_bounds__(kThreads, kThreads / 256) void qkv_proj_kernel(
    const uint8_t *__restrict__ X, const uint8_t *__restrict__ Wq, const uint8_t *__restrict__ Wk,
    const uint8_t *__restrict__ Wv, const float *__restrict__ x_scale, const float *__restrict__ w_scale,
    const float *__restrict__ gamma_q, const float *__restrict__ gamma_k,
    const float *__restrict__ cos_t, const float *__restrict__ sin_t, uint16_t *__restrict__ Qo,
    uint16_t *__restrict__ Ko, uint16_t *__restrict__ Vo, int H, int L, int C, float eps, int n_ttiles) {
  // Bytes of each row per LDS step: 128 for bf16 (measured faster), 64 for
  // fp8 (its 32-byte fragments leave no registers for a longer step).
  constexpr int kStepBytes = kFp8 ? 64 : 128;
  constexpr int kCPR = kStepBytes / 16;         // 16-byte pieces per row and step
  constexpr int kStride = kStepBytes / 2 + 8;   // uint16 slots per LDS row (+16 B: 8 consecutive rows, 8 bank groups)
  constexpr int kWChunks = kRows * kCPR / kThreads;   // 16-byte staging chunks per thread per step
  constexpr int kXChunks = kTok * kCPR / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t w_lds[2][kRows * kStride];
  __shared__ __attribute__((aligned(16))) uint16_t x_lds[2][kTok * kStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  // logical -> (token group, feature tile, token tile within the group)
  const int n_ft = (3 * H + kSlots - 1) / kSlots;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = kGroupTiles * n_ft;
  const int tg = logical / per_group;
  const int rem = logical - tg * per_group;
  const int gsz = min(kGroupTiles, n_ttiles - tg * kGroupTiles);
  const int ft = rem / gsz;
  const int tt = tg * kGroupTiles + (rem - ft * gsz);
  const int t0 = tt * kTok;

  const int row_bytes = C * (kFp8 ? 1 : 2);
  const int tok_rows = L - t0 < kTok ? L - t0 : kTok;
  // One descriptor per slot; a slot past 3H (odd 3H) reads zeros.
  __amdgpu_buffer_rsrc_t rw[kSlots];
#pragma unroll
  for (int sl = 0; sl < kSlots; ++sl) {
    const int j = ft * kSlots + sl;
    const int wh = j / H, hd = j - (j / H) * H;
    const uint8_t *base = wh == 0 ? Wq : wh == 1 ? Wk : Wv;
    rw[sl] = make_rsrc(base + static_cast<size_t>(wh < 3 ? hd : 0) * D * row_bytes, j < 3 * H ? D * row_bytes : 0);
  }
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + static_cast<size_t>(t0) * row_bytes, tok_rows * row_bytes);

  // Staging: chunk c = tid + kThreads i of a step covers row c / kCPR
  // (weight rows 0..255 over the two slots, or token rows), piece c % kCPR
  // of the step's kStepBytes-byte slice of that row.
  uint4 sw[kWChunks], sx[kXChunks];
  auto load = [&](int ks) {
    const uint32_t kb = static_cast<uint32_t>(ks) * kStepBytes;
#pragma unroll
    for (int i = 0; i < kWChunks; ++i) {
      // The first half of the chunks are slot 0's rows 0..127, the rest slot 1's.
      constexpr int kPerSlot = kWChunks / kSlots;
      const int row = tid / kCPR + (kThreads / kCPR) * (i % kPerSlot);
      sw[i] = bload128(rw[i / kPerSlot], row * row_bytes + kb + 16 * (tid % kCPR));
    }
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) {
      const int c = tid + kThreads * i;
      sx[i] = bload128(rx, (c / kCPR) * row_bytes + kb + 16 * (c % kCPR));
    }
  };
  // A row may end half way through its last step (row_bytes is a multiple of
  // 64): pieces past its end are stored as zeros, so they add nothing.  The
  // mask is an AND applied here, where the loads have landed anyway.
  auto store = [&](int buf, int ks) {
    const uint32_t keep =
        kStepBytes == 64 || ks * kStepBytes + 16 * (tid % kCPR) < row_bytes ? 0xFFFFFFFFu : 0u;
    auto masked = [keep](uint4 v) { return make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep); };
#pragma unroll
    for (int i = 0; i < kWChunks; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<uint4 *>(&w_lds[buf][(c / kCPR) * kStride + 8 * (c % kCPR)]) = masked(sw[i]);
    }
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<uint4 *>(&x_lds[buf][(c / kCPR) * kStride + 8 * (c % kCPR)]) = masked(sx[i]);
    }
  };

  // Wave (sl, th): head slot sl of the tile, tokens 32 kTS th .. + 32 kTS - 1.
  const int sl = wave & 1, th = wave >> 1;
  f32x16 acc[4][kTS];
#pragma unroll
  for (int fs = 0; fs < 4; ++fs)
#pragma unroll
    for (int ts = 0; ts < kTS; ++ts) acc[fs][ts] = f32x16{};

  const int n_k = (row_bytes + kStepBytes - 1) / kStepBytes;
  load(0);
  store(0, 0);
  if (n_k > 1) load(1);
  __syncthreads();

  // Fragment addresses: A = weight row 128 sl + 32 fs + l32, B = token row
  // 128 th + 32 ts + l32; bf16: bytes 32kk + 16g of the step's 64, fp8: bytes
  // 32g .. 32g+31.
  const uint16_t *wa = &w_lds[0][(sl * D + l32) * kStride + (kFp8 ? 16 : 8) * g];
  const uint16_t *xb = &x_lds[0][(th * 32 * kTS + l32) * kStride + (kFp8 ? 16 : 8) * g];
  auto frag32 = [](const uint16_t *p) {
    const uint4 lo = *reinterpret_cast<const uint4 *>(p);
    const uint4 hi = *reinterpret_cast<const uint4 *>(p + 8);
    return i32x8{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                 static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
  };
  for (int ks = 0; ks < n_k; ++ks) {
    const int buf = ks & 1;
    const uint16_t *wab = wa + buf * (kRows * kStride);
    const uint16_t *xbb = xb + buf * (kTok * kStride);
    if constexpr (kFp8) {
#pragma unroll
      for (int kk = 0; kk < kStepBytes / 64; ++kk) {
        i32x8 a[4], b[kTS];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = frag32(wab + i * 32 * kStride + 32 * kk);
#pragma unroll
        for (int i = 0; i < kTS; ++i) b[i] = frag32(xbb + i * 32 * kStride + 32 * kk);
#pragma unroll
        for (int fs = 0; fs < 4; ++fs)
#pragma unroll
          for (int ts = 0; ts < kTS; ++ts)
            acc[fs][ts] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[fs], b[ts], acc[fs][ts], 0, 0, 0,
                                                                          kE8M0One, 0, kE8M0One);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < kStepBytes / 32; ++kk) {
        bf16x8 a[4], b[kTS];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8 *>(wab + i * 32 * kStride + 16 * kk);
#pragma unroll
        for (int i = 0; i < kTS; ++i) b[i] = *reinterpret_cast<const bf16x8 *>(xbb + i * 32 * kStride + 16 * kk);
#pragma unroll
        for (int fs = 0; fs < 4; ++fs)
#pragma unroll
          for (int ts = 0; ts < kTS; ++ts)
            acc[fs][ts] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fs], b[ts], acc[fs][ts], 0, 0, 0);
      }
    }
    if (ks + 1 < n_k) {
      // Buffer buf^1 was last read in step ks-1, before the barrier that
      // ended it; step ks+2's loads refill the staging registers.
      store(buf ^ 1, ks + 1);
      if (ks + 2 < n_k) load(ks + 2);
    }
    __syncthreads();
  }

  // Epilogue.  acc[fs][ts][i] = feature 32fs + 8(i/4) + 4g + i%4 of the
  // wave's head slot, token t0 + 128 th + 32 ts + l32.
  const int j = ft * kSlots + sl;
  if (j >= 3 * H) return;
  const int which = j / H, head = j - which * H;   // 0 q, 1 k, 2 v
  uint16_t *Out = which == 0 ? Qo : which == 1 ? Ko : Vo;
  const float *gamma = which == 0 ? gamma_q : gamma_k;
  if constexpr (kFp8) {
    const float sc = x_scale[0] * w_scale[0];
#pragma unroll
    for (int fs = 0; fs < 4; ++fs)
#pragma unroll
      for (int ts = 0; ts < kTS; ++ts) acc[fs][ts] *= sc;
  }
#pragma unroll
  for (int ts = 0; ts < kTS; ++ts) {
    const int t = t0 + th * 32 * kTS + ts * 32 + l32;
    float r = 1.0f;
    if (which < 2) {
      float ss = 0.f;
#pragma unroll
      for (int fs = 0; fs < 4; ++fs)
#pragma unroll
        for (int i = 0; i < 16; ++i) ss = __builtin_fmaf(acc[fs][ts][i], acc[fs][ts][i], ss);
      ss = lane_half_sum(ss);
      r = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
    }
    if (t >= L) continue;
    uint16_t *orow = Out + (static_cast<size_t>(head) * L + t) * D;
#pragma unroll
    for (int fs = 0; fs < 4; ++fs)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int f0 = 32 * fs + 8 * q4 + 4 * g;   // 4 consecutive features f0 .. f0+3
        const float e[4] = {acc[fs][ts][4 * q4], acc[fs][ts][4 * q4 + 1], acc[fs][ts][4 * q4 + 2],
                            acc[fs][ts][4 * q4 + 3]};
        uint2 w;
        if (which < 2) {
          const float4 gm = *reinterpret_cast<const float4 *>(gamma + f0);
          const float2 c = *reinterpret_cast<const float2 *>(cos_t + static_cast<size_t>(t) * (D / 2) + f0 / 2);
          const float2 s = *reinterpret_cast<const float2 *>(sin_t + static_cast<size_t>(t) * (D / 2) + f0 / 2);
          const float y0 = e[0] * r * gm.x, y1 = e[1] * r * gm.y;
          const float y2 = e[2] * r * gm.z, y3 = e[3] * r * gm.w;
          w.x = pack_bf16x2(y0 * c.x - y1 * s.x, y0 * s.x + y1 * c.x);
          w.y = pack_bf16x2(y2 * c.y - y3 * s.y, y2 * s.y + y3 * c.y);
        } else {
          w.x = pack_bf16x2(e[0], e[1]);
          w.y = pack_bf16x2(e[2], e[3]);
        }
        *reinterpret_cast<uint2 *>(orow + f0) = w;
      }
  }
}

}  // namespace

int64_t qkv_proj_grid(int H, int L) {
  return ((static_cast<int64_t>(3) * H + kSlots - 1) / kSlots) * ((static_cast<int64_t>(L) + kTok - 1) / kTok);
}

hipError_t launch_qkv_proj_qknorm_rope(const uint16_t *x, const uint16_t *wq, const uint16_t *wk,
                                       const uint16_t *wv, const float *gamma_q, const float *gamma_k,
                                       const float *cos_t, const float *sin_t, uint16_t *q, uint16_t *k,
                                       uint16_t *v, int H, int L, int C, float eps, hipStream_t stream) {
  const int n_ttiles = (L + kTok - 1) / kTok;
  const int blocks = static_cast<int>(qkv_proj_grid(H, L));
  hipLaunchKernelGGL(qkv_proj_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint8_t *>(x), reinterpret_cast<const uint8_t *>(wq),
                     reinterpret_cast<const uint8_t *>(wk), reinterpret_cast<const uint8_t *>(wv), nullptr, nullptr,
                     gamma_q, gamma_k, cos_t, sin_t, q, k, v, H, L, C, eps, n_ttiles);
  return hipGetLastError();
}

hipError_t launch_qkv_proj_fp8_qknorm_rope(const uint8_t *x, const float *x_scale, const uint8_t *wq,
                                           const uint8_t *wk, const uint8_t *wv, const float *w_scale,
                                           const float *gamma_q, const float *gamma_k, const float *cos_t,
                                           const float *sin_t, uint16_t *q, uint16_t *k, uint16_t *v, int H, int L,
                                           int C, float eps, hipStream_t stream) {
  const int n_ttiles = (L + kTok - 1) / kTok;
  const int blocks = static_cast<int>(qkv_proj_grid(H, L));
  hipLaunchKernelGGL(qkv_proj_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, x, wq, wk, wv, x_scale,
                     w_scale, gamma_q, gamma_k, cos_t, sin_t, q, k, v, H, L, C, eps, n_ttiles);
  return hipGetLastError();
}

}  // namespace h3
