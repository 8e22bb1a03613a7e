// Row-sliced qkv projection with QK-RMSNorm + RoPE in the epilogue, for gfx950.
//
// A rank that holds the whole (gathered) hidden state x [L][C] projects it
// through only its own heads' rows of qkv_proj: wq, wk, wv are [H*128][C]
// ("buqi-minimax-h3-multigpu", How it works: the all_gather form for small
// world sizes, where slicing rows of the weight is exact).  q and k then get
// the head_dim RMSNorm and the rotary embedding ("Tensor parallelism for
// MiniMax-H3", PR description), fused here into the GEMM epilogue so the
// projection never goes through HBM in between and is never rounded before
// the norm.  Outputs are [H][L][128] bf16, the layout the attention reads;
// v may instead be written transposed, [H][128][ldv] with tokens contiguous
// (the layout of h3_attention_vt).
//
// Work decomposition
//   * Workgroup = (feature tile, token tile): head slots (128 output
//     features each; slot j of the 3H q, k, v heads) x 256 tokens.  bf16:
//     three head slots, 12 waves (three per SIMD), each one head slot x 64
//     tokens with 8 accumulator tiles.  fp8, whose 32-byte fragments leave
//     no room for that at three waves per SIMD: two head slots, 16 waves
//     (four per SIMD), each one head slot x 32 tokens with 4 accumulator
//     tiles.
//   * The product is computed transposed, C^T = W . X^T, with
//     v_mfma_f32_32x32x16_bf16: A = weight rows (features), B = hidden rows
//     (tokens).  Both operands are K-contiguous in memory, so every fragment
//     is one 16-byte LDS read.  The accumulator puts one token per lane
//     column and 16 features per lane, so a token's sum of squares over its
//     128 features is lane-local plus one lane-half exchange, and each RoPE
//     pair (2j, 2j+1) sits in one lane.
//   * The hidden dimension streams in steps of 128 bytes per row (64 bf16 or
//     128 fp8 elements) through a 2-slot LDS ring: buffer loads with the
//     LDS-destination bit put each step's weight rows and 256 token rows in
//     LDS one step ahead, with no register staging.  Rows are 128 bytes with
//     their eight 16-byte chunks swizzled by (row / 2) % 8, so the 16 rows of
//     a fragment read hit 16 distinct bank groups.  A hidden size that ends
//     halfway through a step loads zeros into the last step's second half,
//     whose products then add exact zeros.
//     The descriptor ranges make the last partial token tile (and an odd 3H's
//     empty head slot) read zeros, and nothing is written past L.
//   * fp8 form: OCP e4m3 operands on v_mfma_scale_f32_32x32x64_f8f6f4 (unit
//     block scales), each lane's fragment 32 consecutive hidden elements of
//     its row for both operands; any fixed split of a step's elements over
//     lanes and registers pairs every element of A with the same element of
//     B, so the dot product is complete.  The two per-tensor scales multiply
//     the fp32 accumulator before the norm.
//   * Transposed v: a lane holds 4 consecutive features of one token, and the
//     4 lanes of a quad hold 4 consecutive tokens.  Two exchanges inside the
//     quad (DPP, lanes xor 1 then xor 2) transpose that 4 x 4 block, so each
//     lane stores one feature's 4 tokens as 8 bytes, and a half-wave fills 8
//     feature rows with 64 contiguous bytes each.  Token columns from L up to
//     the next multiple of 8 receive the exact zeros of the token rows that
//     read as zeros.
//   * Blocks are ordered so that the workgroups an XCD runs at once cover
//     8 token tiles x 4 feature tiles: each hidden-state tile and each weight
//     tile is then read by several concurrent workgroups through that XCD's
//     L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "h3attn_internal.h"

namespace h3 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int D = kHeadDim;          // features per head slot
constexpr int kTok = 256;            // tokens per workgroup
// 32-token sub-tiles per wave: 2 (64 tokens) for bf16, 1 for fp8.
template <bool kFp8> constexpr int ts_of() { return kFp8 ? 1 : 2; }
template <bool kFp8> constexpr int ranges_of() { return kTok / (32 * ts_of<kFp8>()); }   // waves per head slot
// Head slots (of the 3H q, k, v heads) per workgroup: 3 for bf16 (12 waves
// of 64 tokens, three per SIMD: the bf16 form fits the 168 registers that
// allows), 2 for fp8 (16 waves of 32 tokens, four per SIMD, within 128).
template <bool kFp8> constexpr int slots_of() { return kFp8 ? 2 : 3; }
template <bool kFp8> constexpr int threads_of() { return 64 * ranges_of<kFp8>() * slots_of<kFp8>(); }
constexpr int kGroupTiles = 8;       // token tiles per placement group
constexpr int kBufferFlags = 0x00020000;
constexpr int kStepBytes = 128;      // bytes of each row per step (64 bf16 or 128 fp8 hidden elements)
constexpr int kRowElems = kStepBytes / 2;   // uint16 per LDS row (no padding)
constexpr int kChunks = kStepBytes / 16;    // 16-byte chunks per row
constexpr int kPieceRows = 1024 / kStepBytes;   // rows per 1-KB load
constexpr int kRing = 2;             // LDS ring depth (steps) for each of W and X
constexpr int kE8M0One = 127;        // block-scale exponent of 1.0
// DPP quad permutations (lane i of each quad reads lane perm[i]): xor 1 and xor 2.
constexpr int kQuadXor1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);
constexpr int kQuadXor2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes < 0 ? 0 : bytes, kBufferFlags);
}

typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_char *)(p)));
}

// Chunk swizzle inside a 128-byte LDS row (8 chunks of 16 bytes): a fragment
// read takes one logical chunk from 16 consecutive rows; rows 2 apart share
// banks, and the swizzle puts those 8 pairs of rows in 8 different chunks.
__device__ __forceinline__ int row_swz(int row) { return (row >> 1) & 7; }

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
// Head slot j in [0, 3H) is q head j, k head j - H or v head j - 2H.  ldv = 0
// writes v as [H][L][128]; ldv > 0 (a multiple of 8, at least L) writes it as
// [H][128][ldv].
template <bool kFp8>
__global__ __launch_bounds__(threads_of<kFp8>(), threads_of<kFp8>() / 256) void qkv_proj_kernel(
    const uint8_t *__restrict__ X, const uint8_t *__restrict__ Wq, const uint8_t *__restrict__ Wk,
    const uint8_t *__restrict__ Wv, const float *__restrict__ x_scale, const float *__restrict__ w_scale,
    const float *__restrict__ gamma_q, const float *__restrict__ gamma_k,
    const float *__restrict__ cos_t, const float *__restrict__ sin_t, uint16_t *__restrict__ Qo,
    uint16_t *__restrict__ Ko, uint16_t *__restrict__ Vo, int H, int L, int C, float eps, int n_ttiles, int ldv) {
  constexpr int kSlots = slots_of<kFp8>();
  constexpr int kTS = ts_of<kFp8>();
  constexpr int kWaves = threads_of<kFp8>() / 64;
  constexpr int kRows = kSlots * D;          // weight rows per workgroup
  constexpr int kWPieces = D / kPieceRows / 8;   // 1-KB loads per head slot and weight-loading wave
  constexpr int kXLoads = kTok / kPieceRows;     // 1-KB loads per step for the token rows
  __shared__ __attribute__((aligned(1024))) uint16_t w_lds[kRing][kRows * kRowElems];
  __shared__ __attribute__((aligned(1024))) uint16_t x_lds[kRing][kTok * kRowElems];

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

  // Steps go from global memory straight into LDS (buffer loads with the
  // LDS-destination bit), one step ahead of the one being multiplied.
  // A load writes rows 8n .. 8n+7 of the step's weight rows or 256 token
  // rows as one contiguous kilobyte: lane i lands in row 8n + i/8 at
  // physical chunk i%8 and fetches the row's logical chunk (i%8) ^ swizzle.
  // Rows past 3H or past L read as zeros (descriptor range), and so does the
  // second half of a final half step (its lanes point past the range).  The
  // waits below are explicit.
  // Each load sets m0 (its LDS destination) itself.  m0 cannot be named as
  // clobbered (the compiler reserves it); no compiler-generated instruction
  // in this kernel reads or writes it.
  const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int dma_row = lane / kChunks;
  // Token-row loads: all waves with 8, waves 8.. with 12 or 16.
  constexpr int kXFirst = kWaves == 8 ? 0 : 8;
  constexpr int kXWaves = kWaves - kXFirst;
  // Past every descriptor's range: a tile's descriptor covers at most 256 rows
  // of 2^21 bytes (the API bounds hidden).
  constexpr uint32_t kPastRange = 1u << 30;
  auto dma_step = [&](int ks, int slot) {
    const uint32_t kb = static_cast<uint32_t>(ks) * kStepBytes;
    const bool half = row_bytes - ks * kStepBytes < kStepBytes;   // only the first half exists
    auto off = [&](int row, int ch) {
      return half && ch >= kChunks / 2 ? kPastRange : static_cast<uint32_t>(row * row_bytes) + kb + 16 * ch;
    };
    // Weight rows: waves 0..7 load 16-row block w of every head slot, as
    // kWPieces loads of 8 rows each.
    if (wave_u < 8u) {
#pragma unroll
      for (int h = 0; h < kSlots; ++h)
#pragma unroll
        for (int pc = 0; pc < kWPieces; ++pc) {
          const int row = kPieceRows * (kWPieces * wave + pc) + dma_row;   // row within head slot h
          const int ch = (lane % kChunks) ^ row_swz(row);
          const uint32_t m0 = lds_addr(w_lds[slot]) + ((8u * h + wave_u) * kWPieces + pc) * 1024u;
          asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                       :
                       : "s"(m0), "v"(off(row, ch)), "s"(rw[h])
                       : "memory");
        }
    }
    // Token rows: 32 blocks of 8, four per wave with 8 waves, eight per
    // wave for waves 8..11 with 12, four for waves 8..15 with 16.
    if (wave_u >= static_cast<uint32_t>(kXFirst)) {
#pragma unroll
      for (int j = 0; j < kXLoads / kXWaves; ++j) {
        const uint32_t nu = wave_u - kXFirst + kXWaves * j;
        const int row = kPieceRows * (wave - kXFirst + kXWaves * j) + dma_row;
        const int ch = (lane % kChunks) ^ row_swz(row);
        const uint32_t m0 = lds_addr(x_lds[slot]) + nu * 1024u;
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :
                     : "s"(m0), "v"(off(row, ch)), "s"(rx)
                     : "memory");
      }
    }
  };
  static_assert(kWaves == 8 || kWaves == 12 || kWaves == 16, "load split above");
  static_assert(kXLoads % (kWaves == 8 ? 8 : kWaves - 8) == 0, "token loads split evenly");

  // Wave (sl, th): head slot sl of the tile, tokens 32 kTS th .. + 32 kTS - 1.
  const int sl = wave % kSlots, th = wave / kSlots;
  f32x16 acc[4][kTS];
#pragma unroll
  for (int fs = 0; fs < 4; ++fs)
#pragma unroll
    for (int ts = 0; ts < kTS; ++ts) acc[fs][ts] = f32x16{};

  // hidden is a multiple of half a step (the API checks); a final half step
  // runs as a whole one over zeros.
  const int n_k = (row_bytes + kStepBytes - 1) / kStepBytes;
  dma_step(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // step 0 is in LDS (this wave's share)
  __syncthreads();

  // Fragment addresses: A = weight row 128 sl + 32 fs + l32, B = token row
  // 32 kTS th + 32 ts + l32, both with swizzle (l32 >> 1) & 7.  bf16
  // sub-step kk (16 elements): logical chunk 2kk + g; fp8 sub-step kk (64
  // elements): logical chunks 4kk + 2g and 4kk + 2g + 1 (32 bytes).
  const int sw_l = row_swz(l32);
  const uint16_t *wa = &w_lds[0][(sl * D + l32) * kRowElems];
  const uint16_t *xb = &x_lds[0][(th * 32 * kTS + l32) * kRowElems];
  auto chunk_off = [&](int c) { return 8 * (c ^ sw_l); };   // uint16 offset of logical chunk c
  auto frag32 = [](const uint16_t *p0, const uint16_t *p1) {
    const uint4 lo = *reinterpret_cast<const uint4 *>(p0);
    const uint4 hi = *reinterpret_cast<const uint4 *>(p1);
    return i32x8{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                 static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
  };
  // Step ks multiplies slot ks % kRing (R, a compile-time value) after
  // issuing step ks+1 into the other slot, which held step ks-1: every wave
  // finished reading it before the barrier that ended step ks-1.
  auto step = [&](auto r_c, int ks) {
    constexpr int R = decltype(r_c)::value;
    constexpr int kSub = kFp8 ? kChunks / 4 : kChunks / 2;   // 64-element (fp8) or 16-element (bf16) sub-steps
    if (ks + 1 < n_k) dma_step(ks + 1, (R + 1) % kRing);
    const uint16_t *wab = wa + R * (kRows * kRowElems);
    const uint16_t *xbb = xb + R * (kTok * kRowElems);
    if constexpr (kFp8) {
#pragma unroll
      for (int kk = 0; kk < kSub; ++kk) {
        const int ca = chunk_off(4 * kk + 2 * g), cb = chunk_off(4 * kk + 2 * g + 1);
        i32x8 a[4], b[kTS];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = frag32(wab + i * 32 * kRowElems + ca, wab + i * 32 * kRowElems + cb);
#pragma unroll
        for (int i = 0; i < kTS; ++i) b[i] = frag32(xbb + i * 32 * kRowElems + ca, xbb + i * 32 * kRowElems + cb);
#pragma unroll
        for (int fs = 0; fs < 4; ++fs)
#pragma unroll
          for (int ts = 0; ts < kTS; ++ts)
            acc[fs][ts] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[fs], b[ts], acc[fs][ts], 0, 0, 0,
                                                                          kE8M0One, 0, kE8M0One);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < kSub; ++kk) {
        const int cc = chunk_off(2 * kk + g);
        bf16x8 a[4], b[kTS];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8 *>(wab + i * 32 * kRowElems + cc);
#pragma unroll
        for (int i = 0; i < kTS; ++i) b[i] = *reinterpret_cast<const bf16x8 *>(xbb + i * 32 * kRowElems + cc);
#pragma unroll
        for (int fs = 0; fs < 4; ++fs)
#pragma unroll
          for (int ts = 0; ts < kTS; ++ts)
            acc[fs][ts] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fs], b[ts], acc[fs][ts], 0, 0, 0);
      }
    }
    // Step ks+1 must be in LDS before the barrier.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  for (int ks = 0; ks < n_k; ks += kRing) {
    step(std::integral_constant<int, 0>{}, ks);
    if (ks + 1 < n_k) step(std::integral_constant<int, 1>{}, ks + 1);
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
  if (which == 2 && ldv > 0) {
    // Transposed v (wave-uniform branch; every lane takes part in the
    // exchanges, and stores are predicated afterwards).  Lane qk = l32 % 4 of
    // a quad ends with feature f0 + qk of the quad's tokens tq .. tq+3.
    const int qk = l32 & 3;
    const int l8 = (L + 7) & ~7;   // columns written: the tokens plus their zero padding
    uint16_t *vt = Vo + static_cast<size_t>(head) * D * ldv;
#pragma unroll
    for (int ts = 0; ts < kTS; ++ts) {
      const int tq = t0 + th * 32 * kTS + ts * 32 + (l32 & ~3);
#pragma unroll
      for (int fs = 0; fs < 4; ++fs)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int f0 = 32 * fs + 8 * q4 + 4 * g;   // this lane holds features f0 .. f0+3 of token tq + qk
          const uint32_t x = pack_bf16x2(acc[fs][ts][4 * q4], acc[fs][ts][4 * q4 + 1]);
          const uint32_t y = pack_bf16x2(acc[fs][ts][4 * q4 + 2], acc[fs][ts][4 * q4 + 3]);
          // Lanes xor 1: the even lane of a pair keeps features f0, f0+2 of
          // its two tokens, the odd lane features f0+1, f0+3.
          const uint32_t xp = __builtin_amdgcn_update_dpp(0, x, kQuadXor1, 0xF, 0xF, false);
          const uint32_t yp = __builtin_amdgcn_update_dpp(0, y, kQuadXor1, 0xF, 0xF, false);
          const bool odd = (qk & 1) != 0;
          const uint32_t u = odd ? (xp >> 16) | (x & 0xFFFF0000u) : (x & 0xFFFFu) | (xp << 16);
          const uint32_t w = odd ? (yp >> 16) | (y & 0xFFFF0000u) : (y & 0xFFFFu) | (yp << 16);
          // Lanes xor 2: u holds feature f0 + (qk & 1), w feature f0 + 2 +
          // (qk & 1), both for tokens tq + (qk & 2) and the next one.
          const bool hi = (qk & 2) != 0;
          const uint32_t got = __builtin_amdgcn_update_dpp(0, hi ? u : w, kQuadXor2, 0xF, 0xF, false);
          uint2 out;
          out.x = hi ? got : u;
          out.y = hi ? w : got;
          if (tq < l8) *reinterpret_cast<uint2 *>(vt + static_cast<size_t>(f0 + qk) * ldv + tq) = out;
        }
    }
    return;
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

// The larger of the two forms' grids (fp8: two head slots per workgroup).
int64_t qkv_proj_grid(int H, int L) {
  return ((static_cast<int64_t>(3) * H + 1) / 2) * ((static_cast<int64_t>(L) + kTok - 1) / kTok);
}

hipError_t launch_qkv_proj_qknorm_rope(const uint16_t *x, const uint16_t *wq, const uint16_t *wk,
                                       const uint16_t *wv, const float *gamma_q, const float *gamma_k,
                                       const float *cos_t, const float *sin_t, uint16_t *q, uint16_t *k,
                                       uint16_t *v, int H, int L, int C, float eps, int ldv, hipStream_t stream) {
  const int n_ttiles = (L + kTok - 1) / kTok;
  const int blocks = (3 * H + slots_of<false>() - 1) / slots_of<false>() * n_ttiles;
  hipLaunchKernelGGL(qkv_proj_kernel<false>, dim3(blocks), dim3(threads_of<false>()), 0, stream,
                     reinterpret_cast<const uint8_t *>(x), reinterpret_cast<const uint8_t *>(wq),
                     reinterpret_cast<const uint8_t *>(wk), reinterpret_cast<const uint8_t *>(wv), nullptr, nullptr,
                     gamma_q, gamma_k, cos_t, sin_t, q, k, v, H, L, C, eps, n_ttiles, ldv);
  return hipGetLastError();
}

hipError_t launch_qkv_proj_fp8_qknorm_rope(const uint8_t *x, const float *x_scale, const uint8_t *wq,
                                           const uint8_t *wk, const uint8_t *wv, const float *w_scale,
                                           const float *gamma_q, const float *gamma_k, const float *cos_t,
                                           const float *sin_t, uint16_t *q, uint16_t *k, uint16_t *v, int H, int L,
                                           int C, float eps, int ldv, hipStream_t stream) {
  const int n_ttiles = (L + kTok - 1) / kTok;
  const int blocks = (3 * H + slots_of<true>() - 1) / slots_of<true>() * n_ttiles;
  hipLaunchKernelGGL(qkv_proj_kernel<true>, dim3(blocks), dim3(threads_of<true>()), 0, stream, x, wq, wk, wv, x_scale,
                     w_scale, gamma_q, gamma_k, cos_t, sin_t, q, k, v, H, L, C, eps, n_ttiles, ldv);
  return hipGetLastError();
}

}  // namespace h3
