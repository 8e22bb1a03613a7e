// Exact, unmasked, non-causal attention per head for gfx950 (MI355X).
//
// out[h] = softmax(scale * q[h] k[h]^T) v[h] over the whole packed sequence
// ("buqi-minimax-h3-multigpu", How it works and On accuracy; "Tensor
// parallelism for MiniMax-H3", whn09's Neuron FYI: packed full self-attention,
// no mask, any length).  Flash-style: the L x L scores never leave registers.
//
// Work decomposition
//   * One workgroup = one (head, 256-query tile); 8 waves, 32 query rows each.
//   * Keys stream in tiles of 64 through double-buffered LDS: K row-major
//     [key][d], V transposed [d][key] (the transpose happens on the way in).
//   * Per wave and key tile, with v_mfma_f32_32x32x16_bf16:
//       S^T (64 keys x 32 queries) = K_tile . Q^T        16 MFMAs, Q^T in VGPRs
//       O^T (128 d  x 32 queries) += V_tile^T . P^T      16 MFMAs
//     Computing the transposes puts one query row in each lane column of the
//     accumulators, so softmax's running max/sum and O's rescale are
//     lane-local; only the two lane halves (keys split 16/16 per 32-key block)
//     combine, once per tile for the max and once at the end for the sum.
//   * The S^T accumulator, rounded to bf16, is directly the B operand of the
//     P.V product: K rows are fed to the first MFMA in an order (bits 2 and 3
//     of the row index swapped) that makes each lane's 8 accumulator values
//     8 consecutive keys, matching a 16-byte read of the transposed V tile.
//   * Softmax works in base 2: p = 2^(s * scale*log2(e) - m), the same value
//     as e^(scale*s - m') with m' = m / log2(e).
//
// Determinism: a workgroup's arithmetic depends only on its (head, q-tile)
// and keys are visited in a fixed order, so every head's output is bit-
// identical however many heads one launch covers.  The XCD-aware block remap
// changes only where a tile runs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3attn_internal.h"

namespace h3 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int D = kHeadDim;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBr = kWaves * 32;     // query rows per workgroup
constexpr int kBc = 64;              // keys per tile
constexpr int kKStride = D + 8;      // bf16 per K row in LDS (272 B: rows shift 4 banks)
constexpr int kVStride = kBc + 8;    // bf16 per V^T row in LDS (144 B)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = static_cast<__bf16>(lo);
  __bf16 b = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16 &s, int base) {
  uint4 w;
  w.x = pack_bf16x2(s[base + 0], s[base + 1]);
  w.y = pack_bf16x2(s[base + 2], s[base + 3]);
  w.z = pack_bf16x2(s[base + 4], s[base + 5]);
  w.w = pack_bf16x2(s[base + 6], s[base + 7]);
  return __builtin_bit_cast(bf16x8, w);
}

// Maps the hardware's round-robin placement of blocks over the 8 XCDs onto
// contiguous logical tiles: XCD x runs logical tiles [start_x, start_x + n_x),
// so the CUs sharing one L2 sweep the same head's K/V together.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = nblk >> 3, extra = nblk & 7;
  return xcd < extra ? xcd * (per + 1) + slot : extra * (per + 1) + (xcd - extra) * per + slot;
}

__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    uint16_t *__restrict__ O, int L, int n_qtiles, float scale_log2e) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kBc * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][D * kVStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int head = logical / n_qtiles;
  const int qt = logical - head * n_qtiles;
  const size_t head_off = static_cast<size_t>(head) * L * D;
  const uint16_t *Qh = Q + head_off;
  const uint16_t *Kh = K + head_off;
  const uint16_t *Vh = V + head_off;

  // Q^T fragments (B operand): lane holds query row qrow, d = 16c + 8g .. +7.
  const int qrow = qt * kBr + wave * 32 + l32;
  const bool qvalid = qrow < L;
  bf16x8 qf[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (qvalid) w = *reinterpret_cast<const uint4 *>(Qh + static_cast<size_t>(qrow) * D + 16 * c + 8 * g);
    qf[c] = __builtin_bit_cast(bf16x8, w);
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m_run = -__builtin_inff();  // running max, base-2 scaled units
  float l_run = 0.f;                // this lane's partial row sum

  // Global -> register staging of one key tile.
  //   K: 64 rows x 16 chunks of 16 B; thread takes chunks tid and tid + 512.
  //   V: thread takes d pair (2*vd, 2*vd+1) of keys 8*vk .. 8*vk+7 (4 B each),
  //      so every 64-lane load covers one whole 256-byte V row.
  const int vd = tid & 63, vk = tid >> 6;
  uint4 kreg[2];
  uint32_t vreg[8];
  const int n_kt = (L + kBc - 1) / kBc;

  auto gload = [&](int kt) {
    const int key0 = kt * kBc;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + kThreads * i;
      const int key = key0 + (c >> 4);
      kreg[i] = key < L ? *reinterpret_cast<const uint4 *>(Kh + static_cast<size_t>(key) * D + (c & 15) * 8)
                        : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = key0 + 8 * vk + j;
      vreg[j] = key < L ? *reinterpret_cast<const uint32_t *>(Vh + static_cast<size_t>(key) * D + 2 * vd) : 0u;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<uint4 *>(&k_lds[buf][(c >> 4) * kKStride + (c & 15) * 8]) = kreg[i];
    }
    uint4 lo, hi;
    lo.x = (vreg[0] & 0xffffu) | (vreg[1] << 16);
    lo.y = (vreg[2] & 0xffffu) | (vreg[3] << 16);
    lo.z = (vreg[4] & 0xffffu) | (vreg[5] << 16);
    lo.w = (vreg[6] & 0xffffu) | (vreg[7] << 16);
    hi.x = (vreg[0] >> 16) | (vreg[1] & 0xffff0000u);
    hi.y = (vreg[2] >> 16) | (vreg[3] & 0xffff0000u);
    hi.z = (vreg[4] >> 16) | (vreg[5] & 0xffff0000u);
    hi.w = (vreg[6] >> 16) | (vreg[7] & 0xffff0000u);
    *reinterpret_cast<uint4 *>(&vt_lds[buf][(2 * vd) * kVStride + 8 * vk]) = lo;
    *reinterpret_cast<uint4 *>(&vt_lds[buf][(2 * vd + 1) * kVStride + 8 * vk]) = hi;
  };

  gload(0);
  lstore(0);
  __syncthreads();

  const int krow = swap_bits23(l32);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) gload(kt + 1);

    // S^T = K_tile . Q^T for the two 32-key blocks.
    f32x16 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = f32x16{};
      const uint16_t *kp = &k_lds[buf][(32 * b + krow) * kKStride + 8 * g];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kp + 16 * c);
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[b], 0, 0, 0);
      }
    }

    // Accumulator s[b][i] holds key kt*64 + 32b + 16(i/8) + 8g + i%8.
    const int key_base = kt * kBc;
    if (key_base + kBc > L) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key_base + 32 * b + 16 * (i >> 3) + 8 * g + (i & 7) >= L) s[b][i] = -__builtin_inff();
    }

    float mx = s[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, s[b][i]);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = __builtin_fmaxf(m_run, mx * scale_log2e);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    float psum = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][i], scale_log2e, -m_new));
        s[b][i] = p;
        psum += p;
      }
    l_run = __builtin_fmaf(l_run, alpha, psum);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;

    bf16x8 pf[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      pf[b][0] = to_bf16x8(s[b], 0);
      pf[b][1] = to_bf16x8(s[b], 8);
    }

    // O^T += V_tile^T . P^T
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const uint16_t *vp = &vt_lds[buf][(32 * db + l32) * kVStride + 8 * g];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vp + 32 * b + 16 * t);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[b][t], o[db], 0, 0, 0);
        }
    }

    if (kt + 1 < n_kt) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: full row sum, normalise, round once to bf16.
  l_run += __shfl_xor(l_run, 32);
  const float inv_l = 1.0f / l_run;
  if (qvalid) {
    uint16_t *orow = O + head_off + static_cast<size_t>(qrow) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        // o[db][4*grp + r] holds d = 32db + 8grp + 4g + r.
        uint2 w;
        w.x = pack_bf16x2(o[db][4 * grp + 0] * inv_l, o[db][4 * grp + 1] * inv_l);
        w.y = pack_bf16x2(o[db][4 * grp + 2] * inv_l, o[db][4 * grp + 3] * inv_l);
        *reinterpret_cast<uint2 *>(orow + 32 * db + 8 * grp + 4 * g) = w;
      }
  }
}

}  // namespace

int64_t attention_grid(int H, int L) {
  return static_cast<int64_t>(H) * ((static_cast<int64_t>(L) + kBr - 1) / kBr);
}

hipError_t launch_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *out, int H,
                            int L, float scale, hipStream_t stream) {
  const int n_qtiles = (L + kBr - 1) / kBr;
  const int blocks = static_cast<int>(attention_grid(H, L));
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(blocks), dim3(kThreads), 0, stream, q, k, v, out, L, n_qtiles,
                     scale * kLog2e);
  return hipGetLastError();
}

}  // namespace h3
