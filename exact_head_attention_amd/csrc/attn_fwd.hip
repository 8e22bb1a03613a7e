// Exact, unmasked, non-causal attention per head for gfx950 (MI355X).
//
// out[h] = softmax(scale * q[h] k[h]^T) v[h] over the whole packed sequence
// ("buqi-minimax-h3-multigpu", How it works and On accuracy; "Tensor
// parallelism for MiniMax-H3", whn09's Neuron FYI: packed full self-attention,
// no mask, any length).  Flash-style: the L x L scores never leave registers.
//
// Work decomposition
//   * Work unit = one (head, 256-query tile); each wave owns 32 query rows.
//     A unit runs as one 8-wave workgroup, or, in the tail launch, as two
//     8-wave workgroups of 128 rows (or, when only a few units are left
//     over, four 4-wave workgroups of 64 rows) in which two waves share each
//     32-row group (attn_tail_kernel; see launch_split below).
//   * Keys stream in tiles of 64 through a 4-slot LDS ring per tensor, K and
//     V both row-major [key][d] with an XOR swizzle of the 16-byte chunks.
//     Tiles move from global memory straight into LDS (buffer loads with the
//     LDS-destination bit), K three tiles and V two tiles ahead of their
//     use, so no registers stage them and a load has two steps to land.  V
//     is read as the transposed MFMA operand with ds_read_b64_tr_b16.
//     h3_attention_vt takes V already transposed, [H][D][ldv] with keys
//     contiguous: its tiles sit in LDS as [d][64 keys] and the same operand
//     is a plain 16-byte read (half the LDS instructions for V).
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
// Determinism: a row's arithmetic depends only on its (head, row) and keys
// are visited in a fixed order; the tail kernel performs each row's
// operations in the same order as the main kernel, only split over two
// waves.  So every head's output is bit-identical however many heads one
// launch covers.
// The XCD-aware block remap and the main/tail split change only where and
// when a row runs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "h3attn_internal.h"

namespace h3 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int D = kHeadDim;
constexpr int kUnitRows = 256;       // query rows per work unit (8 waves x 32)
constexpr int kBc = 64;              // keys per tile
constexpr int kSlots = 4;            // LDS ring depth (tiles) for each of K and V
constexpr int kTileElems = kBc * D;  // one tile, rows of 256 B without padding
constexpr float kLog2e = 1.4426950408889634f;
// The running max is raised only when some row of the wave sees a larger
// score (a wave-uniform branch, taken a few dozen times per 32-row block over
// a 32k sequence), so the O rescale is skipped on almost every tile.  The max
// is always exact: a row's largest weight is then exactly 1, which keeps the
// bf16 rounding of P off the dominant term of peaky rows.
constexpr int kBufferFlags = 0x00020000;   // raw buffer, 32-bit data, gfx9 encoding

__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Two floats to bf16 (nearest even) in one v_cvt_pk_bf16_f32; lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Buffer loads: the hardware returns zeros past num_records bytes, so ragged
// tails need no branches and never touch memory outside the head.
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_char *)(p)));
}

// 16-byte chunk swizzles inside a 256-byte LDS row (chunk index ^ swizzle).
//   K: row & 15 -- a fragment read takes one logical chunk from 16 rows that
//      differ in their low four bits, which then sit in 16 distinct chunks.
//   V: 4 (row & 3) -- a transposed read takes 4 chunks (bits 0-1) from 4
//      consecutive rows, which then sit in 4 disjoint groups of 4 chunks.
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 2; }
//   V^T tile [d][64 keys] (128-byte rows): (d / 2) % 8 -- a fragment read
//      takes one logical chunk from 16 consecutive rows; rows 2 apart share
//      banks, and the swizzle puts those 8 row pairs in 8 different chunks.
__device__ __forceinline__ int vt_swz(int d) { return (d >> 1) & 7; }
// A V^T load offset past every descriptor's range (a head's V^T spans at
// most 2^31 bytes): the load reads zeros.
constexpr uint32_t kVtPastRange = 0xC0000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes < 0 ? 0 : bytes, kBufferFlags);
}
__device__ __forceinline__ uint4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Maps the hardware's round-robin placement of blocks over the 8 XCDs onto
// contiguous logical tiles: XCD x runs logical tiles [start_x, start_x + n_x),
// so the CUs sharing one L2 sweep the same head's K/V together.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = nblk >> 3, extra = nblk & 7;
  return xcd < extra ? xcd * (per + 1) + slot : extra * (per + 1) + (xcd - extra) * per + slot;
}

__device__ __forceinline__ float lane_half_max(float x) {
  // Lanes l and l^32 hold the same query row's two key halves.
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __builtin_fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float lane_half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Max of 32 scores (two 16-value accumulators), as a tree of independent maxes.
__device__ __forceinline__ float max32(const f32x16 &a, const f32x16 &b) {
  float t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    t[i] = __builtin_fmaxf(__builtin_fmaxf(a[2 * i], a[2 * i + 1]), __builtin_fmaxf(b[2 * i], b[2 * i + 1]));
#pragma unroll
  for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = __builtin_fmaxf(t[i], t[i + w]);
  return t[0];
}

constexpr int kWaves = 8;   // waves per workgroup in both kernels

// Loader `ld` of kLoaders waves moves its 16 / kLoaders 1-KB pieces of
// 64-key tile t of one tensor from global memory straight into LDS (buffer
// loads with the LDS-destination bit).  Piece j covers rows 4n .. 4n+3,
// n = ld + kLoaders j, as one contiguous kilobyte: lane i lands in row
// 4n + i/16 at physical chunk i%16, so it fetches the row's logical chunk
// (i%16) ^ swizzle.  Keys at or past Lk read as zeros (the descriptor covers
// only the tile's valid rows).  The loads are tracked by the vector-memory
// counter only; callers wait explicitly.  Each load sets m0 (its LDS
// destination) itself.  m0 cannot be named as clobbered (the compiler
// reserves it); no compiler-generated instruction in these kernels reads or
// writes it.  ld_u is ld as a wave-uniform (scalar) value.
template <int kLoaders>
__device__ __forceinline__ void dma_tile(const uint16_t *base, int t, int Lk, const uint16_t *dst, bool is_k,
                                         int ld, uint32_t ld_u, int lane) {
  const int keys_left = Lk - t * kBc;
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(base + static_cast<size_t>(t) * kBc * D, (keys_left < kBc ? keys_left : kBc) * (D * 2));
#pragma unroll
  for (int j = 0; j < 16 / kLoaders; ++j) {
    const int n = ld + kLoaders * j;
    const int row = 4 * n + (lane >> 4);
    const int chunk = (lane & 15) ^ (is_k ? k_swz(row) : v_swz(row));
    const uint32_t m0 = lds_addr(dst) + (ld_u + kLoaders * j) * 1024u;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(row * (D * 2) + 16 * chunk), "s"(rs)
                 : "memory");
  }
}

// The V^T form of dma_tile: tile t of one head's V^T ([D][ldv], keys
// contiguous) goes to LDS as [d][64 keys], 128 bytes per row.  Piece j
// covers rows 8n .. 8n+7 (n = ld + kLoaders j) as one kilobyte: lane i lands
// in row 8n + i/8 at physical chunk i%8 and fetches the row's logical chunk
// (i%8) ^ vt_swz(row), keys t*64 + 8*logical .. +7.  With kMask, a chunk
// whose first key is at or past Lk reads zeros (its offset lies past the
// descriptor); the one chunk that straddles Lk reads the row's padding past
// Lk, which only ever meets exact zero weights (the caller keeps it finite).
// Callers pass kMask = false only for tiles that lie wholly below Lk: the
// extra compare in every step's loads costs ~4% of the kernel's time
// (it changes how the compiler interleaves the step).
template <int kLoaders, bool kMask>
__device__ __forceinline__ void dma_vt_tile(const uint16_t *base, int t, int Lk, int ldv, const uint16_t *dst, int ld,
                                            uint32_t ld_u, int lane) {
  // Row d of the tile starts d*ldv*2 bytes after base + t*64 keys; the range
  // ends with the head (at most 2^31 bytes, so it is passed as raw bits).
  const uint32_t range = static_cast<uint32_t>(D) * static_cast<uint32_t>(ldv) * 2u -
                         static_cast<uint32_t>(t) * static_cast<uint32_t>(kBc * 2);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(base + static_cast<size_t>(t) * kBc), 0, static_cast<int>(range), kBufferFlags);
#pragma unroll
  for (int j = 0; j < 16 / kLoaders; ++j) {
    const int n = ld + kLoaders * j;
    const int row = 8 * n + (lane >> 3);
    const int chunk = (lane & 7) ^ vt_swz(row);
    const uint32_t off = kMask && t * kBc + 8 * chunk >= Lk
                             ? kVtPastRange
                             : static_cast<uint32_t>(row) * static_cast<uint32_t>(ldv) * 2u + 16u * chunk;
    const uint32_t m0 = lds_addr(dst) + (ld_u + kLoaders * j) * 1024u;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(off), "s"(rs)
                 : "memory");
  }
}

// K fragment of chunk pair c (A operand of the score product): row krow
// (+32 for the second key block), logical chunk 2c + g, i.e. physical chunk
// 2c ^ (g ^ (krow & 15)), krow = l32 with bits 2 and 3 swapped.
__device__ __forceinline__ void k_offsets(int lane, int (&koff)[8]) {
  const int krow = swap_bits23(lane & 31), g = lane >> 5;
#pragma unroll
  for (int c = 0; c < 8; ++c) koff[c] = krow * D + 8 * ((2 * c) ^ (g ^ k_swz(krow)));
}
__device__ __forceinline__ bf16x8 kread(const uint16_t *kt_lds, const int (&koff)[8], int b, int c) {
  return *reinterpret_cast<const bf16x8 *>(kt_lds + koff[c] + b * 32 * D);
}

// Transposed V reads: within each 16-lane group, lane L names row
// 8g + L/4 (+4 for the second read) and columns 16*dhalf + 4*(L%4) .. +3;
// the hardware hands lane j of the group column 16*dhalf + j of the four
// named rows, i.e. V[8g + 0..7][32db + l32] across the two reads.
// The columns of d block db sit in logical chunk 4db + 2 dhalf + (L%4)/2 of
// rows 8g + L/4 (+16 per k-step, +4 for the second read), whose swizzle
// 4 (row & 3) depends on L only.
__device__ __forceinline__ void v_offsets(int lane, int (&voff)[4]) {
  const int g = lane >> 5;
  const int vrow = 8 * g + ((lane & 15) >> 2);
  const int vch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
  for (int db = 0; db < 4; ++db) voff[db] = vrow * D + 8 * ((4 * db + vch) ^ v_swz(vrow)) + 4 * (lane & 1);
}
__device__ __forceinline__ bf16x8 vread(const uint16_t *vt, const int (&voff)[4], int bt, int db) {
  const uint16_t *src = vt + voff[db] + 16 * bt * D;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + 4 * D));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// The same fragment from a V^T tile: row d = 32db + l32, keys 16bt + 8g .. +7,
// i.e. logical chunk 2bt + g of row d, one 16-byte read.
__device__ __forceinline__ bf16x8 vread_t(const uint16_t *vt, int bt, int db, int l32, int g) {
  const int d = 32 * db + l32;
  return *reinterpret_cast<const bf16x8 *>(vt + d * kBc + 8 * ((2 * bt + g) ^ vt_swz(d)));
}

// Mask the keys of tile t at or past Lk (only the last, ragged tile has any).
// s[b][i] holds key t*64 + 32b + 16(i/8) + 8g + i%8.
__device__ __forceinline__ void mask_tile(f32x16 (&sv)[2], int t, int Lk, int g) {
  const int key_base = t * kBc;
  if (key_base + kBc > Lk) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key_base + 32 * b + 16 * (i >> 3) + 8 * g + (i & 7) >= Lk) sv[b][i] = -__builtin_inff();
  }
}

// Epilogue of one lane's half of query row qrow: normalise by the full row
// sum and round once to bf16 (or keep fp32 and write the log-sum-exp:
// ln(l * 2^m) = (log2(l) + m) * ln 2).  o[db][4*grp + r] holds
// d = 32db + 8grp + 4g + r.
template <bool kLse>
__device__ __forceinline__ void store_row(const f32x16 (&o)[4], float l_tot, float m_run, size_t head_off, int head,
                                          int qrow, int Lq, int g, uint16_t *O, float *O32, float *lse_out) {
  const float inv_l = 1.0f / l_tot;
  if (kLse && qrow < Lq) {
    float *orow = O32 + head_off + static_cast<size_t>(qrow) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
        *reinterpret_cast<float4 *>(orow + 32 * db + 8 * grp + 4 * g) =
            make_float4(o[db][4 * grp + 0] * inv_l, o[db][4 * grp + 1] * inv_l, o[db][4 * grp + 2] * inv_l,
                        o[db][4 * grp + 3] * inv_l);
    if (g == 0)
      lse_out[static_cast<size_t>(head) * Lq + qrow] = (__builtin_amdgcn_logf(l_tot) + m_run) * 0.69314718055994531f;
  }
  if (!kLse && qrow < Lq) {
    uint16_t *orow = O + head_off + static_cast<size_t>(qrow) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        uint2 w;
        w.x = pack_bf16x2(o[db][4 * grp + 0] * inv_l, o[db][4 * grp + 1] * inv_l);
        w.y = pack_bf16x2(o[db][4 * grp + 2] * inv_l, o[db][4 * grp + 3] * inv_l);
        *reinterpret_cast<uint2 *>(orow + 32 * db + 8 * grp + 4 * g) = w;
      }
  }
}

// kLse = false: out = softmax(scale q k^T) v rounded to bf16 (h3_attention).
// kLse = true:  out_f32 = the same normalised result in fp32 and lse = the
// natural log of sum_j exp(scale q.k_j) over the Lk keys given (the partial
// form h3_attention_merge combines).  Queries: [H][Lq][D]; keys and values:
// element (h, j, d) at h*kv_stride + j*D + d, j < Lk.
// kVt = true (with kLse = false): V is transposed, element (h, j, d) at
// (h*D + d)*ldv + j (h3_attention_vt); otherwise ldv is unused.
//
// One 8-wave workgroup per unit: block b covers unit unit_base + r, with r
// the XCD-remapped b.
template <bool kLse, bool kVt>
__global__ __launch_bounds__(512) void attn_fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    uint16_t *__restrict__ O, float *__restrict__ O32, float *__restrict__ lse_out, int Lq, int Lk,
    long long kv_stride, int ldv, int n_qtiles, int unit_base, float scale_log2e) {
  static_assert(!(kLse && kVt), "the partial form takes V as [H][Lk][D]");
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[kSlots][kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[kSlots][kTileElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = unit_base + logical;
  const int head = unit / n_qtiles;
  const int qt = unit - head * n_qtiles;
  const int row0 = qt * kUnitRows;
  const size_t head_off = static_cast<size_t>(head) * Lq * D;
  const uint16_t *Qh = Q + head_off;
  const uint16_t *Kh = K + static_cast<size_t>(head) * kv_stride;
  const uint16_t *Vh = V + static_cast<size_t>(head) * (kVt ? static_cast<long long>(D) * ldv : kv_stride);
  const int row_bytes = D * 2;

  // Q^T fragments (B operand): lane holds query row qrow, d = 16c + 8g .. +7.
  const int qrow = row0 + wave * 32 + l32;
  bf16x8 qf[8];
  {
    // Descriptor over this workgroup's rows only: sizes stay below 2^31 bytes
    // for any L the API accepts.
    const int rows_left = Lq - row0 < kUnitRows ? Lq - row0 : kUnitRows;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qh + static_cast<size_t>(row0) * D, rows_left * row_bytes);
#pragma unroll
    for (int c = 0; c < 8; ++c)
      qf[c] = __builtin_bit_cast(bf16x8, bload128(rq, (wave * 32 + l32) * row_bytes + 32 * c + 16 * g));
  }

  const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
  // whole: tile t lies wholly below Lk (a compile-time fact at each call).
  auto dma = [&](const uint16_t *base, int t, const uint16_t *dst, bool is_k, auto whole_c) {
    if (kVt && !is_k)
      dma_vt_tile<kWaves, !decltype(whole_c)::value>(base, t, Lk, ldv, dst, wave, wave_u, lane);
    else
      dma_tile<kWaves>(base, t, Lk, dst, is_k, wave, wave_u, lane);
  };
  const std::integral_constant<bool, true> whole{};
  const std::integral_constant<bool, false> ragged{};
  // Each step issues two loads of V and then two of K.  Waiting until at
  // most one step's loads are outstanding completes all older ones.
  auto dma_wait_all_but_one_pair = [&]() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); };

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m_run = -__builtin_inff();  // running max, base-2 scaled units
  float l_run0 = 0.f, l_run1 = 0.f; // this lane's partial row sums of the bf16 weights

  const int n_kt = (Lk + kBc - 1) / kBc;
  // Steps run in groups of kSlots so that every ring slot is a compile-time
  // constant; the up to kSlots-1 extra tiles lie wholly past Lk, so their
  // weights are exactly 0 and their (zero-filled) V rows add exact zeros.
  const int n_steps = (n_kt + kSlots - 1) / kSlots * kSlots;
  dma(Vh, 0, v_lds[0], false, ragged);
  dma(Kh, 0, k_lds[0], true, ragged);
  dma(Kh, 1, k_lds[1], true, ragged);
  dma(Vh, 1, v_lds[1], false, ragged);
  dma(Kh, 2, k_lds[2], true, ragged);
  dma_wait_all_but_one_pair();   // K tiles 0, 1 and V tile 0 are in LDS (this wave's share)
  __syncthreads();

  int koff[8], voff[4];
  k_offsets(lane, koff);
  v_offsets(lane, voff);
  // V fragment db of k-step bt, and the LDS reads one k-step's fragments take.
  auto vfrag = [&](const uint16_t *vp, int bt, int db) {
    if constexpr (kVt)
      return vread_t(vp, bt, db, l32, g);
    else
      return vread(vp, voff, bt, db);
  };
  constexpr int kVReads = kVt ? 4 : 8;

  f32x16 s_a[2], s_b[2];
  {
    s_a[0] = f32x16{};
    s_a[1] = f32x16{};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      s_a[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(k_lds[0], koff, 0, c), qf[c], s_a[0], 0, 0, 0);
      s_a[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(k_lds[0], koff, 1, c), qf[c], s_a[1], 0, 0, 0);
    }
  }
  mask_tile(s_a, 0, Lk, g);
  // Row max (scaled, base 2) of the tile whose softmax the next step does.
  float mx = lane_half_max(max32(s_a[0], s_a[1])) * scale_log2e;

  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  // One key tile.  Everything that does not feed the matrix cores runs in
  // their shadow, so the two waves sharing a SIMD (kept in step by the
  // barrier) leave the matrix pipe idle only around that barrier:
  //   (1) raise the running max if tile kt's max (found last step) exceeds it;
  //   (2) the loads of V tile kt+2 and K tile kt+3 into their ring slots,
  //       then the scores of tile kt+1 on the matrix cores, interleaved with
  //       tile kt's exponentials;
  //   (3) O += P.V for tile kt, interleaved with tile kt+1's row max;
  //   (4) wait for this wave's loads of V tile kt+1 and K tile kt+2 (issued
  //       one step earlier), then the barrier.
  // V slot (kt+2) % kSlots last held V tile kt-2 (read in step kt-2) and K
  // slot (kt+3) % kSlots K tile kt-1 (read for the scores of step kt-2).
  // Each wave's LDS reads of step j have completed once it is past the
  // barrier ending step j (the wait right after it), so both slots are free
  // two barriers after their last reads.  The barrier itself therefore waits
  // for no LDS read: it is a bare s_barrier (with a compiler memory fence),
  // and the compiler's own full LDS wait before it, which would stall on the
  // P.V reads just issued, is avoided.  R = kt % kSlots, a compile-time value.
  auto step = [&](auto r_c, auto mask_c, int kt, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2]) {
    constexpr int R = decltype(r_c)::value;   // mask_c: whether tile kt+1 may hold keys past Lk
    // K tile kt+1 and V tile kt are visible since the barrier that ended the
    // previous step: the first score fragments are read before the ballot,
    // and the first P.V fragments late in the score phase, so neither read's
    // latency opens its phase.
    const uint16_t *kp = k_lds[(R + 1) % kSlots];
    bf16x8 ka[2][2];
    ka[0][0] = kread(kp, koff, 0, 0);
    ka[0][1] = kread(kp, koff, 1, 0);
    const uint16_t *vp = v_lds[R];
    bf16x8 vf[2][4];
    // (1)  A wave that rescales has extra work before the barrier: it runs
    // the rest of its step at a raised issue priority (s_setprio 1, reset
    // after the barrier), so the other wave on its SIMD yields to it
    // (same-box A/B: +0.9% at H = 7, +0.6% at H = 56; bits unchanged).
    if (__builtin_amdgcn_ballot_w64(mx > m_run) != 0) {
      __builtin_amdgcn_s_setprio(1);
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run0 *= alpha;
      l_run1 *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    const float neg_m = -m_run;

    // (2) K fragments are read one MFMA pair ahead (ping-pong registers).
    // Without the mask, V tile kt+2 is whole (see the loops below).
    if constexpr (decltype(mask_c)::value) {
      dma(Vh, kt + 2, v_lds[(R + 2) % kSlots], false, ragged);
      dma(Kh, kt + 3, k_lds[(R + 3) % kSlots], true, ragged);
    } else {
      dma(Vh, kt + 2, v_lds[(R + 2) % kSlots], false, whole);
      dma(Kh, kt + 3, k_lds[(R + 3) % kSlots], true, whole);
    }
    uint32_t pw[16];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int cur = c & 1, nxt = cur ^ 1;
      if (c < 7) {
        ka[nxt][0] = kread(kp, koff, 0, c + 1);
        ka[nxt][1] = kread(kp, koff, 1, c + 1);
      } else {
#pragma unroll
        for (int db = 0; db < 4; ++db) vf[0][db] = vfrag(vp, 0, db);
      }
      s_nxt[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[cur][0], qf[c], c == 0 ? f32x16{} : s_nxt[0], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int b = c >> 2, i = 4 * (c & 3) + 2 * e;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[b][i], scale_log2e, neg_m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[b][i + 1], scale_log2e, neg_m));
        pw[2 * c + e] = pack_bf16x2(p0, p1);
        if (e == 0)
          l_run0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[2 * c + e]), ones, l_run0, false);
        else
          l_run1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[2 * c + e]), ones, l_run1, false);
      }
      s_nxt[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[cur][1], qf[c], c == 0 ? f32x16{} : s_nxt[1], 0, 0, 0);
      if (c < 7)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // next pair's K reads
      else
        __builtin_amdgcn_sched_group_barrier(0x100, kVReads, 0);   // P.V's first V reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
      __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);              // VALU/TRANS
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
      __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);              // VALU/TRANS
    }

    // (3) pw[4*(2b+t) + 0..3] holds the bf16 weights of keys 32b + 16t + 8g
    // + 0..7, the same keys the transposed V reads deliver for k-step
    // bt = 2b + t.  V fragments are read one k-step ahead (ping-pong).
    if constexpr (decltype(mask_c)::value) mask_tile(s_nxt, kt + 1, Lk, g);
    const float mx_next = lane_half_max(max32(s_nxt[0], s_nxt[1])) * scale_log2e;
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
      const int cur = bt & 1, nxt = cur ^ 1;
      if (bt < 3) {
#pragma unroll
        for (int db = 0; db < 4; ++db) vf[nxt][db] = vfrag(vp, bt + 1, db);
      }
      const uint4 w = make_uint4(pw[4 * bt], pw[4 * bt + 1], pw[4 * bt + 2], pw[4 * bt + 3]);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[cur][db], __builtin_bit_cast(bf16x8, w), o[db], 0, 0, 0);
      if (bt < 3) __builtin_amdgcn_sched_group_barrier(0x100, kVReads, 0);   // next k-step's V reads
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);           // VALU (the max tree)
      }
    }
    mx = mx_next;
    // (4)
    dma_wait_all_but_one_pair();
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_s_setprio(0);
    // This wave's P.V reads of this step land here at the latest, whatever
    // the compiler does with the products that consume them.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  // Groups of steps whose scored tiles (kt+1 .. kt+4) are all whole run
  // without the mask.  A data-dependent branch inside a step splits it into
  // basic blocks that the compiler schedules apart: it then sinks the
  // exponentials below the score products instead of interleaving them
  // (measured: 3% for the full-round launch, 5% for the tail launch).  With
  // V^T the group's V loads (tiles kt+2 .. kt+5) must be whole as well.
  const std::integral_constant<bool, true> masked{};
  const std::integral_constant<bool, false> plain{};
  constexpr int kWholeAhead = kVt ? 6 : 5;
  int kt = 0;
  for (; (kt + kWholeAhead) * kBc <= Lk; kt += kSlots) {
    step(std::integral_constant<int, 0>{}, plain, kt, s_a, s_b);
    step(std::integral_constant<int, 1>{}, plain, kt + 1, s_b, s_a);
    step(std::integral_constant<int, 2>{}, plain, kt + 2, s_a, s_b);
    step(std::integral_constant<int, 3>{}, plain, kt + 3, s_b, s_a);
  }
  for (; kt < n_steps; kt += kSlots) {
    step(std::integral_constant<int, 0>{}, masked, kt, s_a, s_b);
    step(std::integral_constant<int, 1>{}, masked, kt + 1, s_b, s_a);
    step(std::integral_constant<int, 2>{}, masked, kt + 2, s_a, s_b);
    step(std::integral_constant<int, 3>{}, masked, kt + 3, s_b, s_a);
  }
  // Loads of tiles past the end are still in flight: they must land before
  // the workgroup's LDS is released.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const float l_run = l_run0 + l_run1;

  store_row<kLse>(o, lane_half_sum(l_run), m_run, head_off, head, qrow, Lq, g, O, O32, lse_out);
}

// Tail form: one workgroup per kGroups 32-row groups (kGroups = 4: 128 rows,
// 8 waves; kGroups = 2: 64 rows, 4 waves).  Wave w < kGroups, the producer
// of group w, computes the scores, the running max and the bf16 weights P.
// Wave w + kGroups, its consumer, holds O and the row sums: one step later
// it applies each tile's rescale, sums the tile's weights and runs P.V, fed
// through LDS with P and the per-row factor alpha.  Every row sees the same
// operations in the same order as in attn_fwd_kernel (a rescale by exactly 1
// is an identity), so its bits do not change; the split only gives each
// SIMD two waves (kGroups = 4: producer w and consumer w + 4 share SIMD w) or
// one wave of its own (kGroups = 2) where a 256-row unit's 8 waves would not
// fill the CUs.  The producer's step is the longer one, so the consumers
// also issue all tile loads.
//   Step kt: producers score tile kt+1 and weigh tile kt; consumers apply
//   tile kt-1 and load V tile kt+1 (3-slot ring, read in step kt+2) and K
//   tile kt+3 (4-slot ring, read in step kt+2), 16 / kGroups 1-KB pieces each
//   per tensor, waiting for all their older loads before the step's barrier.
//   Every LDS access of a step has completed before that barrier
//   (lgkmcnt(0)), so a slot may be rewritten from the step after its last
//   read on.  K + V + P rings: 64 + 48 + 8 kGroups KB.
template <bool kLse, bool kVt, int kGroups>
__global__ __launch_bounds__(128 * kGroups) void attn_tail_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    uint16_t *__restrict__ O, float *__restrict__ O32, float *__restrict__ lse_out, int Lq, int Lk,
    long long kv_stride, int ldv, int n_qtiles, int unit_base, float scale_log2e) {
  static_assert(!(kLse && kVt), "the partial form takes V as [H][Lk][D]");
  constexpr int kVSlots = 3;
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[kSlots][kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[kVSlots][kTileElems];
  __shared__ __attribute__((aligned(1024))) uint4 p_lds[2][kGroups][4 * 64];   // [slot][group][16 B piece j * 64 + lane]
  __shared__ float a_lds[2][kGroups][32];                                         // [slot][group][row]: alpha

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int grp = wave % kGroups;
  constexpr int kWgPerUnit = kUnitRows / (32 * kGroups);

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = unit_base + logical / kWgPerUnit;
  const int head = unit / n_qtiles;
  const int qt = unit - head * n_qtiles;
  const int row0 = qt * kUnitRows + (logical % kWgPerUnit) * (32 * kGroups);
  if (row0 >= Lq) return;   // the empty half of a ragged last unit (uniform per block)
  const size_t head_off = static_cast<size_t>(head) * Lq * D;
  const uint16_t *Kh = K + static_cast<size_t>(head) * kv_stride;
  const uint16_t *Vh = V + static_cast<size_t>(head) * (kVt ? static_cast<long long>(D) * ldv : kv_stride);
  const int qrow = row0 + grp * 32 + l32;

  const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
  // Only the consumers (waves 4-7) load tiles: four 1-KB pieces each.
  auto dma = [&](const uint16_t *base, int t, const uint16_t *dst, bool is_k) {
    if (kVt && !is_k)
      dma_vt_tile<kGroups, true>(base, t, Lk, ldv, dst, wave - kGroups, wave_u - kGroups, lane);
    else
      dma_tile<kGroups>(base, t, Lk, dst, is_k, wave - kGroups, wave_u - kGroups, lane);
  };
  auto end_step = [&]() {
    // All but this step's loads (16 / kGroups pieces per tensor and wave).
    if constexpr (kGroups == 4)
      asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
  };

  const int n_kt = (Lk + kBc - 1) / kBc;
  const int n_steps = (n_kt + kSlots - 1) / kSlots * kSlots;   // as in attn_fwd_kernel
  if (wave_u >= kGroups) {
    dma(Kh, 0, k_lds[0], true);
    dma(Kh, 1, k_lds[1], true);
    dma(Kh, 2, k_lds[2], true);
    dma(Vh, 0, v_lds[0], false);
    // K tiles 0 and 1 (K tile 2 and V tile 0 may still be in flight).
    if constexpr (kGroups == 4)
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  }
  __syncthreads();

  if (wave_u < kGroups) {
    // Producer: scores, running max and weights of attn_fwd_kernel's step; P
    // and alpha to LDS.
    bf16x8 qf[8];
    {
      const int rows_left = Lq - row0 < 32 * kGroups ? Lq - row0 : 32 * kGroups;
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head_off + static_cast<size_t>(row0) * D, rows_left * (D * 2));
#pragma unroll
      for (int c = 0; c < 8; ++c)
        qf[c] = __builtin_bit_cast(bf16x8, bload128(rq, (grp * 32 + l32) * (D * 2) + 32 * c + 16 * g));
    }
    int koff[8];
    k_offsets(lane, koff);
    float m_run = -__builtin_inff();
    f32x16 s_a[2], s_b[2];
    s_a[0] = f32x16{};
    s_a[1] = f32x16{};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      s_a[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(k_lds[0], koff, 0, c), qf[c], s_a[0], 0, 0, 0);
      s_a[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(k_lds[0], koff, 1, c), qf[c], s_a[1], 0, 0, 0);
    }
    mask_tile(s_a, 0, Lk, g);
    float mx = lane_half_max(max32(s_a[0], s_a[1])) * scale_log2e;

    auto pstep = [&](auto r_c, auto mask_c, int kt, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2]) {
      constexpr int R = decltype(r_c)::value;
      const uint16_t *kp = k_lds[(R + 1) % kSlots];
      bf16x8 ka[2][2];
      ka[0][0] = kread(kp, koff, 0, 0);
      ka[0][1] = kread(kp, koff, 1, 0);
      float alpha = 1.0f;
      if (__builtin_amdgcn_ballot_w64(mx > m_run) != 0) {
        const float m_new = __builtin_fmaxf(m_run, mx);
        alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
      }
      if (g == 0) a_lds[R & 1][grp][l32] = alpha;
      const float neg_m = -m_run;
      uint32_t pw[16];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int cur = c & 1, nxt = cur ^ 1;
        if (c < 7) {
          ka[nxt][0] = kread(kp, koff, 0, c + 1);
          ka[nxt][1] = kread(kp, koff, 1, c + 1);
        }
        s_nxt[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[cur][0], qf[c], c == 0 ? f32x16{} : s_nxt[0], 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int b = c >> 2, i = 4 * (c & 3) + 2 * e;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[b][i], scale_log2e, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[b][i + 1], scale_log2e, neg_m));
          pw[2 * c + e] = pack_bf16x2(p0, p1);
        }
        s_nxt[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[cur][1], qf[c], c == 0 ? f32x16{} : s_nxt[1], 0, 0, 0);
        if (c < 7) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // next pair's K reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
        __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);              // VALU/TRANS
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
        __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);              // VALU/TRANS
      }
      // pw[4j .. 4j+3] feeds the consumer's k-step j: lane-major 16-byte pieces.
      uint4 *pd = &p_lds[R & 1][grp][lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) pd[64 * j] = make_uint4(pw[4 * j], pw[4 * j + 1], pw[4 * j + 2], pw[4 * j + 3]);
      if constexpr (decltype(mask_c)::value) mask_tile(s_nxt, kt + 1, Lk, g);
      mx = lane_half_max(max32(s_nxt[0], s_nxt[1])) * scale_log2e;
      end_step();
    };
    const std::integral_constant<bool, true> masked{};
    const std::integral_constant<bool, false> plain{};
    int kt = 0;
    for (; (kt + 5) * kBc <= Lk; kt += kSlots) {
      pstep(std::integral_constant<int, 0>{}, plain, kt, s_a, s_b);
      pstep(std::integral_constant<int, 1>{}, plain, kt + 1, s_b, s_a);
      pstep(std::integral_constant<int, 2>{}, plain, kt + 2, s_a, s_b);
      pstep(std::integral_constant<int, 3>{}, plain, kt + 3, s_b, s_a);
    }
    for (; kt < n_steps; kt += kSlots) {
      pstep(std::integral_constant<int, 0>{}, masked, kt, s_a, s_b);
      pstep(std::integral_constant<int, 1>{}, masked, kt + 1, s_b, s_a);
      pstep(std::integral_constant<int, 2>{}, masked, kt + 2, s_a, s_b);
      pstep(std::integral_constant<int, 3>{}, masked, kt + 3, s_b, s_a);
    }
    // The row's max for the consumer, in P slot 0 (n_steps is even, so slot
    // 0 was last read in step n_steps - 1).
    float *ed = reinterpret_cast<float *>(&p_lds[0][grp][0]);
    if (g == 0) ed[32 + l32] = m_run;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
  } else {
    // Consumer: l = l * alpha + sum(P), O = O * alpha + P.V, one tile behind
    // its producer; all tile loads.
    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
    int voff[4];
    v_offsets(lane, voff);
    auto vfrag = [&](const uint16_t *vp, int bt, int db) {
      if constexpr (kVt)
        return vread_t(vp, bt, db, l32, g);
      else
        return vread(vp, voff, bt, db);
    };
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    float l_run0 = 0.f, l_run1 = 0.f;
    auto apply = [&](int ps, const uint16_t *vp) {
      const float alpha = a_lds[ps][grp][l32];
      const uint4 *src = &p_lds[ps][grp][lane];
      uint4 pw4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pw4[j] = src[64 * j];
      bf16x8 vf[2][4];
#pragma unroll
      for (int db = 0; db < 4; ++db) vf[0][db] = vfrag(vp, 0, db);
      // Rows whose max did not rise have alpha exactly 1.
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
        l_run0 *= alpha;
        l_run1 *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      }
      const uint32_t pw[16] = {pw4[0].x, pw4[0].y, pw4[0].z, pw4[0].w, pw4[1].x, pw4[1].y, pw4[1].z, pw4[1].w,
                               pw4[2].x, pw4[2].y, pw4[2].z, pw4[2].w, pw4[3].x, pw4[3].y, pw4[3].z, pw4[3].w};
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        l_run0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[i]), ones, l_run0, false);
        l_run1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[i + 1]), ones, l_run1, false);
      }
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const int cur = bt & 1, nxt = cur ^ 1;
        if (bt < 3) {
#pragma unroll
          for (int db = 0; db < 4; ++db) vf[nxt][db] = vfrag(vp, bt + 1, db);
        }
#pragma unroll
        for (int db = 0; db < 4; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[cur][db], __builtin_bit_cast(bf16x8, pw4[bt]), o[db], 0, 0, 0);
      }
    };
    // Step 0 has no tile to apply yet.
    dma(Vh, 1, v_lds[1], false);
    dma(Kh, 3, k_lds[3], true);
    end_step();
    int vs = 0;   // V ring slot of tile kt - 1
    for (int kt = 1; kt < n_steps; ++kt) {
      const int vn = vs == kVSlots - 1 ? 0 : vs + 1;
      const int vi = vn == kVSlots - 1 ? 0 : vn + 1;   // slot of tile kt + 1
      dma(Vh, kt + 1, v_lds[vi], false);
      dma(Kh, kt + 3, k_lds[(kt + 3) % kSlots], true);
      apply((kt - 1) & 1, v_lds[vs]);
      vs = vn;
      end_step();
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
    apply((n_steps - 1) & 1, v_lds[vs]);
    const float *es = reinterpret_cast<const float *>(&p_lds[0][grp][0]);
    store_row<kLse>(o, lane_half_sum(l_run0 + l_run1), es[32 + l32], head_off, head, qrow, Lq, g, O, O32, lse_out);
  }
}

}  // namespace

int64_t attention_grid(int H, int L) {
  return static_cast<int64_t>(H) * ((static_cast<int64_t>(L) + kUnitRows - 1) / kUnitRows);
}

namespace {

// Compute units of the current device, queried once per device and cached
// (the count never changes while the process runs; racing first queries
// store the same value).
hipError_t device_cu_count(int *cus) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && (*cus = cached[dev].load(std::memory_order_relaxed)) > 0) return hipSuccess;
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && dev >= 0 && dev < kMaxDevices) cached[dev].store(*cus, std::memory_order_relaxed);
  return e;
}

// Groups of 32 rows per tail workgroup (a producer and a consumer wave
// each).  Four groups put two waves on each SIMD; two give every wave a SIMD
// of its own, which shortens a group's step but runs half the rows per CU.
// Two pay only when the leftover units are few enough that the tail runs on
// a small share of the CUs anyway (same-box A/B, bit-identical: L = 37726 at
// H = 7, 12 leftover units, 4.913 against 4.985 ms; 51 or 128 leftover units
// ran 8% and 60% slower with two).
int tail_groups(int tail, int cus) { return tail * 16 <= cus ? 2 : 4; }

// Main launch + tail launch.  Units run in rounds of one 8-wave workgroup per
// CU; when the last round would leave at least half the CUs idle (r <= CUs/2
// units left over), those r units instead run as 2r attn_tail_kernel
// workgroups of 128 rows (or 4r of 64 rows, see tail_groups), one per CU,
// after the full rounds (the same stream orders the two launches).  The tail round then keeps every SIMD busy with
// half a round's work.  Which launch a unit lands in depends on H and on the
// device, but a row's arithmetic does not.
template <bool kLse, bool kVt>
hipError_t launch_split(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *out, float *out32,
                        float *lse, int H, int Lq, int Lk, long long kv_stride, int ldv, float scale,
                        hipStream_t stream) {
  const int n_qtiles = (Lq + kUnitRows - 1) / kUnitRows;
  const int units = static_cast<int>(attention_grid(H, Lq));
  int cus = 0;
  hipError_t e = device_cu_count(&cus);
  if (e != hipSuccess) return e;
  const int rem = cus > 0 ? units % cus : 0;
  const int tail = (cus > 0 && rem <= cus / 2) ? rem : 0;
  const int main_units = units - tail;
  const float sl2e = scale * kLog2e;
  if (main_units > 0) {
    hipLaunchKernelGGL((attn_fwd_kernel<kLse, kVt>), dim3(main_units), dim3(512), 0, stream, q, k, v, out, out32,
                       lse, Lq, Lk, kv_stride, ldv, n_qtiles, 0, sl2e);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (tail > 0) {
    if (tail_groups(tail, cus) == 2)
      hipLaunchKernelGGL((attn_tail_kernel<kLse, kVt, 2>), dim3(4 * tail), dim3(256), 0, stream, q, k, v, out, out32,
                         lse, Lq, Lk, kv_stride, ldv, n_qtiles, main_units, sl2e);
    else
      hipLaunchKernelGGL((attn_tail_kernel<kLse, kVt, 4>), dim3(2 * tail), dim3(512), 0, stream, q, k, v, out, out32,
                         lse, Lq, Lk, kv_stride, ldv, n_qtiles, main_units, sl2e);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *out, int H,
                            int L, float scale, hipStream_t stream) {
  return launch_split<false, false>(q, k, v, out, nullptr, nullptr, H, L, L, static_cast<long long>(L) * D, 0,
                                    scale, stream);
}

hipError_t launch_attention_vt(const uint16_t *q, const uint16_t *k, const uint16_t *vt, uint16_t *out, int H,
                               int L, int ldv, float scale, hipStream_t stream) {
  return launch_split<false, true>(q, k, vt, out, nullptr, nullptr, H, L, L, static_cast<long long>(L) * D, ldv,
                                   scale, stream);
}

hipError_t launch_attention_lse(const uint16_t *q, const uint16_t *k, const uint16_t *v, float *out, float *lse,
                                int H, int Lq, int Lk, long long kv_stride, float scale, hipStream_t stream) {
  return launch_split<true, false>(q, k, v, nullptr, out, lse, H, Lq, Lk, kv_stride, 0, scale, stream);
}

// Merge of P partial results: one 32-lane half-wave per (head, row); lane
// holds 4 of the 128 columns.  lse = m + log(sum_p exp(lse_p - m)), out =
// sum_p exp(lse_p - lse) * out_p, rounded once to bf16.  The partial rows are
// read once, bypassing the caches.  kP > 0 fixes P at compile time: every
// part's values are then loaded before any is used, so a thread's loads are
// in flight together (P = 2 at H = 7, L = 32768: 50 us instead of 65 us).
// kP = 0 takes P at run time.  Both forms add in the same order.
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <int kP>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float *__restrict__ outs,
                                                         const float *__restrict__ lses, int P, long long rows,
                                                         uint16_t *__restrict__ out, float *__restrict__ lse_out) {
  const long long row = static_cast<long long>(blockIdx.x) * 8 + (threadIdx.x >> 5);
  const int c = (threadIdx.x & 31) * 4;
  if (row >= rows) return;
  auto part_lse = [&](int p) { return lses[p * rows + row]; };
  auto part_row = [&](int p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(outs + (p * rows + row) * D + c));
  };
  float m = -__builtin_inff();
  float z = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto add = [&](float lp, const f32x4 &x) {
    const float w = (m == -__builtin_inff()) ? 0.f : __expf(lp - m);
    z += w;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, x[e], acc[e]);
  };
  if constexpr (kP > 0) {
    float lv[kP];
    f32x4 xv[kP];
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      lv[p] = part_lse(p);
      xv[p] = part_row(p);
    }
#pragma unroll
    for (int p = 0; p < kP; ++p) m = __builtin_fmaxf(m, lv[p]);
#pragma unroll
    for (int p = 0; p < kP; ++p) add(lv[p], xv[p]);
  } else {
    for (int p = 0; p < P; ++p) m = __builtin_fmaxf(m, part_lse(p));
    for (int p = 0; p < P; ++p) add(part_lse(p), part_row(p));
  }
  const float inv = 1.0f / z;
  uint2 wv;
  wv.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  wv.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<uint2 *>(out + row * D + c) = wv;
  if (lse_out != nullptr && c == 0) lse_out[row] = m + __logf(z);
}

hipError_t launch_attention_merge(const float *outs, const float *lses, int P, uint16_t *out, float *lse_out,
                                  int H, int L, hipStream_t stream) {
  const long long rows = static_cast<long long>(H) * L;
  const dim3 grid(static_cast<unsigned>((rows + 7) / 8)), block(256);
  switch (P) {
    case 1: hipLaunchKernelGGL(attn_merge_kernel<1>, grid, block, 0, stream, outs, lses, P, rows, out, lse_out); break;
    case 2: hipLaunchKernelGGL(attn_merge_kernel<2>, grid, block, 0, stream, outs, lses, P, rows, out, lse_out); break;
    case 3: hipLaunchKernelGGL(attn_merge_kernel<3>, grid, block, 0, stream, outs, lses, P, rows, out, lse_out); break;
    case 4: hipLaunchKernelGGL(attn_merge_kernel<4>, grid, block, 0, stream, outs, lses, P, rows, out, lse_out); break;
    default: hipLaunchKernelGGL(attn_merge_kernel<0>, grid, block, 0, stream, outs, lses, P, rows, out, lse_out);
  }
  return hipGetLastError();
}

}  // namespace h3
