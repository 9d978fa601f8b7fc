// HIP kernels of libpkv for gfx950 (MI355X) and their C-ABI launchers.
//
//  * kv_write_kernel          -- slot-mapping scatter of new K/V rows into the
//                                pool ([MiniPaged-Qwen] §11 slot split, §12
//                                cache write).
//  * decode_write_kernel      -- one decode step's write with its metadata in
//                                the kernel arguments; also publishes the
//                                step's table entries and lengths.
//  * table_update_kernel      -- applies the blocks a batched decode append
//                                opened to a device-resident block table
//                                ([MiniPaged-Qwen] §9.2).
//  * table_rows_kernel        -- copies whole block-table rows between
//                                device tables, scattered or gathered by row
//                                lists (publishing admitted sequences' rows,
//                                the per-sequence table of a prefill batch).
//  * attn_split_kernel        -- decode attention over one context partition
//                                of one (sequence, KV head): block-table walk,
//                                GQA group sharing each K/V tile, fp32 online
//                                softmax ([MiniPaged-Qwen] §13, §14, §17.3).
//  * attn_reduce_kernel       -- merges the partitions' (max, sum,
//                                accumulator) triples into the final rows.
//  * attn_stream_kernel,      -- stream-K decode attention: all sequences'
//    attn_stream8_kernel         tiles laid end to end and cut into equal
//                                ranges, one workgroup per CU (16-bit and
//                                8-bit KV; section "stream-K attention").
//  * attn_stream_step_kernel, -- the same, fused with the step's write (the
//    attn_stream8_step_kernel    8-bit form quantises the new rows).
//  * attn_stream_merge_kernel, -- joins the stream kernel's partial
//    attn_stream_merge_waves_kernel  segments (one wave, or four waves when
//                                the sequences hold many pieces).
//
// Shared work mapping of the attention kernels (64-lane wavefronts):
//  - The K/V pool is read in tiles of 16 consecutive logical tokens (a tile
//    never straddles a physical block because block_size % 16 == 0).
//  - Q.K^T runs on the matrix cores: A = the K tile (16 tokens x D), B = the
//    query group transposed (D x 16 heads, heads >= G zero), one
//    V_MFMA_F32_16x16x32_{BF16,F16} per 32 head-dims (16x16x4 F32 for fp32).
//    The result S^T lands with head = l % 16 and tokens 4*(l/16) ..
//    4*(l/16)+3 in lane l's four accumulators.
//  - P.V: for 16-bit KV with D = 128 it runs on the matrix cores too
//    (softmax_pv16m: eight 16x16x16 MFMAs per tile, P as a 16-bit value plus
//    its 16-bit remainder); otherwise (fp32, other D) on the vector ALUs,
//    lane l owning head-dim chunk (l % 16) of tokens 4*(l/16).., the
//    probabilities reaching it by DPP row broadcasts (softmax_pv).  8-bit KV
//    scales the codes per row (softmax_pv8).
//  - Softmax is online in fp32 and in log2 units (scores pre-multiplied by
//    scale*log2(e), exponentials by v_exp_f32).  The running reference max
//    only moves when a tile's max exceeds it by more than 8 (2^8 headroom),
//    so the accumulator rescale is skipped on almost every tile.
//  - Loads run ahead of use: the split kernel keeps the next tile in a
//    second register stage, the stream kernels fetch whole chunks of tiles
//    (K by buffer loads into LDS, V into registers) before consuming them.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>
#include <type_traits>
#include <stdint.h>

#include <utility>

#include "pkv_fp8_codec.h"
#include "pkv_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kSlack = 8.0f;     // allowed growth of exp2 arguments before a rescale
constexpr int kTile = 16;          // tokens per tile == MFMA M dimension
constexpr int kWave = 64;
#ifndef PKV_SPLIT_WAVES_PER_SIMD
#define PKV_SPLIT_WAVES_PER_SIMD 3
#endif
// Occupancy target of the split kernel (waves per SIMD).  The 16-bit D = 128
// instances fit three waves (<= 168 VGPRs) without spills; fp32 takes two.
template <int DT>
constexpr int split_waves_per_simd() { return DT == PKV_F32 ? 2 : PKV_SPLIT_WAVES_PER_SIMD; }

// ------------------------------------------------------------ conversions
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

template <int DT>
__device__ __forceinline__ void unpack2(uint32_t u, float& a, float& b) {
  if constexpr (DT == PKV_BF16) {
    a = bf16lo(u);
    b = bf16hi(u);
  } else {
    f16x2 h = __builtin_bit_cast(f16x2, u);
    a = static_cast<float>(h.x);
    b = static_cast<float>(h.y);
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <int NDW>
struct Dw { uint32_t w[NDW]; };

template <int NDW>
__device__ __forceinline__ Dw<NDW> load_dw(const void* p) {
  Dw<NDW> r;
  if constexpr (NDW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NDW / 4; ++i) {
      uint4 v = reinterpret_cast<const uint4*>(p)[i];
      r.w[4 * i + 0] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
    }
  } else if constexpr (NDW == 2) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
    static_assert(NDW == 1, "unsupported load width");
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
  return r;
}

// ------------------------------------------------------------ cache write
// One thread moves one 16-byte chunk of one token's K row and the same chunk
// of its V row.  Reads are fully coalesced; each (token, head) row lands as
// one contiguous D*elem-byte segment of the pool.
__global__ void __launch_bounds__(256)
kv_write_kernel(const uint4* __restrict__ key, const uint4* __restrict__ value,
                const int64_t* __restrict__ slot_mapping, int64_t total_chunks,
                int32_t chunks_per_head, int32_t chunks_per_token, int64_t capacity,
                int32_t block_size, int64_t block_stride16, int64_t head_stride16,
                int32_t token_stride16, uint4* __restrict__ key_cache,
                uint4* __restrict__ value_cache) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total_chunks) return;
  const int64_t t = idx / chunks_per_token;
  const int32_t r = static_cast<int32_t>(idx - t * chunks_per_token);
  const int32_t h = r / chunks_per_head;
  const int32_t c = r - h * chunks_per_head;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= capacity) return;
  const int64_t pb = slot / block_size;
  const int64_t off = slot - pb * block_size;
  const int64_t dst = pb * block_stride16 + h * head_stride16 + off * token_stride16 + c;
  key_cache[dst] = key[idx];
  value_cache[dst] = value[idx];
}

// ------------------------------------------------------------ decode-step write
// One decode step's metadata travels in the kernel arguments (no separate
// host-to-device copy): per row i the new token's slot and the row's length
// after the append.  The kernel writes the K/V rows like kv_write_kernel,
// publishes the block holding each row's new token (table entry
// (len - 1) / bs: a block the append opened, [MiniPaged-Qwen] §9.2, or one
// it copied on write) into the device block table, and copies the lengths
// to `lens_out` for the attention launch that follows.
using pkv::kStepRows;
using pkv::StepMeta;

__global__ void __launch_bounds__(256)
decode_write_kernel(StepMeta meta, int32_t n, int32_t row0, const uint4* __restrict__ key,
                    const uint4* __restrict__ value, int32_t chunks_per_head,
                    int32_t chunks_per_token, int64_t capacity, int32_t block_size,
                    int64_t block_stride16, int64_t head_stride16, int32_t token_stride16,
                    uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
                    int32_t* __restrict__ tables, int32_t table_rows, int32_t table_stride,
                    int32_t* __restrict__ lens_out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(n) * chunks_per_token) return;
  const int32_t t = static_cast<int32_t>(idx / chunks_per_token);
  const int32_t r = static_cast<int32_t>(idx - static_cast<int64_t>(t) * chunks_per_token);
  const int64_t slot = meta.slots[t];
  if (r == 0) {
    const int32_t len = meta.lens[t];
    const int32_t row = row0 + t;
    if (lens_out) lens_out[row] = len;
    if (tables && row < table_rows && len > 0 && slot >= 0 && slot < capacity) {
      const int32_t col = (len - 1) / block_size;
      if (col < table_stride) tables[static_cast<int64_t>(row) * table_stride + col] =
          static_cast<int32_t>(slot / block_size);
    }
  }
  if (slot < 0 || slot >= capacity) return;
  const int32_t h = r / chunks_per_head;
  const int32_t c = r - h * chunks_per_head;
  const int64_t pb = slot / block_size;
  const int64_t off = slot - pb * block_size;
  const int64_t dst = pb * block_stride16 + h * head_stride16 + off * token_stride16 + c;
  const int64_t src = static_cast<int64_t>(row0 + t) * chunks_per_token + r;
  key_cache[dst] = key[src];
  value_cache[dst] = value[src];
}

// ------------------------------------------------------------ table update
__global__ void __launch_bounds__(256)
table_update_kernel(int32_t* __restrict__ tables, int32_t num_rows, int32_t stride,
                    const int32_t* __restrict__ rows,
                    const int32_t* __restrict__ lens, const int32_t* __restrict__ new_block,
                    int32_t n, int32_t block_size) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t nb = new_block[i];
  if (nb < 0) return;
  const int32_t row = rows ? rows[i] : i;
  const int32_t col = (lens[i] - 1) / block_size;
  if (row < 0 || row >= num_rows || lens[i] <= 0 || col >= stride) return;
  tables[static_cast<int64_t>(row) * stride + col] = nb;
}

// ------------------------------------------------------------ attention
// Whole rows of int32 block tables: row i of the copy goes from source row
// src_rows[i] (or i) to destination row dst_rows[i] (or i); one thread per
// entry, rows outside either table skipped.
__global__ void __launch_bounds__(256)
table_rows_kernel(int32_t* __restrict__ dst, int32_t dst_stride, int32_t dst_num_rows,
                  const int32_t* __restrict__ dst_rows, const int32_t* __restrict__ src,
                  int32_t src_stride, int32_t src_num_rows, const int32_t* __restrict__ src_rows,
                  int32_t n, int32_t width) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= static_cast<int64_t>(n) * width) return;
  const int32_t i = static_cast<int32_t>(e / width), j = static_cast<int32_t>(e - static_cast<int64_t>(i) * width);
  const int32_t dr = dst_rows ? dst_rows[i] : i;
  const int32_t sr = src_rows ? src_rows[i] : i;
  if (dr < 0 || dr >= dst_num_rows || sr < 0 || sr >= src_num_rows) return;
  dst[static_cast<int64_t>(dr) * dst_stride + j] = src[static_cast<int64_t>(sr) * src_stride + j];
}

struct AttnArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  const int32_t* lens;
  float* ws_ml;      // [B, H_q, P, 2]  (m, l)
  float* ws_acc;     // [B, H_q, P, D]
  void* out;
  int64_t block_stride;   // elements
  int64_t head_stride;    // elements
  int32_t table_stride;
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_seqs;
  int32_t hq;
  int32_t hkv;
  int32_t group;
  int32_t max_len;
  int32_t part_tokens;
  int32_t max_parts;
  int32_t out_dtype;
  float scale_log2;       // scale * log2(e)
};

// Per-dtype / head-dim shape of the lane fragments.
template <int DT, int D>
struct Frag {
  static constexpr int kBytes = (DT == PKV_F32) ? 4 : 2;
  // K tile: lane supplies (D * kBytes / 4) bytes of its token = kDwK dwords.
  static constexpr int kDwK = D * kBytes / 4 / 4;        // dwords per lane
  static constexpr int kW = D / 16;                      // head-dim chunk per P.V lane
  static constexpr int kDwV = kW * kBytes / 4;           // dwords per token row chunk
  // 16-bit, D = 128: K is fetched as whole 256-byte rows (like V) and
  // regrouped into the MFMA operand layout through LDS; every load
  // instruction then covers complete cache lines and can stream past the
  // caches (non-temporal).
  static constexpr bool kRowK = (DT != PKV_F32) && (D == 128);
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ Dw<4> load_nt16(const char* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  Dw<4> r;
  r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  return r;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_void;

// V rows of one tile as the P.V lanes hold them: lane (g4, c16) has the
// head-dim chunk c16 of tokens 4*g4 .. 4*g4+3.
template <int DT, int D>
struct VTile {
  Dw<Frag<DT, D>::kDwV> v[4];
};

// K tile as the MFMA A operand (direct path): lane (g4, c16) has token c16.
template <int DT, int D>
struct KFrag {
  Dw<Frag<DT, D>::kDwK> k;
};

// In every loader, rows of tokens >= nvalid (the unused tail of the last
// block, which may hold anything) are not read: those lanes re-read token 0
// instead, so every value that enters the sums is finite; their scores are
// masked to -inf afterwards.

template <int DT, int D>
__device__ __forceinline__ void load_v(VTile<DT, D>& t, const char* vtile, int nvalid, int lane) {
  using F = Frag<DT, D>;
  const int g4 = lane >> 4, c16 = lane & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tok = 4 * g4 + r < nvalid ? 4 * g4 + r : 0;
    // 32-bit lane offset on a wave-uniform tile base
    const uint32_t off = static_cast<uint32_t>((tok * D + c16 * F::kW) * F::kBytes);
    const char* src = vtile + off;
    if constexpr (F::kRowK) t.v[r] = load_nt16(src);
    else t.v[r] = load_dw<F::kDwV>(src);
  }
}

// Direct path: lane (g4, c16) loads its MFMA operand, token c16.
template <int DT, int D>
__device__ __forceinline__ void load_k_direct(KFrag<DT, D>& t, const char* ktile, int nvalid, int lane) {
  const int g4 = lane >> 4, c16 = lane & 15;
  const int tok = c16 < nvalid ? c16 : 0;
  if constexpr (DT == PKV_F32) {
    // floats d = 16 j + 4 g4 .. +3 for j = 0 .. D/16-1
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      Dw<4> x = load_dw<4>(ktile + (static_cast<int64_t>(tok) * D + 16 * j + 4 * g4) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) t.k.w[4 * j + e] = x.w[e];
    }
  } else {
    // halves d = 32 kk + 8 g4 .. +7 for kk = 0 .. D/32-1
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      Dw<4> x = load_dw<4>(ktile + (static_cast<int64_t>(tok) * D + 32 * kk + 8 * g4) * 2);
#pragma unroll
      for (int e = 0; e < 4; ++e) t.k.w[4 * kk + e] = x.w[e];
    }
  }
}

// Row path (16-bit, D = 128): the K tile (16 rows of 256 bytes) goes from
// HBM straight into LDS with four global_load_lds_dwordx4, each filling one
// KiB: lane l of instruction rr writes slot (l % 16) of row 4 rr + l / 16.
// The lane fetches chunk (slot ^ row) of that row, so chunk c of row r sits
// at slot c ^ r; each instruction still reads four whole rows from HBM.
// The asm statements are compiler-only memory barriers: the LDS writes of the
// DMA are not ordered against ordinary LDS reads by the optimiser, so reads
// of `sk` must not be moved across the issue point in either direction.
template <int DT, int D>
__device__ __forceinline__ void issue_k_rows(const char* ktile, uint4* sk, int nvalid, int lane) {
  const int g4 = lane >> 4, c16 = lane & 15;
  asm volatile("" ::: "memory");
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int row = 4 * rr + g4;
    const int src_row = row < nvalid ? row : 0;
    const uint32_t off = static_cast<uint32_t>(src_row * D * 2 + ((c16 ^ row) * 16));
    __builtin_amdgcn_global_load_lds((global_void*)(ktile + off),
                                     (lds_void*)(sk + rr * 64), 16, 0, 0);
  }
  asm volatile("" ::: "memory");
}

// Reads the staged K rows back in the MFMA operand layout: lane (g4, c16)
// takes chunk 4 kk + g4 (head-dims 32 kk + 8 g4 ..) of row c16.  The 16
// lanes of a group hit 16 different slots, so no two share an LDS bank.
template <int DT, int D>
__device__ __forceinline__ Dw<Frag<DT, D>::kDwK> read_k_rows(const uint4* sk, int lane) {
  const int g4 = lane >> 4, c16 = lane & 15;
  Dw<Frag<DT, D>::kDwK> r;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const uint4 x = sk[c16 * 16 + ((4 * kk + g4) ^ c16)];
    r.w[4 * kk] = x.x; r.w[4 * kk + 1] = x.y; r.w[4 * kk + 2] = x.z; r.w[4 * kk + 3] = x.w;
  }
  return r;
}

// S^T[token 4*g4 + r][head c16] for the lane's 4 tokens from the K operand
// and the query group operand (same head-dim map).
template <int DT, int D>
__device__ __forceinline__ f32x4 qk_mfma(const Dw<Frag<DT, D>::kDwK>& kf,
                                         const Dw<Frag<DT, D>::kDwK>& qf) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (DT == PKV_F32) {
#pragma unroll
    for (int i = 0; i < D / 4; ++i)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kf.w[i]), __uint_as_float(qf.w[i]),
                                                 acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      uint4 a4 = make_uint4(kf.w[4 * kk], kf.w[4 * kk + 1], kf.w[4 * kk + 2], kf.w[4 * kk + 3]);
      uint4 b4 = make_uint4(qf.w[4 * kk], qf.w[4 * kk + 1], qf.w[4 * kk + 2], qf.w[4 * kk + 3]);
      if constexpr (DT == PKV_BF16)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a4),
                                                      __builtin_bit_cast(bf16x8, b4), acc, 0, 0, 0);
      else
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a4),
                                                     __builtin_bit_cast(f16x8, b4), acc, 0, 0, 0);
    }
  }
  return acc;
}

// Broadcast lane H of each 16-lane row to the whole row (DPP row_newbcast).
template <int H>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x150 + H, 0xf, 0xf, false));
}

template <typename F, int... Hs>
__device__ __forceinline__ void for_each_head_impl(F&& f, std::integer_sequence<int, Hs...>) {
  (f(std::integral_constant<int, Hs>{}), ...);
}
// Calls f(std::integral_constant<int, h>) for h = 0 .. N-1.
template <int N, typename F>
__device__ __forceinline__ void for_each_head(F&& f) {
  for_each_head_impl(f, std::make_integer_sequence<int, N>{});
}

// Online softmax + P.V for one tile whose scores are `s`.  Tokens >= nvalid
// of the tile get score -inf, hence probability 0 (their K/V rows were
// replaced by token 0's).  The probability of (head h, token 4*g4+r)
// sits in lane 16*g4 + h; the P.V lanes of row g4 pick it up with a DPP row
// broadcast, so the loop needs neither LDS nor barriers.
template <int DT, int D, int GP>
__device__ __forceinline__ void softmax_pv(const f32x4 s, const VTile<DT, D>& t, int nvalid,
                                           float scale_log2, float& m, float& l,
                                           float (&acc)[GP][Frag<DT, D>::kW], int lane) {
  using F = Frag<DT, D>;
  const int g4 = lane >> 4;
  float x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = (4 * g4 + r < nvalid) ? s[r] * scale_log2 : -INFINITY;
  }
  float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  bm = fmaxf(bm, __shfl_xor(bm, 16));
  bm = fmaxf(bm, __shfl_xor(bm, 32));
  const bool grow = bm > m + kSlack;
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float m_new = fmaxf(m, bm);
    const float a = __builtin_amdgcn_exp2f(m - m_new);   // 0 on the first tile (m = -inf)
    l *= a;
    m = m_new;
    for_each_head<GP>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const float ah = row_bcast<h>(a);
#pragma unroll
      for (int e = 0; e < F::kW; ++e) acc[h][e] *= ah;
    });
  }
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p[r] = __builtin_amdgcn_exp2f(x[r] - m);   // masked tokens: exp2(-inf) = 0
  }
  l += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float vf[F::kW];
    if constexpr (DT == PKV_F32) {
#pragma unroll
      for (int e = 0; e < F::kW; ++e) vf[e] = __uint_as_float(t.v[r].w[e]);
    } else {
#pragma unroll
      for (int e = 0; e < F::kW / 2; ++e) unpack2<DT>(t.v[r].w[e], vf[2 * e], vf[2 * e + 1]);
    }
    for_each_head<GP>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const float ph = row_bcast<h>(p[r]);
#pragma unroll
      for (int e = 0; e < F::kW; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
    });
  }
}

// End of a wave's run over one (sequence, KV head) segment: sums the four
// token groups' (l, acc), then for each of the G query heads writes either
// the normalised output row (`final`) or the raw (m, l, acc) partial to
// workspace slot ws_row0 + h * ws_row_stride.  Lane group g4 writes heads
// g4 and g4 + 4; lane c16 writes head-dim chunk c16.  The accumulator sum
// over the four groups is a reduce-scatter in two exchanges (lanes 32 apart,
// then 16 apart), each lane keeping half of the heads per exchange, so it
// ends with just the two heads it writes: half the lane exchanges of an
// all-reduce and a quarter of its registers.
template <int DT, int D, int GP>
__device__ __forceinline__ void wave_epilogue(float m, float l, float (&acc)[GP][Frag<DT, D>::kW],
                                              int lane, int G, bool final, void* out, int out_dtype,
                                              int64_t out_row0, float* ws_acc, float* ws_ml,
                                              int64_t ws_row0, int64_t ws_row_stride) {
  using F = Frag<DT, D>;
  constexpr int kW = F::kW;
  static_assert(GP <= 8, "two heads per lane group");
  const int g4 = lane >> 4, c16 = lane & 15;
  const bool b1 = (g4 & 2) != 0, b0 = (g4 & 1) != 0;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  auto A = [&](int h, int e) -> float { return h < GP ? acc[h][e] : 0.f; };
  // exchange 1 (g4 bit 1): pair p holds heads h0 = p + (p & 2) and h0 + 2;
  // the lane keeps the one whose bit 1 matches its own
  float k1[4][kW];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int h0 = p + (p & 2), h1 = h0 + 2;
#pragma unroll
    for (int e = 0; e < kW; ++e) {
      if (h0 >= GP) {
        k1[p][e] = 0.f;
        continue;
      }
      const float send = b1 ? A(h0, e) : A(h1, e);
      const float keep = b1 ? A(h1, e) : A(h0, e);
      k1[p][e] = keep + __shfl_xor(send, 32);
    }
  }
  // exchange 2 (g4 bit 0): k2[j] ends as head 4 j + g4
  float k2[2][kW];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int e = 0; e < kW; ++e) {
      if (4 * j >= GP) {
        k2[j][e] = 0.f;
        continue;
      }
      const float send = b0 ? k1[2 * j][e] : k1[2 * j + 1][e];
      const float keep = b0 ? k1[2 * j + 1][e] : k1[2 * j][e];
      k2[j][e] = keep + __shfl_xor(send, 16);
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (4 * j >= GP) continue;
    const int h = 4 * j + g4;
    const float lh = __shfl(l, h);     // lane h holds head h's (m, l)
    const float mh = __shfl(m, h);
    if (h >= G) continue;
    if (final) {
      const int64_t row = out_row0 + h;
      const float inv = lh > 0.f ? 1.0f / lh : 0.f;
      if (out_dtype == PKV_F32) {
        float* o = static_cast<float*>(out) + row * D + c16 * kW;
#pragma unroll
        for (int e = 0; e < kW; ++e) o[e] = k2[j][e] * inv;
      } else {
        uint16_t* o = static_cast<uint16_t*>(out) + row * D + c16 * kW;
#pragma unroll
        for (int e = 0; e < kW; ++e) {
          const float y = k2[j][e] * inv;
          o[e] = (out_dtype == PKV_BF16) ? f32_to_bf16_rne(y)
                                         : __builtin_bit_cast(uint16_t, static_cast<_Float16>(y));
        }
      }
    } else {
      const int64_t slot = ws_row0 + h * ws_row_stride;
      float* w = ws_acc + slot * D + c16 * kW;
#pragma unroll
      for (int e = 0; e < kW; ++e) w[e] = k2[j][e];
      if (c16 == 0) {
        ws_ml[2 * slot + 0] = mh;
        ws_ml[2 * slot + 1] = lh;
      }
    }
  }
}

// P.V accumulator of the 8-bit path, computed on the matrix cores:
// O^T[d][h] += sum_t V^T[d][t] P^T[t][h], one 16x16x16 f16 MFMA per eighth
// of the head dims.  MFMA j maps its row index c to head-dim 8 c + j, so its
// A operand (lane (g4, c16): rows 4 g4 .. 4 g4 + 3 at head-dim 8 c16 + j) is
// byte j of the lane's V codes, and its B operand (lane (g4, c16): head c16,
// tokens 4 g4 ..) is the score layout as it comes out of the Q.K MFMA.
// Lane (g4, c16) ends up with head c16's head-dims 32 g4 .. 32 g4 + 31:
// c[j][i] is head-dim 32 g4 + 8 i + j.  The V codes enter the MFMA as exact
// f16 values.  The weight of token t is its probability p(t) = 2^(x(t) - m)
// (the one the sum l takes) times its V row's scale 2^ev(t), taken relative
// to 2^e, an integer exponent kept per head near the largest exponent of
// those products: c holds the head's accumulator times 2^-e.  The largest
// weight of a segment thus enters near 1 however far apart the row scales
// are, and every change of e is an exact power-of-two rescale.  The 16-bit
// path keeps c relative to m and does not use e.
struct Acc8 {
  f32x4 c[8];
  int e;
};
constexpr int kNoRef = -100000;
constexpr int kSlackE = 8;           // allowed growth of the weights' exponent before a rescale

template <int GP>
struct AccV {
  float a[GP][8];
};

template <int GP>
__device__ __forceinline__ void acc_zero(AccV<GP>& x) {
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) x.a[h][e] = 0.f;
}
__device__ __forceinline__ void acc_zero(Acc8& x) {
#pragma unroll
  for (int j = 0; j < 8; ++j) x.c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  x.e = kNoRef;
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// Max over the lanes c16, c16 + 16, c16 + 32, c16 + 48 (every lane gets it)
// on the vector ALU: the 16-lane row swap pairs rows (0, 1) and (2, 3), the
// 32-lane half swap pairs the halves.
__device__ __forceinline__ float max_over_g4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ int max_over_g4(int x) {
  const auto a = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(x), static_cast<uint32_t>(x), false, false);
  x = max(static_cast<int>(a[0]), static_cast<int>(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(x), static_cast<uint32_t>(x), false, false);
  return max(static_cast<int>(b[0]), static_cast<int>(b[1]));
}

// P.V of the 16-bit stream kernel on the matrix cores (false: on the vector
// ALU with DPP broadcasts, softmax_pv above).
constexpr bool kMfmaPV16 = true;

// Two values as a packed pair of the 16-bit type (element 0 low), rounded
// to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t pack16x2(float x0, float x1) {
  if constexpr (DT == PKV_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{x0, x1}, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, f16x2{static_cast<_Float16>(x0), static_cast<_Float16>(x1)});
}

// Online softmax + P.V for one 16-bit tile with P.V on the matrix cores:
// O^T[d][h] += V^T P^T as eight 16x16x16 MFMAs.  MFMA j maps its row index c
// to head-dim 8 c + j, so its A operand is element j of the lane's V rows
// 4 g4 .. 4 g4 + 3 (head-dims 8 c16 .. + 7, as loaded), and its B operand is
// the score layout (head c16, tokens 4 g4 ..) as it leaves Q.K.  P enters as
// a 16-bit value plus its 16-bit remainder (two MFMAs, P to about 2^-17).
// The accumulator is the 8-bit path's, relative to m (e unused): lane
// (g4, c16) ends with head c16's head-dims 32 g4 .. 32 g4 + 31.
template <int DT>
__device__ __forceinline__ void softmax_pv16m(const f32x4 s, const VTile<DT, 128>& t, int nvalid,
                                              float scale_log2, float& m, float& l, Acc8& acc, int lane) {
  const int g4 = lane >> 4;
  float x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = (4 * g4 + r < nvalid) ? s[r] * scale_log2 : -INFINITY;
  const float bm = max_over_g4(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  if (__builtin_amdgcn_ballot_w64(bm > m + kSlack) != 0) {
    const float m_new = fmaxf(m, bm);
    const float a = __builtin_amdgcn_exp2f(m - m_new);   // this lane's head; 0 on the first tile
    l *= a;
    m = m_new;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc.c[j] *= a;
  }
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(x[r] - m);   // masked tokens: 0
  l += (p[0] + p[1]) + (p[2] + p[3]);
  const uint32_t h01 = pack16x2<DT>(p[0], p[1]), h23 = pack16x2<DT>(p[2], p[3]);
  float q0, q1, q2, q3;
  unpack2<DT>(h01, q0, q1);
  unpack2<DT>(h23, q2, q3);
  const u32x2 bh = {h01, h23};
  const u32x2 bl = {pack16x2<DT>(p[0] - q0, p[1] - q1), pack16x2<DT>(p[2] - q2, p[3] - q3)};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    const int w = j >> 1;
    const u32x2 av = {__builtin_amdgcn_perm(t.v[1].w[w], t.v[0].w[w], sel),
                      __builtin_amdgcn_perm(t.v[3].w[w], t.v[2].w[w], sel)};
    if constexpr (DT == PKV_BF16) {
      acc.c[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, av),
                                                           __builtin_bit_cast(i16x4, bh), acc.c[j], 0, 0, 0);
      acc.c[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, av),
                                                           __builtin_bit_cast(i16x4, bl), acc.c[j], 0, 0, 0);
    } else {
      acc.c[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, av),
                                                       __builtin_bit_cast(f16x4, bh), acc.c[j], 0, 0, 0);
      acc.c[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, av),
                                                       __builtin_bit_cast(f16x4, bl), acc.c[j], 0, 0, 0);
    }
  }
}

// End of a segment with the MFMA P.V: lane (g4, c16) holds head c16's
// head-dims 32 g4 .. + 31; the four token groups' sums l are added, and each
// lane of a real head (c16 < G) writes its 32 values (normalised output, or
// the partial with its (m, l) in workspace slot ws_row0 + c16 * ws_row_stride).
// REF: the accumulator holds the partial times 2^-e (8-bit rows).
template <bool REF>
__device__ __forceinline__ void wave_epilogue8(float m, float l, const Acc8& acc, int lane, int G,
                                               bool final, void* out, int out_dtype,
                                               int64_t out_row0, float* ws_acc, float* ws_ml,
                                               int64_t ws_row0, int64_t ws_row_stride = 1) {
  constexpr int D = 128;
  const int g4 = lane >> 4, c16 = lane & 15;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (c16 >= G) return;
  float v[32];
  if constexpr (REF) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) v[8 * i + j] = __builtin_amdgcn_ldexpf(acc.c[j][i], acc.e);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) v[8 * i + j] = acc.c[j][i];
  }
  if (final) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const int64_t o = (out_row0 + c16) * D + 32 * g4;
    if (out_dtype == PKV_F32) {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + o);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        dst[k] = make_float4(v[4 * k] * inv, v[4 * k + 1] * inv, v[4 * k + 2] * inv, v[4 * k + 3] * inv);
    } else {
      uint32_t w[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float y0 = v[2 * k] * inv, y1 = v[2 * k + 1] * inv;
        const uint32_t h0 = out_dtype == PKV_BF16 ? f32_to_bf16_rne(y0)
                                                  : __builtin_bit_cast(uint16_t, static_cast<_Float16>(y0));
        const uint32_t h1 = out_dtype == PKV_BF16 ? f32_to_bf16_rne(y1)
                                                  : __builtin_bit_cast(uint16_t, static_cast<_Float16>(y1));
        w[k] = h0 | (h1 << 16);
      }
      uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + o);
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[k] = make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
    }
  } else {
    const int64_t slot = ws_row0 + c16 * ws_row_stride;
    float4* dst = reinterpret_cast<float4*>(ws_acc + slot * D + 32 * g4);
#pragma unroll
    for (int k = 0; k < 8; ++k) dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
    if (g4 == 0) {
      ws_ml[2 * slot + 0] = m;
      ws_ml[2 * slot + 1] = l;
    }
  }
}

template <int DT, int D, int GP>
__global__ void __launch_bounds__(kWave, split_waves_per_simd<DT>())
attn_split_kernel(AttnArgs a) {
  using F = Frag<DT, D>;
  const int lane = threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;
  // workgroup -> (partition, sequence, kv head), partition slowest
  const int wg = blockIdx.x;
  const int kvh = wg % a.hkv;
  const int b = (wg / a.hkv) % a.num_seqs;
  const int p = wg / (a.hkv * a.num_seqs);
  int L = a.lens[b];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int G = a.group;
  const int64_t out_row0 = static_cast<int64_t>(b) * a.hq + static_cast<int64_t>(kvh) * G;
  if (L == 0) {
    if (p != 0) return;
    for (int i = lane; i < G * D; i += kWave) {
      const int64_t o = out_row0 * D + i;
      if (a.out_dtype == PKV_F32) static_cast<float*>(a.out)[o] = 0.f;
      else static_cast<uint16_t*>(a.out)[o] = 0;
    }
    return;
  }
  // The sequence's ceil(L / part_tokens) partitions split its 16-token tiles
  // evenly (they differ by at most one tile), so partitions of one launch
  // carry nearly equal work.
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (p >= nparts) return;
  const int ntiles_seq = (L + kTile - 1) / kTile;
  const int t0 = kTile * static_cast<int>((static_cast<int64_t>(p) * ntiles_seq) / nparts);
  const int t1 = min(L, kTile * static_cast<int>((static_cast<int64_t>(p + 1) * ntiles_seq) / nparts));

  // query group as the MFMA B operand: head c16, same head-dim map as K
  Dw<F::kDwK> qf;
  {
    const int head = c16 < G ? c16 : 0;
    const char* qrow = static_cast<const char*>(a.q) + (out_row0 + head) * D * F::kBytes;
    if constexpr (DT == PKV_F32) {
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        Dw<4> x = load_dw<4>(qrow + (16 * j + 4 * g4) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) qf.w[4 * j + e] = x.w[e];
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        Dw<4> x = load_dw<4>(qrow + (32 * kk + 8 * g4) * 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) qf.w[4 * kk + e] = x.w[e];
      }
    }
    if (c16 >= G) {
#pragma unroll
      for (int i = 0; i < F::kDwK; ++i) qf.w[i] = 0u;
    }
  }

  const int bs = a.block_size;
  const int32_t* trow = a.tables + static_cast<int64_t>(b) * a.table_stride;
  const char* kc = static_cast<const char*>(a.kc);
  const char* vc = static_cast<const char*>(a.vc);
  const int64_t head_off = static_cast<int64_t>(kvh) * a.head_stride;

  // The partition's slice of the block table is staged in LDS once, so the
  // tile loop reads it with LDS loads (counted apart from the K/V loads and
  // never forcing them to drain).
  extern __shared__ int32_t sh_tbl[];
  __shared__ uint4 sk_buf[F::kRowK ? 256 : 1];
  uint4* sk = sk_buf;
  const int lb0 = t0 / bs;
  const int lb1 = (t1 - 1) / bs;
  for (int j = lane; j <= lb1 - lb0; j += kWave) sh_tbl[j] = trow[lb0 + j];
  __syncthreads();
  // Element offset of tile i.  A table entry outside [0, num_blocks) is
  // clamped into the pool: the kernel never leaves the pool, and the result
  // for such a (caller-broken) table is unspecified.
  auto tile_addr = [&](int i) -> int64_t {
    const int tok = t0 + i * kTile;
    const int lb = tok / bs;
    int pb = __builtin_amdgcn_readfirstlane(sh_tbl[lb - lb0]);
    pb = pb < 0 ? 0 : (pb >= a.num_blocks ? a.num_blocks - 1 : pb);
    const int off = tok - lb * bs;
    return static_cast<int64_t>(pb) * a.block_stride + head_off + static_cast<int64_t>(off) * D;
  };

  float m = -INFINITY;
  float l = 0.f;
  float acc[GP][F::kW];
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int e = 0; e < F::kW; ++e) acc[h][e] = 0.f;
  // 16-bit KV with D = 128: P.V on the matrix cores (softmax_pv16m); fp32
  // and D = 64 keep the vector-ALU P.V
  constexpr bool MPV = F::kRowK && kMfmaPV16 && D == 128 && DT != PKV_F32;
  Acc8 accm;
  acc_zero(accm);
  auto step = [&](const f32x4& sc, const VTile<DT, D>& v, int nvalid) {
    if constexpr (MPV) softmax_pv16m<DT>(sc, v, nvalid, a.scale_log2, m, l, accm, lane);
    else softmax_pv<DT, D, GP>(sc, v, nvalid, a.scale_log2, m, l, acc, lane);
  };

  const int ntiles = (t1 - t0 + kTile - 1) / kTile;
  const int last = ntiles - 1;
  auto nvalid_of = [&](int i) { return min(kTile, t1 - t0 - i * kTile); };
  // Loads past the last tile are issued with the index clamped (re-reading
  // the tile just fetched, which the caches hold), so the loop has no
  // conditional loads and the waits stay exact.
  if constexpr (F::kRowK) {
    // Tile i+1 (K into LDS, V into registers) is fetched while tile i's
    // softmax and P.V run; the K operand of tile i is read out of LDS first.
    VTile<DT, D> va, vb;
    {
      const int64_t e0 = tile_addr(0) * F::kBytes;
      issue_k_rows<DT, D>(kc + e0, sk, nvalid_of(0), lane);
      load_v<DT, D>(va, vc + e0, nvalid_of(0), lane);
    }
    for (int i = 0; i < ntiles; i += 2) {
      const int ib = min(i + 1, last);
      const int ia = min(i + 2, last);
      f32x4 sc = qk_mfma<DT, D>(read_k_rows<DT, D>(sk, lane), qf);
      __builtin_amdgcn_s_waitcnt(0xc07f);   // LDS reads of tile i done before it is refilled
      {
        const int64_t eb = tile_addr(ib) * F::kBytes;
        issue_k_rows<DT, D>(kc + eb, sk, nvalid_of(ib), lane);
        load_v<DT, D>(vb, vc + eb, nvalid_of(ib), lane);
      }
      step(sc, va, nvalid_of(i));
      if (i + 1 < ntiles) {
        sc = qk_mfma<DT, D>(read_k_rows<DT, D>(sk, lane), qf);
        __builtin_amdgcn_s_waitcnt(0xc07f);
        const int64_t ea = tile_addr(ia) * F::kBytes;
        issue_k_rows<DT, D>(kc + ea, sk, nvalid_of(ia), lane);
        load_v<DT, D>(va, vc + ea, nvalid_of(ia), lane);
        step(sc, vb, nvalid_of(i + 1));
      }
    }
    // the last (clamped) K fetch into LDS must land before the wave can exit
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    // Direct path: two register stages, tile i+1 in flight while tile i is
    // consumed.
    KFrag<DT, D> ka, kb;
    VTile<DT, D> va, vb;
    {
      const int64_t e0 = tile_addr(0) * F::kBytes;
      load_k_direct<DT, D>(ka, kc + e0, nvalid_of(0), lane);
      load_v<DT, D>(va, vc + e0, nvalid_of(0), lane);
    }
    for (int i = 0; i < ntiles; i += 2) {
      const int ib = min(i + 1, last);
      const int ia = min(i + 2, last);
      {
        const int64_t eb = tile_addr(ib) * F::kBytes;
        load_k_direct<DT, D>(kb, kc + eb, nvalid_of(ib), lane);
        load_v<DT, D>(vb, vc + eb, nvalid_of(ib), lane);
      }
      softmax_pv<DT, D, GP>(qk_mfma<DT, D>(ka.k, qf), va, nvalid_of(i), a.scale_log2, m, l, acc, lane);
      {
        const int64_t ea = tile_addr(ia) * F::kBytes;
        load_k_direct<DT, D>(ka, kc + ea, nvalid_of(ia), lane);
        load_v<DT, D>(va, vc + ea, nvalid_of(ia), lane);
      }
      if (i + 1 < ntiles)
        softmax_pv<DT, D, GP>(qk_mfma<DT, D>(kb.k, qf), vb, nvalid_of(i + 1), a.scale_log2, m, l,
                              acc, lane);
    }
  }

  if constexpr (MPV)
    wave_epilogue8<false>(m, l, accm, lane, G, nparts == 1, a.out, a.out_dtype, out_row0, a.ws_acc, a.ws_ml,
                   out_row0 * a.max_parts + p, a.max_parts);
  else
    wave_epilogue<DT, D, GP>(m, l, acc, lane, G, nparts == 1, a.out, a.out_dtype, out_row0, a.ws_acc,
                             a.ws_ml, out_row0 * a.max_parts + p, a.max_parts);
}

// Split-K merge: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p with
// M = max_p m_p.  One workgroup of four waves per (sequence, query head);
// sequences with a single partition were finished by attn_split_kernel.
// Every wave reads all the (m, l) pairs, 64 partitions per load round, and
// reduces M and the denominator across its lanes; wave w then sums the
// weighted accumulators of partitions w, w + 4, w + 8, ... (eight loads in
// flight per lane), and wave 0 adds the four wave sums from LDS in a fixed
// order.  The summation order depends only on the partition count, so the
// result is reproducible bit for bit.
constexpr int kReduceWaves = 4;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ void __launch_bounds__(kWave * kReduceWaves)
attn_reduce_kernel(AttnArgs a) {
  constexpr int kPer = D / kWave;
  __shared__ float wsum[kReduceWaves][D];
  const int qh = blockIdx.x % a.hq;
  const int b = blockIdx.x / a.hq;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  int L = a.lens[b];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;
  const int64_t row = static_cast<int64_t>(b) * a.hq + qh;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml + row * a.max_parts * 2);
  const float* acc = a.ws_acc + row * a.max_parts * D;
  float M = -INFINITY;
  for (int p = lane; p < nparts; p += kWave) M = fmaxf(M, ml[p].x);
  M = wave_max(M);
  float den = 0.f;
  for (int p = lane; p < nparts; p += kWave) {
    const float2 x = ml[p];
    den = fmaf(x.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x.x - M), x.y, den);
  }
  den = wave_sum(den);
  float num[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) num[e] = 0.f;
  constexpr int kBatch = 8;
  for (int p0 = wave; p0 < nparts; p0 += kReduceWaves * kBatch) {
    float w[kBatch], v[kBatch][kPer];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = min(p0 + u * kReduceWaves, nparts - 1);
      const float mp = ml[p].x;
      w[u] = (p0 + u * kReduceWaves < nparts && mp != -INFINITY) ? __builtin_amdgcn_exp2f(mp - M) : 0.f;
#pragma unroll
      for (int e = 0; e < kPer; ++e) v[u][e] = acc[static_cast<int64_t>(p) * D + e * kWave + lane];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
#pragma unroll
      for (int e = 0; e < kPer; ++e) num[e] = fmaf(w[u], v[u][e], num[e]);
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) wsum[wave][e * kWave + lane] = num[e];
  __syncthreads();
  if (wave != 0) return;
  const float inv = den > 0.f ? 1.0f / den : 0.f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int d = e * kWave + lane;
    float t = wsum[0][d];
#pragma unroll
    for (int k = 1; k < kReduceWaves; ++k) t += wsum[k][d];
    const int64_t o = row * D + d;
    const float y = t * inv;
    if (a.out_dtype == PKV_F32) static_cast<float*>(a.out)[o] = y;
    else if (a.out_dtype == PKV_BF16) static_cast<uint16_t*>(a.out)[o] = f32_to_bf16_rne(y);
    else static_cast<uint16_t*>(a.out)[o] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(y));
  }
}

// ------------------------------------------------------------ stream-K attention
// The launch's 16-token tiles, with the tiles of all sequences laid end to
// end (sequence b owns tiles [S_b, S_b + T_b), T_b = ceil(L_b / 16)), are
// cut into W equal contiguous ranges: range r takes tiles [r*T/W, (r+1)*T/W),
// so every range carries the same number of tiles whatever the mix of
// context lengths.  One workgroup per CU holds R consecutive ranges.  A job
// is one (range, KV head), and two waves share it: the front worker takes
// the tiles before a split tile x, the back worker those from x on.  The
// two waves on one SIMD do not progress at the same rate (the one in the
// second wave slot runs markedly slower under this load), so the split
// gives the slot-0 wave the larger share (part_split).  x depends only on
// the range and the job, so results are bitwise reproducible and the merge
// kernel recomputes it.  Each worker walks its part in chunks of up to
// kStreamChunk tiles of one sequence (a chunk ends at a sequence end or at
// the part's end).  When every KV head has two waves (2 * R * H_kv <= 8)
// each job has its own pair; otherwise (H_kv > 4) each wave is the front
// worker of job j and then the back worker of job (j + 4) mod H_kv.
//
// Every maximal run of one worker's tiles in one sequence is a segment; a
// segment that covers its whole sequence writes the normalised output,
// other segments leave a (max, sum, accumulator) partial in one of four
// slots of their job: 0 = the front worker's segment starting at the range
// start, 1 = its segment ending at the split tile, 2 = the back worker's
// segment ending at the range end, 3 = its segment starting at the split
// tile.  The merge kernel finds the pieces of each sequence from the range
// bounds and the split tiles.  16-bit KV, D = 128, H_kv <= 8, G <= 8.
struct StreamArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  const int32_t* lens;
  float* ws_acc;     // [W, 4, H_q, D]   (W = num_ranges)
  float* ws_ml;      // [W, 4, H_q, 2]
  int32_t* ws_S;     // [B + 1] tile prefix sums, stored by workgroup 0 for the merge
  void* out;
  int64_t block_stride;
  int64_t head_stride;
  int32_t table_stride;
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_seqs;
  int32_t hq;
  int32_t hkv;
  int32_t group;
  int32_t max_len;
  int32_t out_dtype;
  int32_t range_cap;     // tiles one workgroup may hold
  int32_t num_ranges;    // W
  int32_t ranges_per_wg; // R
  int32_t slot0_share;   // percent of a split job's tiles for its slot-0 worker
  float scale_log2;
  // decode-step form only: the step's new rows [B, H_kv, D] and where the
  // step's write goes (pool, table of table_rows rows, device lengths)
  const void* new_k;
  const void* new_v;
  void* kc_w;
  void* vc_w;
  int32_t* tables_w;
  int32_t table_rows;
  int32_t* lens_out;
  // 8-bit KV only: scale bytes of K and V rows, at ks + pb * sblock_stride
  // + h * shead_stride + off
  const uint8_t* ks;
  const uint8_t* vs;
  int64_t sblock_stride;
  int64_t shead_stride;
  uint8_t* ks_w;     // decode-step form of the 8-bit path: where the new rows' scale bytes go
  uint8_t* vs_w;
};

constexpr int kStreamMaxHeads = 8;
constexpr int kStreamMaxWaves = 8;
constexpr int kStreamSlots = 4;          // partial slots per job
// Percent of a job's chunks taken by the worker in SIMD wave slot 0 when its
// partner is in slot 1: under this load the second slot's wave takes longer
// per chunk (about 26 %, measured per wave with the real-time counter, when
// the P.V ran on the vector ALU).  With both products on the matrix cores a
// sweep of 52 .. 66 put the kernel's time lowest at 60 : 40.  The 8-bit
// kernel's tiles cost less per byte in flight, so it has its own share: a
// sweep of 52 .. 64 put it lowest at 56 : 44.
constexpr int kSlot0Share = 60;
constexpr int kSlot0Share8 = 56;

// How many of a job's n tiles its front worker takes.  The front worker is
// wave `job` of the workgroup, the back worker wave J + job (paired: two
// waves per job) or the wave that runs job's back after its own front
// (J - 4 + job) mod J.  Waves 0-3 sit in SIMD wave slot 0, waves 4-7 in
// slot 1; the slot-0 worker takes `share` percent of the tiles when its
// partner is in slot 1, else the split is even.
__device__ __forceinline__ int part_split(int n, int job, int J, bool paired, int share) {
  const int fw = job;
  const int bw = paired ? J + job : (job + J - 4 % J) % J;
  if ((fw >> 2) == (bw >> 2)) return (n + 1) / 2;
  return (fw >> 2) == 0 ? (n * share + 50) / 100 : (n * (100 - share) + 50) / 100;
}
constexpr int kStreamMaxRanges = 1024;   // W bound (merge kernel's piece list)

__device__ __forceinline__ int clamp_len(int L, int max_len) {
  return L < 0 ? 0 : (L > max_len ? max_len : L);
}

// Largest b in [0, B) with S[b] <= g (S non-decreasing, S[0] = 0 <= g < S[B]);
// that b has T_b > 0 and owns tile g.
__device__ __forceinline__ int seq_of_tile(const int32_t* S, int B, int g) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (S[mid] <= g) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Exclusive prefix sums of T_b into S[0..B], and the clamped context
// lengths into Ls[0..B), by one wave.
template <typename LenOf>
__device__ __forceinline__ void tile_prefix(LenOf lens, int B, int max_len, int32_t* S,
                                            int32_t* Ls, int lane) {
  const int per = (B + kWave - 1) / kWave;
  const int b0 = min(B, lane * per), b1 = min(B, b0 + per);
  int part = 0;
  for (int b = b0; b < b1; ++b) part += (clamp_len(lens(b), max_len) + kTile - 1) / kTile;
  int incl = part;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  int run = incl - part;
  for (int b = b0; b < b1; ++b) {
    const int L = clamp_len(lens(b), max_len);
    S[b] = run;
    Ls[b] = L;
    run += (L + kTile - 1) / kTile;
  }
  if (lane == kWave - 1) S[B] = incl;
}

// A value every lane of the wave holds alike, moved to a scalar register.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint64_t u = static_cast<uint64_t>(x);
  return static_cast<int64_t>(static_cast<uint64_t>(static_cast<uint32_t>(uni(static_cast<int>(u)))) |
                              (static_cast<uint64_t>(static_cast<uint32_t>(uni(static_cast<int>(u >> 32)))) << 32));
}
struct TileOff8 {
  int64_t e;   // element (byte) offset of the tile's first code row
  int64_t s;   // offset of its first scale byte
};

// Tile ranges: range r starts at tile r*T/W; tile g lies in range owner(g).
// Both in 32-bit unsigned arithmetic when T * W fits (every product below
// is at most T * W), else in 64-bit: the same quotients either way.
__device__ __forceinline__ int range_start(int64_t r, int T, int W) {
  if (static_cast<uint64_t>(T) * static_cast<uint64_t>(W) <= 0xffffffffull)
    return static_cast<int>(static_cast<uint32_t>(r) * static_cast<uint32_t>(T) / static_cast<uint32_t>(W));
  return static_cast<int>((r * T) / W);
}
__device__ __forceinline__ int range_owner(int g, int T, int W) {
  if (static_cast<uint64_t>(T) * static_cast<uint64_t>(W) <= 0xffffffffull)
    return static_cast<int>((static_cast<uint32_t>(g + 1) * static_cast<uint32_t>(W) - 1u) /
                            static_cast<uint32_t>(T));
  return static_cast<int>((static_cast<int64_t>(g + 1) * W - 1) / T);
}

// Buffer-resource loads of one 16-row tile (16-bit, D = 128: rows of 256
// bytes).  The resource covers only the tile's first `nvalid` rows, so the
// hardware range check returns zeros for the rows past the context instead
// of whatever the block's unused tail holds; every lane's offset is then a
// constant of its lane, with the tile base in scalar registers.
constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped) buffer, 32-bit data format
constexpr int kCacheNT = 2;              // non-temporal cache policy

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* tile, int nvalid) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(tile), static_cast<short>(0),
                                           nvalid * 256, kRsrcWord3);
}

// K rows into LDS, swizzled as issue_k_rows lays them out: lane l of
// instruction rr fetches chunk ((l % 16) ^ row) of row 4 rr + l / 16.
__device__ __forceinline__ void issue_k_rows_buf(const char* ktile, uint4* sk, int nvalid, int lane) {
  const int g4 = lane >> 4, c16 = lane & 15;
  const __amdgpu_buffer_rsrc_t rs = tile_rsrc(ktile, nvalid);
  asm volatile("" ::: "memory");
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int row = 4 * rr + g4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(sk + rr * 64), 16,
                                             row * 256 + ((c16 ^ row) << 4), 0, 0, 0);
  }
  asm volatile("" ::: "memory");
}

// V rows as the P.V lanes hold them: lane (g4, c16) takes chunk c16 of rows
// 4 g4 .. 4 g4 + 3 (each instruction reads four whole rows).
template <int DT>
__device__ __forceinline__ void load_v_buf(VTile<DT, 128>& t, const char* vtile, int nvalid, int lane) {
  const int g4 = lane >> 4, c16 = lane & 15;
  const __amdgpu_buffer_rsrc_t rs = tile_rsrc(vtile, nvalid);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, (4 * g4 + r) * 256 + (c16 << 4), 0, kCacheNT);
    t.v[r].w[0] = v.x; t.v[r].w[1] = v.y; t.v[r].w[2] = v.z; t.v[r].w[3] = v.w;
  }
}

// A chunk's K rows sit in LDS and its V rows in registers while the next
// chunk is being fetched, so each wave keeps up to kStreamChunk * 8 KiB in
// flight during its compute.
constexpr int kStreamChunk = 2;

// ---- 8-bit KV blocks (PKV_FP8_E4M3): D = 128 one-byte E4M3 codes per row
// and one E8M0 scale byte per row (value 2^(byte - 127); the encoding is in
// pkv_fp8.hip).  A tile is 2 KiB of codes; chunks stay at two tiles (four
// measured slower: the extra per-tile addresses and buffer descriptors
// spill scalar registers).  The hardware conversion on gfx950 reads the
// codes as OCP E4M3 (checked code by code against the definition).
constexpr int kStreamChunk8 = 2;

struct VTile8 {
  uint32_t w[4][2];   // lane (g4, c16): codes 8 c16 .. 8 c16 + 7 of rows 4 g4 + r
  uint32_t ks;        // K scale bytes of rows 4 g4 .. 4 g4 + 3
  uint32_t vs;        // V scale bytes of the same rows
};

// K rows (128 bytes each) into LDS: instruction rr covers rows 8 rr .. 8 rr
// + 7; lane l fetches chunk (l % 8) ^ (row % 8) of row 8 rr + l / 8, so
// chunk c of row r sits at slot c ^ (r % 8).  Rows past nvalid read zeros.
__device__ __forceinline__ void issue_k_rows8(const char* ktile, uint4* sk, int nvalid, int lane) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(ktile), static_cast<short>(0), nvalid * 128, kRsrcWord3);
  const int r8 = lane >> 3, c8 = lane & 7;
  asm volatile("" ::: "memory");
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int row = 8 * rr + r8;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(sk + rr * 64), 16,
                                             row * 128 + ((c8 ^ (row & 7)) << 4), 0, 0, 0);
  }
  asm volatile("" ::: "memory");
}

// V codes as the P.V lanes hold them, and the tile's scale bytes (the 16
// bytes of a tile are always inside the block, written or not).
__device__ __forceinline__ void load_v_buf8(VTile8& t, const char* vtile, const uint8_t* ksc,
                                            const uint8_t* vsc, int nvalid, int lane) {
  const int g4 = lane >> 4, c16 = lane & 15;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(vtile), static_cast<short>(0), nvalid * 128, kRsrcWord3);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, (4 * g4 + r) * 128 + (c16 << 3), 0, kCacheNT);
    t.w[r][0] = v.x;
    t.w[r][1] = v.y;
  }
  t.ks = *reinterpret_cast<const uint32_t*>(ksc + 4 * g4);
  t.vs = *reinterpret_cast<const uint32_t*>(vsc + 4 * g4);
}

// Two float32 of code values (exact in 16 bits) packed as the MFMA's 16-bit type.
// Two E4M3 codes (bytes 0-1 of w, or 2-3 when HI) as a packed pair of the
// 16-bit type, by the hardware conversion with scale 1 (exact: every E4M3
// value is a bf16 and an f16 number).
template <int DT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_16(uint32_t w) {
  if constexpr (DT == PKV_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// The staged K codes of row c16 as the MFMA operand: lane (g4, c16) takes
// bytes 32 g4 .. 32 g4 + 31 of its row; step kk uses bytes 32 g4 + 8 kk ..
// + 7 (the query operand is staged with the same head-dim map).
template <int DT>
__device__ __forceinline__ Dw<16> read_k_rows8(const uint4* sk, int lane) {
  const int g4 = lane >> 4, c16 = lane & 15;
  const uint4 A = sk[c16 * 8 + ((2 * g4) ^ (c16 & 7))];
  const uint4 Bv = sk[c16 * 8 + ((2 * g4 + 1) ^ (c16 & 7))];
  const uint32_t w[8] = {A.x, A.y, A.z, A.w, Bv.x, Bv.y, Bv.z, Bv.w};
  Dw<16> r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    r.w[2 * i] = fp8x2_to_16<DT, false>(w[i]);
    r.w[2 * i + 1] = fp8x2_to_16<DT, true>(w[i]);
  }
  return r;
}

// Online softmax + P.V for one 8-bit tile: the score of token t is the code
// dot product times 2^ek(t) (into the exp2 argument's factor), x(t) in log2
// units.  The sum l and the MFMA take the same p(t) = 2^(x(t) - m); the
// MFMA takes it times 2^(ev(t) - e) for V row t's codes, as an f16 value
// plus its f16 remainder (two MFMAs, the weight to about 2^-22 of the
// segment's largest).  e follows the largest ev(t) + floor(log2 p(t)) (the
// exponent field of p) with the slack kSlackE, and drops by the whole
// powers of two by which a new maximum m shrinks the products, so later
// weights keep their precision.
__device__ __forceinline__ void softmax_pv8(const f32x4 s, const VTile8& t, int nvalid,
                                            float scale_log2, float& m, float& l, Acc8& acc,
                                            int lane) {
  const int g4 = lane >> 4;
  float x[4];
  int ev[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool valid = 4 * g4 + r < nvalid;
    const int ek = static_cast<int>((t.ks >> (8 * r)) & 0xffu) - 127;
    // rows past nvalid: p = 0, and the smallest exponent, so they never set e
    ev[r] = valid ? static_cast<int>((t.vs >> (8 * r)) & 0xffu) - 127 : -127;
    x[r] = valid ? s[r] * __builtin_amdgcn_ldexpf(scale_log2, ek) : -INFINITY;
  }
  const float bm = max_over_g4(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  if (__builtin_amdgcn_ballot_w64(bm > m + kSlack) != 0) {
    const float m_new = fmaxf(m, bm);
    const float a = __builtin_amdgcn_exp2f(m - m_new);   // this lane's head; 0 on the first tile
    // whole powers of two of the shrink, at most 512 (a is 0 beyond that)
    const int dn = m == -INFINITY ? 0 : static_cast<int>(__builtin_floorf(fminf(m_new - m, 512.f)));
    const float ac = __builtin_amdgcn_ldexpf(a, dn);      // in (1/2, 1], or 0
    l *= a;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc.c[j] *= ac;
    acc.e -= dn;
    m = m_new;
  }
  float p[4];
  int et = kNoRef;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p[r] = __builtin_amdgcn_exp2f(x[r] - m);              // masked tokens: 0
    const int pe = static_cast<int>(__float_as_uint(p[r]) >> 23) - 127;   // p >= 0
    et = max(et, ev[r] + pe);
  }
  et = max_over_g4(et);
  if (__builtin_amdgcn_ballot_w64(et > acc.e + kSlackE) != 0) {
    const int e_new = max(acc.e, et);
    const int sh = acc.e - e_new;                           // the accumulator is 0 while e is kNoRef
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc.c[j][i] = __builtin_amdgcn_ldexpf(acc.c[j][i], sh);
    acc.e = e_new;
  }
  l += (p[0] + p[1]) + (p[2] + p[3]);
  float w[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) w[r] = __builtin_amdgcn_ldexpf(p[r], ev[r] - acc.e);
  const uint32_t h01 = pack16x2<PKV_F16>(w[0], w[1]), h23 = pack16x2<PKV_F16>(w[2], w[3]);
  float q0, q1, q2, q3;
  unpack2<PKV_F16>(h01, q0, q1);
  unpack2<PKV_F16>(h23, q2, q3);
  const u32x2 bh = {h01, h23};
  const u32x2 bl = {pack16x2<PKV_F16>(w[0] - q0, w[1] - q1), pack16x2<PKV_F16>(w[2] - q2, w[3] - q3)};
  // 4x4 byte transposes: X[4 q + k] = byte k of t.w[0..3][q] (rows 0..3)
  uint32_t X[8];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t A = __builtin_amdgcn_perm(t.w[1][q], t.w[0][q], 0x05010400u);
    const uint32_t Bq = __builtin_amdgcn_perm(t.w[1][q], t.w[0][q], 0x07030602u);
    const uint32_t C = __builtin_amdgcn_perm(t.w[3][q], t.w[2][q], 0x05010400u);
    const uint32_t Dq = __builtin_amdgcn_perm(t.w[3][q], t.w[2][q], 0x07030602u);
    X[4 * q + 0] = __builtin_amdgcn_perm(C, A, 0x05040100u);
    X[4 * q + 1] = __builtin_amdgcn_perm(C, A, 0x07060302u);
    X[4 * q + 2] = __builtin_amdgcn_perm(Dq, Bq, 0x05040100u);
    X[4 * q + 3] = __builtin_amdgcn_perm(Dq, Bq, 0x07060302u);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x2 av = {fp8x2_to_16<PKV_F16, false>(X[j]), fp8x2_to_16<PKV_F16, true>(X[j])};
    acc.c[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, av),
                                                     __builtin_bit_cast(f16x4, bh), acc.c[j], 0, 0, 0);
    acc.c[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, av),
                                                     __builtin_bit_cast(f16x4, bl), acc.c[j], 0, 0, 0);
  }
}

// s_waitcnt immediates (gfx9 encoding): wait for every vector memory
// operation, or for every LDS operation, the other counters left alone.
constexpr int kWaitVm0 = 0x0f70;
constexpr int kWaitLgkm0 = 0xc07f;

// The stream kernel's body.  FUSED: the decode-step form, which also does
// the step's write: the lengths (after the append) and the new tokens'
// slots come in `meta`; workgroup 0 publishes the lengths and the table
// entry of each new token's block; the tile holding a sequence's new token takes its block
// from the slot, and the one wave per KV head that reads that tile
// replaces the token's row (stale in the pool until then) with the new K/V
// row and stores that row into the pool.  KV8: the cache holds 8-bit rows
// (DT is then the query's type, which the K codes are converted to).
template <int DT, int GP, bool PAIRED, bool FUSED, bool KV8>
__device__ __forceinline__ void stream_body(const StreamArgs& a, const StepMeta* meta) {
  constexpr int D = 128;
  constexpr int CH = KV8 ? kStreamChunk8 : kStreamChunk;
  constexpr int KT = KV8 ? 128 : 256;     // LDS uint4 slots of one staged K tile
  constexpr int EB = KV8 ? 1 : 2;         // bytes per cached element
  using F = Frag<DT, D>;
  using VT = std::conditional_t<KV8, VTile8, VTile<DT, D>>;
  static_assert(F::kRowK, "stream kernel is for 16-bit queries with D = 128");
  // dynamic LDS: [K staging: waves x CH tiles x 4 KiB][q: waves x 4 KiB]
  //              [tile offsets: cap][S: B + 1][Ls: B]
  extern __shared__ uint4 sh_stream[];
  const int wave = uni(threadIdx.x >> 6);    // wave-uniform: keeps all per-job values scalar
  const int lane = threadIdx.x & (kWave - 1);
  const int g4 = lane >> 4, c16 = lane & 15;
  const int nwaves = blockDim.x >> 6;
  const int B = a.num_seqs;
  const int R = a.ranges_per_wg;
  const int H = a.hkv;
  const int J = R * H;
  uint4* sk = sh_stream + static_cast<int64_t>(wave) * CH * KT;
  uint4* sq = sh_stream + static_cast<int64_t>(nwaves) * CH * KT + static_cast<int64_t>(wave) * 256;
  // per tile of the workgroup: element offset of its first row in the pool
  // (block * block_stride + row-in-block * D, head offset excluded) and, for
  // 8-bit KV, the offset of its first scale byte (head excluded)
  using TileOff = std::conditional_t<KV8, TileOff8, int64_t>;
  TileOff* tbl = reinterpret_cast<TileOff*>(sh_stream + static_cast<int64_t>(nwaves) * (CH * KT + 256));
  int32_t* S = reinterpret_cast<int32_t*>(tbl + a.range_cap);
  int32_t* Ls = S + B + 1;
  if (wave == 0) {
    if constexpr (FUSED) tile_prefix([&](int b) { return meta->lens[b]; }, B, a.max_len, S, Ls, lane);
    else tile_prefix([&](int b) { return a.lens[b]; }, B, a.max_len, S, Ls, lane);
  }
  if constexpr (FUSED) {
    if (blockIdx.x == 0) {
      for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int L = meta->lens[b];
        if (a.lens_out) a.lens_out[b] = L;
        if (a.tables_w && b < a.table_rows && L > 0 && (L - 1) / a.block_size < a.table_stride)
          a.tables_w[static_cast<int64_t>(b) * a.table_stride + (L - 1) / a.block_size] =
              static_cast<int32_t>(meta->slots[b] / a.block_size);
      }
    }
  }
  __syncthreads();
  // the prefix sums for the merge (the workspace outlives this launch)
  if (blockIdx.x == 0)
    for (int b = threadIdx.x; b <= B; b += blockDim.x) a.ws_S[b] = S[b];
  const int T = S[B];
  const int W = a.num_ranges;
  const int64_t r_base = static_cast<int64_t>(blockIdx.x) * R;
  // the workgroup's tiles [w0, w1): ranges r_base .. r_base + R - 1
  const int w0 = range_start(r_base, T, W);
  const int w1 = range_start(r_base + R, T, W);
  if (w0 >= w1) return;                // whole workgroup: empty ranges
  const int bs = a.block_size;
  for (int t = threadIdx.x; t < w1 - w0; t += blockDim.x) {
    const int g = w0 + t;
    const int b = seq_of_tile(S, B, g);
    const int tok = (g - S[b]) * kTile;
    const int lb = tok / bs;
    int pb;
    if (FUSED && lb == (Ls[b] - 1) / bs)
      pb = static_cast<int>(meta->slots[b] / bs);   // the new token's block (maybe opened now)
    else
      pb = a.tables[static_cast<int64_t>(b) * a.table_stride + lb];
    pb = pb < 0 ? 0 : (pb >= a.num_blocks ? a.num_blocks - 1 : pb);
    const int off = tok - lb * bs;
    const int64_t e = static_cast<int64_t>(pb) * a.block_stride + static_cast<int64_t>(off) * D;
    if constexpr (KV8) tbl[t] = TileOff8{e, static_cast<int64_t>(pb) * a.sblock_stride + off};
    else tbl[t] = e;
  }
  __syncthreads();

  const int G = a.group;
  const char* kc = static_cast<const char*>(a.kc);
  const char* vc = static_cast<const char*>(a.vc);
  // PAIRED: nwaves == 2 * J, one task per wave; else nwaves == J, two.
  constexpr int ntasks = PAIRED ? 1 : 2;
  for (int task = 0; task < ntasks; ++task) {
    const int job = PAIRED ? (wave % J) : (task == 0 ? wave : (wave + 4) % J);
    const bool back = PAIRED ? (wave >= J) : (task == 1);
    const int r = job / H;
    const int kvh = job - r * H;
    const int64_t rng = r_base + r;
    const int g0 = range_start(rng, T, W);
    const int g1 = range_start(rng + 1, T, W);
    const int64_t head_off = static_cast<int64_t>(kvh) * a.head_stride;
    // The job's tiles [g0, g1) split at x: the front worker takes those
    // before, the back worker those from x on; both walk forward.
    const int x = g0 + part_split(g1 - g0, job, J, PAIRED, a.slot0_share);
    const int p0 = back ? x : g0, p1 = back ? g1 : x;
    // the chunk from tile g of sequence b: up to CH tiles, within b and the part
    auto chunk_len = [&](int g, int b) { return min(CH, min(uni(S[b + 1]), p1) - g); };
    // byte offset of tile g (inside the workgroup's tiles) and, for 8-bit
    // KV, of its first scale byte, from the staged offsets
    auto tile_bytes = [&](int g) -> int64_t {
      if constexpr (KV8) return uni64(tbl[g - w0].e) + head_off;
      else return (uni64(tbl[g - w0]) + head_off) * EB;
    };
    auto tile_scale = [&](int g) -> int64_t {
      if constexpr (KV8) return uni64(tbl[g - w0].s) + static_cast<int64_t>(kvh) * a.shead_stride;
      else return 0;
    };
    // The query group of sequence b, as the MFMA B operand, into the wave's
    // LDS slot by DMA: instruction kk gives lane (g4, c16) head-dims
    // 32 kk + 8 g4 .. + 7 of head c16.  Lanes of the padding heads
    // (c16 >= G) take a copy of the group's first head: their scores track
    // that head's exactly (so they never cause an extra rescale) and are
    // never written.  Kept in LDS, the operand costs no registers while the
    // P.V products run.
    auto load_q = [&](int b) {
      const int head = c16 < G ? c16 : 0;
      const char* qgrp = static_cast<const char*>(a.q) +
                         (static_cast<int64_t>(b) * a.hq + static_cast<int64_t>(kvh) * G) * D * 2;
      asm volatile("" ::: "memory");
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const int d0 = KV8 ? 32 * g4 + 8 * kk : 32 * kk + 8 * g4;   // the K operand's head-dim map
        __builtin_amdgcn_global_load_lds((global_void*)(qgrp + (head * D + d0) * 2),
                                         (lds_void*)(sq + kk * 64), 16, 0, 0);
      }
      asm volatile("" ::: "memory");
    };
    auto read_q = [&]() {
      Dw<F::kDwK> qf;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const uint4 x = sq[kk * 64 + lane];
        qf.w[4 * kk] = x.x; qf.w[4 * kk + 1] = x.y; qf.w[4 * kk + 2] = x.z; qf.w[4 * kk + 3] = x.w;
      }
      return qf;
    };
    auto nvalid_at = [&](int g, int b) { return min(kTile, uni(Ls[b]) - kTile * (g - uni(S[b]))); };
    // K rows of the n tiles from g on of sequence b into LDS, V rows into
    // `v`; the LDS reads for the addresses all come before the first DMA.
    // New-token row of the chunk in flight (decode-step form): held when the
    // chunk holds its sequence's last tile, as tile jn's row rn; lane
    // (g4, c16) has 16-byte chunk c16 of the K and V rows.
    bool hn = false;
    int jn = 0, rn = 0;
    u32x4 nk = {0u, 0u, 0u, 0u}, nvr = {0u, 0u, 0u, 0u};
    auto fetch_new = [&](int g, int n, int b) {
      hn = false;
      if constexpr (FUSED) {
        const int tl = uni(S[b + 1]) - 1;
        if (g <= tl && tl < g + n) {
          hn = true;
          jn = tl - g;
          rn = (uni(Ls[b]) - 1) & (kTile - 1);
          const int64_t off = ((static_cast<int64_t>(b) * H + kvh) * D + c16 * 8) * 2;
          nk = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(static_cast<const char*>(a.new_k) + off));
          nvr = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(static_cast<const char*>(a.new_v) + off));
        }
      }
    };
    // At the head of the chunk holding a new token: its K row into the
    // staged tile, its V row into the P.V registers, both rows into the pool.
    auto place_new = [&](VT (&v)[CH], int b) {
      if constexpr (FUSED && KV8) {
        // the new rows (the query's 16-bit type) quantised here exactly as
        // the 8-bit cache writes do it: each 16-lane group holds the whole
        // row, lane c16 elements 8 c16 .. 8 c16 + 7
        float xk[8], xv[8];
        const uint32_t wk[4] = {nk.x, nk.y, nk.z, nk.w}, wv[4] = {nvr.x, nvr.y, nvr.z, nvr.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          unpack2<DT>(wk[i], xk[2 * i], xk[2 * i + 1]);
          unpack2<DT>(wv[i], xv[2 * i], xv[2 * i + 1]);
        }
        float ak = 0.f, av = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ak = fmaxf(ak, pkv::finite_abs(xk[i]));
          av = fmaxf(av, pkv::finite_abs(xv[i]));
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
          ak = fmaxf(ak, __shfl_xor(ak, o));
          av = fmaxf(av, __shfl_xor(av, o));
        }
        const int ek = pkv::row_exponent(ak), evx = pkv::row_exponent(av);
        uint32_t k0 = 0, k1 = 0, v0 = 0, v1 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          k0 |= pkv::e4m3_code(__builtin_amdgcn_ldexpf(xk[i], -ek)) << (8 * i);
          k1 |= pkv::e4m3_code(__builtin_amdgcn_ldexpf(xk[4 + i], -ek)) << (8 * i);
          v0 |= pkv::e4m3_code(__builtin_amdgcn_ldexpf(xv[i], -evx)) << (8 * i);
          v1 |= pkv::e4m3_code(__builtin_amdgcn_ldexpf(xv[4 + i], -evx)) << (8 * i);
        }
        // K codes into the staged tile (chunk c of row rn at slot c ^ (rn % 8)),
        // V codes and both scale bytes into the P.V registers
        if (g4 == 0)
          reinterpret_cast<uint2*>(sk + jn * KT + rn * 8 + ((c16 >> 1) ^ (rn & 7)))[c16 & 1] = make_uint2(k0, k1);
        const int sh = 8 * (rn & 3);
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (j == jn && r == (rn & 3) && g4 == (rn >> 2)) {
              v[j].w[r][0] = v0;
              v[j].w[r][1] = v1;
              v[j].ks = (v[j].ks & ~(0xffu << sh)) | (static_cast<uint32_t>(ek + 127) << sh);
              v[j].vs = (v[j].vs & ~(0xffu << sh)) | (static_cast<uint32_t>(evx + 127) << sh);
            }
        if (g4 == 0) {
          const int64_t slot = meta->slots[b];
          const int64_t pb = slot / bs, off = slot - pb * bs;
          const int64_t dst = pb * a.block_stride + head_off + off * D + c16 * 8;
          *reinterpret_cast<uint2*>(static_cast<char*>(a.kc_w) + dst) = make_uint2(k0, k1);
          *reinterpret_cast<uint2*>(static_cast<char*>(a.vc_w) + dst) = make_uint2(v0, v1);
          if (c16 == 0) {
            const int64_t so = pb * a.sblock_stride + static_cast<int64_t>(kvh) * a.shead_stride + off;
            a.ks_w[so] = static_cast<uint8_t>(ek + 127);
            a.vs_w[so] = static_cast<uint8_t>(evx + 127);
          }
        }
      } else if constexpr (FUSED) {
        if (g4 == 0) sk[jn * 256 + rn * 16 + (c16 ^ rn)] = make_uint4(nk.x, nk.y, nk.z, nk.w);
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (j == jn && r == (rn & 3) && g4 == (rn >> 2)) {
              v[j].v[r].w[0] = nvr.x; v[j].v[r].w[1] = nvr.y;
              v[j].v[r].w[2] = nvr.z; v[j].v[r].w[3] = nvr.w;
            }
        if (g4 == 0) {
          const int64_t slot = meta->slots[b];
          const int64_t pb = slot / bs, off = slot - pb * bs;
          const int64_t dst = ((pb * a.block_stride + head_off + off * D) + c16 * 8) * 2;
          *reinterpret_cast<u32x4*>(static_cast<char*>(a.kc_w) + dst) = nk;
          *reinterpret_cast<u32x4*>(static_cast<char*>(a.vc_w) + dst) = nvr;
        }
      }
    };
    auto issue_chunk = [&](VT (&v)[CH], int g, int n, int b) {
      int64_t e[CH], so[CH];
      int nv[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        e[j] = j < n ? tile_bytes(g + j) : 0;
        so[j] = (KV8 && j < n) ? tile_scale(g + j) : 0;
        nv[j] = nvalid_at(g + j, b);
      }
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        if (j < n) {
          if constexpr (KV8) {
            issue_k_rows8(kc + e[j], sk + j * KT, nv[j], lane);
            load_v_buf8(v[j], vc + e[j], a.ks + so[j], a.vs + so[j], nv[j], lane);
          } else {
            issue_k_rows_buf(kc + e[j], sk + j * KT, nv[j], lane);
            load_v_buf<DT>(v[j], vc + e[j], nv[j], lane);
          }
        }
      }
    };

    if (p0 < p1) {
      // current chunk: tiles [cs, cs + cn) of sequence bc
      int cs = p0;
      int bc = uni(seq_of_tile(S, B, cs));
      int cn = chunk_len(cs, bc);
      load_q(bc);
      VT vcur[CH], vnext[CH];
      issue_chunk(vcur, cs, cn, bc);
      fetch_new(cs, cn, bc);
      int seg_lo = cs, seg_hi = cs + cn;    // tiles of the current segment
      float m = -INFINITY, l = 0.f;
      constexpr bool MPV = !KV8 && kMfmaPV16;
      std::conditional_t<KV8 || MPV, Acc8, AccV<GP>> acc;
      auto acc_init = [&]() { acc_zero(acc); };
      acc_init();
      // Per chunk: wait for its DMA (and its query group); scores from the K
      // rows in LDS; then the next chunk's fetch (V into `vnext`) and, when
      // that chunk is in another sequence, its query group into LDS; then
      // softmax + P.V of this chunk; then the segment end if the next chunk
      // leaves this sequence.
      while (true) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        if (FUSED && hn) place_new(vcur, bc);
        f32x4 scr[CH];
        {
          const Dw<F::kDwK> qf = read_q();
#pragma unroll
          for (int j = 0; j < CH; ++j) {
            if (j < cn) {
              if constexpr (KV8) scr[j] = qk_mfma<DT, D>(read_k_rows8<DT>(sk + j * KT, lane), qf);
              else scr[j] = qk_mfma<DT, D>(read_k_rows<DT, D>(sk + j * KT, lane), qf);
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // LDS reads done before the buffer is refilled
        const bool more = cs + cn < p1;
        int ns = 0, nn = 0, bn = -1;
        if (more) {
          ns = cs + cn;
          bn = bc;
          while (uni(S[bn + 1]) <= ns) ++bn;       // skips sequences with no tiles
          nn = chunk_len(ns, bn);
          issue_chunk(vnext, ns, nn, bn);
          fetch_new(ns, nn, bn);
          if (bn != bc) load_q(bn);
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          if (j < cn) {
            if constexpr (KV8)
              softmax_pv8(scr[j], vcur[j], nvalid_at(cs + j, bc), a.scale_log2, m, l, acc, lane);
            else if constexpr (MPV)
              softmax_pv16m<DT>(scr[j], vcur[j], nvalid_at(cs + j, bc), a.scale_log2, m, l, acc, lane);
            else
              softmax_pv<DT, D, GP>(scr[j], vcur[j], nvalid_at(cs + j, bc), a.scale_log2, m, l, acc.a, lane);
          }
        }
        if (bn != bc) {
          const bool complete = seg_lo == uni(S[bc]) && seg_hi == uni(S[bc + 1]);
          const int slot = back ? (seg_hi == g1 ? 2 : 3) : (seg_lo == g0 ? 0 : 1);
          const int64_t orow = static_cast<int64_t>(bc) * a.hq + static_cast<int64_t>(kvh) * G;
          const int64_t wrow = (rng * kStreamSlots + slot) * a.hq + static_cast<int64_t>(kvh) * G;
          if constexpr (KV8 || MPV)
            wave_epilogue8<KV8>(m, l, acc, lane, G, complete, a.out, a.out_dtype, orow, a.ws_acc, a.ws_ml, wrow);
          else
            wave_epilogue<DT, D, GP>(m, l, acc.a, lane, G, complete, a.out, a.out_dtype, orow,
                                     a.ws_acc, a.ws_ml, wrow, 1);
          m = -INFINITY;
          l = 0.f;
          acc_init();
          seg_lo = ns;
          seg_hi = ns + nn;
        } else {
          seg_hi = ns + nn;
        }
        if (!more) break;
#pragma unroll
        for (int j = 0; j < CH; ++j) vcur[j] = vnext[j];
        cs = ns;
        cn = nn;
        bc = bn;
      }
    }
  }
}

template <int DT, int GP, bool PAIRED>
__global__ void __launch_bounds__(kWave * kStreamMaxWaves, 2)
attn_stream_kernel(StreamArgs a) {
  stream_body<DT, GP, PAIRED, false, false>(a, nullptr);
}

// Attention over 8-bit KV blocks (DT: the query's type).
template <int DT, int GP, bool PAIRED>
__global__ void __launch_bounds__(kWave * kStreamMaxWaves, 2)
attn_stream8_kernel(StreamArgs a) {
  stream_body<DT, GP, PAIRED, false, true>(a, nullptr);
}

// The 8-bit decode step in one launch: the new rows (the query's type) are
// quantised and written by the wave that reads their tile.
template <int DT, int GP, bool PAIRED>
__global__ void __launch_bounds__(kWave * kStreamMaxWaves, 2)
attn_stream8_step_kernel(StreamArgs a, StepMeta meta) {
  stream_body<DT, GP, PAIRED, true, true>(a, &meta);
}

// The decode step in one launch: the write of the step's new rows (taken
// from `meta` and a.new_k / a.new_v) fused into the attention.
template <int DT, int GP, bool PAIRED>
__global__ void __launch_bounds__(kWave * kStreamMaxWaves, 2)
attn_stream_step_kernel(StreamArgs a, StepMeta meta) {
  stream_body<DT, GP, PAIRED, true, false>(a, &meta);
}

// Merge of the stream kernel's partials, per (sequence, query head).  A
// sequence with L = 0 gets zeros; one that a single segment covered was
// finished already; otherwise its pieces are combined as
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.  The pieces of
// sequence b are, in every range that holds some of its tiles, the part
// before the range's split tile x (front worker) and the part from x on
// (back worker), where not empty.
constexpr int kMergeChunk = 8;
constexpr int kMergeWaves = 4;


// Partial slots of the pieces of the sequence whose tiles are [Sb, Se)
// (Se > Sb, so total >= 1) into plist, in range order; one wave.  Lane i
// looks at ranges r_first + i, r_first + i + 64, ...  Returns their count.
__device__ __forceinline__ int merge_piece_list(const StreamArgs& a, int kvh, int Sb, int Se, int total,
                                                int lane, int32_t* plist) {
  const int W = a.num_ranges;
  const int R = a.ranges_per_wg;
  const int J = R * a.hkv;
  const bool paired = 2 * a.hkv <= kStreamMaxWaves;
  const int r_first = range_owner(Sb, total, W);
  const int r_last = range_owner(Se - 1, total, W);
  int npieces = 0;
  for (int r0 = r_first; r0 <= r_last; r0 += kWave) {
    const int r = r0 + lane;
    int sl[2];
    int n = 0;
    if (r <= r_last) {
      const int g0 = range_start(r, total, W), g1 = range_start(r + 1, total, W);
      if (g0 < g1) {
        const int x = g0 + part_split(g1 - g0, (r % R) * a.hkv + kvh, J, paired, a.slot0_share);
        const int lo = max(g0, Sb), hi = min(g1, Se);
        if (lo < min(x, hi)) sl[n++] = r * kStreamSlots + (lo == g0 ? 0 : 1);
        if (max(x, lo) < hi) sl[n++] = r * kStreamSlots + (hi == g1 ? 2 : 3);
      }
    }
    int incl = n;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int at = npieces + incl - n;
    if (n > 0) plist[at] = sl[0];
    if (n > 1) plist[at + 1] = sl[1];
    npieces += __shfl(incl, kWave - 1);
  }
  return npieces;
}

// Chunks j0, j0 + step, ... of kMergeChunk pieces folded into a running
// (M, den, num): every lane loads each piece's (m, l) and its own
// accumulator slice, all loads of a chunk in flight together, then folds
// the chunk with one rescale.
template <int D>
__device__ __forceinline__ void merge_fold(const StreamArgs& a, const int32_t* plist, int npieces, int qh,
                                           int lane, int j0, int step, float& M, float& den,
                                           float (&num)[D / kWave]) {
  constexpr int kPer = D / kWave;
  for (; j0 < npieces; j0 += step) {
    float mp[kMergeChunk], lp[kMergeChunk], v[kMergeChunk][kPer];
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const int j = min(j0 + u, npieces - 1);
      const int64_t sl = static_cast<int64_t>(plist[j]) * a.hq + qh;
      const float2 ml2 = *reinterpret_cast<const float2*>(a.ws_ml + 2 * sl);
      mp[u] = (j0 + u < npieces) ? ml2.x : -INFINITY;
      lp[u] = ml2.y;
#pragma unroll
      for (int e = 0; e < kPer; ++e) v[u][e] = a.ws_acc[sl * D + lane * kPer + e];
    }
    float Mc = M;
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) Mc = fmaxf(Mc, mp[u]);
    const float r = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mc);
    den *= r;
#pragma unroll
    for (int e = 0; e < kPer; ++e) num[e] *= r;
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const float wt = (mp[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mp[u] - Mc);
      den = fmaf(wt, lp[u], den);
#pragma unroll
      for (int e = 0; e < kPer; ++e) num[e] = fmaf(wt, v[u][e], num[e]);
    }
    M = Mc;
  }
}

// Row out[b, qh] = num / den (zeros when den = 0, as for L = 0).
template <int D>
__device__ __forceinline__ void merge_store(const StreamArgs& a, int b, int qh, int lane, float den,
                                            const float (&num)[D / kWave]) {
  constexpr int kPer = D / kWave;
  const int64_t orow = (static_cast<int64_t>(b) * a.hq + qh) * D;
  const float inv = den > 0.f ? 1.0f / den : 0.f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int64_t o = orow + lane * kPer + e;
    const float y = num[e] * inv;
    if (a.out_dtype == PKV_F32) static_cast<float*>(a.out)[o] = y;
    else if (a.out_dtype == PKV_BF16) static_cast<uint16_t*>(a.out)[o] = f32_to_bf16_rne(y);
    else static_cast<uint16_t*>(a.out)[o] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(y));
  }
}

// One wave per (sequence, query head): the form for launches whose
// sequences have up to about two chunks of pieces.
template <int D>
__global__ void __launch_bounds__(kWave)
attn_stream_merge_kernel(StreamArgs a) {
  constexpr int kPer = D / kWave;
  __shared__ int32_t plist[2 * kStreamMaxRanges];
  const int lane = threadIdx.x;
  const int qh = blockIdx.x % a.hq;
  const int b = blockIdx.x / a.hq;
  // the sequence's tiles [Sb, Se) and the launch's tile count, as the attention kernel summed them
  const int Sb = a.ws_S[b], Se = a.ws_S[b + 1], total = a.ws_S[a.num_seqs];
  float M = -INFINITY, den = 0.f;
  float num[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) num[e] = 0.f;
  if (Se == Sb) {                      // L = 0
    merge_store<D>(a, b, qh, lane, den, num);
    return;
  }
  const int npieces = merge_piece_list(a, qh / a.group, Sb, Se, total, lane, plist);
  __syncthreads();
  if (npieces <= 1) return;            // one segment covered the sequence
  merge_fold<D>(a, plist, npieces, qh, lane, 0, kMergeChunk, M, den, num);
  merge_store<D>(a, b, qh, lane, den, num);
}

// kMergeWaves waves per (sequence, query head), for launches whose
// sequences have many pieces: wave w folds chunks w, w + kMergeWaves, ...
// side by side, and wave 0 joins the waves' (M, den, num) in wave order.
template <int D>
__global__ void __launch_bounds__(kWave * kMergeWaves)
attn_stream_merge_waves_kernel(StreamArgs a) {
  constexpr int kPer = D / kWave;
  __shared__ int32_t plist[2 * kStreamMaxRanges];
  __shared__ int32_t s_npieces;
  __shared__ float s_part[kMergeWaves][2 + D];     // per wave: M, den, num[D]
  const int wave = uni(threadIdx.x >> 6);
  const int lane = threadIdx.x & (kWave - 1);
  const int qh = blockIdx.x % a.hq;
  const int b = blockIdx.x / a.hq;
  float M = -INFINITY, den = 0.f;
  float num[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) num[e] = 0.f;
  if (wave == 0) {
    const int Sb = a.ws_S[b], Se = a.ws_S[b + 1], total = a.ws_S[a.num_seqs];
    const int np = Se == Sb ? -1 : merge_piece_list(a, qh / a.group, Sb, Se, total, lane, plist);
    if (lane == 0) s_npieces = np;
  }
  __syncthreads();
  const int npieces = s_npieces;
  if (npieces < 0) {                   // L = 0: wave 0 writes the zeros
    if (wave == 0) merge_store<D>(a, b, qh, lane, den, num);
    return;
  }
  if (npieces <= 1) return;            // one segment covered the sequence
  merge_fold<D>(a, plist, npieces, qh, lane, wave * kMergeChunk, kMergeChunk * kMergeWaves, M, den, num);
  if (lane == 0) {
    s_part[wave][0] = M;
    s_part[wave][1] = den;
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) s_part[wave][2 + lane * kPer + e] = num[e];
  __syncthreads();
  if (wave != 0) return;
  const int nw = min(kMergeWaves, (npieces + kMergeChunk - 1) / kMergeChunk);
  float Mt = s_part[0][0];
  for (int w = 1; w < nw; ++w) Mt = fmaxf(Mt, s_part[w][0]);
  den = 0.f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) num[e] = 0.f;
  for (int w = 0; w < nw; ++w) {
    const float rw = (s_part[w][0] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_part[w][0] - Mt);
    den = fmaf(rw, s_part[w][1], den);
#pragma unroll
    for (int e = 0; e < kPer; ++e) num[e] = fmaf(rw, s_part[w][2 + lane * kPer + e], num[e]);
  }
  merge_store<D>(a, b, qh, lane, den, num);
}

// ------------------------------------------------------------ dispatch
constexpr int kDefaultPartition = 512;

int device_attr_cached(hipDeviceAttribute_t attr, int (&cache)[64], int fallback) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fallback;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, attr, dev) != hipSuccess || n <= 0) n = fallback;
  if (dev < 64) cache[dev] = n;
  return n;
}

// LDS one workgroup may allocate (160 KiB on gfx950).
size_t device_lds_per_block() {
  static int cached[64] = {0};
  return static_cast<size_t>(device_attr_cached(hipDeviceAttributeMaxSharedMemoryPerBlock, cached, 65536));
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cached[dev] = n;
  return n;
}

// Launch plan of the stream kernel, or ok = false when the shape is not one
// it covers (the partition kernel then runs with the default partition).
struct StreamPlan {
  bool ok = false;
  int wgs = 0;            // workgroups, one per CU
  int waves = 0;          // per workgroup
  int ranges_per_wg = 0;  // R
  int ranges = 0;         // W = wgs * R
  int range_cap = 0;
  size_t dyn_lds = 0;
  size_t acc_floats = 0;  // workspace: accumulators, then (m, l), then the tile prefix sums
  size_t ml_floats = 0;
  size_t workspace = 0;
};

StreamPlan plan_stream(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_context_len, int dtype_or_neg) {
  StreamPlan pl;
  if (head_dim != 128 || num_kv_heads > kStreamMaxHeads || num_kv_heads <= 0) return pl;
  if (num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > 8) return pl;
  if (dtype_or_neg == PKV_F32) return pl;
  // two waves per job when they fit in kStreamMaxWaves, else one wave per
  // job that also works the back of another job
  const int R = 2 * num_kv_heads <= kStreamMaxWaves ? kStreamMaxWaves / (2 * num_kv_heads) : 1;
  const int waves = 2 * num_kv_heads <= kStreamMaxWaves ? 2 * R * num_kv_heads : num_kv_heads;
  const int64_t wgs = device_cu_count();
  const int64_t ranges = wgs * R;
  if (ranges > kStreamMaxRanges) return pl;
  const int64_t tiles_max = static_cast<int64_t>(num_seqs) * ((max_context_len + kTile - 1) / kTile);
  if (tiles_max >= (1LL << 30)) return pl;
  const int64_t cap = (tiles_max + wgs - 1) / wgs + 1;
  const size_t dyn = static_cast<size_t>(waves) * (kStreamChunk + 1) * 4096 +
                     static_cast<size_t>(cap) * sizeof(TileOff8) +   // either entry size fits
                     static_cast<size_t>(2 * num_seqs + 1) * sizeof(int32_t);
  if (dyn > device_lds_per_block()) return pl;
  pl.ok = true;
  pl.wgs = static_cast<int>(wgs);
  pl.waves = waves;
  pl.ranges_per_wg = R;
  pl.ranges = static_cast<int>(ranges);
  pl.range_cap = static_cast<int>(cap);
  pl.dyn_lds = dyn;
  pl.acc_floats = static_cast<size_t>(ranges) * kStreamSlots * num_q_heads * head_dim;
  pl.ml_floats = static_cast<size_t>(ranges) * kStreamSlots * num_q_heads * 2;
  pl.workspace = (pl.acc_floats + pl.ml_floats) * sizeof(float) + (static_cast<size_t>(num_seqs) + 1) * sizeof(int32_t);
  return pl;
}

int pick_partition(int32_t partition_tokens) {
  return partition_tokens > 0 ? partition_tokens : kDefaultPartition;
}

int padded_group(int g) {
  if (g <= 1) return 1;
  if (g <= 2) return 2;
  if (g <= 4) return 4;
  if (g <= 6) return 6;
  if (g <= 7) return 7;
  return 8;
}

// Dynamic LDS of the partition kernel: the block-table entries one
// partition can touch.
size_t table_lds_bytes(int part_tokens, int block_size) {
  return static_cast<size_t>((part_tokens + kTile) / block_size + 2) * sizeof(int32_t);
}

template <int DT, int D, int GP>
hipError_t launch_split_t(const AttnArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_split_kernel<DT, D, GP>), grid, dim3(kWave),
                     table_lds_bytes(a.part_tokens, a.block_size), s, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_split_d(const AttnArgs& a, int gp, dim3 grid, hipStream_t s) {
  switch (gp) {
    case 1: return launch_split_t<DT, D, 1>(a, grid, s);
    case 2: return launch_split_t<DT, D, 2>(a, grid, s);
    case 4: return launch_split_t<DT, D, 4>(a, grid, s);
    case 6: return launch_split_t<DT, D, 6>(a, grid, s);
    case 7: return launch_split_t<DT, D, 7>(a, grid, s);
    default: return launch_split_t<DT, D, 8>(a, grid, s);
  }
}

// Raises a kernel's dynamic-LDS limit to what a launch asks for (the plan
// already checked it against the device's per-block LDS), once per kernel,
// device and size.
template <typename K>
hipError_t raise_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  struct Raised {
    const void* fn;
    int dev;
    int bytes;
  };
  static std::mutex mu;
  static std::vector<Raised> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const void* fn = reinterpret_cast<const void*>(kernel);
  std::lock_guard<std::mutex> lock(mu);
  for (const Raised& r : done)
    if (r.fn == fn && r.dev == dev && r.bytes >= static_cast<int>(bytes)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
  if (e != hipSuccess) return e;
  done.push_back(Raised{fn, dev, static_cast<int>(bytes)});
  return hipSuccess;
}

template <int DT, int GP, bool PAIRED, bool KV8>
hipError_t launch_stream_p(const StreamArgs& a, const StreamPlan& pl, const StepMeta* meta,
                           hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(pl.wgs)), block(kWave * pl.waves);
  if constexpr (KV8) {
    if (meta) {
      const hipError_t e = raise_lds(&attn_stream8_step_kernel<DT, GP, PAIRED>, pl.dyn_lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((attn_stream8_step_kernel<DT, GP, PAIRED>), grid, block, pl.dyn_lds, s, a, *meta);
    } else {
      const hipError_t e = raise_lds(&attn_stream8_kernel<DT, GP, PAIRED>, pl.dyn_lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((attn_stream8_kernel<DT, GP, PAIRED>), grid, block, pl.dyn_lds, s, a);
    }
    return hipGetLastError();
  }
  if (meta) {
    const hipError_t e = raise_lds(&attn_stream_step_kernel<DT, GP, PAIRED>, pl.dyn_lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_stream_step_kernel<DT, GP, PAIRED>), grid, block, pl.dyn_lds, s, a, *meta);
  } else {
    const hipError_t e = raise_lds(&attn_stream_kernel<DT, GP, PAIRED>, pl.dyn_lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_stream_kernel<DT, GP, PAIRED>), grid, block, pl.dyn_lds, s, a);
  }
  return hipGetLastError();
}

template <int DT, int GP, bool KV8>
hipError_t launch_stream_t(const StreamArgs& a, const StreamPlan& pl, const StepMeta* meta,
                           hipStream_t s) {
  return pl.waves == 2 * pl.ranges_per_wg * a.hkv ? launch_stream_p<DT, GP, true, KV8>(a, pl, meta, s)
                                                  : launch_stream_p<DT, GP, false, KV8>(a, pl, meta, s);
}

template <int DT, bool KV8 = false>
hipError_t launch_stream_dt(const StreamArgs& a, int gp, const StreamPlan& pl, const StepMeta* meta,
                            hipStream_t s) {
  // P.V on the matrix cores covers 16 heads whatever G is
  if constexpr (KV8 || kMfmaPV16) {
    return launch_stream_t<DT, 8, KV8>(a, pl, meta, s);
  } else {
    switch (gp) {
      case 1: return launch_stream_t<DT, 1, KV8>(a, pl, meta, s);
      case 2: return launch_stream_t<DT, 2, KV8>(a, pl, meta, s);
      case 4: return launch_stream_t<DT, 4, KV8>(a, pl, meta, s);
      case 6: return launch_stream_t<DT, 6, KV8>(a, pl, meta, s);
      case 7: return launch_stream_t<DT, 7, KV8>(a, pl, meta, s);
      default: return launch_stream_t<DT, 8, KV8>(a, pl, meta, s);
    }
  }
}

template <int DT>
hipError_t launch_split_dt(const AttnArgs& a, int d, int gp, dim3 grid, hipStream_t s) {
  if (d == 64) return launch_split_d<DT, 64>(a, gp, grid, s);
  return launch_split_d<DT, 128>(a, gp, grid, s);
}

}  // namespace

namespace pkv {

int check_layout(const pkv_cache_layout* l) {
  if (!l) return PKV_ERR_INVALID;
  if (l->num_blocks <= 0 || l->num_kv_heads <= 0 || l->block_size <= 0 || l->head_dim <= 0)
    return PKV_ERR_INVALID;
  if (elem_bytes(l->dtype) == 0 || l->reserved != 0) return PKV_ERR_INVALID;
  if (l->head_stride < static_cast<int64_t>(l->block_size) * l->head_dim) return PKV_ERR_INVALID;
  if (l->block_stride < static_cast<int64_t>(l->num_kv_heads) * l->head_stride) return PKV_ERR_INVALID;
  if (l->head_stride % 8 != 0 || l->block_stride % 8 != 0) return PKV_ERR_INVALID;
  return PKV_OK;
}

}  // namespace pkv

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID: return "invalid argument";
    case PKV_ERR_OOM: return "OOM: not enough free KV blocks";
    case PKV_ERR_NOT_LIVE: return "sequence is not live (unknown or already freed)";
    case PKV_ERR_ALREADY_PREFILLED: return "sequence is already live";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_INVARIANT: return "block manager invariant violated";
    default: return "unknown status";
  }
}

const char* pkv_version(void) { return "pkv 0.1.0 gfx950"; }

size_t pkv_pool_span_bytes(const pkv_cache_layout* l) {
  if (pkv::check_layout(l) != PKV_OK) return 0;
  const int64_t elems = static_cast<int64_t>(l->num_blocks - 1) * l->block_stride +
                        static_cast<int64_t>(l->num_kv_heads - 1) * l->head_stride +
                        static_cast<int64_t>(l->block_size) * l->head_dim;
  return static_cast<size_t>(elems) * pkv::elem_bytes(l->dtype);
}

int paged_kv_write(const void* key, const void* value, const int64_t* slot_mapping,
                   int32_t num_tokens, void* key_cache, void* value_cache,
                   const pkv_cache_layout* l, void* stream) {
  if (pkv::check_layout(l) != PKV_OK || num_tokens < 0) return PKV_ERR_INVALID;
  if (l->dtype == PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;   // paged_kv_write_fp8
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !slot_mapping || !key_cache || !value_cache) return PKV_ERR_INVALID;
  const int eb = pkv::elem_bytes(l->dtype);
  const int64_t row_bytes = static_cast<int64_t>(l->head_dim) * eb;
  if (row_bytes % 16 != 0) return PKV_ERR_UNSUPPORTED;
  if ((l->head_stride * eb) % 16 != 0 || (l->block_stride * eb) % 16 != 0) return PKV_ERR_UNSUPPORTED;
  const uintptr_t align = reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value) |
                          reinterpret_cast<uintptr_t>(key_cache) |
                          reinterpret_cast<uintptr_t>(value_cache);
  if (align % 16 != 0) return PKV_ERR_UNSUPPORTED;
  const int32_t chunks_per_head = static_cast<int32_t>(row_bytes / 16);
  const int32_t chunks_per_token = chunks_per_head * l->num_kv_heads;
  const int64_t total = static_cast<int64_t>(num_tokens) * chunks_per_token;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(kv_write_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(key),
                     static_cast<const uint4*>(value), slot_mapping, total, chunks_per_head,
                     chunks_per_token,
                     static_cast<int64_t>(l->num_blocks) * l->block_size, l->block_size,
                     l->block_stride * eb / 16, l->head_stride * eb / 16,
                     static_cast<int32_t>(row_bytes / 16), static_cast<uint4*>(key_cache),
                     static_cast<uint4*>(value_cache));
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_decode_write(const void* key, const void* value, const int64_t* slots, const int32_t* lens,
                     int32_t num_rows, void* key_cache, void* value_cache,
                     const pkv_cache_layout* l, int32_t* block_tables, int32_t table_rows,
                     int32_t block_table_stride, int32_t* lens_out, void* stream) {
  if (pkv::check_layout(l) != PKV_OK || num_rows < 0 || table_rows < 0 || block_table_stride < 0)
    return PKV_ERR_INVALID;
  if (l->dtype == PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;   // pkv_decode_write_fp8
  if (num_rows == 0) return PKV_OK;
  if (!key || !value || !slots || !lens || !key_cache || !value_cache) return PKV_ERR_INVALID;
  if (block_tables && block_table_stride <= 0) return PKV_ERR_INVALID;
  const int eb = pkv::elem_bytes(l->dtype);
  const int64_t row_bytes = static_cast<int64_t>(l->head_dim) * eb;
  if (row_bytes % 16 != 0) return PKV_ERR_UNSUPPORTED;
  if ((l->head_stride * eb) % 16 != 0 || (l->block_stride * eb) % 16 != 0) return PKV_ERR_UNSUPPORTED;
  const uintptr_t align = reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value) |
                          reinterpret_cast<uintptr_t>(key_cache) |
                          reinterpret_cast<uintptr_t>(value_cache);
  if (align % 16 != 0) return PKV_ERR_UNSUPPORTED;
  const int32_t chunks_per_head = static_cast<int32_t>(row_bytes / 16);
  const int32_t chunks_per_token = chunks_per_head * l->num_kv_heads;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t row0 = 0; row0 < num_rows; row0 += kStepRows) {
    const int32_t n = num_rows - row0 < kStepRows ? num_rows - row0 : kStepRows;
    StepMeta meta;
    for (int32_t i = 0; i < n; ++i) {
      meta.slots[i] = slots[row0 + i];
      meta.lens[i] = lens[row0 + i];
    }
    const int64_t total = static_cast<int64_t>(n) * chunks_per_token;
    hipLaunchKernelGGL(decode_write_kernel, dim3(static_cast<uint32_t>((total + 255) / 256)),
                       dim3(256), 0, s, meta, n, row0, static_cast<const uint4*>(key),
                       static_cast<const uint4*>(value), chunks_per_head, chunks_per_token,
                       static_cast<int64_t>(l->num_blocks) * l->block_size, l->block_size,
                       l->block_stride * eb / 16, l->head_stride * eb / 16,
                       static_cast<int32_t>(row_bytes / 16), static_cast<uint4*>(key_cache),
                       static_cast<uint4*>(value_cache), block_tables, table_rows,
                       block_table_stride, lens_out);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

size_t paged_decode_attention_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_context_len, int32_t partition_tokens) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0 || partition_tokens < 0)
    return 0;
  const int part = pick_partition(partition_tokens);
  const int64_t P = (static_cast<int64_t>(max_context_len) + part - 1) / part;
  size_t need = P <= 1 ? 0 : static_cast<size_t>(num_seqs) * num_q_heads * P * (head_dim + 2) * sizeof(float);
  if (partition_tokens == 0) {
    const StreamPlan pl = plan_stream(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, -1);
    if (pl.ok && pl.workspace > need) need = pl.workspace;
  }
  return need;
}

}  // extern "C"

namespace {

constexpr int kPhasePartial = 1;
constexpr int kPhaseMerge = 2;

// 8-bit KV attention: the rows' scale bytes and the query's type.
struct Fp8Args {
  const uint8_t* key_scales;
  const uint8_t* value_scales;
  int32_t q_dtype;
};

// The decode-step form of the stream launch: the step's new rows, its
// metadata, and where its write goes.
struct StepArgs {
  const void* key;
  const void* value;
  const StepMeta* meta;
  void* key_cache;
  void* value_cache;
  int32_t* block_tables;
  int32_t table_rows;
  int32_t* lens_out;
  uint8_t* key_scales = nullptr;     // 8-bit path: where the new rows' scale bytes go
  uint8_t* value_scales = nullptr;
};

// Validates the arguments, then launches the attention kernel (phase 1)
// and/or the split-K merge kernel (phase 2).  With `step` (stream path
// only), phase 1 is the decode-step kernel that also does the step's write.
int attention_impl(int phases, void* out, int32_t out_dtype, const void* q, const void* key_cache,
                   const void* value_cache, const int32_t* block_tables,
                   int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                   int32_t num_q_heads, int32_t max_context_len, float scale,
                   const pkv_cache_layout* l, int32_t partition_tokens, void* workspace,
                   size_t workspace_bytes, void* stream, const StepArgs* step = nullptr,
                   const Fp8Args* f8 = nullptr) {
  if (pkv::check_layout(l) != PKV_OK) return PKV_ERR_INVALID;
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || block_table_stride < 0 ||
      partition_tokens < 0)
    return PKV_ERR_INVALID;
  if ((l->dtype == PKV_FP8_E4M3) != (f8 != nullptr)) return PKV_ERR_UNSUPPORTED;
  // the type of q (and of a non-fp32 output): the cache's, or for 8-bit KV the given one
  const int qt = f8 ? f8->q_dtype : l->dtype;
  if (f8 && ((qt != PKV_BF16 && qt != PKV_F16) || !f8->key_scales || !f8->value_scales))
    return PKV_ERR_INVALID;
  if (f8 && partition_tokens != 0) return PKV_ERR_UNSUPPORTED;
  if (num_q_heads % l->num_kv_heads != 0) return PKV_ERR_INVALID;
  if (out_dtype != PKV_F32 && out_dtype != qt) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(block_table_stride) * l->block_size)
    return PKV_ERR_INVALID;
  if (!(scale == scale)) return PKV_ERR_INVALID;
  const int group = num_q_heads / l->num_kv_heads;
  if (group > 8) return PKV_ERR_UNSUPPORTED;
  if (l->head_dim != 64 && l->head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (l->block_size % kTile != 0) return PKV_ERR_UNSUPPORTED;
  const int part = pick_partition(partition_tokens);
  if (part % kTile != 0) return PKV_ERR_INVALID;
  if (table_lds_bytes(part, l->block_size) > 32768) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !key_cache || !value_cache || !context_lens ||
      (max_context_len > 0 && !block_tables))
    return PKV_ERR_INVALID;
  const int eb = pkv::elem_bytes(l->dtype);
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(key_cache) |
                          reinterpret_cast<uintptr_t>(value_cache);
  if (align % 16 != 0 || (l->head_stride * eb) % 16 != 0 || (l->block_stride * eb) % 16 != 0)
    return PKV_ERR_UNSUPPORTED;
  if (f8) {
    // scale bytes mirror the code layout with one byte per row; a tile's 16
    // scale bytes are read as dwords
    if (l->head_stride % l->head_dim != 0 || l->block_stride % l->head_dim != 0 ||
        (l->head_stride / l->head_dim) % 4 != 0 || (l->block_stride / l->head_dim) % 4 != 0 ||
        ((reinterpret_cast<uintptr_t>(f8->key_scales) | reinterpret_cast<uintptr_t>(f8->value_scales)) % 4) != 0)
      return PKV_ERR_UNSUPPORTED;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (partition_tokens == 0) {
    const StreamPlan pl = plan_stream(num_seqs, num_q_heads, l->num_kv_heads, l->head_dim,
                                      max_context_len, l->dtype);
    if (pl.ok) {
      if (!workspace || workspace_bytes < pl.workspace) return PKV_ERR_WORKSPACE;
      StreamArgs sa;
      sa.q = q;
      sa.kc = key_cache;
      sa.vc = value_cache;
      sa.tables = block_tables;
      sa.lens = context_lens;
      sa.ws_acc = static_cast<float*>(workspace);
      sa.ws_ml = sa.ws_acc + pl.acc_floats;
      sa.ws_S = reinterpret_cast<int32_t*>(sa.ws_ml + pl.ml_floats);
      sa.out = out;
      sa.block_stride = l->block_stride;
      sa.head_stride = l->head_stride;
      sa.table_stride = block_table_stride;
      sa.num_blocks = l->num_blocks;
      sa.block_size = l->block_size;
      sa.num_seqs = num_seqs;
      sa.hq = num_q_heads;
      sa.hkv = l->num_kv_heads;
      sa.group = group;
      sa.max_len = max_context_len;
      sa.out_dtype = out_dtype;
      sa.range_cap = pl.range_cap;
      sa.num_ranges = pl.ranges;
      sa.ranges_per_wg = pl.ranges_per_wg;
      sa.slot0_share = f8 ? kSlot0Share8 : kSlot0Share;
      sa.scale_log2 = scale * kLog2e;
      sa.new_k = step ? step->key : nullptr;
      sa.new_v = step ? step->value : nullptr;
      sa.kc_w = step ? step->key_cache : nullptr;
      sa.vc_w = step ? step->value_cache : nullptr;
      sa.tables_w = step ? step->block_tables : nullptr;
      sa.table_rows = step ? step->table_rows : 0;
      sa.lens_out = step ? step->lens_out : nullptr;
      sa.ks = f8 ? f8->key_scales : nullptr;
      sa.vs = f8 ? f8->value_scales : nullptr;
      sa.ks_w = step ? step->key_scales : nullptr;
      sa.vs_w = step ? step->value_scales : nullptr;
      sa.sblock_stride = l->block_stride / l->head_dim;
      sa.shead_stride = l->head_stride / l->head_dim;
      if (phases & kPhasePartial) {
        const int gp = padded_group(group);
        const StepMeta* meta = step ? step->meta : nullptr;
        hipError_t e;
        if (f8) e = (qt == PKV_BF16) ? launch_stream_dt<PKV_BF16, true>(sa, gp, pl, meta, s)
                                     : launch_stream_dt<PKV_F16, true>(sa, gp, pl, meta, s);
        else e = (l->dtype == PKV_BF16) ? launch_stream_dt<PKV_BF16>(sa, gp, pl, meta, s)
                                        : launch_stream_dt<PKV_F16>(sa, gp, pl, meta, s);
        if (e != hipSuccess) return PKV_ERR_HIP;
      }
      if (phases & kPhaseMerge) {
        // The merge takes each sequence's tile range from the prefix sums the
        // first launch left in the workspace.  A sequence spans about W / B
        // ranges, two pieces each.  Beyond two chunks of pieces the waves of
        // the multi-wave merge fold chunks side by side; below that the
        // one-wave merge measured faster.
        const int64_t pieces = 2 * ((pl.ranges + num_seqs - 1) / num_seqs) + 2;
        const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(num_seqs) * num_q_heads));
        if (pieces > 2 * kMergeChunk)
          hipLaunchKernelGGL(attn_stream_merge_waves_kernel<128>, grid, dim3(kWave * kMergeWaves), 0, s, sa);
        else
          hipLaunchKernelGGL(attn_stream_merge_kernel<128>, grid, dim3(kWave), 0, s, sa);
        if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
      }
      return PKV_OK;
    }
  }
  if (f8) return PKV_ERR_UNSUPPORTED;     // 8-bit KV: stream path shapes only
  const int64_t P = max_context_len > 0 ? (static_cast<int64_t>(max_context_len) + part - 1) / part : 1;
  const size_t need = paged_decode_attention_workspace_size(num_seqs, num_q_heads, l->num_kv_heads,
                                                            l->head_dim, max_context_len, part);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;
  const int64_t wgs = P * num_seqs * l->num_kv_heads;
  if (wgs > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;

  AttnArgs a;
  a.q = q;
  a.kc = key_cache;
  a.vc = value_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  const int64_t acc_floats = static_cast<int64_t>(num_seqs) * num_q_heads * P * l->head_dim;
  a.ws_acc = need > 0 ? static_cast<float*>(workspace) : nullptr;
  a.ws_ml = need > 0 ? static_cast<float*>(workspace) + acc_floats : nullptr;
  a.out = out;
  a.block_stride = l->block_stride;
  a.head_stride = l->head_stride;
  a.table_stride = block_table_stride;
  a.num_blocks = l->num_blocks;
  a.block_size = l->block_size;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = l->num_kv_heads;
  a.group = group;
  a.max_len = max_context_len;
  a.part_tokens = part;
  a.max_parts = static_cast<int32_t>(P);
  a.out_dtype = out_dtype;
  a.scale_log2 = scale * kLog2e;

  if (phases & kPhasePartial) {
    const dim3 grid(static_cast<uint32_t>(wgs));
    const int gp = padded_group(group);
    hipError_t e;
    switch (l->dtype) {
      case PKV_BF16: e = launch_split_dt<PKV_BF16>(a, l->head_dim, gp, grid, s); break;
      case PKV_F16: e = launch_split_dt<PKV_F16>(a, l->head_dim, gp, grid, s); break;
      default: e = launch_split_dt<PKV_F32>(a, l->head_dim, gp, grid, s); break;
    }
    if (e != hipSuccess) return PKV_ERR_HIP;
  }
  if ((phases & kPhaseMerge) && P > 1) {
    const dim3 rgrid(static_cast<uint32_t>(static_cast<int64_t>(num_seqs) * num_q_heads));
    const dim3 rblock(kWave * kReduceWaves);
    if (l->head_dim == 64) hipLaunchKernelGGL(attn_reduce_kernel<64>, rgrid, rblock, 0, s, a);
    else hipLaunchKernelGGL(attn_reduce_kernel<128>, rgrid, rblock, 0, s, a);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

int paged_decode_attention_path(int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                const pkv_cache_layout* l, int32_t partition_tokens) {
  if (pkv::check_layout(l) != PKV_OK || num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 ||
      partition_tokens < 0 || num_q_heads % l->num_kv_heads != 0)
    return PKV_ERR_INVALID;
  if (partition_tokens == 0 &&
      plan_stream(num_seqs, num_q_heads, l->num_kv_heads, l->head_dim, max_context_len, l->dtype).ok)
    return PKV_PATH_STREAM;
  if (l->dtype == PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;   // 8-bit KV: stream path only
  return PKV_PATH_PARTITION;
}

int paged_decode_attention(void* out, int32_t out_dtype, const void* q, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables,
                           int32_t block_table_stride, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                           float scale, const pkv_cache_layout* l, int32_t partition_tokens,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return attention_impl(kPhasePartial | kPhaseMerge, out, out_dtype, q, key_cache, value_cache,
                        block_tables, block_table_stride, context_lens, num_seqs, num_q_heads,
                        max_context_len, scale, l, partition_tokens, workspace, workspace_bytes,
                        stream);
}

int paged_decode_attention_partial(void* out, int32_t out_dtype, const void* q,
                                   const void* key_cache, const void* value_cache,
                                   const int32_t* block_tables, int32_t block_table_stride,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_context_len, float scale,
                                   const pkv_cache_layout* l, int32_t partition_tokens,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return attention_impl(kPhasePartial, out, out_dtype, q, key_cache, value_cache, block_tables,
                        block_table_stride, context_lens, num_seqs, num_q_heads, max_context_len,
                        scale, l, partition_tokens, workspace, workspace_bytes, stream);
}

int paged_decode_attention_merge(void* out, int32_t out_dtype, const void* q,
                                 const void* key_cache, const void* value_cache,
                                 const int32_t* block_tables, int32_t block_table_stride,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_context_len, float scale,
                                 const pkv_cache_layout* l, int32_t partition_tokens,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return attention_impl(kPhaseMerge, out, out_dtype, q, key_cache, value_cache, block_tables,
                        block_table_stride, context_lens, num_seqs, num_q_heads, max_context_len,
                        scale, l, partition_tokens, workspace, workspace_bytes, stream);
}

}  // extern "C"

// Workspace of pkv_decode_step_noalloc: a device array owned by the library,
// one copy per GPU, alive until the process ends.  On the host its name
// stands for the host-side shadow, not for device memory: kernels get the
// address scratch_address() looks up, never `scratch` itself.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_address(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return PKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PKV_ERR_HIP;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return PKV_OK;
}
}  // namespace

extern "C" {

// The decode step (append already done on the host): the write of the
// step's new rows and the attention over the updated cache.  One launch
// (plus the merge) when the stream path applies, at most 256 rows are
// given and every slot and length is in range; otherwise pkv_decode_write
// then paged_decode_attention.
namespace {
// 8-bit decode step: the scale pools (written and read) and the query's type.
struct Fp8Step {
  uint8_t* key_scales;
  uint8_t* value_scales;
  int32_t q_dtype;
};

int decode_step_impl(int phases, void* out, int32_t out_dtype, const void* q, const void* key,
                     const void* value, const int64_t* slots, const int32_t* lens, int32_t num_seqs,
                     void* key_cache, void* value_cache, const pkv_cache_layout* l,
                     int32_t* block_tables, int32_t block_table_stride, int32_t* lens_out,
                     int32_t num_q_heads, int32_t max_context_len, float scale, void* workspace,
                     size_t workspace_bytes, void* stream, const Fp8Step* f8s = nullptr) {
  if (pkv::check_layout(l) != PKV_OK || num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 ||
      block_table_stride <= 0)
    return PKV_ERR_INVALID;
  if ((l->dtype == PKV_FP8_E4M3) != (f8s != nullptr)) return PKV_ERR_UNSUPPORTED;
  if (f8s && (!f8s->key_scales || !f8s->value_scales)) return PKV_ERR_INVALID;
  if (num_seqs == 0) return PKV_OK;
  if (!key || !value || !slots || !lens || !lens_out || !block_tables) return PKV_ERR_INVALID;
  const int64_t capacity = static_cast<int64_t>(l->num_blocks) * l->block_size;
  bool fused = num_seqs <= kStepRows &&
               (reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value)) % 16 == 0 &&
               plan_stream(num_seqs, num_q_heads, l->num_kv_heads, l->head_dim, max_context_len,
                           l->dtype).ok;
  for (int32_t i = 0; fused && i < num_seqs; ++i)
    fused = slots[i] >= 0 && slots[i] < capacity && lens[i] >= 1 && lens[i] <= max_context_len &&
            (lens[i] - 1) / l->block_size < block_table_stride;
  const Fp8Args f8a = f8s ? Fp8Args{f8s->key_scales, f8s->value_scales, f8s->q_dtype} : Fp8Args{};
  if (!fused) {
    if (phases & kPhasePartial) {
      const int r = f8s ? pkv_decode_write_fp8(key, value, f8s->q_dtype, slots, lens, num_seqs, key_cache,
                                               value_cache, f8s->key_scales, f8s->value_scales, l,
                                               block_tables, num_seqs, block_table_stride, lens_out, stream)
                        : pkv_decode_write(key, value, slots, lens, num_seqs, key_cache, value_cache, l,
                                           block_tables, num_seqs, block_table_stride, lens_out, stream);
      if (r != PKV_OK) return r;
    }
    return attention_impl(phases, out, out_dtype, q, key_cache, value_cache, block_tables,
                          block_table_stride, lens_out, num_seqs, num_q_heads, max_context_len,
                          scale, l, 0, workspace, workspace_bytes, stream, nullptr, f8s ? &f8a : nullptr);
  }
  StepMeta meta;
  for (int32_t i = 0; i < num_seqs; ++i) {
    meta.slots[i] = slots[i];
    meta.lens[i] = lens[i];
  }
  StepArgs st{key, value, &meta, key_cache, value_cache, block_tables, num_seqs, lens_out};
  if (f8s) {
    st.key_scales = f8s->key_scales;
    st.value_scales = f8s->value_scales;
  }
  return attention_impl(phases, out, out_dtype, q, key_cache, value_cache, block_tables,
                        block_table_stride, lens_out, num_seqs, num_q_heads, max_context_len,
                        scale, l, 0, workspace, workspace_bytes, stream, &st, f8s ? &f8a : nullptr);
}
}  // namespace

int pkv_decode_step(void* out, int32_t out_dtype, const void* q, const void* key,
                    const void* value, const int64_t* slots, const int32_t* lens, int32_t num_seqs,
                    void* key_cache, void* value_cache, const pkv_cache_layout* layout,
                    int32_t* block_tables, int32_t block_table_stride, int32_t* lens_out,
                    int32_t num_q_heads, int32_t max_context_len, float scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return decode_step_impl(kPhasePartial | kPhaseMerge, out, out_dtype, q, key, value, slots, lens,
                          num_seqs, key_cache, value_cache, layout, block_tables,
                          block_table_stride, lens_out, num_q_heads, max_context_len, scale,
                          workspace, workspace_bytes, stream);
}

int pkv_decode_step_partial(void* out, int32_t out_dtype, const void* q, const void* key,
                            const void* value, const int64_t* slots, const int32_t* lens,
                            int32_t num_seqs, void* key_cache, void* value_cache,
                            const pkv_cache_layout* layout, int32_t* block_tables,
                            int32_t block_table_stride, int32_t* lens_out, int32_t num_q_heads,
                            int32_t max_context_len, float scale, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return decode_step_impl(kPhasePartial, out, out_dtype, q, key, value, slots, lens, num_seqs,
                          key_cache, value_cache, layout, block_tables, block_table_stride,
                          lens_out, num_q_heads, max_context_len, scale, workspace,
                          workspace_bytes, stream);
}

int pkv_decode_step_merge(void* out, int32_t out_dtype, const void* q, const void* key,
                          const void* value, const int64_t* slots, const int32_t* lens,
                          int32_t num_seqs, void* key_cache, void* value_cache,
                          const pkv_cache_layout* layout, int32_t* block_tables,
                          int32_t block_table_stride, int32_t* lens_out, int32_t num_q_heads,
                          int32_t max_context_len, float scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return decode_step_impl(kPhaseMerge, out, out_dtype, q, key, value, slots, lens, num_seqs,
                          key_cache, value_cache, layout, block_tables, block_table_stride,
                          lens_out, num_q_heads, max_context_len, scale, workspace,
                          workspace_bytes, stream);
}

int pkv_decode_step_noalloc(void* out, int32_t out_dtype, const void* q, const void* key,
                            const void* value, const int64_t* slots, const int32_t* lens,
                            int32_t num_seqs, void* key_cache, void* value_cache,
                            const pkv_cache_layout* layout, int32_t* block_tables,
                            int32_t block_table_stride, int32_t* lens_out, int32_t num_q_heads,
                            int32_t max_context_len, float scale, void* stream) {
  if (pkv::check_layout(layout) != PKV_OK || num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0)
    return PKV_ERR_INVALID;
  const size_t need = paged_decode_attention_workspace_size(num_seqs, num_q_heads, layout->num_kv_heads,
                                                            layout->head_dim, max_context_len, 0);
  if (need > kScratchBytes) return PKV_ERR_WORKSPACE;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != PKV_OK) return st;
  return decode_step_impl(kPhasePartial | kPhaseMerge, out, out_dtype, q, key, value, slots, lens,
                          num_seqs, key_cache, value_cache, layout, block_tables,
                          block_table_stride, lens_out, num_q_heads, max_context_len, scale, ws,
                          kScratchBytes, stream);
}

int paged_decode_attention_fp8(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                               const void* key_cache, const void* value_cache,
                               const uint8_t* key_scales, const uint8_t* value_scales,
                               const int32_t* block_tables, int32_t block_table_stride,
                               const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t max_context_len, float scale, const pkv_cache_layout* layout,
                               int32_t phases, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (phases < 1 || phases > 3) return PKV_ERR_INVALID;
  const Fp8Args f8{key_scales, value_scales, q_dtype};
  return attention_impl(phases, out, out_dtype, q, key_cache, value_cache, block_tables,
                        block_table_stride, context_lens, num_seqs, num_q_heads, max_context_len,
                        scale, layout, 0, workspace, workspace_bytes, stream, nullptr, &f8);
}

int pkv_decode_step_fp8(void* out, int32_t out_dtype, const void* q, int32_t q_dtype, const void* key,
                        const void* value, const int64_t* slots, const int32_t* lens, int32_t num_seqs,
                        void* key_cache, void* value_cache, uint8_t* key_scales, uint8_t* value_scales,
                        const pkv_cache_layout* layout, int32_t* block_tables,
                        int32_t block_table_stride, int32_t* lens_out, int32_t num_q_heads,
                        int32_t max_context_len, float scale, int32_t phases, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (phases < 1 || phases > 3) return PKV_ERR_INVALID;
  if (q_dtype != PKV_BF16 && q_dtype != PKV_F16) return PKV_ERR_INVALID;
  const Fp8Step f8s{key_scales, value_scales, q_dtype};
  return decode_step_impl(phases, out, out_dtype, q, key, value, slots, lens, num_seqs, key_cache,
                          value_cache, layout, block_tables, block_table_stride, lens_out, num_q_heads,
                          max_context_len, scale, workspace, workspace_bytes, stream, &f8s);
}

int pkv_copy_table_rows(int32_t* dst, int32_t dst_stride, int32_t dst_num_rows, const int32_t* dst_rows,
                        const int32_t* src, int32_t src_stride, int32_t src_num_rows, const int32_t* src_rows,
                        int32_t n, int32_t width, void* stream) {
  if (n < 0 || width < 0 || dst_stride < width || src_stride < width || dst_num_rows < 0 || src_num_rows < 0)
    return PKV_ERR_INVALID;
  if (n == 0 || width == 0) return PKV_OK;
  if (!dst || !src) return PKV_ERR_INVALID;
  const int64_t total = static_cast<int64_t>(n) * width;
  if ((total + 255) / 256 > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(table_rows_kernel, dim3(static_cast<uint32_t>((total + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), dst, dst_stride, dst_num_rows, dst_rows, src, src_stride,
                     src_num_rows, src_rows, n, width);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_update_block_tables(int32_t* block_tables, int32_t num_rows, int32_t block_table_stride,
                            const int32_t* rows, const int32_t* lens, const int32_t* new_block,
                            int32_t n, int32_t block_size, void* stream) {
  if (n < 0 || num_rows < 0 || block_size <= 0 || block_table_stride <= 0) return PKV_ERR_INVALID;
  if (n == 0) return PKV_OK;
  if (!block_tables || !lens || !new_block) return PKV_ERR_INVALID;
  hipLaunchKernelGGL(table_update_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), block_tables, num_rows, block_table_stride,
                     rows, lens, new_block, n, block_size);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
