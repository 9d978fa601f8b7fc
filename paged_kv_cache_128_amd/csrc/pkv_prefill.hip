// Chunked-prefill attention through block tables.  Sequence b holds L_b
// cached tokens (the chunk's own K/V already written by paged_kv_write,
// [MiniPaged-Qwen] §1.1 and §12); its n_b query rows are the last n_b
// positions, row i at p = L_b - n_b + i attending to positions 0 .. p (the
// causal mask of [impl-detail] "分块注意力"), through the block table
// ([MiniPaged-Qwen] §13) with the GQA map kvh = qh / (H_q / H_kv) (§14).  A
// full prefill is n_b = L_b.
//
// Unlike decode, each K/V tile meets many query rows, so both products are
// dense contractions and run on the matrix cores.  A workgroup takes 128
// query rows of one (sequence, head): four waves of 32 rows, each as two
// 16-column MFMA blocks.  Per tile of 64 keys (four 16-key quarters, one
// staged by each wave) the workgroup stages K and V once in LDS (double-
// buffered, filled by LDS-DMA while the previous tile is being used; K rows
// XOR-swizzled so the operand reads hit distinct banks), then for each
// 32-key half of the tile every wave
//   - forms scores S^T[key][row] = K Q^T with 16x16x32 MFMAs (A = K rows,
//     B = the query rows), so lane (g4, c16) holds row c16's scores for
//     keys 4 g4 .. 4 g4 + 3 of each 16-key quarter;
//   - runs the online softmax per row over those eight scores (exp2 with
//     the scale folded in, fp32 state; the max and sum across the four lanes
//     of a row by lane swaps on the vector ALU);
//   - adds O^T[d][row] += V^T P^T with 16x16x32 MFMAs whose k index 8 g4 + e
//     stands for key 16 (e / 4) + 4 g4 + e % 4, so a lane's own eight
//     probabilities are its B operand; MFMA j maps its row index c to
//     head-dim 16 j + c, so its A operand (V at head-dim 16 j + c16 of keys
//     4 g4 .. 4 g4 + 3 of each 16-key half) comes from two transposed LDS
//     reads (ds_read_b64_tr_b16) with no lane permutes; P enters as a 16-bit
//     value plus its 16-bit remainder (two MFMAs; P to about 2^-17).
// Lane (g4, c16) ends with head-dims 16 j + 4 g4 .. 16 j + 4 g4 + 3 of its
// rows, j = 0 .. 7.  A wave
// skips the products of key ranges wholly past its rows' positions (it still
// takes part in the staging).  Keys past L read zeros (buffer range check)
// and are masked like every key past a row's position.  16-bit KV, head_dim
// 128.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_internal.h"

namespace {

constexpr int kWave = 64;
constexpr int kWavesPF = 4;
constexpr int kBlocksPerWave = 2;                     // 16-row MFMA column blocks per wave
constexpr int kRowsPerWave = 16 * kBlocksPerWave;
constexpr int kRowsPerWG = kRowsPerWave * kWavesPF;
constexpr int kKeys = 16;                             // keys per MFMA sub-tile
constexpr int kSub = 4;                               // sub-tiles per staged tile
constexpr int kD = 128;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kSlack = 8.0f;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format
constexpr int kWaitVm0 = 0x0f70;
constexpr int kSubSlots = kKeys * kD * 2 / 16;        // 16-byte LDS slots of one K sub-tile
constexpr int kTileSlots = kSub * kSubSlots;
// A V sub-tile is four blocks of four rows (block i: rows i, i + 4, i + 8,
// i + 12), each block 1 KiB followed by a 32-byte pad: the four consecutive
// rows one transposed read touches then start 32 bytes apart in the banks.
constexpr int kVBlkSlots = 4 * kD * 2 / 16 + 2;       // 16-byte slots per V block, pad included
constexpr int kVSubSlots = 4 * kVBlkSlots;
constexpr int kVTileSlots = kSub * kVSubSlots;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

struct PrefillArgs {
  const void* q;             // [T, H_q, D]
  const int32_t* q_start;    // [B + 1]
  const int32_t* lens;       // [B]
  const void* kc;
  const void* vc;
  const int32_t* tables;
  void* out;                 // [T, H_q, D]
  int64_t block_stride;      // elements
  int64_t head_stride;
  int32_t table_stride;
  int32_t num_blocks;
  int32_t block_size;
  int32_t hq;
  int32_t group;
  int32_t num_seqs;
  int32_t num_qblk;          // 128-row query blocks per sequence (the longest chunk's)
  int32_t max_len;
  int32_t out_dtype;
  float scale_log2;
};

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int DT>
__device__ __forceinline__ uint16_t to16(float f) {
  if constexpr (DT == PKV_BF16) return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
  else return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
template <int DT>
__device__ __forceinline__ float from16(uint16_t h) {
  if constexpr (DT == PKV_BF16) return __uint_as_float(static_cast<uint32_t>(h) << 16);
  else return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Two floats to a packed pair of 16-bit values (element 0 in the low half),
// rounded to nearest even; and back.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float x0, float x1) {
  if constexpr (DT == PKV_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
  else
    return static_cast<uint32_t>(to16<DT>(x0)) | (static_cast<uint32_t>(to16<DT>(x1)) << 16);
}
template <int DT>
__device__ __forceinline__ void unpack2f(uint32_t w, float& x0, float& x1) {
  if constexpr (DT == PKV_BF16) {
    x0 = __uint_as_float(w << 16);
    x1 = __uint_as_float(w & 0xffff0000u);
  } else {
    x0 = from16<DT>(static_cast<uint16_t>(w));
    x1 = from16<DT>(static_cast<uint16_t>(w >> 16));
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const char* base, int nrows) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), static_cast<short>(0),
                                           nrows * kD * 2, kRsrcWord3);
}

// One 16-byte-per-lane LDS DMA (lane i fills bytes 16 i .. 16 i + 15 from
// `lds`), written out so that the compiler does not track it: left to the
// compiler, every LDS read after a DMA waits for all outstanding DMA, which
// would hold each tile's reads until the next tile had landed and leave the
// double buffer without overlap.  The caller orders it with explicit vmcnt
// waits and barriers.  Nothing else in this file uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, const uint4* lds, int voff) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               ::"s"(m0), "v"(voff), "s"(rsrc) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int DT>
__device__ __forceinline__ f32x4 mfma_k32(const u32x4& a, const u32x4& b, f32x4 c) {
  if constexpr (DT == PKV_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  c, 0, 0, 0);
}

// Max and sum over the lanes c16, c16 + 16, c16 + 32, c16 + 48 (every lane
// gets the result), on the vector ALU: the 16-lane row swap pairs rows
// (0, 1) and (2, 3), the 32-lane half swap pairs the halves.
// The score maxima use v_max3_f32 / v_max_f32 written out: fmaxf quiets
// signalling NaNs first (the kernel runs in IEEE mode), one v_max of each
// operand with itself, and the scores are MFMA results or -inf.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max_over_g4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_g4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int DT>
__global__ void __launch_bounds__(kWave * kWavesPF) __attribute__((amdgpu_waves_per_eu(2)))
prefill_kernel(PrefillArgs a) {
  // dynamic LDS: [K tile x 2][V tile x 2] (16-byte slots), then the table entries
  extern __shared__ uint4 sh_pf[];
  uint4* sk = sh_pf;                                  // 2 x kTileSlots
  uint4* sv = sh_pf + 2 * kTileSlots;                 // 2 x kVTileSlots
  int32_t* tbl = reinterpret_cast<int32_t*>(sh_pf + 2 * kTileSlots + 2 * kVTileSlots);
  const int wave = uni(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & (kWave - 1);
  const int g4 = lane >> 4, c16 = lane & 15;
  // Workgroup order: the longest query blocks first over the whole launch;
  // within one block index, consecutive workgroups cycle through the
  // (sequence, KV head) pairs, and workgroups are handed to the XCDs in
  // turn, so each pair's query heads share one XCD's L2 (exactly when the
  // pair count is a multiple of the XCD count) and its K/V tiles, staged by
  // every one of them, are fetched from HBM about once.
  const int per_level = a.hq * a.num_seqs;
  const int qblk = a.num_qblk - 1 - static_cast<int>(blockIdx.x) / per_level;
  const int rem = static_cast<int>(blockIdx.x) % per_level;
  const int hkv = a.hq / a.group;
  const int npairs = a.num_seqs * hkv;
  const int pair = rem % npairs;
  const int b = pair / hkv;
  const int qh = (pair - b * hkv) * a.group + rem / npairs;
  const int r0 = uni(a.q_start[b]);
  const int n = uni(a.q_start[b + 1]) - r0;
  const int Lraw = uni(a.lens[b]);
  const int L = Lraw < 0 ? 0 : (Lraw > a.max_len ? a.max_len : Lraw);
  const int bs = a.block_size;
  const int wg_first = qblk * kRowsPerWG;
  if (wg_first >= n) return;                          // whole workgroup: no rows
  const int wg_last = min(wg_first + kRowsPerWG, n) - 1;
  const int wg_keys = max(0, min(L, L - n + wg_last + 1));
  const int ntiles = (wg_keys + kSub * kKeys - 1) / (kSub * kKeys);
  const int nblk = (wg_keys + bs - 1) / bs;
  for (int e = threadIdx.x; e < nblk; e += blockDim.x) {
    const int pb = a.tables[static_cast<int64_t>(b) * a.table_stride + e];
    tbl[e] = pb < 0 ? 0 : (pb >= a.num_blocks ? a.num_blocks - 1 : pb);
  }
  __syncthreads();
  const int kvh = qh / a.group;
  const int q0 = wg_first + wave * kRowsPerWave;      // this wave's first row
  // the last key any of this wave's rows sees (-1: none)
  const int w_last = min(q0 + kRowsPerWave, n) - 1;
  const int w_maxkey = q0 < n ? min(L - 1, L - n + w_last) : -1;
  int row[kBlocksPerWave], pos[kBlocksPerWave];
  bool ok[kBlocksPerWave];
  // the first key some row of this wave does not see: keys below it need no mask
  const int w_minpos = min(q0, n - 1) < 0 ? -1 : L - n + q0;
#pragma unroll
  for (int c = 0; c < kBlocksPerWave; ++c) {
    row[c] = q0 + 16 * c + c16;
    ok[c] = row[c] < n;
    pos[c] = ok[c] ? L - n + row[c] : -1;             // keys 0 .. pos
  }
  // query operands: row c16 of block c, head-dims 32 kk + 8 g4 .. + 7
  u32x4 qf[kBlocksPerWave][4];
#pragma unroll
  for (int c = 0; c < kBlocksPerWave; ++c) {
    const char* qrow = static_cast<const char*>(a.q) +
                       ((static_cast<int64_t>(r0) + (ok[c] ? row[c] : 0)) * a.hq + qh) * kD * 2;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + (32 * kk + 8 * g4) * 2);
      qf[c][kk] = ok[c] ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const char* kc = static_cast<const char*>(a.kc);
  const char* vc = static_cast<const char*>(a.vc);
  const int64_t head_off = static_cast<int64_t>(kvh) * a.head_stride;
  // Stage tile kt into buffer kt % 2: wave w moves sub-tile w, K rows
  // (chunk c of row r to slot c ^ r; DMA i: rows 4 i .. 4 i + 3) and V rows
  // (plain; DMA i: rows i, i + 4, i + 8, i + 12 into V block i), four rows
  // per 16-byte-per-lane DMA.  Rows past the workgroup's last key (a sub-tile
  // wholly past it included) read zeros, so every V value that meets a zero
  // probability is finite and only staged table entries are used.
  auto stage = [&](int kt) {
    const int key0 = (kt * kSub + wave) * kKeys;
    const int nvalid = uni(max(0, min(kKeys, wg_keys - key0)));   // uniform: keeps the DMA descriptor scalar
    const int pb = nvalid > 0 ? uni(tbl[key0 / bs]) : 0;
    const int64_t base = nvalid > 0 ? (static_cast<int64_t>(pb) * a.block_stride + head_off +
                                       static_cast<int64_t>(key0 % bs) * kD) * 2 : 0;
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc(kc + base, nvalid);
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc(vc + base, nvalid);
    uint4* dk = sk + (kt & 1) * kTileSlots + wave * kSubSlots;
    uint4* dv = sv + (kt & 1) * kVTileSlots + wave * kVSubSlots;
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * i + g4;
      dma16(rk, dk + 64 * i, r * kD * 2 + ((c16 ^ r) << 4));
      dma16(rv, dv + kVBlkSlots * i, (i + 4 * g4) * kD * 2 + (c16 << 4));
    }
    asm volatile("" ::: "memory");
  };
  float m[kBlocksPerWave], l[kBlocksPerWave];
  f32x4 acc[kBlocksPerWave][8];
#pragma unroll
  for (int c = 0; c < kBlocksPerWave; ++c) {
    m[c] = -INFINITY;
    l[c] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[c][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (ntiles > 0) stage(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();                  // tile kt staged by every wave; tile kt - 1 no longer read
    if (kt + 1 < ntiles) stage(kt + 1);
#pragma unroll 1
    for (int sub = 0; sub < kSub; sub += 2) {
      // keys key0 .. key0 + 31: staged sub-tiles sub (half 0) and sub + 1 (half 1)
      const int key0 = (kt * kSub + sub) * kKeys;
      if (key0 > w_maxkey) break;                     // every key from here on is past this wave's rows
      const uint4* tk = sk + (kt & 1) * kTileSlots + sub * kSubSlots;
      const uint4* tv = sv + (kt & 1) * kVTileSlots + sub * kVSubSlots;
      // K operands: key c16 of half h, chunk 4 kk + g4 (slot (4 kk + g4) ^ c16)
      u32x4 kf[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint4 x = tk[h * kSubSlots + c16 * 16 + ((4 * kk + g4) ^ c16)];
          kf[h][kk] = u32x4{x.x, x.y, x.z, x.w};
        }
      // scores of both halves and both column blocks: four MFMA chains
      f32x4 sa[2][kBlocksPerWave];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < kBlocksPerWave; ++c) sa[h][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int c = 0; c < kBlocksPerWave; ++c) sa[h][c] = mfma_k32<DT>(kf[h][kk], qf[c][kk], sa[h][c]);
      // The P.V A operands, read while the softmax runs: transposed read
      // (h, j) has lane i of each 16-lane group address row 4 g4 + i / 4 of
      // half h (V block i / 4, row g4 in it), head-dims 16 j + 4 (i % 4) ..
      // + 3, and gives lane c16 head-dim 16 j + c16 of rows 4 g4 .. 4 g4 + 3.
      u32x2 vt[2][8];
      {
        const char* vb = reinterpret_cast<const char*>(tv) +
                         ((c16 >> 2) * kVBlkSlots + g4 * (kD * 2 / 16)) * 16 + (c16 & 3) * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            vt[h][j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(vb + h * kVSubSlots * 16 + 32 * j)));
      }
      // P as the B operand of the 32-key P.V: lane (g4, c16) gives row c16's
      // probabilities for k = 8 g4 + e, which stands for key 16 (e / 4) +
      // 4 g4 + e % 4 -- the lane's own scores, in order
      u32x4 bh[kBlocksPerWave], bl[kBlocksPerWave];
      const bool below = key0 + 2 * kKeys - 1 <= w_minpos;   // below every row's diagonal
#pragma unroll
      for (int c = 0; c < kBlocksPerWave; ++c) {
        // raw scores, masked: the scale is positive, so the row max can be
        // taken before scaling and the scale folded into the exponent's fma
        float x[8];
        if (below) {                                  // no key past any row's position (rows past n
#pragma unroll                                        // have zero queries: finite, never written)
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[4 * h + i] = sa[h][c][i];
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              x[4 * h + i] = key0 + 16 * h + 4 * g4 + i <= pos[c] ? sa[h][c][i] : -INFINITY;
        }
        float bm = vmax2(vmax3(x[0], x[1], x[2]), vmax3(x[3], x[4], vmax3(x[5], x[6], x[7])));
        bm = max_over_g4(bm) * a.scale_log2;
        if (__builtin_amdgcn_ballot_w64(bm > m[c] + kSlack) != 0) {
          const float m_new = fmaxf(m[c], bm);
          const float f = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[c] - m_new);
          l[c] *= f;
          m[c] = m_new;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[c][j] *= f;
        }
        // exp2(-inf - m) is 0 for a finite m; a row with no visible key yet
        // (m = -inf) subtracts 0 instead, so its masked scores give 0 too
        const float msub = m[c] == -INFINITY ? 0.f : m[c];
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], a.scale_log2, -msub));
        l[c] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hw[e] = pack2<DT>(p[2 * e], p[2 * e + 1]);
          float h0, h1;
          unpack2f<DT>(hw[e], h0, h1);
          lw[e] = pack2<DT>(p[2 * e] - h0, p[2 * e + 1] - h1);
        }
        bh[c] = u32x4{hw[0], hw[1], hw[2], hw[3]};
        bl[c] = u32x4{lw[0], lw[1], lw[2], lw[3]};
      }
      // P.V: MFMA j maps its row index c to head-dim 16 j + c; its A operand is
      // head-dim 16 j + c16 of keys 4 g4 .. 4 g4 + 3 of half 0, then of half 1
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x4 av{vt[0][j][0], vt[0][j][1], vt[1][j][0], vt[1][j][1]};
#pragma unroll
        for (int c = 0; c < kBlocksPerWave; ++c) {
          acc[c][j] = mfma_k32<DT>(av, bh[c], acc[c][j]);
          acc[c][j] = mfma_k32<DT>(av, bl[c], acc[c][j]);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < kBlocksPerWave; ++c) {
    const float lc = sum_over_g4(l[c]);
    if (!ok[c]) continue;
    const float inv = lc > 0.f ? 1.0f / lc : 0.f;
    // head-dims 16 j + 4 g4 .. + 3 of the row: acc[c][j][i] is head-dim 16 j + 4 g4 + i
    const int64_t o = ((static_cast<int64_t>(r0) + row[c]) * a.hq + qh) * kD + 4 * g4;
    if (a.out_dtype == PKV_F32) {
      float* dst = static_cast<float*>(a.out) + o;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<float4*>(dst + 16 * j) =
            make_float4(acc[c][j][0] * inv, acc[c][j][1] * inv, acc[c][j][2] * inv, acc[c][j][3] * inv);
    } else {
      uint16_t* dst = static_cast<uint16_t*>(a.out) + o;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint2*>(dst + 16 * j) =
            make_uint2(static_cast<uint32_t>(to16<DT>(acc[c][j][0] * inv)) |
                           (static_cast<uint32_t>(to16<DT>(acc[c][j][1] * inv)) << 16),
                       static_cast<uint32_t>(to16<DT>(acc[c][j][2] * inv)) |
                           (static_cast<uint32_t>(to16<DT>(acc[c][j][3] * inv)) << 16));
    }
  }
}

}  // namespace

namespace {

int prefill_generic(void* out, int32_t out_dtype, const void* q, int32_t q_dtype, const int32_t* q_start,
                    const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len, const void* key_cache,
                    const void* value_cache, const uint8_t* key_scales, const uint8_t* value_scales,
                    const pkv_cache_layout* l, const int32_t* block_tables, int32_t block_table_stride,
                    int32_t num_q_heads, int32_t max_context_len, float scale, void* stream);

int prefill_16(void* out, int32_t out_dtype, const void* q, const int32_t* q_start, const int32_t* context_lens,
               int32_t num_seqs, int32_t max_q_len, const void* key_cache, const void* value_cache,
               const pkv_cache_layout* l, const int32_t* block_tables, int32_t block_table_stride,
               int32_t num_q_heads, int32_t max_context_len, float scale, void* stream) {
  if (pkv::check_layout(l) != PKV_OK || num_seqs < 0 || max_q_len < 0 || num_q_heads <= 0 ||
      max_context_len < 0 || block_table_stride < 0)
    return PKV_ERR_INVALID;
  if (num_q_heads % l->num_kv_heads != 0 || !(scale == scale)) return PKV_ERR_INVALID;
  if (l->dtype == PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;          // paged_prefill_attention_fp8
  if (l->head_dim != 64 && l->head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (out_dtype != PKV_F32 && out_dtype != l->dtype) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(block_table_stride) * l->block_size)
    return PKV_ERR_INVALID;
  if (num_seqs == 0 || max_q_len == 0) return PKV_OK;
  if (!out || !q || !q_start || !context_lens || !key_cache || !value_cache ||
      (max_context_len > 0 && !block_tables))
    return PKV_ERR_INVALID;
  // the matrix-core kernel: 16-bit KV, head_dim 128, block_size a multiple
  // of 16, 16-byte aligned rows, the table entries within LDS; any other
  // shape takes the generic kernel
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) |
                          reinterpret_cast<uintptr_t>(key_cache) | reinterpret_cast<uintptr_t>(value_cache);
  const size_t lds = static_cast<size_t>(2 * kTileSlots + 2 * kVTileSlots) * 16 +
                    static_cast<size_t>((max_context_len + l->block_size - 1) / l->block_size + 1) * 4;
  int dev = 0, lds_max = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return PKV_ERR_HIP;
  const bool mfma = (l->dtype == PKV_BF16 || l->dtype == PKV_F16) && l->head_dim == kD &&
                    l->block_size % kKeys == 0 && align % 16 == 0 && (l->head_stride * 2) % 16 == 0 &&
                    (l->block_stride * 2) % 16 == 0 && lds <= static_cast<size_t>(lds_max);
  if (!mfma)
    return prefill_generic(out, out_dtype, q, l->dtype, q_start, context_lens, num_seqs, max_q_len, key_cache,
                           value_cache, nullptr, nullptr, l, block_tables, block_table_stride, num_q_heads,
                           max_context_len, scale, stream);
  const int64_t gx = (static_cast<int64_t>(max_q_len) + kRowsPerWG - 1) / kRowsPerWG;
  if (gx * num_q_heads * num_seqs > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
  PrefillArgs a;
  a.q = q;
  a.q_start = q_start;
  a.lens = context_lens;
  a.kc = key_cache;
  a.vc = value_cache;
  a.tables = block_tables;
  a.out = out;
  a.block_stride = l->block_stride;
  a.head_stride = l->head_stride;
  a.table_stride = block_table_stride;
  a.num_blocks = l->num_blocks;
  a.block_size = l->block_size;
  a.hq = num_q_heads;
  a.group = num_q_heads / l->num_kv_heads;
  a.max_len = max_context_len;
  a.out_dtype = out_dtype;
  a.scale_log2 = scale * kLog2e;
  a.num_seqs = num_seqs;
  a.num_qblk = static_cast<int32_t>(gx);
  const dim3 grid(static_cast<uint32_t>(gx * num_q_heads * num_seqs));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const void* fn = l->dtype == PKV_BF16 ? reinterpret_cast<const void*>(&prefill_kernel<PKV_BF16>)
                                        : reinterpret_cast<const void*>(&prefill_kernel<PKV_F16>);
  if (lds > 65536 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(lds)) != hipSuccess)
    return PKV_ERR_HIP;
  if (l->dtype == PKV_BF16)
    hipLaunchKernelGGL(prefill_kernel<PKV_BF16>, grid, dim3(kWave * kWavesPF), lds, s, a);
  else
    hipLaunchKernelGGL(prefill_kernel<PKV_F16>, grid, dim3(kWave * kWavesPF), lds, s, a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

// ------------------------------------------------------------ generic prefill
// The same causal attention for the shapes the matrix-core kernel does not
// take (fp32 KV, head_dim 64, block sizes that are not a multiple of 16)
// and for 8-bit blocks read in place, each row as E4M3(code) * 2^e with the
// scale applied in fp32 (every scale exact).  One wave per (query row,
// query head), fp32 throughout: lanes take 64 keys at a time, lane l forming
// the score of key k0 + l from its whole K row (the query row broadcast from
// LDS); the wave then takes the tile's max, rescales its running state
// (online softmax, [MiniPaged-Qwen] §17.3), and adds the tile's weighted V
// rows key by key in key order, lane l owning head-dims l and l + 64.  Keys
// past the row's position are never read.  Every sum runs in a fixed order,
// so the result is reproducible bit for bit.
struct GenericArgs {
  const void* q;             // [T, H_q, D], q_dtype
  const int32_t* q_start;    // [B + 1]
  const int32_t* lens;       // [B]
  const void* kc;
  const void* vc;
  const uint8_t* ks;         // 8-bit KV: scale bytes
  const uint8_t* vs;
  const int32_t* tables;
  void* out;                 // [T, H_q, D]
  int64_t block_stride;      // elements
  int64_t head_stride;
  int64_t sblock_stride;     // scale bytes (8-bit KV)
  int64_t shead_stride;
  int32_t table_stride;
  int32_t num_blocks;
  int32_t block_size;
  int32_t hq;
  int32_t group;
  int32_t num_seqs;
  int32_t max_q_len;         // rows per sequence slot of the grid
  int32_t max_len;
  int32_t out_dtype;
  float scale_log2;
};

// Element i of a row of type DT, widened to fp32 (8-bit: the code's value
// before its row scale).
template <int DT>
__device__ __forceinline__ float elem_f32(const void* row, int i) {
  if constexpr (DT == PKV_F32) return static_cast<const float*>(row)[i];
  else if constexpr (DT == PKV_BF16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(row)[i]) << 16);
  else if constexpr (DT == PKV_F16) return static_cast<float>(static_cast<const _Float16*>(row)[i]);
  else {
    const uint8_t c = static_cast<const uint8_t*>(row)[i];
    return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(c), 0);
  }
}

template <int KT, int QT, int D>
__global__ void __launch_bounds__(kWave)
prefill_generic_kernel(GenericArgs a) {
  constexpr int kEb = KT == PKV_F32 ? 4 : (KT == PKV_FP8_E4M3 ? 1 : 2);
  constexpr int kPer = D / kWave;
  __shared__ float qs[D];
  const int lane = threadIdx.x;
  // workgroup (b, i, qh): query row i of sequence b, query head qh
  const int qh = static_cast<int>(blockIdx.x % a.hq);
  const int64_t t = blockIdx.x / a.hq;
  const int i_row = static_cast<int>(t % a.max_q_len);
  const int b = static_cast<int>(t / a.max_q_len);
  const int r0 = a.q_start[b], n = a.q_start[b + 1] - r0;
  if (i_row >= n) return;
  const int64_t trow = static_cast<int64_t>(r0) + i_row;
  const int Lraw = a.lens[b];
  const int L = Lraw < 0 ? 0 : (Lraw > a.max_len ? a.max_len : Lraw);
  const int pos = L - n + i_row;                            // keys 0 .. pos
  const int64_t o = (trow * a.hq + qh) * D;
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  if (pos >= 0) {
    for (int d = lane; d < D; d += kWave) qs[d] = elem_f32<QT>(static_cast<const char*>(a.q) + o * (QT == PKV_F32 ? 4 : 2), d);
    __syncthreads();
    const int kvh = qh / a.group;
    const char* kc = static_cast<const char*>(a.kc);
    const char* vc = static_cast<const char*>(a.vc);
    const int bs = a.block_size;
    for (int k0 = 0; k0 <= pos; k0 += kWave) {
      const int k = k0 + lane;
      const bool valid = k <= pos;
      // this lane's key: its row offset (elements) and, for 8-bit KV, its scale bytes' offset
      int64_t roff = 0, soff = 0;
      if (valid) {
        int pb = a.tables[static_cast<int64_t>(b) * a.table_stride + k / bs];
        pb = pb < 0 ? 0 : (pb >= a.num_blocks ? a.num_blocks - 1 : pb);
        roff = static_cast<int64_t>(pb) * a.block_stride + static_cast<int64_t>(kvh) * a.head_stride +
               static_cast<int64_t>(k % bs) * D;
        soff = static_cast<int64_t>(pb) * a.sblock_stride + static_cast<int64_t>(kvh) * a.shead_stride + k % bs;
      }
      float sc = -INFINITY;
      if (valid) {
        const char* krow = kc + roff * kEb;
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(qs[d], elem_f32<KT>(krow, d), dot);
        if constexpr (KT == PKV_FP8_E4M3) dot = __builtin_amdgcn_ldexpf(dot, static_cast<int>(a.ks[soff]) - 127);
        sc = dot * a.scale_log2;
      }
      float tm = sc;
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) tm = fmaxf(tm, __shfl_xor(tm, off));
      const float m_new = fmaxf(m, tm);
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
      const float p = valid ? __builtin_amdgcn_exp2f(sc - m_new) : 0.f;
      float ps = p;
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
      l = l * alpha + ps;
      m = m_new;
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[e] *= alpha;
      const int nk = min(kWave, pos - k0 + 1);
      for (int j = 0; j < nk; ++j) {
        const float pj = __shfl(p, j);
        const int64_t rj = __shfl(roff, j);
        float vsc = 1.f;
        if constexpr (KT == PKV_FP8_E4M3) vsc = __builtin_amdgcn_ldexpf(1.f, static_cast<int>(a.vs[__shfl(soff, j)]) - 127);
        const char* vrow = vc + rj * kEb;
#pragma unroll
        for (int e = 0; e < kPer; ++e) acc[e] = fmaf(pj, elem_f32<KT>(vrow, e * kWave + lane) * vsc, acc[e]);
      }
    }
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const float y = acc[e] * inv;
    const int64_t i = o + e * kWave + lane;
    if (a.out_dtype == PKV_F32) static_cast<float*>(a.out)[i] = y;
    else if (a.out_dtype == PKV_BF16) static_cast<uint16_t*>(a.out)[i] = to16<PKV_BF16>(y);
    else static_cast<uint16_t*>(a.out)[i] = to16<PKV_F16>(y);
  }
}

template <int KT, int QT>
hipError_t launch_generic(const GenericArgs& a, int D, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.num_seqs) * a.max_q_len * a.hq));
  if (D == 64) hipLaunchKernelGGL((prefill_generic_kernel<KT, QT, 64>), grid, dim3(kWave), 0, s, a);
  else hipLaunchKernelGGL((prefill_generic_kernel<KT, QT, 128>), grid, dim3(kWave), 0, s, a);
  return hipGetLastError();
}

// Validates and launches the generic kernel: cache type l->dtype (8-bit:
// key_scales / value_scales given), queries of type q_dtype (the cache's
// for 16- and 32-bit KV; bf16 or fp16 for 8-bit KV).
int prefill_generic(void* out, int32_t out_dtype, const void* q, int32_t q_dtype, const int32_t* q_start,
                    const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len, const void* key_cache,
                    const void* value_cache, const uint8_t* key_scales, const uint8_t* value_scales,
                    const pkv_cache_layout* l, const int32_t* block_tables, int32_t block_table_stride,
                    int32_t num_q_heads, int32_t max_context_len, float scale, void* stream) {
  if (l->head_dim != 64 && l->head_dim != 128) return PKV_ERR_UNSUPPORTED;
  const int64_t waves = static_cast<int64_t>(num_seqs) * max_q_len * num_q_heads;
  if (waves > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
  GenericArgs a;
  a.q = q;
  a.q_start = q_start;
  a.lens = context_lens;
  a.kc = key_cache;
  a.vc = value_cache;
  a.ks = key_scales;
  a.vs = value_scales;
  a.tables = block_tables;
  a.out = out;
  a.block_stride = l->block_stride;
  a.head_stride = l->head_stride;
  a.sblock_stride = l->block_stride / l->head_dim;
  a.shead_stride = l->head_stride / l->head_dim;
  a.table_stride = block_table_stride;
  a.num_blocks = l->num_blocks;
  a.block_size = l->block_size;
  a.hq = num_q_heads;
  a.group = num_q_heads / l->num_kv_heads;
  a.num_seqs = num_seqs;
  a.max_q_len = max_q_len;
  a.max_len = max_context_len;
  a.out_dtype = out_dtype;
  a.scale_log2 = scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (l->dtype) {
    case PKV_F32: e = launch_generic<PKV_F32, PKV_F32>(a, l->head_dim, s); break;
    case PKV_F16: e = launch_generic<PKV_F16, PKV_F16>(a, l->head_dim, s); break;
    case PKV_BF16: e = launch_generic<PKV_BF16, PKV_BF16>(a, l->head_dim, s); break;
    default:
      e = q_dtype == PKV_BF16 ? launch_generic<PKV_FP8_E4M3, PKV_BF16>(a, l->head_dim, s)
                              : launch_generic<PKV_FP8_E4M3, PKV_F16>(a, l->head_dim, s);
  }
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

// 8-bit blocks for prefill: one workgroup per (sequence b, logical block j,
// K or V, KV head) writes that head's rows of block tables[b][j], read back
// as decode(code) * 2^(scale byte - 127), into 16-bit staging block
// b * W + j, and workgroup (b, j, K, head 0) writes that block's id into
// the staging table [B, W]; blocks past a sequence's length are skipped.
// The staging type is the queries': bf16 holds every row with a scale of
// 2^-124 .. 2^119 exactly; fp16 every row with a scale of 2^-15 .. 2^7 (the
// rows of fp16 tensors, short of the few within 0.05 % of fp16's largest
// value), larger values clamping to +-65504 and smaller scales keeping
// their values to the nearest 2^-24.
struct DequantArgs {
  const uint8_t* kc;
  const uint8_t* vc;
  const uint8_t* ks;
  const uint8_t* vs;
  const int32_t* tables;
  const int32_t* lens;
  uint16_t* staging;        // [B * W, 2, H, bs, D] bf16
  int32_t* table_out;       // [B, W]
  int64_t block_stride;     // elements (= bytes) of the code pool
  int64_t head_stride;
  int64_t sblock_stride;    // scale bytes
  int64_t shead_stride;
  int32_t table_stride;
  int32_t num_blocks;
  int32_t block_size;
  int32_t heads;
  int32_t width;            // W
  int32_t max_len;
  int32_t to_f16;           // staging type: fp16 (else bf16)
};

// fp16's largest finite value in place of anything larger in magnitude;
// NaN stays NaN.
__device__ __forceinline__ float clamp_f16(float x) {
  return fabsf(x) > 65504.f ? copysignf(65504.f, x) : x;
}

__global__ void __launch_bounds__(256)
dequant_blocks_kernel(DequantArgs a) {
  int64_t item = blockIdx.x;
  const int h = static_cast<int>(item % a.heads);
  item /= a.heads;
  const int half = static_cast<int>(item % 2);
  item /= 2;
  const int j = static_cast<int>(item % a.width);
  const int b = static_cast<int>(item / a.width);
  const int bs = a.block_size;
  const int Lraw = a.lens[b];
  const int L = Lraw < 0 ? 0 : (Lraw > a.max_len ? a.max_len : Lraw);
  if (j >= (L + bs - 1) / bs) return;
  int pb = a.tables[static_cast<int64_t>(b) * a.table_stride + j];
  pb = pb < 0 ? 0 : (pb >= a.num_blocks ? a.num_blocks - 1 : pb);
  const int64_t dst = static_cast<int64_t>(b) * a.width + j;
  if (half == 0 && h == 0 && threadIdx.x == 0) a.table_out[dst] = static_cast<int32_t>(dst);
  const uint8_t* codes = (half == 0 ? a.kc : a.vc) + pb * a.block_stride + h * a.head_stride;
  const uint8_t* scales = (half == 0 ? a.ks : a.vs) + pb * a.sblock_stride + h * a.shead_stride;
  uint16_t* o = a.staging + ((dst * 2 + half) * a.heads + h) * static_cast<int64_t>(bs) * kD;
  // eight codes per thread: row (8 i) / D, columns 8 i % D .. + 7
  for (int i = threadIdx.x; i < bs * kD / 8; i += blockDim.x) {
    const int r = (8 * i) / kD;
    const uint2 w = *reinterpret_cast<const uint2*>(codes + static_cast<int64_t>(r) * kD + (8 * i) % kD);
    const int e = static_cast<int>(scales[r]) - 127;
    // the hardware E4M3 conversion: bytes 0-1 (false) or 2-3 (true) of a word
    const f32x2 v[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w.x), false),
                        __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w.x), true),
                        __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w.y), false),
                        __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w.y), true)};
    uint32_t packed[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x0 = __builtin_amdgcn_ldexpf(v[k].x, e), x1 = __builtin_amdgcn_ldexpf(v[k].y, e);
      packed[k] = a.to_f16 ? pack2<PKV_F16>(clamp_f16(x0), clamp_f16(x1)) : pack2<PKV_BF16>(x0, x1);
    }
    *reinterpret_cast<uint4*>(o + 8 * static_cast<int64_t>(i)) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
}

// Staging size for num_seqs sequences of up to max_context_len tokens:
// W = ceil(max_context_len / bs) blocks each (16-bit K and V of every head)
// plus the [B, W] table.
size_t fp8_staging_bytes(int32_t num_seqs, int32_t max_context_len, const pkv_cache_layout* l) {
  const int64_t W = (static_cast<int64_t>(max_context_len) + l->block_size - 1) / l->block_size;
  const int64_t blocks = static_cast<int64_t>(num_seqs) * W;
  const int64_t block_bytes = 2LL * l->num_kv_heads * l->block_size * l->head_dim * 2;
  const int64_t table_off = (blocks * block_bytes + 255) / 256 * 256;
  return static_cast<size_t>(table_off + blocks * 4);
}

}  // namespace

extern "C" int paged_prefill_attention(void* out, int32_t out_dtype, const void* q,
                                       const int32_t* q_start, const int32_t* context_lens,
                                       int32_t num_seqs, int32_t max_q_len, const void* key_cache,
                                       const void* value_cache, const pkv_cache_layout* l,
                                       const int32_t* block_tables, int32_t block_table_stride,
                                       int32_t num_q_heads, int32_t max_context_len, float scale,
                                       void* stream) {
  if (pkv::check_layout(l) == PKV_OK && l->dtype == PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;
  return prefill_16(out, out_dtype, q, q_start, context_lens, num_seqs, max_q_len, key_cache, value_cache, l,
                    block_tables, block_table_stride, num_q_heads, max_context_len, scale, stream);
}

extern "C" size_t paged_prefill_attention_fp8_workspace_size(int32_t num_seqs, int32_t max_context_len,
                                                            const pkv_cache_layout* l) {
  if (pkv::check_layout(l) != PKV_OK || num_seqs < 0 || max_context_len < 0) return 0;
  return fp8_staging_bytes(num_seqs, max_context_len, l);
}

extern "C" int paged_prefill_attention_fp8(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                                           const int32_t* q_start, const int32_t* context_lens, int32_t num_seqs,
                                           int32_t max_q_len, const void* key_cache, const void* value_cache,
                                           const uint8_t* key_scales, const uint8_t* value_scales,
                                           const pkv_cache_layout* l, const int32_t* block_tables,
                                           int32_t block_table_stride, int32_t num_q_heads, int32_t max_context_len,
                                           float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (pkv::check_layout(l) != PKV_OK || num_seqs < 0 || max_q_len < 0 || num_q_heads <= 0 ||
      max_context_len < 0 || block_table_stride < 0)
    return PKV_ERR_INVALID;
  if (l->dtype != PKV_FP8_E4M3 || (q_dtype != PKV_BF16 && q_dtype != PKV_F16)) return PKV_ERR_UNSUPPORTED;
  if (l->head_dim != 64 && l->head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (num_q_heads % l->num_kv_heads != 0 || !(scale == scale)) return PKV_ERR_INVALID;
  if (out_dtype != PKV_F32 && out_dtype != q_dtype) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(block_table_stride) * l->block_size)
    return PKV_ERR_INVALID;
  if (l->head_stride % l->head_dim != 0 || l->block_stride % l->head_dim != 0) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_q_len == 0) return PKV_OK;
  if (!out || !q || !q_start || !key_cache || !value_cache || !key_scales || !value_scales || !context_lens ||
      (max_context_len > 0 && !block_tables))
    return PKV_ERR_INVALID;
  // bf16 queries, head_dim 128, block_size a multiple of 16: the blocks
  // dequantised into the bf16 staging, then the matrix-core kernel; any
  // other case (fp16 queries included, whose 16-bit type could not hold
  // every read-back value) reads the codes in place in the generic kernel
  if (q_dtype != PKV_BF16 || l->head_dim != kD || l->block_size % kKeys != 0 ||
      ((reinterpret_cast<uintptr_t>(key_cache) | reinterpret_cast<uintptr_t>(value_cache)) % 8) != 0 ||
      l->head_stride % 8 != 0 || l->block_stride % 8 != 0)
    return prefill_generic(out, out_dtype, q, q_dtype, q_start, context_lens, num_seqs, max_q_len, key_cache,
                           value_cache, key_scales, value_scales, l, block_tables, block_table_stride, num_q_heads,
                           max_context_len, scale, stream);
  const size_t need = fp8_staging_bytes(num_seqs, max_context_len, l);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return PKV_ERR_WORKSPACE;
  const int32_t W = (max_context_len + l->block_size - 1) / l->block_size;
  const int64_t blocks = static_cast<int64_t>(num_seqs) * W;
  const int64_t block_elems = 2LL * l->num_kv_heads * l->block_size * l->head_dim;
  if (blocks > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
  uint16_t* staging = static_cast<uint16_t*>(workspace);
  int32_t* table_out = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                                  (blocks * block_elems * 2 + 255) / 256 * 256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (blocks > 0) {
    DequantArgs d;
    d.kc = static_cast<const uint8_t*>(key_cache);
    d.vc = static_cast<const uint8_t*>(value_cache);
    d.ks = key_scales;
    d.vs = value_scales;
    d.tables = block_tables;
    d.lens = context_lens;
    d.staging = staging;
    d.table_out = table_out;
    d.block_stride = l->block_stride;
    d.head_stride = l->head_stride;
    d.sblock_stride = l->block_stride / l->head_dim;
    d.shead_stride = l->head_stride / l->head_dim;
    d.table_stride = block_table_stride;
    d.num_blocks = l->num_blocks;
    d.block_size = l->block_size;
    d.heads = l->num_kv_heads;
    d.width = W;
    d.max_len = max_context_len;
    d.to_f16 = q_dtype == PKV_F16;
    const int64_t grid = blocks * 2 * l->num_kv_heads;
    if (grid > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(dequant_blocks_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s, d);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  pkv_cache_layout sl = *l;
  sl.num_blocks = static_cast<int32_t>(blocks > 0 ? blocks : 1);
  sl.dtype = q_dtype;
  sl.block_stride = block_elems;
  sl.head_stride = static_cast<int64_t>(l->block_size) * l->head_dim;
  return prefill_16(out, out_dtype, q, q_start, context_lens, num_seqs, max_q_len, staging,
                    staging + static_cast<int64_t>(l->num_kv_heads) * l->block_size * l->head_dim, &sl,
                    table_out, W, num_q_heads, max_context_len, scale, stream);
}

