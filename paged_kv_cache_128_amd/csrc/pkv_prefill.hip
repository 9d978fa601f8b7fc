// Chunked-prefill attention through block tables.  Sequence b holds L_b
// cached tokens (the chunk's own K/V already written by paged_kv_write,
// [MiniPaged-Qwen] §1.1 and §12); its n_b query rows are the last n_b
// positions, row i at p = L_b - n_b + i attending to positions 0 .. p (the
// causal mask of [impl-detail] "分块注意力"), through the block table
// ([MiniPaged-Qwen] §13) with the GQA map kvh = qh / (H_q / H_kv) (§14).  A
// full prefill is n_b = L_b.
//
// Unlike decode, each K/V tile meets many query rows, so both products are
// dense contractions and run on the matrix cores.  One wave takes 16 query
// rows of one head; a workgroup four waves (64 rows) of one (sequence, head),
// and it stages the sequence's block-table entries in LDS once.  Per tile of
// 16 keys:
//   - scores S^T[key][row] = K Q^T by four 16x16x32 MFMAs (A = K rows as
//     loaded, B = the query rows), so lane (g4, c16) holds row c16's scores
//     for keys 4 g4 .. 4 g4 + 3 -- which is the B operand layout of P.V;
//   - online softmax per row (exp2 with the scale folded in, fp32 state);
//   - O^T[d][row] += V^T P^T by 16x16x16 MFMAs: MFMA j maps its row index c
//     to head-dim 8 c + j, so its A operand is element j of the lane's V
//     rows 4 g4 .. 4 g4 + 3 at head-dims 8 c16 .. 8 c16 + 7 (as loaded), and
//     P enters as a 16-bit high part plus a 16-bit remainder (two MFMAs),
//     which keeps P to about 2^-17 of its value.
// Lane (g4, c16) ends with row c16's head-dims 32 g4 .. 32 g4 + 31.  The next
// tile's K and V are fetched while the current one's P.V runs.  Keys past L
// read zeros (buffer range check) and are masked like every key past the
// row's position.  16-bit KV, head_dim 128.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_internal.h"

namespace {

constexpr int kWave = 64;
constexpr int kRowsPerWave = 16;
constexpr int kWavesPF = 4;
constexpr int kRowsPerWG = kRowsPerWave * kWavesPF;
constexpr int kKeys = 16;
constexpr int kD = 128;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kSlack = 8.0f;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format
constexpr int kWaitVm0 = 0x0f70;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

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
  int32_t max_len;
  int32_t out_dtype;
  float scale_log2;
};

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <int DT>
__device__ __forceinline__ uint16_t to16(float f) {
  if constexpr (DT == PKV_BF16) return f32_to_bf16_rne(f);
  else return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
template <int DT>
__device__ __forceinline__ float from16(uint16_t h) {
  if constexpr (DT == PKV_BF16) return __uint_as_float(static_cast<uint32_t>(h) << 16);
  else return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const char* base, int nrows) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), static_cast<short>(0),
                                           nrows * kD * 2, kRsrcWord3);
}

template <int DT>
__device__ __forceinline__ f32x4 mfma_qk(const u32x4& a, const u32x4& b, f32x4 c) {
  if constexpr (DT == PKV_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ f32x4 mfma_pv(const u32x2& a, const u32x2& b, f32x4 c) {
  if constexpr (DT == PKV_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b),
                                                     c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b),
                                                 c, 0, 0, 0);
}

struct KV {
  u32x4 k[4];   // K operand: key c16, head-dims 32 kk + 8 g4 .. + 7
  u32x4 v[4];   // V rows 4 g4 + r, head-dims 8 c16 .. + 7
};

template <int DT>
__global__ void __launch_bounds__(kWave * kWavesPF)
prefill_kernel(PrefillArgs a) {
  extern __shared__ int32_t sh_tbl[];
  const int wave = uni(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & (kWave - 1);
  const int g4 = lane >> 4, c16 = lane & 15;
  const int b = blockIdx.z, qh = blockIdx.y;
  const int r0 = uni(a.q_start[b]);
  const int n = uni(a.q_start[b + 1]) - r0;
  const int Lraw = uni(a.lens[b]);
  const int L = Lraw < 0 ? 0 : (Lraw > a.max_len ? a.max_len : Lraw);
  const int bs = a.block_size;
  // keys the workgroup's rows can see: up to the last of its rows' positions
  const int wg_last = min(static_cast<int>(blockIdx.x) * kRowsPerWG + kRowsPerWG, n) - 1;
  const int wg_keys = wg_last < 0 ? 0 : max(0, min(L, L - n + wg_last + 1));
  const int nblk = (wg_keys + bs - 1) / bs;
  for (int e = threadIdx.x; e < nblk; e += blockDim.x) {
    const int pb = a.tables[static_cast<int64_t>(b) * a.table_stride + e];
    sh_tbl[e] = pb < 0 ? 0 : (pb >= a.num_blocks ? a.num_blocks - 1 : pb);
  }
  __syncthreads();
  const int q0 = blockIdx.x * kRowsPerWG + wave * kRowsPerWave;
  if (q0 >= n) return;
  const int kvh = qh / a.group;
  const int my_row = q0 + c16;
  const bool row_ok = my_row < n;
  const int my_pos = row_ok ? L - n + my_row : -1;       // keys 0 .. my_pos
  const int last_row = min(q0 + kRowsPerWave, n) - 1;
  const int nkeys = max(0, min(L, L - n + last_row + 1));
  const int ntiles = (nkeys + kKeys - 1) / kKeys;
  // query operand: row c16, head-dims 32 kk + 8 g4 .. + 7
  u32x4 qf[4];
  {
    const char* qrow = static_cast<const char*>(a.q) +
                       ((static_cast<int64_t>(r0) + (row_ok ? my_row : 0)) * a.hq + qh) * kD * 2;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + (32 * kk + 8 * g4) * 2);
      qf[kk] = row_ok ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const char* kc = static_cast<const char*>(a.kc);
  const char* vc = static_cast<const char*>(a.vc);
  const int64_t head_off = static_cast<int64_t>(kvh) * a.head_stride;
  auto fetch = [&](KV& t, int kt) {
    const int key0 = kt * kKeys;
    const int pb = uni(sh_tbl[key0 / bs]);
    const int64_t base = (static_cast<int64_t>(pb) * a.block_stride + head_off +
                          static_cast<int64_t>(key0 % bs) * kD) * 2;
    const int nvalid = min(kKeys, L - key0);
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc(kc + base, nvalid);
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc(vc + base, nvalid);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      t.k[kk] = __builtin_amdgcn_raw_buffer_load_b128(rk, c16 * kD * 2 + (32 * kk + 8 * g4) * 2, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      t.v[r] = __builtin_amdgcn_raw_buffer_load_b128(rv, (4 * g4 + r) * kD * 2 + c16 * 16, 0, 0);
  };
  float m = -INFINITY, l = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  KV cur, nxt;
  if (ntiles > 0) fetch(cur, 0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) s = mfma_qk<DT>(cur.k[kk], qf[kk], s);
    if (kt + 1 < ntiles) fetch(nxt, kt + 1);
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kt * kKeys + 4 * g4 + i;
      x[i] = key <= my_pos ? s[i] * a.scale_log2 : -INFINITY;
    }
    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    if (__builtin_amdgcn_ballot_w64(bm > m + kSlack) != 0) {
      const float m_new = fmaxf(m, bm);
      const float f = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
      l *= f;
      m = m_new;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= f;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = x[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[i] - m);
    l += (p[0] + p[1]) + (p[2] + p[3]);
    // P as a 16-bit high part and remainder (B operand: keys 4 g4 + i, row c16)
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hi[i] = to16<DT>(p[i]);
      lo[i] = to16<DT>(p[i] - from16<DT>(hi[i]));
    }
    const u32x2 bh = {static_cast<uint32_t>(hi[0]) | (static_cast<uint32_t>(hi[1]) << 16),
                      static_cast<uint32_t>(hi[2]) | (static_cast<uint32_t>(hi[3]) << 16)};
    const u32x2 bl = {static_cast<uint32_t>(lo[0]) | (static_cast<uint32_t>(lo[1]) << 16),
                      static_cast<uint32_t>(lo[2]) | (static_cast<uint32_t>(lo[3]) << 16)};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // element j of V rows 4 g4 + r: half (j % 2) of dword j / 2
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      const u32x2 av = {__builtin_amdgcn_perm(cur.v[1][j >> 1], cur.v[0][j >> 1], sel),
                        __builtin_amdgcn_perm(cur.v[3][j >> 1], cur.v[2][j >> 1], sel)};
      acc[j] = mfma_pv<DT>(av, bh, acc[j]);
      acc[j] = mfma_pv<DT>(av, bl, acc[j]);
    }
    if (kt + 1 < ntiles) cur = nxt;
  }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (!row_ok) return;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const int64_t o = ((static_cast<int64_t>(r0) + my_row) * a.hq + qh) * kD + 32 * g4;
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) v[8 * i + j] = acc[j][i] * inv;
  if (a.out_dtype == PKV_F32) {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.out) + o);
#pragma unroll
    for (int k = 0; k < 8; ++k) dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  } else {
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + o);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = static_cast<uint32_t>(to16<DT>(v[8 * k + 2 * e])) |
               (static_cast<uint32_t>(to16<DT>(v[8 * k + 2 * e + 1])) << 16);
      dst[k] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

}  // namespace

extern "C" int paged_prefill_attention(void* out, int32_t out_dtype, const void* q,
                                       const int32_t* q_start, const int32_t* context_lens,
                                       int32_t num_seqs, int32_t max_q_len, const void* key_cache,
                                       const void* value_cache, const pkv_cache_layout* l,
                                       const int32_t* block_tables, int32_t block_table_stride,
                                       int32_t num_q_heads, int32_t max_context_len, float scale,
                                       void* stream) {
  if (pkv::check_layout(l) != PKV_OK || num_seqs < 0 || max_q_len < 0 || num_q_heads <= 0 ||
      max_context_len < 0 || block_table_stride < 0)
    return PKV_ERR_INVALID;
  if (num_q_heads % l->num_kv_heads != 0 || !(scale == scale)) return PKV_ERR_INVALID;
  if (l->dtype != PKV_BF16 && l->dtype != PKV_F16) return PKV_ERR_UNSUPPORTED;
  if (l->head_dim != kD || l->block_size % kKeys != 0) return PKV_ERR_UNSUPPORTED;
  if (out_dtype != PKV_F32 && out_dtype != l->dtype) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(block_table_stride) * l->block_size)
    return PKV_ERR_INVALID;
  if (num_seqs == 0 || max_q_len == 0) return PKV_OK;
  if (!out || !q || !q_start || !context_lens || !key_cache || !value_cache ||
      (max_context_len > 0 && !block_tables))
    return PKV_ERR_INVALID;
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) |
                          reinterpret_cast<uintptr_t>(key_cache) | reinterpret_cast<uintptr_t>(value_cache);
  if (align % 16 != 0 || (l->head_stride * 2) % 16 != 0 || (l->block_stride * 2) % 16 != 0)
    return PKV_ERR_UNSUPPORTED;
  const size_t lds = static_cast<size_t>((max_context_len + l->block_size - 1) / l->block_size + 1) * 4;
  if (lds > 65536) return PKV_ERR_UNSUPPORTED;
  const int64_t gx = (static_cast<int64_t>(max_q_len) + kRowsPerWG - 1) / kRowsPerWG;
  if (gx > 0x7fffffffLL || num_q_heads > 65535 || num_seqs > 65535) return PKV_ERR_UNSUPPORTED;
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
  const dim3 grid(static_cast<uint32_t>(gx), static_cast<uint32_t>(num_q_heads),
                  static_cast<uint32_t>(num_seqs));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (l->dtype == PKV_BF16)
    hipLaunchKernelGGL(prefill_kernel<PKV_BF16>, grid, dim3(kWave * kWavesPF), lds, s, a);
  else
    hipLaunchKernelGGL(prefill_kernel<PKV_F16>, grid, dim3(kWave * kWavesPF), lds, s, a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
