// Cache writes into FP8 KV blocks.  [impl-detail] "实践建议" notes that the
// KV inside a block can be quantised on its own; here every token row of
// every KV head is quantised on its own as it is written, so a filling
// block never needs re-quantising:
//   e    = the smallest integer with max|x| <= 448 * 2^e (clamped to
//          [-126, 127]; 0 for an all-zero row), stored as the OCP E8M0 byte
//          e + 127;
//   code = OCP E4M3 of x * 2^-e, round to nearest even (x * 2^-e is exact
//          in float32, so this is the only rounding); a code of negative
//          zero is stored as 0x00.
// The row's value reads back as E4M3(code) * 2^e.
//
// One group of D / 8 lanes per row: each lane takes eight values, the
// group's max |x| comes from a butterfly over its lanes, and each lane
// stores its eight codes as one 8-byte word; the group's first lane stores
// the scale byte.  Scale bytes mirror the code layout with one byte per
// row: the scale of row (pb, h, off) sits at
//   scales + pb * (block_stride / D) + h * (head_stride / D) + off.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_fp8_codec.h"
#include "pkv_internal.h"

namespace {

constexpr int kThreads = 256;

// Eight source values of one row, widened to float32.
__device__ __forceinline__ void load8(const void* src, int dtype, int64_t elem, float (&x)[8]) {
  if (dtype == PKV_F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(src) + elem);
    const uint4 a = p[0], b = p[1];
    x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
    x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
    x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
    x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + elem);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (dtype == PKV_BF16) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      } else {
        x[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] & 0xffffu)));
        x[2 * i + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16)));
      }
    }
  }
}

// Quantises one row held by a group of `lpr` lanes (lane `sub` has elements
// 8 sub .. 8 sub + 7) and stores codes and scale.
__device__ __forceinline__ void quantize_store(const float (&x)[8], int lpr, int sub,
                                               uint8_t* code_row, uint8_t* scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, pkv::finite_abs(x[i]));
  for (int o = lpr / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const int e = pkv::row_exponent(amax);
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w0 |= pkv::e4m3_code(__builtin_amdgcn_ldexpf(x[i], -e)) << (8 * i);
    w1 |= pkv::e4m3_code(__builtin_amdgcn_ldexpf(x[4 + i], -e)) << (8 * i);
  }
  *reinterpret_cast<uint2*>(code_row + 8 * sub) = make_uint2(w0, w1);
  if (sub == 0) *scale = static_cast<uint8_t>(e + 127);
}

struct Fp8Dst {
  uint8_t* kc;
  uint8_t* vc;
  uint8_t* ks;
  uint8_t* vs;
  int64_t block_stride;   // bytes (= elements)
  int64_t head_stride;
  int64_t capacity;       // num_blocks * block_size
  int32_t block_size;
  int32_t heads;
  int32_t head_dim;
};

// Row r of the launch: token r / (2 H), K (0) or V (1), head r % H.
__device__ __forceinline__ void write_row(const Fp8Dst& d, const void* key, const void* value,
                                          int dtype, int64_t tok_src, int64_t slot, int half, int h,
                                          int lpr, int sub) {
  if (slot < 0 || slot >= d.capacity) return;
  float x[8];
  load8(half == 0 ? key : value, dtype, (tok_src * d.heads + h) * d.head_dim + 8 * sub, x);
  const int64_t pb = slot / d.block_size, off = slot - pb * d.block_size;
  const int64_t row = pb * d.block_stride + h * d.head_stride + off * d.head_dim;
  const int64_t srow = pb * (d.block_stride / d.head_dim) + h * (d.head_stride / d.head_dim) + off;
  quantize_store(x, lpr, sub, (half == 0 ? d.kc : d.vc) + row, (half == 0 ? d.ks : d.vs) + srow);
}

__global__ void __launch_bounds__(kThreads)
kv_write_fp8_kernel(const void* __restrict__ key, const void* __restrict__ value, int32_t dtype,
                    const int64_t* __restrict__ slots, int64_t rows, Fp8Dst d) {
  const int lpr = d.head_dim / 8;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (kThreads / lpr) + threadIdx.x / lpr;
  const int sub = threadIdx.x % lpr;
  if (r >= rows) return;                         // whole groups leave together
  const int64_t t = r / (2 * d.heads);
  const int rem = static_cast<int>(r - t * 2 * d.heads);
  write_row(d, key, value, dtype, t, slots[t], rem / d.heads, rem % d.heads, lpr, sub);
}

__global__ void __launch_bounds__(kThreads)
decode_write_fp8_kernel(pkv::StepMeta meta, int32_t n, int32_t row0, const void* __restrict__ key,
                        const void* __restrict__ value, int32_t dtype, Fp8Dst d,
                        int32_t* __restrict__ tables, int32_t table_rows, int32_t table_stride,
                        int32_t* __restrict__ lens_out) {
  const int lpr = d.head_dim / 8;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (kThreads / lpr) + threadIdx.x / lpr;
  const int sub = threadIdx.x % lpr;
  if (r >= static_cast<int64_t>(n) * 2 * d.heads) return;
  const int32_t t = static_cast<int32_t>(r / (2 * d.heads));
  const int rem = static_cast<int>(r - static_cast<int64_t>(t) * 2 * d.heads);
  const int64_t slot = meta.slots[t];
  if (rem == 0 && sub == 0) {
    const int32_t len = meta.lens[t];
    const int32_t row = row0 + t;
    if (lens_out) lens_out[row] = len;
    if (tables && row < table_rows && len > 0 && slot >= 0 && slot < d.capacity &&
        (len - 1) / d.block_size < table_stride)
      tables[static_cast<int64_t>(row) * table_stride + (len - 1) / d.block_size] =
          static_cast<int32_t>(slot / d.block_size);
  }
  write_row(d, key, value, dtype, row0 + t, slot, rem / d.heads, rem % d.heads, lpr, sub);
}

// Shared argument checks; fills `d`.
int fp8_dst(const pkv_cache_layout* l, const void* key, const void* value, int32_t src_dtype,
            void* key_cache, void* value_cache, uint8_t* key_scales, uint8_t* value_scales,
            Fp8Dst* d) {
  if (pkv::check_layout(l) != PKV_OK || l->dtype != PKV_FP8_E4M3) return PKV_ERR_INVALID;
  if (src_dtype != PKV_F32 && src_dtype != PKV_F16 && src_dtype != PKV_BF16) return PKV_ERR_INVALID;
  if (!key || !value || !key_cache || !value_cache || !key_scales || !value_scales)
    return PKV_ERR_INVALID;
  if (l->head_dim != 64 && l->head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (l->block_stride % l->head_dim != 0 || l->head_stride % l->head_dim != 0) return PKV_ERR_UNSUPPORTED;
  const uintptr_t a16 = reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value);
  const uintptr_t a8 = reinterpret_cast<uintptr_t>(key_cache) | reinterpret_cast<uintptr_t>(value_cache);
  if (a16 % 16 != 0 || a8 % 8 != 0) return PKV_ERR_UNSUPPORTED;
  d->kc = static_cast<uint8_t*>(key_cache);
  d->vc = static_cast<uint8_t*>(value_cache);
  d->ks = key_scales;
  d->vs = value_scales;
  d->block_stride = l->block_stride;
  d->head_stride = l->head_stride;
  d->capacity = static_cast<int64_t>(l->num_blocks) * l->block_size;
  d->block_size = l->block_size;
  d->heads = l->num_kv_heads;
  d->head_dim = l->head_dim;
  return PKV_OK;
}

}  // namespace

extern "C" {

int paged_kv_write_fp8(const void* key, const void* value, int32_t src_dtype,
                       const int64_t* slot_mapping, int32_t num_tokens, void* key_cache,
                       void* value_cache, uint8_t* key_scales, uint8_t* value_scales,
                       const pkv_cache_layout* l, void* stream) {
  if (num_tokens < 0) return PKV_ERR_INVALID;
  if (num_tokens == 0) return pkv::check_layout(l) == PKV_OK ? PKV_OK : PKV_ERR_INVALID;
  if (!slot_mapping) return PKV_ERR_INVALID;
  Fp8Dst d;
  const int st = fp8_dst(l, key, value, src_dtype, key_cache, value_cache, key_scales, value_scales, &d);
  if (st != PKV_OK) return st;
  const int64_t rows = static_cast<int64_t>(num_tokens) * 2 * l->num_kv_heads;
  const int64_t per_block = kThreads / (l->head_dim / 8);
  const int64_t blocks = (rows + per_block - 1) / per_block;
  if (blocks > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(kv_write_fp8_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), key, value, src_dtype, slot_mapping, rows, d);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_decode_write_fp8(const void* key, const void* value, int32_t src_dtype, const int64_t* slots,
                         const int32_t* lens, int32_t num_rows, void* key_cache, void* value_cache,
                         uint8_t* key_scales, uint8_t* value_scales, const pkv_cache_layout* l,
                         int32_t* block_tables, int32_t table_rows, int32_t block_table_stride,
                         int32_t* lens_out, void* stream) {
  if (num_rows < 0 || table_rows < 0 || block_table_stride < 0) return PKV_ERR_INVALID;
  if (num_rows == 0) return pkv::check_layout(l) == PKV_OK ? PKV_OK : PKV_ERR_INVALID;
  if (!slots || !lens || (block_tables && block_table_stride <= 0)) return PKV_ERR_INVALID;
  Fp8Dst d;
  const int st = fp8_dst(l, key, value, src_dtype, key_cache, value_cache, key_scales, value_scales, &d);
  if (st != PKV_OK) return st;
  const int64_t per_block = kThreads / (l->head_dim / 8);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t row0 = 0; row0 < num_rows; row0 += pkv::kStepRows) {
    const int32_t n = num_rows - row0 < pkv::kStepRows ? num_rows - row0 : pkv::kStepRows;
    pkv::StepMeta meta;
    for (int32_t i = 0; i < n; ++i) {
      meta.slots[i] = slots[row0 + i];
      meta.lens[i] = lens[row0 + i];
    }
    const int64_t rows = static_cast<int64_t>(n) * 2 * l->num_kv_heads;
    hipLaunchKernelGGL(decode_write_fp8_kernel, dim3(static_cast<uint32_t>((rows + per_block - 1) / per_block)),
                       dim3(kThreads), 0, s, meta, n, row0, key, value, src_dtype, d, block_tables,
                       table_rows, block_table_stride, lens_out);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

}  // extern "C"
