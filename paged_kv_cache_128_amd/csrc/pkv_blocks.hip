// Whole-block copies for copy-on-write ([impl-detail] "Copy-on-Write机制":
// when a sequence writes into a block other tables still hold, it gets a new
// block that first receives the shared block's K and V).
//
// One workgroup per (pair, K or V, KV head) moves that head's block_size
// token rows, which sit contiguously (head_stride >= block_size * head_dim),
// in 16-byte lanes: a plain HBM-bound copy, coalesced on both sides.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_internal.h"

namespace {

constexpr int kCopyPairs = 256;   // pairs carried by one launch's arguments
constexpr int kCopyThreads = 256;

struct CopyMeta {
  int32_t src[kCopyPairs];
  int32_t dst[kCopyPairs];
};

// The scale bytes of 8-bit blocks, moved beside their codes: the `bs` bytes
// of (block, head) sit at ks/vs + block * block_stride + head * head_stride
// (strides in bytes); staging entry j's go to staging + ((j * 2 + half) *
// heads + head) * bs.  ks == nullptr for 16-bit and fp32 pools.
struct ScaleArgs {
  uint8_t* ks = nullptr;
  uint8_t* vs = nullptr;
  int64_t block_stride = 0, head_stride = 0;
  int32_t bs = 0;
  uint8_t* staging = nullptr;
};

__global__ void __launch_bounds__(kCopyThreads)
block_copy_kernel(CopyMeta meta, int32_t num_blocks, int32_t heads, int64_t block_stride16,
                  int64_t head_stride16, int32_t head_chunks, uint4* __restrict__ key_cache,
                  uint4* __restrict__ value_cache, ScaleArgs sc) {
  const int32_t item = blockIdx.x;
  const int32_t pair = item / (2 * heads);
  const int32_t rem = item - pair * 2 * heads;
  const int32_t half = rem / heads;          // 0: key cache, 1: value cache
  const int32_t h = rem - half * heads;
  const int32_t s = meta.src[pair], d = meta.dst[pair];
  if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) return;
  uint4* base = half == 0 ? key_cache : value_cache;
  const uint4* from = base + s * block_stride16 + h * head_stride16;
  uint4* to = base + d * block_stride16 + h * head_stride16;
  for (int32_t i = threadIdx.x; i < head_chunks; i += kCopyThreads) to[i] = from[i];
  if (sc.ks != nullptr) {
    uint8_t* sb = (half == 0 ? sc.ks : sc.vs) + h * sc.head_stride;
    for (int32_t i = threadIdx.x; i < sc.bs; i += kCopyThreads)
      sb[d * sc.block_stride + i] = sb[s * sc.block_stride + i];
  }
}

// Swap staging ([impl-detail] "异构内存支持"): block ids[j] of the pool <->
// entry j of a contiguous staging array [n, 2, H_kv, bs, D] (K half, then V
// half), one workgroup per (entry, K or V, head) as in the copy.
template <bool TO_STAGING>
__global__ void __launch_bounds__(kCopyThreads)
block_stage_kernel(CopyMeta meta, int32_t num_blocks, int32_t heads, int64_t block_stride16,
                   int64_t head_stride16, int32_t head_chunks, uint4* __restrict__ key_cache,
                   uint4* __restrict__ value_cache, uint4* __restrict__ staging, ScaleArgs sc) {
  const int32_t item = blockIdx.x;
  const int32_t j = item / (2 * heads);
  const int32_t rem = item - j * 2 * heads;
  const int32_t half = rem / heads;
  const int32_t h = rem - half * heads;
  const int32_t id = meta.src[j];
  if (id < 0 || id >= num_blocks) return;
  uint4* pool = (half == 0 ? key_cache : value_cache) + id * block_stride16 + h * head_stride16;
  const int64_t entry = (static_cast<int64_t>(meta.dst[j]) * 2 + half) * heads + h;
  uint4* st = staging + entry * head_chunks;
  for (int32_t i = threadIdx.x; i < head_chunks; i += kCopyThreads) {
    if (TO_STAGING) st[i] = pool[i];
    else pool[i] = st[i];
  }
  if (sc.ks != nullptr) {
    uint8_t* sp = (half == 0 ? sc.ks : sc.vs) + id * sc.block_stride + h * sc.head_stride;
    uint8_t* ss = sc.staging + entry * sc.bs;
    for (int32_t i = threadIdx.x; i < sc.bs; i += kCopyThreads) {
      if (TO_STAGING) ss[i] = sp[i];
      else sp[i] = ss[i];
    }
  }
}

// Shared checks of the copy and staging entry points.
// `with_scales`: the 8-bit entry points, which move scale bytes too; the
// others refuse 8-bit layouts (codes without their scales).
int block_layout_ok(const pkv_cache_layout* l, const void* key_cache, const void* value_cache,
                    bool with_scales) {
  if (pkv::check_layout(l) != PKV_OK) return PKV_ERR_INVALID;
  if ((l->dtype == PKV_FP8_E4M3) != with_scales) return PKV_ERR_UNSUPPORTED;
  if (!key_cache || !value_cache) return PKV_ERR_INVALID;
  const int eb = pkv::elem_bytes(l->dtype);
  const int64_t head_bytes = static_cast<int64_t>(l->block_size) * l->head_dim * eb;
  if (head_bytes % 16 != 0 || (l->head_stride * eb) % 16 != 0 || (l->block_stride * eb) % 16 != 0)
    return PKV_ERR_UNSUPPORTED;
  if (((reinterpret_cast<uintptr_t>(key_cache) | reinterpret_cast<uintptr_t>(value_cache)) % 16) != 0)
    return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

// Scale arguments of an 8-bit layout (strides: the code strides over head_dim).
ScaleArgs scale_args(const pkv_cache_layout* l, uint8_t* ks, uint8_t* vs, uint8_t* staging) {
  ScaleArgs sc;
  sc.ks = ks;
  sc.vs = vs;
  sc.block_stride = l->block_stride / l->head_dim;
  sc.head_stride = l->head_stride / l->head_dim;
  sc.bs = l->block_size;
  sc.staging = staging;
  return sc;
}

template <bool TO_STAGING>
int stage_blocks(const int32_t* ids, int32_t n, void* key_cache, void* value_cache, void* staging,
                 const pkv_cache_layout* l, void* stream, const ScaleArgs& sc) {
  if (n < 0) return PKV_ERR_INVALID;
  const int st = block_layout_ok(l, key_cache, value_cache, sc.ks != nullptr);
  if (st != PKV_OK) return st;
  if (n == 0) return PKV_OK;
  if (!ids || !staging || reinterpret_cast<uintptr_t>(staging) % 16 != 0) return PKV_ERR_INVALID;
  if (sc.ks != nullptr && (!sc.vs || !sc.staging)) return PKV_ERR_INVALID;
  const int eb = pkv::elem_bytes(l->dtype);
  const int64_t head_bytes = static_cast<int64_t>(l->block_size) * l->head_dim * eb;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t p0 = 0; p0 < n; p0 += kCopyPairs) {
    const int32_t m = n - p0 < kCopyPairs ? n - p0 : kCopyPairs;
    CopyMeta meta;
    for (int32_t i = 0; i < m; ++i) {
      meta.src[i] = ids[p0 + i];
      meta.dst[i] = p0 + i;                    // staging entry
    }
    const int64_t grid = static_cast<int64_t>(m) * 2 * l->num_kv_heads;
    hipLaunchKernelGGL(block_stage_kernel<TO_STAGING>, dim3(static_cast<uint32_t>(grid)), dim3(kCopyThreads), 0,
                       s, meta, l->num_blocks, l->num_kv_heads, l->block_stride * eb / 16,
                       l->head_stride * eb / 16, static_cast<int32_t>(head_bytes / 16),
                       static_cast<uint4*>(key_cache), static_cast<uint4*>(value_cache),
                       static_cast<uint4*>(staging), sc);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

int copy_impl(const int32_t* src, const int32_t* dst, int32_t n, void* key_cache, void* value_cache,
              const pkv_cache_layout* l, void* stream, const ScaleArgs& sc) {
  if (n < 0) return PKV_ERR_INVALID;
  const int st = block_layout_ok(l, key_cache, value_cache, sc.ks != nullptr);
  if (st != PKV_OK) return st;
  if (n == 0) return PKV_OK;
  if (!src || !dst) return PKV_ERR_INVALID;
  if (sc.ks != nullptr && !sc.vs) return PKV_ERR_INVALID;
  const int eb = pkv::elem_bytes(l->dtype);
  const int64_t head_bytes = static_cast<int64_t>(l->block_size) * l->head_dim * eb;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t p0 = 0; p0 < n; p0 += kCopyPairs) {
    const int32_t m = n - p0 < kCopyPairs ? n - p0 : kCopyPairs;
    CopyMeta meta;
    for (int32_t i = 0; i < m; ++i) {
      meta.src[i] = src[p0 + i];
      meta.dst[i] = dst[p0 + i];
    }
    const int64_t grid = static_cast<int64_t>(m) * 2 * l->num_kv_heads;
    hipLaunchKernelGGL(block_copy_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kCopyThreads), 0, s,
                       meta, l->num_blocks, l->num_kv_heads, l->block_stride * eb / 16,
                       l->head_stride * eb / 16, static_cast<int32_t>(head_bytes / 16),
                       static_cast<uint4*>(key_cache), static_cast<uint4*>(value_cache), sc);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_gather_blocks(const int32_t* ids, int32_t n, const void* key_cache,
                                 const void* value_cache, void* staging, const pkv_cache_layout* l,
                                 void* stream) {
  return stage_blocks<true>(ids, n, const_cast<void*>(key_cache), const_cast<void*>(value_cache), staging,
                            l, stream, ScaleArgs{});
}

extern "C" int pkv_scatter_blocks(const void* staging, const int32_t* ids, int32_t n, void* key_cache,
                                  void* value_cache, const pkv_cache_layout* l, void* stream) {
  return stage_blocks<false>(ids, n, key_cache, value_cache, const_cast<void*>(staging), l, stream,
                             ScaleArgs{});
}

extern "C" int pkv_copy_blocks(const int32_t* src, const int32_t* dst, int32_t n, void* key_cache,
                               void* value_cache, const pkv_cache_layout* l, void* stream) {
  return copy_impl(src, dst, n, key_cache, value_cache, l, stream, ScaleArgs{});
}

extern "C" int pkv_copy_blocks_fp8(const int32_t* src, const int32_t* dst, int32_t n, void* key_cache,
                                   void* value_cache, uint8_t* key_scales, uint8_t* value_scales,
                                   const pkv_cache_layout* l, void* stream) {
  if (pkv::check_layout(l) != PKV_OK || !key_scales || !value_scales) return PKV_ERR_INVALID;
  return copy_impl(src, dst, n, key_cache, value_cache, l, stream,
                   scale_args(l, key_scales, value_scales, nullptr));
}

extern "C" int pkv_gather_blocks_fp8(const int32_t* ids, int32_t n, const void* key_cache,
                                     const void* value_cache, const uint8_t* key_scales,
                                     const uint8_t* value_scales, void* staging, uint8_t* staging_scales,
                                     const pkv_cache_layout* l, void* stream) {
  if (pkv::check_layout(l) != PKV_OK || !key_scales || !value_scales) return PKV_ERR_INVALID;
  return stage_blocks<true>(ids, n, const_cast<void*>(key_cache), const_cast<void*>(value_cache), staging,
                            l, stream,
                            scale_args(l, const_cast<uint8_t*>(key_scales), const_cast<uint8_t*>(value_scales),
                                       staging_scales));
}

extern "C" int pkv_scatter_blocks_fp8(const void* staging, const uint8_t* staging_scales, const int32_t* ids,
                                      int32_t n, void* key_cache, void* value_cache, uint8_t* key_scales,
                                      uint8_t* value_scales, const pkv_cache_layout* l, void* stream) {
  if (pkv::check_layout(l) != PKV_OK || !key_scales || !value_scales) return PKV_ERR_INVALID;
  return stage_blocks<false>(ids, n, key_cache, value_cache, const_cast<void*>(staging), l, stream,
                             scale_args(l, key_scales, value_scales, const_cast<uint8_t*>(staging_scales)));
}
