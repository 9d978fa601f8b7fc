/*
 * pkv.h -- C ABI of libpkv: paged KV cache write and paged decode attention
 * for MI355X (gfx950), plus the host-side block manager that feeds them.
 *
 * Page shorthands used in the citations below:
 *   [MiniPaged-Qwen] "MiniPaged-Qwen：Paged KV Cache 与 KV Block Manager"
 *                    (blog.zsmgc.love), numbered sections.
 *   [mini-vLLM BM]   "从零实现一个 mini vLLM — Block Manager" (yjxyzxyz.cn),
 *                    section headings.
 *   [leetcode-22]    "22. vLLM PagedAttention | vLLM 分页注意力"
 *                    (datawhalechina llm-algo-leetcode), Step headings.
 *
 * Conventions for every entry point:
 *   - Return value is a status code (PKV_OK or a negative PKV_ERR_*).  Any
 *     error leaves all state unchanged ([leetcode-22] Step 2 table: a failed
 *     growth rolls back; Step 4 TODO 2: OOM leaves no partial allocation).
 *   - "host" pointers are ordinary CPU memory; "device" pointers are HIP
 *     device memory (or managed memory) visible to the GPU that owns the
 *     stream.  The caller owns every buffer and every stream; the library
 *     allocates no device memory and keeps no pointer after a call returns.
 *   - GPU entry points are asynchronous on `stream` (a hipStream_t passed as
 *     void*; NULL is the null stream).  Argument errors are reported
 *     synchronously; a failed launch returns PKV_ERR_HIP.
 *   - Manager objects are host-only and not thread-safe: one owner thread.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
#define PKV_OK                     0
#define PKV_ERR_INVALID           (-1) /* bad argument (ValueError in the pages' Python) */
#define PKV_ERR_OOM               (-2) /* not enough free blocks ("OOM", [leetcode-22] Step 4) */
#define PKV_ERR_NOT_LIVE          (-3) /* unknown or already freed sequence (double free) */
#define PKV_ERR_ALREADY_PREFILLED (-4) /* prefill of a live sequence */
#define PKV_ERR_UNSUPPORTED       (-5) /* shape / dtype combination the kernels do not cover */
#define PKV_ERR_HIP               (-6) /* a HIP runtime call or kernel launch failed */
#define PKV_ERR_WORKSPACE         (-7) /* workspace missing or too small */
#define PKV_ERR_INVARIANT         (-8) /* manager invariant violated */

/* Static, NUL-terminated description of a status code. */
const char* pkv_status_string(int status);

/* ------------------------------------------------------------- cache layout */
/* PKV_FP8_E4M3: 8-bit KV codes (OCP E4M3, largest finite 448) with one
 * power-of-two scale byte per token row; see the FP8 section below. */
typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_FP8_E4M3 = 3 } pkv_dtype;

/*
 * Where token `off` of KV head `h` of physical block `pb` lives:
 *     base + pb * block_stride + h * head_stride + off * head_dim   (elements)
 * with the head_dim elements of that token contiguous.  This is the
 * [N, H_kv, block_size, D] indexing of [MiniPaged-Qwen] §11
 * (KCache[physical_block, kvh, block_offset, :]) with free block and head
 * strides, so that both layouts below are expressible:
 *   - interleaved pool [N, 2, H_kv, bs, D]: key base = pool, value base =
 *     pool + H_kv*bs*D elements, block_stride = 2*H_kv*bs*D,
 *     head_stride = bs*D (one block holds its K half then its V half);
 *   - split pools [N, H_kv, bs, D] each ([MiniPaged-Qwen] §11, §16.3):
 *     block_stride = H_kv*bs*D, head_stride = bs*D.
 * Requirements: head_stride >= block_size*head_dim, block_stride >=
 * num_kv_heads*head_stride, all strides multiples of 8 elements.
 */
typedef struct {
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t head_dim;
  int32_t dtype;          /* pkv_dtype of K, V, q and the new key/value rows */
  int32_t reserved;       /* must be 0 */
  int64_t block_stride;   /* elements */
  int64_t head_stride;    /* elements */
} pkv_cache_layout;

/* Bytes one pool tensor spans: (num_blocks-1)*block_stride +
 * (num_kv_heads-1)*head_stride + block_size*head_dim elements.  Returns 0 on
 * an invalid layout. */
size_t pkv_pool_span_bytes(const pkv_cache_layout* layout);

/* ---------------------------------------------------------- block manager */
/*
 * Host-side block manager ([MiniPaged-Qwen] §8, §9; [mini-vLLM BM]).
 * State: `num_blocks` physical ids, an ordered free list and, per live
 * sequence, its length (tokens written == next write position) and its block
 * table (logical block i -> physical id, covering tokens [i*bs, (i+1)*bs)).
 *
 * Allocation takes ids from the FRONT of the free list; release appends a
 * table to the BACK in logical order, then sorts the whole list when
 * PKV_SORT_ON_RELEASE is set (the order [leetcode-22]'s reference answer
 * keeps).  `initial_free_order` (host, [num_blocks], a permutation of
 * 0..N-1) sets the starting order; NULL means 0, 1, ..., N-1
 * ([MiniPaged-Qwen] §8.2).  The library copies it.
 *
 * Prefix sharing and copy-on-write ([impl-detail] "Copy-on-Write共享"):
 * every block has a reference count, the number of tables holding it
 * (pkv_share_prefix lets several tables hold one block).  Release drops one
 * reference per table entry and appends a block to the free list when its
 * count reaches 0.  An append whose token lands in a block held by more than
 * one table first takes a free block (front of the list), drops one
 * reference from the shared block, puts the new block in the table and
 * queues the pair (shared block, new block); the caller drains the queue
 * with pkv_take_block_copies and runs pkv_copy_blocks on the device before
 * it writes the step's rows.  Without sharing nothing is ever queued.
 */
typedef struct pkv_manager pkv_manager;
#define PKV_SORT_ON_RELEASE 1u

/* Returns NULL on invalid arguments (num_blocks <= 0, block_size <= 0, an
 * order that is not a permutation, unknown flags) or allocation failure. */
pkv_manager* pkv_manager_create(int32_t num_blocks, int32_t block_size,
                                const int32_t* initial_free_order, uint32_t flags);
void pkv_manager_destroy(pkv_manager* mgr);

/* ceil(num_tokens / block_size) <= number of free blocks
 * ([mini-vLLM BM] "prefill 时如何分配 block", can_allocate).
 * Returns 1 (yes), 0 (no) or PKV_ERR_INVALID (num_tokens < 0, NULL mgr). */
int pkv_can_allocate(const pkv_manager* mgr, int32_t num_tokens);
int32_t pkv_num_free_blocks(const pkv_manager* mgr);
int32_t pkv_num_live_sequences(const pkv_manager* mgr);

/*
 * Create live sequence `seq_id` (>= 0) holding `num_tokens` (>= 0) prompt
 * tokens: ceil(num_tokens/bs) blocks from the front of the free list, all or
 * nothing ([mini-vLLM BM] "prefill 时如何分配 block"; [leetcode-22] Step 4
 * TODO 2).  When `slots_out` (host, [num_tokens]) is non-NULL it receives
 * the flat slot of every prompt token, token t at
 * table[t / bs] * bs + t % bs ([mini-vLLM BM] "Block Manager 和 ModelRunner
 * 如何协作").  Errors: INVALID, ALREADY_PREFILLED (seq live), OOM.
 */
int pkv_allocate_for_prefill(pkv_manager* mgr, int64_t seq_id, int32_t num_tokens,
                             int64_t* slots_out);

/*
 * Slot for the next token of `seq_id` ([MiniPaged-Qwen] §9): position
 * L = len, logical_block = L / bs, offset = L % bs; when logical_block ==
 * len(table) one block is taken from the front of the free list; slot =
 * table[logical_block] * bs + offset; then len = L + 1.  `*slot_out` (host)
 * receives the slot.  Errors: NOT_LIVE, OOM (no change), INVALID (NULL).
 */
int pkv_append_slot_for_decode(pkv_manager* mgr, int64_t seq_id, int64_t* slot_out);

/*
 * Batched append for `n` distinct live sequences, processed in array order,
 * all or nothing: the blocks the call takes (one per sequence opening a
 * block, one per copy-on-write, counted in array order) are checked against
 * the free list before anything changes ([mini-vLLM BM] "Block Manager 和
 * Scheduler 如何协作", can_append_slots).  Outputs (host, each [n], any may
 * be NULL): slots_out[i] = slot of seq_ids[i]'s new token; lens_out[i] = its
 * length after the append; new_block_out[i] = physical id this call put in
 * its table (an opened block, or a copy-on-write block at the same logical
 * index), or -1 when none.
 * Errors: INVALID (n < 0, duplicate ids, NULL ids with n > 0), NOT_LIVE, OOM.
 */
int pkv_append_slots_for_decode(pkv_manager* mgr, const int64_t* seq_ids, int32_t n,
                                int64_t* slots_out, int32_t* lens_out,
                                int32_t* new_block_out);

/*
 * Append `num_tokens` (>= 0) tokens to live `seq_id` (a prefill chunk):
 * slots_out (host, [num_tokens], nullable) receives the slots of positions
 * len .. len + num_tokens - 1, each as pkv_append_slot_for_decode computes
 * it (opening blocks, and copying a shared tail block on write), all or
 * nothing: the blocks the call takes are checked against the free list
 * first ([MiniPaged-Qwen] §9; [mini-vLLM BM] "prefill 时如何分配 block").
 * Errors: INVALID, NOT_LIVE, OOM.
 */
int pkv_append_tokens(pkv_manager* mgr, int64_t seq_id, int32_t num_tokens, int64_t* slots_out);

/*
 * A batch of prefill chunks admitted all or nothing ([mini-vLLM BM] "Block
 * Manager 和 Scheduler 如何协作": the scheduler admits only what the free
 * blocks cover).  In array order, sequence seq_ids[i] receives
 * chunk_lens[i] tokens: a sequence that is not live is created as
 * pkv_allocate_for_prefill creates it; a live one is extended as
 * pkv_append_tokens extends it, when `extend_live` is nonzero.  Everything
 * is checked before anything changes: ids >= 0 and distinct, lengths >= 0,
 * no swapped id and no live id unless extend_live (ALREADY_PREFILLED), and
 * the blocks of the whole batch (new tables, opened blocks, a copy of each
 * shared tail block a chunk writes into, counted in array order) against
 * the free list (OOM).  slots_out (host, [sum of chunk_lens], nullable)
 * receives the chunks' slots concatenated in array order; lens_out (host,
 * [n], nullable) the lengths afterwards.  Errors: INVALID,
 * ALREADY_PREFILLED, OOM.
 */
int pkv_admit_batch(pkv_manager* mgr, const int64_t* seq_ids, const int32_t* chunk_lens, int32_t n,
                    int32_t extend_live, int64_t* slots_out, int32_t* lens_out);

/* Release `seq_id`: each block of its table loses one reference, and those
 * whose count reaches 0 are appended to the free list in table order
 * ([MiniPaged-Qwen] §5.3; [mini-vLLM BM] "释放 block").  Errors: NOT_LIVE. */
int pkv_free_sequence(pkv_manager* mgr, int64_t seq_id);

/*
 * Create live sequence `seq_id` (>= 0) holding the first `num_tokens`
 * (0 <= num_tokens <= donor length) tokens of live sequence `donor_id`
 * without copying: its table is the donor's first ceil(num_tokens / bs)
 * blocks, the partial last block included, each gaining one reference
 * ([impl-detail] "前缀共享", share_prefix_blocks).  Its length is
 * num_tokens; its next append copies the last block first when that block is
 * still shared.  With num_tokens equal to the donor's length this forks the
 * donor.  Errors: INVALID, NOT_LIVE (donor), ALREADY_PREFILLED (seq_id
 * live).
 */
int pkv_share_prefix(pkv_manager* mgr, int64_t donor_id, int64_t seq_id, int32_t num_tokens);

/*
 * Swap to host ([impl-detail] "异构内存支持" evict_to_cpu /
 * prefetch_to_gpu).  pkv_swap_out releases every block of live `seq_id` to
 * the free list (table order, then the sort of PKV_SORT_ON_RELEASE) and
 * keeps its length; ids_out (host, [cap]) receives the released blocks in
 * table order and *count_out their number, so the caller can copy them out
 * (pkv_gather_blocks) before anything reuses them.  The sequence is then
 * swapped: not live (appends give NOT_LIVE; prefill and share onto its id
 * give ALREADY_PREFILLED), and pkv_free_sequence forgets it.  A sequence
 * holding a block another table shares cannot be swapped out (INVALID).
 * pkv_swap_in gives a swapped sequence ceil(len / bs) blocks from the front
 * of the free list, all or nothing (OOM leaves it swapped), returns its new
 * table in ids_out, and makes it live with the same length; the caller then
 * copies the contents back (pkv_scatter_blocks).  Errors: INVALID (cap too
 * small, shared blocks), NOT_LIVE, ALREADY_PREFILLED, OOM.
 */
int pkv_swap_out(pkv_manager* mgr, int64_t seq_id, int32_t* ids_out, int32_t cap, int32_t* count_out);
int pkv_swap_in(pkv_manager* mgr, int64_t seq_id, int32_t* ids_out, int32_t cap, int32_t* count_out);
/* 1 when `seq_id` is swapped out, 0 otherwise, or INVALID. */
int pkv_is_swapped(const pkv_manager* mgr, int64_t seq_id);

/* Reference count of physical block `block` (0 when free), or INVALID. */
int32_t pkv_block_ref_count(const pkv_manager* mgr, int32_t block);

/* Drain the copy-on-write queue, oldest first: src[i] (shared block) and
 * dst[i] (the new block that replaced it in one table) for i < *count_out
 * (host arrays of `cap` entries).  INVALID when more than `cap` are queued
 * (nothing is drained then). */
int pkv_take_block_copies(pkv_manager* mgr, int32_t* src, int32_t* dst, int32_t cap,
                          int32_t* count_out);

/* Length of a live sequence, or PKV_ERR_NOT_LIVE. */
int32_t pkv_context_len(const pkv_manager* mgr, int64_t seq_id);

/* Copy the block table of `seq_id` into `out` (host, [cap]); `*len_out`
 * receives its length.  INVALID when cap is too small. */
int pkv_get_block_table(const pkv_manager* mgr, int64_t seq_id, int32_t* out,
                        int32_t cap, int32_t* len_out);

/* Batch block-table tensor ([MiniPaged-Qwen] §16.5): row i of `out` (host,
 * [n, width] row-major) holds seq_ids[i]'s table, padded with `pad`.
 * INVALID when a table is wider than `width`; NOT_LIVE for unknown ids. */
int pkv_get_block_tables(const pkv_manager* mgr, const int64_t* seq_ids, int32_t n,
                         int32_t width, int32_t pad, int32_t* out);

/* Lengths of seq_ids into `out` (host, [n]) ([MiniPaged-Qwen] §16.6). */
int pkv_get_context_lens(const pkv_manager* mgr, const int64_t* seq_ids, int32_t n,
                         int32_t* out);

/* Copy the free list, front first, into `out` (host, [cap]); `*count_out`
 * receives its length.  INVALID when cap is too small. */
int pkv_get_free_list(const pkv_manager* mgr, int32_t* out, int32_t cap, int32_t* count_out);

/* Check the invariants of [MiniPaged-Qwen] §15 and [mini-vLLM BM]
 * "正确性不变量": I1 no physical id twice in one table and each block's
 * reference count equals the number of tables holding it (without sharing:
 * no id in two tables), I2 tables and free list disjoint (free blocks count
 * 0), I3 |distinct allocated| + |free| == N, I4 ids in [0, N),
 * I5 len(table) == ceil(len / bs), I6 no duplicate in the free list.
 * Returns PKV_OK or PKV_ERR_INVARIANT. */
int pkv_check_invariants(const pkv_manager* mgr);

/* Debug check of a write's slot mapping, host only.  The pages' slot of a
 * token is block * block_size + offset ([MiniPaged-Qwen] §11) and a
 * manager hands each slot to one token ([mini-vLLM BM] "正确性不变量"
 * recommends checking such ownership in debug runs); two tokens of one
 * write with the same slot would race in the write kernels, whose result
 * is then undefined.  `slot_mapping` is a HOST array of n int64 slots;
 * entries outside [0, num_slots) are ignored, as the writes skip them.
 * Returns PKV_OK when no in-range slot appears twice; PKV_ERR_INVALID when
 * one does, with *first_repeat (optional) set to the smallest index whose
 * slot an earlier entry already holds, and PKV_ERR_INVALID with
 * *first_repeat = -1 for n < 0, num_slots < 0 or a NULL array with n > 0.
 * O(n log n); nothing is kept. */
int pkv_check_slot_mapping(const int64_t* slot_mapping, int64_t n, int64_t num_slots, int64_t* first_repeat);

/* ------------------------------------------------------------- cache write */
/*
 * Scatter the new tokens' K/V rows into the paged pool ([MiniPaged-Qwen]
 * §12; address split of §11):  for every token t in [0, num_tokens)
 *     pb = slot_mapping[t] / bs,  off = slot_mapping[t] % bs,
 *     K[pb, h, off, :] = key[t, h, :],  V[pb, h, off, :] = value[t, h, :]
 * for all heads h.  A bit-exact copy: key/value have the cache dtype.
 *   key, value    device, [num_tokens, H_kv, D] contiguous, layout->dtype
 *   slot_mapping  device, int64 [num_tokens]; entries outside
 *                 [0, num_blocks*bs) are skipped (nothing written, no fault)
 *   key_cache, value_cache  device pool bases as described by `layout`
 * Slots must be distinct (two tokens with one slot race).  num_tokens == 0
 * is a no-op.  Errors: INVALID, UNSUPPORTED (head_dim*elem_bytes not a
 * multiple of 16), HIP.
 */
int paged_kv_write(const void* key, const void* value, const int64_t* slot_mapping,
                   int32_t num_tokens, void* key_cache, void* value_cache,
                   const pkv_cache_layout* layout, void* stream);

/*
 * The write of one decode step, with the step's metadata taken from HOST
 * memory and carried into the launch as kernel arguments (no separate
 * host-to-device copy; the caller may reuse `slots` and `lens` as soon as
 * the call returns).  For every row i in [0, num_rows):
 *   - key/value row i (device, [num_rows, H_kv, D] contiguous) is written at
 *     slots[i] exactly as paged_kv_write does ([MiniPaged-Qwen] §12);
 *   - when block_tables (device, int32 [table_rows, block_table_stride]) is
 *     not NULL, the table entry [i, (lens[i] - 1) / bs] is set to
 *     slots[i] / bs: the block holding the new token, which the append may
 *     have opened ([MiniPaged-Qwen] §9.2) or copied on write;
 *   - when lens_out (device, int32 [num_rows]) is not NULL, lens_out[i] =
 *     lens[i].
 *   slots (host, int64 [num_rows]) and lens (host, int32 [num_rows]) are the
 *   outputs of pkv_append_slots_for_decode for the rows in order.
 * Slots outside [0, num_blocks*bs) write nothing.  Errors: INVALID,
 * UNSUPPORTED, HIP.
 */
int pkv_decode_write(const void* key, const void* value, const int64_t* slots,
                     const int32_t* lens, int32_t num_rows, void* key_cache, void* value_cache,
                     const pkv_cache_layout* layout, int32_t* block_tables, int32_t table_rows,
                     int32_t block_table_stride, int32_t* lens_out, void* stream);

/*
 * Whole-block copies for copy-on-write ([impl-detail] "Copy-on-Write机制":
 * the new block receives the shared block's K and V): for i < n, every
 * token row of every KV head of block src[i] is copied to block dst[i], in
 * key_cache and in value_cache.  src, dst: host int32 [n], carried into the
 * launches as kernel arguments (256 pairs per launch).  Pairs with an id
 * outside [0, num_blocks) are skipped.  No dst may equal any pair's src or
 * another pair's dst (the pairs run concurrently); pkv_take_block_copies
 * output meets this.  n == 0 is a no-op.  Errors: INVALID, UNSUPPORTED
 * (an 8-bit layout: pkv_copy_blocks_fp8; a head's block_size*head_dim*elem_bytes
 * not a multiple of 16), HIP.
 */
int pkv_copy_blocks(const int32_t* src, const int32_t* dst, int32_t n, void* key_cache,
                    void* value_cache, const pkv_cache_layout* layout, void* stream);

/*
 * Swap staging ([impl-detail] "异构内存支持"): pkv_gather_blocks copies
 * blocks ids[0 .. n-1] (host int32) of both pools into `staging` (device,
 * 16-byte aligned, n * 2 * H_kv * bs * D elements: entry j is block ids[j]'s
 * K half then V half, [n, 2, H_kv, bs, D]); pkv_scatter_blocks copies entry
 * j back into block ids[j].  The caller moves the staging array to and from
 * host memory (a plain device-host copy).  Ids outside [0, num_blocks) are
 * skipped.  16-bit and fp32 layouts (8-bit ones: the _fp8 forms below).
 * Errors: INVALID, UNSUPPORTED, HIP.
 */
int pkv_gather_blocks(const int32_t* ids, int32_t n, const void* key_cache, const void* value_cache,
                      void* staging, const pkv_cache_layout* layout, void* stream);
int pkv_scatter_blocks(const void* staging, const int32_t* ids, int32_t n, void* key_cache,
                       void* value_cache, const pkv_cache_layout* layout, void* stream);

/*
 * The copy and the swap staging for 8-bit blocks (layout->dtype ==
 * PKV_FP8_E4M3): a block's rows are its codes together with their scale
 * bytes, so each of these moves both ([impl-detail] "Copy-on-Write机制",
 * "异构内存支持"; the scale addresses are those of the FP8 section below).
 * key_scales / value_scales (device) are the scale views matching
 * key_cache / value_cache.  staging holds the codes as for
 * pkv_gather_blocks (one byte per element); staging_scales (device,
 * n * 2 * H_kv * bs bytes, no alignment needed) holds entry j's scale bytes,
 * [n, 2, H_kv, bs] (K half, then V half).  Otherwise as pkv_copy_blocks,
 * pkv_gather_blocks and pkv_scatter_blocks.  Errors: INVALID (a NULL scale
 * pointer), UNSUPPORTED (a 16-bit or fp32 layout), HIP.
 */
int pkv_copy_blocks_fp8(const int32_t* src, const int32_t* dst, int32_t n, void* key_cache,
                        void* value_cache, uint8_t* key_scales, uint8_t* value_scales,
                        const pkv_cache_layout* layout, void* stream);
int pkv_gather_blocks_fp8(const int32_t* ids, int32_t n, const void* key_cache, const void* value_cache,
                          const uint8_t* key_scales, const uint8_t* value_scales, void* staging,
                          uint8_t* staging_scales, const pkv_cache_layout* layout, void* stream);
int pkv_scatter_blocks_fp8(const void* staging, const uint8_t* staging_scales, const int32_t* ids,
                           int32_t n, void* key_cache, void* value_cache, uint8_t* key_scales,
                           uint8_t* value_scales, const pkv_cache_layout* layout, void* stream);

/* -------------------------------------------------------- decode attention */
/*
 * Workspace bytes paged_decode_attention needs for the path it takes with
 * these arguments (see paged_decode_attention_path).  Partition path:
 * num_seqs * num_q_heads * P * (head_dim + 2) * 4 bytes of split-K partials,
 * P = ceil(max_context_len / partition_tokens) (0 when P <= 1; a
 * partition_tokens of 0 that cannot take the stream path means 512).  Stream
 * path (partition_tokens == 0): W * 4 * num_q_heads * (head_dim + 2) * 4
 * bytes of partials, with W = CUs * max(1, 4 / num_kv_heads) tile ranges
 * (integer division; 256 CUs on MI355X), then (num_seqs + 1) * 4 bytes of
 * per-sequence tile offsets the attention launch leaves for the merge.  The
 * contents need no initialisation.  Returns 0 for invalid arguments as well.
 */
size_t paged_decode_attention_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_context_len,
                                             int32_t partition_tokens);

/*
 * Decode attention through block tables ([MiniPaged-Qwen] §13, §14, §17.3):
 * for sequence b with L = context_lens[b] and query head qh,
 *     kvh = qh / (H_q / H_kv),
 *     K_pos = K[block_tables[b, pos / bs], kvh, pos % bs, :]  (pos < L),
 *     out[b, qh, :] = softmax_pos(scale * q[b, qh, :] . K_pos) V_pos.
 * No causal mask (one query per sequence at its last position).
 *   out          device, [num_seqs, num_q_heads, D] contiguous, `out_dtype`
 *                (PKV_F32, or the cache dtype)
 *   q            device, [num_seqs, num_q_heads, D] contiguous, layout->dtype
 *   key_cache, value_cache  device pool bases (see pkv_cache_layout)
 *   block_tables device, int32 [num_seqs, block_table_stride] row-major;
 *                entries j >= ceil(L/bs) are never read, so padding may hold
 *                any value; ids outside [0, num_blocks) are skipped
 *   context_lens device, int32 [num_seqs]; L is clamped to
 *                [0, max_context_len]; L == 0 gives zeros
 *   max_context_len  host upper bound of context_lens, and
 *                max_context_len <= block_table_stride * block_size
 *   partition_tokens split-K partition length in tokens (multiple of 16;
 *                0 = library default); sequences longer than one partition
 *                are reduced by a second kernel (max / sum rescaling)
 *   workspace    device, >= paged_decode_attention_workspace_size(...)
 *                bytes (may be NULL when that size is 0)
 * Supported: block_size a multiple of 16, head_dim in {64, 128},
 * H_q % H_kv == 0 with H_q / H_kv <= 8.  Softmax state and all sums are
 * fp32.  Errors: INVALID, UNSUPPORTED, WORKSPACE, HIP.
 */
int paged_decode_attention(void* out, int32_t out_dtype, const void* q,
                           const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, int32_t block_table_stride,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_q_heads, int32_t max_context_len, float scale,
                           const pkv_cache_layout* layout, int32_t partition_tokens,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Which attention kernel paged_decode_attention runs for these arguments:
 * PKV_PATH_STREAM (1): the launch's 16-token tiles cut into equal ranges,
 * one workgroup per CU, each (range, KV head) shared by two waves that
 * split its tiles at a fixed point (16-bit KV, head_dim 128, H_kv <= 8,
 * H_q / H_kv <= 8, partition_tokens == 0); PKV_PATH_PARTITION (2):
 * one workgroup per (sequence, KV head, context partition of
 * partition_tokens tokens, default 512).  Negative status on invalid
 * arguments.  Host-only; the workspace size matches the path.
 */
#define PKV_PATH_STREAM 1
#define PKV_PATH_PARTITION 2
int paged_decode_attention_path(int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                const pkv_cache_layout* layout, int32_t partition_tokens);

/*
 * The two launches of paged_decode_attention, callable separately with the
 * same arguments (for instance to time or overlap them): _partial runs the
 * attention kernel (stream or partition path), which finishes every
 * sequence one segment covers and leaves (max, sum, accumulator) partials in
 * `workspace` for the others; _merge then reduces those partials into `out`.
 * The pair, in this order on one stream, equals one paged_decode_attention
 * call.
 */
int paged_decode_attention_partial(void* out, int32_t out_dtype, const void* q,
                                   const void* key_cache, const void* value_cache,
                                   const int32_t* block_tables, int32_t block_table_stride,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_context_len, float scale,
                                   const pkv_cache_layout* layout, int32_t partition_tokens,
                                   void* workspace, size_t workspace_bytes, void* stream);
int paged_decode_attention_merge(void* out, int32_t out_dtype, const void* q,
                                 const void* key_cache, const void* value_cache,
                                 const int32_t* block_tables, int32_t block_table_stride,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_context_len, float scale,
                                 const pkv_cache_layout* layout, int32_t partition_tokens,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step after the host-side append ([MiniPaged-Qwen] §1.1: write
 * the step's K/V, then attend over the whole context including it):
 * exactly pkv_decode_write(key, value, slots, lens, num_seqs, key_cache,
 * value_cache, layout, block_tables, num_seqs, block_table_stride, lens_out)
 * followed by paged_decode_attention(out, out_dtype, q, key_cache,
 * value_cache, block_tables, block_table_stride, lens_out, num_seqs,
 * num_q_heads, max_context_len, scale, layout, 0, workspace, ...), with
 * the same results bit for bit.  When the stream path applies, at most 256
 * rows are given, every slots[i] lies in [0, num_blocks * bs) and every
 * lens[i] in [1, max_context_len], the write runs inside the attention
 * launch: the one wave per KV head that reads a sequence's last tile takes
 * the new row from `key`/`value` and stores it into the pool, and the new
 * lengths and table entries are published by the same launch.  Otherwise
 * the two calls run one after the other.
 *   key, value   device, [num_seqs, H_kv, D] contiguous, 16-byte aligned
 *   slots, lens  host, the outputs of pkv_append_slots_for_decode in row
 *                order (lens = context lengths after the append)
 *   block_tables device, int32 [num_seqs, block_table_stride]; entry
 *                [i, (lens[i] - 1) / bs] is set to slots[i] / bs (blocks
 *                the append opened or copied on write; the copies
 *                themselves, pkv_copy_blocks, must run before this call)
 *   lens_out     device, int32 [num_seqs], receives lens
 *   workspace    as for paged_decode_attention with partition_tokens 0
 * Errors: INVALID, UNSUPPORTED, WORKSPACE, HIP.
 */
int pkv_decode_step(void* out, int32_t out_dtype, const void* q, const void* key,
                    const void* value, const int64_t* slots, const int32_t* lens,
                    int32_t num_seqs, void* key_cache, void* value_cache,
                    const pkv_cache_layout* layout, int32_t* block_tables,
                    int32_t block_table_stride, int32_t* lens_out, int32_t num_q_heads,
                    int32_t max_context_len, float scale, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * The two launches of pkv_decode_step, callable separately with the same
 * arguments: _partial runs the write and the attention kernel, leaving
 * partials of split sequences in `workspace`; _merge reduces them into
 * `out` (reading the lengths from lens_out).  paged_decode_attention_merge
 * with context_lens = lens_out and the same other arguments may stand in
 * for _merge.  The pair,
 * in this order on one stream, equals one pkv_decode_step call.
 */
int pkv_decode_step_partial(void* out, int32_t out_dtype, const void* q, const void* key,
                            const void* value, const int64_t* slots, const int32_t* lens,
                            int32_t num_seqs, void* key_cache, void* value_cache,
                            const pkv_cache_layout* layout, int32_t* block_tables,
                            int32_t block_table_stride, int32_t* lens_out,
                            int32_t num_q_heads, int32_t max_context_len, float scale,
                            void* workspace, size_t workspace_bytes, void* stream);
int pkv_decode_step_merge(void* out, int32_t out_dtype, const void* q, const void* key,
                          const void* value, const int64_t* slots, const int32_t* lens,
                          int32_t num_seqs, void* key_cache, void* value_cache,
                          const pkv_cache_layout* layout, int32_t* block_tables,
                          int32_t block_table_stride, int32_t* lens_out, int32_t num_q_heads,
                          int32_t max_context_len, float scale, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * pkv_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same step, with the same results bit for bit, and the same arguments
 * except the workspace.  The split-K partials live in a device array the
 * library owns, PKV_NOALLOC_SCRATCH_BYTES per GPU, held from the first call
 * on that GPU until the process ends; the call allocates nothing.  Calls
 * whose workspace (paged_decode_attention_workspace_size with
 * partition_tokens 0) exceeds that size return PKV_ERR_WORKSPACE without
 * doing anything; every shape the stream path takes on a 256-CU device fits.
 * All calls on one GPU share its array, whatever their stream: calls that
 * may overlap on one GPU race and give wrong results; the caller serialises
 * them (one stream, or events).  The array needs no initialisation; each
 * call overwrites what it reads.  The current device must be the one that
 * runs `stream`.  Errors: as pkv_decode_step, WORKSPACE as above, HIP when
 * the array's device address cannot be found.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (36u << 20)
int pkv_decode_step_noalloc(void* out, int32_t out_dtype, const void* q, const void* key,
                            const void* value, const int64_t* slots, const int32_t* lens,
                            int32_t num_seqs, void* key_cache, void* value_cache,
                            const pkv_cache_layout* layout, int32_t* block_tables,
                            int32_t block_table_stride, int32_t* lens_out, int32_t num_q_heads,
                            int32_t max_context_len, float scale, void* stream);

/* --------------------------------------------------------- prefill attention */
/*
 * Chunked-prefill attention through block tables: sequence b holds
 * L = context_lens[b] cached tokens (the chunk's own K/V already written,
 * e.g. by paged_kv_write; [MiniPaged-Qwen] §1.1, §12); its query rows are
 * q[q_start[b] .. q_start[b + 1] - 1], the last n_b positions, row i at
 * p = L - n_b + i attending to positions 0 .. p only (the causal mask of
 * [impl-detail] "分块注意力"), with the GQA map kvh = qh / (H_q / H_kv)
 * ([MiniPaged-Qwen] §14) and the table addressing of §13.  A full prefill
 * is n_b = L; rows with p < 0 get zeros.
 *   out          device, [T, num_q_heads, D], T = q_start[num_seqs];
 *                PKV_F32 or the cache dtype
 *   q            device, [T, num_q_heads, D] contiguous, cache dtype
 *   q_start      device int32 [num_seqs + 1], non-decreasing from 0
 *   context_lens device int32 [num_seqs], clamped to [0, max_context_len]
 *   max_q_len    host, >= every n_b (sizes the grid)
 * With 16-bit KV, head_dim 128 and block_size a multiple of 16 the
 * products run on the matrix cores in the cache's 16-bit type with fp32
 * accumulation, P entering P.V as a 16-bit value plus a 16-bit remainder;
 * any other cache type (fp32) or shape (head_dim 64, other block sizes)
 * takes a generic kernel, fp32 throughout.  Supported: head_dim 64 or 128,
 * fp32, fp16 or bf16 KV (8-bit KV: paged_prefill_attention_fp8).  Errors:
 * INVALID, UNSUPPORTED, HIP.
 */
int paged_prefill_attention(void* out, int32_t out_dtype, const void* q, const int32_t* q_start,
                            const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len,
                            const void* key_cache, const void* value_cache,
                            const pkv_cache_layout* layout, const int32_t* block_tables,
                            int32_t block_table_stride, int32_t num_q_heads,
                            int32_t max_context_len, float scale, void* stream);

/*
 * Chunked-prefill attention over 8-bit blocks (layout->dtype ==
 * PKV_FP8_E4M3; scale bytes as in the FP8 section below).  Computes what
 * paged_prefill_attention computes, with every cached row read back as
 * decode(code) * 2^(scale byte - 127) ([impl-detail] "实践建议": a block's
 * KV quantised on its own).  With bf16 queries, head_dim 128 and
 * block_size a multiple of 16, the blocks the sequences hold (the first
 * ceil(L_b / bs) table entries) are first dequantised into a bf16 staging
 * pool and a table in `workspace` (device, 256-byte aligned, at least
 * paged_prefill_attention_fp8_workspace_size bytes, owned by the caller,
 * overwritten), then the matrix-core kernel runs on them; bf16 holds every
 * read-back value exactly for row scales 2^-124 .. 2^119.  Otherwise (fp16
 * queries, head_dim 64, other block sizes) a generic kernel reads the codes
 * in place, applying each row's scale in fp32, exact for every scale, and
 * the workspace is not used.  q_dtype PKV_BF16 or PKV_F16 (else
 * UNSUPPORTED); out_dtype PKV_F32 or q_dtype (else INVALID).  Other
 * arguments as for paged_prefill_attention.  Errors: INVALID, UNSUPPORTED,
 * WORKSPACE, HIP.
 */
size_t paged_prefill_attention_fp8_workspace_size(int32_t num_seqs, int32_t max_context_len,
                                                  const pkv_cache_layout* layout);
int paged_prefill_attention_fp8(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                                const int32_t* q_start, const int32_t* context_lens, int32_t num_seqs,
                                int32_t max_q_len, const void* key_cache, const void* value_cache,
                                const uint8_t* key_scales, const uint8_t* value_scales,
                                const pkv_cache_layout* layout, const int32_t* block_tables,
                                int32_t block_table_stride, int32_t num_q_heads, int32_t max_context_len,
                                float scale, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------- FP8 KV */
/*
 * 8-bit KV blocks ([impl-detail] "实践建议": the KV inside a block can be
 * quantised on its own).  A cache with layout->dtype == PKV_FP8_E4M3 holds
 * one byte per element: an OCP E4M3 code (bias 7, largest finite 448, no
 * infinities).  Every token row of every KV head is quantised on its own
 * when it is written, with a power-of-two scale 2^e stored as one OCP E8M0
 * byte (e + 127) per row:
 *     e    = smallest integer with max|x| <= 448 * 2^e, clamped to
 *            [-126, 127] (0 for an all-zero row),
 *     code = E4M3(x * 2^-e), round to nearest, ties to even; a negative-zero
 *            code is stored as 0x00,
 * and the row reads back as E4M3(code) * 2^e.  The maximum runs over the
 * row's finite elements; an infinity or a NaN is stored as the E4M3 NaN
 * code with its sign (0x7F, 0xFF), so it reads back as NaN.  Scale bytes mirror the code
 * layout with one byte per row: the scale of row (pb, h, off) is at
 *     scales + pb * (block_stride / head_dim) + h * (head_stride / head_dim) + off
 * (an interleaved scale pool [N, 2, H_kv, bs] next to a code pool
 * [N, 2, H_kv, bs, D]: key scales = pool, value scales = pool + H_kv * bs).
 * The write calls accept head_dim 64 or 128; the
 * attention takes the stream path shapes (head_dim 128, H_kv <= 8,
 * H_q / H_kv <= 8, block_size a multiple of 16).
 */

/*
 * paged_kv_write into 8-bit blocks: key/value (device, [num_tokens, H_kv,
 * D] contiguous, 16-byte aligned) in src_dtype (PKV_F32, PKV_F16 or
 * PKV_BF16) are quantised row by row as above and stored at slot_mapping
 * (device int64 [num_tokens]; slots outside the pool are skipped) with their
 * scale bytes in key_scales / value_scales (device).  Errors: INVALID,
 * UNSUPPORTED, HIP.
 */
int paged_kv_write_fp8(const void* key, const void* value, int32_t src_dtype,
                       const int64_t* slot_mapping, int32_t num_tokens, void* key_cache,
                       void* value_cache, uint8_t* key_scales, uint8_t* value_scales,
                       const pkv_cache_layout* layout, void* stream);

/* pkv_decode_write into 8-bit blocks: the same quantised write with the
 * step's slots and lengths from host memory (kernel arguments), the block
 * table entries and lens_out as pkv_decode_write sets them. */
int pkv_decode_write_fp8(const void* key, const void* value, int32_t src_dtype,
                         const int64_t* slots, const int32_t* lens, int32_t num_rows,
                         void* key_cache, void* value_cache, uint8_t* key_scales,
                         uint8_t* value_scales, const pkv_cache_layout* layout,
                         int32_t* block_tables, int32_t table_rows, int32_t block_table_stride,
                         int32_t* lens_out, void* stream);

/*
 * paged_decode_attention over 8-bit blocks: the same quantity, with each
 * cached row read back as E4M3(code) * 2^e.  Arithmetic: scores and sums in
 * fp32; each row's weight (probability times its V scale) reaches the
 * matrix cores to about 2^-22 of the largest weight of its segment, for any
 * spread of the row scales.  q (device, [num_seqs,
 * num_q_heads, 128]) is q_dtype (PKV_BF16 or PKV_F16); out is PKV_F32 or
 * q_dtype.  phases: 1 = the attention kernel only, 2 = the merge only, 3 =
 * both (the pair 1 then 2 on one stream equals 3).  The workspace is that of
 * paged_decode_attention with partition_tokens 0.  Scale pointers must be
 * 4-byte aligned.  Errors: INVALID, UNSUPPORTED (shapes outside the stream
 * path), WORKSPACE, HIP.
 */
int paged_decode_attention_fp8(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                               const void* key_cache, const void* value_cache,
                               const uint8_t* key_scales, const uint8_t* value_scales,
                               const int32_t* block_tables, int32_t block_table_stride,
                               const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t max_context_len, float scale, const pkv_cache_layout* layout,
                               int32_t phases, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * pkv_decode_step over 8-bit blocks: key/value (device, [num_seqs, H_kv, D],
 * q_dtype) are quantised as paged_kv_write_fp8 quantises them, then the
 * 8-bit attention runs, with the same results, bit for bit, as
 * pkv_decode_write_fp8 followed by paged_decode_attention_fp8.  Under the
 * conditions of pkv_decode_step the write runs inside the attention launch:
 * the one wave per KV head that reads a sequence's last tile quantises the
 * new rows (the same encoding) and stores codes and scale bytes.  phases as
 * for paged_decode_attention_fp8.  Errors: INVALID, UNSUPPORTED, WORKSPACE,
 * HIP.
 */
int pkv_decode_step_fp8(void* out, int32_t out_dtype, const void* q, int32_t q_dtype, const void* key,
                        const void* value, const int64_t* slots, const int32_t* lens, int32_t num_seqs,
                        void* key_cache, void* value_cache, uint8_t* key_scales, uint8_t* value_scales,
                        const pkv_cache_layout* layout, int32_t* block_tables,
                        int32_t block_table_stride, int32_t* lens_out, int32_t num_q_heads,
                        int32_t max_context_len, float scale, int32_t phases, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Apply the table growth of one batched append to a device-resident block
 * table: for every i with new_block[i] >= 0,
 *     block_tables[rows[i] * block_table_stride + (lens[i] - 1) / bs] = new_block[i]
 * (the block a decode append opened holds the token at position lens[i]-1,
 * [MiniPaged-Qwen] §9.2).  block_tables: device int32 [num_rows,
 * block_table_stride]; rows, lens, new_block: device int32 [n]; rows may be
 * NULL, meaning row i.  Entries whose target row or column falls outside the
 * table are skipped.  Errors: INVALID, HIP.
 */
int pkv_update_block_tables(int32_t* block_tables, int32_t num_rows,
                            int32_t block_table_stride, const int32_t* rows,
                            const int32_t* lens, const int32_t* new_block, int32_t n,
                            int32_t block_size, void* stream);

/*
 * Whole rows of device block tables ([MiniPaged-Qwen] §16.5, the batch
 * block-table tensor): for i < n, row src_rows[i] (or row i when src_rows
 * is NULL) of `src` is copied to row dst_rows[i] (or row i) of `dst`,
 * entries 0 .. width-1.  Used to publish the rows of admitted sequences
 * into a device-resident table (dst_rows = their rows, src = the manager's
 * rows staged on the device, pkv_get_block_tables) and to gather the rows
 * of a prefill batch (src_rows = their rows).  dst, src: device int32
 * tables with `*_stride` entries per row (>= width) and `*_num_rows` rows;
 * dst_rows, src_rows: device int32 [n] or NULL.  Rows outside either table
 * are skipped.  dst_rows must be distinct (two copies into one row race).
 * Errors: INVALID, UNSUPPORTED, HIP.
 */
int pkv_copy_table_rows(int32_t* dst, int32_t dst_stride, int32_t dst_num_rows, const int32_t* dst_rows,
                        const int32_t* src, int32_t src_stride, int32_t src_num_rows, const int32_t* src_rows,
                        int32_t n, int32_t width, void* stream);

/* Library version string, e.g. "pkv 0.1.0 gfx950". */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
