/*
 * pagedkv.h -- C ABI of a paged KV-cache decode library for AMD MI355X (gfx950).
 *
 * Sources (web pages on vLLM's PagedAttention):
 *   [card]    "PagedAttention", llm-engineer.pages.dev
 *   [explain] "vLLM KV cache and PagedAttention explained", hrletsgo.me
 *   [velog]   "vLLM의 PagedAttention 아키텍처와 GPU 메모리 최적화 원리", velog.io
 *
 * Cache layout.  K and V are two separate, contiguous pools of fixed-size
 * physical blocks, each laid out [num_blocks, num_heads, block_size, head_dim]
 * ([velog] section 4, the 4-D layout [Block, Head, Block_Size, Head_D]).  One
 * (block, head) tile of block_size * head_dim elements is contiguous, so a
 * block is read as whole coalesced rows ([card] "Kernel은 무엇이 달라지는가":
 * the scatter is per block, not per token).
 *
 * Block tables.  Row i of block_tables (int32, [num_seqs, max_blocks_per_seq],
 * row-major) lists the physical blocks of sequence i: entry j holds logical
 * tokens j*block_size .. j*block_size + block_size - 1 ([card] "OS paging과
 * 같은 발상"; [explain] Step 5).  A sequence of L tokens uses the first
 * ceil(L / block_size) entries ([explain] Step 6); later entries are never
 * read.  One physical block may appear in several rows (read-only prefix
 * sharing, [explain] Step 9).
 *
 * Slot mapping.  slot = block * block_size + offset names offset `offset` of
 * physical block `block` ("slot 6 of block 42", [explain] Steps 6-7); a
 * negative slot means "no write".
 *
 * Element types.  q, the caches and out share one type: PKV_F32, PKV_F16 or
 * PKV_BF16.  Arithmetic is fp32 throughout; out is rounded to nearest even.
 * Supported shapes: head_dim 64 or 128, block_size 16 or 32.
 *
 * Pointers and ownership.  Every array argument is a DEVICE pointer to memory
 * the caller allocated and owns; the library allocates nothing, keeps no state
 * between calls and never retains a pointer (the one exception is the scratch
 * array of paged_attention_decode_step_noalloc, below).  `stream` is a hipStream_t passed
 * as void* (NULL = the legacy default stream).  All work is enqueued
 * asynchronously on `stream`; nothing synchronises with the host except in
 * PKV_DEBUG mode (below).  Outputs must not alias inputs.  Arrays of
 * elements (q, k, v, k_new, v_new, the caches, out) and the workspace are
 * moved in 16-byte vectors and must be 16-byte aligned; int32 metadata must be
 * 4-byte and int64 metadata 8-byte aligned (PKV_EINVAL otherwise).
 *
 * Errors.  Every call validates its scalar arguments and pointers on the host
 * before any HIP call; on failure it returns a non-zero pkv_status, launches
 * nothing and leaves a message for pkv_last_error().  A failed launch returns
 * PKV_EHIP.  Faults inside a kernel surface at the caller's next
 * synchronisation, as for any HIP kernel.
 *
 * Caller contract on metadata (device data the host does not read): block ids
 * in [0, num_blocks), 0 <= context_lens[i] <= max_blocks_per_seq*block_size,
 * no two non-negative equal slots in one write.  The kernels never read or
 * write outside the arrays when it is broken: an out-of-range block id or
 * context length turns that sequence's output rows into NaN, and a slot whose
 * block is out of range is not written.  With the environment variable
 * PKV_DEBUG=1 each call also copies the metadata to the host, synchronising
 * `stream`, and returns PKV_EINVAL naming the first violation.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

/* partition_size value that lets the library choose the split (see below). */
#define PKV_PARTITION_AUTO (-1)

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,        /* bad argument: null pointer, negative or inconsistent size      */
  PKV_EUNSUPPORTED = 2,  /* valid but not built: dtype, head_dim, block_size, grid too big */
  PKV_EWORKSPACE = 3,    /* workspace missing or smaller than paged_attention_workspace_bytes */
  PKV_EHIP = 4,          /* the HIP runtime refused a launch or a copy                      */
  PKV_ENOSPACE = 5       /* block pool: too few free blocks (nothing was changed)          */
} pkv_status;

/*
 * paged_kv_write -- store each new token's K and V rows in its cache slot.
 *
 * For every t in [0, num_tokens) with s = slot_mapping[t] >= 0:
 *   k_cache[s / block_size, h, s % block_size, :] = k[t, h, :]   for all heads h
 *   v_cache[...same...]                           = v[t, h, :]
 * This is the decode step's append of the new token's K/V into the next slot
 * of its sequence's last block ([explain] Step 6: "stored in slot 6 of block
 * 42"; [card] "vLLM에서의 위치": the worker prepares the slot mapping).  The
 * copy moves stored bits and is exact.
 *
 *   k, v          [num_tokens, num_heads, head_dim], dtype, contiguous, read
 *   slot_mapping  [num_tokens] int64, read
 *   k_cache,
 *   v_cache       [num_blocks, num_heads, block_size, head_dim], dtype, written
 *                 only at the named slots
 * Returns PKV_OK, or an error status with nothing launched.  num_tokens == 0
 * is a no-op.
 */
pkv_status paged_kv_write(const void* k, const void* v, const int64_t* slot_mapping, int64_t num_tokens,
                   void* k_cache, void* v_cache, int64_t num_blocks, int32_t num_heads,
                   int32_t head_dim, int32_t block_size, int32_t dtype, void* stream);

/*
 * paged_attention_partition_size -- the partition size, in tokens, that
 * paged_attention_decode uses for these sizes: partition_size itself, or for
 * PKV_PARTITION_AUTO the library's choice.  The automatic choice is 0 (no
 * split) when num_seqs * num_heads >= 1024, since the grid then already holds
 * several work-groups per compute unit; otherwise the smallest multiple of 1024
 * tokens that cuts the table's capacity (max_blocks_per_seq * block_size) into
 * at most ceil(1280 / (num_seqs * num_heads)) partitions, or 0 if that is the
 * whole capacity.  Results do not depend on the split beyond fp32 rounding.
 */
int32_t paged_attention_partition_size(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                       int32_t block_size, int32_t partition_size);

/*
 * paged_attention_workspace_bytes -- device scratch that paged_attention_decode
 * needs for its split-context partials with these sizes (0 when no sequence
 * can span more than one partition).  Returns 0 for invalid sizes as well;
 * paged_attention_decode reports those.
 */
size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                       int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t partition_size);

/*
 * paged_attention_decode -- one query token per sequence attends over that
 * sequence's paged K/V cache, read in place through its block table.
 *
 * For each sequence i with L = context_lens[i] and each head h:
 *   out[i, h, :] = softmax_t( scale * q[i, h, :] . K_i[t, h, :] ) V_i[t, h, :],  t in [0, L)
 * where K_i[t] = k_cache[block_tables[i, t / block_size], :, t % block_size, :]
 * and likewise V_i ([explain] Appendix: Attention(Q,K,V) = softmax(QK^T/sqrt(d))V,
 * evaluated by walking the block table one block at a time with a running
 * softmax normalisation).  Rows with L == 0 are zero.
 *
 * Long contexts are split into partitions of partition_size tokens, each
 * reduced independently and then merged by log-sum-exp weights; the result is
 * the same softmax (the pages name this FlashDecoding, [card] "헷갈리기 쉬운 구분").
 * partition_size must be a multiple of block_size; 0 means never split and
 * PKV_PARTITION_AUTO lets the library choose (paged_attention_partition_size).
 *
 *   q             [num_seqs, num_heads, head_dim], dtype, read
 *   k_cache,
 *   v_cache       [num_blocks, num_heads, block_size, head_dim], dtype, read
 *   block_tables  [num_seqs, max_blocks_per_seq] int32, read
 *   context_lens  [num_seqs] int32, read
 *   out           [num_seqs, num_heads, head_dim], dtype, written
 *   workspace     >= paged_attention_workspace_bytes(...) bytes of device memory,
 *                 used as scratch (may be NULL when that is 0); no initial
 *                 contents needed; must not be shared by concurrent calls
 * Returns PKV_OK, or an error status with nothing launched.
 */
pkv_status paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                           int32_t dtype, void* out, void* workspace, size_t workspace_bytes,
                           int32_t partition_size, void* stream);

/*
 * paged_attention_prefill -- causal attention of a batch of new tokens over
 * their sequences' paged caches (the prefill phase, [explain] Step 6: all
 * prompt tokens are processed in parallel, each attending to the tokens before
 * it and itself; Summary: causal attention).
 *
 * Sequence i brings the queries q[query_start[i] .. query_start[i+1]) (P_i of
 * them) and holds L_i = context_lens[i] >= P_i cached tokens whose last P_i are
 * these queries' own K/V, already written (paged_kv_write).  Query j sits at
 * position p = L_i - P_i + j and
 *   out[query_start[i] + j, h, :] = softmax_t( scale * q[.., h, :] . K_i[t, h, :] ) V_i[t, h, :],  t in [0, p]
 * with K_i, V_i read through block_tables as in paged_attention_decode.  Tokens
 * before the new ones (L_i - P_i > 0) are a cached prefix: an earlier chunk of
 * the prompt, or blocks shared with other requests ([explain] Step 9).
 *
 *   q             [T, num_heads, head_dim], dtype, T = query_start[num_seqs]
 *   k_cache,
 *   v_cache       [num_blocks, num_heads, block_size, head_dim], dtype
 *   block_tables  [num_seqs, max_blocks_per_seq] int32
 *   query_start   [num_seqs + 1] int32, non-decreasing, query_start[0] = 0
 *   context_lens  [num_seqs] int32
 *   max_query_len at least every P_i (sizes the grid)
 *   out           [T, num_heads, head_dim], dtype, written
 * Runs on the matrix cores (MFMA) with fp32 accumulation; the output is
 * rounded to nearest even.  Caller contract, checked under PKV_DEBUG=1:
 * P_i <= max_query_len, P_i <= L_i <= max_blocks_per_seq * block_size, block ids
 * in range; a sequence that breaks it gets NaN rows, and no memory outside the
 * arrays is touched.  Returns PKV_OK, or an error status with nothing launched:
 * PKV_EUNSUPPORTED when num_heads, num_seqs or ceil(max_query_len / 128)
 * exceeds 65535, or (16-bit types) when the launch of one 256-thread
 * work-group per (sequence, head, 128-query tile) would exceed 2^32 threads.
 */
pkv_status paged_attention_prefill(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* query_start, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_query_len, int32_t num_heads, int32_t head_dim,
                            int32_t block_size, int64_t num_blocks, float scale, int32_t dtype, void* out,
                            void* stream);

/*
 * paged_kv_copy_blocks -- copy whole physical blocks, K and V: for every pair
 * i, block block_mapping[2i+1] of each pool receives the contents of block
 * block_mapping[2i].  This is the copy in copy-on-write ([explain] Step 9: a
 * request about to write into a block it shares first gets a private copy, and
 * its table is pointed at the copy); pkv_pool_append_slots reports the pairs.
 * A block is every head and slot: num_heads * block_size * head_dim elements,
 * one contiguous run per pool.  The copy moves stored bits and is exact.
 *
 *   k_cache,
 *   v_cache        [num_blocks, num_heads, block_size, head_dim], dtype
 *   block_mapping  [num_pairs, 2] int64 (source, destination), read
 * Destinations must be distinct and none may also be a source (the copies run
 * concurrently); PKV_DEBUG=1 checks this and the id range on the host.  A pair
 * with an id outside [0, num_blocks) is skipped by the kernel.  Returns PKV_OK,
 * or an error status with nothing launched.  num_pairs == 0 is a no-op.
 */
pkv_status paged_kv_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int64_t num_pairs,
                         int64_t num_blocks, int32_t num_heads, int32_t head_dim, int32_t block_size,
                         int32_t dtype, void* stream);

/*
 * paged_kv_prepare_step -- a decode step's metadata, updated on the device.
 * Applies table updates, sets context lengths, and writes each row's slot
 * mapping: the slot of its newest token, block_tables[r, (L-1) / block_size] *
 * block_size + (L-1) % block_size with L = context_lens[r] ([explain] Step 6:
 * the decode token goes to the next slot of the sequence's last block), or -1
 * for an idle row (L = 0), which paged_kv_write then skips.  pkv_batch_plan_step
 * produces the updates and lengths.
 *
 *   block_tables  [num_seqs, max_blocks_per_seq] int32, device, updated in place
 *   context_lens  [num_seqs] int32, device, overwritten with new_lens when given
 *   updates       [num_updates, 3] int32 (row, column, block id), device; the
 *                 (row, column) pairs of one call are distinct
 *   new_lens      [num_seqs] int32, device, or NULL to keep context_lens
 *   slot_mapping  [num_seqs] int64, device, written (NULL: not computed)
 * All device pointers; the call is asynchronous on `stream`.  Entries outside
 * the arrays are skipped; a row whose length or block id is out of range gets
 * slot -1.  Returns PKV_OK, or an error status with nothing launched.
 */
pkv_status paged_kv_prepare_step(int32_t* block_tables, int32_t max_blocks_per_seq, int32_t* context_lens, int32_t num_seqs,
                          const int32_t* updates, int64_t num_updates, const int32_t* new_lens,
                          int64_t* slot_mapping, int32_t block_size, int64_t num_blocks, void* stream);

/*
 * paged_attention_decode_step -- one decode step in one launch: the append of
 * each sequence's newest token and the attention over its cache.  Equivalent to
 * paged_kv_write of k_new[i], v_new[i] into the slot of position L - 1
 * (block_tables[i, (L-1) / block_size] * block_size + (L-1) % block_size, with
 * L = context_lens[i] the length after the append; [explain] Step 6: the decode
 * token's K/V goes to the next slot of its last block) followed by
 * paged_attention_decode with the same arguments: same results, bit for bit.
 * Within the launch, the one wave of each (sequence, head) that reads the
 * block of position L - 1 first stores that row from k_new / v_new into its
 * slot, and reads the block only once the store has completed.  Rows with
 * L = 0 append nothing and are zero.
 *
 *   k_new, v_new  [num_seqs, num_heads, head_dim], dtype, read
 *   k_cache,
 *   v_cache       written at the newest slots, read everywhere else
 * Other arguments, ownership and errors as for paged_attention_decode.
 */
pkv_status paged_attention_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                int32_t block_size, int64_t num_blocks, float scale, int32_t dtype, void* out,
                                void* workspace, size_t workspace_bytes, int32_t partition_size, void* stream);

/*
 * paged_attention_decode_step_noalloc -- paged_attention_decode_step for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments and
 * results, without the workspace: the split-context partials go to a scratch
 * array of PKV_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on each
 * GPU it runs on, until the process ends.  The call allocates nothing (no
 * hipMalloc, no allocating library routine); its first call on a device looks
 * up that device's copy of the array.
 *
 * Returns PKV_EWORKSPACE, with nothing launched, when the split would need
 * more scratch than that (paged_attention_workspace_bytes for the same sizes
 * and partition_size above 16 MiB): choose a larger partition_size, or call
 * paged_attention_decode_step with a workspace.  Every call on one GPU uses
 * that GPU's one array, so calls that overlap on one GPU (other streams, other
 * host threads) race with each other; the caller must order them.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (16u << 20)
pkv_status paged_attention_decode_step_noalloc(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                        void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                        int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                        int32_t dtype, void* out, int32_t partition_size, void* stream);

/* Text of the calling thread's last non-OK status (empty string if none). */
const char* pkv_last_error(void);

/*
 * ---- Block pool: host-side bookkeeping of physical blocks ----
 *
 * The scheduler's side of paged KV memory ([card] "OS paging과 같은 발상",
 * "vLLM에서의 위치"; [explain] Steps 5-9).  A pool hands out block ids for
 * sequences named by caller-chosen int64 ids, keeps a block table and a token
 * count per sequence, and a reference count per block (the number of tables
 * holding it).  It touches no GPU memory: its outputs (tables, context lengths,
 * slot ids, copy pairs) are host arrays for the caller to upload and pass to
 * paged_kv_copy_blocks, paged_kv_write and paged_attention_decode.
 *
 * Policy.  Token t of a sequence lives in logical block t / block_size.
 * Allocation takes blocks from the front of an ordered free list; blocks whose
 * count drops to zero return to the front in table order, so the next request
 * receives the space just released ([explain] Steps 7-8).  A block is copied
 * before a write only while another table still holds it; the last holder
 * writes in place.  Every call is all-or-nothing: PKV_ENOSPACE and PKV_EINVAL
 * leave the pool unchanged.  A pool is not thread-safe; calls on one pool must
 * not overlap.  All pointers here are HOST pointers.
 */
typedef struct pkv_block_pool pkv_block_pool;

/* A pool of num_blocks blocks of block_size tokens; free_order (may be NULL =
 * 0, 1, 2, ...) lists every block id once, front first.  NULL on bad input. */
pkv_block_pool* pkv_pool_create(int64_t num_blocks, int32_t block_size, const int32_t* free_order);
void pkv_pool_destroy(pkv_block_pool* pool);

/* New sequence `seq` holding num_tokens tokens in ceil(num_tokens / block_size)
 * fresh blocks ([explain] Step 6: blocks are allocated at the start of prefill). */
pkv_status pkv_pool_allocate(pkv_block_pool* pool, int64_t seq, int64_t num_tokens);

/* New sequence `child` sharing all of `parent`'s blocks (each gains a
 * reference): a shared prompt prefix or parallel samples ([explain] Step 9). */
pkv_status pkv_pool_fork(pkv_block_pool* pool, int64_t parent, int64_t child);

/* Reserve slots for n new tokens of `seq`.  slots_out[n] receives each token's
 * flat slot (block * block_size + offset) for paged_kv_write.  A new block is
 * appended at each block boundary ([explain] Step 6).  If the partly filled
 * last block is shared, it is replaced by a fresh block and the pair (old, new)
 * goes to copies_out (int64 [max_copies, 2]); *num_copies receives the count
 * (0 or 1).  The copies must run (paged_kv_copy_blocks) before the write. */
pkv_status pkv_pool_append_slots(pkv_block_pool* pool, int64_t seq, int64_t n, int64_t* slots_out,
                          int64_t* copies_out, int64_t max_copies, int64_t* num_copies);

/* Flat slots (block * block_size + offset) of tokens first .. first + n - 1 of
 * `seq`, which must all be held already (e.g. a prompt just allocated, to be
 * written with paged_kv_write): slots_out[n] ([explain] Steps 5-6: token t
 * of a request sits at offset t % block_size of the block its table lists at
 * t / block_size).  PKV_EINVAL for an unknown sequence or tokens it does not
 * hold. */
pkv_status pkv_pool_slots(const pkv_block_pool* pool, int64_t seq, int64_t first, int64_t n, int64_t* slots_out);

/* Drop `seq`; blocks no other table holds return to the free list ([explain]
 * Step 7: released blocks are immediately reusable). */
pkv_status pkv_pool_free(pkv_block_pool* pool, int64_t seq);

/* Padded int32 block tables [n, width] (unused entries -1) and int32 context
 * lengths [n] of the listed sequences, ready for paged_attention_decode. */
pkv_status pkv_pool_build_tables(const pkv_block_pool* pool, const int64_t* seqs, int32_t n, int32_t width,
                          int32_t* tables_out, int32_t* lens_out);

/* Queries: free block count; a block's reference count (-1 for a bad id);
 * a sequence's token count (-1 if unknown); a sequence's table (writes up to
 * cap ids, returns its length, -1 if unknown); the free list front first
 * (writes up to cap ids, returns its length). */
int64_t pkv_pool_num_free(const pkv_block_pool* pool);
int32_t pkv_pool_refcount(const pkv_block_pool* pool, int64_t block);
int64_t pkv_pool_num_tokens(const pkv_block_pool* pool, int64_t seq);
int64_t pkv_pool_table(const pkv_block_pool* pool, int64_t seq, int32_t* out, int64_t cap);
int64_t pkv_pool_free_list(const pkv_block_pool* pool, int32_t* out, int64_t cap);

/* Slot accounting ([explain] "Why Waste Stays Below 4%" and the step-6 waste
 * calculation).  Paged waste = 1 - stored_tokens / allocated_slots (the empty
 * tail slots of each sequence's last block); static-reservation waste for a
 * maximum length M = 1 - logical_tokens / (sequences * M). */
typedef struct {
  int64_t num_blocks;
  int64_t free_blocks;
  int64_t used_blocks;      /* blocks held by at least one table                          */
  int64_t sequences;
  int64_t logical_tokens;   /* sum of sequence lengths (a shared token once per reader)   */
  int64_t stored_tokens;    /* filled slots of used blocks, a shared block counted once   */
  int64_t allocated_slots;  /* used_blocks * block_size                                   */
  int64_t shared_blocks;    /* used blocks held by more than one table                    */
} pkv_pool_usage_t;
pkv_status pkv_pool_usage(const pkv_block_pool* pool, pkv_pool_usage_t* out);

/* The waste comparison derived from pkv_pool_usage ([explain] the step-6
 * calculation: static reservation of max_model_len slots per request against
 * the paged blocks).  A zero max_model_len or bytes_per_token leaves the
 * fields that need it at zero. */
typedef struct {
  int64_t empty_slots;      /* allocated_slots - stored_tokens: empty tails of last blocks    */
  double paged_waste;       /* empty_slots / allocated_slots (0 when nothing is allocated)    */
  int64_t static_slots;     /* sequences * max_model_len                                      */
  double static_waste;      /* 1 - logical_tokens / static_slots (0 when static_slots is 0)   */
  int64_t paged_bytes;      /* allocated_slots * bytes_per_token                              */
  int64_t stored_bytes;     /* stored_tokens * bytes_per_token                                */
  int64_t static_bytes;     /* static_slots * bytes_per_token                                 */
} pkv_waste_t;
pkv_status pkv_pool_waste(const pkv_block_pool* pool, int64_t max_model_len, int64_t bytes_per_token, pkv_waste_t* out);

/* Usage and waste of n requests of the given lengths, each with `samples`
 * parallel samples sharing its prompt ([explain] Step 9), in a pool of exactly
 * the blocks the prompts need (request i is allocated as sequence i * samples
 * and forked samples - 1 times). */
pkv_status pkv_account(const int64_t* lens, int32_t n, int32_t block_size, int32_t samples, int64_t max_model_len,
                int64_t bytes_per_token, pkv_pool_usage_t* usage_out, pkv_waste_t* waste_out);

/*
 * ---- Batch: decode rows over a pool, with a mirror of the device tables ----
 *
 * A batch of `rows` rows (each idle or running one sequence of `pool`) whose
 * block tables live on the device as [rows, width] int32, filled with -1 before
 * the first step.  The batch keeps a host mirror of them, so a plan lists only
 * the entries that changed since the previous plan: a new block every
 * block_size tokens, a copy-on-write replacement, a reassigned row.  It is the
 * bookkeeping of a continuous-batching loop ([explain] Step 8: a finished
 * request's row is immediately given to a new one; the policy of which request
 * comes next is the caller's).  Host pointers; not thread-safe.  The batch
 * borrows the pool, which must outlive it.
 */
typedef struct pkv_batch pkv_batch;

pkv_batch* pkv_batch_create(pkv_block_pool* pool, int32_t rows, int32_t width);
void pkv_batch_destroy(pkv_batch* batch);

/* Row `row` now runs sequence `seq` (which must exist in the pool and fit in
 * `width` blocks), or is idle when seq < 0.  Takes effect at the next plan. */
pkv_status pkv_batch_set_row(pkv_batch* batch, int32_t row, int64_t seq);

/* One step's bookkeeping.  Every non-idle row's sequence grows by
 * tokens_per_row tokens (pkv_pool_append_slots; 1 for a decode step, 0 to only
 * synchronise the tables).  Outputs: updates_out [n_updates, 3] (row, column,
 * block id; -1 clears an entry), which must hold rows * width entries;
 * lens_out [rows], every row's context length after the step (0 when idle);
 * copies_out [n_copies, 2], the block copies to run before the step's writes.
 * Upload updates and lens, then paged_kv_prepare_step, paged_kv_copy_blocks,
 * paged_kv_write and paged_attention_decode.  PKV_ENOSPACE (too few free
 * blocks) and PKV_EINVAL leave the pool and the batch unchanged. */
pkv_status pkv_batch_plan_step(pkv_batch* batch, int32_t tokens_per_row, int32_t* updates_out, int64_t max_updates,
                        int64_t* n_updates, int32_t* lens_out, int64_t* copies_out, int64_t max_copies,
                        int64_t* n_copies);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
