// C-ABI front end: host-side validation, workspace sizing, dispatch and the
// optional metadata checks.  No HIP call happens before validation succeeds.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <unordered_set>
#include <vector>

#include "pagedkv.h"
#include "pkv_internal.h"

namespace {

thread_local std::string g_last_error;

}  // namespace

pkv_status pkv::set_error(int code, const std::string& message) {
  g_last_error = message;
  return static_cast<pkv_status>(code);
}

namespace {

pkv_status fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return static_cast<pkv_status>(code);
}

pkv_status ok() {
  g_last_error.clear();
  return PKV_OK;
}

bool debug_checks() {
  const char* e = getenv("PKV_DEBUG");
  return e != nullptr && e[0] == '1';
}

int elem_bytes(int32_t dtype) { return dtype == PKV_F32 ? 4 : 2; }

// Shared shape checks of both calls.
pkv_status check_shape(int32_t dtype, int32_t num_heads, int32_t head_dim, int32_t block_size,
                int64_t num_blocks) {
  if (dtype != PKV_F32 && dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(PKV_EUNSUPPORTED, "dtype %d is not PKV_F32, PKV_F16 or PKV_BF16", dtype);
  if (num_heads <= 0) return fail(PKV_EINVAL, "num_heads must be positive (got %d)", num_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (block_size != 16 && block_size != 32)
    return fail(PKV_EUNSUPPORTED, "block_size %d not supported (16 or 32)", block_size);
  if (num_blocks <= 0) return fail(PKV_EINVAL, "num_blocks must be positive (got %lld)", (long long)num_blocks);
  // every byte offset into a cache pool must fit in int64
  const double pool_bytes = double(num_blocks) * num_heads * block_size * head_dim * elem_bytes(dtype);
  if (pool_bytes > 4.0e18) return fail(PKV_EINVAL, "cache pool of %.3g bytes is too large", pool_bytes);
  return PKV_OK;
}

// Element arrays move in 16-byte vectors; metadata is read in whole words.
bool misaligned(const void* p, uintptr_t n) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & (n - 1)) != 0; }

pkv_status hip_fail(hipError_t e, const char* what) {
  return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Partitions the grid spans: ceil(max_blocks / part_blocks).
int64_t partitions_for(int32_t max_blocks, int32_t part_blocks) {
  return (int64_t(max_blocks) + part_blocks - 1) / part_blocks;
}

int32_t part_blocks_for(int32_t max_blocks, int32_t block_size, int32_t partition_size) {
  return partition_size == 0 ? max_blocks : partition_size / block_size;
}

// Automatic split.  With at least kAutoMinRows (sequence, head) rows the grid
// already holds several work-groups per compute unit, and one pass per row
// is fastest (no partials, no merge).  With fewer rows, contexts are cut into
// partitions, multiples of kAutoGrain tokens, so that about
// kAutoTargetGroups work-groups (about 5 per compute unit) cover the longest
// possible context.  Measured on 16-token blocks of 40 heads x 128 dims, one
// sequence of 32k tokens takes 104.7 us at 512-token partitions, 103.7 at
// 1024 (the split this picks), 108.3 at 2048 and 123.5 at 4096; four
// sequences of 32k take 400.1 us at 4096 (picked) and 402.0 at 2048.
constexpr int64_t kAutoMinRows = 1024;
constexpr int64_t kAutoTargetGroups = 1280;
constexpr int64_t kAutoGrain = 1024;

int32_t resolve_partition(int32_t num_seqs, int32_t num_heads, int32_t max_blocks, int32_t block_size,
                          int32_t partition_size) {
  if (partition_size != PKV_PARTITION_AUTO) return partition_size;
  const int64_t rows = int64_t(num_seqs) * num_heads;
  const int64_t cap = int64_t(max_blocks) * block_size;
  if (rows <= 0 || rows >= kAutoMinRows) return 0;
  const int64_t want = (kAutoTargetGroups + rows - 1) / rows;
  int64_t part = (cap + want - 1) / want;
  part = (part + kAutoGrain - 1) / kAutoGrain * kAutoGrain;
  return part >= cap ? 0 : int32_t(part);
}

}  // namespace

extern "C" const char* pkv_last_error(void) { return g_last_error.c_str(); }

extern "C" int32_t paged_attention_partition_size(int32_t num_seqs, int32_t num_heads,
                                                  int32_t max_blocks_per_seq, int32_t block_size,
                                                  int32_t partition_size) {
  return resolve_partition(num_seqs, num_heads, max_blocks_per_seq, block_size, partition_size);
}

extern "C" size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                                  int32_t head_dim, int32_t max_blocks_per_seq,
                                                  int32_t block_size, int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 || block_size <= 0)
    return 0;
  partition_size = resolve_partition(num_seqs, num_heads, max_blocks_per_seq, block_size, partition_size);
  if (partition_size < 0 || partition_size % block_size != 0) return 0;
  const int32_t pb = part_blocks_for(max_blocks_per_seq, block_size, partition_size);
  return pkv::workspace_layout(num_seqs, num_heads, head_dim, partitions_for(max_blocks_per_seq, pb)).bytes;
}

extern "C" pkv_status paged_kv_write(const void* k, const void* v, const int64_t* slot_mapping,
                              int64_t num_tokens, void* k_cache, void* v_cache, int64_t num_blocks,
                              int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                              void* stream) {
  if (num_tokens < 0) return fail(PKV_EINVAL, "num_tokens must be >= 0 (got %lld)", (long long)num_tokens);
  if (pkv_status rc = check_shape(dtype, num_heads, head_dim, block_size, num_blocks)) return rc;
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(PKV_EINVAL, "null pointer among k, v, slot_mapping, k_cache, v_cache");
  if (misaligned(k, 16) || misaligned(v, 16) || misaligned(k_cache, 16) || misaligned(v_cache, 16) ||
      misaligned(slot_mapping, 8))
    return fail(PKV_EINVAL, "k, v, k_cache and v_cache must be 16-byte aligned, slot_mapping 8-byte aligned");
  const int64_t vecs = num_tokens * int64_t(num_heads) * (head_dim * elem_bytes(dtype) / 16);
  if (vecs / 256 >= (int64_t(1) << 31) - 1) return fail(PKV_EUNSUPPORTED, "num_tokens %lld too large for one launch", (long long)num_tokens);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_checks()) {
    std::vector<int64_t> slots(num_tokens);
    hipError_t e = hipMemcpyAsync(slots.data(), slot_mapping, num_tokens * sizeof(int64_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "PKV_DEBUG copy of slot_mapping");
    std::unordered_set<int64_t> seen;
    for (int64_t t = 0; t < num_tokens; ++t) {
      const int64_t s = slots[t];
      if (s < 0) continue;
      if (s / block_size >= num_blocks)
        return fail(PKV_EINVAL, "slot_mapping[%lld] = %lld names block %lld >= num_blocks %lld", (long long)t,
                    (long long)s, (long long)(s / block_size), (long long)num_blocks);
      if (!seen.insert(s).second)
        return fail(PKV_EINVAL, "slot_mapping[%lld] = %lld repeats an earlier slot", (long long)t, (long long)s);
    }
  }
  hipError_t e = pkv::launch_kv_write(dtype, head_dim, k, v, slot_mapping, num_tokens, k_cache, v_cache,
                                      num_blocks, num_heads, block_size, st);
  if (e != hipSuccess) return hip_fail(e, "paged_kv_write launch");
  return ok();
}

extern "C" pkv_status paged_kv_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                                    int64_t num_pairs, int64_t num_blocks, int32_t num_heads,
                                    int32_t head_dim, int32_t block_size, int32_t dtype, void* stream) {
  if (num_pairs < 0) return fail(PKV_EINVAL, "num_pairs must be >= 0 (got %lld)", (long long)num_pairs);
  if (pkv_status rc = check_shape(dtype, num_heads, head_dim, block_size, num_blocks)) return rc;
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !block_mapping)
    return fail(PKV_EINVAL, "null pointer among k_cache, v_cache, block_mapping");
  if (misaligned(k_cache, 16) || misaligned(v_cache, 16) || misaligned(block_mapping, 8))
    return fail(PKV_EINVAL, "k_cache and v_cache must be 16-byte aligned, block_mapping 8-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_checks()) {
    std::vector<int64_t> m(size_t(2 * num_pairs));
    hipError_t e = hipMemcpyAsync(m.data(), block_mapping, m.size() * sizeof(int64_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "PKV_DEBUG copy of block_mapping");
    std::unordered_set<int64_t> dsts;
    for (int64_t i = 0; i < num_pairs; ++i) {
      const int64_t s = m[size_t(2 * i)], d = m[size_t(2 * i + 1)];
      if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks)
        return fail(PKV_EINVAL, "block_mapping[%lld] = (%lld, %lld) outside [0, %lld)", (long long)i,
                    (long long)s, (long long)d, (long long)num_blocks);
      if (!dsts.insert(d).second)
        return fail(PKV_EINVAL, "block_mapping[%lld] repeats destination %lld", (long long)i, (long long)d);
    }
    for (int64_t i = 0; i < num_pairs; ++i)
      if (dsts.count(m[size_t(2 * i)]))
        return fail(PKV_EINVAL, "block_mapping[%lld] reads block %lld, which is also a destination",
                    (long long)i, (long long)m[size_t(2 * i)]);
  }
  const int64_t block_bytes = int64_t(num_heads) * block_size * head_dim * elem_bytes(dtype);
  hipError_t e = pkv::launch_copy_blocks(block_mapping, num_pairs, k_cache, v_cache, num_blocks, block_bytes, st);
  if (e != hipSuccess) return hip_fail(e, "paged_kv_copy_blocks launch");
  return ok();
}

extern "C" pkv_status paged_kv_prepare_step(int32_t* block_tables, int32_t max_blocks_per_seq, int32_t* context_lens,
                                     int32_t num_seqs, const int32_t* updates, int64_t num_updates,
                                     const int32_t* new_lens, int64_t* slot_mapping, int32_t block_size,
                                     int64_t num_blocks, void* stream) {
  if (num_seqs < 0 || num_updates < 0) return fail(PKV_EINVAL, "num_seqs and num_updates must be >= 0");
  if (max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PKV_EINVAL, "max_blocks_per_seq, block_size and num_blocks must be positive");
  if (num_seqs == 0 && num_updates == 0) return ok();
  if (!block_tables || !context_lens || (num_updates > 0 && !updates))
    return fail(PKV_EINVAL, "null pointer among block_tables, context_lens, updates");
  if (misaligned(block_tables, 4) || misaligned(context_lens, 4) || misaligned(updates, 4) ||
      misaligned(new_lens, 4) || misaligned(slot_mapping, 8))
    return fail(PKV_EINVAL, "block_tables, context_lens, updates and new_lens must be 4-byte aligned, "
                "slot_mapping 8-byte aligned");
  hipError_t e = pkv::launch_prepare_step(block_tables, max_blocks_per_seq, context_lens, num_seqs, updates,
                                          num_updates, new_lens, slot_mapping, block_size, num_blocks,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "paged_kv_prepare_step launch");
  return ok();
}

extern "C" pkv_status paged_attention_prefill(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* query_start, const int32_t* context_lens, int32_t num_seqs,
                                       int32_t max_query_len, int32_t num_heads, int32_t head_dim,
                                       int32_t block_size, int64_t num_blocks, float scale, int32_t dtype,
                                       void* out, void* stream) {
  if (num_seqs < 0) return fail(PKV_EINVAL, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (pkv_status rc = check_shape(dtype, num_heads, head_dim, block_size, num_blocks)) return rc;
  if (max_blocks_per_seq <= 0)
    return fail(PKV_EINVAL, "max_blocks_per_seq must be positive (got %d)", max_blocks_per_seq);
  if (int64_t(max_blocks_per_seq) * block_size > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "table capacity of %lld tokens exceeds int32", (long long)max_blocks_per_seq * block_size);
  if (max_query_len < 0) return fail(PKV_EINVAL, "max_query_len must be >= 0 (got %d)", max_query_len);
  if (!isfinite(scale)) return fail(PKV_EINVAL, "scale must be finite");
  if (num_seqs == 0 || max_query_len == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_tables || !query_start || !context_lens || !out)
    return fail(PKV_EINVAL, "null pointer among q, k_cache, v_cache, block_tables, query_start, context_lens, out");
  if (misaligned(q, 16) || misaligned(k_cache, 16) || misaligned(v_cache, 16) || misaligned(out, 16) ||
      misaligned(block_tables, 4) || misaligned(query_start, 4) || misaligned(context_lens, 4))
    return fail(PKV_EINVAL, "q, k_cache, v_cache and out must be 16-byte aligned, block_tables, query_start and "
                "context_lens 4-byte aligned");
  const int64_t tq = pkv::prefill_tile_queries(dtype);
  const int64_t tiles = (int64_t(max_query_len) + tq - 1) / tq;
  if (num_heads > 65535 || num_seqs > 65535 || tiles > 65535)
    return fail(PKV_EUNSUPPORTED, "grid (%d heads, %lld query tiles, %d sequences) exceeds 65535", num_heads,
                (long long)tiles, num_seqs);
  // 16-bit types launch one 256-thread work-group per (sequence, head, tile),
  // (sequence, head) pairs rounded up to a multiple of 8, in a 1-D grid whose
  // size in threads must fit 32 bits.
  if (dtype != PKV_F32 && ((int64_t(num_heads) * num_seqs + 7) / 8 * 8) * tiles * 256 > int64_t(UINT32_MAX))
    return fail(PKV_EUNSUPPORTED, "grid of %d heads x %d sequences x %lld query tiles is too large", num_heads,
                num_seqs, (long long)tiles);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_checks()) {
    std::vector<int32_t> qs(size_t(num_seqs) + 1), lens(num_seqs), tab(size_t(num_seqs) * max_blocks_per_seq);
    hipError_t e = hipMemcpyAsync(qs.data(), query_start, qs.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(lens.data(), context_lens, lens.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(tab.data(), block_tables, tab.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "PKV_DEBUG copy of metadata");
    for (int32_t i = 0; i < num_seqs; ++i) {
      const int64_t P = int64_t(qs[i + 1]) - qs[i], L = lens[i];
      if (P < 0 || P > max_query_len)
        return fail(PKV_EINVAL, "sequence %d has %lld queries, outside [0, max_query_len = %d]", i, (long long)P,
                    max_query_len);
      if (L < P || L > int64_t(max_blocks_per_seq) * block_size)
        return fail(PKV_EINVAL, "context_lens[%d] = %lld outside [%lld queries, %lld]", i, (long long)L,
                    (long long)P, (long long)max_blocks_per_seq * block_size);
      for (int64_t j = 0; j < (L + block_size - 1) / block_size; ++j) {
        const int32_t b = tab[size_t(i) * max_blocks_per_seq + j];
        if (b < 0 || b >= num_blocks)
          return fail(PKV_EINVAL, "block_tables[%d, %lld] = %d outside [0, %lld)", i, (long long)j, b,
                      (long long)num_blocks);
      }
    }
  }
  pkv::PrefillArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.query_start = query_start;
  a.context_lens = context_lens;
  a.out = out;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.max_query_len = max_query_len;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = pkv::launch_prefill(dtype, head_dim, block_size, a, st);
  if (e != hipSuccess) return hip_fail(e, "paged_attention_prefill launch");
  return ok();
}

namespace {

// Decode, optionally with the newest tokens' K/V appended first (k_new, v_new
// non-null: the fused step).
// With static_scratch the split-context partials go to the library's own
// per-device array (pkv::static_scratch) instead of a caller workspace.
pkv_status decode_common(const void* q, const void* k_new, const void* v_new, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                  int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                  float scale, int32_t dtype, void* out, void* workspace, size_t workspace_bytes,
                  int32_t partition_size, void* stream, bool static_scratch = false) {
  if (num_seqs < 0) return fail(PKV_EINVAL, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (pkv_status rc = check_shape(dtype, num_heads, head_dim, block_size, num_blocks)) return rc;
  if (max_blocks_per_seq <= 0)
    return fail(PKV_EINVAL, "max_blocks_per_seq must be positive (got %d)", max_blocks_per_seq);
  if (int64_t(max_blocks_per_seq) * block_size > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "table capacity of %lld tokens exceeds int32", (long long)max_blocks_per_seq * block_size);
  if (partition_size != PKV_PARTITION_AUTO && (partition_size < 0 || partition_size % block_size != 0))
    return fail(PKV_EINVAL, "partition_size %d must be PKV_PARTITION_AUTO (-1), 0 or a positive multiple of "
                "block_size %d", partition_size, block_size);
  partition_size = resolve_partition(num_seqs, num_heads, max_blocks_per_seq, block_size, partition_size);
  if (!isfinite(scale)) return fail(PKV_EINVAL, "scale must be finite");
  if (num_seqs == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return fail(PKV_EINVAL, "null pointer among q, k_cache, v_cache, block_tables, context_lens, out");
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(PKV_EINVAL, "k_new and v_new must both be given");
  if (misaligned(q, 16) || misaligned(k_cache, 16) || misaligned(v_cache, 16) || misaligned(out, 16) ||
      misaligned(k_new, 16) || misaligned(v_new, 16) || misaligned(workspace, 16) || misaligned(block_tables, 4) ||
      misaligned(context_lens, 4))
    return fail(PKV_EINVAL, "q, k_new, v_new, k_cache, v_cache, out and workspace must be 16-byte aligned, "
                "block_tables and context_lens 4-byte aligned");
  if (num_heads > 65535 || num_seqs > 65535)
    return fail(PKV_EUNSUPPORTED, "num_heads %d / num_seqs %d exceed the grid limit 65535", num_heads, num_seqs);
  const int32_t pb = part_blocks_for(max_blocks_per_seq, block_size, partition_size);
  const int64_t parts = partitions_for(max_blocks_per_seq, pb);
  if (parts > 65535) return fail(PKV_EUNSUPPORTED, "%lld partitions exceed the grid limit 65535", (long long)parts);
  const pkv::WorkspaceLayout wl = pkv::workspace_layout(num_seqs, num_heads, head_dim, parts);
  if (static_scratch && wl.bytes > pkv::kStaticScratchBytes)
    return fail(PKV_EWORKSPACE, "the split needs %zu bytes of scratch, more than the %zu bytes the no-allocation "
                "entry point holds per GPU; use a larger partition_size or paged_attention_decode_step with a "
                "workspace", wl.bytes, pkv::kStaticScratchBytes);
  if (!static_scratch && wl.bytes > 0 && (workspace == nullptr || workspace_bytes < wl.bytes))
    return fail(PKV_EWORKSPACE, "workspace of %zu bytes needed, %zu given%s", wl.bytes, workspace_bytes,
                workspace ? "" : " (null)");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_checks()) {
    std::vector<int32_t> lens(num_seqs), tab(size_t(num_seqs) * max_blocks_per_seq);
    hipError_t e = hipMemcpyAsync(lens.data(), context_lens, lens.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(tab.data(), block_tables, tab.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "PKV_DEBUG copy of metadata");
    for (int32_t i = 0; i < num_seqs; ++i) {
      const int64_t L = lens[i];
      if (L < 0 || L > int64_t(max_blocks_per_seq) * block_size)
        return fail(PKV_EINVAL, "context_lens[%d] = %lld outside [0, %lld]", i, (long long)L,
                    (long long)max_blocks_per_seq * block_size);
      for (int64_t j = 0; j < (L + block_size - 1) / block_size; ++j) {
        const int32_t b = tab[size_t(i) * max_blocks_per_seq + j];
        if (b < 0 || b >= num_blocks)
          return fail(PKV_EINVAL, "block_tables[%d, %lld] = %d outside [0, %lld)", i, (long long)j, b,
                      (long long)num_blocks);
      }
    }
  }
  if (static_scratch && wl.bytes > 0) {            // after validation: the first call on a device sets up
    hipError_t e = pkv::static_scratch(&workspace);
    if (e != hipSuccess) return hip_fail(e, "scratch address of the no-allocation entry point");
  }
  pkv::DecodeArgs a{};
  a.q = q;
  a.k_cache = const_cast<void*>(k_cache);          // written only when k_new is given
  a.v_cache = const_cast<void*>(v_cache);
  a.k_new = k_new;
  a.v_new = v_new;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.ws_m = wl.bytes ? reinterpret_cast<float*>(ws + wl.m_off) : nullptr;
  a.ws_l = wl.bytes ? reinterpret_cast<float*>(ws + wl.l_off) : nullptr;
  a.ws_acc = wl.bytes ? reinterpret_cast<float*>(ws + wl.acc_off) : nullptr;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.part_blocks = pb;
  a.partitions = int32_t(parts);
  a.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = pkv::launch_decode(dtype, head_dim, block_size, a, st);
  if (e != hipSuccess) return hip_fail(e, "paged_attention_decode launch");
  return ok();
}

}  // namespace

extern "C" pkv_status paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                      int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                      float scale, int32_t dtype, void* out, void* workspace,
                                      size_t workspace_bytes, int32_t partition_size, void* stream) {
  return decode_common(q, nullptr, nullptr, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_heads, head_dim, block_size, num_blocks, scale, dtype, out, workspace,
                       workspace_bytes, partition_size, stream);
}

extern "C" pkv_status paged_attention_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                           void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                           int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                           int32_t dtype, void* out, void* workspace, size_t workspace_bytes,
                                           int32_t partition_size, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PKV_EINVAL, "null k_new or v_new");
  return decode_common(q, k_new, v_new, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_heads, head_dim, block_size, num_blocks, scale, dtype, out, workspace,
                       workspace_bytes, partition_size, stream);
}

extern "C" pkv_status paged_attention_decode_step_noalloc(const void* q, const void* k_new, const void* v_new,
                                                   void* k_cache, void* v_cache, const int32_t* block_tables,
                                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                                   int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                                   int32_t block_size, int64_t num_blocks, float scale,
                                                   int32_t dtype, void* out, int32_t partition_size, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PKV_EINVAL, "null k_new or v_new");
  return decode_common(q, k_new, v_new, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_heads, head_dim, block_size, num_blocks, scale, dtype, out, nullptr, 0,
                       partition_size, stream, true);
}
