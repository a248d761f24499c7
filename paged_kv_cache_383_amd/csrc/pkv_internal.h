// Internal interface between the C-ABI front end (api.hip) and the kernel
// launchers (kv_write.hip, decode.hip).  Arguments reaching these functions
// have already been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

#include "pagedkv.h"

namespace pkv {

// Records the calling thread's last status text (read by pkv_last_error) and
// returns `code`.
pkv_status set_error(int code, const std::string& message);

// Split-context workspace: three fp32 arrays, each 256-byte aligned.
//   m    [num_seqs, num_heads, P]      running max of a partition (base-2 logits)
//   l    [num_seqs, num_heads, P]      sum of 2^(s - m) over the partition
//   acc  [num_seqs, num_heads, P, D]   sum of 2^(s - m) * V over the partition
struct WorkspaceLayout {
  size_t m_off, l_off, acc_off, bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WorkspaceLayout workspace_layout(int64_t num_seqs, int64_t num_heads, int64_t head_dim,
                                        int64_t partitions) {
  WorkspaceLayout w{};
  if (partitions <= 1 || num_seqs <= 0) return w;
  const size_t n = size_t(num_seqs) * size_t(num_heads) * size_t(partitions);
  w.m_off = 0;
  w.l_off = align256(n * sizeof(float));
  w.acc_off = w.l_off + align256(n * sizeof(float));
  w.bytes = w.acc_off + align256(n * size_t(head_dim) * sizeof(float));
  return w;
}

struct DecodeArgs {
  const void* q;
  void* k_cache;                 // written only by the fused step (k_new != nullptr)
  void* v_cache;
  const void* k_new;             // [B, H, D] newest tokens' K/V for the fused step, or nullptr
  const void* v_new;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* ws_m;
  float* ws_l;
  float* ws_acc;
  int64_t num_blocks;
  int32_t max_blocks;      // block-table row length
  int32_t num_seqs;
  int32_t num_heads;
  int32_t part_blocks;     // blocks per partition
  int32_t partitions;      // ceil(max_blocks / part_blocks): grid size along partitions
  float scale_log2;        // scale * log2(e): scores are kept as base-2 logits
};

hipError_t launch_decode(int dtype, int head_dim, int block_size, const DecodeArgs& a,
                         hipStream_t stream);

// Split-context scratch of paged_attention_decode_step_noalloc: a device array
// of kStaticScratchBytes that the library holds on every GPU it runs on.
// static_scratch() returns the current device's copy (looked up once per
// device, with that device current; decode_noalloc.hip).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
hipError_t static_scratch(void** ptr);

hipError_t launch_kv_write(int dtype, int head_dim, const void* k, const void* v,
                           const int64_t* slot_mapping, int64_t num_tokens, void* k_cache,
                           void* v_cache, int64_t num_blocks, int32_t num_heads,
                           int32_t block_size, hipStream_t stream);

hipError_t launch_copy_blocks(const int64_t* block_mapping, int64_t num_pairs, void* k_cache, void* v_cache,
                              int64_t num_blocks, int64_t block_bytes, hipStream_t stream);

hipError_t launch_prepare_step(int32_t* block_tables, int32_t width, int32_t* context_lens, int32_t rows,
                               const int32_t* updates, int64_t n_updates, const int32_t* new_lens,
                               int64_t* slot_mapping, int32_t block_size, int64_t num_blocks, hipStream_t stream);

struct PrefillArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* query_start;
  const int32_t* context_lens;
  void* out;
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t max_query_len;
  float scale_log2;
};

// Queries per prefill work-group (the grid's y extent is ceil(max_query_len / this)).
int prefill_tile_queries(int dtype);
hipError_t launch_prefill(int dtype, int head_dim, int block_size, const PrefillArgs& a, hipStream_t stream);

}  // namespace pkv
