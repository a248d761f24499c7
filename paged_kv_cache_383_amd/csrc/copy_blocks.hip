// Block copy for copy-on-write: physical block dst of both pools receives the
// contents of block src.
//
// "vLLM KV cache and PagedAttention explained" (hrletsgo.me), Step 9: when a
// request must write into a block it shares with others, the block is first
// copied into a new physical block that only the writer's table points to.
// The unit of sharing is the whole physical block: every head and slot of K
// and of V, i.e. num_heads * block_size * head_dim elements in one contiguous
// run per pool ([Block, Head, Block_Size, Head_D] layout, "vLLM의
// PagedAttention 아키텍처와 GPU 메모리 최적화 원리", velog, section 4).
//
// One work-group copies a 16 KiB chunk of one block of one pool: each lane
// moves four 16-byte pieces, loads first, then stores, so a wave has 4 KiB in
// flight.  Grid x runs over the chunks of K's block then V's, grid y over
// pairs (striding when there are more than 65535).  A pair whose ids fall
// outside the pool is skipped, so a broken mapping never touches memory
// outside the pools.
#include "pagedkv.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kChunkVecs = int64_t(kThreads) * kUnroll;     // 16 KiB

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    const int64_t* __restrict__ mapping, int64_t num_pairs, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, int64_t num_blocks, int64_t vecs_per_block, int64_t chunks_per_block) {
  const int64_t chunk = blockIdx.x % chunks_per_block;
  u32x4* pool = blockIdx.x < chunks_per_block ? k_cache : v_cache;
  for (int64_t pair = blockIdx.y; pair < num_pairs; pair += gridDim.y) {
    const int64_t src = mapping[2 * pair];
    const int64_t dst = mapping[2 * pair + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
    const u32x4* from = pool + src * vecs_per_block;
    u32x4* to = pool + dst * vecs_per_block;
    const int64_t base = chunk * kChunkVecs + threadIdx.x;
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads;
      if (i < vecs_per_block) x[u] = __builtin_nontemporal_load(from + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads;
      if (i < vecs_per_block) to[i] = x[u];
    }
  }
}

}  // namespace

hipError_t launch_copy_blocks(const int64_t* block_mapping, int64_t num_pairs, void* k_cache, void* v_cache,
                              int64_t num_blocks, int64_t block_bytes, hipStream_t stream) {
  const int64_t vecs = block_bytes / 16;
  const int64_t chunks = (vecs + kChunkVecs - 1) / kChunkVecs;
  const dim3 grid(unsigned(2 * chunks), unsigned(num_pairs < 65535 ? num_pairs : 65535));
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kThreads), 0, stream, block_mapping, num_pairs,
                     static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), num_blocks, vecs, chunks);
  return hipGetLastError();
}

}  // namespace pkv
