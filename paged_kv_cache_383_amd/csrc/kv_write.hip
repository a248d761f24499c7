// Slot-mapping write: each new token's K and V rows go to their cache slot.
//
// "vLLM KV cache and PagedAttention explained" (hrletsgo.me), Step 6: after a
// decode step the new token's K/V is appended in the next slot of the
// sequence's block ("slot 6 of block 42"); "PagedAttention" card, section
// "vLLM에서의 위치": the worker hands the kernel a slot mapping.
//
// One lane moves one 16-byte piece of a (token, head) row for both K and V.
// A row is head_dim * elem bytes (128 or 256 B), i.e. 8 or 16 lanes, so every
// wave reads and writes whole contiguous rows.  The copy is of stored bits,
// hence exact for every element type.
#include "pkv_internal.h"
#include "pagedkv.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void kv_write_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const int64_t* __restrict__ slot_mapping, int64_t total_vecs, int32_t vecs_per_token,
    int32_t vecs_per_row, u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
    int64_t num_blocks, int32_t num_heads, int32_t block_size) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total_vecs) return;
  const int64_t t = idx / vecs_per_token;
  const int32_t rem = int32_t(idx - t * vecs_per_token);
  const int32_t h = rem / vecs_per_row;
  const int32_t c = rem - h * vecs_per_row;
  const int64_t slot = slot_mapping[t];
  if (slot < 0) return;                       // padding: no write
  const int64_t blk = slot / block_size;
  const int32_t off = int32_t(slot - blk * block_size);
  if (blk >= num_blocks) return;              // broken caller contract: never write out of bounds
  const int64_t dst = ((blk * num_heads + h) * block_size + off) * vecs_per_row + c;
  k_cache[dst] = k[idx];
  v_cache[dst] = v[idx];
}

}  // namespace

hipError_t launch_kv_write(int dtype, int head_dim, const void* k, const void* v,
                           const int64_t* slot_mapping, int64_t num_tokens, void* k_cache,
                           void* v_cache, int64_t num_blocks, int32_t num_heads,
                           int32_t block_size, hipStream_t stream) {
  const int elem = dtype == PKV_F32 ? 4 : 2;
  const int32_t vecs_per_row = head_dim * elem / 16;
  const int32_t vecs_per_token = vecs_per_row * num_heads;
  const int64_t total = num_tokens * vecs_per_token;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(kv_write_kernel, dim3(unsigned(blocks)), dim3(threads), 0, stream,
                     static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), slot_mapping,
                     total, vecs_per_token, vecs_per_row, static_cast<u32x4*>(k_cache),
                     static_cast<u32x4*>(v_cache), num_blocks, num_heads, block_size);
  return hipGetLastError();
}

}  // namespace pkv
