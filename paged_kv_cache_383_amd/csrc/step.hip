// Decode-step metadata on the device: apply a plan's block-table updates and
// context lengths, then derive each row's slot mapping.
//
// "PagedAttention" card (llm-engineer.pages.dev), "vLLM에서의 위치": the GPU
// worker keeps each request's block table and the slot mapping as device
// tensors.  "vLLM KV cache and PagedAttention explained" (hrletsgo.me), Step 6:
// a decode step stores its new token's K/V in the next slot of the sequence's
// last block, so the slot of row r is
//   block_tables[r, (L - 1) / bs] * bs + (L - 1) % bs,   L = context_lens[r],
// and -1 (no write) for an idle row (L = 0).
//
// One work-group does everything: the work is a few hundred entries, and a
// single group can order the table writes before the slot reads with one
// barrier.  Entries outside the arrays are skipped, and a row whose length or
// block id is out of range gets slot -1, so broken metadata never makes the
// kernel touch memory outside its arrays.
#include "pagedkv.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 1024;

__global__ __launch_bounds__(kThreads) void prepare_step_kernel(
    int32_t* __restrict__ block_tables, int32_t width, int32_t* __restrict__ context_lens, int32_t rows,
    const int32_t* __restrict__ updates, int64_t n_updates, const int32_t* __restrict__ new_lens,
    int64_t* __restrict__ slot_mapping, int32_t block_size, int64_t num_blocks) {
  for (int64_t u = threadIdx.x; u < n_updates; u += kThreads) {
    const int32_t r = updates[3 * u], c = updates[3 * u + 1], b = updates[3 * u + 2];
    if (r >= 0 && r < rows && c >= 0 && c < width) block_tables[int64_t(r) * width + c] = b;
  }
  if (new_lens)
    for (int32_t r = threadIdx.x; r < rows; r += kThreads) context_lens[r] = new_lens[r];
  __syncthreads();
  if (!slot_mapping) return;
  for (int32_t r = threadIdx.x; r < rows; r += kThreads) {
    const int32_t L = context_lens[r];
    int64_t slot = -1;
    if (L > 0 && (int64_t(L) - 1) / block_size < width) {
      const int32_t b = block_tables[int64_t(r) * width + (L - 1) / block_size];
      if (b >= 0 && b < num_blocks) slot = int64_t(b) * block_size + (L - 1) % block_size;
    }
    slot_mapping[r] = slot;
  }
}

}  // namespace

hipError_t launch_prepare_step(int32_t* block_tables, int32_t width, int32_t* context_lens, int32_t rows,
                               const int32_t* updates, int64_t n_updates, const int32_t* new_lens,
                               int64_t* slot_mapping, int32_t block_size, int64_t num_blocks, hipStream_t stream) {
  hipLaunchKernelGGL(prepare_step_kernel, dim3(1), dim3(kThreads), 0, stream, block_tables, width, context_lens,
                     rows, updates, n_updates, new_lens, slot_mapping, block_size, num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
