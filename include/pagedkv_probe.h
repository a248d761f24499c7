/*
 * pagedkv_probe.h -- diagnostic entry points of libpagedkv.so: an HBM read
 * ceiling for the decode kernel's access pattern, and a matrix-core ceiling
 * for the prefill kernel's products.
 *
 * Decode reads the whole K/V cache once per step and is bound by memory
 * bandwidth ("vLLM KV cache and PagedAttention explained", Step 6: every
 * decode step reads the entire KV cache).  Its fraction of the 8 TB/s HBM
 * peak is one yardstick; this probe gives another, measured on the same GPU:
 * how fast the same kind of loads, with no arithmetic at all, can stream the
 * same kind of tiles.  It is not part of the decode path.
 *
 * Same conventions as pagedkv.h: device pointers owned by the caller, the
 * call is asynchronous on `stream` (a hipStream_t passed as void*), host-side
 * validation first, a non-zero pkv_status (see pagedkv.h) with nothing
 * launched on failure, text in pkv_last_error().
 */
#ifndef PAGEDKV_PROBE_H
#define PAGEDKV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pkv_read_probe -- read tiles of tile_bytes bytes (4096 or 8192) from pool a
 * and, when b is not NULL, the tile at the same index of pool b as well (the
 * decode kernel reads a block's K and V tiles together).
 *
 *   a, b          device pools of pool_tiles tiles each, 16-byte aligned
 *   order         int32 [num_groups * group_tiles]: the tile indices to read,
 *                 or NULL for 0, 1, 2, ... (a sequential stream of num_groups *
 *                 group_tiles tiles).  An entry outside [0, pool_tiles) is
 *                 skipped without a memory access (use -1 to pad).
 *   group_len     int32 [num_groups] or NULL: group g reads only its first
 *                 group_len[g] entries (clamped to [0, group_tiles]), as a decode
 *                 work-group stops at its row's length; NULL = all of them
 *   num_groups    work-groups; group g reads entries g*group_tiles ..
 *                 (g+1)*group_tiles - 1 of the order
 *   group_tiles   entries per work-group (>= 1)
 *   depth         stages in the ring of stage buffers: 2 or 3 with two pools, 2 to 4
 *                 with one (depth - 1 stages of loads in flight while one is folded)
 *   sink          uint32 [num_groups * 8], written: one XOR of the data per
 *                 wave, so that no load can be dropped
 *
 * Work decomposition, as in the decode kernel: 8 wave64 per work-group; a
 * wave works in stages of 8 KiB per pool (two 4 KiB tiles or one 8 KiB tile),
 * wave w taking stages w, w + 8, ... of its group; 16-byte non-temporal
 * buffer loads per lane.  With depth 2 this is the decode kernel's own load
 * depth for 16-bit tiles; deeper rings show what more loads in flight give.  With
 * the decode's own tile order (group = (sequence, head) row, entries =
 * block_tables[s, j] * num_heads + h, padded with -1) this is the decode's
 * gather with the arithmetic removed (with group_len = each row's block count); with a random permutation it is a
 * random-tile read; with order NULL a sequential stream.
 * Bytes read per call = (1 or 2 pools) * tile_bytes * number of valid entries.
 */
pkv_status pkv_read_probe(const void* a, const void* b, int64_t pool_tiles, int32_t tile_bytes, const int32_t* order,
                          const int32_t* group_len, int32_t num_groups, int32_t group_tiles, int32_t depth,
                          uint32_t* sink, void* stream);

/*
 * pkv_mfma_probe -- the matrix-core ceiling for the prefill kernel's products.
 * Prefill is the one dense contraction of the path and is compute-bound
 * ("vLLM KV cache and PagedAttention explained", Step 6); the published peak
 * assumes the 2.4 GHz maximum clock, which a long run of dense products does
 * not keep.  This runs the prefill kernel's product instruction with nothing
 * else to do and reports what this GPU sustains.  Not part of the prefill.
 *
 *   dtype        PKV_BF16 or PKV_F16: v_mfma_f32_32x32x16 of that type
 *   num_groups   work-groups of 4 wave64 (one per SIMD of a compute unit);
 *                num_groups = k x the number of compute units gives k waves per SIMD
 *   iters        loop iterations per wave, 8 products each into 4 independent
 *                accumulators; 1 .. PKV_MFMA_PROBE_MAX_ITERS
 *   valu         0, 4 or 8 vector additions after each product (the way a
 *                softmax shares a SIMD with the products)
 *   sink         float [num_groups * 256], written: every operand is 1, so lane
 *                value = 2048 * iters + 8 * valu * iters, exactly
 *   clocks       uint64 [num_groups * 4 * 2] or NULL: per wave (index
 *                group * 4 + wave), the shader-clock cycles and the 100 MHz
 *                reference-clock ticks between its first and last product;
 *                cycles / ticks x 100 MHz is the shader clock over the run
 *
 * Products per call = num_groups * 4 * iters * 8, each 32 * 32 * 16 * 2 flops.
 */
#define PKV_MFMA_PROBE_MAX_ITERS 8000
pkv_status pkv_mfma_probe(int32_t dtype, int32_t num_groups, int32_t iters, int32_t valu, float* sink,
                          uint64_t* clocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_PROBE_H */
