// HBM read ceiling for the decode kernel's access pattern (a diagnostic; see
// include/pagedkv_probe.h).  Decode reads the whole K/V cache every step and
// is memory-bound ("vLLM KV cache and PagedAttention explained", Step 6), so
// the useful yardstick besides the HBM peak is how fast the same loads can
// stream the same tiles on the same GPU with nothing else to do.
//
// The kernel mirrors the decode kernel's memory side and drops its
// arithmetic: 8 wave64 per work-group, stages of 8 KiB per pool, wave w
// taking stages w, w + 8, ..., a buffer resource per tile (an invalid tile
// gets an empty one: its loads return zeros and touch nothing), 16-byte
// non-temporal loads per lane, and a ring of `depth` stage buffers in
// registers so that depth - 1 stages' loads are in flight while one is
// folded (the decode kernel's 16-bit kernels hold two stages).  Folding is an XOR of the loaded words, written out once per wave.
// The loop body has no branch (the tile index is a select), so it is one basic
// block and every wait in it leaves a whole stage in flight; with a branch in
// the index the register allocator moved one stage buffer at the back edge,
// waiting for its loads there (checked in the gfx950 assembly).
#include <hip/hip_runtime.h>

#include "pagedkv.h"
#include "pagedkv_probe.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kStageBytes = 8192;              // per pool, as the decode kernel's 16-bit stages
constexpr int kLoadsPerStage = kStageBytes / 1024;
constexpr int kNonTemporal = 2;                // buffer-load aux bit the decode kernel uses for K/V tiles
constexpr int kBufferWord3 = 0x00020000;       // raw buffer resource: 32-bit data format, no swizzle

template <int TILE, bool TWO, bool ORDERED, int DEPTH>
__global__ __launch_bounds__(64 * kWaves) void read_probe_kernel(const char* __restrict__ a,
                                                                 const char* __restrict__ b, int64_t pool_tiles,
                                                                 const int32_t* __restrict__ order,
                                                                 const int32_t* __restrict__ group_len,
                                                                 int32_t group_tiles, uint32_t* __restrict__ sink) {
  constexpr int kTps = kStageBytes / TILE;      // tiles per stage
  constexpr int kLoadsPerTile = TILE / 1024;    // wave-wide 1 KiB loads per tile
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t e0 = int64_t(blockIdx.x) * group_tiles;
  // Entries this group reads: its first group_len[g] (clamped to [0, group_tiles]), or all of them.
  const int n_entries = group_len ? min(max(group_len[blockIdx.x], 0), group_tiles) : group_tiles;
  const int units = (n_entries + kTps - 1) / kTps;
  const int n_my = units > wave ? (units - wave + kWaves - 1) / kWaves : 0;

  // Tile index of entry u of this wave's stage i, or -1 (past the group, or an invalid entry).  Selects
  // only, no branch: the loop body stays one basic block.
  auto tile_at = [&](int i, int u) -> int64_t {
    const int k = (wave + kWaves * i) * kTps + u;
    const bool live = i < n_my && k < n_entries;
    const int64_t e = e0 + (live ? k : 0);
    int64_t id = e;
    if constexpr (ORDERED) id = __builtin_amdgcn_readfirstlane(order[e]);
    return (live && id >= 0 && id < pool_tiles) ? id : -1;
  };
  auto issue = [&](u32x4* ba, u32x4* bb, int i) {
#pragma unroll
    for (int u = 0; u < kTps; ++u) {
      const int64_t id = tile_at(i, u);
      const int nrec = id >= 0 ? TILE : 0;
      const int64_t off = (id >= 0 ? id : 0) * TILE;
      const __amdgpu_buffer_rsrc_t ra =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a + off), 0, nrec, kBufferWord3);
#pragma unroll
      for (int t = 0; t < kLoadsPerTile; ++t)
        ba[u * kLoadsPerTile + t] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (t * 64 + lane) * 16, 0, kNonTemporal));
      if constexpr (TWO) {
        const __amdgpu_buffer_rsrc_t rb =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(b + off), 0, nrec, kBufferWord3);
#pragma unroll
        for (int t = 0; t < kLoadsPerTile; ++t)
          bb[u * kLoadsPerTile + t] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (t * 64 + lane) * 16, 0, kNonTemporal));
      }
    }
  };
  uint32_t x = 0;
  auto fold = [&](const u32x4* ba, const u32x4* bb) {
#pragma unroll
    for (int i = 0; i < kLoadsPerStage; ++i) {
      x ^= ba[i].x ^ ba[i].y ^ ba[i].z ^ ba[i].w;
      if constexpr (TWO) x ^= bb[i].x ^ bb[i].y ^ bb[i].z ^ bb[i].w;
    }
  };

  // Same loop shape as the decode kernel: step s issues stage s into buffer
  // s % DEPTH and folds stage s - (DEPTH - 1); the first steps fold zeroed
  // buffers and the last ones issue empty loads.
  if (n_my > 0) {
    u32x4 ba[DEPTH][kLoadsPerStage], bb[TWO ? DEPTH : 1][kLoadsPerStage];
#pragma unroll
    for (int r = 0; r < DEPTH; ++r)
#pragma unroll
      for (int i = 0; i < kLoadsPerStage; ++i) {
        ba[r][i] = u32x4{0u, 0u, 0u, 0u};
        if constexpr (TWO) bb[r][i] = u32x4{0u, 0u, 0u, 0u};
      }
    for (int i = 0; i < n_my + DEPTH - 1; i += DEPTH) {
#pragma unroll
      for (int r = 0; r < DEPTH; ++r) {
        issue(ba[r], bb[TWO ? r : 0], i + r);
        __builtin_amdgcn_sched_barrier(0);
        fold(ba[(r + 1) % DEPTH], bb[TWO ? (r + 1) % DEPTH : 0]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), m));
  if (lane == 0) sink[int64_t(blockIdx.x) * kWaves + wave] = x;
}

template <int TILE, bool TWO, bool ORDERED>
hipError_t launch_depth(int depth, const void* a, const void* b, int64_t pool_tiles, const int32_t* order,
                        const int32_t* group_len, int32_t num_groups, int32_t group_tiles, uint32_t* sink,
                        hipStream_t stream) {
  // Two pools stop at depth 3: a fourth pair of stage buffers does not fit the registers.
  void (*kernel)(const char*, const char*, int64_t, const int32_t*, const int32_t*, int32_t, uint32_t*) =
      depth == 2 ? read_probe_kernel<TILE, TWO, ORDERED, 2> : read_probe_kernel<TILE, TWO, ORDERED, 3>;
  if constexpr (!TWO) {
    if (depth == 4) kernel = read_probe_kernel<TILE, TWO, ORDERED, 4>;
  }
  hipLaunchKernelGGL(kernel, dim3(unsigned(num_groups)), dim3(64 * kWaves), 0, stream,
                     static_cast<const char*>(a), static_cast<const char*>(b), pool_tiles, order, group_len,
                     group_tiles, sink);
  return hipGetLastError();
}

template <int TILE>
hipError_t launch_tile(int depth, const void* a, const void* b, int64_t pool_tiles, const int32_t* order,
                       const int32_t* group_len, int32_t num_groups, int32_t group_tiles, uint32_t* sink,
                       hipStream_t stream) {
  if (b != nullptr)
    return order != nullptr ? launch_depth<TILE, true, true>(depth, a, b, pool_tiles, order, group_len, num_groups,
                                                              group_tiles, sink, stream)
                            : launch_depth<TILE, true, false>(depth, a, b, pool_tiles, order, group_len, num_groups,
                                                               group_tiles, sink, stream);
  return order != nullptr ? launch_depth<TILE, false, true>(depth, a, b, pool_tiles, order, group_len, num_groups,
                                                             group_tiles, sink, stream)
                          : launch_depth<TILE, false, false>(depth, a, b, pool_tiles, order, group_len, num_groups,
                                                              group_tiles, sink, stream);
}

}  // namespace
}  // namespace pkv

extern "C" pkv_status pkv_read_probe(const void* a, const void* b, int64_t pool_tiles, int32_t tile_bytes,
                                     const int32_t* order, const int32_t* group_len, int32_t num_groups,
                                     int32_t group_tiles, int32_t depth, uint32_t* sink, void* stream) {
  const auto aligned = [](const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; };
  if (tile_bytes != 4096 && tile_bytes != 8192)
    return pkv::set_error(PKV_EUNSUPPORTED, "tile_bytes must be 4096 or 8192 (got " + std::to_string(tile_bytes) + ")");
  if (pool_tiles <= 0 || num_groups <= 0 || group_tiles <= 0)
    return pkv::set_error(PKV_EINVAL, "pool_tiles, num_groups and group_tiles must be positive");
  if (int64_t(num_groups) * group_tiles > (int64_t(1) << 40) || pool_tiles > (int64_t(1) << 40) / tile_bytes)
    return pkv::set_error(PKV_EINVAL, "probe sizes out of range");
  if (!a || !sink) return pkv::set_error(PKV_EINVAL, "null pool a or sink");
  if (depth < 2 || depth > (b ? 3 : 4))
    return pkv::set_error(PKV_EUNSUPPORTED, "depth must be 2 or 3 with two pools, 2 to 4 with one (got " +
                                                std::to_string(depth) + ")");
  if (!aligned(a, 16) || (b && !aligned(b, 16)) || (order && !aligned(order, 4)) || (group_len && !aligned(group_len, 4)) ||
      !aligned(sink, 4))
    return pkv::set_error(PKV_EINVAL, "pools must be 16-byte aligned, order, group_len and sink 4-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e =
      tile_bytes == 4096
          ? pkv::launch_tile<4096>(depth, a, b, pool_tiles, order, group_len, num_groups, group_tiles, sink, st)
          : pkv::launch_tile<8192>(depth, a, b, pool_tiles, order, group_len, num_groups, group_tiles, sink, st);
  if (e != hipSuccess) return pkv::set_error(PKV_EHIP, std::string("pkv_read_probe launch: ") + hipGetErrorString(e));
  return pkv::set_error(PKV_OK, "");
}
