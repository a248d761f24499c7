// Matrix-core ceiling for the prefill kernel's products (a diagnostic; see
// include/pagedkv_probe.h).  Prefill is a dense contraction and compute-bound
// ("vLLM KV cache and PagedAttention explained", Step 6), so besides the
// matrix cores' published peak the useful yardstick is how fast the same
// product instruction runs on this GPU with nothing else to do: under a long
// run of dense products the shader clock settles below its 2.4 GHz maximum,
// and the published peak assumes the maximum.
//
// Each wave issues iters x 8 products v_mfma_f32_32x32x16 (bf16 or f16, the
// prefill kernel's instruction) into 4 independent accumulators, optionally
// with `valu` vector additions after each product (the way a softmax shares
// the SIMD with the products), and records the shader clock and the 100 MHz
// reference clock around the loop.  All operands are 1, so every product adds
// 16 to each accumulator element and the sums written to `sink` are exact.
#include <hip/hip_runtime.h>

#include <string>
#include <type_traits>

#include "pagedkv.h"
#include "pagedkv_probe.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;     // independent accumulators per wave
constexpr int kPerIter = 8;    // products per loop iteration
constexpr int kThreads = 256;  // 4 wave64: one per SIMD of a compute unit

template <int DT, int VALU>
__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(int32_t iters, float one_value, float* __restrict__ sink,
                                                              uint64_t* __restrict__ clocks) {
  using frag = typename std::conditional<DT == PKV_BF16, bf16x8, f16x8>::type;
  using elem = typename std::conditional<DT == PKV_BF16, __bf16, _Float16>::type;
  frag one;
#pragma unroll
  for (int e = 0; e < 8; ++e) one[e] = static_cast<elem>(one_value);
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = 0.f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kPerIter; ++k) {
      if constexpr (DT == PKV_BF16)
        acc[k % kChains] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(one, one, acc[k % kChains], 0, 0, 0);
      else
        acc[k % kChains] = __builtin_amdgcn_mfma_f32_32x32x16_f16(one, one, acc[k % kChains], 0, 0, 0);
      if constexpr (VALU > 0) {
#pragma unroll
        for (int j = 0; j < VALU; ++j) v[(k * VALU + j) % 16] += one_value;
        // One product, then its vector instructions: keep the interleave.
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, VALU, 0);
      }
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
#pragma unroll
  for (int e = 0; e < 16; ++e) s += v[e];
  sink[int64_t(blockIdx.x) * kThreads + threadIdx.x] = s;
  if (clocks && (threadIdx.x & 63) == 0) {
    const int64_t w = int64_t(blockIdx.x) * (kThreads / 64) + threadIdx.x / 64;
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

template <int DT>
hipError_t launch(int32_t num_groups, int32_t iters, int32_t valu, float* sink, uint64_t* clocks, hipStream_t st) {
  const dim3 grid{unsigned(num_groups)}, block{unsigned(kThreads)};
  switch (valu) {
    case 0: hipLaunchKernelGGL((mfma_probe_kernel<DT, 0>), grid, block, 0, st, iters, 1.f, sink, clocks); break;
    case 4: hipLaunchKernelGGL((mfma_probe_kernel<DT, 4>), grid, block, 0, st, iters, 1.f, sink, clocks); break;
    default: hipLaunchKernelGGL((mfma_probe_kernel<DT, 8>), grid, block, 0, st, iters, 1.f, sink, clocks); break;
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace pkv

extern "C" pkv_status pkv_mfma_probe(int32_t dtype, int32_t num_groups, int32_t iters, int32_t valu, float* sink,
                                     uint64_t* clocks, void* stream) {
  if (dtype != PKV_BF16 && dtype != PKV_F16)
    return pkv::set_error(PKV_EUNSUPPORTED, "dtype must be PKV_BF16 or PKV_F16 (got " + std::to_string(dtype) + ")");
  if (num_groups <= 0 || num_groups > (1 << 20))
    return pkv::set_error(PKV_EINVAL, "num_groups must be in [1, 2^20] (got " + std::to_string(num_groups) + ")");
  if (iters <= 0 || iters > PKV_MFMA_PROBE_MAX_ITERS)
    return pkv::set_error(PKV_EINVAL, "iters must be in [1, " + std::to_string(PKV_MFMA_PROBE_MAX_ITERS) + "] (got " +
                                          std::to_string(iters) + ")");
  if (valu != 0 && valu != 4 && valu != 8)
    return pkv::set_error(PKV_EUNSUPPORTED, "valu must be 0, 4 or 8 (got " + std::to_string(valu) + ")");
  if (!sink) return pkv::set_error(PKV_EINVAL, "null sink");
  if ((reinterpret_cast<uintptr_t>(sink) & 3) || (reinterpret_cast<uintptr_t>(clocks) & 7))
    return pkv::set_error(PKV_EINVAL, "sink must be 4-byte aligned and clocks 8-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == PKV_BF16 ? pkv::launch<PKV_BF16>(num_groups, iters, valu, sink, clocks, st)
                                         : pkv::launch<PKV_F16>(num_groups, iters, valu, sink, clocks, st);
  if (e != hipSuccess) return pkv::set_error(PKV_EHIP, std::string("pkv_mfma_probe launch: ") + hipGetErrorString(e));
  return pkv::set_error(PKV_OK, "");
}
