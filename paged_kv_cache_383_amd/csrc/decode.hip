// Paged-attention decode for gfx950: one query token per sequence attends
// over its K/V cache, read in place through the sequence's block table.
//
// What is computed ("vLLM KV cache and PagedAttention explained", hrletsgo.me,
// Appendix: The Attention Score Formula): out = softmax(q K^T * scale) V over
// the sequence's first L cached tokens, evaluated by walking the block table
// one block at a time, scoring the block's keys, updating a running softmax
// normalisation and accumulating the weighted values.  Blocks are read where
// they are, never compacted ("PagedAttention" card, section "Kernel은 무엇이
// 달라지는가").  Long contexts are cut into partitions that are reduced
// independently and merged by log-sum-exp weights (the card names this
// FlashDecoding in "헷갈리기 쉬운 구분").
//
// Work decomposition.  One work-group of W wave64s (W = 8 for 16-token
// blocks, 4 for 32-token blocks and for split partitions of at most 64
// 16-token blocks) per (head, partition, sequence); the grid's
// fastest index is the head, so work-groups running together read
// neighbouring (block, head) tiles of the same physical blocks.  A wave works
// in stages of TPS consecutive blocks (one 32-token or two 16-token bf16/fp16
// tiles: 8 KiB of K and 8 KiB of V); wave w of a partition takes stages w,
// w+W, w+2W, ...
//
// Data movement.  A (block, head) tile of K is block_size * head_dim elements
// in one contiguous run ("vLLM의 PagedAttention 아키텍처와 GPU 메모리 최적화 원리",
// velog, section 4 layout).  A token row is 256 B for every supported
// shape except 16-bit head_dim 64 (128 B), so a wave-wide 16 B-per-lane load
// moves 1 KiB = 4 whole rows, perfectly coalesced.  Each lane keeps the 16 B
// it loaded and uses them itself (its q slice is the same 16 B column), so
// tiles go straight from HBM to VGPRs: there is no cross-lane reuse for an LDS
// round trip to serve.  Loads use a buffer resource sized to the tile's valid
// rows: rows past the context end (and the whole tile of an invalid block id)
// read as zero without touching memory.  A ring of 2 or 3 stage buffers per
// wave keeps the next stages' K and V loads in flight while one is consumed.
//
// Arithmetic.  q.k uses the packed dot2 instructions for 16-bit types (exact
// products, fp32 sums) and fp32 FMA for fp32; each row's partial dots are
// summed across its 8/16/32 lanes with DPP.  The 16 lanes of a row then hold
// identical scores, so every token row of a wave (4 per 1 KiB load) keeps its own
// running (max, sum, acc) state in registers with no cross-row traffic in the
// loop; rows and waves are merged once at the end through LDS.  Scores are
// base-2 logits (scale * log2 e folded in) so exp is a single v_exp_f32.
#include <hip/hip_fp16.h>

#include "pagedkv.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Cache policy of the K/V tile loads (the buffer-load aux operand).  Every
// tile is read exactly once per call, so the loads are marked non-temporal
// (nt = bit 1 on gfx950): on MI355X this streams the cache through L2 and
// Infinity Cache without displacing reusable lines, and measured 10-12 %
// faster than the default policy on every configuration.
#ifndef PKV_KV_LOAD_POLICY
#define PKV_KV_LOAD_POLICY 2
#endif
constexpr int kLoadPolicy = PKV_KV_LOAD_POLICY;

// Waves per work-group: 8 for 16-token blocks, 4 for 32-token blocks (twice
// the registers per stage).
template <int BS>
constexpr int waves_for() {
  return BS == 16 ? 8 : 4;
}
// Split partitions of at most this many blocks run 4-wave work-groups (see
// launch_typed).
constexpr int kSmallPartitionBlocks = 64;
// Running max before any token is seen.  Finite, so 2^(m - m') is defined
// while a row has seen only masked tokens; any real score exceeds it.
constexpr float kEmptyMax = -3.0e38f;
// Word 3 of a gfx9 raw buffer resource: 32-bit data format, no swizzle.
constexpr int kBufferWord3 = 0x00020000;

template <int DT>
struct Elem {
  static constexpr int kBytes = (DT == PKV_F32) ? 4 : 2;
};

// Blocks loaded per pipeline stage: enough (block, head) tiles for 8 KiB of K
// (and 8 KiB of V) per wave, so a bf16 stage of 16-token blocks takes two
// tiles and moves as much as one 32-token tile does.
constexpr int kStageBytes = 8192;
template <int DT, int D, int BS>
constexpr int tiles_for() {
  constexpr int tile = BS * D * Elem<DT>::kBytes;
  return tile >= kStageBytes ? 1 : kStageBytes / tile;
}
// Pipeline depth: stages in flight per wave.  For 16-bit types, three
// single-tile stages or two double-tile ones keep 16 KiB of loads outstanding
// per wave within the register budget (measured: 3 beats 2 for 32-token fp16
// tiles by 3 %; two double-tile stages beat three single ones for 16-token
// bf16 tiles).  fp32 tiles are twice as large: two stages.
template <int DT, int TPS>
constexpr int stages_for() {
  return (DT == PKV_F32 || TPS > 1) ? 2 : 3;
}

template <int DT, int D, int BS, int WAVES>
struct Geo {
  static constexpr int kBytes = Elem<DT>::kBytes;
  static constexpr int kEpl = 16 / kBytes;       // elements per lane per 16-byte load
  static constexpr int kLpr = D / kEpl;          // lanes per token row
  static constexpr int kRpl = 64 / kLpr;         // token rows per wave-wide load
  static constexpr int kLoads = BS / kRpl;       // wave-wide loads per K (or V) tile
  static constexpr int kRowBytes = D * kBytes;
  static constexpr int kTileBytes = BS * kRowBytes;
  static constexpr int kWaves = WAVES;
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int kStates = WAVES * kRpl;    // softmax states merged per work-group
  static_assert(kLpr >= 8 && kLpr <= 32 && 64 % kLpr == 0, "row must span 8..32 lanes");
  static_assert(BS % kRpl == 0, "block must hold whole wave-wide loads");
};

// ---- cross-lane sums (DPP within a 16-lane row; ds_swizzle-free) ----------
constexpr int kDppQuad1032 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuad2301 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;   // lane i <- lane 15 - i
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7 - i, within each 8

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the LPR lanes of a token row; every lane of the row gets the same
// bits (each step adds a value and its partner's, in either order).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<kDppQuad1032>(x);
  x += dpp<kDppQuad2301>(x);
  x += dpp<kDppRowHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

// ---- element helpers --------------------------------------------------------
template <typename T>
__device__ __forceinline__ T bits_as(unsigned int u) {
  return __builtin_bit_cast(T, u);
}

// Partial dot product of the lane's 16-byte q column with a 16-byte K piece.
template <int DT>
__device__ __forceinline__ float dot16(const u32x4& q, const u32x4& k) {
  if constexpr (DT == PKV_BF16) {
    float a = __builtin_amdgcn_fdot2_f32_bf16(bits_as<bf16x2>(q.x), bits_as<bf16x2>(k.x), 0.f, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(bits_as<bf16x2>(q.y), bits_as<bf16x2>(k.y), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(bits_as<bf16x2>(q.z), bits_as<bf16x2>(k.z), a, false);
    return __builtin_amdgcn_fdot2_f32_bf16(bits_as<bf16x2>(q.w), bits_as<bf16x2>(k.w), a, false);
  } else if constexpr (DT == PKV_F16) {
    float a = __builtin_amdgcn_fdot2(bits_as<f16x2>(q.x), bits_as<f16x2>(k.x), 0.f, false);
    a = __builtin_amdgcn_fdot2(bits_as<f16x2>(q.y), bits_as<f16x2>(k.y), a, false);
    a = __builtin_amdgcn_fdot2(bits_as<f16x2>(q.z), bits_as<f16x2>(k.z), a, false);
    return __builtin_amdgcn_fdot2(bits_as<f16x2>(q.w), bits_as<f16x2>(k.w), a, false);
  } else {
    float a = __uint_as_float(q.x) * __uint_as_float(k.x);
    a = __builtin_fmaf(__uint_as_float(q.y), __uint_as_float(k.y), a);
    a = __builtin_fmaf(__uint_as_float(q.z), __uint_as_float(k.z), a);
    return __builtin_fmaf(__uint_as_float(q.w), __uint_as_float(k.w), a);
  }
}

// acc[0 .. 16/elem) += p * (16-byte V piece)
template <int DT>
__device__ __forceinline__ void axpy16(float p, const u32x4& v, float* acc) {
  const unsigned int w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == PKV_BF16) {
      acc[2 * i] = __builtin_fmaf(p, __uint_as_float(w[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = __builtin_fmaf(p, __uint_as_float(w[i] & 0xFFFF0000u), acc[2 * i + 1]);
    } else if constexpr (DT == PKV_F16) {
      const f16x2 h = bits_as<f16x2>(w[i]);
      acc[2 * i] = __builtin_fmaf(p, float(h.x), acc[2 * i]);
      acc[2 * i + 1] = __builtin_fmaf(p, float(h.y), acc[2 * i + 1]);
    } else {
      acc[i] = __builtin_fmaf(p, __uint_as_float(w[i]), acc[i]);
    }
  }
}

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float x) {
  unsigned int u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;   // NaN stays a quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<unsigned short>(u >> 16);
}

template <int DT>
__device__ __forceinline__ void store_elem(void* base, int64_t i, float x) {
  if constexpr (DT == PKV_F32) {
    static_cast<float*>(base)[i] = x;
  } else if constexpr (DT == PKV_F16) {
    static_cast<unsigned short*>(base)[i] = __half_as_ushort(__float2half(x));
  } else {
    static_cast<unsigned short*>(base)[i] = f32_to_bf16_rne(x);
  }
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bool context_ok(int32_t L, int32_t cap) { return L >= 0 && L <= cap; }

template <int DT, int D, int BS, int WAVES, int TPS, int NST, bool FUSED>
__global__ __launch_bounds__(64 * WAVES) void decode_partition_kernel(
    const void* __restrict__ q, char* __restrict__ k_cache, char* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    void* __restrict__ out, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_acc, int64_t num_blocks, int32_t max_blocks, int32_t part_blocks,
    int32_t partitions, float scale_log2, const char* __restrict__ k_new, const char* __restrict__ v_new) {
  using G = Geo<DT, D, BS, WAVES>;
  constexpr int kWaves = WAVES;
  const int h = blockIdx.x;
  const int p = blockIdx.y;
  const int s = blockIdx.z;
  const int H = gridDim.x;
  const int64_t row = int64_t(s) * H + h;                 // (sequence, head) row of q / out
  const int32_t L = context_lens[s];

  if (L == 0 || !context_ok(L, max_blocks * BS)) {       // empty row, or a broken contract
    if (p == 0 && threadIdx.x < D) store_elem<DT>(out, row * D + threadIdx.x, L == 0 ? 0.f : __builtin_nanf(""));
    return;
  }
  const int nb = (L + BS - 1) / BS;
  const int parts = (nb + part_blocks - 1) / part_blocks;
  if (p >= parts) return;
  const int j0 = p * part_blocks;
  const int j1 = min(j0 + part_blocks, nb);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int r = lane / G::kLpr;                           // token row within a wave-wide load
  const int c = lane % G::kLpr;                           // 16-byte column within the row

  // Decode step with the append fused in (k_new given).  The newest token,
  // position L - 1, goes to its slot of the sequence's last block ("vLLM KV
  // cache and PagedAttention explained", Step 6: the decode token's K/V goes
  // to the next slot of the sequence's last block).  Only one wave of one
  // work-group per (sequence, head) reads that block: the wave of the last
  // partition whose stages hold block nb - 1.  That wave stores the row here,
  // before its loop (lanes of row 0 of a wave-wide load move the K row, lanes
  // of row 1 the V row; every shape has at least 2 rows), and waits for the
  // store only right before it issues the loads of stage i_new, the one
  // holding that block (see await_newest): in all but the shortest rows the
  // store has long completed by then.  The loop itself is the plain decode's,
  // with nothing held across it, so the fused kernel needs no more registers
  // than the plain one.  The stage then reads the stored bits, exactly what a
  // write followed by a decode reads.
  int i_new = -1;                                         // stage index holding the newest row (owner wave)
  if (FUSED && p == parts - 1) {
    const int unit_new = (nb - 1 - j0) / TPS;
    if (wave == unit_new % kWaves) {
      i_new = unit_new / kWaves;
      const int32_t bl = block_tables[int64_t(s) * max_blocks + (L - 1) / BS];
      if (static_cast<uint64_t>(static_cast<int64_t>(bl)) < static_cast<uint64_t>(num_blocks) && r < 2) {
        const int64_t src = row * G::kRowBytes + 16 * c;
        const int64_t dst = ((int64_t(bl) * H + h) * BS + (L - 1) % BS) * G::kRowBytes + 16 * c;
        const char* from = r == 0 ? k_new : v_new;
        char* to = r == 0 ? k_cache : v_cache;
        *reinterpret_cast<u32x4*>(to + dst) = *reinterpret_cast<const u32x4*>(from + src);
      }
    }
  }

  const u32x4 qv = *reinterpret_cast<const u32x4*>(static_cast<const char*>(q) +
                                                   (row * D + c * G::kEpl) * G::kBytes);

  // This wave's stages: stage i covers the TPS consecutive logical blocks
  // j0 + (wave + kWaves * i) * TPS + u, u < TPS (blocks at or past j1 are empty).
  const int span = j1 - j0;
  const int units = (span + TPS - 1) / TPS;
  const int n_my = units > wave ? (units - wave + kWaves - 1) / kWaves : 0;
  const int32_t* trow = block_tables + int64_t(s) * max_blocks;

  float m = kEmptyMax, l = 0.f;
  float acc[G::kEpl];
#pragma unroll
  for (int e = 0; e < G::kEpl; ++e) acc[e] = 0.f;
  bool bad = false;

  auto first_block = [&](int i) { return j0 + (wave + kWaves * i) * TPS; };
  // Physical ids of stage i's blocks (entries past the span are not read).
  auto table_at = [&](int i, int32_t* ids) {
#pragma unroll
    for (int u = 0; u < TPS; ++u) {
      const int j = first_block(i) + u;
      ids[u] = (i < n_my && j < j1) ? __builtin_amdgcn_readfirstlane(trow[j]) : 0;
    }
  };

  // Issue the loads of stage i into (kb, vb).  A block past the stage's live
  // range gets an empty resource: its loads return zeros and touch nothing.
  auto issue = [&](u32x4* kb, u32x4* vb, int i, const int32_t* ids) {
#pragma unroll
    for (int u = 0; u < TPS; ++u) {
      const int j = first_block(i) + u;
      const bool live = i < n_my && j < j1;
      const int ntok = min(L - j * BS, BS);
      const bool id_ok = static_cast<uint64_t>(static_cast<int64_t>(ids[u])) < static_cast<uint64_t>(num_blocks);
      bad = bad || (live && !id_ok);
      const int nrec = (live && id_ok) ? ntok * G::kRowBytes : 0;
      const int64_t tile = (int64_t(id_ok ? ids[u] : 0) * H + h) * G::kTileBytes;
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(k_cache + tile), 0, nrec, kBufferWord3);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(v_cache + tile), 0, nrec, kBufferWord3);
#pragma unroll
      for (int t = 0; t < G::kLoads; ++t)
        kb[u * G::kLoads + t] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (t * 64 + lane) * 16, 0, kLoadPolicy));
#pragma unroll
      for (int t = 0; t < G::kLoads; ++t)
        vb[u * G::kLoads + t] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (t * 64 + lane) * 16, 0, kLoadPolicy));
    }
  };

  // Fold stage i into the row's running softmax state.
  constexpr int kRows = TPS * G::kLoads;                  // token rows per lane per stage
  auto consume = [&](const u32x4* kb, const u32x4* vb, int i) {
    float sc[kRows];
    float bm = kEmptyMax;
#pragma unroll
    for (int u = 0; u < TPS; ++u) {
      const int j = first_block(i) + u;
      const int ntok = (i >= 0 && i < n_my && j < j1) ? L - j * BS : 0;   // rows at or past it are masked
#pragma unroll
      for (int t = 0; t < G::kLoads; ++t) {
        const int x = u * G::kLoads + t;
        const float d = row_sum<G::kLpr>(dot16<DT>(qv, kb[x])) * scale_log2;
        sc[x] = (t * G::kRpl + r < ntok) ? d : -__builtin_inff();
        bm = fmaxf(bm, sc[x]);
      }
    }
    const float m_new = fmaxf(m, bm);
    const float alpha = exp2_fast(m - m_new);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < G::kEpl; ++e) acc[e] *= alpha;
#pragma unroll
    for (int x = 0; x < kRows; ++x) {
      const float pr = exp2_fast(sc[x] - m_new);
      l += pr;
      axpy16<DT>(pr, vb[x], acc);
    }
    m = m_new;
  };

  // Before the owner wave issues the loads of stage i_new, the newest row's
  // store has completed.  On gfx9-family GPUs (CDNA included) one vector
  // memory counter covers a wave's loads and stores, and it counts them down
  // in the order they were issued, a store once its data has reached the L2
  // cache (AMD's CDNA3 and CDNA4 ISA reference guides, section "Data
  // Dependency Resolution", the S_WAITCNT vector-memory counter).  The store
  // is older than every stage load, so it is enough to wait until no more
  // than the loads of the stages issued since are outstanding: min(i, NST - 1)
  // stages (later ones than that have been consumed, hence waited for,
  // already).  For i = 0 nothing has been issued
  // since, and the wait is for everything.  For any other stage, and any
  // other wave, this is not reached.
  constexpr int kLoadsPerStage = 2 * TPS * G::kLoads;
  static_assert(NST <= 3 && (NST - 1) * kLoadsPerStage < 64, "vmcnt holds 6 bits; cases below cover NST <= 3");
  auto await_newest = [&](int i) {
    if (FUSED && i == i_new) {
      constexpr int kOthers = (7 << 4) | (15 << 8);            // expcnt, lgkmcnt: no wait
      constexpr auto vm = [](int n) { return (n & 15) | ((n >> 4) << 14); };
      if (i == 0)
        __builtin_amdgcn_s_waitcnt(vm(0) | kOthers);
      else if (NST > 2 && i == 1)
        __builtin_amdgcn_s_waitcnt(vm(kLoadsPerStage) | kOthers);
      else
        __builtin_amdgcn_s_waitcnt(vm((NST - 1) * kLoadsPerStage) | kOthers);
    }
  };

  // NST-deep pipeline over register buffers.  Step s issues the loads of
  // stage s into buffer s % NST, then consumes stage s - (NST - 1), whose
  // loads were issued NST - 1 steps earlier.  The first NST - 1 steps consume
  // stages below 0 from zeroed buffers and steps past the wave's last stage
  // issue empty loads; both leave the state bit-for-bit unchanged.  There is
  // no prologue: every buffer is written only inside the loop, so the
  // register allocator keeps each one in the same registers across the back
  // edge (with a prologue it gave the V buffers other registers there and
  // copied them, which forced a wait for every load in flight once per
  // iteration).  The body has no branch between a buffer's loads and its
  // consumer, so the compiler cannot sink the loads below the consumer; the
  // scheduling barriers keep the machine scheduler from doing the same
  // inside a step.
  if (n_my > 0) {
    u32x4 kb[NST][kRows], vb[NST][kRows];
#pragma unroll
    for (int b = 0; b < NST; ++b)
#pragma unroll
      for (int x = 0; x < kRows; ++x) kb[b][x] = vb[b][x] = u32x4{0u, 0u, 0u, 0u};
    int32_t ids[TPS];
    for (int i = 0; i < n_my + NST - 1; i += NST) {
#pragma unroll
      for (int b = 0; b < NST; ++b) {
        table_at(i + b, ids);
        await_newest(i + b);
        issue(kb[b], vb[b], i + b, ids);
        __builtin_amdgcn_sched_barrier(0);
        consume(kb[(b + 1) % NST], vb[(b + 1) % NST], i + b - (NST - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Merge the kStates row states of the work-group.
  __shared__ float sm_m[G::kStates];
  __shared__ float sm_l[G::kStates];
  // The 3-deep ring of 32-token tiles runs one 4-wave work-group per compute
  // unit: with two (a version of the fused kernel whose registers allowed it)
  // it measured 3 % slower.  Its registers alone keep it to one today; the
  // merge buffer is also sized past half of the compute unit's 160 KiB of
  // LDS, so that stays true whatever the register count.
  constexpr int kAccFloats = G::kStates * D;
  constexpr int kOneGroupFloats = NST > 2 ? 96 * 1024 / 4 : 0;
  __shared__ float sm_acc[kAccFloats > kOneGroupFloats ? kAccFloats : kOneGroupFloats];
  __shared__ int sm_bad[kWaves];
  const int st = wave * G::kRpl + r;
  if (c == 0) {
    sm_m[st] = m;
    sm_l[st] = l;
  }
  if (lane == 0) sm_bad[wave] = bad ? 1 : 0;
#pragma unroll
  for (int e = 0; e < G::kEpl; ++e) sm_acc[st * D + c * G::kEpl + e] = acc[e];
  __syncthreads();

  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    float M = kEmptyMax;
#pragma unroll
    for (int k = 0; k < G::kStates; ++k) M = fmaxf(M, sm_m[k]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int k = 0; k < G::kStates; ++k) {
      const float w = exp2_fast(sm_m[k] - M);
      num = __builtin_fmaf(w, sm_acc[k * D + d], num);
      den = __builtin_fmaf(w, sm_l[k], den);
    }
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) any_bad |= sm_bad[w];
    if (any_bad) den = __builtin_nanf("");
    if (parts == 1) {
      store_elem<DT>(out, row * D + d, num / den);
    } else {
      const int64_t wi = row * partitions + p;
      ws_acc[wi * D + d] = num;
      if (d == 0) {
        ws_m[wi] = M;
        ws_l[wi] = den;
      }
    }
  }
}

// Merge the partitions of every (sequence, head) whose context spans more
// than one: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p, M = max_p
// m_p.  Four waves per (head, sequence): wave w folds partitions w, w + 4, ...
// into a running (max, numerator, denominator) with each lane holding D / 64
// dims, so up to four partitions' loads are in flight per row at once; the
// four states are then merged through LDS.  A wave that got no partition
// keeps the empty state, whose weight 2^(kEmptyMax - M) is 0.
constexpr int kReduceWaves = 4;
template <int DT, int D>
__global__ __launch_bounds__(64 * kReduceWaves) void lse_reduce_kernel(
    const int32_t* __restrict__ context_lens, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, const float* __restrict__ ws_acc, void* __restrict__ out,
    int32_t max_blocks, int32_t block_size, int32_t part_blocks, int32_t partitions) {
  constexpr int kDpl = D / 64;                            // dims per lane
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int H = gridDim.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t L = context_lens[s];
  if (L <= 0 || !context_ok(L, max_blocks * block_size)) return;
  const int nb = (L + block_size - 1) / block_size;
  const int parts = (nb + part_blocks - 1) / part_blocks;
  if (parts <= 1) return;
  const int64_t row = int64_t(s) * H + h;
  const int64_t base = row * partitions;
  float m = kEmptyMax, den = 0.f, num[kDpl];
#pragma unroll
  for (int e = 0; e < kDpl; ++e) num[e] = 0.f;
  for (int p = wave; p < parts; p += kReduceWaves) {
    const float mp = ws_m[base + p];
    const float lp = ws_l[base + p];
    const float m_new = fmaxf(m, mp);
    const float a = exp2_fast(m - m_new);
    const float b = exp2_fast(mp - m_new);
    den = __builtin_fmaf(den, a, lp * b);
    const float* accp = ws_acc + (base + p) * D + lane * kDpl;
#pragma unroll
    for (int e = 0; e < kDpl; ++e) num[e] = __builtin_fmaf(num[e], a, accp[e] * b);
    m = m_new;
  }
  __shared__ float sm_m[kReduceWaves];
  __shared__ float sm_den[kReduceWaves];
  __shared__ float sm_num[kReduceWaves * D];
  if (lane == 0) {
    sm_m[wave] = m;
    sm_den[wave] = den;
  }
#pragma unroll
  for (int e = 0; e < kDpl; ++e) sm_num[wave * D + lane * kDpl + e] = num[e];
  __syncthreads();
  if (wave != 0) return;
  float M = kEmptyMax;
#pragma unroll
  for (int w = 0; w < kReduceWaves; ++w) M = fmaxf(M, sm_m[w]);
  float d = 0.f, n[kDpl];
#pragma unroll
  for (int e = 0; e < kDpl; ++e) n[e] = 0.f;
#pragma unroll
  for (int w = 0; w < kReduceWaves; ++w) {
    const float f = exp2_fast(sm_m[w] - M);
    d = __builtin_fmaf(f, sm_den[w], d);
#pragma unroll
    for (int e = 0; e < kDpl; ++e) n[e] = __builtin_fmaf(f, sm_num[w * D + lane * kDpl + e], n[e]);
  }
#pragma unroll
  for (int e = 0; e < kDpl; ++e) store_elem<DT>(out, row * D + lane * kDpl + e, n[e] / d);
}

template <int DT, int D, int BS>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(unsigned(a.num_heads), unsigned(a.partitions), unsigned(a.num_seqs));
  constexpr int kWaves = waves_for<BS>();
  constexpr int kTps = tiles_for<DT, D, BS>();
  constexpr int kNst = stages_for<DT, kTps>();
  auto* kernel = a.k_new != nullptr ? decode_partition_kernel<DT, D, BS, kWaves, kTps, kNst, true>
                                    : decode_partition_kernel<DT, D, BS, kWaves, kTps, kNst, false>;
  int waves = kWaves;
  // Partitions of at most 64 blocks (1024 tokens of 16-token blocks) give an
  // 8-wave work-group at most four stages per wave; 4-wave work-groups (the
  // same per-wave pipeline, two of them per compute unit) overlap one's start
  // and merge with the other's loads (8 x 40 x 32k at 512-token partitions:
  // 857 vs 876 us per step; 1 x 40 x 32k at 1024-token partitions: 103.7 vs
  // 105.7 us per call).  At 128 blocks they lose on some shapes.
  if constexpr (kWaves == 8) {
    if (a.partitions > 1 && a.part_blocks <= kSmallPartitionBlocks) {
      kernel = a.k_new != nullptr ? decode_partition_kernel<DT, D, BS, 4, kTps, kNst, true>
                                  : decode_partition_kernel<DT, D, BS, 4, kTps, kNst, false>;
      waves = 4;
    }
  }
  hipLaunchKernelGGL(kernel, grid, dim3(64 * waves), 0, stream, a.q,
                     static_cast<char*>(a.k_cache), static_cast<char*>(a.v_cache),
                     a.block_tables, a.context_lens, a.out, a.ws_m, a.ws_l, a.ws_acc, a.num_blocks,
                     a.max_blocks, a.part_blocks, a.partitions, a.scale_log2,
                     static_cast<const char*>(a.k_new), static_cast<const char*>(a.v_new));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.partitions <= 1) return e;
  hipLaunchKernelGGL((lse_reduce_kernel<DT, D>), dim3(unsigned(a.num_heads), unsigned(a.num_seqs)),
                     dim3(64 * kReduceWaves), 0, stream, a.context_lens, a.ws_m, a.ws_l, a.ws_acc, a.out,
                     a.max_blocks, BS, a.part_blocks, a.partitions);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(int head_dim, int block_size, const DecodeArgs& a, hipStream_t stream) {
  if (head_dim == 64) {
    return block_size == 16 ? launch_typed<DT, 64, 16>(a, stream) : launch_typed<DT, 64, 32>(a, stream);
  }
  return block_size == 16 ? launch_typed<DT, 128, 16>(a, stream) : launch_typed<DT, 128, 32>(a, stream);
}

}  // namespace

hipError_t launch_decode(int dtype, int head_dim, int block_size, const DecodeArgs& a,
                         hipStream_t stream) {
  switch (dtype) {
    case PKV_F32: return launch_dt<PKV_F32>(head_dim, block_size, a, stream);
    case PKV_F16: return launch_dt<PKV_F16>(head_dim, block_size, a, stream);
    default: return launch_dt<PKV_BF16>(head_dim, block_size, a, stream);
  }
}

}  // namespace pkv
