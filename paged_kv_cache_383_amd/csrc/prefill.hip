// Paged prefill for gfx950: causal attention of a batch of new tokens over
// their sequences' block-paged K/V caches, on the matrix cores.
//
// What is computed ("vLLM KV cache and PagedAttention explained", hrletsgo.me,
// Step 6 and Appendix: The Attention Score Formula): a sequence's prompt
// tokens are processed in parallel, each attending, by softmax(q K^T * scale) V,
// to the cached tokens up to and including its own position (causal
// attention).  The new tokens' K/V are already in the cache (paged_kv_write);
// tokens before them (a cached or shared prefix, Step 9) are read the same
// way, through the block table, in place ("PagedAttention" card, "Kernel은
// 무엇이 달라지는가").
//
// Unlike decode, this is a dense contraction: a tile of queries meets every
// key of a chunk, so the products go to MFMA.  Both kernels walk the keys in
// 32-key chunks staged in LDS.  bf16/f16 take prefill32_kernel (32x32x16
// tiles, K/V loaded straight into LDS; described above it): 4 wave64s per
// (sequence, head, 128-query tile), 32 queries per wave.  fp32 takes
// prefill_kernel (16x16x4 tiles), described
// here: one work-group of 8 wave64s per (head, 128-query tile, sequence); each
// wave owns 16 queries (kSub 16-query sub-tiles; one keeps the kernel at about
// 110 VGPRs, so two work-groups share a compute unit and hide each other's
// latencies).  Keys are walked in chunks of 32
// (one 32-token block or two 16-token blocks), staged once per work-group in
// LDS and shared by its 8 waves (double-buffered: the next chunk's rows are
// fetched into registers while this one is computed):
//   K chunk as [key][d] (the cache's own row order),
//   V chunk as [key][d] too, read as V^T with the transposing LDS load, so
//   each lane's MFMA operand is a run of consecutive keys (fp32: stored
//   transposed).
// Per chunk and sub-tile a wave computes S^T = K Q^T with
// v_mfma_f32_16x16x32_{bf16,f16} (fp32: 16x16x4), keeps each query's running
// max across its four lane groups, and accumulates O^T += V^T P^T with P^T
// taken straight from the S^T registers: a lane of S^T holds keys
// {4g..4g+3} and {16+4g..16+4g+3} of one query (g = lane / 16), and the V^T
// operand lists the same keys in the same k-slot order, so no transpose of P
// is needed.  Keys past the query's position or past the context are masked;
// their V rows are staged as zeros so that 0 * garbage never enters a sum.
#include <hip/hip_fp16.h>

#include "pagedkv.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSub = 1;                        // 16-query sub-tiles per wave
constexpr int kTileQ = kWaves * kSub * 16;     // queries per work-group
constexpr int kChunk = 32;                     // keys per chunk
constexpr float kEmptyMax = -3.0e38f;
// Word 3 of a gfx9 raw buffer resource: 32-bit data format, no swizzle.
constexpr int kBufferWord3 = 0x00020000;

template <int DT>
struct Mfma;

// 16-bit types: 16x16x32, 8 elements per lane per operand.
template <>
struct Mfma<PKV_BF16> {
  static constexpr int kStep = 32, kEpl = 8, kBytes = 2;
  using frag = bf16x8;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ __bf16 from_f32(float x) { return static_cast<__bf16>(x); }
};
template <>
struct Mfma<PKV_F16> {
  static constexpr int kStep = 32, kEpl = 8, kBytes = 2;
  using frag = f16x8;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ _Float16 from_f32(float x) { return _Float16(x); }
};
// fp32: 16x16x4, one element per lane per operand.
template <>
struct Mfma<PKV_F32> {
  static constexpr int kStep = 4, kEpl = 1, kBytes = 4;
  using frag = float;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float from_f32(float x) { return x; }
};

template <int DT>
using elem_t = typename std::conditional<DT == PKV_BF16, __bf16,
                                         typename std::conditional<DT == PKV_F16, _Float16, float>::type>::type;

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float x) {
  unsigned int u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<unsigned short>(u >> 16);
}

template <int DT>
__device__ __forceinline__ void store_out(void* base, int64_t i, float x) {
  if constexpr (DT == PKV_F32) {
    static_cast<float*>(base)[i] = x;
  } else if constexpr (DT == PKV_F16) {
    static_cast<unsigned short*>(base)[i] = __half_as_ushort(__float2half(x));
  } else {
    static_cast<unsigned short*>(base)[i] = f32_to_bf16_rne(x);
  }
}

// LDS staging of one 32-key chunk.  K keeps the cache's [key][d] order (a
// 16-byte pad per row puts the 16 rows an MFMA operand read touches in
// distinct banks).  For 16-bit types V keeps it too: the V^T operand is read
// with the gfx950 transposing LDS load (ds_read_tr16_b64), which hands each
// lane four consecutive keys of one dimension; a 32-byte pad per row spreads
// the 16 keys one such read touches over the banks.  fp32 has no transposing
// load: V is stored transposed, [d][key].
template <int DT, int D>
struct Smem {
  using E = elem_t<DT>;
  static constexpr bool kTr = Mfma<DT>::kBytes == 2;
  static constexpr int kPitchK = D + 16 / Mfma<DT>::kBytes;
  static constexpr int kPitchV = kTr ? D + 32 / Mfma<DT>::kBytes : kChunk + 16 / Mfma<DT>::kBytes;
  alignas(16) E k[kChunk * kPitchK];
  alignas(16) E v[kTr ? kChunk * kPitchV : D * kPitchV];
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int DT, int D, int BS>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const void* __restrict__ q, const char* __restrict__ k_cache, const char* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ query_start,
    const int32_t* __restrict__ context_lens, void* __restrict__ out, int64_t num_blocks, int32_t max_blocks,
    int32_t tiles, float scale_log2) {
  using M = Mfma<DT>;
  using E = elem_t<DT>;
  using S = Smem<DT, D>;
  constexpr int kEs = M::kBytes;
  constexpr int kVpr = D * kEs / 16;                 // 16-byte vectors per K/V row
  constexpr int kVecs = kChunk * kVpr;               // per chunk per tensor
  constexpr int kEpv = 16 / kEs;                     // elements per 16-byte vector
  constexpr int kDSteps = D / M::kStep;              // MFMA k-steps over head_dim
  constexpr int kDTiles = D / 16;                    // 16-dim output tiles
  constexpr int kBufs = 2 * sizeof(S) <= 48 * 1024 ? 2 : 1;   // fp32 head_dim 128 keeps one buffer
  __shared__ S sm[kBufs];
  __shared__ int sm_bad;

  const int h = blockIdx.x;
  const int tile = tiles - 1 - int(blockIdx.y);      // longest-running tiles first
  const int s = blockIdx.z;
  const int H = gridDim.x;
  const int qa = query_start[s], qb = query_start[s + 1];
  const int P = qb - qa;
  const int L = context_lens[s];
  const int q0 = tile * kTileQ;
  if (P <= 0 || q0 >= P) return;
  // Broken contract (more queries than context, a context past the table, or
  // more queries than max_query_len covers): the sequence's rows become NaN
  // and no cache memory is touched.
  const bool ok = P <= L && L <= max_blocks * BS && P <= tiles * kTileQ;
  const int first = L - P;                           // position of the sequence's first query

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;                         // query within a sub-tile (column of S^T)
  const int grp = lane >> 4;                         // lane group: keys 4g.., dims 4g..

  if (!ok) {
    const int hi = tile == tiles - 1 ? P : min(q0 + kTileQ, P);     // the last tile also covers the rest
    for (int64_t i = threadIdx.x; i < int64_t(hi - q0) * D; i += kThreads)
      store_out<DT>(out, (int64_t(qa + q0 + int(i / D)) * H + h) * D + i % D, __builtin_nanf(""));
    return;
  }
  if (threadIdx.x == 0) sm_bad = 0;

  // Query fragments (B operand of S^T = K Q^T): lane holds Q[col][step * kStep + grp * kEpl + e].
  typename M::frag qf[kSub][kDSteps];
  int qpos[kSub];
#pragma unroll
  for (int u = 0; u < kSub; ++u) {
    const int qi = q0 + (wave * kSub + u) * 16 + col;
    qpos[u] = qi < P ? first + qi : -1;              // -1: no query (every key masked)
    const E* qrow = static_cast<const E*>(q) + (int64_t(qa + (qi < P ? qi : 0)) * H + h) * D;
#pragma unroll
    for (int st = 0; st < kDSteps; ++st) {
      if constexpr (M::kEpl == 1) {
        qf[u][st] = qi < P ? qrow[st * M::kStep + grp] : 0.f;
      } else {
        const u32x4 raw = qi < P ? *reinterpret_cast<const u32x4*>(qrow + st * M::kStep + grp * M::kEpl)
                                 : u32x4{0, 0, 0, 0};
        qf[u][st] = __builtin_bit_cast(typename M::frag, raw);
      }
    }
  }

  f32x4 acc[kSub][kDTiles];
  float m[kSub], l[kSub];
#pragma unroll
  for (int u = 0; u < kSub; ++u) {
    m[u] = kEmptyMax;
    l[u] = 0.f;
#pragma unroll
    for (int t = 0; t < kDTiles; ++t) acc[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int wave_first = first + q0 + wave * kSub * 16;      // position of the wave's first query
  const int wave_q1 = min(q0 + (wave + 1) * kSub * 16, P);   // one past the wave's last query
  const int wave_last = q0 + wave * kSub * 16 < P ? first + wave_q1 - 1 : -1;
  // Keys this work-group needs: up to its last query's position.
  const int last_q = min(q0 + kTileQ, P) - 1;
  const int nkeys = first + last_q + 1;
  const int nchunks = (nkeys + kChunk - 1) / kChunk;
  const int32_t* trow = block_tables + int64_t(s) * max_blocks;
  bool bad = false;

  // Software pipeline over chunks: chunk c + 1's K/V rows are fetched into
  // registers while chunk c is computed from LDS; with two LDS buffers a
  // single barrier per chunk orders the staging against the readers.
  constexpr int kNv = (kVecs + kThreads - 1) / kThreads;   // 16-byte vectors per thread per tensor
  u32x4 rk[kNv], rv[kNv];
  const int nblocks = (L + BS - 1) / BS;
  auto fetch = [&](int c) {
    const int k0 = c * kChunk;
    // The chunk's physical blocks (one or two), read once as wave-uniform values.
    constexpr int kBlk = kChunk / BS;
    int32_t bid[kBlk];
#pragma unroll
    for (int u = 0; u < kBlk; ++u) {
      const int j = k0 / BS + u;
      bid[u] = j < nblocks ? __builtin_amdgcn_readfirstlane(trow[j]) : 0;
    }
#pragma unroll
    for (int i = 0; i < kNv; ++i) {
      const int v = threadIdx.x + i * kThreads;
      const int key = v / kVpr, cv = v % kVpr;
      const int kg = k0 + key;
      rk[i] = u32x4{0, 0, 0, 0};
      rv[i] = u32x4{0, 0, 0, 0};
      if (v < kVecs && kg < L) {                     // keys past the context stay zero
        int32_t b = bid[0];
#pragma unroll
        for (int u = 1; u < kBlk; ++u)
          if (key / BS == u) b = bid[u];
        if (static_cast<uint64_t>(static_cast<int64_t>(b)) < static_cast<uint64_t>(num_blocks)) {
          const int64_t off = ((int64_t(b) * H + h) * BS + kg % BS) * int64_t(D * kEs) + cv * 16;
          rk[i] = *reinterpret_cast<const u32x4*>(k_cache + off);
          rv[i] = *reinterpret_cast<const u32x4*>(v_cache + off);
        } else {
          bad = true;
        }
      }
    }
  };
  // K as [key][d]; V as [key][d] (16-bit types) or transposed (fp32).
  auto stage = [&](S& buf) {
#pragma unroll
    for (int i = 0; i < kNv; ++i) {
      const int v = threadIdx.x + i * kThreads;
      if (v >= kVecs) continue;
      const int key = v / kVpr, cv = v % kVpr;
      *reinterpret_cast<u32x4*>(&buf.k[key * S::kPitchK + cv * kEpv]) = rk[i];
      if constexpr (S::kTr) {
        *reinterpret_cast<u32x4*>(&buf.v[key * S::kPitchV + cv * kEpv]) = rv[i];
      } else {
        const E* ve = reinterpret_cast<const E*>(&rv[i]);
#pragma unroll
        for (int e = 0; e < kEpv; ++e) buf.v[(cv * kEpv + e) * S::kPitchV + key] = ve[e];
      }
    }
  };

  fetch(0);
  for (int c = 0; c < nchunks; ++c) {
    const int k0 = c * kChunk;
    S& sb = sm[c % kBufs];
    if (kBufs == 1 && c > 0) __syncthreads();         // every wave is done reading the one buffer
    stage(sb);
    __syncthreads();
    if (c + 1 < nchunks) fetch(c + 1);
    // A wave skips chunks that start past its last query's position (every
    // key would be masked); a wave without queries skips them all.  It still
    // stages its share of every chunk for the other waves.
    if (k0 > wave_last) continue;

    // S^T for keys [k0, k0 + 32) as two 16-key tiles.  Each K fragment is read
    // from LDS once and used for every sub-tile of the wave.
    f32x4 st0[kSub], st1[kSub];
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      st0[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      st1[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int st = 0; st < kDSteps; ++st) {
      typename M::frag a0, a1;
      if constexpr (M::kEpl == 1) {
        a0 = sb.k[col * S::kPitchK + st * M::kStep + grp];
        a1 = sb.k[(16 + col) * S::kPitchK + st * M::kStep + grp];
      } else {
        a0 = __builtin_bit_cast(typename M::frag,
                                *reinterpret_cast<const u32x4*>(&sb.k[col * S::kPitchK + st * M::kStep + grp * M::kEpl]));
        a1 = __builtin_bit_cast(typename M::frag,
                                *reinterpret_cast<const u32x4*>(&sb.k[(16 + col) * S::kPitchK + st * M::kStep + grp * M::kEpl]));
      }
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        st0[u] = M::mma(a0, qf[u][st], st0[u]);
        st1[u] = M::mma(a1, qf[u][st], st1[u]);
      }
    }
    // Scale, mask (key position > query position), running max, P.  Chunks
    // wholly before the wave's first query need no mask.
    const bool masked = k0 + kChunk - 1 > wave_first;
    float p[kSub][8];
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      float sc[8];
      float bm = kEmptyMax;
      if (masked) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ka = k0 + 4 * grp + e, kb = k0 + 16 + 4 * grp + e;
          sc[e] = ka <= qpos[u] ? st0[u][e] * scale_log2 : -__builtin_inff();
          sc[4 + e] = kb <= qpos[u] ? st1[u][e] * scale_log2 : -__builtin_inff();
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc[e] = st0[u][e] * scale_log2;
          sc[4 + e] = st1[u][e] * scale_log2;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) bm = fmaxf(bm, sc[e]);
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float m_new = fmaxf(m[u], bm);
      const float alpha = __builtin_amdgcn_exp2f(m[u] - m_new);
      m[u] = m_new;
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[u][e] = __builtin_amdgcn_exp2f(sc[e] - m_new);
        ps += p[u][e];
      }
      l[u] = l[u] * alpha + ps;                      // this lane's share; groups summed at the end
      if (__any(alpha != 1.f)) {                     // the running max moved for some query
#pragma unroll
        for (int t = 0; t < kDTiles; ++t) acc[u][t] *= alpha;
      }
    }
    // O^T += V^T P^T; each V fragment is read once for all sub-tiles.
    if constexpr (M::kEpl == 1) {
#pragma unroll
      for (int t = 0; t < kDTiles; ++t) {
        const E* vrow = &sb.v[(16 * t + col) * S::kPitchV];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const E vv = vrow[16 * half + 4 * grp + e];
#pragma unroll
            for (int u = 0; u < kSub; ++u) acc[u][t] = M::mma(vv, p[u][4 * half + e], acc[u][t]);
          }
      }
    } else {
      typename M::frag pf[kSub];
#pragma unroll
      for (int u = 0; u < kSub; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[u][e] = M::from_f32(p[u][e]);
      // Lane j of a 16-lane group points the transposing load at 4 dims of
      // key 4g + j/4 (dims 16t + 4 (j % 4) ..); lane i then holds dim 16t + i
      // of keys 4g .. 4g+3.  A second load does keys 16 + 4g .. 16 + 4g + 3.
      const E* vbase = &sb.v[(4 * grp + col / 4) * S::kPitchV + 4 * (col % 4)];
#pragma unroll
      for (int t = 0; t < kDTiles; ++t) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbase + 16 * t));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbase + 16 * S::kPitchV + 16 * t));
        const typename M::frag vf = __builtin_bit_cast(
            typename M::frag, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
        for (int u = 0; u < kSub; ++u) acc[u][t] = M::mma(vf, pf[u], acc[u][t]);
      }
    }
  }

  if (bad) sm_bad = 1;
  __syncthreads();
  const bool any_bad = sm_bad != 0;
#pragma unroll
  for (int u = 0; u < kSub; ++u) {
    const int qi = q0 + (wave * kSub + u) * 16 + col;
    float lt = l[u];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (qi >= P) continue;
    const float inv = any_bad ? __builtin_nanf("") : 1.f / lt;
    const int64_t base = (int64_t(qa + qi) * H + h) * D;
#pragma unroll
    for (int t = 0; t < kDTiles; ++t) {
      if constexpr (DT == PKV_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + base + 16 * t + 4 * grp) = acc[u][t] * inv;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) store_out<DT>(out, base + 16 * t + 4 * grp + e, acc[u][t][e] * inv);
      }
    }
  }
}

// 16-bit types: 32x32x16 MFMA tiles.  Each wave owns 32 queries (the columns
// of a 32x32 S^T tile), so a K or V fragment read from LDS serves twice as
// many queries as with 16-query tiles and a query's running max needs one
// cross-lane step.  Layouts of v_mfma_f32_32x32x16: A[i][k] lane = i + 32
// (k / 8), B[k][j] lane = j + 32 (k / 8), C[i][j] lane = j + 32 ((i / 4) % 2)
// with element 4 (i / 8) + i % 4.  A lane of S^T therefore holds, for its query,
// the keys 8 (e / 4) + 4 h + e % 4 (h = lane / 32, e < 16); the P^T operand of
// k-step s is its elements 8 s .. 8 s + 7 as they are, and the V^T operand
// lists the same keys in the same k-slot order (two transposing loads of four
// keys each).  K/V chunks reach LDS by loads that write it directly (no
// register staging), three buffers deep: chunk c + 2 is in flight while c is
// computed, and a chunk costs one barrier.
constexpr int kWaves32 = 4;
constexpr int kTileQ32 = 32 * kWaves32;
// Work order (one work-group per (sequence, head, 128-query tile)).  Work-
// groups go to the 8 XCDs round robin by linear id, and the tiles of one
// (sequence, head) read the same K/V chunks from position 0 up, so they are
// placed on one XCD back to back, where they run together and share its L2;
// measured ~8 % faster than launching every sequence's last tiles first.
// For balance the tiles are split into kBands bands (longest tiles first):
// band 0 of every (sequence, head) is launched before band 1, and so on, so
// that the longest tiles never start last.
constexpr int kBands = 3;
constexpr float kLazy = 8.f;

// x of lane i and of lane i ^ 32, in every lane, by the gfx950 cross-half
// lane swap (no round trip through LDS): swapping the upper half of one copy
// of x with the lower half of another leaves the lower halves' values in the
// first result and the upper halves' in the second.
struct Halves {
  float lo, hi;
};
__device__ inline Halves halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// 16-byte buffer load straight into LDS: lane i's 16 bytes land at LDS byte
// address lds + 16 i; bytes at or past nrec read as zero.  base, nrec and lds
// must be wave-uniform.  Written as inline assembly so that the compiler's
// wait-count insertion, which cannot tell which LDS buffer such a load
// writes, does not hold LDS reads of the other buffers behind it; the caller
// waits for completion itself (vmcnt, then a barrier).  The compiler does not
// see the instruction inside, so the asm supplies the wait states the gfx9
// hazard rules ask for before it: one after an SALU write of M0 (the LDS
// address) and five after a VALU write (v_readfirstlane) of an SGPR of the
// buffer descriptor.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ inline void load_lds16(const char* base, int nrec, uint32_t voff, uint32_t lds) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const i32x4 desc = {__builtin_amdgcn_readfirstlane(int(uint32_t(a))),
                      __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffff)),
                      __builtin_amdgcn_readfirstlane(nrec), kBufferWord3};
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(desc), "{m0}"(lds) : "memory");
}
__device__ inline uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>((uintptr_t)(__attribute__((address_space(3))) const void*)p);
}

// Two fp32 values rounded to nearest even into one word of 16-bit elements
// (the first in the low half).
template <int DT>
__device__ inline uint32_t pack2(float x, float y) {
  if constexpr (DT == PKV_BF16) {
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, v2{static_cast<__bf16>(x), static_cast<__bf16>(y)});
  } else {
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, v2{static_cast<_Float16>(x), static_cast<_Float16>(y)});
  }
}

template <int DT, int D, int BS>
__global__ __launch_bounds__(64 * kWaves32) __attribute__((amdgpu_waves_per_eu(3))) void prefill32_kernel(
    const void* __restrict__ q, const char* __restrict__ k_cache, const char* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ query_start,
    const int32_t* __restrict__ context_lens, void* __restrict__ out, int64_t num_blocks, int32_t max_blocks,
    int32_t tiles, float scale_log2, int32_t num_heads, int32_t num_seqs) {
  static_assert(Mfma<DT>::kBytes == 2, "16-bit types only");
  using E = elem_t<DT>;
  using frag = typename Mfma<DT>::frag;
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  constexpr int kT = 64 * kWaves32;
  constexpr int kVpr = D * 2 / 16;                   // 16-byte columns per K/V row
  constexpr int kRowsPerLoad = 64 / kVpr;            // rows one wave-wide 16-byte load fills
  constexpr int kNl = kChunk / kRowsPerLoad / kWaves32;  // such loads per wave per tensor per chunk
  constexpr int kDSteps = D / 16;                    // k-steps of S^T over head_dim
  constexpr int kDTiles = D / 32;                    // 32-dim output tiles
  static_assert(kNl * kWaves32 * kRowsPerLoad == kChunk && BS % kRowsPerLoad == 0, "load tiling");
  // Three chunk buffers (K and V rows, [key][d], no padding; 16-byte columns
  // swizzled against bank conflicts, see below), filled by loads that write
  // LDS directly: two chunks are in flight while a third is computed.  One
  // array (buffer b: K at ring[2 b], V at ring[2 b + 1]), so that every LDS
  // read is a per-lane register plus a constant offset; separate arrays cost
  // a register per buffer and operand (168 VGPRs against 144).
  __shared__ __attribute__((aligned(16))) E ring[6][kChunk * D];
  __shared__ int sm_bad;
  E* const lk0 = ring[0];
  E* const lv0 = ring[1];
  E* const lk1 = ring[2];
  E* const lv1 = ring[3];
  E* const lk2 = ring[4];
  E* const lv2 = ring[5];

  // Linear id n: XCD x = n % 8 takes (sequence, head) pairs x, x + 8, ...
  // (pair = sequence * H + head); its r-th work-group (r = n / 8) is, in band
  // order, tile k of the band of its local pair r / w (w = the band's tile
  // count), tiles counted from the last (longest) one.
  const int H = num_heads;
  int h, s, tile;
  {
    const int n = blockIdx.x, x = n % 8;
    int r = n / 8;
    const int J = (num_heads * num_seqs + 7) / 8;      // pairs per XCD (rounded up)
    int b = 0, klo = 0, khi = tiles / kBands;
    while (r >= J * (khi - klo)) {
      r -= J * (khi - klo);
      ++b;
      klo = khi;
      khi = (b + 1) * tiles / kBands;
    }
    const int w = khi - klo;
    const int pr = (r / w) * 8 + x;
    if (pr >= num_heads * num_seqs) return;
    s = pr / num_heads;
    h = pr % num_heads;
    tile = klo + r % w;                              // rank from the sequence's own last tile
  }
  const int qa = query_start[s], qb = query_start[s + 1];
  const int P = qb - qa;
  const int L = context_lens[s];
  // Rank k is the sequence's k-th longest tile, so every pair's longest tile
  // is in the first band and the ranks past a short sequence's tile count
  // (work-groups with nothing to do) gather at the end of the grid.
  const int ntiles = P > 0 ? min((P + kTileQ32 - 1) / kTileQ32, tiles) : 0;
  if (tile >= ntiles) return;
  tile = ntiles - 1 - tile;
  const int q0 = tile * kTileQ32;
  const bool ok = P <= L && L <= max_blocks * BS && P <= tiles * kTileQ32;
  const int first = L - P;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;                         // query of the wave (column of S^T)
  const int hh = lane >> 5;                          // lane half
  if (!ok) {
    const int hi = tile == tiles - 1 ? P : min(q0 + kTileQ32, P);
    for (int64_t i = threadIdx.x; i < int64_t(hi - q0) * D; i += kT)
      store_out<DT>(out, (int64_t(qa + q0 + int(i / D)) * H + h) * D + i % D, __builtin_nanf(""));
    return;
  }
  if (threadIdx.x == 0) sm_bad = 0;

  const int qi = q0 + wave * 32 + col;
  const int qpos = qi < P ? first + qi : -1;
  frag qf[kDSteps];                                  // B operand: Q[col][16 st + 8 hh + e]
  f32x16 acc[kDTiles];
#pragma unroll
  for (int t = 0; t < kDTiles; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  float m = kEmptyMax, l = 0.f;

  const int wave_first = first + q0 + wave * 32;
  const int wave_last = q0 + wave * 32 < P ? first + min(q0 + wave * 32 + 32, P) - 1 : -1;
  const int last_q = min(q0 + kTileQ32, P) - 1;
  const int nchunks = (first + last_q + 1 + kChunk - 1) / kChunk;
  const int32_t* trow = block_tables + int64_t(s) * max_blocks;
  bool bad = false;

  // Swizzle (LDS of 64 four-byte banks, one 256-byte bank row holding
  // kRb = 128 / D chunk rows): 16-byte column c of chunk row r sits at
  // column c ^ (b % kVpr) in K and c ^ 4 (b % (kVpr / 4)) in V, b = r / kRb.
  // The S^T operand read (16 lanes: 16 rows, one column) and the transposing
  // V^T read (32 lanes: 4 rows, 4 columns, 2 halves) then touch distinct
  // banks.  Wave w loads rows 8 w .. 8 w + 7 of each chunk (one
  // block: blocks hold 16 or 32 rows), kRowsPerLoad rows per wave-wide load:
  // lane i writes 16 bytes at LDS offset 16 i of the load's rows (the
  // load-to-LDS layout) and therefore fetches the logical column whose
  // swizzled position that is.  Chunks start on block boundaries, so a
  // lane's offset within its block is the same for every chunk.
  constexpr int kRowsPerWave = kChunk / kWaves32;
  constexpr int kRb = 128 / D;                       // chunk rows per 256-byte bank row
  static_assert(kRowsPerWave == kNl * kRowsPerLoad && BS % kRowsPerWave == 0, "a wave loads within one block");
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t koff[kNl], voff[kNl];
#pragma unroll
  for (int i = 0; i < kNl; ++i) {
    const int r = wave_s * kRowsPerWave + i * kRowsPerLoad + lane / kVpr;
    const int pc = lane % kVpr;
    const int b = r / kRb;
    koff[i] = uint32_t((r % BS) * D * 2 + (pc ^ (b % kVpr)) * 16);
    voff[i] = uint32_t((r % BS) * D * 2 + (pc ^ (4 * (b % (kVpr / 4)))) * 16);
  }
  const int64_t block_stride = int64_t(H) * BS * D * 2;
  const char* kh = k_cache + int64_t(h) * BS * D * 2;
  const char* vh = v_cache + int64_t(h) * BS * D * 2;
  const uint32_t nb32 = uint32_t(min<int64_t>(num_blocks, INT32_MAX));
  constexpr int kBlk = kChunk / BS;
  const int ublk = wave_s * kRowsPerWave / BS;       // the wave's block within a chunk
  // Block id of the wave's rows of chunk c (0 past the context).
  auto block_of = [&](int c) -> int32_t {
    const int j = c * kBlk + ublk;
    return j * BS < L ? __builtin_amdgcn_readfirstlane(trow[j]) : 0;
  };
  auto issue = [&](int c, int32_t b, E* dk, E* dv) {
    const int j = c * kBlk + ublk;
    const int rows = min(max(L - j * BS, 0), BS);
    const bool in = uint32_t(b) < nb32;
    if (rows > 0 && !in) bad = true;
    const int64_t off = in ? int64_t(b) * block_stride : 0;
    const int n = in ? rows * D * 2 : 0;             // rows past the context read as zero
#pragma unroll
    for (int i = 0; i < kNl; ++i) {
      const int r0 = wave_s * kRowsPerWave + i * kRowsPerLoad;
      load_lds16(kh + off, n, koff[i], lds_address(dk + r0 * D));
      load_lds16(vh + off, n, voff[i], lds_address(dv + r0 * D));
    }
  };

  // Reader addresses (elements).  S^T operand of k-step k: row col, logical
  // column 2 k + hh.  V^T operand of tile t, k-step ks: lane j of its 16-lane
  // group G reads 4 keys from row r = 16 ks + 4 hh + j / 4 (+8) at dims
  // 32 t + 16 (G % 2) + 4 (j % 4): logical column 4 t + a, a = 2 (G % 2) +
  // (j % 4) / 2, swizzled to 4 (t ^ q) + a, where q = (r / kRb) % (kVpr / 4)
  // depends on j (and hh) only: 16 ks + 8 and 4 hh add whole multiples.
  int ka[kDSteps];
#pragma unroll
  for (int k = 0; k < kDSteps; ++k) ka[k] = col * D + 8 * ((2 * k + hh) ^ ((col / kRb) % kVpr));
  const int j16 = lane & 15;
  const int vr = 4 * hh + j16 / 4;
  const int qv = (vr / kRb) % (kVpr / 4);
  const int av = 2 * ((lane >> 4) & 1) + (j16 % 4) / 2;
  int vb[kDTiles];
#pragma unroll
  for (int t = 0; t < kDTiles; ++t) vb[t] = vr * D + 8 * (4 * (t ^ qv) + av) + 4 * (j16 % 2);

  auto compute = [&](int c, const E* sk, const E* sv) {
    const int k0 = c * kChunk;
    // Matrix products issue at raised wave priority, so that a wave with
    // products ready goes ahead of the other waves' softmax arithmetic on its
    // SIMD (measured 1-3 % faster).
    __builtin_amdgcn_s_setprio(1);
    // S^T (32 keys x 32 queries).
    f32x16 st;
#pragma unroll
    for (int e = 0; e < 16; ++e) st[e] = 0.f;
#pragma unroll
    for (int k = 0; k < kDSteps; ++k) {
      const frag a = __builtin_bit_cast(frag, *reinterpret_cast<const u32x4*>(sk + ka[k]));
      if constexpr (DT == PKV_BF16)
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[k], st, 0, 0, 0);
      else
        st = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[k], st, 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    // Mask, running max (in-lane over 16 keys, then across the lane halves).
    // The scale (> 0) keeps the order of scores, so the max is taken on the
    // raw products and the scale enters once per key, in the exponent's fma.
    float sc[16];
    if (k0 + kChunk - 1 > wave_first) {
      const int lim = qpos - k0 - 4 * hh;            // key k0 + 8 (e/4) + 4 hh + e%4 <= qpos
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = 8 * (e / 4) + e % 4 <= lim ? st[e] : -__builtin_inff();
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = st[e];
    }
    float rmax = sc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) rmax = fmaxf(rmax, sc[e]);
    const Halves hm = halves(rmax);
    rmax = fmaxf(hm.lo, hm.hi);
    const float bm = fmaxf(rmax * scale_log2, kEmptyMax);
    // The reference max moves only when the chunk's max exceeds it by more
    // than kLazy (base-2 units): until then p <= 2^kLazy, harmless in fp32 and
    // in the 16-bit P operand, and the softmax is the same for any reference.
    const float m_new = bm > m + kLazy ? bm : m;
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    frag pf[2];
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], scale_log2, -m_new));
      ps += pe;
      pf[e / 8][e % 8] = Mfma<DT>::from_f32(pe);
    }
    l = l * alpha + ps;
    if (c > 0 && __any(alpha != 1.f)) {           // chunk 0: acc is still zero
#pragma unroll
      for (int t = 0; t < kDTiles; ++t) acc[t] *= alpha;
    }
    __builtin_amdgcn_s_setprio(1);
    // O^T += V^T P^T: per 32-dim tile, two k-steps of 16 keys.
#pragma unroll
    for (int t = 0; t < kDTiles; ++t)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const E* p0 = sv + vb[t] + 16 * ks * D;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * D));
        const frag vf = __builtin_bit_cast(
            frag, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        if constexpr (DT == PKV_BF16)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], acc[t], 0, 0, 0);
        else
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[ks], acc[t], 0, 0, 0);
      }
    __builtin_amdgcn_s_setprio(0);
  };

  // Chunk c: wait for this wave's loads of chunk c (those of chunk c + 1 may
  // still be in flight), barrier (every wave's loads of c have landed and
  // every wave is done with chunk c - 1), start chunk c + 2 into the buffer
  // chunk c - 1 used, then compute.
  constexpr int kWaitOne = (2 * kNl) | (7 << 4) | (15 << 8);  // vmcnt(2 kNl), other counters free
  constexpr int kWaitAll = (7 << 4) | (15 << 8);              // vmcnt(0)
  // The block id of chunk c + 2 is read before the wait and the barrier,
  // which hide its latency; no scalar load is then in flight during the
  // compute (its LDS reads could only wait for all outstanding LDS and
  // scalar loads together).
  auto step = [&](int c, const E* sk, const E* sv, E* nk, E* nv) {
    const int32_t b = c + 2 < nchunks ? block_of(c + 2) : 0;
    if (c + 1 < nchunks)
      __builtin_amdgcn_s_waitcnt(kWaitOne);
    else
      __builtin_amdgcn_s_waitcnt(kWaitAll);
    __builtin_amdgcn_s_barrier();
    if (c + 2 < nchunks) issue(c + 2, b, nk, nv);
    if (c * kChunk <= wave_last) compute(c, sk, sv);
  };
  // Chunk 0's loads, then the query fragments, then a full wait: both are
  // needed first, and the compiler's own count of outstanding loads (it does
  // not see the loads to LDS) is then zero, so it adds no waits of its own
  // inside the loop.
  issue(0, block_of(0), lk0, lv0);
  {
    const E* qrow = static_cast<const E*>(q) + (int64_t(qa + (qi < P ? qi : 0)) * H + h) * D;
#pragma unroll
    for (int st = 0; st < kDSteps; ++st) {
      const u32x4 raw = qi < P ? *reinterpret_cast<const u32x4*>(qrow + 16 * st + 8 * hh) : u32x4{0, 0, 0, 0};
      qf[st] = __builtin_bit_cast(frag, raw);
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  if (nchunks > 1) issue(1, block_of(1), lk1, lv1);
  for (int c = 0; c < nchunks; c += 3) {
    step(c, lk0, lv0, lk2, lv2);
    if (c + 1 < nchunks) step(c + 1, lk1, lv1, lk0, lv0);
    if (c + 2 < nchunks) step(c + 2, lk2, lv2, lk1, lv1);
  }

  if (bad) sm_bad = 1;
  __syncthreads();
  const Halves hl = halves(l);
  const float lt = hl.lo + hl.hi;
  if (qi >= P) return;
  const float inv = sm_bad ? __builtin_nanf("") : 1.f / lt;
  // Lane (query, half hh) holds dims 32 t + 8 g + 4 hh + (0..3) of its
  // query.  Packed into 16-bit pairs and exchanged across the lane halves
  // (group g = 2 m with g = 2 m + 1), each lane ends with the 8 consecutive
  // dims 32 t + 16 m + 8 hh + (0..7) and writes them with one 16-byte store.
  E* orow = static_cast<E*>(out) + (int64_t(qa + qi) * H + h) * D;
#pragma unroll
  for (int t = 0; t < kDTiles; ++t)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const f32x16& a = acc[t];
      const uint32_t a0 = pack2<DT>(a[8 * m] * inv, a[8 * m + 1] * inv);
      const uint32_t a1 = pack2<DT>(a[8 * m + 2] * inv, a[8 * m + 3] * inv);
      const uint32_t b0 = pack2<DT>(a[8 * m + 4] * inv, a[8 * m + 5] * inv);
      const uint32_t b1 = pack2<DT>(a[8 * m + 6] * inv, a[8 * m + 7] * inv);
      const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
      *reinterpret_cast<u32x4*>(orow + 32 * t + 16 * m + 8 * hh) = u32x4{s0[0], s1[0], s0[1], s1[1]};
    }
}

template <int DT, int D, int BS>
hipError_t launch_prefill_typed(const PrefillArgs& a, hipStream_t stream) {
  if constexpr (DT == PKV_F32) {
    const int tiles = (a.max_query_len + kTileQ - 1) / kTileQ;
    const dim3 grid(unsigned(a.num_heads), unsigned(tiles), unsigned(a.num_seqs));
    hipLaunchKernelGGL((prefill_kernel<DT, D, BS>), grid, dim3(kThreads), 0, stream, a.q,
                       static_cast<const char*>(a.k_cache), static_cast<const char*>(a.v_cache), a.block_tables,
                       a.query_start, a.context_lens, a.out, a.num_blocks, a.max_blocks, tiles, a.scale_log2);
  } else {
    const int tiles = (a.max_query_len + kTileQ32 - 1) / kTileQ32;
    const int64_t pairs8 = (int64_t(a.num_heads) * a.num_seqs + 7) / 8 * 8;
    const dim3 grid(unsigned(pairs8 * tiles));
    hipLaunchKernelGGL((prefill32_kernel<DT, D, BS>), grid, dim3(64 * kWaves32), 0, stream, a.q,
                       static_cast<const char*>(a.k_cache), static_cast<const char*>(a.v_cache), a.block_tables,
                       a.query_start, a.context_lens, a.out, a.num_blocks, a.max_blocks, tiles, a.scale_log2,
                       a.num_heads, a.num_seqs);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_prefill_dt(int head_dim, int block_size, const PrefillArgs& a, hipStream_t stream) {
  if (head_dim == 64)
    return block_size == 16 ? launch_prefill_typed<DT, 64, 16>(a, stream) : launch_prefill_typed<DT, 64, 32>(a, stream);
  return block_size == 16 ? launch_prefill_typed<DT, 128, 16>(a, stream) : launch_prefill_typed<DT, 128, 32>(a, stream);
}

}  // namespace

int prefill_tile_queries(int dtype) { return dtype == PKV_F32 ? kTileQ : kTileQ32; }

hipError_t launch_prefill(int dtype, int head_dim, int block_size, const PrefillArgs& a, hipStream_t stream) {
  switch (dtype) {
    case PKV_F32: return launch_prefill_dt<PKV_F32>(head_dim, block_size, a, stream);
    case PKV_F16: return launch_prefill_dt<PKV_F16>(head_dim, block_size, a, stream);
    default: return launch_prefill_dt<PKV_BF16>(head_dim, block_size, a, stream);
  }
}

}  // namespace pkv
