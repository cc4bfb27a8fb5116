// HIP kernels for layerwise QK-Norm on gfx950 (CDNA4), and their launcher.
//
// Source of the operation: "SwiftQK: Fast and Communication-Efficient Tensor
// Parallelism for Query-Key Normalization" (arXiv 2608.09160v1).
//   - RMS-Norm, Eq. 1: y = x * gamma / sqrt(sum(x^2)/H + eps), one factor for
//     a token's whole Q vector and one for its whole K vector (layerwise).
//   - Phase A: per-shard squared sums, combined in FP32.
//   - Phase B and the final scaling: x * gamma, then times the RMS factor;
//     only the final result is written to memory.
//
// One kernel template, qknorm_rows, serves the three layerwise entry points
// (MODE_FUSED, MODE_STATS, MODE_APPLY) so that the per-shard sums are
// produced by the same instructions in every mode, which is what makes the
// fused call and the split calls agree bit for bit. qknorm_heads_packed and
// qknorm_heads serve the headwise entry point (the introduction's per-head
// granularity) with the same load, convert, scale and store helpers.
//
// This is a streaming, HBM-bound operation (about 1 flop per byte): there is
// no contraction, so no MFMA. What matters is that every Q/K element is read
// once with a 16-byte load, kept in registers through the reduction, and
// written once with a 16-byte store, with enough loads in flight per CU.
//
// Work layout (see Plan in qknorm_internal.hpp): G = S * L threads handle
// one token; the L lanes of shard group s own the 16-byte chunks of Q shard
// s followed by K shard s, lane m taking chunks m, m+L, m+2L, ... (`slots`
// of them, about three). A block holds one or a few tokens side by side
// (narrow rows: several tokens per wave) and there is one block per such
// group of tokens, so many independent tokens have their loads in flight on
// every CU; gamma is reloaded per block from the caches (it is small and
// shared by all tokens).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>
#include <string>

#include "qknorm_internal.hpp"

namespace qkn {
namespace {

// I/O types. kVW: elements per 16-byte row chunk; kBytes: bytes per row
// element; kGW / kGBytes: 32-bit words of gamma per chunk and bytes per gamma
// element (FP8 rows take bf16 gamma).
struct BF16 {
  static constexpr int kVW = 8, kBytes = 2, kGW = 4, kGBytes = 2, kDtype = kDtypeBF16;
};
struct F32 {
  static constexpr int kVW = 4, kBytes = 4, kGW = 4, kGBytes = 4, kDtype = kDtypeF32;
};
struct FP8 {  // OCP FP8 E4M3 (E4M3FN) rows, bf16 gamma
  static constexpr int kVW = 16, kBytes = 1, kGW = 8, kGBytes = 2, kDtype = kDtypeFP8;
};

template <int W>
struct Words {
  uint32_t w[W];
};
using Chunk = Words<4>;  // 16 bytes of row data
template <class IO>
using GChunk = Words<IO::kGW>;  // the gamma of one chunk

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// All elements of a row chunk as float32 (exact widening).
template <class IO>
__device__ __forceinline__ void decode(const Chunk& c, float (&v)[IO::kVW]);
template <>
__device__ __forceinline__ void decode<BF16>(const Chunk& c, float (&v)[8]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    v[2 * p] = bf16_lo(c.w[p]);
    v[2 * p + 1] = bf16_hi(c.w[p]);
  }
}
template <>
__device__ __forceinline__ void decode<F32>(const Chunk& c, float (&v)[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) v[p] = __uint_as_float(c.w[p]);
}
template <>
__device__ __forceinline__ void decode<FP8>(const Chunk& c, float (&v)[16]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {  // v_cvt_pk_f32_fp8: two E4M3 values of one 16-bit half per instruction
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(c.w[p], false);
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(c.w[p], true);
    v[4 * p] = lo[0];
    v[4 * p + 1] = lo[1];
    v[4 * p + 2] = hi[0];
    v[4 * p + 3] = hi[1];
  }
}

// The gamma of a chunk as float32 (exact).
template <class IO>
__device__ __forceinline__ void decode_gamma(const GChunk<IO>& g, float (&v)[IO::kVW]) {
  if (IO::kGBytes == 2) {
#pragma unroll
    for (int p = 0; p < IO::kGW; ++p) {
      v[2 * p] = bf16_lo(g.w[p]);
      v[2 * p + 1] = bf16_hi(g.w[p]);
    }
  } else {
#pragma unroll
    for (int p = 0; p < IO::kGW; ++p) v[p] = __uint_as_float(g.w[p]);
  }
}

// float32 results -> a chunk of the I/O type, one rounding to nearest even.
// For FP8 the caller saturates to +-448 first where needed (sat_e4m3; NaN
// stays NaN): the hardware conversion turns magnitudes past 464 into NaN.
template <class IO>
__device__ __forceinline__ void pack(Chunk& c, const float (&v)[IO::kVW]);
template <>
__device__ __forceinline__ void pack<BF16>(Chunk& c, const float (&v)[8]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const f32x2_t f = {v[2 * p], v[2 * p + 1]};
    c.w[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
  }
}
template <>
__device__ __forceinline__ void pack<F32>(Chunk& c, const float (&v)[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) c.w[p] = __float_as_uint(v[p]);
}
__device__ __forceinline__ float sat_e4m3(float x) { return x > 448.0f ? 448.0f : (x < -448.0f ? -448.0f : x); }
template <>
__device__ __forceinline__ void pack<FP8>(Chunk& c, const float (&v)[16]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * p], v[4 * p + 1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * p + 2], v[4 * p + 3], w, true);
    c.w[p] = (uint32_t)w;
  }
}

// Loads `W` words at `p`: 16-byte loads (p 16-byte aligned) on the aligned
// path; on the element-wise path the first `n` elements of `esz` bytes, the
// rest reading as 0.
//
// Every load is unconditional: a lane whose slot is idle passes the row's
// first chunk (always a valid address) and its value is masked by the caller.
// Predicated loads would put each load in its own branch with a wait for it
// before the join, leaving one load in flight per wave.
template <int W, int ESZ, bool ALIGNED>
__device__ __forceinline__ Words<W> load_words(const char* p, int n) {
  Words<W> c;
#pragma unroll
  for (int q = 0; q < W; ++q) c.w[q] = 0u;
  if (ALIGNED) {
#pragma unroll
    for (int q = 0; q < W; q += 4) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p + 4 * q);
      c.w[q] = v.x;
      c.w[q + 1] = v.y;
      c.w[q + 2] = v.z;
      c.w[q + 3] = v.w;
    }
  } else {
    constexpr int kElems = W * 4 / ESZ;
#pragma unroll
    for (int e = 0; e < kElems; ++e) {
      const int ee = e < n ? e : 0;
      uint32_t v;
      if (ESZ == 1) v = reinterpret_cast<const uint8_t*>(p)[ee];
      else if (ESZ == 2) v = reinterpret_cast<const uint16_t*>(p)[ee];
      else v = reinterpret_cast<const uint32_t*>(p)[ee];
      c.w[(e * ESZ) / 4] |= (e < n ? v : 0u) << (((e * ESZ) % 4) * 8);
    }
  }
  return c;
}

// The chunk at element offset `col` of row `row` (the first `n` elements on
// the element-wise path).
template <class IO, bool ALIGNED>
__device__ __forceinline__ Chunk load_chunk(const char* row, int col, int n) {
  return load_words<4, IO::kBytes, ALIGNED>(row + (int64_t)col * IO::kBytes, n);
}

// The gamma of the chunk at column `col`, from gamma base `base`.
template <class IO, bool ALIGNED>
__device__ __forceinline__ GChunk<IO> load_gamma(const char* base, int col, int n) {
  return load_words<IO::kGW, IO::kGBytes, ALIGNED>(base + (int64_t)col * IO::kGBytes, n);
}

// Stores the first `n` elements of a chunk. Results are written once and not
// read again by this kernel, so the 16-byte path marks them non-temporal
// (streamed past the caches), which measured faster on MI355X.
template <class IO, bool ALIGNED>
__device__ __forceinline__ void store_chunk(char* row, int col, int n, const Chunk& c) {
  char* p = row + (int64_t)col * IO::kBytes;
  if (ALIGNED) {
    const u32x4_t v = {c.w[0], c.w[1], c.w[2], c.w[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
  } else {
#pragma unroll
    for (int e = 0; e < IO::kVW; ++e) {
      if (e < n) {
        const uint32_t v = c.w[(e * IO::kBytes) / 4] >> (((e * IO::kBytes) % 4) * 8);
        if (IO::kBytes == 1) reinterpret_cast<uint8_t*>(p)[e] = (uint8_t)v;
        else if (IO::kBytes == 2) reinterpret_cast<uint16_t*>(p)[e] = (uint16_t)v;
        else reinterpret_cast<uint32_t*>(p)[e] = v;
      }
    }
  }
}

// Sum of squares of one chunk, in element order (Phase A, in-lane part).
template <class IO>
__device__ __forceinline__ float chunk_sumsq(const Chunk& c) {
  float v[IO::kVW];
  decode<IO>(c, v);
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < IO::kVW; ++e) s = __builtin_fmaf(v[e], v[e], s);
  return s;
}

// Largest magnitude of N values (NaN if any is NaN): one three-operand
// maximum per two elements.
template <int N>
__device__ __forceinline__ float max_abs(const float (&v)[N]) {
  float m = __builtin_fabsf(v[0]);
#pragma unroll
  for (int e = 1; e + 1 < N; e += 2)
    m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, __builtin_fabsf(v[e])), __builtin_fabsf(v[e + 1]));
  if (N % 2 == 0) m = __builtin_elementwise_maximum(m, __builtin_fabsf(v[N - 1]));
  return m;
}

// Phase B and the final scaling for this lane's chunks of one token:
// y = (x * gamma) * r[i], one rounding to the I/O type, stores of the valid
// chunks (slot i goes to the Q or the K row). For FP8 the saturating
// conversion costs four operations per element, so with up to 4 slots the
// wave first checks whether any result exceeds 448 in magnitude or is NaN,
// and clamps only then.
template <class IO, int V, bool ALIGNED>
__device__ __forceinline__ void scale_store(const Chunk (&xv)[V], const GChunk<IO> (&g)[V], const float (&r)[V],
                                            const bool (&isq)[V], const int (&col)[V], const int (&cnt)[V],
                                            char* yq_row, char* yk_row, bool active) {
  constexpr int VW = IO::kVW;
  if (IO::kDtype == kDtypeFP8 && V <= 4) {
    float y[V][VW];
    float big = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float xf[VW], gf[VW];
      decode<IO>(xv[i], xf);
      decode_gamma<IO>(g[i], gf);
#pragma unroll
      for (int e = 0; e < VW; ++e) y[i][e] = (xf[e] * gf[e]) * r[i];
      if (cnt[i] > 0) big = __builtin_elementwise_maximum(big, max_abs(y[i]));  // idle slots left out
    }
    // A NaN (from gamma, say) sends the wave through the saturating path too,
    // which keeps NaN and clamps the rest.
    const bool clamp = __builtin_amdgcn_ballot_w64(active && !(big <= 448.0f)) != 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      if (clamp) {
#pragma unroll
        for (int e = 0; e < VW; ++e) y[i][e] = sat_e4m3(y[i][e]);
      }
      Chunk out;
      pack<IO>(out, y[i]);
      if (active && cnt[i] > 0) store_chunk<IO, ALIGNED>(isq[i] ? yq_row : yk_row, col[i], cnt[i], out);
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      if (active && cnt[i] > 0) {
        float xf[VW], gf[VW], y[VW];
        decode<IO>(xv[i], xf);
        decode_gamma<IO>(g[i], gf);
#pragma unroll
        for (int e = 0; e < VW; ++e) {
          y[e] = (xf[e] * gf[e]) * r[i];
          if (IO::kDtype == kDtypeFP8) y[e] = sat_e4m3(y[e]);  // many slots: clamp unconditionally
        }
        Chunk out;
        pack<IO>(out, y);
        store_chunk<IO, ALIGNED>(isq[i] ? yq_row : yk_row, col[i], cnt[i], out);
      }
    }
  }
}

// RMS factor of Eq. 1 for a global squared sum `ss`, full width H given as
// inv_div = 1/H (rounded once on the host): r = rsq(fma(ss, 1/H, eps)) with
// the hardware reciprocal square root (1 ulp). Where m = ss/H + eps falls
// below the float32 normal range, a subnormal m would keep too few bits, so
// m is formed again from ss * 2^64 and eps * 2^64 (both exact there) and r is
// scaled back by 2^32: one rounding in the normal range, as everywhere else.
// 0 gives +inf and +inf gives 0, as the formula does.
__device__ __forceinline__ float rms_factor(float ss, float inv_div, float eps) {
  float m = __builtin_fmaf(ss, inv_div, eps);
  const bool tiny = m < 1.17549435e-38f;  // false for NaN
  if (tiny) m = __builtin_fmaf(ss * 0x1p64f, inv_div, eps * 0x1p64f);
  const float r = __builtin_amdgcn_rsqf(m);
  return tiny ? r * 0x1p32f : r;
}

// Register-pressure guard: empty asm statements that claim to rewrite the
// words of `c`. Values the compiler widened from them earlier (bf16 or fp8 ->
// float32) can then not be kept alive across this point and are widened
// again where they are used, so packed data stays packed in registers.
template <int W>
__device__ __forceinline__ void keep_packed(Words<W>& c) {
#pragma unroll
  for (int q = 0; q < W; ++q) asm volatile("" : "+v"(c.w[q]));
}

// Sum over aligned groups of `group` lanes (a power of two, 1..64); every
// lane of a group ends with the same value. Inside a 16-lane row the steps
// are DPP moves fused into the adds (quad permutes, then the half-row and
// row mirrors, which pair lanes of the two halves once each half is
// uniform). The 16- and 32-lane steps cross rows with gfx950's permlane
// swaps (measured faster than the LDS crossbar for every I/O type):
// swapping the odd rows (or the upper half) of one copy with the even rows
// (lower half) of another leaves row pairs (halves) side by side in the two
// results, so one add gives every lane the pair's sum. Each step adds two
// lanes' values, a + b on one and b + a (or a + b) on the other, so all
// lanes of a group hold bitwise the same sum.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float swap_add16(float v) {  // lanes i ^ 16
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float swap_add32(float v) {  // lanes i ^ 32
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int GROUP>
__device__ __forceinline__ float group_sum_of(float v) {
  if (GROUP > 1) v += dpp_move<0xB1>(v);    // lanes i ^ 1   (quad_perm 1,0,3,2)
  if (GROUP > 2) v += dpp_move<0x4E>(v);    // lanes i ^ 2   (quad_perm 2,3,0,1)
  if (GROUP > 4) v += dpp_move<0x141>(v);   // lanes 7 - i within 8 (row_half_mirror)
  if (GROUP > 8) v += dpp_move<0x140>(v);   // lanes 15 - i within 16 (row_mirror)
  if (GROUP > 16) v = swap_add16(v);
  if (GROUP > 32) v = swap_add32(v);
  return v;
}

// The group width is uniform over the launch: one test picks the straight
// sequence of steps (a test per step compiled to a branch and a
// materialised condition each, for every token).
__device__ __forceinline__ float group_sum(float v, int group) {
  if (group == 64) return group_sum_of<64>(v);  // most launches: tested first
  switch (group) {
    case 32: return group_sum_of<32>(v);
    case 16: return group_sum_of<16>(v);
    case 8: return group_sum_of<8>(v);
    case 4: return group_sum_of<4>(v);
    case 2: return group_sum_of<2>(v);
    default: return v;
  }
}

__device__ __forceinline__ float lane_read(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

template <class IO, int V, int MODE, bool ALIGNED>
__global__ void __launch_bounds__(max_threads_for_slots(V, IO::kDtype, ALIGNED)) qknorm_rows(const RowArgs a) {
  extern __shared__ float red[];  // [2 buffers][tokens per block][groups per token] float2 (Q, K)
  constexpr int VW = IO::kVW;
  const int tid = threadIdx.x;
  const int G = a.tok_threads;
  const int L = a.lanes;
  // Tokens share a block only when each takes a power-of-two share of one
  // wave (64 lanes, or 4..32 so that several tokens share a wave), and shards
  // share a token only with power-of-two lane groups, so the lane
  // decomposition is shifts and masks.
  const int j = a.tokens_per_block > 1 ? tid >> a.log2_tok : 0;   // token slot within the block
  const int r = a.tokens_per_block > 1 ? tid & (G - 1) : tid;     // thread within the token
  const int s = a.shards > 1 ? r >> a.log2_lanes : 0;     // shard group
  const int m = a.shards > 1 ? r & (L - 1) : r;           // lane within the group
  const int qbase = __umul24(s, a.hq_s), kbase = __umul24(s, a.hk_s);

  // Token-invariant geometry of this lane's chunk slots.
  bool isq[V];
  int col[V];
  int cnt[V];
  // Selects rather than branches: an idle slot (u past the last chunk) reads
  // and ignores the first chunk of the Q row.
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int u = i * L + m;
    const bool q = u < a.ncq;
    const bool idle = u >= a.ncq + a.nck;
    const int c = (q ? u : u - a.ncq) * VW;
    isq[i] = q || idle;
    col[i] = idle ? 0 : (q ? qbase : kbase) + c;
    cnt[i] = idle ? 0 : ALIGNED ? VW : min(VW, (q ? a.hq_s : a.hk_s) - c);
  }

  GChunk<IO> g[MODE == MODE_STATS ? 1 : V];
  if (MODE != MODE_STATS) {
#pragma unroll
    for (int i = 0; i < V; ++i)
      g[i] = load_gamma<IO, ALIGNED>(static_cast<const char*>(isq[i] ? a.gq : a.gk), col[i], max(cnt[i], 1));
  }

  const int group = a.group;            // butterfly width: min(L, 64)
  const int gps = a.groups_per_shard;   // L / group
  const int gpt = a.groups_per_token;   // G / group
  const int tpb = a.tokens_per_block;
  const int64_t step = (int64_t)gridDim.x * tpb;
  int buf = 0;

  // The loop bound is uniform over the block (barriers inside); a token slot
  // past the end reads a valid row and writes nothing.
  for (int64_t tb = (int64_t)blockIdx.x * tpb; tb < a.T; tb += step) {
    const int64_t t = tb + j;
    const bool active = t < a.T;
    const int64_t tr = active ? t : a.T - 1;
    const char* xq_row = static_cast<const char*>(a.xq) + tr * a.ldxq * IO::kBytes;
    const char* xk_row = static_cast<const char*>(a.xk) + tr * a.ldxk * IO::kBytes;

    Chunk xv[V];
#pragma unroll
    for (int i = 0; i < V; ++i) xv[i] = load_chunk<IO, ALIGNED>(isq[i] ? xq_row : xk_row, col[i], max(cnt[i], 1));
    if (MODE != MODE_STATS && IO::kBytes < 4) {
#pragma unroll
      for (int i = 0; i < V; ++i) keep_packed(g[i]);
    }

    float ssq = 0.0f, ssk = 0.0f;
    if (MODE != MODE_APPLY) {
      // Phase A, in-lane: slot by slot, each chunk summed in element order.
      float aq = 0.0f, ak = 0.0f;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const float cs = cnt[i] > 0 ? chunk_sumsq<IO>(xv[i]) : 0.0f;
        aq += isq[i] ? cs : 0.0f;
        ak += isq[i] ? 0.0f : cs;
      }
      // Across the lanes of a group: every lane ends with the group's sum.
      aq = group_sum(aq, group);
      ak = group_sum(ak, group);
      if (G <= 64) {
        // One wave per token: group s is shard s; its sum sits in lane s*L.
        // Several tokens per wave (one shard each): the group is the token.
        if (MODE == MODE_STATS) {
          if (m == 0 && active) {
            a.partials[(int64_t)(2 * s) * a.T + t] = aq;
            a.partials[(int64_t)(2 * s + 1) * a.T + t] = ak;
          }
        } else if (G < 64) {
          ssq = aq;
          ssk = ak;
        } else {
          ssq = lane_read(aq, 0);
          ssk = lane_read(ak, 0);
          for (int sh = 1; sh < a.shards; ++sh) {
            ssq += lane_read(aq, sh * L);
            ssk += lane_read(ak, sh * L);
          }
        }
      } else {
        // Several waves per token: group sums meet in LDS (double-buffered
        // by iteration, so one barrier per iteration suffices). Lane q of
        // every wave then reads group q's pair (at most 64 groups per token),
        // and each wave adds them lane by lane, group by group within a
        // shard and then shard by shard, with no LDS wait per group.
        float2* rb = reinterpret_cast<float2*>(red) + (buf * tpb + j) * gpt;
        if ((r & (group - 1)) == 0) rb[r >> a.log2_group] = make_float2(aq, ak);
        __syncthreads();
        const int lane = tid & 63;
        const float2 pv = rb[lane < gpt ? lane : 0];
        float mq = 0.0f, mk = 0.0f;  // partial_stats: the sums of shard r
        for (int sh = 0, q0 = 0; sh < a.shards; ++sh, q0 += gps) {
          float pq = lane_read(pv.x, q0), pk = lane_read(pv.y, q0);
          for (int q = 1; q < gps; ++q) {
            pq += lane_read(pv.x, q0 + q);
            pk += lane_read(pv.y, q0 + q);
          }
          if (MODE == MODE_STATS) {
            mq = r == sh ? pq : mq;
            mk = r == sh ? pk : mk;
          } else {
            ssq = sh == 0 ? pq : ssq + pq;
            ssk = sh == 0 ? pk : ssk + pk;
          }
        }
        if (MODE == MODE_STATS && r < a.shards && active) {
          a.partials[(int64_t)(2 * r) * a.T + t] = mq;
          a.partials[(int64_t)(2 * r + 1) * a.T + t] = mk;
        }
        buf ^= 1;
      }
    } else {
      // Statistics from outside: planes added in order (the combination step).
      ssq = a.stats[tr];
      ssk = a.stats[a.T + tr];
      for (int p = 1; p < a.n_planes; ++p) {
        ssq += a.stats[(int64_t)(2 * p) * a.T + tr];
        ssk += a.stats[(int64_t)(2 * p + 1) * a.T + tr];
      }
    }

    if constexpr (MODE != MODE_STATS) {
      // Packed rows widened once for the sums are widened again for the
      // scaling above a few slots (bf16: 2, FP8: 4), so that only the packed
      // words stay live across the exchange: fewer registers, more waves.
      if (IO::kBytes < 4 && V > (IO::kBytes == 2 ? 2 : 4)) {
#pragma unroll
        for (int i = 0; i < V; ++i) keep_packed(xv[i]);
      }
      const float rq = rms_factor(ssq, a.inv_divq, a.eps);
      const float rk = rms_factor(ssk, a.inv_divk, a.eps);
      float rr[V];
#pragma unroll
      for (int i = 0; i < V; ++i) rr[i] = isq[i] ? rq : rk;
      char* yq_row = static_cast<char*>(a.yq) + tr * a.ldyq * IO::kBytes;
      char* yk_row = static_cast<char*>(a.yk) + tr * a.ldyk * IO::kBytes;
      scale_store<IO, V, ALIGNED>(xv, g, rr, isq, col, cnt, yq_row, yk_row, active);
    }
  }
}

// Headwise QK-Norm (the introduction's per-head granularity): Eq. 1 for every
// head of head_dim columns, H = head_dim, with no combination across heads.
// Head g of a token (Q heads first, then K heads) is owned by an aligned group
// of L lanes; lane m takes the head's chunks m, m+L, ... The group sum leaves
// the head's sum of squares in all L lanes, so no LDS and no barrier are
// needed. Blocks are rounded up to whole waves; lanes past the last token
// slot only read valid addresses and write nothing.
template <class IO, int V, bool ALIGNED>
__global__ void __launch_bounds__(max_threads_for_slots(V, IO::kDtype, ALIGNED)) qknorm_heads(const HeadArgs a) {
  constexpr int VW = IO::kVW;
  const int tid = threadIdx.x;
  const int G = a.tok_threads;
  const int L = a.lanes;
  const int j = tid / G;                       // token slot within the block
  const int r = tid - j * G;
  const bool live = j < a.tokens_per_block;    // false for the round-up lanes
  const int seg = r / L;                       // head within the token
  const int m = r - seg * L;
  const bool isq = seg < a.heads_q;
  const int head = isq ? seg : seg - a.heads_q;

  int col[V], gcol[V], cnt[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int u = i * L + m;
    if (live && u < a.nc) {
      const int c = u * VW;
      col[i] = head * a.head_dim + c;
      gcol[i] = c;
      cnt[i] = min(VW, a.head_dim - c);
    } else {  // idle slot: reads (and ignores) the first chunk of the row and of the head's gamma
      col[i] = 0;
      gcol[i] = 0;
      cnt[i] = 0;
    }
  }
  // this head's gamma (head * stride elements in; the first head's for stride 0)
  const char* gbase = static_cast<const char*>(isq ? a.gq : a.gk) + (int64_t)head * a.gstride * IO::kGBytes;
  const char* xbase = static_cast<const char*>(isq ? a.xq : a.xk);
  char* ybase = static_cast<char*>(isq ? a.yq : a.yk);
  const int64_t ldx = isq ? a.ldxq : a.ldxk;
  const int64_t ldy = isq ? a.ldyq : a.ldyk;

  GChunk<IO> g[V];
#pragma unroll
  for (int i = 0; i < V; ++i) g[i] = load_gamma<IO, ALIGNED>(gbase, gcol[i], max(cnt[i], 1));

  const int tpb = a.tokens_per_block;
  const int64_t step = (int64_t)gridDim.x * tpb;
  for (int64_t tb = (int64_t)blockIdx.x * tpb; tb < a.T; tb += step) {
    const int64_t t = tb + j;
    const bool active = live && t < a.T;
    const int64_t tr = t < a.T ? t : a.T - 1;
    const char* x_row = xbase + tr * ldx * IO::kBytes;

    Chunk xv[V];
#pragma unroll
    for (int i = 0; i < V; ++i) xv[i] = load_chunk<IO, ALIGNED>(x_row, col[i], max(cnt[i], 1));
    if (IO::kBytes < 4) {
#pragma unroll
      for (int i = 0; i < V; ++i) keep_packed(g[i]);
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) acc += cnt[i] > 0 ? chunk_sumsq<IO>(xv[i]) : 0.0f;
    acc = group_sum(acc, L);

    {
      if (IO::kBytes < 4 && V > (IO::kBytes == 2 ? 2 : 4)) {
#pragma unroll
        for (int i = 0; i < V; ++i) keep_packed(xv[i]);
      }
      const float f = rms_factor(acc, a.inv_div, a.eps);
      float rr[V];
      bool isqv[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        rr[i] = f;
        isqv[i] = true;
      }
      char* y_row = ybase + tr * ldy * IO::kBytes;
      scale_store<IO, V, ALIGNED>(xv, g, rr, isqv, col, cnt, y_row, y_row, active);
    }
  }
}

// Headwise QK-Norm when a head is a power-of-two number of chunks (up to 64,
// e.g. 128 bf16 = 16 chunks): the token's chunks (Q heads, then K heads) are
// laid over G lanes exactly as in the layerwise kernel, lane m of slot i
// taking chunk i*G + m, so every load instruction reads consecutive 16-byte
// chunks. Because G is a multiple of the head's chunk count nc, the nc
// consecutive lanes of a slot hold exactly one head: each slot is reduced
// over its aligned nc-lane group and scaled by that head's factor.
template <class IO, int V, bool ALIGNED>
__global__ void __launch_bounds__(max_threads_for_slots(V, IO::kDtype, ALIGNED)) qknorm_heads_packed(const HeadArgs a) {
  constexpr int VW = IO::kVW;
  const int tid = threadIdx.x;
  const int G = a.tok_threads;                 // lanes per token, a multiple of 64 and of nc
  const int nc = a.lanes;                      // chunks per head (power of two, <= 64)
  const int j = a.tokens_per_block > 1 ? tid >> 6 : 0;  // token slot (several only with G = 64)
  const int m = a.tokens_per_block > 1 ? tid & 63 : tid;
  const int total = (a.heads_q + a.heads_k) * nc;

  bool isq[V];
  int col[V], cnt[V];
  const char* gp[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int u = i * G + m;
    if (u < total) {
      const int head = u >> a.log2_nc;
      const int c = (u & (nc - 1)) * VW;
      isq[i] = head < a.heads_q;
      const int hh = isq[i] ? head : head - a.heads_q;
      col[i] = __umul24(hh, a.head_dim) + c;
      cnt[i] = ALIGNED ? VW : min(VW, a.head_dim - c);
      gp[i] = static_cast<const char*>(isq[i] ? a.gq : a.gk) + ((int64_t)hh * a.gstride + c) * IO::kGBytes;
    } else {  // idle slot: reads (and ignores) the first chunk of the Q row and of gamma
      isq[i] = true;
      col[i] = 0;
      cnt[i] = 0;
      gp[i] = static_cast<const char*>(a.gq);
    }
  }
  GChunk<IO> g[V];
#pragma unroll
  for (int i = 0; i < V; ++i) g[i] = load_gamma<IO, ALIGNED>(gp[i], 0, max(cnt[i], 1));

  const int tpb = a.tokens_per_block;
  const int64_t step = (int64_t)gridDim.x * tpb;
  for (int64_t tb = (int64_t)blockIdx.x * tpb; tb < a.T; tb += step) {
    const int64_t t = tb + j;
    const bool active = t < a.T;
    const int64_t tr = active ? t : a.T - 1;
    const char* xq_row = static_cast<const char*>(a.xq) + tr * a.ldxq * IO::kBytes;
    const char* xk_row = static_cast<const char*>(a.xk) + tr * a.ldxk * IO::kBytes;
    Chunk xv[V];
#pragma unroll
    for (int i = 0; i < V; ++i) xv[i] = load_chunk<IO, ALIGNED>(isq[i] ? xq_row : xk_row, col[i], max(cnt[i], 1));
    if (IO::kBytes < 4) {
#pragma unroll
      for (int i = 0; i < V; ++i) keep_packed(g[i]);
    }
    float ss[V];
#pragma unroll
    for (int i = 0; i < V; ++i) ss[i] = group_sum(cnt[i] > 0 ? chunk_sumsq<IO>(xv[i]) : 0.0f, nc);

    {
      if (IO::kBytes < 4 && V > (IO::kBytes == 2 ? 2 : 4)) {
#pragma unroll
        for (int i = 0; i < V; ++i) keep_packed(xv[i]);
      }
      float rr[V];
#pragma unroll
      for (int i = 0; i < V; ++i) rr[i] = rms_factor(ss[i], a.inv_div, a.eps);
      char* yq_row = static_cast<char*>(a.yq) + tr * a.ldyq * IO::kBytes;
      char* yk_row = static_cast<char*>(a.yk) + tr * a.ldyk * IO::kBytes;
      scale_store<IO, V, ALIGNED>(xv, g, rr, isq, col, cnt, yq_row, yk_row, active);
    }
  }
}

using KernelFn = void (*)(const RowArgs);
using HeadKernelFn = void (*)(const HeadArgs);

constexpr int64_t kMaxGrid = (int64_t)1 << 30;

// Largest grid a launch uses: kMaxGrid, or a smaller cap from the
// QKNORM_MAX_GRID environment variable (read at each launch), under which
// blocks loop over several token groups; tests use it to run that loop.
int64_t grid_cap() {
  const char* e = std::getenv("QKNORM_MAX_GRID");
  const long long v = e ? std::atoll(e) : 0;
  return v > 0 && v < kMaxGrid ? (int64_t)v : kMaxGrid;
}

template <class IO, int MODE, bool ALIGNED>
KernelFn pick_slots(int v) {
  switch (v) {
    case 1: return qknorm_rows<IO, 1, MODE, ALIGNED>;
    case 2: return qknorm_rows<IO, 2, MODE, ALIGNED>;
    case 3: return qknorm_rows<IO, 3, MODE, ALIGNED>;
    case 4: return qknorm_rows<IO, 4, MODE, ALIGNED>;
    case 6: return qknorm_rows<IO, 6, MODE, ALIGNED>;
    case 8: return qknorm_rows<IO, 8, MODE, ALIGNED>;
  }
  if constexpr (max_slots(IO::kDtype, ALIGNED) == kMaxSlots) {
    if (v == 12) return qknorm_rows<IO, 12, MODE, ALIGNED>;
    if (v == 16) return qknorm_rows<IO, 16, MODE, ALIGNED>;
  }
  return nullptr;
}

template <class IO, int MODE>
KernelFn pick_aligned(bool aligned, int v) {
  return aligned ? pick_slots<IO, MODE, true>(v) : pick_slots<IO, MODE, false>(v);
}

template <class IO>
KernelFn pick_mode(int mode, bool aligned, int v) {
  switch (mode) {
    case MODE_FUSED: return pick_aligned<IO, MODE_FUSED>(aligned, v);
    case MODE_STATS: return pick_aligned<IO, MODE_STATS>(aligned, v);
    case MODE_APPLY: return pick_aligned<IO, MODE_APPLY>(aligned, v);
  }
  return nullptr;
}

template <class IO, bool ALIGNED, bool PACKED>
HeadKernelFn pick_head_slots(int v) {
#define QKN_HEAD_KERNEL(V) (PACKED ? qknorm_heads_packed<IO, V, ALIGNED> : qknorm_heads<IO, V, ALIGNED>)
  switch (v) {
    case 1: return QKN_HEAD_KERNEL(1);
    case 2: return QKN_HEAD_KERNEL(2);
    case 3: return QKN_HEAD_KERNEL(3);
    case 4: return QKN_HEAD_KERNEL(4);
    case 6: return QKN_HEAD_KERNEL(6);
    case 8: return QKN_HEAD_KERNEL(8);
  }
  if constexpr (max_slots(IO::kDtype, ALIGNED) == kMaxSlots) {
    if (v == 12) return QKN_HEAD_KERNEL(12);
    if (v == 16) return QKN_HEAD_KERNEL(16);
  }
#undef QKN_HEAD_KERNEL
  return nullptr;
}

template <class IO>
HeadKernelFn pick_head_io(const Plan& p) {
  if (p.heads_packed)
    return p.aligned ? pick_head_slots<IO, true, true>(p.slots) : pick_head_slots<IO, false, true>(p.slots);
  return p.aligned ? pick_head_slots<IO, true, false>(p.slots) : pick_head_slots<IO, false, false>(p.slots);
}

HeadKernelFn pick_head_kernel(const Plan& p) {
  switch (p.dtype) {
    case kDtypeBF16: return pick_head_io<BF16>(p);
    case kDtypeF32: return pick_head_io<F32>(p);
    case kDtypeFP8: return pick_head_io<FP8>(p);
  }
  return nullptr;
}

KernelFn pick_kernel(const Plan& p) {
  switch (p.dtype) {
    case kDtypeBF16: return pick_mode<BF16>(p.mode, p.aligned, p.slots);
    case kDtypeF32: return pick_mode<F32>(p.mode, p.aligned, p.slots);
    case kDtypeFP8: return pick_mode<FP8>(p.mode, p.aligned, p.slots);
  }
  return nullptr;
}

}  // namespace

int launch(const Plan& p, const RowArgs& args, void* stream, std::string* err) {
  KernelFn fn = pick_kernel(p);
  if (!fn) {
    *err = "no kernel compiled for " + describe(p);
    return (int)hipErrorInvalidValue;
  }
  // One block per tokens_per_block tokens; the kernel's token loop covers
  // any remainder beyond the largest grid.
  const int64_t blocks = (args.T + p.tokens_per_block - 1) / p.tokens_per_block;
  const int64_t cap = grid_cap();
  const int64_t grid = blocks < cap ? blocks : cap;
  // hipLaunchKernel returns this launch's own status (no sticky error from
  // an earlier, unrelated call is reported as ours).
  RowArgs a = args;
  void* kargs[] = {&a};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)grid),
                                       dim3((unsigned)p.threads), kargs, (size_t)p.lds_bytes,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    *err = std::string("kernel launch: ") + hipGetErrorString(e);
    return (int)e;
  }
  return 0;
}

}  // namespace qkn

namespace qkn {

int launch_heads(const Plan& p, const HeadArgs& args, void* stream, std::string* err) {
  HeadKernelFn fn = pick_head_kernel(p);
  if (!fn) {
    *err = "no kernel compiled for " + describe(p);
    return (int)hipErrorInvalidValue;
  }
  const int64_t blocks = (args.T + p.tokens_per_block - 1) / p.tokens_per_block;
  const int64_t cap = grid_cap();
  const int64_t grid = blocks < cap ? blocks : cap;
  HeadArgs a = args;
  void* kargs[] = {&a};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)grid),
                                       dim3((unsigned)p.threads), kargs, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    *err = std::string("kernel launch: ") + hipGetErrorString(e);
    return (int)e;
  }
  return 0;
}

}  // namespace qkn
