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
// One kernel template serves the three entry points (MODE_FUSED,
// MODE_STATS, MODE_APPLY) so that the per-shard sums are produced by the
// same instructions in every mode, which is what makes the fused call and
// the split calls agree bit for bit.
//
// This is a streaming, HBM-bound operation (about 1 flop per byte): there is
// no contraction, so no MFMA. What matters is that every Q/K element is read
// once with a 16-byte load, kept in registers through the reduction, and
// written once with a 16-byte store, with enough loads in flight per CU.
//
// Work layout (see Plan in qknorm_internal.hpp): G = S * L threads handle
// one token; the L lanes of shard group s own the 16-byte chunks of Q shard
// s followed by K shard s, lane m taking chunks m, m+L, m+2L, ... (`slots`
// of them, about three). A block holds one or a few tokens side by side and
// there is one block per such group of tokens, so many independent tokens
// have their loads in flight on every CU; gamma is reloaded per block from
// the caches (it is small and shared by all tokens).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "qknorm_internal.hpp"

namespace qkn {
namespace {

struct BF16 {
  static constexpr int kVW = 8;  // elements per 16-byte chunk
  static constexpr int kBytes = 2;
};
struct F32 {
  static constexpr int kVW = 4;
  static constexpr int kBytes = 4;
};

struct Chunk {
  uint32_t w[4];
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Element e of a chunk as float32 (exact widening).
template <class IO>
__device__ __forceinline__ float elem(const Chunk& c, int e);
template <>
__device__ __forceinline__ float elem<BF16>(const Chunk& c, int e) {
  const uint32_t w = c.w[e >> 1];
  return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}
template <>
__device__ __forceinline__ float elem<F32>(const Chunk& c, int e) {
  return __uint_as_float(c.w[e]);
}

// Packs float32 results into a chunk of the I/O type (bf16: round to nearest even).
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

// Loads a chunk at element offset `col` of row `row`: all kVW elements on the
// 16-byte path (which requires a 16-byte aligned address), the first `n`
// (1 <= n <= kVW) on the element-wise path, where elements past `n` read as 0.
//
// Every load is unconditional: a lane whose slot is idle passes the row's
// first chunk (always a valid address) and its value is masked by the caller.
// Predicated loads would put each load in its own branch with a wait for it
// before the join, leaving one load in flight per wave.
template <class IO, bool ALIGNED>
__device__ __forceinline__ Chunk load_chunk(const char* row, int col, int n) {
  Chunk c = {{0u, 0u, 0u, 0u}};
  const char* p = row + (int64_t)col * IO::kBytes;
  if (ALIGNED) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
    c.w[0] = v.x;
    c.w[1] = v.y;
    c.w[2] = v.z;
    c.w[3] = v.w;
  } else if (IO::kBytes == 2) {
    const uint16_t* s = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
    for (int e = 0; e < IO::kVW; ++e) {
      const uint32_t v = s[e < n ? e : 0];
      c.w[e >> 1] |= (e < n ? v : 0u) << ((e & 1) * 16);
    }
  } else {
    const uint32_t* s = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
    for (int e = 0; e < IO::kVW; ++e) {
      const uint32_t v = s[e < n ? e : 0];
      c.w[e] = e < n ? v : 0u;
    }
  }
  return c;
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
  } else if (IO::kBytes == 2) {
    uint16_t* d = reinterpret_cast<uint16_t*>(p);
#pragma unroll
    for (int e = 0; e < IO::kVW; ++e)
      if (e < n) d[e] = (uint16_t)(c.w[e >> 1] >> ((e & 1) * 16));
  } else {
    uint32_t* d = reinterpret_cast<uint32_t*>(p);
#pragma unroll
    for (int e = 0; e < IO::kVW; ++e)
      if (e < n) d[e] = c.w[e];
  }
}

// Sum of squares of one chunk, in element order (Phase A, in-lane part).
template <class IO>
__device__ __forceinline__ float chunk_sumsq(const Chunk& c) {
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < IO::kVW; ++e) {
    const float x = elem<IO>(c, e);
    s = __builtin_fmaf(x, x, s);
  }
  return s;
}

// RMS factor of Eq. 1 for a global squared sum `ss` over full width `div`:
// 1 / sqrt(ss / div + eps), each step correctly rounded in float32 (it runs
// once per token, so the exact forms cost nothing measurable).
__device__ __forceinline__ float rms_factor(float ss, float div, float eps) {
  return 1.0f / __builtin_sqrtf(ss / div + eps);
}

// Register-pressure guard: an empty asm that claims to rewrite the four words
// of `c`. Values the compiler decoded from them earlier (bf16 -> float32
// widenings) can then not be kept alive across this point and are decoded
// again where they are used, so a chunk costs 4 VGPRs instead of 8.
__device__ __forceinline__ void keep_packed(Chunk& c) {
  asm volatile("" : "+v"(c.w[0]), "+v"(c.w[1]), "+v"(c.w[2]), "+v"(c.w[3]));
}

// Sum over aligned groups of `group` lanes (a power of two, 1..64); every
// lane of a group ends with the same value. Inside a 16-lane row the steps
// are DPP moves fused into the adds (quad permutes, then the half-row and
// row mirrors, which pair lanes of the two halves once each half is
// uniform); only the 16- and 32-lane steps cross rows through the LDS
// crossbar. Each step adds two lanes' values, a + b on one and b + a on the
// other, so all lanes of a group hold bitwise the same sum.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float group_sum(float v, int group) {
  if (group > 1) v += dpp_move<0xB1>(v);    // lanes i ^ 1   (quad_perm 1,0,3,2)
  if (group > 2) v += dpp_move<0x4E>(v);    // lanes i ^ 2   (quad_perm 2,3,0,1)
  if (group > 4) v += dpp_move<0x141>(v);   // lanes 7 - i within 8 (row_half_mirror)
  if (group > 8) v += dpp_move<0x140>(v);   // lanes 15 - i within 16 (row_mirror)
  if (group > 16) v += __shfl_xor(v, 16);
  if (group > 32) v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float lane_read(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

template <class IO, int V, int MODE, bool ALIGNED>
__global__ void __launch_bounds__(max_threads_for_slots(V)) qknorm_rows(const RowArgs a) {
  extern __shared__ float red[];  // [2 buffers][tokens per block][groups per token][2]
  constexpr int VW = IO::kVW;
  const int tid = threadIdx.x;
  const int G = a.tok_threads;
  const int L = a.lanes;
  const int j = tid / G;          // token slot within the block
  const int r = tid - j * G;      // thread within the token
  const int s = r / L;            // shard group
  const int m = r - s * L;        // lane within the group

  // Token-invariant geometry of this lane's chunk slots.
  bool isq[V];
  int col[V];
  int cnt[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int u = i * L + m;
    if (u < a.ncq) {
      const int c = u * VW;
      isq[i] = true;
      col[i] = s * a.hq_s + c;
      cnt[i] = min(VW, a.hq_s - c);
    } else if (u < a.ncq + a.nck) {
      const int c = (u - a.ncq) * VW;
      isq[i] = false;
      col[i] = s * a.hk_s + c;
      cnt[i] = min(VW, a.hk_s - c);
    } else {  // idle slot: reads (and ignores) the first chunk of the Q row
      isq[i] = true;
      col[i] = 0;
      cnt[i] = 0;
    }
  }

  Chunk g[MODE == MODE_STATS ? 1 : V];
  if (MODE != MODE_STATS) {
#pragma unroll
    for (int i = 0; i < V; ++i)
      g[i] = load_chunk<IO, ALIGNED>(static_cast<const char*>(isq[i] ? a.gq : a.gk), col[i], max(cnt[i], 1));
  }

  const int group = a.group;            // butterfly width: min(L, 64)
  const int gps = L / group;            // groups per shard
  const int gpt = G / group;            // groups per token
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
    if (MODE != MODE_STATS && IO::kBytes == 2) {
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
      if (G == 64) {
        // One wave per token: group s is shard s; its sum sits in lane s*L.
        if (MODE == MODE_STATS) {
          if (m == 0 && active) {
            a.partials[(int64_t)(2 * s) * a.T + t] = aq;
            a.partials[(int64_t)(2 * s + 1) * a.T + t] = ak;
          }
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
        // by iteration, so one barrier per iteration suffices).
        float* rb = red + ((buf * tpb + j) * gpt) * 2;
        if ((r & (group - 1)) == 0) {
          rb[(r / group) * 2 + 0] = aq;
          rb[(r / group) * 2 + 1] = ak;
        }
        __syncthreads();
        if (MODE == MODE_STATS) {
          if (r < a.shards && active) {
            float pq = rb[(r * gps) * 2 + 0], pk = rb[(r * gps) * 2 + 1];
            for (int q = 1; q < gps; ++q) {
              pq += rb[(r * gps + q) * 2 + 0];
              pk += rb[(r * gps + q) * 2 + 1];
            }
            a.partials[(int64_t)(2 * r) * a.T + t] = pq;
            a.partials[(int64_t)(2 * r + 1) * a.T + t] = pk;
          }
        } else {
          for (int sh = 0; sh < a.shards; ++sh) {
            float pq = rb[(sh * gps) * 2 + 0], pk = rb[(sh * gps) * 2 + 1];
            for (int q = 1; q < gps; ++q) {
              pq += rb[(sh * gps + q) * 2 + 0];
              pk += rb[(sh * gps + q) * 2 + 1];
            }
            ssq = sh == 0 ? pq : ssq + pq;
            ssk = sh == 0 ? pk : ssk + pk;
          }
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

    if (MODE != MODE_STATS && active) {
      if (IO::kBytes == 2) {
#pragma unroll
        for (int i = 0; i < V; ++i) keep_packed(xv[i]);
      }
      const float rq = rms_factor(ssq, a.divq, a.eps);
      const float rk = rms_factor(ssk, a.divk, a.eps);
      char* yq_row = static_cast<char*>(a.yq) + t * a.ldyq * IO::kBytes;
      char* yk_row = static_cast<char*>(a.yk) + t * a.ldyk * IO::kBytes;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        if (cnt[i] > 0) {
          const float rr = isq[i] ? rq : rk;
          float y[VW];
#pragma unroll
          for (int e = 0; e < VW; ++e) y[e] = (elem<IO>(xv[i], e) * elem<IO>(g[i], e)) * rr;
          Chunk out;
          pack<IO>(out, y);
          store_chunk<IO, ALIGNED>(isq[i] ? yq_row : yk_row, col[i], cnt[i], out);
        }
      }
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
__global__ void __launch_bounds__(max_threads_for_slots(V)) qknorm_heads(const HeadArgs a) {
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
  const char* gbase = static_cast<const char*>(isq ? a.gq : a.gk) + (int64_t)head * a.gstride * IO::kBytes;
  const char* xbase = static_cast<const char*>(isq ? a.xq : a.xk);
  char* ybase = static_cast<char*>(isq ? a.yq : a.yk);
  const int64_t ldx = isq ? a.ldxq : a.ldxk;
  const int64_t ldy = isq ? a.ldyq : a.ldyk;

  Chunk g[V];
#pragma unroll
  for (int i = 0; i < V; ++i) g[i] = load_chunk<IO, ALIGNED>(gbase, gcol[i], max(cnt[i], 1));

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
    if (IO::kBytes == 2) {
#pragma unroll
      for (int i = 0; i < V; ++i) keep_packed(g[i]);
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) acc += cnt[i] > 0 ? chunk_sumsq<IO>(xv[i]) : 0.0f;
    acc = group_sum(acc, L);

    if (active) {
      if (IO::kBytes == 2) {
#pragma unroll
        for (int i = 0; i < V; ++i) keep_packed(xv[i]);
      }
      const float rr = rms_factor(acc, a.div, a.eps);
      char* y_row = ybase + t * ldy * IO::kBytes;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        if (cnt[i] > 0) {
          float y[VW];
#pragma unroll
          for (int e = 0; e < VW; ++e) y[e] = (elem<IO>(xv[i], e) * elem<IO>(g[i], e)) * rr;
          Chunk out;
          pack<IO>(out, y);
          store_chunk<IO, ALIGNED>(y_row, col[i], cnt[i], out);
        }
      }
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
__global__ void __launch_bounds__(max_threads_for_slots(V)) qknorm_heads_packed(const HeadArgs a) {
  constexpr int VW = IO::kVW;
  const int tid = threadIdx.x;
  const int G = a.tok_threads;                 // lanes per token, a multiple of 64 and of nc
  const int nc = a.lanes;                      // chunks per head (power of two, <= 64)
  const int j = tid / G;                       // token slot within the block
  const int m = tid - j * G;
  const int total = (a.heads_q + a.heads_k) * nc;

  bool isq[V];
  int col[V], cnt[V];
  const char* gp[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int u = i * G + m;
    if (u < total) {
      const int head = u / nc;
      const int c = (u - head * nc) * VW;
      isq[i] = head < a.heads_q;
      const int hh = isq[i] ? head : head - a.heads_q;
      col[i] = hh * a.head_dim + c;
      cnt[i] = min(VW, a.head_dim - c);
      gp[i] = static_cast<const char*>(isq[i] ? a.gq : a.gk) + ((int64_t)hh * a.gstride + c) * IO::kBytes;
    } else {  // idle slot: reads (and ignores) the first chunk of the Q row and of gamma
      isq[i] = true;
      col[i] = 0;
      cnt[i] = 0;
      gp[i] = static_cast<const char*>(a.gq);
    }
  }
  Chunk g[V];
#pragma unroll
  for (int i = 0; i < V; ++i) g[i] = load_chunk<IO, ALIGNED>(gp[i], 0, max(cnt[i], 1));

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
    if (IO::kBytes == 2) {
#pragma unroll
      for (int i = 0; i < V; ++i) keep_packed(g[i]);
    }
    float ss[V];
#pragma unroll
    for (int i = 0; i < V; ++i) ss[i] = group_sum(cnt[i] > 0 ? chunk_sumsq<IO>(xv[i]) : 0.0f, nc);

    if (active) {
      if (IO::kBytes == 2) {
#pragma unroll
        for (int i = 0; i < V; ++i) keep_packed(xv[i]);
      }
      char* yq_row = static_cast<char*>(a.yq) + t * a.ldyq * IO::kBytes;
      char* yk_row = static_cast<char*>(a.yk) + t * a.ldyk * IO::kBytes;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        if (cnt[i] > 0) {
          const float rr = rms_factor(ss[i], a.div, a.eps);
          float y[VW];
#pragma unroll
          for (int e = 0; e < VW; ++e) y[e] = (elem<IO>(xv[i], e) * elem<IO>(g[i], e)) * rr;
          Chunk out;
          pack<IO>(out, y);
          store_chunk<IO, ALIGNED>(isq[i] ? yq_row : yk_row, col[i], cnt[i], out);
        }
      }
    }
  }
}

using KernelFn = void (*)(const RowArgs);
using HeadKernelFn = void (*)(const HeadArgs);

constexpr int64_t kMaxGrid = (int64_t)1 << 30;

template <class IO, int MODE, bool ALIGNED>
KernelFn pick_slots(int v) {
  switch (v) {
    case 1: return qknorm_rows<IO, 1, MODE, ALIGNED>;
    case 2: return qknorm_rows<IO, 2, MODE, ALIGNED>;
    case 3: return qknorm_rows<IO, 3, MODE, ALIGNED>;
    case 4: return qknorm_rows<IO, 4, MODE, ALIGNED>;
    case 6: return qknorm_rows<IO, 6, MODE, ALIGNED>;
    case 8: return qknorm_rows<IO, 8, MODE, ALIGNED>;
    case 12: return qknorm_rows<IO, 12, MODE, ALIGNED>;
    case 16: return qknorm_rows<IO, 16, MODE, ALIGNED>;
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
    case 12: return QKN_HEAD_KERNEL(12);
    case 16: return QKN_HEAD_KERNEL(16);
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

HeadKernelFn pick_head_kernel(const Plan& p) { return p.bf16 ? pick_head_io<BF16>(p) : pick_head_io<F32>(p); }

KernelFn pick_kernel(const Plan& p) {
  return p.bf16 ? pick_mode<BF16>(p.mode, p.aligned, p.slots) : pick_mode<F32>(p.mode, p.aligned, p.slots);
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
  const int64_t grid = blocks < kMaxGrid ? blocks : kMaxGrid;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3((unsigned)p.threads), (size_t)p.lds_bytes,
                     static_cast<hipStream_t>(stream), args);
  const hipError_t e = hipGetLastError();
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
  const int64_t grid = blocks < kMaxGrid ? blocks : kMaxGrid;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3((unsigned)p.threads), 0, static_cast<hipStream_t>(stream), args);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = std::string("kernel launch: ") + hipGetErrorString(e);
    return (int)e;
  }
  return 0;
}

}  // namespace qkn
