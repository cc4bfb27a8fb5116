// Internal interface between the C ABI layer (qknorm_api.cpp: validation and
// planning, no HIP calls) and the kernel layer (qknorm_kernels.hip).
#pragma once

#include <stdint.h>

#include <string>

namespace qkn {

enum Mode : int { MODE_FUSED = 0, MODE_STATS = 1, MODE_APPLY = 2, MODE_HEADWISE = 3 };

// I/O types (the values of qknorm_dtype_t).
enum Dtype : int { kDtypeF32 = 0, kDtypeBF16 = 1, kDtypeFP8 = 2 };

// Elements per 16-byte chunk, bytes per row element, bytes per gamma element.
constexpr int chunk_elems(int dtype) { return dtype == kDtypeF32 ? 4 : dtype == kDtypeBF16 ? 8 : 16; }
constexpr int row_elem_bytes(int dtype) { return dtype == kDtypeF32 ? 4 : dtype == kDtypeBF16 ? 2 : 1; }
constexpr int gamma_elem_bytes(int dtype) { return dtype == kDtypeF32 ? 4 : 2; }

// Chunk-slot counts per lane that have a compiled kernel.
constexpr int kSlotSizes[] = {1, 2, 3, 4, 6, 8, 12, 16};
constexpr int kMaxSlots = 16;
constexpr int kMaxThreads = 1024;   // threads working on one token (one block)
constexpr int kMinLanesPerShard = 4;

// Largest block that a kernel with `v` chunk slots per lane is compiled for.
// A 1024-thread block leaves each lane 128 VGPRs. On the 16-byte path that
// holds the data and gamma of up to 8 slots (3 for FP8 rows, whose bf16
// gamma takes twice the registers of the data); the element-wise path keeps
// one register per element in flight, so it fits fewer (6 fp32, 4 bf16, 1
// FP8). Kernels with more slots take at most 256 threads (512 VGPRs).
constexpr int max_threads_for_slots(int v, int dtype, bool aligned) {
  return v <= (aligned ? (dtype == 2 ? 3 : 8) : (dtype == 0 ? 6 : dtype == 1 ? 4 : 1)) ? kMaxThreads : 256;
}

// Most chunk slots per lane with a compiled kernel. Element-wise FP8 rows stop
// at 8: 12 or 16 slots of single-byte loads need more than 512 VGPRs.
constexpr int max_slots(int dtype, bool aligned) { return (dtype == 2 && !aligned) ? 8 : kMaxSlots; }

// How one token's Q and K columns are spread over a block.
//
// Each shard's columns are cut into 16-byte chunks (8 bf16 or 4 fp32; the
// last chunk of a shard may be partial on the element-wise path). Q shard s
// and K shard s form one list of ncq + nck chunks, handled by a group of L
// lanes: lane m of the group takes chunks m, m + L, m + 2L, ... (`slots` of
// them), so each instruction of the group touches L consecutive chunks. S
// groups form the G = S * L threads of one token, G a multiple of the
// 64-lane wavefront; L is a power of two below 64 or a multiple of 64. A
// block holds `tokens_per_block` such tokens side by side.
struct Plan {
  int mode = 0;
  int dtype = kDtypeBF16;
  int aligned = 0;    // 1: 16-byte loads/stores; 0: element-wise path
  int vw = 8;         // elements per chunk
  int shards = 1;     // S
  int hq_s = 0;       // Q shard width (elements)
  int hk_s = 0;       // K shard width (elements)
  int ncq = 0;        // Q chunks per shard
  int nck = 0;        // K chunks per shard
  int lanes = 0;      // L, lanes per shard
  int group = 0;      // lanes per butterfly group: min(L, 64)
  int tok_threads = 0;       // G = S * L
  int tokens_per_block = 1;  // tokens handled side by side in one block
  int threads = 0;           // block size: tokens_per_block * G
  int slots = 0;      // chunk slots per lane (one of kSlotSizes)
  int waves = 0;      // waves per token: G / 64
  int lds_bytes = 0;  // dynamic LDS for the cross-wave reduction (0 if one wave per token)
  // headwise only: heads of Q and of K, head width, gamma stride between heads
  int heads_q = 0;
  int heads_k = 0;
  int head_dim = 0;
  int heads_packed = 0;  // 1: token-wide chunk layout, one nc-lane group per head per slot
  // partial_stats only: 1 for the slot-wave form (a chunk per thread, the
  // chunk sums exchanged in LDS; see qknorm_stats_slot_waves), with runs of
  // 8 * xrun blocks ordered so that each XCD takes xrun consecutive blocks of
  // tokens
  int slot_waves = 0;
  int xrun = 0;
  // token groups per block (the grid is ceil(groups / group_loop), so no
  // block takes more than group_loop of them); 1 except for the FP8 rule in
  // make_plan
  int group_loop = 1;
  // at most this many blocks share a compute unit (0: no cap), by padding the
  // launch's LDS (launch_lds_bytes)
  int blocks_per_cu = 0;
};

// Kernel arguments (passed by value).
struct RowArgs {
  const void* xq;
  void* yq;
  const void* gq;
  int64_t ldxq, ldyq;
  const void* xk;
  void* yk;
  const void* gk;
  int64_t ldxk, ldyk;
  int64_t T;
  int hq_s, hk_s;
  int ncq, nck;
  int shards;
  int lanes, group, tok_threads, tokens_per_block;
  int log2_lanes;     // log2(lanes) when shards > 1 (lanes is then a power of two)
  int log2_tok;       // log2(tok_threads) when several tokens share a block (a power of two <= 64)
  int log2_group;     // log2(group)
  int groups_per_shard, groups_per_token;
  float inv_divq, inv_divk;  // 1/H for Q and K in Eq. 1, rounded once
  float eps;
  float* partials;    // MODE_STATS: [S][2][T]
  const float* stats; // MODE_APPLY: [P][2][T]
  int n_planes;
  int stagger;        // 1: the first resident generation of blocks starts staggered (large launches)
#ifdef QKNORM_BLOCK_CLOCKS
  unsigned long long* clocks;  // timing-only builds: per block {start, end, XCC id << 32 | hardware id}
#endif
};

// Headwise kernel arguments: every head of head_dim columns is normalized on
// its own; a token's heads (Q heads, then K heads) each take an aligned group
// of `lanes` lanes.
struct HeadArgs {
  const void* xq;
  void* yq;
  const void* gq;
  int64_t ldxq, ldyq;
  const void* xk;
  void* yk;
  const void* gk;
  int64_t ldxk, ldyk;
  int64_t T;
  int64_t gstride;    // gamma elements between consecutive heads (0: shared)
  int head_dim;
  int heads_q, heads_k;
  int nc;             // chunks per head
  int lanes;          // per-head layout: lanes per head (power of two, 4..64);
                      // token-wide layout: nc (the lane group of one head)
  int tok_threads;    // threads per token
  int tokens_per_block;
  int log2_nc;        // token-wide layout: log2(nc)
  float inv_div;      // 1/head_dim, rounded once (H of Eq. 1)
  float eps;
};

// Plans a headwise launch; false (with a reason) if no kernel holds a head.
bool make_head_plan(int dtype, bool aligned, int64_t head_dim, int64_t heads_q, int64_t heads_k, int64_t T,
                    Plan* plan, std::string* why);

int launch_heads(const Plan& plan, const HeadArgs& args, void* stream, std::string* err);

// Fills `plan` for the given shapes; returns false (with a reason) if no
// compiled kernel can hold the row.
// packed: Q and K are adjacent column ranges of the same rows (K's first
// element right after Q's last, one row stride).
bool make_plan(int mode, int dtype, bool aligned, bool packed, int shards, int64_t hq, int64_t hk, int64_t T,
               Plan* plan, std::string* why);

std::string describe(const Plan& p);
// The dynamic LDS a launch of `p` asks for: the reduction's own, or, where the
// plan caps the blocks per compute unit, enough of the 160 KiB LDS that no
// more than that many blocks fit (a multiple of 2560 bytes, so that the cap
// holds for any allocation granularity that divides it).
int launch_lds_bytes(const Plan& p);

// FP8 rows in up to 4 slots, fused or apply_with_stats on the 16-byte path,
// blocks looping over several token groups: the row kernel holds gamma
// widened to float32 in registers across the block's tokens.
inline bool gamma_in_registers(const Plan& p) {
  return p.dtype == kDtypeFP8 && p.aligned && !p.slot_waves && p.group_loop > 1 && p.slots <= 4 &&
         (p.mode == MODE_FUSED || p.mode == MODE_APPLY);
}

// Launches the kernel for `plan` on `stream`. Returns 0 or a HIP error code,
// with a message in *err.
int launch(const Plan& plan, const RowArgs& args, void* stream, std::string* err);

}  // namespace qkn
