// C ABI of libqknorm.so: argument validation, launch planning, error strings.
//
// Everything in this file is plain C++ with no HIP call, so every argument
// error is detected (and testable) without a GPU; only qkn::launch, in
// qknorm_kernels.hip, touches the HIP runtime.
//
// Source of the operation: "SwiftQK: Fast and Communication-Efficient Tensor
// Parallelism for Query-Key Normalization" (arXiv 2608.09160v1): RMS-Norm,
// Eq. 1; Phase A (per-shard squared sums, FP32 aggregation); Phase B and the
// final scaling.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "qknorm.h"
#include "qknorm_internal.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return QKNORM_OK;
}

size_t elem_size(int dtype) {
  if (dtype == QKNORM_F32) return 4;
  if (dtype == QKNORM_BF16) return 2;
  if (dtype == QKNORM_FP8_E4M3) return 1;
  return 0;
}

// gamma is bf16 for FP8 rows, the row type otherwise
size_t gamma_size(int dtype) { return dtype == QKNORM_F32 ? 4 : 2; }

// The set of bytes touched by rows t < T, columns j < h of a strided matrix.
struct Region {
  uintptr_t base;
  int64_t ld;   // elements
  int64_t h;    // elements
  int64_t T;
  int64_t esz;  // bytes per element
  int64_t span_bytes() const { return ((T - 1) * ld + h) * esz; }
};

// True if the two element sets may share a byte. Exact for equal strides and
// element sizes (the packed-QKV case); conservative (byte spans) otherwise.
bool may_overlap(const Region& a, const Region& b) {
  if (a.T <= 0 || b.T <= 0 || a.h <= 0 || b.h <= 0) return false;
  const uintptr_t a0 = a.base, a1 = a.base + (uintptr_t)a.span_bytes();
  const uintptr_t b0 = b.base, b1 = b.base + (uintptr_t)b.span_bytes();
  if (a1 <= b0 || b1 <= a0) return false;
  if (a.ld != b.ld || a.esz != b.esz || a.T == 1 || b.T == 1) return true;
  const int64_t d = (int64_t)(b.base - a.base);  // may be negative
  if (d % a.esz != 0) return true;
  const int64_t de = d / a.esz;
  // Column of a's row grid where b's rows start.
  const int64_t r = ((de % a.ld) + a.ld) % a.ld;
  if (r + b.h <= a.ld) return r < a.h;                  // b occupies [r, r + b.h)
  return true;                                          // b wraps into a's next row
}

bool same_region(const Region& a, const Region& b) {
  return a.base == b.base && a.ld == b.ld && a.h == b.h && a.esz == b.esz;
}

bool fits(int64_t T, int64_t ld, int64_t h, int64_t esz) {
  // (T - 1) * ld + h elements, times esz bytes, must fit in int64.
  if (T <= 0) return true;
  const int64_t lim = INT64_MAX / esz;
  if (T - 1 > 0 && ld > (lim - h) / (T - 1)) return false;
  return true;
}

struct Checked {
  qkn::Plan plan;
  qkn::RowArgs args;
};

const char* kName[3] = {"qknorm_fused", "qknorm_partial_stats", "qknorm_apply_with_stats"};

// Validates the arguments shared by the three entry points and builds the
// plan. Returns QKNORM_OK, or an error code with the message set.
int check_and_plan(int mode, const qknorm_operand_t* q, const qknorm_operand_t* k, int64_t T,
                   int dtype, float eps, int shards, const void* stat_buf, int n_planes,
                   int64_t hq_full, int64_t hk_full, Checked* out, bool* noop) {
  const char* fn = kName[mode];
  *noop = false;
  if (!q || !k) return fail(QKNORM_ERR_INVALID_ARG, "%s: q and k operand descriptors are required", fn);
  const size_t esz = elem_size(dtype);
  if (!esz) return fail(QKNORM_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
  if (T < 0) return fail(QKNORM_ERR_INVALID_ARG, "%s: T = %lld < 0", fn, (long long)T);
  if (mode != qkn::MODE_APPLY) {
    if (shards < 1 || shards > QKNORM_MAX_SHARDS)
      return fail(QKNORM_ERR_INVALID_ARG, "%s: shards = %d outside [1, %d]", fn, shards, QKNORM_MAX_SHARDS);
  } else {
    shards = 1;
  }
  if (mode != qkn::MODE_STATS && !(std::isfinite(eps) && eps >= 0.0f))
    return fail(QKNORM_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  const qknorm_operand_t* ops[2] = {q, k};
  const char* nm[2] = {"q", "k"};
  for (int c = 0; c < 2; ++c) {
    const qknorm_operand_t* o = ops[c];
    if (o->h <= 0) return fail(QKNORM_ERR_INVALID_ARG, "%s: %s->h = %lld must be > 0", fn, nm[c], (long long)o->h);
    if (o->h % shards)
      return fail(QKNORM_ERR_INVALID_ARG, "%s: %s->h = %lld is not divisible into %d shards", fn, nm[c],
                  (long long)o->h, shards);
    if (o->ld_x < o->h)
      return fail(QKNORM_ERR_INVALID_ARG, "%s: %s->ld_x = %lld < h = %lld", fn, nm[c], (long long)o->ld_x,
                  (long long)o->h);
    if (mode != qkn::MODE_STATS && o->ld_y < o->h)
      return fail(QKNORM_ERR_INVALID_ARG, "%s: %s->ld_y = %lld < h = %lld", fn, nm[c], (long long)o->ld_y,
                  (long long)o->h);
    if (o->h > (int64_t)1 << 30)
      return fail(QKNORM_ERR_UNSUPPORTED, "%s: %s->h = %lld is too wide", fn, nm[c], (long long)o->h);
  }
  if (mode == qkn::MODE_APPLY) {
    if (n_planes < 1 || n_planes > QKNORM_MAX_PLANES)
      return fail(QKNORM_ERR_INVALID_ARG, "%s: n_planes = %d outside [1, %d]", fn, n_planes, QKNORM_MAX_PLANES);
    if (hq_full < q->h || hk_full < k->h)
      return fail(QKNORM_ERR_INVALID_ARG, "%s: full widths (%lld, %lld) must be >= local widths (%lld, %lld)", fn,
                  (long long)hq_full, (long long)hk_full, (long long)q->h, (long long)k->h);
    if (hq_full > QKNORM_MAX_FULL_WIDTH || hk_full > QKNORM_MAX_FULL_WIDTH)
      return fail(QKNORM_ERR_INVALID_ARG, "%s: full widths must be <= %d", fn, QKNORM_MAX_FULL_WIDTH);
  }
  if (T == 0) {
    *noop = true;
    return ok();
  }

  // Pointers.
  for (int c = 0; c < 2; ++c) {
    const qknorm_operand_t* o = ops[c];
    if (!o->x) return fail(QKNORM_ERR_INVALID_ARG, "%s: %s->x is NULL", fn, nm[c]);
    if (mode != qkn::MODE_STATS && (!o->y || !o->gamma))
      return fail(QKNORM_ERR_INVALID_ARG, "%s: %s->y and %s->gamma are required", fn, nm[c], nm[c]);
    if ((uintptr_t)o->x % esz ||
        (mode != qkn::MODE_STATS && ((uintptr_t)o->y % esz || (uintptr_t)o->gamma % gamma_size(dtype))))
      return fail(QKNORM_ERR_INVALID_ARG, "%s: %s pointers must be aligned to their element size", fn, nm[c]);
    if (!fits(T, o->ld_x, o->h, esz) || (mode != qkn::MODE_STATS && !fits(T, o->ld_y, o->h, esz)))
      return fail(QKNORM_ERR_INVALID_ARG, "%s: %s rows exceed the address range", fn, nm[c]);
  }
  if (mode != qkn::MODE_FUSED && !stat_buf)
    return fail(QKNORM_ERR_INVALID_ARG, "%s: %s buffer is NULL", fn, mode == qkn::MODE_STATS ? "partials" : "stats");
  if (mode != qkn::MODE_FUSED && (uintptr_t)stat_buf % sizeof(float))
    return fail(QKNORM_ERR_INVALID_ARG, "%s: %s buffer must be 4-byte aligned", fn,
                mode == qkn::MODE_STATS ? "partials" : "stats");
  if (mode == qkn::MODE_STATS && T > INT64_MAX / (8 * (int64_t)shards))
    return fail(QKNORM_ERR_INVALID_ARG, "%s: partials size overflows", fn);

  // Overlaps.
  const int64_t e = (int64_t)esz;
  Region xr[2], yr[2], gr[2];
  for (int c = 0; c < 2; ++c) {
    xr[c] = Region{(uintptr_t)ops[c]->x, ops[c]->ld_x, ops[c]->h, T, e};
    yr[c] = Region{(uintptr_t)ops[c]->y, ops[c]->ld_y, ops[c]->h, T, e};
    gr[c] = Region{(uintptr_t)ops[c]->gamma, ops[c]->h, ops[c]->h, 1, (int64_t)gamma_size(dtype)};
  }
  if (mode != qkn::MODE_STATS) {
    if (may_overlap(yr[0], yr[1])) return fail(QKNORM_ERR_INVALID_ARG, "%s: q and k outputs overlap", fn);
    for (int c = 0; c < 2; ++c) {
      if (may_overlap(yr[c], xr[1 - c]))
        return fail(QKNORM_ERR_INVALID_ARG, "%s: %s output overlaps the %s input", fn, nm[c], nm[1 - c]);
      if (may_overlap(yr[c], xr[c]) && !same_region(yr[c], xr[c]))
        return fail(QKNORM_ERR_INVALID_ARG,
                    "%s: %s output partially overlaps its input (only exact in-place is allowed)", fn, nm[c]);
      for (int g = 0; g < 2; ++g)
        if (may_overlap(yr[c], gr[g]))
          return fail(QKNORM_ERR_INVALID_ARG, "%s: %s output overlaps gamma of %s", fn, nm[c], nm[g]);
    }
  }
  if (mode == qkn::MODE_STATS) {
    const Region pr{(uintptr_t)stat_buf, 1, (int64_t)shards * 2 * T, 1, 4};
    for (int c = 0; c < 2; ++c)
      if (may_overlap(pr, xr[c])) return fail(QKNORM_ERR_INVALID_ARG, "%s: partials overlap the %s input", fn, nm[c]);
  }
  if (mode == qkn::MODE_APPLY) {
    const Region sr{(uintptr_t)stat_buf, 1, (int64_t)n_planes * 2 * T, 1, 4};
    for (int c = 0; c < 2; ++c)
      if (may_overlap(sr, yr[c])) return fail(QKNORM_ERR_INVALID_ARG, "%s: stats overlap the %s output", fn, nm[c]);
  }

  // Path selection: 16-byte chunks need every base 16-byte aligned, every row
  // stride and every shard width a whole number of chunks.
  const int vw = (int)(16 / esz);
  bool aligned = true;
  for (int c = 0; c < 2; ++c) {
    const qknorm_operand_t* o = ops[c];
    aligned = aligned && ((uintptr_t)o->x % 16 == 0) && (o->ld_x % vw == 0) && ((o->h / shards) % vw == 0);
    if (mode != qkn::MODE_STATS)
      aligned = aligned && ((uintptr_t)o->y % 16 == 0) && (o->ld_y % vw == 0) && ((uintptr_t)o->gamma % 16 == 0);
  }

  // Packed rows: K starts right after Q's last column, with the same stride.
  const bool packed = (const char*)k->x == (const char*)q->x + q->h * esz && k->ld_x == q->ld_x;

  std::string why;
  if (!qkn::make_plan(mode, dtype, aligned, packed, shards, q->h, k->h, T, &out->plan, &why))
    return fail(QKNORM_ERR_UNSUPPORTED, "%s: %s", fn, why.c_str());

  qkn::RowArgs& a = out->args;
  std::memset(&a, 0, sizeof a);
  a.xq = q->x;
  a.yq = q->y;
  a.gq = q->gamma;
  a.ldxq = q->ld_x;
  a.ldyq = q->ld_y;
  a.xk = k->x;
  a.yk = k->y;
  a.gk = k->gamma;
  a.ldxk = k->ld_x;
  a.ldyk = k->ld_y;
  a.T = T;
  a.hq_s = out->plan.hq_s;
  a.hk_s = out->plan.hk_s;
  a.ncq = out->plan.ncq;
  a.nck = out->plan.nck;
  a.shards = out->plan.shards;
  a.lanes = out->plan.lanes;
  a.group = out->plan.group;
  a.tok_threads = out->plan.tok_threads;
  a.tokens_per_block = out->plan.tokens_per_block;
  a.inv_divq = (float)(1.0 / (double)(mode == qkn::MODE_APPLY ? hq_full : q->h));
  a.inv_divk = (float)(1.0 / (double)(mode == qkn::MODE_APPLY ? hk_full : k->h));
  a.log2_lanes = 0;
  while ((1 << a.log2_lanes) < a.lanes) ++a.log2_lanes;
  a.log2_tok = 0;
  while ((1 << a.log2_tok) < a.tok_threads) ++a.log2_tok;
  a.log2_group = 0;
  while ((1 << a.log2_group) < out->plan.group) ++a.log2_group;
  a.groups_per_shard = out->plan.lanes / out->plan.group;
  a.groups_per_token = out->plan.tok_threads / out->plan.group;
  a.eps = eps;
  a.partials = mode == qkn::MODE_STATS ? (float*)stat_buf : nullptr;
  a.stats = mode == qkn::MODE_APPLY ? (const float*)stat_buf : nullptr;
  a.n_planes = mode == qkn::MODE_APPLY ? n_planes : 0;
  return QKNORM_OK;
}

struct HeadChecked {
  qkn::Plan plan;
  qkn::HeadArgs args;
};

// Validation and planning for qknorm_headwise (no HIP calls).
int check_and_plan_heads(const qknorm_operand_t* q, const qknorm_operand_t* k, int64_t T, int dtype, float eps,
                         int64_t head_dim, int64_t gstride, HeadChecked* out, bool* noop) {
  const char* fn = "qknorm_headwise";
  *noop = false;
  if (!q || !k) return fail(QKNORM_ERR_INVALID_ARG, "%s: q and k operand descriptors are required", fn);
  const size_t esz = elem_size(dtype);
  if (!esz) return fail(QKNORM_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
  if (T < 0) return fail(QKNORM_ERR_INVALID_ARG, "%s: T = %lld < 0", fn, (long long)T);
  if (!(std::isfinite(eps) && eps >= 0.0f)) return fail(QKNORM_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  if (head_dim <= 0 || head_dim > ((int64_t)1 << 20))
    return fail(QKNORM_ERR_INVALID_ARG, "%s: head_dim = %lld", fn, (long long)head_dim);
  if (gstride < 0 || gstride > ((int64_t)1 << 30))
    return fail(QKNORM_ERR_INVALID_ARG, "%s: gamma_head_stride = %lld", fn, (long long)gstride);
  const qknorm_operand_t* ops[2] = {q, k};
  const char* nm[2] = {"q", "k"};
  for (int c = 0; c < 2; ++c) {
    const qknorm_operand_t* o = ops[c];
    if (o->h <= 0 || o->h % head_dim)
      return fail(QKNORM_ERR_INVALID_ARG, "%s: %s->h = %lld is not a positive multiple of head_dim %lld", fn, nm[c],
                  (long long)o->h, (long long)head_dim);
    if (o->ld_x < o->h || o->ld_y < o->h)
      return fail(QKNORM_ERR_INVALID_ARG, "%s: %s row strides must be >= h", fn, nm[c]);
    if (o->h > (int64_t)1 << 30) return fail(QKNORM_ERR_UNSUPPORTED, "%s: %s->h is too wide", fn, nm[c]);
  }
  if (T == 0) {
    *noop = true;
    return ok();
  }
  for (int c = 0; c < 2; ++c) {
    const qknorm_operand_t* o = ops[c];
    if (!o->x || !o->y || !o->gamma) return fail(QKNORM_ERR_INVALID_ARG, "%s: %s->x, y and gamma are required", fn, nm[c]);
    if ((uintptr_t)o->x % esz || (uintptr_t)o->y % esz || (uintptr_t)o->gamma % gamma_size(dtype))
      return fail(QKNORM_ERR_INVALID_ARG, "%s: %s pointers must be aligned to their element size", fn, nm[c]);
    if (!fits(T, o->ld_x, o->h, esz) || !fits(T, o->ld_y, o->h, esz))
      return fail(QKNORM_ERR_INVALID_ARG, "%s: %s rows exceed the address range", fn, nm[c]);
  }
  const int64_t e = (int64_t)esz;
  Region xr[2], yr[2], gr[2];
  for (int c = 0; c < 2; ++c) {
    const int64_t heads = ops[c]->h / head_dim;
    xr[c] = Region{(uintptr_t)ops[c]->x, ops[c]->ld_x, ops[c]->h, T, e};
    yr[c] = Region{(uintptr_t)ops[c]->y, ops[c]->ld_y, ops[c]->h, T, e};
    const int64_t gext = (heads - 1) * gstride + head_dim;  // gamma elements read
    gr[c] = Region{(uintptr_t)ops[c]->gamma, gext, gext, 1, (int64_t)gamma_size(dtype)};
  }
  if (may_overlap(yr[0], yr[1])) return fail(QKNORM_ERR_INVALID_ARG, "%s: q and k outputs overlap", fn);
  for (int c = 0; c < 2; ++c) {
    if (may_overlap(yr[c], xr[1 - c]))
      return fail(QKNORM_ERR_INVALID_ARG, "%s: %s output overlaps the %s input", fn, nm[c], nm[1 - c]);
    if (may_overlap(yr[c], xr[c]) && !same_region(yr[c], xr[c]))
      return fail(QKNORM_ERR_INVALID_ARG, "%s: %s output partially overlaps its input", fn, nm[c]);
    for (int g = 0; g < 2; ++g)
      if (may_overlap(yr[c], gr[g]))
        return fail(QKNORM_ERR_INVALID_ARG, "%s: %s output overlaps gamma of %s", fn, nm[c], nm[g]);
  }
  const int vw = (int)(16 / esz);
  bool aligned = head_dim % vw == 0 && gstride % vw == 0;
  for (int c = 0; c < 2; ++c) {
    const qknorm_operand_t* o = ops[c];
    aligned = aligned && (uintptr_t)o->x % 16 == 0 && (uintptr_t)o->y % 16 == 0 && (uintptr_t)o->gamma % 16 == 0 &&
              o->ld_x % vw == 0 && o->ld_y % vw == 0;
  }
  std::string why;
  if (!qkn::make_head_plan(dtype, aligned, head_dim, q->h / head_dim, k->h / head_dim, T, &out->plan,
                           &why))
    return fail(QKNORM_ERR_UNSUPPORTED, "%s: %s", fn, why.c_str());
  qkn::HeadArgs& a = out->args;
  std::memset(&a, 0, sizeof a);
  a.xq = q->x;
  a.yq = q->y;
  a.gq = q->gamma;
  a.ldxq = q->ld_x;
  a.ldyq = q->ld_y;
  a.xk = k->x;
  a.yk = k->y;
  a.gk = k->gamma;
  a.ldxk = k->ld_x;
  a.ldyk = k->ld_y;
  a.T = T;
  a.gstride = gstride;
  a.head_dim = (int)head_dim;
  a.heads_q = out->plan.heads_q;
  a.heads_k = out->plan.heads_k;
  a.nc = out->plan.ncq;
  a.lanes = out->plan.lanes;
  a.tok_threads = out->plan.tok_threads;
  a.tokens_per_block = out->plan.tokens_per_block;
  a.inv_div = (float)(1.0 / (double)head_dim);
  a.log2_nc = 0;
  while ((1 << a.log2_nc) < out->plan.ncq) ++a.log2_nc;
  a.eps = eps;
  return QKNORM_OK;
}

int run(int mode, const Checked& c, void* stream) {
  std::string err;
  const int rc = qkn::launch(c.plan, c.args, stream, &err);
  if (rc) return fail(QKNORM_ERR_HIP, "%s: %s", kName[mode], err.c_str());
  return ok();
}

}  // namespace

namespace qkn {

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Smallest compiled slot count >= v, or 0 if it exceeds `max`.
static int slots_for(int v, int max) {
  for (int s : kSlotSizes)
    if (s >= v) return s <= max ? s : 0;
  return 0;
}

// Launch geometry, from timings of every feasible lane layout on MI355X over
// prefill rows of 1280 to 18432 normalized elements (bf16, FP8 and fp32,
// T = 8192). Costs are per candidate; the cheapest wins, ties going to fewer
// waves (launches of few tokens are scored on their own, below):
// - chunks per lane: three is best for every row type; one is always slow
//   (too few loads in flight); fp32 rows, whose kernel keeps its occupancy
//   at 4 and 6 slots, are indifferent between 3, 4 and 6; bf16 pays for 6
//   slots (5 waves per SIMD instead of 8);
// - idle slots cost little up to a quarter of a lane's slots, much beyond;
// - blocks of 13 or more waves are slow (fp32: 12 to 25% against 6 to 12
//   waves), and more than 8 waves per token cost a little (a longer
//   cross-wave sum);
// - FP8 rows (4 waves per SIMD at 3 slots) want at most 4 waves per token:
//   5 to 12 are 8 to 60% slower; one wave per token (several tokens to a
//   block) and 3 waves cost a little.
static double prefill_slot_cost(int dtype, int v) {
  if (v == 3) return 0.0;
  if (v == 1) return 10.0;
  switch (dtype) {
    case kDtypeF32: return v == 4 || v == 6 ? 0.1 : v == 2 ? 0.5 : v == 8 ? 0.8 : 1.5;
    case kDtypeFP8: return v == 2 ? 0.25 : v == 4 ? 0.3 : v == 6 ? 0.6 : v == 8 ? 1.0 : 2.0;
    default: return v == 4 ? 0.3 : v == 2 ? 0.5 : v == 6 ? 1.0 : 2.0;
  }
}

bool make_plan(int mode, int dtype, bool aligned, bool packed, int shards, int64_t hq, int64_t hk, int64_t T,
               Plan* p, std::string* why) {
  Plan r;
  r.mode = mode;
  r.dtype = dtype;
  r.aligned = aligned ? 1 : 0;
  r.vw = chunk_elems(dtype);
  r.shards = shards;
  const int64_t hq_s = hq / shards, hk_s = hk / shards;
  const int64_t max_chunks = (int64_t)kMaxThreads * 8;  // per token: 1024 threads x 8 slots
  const int64_t ncq = (hq_s + r.vw - 1) / r.vw, nck = (hk_s + r.vw - 1) / r.vw;
  if ((ncq + nck) * shards > max_chunks) {
    *why = "rows of " + std::to_string(hq + hk) + " elements (" + std::to_string(ncq + nck) +
           " chunks per shard x " + std::to_string(shards) + " shards) exceed the " +
           std::to_string(max_chunks) + " chunks a block holds";
    return false;
  }
  r.hq_s = (int)hq_s;
  r.hk_s = (int)hk_s;
  r.ncq = (int)ncq;
  r.nck = (int)nck;
  const int nc = r.ncq + r.nck;

  // Candidate lane counts per shard: powers of two below 64 (several shards,
  // or several tokens, share a wave) and multiples of 64 (a shard spans whole
  // waves).
  struct Cand {
    int lanes, slots;
    int64_t waste;
  };
  Cand best{0, 0, 0};
  double best_score = 1e30;
  const bool few_tokens = T < 1024;  // under ~4 tokens per CU: favour latency
  // Slots per lane for `l` lanes per shard, or 0 if that layout does not fit a block.
  // Several tokens share a wave only without shards and with enough tokens
  // to fill the waves.
  const bool sub_wave = shards == 1 && !few_tokens;
  auto fits_block = [&](int l) {
    const int g = shards * l;
    if (g > kMaxThreads || (g % 64 && !(sub_wave && g < 64))) return 0;
    const int v = slots_for(ceil_div(nc, l), max_slots(dtype, aligned));
    return (v && g <= max_threads_for_slots(v, dtype, aligned)) ? v : 0;
  };
  for (int l = kMinLanesPerShard; l <= kMaxThreads; l = l < 64 ? l * 2 : l + 64) {
    if (shards > 1 && (l & (l - 1))) continue;  // several shards: power-of-two lane groups only
    const int v = fits_block(l);
    if (!v) continue;
    const int g = shards * l;
    const int64_t waste = (int64_t)l * v - nc;
    const double wfrac = (double)waste / (double)(l * v);
    // With few tokens, spread each over more waves at 2 slots per lane, but
    // over at most 8 waves, and on a tie over more waves (timed under graph
    // replay for T = 1 to 256 and rows of 2560 to 18432 elements: a decode
    // token of 1024 chunks is 10% faster over 8 waves x 2 slots than over 16
    // waves x 1 slot, and 1152 chunks 7-12% faster over 6-7 waves x 3 slots
    // than over 9 waves x 2, whose longer cross-wave sums cost more).
    // Otherwise follow the prefill measurements above.
    const int waves = (g + 63) / 64;
    double score;
    if (few_tokens) {
      score = (v > 2 ? (v - 2) : (2 - v)) + (wfrac > 0.25 ? 8.0 : 0.0) + 2.0 * wfrac + (waves > 8 ? 1.5 : 0.0) -
              0.01 * waves;
    } else if (dtype == kDtypeBF16 && mode != MODE_APPLY && T <= 4096) {
      // Mid-size fused bf16 launches (1024 to 4096 tokens, the range timed)
      // run best over fewer waves with 3 to 6 chunks per lane, whether their
      // rows stream from HBM or sit in the last-level cache (timed with and
      // without rotating buffers at T = 512 to 4096: 1.8% from the fastest
      // layout on average, against 3.6% and 11% for the rule below). Larger
      // launches and apply_with_stats keep the prefill rule. partial_stats
      // takes the fused call's layout: the lanes per shard and chunks per
      // lane fix the order in which a shard's squares are added, and the
      // split path must add them as the fused call does to reproduce it bit
      // for bit (apply_with_stats adds nothing within a row, so its layout
      // is free).
      score = (v == 3 || v == 4 ? 0.0 : v == 6 ? 0.1 : v == 2 ? 0.3 : v == 8 ? 0.4 : v == 1 ? 10.0 : 1.0) +
              (wfrac > 0.25 ? 8.0 : 2.0 * wfrac) + (waves > 4 ? 0.3 : 0.0) + (waves >= 13 ? 3.0 : 0.0) +
              0.01 * waves;
    } else {
      score = prefill_slot_cost(dtype, v) + (wfrac > 0.25 ? 8.0 : 2.0 * wfrac) + (waves >= 13 ? 3.0 : 0.0);
      if (dtype == kDtypeFP8)
        score += waves >= 5 ? 3.0 : waves == 3 ? 0.35 : waves == 1 ? 0.8 : 0.0;
      else if (waves > 8)
        score += 0.5;
      score += 0.01 * waves;
    }
    if (score < best_score) {
      best_score = score;
      best = Cand{l, v, waste};
    }
  }
  if (!best.lanes) {
    *why = "no lane layout holds " + std::to_string(nc) + " chunks per shard with " + std::to_string(shards) +
           " shards";
    return false;
  }
  r.lanes = best.lanes;
  r.slots = best.slots;
  r.group = best.lanes < 64 ? best.lanes : 64;
  r.tok_threads = shards * best.lanes;
  r.waves = (r.tok_threads + 63) / 64;
  // Tokens of one wave or less are packed four waves to a block; wider tokens
  // get a block each.
  r.tokens_per_block = r.tok_threads < 64 ? 4 * 64 / r.tok_threads : (r.waves == 1 && !few_tokens) ? 4 : 1;
  if (r.tokens_per_block * r.tok_threads > max_threads_for_slots(r.slots, dtype, aligned)) r.tokens_per_block = 1;
  r.threads = r.tokens_per_block * r.tok_threads;
  const int groups_per_token = r.tok_threads / r.group;
  if (groups_per_token > 64) {  // the kernel reads one group per lane of a wave
    *why = "internal: " + std::to_string(groups_per_token) + " lane groups per token";
    return false;
  }
  r.lds_bytes = r.waves > 1 ? 2 * r.tokens_per_block * groups_per_token * 2 * (int)sizeof(float) : 0;
  // partial_stats of one shard of packed rows with 32- or 64-lane tokens and
  // 2 to 4 chunks per lane on the 16-byte path (the rank slices) takes the
  // slot-wave form: the same lanes, slots and sums, with each chunk loaded by
  // a thread of its own in row order and the sums exchanged in LDS; a block
  // holds one wave's worth of tokens, and each XCD takes runs of 128
  // consecutive tokens (whole 128-byte lines of the partial planes). It has
  // no token loop, so it takes launches of at most 2^30 tokens (one block per
  // token group).
  if (mode == MODE_STATS && aligned && packed && shards == 1 && (r.lanes == 32 || r.lanes == 64) &&
      r.slots >= 2 && r.slots <= 4 && T <= ((int64_t)1 << 30)) {
    r.slot_waves = 1;
    r.tokens_per_block = 64 / r.lanes;
    r.threads = 64 * r.slots;
    r.lds_bytes = 0;  // static: slots x 64 floats
    r.xrun = 128 / r.tokens_per_block;
  }
  // FP8 rows, fused and apply_with_stats on the 16-byte path: a launch of one
  // to four grids of 4096 waves runs as one such grid whose blocks each take
  // k = ceil(groups / that grid) token groups. The FP8 kernels are bound by
  // instruction issue, and a block's set-up (slot geometry, gamma loads) is
  // then paid once per k groups. Alternated on one MI355X against one group
  // per block: GQA prefill rows (5120/1024, 8192 tokens) 2-3% faster, 3072 to
  // 6144 tokens 2-7%; the rank-slice apply (1280/256, 12288 to 32768 tokens)
  // 3-8%; rows of 2048/512 at 8192 tokens 6%, of 8192/1024 at 2048 tokens
  // 14%; rows of 4096/1024 at 8192 tokens timed 3% slower, inside that
  // shape's own spread of 10%. Loops over more groups per block were slower
  // (GQA rows at 16384 tokens 1%, tokens of 3 waves 1-9%), and so were bf16
  // rows at any such cap (2-7%). Such launches (up to 4 slots) also hold gamma
  // widened in registers across a block's tokens (gamma_in_registers): their
  // grid is resident at 4 waves per SIMD, so the registers cost no
  // occupancy; GQA prefill rows at 8192 tokens 3.1% faster, the rank-slice
  // apply 1.4%, rows of 2048/512 1%, GQA rows at 4096 tokens unchanged, where
  // launches of one group per block lost 1.3-3.4% (the waves per SIMD fall
  // from 7 to 4).
  if (dtype == kDtypeFP8 && aligned && !r.slot_waves && mode != MODE_STATS) {
    const int64_t groups = (T + r.tokens_per_block - 1) / r.tokens_per_block;
    const int64_t c = 4096 / ((r.threads + 63) / 64);
    if (groups > c && groups <= 4 * c) r.group_loop = (int)((groups + c - 1) / c);
  }
  // Fused bf16 launches of one shard whose tokens fill 4 waves x 3 chunks or
  // 3 waves x 4 chunks with no idle slot (the GQA prefill rows, 5120/1024:
  // the prefill layout and, up to 4096 tokens, the mid-size one), from 3072
  // tokens: at most 5 blocks per compute unit instead of the 7 (or 10) their
  // registers allow. Fewer reads in flight shorten the wait of each block's
  // last load, and the memory system keeps up. Alternated on one MI355X
  // against the register-bound residency: 3072 tokens 1.3% faster, 4096
  // 0.9%, 5000 1.4%, 6144 1.3%, 8192 1.6%, 12288 1.8%, 16384 1.5-1.8% (6
  // blocks: 0.4-1.6%, 4 blocks at 8192 tokens: 1.2%). Rows of 4096/1024 (4
  // waves, a sixth of the slots idle) ran 0.9% slower at 5 blocks and 0.3% at
  // 6; other widths were unchanged or slower (tokens of 3 waves x 3 chunks at
  // 6 blocks +1.8%, of 6 waves at 3 blocks +19%), and so were
  // apply_with_stats (+0.6% to +4.7%) and partial_stats, so only this shape
  // takes the cap.
  if (mode == MODE_FUSED && dtype == kDtypeBF16 && aligned && shards == 1 && r.tokens_per_block == 1 &&
      ((r.tok_threads == 256 && r.slots == 3) || (r.tok_threads == 192 && r.slots == 4)) &&
      r.lanes * r.slots == nc && T >= 3072)
    r.blocks_per_cu = 5;
  *p = r;
  return true;
}

// Headwise launch geometry: the same rule as the layerwise planner (about 3
// chunks per lane, few idle slots; few tokens: fewer chunks per lane), with
// a group of L lanes per head and blocks of about 512 threads.
bool make_head_plan(int dtype, bool aligned, int64_t head_dim, int64_t heads_q, int64_t heads_k, int64_t T,
                    Plan* p, std::string* why) {
  Plan r;
  r.mode = MODE_HEADWISE;
  r.dtype = dtype;
  r.aligned = aligned ? 1 : 0;
  r.vw = chunk_elems(dtype);
  const int64_t nc = (head_dim + r.vw - 1) / r.vw;
  const int64_t heads = heads_q + heads_k;
  if (nc > 64 * 8) {
    *why = "heads of " + std::to_string(head_dim) + " elements exceed the " + std::to_string(64 * 8 * r.vw) +
           " a lane group holds";
    return false;
  }
  if (heads * kMinLanesPerShard > kMaxThreads) {
    *why = std::to_string(heads) + " heads per token exceed the " + std::to_string(kMaxThreads / kMinLanesPerShard) +
           " a block holds";
    return false;
  }
  const bool few_tokens = T < 1024;
  r.heads_q = (int)heads_q;
  r.heads_k = (int)heads_k;
  r.head_dim = (int)head_dim;
  r.ncq = (int)nc;
  r.shards = (int)heads;

  // A head of a power-of-two number of chunks (<= 64) fits an aligned lane
  // group, so the token's chunks can be laid out as in the layerwise kernel
  // (consecutive chunks on consecutive lanes), a slot per lane group per head.
  //
  // Token width G for prefill launches, from timings of every feasible G on
  // MI355X (prefill rows of 1280 to 18432 elements in 64- and 128-wide heads,
  // bf16, FP8 and fp32, T = 8192). With no exchange across waves, bf16 and
  // fp32 rows run best over as many waves as fit (up to 16) at 2 to 6 chunks
  // per lane with at most a quarter of the slots idle; FP8 rows (4 waves per
  // SIMD at 3 chunks) over 2 to 4 waves, 5 or more being 8-20% slower.
  const int64_t total = heads * nc;
  if ((nc & (nc - 1)) == 0 && nc <= 64 && total <= (int64_t)kMaxThreads * 8) {
    int best_g = 0, best_v = 0;
    double best_score = 1e30, best_wfrac = 0.0;
    for (int g = 64; g <= kMaxThreads; g += 64) {
      const int v = slots_for((int)((total + g - 1) / g), max_slots(dtype, aligned));
      if (!v || g > max_threads_for_slots(v, dtype, aligned)) continue;
      const double wfrac = (double)((int64_t)g * v - total) / (double)(g * v);
      const int waves = g / 64;
      double score;
      if (few_tokens) {
        score = (double)v + (wfrac > 0.25 ? 8.0 : 0.0) + 2.0 * wfrac;
      } else if (dtype == kDtypeFP8) {
        score = (v == 2 ? 0.0 : v == 3 ? 0.1 : v == 4 ? 0.2 : v == 6 ? 0.3 : v == 8 ? 0.6 : v == 1 ? 1.0 : 2.0) +
                (wfrac > 0.25 ? 8.0 : 2.0 * wfrac) + (waves >= 5 ? 3.0 : waves == 1 ? 0.8 : 0.0) - 0.1 * waves;
      } else {
        score = (v == 2 ? 0.0 : v == 3 ? 0.05 : v == 4 ? 0.1 : v == 6 ? 0.2 : v == 8 ? 1.0 : 2.0) +
                (wfrac > 0.25 ? 8.0 : 0.5 * wfrac) - 0.1 * waves;
      }
      if (score < best_score) {
        best_score = score;
        best_g = g;
        best_v = v;
        best_wfrac = wfrac;
      }
    }
    // FP8 rows too narrow to fill whole waves (every candidate leaves more
    // than a quarter of its slots idle, e.g. 10 heads of 8 chunks) take the
    // per-head layout below, which packs several tokens into a block:
    // 1024/256 columns in 128-wide heads as 6 tokens of 80 lanes per block
    // ran in 7.5 us instead of 11.2 (256 threads per token), 512/128 in 4.9
    // instead of 10.1. bf16 rows of that kind keep the token-wide layout
    // (512/128: 6.1 us against 6.45 per-head).
    if (best_g && !few_tokens && dtype == kDtypeFP8 && best_wfrac > 0.25) best_g = 0;
    if (best_g) {
      r.heads_packed = 1;
      r.lanes = (int)nc;
      r.group = (int)nc;
      r.slots = best_v;
      r.tok_threads = best_g;
      r.tokens_per_block = (best_g == 64 && !few_tokens) ? 4 : 1;
      if (r.tokens_per_block * best_g > max_threads_for_slots(best_v, dtype, aligned)) r.tokens_per_block = 1;
      r.threads = r.tokens_per_block * best_g;
      r.waves = r.threads / 64;
      // FP8 rows from 4096 token groups: each block takes two groups (grid
      // ceil(groups / 2)), paying its set-up (slot geometry, gamma loads)
      // once for both. Alternated on one MI355X against one group per block,
      // 128-wide heads: GQA prefill rows (5120/1024) at 4096, 8192 and 16384
      // tokens 1.0%, 1.7% and 5.7% faster; rows of 4096/1024 6.9%, 8192/1024
      // 2.7%, 16384/2048 1.4%, 2048/512 0.2%. Three or more groups per block
      // were slower than two on the GQA rows at 8192 tokens (3: +2.7%,
      // 4: +5.7%, 6: +5.4% against two).
      if (dtype == kDtypeFP8 && aligned && (T + r.tokens_per_block - 1) / r.tokens_per_block >= 4096)
        r.group_loop = 2;
      *p = r;
      return true;
    }
  }

  int best_l = 0, best_v = 0;
  double best_score = 1e30;
  for (int l = kMinLanesPerShard; l <= 64; l *= 2) {
    const int v = slots_for(ceil_div((int)nc, l), max_slots(dtype, aligned));
    if (!v) continue;
    const int64_t g = heads * l;
    const int64_t threads = (g + 63) / 64 * 64;
    if (threads > max_threads_for_slots(v, dtype, aligned)) continue;
    const double wfrac = (double)((int64_t)l * v - nc) / (double)(l * v);
    // Prefill: from timings of every lane group on MI355X (heads of 80 and 96
    // columns, 40 to 128 heads per token, T = 8192), the best chunks per lane
    // are 2 for bf16 rows (8 lanes per head: 7-52% faster than 4 lanes x 3
    // chunks, idle slots notwithstanding), 1 for FP8 rows up to 512 threads
    // per token (else 2), and 3 for fp32 rows.
    double score;
    if (few_tokens) {
      score = (double)v + (wfrac > 0.25 ? 8.0 : 0.0) + 2.0 * wfrac;
    } else {
      if (dtype == kDtypeBF16)
        score = v == 2 ? 0.0 : (v == 1 || v == 3) ? 0.5 : 1.0 + 0.1 * v;
      else if (dtype == kDtypeFP8)
        score = (v == 1 ? 0.0 : v == 2 ? 0.2 : 1.0 + 0.1 * v) + (threads >= 640 ? 0.5 : 0.0);
      else
        score = v == 3 ? 0.0 : v == 2 ? 0.2 : v == 4 ? 0.3 : 1.0 + 0.1 * v;
      score += wfrac > 0.5 ? 8.0 : wfrac;
    }
    if (score < best_score) {
      best_score = score;
      best_l = l;
      best_v = v;
    }
  }
  if (!best_l) {
    *why = "no lane layout holds " + std::to_string(heads) + " heads of " + std::to_string(nc) + " chunks";
    return false;
  }
  r.lanes = best_l;
  r.group = best_l;
  r.slots = best_v;
  r.tok_threads = (int)heads * best_l;
  int tpb = few_tokens ? 1 : (int)(512 / r.tok_threads);
  if (tpb < 1) tpb = 1;
  while (tpb > 1 && (tpb * r.tok_threads + 63) / 64 * 64 > max_threads_for_slots(best_v, dtype, aligned)) --tpb;
  r.tokens_per_block = tpb;
  r.threads = (tpb * r.tok_threads + 63) / 64 * 64;
  r.waves = r.threads / 64;
  *p = r;
  return true;
}

static const char* dtype_name(int d) { return d == kDtypeF32 ? "f32" : d == kDtypeBF16 ? "bf16" : "fp8_e4m3"; }

int launch_lds_bytes(const Plan& p) {
  constexpr int kLdsPerCu = 160 * 1024;  // gfx950
  if (p.blocks_per_cu <= 0) return p.lds_bytes;
  const int pad = kLdsPerCu / p.blocks_per_cu / 2560 * 2560;
  return pad > p.lds_bytes ? pad : p.lds_bytes;
}

std::string describe(const Plan& p) {
  if (p.mode == MODE_HEADWISE) {
    char buf[320];
    snprintf(buf, sizeof buf,
             "headwise %s path=%s layout=%s heads=(%d,%d) head_dim=%d chunks/head=%d lanes/head=%d "
             "threads/token=%d tokens/block=%d threads/block=%d slots=%d",
             dtype_name(p.dtype), p.aligned ? "16B" : "elementwise", p.heads_packed ? "token-wide" : "per-head",
             p.heads_q, p.heads_k, p.head_dim, p.ncq, p.heads_packed ? p.ncq : p.lanes, p.tok_threads,
             p.tokens_per_block, p.threads, p.slots);
    if (p.group_loop > 1) {
      const size_t n = strlen(buf);
      snprintf(buf + n, sizeof buf - n, " groups/block=%d", p.group_loop);
    }
    return buf;
  }
  char buf[384];
  int n = snprintf(buf, sizeof buf,
                   "%s %s path=%s shards=%d shard_w=(%d,%d) chunks=(%d,%d) lanes/shard=%d threads/token=%d "
                   "tokens/block=%d waves/token=%d slots=%d lds=%d",
                   p.mode == MODE_FUSED ? "fused" : p.mode == MODE_STATS ? "partial_stats" : "apply_with_stats",
                   dtype_name(p.dtype), p.aligned ? "16B" : "elementwise", p.shards, p.hq_s, p.hk_s, p.ncq, p.nck,
                   p.lanes, p.tok_threads, p.tokens_per_block, p.waves, p.slots, p.lds_bytes);
  if (p.slot_waves && n > 0 && n < (int)sizeof buf)
    n += snprintf(buf + n, sizeof buf - n, " form=slot-waves threads/block=%d xcd_run=%d", p.threads, p.xrun);
  if (p.group_loop > 1 && n > 0 && n < (int)sizeof buf)
    n += snprintf(buf + n, sizeof buf - n, " groups/block=%d%s", p.group_loop,
                  gamma_in_registers(p) ? " gamma=registers" : "");
  if (p.blocks_per_cu > 0 && n > 0 && n < (int)sizeof buf)
    snprintf(buf + n, sizeof buf - n, " max_blocks/cu=%d", p.blocks_per_cu);
  return buf;
}

}  // namespace qkn

extern "C" {

int qknorm_fused(const qknorm_operand_t* q, const qknorm_operand_t* k, int64_t T, int dtype, float eps,
                 int shards, void* stream) {
  Checked c;
  bool noop;
  const int rc = check_and_plan(qkn::MODE_FUSED, q, k, T, dtype, eps, shards, nullptr, 0, 0, 0, &c, &noop);
  if (rc || noop) return rc;
  return run(qkn::MODE_FUSED, c, stream);
}

int qknorm_partial_stats(const qknorm_operand_t* q, const qknorm_operand_t* k, int64_t T, int dtype, int shards,
                         float* partials, void* stream) {
  Checked c;
  bool noop;
  const int rc =
      check_and_plan(qkn::MODE_STATS, q, k, T, dtype, 0.0f, shards, partials, 0, 0, 0, &c, &noop);
  if (rc || noop) return rc;
  return run(qkn::MODE_STATS, c, stream);
}

int qknorm_apply_with_stats(const qknorm_operand_t* q, const qknorm_operand_t* k, int64_t T, int dtype,
                            float eps, const float* stats, int n_planes, int64_t hq_full, int64_t hk_full,
                            void* stream) {
  Checked c;
  bool noop;
  const int rc = check_and_plan(qkn::MODE_APPLY, q, k, T, dtype, eps, 1, stats, n_planes, hq_full, hk_full, &c,
                                &noop);
  if (rc || noop) return rc;
  return run(qkn::MODE_APPLY, c, stream);
}

const char* qknorm_last_error(void) { return g_last_error.c_str(); }

int qknorm_headwise(const qknorm_operand_t* q, const qknorm_operand_t* k, int64_t T, int dtype, float eps,
                    int64_t head_dim, int64_t gamma_head_stride, void* stream) {
  HeadChecked c;
  bool noop;
  const int rc = check_and_plan_heads(q, k, T, dtype, eps, head_dim, gamma_head_stride, &c, &noop);
  if (rc || noop) return rc;
  std::string err;
  if (qkn::launch_heads(c.plan, c.args, stream, &err)) return fail(QKNORM_ERR_HIP, "qknorm_headwise: %s", err.c_str());
  return ok();
}

int qknorm_describe_headwise_plan(const qknorm_operand_t* q, const qknorm_operand_t* k, int64_t T, int dtype,
                                  int64_t head_dim, int64_t gamma_head_stride, char* buf, size_t len) {
  if (!buf || !len) return fail(QKNORM_ERR_INVALID_ARG, "qknorm_describe_headwise_plan: no output buffer");
  HeadChecked c;
  bool noop;
  const int rc = check_and_plan_heads(q, k, T, dtype, 1e-6f, head_dim, gamma_head_stride, &c, &noop);
  if (rc) return rc;
  const std::string s = noop ? std::string("no-op (T = 0)") : qkn::describe(c.plan);
  snprintf(buf, len, "%s", s.c_str());
  return ok();
}

int qknorm_abi_version(void) { return QKNORM_ABI_VERSION; }

int qknorm_describe_plan(int op, const qknorm_operand_t* q, const qknorm_operand_t* k, int64_t T, int dtype,
                         int shards, char* buf, size_t len) {
  if (op < 0 || op > 2) return fail(QKNORM_ERR_INVALID_ARG, "qknorm_describe_plan: unknown op %d", op);
  if (!buf || !len) return fail(QKNORM_ERR_INVALID_ARG, "qknorm_describe_plan: no output buffer");
  Checked c;
  bool noop;
  // Stand-in statistic buffer address: only compared, never dereferenced.
  // It sits just past the address space the operands use.
  const void* fake = (const void*)(uintptr_t)0xFFFF000000000000ull;
  int64_t hqf = q ? q->h : 0, hkf = k ? k->h : 0;
  const int rc = check_and_plan(op, q, k, T, dtype, 1e-6f, shards, op == qkn::MODE_FUSED ? nullptr : fake, 1,
                                hqf, hkf, &c, &noop);
  if (rc) return rc;
  const std::string s = noop ? std::string("no-op (T = 0)") : qkn::describe(c.plan);
  snprintf(buf, len, "%s", s.c_str());
  return ok();
}

}  // extern "C"
