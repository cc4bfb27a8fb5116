/*
 * qknorm.h -- layerwise QK-Norm on one MI355X (gfx950), as a C ABI.
 *
 * Library: libqknorm.so (HIP kernels for gfx950 behind plain C entry points).
 *
 * What is computed
 * ----------------
 * Source: "SwiftQK: Fast and Communication-Efficient Tensor Parallelism for
 * Query-Key Normalization" (Kim, Han, Kim; arXiv 2608.09160v1).
 *
 * Layerwise QK-Norm (introduction of the paper) normalizes each token's whole
 * projected Q vector with one RMS factor and, independently, its whole
 * projected K vector with another, before attention; V is not touched. For one
 * vector x of full width H, RMS-Norm (Eq. 1; its body is missing from the
 * page text, and this library reads it as the standard RMSNorm) is
 *
 *     y_j = x_j * gamma_j / sqrt( (sum_i x_i^2) / H + eps ).
 *
 * Phase A of the paper: the only cross-shard quantity the factor needs is the
 * plain sum of squares, so each column shard of x produces one float32
 * partial sum and the global sum is the float32 sum of the partials. Phase B
 * and the final scaling: each element is multiplied by gamma_j (independent
 * of the global sum) and then by the factor r = 1/sqrt(sum/H + eps).
 *
 * Arithmetic (identical in every entry point, so results compose bit for bit):
 *   - inputs are widened exactly to float32;
 *   - partial[s] = float32 sum of x_j^2 over shard s, in a fixed order that
 *     depends only on the shapes, the shard count and T;
 *   - sum = ((partial[0] + partial[1]) + ...) + partial[S-1]   (float32);
 *   - m = fma(sum, 1/H, eps), with 1/H rounded once to float32 on the host;
 *   - r = reciprocal square root of m from the hardware's float32 rsqrt
 *     (within about one float32 ulp; where m would fall below the float32
 *     normal range it is formed from 2^64 * sum and 2^64 * eps instead, both
 *     exact, and r is scaled back by 2^32, keeping that accuracy);
 *   - y_j = (x_j * gamma_j) * r, rounded once to the I/O type (bf16 and FP8:
 *     round to nearest even; FP8 saturates to +-448).
 *   The float32 accumulation is the paper's (Fig. 2(b) accumulates squared
 *   sums in FP32 for BF16 activations); rows whose sum of squares overflows
 *   float32 (|x| around 1e19) give 0 or NaN instead of the real result, and
 *   rows whose squares fall below the float32 normal range (|x| below about
 *   1e-19) lose accuracy in the sum (with eps = 0 and |x| below about 1e-23
 *   the squares vanish and the result is inf or NaN).
 *
 * Data layout
 * -----------
 * An operand describes one of Q or K as row-major rows in device memory:
 * element (t, j) of the input is x[t * ld_x + j], 0 <= t < T, 0 <= j < h.
 * A packed QKV buffer [T, Hq + Hk + Hv] is described by two operands with
 * the same ld (Hq + Hk + Hv): Q at column 0, K at column Hq. V columns and
 * any other memory are never read or written.
 *
 * A shard count S splits each of Q and K into S contiguous column shards of
 * width h/S (h % S == 0 is required): shard s covers columns [s*h/S,
 * (s+1)*h/S). This emulates one rank's view under tensor parallelism.
 *
 * Ownership and streams
 * ---------------------
 * The caller owns every buffer. The library allocates nothing and keeps no
 * state except a per-thread error message. Work is enqueued on `stream` (a
 * hipStream_t; NULL means the default stream of the calling thread's current
 * device) and the call returns without synchronizing. The kernel runs on the
 * stream's device; all pointers are device pointers that this device can
 * access. Calls on different streams or threads are independent; two calls
 * whose outputs overlap race, as any two kernels would. The kernels are
 * built for gfx950 only. The environment variable QKNORM_MAX_GRID, read once
 * when the library first launches a kernel, caps the number of blocks per
 * launch (blocks then loop over several token groups), which leaves compute
 * units to kernels running beside these on other streams; results do not
 * depend on it.
 *
 * Errors
 * ------
 * Argument errors return QKNORM_ERR_INVALID_ARG before anything is launched
 * and nothing is written; QKNORM_ERR_UNSUPPORTED means valid arguments that
 * this library cannot run (a row wider than the kernels hold). With one
 * shard a token's Q plus K columns may span up to 8192 16-byte chunks for
 * bf16 and fp32 and 4096 for FP8 (65536 bf16 / 32768 fp32 / 65536 FP8
 * elements) on the 16-byte path, and about 4096 / 6144 / 2048 chunks on the
 * element-wise path. With S > 1 shards each shard takes a power-of-two lane
 * group of at most 1024/S lanes, so a shard holds proportionally fewer.
 * QKNORM_ERR_HIP means a HIP runtime call failed. qknorm_last_error() gives
 * the message.
 * Faults inside kernels surface at the caller's next synchronization. T == 0
 * is a no-op that returns QKNORM_OK after the scalar arguments are checked.
 * Pointers must be aligned to their element size (bf16 and bf16 gamma: 2
 * bytes; fp32, fp32 gamma and the float32 statistics: 4 bytes); a
 * misaligned element pointer is an argument error. Pointers or strides that
 * are not 16-byte multiples, or shard widths that are not a multiple of 16
 * bytes of elements, are not errors: they run a slower element-wise path
 * with bit-identical results.
 */
#ifndef QKNORM_H
#define QKNORM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKNORM_ABI_VERSION 3

/* Largest shard count and number of statistic planes accepted. */
#define QKNORM_MAX_SHARDS 64
#define QKNORM_MAX_PLANES 64
/* Largest full width H accepted by qknorm_apply_with_stats (exact in float32). */
#define QKNORM_MAX_FULL_WIDTH (1 << 24)

typedef enum qknorm_dtype {
  QKNORM_F32 = 0,      /* float32 rows and gamma */
  QKNORM_BF16 = 1,     /* bfloat16 rows and gamma, float32 arithmetic */
  QKNORM_FP8_E4M3 = 2  /* FP8 E4M3 rows (OCP E4M3FN: bias 7, max 448, NaN 0x7F/0xFF,
                          no infinity), bfloat16 gamma, float32 arithmetic. Outputs are
                          rounded to nearest even and saturated to +-448; NaN stays NaN.
                          Fig. 2(b) of the paper evaluates FP8-E4M3 activations with
                          FP32 accumulation. */
} qknorm_dtype_t;

typedef enum qknorm_status {
  QKNORM_OK = 0,
  QKNORM_ERR_INVALID_ARG = 1,
  QKNORM_ERR_UNSUPPORTED = 2,
  QKNORM_ERR_HIP = 3
} qknorm_status_t;

/* Which entry point a plan is described for (qknorm_describe_plan). */
typedef enum qknorm_op {
  QKNORM_OP_FUSED = 0,
  QKNORM_OP_PARTIAL_STATS = 1,
  QKNORM_OP_APPLY_WITH_STATS = 2
} qknorm_op_t;

/* One of Q or K. */
typedef struct qknorm_operand {
  const void* x;     /* input rows, element (t, j) at x[t*ld_x + j] (elements of the I/O type) */
  int64_t ld_x;      /* input row stride in elements, >= h */
  void* y;           /* output rows, element (t, j) at y[t*ld_y + j]; y == x with ld_y == ld_x
                        is in place; any other overlap with an input or output is rejected.
                        Not used by qknorm_partial_stats (may be NULL there). */
  int64_t ld_y;      /* output row stride in elements, >= h (ignored by qknorm_partial_stats) */
  const void* gamma; /* h per-column scales: the row type, bf16 for FP8 rows
                        (not used by qknorm_partial_stats) */
  int64_t h;         /* local width: number of columns normalized, > 0 */
} qknorm_operand_t;

/*
 * qknorm_fused -- the whole path in one kernel: Phase A partial sums for S
 * shards, their combination, Phase B (x * gamma) and the final scaling
 * (Eq. 1 with H = h, the local width). Each Q/K element is read once and
 * written once.
 *
 *   q, k    operand descriptors (host pointers to structs holding device pointers)
 *   T       tokens (rows), >= 0
 *   dtype   QKNORM_F32, QKNORM_BF16 (x, y and gamma alike) or QKNORM_FP8_E4M3
 *           (x and y FP8, gamma bf16)
 *   eps     finite, >= 0
 *   shards  S in [1, QKNORM_MAX_SHARDS]; q->h % S == 0 and k->h % S == 0
 *   stream  hipStream_t or NULL
 */
int qknorm_fused(const qknorm_operand_t* q, const qknorm_operand_t* k, int64_t T, int dtype,
                 float eps, int shards, void* stream);

/*
 * qknorm_partial_stats -- Phase A alone: the float32 sum of squares of every
 * shard of every row, which is what each tensor-parallel rank would
 * contribute to the exchange.
 *
 *   partials  device float32 [S][2][T]: partials[(s*2 + c)*T + t] is shard s of
 *             Q (c = 0) or K (c = 1) for token t. Must not overlap the inputs.
 *   other arguments as for qknorm_fused (y, ld_y and gamma are ignored).
 */
int qknorm_partial_stats(const qknorm_operand_t* q, const qknorm_operand_t* k, int64_t T,
                         int dtype, int shards, float* partials, void* stream);

/*
 * qknorm_apply_with_stats -- the combination and Phase B / final scaling for a
 * local slice, given the statistic planes received from all shards: the
 * planes are added in order p = 0 .. n_planes-1 in float32 and Eq. 1 divides
 * by the full width (hq_full for Q, hk_full for K), not the local width.
 *
 *   stats     device float32 [n_planes][2][T], same layout as `partials`
 *             (a qknorm_partial_stats output is a valid input, n_planes = S);
 *             n_planes = 1 passes an already combined sum. Must not overlap
 *             the outputs.
 *   n_planes  in [1, QKNORM_MAX_PLANES]
 *   hq_full, hk_full  full widths H, with h <= H_full <= QKNORM_MAX_FULL_WIDTH
 *   q, k, T, dtype, eps, stream as for qknorm_fused.
 *
 * qknorm_fused with S shards gives bit-identical outputs to
 * qknorm_partial_stats with S shards followed by this call with n_planes = S
 * and H_full = h.
 */
int qknorm_apply_with_stats(const qknorm_operand_t* q, const qknorm_operand_t* k, int64_t T,
                            int dtype, float eps, const float* stats, int n_planes,
                            int64_t hq_full, int64_t hk_full, void* stream);

/*
 * qknorm_headwise -- headwise QK-Norm: the paper's introduction names this
 * granularity as one independent normalization factor per attention head.
 * Every head (head_dim contiguous columns; Q has q->h / head_dim heads and K
 * has k->h / head_dim) is normalized with Eq. 1 on its own, H = head_dim:
 * y_j = (x_j * gamma_j) * rsqrt(sum over the head of x^2 / head_dim + eps),
 * with the same float32 arithmetic as the layerwise calls. There is no
 * combination across heads, so nothing here needs an exchange between
 * tensor-parallel ranks.
 *
 *   head_dim           > 0; q->h and k->h must be multiples of it
 *   gamma_head_stride  gamma element (head, j) is gamma[head * stride + j]:
 *                      0 shares one [head_dim] vector across heads (the usual
 *                      per-head RMSNorm weight), head_dim reads a full [h]
 *                      vector; any stride >= 0 is accepted
 *   q, k, T, dtype, eps, stream as for qknorm_fused (gamma holds
 *   (heads - 1) * stride + head_dim elements).
 *
 * Heads of up to 4096 bf16 / 2048 fp32 / 8192 FP8 elements and up to 256 heads per
 * token (Q and K together) are supported; larger ones return
 * QKNORM_ERR_UNSUPPORTED.
 */
int qknorm_headwise(const qknorm_operand_t* q, const qknorm_operand_t* k, int64_t T, int dtype,
                    float eps, int64_t head_dim, int64_t gamma_head_stride, void* stream);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char* qknorm_last_error(void);

/* QKNORM_ABI_VERSION of the built library. */
int qknorm_abi_version(void);

/*
 * qknorm_describe_plan -- writes a one-line description of the launch the
 * given call would make (element-wise or 16-byte path, lanes per shard,
 * chunks per lane, waves per token, and where they apply: token groups per
 * block, gamma held widened in registers, a cap on blocks per compute unit)
 * into buf (NUL-terminated, truncated to len). Validates like the call itself (op selects which one; `shards` is
 * ignored for QKNORM_OP_APPLY_WITH_STATS) and makes no HIP call, so it works
 * without a GPU. Device pointers are only compared, never dereferenced.
 */
int qknorm_describe_plan(int op, const qknorm_operand_t* q, const qknorm_operand_t* k,
                         int64_t T, int dtype, int shards, char* buf, size_t len);

/* As qknorm_describe_plan, for qknorm_headwise. */
int qknorm_describe_headwise_plan(const qknorm_operand_t* q, const qknorm_operand_t* k, int64_t T,
                                  int dtype, int64_t head_dim, int64_t gamma_head_stride, char* buf,
                                  size_t len);

#ifdef __cplusplus
}
#endif

#endif /* QKNORM_H */
