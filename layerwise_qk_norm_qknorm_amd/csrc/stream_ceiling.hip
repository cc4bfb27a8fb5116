// Streaming reference kernels: the practical HBM ceiling that the QK-Norm
// kernels are measured against. Benchmark-side only (libstreamceil.so, loaded
// by bench.py); this is not part of the QK-Norm boundary and computes nothing
// of the method.
//
// A kernel here moves the first `row_bytes` bytes of each of `rows` rows of
// stride `ldx` (bytes): either copying them into the same columns of a second
// buffer of stride `ldy` with non-temporal 16-byte stores (the bytes a fused or
// apply call reads and writes once), or only reading them (the bytes a
// partial-statistics call reads). A contiguous buffer is one row. The rows are
// cut into 16-byte chunks numbered row by row; a block of `block` threads
// takes `per` runs of `block` consecutive chunks, so every load instruction of
// a wave reads 64 consecutive chunks (1 KiB) and every thread keeps `per`
// loads in flight before its first store. With `xcd_run` = K > 0, each run of
// 8 K blocks is ordered so that the K blocks the hardware places on one XCD
// (block i on XCD i mod 8) take K consecutive pieces of the rows (measured up
// to 1% faster for the GQA prefill bytes with K = 16). With `nt_loads` = 1 the
// loads are non-temporal too, as the QK-Norm kernels' row loads are.
//
// C ABI (ctypes from bench.py):
//   int qkceil_stream(const void* x, int64_t ldx, void* y, int64_t ldy,
//                     int64_t rows, int64_t row_bytes, int per, int block,
//                     int xcd_run, int nt_loads, void* sink, void* stream);
//     y != NULL: copy; y == NULL: read only (sink: a device word that a
//     data-dependent test may write, so the loads are not optimised away).
//     xcd_run: 0 (blocks in order) or 2, 4, 8, 16 (see above); nt_loads: 0 or 1.
//     Returns 0, or 1 for an invalid argument (nothing launched) and 3 for a
//     launch failure; the message is in qkceil_last_error().
//   const char* qkceil_last_error(void);
//
// Built with QKNORM_BLOCK_CLOCKS (libstreamceil_clocks.so, for bench.py
// --timeline), the kernel also records per block the 100 MHz real-time
// counter at its start and, once its loads and stores have completed, at its
// end, with the XCC and hardware ids of its CU, into the buffer set by
//   void qkceil_set_block_clocks(void* clocks);   (3 words per block, or NULL)

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

thread_local std::string g_err;
#ifdef QKNORM_BLOCK_CLOCKS
unsigned long long* g_clocks = nullptr;
#endif

template <int PER, bool COPY, int XK, bool NTL>
__global__ void __launch_bounds__(1024) stream_rows(const char* __restrict__ x, int64_t ldx, char* __restrict__ y,
                                                     int64_t ldy, uint32_t nc, uint32_t total,
                                                     uint32_t* __restrict__ sink
#ifdef QKNORM_BLOCK_CLOCKS
                                                     , unsigned long long* clocks
#endif
) {
#ifdef QKNORM_BLOCK_CLOCKS
  if (clocks && threadIdx.x == 0) clocks[3 * (size_t)blockIdx.x] = __builtin_amdgcn_s_memrealtime();
#endif
  const uint32_t b = blockDim.x;
  uint32_t bx = blockIdx.x;
  if (XK > 0) {
    constexpr uint32_t RUN = 8 * XK;
    if (bx < (gridDim.x & ~(RUN - 1))) {
      const uint32_t r = bx & (RUN - 1);
      bx = (bx & ~(RUN - 1)) | ((r & 7) * XK + (r >> 3));
    }
  }
  const uint32_t first = bx * PER * b + threadIdx.x;
  u32x4_t v[PER];
  uint32_t row[PER], col[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    // Past the end: read the last chunk again (a valid address), store nothing.
    const uint32_t f = min(first + k * b, total - 1u);
    row[k] = f / nc;
    col[k] = f - row[k] * nc;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (int64_t)row[k] * ldx + (int64_t)col[k] * 16);
    v[k] = NTL ? __builtin_nontemporal_load(src) : *src;
  }
  // Every load is issued before the first store: the empty asm takes the
  // loaded registers, so no load can be moved into a store's branch.
#pragma unroll
  for (int k = 0; k < PER; ++k) asm volatile("" : "+v"(v[k]));
  if (COPY) {
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (first + k * b < total)
        __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4_t*>(y + (int64_t)row[k] * ldy + (int64_t)col[k] * 16));
  } else {
    uint32_t acc = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    if (acc == 0x9E3779B9u) *sink = acc;  // data-dependent, so the loads stay
  }
#ifdef QKNORM_BLOCK_CLOCKS
  if (clocks) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      clocks[3 * (size_t)blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
      const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_ID
      const unsigned xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
      clocks[3 * (size_t)blockIdx.x + 2] = ((unsigned long long)xcc << 32) | hw;
    }
  }
#endif
}

template <bool COPY, int XK, bool NTL>
void* pick_per(int per) {
  switch (per) {
    case 1: return reinterpret_cast<void*>(stream_rows<1, COPY, XK, NTL>);
    case 2: return reinterpret_cast<void*>(stream_rows<2, COPY, XK, NTL>);
    case 3: return reinterpret_cast<void*>(stream_rows<3, COPY, XK, NTL>);
    case 4: return reinterpret_cast<void*>(stream_rows<4, COPY, XK, NTL>);
    case 6: return reinterpret_cast<void*>(stream_rows<6, COPY, XK, NTL>);
    case 8: return reinterpret_cast<void*>(stream_rows<8, COPY, XK, NTL>);
  }
  return nullptr;
}

template <bool COPY, bool NTL>
void* pick_xk(int per, int xk) {
  switch (xk) {
    case 0: return pick_per<COPY, 0, NTL>(per);
    case 2: return pick_per<COPY, 2, NTL>(per);
    case 4: return pick_per<COPY, 4, NTL>(per);
    case 8: return pick_per<COPY, 8, NTL>(per);
    case 16: return pick_per<COPY, 16, NTL>(per);
  }
  return nullptr;
}

template <bool COPY>
void* pick(int per, int xk, int ntl) {
  return ntl ? pick_xk<COPY, true>(per, xk) : pick_xk<COPY, false>(per, xk);
}

int bad(const char* msg) {
  g_err = msg;
  return 1;
}

}  // namespace

extern "C" {

const char* qkceil_last_error(void) { return g_err.c_str(); }

#ifdef QKNORM_BLOCK_CLOCKS
void qkceil_set_block_clocks(void* clocks) { g_clocks = static_cast<unsigned long long*>(clocks); }
#endif

int qkceil_stream(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t row_bytes, int per,
                  int block, int xcd_run, int nt_loads, void* sink, void* stream) {
  if (!x || (!y && !sink)) return bad("x, and y or sink, are required");
  if ((uintptr_t)x % 16 || (uintptr_t)y % 16 || (uintptr_t)sink % 4) return bad("pointers must be 16-byte aligned");
  if (rows < 1 || row_bytes < 16 || row_bytes % 16) return bad("rows >= 1 and row_bytes a positive multiple of 16");
  if (ldx < row_bytes || ldx % 16 || (y && (ldy < row_bytes || ldy % 16)))
    return bad("strides must be multiples of 16 and >= row_bytes");
  if (block < 64 || block > 1024 || block % 64) return bad("block must be a multiple of 64 in [64, 1024]");
  if (xcd_run != 0 && xcd_run != 2 && xcd_run != 4 && xcd_run != 8 && xcd_run != 16)
    return bad("xcd_run must be 0, 2, 4, 8 or 16");
  if (nt_loads != 0 && nt_loads != 1) return bad("nt_loads must be 0 or 1");
  void* fn = y ? pick<true>(per, xcd_run, nt_loads) : pick<false>(per, xcd_run, nt_loads);
  if (!fn) return bad("per must be 1, 2, 3, 4, 6 or 8");
  const int64_t nc = row_bytes / 16;
  const int64_t total = rows * nc;
  if (total >= ((int64_t)1 << 32) - (int64_t)per * block) return bad("too many chunks for one launch");
  const int64_t grid = (total + (int64_t)per * block - 1) / ((int64_t)per * block);
  const char* xp = static_cast<const char*>(x);
  char* yp = static_cast<char*>(y);
  uint32_t nc32 = (uint32_t)nc, total32 = (uint32_t)total;
  uint32_t* sp = static_cast<uint32_t*>(sink);
#ifdef QKNORM_BLOCK_CLOCKS
  unsigned long long* cp = g_clocks;
  void* args[] = {&xp, &ldx, &yp, &ldy, &nc32, &total32, &sp, &cp};
#else
  void* args[] = {&xp, &ldx, &yp, &ldy, &nc32, &total32, &sp};
#endif
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)block), args, 0,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_err = std::string("kernel launch: ") + hipGetErrorString(e);
    return 3;
  }
  g_err.clear();
  return 0;
}

}  // extern "C"
