// Shared pieces of the gfx950 engram kernels: bf16 conversion, wave
// reductions and the host-side launch helpers.  Internal to the library.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "engram.h"

namespace engram {

// ---------------------------------------------------------------- device

// f32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Sum over the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// ------------------------------------------------------------------ host

// Records the message of a failed call for engram_last_error (abi.hip).
int32_t fail(int32_t code, const char *fmt, ...);

// Turns the HIP launch status into ENGRAM_E_HIP with a message.
int32_t launch_status(const char *what);

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Where a launcher enqueues: the stream, and optionally a pair of events the
// runtime records with the dispatch of the launcher's first kernel and the
// completion of its last (stage timing; null events = a plain launch).
struct Launch {
    hipStream_t stream = nullptr;
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

template <class F, class... Args>
inline void dispatch(F kernel, dim3 grid, dim3 block, const Launch &l, bool first, bool last,
                     Args... args)
{
    hipExtLaunchKernelGGL(kernel, grid, block, 0, l.stream, first ? l.start : nullptr,
                          last ? l.stop : nullptr, 0, args...);
}

// Hash constants, passed by value as a kernel argument.
struct HashConsts {
    int32_t nl, ng, nh, cols;
    int64_t vocab, pad_id;
    int64_t mult[ENGRAM_MAX_LAYERS * ENGRAM_MAX_NGRAM];
    int64_t prime[ENGRAM_MAX_SLOTS];
    int64_t offset[ENGRAM_MAX_SLOTS];
};

// Launchers (each in its kernel's source file).  Arguments are validated by
// the caller; these only enqueue.
int32_t launch_hash(const HashConsts &c, const int64_t *token_map, const int32_t *ids, int64_t T,
                    int64_t start_pos, int64_t *history, int64_t *row_ids, int32_t *err,
                    const Launch &l);
int32_t launch_gather(const engram_table &tab, const int64_t *row_ids, int64_t T, int32_t cols,
                      int64_t id_stride, uint16_t *rows, int32_t *err, const Launch &l);
int32_t launch_gemv(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t T, int64_t K,
                    int64_t N, const Launch &l);
int32_t launch_gemm(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M, int64_t K,
                    int64_t N, const Launch &l);
int32_t launch_gate(float *h, const uint16_t *kv, const float *qk, int64_t T, int32_t hc,
                    int64_t dim, float eps, const Launch &l);
int32_t launch_qk_product(const uint16_t *q, const uint16_t *k, float *qk, int64_t n,
                          const Launch &l);
int32_t launch_fill_zero(void *p, size_t bytes, const Launch &l);

// GEMV covers T <= kGemvMaxT with K <= kGemvMaxK; larger T goes to the GEMM.
constexpr int64_t kGemvMaxT = 4;
constexpr int64_t kGemvMaxK = 8192;

}  // namespace engram
