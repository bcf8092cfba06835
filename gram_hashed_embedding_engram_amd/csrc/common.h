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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Euclidean remainder a mod p for p > 0, in [0, p).
__device__ __forceinline__ int64_t rem_euclid(int64_t a, int64_t p)
{
    const int64_t r = a % p;
    return r < 0 ? r + p : r;
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// e4m3fn code -> f32, from the format: sign, 4 exponent bits (bias 7), 3
// mantissa bits; exponent 0 is subnormal m * 2^-9; S.1111.111 is NaN, the
// positive quiet NaN for either sign (metrale "deepseek_v41_ref/engram.rs",
// e4m3_to_f32, returns f32::NAN for both codes).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c)
{
    const uint32_t sign = (c & 0x80u) << 24;
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    if (e == 0)
        return __uint_as_float(__float_as_uint((float)m * 0x1p-9f) | sign);
    if (e == 15 && m == 7)              // both NaN codes: the positive quiet NaN
        return __uint_as_float(0x7FC00000u);
    return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

// Values 8*sub .. 8*sub+7 (sub in 0..31) of one Q2_K block, given as its 21
// dwords at b, as four packed bf16 pairs.  Block layout (GGML k-quant; the
// pages give the size only): bytes 0..15 scale/min nibbles of the 16
// sub-blocks of 16 values, bytes 16..79 the 2-bit quants, bytes 80..83 fp16
// d and dmin.  Value e uses quant byte 32*(e/128) + e%32 at bit
// 2*((e%128)/32) and sub-block e/16; for values 8*sub.. that is 8
// consecutive quant bytes at 32*(sub/16) + 8*(sub%4), shift 2*((sub%16)/4),
// sub-block sub/2.  y = d*scale*q - dmin*min: both products are exact in
// f32, so the single subtraction and the bf16 rounding fix the result.
template <class P>
__device__ __forceinline__ u32x4 q2k_dequant8(P b, int sub)
{
    const uint32_t dd = b[20];
    const float d = half_bits_to_f32(dd & 0xFFFFu);
    const float dmin = half_bits_to_f32(dd >> 16);
    const int sb = sub >> 1;
    const uint32_t sc = (b[sb >> 2] >> (8 * (sb & 3))) & 0xFFu;
    const float dl = d * (float)(sc & 15u);
    const float ml = dmin * (float)(sc >> 4);
    const int qw = 4 + 8 * (sub >> 4) + 2 * (sub & 3);      // dword of the 8 quants
    const int shift = 2 * ((sub & 15) >> 2);
    const uint32_t q0 = b[qw] >> shift, q1 = b[qw + 1] >> shift;
    float y[8];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        y[k] = dl * (float)((q0 >> (8 * k)) & 3u) - ml;
        y[4 + k] = dl * (float)((q1 >> (8 * k)) & 3u) - ml;
    }
    u32x4 o;
    o.x = pack_bf16x2(y[0], y[1]);
    o.y = pack_bf16x2(y[2], y[3]);
    o.z = pack_bf16x2(y[4], y[5]);
    o.w = pack_bf16x2(y[6], y[7]);
    return o;
}

// Eight e4m3 codes (two dwords, first code in the low byte) times one
// power-of-two scale, as four packed bf16 pairs (exact: e4m3 x 2^k fits bf16).
__device__ __forceinline__ u32x4 e4m3_dequant8(uint32_t w0, uint32_t w1, float s)
{
    u32x4 o;
    o.x = pack_bf16x2(e4m3_to_f32(w0 & 0xFFu) * s, e4m3_to_f32((w0 >> 8) & 0xFFu) * s);
    o.y = pack_bf16x2(e4m3_to_f32((w0 >> 16) & 0xFFu) * s, e4m3_to_f32(w0 >> 24) * s);
    o.z = pack_bf16x2(e4m3_to_f32(w1 & 0xFFu) * s, e4m3_to_f32((w1 >> 8) & 0xFFu) * s);
    o.w = pack_bf16x2(e4m3_to_f32((w1 >> 16) & 0xFFu) * s, e4m3_to_f32(w1 >> 24) * s);
    return o;
}

// ---- the summation order of every one-token projection
//
// Lane l of the wavefront that owns an output row takes the row's 16-value
// sub-blocks g = l, l+64, l+128, ... (8-value chunks 2g and 2g+1).  In a
// sub-block the bf16 pairs 0, 2, 4, 6 go into one f32 partial sum and the
// pairs 1, 3, 5, 7 into another, one v_dot2_f32_bf16 per pair, in that
// order; the lane's two sums are added, then the 64 lane sums by wave_sum.
// The bf16 GEMV, the one-launch decode kernel and the kernels over Q2_K wkv
// blocks all follow it, so a row gives the same bits whether its weights
// arrive as bf16 or as the Q2_K blocks they expand to.

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + w.lo*x.lo + w.hi*x.hi for two packed bf16 pairs.
__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                           __builtin_bit_cast(bf16x2_t, x), acc, false);
}

// One sub-block: weights wa, wb (chunks 2g, 2g+1) against activations xa, xb.
__device__ __forceinline__ void subblock_dot(const u32x4 &wa, const u32x4 &wb, const u32x4 &xa,
                                             const u32x4 &xb, float &acc, float &acc2)
{
    acc = dot2(wa.x, xa.x, acc);
    acc2 = dot2(wa.y, xa.y, acc2);
    acc = dot2(wa.z, xa.z, acc);
    acc2 = dot2(wa.w, xa.w, acc2);
    acc = dot2(wb.x, xb.x, acc);
    acc2 = dot2(wb.y, xb.y, acc2);
    acc = dot2(wb.z, xb.z, acc);
    acc2 = dot2(wb.w, xb.w, acc2);
}

// Activations kept in LDS for the one-token order: chunk c (8 values) sits at
// slot xslot(c), so lane l's chunks 2g and 2g+1 of sub-block g = 64s + l are
// at 128s + l and 128s + 64 + l -- a wavefront's reads of either are 64
// consecutive 16-byte slots, free of bank conflicts (in chunk order they
// would be 32 bytes apart).  A buffer of kc chunks needs kc rounded up to a
// multiple of 128 slots.
__device__ __forceinline__ int xslot(int c)
{
    return (c & ~127) + ((c & 1) << 6) + ((c & 127) >> 1);
}

// A bf16 row read as NI coalesced 1 KiB loads (lane l holds chunk 64m + l of
// load m) is brought into sub-block order through the wavefront's own 2 KiB
// LDS buffer `stage`, one 128-chunk segment (loads 2s, 2s+1) at a time:
// f(s, a, b) then gets chunks 2g, 2g+1 of sub-block g = 64s + lane, for the
// lanes with g < n_sb.  Only this wavefront touches `stage`, and a
// wavefront's LDS accesses execute in program order, so no barrier is needed.
template <int NI, class F>
__device__ __forceinline__ void for_each_subblock(const u32x4 (&wv)[NI], u32x4 *stage, int lane,
                                                  int n_sb, F f)
{
#pragma unroll
    for (int s = 0; s < (NI + 1) / 2; s++) {
        stage[lane] = wv[2 * s];
        if (2 * s + 1 < NI)
            stage[64 + lane] = wv[2 * s + 1];
        if (64 * s + lane < n_sb)
            f(s, stage[2 * lane], stage[2 * lane + 1]);
    }
}

// v + (v of the lane that DPP control CTRL selects; 0 in rows outside ROWS).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float v)
{
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                             0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false));
}

// Sum over the 64 lanes of a wavefront; every lane gets the total.  All in
// VALU data-parallel moves (no LDS round trips): pairs and quads by quad
// permutes, the 16-lane rows by half-row and row mirrors, then row 0 into
// row 1 and row 2 into row 3 (row_bcast:15), rows 0..1 into row 3
// (row_bcast:31), and lane 63's total read back as a uniform value.  The
// order of the additions is fixed, so the sum is deterministic.
__device__ __forceinline__ float wave_sum(float v)
{
    v = dpp_add<0xB1, 0xF>(v);     // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);     // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xF>(v);    // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);    // row_mirror
    v = dpp_add<0x142, 0xA>(v);    // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);    // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// ------------------------------------------------------------------ host

// Records the message of a failed call for engram_last_error (abi.hip).
int32_t fail(int32_t code, const char *fmt, ...);

// Turns the HIP launch status into ENGRAM_E_HIP with a message.
int32_t launch_status(const char *what);

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Compute units of the current device, which sizes the grids of the
// streaming kernels (queried once per device; 256 if the query fails).
int device_cus();

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
    hipEvent_t start = first ? l.start : nullptr, stop = last ? l.stop : nullptr;
    if (start || stop)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, l.stream, start, stop, 0, args...);
    else   // a plain launch, which stream capture records as a kernel node
        hipLaunchKernelGGL(kernel, grid, block, 0, l.stream, args...);
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
// B sequences of T tokens at position start_pos: ids [B][T], history
// [B][hist_stride], row_ids [B*T][n_layers][cols].
int32_t launch_hash(const HashConsts &c, const int64_t *token_map, const int32_t *ids, int64_t B,
                    int64_t T, int64_t start_pos, int64_t *history, int64_t hist_stride,
                    int64_t *row_ids, int32_t *err, const Launch &l);
int32_t launch_gather(const engram_table &tab, const int64_t *row_ids, int64_t T, int32_t cols,
                      int64_t id_stride, uint16_t *rows, int32_t *err, const Launch &l);
int32_t launch_gemv(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t T, int64_t K,
                    int64_t N, const Launch &l);
// One token through wkv given as Q2_K blocks [N][K/256][84] (gemv_q2k.hip).
int32_t launch_gemv_q2k(const uint16_t *x, const uint8_t *w, uint16_t *y, int64_t K, int64_t N,
                        const Launch &l);
// Blocks 0..n_blocks-1 of a Q2_K array -> bf16 [n_blocks][256] (gather.hip).
int32_t launch_dequant_q2k(const uint8_t *blocks, int64_t n_blocks, uint16_t *out,
                           const Launch &l);
int32_t launch_gemm(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M, int64_t K,
                    int64_t N, const Launch &l);
// advance (nullable): a device position word that workgroup 0 moves one
// step on, up to max_seq, after its row (the last layer of a replayed step);
// err (nullable, graph mode): the device error word -- while it holds
// ENGRAM_DEVERR_POSITION the gate leaves h untouched
int32_t launch_gate(float *h, const uint16_t *kv, const float *qk, int64_t T, int32_t hc,
                    int64_t dim, float eps, const Launch &l, int64_t *advance = nullptr,
                    int64_t max_seq = 0, const int32_t *err = nullptr);
int32_t launch_set_word(int64_t *p, int64_t v, const Launch &l);
int32_t launch_qk_product(const uint16_t *q, const uint16_t *k, float *qk, int64_t n,
                          const Launch &l);
int32_t launch_fill_zero(void *p, size_t bytes, const Launch &l);
int32_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, const Launch &l);

// One decode token through hash, gather + dequant and the projection of one
// layer in a single launch (decode.hip).  first_layer: the token's compressed
// id comes from token_map[*ids] and is recorded in history[pos], and the row
// ids of every layer are written to row_ids [n_layers][cols]; otherwise it is
// read back from history[pos].  rows [cols*256] receives the dequantised rows.
// w_q2k non-null: the projection reads wkv's Q2_K blocks [N][K/256][84]
// instead of the bf16 w.
// The one-launch decode step of B = 2..kDecodeMultiMaxB sequences at one
// position (history [B][hist_stride]); bf16 wkv; n_layers*cols <= 64.
constexpr int64_t kDecodeMultiMaxB = 4;
// The position of a decode step: the host's value, or (word non-null: graph
// replay) a device word holding it, checked on the device against max_seq.
struct DecodePos {
    int64_t pos;
    const int64_t *word;
    int64_t max_seq;
};
int32_t launch_decode_multi(const HashConsts &c, const int64_t *token_map, const int32_t *ids,
                            const DecodePos &pos, int64_t *history, int64_t hist_stride, int32_t layer,
                            bool first_layer, const engram_table &tab, const uint16_t *w,
                            uint16_t *y, int64_t N, int64_t *row_ids, uint16_t *rows,
                            int32_t *err, int64_t B, const Launch &l);
int32_t launch_decode(const HashConsts &c, const int64_t *token_map, const int32_t *ids,
                      const DecodePos &pos, int64_t *history, int32_t layer, bool first_layer,
                      const engram_table &tab, const uint16_t *w, const uint8_t *w_q2k,
                      uint16_t *y, int64_t N, int64_t *row_ids, uint16_t *rows, int32_t *err,
                      const Launch &l);
constexpr int64_t kDecodeMaxCols = 32;      // cols*256 <= 8192 activations in LDS

// The Q2_K-wkv projection holds a token's activations for K <= 8192 in registers.
constexpr int64_t kQ2kWkvMaxK = 8192;

// A few tokens (2..kGemmSmallMaxM) through the MFMA GEMM laid out as a weight
// stream (gemm_small.hip); gemm_small_fits says whether the shape qualifies.
constexpr int64_t kGemmSmallMaxM = 128;
bool gemm_small_fits(int64_t M, int64_t K, int64_t N);
int32_t launch_gemm_small(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M,
                          int64_t K, int64_t N, const Launch &l);

// GEMV covers T <= kGemvMaxT with K <= kGemvMaxK; larger T goes to the GEMM.
constexpr int64_t kGemvMaxT = 4;
constexpr int64_t kGemvMaxK = 8192;
// The multi-token GEMV (2..kGemvMultiMaxT tokens in one pass, activations in
// LDS: T*K <= kGemvMultiMaxX values, 96 KiB).  From 5 tokens the MFMA weight
// stream is faster (and the GEMV's registers spill from 6).
constexpr int64_t kGemvMultiMaxT = 4;
constexpr int64_t kGemvMultiMaxX = 49152;   // values: T * (K rounded up to 1024)
bool gemv_multi_fits(int64_t T, int64_t K);
int32_t launch_gemv_multi(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t T,
                          int64_t K, int64_t N, const Launch &l);

}  // namespace engram
