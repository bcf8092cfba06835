// One output row of the one-token projection read straight from wkv's Q2_K
// blocks (atlascybernetics "spark_model/layers/engram_v41.rs",
// EngramLayerWeights::wkv_q2k and EngramV41's engram_v41_wkv_q2k_gemv: wkv
// as the GGUF ships it, [N][K/256] blocks of 84 bytes, 6x fewer bytes a token
// than its bf16 expansion).  Shared by gemv_q2k.hip (stateless) and
// decode.hip (the one-launch decode layer).  Internal to the library.
//
// A wavefront handles one row at a time.  The row's 21*K/256 dwords arrive
// as coalesced dword loads (the row is only 4-byte aligned) and are staged in
// the wavefront's own LDS buffer; lane l then takes the row's 16-value
// sub-blocks l, l+64, ..., with the token's activations for those sub-blocks
// held in registers for the whole kernel.
//
// A weight is bf16(d*scale*q - dmin*min) with q in 0..3 (the table rows'
// decode, rounded the same way), so a sub-block has only four distinct
// weights.  The lane computes those four (fma: exact product, one rounding,
// then v_cvt_pk_bf16_f32's round to nearest even), spreads their low and
// high bytes into two dwords, and turns every four 2-bit quants into two
// bf16 weight pairs with byte permutes: the quants (one byte each after a
// shift and mask) select the low byte and, offset by 4, the high byte.  Each
// pair then meets its pair of activations in a v_dot2_f32_bf16.  About three
// vector instructions a weight: the kernel is bound by the vector ALUs, not
// by the 41 MB a layer it reads at the decode shape.
#pragma once

#include "common.h"

namespace engram {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kQ2kMaxSubBlocks = 8;                       // sub-blocks per lane: K <= 8192
constexpr int kQ2kWkvMaxRowDwords = 21 * (8192 / 256);    // 672

// dwords per lane that cover a row of NSB*1024 values (21 dwords a block)
template <int NSB>
constexpr int q2k_row_loads() { return (84 * NSB + 63) / 64; }

template <int NLD>
__device__ __forceinline__ void q2k_row_load(const uint32_t *__restrict__ row, int row_dwords,
                                             int lane, uint32_t (&r)[NLD])
{
#pragma unroll
    for (int j = 0; j < NLD; j++) {
        const int idx = j * 64 + lane;
        r[j] = idx < row_dwords ? __builtin_nontemporal_load(row + idx) : 0u;
    }
}

template <int NLD>
__device__ __forceinline__ void q2k_row_stage(uint32_t *lds, const uint32_t (&r)[NLD],
                                              int row_dwords, int lane)
{
#pragma unroll
    for (int j = 0; j < NLD; j++) {
        const int idx = j * 64 + lane;
        if (idx < row_dwords)
            lds[idx] = r[j];
    }
}

// The row's dot product with the activations, this lane's share: sub-blocks
// g = lane + 64*i < n_sb (n_sb = K/16); x[i][m] holds the bf16 pair of values
// 16g+2m, 16g+2m+1.  lds = the row's blocks, 21 dwords each.
template <int NSB>
__device__ __forceinline__ float q2k_row_dot(const uint32_t *lds, const uint32_t (&x)[NSB][8],
                                             int n_sb, int lane)
{
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < NSB; i++) {
        const int g = lane + 64 * i;
        if (g >= n_sb)
            break;
        const int b = g >> 4, sb = g & 15;
        const uint32_t *blk = lds + b * 21;
        const uint32_t dd = blk[20];
        const float d = half_bits_to_f32(dd & 0xFFFFu);
        const float dmin = half_bits_to_f32(dd >> 16);
        const uint32_t scb = blk[sb >> 2] >> (8 * (sb & 3));
        const float dl = d * (float)(scb & 15u);
        const float ml = dmin * (float)((scb >> 4) & 15u);
        // the four weights of the sub-block, each rounded as the expansion does
        const bf16x2_t w01 = {(__bf16)fmaf(0.0f, dl, -ml), (__bf16)(dl - ml)};
        const bf16x2_t w23 = {(__bf16)fmaf(2.0f, dl, -ml), (__bf16)fmaf(3.0f, dl, -ml)};
        const uint32_t p01 = __builtin_bit_cast(uint32_t, w01);
        const uint32_t p23 = __builtin_bit_cast(uint32_t, w23);
        // byte q of pool_lo / pool_hi = low / high byte of weight q
        const uint32_t pool_lo = __builtin_amdgcn_perm(p23, p01, 0x06040200u);
        const uint32_t pool_hi = __builtin_amdgcn_perm(p23, p01, 0x07050301u);
        // value v of the sub-block: quant byte 16*(sb&1) + 32*(sb>>3) + v at
        // bit 2*((sb>>1)&3) -- four dwords of quants, one shift
        const uint32_t *q = blk + 4 + 8 * (sb >> 3) + 4 * (sb & 1);
        const int shift = 2 * ((sb >> 1) & 3);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t u = (q[j] >> shift) & 0x03030303u;     // quants of values 4j..4j+3
            const uint32_t u4 = u | 0x04040404u;
            const uint32_t s01 = __builtin_amdgcn_perm(u4, u, 0x05010400u);
            const uint32_t s23 = __builtin_amdgcn_perm(u4, u, 0x07030602u);
            const uint32_t wa = __builtin_amdgcn_perm(pool_hi, pool_lo, s01);
            const uint32_t wb = __builtin_amdgcn_perm(pool_hi, pool_lo, s23);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wa),
                                                  __builtin_bit_cast(bf16x2_t, x[i][2 * j]), acc,
                                                  false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wb),
                                                  __builtin_bit_cast(bf16x2_t, x[i][2 * j + 1]),
                                                  acc, false);
        }
    }
    return acc;
}

}  // namespace engram
