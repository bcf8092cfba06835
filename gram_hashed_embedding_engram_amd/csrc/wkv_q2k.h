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
// sub-blocks l, l+64, ..., reading their activations from the token's copy in
// LDS (registers stay few, so eight wavefronts fit on each SIMD to cover the
// LDS and memory latencies).
//
// A weight is bf16(d*scale*q - dmin*min) with q in 0..3 (the table rows'
// decode, rounded the same way), so a sub-block has only four distinct
// weights.  The lane computes those four (fma: exact product, one rounding,
// then v_cvt_pk_bf16_f32's round to nearest even) and spreads their low and
// high bytes into two dwords.  Every four 2-bit quants, after a shift and a
// mask one byte each, are then byte-permute selectors: one permute gathers
// the four weights' low bytes, one their high bytes, and two more interleave
// them into two bf16 weight pairs, each of which meets its pair of
// activations in a v_dot2_f32_bf16.  About three vector instructions a
// weight: the kernel is bound by the vector ALUs, not by the 41 MB a layer
// it reads at the decode shape.
#pragma once

#include "common.h"

namespace engram {

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
    for (int j = 0; j < NLD; j++)     // past the row's end: its last dword again (never staged)
        r[j] = __builtin_nontemporal_load(row + min(j * 64 + lane, row_dwords - 1));
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
// g = lane + 64*i < n_sb (n_sb = K/16, so only the last round, i = NSB-1,
// can leave lanes idle).  xs = the token's activations in LDS as 8-value
// chunks, chunk c at slot xslot(c) (chunks 2g, 2g+1 belong to sub-block g);
// lds = the row's blocks, 21 dwords each.  The order is the one-token projection order of common.h
// (pairs 0, 2, 4, 6 of a sub-block into acc, 1, 3, 5, 7 into acc2), so the
// result equals the bf16 GEMV's over the expanded weights bit for bit.
template <int NSB>
__device__ __forceinline__ float q2k_row_dot(const uint32_t *lds, const u32x4 *xs, int n_sb,
                                             int lane)
{
    float acc = 0.0f, acc2 = 0.0f;
#pragma unroll 1
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
        const u32x4 xa = xs[128 * i + lane], xb = xs[128 * i + 64 + lane];   // xslot(2g), xslot(2g+1)
        const uint32_t x[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t u = (q[j] >> shift) & 0x03030303u;     // quants of values 4j..4j+3
            const uint32_t lo = __builtin_amdgcn_perm(0u, pool_lo, u);   // low bytes of their weights
            const uint32_t hi = __builtin_amdgcn_perm(0u, pool_hi, u);   // high bytes
            const uint32_t wa = __builtin_amdgcn_perm(hi, lo, 0x05010400u);   // values 4j, 4j+1
            const uint32_t wb = __builtin_amdgcn_perm(hi, lo, 0x07030602u);   // values 4j+2, 4j+3
            acc = dot2(wa, x[2 * j], acc);
            acc2 = dot2(wb, x[2 * j + 1], acc2);
        }
    }
    return acc + acc2;
}

}  // namespace engram
