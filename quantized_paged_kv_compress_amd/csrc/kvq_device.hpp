// kvq_device.hpp -- per-lane building blocks shared by the gfx950 kernels.
//
// Work mapping: one 64-lane wavefront owns one 512-channel row; lane l owns channels
// 8l..8l+7 (one 16-byte bf16 load, or two 16-byte fp32 loads).  The eight-elements-per-
// lane and 128-bit-load choices follow the compressor kernel of "DeepSeek V4 Sparse FP8
// Compressor kernel optimisation with CuteDSL" (vLLM PR #44161 analysis), section 1; on a
// 64-wide wavefront they make one wavefront cover the whole row, and a 32-value scale
// block is exactly one 4-lane DPP quad, so the block absmax needs two DPP max steps and
// no LDS (the wave64 counterpart of the group butterfly of that page's section 3).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvq_layout.hpp"

namespace kvq {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> nearest bfloat16 (ties to even), kept as a float32 value.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float round_bf16(float f) {
    return __uint_as_float(bf16_rne_bits(f) << 16);
}

// ---------------------------------------------------------------- cross-lane
// quad_perm [1,0,3,2] and [2,3,0,1]: exchange within each group of 4 lanes.
__device__ __forceinline__ uint32_t dpp_quad_xor1(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t dpp_quad_xor2(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false));
}
// row_ror:4 and row_ror:8 inside each 16-lane DPP row.
__device__ __forceinline__ uint32_t dpp_row_ror4(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x124, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t dpp_row_ror8(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xF, 0xF, false));
}

// Max over the 4 lanes of a quad, for non-negative float bit patterns (unsigned order
// equals float order for them).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
    v = max(v, dpp_quad_xor1(v));
    v = max(v, dpp_quad_xor2(v));
    return v;
}

// Lane l contributes one byte per quad (block l/4); returns, on every lane of a 16-lane
// row, the dword holding the 4 bytes of that row's 4 blocks (block 4r+j in byte j).
__device__ __forceinline__ uint32_t gather_quad_bytes(uint32_t byte, int lane) {
    uint32_t w = byte << (8 * ((lane >> 2) & 3));
    w |= dpp_row_ror4(w);
    w |= dpp_row_ror8(w);
    return w;
}

// ---------------------------------------------------------------- e4m3 / e2m1
// e4m3fn magnitude code of a non-negative float q, round to nearest even.  For q at or
// above the smallest normal 2^-6 the 20 dropped mantissa bits are rounded in the integer
// domain (a carry moves into the exponent); below it the spacing is 2^-9, so the code is
// the nearest-even integer of q * 2^9 (8 = 2^-6 is the first normal code, which the
// subnormal formula reaches correctly).  Results above 0x7E mean q > 448 + rounding.
__device__ __forceinline__ uint32_t e4m3_mag_code(float q) {
    const uint32_t r = __float_as_uint(q);
    const uint32_t norm = ((r + 0x7FFFFu + ((r >> 20) & 1u)) >> 20) - 960u;  // (e-120)<<3 | m
    const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(q * 512.0f));
    return q >= 0x1p-6f ? norm : sub;
}

// Value of a non-negative e4m3fn magnitude code (0..0x7E).
__device__ __forceinline__ float e4m3_mag_value(uint32_t c) {
    const uint32_t e = c >> 3, m = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : static_cast<float>(m) * 0x1p-9f;
}

// ---------------------------------------------------------------- RoPE
// NeoX half rotation of channels 448..511 (lanes 56..63): channel 448+i (lane 56 + i/8)
// pairs with 480+i (lane 60 + i/8), i.e. lanes l and l^4.  cos_sin_row holds the 32
// cosines then the 32 sines of the position.  Products and sums are rounded one at a
// time (the file is compiled without contraction) and the results rounded to bf16.
// Every lane must call this (the partner exchange is wave-wide).
__device__ __forceinline__ void rope_lane(float (&v)[8], const float* __restrict__ cos_sin_row,
                                          int lane) {
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = __shfl_xor(v[e], 4);
    if (lane >= kWave - kRopeDim / kElemsPerLane) {
        const int i0 = (lane & 3) * kElemsPerLane;
        const float4 c0 = *reinterpret_cast<const float4*>(cos_sin_row + i0);
        const float4 c1 = *reinterpret_cast<const float4*>(cos_sin_row + i0 + 4);
        const float4 s0 = *reinterpret_cast<const float4*>(cos_sin_row + kRopeDim / 2 + i0);
        const float4 s1 = *reinterpret_cast<const float4*>(cos_sin_row + kRopeDim / 2 + i0 + 4);
        const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const bool first_half = lane < kWave - kRopeDim / (2 * kElemsPerLane);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float a = v[e] * c[e];
            const float b = p[e] * s[e];
            v[e] = round_bf16(first_half ? a - b : a + b);
        }
    }
}

// ---------------------------------------------------------------- quantise + store
// Quantise this lane's 8 bf16-valued floats of a row and write its share of the row at
// `slot` (the caller has checked the slot is inside the pool).
template <Layout L>
__device__ __forceinline__ void quantize_store_row(uint8_t* __restrict__ pool, uint32_t slot,
                                                   const float (&v)[8], int lane) {
    using PK = PagedKV<L, kPageBits>;
    uint32_t amax_bits = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax_bits = max(amax_bits, __float_as_uint(v[e]) & 0x7FFFFFFFu);
    amax_bits = quad_max_u32(amax_bits);

    uint8_t* code_row = PK::code_row(pool, slot);
    uint8_t* scale_row = PK::scale_row(pool, slot);
    uint32_t scale_byte;

    if constexpr (L == Layout::V41) {
        // ue8m0: smallest k >= -127 with amax <= 448 * 2^k.  With amax = 2^E * (1+f),
        // amax / 448 = 2^(E-8) * (1+f) / 1.75, so k = E - 8 + (1+f > 1.75): read off the
        // exponent and mantissa bits, no division.  Byte = k + 127, clamped at 0.
        const int biased = static_cast<int>(amax_bits >> 23);
        const int byte = max(0, biased - 8 + static_cast<int>((amax_bits & 0x7FFFFFu) > 0x600000u));
        scale_byte = static_cast<uint32_t>(byte);
        const float inv_scale = __uint_as_float(static_cast<uint32_t>(254 - byte) << 23);  // 2^-k
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sign = (__float_as_uint(v[e]) >> 24) & 0x80u;
            const uint32_t code = e4m3_mag_code(fabsf(v[e]) * inv_scale) | sign;  // exact scaling
            if (e < 4) lo |= code << (8 * e);
            else hi |= code << (8 * (e - 4));
        }
        *reinterpret_cast<uint2*>(code_row + kElemsPerLane * lane) = make_uint2(lo, hi);
    } else {
        // e4m3 scale = RNE(fl32(amax / 6)), held at 448; codes = e2m1 RNE of fl32(x / s).
        // fl32(x / s) lands exactly on a rounding midpoint t only when x / s == t (x has 8
        // significant bits, s 4, t 3), so the code equals counting the midpoints t*s
        // (exact products) that |x| passes, with ">=" at midpoints whose upper
        // neighbour has the even code.
        const float amax = __uint_as_float(amax_bits);
        const float t = amax / 6.0f;  // IEEE-correct single-precision division
        const uint32_t sc = min(e4m3_mag_code(t), 0x7Eu);
        scale_byte = sc;
        const float s = e4m3_mag_value(sc);
        const float m0 = 0.25f * s, m1 = 0.75f * s, m2 = 1.25f * s, m3 = 1.75f * s;
        const float m4 = 2.5f * s, m5 = 3.5f * s, m6 = 5.0f * s;
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float a = fabsf(v[e]);
            uint32_t c = static_cast<uint32_t>(a > m0) + static_cast<uint32_t>(a >= m1) +
                         static_cast<uint32_t>(a > m2) + static_cast<uint32_t>(a >= m3) +
                         static_cast<uint32_t>(a > m4) + static_cast<uint32_t>(a >= m5) +
                         static_cast<uint32_t>(a > m6);
            c |= (__float_as_uint(v[e]) >> 28) & 8u;
            word |= c << (4 * e);
        }
        if (sc == 0) word = 0;  // a zero scale stores all-zero codes
        *reinterpret_cast<uint32_t*>(code_row + LayoutTraits<L>::kCodeBytesPerLane * lane) = word;
    }

    // Scale row: lane 16r writes the dword of blocks 4r..4r+3; FP4 lanes 16r+1 zero the
    // pad dword r.  Four (eight) lanes of one store instruction cover the 16 (32) bytes.
    const uint32_t sw = gather_quad_bytes(scale_byte, lane);
    if ((lane & 15) == 0) *reinterpret_cast<uint32_t*>(scale_row + 4 * (lane >> 4)) = sw;
    if constexpr (L == Layout::V41_FP4) {
        if ((lane & 15) == 1) *reinterpret_cast<uint32_t*>(scale_row + kBlocks + 4 * (lane >> 4)) = 0u;
    }
}

}  // namespace kvq
