// kvq_kernels.hpp -- gfx950 kernels of the compress -> quantise -> paged-store path.
//
// All kernels are HBM-bound streaming kernels (about 1-2 flop and at most 1/4 exp per
// byte moved), so there is no MFMA here: the design is about wide coalesced loads,
// enough bytes in flight per CU, and keeping every reduction inside a wavefront.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvq_device.hpp"
#include "kvq_layout.hpp"

namespace kvq {

constexpr int kRowsPerBlock = 4;  // one wavefront per row, 4 wavefronts per workgroup

__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
}

__device__ __forceinline__ void load_bf16x8(const uint16_t* __restrict__ p, float (&v)[8]) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming fp32 inputs are read once: non-temporal 16-byte loads.
__device__ __forceinline__ void load_f32x8(const float* __restrict__ p, float (&v)[8]) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// ------------------------------------------------------------------ store / store+RoPE
// One wavefront per bf16 row: load 16 B per lane, optional RoPE, quantise, store.
template <Layout L, bool kRope>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void store_kernel(
    uint8_t* __restrict__ pool, int64_t nslots, const uint16_t* __restrict__ k, int64_t ld,
    const int32_t* __restrict__ pos, const float* __restrict__ cos_sin, int64_t max_pos,
    const int32_t* __restrict__ slots, int64_t n) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave_id();
    if (i >= n) return;
    const int32_t slot = slots[i];
    if (slot < 0 || slot >= nslots) return;
    int32_t p = 0;
    if constexpr (kRope) {
        p = pos[i];
        if (p < 0 || p >= max_pos) return;
    }
    float v[8];
    load_bf16x8(k + i * ld + kElemsPerLane * lane, v);
    if constexpr (kRope) rope_lane(v, cos_sin + static_cast<int64_t>(p) * kRopeDim, lane);
    quantize_store_row<L>(pool, static_cast<uint32_t>(slot), v, lane);
}

// ------------------------------------------------------------------ short-window compressor
// Ratio r <= 4: one wavefront per output row; the r window rows of kv and score are all
// loaded up front (2r + 2r 16-byte loads per lane in flight), so the per-channel maximum
// is exact and needs no online rescaling.  Ratio 1 is the identity and skips the scores.
template <Layout L, int kRatio>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void compress_short_kernel(
    uint8_t* __restrict__ pool, int64_t nslots, const float* __restrict__ kv,
    const float* __restrict__ score, int64_t ld, const int32_t* __restrict__ pos,
    const float* __restrict__ cos_sin, int64_t max_pos, const int32_t* __restrict__ slots,
    int64_t R) {
    static_assert(kRatio >= 1 && kRatio <= 4, "short window");
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave_id();
    if (i >= R) return;
    const int32_t slot = slots[i];
    const int32_t p = pos[i];
    if (slot < 0 || slot >= nslots || p < 0 || p >= max_pos) return;

    const int64_t base = i * kRatio * ld + kElemsPerLane * lane;
    float v[8];
    if constexpr (kRatio == 1) {
        load_f32x8(kv + base, v);
    } else {
        float x[kRatio][8], s[kRatio][8];
#pragma unroll
        for (int j = 0; j < kRatio; ++j) {
            load_f32x8(kv + base + j * ld, x[j]);
            load_f32x8(score + base + j * ld, s[j]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float m = s[0][e];
#pragma unroll
            for (int j = 1; j < kRatio; ++j) m = fmaxf(m, s[j][e]);
            const float mb = m * kLog2e;
            float den = 0.0f, num = 0.0f;
#pragma unroll
            for (int j = 0; j < kRatio; ++j) {
                const float w = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][e], kLog2e, -mb));
                den += w;
                num = __builtin_fmaf(w, x[j][e], num);
            }
            v[e] = num * __builtin_amdgcn_rcpf(den);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = round_bf16(v[e]);
    rope_lane(v, cos_sin + static_cast<int64_t>(p) * kRopeDim, lane);
    quantize_store_row<L>(pool, static_cast<uint32_t>(slot), v, lane);
}

// ------------------------------------------------------------------ long-window compressor
// Large ratios (128): one workgroup of kWaves wavefronts per output row.  Wavefront w
// streams window rows [w*r/kWaves, (w+1)*r/kWaves) in chunks of kChunk rows, keeping a
// per-channel online softmax state (running max m, denominator l, numerator acc) in
// registers (the online form of the vLLM page's section 2, rescaling once per chunk).
// The kWaves partial states are merged through LDS by wavefront 0 -- the only LDS use in
// the library -- which then rounds, rotates, quantises and stores the row.
template <Layout L, int kRatio, int kWaves, int kChunk>
__global__ __launch_bounds__(kWave * kWaves) void compress_long_kernel(
    uint8_t* __restrict__ pool, int64_t nslots, const float* __restrict__ kv,
    const float* __restrict__ score, int64_t ld, const int32_t* __restrict__ pos,
    const float* __restrict__ cos_sin, int64_t max_pos, const int32_t* __restrict__ slots,
    int64_t R) {
    constexpr int kRowsPerWave = kRatio / kWaves;
    static_assert(kRatio % kWaves == 0 && kRowsPerWave % kChunk == 0, "window split");
    __shared__ float4 part[kWaves - 1][3][kWave * 2];

    const int64_t i = blockIdx.x;
    const int32_t slot = slots[i];
    const int32_t p = pos[i];
    if (slot < 0 || slot >= nslots || p < 0 || p >= max_pos) return;  // whole workgroup

    const int lane = threadIdx.x & (kWave - 1);
    const int w = wave_id();
    const int64_t base = (i * kRatio + static_cast<int64_t>(w) * kRowsPerWave) * ld + kElemsPerLane * lane;

    float m[8], l[8], acc[8];  // m in log2 units
#pragma unroll
    for (int e = 0; e < 8; ++e) { m[e] = -__builtin_inff(); l[e] = 0.0f; acc[e] = 0.0f; }

#pragma unroll 1
    for (int c = 0; c < kRowsPerWave; c += kChunk) {
        float x[kChunk][8], s[kChunk][8];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            load_f32x8(kv + base + (c + j) * ld, x[j]);
            load_f32x8(score + base + (c + j) * ld, s[j]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float cm = s[0][e];
#pragma unroll
            for (int j = 1; j < kChunk; ++j) cm = fmaxf(cm, s[j][e]);
            const float mn = fmaxf(m[e], cm * kLog2e);
            const float alpha = __builtin_amdgcn_exp2f(m[e] - mn);
            float le = l[e] * alpha, ae = acc[e] * alpha;
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                const float wt = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][e], kLog2e, -mn));
                le += wt;
                ae = __builtin_fmaf(wt, x[j][e], ae);
            }
            m[e] = mn; l[e] = le; acc[e] = ae;
        }
    }

    if (w != 0) {
        float4* dst = &part[w - 1][0][2 * lane];
        dst[0] = make_float4(m[0], m[1], m[2], m[3]);
        dst[1] = make_float4(m[4], m[5], m[6], m[7]);
        dst = &part[w - 1][1][2 * lane];
        dst[0] = make_float4(l[0], l[1], l[2], l[3]);
        dst[1] = make_float4(l[4], l[5], l[6], l[7]);
        dst = &part[w - 1][2][2 * lane];
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    __syncthreads();
    if (w != 0) return;

    float pm[kWaves - 1][8], pl[kWaves - 1][8], pa[kWaves - 1][8];
#pragma unroll
    for (int q = 0; q < kWaves - 1; ++q) {
        const float4* src = &part[q][0][2 * lane];
        pm[q][0] = src[0].x; pm[q][1] = src[0].y; pm[q][2] = src[0].z; pm[q][3] = src[0].w;
        pm[q][4] = src[1].x; pm[q][5] = src[1].y; pm[q][6] = src[1].z; pm[q][7] = src[1].w;
        src = &part[q][1][2 * lane];
        pl[q][0] = src[0].x; pl[q][1] = src[0].y; pl[q][2] = src[0].z; pl[q][3] = src[0].w;
        pl[q][4] = src[1].x; pl[q][5] = src[1].y; pl[q][6] = src[1].z; pl[q][7] = src[1].w;
        src = &part[q][2][2 * lane];
        pa[q][0] = src[0].x; pa[q][1] = src[0].y; pa[q][2] = src[0].z; pa[q][3] = src[0].w;
        pa[q][4] = src[1].x; pa[q][5] = src[1].y; pa[q][6] = src[1].z; pa[q][7] = src[1].w;
    }
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float M = m[e];
#pragma unroll
        for (int q = 0; q < kWaves - 1; ++q) M = fmaxf(M, pm[q][e]);
        const float a0 = __builtin_amdgcn_exp2f(m[e] - M);
        float den = l[e] * a0, num = acc[e] * a0;
#pragma unroll
        for (int q = 0; q < kWaves - 1; ++q) {
            const float a = __builtin_amdgcn_exp2f(pm[q][e] - M);
            den = __builtin_fmaf(pl[q][e], a, den);
            num = __builtin_fmaf(pa[q][e], a, num);
        }
        v[e] = round_bf16(num * __builtin_amdgcn_rcpf(den));
    }
    rope_lane(v, cos_sin + static_cast<int64_t>(p) * kRopeDim, lane);
    quantize_store_row<L>(pool, static_cast<uint32_t>(slot), v, lane);
}

// ------------------------------------------------------------------ dequant
// One wavefront per output row (page p of the list, row r): lane l reads its 8 codes
// and the scale byte of its block, and writes 8 bf16 (16 B).
template <Layout L>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void dequant_kernel(
    const uint8_t* __restrict__ pool, int64_t num_pages, const int32_t* __restrict__ page_ids,
    int64_t P, uint16_t* __restrict__ out) {
    using T = LayoutTraits<L>;
    constexpr int64_t kPB = kv_page_bytes<L>(1 << kPageBits);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave_id();
    if (g >= P * (1 << kPageBits)) return;
    const int32_t page = page_ids[g >> kPageBits];
    if (page < 0 || page >= num_pages) return;
    const int row = static_cast<int>(g & ((1 << kPageBits) - 1));
    const uint8_t* pg = pool + static_cast<int64_t>(page) * kPB;
    const uint8_t* code_row = pg + row * T::kCodeRowBytes;
    const uint32_t sb = pg[(int64_t(1) << kPageBits) * T::kCodeRowBytes + row * T::kScaleRowBytes + (lane >> 2)];

    uint32_t o[8];
    if constexpr (L == Layout::V41) {
        const uint2 cw = *reinterpret_cast<const uint2*>(code_row + kElemsPerLane * lane);
        const int k = static_cast<int>(sb) - 127;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t c = ((e < 4 ? cw.x : cw.y) >> (8 * (e & 3))) & 0xFFu;
            const uint32_t mag = c & 0x7Fu;
            const float val = __builtin_amdgcn_ldexpf(e4m3_mag_value(mag), k);  // exact unless it
            uint32_t b = bf16_rne_bits(val) | ((c & 0x80u) << 8);               // under/overflows
            if (mag == 0x7Fu || sb == 0xFFu) b = 0x7FC0u;
            o[e] = b;
        }
    } else {
        const uint32_t cw = *reinterpret_cast<const uint32_t*>(code_row + T::kCodeBytesPerLane * lane);
        const bool nan_scale = (sb & 0x7Fu) == 0x7Fu;
        const float s = (sb & 0x80u) ? -e4m3_mag_value(sb & 0x7Fu) : e4m3_mag_value(sb & 0x7Fu);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t nib = (cw >> (4 * e)) & 0xFu;
            const uint32_t ex = (nib >> 1) & 3u, mb = nib & 1u;
            const float mag = ex ? __uint_as_float(((ex + 126u) << 23) | (mb << 22)) : 0.5f * static_cast<float>(mb);
            const float val = ((nib & 8u) ? -mag : mag) * s;  // exact: at most 5 significant bits
            o[e] = nan_scale ? 0x7FC0u : bf16_rne_bits(val);
        }
    }
    uint4 st;
    st.x = o[0] | (o[1] << 16);
    st.y = o[2] | (o[3] << 16);
    st.z = o[4] | (o[5] << 16);
    st.w = o[6] | (o[7] << 16);
    *reinterpret_cast<uint4*>(out + g * kHeadDim + kElemsPerLane * lane) = st;
}

// ------------------------------------------------------------------ full -> SWA slots
__global__ __launch_bounds__(256) void translate_kernel(const int32_t* __restrict__ table,
                                                        int64_t table_len,
                                                        const int32_t* __restrict__ full,
                                                        int64_t n, int32_t* __restrict__ out,
                                                        int64_t cap) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= cap) return;
    int32_t v = 0;
    if (i < n) {
        const int32_t f = full[i];
        v = (f >= 0 && f < table_len) ? table[f] : -1;
    }
    out[i] = v;
}

}  // namespace kvq
