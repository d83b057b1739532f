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

// ------------------------------------------------------------------ store / store+RoPE
// One wavefront per bf16 row: two 8-byte loads per lane, optional RMS norm (kNorm, always
// followed by RoPE), optional RoPE, quantise, store.
template <Layout L, bool kRope, bool kNorm>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void store_kernel(
    uint8_t* __restrict__ pool, int64_t nslots, const uint16_t* __restrict__ k, int64_t ld,
    const uint16_t* __restrict__ weight, float eps, const int32_t* __restrict__ pos,
    const float* __restrict__ cos_sin, int64_t max_pos, const int32_t* __restrict__ slots, int64_t n) {
    static_assert(kRope || !kNorm, "the norm is fused with RoPE");
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave_id();
    if (i >= n) return;
    const int32_t slot = slots[i];
    if (slot < 0 || slot >= nslots) return;
    RopeCS cs;
    if constexpr (kRope) {
        const int32_t p = pos[i];
        if (p < 0 || p >= max_pos) return;
        rope_load_cs(cos_sin + static_cast<int64_t>(p) * kRopeDim, lane, cs);
    }
    float v[8];
    load_row_bf16(k + i * ld, lane, v);
    if constexpr (kNorm) rms_norm_row(v, weight, eps, lane);
    if constexpr (kRope) rope_apply(v, cs, lane);
    quantize_store_row<L>(pool, static_cast<uint32_t>(slot), v, lane);
}

// ------------------------------------------------------------------ short-window compressor
// Ratio r <= 4: one wavefront per output row; the r window rows of kv and score are all
// loaded up front (4r 16-byte loads per lane in flight), so the per-channel maximum is
// exact and needs no online rescaling.  The loads and the cos/sin gather are issued
// before the slot / position checks (which only gate the stores), so a wavefront waits
// on memory once.  Ratio 1 is the identity and skips the scores.
template <Layout L, int kRatio>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void compress_short_kernel(
    uint8_t* __restrict__ pool, int64_t nslots, const float* __restrict__ kv,
    const float* __restrict__ score, int64_t ld, const int32_t* __restrict__ pos,
    const float* __restrict__ cos_sin, int64_t max_pos, const int32_t* __restrict__ slots,
    int64_t R) {
    static_assert(kRatio >= 1 && kRatio <= 4, "short window");
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t i_raw = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave_id();
    const int64_t i = i_raw < R ? i_raw : R - 1;  // rows past R (last block) read row R-1, store nothing

    const int64_t base = i * kRatio * ld;
    float x[kRatio][8];
    float s[kRatio > 1 ? kRatio : 1][8];
#pragma unroll
    for (int j = 0; j < kRatio; ++j) {
        load_row_f32(kv + base + j * ld, lane, x[j]);
        if constexpr (kRatio > 1) load_row_f32(score + base + j * ld, lane, s[j]);
    }
    const int32_t slot = slots[i];
    const int32_t p = pos[i];
    const bool valid = i_raw < R && slot >= 0 && slot < nslots && p >= 0 && p < max_pos;
    RopeCS cs;
    rope_load_cs(cos_sin + static_cast<int64_t>(valid ? p : 0) * kRopeDim, lane, cs);

    float v[8];
    if constexpr (kRatio == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = x[0][e];
    } else {
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
    rope_apply(v, cs, lane);
    if (!valid) return;
    quantize_store_row<L>(pool, static_cast<uint32_t>(slot), v, lane);
}

// ------------------------------------------------------------------ long-window compressor
// Large ratios (8..128): one workgroup of kWaves wavefronts per output row.  The window is
// cut into chunks of kChunk rows dealt round-robin to the wavefronts (wavefront w folds
// chunks w, w + kWaves, ...), so the whole workgroup sweeps its window front to back
// together -- measured on MI355X about 3 % faster than giving each wavefront a contiguous
// slice.  Each wavefront double-buffers its chunks (the next chunk's loads are in flight
// while the current one is folded in; a share of at most four chunks is loaded whole
// before folding, which measured faster at ratio 64) and keeps a per-channel online softmax state --
// running max m (log2 units), denominator l, numerator acc -- rescaling once per chunk
// (the online form of the vLLM page's section 2).  The kWaves partial states are merged
// through LDS by wavefront 0 -- the only LDS use in the library -- which then rounds,
// rotates, quantises and stores the row.
template <int kChunk>
__device__ __forceinline__ void load_chunk(const float* __restrict__ kv, const float* __restrict__ score,
                                           int64_t base, int64_t ld, int lane, float (&x)[kChunk][8],
                                           float (&s)[kChunk][8]) {
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
        load_row_f32(kv + base + j * ld, lane, x[j]);
        load_row_f32(score + base + j * ld, lane, s[j]);
    }
}

template <int kChunk>
__device__ __forceinline__ void fold_chunk(const float (&x)[kChunk][8], const float (&s)[kChunk][8],
                                           float (&m)[8], float (&l)[8], float (&acc)[8]) {
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

template <Layout L, int kRatio, int kWaves, int kChunk>
__global__ __launch_bounds__(kWave * kWaves) void compress_long_kernel(
    uint8_t* __restrict__ pool, int64_t nslots, const float* __restrict__ kv,
    const float* __restrict__ score, int64_t ld, const int32_t* __restrict__ pos,
    const float* __restrict__ cos_sin, int64_t max_pos, const int32_t* __restrict__ slots,
    int64_t R) {
    constexpr int kChunksPerWave = kRatio / (kWaves * kChunk);
    static_assert(kRatio % (kWaves * kChunk) == 0 && kChunksPerWave % 2 == 0, "window split");
    __shared__ float4 part[kWaves - 1][3][kWave * 2];

    const int64_t i = blockIdx.x;
    const int32_t slot = slots[i];
    const int32_t p = pos[i];
    if (slot < 0 || slot >= nslots || p < 0 || p >= max_pos) return;  // whole workgroup

    const int lane = threadIdx.x & (kWave - 1);
    const int w = wave_id();
    const int64_t base = (i * kRatio + static_cast<int64_t>(w) * kChunk) * ld;   // chunk w
    const int64_t step = static_cast<int64_t>(kWaves) * kChunk * ld;            // to chunk w + kWaves

    float m[8], l[8], acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { m[e] = -__builtin_inff(); l[e] = 0.0f; acc[e] = 0.0f; }

    if constexpr (kChunksPerWave <= 4) {
        // the wavefront's whole share fits in registers: issue every load, then fold
        float x[kChunksPerWave][kChunk][8], sc[kChunksPerWave][kChunk][8];
#pragma unroll
        for (int c = 0; c < kChunksPerWave; ++c) load_chunk<kChunk>(kv, score, base + c * step, ld, lane, x[c], sc[c]);
#pragma unroll
        for (int c = 0; c < kChunksPerWave; ++c) fold_chunk<kChunk>(x[c], sc[c], m, l, acc);
    } else {
        float xa[kChunk][8], sa[kChunk][8], xb[kChunk][8], sb[kChunk][8];
        load_chunk<kChunk>(kv, score, base, ld, lane, xa, sa);
#pragma unroll 1
        for (int c = 0; c < kChunksPerWave; c += 2) {
            load_chunk<kChunk>(kv, score, base + (c + 1) * step, ld, lane, xb, sb);
            fold_chunk<kChunk>(xa, sa, m, l, acc);
            if (c + 2 < kChunksPerWave) load_chunk<kChunk>(kv, score, base + (c + 2) * step, ld, lane, xa, sa);
            fold_chunk<kChunk>(xb, sb, m, l, acc);
        }
    }

    RopeCS cs;
    if (w == 0) rope_load_cs(cos_sin + static_cast<int64_t>(p) * kRopeDim, lane, cs);
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

    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float pm[kWaves - 1], pl[kWaves - 1], pa[kWaves - 1];
        float M = m[e];
#pragma unroll
        for (int q = 0; q < kWaves - 1; ++q) {
            pm[q] = reinterpret_cast<const float*>(&part[q][0][2 * lane])[e];
            pl[q] = reinterpret_cast<const float*>(&part[q][1][2 * lane])[e];
            pa[q] = reinterpret_cast<const float*>(&part[q][2][2 * lane])[e];
            M = fmaxf(M, pm[q]);
        }
        const float a0 = __builtin_amdgcn_exp2f(m[e] - M);
        float den = l[e] * a0, num = acc[e] * a0;
#pragma unroll
        for (int q = 0; q < kWaves - 1; ++q) {
            const float a = __builtin_amdgcn_exp2f(pm[q] - M);
            den = __builtin_fmaf(pl[q], a, den);
            num = __builtin_fmaf(pa[q], a, num);
        }
        v[e] = round_bf16(num * __builtin_amdgcn_rcpf(den));
    }
    rope_apply(v, cs, lane);
    quantize_store_row<L>(pool, static_cast<uint32_t>(slot), v, lane);
}

// ------------------------------------------------------------------ decode-step compressor state
// One row per state (sequence) per call: fold the row into the state's online softmax
// (m in log2 units, l, acc per channel; 3 x 512 fp32 in channel order), count it, and
// when the window is complete, finalise like the window kernels (acc / l rounded to bf16,
// RoPE at the completing row's position, quantise, store at its slot) and reset the
// count.  count == 0 means an empty state, so a zeroed buffer is a valid start.
template <Layout L>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void compress_state_kernel(
    uint8_t* __restrict__ pool, int64_t nslots, float* __restrict__ state, int32_t* __restrict__ count,
    int64_t num_states, int32_t ratio, const int32_t* __restrict__ state_ids, const float* __restrict__ kv,
    const float* __restrict__ score, int64_t ld, const int32_t* __restrict__ pos,
    const float* __restrict__ cos_sin, int64_t max_pos, const int32_t* __restrict__ slots, int64_t n) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t j = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave_id();
    if (j >= n) return;
    const int32_t sid = state_ids[j];
    if (sid < 0 || sid >= num_states) return;
    float x[8], s[8];
    load_row_f32(kv + j * ld, lane, x);
    load_row_f32(score + j * ld, lane, s);
    float* st = state + static_cast<int64_t>(sid) * 3 * kHeadDim;
    const int32_t c = count[sid];
    float m[8], l[8], acc[8];
    if (c == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { m[e] = s[e] * kLog2e; l[e] = 1.0f; acc[e] = x[e]; }
    } else {
        float pm[8], pl[8], pa[8];
        load_row_f32(st, lane, pm);
        load_row_f32(st + kHeadDim, lane, pl);
        load_row_f32(st + 2 * kHeadDim, lane, pa);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float mn = fmaxf(pm[e], s[e] * kLog2e);
            const float alpha = __builtin_amdgcn_exp2f(pm[e] - mn);
            const float w = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], kLog2e, -mn));
            m[e] = mn;
            l[e] = __builtin_fmaf(pl[e], alpha, w);
            acc[e] = __builtin_fmaf(pa[e], alpha, w * x[e]);
        }
    }
    if (c + 1 < ratio) {
        float* dst[3] = {st, st + kHeadDim, st + 2 * kHeadDim};
        const float* src[3] = {m, l, acc};
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            *reinterpret_cast<float4*>(dst[q] + 4 * lane) = make_float4(src[q][0], src[q][1], src[q][2], src[q][3]);
            *reinterpret_cast<float4*>(dst[q] + kHalf + 4 * lane) = make_float4(src[q][4], src[q][5], src[q][6], src[q][7]);
        }
        if (lane == 0) count[sid] = c + 1;
        return;
    }
    if (lane == 0) count[sid] = 0;  // the window is complete: the state is consumed
    const int32_t p = pos[j];
    const int32_t slot = slots[j];
    const bool valid = slot >= 0 && slot < nslots && p >= 0 && p < max_pos;
    RopeCS cs;
    rope_load_cs(cos_sin + static_cast<int64_t>(valid ? p : 0) * kRopeDim, lane, cs);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = round_bf16(acc[e] * __builtin_amdgcn_rcpf(l[e]));
    rope_apply(v, cs, lane);
    if (!valid) return;
    quantize_store_row<L>(pool, static_cast<uint32_t>(slot), v, lane);
}

// ------------------------------------------------------------------ dequant
// Lane l's share of one stored row: its 8 codes (channels 8l..8l+7; one 8-byte V41 load
// or one 4-byte FP4 load) and the scale byte of its block.
template <Layout L>
__device__ __forceinline__ void load_stored_row(const uint8_t* __restrict__ pg, int row, int lane,
                                                uint32_t (&cw)[2], uint32_t& sb) {
    using T = LayoutTraits<L>;
    const uint8_t* code_row = pg + row * T::kCodeRowBytes;
    if constexpr (L == Layout::V41) {
        const uint2 c = *reinterpret_cast<const uint2*>(code_row + kElemsPerLane * lane);
        cw[0] = c.x;
        cw[1] = c.y;
    } else {
        cw[0] = *reinterpret_cast<const uint32_t*>(code_row + T::kCodeBytesPerLane * lane);
        cw[1] = 0;
    }
    sb = pg[(int64_t(1) << kPageBits) * T::kCodeRowBytes + row * T::kScaleRowBytes + (lane >> 2)];
}

// decode(code) * decode(scale) in fp32, rounded to bf16; NaN codes or scales give 0x7FC0.
// Writes the lane's 8 bf16 values (16 bytes) at dst.
template <Layout L>
__device__ __forceinline__ void dequant_lane(const uint32_t (&cw)[2], uint32_t sb, uint16_t* __restrict__ dst,
                                             int lane) {
    uint32_t o[8];
    if constexpr (L == Layout::V41) {
        const int k = static_cast<int>(sb) - 127;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t c = (cw[e >> 2] >> (8 * (e & 3))) & 0xFFu;
            const uint32_t mag = c & 0x7Fu;
            const float val = __builtin_amdgcn_ldexpf(e4m3_mag_value(mag), k);  // exact unless it
            uint32_t b = bf16_rne_bits(val) | ((c & 0x80u) << 8);               // under/overflows
            if (mag == 0x7Fu || sb == 0xFFu) b = 0x7FC0u;
            o[e] = b;
        }
    } else {
        const bool nan_scale = (sb & 0x7Fu) == 0x7Fu;
        const float s = (sb & 0x80u) ? -e4m3_mag_value(sb & 0x7Fu) : e4m3_mag_value(sb & 0x7Fu);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t nib = (cw[0] >> (4 * e)) & 0xFu;
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
    *reinterpret_cast<uint4*>(dst + kElemsPerLane * lane) = st;
}

// Whole pages: each wavefront dequantises kRowsPerWave consecutive rows of one listed
// page (all loads issued before any use).  One row per wavefront suits short page lists
// (more wavefronts to spread the launch); longer lists use 4 rows per wavefront to keep
// more bytes in flight per wavefront.
template <Layout L, int kRowsPerWave>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void dequant_kernel(
    const uint8_t* __restrict__ pool, int64_t num_pages, const int32_t* __restrict__ page_ids,
    int64_t P, uint16_t* __restrict__ out) {
    static_assert((1 << kPageBits) % kRowsPerWave == 0, "a wavefront stays inside one page");
    constexpr int64_t kPB = kv_page_bytes<L>(1 << kPageBits);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t g0 = (static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave_id()) * kRowsPerWave;
    if (g0 >= P * (1 << kPageBits)) return;
    const int32_t page = page_ids[g0 >> kPageBits];
    if (page < 0 || page >= num_pages) return;
    const int row0 = static_cast<int>(g0 & ((1 << kPageBits) - 1));
    const uint8_t* pg = pool + static_cast<int64_t>(page) * kPB;
    uint32_t cw[kRowsPerWave][2], sb[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) load_stored_row<L>(pg, row0 + r, lane, cw[r], sb[r]);
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) dequant_lane<L>(cw[r], sb[r], out + (g0 + r) * kHeadDim, lane);
}

// Token gather: output row g is the dequantised row at slots[g]; rows whose slot is
// outside the pool are left untouched.
template <Layout L>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void dequant_slots_kernel(
    const uint8_t* __restrict__ pool, int64_t nslots, const int32_t* __restrict__ slots, int64_t n,
    uint16_t* __restrict__ out) {
    constexpr int64_t kPB = kv_page_bytes<L>(1 << kPageBits);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave_id();
    if (g >= n) return;
    const int32_t slot = slots[g];
    if (slot < 0 || slot >= nslots) return;
    const uint8_t* pg = pool + static_cast<int64_t>(slot >> kPageBits) * kPB;
    uint32_t cw[2], sb;
    load_stored_row<L>(pg, slot & ((1 << kPageBits) - 1), lane, cw, sb);
    dequant_lane<L>(cw, sb, out + g * kHeadDim, lane);
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
