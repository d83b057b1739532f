// kvq_kernels.hpp -- gfx950 kernels of the compress -> quantise -> paged-store path.
//
// All kernels are HBM-bound streaming kernels (the compressors: one exponential per 8
// input bytes and about 2 float64 flop per byte moved, against a float64 ridge near 10),
// so there is no MFMA here: nothing is a contraction.  The design is about wide coalesced
// loads, enough bytes in flight per CU, each kernel's store policy, and keeping every
// reduction inside a wavefront.
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
// One wavefront per bf16 row: two 8-byte loads per lane (issued before the slot and
// position checks, which only gate the store), optional RMS norm (kNorm, always followed
// by RoPE), optional RoPE, quantise, store.
template <Layout L, bool kRope, bool kNorm>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void store_kernel(
    uint8_t* __restrict__ pool, int64_t nslots, const uint16_t* __restrict__ k, int64_t ld,
    const uint16_t* __restrict__ weight, float eps, const int32_t* __restrict__ pos,
    const float* __restrict__ cos_sin, int64_t max_pos, const int32_t* __restrict__ slots, int64_t n) {
    static_assert(kRope || !kNorm, "the norm is fused with RoPE");
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave_id();
    if (i >= n) return;
    float v[8];
    load_row_bf16(k + i * ld, lane, v);  // issued before the checks, which only gate the store
    const int32_t slot = slots[i];
    RopeCS cs;
    bool valid = slot >= 0 && slot < nslots;
    if constexpr (kRope) {
        const int32_t p = pos[i];
        valid = valid && p >= 0 && p < max_pos;
        rope_load_cs(cos_sin + static_cast<int64_t>(valid ? p : 0) * kRopeDim, lane, cs);
    }
    if (!valid) return;
    if constexpr (kNorm) rms_norm_row(v, weight, eps, lane);
    if constexpr (kRope) rope_apply(v, cs, lane);
    quantize_store_row<L>(pool, static_cast<uint32_t>(slot), v, lane);
}

// ------------------------------------------------------------------ store + RoPE, many layers
// kv_store_rope for up to kMaxLayers layers in one launch: the pool and K pointers of
// every layer travel by value in the kernel arguments.  A wavefront stores one token in
// kLayersPerWave consecutive layers: it issues the token's K row loads of all its layers
// first, then the slot, position and cos/sin loads (shared by its layers), then rotates,
// quantises and stores each row.  Wavefront g takes layer group g / n, token g % n, so
// consecutive wavefronts stream consecutive rows of the same layers.  Measured on MI355X
// at 61 layers x 512 tokens with cold, clean caches: 4 layers per wavefront is 9-12 %
// faster than 1 (fewer wavefronts, each with more loads in flight), 2 and 8 are slower
// than 4, and so are workgroups of 1, 2 or 8 wavefronts.  Non-temporal row stores: 2-4 %
// faster than plain ones right after a large write, 2-3 % slower with clean caches.
constexpr int kMaxLayers = 64;
constexpr int kLayersPerWave = 4;

struct LayerPtrs {
    uint8_t* pool[kMaxLayers];
    const uint16_t* k[kMaxLayers];
};

template <Layout L>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void store_layers_kernel(
    LayerPtrs layers, int32_t num_layers, int64_t nslots, int64_t ld, const int32_t* __restrict__ pos,
    const float* __restrict__ cos_sin, int64_t max_pos, const int32_t* __restrict__ slots, int64_t n) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave_id();
    const int64_t groups = (num_layers + kLayersPerWave - 1) / kLayersPerWave;
    if (g >= n * groups) return;
    const int group = static_cast<int>(g / n);
    const int64_t i = g - static_cast<int64_t>(group) * n;
    const int l0 = group * kLayersPerWave;
    float v[kLayersPerWave][8];
#pragma unroll
    for (int q = 0; q < kLayersPerWave; ++q) {
        const int l = min(l0 + q, num_layers - 1);  // past the last layer: reload it, store nothing
        load_row_bf16(layers.k[l] + i * ld, lane, v[q]);
    }
    const int32_t slot = slots[i];
    const int32_t p = pos[i];
    const bool valid = slot >= 0 && slot < nslots && p >= 0 && p < max_pos;
    RopeCS cs;
    rope_load_cs(cos_sin + static_cast<int64_t>(valid ? p : 0) * kRopeDim, lane, cs);
    if (!valid) return;
#pragma unroll
    for (int q = 0; q < kLayersPerWave; ++q) {
        if (l0 + q < num_layers) {
            rope_apply(v[q], cs, lane);
            quantize_store_row<L, true>(layers.pool[l0 + q], static_cast<uint32_t>(slot), v[q], lane);
        }
    }
}

// ------------------------------------------------------------------ where a compressed row's slot comes from
// Either the caller's slots[i], or -- the full -> SWA translation of the SGLang SWA-hoisting
// page, section 1, fused into the compressor -- table[full[i]] (-1 for a full slot outside
// the table), which is also written to out[i] for the later consumers of the step; the
// wavefronts of the grid then zero out[n:cap] between them, as the separate translation
// does.  table == nullptr selects the plain form.  The kernels take the pointers as
// separate __restrict__ parameters (and rebuild this struct): only then can the compiler
// read slots and table through the scalar cache, off the vector-memory counter that the
// window loads are waited on.
struct SlotSrc {
    const int32_t* slots;  // slots, or full-pool slots when table is set
    const int32_t* table;
    int64_t table_len;
    int32_t* out;          // translated slots [cap]
    int64_t n, cap;
};

__device__ __forceinline__ int32_t row_slot(const SlotSrc& src, int64_t i) {
    const int32_t s = src.slots[i];
    if (src.table == nullptr) return s;
    return (s >= 0 && s < src.table_len) ? src.table[s] : -1;
}

// Row i's translated slot, written back by one lane (fused form only).
__device__ __forceinline__ void put_translated(const SlotSrc& src, int64_t i, int32_t slot, int lane) {
    if (src.table != nullptr && lane == 0 && i < src.n) src.out[i] = slot;
}

// Wavefront `wave` of `num_waves` zeroes its share of out[n:cap] in 64-entry chunks
// (fused form only; the host takes the fused form only when every wavefront has at most
// kMaxTailChunks chunks).
constexpr int64_t kMaxTailChunks = 16;

__device__ __forceinline__ void clear_tail(const SlotSrc& src, int64_t wave, int64_t num_waves, int lane) {
    if (src.table == nullptr) return;
    const int64_t chunks = (src.cap - src.n + 63) / 64;
    for (int64_t c = wave; c < chunks; c += num_waves) {
        const int64_t j = src.n + c * 64 + lane;
        if (j < src.cap) src.out[j] = 0;
    }
}

// ------------------------------------------------------------------ ratio 1 (c1)
// A one-row window pools to the row itself: round the fp32 kv row to bf16, RoPE, quantise,
// store (scores are not read).  One wavefront per row, 4 rows per workgroup; rows past R
// (last block) read row R-1 and store nothing.
template <Layout L>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void compress_c1_kernel(
    uint8_t* __restrict__ pool, int64_t nslots, const float* __restrict__ kv, int64_t ld,
    const int32_t* __restrict__ pos, const float* __restrict__ cos_sin, int64_t max_pos,
    const int32_t* __restrict__ slots, const int32_t* __restrict__ table,
    int64_t table_len, int32_t* __restrict__ out, int64_t cap, int64_t R) {
    const SlotSrc src{slots, table, table_len, out, R, cap};
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t i_raw = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave_id();
    const int64_t i = i_raw < R ? i_raw : R - 1;
    float v[8];
    load_row_f32(kv + i * ld, lane, v);
    // the cos/sin gather depends on the position only, so that it is not held up behind
    // the slot (and, when translating, the table lookup); the slot only gates the store
    const int32_t p = pos[i];
    const bool pos_ok = p >= 0 && p < max_pos;
    RopeCS cs;
    rope_load_cs(cos_sin + static_cast<int64_t>(pos_ok ? p : 0) * kRopeDim, lane, cs);
    clear_tail(src, i_raw, static_cast<int64_t>(gridDim.x) * kRowsPerBlock, lane);
    const int32_t slot = row_slot(src, i);
    put_translated(src, i_raw, slot, lane);
    const bool valid = i_raw < R && pos_ok && slot >= 0 && slot < nslots;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = round_bf16(v[e]);
    rope_apply(v, cs, lane);
    if (!valid) return;
    quantize_store_row<L>(pool, static_cast<uint32_t>(slot), v, lane);
}

// ------------------------------------------------------------------ short-window compressor
// Ratios 2 and 4: one wavefront per output row, the whole window loaded up front (4r
// 16-byte loads per lane in flight), so the per-channel maximum m is exact.  The pooled
// value is computed in float32 with the hardware exp2 -- as cheap as the loads need --
// together with a rigorous bound E on its error against the exact value; wherever the one
// bf16 rounding midpoint next to it lies within E, the channel is recomputed in float64
// from the registers (exp_f64, IEEE division), so the stored bf16 is always the correctly
// rounded exact value.  Ingredients of E (u = 2^-24):
//  - v_exp_f32, measured on gfx950 over every input in [-160, 1]: within 0.79 ulp
//    (< 2^-23 relative) for normal results; results below 2^-126 are flushed to zero, so
//    a channel with an exponent argument below -126 is recomputed;
//  - the argument a = fma(s, L32, -fl(m * L32)) with L32 = fl(log2 e): against the exact
//    (s - m) log2 e it is off by a term common to the window (it cancels in the ratio)
//    plus at most (|a| + 2^-23 |m L32|) (u + 2^-26) in log2 units (|L32 / log2 e - 1| <
//    2^-26), i.e. a relative weight error of ln 2 times that;
//  - the float32 sums of r positive weights and of r products w x: r u (A + |p| l), with
//    A = sum of w |x| and l = sum of w;
//  - the reciprocal and the product that form p = acc / l: 3 u |p|.
// E = 1.01 ((d_w + r u) (A + |p| l) / l + 3 u |p|), d_w = 2^-23 + the argument term.  The
// CPU simulation of the workloads' distributions recomputes about 0.06 % of the values.
template <Layout L, int kRatio, bool kNt>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void compress_short_kernel(
    uint8_t* __restrict__ pool, int64_t nslots, const float* __restrict__ kv,
    const float* __restrict__ score, int64_t ld, const int32_t* __restrict__ pos,
    const float* __restrict__ cos_sin, int64_t max_pos, const int32_t* __restrict__ slots, const int32_t* __restrict__ table,
    int64_t table_len, int32_t* __restrict__ out, int64_t cap,
    int64_t R) {
    const SlotSrc src{slots, table, table_len, out, R, cap};
    static_assert(kRatio == 2 || kRatio == 4, "short window");
    constexpr float kU = 0x1p-24f;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t i_raw = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave_id();
    const int64_t i = i_raw < R ? i_raw : R - 1;  // rows past R (last block) read row R-1, store nothing

    const int64_t base = i * kRatio * ld;
    float x[kRatio][8], s[kRatio][8];
#pragma unroll
    for (int j = 0; j < kRatio; ++j) {
        load_row_f32(kv + base + j * ld, lane, x[j]);
        load_row_f32(score + base + j * ld, lane, s[j]);
    }
    // the cos/sin gather depends on the position only, so that it is not held up behind
    // the slot (and, when translating, the table lookup); the slot only gates the store
    const int32_t p = pos[i];
    const bool pos_ok = p >= 0 && p < max_pos;
    RopeCS cs;
    rope_load_cs(cos_sin + static_cast<int64_t>(pos_ok ? p : 0) * kRopeDim, lane, cs);
    clear_tail(src, i_raw, static_cast<int64_t>(gridDim.x) * kRowsPerBlock, lane);
    const int32_t slot = row_slot(src, i);
    put_translated(src, i_raw, slot, lane);
    const bool valid = i_raw < R && pos_ok && slot >= 0 && slot < nslots;

    float v[8], mx[8];
    uint32_t redo = 0;  // bit e: channel e is recomputed in float64
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float m = s[0][e];
#pragma unroll
        for (int j = 1; j < kRatio; ++j) m = fmaxf(m, s[j][e]);
        mx[e] = m;
        const float mL = m * kLog2e;
        float l = 0.0f, acc = 0.0f, A = 0.0f, amin = 0.0f;
#pragma unroll
        for (int j = 0; j < kRatio; ++j) {
            const float a = __builtin_fmaf(s[j][e], kLog2e, -mL);
            const float w = __builtin_amdgcn_exp2f(a);
            l += w;
            acc = __builtin_fmaf(w, x[j][e], acc);
            A = __builtin_fmaf(w, fabsf(x[j][e]), A);
            amin = fminf(amin, a);
        }
        const float rl = __builtin_amdgcn_rcpf(l);
        const float pc = acc * rl;
        const float ap = fabsf(pc);
        const float dw = 0x1p-23f + (0x1p-23f * fabsf(mL) - amin) * (0.6931472f * 1.25f * kU);
        const float E = 1.01f * ((dw + kRatio * kU) * __builtin_fmaf(ap, l, A) * rl + 3.0f * kU * ap);
        const float mid = __uint_as_float((__float_as_uint(pc) & 0xFFFF0000u) | 0x8000u);
        const bool certain = fabsf(pc - mid) > E && E < ap * 0x1p-10f && ap >= 0x1p-100f &&
                             amin >= -126.0f && fabsf(mL) < 0x1p20f;
        v[e] = round_bf16(pc);
        redo |= certain ? 0u : (1u << e);
    }
    if (redo) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (redo & (1u << e)) {
                const double md = mx[e];
                double den = 0.0, num = 0.0;
#pragma unroll
                for (int j = 0; j < kRatio; ++j) {
                    const double w = exp_f64(static_cast<double>(s[j][e]) - md);
                    den += w;
                    num = __builtin_fma(w, static_cast<double>(x[j][e]), num);
                }
                v[e] = pool_result(den, num);
            }
        }
    }
    rope_apply(v, cs, lane);
    if (!valid) return;
    quantize_store_row<L, kNt>(pool, static_cast<uint32_t>(slot), v, lane);
}

// ------------------------------------------------------------------ window per wavefront
// Ratios 8..32: one wavefront per output row, 4 rows per workgroup, no cross-wavefront
// merge (measured on MI355X faster than a workgroup per row up to ratio 32).  The wavefront keeps kDepth - 1 chunks of kChunk window rows in flight while it
// folds the current one into its float64 online softmax state (PoolF64, exp_tab), with
// the window's first score row as the reference; ratios up to 4 are a single chunk (all
// loads issued at once).  The loads and the cos/sin gather are issued before the slot /
// position checks, which only gate the store; rows past R (last block) read row R-1 and
// store nothing.  From ratio 16 on the row is written with non-temporal stores (measured
// 2-4 % faster at 16 and 32; at ratio 8 plain stores are faster).
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

template <Layout L, int kRatio, int kChunk, int kDepth>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void compress_wave_kernel(
    uint8_t* __restrict__ pool, int64_t nslots, const float* __restrict__ kv,
    const float* __restrict__ score, int64_t ld, const int32_t* __restrict__ pos,
    const float* __restrict__ cos_sin, int64_t max_pos, const int32_t* __restrict__ slots, const int32_t* __restrict__ table,
    int64_t table_len, int32_t* __restrict__ out, int64_t cap,
    int64_t R) {
    const SlotSrc src{slots, table, table_len, out, R, cap};
    constexpr int kChunks = kRatio / kChunk;
    static_assert(kRatio % kChunk == 0 && kDepth >= 2, "window split");
    __shared__ double tab[256];
    ExpTableCopy<kWave * kRowsPerBlock> tcopy;
    tcopy.fetch();
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t i_raw = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave_id();
    const int64_t i = i_raw < R ? i_raw : R - 1;
    const int64_t base = i * kRatio * ld;
    const int64_t step = static_cast<int64_t>(kChunk) * ld;
    float x[kDepth][kChunk][8], sc[kDepth][kChunk][8];
#pragma unroll
    for (int c = 0; c < kDepth - 1 && c < kChunks; ++c)
        load_chunk<kChunk>(kv, score, base + c * step, ld, lane, x[c], sc[c]);
    // the cos/sin gather depends on the position only, so that it is not held up behind
    // the slot (and, when translating, the table lookup); the slot only gates the store
    const int32_t p = pos[i];
    const bool pos_ok = p >= 0 && p < max_pos;
    RopeCS cs;
    rope_load_cs(cos_sin + static_cast<int64_t>(pos_ok ? p : 0) * kRopeDim, lane, cs);
    tcopy.put(tab);
    __syncthreads();  // the exp table is in LDS
    // after the barrier, whose wait would otherwise include the slot's (table) lookup
    clear_tail(src, i_raw, static_cast<int64_t>(gridDim.x) * kRowsPerBlock, lane);
    const int32_t slot = row_slot(src, i);
    put_translated(src, i_raw, slot, lane);
    const bool valid = i_raw < R && pos_ok && slot >= 0 && slot < nslots;

    PoolF64 st;
    pool_init(st, sc[0][0]);
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        if (c + kDepth - 1 < kChunks)
            load_chunk<kChunk>(kv, score, base + (c + kDepth - 1) * step, ld, lane, x[(c + kDepth - 1) % kDepth],
                               sc[(c + kDepth - 1) % kDepth]);
        pool_fold<kChunk>(st, x[c % kDepth], sc[c % kDepth], tab);
    }
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = pool_result(st.l[e], st.acc[e]);
    rope_apply(v, cs, lane);
    if (!valid) return;
    quantize_store_row<L, (kRatio >= 16)>(pool, static_cast<uint32_t>(slot), v, lane);
}

// ------------------------------------------------------------------ long-window compressor
// Ratios 64 and 128: one workgroup of kWaves wavefronts per output row.  The window is
// cut into chunks of kChunk rows dealt round-robin to the wavefronts (wavefront w folds
// chunks w, w + kWaves, ...), so the whole workgroup sweeps its window front to back
// together.  Each wavefront keeps kDepth - 1 chunks in flight while it folds the current
// one into a float64 online softmax state per channel (the online form of the vLLM page's
// section 2; PoolF64, weights from exp_tab).  Every wavefront starts from the same
// reference, the window's first score row, so the partial states normally merge by plain
// addition.  Wavefronts 1.. write their states to LDS and wavefront 0 merges them, rounds,
// rotates, quantises and stores the row.  Measured on MI355X: ratio 128 is fastest with 4
// wavefronts, 1-row chunks and 2 chunks in flight, ratio 64 with 2 wavefronts, 2-row
// chunks and 2 in flight; 8 wavefronts per row run 10-20 % slower with float64 pooling.
// The row is written with non-temporal stores: 2-5 % faster than plain ones at both ratios.
// This lane's 8 channels (two-half mapping) of a channel-indexed row held in LDS.
__device__ __forceinline__ void load_lds_f32x8(const float* row, int lane, float (&v)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float4 a = *reinterpret_cast<const float4*>(row + h * kHalf + 4 * lane);
        v[4 * h] = a.x; v[4 * h + 1] = a.y; v[4 * h + 2] = a.z; v[4 * h + 3] = a.w;
    }
}

__device__ __forceinline__ void load_lds_f64x8(const double* row, int lane, double (&v)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const double2 a = *reinterpret_cast<const double2*>(row + h * kHalf + 4 * lane);
        const double2 b = *reinterpret_cast<const double2*>(row + h * kHalf + 4 * lane + 2);
        v[4 * h] = a.x; v[4 * h + 1] = a.y; v[4 * h + 2] = b.x; v[4 * h + 3] = b.y;
    }
}

// Two wavefronts per SIMD, a 256-register budget (the compiler would otherwise aim for
// more wavefronts and spill the in-flight chunks; three per SIMD measured 1 % slower).
template <Layout L, int kRatio, int kWaves, int kChunk, int kDepth>
__global__ __launch_bounds__(kWave * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void compress_long_kernel(
    uint8_t* __restrict__ pool, int64_t nslots, const float* __restrict__ kv,
    const float* __restrict__ score, int64_t ld, const int32_t* __restrict__ pos,
    const float* __restrict__ cos_sin, int64_t max_pos, const int32_t* __restrict__ slots, const int32_t* __restrict__ table,
    int64_t table_len, int32_t* __restrict__ out, int64_t cap,
    int64_t R) {
    const SlotSrc src{slots, table, table_len, out, R, cap};
    constexpr int kChunks = kRatio / (kWaves * kChunk);   // chunks per wavefront
    static_assert(kRatio % (kWaves * kChunk) == 0 && kChunks >= 1 && kDepth >= 2, "window split");
    // partial states of wavefronts 1..kWaves-1, channel-indexed; the exp table
    __shared__ __attribute__((aligned(16))) double part_l[kWaves - 1][kHeadDim];
    __shared__ __attribute__((aligned(16))) double part_a[kWaves - 1][kHeadDim];
    __shared__ __attribute__((aligned(16))) float part_r[kWaves - 1][kHeadDim];
    __shared__ double tab[256];

    const int64_t i = blockIdx.x;
    clear_tail(src, i * kWaves + wave_id(), static_cast<int64_t>(gridDim.x) * kWaves, threadIdx.x & (kWave - 1));
    const int32_t slot = row_slot(src, i);
    if (threadIdx.x == 0) put_translated(src, i, slot, 0);
    const int32_t p = pos[i];
    if (slot < 0 || slot >= nslots || p < 0 || p >= max_pos) return;  // whole workgroup
    ExpTableCopy<kWave * kWaves> tcopy;
    tcopy.fetch();

    const int lane = threadIdx.x & (kWave - 1);
    const int w = wave_id();
    const int64_t row0 = i * kRatio * ld;
    const int64_t base = row0 + static_cast<int64_t>(w) * kChunk * ld;   // chunk w
    const int64_t step = static_cast<int64_t>(kWaves) * kChunk * ld;     // to chunk w + kWaves

    PoolF64 st;
    {
        float ref[8];
        load_row_f32(score + row0, lane, ref);
        pool_init(st, ref);
    }
    float x[kDepth][kChunk][8], sc[kDepth][kChunk][8];
#pragma unroll
    for (int c = 0; c < kDepth - 1 && c < kChunks; ++c)
        load_chunk<kChunk>(kv, score, base + c * step, ld, lane, x[c], sc[c]);
    tcopy.put(tab);
    __syncthreads();  // the exp table is in LDS
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        if (c + kDepth - 1 < kChunks)
            load_chunk<kChunk>(kv, score, base + (c + kDepth - 1) * step, ld, lane, x[(c + kDepth - 1) % kDepth],
                               sc[(c + kDepth - 1) % kDepth]);
        pool_fold<kChunk>(st, x[c % kDepth], sc[c % kDepth], tab);
    }

    RopeCS cs;
    if (w == 0) rope_load_cs(cos_sin + static_cast<int64_t>(p) * kRopeDim, lane, cs);
    if (w != 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c0 = h * kHalf + 4 * lane;
            double2* dl = reinterpret_cast<double2*>(&part_l[w - 1][c0]);
            double2* da = reinterpret_cast<double2*>(&part_a[w - 1][c0]);
            dl[0] = make_double2(st.l[4 * h], st.l[4 * h + 1]);
            dl[1] = make_double2(st.l[4 * h + 2], st.l[4 * h + 3]);
            da[0] = make_double2(st.acc[4 * h], st.acc[4 * h + 1]);
            da[1] = make_double2(st.acc[4 * h + 2], st.acc[4 * h + 3]);
            *reinterpret_cast<float4*>(&part_r[w - 1][c0]) =
                make_float4(st.ref[4 * h], st.ref[4 * h + 1], st.ref[4 * h + 2], st.ref[4 * h + 3]);
        }
    }
    __syncthreads();
    if (w != 0) return;

    // merge: M = the largest reference per channel; a state on another reference is
    // rescaled to it (rare: only after a score exceeded the first row's by kRefSlack).
    // One partner at a time (no unrolling), so only its state is live in registers.
    double M[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) M[e] = st.ref[e];
#pragma unroll 1
    for (int q = 0; q < kWaves - 1; ++q) {
        float rq[8];
        load_lds_f32x8(&part_r[q][0], lane, rq);
#pragma unroll
        for (int e = 0; e < 8; ++e) M[e] = __builtin_fmax(M[e], static_cast<double>(rq[e]));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) pool_rebase(st.ref[e], M[e], st.l[e], st.acc[e]);
#pragma unroll 1
    for (int q = 0; q < kWaves - 1; ++q) {
        float rq[8];
        double lq[8], aq[8];
        load_lds_f32x8(&part_r[q][0], lane, rq);
        load_lds_f64x8(&part_l[q][0], lane, lq);
        load_lds_f64x8(&part_a[q][0], lane, aq);
        bool moved = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) moved |= static_cast<double>(rq[e]) != M[e];
        if (moved) {
#pragma unroll
            for (int e = 0; e < 8; ++e) pool_rebase(rq[e], M[e], lq[e], aq[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            st.l[e] += lq[e];
            st.acc[e] += aq[e];
        }
    }
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = pool_result(st.l[e], st.acc[e]);
    rope_apply(v, cs, lane);
    quantize_store_row<L, true>(pool, static_cast<uint32_t>(slot), v, lane);
}

// ------------------------------------------------------------------ decode-step compressor state
// One row per state (sequence) per call: fold the row into the state's float64 online
// softmax (reference score, l and acc per channel, as PoolF64), count it, and when the
// window is complete, finalise like the window kernels (acc / l rounded once to bf16, RoPE
// at the completing row's position, quantise, store at its slot) and reset the count.
// State layout, kStateBytes per sequence: ref fp32 [512], l fp64 [512], acc fp64 [512].
// count == 0 means an empty state, so a zeroed buffer is a valid start.
constexpr int64_t kStateBytes = kHeadDim * (4 + 8 + 8);

__device__ __forceinline__ void load_f64x8(const double* __restrict__ row, int lane, double (&v)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const double2 a = *reinterpret_cast<const double2*>(row + h * kHalf + 4 * lane);
        const double2 b = *reinterpret_cast<const double2*>(row + h * kHalf + 4 * lane + 2);
        v[4 * h] = a.x; v[4 * h + 1] = a.y; v[4 * h + 2] = b.x; v[4 * h + 3] = b.y;
    }
}

__device__ __forceinline__ void store_f64x8(double* __restrict__ row, int lane, const double (&v)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        *reinterpret_cast<double2*>(row + h * kHalf + 4 * lane) = make_double2(v[4 * h], v[4 * h + 1]);
        *reinterpret_cast<double2*>(row + h * kHalf + 4 * lane + 2) = make_double2(v[4 * h + 2], v[4 * h + 3]);
    }
}


template <Layout L>
__global__ __launch_bounds__(kWave * kRowsPerBlock) void compress_state_kernel(
    uint8_t* __restrict__ pool, int64_t nslots, uint8_t* __restrict__ state, int32_t* __restrict__ count,
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
    uint8_t* st = state + static_cast<int64_t>(sid) * kStateBytes;
    float* st_ref = reinterpret_cast<float*>(st);
    double* st_l = reinterpret_cast<double*>(st + kHeadDim * 4);
    double* st_a = reinterpret_cast<double*>(st + kHeadDim * 12);
    const int32_t c = count[sid];
    float ref[8];
    double l[8], acc[8];
    if (c == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { ref[e] = s[e]; l[e] = 1.0; acc[e] = x[e]; }
    } else {
        float r0[8];
        *reinterpret_cast<float4*>(&r0[0]) = *reinterpret_cast<const float4*>(st_ref + 4 * lane);
        *reinterpret_cast<float4*>(&r0[4]) = *reinterpret_cast<const float4*>(st_ref + kHalf + 4 * lane);
        load_f64x8(st_l, lane, l);
        load_f64x8(st_a, lane, acc);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ref[e] = r0[e];
            if (s[e] > ref[e] + kRefSlack) {
                const double a = exp_f64(static_cast<double>(ref[e]) - static_cast<double>(s[e]));
                l[e] *= a;
                acc[e] *= a;
                ref[e] = s[e];
            }
            const double w = exp_f64(static_cast<double>(s[e]) - static_cast<double>(ref[e]));
            l[e] += w;
            acc[e] = __builtin_fma(w, static_cast<double>(x[e]), acc[e]);
        }
    }
    if (c + 1 < ratio) {
        // plain stores: the state is read again by the next step's call (non-temporal
        // state stores measured 7 % slower at ratio 4)
        *reinterpret_cast<float4*>(st_ref + 4 * lane) = make_float4(ref[0], ref[1], ref[2], ref[3]);
        *reinterpret_cast<float4*>(st_ref + kHalf + 4 * lane) = make_float4(ref[4], ref[5], ref[6], ref[7]);
        store_f64x8(st_l, lane, l);
        store_f64x8(st_a, lane, acc);
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
    for (int e = 0; e < 8; ++e) v[e] = pool_result(l[e], acc[e]);
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
// Writes the lane's 8 bf16 values (16 bytes) at dst, plain or non-temporal (kNt).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <Layout L, bool kNt = false>
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
    const u32x4 st = {o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16)};
    put<kNt>(reinterpret_cast<u32x4*>(dst + kElemsPerLane * lane), st);
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
// outside the pool are left untouched.  Non-temporal stores (14 % faster than plain ones
// for 16,384 rows; the page kernel above gains nothing from them).
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
    dequant_lane<L, true>(cw, sb, out + g * kHeadDim, lane);
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
