// kvq_capi.hip -- the C ABI of libkvq.so: host-side validation and kernel launches.
//
// Every entry point validates its arguments on the host, then enqueues kernels on the
// caller's stream with hipLaunchKernel (whose return code reports a rejected launch
// without touching the process-wide last-error state).  Nothing allocates, frees or
// synchronises.  Declarations, argument meaning and error behaviour: include/kvq.h.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <tuple>

#include "kvq.h"
#include "kvq_kernels.hpp"
#include "kvq_layout.hpp"

namespace {

using kvq::Layout;

// Largest request of one call: each kernel's grid must stay below 2^32 work-items in x
// (64 per row for the row kernels, up to 512 per output row for the workgroup-per-row
// compressor of ratios 64 and 128, 64 per row of each listed page for the page dequant).
constexpr int64_t kMaxRows = KVQ_MAX_ROWS;
constexpr int64_t kMaxLongRows = KVQ_MAX_LONG_ROWS;
constexpr int64_t kMaxDequantPages = KVQ_MAX_PAGES;
constexpr int64_t kMaxCap = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxPages = int64_t(1) << 32;  // far beyond any pool; keeps num_pages * 64 exact
static_assert(kMaxRows * 64 < (int64_t(1) << 32) && kMaxLongRows * 512 < (int64_t(1) << 32) &&
                  kMaxDequantPages * 64 * 64 < (int64_t(1) << 32),
              "every grid stays below 2^32 work-items");
constexpr int64_t kDequantLongList = 1024;  // pages; from here on 4 rows per wavefront
constexpr int32_t kMaxStateRatio = 1 << 20;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool known_layout(int32_t layout) {
    return layout == KVQ_LAYOUT_V41 || layout == KVQ_LAYOUT_V41_FP4;
}

// Events requested by kvq_profile_next_launch for this thread's next launch.
thread_local hipEvent_t t_start_event = nullptr;
thread_local hipEvent_t t_stop_event = nullptr;

template <typename... KArgs, typename... Args>
int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, void* stream, Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    std::tuple<KArgs...> vals(static_cast<KArgs>(args)...);
    void* ptrs[sizeof...(KArgs)];
    std::apply([&](auto&... a) {
        int j = 0;
        ((ptrs[j++] = const_cast<void*>(static_cast<const void*>(&a))), ...);
    }, vals);
    const hipEvent_t e0 = t_start_event, e1 = t_stop_event;
    t_start_event = t_stop_event = nullptr;
    const hipError_t e =
        (e0 || e1) ? hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0,
                                        static_cast<hipStream_t>(stream), e0, e1, 0)
                   : hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0,
                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : KVQ_ELAUNCH;
}

unsigned blocks_for(int64_t rows, int per_block) {
    return static_cast<unsigned>((rows + per_block - 1) / per_block);
}

template <Layout L>
int store_impl(int mode, void* pool, int64_t num_pages, const uint16_t* k, int64_t ld,
               const uint16_t* weight, float eps, const int32_t* pos, const float* cos_sin,
               int64_t max_pos, const int32_t* slots, int64_t n, void* stream) {
    const dim3 grid(blocks_for(n, kvq::kRowsPerBlock)), block(kvq::kWave * kvq::kRowsPerBlock);
    const int64_t nslots = num_pages << kvq::kPageBits;
    auto* p = static_cast<uint8_t*>(pool);
    if (mode == 2)
        return launch(kvq::store_kernel<L, true, true>, grid, block, stream, p, nslots, k, ld, weight,
                      eps, pos, cos_sin, max_pos, slots, n);
    if (mode == 1)
        return launch(kvq::store_kernel<L, true, false>, grid, block, stream, p, nslots, k, ld, weight,
                      eps, pos, cos_sin, max_pos, slots, n);
    return launch(kvq::store_kernel<L, false, false>, grid, block, stream, p, nslots, k, ld, weight,
                  eps, pos, cos_sin, max_pos, slots, n);
}

template <Layout L>
int compress_c1(void* pool, int64_t num_pages, const float* kv, int64_t ld, const int32_t* pos,
                const float* cos_sin, int64_t max_pos, kvq::SlotSrc slots, int64_t R, void* stream) {
    return launch(kvq::compress_c1_kernel<L>, dim3(blocks_for(R, kvq::kRowsPerBlock)),
                  dim3(kvq::kWave * kvq::kRowsPerBlock), stream, static_cast<uint8_t*>(pool),
                  num_pages << kvq::kPageBits, kv, ld, pos, cos_sin, max_pos, slots.slots, slots.table,
                  slots.table_len, slots.out, slots.cap, R);
}

// Ratios 2 and 4 store their rows with non-temporal stores when the rows written reach
// the size of the 256 MiB last-level cache, plain stores below.  Measured on MI355X on
// cold inputs: plain stores are 4-10 % faster from 256 MiB up to 4 GiB of input (up to
// 138 MB of ratio-4 output, 277 MB at ratio 2 where both are even), non-temporal ones
// 1-3 % faster at 8 GiB (277 MB of ratio-4 output, 553 MB at ratio 2).
constexpr int64_t kShortNtOutputBytes = int64_t(256) << 20;

template <Layout L, int kRatio>
int compress_short(void* pool, int64_t num_pages, const float* kv, const float* score, int64_t ld,
                   const int32_t* pos, const float* cos_sin, int64_t max_pos,
                   kvq::SlotSrc slots, int64_t R, void* stream) {
    if (R * kvq::kTokenBytes<L> >= kShortNtOutputBytes)
        return launch(kvq::compress_short_kernel<L, kRatio, true>, dim3(blocks_for(R, kvq::kRowsPerBlock)),
                      dim3(kvq::kWave * kvq::kRowsPerBlock), stream, static_cast<uint8_t*>(pool),
                      num_pages << kvq::kPageBits, kv, score, ld, pos, cos_sin, max_pos, slots.slots, slots.table,
                      slots.table_len, slots.out, slots.cap, R);
    return launch(kvq::compress_short_kernel<L, kRatio, false>, dim3(blocks_for(R, kvq::kRowsPerBlock)),
                  dim3(kvq::kWave * kvq::kRowsPerBlock), stream, static_cast<uint8_t*>(pool),
                  num_pages << kvq::kPageBits, kv, score, ld, pos, cos_sin, max_pos, slots.slots, slots.table,
                  slots.table_len, slots.out, slots.cap, R);
}

template <Layout L, int kRatio, int kChunk, int kDepth>
int compress_wave(void* pool, int64_t num_pages, const float* kv, const float* score, int64_t ld,
                  const int32_t* pos, const float* cos_sin, int64_t max_pos,
                  kvq::SlotSrc slots, int64_t R, void* stream) {
    return launch(kvq::compress_wave_kernel<L, kRatio, kChunk, kDepth>, dim3(blocks_for(R, kvq::kRowsPerBlock)),
                  dim3(kvq::kWave * kvq::kRowsPerBlock), stream, static_cast<uint8_t*>(pool),
                  num_pages << kvq::kPageBits, kv, score, ld, pos, cos_sin, max_pos, slots.slots, slots.table,
                  slots.table_len, slots.out, slots.cap, R);
}

template <Layout L, int kRatio, int kWaves, int kChunk, int kDepth>
int compress_long(void* pool, int64_t num_pages, const float* kv, const float* score, int64_t ld,
                  const int32_t* pos, const float* cos_sin, int64_t max_pos,
                  kvq::SlotSrc slots, int64_t R, void* stream) {
    return launch(kvq::compress_long_kernel<L, kRatio, kWaves, kChunk, kDepth>, dim3(static_cast<unsigned>(R)),
                  dim3(kvq::kWave * kWaves), stream, static_cast<uint8_t*>(pool),
                  num_pages << kvq::kPageBits, kv, score, ld, pos, cos_sin, max_pos, slots.slots, slots.table,
                  slots.table_len, slots.out, slots.cap, R);
}

template <Layout L>
int compress_dispatch(int32_t ratio, void* pool, int64_t num_pages, const float* kv,
                      const float* score, int64_t ld, const int32_t* pos, const float* cos_sin,
                      int64_t max_pos, kvq::SlotSrc slots, int64_t R, void* stream) {
    // per ratio: wave <rows per chunk, chunks in flight + 1>, long <wavefronts, rows per
    // chunk, chunks in flight + 1>; measured fastest on MI355X
    const auto* sc = score;
    switch (ratio) {
        case 1: return compress_c1<L>(pool, num_pages, kv, ld, pos, cos_sin, max_pos, slots, R, stream);
        case 2: return compress_short<L, 2>(pool, num_pages, kv, sc, ld, pos, cos_sin, max_pos, slots, R, stream);
        case 4: return compress_short<L, 4>(pool, num_pages, kv, sc, ld, pos, cos_sin, max_pos, slots, R, stream);
        case 8: return compress_wave<L, 8, 2, 4>(pool, num_pages, kv, sc, ld, pos, cos_sin, max_pos, slots, R, stream);
        case 16: return compress_wave<L, 16, 2, 4>(pool, num_pages, kv, sc, ld, pos, cos_sin, max_pos, slots, R, stream);
        case 32: return compress_wave<L, 32, 1, 4>(pool, num_pages, kv, sc, ld, pos, cos_sin, max_pos, slots, R, stream);
        case 64: return compress_long<L, 64, 2, 2, 3>(pool, num_pages, kv, sc, ld, pos, cos_sin, max_pos, slots, R, stream);
        case 128: return compress_long<L, 128, 4, 1, 3>(pool, num_pages, kv, sc, ld, pos, cos_sin, max_pos, slots, R, stream);
        default: return KVQ_ERATIO;
    }
}

}  // namespace

extern "C" {

const char* kvq_build_id(void) { return KVQ_BUILD_ID; }

int64_t kvq_compress_state_bytes(void) { return kvq::kStateBytes; }

int kvq_profile_next_launch(void* start_event, void* stop_event) {
    t_start_event = static_cast<hipEvent_t>(start_event);
    t_stop_event = static_cast<hipEvent_t>(stop_event);
    return KVQ_OK;
}

const char* kvq_status_string(int status) {
    switch (status) {
        case KVQ_OK: return "ok";
        case KVQ_EINVAL: return "invalid argument (null pointer, stride, alignment or size)";
        case KVQ_ELAYOUT: return "unknown layout id";
        case KVQ_ERATIO: return "compression ratio not supported (1, 2, 4, 8, 16, 32, 64, 128)";
        case KVQ_ECAPACITY: return "more slots than the translation buffer holds";
        case KVQ_ELAUNCH: return "kernel launch rejected by the HIP runtime";
        default: return "unknown status";
    }
}

int64_t kvq_code_row_bytes(int32_t layout) {
    if (layout == KVQ_LAYOUT_V41) return kvq::LayoutTraits<Layout::V41>::kCodeRowBytes;
    if (layout == KVQ_LAYOUT_V41_FP4) return kvq::LayoutTraits<Layout::V41_FP4>::kCodeRowBytes;
    return KVQ_ELAYOUT;
}

int64_t kvq_scale_row_bytes(int32_t layout) {
    if (layout == KVQ_LAYOUT_V41) return kvq::LayoutTraits<Layout::V41>::kScaleRowBytes;
    if (layout == KVQ_LAYOUT_V41_FP4) return kvq::LayoutTraits<Layout::V41_FP4>::kScaleRowBytes;
    return KVQ_ELAYOUT;
}

int64_t kvq_bytes_per_token(int32_t layout) {
    if (layout == KVQ_LAYOUT_V41) return kvq::kTokenBytes<Layout::V41>;
    if (layout == KVQ_LAYOUT_V41_FP4) return kvq::kTokenBytes<Layout::V41_FP4>;
    return KVQ_ELAYOUT;
}

int64_t kvq_page_bytes(int32_t layout) {
    if (layout == KVQ_LAYOUT_V41) return kvq::PagedKV<Layout::V41, kvq::kPageBits>::kPageBytes;
    if (layout == KVQ_LAYOUT_V41_FP4) return kvq::PagedKV<Layout::V41_FP4, kvq::kPageBits>::kPageBytes;
    return KVQ_ELAYOUT;
}

// mode 0: plain store, 1: RoPE, 2: RMS norm + RoPE
static int store_common(int mode, int32_t layout, void* pool, int64_t num_pages, const uint16_t* k,
                        int64_t ld, const uint16_t* weight, float eps, const int32_t* pos,
                        const float* cos_sin, int64_t max_pos, const int32_t* slots, int64_t n,
                        void* stream) {
    const bool rope = mode >= 1, norm = mode == 2;
    if (!known_layout(layout)) return KVQ_ELAYOUT;
    if (n < 0 || n > kMaxRows || num_pages < 0 || num_pages > kMaxPages) return KVQ_EINVAL;
    if (rope && max_pos <= 0) return KVQ_EINVAL;
    if (norm && !(eps >= 0.0f && eps < __builtin_huge_valf())) return KVQ_EINVAL;
    if (n == 0) return KVQ_OK;
    if (!pool || !k || !slots || (rope && (!pos || !cos_sin)) || (norm && !weight)) return KVQ_EINVAL;
    if (ld < kvq::kHeadDim || ld % 8 != 0) return KVQ_EINVAL;
    if (!aligned16(pool) || !aligned16(k) || (rope && !aligned16(cos_sin)) || (norm && !aligned16(weight)))
        return KVQ_EINVAL;
    if (layout == KVQ_LAYOUT_V41)
        return store_impl<Layout::V41>(mode, pool, num_pages, k, ld, weight, eps, pos, cos_sin, max_pos,
                                       slots, n, stream);
    return store_impl<Layout::V41_FP4>(mode, pool, num_pages, k, ld, weight, eps, pos, cos_sin, max_pos,
                                       slots, n, stream);
}

int kv_store(int32_t layout, void* pool, int64_t num_pages, const uint16_t* k, int64_t ld,
             const int32_t* slots, int64_t n, void* stream) {
    return store_common(0, layout, pool, num_pages, k, ld, nullptr, 0.0f, nullptr, nullptr, 1, slots, n,
                        stream);
}

int kv_store_rope(int32_t layout, void* pool, int64_t num_pages, const uint16_t* k, int64_t ld,
                  const int32_t* pos, const float* cos_sin, int64_t max_pos, const int32_t* slots,
                  int64_t n, void* stream) {
    return store_common(1, layout, pool, num_pages, k, ld, nullptr, 0.0f, pos, cos_sin, max_pos, slots, n,
                        stream);
}

int kv_store_rope_layers(int32_t layout, void* const* pools, int64_t num_pages, const uint16_t* const* k_layers,
                         int64_t ld, int32_t L, const int32_t* pos, const float* cos_sin, int64_t max_pos,
                         const int32_t* slots, int64_t n, void* stream) {
    static_assert(kvq::kMaxLayers == KVQ_MAX_LAYERS, "layer capacity");
    if (!known_layout(layout)) return KVQ_ELAYOUT;
    if (L < 1 || n < 0 || n > kMaxRows / L || num_pages < 0 || num_pages > kMaxPages || max_pos <= 0)
        return KVQ_EINVAL;
    if (n == 0) return KVQ_OK;
    if (!pools || !k_layers || !pos || !cos_sin || !slots || !aligned16(cos_sin)) return KVQ_EINVAL;
    if (ld < kvq::kHeadDim || ld % 8 != 0) return KVQ_EINVAL;
    for (int32_t l = 0; l < L; ++l)
        if (!pools[l] || !k_layers[l] || !aligned16(pools[l]) || !aligned16(k_layers[l])) return KVQ_EINVAL;
    const int64_t nslots = num_pages << kvq::kPageBits;
    for (int32_t l0 = 0; l0 < L; l0 += kvq::kMaxLayers) {
        const int32_t cnt = L - l0 < kvq::kMaxLayers ? L - l0 : kvq::kMaxLayers;
        kvq::LayerPtrs ptrs = {};
        for (int32_t j = 0; j < cnt; ++j) {
            ptrs.pool[j] = static_cast<uint8_t*>(pools[l0 + j]);
            ptrs.k[j] = k_layers[l0 + j];
        }
        const int64_t groups = (cnt + kvq::kLayersPerWave - 1) / kvq::kLayersPerWave;
        const dim3 grid(blocks_for(n * groups, kvq::kRowsPerBlock)), block(kvq::kWave * kvq::kRowsPerBlock);
        const int st = layout == KVQ_LAYOUT_V41
                           ? launch(kvq::store_layers_kernel<Layout::V41>, grid, block, stream, ptrs, cnt, nslots,
                                    ld, pos, cos_sin, max_pos, slots, n)
                           : launch(kvq::store_layers_kernel<Layout::V41_FP4>, grid, block, stream, ptrs, cnt,
                                    nslots, ld, pos, cos_sin, max_pos, slots, n);
        if (st != KVQ_OK) return st;
    }
    return KVQ_OK;
}

int kv_store_norm_rope(int32_t layout, void* pool, int64_t num_pages, const uint16_t* k, int64_t ld,
                       const uint16_t* weight, float eps, const int32_t* pos, const float* cos_sin,
                       int64_t max_pos, const int32_t* slots, int64_t n, void* stream) {
    return store_common(2, layout, pool, num_pages, k, ld, weight, eps, pos, cos_sin, max_pos, slots, n,
                        stream);
}

// Checks of a compressor call apart from its slots (layout, ratio, sizes, the input
// pointers when there is work, strides, alignment).
static int compress_check(int32_t layout, const void* pool, int64_t num_pages, const float* kv,
                          const float* score, int64_t ld, int32_t ratio, const int32_t* pos,
                          const float* cos_sin, int64_t max_pos, int64_t R) {
    if (!known_layout(layout)) return KVQ_ELAYOUT;
    if (ratio != 1 && ratio != 2 && ratio != 4 && ratio != 8 && ratio != 16 && ratio != 32 &&
        ratio != 64 && ratio != 128)
        return KVQ_ERATIO;
    if (R < 0 || R > (ratio >= 64 ? kMaxLongRows : kMaxRows) || num_pages < 0 || num_pages > kMaxPages ||
        max_pos <= 0)
        return KVQ_EINVAL;
    if (R == 0) return KVQ_OK;
    if (!pool || !kv || (ratio > 1 && !score) || !pos || !cos_sin) return KVQ_EINVAL;
    if (ld < kvq::kHeadDim || ld % 4 != 0) return KVQ_EINVAL;
    if (!aligned16(pool) || !aligned16(kv) || (ratio > 1 && !aligned16(score)) || !aligned16(cos_sin))
        return KVQ_EINVAL;
    return KVQ_OK;
}

static int compress_launch(int32_t layout, void* pool, int64_t num_pages, const float* kv, const float* score,
                           int64_t ld, int32_t ratio, const int32_t* pos, const float* cos_sin,
                           int64_t max_pos, kvq::SlotSrc src, int64_t R, void* stream) {
    if (layout == KVQ_LAYOUT_V41)
        return compress_dispatch<Layout::V41>(ratio, pool, num_pages, kv, score, ld, pos, cos_sin, max_pos, src, R, stream);
    return compress_dispatch<Layout::V41_FP4>(ratio, pool, num_pages, kv, score, ld, pos, cos_sin, max_pos, src, R, stream);
}

int kv_compress_store(int32_t layout, void* pool, int64_t num_pages, const float* kv,
                      const float* score, int64_t ld, int32_t ratio, const int32_t* pos,
                      const float* cos_sin, int64_t max_pos, const int32_t* slots, int64_t R,
                      void* stream) {
    const int st = compress_check(layout, pool, num_pages, kv, score, ld, ratio, pos, cos_sin, max_pos, R);
    if (st != KVQ_OK || R == 0) return st;
    if (!slots) return KVQ_EINVAL;
    return compress_launch(layout, pool, num_pages, kv, score, ld, ratio, pos, cos_sin, max_pos,
                           kvq::SlotSrc{slots, nullptr, 0, nullptr, R, R}, R, stream);
}

int kv_compress_store_translate(int32_t layout, void* pool, int64_t num_pages, const float* kv,
                                const float* score, int64_t ld, int32_t ratio, const int32_t* pos,
                                const float* cos_sin, int64_t max_pos, const int32_t* table,
                                int64_t table_len, const int32_t* full_loc, int32_t* out_loc, int64_t cap,
                                int64_t R, void* stream) {
    const int st = compress_check(layout, pool, num_pages, kv, score, ld, ratio, pos, cos_sin, max_pos, R);
    if (st != KVQ_OK) return st;
    if (cap < 0 || cap > kMaxCap || table_len < 0) return KVQ_EINVAL;
    if (R > cap) return KVQ_ECAPACITY;
    if (R == 0) return kv_translate_slots(table, table_len, full_loc, 0, out_loc, cap, stream);
    if (!table || !full_loc || !out_loc) return KVQ_EINVAL;
    // The grid's wavefronts zero out[R:cap] between them; a tail longer than
    // kMaxTailChunks chunks of 64 per wavefront is left to the translation kernel instead.
    const int64_t waves = ratio == 128 ? R * 4 : ratio == 64 ? R * 2
                                                             : int64_t(blocks_for(R, kvq::kRowsPerBlock)) * kvq::kRowsPerBlock;
    if ((cap - R + 63) / 64 > kvq::kMaxTailChunks * waves) {
        const int t = kv_translate_slots(table, table_len, full_loc, R, out_loc, cap, stream);
        if (t != KVQ_OK) return t;
        return compress_launch(layout, pool, num_pages, kv, score, ld, ratio, pos, cos_sin, max_pos,
                               kvq::SlotSrc{out_loc, nullptr, 0, nullptr, R, R}, R, stream);
    }
    return compress_launch(layout, pool, num_pages, kv, score, ld, ratio, pos, cos_sin, max_pos,
                           kvq::SlotSrc{full_loc, table, table_len, out_loc, R, cap}, R, stream);
}

int kv_compress_state_update(int32_t layout, void* pool, int64_t num_pages, void* state, int32_t* count,
                             int64_t num_states, int32_t ratio, const int32_t* state_ids, const float* kv,
                             const float* score, int64_t ld, const int32_t* pos, const float* cos_sin,
                             int64_t max_pos, const int32_t* slots, int64_t n, void* stream) {
    if (!known_layout(layout)) return KVQ_ELAYOUT;
    if (ratio < 1 || ratio > kMaxStateRatio) return KVQ_ERATIO;
    if (n < 0 || n > kMaxRows || num_pages < 0 || num_pages > kMaxPages || num_states < 0 || max_pos <= 0) return KVQ_EINVAL;
    if (n == 0) return KVQ_OK;
    if (!pool || !state || !count || !state_ids || !kv || !score || !pos || !cos_sin || !slots)
        return KVQ_EINVAL;
    if (ld < kvq::kHeadDim || ld % 4 != 0) return KVQ_EINVAL;
    if (!aligned16(pool) || !aligned16(state) || !aligned16(kv) || !aligned16(score) || !aligned16(cos_sin))
        return KVQ_EINVAL;
    const dim3 grid(blocks_for(n, kvq::kRowsPerBlock)), block(kvq::kWave * kvq::kRowsPerBlock);
    auto* p = static_cast<uint8_t*>(pool);
    auto* st = static_cast<uint8_t*>(state);
    const int64_t nslots = num_pages << kvq::kPageBits;
    if (layout == KVQ_LAYOUT_V41)
        return launch(kvq::compress_state_kernel<Layout::V41>, grid, block, stream, p, nslots, st, count,
                      num_states, ratio, state_ids, kv, score, ld, pos, cos_sin, max_pos, slots, n);
    return launch(kvq::compress_state_kernel<Layout::V41_FP4>, grid, block, stream, p, nslots, st, count,
                  num_states, ratio, state_ids, kv, score, ld, pos, cos_sin, max_pos, slots, n);
}

int kv_dequant(int32_t layout, const void* pool, int64_t num_pages, const int32_t* page_ids,
               int64_t P, uint16_t* out, void* stream) {
    if (!known_layout(layout)) return KVQ_ELAYOUT;
    if (P < 0 || P > kMaxDequantPages || num_pages < 0 || num_pages > kMaxPages) return KVQ_EINVAL;
    if (P == 0) return KVQ_OK;
    if (!pool || !page_ids || !out) return KVQ_EINVAL;
    if (!aligned16(pool) || !aligned16(out)) return KVQ_EINVAL;
    const auto* p = static_cast<const uint8_t*>(pool);
    const dim3 block(kvq::kWave * kvq::kRowsPerBlock);
    const int64_t rows = P << kvq::kPageBits;
    if (P >= kDequantLongList) {  // 4 rows per wavefront
        const dim3 grid(blocks_for(rows, 4 * kvq::kRowsPerBlock));
        if (layout == KVQ_LAYOUT_V41)
            return launch(kvq::dequant_kernel<Layout::V41, 4>, grid, block, stream, p, num_pages, page_ids, P, out);
        return launch(kvq::dequant_kernel<Layout::V41_FP4, 4>, grid, block, stream, p, num_pages, page_ids, P, out);
    }
    const dim3 grid(blocks_for(rows, kvq::kRowsPerBlock));
    if (layout == KVQ_LAYOUT_V41)
        return launch(kvq::dequant_kernel<Layout::V41, 1>, grid, block, stream, p, num_pages, page_ids, P, out);
    return launch(kvq::dequant_kernel<Layout::V41_FP4, 1>, grid, block, stream, p, num_pages, page_ids, P, out);
}

int kv_dequant_slots(int32_t layout, const void* pool, int64_t num_pages, const int32_t* slots, int64_t n,
                     uint16_t* out, void* stream) {
    if (!known_layout(layout)) return KVQ_ELAYOUT;
    if (n < 0 || n > kMaxRows || num_pages < 0 || num_pages > kMaxPages) return KVQ_EINVAL;
    if (n == 0) return KVQ_OK;
    if (!pool || !slots || !out) return KVQ_EINVAL;
    if (!aligned16(pool) || !aligned16(out)) return KVQ_EINVAL;
    const dim3 grid(blocks_for(n, kvq::kRowsPerBlock)), block(kvq::kWave * kvq::kRowsPerBlock);
    const auto* p = static_cast<const uint8_t*>(pool);
    const int64_t nslots = num_pages << kvq::kPageBits;
    if (layout == KVQ_LAYOUT_V41)
        return launch(kvq::dequant_slots_kernel<Layout::V41>, grid, block, stream, p, nslots, slots, n, out);
    return launch(kvq::dequant_slots_kernel<Layout::V41_FP4>, grid, block, stream, p, nslots, slots, n, out);
}

int kv_translate_slots(const int32_t* table, int64_t table_len, const int32_t* full_loc, int64_t n,
                       int32_t* out, int64_t cap, void* stream) {
    if (n < 0 || cap < 0 || table_len < 0 || cap > kMaxCap) return KVQ_EINVAL;
    if (n > cap) return KVQ_ECAPACITY;
    if (cap == 0) return KVQ_OK;
    if (!out || (n > 0 && (!table || !full_loc))) return KVQ_EINVAL;
    return launch(kvq::translate_kernel, dim3(blocks_for(cap, 256)), dim3(256), stream, table, table_len,
                  full_loc, n, out, cap);
}

}  // extern "C"
