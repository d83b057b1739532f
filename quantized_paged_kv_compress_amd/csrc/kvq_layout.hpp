// kvq_layout.hpp -- compile-time description of the paged KV layouts.
//
// The V41 and V41_FP4 token layouts and the PagedKV page / row / scale-row addressing
// follow "sglang, DeepSeek V4.1 Paged KV Cache: V41 and FP4 formats" (sglang PR #39123
// analysis), section 1: V41 = 512 fp8 e4m3 codes + 16 ue8m0 scales (528 B/token);
// V41_FP4 = 512 e2m1 codes + one e4m3 scale per 32 values, quoted at 288 B/token, the
// difference being padding kept in the scale row.  A page is 64 code rows followed by
// 64 scale rows; every offset below is a compile-time constant.
#pragma once

#include <cstdint>

namespace kvq {

enum class Layout : int32_t { V41 = 1, V41_FP4 = 2 };

constexpr int kHeadDim = 512;  // channels per token row
constexpr int kRopeDim = 64;   // rotated channels, the last 64 of the row
constexpr int kBlock = 32;     // values per scale
constexpr int kBlocks = kHeadDim / kBlock;
constexpr int kPageBits = 6;   // 64 tokens per page
constexpr int kWave = 64;      // gfx950 wavefront
constexpr int kElemsPerLane = kHeadDim / kWave;        // one wavefront per row
constexpr int kLanesPerBlock = kBlock / kElemsPerLane; // lanes sharing one scale

static_assert(kHeadDim == 512, "rows are 512 channels");
static_assert(kRopeDim == 64 && kRopeDim % (2 * kElemsPerLane) == 0, "rope region splits into lane halves");
static_assert(kElemsPerLane == 8, "each lane owns 8 channels (one 16-byte bf16 load)");
static_assert(kLanesPerBlock == 4, "a 32-value block is one DPP quad");
static_assert(kPageBits == 6, "page size is 64 tokens");

template <Layout L> struct LayoutTraits;

template <> struct LayoutTraits<Layout::V41> {
    static constexpr int kCodeRowBytes = kHeadDim;          // one e4m3 byte per channel
    static constexpr int kScaleBytes = kBlocks;             // one ue8m0 byte per block
    static constexpr int kScaleRowBytes = kBlocks;          // no padding
    static constexpr int kCodeBytesPerLane = kElemsPerLane; // 8 bytes
};

template <> struct LayoutTraits<Layout::V41_FP4> {
    static constexpr int kCodeRowBytes = kHeadDim / 2;          // two e2m1 codes per byte
    static constexpr int kScaleBytes = kBlocks;                 // one e4m3 byte per block
    static constexpr int kScaleRowBytes = kBlocks + 16;         // + 16 zero pad bytes
    static constexpr int kCodeBytesPerLane = kElemsPerLane / 2; // 4 bytes
};

template <Layout L> constexpr int kTokenBytes =
    LayoutTraits<L>::kCodeRowBytes + LayoutTraits<L>::kScaleRowBytes;

static_assert(kTokenBytes<Layout::V41> == 528, "V41 is 528 B/token");
static_assert(kTokenBytes<Layout::V41_FP4> == 288, "V41_FP4 is 288 B/token");

// Bytes of one page of 2^page_bits tokens.
template <Layout L> constexpr int64_t kv_page_bytes(int page_rows) {
    return int64_t(page_rows) * kTokenBytes<L>;
}

template <Layout L, int PageBits> struct PagedKV {
    using T = LayoutTraits<L>;
    static constexpr int kRows = 1 << PageBits;
    static constexpr int64_t kPageBytes = kv_page_bytes<L>(kRows);
    static constexpr int64_t kScaleBase = int64_t(kRows) * T::kCodeRowBytes;
    static_assert(kPageBytes % 256 == 0, "pages stay 256-byte aligned");
    static_assert(T::kCodeRowBytes % 16 == 0 && T::kScaleRowBytes % 16 == 0, "rows are 16-byte aligned");

    __host__ __device__ static inline uint8_t* code_row(uint8_t* base, uint32_t slot) {
        return base + int64_t(slot >> PageBits) * kPageBytes
                    + int64_t(slot & (kRows - 1)) * T::kCodeRowBytes;
    }
    __host__ __device__ static inline uint8_t* scale_row(uint8_t* base, uint32_t slot) {
        return base + int64_t(slot >> PageBits) * kPageBytes + kScaleBase
                    + int64_t(slot & (kRows - 1)) * T::kScaleRowBytes;
    }
};

static_assert(PagedKV<Layout::V41, kPageBits>::kPageBytes == 33792, "V41 page");
static_assert(PagedKV<Layout::V41_FP4, kPageBits>::kPageBytes == 18432, "V41_FP4 page");

}  // namespace kvq
