// kvq_device.hpp -- per-lane building blocks shared by the gfx950 kernels.
//
// Work mapping ("two-half" mapping): one 64-lane wavefront owns one 512-channel row and
// lane l owns channels 4l..4l+3 (v[0..3]) and 256+4l..256+4l+3 (v[4..7]).  Every load
// instruction of a row then covers one contiguous run (1 KiB of fp32 or 512 B of bf16)
// -- measured on MI355X, fully contiguous 16-byte-per-lane streams reach ~7.0 TB/s where
// a lane reading 32 contiguous bytes as two 16-byte halves tops out near 6.4 TB/s.
// Eight values per lane and 128-bit loads follow the compressor kernel of "DeepSeek V4
// Sparse FP8 Compressor kernel optimisation with CuteDSL" (vLLM PR #44161 analysis),
// section 1.  A 32-value scale block is then 8 adjacent lanes (block l/8 in the first
// half, 8 + l/8 in the second), so the block absmax is three DPP max steps with no LDS,
// the wave64 counterpart of that page's section-3 group butterfly.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvq_layout.hpp"

namespace kvq {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kHalf = kHeadDim / 2;                        // 256 channels per half
constexpr int kRopeLane0 = (kHeadDim - kRopeDim - kHalf) / 4;  // 48: first lane of the rope region
static_assert(kRopeLane0 == 48 && kRopeDim / 2 / 4 == 8, "rope pairs are lanes l and l+8 of DPP row 3");

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> nearest bfloat16 (ties to even): the 16-bit pattern, and the value.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float round_bf16(float f) {
    return __uint_as_float(bf16_rne_bits(f) << 16);
}

// float64 -> nearest bfloat16 bit pattern (ties to even), rounded once from the float64
// value: going through float32 first could land exactly on a bf16 midpoint and round
// twice.  At or above 2^-126 the 45 low mantissa bits are rounded away in the integer
// domain (a carry moves into the exponent, and past the bf16 range the float32
// conversion gives infinity); below it the bf16 spacing is the fixed 2^-133.
__device__ __forceinline__ uint32_t bf16_rne_bits_f64(double p) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(p));
    if ((u & 0x7FFFFFFFFFFFFFFFull) < 0x3810000000000000ull) {
        const double q = __builtin_rint(p * 0x1p133) * 0x1p-133;
        return __float_as_uint(static_cast<float>(q)) >> 16;
    }
    const uint64_t r = (u + 0x00000FFFFFFFFFFFull + ((u >> 45) & 1u)) & ~0x00001FFFFFFFFFFFull;
    return __float_as_uint(static_cast<float>(__longlong_as_double(static_cast<long long>(r)))) >> 16;
}

// ---------------------------------------------------------------- float64 exponential
// exp(d) for float64 d up to 700, written out for the softmax weights.  k = rint(d / ln 2)
// comes from the low bits of d / ln 2 + 1.5 * 2^52 (one fma, ties to even); r = d - k ln 2
// is reduced in two steps with ln 2 split so that k * kLn2Hi is exact (Cody and Waite), and
// exp(r) on |r| <= 0.35 is a degree-11 polynomial (the Chebyshev interpolant of exp on
// [-0.35, 0.35], relative error 7e-18 before rounding; constants from gen_exp_poly.py).
// d is held at -1000 first: exp(-1000) is already 0 in float64 and k stays small.
// The constants sit in constant memory so that they are loaded once into scalar registers
// and feed v_fma_f64 directly (as literals each would cost two moves per use).
__constant__ double kExpConst[16] = {
    0x1.af682e715258ap-26, 0x1.28b82404fa64fp-22, 0x1.71ddf2b060bb0p-19, 0x1.a0198d2d43afbp-16,
    0x1.a01a01b24ec34p-13, 0x1.6c16c189ae5d5p-10, 0x1.111111110ef9cp-7,  0x1.555555554e892p-5,
    0x1.555555555555bp-3,  0x1.0000000000012p-1,  1.0,                   1.0,
    1.4426950408889634,    0x1.62e42fee00000p-1,  0x1.a39ef35793c76p-33, 0x1.8p52};

__device__ __forceinline__ double exp_f64(double d) {
    const double kInvLn2 = kExpConst[12], kLn2Hi = kExpConst[13], kLn2Lo = kExpConst[14];
    const double kShift = kExpConst[15];
    d = __builtin_fmax(d, -1000.0);
    const double kd = __builtin_fma(d, kInvLn2, kShift);
    const double k = kd - kShift;
    double r = __builtin_fma(-k, kLn2Hi, d);
    r = __builtin_fma(-k, kLn2Lo, r);
    double p = kExpConst[0];
#pragma unroll
    for (int j = 1; j < 12; ++j) p = __builtin_fma(p, r, kExpConst[j]);
    return __builtin_ldexp(p, static_cast<int>(__double_as_longlong(kd)));  // low word of kd = k
}

// Table-driven exp(d) for the softmax weights, -512 <= d <= 65 (callers guarantee it):
// k = rint(256 d / ln 2) from the low bits of 256 d / ln 2 + 1.5 * 2^52, r = d - k ln(2)/256
// (Cody and Waite, ln(2)/256 split with 33 significant bits in the high part, so k * hi is
// exact), |r| <= ln(2)/512, and exp(d) = 2^(k >> 8) * 2^((k & 255)/256) * exp(r).  The
// 256 values 2^(j/256) are correctly rounded float64 constants (kExpTab, copied to LDS by
// ExpTableCopy), exp(r) - 1 is its Taylor polynomial to r^4 (the first dropped term is
// below 4e-17 relative), and 2^(k >> 8) is added to the exponent field in the integer
// domain (the result stays a normal number for d >= -512).  About 14 float64 operations
// per weight against 22 for exp_f64: fewer float64 operations per byte keep the clocks up.
__constant__ double kExpTab[256] = {
    0x1.0000000000000p+0, 0x1.00b1afa5abcbfp+0, 0x1.0163da9fb3335p+0, 0x1.02168143b0281p+0,
    0x1.02c9a3e778061p+0, 0x1.037d42e11bbccp+0, 0x1.04315e86e7f85p+0, 0x1.04e5f72f654b1p+0,
    0x1.059b0d3158574p+0, 0x1.0650a0e3c1f89p+0, 0x1.0706b29ddf6dep+0, 0x1.07bd42b72a836p+0,
    0x1.0874518759bc8p+0, 0x1.092bdf66607e0p+0, 0x1.09e3ecac6f383p+0, 0x1.0a9c79b1f3919p+0,
    0x1.0b5586cf9890fp+0, 0x1.0c0f145e46c85p+0, 0x1.0cc922b7247f7p+0, 0x1.0d83b23395decp+0,
    0x1.0e3ec32d3d1a2p+0, 0x1.0efa55fdfa9c5p+0, 0x1.0fb66affed31bp+0, 0x1.1073028d7233ep+0,
    0x1.11301d0125b51p+0, 0x1.11edbab5e2ab6p+0, 0x1.12abdc06c31ccp+0, 0x1.136a814f204abp+0,
    0x1.1429aaea92de0p+0, 0x1.14e95934f312ep+0, 0x1.15a98c8a58e51p+0, 0x1.166a45471c3c2p+0,
    0x1.172b83c7d517bp+0, 0x1.17ed48695bbc0p+0, 0x1.18af9388c8deap+0, 0x1.1972658375d2fp+0,
    0x1.1a35beb6fcb75p+0, 0x1.1af99f8138a1cp+0, 0x1.1bbe084045cd4p+0, 0x1.1c82f95281c6bp+0,
    0x1.1d4873168b9aap+0, 0x1.1e0e75eb44027p+0, 0x1.1ed5022fcd91dp+0, 0x1.1f9c18438ce4dp+0,
    0x1.2063b88628cd6p+0, 0x1.212be3578a819p+0, 0x1.21f49917ddc96p+0, 0x1.22bdda27912d1p+0,
    0x1.2387a6e756238p+0, 0x1.2451ffb82140ap+0, 0x1.251ce4fb2a63fp+0, 0x1.25e85711ece75p+0,
    0x1.26b4565e27cddp+0, 0x1.2780e341ddf29p+0, 0x1.284dfe1f56381p+0, 0x1.291ba7591bb70p+0,
    0x1.29e9df51fdee1p+0, 0x1.2ab8a66d10f13p+0, 0x1.2b87fd0dad990p+0, 0x1.2c57e39771b2fp+0,
    0x1.2d285a6e4030bp+0, 0x1.2df961f641589p+0, 0x1.2ecafa93e2f56p+0, 0x1.2f9d24abd886bp+0,
    0x1.306fe0a31b715p+0, 0x1.31432edeeb2fdp+0, 0x1.32170fc4cd831p+0, 0x1.32eb83ba8ea32p+0,
    0x1.33c08b26416ffp+0, 0x1.3496266e3fa2dp+0, 0x1.356c55f929ff1p+0, 0x1.36431a2de883bp+0,
    0x1.371a7373aa9cbp+0, 0x1.37f26231e754ap+0, 0x1.38cae6d05d866p+0, 0x1.39a401b7140efp+0,
    0x1.3a7db34e59ff7p+0, 0x1.3b57fbfec6cf4p+0, 0x1.3c32dc313a8e5p+0, 0x1.3d0e544ede173p+0,
    0x1.3dea64c123422p+0, 0x1.3ec70df1c5175p+0, 0x1.3fa4504ac801cp+0, 0x1.40822c367a024p+0,
    0x1.4160a21f72e2ap+0, 0x1.423fb2709468ap+0, 0x1.431f5d950a897p+0, 0x1.43ffa3f84b9d4p+0,
    0x1.44e086061892dp+0, 0x1.45c2042a7d232p+0, 0x1.46a41ed1d0057p+0, 0x1.4786d668b3237p+0,
    0x1.486a2b5c13cd0p+0, 0x1.494e1e192aed2p+0, 0x1.4a32af0d7d3dep+0, 0x1.4b17dea6db7d7p+0,
    0x1.4bfdad5362a27p+0, 0x1.4ce41b817c114p+0, 0x1.4dcb299fddd0dp+0, 0x1.4eb2d81d8abffp+0,
    0x1.4f9b2769d2ca7p+0, 0x1.508417f4531eep+0, 0x1.516daa2cf6642p+0, 0x1.5257de83f4eefp+0,
    0x1.5342b569d4f82p+0, 0x1.542e2f4f6ad27p+0, 0x1.551a4ca5d920fp+0, 0x1.56070dde910d2p+0,
    0x1.56f4736b527dap+0, 0x1.57e27dbe2c4cfp+0, 0x1.58d12d497c7fdp+0, 0x1.59c0827ff07ccp+0,
    0x1.5ab07dd485429p+0, 0x1.5ba11fba87a03p+0, 0x1.5c9268a5946b7p+0, 0x1.5d84590998b93p+0,
    0x1.5e76f15ad2148p+0, 0x1.5f6a320dceb71p+0, 0x1.605e1b976dc09p+0, 0x1.6152ae6cdf6f4p+0,
    0x1.6247eb03a5585p+0, 0x1.633dd1d1929fdp+0, 0x1.6434634ccc320p+0, 0x1.652b9febc8fb7p+0,
    0x1.6623882552225p+0, 0x1.671c1c70833f6p+0, 0x1.68155d44ca973p+0, 0x1.690f4b19e9538p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6b052fa75173ep+0, 0x1.6c012750bdabfp+0, 0x1.6cfdcddd47645p+0,
    0x1.6dfb23c651a2fp+0, 0x1.6ef9298593ae5p+0, 0x1.6ff7df9519484p+0, 0x1.70f7466f42e87p+0,
    0x1.71f75e8ec5f74p+0, 0x1.72f8286ead08ap+0, 0x1.73f9a48a58174p+0, 0x1.74fbd35d7cbfdp+0,
    0x1.75feb564267c9p+0, 0x1.77024b1ab6e09p+0, 0x1.780694fde5d3fp+0, 0x1.790b938ac1cf6p+0,
    0x1.7a11473eb0187p+0, 0x1.7b17b0976cfdbp+0, 0x1.7c1ed0130c132p+0, 0x1.7d26a62ff86f0p+0,
    0x1.7e2f336cf4e62p+0, 0x1.7f3878491c491p+0, 0x1.80427543e1a12p+0, 0x1.814d2add106d9p+0,
    0x1.82589994cce13p+0, 0x1.8364c1eb941f7p+0, 0x1.8471a4623c7adp+0, 0x1.857f4179f5b21p+0,
    0x1.868d99b4492edp+0, 0x1.879cad931a436p+0, 0x1.88ac7d98a6699p+0, 0x1.89bd0a478580fp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8be05bad61778p+0, 0x1.8cf3216b5448cp+0, 0x1.8e06a5e0866d9p+0,
    0x1.8f1ae99157736p+0, 0x1.902fed0282c8ap+0, 0x1.9145b0b91ffc6p+0, 0x1.925c353aa2fe2p+0,
    0x1.93737b0cdc5e5p+0, 0x1.948b82b5f98e5p+0, 0x1.95a44cbc8520fp+0, 0x1.96bdd9a7670b3p+0,
    0x1.97d829fde4e50p+0, 0x1.98f33e47a22a2p+0, 0x1.9a0f170ca07bap+0, 0x1.9b2bb4d53fe0dp+0,
    0x1.9c49182a3f090p+0, 0x1.9d674194bb8d5p+0, 0x1.9e86319e32323p+0, 0x1.9fa5e8d07f29ep+0,
    0x1.a0c667b5de565p+0, 0x1.a1e7aed8eb8bbp+0, 0x1.a309bec4a2d33p+0, 0x1.a42c980460ad8p+0,
    0x1.a5503b23e255dp+0, 0x1.a674a8af46052p+0, 0x1.a799e1330b358p+0, 0x1.a8bfe53c12e59p+0,
    0x1.a9e6b5579fdbfp+0, 0x1.ab0e521356ebap+0, 0x1.ac36bbfd3f37ap+0, 0x1.ad5ff3a3c2774p+0,
    0x1.ae89f995ad3adp+0, 0x1.afb4ce622f2ffp+0, 0x1.b0e07298db666p+0, 0x1.b20ce6c9a8952p+0,
    0x1.b33a2b84f15fbp+0, 0x1.b468415b749b1p+0, 0x1.b59728de5593ap+0, 0x1.b6c6e29f1c52ap+0,
    0x1.b7f76f2fb5e47p+0, 0x1.b928cf22749e4p+0, 0x1.ba5b030a1064ap+0, 0x1.bb8e0b79a6f1fp+0,
    0x1.bcc1e904bc1d2p+0, 0x1.bdf69c3f3a207p+0, 0x1.bf2c25bd71e09p+0, 0x1.c06286141b33dp+0,
    0x1.c199bdd85529cp+0, 0x1.c2d1cd9fa652cp+0, 0x1.c40ab5fffd07ap+0, 0x1.c544778fafb22p+0,
    0x1.c67f12e57d14bp+0, 0x1.c7ba88988c933p+0, 0x1.c8f6d9406e7b5p+0, 0x1.ca3405751c4dbp+0,
    0x1.cb720dcef9069p+0, 0x1.ccb0f2e6d1675p+0, 0x1.cdf0b555dc3fap+0, 0x1.cf3155b5bab74p+0,
    0x1.d072d4a07897cp+0, 0x1.d1b532b08c968p+0, 0x1.d2f87080d89f2p+0, 0x1.d43c8eacaa1d6p+0,
    0x1.d5818dcfba487p+0, 0x1.d6c76e862e6d3p+0, 0x1.d80e316c98398p+0, 0x1.d955d71ff6075p+0,
    0x1.da9e603db3285p+0, 0x1.dbe7cd63a8315p+0, 0x1.dd321f301b460p+0, 0x1.de7d5641c0658p+0,
    0x1.dfc97337b9b5fp+0, 0x1.e11676b197d17p+0, 0x1.e264614f5a129p+0, 0x1.e3b333b16ee12p+0,
    0x1.e502ee78b3ff6p+0, 0x1.e653924676d76p+0, 0x1.e7a51fbc74c83p+0, 0x1.e8f7977cdb740p+0,
    0x1.ea4afa2a490dap+0, 0x1.eb9f4867cca6ep+0, 0x1.ecf482d8e67f1p+0, 0x1.ee4aaa2188510p+0,
    0x1.efa1bee615a27p+0, 0x1.f0f9c1cb6412ap+0, 0x1.f252b376bba97p+0, 0x1.f3ac948dd7274p+0,
    0x1.f50765b6e4540p+0, 0x1.f6632798844f8p+0, 0x1.f7bfdad9cbe14p+0, 0x1.f91d802243c89p+0,
    0x1.fa7c1819e90d8p+0, 0x1.fbdba3692d514p+0, 0x1.fd3c22b8f71f1p+0, 0x1.fe9d96b2a23d9p+0,
};
__constant__ double kExpTabConst[6] = {0x1.71547652b82fep+8,   // 256 / ln 2
                                       0x1.8p52,               // rounding shift
                                       0x1.62e42fef00000p-9,   // ln(2)/256, high part
                                       0x1.473de6af278edp-42,  // ln(2)/256, low part
                                       1.0 / 24.0, 1.0 / 6.0};

// Copying the table into LDS is split in two so that the window's loads can be issued in
// between: fetch (this thread's entries into registers, issued before the window loads, so
// that waiting for them does not wait for the window), then put (after them), then a
// barrier.  kThreads is the block size; with 256 or more threads, threads 0..255 take one
// entry each.
template <int kThreads>
struct ExpTableCopy {
    static constexpr int kPer = kThreads >= 256 ? 1 : 256 / kThreads;
    double v[kPer];
    __device__ __forceinline__ void fetch() {
        const int t = static_cast<int>(threadIdx.x);
#pragma unroll
        for (int m = 0; m < kPer; ++m) v[m] = (t < 256) ? kExpTab[(t + m * kThreads) & 255] : 0.0;
    }
    __device__ __forceinline__ void put(double* tab) const {
        const int t = static_cast<int>(threadIdx.x);
        __builtin_amdgcn_sched_barrier(0);  // keep the window loads ahead of this wait
#pragma unroll
        for (int m = 0; m < kPer; ++m)
            if (t < 256) tab[t + m * kThreads] = v[m];
    }
};

__device__ __forceinline__ double exp_tab(double d, const double* tab) {
    const double kd = __builtin_fma(d, kExpTabConst[0], kExpTabConst[1]);
    const double k = kd - kExpTabConst[1];
    double r = __builtin_fma(-k, kExpTabConst[2], d);
    r = __builtin_fma(-k, kExpTabConst[3], r);
    const int ki = static_cast<int>(__double_as_longlong(kd));  // low word of kd = k
    const double t = tab[ki & 255];
    double q = __builtin_fma(r, kExpTabConst[4], kExpTabConst[5]);
    q = __builtin_fma(q, r, 0.5);
    q = __builtin_fma(q, r, 1.0);
    q = q * r;                                                   // exp(r) - 1
    const double w = __builtin_fma(t, q, t);
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(w)) +
                       (static_cast<uint64_t>(static_cast<int64_t>(ki >> 8)) << 52);
    return __longlong_as_double(static_cast<long long>(b));
}

// ---------------------------------------------------------------- cross-lane
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float dppf_row_ror8(float v) {
    return __uint_as_float(dpp<0x128>(__float_as_uint(v)));
}
// swap lane groups of 16 inside each 32 (ds_swizzle bit mode, xor mask 0x10)
__device__ __forceinline__ uint32_t swizzle_xor16(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), 0x401F));
}

// Max over each group of 8 lanes, for non-negative float bit patterns (unsigned order
// equals float order for them): quad_perm [1,0,3,2], quad_perm [2,3,0,1], then
// row_half_mirror, which maps each quad onto the other quad of its 8-lane half-row.
__device__ __forceinline__ uint32_t oct_max_u32(uint32_t v) {
    v = max(v, dpp<0xB1>(v));
    v = max(v, dpp<0x4E>(v));
    v = max(v, dpp<0x141>(v));
    return v;
}

// Lane l contributes the byte of block l/8 of one half; returns on lanes 0 and 32 the
// dword of blocks 0..3 and 4..7 of that half (block 4r+j in byte j).
__device__ __forceinline__ uint32_t gather_block_bytes(uint32_t byte, int lane) {
    uint32_t w = byte << (8 * ((lane >> 3) & 3));
    w |= dpp<0x128>(w);      // row_ror:8 joins lanes l and l^8 (blocks b, b^1)
    w |= swizzle_xor16(w);   // joins the two DPP rows of each 32 lanes (blocks b^2)
    return w;
}

// ---------------------------------------------------------------- loads
typedef float f32x4 __attribute__((ext_vector_type(4)));

// This lane's 8 channels of a bf16 row (two 8-byte loads; each instruction reads 512
// contiguous bytes across the wavefront).
__device__ __forceinline__ void load_row_bf16(const uint16_t* __restrict__ row, int lane, float (&v)[8]) {
    const uint2 a = *reinterpret_cast<const uint2*>(row + 4 * lane);
    const uint2 b = *reinterpret_cast<const uint2*>(row + kHalf + 4 * lane);
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(b.x); v[5] = bf16_hi(b.x); v[6] = bf16_lo(b.y); v[7] = bf16_hi(b.y);
}

// This lane's 8 channels of an fp32 row: two non-temporal 16-byte loads (each
// instruction reads 1 KiB contiguous); streaming inputs are read exactly once.
__device__ __forceinline__ void load_row_f32(const float* __restrict__ row, int lane, float (&v)[8]) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + 4 * lane));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + kHalf + 4 * lane));
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
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
// NeoX half rotation of channels 448..511: channel 448+i is the second-half value
// v[4 + i%4] of lane 48 + i/4 and its partner 480+i sits in lane 56 + i/4, i.e. lanes
// l and l+8 of DPP row 3, exchanged with one row_ror:8 per value.  The cosines and sines
// of a lane's four angles (i = 4*(l%8) .. +3) are loaded ahead by rope_load_cs.
struct RopeCS {
    float c[4], s[4];
};

__device__ __forceinline__ void rope_load_cs(const float* __restrict__ cos_sin_row, int lane, RopeCS& cs) {
    if (lane >= kRopeLane0) {
        const int i0 = 4 * (lane & 7);
        const float4 c = *reinterpret_cast<const float4*>(cos_sin_row + i0);
        const float4 s = *reinterpret_cast<const float4*>(cos_sin_row + kRopeDim / 2 + i0);
        cs.c[0] = c.x; cs.c[1] = c.y; cs.c[2] = c.z; cs.c[3] = c.w;
        cs.s[0] = s.x; cs.s[1] = s.y; cs.s[2] = s.z; cs.s[3] = s.w;
    }
}

// Products and sums are rounded one at a time (the file is compiled without
// contraction) and the results rounded to bf16.  Every lane must call this.
__device__ __forceinline__ void rope_apply(float (&v)[8], const RopeCS& cs, int lane) {
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = dppf_row_ror8(v[4 + e]);
    if (lane >= kRopeLane0) {
        const bool first = lane < kRopeLane0 + 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = v[4 + e] * cs.c[e];
            const float b = p[e] * cs.s[e];
            v[4 + e] = round_bf16(first ? a - b : a + b);
        }
    }
}

// ---------------------------------------------------------------- float64 softmax pooling
// Online per-channel softmax pooling of a lane's 8 channels, in float64 so that the pooled
// value rounds to the same bf16 as the exact one (an error near 1e-16 relative can only
// change the rounding of a value that far from a bf16 midpoint).  The weights are taken
// relative to a reference score `ref` that is a score of the window (so the largest weight
// is at least 1): l = sum of exp(s - ref), acc = sum of exp(s - ref) * x.  The reference
// moves, and the sums are rescaled, only when a score exceeds it by more than kRefSlack,
// so states that start from the same reference (the window's first row) usually still
// share it at the end and merge by plain addition.  Weights stay below e^kRefSlack, and
// s - ref is held at -512 (exp_tab's range): a weight below e^-512 times any finite kv
// cannot reach the smallest bf16, so holding it there changes no result.
constexpr float kRefSlack = 64.0f;

struct PoolF64 {
    double ref[8];
    float ref_hi[8];  // ref + kRefSlack
    double l[8], acc[8];
};

__device__ __forceinline__ void pool_init(PoolF64& st, const float (&ref)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        st.ref[e] = ref[e];
        st.ref_hi[e] = ref[e] + kRefSlack;
        st.l[e] = 0.0;
        st.acc[e] = 0.0;
    }
}

// Fold kRows window rows (this lane's 8 kv and score values of each) into the state;
// tab is the LDS copy of kExpTab.
template <int kRows>
__device__ __forceinline__ void pool_fold(PoolF64& st, const float (&x)[kRows][8], const float (&s)[kRows][8],
                                          const double* tab) {
    float cm[8];
    bool move = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        cm[e] = s[0][e];
#pragma unroll
        for (int j = 1; j < kRows; ++j) cm[e] = fmaxf(cm[e], s[j][e]);
        move |= cm[e] > st.ref_hi[e];
    }
    if (move) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (cm[e] > st.ref_hi[e]) {
                const double a = exp_f64(st.ref[e] - static_cast<double>(cm[e]));
                st.l[e] *= a;
                st.acc[e] *= a;
                st.ref[e] = cm[e];
                st.ref_hi[e] = cm[e] + kRefSlack;
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
            const double d = __builtin_fmax(static_cast<double>(s[j][e]) - st.ref[e], -512.0);
            const double w = exp_tab(d, tab);
            st.l[e] += w;
            st.acc[e] = __builtin_fma(w, static_cast<double>(x[j][e]), st.acc[e]);
        }
    }
}

// Bring a partial state (ref, l, acc of one channel) to the reference M >= ref.
__device__ __forceinline__ void pool_rebase(double ref, double M, double& l, double& acc) {
    if (ref != M) {
        const double a = exp_f64(ref - M);
        l *= a;
        acc *= a;
    }
}

// The pooled value acc / l (IEEE float64 division) as a bf16-valued float.
__device__ __forceinline__ float pool_result(double l, double acc) {
    return __uint_as_float(bf16_rne_bits_f64(acc / l) << 16);
}

// ---------------------------------------------------------------- K norm (RMS)
// One float64 DPP step of a wave reduction (the two 32-bit halves move separately).
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint64_t lo = dpp<kCtrl>(static_cast<uint32_t>(b));
    const uint64_t hi = dpp<kCtrl>(static_cast<uint32_t>(b >> 32));
    return __longlong_as_double(static_cast<long long>((hi << 32) | lo));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b), lane));
    const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane));
    return __longlong_as_double(static_cast<long long>((hi << 32) | lo));
}

// Sum of a float64 over the whole wavefront in a fixed order: quad, pairs of quads and the
// 16-lane DPP row by DPP adds, then the four rows through readlane.  Every lane gets the
// same value.
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x124>(v);   // row_ror:4
    v += dpp_f64<0x128>(v);   // row_ror:8
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// RMS normalisation of a row with a per-channel bf16 weight (the "fused K norm + RoPE"
// store of the sglang V41 page's latency table, read as y = x * w / sqrt(mean(x^2) + eps)),
// in float64: the squares and the products x * w are exact, the sum of squares is a
// wave-wide float64 sum, 1 / sqrt(...) is IEEE float64, and each y is rounded once to
// bf16.  Every lane must call this.
__device__ __forceinline__ void rms_norm_row(float (&v)[8], const uint16_t* __restrict__ weight, float eps,
                                             int lane) {
    float w[8];
    load_row_bf16(weight, lane, w);
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fma(static_cast<double>(v[e]), static_cast<double>(v[e]), ss);
    const double r = 1.0 / __builtin_sqrt(wave_sum_f64(ss) / kHeadDim + static_cast<double>(eps));
#pragma unroll
    for (int e = 0; e < 8; ++e)
        v[e] = __uint_as_float(bf16_rne_bits_f64((static_cast<double>(v[e]) * static_cast<double>(w[e])) * r) << 16);
}

// ---------------------------------------------------------------- stores
// A store of the output bytes, either plain (the line stays in L2 as dirty data and is
// written back later) or non-temporal (the `nt` form: streamed out with evict-first
// priority).  Which one is faster depends on the kernel and was measured per kernel on
// MI355X: non-temporal pays for kernels that read far more than they write over a long
// run (the long-window compressors) and for the scattered row writers (the multi-layer
// store, the token gather); a short kernel whose few MB of output can sit in L2 until it
// ends (C4A) is faster with plain stores, and the short-window compressors switch to
// non-temporal stores only once their output outgrows the 256 MiB last-level cache.
template <bool kNt, typename T>
__device__ __forceinline__ void put(T* p, T v) {
    if constexpr (kNt)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// ---------------------------------------------------------------- quantise + store
// Quantise this lane's 8 bf16-valued floats of a row and write its share of the row at
// `slot` (the caller has checked the slot is inside the pool), with plain or
// non-temporal stores (kNt).  Every lane must call this.
template <Layout L, bool kNt = false>
__device__ __forceinline__ void quantize_store_row(uint8_t* __restrict__ pool, uint32_t slot,
                                                   const float (&v)[8], int lane) {
    using PK = PagedKV<L, kPageBits>;
    uint32_t amax[2] = {0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) amax[e >> 2] = max(amax[e >> 2], __float_as_uint(v[e]) & 0x7FFFFFFFu);
    amax[0] = oct_max_u32(amax[0]);
    amax[1] = oct_max_u32(amax[1]);

    uint8_t* code_row = PK::code_row(pool, slot);
    uint8_t* scale_row = PK::scale_row(pool, slot);
    uint32_t sbyte[2];

    if constexpr (L == Layout::V41) {
        // ue8m0: smallest k >= -127 with amax <= 448 * 2^k.  With amax = 2^E * (1+f),
        // amax / 448 = 2^(E-8) * (1+f) / 1.75, so k = E - 8 + (1+f > 1.75): read off the
        // exponent and mantissa bits, no division.  Byte = k + 127, clamped at 0.
        uint32_t word[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int biased = static_cast<int>(amax[h] >> 23);
            const int byte = max(0, biased - 8 + static_cast<int>((amax[h] & 0x7FFFFFu) > 0x600000u));
            sbyte[h] = static_cast<uint32_t>(byte);
            const float inv_scale = __uint_as_float(static_cast<uint32_t>(254 - byte) << 23);  // 2^-k
            // x * 2^-k is exact; the gfx950 pack convert rounds to nearest even into OCP
            // e4m3fn with the sign kept (|x * 2^-k| <= 448, so it never saturates).
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * h] * inv_scale, v[4 * h + 1] * inv_scale, 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * h + 2] * inv_scale, v[4 * h + 3] * inv_scale, w, true);
            word[h] = static_cast<uint32_t>(w);
        }
        put<kNt>(reinterpret_cast<uint32_t*>(code_row + 4 * lane), word[0]);
        put<kNt>(reinterpret_cast<uint32_t*>(code_row + kHalf + 4 * lane), word[1]);
    } else {
        // e4m3 scale = RNE(fl32(amax / 6)), held at 448; codes = e2m1 RNE of fl32(x / s).
        // fl32(x / s) lands exactly on a rounding midpoint t only when x / s == t (x has 8
        // significant bits, s 4, t 3), so the code equals counting the midpoints t*s
        // (exact products) that |x| passes, with ">=" at midpoints whose upper
        // neighbour has the even code.
        uint32_t half_word[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float t = __uint_as_float(amax[h]) / 6.0f;  // IEEE-correct division
            const uint32_t sc = min(e4m3_mag_code(t), 0x7Eu);
            sbyte[h] = sc;
            const float s = e4m3_mag_value(sc);
            const float m0 = 0.25f * s, m1 = 0.75f * s, m2 = 1.25f * s, m3 = 1.75f * s;
            const float m4 = 2.5f * s, m5 = 3.5f * s, m6 = 5.0f * s;
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = v[4 * h + e];
                const float a = fabsf(x);
                uint32_t c = static_cast<uint32_t>(a > m0) + static_cast<uint32_t>(a >= m1) +
                             static_cast<uint32_t>(a > m2) + static_cast<uint32_t>(a >= m3) +
                             static_cast<uint32_t>(a > m4) + static_cast<uint32_t>(a >= m5) +
                             static_cast<uint32_t>(a > m6);
                c |= (__float_as_uint(x) >> 28) & 8u;
                w |= c << (4 * e);
            }
            half_word[h] = sc == 0 ? 0u : w;  // a zero scale stores all-zero codes
        }
        put<kNt>(reinterpret_cast<uint16_t*>(code_row + 2 * lane), static_cast<uint16_t>(half_word[0]));
        put<kNt>(reinterpret_cast<uint16_t*>(code_row + kHalf / 2 + 2 * lane), static_cast<uint16_t>(half_word[1]));
    }

    // Scale row: lanes 0 and 32 hold the dwords of blocks 0-3 / 4-7 (first half) and
    // 8-11 / 12-15 (second half).  FP4 rows also get their 16 zero pad bytes.
    const uint32_t w0 = gather_block_bytes(sbyte[0], lane);
    const uint32_t w1 = gather_block_bytes(sbyte[1], lane);
    if ((lane & 31) == 0) {
        const int q = lane >> 5;
        put<kNt>(reinterpret_cast<uint32_t*>(scale_row + 4 * q), w0);
        put<kNt>(reinterpret_cast<uint32_t*>(scale_row + 8 + 4 * q), w1);
        if constexpr (L == Layout::V41_FP4)
            put<kNt>(reinterpret_cast<uint64_t*>(scale_row + kBlocks + 8 * q), uint64_t{0});
    }
}

}  // namespace kvq
