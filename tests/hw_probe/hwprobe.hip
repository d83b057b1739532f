// hwprobe.hip -- test support, not part of libkvq.so: measures, on the GPU the tests run
// on, the two hardware approximations whose error the ratio-2 / ratio-4 compressor's
// float32 error bound takes as given:
//   - v_exp_f32 (__builtin_amdgcn_exp2f): at most 1 ulp from 2^a wherever 2^a >= 2^-126,
//     for every float32 a in [-160, 1] (the kernel's exponent arguments are <= ~0, and
//     the kernel recomputes in float64 any channel whose argument falls below -126);
//   - v_rcp_f32 (__builtin_amdgcn_rcpf): at most 1 ulp from 1/l for every float32 l in
//     [1/2, 256) (the kernel's weight sums lie in [1, ratio] up to rounding).
// The references are the device library's float64 exp2 and IEEE float64 division, far
// more accurate than the 1-ulp float32 allowance being checked.  Results go to a
// caller-provided device buffer of 4 uint64 (zeroed by the caller):
//   out[0]  largest error seen, in units of 2^-32 ulp of the float32 result
//   out[1]  inputs whose reference is >= 2^-126 but whose result is below it (flushes)
//   out[2]  float32 bits of an input whose error is above 1 ulp (0 if none)
//   out[3]  number of inputs checked
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr unsigned kThreads = 256;
constexpr unsigned kBlocks = 65536;

__device__ void record(double y, double ref, uint32_t bits, unsigned long long* out) {
    int e;
    __builtin_frexp(ref, &e);                        // ref in [2^(e-1), 2^e)
    const double ulp = __builtin_ldexp(1.0, e - 24);  // float32 spacing at ref
    const double err = __builtin_fabs(y - ref) / ulp;
    const unsigned long long q = static_cast<unsigned long long>(err * 4294967296.0);
    atomicMax(&out[0], q);
    if (y < 0x1p-126) atomicAdd(&out[1], 1ull);
    if (err > 1.0) atomicMax(&out[2], static_cast<unsigned long long>(bits));
}

// inputs: float32 bit patterns lo..hi (inclusive), with the sign bit `sign` or'ed in
__global__ __launch_bounds__(kThreads) void exp2_sweep(uint32_t lo, uint32_t hi, uint32_t sign,
                                                       unsigned long long* out) {
    const uint64_t n = static_cast<uint64_t>(hi) - lo + 1;
    unsigned long long local = 0;
    for (uint64_t k = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x; k < n;
         k += static_cast<uint64_t>(gridDim.x) * kThreads) {
        const uint32_t bits = (lo + static_cast<uint32_t>(k)) | sign;
        const float a = __uint_as_float(bits);
        const double ref = exp2(static_cast<double>(a));
        ++local;
        if (ref < 0x1p-126) continue;
        record(static_cast<double>(__builtin_amdgcn_exp2f(a)), ref, bits, out);
    }
    atomicAdd(&out[3], local);
}

__global__ __launch_bounds__(kThreads) void rcp_sweep(uint32_t lo, uint32_t hi, unsigned long long* out) {
    const uint64_t n = static_cast<uint64_t>(hi) - lo + 1;
    unsigned long long local = 0;
    for (uint64_t k = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x; k < n;
         k += static_cast<uint64_t>(gridDim.x) * kThreads) {
        const uint32_t bits = lo + static_cast<uint32_t>(k);
        const float l = __uint_as_float(bits);
        ++local;
        record(static_cast<double>(__builtin_amdgcn_rcpf(l)), 1.0 / static_cast<double>(l), bits, out);
    }
    atomicAdd(&out[3], local);
}

}  // namespace

extern "C" {

// v_exp_f32 over every float32 in [-160, 1]; 0 on success, else the HIP error code.
int hwprobe_exp2(unsigned long long* out, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(exp2_sweep, dim3(kBlocks), dim3(kThreads), 0, s, 0u, 0x43200000u, 0x80000000u, out);  // -0 .. -160
    hipLaunchKernelGGL(exp2_sweep, dim3(kBlocks), dim3(kThreads), 0, s, 0u, 0x3F800000u, 0u, out);           // +0 .. 1
    return static_cast<int>(hipGetLastError());
}

// v_rcp_f32 over every float32 in [1/2, 256); 0 on success, else the HIP error code.
int hwprobe_rcp(unsigned long long* out, void* stream) {
    hipLaunchKernelGGL(rcp_sweep, dim3(kBlocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       0x3F000000u, 0x437FFFFFu, out);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
