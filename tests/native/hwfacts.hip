// Test-only GPU library: sweeps of the gfx950 hardware operations the cast's
// fast path relies on, each through the library's own device helpers
// (nvfp4_device.hpp), so that the instructions tested are the ones the
// kernels execute.  The tests (tests/test_gpu_hwfacts.py) compare the
// results with references computed on the host: IEEE binary64 division for
// the reciprocals, the CPU oracle's E2M1 encoder for the FP4 conversion, and
// for the bf16 conversion the integer round-to-nearest-even of the fp32
// encoding, written out below independently of the library.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4_device.hpp"

using namespace nvfp4;

namespace {

// r = (1 + m * 2^-23) * 2^e for m = 0 .. 2^23 - 1: the hardware reciprocal,
// the library's RN(1/r) and RD(1/r)
__global__ void k_rcp(int e, float* __restrict__ y0, float* __restrict__ yrn, float* __restrict__ yrd) {
    const uint32_t m = blockIdx.x * blockDim.x + threadIdx.x;
    if (m >= (1u << 23)) return;
    const float r = __uint_as_float(((uint32_t)(e + 127) << 23) | m);
    y0[m] = __builtin_amdgcn_rcpf(r);
    yrn[m] = rcp_rn(r);
    yrd[m] = rcp_rd(r);
}

// byte i of the chunk = E2M1 nibbles of fp32 patterns start + 2i (low) and
// start + 2i + 1 (high), by the scaled conversion with scale 1.0
__global__ void k_fp4(uint64_t start, uint64_t npairs, uint8_t* __restrict__ out) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= npairs) return;
    const uint32_t u = (uint32_t)(start + 2 * i);
    const uint32_t w = put_fp4x2<0>(0u, __uint_as_float(u), __uint_as_float(u + 1u));
    out[i] = (uint8_t)(w & 0xffu);
}

// every fp32 pattern p in [start, start + n) that is not a NaN: the library's
// packed bf16 conversion against the integer rounding
//   bf16 = (p + 0x7FFF + ((p >> 16) & 1)) >> 16
// mismatches counted; the smallest mismatching pattern kept
__global__ void k_bf16(uint64_t start, uint64_t n, unsigned long long* __restrict__ bad,
                       uint32_t* __restrict__ first) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (2 * i >= n) return;
    const uint32_t p0 = (uint32_t)(start + 2 * i), p1 = p0 + 1u;
    const uint32_t hw = bf16x2_rne(__uint_as_float(p0), __uint_as_float(p1));
    const uint32_t ps[2] = {p0, p1};
    const uint32_t got[2] = {hw & 0xffffu, hw >> 16};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t p = ps[k];
        if ((p & 0x7F800000u) == 0x7F800000u && (p & 0x007FFFFFu) != 0u) continue;   // NaN
        const uint32_t ref = (uint32_t)(((uint64_t)p + 0x7FFFu + ((p >> 16) & 1u)) >> 16);
        if (got[k] != ref) {
            atomicAdd(bad, 1ull);
            atomicMin(first, p);
        }
    }
}

int check(hipError_t e) { return e == hipSuccess ? 0 : (int)e; }

}  // namespace

extern "C" {

// the three results for exponent e (2^23 values each, host arrays)
__attribute__((visibility("default"))) int hwf_rcp(int e, float* y0, float* yrn, float* yrd) {
    if (e < -126 || e > 127) return -1;
    const size_t n = (size_t)1 << 23;
    float *d0 = nullptr, *d1 = nullptr, *d2 = nullptr;
    int rc = check(hipMalloc(&d0, 3 * n * sizeof(float)));
    if (rc) return rc;
    d1 = d0 + n;
    d2 = d1 + n;
    hipLaunchKernelGGL(k_rcp, dim3((unsigned)(n / 256)), dim3(256), 0, nullptr, e, d0, d1, d2);
    rc = check(hipGetLastError());
    if (!rc) rc = check(hipMemcpy(y0, d0, n * sizeof(float), hipMemcpyDeviceToHost));
    if (!rc) rc = check(hipMemcpy(yrn, d1, n * sizeof(float), hipMemcpyDeviceToHost));
    if (!rc) rc = check(hipMemcpy(yrd, d2, n * sizeof(float), hipMemcpyDeviceToHost));
    (void)hipFree(d0);
    return rc;
}

// packed nibbles of patterns [start, start + 2 * npairs) into host out[npairs]
__attribute__((visibility("default"))) int hwf_fp4(uint64_t start, uint64_t npairs, uint8_t* out) {
    if (start % 2 != 0 || start + 2 * npairs > ((uint64_t)1 << 32)) return -1;
    uint8_t* d = nullptr;
    int rc = check(hipMalloc(&d, npairs));
    if (rc) return rc;
    hipLaunchKernelGGL(k_fp4, dim3((unsigned)((npairs + 255) / 256)), dim3(256), 0, nullptr, start, npairs, d);
    rc = check(hipGetLastError());
    if (!rc) rc = check(hipMemcpy(out, d, npairs, hipMemcpyDeviceToHost));
    (void)hipFree(d);
    return rc;
}

// all 2^32 patterns; *bad = number of non-NaN mismatches, *first = the
// smallest mismatching pattern (0xFFFFFFFF when none)
__attribute__((visibility("default"))) int hwf_bf16(unsigned long long* bad, uint32_t* first) {
    unsigned long long* d = nullptr;
    int rc = check(hipMalloc(&d, 16));
    if (rc) return rc;
    uint32_t* df = reinterpret_cast<uint32_t*>(d + 1);
    const unsigned long long zero = 0ull;
    const uint32_t none = 0xFFFFFFFFu;
    rc = check(hipMemcpy(d, &zero, 8, hipMemcpyHostToDevice));
    if (!rc) rc = check(hipMemcpy(df, &none, 4, hipMemcpyHostToDevice));
    const uint64_t chunk = (uint64_t)1 << 30;
    for (uint64_t s = 0; !rc && s < ((uint64_t)1 << 32); s += chunk) {
        hipLaunchKernelGGL(k_bf16, dim3((unsigned)(chunk / 2 / 256)), dim3(256), 0, nullptr, s, chunk, d, df);
        rc = check(hipGetLastError());
    }
    if (!rc) rc = check(hipMemcpy(bad, d, 8, hipMemcpyDeviceToHost));
    if (!rc) rc = check(hipMemcpy(first, df, 4, hipMemcpyDeviceToHost));
    (void)hipFree(d);
    return rc;
}

}  // extern "C"
