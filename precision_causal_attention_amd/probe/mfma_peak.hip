// Issue-rate probe of the block-scaled FP8 matrix core of gfx950
// (v_mfma_scale_f32_32x32x64_f8f6f4, the instruction behind every product of
// the attention kernels).  It measures the achievable peak that the
// benchmark reports beside the specification's 5.0 PFLOP/s: every wave runs
// `iters` rounds of four independent products on register operands, with no
// memory traffic inside the loop.  Not part of the attention library's ABI:
// a separate shared library that only the benchmark loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) mfma_peak_kernel(int iters, float* sink) {
    const int t = (int)threadIdx.x;
    // E4M3 codes of small positive values (exponent field 6 or 7): finite
    // products, no NaN codes
    const int ca = 0x30303030 | ((t & 7) * 0x01010101), cb = 0x38383838 | (((t >> 3) & 7) * 0x01010101);
    const v8i a = {ca, ca, ca, ca, ca, ca, ca, ca};
    const v8i b = {cb, cb, cb, cb, cb, cb, cb, cb};
    v16f c0 = {0}, c1 = {0}, c2 = {0}, c3 = {0};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
        c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 127, 0, 127);
        c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, 127, 0, 127);
        c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, 127, 0, 127);
    }
    const float s = (c0[0] + c1[5]) + (c2[10] + c3[15]);
    // keeps the products live; the sums are finite, so nothing is written
    if (s != s) sink[(size_t)blockIdx.x * 256 + t] = s;
}

// Launches `workgroups` workgroups of 256 threads on `stream`; each of the
// 4 waves issues 4 * iters products of 2 * 32 * 32 * 64 FLOP.  sink: a device
// buffer of workgroups * 256 floats (never written for finite products).
// Returns 0 or the HIP error code of the launch.
extern "C" int flamia_probe_mfma_peak(int workgroups, int iters, float* sink, void* stream) {
    if (workgroups <= 0 || iters <= 0 || !sink) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                       iters, sink);
    return (int)hipGetLastError();
}
