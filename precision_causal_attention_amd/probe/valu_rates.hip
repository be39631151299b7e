// Issue-rate probe of the vector ALU instructions the attention kernels'
// softmax is made of (gfx950).  Every thread runs 8 independent chains of one
// instruction (or of one pair of instructions), register operands only and no
// memory traffic inside the loop, so the time per launch divided by the
// wave-instructions each SIMD issues is the instruction's issue cost.  The
// fp32 arithmetic chains read a register of their own besides the chained
// one: with one constant register shared by all chains v_fma_f32 ran half
// again as slow (an operand-fetch effect, not the ALU's rate).
// Not part of the attention library's ABI: it lives in the separate probe
// library beside the matrix-core probe.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kChains = 8;

// One chain step of instruction `op` (the list is the table of
// flamia_probe_valu_name).  Only ALU instructions on registers.
template <int OP>
__device__ __forceinline__ void step(float& x, float& y, uint32_t& u, const float c, const uint32_t cu) {
    if constexpr (OP == 0) asm volatile("v_fma_f32 %0, %0, %1, %1" : "+v"(x) : "v"(y));
    if constexpr (OP == 1) asm volatile("v_add_f32 %0, %0, %1" : "+v"(x) : "v"(y));
    if constexpr (OP == 2) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(x) : "v"(y));
    if constexpr (OP == 3) asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(x) : "v"(y), "v"(c));
    if constexpr (OP == 4) asm volatile("v_exp_f32 %0, %0" : "+v"(x));
    if constexpr (OP == 5) asm volatile("v_exp_f16 %0, %0" : "+v"(u));
    if constexpr (OP == 6) asm volatile("v_cvt_pk_fp8_f32 %0, %1, %2" : "+v"(u) : "v"(x), "v"(y));
    if constexpr (OP == 7) asm volatile("v_cvt_scalef32_pk_fp8_f32 %0, %1, %2, %3" : "+v"(u) : "v"(x), "v"(y), "v"(c));
    if constexpr (OP == 8) asm volatile("v_cvt_scalef32_pk_fp8_f16 %0, %1, %2" : "+v"(u) : "v"(cu), "v"(c));
    if constexpr (OP == 9) asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(u) : "v"(x), "v"(y));
    if constexpr (OP == 10) asm volatile("v_pk_fma_f16 %0, %0, %1, %1" : "+v"(u) : "v"(cu));
    if constexpr (OP == 11) asm volatile("v_pk_add_f16 %0, %0, %1" : "+v"(u) : "v"(cu));
    if constexpr (OP == 12) asm volatile("v_dot2_f32_bf16 %0, %1, %2, %0" : "+v"(x) : "v"(u), "v"(cu));
    // pairs: does the transcendental or the convert overlap with other work?
    if constexpr (OP == 13) asm volatile("v_exp_f32 %0, %0\n\tv_fma_f32 %1, %1, %2, %2" : "+v"(x), "+v"(y) : "v"(y));
    if constexpr (OP == 14) asm volatile("v_exp_f32 %0, %0\n\tv_cvt_pk_fp8_f32 %1, %2, %3" : "+v"(x), "+v"(u) : "v"(y), "v"(c));
    if constexpr (OP == 15) asm volatile("v_fma_f32 %0, %0, %1, %1\n\tv_cvt_pk_fp8_f32 %2, %3, %4" : "+v"(x), "+v"(u) : "v"(y), "v"(y), "v"(c));
}

template <int OP>
__global__ void __launch_bounds__(256) valu_rate_kernel(int iters, float* sink) {
    const int t = (int)threadIdx.x;
    float x[kChains], y[kChains];
    uint32_t u[kChains];
#pragma unroll
    for (int i = 0; i < kChains; ++i) {
        x[i] = 1e-3f * (float)(t + i + 1);
        y[i] = 0.5f + (float)i;
        u[i] = 0x3c003c00u + (uint32_t)i;
    }
    const float c = 0.75f;
    const uint32_t cu = 0x3a003a00u;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kChains; ++i) step<OP>(x[i], y[i], u[i], c, cu);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kChains; ++i) s += x[i] + y[i] + (float)u[i];
    // keeps the chains live; written only when the sum is NaN (the exponential
    // chains may reach it); the sink holds workgroups * 256 floats
    if (s != s) sink[(size_t)blockIdx.x * 256 + t] = s;
}

template <int OP>
void launch(int workgroups, int iters, float* sink, hipStream_t st) {
    hipLaunchKernelGGL(valu_rate_kernel<OP>, dim3((unsigned)workgroups), dim3(256), 0, st, iters, sink);
}

constexpr int kOps = 16;
const char* const kNames[kOps] = {
    "v_fma_f32", "v_add_f32", "v_mul_f32", "v_max3_f32", "v_exp_f32", "v_exp_f16", "v_cvt_pk_fp8_f32",
    "v_cvt_scalef32_pk_fp8_f32", "v_cvt_scalef32_pk_fp8_f16", "v_cvt_pk_bf16_f32", "v_pk_fma_f16",
    "v_pk_add_f16", "v_dot2_f32_bf16", "v_exp_f32 + v_fma_f32", "v_exp_f32 + v_cvt_pk_fp8_f32",
    "v_fma_f32 + v_cvt_pk_fp8_f32"};

}  // namespace

// Number of probed instructions (or pairs), and the name of probe `op`.
extern "C" int flamia_probe_valu_count(void) { return kOps; }
extern "C" const char* flamia_probe_valu_name(int op) { return (op >= 0 && op < kOps) ? kNames[op] : ""; }

// Launches `workgroups` workgroups of 256 threads on `stream`; each wave
// issues iters * 8 instructions (pairs: iters * 8 pairs) of probe `op`.
// sink: a device buffer of workgroups * 256 floats.  Returns 0 or a HIP
// error code.
extern "C" int flamia_probe_valu_rate(int op, int workgroups, int iters, float* sink, void* stream) {
    if (op < 0 || op >= kOps || workgroups <= 0 || iters <= 0 || !sink) return (int)hipErrorInvalidValue;
    const hipStream_t st = (hipStream_t)stream;
    switch (op) {
        case 0: launch<0>(workgroups, iters, sink, st); break;
        case 1: launch<1>(workgroups, iters, sink, st); break;
        case 2: launch<2>(workgroups, iters, sink, st); break;
        case 3: launch<3>(workgroups, iters, sink, st); break;
        case 4: launch<4>(workgroups, iters, sink, st); break;
        case 5: launch<5>(workgroups, iters, sink, st); break;
        case 6: launch<6>(workgroups, iters, sink, st); break;
        case 7: launch<7>(workgroups, iters, sink, st); break;
        case 8: launch<8>(workgroups, iters, sink, st); break;
        case 9: launch<9>(workgroups, iters, sink, st); break;
        case 10: launch<10>(workgroups, iters, sink, st); break;
        case 11: launch<11>(workgroups, iters, sink, st); break;
        case 12: launch<12>(workgroups, iters, sink, st); break;
        case 13: launch<13>(workgroups, iters, sink, st); break;
        case 14: launch<14>(workgroups, iters, sink, st); break;
        default: launch<15>(workgroups, iters, sink, st); break;
    }
    return (int)hipGetLastError();
}
