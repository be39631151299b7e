// Token-block quantization kernels (FLAMIA paper, Section 3.1 token-block
// scaling, Section 3.2 rounded-up shared exponent, Section 3.5.1 one fused
// launch per input tensor, Section 3.6.1 document-local blocks and dense
// per-token scale tables).
//
// Grid: one workgroup per 32-token window of the packed axis.  A workgroup
// owns every document-local block whose first token falls in its window (a
// document contributes at most one block start per window), so all blocks are
// covered exactly once without a host-side or device-side block list.
// Four waves per workgroup; a wave quantizes one (block, head) pair at a time:
// lane l carries token l/2 of the block and half l%2 of its d channels.
// HBM-bound: the input is read once, codes and scales written once.
#include "device.h"
#include "kernels.h"

namespace flamia {

template <int D, bool kDO>
__global__ void __launch_bounds__(256)
quantize_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ cu, int ndocs,
                int ttot, int heads, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                const uint16_t* __restrict__ o, float* __restrict__ dvec) {
    constexpr int HALF = D / 2;              // channels per lane
    constexpr int NV = HALF / 8;             // 16-byte bf16 vectors per lane
    const int w0 = blockIdx.x * kBlock;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int tok = lane >> 1, half = lane & 1;
    if (ndocs <= 0 || w0 >= ttot) return;

    for (int doc = find_doc(cu, ndocs, w0); doc < ndocs; ++doc) {
        const int ds = cu[doc], de = cu[doc + 1];
        if (ds >= w0 + kBlock) break;
        if (de <= w0) continue;
        const int rel = w0 - ds;
        const int bs = rel <= 0 ? ds : ds + ((rel + kBlock - 1) / kBlock) * kBlock;
        if (bs >= w0 + kBlock || bs >= de) continue;
        const int nt = min(kBlock, de - bs);
        const bool active = tok < nt;
        const int t = bs + (active ? tok : 0);

        for (int h = wave; h < heads; h += 4) {
            const long base = ((long)t * heads + h) * D + half * HALF;
            float v[HALF];
            float amax = 0.f;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                uint4 u = active ? *reinterpret_cast<const uint4*>(x + base + 8 * j) : make_uint4(0, 0, 0, 0);
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[8 * j + 2 * k] = bf16_to_f32(w[k] & 0xFFFFu);
                    v[8 * j + 2 * k + 1] = bf16_to_f32(w[k] >> 16);
                }
            }
#pragma unroll
            for (int j = 0; j < HALF; ++j) amax = fmaxf(amax, fabsf(v[j]));
            amax = wave_max(amax);
            const int e = block_exponent(amax, -127);
            // codes = E4M3(x * 2^-e): the power-of-two scaling is exact, the
            // convert rounds to nearest even.
            uint32_t packed[HALF / 4];
#pragma unroll
            for (int j = 0; j < HALF / 4; ++j) {
                packed[j] = (uint32_t)pack_fp8x4(ldexpf(v[4 * j], -e), ldexpf(v[4 * j + 1], -e),
                                                 ldexpf(v[4 * j + 2], -e), ldexpf(v[4 * j + 3], -e));
            }
            if (active) {
#pragma unroll
                for (int j = 0; j < HALF / 16; ++j)
                    *reinterpret_cast<uint4*>(codes + base + 16 * j) =
                        make_uint4(packed[4 * j], packed[4 * j + 1], packed[4 * j + 2], packed[4 * j + 3]);
                if (half == 0) scales[(long)h * ttot + t] = (uint8_t)(e + 127);
            }
            if constexpr (kDO) {
                // D_i = dO~_i . O_i with the dequantized dO and the bf16 output
                // (paper, Section 3.3), fp32 accumulation.
                float dot = 0.f;
#pragma unroll
                for (int j = 0; j < NV; ++j) {
                    uint4 u = active ? *reinterpret_cast<const uint4*>(o + base + 8 * j) : make_uint4(0, 0, 0, 0);
                    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t cw = packed[(8 * j + 2 * k) / 4] >> (8 * ((8 * j + 2 * k) % 4));
                        const float d0 = ldexpf(fp8_to_f32(cw & 0xFFu), e);
                        const float d1 = ldexpf(fp8_to_f32((cw >> 8) & 0xFFu), e);
                        dot = fmaf(d0, bf16_to_f32(w[k] & 0xFFFFu), dot);
                        dot = fmaf(d1, bf16_to_f32(w[k] >> 16), dot);
                    }
                }
                dot += __shfl_xor(dot, 1, 64);
                if (active && half == 0) dvec[(long)h * ttot + t] = dot;
            }
        }
    }
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st) {
    if (a.ttot <= 0) return hipSuccess;
    const dim3 grid((a.ttot + kBlock - 1) / kBlock), block(256);
    const bool dO = a.o != nullptr;
    if (a.d == 64) {
        if (dO) hipLaunchKernelGGL((quantize_kernel<64, true>), grid, block, 0, st, a.x, a.cu, a.ndocs, a.ttot, a.heads, a.codes, a.scales, a.o, a.dvec);
        else hipLaunchKernelGGL((quantize_kernel<64, false>), grid, block, 0, st, a.x, a.cu, a.ndocs, a.ttot, a.heads, a.codes, a.scales, a.o, a.dvec);
    } else {
        if (dO) hipLaunchKernelGGL((quantize_kernel<128, true>), grid, block, 0, st, a.x, a.cu, a.ndocs, a.ttot, a.heads, a.codes, a.scales, a.o, a.dvec);
        else hipLaunchKernelGGL((quantize_kernel<128, false>), grid, block, 0, st, a.x, a.cu, a.ndocs, a.ttot, a.heads, a.codes, a.scales, a.o, a.dvec);
    }
    return hipGetLastError();
}

}  // namespace flamia
