// Token-block quantization (FLAMIA paper, Section 3.1 token-block scaling,
// Section 3.2 rounded-up shared exponent, Section 3.5.1 fused quantization
// launch, Section 3.6.1 document-local blocks and dense per-token scale
// tables).
//
// One launch quantizes up to three tensors of the packed layout [T][H][d]
// (bf16 in, E4M3 codes [T][H][d] and one UE8M0 scale per (head, token) out).
// Grid: x = head chunk of 4 heads (over all tensors of the launch), y = 32-token
// window of the packed axis.  A workgroup owns every document-local block
// whose first token falls in its window (a document contributes at most one
// block start per window), so all blocks are covered exactly once without a
// block list.  Wave w of the workgroup takes head 4 * chunk + w.
// A wave quantizes one (block, head) pair of 32 tokens x d channels with all
// loads and stores coalesced: chunk c = lane + 64 r (r < d/16) is the 16-byte
// piece c % (d/8) of token c / (d/8), so each load instruction of the wave
// reads whole 2d-byte rows.
// HBM-bound: the input is read once, codes and scales are written once (and,
// for Q and K on the mixed path, their NVFP4 values).
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace flamia {

namespace {

// Sum over the d/8 consecutive lanes that hold the chunks of one token
// (8 lanes at d = 64, 16 at d = 128), returned in each of them.
template <int CPT>
__device__ __forceinline__ float token_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));   // lane ^ 1
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));   // lane ^ 2
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // other quad of 8
    if constexpr (CPT == 16)
        v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));  // other 8 of 16
    return v;
}

// Normalized Hadamard rotation of the token rows (Section 3.4, Appendix A.2):
// fp32 butterflies (a, b) -> (a + b, a - b) on channel pairs (j, j + h) for
// h = 1, 2, ..., d/2 in that order, then x fp32(1/sqrt(d)).  Lane chunk ch
// holds channels 8 ch .. 8 ch + 7 of its token, so h = 1, 2, 4 pair values of
// one lane and h = 8, 16, 32, 64 pair lanes ch ^ 1, ^ 2, ^ 4, ^ 8 of the
// same token (one 16-lane DPP row at most).
template <int CPT, int R>
__device__ __forceinline__ void rotate_rows(float (&v)[R][8], int ch) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if ((i & h) == 0) {
                    const float a = v[r][i], b = v[r][i + h];
                    v[r][i] = a + b;
                    v[r][i + h] = a - b;
                }
    auto stage = [&](auto down, auto up, int bit) {   // partner lane ch ^ bit
        const bool hi = (ch & bit) != 0;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int x = __float_as_int(v[r][i]);
                const float from_up = __int_as_float(__builtin_amdgcn_mov_dpp(x, decltype(up)::value, 0xF, 0xF, true));
                const float from_down = __int_as_float(__builtin_amdgcn_mov_dpp(x, decltype(down)::value, 0xF, 0xF, true));
                const float p = hi ? from_down : from_up;
                v[r][i] = hi ? p - v[r][i] : v[r][i] + p;
            }
    };
    // quad_perm [1,0,3,2] and [2,3,0,1] serve both lanes of a pair
    stage(std::integral_constant<int, 0xB1>{}, std::integral_constant<int, 0xB1>{}, 1);
    stage(std::integral_constant<int, 0x4E>{}, std::integral_constant<int, 0x4E>{}, 2);
    // row_shr:4 brings lane - 4, row_shl:4 brings lane + 4 (same for 8)
    stage(std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0x104>{}, 4);
    if constexpr (CPT == 16)
        stage(std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0x108>{}, 8);
    constexpr float rs = CPT == 8 ? 0.125f : 0x1.6a09e6p-4f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[r][i] = v[r][i] * rs;
}

// NVFP4 scale of a 16-channel group with largest magnitude amax (Section 2
// "Microscaling floating-point formats": E4M3 scale per 16 elements; rounded
// up like the MX exponents of Section 3.2): the smallest E4M3 value s with
// 6 s >= amax, 448 above 6 x 448, 0 for amax = 0.  The converted quotient
// lands within one code of the answer; exact comparisons settle it (6 s has
// at most 6 significant bits, so it is exact in fp32).
__device__ __forceinline__ float nvfp4_scale(float amax) {
    const float t = fminf(amax * (1.f / 6.f), 448.f);
    const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, t, 0, false) & 0x7Fu;
    const float s = fp8_to_f32(c);
    const float up = fp8_to_f32(min(c + 1u, 0x7Eu));
    const float dn = fp8_to_f32(c > 0u ? c - 1u : 0u);
    const float r = (6.f * s < amax) ? up : s;
    return (c > 0u && 6.f * dn >= amax) ? dn : r;
}

// value(E2M1(x / s)) * s as a bf16 pattern (s > 0): the nearest of
// s x {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturating at 6 s.
// |x| is compared with the exact midpoints m s (at most 7 significant bits),
// so no rounded quotient decides a code; the value is exact in bf16.  Ties at
// 0.25, 1.25, 2.5 and 5 go down (to codes 0, 2, 4, 6), those at 0.75, 1.75
// and 3.5 go up (to codes 2, 4, 6).  s = 0 (an all-zero group) gives +0.
__device__ __forceinline__ uint32_t nvfp4_bf16(float x, float s) {
    const float a = fabsf(x);
    float v = 0.f;
    v = a > 0.25f * s ? 0.5f * s : v;
    v = a >= 0.75f * s ? s : v;
    v = a > 1.25f * s ? 1.5f * s : v;
    v = a >= 1.75f * s ? 2.f * s : v;
    v = a > 2.5f * s ? 3.f * s : v;
    v = a >= 3.5f * s ? 4.f * s : v;
    v = a > 5.f * s ? 6.f * s : v;
    const uint32_t b = (__float_as_uint(v) >> 16) | ((__float_as_uint(x) >> 16) & 0x8000u);
    return s > 0.f ? b : 0u;
}

// Largest of a non-negative value over the d/8 consecutive lanes that hold
// one token's chunks, returned in each of them (bit patterns of non-negative
// floats order like the values).
template <int CPT>
__device__ __forceinline__ float token_max(float x) {
    uint32_t v = __float_as_uint(x);
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));    // lane ^ 1
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));    // lane ^ 2
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));   // other quad of 8
    if constexpr (CPT == 16)
        v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));  // other 8 of 16
    return __uint_as_float(v);
}

}  // namespace

// TOK: the exact options' per-token exponents (Appendix A.3): each token row
// gets the exponent of its own maximum instead of the block's.
template <int D, bool kDO, bool TOK>
__global__ void __launch_bounds__(256) quantize_kernel(const QuantArgs a) {
    constexpr int CPT = D / 8;               // 16-byte bf16 chunks per token row
    constexpr int R = kBlock * CPT / 64;     // chunks per lane
    const int w0 = blockIdx.y * kBlock;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (a.ndocs <= 0 || w0 >= a.ttot) return;

    // tensor and head of this wave
    int chunk = blockIdx.x, ti = 0;
    while (ti < a.ntensors && chunk >= (a.t[ti].heads + 3) / 4) { chunk -= (a.t[ti].heads + 3) / 4; ++ti; }
    if (ti >= a.ntensors) return;
    const QuantTensor tz = a.t[ti];
    const int h = 4 * chunk + wave;
    if (h >= tz.heads) return;
    const int H = tz.heads;

    const int ch = lane % CPT;               // chunk of the token row
    const int tok0 = lane / CPT;             // token of chunk r is tok0 + r * (64 / CPT)

    for (int doc = find_doc(a.cu, a.ndocs, w0); doc < a.ndocs; ++doc) {
        // boundaries clamped into [0, ttot], non-decreasing: a malformed
        // cu_seqlens (reported by the work-list kernel) never reads or
        // writes outside the tensors
        const int ds = min(max(a.cu[doc], 0), a.ttot), de = min(max(a.cu[doc + 1], ds), a.ttot);
        if (ds >= w0 + kBlock) break;
        if (de <= w0) continue;
        const int rel = w0 - ds;
        const int bs = rel <= 0 ? ds : ds + ((rel + kBlock - 1) / kBlock) * kBlock;
        if (bs >= w0 + kBlock || bs >= de) continue;
        const int nt = min(kBlock, de - bs);

        float v[R][8];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int tok = tok0 + r * (64 / CPT);
            uint4 u = make_uint4(0, 0, 0, 0);
            if (tok < nt) u = *reinterpret_cast<const uint4*>(tz.x + ((long)(bs + tok) * H + h) * D + 8 * ch);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[r][2 * k] = bf16_to_f32(w[k] & 0xFFFFu);
                v[r][2 * k + 1] = bf16_to_f32(w[k] >> 16);
            }
        }
        if (tz.rot) rotate_rows<CPT, R>(v, ch);
        // exponent of chunk row r (the block's, or with TOK the token's)
        int er[R];
        if constexpr (TOK) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float m = 0.f;
#pragma unroll
                for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[r][k]));
                er[r] = block_exponent(token_max<CPT>(m), -127);
            }
        } else {
            float amax = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[r][k]));
            amax = wave_max_nonneg(amax);
            const int e = block_exponent_uniform(amax, -127);
#pragma unroll
            for (int r = 0; r < R; ++r) er[r] = e;
        }
        // codes = E4M3(x * 2^-e): the power-of-two scaling is exact, the
        // convert rounds to nearest even.
        uint32_t packed[R][2];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int tok = tok0 + r * (64 / CPT);
            const int e = er[r];
#pragma unroll
            for (int k = 0; k < 2; ++k)
                packed[r][k] = (uint32_t)pack_fp8x4(ldexpf(v[r][4 * k], -e), ldexpf(v[r][4 * k + 1], -e),
                                                    ldexpf(v[r][4 * k + 2], -e), ldexpf(v[r][4 * k + 3], -e));
            if (tok < nt)
                *reinterpret_cast<uint2*>(tz.codes + ((long)(bs + tok) * H + h) * D + 8 * ch) =
                    make_uint2(packed[r][0], packed[r][1]);
        }
        if constexpr (TOK) {
            // lane t < 32 stores token t's exponent, held in chunk row t / G by
            // the lanes (t % G) CPT .. + CPT - 1, G = 64 / CPT tokens per row
            constexpr int G = 64 / CPT;
            const int src = (lane % G) * CPT;
            int et = 0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int x = __shfl(er[r], src);
                if (r == lane / G) et = x;
            }
            if (lane < nt) tz.scales[(long)h * a.ttot + bs + lane] = (uint8_t)(et + 127);
        } else {
            if (lane < nt) tz.scales[(long)h * a.ttot + bs + lane] = (uint8_t)(er[0] + 127);
        }

        // mixed path (Section 3.4): the NVFP4 values of the same rows, one
        // scale per 16 channels of each token (lanes ch and ch ^ 1 hold the
        // two halves of a group), expanded to bf16
        if (tz.nv) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int tok = tok0 + r * (64 / CPT);
                float gm = 0.f;
#pragma unroll
                for (int k = 0; k < 8; ++k) gm = fmaxf(gm, fabsf(v[r][k]));
                gm = fmaxf(gm, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(gm), 0xB1, 0xF, 0xF, true)));
                const float sg = nvfp4_scale(gm);
                uint32_t w[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    w[k] = nvfp4_bf16(v[r][2 * k], sg) | (nvfp4_bf16(v[r][2 * k + 1], sg) << 16);
                if (tok < nt)
                    *reinterpret_cast<uint4*>(tz.nv + ((long)(bs + tok) * H + h) * D + 8 * ch) =
                        make_uint4(w[0], w[1], w[2], w[3]);
            }
        }

        if constexpr (kDO) {
            // D_i = dO~_i . O_i with the dequantized dO and the bf16 output
            // (paper, Section 3.3), fp32 accumulation: each lane sums its 8
            // products code value x O (exact in fp32), the lanes of a token
            // are summed, and the block factor 2^e is applied last (exact).
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int tok = tok0 + r * (64 / CPT);
                uint4 u = make_uint4(0, 0, 0, 0);
                if (tok < nt) u = *reinterpret_cast<const uint4*>(a.o + ((long)(bs + tok) * H + h) * D + 8 * ch);
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
                float dot = 0.f;
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)packed[r][k], false);
                    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)packed[r][k], true);
                    dot = fmaf(lo[0], bf16_to_f32(w[2 * k] & 0xFFFFu), dot);
                    dot = fmaf(lo[1], bf16_to_f32(w[2 * k] >> 16), dot);
                    dot = fmaf(hi[0], bf16_to_f32(w[2 * k + 1] & 0xFFFFu), dot);
                    dot = fmaf(hi[1], bf16_to_f32(w[2 * k + 1] >> 16), dot);
                }
                dot = ldexpf(token_sum<CPT>(dot), er[r]);
                if (tok < nt && ch == 0) a.dvec[(long)h * a.ttot + bs + tok] = -dot;   // stored as -D
            }
        }
    }
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st) {
    if (a.ttot <= 0 || a.ntensors <= 0) return hipSuccess;
    int chunks = 0;
    for (int i = 0; i < a.ntensors; ++i) chunks += (a.t[i].heads + 3) / 4;
    const dim3 grid((unsigned)chunks, (unsigned)((a.ttot + kBlock - 1) / kBlock)), block(256);
    const bool dO = a.o != nullptr;
    // per-token exponents serve the operands of the exact options; their dO
    // is quantized inside the dQ pass, so this launch has no D variant for them
    if (a.per_token && dO) return hipErrorInvalidValue;
    if (a.d == 64) {
        if (a.per_token) hipLaunchKernelGGL((quantize_kernel<64, false, true>), grid, block, 0, st, a);
        else if (dO) hipLaunchKernelGGL((quantize_kernel<64, true, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((quantize_kernel<64, false, false>), grid, block, 0, st, a);
    } else {
        if (a.per_token) hipLaunchKernelGGL((quantize_kernel<128, false, true>), grid, block, 0, st, a);
        else if (dO) hipLaunchKernelGGL((quantize_kernel<128, true, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((quantize_kernel<128, false, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace flamia
