// MXFP8 causal forward over packed documents (FLAMIA paper: Section 2
// equations S = QK^T/sqrt(d), P = softmax(S), O = PV; Section 3.1 token-block
// scales applied by the block-scaled product; Appendix B.1 P-hat = E4M3(2^c p)
// with a conditional running maximum; Section 3.6.1 masking of keys outside
// the document and of the causal boundary on the diagonal tile only).
//
// One workgroup = one work item (document, query head, 128-query tile
// anchored at the document start); four waves, each owning 32 queries.
// Per 128-key tile (ascending, anchored at the document start):
//   S^T[key][query] = K^ Q^T      4 block-scaled MFMAs 32x32x64 per 64 channels
//                                 (A = key rows from LDS, B = the wave's query rows
//                                 kept in registers; the MFMA applies 2^(e_K + e_Q))
//   x = S * softmax_scale * log2(e);  tile max -> conditional rescale (tau)
//   p' = 2^(x - (m - c)) = 2^c p;  P-hat = E4M3(p')
//   O^T[d][query] += V^T P-hat^T   A = V^T read from LDS with the transposing
//                                 ds_read_b64_tr_b8, B = P-hat straight from the
//                                 S^T accumulators (their layout is the operand
//                                 layout), scale of each 32-key block of V.
// The accumulator layout puts one query per lane column, so the online-softmax
// statistics are per-lane scalars (plus one exchange between lane halves).
// Mixed NVFP4/FP8 path (Section 3.4): S^T comes from the NVFP4 values of K and
// Q instead, expanded to bf16 by the quantizer (an E2M1 element times an E4M3
// scale has at most 6 significant bits, so bf16 holds it exactly; the
// block-scaled MFMA cannot apply one E4M3 scale per 16 channels): D/16 bf16
// MFMAs 32x32x16 per sub-tile, no scale operands; everything after S is the
// same.
// Exact options (Appendix A.3): Q, K and V carry one exponent per token.  S
// applies Q's and K's per lane as before.  P-hat V contracts over keys, so V's
// token exponent e_j moves into P-hat: P-hat = E4M3(p' 2^(e_j - E)), and the
// product's B-operand scale (one per query column and 32-key block) is
// 2^E, with E the largest e_j of the block's keys up to the query: the block
// maximum below the diagonal, the running maximum on the diagonal block.
// The row sum keeps the unfolded p'.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace flamia {

template <int D, int MIX, int EXACT>
struct FwdSmem {
    static constexpr int kStride = D + 16;        // row pitch of a code tile in LDS (bank spread)
    static constexpr int kKStride = MIX ? 2 * D + 16 : kStride;   // K: bf16 NVFP4 values when mixed
    uint8_t k[kTile * kKStride];
    uint8_t v[kTile * kStride];
    uint8_t ek[kTile];
    uint8_t ev[kTile];
    // exact options: 2^(e_j - block maximum) per key, the running maximum of
    // e_j from the block start (UE8M0 byte) per key, the block maxima
    alignas(16) float dvp[EXACT ? kTile : 4];
    uint8_t pmx[EXACT ? kTile : 4];
    uint8_t bmx[4];
};

// Schraudolph's exponential (inference only; paper Section 3.7, Appendix
// C.2): t = 2^7 y + K in one fp32 FMA, K = 1.5 * 2^23 + 2^7 (127 - 0.0573)
// rounded to fp32 (an integer), so 2^7 y is rounded to an integer in the low
// mantissa bits of t; those low 16 bits are the bf16 pattern of
// 2^floor(z) (1 + {z}), z = y - 7/128, moved to the high half of a float and
// clamped at zero.  Here y = x c1 + (c - m) and the per-row part is folded
// into the constant: t = s * (2^7 c1) + (2^7 (c - m) + K), one FMA per score.
constexpr float kSchraudolphK = (float)(12582912.0 + 128.0 * (127.0 - 0.0573));

// Key-pair class of accumulator register i (key bits 1, 3, 4; see the key
// layout of the S^T tiles): registers of classes below FAST take the
// approximation.
__device__ __forceinline__ constexpr int pair_class(int i) {
    return ((i >> 1) & 1) | (((i >> 2) & 1) << 1) | (((i >> 3) & 1) << 2);
}

// At least two workgroups per CU (two waves per SIMD) at both head
// dimensions: at d = 128 one wave per SIMD leaves the matrix-core and memory
// latencies exposed (the kernel ran 35% longer), and the few registers the
// mixed and inference variants spill cost less than that.  The exact
// options' d = 64 variant is held to three waves per SIMD, like the default
// one reaches by itself: three spilled registers cost less than the lost
// wave (the forward ran 14% faster).
// PROBE = 1: the diagnostics instantiation (writes the probed raw scores).
template <int D, int ROWSUM, int FAST, int MIX, int EXACT, int PROBE = 0>
__global__ void __launch_bounds__(256, (D == 64 && EXACT) ? 3 : 2) fwd_kernel(const FwdArgs a) {
    constexpr int KC = D / 64;                    // 64-channel contraction steps of S
    constexpr int NC = D / 16;                    // 16-channel steps of S on the mixed path
    constexpr int DT = D / 32;                    // 32-row channel tiles of O^T
    constexpr int STR = FwdSmem<D, MIX, EXACT>::kStride;
    constexpr int KSTR = FwdSmem<D, MIX, EXACT>::kKStride;
    constexpr int CHUNKS = kTile * D / 16;        // 16-byte chunks of one code tile
    constexpr int KCHUNKS = MIX ? 2 * CHUNKS : CHUNKS;   // 16-byte chunks of one K tile
    constexpr int KRB = MIX ? 2 * D / 16 : D / 16;       // 16-byte chunks of one K row
    __shared__ FwdSmem<D, MIX, EXACT> sm;

    const int ti = (int)blockIdx.x / a.hq;
    if (ti >= *a.ntiles) return;
    const int4 it = a.tiles[ti];
    const int q0 = it.x, ds = it.y, de = it.z;
    const int h = xcd_head((int)blockIdx.x - ti * a.hq, a.hq, it.w);
    const int g = h / (a.hq / a.hkv);
    const int L = de - ds;
    const int lq0 = q0 - ds;
    const int ntiles = lq0 / kTile + 1;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // provably wave-uniform copy
    const int lg = lane >> 5, lr = lane & 31;
    const int q_loc = lq0 + 32 * wave + lr;       // document-local query of this lane
    const bool q_valid = q_loc < L;
    const int q_row = ds + min(q_loc, L - 1);     // clamped row inside the document for loads

    // The wave's 32 query rows as the B operand (column = query, k = channel):
    // bytes 0..15 = channels 64kc + 16lg .. +16, bytes 16..31 = 64kc + 32 + 16lg .. +16.
    v8i qb[MIX ? 1 : KC];
    // mixed path: channels 16 kc + 8 lg .. + 8 of the query's NVFP4 values
    // (the K rows use the same assignment)
    u32x4 qn[MIX ? NC : 1];
    if constexpr (MIX) {
        const uint16_t* qp = a.qn + ((long)q_row * a.hq + h) * D;
#pragma unroll
        for (int kc = 0; kc < NC; ++kc) qn[kc] = *reinterpret_cast<const u32x4*>(qp + 16 * kc + 8 * lg);
    } else {
        const uint8_t* qp = a.qc + ((long)q_row * a.hq + h) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const uint4 lo = *reinterpret_cast<const uint4*>(qp + 64 * kc + 16 * lg);
            const uint4 hi = *reinterpret_cast<const uint4*>(qp + 64 * kc + 32 + 16 * lg);
            qb[kc] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
    }
    const int eq = MIX ? 127 : a.qs[(long)h * a.ttot + q_row];

    v16f acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = v16f{0};
    float m = -INFINITY;       // running maximum of x (retained until exceeded by > tau)
    float l = 0.f;             // running sum of p' = 2^c p over this lane's keys

    // transposed-read source address pattern (see lds_read_tr8): within the
    // 16-lane group, source lane s points at key (s/2)-pattern, channel half s%2
    const int s16 = lane & 15, grp = (lane >> 4) & 1;
    const int tr_key = 8 * ((s16 >> 1) >> 2) + 4 * lg + ((s16 >> 1) & 3);
    const int tr_col = 16 * grp + 8 * (s16 & 1);

    // ---- K^/V^ code tiles and scales (mixed: K's NVFP4 values), prefetched
    // into registers one tile ahead
    u32x4 kr[KCHUNKS / 256], vr[CHUNKS / 256];
    uint32_t ekr, evr;
    auto fetch = [&](const int k0) {
        if constexpr (MIX) {
#pragma unroll
            for (int r = 0; r < CHUNKS / 256; ++r) {
                const int c = tid + 256 * r;
                const int row = c / (D / 16), col = (c % (D / 16)) * 16;
                const long krow = min(k0 + row, a.ttot - 1);
                vr[r] = *reinterpret_cast<const u32x4*>(a.vc + (krow * a.hkv + g) * D + col);
            }
            ekr = 127;
            evr = a.vs[(long)g * a.ttot + min(k0 + (tid & 127), a.ttot - 1)];
#pragma unroll
            for (int r = 0; r < KCHUNKS / 256; ++r) {
                const int c = tid + 256 * r;
                const int row = c / KRB, col = (c % KRB) * 8;      // col in bf16 elements
                const long krow = min(k0 + row, a.ttot - 1);
                kr[r] = *reinterpret_cast<const u32x4*>(a.kn + (krow * a.hkv + g) * D + col);
            }
        } else {
            fetch_kv_tile<D>(kr, vr, ekr, evr, a.kc, a.ks, a.vc, a.vs, k0, a.ttot, a.hkv, g, tid);
        }
    };
    fetch(ds);

    // One 128-key tile; DIAG marks the last (diagonal) tile, the only one that
    // needs the causal mask and the only one with nothing left to prefetch.
    auto tile = [&](const int t, auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < KCHUNKS / 256; ++r) {
            const int c = tid + 256 * r;
            const int row = c / KRB, col = (c % KRB) * 16;
            *reinterpret_cast<u32x4*>(&sm.k[row * KSTR + col]) = kr[r];
        }
#pragma unroll
        for (int r = 0; r < CHUNKS / 256; ++r) {
            const int c = tid + 256 * r;
            const int row = c / (D / 16), col = (c % (D / 16)) * 16;
            *reinterpret_cast<u32x4*>(&sm.v[row * STR + col]) = vr[r];
        }
        if (tid < kTile) {
            sm.ek[tid] = (uint8_t)ekr;
            sm.ev[tid] = (uint8_t)evr;
        }
        if constexpr (EXACT) {
            // V's token exponents (biased bytes): thread tid holds key tid % 128,
            // and each 32-lane half-wave holds one 32-key block.  Block maximum
            // by DPP over 16 lanes plus one row swap; running maximum from the
            // block start by shifted reads.
            const uint32_t bm = halfwave_max(evr);
            const int l32 = tid & 31;
            uint32_t pm = evr;
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) {
                const uint32_t u = (uint32_t)__shfl_up((int)pm, off, 32);
                if (l32 >= off) pm = max(pm, u);
            }
            if (tid < kTile) {
                sm.dvp[tid] = ldexpf(1.f, (int)evr - (int)bm);
                sm.pmx[tid] = (uint8_t)pm;
                if (l32 == 0) sm.bmx[tid >> 5] = (uint8_t)bm;
            }
        }
        __syncthreads();
        if constexpr (!DIAG) fetch(ds + kTile * (t + 1));

        // On the diagonal tile, sub-tiles kk > wave lie entirely after every
        // query of the wave: they contribute p = 0, so they are skipped (no
        // product, no exponential); sub-tile kk == wave is the only one that
        // needs the mask, sub-tiles kk < wave lie entirely before the queries.
        // ---- S^T = K^ Q^T for the 4 sub-tiles of 32 keys
        v16f s[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (DIAG && kk > wave_u) continue;
            const int row = 32 * kk + lr;
            s[kk] = v16f{0};
            if constexpr (MIX) {
#pragma unroll
                for (int kc = 0; kc < NC; ++kc) {
                    const u32x4 ka = *reinterpret_cast<const u32x4*>(&sm.k[row * KSTR + 32 * kc + 16 * lg]);
                    s[kk] = mfma_bf16(ka, qn[kc], s[kk]);
                }
            } else {
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const uint4 lo = *reinterpret_cast<const uint4*>(&sm.k[row * KSTR + 64 * kc + 16 * lg]);
                    const uint4 hi = *reinterpret_cast<const uint4*>(&sm.k[row * KSTR + 64 * kc + 32 + 16 * lg]);
                    const v8i ka = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    s[kk] = mfma_mx(ka, qb[kc], s[kk], sm.ek[row], eq);
                }
            }
        }
        if constexpr (PROBE) {
            // diagnostics: the raw scores of the probed query tile (before the mask)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (DIAG && kk > wave_u) continue;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float* sp = probe_slot(a.probe, 0, h, ds, ds + q_loc,
                                           kTile * t + 32 * kk + 8 * (i >> 2) + 4 * lg + (i & 3));
                    if (sp) *sp = s[kk][i];
                }
            }
        }
        // ---- causal mask (sub-tile kk == wave of the diagonal tile):
        // accumulator register i of sub-tile kk holds key 128t + 32kk +
        // 8(i/4) + 4lg + i%4; it is masked when that key lies after the lane's
        // query.  Tile maximum on the raw scores (rounding is monotonic, so
        // max(S) * c1 = max(S * c1) exactly).
        float smax = -INFINITY;
        const int lim = q_loc - kTile * t - 4 * lg;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (DIAG && kk > wave_u) continue;
            if (DIAG && kk == wave_u) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * kk + 8 * (i >> 2) + (i & 3) > lim) s[kk][i] = -INFINITY;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) smax = fmaxf(smax, s[kk][i]);
        }
        const float mu = max_xor32(smax) * a.c1;
        // ---- conditional running maximum (replace when exceeded by more than tau)
        const float m_new = (m == -INFINITY || mu - m > a.tau) ? mu : m;
        if (__any(m_new != m)) {
            const float alpha = (m == -INFINITY) ? 0.f : exp2_fast(m - m_new);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
        }
        m = m_new;
        const float nmc = a.c_log2 - m;                 // p' = 2^(x - m + c)
        const float c1x128 = a.c1 * 128.f;              // exact (power of two)
        const float kofs = fmaf(128.f, nmc, kSchraudolphK);
        auto pexp = [&](float sv, int i) -> float {
            if (FAST > 0 && pair_class(i) < FAST) {
                const int b = max(__float_as_int(fmaf(sv, c1x128, kofs)) << 16, 0);
                return __int_as_float(b);
            }
            return exp2_fast(fmaf(sv, a.c1, nmc));
        };
        // ---- p' = 2^c p and P-hat codes in operand byte order (byte i of a
        // sub-tile = accumulator register i)
        int pc[4][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (DIAG && kk > wave_u) {
                    pc[kk][j] = 0;
                    continue;
                }
                const float p0 = pexp(s[kk][4 * j], 4 * j);
                const float p1 = pexp(s[kk][4 * j + 1], 4 * j + 1);
                const float p2 = pexp(s[kk][4 * j + 2], 4 * j + 2);
                const float p3 = pexp(s[kk][4 * j + 3], 4 * j + 3);
                int w;
                if constexpr (EXACT) {
                    // fold 2^(e_j - E) (exact scaling): keys 32kk + 8j + 4lg + 0..3
                    const int kb = 32 * kk + 8 * j + 4 * lg;
                    float4 f;
                    if (DIAG && kk == wave_u) {
                        const int pe = sm.pmx[32 * kk + lr];   // E of the lane's query
                        f = make_float4(ldexpf(1.f, (int)sm.ev[kb] - pe), ldexpf(1.f, (int)sm.ev[kb + 1] - pe),
                                        ldexpf(1.f, (int)sm.ev[kb + 2] - pe), ldexpf(1.f, (int)sm.ev[kb + 3] - pe));
                    } else {
                        f = *reinterpret_cast<const float4*>(&sm.dvp[kb]);
                    }
                    w = pack_fp8x4(p0 * f.x, p1 * f.y, p2 * f.z, p3 * f.w);
                } else {
                    w = pack_fp8x4(p0, p1, p2, p3);
                }
                pc[kk][j] = w;
                if constexpr (ROWSUM == 0) l += (p0 + p1) + (p2 + p3);
                else l += fp8x4_sum(w);
            }
        // ---- O^T += V^T P-hat^T, two 64-key chunks
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            if (DIAG && 2 * c > wave_u) continue;      // both sub-tiles skipped: P-hat = 0
            const v8i pb = v8i{pc[2 * c][0], pc[2 * c][1], pc[2 * c][2], pc[2 * c][3],
                               pc[2 * c + 1][0], pc[2 * c + 1][1], pc[2 * c + 1][2], pc[2 * c + 1][3]};
            // scales: V's block (A), or with the exact options E of the lane's
            // query and key block 2c + lg (B)
            int sv = 127, sp = 127;
            if constexpr (EXACT) {
                const int b = 2 * c + lg;
                sp = (DIAG && b == wave_u) ? (int)sm.pmx[32 * b + lr] : (int)sm.bmx[b];
            } else {
                sv = sm.ev[64 * c + 32 * lg];
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                v2i r[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    r[rr] = lds_read_tr8(&sm.v[(64 * c + 16 * rr + tr_key) * STR + 32 * dt + tr_col]);
                const v8i va = v8i{r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
                acc[dt] = mfma_mx(va, pb, acc[dt], sv, sp);
            }
        }
    };
    for (int t = 0; t + 1 < ntiles; ++t) tile(t, std::false_type{});
    tile(ntiles - 1, std::true_type{});
    // ---- epilogue: O = acc / l (both carry the 2^c factor), lse2 = m + log2(l/2^c)
    const float lt = add_xor32(l);
    if (q_valid) {
        const float inv = 1.f / lt;
        uint16_t* op = a.o + ((long)(ds + q_loc) * a.hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t b01 = pack_bf16x2(acc[dt][4 * j] * inv, acc[dt][4 * j + 1] * inv);
                const uint32_t b23 = pack_bf16x2(acc[dt][4 * j + 2] * inv, acc[dt][4 * j + 3] * inv);
                *reinterpret_cast<uint2*>(op + 32 * dt + 8 * j + 4 * lg) = make_uint2(b01, b23);
            }
        if (lg == 0) a.lse2[(long)h * a.ttot + ds + q_loc] = m + (log2_fast(lt) - a.c_log2);
    }
}

template <int D, int ROWSUM>
static void launch_fwd_fast(const FwdArgs& a, dim3 g, dim3 b, hipStream_t st) {
    // the inference exponential is offered on the MXFP8 path only
    if (a.qn) hipLaunchKernelGGL((fwd_kernel<D, ROWSUM, 0, 1, 0>), g, b, 0, st, a);
    else if (a.fast_exp == 8) hipLaunchKernelGGL((fwd_kernel<D, ROWSUM, 8, 0, 0>), g, b, 0, st, a);
    else if (a.fast_exp == 5) hipLaunchKernelGGL((fwd_kernel<D, ROWSUM, 5, 0, 0>), g, b, 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<D, ROWSUM, 0, 0, 0>), g, b, 0, st, a);
}

hipError_t launch_fwd(const FwdArgs& a, int d, long grid, hipStream_t st) {
    if (grid <= 0) return hipSuccess;
    const dim3 g((unsigned)grid), b(256);
    // the exact options take the unquantized row sum, the exact exponential
    // and the MXFP8 scores (checked by the host layer)
    if (a.exact && (a.rowsum || a.fast_exp || a.qn)) return hipErrorInvalidValue;
    if (a.probe.scores) {
        // diagnostics: the MXFP8 path with the exact exponential (checked by the host layer)
        if (a.exact || a.fast_exp || a.qn) return hipErrorInvalidValue;
        if (d == 64) {
            if (a.rowsum) hipLaunchKernelGGL((fwd_kernel<64, 1, 0, 0, 0, 1>), g, b, 0, st, a);
            else hipLaunchKernelGGL((fwd_kernel<64, 0, 0, 0, 0, 1>), g, b, 0, st, a);
        } else {
            if (a.rowsum) hipLaunchKernelGGL((fwd_kernel<128, 1, 0, 0, 0, 1>), g, b, 0, st, a);
            else hipLaunchKernelGGL((fwd_kernel<128, 0, 0, 0, 0, 1>), g, b, 0, st, a);
        }
        return hipGetLastError();
    }
    if (d == 64) {
        if (a.exact) hipLaunchKernelGGL((fwd_kernel<64, 0, 0, 0, 1>), g, b, 0, st, a);
        else if (a.rowsum) launch_fwd_fast<64, 1>(a, g, b, st);
        else launch_fwd_fast<64, 0>(a, g, b, st);
    } else {
        if (a.exact) hipLaunchKernelGGL((fwd_kernel<128, 0, 0, 0, 1>), g, b, 0, st, a);
        else if (a.rowsum) launch_fwd_fast<128, 1>(a, g, b, st);
        else launch_fwd_fast<128, 0>(a, g, b, st);
    }
    return hipGetLastError();
}

}  // namespace flamia
