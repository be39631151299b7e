// Query-major dQ pass of the MXFP8 causal backward (FLAMIA paper: Section 2
// equation dQ = dS K; Section 3.3: dS rebuilt from the forward's quantized
// Q/K and the saved row statistic, one E4M3 exponent per 32x32
// document-local block).
//
// One workgroup = one work item (document, query head, 128-query tile
// anchored at the document start); wave w owns queries 32w..32w+31; key
// tiles are visited in ascending order up to the diagonal, as in the forward.
// Per 128-key tile:
//   S^T [key][query] = K^ Q^T     (A = key rows from LDS, B = query rows in registers)
//   dP^T[key][query] = V^ dO^T    (A = value rows from LDS, B = dO rows in registers)
//   P = 2^(x - lse2), dS = P (dP - D) (the dP product starts from -D); each
//   32x32 accumulator tile is one dS
//   block: its maximum gives the exponent, the convert divides by 2^e
//   dQ^T[d][query] += K^T dS-hat^T   (A = K^T by the transposing LDS read,
//                                     B = dS-hat straight from the accumulators)
// The score and dP products use the same operands, instructions and order as
// the key-major pass (role-swapped MFMA operands give identical bits), so
// dS-hat here is bitwise the payload the key-major pass feeds to dK.  dQ is
// owned by one workgroup: no atomics, deterministic, written once as bf16.
// Mixed NVFP4/FP8 path (Section 3.4): S^T comes from the NVFP4 values of K
// and Q (bf16 MFMAs, as in the forward), while dQ still contracts over the
// E4M3 token-block K^, so a key tile stages both forms of its rows.
// Without a dS store the pass runs before the key-major one and quantizes dO
// itself (Section 3.5.1 fused quantization): the wave's 32 queries are one
// document-local 32-token block, so the wave computes the block exponent,
// the codes (its own dP operand) and D = dO~ . O, and writes them for the
// key-major pass, in the order of the standalone quantizer, so D is the same
// bit for bit.
// Exact options (Appendix A.3): dO gets one exponent per query (the lane's own
// maximum); dQ contracts over keys, so K's token exponent e_j moves into dS:
// z = dS 2^e_j, and each query row takes its own exponent per 32-key block
// (the maximum of |z| over the lane's 16 registers and its partner lane's),
// which the product applies as its per-column B scale; K^T's A scale is 1.
// Nothing a query row computes then depends on later tokens.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace flamia {

template <int D, int MIX, int EXACT>
struct DqSmem {
    static constexpr int kStride = D + 16;
    static constexpr int kNStride = 2 * D + 16;   // bf16 NVFP4 rows of K (mixed path)
    uint8_t k[kTile * kStride];
    uint8_t v[kTile * kStride];
    uint8_t ek[kTile];
    uint8_t ev[kTile];
    alignas(16) uint8_t kn[MIX ? kTile * kNStride : 16];
    alignas(16) float kf[EXACT ? kTile : 4];      // exact options: 2^(K's token exponent)
};

// At least two workgroups per CU at both head dimensions (at d = 128 one wave
// per SIMD left latencies exposed: 36% longer).
// PROBE = 1: the diagnostics instantiation (writes the probed raw scores).
template <int D, int MIX, bool FUSED, int EXACT, int PROBE = 0>
__global__ void __launch_bounds__(256, (D == 64 && !MIX && !PROBE) ? 3 : 2) dq_kernel(const DqArgs a) {
    constexpr int KC = D / 64;
    constexpr int NC = D / 16;                    // 16-channel steps of S on the mixed path
    constexpr int DT = D / 32;
    constexpr int STR = DqSmem<D, MIX, EXACT>::kStride;
    constexpr int NSTR = DqSmem<D, MIX, EXACT>::kNStride;
    constexpr int CHUNKS = kTile * D / 16;
    constexpr int NCH = MIX ? 2 * CHUNKS / 256 : 1;   // 16-byte chunks per thread of a bf16 K tile
    static_assert(!EXACT || (FUSED && !MIX), "the exact options run the fused MXFP8 pass");
    // d = 64: two tile buffers.  Tile t is stored into buffer t % 2, last
    // read by the products of tile t - 2, which every wave finished before
    // the barrier of tile t - 1, so one barrier per tile suffices (1% faster
    // than one buffer and two barriers).  The second buffer raises the
    // registers the compiler plans for; the MXFP8 variants are held to three
    // waves per SIMD (168 VGPRs, two spilled outside the tile loop).  d = 128
    // keeps one buffer and a barrier before the store (two buffers spill
    // there).
    constexpr int NB = D == 64 ? 2 : 1;
    __shared__ DqSmem<D, MIX, EXACT> smr[NB];

    if (a.ntiles[1] != 0) return;                    // the dS store is in use: dq_store.hip runs
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
    const int q_loc = lq0 + 32 * wave + lr;
    const bool q_valid = q_loc < L;
    const int q_row = ds + min(q_loc, L - 1);

    // query rows of Q^ and dO^ as B operands (column = query, k = channel);
    // mixed path: channels 16 kc + 8 lg .. + 8 of the query's NVFP4 values for S
    v8i qb[MIX ? 1 : KC], ob[KC];
    u32x4 qn[MIX ? NC : 1];
    {
        const uint8_t* qp = a.qc + ((long)q_row * a.hq + h) * D;
        const uint8_t* op = a.oc + ((long)q_row * a.hq + h) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            uint4 lo, hi;
            if constexpr (!MIX) {
                lo = *reinterpret_cast<const uint4*>(qp + 64 * kc + 16 * lg);
                hi = *reinterpret_cast<const uint4*>(qp + 64 * kc + 32 + 16 * lg);
                qb[kc] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
            if constexpr (!FUSED) {
                lo = *reinterpret_cast<const uint4*>(op + 64 * kc + 16 * lg);
                hi = *reinterpret_cast<const uint4*>(op + 64 * kc + 32 + 16 * lg);
                ob[kc] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
        }
        if constexpr (MIX) {
            const uint16_t* np = a.qn + ((long)q_row * a.hq + h) * D;
#pragma unroll
            for (int kc = 0; kc < NC; ++kc) qn[kc] = *reinterpret_cast<const u32x4*>(np + 16 * kc + 8 * lg);
        }
    }
    const int eq = MIX ? 127 : a.qs[(long)h * a.ttot + q_row];
    int eo;
    float nD;
    if constexpr (FUSED) {
        // the lane's dO channels: run 0 = 64 kc + 16 lg .. + 16, run 1 = 64 kc
        // + 32 + 16 lg .. + 16 (the operand's byte order); zero outside the document
        const long rowoff = ((long)q_row * a.hq + h) * D;
        float x[KC][2][16];
        float amax = 0.f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int run = 0; run < 2; ++run) {
                const uint16_t* src = a.d_o + rowoff + 64 * kc + 32 * run + 16 * lg;
                uint4 u0 = make_uint4(0, 0, 0, 0), u1 = make_uint4(0, 0, 0, 0);
                if (q_valid) {
                    u0 = *reinterpret_cast<const uint4*>(src);
                    u1 = *reinterpret_cast<const uint4*>(src + 8);
                }
                const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    x[kc][run][2 * k] = bf16_to_f32(w[k] & 0xFFFFu);
                    x[kc][run][2 * k + 1] = bf16_to_f32(w[k] >> 16);
                }
#pragma unroll
                for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(x[kc][run][k]));
            }
        // the block of the wave's 32 queries, or (exact options) the lane's
        // query: its channels lie in this lane and its partner l ^ 32
        int e;
        if constexpr (EXACT) e = block_exponent(max_xor32(amax), -127);
        else e = block_exponent_uniform(wave_max_nonneg(amax), -127);
        eo = e + 127;
        // codes = E4M3(x 2^-e); D = sum over 8-channel chunks c of the chain
        // fma(code value, O, .) in channel order, chunks summed as the
        // standalone quantizer's lane tree sums them: ((c0 + c1) + (c2 + c3)) +
        // ((c4 + c5) + (c6 + c7)) per 64 channels, then the two halves at d = 128
        float tot = 0.f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            float pr[2];
#pragma unroll
            for (int run = 0; run < 2; ++run) {
                const uint16_t* osrc = a.o + rowoff + 64 * kc + 32 * run + 16 * lg;
                const uint4 o0 = *reinterpret_cast<const uint4*>(osrc);
                const uint4 o1 = *reinterpret_cast<const uint4*>(osrc + 8);
                const uint32_t ow[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
                int cw[4];
                float chunk[2];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float* v = &x[kc][run][4 * q];
                    cw[q] = pack_fp8x4(ldexpf(v[0], -e), ldexpf(v[1], -e), ldexpf(v[2], -e), ldexpf(v[3], -e));
                }
#pragma unroll
                for (int c = 0; c < 2; ++c) {     // chunk c of the run: channels 8 c .. 8 c + 7
                    float dot = 0.f;
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(cw[2 * c + q], false);
                        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(cw[2 * c + q], true);
                        const uint32_t o01 = ow[4 * c + 2 * q], o23 = ow[4 * c + 2 * q + 1];
                        dot = fmaf(lo[0], bf16_to_f32(o01 & 0xFFFFu), dot);
                        dot = fmaf(lo[1], bf16_to_f32(o01 >> 16), dot);
                        dot = fmaf(hi[0], bf16_to_f32(o23 & 0xFFFFu), dot);
                        dot = fmaf(hi[1], bf16_to_f32(o23 >> 16), dot);
                    }
                    chunk[c] = dot;
                }
                pr[run] = chunk[0] + chunk[1];
#pragma unroll
                for (int q = 0; q < 4; ++q) ob[kc][4 * run + q] = cw[q];
                if (q_valid)
                    *reinterpret_cast<uint4*>(a.oc_w + rowoff + 64 * kc + 32 * run + 16 * lg) =
                        make_uint4((uint32_t)cw[0], (uint32_t)cw[1], (uint32_t)cw[2], (uint32_t)cw[3]);
            }
            // the partner lane (l ^ 32) holds the other chunk pair of each run
            const float half = add_xor32(pr[0]) + add_xor32(pr[1]);
            tot = kc == 0 ? half : tot + half;
        }
        const float dval = ldexpf(tot, e);
        if (q_valid && lg == 0) {
            a.os_w[(long)h * a.ttot + q_row] = (uint8_t)eo;
            a.dvec_w[(long)h * a.ttot + q_row] = -dval;   // stored as -D
        }
        nD = -dval;
    } else {
        eo = a.os[(long)h * a.ttot + q_row];
        nD = a.dvec[(long)h * a.ttot + q_row];
    }
    const float lse_raw = a.lse2[(long)h * a.ttot + q_row];
    const float lse = q_valid ? lse_raw : INFINITY;      // P = 0 on rows outside the document
    // -D as the accumulator input of the dP^T product (every register of a
    // lane belongs to the lane's query): the MFMA returns dP - D directly,
    // with the same error as a separate fp32 subtraction
    v16f negD;
#pragma unroll
    for (int i = 0; i < 16; ++i) negD[i] = nD;

    v16f acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = v16f{0};

    const int s16 = lane & 15, grp = (lane >> 4) & 1;
    const int tr_key = 8 * ((s16 >> 1) >> 2) + 4 * lg + ((s16 >> 1) & 3);
    const int tr_col = 16 * grp + 8 * (s16 & 1);

    u32x4 kr[CHUNKS / 256], vr[CHUNKS / 256], knr[NCH];
    uint32_t ekr, evr;
    auto fetch = [&](const int k0) {
        fetch_kv_tile<D>(kr, vr, ekr, evr, a.kc, a.ks, a.vc, a.vs, k0, a.ttot, a.hkv, g, tid);
        if constexpr (MIX) {
#pragma unroll
            for (int r = 0; r < NCH; ++r) {
                const int c = tid + 256 * r;
                const int row = c / (D / 8), col = (c % (D / 8)) * 8;   // col in bf16 elements
                const long krow = min(k0 + row, a.ttot - 1);
                knr[r] = *reinterpret_cast<const u32x4*>(a.kn + (krow * a.hkv + g) * D + col);
            }
        }
    };
    fetch(ds);


    // One 128-key tile; DIAG marks the last (diagonal) tile, the only one that
    // needs the causal mask and the only one with nothing left to prefetch.
    int cur = 0;                                     // buffer of the current tile
    auto tile = [&](const int t, auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        auto& sm = smr[cur];
        if constexpr (NB == 1) __syncthreads();   // every wave is past the previous tile
#pragma unroll
        for (int r = 0; r < CHUNKS / 256; ++r) {
            const int c = tid + 256 * r;
            const int row = c / (D / 16), col = (c % (D / 16)) * 16;
            *reinterpret_cast<u32x4*>(&sm.k[row * STR + col]) = kr[r];
            *reinterpret_cast<u32x4*>(&sm.v[row * STR + col]) = vr[r];
        }
        if constexpr (MIX) {
#pragma unroll
            for (int r = 0; r < NCH; ++r) {
                const int c = tid + 256 * r;
                const int row = c / (D / 8), col = (c % (D / 8)) * 16;   // col in bytes
                *reinterpret_cast<u32x4*>(&sm.kn[row * NSTR + col]) = knr[r];
            }
        }
        if (tid < kTile) {
            sm.ek[tid] = (uint8_t)ekr;
            sm.ev[tid] = (uint8_t)evr;
            if constexpr (EXACT) sm.kf[tid] = ldexpf(1.f, (int)ekr - 127);
        }
        __syncthreads();
        if constexpr (!DIAG) fetch(ds + kTile * (t + 1));

        // accumulator register i of sub-tile kk holds key 128t + 32kk + 8(i/4)
        // + 4lg + i%4; on the diagonal tile it is masked past the lane's query
        const int lim = q_loc - kTile * t - 4 * lg;
        // On the diagonal tile, sub-tiles kk > wave lie entirely after every
        // query of the wave (P = 0, dS = 0): skipped; only kk == wave needs
        // the mask.
        // S^T and dP^T of 32-key block kk (dP starts from -D)
        auto products = [&](const int kk, v16f& sb, v16f& dpb) {
            const int row = 32 * kk + lr;
            sb = v16f{0};
            dpb = negD;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                if constexpr (MIX) {
#pragma unroll
                    for (int n = 4 * kc; n < 4 * kc + 4; ++n) {
                        const u32x4 ka = *reinterpret_cast<const u32x4*>(&sm.kn[row * NSTR + 32 * n + 16 * lg]);
                        sb = mfma_bf16(ka, qn[n], sb);
                    }
                } else {
                    const uint4 lo = *reinterpret_cast<const uint4*>(&sm.k[row * STR + 64 * kc + 16 * lg]);
                    const uint4 hi = *reinterpret_cast<const uint4*>(&sm.k[row * STR + 64 * kc + 32 + 16 * lg]);
                    const v8i ka = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    sb = mfma_mx(ka, qb[kc], sb, sm.ek[row], eq);
                }
                const uint4 lo = *reinterpret_cast<const uint4*>(&sm.v[row * STR + 64 * kc + 16 * lg]);
                const uint4 hi = *reinterpret_cast<const uint4*>(&sm.v[row * STR + 64 * kc + 32 + 16 * lg]);
                const v8i va = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                dpb = mfma_mx(va, ob[kc], dpb, sm.ev[row], eo);
            }
        };
        // P, dS and the dS-hat codes of block kk (in place in dpb); `masked`:
        // the block holds the diagonal of the wave's queries
        auto softmax = [&](const int kk, const v16f& sb, v16f& dpb, int (&codes)[4], int& ebyte, bool masked) {
            if constexpr (PROBE) {
                // diagnostics: the raw scores of the probed query tile
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float* sp = probe_slot(a.probe, 1, h, ds, ds + q_loc,
                                           kTile * t + 32 * kk + 8 * (i >> 2) + 4 * lg + (i & 3));
                    if (sp) *sp = sb[i];
                }
            }
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float p = exp2_fast(fmaf(sb[i], a.c1, -lse));
                if (masked && 32 * kk + 8 * (i >> 2) + (i & 3) > lim) p = 0.f;
                dpb[i] = p * dpb[i];
                if constexpr (EXACT) {   // z = dS 2^e_j (exact scaling)
                    dpb[i] *= sm.kf[32 * kk + 8 * (i >> 2) + 4 * lg + (i & 3)];
                }
                amax = fmaxf(amax, fabsf(dpb[i]));
            }
            int e;
            if constexpr (EXACT) e = block_exponent(max_xor32(amax), -126);   // the lane's query row
            else e = block_exponent_uniform(wave_max_nonneg(amax), -126);
            ebyte = e + 127;
            const float sc = __uint_as_float((uint32_t)(e + 127) << 23);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                codes[j] = pack_fp8x4_div(dpb[4 * j], dpb[4 * j + 1], dpb[4 * j + 2], dpb[4 * j + 3], sc);
        };
        // dQ^T += K^T dS-hat^T over the 64 keys of chunk c
        auto dq_chunk = [&](const int c, const int (&c0)[4], const int (&c1)[4], int e0, int e1) {
            const v8i db = v8i{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
            const int sk = EXACT ? 127 : (int)sm.ek[64 * c + 32 * lg];
            const int sd = lg ? e1 : e0;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                v2i r[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    r[rr] = lds_read_tr8(&sm.k[(64 * c + 16 * rr + tr_key) * STR + 32 * dt + tr_col]);
                const v8i ka = v8i{r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
                acc[dt] = mfma_mx(ka, db, acc[dt], sk, sd);
            }
        };
        int dsc[4][4], es[4];
        if constexpr (!DIAG) {
            // software pipeline: the products of block kk + 1 are issued before
            // the softmax of block kk, so the matrix cores run under the VALU work
            v16f sA, dpA, sB, dpB;
            products(0, sA, dpA);
            products(1, sB, dpB);
            softmax(0, sA, dpA, dsc[0], es[0], false);
            products(2, sA, dpA);
            softmax(1, sB, dpB, dsc[1], es[1], false);
            dq_chunk(0, dsc[0], dsc[1], es[0], es[1]);
            products(3, sB, dpB);
            softmax(2, sA, dpA, dsc[2], es[2], false);
            softmax(3, sB, dpB, dsc[3], es[3], false);
            dq_chunk(1, dsc[2], dsc[3], es[2], es[3]);
        } else {
            // diagonal tile: blocks kk > wave are skipped (P = 0), block
            // kk == wave is masked
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk > wave_u) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) dsc[kk][j] = 0;
                    es[kk] = 127;
                    continue;
                }
                v16f sb, dpb;
                products(kk, sb, dpb);
                softmax(kk, sb, dpb, dsc[kk], es[kk], kk == wave_u);
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                if (2 * c > wave_u) continue;      // both blocks skipped: dS-hat = 0
                dq_chunk(c, dsc[2 * c], dsc[2 * c + 1], es[2 * c], es[2 * c + 1]);
            }
        }
        if constexpr (NB == 2) cur ^= 1;
    };
    for (int t = 0; t + 1 < ntiles; ++t) tile(t, std::false_type{});
    tile(ntiles - 1, std::true_type{});
    // ---- epilogue: dQ = softmax_scale * sum, bf16; with the Hadamard option
    // the sum is the gradient of the rotated Q and is rotated back first
    float sc = a.scale;
    if (a.hadamard) {
        hadamard_rows<DT>(acc, lg);
        sc *= inv_sqrt_d<D>();
    }
    if (q_valid) {
        uint16_t* qp = a.dq + ((long)(ds + q_loc) * a.hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t b01 = pack_bf16x2(acc[dt][4 * j] * sc, acc[dt][4 * j + 1] * sc);
                const uint32_t b23 = pack_bf16x2(acc[dt][4 * j + 2] * sc, acc[dt][4 * j + 3] * sc);
                *reinterpret_cast<uint2*>(qp + 32 * dt + 8 * j + 4 * lg) = make_uint2(b01, b23);
            }
    }
}

hipError_t launch_dq(const DqArgs& a, int d, long grid, hipStream_t st) {
    if (grid <= 0) return hipSuccess;
    const dim3 g((unsigned)grid), b(256);
    const bool fused = a.d_o != nullptr;
    if (a.probe.scores) {
        // diagnostics: the MXFP8 path (checked by the host layer)
        if (a.exact || a.qn) return hipErrorInvalidValue;
        if (d == 64) {
            if (fused) hipLaunchKernelGGL((dq_kernel<64, 0, true, 0, 1>), g, b, 0, st, a);
            else hipLaunchKernelGGL((dq_kernel<64, 0, false, 0, 1>), g, b, 0, st, a);
        } else {
            if (fused) hipLaunchKernelGGL((dq_kernel<128, 0, true, 0, 1>), g, b, 0, st, a);
            else hipLaunchKernelGGL((dq_kernel<128, 0, false, 0, 1>), g, b, 0, st, a);
        }
        return hipGetLastError();
    }
    if (a.exact) {
        if (!fused || a.qn) return hipErrorInvalidValue;
        if (d == 64) hipLaunchKernelGGL((dq_kernel<64, 0, true, 1>), g, b, 0, st, a);
        else hipLaunchKernelGGL((dq_kernel<128, 0, true, 1>), g, b, 0, st, a);
        return hipGetLastError();
    }
    if (d == 64) {
        if (a.qn) {
            if (fused) hipLaunchKernelGGL((dq_kernel<64, 1, true, 0>), g, b, 0, st, a);
            else hipLaunchKernelGGL((dq_kernel<64, 1, false, 0>), g, b, 0, st, a);
        } else {
            if (fused) hipLaunchKernelGGL((dq_kernel<64, 0, true, 0>), g, b, 0, st, a);
            else hipLaunchKernelGGL((dq_kernel<64, 0, false, 0>), g, b, 0, st, a);
        }
    } else {
        if (a.qn) {
            if (fused) hipLaunchKernelGGL((dq_kernel<128, 1, true, 0>), g, b, 0, st, a);
            else hipLaunchKernelGGL((dq_kernel<128, 1, false, 0>), g, b, 0, st, a);
        } else {
            if (fused) hipLaunchKernelGGL((dq_kernel<128, 0, true, 0>), g, b, 0, st, a);
            else hipLaunchKernelGGL((dq_kernel<128, 0, false, 0>), g, b, 0, st, a);
        }
    }
    return hipGetLastError();
}

}  // namespace flamia
