// Key-major dK/dV pass of the causal backward at head dimension 128 (FLAMIA
// paper: Section 2 equations dV = P^T dO, dP = dO V^T, dS = P o (dP - D),
// dK = dS^T Q; Section 3.3 consistency with the forward; Appendix B.1 dV
// operand E4M3(2^8 P)).  The arithmetic is that of the d = 64 kernel in
// bwd.hip, value for value; only the division of the work differs.
//
// At d = 128 a wave that owns 32 keys holds their dK and dV accumulators over
// all 128 channels (128 registers) next to its S and dP tiles, which leaves
// one wave per SIMD and the latencies exposed.  Here a workgroup has eight
// waves and waves w and w + 4 share keys 32w .. 32w + 31 of the 128-key tile:
// for each 64-query step, wave half hf = wave / 4
//   - computes S, dP, P, P-hat_b, dS and the dS-hat block of queries
//     32 hf .. 32 hf + 31 (one 32x32 block: its exponent needs no exchange),
//   - writes its P-hat_b and dS-hat codes and the block exponent to LDS, and
//     after a barrier reads its partner's,
//   - accumulates dV and dK for channels 64 hf .. 64 hf + 63 over all 64
//     queries (the MFMA contracts over the two blocks at once).
// With half the accumulators a wave fits two per SIMD.  The Hadamard
// back-rotation of dK runs channel bits 0-5 inside the wave and bit 6 across
// the pair through LDS, in the same order as the unsplit kernel.
// Exact options (Appendix A.3): the same folds as the d = 64 kernel (dO's
// token exponent into P-hat_b relative to its 32-query block maximum, Q's
// into dS).
#include <atomic>
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace flamia {

namespace {

constexpr int kSD = 128;                  // head dimension of this kernel
constexpr int kSStep = 64;                // queries per step

template <int MIX, int EXACT>
struct SplitStep {
    static constexpr int kStride = kSD + 16;       // row pitch of code tiles
    static constexpr int kNStride = 2 * kSD + 16;  // row pitch of the bf16 NVFP4 rows (mixed path)
    uint8_t q[kSStep * kStride];
    uint8_t o[kSStep * kStride];                    // quantized dO
    alignas(16) float lse[kSStep];
    alignas(16) float dv[kSStep];                   // -D
    uint8_t eq[kSStep];
    uint8_t eo[kSStep];
    alignas(16) uint8_t qn[MIX ? kSStep * kNStride : 16];
    // exact options: per query 2^(e_o - E_o) and 2^e_q; E_o per 32-query block
    alignas(16) float fo[EXACT ? kSStep : 4];
    alignas(16) float fq[EXACT ? kSStep : 4];
    uint8_t eob[4];
};

// Codes a wave hands to its partner each step: per lane 4 words of P-hat_b
// and 4 of dS-hat (the lane's accumulator registers), plus the block exponent.
struct SplitXchg {
    u32x4 pb[8][64];
    u32x4 db[8][64];
    int es[8];
};

template <int MIX, int EXACT>
struct SplitSmem {
    union {
        struct {
            SplitStep<MIX, EXACT> buf[2];   // ring: step i fills buffer i % 2
            SplitXchg x;
        } loop;
        float rot[4][2][16][64];     // epilogue: dK tiles of the waves 4 .. 7 or 0 .. 3
    };
};

// Step buffer of the direct-LDS staging (the MXFP8 variants): the loads
// write LDS 16 bytes per lane in lane order, so rows are unpadded and
// 16-byte chunk c of row r sits at chunk c ^ ((r ^ (r >> 1)) & 7) (no bank
// conflicts for the row and transposed reads); scale bytes arrive
// zero-extended to dwords.
struct SplitStepDma {
    static constexpr int kStride = kSD;
    static constexpr int kNStride = 0;
    alignas(16) uint8_t q[kSStep * kSD];
    alignas(16) uint8_t o[kSStep * kSD];            // quantized dO
    alignas(16) float lse[kSStep];
    alignas(16) float dv[kSStep];                   // -D
    uint32_t eq[kSStep];
    uint32_t eo[kSStep];
};

// Ring of three steps and two exchange buffers, one barrier per step (after
// the exchange writes).  Step k is fetched right after the barrier of step
// k - 2 into the buffer of step k - 3, whose last reads (its dV/dK products,
// after the barrier of step k - 3) every wave finished before the barrier of
// step k - 2; each wave waits for its own loads of step k before the barrier
// of step k - 1, after which step k's products start.  Step i writes its
// codes into exchange buffer i % 2, read by the partner after the barrier of
// step i; the next write to it (step i + 2) comes after the barrier of step
// i + 1.
struct SplitSmemDma {
    union {
        struct {
            SplitStepDma buf[3];
            SplitXchg x[2];
        } loop;
        float rot[4][2][16][64];
    };
};

}  // namespace

// PROBE = 1: the diagnostics instantiation (probed raw scores, dS-hat zero count).
template <bool STORE, int MIX, int EXACT, int PROBE = 0>
__global__ void __launch_bounds__(512, 1) bwd_split_kernel(const BwdArgs a) {
    constexpr int D = kSD;
    constexpr int KC = D / 64;
    constexpr int NC = D / 16;
    constexpr int DTH = 2;                        // 32-channel tiles of dK / dV per wave
    using Step = std::conditional_t<!MIX && !EXACT, SplitStepDma, SplitStep<MIX, EXACT>>;
    constexpr int STR = Step::kStride;
    constexpr int NSTR = Step::kNStride;
    static_assert(!EXACT || (!STORE && !MIX), "the exact options run without the store, on MXFP8");
    constexpr int NQ = kSStep * D / 16 / 512;     // 16-byte chunks per thread of a 64-row code tile
    constexpr int NQN = MIX ? 2 * NQ : 1;
    // Steps staged by direct LDS loads one step ahead with one barrier per
    // step (MXFP8); the mixed path and the exact options load a step into
    // registers and store it behind a second barrier.
    constexpr bool DMA = !MIX && !EXACT;
    __shared__ std::conditional_t<DMA, SplitSmemDma, SplitSmem<MIX, EXACT>> sm;
    // byte offset of (row, col) in a staged code tile
    auto toff = [](int row, int col) -> int {
        if constexpr (DMA) return row * D + ((((col >> 4) ^ row ^ (row >> 1)) & 7) << 4) + (col & 15);
        else return row * STR + col;
    };

    // Persistent workgroups: one per CU (an eight-wave workgroup fills a CU's
    // registers).  Workgroup b takes item b of the cost-ordered list first,
    // then the next unclaimed one from a work queue (a counter the work-list
    // kernel zeroes), as the hardware dispatcher would hand out workgroups,
    // but without relaunching one per item: that left the CU idle between
    // items (thousands of cycles each, measured), since no second workgroup
    // fits to cover the gap.  The next item is claimed during the current
    // one's last step, which hides the atomic's latency; claiming at the start
    // held a claimed item behind a long current one (30% slower where a few
    // long items set the time).  Every workgroup leaves the loop once the
    // counter passes the item count.  The mixed path's
    // variant keeps one workgroup per item: the loop's extra live registers
    // make it spill (8% slower).
    constexpr bool PERSIST = !MIX;
    __shared__ int next_item;
    const int nitems = *a.ntiles * a.hkv;
    int item = (int)blockIdx.x;
    unsigned nzero = 0;     // diagnostics: nonzero dS entries whose dS-hat code is zero
    while (item < nitems) {
    int claim = 0;   // the next item, claimed during this item's last step
    const int ti = item / a.hkv;
    const int4 it = a.tiles[ti];
    const int k0 = it.x, ds = it.y, de = it.z, doc = it.w;
    const int g = item - ti * a.hkv;
    const bool use_store = STORE && a.ntiles[1] != 0;
    const long doc_blk = use_store ? (long)a.dboff[doc] : 0;
    const int G = a.hq / a.hkv;
    const int L = de - ds;
    const int kt0 = k0 - ds;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int kw = wave_u & 3;                    // key group of the pair
    const int hf = wave_u >> 2;                   // query block of S / channel half of dK, dV
    const int lg = lane >> 5, lr = lane & 31;
    const int key_loc = kt0 + 32 * kw + lr;
    const bool key_valid = key_loc < L;
    const int key_row = ds + min(key_loc, L - 1);

    // ---- staging of one 64-query step (prefetched into registers one step ahead)
    u32x4 pq[NQ], po[NQ], pqn[NQN];
    uint32_t p_eq = 0, p_eo = 0;
    float p_lse = 0.f, p_dv = 0.f;
    bool p_in = true;
    auto load_step = [&](int h, int q0) {
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            const int c = tid + 512 * r;
            const int row = c / (D / 16), col = (c % (D / 16)) * 16;
            const long qr = ds + min(q0 + row, L - 1);
            pq[r] = *reinterpret_cast<const u32x4*>(a.qc + (qr * a.hq + h) * D + col);
            po[r] = *reinterpret_cast<const u32x4*>(a.oc + (qr * a.hq + h) * D + col);
        }
        if constexpr (MIX) {
#pragma unroll
            for (int r = 0; r < NQN; ++r) {
                const int c = tid + 512 * r;
                const int row = c / (D / 8), col = (c % (D / 8)) * 8;   // col in bf16 elements
                const long qr = ds + min(q0 + row, L - 1);
                pqn[r] = *reinterpret_cast<const u32x4*>(a.qn + (qr * a.hq + h) * D + col);
            }
        }
        const int ql = q0 + (tid & (kSStep - 1));
        const long qr = ds + min(ql, L - 1);
        p_eq = a.qs[(long)h * a.ttot + qr];
        p_eo = a.os[(long)h * a.ttot + qr];
        p_lse = a.lse2[(long)h * a.ttot + qr];
        p_in = ql < L;
        p_dv = a.dvec[(long)h * a.ttot + qr];
    };
    auto store_step = [&](Step& b) {
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            const int c = tid + 512 * r;
            const int row = c / (D / 16), col = (c % (D / 16)) * 16;
            *reinterpret_cast<u32x4*>(&b.q[row * STR + col]) = pq[r];
            *reinterpret_cast<u32x4*>(&b.o[row * STR + col]) = po[r];
        }
        if constexpr (MIX) {
#pragma unroll
            for (int r = 0; r < NQN; ++r) {
                const int c = tid + 512 * r;
                const int row = c / (D / 8), col = (c % (D / 8)) * 16;   // col in bytes
                *reinterpret_cast<u32x4*>(&b.qn[row * NSTR + col]) = pqn[r];
            }
        }
        if (tid < kSStep) {
            b.eq[tid] = (uint8_t)p_eq;
            b.eo[tid] = (uint8_t)p_eo;
            b.lse[tid] = p_in ? p_lse : INFINITY;   // +inf: row outside the document
            b.dv[tid] = p_dv;                        // -D: accumulator input of dP
        }
        if constexpr (EXACT) {
            // thread tid holds query tid % 64: each half-wave one 32-query block
            const uint32_t eb = halfwave_max(p_eo);
            if (tid < kSStep) {
                b.fo[tid] = ldexpf(1.f, (int)p_eo - (int)eb);
                b.fq[tid] = ldexpf(1.f, (int)p_eq - 127);
                if ((tid & 31) == 0) b.eob[tid >> 5] = (uint8_t)eb;
            }
        }
    };
    // Direct staging: wave w fetches rows 8w .. 8w + 7 of both code tiles
    // (lane l: row 8w + l / 8 into physical chunk l % 8) and waves 0 .. 3 one
    // per-query array each: lse2, -D, Q's and dO's scale bytes.  Rows past
    // the end of the document read zeros: a zero Q and dO row with lse2 =
    // D = 0 has S = dP = dS = 0 and P = 1 against a zero dO row, so it adds
    // nothing to dK or dV.
    auto issue_step = [&](auto& b, int h, int q0) {
        const int row = 8 * wave_u + (lane >> 3);
        const int c = (lane & 7) ^ ((row ^ (row >> 1)) & 7);
        const bool in = q0 + row < L;
        const long off = ((long)(ds + q0 + row) * a.hq + h) * D + 16 * c;
        dma16(in ? (const void*)(a.qc + off) : (const void*)a.zero, &b.q[8 * D * wave_u]);
        dma16(in ? (const void*)(a.oc + off) : (const void*)a.zero, &b.o[8 * D * wave_u]);
        if (wave_u < 4) {
            const bool vin = q0 + lane < L;
            const long vo = (long)h * a.ttot + ds + q0 + lane;
            if (wave_u == 0) dma4(vin ? (const void*)(a.lse2 + vo) : (const void*)a.zero, b.lse);
            else if (wave_u == 1) dma4(vin ? (const void*)(a.dvec + vo) : (const void*)a.zero, b.dv);
            else if (wave_u == 2) dma1(vin ? (const void*)(a.qs + vo) : (const void*)a.zero, b.eq);
            else dma1(vin ? (const void*)(a.os + vo) : (const void*)a.zero, b.eo);
        }
    };
    if constexpr (DMA) issue_step(sm.loop.buf[0], g * G, kt0);
    else load_step(g * G, kt0);

    // The pair's key rows as B operands of S and dP (column = key, k = channel)
    v8i kb[MIX ? 1 : KC], vb[KC];
    u32x4 kn[MIX ? NC : 1];
    {
        const uint8_t* kp = a.kc + ((long)key_row * a.hkv + g) * D;
        const uint8_t* vp = a.vc + ((long)key_row * a.hkv + g) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            uint4 lo, hi;
            if constexpr (!MIX) {
                lo = *reinterpret_cast<const uint4*>(kp + 64 * kc + 16 * lg);
                hi = *reinterpret_cast<const uint4*>(kp + 64 * kc + 32 + 16 * lg);
                kb[kc] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
            lo = *reinterpret_cast<const uint4*>(vp + 64 * kc + 16 * lg);
            hi = *reinterpret_cast<const uint4*>(vp + 64 * kc + 32 + 16 * lg);
            vb[kc] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        if constexpr (MIX) {
            const uint16_t* np = a.kn + ((long)key_row * a.hkv + g) * D;
#pragma unroll
            for (int kc = 0; kc < NC; ++kc) kn[kc] = *reinterpret_cast<const u32x4*>(np + 16 * kc + 8 * lg);
        }
    }
    const int ek = MIX ? 127 : a.ks[(long)g * a.ttot + key_row];
    const int ev = a.vs[(long)g * a.ttot + key_row];

    v16f dvt[DTH], dkt[DTH];                      // channel tiles 2 hf, 2 hf + 1
#pragma unroll
    for (int t = 0; t < DTH; ++t) { dvt[t] = v16f{0}; dkt[t] = v16f{0}; }

    const int s16 = lane & 15, grp = (lane >> 4) & 1;
    const int tr_key = 8 * ((s16 >> 1) >> 2) + 4 * lg + ((s16 >> 1) & 3);
    const int tr_col = 16 * grp + 8 * (s16 & 1);
    const float inv256 = 1.f / 256.f;

    int cur = 0;
    int xi = 0;                   // exchange buffer of the current step (direct staging)
    int hh = 0, q0 = kt0;
    int lh = 0, lq0 = kt0;        // next step to fetch (direct staging)
    bool lmore = true;
    auto advance = [&](int& hx, int& qx) {
        qx += kSStep;
        if (qx >= L) { qx = kt0; ++hx; }
    };
    if constexpr (DMA) {
        // the key rows and scales are in registers before the next loads go out
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            keep_loaded(kb[kc]);
            keep_loaded(vb[kc]);
        }
        keep_loaded(ek);
        keep_loaded(ev);
        // the first step's loads, then the second step's
        vm_drain_barrier();
        advance(lh, lq0);
        lmore = lh < G;
        if (lmore) {
            issue_step(sm.loop.buf[1], g * G + lh, lq0);
            advance(lh, lq0);
            lmore = lh < G;
        }
    }
    // this wave's dS block of the previous step, stored at the start of the next one
    u32x4 pend_w = u32x4{0, 0, 0, 0};
    long pend_blk = 0;
    int pend_e = 127;
    bool pend_ok = false;
    auto flush_store = [&]() {
        if (!use_store || !pend_ok) return;
        *reinterpret_cast<u32x4*>(a.ds_codes + pend_blk * kDsBlockBytes + 16 * lane) = pend_w;
        if (lane == 0) a.ds_scales[pend_blk] = (uint8_t)pend_e;
        pend_ok = false;
    };
    // One 64-query step; MASK marks the steps that meet the causal boundary
    // (the first two of every head, starting at the diagonal).
    auto step = [&](auto mask_tag) -> bool {
        constexpr bool MASK = decltype(mask_tag)::value;
        Step& B = sm.loop.buf[cur];
        if constexpr (!DMA) {
            store_step(B);
            __syncthreads();
        }
        const int h = g * G + hh;
        const int qs0 = q0;
        advance(hh, q0);
        const bool more = hh < G;
        if (PERSIST && !more && threadIdx.x == 0) claim = (int)gridDim.x + atomicAdd(a.queue, 1);
        flush_store();
        if constexpr (!DMA) load_step(g * G + min(hh, G - 1), q0);

        // the step's 32-query blocks are blocks qb0 and qb0 + 1 of the key
        // tile's diagonal: a block before the pair's keys is skipped (P = 0),
        // the block on it is masked
        const int qb0 = (qs0 - kt0) >> 5;
        const bool skip = MASK && qb0 + hf < kw;
        const bool part = MASK && qb0 + hf == kw;
        const bool skip1 = MASK && qb0 + 1 < kw;  // the step's second block skipped: both are
        int pbc[4] = {0, 0, 0, 0}, dsc[4] = {0, 0, 0, 0}, es = 127;
        if (!skip) {
            // ---- S and dP for the pair's 32 keys x the wave's 32 queries
            const int row = 32 * hf + lr;
            v16f sacc = v16f{0}, pacc;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 d4 = *reinterpret_cast<const float4*>(&B.dv[32 * hf + 8 * j + 4 * lg]);
                pacc[4 * j] = d4.x;
                pacc[4 * j + 1] = d4.y;
                pacc[4 * j + 2] = d4.z;
                pacc[4 * j + 3] = d4.w;
            }
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                if constexpr (MIX) {
#pragma unroll
                    for (int n = 4 * kc; n < 4 * kc + 4; ++n) {
                        const u32x4 qa = *reinterpret_cast<const u32x4*>(&B.qn[row * NSTR + 32 * n + 16 * lg]);
                        sacc = mfma_bf16(qa, kn[n], sacc);
                    }
                } else {
                    const uint4 lo = *reinterpret_cast<const uint4*>(&B.q[toff(row, 64 * kc + 16 * lg)]);
                    const uint4 hi = *reinterpret_cast<const uint4*>(&B.q[toff(row, 64 * kc + 32 + 16 * lg)]);
                    const v8i qa = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    sacc = mfma_mx(qa, kb[kc], sacc, B.eq[row], ek);
                }
                const uint4 lo = *reinterpret_cast<const uint4*>(&B.o[toff(row, 64 * kc + 16 * lg)]);
                const uint4 hi = *reinterpret_cast<const uint4*>(&B.o[toff(row, 64 * kc + 32 + 16 * lg)]);
                const v8i oa = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                pacc = mfma_mx(oa, vb[kc], pacc, B.eo[row], ev);
            }
            // ---- P, P-hat_b, dS, dS-hat; register i = 4j + r holds query
            // qs0 + 32 hf + 8j + 4lg + r, masked while the key lies after it
            const int lim = key_loc - qs0 - 32 * hf - 4 * lg;
            if constexpr (PROBE) {
                // diagnostics: the raw scores of the probed query tile
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float* sp = probe_slot(a.probe, 2, h, ds, ds + qs0 + 32 * hf + 8 * (i >> 2) + 4 * lg + (i & 3),
                                           key_loc);
                    if (sp) *sp = sacc[i];
                }
            }
            float amax = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int q4 = 32 * hf + 8 * j + 4 * lg;
                const float4 l4 = *reinterpret_cast<const float4*>(&B.lse[q4]);
                const float lq[4] = {l4.x, l4.y, l4.z, l4.w};
                float fo[4] = {1.f, 1.f, 1.f, 1.f}, fq[4] = {1.f, 1.f, 1.f, 1.f};
                if constexpr (EXACT) {
                    const float4 o4 = *reinterpret_cast<const float4*>(&B.fo[q4]);
                    const float4 g4 = *reinterpret_cast<const float4*>(&B.fq[q4]);
                    fo[0] = o4.x; fo[1] = o4.y; fo[2] = o4.z; fo[3] = o4.w;
                    fq[0] = g4.x; fq[1] = g4.y; fq[2] = g4.z; fq[3] = g4.w;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * j + r;
                    float p = exp2_fast(fmaf(sacc[i], a.c1, -lq[r]));
                    if (part)
                        if (8 * j + r < lim) p = 0.f;
                    // exact options: the folds are exact power-of-two scalings
                    sacc[i] = EXACT ? p * fo[r] : p;
                    pacc[i] = p * pacc[i];
                    if constexpr (EXACT) pacc[i] *= fq[r];
                    amax = fmaxf(amax, fabsf(pacc[i]));
                }
            }
            amax = wave_max_nonneg(amax);
            const int e = block_exponent_uniform(amax, -126);
            es = e + 127;
            const float sc = __uint_as_float((uint32_t)(e + 127) << 23);   // 2^e
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pbc[j] = pack_fp8x4_div(sacc[4 * j], sacc[4 * j + 1], sacc[4 * j + 2], sacc[4 * j + 3], inv256);
                dsc[j] = pack_fp8x4_div(pacc[4 * j], pacc[4 * j + 1], pacc[4 * j + 2], pacc[4 * j + 3], sc);
            }
            if constexpr (PROBE) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    nzero += (pacc[i] != 0.f && ((((uint32_t)dsc[i >> 2] >> (8 * (i & 3))) & 0x7Fu) == 0u)) ? 1u : 0u;
            }
        }
        // ---- dS store: this wave's block (qb, kb) as [query half][32 keys][16 queries]
        if (use_store) {
            const int qb = (qs0 >> 5) + hf, kb = (kt0 >> 5) + kw;
            pend_ok = !skip && qs0 + 32 * hf < L;
            pend_blk = (long)h * a.ds_blocks + doc_blk + (long)qb * (qb + 1) / 2 + kb;
            const auto x02 = __builtin_amdgcn_permlane32_swap(dsc[0], dsc[2], false, false);
            const auto x13 = __builtin_amdgcn_permlane32_swap(dsc[1], dsc[3], false, false);
            pend_w = u32x4{(uint32_t)x02[0], (uint32_t)x02[1], (uint32_t)x13[0], (uint32_t)x13[1]};
            pend_e = es;
        }
        // ---- exchange with the partner wave, then dV^T += dO^T P-hat_b and
        // dK^T += Q^T dS-hat for the wave's channel half over the 64 queries
        SplitXchg& X = [&]() -> SplitXchg& {
            if constexpr (DMA) return sm.loop.x[xi];
            else return sm.loop.x;
        }();
        X.pb[wave_u][lane] = u32x4{(uint32_t)pbc[0], (uint32_t)pbc[1], (uint32_t)pbc[2], (uint32_t)pbc[3]};
        X.db[wave_u][lane] = u32x4{(uint32_t)dsc[0], (uint32_t)dsc[1], (uint32_t)dsc[2], (uint32_t)dsc[3]};
        if (lane == 0) X.es[wave_u] = es;
        if constexpr (DMA) {
            // the exchange, and this wave's loads of the next step; then fetch
            // the step after it
            vm_drain_barrier();
            if (lmore) {
                issue_step(sm.loop.buf[cur == 0 ? 2 : cur - 1], g * G + lh, lq0);
                advance(lh, lq0);
                lmore = lh < G;
            }
        } else {
            __syncthreads();
        }
        if (!skip1) {
            const int pw = wave_u ^ 4;
            const u32x4 ppb = X.pb[pw][lane], pdb = X.db[pw][lane];
            const int pes = X.es[pw];
            // block 0 of the contraction is wave half 0's, block 1 wave half 1's
            const u32x4 b0 = hf ? ppb : u32x4{(uint32_t)pbc[0], (uint32_t)pbc[1], (uint32_t)pbc[2], (uint32_t)pbc[3]};
            const u32x4 b1 = hf ? u32x4{(uint32_t)pbc[0], (uint32_t)pbc[1], (uint32_t)pbc[2], (uint32_t)pbc[3]} : ppb;
            const u32x4 d0 = hf ? pdb : u32x4{(uint32_t)dsc[0], (uint32_t)dsc[1], (uint32_t)dsc[2], (uint32_t)dsc[3]};
            const u32x4 d1 = hf ? u32x4{(uint32_t)dsc[0], (uint32_t)dsc[1], (uint32_t)dsc[2], (uint32_t)dsc[3]} : pdb;
            const v8i pb = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
            const v8i db = v8i{(int)d0.x, (int)d0.y, (int)d0.z, (int)d0.w, (int)d1.x, (int)d1.y, (int)d1.z, (int)d1.w};
            const int e0 = hf ? pes : es, e1 = hf ? es : pes;
            // A scales: dO's and Q's token blocks, or (exact options) dO's
            // block maximum and 1 (Q's exponents are inside dS-hat)
            int so, sq;
            if constexpr (EXACT) {
                so = B.eob[lg];
                sq = 127;
            } else {
                so = B.eo[32 * lg];
                sq = B.eq[32 * lg];
            }
            const int sd = lg ? e1 : e0;
#pragma unroll
            for (int t = 0; t < DTH; ++t) {
                const int dt = 2 * hf + t;
                v2i r[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    r[rr] = lds_read_tr8(&B.o[toff(16 * rr + tr_key, 32 * dt + tr_col)]);
                const v8i oa = v8i{r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
                dvt[t] = mfma_mx(oa, pb, dvt[t], so, 127 - 8);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    r[rr] = lds_read_tr8(&B.q[toff(16 * rr + tr_key, 32 * dt + tr_col)]);
                const v8i qa = v8i{r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
                dkt[t] = mfma_mx(qa, db, dkt[t], sq, sd);
            }
        }
        if constexpr (DMA) {
            cur = cur == 2 ? 0 : cur + 1;
            xi ^= 1;
        } else {
            cur ^= 1;
        }
        return more;
    };
    bool more = true;
    while (more) {
        while (more && q0 < kt0 + kTile) more = step(std::true_type{});
        while (more && q0 >= kt0 + kTile) more = step(std::false_type{});
    }
    flush_store();
    // ---- epilogue: dK = softmax_scale * sum (rotated back with the Hadamard
    // option: channel bits 0-5 in the wave, bit 6 with the partner), dV
    float sck = a.scale;
    if (a.hadamard) {
        hadamard_rows<DTH>(dkt, lg);
        sck *= inv_sqrt_d<D>();
        // channel bit 6: (x_lo, x_hi) -> (x_lo + x_hi, x_lo - x_hi); wave half
        // 0 holds x_lo, half 1 x_hi.  The loop's buffers are no longer read
        // once every wave is past this barrier.
        __syncthreads();
        float (&rt)[4][2][16][64] = sm.rot;
        if (hf == 1)
#pragma unroll
            for (int t = 0; t < DTH; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) rt[kw][t][i][lane] = dkt[t][i];
        __syncthreads();
        v16f hi_in[DTH];
        if (hf == 0) {
#pragma unroll
            for (int t = 0; t < DTH; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) hi_in[t][i] = rt[kw][t][i][lane];
        }
        __syncthreads();
        if (hf == 0)
#pragma unroll
            for (int t = 0; t < DTH; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) rt[kw][t][i][lane] = dkt[t][i];
        __syncthreads();
#pragma unroll
        for (int t = 0; t < DTH; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (hf == 0) {
                    dkt[t][i] = dkt[t][i] + hi_in[t][i];
                } else {
                    const float lo = rt[kw][t][i][lane];
                    dkt[t][i] = lo - dkt[t][i];
                }
            }
    }
    if (key_valid) {
        uint16_t* kp = a.dk + ((long)(ds + key_loc) * a.hkv + g) * D;
        uint16_t* vp = a.dv + ((long)(ds + key_loc) * a.hkv + g) * D;
#pragma unroll
        for (int t = 0; t < DTH; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int dd = 32 * (2 * hf + t) + 8 * j + 4 * lg;
                *reinterpret_cast<uint2*>(kp + dd) = make_uint2(
                    pack_bf16x2(dkt[t][4 * j] * sck, dkt[t][4 * j + 1] * sck),
                    pack_bf16x2(dkt[t][4 * j + 2] * sck, dkt[t][4 * j + 3] * sck));
                *reinterpret_cast<uint2*>(vp + dd) = make_uint2(
                    pack_bf16x2(dvt[t][4 * j], dvt[t][4 * j + 1]),
                    pack_bf16x2(dvt[t][4 * j + 2], dvt[t][4 * j + 3]));
            }
    }
    if constexpr (!PERSIST) break;
    // hand the claimed item to every wave; past this barrier the item's step
    // buffers and epilogue tiles are read no more
    if (threadIdx.x == 0) next_item = claim;
    __syncthreads();
    item = next_item;
    }   // work items
    if constexpr (PROBE) {
        const unsigned n = wave_sum_u32(nzero);
        if (a.probe.ds_zero && (threadIdx.x & 63) == 0 && n) atomicAdd(a.probe.ds_zero, (unsigned long long)n);
    }
}

hipError_t device_cus(int* n) {
    // the current device's CU count, read once per device (host threads may
    // race to fill an entry; they store the same value)
    static std::atomic<int> cus[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    int c = cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int v = 0;
        e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        c = v > 0 ? v : 1;
        cus[dev].store(c, std::memory_order_relaxed);
    }
    *n = c;
    return hipSuccess;
}

hipError_t launch_bwd_split(const BwdArgs& a, long grid, hipStream_t st) {
    if (grid <= 0) return hipSuccess;
    const bool store = a.ds_blocks > 0;
    // persistent: at most one workgroup per CU (grid = the item capacity
    // otherwise)
    int cus = 0;
    const hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    const long pgrid = (a.qn || grid < cus) ? grid : cus;
    const dim3 g((unsigned)pgrid), b(512);
    if (a.exact) {
        if (store || a.qn) return hipErrorInvalidValue;
        hipLaunchKernelGGL((bwd_split_kernel<false, 0, 1>), g, b, 0, st, a);
    } else if (a.probe.scores || a.probe.ds_zero) {
        // diagnostics: the MXFP8 path (checked by the host layer)
        if (a.qn) return hipErrorInvalidValue;
        if (store) hipLaunchKernelGGL((bwd_split_kernel<true, 0, 0, 1>), g, b, 0, st, a);
        else hipLaunchKernelGGL((bwd_split_kernel<false, 0, 0, 1>), g, b, 0, st, a);
    } else if (a.qn) {
        if (store) hipLaunchKernelGGL((bwd_split_kernel<true, 1, 0>), g, b, 0, st, a);
        else hipLaunchKernelGGL((bwd_split_kernel<false, 1, 0>), g, b, 0, st, a);
    } else {
        if (store) hipLaunchKernelGGL((bwd_split_kernel<true, 0, 0>), g, b, 0, st, a);
        else hipLaunchKernelGGL((bwd_split_kernel<false, 0, 0>), g, b, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace flamia
