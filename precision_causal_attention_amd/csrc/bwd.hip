// MXFP8 causal backward over packed documents (FLAMIA paper: Section 2
// equations dV = P^T dO, dP = dO V^T, dS = P o (dP - D), dQ = dS K,
// dK = dS^T Q; Section 3.3: scores rebuilt from the forward's quantized Q/K
// with the same tiling, masking and exponential, P from the saved row
// statistic, dS quantized on 32x32 document-local blocks from the block
// maximum; Appendix B.1: the dV operand is E4M3(2^8 P) with no stored scale).
//
// Key-major dK/dV pass at d = 64 (d = 128: bwd_split.hip, same arithmetic in
// wave pairs).  One workgroup = one work item (document,
// key/value head, 128-key tile anchored at the document start); wave w owns
// keys 32w..32w+31 of the tile.  For every 64-query step, from the end of the
// document down to the diagonal, and every query head of the group (heads
// innermost; with the document-major work list the key tiles of a document
// run together and read the same query rows at the same time, so those rows
// come from L2: 4x less HBM traffic than sweeping each head upwards from the
// tile's own diagonal):
//   S  [query][key] = Q^ K^T    A = query rows (LDS), B = the wave's key rows (registers)
//   dP [query][key] = dO^ V^T   same structure; both bitwise equal to the
//                               forward's S^T (role-swapped operands give identical
//                               accumulator bits on this hardware)
//   P = 2^(x - lse2), P-hat_b = E4M3(2^8 P), dS = P (dP - D) (the dP product
//   starts from -D)
//   dS-hat: one exponent per 32x32 block = one accumulator tile (block max via
//   a wave reduction):
//   dV^T += dO^T P-hat_b   (A = dO^T by transposed LDS read, B = accumulator bytes)
//   dK^T += Q^T dS-hat     (A = Q^T by transposed LDS read, B = accumulator bytes)
// dK and dV accumulate in registers across the query heads of the group
// (GQA sum in fp32) and are written once.  dQ is the query-major pass
// (dq.hip), which rebuilds the same dS-hat bit for bit.
// Mixed NVFP4/FP8 path (Section 3.4): S is rebuilt from the NVFP4 values of Q
// and K (bf16, D/16 bf16 MFMAs per 32x32 tile, the forward's instruction with
// the roles swapped, which gives the same bits); dK still contracts over the
// E4M3 token-block Q^, so a step stages both forms of its query rows.
// Exact options (Appendix A.3): Q and dO carry one exponent per query.  S and
// dP apply them per lane as before; dV and dK contract over queries, so dO's
// exponent moves into P-hat_b relative to the largest of its 32-query block
// (E4M3(2^8 P 2^(e_o - E_o)), A scale 2^E_o) and Q's into dS (dS 2^e_q, one
// exponent per 32x32 block as before, A scale 1).
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace flamia {

constexpr int kQStep = 64;

template <int D, int MIX, int EXACT = 0>
struct BwdStep {
    static constexpr int kStride = D + 16;       // row pitch of code tiles
    static constexpr int kNStride = 2 * D + 16;  // row pitch of the bf16 NVFP4 rows (mixed path)
    uint8_t q[kQStep * kStride];
    uint8_t o[kQStep * kStride];                 // quantized dO
    alignas(16) float lse[kQStep];
    alignas(16) float dv[kQStep];                // -D
    uint8_t eq[kQStep];
    uint8_t eo[kQStep];
    alignas(16) uint8_t qn[MIX ? kQStep * kNStride : 16];   // NVFP4 values of Q (mixed path)
    // exact options: per query 2^(e_o - E_o) and 2^e_q; E_o per 32-query block
    alignas(16) float fo[EXACT ? kQStep : 4];
    alignas(16) float fq[EXACT ? kQStep : 4];
    uint8_t eob[4];
};


// Step buffer of the LDS DMA staging (MXFP8 pipeline without the dS store):
// the loads write LDS directly, 16 bytes per lane in lane order, so the code
// tiles have unpadded rows and bank conflicts are avoided by placing 16-byte
// chunk c of row r at chunk c ^ ((r >> 2) & 3) instead; the scale bytes
// arrive zero-extended to dwords.
template <int D>
struct BwdStepDma {
    static constexpr int kStride = D;
    static constexpr int kNStride = 0;
    uint8_t q[kQStep * D];
    uint8_t o[kQStep * D];                       // quantized dO
    alignas(16) float lse[kQStep];
    alignas(16) float dv[kQStep];                // -D
    uint32_t eq[kQStep];
    uint32_t eo[kQStep];
};

// A ring of step buffers, so that a step fills its buffer without waiting.
// Register staging: step i is stored into buffer i % N at its start, after
// the barrier of step i - 1; the buffer was last read by the products of
// step i - N and, with the software pipeline (N = 3), by the dV/dK products
// of that step issued in step i - N + 1, and every wave is past both before
// it reaches that barrier.  LDS DMA staging (N = 6): steps go in pairs with
// one barrier per pair, at its first step; pair j + 1 is fetched right after
// the barrier of pair j (two steps ahead) into the buffers of pair j - 2,
// last read by that pair's products and, pipelined, in the first step of
// pair j - 1.
template <class S, int N>
struct StepRing {
    S buf[N];
};

// PROBE = 1: the diagnostics instantiation (probed raw scores, dS-hat zero count).
template <int D, bool STORE, int MIX, int EXACT, int PROBE = 0>
__global__ void __launch_bounds__(256, 2) bwd_kernel(const BwdArgs a) {
    constexpr int KC = D / 64;
    constexpr int NC = D / 16;                    // 16-channel steps of S on the mixed path
    constexpr int DT = D / 32;
    // The mixed path's bf16 operands take the registers the pipeline needs.
    static_assert(D == 64, "d = 128 runs in bwd_split.hip");
    static_assert(!EXACT || (!STORE && !MIX), "the exact options run without the store, on MXFP8");
    constexpr bool PIPE = !STORE && !MIX;
    // Steps staged by LDS DMA two steps ahead with one barrier per two steps
    // (the MXFP8 pipeline; 2.5% faster than a barrier per step at the same
    // depth); the other variants load a step into registers one step ahead
    // and store it.
    constexpr bool DMA = PIPE && !EXACT;
    constexpr int NBUF = DMA ? 6 : PIPE ? 3 : 2;
    using Step = std::conditional_t<DMA, BwdStepDma<D>, BwdStep<D, MIX, EXACT>>;
    constexpr int STR = Step::kStride;
    constexpr int NSTR = Step::kNStride;
    constexpr int NQ = kQStep * D / 16 / 256;     // 16-byte chunks per thread of a 64-row code tile
    constexpr int NQN = MIX ? 2 * NQ : 1;         // same for the bf16 NVFP4 rows
    __shared__ StepRing<Step, NBUF> sm;
    // byte offset of (row, col) in a staged code tile
    auto toff = [](int row, int col) -> int {
        if constexpr (DMA) return row * D + ((((col >> 4) ^ (row >> 2)) & 3) << 4) + (col & 15);
        else return row * STR + col;
    };

    const int ti = (int)blockIdx.x / a.hkv;
    if (ti >= *a.ntiles) return;
    const int4 it = a.tiles[ti];
    const int k0 = it.x, ds = it.y, de = it.z, doc = it.w;
    const int g = (int)blockIdx.x - ti * a.hkv;
    // the dS store holds this call's blocks: write each dS-hat block once
    const bool use_store = STORE && a.ntiles[1] != 0;
    const long doc_blk = use_store ? (long)a.dboff[doc] : 0;
    const int G = a.hq / a.hkv;
    const int L = de - ds;
    const int kt0 = k0 - ds;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // provably wave-uniform copy
    const int lg = lane >> 5, lr = lane & 31;
    const int key_loc = kt0 + 32 * wave + lr;
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
            const int c = tid + 256 * r;
            const int row = c / (D / 16), col = (c % (D / 16)) * 16;
            const long qr = ds + min(q0 + row, L - 1);
            pq[r] = *reinterpret_cast<const u32x4*>(a.qc + (qr * a.hq + h) * D + col);
            po[r] = *reinterpret_cast<const u32x4*>(a.oc + (qr * a.hq + h) * D + col);
        }
        if constexpr (MIX) {
#pragma unroll
            for (int r = 0; r < NQN; ++r) {
                const int c = tid + 256 * r;
                const int row = c / (D / 8), col = (c % (D / 8)) * 8;   // col in bf16 elements
                const long qr = ds + min(q0 + row, L - 1);
                pqn[r] = *reinterpret_cast<const u32x4*>(a.qn + (qr * a.hq + h) * D + col);
            }
        }
        // Every thread issues the same loads (rows clamped into the document),
        // so the number of outstanding memory operations is static.
        {
            const int ql = q0 + (tid & (kQStep - 1));
            const long qr = ds + min(ql, L - 1);
            p_eq = a.qs[(long)h * a.ttot + qr];
            p_eo = a.os[(long)h * a.ttot + qr];
            p_lse = a.lse2[(long)h * a.ttot + qr];
            p_in = ql < L;
            p_dv = a.dvec[(long)h * a.ttot + qr];
        }
    };
    auto store_step = [&](Step& b) {
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            const int c = tid + 256 * r;
            const int row = c / (D / 16), col = (c % (D / 16)) * 16;
            *reinterpret_cast<u32x4*>(&b.q[row * STR + col]) = pq[r];
            *reinterpret_cast<u32x4*>(&b.o[row * STR + col]) = po[r];
        }
        if constexpr (MIX) {
#pragma unroll
            for (int r = 0; r < NQN; ++r) {
                const int c = tid + 256 * r;
                const int row = c / (D / 8), col = (c % (D / 8)) * 16;   // col in bytes
                *reinterpret_cast<u32x4*>(&b.qn[row * NSTR + col]) = pqn[r];
            }
        }
        if (tid < kQStep) {
            b.eq[tid] = (uint8_t)p_eq;
            b.eo[tid] = (uint8_t)p_eo;
            b.lse[tid] = p_in ? p_lse : INFINITY;   // +inf: row outside the document
            b.dv[tid] = p_dv;                        // -D: accumulator input of dP
        }
        if constexpr (EXACT) {
            // thread tid holds query tid % 64: each half-wave one 32-query block
            const uint32_t eb = halfwave_max(p_eo);
            if (tid < kQStep) {
                b.fo[tid] = ldexpf(1.f, (int)p_eo - (int)eb);
                b.fq[tid] = ldexpf(1.f, (int)p_eq - 127);
                if ((tid & 31) == 0) b.eob[tid >> 5] = (uint8_t)eb;
            }
        }
    };
    // LDS DMA staging: wave w fetches rows 16w .. 16w + 15 of both code tiles
    // (lane l: row 16w + l / 4 into physical chunk l % 4, which holds logical
    // chunk (l % 4) ^ (l / 16)) and one per-query array: lse2 (wave 0), -D (1),
    // Q's (2) and dO's (3) scale bytes.  Rows past the end of the document read zeros: a zero Q and dO row
    // with lse2 = D = 0 has S = dP = dS = 0 and P = 1 against a zero dO row,
    // so it adds nothing to dK or dV.
    auto issue_step = [&](Step& b, int h, int q0) {
        if constexpr (DMA) {
            const int row = 16 * wave_u + (lane >> 2);
            const int c = (lane & 3) ^ (lane >> 4);
            const bool in = q0 + row < L;
            const long off = ((long)(ds + q0 + row) * a.hq + h) * D + 16 * c;
            dma16(in ? (const void*)(a.qc + off) : (const void*)a.zero, &b.q[kQStep * D / 4 * wave_u]);
            dma16(in ? (const void*)(a.oc + off) : (const void*)a.zero, &b.o[kQStep * D / 4 * wave_u]);
            const bool vin = q0 + lane < L;
            const long vo = (long)h * a.ttot + ds + q0 + lane;
            if (wave_u == 0) dma4(vin ? (const void*)(a.lse2 + vo) : (const void*)a.zero, b.lse);
            else if (wave_u == 1) dma4(vin ? (const void*)(a.dvec + vo) : (const void*)a.zero, b.dv);
            else if (wave_u == 2) dma1(vin ? (const void*)(a.qs + vo) : (const void*)a.zero, b.eq);
            else dma1(vin ? (const void*)(a.os + vo) : (const void*)a.zero, b.eo);
        }
    };
    if constexpr (!DMA) load_step(g * G, kt0 + ((L - 1 - kt0) & ~(kQStep - 1)));

    // The wave's key rows as B operands of S and dP (column = key, k = channel);
    // mixed path: channels 16 kc + 8 lg .. + 8 of the key's NVFP4 values for S
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
    // the first pair of steps (issued after the key rows, so that waiting
    // for it waits for the key rows too and for nothing younger)
    const int qlast = kt0 + ((L - 1 - kt0) & ~(kQStep - 1));   // first query of the last step
    int lh = 0, lq0 = qlast;    // next step to fetch
    bool lmore = true;
    bool odd = false;           // the current step is the second of its pair
    // the step after (head hx, queries qx ..): the next head, else the
    // previous 64 queries (the item ends below the diagonal, qx < kt0)
    auto advance = [&](int& hx, int& qx) {
        if (++hx == G) { hx = 0; qx -= kQStep; }
    };
    if constexpr (DMA) {
        issue_step(sm.buf[0], g * G, qlast);
        advance(lh, lq0);
        lmore = lq0 >= kt0;
        if (lmore) {
            issue_step(sm.buf[1], g * G + lh, lq0);
            advance(lh, lq0);
            lmore = lq0 >= kt0;
        }
    }

    v16f dvt[DT], dkt[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) { dvt[dt] = v16f{0}; dkt[dt] = v16f{0}; }
    unsigned nzero = 0;     // diagnostics: nonzero dS entries whose dS-hat code is zero

    const int s16 = lane & 15, grp = (lane >> 4) & 1;
    const int tr_key = 8 * ((s16 >> 1) >> 2) + 4 * lg + ((s16 >> 1) & 3);
    const int tr_col = 16 * grp + 8 * (s16 & 1);
    const float inv256 = 1.f / 256.f;

    // dV^T += dO^T P-hat_b and dK^T += Q^T dS-hat of one step (contraction
    // over its 64 queries), from its codes and its step buffer
    auto dvdk = [&](const Step& b, const int (&pbc)[2][4], const int (&dsc)[2][4], const int (&es)[2]) {
        const v8i pb = v8i{pbc[0][0], pbc[0][1], pbc[0][2], pbc[0][3], pbc[1][0], pbc[1][1], pbc[1][2], pbc[1][3]};
        const v8i db = v8i{dsc[0][0], dsc[0][1], dsc[0][2], dsc[0][3], dsc[1][0], dsc[1][1], dsc[1][2], dsc[1][3]};
        // A scales: dO's and Q's token blocks, or (exact options) dO's block
        // maximum and 1 (Q's exponents are inside dS-hat)
        int so, sq;
        if constexpr (EXACT) {
            so = b.eob[lg];
            sq = 127;
        } else {
            so = b.eo[32 * lg];
            sq = b.eq[32 * lg];
        }
        const int sd = lg ? es[1] : es[0];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            v2i r[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                r[rr] = lds_read_tr8(&b.o[toff(16 * rr + tr_key, 32 * dt + tr_col)]);
            const v8i oa = v8i{r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
            dvt[dt] = mfma_mx(oa, pb, dvt[dt], so, 127 - 8);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                r[rr] = lds_read_tr8(&b.q[toff(16 * rr + tr_key, 32 * dt + tr_col)]);
            const v8i qa = v8i{r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
            dkt[dt] = mfma_mx(qa, db, dkt[dt], sq, sd);
        }
    };
    // Software pipeline (MXFP8, no dS store): the dV/dK products of a step are
    // issued in the next step, right after its S and dP products, so that they
    // run on the matrix cores while the wave computes the next softmax.  With
    // the store, or the mixed path's bf16 operands, the extra live codes spill,
    // so the products follow their own step there.
    int cur = 0;                           // step buffer of the current step
    int prv = 0;                           // step buffer of the previous step
    bool dvdk_due = false;                 // the previous step's dV/dK products are pending
    int ppbc[2][4], pdsc[2][4], pes[2];

    int hh = 0, q0 = qlast;
    // dS blocks of the previous step, stored at the start of the next one
    u32x4 pend_w[2];
    long pend_blk[2] = {0, 0};
    int pend_e[2] = {127, 127};
    bool pend_ok[2] = {false, false};
    auto flush_store = [&]() {
        if (!use_store) return;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (!pend_ok[st]) continue;
            *reinterpret_cast<u32x4*>(a.ds_codes + pend_blk[st] * kDsBlockBytes + 16 * lane) = pend_w[st];
            if (lane == 0) a.ds_scales[pend_blk[st]] = (uint8_t)pend_e[st];
            pend_ok[st] = false;
        }
    };
    // One 64-query step; MASK marks the steps that meet the causal boundary
    // (the last two query steps of every head).  Returns whether another
    // step follows.
    auto step = [&](auto mask_tag) -> bool {
        constexpr bool MASK = decltype(mask_tag)::value;
        Step& B = sm.buf[cur];
        const int h = g * G + hh;
        const int qs0 = q0;
        advance(hh, q0);
        const bool more = q0 >= kt0;
        if constexpr (DMA) {
            // at the first step of a pair: wait for both of its steps' loads
            // (the only ones outstanding), then fetch the next pair
            if (!odd) {
                vm_drain_barrier();
#pragma unroll
                for (int k = 2; k < 4; ++k) {
                    if (lmore) {
                        int b = cur + k;
                        if (b >= NBUF) b -= NBUF;
                        issue_step(sm.buf[b], g * G + lh, lq0);
                        advance(lh, lq0);
                        lmore = lq0 >= kt0;
                    }
                }
            }
            odd = !odd;
        } else {
            // publish the prefetched step in LDS, start fetching the next one
            store_step(B);
            __syncthreads();
            flush_store();
            // unconditional (the last step re-fetches a valid step): a
            // conditional update would keep the prefetch registers in scratch
            load_step(g * G + hh, max(q0, kt0));
        }

        // In a step that meets the causal boundary, the 32-query block st is
        // block qb = (qs0 - kt0) / 32 + st of the key tile's diagonal: blocks
        // qb < wave lie entirely before the wave's keys (P = 0, dS = 0) and
        // are skipped, qb == wave is the only one that needs the mask.
        const int qb0 = (qs0 - kt0) >> 5;
        auto skipped = [&](int st) { return MASK && qb0 + st < wave_u; };
        auto partial = [&](int st) { return MASK && qb0 + st == wave_u; };
        // ---- S and dP for the wave's 32 keys x 64 queries
        v16f sacc[2], pacc[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (skipped(st)) continue;
            const int row = 32 * st + lr;
            sacc[st] = v16f{0};
            // dP starts from -D of each register's query (register 4j + r holds
            // query 32st + 8j + 4lg + r): the MFMA returns dP - D directly, with
            // the same error as a separate fp32 subtraction
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 d4 = *reinterpret_cast<const float4*>(&B.dv[32 * st + 8 * j + 4 * lg]);
                pacc[st][4 * j] = d4.x;
                pacc[st][4 * j + 1] = d4.y;
                pacc[st][4 * j + 2] = d4.z;
                pacc[st][4 * j + 3] = d4.w;
            }
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                if constexpr (MIX) {
#pragma unroll
                    for (int n = 4 * kc; n < 4 * kc + 4; ++n) {
                        const u32x4 qa = *reinterpret_cast<const u32x4*>(&B.qn[row * NSTR + 32 * n + 16 * lg]);
                        sacc[st] = mfma_bf16(qa, kn[n], sacc[st]);
                    }
                } else {
                    const uint4 lo = *reinterpret_cast<const uint4*>(&B.q[toff(row, 64 * kc + 16 * lg)]);
                    const uint4 hi = *reinterpret_cast<const uint4*>(&B.q[toff(row, 64 * kc + 32 + 16 * lg)]);
                    const v8i qa = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    sacc[st] = mfma_mx(qa, kb[kc], sacc[st], B.eq[row], ek);
                }
                const uint4 lo = *reinterpret_cast<const uint4*>(&B.o[toff(row, 64 * kc + 16 * lg)]);
                const uint4 hi = *reinterpret_cast<const uint4*>(&B.o[toff(row, 64 * kc + 32 + 16 * lg)]);
                const v8i oa = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                pacc[st] = mfma_mx(oa, vb[kc], pacc[st], B.eo[row], ev);
            }
        }
        // ---- the previous step's dV/dK products, under this step's softmax
        if (PIPE && dvdk_due) dvdk(sm.buf[prv], ppbc, pdsc, pes);
        // ---- P, P-hat_b, dS, dS-hat (one 32x32 block per accumulator tile)
        // accumulator register i = 4j + r of query block st holds query
        // qs0 + 32st + 8j + 4lg + r; masked while the wave's key lies after it
        const int lim = key_loc - qs0 - 4 * lg;
        int pbc[2][4], dsc[2][4], es[2];   // es: dS block exponent + 127 per query block
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (skipped(st)) {
#pragma unroll
                for (int j = 0; j < 4; ++j) pbc[st][j] = dsc[st][j] = 0;
                es[st] = 127;
                continue;
            }
            if constexpr (PROBE) {
                // diagnostics: the raw scores of the probed query tile
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float* sp = probe_slot(a.probe, 2, h, ds, ds + qs0 + 32 * st + 8 * (i >> 2) + 4 * lg + (i & 3),
                                           key_loc);
                    if (sp) *sp = sacc[st][i];
                }
            }
            float dsv[16];
            float amax = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int q4 = 32 * st + 8 * j + 4 * lg;            // 4 consecutive query rows
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
                    float p = exp2_fast(fmaf(sacc[st][i], a.c1, -lq[r]));
                    if (partial(st))
                        if (32 * st + 8 * j + r < lim) p = 0.f;
                    // exact options: the folds are exact power-of-two scalings
                    sacc[st][i] = EXACT ? p * fo[r] : p;
                    float dsi = p * pacc[st][i];
                    if constexpr (EXACT) dsi *= fq[r];
                    dsv[i] = dsi;
                    amax = fmaxf(amax, fabsf(dsi));
                }
            }
            amax = wave_max_nonneg(amax);
            const int e = block_exponent_uniform(amax, -126);
            es[st] = e + 127;
            const float sc = __uint_as_float((uint32_t)(e + 127) << 23);   // 2^e
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pbc[st][j] = pack_fp8x4_div(sacc[st][4 * j], sacc[st][4 * j + 1], sacc[st][4 * j + 2],
                                            sacc[st][4 * j + 3], inv256);
                dsc[st][j] = pack_fp8x4_div(dsv[4 * j], dsv[4 * j + 1], dsv[4 * j + 2], dsv[4 * j + 3], sc);
            }
            if constexpr (PROBE) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    nzero += (dsv[i] != 0.f && ((((uint32_t)dsc[st][i >> 2] >> (8 * (i & 3))) & 0x7Fu) == 0u)) ? 1u : 0u;
            }
        }
        // ---- dS store: block (qb, kb) as [query half][32 keys][16 queries]
        // (lane l writes bytes 16 l .. 16 l + 15: whole lines per wave); lane
        // half lg holds queries 8j + 4lg + (0..3) in word j and stores queries
        // 16 lg .. 16 lg + 15 of its key after one exchange with lane l ^ 32.
        // The stores are issued at the start of the next step, before its
        // prefetch loads: vector memory operations complete in issue order,
        // so a store issued after a load would make the wait for that load
        // wait for the store as well.
        if (use_store) {
            const int kb = (kt0 >> 5) + wave_u;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                // skipped blocks lie above the diagonal; blocks past the end
                // of the document do not exist in the store
                pend_ok[st] = !skipped(st) && qs0 + 32 * st < L;
                const int qb = (qs0 >> 5) + st;
                pend_blk[st] = (long)h * a.ds_blocks + doc_blk + (long)qb * (qb + 1) / 2 + kb;
                const auto x02 = __builtin_amdgcn_permlane32_swap(dsc[st][0], dsc[st][2], false, false);
                const auto x13 = __builtin_amdgcn_permlane32_swap(dsc[st][1], dsc[st][3], false, false);
                pend_w[st] = u32x4{(uint32_t)x02[0], (uint32_t)x02[1], (uint32_t)x13[0], (uint32_t)x13[1]};
                pend_e[st] = es[st];
            }
        }
        // ---- this step's dV/dK products (block 1 skipped implies block 0
        // skipped: nothing to add), in the next step when pipelined
        if constexpr (PIPE) {
            dvdk_due = !skipped(1);
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ppbc[st][j] = pbc[st][j];
                    pdsc[st][j] = dsc[st][j];
                }
                pes[st] = es[st];
            }
        } else if (!skipped(1)) {
            dvdk(B, pbc, dsc, es);
        }
        // Scheduling hint for the unmasked steps: spread the step's eight
        // MFMAs over its VALU stream (one per 24 VALU instructions), so that
        // the matrix pipe keeps working through the second block's softmax
        // (2% faster than the compiler's own order, which issues the last
        // products early and leaves the tail of the step without any).
        if constexpr (!MASK) {
#pragma unroll
            for (int g8 = 0; g8 < 8; ++g8) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);   // then 24 VALU
            }
        }
        prv = cur;
        cur = cur + 1 == NBUF ? 0 : cur + 1;
        return more;
    };
    // two loops instead of a per-step choice, so that both bodies keep the
    // accumulators in the same registers
    bool more = true;
    while (more) {
        while (more && q0 >= kt0 + kTile) more = step(std::false_type{});
        while (more && q0 < kt0 + kTile) more = step(std::true_type{});
    }
    if (PIPE && dvdk_due) dvdk(sm.buf[prv], ppbc, pdsc, pes);
    flush_store();
    if constexpr (PROBE) {
        const unsigned n = wave_sum_u32(nzero);
        if (a.probe.ds_zero && lane == 0 && n) atomicAdd(a.probe.ds_zero, (unsigned long long)n);
    }
    // ---- epilogue: dK = softmax_scale * sum, dV; summed over the group's heads.
    // With the Hadamard option the dK sum is the gradient of the rotated K and
    // is rotated back first.
    float sck = a.scale;
    if (a.hadamard) {
        hadamard_rows<DT>(dkt, lg);
        sck *= inv_sqrt_d<D>();
    }
    if (key_valid) {
        uint16_t* kp = a.dk + ((long)(ds + key_loc) * a.hkv + g) * D;
        uint16_t* vp = a.dv + ((long)(ds + key_loc) * a.hkv + g) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int dd = 32 * dt + 8 * j + 4 * lg;
                *reinterpret_cast<uint2*>(kp + dd) = make_uint2(
                    pack_bf16x2(dkt[dt][4 * j] * sck, dkt[dt][4 * j + 1] * sck),
                    pack_bf16x2(dkt[dt][4 * j + 2] * sck, dkt[dt][4 * j + 3] * sck));
                *reinterpret_cast<uint2*>(vp + dd) = make_uint2(
                    pack_bf16x2(dvt[dt][4 * j], dvt[dt][4 * j + 1]),
                    pack_bf16x2(dvt[dt][4 * j + 2], dvt[dt][4 * j + 3]));
            }
    }
}

template <int D, bool STORE>
static void launch_bwd_mix(const BwdArgs& a, dim3 g, hipStream_t st) {
    if (a.qn) hipLaunchKernelGGL((bwd_kernel<D, STORE, 1, 0>), g, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((bwd_kernel<D, STORE, 0, 0>), g, dim3(256), 0, st, a);
}

hipError_t launch_bwd(const BwdArgs& a, int d, long grid, hipStream_t st) {
    if (grid <= 0) return hipSuccess;
    // d = 128: eight-wave workgroups that split each step between wave pairs
    // (bwd_split.hip)
    if (d != 64) return launch_bwd_split(a, grid, st);
    // the store variant only where the workspace has a dS store
    const bool store = a.ds_blocks > 0;
    const dim3 g((unsigned)grid);
    if (a.exact) {
        if (store || a.qn) return hipErrorInvalidValue;
        hipLaunchKernelGGL((bwd_kernel<64, false, 0, 1>), g, dim3(256), 0, st, a);
        return hipGetLastError();
    }
    if (a.probe.scores || a.probe.ds_zero) {
        // diagnostics: the MXFP8 path (checked by the host layer)
        if (a.qn) return hipErrorInvalidValue;
        if (store) hipLaunchKernelGGL((bwd_kernel<64, true, 0, 0, 1>), g, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((bwd_kernel<64, false, 0, 0, 1>), g, dim3(256), 0, st, a);
        return hipGetLastError();
    }
    if (store) launch_bwd_mix<64, true>(a, g, st);
    else launch_bwd_mix<64, false>(a, g, st);
    return hipGetLastError();
}

}  // namespace flamia
