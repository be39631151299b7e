// Query-major dQ pass from the stored dS-hat blocks (FLAMIA paper: Section 2
// equation dQ = dS K; the dS-hat payload is the one the key-major pass
// quantized, Section 3.3, one E4M3 exponent per 32x32 document-local block).
//
// One workgroup = one work item (document, query head, 128-query tile
// anchored at the document start); wave w owns query block qb = 4T + w (32
// queries).  Per 128-key tile, ascending up to the diagonal:
//   the K^ code tile goes to LDS (shared by the four waves), the wave's four
//   dS-hat blocks (qb, 4t + m) go to LDS as [128 keys][32 queries] (per wave);
//   both are read with the transposing ds_read_b64_tr_b8 in the same key order:
//   dQ^T[d][query] += K^T dS-hat^T   (A = K^T, scale per 32-key block of K;
//                                     B = dS-hat^T, scale per dS block)
// The operands, their byte order and the order of accumulation are those of
// the rebuilding pass (dq.hip), so dQ is bitwise the same.  Blocks above the
// diagonal or past the end of the document are zero (not stored).
// Memory-bound: each stored block is read once.
#include "device.h"
#include "kernels.h"

namespace flamia {

template <int D>
struct DqsSmem {
    static constexpr int kStride = D + 16;          // K tile row pitch (bank spread)
    static constexpr int kDsStride = kBlock + 8;    // dS rows: 40 bytes (bank spread for the transposed reads)
    uint8_t k[kTile * kStride];
    uint8_t ek[kTile];
    alignas(16) uint8_t ds[4][kTile * kDsStride];   // one region per wave
};

template <int D>
__global__ void __launch_bounds__(256, D == 64 ? 3 : 2) dq_store_kernel(const DqArgs a) {
    constexpr int DT = D / 32;
    constexpr int STR = DqsSmem<D>::kStride;
    constexpr int DSTR = DqsSmem<D>::kDsStride;
    constexpr int KCH = kTile * D / 16 / 256;        // 16-byte K chunks per thread
    __shared__ DqsSmem<D> sm;

    if (a.ntiles[1] == 0) return;                    // no store this call: dq.hip runs
    const int ti = (int)blockIdx.x / a.hq;
    if (ti >= a.ntiles[0]) return;
    const int4 it = a.tiles[ti];
    const int q0 = it.x, ds = it.y, de = it.z, doc = it.w;
    const int h = xcd_head((int)blockIdx.x - ti * a.hq, a.hq, it.w);
    const int g = h / (a.hq / a.hkv);
    const int L = de - ds;
    const int lq0 = q0 - ds;
    const int ntiles = lq0 / kTile + 1;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int lg = lane >> 5;
    const int q_loc = lq0 + 32 * wave + (lane & 31);
    const bool q_valid = q_loc < L;

    // the wave's query block; blocks are addressed inside the document's
    // triangle (rows clamped to the last block of the document)
    const int nb = (L + kBlock - 1) / kBlock;
    const int qb = (lq0 >> 5) + wave_u;
    const bool qb_valid = qb < nb;
    const int qa = min(qb, nb - 1);
    const long row0 = (long)h * a.ds_blocks + a.dboff[doc] + (long)qa * (qa + 1) / 2;   // block (qa, 0)

    // ---- prefetch of one key tile: K codes + scales (shared), the wave's four
    // dS blocks (lane l: bytes 16 l .. 16 l + 15 of each block = key l % 32,
    // queries 16 (l / 32) .. + 15) and the two dS scales the lane needs.
    // Two register sets alternate, so two tiles are in flight per workgroup
    // (the pass is bound by the bytes in flight against the memory latency).
    struct Pre {
        u32x4 kr[KCH];
        uint32_t ekr;
        u32x4 dr[4];
        uint32_t e0, e1;
    };
    auto fetch = [&](Pre& f, int t) {
        const int k0 = ds + kTile * t;
#pragma unroll
        for (int r = 0; r < KCH; ++r) {
            const int c = tid + 256 * r;
            const int row = c / (D / 16), col = (c % (D / 16)) * 16;
            const long krow = min(k0 + row, a.ttot - 1);
            f.kr[r] = *reinterpret_cast<const u32x4*>(a.kc + (krow * a.hkv + g) * D + col);
        }
        f.ekr = a.ks[(long)g * a.ttot + min(k0 + (tid & 127), a.ttot - 1)];
        // raw loads only: blocks above the diagonal are zeroed where the
        // data is used (a select here would wait for the load at once)
#pragma unroll
        for (int m = 0; m < 4; ++m)
            f.dr[m] = *reinterpret_cast<const u32x4*>(a.ds_codes + (row0 + min(4 * t + m, qa)) * kDsBlockBytes + 16 * lane);
        f.e0 = a.ds_scales[row0 + min(4 * t + lg, qa)];          // chunk 0 block of this lane half
        f.e1 = a.ds_scales[row0 + min(4 * t + 2 + lg, qa)];      // chunk 1 block
    };

    v16f acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = v16f{0};

    const int s16 = lane & 15, grp = (lane >> 4) & 1;
    const int tr_key = 8 * ((s16 >> 1) >> 2) + 4 * lg + ((s16 >> 1) & 3);
    const int tr_col = 16 * grp + 8 * (s16 & 1);
    uint8_t* dsl = sm.ds[wave_u];

    // tile t from register set f, then f refetches tile t + 2 (clamped: the
    // last tiles re-fetch the last one, unused)
    auto step = [&](Pre& f, const int t) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < KCH; ++r) {
            const int c = tid + 256 * r;
            const int row = c / (D / 16), col = (c % (D / 16)) * 16;
            *reinterpret_cast<u32x4*>(&sm.k[row * STR + col]) = f.kr[r];
        }
        if (tid < kTile) sm.ek[tid] = (uint8_t)f.ekr;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const bool live = qb_valid && 4 * t + m <= qb;     // wave-uniform
            uint8_t* p = dsl + (32 * m + (lane & 31)) * DSTR + 16 * lg;
            *reinterpret_cast<v2i*>(p) = live ? v2i{(int)f.dr[m][0], (int)f.dr[m][1]} : v2i{0, 0};
            *reinterpret_cast<v2i*>(p + 8) = live ? v2i{(int)f.dr[m][2], (int)f.dr[m][3]} : v2i{0, 0};
        }
        const uint32_t sd0 = (qb_valid && 4 * t + lg <= qb) ? f.e0 : 127u;
        const uint32_t sd1 = (qb_valid && 4 * t + 2 + lg <= qb) ? f.e1 : 127u;
        __syncthreads();
        fetch(f, min(t + 2, ntiles - 1));

#pragma unroll
        for (int c = 0; c < 2; ++c) {
            if (!qb_valid || 4 * t + 2 * c > qb) continue;   // both blocks of the chunk are zero
            v2i r[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) r[rr] = lds_read_tr8(&dsl[(64 * c + 16 * rr + tr_key) * DSTR + tr_col]);
            const v8i db = v8i{r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
            const int sk = sm.ek[64 * c + 32 * lg];
            const int sd = (int)(c ? sd1 : sd0);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    r[rr] = lds_read_tr8(&sm.k[(64 * c + 16 * rr + tr_key) * STR + 32 * dt + tr_col]);
                const v8i ka = v8i{r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
                acc[dt] = mfma_mx(ka, db, acc[dt], sk, sd);
            }
        }
    };
    Pre fa, fb;
    fetch(fa, 0);
    fetch(fb, min(1, ntiles - 1));
    for (int t = 0; t < ntiles; t += 2) {
        step(fa, t);
        if (t + 1 < ntiles) step(fb, t + 1);          // workgroup-uniform
    }
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

hipError_t launch_dq_store(const DqArgs& a, int d, long grid, hipStream_t st) {
    if (grid <= 0) return hipSuccess;
    if (d == 64) hipLaunchKernelGGL(dq_store_kernel<64>, dim3((unsigned)grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(dq_store_kernel<128>, dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace flamia
