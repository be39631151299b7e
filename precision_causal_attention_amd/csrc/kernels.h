// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flamia {

constexpr int kTile = 128;     // query and key tile (B_r = B_c = 128)
constexpr int kBlock = 32;     // token block of the operand scales and of the dS blocks

// One tensor of a quantization launch: bf16 [T][heads][d] in, E4M3 codes
// [T][heads][d] and UE8M0 scales [heads][T] out; optionally the NVFP4 values
// of the same rows (one E4M3 scale per 16 channels of a token, E2M1
// elements) expanded to bf16 [T][heads][d].
struct QuantTensor {
    const uint16_t* x;
    uint8_t* codes;
    uint8_t* scales;
    int heads;
    int rot;                  // 1: quantize the Hadamard-rotated rows
    uint16_t* nv;             // NVFP4 values (nullptr: not written)
};

struct QuantArgs {
    const int32_t* cu;
    int ndocs, ttot, d;
    QuantTensor t[3];
    int ntensors;
    int per_token;            // 1: one exponent per token instead of per 32-token block
    // dO variant only (nullptr otherwise; then t[0] is dO): -D with D = dO~ . O
    // (stored negated: the backward products start their dP accumulators from it)
    const uint16_t* o;
    float* dvec;
};

// Tile lists: int4 {first token of the 128-token tile (global), document
// start, document end, document index}, expensive items first (plan.hip);
// ctrl[0]
// holds the number of tiles.  A work item is (tile, head): the attention
// kernels decode it from the workgroup index (tile = index / heads).
// dS store: per query head, the 32x32 causal blocks (qb >= kb, document-local
// 32-token block indices) of every document; block (qb, kb) of document d is
// block dboff[d] + qb (qb + 1) / 2 + kb of the head, 1024 code bytes
// ([2][32][16]: query half, key, 16 queries) and one UE8M0 scale byte.
constexpr int kDsBlockBytes = kBlock * kBlock;

// Optional diagnostics of the attention kernels, run by separate
// instantiations (PROBE = 1) that the default launches never use.
//   scores: fp32 [3][128][keys], the raw scores S = q.k (block scales
//   applied, before the softmax scale) of the 128-query tile that starts at
//   packed token q0 of the document starting at packed token doc_start, query
//   head `head`, keys in document-local order: [0] as the forward computes
//   them, [1] the dQ pass, [2] the dK/dV pass (nullptr: none);
//   ds_zero: the dK/dV pass adds the number of nonzero dS entries whose
//   dS-hat code is zero (nullptr: none).
struct ProbeArgs {
    float* scores;
    int doc_start, q0, head, keys;
    unsigned long long* ds_zero;
};

// Address of the probed score of query `qrow` (packed token) and
// key `key` (document-local) in table `which` (0 forward, 1 dQ pass, 2 dK/dV
// pass), or nullptr when this (head, document, query, key) is not probed.
__device__ __forceinline__ float* probe_slot(const ProbeArgs& p, int which, int head, int doc_start,
                                             int qrow, int key) {
    const int qi = qrow - p.q0;
    if (!p.scores || head != p.head || doc_start != p.doc_start || qi < 0 || qi >= kTile || key < 0 ||
        key >= p.keys)
        return nullptr;
    return p.scores + ((long)which * kTile + qi) * p.keys + key;
}

struct PlanArgs {
    const int32_t* cu;
    int ndocs;
    int ttot;
    int32_t* cu_status;    // nonzero bits when cu_seqlens is malformed (nullptr: not reported)
    int max_cost;          // >= max tiles of one document
    int32_t* tiles_prefix; // [ndocs + 1]
    int32_t* ctrl;         // control block, see plan.hip
    long max_tiles;
    int4* tiles_q;         // query-major order: cost = tile index + 1 (forward, dQ)
    int4* tiles_k;         // key-major order: cost = tiles from the diagonal to the end
                           // (dK/dV); nullptr: not built
    int key_docmajor;      // 1: the key-major list in document-major order (else cost-major)
    int32_t* dboff;        // [ndocs] first dS block of each document (nullptr: none)
    long ds_blocks;        // dS store capacity in blocks per head (0: no store)
};

struct FwdArgs {
    const uint8_t *qc, *qs, *kc, *ks, *vc, *vs;
    uint16_t* o;
    float* lse2;
    const int4* tiles;
    const int32_t* ntiles;
    int ttot, hq, hkv;
    float c1;              // softmax_scale * log2(e)
    float c_log2, tau;
    int rowsum;
    int fast_exp;          // 0, or 5 / 8 key-pair classes of 8 with the approximate exponential
    const uint16_t *qn, *kn;   // mixed path: NVFP4 values of Q and K (bf16) for the scores; else nullptr
    int exact;                 // 1: the exact options (per-token scales, V's folded into P-hat)
    ProbeArgs probe;           // diagnostics (launches the PROBE instantiation when set)
};

struct BwdArgs {
    const uint8_t *qc, *qs, *kc, *ks, *vc, *vs, *oc, *os;   // oc/os: quantized dO
    const float* lse2;
    const float* dvec;        // -D per (head, token)
    uint16_t *dk, *dv;
    const int4* tiles;
    const int32_t* ntiles;    // ntiles[1] != 0: store dS-hat blocks
    int32_t* queue;           // work-queue counter of the persistent d = 128 pass (zeroed by the work lists)
    int ttot, hq, hkv;
    float c1, scale;
    int hadamard;             // 1: rotate dK back (Q and K were rotated)
    const uint16_t *qn, *kn;  // mixed path: NVFP4 values of Q and K for the scores; else nullptr
    uint8_t* ds_codes;        // dS store (see PlanArgs)
    uint8_t* ds_scales;
    const int32_t* dboff;
    long ds_blocks;
    int exact;                // 1: the exact options (dO's and Q's token exponents folded)
    const uint8_t* zero;      // 64 zero bytes, 16-byte aligned (the rows past a document's end)
    ProbeArgs probe;
};

struct DqArgs {
    const uint8_t *qc, *qs, *kc, *ks, *vc, *vs, *oc, *os;
    const float* lse2;
    const float* dvec;
    uint16_t* dq;
    const int4* tiles;
    const int32_t* ntiles;    // ntiles[1]: the dS store is in use (the rebuilding
                              // pass runs when it is 0, the store pass when it is 1)
    int ttot, hq, hkv;
    float c1, scale;
    int hadamard;             // 1: rotate dQ back (Q and K were rotated)
    const uint16_t *qn, *kn;  // mixed path: NVFP4 values of Q and K for the scores; else nullptr
    // Without a dS store this pass runs first and quantizes dO itself: bf16
    // dO and O in; the dO codes, scales and D out (read by the key-major
    // pass that follows).  nullptr: the codes, scales and D are inputs.
    const uint16_t *d_o, *o;
    uint8_t *oc_w, *os_w;
    float* dvec_w;
    const uint8_t* ds_codes;  // dS store (see PlanArgs)
    const uint8_t* ds_scales;
    const int32_t* dboff;
    long ds_blocks;
    int exact;                // 1: the exact options (K's token exponent folded, per-row dS exponent)
    ProbeArgs probe;
};

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st);
hipError_t launch_plan(const PlanArgs& a, hipStream_t st);
hipError_t launch_fwd(const FwdArgs& a, int d, long grid, hipStream_t st);
hipError_t launch_bwd(const BwdArgs& a, int d, long grid, hipStream_t st);
hipError_t launch_bwd_split(const BwdArgs& a, long grid, hipStream_t st);   // d = 128
hipError_t device_cus(int* n);   // CU count of the current device (cached per device)
hipError_t launch_dq(const DqArgs& a, int d, long grid, hipStream_t st);
hipError_t launch_dq_store(const DqArgs& a, int d, long grid, hipStream_t st);

}  // namespace flamia
