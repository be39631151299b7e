// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flamia {

constexpr int kTile = 128;     // query and key tile (B_r = B_c = 128)
constexpr int kBlock = 32;     // token block of the operand scales and of the dS blocks

struct QuantArgs {
    const uint16_t* x;
    const int32_t* cu;
    int ndocs, ttot, heads, d;
    uint8_t* codes;
    uint8_t* scales;
    // dO variant only (nullptr otherwise): D = dO~ . O
    const uint16_t* o;
    float* dvec;
};

// Work items: int4 {first token of the tile (global), document start,
// document end, head}.
struct PlanArgs {
    const int32_t* cu;
    int ndocs;
    int max_cost;          // >= max tiles of one document
    int32_t* tiles_prefix; // [ndocs + 1]
    int32_t* ctrl;         // control block, see plan.hip
    long max_tiles;
    int heads_q;           // query-major list: cost = tile index + 1 (forward, dQ)
    int4* items_q;
    int heads_k;           // key-major list: cost = tiles from the diagonal to the end (dK/dV);
    int4* items_k;         // nullptr: not built
};

struct FwdArgs {
    const uint8_t *qc, *qs, *kc, *ks, *vc, *vs;
    uint16_t* o;
    float* lse2;
    const int4* items;
    const int32_t* nitems;
    int ttot, hq, hkv;
    float c1;              // softmax_scale * log2(e)
    float c_log2, tau;
    int rowsum;
};

struct BwdArgs {
    const uint8_t *qc, *qs, *kc, *ks, *vc, *vs, *oc, *os;   // oc/os: quantized dO
    const float* lse2;
    const float* dvec;
    uint16_t *dk, *dv;
    const int4* items;
    const int32_t* nitems;
    int ttot, hq, hkv;
    float c1, scale;
};

struct DqArgs {
    const uint8_t *qc, *qs, *kc, *ks, *vc, *vs, *oc, *os;
    const float* lse2;
    const float* dvec;
    uint16_t* dq;
    const int4* items;
    const int32_t* nitems;
    int ttot, hq, hkv;
    float c1, scale;
};

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st);
hipError_t launch_plan(const PlanArgs& a, hipStream_t st);
hipError_t launch_fwd(const FwdArgs& a, int d, long grid, hipStream_t st);
hipError_t launch_bwd(const BwdArgs& a, int d, long grid, hipStream_t st);
hipError_t launch_dq(const DqArgs& a, int d, long grid, hipStream_t st);

}  // namespace flamia
