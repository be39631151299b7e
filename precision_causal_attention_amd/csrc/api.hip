// C-ABI host layer: argument validation, workspace layout and the launch
// sequence of the training call.  Nothing here synchronizes with the device
// or allocates memory; every launch goes to the caller's stream.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "flamia.h"
#include "kernels.h"

using namespace flamia;

// Static scratch of flamia_fwd_noalloc: the forward's control block, tile
// prefix and work list, one copy per device (each device's copy lives at its
// own address, found with hipGetSymbolAddress).  Host code never passes the
// array's name to a kernel or a copy, only the per-device addresses.
constexpr size_t kNoallocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {

thread_local char g_last_error[256] = "";

flamia_status_t hip_fail(hipError_t e) {
    strncpy(g_last_error, hipGetErrorString(e), sizeof g_last_error - 1);
    g_last_error[sizeof g_last_error - 1] = 0;
    return FLAMIA_ERR_HIP;
}

constexpr long kMaxTokens = 1L << 20;        // ttot_cap limit (1M tokens; bounds the plan kernel's LDS histogram)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Capacities and head layout (all the workspace size depends on).
flamia_status_t check_caps(const flamia_dims_t* d) {
    if (!d) return FLAMIA_ERR_NULL;
    if (d->d != 64 && d->d != 128) return FLAMIA_ERR_SHAPE;
    if (d->hq <= 0 || d->hkv <= 0 || d->hq % d->hkv) return FLAMIA_ERR_SHAPE;
    if (d->ttot_cap < 0 || d->ttot_cap > kMaxTokens) return FLAMIA_ERR_SHAPE;
    if (d->ndocs_cap < 0 || d->ndocs_cap > kMaxTokens) return FLAMIA_ERR_SHAPE;
    if (d->doclen_cap < 0 || d->doclen_cap > d->ttot_cap) return FLAMIA_ERR_SHAPE;
    return FLAMIA_OK;
}

// Everything a call needs: capacities plus the current sizes within them.
flamia_status_t check_dims(const flamia_dims_t* d) {
    const flamia_status_t s = check_caps(d);
    if (s != FLAMIA_OK) return s;
    if (d->ttot < 0 || d->ttot > d->ttot_cap) return FLAMIA_ERR_SHAPE;
    if (d->ndocs < 0 || d->ndocs > d->ndocs_cap) return FLAMIA_ERR_SHAPE;
    if (d->ttot > 0 && d->ndocs == 0) return FLAMIA_ERR_SHAPE;
    return FLAMIA_OK;
}

flamia_status_t check_opts(const flamia_opts_t* o) {
    // Section 3.4 / Appendix B.1: 2^(c + tau) must stay within 448.
    if (o->c_log2 < 0 || o->tau < 0 || o->c_log2 + o->tau > 8) return FLAMIA_ERR_OPTS;
    if (o->key_tile != kTile) return FLAMIA_ERR_OPTS;
    if (o->rowsum != 0 && o->rowsum != 1) return FLAMIA_ERR_OPTS;
    if (o->hadamard != 0 && o->hadamard != 1) return FLAMIA_ERR_OPTS;
    if (o->fast_exp != 0 && o->fast_exp != 5 && o->fast_exp != 8) return FLAMIA_ERR_OPTS;
    if (o->mixed != 0 && o->mixed != 1) return FLAMIA_ERR_OPTS;
    if (o->mixed && o->fast_exp) return FLAMIA_ERR_OPTS;   // the inference exponential is MXFP8-only
    if (o->exact != 0 && o->exact != 1) return FLAMIA_ERR_OPTS;
    // the exact options run on the MXFP8 path with the unquantized row sum
    // and the exact exponential
    if (o->exact && (o->rowsum || o->fast_exp || o->mixed)) return FLAMIA_ERR_OPTS;
    if (!(o->softmax_scale <= 0.f || isfinite(o->softmax_scale))) return FLAMIA_ERR_OPTS;
    if (o->n_events < 0 || (o->n_events > 0 && !o->phase_events)) return FLAMIA_ERR_OPTS;
    // diagnostics instantiations exist for the MXFP8 path with the exact exponential
    if ((o->probe_scores || o->ds_zero_count) && (o->mixed || o->exact || o->fast_exp)) return FLAMIA_ERR_OPTS;
    if (o->probe_scores && (o->probe_keys <= 0 || o->probe_head < 0 || o->probe_doc_start < 0 ||
                            o->probe_q0 < o->probe_doc_start || (o->probe_q0 - o->probe_doc_start) % kTile))
        return FLAMIA_ERR_OPTS;
    return FLAMIA_OK;
}

ProbeArgs probe_of(const flamia_opts_t& o) {
    return ProbeArgs{o.probe_scores, o.probe_doc_start, o.probe_q0, o.probe_head, o.probe_keys,
                     (unsigned long long*)o.ds_zero_count};
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
    long max_tiles;
    int max_cost;
    long ds_blocks;        // dS store capacity, 32x32 blocks per head (0: none)
    size_t ctrl, prefix, tiles_q, tiles_k, ocodes, oscales, dvec, dboff, ds_codes, ds_scales, total;
};

Layout layout(const flamia_dims_t* d) {
    Layout w;
    const long tc = d->ttot_cap;
    w.max_cost = (int)((tc + kTile - 1) / kTile) + 1;
    w.max_tiles = tc / kTile + d->ndocs_cap + 1;
    size_t off = 0;
    w.ctrl = off;    off += up256(sizeof(int32_t) * 16);
    w.prefix = off;  off += up256(sizeof(int32_t) * ((size_t)d->ndocs_cap + 1));
    w.tiles_q = off; off += up256(sizeof(int4) * (size_t)w.max_tiles);
    w.tiles_k = off; off += up256(sizeof(int4) * (size_t)w.max_tiles);
    w.ocodes = off;  off += up256((size_t)tc * d->hq * d->d);
    w.oscales = off; off += up256((size_t)tc * d->hq);
    w.dvec = off;    off += up256(sizeof(float) * (size_t)tc * d->hq);
    // dS store: sum over documents of nb (nb + 1) / 2 with nb = ceil(L / 32)
    // is at most (sum of nb) * (max nb + 1) / 2, sum of nb <= ttot / 32 + ndocs
    if (d->doclen_cap > 0) {
        const long nb_sum = tc / kBlock + d->ndocs_cap;
        const long nb_max = (d->doclen_cap + kBlock - 1) / kBlock;
        w.ds_blocks = nb_sum * (nb_max + 1) / 2;
    } else {
        w.ds_blocks = 0;
    }
    w.dboff = off;     off += up256(sizeof(int32_t) * ((size_t)d->ndocs_cap + 1));
    w.ds_codes = off;  off += up256((size_t)w.ds_blocks * d->hq * kDsBlockBytes);
    w.ds_scales = off; off += up256((size_t)w.ds_blocks * d->hq);
    w.total = off;
    return w;
}

flamia_opts_t resolve(const flamia_opts_t* o) { return o ? *o : flamia_default_opts(); }

// Records the caller's phase event i (if provided) on the stream.
struct PhaseMarks {
    const flamia_opts_t& o;
    hipStream_t st;
    int next = 0;
    hipError_t mark() {
        const int i = next++;
        if (!o.phase_events || i >= o.n_events || !o.phase_events[i]) return hipSuccess;
        return hipEventRecord((hipEvent_t)o.phase_events[i], st);
    }
};

float scale_of(const flamia_opts_t& o, int d) {
    return o.softmax_scale > 0.f ? o.softmax_scale : 1.0f / sqrtf((float)d);
}

bool mx_ok(flamia_mx_t m) { return m.codes && m.scales && aligned16(m.codes); }

// Mixed path: Q and K must carry their NVFP4 values.
flamia_status_t check_nv(const flamia_opts_t& o, flamia_mx_t q, flamia_mx_t k) {
    if (!o.mixed) return FLAMIA_OK;
    if (!q.nv || !k.nv) return FLAMIA_ERR_NULL;
    if (!aligned16(q.nv) || !aligned16(k.nv)) return FLAMIA_ERR_ALIGN;
    return FLAMIA_OK;
}

// Validation shared by flamia_fwd and flamia_fwd_noalloc (everything but
// the workspace).
flamia_status_t check_fwd(const flamia_dims_t* dims, const flamia_opts_t& opts,
                          const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const int32_t* cu_seqlens, flamia_mx_t q_mx, flamia_mx_t k_mx, flamia_mx_t v_mx,
                          const uint16_t* o, const float* lse2) {
    flamia_status_t s;
    if ((s = check_opts(&opts)) != FLAMIA_OK) return s;
    if (!q || !k || !v || !cu_seqlens || !o || !lse2 || !q_mx.codes || !q_mx.scales ||
        !k_mx.codes || !k_mx.scales || !v_mx.codes || !v_mx.scales)
        return FLAMIA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !mx_ok(q_mx) ||
        !mx_ok(k_mx) || !mx_ok(v_mx))
        return FLAMIA_ERR_ALIGN;
    return check_nv(opts, q_mx, k_mx);
}

// The forward's launches; `base` holds the forward's part of the layout `w`
// (control block, tile prefix, query-major work list).
flamia_status_t fwd_enqueue(const flamia_dims_t* dims, const flamia_opts_t& opts,
                            const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* cu_seqlens, flamia_mx_t q_mx, flamia_mx_t k_mx, flamia_mx_t v_mx,
                            uint16_t* o, float* lse2, uint8_t* base, const Layout& w, hipStream_t st) {
    const int d = dims->d;
    // quantization of the three operands in one launch (Section 3.5.1)
    QuantArgs qa{};
    qa.cu = cu_seqlens; qa.ndocs = dims->ndocs; qa.ttot = dims->ttot; qa.d = d;
    // with the Hadamard option Q and K are quantized from their rotated rows
    // (Section 3.4: the rotation is fused into the quantizer), V never is;
    // on the mixed path Q and K also get their NVFP4 values
    uint16_t* qn = opts.mixed ? q_mx.nv : nullptr;
    uint16_t* kn = opts.mixed ? k_mx.nv : nullptr;
    qa.t[0] = QuantTensor{q, q_mx.codes, q_mx.scales, dims->hq, opts.hadamard, qn};
    qa.t[1] = QuantTensor{k, k_mx.codes, k_mx.scales, dims->hkv, opts.hadamard, kn};
    qa.t[2] = QuantTensor{v, v_mx.codes, v_mx.scales, dims->hkv, 0, nullptr};
    qa.ntensors = 3;
    qa.per_token = opts.exact;
    PhaseMarks pm{opts, st};
    hipError_t e;
    if ((e = pm.mark()) != hipSuccess || (e = launch_quantize(qa, st)) != hipSuccess) return hip_fail(e);
    int32_t* ctrl = (int32_t*)(base + w.ctrl);
    int4* tiles = (int4*)(base + w.tiles_q);
    PlanArgs pa{cu_seqlens, dims->ndocs, dims->ttot, opts.cu_status, w.max_cost, (int32_t*)(base + w.prefix),
                ctrl, w.max_tiles, tiles, nullptr, 0, nullptr, 0};
    if ((e = pm.mark()) != hipSuccess || (e = launch_plan(pa, st)) != hipSuccess) return hip_fail(e);
    FwdArgs fa;
    fa.qc = q_mx.codes; fa.qs = q_mx.scales;
    fa.kc = k_mx.codes; fa.ks = k_mx.scales;
    fa.vc = v_mx.codes; fa.vs = v_mx.scales;
    fa.o = o; fa.lse2 = lse2;
    fa.tiles = tiles; fa.ntiles = ctrl;
    fa.ttot = dims->ttot; fa.hq = dims->hq; fa.hkv = dims->hkv;
    fa.c1 = scale_of(opts, d) * 1.4426950408889634f;
    fa.c_log2 = (float)opts.c_log2;
    fa.tau = (float)opts.tau;
    fa.rowsum = opts.rowsum;
    fa.fast_exp = opts.fast_exp;
    fa.qn = qn; fa.kn = kn;
    fa.exact = opts.exact;
    fa.probe = probe_of(opts);
    fa.probe.ds_zero = nullptr;
    if ((e = pm.mark()) != hipSuccess || (e = launch_fwd(fa, d, w.max_tiles * dims->hq, st)) != hipSuccess)
        return hip_fail(e);
    e = pm.mark();
    return e == hipSuccess ? FLAMIA_OK : hip_fail(e);
}

constexpr int kMaxDevices = 64;
std::atomic<uint8_t*> g_scratch_ptr[kMaxDevices];

// The current device's copy of the scratch array (looked up once per device).
hipError_t scratch_of_current_device(uint8_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    uint8_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        void* a = nullptr;
        if ((e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        p = (uint8_t*)a;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

flamia_opts_t flamia_default_opts(void) {
    flamia_opts_t o;
    o.c_log2 = 4;
    o.tau = 4;
    o.key_tile = kTile;
    o.rowsum = 0;
    o.softmax_scale = 0.f;
    o.hadamard = 0;
    o.fast_exp = 0;
    o.mixed = 0;
    o.exact = 0;
    o.phase_events = nullptr;
    o.n_events = 0;
    o.cu_status = nullptr;
    o.ds_zero_count = nullptr;
    o.probe_scores = nullptr;
    o.probe_doc_start = o.probe_q0 = o.probe_head = 0;
    o.probe_keys = 0;
    return o;
}

int flamia_abi_version(void) { return FLAMIA_ABI_VERSION; }

const char* flamia_status_str(flamia_status_t s) {
    switch (s) {
        case FLAMIA_OK: return "ok";
        case FLAMIA_ERR_NULL: return "null pointer argument";
        case FLAMIA_ERR_SHAPE: return "unsupported or inconsistent shape";
        case FLAMIA_ERR_ALIGN: return "pointer not 16-byte aligned";
        case FLAMIA_ERR_OPTS: return "invalid options (c_log2 + tau must be <= 8, key_tile 128)";
        case FLAMIA_ERR_WORKSPACE: return "workspace missing or too small";
        case FLAMIA_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

const char* flamia_last_error(void) { return g_last_error; }

size_t flamia_workspace_bytes(const flamia_dims_t* dims, const flamia_opts_t* opts) {
    if (check_caps(dims) != FLAMIA_OK) return 0;
    (void)opts;
    return layout(dims).total;
}

flamia_status_t flamia_quantize(const flamia_dims_t* dims, int32_t heads, const uint16_t* x,
                                const int32_t* cu_seqlens, flamia_mx_t out, void* stream) {
    flamia_status_t s = check_dims(dims);
    if (s != FLAMIA_OK) return s;
    if (heads <= 0) return FLAMIA_ERR_SHAPE;
    if (!x || !cu_seqlens || !out.codes || !out.scales) return FLAMIA_ERR_NULL;
    if (!aligned16(x) || !aligned16(out.codes) || !aligned16(out.nv)) return FLAMIA_ERR_ALIGN;
    QuantArgs a{};
    a.cu = cu_seqlens; a.ndocs = dims->ndocs; a.ttot = dims->ttot; a.d = dims->d;
    a.t[0] = QuantTensor{x, out.codes, out.scales, heads, 0, out.nv};
    a.ntensors = 1;
    hipError_t e = launch_quantize(a, (hipStream_t)stream);
    return e == hipSuccess ? FLAMIA_OK : hip_fail(e);
}

flamia_status_t flamia_fwd(const flamia_dims_t* dims, const flamia_opts_t* opts_in,
                           const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int32_t* cu_seqlens,
                           flamia_mx_t q_mx, flamia_mx_t k_mx, flamia_mx_t v_mx,
                           uint16_t* o, float* lse2, void* ws, size_t ws_bytes, void* stream) {
    flamia_status_t s = check_dims(dims);
    if (s != FLAMIA_OK) return s;
    const flamia_opts_t opts = resolve(opts_in);
    if ((s = check_fwd(dims, opts, q, k, v, cu_seqlens, q_mx, k_mx, v_mx, o, lse2)) != FLAMIA_OK) return s;
    const Layout w = layout(dims);
    if (!ws || ws_bytes < w.total) return FLAMIA_ERR_WORKSPACE;
    if (!aligned16(ws)) return FLAMIA_ERR_ALIGN;
    if (dims->ttot == 0) return FLAMIA_OK;
    return fwd_enqueue(dims, opts, q, k, v, cu_seqlens, q_mx, k_mx, v_mx, o, lse2, (uint8_t*)ws, w,
                       (hipStream_t)stream);
}

flamia_status_t flamia_fwd_noalloc(const flamia_dims_t* dims, const flamia_opts_t* opts_in,
                                   const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const int32_t* cu_seqlens,
                                   flamia_mx_t q_mx, flamia_mx_t k_mx, flamia_mx_t v_mx,
                                   uint16_t* o, float* lse2, void* stream) {
    flamia_status_t s = check_dims(dims);
    if (s != FLAMIA_OK) return s;
    const flamia_opts_t opts = resolve(opts_in);
    if ((s = check_fwd(dims, opts, q, k, v, cu_seqlens, q_mx, k_mx, v_mx, o, lse2)) != FLAMIA_OK) return s;
    const Layout w = layout(dims);
    // the forward uses the layout's leading part only: control block, tile
    // prefix and the query-major work list
    const size_t need = w.tiles_q + up256(sizeof(int4) * (size_t)w.max_tiles);
    if (need > kNoallocScratchBytes) {
        snprintf(g_last_error, sizeof g_last_error,
                 "flamia_fwd_noalloc: capacities need %zu bytes of scratch, the static array holds %zu",
                 need, kNoallocScratchBytes);
        return FLAMIA_ERR_WORKSPACE;
    }
    if (dims->ttot == 0) return FLAMIA_OK;
    uint8_t* base = nullptr;
    hipError_t e = scratch_of_current_device(&base);
    if (e != hipSuccess) return hip_fail(e);
    return fwd_enqueue(dims, opts, q, k, v, cu_seqlens, q_mx, k_mx, v_mx, o, lse2, base, w,
                       (hipStream_t)stream);
}

flamia_status_t flamia_bwd(const flamia_dims_t* dims, const flamia_opts_t* opts_in,
                           const uint16_t* d_o, const uint16_t* o, const float* lse2,
                           const int32_t* cu_seqlens,
                           flamia_mx_t q_mx, flamia_mx_t k_mx, flamia_mx_t v_mx,
                           uint16_t* dq, uint16_t* dk, uint16_t* dv,
                           void* ws, size_t ws_bytes, void* stream) {
    flamia_status_t s = check_dims(dims);
    if (s != FLAMIA_OK) return s;
    const flamia_opts_t opts = resolve(opts_in);
    if ((s = check_opts(&opts)) != FLAMIA_OK) return s;
    if (opts.fast_exp != 0) return FLAMIA_ERR_OPTS;     // inference-only exponential (Section 3.7)
    if (!d_o || !o || !lse2 || !cu_seqlens || !dq || !dk || !dv || !q_mx.codes || !q_mx.scales ||
        !k_mx.codes || !k_mx.scales || !v_mx.codes || !v_mx.scales)
        return FLAMIA_ERR_NULL;
    if (!aligned16(d_o) || !aligned16(o) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
        !mx_ok(q_mx) || !mx_ok(k_mx) || !mx_ok(v_mx))
        return FLAMIA_ERR_ALIGN;
    if ((s = check_nv(opts, q_mx, k_mx)) != FLAMIA_OK) return s;
    const Layout w = layout(dims);
    if (!ws || ws_bytes < w.total) return FLAMIA_ERR_WORKSPACE;
    if (!aligned16(ws)) return FLAMIA_ERR_ALIGN;
    if (dims->ttot == 0) return FLAMIA_OK;
    hipStream_t st = (hipStream_t)stream;
    uint8_t* base = (uint8_t*)ws;
    const int d = dims->d;
    uint8_t* oc = base + w.ocodes;
    uint8_t* os = base + w.oscales;
    float* dvec = (float*)(base + w.dvec);

    // the exact options rebuild dS in the dQ pass (its dS operand differs
    // from the dK one), so the store is not used
    const long ds_blocks = opts.exact ? 0 : w.ds_blocks;
    int32_t* ctrl = (int32_t*)(base + w.ctrl);
    int4* tiles_q = (int4*)(base + w.tiles_q);
    int4* tiles_k = (int4*)(base + w.tiles_k);
    int32_t* dboff = (int32_t*)(base + w.dboff);
    uint8_t* ds_codes = base + w.ds_codes;
    uint8_t* ds_scales = base + w.ds_scales;
    PlanArgs pa{cu_seqlens, dims->ndocs, dims->ttot, opts.cu_status, w.max_cost, (int32_t*)(base + w.prefix),
                ctrl, w.max_tiles, tiles_q, tiles_k, 1, dboff, ds_blocks};
    const float scale = scale_of(opts, d);
    BwdArgs ba;
    ba.qc = q_mx.codes; ba.qs = q_mx.scales;
    ba.kc = k_mx.codes; ba.ks = k_mx.scales;
    ba.vc = v_mx.codes; ba.vs = v_mx.scales;
    ba.oc = oc; ba.os = os;
    ba.lse2 = lse2; ba.dvec = dvec;
    ba.dk = dk; ba.dv = dv;
    ba.tiles = tiles_k; ba.ntiles = ctrl; ba.queue = ctrl + 2;
    ba.zero = (const uint8_t*)(ctrl + 32);
    ba.ttot = dims->ttot; ba.hq = dims->hq; ba.hkv = dims->hkv;
    ba.scale = scale;
    ba.c1 = scale * 1.4426950408889634f;
    ba.hadamard = opts.hadamard;
    ba.qn = opts.mixed ? q_mx.nv : nullptr;
    ba.kn = opts.mixed ? k_mx.nv : nullptr;
    ba.ds_codes = ds_codes; ba.ds_scales = ds_scales; ba.dboff = dboff; ba.ds_blocks = ds_blocks;
    ba.exact = opts.exact;
    ba.probe = probe_of(opts);
    DqArgs qd;
    qd.qc = q_mx.codes; qd.qs = q_mx.scales;
    qd.kc = k_mx.codes; qd.ks = k_mx.scales;
    qd.vc = v_mx.codes; qd.vs = v_mx.scales;
    qd.oc = oc; qd.os = os;
    qd.lse2 = lse2; qd.dvec = dvec;
    qd.dq = dq;
    qd.tiles = tiles_q; qd.ntiles = ctrl;
    qd.ttot = dims->ttot; qd.hq = dims->hq; qd.hkv = dims->hkv;
    qd.scale = scale;
    qd.c1 = ba.c1;
    qd.hadamard = opts.hadamard;
    qd.qn = ba.qn; qd.kn = ba.kn;
    qd.d_o = nullptr; qd.o = nullptr; qd.oc_w = nullptr; qd.os_w = nullptr; qd.dvec_w = nullptr;
    qd.ds_codes = ds_codes; qd.ds_scales = ds_scales; qd.dboff = dboff; qd.ds_blocks = ds_blocks;
    qd.exact = opts.exact;
    qd.probe = probe_of(opts);
    qd.probe.ds_zero = nullptr;
    PhaseMarks pm{opts, st};
    hipError_t e;
    const long gq = w.max_tiles * dims->hq, gk = w.max_tiles * dims->hkv;
    if (ds_blocks == 0) {
        // No dS store: the query-major dQ pass runs first and quantizes dO
        // itself (codes, scales and D for the key-major pass), so no separate
        // dO launch (Section 3.5.1 fused quantization).
        qd.d_o = d_o; qd.o = o; qd.oc_w = oc; qd.os_w = os; qd.dvec_w = dvec;
        if ((e = pm.mark()) != hipSuccess || (e = launch_plan(pa, st)) != hipSuccess) return hip_fail(e);
        if ((e = pm.mark()) != hipSuccess || (e = launch_dq(qd, d, gq, st)) != hipSuccess) return hip_fail(e);
        if ((e = pm.mark()) != hipSuccess || (e = launch_bwd(ba, d, gk, st)) != hipSuccess) return hip_fail(e);
    } else {
        // dS store: dO launch (codes, scales and D = dO~ . O, Section 3.5.1),
        // work lists, the key-major pass (which stores the dS-hat blocks),
        // then dQ from the store when the call fits it (decided on the
        // device; the other dQ kernel returns at once), else by rebuilding
        QuantArgs qa{};
        qa.cu = cu_seqlens; qa.ndocs = dims->ndocs; qa.ttot = dims->ttot; qa.d = d;
        qa.t[0] = QuantTensor{d_o, oc, os, dims->hq, 0, nullptr};
        qa.ntensors = 1;
        qa.o = o; qa.dvec = dvec;
        if ((e = pm.mark()) != hipSuccess || (e = launch_quantize(qa, st)) != hipSuccess) return hip_fail(e);
        if ((e = pm.mark()) != hipSuccess || (e = launch_plan(pa, st)) != hipSuccess) return hip_fail(e);
        if ((e = pm.mark()) != hipSuccess || (e = launch_bwd(ba, d, gk, st)) != hipSuccess) return hip_fail(e);
        if ((e = pm.mark()) != hipSuccess) return hip_fail(e);
        if ((e = launch_dq_store(qd, d, gq, st)) != hipSuccess) return hip_fail(e);
        if ((e = launch_dq(qd, d, gq, st)) != hipSuccess) return hip_fail(e);
    }
    e = pm.mark();
    return e == hipSuccess ? FLAMIA_OK : hip_fail(e);
}

}  // extern "C"
