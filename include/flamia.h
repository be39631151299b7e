/*
 * flamia.h -- C ABI of an MI355X (gfx950) library for microscaled (MXFP8, and
 * mixed NVFP4/FP8) causal flash attention over packed variable-length
 * documents: the training call (forward and backward) with the operand
 * quantization fused in; options for the Hadamard rotation, the inference
 * exponential and the exact options (per-token operand scales).
 *
 * Method: "FLAMIA: FLAsh MIcroscaling Attention for Fast and Causally Safe
 * Training on Blackwell".  Section numbers below refer to that paper.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are packed (Section 3.6.1): T = dims->ttot tokens, documents
 *    contiguous, document d occupies tokens [cu_seqlens[d], cu_seqlens[d+1]).
 *    cu_seqlens is an int32 device array of ndocs+1 entries, non-decreasing,
 *    cu_seqlens[0] = 0, cu_seqlens[ndocs] = ttot.  Empty documents are allowed
 *    (pad a list with trailing empty documents to reuse one captured graph for
 *    different document counts).  The library reads it only on the device and
 *    never synchronizes with the host.
 *  - Activations are bf16 (passed as uint16_t bit patterns), layout
 *    [T][heads][d], row-major, d contiguous.  Q, dO, O and dQ have hq heads;
 *    K, V, dK and dV have hkv heads; query head h reads key/value head
 *    h / (hq / hkv) (grouped-query attention).
 *  - Quantized operands (flamia_mx_t): E4M3 codes [T][heads][d] (uint8) and a
 *    dense per-token UE8M0 scale table [heads][T] (uint8, value 2^(byte-127)).
 *    Every token of a 32-token block, counted from its document's start,
 *    stores the block's exponent (Section 3.1 token-block scaling, Section
 *    3.6.1 dense per-token metadata); with opts.exact = 1 every token stores
 *    its own.  The exponent is the smallest e with max|x| <= 448 * 2^e over
 *    the block (or the token), so no code saturates (Section 3.2).
 *    On the mixed NVFP4/FP8 path (opts.mixed = 1, Section 3.4) Q and K also
 *    carry their NVFP4 form (Section 2, "Microscaling floating-point
 *    formats"): per token, one E4M3 scale s per 16 consecutive channels, the
 *    smallest E4M3 value with 6 s >= the group's largest magnitude (0 for an
 *    all-zero group), tensor scale 1, and each element the nearest E2M1 value
 *    of x / s (ties to the even code, saturating at 6).  The library stores
 *    each element's value E2M1 x s, which is exact in bf16, as bf16
 *    [T][heads][d] (`nv`); the score products read these, the gradient
 *    products the E4M3 token-block codes.
 *  - lse2 is the saved row statistic, [hq][T] fp32, base 2, in the domain of
 *    the scaled scores x = (q.k) * softmax_scale * log2(e):
 *    lse2_i = log2(sum_j 2^(x_ij)).  Natural-log LSE = lse2 * ln 2.
 *  - All pointers are device pointers unless stated otherwise, 16-byte
 *    aligned.  The caller owns every buffer; the library allocates nothing.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *    Calls on one stream are ordered.  Concurrent calls on different streams
 *    need separate workspaces and outputs.
 *  - Errors: arguments are validated on the host before anything is enqueued;
 *    on any error nothing is enqueued and a status code is returned.
 *    FLAMIA_ERR_HIP reports a failed launch (the HIP error text is kept per
 *    thread, see flamia_last_error()).  cu_seqlens is checked on the device
 *    by the work-list kernel of every flamia_fwd / flamia_bwd call: a
 *    malformed array (cu[0] != 0, a decreasing pair, a boundary outside
 *    [0, ttot], cu[ndocs] != ttot) makes the call do no attention work (its
 *    outputs are then unspecified, and nothing is read or written outside the
 *    tensors) and is reported through opts->cu_status.
 */
#ifndef FLAMIA_H
#define FLAMIA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLAMIA_ABI_VERSION 7

typedef enum {
    FLAMIA_OK = 0,
    FLAMIA_ERR_NULL = 1,      /* a required pointer is NULL */
    FLAMIA_ERR_SHAPE = 2,     /* d not 64/128, hq % hkv != 0, ttot > ttot_cap, ... */
    FLAMIA_ERR_ALIGN = 3,     /* a tensor pointer is not 16-byte aligned */
    FLAMIA_ERR_OPTS = 4,      /* c_log2 + tau > 8 (Section 3.4), key_tile != 128, ... */
    FLAMIA_ERR_WORKSPACE = 5, /* workspace NULL or smaller than flamia_workspace_bytes() */
    FLAMIA_ERR_HIP = 6        /* a kernel launch failed */
} flamia_status_t;

/* Host struct.  ttot_cap / ndocs_cap are the capacities the workspace is sized
 * for (Section 3.6.1: buffer capacities depend on T only); ttot <= ttot_cap,
 * ndocs <= ndocs_cap.
 * doclen_cap sizes the backward's dS store: the longest document the
 * workspace keeps the quantized dS blocks for (at most ttot_cap; 0 = no store).
 * With a store, the key-major pass writes each 32x32 dS-hat block once and the
 * dQ pass reads it back instead of rebuilding S, P and dP; whether a call's
 * documents fit is decided on the device, and a call that does not fit takes
 * the rebuilding dQ pass (same result, bit for bit). */
typedef struct {
    int32_t ttot, ttot_cap, ndocs, ndocs_cap, hq, hkv, d;
    int32_t doclen_cap;
} flamia_dims_t;

/* Host struct of numerical options.  A NULL opts pointer means the defaults
 * of flamia_default_opts(). */
typedef struct {
    int32_t c_log2;        /* P-hat = E4M3(2^c p) in the forward (Appendix B.1); default 4 */
    int32_t tau;           /* conditional rescale threshold (Appendix B.1); default 4;
                              c_log2 + tau <= 8 is enforced (2^(c+tau) <= 448) */
    int32_t key_tile;      /* B_c; only 128 is supported (Section 3.2, Figure 1) */
    int32_t rowsum;        /* 0: the forward row sum accumulates the unquantized p;
                              1: it accumulates the represented value(P-hat)/2^c */
    float softmax_scale;   /* <= 0 selects 1/sqrt(d) */
    int32_t hadamard;      /* 1: Q and K are rotated by the normalized d x d Hadamard
                              transform before quantization (Section 3.4, Appendix A.2):
                              the saved Q-hat / K-hat codes are those of the rotated rows
                              (fp32 butterfly, strides 1, 2, ..., d/2, then x fp32(1/sqrt(d))),
                              and flamia_bwd rotates dQ and dK back.  flamia_bwd must be
                              given the value flamia_fwd had.  0 (default): off */
    int32_t fast_exp;      /* inference only (Section 3.7, Appendix C.2): 0 (default) = exact
                              exponential; 5 or 8 = Schraudolph's approximation of
                              p' = 2^(x - m + c) for the keys of 5 (the paper's split) or all 8
                              of the 8 key-pair classes (class = bits 1, 3, 4 of the
                              document-local key index).  The forward's O and lse2 then come from
                              the approximate values; flamia_bwd returns FLAMIA_ERR_OPTS for a
                              non-zero value (the backward rebuilds P with the exact exponential);
                              it is offered on the MXFP8 path only (FLAMIA_ERR_OPTS with mixed) */
    int32_t mixed;         /* 1: the mixed NVFP4/FP8 path (Section 3.4): the scores (forward and
                              backward recomputation) come from the NVFP4 values of Q and K,
                              which flamia_fwd writes to q_mx.nv and k_mx.nv and flamia_bwd
                              reads from there (both must be non-NULL); every other product
                              is unchanged.  flamia_bwd must be given the value flamia_fwd had.
                              0 (default): the MXFP8 path */
    int32_t exact;         /* 1: the exact options (Appendix A.3, Section 4.5): every output of
                              query row i depends on tokens <= i only, bit for bit.  Q, K, V
                              and dO get one exponent per token (the scale table then differs
                              between the tokens of a block).  A product that contracts over
                              tokens carries the other operand's token exponent in its 8-bit
                              entry, relative to a shared exponent: P-hat takes V's, relative
                              to the largest V exponent of the visible keys of the 32-key
                              block; the dV operand takes dO's, relative to the largest of
                              the 32-query block; dK's dS takes Q's, with one exponent per
                              32x32 block; dQ's dS takes K's, with one exponent per query row
                              and 32-key block (the per-query-row dS exponent).  The backward
                              does not use the dS store (doclen_cap is ignored).  Not with
                              rowsum, fast_exp or mixed (FLAMIA_ERR_OPTS).  flamia_bwd must be
                              given the value flamia_fwd had.  0 (default): token blocks */
    /* Optional phase timing: when phase_events is non-NULL it points to
     * n_events hipEvent_t handles (created by the caller); the call records
     * event i on `stream` before its i-th internal launch and the next one
     * after its last launch, as far as n_events allows; NULL entries are
     * skipped (no event recorded there).  flamia_fwd has 3 phases (quantize
     * Q, K and V in one launch; work list; forward kernel); flamia_bwd has 4
     * with a dS store (doclen_cap > 0: quantize dO with D; work lists;
     * key-major dK/dV kernel; query-major dQ kernels) and 3 without one
     * (work lists; query-major dQ kernel, which also quantizes dO and
     * computes D; key-major dK/dV kernel).  NULL disables it. */
    void **phase_events;
    int32_t n_events;
    /* Optional diagnostics; NULL pointers (the defaults) switch them off.
     * cu_status: device int32, written by every flamia_fwd / flamia_bwd call:
     *   0 when cu_seqlens is well formed (Section 3.6.1 packed layout), else
     *   bit 0 (cu[0] != 0) | bit 1 (a decreasing pair) | bit 2 (a boundary
     *   outside [0, ttot] or cu[ndocs] != ttot).
     * ds_zero_count: device uint64, flamia_bwd adds the number of dS entries
     *   that are nonzero but quantize to a zero dS-hat code (the fraction of
     *   such entries tracks degradation, Sections 3.3 and 4.5); the caller
     *   zeroes it.
     * probe_scores: device fp32 [3][128][probe_keys]: the raw scores
     *   S = q . k (block scales applied, before softmax_scale) of the 128
     *   queries that start at packed token probe_q0 (a query tile: probe_q0 -
     *   probe_doc_start a multiple of 128) of the document that starts at
     *   packed token probe_doc_start, query head probe_head, document-local
     *   keys 0 .. probe_keys - 1: table 0 as flamia_fwd computes them, 1 as
     *   the dQ pass of flamia_bwd rebuilds them (without a dS store), 2 as
     *   the dK/dV pass does (Section 3.3: the backward reproduces the
     *   forward's scores).  Entries of keys after the query, or outside the
     *   document, are not written.
     * Diagnostics run separate kernel instantiations, on the MXFP8 path with
     * the exact exponential only (FLAMIA_ERR_OPTS with mixed, exact or
     * fast_exp). */
    int32_t *cu_status;
    uint64_t *ds_zero_count;
    float *probe_scores;
    int32_t probe_doc_start, probe_q0, probe_head, probe_keys;
} flamia_opts_t;

typedef struct {
    uint8_t *codes;        /* [T][heads][d] E4M3 */
    uint8_t *scales;       /* [heads][T] UE8M0 */
    uint16_t *nv;          /* [T][heads][d] bf16 NVFP4 values (mixed path, Q and K only);
                              ignored (may be NULL) elsewhere */
} flamia_mx_t;

flamia_opts_t flamia_default_opts(void);
int flamia_abi_version(void);
const char *flamia_status_str(flamia_status_t s);
/* Text of the last HIP error seen by a call on this host thread ("" if none). */
const char *flamia_last_error(void);

/* Bytes of device workspace that flamia_fwd / flamia_bwd need for these
 * capacities; depends on ttot_cap, ndocs_cap, doclen_cap, d and the head
 * counts only.  ttot and ndocs are ignored.  Returns 0 if dims is NULL or the
 * head layout or a capacity is invalid.  With doclen_cap > 0 the dS store takes
 * hq * B * 1025 bytes, B = (ttot_cap / 32 + ndocs_cap) * (ceil(doclen_cap / 32) + 1) / 2
 * (a bound on the number of 32x32 causal blocks per head). */
size_t flamia_workspace_bytes(const flamia_dims_t *dims, const flamia_opts_t *opts);

/*
 * flamia_quantize -- token-block quantization of one packed tensor
 * (Section 3.1, Section 3.2 rounded-up exponent, Section 3.6.1 document-local
 * blocks).
 *   x      : bf16 [ttot][heads][d] (input)
 *   out    : codes [ttot][heads][d] and scales [heads][ttot] (outputs); when
 *            out.nv is non-NULL also the NVFP4 values of the same rows (the
 *            mixed path's form, see the conventions above)
 * No workspace.  heads must be >= 1; only dims->ttot, ndocs and d are read.
 * The blocks are always 32 tokens and no rotation is applied: the per-token
 * exponents of the exact options and the rotated Q and K of the Hadamard
 * option are written by flamia_fwd into the q_mx, k_mx, v_mx it returns.
 */
flamia_status_t flamia_quantize(const flamia_dims_t *dims, int32_t heads, const uint16_t *x,
                                const int32_t *cu_seqlens, flamia_mx_t out, void *stream);

/*
 * flamia_fwd -- forward of the training call (Section 2 equations for S, P, O;
 * Section 3.5.1 fused quantization; Appendix B.1 P-hat with the fixed 2^c
 * factor and the conditional running maximum; Section 3.6.2 GPU-built,
 * cost-sorted work list).
 *   q, k, v            : bf16 inputs
 *   q_mx, k_mx, v_mx   : outputs -- the quantized operands, which the caller
 *                        keeps for flamia_bwd (the backward rebuilds the scores
 *                        from exactly these codes, Section 3.3); with
 *                        opts.mixed = 1 also q_mx.nv and k_mx.nv
 *   o                  : bf16 output [ttot][hq][d]
 *   lse2               : fp32 output [hq][ttot]
 *   ws / ws_bytes      : workspace of at least flamia_workspace_bytes()
 * Deterministic: the same inputs give bitwise-identical outputs (Appendix B.5).
 */
flamia_status_t flamia_fwd(const flamia_dims_t *dims, const flamia_opts_t *opts,
                           const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const int32_t *cu_seqlens,
                           flamia_mx_t q_mx, flamia_mx_t k_mx, flamia_mx_t v_mx,
                           uint16_t *o, float *lse2, void *ws, size_t ws_bytes, void *stream);

/*
 * flamia_fwd_noalloc -- flamia_fwd without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments (minus
 * ws / ws_bytes), kernels and results as flamia_fwd, bit for bit.  The
 * forward's control block, tile prefix and work list live in a static device
 * array of 4 MiB instead, one per GPU the library runs on, held until the
 * process ends.  Capacities whose work list does not fit it (ndocs_cap + 1
 * prefix entries of 4 bytes and ttot_cap / 128 + ndocs_cap + 1 tiles of 16
 * bytes, 256-byte aligned: about 200,000 documents at the largest ttot_cap)
 * return FLAMIA_ERR_WORKSPACE, with the sizes in flamia_last_error().
 * Nothing is allocated and nothing synchronizes with the host.  Every call on
 * a GPU uses that GPU's one array, which keeps the last call's contents
 * (nothing in it needs to start at zero): calls that overlap on one GPU (on
 * different streams or host threads) race, so order them on one stream.
 */
flamia_status_t flamia_fwd_noalloc(const flamia_dims_t *dims, const flamia_opts_t *opts,
                                   const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                   const int32_t *cu_seqlens,
                                   flamia_mx_t q_mx, flamia_mx_t k_mx, flamia_mx_t v_mx,
                                   uint16_t *o, float *lse2, void *stream);

/*
 * flamia_bwd -- backward of the training call (Section 2 equations for dV,
 * dP, dS, dQ, dK; Section 3.3: scores rebuilt from the forward's quantized
 * Q/K, the same tiling, diagonal handling, exponential and saved row
 * statistic; D_i = dO~_i . O_i from the quantized dO and the bf16 output;
 * dS quantized on 32x32 document-local blocks; Appendix B.1: the dV operand
 * is E4M3(2^8 P) with no stored scale).
 *   d_o                : bf16 [ttot][hq][d] (input)
 *   o, lse2            : the forward's outputs (inputs here)
 *   q_mx, k_mx, v_mx   : the forward's quantized operands (inputs here)
 *   dq                 : bf16 output [ttot][hq][d]
 *   dk, dv             : bf16 outputs [ttot][hkv][d] (summed over the query
 *                        heads of each group)
 *   ws / ws_bytes      : workspace (holds the dO codes and scales, D, the work
 *                        lists and, with doclen_cap > 0, the dS store)
 * A key-major pass accumulates dK and dV; a query-major pass accumulates dQ,
 * either from the dS-hat blocks the key-major pass stored or, without a store
 * (or when the call's documents do not fit it), by rebuilding the same dS-hat
 * payload bit for bit.  Without a store the query-major pass runs first and
 * quantizes dO itself (same codes, scales and D as the separate quantization
 * launch that precedes the key-major pass when a store is configured).  Each output element is owned by one workgroup, so the
 * backward is deterministic (no atomics).
 */
flamia_status_t flamia_bwd(const flamia_dims_t *dims, const flamia_opts_t *opts,
                           const uint16_t *d_o, const uint16_t *o, const float *lse2,
                           const int32_t *cu_seqlens,
                           flamia_mx_t q_mx, flamia_mx_t k_mx, flamia_mx_t v_mx,
                           uint16_t *dq, uint16_t *dk, uint16_t *dv,
                           void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* FLAMIA_H */
