/*
 * Reference oracle for MXFP8 causal packed-document attention (forward and
 * backward, quantization included).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the HIP
 * library.
 *
 * Source of the method: "FLAMIA: FLAsh MIcroscaling Attention for Fast and
 * Causally Safe Training on Blackwell" (arXiv 2611.03344).  Every step below
 * names the section it follows.  All arithmetic is IEEE binary64; the only
 * roundings are the ones the method itself prescribes (E4M3 codes, bf16
 * outputs, the fp32 log-sum-exp that the forward saves).
 *
 * Readings taken where the paper is silent (each also listed in the design
 * notes of the repository):
 *   - scale exponent "rounded up" = the smallest e with amax <= 448 * 2^e;
 *     an all-zero block gets e = -127 (its codes are zero for any e);
 *   - token blocks are anchored at the document start;
 *   - key tiles of B_c keys are visited in ascending order, anchored at the
 *     document start; the running maximum is replaced when the tile maximum
 *     exceeds it by more than tau (or on the first tile);
 *   - the forward row sum accumulates the unquantized p (FlashAttention
 *     convention); rowsum = 1 accumulates the represented value(P-hat)/2^c;
 *   - the saved row statistic is lse2 = m + log2(l) in fp32, and the backward
 *     rebuilds P = 2^(x - lse2) with the same scores x;
 *   - dS is quantized before the 1/sqrt(d) factor, which multiplies dQ and dK
 *     after accumulation;
 *   - D_i = dO~_i . O_i uses the bf16 output that the forward returns;
 *   - GQA: query head h reads key/value head h / (Hq/Hkv); dK and dV sum over
 *     the heads of the group before rounding;
 *   - the optional Hadamard rotation of Q and K is computed in fp32 by the
 *     butterfly in a fixed stage order (its values decide codes), and the
 *     gradients are rotated back in binary64;
 *   - the optional inference exponential (Schraudolph) is evaluated bit for
 *     bit on the fp32 argument, for the keys of k of every 8 key-pair classes;
 *   - the mixed path's NVFP4 Q and K: one E4M3 scale per 16 channels of each
 *     token, rounded up (the smallest with 6 s >= the group maximum), tensor
 *     scale 1 (a constant: no statistic over the sequence), E2M1 codes to
 *     nearest even; they serve the scores only;
 *   - the exact options: per-token exponents (rounded up) for Q, K, V and dO;
 *     a product that contracts over tokens takes the other operand's token
 *     exponent into its 8-bit entry, relative to a shared exponent: the
 *     largest V exponent of the visible keys of the 32-key block (P-hat), the
 *     largest dO exponent of the 32-query block (P-hat_b), the 32x32 block
 *     exponent of dS 2^eQ (dK), and one exponent per query row and 32-key
 *     block of dS 2^eK (dQ).
 *
 * Parity: every exported function is pinned by CPU tests against definitions
 * that do not go through this file (a library FP8 codec, brute-force nearest
 * search, exact attention written as dense matrix algebra, finite differences,
 * closed forms of single-document calls, and the causal and
 * document-isolation invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_BOUND 2
#define ORC_ERR_NOMEM 3

enum { QUANT_CEIL = 0, QUANT_FLOOR = 1, QUANT_NONE = 2 };

typedef struct {
    int32_t ttot, ndocs, hq, hkv, d;
    int32_t c_log2;       /* P-hat is E4M3(2^c p) (Appendix B.1) */
    int32_t tau;          /* conditional rescale threshold (Appendix B.1) */
    int32_t key_tile;     /* B_c (Section 3.2, Figure 1: 128) */
    int32_t quant;        /* QUANT_CEIL / QUANT_FLOOR / QUANT_NONE */
    int32_t rowsum;       /* 0: unquantized p, 1: represented value(P-hat)/2^c */
    double softmax_scale; /* <= 0 selects 1/sqrt(d) */
    int32_t unsafe_bound; /* 1 skips the c + tau <= 8 check (negative tests only) */
    /* Hadamard rotation of Q and K before quantization (Section 3.4 and
     * Appendix A.2): 0 off, 1 on. */
    int32_t hadamard;
    /* Inference-only exponential (Section 3.7, Appendix C.2): 0 = exact;
     * k in 1..8 = Schraudolph's approximation for the forward's p' of keys
     * whose pair class (bits 1, 3, 4 of the document-local key index) is
     * below k, i.e. k of every 8 key pairs.  Forward only. */
    int32_t fast_exp;
    /* Mixed NVFP4/FP8 path (Section 3.4): 1 = the scores S = Q K^T (forward
     * and backward) use NVFP4 Q and K (E2M1 codes, one E4M3 scale per 16
     * channels of each token, tensor scale 1); dQ = dS K and dK = dS^T Q use
     * the E4M3 token-block Q and K as in the MXFP8 path. */
    int32_t mixed;
    /* Exact options (Appendix A.3; Section 4.5): 1 = every operand of the
     * products (Q, K, V and dO) carries one exponent per token instead of
     * per 32-token block, and the dS operand of dQ carries one exponent per
     * (query row, 32-key block) taken over the row's visible keys.  The
     * products that contract over tokens (P-hat V, dV, dK, dQ) take the
     * other operand's per-token exponent into the 8-bit P-hat, P-hat_b or dS
     * entry, relative to a shared exponent of the 32-token block (see
     * fwd_row and unit_run).  Every output of query row i then depends on
     * tokens <= i only.  Not combined with rowsum = 1, fast_exp or mixed. */
    int32_t exact;
    /* Test hook, not part of the method (zero by default): a model of a
     * kernel's dot-product error, see score_dot below. */
    double dot_noise;
    int64_t noise_seed;
} orc_params;

/* ---------------------------------------------------------------------------
 * Scalar formats.
 * E4M3 (OCP "E4M3FN", the 8-bit code of Section 2, "Microscaling
 * floating-point formats"): 1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN, so the
 * largest finite value is 1.75 * 2^8 = 448 (Section 3.2).
 * ------------------------------------------------------------------------- */
double orc_e4m3_value(uint8_t code)
{
    int s = code >> 7, ef = (code >> 3) & 15, m = code & 7;
    double v;
    if (ef == 15 && m == 7) return NAN;
    if (ef == 0) v = ldexp((double)m, -9);
    else v = ldexp((double)(8 + m), ef - 10);
    return s ? -v : v;
}

/* Round-to-nearest-even into E4M3 (Appendix A.5: every element rounds to
 * nearest).  Magnitudes that round above 448 saturate to 448: that is the
 * clamping of the reference microscaling conversion that Section 3.2
 * describes; the causally safe exponent never lets it happen. */
uint8_t orc_e4m3_encode(double y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs(y);
    int ex, ef;
    double f, n;
    if (isnan(y)) return 0x7F;
    if (a < 0x1p-6) {                 /* subnormal range: quantum 2^-9 */
        n = nearbyint(a * 512.0);     /* 0..8; 8 is the smallest normal */
        return (uint8_t)(sign | (uint8_t)n);
    }
    f = frexp(a, &ex);                /* a = f 2^ex, f in [0.5, 1) */
    n = nearbyint(f * 16.0);          /* mantissa with the hidden bit, 8..16 */
    ef = ex - 1;                      /* unbiased exponent of a */
    if (n == 16.0) { n = 8.0; ef += 1; }
    if (ef > 8 || (ef == 8 && n > 14.0)) return (uint8_t)(sign | 0x7E);
    return (uint8_t)(sign | ((ef + 7) << 3) | ((int)n - 8));
}

/* E2M1 (OCP FP4, the 4-bit element of NVFP4, Section 2 "Microscaling
 * floating-point formats"): 1 sign, 2 exponent bits, 1 mantissa bit; the
 * magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
static const double e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(uint8_t code)
{
    double v = e2m1_mag[code & 7];
    return (code & 8) ? -v : v;
}

/* Round to the nearest E2M1 magnitude, ties to the even code (the one whose
 * mantissa bit is 0); magnitudes above 6 saturate to 6. */
uint8_t orc_e2m1_encode(double y)
{
    uint8_t sign = signbit(y) ? 8 : 0;
    double a = fabs(y);
    int best = 0;
    for (int k = 1; k < 8; ++k) {
        double dk = fabs(a - e2m1_mag[k]), db = fabs(a - e2m1_mag[best]);
        if (dk < db || (dk == db && (k & 1) == 0)) best = k;
    }
    return (uint8_t)(sign | best);
}

/* NVFP4 scale of a group of 16 whose largest magnitude is amax: the smallest
 * E4M3 value s with 6 s >= amax (rounded up, like the MX exponents of
 * Section 3.2, so that no element is clamped), 0 for an all-zero group; a
 * group above 6 x 448 gets 448 and saturates.  Returns the E4M3 code. */
uint8_t orc_nvfp4_scale(double amax)
{
    for (int c = 0; c <= 0x7E; ++c)
        if (6.0 * orc_e4m3_value((uint8_t)c) >= amax) return (uint8_t)c;
    return 0x7E;
}

/* NVFP4 values of one row of d channels (d a multiple of 16): groups of 16
 * consecutive channels, one E4M3 scale each, tensor scale 1; each element
 * becomes value(E2M1(x / s)) * s.  The row never shares a statistic with
 * another token. */
static void nvfp4_row(const double *x, int d, double *out)
{
    for (int g0 = 0; g0 < d; g0 += 16) {
        double amax = 0.0, s;
        for (int k = g0; k < g0 + 16; ++k)
            if (fabs(x[k]) > amax) amax = fabs(x[k]);
        s = orc_e4m3_value(orc_nvfp4_scale(amax));
        for (int k = g0; k < g0 + 16; ++k)
            out[k] = s == 0.0 ? 0.0 : orc_e2m1_value(orc_e2m1_encode(x[k] / s)) * s;
    }
}

/* Shared block exponent for a block whose largest magnitude is amax.
 * rule 0 (Section 3.2, "round each scale's exponent up"): the smallest e with
 *   amax <= 448 * 2^e, so the scaled maximum never exceeds the largest code.
 * rule 1 (the reference conversion quoted in Section 3.2):
 *   floor(log2 amax) - e_max with e_max = 8; the scaled maximum may exceed 448.
 * The result is clamped to the UE8M0 range [-127, 127]; amax = 0 gives -127. */
int orc_scale_exp(double amax, int rule)
{
    int ex, e;
    double f;
    if (!(amax > 0.0)) return -127;
    f = frexp(amax, &ex);             /* amax = (2f) 2^(ex-1), 2f in [1, 2) */
    e = (ex - 1) - 8;
    if (rule == 0 && 2.0 * f > 1.75) e += 1;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* bf16 round-to-nearest-even directly from binary64 (one rounding). */
uint16_t orc_double_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x), r;
    int ex;
    float fl;
    uint32_t u;
    if (isnan(x)) return 0x7FC0;
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    if (a >= 0x1p-126) {
        double f = frexp(a, &ex);             /* a = f 2^ex */
        r = ldexp(nearbyint(ldexp(f, 8)), ex - 8);
    } else {
        r = ldexp(nearbyint(ldexp(a, 133)), -133);
    }
    if (r >= 0x1p128) return (uint16_t)(sign | 0x7F80);
    fl = (float)r;                            /* exact */
    memcpy(&u, &fl, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* ---------------------------------------------------------------------------
 * Hadamard rotation (Section 3.4 "a normalized Hadamard transform ... mixes
 * the head channels of both Q and K before quantization"; Appendix A.2).
 * The rotated values decide E4M3 codes, so their precision is part of the
 * definition; the reading taken: the bf16 row is widened to fp32, transformed
 * by the fast Walsh-Hadamard butterfly in fp32 (stages of stride 1, 2, 4, ...,
 * d/2; each butterfly maps (a, b) at channels (j, j + h) to (a + b, a - b)),
 * then multiplied by fp32(1/sqrt(d)) (exactly 2^-3 at d = 64, the nearest
 * fp32 to 2^-3.5 at d = 128).  The butterfly computes x H with the Sylvester
 * matrix H[i][j] = (-1)^popcount(i & j), so the rotation is x H / sqrt(d),
 * orthogonal and its own inverse.
 * ------------------------------------------------------------------------- */
void orc_hadamard_f32(const uint16_t *x, int d, float *y)
{
    for (int i = 0; i < d; ++i) y[i] = (float)orc_bf16_to_double(x[i]);
    for (int h = 1; h < d; h <<= 1)
        for (int i = 0; i < d; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                float a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
    const float rs = sqrtf(1.0f / (float)d);
    for (int i = 0; i < d; ++i) y[i] = y[i] * rs;
}

/* The same rotation of a binary64 row, in binary64 (used to rotate the
 * gradients back: dQ = dQ' H / sqrt(d), dK = dK' H / sqrt(d)). */
static void hadamard_f64(double *y, int d)
{
    for (int h = 1; h < d; h <<= 1)
        for (int i = 0; i < d; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                double a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
    const double rs = 1.0 / sqrt((double)d);
    for (int i = 0; i < d; ++i) y[i] *= rs;
}

/* ---------------------------------------------------------------------------
 * Token-block quantizer (Section 3.1 "token-block scaling"; Section 3.6.1,
 * blocks and statistics kept inside document boundaries).
 * One document slice of L tokens, d channels, rows `rstride` elements apart;
 * rot = 1 quantizes the Hadamard-rotated rows instead of the bf16 rows.
 * Blocks are [blk b, min(blk b + blk, L)) from the document start, blk = 32
 * (token blocks) or 1 (the exact options' per-token exponents); one exponent
 * per block over all d channels; every token of the block stores it, in
 * scales (UE8M0 byte) and ex (the exponent itself).
 * deq (L x d, dense) receives value(code) * 2^e, or the (rotated) values
 * themselves when quant is QUANT_NONE.  codes/scales/nv/ex may be NULL.
 * Returns 0, or ORC_ERR_NOMEM.
 * ------------------------------------------------------------------------- */
static int tbq_slice(const uint16_t *x, long rstride, int L, int d, int quant, int rot,
                     double *deq, uint8_t *codes, long cstride, uint8_t *scales, double *nv,
                     int blk, int *ex)
{
    double *xv = malloc(sizeof(double) * (size_t)L * d);
    float *row = malloc(sizeof(float) * (size_t)d);
    if (!xv || !row) { free(xv); free(row); return ORC_ERR_NOMEM; }
    for (int t = 0; t < L; ++t) {
        if (rot) {
            orc_hadamard_f32(x + (long)t * rstride, d, row);
            for (int k = 0; k < d; ++k) xv[(long)t * d + k] = (double)row[k];
        } else {
            for (int k = 0; k < d; ++k) xv[(long)t * d + k] = orc_bf16_to_double(x[(long)t * rstride + k]);
        }
    }
    /* the NVFP4 values of the same (rotated) rows, for the mixed path */
    if (nv)
        for (int t = 0; t < L; ++t) nvfp4_row(xv + (long)t * d, d, nv + (long)t * d);
    for (int b0 = 0; b0 < L; b0 += blk) {
        int b1 = b0 + blk < L ? b0 + blk : L;
        double amax = 0.0;
        int e = 0;
        for (int t = b0; t < b1; ++t)
            for (int k = 0; k < d; ++k) {
                double v = fabs(xv[(long)t * d + k]);
                if (v > amax) amax = v;
            }
        if (quant != QUANT_NONE) e = orc_scale_exp(amax, quant == QUANT_FLOOR ? 1 : 0);
        for (int t = b0; t < b1; ++t) {
            if (scales) scales[t] = (uint8_t)(e + 127);
            if (ex) ex[t] = e;
            for (int k = 0; k < d; ++k) {
                double v = xv[(long)t * d + k];
                if (quant == QUANT_NONE) {
                    deq[(long)t * d + k] = v;
                } else {
                    uint8_t c = orc_e4m3_encode(ldexp(v, -e));
                    if (codes) codes[(long)t * cstride + k] = c;
                    deq[(long)t * d + k] = ldexp(orc_e4m3_value(c), e);
                }
            }
        }
    }
    free(xv);
    free(row);
    return ORC_OK;
}

static int check_cu(const orc_params *p, const int32_t *cu)
{
    if (!cu || p->ndocs < 0 || cu[0] != 0 || cu[p->ndocs] != p->ttot) return 0;
    for (int i = 0; i < p->ndocs; ++i)
        if (cu[i + 1] < cu[i]) return 0;
    return 1;
}

/* codes [ttot][heads][d], scales [heads][ttot] (UE8M0 byte = e + 127). */
int orc_quantize(const orc_params *p, int heads, const uint16_t *x, const int32_t *cu,
                 uint8_t *codes, uint8_t *scales)
{
    int d = p->d, nd = p->ndocs;
    long nunits = (long)nd * heads;
    int err = ORC_OK;
    if (!x || !codes || !scales || heads <= 0 || d <= 0 || !check_cu(p, cu)) return ORC_ERR_ARG;
    if (p->quant == QUANT_NONE) return ORC_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < nunits; ++u) {
        int doc = (int)(u / heads), h = (int)(u % heads);
        int base = cu[doc], L = cu[doc + 1] - cu[doc];
        double *deq;
        if (L == 0) continue;
        deq = (double *)malloc(sizeof(double) * (size_t)L * d);
        if (!deq) { err = ORC_ERR_NOMEM; continue; }
        if (tbq_slice(x + ((long)base * heads + h) * d, (long)heads * d, L, d, p->quant, p->hadamard != 0,
                      deq, codes + ((long)base * heads + h) * d, (long)heads * d,
                      scales + (long)h * p->ttot + base, 0, p->exact ? 1 : 32, 0) != ORC_OK)
            err = ORC_ERR_NOMEM;
        free(deq);
    }
    return err;
}


/* ---------------------------------------------------------------------------
 * Attention.  One unit = one document x one key/value head (all G query heads
 * of the group), so every statistic stays inside the document.
 * ------------------------------------------------------------------------- */
typedef struct {
    double *o64; uint16_t *o16; float *lse2; double *dvec;
    double *dq64, *dk64, *dv64; uint16_t *dq16, *dk16, *dv16;
    int64_t *stats;   /* [0] P-hat entries that saturated, [1] dS entries
                         (causal, in-document), [2] nonzero dS quantized to 0 */
} orc_out;

static double dotd(const double *a, const double *b, int d)
{
    double s = 0.0;
    for (int k = 0; k < d; ++k) s += a[k] * b[k];
    return s;
}

/* splitmix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", 2014) */
static uint64_t mix64(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* The dot products that a kernel computes on its matrix cores: the scores
 * q_i . k_j (forward and backward) and dP_ij = dO_i . v_j.  With dot_noise = 0
 * (the default, and the method) this is the exact binary64 dot product.
 * Test hook: with dot_noise > 0 the result gets u * dot_noise * max_k |a_k b_k|
 * added, u in [-1, 1) from a hash of (noise_seed, query head h, packed token
 * indices ti and tj, which product), so a forward score and its backward
 * recomputation carry the same error.  It models a matrix core whose reduction
 * is exact only to a fraction of its largest single product; the tests use it
 * to check that the GPU comparison tolerates that much and no more. */
static double score_dot(const orc_params *p, const double *a, const double *b, int d,
                        int h, long ti, long tj, int which)
{
    double s = dotd(a, b, d);
    if (p->dot_noise > 0.0) {
        double mp = 0.0, u;
        uint64_t z;
        for (int k = 0; k < d; ++k) {
            double t = fabs(a[k] * b[k]);
            if (t > mp) mp = t;
        }
        z = mix64((uint64_t)p->noise_seed ^ mix64(((uint64_t)h << 2) | (uint64_t)which));
        z = mix64(z ^ mix64((uint64_t)ti) ^ (mix64((uint64_t)tj) << 1));
        u = (double)(z >> 11) * 0x1p-52 - 1.0;
        s += u * p->dot_noise * mp;
    }
    return s;
}


/* ---------------------------------------------------------------------------
 * Schraudolph's exponential (Section 3.7; Appendix C.2).  One fp32 fused
 * multiply-add t = 2^7 y + K, K = fp32(1.5 * 2^23 + 2^7 (127 - sigma)),
 * sigma = 0.0573: adding 1.5 * 2^23 rounds 2^7 y to an integer held in the
 * low mantissa bits of t, and those low 16 bits, read as a bf16 pattern,
 * are 2^floor(z) (1 + {z}) with z = y - sigma' (7 fraction bits; K is an
 * integer, so the offset in effect is sigma' = 7/128).  The pattern is
 * moved to the high half of a float and clamped at zero.  The argument y is
 * the fp32 value the kernel exponentiates.
 * ------------------------------------------------------------------------- */
float orc_schraudolph_exp2(float y)
{
    const float K = (float)(12582912.0 + 128.0 * (127.0 - 0.0573));
    float t = fmaf(128.0f, y, K);
    uint32_t bits;
    int32_t hi;
    float v;
    memcpy(&bits, &t, 4);
    hi = (int32_t)(bits << 16);
    if (hi < 0) hi = 0;
    memcpy(&v, &hi, 4);
    return v;
}

/* pair class of a document-local key: bits 1, 3 and 4 of its index */
static int key_pair_class(int j)
{
    return ((j >> 1) & 1) | (((j >> 3) & 1) << 1) | (((j >> 4) & 1) << 2);
}

/* Forward for query row i of a document (Section 2 equations for S, P, O;
 * Appendix B.1 for the fixed 2^c factor and the conditional running maximum).
 * Keys j <= i in tiles of B_c keys from the document start, ascending; x_ij =
 * (q_i . k_j) s log2(e).  h and tok0 (the document's first packed token) only
 * key the test hook of score_dot. */
static void fwd_row(const orc_params *p, int h, long tok0, int i, const double *qi, const double *Kt,
                    const double *Vt, const int *ev, double c1, double *acc, double *x,
                    double *o_out, double *lse_out, int64_t *sat)
{
    int d = p->d, B = p->key_tile, quant = p->quant;
    double m = -INFINITY, l = 0.0;
    int eblk = -1, E = 0;      /* exact options: key block of E, and E */
    double two_c = ldexp(1.0, p->c_log2);
    for (int k = 0; k < d; ++k) acc[k] = 0.0;
    for (int j0 = 0; j0 <= i; j0 += B) {
        int j1 = j0 + B <= i + 1 ? j0 + B : i + 1;
        double mu = -INFINITY;
        for (int j = j0; j < j1; ++j) {
            x[j - j0] = score_dot(p, qi, Kt + (long)j * d, d, h, tok0 + i, tok0 + j, 0) * c1;
            if (x[j - j0] > mu) mu = x[j - j0];
        }
        /* replace the running maximum on the first tile, or when the tile's
         * maximum exceeds it by more than tau */
        if (m == -INFINITY || mu - m > (double)p->tau) {
            double alpha = (m == -INFINITY) ? 0.0 : exp2(m - mu);
            l *= alpha;
            for (int k = 0; k < d; ++k) acc[k] *= alpha;
            m = mu;
        }
        for (int j = j0; j < j1; ++j) {
            const int approx = p->fast_exp > 0 && quant != QUANT_NONE && key_pair_class(j) < p->fast_exp;
            /* approximated: p' = 2^c p is formed from the fp32 argument x - m + c */
            double pj = approx ? (double)orc_schraudolph_exp2((float)(x[j - j0] - m + p->c_log2)) / two_c
                               : exp2(x[j - j0] - m), w;
            const double *vj = Vt + (long)j * d;
            if (quant == QUANT_NONE) {
                w = pj;
                l += pj;
            } else {
                double y = pj * two_c, f = 1.0;
                uint8_t code;
                if (ev) {
                    /* Exact options (Appendix A.3): V~_j carries its own
                     * exponent e_j.  The entry is taken relative to E, the
                     * largest exponent of the keys j' <= i in j's 32-key
                     * block, so that the product applies one factor 2^E per
                     * (query, key block): y = 2^c p 2^(e_j - E), and
                     * value(code) 2^(E - e_j) multiplies V~_j.  E never looks
                     * past key i. */
                    if ((j >> 5) != eblk) {
                        int jb1 = (j | 31) < i ? (j | 31) : i;
                        eblk = j >> 5;
                        E = ev[j & ~31];
                        for (int jj = (j & ~31) + 1; jj <= jb1; ++jj)
                            if (ev[jj] > E) E = ev[jj];
                    }
                    f = ldexp(1.0, ev[j] - E);
                    y *= f;
                }
                if (y > 448.0) (*sat)++;
                code = orc_e4m3_encode(y);
                w = orc_e4m3_value(code) / f;
                l += (p->rowsum == 1) ? w / two_c : pj;
            }
            for (int k = 0; k < d; ++k) acc[k] += w * vj[k];
        }
    }
    {
        double den = (quant == QUANT_NONE) ? l : l * two_c;
        for (int k = 0; k < d; ++k) o_out[k] = acc[k] / den;
        *lse_out = m + log2(l);
    }
}

static void unit_run(const orc_params *p, int doc, int g, const int32_t *cu,
                     const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const uint16_t *dout, const orc_out *out, int *err)
{
    const int d = p->d, hq = p->hq, hkv = p->hkv, G = hq / hkv, quant = p->quant;
    const int base = cu[doc], L = cu[doc + 1] - cu[doc];
    const double s = p->softmax_scale > 0 ? p->softmax_scale : 1.0 / sqrt((double)d);
    const double c1 = s * (1.0 / log(2.0));     /* s * log2(e) */
    const int need_bwd = dout != NULL;
    double *Kt = 0, *Vt = 0, *Qt = 0, *dOt = 0, *O = 0, *lse = 0, *Dv = 0;
    /* mixed path: NVFP4 values of K and Q for the scores (Section 3.4) */
    const int mixed = p->mixed != 0 && quant != QUANT_NONE;
    double *Kn = 0, *Qn = 0;
    const double *Ks, *Qs;
    /* exact options: per-token exponents of K, V, Q, dO (doc-local index) */
    const int exact = p->exact != 0 && quant != QUANT_NONE;
    const int blk = exact ? 1 : 32;
    int *eK = 0, *eV = 0, *eQ = 0, *eO = 0, *erow = 0;
    double *acc = 0, *xbuf = 0, *dS = 0, *dQa = 0, *dKa = 0, *dVa = 0;
    float *lsef = 0;
    int64_t sat = 0, nds = 0, nds0 = 0;
    size_t Ld = (size_t)L * d;

    if (L == 0) return;
    Kt = malloc(sizeof(double) * Ld);
    if (mixed) {
        Kn = malloc(sizeof(double) * Ld);
        Qn = malloc(sizeof(double) * Ld);
        if (!Kn || !Qn) { *err = ORC_ERR_NOMEM; goto done; }
    }
    if (exact) {
        eK = malloc(sizeof(int) * (size_t)L);
        eV = malloc(sizeof(int) * (size_t)L);
        eQ = malloc(sizeof(int) * (size_t)L);
        eO = malloc(sizeof(int) * (size_t)L);
        erow = malloc(sizeof(int) * 32);
        if (!eK || !eV || !eQ || !eO || !erow) { *err = ORC_ERR_NOMEM; goto done; }
    }
    Vt = malloc(sizeof(double) * Ld);
    Qt = malloc(sizeof(double) * Ld);
    O = malloc(sizeof(double) * Ld);
    lse = malloc(sizeof(double) * L);
    lsef = malloc(sizeof(float) * L);
    acc = malloc(sizeof(double) * d);
    xbuf = malloc(sizeof(double) * (p->key_tile > 32 ? p->key_tile : 32));
    if (need_bwd) {
        dOt = malloc(sizeof(double) * Ld);
        Dv = malloc(sizeof(double) * L);
        dS = malloc(sizeof(double) * 32 * (size_t)L);
        dQa = malloc(sizeof(double) * Ld);
        dKa = calloc(Ld, sizeof(double));
        dVa = calloc(Ld, sizeof(double));
    }
    if (!Kt || !Vt || !Qt || !O || !lse || !lsef || !acc || !xbuf ||
        (need_bwd && (!dOt || !Dv || !dS || !dQa || !dKa || !dVa))) {
        *err = ORC_ERR_NOMEM;
        goto done;
    }
    /* K~ and V~: token blocks of this document and this key/value head. */
    /* K~ is quantized from the rotated rows when the Hadamard rotation is on
     * (Section 3.4); V~ never is. */
    if (tbq_slice(k + ((long)base * hkv + g) * d, (long)hkv * d, L, d, quant, p->hadamard != 0, Kt, 0, 0, 0, Kn,
                  blk, eK) ||
        tbq_slice(v + ((long)base * hkv + g) * d, (long)hkv * d, L, d, quant, 0, Vt, 0, 0, 0, 0, blk, eV)) {
        *err = ORC_ERR_NOMEM;
        goto done;
    }

    Ks = mixed ? Kn : Kt;     /* score operands; the gradient products keep Kt and Qt */
    Qs = mixed ? Qn : Qt;
    for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        if (tbq_slice(q + ((long)base * hq + h) * d, (long)hq * d, L, d, quant, p->hadamard != 0, Qt, 0, 0, 0, Qn,
                      blk, eQ)) {
            *err = ORC_ERR_NOMEM;
            goto done;
        }
        /* ---- forward, row by row ---- */
        for (int i = 0; i < L; ++i) {
            fwd_row(p, h, base, i, Qs + (long)i * d, Ks, Vt, eV, c1, acc, xbuf, O + (long)i * d, &lse[i], &sat);
            lsef[i] = (float)lse[i];
            /* MX modes return a bf16 O and the backward reads it back
             * (Section 3.4: returned outputs are BF16); the unquantized mode
             * keeps binary64 throughout. */
            for (int c = 0; c < d; ++c) {
                long gi = ((long)(base + i) * hq + h) * d + c;
                uint16_t b = orc_double_to_bf16(O[(long)i * d + c]);
                if (out->o64) out->o64[gi] = O[(long)i * d + c];
                if (out->o16) out->o16[gi] = b;
                if (quant != QUANT_NONE) O[(long)i * d + c] = orc_bf16_to_double(b);
            }
            if (out->lse2) out->lse2[(long)h * p->ttot + base + i] = lsef[i];
        }
        if (!need_bwd) continue;

        /* ---- backward (Section 2 equations; Section 3.3 consistency) ---- */
        if (tbq_slice(dout + ((long)base * hq + h) * d, (long)hq * d, L, d, quant, 0, dOt, 0, 0, 0, 0, blk, eO)) {
            *err = ORC_ERR_NOMEM;
            goto done;
        }
        for (int i = 0; i < L; ++i) {
            Dv[i] = dotd(dOt + (long)i * d, O + (long)i * d, d);
            if (out->dvec) out->dvec[(long)h * p->ttot + base + i] = Dv[i];
        }
        memset(dQa, 0, sizeof(double) * Ld);
        for (int i0 = 0; i0 < L; i0 += 32) {
            int i1 = i0 + 32 < L ? i0 + 32 : L;
            /* exact options: the dV product applies one factor 2^Eo per
             * 32-query block, Eo = the block's largest dO~ exponent */
            int Eo = 0;
            if (exact) {
                Eo = eO[i0];
                for (int i = i0 + 1; i < i1; ++i)
                    if (eO[i] > Eo) Eo = eO[i];
            }
            /* dS for the 32 query rows of this block, every visible key. */
            for (int i = i0; i < i1; ++i) {
                double li = (quant == QUANT_NONE) ? lse[i] : (double)lsef[i];
                const double *qi = Qs + (long)i * d, *doi = dOt + (long)i * d;
                double *row = dS + (size_t)(i - i0) * L;
                for (int j = 0; j < L; ++j) row[j] = 0.0;
                for (int j = 0; j <= i; ++j) {
                    double xij = score_dot(p, qi, Ks + (long)j * d, d, h, base + i, base + j, 0) * c1;
                    double P = exp2(xij - li), wb;
                    double dP = score_dot(p, doi, Vt + (long)j * d, d, h, base + i, base + j, 1);
                    if (quant == QUANT_NONE) {
                        wb = P;
                    } else {
                        /* Appendix B.1: the dV operand is E4M3(2^8 P), no scale.
                         * Exact options: it also takes dO~_i's own exponent,
                         * relative to the block's Eo: E4M3(2^8 P 2^(e_i - Eo)). */
                        const double fo = exact ? ldexp(1.0, eO[i] - Eo) : 1.0;
                        wb = ldexp(orc_e4m3_value(orc_e4m3_encode(ldexp(P, 8) * fo)), -8) / fo;
                    }
                    for (int c = 0; c < d; ++c) dVa[(long)j * d + c] += wb * doi[c];
                    row[j] = P * (dP - Dv[i]);
                }
            }
            /* dS~: one exponent per 32x32 document-local block (Section 3.3),
             * then dQ += dS~ K~ and dK += dS~^T Q~. */
            for (int j0 = 0; j0 <= i1 - 1; j0 += 32) {
                int j1 = j0 + 32 < L ? j0 + 32 : L;
                int e = 0;
                if (exact) {
                    /* Exact options (Appendix A.3): the two gradient products
                     * contract over different tokens, so dS~ differs between
                     * them.  dK's operand takes Q~_i's exponent, y = dS 2^eQ_i,
                     * with one exponent per 32x32 block of y; dQ's operand
                     * takes K~_j's exponent, z = dS 2^eK_j, with one exponent
                     * per query row of the block (the per-query-row dS
                     * exponent), over that row's visible keys only.  The
                     * products apply 2^(block or row exponent) and the folded
                     * exponent returns with the other operand's codes. */
                    const int rule = quant == QUANT_FLOOR ? 1 : 0;
                    int *ez = erow;
                    double ay = 0.0;
                    for (int i = i0; i < i1; ++i) {
                        double az = 0.0;
                        for (int j = j0; j < j1 && j <= i; ++j) {
                            double a = fabs(dS[(size_t)(i - i0) * L + j]);
                            double yk = ldexp(a, eQ[i]), zq = ldexp(a, eK[j]);
                            if (yk > ay) ay = yk;
                            if (zq > az) az = zq;
                        }
                        ez[i - i0] = orc_scale_exp(az, rule);
                    }
                    e = orc_scale_exp(ay, rule);
                    for (int i = i0; i < i1; ++i)
                        for (int j = j0; j < j1 && j <= i; ++j) {
                            double ds = dS[(size_t)(i - i0) * L + j];
                            double yk = ldexp(ds, eQ[i]), zq = ldexp(ds, eK[j]);
                            double dkv = ldexp(ldexp(orc_e4m3_value(orc_e4m3_encode(ldexp(yk, -e))), e), -eQ[i]);
                            double dqv = ldexp(ldexp(orc_e4m3_value(orc_e4m3_encode(ldexp(zq, -ez[i - i0]))),
                                                     ez[i - i0]), -eK[j]);
                            nds++;
                            if (ds != 0.0 && dqv == 0.0) nds0++;
                            for (int c = 0; c < d; ++c) {
                                dQa[(long)i * d + c] += dqv * Kt[(long)j * d + c];
                                dKa[(long)j * d + c] += dkv * Qt[(long)i * d + c];
                            }
                        }
                    continue;
                }
                if (quant != QUANT_NONE) {
                    double amax = 0.0;
                    for (int i = i0; i < i1; ++i)
                        for (int j = j0; j < j1 && j <= i; ++j) {
                            double a = fabs(dS[(size_t)(i - i0) * L + j]);
                            if (a > amax) amax = a;
                        }
                    e = orc_scale_exp(amax, quant == QUANT_FLOOR ? 1 : 0);
                }
                for (int i = i0; i < i1; ++i)
                    for (int j = j0; j < j1 && j <= i; ++j) {
                        double ds = dS[(size_t)(i - i0) * L + j], dq;
                        if (quant == QUANT_NONE) {
                            dq = ds;
                        } else {
                            dq = ldexp(orc_e4m3_value(orc_e4m3_encode(ldexp(ds, -e))), e);
                            nds++;
                            if (ds != 0.0 && dq == 0.0) nds0++;
                        }
                        if (dq == 0.0) continue;
                        for (int c = 0; c < d; ++c) {
                            dQa[(long)i * d + c] += dq * Kt[(long)j * d + c];
                            dKa[(long)j * d + c] += dq * Qt[(long)i * d + c];
                        }
                    }
            }
        }
        if (p->hadamard) {
            /* dQ' is the gradient for the rotated Q' = Q H / sqrt(d): dQ = dQ' H / sqrt(d)
             * (H / sqrt(d) is symmetric and its own inverse). */
            for (int i = 0; i < L; ++i) hadamard_f64(dQa + (long)i * d, d);
        }
        for (int i = 0; i < L; ++i)
            for (int c = 0; c < d; ++c) {
                long gi = ((long)(base + i) * hq + h) * d + c;
                double val = s * dQa[(long)i * d + c];
                if (out->dq64) out->dq64[gi] = val;
                if (out->dq16) out->dq16[gi] = orc_double_to_bf16(val);
            }
    }
    if (need_bwd) {
        if (p->hadamard)   /* dK = dK' H / sqrt(d), as for dQ */
            for (int j = 0; j < L; ++j) hadamard_f64(dKa + (long)j * d, d);
        for (int j = 0; j < L; ++j)
            for (int c = 0; c < d; ++c) {
                long gj = ((long)(base + j) * hkv + g) * d + c;
                double kv = s * dKa[(long)j * d + c], vv = dVa[(long)j * d + c];
                if (out->dk64) out->dk64[gj] = kv;
                if (out->dv64) out->dv64[gj] = vv;
                if (out->dk16) out->dk16[gj] = orc_double_to_bf16(kv);
                if (out->dv16) out->dv16[gj] = orc_double_to_bf16(vv);
            }
    }
    if (out->stats) {
#pragma omp atomic
        out->stats[0] += sat;
#pragma omp atomic
        out->stats[1] += nds;
#pragma omp atomic
        out->stats[2] += nds0;
    }
done:
    free(Kt); free(Vt); free(Qt); free(O); free(lse); free(lsef); free(acc); free(xbuf);
    free(Kn); free(Qn); free(eK); free(eV); free(eQ); free(eO); free(erow);
    free(dOt); free(Dv); free(dS); free(dQa); free(dKa); free(dVa);
}


typedef struct { long len; int doc, g; } unit_t;

static int cmp_unit(const void *a, const void *b)
{
    const unit_t *x = a, *y = b;
    if (x->len != y->len) return x->len < y->len ? 1 : -1;
    if (x->doc != y->doc) return x->doc - y->doc;
    return x->g - y->g;
}

/*
 * Forward (and, when dout != NULL, backward) for the units selected by
 * kv_mask[g] and doc_mask[doc] (NULL = all).  Layouts: q/dout/o/dq
 * [ttot][hq][d]; k/v/dk/dv [ttot][hkv][d]; lse2/dvec [hq][ttot].  Any output
 * pointer may be NULL.  Outputs of units that are not selected are left as
 * the caller initialised them.
 */
int orc_attention(const orc_params *p, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const uint16_t *dout, const int32_t *cu, const uint8_t *kv_mask,
                  const uint8_t *doc_mask,
                  double *o64, uint16_t *o16, float *lse2, double *dvec,
                  double *dq64, double *dk64, double *dv64,
                  uint16_t *dq16, uint16_t *dk16, uint16_t *dv16, int64_t *stats)
{
    orc_out out = {o64, o16, lse2, dvec, dq64, dk64, dv64, dq16, dk16, dv16, stats};
    unit_t *units;
    long nu = 0;
    int err = ORC_OK;
    if (!p || !q || !k || !v || p->d <= 0 || p->hq <= 0 || p->hkv <= 0 || p->hq % p->hkv)
        return ORC_ERR_ARG;
    /* the approximate exponential is for the forward only (Section 3.7) */
    if (p->fast_exp < 0 || p->fast_exp > 8 || (p->fast_exp > 0 && dout)) return ORC_ERR_ARG;
    if (p->key_tile <= 0 || p->quant < 0 || p->quant > 2 || !check_cu(p, cu)) return ORC_ERR_ARG;
    /* the exact options take the unquantized row sum and the exact exponential,
     * on the MXFP8 path */
    if (p->exact && (p->rowsum || p->fast_exp || p->mixed)) return ORC_ERR_ARG;
    /* Section 3.4 / Appendix B.1: c + tau <= log2(448) keeps 2^c p below the
     * largest E4M3 value; anything else is rejected. */
    if (p->c_log2 < 0 || p->tau < 0) return ORC_ERR_ARG;
    if (p->quant != QUANT_NONE && p->c_log2 + p->tau > 8 && !p->unsafe_bound)
        return ORC_ERR_BOUND;
    if (stats) stats[0] = stats[1] = stats[2] = 0;
    units = malloc(sizeof(unit_t) * ((size_t)p->ndocs * p->hkv + 1));
    if (!units) return ORC_ERR_NOMEM;
    for (int doc = 0; doc < p->ndocs; ++doc) {
        if (doc_mask && !doc_mask[doc]) continue;
        for (int g = 0; g < p->hkv; ++g) {
            if (kv_mask && !kv_mask[g]) continue;
            units[nu].len = cu[doc + 1] - cu[doc];
            units[nu].doc = doc;
            units[nu].g = g;
            nu++;
        }
    }
    qsort(units, (size_t)nu, sizeof(unit_t), cmp_unit);   /* longest first */
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < nu; ++u) {
        int e = ORC_OK;
        unit_run(p, units[u].doc, units[u].g, cu, q, k, v, dout, &out, &e);
        if (e) err = e;
    }
    free(units);
    return err;
}

/* rows x d bf16 patterns -> their NVFP4 values (rot = 1: of the rotated rows) */
void orc_nvfp4_rows(const uint16_t *x, long rows, int d, int rot, double *out)
{
    double *xv = malloc(sizeof(double) * (size_t)d);
    float *row = malloc(sizeof(float) * (size_t)d);
    if (!xv || !row) { free(xv); free(row); return; }
    for (long r = 0; r < rows; ++r) {
        if (rot) {
            orc_hadamard_f32(x + r * d, d, row);
            for (int k = 0; k < d; ++k) xv[k] = (double)row[k];
        } else {
            for (int k = 0; k < d; ++k) xv[k] = orc_bf16_to_double(x[r * d + k]);
        }
        nvfp4_row(xv, d, out + r * d);
    }
    free(xv);
    free(row);
}

/* rows x d bf16 patterns -> rows x d fp32 rotated values */
void orc_hadamard_f32_array(const uint16_t *x, long rows, int d, float *y)
{
    for (long r = 0; r < rows; ++r) orc_hadamard_f32(x + r * d, d, y + r * d);
}

void orc_e4m3_encode_array(const double *y, long n, uint8_t *codes)
{
    for (long i = 0; i < n; ++i) codes[i] = orc_e4m3_encode(y[i]);
}

void orc_e4m3_value_array(const uint8_t *codes, long n, double *v)
{
    for (long i = 0; i < n; ++i) v[i] = orc_e4m3_value(codes[i]);
}

void orc_scale_exp_array(const double *a, long n, int rule, int32_t *e)
{
    for (long i = 0; i < n; ++i) e[i] = orc_scale_exp(a[i], rule);
}

void orc_double_to_bf16_array(const double *x, long n, uint16_t *b)
{
    for (long i = 0; i < n; ++i) b[i] = orc_double_to_bf16(x[i]);
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
