// Internal device helpers of the HIP library (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // register-friendly 16-byte chunk

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

namespace flamia {

// ---------------------------------------------------------------------------
// Block-scaled FP8 MFMA, 32x32x64, E4M3 x E4M3 -> fp32.
// Operand layout (measured on gfx950): lane l carries row (A) / column (B)
// l % 32; bytes 0..15 of lanes l and l+32 form the first 32-element
// contraction block, scaled by the UE8M0 byte of lane l % 32; bytes 16..31
// form the second block, scaled by the byte of lane l % 32 + 32.  A and B use
// the same (lane / 32, byte) -> k assignment.  Accumulator: lane l holds
// column l % 32, rows 8*(i/4) + 4*(l/32) + i%4 for i = 0..15.
// ---------------------------------------------------------------------------
__device__ __forceinline__ v16f mfma_mx(v8i a, v8i b, v16f c, int scale_a, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

// bf16 MFMA 32x32x16 -> fp32 (the score product of the mixed NVFP4 path,
// whose values are exact in bf16).  Lane l carries row (A) / column (B)
// l % 32 and eight contraction elements; A and B use the same (lane / 32,
// element) -> k assignment (measured on gfx950), so any channel order that
// both operands share gives the dot product.  Swapping the A and B roles
// gives bitwise the transposed result (measured).  Accumulator layout as
// mfma_mx.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v16f mfma_bf16(u32x4 a, u32x4 b, v16f c) {
    bf16x8_t x, y;
    __builtin_memcpy(&x, &a, 16);
    __builtin_memcpy(&y, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
}

// Transposed LDS read of 8-bit elements (ds_read_b64_tr_b8).  Within each
// group of 16 lanes, lane s supplies the address of an 8-byte row R_s; lane j
// receives byte i = R_{2i + (j%16)/8}[j % 8] for i = 0..7.
__device__ __forceinline__ v2i lds_read_tr8(const uint8_t* lds_addr) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(v2i, const_cast<uint8_t*>(lds_addr)));
}

// Direct global -> LDS loads (global_load_lds_*): lane l of the wave writes
// its 16 / 4 bytes at lds_base + 16 l / 4 l; the one-byte form writes the
// byte zero-extended to a dword at lds_base + 4 l (all measured on gfx950).
// The LDS base must be wave-uniform (it goes through M0, which is saved and
// restored around the load).  They count in vmcnt like any vector load and
// bypass the registers.  They are issued from inline assembly on purpose:
// the compiler would otherwise treat every later LDS read as dependent on
// them and wait for all outstanding loads before it, which defeats fetching
// ahead.  Since the compiler does not know of them, its own waits do not
// cover them (__syncthreads does not wait for them either): the caller waits
// with vm_wait_barrier before reading the LDS they wrote.  Waits that the
// compiler inserts for its own loads can only wait longer than needed, never
// too little (loads complete in issue order).
__device__ __forceinline__ uint32_t lds_addr_of(void* p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) void*)p);
}
#define FLAMIA_DMA_ASM(OP)                                                                     \
    "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t" OP " %1, off\n\ts_mov_b32 m0, %0\n\ts_nop 0"
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
    uint32_t save;
    asm volatile(FLAMIA_DMA_ASM("global_load_lds_dwordx4") : "=&s"(save) : "v"(src), "s"(lds_addr_of(lds_base))
                 : "memory");
}
__device__ __forceinline__ void dma4(const void* src, void* lds_base) {
    uint32_t save;
    asm volatile(FLAMIA_DMA_ASM("global_load_lds_dword") : "=&s"(save) : "v"(src), "s"(lds_addr_of(lds_base))
                 : "memory");
}
__device__ __forceinline__ void dma1(const void* src, void* lds_base) {
    uint32_t save;
    asm volatile(FLAMIA_DMA_ASM("global_load_lds_ubyte") : "=&s"(save) : "v"(src), "s"(lds_addr_of(lds_base))
                 : "memory");
}
#undef FLAMIA_DMA_ASM
// Waits until at most N vector memory operations of the wave are
// outstanding (the direct LDS loads above included), then joins the
// workgroup barrier.  Loads complete in issue order, so with N = the number
// of loads issued after a given one this waits for that load whatever the
// stores in between do.  No LDS access moves across it (opaque memory
// clobbers on both sides).
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void vm_drain_barrier() { vm_wait_barrier<0>(); }
// Makes the compiler have x in registers here, so that its wait for the load
// of x is placed here and not at a later first use, where it would also wait
// for the direct LDS loads issued in between (the compiler cannot tell them
// apart).  Device pass only: the host pass has no VGPR constraint, and the
// failed substitution would silently drop the kernel's host stub.
template <class T>
__device__ __forceinline__ void keep_loaded(const T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" ::"v"(x));
#else
    (void)x;
#endif
}

// Four fp32 -> four E4M3 bytes (byte i = element i), round to nearest even;
// bit-identical to the format's definition for |x| <= 448.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
    // Both halves are overwritten, so the destination's incoming content is
    // irrelevant; leaving the seed undefined lets the compiler convert in
    // place instead of first copying a live value into the destination (one
    // VALU move per four codes).
    int seed;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, seed, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}
// Same with an exact power-of-two divisor: byte i = E4M3(x_i / scale).
__device__ __forceinline__ int pack_fp8x4_div(float a, float b, float c, float d, float scale) {
    // both halves are overwritten, so the incoming register content is irrelevant
    v2s w;
    __builtin_memcpy(&w, &a, 4);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, scale, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, scale, true);
    int out;
    __builtin_memcpy(&out, &w, 4);
    return out;
}

// Sum of the four E4M3 values packed in w (hardware decode, exact).
__device__ __forceinline__ float fp8x4_sum(int w) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    return (lo[0] + lo[1]) + (hi[0] + hi[1]);
}

// Cooperative fetch of one 128-row tile of two code tensors (K and V, [T][H][D])
// plus their per-token scales into registers; rows are clamped into the buffer.
template <int D, int N>
__device__ __forceinline__ void fetch_kv_tile(u32x4 (&kr)[N], u32x4 (&vr)[N], uint32_t& ek, uint32_t& ev,
                                              const uint8_t* kc, const uint8_t* ks, const uint8_t* vc,
                                              const uint8_t* vs, int k0, int ttot, int heads, int g, int tid) {
#pragma unroll
    for (int r = 0; r < N; ++r) {
        const int c = tid + 256 * r;
        const int row = c / (D / 16), col = (c % (D / 16)) * 16;
        const long krow = min(k0 + row, ttot - 1);
        kr[r] = *reinterpret_cast<const u32x4*>(kc + (krow * heads + g) * D + col);
        vr[r] = *reinterpret_cast<const u32x4*>(vc + (krow * heads + g) * D + col);
    }
    const long kt = min(k0 + (tid & 127), ttot - 1);
    ek = ks[(long)g * ttot + kt];
    ev = vs[(long)g * ttot + kt];
}

__device__ __forceinline__ float fp8_to_f32(uint32_t code) {
    // E4M3 byte -> float, exact (subnormals 2^-9 m, normals 2^(E-7) (1 + m/8)).
    const uint32_t s = code & 0x80u, e = (code >> 3) & 15u, m = code & 7u;
    float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    return s ? -v : v;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ unsigned wave_sum_u32(unsigned v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += (unsigned)__shfl_xor((int)v, off);
    return v;
}

__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Two fp32 -> two bf16 packed in one word (a in the low half), round to
// nearest even (one v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_t r = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
    uint32_t u;
    __builtin_memcpy(&u, &r, 4);
    return u;
}
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Shared exponent of a block with largest magnitude `amax` (fp32, >= 0):
// the smallest e with amax <= 448 * 2^e ("rounded up", so no element of the
// block saturates), clamped to [lo, 127]; amax == 0 gives lo.
__device__ __forceinline__ int block_exponent(float amax, int lo) {
    // Branch-free (a compare and two clamps), so that callers stay one basic
    // block.  With amax = 1.f x 2^E, 448 = 1.75 x 2^8: the exponent is E - 8,
    // plus one when the mantissa exceeds 1.75.  A subnormal or zero amax
    // (biased exponent 0) gives at most -134 here and a true exponent below
    // -133, so for lo >= -133 the clamp alone yields the right result.
    const uint32_t u = __float_as_uint(amax);
    const int e = (int)(u >> 23) - 135 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return min(max(e, lo), 127);
}

// block_exponent of a wave-uniform maximum, evaluated on the scalar unit
// (the value is read from lane 0; every lane must hold the same value).
__device__ __forceinline__ int block_exponent_uniform(float amax, int lo) {
    const uint32_t u = __builtin_amdgcn_readfirstlane(__float_as_uint(amax));
    return block_exponent(__uint_as_float(u), lo);
}

// fp32 nearest to 1/sqrt(d) for d = 64 (exact) and d = 128 (2^-3.5 rounded).
template <int D>
__device__ __forceinline__ constexpr float inv_sqrt_d() {
    return D == 64 ? 0.125f : 0x1.6a09e6p-4f;
}

// Normalized Hadamard rotation over the d channels of a transposed gradient
// accumulator (dQ^T or dK^T: register 4j + r of tile dt holds channel
// 32 dt + 8 j + 4 lg + r of the lane's row, lg = lane / 32).  H / sqrt(d) is
// symmetric and its own inverse, so this takes the gradient of a rotated
// operand back to the unrotated one.  fp32 butterflies in the order of the
// channel bits; the lane-half bit (channel bit 2) pairs lanes l and l ^ 32.
template <int DT>
__device__ __forceinline__ void hadamard_rows(v16f (&acc)[DT], int lg) {
    // channel bits 0, 1 (r) and 3, 4 (j): register bits 0, 1, 2, 3
    auto in_reg = [&](int rbit) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if ((i & rbit) == 0) {
                    const float a = acc[dt][i], b = acc[dt][i + rbit];
                    acc[dt][i] = a + b;
                    acc[dt][i + rbit] = a - b;
                }
    };
    in_reg(1);
    in_reg(2);
    // channel bit 2: the other lane half
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float v = acc[dt][i];
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
            const float p = __uint_as_float(lg ? r[0] : r[1]);
            acc[dt][i] = lg ? p - v : v + p;
        }
    in_reg(4);
    in_reg(8);
    // channel bits 5, 6: the tiles
#pragma unroll
    for (int h = 1; h < DT; h <<= 1)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            if ((dt & h) == 0)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float a = acc[dt][i], b = acc[dt + h][i];
                    acc[dt][i] = a + b;
                    acc[dt + h][i] = a - b;
                }
}

// Lane exchange without the LDS crossbar: DPP within 16-lane rows, then
// v_permlane16_swap / v_permlane32_swap across rows.  Each swap returns the
// pair {own value, partner value} (order depends on the lane), so a
// commutative combine of the two halves gives the same result in both lanes.
__device__ __forceinline__ float max_xor32(float v) {      // lanes l <-> l ^ 32
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Maximum over all 64 lanes of a non-negative value (+0 included, no NaN),
// returned in every lane.  Non-negative IEEE floats order like their bit
// patterns, so the reduction runs on unsigned integers: no NaN quieting, and
// each DPP step fuses into one v_max_u32_dpp.
template <int CTRL>
__device__ __forceinline__ uint32_t umax_dpp(uint32_t v) {
    return max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_max_nonneg(float x) {
    uint32_t v = __float_as_uint(x);
    v = umax_dpp<0xB1>(v);          // quad_perm [1,0,3,2]
    v = umax_dpp<0x4E>(v);          // quad_perm [2,3,0,1]
    v = umax_dpp<0x141>(v);         // row_half_mirror: the two quads of each 8
    v = umax_dpp<0x140>(v);         // row_mirror: the two halves of each 16
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);   // rows 0<->1, 2<->3
    v = max((uint32_t)r[0], (uint32_t)r[1]);
    r = __builtin_amdgcn_permlane32_swap(v, v, false, false);        // lanes l <-> l ^ 32
    return __uint_as_float(max((uint32_t)r[0], (uint32_t)r[1]));
}

// Largest of a non-negative integer over each half-wave (lanes 0-31, 32-63), in every
// lane of the half: DPP over 16-lane rows, then one row swap.
__device__ __forceinline__ uint32_t halfwave_max(uint32_t v) {
    v = umax_dpp<0xB1>(v);
    v = umax_dpp<0x4E>(v);
    v = umax_dpp<0x141>(v);
    v = umax_dpp<0x140>(v);
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return max((uint32_t)r[0], (uint32_t)r[1]);
}

// Head of work item `local` (0 <= local < heads) of one tile of document
// `doc`.  Workgroups are dispatched round-robin over the 8 XCDs (workgroup
// index % 8), each with its own L2.  When heads % 8 == 0 the tile's items
// start at a multiple of 8, and XCD x receives a contiguous run of heads/8
// heads, so query heads that share a key/value head (GQA) read its tiles
// through the same L2.  Which run goes to which XCD rotates with the
// document: the heads' costs differ with their data (by up to 13% on the
// 4 x 8192 GQA call), and a fixed assignment left the most expensive XCD
// finishing last (forward and dQ pass 1.5% faster rotated).
__device__ __forceinline__ int xcd_head(int local, int heads, int doc) {
    return (heads & 7) ? local : (((local & 7) + doc) & 7) * (heads >> 3) + (local >> 3);
}

// Position of document `doc`'s boundaries; binary search of the largest
// d with cu[d] <= t among [0, ndocs).
__device__ __forceinline__ int find_doc(const int32_t* cu, int ndocs, int t) {
    int lo = 0, hi = ndocs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace flamia
