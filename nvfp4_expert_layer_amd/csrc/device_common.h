// Device-side helpers shared by the gfx950 kernels of the NVFP4 MoE layer.
//
// NVFP4 (NVIDIA's format; the page "Serving Solar Open 2 on DGX Spark",
// section "b12x 버전이 실제 NVFP4 체크포인트를 읽어들이도록 만들기", names its
// parts: packed FP4 codes, FP8 block scales clamped to 448, per-expert fp32
// global scale): E2M1 codes two per byte (even element in the low nibble), one
// E4M3fn scale per 16 elements along K, a fp32 global multiplier per tensor.
//
// gfx950 conversion instructions used here (their behaviour was checked on the
// device for every input byte):
//   v_cvt_scalef32_pk_bf16_fp4 / _pk_f32_fp4: two E2M1 codes of one byte -> two
//     bf16 / fp32 values, multiplied by 2^exponent(scale) (only the exponent of
//     the fp32 scale operand is used).  With scale 1.0 the result is the exact
//     code value.  byte_sel picks the byte of the source dword.
//   v_cvt_f32_fp8: one E4M3fn byte -> fp32 (OCP encoding, bias 7, max 448).
//   v_cvt_scalef32_pk_f16_fp4: the same two codes -> two f16 (exact; with scale
//     1.0 the code value), used with a packed f16 multiply by the block scale on
//     the W4A4 tiled path (exact: products of at most 6 significant bits in
//     f16's normal range); covered by that path's parity tests.
//   v_cvt_scalef32_pk_f16_fp8: two E4M3fn bytes (the low or high 16 bits of
//     the source) -> two f16; with scale 1.0 exact for every finite E4M3 value
//     (its subnormals, down to 2^-9, are f16 normals).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace moe {

constexpr int kBlock = 16;          // NVFP4 elements per block scale

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even: the hardware conversion
// (v_cvt_pk_bf16_f32), one instruction where the integer rounding took four.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> bf16x2 bits {lo, hi}, round to nearest even, one instruction.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v_t){lo, hi}, bf16x2v_t));
}

// Upper halves of two fp32 values packed as bf16x2 (exact when both values are
// representable in bf16, which holds for code * E4M3 scale products).
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
    return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// Two E4M3 block scales (bytes 0 and 1 of `pair`) -> f16 {byte 0, byte 1}.
__device__ __forceinline__ f16x2_t e4m3x2_to_f16(uint32_t pair) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pair, 1.0f, false);
}

// Bytes 2 and 3 of `quad` -> f16 {byte 2, byte 3}.
__device__ __forceinline__ f16x2_t e4m3x2_hi_to_f16(uint32_t quad) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(quad, 1.0f, true);
}

// Block scales of a weight-streaming step in 16-byte segments.  A step covers
// 256 elements of K: lane group g (lanes 16 g .. 16 g + 15) takes the 64-element
// chunk 4 s + g of its row, whose four E4M3 scales are dword g of the row's
// 16-byte scale segment of step s.  Lane group m loads the whole segment of step
// 4 G + m (one 16-byte load per four steps instead of a 4-byte load per step);
// this 4 x 4 transpose across the lane groups (two permlane32 and two permlane16
// swaps) then leaves in lane group g, dword m, the scales of its own chunk at
// step 4 G + m.
__device__ __forceinline__ u32x4_t scale_seg_transpose(u32x4_t x) {
    unsigned r0 = x.x, r1 = x.y, r2 = x.z, r3 = x.w;
    auto p = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
    r0 = p[0];
    r2 = p[1];
    p = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
    r1 = p[0];
    r3 = p[1];
    p = __builtin_amdgcn_permlane16_swap(r0, r1, false, false);
    r0 = p[0];
    r1 = p[1];
    p = __builtin_amdgcn_permlane16_swap(r2, r3, false, false);
    r2 = p[0];
    r3 = p[1];
    return u32x4_t{r0, r1, r2, r3};
}

// Dword i (0..3, runtime) of a segment.
__device__ __forceinline__ uint32_t seg_word(const u32x4_t& x, int i) {
    return i == 0 ? x.x : (i == 1 ? x.y : (i == 2 ? x.z : x.w));
}

// Two E2M1 codes (byte `sel` of `src`) -> exact fp32 values.
template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32(uint32_t src) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(src, 1.0f, SEL);
}

// Eight E2M1 codes (one dword) times a block scale -> 8 exact bf16 (4 dwords).
__device__ __forceinline__ u32x4_t dequant8_bf16(uint32_t codes, float scale) {
    f32x2_t a = fp4x2_to_f32<0>(codes), b = fp4x2_to_f32<1>(codes);
    f32x2_t c = fp4x2_to_f32<2>(codes), d = fp4x2_to_f32<3>(codes);
    u32x4_t r;
    r.x = pack_hi16(a[0] * scale, a[1] * scale);
    r.y = pack_hi16(b[0] * scale, b[1] * scale);
    r.z = pack_hi16(c[0] * scale, c[1] * scale);
    r.w = pack_hi16(d[0] * scale, d[1] * scale);
    return r;
}

// Eight E2M1 codes -> 8 exact bf16 code values (no scale), 4 dwords.
__device__ __forceinline__ u32x4_t fp4x8_to_bf16(uint32_t codes) {
    bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 0);
    bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 1);
    bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 2);
    bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 3);
    u32x4_t r;
    r.x = __builtin_bit_cast(uint32_t, a);
    r.y = __builtin_bit_cast(uint32_t, b);
    r.z = __builtin_bit_cast(uint32_t, c);
    r.w = __builtin_bit_cast(uint32_t, d);
    return r;
}

// Eight E2M1 codes times a block scale (as an f16 pair) -> 8 exact f16 values
// (4 dwords): a code times an E4M3 scale has at most 6 significant bits and lies
// in [2^-10, 2688], inside f16's normal range, so the packed f16 products are
// exact.
__device__ __forceinline__ u32x4_t dequant8_f16(uint32_t codes, f16x2_t s2) {
    const f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
    const f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
    const f16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
    const f16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
    u32x4_t r;
    r.x = __builtin_bit_cast(uint32_t, a);
    r.y = __builtin_bit_cast(uint32_t, b);
    r.z = __builtin_bit_cast(uint32_t, c);
    r.w = __builtin_bit_cast(uint32_t, d);
    return r;
}

// fp32 -> f16 bits (round to nearest even; exact for NVFP4 products).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// ---------------------------------------------------------------------------
// NVFP4 encoders (fp32 decisions, round to nearest with ties to the even code,
// saturating).  Written from the bit layout, not from a table of the host side.
// ---------------------------------------------------------------------------

// Non-negative finite fp32 -> E4M3fn byte (0x00..0x7E).
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float v) {
    if (!(v < 448.0f)) return 0x7Eu;                  // saturate (v >= 448)
    // Smallest normal is 2^-6; below it the grid step is 2^-9 (subnormals).
    if (v < 0.015625f) {
        // value = m * 2^-9, m in 0..8 (8 == the first normal 2^-6, code 0x08)
        float q = v * 512.0f;                           // exact (power-of-two scale)
        float r = __builtin_rintf(q);                   // ties to even integer = even code
        return (uint32_t)r;                             // m = 8 encodes as 0x08 (normal 2^-6)
    }
    // normal: v = 2^e * (1 + m/8), e in [-6, 8]
    uint32_t u = __float_as_uint(v);
    int e = (int)((u >> 23) & 0xFF) - 127;
    uint32_t mant = u & 0x7FFFFFu;                       // 23-bit fraction
    // keep 3 fraction bits, round to nearest even on the remaining 20 bits
    uint32_t keep = mant >> 20;
    uint32_t rest = mant & 0xFFFFFu;
    uint32_t code = (uint32_t)((e + 7) << 3) | keep;     // monotone in value
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) code += 1;   // may carry into exponent
    return code > 0x7Eu ? 0x7Eu : code;
}

// fp32 -> E2M1 code (4 bits), zero magnitude -> +0.  The magnitude index is
// the number of midpoints between {0, .5, 1, 1.5, 2, 3, 4, 6} (.25 .75 1.25
// 1.75 2.5 3.5 5) that |r| passes; at a midpoint the even code wins, so the
// comparison is strict where the upper neighbour is odd (.5, 1.5, 3, 6) and
// inclusive where it is even (1, 2, 4).  Branch-free: seven compares and adds
// instead of a chain of divergent branches.  Above 5, and for NaN, the index
// is 7 (magnitude 6).
__device__ __forceinline__ uint32_t e2m1_encode(float r) {
    const float a = fabsf(r);
    const uint32_t m6 = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                        (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f);
    const uint32_t m = a <= 5.0f ? m6 : 7u;
    return (m != 0 && r < 0.0f) ? (m | 8u) : m;
}

// E2M1 code (4 bits) -> its exact fp32 value.
__device__ __forceinline__ float e2m1_value(uint32_t code) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code & 0xFu, 1.0f, 0)[0];
}

// NVFP4 activation block step with an activation global scale g (g = 1: the
// dynamic rule, scale = E4M3(amax / 6), code = E2M1(x / scale); static: the
// calibrated g, scale = E4M3(amax / (6 g)), code = E2M1(x / (scale g)), fp32
// products and correctly rounded divisions, as for weights).
__device__ __forceinline__ uint32_t nvfp4_act_scale(float block_amax, float g) {
    return e4m3_encode_nonneg(__fdiv_rn(block_amax, 6.0f * g));
}
__device__ __forceinline__ uint32_t nvfp4_act_code(float x, float s, float g) {
    const float sg = s * g;
    return sg > 0.0f ? e2m1_encode(__fdiv_rn(x, sg)) : 0u;
}
// Quantize-dequantize of one value: returns code * scale exactly (the global g
// is applied after the GEMM's accumulation).
__device__ __forceinline__ float nvfp4_fake_quant(float x, float block_amax, float g) {
    const float s = e4m3_to_f32(nvfp4_act_scale(block_amax, g));
    return e2m1_value(nvfp4_act_code(x, s, g)) * s;
}

// Wave-wide reductions (wave64).
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace moe
