// NVFP4 quantizers (gfx950): weights (with a per-tensor fp32 global scale) and
// W4A4 activations (block scale only).
//
// Rule (NVFP4 as NVIDIA defines it; the page "Serving Solar Open 2 on DGX
// Spark", section "b12x 버전이 실제 NVFP4 체크포인트를 읽어들이도록 만들기",
// lists the tensors: packed FP4 codes, FP8 block scales clamped to 448, per-expert
// global scale), with every code-deciding step in fp32, correctly rounded:
//   weights:      g = amax_tensor / 2688  (1 if amax = 0),   2688 = 6 * 448
//                 s = E4M3(amax_block / (6 * g)),  c = E2M1(w / (s * g))
//   activations:  s = E4M3(amax_block / 6),        c = E2M1(x / s)
//                 (static W4A4: a calibrated global g_a, s = E4M3(amax_block /
//                 (6 g_a)), c = E2M1(x / (s g_a)), the weight rule's block step)
// E4M3 and E2M1 round to nearest, ties to the even code, and saturate (448, 6);
// a block whose scale rounds to 0 gets all-zero codes.
#include "device_common.h"
#include "kernels.h"

namespace moe {

// One thread per 16-element block.  x: bf16 [R][C]; amax_or_null: per-tensor
// amax (weights: g = amax / 2688 of tensor row / rows_per_tensor), or nullptr
// for activations with the global g_act (1 for the dynamic rule).
__global__ __launch_bounds__(256) void quantize_blocks_kernel(
    const uint16_t* __restrict__ x, long long nblocks, int C, int rows_per_tensor,
    const float* __restrict__ amax_or_null, float g_act, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
    long long b = (long long)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    const int bpr = C / kBlock;
    const long long row = b / bpr;
    float g = g_act;
    if (amax_or_null) {
        float amax = amax_or_null[row / rows_per_tensor];
        g = amax > 0.0f ? __fdiv_rn(amax, 2688.0f) : 1.0f;
    }
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + b * kBlock);
    u32x4_t v0 = src[0], v1 = src[1];
    uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float f[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    float bmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) bmax = fmaxf(bmax, fabsf(f[i]));
    const float denom6 = 6.0f * g;
    const uint32_t sbyte = e4m3_encode_nonneg(__fdiv_rn(bmax, denom6));
    const float s = e4m3_to_f32(sbyte);
    const float sg = s * g;
    uint32_t lo = 0u, hi = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        uint32_t c = sg > 0.0f ? e2m1_encode(__fdiv_rn(f[i], sg)) : 0u;
        if (i < 8) lo |= c << (4 * i);
        else hi |= c << (4 * (i - 8));
    }
    u32x2_t packed = {lo, hi};
    *reinterpret_cast<u32x2_t*>(codes + b * (kBlock / 2)) = packed;
    scales[b] = (uint8_t)sbyte;
}

// W4A4 activations: NVFP4 quantize-dequantize, one thread per 16-element block,
// writing the exact dequantized values (code * scale) as bf16, or as f16 (F16)
// for the tiled GEMMs, which multiply W4A4 operands in f16.  Both are exact: the
// product has at most 6 significant bits and lies in f16's normal range.
template <bool F16>
__global__ __launch_bounds__(256) void fake_quant_act_kernel(const uint16_t* __restrict__ x, long long nblocks,
                                                             float g, uint16_t* __restrict__ out) {
    long long b = (long long)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + b * kBlock);
    u32x4_t v0 = src[0], v1 = src[1];
    uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float f[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    float bmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) bmax = fmaxf(bmax, fabsf(f[i]));
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float lo = nvfp4_fake_quant(f[2 * i], bmax, g), hi = nvfp4_fake_quant(f[2 * i + 1], bmax, g);
        o[i] = F16 ? f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16) : pack_hi16(lo, hi);
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + b * kBlock);
    dst[0] = u32x4_t{o[0], o[1], o[2], o[3]};
    dst[1] = u32x4_t{o[4], o[5], o[6], o[7]};
}

__global__ void fill_zero_f32_kernel(float* p, int n) {
    int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// Per-tensor amax: grid (chunks, n); atomicMax on the bit pattern (non-negative floats).
__global__ __launch_bounds__(256) void tensor_amax_kernel(const uint16_t* __restrict__ w,
                                                          long long per_tensor, float* __restrict__ amax) {
    const int t = blockIdx.y;
    const uint16_t* base = w + (long long)t * per_tensor;
    float m = 0.0f;
    const long long n8 = per_tensor / 8;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long long)gridDim.x * 256) {
        u32x4_t v = reinterpret_cast<const u32x4_t*>(base)[i];
        uint32_t a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            m = fmaxf(m, fabsf(__uint_as_float(a[q] << 16)));
            m = fmaxf(m, fabsf(__uint_as_float(a[q] & 0xFFFF0000u)));
        }
    }
    m = wave_max_f32(m);
    __shared__ float sm[4];
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
        atomicMax(reinterpret_cast<unsigned int*>(amax + t), __float_as_uint(r));
    }
}

__global__ void amax_to_global_kernel(float* p, int n) {
    int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        float a = p[i];
        p[i] = a > 0.0f ? __fdiv_rn(a, 2688.0f) : 1.0f;
    }
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_quantize_act(const uint16_t* x, int R, int C, float g, uint8_t* codes, uint8_t* scales,
                               hipStream_t s) {
    long long nb = (long long)R * (C / kBlock);
    if (nb == 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_blocks_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, x, nb,
                       C, 1, (const float*)nullptr, g, codes, scales);
    return hipGetLastError();
}

hipError_t launch_fake_quant_act(const uint16_t* x, int R, int C, float g, uint16_t* out, bool f16_out,
                                 hipStream_t s) {
    long long nb = (long long)R * (C / kBlock);
    if (nb == 0) return hipSuccess;
    if (f16_out)
        hipLaunchKernelGGL(fake_quant_act_kernel<true>, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, x, nb,
                           g, out);
    else
        hipLaunchKernelGGL(fake_quant_act_kernel<false>, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, x, nb,
                           g, out);
    return hipGetLastError();
}

hipError_t launch_quantize_weights(const uint16_t* w, int n, int R, int C, uint8_t* codes,
                                   uint8_t* scales, float* global, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, global, n);
    const long long per = (long long)R * C;
    long long chunks = (per / 8 + 255) / 256;
    if (chunks > 256) chunks = 256;
    if (chunks < 1) chunks = 1;
    hipLaunchKernelGGL(tensor_amax_kernel, dim3((unsigned)chunks, n), dim3(256), 0, s, w, per, global);
    long long nb = (long long)n * R * (C / kBlock);
    if (nb > 0)
        hipLaunchKernelGGL(quantize_blocks_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, w, nb,
                           C, R, (const float*)global, 1.0f, codes, scales);
    hipLaunchKernelGGL(amax_to_global_kernel, dim3((n + 255) / 256), dim3(256), 0, s, global, n);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Checkpoint preparation: expert tensors copied 4 bytes at a time, the two row
// halves of each expert optionally swapped (fused w13 stored up-then-gate), and
// global scales taken as they are or inverted (one correctly rounded fp32
// division).  The page "Serving Solar Open 2 on DGX Spark", section "b12x 버전이
// 실제 NVFP4 체크포인트를 읽어들이도록 만들기".
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prepare_rows_kernel(const uint32_t* __restrict__ src,
                                                           uint32_t* __restrict__ dst, int rows, int row_words,
                                                           int swap_halves) {
    const size_t per_expert = (size_t)rows * row_words;
    const size_t e = blockIdx.y;
    const uint32_t* s = src + e * per_expert;
    uint32_t* o = dst + e * per_expert;
    const int half = rows / 2;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < per_expert; i += (size_t)gridDim.x * 256) {
        const int r = (int)(i / row_words), c = (int)(i - (size_t)r * row_words);
        const int sr = swap_halves ? (r < half ? r + half : r - half) : r;
        o[i] = s[(size_t)sr * row_words + c];
    }
}

__global__ void prepare_global_kernel(const float* __restrict__ src, float* __restrict__ dst, int n, int inverse) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = inverse ? __fdiv_rn(1.0f, src[i]) : src[i];
}

hipError_t launch_prepare_rows(const uint8_t* src, uint8_t* dst, int n, int rows, int row_bytes, bool swap_halves,
                               hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const size_t words = (size_t)rows * (row_bytes / 4);
    const size_t blocks = (words + 255) / 256;
    const unsigned gx = (unsigned)(blocks < 1024 ? blocks : 1024);
    hipLaunchKernelGGL(prepare_rows_kernel, dim3(gx, n), dim3(256), 0, s, reinterpret_cast<const uint32_t*>(src),
                       reinterpret_cast<uint32_t*>(dst), rows, row_bytes / 4, swap_halves ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_prepare_global(const float* src, float* dst, int n, bool inverse, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(prepare_global_kernel, dim3((n + 255) / 256), dim3(256), 0, s, src, dst, n, inverse ? 1 : 0);
    return hipGetLastError();
}

}  // namespace moe
