// Grouped expert GEMMs with NVFP4 weights (gfx950, bf16 MFMA 16x16x32, fp32
// accumulation) and the weighted combine.
//
// Per tile of BM permuted-pair rows of one expert group (a local expert, or the
// shared expert over all tokens):
//   GEMM1: U = A W13^T with A = hidden rows gathered through the permutation
//          (W4A4: their NVFP4 codes dequantized), W13 rows [0,F) gate and [F,2F)
//          up decoded exactly to bf16 (E2M1 code * E4M3 scale); the fp32 global
//          scale multiplies the fp32 accumulator; epilogue a = silu(gate) * up,
//          stored bf16 (W4A16) or NVFP4-quantized per 16 along F (W4A4).
//   GEMM2: Y = a W2^T * g2, fp32 rows staged per pair.
//   combine: out[t] = sum_j w_tj Y[row(t, j)] (kept pairs, slot order) + Y[shared row of t],
//            a fixed summation order, so the output is deterministic.
// The layer follows the page "Serving Solar Open 2 on DGX Spark", sections "수정
// 사항 › b12x에서의 Expert Parallelism 구현 추가" (shard-relative expert ids,
// per-shard partial sum) and "b12x 버전이 실제 NVFP4 체크포인트를 읽어들이도록
// 만들기" (packed FP4 weights, FP8 block scales, per-expert global scale, fused
// gate/up projection).
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kBK = 64;
constexpr int kPad = 8;

// Stage one 16-element K-chunk of NVFP4 data (8 code bytes + 1 scale byte) as
// 16 exact bf16 into LDS.
__device__ __forceinline__ void stage_fp4_chunk(uint16_t* dst, const uint8_t* codes, uint8_t sbyte) {
    u32x2_t c = *reinterpret_cast<const u32x2_t*>(codes);
    float s = e4m3_to_f32(sbyte);
    *reinterpret_cast<u32x4_t*>(dst) = dequant8_bf16(c.x, s);
    *reinterpret_cast<u32x4_t*>(dst + 8) = dequant8_bf16(c.y, s);
}

__device__ __forceinline__ void stage_bf16_chunk(uint16_t* dst, const uint16_t* src) {
    *reinterpret_cast<u32x4_t*>(dst) = *reinterpret_cast<const u32x4_t*>(src);
    *reinterpret_cast<u32x4_t*>(dst + 8) = *reinterpret_cast<const u32x4_t*>(src + 8);
}

__device__ __forceinline__ void zero_chunk(uint16_t* dst) {
    u32x4_t z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4_t*>(dst) = z;
    *reinterpret_cast<u32x4_t*>(dst + 8) = z;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------
// GEMM1 + SwiGLU.  Tile: BM rows x 64 SwiGLU columns (64 gate + 64 up weight rows).
// Waves: WM x WN = 4; a wave owns BM/WM rows and 64/WN SwiGLU columns.
// ---------------------------------------------------------------------------
template <int BM, int WM, int MODE>
__global__ __launch_bounds__(256) void gemm1_swiglu_kernel(GemmArgs a) {
    constexpr int WN = 4 / WM;
    constexpr int RT = BM / (16 * WM);        // 16-row tiles per wave
    constexpr int CT = 4 / WN;                 // 16-column gate tiles per wave (same for up)
    constexpr int BNH = 64;
    static_assert(RT >= 1 && CT >= 1, "tile shape");
    __shared__ __attribute__((aligned(16))) uint16_t As[BM][kBK + kPad];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2 * BNH][kBK + kPad];

    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int4 tl = a.tiles[tile];
    const int grp = tl.x, rb = tl.y, re = tl.z;
    const bool shared = grp == a.L;
    const ExpertWeights& W = shared ? a.shared : a.local;
    const size_t ex = shared ? 0 : (size_t)grp;
    const int d = a.d, F = a.F;
    const int n0 = blockIdx.y * BNH;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    const uint8_t* w13 = W.w13 + ex * (size_t)(2 * F) * (d / 2);
    const uint8_t* w13s = W.w13_s + ex * (size_t)(2 * F) * (d / 16);
    const float g13 = W.g13[ex];

    // tokens of the A chunks this thread stages (fixed over the K loop)
    constexpr int ACH = (BM * (kBK / 16) + 255) / 256;
    int atok[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        int c = tid + i * 256;
        int r = c / (kBK / 16);
        int gr = rb + r;
        int t = -1;
        if (c < BM * (kBK / 16) && gr < re) {
            if (shared) t = gr - a.T * a.topk;
            else t = a.perm[gr] / a.topk;
        }
        atok[i] = t;
    }

    f32x4_t acc[RT][2 * CT];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < 2 * CT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < d; k0 += kBK) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            int c = tid + i * 256;
            if (c < BM * (kBK / 16)) {
                int r = c / (kBK / 16), kc = (c % (kBK / 16)) * 16;
                uint16_t* dst = &As[r][kc];
                int t = atok[i];
                if (t < 0) zero_chunk(dst);
                else stage_bf16_chunk(dst, (MODE == 0 ? a.hidden : a.hq) + (size_t)t * d + k0 + kc);
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int c = tid + i * 256;               // 0..511: 128 rows x 4 chunks
            int j = c >> 2, kc = (c & 3) * 16;
            int wrow = j < BNH ? n0 + j : F + n0 + (j - BNH);
            stage_fp4_chunk(&Bs[j][kc], w13 + (size_t)wrow * (d / 2) + (k0 + kc) / 2,
                            w13s[(size_t)wrow * (d / 16) + (k0 + kc) / 16]);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 32) {
            bf16x8_t av[RT], bv[2 * CT];
#pragma unroll
            for (int i = 0; i < RT; ++i)
                av[i] = *reinterpret_cast<const bf16x8_t*>(
                    &As[wm * (BM / WM) + i * 16 + (lane & 15)][kk + (lane >> 4) * 8]);
#pragma unroll
            for (int j = 0; j < CT; ++j) {
                int col = wn * (BNH / WN) + j * 16 + (lane & 15);
                bv[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[col][kk + (lane >> 4) * 8]);
                bv[CT + j] = *reinterpret_cast<const bf16x8_t*>(&Bs[BNH + col][kk + (lane >> 4) * 8]);
            }
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int j = 0; j < 2 * CT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // epilogue: SwiGLU, store
#pragma unroll
    for (int i = 0; i < RT; ++i) {
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            const int col = n0 + wn * (BNH / WN) + j * 16 + (lane & 15);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = rb + wm * (BM / WM) + i * 16 + (lane >> 4) * 4 + q;
                const float gt = acc[i][j][q] * g13;
                const float up = acc[i][CT + j][q] * g13;
                float av = silu_f32(gt) * up;
                if (MODE == 1) {
                    // NVFP4 quantize-dequantize over the 16 consecutive columns held
                    // by the 16 lanes of this row group
                    float m = fabsf(av);
                    m = fmaxf(m, __shfl_xor(m, 1, 64));
                    m = fmaxf(m, __shfl_xor(m, 2, 64));
                    m = fmaxf(m, __shfl_xor(m, 4, 64));
                    m = fmaxf(m, __shfl_xor(m, 8, 64));
                    av = nvfp4_fake_quant(av, m);
                }
                if (row < re) a.act[(size_t)row * F + col] = (uint16_t)f32_to_bf16_rne(av);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// GEMM2: Y = a W2^T * g2.  Tile: BM rows x 128 output columns.
// ---------------------------------------------------------------------------
template <int BM, int WM, int MODE>
__global__ __launch_bounds__(256) void gemm2_kernel(GemmArgs a) {
    constexpr int WN = 4 / WM;
    constexpr int RT = BM / (16 * WM);
    constexpr int BN = 128;
    constexpr int CT = BN / (16 * WN);
    static_assert(RT >= 1 && CT >= 1, "tile shape");
    __shared__ __attribute__((aligned(16))) uint16_t As[BM][kBK + kPad];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN][kBK + kPad];

    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int4 tl = a.tiles[tile];
    const int grp = tl.x, rb = tl.y, re = tl.z;
    const bool shared = grp == a.L;
    const ExpertWeights& W = shared ? a.shared : a.local;
    const size_t ex = shared ? 0 : (size_t)grp;
    const int d = a.d, F = a.F;
    const int n0 = blockIdx.y * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    const uint8_t* w2 = W.w2 + ex * (size_t)d * (F / 2);
    const uint8_t* w2s = W.w2_s + ex * (size_t)d * (F / 16);
    const float g2 = W.g2[ex];

    f32x4_t acc[RT][CT];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    constexpr int ACH = (BM * (kBK / 16) + 255) / 256;
    for (int k0 = 0; k0 < F; k0 += kBK) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            int c = tid + i * 256;
            if (c < BM * (kBK / 16)) {
                int r = c / (kBK / 16), kc = (c % (kBK / 16)) * 16;
                int gr = rb + r;
                uint16_t* dst = &As[r][kc];
                if (gr >= re) zero_chunk(dst);
                else stage_bf16_chunk(dst, a.act + (size_t)gr * F + k0 + kc);
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int c = tid + i * 256;               // 128 rows x 4 chunks
            int j = c >> 2, kc = (c & 3) * 16;
            int wrow = n0 + j;
            stage_fp4_chunk(&Bs[j][kc], w2 + (size_t)wrow * (F / 2) + (k0 + kc) / 2,
                            w2s[(size_t)wrow * (F / 16) + (k0 + kc) / 16]);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 32) {
            bf16x8_t av[RT], bv[CT];
#pragma unroll
            for (int i = 0; i < RT; ++i)
                av[i] = *reinterpret_cast<const bf16x8_t*>(
                    &As[wm * (BM / WM) + i * 16 + (lane & 15)][kk + (lane >> 4) * 8]);
#pragma unroll
            for (int j = 0; j < CT; ++j)
                bv[j] = *reinterpret_cast<const bf16x8_t*>(
                    &Bs[wn * (BN / WN) + j * 16 + (lane & 15)][kk + (lane >> 4) * 8]);
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int j = 0; j < CT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            const int col = n0 + wn * (BN / WN) + j * 16 + (lane & 15);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = rb + wm * (BM / WM) + i * 16 + (lane >> 4) * 4 + q;
                if (row < re) a.Y[(size_t)row * d + col] = acc[i][j][q] * g2;
            }
        }
}

// ---------------------------------------------------------------------------
// combine: one thread per 8 output columns of a token.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const int per_row = a.d / 8;
    if (idx >= (long long)a.T * per_row) return;
    const int t = (int)(idx / per_row), c0 = (int)(idx % per_row) * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < a.topk; ++j) {
        const int row = a.inv[(size_t)t * a.topk + j];
        if (row < 0) continue;
        const float w = a.topk_w[(size_t)t * a.topk + j];
        const f32x4_t* y = reinterpret_cast<const f32x4_t*>(a.Y + (size_t)row * a.d + c0);
        f32x4_t y0 = y[0], y1 = y[1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            s[q] = fmaf(w, y0[q], s[q]);
            s[4 + q] = fmaf(w, y1[q], s[4 + q]);
        }
    }
    if (a.has_shared) {
        const f32x4_t* y = reinterpret_cast<const f32x4_t*>(a.Y + ((size_t)a.T * a.topk + t) * a.d + c0);
        f32x4_t y0 = y[0], y1 = y[1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            s[q] += y0[q];
            s[4 + q] += y1[q];
        }
    }
    u32x4_t o;
    o.x = f32_to_bf16_rne(s[0]) | (f32_to_bf16_rne(s[1]) << 16);
    o.y = f32_to_bf16_rne(s[2]) | (f32_to_bf16_rne(s[3]) << 16);
    o.z = f32_to_bf16_rne(s[4]) | (f32_to_bf16_rne(s[5]) << 16);
    o.w = f32_to_bf16_rne(s[6]) | (f32_to_bf16_rne(s[7]) << 16);
    *reinterpret_cast<u32x4_t*>(a.out + (size_t)t * a.d + c0) = o;
}

// ---------------------------------------------------------------------------
int gemm_bm(int path, int T, int topk, int E) { return path == 1 ? dec_rows(T, topk, E) : 64; }

hipError_t launch_gemm1(const GemmArgs& a, int path, hipStream_t s) {
    dim3 grid(a.max_tiles, a.F / 64);
    if (path == 1) {
        if (a.mode == 0) hipLaunchKernelGGL((gemm1_swiglu_kernel<16, 1, 0>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((gemm1_swiglu_kernel<16, 1, 1>), grid, dim3(256), 0, s, a);
    } else {
        if (a.mode == 0) hipLaunchKernelGGL((gemm1_swiglu_kernel<64, 4, 0>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((gemm1_swiglu_kernel<64, 4, 1>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_gemm2(const GemmArgs& a, int path, hipStream_t s) {
    dim3 grid(a.max_tiles, a.d / 128);
    if (path == 1) hipLaunchKernelGGL((gemm2_kernel<16, 1, 0>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gemm2_kernel<64, 4, 0>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    long long n = (long long)a.T * (a.d / 8);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
