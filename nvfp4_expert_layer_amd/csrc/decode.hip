// Weight-streaming expert GEMMs for small token counts per expert (gfx950).
//
// When each expert sees only a few tokens (decode, or a shard's share of a small
// batch) the layer is bound by streaming the NVFP4 weights from HBM once.  Each
// wave owns 16 weight rows, loads 32 contiguous code bytes per lane per step with
// a two-step register prefetch, and the workgroup's waves share the token rows
// through LDS, staged in double-buffered 512-element K chunks.
//
// Block-diagonal MFMA (v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8 k] and
// B[8 k][l%16]; D[4 rows][l%16]).  The reduction index is a free permutation:
// K is cut into chunks of 64 elements (32 code bytes, 4 E4M3 scale bytes); at
// step i lane group g = l/16 takes chunk 4i + g, so the four lanes of a weight
// row read one whole 128-byte line per step.  B = the codes decoded UNSCALED to bf16 (v_cvt_scalef32_pk_bf16_fp4
// with scale 1: exact, one instruction per two codes).  A row m = 4 j + t holds
// token t of the current group of four, restricted to the K elements of lane
// group j (zero elsewhere).  An MFMA pair over 16 consecutive elements of the
// chunk then yields, in lane group j, the four tokens' partial dot products
// over exactly one 16-element block of row n -- the block whose E4M3 scale that
// lane already holds -- so the scale is applied with one fp32 FMA per output.
// After the K loop the four lane groups are summed (two xor-shuffles) and the
// fp32 global scale is applied.  Cost: ~0.8 VALU op per weight element for four
// tokens, against ~2 for dequantize-then-MFMA.
//
// GEMM1 epilogue: a = silu(gate) * up (rows [0,F) of w13 gate, [F,2F) up), bf16;
// W4A4 quantize-dequantizes a per 16 columns.  GEMM2: Y = acc * g2 (fp32 rows).
// Layer semantics: the page "Serving Solar Open 2 on DGX Spark", sections "수정
// 사항 › b12x에서의 Expert Parallelism 구현 추가" and "b12x 버전이 실제 NVFP4
// 체크포인트를 읽어들이도록 만들기".
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kDecWaves = 4;        // waves per workgroup, 16 weight rows each
constexpr int kDecRows = 16;        // token rows per tile (four groups of four)
constexpr int kChunk = 512;         // K elements per LDS chunk (4 steps of 128)
constexpr int kAPad = 8;            // bf16 padding per LDS row
constexpr int kLdsElems = 2 * kDecRows * (kChunk + kAPad);

__device__ __forceinline__ uint32_t load_u16(const uint8_t* p) {
    return *reinterpret_cast<const uint16_t*>(p);
}

// Streams K for NR weight-row groups (16 rows each) against the tile's token
// rows.  codes[r]/scales[r]: this lane's row at its first chunk.  arows: the
// tile's token rows (bf16, K long), ntok of them valid.  Leaves per lane, for
// each of the 4 token groups, the 4 tokens' sums over this lane group's K share.
// A step covers 256 elements of K: lane group g takes the 64-element chunk
// 4 i + g (32 code bytes, 4 scale bytes); chunks past K (K % 256 == 128) are
// skipped by the two upper lane groups.
template <int NR>
__device__ __forceinline__ void dec_stream(const uint16_t* const* __restrict__ arows, int ntok, int K,
                                           const uint8_t* const (&codes)[NR],
                                           const uint8_t* const (&scales)[NR], uint16_t* lds,
                                           f32x4_t (&acc)[4][NR]) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const int ntg = (ntok + 3) >> 2;
    const int nsteps = (K + 255) / 256, nchunks = (K + kChunk - 1) / kChunk;   // K % 128 == 0
    constexpr int LDW = kChunk + kAPad;                      // LDS row stride (elements)
    uint16_t* const buf0 = lds;
    uint16_t* const buf1 = lds + kDecRows * LDW;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg)
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[tg][r] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // A staging: 16 rows x 512 elements = 1024 pieces of 16 bytes, 4 per thread;
    // rows >= ntok are neither loaded nor read.
    static_assert(64 * kDecWaves * 4 == kDecRows * kChunk / 8, "A staging covers the chunk");
    u32x4_t va[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int piece = tid + j * (64 * kDecWaves);
        const int row = piece >> 6, col = (piece & 63) * 8;
        if (row < ntok && col < K) {
            va[j] = *reinterpret_cast<const u32x4_t*>(arows[row] + col);
            *reinterpret_cast<u32x4_t*>(buf0 + row * LDW + col) = va[j];
        }
    }

    // weight prefetch, two steps ahead (32 code bytes + 4 scale bytes per step)
    const u32x4_t zero4 = {0u, 0u, 0u, 0u};
    auto load_codes = [&](int r, int step, u32x4_t& lo, u32x4_t& hi, uint32_t& sc) {
        if ((step * 4 + g) * 64 < K) {
            const u32x4_t* p = reinterpret_cast<const u32x4_t*>(codes[r] + (size_t)step * 128);
            lo = p[0];
            hi = p[1];
            sc = *reinterpret_cast<const uint32_t*>(scales[r] + (size_t)step * 16);
        } else {
            lo = zero4;
            hi = zero4;
            sc = 0u;
        }
    };
    u32x4_t c0l[NR], c0h[NR], c1l[NR], c1h[NR];
    uint32_t s0[NR], s1[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        load_codes(r, 0, c0l[r], c0h[r], s0[r]);
        c1l[r] = zero4; c1h[r] = zero4; s1[r] = 0u;
        if (nsteps > 1) load_codes(r, 1, c1l[r], c1h[r], s1[r]);
    }
    // block-diagonal ownership: A row m = 4 j + t is non-zero only in lane group j
    const bool aown = (n >> 2) == g;
    const int tsub = n & 3;

    for (int ch = 0; ch < nchunks; ++ch) {
        __syncthreads();                                     // chunk ch staged, chunk ch-1 consumed
        const bool more = ch + 1 < nchunks;
        if (more) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int piece = tid + j * (64 * kDecWaves);
                const int row = piece >> 6, col = (piece & 63) * 8;
                if (row < ntok && (ch + 1) * kChunk + col < K)
                    va[j] = *reinterpret_cast<const u32x4_t*>(arows[row] + (ch + 1) * kChunk + col);
            }
        }
        const uint16_t* ab = (ch & 1) ? buf1 : buf0;
#pragma unroll
        for (int si = 0; si < kChunk / 256; ++si) {
            const int step = ch * (kChunk / 256) + si;
            if (step >= nsteps) break;                       // last chunk may hold fewer steps
            u32x4_t cl[NR], chh[NR];
            uint32_t sc[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                cl[r] = c0l[r]; chh[r] = c0h[r]; sc[r] = s0[r];
                c0l[r] = c1l[r]; c0h[r] = c1h[r]; s0[r] = s1[r];
            }
            if (step + 2 < nsteps) {
#pragma unroll
                for (int r = 0; r < NR; ++r) load_codes(r, step + 2, c1l[r], c1h[r], s1[r]);
            }
            const bool kvalid = (step * 4 + g) * 64 < K;
            const int kcol = (si * 4 + g) * 64;              // this lane group's chunk inside the LDS chunk
#pragma unroll
            for (int r = 0; r < NR; ++r) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    // 32 of the chunk's 64 elements: two 16-element blocks
                    const u32x4_t c = h ? chh[r] : cl[r];
                    bf16x8_t b[4];
                    b[0] = __builtin_bit_cast(bf16x8_t, fp4x8_to_bf16(c.x));
                    b[1] = __builtin_bit_cast(bf16x8_t, fp4x8_to_bf16(c.y));
                    b[2] = __builtin_bit_cast(bf16x8_t, fp4x8_to_bf16(c.z));
                    b[3] = __builtin_bit_cast(bf16x8_t, fp4x8_to_bf16(c.w));
                    const float sa = e4m3_to_f32((sc[r] >> (16 * h)) & 0xFFu);
                    const float sb = e4m3_to_f32((sc[r] >> (16 * h + 8)) & 0xFFu);
#pragma unroll
                    for (int tg = 0; tg < 4; ++tg) {
                        if (tg < ntg) {
                            u32x4_t av[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q) av[q] = zero4;
                            const int tok = tg * 4 + tsub;
                            if (aown && kvalid && tok < ntok) {
                                const uint16_t* p = ab + tok * LDW + kcol + h * 32;
#pragma unroll
                                for (int q = 0; q < 4; ++q) av[q] = *reinterpret_cast<const u32x4_t*>(p + q * 8);
                            }
                            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
                            f32x4_t da = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, av[0]), b[0], z, 0, 0, 0);
                            da = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[1]),
                                                                         b[1], da, 0, 0, 0);
                            f32x4_t db = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, av[2]), b[2], z, 0, 0, 0);
                            db = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[3]),
                                                                         b[3], db, 0, 0, 0);
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                acc[tg][r][q] = fmaf(sb, db[q], fmaf(sa, da[q], acc[tg][r][q]));
                        }
                    }
                }
            }
        }
        if (more) {
            uint16_t* nb = (ch & 1) ? buf0 : buf1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int piece = tid + j * (64 * kDecWaves);
                const int row = piece >> 6, col = (piece & 63) * 8;
                if (row < ntok && (ch + 1) * kChunk + col < K) *reinterpret_cast<u32x4_t*>(nb + row * LDW + col) = va[j];
            }
        }
    }
}

// Sum of a value over the four lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float lane_group_sum(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// Tile set-up shared by both GEMMs.
struct DecTile {
    int grp, rb, re;
    bool shared;
    size_t ex;
};

__device__ __forceinline__ DecTile dec_tile(const GemmArgs& a) {
    const int4 tl = a.tiles[blockIdx.x];
    DecTile t;
    t.grp = tl.x;
    t.rb = tl.y;
    t.re = tl.z;
    t.shared = tl.x == a.L;
    t.ex = t.shared ? 0 : (size_t)tl.x;
    return t;
}

// ---------------------------------------------------------------------------
// GEMM1 + SwiGLU: a wave = 16 SwiGLU columns (16 gate + 16 up rows of w13) for a
// tile of <= 16 token rows.  grid (max_tiles, F / (16 * kDecWaves)).
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(3))) void dec_gemm1_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsElems];
    __shared__ const uint16_t* s_arow[kDecRows];
    if ((int)blockIdx.x >= *a.ntiles) return;
    const DecTile tl = dec_tile(a);
    const ExpertWeights& W = tl.shared ? a.shared : a.local;
    const int d = a.d, F = a.F;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col0 = (blockIdx.y * kDecWaves + wave) * 16;
    const int n = lane & 15, g = lane >> 4;
    const int ntok = tl.re - tl.rb;
    const uint16_t* act_in = MODE == 0 ? a.hidden : a.hq;
    if (tid < kDecRows) {
        const int row = tl.rb + tid;
        int t = 0;
        if (row < tl.re) t = tl.shared ? row - a.T * a.topk : a.perm[row] / a.topk;
        s_arow[tid] = act_in + (size_t)t * d;
    }
    __syncthreads();
    const uint8_t* w13 = W.w13 + tl.ex * (size_t)(2 * F) * (d / 2);
    const uint8_t* w13s = W.w13_s + tl.ex * (size_t)(2 * F) * (d / 16);
    const uint8_t* const codes[2] = {w13 + (size_t)(col0 + n) * (d / 2) + g * 32,
                                     w13 + (size_t)(F + col0 + n) * (d / 2) + g * 32};
    const uint8_t* const scales[2] = {w13s + (size_t)(col0 + n) * (d / 16) + g * 4,
                                      w13s + (size_t)(F + col0 + n) * (d / 16) + g * 4};
    f32x4_t acc[4][2];
    dec_stream<2>(s_arow, ntok, d, codes, scales, lds, acc);

    const float g13 = W.g13[tl.ex];
    const int col = col0 + n;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
        // every lane group joins the shuffles; lane group g keeps token 4 tg + g
        float gt = 0.f, up = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float sgt = lane_group_sum(acc[tg][0][q]), sup = lane_group_sum(acc[tg][1][q]);
            if (q == g) { gt = sgt; up = sup; }
        }
        gt *= g13;
        up *= g13;
        float av = gt / (1.0f + expf(-gt)) * up;
        if (MODE == 1) {
            // NVFP4 quantize-dequantize over the 16 columns of this lane group
            float m = fabsf(av);
            m = fmaxf(m, __shfl_xor(m, 1, 64));
            m = fmaxf(m, __shfl_xor(m, 2, 64));
            m = fmaxf(m, __shfl_xor(m, 4, 64));
            m = fmaxf(m, __shfl_xor(m, 8, 64));
            av = nvfp4_fake_quant(av, m);
        }
        const int r = tl.rb + tg * 4 + g;
        if (r < tl.re) a.act[(size_t)r * F + col] = (uint16_t)f32_to_bf16_rne(av);
    }
}

// ---------------------------------------------------------------------------
// GEMM2: a wave = 16 output columns (16 rows of w2).  grid (max_tiles, d / 64).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * kDecWaves) void dec_gemm2_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsElems];
    __shared__ const uint16_t* s_arow[kDecRows];
    if ((int)blockIdx.x >= *a.ntiles) return;
    const DecTile tl = dec_tile(a);
    const ExpertWeights& W = tl.shared ? a.shared : a.local;
    const int d = a.d, F = a.F;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col0 = (blockIdx.y * kDecWaves + wave) * 16;
    const int n = lane & 15, g = lane >> 4;
    const int ntok = tl.re - tl.rb;
    if (tid < kDecRows) s_arow[tid] = a.act + (size_t)(tl.rb + (tid < ntok ? tid : 0)) * F;
    __syncthreads();
    const uint8_t* w2 = W.w2 + tl.ex * (size_t)d * (F / 2);
    const uint8_t* w2s = W.w2_s + tl.ex * (size_t)d * (F / 16);
    const uint8_t* const codes[1] = {w2 + (size_t)(col0 + n) * (F / 2) + g * 32};
    const uint8_t* const scales[1] = {w2s + (size_t)(col0 + n) * (F / 16) + g * 4};
    f32x4_t acc[4][1];
    dec_stream<1>(s_arow, ntok, F, codes, scales, lds, acc);
    const float g2 = W.g2[tl.ex];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
        float y = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float v = lane_group_sum(acc[tg][0][q]);
            if (q == g) y = v;
        }
        const int r = tl.rb + tg * 4 + g;
        if (r < tl.re) a.Y[(size_t)r * d + col0 + n] = y * g2;
    }
}

hipError_t launch_dec_gemm1(const GemmArgs& a, hipStream_t s) {
    dim3 grid(a.max_tiles, a.F / (16 * kDecWaves));
    if (a.mode == 0) hipLaunchKernelGGL(dec_gemm1_kernel<0>, grid, dim3(64 * kDecWaves), 0, s, a);
    else hipLaunchKernelGGL(dec_gemm1_kernel<1>, grid, dim3(64 * kDecWaves), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_dec_gemm2(const GemmArgs& a, hipStream_t s) {
    dim3 grid(a.max_tiles, a.d / (16 * kDecWaves));
    hipLaunchKernelGGL(dec_gemm2_kernel, grid, dim3(64 * kDecWaves), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
