// Tiled expert GEMMs for many tokens per expert (prefill), gfx950.
//
// A tile is 256 pair rows of one expert group (a local expert, or the shared
// expert over all tokens) x 256 weight rows, K staged 64 at a time through two
// LDS stages (64 KB each):
//   A: the tile's bf16 activation rows, copied straight from global memory into
//      LDS (global_load_lds_dwordx4, no registers), gathered through the
//      permutation for GEMM1;
//   B: the 256 weight rows' NVFP4 codes and E4M3 block scales, decoded ONCE per
//      workgroup to exact bf16 (code * scale has at most 6 significant bits) and
//      written to LDS.
// Both are [row][64] bf16 with the eight 16-byte chunks of a row XOR-swizzled by
// (row & 7), so the MFMA operand reads (32 rows x one chunk) hit distinct banks.
// Eight waves, 2 (rows) x 4 (weight rows); a wave owns 128 x 64 of the tile as
// 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  Lane layout of
// that instruction (checked on the device): lane l holds A[l%32][8(l/32)..+8]
// and B[8(l/32)..+8][l%32]; accumulator value v sits at row 8(v/4) + 4(l/32) +
// v%4, column l%32.
//
// GEMM1 (KIND 1): the 256 weight rows are 128 gate rows [n, n+128) and the
// matching up rows [F+n, F+n+128); a wave's two column blocks are 32 gate and the
// same 32 up columns, so the SwiGLU a = silu(g13*gate) * (g13*up) is formed in
// registers; W4A4 quantize-dequantizes a per 16 columns (16 lanes).  Stored bf16.
// GEMM2 (KIND 2): Y = g2 * acc, fp32 rows.
//
// Workgroups are mapped so that each of the 8 XCDs (hardware workgroup b runs on
// XCD b % 8) takes a contiguous range of (tile, column block) pairs, tile-major:
// the column blocks of a tile share its activation rows in that XCD's L2.
//
// Layer semantics: the page "Serving Solar Open 2 on DGX Spark", sections "수정
// 사항 › b12x에서의 Expert Parallelism 구현 추가" and "b12x 버전이 실제 NVFP4
// 체크포인트를 읽어들이도록 만들기".
#include <type_traits>
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kPM = 256;                       // tile rows
constexpr int kPN = 256;                       // tile weight rows
constexpr int kPK = 64;                        // K per stage
constexpr int kPThreads = 512;
constexpr int kPStage = (kPM + kPN) * kPK * 2; // bytes per stage (A then B)
constexpr int kPLds = 2 * kPStage;             // 128 KB

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ float silu_fast(float z) { return z / (1.0f + __expf(-z)); }

// byte offset of 16-byte chunk c of row r in a swizzled [rows][64 bf16] tile
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

template <int KIND, int MODE>
__global__ __launch_bounds__(kPThreads) void pf_gemm_kernel(GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int d = a.d, F = a.F;
    const int NT = KIND == 1 ? (2 * F) / kPN : (d + kPN - 1) / kPN;
    const int total = *a.ntiles * NT;
    const int b = blockIdx.x, per = (total + 7) >> 3;
    if ((b >> 3) >= per) return;
    const int logical = (b & 7) * per + (b >> 3);
    if (logical >= total) return;
    const int tile = logical / NT, nt = logical - tile * NT;
    const int4 tl = a.tiles[tile];
    const int grp = tl.x, rb = tl.y, re = tl.z;
    const bool shared = grp == a.L;
    const ExpertWeights& W = shared ? a.shared : a.local;
    const size_t ex = shared ? 0 : (size_t)grp;
    const int K = KIND == 1 ? d : F;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;

    // ---- A sources: 4 rows per lane (one per direct load), fixed over K ----
    // load i of wave w fills LDS rows (4w + i) * 8 .. +8; lane -> row + lane/8,
    // LDS slot lane%8, which holds chunk (lane%8) ^ (row & 7) = (lane&7) ^ (lane>>3)
    const uint16_t* asrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (wave * 4 + i) * 8 + (lane >> 3);
        int gr = rb + r;
        if (gr >= re) gr = rb;                           // padding rows: any valid row
        size_t off;
        if (KIND == 1) {
            const int t = shared ? gr - a.T * a.topk : a.perm[gr] / a.topk;
            off = (size_t)t * d;
        } else {
            off = (size_t)gr * F;
        }
        asrc[i] = (KIND == 1 ? (MODE == 1 ? a.hq : a.hidden) : a.act) + off +
                  (((lane & 7) ^ (lane >> 3)) << 3);
    }

    // ---- B source: thread -> LDS weight row j = tid/2, K half h = tid%2 ----
    const int bj = tid >> 1, bh = tid & 1;
    int wrow;
    if (KIND == 1) wrow = (bj < 128 ? 0 : F - 128) + nt * 128 + bj;
    else wrow = min(nt * kPN + bj, d - 1);               // columns past d: any valid row
    const uint8_t* bcode = (KIND == 1 ? W.w13 + ex * (size_t)(2 * F) * (d / 2) : W.w2 + ex * (size_t)d * (F / 2)) +
                           (size_t)wrow * (K / 2) + bh * 16;
    const uint8_t* bscale = (KIND == 1 ? W.w13_s + ex * (size_t)(2 * F) * (d / 16) : W.w2_s + ex * (size_t)d * (F / 16)) +
                            (size_t)wrow * (K / 16) + bh * 2;
    const float gscale = KIND == 1 ? W.g13[ex] : W.g2[ex];

    // valid 32-row blocks of this wave (rows past re are padding)
    const int nvi = max(0, min(4, (re - rb - wm * 128 + 31) >> 5));
    const bool colv = KIND == 1 || nt * kPN + wn * 64 < d;

    auto issue_a = [&](int ks, int buf) {
        uint8_t* base = smem + buf * kPStage + wave * 4 * 1024;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(asrc[i] + ks * kPK), (lds_void_t*)(base + i * 1024),
                                             16, 0, 0);
    };
    auto store_b = [&](u32x4_t codes, uint32_t sc, int buf) {
        uint8_t* base = smem + buf * kPStage + kPM * 128;
        const float s0 = e4m3_to_f32(sc & 0xFFu), s1 = e4m3_to_f32((sc >> 8) & 0xFFu);
        const u32x4_t q0 = dequant8_bf16(codes.x, s0), q1 = dequant8_bf16(codes.y, s0);
        const u32x4_t q2 = dequant8_bf16(codes.z, s1), q3 = dequant8_bf16(codes.w, s1);
        *reinterpret_cast<u32x4_t*>(base + swz(bj, bh * 4 + 0)) = q0;
        *reinterpret_cast<u32x4_t*>(base + swz(bj, bh * 4 + 1)) = q1;
        *reinterpret_cast<u32x4_t*>(base + swz(bj, bh * 4 + 2)) = q2;
        *reinterpret_cast<u32x4_t*>(base + swz(bj, bh * 4 + 3)) = q3;
    };
    auto load_codes = [&](int ks) { return *reinterpret_cast<const u32x4_t*>(bcode + ks * (kPK / 2)); };
    auto load_scales = [&](int ks) {
        return (uint32_t)*reinterpret_cast<const uint16_t*>(bscale + ks * (kPK / 16));
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // LDS rows of this lane's operands
    const int arow0 = wm * 128 + (lane & 31);
    const int brow0 = KIND == 1 ? wn * 32 + (lane & 31) : wn * 64 + (lane & 31);
    const int brow1 = KIND == 1 ? 128 + wn * 32 + (lane & 31) : wn * 64 + 32 + (lane & 31);
    const int khalf = lane >> 5;

    auto compute = [&](int buf, auto nvi_c) {
        constexpr int NV = decltype(nvi_c)::value;
        const uint8_t* As = smem + buf * kPStage;
        const uint8_t* Bs = As + kPM * 128;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int c = kk * 2 + khalf;
            bf16x8_t av[4], bv[2];
            bv[0] = *reinterpret_cast<const bf16x8_t*>(Bs + swz(brow0, c));
            bv[1] = *reinterpret_cast<const bf16x8_t*>(Bs + swz(brow1, c));
#pragma unroll
            for (int i = 0; i < NV; ++i) av[i] = *reinterpret_cast<const bf16x8_t*>(As + swz(arow0 + i * 32, c));
#pragma unroll
            for (int i = 0; i < NV; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
    };
    auto compute_any = [&](int buf) {
        if (!colv) return;
        switch (nvi) {
            case 4: compute(buf, std::integral_constant<int, 4>{}); break;
            case 3: compute(buf, std::integral_constant<int, 3>{}); break;
            case 2: compute(buf, std::integral_constant<int, 2>{}); break;
            case 1: compute(buf, std::integral_constant<int, 1>{}); break;
            default: break;
        }
    };

    const int nk = K / kPK;
    // prologue: stage 0
    issue_a(0, 0);
    store_b(load_codes(0), load_scales(0), 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
        const int cur = ks & 1;
        const bool more = ks + 1 < nk;
        u32x4_t nc = {0u, 0u, 0u, 0u};
        uint32_t nsc = 0u;
        if (more) {
            issue_a(ks + 1, cur ^ 1);
            nc = load_codes(ks + 1);
            nsc = load_scales(ks + 1);
        }
        compute_any(cur);
        if (more) store_b(nc, nsc, cur ^ 1);
        __builtin_amdgcn_s_waitcnt(0);      // the direct LDS loads are not tracked by the compiler
        __syncthreads();
    }

    // ---- epilogue ----
    if (!colv) return;
    const int lr = (lane >> 5) * 4;                       // row offset of this lane within an 8-row group
    if (KIND == 1) {
        const int col = nt * 128 + wn * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i >= nvi) break;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = rb + wm * 128 + i * 32 + (v >> 2) * 8 + lr + (v & 3);
                float av = silu_fast(acc[i][0][v] * gscale) * (acc[i][1][v] * gscale);
                if (MODE == 1) {
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
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i >= nvi) break;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = nt * kPN + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = rb + wm * 128 + i * 32 + (v >> 2) * 8 + lr + (v & 3);
                    if (row < re) a.Y[(size_t)row * d + col] = acc[i][j][v] * gscale;
                }
            }
        }
    }
}

template <int KIND, int MODE>
static hipError_t launch_pf(const GemmArgs& a, hipStream_t s) {
    static bool attr_set = false;   // per process; the attribute is per function
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)pf_gemm_kernel<KIND, MODE>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kPLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int NT = KIND == 1 ? (2 * a.F) / kPN : (a.d + kPN - 1) / kPN;
    const long long n = (long long)a.max_tiles * NT;
    const long long grid = (n + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((pf_gemm_kernel<KIND, MODE>), dim3((unsigned)grid), dim3(kPThreads), kPLds, s, a);
    return hipGetLastError();
}

int pf_rows() { return kPM; }

hipError_t launch_gemm1(const GemmArgs& a, int /*path*/, hipStream_t s) {
    return a.mode == 0 ? launch_pf<1, 0>(a, s) : launch_pf<1, 1>(a, s);
}

hipError_t launch_gemm2(const GemmArgs& a, int /*path*/, hipStream_t s) {
    return launch_pf<2, 0>(a, s);
}

}  // namespace moe
