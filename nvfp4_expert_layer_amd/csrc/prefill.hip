// Tiled expert GEMMs for many tokens per expert (prefill), gfx950.
//
// A tile is 256 pair rows of one expert group (a local expert, or the shared
// expert over all tokens) x 256 weight rows, K staged 64 at a time (160 KB of
// LDS, the whole of a CU's):
//   A: the tile's bf16 activation rows, copied straight from global memory into
//      a 3-slot LDS ring (global_load_lds_dwordx4, no registers), gathered
//      through the permutation for GEMM1;
//   B: the 256 weight rows' NVFP4 codes and E4M3 block scales, decoded ONCE per
//      workgroup to exact bf16 (code * scale has at most 6 significant bits)
//      into a 2-slot LDS buffer.
// Both are [row][64] bf16 with the eight 16-byte chunks of a row XOR-swizzled by
// (row & 7), so the MFMA operand reads (32 rows x one chunk) hit distinct banks.
// WAVES = 8 (two per SIMD, the default) or 4 (one per SIMD) waves as 2 (rows) x
// WAVES/2 (weight rows); a wave owns 128 x (512/WAVES) of the tile as blocks of
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  Two waves per SIMD hide each
// other's LDS waits; one wave per SIMD halves the B operand reads but stalls on
// every LDS wait (measured slower).  Lane layout of
// that instruction (checked on the device): lane l holds A[l%32][8(l/32)..+8]
// and B[8(l/32)..+8][l%32]; accumulator value v sits at row 8(v/4) + 4(l/32) +
// v%4, column l%32.
//
// GEMM1 (KIND 1): the 256 weight rows are 128 gate rows [n, n+128) and the
// matching up rows [F+n, F+n+128); a wave's column blocks are gate columns and
// the same up columns, so the SwiGLU a = silu(g13*gate) * (g13*up) is formed
// in registers; W4A4 quantize-dequantizes a per 16 columns (16 lanes).  Stored
// bf16.
// GEMM2 (KIND 2): Y = g2 * acc, bf16 rows (through LDS, 16-byte stores).
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
constexpr int kPA = kPM * kPK * 2;             // bytes of one A stage (32 KB)
constexpr int kPB = kPN * kPK * 2;             // bytes of one decoded B stage (32 KB)
constexpr int kPRawC = kPN * (kPK / 2);        // raw codes of one step (8 KB: 32 B per weight row)
constexpr int kPRaw = kPRawC + kPN * 4;        // + raw scales (1 KB: 4 B per weight row)
constexpr int kPOffB = 2 * kPA;                // LDS map: A[2] | B[2] | raw[3]
constexpr int kPOffR = kPOffB + 2 * kPB;
constexpr int kPLds = kPOffR + 3 * kPRaw;      // 155 KB of the CU's 160 KB

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ float silu_fast(float z) { return z / (1.0f + __expf(-z)); }

// Byte offset of 16-byte chunk c of row r in a swizzled [rows][64 bf16] tile.
// Any 8 consecutive rows (aligned) put a given chunk in 8 different 16-byte
// slots, and rows r, r + 8 differ again in the slot's low bit, so a 32-row
// operand read is free of bank conflicts whether the LDS serves 8 or 16 lanes of
// a 16-byte access per cycle.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 4); }

template <int KIND, int MODE, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void pf_gemm_kernel(GemmArgs a) {
    constexpr int WN = WAVES / 2;                  // waves along the weight rows
    constexpr int NJ = kPN / WN / 32;              // 32-column blocks per wave (2 or 4)
    constexpr int NA = 32 / WAVES;                 // A loads (1 KB) per wave per step
    constexpr int NC = 8 / WAVES;                  // raw code loads (1 KB) per wave per step
    constexpr int SL = 256 / WAVES;                // raw scale rows per wave (lanes)
    constexpr int NLOAD = NA + NC + 1;             // direct loads per wave per step
    constexpr int NRAW = NC + 1;                   // of which raw (issued last)
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
    const int wm = wave / WN, wn = wave % WN;

    // ---- A sources: NA rows per lane (one per direct load), fixed over K ----
    // load q of wave w fills LDS rows 8 (NA w + q) .. +8 (1 KB, lane i at byte 16 i):
    // lane i -> row r = 8 (NA w + q) + i/8, 16-byte slot i%8, which must hold chunk
    // (i%8) ^ (r & 7) ^ ((r >> 3) & 1) = (i & 7) ^ (i >> 3) ^ (q & 1)  (NA is even)
    const uint16_t* asrc[NA];
#pragma unroll
    for (int q = 0; q < NA; ++q) {
        const int r = (wave * NA + q) * 8 + (lane >> 3);
        int gr = rb + r;
        if (gr >= re) gr = rb;                           // padding rows: any valid row
        size_t off;
        if (KIND == 1) {
            const int t = shared ? gr - a.T * a.topk : a.perm[gr] / a.topk;
            off = (size_t)t * d;
        } else {
            off = (size_t)gr * F;
        }
        asrc[q] = (KIND == 1 ? (MODE == 1 ? a.hq : a.hidden) : a.act) + off +
                  (((lane & 7) ^ (lane >> 3) ^ (q & 1)) << 3);
    }

    // ---- raw weight sources (copied to LDS as they are, decoded from there) ----
    // codes: load q of wave w, lane i -> weight row r = 32 (NC w + q) + i/2, bytes
    // 16 (i%2) .. +16 of its 32 code bytes per step, landing at raw + 32 r + 16 (i%2)
    // = raw + 1024 (NC w + q) + 16 i;  scales: lane i < SL -> row SL w + i, its 4
    // scale bytes per step at raw + 8 KB + 4 r = raw + 8 KB + 4 SL w + 4 i.
    auto weight_row = [&](int r) {
        if (KIND == 1) return (r < 128 ? 0 : F - 128) + nt * 128 + r;
        return min(nt * kPN + r, d - 1);                 // columns past d: any valid row
    };
    const uint8_t* wcodes = KIND == 1 ? W.w13 + ex * (size_t)(2 * F) * (d / 2) : W.w2 + ex * (size_t)d * (F / 2);
    const uint8_t* wscales = KIND == 1 ? W.w13_s + ex * (size_t)(2 * F) * (d / 16) : W.w2_s + ex * (size_t)d * (F / 16);
    const uint8_t* csrc[NC];
#pragma unroll
    for (int q = 0; q < NC; ++q)
        csrc[q] = wcodes + (size_t)weight_row((wave * NC + q) * 32 + (lane >> 1)) * (K / 2) + (lane & 1) * 16;
    const uint8_t* ssrc = wscales + (size_t)weight_row(wave * SL + (lane & (SL - 1))) * (K / 16);
    const float gscale = KIND == 1 ? W.g13[ex] : W.g2[ex];

    // valid 32-row blocks of this wave (rows past re are padding)
    const int nvi = max(0, min(4, (re - rb - wm * 128 + 31) >> 5));
    const bool colv = KIND == 1 || nt * kPN + wn * (32 * NJ) < d;
    const int nk = K / kPK;

    // Every wave issues exactly NLOAD direct loads per step, in this order: NA
    // A loads, then NC raw code loads and one raw scale load (lanes < SL).
    auto issue_raw = [&](int ks_r, int rslot) {
        uint8_t* rbase = smem + kPOffR + rslot * kPRaw;
#pragma unroll
        for (int q = 0; q < NC; ++q)
            __builtin_amdgcn_global_load_lds((const void*)(csrc[q] + ks_r * (kPK / 2)),
                                             (lds_void_t*)(rbase + (wave * NC + q) * 1024), 16, 0, 0);
        if (SL == 64 || lane < SL)
            __builtin_amdgcn_global_load_lds((const void*)(ssrc + ks_r * (kPK / 16)),
                                             (lds_void_t*)(rbase + kPRawC + wave * SL * 4), 4, 0, 0);
    };
    auto issue = [&](int ks_a, int aslot, int ks_r, int rslot) {
        uint8_t* abase = smem + aslot * kPA + wave * NA * 1024;
#pragma unroll
        for (int q = 0; q < NA; ++q)
            __builtin_amdgcn_global_load_lds((const void*)(asrc[q] + ks_a * kPK), (lds_void_t*)(abase + q * 1024),
                                             16, 0, 0);
        asm volatile("" ::: "memory");               // keep the A loads ahead of the raw loads
        issue_raw(ks_r, rslot);
    };

    // decode: thread -> B row bj = tid % 256, chunks CB .. CB + NQ of the row's 8
    // (8 waves: two threads per row, a K half each; 4 waves: one thread per row);
    // 16 lanes of a wave write 16 consecutive rows' same chunk: conflict-free
    constexpr int NQ = WAVES == 8 ? 4 : 8;
    const int bj = tid & 255, cb = (tid >> 8) * NQ;
    struct Raw { u32x4_t c[NQ / 4]; uint32_t s; };
    auto read_raw = [&](int rslot) {
        const uint8_t* rb0 = smem + kPOffR + rslot * kPRaw;
        Raw r;
#pragma unroll
        for (int h = 0; h < NQ / 4; ++h) r.c[h] = *reinterpret_cast<const u32x4_t*>(rb0 + bj * 32 + cb * 4 + h * 16);
        r.s = *reinterpret_cast<const uint32_t*>(rb0 + kPRawC + bj * 4);
        return r;
    };
    // chunk q (0..NQ) of this thread: 8 elements, scale byte (cb + q) / 2
    auto store_b8 = [&](const Raw& r, int q, int bslot) {
        uint8_t* base = smem + kPOffB + bslot * kPB;
        const int c = cb + q;
        const float s = e4m3_to_f32((r.s >> ((c >> 1) * 8)) & 0xFFu);
        const uint32_t codes = r.c[q >> 2][q & 3];
        *reinterpret_cast<u32x4_t*>(base + swz(bj, c)) = dequant8_bf16(codes, s);
    };

    f32x16_t acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // LDS rows of this lane's operands: A rows wm*128 + 32 i; B blocks j < NJ
    // (GEMM1: gate (NJ/2) 32 wn + 32 j for j < NJ/2, the matching up rows 128
    // further; GEMM2: 32 NJ wn + 32 j)
    const int arow0 = wm * 128 + (lane & 31);
    int brow[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        brow[j] = (KIND == 1 ? (j < NJ / 2 ? wn * 16 * NJ + j * 32 : 128 + wn * 16 * NJ + (j - NJ / 2) * 32)
                             : wn * 32 * NJ + j * 32) +
                  (lane & 31);
    const int khalf = lane >> 5;

    // Pipeline, step ks (A slot ks % 2, B slot ks % 2, raw slot ks % 3):
    //   issue A(ks+1) and the raw weights of step ks+3 (three raw slots);
    //   decode the raw weights of step ks+1 into the other B slot, between the
    //   MFMAs of step ks;
    //   end: wait until only this step's NRAW raw loads may be outstanding, so
    //   A(ks+1) and raw(ks+2) have landed; LDS writes done; workgroup barrier.
    // Nothing in the loop loads into registers from global memory, so every wait
    // on the direct loads is this explicit one.  Past the end the loads are
    // clamped to the last step (re-loads of valid data into free slots).
    auto kloop = [&](auto nv_c) {
        constexpr int NV = decltype(nv_c)::value;
        int r0 = 0;                                      // raw slot of step ks
        for (int ks = 0; ks < nk; ++ks) {
            const int cur = ks & 1;
            const int r1 = r0 == 2 ? 0 : r0 + 1;          // raw slot of ks + 1 (and of ks + 4)
            issue(min(ks + 1, nk - 1), cur ^ 1, min(ks + 3, nk - 1), r0);
            const Raw raw = read_raw(r1);
            const uint8_t* As = smem + cur * kPA;
            const uint8_t* Bs = smem + kPOffB + cur * kPB;
            bf16x8_t av[2][4], bv[2][NJ];
            auto frag = [&](int kk, int f) {
                const int c = kk * 2 + khalf;
#pragma unroll
                for (int j = 0; j < NJ; ++j) bv[f][j] = *reinterpret_cast<const bf16x8_t*>(Bs + swz(brow[j], c));
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    av[f][i] = *reinterpret_cast<const bf16x8_t*>(As + swz(arow0 + i * 32, c));
            };
            if (NV > 0) frag(0, 0);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (NV > 0) {
                    if (kk < 3) frag(kk + 1, (kk + 1) & 1);
#pragma unroll
                    for (int i = 0; i < NV; ++i)
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kk & 1][i], bv[kk & 1][j],
                                                                                acc[i][j], 0, 0, 0);
                }
#pragma unroll
                for (int q = kk * NQ / 4; q < (kk + 1) * NQ / 4; ++q) store_b8(raw, q, cur ^ 1);
            }
            // Written out because __syncthreads() would also wait for every
            // outstanding load (vmcnt(0)) and drain the pipeline; the memory
            // clobber keeps the compiler from moving LDS accesses across it.
            if (NRAW == 2) asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            r0 = r1;
        }
    };

    // prologue: A(0); raw of steps 0, 1, 2; decode step 0
    {
        uint8_t* abase = smem + wave * NA * 1024;
#pragma unroll
        for (int q = 0; q < NA; ++q)
            __builtin_amdgcn_global_load_lds((const void*)asrc[q], (lds_void_t*)(abase + q * 1024), 16, 0, 0);
        for (int st = 0; st < 3; ++st) issue_raw(min(st, nk - 1), st);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const Raw raw = read_raw(0);
#pragma unroll
        for (int q = 0; q < NQ; ++q) store_b8(raw, q, 0);
        __syncthreads();
    }
    switch (colv ? nvi : 0) {
        case 4: kloop(std::integral_constant<int, 4>{}); break;
        case 3: kloop(std::integral_constant<int, 3>{}); break;
        case 2: kloop(std::integral_constant<int, 2>{}); break;
        case 1: kloop(std::integral_constant<int, 1>{}); break;
        default: kloop(std::integral_constant<int, 0>{}); break;
    }
    __builtin_amdgcn_s_waitcnt(0);

    // ---- epilogue ----
    if (KIND == 1) {
        // SwiGLU in registers, then through LDS (fp32 [256][136]: the 4-row offset
        // of the two half-waves is half a bank period) so that each thread owns
        // whole 16-column blocks of a row: the W4A4 block scale is computed once
        // per block, and the bf16 row pieces leave in 16-byte stores.
        constexpr int ES = 136;                           // row stride (floats)
        float* E = reinterpret_cast<float*>(smem);
        __syncthreads();                                  // every wave's direct loads have landed
        const int lr = (lane >> 5) * 4;
        if (colv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i >= nvi) break;
#pragma unroll
                for (int j = 0; j < NJ / 2; ++j) {
                    const int col = wn * 16 * NJ + j * 32 + (lane & 31);
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int row = wm * 128 + i * 32 + (v >> 2) * 8 + lr + (v & 3);
                        E[row * ES + col] = silu_fast(acc[i][j][v] * gscale) * (acc[i][j + NJ / 2][v] * gscale);
                    }
                }
            }
        }
        __syncthreads();
        const int nrow = re - rb;
        for (int blk = tid; blk < kPM * 8; blk += 64 * WAVES) {
            const int row = blk >> 3, cb = (blk & 7) * 16;
            if (row >= nrow) break;                       // rows grow with blk
            float x[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(E + row * ES + cb + q * 4);
                x[4 * q] = v4[0]; x[4 * q + 1] = v4[1]; x[4 * q + 2] = v4[2]; x[4 * q + 3] = v4[3];
            }
            if (MODE == 1) {
                float m = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(x[e]));
                const float sc = e4m3_to_f32(e4m3_encode_nonneg(__fdiv_rn(m, 6.0f)));
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    x[e] = sc > 0.0f ? e2m1_value(e2m1_encode(__fdiv_rn(x[e], sc))) * sc : 0.0f;
            }
            u32x4_t o0, o1;
            o0.x = f32_to_bf16_rne(x[0]) | (f32_to_bf16_rne(x[1]) << 16);
            o0.y = f32_to_bf16_rne(x[2]) | (f32_to_bf16_rne(x[3]) << 16);
            o0.z = f32_to_bf16_rne(x[4]) | (f32_to_bf16_rne(x[5]) << 16);
            o0.w = f32_to_bf16_rne(x[6]) | (f32_to_bf16_rne(x[7]) << 16);
            o1.x = f32_to_bf16_rne(x[8]) | (f32_to_bf16_rne(x[9]) << 16);
            o1.y = f32_to_bf16_rne(x[10]) | (f32_to_bf16_rne(x[11]) << 16);
            o1.z = f32_to_bf16_rne(x[12]) | (f32_to_bf16_rne(x[13]) << 16);
            o1.w = f32_to_bf16_rne(x[14]) | (f32_to_bf16_rne(x[15]) << 16);
            uint16_t* dst = a.act + (size_t)(rb + row) * F + nt * 128 + cb;
            *reinterpret_cast<u32x4_t*>(dst) = o0;
            *reinterpret_cast<u32x4_t*>(dst + 8) = o1;
        }
        return;
    }
    // GEMM2: Y = g2 * acc in bf16, through LDS (bf16 [256][264]: the two
    // half-waves' rows land half a bank period apart) so that each thread
    // writes whole 16-byte pieces of rows
    constexpr int YS = 264;                               // row stride (bf16 elements)
    uint16_t* Ys = reinterpret_cast<uint16_t*>(smem);
    __syncthreads();                                      // every wave's direct loads have landed
    const int lr = (lane >> 5) * 4;
    if (colv) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i >= nvi) break;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int col = wn * 32 * NJ + j * 32 + (lane & 31);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = wm * 128 + i * 32 + (v >> 2) * 8 + lr + (v & 3);
                    Ys[row * YS + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][v] * gscale);
                }
            }
        }
    }
    __syncthreads();
    const int nrow = re - rb, ncol = min(kPN, d - nt * kPN);
    for (int pc = tid; pc < kPM * (kPN / 8); pc += 64 * WAVES) {
        const int row = pc >> 5, c8 = (pc & 31) * 8;
        if (row >= nrow) break;                           // rows grow with pc
        if (c8 < ncol)
            *reinterpret_cast<u32x4_t*>(a.Y + (size_t)(rb + row) * d + nt * kPN + c8) =
                *reinterpret_cast<const u32x4_t*>(Ys + row * YS + c8);
    }
}

constexpr int kPWaves = 8;

template <int KIND, int MODE>
static hipError_t launch_pf(const GemmArgs& a, hipStream_t s) {
    static bool attr_set = false;   // per process; the attribute is per function
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)pf_gemm_kernel<KIND, MODE, kPWaves>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kPLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int NT = KIND == 1 ? (2 * a.F) / kPN : (a.d + kPN - 1) / kPN;
    const long long n = (long long)a.max_tiles * NT;
    const long long grid = (n + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((pf_gemm_kernel<KIND, MODE, kPWaves>), dim3((unsigned)grid), dim3(64 * kPWaves), kPLds, s, a);
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
