// Tiled expert GEMMs for many tokens per expert (prefill), gfx950.
//
// A tile is 256 pair rows of one expert group (a local expert, or the shared
// expert over all tokens) x 256 weight rows, K advanced 64 at a time.  Eight
// waves as 2 (rows) x 4 (weight rows); a wave owns 128 x 64 of the tile as
// 4 x 2 blocks of 32x32x16 MFMAs with fp32 accumulation.  Two kernels:
//
// pf_gemm_kernel (16-bit activations).  LDS (150 KB of the CU's 160 KB):
//   A ring, 3 slots of [256 rows][64] 16-bit activations, two steps ahead,
//     copied straight from global memory (global_load_lds_dwordx4, no
//     registers), gathered through the permutation for GEMM1; the eight
//     16-byte chunks of a row are XOR-swizzled by the row so that a 32-row
//     operand read is conflict-free;
//   raw ring, 3 slots of the 256 weight rows' NVFP4 codes (64 bytes a row) and
//     E4M3 block scales (8 bytes a row) for two steps, copied the same way.
// Every wave decodes its own weight operand from the raw ring into registers:
// code * block scale is exact in 16 bits (at most 6 significant bits).  The
// weight tile is never written back to LDS, so the LDS carries only the A
// operand reads and the two rings' fills.
//
// pf4_gemm_kernel (W4A4 with NVFP4 activations; see its own comment): both
// operands arrive raw, 256 k per chunk, and both are decoded per wave.
//
// K order inside a step: the MFMA sums over its 16 k in any order as long as
// both operands use the same one.  Lane half h of MFMA kk (0..3) takes the
// step's k = 32h + 8kk .. +8, so one 16-byte read of a weight row's raw codes
// (k = 32h .. 32h + 32) gives a lane its codes for all four MFMAs, and the A
// operand is chunk 4h + kk of the row.
//
// Operand type: W4A16 multiplies bf16 activations by bf16-decoded weights.  In
// W4A4 both operands are NVFP4 products (code * E4M3 scale), exact in f16 as in
// bf16, so the activations arrive as f16 and the weights decode with packed f16
// multiplies (v_mfma_f32_32x32x16_f16); the arithmetic is the same.
//
// Lane layout of v_mfma_f32_32x32x16_{bf16,f16} (checked on the device): lane
// l holds A[l%32][8(l/32)..+8] and B[8(l/32)..+8][l%32]; accumulator value v
// sits at row 8(v/4) + 4(l/32) + v%4, column l%32.
//
// GEMM1 (KIND 1): the 256 weight rows are 128 gate rows [n, n+128) and the
// matching up rows [F+n, F+n+128); a wave's two column blocks are gate columns
// and the same up columns, so the SwiGLU a = silu(g13*gate) * (g13*up) is formed
// in registers; W4A4 quantize-dequantizes a per 16 columns.  Stored bf16
// (W4A16) or f16 (W4A4, exact).
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
constexpr int kPWaves = 8;
constexpr int kPA = kPM * kPK * 2;             // bytes of one A stage (32 KB)
constexpr int kPASlots = 3;
constexpr int kPRawC = kPN * 64;               // raw codes of a two-step chunk (16 KB: 64 B per weight row)
constexpr int kPRaw = kPRawC + kPN * 8;        // + raw scales (2 KB: 8 B per weight row)
constexpr int kPRSlots = 3;
constexpr int kPOffR = kPASlots * kPA;         // LDS map: A[3] | raw[3]
constexpr int kPLds = kPOffR + kPRSlots * kPRaw;   // 150 KB

typedef __attribute__((address_space(3))) void lds_void_t;

// silu(z) = z / (1 + e^-z) with the hardware exponential and reciprocal (each
// within ~1 ulp) in place of a correctly rounded division; z -> -inf gives -0.
__device__ __forceinline__ float silu_fast(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Byte offset of 16-byte chunk c of row r in a swizzled [rows][64 x 16-bit]
// tile.  Any 8 consecutive rows (aligned) put a given chunk in 8 different
// 16-byte slots, and rows r, r + 8 differ again in the slot's low bit, so a
// 32-row operand read is free of bank conflicts whether the LDS serves 8 or 16
// lanes of a 16-byte access per cycle.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 4); }

// 16-byte unit u of a 64-byte raw code row r (two 64-k steps): 32 lanes reading
// one unit of 32 consecutive rows, or 8 / 16 consecutive rows' same unit, hit
// distinct bank groups whether the LDS serves 8 or 16 lanes of a 16-byte access
// per cycle.
__device__ __forceinline__ int cwz(int r, int u) { return r * 64 + ((u ^ (((r >> 1) ^ (r >> 3)) & 3)) << 4); }

template <int MODE>
__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
    if constexpr (MODE == 1)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int KIND, int MODE>
__global__ __launch_bounds__(64 * kPWaves) void pf_gemm_kernel(GemmArgs a) {
    constexpr int WN = kPWaves / 2;                // waves along the weight rows
    constexpr int NJ = kPN / WN / 32;              // 32-column blocks per wave (2)
    constexpr int NA = 32 / kPWaves;               // A loads (1 KB) per wave per step (4)
    static_assert(NJ == 2 && NA == 4, "tile shape");
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

    // ---- raw weight sources: two 64-k steps per chunk ----
    // codes: load q (0, 1) of wave w fills rows 16 (2w + q) .. +16 of the chunk's
    // [256][64 B] code tile (1 KB, lane i at byte 16 i): lane i -> row r =
    // 16 (2w + q) + i/4, 16-byte slot i%4 of the row, which holds unit
    // (i%4) ^ g(r) (cwz).  scales: lane i -> row 32 w + i/2, dword i%2 (the
    // chunk's two steps) at raw + 16 KB + 8 r + 4 (i%2) = raw + 16 KB + 256 w + 4 i.
    auto weight_row = [&](int r) {
        if (KIND == 1) return (r < 128 ? 0 : F - 128) + nt * 128 + r;
        return min(nt * kPN + r, d - 1);                 // columns past d: any valid row
    };
    const uint8_t* wcodes = KIND == 1 ? W.w13 + ex * (size_t)(2 * F) * (d / 2) : W.w2 + ex * (size_t)d * (F / 2);
    const uint8_t* wscales = KIND == 1 ? W.w13_s + ex * (size_t)(2 * F) * (d / 16) : W.w2_s + ex * (size_t)d * (F / 16);
    const uint8_t* csrc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = (wave * 2 + q) * 16 + (lane >> 2);
        csrc[q] = wcodes + (size_t)weight_row(r) * (K / 2) + (((lane & 3) ^ (((r >> 1) ^ (r >> 3)) & 3)) << 4);
    }
    const uint8_t* ssrc = wscales + (size_t)weight_row(wave * 32 + (lane >> 1)) * (K / 16) + (lane & 1) * 4;
    const float gscale = KIND == 1 ? W.g13[ex] * a.a1g : W.g2[ex] * a.a2g;   // weight x activation globals

    // valid 32-row blocks of this wave (rows past re are padding)
    const int nvi = max(0, min(4, (re - rb - wm * 128 + 31) >> 5));
    const bool colv = KIND == 1 || nt * kPN + wn * (32 * NJ) < d;
    const int nk = K / kPK, nc = nk / 2;             // K % 128 == 0: whole chunks

    // Direct loads per wave: NA A loads per step; at even steps also the next
    // chunk's two code loads and one scale load.
    auto issue_raw = [&](int c, int slot) {
        uint8_t* rbase = smem + kPOffR + slot * kPRaw;
#pragma unroll
        for (int q = 0; q < 2; ++q)
            __builtin_amdgcn_global_load_lds((const void*)(csrc[q] + c * 64),
                                             (lds_void_t*)(rbase + (wave * 2 + q) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(ssrc + c * 8), (lds_void_t*)(rbase + kPRawC + wave * 256), 4,
                                         0, 0);
    };
    auto issue_a = [&](int ks, int slot) {
        uint8_t* abase = smem + slot * kPA + wave * NA * 1024;
#pragma unroll
        for (int q = 0; q < NA; ++q)
            __builtin_amdgcn_global_load_lds((const void*)(asrc[q] + ks * kPK), (lds_void_t*)(abase + q * 1024), 16,
                                             0, 0);
    };

    f32x16_t acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // operand rows of this lane: A rows wm*128 + 32 i + l%32; weight rows (tile
    // local) GEMM1: gate 32 wn + l%32 and up 128 + 32 wn + l%32; GEMM2: 64 wn +
    // 32 j + l%32
    const int arow0 = wm * 128 + (lane & 31);
    const int h = lane >> 5;
    int brow[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) brow[j] = (KIND == 1 ? j * 128 + wn * 32 : wn * 64 + j * 32) + (lane & 31);

    // Pipeline, step ks (A slot ks % 3; chunk ks/2 in raw slot (ks/2) % 3):
    //   issue A(ks+2) and, at even steps, chunk ks/2 + 1, into slots freed by
    //   the last barrier (past the end both are clamped: re-loads of valid data
    //   into free slots, so every step issues the same loads);
    //   read this step's raw codes (unit 2 (ks%2) + h of the row) and scales,
    //   decode each MFMA's weight operand in registers just before it, A
    //   operands double-buffered in registers;
    //   end: wait until only this step's own loads may be in flight (so A(ks+1)
    //   and the chunk of step ks+1 have landed); LDS reads done; barrier.
    // Nothing in the loop loads into registers from global memory, so every wait
    // on the direct loads is this explicit one.
    auto step = [&](auto nv_c, auto st_c, int ks, int as, int rs) {
        constexpr int NV = decltype(nv_c)::value;
        constexpr int ST = decltype(st_c)::value;      // ks % 2
        issue_a(min(ks + 2, nk - 1), as == 0 ? 2 : as - 1);
        if (ST == 0) issue_raw(min(ks / 2 + 1, nc - 1), rs == 2 ? 0 : rs + 1);
        if (NV > 0) {
            const uint8_t* As = smem + as * kPA;
            const uint8_t* Rs = smem + kPOffR + rs * kPRaw;
            u32x4_t rc[NJ];
            uint32_t sc[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                rc[j] = *reinterpret_cast<const u32x4_t*>(Rs + cwz(brow[j], 2 * ST + h));
                sc[j] = *reinterpret_cast<const uint32_t*>(Rs + kPRawC + brow[j] * 8 + ST * 4) >> (16 * h);
            }
            u32x4_t av[2][4];
            auto frag = [&](int kk, int f) {
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    av[f][i] = *reinterpret_cast<const u32x4_t*>(As + swz(arow0 + i * 32, 4 * h + kk));
            };
            frag(0, 0);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk < 3) frag(kk + 1, (kk + 1) & 1);
                u32x4_t bv[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if constexpr (MODE == 1) {
                        const f16x2_t sp = e4m3x2_to_f16(sc[j]);
                        const _Float16 s = kk < 2 ? sp.x : sp.y;
                        bv[j] = dequant8_f16(rc[j][kk], f16x2_t{s, s});
                    } else {
                        bv[j] = dequant8_bf16(rc[j][kk], e4m3_to_f32((sc[j] >> (8 * (kk >> 1))) & 0xFFu));
                    }
                }
#pragma unroll
                for (int i = 0; i < NV; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32<MODE>(av[kk & 1][i], bv[j], acc[i][j]);
            }
        }
        // Written out because __syncthreads() would also wait for every
        // outstanding load (vmcnt(0)) and drain the pipeline; the memory
        // clobber keeps the compiler from moving LDS accesses across it.
        if (ST == 0) asm volatile("s_waitcnt vmcnt(7) lgkmcnt(0)\n\ts_barrier" ::: "memory");   // NA + 3
        else asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");           // NA
    };
    auto kloop = [&](auto nv_c) {
        int as = 0, rs = 0;                                // A slot of step ks, raw slot of its chunk
        for (int ks = 0; ks < nk; ks += 2) {
            step(nv_c, std::integral_constant<int, 0>{}, ks, as, rs);
            as = as == 2 ? 0 : as + 1;
            step(nv_c, std::integral_constant<int, 1>{}, ks + 1, as, rs);
            as = as == 2 ? 0 : as + 1;
            rs = rs == 2 ? 0 : rs + 1;
        }
    };

    // prologue: A(0), A(1), chunk 0; all landed before the loop
    issue_a(0, 0);
    issue_a(1, 1);
    issue_raw(0, 0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
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
        // per block, and the 16-bit row pieces leave in 16-byte stores.
        constexpr int ES = 136;                           // row stride (floats)
        float* E = reinterpret_cast<float*>(smem);
        __syncthreads();                                  // every wave's direct loads have landed
        const int lr = (lane >> 5) * 4;
        if (colv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i >= nvi) break;
                const int col = wn * 32 + (lane & 31);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = wm * 128 + i * 32 + (v >> 2) * 8 + lr + (v & 3);
                    E[row * ES + col] = silu_fast(acc[i][0][v] * gscale) * (acc[i][1][v] * gscale);
                }
            }
        }
        __syncthreads();
        const int nrow = re - rb;
        for (int blk = tid; blk < kPM * 8; blk += 64 * kPWaves) {
            const int row = blk >> 3, cb = (blk & 7) * 16;
            if (row >= nrow) break;                       // rows grow with blk
            float x[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(E + row * ES + cb + q * 4);
                x[4 * q] = v4[0]; x[4 * q + 1] = v4[1]; x[4 * q + 2] = v4[2]; x[4 * q + 3] = v4[3];
            }
            uint32_t o[8];
            if (MODE == 1) {
                float m = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(x[e]));
                const float sc = e4m3_to_f32(nvfp4_act_scale(m, a.a2g));
#pragma unroll
                for (int e = 0; e < 16; ++e) x[e] = e2m1_value(nvfp4_act_code(x[e], sc, a.a2g)) * sc;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = f32_to_f16_bits(x[2 * e]) | (f32_to_f16_bits(x[2 * e + 1]) << 16);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = f32x2_to_bf16x2(x[2 * e], x[2 * e + 1]);
            }
            uint16_t* dst = a.act + (size_t)(rb + row) * F + nt * 128 + cb;
            *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{o[0], o[1], o[2], o[3]};
            *reinterpret_cast<u32x4_t*>(dst + 8) = u32x4_t{o[4], o[5], o[6], o[7]};
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
    for (int pc = tid; pc < kPM * (kPN / 8); pc += 64 * kPWaves) {
        const int row = pc >> 5, c8 = (pc & 31) * 8;
        if (row >= nrow) break;                           // rows grow with pc
        if (c8 < ncol)
            *reinterpret_cast<u32x4_t*>(a.Y + (size_t)(rb + row) * d + nt * kPN + c8) =
                *reinterpret_cast<const u32x4_t*>(Ys + row * YS + c8);
    }
}

// ---------------------------------------------------------------------------
// W4A4 with the activations as NVFP4 (codes + E4M3 block scales), for d and F
// multiples of 256.  The same tile, waves and K order as above, but K is staged
// 256 at a time (a chunk of four 64-k steps) and BOTH operands arrive raw:
// per chunk and operand, 256 rows x 128 code bytes (one full 128-byte line a
// row) and 256 rows x 16 scale bytes, 72 KB a slot, two slots.  Every wave
// decodes its A and B operands in registers (code * scale, exact in f16).
// Compared with 16-bit activations this moves 3.5x fewer activation bytes and
// touches 4x fewer cache lines per step, and the LDS carries no decoded tile.
// ---------------------------------------------------------------------------
constexpr int kQK = 256;                             // K per chunk
constexpr int kQCodes = kPM * (kQK / 2);             // 32 KB of codes per operand and chunk
constexpr int kQScales = kPM * (kQK / 16);           // 4 KB of scales per operand and chunk
constexpr int kQSlot = 2 * kQCodes + 2 * kQScales;   // A codes | B codes | A scales | B scales
constexpr int kQLds = 2 * kQSlot;                    // 144 KB

bool pf_packed_ok(int d, int F) { return d % kQK == 0 && F % kQK == 0; }

template <int KIND, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void pf4_gemm_kernel(GemmArgs a) {
    constexpr int WN = 4;                          // waves along the weight rows
    constexpr int WM = WAVES / WN;                 // waves along the tile rows (2 or 4)
    constexpr int NVM = kPM / (32 * WM);           // 32-row blocks per wave (4 or 2)
    constexpr int NJ = kPN / WN / 32;              // 32-column blocks per wave
    constexpr int NQ = 32 / WAVES;                 // code loads per operand, wave and chunk
    constexpr int SR = 256 / WAVES;                // scale rows per wave (lanes)
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int d = a.d, F = a.F;
    const int NT = KIND == 1 ? (2 * F) / kPN : d / kPN;
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

    // activation row of tile row r (padding rows read the tile's first row)
    auto arow = [&](int r) {
        int gr = rb + r;
        if (gr >= re) gr = rb;
        if (KIND == 2) return gr;
        return shared ? gr - a.T * a.topk : a.perm[gr] / a.topk;
    };
    auto weight_row = [&](int r) {
        if (KIND == 1) return (r < 128 ? 0 : F - 128) + nt * 128 + r;
        return nt * kPN + r;
    };
    const uint8_t* acodes = KIND == 1 ? a.hq_codes : a.act_codes;
    const uint8_t* ascales = KIND == 1 ? a.hq_scales : a.act_scales;
    const uint8_t* wcodes = KIND == 1 ? W.w13 + ex * (size_t)(2 * F) * (d / 2) : W.w2 + ex * (size_t)d * (F / 2);
    const uint8_t* wscales = KIND == 1 ? W.w13_s + ex * (size_t)(2 * F) * (d / 16) : W.w2_s + ex * (size_t)d * (F / 16);

    // code loads: load q (0..3) of wave w fills rows 8 (4w + q) .. +8 of an
    // operand's [256][128 B] chunk tile (1 KB, lane i at byte 16 i): lane i ->
    // row r = 8 (4w + q) + i/8, 16-byte slot i%8, which holds unit
    // (i & 7) ^ (i >> 3) ^ (q & 1) of the row's chunk (the swz layout)
    const uint8_t* acs[NQ];
    const uint8_t* bcs[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int r = (wave * NQ + q) * 8 + (lane >> 3);
        const int u = (lane & 7) ^ (lane >> 3) ^ (q & 1);
        acs[q] = acodes + (size_t)arow(r) * (K / 2) + u * 16;
        bcs[q] = wcodes + (size_t)weight_row(r) * (K / 2) + u * 16;
    }
    // scale loads (lanes < SR): row SR w + i, its 16 scale bytes of the chunk at
    // 16 (SR w + i)
    const int sr = wave * SR + (lane & (SR - 1));
    const uint8_t* ass = ascales + (size_t)arow(sr) * (K / 16);
    const uint8_t* bss = wscales + (size_t)weight_row(sr) * (K / 16);
    const float gscale = KIND == 1 ? W.g13[ex] * a.a1g : W.g2[ex] * a.a2g;   // weight x activation globals

    const int nvi = max(0, min(NVM, (re - rb - wm * (32 * NVM) + 31) >> 5));
    const int nc = K / kQK;

    auto issue = [&](int c, int slot) {
        uint8_t* base = smem + slot * kQSlot;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            __builtin_amdgcn_global_load_lds((const void*)(acs[q] + c * (kQK / 2)),
                                             (lds_void_t*)(base + (wave * NQ + q) * 1024), 16, 0, 0);
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            __builtin_amdgcn_global_load_lds((const void*)(bcs[q] + c * (kQK / 2)),
                                             (lds_void_t*)(base + kQCodes + (wave * NQ + q) * 1024), 16, 0, 0);
        if (SR == 64 || lane < SR) {
            __builtin_amdgcn_global_load_lds((const void*)(ass + c * (kQK / 16)),
                                             (lds_void_t*)(base + 2 * kQCodes + wave * SR * 16), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(bss + c * (kQK / 16)),
                                             (lds_void_t*)(base + 2 * kQCodes + kQScales + wave * SR * 16), 16, 0,
                                             0);
        }
    };

    f32x16_t acc[NVM][NJ];
#pragma unroll
    for (int i = 0; i < NVM; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int h = lane >> 5;
    int brow[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        brow[j] = (KIND == 1 ? (j < NJ / 2 ? wn * 16 * NJ + j * 32 : 128 + wn * 16 * NJ + (j - NJ / 2) * 32)
                             : wn * 32 * NJ + j * 32) +
                  (lane & 31);
    const int arow0 = wm * (32 * NVM) + (lane & 31);

    // one step (64 k) of a chunk: lane half h of MFMA kk takes k = 32h + 8kk ..
    // +8 of the step: dword kk of the row's 16-byte code unit 2s + h, scale byte
    // 2h + kk/2 of the step's 4
    auto step = [&](auto nv_c, const uint8_t* S, int s) {
        constexpr int NV = decltype(nv_c)::value;
        u32x4_t ac[NVM], bc[NJ];
        uint32_t as[NVM], bs[NJ];
        static_assert(NJ <= 4, "operand blocks");
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int r = arow0 + i * 32;
            ac[i] = *reinterpret_cast<const u32x4_t*>(S + swz(r, 2 * s + h));
            as[i] = *reinterpret_cast<const uint32_t*>(S + 2 * kQCodes + r * 16 + s * 4) >> (16 * h);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            bc[j] = *reinterpret_cast<const u32x4_t*>(S + kQCodes + swz(brow[j], 2 * s + h));
            bs[j] = *reinterpret_cast<const uint32_t*>(S + 2 * kQCodes + kQScales + brow[j] * 16 + s * 4) >> (16 * h);
        }
        // the lane half's two block scales of the step, as f16 {MFMAs 0-1, 2-3}
        f16x2_t asc[NVM], bsc[NJ];
#pragma unroll
        for (int i = 0; i < NV; ++i) asc[i] = e4m3x2_to_f16(as[i]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) bsc[j] = e4m3x2_to_f16(bs[j]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4_t av[NVM], bv[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const _Float16 sc = kk < 2 ? bsc[j].x : bsc[j].y;
                bv[j] = dequant8_f16(bc[j][kk], f16x2_t{sc, sc});
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const _Float16 sc = kk < 2 ? asc[i].x : asc[i].y;
                av[i] = dequant8_f16(ac[i][kk], f16x2_t{sc, sc});
            }
#pragma unroll
            for (int i = 0; i < NV; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32<1>(av[i], bv[j], acc[i][j]);
        }
    };

    // Pipeline: chunk c+1 is loaded into the other slot while chunk c is
    // multiplied; at the end of a chunk every wave waits for its own loads and
    // the workgroup meets at a barrier (no LDS reads of slot c remain, chunk c+1
    // has landed).  Nothing loads into registers from global memory in the loop.
    auto kloop = [&](auto nv_c) {
        for (int c = 0; c < nc; ++c) {
            if (c + 1 < nc) issue(c + 1, (c + 1) & 1);
            const uint8_t* S = smem + (c & 1) * kQSlot;
            if (decltype(nv_c)::value > 0) {
#pragma unroll
                for (int s = 0; s < 4; ++s) step(nv_c, S, s);
            }
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
    };
    issue(0, 0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    switch (nvi) {
        case 4: if constexpr (NVM >= 4) kloop(std::integral_constant<int, 4>{}); break;
        case 3: if constexpr (NVM >= 3) kloop(std::integral_constant<int, 3>{}); break;
        case 2: kloop(std::integral_constant<int, 2>{}); break;
        case 1: kloop(std::integral_constant<int, 1>{}); break;
        default: kloop(std::integral_constant<int, 0>{}); break;
    }

    const int lr = (lane >> 5) * 4;
    if (KIND == 1) {
        // SwiGLU, then NVFP4 per 16 columns: packed codes and E4M3 scales of
        // the act rows (the next GEMM's raw A)
        constexpr int ES = 136;
        float* E = reinterpret_cast<float*>(smem);
#pragma unroll
        for (int i = 0; i < NVM; ++i) {
            if (i >= nvi) break;
#pragma unroll
            for (int j = 0; j < NJ / 2; ++j) {
                const int col = wn * 16 * NJ + j * 32 + (lane & 31);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = wm * (32 * NVM) + i * 32 + (v >> 2) * 8 + lr + (v & 3);
                    E[row * ES + col] = silu_fast(acc[i][j][v] * gscale) * (acc[i][j + NJ / 2][v] * gscale);
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
            float m = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(x[e]));
            const uint32_t sbyte = nvfp4_act_scale(m, a.a2g);
            const float sc = e4m3_to_f32(sbyte);
            uint32_t lo = 0u, hi = 0u;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t cd = nvfp4_act_code(x[e], sc, a.a2g);
                if (e < 8) lo |= cd << (4 * e);
                else hi |= cd << (4 * (e - 8));
            }
            const size_t col = (size_t)nt * 128 + cb;
            *reinterpret_cast<u32x2_t*>(a.act_codes + (size_t)(rb + row) * (F / 2) + col / 2) = u32x2_t{lo, hi};
            a.act_scales[(size_t)(rb + row) * (F / 16) + col / 16] = (uint8_t)sbyte;
        }
        return;
    }
    constexpr int YS = 264;
    uint16_t* Ys = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int i = 0; i < NVM; ++i) {
        if (i >= nvi) break;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int col = wn * 32 * NJ + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * (32 * NVM) + i * 32 + (v >> 2) * 8 + lr + (v & 3);
                Ys[row * YS + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][v] * gscale);
            }
        }
    }
    __syncthreads();
    const int nrow = re - rb;
    for (int pc = tid; pc < kPM * (kPN / 8); pc += 64 * WAVES) {
        const int row = pc >> 5, c8 = (pc & 31) * 8;
        if (row >= nrow) break;
        *reinterpret_cast<u32x4_t*>(a.Y + (size_t)(rb + row) * d + nt * kPN + c8) =
            *reinterpret_cast<const u32x4_t*>(Ys + row * YS + c8);
    }
}

// 8 waves (2 per SIMD, 128 x 64 wave tiles); the kernel also builds with 4
// (one per SIMD, 128 x 128 wave tiles), measured slower.
constexpr int kQWaves = 8;

template <int KIND>
static hipError_t launch_pf4(const GemmArgs& a, hipStream_t s) {
    const hipError_t e = allow_dynamic_lds<pf4_gemm_kernel<KIND, kQWaves>>(kQLds);
    if (e != hipSuccess) return e;
    const int NT = KIND == 1 ? (2 * a.F) / kPN : a.d / kPN;
    const long long n = (long long)a.max_tiles * NT;
    const long long grid = (n + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((pf4_gemm_kernel<KIND, kQWaves>), dim3((unsigned)grid), dim3(64 * kQWaves), kQLds, s, a);
    return hipGetLastError();
}

template <int KIND, int MODE>
static hipError_t launch_pf(const GemmArgs& a, hipStream_t s) {
    const hipError_t e = allow_dynamic_lds<pf_gemm_kernel<KIND, MODE>>(kPLds);
    if (e != hipSuccess) return e;
    const int NT = KIND == 1 ? (2 * a.F) / kPN : (a.d + kPN - 1) / kPN;
    const long long n = (long long)a.max_tiles * NT;
    const long long grid = (n + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((pf_gemm_kernel<KIND, MODE>), dim3((unsigned)grid), dim3(64 * kPWaves), kPLds, s, a);
    return hipGetLastError();
}

int pf_rows() { return kPM; }

// W4A4 (mode 1): activations and the SwiGLU output are f16 on this path.
hipError_t launch_gemm1(const GemmArgs& a, int /*path*/, hipStream_t s) {
    if (a.packed) return launch_pf4<1>(a, s);
    return a.mode == 0 ? launch_pf<1, 0>(a, s) : launch_pf<1, 1>(a, s);
}

hipError_t launch_gemm2(const GemmArgs& a, int /*path*/, hipStream_t s) {
    if (a.packed) return launch_pf4<2>(a, s);
    return a.mode == 0 ? launch_pf<2, 0>(a, s) : launch_pf<2, 1>(a, s);
}

}  // namespace moe
