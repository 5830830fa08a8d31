// Dense expert GEMMs over tiles of at most 32 token rows, gfx950: the weight
// stream staged through a deep LDS ring.
//
// Between a few and a few tens of pairs per expert the layer is bound by
// streaming every touched expert's NVFP4 weights from HBM once.  Under load the
// memory latency is several microseconds, so a compute unit needs well over
// 100 KB in flight to take its share of the bandwidth, more than registers can
// hold next to the arithmetic.  Here the weights (and the tile's activation
// rows) are copied straight into LDS with global_load_lds, up to kTDepth chunks
// of 128 k ahead (about 120 KB per compute unit), and every wave decodes its own
// weight rows from there with their E4M3 block scales into the B operand of a
// dense v_mfma_f32_32x32x16_{f16,bf16} (code * scale is exact in 16 bits: at
// most 6 significant bits); the A operand is the tile's 32 token rows.
//
// Workgroup: 8 waves over one tile (<= 32 rows of one expert group) and 256
// weight rows; wave w owns weight rows 32 w .. 32 w + 32 of the workgroup:
//   GEMM1: SwiGLU columns c0 = 128 cb + 16 w .. + 16, its rows being those
//          gate rows (MFMA columns 0..15) and the matching up rows F + c0 ..
//          (columns 16..31); silu(gate) * up pairs lanes l and l ^ 16;
//   GEMM2: output columns 256 cb + 32 w .. + 32.
// K order (the MFMA sums its 16 k in any order if both operands use the same
// one): in a chunk of 128 k, lane half h = l / 32 of MFMA kk (0..7) takes the
// chunk's k = 64 h + 8 kk .. + 8, so a lane's codes for the whole chunk are 32
// contiguous bytes of its row (two 16-byte LDS reads) and its block scales are
// 4 contiguous bytes (blocks 4 h .. 4 h + 3).
// Lane layout of v_mfma_f32_32x32x16 (checked on the device): lane l holds
// A[l%32][8 (l/32) ..] and B[8 (l/32) ..][l%32]; accumulator value v sits at
// row 8 (v/4) + 4 (l/32) + v%4, column l%32.  A rows are tokens, B columns
// weight rows.
//
// Activation operand AT: 0 bf16 (W4A16), 1 f16 (W4A4 quantize-dequantized,
// exact in f16), 2 NVFP4 codes and scales (W4A4, decoded per wave like the
// weights).
//
// Pipeline: kTSlots LDS slots hold chunks c .. c + kTDepth - 1 in flight.  At
// chunk c every wave waits for its own copies of chunk c (s_waitcnt vmcnt: the
// loop issues no other vector memory instruction), the workgroup meets at a
// barrier (so the slot of chunk c - 1 is free), the copies of chunk c + kTDepth
// are issued into that slot, and chunk c is multiplied.
//
// Layer semantics: the page "Serving Solar Open 2 on DGX Spark", sections "수정
// 사항 › b12x에서의 Expert Parallelism 구현 추가" (one shard's experts, partial sum)
// and "b12x 버전이 실제 NVFP4 체크포인트를 읽어들이도록 만들기" (packed FP4 codes,
// FP8 block scales, per-expert fp32 global scale, fused gate/up).
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kTM = 32;                  // tile rows
constexpr int kTN = 256;                 // weight rows per workgroup
constexpr int kTK = 128;                 // K per chunk
constexpr int kTWaves = 8;
constexpr int kTBC = kTN * 64;           // B codes of a chunk: [256 rows][64 B]
constexpr int kTBS = kTN * 8;            // B scales of a chunk: [256 rows][8 B]

template <int AT> __host__ __device__ constexpr int t32_abytes() { return AT == 2 ? kTM * 64 + kTM * 8 : kTM * kTK * 2; }
template <int AT> __host__ __device__ constexpr int t32_slot() { return kTBC + kTBS + t32_abytes<AT>(); }
// 7 x 20736 B (NVFP4 activations) or 6 x 26624 B (16-bit activations)
template <int AT> __host__ __device__ constexpr int t32_slots() { return AT == 2 ? 7 : 6; }
template <int AT> __host__ __device__ constexpr int t32_lds() { return t32_slots<AT>() * t32_slot<AT>(); }

typedef __attribute__((address_space(3))) void t32_lds_t;

// 16-byte unit u (0..3) of a 64-byte code row r: 16 consecutive rows' same
// unit (and 8 consecutive rows') fall in distinct bank groups whether the LDS
// serves 8 or 16 lanes of a 16-byte access per cycle.
__device__ __forceinline__ int t32_cu(int r, int u) { return r * 64 + ((u ^ (((r >> 1) ^ (r >> 3)) & 3)) << 4); }
// 16-byte unit u (0..15) of a 256-byte 16-bit activation row r: 16 consecutive
// rows' same unit are 16 distinct units.
__device__ __forceinline__ int t32_au(int r, int u) { return r * 256 + ((u ^ (r & 15)) << 4); }

template <int AT>
__device__ __forceinline__ f32x16_t t32_mfma(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
    if constexpr (AT == 0)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
}

template <int KIND, int AT>
__global__ __launch_bounds__(64 * kTWaves) void t32_gemm_kernel(GemmArgs a) {
    constexpr int SLOT = t32_slot<AT>(), NS = t32_slots<AT>(), DEPTH = NS - 1;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int d = a.d, F = a.F;
    const int ncb = KIND == 1 ? F / 128 : d / kTN;
    const long long lin = blockIdx.x + (long long)blockIdx.y * gridDim.x;
    const int tile = (int)(lin / ncb), cb = (int)(lin - (long long)tile * ncb);
    if (tile >= *a.ntiles) return;
    const int4 tt = a.tiles[tile];
    const int rb = tt.y, re = tt.z, ntok = re - rb;
    const bool shared = tt.x == a.L;
    const ExpertWeights& W = shared ? a.shared : a.local;
    const size_t ex = shared ? 0 : (size_t)tt.x;
    const int K = KIND == 1 ? d : F;
    const int nc = K / kTK;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // activation row of tile row r (padding rows read the tile's first row)
    auto arow = [&](int r) -> size_t {
        const int row = rb + (r < ntok ? r : 0);
        if (KIND == 2) return (size_t)row;
        return (size_t)(shared ? row - a.T * a.topk : a.perm[row] / a.topk);
    };
    // weight row of workgroup row r (0..255)
    auto wrow = [&](int r) -> size_t {
        if (KIND == 2) return (size_t)(cb * kTN + r);
        const int w = r >> 5, c = r & 31;
        return (size_t)((c < 16 ? 0 : F - 16) + cb * 128 + 16 * w + c);
    };
    const uint8_t* wcodes = KIND == 1 ? W.w13 + ex * (size_t)(2 * F) * (d / 2) : W.w2 + ex * (size_t)d * (F / 2);
    const uint8_t* wscales = KIND == 1 ? W.w13_s + ex * (size_t)(2 * F) * (d / 16) : W.w2_s + ex * (size_t)d * (F / 16);

    // ---- copy sources (per lane, fixed over K) ----
    // B codes: copy q (0, 1) of wave w fills rows 16 (2 w + q) .. + 16 of the
    // chunk's code tile (1 KB, lane i at byte 16 i): row r = 16 (2 w + q) + i/4,
    // physical unit i%4, which holds logical unit (i%4) ^ g(r) (t32_cu)
    const uint8_t* bsrc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = 16 * (2 * wave + q) + (lane >> 2);
        const int u = (lane & 3) ^ (((r >> 1) ^ (r >> 3)) & 3);
        bsrc[q] = wcodes + wrow(r) * (K / 2) + u * 16;
    }
    // B scales: wave w, lane i: row 32 w + i/2, dword i%2 of its 8 bytes
    const uint8_t* bssrc = wscales + wrow(32 * wave + (lane >> 1)) * (K / 16) + (lane & 1) * 4;
    // A: NVFP4 codes (waves 0, 1: rows 16 w + i/4, as for B) and scales (wave
    // 2: row i/2, dword i%2); 16-bit rows (every wave: rows 4 w + i/16, physical
    // unit i%16 holding logical unit (i%16) ^ (r & 15))
    const uint8_t* asrc = nullptr;
    if constexpr (AT == 2) {
        const uint8_t* acodes = KIND == 1 ? a.hq_codes : a.act_codes;
        const uint8_t* ascales = KIND == 1 ? a.hq_scales : a.act_scales;
        if (wave < 2) {
            const int r = 16 * wave + (lane >> 2);
            const int u = (lane & 3) ^ (((r >> 1) ^ (r >> 3)) & 3);
            asrc = acodes + arow(r) * (K / 2) + u * 16;
        } else if (wave == 2) {
            asrc = ascales + arow(lane >> 1) * (K / 16) + (lane & 1) * 4;
        }
    } else {
        const uint16_t* abase = KIND == 1 ? (AT == 0 ? a.hidden : a.hq) : a.act;
        const int r = 4 * wave + (lane >> 4);
        const int u = (lane & 15) ^ (r & 15);
        asrc = reinterpret_cast<const uint8_t*>(abase + arow(r) * K + u * 8);
    }

    auto issue = [&](int c, int slot) {
        uint8_t* base = smem + slot * SLOT;
#pragma unroll
        for (int q = 0; q < 2; ++q)
            __builtin_amdgcn_global_load_lds((const void*)(bsrc[q] + c * 64), (t32_lds_t*)(base + (2 * wave + q) * 1024),
                                             16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(bssrc + c * 8), (t32_lds_t*)(base + kTBC + wave * 256), 4, 0, 0);
        uint8_t* abuf = base + kTBC + kTBS;
        if constexpr (AT == 2) {
            if (wave < 2)
                __builtin_amdgcn_global_load_lds((const void*)(asrc + c * 64), (t32_lds_t*)(abuf + wave * 1024), 16, 0, 0);
            else if (wave == 2)
                __builtin_amdgcn_global_load_lds((const void*)(asrc + c * 8), (t32_lds_t*)(abuf + kTM * 64), 4, 0, 0);
        } else {
            __builtin_amdgcn_global_load_lds((const void*)(asrc + c * (kTK * 2)), (t32_lds_t*)(abuf + wave * 1024), 16,
                                             0, 0);
        }
    };

    f32x16_t acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    const int h = lane >> 5, br = 32 * wave + (lane & 31), ar = lane & 31;

    auto compute = [&](const uint8_t* S) {
        const u32x4_t b0 = *reinterpret_cast<const u32x4_t*>(S + t32_cu(br, 2 * h));
        const u32x4_t b1 = *reinterpret_cast<const u32x4_t*>(S + t32_cu(br, 2 * h + 1));
        const uint32_t bs = *reinterpret_cast<const uint32_t*>(S + kTBC + br * 8 + 4 * h);
        const uint8_t* A = S + kTBC + kTBS;
        u32x4_t a0, a1;
        uint32_t as = 0;
        if constexpr (AT == 2) {
            a0 = *reinterpret_cast<const u32x4_t*>(A + t32_cu(ar, 2 * h));
            a1 = *reinterpret_cast<const u32x4_t*>(A + t32_cu(ar, 2 * h + 1));
            as = *reinterpret_cast<const uint32_t*>(A + kTM * 64 + ar * 8 + 4 * h);
        }
        f16x2_t bsl{}, bsh{}, asl{}, ash{};
        if constexpr (AT != 0) {
            bsl = e4m3x2_to_f16(bs);
            bsh = e4m3x2_hi_to_f16(bs);
        }
        if constexpr (AT == 2) {
            asl = e4m3x2_to_f16(as);
            ash = e4m3x2_hi_to_f16(as);
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const uint32_t bcw = kk < 4 ? b0[kk] : b1[kk - 4];
            u32x4_t bv, av;
            if constexpr (AT == 0) {
                bv = dequant8_bf16(bcw, e4m3_to_f32((bs >> (8 * (kk >> 1))) & 0xFFu));
            } else {
                const f16x2_t sp = kk < 4 ? bsl : bsh;
                const _Float16 s = (kk & 2) ? sp.y : sp.x;
                bv = dequant8_f16(bcw, f16x2_t{s, s});
            }
            if constexpr (AT == 2) {
                const f16x2_t sp = kk < 4 ? asl : ash;
                const _Float16 s = (kk & 2) ? sp.y : sp.x;
                av = dequant8_f16(kk < 4 ? a0[kk] : a1[kk - 4], f16x2_t{s, s});
            } else {
                av = *reinterpret_cast<const u32x4_t*>(A + t32_au(ar, 8 * h + kk));
            }
            acc = t32_mfma<AT>(av, bv, acc);
        }
    };

    // copies per chunk of this wave, for the waits
    const int ncopy = AT == 2 ? (wave < 3 ? 4 : 3) : 4;

    // prologue: chunks 0 .. DEPTH - 1 (those that exist)
#pragma unroll
    for (int c = 0; c < DEPTH; ++c)
        if (c < nc) issue(c, c);
    for (int c = 0; c < nc; ++c) {
        // chunk c has landed once at most the copies of chunks c + 1 .. c +
        // DEPTH - 1 are outstanding (when they were all issued)
        if (c + DEPTH - 1 < nc) {
            if (ncopy == 4)
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((DEPTH - 1) * 4) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((DEPTH - 1) * 3) : "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
        if (c + DEPTH < nc) issue(c + DEPTH, (c + DEPTH) % NS);
        compute(smem + (c % NS) * SLOT);
    }

    // ---- epilogue: lane holds rows 8 (v/4) + 4 h + v%4 of column l%32 ----
    const float gsc = KIND == 1 ? W.g13[ex] * a.a1g : W.g2[ex] * a.a2g;   // weight x activation globals
    const int n = lane & 31;
    if constexpr (KIND == 2) {
        const int col = cb * kTN + 32 * wave + n;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = 8 * (v >> 2) + 4 * h + (v & 3);
            if (m < ntok) a.Y[(size_t)(rb + m) * d + col] = (uint16_t)f32_to_bf16_rne(acc[v] * gsc);
        }
    } else {
        const int col = cb * 128 + 16 * wave + (n & 15);      // SwiGLU column (lanes n < 16)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float up = __shfl_xor(acc[v], 16, 64) * gsc;
            const float gt = acc[v] * gsc;
            const float y = gt / (1.0f + expf(-gt)) * up;    // valid in lanes n < 16
            const int m = 8 * (v >> 2) + 4 * h + (v & 3);
            if constexpr (AT == 0) {
                if (n < 16 && m < ntok) a.act[(size_t)(rb + m) * F + col] = (uint16_t)f32_to_bf16_rne(y);
            } else {
                // NVFP4 over the 16 columns of this wave (lanes n = 0..15 of the half)
                float mx = n < 16 ? fabsf(y) : 0.f;
                mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 8, 64));
                const uint32_t sbyte = nvfp4_act_scale(mx, a.a2g);
                const float sc = e4m3_to_f32(sbyte);
                const uint32_t code = nvfp4_act_code(y, sc, a.a2g);
                if constexpr (AT == 1) {
                    if (n < 16 && m < ntok)
                        a.act[(size_t)(rb + m) * F + col] = (uint16_t)f32_to_f16_bits(e2m1_value(code) * sc);
                } else {
                    // element n -> nibble n % 8 of dword n / 8
                    uint32_t wd = n < 16 ? code << (4 * (n & 7)) : 0u;
                    wd |= __shfl_xor(wd, 1, 64);
                    wd |= __shfl_xor(wd, 2, 64);
                    wd |= __shfl_xor(wd, 4, 64);
                    const uint32_t wd_hi = __shfl_down(wd, 8, 64);   // lane n = 0 gets elements 8..15
                    if (n == 0 && m < ntok) {
                        const size_t row = (size_t)(rb + m);
                        const int c0 = cb * 128 + 16 * wave;
                        *reinterpret_cast<u32x2_t*>(a.act_codes + row * (F / 2) + c0 / 2) = u32x2_t{wd, wd_hi};
                        a.act_scales[row * (F / 16) + c0 / 16] = (uint8_t)sbyte;
                    }
                }
            }
        }
    }
}

template <int KIND, int AT>
static hipError_t launch_t32(const GemmArgs& a, hipStream_t s) {
    const hipError_t e = allow_dynamic_lds<t32_gemm_kernel<KIND, AT>>(t32_lds<AT>());
    if (e != hipSuccess) return e;
    const int ncb = KIND == 1 ? a.F / 128 : a.d / kTN;
    const long long n = (long long)a.max_tiles * ncb;
    if (n == 0) return hipSuccess;
    // (max_tiles x ncb) as a 2-D grid whose x extent stays within the limit
    const unsigned gx = (unsigned)(n < 65536 ? n : 65536);
    const unsigned gy = (unsigned)((n + gx - 1) / gx);
    hipLaunchKernelGGL((t32_gemm_kernel<KIND, AT>), dim3(gx, gy), dim3(64 * kTWaves), t32_lds<AT>(), s, a);
    return hipGetLastError();
}

bool t32_ok(int d, int F) { return d % kTN == 0 && F % 128 == 0; }
int t32_rows() { return kTM; }

hipError_t launch_t32_gemm1(const GemmArgs& a, hipStream_t s) {
    if (a.packed) return launch_t32<1, 2>(a, s);
    return a.mode == 0 ? launch_t32<1, 0>(a, s) : launch_t32<1, 1>(a, s);
}

hipError_t launch_t32_gemm2(const GemmArgs& a, hipStream_t s) {
    if (a.packed) return launch_t32<2, 2>(a, s);
    return a.mode == 0 ? launch_t32<2, 0>(a, s) : launch_t32<2, 1>(a, s);
}

}  // namespace moe
