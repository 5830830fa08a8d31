// Dense weight-streaming expert GEMMs for mid-size token counts per expert
// (tiles of 16 token rows), gfx950.
//
// Between decode (a few tokens per expert: the block-diagonal kernels of
// decode.hip) and prefill (hundreds: the 256-row tiles of prefill.hip), each
// expert sees tens of tokens.  The layer is still bound by streaming every
// touched expert's NVFP4 weights from HBM once, but a block-diagonal MFMA,
// which wastes 3/4 of each instruction to apply the block scales after the
// product, is then short of MFMA throughput, and a 256-row tile is mostly
// padding.  Here each weight element is decoded WITH its E4M3 block scale
// (code * scale is exact in 16 bits: at most 6 significant bits) straight
// into the B fragment of a dense v_mfma_f32_16x16x32_{f16,bf16}, whose A
// fragment is 16 token rows: every MFMA is fully used, and the decode costs one
// VALU op per element (W4A4: packed f16 multiply) or two (W4A16: fp32 multiply,
// bf16 pack).
//
// Workgroup: 4 waves over one tile of at most 16 TG token rows and 256 weight
// rows; a wave owns NR = 4 groups of 16 weight rows for the whole K range:
//   GEMM1: SwiGLU columns [c, c + 32) with c = 128 cb + 32 wave; row groups 0, 1
//          are the gate rows c .. c + 32, row groups 2, 3 the matching up rows
//          F + c .. F + c + 32, so silu(gate) * up is formed in registers;
//   GEMM2: output columns 256 cb + 64 wave + 16 r, r = 0..3.
// K order (the MFMA sums its 32 k in any order if both operands use the same
// one): K is cut into 64-element chunks; at step s (256 k) lane group g = l/16
// takes chunk 4 s + g -- its 32 code bytes and 4 scale bytes, so the four lane
// groups of a weight row read one whole 128-byte line -- and MFMA q (0..7) of
// the step takes elements 8 q .. 8 q + 8 of each lane group's chunk (block q/2).
// Lane layout of v_mfma_f32_16x16x32 (checked on the device for the bf16 form
// the decode kernels use; the f16 form is the same): lane l holds A[l%16][8 k]
// and B[8 k][l%16] of its lane group's 8 k; D[4 (l/16) + i][l%16], i = 0..3.
// Here A rows are tokens and B columns are weight rows.
//
// Weights stream through a register prefetch ring kMidDepth steps deep (every
// row group of a step is loaded together).  Token rows are staged in LDS one
// step (256 k) at a time, double-buffered: the next step's pieces are loaded
// into registers at the start of a step and stored at its end, and the
// workgroup then meets at an LDS-only barrier (s_waitcnt lgkmcnt(0);
// s_barrier), so the weight ring is never drained.  (Copying the token rows
// straight into LDS with global_load_lds saves those registers, but the
// compiler then waits for every outstanding load before each LDS read.)
//
// Layer semantics: the page "Serving Solar Open 2 on DGX Spark", sections "수정
// 사항 › b12x에서의 Expert Parallelism 구현 추가" (one shard's experts, partial sum)
// and "b12x 버전이 실제 NVFP4 체크포인트를 읽어들이도록 만들기" (packed FP4 codes,
// FP8 block scales, per-expert fp32 global scale, fused gate/up).
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kMidWaves = 8;
constexpr int kMidNR = 2;            // row groups of 16 weight rows per wave
constexpr int kMidDepth = 2;         // weight prefetch ring depth (steps of 256 k)
constexpr int kMidKS = 256;          // K elements per step (and per LDS stage)
constexpr int kMidPad = 8;           // 16-bit elements of padding per LDS row
constexpr int kMidLdw = kMidKS + kMidPad;
// dword 3 of a raw (untyped) buffer resource on gfx9-family parts: 32-bit data
// format, no swizzle; offsets at or past num_records read 0
constexpr int kBufferFlags = 0x00020000;


template <int MODE>
__device__ __forceinline__ f32x4_t mid_mfma(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
    if constexpr (MODE == 1)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// KIND 1: GEMM1 + SwiGLU (A = hidden rows, or the W4A4 hidden quantized to
// exact f16, gathered through the permutation; writes act).  KIND 2: GEMM2
// (A = act rows; writes Y).  MODE 0: bf16 operands; 1: f16 (W4A4).  The
// grid is (max_tiles x column blocks), column blocks varying fastest so that
// the workgroups of tiles past the table's end (which only return) come last.
// SEG (K % 1024 == 0): the block scales arrive as one 16-byte segment per row
// group every four steps (scale_seg_transpose) instead of a 4-byte load per
// step; a streaming probe with this kernel's ring (2 steps, 2 row groups, 4
// waves per SIMD) reads 6.14 TB/s that way against 5.63 TB/s.
template <int KIND, int MODE, int TG, bool SEG>
__global__ __launch_bounds__(64 * kMidWaves) __attribute__((amdgpu_waves_per_eu(4))) void mid_gemm_kernel(GemmArgs a) {
    constexpr int ROWS = 16 * TG;
    constexpr int NR = kMidNR, DEPTH = kMidDepth;
    constexpr int APT = ROWS * (kMidKS / 8) / (64 * kMidWaves);   // 16-byte A pieces per thread per step
    static_assert(APT * 64 * kMidWaves == ROWS * kMidKS / 8, "A staging covers the step");
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * ROWS * kMidLdw];
    __shared__ const uint16_t* s_arow[ROWS];

    const int d = a.d, F = a.F;
    const int ncb = KIND == 1 ? F / 128 : d / 256;
    const long long lin = blockIdx.x + (long long)blockIdx.y * gridDim.x;
    const int tile = (int)(lin / ncb), cb = (int)(lin - (long long)tile * ncb);
    if (tile >= *a.ntiles) return;
    const int4 tt = a.tiles[tile];
    const int rb = tt.y, re = tt.z, ntok = re - rb;
    const bool shared = tt.x == a.L;
    const ExpertWeights& W = shared ? a.shared : a.local;
    const size_t ex = shared ? 0 : (size_t)tt.x;
    const int K = KIND == 1 ? d : F;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;

    // token rows of the tile (padding rows repeat the first row; discarded)
    if (tid < ROWS) {
        const int row = rb + (tid < ntok ? tid : 0);
        const uint16_t* p;
        if (KIND == 1) {
            const int t = shared ? row - a.T * a.topk : a.perm[row] / a.topk;
            p = (MODE == 0 ? a.hidden : a.hq) + (size_t)t * d;
        } else {
            p = a.act + (size_t)row * F;
        }
        s_arow[tid] = p;
    }

    // weight rows of this wave's row groups: row group r sits roff(r) rows past
    // the wave's first row (a wave-uniform offset)
    // the expert's weight tensors as buffer resources (wave-uniform bases in
    // SGPRs): a load is the lane's 32-bit offset (its row's start, plus the
    // step's chunk) plus row group r's wave-uniform offset roff(r) rows, so the
    // ring needs no 64-bit address per row group and step
    __amdgpu_buffer_rsrc_t crs, srs;
    int lane_c, lane_s;
    {
        const int rows = KIND == 1 ? 2 * F : d;
        const uint8_t* codes = KIND == 1 ? W.w13 + ex * (size_t)rows * (d / 2) : W.w2 + ex * (size_t)rows * (F / 2);
        const uint8_t* scales =
            KIND == 1 ? W.w13_s + ex * (size_t)rows * (d / 16) : W.w2_s + ex * (size_t)rows * (F / 16);
        crs = __builtin_amdgcn_make_buffer_rsrc((void*)codes, (short)0, rows * (K / 2), kBufferFlags);
        srs = __builtin_amdgcn_make_buffer_rsrc((void*)scales, (short)0, rows * (K / 16), kBufferFlags);
        const int wrow = KIND == 1 ? cb * 128 + wave * (8 * NR) + n : cb * 256 + wave * (16 * NR) + n;
        lane_c = wrow * (K / 2);
        lane_s = wrow * (K / 16);
    }
    auto roff = [&](int r) -> int { return KIND == 1 ? (r >= NR / 2 ? F : 0) + (r % (NR / 2)) * 16 : r * 16; };
    const float gsc = KIND == 1 ? W.g13[ex] * a.a1g : W.g2[ex] * a.a2g;   // weight x activation globals

    const int nsteps = (K + 255) / 256;                 // K % 128 == 0
    const int last_chunk = K / 64 - 1;
    // ring slot: per row group, the lane's 32 code bytes and 4 scale bytes of step v
    u32x4_t rl[DEPTH][NR], rh[DEPTH][NR];
    uint32_t rs[DEPTH][NR];
    auto load_step = [&](int v, u32x4_t (&lo)[NR], u32x4_t (&hi)[NR], uint32_t (&sc)[NR]) {
        const int st = v < nsteps ? v : nsteps - 1;
        const int ci = min(st * 4 + g, last_chunk);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            lo[r] = __builtin_amdgcn_raw_buffer_load_b128(crs, lane_c + ci * 32, roff(r) * (K / 2), 0);
            hi[r] = __builtin_amdgcn_raw_buffer_load_b128(crs, lane_c + ci * 32 + 16, roff(r) * (K / 2), 0);
            if (!SEG) sc[r] = __builtin_amdgcn_raw_buffer_load_b32(srs, lane_s + ci * 4, roff(r) * (K / 16), 0);
        }
    };
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) load_step(u, rl[u], rh[u], rs[u]);
    // SEG: the segments of the current group of four steps (transposed) and of
    // the next one (in flight); lane group m loads step 4 G + m's segment
    u32x4_t seg_cur[NR], seg_next[NR];
    auto load_seg = [&](int r, int grp) -> u32x4_t {
        const int st = min(grp * 4 + g, nsteps - 1);
        return __builtin_amdgcn_raw_buffer_load_b128(srs, lane_s + st * 16, roff(r) * (K / 16), 0);
    };
    if (SEG) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            seg_cur[r] = scale_seg_transpose(load_seg(r, 0));
            seg_next[r] = load_seg(r, 1);
        }
    }

    // ---- A: the step's 256 elements of every token row, double-buffered in
    // LDS; the next step's pieces are loaded into registers at the start of a
    // step and stored at its end, then the workgroup meets at a barrier that
    // waits only for LDS traffic (the weight ring stays in flight)
    __syncthreads();                                    // s_arow visible
    u32x4_t va[APT];
    auto a_load = [&](int st) {
#pragma unroll
        for (int j = 0; j < APT; ++j) {
            const int piece = tid + j * (64 * kMidWaves);
            const int row = piece >> 5, col = st * kMidKS + (piece & 31) * 8;
            va[j] = *reinterpret_cast<const u32x4_t*>(s_arow[row] + (col < K ? col : K - 8));   // unconditional
        }
    };
    auto a_store = [&](int st, uint16_t* b) {
#pragma unroll
        for (int j = 0; j < APT; ++j) {
            const int piece = tid + j * (64 * kMidWaves);
            const int row = piece >> 5, colc = (piece & 31) * 8;
            if (st * kMidKS + colc < K) *reinterpret_cast<u32x4_t*>(b + row * kMidLdw + colc) = va[j];
        }
    };
    a_load(0);
    a_store(0, lds);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    f32x4_t acc[NR][TG];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < TG; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const u32x4_t zero4 = {0u, 0u, 0u, 0u};

    // one step: ring slot u holds step s; A of step s is in LDS buffer s & 1
    auto do_step = [&](const int u, const int s) {
        const bool more = s + 1 < nsteps;
        if (more) a_load(s + 1);
        if (SEG && (s & 3) == 0 && s > 0) {
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                seg_cur[r] = scale_seg_transpose(seg_next[r]);
                seg_next[r] = load_seg(r, s / 4 + 1);
            }
        }
        uint32_t sw[NR];                                // this lane's chunk scales of step s
#pragma unroll
        for (int r = 0; r < NR; ++r) sw[r] = SEG ? seg_word(seg_cur[r], s & 3) : rs[u][r];
        const bool kvalid = (s * 4 + g) * 64 < K;
        const uint16_t* ab = lds + (s & 1) * (ROWS * kMidLdw) + g * 64;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            u32x4_t af[TG];
#pragma unroll
            for (int t = 0; t < TG; ++t)
                af[t] = kvalid ? *reinterpret_cast<const u32x4_t*>(ab + (t * 16 + n) * kMidLdw + q * 8) : zero4;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const uint32_t cw = q < 4 ? rl[u][r][q] : rh[u][r][q - 4];
                u32x4_t bf;
                if constexpr (MODE == 1) {
                    const f16x2_t sp = q < 4 ? e4m3x2_to_f16(sw[r]) : e4m3x2_hi_to_f16(sw[r]);
                    const _Float16 sh = (q & 2) ? sp.y : sp.x;
                    bf = dequant8_f16(cw, f16x2_t{sh, sh});
                } else {
                    bf = dequant8_bf16(cw, e4m3_to_f32((sw[r] >> (8 * (q >> 1))) & 0xFFu));
                }
#pragma unroll
                for (int t = 0; t < TG; ++t) acc[r][t] = mid_mfma<MODE>(af[t], bf, acc[r][t]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // refill the slot with step s + DEPTH only after its last use, so the new
        // loads take over the same registers
        load_step(s + DEPTH, rl[u], rh[u], rs[u]);
        if (more) {
            a_store(s + 1, lds + ((s + 1) & 1) * (ROWS * kMidLdw));
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
    };
    // whole ring rounds; a step past K (when DEPTH does not divide the step
    // count) multiplies zero A fragments and loads nothing new (a separate
    // tail would make the compiler keep a second copy of the ring)
    for (int s0 = 0; s0 < nsteps; s0 += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) do_step(u, s0 + u);
    }

    // ---- epilogue: lane holds rows 4 g + i (+16 t) of columns n of each row group ----
    if (KIND == 1) {
#pragma unroll
        for (int h = 0; h < NR / 2; ++h) {
            const int col = cb * 128 + wave * (8 * NR) + h * 16 + n;
#pragma unroll
            for (int t = 0; t < TG; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float gt = acc[h][t][i] * gsc, up = acc[h + NR / 2][t][i] * gsc;
                    float av = gt / (1.0f + expf(-gt)) * up;
                    if (MODE == 1) {
                        // NVFP4 quantize-dequantize over the 16 columns held by lanes n = 0..15
                        float m = fabsf(av);
                        m = fmaxf(m, __shfl_xor(m, 1, 64));
                        m = fmaxf(m, __shfl_xor(m, 2, 64));
                        m = fmaxf(m, __shfl_xor(m, 4, 64));
                        m = fmaxf(m, __shfl_xor(m, 8, 64));
                        av = nvfp4_fake_quant(av, m, a.a2g);
                    }
                    const int m_row = t * 16 + g * 4 + i;
                    if (m_row < ntok)
                        a.act[(size_t)(rb + m_row) * F + col] =
                            (uint16_t)(MODE == 1 ? f32_to_f16_bits(av) : f32_to_bf16_rne(av));
                }
        }
    } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int col = cb * 256 + wave * (16 * NR) + r * 16 + n;
#pragma unroll
            for (int t = 0; t < TG; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m_row = t * 16 + g * 4 + i;
                    if (m_row < ntok)
                        a.Y[(size_t)(rb + m_row) * d + col] = (uint16_t)f32_to_bf16_rne(acc[r][t][i] * gsc);
                }
        }
    }
}

// ---------------------------------------------------------------------------
// W4A4 with the activations as NVFP4 (codes + E4M3 block scales, the packed
// activation quantizer's output for GEMM1, GEMM1's own packed output for
// GEMM2).  The tile's 16 TG token rows are staged in LDS ONCE, for the whole
// K range, as NVFP4 (a ninth of their 16-bit size: 75 KB for 32 rows at
// K = 4096), so the K loop has no barrier and the weight ring runs kMid4Depth
// steps deep.  A workgroup walks CBW column blocks back to back (the ring runs
// on across them, and the staged rows serve them all).  Per step a lane reads
// its tokens' 32 code bytes and 4 scale bytes of its lane group's chunk and
// decodes each A fragment once (shared by the four row groups); B is decoded
// as in mid_gemm_kernel.  GEMM1's epilogue quantizes the SwiGLU output per 16
// columns and writes it packed.
// ---------------------------------------------------------------------------
constexpr int kMid4Depth = 2;
constexpr int kMid4Waves = 8;
constexpr int kMid4NR = 2;           // row groups of 16 weight rows per wave
constexpr int kMid4TG = 2;           // token groups: 32-row tiles
constexpr int kMid4CodePad = 16;     // bytes of padding per LDS code row
constexpr int kMid4ScalePad = 16;    // bytes of padding per LDS scale row (16 lanes read 16 rows' dwords)
constexpr int kMid4MaxK = 8192;      // largest K whose 32-row NVFP4 stage fits (148 KB)

__host__ __device__ constexpr int mid4_lds_bytes(int K) {
    return 16 * kMid4TG * ((K / 2 + kMid4CodePad) + (K / 16 + kMid4ScalePad));
}

template <int KIND, int CBW, bool SEG>
__global__ __launch_bounds__(64 * kMid4Waves) __attribute__((amdgpu_waves_per_eu(4))) void mid4_gemm_kernel(GemmArgs a) {
    constexpr int NR = kMid4NR, DEPTH = kMid4Depth, TG = kMid4TG, ROWS = 16 * TG;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int s_arow[ROWS];

    const int d = a.d, F = a.F;
    const int ncb = (KIND == 1 ? F / 128 : d / 256) / CBW;   // workgroups per tile
    const long long lin = blockIdx.x + (long long)blockIdx.y * gridDim.x;
    const int tile = (int)(lin / ncb), cbw = (int)(lin - (long long)tile * ncb);
    if (tile >= *a.ntiles) return;
    const int4 tt = a.tiles[tile];
    const int rb = tt.y, re = tt.z, ntok = re - rb;
    const bool shared = tt.x == a.L;
    const ExpertWeights& W = shared ? a.shared : a.local;
    const size_t ex = shared ? 0 : (size_t)tt.x;
    const int K = KIND == 1 ? d : F;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int CR = K / 2 + kMid4CodePad;                 // LDS code row stride (bytes)
    const int SR = K / 16 + kMid4ScalePad;               // LDS scale row stride (bytes)
    uint8_t* const lcodes = smem;
    uint8_t* const lscales = smem + ROWS * CR;

    // activation row of each tile row (padding rows repeat the first row)
    if (tid < ROWS) {
        const int row = rb + (tid < ntok ? tid : 0);
        s_arow[tid] = KIND == 1 ? (shared ? row - a.T * a.topk : a.perm[row] / a.topk) : row;
    }

    // the expert's weight tensors as buffer resources (see mid_gemm_kernel);
    // column block j of this workgroup starts cstep(j) rows past block 0
    __amdgpu_buffer_rsrc_t crs, srs;
    int lane_c, lane_s;
    {
        const int rows = KIND == 1 ? 2 * F : d;
        const uint8_t* codes = KIND == 1 ? W.w13 + ex * (size_t)rows * (d / 2) : W.w2 + ex * (size_t)rows * (F / 2);
        const uint8_t* scales =
            KIND == 1 ? W.w13_s + ex * (size_t)rows * (d / 16) : W.w2_s + ex * (size_t)rows * (F / 16);
        crs = __builtin_amdgcn_make_buffer_rsrc((void*)codes, (short)0, rows * (K / 2), kBufferFlags);
        srs = __builtin_amdgcn_make_buffer_rsrc((void*)scales, (short)0, rows * (K / 16), kBufferFlags);
        const int wrow = KIND == 1 ? cbw * CBW * 128 + wave * (8 * NR) + n : cbw * CBW * 256 + wave * (16 * NR) + n;
        lane_c = wrow * (K / 2);
        lane_s = wrow * (K / 16);
    }
    auto roff = [&](int r, int j) -> int {
        return KIND == 1 ? (r >= NR / 2 ? F : 0) + (r % (NR / 2)) * 16 + j * 128 : r * 16 + j * 256;
    };
    const float gsc = KIND == 1 ? W.g13[ex] * a.a1g : W.g2[ex] * a.a2g;

    const int nsteps = (K + 255) / 256;
    const int nsp = (nsteps + DEPTH - 1) / DEPTH * DEPTH;   // steps per column block, whole ring rounds
    const int nvirt = CBW * nsp;
    const int last_chunk = K / 64 - 1;
    u32x4_t rl[DEPTH][NR], rh[DEPTH][NR];
    uint32_t rs[DEPTH][NR];
    auto load_step = [&](int v, u32x4_t (&lo)[NR], u32x4_t (&hi)[NR], uint32_t (&sc)[NR]) {
        const int vv = v < nvirt ? v : nvirt - 1;
        const int j = vv / nsp, st = min(vv - j * nsp, nsteps - 1);
        const int ci = min(st * 4 + g, last_chunk);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            lo[r] = __builtin_amdgcn_raw_buffer_load_b128(crs, lane_c + ci * 32, roff(r, j) * (K / 2), 0);
            hi[r] = __builtin_amdgcn_raw_buffer_load_b128(crs, lane_c + ci * 32 + 16, roff(r, j) * (K / 2), 0);
            if (!SEG)
                sc[r] = __builtin_amdgcn_raw_buffer_load_b32(srs, lane_s + ci * 4, roff(r, j) * (K / 16), 0);
        }
    };
    // SEG (K % 1024 == 0, so a column block's steps are whole groups of four):
    // scales in 16-byte segments, as in mid_gemm_kernel; groups count virtual steps
    u32x4_t seg_cur[NR], seg_next[NR];
    auto load_seg = [&](int r, int grp) -> u32x4_t {
        const int vv = min(grp * 4 + g, nvirt - 1);
        const int j = vv / nsp, st = min(vv - j * nsp, nsteps - 1);
        return __builtin_amdgcn_raw_buffer_load_b128(srs, lane_s + st * 16, roff(r, j) * (K / 16), 0);
    };
    // the ring's first loads go out before the A stage, so both are in flight together
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) load_step(u, rl[u], rh[u], rs[u]);
    if (SEG) {
#pragma unroll
        for (int r = 0; r < NR; ++r) seg_next[r] = load_seg(r, 0);   // transposed before step 0
    }

    // ---- whole-K NVFP4 stage of the token rows ----
    __syncthreads();                                     // s_arow visible
    {
        const uint8_t* acodes = KIND == 1 ? a.hq_codes : a.act_codes;
        const uint8_t* ascales = KIND == 1 ? a.hq_scales : a.act_scales;
        const int cp = K / 32;                           // 16-byte code pieces per row
        const int sp = K / 256;                          // 16-byte scale pieces per row
        const int total = ROWS * (cp + sp);
        for (int p0 = 0; p0 < total; p0 += 8 * 64 * kMid4Waves) {
            u32x4_t v[8];
            // loads unconditional (clamped; see dec_stream), stores conditional
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int p = min(p0 + j * 64 * kMid4Waves + tid, total - 1);
                const bool code = p < ROWS * cp;
                const int q = code ? p : p - ROWS * cp;
                const int per = code ? cp : sp;
                const int row = q / per, c = q - row * per;
                const uint8_t* src = code ? acodes + (size_t)s_arow[row] * (K / 2) : ascales + (size_t)s_arow[row] * (K / 16);
                v[j] = *reinterpret_cast<const u32x4_t*>(src + c * 16);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int p = p0 + j * 64 * kMid4Waves + tid;
                if (p < ROWS * cp) {
                    const int row = p / cp, c = p - row * cp;
                    *reinterpret_cast<u32x4_t*>(lcodes + row * CR + c * 16) = v[j];
                } else if (p < total) {
                    const int q = p - ROWS * cp, row = q / sp, c = q - row * sp;
                    *reinterpret_cast<u32x4_t*>(lscales + row * SR + c * 16) = v[j];
                }
            }
        }
    }
    __syncthreads();

    f32x4_t acc[NR][TG];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < TG; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const u32x4_t zero4 = {0u, 0u, 0u, 0u};

    // ---- epilogue of column block j: lane holds rows 16 t + 4 g + i of columns n ----
    auto epilogue = [&](int j) {
        if (KIND == 1) {
#pragma unroll
            for (int h = 0; h < NR / 2; ++h) {
                const int col0 = (cbw * CBW + j) * 128 + wave * (8 * NR) + h * 16;   // the block's first column
#pragma unroll
                for (int t = 0; t < TG; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float gt = acc[h][t][i] * gsc, up = acc[h + NR / 2][t][i] * gsc;
                        const float av = gt / (1.0f + expf(-gt)) * up;
                        // NVFP4 over the block's 16 columns (lanes n = 0..15 of lane group g)
                        float m = fabsf(av);
                        m = fmaxf(m, __shfl_xor(m, 1, 64));
                        m = fmaxf(m, __shfl_xor(m, 2, 64));
                        m = fmaxf(m, __shfl_xor(m, 4, 64));
                        m = fmaxf(m, __shfl_xor(m, 8, 64));
                        const uint32_t sbyte = nvfp4_act_scale(m, a.a2g);
                        const uint32_t code = nvfp4_act_code(av, e4m3_to_f32(sbyte), a.a2g);
                        // element n -> nibble n % 8 of dword n / 8
                        uint32_t w = code << (4 * (n & 7));
                        w |= __shfl_xor(w, 1, 64);
                        w |= __shfl_xor(w, 2, 64);
                        w |= __shfl_xor(w, 4, 64);
                        const uint32_t w_hi = __shfl_down(w, 8, 64);   // lane n = 0 gets elements 8..15
                        const int m_row = t * 16 + g * 4 + i;
                        if (n == 0 && m_row < ntok) {
                            const size_t row = (size_t)(rb + m_row);
                            *reinterpret_cast<u32x2_t*>(a.act_codes + row * (F / 2) + col0 / 2) = u32x2_t{w, w_hi};
                            a.act_scales[row * (F / 16) + col0 / 16] = (uint8_t)sbyte;
                        }
                    }
            }
        } else {
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int col = (cbw * CBW + j) * 256 + wave * (16 * NR) + r * 16 + n;
#pragma unroll
                for (int t = 0; t < TG; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m_row = t * 16 + g * 4 + i;
                        if (m_row < ntok)
                            a.Y[(size_t)(rb + m_row) * d + col] = (uint16_t)f32_to_bf16_rne(acc[r][t][i] * gsc);
                    }
            }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int t = 0; t < TG; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    };

    // one step: ring slot u holds virtual step v (column block v / nsp, K step st = v % nsp)
    auto do_step = [&](const int u, const int st, const int v) {
        if (SEG && (v & 3) == 0) {
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                seg_cur[r] = scale_seg_transpose(seg_next[r]);
                seg_next[r] = load_seg(r, v / 4 + 1);
            }
        }
        uint32_t sw[NR];                                // this lane's chunk scales of step st
#pragma unroll
        for (int r = 0; r < NR; ++r) sw[r] = SEG ? seg_word(seg_cur[r], v & 3) : rs[u][r];
        const int ci = st * 4 + g;
        const bool kvalid = ci * 64 < K;
        const int cic = kvalid ? ci : 0;
        // this lane's token rows n and 16 + n: 32 code bytes and 4 scale bytes of chunk ci
        u32x4_t alo[TG], ahi[TG];
        uint32_t asc[TG];
#pragma unroll
        for (int t = 0; t < TG; ++t) {
            alo[t] = *reinterpret_cast<const u32x4_t*>(lcodes + (t * 16 + n) * CR + cic * 32);
            ahi[t] = *reinterpret_cast<const u32x4_t*>(lcodes + (t * 16 + n) * CR + cic * 32 + 16);
            asc[t] = *reinterpret_cast<const uint32_t*>(lscales + (t * 16 + n) * SR + cic * 4);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            u32x4_t af[TG];
#pragma unroll
            for (int t = 0; t < TG; ++t) {
                const f16x2_t sp = q < 4 ? e4m3x2_to_f16(asc[t]) : e4m3x2_hi_to_f16(asc[t]);
                const _Float16 sa = (q & 2) ? sp.y : sp.x;
                af[t] = kvalid ? dequant8_f16(q < 4 ? alo[t][q] : ahi[t][q - 4], f16x2_t{sa, sa}) : zero4;
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const uint32_t cw = q < 4 ? rl[u][r][q] : rh[u][r][q - 4];
                const f16x2_t sp = q < 4 ? e4m3x2_to_f16(sw[r]) : e4m3x2_hi_to_f16(sw[r]);
                const _Float16 sb = (q & 2) ? sp.y : sp.x;
                const u32x4_t bf = dequant8_f16(cw, f16x2_t{sb, sb});
#pragma unroll
                for (int t = 0; t < TG; ++t) acc[r][t] = mid_mfma<1>(af[t], bf, acc[r][t]);
            }
            // decode each column's operands next to its MFMAs
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // whole ring rounds per column block (steps past K multiply zero A
    // fragments); the ring runs on from one column block into the next
    for (int v0 = 0; v0 < nvirt; v0 += DEPTH) {
        const int j = v0 / nsp, st0 = v0 - j * nsp;
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            do_step(u, st0 + u, v0 + u);
            load_step(v0 + u + DEPTH, rl[u], rh[u], rs[u]);
        }
        if constexpr (CBW > 1) {
            if (st0 + DEPTH == nsp) epilogue(j);
        }
    }
    // one column block: its epilogue after the loop, where the ring is dead
    if constexpr (CBW == 1) epilogue(0);
}

// Shapes the mid path takes: d a multiple of 256 (GEMM2's 256-column blocks),
// F a multiple of 128 (always).
bool mid_ok(int d, int F) { return d % 256 == 0 && F % 128 == 0; }

// Token rows per tile, from the expected pairs per local expert T k / E: 16
// (one MFMA token group) up to 12, else 32 (one weight stream for up to 32
// pairs, at twice the MFMA work per weight element).  An expert with more pairs
// than a tile holds streams its weights once per tile, the later tiles'
// workgroups right after the first's (column blocks vary fastest).  Measured on
// the 4096 x 1024 layer with 160 local experts, W4A16, per layer: T = 384 (9.6
// pairs per expert) 372 us with 16 rows against 396 with 32; T = 512 (12.8)
// 413 against 408; T = 768 567 against 441.
int mid_rows(int T, int topk, int E) { return (double)T * topk / E <= 12.0 ? 16 : 32; }

template <int KIND, int MODE, int TG>
static hipError_t launch_mid(const GemmArgs& a, hipStream_t s) {
    const int ncb = KIND == 1 ? a.F / 128 : a.d / 256;
    const long long n = (long long)a.max_tiles * ncb;
    if (n == 0) return hipSuccess;
    // (max_tiles x ncb) as a 2-D grid whose x extent stays within the limit
    const unsigned gx = (unsigned)(n < 65536 ? n : 65536);
    const unsigned gy = (unsigned)((n + gx - 1) / gx);
    if ((KIND == 1 ? a.d : a.F) % 1024 == 0)
        hipLaunchKernelGGL((mid_gemm_kernel<KIND, MODE, TG, true>), dim3(gx, gy), dim3(64 * kMidWaves), 0, s, a);
    else
        hipLaunchKernelGGL((mid_gemm_kernel<KIND, MODE, TG, false>), dim3(gx, gy), dim3(64 * kMidWaves), 0, s, a);
    return hipGetLastError();
}

bool mid_packed_ok(int d, int F) {
    return d % 256 == 0 && F % 256 == 0 && d <= kMid4MaxK && F <= kMid4MaxK;
}

int mid_rows_packed() { return 16 * kMid4TG; }

// Column blocks a workgroup walks: GEMM1 1 (its 16-step K is long enough),
// GEMM2 2 (512 output columns: 8 steps at K = 1024), where they divide the
// blocks of the layer.
template <int KIND, int CBW, bool SEG>
static hipError_t launch_mid4_seg(const GemmArgs& a, hipStream_t s) {
    const int K = KIND == 1 ? a.d : a.F;
    const int lds = mid4_lds_bytes(K);
    const hipError_t e = allow_dynamic_lds<mid4_gemm_kernel<KIND, CBW, SEG>>(lds);
    if (e != hipSuccess) return e;
    const int ncb = (KIND == 1 ? a.F / 128 : a.d / 256) / CBW;
    const long long n = (long long)a.max_tiles * ncb;
    if (n == 0) return hipSuccess;
    const unsigned gx = (unsigned)(n < 65536 ? n : 65536);
    const unsigned gy = (unsigned)((n + gx - 1) / gx);
    hipLaunchKernelGGL((mid4_gemm_kernel<KIND, CBW, SEG>), dim3(gx, gy), dim3(64 * kMid4Waves), lds, s, a);
    return hipGetLastError();
}

template <int KIND, int CBW>
static hipError_t launch_mid4_cbw(const GemmArgs& a, hipStream_t s) {
    const int K = KIND == 1 ? a.d : a.F;
    return K % 1024 == 0 ? launch_mid4_seg<KIND, CBW, true>(a, s) : launch_mid4_seg<KIND, CBW, false>(a, s);
}

template <int KIND>
static hipError_t launch_mid4(const GemmArgs& a, hipStream_t s) {
    const int blocks = KIND == 1 ? a.F / 128 : a.d / 256;
    if (KIND == 1) return launch_mid4_cbw<1, 1>(a, s);
    return blocks % 2 == 0 ? launch_mid4_cbw<2, 2>(a, s) : launch_mid4_cbw<2, 1>(a, s);
}

// packed (W4A4 with NVFP4 activations): mid4 kernels; else 16-bit activations
hipError_t launch_mid_gemm1(const GemmArgs& a, hipStream_t s) {
    if (a.packed) return launch_mid4<1>(a, s);
    if (mid_rows(a.T, a.topk, a.E) == 16)
        return a.mode == 0 ? launch_mid<1, 0, 1>(a, s) : launch_mid<1, 1, 1>(a, s);
    return a.mode == 0 ? launch_mid<1, 0, 2>(a, s) : launch_mid<1, 1, 2>(a, s);
}

hipError_t launch_mid_gemm2(const GemmArgs& a, hipStream_t s) {
    if (a.packed) return launch_mid4<2>(a, s);
    if (mid_rows(a.T, a.topk, a.E) == 16)
        return a.mode == 0 ? launch_mid<2, 0, 1>(a, s) : launch_mid<2, 1, 1>(a, s);
    return a.mode == 0 ? launch_mid<2, 0, 2>(a, s) : launch_mid<2, 1, 2>(a, s);
}

}  // namespace moe
