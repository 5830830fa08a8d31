// Weight-streaming expert GEMMs for small token counts per expert (gfx950).
//
// When each expert sees only a few tokens (decode, or a shard's share of a small
// batch) the layer is bound by streaming the NVFP4 weights from HBM once.  Each
// wave owns 16 weight rows at a time, loads 32 contiguous code bytes per lane per
// step with a register prefetch ring DEPTH steps deep, and walks RGS row groups
// back to back so the ring never drains between them.  The workgroup's waves
// share the token rows through LDS: the whole K range when it fits, else
// double-buffered 512-element chunks.
//
// Block-diagonal MFMA (v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8 k] and
// B[8 k][l%16]; D[4 rows][l%16]).  The reduction index is a free permutation:
// K is cut into chunks of 64 elements (32 code bytes, 4 E4M3 scale bytes); at
// step i lane group g = l/16 takes chunk 4i + g, so the four lanes of a weight
// row read one whole 128-byte line per step.  B = the codes decoded UNSCALED to
// bf16 (v_cvt_scalef32_pk_bf16_fp4 with scale 1: exact, one instruction per two
// codes).  A row m = 4 j + t holds token t of the current group of four,
// restricted to the K elements of lane group j (zero elsewhere).  An MFMA pair
// over 16 consecutive elements of the chunk then yields, in lane group j, the
// four tokens' partial dot products over exactly one 16-element block of row n
// -- the block whose E4M3 scale that lane already holds -- so the scale is
// applied with one fp32 FMA per output.  After the K loop the four lane groups
// are summed (two xor-shuffles) and the fp32 global scale is applied.  Cost:
// ~0.8 VALU op per weight element for four tokens, against ~2 for
// dequantize-then-MFMA.
//
// GEMM1 epilogue: a = silu(gate) * up (rows [0,F) of w13 gate, [F,2F) up), bf16;
// W4A4 quantize-dequantizes a per 16 columns.  GEMM2: Y = acc * g2 (bf16 rows).
// Layer semantics: the page "Serving Solar Open 2 on DGX Spark", sections "수정
// 사항 › b12x에서의 Expert Parallelism 구현 추가" and "b12x 버전이 실제 NVFP4
// 체크포인트를 읽어들이도록 만들기".
#include <cmath>
#include <type_traits>
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kDecWaves = 4;        // waves per workgroup, 16 weight rows each at a time
constexpr int kChunk = 512;         // K elements per LDS chunk when A is staged in chunks
constexpr int kAPad = 8;            // bf16 padding per LDS row
constexpr int kFullALds = 67584;    // largest whole-K A stage (bytes): 8 rows of K = 4096 fit
constexpr int kABatch = 4;          // whole-K A stage: chunks whose loads go out together

// LDS bytes of the A stage: whole K, or two chunks.
__host__ __device__ constexpr int dec_lds_bytes(int rows, int K, bool full) {
    return full ? rows * (K + kAPad) * 2 : 2 * rows * (kChunk + kAPad) * 2;
}

// Streams RGS x K for NR weight-row groups (16 rows each) against the tile's
// token rows (at most 4 * TGM, in TGM groups of four).
//   codes[r] / scales[r]: start of this lane's row of row group r;
//   cstride / sstride: bytes to the same lane's row in the next sequential row group;
//   arows: the tile's token rows (bf16, K long), ntok of them valid;
//   epi(j, acc): called after sequential row group j with, per token group, the
//   four tokens' sums over this lane group's K share;
//   setup(): called once the weight ring's first loads are out and before the
//   token rows are staged (it fills arows and synchronises the workgroup), so
//   that its own memory round trips overlap the ring's.
// A step covers 256 elements of K: lane group g takes the 64-element chunk
// 4 i + g; chunks past K (K % 256 == 128) are skipped by the upper lane groups.
struct NoSetup {
    __device__ void operator()() const {}
};

template <int NR, int TGM, int DEPTH, int RGS, bool FULLA, bool SEG, class Epi, class Setup = NoSetup>
__device__ __forceinline__ void dec_stream(const uint16_t* const* __restrict__ arows, int ntok, int K,
                                           const uint8_t* const (&codes)[NR],
                                           const uint8_t* const (&scales)[NR], size_t cstride,
                                           size_t sstride, uint16_t* lds, Epi epi, Setup setup = Setup{}) {
    constexpr int ROWS = 4 * TGM;
    static_assert(FULLA || RGS == 1, "chunked A stages serve one row group");
    static_assert(!SEG || DEPTH % 4 == 0, "scale segments cover four steps");
    // (in a workgroup of several K groups of kDecWaves waves, a group's own threads)
    const int tid = threadIdx.x & (64 * kDecWaves - 1), lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const int ntg = (ntok + 3) >> 2;
    const int nsteps = (K + 255) / 256;                      // K % 128 == 0
    const int nvirt = RGS * nsteps;
    const int LDW = FULLA ? K + kAPad : kChunk + kAPad;      // LDS row stride (elements)
    uint16_t* const buf0 = lds;
    uint16_t* const buf1 = lds + ROWS * LDW;

    // ---- A stage: whole K once, or chunk 0 (the rest double-buffered below)
    constexpr int APT = ROWS * (kChunk / 8) / (64 * kDecWaves);   // 16-byte pieces per thread per chunk
    static_assert(APT * 64 * kDecWaves == ROWS * kChunk / 8, "A staging covers the chunk");
    // loads are unconditional (a piece past the tile's rows or past K reads row 0
    // or the row's last 16 bytes instead; only the stores are conditional): a
    // load under a per-lane condition makes the compiler wait for it at the
    // branch's end, one memory round trip per piece
    auto a_load_to = [&](int ch, u32x4_t (&v)[APT]) {
#pragma unroll
        for (int j = 0; j < APT; ++j) {
            const int piece = tid + j * (64 * kDecWaves);
            const int row = piece >> 6, col = ch * kChunk + (piece & 63) * 8;
            v[j] = *reinterpret_cast<const u32x4_t*>(arows[row < ntok ? row : 0] + (col < K ? col : K - 8));
        }
    };
    auto a_store_from = [&](int ch, const u32x4_t (&v)[APT], uint16_t* b) {
#pragma unroll
        for (int j = 0; j < APT; ++j) {
            const int piece = tid + j * (64 * kDecWaves);
            const int row = piece >> 6, colc = (piece & 63) * 8, col = ch * kChunk + colc;
            if (row < ntok && col < K) *reinterpret_cast<u32x4_t*>(b + row * LDW + (FULLA ? col : colc)) = v[j];
        }
    };
    u32x4_t va[APT];
    auto a_load = [&](int ch) { a_load_to(ch, va); };
    auto a_store = [&](int ch, uint16_t* b) { a_store_from(ch, va, b); };

    // ---- weight prefetch ring.  Loads are unconditional and never selected on:
    // a prefetch past the last step re-reads the last step, and a chunk past K
    // (K % 256 == 128) reads the last chunk of K -- both lines were just fetched,
    // and such data is either unused or multiplied by a zero A fragment.  This
    // lets the compiler keep DEPTH steps of loads in flight across the loop.
    const int last_chunk = K / 64 - 1;
    auto load_codes = [&](int r, int v, u32x4_t& lo, u32x4_t& hi, uint32_t& sc) {
        const int vv = v < nvirt ? v : nvirt - 1;
        const int j = vv / nsteps, step = vv - j * nsteps;
        const int chunk = min(step * 4 + g, last_chunk);
        const u32x4_t* p = reinterpret_cast<const u32x4_t*>(codes[r] + j * cstride + (size_t)chunk * 32);
        lo = p[0];
        hi = p[1];
        if (!SEG) sc = *reinterpret_cast<const uint32_t*>(scales[r] + j * sstride + (size_t)chunk * 4);
    };
    // SEG: scales come in 16-byte segments, one per step (the four lane groups'
    // chunks); lane group m loads the segment of step 4G + m of group G (64
    // adjacent bytes per row), and scale_seg_transpose leaves in lane group g,
    // register m, the 4 scale bytes of its own chunk at step 4G + m.  Needs
    // K % 1024 == 0.
    auto load_seg = [&](int r, int grp) -> u32x4_t {
        int v = grp * 4 + g;
        v = v < nvirt ? v : nvirt - 1;
        const int j = v / nsteps, step = v - j * nsteps;
        return *reinterpret_cast<const u32x4_t*>(scales[r] + j * sstride + (size_t)step * 16);
    };
    // (the first segment is transposed once the token rows are staged, so
    // that nothing before the stage waits for it)
    u32x4_t seg_next[NR], seg_cur[NR];
    if (SEG) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            seg_cur[r] = load_seg(r, 0);
            seg_next[r] = load_seg(r, 1);
        }
    }
    const u32x4_t zero4 = {0u, 0u, 0u, 0u};
    u32x4_t wl[DEPTH][NR], wh[DEPTH][NR];
    uint32_t ws[DEPTH][NR];
#pragma unroll
    for (int u = 0; u < DEPTH; ++u)
#pragma unroll
        for (int r = 0; r < NR; ++r) load_codes(r, u, wl[u][r], wh[u][r], ws[u][r]);
    setup();

    if (FULLA) {
        // the whole K in batches of kABatch chunks: a batch's loads go out
        // together, so a workgroup waits ceil(chunks / kABatch) L2 round trips
        // for its token rows instead of one per chunk
        const int nch = (K + kChunk - 1) / kChunk;
        for (int ch0 = 0; ch0 < nch; ch0 += kABatch) {
            u32x4_t vb[kABatch][APT];
#pragma unroll
            for (int c = 0; c < kABatch; ++c)
                if (ch0 + c < nch) a_load_to(ch0 + c, vb[c]);
#pragma unroll
            for (int c = 0; c < kABatch; ++c)
                if (ch0 + c < nch) a_store_from(ch0 + c, vb[c], buf0);
        }
        __syncthreads();
    } else {
        a_load(0);
        a_store(0, buf0);
    }
    if (SEG) {
#pragma unroll
        for (int r = 0; r < NR; ++r) seg_cur[r] = scale_seg_transpose(seg_cur[r]);
    }

    f32x4_t acc[TGM][NR];
#pragma unroll
    for (int tg = 0; tg < TGM; ++tg)
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[tg][r] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // block-diagonal ownership: A row m = 4 j + t is non-zero only in lane group j
    const bool aown = (n >> 2) == g;
    const int tsub = n & 3;
    constexpr int SPC = kChunk / 256;                        // steps per LDS chunk
    // with scale segments (K % 1024 == 0) and a 4-step ring, every row group ends
    // on the last step of a ring round: one epilogue after the round
    constexpr bool kEpiAfter = SEG && FULLA && DEPTH == 4;
    static_assert(FULLA || DEPTH % SPC == 0, "ring aligned with LDS chunks");

    auto do_step = [&](const int u, const int v) {
        const int j = v / nsteps, step = v - j * nsteps;
        const int ch = step / SPC, si = step % SPC;
        if (!FULLA && si == 0) {
            __syncthreads();                                 // chunk ch staged, chunk ch-1 consumed
            if ((ch + 1) * kChunk < K) a_load(ch + 1);
        }
        const uint16_t* ab = FULLA ? buf0 : ((ch & 1) ? buf1 : buf0);
        u32x4_t cl[NR], chh[NR];
        uint32_t sc[NR];
        if (SEG && u % 4 == 0 && v > 0) {
            // next group of four steps: its segment arrived long ago; fetch the one after
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                seg_cur[r] = scale_seg_transpose(seg_next[r]);
                seg_next[r] = load_seg(r, v / 4 + 1);
            }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            cl[r] = wl[u][r];
            chh[r] = wh[u][r];
            if (SEG) {
                const u32x4_t sgc = seg_cur[r];
                sc[r] = (u % 4 == 0) ? sgc.x : (u % 4 == 1) ? sgc.y : (u % 4 == 2) ? sgc.z : sgc.w;
            } else {
                sc[r] = ws[u][r];
            }
        }
        const bool kvalid = (step * 4 + g) * 64 < K;
        const int kcol = FULLA ? (step * 4 + g) * 64 : (si * 4 + g) * 64;
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
                for (int tg = 0; tg < TGM; ++tg) {
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
                        da = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[1]), b[1],
                                                                     da, 0, 0, 0);
                        f32x4_t db = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, av[2]), b[2], z, 0, 0, 0);
                        db = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[3]), b[3],
                                                                     db, 0, 0, 0);
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[tg][r][q] = fmaf(sb, db[q], fmaf(sa, da[q], acc[tg][r][q]));
                    }
                }
            }
        }
        // refill this ring slot only after its last use: the new load then takes
        // over the same registers and no copies of in-flight data are needed
#pragma unroll
        for (int r = 0; r < NR; ++r) load_codes(r, v + DEPTH, wl[u][r], wh[u][r], ws[u][r]);
        if (!FULLA && si == SPC - 1 && (ch + 1) * kChunk < K) a_store(ch + 1, (ch & 1) ? buf0 : buf1);
        if (!kEpiAfter && step == nsteps - 1) {
            epi(j, acc);
#pragma unroll
            for (int tg = 0; tg < TGM; ++tg)
#pragma unroll
                for (int r = 0; r < NR; ++r) acc[tg][r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    };
    // whole ring rounds without bounds checks, then the tail
    int v0 = 0;
    for (; v0 + DEPTH <= nvirt; v0 += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) do_step(u, v0 + u);
        if (kEpiAfter) {
            const int v = v0 + DEPTH - 1, j = v / nsteps;
            if (v - j * nsteps == nsteps - 1) {
                epi(j, acc);
#pragma unroll
                for (int tg = 0; tg < TGM; ++tg)
#pragma unroll
                    for (int r = 0; r < NR; ++r) acc[tg][r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
#pragma unroll
    for (int u = 0; u < DEPTH; ++u)
        if (v0 + u < nvirt) do_step(u, v0 + u);
}

// Sum of a value over the four lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float lane_group_sum(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// Token-group sum of row group r for token 4 tg + g (every lane takes part in
// the shuffles; lane group g keeps its own token).
template <int TGM, int NR>
__device__ __forceinline__ float dec_result(const f32x4_t (&acc)[TGM][NR], int tg, int r, int g) {
    float out = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float v = lane_group_sum(acc[tg][r][q]);
        if (q == g) out = v;
    }
    return out;
}

struct DecTile {
    int rb, re;
    bool shared;
    size_t ex;
};

// Workgroup -> (table tile, column block); the grid is (max_tiles, column
// blocks).  COL: column blocks vary fastest in dispatch order, so the tiles
// past ntiles (which only return) are dispatched last; else tiles vary
// fastest.  Measured on the 4096 x 1024 layer with 160 local experts, column
// blocks first: T = 8 -2.5 us, T = 128 -12 us, T = 360 -14 us per layer; but
// GEMM1 with two row groups per wave (T = 32, 64) 1-3 us slower and GEMM2 on
// merged tiles (T = 240) 7 us slower, which keep tiles first.
template <bool COL>
__device__ __forceinline__ void dec_block(int& tile, int& cb) {
    if (!COL) {
        tile = blockIdx.x;
        cb = blockIdx.y;
        return;
    }
    const unsigned long long lin = blockIdx.x + (unsigned long long)blockIdx.y * gridDim.x;
    const unsigned long long q = lin / gridDim.y;
    tile = (int)q;
    cb = (int)(lin - q * gridDim.y);
}

__device__ __forceinline__ DecTile dec_tile(const GemmArgs& a, int tile) {
    const int4 tl = a.tiles[tile];
    DecTile t;
    t.rb = tl.y;
    t.re = tl.z;
    t.shared = tl.x == a.L;
    t.ex = t.shared ? 0 : (size_t)tl.x;
    return t;
}

// The tile entry and the live-tile count, loaded together (the grid's first
// dimension is the table's capacity, so the entry is always inside the table);
// false for a workgroup past the count.
__device__ __forceinline__ bool dec_tile_live(const GemmArgs& a, int tile, DecTile& t) {
    const int4 e = a.tiles[tile];
    const int nt = *a.ntiles;
    asm volatile("" ::: "memory");                   // both loads go out before the count is tested
    if (tile >= nt) return false;
    t.rb = e.y;
    t.re = e.z;
    t.shared = e.x == a.L;
    t.ex = t.shared ? 0 : (size_t)e.x;
    return true;
}

// MERGE consecutive table tiles of one group as one workgroup's rows: the tile
// whose index within its group is a multiple of MERGE takes the rows of the
// next MERGE - 1 tiles of the same group too; the others return (false).
template <int MERGE>
__device__ __forceinline__ bool dec_merge_tiles(const GemmArgs& a, DecTile& t, int tile) {
    if (MERGE == 1) return true;
    const int4 t0 = a.tiles[tile];
    if (t0.w % MERGE != 0) return false;
    const int nt = *a.ntiles;
#pragma unroll
    for (int m = 1; m < MERGE; ++m) {
        const int x = tile + m;
        if (x >= nt) break;
        const int4 tn = a.tiles[x];
        if (tn.x != t0.x) break;
        t.re = tn.z;
    }
    return true;
}

// ---------------------------------------------------------------------------
// GEMM1 + SwiGLU: a workgroup = 32 RG SwiGLU columns of a tile of <= 4 TGM
// token rows; in row group j < RG, waves 0,1 stream the gate rows of columns
// [c0 + 32 j, +16) and [c0 + 32 j + 16, +16), waves 2,3 the matching up rows (the
// prefetch ring runs on across row groups); the up results meet the gate
// results in LDS.  grid (max_tiles, F / (32 RG)).
// KSPLIT > 1 (few experts touched, so few workgroups): the workgroup holds
// KSPLIT groups of those four waves, group q streaming K slice q of d (its own
// token-row stage); the groups' sums meet in LDS and are added in slice order.
// A wave's stream, a chain of dependent ring rounds, is then KSPLIT times
// shorter, with no synchronisation beyond the workgroup.
// ---------------------------------------------------------------------------
template <int MODE, int TGM, int DEPTH, bool FULLA, bool SEG, int RG, int KSPLIT = 1>
__global__ __launch_bounds__(64 * kDecWaves * KSPLIT) void dec_gemm1_kernel(GemmArgs a) {
    constexpr int ROWS = 4 * TGM;
    static_assert(KSPLIT == 1 || FULLA, "K slices stage their whole slice");
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    __shared__ const uint16_t* s_arow[KSPLIT][ROWS];
    // up results of row group j at [j & 1]: a gate wave reads group j before it
    // reaches the barrier of group j + 1, so group j + 2 can reuse the buffer
    __shared__ float s_up[2][2][TGM][64];
    __shared__ float s_kred[KSPLIT > 1 ? KSPLIT - 1 : 1][kDecWaves][TGM][64];   // slices 1.. of the sums
    int tile, cb;
    dec_block<RG != 2>(tile, cb);
    DecTile tl;
    if (!dec_tile_live(a, tile, tl)) return;
    const ExpertWeights& W = tl.shared ? a.shared : a.local;
    const int d = a.d, F = a.F;
    const int tid = threadIdx.x & (64 * kDecWaves - 1), lane = tid & 63, wave = tid >> 6;
    const int kq = threadIdx.x / (64 * kDecWaves);   // K slice of this wave's group
    const int kk = d / KSPLIT, kb = kq * kk;
    const int half = wave & 1;                       // which 16 columns
    const bool is_up = wave >= 2;
    const int col0 = cb * (32 * RG) + half * 16;
    const int n = lane & 15, g = lane >> 4;
    const int ntok = tl.re - tl.rb;
    const uint16_t* act_in = MODE == 0 ? a.hidden : a.hq;
    // the pair of tile row tid % ROWS (the tile's last row past its end; any
    // valid entry for the shared expert's rows, which need none), loaded by
    // every thread before the weight ring goes out and used after it (setup)
    const int pv = a.perm[min(min(tl.rb + (tid % ROWS), tl.re - 1), a.T * a.topk - 1)];
    asm volatile("" ::: "memory");                   // issued here, not sunk to its use
    auto setup = [&]() {
        if (tid < ROWS) {
            const int row = tl.rb + tid;
            int t = 0;
            if (row < tl.re) t = tl.shared ? row - a.T * a.topk : pv / a.topk;
            s_arow[kq][tid] = act_in + (size_t)t * d + kb;
        }
        __syncthreads();
    };
    const uint8_t* w13 = W.w13 + tl.ex * (size_t)(2 * F) * (d / 2);
    const uint8_t* w13s = W.w13_s + tl.ex * (size_t)(2 * F) * (d / 16);
    const int wrow = (is_up ? F : 0) + col0 + n;
    const uint8_t* const codes[1] = {w13 + (size_t)wrow * (d / 2) + kb / 2};
    const uint8_t* const scales[1] = {w13s + (size_t)wrow * (d / 16) + kb / 16};
    const float g13 = W.g13[tl.ex] * a.a1g;          // weight global x activation global
    auto epi = [&](int j, const f32x4_t (&acc)[TGM][1]) {
        const int col = col0 + 32 * j + n;
        float v[TGM];
#pragma unroll
        for (int tg = 0; tg < TGM; ++tg) v[tg] = dec_result<TGM, 1>(acc, tg, 0, g);
        if (KSPLIT > 1) {
            if (kq > 0) {
#pragma unroll
                for (int tg = 0; tg < TGM; ++tg) s_kred[kq > 0 ? kq - 1 : 0][wave][tg][lane] = v[tg];
            }
            __syncthreads();
            if (kq == 0) {
#pragma unroll
                for (int q = 1; q < KSPLIT; ++q)
#pragma unroll
                    for (int tg = 0; tg < TGM; ++tg) v[tg] += s_kred[q - 1][wave][tg][lane];
            }
        }
#pragma unroll
        for (int tg = 0; tg < TGM; ++tg) v[tg] *= g13;
        if (is_up && kq == 0) {
#pragma unroll
            for (int tg = 0; tg < TGM; ++tg) s_up[j & 1][half][tg][lane] = v[tg];
        }
        __syncthreads();
        if (!is_up && kq == 0) {
#pragma unroll
            for (int tg = 0; tg < TGM; ++tg) {
                const float gt = v[tg], up = s_up[j & 1][half][tg][lane];
                float av = gt / (1.0f + expf(-gt)) * up;
                if (MODE == 1) {
                    // NVFP4 quantize-dequantize over the 16 columns of this lane group
                    float m = fabsf(av);
                    m = fmaxf(m, __shfl_xor(m, 1, 64));
                    m = fmaxf(m, __shfl_xor(m, 2, 64));
                    m = fmaxf(m, __shfl_xor(m, 4, 64));
                    m = fmaxf(m, __shfl_xor(m, 8, 64));
                    av = nvfp4_fake_quant(av, m, a.a2g);
                }
                const int r = tl.rb + tg * 4 + g;
                if (r < tl.re) a.act[(size_t)r * F + col] = (uint16_t)f32_to_bf16_rne(av);
            }
        }
    };
    const size_t cstride = (size_t)32 * (d / 2), sstride = (size_t)32 * (d / 16);
    uint16_t* const stage = lds + (size_t)kq * (dec_lds_bytes(ROWS, kk, FULLA) / 2);
    dec_stream<1, TGM, DEPTH, RG, FULLA, SEG>(s_arow[kq], ntok, kk, codes, scales, cstride, sstride, stage, epi,
                                              setup);
}

// ---------------------------------------------------------------------------
// GEMM2: a wave walks RGS groups of 16 output columns (16 rows of w2 each); the
// workgroup covers 16 * kDecWaves * RGS columns of the rows of MERGE table
// tiles (at most 4 TGM rows).  grid (max_tiles, d / that).
// ---------------------------------------------------------------------------
template <int TGM, int DEPTH, int RGS, bool FULLA, bool SEG, int MERGE>
__global__ __launch_bounds__(64 * kDecWaves) void dec_gemm2_kernel(GemmArgs a) {
    constexpr int ROWS = 4 * TGM;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    __shared__ const uint16_t* s_arow[ROWS];
    int tile, cb;
    dec_block<MERGE == 1>(tile, cb);
    if (tile >= *a.ntiles) return;
    DecTile tl = dec_tile(a, tile);
    if (!dec_merge_tiles<MERGE>(a, tl, tile)) return;
    const ExpertWeights& W = tl.shared ? a.shared : a.local;
    const int d = a.d, F = a.F;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cbase = cb * (16 * kDecWaves * RGS) + wave * 16;   // row group j: cbase + 64 j
    const int n = lane & 15, g = lane >> 4;
    const int ntok = tl.re - tl.rb;
    if (tid < ROWS) s_arow[tid] = a.act + (size_t)(tl.rb + (tid < ntok ? tid : 0)) * F;
    __syncthreads();
    const uint8_t* w2 = W.w2 + tl.ex * (size_t)d * (F / 2);
    const uint8_t* w2s = W.w2_s + tl.ex * (size_t)d * (F / 16);
    const uint8_t* const codes[1] = {w2 + (size_t)(cbase + n) * (F / 2)};
    const uint8_t* const scales[1] = {w2s + (size_t)(cbase + n) * (F / 16)};
    const size_t cstride = (size_t)(16 * kDecWaves) * (F / 2), sstride = (size_t)(16 * kDecWaves) * (F / 16);
    const float g2 = W.g2[tl.ex] * a.a2g;            // weight global x activation global
    auto epi = [&](int j, const f32x4_t (&acc)[TGM][1]) {
        const int col = cbase + j * (16 * kDecWaves) + n;
#pragma unroll
        for (int tg = 0; tg < TGM; ++tg) {
            const float y = dec_result<TGM, 1>(acc, tg, 0, g);
            const int r = tl.rb + tg * 4 + g;
            if (r < tl.re) a.Y[(size_t)r * d + col] = (uint16_t)f32_to_bf16_rne(y * g2);
        }
    };
    dec_stream<1, TGM, DEPTH, RGS, FULLA, SEG>(s_arow, ntok, F, codes, scales, cstride, sstride, lds, epi);
}

// ---------------------------------------------------------------------------
// Small-batch layer in one persistent launch (T <= 16 tokens, d, F <= 4096).
//
// At a few tokens the layer's own work is small (T = 1 on the 160-expert shard
// streams ~5 experts, 35 MB) and separate launches for routing, permutation,
// the two GEMMs and the combine cost more than the work.  One workgroup per
// CU runs every step, with three grid-wide barriers:
//   1. router logits in fp64 (exact sums of the bf16 x bf16 products, in a
//      fixed order; experts spread over the workgroups) and, in W4A4, the
//      NVFP4 quantize-dequantize of the token rows;           -- barrier --
//   2. every workgroup reads the logits and takes the same top-k selection
//      (descending logit, equal logits: lower id), softmax over the k, shard
//      filter and the pair order (local expert, token) into its own LDS, so no
//      table crosses workgroups;
//   3. GEMM1 + SwiGLU in units of 32 SwiGLU columns of one expert (the
//      weight-streaming kernel's block-diagonal MFMA, the expert's tokens as up
//      to four token groups);                                  -- barrier --
//   4. GEMM2 in units of 256 output columns;                   -- barrier --
//   5. the weighted combine (slot order, then the shared row), as combine_kernel.
// The barriers need every workgroup resident at once: the launch has one
// workgroup per CU and ~150 KB of LDS each, so no two share a CU, and the
// preceding stream work has finished.  A barrier's wait is bounded: past
// kMicroSpin polls the workgroup sets the error word and goes on (the output
// is then wrong, but the kernel ends).  The counter and the error word are
// zeroed by micro_reset_kernel, enqueued just before.
// ---------------------------------------------------------------------------
constexpr int kMicroMaxT = 16;
constexpr int kMicroMaxDim = 4096;          // d and F: the 16-row whole-K token stage fits the LDS
                                            // (also the T x d token rows of the logits phase)
constexpr int kMicroMaxL = 1024;
constexpr unsigned kMicroSpin = 1u << 22;   // polls (each after a ~60 ns sleep) before giving up

__global__ void micro_reset_kernel(unsigned* bar) {
    if (threadIdx.x < 2) bar[threadIdx.x] = 0u;
}

// Arrive at barrier number `n` (1, 2, 3) of the launch and wait for all `nwg`
// workgroups: release this workgroup's writes device-wide, count, wait
// (bounded), acquire the others'.  The wait polls with relaxed device-scope
// loads (coherent, and no cache invalidation per poll: an acquire in the loop
// would invalidate the caches on every poll while other workgroups still
// stream); the acquire fence comes once, after the wait.
__device__ __forceinline__ void micro_grid_barrier(unsigned* bar, unsigned n, unsigned nwg) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned target = n * nwg;
        unsigned polls = 0;
        while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(2);
            if (++polls > kMicroSpin) {
                __hip_atomic_fetch_or(bar + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

template <bool SEG1, bool SEG2>
__global__ __launch_bounds__(64 * kDecWaves) void micro_layer_kernel(MicroArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];   // dec_stream's token stage
    __shared__ uint32_t s_mask[kMicroMaxL];          // per local expert: its tokens (bit t)
    __shared__ int s_off[kMicroMaxL + 1];            // first pair row of each local expert
    __shared__ int s_list[kMicroMaxL + 1];           // touched local experts, ascending
    __shared__ int s_nlist;
    __shared__ float s_w[kMicroMaxT * 32];           // routing weight of pair t k + j
    __shared__ int s_inv[kMicroMaxT * 32];           // its row (-1: outside the shard)
    __shared__ const uint16_t* s_arow[16];
    __shared__ float s_up[2][2][4][64];
    __shared__ double s_red[kDecWaves][kMicroMaxT];
    __shared__ double s_top[kMicroMaxT][32];         // selected logits of each token, slot order
    __shared__ int s_topid[kMicroMaxT][32];
    __shared__ int s_wsum[kDecWaves];

    const int T = a.T, d = a.d, F = a.F, E = a.E, k = a.topk, L = a.L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const unsigned wg = blockIdx.x, nwg = gridDim.x;
    const uint16_t* act_in = a.mode == 0 ? a.X : a.hq;

    // ---- 1. logits (fp64, fixed order) and the W4A4 token rows ----
    // the T token rows go to LDS once (the token-stage region is free until the
    // GEMMs); a thread then takes 8 consecutive k of an expert's gate row per
    // 16-byte load, pieces tid, tid + 256, ... in order
    if ((int)wg < E) {
        const int pieces = T * (d / 8);
        for (int q0 = 0; q0 < pieces; q0 += 8 * 64 * kDecWaves) {
            u32x4_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int q = q0 + j * 64 * kDecWaves + tid;
                v[j] = *reinterpret_cast<const u32x4_t*>(a.X + (size_t)(q < pieces ? q : pieces - 1) * 8);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int q = q0 + j * 64 * kDecWaves + tid;
                if (q < pieces) *reinterpret_cast<u32x4_t*>(lds + (size_t)q * 8) = v[j];
            }
        }
        __syncthreads();
    }
    for (int e = (int)wg; e < E; e += (int)nwg) {
        double acc[kMicroMaxT];
#pragma unroll
        for (int t = 0; t < kMicroMaxT; ++t) acc[t] = 0.0;
        const uint16_t* g = a.G + (size_t)e * d;
        for (int q = tid; q < d / 8; q += 64 * kDecWaves) {
            const u32x4_t gv4 = *reinterpret_cast<const u32x4_t*>(g + q * 8);
            const uint32_t gw[4] = {gv4.x, gv4.y, gv4.z, gv4.w};
            double gv[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gv[2 * i] = (double)bf16_bits_to_f32(gw[i] & 0xFFFFu);
                gv[2 * i + 1] = (double)bf16_bits_to_f32(gw[i] >> 16);
            }
#pragma unroll
            for (int t = 0; t < kMicroMaxT; ++t) {
                if (t < T) {
                    const u32x4_t xv4 = *reinterpret_cast<const u32x4_t*>(lds + (size_t)t * d + q * 8);
                    const uint32_t xw[4] = {xv4.x, xv4.y, xv4.z, xv4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[t] = fma((double)bf16_bits_to_f32(xw[i] & 0xFFFFu), gv[2 * i], acc[t]);
                        acc[t] = fma((double)bf16_bits_to_f32(xw[i] >> 16), gv[2 * i + 1], acc[t]);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < kMicroMaxT; ++t) {
            if (t < T) {
                const double v = wave_sum_f64(acc[t]);
                if (lane == 0) s_red[wave][t] = v;
            }
        }
        __syncthreads();
        if (tid < T) {
            double v = s_red[0][tid];
#pragma unroll
            for (int w = 1; w < kDecWaves; ++w) v += s_red[w][tid];
            a.logits[(size_t)tid * E + e] = v;
        }
        __syncthreads();
    }
    if (a.mode == 1) {
        const int nb = T * (d / kBlock);
        for (int b = (int)(wg * 64 * kDecWaves) + tid; b < nb; b += (int)(nwg * 64 * kDecWaves)) {
            const uint16_t* x = a.X + (size_t)b * kBlock;
            float f[16];
            float bmax = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                f[i] = bf16_bits_to_f32(x[i]);
                bmax = fmaxf(bmax, fabsf(f[i]));
            }
            uint32_t o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                o[i] = pack_hi16(nvfp4_fake_quant(f[2 * i], bmax, a.a1g), nvfp4_fake_quant(f[2 * i + 1], bmax, a.a1g));
            u32x4_t* dst = reinterpret_cast<u32x4_t*>(a.hq + (size_t)b * kBlock);
            dst[0] = u32x4_t{o[0], o[1], o[2], o[3]};
            dst[1] = u32x4_t{o[4], o[5], o[6], o[7]};
        }
    }
    micro_grid_barrier(a.bar, 1, nwg);

    // ---- 2. selection, shard filter and pair order (every workgroup alike) ----
    for (int l = tid; l < L; l += 64 * kDecWaves) s_mask[l] = 0u;
    __syncthreads();
    for (int t = wave; t < T; t += kDecWaves) {
        constexpr int EPL = kMaxExpertsMicro / 64;
        double v[EPL];
#pragma unroll
        for (int sl = 0; sl < EPL; ++sl) {
            const int e = lane + 64 * sl;
            v[sl] = a.logits[(size_t)t * E + (e < E ? e : E - 1)];   // unconditional (slots past E are never taken)
        }
        bool taken[EPL];
#pragma unroll
        for (int sl = 0; sl < EPL; ++sl) taken[sl] = lane + 64 * sl >= E;
        for (int r = 0; r < k; ++r) {
            double bv = -INFINITY;
            int bi = 0x7FFFFFFF;
#pragma unroll
            for (int sl = 0; sl < EPL; ++sl)
                if (!taken[sl] && (v[sl] > bv || (v[sl] == bv && lane + 64 * sl < bi))) {
                    bv = v[sl];
                    bi = lane + 64 * sl;
                }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const double ov = __shfl_xor(bv, o, 64);
                const int oi = __shfl_xor(bi, o, 64);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
#pragma unroll
            for (int sl = 0; sl < EPL; ++sl)
                if (lane + 64 * sl == bi) taken[sl] = true;
            if (lane == 0) {
                s_top[t][r] = bv;
                s_topid[t][r] = bi;
            }
        }
        __builtin_amdgcn_wave_barrier();
        if (lane == 0) {
            double zs = 0.0;
            for (int j = 0; j < k; ++j) zs += exp(s_top[t][j] - s_top[t][0]);
            for (int j = 0; j < k; ++j) {
                s_w[t * k + j] = (float)(exp(s_top[t][j] - s_top[t][0]) / zs);
                const int lam = s_topid[t][j] - a.offset;
                s_inv[t * k + j] = (lam >= 0 && lam < L) ? lam : -1;     // local id for now
                if (lam >= 0 && lam < L) atomicOr(&s_mask[lam], 1u << t);
            }
        }
    }
    __syncthreads();
    // exclusive scans over the local experts of (pair count, touched), in order
    {
        constexpr int PER = kMicroMaxL / (64 * kDecWaves);
        int c[PER], u[PER], cs = 0, us = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int l = tid * PER + i;
            c[i] = l < L ? __popc(s_mask[l]) : 0;
            u[i] = c[i] > 0;
            cs += c[i];
            us += u[i];
        }
        // wave-inclusive scans of (cs, us) packed in one int (counts < 2^15 each)
        int pk = cs | (us << 16), inc = pk;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        if (lane == 63) s_wsum[wave] = inc;
        __syncthreads();
        int base = 0;
        for (int w = 0; w < wave; ++w) base += s_wsum[w];
        int ex = base + inc - pk;
        int pc = ex & 0xFFFF, pu = ex >> 16;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int l = tid * PER + i;
            if (l < L) {
                s_off[l] = pc;
                if (u[i]) s_list[pu] = l;
            }
            pc += c[i];
            pu += u[i];
        }
        if (tid == 64 * kDecWaves - 1) {
            s_off[L] = pc;
            s_nlist = pu;
        }
    }
    __syncthreads();
    // pair rows for the combine: local pair (t, j) -> s_off[lam] + rank of t
    for (int p = tid; p < T * k; p += 64 * kDecWaves) {
        const int lam = s_inv[p];
        if (lam >= 0) {
            const int t = p / k;
            s_inv[p] = s_off[lam] + __popc(s_mask[lam] & ((1u << t) - 1u));
        }
    }
    __syncthreads();
    const int nlist = s_nlist;
    const int ngroups = nlist + (a.has_shared ? 1 : 0);
    const int shared_row0 = T * k;

    // the unit's token rows: group i < nlist is local expert s_list[i], else the shared expert
    auto group_rows = [&](int i, const uint16_t* base, int stride, bool pair_rows) -> int {
        int ntok;
        if (i < nlist) {
            const int lam = s_list[i];
            const uint32_t m = s_mask[lam];
            ntok = __popc(m);
            if (tid < 16 && tid < ntok) {
                // tid-th set bit of m
                uint32_t mm = m;
                for (int q = 0; q < tid; ++q) mm &= mm - 1u;
                const int t = __ffs(mm) - 1;
                s_arow[tid] = base + (size_t)(pair_rows ? s_off[lam] + tid : t) * stride;
            }
        } else {
            ntok = T;
            if (tid < T) s_arow[tid] = base + (size_t)(pair_rows ? shared_row0 + tid : tid) * stride;
        }
        __syncthreads();
        return ntok;
    };
    auto group_weights = [&](int i, const ExpertWeights*& W, size_t& ex) {
        const bool sh = i >= nlist;
        W = sh ? &a.shared : &a.local;
        ex = sh ? 0 : (size_t)s_list[i];
    };

    // ---- 3. GEMM1 + SwiGLU: unit = (group, 32 SwiGLU columns) ----
    {
        const int half = wave & 1;
        const bool is_up = wave >= 2;
        const int n = lane & 15, g = lane >> 4;
        const int ncg = F / 32;
        for (int u = (int)wg; u < ngroups * ncg; u += (int)nwg) {
            const int i = u / ncg, cg = u - i * ncg;
            const ExpertWeights* W;
            size_t ex;
            group_weights(i, W, ex);
            const int ntok = group_rows(i, act_in, d, false);
            const int row0 = i < nlist ? s_off[s_list[i]] : shared_row0;
            const int col0 = cg * 32 + half * 16;
            const uint8_t* w13 = W->w13 + ex * (size_t)(2 * F) * (d / 2);
            const uint8_t* w13s = W->w13_s + ex * (size_t)(2 * F) * (d / 16);
            const int wrow = (is_up ? F : 0) + col0 + n;
            const uint8_t* const codes[1] = {w13 + (size_t)wrow * (d / 2)};
            const uint8_t* const scales[1] = {w13s + (size_t)wrow * (d / 16)};
            const float g13 = W->g13[ex] * a.a1g;
            auto epi = [&](int j, const f32x4_t (&acc)[4][1]) {
                const int col = col0 + n;
                float v[4];
#pragma unroll
                for (int tg = 0; tg < 4; ++tg) v[tg] = dec_result<4, 1>(acc, tg, 0, g) * g13;
                if (is_up) {
#pragma unroll
                    for (int tg = 0; tg < 4; ++tg) s_up[j & 1][half][tg][lane] = v[tg];
                }
                __syncthreads();
                if (!is_up) {
#pragma unroll
                    for (int tg = 0; tg < 4; ++tg) {
                        const float gt = v[tg], up = s_up[j & 1][half][tg][lane];
                        float av = gt / (1.0f + expf(-gt)) * up;
                        if (a.mode == 1) {
                            float m = fabsf(av);
                            m = fmaxf(m, __shfl_xor(m, 1, 64));
                            m = fmaxf(m, __shfl_xor(m, 2, 64));
                            m = fmaxf(m, __shfl_xor(m, 4, 64));
                            m = fmaxf(m, __shfl_xor(m, 8, 64));
                            av = nvfp4_fake_quant(av, m, a.a2g);
                        }
                        const int r = tg * 4 + g;
                        if (r < ntok) a.act[(size_t)(row0 + r) * F + col] = (uint16_t)f32_to_bf16_rne(av);
                    }
                }
            };
            dec_stream<1, 4, 4, 1, true, SEG1>(s_arow, ntok, d, codes, scales, (size_t)32 * (d / 2),
                                              (size_t)32 * (d / 16), lds, epi);
            __syncthreads();                         // s_arow, s_up and the token stage are free again
        }
    }
    micro_grid_barrier(a.bar, 2, nwg);

    // ---- 4. GEMM2: unit = (group, 256 output columns; four row groups per wave) ----
    {
        const int n = lane & 15, g = lane >> 4;
        const int ncb = d / 256;
        for (int u = (int)wg; u < ngroups * ncb; u += (int)nwg) {
            const int i = u / ncb, cb = u - i * ncb;
            const ExpertWeights* W;
            size_t ex;
            group_weights(i, W, ex);
            const int ntok = group_rows(i, a.act, F, true);
            const int row0 = i < nlist ? s_off[s_list[i]] : shared_row0;
            const int cbase = cb * 256 + wave * 16;
            const uint8_t* w2 = W->w2 + ex * (size_t)d * (F / 2);
            const uint8_t* w2s = W->w2_s + ex * (size_t)d * (F / 16);
            const uint8_t* const codes[1] = {w2 + (size_t)(cbase + n) * (F / 2)};
            const uint8_t* const scales[1] = {w2s + (size_t)(cbase + n) * (F / 16)};
            const float g2 = W->g2[ex] * a.a2g;
            auto epi = [&](int j, const f32x4_t (&acc)[4][1]) {
                const int col = cbase + j * 64 + n;
#pragma unroll
                for (int tg = 0; tg < 4; ++tg) {
                    const float y = dec_result<4, 1>(acc, tg, 0, g);
                    const int r = tg * 4 + g;
                    if (r < ntok) a.Y[(size_t)(row0 + r) * d + col] = (uint16_t)f32_to_bf16_rne(y * g2);
                }
            };
            dec_stream<1, 4, 4, 4, true, SEG2>(s_arow, ntok, F, codes, scales, (size_t)64 * (F / 2),
                                              (size_t)64 * (F / 16), lds, epi);
            __syncthreads();
        }
    }
    micro_grid_barrier(a.bar, 3, nwg);

    // ---- 5. combine: slot order, then the shared row ----
    const int per_row = d / 8;
    for (int idx = (int)(wg * 64 * kDecWaves) + tid; idx < T * per_row; idx += (int)(nwg * 64 * kDecWaves)) {
        const int t = idx / per_row, c0 = (idx - t * per_row) * 8;
        float sacc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const int row = s_inv[t * k + j];
            if (row < 0) continue;
            const float wj = s_w[t * k + j];
            const u32x4_t y = *reinterpret_cast<const u32x4_t*>(a.Y + (size_t)row * d + c0);
            const uint32_t yw[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sacc[2 * e] = fmaf(wj, bf16_bits_to_f32(yw[e] & 0xFFFFu), sacc[2 * e]);
                sacc[2 * e + 1] = fmaf(wj, bf16_bits_to_f32(yw[e] >> 16), sacc[2 * e + 1]);
            }
        }
        if (a.has_shared) {
            const u32x4_t y = *reinterpret_cast<const u32x4_t*>(a.Y + (size_t)(shared_row0 + t) * d + c0);
            const uint32_t yw[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sacc[2 * e] = fmaf(1.0f, bf16_bits_to_f32(yw[e] & 0xFFFFu), sacc[2 * e]);
                sacc[2 * e + 1] = fmaf(1.0f, bf16_bits_to_f32(yw[e] >> 16), sacc[2 * e + 1]);
            }
        }
        u32x4_t o;
        o.x = f32x2_to_bf16x2(sacc[0], sacc[1]);
        o.y = f32x2_to_bf16x2(sacc[2], sacc[3]);
        o.z = f32x2_to_bf16x2(sacc[4], sacc[5]);
        o.w = f32x2_to_bf16x2(sacc[6], sacc[7]);
        *reinterpret_cast<u32x4_t*>(a.out + (size_t)t * d + c0) = o;
    }
}

bool micro_ok(int T, int d, int F, int E, int topk, int L) {
    return T >= 1 && T <= kMicroMaxT && d <= kMicroMaxDim && F <= kMicroMaxDim && d % 256 == 0 && F % 32 == 0 &&
           E <= kMaxExpertsMicro && topk <= 32 && L <= kMicroMaxL;
}

int micro_lds_bytes(int d, int F) { return dec_lds_bytes(16, d > F ? d : F, true); }

hipError_t launch_micro(const MicroArgs& a, int ncu, hipStream_t s) {
    hipLaunchKernelGGL(micro_reset_kernel, dim3(1), dim3(64), 0, s, a.bar);
    const int lds = micro_lds_bytes(a.d, a.F);
    const bool seg1 = a.d % 1024 == 0, seg2 = a.F % 1024 == 0;
    auto go = [&](auto kern) {
        if (allow_dynamic_lds<decltype(kern)::value>(lds) != hipSuccess) return;
        hipLaunchKernelGGL(decltype(kern)::value, dim3(ncu), dim3(64 * kDecWaves), lds, s, a);
    };
    if (seg1 && seg2) go(std::integral_constant<decltype(&micro_layer_kernel<true, true>), &micro_layer_kernel<true, true>>{});
    else if (seg1) go(std::integral_constant<decltype(&micro_layer_kernel<true, false>), &micro_layer_kernel<true, false>>{});
    else if (seg2) go(std::integral_constant<decltype(&micro_layer_kernel<false, true>), &micro_layer_kernel<false, true>>{});
    else go(std::integral_constant<decltype(&micro_layer_kernel<false, false>), &micro_layer_kernel<false, false>>{});
    return hipGetLastError();
}

// Tile height of the decode path: 4 token rows (one group) while experts expect
// at most ~6 tokens, 8 rows (two groups) up to ~12, else 16 rows (four groups;
// only when the decode path is forced beyond that).  The 4- and 8-row tiles
// stage the whole K of their token rows in LDS (up to K = 4096 for 8 rows).
// Measured on the 4096 x 1024 layer with 160 local experts: 4-row tiles beat
// 8-row tiles up to T k / E ~ 6 (T = 128: 316 against 344 us), although an
// expert with more than 4 pairs streams its weights once per tile; beyond,
// 8-row tiles win (T = 288: 478 against 485 us); both beat 16-row tiles by
// 20-30% (T = 128: 457 us).
int dec_rows(int T, int topk, int E) {
    const long long p = (long long)T * topk;
    return p <= 6LL * E ? 4 : (p <= 12LL * E ? 8 : 16);
}

// Launch of a decode kernel with `lds` bytes of dynamic LDS (above 64 KB the
// kernel's limit is raised first; a failure is left for hipGetLastError).
template <auto Kern, int GROUPS = 1>
static void launch_dec(dim3 grid, int lds, hipStream_t s, const GemmArgs& a) {
    if (allow_dynamic_lds<Kern>(lds) != hipSuccess) return;
    hipLaunchKernelGGL(Kern, grid, dim3(64 * kDecWaves * GROUPS), lds, s, a);
}

constexpr int kG1Depth = 4;         // prefetch ring depth of the small-tile GEMM1
// GEMM1 in two K slices per workgroup up to this many expected workgroups.
// Measured on the 4096 x 1024 layer with 160 local experts (GEMM1 stage time,
// one slice / two / four): T = 1 (160 workgroups) 15.3 / 13.8 / 16.2 us; T = 2
// (285) 19.2 / 19.5 / 26.3; T = 4 (525) 24.6 / 28.8 / 37.9; T = 8 40.1 / 44.6 /
// 60.5.  Four slices (1024-thread workgroups) never paid.
constexpr double kG1Split2Wgs = 200.0;

// Expected number of expert tiles (touched local experts, plus the shared
// expert) under uniform routing: L (1 - (1 - k/E)^T) + shared.
static double expected_tiles(const GemmArgs& a) {
    const double miss = std::pow(1.0 - (double)a.topk / a.E, (double)a.T);
    return a.L * (1.0 - miss) + (a.shared.w13 ? 1.0 : 0.0);
}

// Row groups a wave walks back to back: long streams amortise the prefetch
// ring's fill when many experts keep the chip busy; with few experts, fewer
// row groups per wave give the grid more workgroups.  Measured on the
// 4096 x 1024 layer with 160 local experts (expected tiles in brackets): GEMM1
// at T = 1..16 (5..55) runs 1.4-2.4x faster with one row group than with four;
// at T = 24..80 (75..140) two row groups are up to 15% faster than four
// (T = 72, 80: 137, 139 against 142 us; T = 64 within 1.5%); from T = 96 (147)
// on four are faster (T = 96: 144 against 150 us; T = 128: 175 against 182).
static int g1_row_groups(const GemmArgs& a) {
    const double t = expected_tiles(a);
    return t <= 64.0 ? 1 : (t <= 141.0 ? 2 : 4);
}
static int g2_row_groups(const GemmArgs& a) {
    const double t = expected_tiles(a);
    return t <= 8.0 ? 1 : (t <= 32.0 ? 2 : 4);
}

template <int MODE, int TGM, int DEPTH, int RG>
static void launch_g1(const GemmArgs& a, hipStream_t s) {
    const int full = dec_lds_bytes(4 * TGM, a.d, true);
    if (full <= kFullALds && a.F % (32 * RG) == 0) {
        const dim3 grid(a.max_tiles, a.F / (32 * RG));
        if (DEPTH % 4 == 0 && a.d % 1024 == 0)
            launch_dec<dec_gemm1_kernel<MODE, TGM, DEPTH, true, (DEPTH % 4 == 0), RG>>(grid, full, s, a);
        else
            launch_dec<dec_gemm1_kernel<MODE, TGM, DEPTH, true, false, RG>>(grid, full, s, a);
    } else if (full <= kFullALds) {
        launch_dec<dec_gemm1_kernel<MODE, TGM, DEPTH, true, false, 1>>(dim3(a.max_tiles, a.F / 32), full, s, a);
    } else {
        launch_dec<dec_gemm1_kernel<MODE, TGM, 2, false, false, 1>>(dim3(a.max_tiles, a.F / 32),
                                                                     dec_lds_bytes(4 * TGM, a.d, false), s, a);
    }
}

template <int MODE, int TGM, int DEPTH>
static void launch_g1_rg(const GemmArgs& a, hipStream_t s) {
    switch (g1_row_groups(a)) {
        case 1: launch_g1<MODE, TGM, DEPTH, 1>(a, s); break;
        case 2: launch_g1<MODE, TGM, DEPTH, 2>(a, s); break;
        default: launch_g1<MODE, TGM, DEPTH, 4>(a, s); break;
    }
}

// K slices of GEMM1 within a workgroup (4-row tiles, one row group per wave):
// when the grid's expected workgroups are few, KSPLIT groups of four waves share
// each workgroup's columns, each streaming 1/KSPLIT of d.
static int g1_kslices(const GemmArgs& a) {
    if (dec_rows(a.T, a.topk, a.E) != 4 || g1_row_groups(a) != 1 || a.F % 32 != 0) return 1;
    const double wgs = expected_tiles(a) * (a.F / 32);
    if (wgs <= kG1Split2Wgs && a.d % 2048 == 0 && 2 * dec_lds_bytes(4, a.d / 2, true) <= kFullALds) return 2;
    return 1;
}

template <int MODE, int KSPLIT>
static void launch_g1_ksplit(const GemmArgs& a, hipStream_t s) {
    const int lds = KSPLIT * dec_lds_bytes(4, a.d / KSPLIT, true);
    launch_dec<dec_gemm1_kernel<MODE, 1, kG1Depth, true, true, 1, KSPLIT>, KSPLIT>(dim3(a.max_tiles, a.F / 32), lds,
                                                                                   s, a);
}

hipError_t launch_dec_gemm1(const GemmArgs& a, hipStream_t s) {
    const int rows = dec_rows(a.T, a.topk, a.E);
    if (g1_kslices(a) == 2) a.mode == 0 ? launch_g1_ksplit<0, 2>(a, s) : launch_g1_ksplit<1, 2>(a, s);
    else if (rows == 4) a.mode == 0 ? launch_g1_rg<0, 1, kG1Depth>(a, s) : launch_g1_rg<1, 1, kG1Depth>(a, s);
    else if (rows == 8) a.mode == 0 ? launch_g1_rg<0, 2, kG1Depth>(a, s) : launch_g1_rg<1, 2, kG1Depth>(a, s);
    else a.mode == 0 ? launch_g1_rg<0, 4, 2>(a, s) : launch_g1_rg<1, 4, 2>(a, s);
    return hipGetLastError();
}

// TGM: token groups of the kernel (4 TGM rows); the table's tiles are 4 TGM /
// MERGE rows high.
template <int TGM, int DEPTH, int RG, int MERGE>
static void launch_g2(const GemmArgs& a, hipStream_t s) {
    const int full = dec_lds_bytes(4 * TGM, a.F, true);
    constexpr bool kSeg = DEPTH % 4 == 0;
    if (full <= kFullALds) {
        const bool seg = kSeg && a.F % 1024 == 0;
        if (a.d % (16 * kDecWaves * RG) == 0) {
            const dim3 grid(a.max_tiles, a.d / (16 * kDecWaves * RG));
            if (seg) launch_dec<dec_gemm2_kernel<TGM, DEPTH, RG, true, kSeg, MERGE>>(grid, full, s, a);
            else launch_dec<dec_gemm2_kernel<TGM, DEPTH, RG, true, false, MERGE>>(grid, full, s, a);
        } else {
            const dim3 grid(a.max_tiles, a.d / (16 * kDecWaves * 2));
            if (seg) launch_dec<dec_gemm2_kernel<TGM, DEPTH, 2, true, kSeg, MERGE>>(grid, full, s, a);
            else launch_dec<dec_gemm2_kernel<TGM, DEPTH, 2, true, false, MERGE>>(grid, full, s, a);
        }
    } else {
        launch_dec<dec_gemm2_kernel<TGM, 2, 1, false, false, MERGE>>(dim3(a.max_tiles, a.d / (16 * kDecWaves)),
                                                                      dec_lds_bytes(4 * TGM, a.F, false), s, a);
    }
}

template <int TGM, int DEPTH, int MERGE>
static void launch_g2_rg(const GemmArgs& a, hipStream_t s) {
    switch (g2_row_groups(a)) {
        case 1: launch_g2<TGM, DEPTH, 1, MERGE>(a, s); break;
        case 2: launch_g2<TGM, DEPTH, 2, MERGE>(a, s); break;
        default: launch_g2<TGM, DEPTH, 4, MERGE>(a, s); break;
    }
}

// The down projection takes 8-row tiles (two 4-row table tiles of one group)
// where the table has 4-row tiles and experts expect more than kG2MergePairs
// pairs.  Measured on the 4096 x 1024 layer with 160 local experts: GEMM2 at
// T = 240 (6 pairs per expert) 132 -> 115 us; at T = 192 equal; at T <= 160
// 7-13 us slower (the second row group of an 8-row tile is mostly empty, and
// half the workgroups only return).  Merging 8-row table tiles into 16-row
// tiles is slower at every T tried (256-320).
constexpr double kG2MergePairs = 5.0;
static bool g2_merge(const GemmArgs& a) {
    return (double)a.T * a.topk > kG2MergePairs * a.E;
}

hipError_t launch_dec_gemm2(const GemmArgs& a, hipStream_t s) {
    const int rows = dec_rows(a.T, a.topk, a.E);
    if (rows == 4) g2_merge(a) ? launch_g2_rg<2, 4, 2>(a, s) : launch_g2_rg<1, 4, 1>(a, s);
    else if (rows == 8) launch_g2_rg<2, 4, 1>(a, s);
    else launch_g2_rg<4, 2, 1>(a, s);
    return hipGetLastError();
}

}  // namespace moe
