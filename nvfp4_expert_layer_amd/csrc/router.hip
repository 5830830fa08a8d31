// Router, shard filter and permutation kernels (gfx950).
//
// Routing (the page "Serving Solar Open 2 on DGX Spark", section "Solar Open 2
// 개요": routed experts, top-k, one shared expert; section "수정 사항 › b12x에서의
// Expert Parallelism 구현 추가": routing is global, the kernel maps the globally
// routed id to a shard-relative index and drops pairs outside the shard):
//   logits over ALL experts, top-k by logit (ties -> lower id), weights = softmax
//   over the k selected logits, local id = id - offset if inside [0, L) else -1.
//
// Exactness of the selection.  Up to 128 tokens the logits are computed in fp64
// outright on the fp64 matrix cores (bf16 x bf16 products are exact in fp64),
// and the top-k is taken on them directly.  Beyond that, logits are first
// computed with bf16 MFMA (the bf16 x bf16 products are exact in fp32; the
// accumulation rounds) and certified.  For any
// order of at most n fp32 additions with relative error <= u' each (u' = 2^-23
// covers round-to-nearest and truncation), |lhat - l| <= gamma_n * sum_k |x_k g_k|
// <= gamma_n * ||x||_2 * ||g_e||_2 (Cauchy-Schwarz), gamma_n = n u' / (1 - n u'),
// plus d * 2^-126 for products that fall below the fp32 normal range.  With
// lower/upper bounds lo_e, hi_e, let lowk be the k-th largest lo.  An expert with
// hi_e < lowk has at least k experts certainly above it, so it cannot be in the
// top-k.  Every other expert (the candidates) is re-scored in fp64 (exact
// products, fixed summation order) and the top-k is taken among them.
//
// Permutation: pairs grouped by local expert, stable by token.  An LDS bitmask
// per local expert records which tokens chose it; a pair's rank is a popcount of
// the lower bits, so the order is deterministic without sorting.  Up to 512
// tokens one workgroup does it all; beyond, per block of 256 tokens, and a
// single-workgroup scan turns per-block counts into per-block bases, counts,
// offsets and the GEMM tile table.
#include "device_common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// R1: partial logits [ks][T][E] (fp32, bf16 MFMA) and partial squared norms
//     of hidden rows [ks][T] and gate rows [ks][E] (fp64), over K slice ks.
// ---------------------------------------------------------------------------
constexpr int kR1Tile = 64;     // tokens x experts per workgroup
constexpr int kR1BK = 64;
constexpr int kR1Pad = 8;       // bf16 elements of row padding in LDS
constexpr int kR1Depth = 4;     // K chunks of loads in flight per workgroup

__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ G, int T, int E, int d,
    int kslice, float* __restrict__ part, double* __restrict__ xn2, double* __restrict__ gn2) {
    // double-buffered LDS tiles, fed from a register ring that keeps the loads
    // of the next kR1Depth chunks in flight (the chunks come mostly from L2,
    // and one chunk of MFMA work is far shorter than an L2 round trip)
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][kR1Tile][kR1BK + kR1Pad];
    __shared__ __attribute__((aligned(16))) uint16_t gs[2][kR1Tile][kR1BK + kR1Pad];
    const int t0 = blockIdx.x * kR1Tile, e0 = blockIdx.y * kR1Tile, ks = blockIdx.z;
    const int kbeg = ks * kslice, kend = min(d, kbeg + kslice);
    const int nchunk = kend > kbeg ? (kend - kbeg) / kR1BK : 0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // wave layout 2x2: wave (wm, wn) owns tokens [32 wm, +32) x experts [32 wn, +32)
    const int wm = wave >> 1, wn = wave & 1;
    f32x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // 64 rows x 64 bf16 of X and of G per chunk: 512 16-byte pieces each, 2 per
    // thread; rows past T or E read row 0 of the tile (discarded at the end)
    const int r0 = tid >> 3, cc = (tid & 7) * 8;
    const uint16_t* xsrc[2];
    const uint16_t* gsrc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int r = r0 + 32 * c;
        xsrc[c] = X + (size_t)(t0 + (t0 + r < T ? r : 0)) * d + cc;
        gsrc[c] = G + (size_t)(e0 + (e0 + r < E ? r : 0)) * d + cc;
    }
    u32x4_t vx[kR1Depth][2], vg[kR1Depth][2];
    auto load = [&](int ci, u32x4_t (&x)[2], u32x4_t (&g)[2]) {
        const int k0 = kbeg + min(ci, nchunk - 1) * kR1BK;   // past the end: re-load the last chunk
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            x[c] = *reinterpret_cast<const u32x4_t*>(xsrc[c] + k0);
            g[c] = *reinterpret_cast<const u32x4_t*>(gsrc[c] + k0);
        }
    };
    auto store = [&](int b, const u32x4_t (&x)[2], const u32x4_t (&g)[2]) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            *reinterpret_cast<u32x4_t*>(&xs[b][r0 + 32 * c][cc]) = x[c];
            *reinterpret_cast<u32x4_t*>(&gs[b][r0 + 32 * c][cc]) = g[c];
        }
    };
    // squared norms (token rows in the first expert tile, expert rows in the
    // first token tile): four threads per row, each a quarter of every chunk in
    // two chains; the quarters are added by a fixed butterfly at the end
    double nx[2] = {0.0, 0.0}, ng[2] = {0.0, 0.0};
    const bool want_x = blockIdx.y == 0, want_g = blockIdx.x == 0;
    const int nrow = tid >> 2, nq = (tid & 3) * 16;
    auto chunk = [&](int b) {
        auto sq16 = [&](const uint16_t* row, double (&acc)[2]) {
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(row);
            const u32x4_t c = *reinterpret_cast<const u32x4_t*>(row + 8);
            const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const double lo = (double)__uint_as_float(w[q] << 16), hi = (double)__uint_as_float(w[q] & 0xFFFF0000u);
                acc[q & 1] = fma(lo, lo, acc[q & 1]);
                acc[q & 1] = fma(hi, hi, acc[q & 1]);
            }
        };
        if (want_x) sq16(&xs[b][nrow][nq], nx);
        if (want_g) sq16(&gs[b][nrow][nq], ng);
#pragma unroll
        for (int kk = 0; kk < kR1BK; kk += 32) {
            bf16x8_t a[2], bb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const bf16x8_t*>(&xs[b][wm * 32 + i * 16 + (lane & 15)][kk + (lane >> 4) * 8]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bb[j] = *reinterpret_cast<const bf16x8_t*>(&gs[b][wn * 32 + j * 16 + (lane & 15)][kk + (lane >> 4) * 8]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
        }
    };
    if (nchunk > 0) {
        // ring slot u holds chunk u + kR1Depth * round; chunk 0 goes to LDS first
#pragma unroll
        for (int u = 0; u < kR1Depth; ++u) load(u, vx[u], vg[u]);
        store(0, vx[0], vg[0]);
        load(kR1Depth, vx[0], vg[0]);
        __syncthreads();
        // whole ring rounds (chunks past the end re-load the last chunk and
        // are not multiplied)
        for (int c0 = 0; c0 < nchunk; c0 += kR1Depth) {
#pragma unroll
            for (int u = 0; u < kR1Depth; ++u) {
                const int c = c0 + u;                          // chunk in LDS buffer c & 1
                if (c < nchunk) chunk(c & 1);
                const int un = (u + 1) % kR1Depth;             // slot of chunk c + 1
                if (c + 1 < nchunk) store((c + 1) & 1, vx[un], vg[un]);
                load(c + 1 + kR1Depth, vx[un], vg[un]);
                __syncthreads();
            }
        }
    }
    float* out = part + (size_t)ks * T * E;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
                const int e = e0 + wn * 32 + j * 16 + (lane & 15);
                if (t < T && e < E) out[(size_t)t * E + e] = acc[i][j][r];
            }
    double sx = nx[0] + nx[1], sg = ng[0] + ng[1];
    sx += __shfl_xor(sx, 1, 64);
    sx += __shfl_xor(sx, 2, 64);
    sg += __shfl_xor(sg, 1, 64);
    sg += __shfl_xor(sg, 2, 64);
    if ((tid & 3) == 0) {
        if (want_x && t0 + nrow < T) xn2[(size_t)ks * T + t0 + nrow] = sx;
        if (want_g && e0 + nrow < E) gn2[(size_t)ks * E + e0 + nrow] = sg;
    }
}

// ---------------------------------------------------------------------------
// The same logits for many tokens and at most 320 experts: a workgroup takes
// 64 tokens x ALL experts (eight waves, 2 x 4: a wave owns 32 tokens x 80
// experts as 2 x 5 MFMA blocks).  The 64 x 64 kernel above reads every token
// row once per 64-expert tile and the whole router weight once per 64-token
// tile; here the token rows are read once, which cuts the traffic between L2
// and the CUs by ~40% (T = 16384: 0.80 against 1.34 GB).  Same partials and
// per-slice squared norms as above: the bound and the selection are unchanged.
// ---------------------------------------------------------------------------
constexpr int kWideTok = 64;                 // tokens per workgroup
constexpr int kWideEx = 320;                 // expert rows staged (E <= 320)
constexpr int kWideDepth = 2;                // K chunks of loads in flight per thread (3 and 4 measured slower)
template <int TOK>
constexpr int wide_pieces() { return (TOK + kWideEx) * (kR1BK / 8) / 512; }   // 16-byte loads per thread per chunk
template <int TOK>
constexpr int wide_lds() { return 2 * (TOK + kWideEx) * (kR1BK + kR1Pad) * 2; }
constexpr int kWideLds = wide_lds<kWideTok>();

bool router_wide(int T, int E) { return E > 128 && E <= kWideEx && T >= 4096; }

template <int TOK>
__global__ __launch_bounds__(512) void router_logits_wide_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ G, int T, int E, int d,
    int kslice, float* __restrict__ part, double* __restrict__ xn2, double* __restrict__ gn2) {
    constexpr int NP = wide_pieces<TOK>(), NI = TOK / 32;   // loads per thread; 16-token blocks per wave
    static_assert(NP * 512 == (TOK + kWideEx) * (kR1BK / 8), "loads cover the chunk");
    extern __shared__ __attribute__((aligned(16))) uint16_t wl[];
    constexpr int RS = kR1BK + kR1Pad;                    // LDS row stride (bf16)
    constexpr int BUF = (TOK + kWideEx) * RS;             // one buffer: token rows, then expert rows
    const int t0 = blockIdx.x * TOK, ks = blockIdx.y;
    const int kbeg = ks * kslice, kend = min(d, kbeg + kslice);
    const int nchunk = kend > kbeg ? (kend - kbeg) / kR1BK : 0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;              // tokens [TOK/2 wm, +TOK/2) x experts [80 wn, +80)
    f32x4_t acc[NI][5];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 5; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // piece p = tid + 512 q of a chunk: staged row p / 8 (the first TOK are
    // token rows, then the expert rows), 16-byte column p % 8; rows past T or E
    // read row 0 (their results are discarded)
    const uint16_t* src[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
        const int p = tid + 512 * q, r = p >> 3, c = (p & 7) * 8;
        if (r < TOK) src[q] = X + (size_t)(t0 + r < T ? t0 + r : 0) * d + c;
        else src[q] = G + (size_t)(r - TOK < E ? r - TOK : 0) * d + c;
    }
    u32x4_t ring[kWideDepth][NP];
    auto load = [&](int ci, u32x4_t (&v)[NP]) {
        const int k0 = kbeg + min(ci, nchunk - 1) * kR1BK;   // past the end: re-load the last chunk
#pragma unroll
        for (int q = 0; q < NP; ++q) v[q] = *reinterpret_cast<const u32x4_t*>(src[q] + k0);
    };
    auto store = [&](int b, const u32x4_t (&v)[NP]) {
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const int p = tid + 512 * q;
            *reinterpret_cast<u32x4_t*>(wl + b * BUF + (p >> 3) * RS + (p & 7) * 8) = v[q];
        }
    };
    // squared norms: token rows by threads 0..255 (256 / TOK per row, each
    // TOK / 4 elements of every chunk), expert rows (64 per workgroup,
    // workgroups 0..4 of the slice) by threads 256..511 (four per row, 16
    // elements each); two chains per thread, the threads of a row added by a
    // fixed butterfly at the end
    constexpr int XT = 256 / TOK;                         // threads per token row
    const bool norm_x = tid < 256;
    const int nrow = norm_x ? tid / XT : (tid - 256) >> 2;
    const int nq = norm_x ? (tid % XT) * (kR1BK / XT) : ((tid - 256) & 3) * 16;
    const int grow = (int)blockIdx.x * 64 + nrow;         // this thread's expert row (norm_x false)
    const bool norm_g = !norm_x && grow < kWideEx && blockIdx.x * 64 < (unsigned)E;
    double nn[2] = {0.0, 0.0};
    auto chunk = [&](int b) {
        const uint16_t* B = wl + b * BUF;
        if (norm_x || norm_g) {
            const uint16_t* row = B + (norm_x ? nrow : TOK + grow) * RS + nq;
#pragma unroll
            for (int h = 0; h < (norm_x ? kR1BK / XT / 16 : 1); ++h) {
                const u32x4_t a = *reinterpret_cast<const u32x4_t*>(row + 16 * h);
                const u32x4_t c = *reinterpret_cast<const u32x4_t*>(row + 16 * h + 8);
                const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const double lo = (double)__uint_as_float(w[q] << 16), hi = (double)__uint_as_float(w[q] & 0xFFFF0000u);
                    nn[q & 1] = fma(lo, lo, nn[q & 1]);
                    nn[q & 1] = fma(hi, hi, nn[q & 1]);
                }
            }
        }
#pragma unroll
        for (int kk = 0; kk < kR1BK; kk += 32) {
            bf16x8_t a[NI], bb[5];
#pragma unroll
            for (int i = 0; i < NI; ++i)
                a[i] = *reinterpret_cast<const bf16x8_t*>(B + (wm * (TOK / 2) + i * 16 + (lane & 15)) * RS + kk +
                                                          (lane >> 4) * 8);
#pragma unroll
            for (int j = 0; j < 5; ++j)
                bb[j] = *reinterpret_cast<const bf16x8_t*>(B + (TOK + wn * 80 + j * 16 + (lane & 15)) * RS + kk +
                                                           (lane >> 4) * 8);
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int j = 0; j < 5; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
        }
    };
    if (nchunk > 0) {
        // ring slot u holds chunk u + kWideDepth * round; chunk 0 goes to LDS first
#pragma unroll
        for (int u = 0; u < kWideDepth; ++u) load(u, ring[u]);
        store(0, ring[0]);
        load(kWideDepth, ring[0]);
        __syncthreads();
        for (int c0 = 0; c0 < nchunk; c0 += kWideDepth) {
#pragma unroll
            for (int u = 0; u < kWideDepth; ++u) {
                const int c = c0 + u;                          // chunk in LDS buffer c & 1
                if (c < nchunk) chunk(c & 1);
                const int un = (u + 1) % kWideDepth;           // slot of chunk c + 1
                if (c + 1 < nchunk) store((c + 1) & 1, ring[un]);
                load(c + 1 + kWideDepth, ring[un]);
                __syncthreads();
            }
        }
    }
    float* out = part + (size_t)ks * T * E;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 5; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + wm * (TOK / 2) + i * 16 + (lane >> 4) * 4 + r;
                const int e = wn * 80 + j * 16 + (lane & 15);
                if (t < T && e < E) out[(size_t)t * E + e] = acc[i][j][r];
            }
    double sn = nn[0] + nn[1];
    sn += __shfl_xor(sn, 1, 64);
    if (!norm_x || XT == 4) sn += __shfl_xor(sn, 2, 64);  // (wave-uniform: threads 0..255 are waves 0..3)
    if (norm_x ? (tid % XT) == 0 : (tid & 3) == 0) {
        if (norm_x && t0 + nrow < T) xn2[(size_t)ks * T + t0 + nrow] = sn;
        if (norm_g && grow < E) gn2[(size_t)ks * E + grow] = sn;
    }
}

// ---------------------------------------------------------------------------
// R2 for few tokens (latency): one workgroup of 1024 threads per token.
//   bounds: thread e < E takes expert e (all of its split-K partial loads in one
//     batch);
//   threshold: wave 0 runs a tournament (k rounds of a wave max) over the
//     unique rank keys;
//   candidates: hi >= threshold, listed in any order (the final rank is by
//     (score, id));
//   fp64 re-scoring: item (candidate c, K slice s) for kSlices slices of K, so
//     each item's loads go out together; the slice sums of a candidate are
//     added in slice order by one thread (deterministic);
//   rank by (score desc, id asc), softmax over the first k.
// ---------------------------------------------------------------------------
constexpr int kMaxExperts = 1024;
constexpr int kMaxKS = 16;          // split-K slices of the logits GEMM
constexpr int kSlices = 64;         // at most this many K slices of one fp64 candidate dot product
constexpr int kSelThreads = 1024;
// From here on, one wave per token.  Routing stage time on the 320-expert
// layer, workgroup per token against wave per token: T = 129 30.6 / 42.6 us,
// T = 256 33.6 / 45.0, T = 512 53.2 / 50.9, T = 768 66.0 / 54.2.
constexpr int kWideSelectTokens = 512;
// Below kSplitSelectTokens the four waves of a workgroup share each token's K
// chunks.  Routing stage time on the 320-expert layer, one wave against four
// per token: T = 512 ~51 / 46.5 us, T = 768 54.2 / 53.2; T = 1024 56.8 / 64.6
// (four slower).  Against the workgroup per token below 512: T = 129 30.6 /
// 33.7, T = 256 33.5 / 35.9.
constexpr int kSplitSelectTokens = 1024;
// From kOccSelectTokens the one-wave-per-token kernel is held to 128 VGPRs, for
// four waves per SIMD instead of three (a few registers then spill).
constexpr int kOccSelectTokens = 4096;

// Wave-wide unsigned max through DPP row shifts and row broadcasts (lanes that
// read outside their row get 0, the identity): after the row_shr steps lane 15
// of each row holds the row's max, row_bcast15 / row_bcast31 carry it up to lane
// 63, which readlane then hands to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    auto step = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
    v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true));   // row_shr:1
    v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true));   // row_shr:2
    v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true));   // row_shr:4
    v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true));   // row_shr:8
    v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
    v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Wave-wide max of 64-bit keys: the max of the high words, then the max of the
// low words among the lanes that hold that high word.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
    const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
    return ((uint64_t)hi << 32) | lo;
}

// Rank key of a lower bound: lo rounded DOWN to fp32, made order-preserving as
// an unsigned integer, with the expert id below it (equal values: lower id
// first).  Keys are unique; 0 is below every key.
__device__ __forceinline__ uint64_t rank_key(double lo, int e) {
    float lf = (float)lo;
    uint32_t bits = __float_as_uint(lf);
    if ((double)lf > lo)   // one fp32 step toward -inf (lo is finite)
        bits = (lf > 0.0f) ? bits - 1u : (lf == 0.0f ? 0x80000001u : bits + 1u);
    const uint32_t ord = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

// The fp32 lower bound a rank key was made from.
__device__ __forceinline__ double key_value(uint64_t key) {
    const uint32_t ord = (uint32_t)(key >> 32);
    return (double)__uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

template <int EPL>   // experts per lane of wave 0 in the tournament: 64 EPL >= E
__global__ __launch_bounds__(kSelThreads) void router_select_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ G, const float* __restrict__ part,
    const double* __restrict__ xn2, const double* __restrict__ gn2, int T, int E, int d, int KS,
    int topk, int offset, int L, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ local_ids) {
    __shared__ int32_t s_cand[kMaxExperts];
    __shared__ double s_score[kMaxExperts];
    __shared__ double s_part[kSelThreads];
    __shared__ double s_hi[kMaxExperts];
    __shared__ uint64_t s_key[kMaxExperts];
    __shared__ int32_t s_ncand;
    __shared__ double s_lowk;
    __shared__ int32_t s_sel_id[32];
    __shared__ double s_sel_sc[32];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = blockIdx.x;
    const uint16_t* xrow = X + (size_t)t * d;
    if (tid == 0) s_ncand = 0;
    {
        // Bounds: the split-K partial sums are added in slice order.  The fp32
        // logit differs from the exact dot product by at most
        // gamma_n ||x|| ||g_e|| + d 2^-126 with n = d + KS (see the file header).
        const double u = 1.0 / 8388608.0;
        const double n = (double)(d + KS);
        const double gamma = n * u / (1.0 - n * u) * (1.0 + 1e-6);
        const double tiny = (double)d * 1.1754943508222875e-38;
        const int e = tid;
        double xv[kMaxKS], gv[kMaxKS];
        float pv[kMaxKS];
#pragma unroll
        for (int s = 0; s < kMaxKS; ++s) {
            const bool in = s < KS && e < E;
            xv[s] = s < KS ? xn2[(size_t)s * T + t] : 0.0;
            pv[s] = in ? part[((size_t)s * T + t) * E + e] : 0.f;
            gv[s] = in ? gn2[(size_t)s * E + e] : 0.0;
        }
        if (e < E) {
            double xs2 = 0.0, gs2 = 0.0;
            float lh = 0.f;
#pragma unroll
            for (int s = 0; s < kMaxKS; ++s) {
                xs2 += xv[s];
                gs2 += gv[s];
                lh += pv[s];
            }
            const double xnorm = sqrt(xs2) * (1.0 + 1e-12);
            const double beta = gamma * xnorm * (sqrt(gs2) * (1.0 + 1e-12)) + tiny;
            s_hi[e] = (double)lh + beta;
            s_key[e] = rank_key((double)lh - beta, e);
        }
    }
    __syncthreads();
    // Threshold: the k-th largest rank key (it is <= the k-th largest exact
    // lower bound, so the candidates below are a superset of the exact ones).
    if (wave == 0) {
        // lane's keys (experts lane + 64 sl) in registers; k rounds of a wave max,
        // the owner of each maximum dropping it
        uint64_t key[EPL];
#pragma unroll
        for (int sl = 0; sl < EPL; ++sl) {
            const int e = lane + 64 * sl;
            key[sl] = e < E ? s_key[e] : 0;
        }
        uint64_t kth = 0;
        for (int r = 0; r < topk; ++r) {
            uint64_t m = 0;
#pragma unroll
            for (int sl = 0; sl < EPL; ++sl) m = key[sl] > m ? key[sl] : m;
            kth = wave_max_u64(m);
#pragma unroll
            for (int sl = 0; sl < EPL; ++sl) key[sl] = key[sl] == kth ? 0 : key[sl];
        }
        if (lane == 0) s_lowk = key_value(kth);
    }
    __syncthreads();
    // candidates: every expert whose upper bound reaches the threshold
    if (tid < E && s_hi[tid] >= s_lowk) s_cand[atomicAdd(&s_ncand, 1)] = tid;
    __syncthreads();
    const int nc = s_ncand;
    // fp64 re-scoring: item (c, sl) = candidate c over K slice sl.  nsl slices
    // of len elements, len a multiple of 8 (one 16-byte load): nsl = the largest
    // divisor of d / 8 up to kSlices; kSelThreads / nsl candidates per pass.
    int nsl = kSlices;
    while ((d / 8) % nsl) --nsl;
    const int len = d / nsl, maxc = kSelThreads / nsl;
    for (int cb = 0; cb < nc; cb += maxc) {
        const int ncb = min(maxc, nc - cb);
        {
            const int c = tid / nsl, sl = tid - c * nsl;
            if (c < ncb) {
                const int k0 = sl * len;
                const uint16_t* gx = xrow + k0;
                const uint16_t* gg = G + (size_t)s_cand[cb + c] * d + k0;
                double acc4[4] = {0.0, 0.0, 0.0, 0.0};   // four chains, added in a fixed order
                for (int kk = 0; kk < len; kk += 64) {
                    u32x4_t vx[8], vg[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const bool in = kk + j * 8 < len;
                        vx[j] = in ? *reinterpret_cast<const u32x4_t*>(gx + kk + j * 8) : u32x4_t{0u, 0u, 0u, 0u};
                        vg[j] = in ? *reinterpret_cast<const u32x4_t*>(gg + kk + j * 8) : u32x4_t{0u, 0u, 0u, 0u};
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint32_t ax[4] = {vx[j].x, vx[j].y, vx[j].z, vx[j].w};
                        const uint32_t ag[4] = {vg[j].x, vg[j].y, vg[j].z, vg[j].w};
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            acc4[q] = fma((double)__uint_as_float(ax[q] << 16), (double)__uint_as_float(ag[q] << 16),
                                          acc4[q]);
                            acc4[q] = fma((double)__uint_as_float(ax[q] & 0xFFFF0000u),
                                          (double)__uint_as_float(ag[q] & 0xFFFF0000u), acc4[q]);
                        }
                    }
                }
                s_part[tid] = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
            }
        }
        __syncthreads();
        if (tid < ncb) {
            // slices dealt round-robin to four chains, combined in a fixed order
            double c4[4] = {0.0, 0.0, 0.0, 0.0};
            for (int sl = 0; sl < nsl; ++sl) c4[sl & 3] += s_part[tid * nsl + sl];
            s_score[cb + tid] = (c4[0] + c4[1]) + (c4[2] + c4[3]);
        }
        __syncthreads();
    }
    // top-k among candidates by (fp64 score desc, id asc): a candidate's rank is
    // the number of candidates ahead of it; ranks 0..k-1 are the selected slots
    for (int c = tid; c < nc; c += kSelThreads) {
        const double v = s_score[c];
        const int id = s_cand[c];
        int rank = 0;
        for (int f = 0; f < nc; ++f) {
            const double w = s_score[f];
            rank += (int)(w > v) | ((int)(w == v) & (int)(s_cand[f] < id));
        }
        if (rank < topk) {
            s_sel_id[rank] = id;
            s_sel_sc[rank] = v;
        }
    }
    __syncthreads();
    if (wave != 0) return;
    // softmax over the k selected fp64 scores (slot 0 holds the largest)
    const double my_score = lane < topk ? s_sel_sc[lane] : 0.0;
    const double z = lane < topk ? exp(my_score - s_sel_sc[0]) : 0.0;
    const double zs = wave_sum_f64(z);
    if (lane < topk) {
        const int my_id = s_sel_id[lane];
        const size_t o = (size_t)t * topk + lane;
        topk_ids[o] = my_id;
        topk_w[o] = (float)(z / zs);
        const int lam = my_id - offset;
        local_ids[o] = (lam >= 0 && lam < L) ? lam : -1;
    }
}

// ---------------------------------------------------------------------------
// R2 for many tokens: the same certified selection, one wave per token (four
// tokens per workgroup, waves independent).  Experts e = lane + 64 s, s < EPL
// (the smallest instantiated EPL with 64 EPL >= E).
//   bounds  -> registers;
//   threshold: the k-th largest rank key by a tournament (k rounds of a wave
//     max; keys are unique, so exactly one lane owns each maximum);
//   candidates (hi >= threshold), in ascending id order -> per-wave LDS list;
//   fp64 re-scoring: K in chunks of 512 (8 elements per lane, converted to fp64
//     once per chunk and shared by up to 16 candidates whose loads are all in
//     flight together); per-lane partial sums are reduced in a fixed butterfly
//     order, so scores are deterministic;
//   rank of each candidate by (score desc, id asc), softmax over the first k.
// ---------------------------------------------------------------------------
constexpr int kWTok = 4;            // tokens (waves) per workgroup
constexpr int kWGroup = 8;          // candidates scored together

// WPT waves per token (1, or kWTok: the workgroup's waves share one token).
// With several, every wave of the token computes the same bounds and candidate
// list, each re-scores its own share of the K chunks, and the shares' sums are
// added in wave order; one wave then ranks.  A token's latency is a chain of
// dependent round trips (the candidates' chunks above all), which the split
// shortens where few tokens leave the chip idle.
template <int kWSlots, int WPT, int OCC = 1>
__global__ __launch_bounds__(64 * kWTok) __attribute__((amdgpu_waves_per_eu(OCC))) void router_select_wave_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ G, const float* __restrict__ part,
    const double* __restrict__ xn2, const double* __restrict__ gn2, int T, int E, int d, int KS,
    int topk, int offset, int L, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ local_ids) {
    static_assert(WPT == 1 || WPT == kWTok, "one token per wave or per workgroup");
    __shared__ int32_t s_cid[kWTok][kWSlots * 64];       // candidates are experts: at most E <= 64 kWSlots
    __shared__ double s_csc[kWTok][kWSlots * 64];
    __shared__ int32_t s_sel_id[kWTok][32];
    __shared__ double s_sel_sc[kWTok][32];
    __shared__ double s_share[WPT > 1 ? WPT : 1][kWGroup];
    // (held to fewer registers, the kernel keeps its wave-uniform values -- the
    // wave index and the candidates' row addresses -- in scalar registers: at
    // four waves per SIMD, T = 8192 83.7 -> 78.6 us, 16384 147.7 -> 139.8; with
    // no register limit that measured 1-5% slower, so it is left to the compiler)
    const int lane = threadIdx.x & 63;
    const int w = OCC > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : (int)(threadIdx.x >> 6);
    const int sub = w % WPT;                             // this wave's share of the token's K chunks
    const int t = blockIdx.x * (kWTok / WPT) + w / WPT;
    // whole wave (WPT == 1: no workgroup barriers below), or whole workgroup
    if (t >= T) return;
    int32_t* cid = s_cid[w];
    double* csc = s_csc[w];

    // ---- bounds (same arithmetic and order as router_select_kernel) ----
    const double u = 1.0 / 8388608.0;
    const double n = (double)(d + KS);
    const double gamma = n * u / (1.0 - n * u) * (1.0 + 1e-6);
    const double tiny = (double)d * 1.1754943508222875e-38;
    // the split-K partials are added in slice order; four slices' loads (for
    // every slot) go out together
    double xs2 = 0.0;
    float lh[kWSlots];
    double gs2[kWSlots];
#pragma unroll
    for (int sl = 0; sl < kWSlots; ++sl) {
        lh[sl] = 0.f;
        gs2[sl] = 0.0;
    }
    const int ec = E - 1;
    for (int s0 = 0; s0 < KS; s0 += 4) {
        double xv[4], gv[4][kWSlots];
        float pv[4][kWSlots];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s = min(s0 + j, KS - 1);
            xv[j] = xn2[(size_t)s * T + t];
#pragma unroll
            for (int sl = 0; sl < kWSlots; ++sl) {
                const int e = min(lane + 64 * sl, ec);
                pv[j][sl] = part[((size_t)s * T + t) * E + e];
                gv[j][sl] = gn2[(size_t)s * E + e];
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (s0 + j < KS) {
                xs2 += xv[j];
#pragma unroll
                for (int sl = 0; sl < kWSlots; ++sl) {
                    lh[sl] += pv[j][sl];
                    gs2[sl] += gv[j][sl];
                }
            }
        }
    }
    const double xnorm = sqrt(xs2) * (1.0 + 1e-12);
    double hi[kWSlots];
    uint64_t key[kWSlots];
#pragma unroll
    for (int sl = 0; sl < kWSlots; ++sl) {
        hi[sl] = -INFINITY;
        key[sl] = 0;                                     // below every valid key
        const int e = lane + 64 * sl;
        if (e < E) {
            const double beta = gamma * xnorm * (sqrt(gs2[sl]) * (1.0 + 1e-12)) + tiny;
            hi[sl] = (double)lh[sl] + beta;
            key[sl] = rank_key((double)lh[sl] - beta, e);
        }
    }

    // ---- threshold: k rounds of a wave max over the remaining keys ----
    uint64_t kth = 0;
    for (int r = 0; r < topk; ++r) {
        uint64_t m = 0;
#pragma unroll
        for (int sl = 0; sl < kWSlots; ++sl) m = key[sl] > m ? key[sl] : m;
        kth = wave_max_u64(m);
#pragma unroll
        for (int sl = 0; sl < kWSlots; ++sl) key[sl] = key[sl] == kth ? 0 : key[sl];
    }
    const double lowk = key_value(kth);

    // ---- candidates in ascending id order ----
    int nc = 0;
#pragma unroll
    for (int sl = 0; sl < kWSlots; ++sl) {
        const bool c = hi[sl] >= lowk;
        const uint64_t mask = __ballot(c);
        if (c) cid[nc + __popcll(mask & ((1ull << lane) - 1ull))] = lane + 64 * sl;
        nc += __popcll(mask);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();

    // ---- fp64 re-scoring: groups of up to kWGroup candidates; the K loop is
    // software-pipelined (the next 512-element chunk's loads go out before
    // this chunk is multiplied); a short last group skips its empty slots ----
    const uint16_t* xrow = X + (size_t)t * d;
    // this wave's chunks of 512 elements: [c_lo, c_hi)
    const int nchunk = (d + 511) / 512;
    const int c_lo = sub * nchunk / WPT, c_hi = (sub + 1) * nchunk / WPT;
    const int k_end = min(d, 512 * c_hi);
    for (int g0 = 0; g0 < nc; g0 += kWGroup) {
        const int ng = min(kWGroup, nc - g0);
        const uint16_t* grow[kWGroup];
#pragma unroll
        for (int c = 0; c < kWGroup; ++c) {
            const int id = cid[g0 + (c < ng ? c : 0)];
            grow[c] = G + (size_t)(OCC > 1 ? __builtin_amdgcn_readfirstlane(id) : id) * d;
        }
        double acc[kWGroup];
#pragma unroll
        for (int c = 0; c < kWGroup; ++c) acc[c] = 0.0;
        int k0 = 512 * c_lo + lane * 8;
        u32x4_t xv{0u, 0u, 0u, 0u}, gv[kWGroup];
        if (k0 < k_end) {
            xv = *reinterpret_cast<const u32x4_t*>(xrow + k0);
#pragma unroll
            for (int c = 0; c < kWGroup; ++c)
                if (c < ng) gv[c] = *reinterpret_cast<const u32x4_t*>(grow[c] + k0);
        }
        for (; k0 < k_end; k0 += 512) {
            const u32x4_t xc = xv;
            u32x4_t gc[kWGroup];
#pragma unroll
            for (int c = 0; c < kWGroup; ++c) gc[c] = gv[c];
            if (k0 + 512 < k_end) {
                xv = *reinterpret_cast<const u32x4_t*>(xrow + k0 + 512);
#pragma unroll
                for (int c = 0; c < kWGroup; ++c)
                    if (c < ng) gv[c] = *reinterpret_cast<const u32x4_t*>(grow[c] + k0 + 512);
            }
            double xd[8];
            const uint32_t xw[4] = {xc.x, xc.y, xc.z, xc.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xd[2 * q] = (double)__uint_as_float(xw[q] << 16);
                xd[2 * q + 1] = (double)__uint_as_float(xw[q] & 0xFFFF0000u);
            }
#pragma unroll
            for (int c = 0; c < kWGroup; ++c) {
                if (c < ng) {
                    const uint32_t gw[4] = {gc[c].x, gc[c].y, gc[c].z, gc[c].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[c] = fma(xd[2 * q], (double)__uint_as_float(gw[q] << 16), acc[c]);
                        acc[c] = fma(xd[2 * q + 1], (double)__uint_as_float(gw[q] & 0xFFFF0000u), acc[c]);
                    }
                }
            }
        }
        if (WPT == 1) {
#pragma unroll
            for (int c = 0; c < kWGroup; ++c) {
                if (c < ng) {
                    const double sc = wave_sum_f64(acc[c]);
                    if (lane == 0) csc[g0 + c] = sc;
                }
            }
        } else {
            // the waves' shares meet in LDS and are added in wave order
#pragma unroll
            for (int c = 0; c < kWGroup; ++c) {
                const double sc = wave_sum_f64(acc[c]);
                if (lane == 0) s_share[sub][c] = sc;
            }
            __syncthreads();
            if (sub == 0 && lane < ng) {
                double sc = s_share[0][lane];
#pragma unroll
                for (int q = 1; q < WPT; ++q) sc += s_share[q][lane];
                csc[g0 + lane] = sc;
            }
            __syncthreads();
        }
    }
    if (WPT > 1 && sub != 0) return;                     // the token's first wave ranks
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();

    // ---- rank by (score desc, id asc); ranks 0..k-1 are the slots ----
    for (int c = lane; c < nc; c += 64) {
        const double v = csc[c];
        const int id = cid[c];
        int rank = 0;
        for (int f = 0; f < nc; ++f) {
            const double x = csc[f];
            rank += (int)(x > v) | ((int)(x == v) & (int)(cid[f] < id));
        }
        if (rank < topk) {
            s_sel_id[w][rank] = id;
            s_sel_sc[w][rank] = v;
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    const double my_score = lane < topk ? s_sel_sc[w][lane] : 0.0;
    const double z = lane < topk ? exp(my_score - s_sel_sc[w][0]) : 0.0;
    const double zs = wave_sum_f64(z);
    if (lane < topk) {
        const int my_id = s_sel_id[w][lane];
        const size_t o = (size_t)t * topk + lane;
        topk_ids[o] = my_id;
        topk_w[o] = (float)(z / zs);
        const int lam = my_id - offset;
        local_ids[o] = (lam >= 0 && lam < L) ? lam : -1;
    }
}

// ---------------------------------------------------------------------------
// P1: per-block (256 tokens) counts per local expert and ranks of pairs.
// ---------------------------------------------------------------------------
constexpr int kPermBlock = 256;

__global__ __launch_bounds__(kPermBlock) void perm_block_kernel(
    const int32_t* __restrict__ local_ids, int T, int topk, int L, int32_t* __restrict__ block_counts,
    int32_t* __restrict__ rank) {
    extern __shared__ uint32_t masks[];                    // [L][kPermBlock/32]
    constexpr int W = kPermBlock / 32;
    const int tid = threadIdx.x;
    for (int i = tid; i < L * W; i += kPermBlock) masks[i] = 0u;
    __syncthreads();
    const int t = blockIdx.x * kPermBlock + tid;
    if (t < T) {
        for (int j = 0; j < topk; ++j) {
            int lam = local_ids[(size_t)t * topk + j];
            if (lam >= 0) atomicOr(&masks[lam * W + (tid >> 5)], 1u << (tid & 31));
        }
    }
    __syncthreads();
    if (t < T) {
        for (int j = 0; j < topk; ++j) {
            int lam = local_ids[(size_t)t * topk + j];
            int r = -1;
            if (lam >= 0) {
                r = 0;
                for (int w = 0; w < (tid >> 5); ++w) r += __popc(masks[lam * W + w]);
                r += __popc(masks[lam * W + (tid >> 5)] & ((1u << (tid & 31)) - 1u));
            }
            rank[(size_t)t * topk + j] = r;
        }
    }
    for (int l = tid; l < L; l += kPermBlock) {
        int c = 0;
        for (int w = 0; w < W; ++w) c += __popc(masks[l * W + w]);
        block_counts[(size_t)blockIdx.x * L + l] = c;
    }
}

// ---------------------------------------------------------------------------
// P2: one workgroup.  block_counts -> per-block bases (in place), counts,
// offsets, and the GEMM tile table (group, row_begin, row_end, index of the tile
// within its group) with BM rows per tile.  Groups 0..L-1 are the local experts (rows [offsets[g], offsets[g+1])
// of the permuted-pair row space), group L the shared expert (rows [Tk, Tk+T)).
// ---------------------------------------------------------------------------
// Block-wide exclusive scans of (count, tiles) over 1024 threads (one per expert),
// then the tile table: rows [offsets[g], offsets[g+1]) of expert g in BM-row
// tiles, followed by the shared expert's rows [Tk, Tk+T).
__device__ void scan_and_emit_tiles(int c, int L, int T, int topk, int has_shared, int BM,
                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                    int4* __restrict__ tiles, int32_t* __restrict__ ntiles, int max_tiles,
                                    int32_t* s_off) {
    __shared__ int32_t s_wsum[16], s_wsum_t[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tc = tid < L ? (c + BM - 1) / BM : 0;
    int ic = c, it = tc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int vc = __shfl_up(ic, o, 64), vt = __shfl_up(it, o, 64);
        if (lane >= o) { ic += vc; it += vt; }
    }
    if (lane == 63) { s_wsum[wave] = ic; s_wsum_t[wave] = it; }
    __syncthreads();
    int basec = 0, baset = 0;
    for (int w = 0; w < wave; ++w) { basec += s_wsum[w]; baset += s_wsum_t[w]; }
    const int exc = basec + ic - c, ext = baset + it - tc;
    if (tid < L) {
        counts[tid] = c;
        offsets[tid] = exc;
        if (s_off) s_off[tid] = exc;
        for (int i = 0; i < tc; ++i) {
            const int rb = exc + i * BM;
            tiles[ext + i] = make_int4(tid, rb, min(rb + BM, exc + c), i);
        }
    }
    if (tid == L - 1) {
        offsets[L] = exc + c;
        int n = ext + tc;
        if (has_shared) {
            const int base = T * topk;
            const int st = (T + BM - 1) / BM;
            for (int i = 0; i < st; ++i)
                tiles[n + i] = make_int4(L, base + i * BM, min(base + (i + 1) * BM, base + T), i);
            n += st;
        }
        ntiles[0] = n < max_tiles ? n : max_tiles;
    }
}

__global__ __launch_bounds__(1024) void perm_scan_kernel(
    int32_t* __restrict__ block_counts, int nblk, int L, int T, int topk, int has_shared, int BM,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int4* __restrict__ tiles,
    int32_t* __restrict__ ntiles, int max_tiles) {
    const int tid = threadIdx.x;
    // per-expert scan over blocks (L <= 1024: one thread per expert)
    int total = 0;
    if (tid < L) {
        // eight blocks' counts are loaded together, then scanned in block order
        for (int b0 = 0; b0 < nblk; b0 += 8) {
            int c[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = block_counts[(size_t)min(b0 + j, nblk - 1) * L + tid];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (b0 + j < nblk) {
                    block_counts[(size_t)(b0 + j) * L + tid] = total;
                    total += c[j];
                }
            }
        }
    }
    scan_and_emit_tiles(total, L, T, topk, has_shared, BM, counts, offsets, tiles, ntiles, max_tiles, nullptr);
}

// All three permutation steps in one workgroup of 1024 threads, for T <= 1024:
// a bitmask of ceil(T/32) words per local expert (masks, [L][W]) marks the
// tokens that chose it, and an exclusive prefix of its words' popcounts (pre,
// 16-bit, [L][W]) makes a pair's rank within its expert two LDS reads: the
// prefix of the token's word plus the popcount of the lower bits in it.
// Kernel time against the three-launch path on the 160-expert shard: T = 640
// 7.9 us against 7.5 + 4.6 + 4.7, T = 1024 13.3 against 7.6 + 4.6 + 4.6 (plus
// two launch gaps).
constexpr int kPermSmallTokens = 1024;
constexpr int kPermSmallLds = 57344;        // bytes of bitmask + prefix (dynamic; the static arrays take the rest of 64 KB)

__host__ __device__ constexpr size_t perm_small_lds(int T, int L) {
    return (size_t)L * ((T + 31) / 32) * 6;
}

__device__ void perm_small_body(const int32_t* __restrict__ local_ids, int T, int topk, int L, int has_shared,
                                int BM, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                int4* __restrict__ tiles, int32_t* __restrict__ ntiles, int max_tiles,
                                int32_t* __restrict__ perm, int32_t* __restrict__ inv, uint32_t* masks) {
    __shared__ int32_t s_off[1024];
    const int W = (T + 31) >> 5;
    uint16_t* const pre = reinterpret_cast<uint16_t*>(masks + L * W);
    const int tid = threadIdx.x;
    const bool tok = tid < T;
    const int wd = tid >> 5;
    const uint32_t bit = 1u << (tid & 31);
    const size_t row = (size_t)(tok ? tid : 0) * topk;
    // the token's first eight ids, loaded by the waves that hold tokens (a
    // wave-uniform branch; within it a clamped index re-reads the last id, and
    // only the uses are conditional)
    int lj[8] = {-1, -1, -1, -1, -1, -1, -1, -1};
    if (topk > 0 && __builtin_amdgcn_readfirstlane(tid) < T) {
#pragma unroll
        for (int q = 0; q < 8; ++q) lj[q] = local_ids[row + min(q, topk - 1)];
    }
    for (int i = tid; i < L * W; i += 1024) masks[i] = 0u;
    __syncthreads();
    if (tok) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (q < topk && (unsigned)lj[q] < (unsigned)L) atomicOr(&masks[lj[q] * W + wd], bit);
        for (int j = 8; j < topk; ++j) {
            const int lam = local_ids[row + j];
            if ((unsigned)lam < (unsigned)L) atomicOr(&masks[lam * W + wd], bit);
        }
    }
    __syncthreads();
    int c = 0;
    if (tid < L)
        for (int w = 0; w < W; ++w) {
            pre[tid * W + w] = (uint16_t)c;
            c += __popc(masks[tid * W + w]);
        }
    scan_and_emit_tiles(c, L, T, topk, has_shared, BM, counts, offsets, tiles, ntiles, max_tiles, s_off);
    __syncthreads();
    // one thread per pair (up to four each, their ids loaded together; a wave
    // whose first pair is past the end loads nothing)
    const int np = T * topk;
    for (int p0 = 0; p0 < np; p0 += 4096) {
        int lp[4] = {-1, -1, -1, -1};
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (__builtin_amdgcn_readfirstlane(p0 + u * 1024 + tid) < np)
                lp[u] = local_ids[min(p0 + u * 1024 + tid, np - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = p0 + u * 1024 + tid;
            if (p >= np) break;
            const int t = p / topk, lam = lp[u];
            int pos = -1;
            if ((unsigned)lam < (unsigned)L) {
                const int w = t >> 5;
                pos = s_off[lam] + pre[lam * W + w] + __popc(masks[lam * W + w] & ((1u << (t & 31)) - 1u));
                perm[pos] = p;
            }
            inv[p] = pos;
        }
    }
}

__global__ __launch_bounds__(1024) void perm_small_kernel(
    const int32_t* __restrict__ local_ids, int T, int topk, int L, int has_shared, int BM,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int4* __restrict__ tiles,
    int32_t* __restrict__ ntiles, int max_tiles, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    extern __shared__ uint32_t masks[];                    // [L][ceil(T/32)] words, then the 16-bit prefix
    perm_small_body(local_ids, T, topk, L, has_shared, BM, counts, offsets, tiles, ntiles, max_tiles, perm, inv,
                    masks);
}

// ---------------------------------------------------------------------------
// Few tokens: exact routing in two launches.  With few rows the logits are
// computed in fp64 outright, so the selection needs no error bounds and no
// candidate re-scoring.  bf16 x bf16 products are exact in fp64; they are
// summed on the fp64 matrix cores (v_mfma_f64_16x16x4_f64), whose order is
// fixed by the hardware, then over the four waves of a workgroup in wave
// order, then over the K slices in slice order: the logits are deterministic
// fp64 sums of the exact products.
//
// v_mfma_f64_16x16x4_f64: lane l supplies A[l%16][l/16] and B[l/16][l%16]; item
// r of the result is D[l/16 + 4r][l%16] (checked on the hardware).  A = 16 gate
// rows, B = 16 token rows.  The reduction index is a free permutation: lane
// group q = l/16 loads 8 consecutive elements k0 + 8q .. +8 of its row and
// feeds element j to MFMA j, so one 16-byte load per lane and row serves
// eight MFMAs over 32 elements of K.
// ---------------------------------------------------------------------------
typedef double f64x4_t __attribute__((ext_vector_type(4)));
constexpr int kXMaxTG = 4;          // token groups of 16 per workgroup (64 tokens)
constexpr int kXWaves = 8;          // waves per workgroup, each a share of the K slice
constexpr int kXTokens = 128;       // exact routing up to this many tokens
constexpr double kXMaxMacs = 536870912.0;   // ... and up to T E d = 2^29 products

__device__ __forceinline__ double bf16_elem_f64(const u32x4_t& v, int j) {
    const uint32_t w = v[j >> 1];
    return (double)__uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

// partial logits [ks][T][E] over K slice ks: workgroup = 16 experts x 16 TG
// tokens; wave w takes the w-th quarter of the slice.
template <int TG, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void router_exact_logits_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ G, int T, int E, int d, int kslice,
    double* __restrict__ part) {
    __shared__ f64x4_t s_red[WAVES / 2][TG][64];
    __shared__ double s_out[16 * TG][17];                    // [token][expert], padded
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int e0 = blockIdx.x * 16, ks = blockIdx.y, t0 = blockIdx.z * (16 * TG);
    const int i = lane & 15, q = lane >> 4;
    // rows past E or T repeat the last row; their results are not stored
    const uint16_t* gp = G + (size_t)min(e0 + i, E - 1) * d + 8 * q;
    const uint16_t* xp[TG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) xp[tg] = X + (size_t)min(t0 + 16 * tg + i, T - 1) * d + 8 * q;
    const int wlen = kslice / WAVES;                         // a multiple of 32
    const int kb = ks * kslice + wave * wlen, ke = min(kb + wlen, d);
    f64x4_t acc[TG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) acc[tg] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    u32x4_t ga{0u, 0u, 0u, 0u}, xb[TG];
    if (kb < ke) {
        ga = *reinterpret_cast<const u32x4_t*>(gp + kb);
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) xb[tg] = *reinterpret_cast<const u32x4_t*>(xp[tg] + kb);
    }
    for (int k0 = kb; k0 < ke; k0 += 32) {
        const u32x4_t gc = ga;
        u32x4_t xc[TG];
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) xc[tg] = xb[tg];
        if (k0 + 32 < ke) {                                  // next step's loads go out first
            ga = *reinterpret_cast<const u32x4_t*>(gp + k0 + 32);
#pragma unroll
            for (int tg = 0; tg < TG; ++tg) xb[tg] = *reinterpret_cast<const u32x4_t*>(xp[tg] + k0 + 32);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const double av = bf16_elem_f64(gc, j);
#pragma unroll
            for (int tg = 0; tg < TG; ++tg)
                acc[tg] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bf16_elem_f64(xc[tg], j), acc[tg], 0, 0, 0);
        }
    }
    // the waves' sums meet in a fixed pairwise tree: at each level the upper
    // half of the remaining waves hands its sums to the lower half
#pragma unroll
    for (int h = WAVES / 2; h >= 1; h >>= 1) {
        if (wave >= h && wave < 2 * h) {
#pragma unroll
            for (int tg = 0; tg < TG; ++tg) s_red[wave - h][tg][lane] = acc[tg];
        }
        __syncthreads();
        if (wave < h) {
#pragma unroll
            for (int tg = 0; tg < TG; ++tg) acc[tg] += s_red[wave][tg][lane];
        }
        __syncthreads();
    }
    if (wave == 0) {
#pragma unroll
        for (int tg = 0; tg < TG; ++tg)
#pragma unroll
            for (int r = 0; r < 4; ++r) s_out[16 * tg + i][q + 4 * r] = acc[tg][r];
    }
    __syncthreads();
    // each token's 16 experts are 128 contiguous bytes of the partial row
    for (int c = tid; c < 16 * TG * 16; c += 64 * WAVES) {
        const int tt = c >> 4, ee = c & 15;
        if (t0 + tt < T && e0 + ee < E) part[((size_t)ks * T + t0 + tt) * E + e0 + ee] = s_out[tt][ee];
    }
}

// Order-preserving 64-bit key of an fp64 value (+0 and -0 share a key: the
// value is canonicalised first); 0 is below every key.
__device__ __forceinline__ uint64_t f64_key(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v + 0.0);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// top-k of token t: logits = the K-slice partials added in slice order; wave 0
// takes k rounds of (the largest remaining key, then the lowest id holding it);
// softmax over the k in fp64.  Experts e = lane + 64 s, s < EPL.
template <int EPL>
__global__ __launch_bounds__(1024) void router_exact_select_kernel(
    const double* __restrict__ part, int T, int E, int KS, int topk, int offset, int L,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, int32_t* __restrict__ local_ids) {
    __shared__ double s_val[kMaxExperts];
    __shared__ int32_t s_id[32];
    __shared__ double s_sc[32];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = blockIdx.x;
    if (tid < E) {
        double pv[kMaxKS];
#pragma unroll
        for (int sl = 0; sl < kMaxKS; ++sl) pv[sl] = part[((size_t)min(sl, KS - 1) * T + t) * E + tid];
        double v = pv[0];
#pragma unroll
        for (int sl = 1; sl < kMaxKS; ++sl)
            if (sl < KS) v += pv[sl];
        s_val[tid] = v;
    }
    __syncthreads();
    if (wave != 0) return;
    uint64_t key[EPL];
#pragma unroll
    for (int sl = 0; sl < EPL; ++sl) {
        const int e = lane + 64 * sl;
        key[sl] = e < E ? f64_key(s_val[e]) : 0ull;
    }
    for (int r = 0; r < topk; ++r) {
        uint64_t m = 0;
#pragma unroll
        for (int sl = 0; sl < EPL; ++sl) m = key[sl] > m ? key[sl] : m;
        const uint64_t M = wave_max_u64(m);
        uint32_t c = 0;                                  // 0xFFFFFFFF - id: the max is the lowest id
#pragma unroll
        for (int sl = EPL - 1; sl >= 0; --sl)
            if (key[sl] == M) c = 0xFFFFFFFFu - (uint32_t)(lane + 64 * sl);
        const int id = (int)(0xFFFFFFFFu - wave_max_u32(c));
#pragma unroll
        for (int sl = 0; sl < EPL; ++sl)
            if (lane + 64 * sl == id) key[sl] = 0;
        if (lane == 0) {
            s_id[r] = id;
            s_sc[r] = s_val[id];
        }
    }
    __builtin_amdgcn_wave_barrier();                     // (a wave's LDS accesses complete in order)
    const double my = lane < topk ? s_sc[lane] : 0.0;
    const double z = lane < topk ? exp(my - s_sc[0]) : 0.0;
    const double zs = wave_sum_f64(z);
    if (lane < topk) {
        const int my_id = s_id[lane];
        const size_t o = (size_t)t * topk + lane;
        topk_ids[o] = my_id;
        topk_w[o] = (float)(z / zs);
        const int lam = my_id - offset;
        local_ids[o] = (lam >= 0 && lam < L) ? lam : -1;
    }
}

// ---------------------------------------------------------------------------
// At most kFuseTokens tokens and kFuseItems (token, expert) logits: the exact
// selection and the permutation in one workgroup (one launch after the logits
// instead of two).  The T x E logits are the slice partials added in slice
// order, as in router_exact_select_kernel (two items' loads in flight per
// thread), kept in LDS; wave t then selects for token t exactly as that
// kernel's wave 0 does; then the whole workgroup runs the permutation of
// perm_small_kernel.  One CU then reads all T x E x (K slices) partials, so the
// fusion pays only while they are few.  Measured on the 320-expert shard
// (routing stage time, 16 K slices): T = 1 15.7 -> 14.5 us, T = 2 15.9 -> 15.3;
// T = 6 16.5 -> 18.1 and T = 16 17.3 -> 26.1 (slower); on the 16-expert layer
// (one K slice) at T = 16: 13.3 -> 12.4 us.
// ---------------------------------------------------------------------------
constexpr int kFuseTokens = 16;
constexpr int kFuseItems = 640;             // token-expert logits

template <int EPL>
__global__ __launch_bounds__(1024) void router_exact_finish_kernel(RouterArgs r, PermArgs q) {
    extern __shared__ __attribute__((aligned(16))) unsigned char fl[];
    double* const s_val = reinterpret_cast<double*>(fl);                              // [T][E]
    uint32_t* const masks = reinterpret_cast<uint32_t*>(fl + (size_t)r.T * r.E * 8);   // [L][ceil(T/32)] + prefix
    __shared__ int32_t s_id[kFuseTokens][32];
    __shared__ double s_sc[kFuseTokens][32];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = r.T, E = r.E, KS = r.KS, topk = r.topk;
    const int n = T * E;
    for (int i0 = tid; i0 < n; i0 += 2048) {
        double pv[2][kMaxKS];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = min(i0 + h * 1024, n - 1);
            const int t = i / E, e = i - t * E;
#pragma unroll
            for (int sl = 0; sl < kMaxKS; ++sl) pv[h][sl] = r.xpart[((size_t)min(sl, KS - 1) * T + t) * E + e];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = i0 + h * 1024;
            if (i < n) {
                double v = pv[h][0];
#pragma unroll
                for (int sl = 1; sl < kMaxKS; ++sl)
                    if (sl < KS) v += pv[h][sl];
                s_val[i] = v;
            }
        }
    }
    __syncthreads();
    if (wave < T) {
        const int t = wave;
        const double* val = s_val + (size_t)t * E;
        uint64_t key[EPL];
#pragma unroll
        for (int sl = 0; sl < EPL; ++sl) {
            const int e = lane + 64 * sl;
            key[sl] = e < E ? f64_key(val[e]) : 0ull;
        }
        for (int rr = 0; rr < topk; ++rr) {
            uint64_t m = 0;
#pragma unroll
            for (int sl = 0; sl < EPL; ++sl) m = key[sl] > m ? key[sl] : m;
            const uint64_t M = wave_max_u64(m);
            uint32_t c = 0;                              // 0xFFFFFFFF - id: the max is the lowest id
#pragma unroll
            for (int sl = EPL - 1; sl >= 0; --sl)
                if (key[sl] == M) c = 0xFFFFFFFFu - (uint32_t)(lane + 64 * sl);
            const int id = (int)(0xFFFFFFFFu - wave_max_u32(c));
#pragma unroll
            for (int sl = 0; sl < EPL; ++sl)
                if (lane + 64 * sl == id) key[sl] = 0;
            if (lane == 0) {
                s_id[t][rr] = id;
                s_sc[t][rr] = val[id];
            }
        }
        __builtin_amdgcn_wave_barrier();                 // (a wave's LDS accesses complete in order)
        const double my = lane < topk ? s_sc[t][lane] : 0.0;
        const double z = lane < topk ? exp(my - s_sc[t][0]) : 0.0;
        const double zs = wave_sum_f64(z);
        if (lane < topk) {
            const int my_id = s_id[t][lane];
            const size_t o = (size_t)t * topk + lane;
            r.topk_ids[o] = my_id;
            r.topk_w[o] = (float)(z / zs);
            const int lam = my_id - r.offset;
            r.local_ids[o] = (lam >= 0 && lam < r.L) ? lam : -1;
        }
    }
    __syncthreads();                                     // the local ids are visible to the workgroup
    perm_small_body(q.local_ids, T, topk, q.L, q.has_shared, q.BM, q.counts, q.offsets, q.tiles, q.ntiles,
                    q.max_tiles, q.perm, q.inv, masks);
}

// ---------------------------------------------------------------------------
// P3: scatter pair ids into the permutation; inverse map pair -> row (-1 dropped).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void perm_scatter_kernel(
    const int32_t* __restrict__ local_ids, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ block_bases, const int32_t* __restrict__ offsets, int T, int topk, int L,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= T * topk) return;
    const int t = p / topk;
    const int lam = local_ids[p];
    int pos = -1;
    if (lam >= 0) {
        const int blk = t / kPermBlock;
        pos = offsets[lam] + block_bases[(size_t)blk * L + lam] + rank[p];
        perm[pos] = p;
    }
    inv[p] = pos;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
int router_ksplit(int T, int E, int d) {
    // Enough slices for ~512 workgroups of the 64 x 64 kernel; for the wide
    // kernel (one workgroup per 64 tokens) ~256; for 512..1023 tokens ~192,
    // since the four-wave select kernel loads the slices in batches of four
    // (T = 512: 13 -> 5 slices, logits 11.2 -> 12.5 us, select 22.6 -> 18.8 us;
    // T = 768: 12.5 -> 14.5 and 29.0 -> 24.4 us; 128 measured worse at 768).
    int base = router_wide(T, E) ? (T + kWideTok - 1) / kWideTok
                                 : ((T + kR1Tile - 1) / kR1Tile) * ((E + kR1Tile - 1) / kR1Tile);
    const int want = router_wide(T, E) ? 256 : (T >= kWideSelectTokens && T < kSplitSelectTokens ? 192 : 512);
    if (base < 1) return 1;                      // empty batch
    int ks = (want + base - 1) / base;
    int maxks = d / 256 > 0 ? d / 256 : 1;
    if (maxks > kMaxKS) maxks = kMaxKS;
    if (ks > maxks) ks = maxks;
    if (ks < 1) ks = 1;
    return ks;
}

hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
    const int KS = a.KS;
    const int kslice = ((a.d / KS + kR1BK - 1) / kR1BK) * kR1BK;
    if (router_wide(a.T, a.E)) {
        const hipError_t e = allow_dynamic_lds<router_logits_wide_kernel<kWideTok>>(kWideLds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(router_logits_wide_kernel<kWideTok>, dim3((a.T + kWideTok - 1) / kWideTok, KS), dim3(512),
                           kWideLds, s, a.X, a.G, a.T, a.E, a.d, kslice, a.part, a.xn2, a.gn2);
    } else {
        dim3 g1((a.T + kR1Tile - 1) / kR1Tile, (a.E + kR1Tile - 1) / kR1Tile, KS);
        hipLaunchKernelGGL(router_logits_kernel, g1, dim3(256), 0, s, a.X, a.G, a.T, a.E, a.d, kslice,
                           a.part, a.xn2, a.gn2);
    }
    if (a.T >= kWideSelectTokens) {
        // many tokens: one wave per token (throughput)
        if (a.T < kSplitSelectTokens) {
            // few tokens for a wave each: every token's K chunks split over a workgroup
            dim3 g2(a.T);
            auto k = a.E <= 128 ? router_select_wave_kernel<2, kWTok>
                     : a.E <= 320 ? router_select_wave_kernel<5, kWTok>
                     : a.E <= 512 ? router_select_wave_kernel<8, kWTok>
                                  : router_select_wave_kernel<kMaxExperts / 64, kWTok>;
            hipLaunchKernelGGL(k, g2, dim3(64 * kWTok), 0, s, a.X, a.G, a.part, a.xn2, a.gn2, a.T, a.E, a.d, KS,
                               a.topk, a.offset, a.L, a.topk_ids, a.topk_w, a.local_ids);
        } else {
            dim3 g2((a.T + kWTok - 1) / kWTok);
            auto k = a.E <= 128 ? router_select_wave_kernel<2, 1>
                     : a.E <= 320 ? (a.T >= kOccSelectTokens ? router_select_wave_kernel<5, 1, 4>
                                                              : router_select_wave_kernel<5, 1>)
                     : a.E <= 512 ? router_select_wave_kernel<8, 1>
                                  : router_select_wave_kernel<kMaxExperts / 64, 1>;
            hipLaunchKernelGGL(k, g2, dim3(64 * kWTok), 0, s, a.X, a.G, a.part, a.xn2, a.gn2, a.T, a.E, a.d, KS,
                               a.topk, a.offset, a.L, a.topk_ids, a.topk_w, a.local_ids);
        }
    } else {
        // few tokens: a workgroup per token (latency)
        dim3 g2(a.T);
        auto k = a.E <= 128 ? router_select_kernel<2>
                 : a.E <= 320 ? router_select_kernel<5>
                 : a.E <= 512 ? router_select_kernel<8>
                              : router_select_kernel<kMaxExperts / 64>;
        hipLaunchKernelGGL(k, g2, dim3(kSelThreads), 0, s, a.X, a.G, a.part, a.xn2, a.gn2, a.T, a.E, a.d, KS,
                           a.topk, a.offset, a.L, a.topk_ids, a.topk_w, a.local_ids);
    }
    return hipGetLastError();
}

bool router_exact(int T, int E, int d) {
    return T >= 1 && T <= kXTokens && (double)T * E * d <= kXMaxMacs;
}

// K slices of the exact logits: enough workgroups for the chip (about 320),
// at most kMaxKS, each slice at least 32 elements per wave.
// K slices of the exact logits: enough for ~640 workgroups, at most 16 (on the
// 320-expert layer: 16 slices for every T <= 128; against a 320-workgroup
// target, T = 65..128 took 8 and routed 2 us slower at T = 128).
int router_exact_ksplit(int T, int E, int d) {
    const int base = ((E + 15) / 16) * ((T + 16 * kXMaxTG - 1) / (16 * kXMaxTG));
    int ks = (640 + base - 1) / base;
    if (ks > kMaxKS) ks = kMaxKS;
    if (ks > d / (32 * kXWaves)) ks = d / (32 * kXWaves);
    return ks < 1 ? 1 : ks;
}

static hipError_t launch_exact_logits(const RouterArgs& a, hipStream_t s) {
    if (!router_exact(a.T, a.E, a.d) || a.KS < 1 || a.KS > kMaxKS) return hipErrorInvalidValue;
    constexpr int W = kXWaves;
    const int kslice = ((a.d + a.KS - 1) / a.KS + 32 * W - 1) / (32 * W) * (32 * W);
    const int tg = a.T <= 16 ? 1 : (a.T <= 32 ? 2 : kXMaxTG);
    const dim3 g1((a.E + 15) / 16, a.KS, (a.T + 16 * tg - 1) / (16 * tg));
    if (tg == 1)
        hipLaunchKernelGGL((router_exact_logits_kernel<1, W>), g1, dim3(64 * W), 0, s, a.X, a.G, a.T, a.E, a.d, kslice,
                           a.xpart);
    else if (tg == 2)
        hipLaunchKernelGGL((router_exact_logits_kernel<2, W>), g1, dim3(64 * W), 0, s, a.X, a.G, a.T, a.E, a.d, kslice,
                           a.xpart);
    else
        hipLaunchKernelGGL((router_exact_logits_kernel<kXMaxTG, W>), g1, dim3(64 * W), 0, s, a.X, a.G, a.T, a.E, a.d,
                           kslice, a.xpart);
    return hipSuccess;
}

hipError_t launch_route_exact(const RouterArgs& a, hipStream_t s) {
    const hipError_t e = launch_exact_logits(a, s);
    if (e != hipSuccess) return e;
    auto k = a.E <= 128 ? router_exact_select_kernel<2>
             : a.E <= 320 ? router_exact_select_kernel<5>
             : a.E <= 512 ? router_exact_select_kernel<8>
                          : router_exact_select_kernel<kMaxExperts / 64>;
    hipLaunchKernelGGL(k, dim3(a.T), dim3(1024), 0, s, a.xpart, a.T, a.E, a.KS, a.topk, a.offset, a.L, a.topk_ids,
                       a.topk_w, a.local_ids);
    return hipGetLastError();
}

static size_t route_fused_lds(int T, int E, int L) {
    return (size_t)T * E * 8 + perm_small_lds(T, L);
}

bool route_fused_ok(int T, int E, int d, int L) {
    return router_exact(T, E, d) && T <= kFuseTokens && T * E <= kFuseItems && L <= 1024 &&
           route_fused_lds(T, E, L) <= 65536;
}

hipError_t launch_route_exact_fused(const RouterArgs& a, const PermArgs& q, hipStream_t s) {
    if (!route_fused_ok(a.T, a.E, a.d, a.L) || q.T != a.T || q.L != a.L || q.topk != a.topk ||
        q.local_ids != a.local_ids)
        return hipErrorInvalidValue;
    const hipError_t e = launch_exact_logits(a, s);
    if (e != hipSuccess) return e;
    auto k = a.E <= 128 ? router_exact_finish_kernel<2>
             : a.E <= 320 ? router_exact_finish_kernel<5>
             : a.E <= 512 ? router_exact_finish_kernel<8>
                          : router_exact_finish_kernel<kMaxExperts / 64>;
    hipLaunchKernelGGL(k, dim3(1), dim3(1024), route_fused_lds(a.T, a.E, a.L), s, a, q);
    return hipGetLastError();
}

hipError_t launch_permute(const PermArgs& a, hipStream_t s) {
    const int nblk = (a.T + kPermBlock - 1) / kPermBlock;
    const size_t lds = (size_t)a.L * (kPermBlock / 32) * sizeof(uint32_t);
    const size_t small_lds = perm_small_lds(a.T, a.L);
    if (a.T <= kPermSmallTokens && small_lds <= (size_t)kPermSmallLds) {
        // one workgroup (one launch) when the bitmask fits
        hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(1024), small_lds, s, a.local_ids, a.T, a.topk, a.L,
                           a.has_shared, a.BM, a.counts, a.offsets, a.tiles, a.ntiles, a.max_tiles, a.perm,
                           a.inv);
        return hipGetLastError();
    }
    if (nblk > 0)
        hipLaunchKernelGGL(perm_block_kernel, dim3(nblk), dim3(kPermBlock), lds, s, a.local_ids, a.T,
                           a.topk, a.L, a.block_counts, a.rank);
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, s, a.block_counts, nblk, a.L, a.T,
                       a.topk, a.has_shared, a.BM, a.counts, a.offsets, a.tiles, a.ntiles, a.max_tiles);
    const int np = a.T * a.topk;
    if (np > 0)
        hipLaunchKernelGGL(perm_scatter_kernel, dim3((np + 255) / 256), dim3(256), 0, s, a.local_ids,
                           a.rank, a.block_counts, a.offsets, a.T, a.topk, a.L, a.perm, a.inv);
    return hipGetLastError();
}

}  // namespace moe
