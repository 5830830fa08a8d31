// Router, shard filter and permutation kernels (gfx950).
//
// Routing (the page "Serving Solar Open 2 on DGX Spark", section "Solar Open 2
// 개요": routed experts, top-k, one shared expert; section "수정 사항 › b12x에서의
// Expert Parallelism 구현 추가": routing is global, the kernel maps the globally
// routed id to a shard-relative index and drops pairs outside the shard):
//   logits over ALL experts, top-k by logit (ties -> lower id), weights = softmax
//   over the k selected logits, local id = id - offset if inside [0, L) else -1.
//
// Exactness of the selection.  Logits are first computed with bf16 MFMA (the
// bf16 x bf16 products are exact in fp32; the accumulation rounds).  For any
// order of at most n fp32 additions with relative error <= u' each (u' = 2^-23
// covers round-to-nearest and truncation), |lhat - l| <= gamma_n * sum_k |x_k g_k|
// <= gamma_n * ||x||_2 * ||g_e||_2 (Cauchy-Schwarz), gamma_n = n u' / (1 - n u'),
// plus d * 2^-126 for products that fall below the fp32 normal range.  With
// lower/upper bounds lo_e, hi_e, let lowk be the k-th largest lo.  An expert with
// hi_e < lowk has at least k experts certainly above it, so it cannot be in the
// top-k.  Every other expert (the candidates) is re-scored in fp64 (exact
// products, fixed summation order) and the top-k is taken among them.
//
// Permutation: pairs grouped by local expert, stable by token.  Per block of 256
// tokens an LDS bitmask per local expert records which tokens chose it; a pair's
// rank inside its block is a popcount of the lower bits, so the order is
// deterministic without sorting.  A single-workgroup scan turns per-block counts
// into per-block bases, counts, offsets and the GEMM tile table.
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

__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ G, int T, int E, int d,
    int kslice, float* __restrict__ part, double* __restrict__ xn2, double* __restrict__ gn2) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[kR1Tile][kR1BK + kR1Pad];
    __shared__ __attribute__((aligned(16))) uint16_t gs[kR1Tile][kR1BK + kR1Pad];
    const int t0 = blockIdx.x * kR1Tile, e0 = blockIdx.y * kR1Tile, ks = blockIdx.z;
    const int kbeg = ks * kslice, kend = min(d, kbeg + kslice);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // wave layout 2x2: wave (wm, wn) owns tokens [32 wm, +32) x experts [32 wn, +32)
    const int wm = wave >> 1, wn = wave & 1;
    f32x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // squared norms: thread tid < 64 -> token row t0+tid; 64..127 -> expert row e0+tid-64
    double nrm = 0.0;
    for (int k0 = kbeg; k0 < kend; k0 += kR1BK) {
        // stage 64 rows x 64 bf16 of X and of G: 512 16-byte chunks each, 2 per thread
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            int chunk = tid + c * 256;          // 0..511
            int r = chunk >> 3, cc = (chunk & 7) * 8;
            u32x4_t vx = {0u, 0u, 0u, 0u}, vg = {0u, 0u, 0u, 0u};
            if (t0 + r < T) vx = *reinterpret_cast<const u32x4_t*>(X + (size_t)(t0 + r) * d + k0 + cc);
            if (e0 + r < E) vg = *reinterpret_cast<const u32x4_t*>(G + (size_t)(e0 + r) * d + k0 + cc);
            *reinterpret_cast<u32x4_t*>(&xs[r][cc]) = vx;
            *reinterpret_cast<u32x4_t*>(&gs[r][cc]) = vg;
        }
        __syncthreads();
        if (tid < 128) {
            const uint16_t* row = tid < 64 ? xs[tid] : gs[tid - 64];
            bool want = tid < 64 ? (blockIdx.y == 0) : (blockIdx.x == 0);
            if (want) {
                for (int j = 0; j < kR1BK; ++j) {
                    double v = (double)bf16_bits_to_f32(row[j]);
                    nrm = fma(v, v, nrm);
                }
            }
        }
#pragma unroll
        for (int kk = 0; kk < kR1BK; kk += 32) {
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const bf16x8_t*>(&xs[wm * 32 + i * 16 + (lane & 15)][kk + (lane >> 4) * 8]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const bf16x8_t*>(&gs[wn * 32 + j * 16 + (lane & 15)][kk + (lane >> 4) * 8]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    float* out = part + (size_t)ks * T * E;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int t = t0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
                int e = e0 + wn * 32 + j * 16 + (lane & 15);
                if (t < T && e < E) out[(size_t)t * E + e] = acc[i][j][r];
            }
    if (tid < 64 && blockIdx.y == 0 && t0 + tid < T) xn2[(size_t)ks * T + t0 + tid] = nrm;
    if (tid >= 64 && tid < 128 && blockIdx.x == 0 && e0 + tid - 64 < E) gn2[(size_t)ks * E + e0 + tid - 64] = nrm;
}

// ---------------------------------------------------------------------------
// R2: certified top-k per token (one wave per token).
// ---------------------------------------------------------------------------
constexpr int kMaxExperts = 1024;
constexpr int kMaxKS = 16;          // split-K slices of the logits GEMM
constexpr int kSelWaves = 4;

__device__ __forceinline__ double dot_f64(const uint16_t* __restrict__ x, const uint16_t* __restrict__ g,
                                          int d, int lane) {
    // fp64 products of bf16 pairs are exact; a lane sums its elements in a fixed
    // order, then the wave reduces in a fixed tree.  Loads are issued 8 chunks at
    // a time so one latency covers d = 4096.
    double s = 0.0;
    for (int c0 = lane * 8; c0 < d; c0 += 512 * 8) {
        u32x4_t vx[8], vg[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = c0 + j * 512;
            const u32x4_t z = {0u, 0u, 0u, 0u};
            vx[j] = c < d ? *reinterpret_cast<const u32x4_t*>(x + c) : z;
            vg[j] = c < d ? *reinterpret_cast<const u32x4_t*>(g + c) : z;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t ax[4] = {vx[j].x, vx[j].y, vx[j].z, vx[j].w};
            const uint32_t ag[4] = {vg[j].x, vg[j].y, vg[j].z, vg[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s = fma((double)__uint_as_float(ax[q] << 16), (double)__uint_as_float(ag[q] << 16), s);
                s = fma((double)__uint_as_float(ax[q] & 0xFFFF0000u), (double)__uint_as_float(ag[q] & 0xFFFF0000u), s);
            }
        }
    }
    return wave_sum_f64(s);
}

// Wave-wide arg-max over `vals` (per-lane slots e = lane + 64 i), largest value,
// ties -> lowest index; returns the index (or -1 if all are -inf / taken).
template <int NS>
__device__ __forceinline__ int wave_argmax(const double (&vals)[NS], int E, int lane) {
    double best = -INFINITY;
    int bidx = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        int e = lane + 64 * i;
        if (e < E && (vals[i] > best || (vals[i] == best && e < bidx)) && vals[i] != -INFINITY) {
            best = vals[i];
            bidx = e;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        double ob = __shfl_xor(best, o, 64);
        int oi = __shfl_xor(bidx, o, 64);
        if (ob > best || (ob == best && oi < bidx)) { best = ob; bidx = oi; }
    }
    return bidx == 0x7FFFFFFF ? -1 : bidx;
}

template <int NS>
__global__ __launch_bounds__(64 * kSelWaves) void router_select_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ G, const float* __restrict__ part,
    const double* __restrict__ xn2, const double* __restrict__ gn2, int T, int E, int d, int KS,
    int topk, int offset, int L, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ local_ids) {
    // one workgroup per token: wave 0 bounds the logits and lists the candidates,
    // all waves re-score candidates in fp64, wave 0 selects and normalises.
    __shared__ int32_t s_cand[kMaxExperts];
    __shared__ double s_score[kMaxExperts];
    __shared__ int32_t s_ncand;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x;
    const uint16_t* xrow = X + (size_t)t * d;
    __shared__ double s_lo[kMaxExperts], s_hi[kMaxExperts];
    {
        // bounds for every expert, spread over the whole workgroup; the split-K
        // partial sums are loaded together (KS <= kMaxKS) and added in slice order
        const double u = 1.0 / 8388608.0;                  // bound factor gamma_n, n = d + KS, u' = 2^-23
        const double n = (double)(d + KS);
        const double gamma = n * u / (1.0 - n * u) * (1.0 + 1e-6);
        const double tiny = (double)d * 1.1754943508222875e-38;   // d * 2^-126
        double xv[kMaxKS];
#pragma unroll
        for (int s = 0; s < kMaxKS; ++s) xv[s] = s < KS ? xn2[(size_t)s * T + t] : 0.0;
        double xs2 = 0.0;
#pragma unroll
        for (int s = 0; s < kMaxKS; ++s) xs2 += xv[s];
        const double xnorm = sqrt(xs2) * (1.0 + 1e-12);
        for (int e = threadIdx.x; e < E; e += 64 * kSelWaves) {
            float pv[kMaxKS];
            double gv[kMaxKS];
#pragma unroll
            for (int s = 0; s < kMaxKS; ++s) {
                pv[s] = s < KS ? part[((size_t)s * T + t) * E + e] : 0.f;
                gv[s] = s < KS ? gn2[(size_t)s * E + e] : 0.0;
            }
            float lh = 0.f;
            double gs2 = 0.0;
#pragma unroll
            for (int s = 0; s < kMaxKS; ++s) { lh += pv[s]; gs2 += gv[s]; }
            const double beta = gamma * xnorm * (sqrt(gs2) * (1.0 + 1e-12)) + tiny;
            s_lo[e] = (double)lh - beta;
            s_hi[e] = (double)lh + beta;
        }
    }
    __syncthreads();
    if (wave == 0) {
        double lo[NS], hi[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int e = lane + 64 * i;
            lo[i] = e < E ? s_lo[e] : -INFINITY;
            hi[i] = e < E ? s_hi[e] : -INFINITY;
        }
        // lowk = k-th largest lower bound
        double tmp[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) tmp[i] = lo[i];
        int idx = -1;
        for (int r = 0; r < topk; ++r) {
            idx = wave_argmax<NS>(tmp, E, lane);
#pragma unroll
            for (int i = 0; i < NS; ++i)
                if (lane + 64 * i == idx) tmp[i] = -INFINITY;
        }
        double v = -INFINITY;
#pragma unroll
        for (int i = 0; i < NS; ++i)
            if (lane + 64 * i == idx) v = lo[i];
        const double lowk = __shfl(v, idx & 63, 64);
        // candidates (hi >= lowk), listed in increasing expert id
        int base = 0;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const bool c = lane + 64 * i < E && hi[i] >= lowk;
            const uint64_t m = __ballot(c);
            if (c) s_cand[base + __popcll(m & ((1ull << lane) - 1ull))] = lane + 64 * i;
            base += __popcll(m);
        }
        if (lane == 0) s_ncand = base;
    }
    __syncthreads();
    const int nc = s_ncand;
    for (int c = wave; c < nc; c += kSelWaves) {
        const int e = s_cand[c];
        const double sc = dot_f64(xrow, G + (size_t)e * d, d, lane);
        if (lane == 0) s_score[c] = sc;
    }
    __syncthreads();
    if (wave != 0) return;
    // top-k among candidates by (fp64 score desc, id asc): candidate slots c = lane + 64 i
    double sc[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int c = lane + 64 * i;
        sc[i] = c < nc ? s_score[c] : -INFINITY;
    }
    int my_id = -1;
    double my_score = 0.0, top_score = 0.0;
    for (int r = 0; r < topk; ++r) {
        const int idx = wave_argmax<NS>(sc, nc, lane);
        double v = -INFINITY;
#pragma unroll
        for (int i = 0; i < NS; ++i)
            if (lane + 64 * i == idx) { v = sc[i]; sc[i] = -INFINITY; }
        v = __shfl(v, idx & 63, 64);    // broadcast from the owner lane
        if (r == 0) top_score = v;
        if (lane == r) { my_id = s_cand[idx]; my_score = v; }
    }
    // softmax over the k selected fp64 scores
    const double z = lane < topk ? exp(my_score - top_score) : 0.0;
    const double zs = wave_sum_f64(z);
    if (lane < topk) {
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
// offsets, and the GEMM tile table (group, row_begin, row_end) with BM rows per
// tile.  Groups 0..L-1 are the local experts (rows [offsets[g], offsets[g+1])
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
            tiles[ext + i] = make_int4(tid, rb, min(rb + BM, exc + c), 0);
        }
    }
    if (tid == L - 1) {
        offsets[L] = exc + c;
        int n = ext + tc;
        if (has_shared) {
            const int base = T * topk;
            const int st = (T + BM - 1) / BM;
            for (int i = 0; i < st; ++i)
                tiles[n + i] = make_int4(L, base + i * BM, min(base + (i + 1) * BM, base + T), 0);
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
        for (int b = 0; b < nblk; ++b) {
            int c = block_counts[(size_t)b * L + tid];
            block_counts[(size_t)b * L + tid] = total;
            total += c;
        }
    }
    scan_and_emit_tiles(total, L, T, topk, has_shared, BM, counts, offsets, tiles, ntiles, max_tiles, nullptr);
}

// All three permutation steps in one workgroup, for T <= kPermBlock.
__global__ __launch_bounds__(1024) void perm_small_kernel(
    const int32_t* __restrict__ local_ids, int T, int topk, int L, int has_shared, int BM,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int4* __restrict__ tiles,
    int32_t* __restrict__ ntiles, int max_tiles, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    extern __shared__ uint32_t masks[];                    // [L][kPermBlock/32]
    __shared__ int32_t s_off[1024];
    constexpr int W = kPermBlock / 32;
    const int tid = threadIdx.x;
    for (int i = tid; i < L * W; i += 1024) masks[i] = 0u;
    __syncthreads();
    if (tid < T)
        for (int j = 0; j < topk; ++j) {
            const int lam = local_ids[(size_t)tid * topk + j];
            if (lam >= 0) atomicOr(&masks[lam * W + (tid >> 5)], 1u << (tid & 31));
        }
    __syncthreads();
    int c = 0;
    if (tid < L)
        for (int w = 0; w < W; ++w) c += __popc(masks[tid * W + w]);
    scan_and_emit_tiles(c, L, T, topk, has_shared, BM, counts, offsets, tiles, ntiles, max_tiles, s_off);
    __syncthreads();
    for (int p = tid; p < T * topk; p += 1024) {
        const int t = p / topk;
        const int lam = local_ids[p];
        int pos = -1;
        if (lam >= 0) {
            int r = 0;
            for (int w = 0; w < (t >> 5); ++w) r += __popc(masks[lam * W + w]);
            r += __popc(masks[lam * W + (t >> 5)] & ((1u << (t & 31)) - 1u));
            pos = s_off[lam] + r;
            perm[pos] = p;
        }
        inv[p] = pos;
    }
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
    int base = ((T + kR1Tile - 1) / kR1Tile) * ((E + kR1Tile - 1) / kR1Tile);
    if (base < 1) return 1;                      // empty batch
    int ks = (512 + base - 1) / base;
    int maxks = d / 256 > 0 ? d / 256 : 1;
    if (maxks > kMaxKS) maxks = kMaxKS;
    if (ks > maxks) ks = maxks;
    if (ks < 1) ks = 1;
    return ks;
}

hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
    const int KS = a.KS;
    const int kslice = ((a.d / KS + kR1BK - 1) / kR1BK) * kR1BK;
    dim3 g1((a.T + kR1Tile - 1) / kR1Tile, (a.E + kR1Tile - 1) / kR1Tile, KS);
    hipLaunchKernelGGL(router_logits_kernel, g1, dim3(256), 0, s, a.X, a.G, a.T, a.E, a.d, kslice,
                       a.part, a.xn2, a.gn2);
    dim3 g2(a.T);
    const int ns = (a.E + 63) / 64;
#define SEL(NSV)                                                                                       \
    hipLaunchKernelGGL(router_select_kernel<NSV>, g2, dim3(64 * kSelWaves), 0, s, a.X, a.G, a.part, \
                       a.xn2, a.gn2, a.T, a.E, a.d, KS, a.topk, a.offset, a.L, a.topk_ids, a.topk_w,   \
                       a.local_ids)
    if (ns <= 1) SEL(1);
    else if (ns <= 2) SEL(2);
    else if (ns <= 4) SEL(4);
    else if (ns <= 6) SEL(6);
    else if (ns <= 8) SEL(8);
    else if (ns <= 12) SEL(12);
    else SEL(16);
#undef SEL
    return hipGetLastError();
}

hipError_t launch_permute(const PermArgs& a, hipStream_t s) {
    const int nblk = (a.T + kPermBlock - 1) / kPermBlock;
    const size_t lds = (size_t)a.L * (kPermBlock / 32) * sizeof(uint32_t);
    if (nblk <= 1) {
        hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(1024), lds, s, a.local_ids, a.T, a.topk, a.L,
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
