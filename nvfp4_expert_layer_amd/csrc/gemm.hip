// Weighted combine of the expert outputs (gfx950):
//   out[t] = sum_j w_tj Y[row(t, j)] (kept pairs, slot order) + Y[shared row of t],
// a fixed summation order, so the output is deterministic.  The output is this
// shard's partial sum: the page "Serving Solar Open 2 on DGX Spark", section "수정
// 사항 › b12x에서의 Expert Parallelism 구현 추가".
#include "device_common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// combine: one thread per 8 output columns of a token.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const int per_row = a.d / 8;
    if (idx >= (long long)a.T * per_row) return;
    const int t = (int)(idx / per_row), c0 = (int)(idx % per_row) * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // the shared expert's row needs no slot lookup: its load is issued first and
    // overlaps the slots' round trips (it is still added last)
    u32x4_t ysh = {0u, 0u, 0u, 0u};
    if (a.has_shared)
        ysh = *reinterpret_cast<const u32x4_t*>(a.Y + ((size_t)a.T * a.topk + t) * a.d + c0);
    // slots in groups of 8: the group's row indices and weights first, then its
    // expert rows, so each group costs two memory round trips, not 2 per slot;
    // the sum still runs in slot order
    for (int j0 = 0; j0 < a.topk; j0 += 8) {
        int row[8];
        float w[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int j = j0 + q;
            row[q] = j < a.topk ? a.inv[(size_t)t * a.topk + j] : -1;
            w[q] = j < a.topk ? a.topk_w[(size_t)t * a.topk + j] : 0.f;
        }
        u32x4_t y[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (row[q] >= 0) y[q] = *reinterpret_cast<const u32x4_t*>(a.Y + (size_t)row[q] * a.d + c0);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (row[q] < 0) continue;
            const uint32_t yw[4] = {y[q].x, y[q].y, y[q].z, y[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[2 * e] = fmaf(w[q], bf16_bits_to_f32(yw[e] & 0xFFFFu), s[2 * e]);
                s[2 * e + 1] = fmaf(w[q], bf16_bits_to_f32(yw[e] >> 16), s[2 * e + 1]);
            }
        }
    }
    if (a.has_shared) {
        const uint32_t yw[4] = {ysh.x, ysh.y, ysh.z, ysh.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s[2 * e] = fmaf(1.0f, bf16_bits_to_f32(yw[e] & 0xFFFFu), s[2 * e]);
            s[2 * e + 1] = fmaf(1.0f, bf16_bits_to_f32(yw[e] >> 16), s[2 * e + 1]);
        }
    }
    u32x4_t o;
    o.x = f32x2_to_bf16x2(s[0], s[1]);
    o.y = f32x2_to_bf16x2(s[2], s[3]);
    o.z = f32x2_to_bf16x2(s[4], s[5]);
    o.w = f32x2_to_bf16x2(s[6], s[7]);
    *reinterpret_cast<u32x4_t*>(a.out + (size_t)t * a.d + c0) = o;
}

// ---------------------------------------------------------------------------
int gemm_bm(int path, int T, int topk, int E, bool packed_mid) {
    return path == 1 ? dec_rows(T, topk, E) : (path == 3 ? (packed_mid ? mid_rows_packed() : mid_rows(T, topk, E)) : pf_rows());
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    long long n = (long long)a.T * (a.d / 8);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
