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
    for (int j = 0; j < a.topk; ++j) {
        const int row = a.inv[(size_t)t * a.topk + j];
        if (row < 0) continue;
        const float w = a.topk_w[(size_t)t * a.topk + j];
        const f32x4_t* y = reinterpret_cast<const f32x4_t*>(a.Y + (size_t)row * a.d + c0);
        f32x4_t y0 = y[0], y1 = y[1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            s[q] = fmaf(w, y0[q], s[q]);
            s[4 + q] = fmaf(w, y1[q], s[4 + q]);
        }
    }
    if (a.has_shared) {
        const f32x4_t* y = reinterpret_cast<const f32x4_t*>(a.Y + ((size_t)a.T * a.topk + t) * a.d + c0);
        f32x4_t y0 = y[0], y1 = y[1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            s[q] += y0[q];
            s[4 + q] += y1[q];
        }
    }
    u32x4_t o;
    o.x = f32_to_bf16_rne(s[0]) | (f32_to_bf16_rne(s[1]) << 16);
    o.y = f32_to_bf16_rne(s[2]) | (f32_to_bf16_rne(s[3]) << 16);
    o.z = f32_to_bf16_rne(s[4]) | (f32_to_bf16_rne(s[5]) << 16);
    o.w = f32_to_bf16_rne(s[6]) | (f32_to_bf16_rne(s[7]) << 16);
    *reinterpret_cast<u32x4_t*>(a.out + (size_t)t * a.d + c0) = o;
}

// ---------------------------------------------------------------------------
int gemm_bm(int path, int T, int topk, int E) { return path == 1 ? dec_rows(T, topk, E) : pf_rows(); }

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    long long n = (long long)a.T * (a.d / 8);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
