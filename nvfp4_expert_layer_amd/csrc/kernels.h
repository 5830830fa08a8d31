// Internal interface between the host engine and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace moe {

struct ExpertWeights {            // device pointers, n experts, expert-major
    const uint8_t* w13;           // [n][2F][d/2]
    const uint8_t* w13_s;         // [n][2F][d/16]
    const float* g13;             // [n]
    const uint8_t* w2;            // [n][d][F/2]
    const uint8_t* w2_s;          // [n][d][F/16]
    const float* g2;              // [n]
};

struct RouterArgs {
    const uint16_t* X;            // bf16 [T][d]
    const uint16_t* G;            // bf16 [E][d]
    int T, E, d, KS, topk, offset, L;
    float* part;                  // [KS][T][E]  (certified routing)
    double* xpart;                // [KS][T][E]  (exact routing)
    double* xn2;                  // [KS][T]
    double* gn2;                  // [KS][E]
    int32_t* topk_ids;            // [T][k]
    float* topk_w;                // [T][k]
    int32_t* local_ids;           // [T][k]
};

struct PermArgs {
    const int32_t* local_ids;     // [T][k]
    int T, topk, L, has_shared, BM, max_tiles;
    int32_t* block_counts;        // [nblk][L]  (becomes per-block bases)
    int32_t* rank;                // [T][k]
    int32_t* counts;              // [L]
    int32_t* offsets;             // [L+1]
    int4* tiles;                  // [max_tiles]
    int32_t* ntiles;              // [1]
    int32_t* perm;                // [T*k]
    int32_t* inv;                 // [T*k]
};

struct GemmArgs {
    int T, d, F, topk, L, mode, E;
    float a1g, a2g;               // activation global scales of the GEMM1 / GEMM2 inputs
                                  //   (1 unless static W4A4); GEMM inputs hold code * scale
    const int32_t* perm;          // [T*k]
    const int4* tiles;            // (group, row_begin, row_end, index within the group)
    const int32_t* ntiles;
    int max_tiles;
    const uint16_t* hidden;       // bf16 [T][d]
    const uint16_t* hq;           // W4A4: hidden NVFP4-quantized, exact dequantized [T][d]
                                  //   (bf16 on the decode path, f16 on the tiled and mid paths)
    ExpertWeights local, shared;
    uint16_t* act;                // SwiGLU output [R][F]: bf16; W4A4: exact dequantized NVFP4
                                  //   values, bf16 (decode path) or f16 (tiled and mid paths)
    uint16_t* Y;                  // expert outputs, bf16 [R][d];  R = T*k + T
    // W4A4 on the tiled path when d and F are multiples of 256, and on the dense
    // weight-streaming path when they are also at most 8192 (packed != 0):
    // activations travel as NVFP4 codes and E4M3 block scales instead of 16-bit
    // values (in the hq and act regions)
    int packed;
    const uint8_t* hq_codes;      // [T][d/2]
    const uint8_t* hq_scales;     // [T][d/16]
    uint8_t* act_codes;           // [R][F/2]
    uint8_t* act_scales;          // [R][F/16]
};

// The small-batch layer in one launch (T <= 16): workspace regions and the problem.
struct MicroArgs {
    int T, d, F, E, topk, offset, L, has_shared, mode;
    float a1g, a2g;
    const uint16_t* X;            // bf16 [T][d]
    const uint16_t* G;            // bf16 [E][d]
    ExpertWeights local, shared;
    unsigned* bar;                // [2]: grid barrier counter, error word (zeroed per launch)
    double* logits;               // [T][E]
    uint16_t* hq;                 // W4A4: [T][d] bf16 quantize-dequantized token rows
    uint16_t* act;                // [T*k + T][F] bf16
    uint16_t* Y;                  // [T*k + T][d] bf16
    uint16_t* out;                // [T][d]
};
constexpr int kMaxExpertsMicro = 1024;

struct CombineArgs {
    int T, d, topk, has_shared;
    const float* topk_w;          // [T][k]
    const int32_t* inv;           // [T][k] row of each pair, -1 dropped
    const uint16_t* Y;            // bf16 [R][d]
    uint16_t* out;                // bf16 [T][d]
};

int router_ksplit(int T, int E, int d);
hipError_t launch_router(const RouterArgs& a, hipStream_t s);
bool router_exact(int T, int E, int d);           // exact fp64 logits for this batch
int router_exact_ksplit(int T, int E, int d);
hipError_t launch_route_exact(const RouterArgs& a, hipStream_t s);
// few tokens: exact logits, then selection and permutation in one launch
bool route_fused_ok(int T, int E, int d, int L);
hipError_t launch_route_exact_fused(const RouterArgs& a, const PermArgs& q, hipStream_t s);
hipError_t launch_permute(const PermArgs& a, hipStream_t s);
hipError_t launch_quantize_act(const uint16_t* x, int R, int C, float g, uint8_t* codes, uint8_t* scales,
                               hipStream_t s);
hipError_t launch_fake_quant_act(const uint16_t* x, int R, int C, float g, uint16_t* out, bool f16_out,
                                 hipStream_t s);
hipError_t launch_quantize_weights(const uint16_t* w, int n, int R, int C, uint8_t* codes,
                                   uint8_t* scales, float* global, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
hipError_t launch_prepare_rows(const uint8_t* src, uint8_t* dst, int n, int rows, int row_bytes, bool swap_halves,
                               hipStream_t s);
hipError_t launch_prepare_global(const float* src, float* dst, int n, bool inverse, hipStream_t s);
int gemm_bm(int path, int T, int topk, int E, bool packed_mid);   // rows per tile of the chosen path
int pf_rows();                                    // rows per tile of the prefill GEMMs
bool pf_packed_ok(int d, int F);                  // W4A4 packed-activation GEMMs apply
int dec_rows(int T, int topk, int E);
hipError_t launch_gemm1(const GemmArgs& a, int path, hipStream_t s);
hipError_t launch_gemm2(const GemmArgs& a, int path, hipStream_t s);
hipError_t launch_dec_gemm1(const GemmArgs& a, hipStream_t s);
hipError_t launch_dec_gemm2(const GemmArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
bool micro_ok(int T, int d, int F, int E, int topk, int L);   // the one-launch small-batch layer applies
int micro_lds_bytes(int d, int F);
hipError_t launch_micro(const MicroArgs& a, int ncu, hipStream_t s);
bool mid_ok(int d, int F);                        // dense weight-streaming kernels apply
bool mid_packed_ok(int d, int F);                 // ... with W4A4 activations as NVFP4
int mid_rows(int T, int topk, int E);             // rows per tile of the dense weight-streaming path
int mid_rows_packed();                            // ... with W4A4 activations as NVFP4
hipError_t launch_mid_gemm1(const GemmArgs& a, hipStream_t s);
hipError_t launch_mid_gemm2(const GemmArgs& a, hipStream_t s);

// Raise kernel Kern's dynamic-LDS limit to `bytes` on the current device when
// that is above the 64 KB default; the attribute is per device, so the largest
// size set so far is kept per device and each is set once.
template <auto Kern>
inline hipError_t allow_dynamic_lds(int bytes) {
    static std::atomic<int> allowed[64];
    if (bytes <= 65536) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (allowed[dev].load(std::memory_order_relaxed) >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) allowed[dev].store(bytes, std::memory_order_relaxed);
    return e;
}

}  // namespace moe
