// Host engine of the NVFP4 MoE layer: device-free validation, workspace
// planning, kernel-path dispatch and the C ABI declared in include/moe_nvfp4.h.
//
// The boundary follows the page "Serving Solar Open 2 on DGX Spark", section
// "수정 사항 › b12x에서의 Expert Parallelism 구현 추가": the shard is given by
// `local_expert_offset` and a count of local experts; the output is a per-shard
// partial sum; scale tensors of a shard may start at any expert; scratch comes
// from one caller-owned pool (the workspace) that every layer can reuse; the
// kernel path is chosen from the shard's expected local load, not the global one.
#include "../../include/moe_nvfp4.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return MOE_NVFP4_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// an activation global scale the fp32 quantizer arithmetic handles without
// overflow or underflow (6 g and 448 g stay finite and normal)
bool global_ok(float g) { return g >= 0x1p-100f && g <= 0x1p100f; }

// W4A4 in either form (the kernels see mode 1 and the activation globals)
bool is_w4a4(int mode) { return mode == MOE_NVFP4_W4A4 || mode == MOE_NVFP4_W4A4_STATIC; }

// Path actually used for a problem (AUTO resolved by the expected local load).
int resolve_path(const moe_nvfp4_problem& p) {
    if (p.path != MOE_NVFP4_PATH_AUTO) return p.path;
    // expected local pairs per local expert: T * k / E (uniform routing).  The
    // crossovers were measured on the 4096 x 1024 layer with 160 local experts
    // (per-call medians, us):
    //   W4A16: block-diagonal weight streaming up to ~3.9 pairs per expert
    //   (T = 152: 303 against 307 dense; T = 160: 318 against 308), the dense
    //   weight-streaming kernels up to ~64 (T = 2304: 746 against 809 tiled;
    //   T = 2560: 811 against 811; T = 2816: 893 against 829), then the tiles;
    //   W4A4 with the activations as NVFP4: block-diagonal up to 5 (T = 192:
    //   311 against 313 dense; T = 224: 357 against 315), dense up to 18
    //   (T = 704: 368 against 388 tiled; T = 768: 403 against 391), tiles above;
    //   other shapes (no dense path, or W4A4 with 16-bit activations):
    //   block-diagonal up to 6 (packed tiles) or 9, tiles above.
    const double per_expert = (double)p.num_tokens * p.top_k / p.num_experts;
    const bool w4a4 = is_w4a4(p.mode);
    if (!w4a4 && moe::mid_ok(p.d_model, p.d_ff)) {
        if (per_expert <= 3.9) return MOE_NVFP4_PATH_DECODE;
        return per_expert <= 64.0 ? MOE_NVFP4_PATH_MID : MOE_NVFP4_PATH_PREFILL;
    }
    if (w4a4 && moe::mid_packed_ok(p.d_model, p.d_ff)) {
        if (per_expert <= 5.0) return MOE_NVFP4_PATH_DECODE;
        return per_expert <= 18.0 ? MOE_NVFP4_PATH_MID : MOE_NVFP4_PATH_PREFILL;
    }
    const bool packed = w4a4 && moe::pf_packed_ok(p.d_model, p.d_ff);
    return per_expert <= (packed ? 6.0 : 9.0) ? MOE_NVFP4_PATH_DECODE : MOE_NVFP4_PATH_PREFILL;
}

struct Plan {
    int KS = 1, path = 1, BM = 16, max_tiles = 0, nblk = 0;
    bool exact = false;  // routing by exact fp64 logits (few tokens), else certified
    size_t rows = 0;  // rows of the expanded (pair + shared) activation space
    size_t bar, part, xn2, gn2, topk_ids, topk_w, local_ids, rank, block_counts, counts, offsets, tiles,
        ntiles, perm, inv, hq, act, Y, total;
};

int check_problem(const moe_nvfp4_problem* p) {
    if (!p) return fail(MOE_NVFP4_ERR_INVALID_ARG, "problem is NULL");
    if (p->num_tokens < 0) return fail(MOE_NVFP4_ERR_INVALID_ARG, "num_tokens < 0");
    if (p->mode != MOE_NVFP4_W4A16 && p->mode != MOE_NVFP4_W4A4 && p->mode != MOE_NVFP4_W4A4_STATIC)
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "unknown mode %d", p->mode);
    if (p->mode == MOE_NVFP4_W4A4_STATIC && (!global_ok(p->act_global13) || !global_ok(p->act_global2)))
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "static W4A4 activation globals must be finite, in 2^-100..2^100");
    if (p->path < MOE_NVFP4_PATH_AUTO || p->path > MOE_NVFP4_PATH_MICRO)
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "unknown path %d", p->path);
    if (p->has_shared != 0 && p->has_shared != 1)
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "has_shared must be 0 or 1");
    if (p->num_experts < 1 || p->num_experts > 1024)
        return fail(MOE_NVFP4_ERR_UNSUPPORTED_SHAPE, "num_experts %d outside 1..1024", p->num_experts);
    if (p->top_k < 1 || p->top_k > 32 || p->top_k > p->num_experts)
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "top_k %d outside 1..min(E, 32)", p->top_k);
    if (p->num_local_experts < 1) return fail(MOE_NVFP4_ERR_INVALID_ARG, "num_local_experts < 1");
    if (p->local_expert_offset < 0) return fail(MOE_NVFP4_ERR_INVALID_ARG, "local_expert_offset < 0");
    if ((long long)p->local_expert_offset + p->num_local_experts > p->num_experts)
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "local_expert_offset + num_local_experts > num_experts");
    if (p->d_model < 128 || p->d_model > 16384 || p->d_model % 128)
        return fail(MOE_NVFP4_ERR_UNSUPPORTED_SHAPE, "d_model %d: need a multiple of 128 in 128..16384",
                    p->d_model);
    if (p->d_ff < 128 || p->d_ff > 16384 || p->d_ff % 128)
        return fail(MOE_NVFP4_ERR_UNSUPPORTED_SHAPE, "d_ff %d: need a multiple of 128 in 128..16384", p->d_ff);
    if (p->path == MOE_NVFP4_PATH_MID && !moe::mid_ok(p->d_model, p->d_ff))
        return fail(MOE_NVFP4_ERR_UNSUPPORTED_SHAPE, "the dense weight-streaming path needs d_model %% 256 == 0");
    if (p->path == MOE_NVFP4_PATH_MICRO && p->num_tokens > 0 &&
        !moe::micro_ok(p->num_tokens, p->d_model, p->d_ff, p->num_experts, p->top_k, p->num_local_experts))
        return fail(MOE_NVFP4_ERR_UNSUPPORTED_SHAPE,
                    "the one-launch small-batch path needs 1..16 tokens, d_model and d_ff <= 4096, d_model %% 256 == 0");
    // index arithmetic: pair rows and per-row offsets stay within int32
    const long long rows = (long long)p->num_tokens * (p->top_k + 1);
    if (rows > (1LL << 27)) return fail(MOE_NVFP4_ERR_UNSUPPORTED_SHAPE, "num_tokens * (top_k + 1) > 2^27");
    return MOE_NVFP4_OK;
}

void make_plan(const moe_nvfp4_problem& p, Plan& pl) {
    const size_t T = p.num_tokens, k = p.top_k, E = p.num_experts, L = p.num_local_experts;
    const size_t d = p.d_model, F = p.d_ff;
    pl.exact = moe::router_exact((int)T, (int)E, (int)d);
    pl.KS = pl.exact ? moe::router_exact_ksplit((int)T, (int)E, (int)d) : moe::router_ksplit((int)T, (int)E, (int)d);
    pl.path = resolve_path(p);
    pl.BM = moe::gemm_bm(pl.path, (int)T, (int)k, (int)E, is_w4a4(p.mode) && moe::mid_packed_ok((int)d, (int)F));
    const size_t bm = pl.BM;
    pl.max_tiles = (int)((T * k + bm - 1) / bm + L + (p.has_shared ? (T + bm - 1) / bm : 0));
    pl.nblk = (int)((T + 255) / 256);
    pl.rows = T * k + (p.has_shared ? T : 0);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
    pl.bar = take(2 * sizeof(unsigned));              // the one-launch path's grid barrier and error word
    pl.part = take(std::max((size_t)pl.KS * T * E * (pl.exact ? 8 : 4), T * E * 8));
    pl.xn2 = take(pl.exact ? 0 : (size_t)pl.KS * T * 8);
    pl.gn2 = take(pl.exact ? 0 : (size_t)pl.KS * E * 8);
    pl.topk_ids = take(T * k * 4);
    pl.topk_w = take(T * k * 4);
    pl.local_ids = take(T * k * 4);
    pl.rank = take(T * k * 4);
    pl.block_counts = take((size_t)pl.nblk * L * 4);
    pl.counts = take(L * 4);
    pl.offsets = take((L + 1) * 4);
    pl.tiles = take((size_t)pl.max_tiles * 16);
    pl.ntiles = take(4);
    pl.perm = take(T * k * 4);
    pl.inv = take(T * k * 4);
    const bool w4a4 = is_w4a4(p.mode);
    pl.hq = take(w4a4 ? T * d * 2 : 0);
    pl.act = take(pl.rows * F * 2);
    pl.Y = take(pl.rows * d * 2);
    pl.total = o;
}

bool arch_ok(const char* arch) { return arch && std::strncmp(arch, "gfx950", 6) == 0; }

// Architecture of the current device, cached per device id.
int current_arch_ok(int* dev_out) {
    static std::mutex mu;
    static int cache[64];  // 0 unknown, 1 gfx950, 2 other
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_NVFP4_ERR_HIP, "hipGetDevice failed");
    *dev_out = dev;
    if (dev < 0 || dev >= 64) return fail(MOE_NVFP4_ERR_HIP, "device id %d out of range", dev);
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(MOE_NVFP4_ERR_HIP, "hipGetDeviceProperties failed");
        cache[dev] = arch_ok(prop.gcnArchName) ? 1 : 2;
    }
    if (cache[dev] != 1) return fail(MOE_NVFP4_ERR_ARCH, "device %d is not gfx950", dev);
    return MOE_NVFP4_OK;
}

// Compute units of the current device `dev` (cached per device).
int cu_count(int dev, int* out) {
    static std::mutex mu;
    static int cache[64];
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return fail(MOE_NVFP4_ERR_HIP, "hipDeviceGetAttribute(multiprocessor count) failed");
        cache[dev] = n;
    }
    *out = cache[dev];
    return MOE_NVFP4_OK;
}

int check_weights(const moe_nvfp4_weights* w, const char* what) {
    if (!w) return fail(MOE_NVFP4_ERR_INVALID_ARG, "%s weights are NULL", what);
    if (!w->w13 || !w->w13_scale || !w->w13_global || !w->w2 || !w->w2_scale || !w->w2_global)
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "%s weights have a NULL tensor pointer", what);
    auto mis = [](const void* q, uintptr_t al) { return (reinterpret_cast<uintptr_t>(q) & (al - 1)) != 0; };
    if (mis(w->w13, 16) || mis(w->w13_scale, 16) || mis(w->w2, 16) || mis(w->w2_scale, 16))
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "%s weight codes and scales must be 16-byte aligned", what);
    if (mis(w->w13_global, 4) || mis(w->w2_global, 4))
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "%s global scales must be 4-byte aligned", what);
    return MOE_NVFP4_OK;
}

moe::ExpertWeights to_internal(const moe_nvfp4_weights* w) {
    moe::ExpertWeights e{};
    if (w) {
        e.w13 = w->w13; e.w13_s = w->w13_scale; e.g13 = w->w13_global;
        e.w2 = w->w2; e.w2_s = w->w2_scale; e.g2 = w->w2_global;
    }
    return e;
}

template <class T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

int hip_status(hipError_t e, const char* where) {
    if (e != hipSuccess) return fail(MOE_NVFP4_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
    return MOE_NVFP4_OK;
}

// Routing + permutation into the workspace (or the caller's buffers where given).
int run_route(const moe_nvfp4_problem& p, const Plan& pl, const void* hidden, const void* gate_w,
              void* ws, hipStream_t s, int32_t* ids_out, float* w_out, int32_t* counts_out,
              int32_t* offsets_out, int32_t* perm_out) {
    moe::RouterArgs r{};
    r.X = static_cast<const uint16_t*>(hidden);
    r.G = static_cast<const uint16_t*>(gate_w);
    r.T = p.num_tokens; r.E = p.num_experts; r.d = p.d_model; r.KS = pl.KS; r.topk = p.top_k;
    r.offset = p.local_expert_offset; r.L = p.num_local_experts;
    r.part = at<float>(ws, pl.part); r.xn2 = at<double>(ws, pl.xn2); r.gn2 = at<double>(ws, pl.gn2);
    r.xpart = at<double>(ws, pl.part);
    r.topk_ids = ids_out ? ids_out : at<int32_t>(ws, pl.topk_ids);
    r.topk_w = w_out ? w_out : at<float>(ws, pl.topk_w);
    r.local_ids = at<int32_t>(ws, pl.local_ids);
    moe::PermArgs q{};
    q.local_ids = r.local_ids; q.T = p.num_tokens; q.topk = p.top_k; q.L = p.num_local_experts;
    q.has_shared = p.has_shared; q.BM = pl.BM; q.max_tiles = pl.max_tiles;
    q.block_counts = at<int32_t>(ws, pl.block_counts); q.rank = at<int32_t>(ws, pl.rank);
    q.counts = counts_out ? counts_out : at<int32_t>(ws, pl.counts);
    q.offsets = offsets_out ? offsets_out : at<int32_t>(ws, pl.offsets);
    q.tiles = at<int4>(ws, pl.tiles); q.ntiles = at<int32_t>(ws, pl.ntiles);
    q.perm = perm_out ? perm_out : at<int32_t>(ws, pl.perm); q.inv = at<int32_t>(ws, pl.inv);
    if (pl.exact && moe::route_fused_ok(r.T, r.E, r.d, r.L))
        return hip_status(moe::launch_route_exact_fused(r, q, s), "router launch");
    int st = hip_status(pl.exact ? moe::launch_route_exact(r, s) : moe::launch_router(r, s), "router launch");
    if (st) return st;
    return hip_status(moe::launch_permute(q, s), "permutation launch");
}

// Scratch of the no-allocation forward: one array per device (each GPU the
// library runs on holds its own copy until the process ends).  Host code never
// uses the array's name as an address: it is a host-side stand-in; the device
// address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = MOE_NVFP4_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Device address of `scratch` on the current device `dev` (looked up on the
// first call on that device, with that device current, and kept).
int scratch_address(int dev, void** out) {
    static std::mutex mu;
    static void* addr[64];
    if (dev < 0 || dev >= 64) return fail(MOE_NVFP4_ERR_HIP, "device id %d out of range", dev);
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(MOE_NVFP4_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        addr[dev] = ptr;
    }
    *out = addr[dev];
    return MOE_NVFP4_OK;
}

}  // namespace

extern "C" {

const char* moe_nvfp4_strerror(int status) {
    switch (status) {
        case MOE_NVFP4_OK: return "ok";
        case MOE_NVFP4_ERR_INVALID_ARG: return "invalid argument";
        case MOE_NVFP4_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case MOE_NVFP4_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MOE_NVFP4_ERR_ARCH: return "device architecture is not gfx950";
        case MOE_NVFP4_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* moe_nvfp4_last_error(void) { return g_last_error.c_str(); }

int moe_nvfp4_workspace_size(const moe_nvfp4_problem* p, size_t* bytes) {
    if (!bytes) return fail(MOE_NVFP4_ERR_INVALID_ARG, "bytes is NULL");
    int st = check_problem(p);
    if (st) return st;
    Plan pl;
    make_plan(*p, pl);
    *bytes = pl.total;
    return ok();
}

int moe_nvfp4_validate(const moe_nvfp4_problem* p, size_t workspace_bytes, const char* arch) {
    int st = check_problem(p);
    if (st) return st;
    Plan pl;
    make_plan(*p, pl);
    if (workspace_bytes < pl.total)
        return fail(MOE_NVFP4_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < required %zu", workspace_bytes,
                    pl.total);
    if (arch && !arch_ok(arch)) return fail(MOE_NVFP4_ERR_ARCH, "architecture '%s' is not gfx950", arch);
    return ok();
}

int moe_nvfp4_resolved_path(const moe_nvfp4_problem* p, int32_t* path) {
    if (!path) return fail(MOE_NVFP4_ERR_INVALID_ARG, "path is NULL");
    const int st = check_problem(p);
    if (st) return st;
    *path = resolve_path(*p);
    return ok();
}

int moe_nvfp4_forward(const moe_nvfp4_problem* p, const void* hidden, const void* gate_w,
                      const moe_nvfp4_weights* local, const moe_nvfp4_weights* shared, void* workspace,
                      size_t workspace_bytes, void* out, void* stream) {
    return moe_nvfp4_forward_timed(p, hidden, gate_w, local, shared, workspace, workspace_bytes, out, stream,
                                   nullptr, 0);
}

int moe_nvfp4_forward_timed(const moe_nvfp4_problem* p, const void* hidden, const void* gate_w,
                            const moe_nvfp4_weights* local, const moe_nvfp4_weights* shared, void* workspace,
                            size_t workspace_bytes, void* out, void* stream, void* const* events,
                            int num_events) {
    if (num_events < 0 || num_events > 6 || (num_events > 0 && !events))
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "num_events must be 0..6 with a non-NULL array");
    int st = moe_nvfp4_validate(p, workspace_bytes, nullptr);
    if (st) return st;
    if (!hidden || !gate_w || !out) return fail(MOE_NVFP4_ERR_INVALID_ARG, "hidden/gate_w/out is NULL");
    if (((reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(gate_w) |
          reinterpret_cast<uintptr_t>(out)) & 15u) != 0)
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "hidden/gate_w/out must be 16-byte aligned");
    if ((st = check_weights(local, "local"))) return st;
    if (p->has_shared) {
        if ((st = check_weights(shared, "shared"))) return st;
    } else if (shared) {
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "shared weights given but has_shared == 0");
    }
    Plan pl;
    make_plan(*p, pl);
    if (!workspace && pl.total) return fail(MOE_NVFP4_ERR_INVALID_ARG, "workspace is NULL");
    int dev;
    if ((st = current_arch_ok(&dev))) return st;
    if (p->num_tokens == 0) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto mark = [&](int i) -> int {
        if (i < num_events && events[i])
            return hip_status(hipEventRecord(static_cast<hipEvent_t>(events[i]), s), "hipEventRecord");
        return MOE_NVFP4_OK;
    };
    if ((st = mark(0))) return st;
    if (pl.path == MOE_NVFP4_PATH_MICRO) {
        // the whole layer in one persistent launch (after the barrier reset)
        int ncu;
        if ((st = cu_count(dev, &ncu))) return st;
        const bool stat = p->mode == MOE_NVFP4_W4A4_STATIC;
        moe::MicroArgs m{};
        m.T = p->num_tokens; m.d = p->d_model; m.F = p->d_ff; m.E = p->num_experts; m.topk = p->top_k;
        m.offset = p->local_expert_offset; m.L = p->num_local_experts; m.has_shared = p->has_shared;
        m.mode = is_w4a4(p->mode) ? 1 : 0;
        m.a1g = stat ? p->act_global13 : 1.0f;
        m.a2g = stat ? p->act_global2 : 1.0f;
        m.X = static_cast<const uint16_t*>(hidden);
        m.G = static_cast<const uint16_t*>(gate_w);
        m.local = to_internal(local);
        m.shared = to_internal(p->has_shared ? shared : nullptr);
        m.bar = at<unsigned>(workspace, pl.bar);
        m.logits = at<double>(workspace, pl.part);
        m.hq = at<uint16_t>(workspace, pl.hq);
        m.act = at<uint16_t>(workspace, pl.act);
        m.Y = at<uint16_t>(workspace, pl.Y);
        m.out = static_cast<uint16_t*>(out);
        if ((st = hip_status(moe::launch_micro(m, ncu, s), "small-batch layer launch"))) return st;
        for (int i = 1; i < 6; ++i)
            if ((st = mark(i))) return st;
        return ok();
    }
    if ((st = run_route(*p, pl, hidden, gate_w, workspace, s, nullptr, nullptr, nullptr, nullptr, nullptr)))
        return st;
    if ((st = mark(1))) return st;
    const bool w4a4 = is_w4a4(p->mode);
    const bool stat = p->mode == MOE_NVFP4_W4A4_STATIC;
    const float a1g = stat ? p->act_global13 : 1.0f, a2g = stat ? p->act_global2 : 1.0f;
    const bool tiled = pl.path == MOE_NVFP4_PATH_PREFILL;
    const bool mid = pl.path == MOE_NVFP4_PATH_MID;
    // W4A4 on the tiled path: the activations travel as NVFP4 codes and scales
    // when d and F allow it, else as exact f16 values
    const bool packed = w4a4 && ((tiled && moe::pf_packed_ok(p->d_model, p->d_ff)) ||
                                 (mid && moe::mid_packed_ok(p->d_model, p->d_ff)));
    uint8_t* hq_codes = at<uint8_t>(workspace, pl.hq);
    uint8_t* hq_scales = hq_codes + (size_t)p->num_tokens * (p->d_model / 2);
    uint8_t* act_codes = at<uint8_t>(workspace, pl.act);
    uint8_t* act_scales = act_codes + (size_t)pl.rows * (p->d_ff / 2);
    if (w4a4) {
        if (packed)
            st = hip_status(moe::launch_quantize_act(static_cast<const uint16_t*>(hidden), p->num_tokens,
                                                     p->d_model, a1g, hq_codes, hq_scales, s),
                            "activation quantizer launch");
        else
            st = hip_status(moe::launch_fake_quant_act(static_cast<const uint16_t*>(hidden), p->num_tokens,
                                                       p->d_model, a1g, at<uint16_t>(workspace, pl.hq),
                                                       tiled || mid, s),
                            "activation quantizer launch");
        if (st) return st;
    }
    if ((st = mark(2))) return st;
    moe::GemmArgs g{};
    g.T = p->num_tokens; g.d = p->d_model; g.F = p->d_ff; g.topk = p->top_k; g.L = p->num_local_experts;
    g.mode = w4a4 ? 1 : 0;
    g.a1g = a1g;
    g.a2g = a2g;
    g.E = p->num_experts;
    g.perm = at<int32_t>(workspace, pl.perm);
    g.tiles = at<int4>(workspace, pl.tiles);
    g.ntiles = at<int32_t>(workspace, pl.ntiles);
    g.max_tiles = pl.max_tiles;
    g.hidden = static_cast<const uint16_t*>(hidden);
    g.hq = at<uint16_t>(workspace, pl.hq);
    g.local = to_internal(local);
    g.shared = to_internal(p->has_shared ? shared : nullptr);
    g.act = at<uint16_t>(workspace, pl.act);
    g.Y = at<uint16_t>(workspace, pl.Y);
    g.packed = packed ? 1 : 0;
    g.hq_codes = hq_codes;
    g.hq_scales = hq_scales;
    g.act_codes = act_codes;
    g.act_scales = act_scales;
    const bool dec = pl.path == MOE_NVFP4_PATH_DECODE;
    if ((st = hip_status(dec ? moe::launch_dec_gemm1(g, s)
                             : (mid ? moe::launch_mid_gemm1(g, s) : moe::launch_gemm1(g, pl.path, s)),
                         "gemm1 launch")))
        return st;
    if ((st = mark(3))) return st;
    if ((st = hip_status(dec ? moe::launch_dec_gemm2(g, s)
                             : (mid ? moe::launch_mid_gemm2(g, s) : moe::launch_gemm2(g, pl.path, s)),
                         "gemm2 launch")))
        return st;
    if ((st = mark(4))) return st;
    moe::CombineArgs c{};
    c.T = p->num_tokens; c.d = p->d_model; c.topk = p->top_k; c.has_shared = p->has_shared;
    c.topk_w = at<float>(workspace, pl.topk_w);
    c.inv = at<int32_t>(workspace, pl.inv);
    c.Y = g.Y;
    c.out = static_cast<uint16_t*>(out);
    if ((st = hip_status(moe::launch_combine(c, s), "combine launch"))) return st;
    if ((st = mark(5))) return st;
    return ok();
}

int moe_nvfp4_forward_noalloc(const moe_nvfp4_problem* p, const void* hidden, const void* gate_w,
                              const moe_nvfp4_weights* local, const moe_nvfp4_weights* shared, void* out,
                              void* stream) {
    int st = check_problem(p);
    if (st) return st;
    Plan pl;
    make_plan(*p, pl);
    if (pl.total > kNoAllocScratchBytes)
        return fail(MOE_NVFP4_ERR_WORKSPACE_TOO_SMALL,
                    "this problem needs %zu bytes of scratch; the no-allocation forward holds %zu "
                    "(use moe_nvfp4_forward with a workspace)",
                    pl.total, kNoAllocScratchBytes);
    int dev;
    if ((st = current_arch_ok(&dev))) return st;
    void* ws = nullptr;
    if ((st = scratch_address(dev, &ws))) return st;
    return moe_nvfp4_forward_timed(p, hidden, gate_w, local, shared, ws, kNoAllocScratchBytes, out, stream,
                                   nullptr, 0);
}

int moe_nvfp4_route(const moe_nvfp4_problem* p, const void* hidden, const void* gate_w, int32_t* topk_ids,
                    float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm, void* workspace,
                    size_t workspace_bytes, void* stream) {
    int st = moe_nvfp4_validate(p, workspace_bytes, nullptr);
    if (st) return st;
    if (!hidden || !gate_w) return fail(MOE_NVFP4_ERR_INVALID_ARG, "hidden/gate_w is NULL");
    if (((reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(gate_w)) & 15u) != 0)
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "hidden/gate_w must be 16-byte aligned");
    Plan pl;
    make_plan(*p, pl);
    if (!workspace && pl.total) return fail(MOE_NVFP4_ERR_INVALID_ARG, "workspace is NULL");
    int dev;
    if ((st = current_arch_ok(&dev))) return st;
    if (p->num_tokens == 0) {
        // counts = 0, offsets = 0 still have to be written
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (counts && (st = hip_status(moe::launch_fill_u32(reinterpret_cast<uint32_t*>(counts),
                                                             (size_t)p->num_local_experts, 0u, s), "fill")))
            return st;
        if (offsets && (st = hip_status(moe::launch_fill_u32(reinterpret_cast<uint32_t*>(offsets),
                                                              (size_t)p->num_local_experts + 1, 0u, s), "fill")))
            return st;
        return ok();
    }
    st = run_route(*p, pl, hidden, gate_w, workspace, static_cast<hipStream_t>(stream), topk_ids, topk_w,
                   counts, offsets, perm);
    if (st) return st;
    return ok();
}

int moe_nvfp4_quantize_weights(const void* w, int32_t n, int32_t R, int32_t C, uint8_t* codes,
                               uint8_t* scales, float* global, void* stream) {
    if (!w || !codes || !scales || !global) return fail(MOE_NVFP4_ERR_INVALID_ARG, "NULL pointer");
    if (n < 0 || R < 0 || C < 0) return fail(MOE_NVFP4_ERR_INVALID_ARG, "negative size");
    if (C % 16) return fail(MOE_NVFP4_ERR_UNSUPPORTED_SHAPE, "C %d is not a multiple of 16", C);
    if ((long long)n * R * C > (1LL << 40)) return fail(MOE_NVFP4_ERR_UNSUPPORTED_SHAPE, "tensor too large");
    int dev, st;
    if ((st = current_arch_ok(&dev))) return st;
    if (n == 0 || R == 0 || C == 0) {
        // all-zero (empty) tensors: global scale 1, as for any all-zero tensor
        if (n > 0 && (st = hip_status(moe::launch_fill_u32(reinterpret_cast<uint32_t*>(global), (size_t)n,
                                                            0x3F800000u, static_cast<hipStream_t>(stream)),
                                       "fill")))
            return st;
        return ok();
    }
    st = hip_status(moe::launch_quantize_weights(static_cast<const uint16_t*>(w), n, R, C, codes, scales, global,
                                                 static_cast<hipStream_t>(stream)),
                    "weight quantizer launch");
    return st ? st : ok();
}

int moe_nvfp4_quantize_activations(const void* x, int32_t R, int32_t C, uint8_t* codes, uint8_t* scales,
                                   void* stream) {
    return moe_nvfp4_quantize_activations_static(x, R, C, 1.0f, codes, scales, stream);
}

int moe_nvfp4_quantize_activations_static(const void* x, int32_t R, int32_t C, float g, uint8_t* codes,
                                          uint8_t* scales, void* stream) {
    if (!x || !codes || !scales) return fail(MOE_NVFP4_ERR_INVALID_ARG, "NULL pointer");
    if (!global_ok(g)) return fail(MOE_NVFP4_ERR_INVALID_ARG, "global %g outside 2^-100..2^100", (double)g);
    if (R < 0 || C < 0) return fail(MOE_NVFP4_ERR_INVALID_ARG, "negative size");
    if (C % 16) return fail(MOE_NVFP4_ERR_UNSUPPORTED_SHAPE, "C %d is not a multiple of 16", C);
    int dev, st;
    if ((st = current_arch_ok(&dev))) return st;
    st = hip_status(moe::launch_quantize_act(static_cast<const uint16_t*>(x), R, C, g, codes, scales,
                                             static_cast<hipStream_t>(stream)),
                    "activation quantizer launch");
    return st ? st : ok();
}

int moe_nvfp4_prepare(const moe_nvfp4_checkpoint* ck, int32_t first_expert, int32_t count,
                      const moe_nvfp4_weights* dst, void* stream) {
    if (!ck || !dst) return fail(MOE_NVFP4_ERR_INVALID_ARG, "checkpoint or destination is NULL");
    const int d = ck->d_model, F = ck->d_ff;
    if (d < 128 || d > 16384 || d % 128)
        return fail(MOE_NVFP4_ERR_UNSUPPORTED_SHAPE, "d_model %d: need a multiple of 128 in 128..16384", d);
    if (F < 128 || F > 16384 || F % 128)
        return fail(MOE_NVFP4_ERR_UNSUPPORTED_SHAPE, "d_ff %d: need a multiple of 128 in 128..16384", F);
    if (ck->global_convention != MOE_NVFP4_GLOBAL_MULTIPLIER && ck->global_convention != MOE_NVFP4_GLOBAL_INVERSE)
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "unknown global scale convention %d", ck->global_convention);
    if (ck->w13_order != MOE_NVFP4_GATE_UP && ck->w13_order != MOE_NVFP4_UP_GATE)
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "unknown w13 row order %d", ck->w13_order);
    if (ck->num_experts < 1 || first_expert < 0 || count < 0 || (long long)first_expert + count > ck->num_experts)
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "experts [%d, %d) outside the checkpoint's %d", first_expert,
                    first_expert + count, ck->num_experts);
    if (count > 65535) return fail(MOE_NVFP4_ERR_INVALID_ARG, "count %d: at most 65535 experts per call", count);
    int st;
    const moe_nvfp4_weights src = {ck->w13, ck->w13_scale, ck->w13_global, ck->w2, ck->w2_scale, ck->w2_global};
    if ((st = check_weights(&src, "checkpoint"))) return st;
    if ((st = check_weights(dst, "destination"))) return st;
    // per-expert sizes of the six tensors; destination ranges must not overlap the sources
    const size_t b13 = (size_t)2 * F * (d / 2), s13 = (size_t)2 * F * (d / 16);
    const size_t b2 = (size_t)d * (F / 2), s2 = (size_t)d * (F / 16);
    auto overlap = [&](const void* a, const void* b, size_t na, size_t nb) {
        const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
        return x < y + nb && y < x + na;
    };
    const size_t n = (size_t)count, E = (size_t)ck->num_experts;
    if (overlap(dst->w13, ck->w13, n * b13, E * b13) || overlap(dst->w13_scale, ck->w13_scale, n * s13, E * s13) ||
        overlap(dst->w2, ck->w2, n * b2, E * b2) || overlap(dst->w2_scale, ck->w2_scale, n * s2, E * s2) ||
        overlap(dst->w13_global, ck->w13_global, n * 4, E * 4) || overlap(dst->w2_global, ck->w2_global, n * 4, E * 4))
        return fail(MOE_NVFP4_ERR_INVALID_ARG, "destination overlaps the checkpoint");
    int dev;
    if ((st = current_arch_ok(&dev))) return st;
    if (count == 0) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t f = (size_t)first_expert;
    const bool swap = ck->w13_order == MOE_NVFP4_UP_GATE, inv = ck->global_convention == MOE_NVFP4_GLOBAL_INVERSE;
    uint8_t* d13 = const_cast<uint8_t*>(dst->w13);
    uint8_t* d13s = const_cast<uint8_t*>(dst->w13_scale);
    uint8_t* d2 = const_cast<uint8_t*>(dst->w2);
    uint8_t* d2s = const_cast<uint8_t*>(dst->w2_scale);
    if ((st = hip_status(moe::launch_prepare_rows(ck->w13 + f * b13, d13, count, 2 * F, d / 2, swap, s),
                         "prepare w13 codes")) ||
        (st = hip_status(moe::launch_prepare_rows(ck->w13_scale + f * s13, d13s, count, 2 * F, d / 16, swap, s),
                         "prepare w13 scales")) ||
        (st = hip_status(moe::launch_prepare_rows(ck->w2 + f * b2, d2, count, d, F / 2, false, s),
                         "prepare w2 codes")) ||
        (st = hip_status(moe::launch_prepare_rows(ck->w2_scale + f * s2, d2s, count, d, F / 16, false, s),
                         "prepare w2 scales")) ||
        (st = hip_status(moe::launch_prepare_global(ck->w13_global + f, const_cast<float*>(dst->w13_global), count,
                                                    inv, s),
                         "prepare w13 global")) ||
        (st = hip_status(moe::launch_prepare_global(ck->w2_global + f, const_cast<float*>(dst->w2_global), count,
                                                    inv, s),
                         "prepare w2 global")))
        return st;
    return ok();
}

}  // extern "C"
