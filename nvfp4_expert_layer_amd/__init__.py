"""Python binding of libmoe_nvfp4.so (the fused NVFP4 MoE layer for MI355X).

Argument marshalling only: every step of the layer runs in the library's gfx950
kernels.  Functions carry the names of the C entry points declared in
include/moe_nvfp4.h and take torch tensors (device memory) and the current
torch stream.  There is no fallback: if the shared library is missing, every
call raises.
"""
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_nvfp4.so")

W4A16 = 0
W4A4 = 1
W4A4_STATIC = 2
PATH_AUTO, PATH_DECODE, PATH_PREFILL, PATH_MID, PATH_MICRO = 0, 1, 2, 3, 4

OK = 0
ERR_INVALID_ARG = 1
ERR_UNSUPPORTED_SHAPE = 2
ERR_WORKSPACE_TOO_SMALL = 3
ERR_ARCH = 4
ERR_HIP = 5


class MoeNvfp4Error(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"moe_nvfp4 status {status}: {msg}")
        self.status = status


class moe_nvfp4_problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tokens", "d_model", "d_ff", "num_experts", "top_k", "local_expert_offset",
        "num_local_experts", "has_shared", "mode", "path")] + [
        ("act_global13", ctypes.c_float), ("act_global2", ctypes.c_float)]


class moe_nvfp4_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w13", "w13_scale", "w13_global", "w2", "w2_scale", "w2_global")]


GLOBAL_MULTIPLIER, GLOBAL_INVERSE = 0, 1
GATE_UP, UP_GATE = 0, 1


class moe_nvfp4_checkpoint(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w13", "w13_scale", "w13_global", "w2", "w2_scale", "w2_global")] + [
        (n, ctypes.c_int32) for n in ("num_experts", "d_model", "d_ff", "global_convention", "w13_order")]


_lib = None


def lib():
    """The loaded shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m nvfp4_expert_layer_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.moe_nvfp4_workspace_size.argtypes = [P(moe_nvfp4_problem), P(sz)]
        L.moe_nvfp4_validate.argtypes = [P(moe_nvfp4_problem), sz, ctypes.c_char_p]
        L.moe_nvfp4_resolved_path.argtypes = [P(moe_nvfp4_problem), P(i32)]
        L.moe_nvfp4_forward.argtypes = [P(moe_nvfp4_problem), vp, vp, P(moe_nvfp4_weights),
                                        P(moe_nvfp4_weights), vp, sz, vp, vp]
        L.moe_nvfp4_forward_timed.argtypes = [P(moe_nvfp4_problem), vp, vp, P(moe_nvfp4_weights),
                                              P(moe_nvfp4_weights), vp, sz, vp, vp,
                                              P(ctypes.c_void_p), ctypes.c_int]
        L.moe_nvfp4_forward_noalloc.argtypes = [P(moe_nvfp4_problem), vp, vp, P(moe_nvfp4_weights),
                                                P(moe_nvfp4_weights), vp, vp]
        L.moe_nvfp4_route.argtypes = [P(moe_nvfp4_problem), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_nvfp4_quantize_weights.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        L.moe_nvfp4_quantize_activations.argtypes = [vp, i32, i32, vp, vp, vp]
        L.moe_nvfp4_quantize_activations_static.argtypes = [vp, i32, i32, ctypes.c_float, vp, vp, vp]
        L.moe_nvfp4_prepare.argtypes = [P(moe_nvfp4_checkpoint), i32, i32, P(moe_nvfp4_weights), vp]
        L.moe_nvfp4_strerror.argtypes = [ctypes.c_int]
        L.moe_nvfp4_strerror.restype = ctypes.c_char_p
        L.moe_nvfp4_last_error.argtypes = []
        L.moe_nvfp4_last_error.restype = ctypes.c_char_p
        for f in ("workspace_size", "validate", "forward", "forward_timed", "forward_noalloc", "route", "quantize_weights",
                  "quantize_activations", "quantize_activations_static", "prepare", "resolved_path"):
            getattr(L, "moe_nvfp4_" + f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status):
    if status != OK:
        raise MoeNvfp4Error(status, lib().moe_nvfp4_last_error().decode() or
                            lib().moe_nvfp4_strerror(status).decode())


def _ptr(t, cur=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    # the library launches on the current device (and the stream): a tensor of
    # another device would be read through pointers that device does not map
    if cur is None:
        cur = torch.cuda.current_device()
    if t.get_device() != cur:
        raise ValueError(f"tensor is on {t.device}, the current device is cuda:{cur}")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _ptrs(*specs):
    """Device pointers of the tensors of specs (tensor, name, dtype, shape), after
    checking every tensor's dtype and shape (a None entry of `shape` matches any
    size) -- the library reads and writes exactly these extents, so a smaller
    tensor would be accessed out of bounds.  None tensors pass as NULL.  The
    current device is looked up once per call."""
    for t, name, dtype, shape in specs:
        if t is None:
            continue
        if t.dtype != dtype:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
        ts = t.shape
        if ts != shape and (len(ts) != len(shape) or
                            any(want is not None and ts[i] != want for i, want in enumerate(shape))):
            raise ValueError(f"{name}: shape {tuple(ts)}, expected {tuple(shape)}")
    cur = None
    ptrs = []
    for t, *_ in specs:
        if cur is None and t is not None and t.is_cuda:
            cur = torch.cuda.current_device()
        ptrs.append(_ptr(t, cur))
    return ptrs


def _layer_ptrs(p, specs, local, shared):
    """_ptrs of the token tensors `specs` and of the local and shared experts'
    tensors; returns (token pointers, local weights struct, shared struct or None)."""
    d, F = p.d_model, p.d_ff
    specs = specs + local.specs(p.num_local_experts, d, F, "local")
    if shared is not None:
        specs += shared.specs(1, d, F, "shared")
    ptrs = _ptrs(*specs)
    n = len(specs) - (12 if shared is not None else 6)
    lw = moe_nvfp4_weights(*ptrs[n:n + 6])
    sw = moe_nvfp4_weights(*ptrs[n + 6:]) if shared is not None else None
    return ptrs[:n], lw, sw


def _rows(p):
    """Row count of the token tensors of problem p: T (any, when T = 0: an empty
    batch reads nothing, but the library still wants non-NULL pointers)."""
    return p.num_tokens if p.num_tokens > 0 else None


def _stream(stream):
    cur = torch.cuda.current_device()
    s = torch.cuda.current_stream(cur) if stream is None else stream
    if s.device_index != cur:
        raise ValueError(f"stream is on {s.device}, the current device is cuda:{cur}")
    return ctypes.c_void_p(s.cuda_stream)


def make_problem(T, d, F, E, k, offset, L, has_shared, mode, path=PATH_AUTO, act_global=(1.0, 1.0)):
    """act_global: the static W4A4 activation globals of the GEMM1 and GEMM2
    inputs (ignored in the other modes)."""
    return moe_nvfp4_problem(T, d, F, E, k, offset, L, int(bool(has_shared)), mode, path,
                             float(act_global[0]), float(act_global[1]))


@dataclass
class NVFP4Experts:
    """NVFP4 weights of n experts (device tensors), the layout of moe_nvfp4_weights."""
    w13: torch.Tensor         # uint8 [n, 2F, d/2]
    w13_scale: torch.Tensor   # uint8 [n, 2F, d/16]
    w13_global: torch.Tensor  # fp32 [n]
    w2: torch.Tensor          # uint8 [n, d, F/2]
    w2_scale: torch.Tensor    # uint8 [n, d, F/16]
    w2_global: torch.Tensor   # fp32 [n]

    def c_struct(self, n=None, d=None, F=None, name="experts"):
        """The C view; with n, d, F given, the tensors are first checked against
        n experts of a d x F layer (dtype, shape, GPU, contiguity)."""
        if n is not None:
            _ptrs(*self.specs(n, d, F, name))
        return moe_nvfp4_weights(*(t.data_ptr() for t in (
            self.w13, self.w13_scale, self.w13_global, self.w2, self.w2_scale, self.w2_global)))

    def specs(self, n, d, F, name):
        """(tensor, name, dtype, shape) of each tensor for n experts (None: any
        number) of a d x F layer."""
        u8, f32 = torch.uint8, torch.float32
        return [(self.w13, f"{name}.w13", u8, (n, 2 * F, d // 2)),
                (self.w13_scale, f"{name}.w13_scale", u8, (n, 2 * F, d // 16)),
                (self.w13_global, f"{name}.w13_global", f32, (n,)),
                (self.w2, f"{name}.w2", u8, (n, d, F // 2)),
                (self.w2_scale, f"{name}.w2_scale", u8, (n, d, F // 16)),
                (self.w2_global, f"{name}.w2_global", f32, (n,))]

    def slice(self, start, count):
        """Experts [start, start+count) (views; any start is accepted by the library)."""
        return NVFP4Experts(*(t[start:start + count] for t in (
            self.w13, self.w13_scale, self.w13_global, self.w2, self.w2_scale, self.w2_global)))

    @staticmethod
    def empty(n, d, F, device="cuda"):
        u8 = dict(dtype=torch.uint8, device=device)
        return NVFP4Experts(torch.empty(n, 2 * F, d // 2, **u8), torch.empty(n, 2 * F, d // 16, **u8),
                            torch.empty(n, dtype=torch.float32, device=device),
                            torch.empty(n, d, F // 2, **u8), torch.empty(n, d, F // 16, **u8),
                            torch.empty(n, dtype=torch.float32, device=device))


def moe_nvfp4_prepare(ck, global_convention, w13_order, first_expert, count, dst, stream=None):
    """Checkpoint tensors `ck` (an NVFP4Experts holding a checkpoint's E experts,
    w13 in `w13_order`, global scales in `global_convention`) -> experts
    [first_expert, first_expert + count) written into `dst` (an NVFP4Experts of
    count experts, the kernel layout)."""
    if ck.w13.dim() != 3:
        raise ValueError(f"ck.w13: shape {tuple(ck.w13.shape)}, expected (E, 2F, d/2)")
    E, twoF, dh = ck.w13.shape
    d, F = dh * 2, twoF // 2
    # dtypes, shapes (dst holds at least `count` experts), GPU, contiguity
    dspecs = dst.specs(None, d, F, "dst")
    for tt, name, _, _ in dspecs:
        if tt.dim() >= 1 and tt.shape[0] < count:
            raise ValueError(f"{name}: {tt.shape[0]} experts, expected at least {count}")
    _ptrs(*ck.specs(E, d, F, "ck"), *dspecs)
    c = moe_nvfp4_checkpoint(*(t.data_ptr() for t in (ck.w13, ck.w13_scale, ck.w13_global, ck.w2, ck.w2_scale,
                                                      ck.w2_global)),
                             E, dh * 2, twoF // 2, global_convention, w13_order)
    dw = dst.c_struct()
    _check(lib().moe_nvfp4_prepare(ctypes.byref(c), first_expert, count, ctypes.byref(dw), _stream(stream)))
    return dst


def moe_nvfp4_strerror(status):
    return lib().moe_nvfp4_strerror(status).decode()


def moe_nvfp4_last_error():
    return lib().moe_nvfp4_last_error().decode()


def moe_nvfp4_workspace_size(problem):
    n = ctypes.c_size_t(0)
    _check(lib().moe_nvfp4_workspace_size(ctypes.byref(problem), ctypes.byref(n)))
    return n.value


def moe_nvfp4_resolved_path(problem):
    """PATH_DECODE, PATH_MID, PATH_PREFILL or PATH_MICRO: the path the forward takes for `problem`."""
    out = ctypes.c_int32(0)
    _check(lib().moe_nvfp4_resolved_path(ctypes.byref(problem), ctypes.byref(out)))
    return out.value


def moe_nvfp4_validate(problem, workspace_bytes, arch=None):
    """Returns the status code (does not raise)."""
    a = arch.encode() if isinstance(arch, str) else arch
    return lib().moe_nvfp4_validate(ctypes.byref(problem), workspace_bytes, a)


def alloc_workspace(problem, device="cuda"):
    n = moe_nvfp4_workspace_size(problem)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def _forward_args(p, hidden, gate_w, local, shared, workspace, out):
    T, d, bf = _rows(p), p.d_model, torch.bfloat16
    (h, g, ws, o), lw, sw = _layer_ptrs(p, [
        (hidden, "hidden", bf, (T, d)), (gate_w, "gate_w", bf, (p.num_experts, d)),
        (workspace, "workspace", torch.uint8, (None,)), (out, "out", bf, (T, d))], local, shared)
    return (ctypes.byref(p), h, g, ctypes.byref(lw), ctypes.byref(sw) if sw is not None else None,
            ws, workspace.numel(), o)


def moe_nvfp4_forward(problem, hidden, gate_w, local, shared, workspace, out, stream=None):
    """hidden bf16 [T, d]; gate_w bf16 [E, d]; local/shared: NVFP4Experts of L and 1
    experts (shared may be None); workspace uint8 [n] device tensor; out bf16 [T, d]
    (overwritten).  Tensors of another dtype or shape raise ValueError."""
    _check(lib().moe_nvfp4_forward(*_forward_args(problem, hidden, gate_w, local, shared, workspace, out),
                                   _stream(stream)))
    return out


def moe_nvfp4_forward_timed(problem, hidden, gate_w, local, shared, workspace, out, events,
                            stream=None):
    """moe_nvfp4_forward recording raw hipEvent_t handles (ints, or None) at the
    kernel boundaries; see the header for the event slots."""
    args = _forward_args(problem, hidden, gate_w, local, shared, workspace, out)
    arr = (ctypes.c_void_p * len(events))(*[e if e else None for e in events])
    _check(lib().moe_nvfp4_forward_timed(*args, _stream(stream), arr, len(events)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20     # MOE_NVFP4_NOALLOC_SCRATCH_BYTES


def moe_nvfp4_forward_noalloc(problem, hidden, gate_w, local, shared, out, stream=None):
    """moe_nvfp4_forward without a workspace: the library's own per-device
    scratch (NOALLOC_SCRATCH_BYTES) serves; problems needing more raise.  Calls
    that overlap on one device race (they share the scratch)."""
    p, T, d, bf = problem, _rows(problem), problem.d_model, torch.bfloat16
    (h, g, o), lw, sw = _layer_ptrs(p, [
        (hidden, "hidden", bf, (T, d)), (gate_w, "gate_w", bf, (p.num_experts, d)),
        (out, "out", bf, (T, d))], local, shared)
    _check(lib().moe_nvfp4_forward_noalloc(ctypes.byref(p), h, g, ctypes.byref(lw),
                                           ctypes.byref(sw) if sw is not None else None, o, _stream(stream)))
    return out


def moe_nvfp4_route(problem, hidden, gate_w, workspace, topk_ids=None, topk_w=None, counts=None,
                    offsets=None, perm=None, stream=None):
    """Routing and permutation only.  hidden bf16 [T, d], gate_w bf16 [E, d];
    optional outputs topk_ids int32 [T, k], topk_w fp32 [T, k], counts int32 [L],
    offsets int32 [L + 1], perm int32 [T k]."""
    p, i32 = problem, torch.int32
    T, k, L = _rows(p), p.top_k, p.num_local_experts
    ptrs = _ptrs((hidden, "hidden", torch.bfloat16, (T, p.d_model)),
                 (gate_w, "gate_w", torch.bfloat16, (p.num_experts, p.d_model)),
                 (topk_ids, "topk_ids", i32, (T, k)), (topk_w, "topk_w", torch.float32, (T, k)),
                 (counts, "counts", i32, (L,)), (offsets, "offsets", i32, (L + 1,)),
                 (perm, "perm", i32, (p.num_tokens * k,)), (workspace, "workspace", torch.uint8, (None,)))
    _check(lib().moe_nvfp4_route(ctypes.byref(p), *ptrs, workspace.numel(), _stream(stream)))


def moe_nvfp4_quantize_weights(w, codes, scales, global_scale, stream=None):
    """w bf16 [n, R, C] -> codes uint8 [n, R, C/2], scales uint8 [n, R, C/16], global fp32 [n]."""
    n, R, C = w.shape
    u8 = torch.uint8
    pw, pc, ps, pg = _ptrs((w, "w", torch.bfloat16, (n, R, C)), (codes, "codes", u8, (n, R, C // 2)),
                           (scales, "scales", u8, (n, R, C // 16)),
                           (global_scale, "global_scale", torch.float32, (n,)))
    _check(lib().moe_nvfp4_quantize_weights(pw, n, R, C, pc, ps, pg, _stream(stream)))


def _act_ptrs(x, codes, scales):
    R, C = x.shape
    return _ptrs((x, "x", torch.bfloat16, (R, C)), (codes, "codes", torch.uint8, (R, C // 2)),
                 (scales, "scales", torch.uint8, (R, C // 16)))


def moe_nvfp4_quantize_activations(x, codes, scales, stream=None):
    """x bf16 [R, C] -> codes uint8 [R, C/2], scales uint8 [R, C/16]."""
    R, C = x.shape
    px, pc, ps = _act_ptrs(x, codes, scales)
    _check(lib().moe_nvfp4_quantize_activations(px, R, C, pc, ps, _stream(stream)))


def moe_nvfp4_quantize_activations_static(x, g, codes, scales, stream=None):
    """Static W4A4 rule with activation global g: x bf16 [R, C] -> codes uint8
    [R, C/2], scales uint8 [R, C/16]."""
    R, C = x.shape
    px, pc, ps = _act_ptrs(x, codes, scales)
    _check(lib().moe_nvfp4_quantize_activations_static(px, R, C, float(g), pc, ps, _stream(stream)))


def quantize_experts(w13, w2, out=None, start=0):
    """Quantize bf16 expert weights w13 [n, 2F, d], w2 [n, d, F] into `out`
    (an NVFP4Experts, experts [start, start+n)) on the GPU."""
    n, twoF, d = w13.shape
    F = twoF // 2
    if out is None:
        out = NVFP4Experts.empty(n, d, F, device=w13.device)
        start = 0
    moe_nvfp4_quantize_weights(w13, out.w13[start:start + n], out.w13_scale[start:start + n],
                               out.w13_global[start:start + n])
    moe_nvfp4_quantize_weights(w2, out.w2[start:start + n], out.w2_scale[start:start + n],
                               out.w2_global[start:start + n])
    return out
