"""The Python binding checks every tensor's dtype and shape against the problem
before any pointer reaches the library (CPU only: checks come before the GPU
check, so correctly shaped host tensors stop at "must be on the GPU")."""
import pytest
import torch

import nvfp4_expert_layer_amd as nv

T, D, F, E, K, L = 4, 256, 128, 16, 2, 16
BF = torch.bfloat16


def args(**over):
    a = dict(problem=nv.make_problem(T, D, F, E, K, 0, L, True, nv.W4A16),
             hidden=torch.zeros(T, D, dtype=BF), gate_w=torch.zeros(E, D, dtype=BF),
             local=nv.NVFP4Experts.empty(L, D, F, device="cpu"), shared=nv.NVFP4Experts.empty(1, D, F, device="cpu"),
             workspace=torch.zeros(64, dtype=torch.uint8), out=torch.zeros(T, D, dtype=BF))
    a.update(over)
    return a


def forward(a):
    nv.moe_nvfp4_forward(a["problem"], a["hidden"], a["gate_w"], a["local"], a["shared"], a["workspace"], a["out"])


@pytest.mark.parametrize("over,msg", [
    (dict(hidden=torch.zeros(T - 1, D, dtype=BF)), "hidden: shape"),
    (dict(hidden=torch.zeros(T, D, dtype=torch.float32)), "hidden: dtype"),
    (dict(hidden=torch.zeros(T * D, dtype=BF)), "hidden: shape"),
    (dict(gate_w=torch.zeros(E - 1, D, dtype=BF)), "gate_w: shape"),
    (dict(out=torch.zeros(T, D // 2, dtype=BF)), "out: shape"),
    (dict(local=nv.NVFP4Experts.empty(L - 1, D, F, device="cpu")), "local.w13: shape"),
    (dict(local=nv.NVFP4Experts.empty(L, D, F // 2, device="cpu")), "local.w13: shape"),
    (dict(shared=nv.NVFP4Experts.empty(2, D, F, device="cpu")), "shared.w13: shape"),
    (dict(workspace=torch.zeros(16, dtype=torch.int32)), "workspace: dtype"),
    (dict(workspace=torch.zeros(4, 16, dtype=torch.uint8)), "workspace: shape"),
])
def test_forward_rejects_mismatched_tensors(over, msg):
    with pytest.raises(ValueError, match=msg):
        forward(args(**over))


def test_forward_checks_every_expert_tensor():
    bad = nv.NVFP4Experts.empty(L, D, F, device="cpu")
    bad.w2_global = torch.zeros(L, dtype=torch.float64)
    with pytest.raises(ValueError, match="local.w2_global: dtype"):
        forward(args(local=bad))
    bad = nv.NVFP4Experts.empty(L, D, F, device="cpu")
    bad.w2_scale = bad.w2_scale[:, :, :4]
    with pytest.raises(ValueError, match="local.w2_scale: shape"):
        forward(args(local=bad))


def test_well_formed_host_tensors_stop_at_the_device_check():
    with pytest.raises(ValueError, match="must be on the GPU"):
        forward(args())
    with pytest.raises(ValueError, match="must be on the GPU"):
        forward(args(shared=None))
    # an empty batch takes token tensors of any row count (no rows are read)
    p0 = nv.make_problem(0, D, F, E, K, 0, L, True, nv.W4A16)
    with pytest.raises(ValueError, match="must be on the GPU"):
        forward(args(problem=p0, hidden=torch.zeros(E, D, dtype=BF), out=torch.zeros(1, D, dtype=BF)))


@pytest.mark.parametrize("name,tensor,msg", [
    ("topk_ids", torch.zeros(T, K + 1, dtype=torch.int32), "topk_ids: shape"),
    ("topk_w", torch.zeros(T, K, dtype=torch.float16), "topk_w: dtype"),
    ("counts", torch.zeros(L - 1, dtype=torch.int32), "counts: shape"),
    ("offsets", torch.zeros(L, dtype=torch.int32), "offsets: shape"),
    ("perm", torch.zeros(T * K - 1, dtype=torch.int32), "perm: shape"),
])
def test_route_rejects_mismatched_outputs(name, tensor, msg):
    a = args()
    with pytest.raises(ValueError, match=msg):
        nv.moe_nvfp4_route(a["problem"], a["hidden"], a["gate_w"], a["workspace"], **{name: tensor})


def test_quantizers_reject_mismatched_outputs():
    u8 = torch.uint8
    x = torch.zeros(8, 64, dtype=BF)
    with pytest.raises(ValueError, match="codes: shape"):
        nv.moe_nvfp4_quantize_activations(x, torch.zeros(8, 16, dtype=u8), torch.zeros(8, 4, dtype=u8))
    with pytest.raises(ValueError, match="scales: shape"):
        nv.moe_nvfp4_quantize_activations_static(x, 1.0, torch.zeros(8, 32, dtype=u8), torch.zeros(8, 2, dtype=u8))
    w = torch.zeros(2, 8, 64, dtype=BF)
    with pytest.raises(ValueError, match="global_scale: shape"):
        nv.moe_nvfp4_quantize_weights(w, torch.zeros(2, 8, 32, dtype=u8), torch.zeros(2, 8, 4, dtype=u8),
                                      torch.zeros(1, dtype=torch.float32))
    with pytest.raises(ValueError, match="must be on the GPU"):
        nv.moe_nvfp4_quantize_weights(w, torch.zeros(2, 8, 32, dtype=u8), torch.zeros(2, 8, 4, dtype=u8),
                                      torch.zeros(2, dtype=torch.float32))


def test_prepare_checks_checkpoint_and_destination():
    ck = nv.NVFP4Experts.empty(6, D, F, device="cpu")
    dst = nv.NVFP4Experts.empty(2, D, F, device="cpu")
    with pytest.raises(ValueError, match="dst.w13: 2 experts, expected at least 3"):
        nv.moe_nvfp4_prepare(ck, 0, 0, 1, 3, dst)
    bad = nv.NVFP4Experts.empty(2, D, F // 2, device="cpu")
    with pytest.raises(ValueError, match="dst.w13: shape"):
        nv.moe_nvfp4_prepare(ck, 0, 0, 1, 2, bad)
    ck.w2_scale = ck.w2_scale[:5]
    with pytest.raises(ValueError, match="ck.w2_scale: shape"):
        nv.moe_nvfp4_prepare(ck, 0, 0, 1, 2, dst)
    ck = nv.NVFP4Experts.empty(6, D, F, device="cpu")
    with pytest.raises(ValueError, match="must be on the GPU"):
        nv.moe_nvfp4_prepare(ck, 0, 0, 1, 2, dst)


def test_tensors_and_stream_of_another_device_are_refused(monkeypatch):
    """The library launches on the current device: a tensor or a stream of
    another device is refused before any pointer reaches it."""
    from types import SimpleNamespace
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    other = SimpleNamespace(is_cuda=True, device=torch.device("cuda", 1), get_device=lambda: 1,
                            is_contiguous=lambda: True, data_ptr=lambda: 0)
    with pytest.raises(ValueError, match="current device is cuda:0"):
        nv._ptr(other)
    stream = SimpleNamespace(device=torch.device("cuda", 1), device_index=1, cuda_stream=0)
    with pytest.raises(ValueError, match="current device is cuda:0"):
        nv._stream(stream)


def test_weight_structs_carry_each_tensor_in_its_field(monkeypatch):
    """The forward's weight structs are built from the checked pointers: each
    field must hold the pointer of the tensor of the same name (local and shared)."""
    import ctypes
    monkeypatch.setattr(nv, "_ptr", lambda t, cur=None: None if t is None else ctypes.c_void_p(id(t)))
    a = args()
    fields = ("w13", "w13_scale", "w13_global", "w2", "w2_scale", "w2_global")
    for shared in (a["shared"], None):
        out = nv._forward_args(a["problem"], a["hidden"], a["gate_w"], a["local"], shared, a["workspace"], a["out"])
        h, g, ws, o = out[1], out[2], out[5], out[7]
        assert (h.value, g.value, ws.value, o.value) == (id(a["hidden"]), id(a["gate_w"]), id(a["workspace"]),
                                                         id(a["out"]))
        lw = out[3]._obj
        assert [getattr(lw, f) for f in fields] == [id(getattr(a["local"], f)) for f in fields]
        if shared is None:
            assert out[4] is None
        else:
            sw = out[4]._obj
            assert [getattr(sw, f) for f in fields] == [id(getattr(shared, f)) for f in fields]
