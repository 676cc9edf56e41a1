"""The C-ABI library loads and exports every declared entry point, and host
validation rejects bad arguments before anything reaches a device.

These tests make no compute call: every call here fails validation on the
host (or only queries a workspace size), so no GPU is needed.
"""
import ctypes
import os
import re

import pytest

import moe_expert_dispatch_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def so():
    if not os.path.exists(moe.library_path()):
        pytest.fail("libmoe_hip.so not built: run __graft_entry__.build()")
    return moe.lib()


def test_exports_every_declared_symbol(so):
    names = declared_symbols()
    assert set(names) == set(moe.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(so, n), n


def test_status_strings(so):
    for code in range(5):
        assert moe.status_str(code).startswith("MOE_")


def test_route_validation(so):
    f = so.moe_route
    assert f(None, 4, 4, 5, 1, None, None, None) == INVALID      # K > E
    assert f(None, 4, 4, 0, 1, None, None, None) == INVALID      # K < 1
    assert f(None, -1, 4, 2, 1, None, None, None) == INVALID     # T < 0
    assert f(None, 4, 4, 2, 1, None, None, None) == INVALID      # null pointers
    assert f(None, 4, 2048, 2, 1, None, None, None) == UNSUPPORTED  # E > 1024
    assert f(None, 4, 64, 33, 1, None, None, None) == UNSUPPORTED   # K > 32


def test_route_grouped_validation(so):
    f = so.moe_route_grouped
    fake = ctypes.c_void_p(256)

    def call(E=16, K=3, G=4, TG=2, T=4):
        return f(fake, T, E, K, 1, G, TG, fake, fake, None)
    assert call(G=0) == INVALID
    assert call(TG=0) == INVALID
    assert call(TG=5) == INVALID           # more groups kept than exist
    assert call(G=3) == INVALID            # 16 % 3
    assert call(K=9, TG=2) == INVALID      # two groups of 4 hold only 8 experts
    assert call(E=256, K=4, G=128, TG=2) == UNSUPPORTED
    assert f(None, 4, 16, 3, 1, 4, 2, None, None, None) == INVALID  # null pointers


def test_slot_map_validation(so):
    f = so.moe_slot_map
    # E_global % ep_size != 0 (the divisibility the EP partition asserts)
    assert f(None, None, 1, 2, 10, 4, 0, None, None, 2, None, None, None, None) == INVALID
    # ep_rank out of range
    assert f(None, None, 1, 2, 8, 4, 4, None, None, 2, None, None, None, None) == INVALID
    # S < E_local
    assert f(None, None, 1, 2, 8, 2, 0, None, None, 3, None, None, None, None) == INVALID
    # identity table needs S == E_local
    assert f(None, None, 1, 2, 8, 2, 0, None, None, 5, None, None, None, None) == INVALID
    # null data pointers
    assert f(None, None, 1, 2, 8, 2, 0, None, None, 4, None, None, None, None) == INVALID


def test_permute_validation_and_workspace(so):
    ws = so.moe_permute_workspace_size
    assert ws(0, 1, 1) > 0
    assert ws(-1, 1, 1) == 0
    # monotone in T for a fixed (K, S)
    sizes = [ws(t, 8, 80) for t in range(0, 70000, 997)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))
    f = so.moe_permute
    assert f(None, 1, 4, 12, 2, None, None, 4, None, None, None, None, None, 0, None) == UNSUPPORTED  # H % 8
    assert f(None, 1, 4, 16, 2, None, None, 4, None, None, None, None, None, 0, None) == INVALID
    assert f(None, 7, 4, 16, 2, None, None, 4, None, None, None, None, None, 0, None) == UNSUPPORTED
    fake = ctypes.c_void_p(256)
    assert f(None, 1, 4, 16, 2, fake, fake, 4, fake, fake, fake, None, None, 0, None) == WORKSPACE


def test_gemm_validation(so):
    f = so.moe_grouped_gemm
    fake = ctypes.c_void_p(256)
    assert f(5, 1, fake, fake, 4, 16, fake, 64, 64, fake, None) == INVALID   # bad op
    assert f(0, 1, fake, fake, 0, 16, fake, 64, 64, fake, None) == INVALID   # S < 1
    assert f(0, 1, fake, fake, 4, 16, fake, 60, 64, fake, None) == UNSUPPORTED  # H % 8
    assert f(0, 1, fake, fake, 4, 16, fake, 64, 68, fake, None) == UNSUPPORTED  # I % 8
    assert f(0, 1, ctypes.c_void_p(264), fake, 4, 16, fake, 64, 64, fake, None) == INVALID  # misaligned
    assert f(0, 1, None, fake, 4, 16, fake, 64, 64, fake, None) == INVALID   # null a


def test_combine_validation(so):
    f = so.moe_combine
    fake = ctypes.c_void_p(256)
    assert f(fake, 1, fake, fake, 4, 0, 64, fake, 1, 0, None) == INVALID     # K < 1
    assert f(fake, 1, fake, fake, 4, 2, 60, fake, 1, 0, None) == UNSUPPORTED  # H % 8
    assert f(None, 1, fake, fake, 4, 2, 64, fake, 1, 0, None) == INVALID
    assert f(fake, 1, fake, fake, 4, 2, 64, ctypes.c_void_p(260), 1, 0, None) == INVALID


def test_a2a_validation_and_workspace(so):
    ws = moe.a2a_dispatch_workspace_size
    assert ws(64, 4, 64) > 0
    assert ws(0, 2, 0) > 0            # empty batch still has a layout
    assert ws(64, 4, 32) == 0         # cap < T
    assert ws(64, 0, 64) == 0
    assert ws(64, 33, 64) == 0        # more ranks than supported
    f = so.moe_a2a_dispatch
    fake = ctypes.c_void_p(256)
    big = ctypes.c_size_t(1 << 30)

    def call(x=fake, dt=1, T=8, H=64, K=2, E=8, ep=2, cap=8, send_x=fake, wsz=big):
        return f(x, dt, T, H, K, fake, fake, E, ep, cap, fake, fake, fake, send_x, fake, fake,
                 fake, wsz, None)
    assert call(cap=4) == INVALID                      # block could overflow
    assert call(E=9) == INVALID                        # E % ep_size
    assert call(ep=0) == INVALID
    assert call(ep=64, E=64) == UNSUPPORTED
    assert call(K=33, E=64) == UNSUPPORTED
    assert call(H=4) == UNSUPPORTED                    # 8-byte rows
    assert call(dt=7) == UNSUPPORTED
    assert call(x=None) == INVALID
    assert call(send_x=ctypes.c_void_p(264)) == INVALID  # misaligned
    assert call(wsz=ctypes.c_size_t(16)) == WORKSPACE
    g = so.moe_a2a_combine
    assert g(fake, 1, fake, 8, 0, 64, fake, 1, None) == INVALID
    assert g(fake, 1, fake, 8, 2, 60, fake, 1, None) == UNSUPPORTED
    assert g(fake, 1, fake, 8, 33, 64, fake, 1, None) == UNSUPPORTED
    assert g(None, 1, fake, 8, 2, 64, fake, 1, None) == INVALID


def test_scaled_permute_and_shared_combine_validation(so):
    fake = ctypes.c_void_p(256)
    big = ctypes.c_size_t(1 << 30)
    f = so.moe_permute_scaled
    # pair_w missing, x_perm missing: rejected before any launch
    assert f(fake, 1, 4, 64, 2, fake, fake, 4, None, fake, fake, fake, fake, fake, big,
             None) == INVALID
    assert f(fake, 1, 4, 64, 2, fake, fake, 4, fake, fake, fake, fake, None, fake, big,
             None) == INVALID
    g = so.moe_combine_shared
    assert g(fake, 1, fake, None, 4, 0, 64, None, 1, fake, 1, 0, None) == INVALID   # K < 1
    assert g(fake, 1, fake, None, 4, 2, 64, fake, 9, fake, 1, 0, None) == UNSUPPORTED
    assert g(fake, 1, fake, None, 4, 2, 64, ctypes.c_void_p(264), 1, fake, 1, 0,
             None) == INVALID  # misaligned shared rows
    assert g(None, 1, fake, None, 4, 2, 64, None, 1, fake, 1, 0, None) == INVALID


def _cfg(**kw):
    base = dict(T=16, H=64, I=64, E_global=8, K=2, renormalize=True, S=8,
                dtype=__import__("torch").bfloat16)
    base.update(kw)
    return moe.ForwardConfig(**base)


def test_forward_workspace_and_validation(so):
    c = _cfg()
    n = so.moe_forward_workspace_size(ctypes.byref(c.c_struct()))
    P = 16 * 2
    assert n >= P * (4 * 6 + 1) + P * 64 * 2 * 2  # index arrays + x_perm + activations
    bad = [_cfg(K=9), _cfg(E_global=10, ep_size=4), _cfg(ep_size=2, ep_rank=2, S=4),
           _cfg(S=3), _cfg(H=60), _cfg(T=32, T_max=16),
           _cfg(num_expert_group=3, topk_group=1),      # 8 % 3
           _cfg(num_expert_group=4, topk_group=0),
           _cfg(num_expert_group=8, topk_group=1, K=2)]  # one group of 1 expert < K
    assert so.moe_forward_workspace_size(
        ctypes.byref(_cfg(num_expert_group=4, topk_group=2).c_struct())) > 0
    for b in bad:
        assert so.moe_forward_workspace_size(ctypes.byref(b.c_struct())) == 0
    # workspace too small is reported before any launch
    args = moe._ForwardArgs()
    fake = 256
    for name in ("x", "logits", "w_gate_up", "w_down", "out"):
        setattr(args, name, fake)
    st = so.moe_forward(ctypes.byref(c.c_struct()), ctypes.byref(args), ctypes.c_void_p(256),
                        n - 1, None)
    assert st == WORKSPACE
    # identity table with S != E_local
    c2 = _cfg(S=9)
    n2 = so.moe_forward_workspace_size(ctypes.byref(c2.c_struct()))
    st = so.moe_forward(ctypes.byref(c2.c_struct()), ctypes.byref(args), ctypes.c_void_p(256),
                        n2, None)
    assert st == INVALID


def test_python_layer_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        moe.route(torch.zeros(4, 8), 2, True)


def test_quantize_fp8_validation(so):
    f = so.moe_quantize_fp8
    fake = ctypes.c_void_p(256)
    assert f(fake, 1, -1, 1.0, fake, None) == INVALID                  # n < 0
    assert f(fake, 1, 16, 0.0, fake, None) == INVALID                  # scale <= 0
    assert f(fake, 1, 16, float("nan"), fake, None) == INVALID
    assert f(fake, 1, 16, float("inf"), fake, None) == INVALID
    assert f(fake, 2, 16, 1.0, fake, None) == UNSUPPORTED              # fp8 input
    assert f(None, 1, 16, 1.0, fake, None) == INVALID                  # null x
    assert f(fake, 1, 16, 1.0, ctypes.c_void_p(264), None) == INVALID  # misaligned q
    assert f(None, 1, 0, 1.0, None, None) == 0                         # empty: no work


def test_grouped_gemm_fp8_validation(so):
    f = so.moe_grouped_gemm_fp8
    fake = ctypes.c_void_p(256)

    def call(op=0, a_scale=1.0, S=4, rows=16, H=256, I=256, c_scale=1.0, w_scale=fake, a=fake):
        return f(op, a, a_scale, fake, S, rows, fake, w_scale, H, I, fake, c_scale, None)

    assert call(op=5) == INVALID
    assert call(a_scale=0.0) == INVALID
    assert call(c_scale=-1.0) == INVALID              # gate/up output scale
    assert call(w_scale=None) == INVALID
    assert call(a=None) == INVALID
    assert call(H=192) == UNSUPPORTED                 # gate/up contraction not a multiple of 128
    assert call(H=128) == UNSUPPORTED                 # one 128-wide slice only
    assert call(op=1, I=320) == UNSUPPORTED           # down contraction is I
    # zero rows: validation passes and nothing is launched; down ignores c_scale
    assert call(op=1, c_scale=0.0, H=64, rows=0) == 0
    assert call(op=0, c_scale=0.0, rows=0) == INVALID


def test_forward_fp8_config_validation(so):
    import torch
    ok = _cfg(H=256, I=256, dtype=moe.FP8, a1_scale=0.5, a2_scale=0.25)
    n = so.moe_forward_workspace_size(ctypes.byref(ok.c_struct()))
    P = 16 * 2
    # bf16 expert outputs, fp8 activations and the quantized input
    assert n >= P * 256 * 2 + P * 256 + 16 * 256
    assert ok.out_dtype == torch.bfloat16
    bad = [_cfg(H=192, I=256, dtype=moe.FP8),              # H % 128
           _cfg(H=256, I=128, dtype=moe.FP8),              # I < 256
           _cfg(H=256, I=256, dtype=moe.FP8, a1_scale=0.0),
           _cfg(H=256, I=256, dtype=moe.FP8, a2_scale=float("nan")),
           _cfg(H=256, I=256, dtype=moe.FP8, routing_on_input=True),
           _cfg(H=256, I=256, dtype=moe.FP8, out_dtype=moe.FP8)]
    for b in bad:
        assert so.moe_forward_workspace_size(ctypes.byref(b.c_struct())) == 0
    # missing weight scales are rejected before any launch
    args = moe._ForwardArgs()
    for name in ("x", "logits", "w_gate_up", "w_down", "out"):
        setattr(args, name, 256)
    st = so.moe_forward(ctypes.byref(ok.c_struct()), ctypes.byref(args), ctypes.c_void_p(256),
                        n, None)
    assert st == INVALID


def test_weight_panel_limit(so):
    """A slot's gate/up panel (2 * I * H elements) must stay under 2^31 bytes:
    the GEMMs address it with 32-bit buffer offsets and use 2^31 as their
    out-of-range offset. Zero rows: validation runs, nothing is launched."""
    fake = ctypes.c_void_p(256)
    g = so.moe_grouped_gemm
    for op in (0, 1):
        assert g(op, 1, fake, fake, 4, 0, fake, 16384, 32768, fake, None) == UNSUPPORTED
        assert g(op, 1, fake, fake, 4, 0, fake, 16384, 32760, fake, None) == 0
        assert g(op, 0, fake, fake, 4, 0, fake, 16384, 16384, fake, None) == UNSUPPORTED  # f32
        assert g(op, 0, fake, fake, 4, 0, fake, 16384, 16376, fake, None) == 0
    f8 = so.moe_grouped_gemm_fp8
    for op in (0, 1):
        assert f8(op, fake, 1.0, fake, 4, 0, fake, fake, 32768, 32768, fake, 1.0,
                  None) == UNSUPPORTED
        assert f8(op, fake, 1.0, fake, 4, 0, fake, fake, 32768, 32640, fake, 1.0, None) == 0
    ws = so.moe_forward_workspace_size
    assert ws(ctypes.byref(_cfg(H=16384, I=32768).c_struct())) == 0
    assert ws(ctypes.byref(_cfg(H=16384, I=32760, T=1).c_struct())) > 0


def test_gemm_blocks_validation(so):
    ws = so.moe_forward_workspace_size
    assert ws(ctypes.byref(_cfg(gemm_blocks=-1).c_struct())) == 0
    assert ws(ctypes.byref(_cfg(gemm_blocks=8).c_struct())) == \
        ws(ctypes.byref(_cfg().c_struct()))
