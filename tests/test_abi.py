"""CPU checks of the C ABI: the library loads, exports every declared symbol, and its
host-only entry points (sizes, layout, argument validation) behave as documented.
Validation failures return before any HIP call, so these run without a GPU."""

import ctypes
import os
import re

import pytest

import routed_moe_layer_amd as rm

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "routed_moe.h")
FULL = rm.MoeDims(3584, 384, 896, 16)
TINY = rm.MoeDims(256, 64, 16, 4)


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(moe_[a-z0-9_]+)\(", text, re.M)))


def test_header_declarations_match_binding():
    assert _declared() == sorted(rm.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(rm.library_path)
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings():
    assert rm.moe_status_string(0) == "ok"
    assert rm.moe_status_string(-3) == "workspace too small"


def test_workspace_size_is_monotone_and_covers_the_layout():
    prev = 0
    for T in (1, 2, 15, 16, 17, 64, 255, 1024, 4097, 16384):
        n = rm.moe_workspace_size(FULL, T)
        assert n >= prev
        prev = n
        lay = rm.moe_workspace_layout(FULL, T)
        assert lay["total"] == n
        offs = sorted(v for k, v in lay.items() if k != "total")
        assert all(o % 256 == 0 for o in offs) and offs[-1] < n
    assert rm.moe_workspace_size(FULL, 16384) < 4 * 2 ** 30


def test_workspace_size_is_monotone_at_every_T_near_the_tile_thresholds():
    # small H and I with many experts, so the tile-list bounds weigh in the layout: every
    # T around 1024 routed rows (small tiles only at or below it) keeps the size monotone,
    # so a workspace sized for max_tokens covers every smaller call
    d = rm.MoeDims(128, 64, 4096, 4)
    prev = 0
    for T in list(range(1, 41)) + list(range(240, 272)):
        n = rm.moe_workspace_size(d, T)
        assert n >= prev, T
        prev = n
        assert rm.moe_workspace_layout(d, T)["total"] == n


def test_prepared_size_matches_the_page_storage_shapes():
    # FC1 [896,768,1792] + [896,768,224], FC2 [896,3584,192] + [896,3584,24]: I = 384 is
    # a multiple of 128, so the prepared layout is exactly as large as the canonical one.
    want = 896 * (768 * 1792 + 768 * 224 + 3584 * 192 + 3584 * 24)
    assert rm.moe_prepared_weights_size(FULL) == want
    # I = 64 pads FC2's K to 128
    assert rm.moe_prepared_weights_size(TINY) == 16 * (128 * 128 + 128 * 16 + 256 * 64 + 256 * 8)


@pytest.mark.parametrize("dims,code", [
    (rm.MoeDims(3584, 384, 896, 0), -1),
    (rm.MoeDims(3500, 384, 896, 16), -2),     # H % 128
    (rm.MoeDims(3584, 96, 896, 16), -2),      # I % 64
    (rm.MoeDims(3584, 384, 5000, 16), -2),    # E too large
    (rm.MoeDims(3584, 384, 896, 65), -2),     # k too large
])
def test_bad_dims_are_rejected(dims, code):
    with pytest.raises(rm.MoeError) as ei:
        rm.moe_workspace_size(dims, 16)
    assert ei.value.status == code


def test_token_count_limits():
    for T in (0, 16385):
        with pytest.raises(rm.MoeError) as ei:
            rm.moe_workspace_size(FULL, T)
        assert ei.value.status == -1


def _forward(**kw):
    args = dict(dims=FULL, T=16, x=4096, expert_ids=8192, route_weights=8192, prepared=1 << 20,
                qx=256, alpha1=512, qa=768, alpha2=1024, situ_beta=None, situ_linear_beta=None,
                workspace=1 << 24, out=1 << 22, workspace_bytes=rm.moe_workspace_size(FULL, 16),
                stream=0)
    args.update(kw)
    rm.moe_forward(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1),
    (dict(out=None), -1),
    (dict(qx=None), -1),
    (dict(x=4097), -1),                        # misaligned
    (dict(workspace=(1 << 24) + 16), -1),      # workspace must be 256-aligned
    (dict(T=0), -1),
    (dict(T=16385), -1),
    (dict(workspace_bytes=100), -3),
    (dict(dims=rm.MoeDims(100, 384, 896, 16)), -2),
])
def test_forward_validation_happens_before_any_hip_call(kw, code):
    with pytest.raises(rm.MoeError) as ei:
        _forward(**kw)
    assert ei.value.status == code


def test_route_validation():
    d = rm.MoeDims(7168, 0, 256, 8)                   # moe_route ignores inter
    ws = rm.moe_route_workspace_size(8192, 8, 256)
    assert rm.moe_workspace_size(d, 8192, rm.MOE_QUANT_INT8_ROW_DYNAMIC) == ws
    assert rm.moe_workspace_size(d, 8192, rm.MOE_QUANT_NONE) == ws
    base = dict(dims=d, T=8192, x=4096, expert_ids=8192, quant=rm.MOE_QUANT_INT8_ROW_DYNAMIC,
                qx=None, sorted_expert_ids=None, sorted_row_idx=None, expanded_row_idx=1 << 22,
                expert_cumsum=1 << 23, expanded_x=1 << 20, expanded_sf_or_scale=1 << 21,
                workspace=1 << 24, workspace_bytes=ws, stream=0)
    for kw, code in ((dict(expanded_sf_or_scale=None), -1), (dict(quant=5), -1),
                     (dict(workspace_bytes=ws - 1), -3),
                     (dict(dims=rm.MoeDims(7, 0, 256, 8)), -2),
                     (dict(dims=rm.MoeDims(7168, 0, 10241, 8)), -2), (dict(T=0), -1),
                     # NVFP4 needs the encoding scale, a scale buffer and H % 16 == 0
                     (dict(quant=rm.MOE_QUANT_NVFP4_G16), -1),
                     (dict(quant=rm.MOE_QUANT_NVFP4_G16, qx=256, expanded_sf_or_scale=None), -1),
                     (dict(quant=rm.MOE_QUANT_NVFP4_G16, qx=256,
                           dims=rm.MoeDims(7160, 0, 256, 8)), -2),
                     (dict(quant=rm.MOE_QUANT_NVFP4_G16, qx=258), -1)):   # misaligned qx
        a = dict(base); a.update(kw)
        with pytest.raises(rm.MoeError) as ei:
            rm.moe_route(**a)
        assert ei.value.status == code


def test_workspace_size_of_the_layer_serves_the_router_in_every_mode():
    for T in (1, 16, 1024, 16384):
        n = rm.moe_workspace_size(FULL, T, rm.MOE_QUANT_NVFP4_G16)
        assert n == rm.moe_workspace_layout(FULL, T)["total"]
        for q in (rm.MOE_QUANT_NONE, rm.MOE_QUANT_INT8_ROW_DYNAMIC):
            assert rm.moe_workspace_size(FULL, T, q) <= n
    # routing-only sizes go past the layer's token limit; the layer's do not
    assert rm.moe_workspace_size(FULL, 65536, rm.MOE_QUANT_NONE) > 0
    with pytest.raises(rm.MoeError):
        rm.moe_workspace_size(FULL, 16385, rm.MOE_QUANT_NVFP4_G16)
    with pytest.raises(rm.MoeError):
        rm.moe_workspace_size(FULL, 16, 7)


def test_route_v2_validation():
    ws = rm.moe_route_workspace_size(64, 8, 32)
    base = dict(num_rows=64, hidden=256, num_experts=32, top_k=8, x=4096, expert_idx=8192,
                expanded_x=1 << 20, expanded_row_idx=1 << 22, expert_tokens=1 << 23,
                expanded_scale=1 << 21, available_idx_num=None, scale=None, offset=None,
                workspace=1 << 24, workspace_bytes=ws, stream=0)
    O = rm.MoeRouteOptions
    cases = [
        (dict(options=O(expert_start=4, expert_end=4)), -1),            # empty range
        (dict(options=O(expert_start=0, expert_end=33)), -1),           # past num_experts
        (dict(options=O(expert_start=-1, expert_end=3)), -1),
        (dict(options=O(row_idx_type=2)), -1),
        (dict(options=O(expert_tokens_num_type=3)), -1),
        (dict(options=O(quant_mode=2)), -1),
        (dict(options=O(quant_mode=0)), -1),                             # static needs scale
        (dict(options=O(quant_mode=0), scale=256), -1),                 # ... and offset
        (dict(options=O(quant_mode=1), expanded_scale=None), -1),
        (dict(options=O(quant_mode=-1), scale=256, expanded_scale=None), -1),
        (dict(options=O(drop_pad_mode=2)), -1),
        (dict(options=O(drop_pad_mode=1, expert_capacity=0)), -1),
        (dict(options=O(drop_pad_mode=1, expert_capacity=513)), -1),    # > N*K
        (dict(options=O(drop_pad_mode=1, expert_capacity=4, row_idx_type=1)), -1),
        (dict(options=O(drop_pad_mode=1, expert_capacity=4, expert_start=0, expert_end=16)), -1),
        (dict(options=O(drop_pad_mode=1, expert_capacity=4, active_num=10)), -1),
        (dict(options=O(), workspace_bytes=ws - 1), -3),
        (dict(options=O(), hidden=12), -2),
        (dict(options=O(), x=4098), -1),
        (dict(options=O(), expanded_row_idx=None), -1),
        # the page's expert_num limits: 10240, and 5120 with the key_value histogram
        (dict(options=O(), num_experts=10241), -2),
        (dict(options=O(expert_tokens_num_type=2), num_experts=5121), -2),
    ]
    for kw, code in cases:
        a = dict(base); a.update(kw)
        with pytest.raises(rm.MoeError) as ei:
            rm.moe_route_v2(**a)
        assert ei.value.status == code, kw


def test_route_workspace_holds_the_position_map():
    # tile histograms + counts + offsets + one int32 per routed row, 256-byte aligned
    n = 8192 * 8
    assert rm.moe_route_workspace_size(8192, 8, 256) >= (n // 1024) * 256 * 4 + 257 * 4 + 4 * n


def test_topk_softmax_validation():
    base = dict(T=16, num_experts=896, top_k=16, logits=4096, expert_ids=8192,
                route_weights=16384, stream=0)
    for kw, code in ((dict(T=0), -1), (dict(top_k=0), -1), (dict(top_k=897), -1),
                     (dict(num_experts=5000, top_k=8), -2), (dict(top_k=65, num_experts=100), -2),
                     (dict(logits=None), -1), (dict(logits=4098), -1),
                     (dict(route_weights=16385), -1)):
        a = dict(base); a.update(kw)
        with pytest.raises(rm.MoeError) as ei:
            rm.moe_topk_softmax(**a)
        assert ei.value.status == code, kw


def test_quantize_validation():
    for kw in (dict(K=24), dict(src=None), dict(src=4098), dict(groups=0)):
        a = dict(src=4096, groups=1, rows_per_group=4, K=256, q=256, codes=8192, scales=16384,
                 stream=0)
        a.update(kw)
        with pytest.raises(rm.MoeError) as ei:
            rm.moe_quantize_nvfp4(**a)
        assert ei.value.status == -1


def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(rm, "_lib_handle", None)
    monkeypatch.setattr(rm, "library_path", "/nonexistent/libroutedmoe.so")
    with pytest.raises(RuntimeError, match="not built"):
        rm.moe_workspace_size(FULL, 16)


def test_plain_c_program_uses_the_abi(tmp_path):
    """A C program compiled with gcc against include/routed_moe.h and linked to the shared
    library calls the host-side entry points and the validation paths."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    root = os.path.dirname(os.path.dirname(__file__))
    libdir = os.path.dirname(rm.library_path)
    exe = tmp_path / "abi_check"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(root, "include"),
                    os.path.join(root, "tests", "c", "abi_check.c"), "-L", libdir,
                    "-lroutedmoe", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"


def test_routing_takes_the_pages_expert_counts():
    for E in (4097, 5120, 10240):
        assert rm.moe_route_workspace_size(64, 8, E) > 0
    d = rm.MoeDims(256, 0, 10240, 8)
    assert rm.moe_workspace_size(d, 64, rm.MOE_QUANT_NONE) == rm.moe_route_workspace_size(64, 8, 10240)
    with pytest.raises(rm.MoeError):
        rm.moe_route_workspace_size(64, 8, 10241)
    with pytest.raises(rm.MoeError):                   # the layer stays at 4096 experts
        rm.moe_workspace_size(rm.MoeDims(256, 64, 4097, 8), 16)
