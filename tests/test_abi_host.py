"""Host-side checks of the C ABI (no GPU): the library loads, exports every function
include/moe.h declares, and validates layers and arguments before any launch."""
import ctypes
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", src, flags=re.M)) - {"if"})


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("moe_route", "moe_expert_forward", "moe_forward", "quantize_nvfp4_4o6", "moe_requant_mxfp4",
              "moe_requant_nvfp4", "moe_requant_mxfp8", "moe_requant_fp8_block_mxfp4",
              "moe_layer_check",
              "moe_workspace_bytes", "moe_workspace_init", "moe_xq_bytes", "moe_last_error",
              "moe_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    so = ctypes.CDLL(lib.LIB_PATH)
    for n in _declared_functions():
        assert hasattr(so, n), n
    assert so.moe_abi_version() == 5


def _fake_layer(lib, name, **over):
    """A moe_layer_t with non-NULL aligned dummy pointers: only host checks read it."""
    cfg = synth.CONFIGS[name]
    s = lib.LayerT()
    s.H, s.I, s.E, s.k = cfg.H, cfg.I, cfg.E, cfg.k
    s.has_shared, s.I_shared = int(cfg.has_shared), cfg.Ish if cfg.has_shared else 0
    s.wfmt, s.shared_wfmt, s.afmt = lib.WFMT[cfg.wfmt], lib.WFMT[cfg.shared_wfmt], lib.AFMT[cfg.afmt]
    p = 1 << 20
    s.router_w = p
    for f in ("w13", "w2", "sh13", "sh2"):
        setattr(s, f, lib.WeightsT(p, p, p))
    for k, v in over.items():
        setattr(s, k, v)
    return s


def _check(lib, s, max_tokens):
    buf = ctypes.create_string_buffer(2048)
    st = lib.lib().moe_layer_check(ctypes.byref(s), max_tokens, buf, len(buf))
    return st, buf.value.decode()


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_every_config_is_accepted_and_sized(lib, name):
    s = _fake_layer(lib, name)
    for T in (1, 8, 64):
        st, why = _check(lib, s, T)
        assert st == 0, why
        assert lib.lib().moe_workspace_bytes(ctypes.byref(s), T) > 0
    assert lib.lib().moe_workspace_bytes(ctypes.byref(s), 8) <= lib.lib().moe_workspace_bytes(ctypes.byref(s), 64)


def test_default_deny_lists_every_reason(lib):
    s = _fake_layer(lib, "flint_w4a16", H=100, k=0, afmt=1, router_w=None)
    st, why = _check(lib, s, 257)
    assert st == lib.MOE_EUNSUPPORTED
    assert "H=100" in why and "k=0" in why and "max_tokens=257" in why
    assert "router_w is NULL" in why
    s = _fake_layer(lib, "mistral_mxfp4", afmt=1)
    st, why = _check(lib, s, 8)
    assert "NVFP4_4O6 needs NVFP4" in why
    s = _fake_layer(lib, "flint_w4a16", router_score=5, bias_select_only=2)
    st, why = _check(lib, s, 8)
    assert st == lib.MOE_EUNSUPPORTED
    assert "router_score=5" in why and "bias_select_only must be 0 or 1" in why
    s = _fake_layer(lib, "flint_w4a16", shared_wfmt=2)
    st, why = _check(lib, s, 8)
    assert "shared expert must use" in why
    assert lib.lib().moe_workspace_bytes(ctypes.byref(s), 8) == 0


def test_nvfp4_row_lengths(lib):
    # NVFP4 walks stage a batch's block scales in 16-byte chunks: K a multiple of 256 plans
    # at any length (H = 7168: 7 batches per row; H = 256, where gate/up's preferred 8
    # pieces per lane would take two batches of 8 scale bytes, falls back to 4 pieces),
    # K = 1408 (11 batches of 8 scale bytes) is refused; MX weights load their scales per
    # piece and take any multiple of 32.
    for H in (7168, 5120, 1792, 512, 256):
        st, why = _check(lib, _fake_layer(lib, "flint_w4a16", H=H), 8)
        assert st == 0, (H, why)
    st, why = _check(lib, _fake_layer(lib, "flint_w4a16", H=1408), 8)
    assert st == lib.MOE_EUNSUPPORTED and "no workgroup row mapping" in why
    st, why = _check(lib, _fake_layer(lib, "flint_w4a16", I=1408), 8)
    assert st == lib.MOE_EUNSUPPORTED and "no workgroup row mapping" in why
    st, why = _check(lib, _fake_layer(lib, "mistral_mxfp4", H=1408, I=1408), 8)
    assert st == 0, why


def test_misaligned_and_null_weights_are_refused(lib):
    s = _fake_layer(lib, "flint_w4a16")
    s.w13 = lib.WeightsT((1 << 20) + 4, 0, 0)
    st, why = _check(lib, s, 8)
    assert st != 0 and "w13.codes must be 16-byte aligned" in why
    assert "w13.scales is NULL" in why and "w13.gscale is NULL" in why


def test_calls_validate_before_launching(lib):
    so = lib.lib()
    s = _fake_layer(lib, "flint_w4a16")
    # NULL x, ids, w: rejected without touching the device
    st = so.moe_route(ctypes.byref(s), None, 1, None, None, None, None, 0, None)
    assert st == lib.MOE_EINVAL
    msg = so.moe_last_error().decode()
    assert "x_bf16" in msg and "topk_ids" in msg
    # workspace too small
    st = so.moe_route(ctypes.byref(s), 1 << 20, 1, 1 << 20, 1 << 20, None, 1 << 20, 16, None)
    assert st == lib.MOE_EWORKSPACE
    assert so.quantize_nvfp4_4o6(1 << 20, 4, 24, 1 << 20, 1 << 20, 1 << 20, None, None) == lib.MOE_EINVAL
    assert so.moe_route(None, None, 1, None, None, None, None, 0, None) == lib.MOE_EINVAL
    # zero rows / zero tokens enqueue nothing and succeed
    assert so.quantize_nvfp4_4o6(None, 0, 32, None, None, None, None, None) == 0
    # load-time MXFP4 requantization: the same conventions
    i64 = ctypes.c_int64
    assert so.moe_requant_mxfp4(1 << 20, i64(4), 48, 1 << 20, 1 << 20, None) == lib.MOE_EINVAL
    assert "multiple of 32" in so.moe_last_error().decode()
    assert so.moe_requant_mxfp4(None, i64(1), 64, (1 << 20) + 8, None, None) == lib.MOE_EINVAL
    msg = so.moe_last_error().decode()
    assert "w_bf16" in msg and "codes" in msg and "scales" in msg
    assert so.moe_requant_mxfp4(1 << 20, i64(-1), 64, 1 << 20, 1 << 20, None) == lib.MOE_EINVAL
    assert so.moe_requant_mxfp4(None, i64(0), 64, None, None, None) == 0
    assert so.moe_requant_nvfp4(1 << 20, 2, i64(4), 24, 1 << 20, 1 << 20, 1 << 20, None) == lib.MOE_EINVAL
    assert "multiple of 16" in so.moe_last_error().decode()
    assert so.moe_requant_nvfp4(None, 2, i64(4), 32, None, None, None, None) == lib.MOE_EINVAL
    msg = so.moe_last_error().decode()
    assert "w_bf16" in msg and "gscale" in msg
    assert so.moe_requant_nvfp4(None, 0, i64(4), 32, None, None, None, None) == 0
    assert so.moe_requant_nvfp4(1 << 20, 70000, i64(4), 32, 1 << 20, 1 << 20, 1 << 20, None) == lib.MOE_EINVAL
    assert so.moe_requant_mxfp8(1 << 20, i64(4), 48, 1 << 20, 1 << 20, None) == lib.MOE_EINVAL
    assert so.moe_requant_mxfp8(None, i64(0), 64, None, None, None) == 0
    # block-scaled FP8 input: the same conventions, plus the block shape
    fb = so.moe_requant_fp8_block_mxfp4
    assert fb(1 << 20, 1 << 20, i64(4), 48, 128, 128, 1 << 20, 1 << 20, None) == lib.MOE_EINVAL
    assert "multiple of 32" in so.moe_last_error().decode()
    assert fb(1 << 20, 1 << 20, i64(4), 64, 0, 128, 1 << 20, 1 << 20, None) == lib.MOE_EINVAL
    assert "block_rows" in so.moe_last_error().decode()
    assert fb(None, None, i64(1), 64, 128, 128, (1 << 20) + 8, None, None) == lib.MOE_EINVAL
    msg = so.moe_last_error().decode()
    assert "w_fp8" in msg and "block_scales" in msg and "codes" in msg and "scales is NULL" in msg
    assert fb(1 << 20, 1 << 20, i64(-1), 64, 128, 128, 1 << 20, 1 << 20, None) == lib.MOE_EINVAL
    assert fb(None, None, i64(0), 64, 128, 128, None, None, None) == 0
    # moe_forward: every check of both halves before the first launch
    st = so.moe_forward(ctypes.byref(s), 1 << 20, 1, 1 << 20, 1 << 20, None, None, 1 << 20, 1 << 24, None, None)
    assert st == lib.MOE_EINVAL and "y_bf16" in so.moe_last_error().decode()
    st = so.moe_forward(ctypes.byref(s), None, 1, None, None, None, 1 << 20, 1 << 20, 1 << 24, None, None)
    assert st == lib.MOE_EINVAL
    msg = so.moe_last_error().decode()
    assert "x_bf16" in msg and "topk_ids" in msg
    st = so.moe_forward(ctypes.byref(s), 1 << 20, 1, 1 << 20, 1 << 20, None, 1 << 20, 1 << 20, 16, None, None)
    assert st == lib.MOE_EWORKSPACE
    assert so.moe_forward(ctypes.byref(s), None, 0, None, None, None, None, None, 0, None, None) == 0


def test_xq_bytes_layout(lib):
    s = _fake_layer(lib, "inkling_w4a4")
    n = lib.lib().moe_xq_bytes(ctypes.byref(s), 3)
    assert n == 3 * 4096 // 2 + 768 + 256      # codes | scales (padded to 256) | g (padded)
    s = _fake_layer(lib, "mistral_mxfp4_a8")
    assert lib.lib().moe_xq_bytes(ctypes.byref(s), 2) == 2 * 6144 + 256
    s = _fake_layer(lib, "flint_w4a16")
    assert lib.lib().moe_xq_bytes(ctypes.byref(s), 2) == 0


def test_noalloc_refuses_calls_past_its_scratch_before_any_device_call(lib):
    """moe_forward_noalloc checks the workspace a call needs against its static scratch
    (16 MiB) on the host: the Flint-shaped BF16 layer at 256 tokens needs ~21 MB."""
    s = _fake_layer(lib, "flint_bf16")
    T = 256
    need = lib.lib().moe_workspace_bytes(ctypes.byref(s), T)
    assert need > lib.lib().moe_noalloc_scratch_bytes() == 16 << 20
    p = 1 << 20
    st = lib.lib().moe_forward_noalloc(ctypes.byref(s), p, T, p, p, None, p, None, None)
    assert st == lib.MOE_EWORKSPACE
    assert "static scratch" in lib.lib().moe_last_error().decode()
    assert lib.lib().moe_workspace_bytes(ctypes.byref(s), 8) <= lib.lib().moe_noalloc_scratch_bytes()


def test_fused_entry_checks_its_arguments_before_any_launch(lib):
    """moe_forward_fused refuses a NULL norm, a misaligned gamma, a negative eps and an
    x_out that overlaps resid_in, on the host."""
    s = _fake_layer(lib, "flint_w4a16")
    p = 1 << 20
    st = lib.lib().moe_forward_fused(ctypes.byref(s), None, p, 2, p + (1 << 16), p, p, None, p, p, 1 << 30,
                                     None, None)
    assert st == lib.MOE_EINVAL and "norm is NULL" in lib.lib().moe_last_error().decode()
    norm = lib.NormT(p + 2, -1.0)
    st = lib.lib().moe_forward_fused(ctypes.byref(s), ctypes.byref(norm), p, 2, p + 64, p, p, None, p, p, 1 << 30,
                                     None, None)
    why = lib.lib().moe_last_error().decode()
    assert st == lib.MOE_EINVAL
    assert "gamma" in why and "eps" in why and "overlap" in why
