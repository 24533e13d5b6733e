"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function the header declares, and its host logic (workspace sizing,
offsets, argument validation, error strings) behaves as documented.  No call
here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

from efficient_transformer_attention_mean_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nystrom.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nystrom_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libnystrom.so not built")
    return _lib.load()


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_strerror(lib):
    assert _lib.nystrom_abi_version() == 100
    for code in (0, -1, -2, -3, -4, -5):
        assert isinstance(_lib.nystrom_strerror(code), str) and _lib.nystrom_strerror(code)
    assert "unknown" in _lib.nystrom_strerror(-99)


def test_workspace_sizes_and_offsets(lib):
    B, H, n, d, m = 2, 12, 8192, 64, 64
    total = _lib.nystrom_attn_workspace_bytes(B, H, n, d, m)
    assert total > 0
    md, mm = B * H * m * d * 4, B * H * m * m * 4
    offs = [_lib.nystrom_attn_workspace_offset(w, B, H, n, d, m) for w in range(6)]
    sizes = [md, md, mm, mm, md, md]
    for o, s in zip(offs, sizes):
        assert o >= 0 and o % 256 == 0 and o + s <= total
    # regions do not overlap
    spans = sorted(zip(offs, sizes))
    for (o1, s1), (o2, _) in zip(spans, spans[1:]):
        assert o1 + s1 <= o2
    assert _lib.nystrom_attn_workspace_offset(6, B, H, n, d, m) == -1
    assert _lib.nystrom_attn_workspace_offset(-1, B, H, n, d, m) == -1


@pytest.mark.parametrize("shape", [
    (1, 1, 64, 16, 8), (8, 12, 512, 64, 64), (4, 12, 4096, 64, 64),
    (2, 12, 8192, 64, 32), (1, 16, 32768, 128, 256), (1, 1, 48, 32, 3), (1, 1, 7, 16, 7),
    (1, 1, 63, 16, 8), (2, 12, 8191, 64, 64), (1, 1, 100, 16, 64),  # n not a multiple of m: padded
])
def test_workspace_valid_shapes(lib, shape):
    assert _lib.nystrom_attn_workspace_bytes(*shape) > 0


@pytest.mark.parametrize("shape", [
    (0, 1, 64, 16, 8), (1, 0, 64, 16, 8), (1, 1, 64, 16, 0), (1, 1, 64, 16, 65),
    (1, 1, 7, 16, 8), (1, 1, 64, 24, 8), (1, 1, 64, 256, 8), (1, 1, 1024, 64, 512),
])
def test_workspace_invalid_shapes(lib, shape):
    assert _lib.nystrom_attn_workspace_bytes(*shape) == 0


FAKE = 0x10000  # never dereferenced: every case below is rejected on the host


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), _lib.NYS_EINVAL),
    (dict(out=None), _lib.NYS_EINVAL),
    (dict(n=7), _lib.NYS_EINVAL),  # m = 8 > n
    (dict(m=0), _lib.NYS_EINVAL),
    (dict(m=128, n=64), _lib.NYS_EINVAL),
    (dict(iters=-1), _lib.NYS_EINVAL),
    (dict(dtype=2), _lib.NYS_EINVAL),
    (dict(conv_w=FAKE, conv_k=4), _lib.NYS_EINVAL),
    (dict(conv_w=FAKE, conv_k=0), _lib.NYS_EINVAL),
    (dict(batch=0), _lib.NYS_EINVAL),
    (dict(heads=-2), _lib.NYS_EINVAL),
    (dict(d=48), _lib.NYS_EUNSUPPORTED),
    (dict(d=256), _lib.NYS_EUNSUPPORTED),
    (dict(m=512, n=1024), _lib.NYS_EUNSUPPORTED),
    (dict(n=1 << 22, d=128, m=64), _lib.NYS_EUNSUPPORTED),
    (dict(workspace=FAKE, workspace_bytes=16), _lib.NYS_EWORKSPACE),
])
def test_fwd_rejects_bad_arguments_before_launch(lib, kw, code):
    args = dict(Q=FAKE, K=FAKE, V=FAKE, conv_w=None, n=64, d=16, m=8, heads=1, iters=6, out=FAKE,
                batch=1, conv_k=0, dtype=_lib.NYS_F32, workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    assert _lib.nystrom_attn_fwd(**args) == code


@pytest.mark.parametrize("kw,code", [
    (dict(V=None), _lib.NYS_EINVAL),
    (dict(conv_w=None), _lib.NYS_EINVAL),
    (dict(conv_k=2), _lib.NYS_EINVAL),
    (dict(dtype=5), _lib.NYS_EINVAL),
    (dict(n=0), _lib.NYS_EINVAL),
    (dict(d=24), _lib.NYS_EUNSUPPORTED),
    (dict(n=1 << 22, d=128), _lib.NYS_EUNSUPPORTED),
])
def test_dconv_rejects_bad_arguments_before_launch(lib, kw, code):
    args = dict(V=FAKE, conv_w=FAKE, n=64, d=16, heads=1, batch=1, conv_k=3, dtype=_lib.NYS_F32, out=FAKE,
                stream=None)
    args.update(kw)
    assert _lib.nystrom_dconv_fwd(**args) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dO=None), _lib.NYS_EINVAL),
    (dict(dK=None), _lib.NYS_EINVAL),
    (dict(m=0), _lib.NYS_EINVAL),
    (dict(iters=-1), _lib.NYS_EINVAL),
    (dict(conv_w=FAKE, conv_k=4), _lib.NYS_EINVAL),
    (dict(dtype=3), _lib.NYS_EINVAL),
    (dict(m=80, n=640), _lib.NYS_EUNSUPPORTED),       # the backward handles m <= 64
    (dict(conv_w=FAKE, conv_k=35), _lib.NYS_EUNSUPPORTED),
    (dict(d=24), _lib.NYS_EUNSUPPORTED),
    (dict(workspace=FAKE, workspace_bytes=16), _lib.NYS_EWORKSPACE),
])
def test_bwd_rejects_bad_arguments_before_launch(lib, kw, code):
    args = dict(Q=FAKE, K=FAKE, V=FAKE, conv_w=None, dO=FAKE, n=64, d=16, m=8, heads=1, iters=6, dQ=FAKE, dK=FAKE,
                dV=FAKE, dconv_w=None, batch=1, conv_k=0, dtype=_lib.NYS_F32, workspace=None, workspace_bytes=0,
                stream=None)
    args.update(kw)
    assert _lib.nystrom_attn_bwd(**args) == code
    # The masked entry point checks the same arguments the same way.
    assert _lib.nystrom_attn_bwd_masked(**args, lengths=FAKE) == code


@pytest.mark.parametrize("kw,code", [
    (dict(saved=None), _lib.NYS_EINVAL),                  # the saved state is the caller's buffer
    (dict(out=None), _lib.NYS_EINVAL),
    (dict(conv_w=FAKE, conv_k=4), _lib.NYS_EINVAL),
    (dict(m=80, n=640), _lib.NYS_EUNSUPPORTED),
    (dict(saved_bytes=16), _lib.NYS_EWORKSPACE),
])
def test_fwd_save_rejects_bad_arguments_before_launch(lib, kw, code):
    args = dict(Q=FAKE, K=FAKE, V=FAKE, conv_w=None, n=64, d=16, m=8, heads=1, iters=6, out=FAKE, batch=1, conv_k=0,
                dtype=_lib.NYS_BF16, saved=FAKE, saved_bytes=1 << 30, stream=None)
    args.update(kw)
    assert _lib.nystrom_attn_fwd_save(**args) == code


@pytest.mark.parametrize("kw,code", [
    (dict(saved=None), _lib.NYS_EINVAL),                  # no allocation: the forward's state must be given
    (dict(dO=None), _lib.NYS_EINVAL),
    (dict(dtype=3), _lib.NYS_EINVAL),
    (dict(conv_w=FAKE, conv_k=35), _lib.NYS_EUNSUPPORTED),
    (dict(saved_bytes=16), _lib.NYS_EWORKSPACE),
])
def test_bwd_saved_rejects_bad_arguments_before_launch(lib, kw, code):
    args = dict(Q=FAKE, K=FAKE, V=FAKE, conv_w=None, dO=FAKE, n=64, d=16, m=8, heads=1, iters=6, dQ=FAKE, dK=FAKE,
                dV=FAKE, dconv_w=None, batch=1, conv_k=0, dtype=_lib.NYS_F32, saved=FAKE, saved_bytes=1 << 30,
                stream=None)
    args.update(kw)
    assert _lib.nystrom_attn_bwd_saved(**args) == code


@pytest.mark.parametrize("kw,code", [
    (dict(state=None), _lib.NYS_EINVAL),                  # the forward's state must be given
    (dict(dO=None), _lib.NYS_EINVAL),
    (dict(conv_w=FAKE, conv_k=35), _lib.NYS_EUNSUPPORTED),
    (dict(state_bytes=16), _lib.NYS_EWORKSPACE),
    (dict(scratch_bytes=16), _lib.NYS_EWORKSPACE),         # a scratch buffer that is too small
])
def test_bwd_from_state_rejects_bad_arguments_before_launch(lib, kw, code):
    args = dict(Q=FAKE, K=FAKE, V=FAKE, conv_w=None, dO=FAKE, n=64, d=16, m=8, heads=1, iters=6, dQ=FAKE, dK=FAKE,
                dV=FAKE, dconv_w=None, batch=1, conv_k=0, dtype=_lib.NYS_F32, state=FAKE, state_bytes=1 << 30,
                scratch=FAKE, scratch_bytes=1 << 30, stream=None)
    args.update(kw)
    assert _lib.nystrom_attn_bwd_from_state(**args) == code


def test_bwd_state_is_a_prefix_of_the_workspace(lib):
    # The training pair keeps only the state; fwd_save accepts a buffer of
    # exactly that size and rejects one byte less before launching.
    for shape in ((1, 1, 64, 16, 8), (2, 12, 8192, 64, 64), (1, 3, 777, 32, 48)):
        state = _lib.nystrom_attn_bwd_state_bytes(*shape, 6, 33)
        total = _lib.nystrom_attn_bwd_workspace_bytes(*shape, 6, 33)
        assert 0 < state < total
        assert state > _lib.nystrom_attn_workspace_bytes(*shape)  # the forward's regions and its steps
    assert _lib.nystrom_attn_bwd_state_bytes(1, 1, 640, 16, 80, 6, 0) == 0  # m > 64: no backward
    args = dict(Q=FAKE, K=FAKE, V=FAKE, conv_w=None, n=64, d=16, m=8, heads=1, iters=6, out=FAKE, batch=1, conv_k=0,
                dtype=_lib.NYS_BF16, saved=FAKE, stream=None)
    state = _lib.nystrom_attn_bwd_state_bytes(1, 1, 64, 16, 8, 6, 0)
    assert _lib.nystrom_attn_fwd_save(**args, saved_bytes=state - 1) == _lib.NYS_EWORKSPACE


def test_bwd_workspace_covers_the_forward_layout(lib):
    for shape in ((1, 1, 64, 16, 8), (2, 12, 8192, 64, 64), (1, 3, 777, 32, 48)):
        fwd = _lib.nystrom_attn_workspace_bytes(*shape)
        bwd = _lib.nystrom_attn_bwd_workspace_bytes(*shape, 6, 33)
        assert bwd > fwd > 0
    assert _lib.nystrom_attn_bwd_workspace_bytes(1, 1, 640, 64, 80, 6, 0) == 0
    assert _lib.nystrom_attn_bwd_workspace_bytes(1, 1, 64, 16, 8, 6, 35) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(X=None), _lib.NYS_EINVAL),
    (dict(Wo=None), _lib.NYS_EINVAL),
    (dict(dtype=7), _lib.NYS_EINVAL),
    (dict(conv_w=FAKE, conv_k=2), _lib.NYS_EINVAL),
    (dict(m=0), _lib.NYS_EINVAL),
    (dict(d=48), _lib.NYS_EUNSUPPORTED),
    (dict(workspace=FAKE, workspace_bytes=16), _lib.NYS_EWORKSPACE),
])
def test_layer_rejects_bad_arguments_before_launch(lib, kw, code):
    args = dict(X=FAKE, Wqkv=FAKE, Wo=FAKE, conv_w=None, n=64, d=16, m=8, heads=2, iters=6, Y=FAKE, batch=1,
                conv_k=0, dtype=_lib.NYS_BF16, workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    assert _lib.nystrom_layer_fwd(**args) == code


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), _lib.NYS_EINVAL),
    (dict(err=None), _lib.NYS_EINVAL),
    (dict(dtype=2), _lib.NYS_EINVAL),
    (dict(m=65), _lib.NYS_EINVAL),
    (dict(d=12), _lib.NYS_EUNSUPPORTED),
    (dict(workspace=FAKE, workspace_bytes=16), _lib.NYS_EWORKSPACE),
])
def test_error_rejects_bad_arguments_before_launch(lib, kw, code):
    args = dict(Q=FAKE, K=FAKE, V=FAKE, n=64, d=16, m=8, heads=1, iters=6, err=FAKE, batch=1, dtype=_lib.NYS_F32,
                workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    assert _lib.nystrom_attn_error(**args) == code


def test_layer_and_error_workspaces_cover_the_forward(lib):
    for shape in ((1, 1, 64, 16, 8), (8, 12, 512, 64, 64), (1, 3, 777, 32, 48)):
        fwd = _lib.nystrom_attn_workspace_bytes(*shape)
        for dt, es in ((_lib.NYS_F32, 4), (_lib.NYS_BF16, 2)):
            B, H, n, d, m = shape
            lay = _lib.nystrom_layer_workspace_bytes(*shape, dt)
            err = _lib.nystrom_attn_error_workspace_bytes(*shape, dt)
            assert lay >= fwd + 6 * B * H * n * d * es
            assert err >= fwd + B * H * n * d * es
    assert _lib.nystrom_layer_workspace_bytes(1, 1, 64, 16, 8, 9) == 0
    assert _lib.nystrom_attn_error_workspace_bytes(1, 1, 64, 24, 8, 0) == 0


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="fake device pointers: only where no GPU is visible")
def test_failed_hip_call_maps_to_nys_ehip(lib):
    # With no device visible, a call that passes validation fails at its first
    # HIP call (the stream-ordered workspace allocation, or the launch) and
    # reports NYS_EHIP; nothing reaches a device.
    P = 0x10000
    assert _lib.nystrom_attn_fwd(P, P, P, None, 128, 16, 8, 1, 6, P, 1, 0, _lib.NYS_F32) == _lib.NYS_EHIP
    assert _lib.nystrom_attn_fwd(P, P, P, None, 128, 16, 8, 1, 6, P, 1, 0, _lib.NYS_BF16, P, 1 << 30) == _lib.NYS_EHIP
    assert _lib.nystrom_attn_bwd(P, P, P, None, P, 128, 16, 8, 1, 6, P, P, P, None, 1, 0, _lib.NYS_F32) == _lib.NYS_EHIP
    assert _lib.nystrom_layer_fwd(P, P, P, None, 128, 16, 8, 1, 6, P, 1, 0, _lib.NYS_F32) == _lib.NYS_EHIP
    assert _lib.nystrom_attn_error(P, P, P, 128, 16, 8, 1, 6, P, 1, _lib.NYS_F32) == _lib.NYS_EHIP
    assert _lib.nystrom_dconv_fwd(P, P, 128, 16, 1, 1, 3, _lib.NYS_F32, P) == _lib.NYS_EHIP
    assert "HIP" in _lib.nystrom_strerror(_lib.NYS_EHIP)


@pytest.mark.skipif(_gpu_visible(), reason="fake device pointers: only where no GPU is visible")
def test_host_code_under_address_and_undefined_behaviour_sanitizers():
    # The library's host code (validation, workspace layout, error mapping,
    # timing switches) built with -fsanitize=address,undefined on the host side
    # and driven by tests/sanitize/host_checks.cpp; objects are cached under
    # the package's _build folder and rebuilt when a source changes.
    import subprocess
    out = os.path.join(ROOT, "efficient_transformer_attention_mean_amd", "_build", "host_sanitize")
    r = subprocess.run([os.path.join(ROOT, "tests", "sanitize", "build_and_run.sh"), out], capture_output=True,
                       text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "host checks passed" in r.stdout
