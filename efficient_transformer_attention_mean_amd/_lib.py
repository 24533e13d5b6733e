"""ctypes binding of libnystrom.so: the C entry points under the same names.

Argument marshalling only.  Every computation runs in the HIP library; if
the library is missing, loading fails loudly (there is no fallback).

torch is imported before the library is opened: torch ships its own HIP
runtime with the same SONAME as ROCm's, so loading torch first makes the
library bind to that one runtime instead of a second copy.
"""
from __future__ import annotations

import ctypes
import os

try:  # bind to torch's HIP runtime when torch is present (see module doc)
    import torch  # noqa: F401
except Exception:  # pragma: no cover - torch is part of the image
    torch = None

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnystrom.so")

NYS_F32, NYS_BF16 = 0, 1
NYS_OK, NYS_EINVAL, NYS_EUNSUPPORTED, NYS_EWORKSPACE, NYS_EHIP, NYS_ENOTIMPL = 0, -1, -2, -3, -4, -5
NYS_WS_QT, NYS_WS_KT, NYS_WS_A, NYS_WS_Z, NYS_WS_BV, NYS_WS_W = range(6)

EXPORTS = (
    "nystrom_attn_workspace_bytes",
    "nystrom_attn_workspace_offset",
    "nystrom_attn_fwd",
    "nystrom_attn_fwd_masked",
    "nystrom_attn_fwd_noalloc",
    "nystrom_attn_bwd_workspace_bytes",
    "nystrom_attn_bwd",
    "nystrom_attn_bwd_masked",
    "nystrom_attn_fwd_save",
    "nystrom_attn_bwd_saved",
    "nystrom_attn_bwd_state_bytes",
    "nystrom_attn_bwd_from_state",
    "nystrom_layer_workspace_bytes",
    "nystrom_layer_fwd",
    "nystrom_attn_error_workspace_bytes",
    "nystrom_attn_error",
    "nystrom_dconv_fwd",
    "nystrom_strerror",
    "nystrom_abi_version",
    "nystrom_timing_enable",
    "nystrom_timing_read",
)

_lib = None


def load():
    """Open libnystrom.so (once) and declare every entry point's signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m efficient_transformer_attention_mean_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.nystrom_attn_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.nystrom_attn_workspace_bytes.restype = sz
    lib.nystrom_attn_workspace_offset.argtypes = [i, i, i, i, i, i]
    lib.nystrom_attn_workspace_offset.restype = ctypes.c_longlong
    lib.nystrom_attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, i, i, i, vp, sz, vp]
    lib.nystrom_attn_fwd.restype = i
    lib.nystrom_attn_fwd_masked.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, i, i, i, vp, vp, sz, vp]
    lib.nystrom_attn_fwd_masked.restype = i
    lib.nystrom_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, i, i, i, vp]
    lib.nystrom_attn_fwd_noalloc.restype = i
    lib.nystrom_attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.nystrom_attn_bwd_workspace_bytes.restype = sz
    lib.nystrom_attn_bwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, i, i, i, vp, sz, vp]
    lib.nystrom_attn_bwd.restype = i
    lib.nystrom_attn_bwd_masked.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, i, i, i, vp, vp, sz, vp]
    lib.nystrom_attn_bwd_masked.restype = i
    lib.nystrom_attn_fwd_save.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, i, i, i, vp, sz, vp]
    lib.nystrom_attn_fwd_save.restype = i
    lib.nystrom_attn_bwd_saved.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, i, i, i, vp, sz, vp]
    lib.nystrom_attn_bwd_saved.restype = i
    lib.nystrom_attn_bwd_state_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.nystrom_attn_bwd_state_bytes.restype = sz
    lib.nystrom_attn_bwd_from_state.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, i, i, i, vp, sz,
                                                vp, sz, vp]
    lib.nystrom_attn_bwd_from_state.restype = i
    lib.nystrom_layer_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.nystrom_layer_workspace_bytes.restype = sz
    lib.nystrom_layer_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, i, i, i, vp, sz, vp]
    lib.nystrom_layer_fwd.restype = i
    lib.nystrom_attn_error_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.nystrom_attn_error_workspace_bytes.restype = sz
    lib.nystrom_attn_error.argtypes = [vp, vp, vp, i, i, i, i, i, vp, i, i, vp, sz, vp]
    lib.nystrom_attn_error.restype = i
    lib.nystrom_dconv_fwd.argtypes = [vp, vp, i, i, i, i, i, i, vp, vp]
    lib.nystrom_dconv_fwd.restype = i
    lib.nystrom_strerror.argtypes = [i]
    lib.nystrom_strerror.restype = ctypes.c_char_p
    lib.nystrom_abi_version.argtypes = []
    lib.nystrom_abi_version.restype = i
    lib.nystrom_timing_enable.argtypes = [i]
    lib.nystrom_timing_enable.restype = i
    lib.nystrom_timing_read.argtypes = [i, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_longlong)]
    lib.nystrom_timing_read.restype = i
    _lib = lib
    return lib


def _ptr(x):
    """A device pointer from a torch tensor, an int, or None (-> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError(f"expected a tensor, an int pointer or None, got {type(x)!r}")


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    raise TypeError(f"expected a stream, an int handle or None, got {type(s)!r}")


def nystrom_attn_workspace_bytes(batch, heads, n, d, m) -> int:
    return int(load().nystrom_attn_workspace_bytes(batch, heads, n, d, m))


def nystrom_attn_workspace_offset(which, batch, heads, n, d, m) -> int:
    return int(load().nystrom_attn_workspace_offset(which, batch, heads, n, d, m))


def nystrom_attn_fwd(Q, K, V, conv_w, n, d, m, heads, iters, out, batch, conv_k, dtype,
                     workspace=None, workspace_bytes=0, stream=None) -> int:
    return int(load().nystrom_attn_fwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(conv_w), n, d, m, heads, iters,
                                       _ptr(out), batch, conv_k, dtype, _ptr(workspace), workspace_bytes,
                                       _stream(stream)))


def nystrom_attn_fwd_masked(Q, K, V, conv_w, n, d, m, heads, iters, out, batch, conv_k, dtype, lengths,
                            workspace=None, workspace_bytes=0, stream=None) -> int:
    return int(load().nystrom_attn_fwd_masked(_ptr(Q), _ptr(K), _ptr(V), _ptr(conv_w), n, d, m, heads, iters,
                                              _ptr(out), batch, conv_k, dtype, _ptr(lengths), _ptr(workspace),
                                              workspace_bytes, _stream(stream)))


def nystrom_attn_fwd_noalloc(Q, K, V, conv_w, n, d, m, heads, iters, out, batch, conv_k, dtype,
                             stream=None) -> int:
    return int(load().nystrom_attn_fwd_noalloc(_ptr(Q), _ptr(K), _ptr(V), _ptr(conv_w), n, d, m, heads, iters,
                                               _ptr(out), batch, conv_k, dtype, _stream(stream)))


def nystrom_attn_bwd_workspace_bytes(batch, heads, n, d, m, iters, conv_k) -> int:
    return int(load().nystrom_attn_bwd_workspace_bytes(batch, heads, n, d, m, iters, conv_k))


def nystrom_attn_bwd(Q, K, V, conv_w, dO, n, d, m, heads, iters, dQ, dK, dV, dconv_w, batch, conv_k, dtype,
                     workspace=None, workspace_bytes=0, stream=None) -> int:
    return int(load().nystrom_attn_bwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(conv_w), _ptr(dO), n, d, m, heads, iters,
                                       _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dconv_w), batch, conv_k, dtype,
                                       _ptr(workspace), workspace_bytes, _stream(stream)))


def nystrom_attn_bwd_masked(Q, K, V, conv_w, dO, n, d, m, heads, iters, dQ, dK, dV, dconv_w, batch, conv_k, dtype,
                            lengths, workspace=None, workspace_bytes=0, stream=None) -> int:
    return int(load().nystrom_attn_bwd_masked(_ptr(Q), _ptr(K), _ptr(V), _ptr(conv_w), _ptr(dO), n, d, m, heads,
                                              iters, _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dconv_w), batch, conv_k,
                                              dtype, _ptr(lengths), _ptr(workspace), workspace_bytes,
                                              _stream(stream)))


def nystrom_attn_fwd_save(Q, K, V, conv_w, n, d, m, heads, iters, out, batch, conv_k, dtype, saved, saved_bytes,
                          stream=None) -> int:
    return load().nystrom_attn_fwd_save(_ptr(Q), _ptr(K), _ptr(V), _ptr(conv_w), n, d, m, heads, iters, _ptr(out),
                                        batch, conv_k, dtype, _ptr(saved), saved_bytes, _stream(stream))


def nystrom_attn_bwd_saved(Q, K, V, conv_w, dO, n, d, m, heads, iters, dQ, dK, dV, dconv_w, batch, conv_k, dtype,
                           saved, saved_bytes, stream=None) -> int:
    return load().nystrom_attn_bwd_saved(_ptr(Q), _ptr(K), _ptr(V), _ptr(conv_w), _ptr(dO), n, d, m, heads, iters,
                                         _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dconv_w), batch, conv_k, dtype,
                                         _ptr(saved), saved_bytes, _stream(stream))


def nystrom_attn_bwd_state_bytes(batch, heads, n, d, m, iters, conv_k) -> int:
    return int(load().nystrom_attn_bwd_state_bytes(batch, heads, n, d, m, iters, conv_k))


def nystrom_attn_bwd_from_state(Q, K, V, conv_w, dO, n, d, m, heads, iters, dQ, dK, dV, dconv_w, batch, conv_k,
                                dtype, state, state_bytes, scratch=None, scratch_bytes=0, stream=None) -> int:
    return load().nystrom_attn_bwd_from_state(_ptr(Q), _ptr(K), _ptr(V), _ptr(conv_w), _ptr(dO), n, d, m, heads,
                                              iters, _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dconv_w), batch, conv_k,
                                              dtype, _ptr(state), state_bytes, _ptr(scratch), scratch_bytes,
                                              _stream(stream))


def nystrom_layer_workspace_bytes(batch, heads, n, d, m, dtype) -> int:
    return int(load().nystrom_layer_workspace_bytes(batch, heads, n, d, m, dtype))


def nystrom_layer_fwd(X, Wqkv, Wo, conv_w, n, d, m, heads, iters, Y, batch, conv_k, dtype, workspace=None,
                      workspace_bytes=0, stream=None) -> int:
    return int(load().nystrom_layer_fwd(_ptr(X), _ptr(Wqkv), _ptr(Wo), _ptr(conv_w), n, d, m, heads, iters, _ptr(Y),
                                        batch, conv_k, dtype, _ptr(workspace), workspace_bytes, _stream(stream)))


def nystrom_attn_error_workspace_bytes(batch, heads, n, d, m, dtype) -> int:
    return int(load().nystrom_attn_error_workspace_bytes(batch, heads, n, d, m, dtype))


def nystrom_attn_error(Q, K, V, n, d, m, heads, iters, err, batch, dtype, workspace=None, workspace_bytes=0,
                       stream=None) -> int:
    return int(load().nystrom_attn_error(_ptr(Q), _ptr(K), _ptr(V), n, d, m, heads, iters, _ptr(err), batch, dtype,
                                         _ptr(workspace), workspace_bytes, _stream(stream)))


def nystrom_dconv_fwd(V, conv_w, n, d, heads, batch, conv_k, dtype, out, stream=None) -> int:
    return int(load().nystrom_dconv_fwd(_ptr(V), _ptr(conv_w), n, d, heads, batch, conv_k, dtype, _ptr(out),
                                        _stream(stream)))


def nystrom_strerror(code) -> str:
    return load().nystrom_strerror(code).decode()


def nystrom_abi_version() -> int:
    return int(load().nystrom_abi_version())


def nystrom_timing_enable(on) -> int:
    return int(load().nystrom_timing_enable(1 if on else 0))


def nystrom_timing_read(max_entries=64):
    """Returns {kernel name: (total_ms, launches)} since the previous read."""
    names = (ctypes.c_char_p * max_entries)()
    ms = (ctypes.c_double * max_entries)()
    cnt = (ctypes.c_longlong * max_entries)()
    k = int(load().nystrom_timing_read(max_entries, names, ms, cnt))
    return {names[i].decode(): (ms[i], int(cnt[i])) for i in range(min(k, max_entries))}
