"""Python binding of libparallax, the MI355X Parallax forward pass.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (``include/parallax.h``). PyTorch supplies device
memory and the current stream. There is no CPU fallback: if the library is
not built, every call raises.

Functions mirror the C entry points:

* ``decode_plan``, ``decode_workspace_size``
* ``decode`` (one shot), ``decode_partial`` + ``decode_combine`` (two phases)
* ``decode_noalloc`` (one shot, with the library's built-in scratch instead of a workspace)
* ``prefill`` (causal), ``prefill_chunked`` (causal against an existing cache)
* ``decode_tokens`` (the chunked result for a few new tokens, by the split-KV decode)
* ``prefill_train`` + ``prefill_backward`` (gradients of the causal prefill)
* ``qkvr_projection`` (fused q, k, v, rho projection into the attention layouts)
* ``read_probe`` (measurement support: a plain streaming read of two buffers)
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "ParallaxError", "lib", "library_path", "abi_version", "status_string", "decode_plan",
    "decode_workspace_size", "decode", "decode_partial", "decode_combine", "decode_noalloc",
    "prefill",
    "prefill_chunked", "decode_tokens", "prefill_train", "prefill_backward_workspace_size",
    "prefill_backward",
    "qkvr_projection", "read_probe",
    "STATUS", "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libparallax.so")

STATUS = {
    0: "PARALLAX_OK",
    1: "PARALLAX_ERR_NULL_POINTER",
    2: "PARALLAX_ERR_BAD_SHAPE",
    3: "PARALLAX_ERR_UNSUPPORTED",
    4: "PARALLAX_ERR_MISALIGNED",
    5: "PARALLAX_ERR_WORKSPACE",
    6: "PARALLAX_ERR_HIP",
    7: "PARALLAX_ERR_TOO_LARGE",
}
_BF16, _F32 = 0, 1

EXPORTED_SYMBOLS = (
    "parallax_abi_version", "parallax_status_string", "parallax_decode_plan",
    "parallax_decode_workspace_size", "parallax_decode", "parallax_decode_partial",
    "parallax_decode_combine", "parallax_prefill", "parallax_prefill_chunked",
    "parallax_decode_tokens", "parallax_decode_noalloc",
    "parallax_prefill_train", "parallax_prefill_backward_workspace_size",
    "parallax_prefill_backward", "parallax_qkvr_projection", "parallax_read_probe",
)


class ParallaxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libparallax.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m local_linear_attention_amd.build`")
    _lib = load_library(_LIB_PATH)
    return _lib


def load_library(path: str) -> ctypes.CDLL:
    """Loads a libparallax build from ``path`` and declares its C signatures."""
    L = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.parallax_abi_version.restype = i
    L.parallax_abi_version.argtypes = []
    L.parallax_status_string.restype = ctypes.c_char_p
    L.parallax_status_string.argtypes = [i]
    L.parallax_decode_plan.restype = i
    L.parallax_decode_plan.argtypes = [i, i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
    L.parallax_decode_workspace_size.restype = sz
    L.parallax_decode_workspace_size.argtypes = [i, i, i, i]
    dec = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    L.parallax_decode.restype = i
    L.parallax_decode.argtypes = dec
    L.parallax_decode_partial.restype = i
    L.parallax_decode_partial.argtypes = dec
    L.parallax_decode_noalloc.restype = i
    L.parallax_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    L.parallax_decode_combine.restype = i
    L.parallax_decode_combine.argtypes = [vp, vp, i, i, i, i, i, i, vp, sz, vp]
    L.parallax_prefill.restype = i
    L.parallax_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    L.parallax_prefill_chunked.restype = i
    L.parallax_prefill_chunked.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    L.parallax_decode_tokens.restype = i
    L.parallax_decode_tokens.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i,
                                         vp, sz, vp]
    L.parallax_prefill_train.restype = i
    L.parallax_prefill_train.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    L.parallax_prefill_backward_workspace_size.restype = sz
    L.parallax_prefill_backward_workspace_size.argtypes = [i, i, i, i]
    L.parallax_prefill_backward.restype = i
    L.parallax_prefill_backward.argtypes = [vp] * 13 + [i, i, i, i, i, i, f, i, vp, sz, vp]
    L.parallax_qkvr_projection.restype = i
    L.parallax_qkvr_projection.argtypes = [vp] * 7 + [i] * 7 + [vp]
    L.parallax_read_probe.restype = i
    L.parallax_read_probe.argtypes = [vp, vp, ctypes.c_size_t, vp, i, vp]
    return L


def abi_version() -> int:
    return lib().parallax_abi_version()


def status_string(status: int) -> str:
    return lib().parallax_status_string(status).decode()


def _check(status: int, where: str):
    if status != 0:
        raise ParallaxError(status, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev_tensor(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _one_device(*named):
    """Every (name, tensor) pair on the first one's device (a kernel reads all
    of them on that device)."""
    dev = named[0][1].device
    for name, t in named[1:]:
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, not on {dev} with {named[0][0]}")


def _out_tensor(out, shape, device):
    """A fresh fp32 output, or the caller's after checking that the kernels
    can write all of it in place."""
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    _dev_tensor(out, "out")
    if out.dtype != torch.float32 or tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must be float32 of shape {tuple(shape)}")
    if out.device != device:
        raise ValueError(f"out is on {out.device}, the inputs on {device}")
    return out


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def decode_plan(B: int, H_q: int, H_kv: int, d: int, S_max: int, num_splits: int = 0):
    """(num_splits, chunk) the library uses for these sizes (0 = automatic)."""
    ns, ch = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().parallax_decode_plan(B, H_q, H_kv, d, S_max, num_splits, ctypes.byref(ns),
                                      ctypes.byref(ch)), "parallax_decode_plan")
    return ns.value, ch.value


def decode_workspace_size(B: int, H_q: int, d: int, num_splits: int) -> int:
    return int(lib().parallax_decode_workspace_size(B, H_q, d, num_splits))


def _decode_shapes(q, rho, k_cache, v_cache, seq_lens):
    for name, t in (("q", q), ("rho", rho), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("seq_lens", seq_lens)):
        _dev_tensor(t, name)
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q is [B, H_q, d] and k_cache is [B, H_kv, S_max, d]")
    B, H_q, d = q.shape
    _, H_kv, S_max, _ = k_cache.shape
    if rho.shape != q.shape or v_cache.shape != k_cache.shape or k_cache.shape[0] != B \
            or k_cache.shape[3] != d:
        raise ValueError("inconsistent decode shapes")
    if not (q.dtype == rho.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q, rho, k_cache and v_cache must share one dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    _one_device(("q", q), ("rho", rho), ("k_cache", k_cache), ("v_cache", v_cache),
                ("seq_lens", seq_lens))
    return B, H_q, H_kv, d, S_max


def _workspace(B, H_q, H_kv, d, S_max, num_splits, workspace, device):
    ns, _ = decode_plan(B, H_q, H_kv, d, S_max, num_splits)
    need = decode_workspace_size(B, H_q, d, ns)
    if workspace is None:
        # zeroed: the fused merge's arrival counters must start at zero
        workspace = torch.zeros(max(need, 16) // 4, dtype=torch.float32, device=device)
    else:
        _dev_tensor(workspace, "workspace")
        if workspace.device != device:
            raise ValueError(f"workspace is on {workspace.device}, the inputs on {device}")
    return workspace, workspace.numel() * workspace.element_size()


def decode(q, rho, k_cache, v_cache, seq_lens, scale: float, *, num_splits: int = 0, out=None,
           workspace=None):
    """Parallax decode; returns out [B, H_q, d] fp32 (see parallax_decode)."""
    B, H_q, H_kv, d, S_max = _decode_shapes(q, rho, k_cache, v_cache, seq_lens)
    out = _out_tensor(out, (B, H_q, d), q.device)
    ws, ws_bytes = _workspace(B, H_q, H_kv, d, S_max, num_splits, workspace, q.device)
    with torch.cuda.device(q.device):
        _check(lib().parallax_decode(
            q.data_ptr(), rho.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            seq_lens.data_ptr(), out.data_ptr(), B, H_q, H_kv, d, S_max, float(scale),
            _dtype_code(q), int(num_splits), ws.data_ptr(), ws_bytes, _stream_ptr(q.device)),
            "parallax_decode")
    return out


def decode_noalloc(q, rho, k_cache, v_cache, seq_lens, scale: float, *, num_splits: int = 0,
                   out=None):
    """Parallax decode with the library's built-in per-device scratch instead of a
    workspace (see parallax_decode_noalloc); returns out [B, H_q, d] fp32."""
    B, H_q, H_kv, d, S_max = _decode_shapes(q, rho, k_cache, v_cache, seq_lens)
    out = _out_tensor(out, (B, H_q, d), q.device)
    with torch.cuda.device(q.device):
        _check(lib().parallax_decode_noalloc(
            q.data_ptr(), rho.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            seq_lens.data_ptr(), out.data_ptr(), B, H_q, H_kv, d, S_max, float(scale),
            _dtype_code(q), int(num_splits), _stream_ptr(q.device)), "parallax_decode_noalloc")
    return out


def decode_partial(q, rho, k_cache, v_cache, seq_lens, scale: float, workspace, *,
                   num_splits: int = 0, out=None):
    """First decode phase (partial states into ``workspace``; see parallax_decode_partial)."""
    B, H_q, H_kv, d, S_max = _decode_shapes(q, rho, k_cache, v_cache, seq_lens)
    if out is not None:
        out = _out_tensor(out, (B, H_q, d), q.device)
    _dev_tensor(workspace, "workspace")
    _one_device(("q", q), ("workspace", workspace))
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        _check(lib().parallax_decode_partial(
            q.data_ptr(), rho.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            seq_lens.data_ptr(), 0 if out is None else out.data_ptr(), B, H_q, H_kv, d, S_max,
            float(scale), _dtype_code(q), int(num_splits), workspace.data_ptr(), ws_bytes,
            _stream_ptr(q.device)), "parallax_decode_partial")
    return out


def decode_combine(seq_lens, out, workspace, *, H_kv: int, S_max: int, num_splits: int = 0):
    """Second decode phase: merges the workspace into ``out`` [B, H_q, d]."""
    for name, t in (("seq_lens", seq_lens), ("out", out), ("workspace", workspace)):
        _dev_tensor(t, name)
    if out.dim() != 3 or out.dtype != torch.float32:
        raise ValueError("out must be float32 [B, H_q, d]")
    B, H_q, d = out.shape
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    _one_device(("out", out), ("seq_lens", seq_lens), ("workspace", workspace))
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(out.device):
        _check(lib().parallax_decode_combine(
            seq_lens.data_ptr(), out.data_ptr(), B, H_q, H_kv, d, S_max, int(num_splits),
            workspace.data_ptr(), ws_bytes, _stream_ptr(out.device)), "parallax_decode_combine")
    return out


def prefill(q, rho, k, v, seq_lens, scale: float, *, out=None):
    """Causal Parallax prefill; returns out [B, H_q, T, d] fp32 (see parallax_prefill)."""
    for name, t in (("q", q), ("rho", rho), ("k", k), ("v", v), ("seq_lens", seq_lens)):
        _dev_tensor(t, name)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q is [B, H_q, T, d] and k is [B, H_kv, S_max, d]")
    B, H_q, T, d = q.shape
    _, H_kv, S_max, _ = k.shape
    if rho.shape != q.shape or v.shape != k.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("inconsistent prefill shapes")
    if not (q.dtype == rho.dtype == k.dtype == v.dtype):
        raise TypeError("q, rho, k and v must share one dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    _one_device(("q", q), ("rho", rho), ("k", k), ("v", v), ("seq_lens", seq_lens))
    out = _out_tensor(out, (B, H_q, T, d), q.device)
    with torch.cuda.device(q.device):
        _check(lib().parallax_prefill(
            q.data_ptr(), rho.data_ptr(), k.data_ptr(), v.data_ptr(), seq_lens.data_ptr(),
            out.data_ptr(), B, H_q, H_kv, d, T, S_max, float(scale), _dtype_code(q),
            _stream_ptr(q.device)), "parallax_prefill")
    return out


def _chunk_shapes(q, rho, k_cache, v_cache, past_lens, chunk_lens):
    for name, t in (("q", q), ("rho", rho), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("past_lens", past_lens), ("chunk_lens", chunk_lens)):
        _dev_tensor(t, name)
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q is [B, H_q, T, d] and k_cache is [B, H_kv, S_max, d]")
    B, H_q, T, d = q.shape
    _, H_kv, S_max, _ = k_cache.shape
    if rho.shape != q.shape or v_cache.shape != k_cache.shape or k_cache.shape[0] != B \
            or k_cache.shape[3] != d:
        raise ValueError("inconsistent chunked-prefill shapes")
    if not (q.dtype == rho.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q, rho, k_cache and v_cache must share one dtype")
    for name, t in (("past_lens", past_lens), ("chunk_lens", chunk_lens)):
        if t.dtype != torch.int32 or t.shape != (B,):
            raise ValueError(f"{name} must be int32 [B]")
    _one_device(("q", q), ("rho", rho), ("k_cache", k_cache), ("v_cache", v_cache),
                ("past_lens", past_lens), ("chunk_lens", chunk_lens))
    return B, H_q, T, H_kv, d, S_max


def prefill_chunked(q, rho, k_cache, v_cache, past_lens, chunk_lens, scale: float, *, out=None):
    """Chunked causal prefill: row t attends keys 0..past_lens[b] + t of the cache.

    The cache must already hold the chunk's keys and values (see
    parallax_prefill_chunked). Returns out [B, H_q, T, d] fp32.
    """
    B, H_q, T, H_kv, d, S_max = _chunk_shapes(q, rho, k_cache, v_cache, past_lens, chunk_lens)
    out = _out_tensor(out, (B, H_q, T, d), q.device)
    with torch.cuda.device(q.device):
        _check(lib().parallax_prefill_chunked(
            q.data_ptr(), rho.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            past_lens.data_ptr(), chunk_lens.data_ptr(), out.data_ptr(), B, H_q, H_kv, d, T, S_max,
            float(scale), _dtype_code(q), _stream_ptr(q.device)), "parallax_prefill_chunked")
    return out


def decode_tokens(q, rho, k_cache, v_cache, past_lens, chunk_lens, scale: float, *,
                  num_splits: int = 0, out=None, workspace=None):
    """Multi-token decode: prefill_chunked's result for a few new tokens per
    sequence, by the split-KV decode kernel (see parallax_decode_tokens).
    Returns out [B, H_q, T, d] fp32."""
    B, H_q, T, H_kv, d, S_max = _chunk_shapes(q, rho, k_cache, v_cache, past_lens, chunk_lens)
    out = _out_tensor(out, (B, H_q, T, d), q.device)
    ws, ws_bytes = _workspace(B, H_q * T, H_kv, d, S_max, num_splits, workspace, q.device)
    with torch.cuda.device(q.device):
        _check(lib().parallax_decode_tokens(
            q.data_ptr(), rho.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            past_lens.data_ptr(), chunk_lens.data_ptr(), out.data_ptr(), B, H_q, H_kv, d, T, S_max,
            float(scale), _dtype_code(q), int(num_splits), ws.data_ptr(), ws_bytes,
            _stream_ptr(q.device)), "parallax_decode_tokens")
    return out


def _prefill_shapes(q, rho, k, v, seq_lens):
    for name, t in (("q", q), ("rho", rho), ("k", k), ("v", v), ("seq_lens", seq_lens)):
        _dev_tensor(t, name)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q is [B, H_q, T, d] and k is [B, H_kv, S_max, d]")
    B, H_q, T, d = q.shape
    _, H_kv, S_max, _ = k.shape
    if rho.shape != q.shape or v.shape != k.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("inconsistent prefill shapes")
    if not (q.dtype == rho.dtype == k.dtype == v.dtype):
        raise TypeError("q, rho, k and v must share one dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    _one_device(("q", q), ("rho", rho), ("k", k), ("v", v), ("seq_lens", seq_lens))
    return B, H_q, H_kv, T, S_max, d


def prefill_train(q, rho, k, v, seq_lens, scale: float):
    """Causal prefill that also returns what the backward needs.

    Returns (out, mu_v, stats): out and mu_v [B, H_q, T, d] fp32, stats
    [B, H_q, T, 4] fp32 (see parallax_prefill_train).
    """
    B, H_q, H_kv, T, S_max, d = _prefill_shapes(q, rho, k, v, seq_lens)
    out = torch.empty((B, H_q, T, d), dtype=torch.float32, device=q.device)
    mu = torch.empty_like(out)
    stats = torch.empty((B, H_q, T, 4), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        _check(lib().parallax_prefill_train(
            q.data_ptr(), rho.data_ptr(), k.data_ptr(), v.data_ptr(), seq_lens.data_ptr(),
            out.data_ptr(), mu.data_ptr(), stats.data_ptr(), B, H_q, H_kv, d, T, S_max,
            float(scale), _dtype_code(q), _stream_ptr(q.device)), "parallax_prefill_train")
    return out, mu, stats


def prefill_backward_workspace_size(B: int, H_q: int, T: int, d: int) -> int:
    return int(lib().parallax_prefill_backward_workspace_size(B, H_q, T, d))


def prefill_backward(q, rho, k, v, seq_lens, out, mu_v, stats, dout, scale: float, *,
                     workspace=None):
    """Gradients (dq, drho, dk, dv) of the causal prefill for upstream dout.

    dq, drho are shaped like q; dk, dv like k (summed over each KV head's
    query heads). See parallax_prefill_backward.
    """
    B, H_q, H_kv, T, S_max, d = _prefill_shapes(q, rho, k, v, seq_lens)
    for name, t in (("out", out), ("mu_v", mu_v), ("stats", stats), ("dout", dout)):
        _dev_tensor(t, name)
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be fp32")
    if out.shape != q.shape or mu_v.shape != q.shape or dout.shape != q.shape or \
            stats.shape != (B, H_q, T, 4):
        raise ValueError("out, mu_v, dout are [B, H_q, T, d] and stats [B, H_q, T, 4]")
    need = prefill_backward_workspace_size(B, H_q, T, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _dev_tensor(workspace, "workspace")
    _one_device(("q", q), ("out", out), ("mu_v", mu_v), ("stats", stats), ("dout", dout),
                ("workspace", workspace))
    ws_bytes = workspace.numel() * workspace.element_size()
    dq = torch.empty((B, H_q, T, d), dtype=torch.float32, device=q.device)
    drho = torch.empty_like(dq)
    dk = torch.empty((B, H_kv, S_max, d), dtype=torch.float32, device=q.device)
    dv = torch.empty_like(dk)
    with torch.cuda.device(q.device):
        _check(lib().parallax_prefill_backward(
            q.data_ptr(), rho.data_ptr(), k.data_ptr(), v.data_ptr(), seq_lens.data_ptr(),
            out.data_ptr(), mu_v.data_ptr(), stats.data_ptr(), dout.data_ptr(), dq.data_ptr(),
            drho.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H_q, H_kv, d, T, S_max,
            float(scale), _dtype_code(q), workspace.data_ptr(), ws_bytes,
            _stream_ptr(q.device)), "parallax_prefill_backward")
    return dq, drho, dk, dv


def qkvr_projection(x, w, H_q: int, H_kv: int, d: int, *, k_cache=None, v_cache=None,
                    past_lens=None, S_max: int | None = None):
    """Fused projection of x [B, T, d_model] (bf16) by the packed weight
    w [(2 H_q + 2 H_kv) d, d_model] (rows of W_Q, W_K, W_V, W_R).

    Returns (q, k_cache, v_cache, rho): q, rho [B, H_q, T, d] bf16; k and v
    written into rows past_lens[b] + t of the caches [B, H_kv, S_max, d]
    (allocated, zero-filled, with S_max = T when not given). See
    parallax_qkvr_projection.
    """
    # shapes first (the caches' rows decide where the kernel writes), devices after
    if x.dim() != 3 or w.dim() != 2 or w.shape[1] != x.shape[2] or \
            w.shape[0] != (2 * H_q + 2 * H_kv) * d:
        raise ValueError("x is [B, T, d_model] and w [(2 H_q + 2 H_kv) d, d_model]")
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("x and w must be bf16")
    B, T, d_model = x.shape
    if (k_cache is None) != (v_cache is None):
        raise ValueError("pass both k_cache and v_cache, or neither")
    if k_cache is None:
        S = T if S_max is None else int(S_max)
        k_cache = torch.zeros((B, H_kv, S, d), dtype=torch.bfloat16, device=x.device)
        v_cache = torch.zeros_like(k_cache)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dim() != 4 or t.shape[:2] != (B, H_kv) or t.shape[3] != d or \
                t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bf16 [B, H_kv, S_max, d]")
    # the kernel writes both caches at k_cache's row stride: V must have the same rows
    if v_cache.shape != k_cache.shape:
        raise ValueError(f"v_cache {tuple(v_cache.shape)} must have k_cache's shape "
                         f"{tuple(k_cache.shape)}")
    if S_max is not None and int(S_max) != k_cache.shape[2]:
        raise ValueError(f"S_max={S_max} disagrees with the caches' {k_cache.shape[2]} rows")
    for name, t in (("x", x), ("w", w), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, name)
    if past_lens is not None:
        _dev_tensor(past_lens, "past_lens")
        if past_lens.dtype != torch.int32 or past_lens.shape != (B,):
            raise ValueError("past_lens must be int32 [B]")
        _one_device(("x", x), ("past_lens", past_lens))
    _one_device(("x", x), ("w", w), ("k_cache", k_cache), ("v_cache", v_cache))
    q = torch.empty((B, H_q, T, d), dtype=torch.bfloat16, device=x.device)
    rho = torch.empty_like(q)
    with torch.cuda.device(x.device):
        _check(lib().parallax_qkvr_projection(
            x.data_ptr(), w.data_ptr(), q.data_ptr(), rho.data_ptr(), k_cache.data_ptr(),
            v_cache.data_ptr(), 0 if past_lens is None else past_lens.data_ptr(), B, T, d_model,
            H_q, H_kv, d, k_cache.shape[2], _stream_ptr(x.device)), "parallax_qkvr_projection")
    return q, k_cache, v_cache, rho


def read_probe(a, b, sink):
    """Measurement support: reads every byte of the same-sized device tensors
    a and b once and XORs their 32-bit words into the words of sink (a device
    int32 tensor); the XOR of all of sink's words changes by the XOR of the
    data. See parallax_read_probe."""
    _dev_tensor(a, "a")
    _dev_tensor(b, "b")
    _dev_tensor(sink, "sink")
    nbytes = a.numel() * a.element_size()
    if b.numel() * b.element_size() != nbytes or sink.dtype != torch.int32:
        raise ValueError("a and b must hold the same number of bytes; sink is int32")
    _one_device(("a", a), ("b", b), ("sink", sink))
    with torch.cuda.device(a.device):
        _check(lib().parallax_read_probe(a.data_ptr(), b.data_ptr(), nbytes, sink.data_ptr(),
                                         sink.numel(), _stream_ptr(a.device)), "parallax_read_probe")
