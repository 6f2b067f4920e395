"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.

The fake device pointers below are never dereferenced: each call returns an
error status from the host-side checks, which run before any HIP call. The
tests that pass them are skipped wherever a GPU is visible, so that a host
check that ever regressed could not launch a kernel on a fake address.
"""

import ctypes
import os
import re

import pytest

import local_linear_attention_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "parallax.h")

OK, NULLP, SHAPE, UNSUP, MISAL, WS, HIP, TOO_LARGE = range(8)
BF16, F32 = 0, 1
P = 0x10000  # 16-byte aligned fake device address


def _gpu_visible():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


fake_pointers = pytest.mark.skipif(_gpu_visible(), reason="fake device pointers: CPU-only checks")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pa.library_path()):
        from local_linear_attention_amd.build import build

        build()
    return pa.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(parallax_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported(L):
    names = header_functions()
    assert len(names) == 16
    assert set(names) == set(pa.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version(L):
    text = open(HEADER).read()
    v = int(re.search(r"#define PARALLAX_ABI_VERSION (\d+)", text).group(1))
    assert pa.abi_version() == v


def test_status_strings(L):
    for code, name in pa.STATUS.items():
        assert pa.status_string(code).startswith(name)
    assert "unknown" in pa.status_string(99)


def _plan(L, B, Hq, Hkv, S, req, d=128):
    ns, ch = ctypes.c_int(-1), ctypes.c_int(-1)
    st = L.parallax_decode_plan(B, Hq, Hkv, d, S, req, ctypes.byref(ns), ctypes.byref(ch))
    return st, ns.value, ch.value


def test_plan_requested(L):
    assert _plan(L, 8, 16, 8, 4096, 16) == (OK, 16, 256)
    assert _plan(L, 8, 16, 8, 4096, 1) == (OK, 1, 4096)
    assert _plan(L, 1, 32, 8, 131072, 128) == (OK, 128, 1024)
    st, ns, ch = _plan(L, 1, 1, 1, 100, 7)  # chunk rounds to 128 -> one split
    assert (st, ns, ch) == (OK, 1, 128)
    st, ns, ch = _plan(L, 2, 4, 2, 1000, 3)
    assert st == OK and ch % 128 == 0 and ns * ch >= 1000 and (ns - 1) * ch < 1000


def test_plan_bad_shapes(L):
    for args in [(0, 1, 1, 10, 1), (1, 3, 2, 10, 1), (1, 2, 2, 0, 1), (1, 2, 2, 10, -1)]:
        assert _plan(L, *args)[0] == SHAPE
    assert _plan(L, 1, 2, 2, 10, 1, d=0)[0] == SHAPE
    assert _plan(L, 1, 2, 2, 10, 1, d=96)[0] == UNSUP


def test_plan_largest_key_range(L):
    """Key ranges whose padding to a multiple of 128 would not fit an int are
    refused instead of producing a plan with no splits."""
    import ctypes as ct

    int_max = 2 ** 31 - 1
    for req in (1, 3):
        st, ns, ch = _plan(L, 1, 1, 1, int_max, req)
        assert st == UNSUP
        st, ns, ch = _plan(L, 1, 1, 1, int_max - 128, req)
        assert st == OK and ns >= 1 and ch > 0 and ch % 128 == 0
        assert ns * ch >= int_max - 128


def test_workspace_size(L):
    # records, then one 32-bit arrival counter per (b, h_q), rounded to 16 bytes
    assert pa.decode_workspace_size(8, 16, 128, 16) == 8 * 16 * 16 * 260 * 4 + 8 * 16 * 4
    assert pa.decode_workspace_size(1, 3, 64, 2) == 1 * 3 * 2 * 132 * 4 + 16
    assert pa.decode_workspace_size(8, 16, 128, 1) == 0
    assert pa.decode_workspace_size(0, 16, 128, 4) == 0


def _decode(L, fn="parallax_decode", q=P, rho=P, k=P, v=P, lens=P, out=P, B=2, Hq=4, Hkv=2,
            d=128, S=512, scale=1.0, dtype=BF16, ns=2, ws=P, ws_bytes=1 << 30):
    return getattr(L, fn)(q, rho, k, v, lens, out, B, Hq, Hkv, d, S, scale, dtype, ns, ws,
                          ws_bytes, None)


@fake_pointers
@pytest.mark.parametrize("fn", ["parallax_decode", "parallax_decode_partial"])
def test_decode_argument_errors(L, fn):
    assert _decode(L, fn, q=0) == NULLP
    assert _decode(L, fn, lens=0) == NULLP
    assert _decode(L, fn, B=0) == SHAPE
    assert _decode(L, fn, Hq=3, Hkv=2) == SHAPE
    assert _decode(L, fn, ns=-1) == SHAPE
    assert _decode(L, fn, scale=float("nan")) == SHAPE
    assert _decode(L, fn, scale=float("inf")) == SHAPE
    assert _decode(L, fn, d=96) == UNSUP
    assert _decode(L, fn, dtype=7) == UNSUP
    assert _decode(L, fn, S=1 << 24) == UNSUP    # a (b, h_kv) slice of 4 GiB
    assert _decode(L, fn, S=(1 << 23) - 64) == UNSUP  # (S + 64) d 2 bytes reaches 2^31
    assert _decode(L, fn, k=P + 8) == MISAL
    assert _decode(L, fn, lens=P + 2) == MISAL
    assert _decode(L, fn, ws=0) == WS
    assert _decode(L, fn, ws_bytes=100) == WS
    assert _decode(L, fn, ws=P + 4) == MISAL
    assert _decode(L, fn, out=P + 4) == MISAL


def _noalloc(L, q=P, rho=P, k=P, v=P, lens=P, out=P, B=2, Hq=4, Hkv=2, d=128, S=512, scale=1.0,
             dtype=BF16, ns=2):
    return L.parallax_decode_noalloc(q, rho, k, v, lens, out, B, Hq, Hkv, d, S, scale, dtype, ns,
                                     None)


@fake_pointers
def test_decode_noalloc_argument_errors(L):
    """Every check runs on the host before the scratch is set up or anything is
    launched (an explicit split count needs no device query)."""
    assert _noalloc(L, q=0) == NULLP
    assert _noalloc(L, out=0) == NULLP
    assert _noalloc(L, B=0) == SHAPE
    assert _noalloc(L, Hq=3, Hkv=2) == SHAPE
    assert _noalloc(L, ns=-1) == SHAPE
    assert _noalloc(L, scale=float("nan")) == SHAPE
    assert _noalloc(L, d=96) == UNSUP
    assert _noalloc(L, dtype=7) == UNSUP
    assert _noalloc(L, k=P + 8) == MISAL
    assert _noalloc(L, out=P + 4) == MISAL
    # records of 64 x 16 heads x 32 splits x 260 floats: 34 MB, past the 32 MiB scratch
    assert _noalloc(L, B=64, Hq=16, Hkv=8, S=32768, ns=32) == TOO_LARGE
    # d = 64: 2048 x 64 heads x 2 splits x 132 floats = 138 MB
    assert _noalloc(L, B=2048, Hq=64, Hkv=8, d=64, S=256, ns=2) == TOO_LARGE
    assert "scratch" in pa.status_string(TOO_LARGE)


@fake_pointers
def test_decode_out_required(L):
    assert _decode(L, "parallax_decode", out=0) == NULLP
    # one split: the partial kernel finalises into out, so out is required
    assert _decode(L, "parallax_decode_partial", out=0, ns=1, S=128) == NULLP


@fake_pointers
def test_combine_argument_errors(L):
    f = L.parallax_decode_combine
    assert f(0, P, 2, 4, 2, 128, 512, 2, P, 1 << 30, None) == NULLP
    assert f(P, 0, 2, 4, 2, 128, 512, 2, P, 1 << 30, None) == NULLP
    assert f(P, P, 2, 3, 2, 128, 512, 2, P, 1 << 30, None) == SHAPE
    assert f(P, P, 2, 4, 2, 80, 512, 2, P, 1 << 30, None) == UNSUP
    assert f(P, P + 4, 2, 4, 2, 128, 512, 2, P, 1 << 30, None) == MISAL
    assert f(P, P, 2, 4, 2, 128, 512, 2, 0, 1 << 30, None) == WS
    assert f(P, P, 2, 4, 2, 128, 512, 2, P, 64, None) == WS
    # one split: nothing to merge, returns OK without launching
    assert f(P, P, 2, 4, 2, 128, 128, 1, 0, 0, None) == OK


def _prefill(L, q=P, rho=P, k=P, v=P, lens=P, out=P, B=2, Hq=4, Hkv=2, d=128, T=256, S=256,
             scale=1.0, dtype=BF16):
    return L.parallax_prefill(q, rho, k, v, lens, out, B, Hq, Hkv, d, T, S, scale, dtype, None)


@fake_pointers
def test_prefill_argument_errors(L):
    assert _prefill(L, out=0) == NULLP
    assert _prefill(L, v=0) == NULLP
    assert _prefill(L, T=0) == SHAPE
    assert _prefill(L, T=300, S=256) == SHAPE
    assert _prefill(L, Hq=5, Hkv=2) == SHAPE
    assert _prefill(L, scale=float("nan")) == SHAPE
    assert _prefill(L, scale=-float("inf")) == SHAPE
    assert _prefill(L, dtype=F32) == UNSUP
    assert _prefill(L, d=32) == UNSUP
    assert _prefill(L, q=P + 2) == MISAL
    assert _prefill(L, out=P + 8) == MISAL


def test_python_binding_rejects_cpu_tensors():
    import torch

    t = torch.zeros(1, 1, 64)
    with pytest.raises(ValueError):
        pa.decode(t, t, t[None], t[None], torch.ones(1, dtype=torch.int32), 1.0)


def _tokens(L, q=P, rho=P, k=P, v=P, past=P, clen=P, out=P, B=2, Hq=4, Hkv=2, d=128, T=2,
            S=512, scale=1.0, dtype=BF16, ns=2, ws=P, ws_bytes=1 << 30):
    return L.parallax_decode_tokens(q, rho, k, v, past, clen, out, B, Hq, Hkv, d, T, S, scale,
                                    dtype, ns, ws, ws_bytes, None)


@fake_pointers
def test_decode_tokens_argument_errors(L):
    assert _tokens(L, past=0) == NULLP
    assert _tokens(L, clen=0) == NULLP
    assert _tokens(L, out=0) == NULLP
    assert _tokens(L, T=0) == SHAPE
    assert _tokens(L, T=513) == SHAPE             # more tokens than cache rows
    assert _tokens(L, Hq=3, Hkv=2) == SHAPE       # H_q not a multiple of H_kv
    assert _tokens(L, d=96) == UNSUP
    assert _tokens(L, past=P + 2) == MISAL
    assert _tokens(L, ws_bytes=16) == WS
    assert _tokens(L, scale=float("nan")) == SHAPE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback path: without the built library every entry point raises."""
    monkeypatch.setattr(pa, "_LIB_PATH", str(tmp_path / "libparallax.so"))
    monkeypatch.setattr(pa, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        pa.lib()
    with pytest.raises(RuntimeError, match="missing"):
        pa.decode_plan(1, 2, 1, 64, 128, 2)


@fake_pointers
def test_prefill_chunked_argument_errors(L):
    f = L.parallax_prefill_chunked

    def call(past=P, lens=P, q=P, out=P, T=256, S=512, dtype=BF16, Hq=4, Hkv=2):
        return f(q, P, P, P, past, lens, out, 2, Hq, Hkv, 128, T, S, 1.0, dtype, None)

    assert call(past=0) == NULLP
    assert call(lens=0) == NULLP
    assert call(T=600, S=512) == SHAPE
    assert call(Hq=5) == SHAPE
    assert call(dtype=F32) == UNSUP
    assert call(past=P + 2) == MISAL
    assert call(q=P + 8) == MISAL


def _train(L, q=P, rho=P, k=P, v=P, lens=P, out=P, mu=P, st=P, B=1, Hq=2, Hkv=1, d=128, T=256,
           S=256, scale=1.0, dtype=BF16):
    return L.parallax_prefill_train(q, rho, k, v, lens, out, mu, st, B, Hq, Hkv, d, T, S, scale,
                                    dtype, None)


@fake_pointers
def test_prefill_train_argument_errors(L):
    assert _train(L, mu=0) == NULLP
    assert _train(L, st=0) == NULLP
    assert _train(L, T=0) == SHAPE
    assert _train(L, T=300, S=256) == SHAPE
    assert _train(L, dtype=F32) == UNSUP
    assert _train(L, d=96) == UNSUP
    assert _train(L, mu=P + 4) == MISAL
    assert _train(L, st=P + 8) == MISAL


def test_backward_workspace_size(L):
    f = L.parallax_prefill_backward_workspace_size
    # dO high and low parts (bf16) plus (G, Dt) per row
    assert f(4, 16, 4096, 128) == 2 * 4 * 16 * 4096 * 128 * 2 + 4 * 16 * 4096 * 8
    assert f(1, 1, 3, 64) == (2 * 3 * 64 * 2 + 3 * 8 + 15) // 16 * 16
    assert f(0, 1, 3, 64) == 0 and f(1, 1, 0, 64) == 0


def _bwd(L, ptrs=None, B=1, Hq=2, Hkv=1, d=128, T=256, S=256, scale=1.0, dtype=BF16, ws=P,
         ws_bytes=1 << 30):
    p = [P] * 13 if ptrs is None else ptrs
    return L.parallax_prefill_backward(*p, B, Hq, Hkv, d, T, S, scale, dtype, ws, ws_bytes, None)


@fake_pointers
def test_prefill_backward_argument_errors(L):
    for i in range(13):
        p = [P] * 13
        p[i] = 0
        assert _bwd(L, p) == NULLP, i
    assert _bwd(L, ws=0) == NULLP
    assert _bwd(L, Hq=3, Hkv=2) == SHAPE
    assert _bwd(L, T=257, S=256) == SHAPE
    assert _bwd(L, scale=float("nan")) == SHAPE
    assert _bwd(L, dtype=F32) == UNSUP
    assert _bwd(L, d=256) == UNSUP
    for i in range(13):
        p = [P] * 13
        p[i] = P + 8 if i != 4 else P + 2
        assert _bwd(L, p) == MISAL, i
    assert _bwd(L, ws=P + 4) == MISAL
    need = L.parallax_prefill_backward_workspace_size(1, 2, 256, 128)
    assert _bwd(L, ws_bytes=need - 1) == WS


def _proj(L, x=P, w=P, q=P, rho=P, k=P, v=P, past=0, B=2, T=64, C=256, Hq=4, Hkv=2, d=128, S=64):
    return L.parallax_qkvr_projection(x, w, q, rho, k, v, past, B, T, C, Hq, Hkv, d, S, None)


@fake_pointers
def test_projection_argument_errors(L):
    assert _proj(L, x=0) == NULLP
    assert _proj(L, v=0) == NULLP
    assert _proj(L, T=0) == SHAPE
    assert _proj(L, T=65, S=64) == SHAPE
    assert _proj(L, C=96) == SHAPE          # d_model not a multiple of 64
    assert _proj(L, d=96) == UNSUP
    assert _proj(L, C=1 << 22) == UNSUP                  # a 256-row tile of x past 32-bit offsets
    assert _proj(L, B=1, T=65535 * 256 + 1, S=1 << 25) == UNSUP  # more than 65535 token tiles
    assert _proj(L, w=P + 8) == MISAL
    assert _proj(L, past=P + 2) == MISAL


@fake_pointers
def test_read_probe_argument_errors(L):
    f = L.parallax_read_probe
    assert f(0, P, 1 << 20, P, 512, None) == NULLP
    assert f(P, P, 1 << 20, 0, 512, None) == NULLP
    assert f(P, P, 0, P, 512, None) == SHAPE
    assert f(P, P, (1 << 20) + 8, P, 512, None) == SHAPE  # not a multiple of 16
    assert f(P, P, 1 << 20, P, 0, None) == SHAPE
    assert f(P + 8, P, 1 << 20, P, 512, None) == MISAL
    assert f(P, P, 1 << 20, P + 2, 512, None) == MISAL
