"""The Python binding rejects, before any launch, a caller's output or
workspace that the kernels could not use in place."""

import pytest
import torch

import local_linear_attention_amd as pa
from workloads import WORKLOADS, make_decode_inputs, make_prefill_inputs, replace_shape


def _cuda(inp):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def test_host_output_rejected():
    with pytest.raises(ValueError, match="GPU tensor"):
        pa._out_tensor(torch.empty(2, 3), (2, 3), torch.device("cuda:0"))


@pytest.mark.gpu
def test_decode_output_checked():
    d = _cuda(make_decode_inputs(replace_shape(WORKLOADS[2], B=2, S_max=256)))
    args = (d["q"], d["rho"], d["k_cache"], d["v_cache"], d["seq_lens"], d["scale"])
    B, H, D = d["q"].shape
    for bad in (torch.empty((B, H, D - 1), device="cuda"),
                torch.empty((B, H, D), dtype=torch.float16, device="cuda"),
                torch.empty((B, H, 2 * D), device="cuda")[..., :D]):
        with pytest.raises(ValueError):
            pa.decode(*args, out=bad)
    good = torch.full((B, H, D), float("nan"), device="cuda")
    assert pa.decode(*args, out=good) is good
    torch.cuda.synchronize()
    assert torch.isfinite(good).all()


@pytest.mark.gpu
def test_host_workspace_rejected():
    d = _cuda(make_decode_inputs(replace_shape(WORKLOADS[2], B=2, S_max=256)))
    with pytest.raises(ValueError, match="GPU tensor"):
        pa.decode(d["q"], d["rho"], d["k_cache"], d["v_cache"], d["seq_lens"], d["scale"],
                  num_splits=4, workspace=torch.zeros(1 << 16))


@pytest.mark.gpu
def test_prefill_and_chunk_outputs_checked():
    p = _cuda(make_prefill_inputs(replace_shape(WORKLOADS[5], B=1, T=64, H_q=2, H_kv=1)))
    with pytest.raises(ValueError):
        pa.prefill(p["q"], p["rho"], p["k"], p["v"], p["seq_lens"], p["scale"],
                   out=torch.empty((1, 2, 63, 128), device="cuda"))
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    lens = torch.full((1,), 64, dtype=torch.int32, device="cuda")
    for fn in (pa.prefill_chunked, pa.decode_tokens):
        with pytest.raises(ValueError):
            fn(p["q"], p["rho"], p["k"], p["v"], zero, lens, p["scale"],
               out=torch.empty((1, 2, 64, 64), device="cuda"))


def test_projection_cache_shapes_rejected_before_launch():
    """The projection writes K and V rows at k_cache's row stride: a v_cache with
    other rows, a lone cache, or an S_max the caches disagree with is refused
    (checked before any device work, so this runs on the CPU)."""
    B, T, C, Hq, Hkv, d = 1, 8, 64, 2, 1, 64
    x = torch.zeros((B, T, C), dtype=torch.bfloat16)
    w = torch.zeros(((2 * Hq + 2 * Hkv) * d, C), dtype=torch.bfloat16)
    k = torch.zeros((B, Hkv, 16, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="v_cache"):
        pa.qkvr_projection(x, w, Hq, Hkv, d, k_cache=k,
                           v_cache=torch.zeros((B, Hkv, 12, d), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="both"):
        pa.qkvr_projection(x, w, Hq, Hkv, d, k_cache=k)
    with pytest.raises(ValueError, match="S_max"):
        pa.qkvr_projection(x, w, Hq, Hkv, d, k_cache=k, v_cache=k.clone(), S_max=32)
    with pytest.raises(ValueError, match="GPU tensor"):  # consistent shapes reach the device check
        pa.qkvr_projection(x, w, Hq, Hkv, d, k_cache=k, v_cache=k.clone(), S_max=16)
