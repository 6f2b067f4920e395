"""Decode captured in a HIP graph (as a serving loop would): every replay,
with new inputs copied in between and eager work and synchronisation around
it, matches the eager call bit for bit. The fused merge's arrival counters
return to zero inside each call, so the graph holds no memset."""

import pytest
import torch

import local_linear_attention_amd as pa
from workloads import WORKLOADS, make_decode_inputs, replace_shape

pytestmark = pytest.mark.gpu


def test_decode_graph_replays_match_eager():
    w = replace_shape(WORKLOADS[2], B=4, S_max=1024)
    inputs = [{k: (v.cuda() if isinstance(v, torch.Tensor) else v)
               for k, v in make_decode_inputs(w, seed=s, seq_lens=[1024, 700, 3, 0]).items()}
              for s in range(4)]
    st = {k: v.clone() for k, v in inputs[0].items() if isinstance(v, torch.Tensor)}
    scale = inputs[0]["scale"]
    ns, _ = pa.decode_plan(w.B, w.H_q, w.H_kv, w.d, w.S_max, 4)
    ws = torch.zeros(pa.decode_workspace_size(w.B, w.H_q, w.d, ns) // 4, dtype=torch.float32,
                     device="cuda")
    out = torch.empty((w.B, w.H_q, w.d), dtype=torch.float32, device="cuda")

    def call():
        pa.decode(st["q"], st["rho"], st["k_cache"], st["v_cache"], st["seq_lens"], scale,
                  num_splits=4, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(8):
        inp = inputs[rep % len(inputs)]
        for k in st:
            st[k].copy_(inp[k])
        eager = pa.decode(inp["q"], inp["rho"], inp["k_cache"], inp["v_cache"], inp["seq_lens"],
                          scale, num_splits=4)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        assert int(ws[-w.B * w.H_q:].view(torch.int32).abs().sum()) == 0
