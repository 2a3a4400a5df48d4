"""dsa_forward captured in a HIP graph: every replay, with eager work and
synchronisations in between, reproduces the eager result bit for bit."""
import pytest
import torch

import indexed_sparse_attention_amd as dsa
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


@pytest.mark.parametrize("name,kw", [
    ("decode128k", dict(batch=3, max_seq_len=16384, len_range=(9000, 16384))),
    ("fp8_1m", dict(batch=2, max_seq_len=12000, len_range=(8000, 12000), top_k=1024)),
    ("mx128k", dict(batch=2, q_len=2, max_seq_len=12000, len_range=(8000, 12000), top_k=1024)),
])
def test_graph_replays_match_eager(name, kw):
    w = synth.make(name, **kw)
    d = G.to_device(w)
    out_dtype = G.out_torch_dtype(w)
    prob = dsa.forward_problem(d["q_idx"], d["k_idx"], d["q"], d["kv"], d["seq_lens"], w.top_k, w.v_dim,
                               w.softmax_scale, out_dtype, d["k_scale"], d["kv_scale"])
    ws = torch.zeros(dsa.forward_workspace_size(prob), dtype=torch.uint8, device="cuda")
    B, T, H = w.batch, w.q_len, w.heads
    outs = {"out": torch.empty((B, T, H, w.v_dim), dtype=out_dtype, device="cuda"),
            "lse": torch.empty((B, T, H), dtype=torch.float32, device="cuda"),
            "topk_idx": torch.empty((B, T, w.top_k), dtype=torch.int32, device="cuda"),
            "topk_count": torch.empty((B, T), dtype=torch.int32, device="cuda"),
            "scores": torch.empty((B, T, w.max_seq_len), dtype=torch.float32, device="cuda")}

    def step():
        dsa.dsa_forward(d["q_idx"], d["head_w"], d["k_idx"], d["q"], d["kv"], d["seq_lens"], w.top_k,
                        w.v_dim, w.softmax_scale, k_scale=d["k_scale"], kv_scale=d["kv_scale"],
                        out_dtype=out_dtype, out=outs, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for v in outs.values():
            v.fill_(0)                 # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("out", "lse", "topk_idx", "topk_count"):
            assert torch.equal(outs[k], eager[k]), f"replay {rep}: {k} differs from eager"
        vis = [w.vis(b, 0) for b in range(B)]
        for b in range(B):
            assert torch.equal(outs["scores"][b, :, :vis[b] - T + 1], eager["scores"][b, :, :vis[b] - T + 1])
