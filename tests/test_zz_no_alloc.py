"""dsa_forward_noalloc: the whole path with the workspace the library keeps
on each GPU, for callers that cannot allocate.  Called through the C ABI
(the ctypes binding) and compared with dsa_forward, which runs the same
kernels on a caller-allocated workspace: every output must be equal bit for
bit (which implies the oracle bar dsa_forward is held to elsewhere), on two
calls in a row, the second with a smaller input, plus one check against the
oracle."""
import numpy as np
import pytest
import torch

import indexed_sparse_attention_amd as dsa
import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _run_both(w):
    d = G.to_device(w)
    B, T, H = w.batch, w.q_len, w.heads
    dev = d["q"].device
    kw = dict(k_scale=d["k_scale"], kv_scale=d["kv_scale"], out_dtype=G.out_torch_dtype(w))

    def outs():  # every output preallocated: the no-alloc call allocates nothing
        return {"out": torch.full((B, T, H, w.v_dim), 7.0, dtype=G.out_torch_dtype(w), device=dev),
                "lse": torch.full((B, T, H), 7.0, device=dev),
                "topk_idx": torch.full((B, T, w.top_k), 7, dtype=torch.int32, device=dev),
                "topk_count": torch.full((B, T), 7, dtype=torch.int32, device=dev),
                "scores": torch.full((B, T, w.max_seq_len), 7.0, device=dev)}

    a = dsa.dsa_forward_noalloc(d["q_idx"], d["head_w"], d["k_idx"], d["q"], d["kv"], d["seq_lens"], w.top_k,
                                w.v_dim, w.softmax_scale, out=outs(), **kw)
    b = dsa.dsa_forward(d["q_idx"], d["head_w"], d["k_idx"], d["q"], d["kv"], d["seq_lens"], w.top_k, w.v_dim,
                        w.softmax_scale, out=outs(), **kw)
    torch.cuda.synchronize()
    for k in ("topk_idx", "topk_count", "out", "lse"):
        assert torch.equal(a[k], b[k]), f"{k}: dsa_forward_noalloc differs from dsa_forward"
    for bb in range(B):
        for t in range(T):
            vis = max(w.vis(bb, t), 0)
            assert torch.equal(a["scores"][bb, t, :vis], b["scores"][bb, t, :vis]), f"scores differ b={bb} t={t}"
    return a


def test_noalloc_equals_forward_twice_second_smaller():
    big = synth.make("decode128k", batch=4, max_seq_len=30000, len_range=(20000, 30000))
    small = synth.make("decode128k", batch=2, max_seq_len=9000, len_range=(3000, 9000), top_k=1024)
    for w in (big, small):
        print(f"\n[noalloc] B={w.batch} Lmax={w.max_seq_len} K={w.top_k} lens={w.seq_lens.tolist()}", flush=True)
        _run_both(w)
    # the smaller call against the oracle as well
    r = _run_both(small)
    ref = oracle.forward(small)
    got = {k: v.float().cpu().numpy() if v.dtype == torch.bfloat16 else v.cpu().numpy() for k, v in r.items()}
    G.check_scores(small, got["scores"], ref["scores"])
    G.check_topk(small, got["topk_idx"], got["topk_count"], ref["idx"], ref["count"])
    G.check_attention(small, got["out"], got["lse"], ref["out"], ref["lse"])


def test_noalloc_fp8_two_tokens():
    w = synth.make("fp8_1m", batch=2, max_seq_len=12000, len_range=(6000, 12000), top_k=512)
    print(f"\n[noalloc fp8] B={w.batch} T={w.q_len} Lmax={w.max_seq_len}", flush=True)
    _run_both(w)


def test_noalloc_many_tokens():
    # sixteen query tokens: the shared-key score kernel and the row-mode Top-K
    w = synth.make("prefill64k", batch=2, q_len=16, max_seq_len=4000, len_range=(2500, 4000), top_k=700)
    print(f"\n[noalloc prefill] B={w.batch} T={w.q_len} Lmax={w.max_seq_len}", flush=True)
    _run_both(w)


def test_noalloc_rejects_a_problem_larger_than_its_workspace():
    w = synth.make("decode8k", batch=2, max_seq_len=4096, top_k=256)
    d = G.to_device(w)
    p = dsa.forward_problem(d["q_idx"], d["k_idx"], d["q"], d["kv"], d["seq_lens"], w.top_k, w.v_dim)
    assert dsa.forward_workspace_size(p) <= dsa.NOALLOC_WORKSPACE_BYTES
    big = dict(batch=8, q_len=2, max_seq_len=1 << 20, idx_heads=64, idx_dim=128, heads=128, qk_dim=576,
               v_dim=512, top_k=2048)
    assert dsa.forward_workspace_size(dsa.make_problem(**big)) > dsa.NOALLOC_WORKSPACE_BYTES
