"""The workgroup timeline: every traced launch stamps each of its workgroups
once (start <= end, every slot of the grid written), tracing changes no
result, and a launch larger than the buffer's slots writes nothing."""
import numpy as np
import pytest
import torch

import indexed_sparse_attention_amd as dsa
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _traced(w, slots):
    buf = torch.zeros(len(dsa.TRACE_KINDS) * slots * 2, dtype=torch.int64, device="cuda:0")
    dsa.set_workgroup_trace(buf, slots)
    try:
        got = G.run_forward(w)
        torch.cuda.synchronize()
    finally:
        dsa.set_workgroup_trace(None)
    return got, buf.view(len(dsa.TRACE_KINDS), slots, 2).cpu().numpy()


@pytest.mark.parametrize("name,kw,kinds", [
    # decode: chunked Top-K and split attention with its merge
    ("decode128k", dict(batch=3, max_seq_len=20000, len_range=(12000, 20000)),
     ("scores", "topk_chunk", "topk_emit", "attention", "attention_merge")),
    # many queries: row-mode Top-K
    ("prefill64k", dict(q_len=512, max_seq_len=4096, len_range=(4096, 4096), top_k=512),
     ("scores", "topk_row", "attention")),
])
def test_trace_stamps_every_workgroup_once(name, kw, kinds):
    w = synth.make(name, **kw)
    print(f"\n[case] {name} B={w.batch} T={w.q_len} Lmax={w.max_seq_len} K={w.top_k}", flush=True)
    plain = G.run_forward(w)
    got, tr = _traced(w, 1 << 16)
    for k in ("topk_idx", "topk_count", "out", "lse"):
        assert np.array_equal(got[k], plain[k], equal_nan=True), f"tracing changed {k}"
    for name_k in kinds:
        st, en = tr[dsa.TRACE_KINDS.index(name_k), :, 0], tr[dsa.TRACE_KINDS.index(name_k), :, 1]
        n = int(np.count_nonzero(st))
        assert n > 0, f"{name_k}: no workgroup stamped"
        # the grid's workgroups are slots 0 .. n-1, each with start <= end
        assert np.all(st[:n] > 0) and np.all(en[:n] > 0) and np.all(st[n:] == 0) and np.all(en[n:] == 0)
        assert np.all(en[:n] >= st[:n]), f"{name_k}: a workgroup ends before it starts"
        span_us = (en[:n].max() - st[:n].min()) / 100.0
        assert 0 < span_us < 1e5, f"{name_k}: span {span_us} us"


def test_trace_skips_launches_past_its_slots():
    w = synth.make("decode128k", batch=2, max_seq_len=9000, len_range=(5000, 9000))
    _, tr = _traced(w, 1)  # every launch here has more than one workgroup
    assert not tr.any()
