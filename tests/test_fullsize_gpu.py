"""Every workload at its full size, in the launch configuration the benchmark
uses (dsa_forward with the default kernel choice), checked three ways:

  * against the CPU oracle: every query of the decode workloads, and the
    first, last and every 64th token of the 4096-token prefill chunk and of
    the 8192-token fresh prompt (65 and 129 tokens): scores bit for bit over
    the visible range, Top-K sets and counts exactly, attention within the
    stated tolerance;
  * the Top-K defining property for every query against the GPU's own
    scores: count = min(K, vis), only visible positions, every unselected
    score below the K-th or tied with it at a higher position; positions
    strictly ascending, -1 padding after them;
  * finite outputs everywhere.
The tiny workload runs at full size in test_parity_gpu.py.
"""
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


def _samples(w):
    """Queries compared with the oracle at full size.  Decode workloads: all
    of them.  The 4096-token prefill chunk (the oracle needs ~0.5 s of fp64
    work per token there): the first and last token and every 64th, 65 in
    all; every one of its tokens is checked by the Top-K defining property
    against the GPU's own scores instead."""
    B, T = w.batch, w.q_len
    want = np.zeros((B, T), bool)
    if T <= 8:
        want[:] = True
    else:
        want[:, ::64] = True
        want[:, T - 1] = True
    return want


def check_topk_property(w, scores, idx, cnt, chunk=256):
    """The Top-K defining property for every query, on the device: the
    count is min(K, vis), the selected positions are visible, and every
    unselected visible score is below the smallest selected one, or equal to
    it at a higher position than every selected position holding it."""
    B, T, K, L = w.batch, w.q_len, w.top_k, w.max_seq_len
    dev = scores.device
    pos = torch.arange(L, device=dev)
    for b in range(B):
        for t0 in range(0, T, chunk):
            t1 = min(T, t0 + chunk)
            vis = torch.clamp(int(w.seq_lens[b]) - T + 1 + torch.arange(t0, t1, device=dev), min=0)
            n = torch.clamp(vis, max=K)
            assert torch.equal(cnt[b, t0:t1].long(), n), f"counts differ at b={b} t in [{t0},{t1})"
            S = scores[b, t0:t1]
            sel_idx = idx[b, t0:t1].long()
            valid = torch.arange(K, device=dev)[None, :] < n[:, None]
            assert torch.all(torch.where(valid, sel_idx, -1) == sel_idx), "padding must be -1"
            # (checked before the scatter below, which needs in-range indices)
            assert torch.all(~valid | ((sel_idx >= 0) & (sel_idx < L))), f"a selected index is out of range (b={b})"
            visible = pos[None, :] < vis[:, None]
            # padding entries scatter into a spare last column: written to a
            # real column, their False could land after a True there (the
            # order of duplicate scatter writes is undefined)
            sel = torch.zeros((t1 - t0, L + 1), dtype=torch.bool, device=dev)
            sel.scatter_(1, torch.where(valid, sel_idx, L), torch.ones_like(valid))
            sel = sel[:, :L]
            assert torch.all(~sel | visible), f"an invisible position is selected (b={b})"
            neg = torch.tensor(float("-inf"), device=dev)
            tau = torch.where(sel, S, torch.tensor(float("inf"), device=dev)).amin(dim=1)
            rest = visible & ~sel
            top_rest = torch.where(rest, S, neg).amax(dim=1)
            has = n > 0
            assert torch.all(~has | (top_rest <= tau)), f"an unselected score exceeds the K-th (b={b})"
            last_sel_tie = torch.where(sel & (S == tau[:, None]), pos[None, :], -1).amax(dim=1)
            first_rest_tie = torch.where(rest & (S == tau[:, None]), pos[None, :], L).amin(dim=1)
            assert torch.all(~has | (first_rest_tie > last_sel_tie)), f"a tie at the K-th score went to a higher position (b={b})"


@pytest.mark.parametrize("name", ["decode8k", "decode128k", "prefill64k", "fp8_1m", "mx128k", "prompt8k"])
def test_full_size_workload(name):
    w = synth.make(name)
    print(f"\n[full] {name} B={w.batch} T={w.q_len} Lmax={w.max_seq_len} K={w.top_k}", flush=True)
    d = G.to_device(w)
    r = dsa.dsa_forward(d["q_idx"], d["head_w"], d["k_idx"], d["q"], d["kv"], d["seq_lens"], w.top_k, w.v_dim,
                        w.softmax_scale, k_scale=d["k_scale"], kv_scale=d["kv_scale"],
                        out_dtype=G.out_torch_dtype(w), return_scores=True)
    torch.cuda.synchronize()
    B, T, K = w.batch, w.q_len, w.top_k
    want = _samples(w)
    bs, ts = np.nonzero(want)

    # properties of every query: the Top-K against the GPU's own scores,
    # ascending order, finite outputs
    check_topk_property(w, r["scores"], r["topk_idx"], r["topk_count"])
    idx = r["topk_idx"].cpu().numpy()
    cnt = r["topk_count"].cpu().numpy()
    for b in range(B):
        for t in range(T):
            n = cnt[b, t]
            assert np.all(np.diff(idx[b, t, :n]) > 0)
    assert bool(torch.isfinite(r["out"].float()).all())

    # the compared queries against the oracle: scores bit for bit over the
    # visible range, Top-K sets exactly, attention at the stated bar
    scores = np.zeros((B, T, w.max_seq_len), np.float32)
    for b, t in zip(bs, ts):
        scores[b, t] = r["scores"][b, t].cpu().numpy()
    ref_scores = oracle.index_scores(w, want)
    G.check_scores(w, scores, ref_scores, want)
    ref_idx, ref_cnt = oracle.topk(w, ref_scores, want)
    G.check_topk(w, idx, cnt, ref_idx, ref_cnt, want)
    ref_out, ref_lse = oracle.sparse_mla(w, ref_idx, want)
    out = r["out"].float().cpu().numpy()
    err = G.check_attention(w, out, r["lse"].cpu().numpy(), ref_out, ref_lse, want)
    print(f"[ok] {name}: {want.sum()} of {B * T} queries equal to the oracle (scores, Top-K), "
          f"max abs attention err {err:.3e}; Top-K property on all {B * T}", flush=True)


@pytest.mark.parametrize("name,page_size", [("decode128k", 64), ("mx128k", 256)])
def test_full_size_paged_equals_contiguous(name, page_size):
    # the paged launch at full size: the caches scattered over a pool of
    # pages in a seeded random order (built on the device), every output equal
    # to the contiguous path's bit for bit, sampled queries against the oracle
    w = synth.make(name)
    print(f"\n[full paged] {name} B={w.batch} Lmax={w.max_seq_len} page={page_size}", flush=True)
    d = G.to_device(w)
    B, L = w.batch, w.max_seq_len
    max_pages = (L + page_size - 1) // page_size
    num_pages = B * max_pages + 5
    gen = torch.Generator(device="cpu").manual_seed(1234)
    perm = torch.randperm(num_pages, generator=gen)[:B * max_pages]
    table = perm.view(B, max_pages).to(torch.int32).cuda()

    def pool(x):
        if x is None:
            return None
        row = tuple(x.shape[2:])
        pad = max_pages * page_size - L
        if pad:
            x = torch.cat([x, torch.zeros((B, pad) + row, dtype=x.dtype, device=x.device)], dim=1)
        out = torch.zeros((num_pages, page_size) + row, dtype=x.dtype, device=x.device)
        out[perm.cuda().long()] = x.reshape((B * max_pages, page_size) + row)
        return out

    kw = dict(out_dtype=G.out_torch_dtype(w), return_scores=True)
    cont = dsa.dsa_forward(d["q_idx"], d["head_w"], d["k_idx"], d["q"], d["kv"], d["seq_lens"], w.top_k, w.v_dim,
                           w.softmax_scale, k_scale=d["k_scale"], kv_scale=d["kv_scale"], **kw)
    paged = dsa.dsa_forward_paged(d["q_idx"], d["head_w"], pool(d["k_idx"]), d["q"], pool(d["kv"]), d["seq_lens"],
                                  table, w.top_k, w.v_dim, L, w.softmax_scale, k_scales=pool(d["k_scale"]),
                                  kv_scales=pool(d["kv_scale"]), **kw)
    torch.cuda.synchronize()
    for k in ("topk_idx", "topk_count", "out", "lse"):
        assert torch.equal(paged[k], cont[k]), f"paged {k} differs from the contiguous path"
    for b in range(B):
        vis = w.vis(b, w.q_len - 1)
        assert torch.equal(paged["scores"][b, :, :vis - w.q_len + 1], cont["scores"][b, :, :vis - w.q_len + 1])
    want = _samples(w)
    ref_scores = oracle.index_scores(w, want)
    scores = paged["scores"].cpu().numpy()
    G.check_scores(w, scores, ref_scores, want)
    ref_idx, ref_cnt = oracle.topk(w, ref_scores, want)
    G.check_topk(w, paged["topk_idx"].cpu().numpy(), paged["topk_count"].cpu().numpy(), ref_idx, ref_cnt, want)
    print(f"[ok] {name} paged: equal to contiguous, {want.sum()} sampled queries exact", flush=True)


@pytest.mark.parametrize("name,row_bytes", [("decode128k", 256), ("mx128k", 128)])
def test_index_and_topk_at_the_largest_contiguous_length(name, row_bytes):
    # the matrix-core indexer addresses a sequence's key rows with 32-bit byte
    # offsets: Lmax * row bytes < 2^31, so 8,388,544 bf16 or 16,777,152 MXFP8
    # positions is the largest length it takes (for MXFP8 a skipped ring read
    # then lands just past the scale buffer's bound); scores and the Top-K of
    # the one query against the oracle
    L = (2 ** 31 // row_bytes) - 64
    w = synth.make(name, batch=1, max_seq_len=L, len_range=(L - 5, L - 5), heads=1, qk_dim=8, v_dim=8)
    print(f"\n[max] {name} Lmax={L} len={int(w.seq_lens[0])}", flush=True)
    d = G.to_device(w)
    p = dsa.make_problem(batch=1, q_len=1, max_seq_len=L, idx_heads=64, idx_dim=128, top_k=w.top_k,
                         idx_key_dtype=w.idx_key_dtype)
    assert "score=mfma" in dsa.kernel_choice(p)
    scores = dsa.dsa_index_score(d["q_idx"], d["head_w"], d["k_idx"], d["seq_lens"], k_scale=d["k_scale"])
    idx, cnt = dsa.dsa_topk(scores, d["seq_lens"], w.top_k)
    torch.cuda.synchronize()
    ref = oracle.index_scores(w)
    G.check_scores(w, scores.cpu().numpy(), ref)
    ref_idx, ref_cnt = oracle.topk(w, ref)
    G.check_topk(w, idx.cpu().numpy(), cnt.cpu().numpy(), ref_idx, ref_cnt)
    print("[ok] largest length: scores exact, Top-K equal", flush=True)
