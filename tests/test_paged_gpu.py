"""GPU parity of the paged-cache entry points.

The same logical caches are laid out in pages of a physical pool in a
random order (plus unused pages), with one block table for the index keys
and the latent rows.  The paged path must give the oracle's results on the
contiguous caches, at the same bar as the contiguous path (scores and Top-K
sets exactly), and in fact the contiguous GPU path's results bit for bit: the
arithmetic is the same, only the addresses differ.
"""
import ctypes
import os

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


def _case(name, **kw):
    w = synth.make(name, **kw)
    print(f"\n[case] {name} B={w.batch} T={w.q_len} Lmax={w.max_seq_len} K={w.top_k} "
          f"lens={w.seq_lens.tolist()[:8]}", flush=True)
    return w


def paginate(w, page_size, seed, spare=7):
    """Physical pools and a block table holding the workload's caches: the
    logical pages of every sequence (through max_seq_len) go to distinct
    physical pages in a random order; `spare` pages more stay unused."""
    B, L = w.batch, w.max_seq_len
    max_pages = (L + page_size - 1) // page_size
    num_pages = B * max_pages + spare
    rng = np.random.default_rng(seed)
    table = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages).astype(np.int32)

    def pool(a, row_shape):
        if a is None:
            return None
        a = a.reshape((B, L) + row_shape)
        pad = max_pages * page_size - L
        if pad:
            a = np.concatenate([a, np.zeros((B, pad) + row_shape, a.dtype)], axis=1)
        out = np.zeros((num_pages, page_size) + row_shape, a.dtype)
        out[table.reshape(-1)] = a.reshape((B * max_pages, page_size) + row_shape)
        return out

    Di, Dqk = w.idx_dim, w.qk_dim
    return dict(table=table, num_pages=num_pages, page_size=page_size,
                k_pages=pool(w.k_idx, (Di,)),
                k_scales=None if w.k_scale is None else pool(w.k_scale, w.k_scale.shape[2:]),
                kv_pages=pool(w.kv, (Dqk,)),
                kv_scales=None if w.kv_scale is None else pool(w.kv_scale, w.kv_scale.shape[2:]))


def run_paged(w, pgd, dev="cuda:0"):
    d = G.to_device(w, dev)
    t = G._t
    k_pages = t(pgd["k_pages"], w.idx_key_dtype, dev)
    kv_pages = t(pgd["kv_pages"], w.kv_dtype, dev)
    r = dsa.dsa_forward_paged(d["q_idx"], d["head_w"], k_pages, d["q"], kv_pages, d["seq_lens"],
                              torch.from_numpy(pgd["table"]).to(dev), w.top_k, w.v_dim, w.max_seq_len,
                              w.softmax_scale, k_scales=t(pgd["k_scales"], synth.F32, dev),
                              kv_scales=t(pgd["kv_scales"], synth.F32, dev), out_dtype=G.out_torch_dtype(w),
                              return_scores=True)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() if v.dtype == torch.bfloat16 else v.cpu().numpy() for k, v in r.items()}


CASES = {
    "decode_ragged_p64": (dict(name="decode128k", batch=3, max_seq_len=20000, len_range=(12000, 20000)), 64),
    "decode_p256": (dict(name="decode8k", batch=4, max_seq_len=4096, top_k=512), 256),
    "prefill_chunk_p128": (dict(name="prefill64k", q_len=16, max_seq_len=4096, len_range=(4096, 4096),
                                top_k=512), 128),
    "fp8_drafts_p64": (dict(name="fp8_1m", batch=2, max_seq_len=16384, len_range=(9000, 16384), top_k=1024), 64),
}


@pytest.mark.parametrize("case", list(CASES))
def test_paged_forward_matches_oracle_and_contiguous(case):
    kw, page_size = CASES[case]
    kw = dict(kw)
    w = _case(kw.pop("name"), **kw)
    pgd = paginate(w, page_size, seed=11)
    got = run_paged(w, pgd)
    ref = oracle.forward(w)
    G.check_scores(w, got["scores"], ref["scores"])
    G.check_topk(w, got["topk_idx"], got["topk_count"], ref["idx"], ref["count"])
    err = G.check_attention(w, got["out"], got["lse"], ref["out"], ref["lse"])
    print(f"[ok] max abs attention err {err:.3e}", flush=True)
    cont = G.run_forward(w)
    for k in ("topk_idx", "topk_count", "out", "lse"):
        assert np.array_equal(got[k], cont[k], equal_nan=True), f"paged {k} differs from the contiguous path"
    for b in range(w.batch):
        for t in range(w.q_len):
            vis = max(w.vis(b, t), 0)
            assert np.array_equal(got["scores"][b, t, :vis], cont["scores"][b, t, :vis])


@pytest.mark.parametrize("case", ["prefill_chunk_p128", "fp8_drafts_p64"])
def test_paged_exact_score_split(case):
    # paged key reads when each workgroup takes an exact contiguous share of
    # a segment's units (the default split of short segments)
    kw, page_size = CASES[case]
    kw = dict(kw)
    w = _case(kw.pop("name"), **kw)
    os.environ["DSA_SCORE_SPLIT"] = "2"
    try:
        got = run_paged(w, paginate(w, page_size, seed=12))
    finally:
        del os.environ["DSA_SCORE_SPLIT"]
    ref = oracle.forward(w)
    G.check_scores(w, got["scores"], ref["scores"])
    G.check_topk(w, got["topk_idx"], got["topk_count"], ref["idx"], ref["count"])
    G.check_attention(w, got["out"], got["lse"], ref["out"], ref["lse"])


def test_paged_entry_points_separately():
    # dsa_index_score_paged and dsa_sparse_mla_decode_paged through the C ABI
    w = _case("decode128k", batch=2, max_seq_len=9000, len_range=(5000, 9000), top_k=1024)
    pgd = paginate(w, 64, seed=5)
    dev = "cuda:0"
    d = G.to_device(w, dev)
    lib = dsa.load_library()
    table = torch.from_numpy(pgd["table"]).to(dev)
    pg = dsa.make_paging(table, 64, pgd["num_pages"])
    k_pages = G._t(pgd["k_pages"], w.idx_key_dtype, dev)
    kv_pages = G._t(pgd["kv_pages"], w.kv_dtype, dev)
    p = dsa.make_problem(batch=w.batch, q_len=w.q_len, max_seq_len=w.max_seq_len, idx_heads=w.idx_heads,
                         idx_dim=w.idx_dim, heads=w.heads, qk_dim=w.qk_dim, v_dim=w.v_dim, top_k=w.top_k,
                         softmax_scale=w.softmax_scale)
    scores = torch.empty((w.batch, w.q_len, w.max_seq_len), dtype=torch.float32, device=dev)
    assert lib.dsa_index_score_paged(ctypes.byref(p), ctypes.byref(pg), d["q_idx"].data_ptr(),
                                     d["head_w"].data_ptr(), k_pages.data_ptr(), None, d["seq_lens"].data_ptr(),
                                     scores.data_ptr(), None) == 0, lib.dsa_last_error()
    idx, cnt = dsa.dsa_topk(scores, d["seq_lens"], w.top_k)
    out = torch.empty((w.batch, w.q_len, w.heads, w.v_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.q_len, w.heads), dtype=torch.float32, device=dev)
    nb = lib.dsa_sparse_mla_workspace_size(ctypes.byref(p))
    ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=dev)
    assert lib.dsa_sparse_mla_decode_paged(ctypes.byref(p), ctypes.byref(pg), d["q"].data_ptr(),
                                           kv_pages.data_ptr(), None, idx.data_ptr(), d["seq_lens"].data_ptr(),
                                           out.data_ptr(), lse.data_ptr(), ws.data_ptr(), nb, None) == 0
    torch.cuda.synchronize()
    ref = oracle.forward(w)
    G.check_scores(w, scores.cpu().numpy(), ref["scores"])
    G.check_topk(w, idx.cpu().numpy(), cnt.cpu().numpy(), ref["idx"], ref["count"])
    G.check_attention(w, out.float().cpu().numpy(), lse.cpu().numpy(), ref["out"], ref["lse"])
