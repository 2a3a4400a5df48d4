"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Index scores and Top-K index sets must match bit for bit (integer-valued
indexer inputs make every score exact); attention outputs must satisfy
|gpu - ref| <= 1e-2 + 2e-2 |ref| (bf16 paths, fp32 tiny path) or <= 3e-2
(fp8 cache).  Sizes span several tiles, chunks and splits plus ragged tails.
"""
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


def _full_check(w, **run_kw):
    got = G.run_forward(w, **run_kw)
    ref = oracle.forward(w)
    G.check_scores(w, got["scores"], ref["scores"])
    G.check_topk(w, got["topk_idx"], got["topk_count"], ref["idx"], ref["count"])
    err = G.check_attention(w, got["out"], got["lse"], ref["out"], ref["lse"])
    print(f"[ok] max abs attention err {err:.3e}", flush=True)
    return got, ref


CASES = {
    # the tiny fp32 workload at its full size (portable kernels)
    "tiny": dict(name="tiny"),
    # decode, 64x128 indexer, 128-head MLA, several chunks/splits, ragged lengths
    "decode_ragged": dict(name="decode128k", batch=3, max_seq_len=20000, len_range=(12000, 20000)),
    "decode_uniform": dict(name="decode8k", batch=4, max_seq_len=4096, top_k=512),
    # causal multi-token chunk
    "prefill_chunk": dict(name="prefill64k", q_len=16, max_seq_len=4096, len_range=(4096, 4096),
                          top_k=512),
    # a fresh prompt: every row is a new token (T = L), so token t sees t + 1
    # positions and the first K - 1 tokens have fewer than K to select from
    "prefill_fresh_prompt": dict(name="prefill64k", q_len=512, max_seq_len=512, len_range=(512, 512),
                                 top_k=128),
    # fp8 index keys + fp8 latent cache, two draft tokens
    "fp8_drafts": dict(name="fp8_1m", batch=2, max_seq_len=16384, len_range=(9000, 16384), top_k=1024),
    # an odd token count: the two-token score kernels (bf16 and per-row e4m3
    # keys) then run a last token pair whose second token does not exist
    # (its loads are clamped, its stores and histogram updates skipped)
    "prefill_chunk_odd": dict(name="prefill64k", q_len=3, max_seq_len=5000, len_range=(3000, 5000),
                              batch=2, top_k=700),
    "fp8_drafts_odd": dict(name="fp8_1m", batch=2, q_len=3, max_seq_len=9000, len_range=(5000, 9000),
                           top_k=600),
    # eight or more tokens: the shared-key score kernel (eight tokens per
    # segment) with a token count that leaves a partial last group (13 = 8 + 5:
    # three tokens of it do not exist), ragged sequences of several lengths
    # that are not whole units of 64 positions, and one sequence shorter than
    # a unit
    "prefill_shared_keys_ragged": dict(name="prefill64k", batch=4, q_len=13, max_seq_len=7000,
                                       len_range=(13, 7000), top_k=600),
}


@pytest.mark.parametrize("case", list(CASES))
def test_forward_matches_oracle(case):
    kw = dict(CASES[case])
    w = _case(kw.pop("name"), **kw)
    _full_check(w)


@pytest.mark.parametrize("mode", ["row", "chunk"])
def test_topk_modes_match_oracle(mode):
    # both Top-K strategies (one workgroup per query; chunked with a finishing
    # workgroup) on ragged decode and on two draft tokens with fp8 keys
    os.environ["DSA_TOPK_MODE"] = mode
    try:
        _full_check(_case("decode128k", batch=3, max_seq_len=30000, len_range=(17000, 30000)))
        _full_check(_case("fp8_1m", batch=2, max_seq_len=20000, len_range=(12000, 20000), top_k=1500))
    finally:
        del os.environ["DSA_TOPK_MODE"]


SPLIT_CASES = {
    "prefill_chunk": CASES["prefill_chunk"],
    "prefill_fresh_prompt": CASES["prefill_fresh_prompt"],
    "fp8_drafts_odd": CASES["fp8_drafts_odd"],
    "decode_ragged": CASES["decode_ragged"],
    "mx_two_tokens": dict(name="mx128k", batch=3, q_len=2, max_seq_len=6000, len_range=(3000, 6000), top_k=400),
}


@pytest.mark.parametrize("split", [1, 2])
@pytest.mark.parametrize("case", list(SPLIT_CASES))
def test_score_work_splits_match_oracle(case, split):
    # the score kernels share a segment's key units among workgroups either
    # round-robin over all their waves (1) or as exact contiguous shares (2);
    # by default each segment takes one by its size, so these small problems
    # run mostly one way: force each on every case
    kw = dict(SPLIT_CASES[case])
    w = _case(kw.pop("name"), **kw)
    os.environ["DSA_SCORE_SPLIT"] = str(split)
    try:
        _full_check(w)
    finally:
        del os.environ["DSA_SCORE_SPLIT"]


@pytest.mark.parametrize("name,kw,splits", [
    # one split of 2048 rows: two chunks of 1024 through LDS (bf16, e4m3, tile-scaled e4m3)
    ("decode128k", dict(batch=3, max_seq_len=20000, len_range=(12000, 20000)), 1),
    ("fp8_1m", dict(batch=2, max_seq_len=16384, len_range=(9000, 16384), top_k=2048), 1),
    ("mx128k", dict(batch=2, max_seq_len=9000, len_range=(5000, 9000), top_k=2048), 1),
    # 1600 rows: chunks of 832 and 768, the second ending mid-tile
    ("decode128k", dict(batch=2, max_seq_len=9000, len_range=(5000, 9000), top_k=1600), 1),
    # many queries: one split per query by default, no merge
    ("prefill64k", dict(q_len=128, max_seq_len=2304, len_range=(2304, 2304), top_k=2048), 0),
])
def test_attention_index_list_in_chunks(name, kw, splits):
    # a workgroup whose split holds more entries than its LDS list takes
    # them in chunks, one after another, with its softmax state carried over
    w = _case(name, **kw)
    if splits:
        os.environ["DSA_MLA_SPLITS"] = str(splits)
    try:
        _full_check(w)
    finally:
        os.environ.pop("DSA_MLA_SPLITS", None)


@pytest.mark.parametrize("name", ["decode8k", "fp8_1m", "mx128k"])
@pytest.mark.parametrize("split", [0, 2])
def test_two_tokens_with_fewer_rows_than_tokens(name, split):
    # q_len 2 with len_b = 0 (no token sees anything), 1 (the first token
    # sees nothing, the second one position), 2, and a long ragged row, on
    # the two-token score kernels of bf16, per-row e4m3 and MXFP8 keys
    w = _case(name, batch=4, q_len=2, max_seq_len=3000, len_range=(2, 3000), top_k=256)
    w.seq_lens[:] = [0, 1, 2, 2999]
    os.environ["DSA_SCORE_SPLIT"] = str(split)
    try:
        got, _ = _full_check(w)
    finally:
        del os.environ["DSA_SCORE_SPLIT"]
    assert got["topk_count"].tolist() == [[0, 0], [0, 1], [1, 2], [256, 256]]
    assert np.all(got["topk_idx"][0] == -1) and np.all(got["out"][0] == 0)
    assert np.all(np.isneginf(got["lse"][0])) and np.isneginf(got["lse"][1, 0]).all()
    assert got["topk_idx"][1, 1, 0] == 0 and np.all(got["topk_idx"][1, 1, 1:] == -1)


def test_shared_key_score_kernel_short_rows():
    # eight tokens per segment on rows shorter than the token count (len 5 <
    # T = 13: tokens 0..7 see nothing), an empty row, a row of exactly T, one
    # shorter than a unit of 64 positions and a long ragged one
    w = _case("prefill64k", batch=5, q_len=13, max_seq_len=7000, len_range=(13, 7000), top_k=300)
    w.seq_lens[:] = [0, 5, 13, 40, 6999]
    got, _ = _full_check(w)
    counts = got["topk_count"]
    assert np.all(counts[0] == 0) and np.all(counts[1, :8] == 0)
    assert counts[1, 8:].tolist() == [1, 2, 3, 4, 5] and counts[2].tolist() == list(range(1, 14))
    assert np.all(counts[4] == 300)


def test_shared_key_score_kernel_flushes_its_counters():
    # one workgroup takes all 1110 units of an 8-token segment over 70000
    # positions: its 16-bit histogram counters are flushed after 1008 units,
    # before any can overflow, and the histogram (hence the Top-K) stays exact
    w = _case("prefill64k", batch=1, q_len=8, max_seq_len=70000, len_range=(70000, 70000), top_k=700)
    os.environ["DSA_SCORE_WGS"] = "1"
    try:
        _full_check(w)
    finally:
        del os.environ["DSA_SCORE_WGS"]


@pytest.mark.parametrize("variant", [1, 5])
def test_one_token_score_kernels(variant):
    # one query token per sequence: the deep-ring kernel at one workgroup
    # per CU (the default for short rows) and the kernel at two per CU (the
    # default for long rows), each forced on a ragged decode batch
    w = _case("decode128k", batch=3, max_seq_len=20000, len_range=(12000, 20000))
    os.environ["DSA_SCORE_VARIANT"] = str(variant)
    try:
        _full_check(w)
    finally:
        del os.environ["DSA_SCORE_VARIANT"]


@pytest.mark.parametrize("name,kw", [
    ("decode128k", dict(batch=2, max_seq_len=9000, len_range=(5000, 9000), top_k=1024)),
    # many tokens: the shared-key score kernel without a histogram to fill
    ("prefill64k", dict(batch=2, q_len=13, max_seq_len=3000, len_range=(1500, 3000), top_k=500)),
])
def test_entry_points_separately(name, kw):
    w = _case(name, **kw)
    d = G.to_device(w)
    ref = oracle.forward(w)
    scores = dsa.dsa_index_score(d["q_idx"], d["head_w"], d["k_idx"], d["seq_lens"])
    idx, cnt = dsa.dsa_topk(scores, d["seq_lens"], w.top_k)
    out, lse = dsa.dsa_sparse_mla_decode(d["q"], d["kv"], idx, d["seq_lens"], w.v_dim, w.softmax_scale)
    torch.cuda.synchronize()
    G.check_scores(w, scores.cpu().numpy(), ref["scores"])
    G.check_topk(w, idx.cpu().numpy(), cnt.cpu().numpy(), ref["idx"], ref["count"])
    G.check_attention(w, out.float().cpu().numpy(), lse.cpu().numpy(), ref["out"], ref["lse"])


def test_generic_path_matches_oracle():
    w = _case("decode8k", batch=2, max_seq_len=3000, len_range=(2000, 3000), top_k=256)
    os.environ["DSA_FORCE_GENERIC"] = "1"
    try:
        _full_check(w)
    finally:
        del os.environ["DSA_FORCE_GENERIC"]


def test_fp8_generic_path_matches_oracle():
    w = _case("fp8_1m", batch=1, max_seq_len=4000, len_range=(3000, 4000), top_k=128)
    os.environ["DSA_FORCE_GENERIC"] = "1"
    try:
        _full_check(w)
    finally:
        del os.environ["DSA_FORCE_GENERIC"]


def test_fp8_cache_scales_not_powers_of_two():
    # The matrix-core path expands e4m3 rows with the hardware's scaled
    # conversion, which takes only a scale's exponent; a row whose scale is
    # not a power of two is converted unscaled and multiplied in fp32.  Half
    # the rows (at random, so waves mix both kinds) get such a scale: the
    # power of two times a factor in [0.55, 0.95], which keeps the values at
    # most as large as the power-of-two rows' (the fp8 bound is absolute),
    # while taking the exponent alone would be off by 10-45 %.
    w = _case("fp8_1m", batch=2, max_seq_len=6000, len_range=(4000, 6000), top_k=512)
    rng = np.random.default_rng(7)
    factor = rng.uniform(0.55, 0.95, size=w.kv_scale.shape).astype(np.float32)
    w.kv_scale[:] = np.where(rng.random(w.kv_scale.shape) < 0.5, w.kv_scale, w.kv_scale * factor)
    _full_check(w)


def test_edge_fewer_visible_than_k_and_empty():
    # sequence 0: 100 rows (< K), sequence 1: 0 rows (nothing visible), sequence 2: exactly Lmax
    w = _case("decode8k", batch=3, max_seq_len=1024, top_k=512)
    w.seq_lens[:] = [100, 0, 1024]
    got, ref = _full_check(w)
    assert got["topk_count"].tolist() == [[100], [0], [512]]
    assert np.all(got["topk_idx"][1] == -1) and np.all(got["out"][1] == 0)
    assert np.all(np.isneginf(got["lse"][1]))


@pytest.mark.parametrize("mode", ["row", "chunk"])
def test_edge_all_scores_tie(mode):
    # q_idx = 0 makes every score 0: the K lowest positions win; 9000 tied
    # candidates also overflow the row-mode LDS candidate buffer
    w = _case("decode8k", batch=2, max_seq_len=9000, top_k=300)
    w.q_idx[:] = 0
    os.environ["DSA_TOPK_MODE"] = mode
    try:
        got, _ = _full_check(w)
    finally:
        del os.environ["DSA_TOPK_MODE"]
    assert np.array_equal(got["topk_idx"][:, 0], np.tile(np.arange(300), (2, 1)))


def test_edge_ties_at_threshold():
    # scores drawn from few distinct values: many ties straddle the K-th value
    w = _case("decode8k", batch=2, max_seq_len=6000, top_k=1000)
    w.q_idx[:] = 0
    w.q_idx[..., 0] = 0x3F80  # bf16 1.0 on dim 0 -> score_s = sum_h w_h * relu(k[s,0])
    _full_check(w)


def test_attention_ignores_invalid_and_padded_entries():
    w = _case("decode8k", batch=2, max_seq_len=2048, top_k=96)
    d = G.to_device(w)
    idx = np.full((2, 1, 96), -1, np.int32)
    rng = np.random.default_rng(5)
    idx[0, 0, :80] = rng.permutation(2048)[:80]          # unordered
    idx[1, 0, :50] = np.sort(rng.permutation(2048)[:50])
    idx[1, 0, 50:60] = 5000                               # out of range: ignored
    out, lse = dsa.dsa_sparse_mla_decode(d["q"], d["kv"], torch.from_numpy(idx).cuda(), d["seq_lens"],
                                         w.v_dim, w.softmax_scale)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.sparse_mla(w, idx)
    G.check_attention(w, out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse)


def test_deterministic_and_no_writes_outside_outputs():
    w = _case("decode128k", batch=2, max_seq_len=12000, len_range=(9000, 12000), top_k=2048)
    d = G.to_device(w)
    B, T, H = w.batch, w.q_len, w.heads
    guard = 4096
    canary = torch.full((guard * 2 + B * T * H * w.v_dim,), 12345, dtype=torch.int16, device="cuda")
    out = canary[guard:guard + B * T * H * w.v_dim].view(torch.bfloat16).view(B, T, H, w.v_dim)
    res = []
    for _ in range(2):
        r = dsa.dsa_forward(d["q_idx"], d["head_w"], d["k_idx"], d["q"], d["kv"], d["seq_lens"], w.top_k,
                            w.v_dim, w.softmax_scale, out={"out": out})
        torch.cuda.synchronize()
        res.append((r["topk_idx"].cpu().clone(), out.float().cpu().clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    c = canary.cpu()
    assert torch.all(c[:guard] == 12345) and torch.all(c[-guard:] == 12345)


def test_invisible_positions_never_selected_causal():
    w = _case("prefill64k", q_len=8, max_seq_len=600, len_range=(600, 600), top_k=2048)
    got = G.run_forward(w)
    for t in range(8):
        vis = w.vis(0, t)
        sel = got["topk_idx"][0, t]
        assert got["topk_count"][0, t] == vis
        assert np.array_equal(sel[:vis], np.arange(vis)) and np.all(sel[vis:] == -1)


@pytest.mark.parametrize("mode", ["row", "chunk"])
def test_workspace_reused_and_counters_left_zero(mode):
    # one workspace serves three different problems of the same shape; the
    # counters at its start must be zero after every call (the library clears
    # them as it goes), and every result must still match the oracle
    os.environ["DSA_TOPK_MODE"] = mode
    try:
        ws = None
        for i, lens in enumerate([(15000, 20000), (9000, 20000), (20000, 20000)]):
            w = _case("decode128k", batch=3, max_seq_len=20000, len_range=lens, top_k=2048)
            w.q_idx[...] = np.roll(w.q_idx, i, axis=-1)  # different scores per round
            if i == 1:
                w.seq_lens[:] = [1500, 0, 20000]  # fewer visible than K, and an empty sequence
            d = G.to_device(w)
            prob = dsa.forward_problem(d["q_idx"], d["k_idx"], d["q"], d["kv"], d["seq_lens"], w.top_k, w.v_dim,
                                       w.softmax_scale, torch.bfloat16)
            if ws is None:
                ws = torch.empty(dsa.forward_workspace_size(prob), dtype=torch.uint8, device="cuda")
                dsa.workspace_init(ws)
            r = dsa.dsa_forward(d["q_idx"], d["head_w"], d["k_idx"], d["q"], d["kv"], d["seq_lens"], w.top_k,
                                w.v_dim, w.softmax_scale, workspace=ws)
            torch.cuda.synchronize()
            nz = dsa.workspace_zero_bytes(prob)
            assert nz > 0 and int(torch.count_nonzero(ws[:nz])) == 0, "counters not cleared"
            ref = oracle.forward(w)
            G.check_topk(w, r["topk_idx"].cpu().numpy(), r["topk_count"].cpu().numpy(), ref["idx"], ref["count"])
            G.check_attention(w, r["out"].float().cpu().numpy(), r["lse"].cpu().numpy(), ref["out"], ref["lse"])
    finally:
        del os.environ["DSA_TOPK_MODE"]


@pytest.mark.parametrize("name,kw", [
    ("prefill64k", dict(batch=2, q_len=40, max_seq_len=3000, len_range=(1500, 3000), top_k=700)),
    ("fp8_1m", dict(batch=3, q_len=2, max_seq_len=5000, len_range=(2500, 5000), top_k=600)),
    ("mx128k", dict(batch=2, q_len=7, max_seq_len=4000, len_range=(3000, 4000), top_k=500)),
])
def test_token_tiles_match_oracle(name, kw):
    # A call whose workspace would pass its budget runs tile after tile of
    # one sequence's query tokens, each tile seeing exactly what its tokens
    # see in the whole problem; a small budget makes these problems tile
    # (several sequences, ragged lengths, tiles ending before the last
    # token).  Every entry point is checked against the oracle.
    w = _case(name, **kw)
    ref = oracle.forward(w)
    d = G.to_device(w)
    whole = G.run_forward(w)
    os.environ["DSA_TILE_BUDGET"] = str(256 * 1024)
    try:
        p = dsa.forward_problem(d["q_idx"], d["k_idx"], d["q"], d["kv"], d["seq_lens"], w.top_k, w.v_dim,
                                w.softmax_scale, k_scale=d["k_scale"], kv_scale=d["kv_scale"])
        tiled_ws = dsa.forward_workspace_size(p)
        got = G.run_forward(w, d)
        scores = torch.from_numpy(got["scores"]).cuda()
        idx, cnt = dsa.dsa_topk(scores, d["seq_lens"], w.top_k)
        out, lse = dsa.dsa_sparse_mla_decode(d["q"], d["kv"], torch.from_numpy(ref["idx"]).cuda(), d["seq_lens"],
                                             w.v_dim, w.softmax_scale, kv_scale=d["kv_scale"],
                                             out_dtype=G.out_torch_dtype(w))
        torch.cuda.synchronize()
    finally:
        del os.environ["DSA_TILE_BUDGET"]
    assert tiled_ws < dsa.forward_workspace_size(p), "the budget did not make the call tile"
    G.check_scores(w, got["scores"], ref["scores"])
    G.check_topk(w, got["topk_idx"], got["topk_count"], ref["idx"], ref["count"])
    G.check_attention(w, got["out"], got["lse"], ref["out"], ref["lse"])
    G.check_topk(w, idx.cpu().numpy(), cnt.cpu().numpy(), ref["idx"], ref["count"])
    G.check_attention(w, out.float().cpu().numpy(), lse.cpu().numpy(), ref["out"], ref["lse"])
    for k in ("topk_idx", "topk_count"):  # (the attention's split count follows the launch's size)
        assert np.array_equal(got[k], whole[k]), f"tiled {k} differs from the whole call"


def test_token_tiles_on_paged_caches():
    from tests.test_paged_gpu import paginate, run_paged
    w = _case("prefill64k", batch=2, q_len=24, max_seq_len=3000, len_range=(1800, 3000), top_k=600)
    ref = oracle.forward(w)
    pgd = paginate(w, 64, seed=3)
    os.environ["DSA_TILE_BUDGET"] = str(256 * 1024)
    try:
        got = run_paged(w, pgd)
    finally:
        del os.environ["DSA_TILE_BUDGET"]
    G.check_scores(w, got["scores"], ref["scores"])
    G.check_topk(w, got["topk_idx"], got["topk_count"], ref["idx"], ref["count"])
    G.check_attention(w, got["out"], got["lse"], ref["out"], ref["lse"])
