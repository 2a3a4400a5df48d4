"""GPU parity of the pages' quantisation scheme against the oracle: MXFP8
index keys with an E8M0 scale per 32 dims and an index query quantised to
MXFP8 on the fly ("Inference Acceleration for New Large Model
Architectures" §4.1; "Long-Context LLM Inference Optimization", Layered
Quantization), and an FP8 latent cache with one scale per 128-column tile
(same page, §4.2).  Scores with integer-valued inputs are exact and compared
bit for bit; the Top-K is compared exactly; attention at the FP8 bar."""
import os

import numpy as np
import pytest
import torch

import indexed_sparse_attention_amd as dsa
import oracle
import synth
from tests import gpu_util as G
from tests.test_paged_gpu import paginate, run_paged

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _case(**kw):
    w = synth.make("mx128k", **kw)
    print(f"\n[case] mx128k B={w.batch} T={w.q_len} Lmax={w.max_seq_len} K={w.top_k} "
          f"lens={w.seq_lens.tolist()[:8]}", flush=True)
    return w


def _full_check(w):
    got = G.run_forward(w)
    ref = oracle.forward(w)
    G.check_scores(w, got["scores"], ref["scores"])
    G.check_topk(w, got["topk_idx"], got["topk_count"], ref["idx"], ref["count"])
    err = G.check_attention(w, got["out"], got["lse"], ref["out"], ref["lse"])
    print(f"[ok] max abs attention err {err:.3e}", flush=True)
    return got


@pytest.mark.parametrize("T", [1, 2, 3])
def test_mx_forward_matches_oracle(T):
    # several sub-tile rings per wave, ragged lengths, one to three query tokens
    _full_check(_case(batch=3, q_len=T, max_seq_len=9000, len_range=(5000, 9000), top_k=768))


def test_mx_generic_path_matches_oracle():
    w = _case(batch=2, q_len=2, max_seq_len=2500, len_range=(1800, 2500), top_k=200)
    os.environ["DSA_FORCE_GENERIC"] = "1"
    try:
        _full_check(w)
    finally:
        del os.environ["DSA_FORCE_GENERIC"]


def _rounding_queries(w, seed):
    """Index queries whose MX quantisation rounds: normal values with a
    different magnitude per (head, group), one group with an outlier, one
    all-zero group and one group at bf16's smallest normals (its shared
    exponent clamps at -127)."""
    rng = np.random.default_rng(seed)
    B, T, Hi, Di = w.q_idx.shape
    x = rng.normal(size=(B, T, Hi, Di // 32, 32)) * 2.0 ** rng.integers(-6, 7, (B, T, Hi, Di // 32, 1))
    x[:, :, 0, 0, 5] *= 1000.0
    x[:, :, 1, 2, :] = 0.0
    x[:, :, 2, 1, :] = rng.normal(size=(B, T, 32)) * 2.0 ** -124
    x = x.reshape(B, T, Hi, Di).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation to bf16 is a valid bf16 input


def _check_scores_close(w, got, ref):
    """fp32 accumulation bar: a dot product of n terms summed in fp32 is off by
    at most about n 2^-24 times the sum of its terms' magnitudes, so the bound
    is 2^-14 (128 dims, with margin) times sum_h w_h sum_i |q_hi| |k_i|; the
    dequantised query is within 1/16 of q, which the margin covers."""
    G_ = w.idx_dim // 32
    kdec = np.abs(np.array([oracle.e4m3_value(c) for c in range(256)])[w.k_idx]) * \
        np.repeat(2.0 ** (w.k_scale.astype(np.float64) - 127), 32, axis=-1)  # [B, L, Di]
    if w.q_idx_dtype == synth.F32:
        qv = np.abs(w.q_idx.astype(np.float64))
    else:
        qv = np.abs((w.q_idx.astype(np.uint32) << 16).view(np.float32).astype(np.float64))  # [B, T, Hi, Di]
    for b in range(w.batch):
        for t in range(w.q_len):
            vis = max(w.vis(b, t), 0)
            g, r = got[b, t, :vis].astype(np.float64), ref[b, t, :vis]
            mag = w.head_w[b, t].astype(np.float64) @ (qv[b, t] @ kdec[b, :vis].T)  # [vis]
            bad = np.flatnonzero(np.abs(g - r) > 2.0 ** -14 * mag)
            assert bad.size == 0, (f"b={b} t={t}: {bad.size} scores off, first s={bad[0]} gpu={g[bad[0]]} "
                                   f"ref={r[bad[0]]} bound={2.0 ** -14 * mag[bad[0]]}")
    assert G_ * 32 == w.idx_dim


@pytest.mark.parametrize("generic", [False, True])
def test_mx_query_quantisation_rounds_like_oracle(generic):
    w = _case(batch=2, q_len=2, max_seq_len=3000, len_range=(2000, 3000), top_k=128)
    w.q_idx[:] = _rounding_queries(w, 3)
    d = G.to_device(w)
    if generic:
        os.environ["DSA_FORCE_GENERIC"] = "1"
    try:
        s = dsa.dsa_index_score(d["q_idx"], d["head_w"], d["k_idx"], d["seq_lens"], k_scale=d["k_scale"])
        torch.cuda.synchronize()
    finally:
        if generic:
            del os.environ["DSA_FORCE_GENERIC"]
    _check_scores_close(w, s.cpu().numpy(), oracle.index_scores(w))


def _one_element_probe(w, seed):
    """Rounding queries, and keys and head weights that turn each score into
    one dequantised query element: key row s is +-1 (E4M3 0x38 / 0xB8) in
    dimension (s // 2) % Di alone, with every E8M0 group scale 1 (byte 127),
    and each query token weights one head by 1 and the rest by 0.  Then
    S[s] = max(0, +-q^[h, i]) exactly (every other product and head term is
    an exact zero), so the scores show every element of the query as the
    kernel quantised it, bit for bit."""
    B, T, Hi, Di = w.q_idx.shape
    w.q_idx[:] = _rounding_queries(w, seed)
    L = w.max_seq_len
    s = np.arange(L)
    k = np.zeros((L, Di), np.uint8)
    k[s, (s // 2) % Di] = np.where(s % 2 == 0, 0x38, 0xB8)
    w.k_idx[:] = k[None]
    w.k_scale[:] = 127
    heads = [0, 1, 2, 3, 17, 33, 50, 63]  # 0: outlier group, 1: zero group, 2: clamped group
    w.head_w[:] = 0.0
    for n, (b, t) in enumerate(np.ndindex(B, T)):
        w.head_w[b, t, heads[n % len(heads)]] = 1.0
    return w


@pytest.mark.parametrize("generic", [False, True])
@pytest.mark.parametrize("T", [1, 2])
def test_mx_query_rounding_exact(T, generic):
    # both score kernels (one and two tokens per segment) and the portable
    # kernel must quantise the index query exactly as the oracle does
    w = _one_element_probe(_case(batch=4, q_len=T, max_seq_len=2 * 128 * 3, len_range=(2 * 128 * 3,) * 2,
                                 top_k=64), seed=5 + T)
    d = G.to_device(w)
    if generic:
        os.environ["DSA_FORCE_GENERIC"] = "1"
    try:
        got = dsa.dsa_index_score(d["q_idx"], d["head_w"], d["k_idx"], d["seq_lens"], k_scale=d["k_scale"])
        torch.cuda.synchronize()
    finally:
        if generic:
            del os.environ["DSA_FORCE_GENERIC"]
    ref = oracle.index_scores(w)
    got = got.cpu().numpy().astype(np.float64)
    for b in range(w.batch):
        for t in range(w.q_len):
            vis = w.vis(b, t)
            g, r = got[b, t, :vis], ref[b, t, :vis]
            # the group whose exponent clamps at -127 holds values near 2^-124:
            # their dequantised elements are fp32 subnormals, which the matrix
            # core may flush; everywhere else equality is exact
            tiny = np.abs(r) < 2.0 ** -126
            bad = np.flatnonzero((g != r) & ~(tiny & (g == 0.0)))
            assert bad.size == 0, (f"b={b} t={t}: {bad.size} of {vis} scores differ, first s={bad[0]} "
                                   f"gpu={g[bad[0]]!r} oracle={r[bad[0]]!r}")
            assert np.count_nonzero(r) > vis // 4  # the probe does see the query's elements


def test_mx_paged_matches_oracle_and_contiguous():
    w = _case(batch=3, q_len=2, max_seq_len=7000, len_range=(4000, 7000), top_k=512)
    got = run_paged(w, paginate(w, 64, seed=13))
    ref = oracle.forward(w)
    G.check_scores(w, got["scores"], ref["scores"])
    G.check_topk(w, got["topk_idx"], got["topk_count"], ref["idx"], ref["count"])
    G.check_attention(w, got["out"], got["lse"], ref["out"], ref["lse"])
    cont = G.run_forward(w)
    for k in ("topk_idx", "topk_count", "out", "lse"):
        assert np.array_equal(got[k], cont[k], equal_nan=True), f"paged {k} differs from the contiguous path"


def test_tile_scales_not_powers_of_two():
    # a scale that is not a power of two is applied in fp32 after an unscaled
    # hardware conversion; half the tiles, at random, get one (factor in
    # [0.55, 0.95] keeps values within the absolute fp8 bar's range)
    w = _case(batch=2, q_len=1, max_seq_len=6000, len_range=(4000, 6000), top_k=512)
    rng = np.random.default_rng(17)
    factor = rng.uniform(0.55, 0.95, size=w.kv_scale.shape).astype(np.float32)
    w.kv_scale[:] = np.where(rng.random(w.kv_scale.shape) < 0.5, w.kv_scale, w.kv_scale * factor)
    _full_check(w)


def test_partial_last_group_and_tile_on_portable_kernels():
    # idx_dim 80 = groups of 32, 32 and 16; qk_dim 300 = tiles of 128, 128 and
    # 44 (the scale shapes use ceil(dim / 32) and ceil(dim / 128)); these
    # dims run on the portable kernels
    w = _case(batch=2, q_len=2, max_seq_len=700, len_range=(400, 700), top_k=50, idx_heads=4, idx_dim=80,
              heads=4, qk_dim=300, v_dim=260)
    assert w.k_scale.shape[-1] == 3 and w.kv_scale.shape[-1] == 3
    _full_check(w)


def test_mx_fp32_queries_on_the_matrix_core_path():
    # fp32 index queries (values bf16 cannot hold) quantised by the staging
    # code of the scaled-MFMA kernel, one and two tokens
    for T in (1, 2):
        w = _case(batch=2, q_len=T, max_seq_len=2500, len_range=(1500, 2500), top_k=128)
        rng = np.random.default_rng(21 + T)
        x = rng.normal(size=w.q_idx.shape) * 2.0 ** rng.integers(-5, 6, w.q_idx.shape[:-1] + (1,))
        w.q_idx = np.ascontiguousarray(x.astype(np.float32))
        w.q_idx_dtype = synth.F32
        d = G.to_device(w)
        s = dsa.dsa_index_score(d["q_idx"], d["head_w"], d["k_idx"], d["seq_lens"], k_scale=d["k_scale"])
        torch.cuda.synchronize()
        _check_scores_close(w, s.cpu().numpy(), oracle.index_scores(w))
