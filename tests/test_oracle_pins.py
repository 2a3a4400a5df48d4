"""Pins for the CPU oracle: each check ties it to something other than itself.

The pages print no worked example, so the oracle is pinned by closed forms,
identities that follow from the definitions, special cases that reduce to a
library routine (torch dtype decoders, torch scaled-dot-product attention,
numpy lexsort, numpy matmul) and brute force on tiny inputs.  Each pin is
chosen so a plausible slip (dropped ReLU, transposed operand, wrong index,
wrong tie rule, missing scale, off-by-one visibility) fails at least one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import problem

RNG = np.random.default_rng(1234)


# ------------------------------------------------------------------ decoders
def test_e4m3_decoder_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    mine = np.array([oracle.e4m3_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF only
    assert np.array_equal(mine[~nan], ref[~nan])


def test_e4m3_decoder_anchors():
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0xC0) == -2.0
    assert oracle.e4m3_value(0x80) == 0.0


def test_bf16_decoder_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    mine = np.array([oracle.bf16_value(int(c)) for c in codes[::97]])
    sub = ref[::97]
    nan = np.isnan(sub)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], sub[~nan])


def test_e4m3_quantizer_matches_torch_rne_in_range():
    # every representable value, every midpoint (ties) and random points
    vals = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mids = (vals[1:] + vals[:-1]) / 2
    pts = np.concatenate([vals, mids, RNG.uniform(-440, 440, 2000), RNG.normal(0, 1, 2000)])
    pts = np.concatenate([pts, -pts])
    ref = torch.from_numpy(pts).to(torch.float8_e4m3fn).double().numpy()
    mine = np.array([oracle.e4m3_quantize(float(x)) for x in pts])
    assert np.array_equal(mine, ref)


def test_e4m3_quantizer_saturates():
    assert oracle.e4m3_quantize(500.0) == 448.0
    assert oracle.e4m3_quantize(-1e9) == -448.0
    assert oracle.e4m3_quantize(4.3) == 4.5  # 4.3 is nearer 4.5 than 4.0


# ------------------------------------------------------------------ scores
def _nan_eq(a, b):
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_scores_hand_example():
    # 2 heads x 3 dims, 3 positions, w = (1, 3).
    #   q0 = ( 1, 0, 2)  q1 = (0,-1, 1)
    #   k0 = ( 1, 1, 1): q0.k0 = 3, q1.k0 = 0  -> S = 1*3 + 3*0   = 3
    #   k1 = ( 2, 0,-1): q0.k1 = 0, q1.k1 = -1 -> S = 1*0 + 3*0   = 0  (ReLU)
    #   k2 = ( 0,-3, 1): q0.k2 = 2, q1.k2 = 4  -> S = 1*2 + 3*4   = 14
    # A transposed operand (k used as query) or a missing ReLU gives other values.
    q_idx = np.array([[[[1, 0, 2], [0, -1, 1]]]], np.float32)
    k_idx = np.array([[[1, 1, 1], [2, 0, -1], [0, -3, 1]]], np.float32)
    w = problem(q_idx, [[[1, 3]]], k_idx, top_k=2)
    s = oracle.index_scores(w)
    assert s.tolist() == [[[3.0, 0.0, 14.0]]]


def test_scores_all_ones_closed_form():
    Hi, Di, L = 5, 7, 9
    w_h = RNG.integers(1, 9, (1, 1, Hi)).astype(np.float32)
    w = problem(np.ones((1, 1, Hi, Di), np.float32), w_h, np.ones((1, L, Di), np.float32))
    s = oracle.index_scores(w)
    assert np.all(s == Di * w_h.sum())


def test_scores_opposite_head_contributes_nothing():
    k = RNG.integers(-4, 5, (1, 4, 6)).astype(np.float32)
    q_idx = np.stack([k[0, 2], -k[0, 2]])[None, None]  # head 0 = k2, head 1 = -k2
    w = problem(q_idx, [[[2.0, 5.0]]], k)
    s = oracle.index_scores(w)
    assert s[0, 0, 2] == 2.0 * float(k[0, 2] @ k[0, 2])


@pytest.mark.parametrize("T", [1, 3])
def test_scores_relu_identities_against_matmul(T):
    # relu(x) - relu(-x) = x and relu(x) + relu(-x) = |x| give, for every
    # visible s:  S(q) - S(-q) = sum_h w_h (q_h . k_s)  and
    #             S(q) + S(-q) = sum_h w_h |q_h . k_s|,
    # both of which numpy computes with a plain matmul.
    B, Hi, Di, L = 2, 3, 5, 11
    qi = RNG.integers(-4, 5, (B, T, Hi, Di)).astype(np.float32)
    ki = RNG.integers(-4, 5, (B, L, Di)).astype(np.float32)
    wh = RNG.integers(1, 9, (B, T, Hi)).astype(np.float32)
    lens = np.array([L, L - 4], np.int32)
    sp = oracle.index_scores(problem(qi, wh, ki, seq_lens=lens))
    sn = oracle.index_scores(problem(-qi, wh, ki, seq_lens=lens))
    for b in range(B):
        dots = np.einsum("thi,si->ths", qi[b].astype(np.float64), ki[b].astype(np.float64))
        lin = np.einsum("th,ths->ts", wh[b].astype(np.float64), dots)
        absd = np.einsum("th,ths->ts", wh[b].astype(np.float64), np.abs(dots))
        for t in range(T):
            vis = lens[b] - T + 1 + t
            assert np.array_equal(sp[b, t, :vis] - sn[b, t, :vis], lin[t, :vis])
            assert np.array_equal(sp[b, t, :vis] + sn[b, t, :vis], absd[t, :vis])
            assert np.all(np.isnan(sp[b, t, vis:]))  # causal: not visible


@pytest.mark.parametrize("T", [1, 2])
def test_scores_int64_brute_force(T):
    # Small integer inputs make every score an integer, so plain Python
    # integer arithmetic (no floating point anywhere: products, the ReLU as a
    # comparison, the weighted head sum) gives the exact value, which the
    # fp64 oracle must reproduce exactly.  Lengths are ragged and causal.
    B, Hi, Di, L = 2, 4, 9, 13
    rng = np.random.default_rng(99 + T)
    qi = rng.integers(-4, 5, (B, T, Hi, Di))
    ki = rng.integers(-4, 5, (B, L, Di))
    wh = rng.integers(1, 9, (B, T, Hi))
    lens = np.array([L, L - 5], np.int32)
    got = oracle.index_scores(problem(qi.astype(np.float32), wh.astype(np.float32), ki.astype(np.float32),
                                      seq_lens=lens))
    for b in range(B):
        for t in range(T):
            vis = int(lens[b]) - T + 1 + t
            for s in range(vis):
                want = 0
                for h in range(Hi):
                    dot = sum(int(qi[b, t, h, i]) * int(ki[b, s, i]) for i in range(Di))
                    want += int(wh[b, t, h]) * (dot if dot > 0 else 0)
                assert got[b, t, s] == want, (b, t, s, got[b, t, s], want)
            assert np.all(np.isnan(got[b, t, vis:]))


def test_scores_bf16_inputs_equal_f32_inputs():
    qi = RNG.integers(-4, 5, (1, 2, 3, 8)).astype(np.float32)
    ki = RNG.integers(-4, 5, (1, 6, 8)).astype(np.float32)
    wh = RNG.integers(1, 9, (1, 2, 3)).astype(np.float32)
    to_bf16 = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)  # exact for small ints
    a = oracle.index_scores(problem(qi, wh, ki))
    b = oracle.index_scores(problem(to_bf16(qi), wh, to_bf16(ki), q_idx_dtype=synth.BF16,
                                    idx_key_dtype=synth.BF16))
    assert _nan_eq(a, b)


def test_scores_fp8_keys_scale_and_query_quantisation():
    # With e4m3 keys: S = scale_s * S(unscaled) (ReLU is positively homogeneous),
    # and the index query is quantised to e4m3 first (4.3 -> 4.5).
    Di, L = 4, 5
    codes = np.array([[[0x38, 0x40, 0xB8, 0x00], [0x44, 0x38, 0x38, 0xC0], [0x00] * 4,
                       [0x40, 0x40, 0x40, 0x40], [0xB8, 0x38, 0x44, 0x30]]], np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    scale = np.array([[0.25, 4.0, 1.0, 0.5, 2.0]], np.float32)
    qi = np.array([[[[4.3, -1.0, 2.0, 0.5]]]], np.float32)
    wh = np.array([[[3.0]]], np.float32)
    s8 = oracle.index_scores(problem(qi, wh, codes, k_scale=scale, idx_key_dtype=synth.E4M3))
    q_quant = np.array([[[[4.5, -1.0, 2.0, 0.5]]]], np.float32)
    sf = oracle.index_scores(problem(q_quant, wh, vals))
    assert np.array_equal(s8[0, 0], sf[0, 0] * scale[0])


# ------------------------------------------------------------------ Top-K
def _check_topk_property(scores, vis, K, sel, cnt):
    n = min(K, vis)
    assert cnt == n
    chosen = sel[:n]
    assert np.all(sel[n:] == -1)
    assert np.all(np.diff(chosen) > 0), "ascending, no duplicates"
    assert np.all((chosen >= 0) & (chosen < vis))
    others = np.setdiff1d(np.arange(vis), chosen)
    for i in chosen:  # exhaustive pair check of the defining property
        for j in others:
            assert scores[i] > scores[j] or (scores[i] == scores[j] and i < j)


def test_topk_defining_property_bruteforce_many_ties():
    for trial in range(60):
        L = int(RNG.integers(1, 40))
        K = int(RNG.integers(1, 45))
        T = int(RNG.integers(1, 3))
        lens = np.array([int(RNG.integers(T, L + 1))], np.int32)
        sc = RNG.integers(0, 4, (1, T, L)).astype(np.float64)  # heavy ties
        w = problem(np.zeros((1, T, 1, 1), np.float32), [[[1.0]] * T], np.zeros((1, L, 1), np.float32),
                    seq_lens=lens, top_k=K)
        idx, cnt = oracle.topk(w, sc)
        for t in range(T):
            vis = int(lens[0]) - T + 1 + t
            _check_topk_property(sc[0, t], vis, K, idx[0, t], cnt[0, t])


def test_topk_matches_numpy_lexsort():
    L, K = 500, 37
    sc = RNG.integers(-20, 20, (1, 1, L)).astype(np.float64)
    w = problem(np.zeros((1, 1, 1, 1), np.float32), [[[1.0]]], np.zeros((1, L, 1), np.float32), top_k=K)
    idx, _ = oracle.topk(w, sc)
    order = np.lexsort((np.arange(L), -sc[0, 0]))  # primary: score desc, then position asc
    assert np.array_equal(idx[0, 0], np.sort(order[:K]))


def test_topk_special_cases():
    L = 30
    z = np.zeros((1, 1, L))
    mk = lambda K, lens=L: problem(np.zeros((1, 1, 1, 1), np.float32), [[[1.0]]],
                                   np.zeros((1, L, 1), np.float32), top_k=K,
                                   seq_lens=np.array([lens], np.int32))
    idx, cnt = oracle.topk(mk(8), z)  # all equal -> the lowest positions
    assert idx[0, 0].tolist() == list(range(8)) and cnt[0, 0] == 8
    idx, cnt = oracle.topk(mk(50, 12), z)  # K >= vis -> every visible position
    assert idx[0, 0, :12].tolist() == list(range(12)) and np.all(idx[0, 0, 12:] == -1)
    assert cnt[0, 0] == 12
    idx, cnt = oracle.topk(mk(5, 0), z)  # nothing visible
    assert cnt[0, 0] == 0 and np.all(idx == -1)


def test_topk_causal_draft_tokens():
    # T = 2: token 0 never sees the last filled row, token 1 does.
    L = 10
    sc = np.zeros((1, 2, L))
    sc[:, :, L - 1] = 100.0
    w = problem(np.zeros((1, 2, 1, 1), np.float32), [[[1.0], [1.0]]], np.zeros((1, L, 1), np.float32),
                top_k=3)
    idx, _ = oracle.topk(w, sc)
    assert L - 1 not in idx[0, 0] and L - 1 in idx[0, 1]


# ------------------------------------------------------------------ attention
def _rand_attn(B=2, T=2, H=3, Dqk=10, Dv=6, L=17, K=5, lens=None):
    q = RNG.normal(size=(B, T, H, Dqk)).astype(np.float32)
    kv = RNG.normal(size=(B, L, Dqk)).astype(np.float32)
    if lens is None:
        lens = np.array([L, L - 5][:B], np.int32)
    w = problem(np.zeros((B, T, 1, 1), np.float32), np.ones((B, T, 1), np.float32),
                np.zeros((B, L, 1), np.float32), q=q, kv=kv, seq_lens=lens, top_k=K, v_dim=Dv)
    return w


def _sdpa(w, b, t, rows):
    """torch scaled-dot-product attention (float64, CPU) of one query over `rows`."""
    q = torch.from_numpy(w.q[b, t].astype(np.float64))[None, :, None, :]       # [1,H,1,Dqk]
    c = torch.from_numpy(w.kv[b, rows].astype(np.float64))                     # [n,Dqk]
    k = c[None, None].expand(1, w.heads, -1, -1)
    v = c[:, : w.v_dim][None, None].expand(1, w.heads, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=w.softmax_scale)
    return o[0, :, 0].numpy()


def test_attention_all_visible_equals_dense_sdpa():
    w = _rand_attn(K=40)
    idx = np.full((w.batch, w.q_len, w.top_k), -1, np.int32)
    for b in range(w.batch):
        for t in range(w.q_len):
            vis = w.vis(b, t)
            idx[b, t, :vis] = np.arange(vis)
    out, lse = oracle.sparse_mla(w, idx)
    for b in range(w.batch):
        for t in range(w.q_len):
            rows = np.arange(w.vis(b, t))
            np.testing.assert_allclose(out[b, t], _sdpa(w, b, t, rows), rtol=1e-12, atol=1e-13)
            logits = torch.from_numpy(w.q[b, t].astype(np.float64)) @ torch.from_numpy(
                w.kv[b, rows].astype(np.float64)).T * w.softmax_scale
            np.testing.assert_allclose(lse[b, t], torch.logsumexp(logits, -1).numpy(), rtol=1e-13)


def test_attention_selected_equals_masked_dense_sdpa():
    w = _rand_attn(K=5)
    idx = np.full((w.batch, w.q_len, w.top_k), -1, np.int32)
    for b in range(w.batch):
        for t in range(w.q_len):
            idx[b, t, :4] = np.sort(RNG.choice(w.vis(b, t), 4, replace=False))
    out, _ = oracle.sparse_mla(w, idx)
    for b in range(w.batch):
        for t in range(w.q_len):
            L = w.max_seq_len
            mask = torch.zeros(L, dtype=torch.bool)
            mask[idx[b, t, :4]] = True
            q = torch.from_numpy(w.q[b, t].astype(np.float64))[None, :, None, :]
            c = torch.from_numpy(w.kv[b].astype(np.float64))
            o = torch.nn.functional.scaled_dot_product_attention(
                q, c[None, None].expand(1, w.heads, -1, -1),
                c[:, : w.v_dim][None, None].expand(1, w.heads, -1, -1),
                attn_mask=mask[None, None, None, :], scale=w.softmax_scale)
            np.testing.assert_allclose(out[b, t], o[0, :, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_attention_weights_sum_to_one_and_reproduce_output():
    w = _rand_attn(K=6)
    idx = np.full((w.batch, w.q_len, w.top_k), -1, np.int32)
    idx[:, :, :5] = [0, 2, 3, 7, 9]
    out, _ = oracle.sparse_mla(w, idx)
    for b in range(w.batch):
        for t in range(w.q_len):
            for h in range(w.heads):
                p = oracle.attention_weights(w, idx, b, t, h)
                assert abs(p.sum() - 1.0) <= 1e-12
                assert p[5] == 0.0
                recon = p[:5] @ w.kv[b, idx[b, t, :5], : w.v_dim].astype(np.float64)
                np.testing.assert_allclose(out[b, t, h], recon, rtol=1e-12, atol=1e-14)


def test_attention_closed_forms():
    w = _rand_attn(B=1, T=1, K=4, lens=np.array([17], np.int32))
    rows = [1, 5, 6, 12]
    idx = np.array([[rows]], np.int32)
    # q = 0 -> uniform weights -> mean of the selected value rows
    w0 = _rand_attn(B=1, T=1, K=4, lens=np.array([17], np.int32))
    w0.q[:] = 0
    w0.kv[:] = w.kv
    out, lse = oracle.sparse_mla(w0, idx)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(
        w.kv[0, rows, : w.v_dim].astype(np.float64).mean(0), out[0, 0].shape), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, math.log(4.0), rtol=1e-14)
    # a single selected row -> that row's value part
    idx1 = np.array([[[7, -1, -1, -1]]], np.int32)
    out, _ = oracle.sparse_mla(w, idx1)
    assert np.array_equal(out[0, 0], np.broadcast_to(w.kv[0, 7, : w.v_dim].astype(np.float64),
                                                     out[0, 0].shape))
    # two rows with logit gap D -> weights sigmoid(D), sigmoid(-D)
    w2 = _rand_attn(B=1, T=1, H=1, Dqk=4, Dv=4, L=3, K=2, lens=np.array([3], np.int32))
    w2.q[:] = 0
    w2.q[0, 0, 0, 0] = 2.0
    w2.kv[:] = 0
    w2.kv[0, 0] = [1.5, 1.0, 0.0, 0.0]
    w2.kv[0, 2] = [-0.5, 0.0, 1.0, 0.0]
    D = w2.softmax_scale * 2.0 * (1.5 - (-0.5))
    s = 1.0 / (1.0 + math.exp(-D))
    out, _ = oracle.sparse_mla(w2, np.array([[[0, 2]]], np.int32))
    np.testing.assert_allclose(out[0, 0, 0], [s * 1.5 + (1 - s) * -0.5, s, 1 - s, 0.0], rtol=1e-14)


def test_attention_index_order_invariance_and_empty():
    w = _rand_attn(K=5)
    idx = np.full((w.batch, w.q_len, 5), -1, np.int32)
    idx[:, :, :4] = [2, 8, 3, 11]
    a, la = oracle.sparse_mla(w, idx)
    idx2 = idx.copy()
    idx2[:, :, :4] = [11, 3, 2, 8]
    b, lb = oracle.sparse_mla(w, idx2)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(la, lb, rtol=1e-14)
    out, lse = oracle.sparse_mla(w, np.full_like(idx, -1))
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_attention_fp8_cache_with_row_scales_equals_decoded_f32():
    B, T, H, Dqk, Dv, L, K = 1, 1, 2, 8, 6, 9, 4
    codes = RNG.integers(0, 256, (B, L, Dqk)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30  # no NaN codes
    scale = (2.0 ** RNG.integers(-2, 3, (B, L))).astype(np.float32)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy() * scale[..., None]
    q = RNG.normal(size=(B, T, H, Dqk)).astype(np.float32)
    idx = np.array([[[0, 4, 5, 8]]], np.int32)
    mk = lambda kv, kvd, sc: problem(np.zeros((B, T, 1, 1), np.float32), np.ones((B, T, 1), np.float32),
                                     np.zeros((B, L, 1), np.float32), q=q, kv=kv, top_k=K, v_dim=Dv,
                                     kv_dtype=kvd, kv_scale=sc)
    a, _ = oracle.sparse_mla(mk(codes, synth.E4M3, scale), idx)
    b, _ = oracle.sparse_mla(mk(vals.astype(np.float32), synth.F32, None), idx)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ MXFP8 index keys
# The pages quantise index Q and K in groups of 32 with one scale each
# ("Inference Acceleration for New Large Model Architectures" §4.1) in the MXFP8
# format ("Long-Context LLM Inference Optimization", Layered Quantization).  The
# quantiser follows the OCP MX v1.0 conversion (shared exponent floor(log2 amax)
# minus 8, saturating E4M3 elements).

def test_e8m0_decoder_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([oracle.e8m0_value(int(c)) for c in codes])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


def test_mx_quantize_closed_forms():
    e, el = oracle.mx_quantize(np.ones(32))
    assert e == 127 - 8 and np.all(el == 256.0)          # 1 = 256 * 2^-8
    e, el = oracle.mx_quantize([1.875, 1.0, -0.5])
    assert e == 119 and list(el) == [448.0, 256.0, -128.0]  # 480 saturates to 448
    e, el = oracle.mx_quantize([0.0] * 8)
    assert e == 0 and np.all(el == 0.0)
    e, el = oracle.mx_quantize([2.0 ** 10, 3.0])            # amax a power of two -> 256
    assert e == 127 + 10 - 8 and list(el) == [256.0, 0.75]
    e, el = oracle.mx_quantize([2.0 ** -130])              # shared exponent clamps at -127
    assert e == 0 and list(el) == [0.125]
    e, el = oracle.mx_quantize([2.0 ** 140, -2.0 ** 139])  # and at +127: elements saturate
    assert e == 254 and list(el) == [448.0, -448.0]


def test_mx_quantize_error_bound_and_top_binade():
    rng = np.random.default_rng(11)
    for trial in range(300):
        v = rng.normal(size=32) * 2.0 ** rng.integers(-20, 20)
        if trial % 7 == 0:
            v[rng.integers(0, 32)] *= 1000.0  # an outlier in the group
        e, el = oracle.mx_quantize(v)
        X = 2.0 ** (e - 127)
        deq = el * X
        # the largest magnitude lands in E4M3's top binade [256, 512) before saturation
        assert 256.0 <= np.max(np.abs(v)) / X < 512.0
        for x, d, q in zip(v, deq, el):
            if abs(x) / X > 448.0:
                assert q == math.copysign(448.0, x)
            else:  # half an ulp: 2^-4 relative for normals, 2^-10 * X for subnormals
                assert abs(d - x) <= max(abs(x) * 2.0 ** -4, X * 2.0 ** -10) * (1 + 1e-12)


def _mx_problem(q_idx, head_w, codes, scale_bytes, seq_lens=None):
    return problem(q_idx, head_w, codes, k_scale=scale_bytes, idx_key_dtype=synth.MXE4M3,
                   q_idx_dtype=synth.F32, seq_lens=seq_lens)


def test_mx_scores_equal_exact_dot_products_of_decoded_keys():
    # Queries whose groups quantise exactly (integers up to 4, plus an outlier
    # group: each group has its own scale so the small groups stay exact):
    # the score is the plain definition over the decoded keys.
    rng = np.random.default_rng(5)
    B, T, Hi, Di, L = 2, 2, 3, 96, 11
    qi = rng.integers(-4, 5, (B, T, Hi, Di)).astype(np.float32)
    qi[0, 0, 1, :32] *= 64.0  # group 0 of one head much larger than its other groups
    codes = rng.integers(0, 0x7F, (B, L, Di)).astype(np.uint8) | (rng.integers(0, 2, (B, L, Di)) << 7).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    sb = rng.integers(120, 135, (B, L, Di // 32)).astype(np.uint8)
    wh = rng.integers(1, 6, (B, T, Hi)).astype(np.float32)
    got = oracle.index_scores(_mx_problem(qi, wh, codes, sb))
    kdec = np.array([[[oracle.e4m3_value(int(c)) * oracle.e8m0_value(int(sb[b, s, i // 32]))
                       for i, c in enumerate(codes[b, s])] for s in range(L)] for b in range(B)])
    for b in range(B):
        for t in range(T):
            vis = L - T + 1 + t
            dots = qi[b, t].astype(np.float64) @ kdec[b, :vis].T  # [Hi, vis]
            want = (wh[b, t][:, None] * np.maximum(dots, 0.0)).sum(0)
            assert np.array_equal(got[b, t, :vis], want)
            assert np.all(np.isnan(got[b, t, vis:]))


def test_mx_scores_reduce_to_row_scaled_fp8_when_group_scales_agree():
    rng = np.random.default_rng(6)
    B, T, Hi, Di, L = 1, 1, 4, 64, 9
    qi = rng.integers(-4, 5, (B, T, Hi, Di)).astype(np.float32)
    codes = (rng.integers(0, 9, (B, L, Di)) * 8 + 0x30).astype(np.uint8)  # values 0.5 .. 16
    codes |= (rng.integers(0, 2, (B, L, Di)) << 7).astype(np.uint8)
    ex = rng.integers(-3, 4, (B, L))
    wh = np.ones((B, T, Hi), np.float32)
    mx = oracle.index_scores(_mx_problem(qi, wh, codes, np.repeat((ex + 127)[..., None], 2, -1)))
    row = oracle.index_scores(problem(qi, wh, codes, k_scale=2.0 ** ex, idx_key_dtype=synth.E4M3))
    assert np.array_equal(mx, row, equal_nan=True)


def test_mx_scores_scale_equivariance_and_group_locality():
    rng = np.random.default_rng(8)
    B, T, Hi, Di, L = 1, 1, 2, 128, 7
    qi = rng.normal(size=(B, T, Hi, Di)).astype(np.float32)  # quantisation rounds here
    codes = rng.integers(0, 0x7E, (B, L, Di)).astype(np.uint8)
    sb = rng.integers(124, 131, (B, L, 4)).astype(np.uint8)
    wh = np.array([[[1.0, 2.0]]], np.float32)
    base = oracle.index_scores(_mx_problem(qi, wh, codes, sb))
    # doubling the query doubles every group's scale and leaves the elements
    assert np.array_equal(oracle.index_scores(_mx_problem(2 * qi, wh, codes, sb)), 2 * base, equal_nan=True)
    # one more in every scale byte of row 3 doubles that row's score only
    sb2 = sb.copy()
    sb2[0, 3] += 1
    s2 = oracle.index_scores(_mx_problem(qi, wh, codes, sb2))
    assert s2[0, 0, 3] == 2 * base[0, 0, 3]
    assert np.array_equal(np.delete(s2, 3, axis=2), np.delete(base, 3, axis=2), equal_nan=True)
    # zeroing the key elements of group 2 of row 1 equals dropping that group's products
    c3 = codes.copy()
    c3[0, 1, 64:96] = 0
    s3 = oracle.index_scores(_mx_problem(qi, wh, c3, sb))
    qdeq = np.zeros((Hi, Di))
    for h in range(Hi):
        for g in range(4):
            e, el = oracle.mx_quantize(qi[0, 0, h, 32 * g:32 * g + 32].astype(np.float64))
            qdeq[h, 32 * g:32 * g + 32] = el * 2.0 ** (e - 127)
    kdec = np.array([oracle.e4m3_value(int(c)) for c in c3[0, 1]]) * \
        np.repeat([2.0 ** (int(x) - 127) for x in sb[0, 1]], 32)
    assert math.isclose(s3[0, 0, 1], float((wh[0, 0] * np.maximum(qdeq @ kdec, 0)).sum()), rel_tol=1e-12)


# ------------------------------------------------------------------ FP8 cache, 128-column tiles
# One scale per token and 128-element tile of the main cache ("Inference
# Acceleration for New Large Model Architectures" §4.2).

def test_attention_tile_scales_single_row_reproduces_decoded_row():
    B, T, H, Dqk, Dv, L, K = 1, 1, 2, 300, 260, 4, 3  # tiles of 128, 128, 44 columns
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 0x7E, (B, L, Dqk)).astype(np.uint8) | (rng.integers(0, 2, (B, L, Dqk)) << 7).astype(np.uint8)
    scale = np.array([[[0.5, 4.0, 0.25]] * L], np.float32) * (1 + np.arange(L))[None, :, None].astype(np.float32)
    q = rng.normal(size=(B, T, H, Dqk)).astype(np.float32)
    w = problem(np.zeros((B, T, 1, 1), np.float32), np.ones((B, T, 1), np.float32),
                np.zeros((B, L, 1), np.float32), q=q, kv=codes, top_k=K, v_dim=Dv,
                kv_dtype=synth.E4M3T128, kv_scale=scale, softmax_scale=0.125)
    out, lse = oracle.sparse_mla(w, np.array([[[2, -1, -1]]], np.int32))
    row = torch.from_numpy(codes[0, 2]).view(torch.float8_e4m3fn).double().numpy() * \
        np.repeat(scale[0, 2], [128, 128, 44])
    assert np.array_equal(out[0, 0], np.stack([row[:Dv]] * H))
    np.testing.assert_allclose(lse[0, 0], 0.125 * (q[0, 0].astype(np.float64) @ row), rtol=1e-13)


def test_attention_tile_scales_reduce_to_row_scales():
    B, T, H, Dqk, Dv, L, K = 1, 2, 3, 256 + 64, 256, 10, 4
    rng = np.random.default_rng(10)
    codes = rng.integers(0, 0x7E, (B, L, Dqk)).astype(np.uint8)
    rs = (2.0 ** rng.integers(-2, 3, (B, L))).astype(np.float32)
    q = rng.normal(size=(B, T, H, Dqk)).astype(np.float32)
    idx = np.array([[[1, 3, 7, 9], [0, 2, 5, -1]]], np.int32)
    mk = lambda kvd, sc: problem(np.zeros((B, T, 1, 1), np.float32), np.ones((B, T, 1), np.float32),
                                 np.zeros((B, L, 1), np.float32), q=q, kv=codes, top_k=K, v_dim=Dv,
                                 kv_dtype=kvd, kv_scale=sc)
    a = oracle.sparse_mla(mk(synth.E4M3T128, np.repeat(rs[..., None], 3, -1)), idx)
    b = oracle.sparse_mla(mk(synth.E4M3, rs), idx)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
