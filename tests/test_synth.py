"""The seeded input generator: stream definition, encodings and recipes."""
import numpy as np
import torch

import synth


def test_splitmix64_published_outputs():
    # SplitMix64 started from state 0 (Steele, Lea, Flood 2014; the same
    # generator as java.util.SplittableRandom's mixer): first three outputs.
    out = synth.splitmix64_from_state(0, 3)
    assert [int(x) for x in out] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_stream_is_counter_based_and_keyed():
    a = synth.raw(1000, 7, 3)
    b = synth.raw(10, 7, 3)
    assert np.array_equal(a[:10], b)
    assert not np.array_equal(synth.raw(10, 7, 4), b)
    assert not np.array_equal(synth.raw(10, 8, 3), b)


def test_int_fill_range_and_uniformity():
    x = synth.ints((200000,), synth.F32, -4, 4, 11, 1)
    assert x.min() == -4 and x.max() == 4 and np.all(x == np.round(x))
    counts = np.bincount((x + 4).astype(int))
    assert np.all(np.abs(counts / len(x) - 1 / 9) < 0.005)


def test_bf16_and_e4m3_encodings_match_torch_rounding():
    x = synth.normals((50000,), synth.F32, 5, 4)
    bf = synth.normals((50000,), synth.BF16, 5, 4)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf, ref)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    # e4m3 of N(0,1)/scale: decoding with torch and multiplying by the row
    # scale recovers the sample to e4m3 precision
    scale = synth.pow2_scales((500,), -2, 2, 5, 8)
    assert set(np.log2(scale).astype(int)) <= {-2, -1, 0, 1, 2}
    codes = synth.normals_e4m3((500, 100), scale, 5, 4)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy() * scale[:, None]
    xs = x[:50000].astype(np.float64).reshape(500, 100)
    want = torch.from_numpy(xs / scale[:, None]).to(torch.float8_e4m3fn).double().numpy() * scale[:, None]
    assert np.array_equal(dec, want)


def test_e4m3_integer_codes_exact():
    c = synth.ints((1000,), synth.E4M3, -4, 4, 3, 2)
    v = torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    assert set(v.tolist()) <= set(range(-4, 5)) and len(set(v.tolist())) == 9


def test_recipes_shapes_small():
    for name in synth.WORKLOADS:
        r = synth.WORKLOADS[name]
        L = 1024
        T = min(r["q_len"], 8)
        w = synth.make(name, batch=2, q_len=T, max_seq_len=L, len_range=(L // 2, L), top_k=16)
        assert w.q_idx.shape == (2, T, w.idx_heads, w.idx_dim)
        assert w.k_idx.shape == (2, L, w.idx_dim)
        assert w.q.shape == (2, T, w.heads, w.qk_dim)
        assert w.kv.shape == (2, L, w.qk_dim)
        assert w.head_w.shape == (2, T, w.idx_heads)
        assert np.all((w.seq_lens >= L // 2) & (w.seq_lens <= L))
        assert (w.k_scale is not None) == (name in ("fp8_1m", "mx128k"))
        if name == "mx128k":  # one E8M0 byte per 32 dims, one scale per 128-column tile
            assert w.k_scale.shape == (2, L, w.idx_dim // 32) and w.k_scale.dtype == np.uint8
            assert w.kv_scale.shape == (2, L, -(-w.qk_dim // 128))
        assert abs(w.softmax_scale - w.qk_dim ** -0.5) < 1e-15


def test_recipe_is_reproducible():
    a = synth.make("decode128k", batch=2, max_seq_len=512, len_range=(300, 512))
    b = synth.make("decode128k", batch=2, max_seq_len=512, len_range=(300, 512))
    for f in ("q_idx", "k_idx", "head_w", "q", "kv", "seq_lens"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
