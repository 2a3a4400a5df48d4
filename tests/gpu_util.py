"""Helpers for GPU parity tests: move a synth.Workload to the device, run the
library through its C ABI, compare with the oracle at the stated bar."""
import numpy as np
import torch

import indexed_sparse_attention_amd as dsa
import synth

BF16_ABS, BF16_REL = 1e-2, 2e-2   # bf16 paths: |gpu - ref| <= 1e-2 + 2e-2 |ref|
FP8_ABS = 3e-2                    # fp8-cache paths: |gpu - ref| <= 3e-2


def _t(a, dtype_code, dev):
    if a is None:
        return None
    x = torch.from_numpy(np.ascontiguousarray(a))
    if dtype_code == synth.BF16:
        x = x.view(torch.bfloat16)
    return x.to(dev)


def to_device(w, dev="cuda:0"):
    return dict(
        q_idx=_t(w.q_idx, w.q_idx_dtype, dev), head_w=_t(w.head_w, synth.F32, dev),
        k_idx=_t(w.k_idx, w.idx_key_dtype, dev), k_scale=_t(w.k_scale, synth.F32, dev),
        q=_t(w.q, w.q_dtype, dev), kv=_t(w.kv, w.kv_dtype, dev), kv_scale=_t(w.kv_scale, synth.F32, dev),
        seq_lens=_t(w.seq_lens, synth.F32, dev))


def out_torch_dtype(w):
    return torch.float32 if w.out_dtype == synth.F32 else torch.bfloat16


def run_forward(w, d=None, **kw):
    d = d or to_device(w)
    r = dsa.dsa_forward(d["q_idx"], d["head_w"], d["k_idx"], d["q"], d["kv"], d["seq_lens"], w.top_k,
                        w.v_dim, w.softmax_scale, k_scale=d["k_scale"], kv_scale=d["kv_scale"],
                        out_dtype=out_torch_dtype(w), return_scores=True, **kw)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() if v.dtype == torch.bfloat16 else v.cpu().numpy()
            for k, v in r.items()}


def check_scores(w, got, ref, want=None):
    for b in range(w.batch):
        for t in range(w.q_len):
            if want is not None and not want[b, t]:
                continue
            vis = max(w.vis(b, t), 0)
            g = got[b, t, :vis].astype(np.float64)
            r = ref[b, t, :vis]
            bad = np.flatnonzero(g != r)
            assert bad.size == 0, (f"scores differ at b={b} t={t}: {bad.size} positions, first "
                                   f"s={bad[0]} gpu={g[bad[0]]} oracle={r[bad[0]]}")


def check_topk(w, idx, cnt, ref_idx, ref_cnt, want=None):
    for b in range(w.batch):
        for t in range(w.q_len):
            if want is not None and not want[b, t]:
                continue
            assert cnt[b, t] == ref_cnt[b, t], f"count b={b} t={t}: {cnt[b, t]} vs {ref_cnt[b, t]}"
            if not np.array_equal(idx[b, t], ref_idx[b, t]):
                diff = np.setxor1d(idx[b, t], ref_idx[b, t])
                raise AssertionError(f"Top-K differs at b={b} t={t}: {diff.size} positions differ, "
                                     f"e.g. {diff[:8].tolist()}")


def check_attention(w, out, lse, ref_out, ref_lse, want=None):
    sel = np.ones((w.batch, w.q_len), bool) if want is None else want.astype(bool)
    g = out[sel].astype(np.float64)
    r = ref_out[sel]
    err = np.abs(g - r)
    if w.kv_dtype in (synth.E4M3, synth.E4M3T128):
        ok = err <= FP8_ABS
        bar = f"abs {FP8_ABS}"
    else:
        ok = err <= BF16_ABS + BF16_REL * np.abs(r)
        bar = f"{BF16_ABS} + {BF16_REL}|ref|"
    assert ok.all(), f"attention outside {bar}: max abs err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"
    if lse is not None:
        gl, rl = lse[sel].astype(np.float64), ref_lse[sel]
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(gl), fin)
        assert np.all(np.abs(gl[fin] - rl[fin]) <= 1e-3 + 1e-4 * np.abs(rl[fin])), \
            f"lse max abs err {np.abs(gl[fin] - rl[fin]).max():.3e}"
    return float(err.max()) if err.size else 0.0
