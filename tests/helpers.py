"""Small helpers for building hand-made DSA problems in tests."""
import math

import numpy as np

import synth


def problem(q_idx, head_w, k_idx, q=None, kv=None, seq_lens=None, top_k=4, k_scale=None,
            kv_scale=None, q_idx_dtype=synth.F32, idx_key_dtype=synth.F32, q_dtype=synth.F32,
            kv_dtype=synth.F32, v_dim=None, softmax_scale=None):
    """Wrap explicit arrays as a synth.Workload (shapes are inferred)."""
    q_idx = np.ascontiguousarray(q_idx)
    k_idx = np.ascontiguousarray(k_idx)
    B, T, Hi, Di = q_idx.shape
    L = k_idx.shape[1]
    if q is None:
        q = np.zeros((B, T, 1, 2), np.float32)
    if kv is None:
        kv = np.zeros((B, L, 2), np.float32)
    q = np.ascontiguousarray(q)
    kv = np.ascontiguousarray(kv)
    H, Dqk = q.shape[2], q.shape[3]
    if seq_lens is None:
        seq_lens = np.full((B,), L, np.int32)
    if v_dim is None:
        v_dim = Dqk
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    return synth.Workload(
        name="hand", batch=B, q_len=T, max_seq_len=L, idx_heads=Hi, idx_dim=Di, heads=H,
        qk_dim=Dqk, v_dim=v_dim, top_k=top_k, softmax_scale=softmax_scale,
        q_idx_dtype=q_idx_dtype, idx_key_dtype=idx_key_dtype, q_dtype=q_dtype,
        kv_dtype=kv_dtype, out_dtype=synth.F32,
        seq_lens=np.ascontiguousarray(seq_lens, dtype=np.int32), q_idx=q_idx,
        head_w=np.ascontiguousarray(head_w, dtype=np.float32), k_idx=k_idx,
        k_scale=None if k_scale is None else np.ascontiguousarray(
            k_scale, dtype=np.uint8 if idx_key_dtype == synth.MXE4M3 else np.float32),
        q=q, kv=kv,
        kv_scale=None if kv_scale is None else np.ascontiguousarray(kv_scale, dtype=np.float32),
        seed=0)
