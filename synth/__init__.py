"""Seeded synthetic inputs for the DSA decode/prefill workloads.

Test and benchmark infrastructure shared by the oracle side and the GPU side.
It only fills input tensors (queries, index keys, head weights, latent cache,
lengths, scales) from a counter-based SplitMix64 stream; it contains none of
the method's arithmetic.  The C generator lives in ``gen.c`` and is built into
``libsynth.so`` next to this file.

Workloads (``WORKLOADS``) follow the shapes the pages' long-context decode
discussion implies (indexer heads x dim, MLA latent 512 + rope 64, Top-K),
scaled as listed:

  tiny      B=1,  T=1,    L=256,        fp32, indexer 4x32,  MLA 4 heads 80/64,   K=32
  decode8k  B=32, T=1,    L=8192,       bf16, indexer 64x128, MLA 128 heads 576/512, K=2048
  decode128k B=8, T=1,    L=131072 max, lengths uniform in [98304, 131072], as decode8k
  prefill64k B=1, T=4096, L=65536 (61440 cached + 4096 new), causal, as decode8k
  prompt8k  B=1, T=8192, L=8192: a fresh prompt (token t sees t + 1 rows), as decode8k
  fp8_1m    B=4,  T=2,    L=1048576,    e4m3 index keys and latent cache with one
            power-of-two scale per token in {2^-2..2^2}; bf16 queries
  mx128k    as decode128k, with MXFP8 index keys (e4m3 integers, one E8M0 scale
            byte 2^-2..2^2 per 32 dims) and an e4m3 latent cache with one
            power-of-two scale 2^-2..2^2 per 128-column tile of each row

Index inputs are integers so every score is an exactly representable integer.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# (DSA_SYNTH_LIBRARY: another build of gen.c, e.g. a sanitised one)
_LIB_PATH = os.environ.get("DSA_SYNTH_LIBRARY") or os.path.join(_HERE, "libsynth.so")
_lib = None

F32, BF16, E4M3, MXE4M3, E4M3T128 = 0, 1, 2, 3, 4
DTYPE_NAMES = {F32: "f32", BF16: "bf16", E4M3: "e4m3", MXE4M3: "mxfp8", E4M3T128: "e4m3-t128"}
_NP = {F32: np.float32, BF16: np.uint16, E4M3: np.uint8, MXE4M3: np.uint8, E4M3T128: np.uint8}
MX_GROUP, KV_TILE = 32, 128

# tensor ids of the stream keys
T_QIDX, T_KIDX, T_W, T_Q, T_KV, T_LENS, T_KSCALE, T_KVSCALE = 1, 2, 3, 4, 5, 6, 7, 8


def build(force: bool = False) -> str:
    """Compile gen.c into libsynth.so (gcc, OpenMP)."""
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P, I64, U64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int
        lib.synth_fill_int.argtypes = [P, I, I64, U64, U64, I64, I64]
        lib.synth_fill_normal.argtypes = [P, I, I64, U64, U64]
        lib.synth_fill_i32.argtypes = [P, I64, U64, U64, I64, I64]
        lib.synth_fill_pow2_scale.argtypes = [P, I64, U64, U64, I, I]
        lib.synth_fill_normal_e4m3_scaled.argtypes = [P, P, I64, I64, U64, U64]
        lib.synth_fill_normal_e4m3_tiled.argtypes = [P, P, I64, I64, I64, U64, U64]
        lib.synth_raw.argtypes = [P, I64, U64, U64]
        lib.synth_splitmix64_from_state.argtypes = [U64, I64, P]
        lib.synth_splitmix64_from_state.restype = None
        for f in (lib.synth_fill_int, lib.synth_fill_normal, lib.synth_fill_i32,
                  lib.synth_fill_pow2_scale, lib.synth_fill_normal_e4m3_scaled,
                  lib.synth_fill_normal_e4m3_tiled, lib.synth_raw):
            f.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def raw(n: int, seed: int, tensor_id: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _load().synth_raw(_ptr(out), n, seed, tensor_id)
    return out


def splitmix64_from_state(state: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _load().synth_splitmix64_from_state(state, n, _ptr(out))
    return out


def ints(shape, dtype: int, lo: int, hi: int, seed: int, tensor_id: int) -> np.ndarray:
    out = np.empty(shape, _NP[dtype])
    _load().synth_fill_int(_ptr(out), dtype, out.size, seed, tensor_id, lo, hi)
    return out


def normals(shape, dtype: int, seed: int, tensor_id: int) -> np.ndarray:
    assert dtype in (F32, BF16)
    out = np.empty(shape, _NP[dtype])
    _load().synth_fill_normal(_ptr(out), dtype, out.size, seed, tensor_id)
    return out


def i32(shape, lo: int, hi: int, seed: int, tensor_id: int) -> np.ndarray:
    out = np.empty(shape, np.int32)
    _load().synth_fill_i32(_ptr(out), out.size, seed, tensor_id, lo, hi)
    return out


def pow2_scales(shape, elo: int, ehi: int, seed: int, tensor_id: int) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _load().synth_fill_pow2_scale(_ptr(out), out.size, seed, tensor_id, elo, ehi)
    return out


def normals_e4m3(shape, scale: np.ndarray, seed: int, tensor_id: int) -> np.ndarray:
    """e4m3 codes of N(0,1)/scale[row]; rows are the leading dims of ``shape``."""
    out = np.empty(shape, np.uint8)
    row_len = shape[-1]
    n_rows = out.size // row_len
    assert scale.size == n_rows and scale.dtype == np.float32
    _load().synth_fill_normal_e4m3_scaled(_ptr(out), _ptr(np.ascontiguousarray(scale)),
                                          n_rows, row_len, seed, tensor_id)
    return out


def normals_e4m3_tiled(shape, scale: np.ndarray, tile: int, seed: int, tensor_id: int) -> np.ndarray:
    """e4m3 codes of N(0,1)/scale[row, tile]; scale has shape [rows, ceil(row_len/tile)]."""
    out = np.empty(shape, np.uint8)
    row_len = shape[-1]
    n_rows = out.size // row_len
    assert scale.size == n_rows * -(-row_len // tile) and scale.dtype == np.float32
    _load().synth_fill_normal_e4m3_tiled(_ptr(out), _ptr(np.ascontiguousarray(scale)),
                                         n_rows, row_len, tile, seed, tensor_id)
    return out


def e8m0_scales(shape, elo: int, ehi: int, seed: int, tensor_id: int) -> np.ndarray:
    """E8M0 scale bytes 127 + e with e uniform on [elo, ehi] (scale 2^e)."""
    return (i32(shape, elo, ehi, seed, tensor_id) + 127).astype(np.uint8)


@dataclasses.dataclass
class Workload:
    """One seeded DSA problem instance (host arrays, C-contiguous)."""
    name: str
    batch: int
    q_len: int
    max_seq_len: int
    idx_heads: int
    idx_dim: int
    heads: int
    qk_dim: int
    v_dim: int
    top_k: int
    softmax_scale: float
    q_idx_dtype: int
    idx_key_dtype: int
    q_dtype: int
    kv_dtype: int
    out_dtype: int
    seq_lens: np.ndarray          # [B] int32
    q_idx: np.ndarray             # [B,T,Hi,Di]
    head_w: np.ndarray            # [B,T,Hi] float32
    k_idx: np.ndarray             # [B,Lmax,Di]
    k_scale: Optional[np.ndarray]  # [B,Lmax] float32 (e4m3), [B,Lmax,Di/32] uint8 E8M0 (mxfp8) or None
    q: np.ndarray                 # [B,T,H,Dqk]
    kv: np.ndarray                # [B,Lmax,Dqk]
    kv_scale: Optional[np.ndarray]  # [B,Lmax] float32 (e4m3), [B,Lmax,ceil(Dqk/128)] (e4m3-t128) or None
    seed: int

    def vis(self, b: int, t: int) -> int:
        """Visible prefix of query token t of sequence b (causal)."""
        return int(self.seq_lens[b]) - self.q_len + 1 + t

    def dims(self) -> dict:
        return {k: getattr(self, k) for k in (
            "batch", "q_len", "max_seq_len", "idx_heads", "idx_dim", "heads", "qk_dim",
            "v_dim", "top_k", "softmax_scale", "q_idx_dtype", "idx_key_dtype", "q_dtype",
            "kv_dtype", "out_dtype")}


# name -> (number, recipe defaults)
WORKLOADS = {
    "tiny": dict(number=1, batch=1, q_len=1, max_seq_len=256, len_range=(256, 256),
                 idx_heads=4, idx_dim=32, idx_int=(-3, 3), w_int=(1, 4), heads=4, qk_dim=80,
                 v_dim=64, top_k=32, idx_dtype=F32, q_dtype=F32, kv_dtype=F32, out_dtype=F32,
                 fp8=False),
    "decode8k": dict(number=2, batch=32, q_len=1, max_seq_len=8192, len_range=(8192, 8192),
                     idx_heads=64, idx_dim=128, idx_int=(-4, 4), w_int=(1, 8), heads=128,
                     qk_dim=576, v_dim=512, top_k=2048, idx_dtype=BF16, q_dtype=BF16,
                     kv_dtype=BF16, out_dtype=BF16, fp8=False),
    "decode128k": dict(number=3, batch=8, q_len=1, max_seq_len=131072,
                       len_range=(98304, 131072), idx_heads=64, idx_dim=128, idx_int=(-4, 4),
                       w_int=(1, 8), heads=128, qk_dim=576, v_dim=512, top_k=2048,
                       idx_dtype=BF16, q_dtype=BF16, kv_dtype=BF16, out_dtype=BF16, fp8=False),
    "prefill64k": dict(number=4, batch=1, q_len=4096, max_seq_len=65536,
                       len_range=(65536, 65536), idx_heads=64, idx_dim=128, idx_int=(-4, 4),
                       w_int=(1, 8), heads=128, qk_dim=576, v_dim=512, top_k=2048,
                       idx_dtype=BF16, q_dtype=BF16, kv_dtype=BF16, out_dtype=BF16, fp8=False),
    "prompt8k": dict(number=7, batch=1, q_len=8192, max_seq_len=8192, len_range=(8192, 8192),
                     idx_heads=64, idx_dim=128, idx_int=(-4, 4), w_int=(1, 8), heads=128, qk_dim=576,
                     v_dim=512, top_k=2048, idx_dtype=BF16, q_dtype=BF16, kv_dtype=BF16, out_dtype=BF16,
                     fp8=False),
    "fp8_1m": dict(number=5, batch=4, q_len=2, max_seq_len=1048576,
                   len_range=(1048576, 1048576), idx_heads=64, idx_dim=128, idx_int=(-4, 4),
                   w_int=(1, 8), heads=128, qk_dim=576, v_dim=512, top_k=2048,
                   idx_dtype=BF16, q_dtype=BF16, kv_dtype=E4M3, out_dtype=BF16, fp8=True,
                   scale_exp=(-2, 2)),
    "mx128k": dict(number=6, batch=8, q_len=1, max_seq_len=131072,
                   len_range=(98304, 131072), idx_heads=64, idx_dim=128, idx_int=(-4, 4),
                   w_int=(1, 8), heads=128, qk_dim=576, v_dim=512, top_k=2048,
                   idx_dtype=BF16, q_dtype=BF16, kv_dtype=E4M3T128, out_dtype=BF16, fp8="mx",
                   scale_exp=(-2, 2)),
}


def make(name: str, seed: Optional[int] = None, **overrides) -> Workload:
    """Generate workload ``name`` (see WORKLOADS), optionally with smaller sizes.

    ``overrides`` may replace any recipe entry (batch, q_len, max_seq_len,
    len_range, top_k, heads, ...) so tests can run the same recipe at sizes the
    oracle finishes in seconds.
    """
    r = dict(WORKLOADS[name])
    if "max_seq_len" in overrides and "len_range" not in overrides:
        L = overrides["max_seq_len"]
        lo, hi = r["len_range"]
        overrides = dict(overrides, len_range=(min(lo, L), min(hi, L)))
    r.update(overrides)
    if seed is None:
        seed = 0xD5A00000 + r["number"]
    B, T, L = r["batch"], r["q_len"], r["max_seq_len"]
    Hi, Di, H, Dqk = r["idx_heads"], r["idx_dim"], r["heads"], r["qk_dim"]
    lo, hi = r["len_range"]
    assert T <= lo <= hi <= L
    lens = i32((B,), lo, hi, seed, T_LENS) if lo != hi else np.full((B,), lo, np.int32)
    ilo, ihi = r["idx_int"]
    fp8 = r["fp8"]
    q_idx = ints((B, T, Hi, Di), r["idx_dtype"], ilo, ihi, seed, T_QIDX)
    head_w = ints((B, T, Hi), F32, r["w_int"][0], r["w_int"][1], seed, T_W)
    if fp8 == "mx":
        elo, ehi = r["scale_exp"]
        k_idx = ints((B, L, Di), E4M3, ilo, ihi, seed, T_KIDX)
        k_scale = e8m0_scales((B, L, -(-Di // MX_GROUP)), elo, ehi, seed, T_KSCALE)
        kv_scale = pow2_scales((B, L, -(-Dqk // KV_TILE)), elo, ehi, seed, T_KVSCALE)
        kv = normals_e4m3_tiled((B, L, Dqk), kv_scale, KV_TILE, seed, T_KV)
        key_dtype = MXE4M3
    elif fp8:
        elo, ehi = r["scale_exp"]
        k_idx = ints((B, L, Di), E4M3, ilo, ihi, seed, T_KIDX)
        k_scale = pow2_scales((B, L), elo, ehi, seed, T_KSCALE)
        kv_scale = pow2_scales((B, L), elo, ehi, seed, T_KVSCALE)
        kv = normals_e4m3((B, L, Dqk), kv_scale, seed, T_KV)
        key_dtype = E4M3
    else:
        k_idx = ints((B, L, Di), r["idx_dtype"], ilo, ihi, seed, T_KIDX)
        k_scale = kv_scale = None
        kv = normals((B, L, Dqk), r["kv_dtype"], seed, T_KV)
        key_dtype = r["idx_dtype"]
    q = normals((B, T, H, Dqk), r["q_dtype"], seed, T_Q)
    return Workload(
        name=name, batch=B, q_len=T, max_seq_len=L, idx_heads=Hi, idx_dim=Di, heads=H,
        qk_dim=Dqk, v_dim=r["v_dim"], top_k=r["top_k"], softmax_scale=1.0 / math.sqrt(Dqk),
        q_idx_dtype=r["idx_dtype"], idx_key_dtype=key_dtype, q_dtype=r["q_dtype"],
        kv_dtype=r["kv_dtype"], out_dtype=r["out_dtype"], seq_lens=lens, q_idx=q_idx,
        head_w=head_w, k_idx=k_idx, k_scale=k_scale, q=q, kv=kv, kv_scale=kv_scale, seed=seed)
