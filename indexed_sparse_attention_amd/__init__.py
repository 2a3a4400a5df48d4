"""Indexed sparse attention (DSA) for AMD Instinct MI355X (gfx950).

Thin Python binding of ``libdsa.so``: it checks tensor dtypes, shapes and
devices, fills the ``dsa_problem`` struct, allocates outputs and workspace
with torch, and passes raw device pointers plus torch's current HIP stream to
the C ABI declared in ``include/dsa.h``.  Every step of the computation runs in
the library's HIP kernels; nothing here computes.  If the library is missing
the import still works but every call raises ``DsaError``: there is no
fallback.

Entry points (same names as the C ABI):
  dsa_index_score(q_idx, head_w, k_idx, seq_lens, k_scale=None)       -> scores
  dsa_topk(scores, seq_lens, top_k, q_len)                             -> (idx, count)
  dsa_sparse_mla_decode(q, kv, topk_idx, seq_lens, v_dim, ...)         -> (out, lse)
  dsa_forward(q_idx, head_w, k_idx, q, kv, seq_lens, top_k, v_dim, ...) -> dict
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_F32, DSA_BF16, DSA_FP8_E4M3, DSA_MXFP8_E4M3, DSA_FP8_E4M3_T128 = 0, 1, 2, 3, 4
FORWARD_STAGES = 3
_STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED",
           3: "DSA_ERR_WORKSPACE_TOO_SMALL", 4: "DSA_ERR_HIP"}


class DsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


class Problem(ctypes.Structure):
    """Mirror of ``dsa_problem`` in include/dsa.h."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int64),
        ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("qk_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_idx_dtype", ctypes.c_int32), ("idx_key_dtype", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
    ]


_lib = None


class Paging(ctypes.Structure):
    """dsa_paging: block table (device int32 [batch, max_pages]) of paged caches."""
    _fields_ = [("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("num_pages", ctypes.c_int64)]


def make_paging(block_table: torch.Tensor, page_size: int, num_pages: int) -> Paging:
    assert block_table.dim() == 2 and block_table.dtype == torch.int32 and block_table.is_contiguous()
    return Paging(block_table.data_ptr(), page_size, block_table.shape[1], num_pages)


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdsa.so (torch is imported first so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise DsaError(4, f"{path} is not built; run __graft_entry__.build() "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    P, PP = ctypes.c_void_p, ctypes.POINTER(Problem)
    S = ctypes.c_int
    lib.dsa_abi_version.restype = ctypes.c_int
    lib.dsa_status_string.argtypes = [S]
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_index_score.argtypes = [PP, P, P, P, P, P, P, P]
    lib.dsa_topk_workspace_size.argtypes = [PP]
    lib.dsa_workspace_zero_bytes.argtypes = [PP]
    lib.dsa_workspace_init.argtypes = [P, ctypes.c_size_t, P]
    lib.dsa_topk.argtypes = [PP, P, P, P, P, P, ctypes.c_size_t, P]
    lib.dsa_sparse_mla_workspace_size.argtypes = [PP]
    lib.dsa_sparse_mla_decode.argtypes = [PP, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.dsa_forward_workspace_size.argtypes = [PP]
    lib.dsa_forward.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P, P]
    lib.dsa_kernel_choice.argtypes = [PP, ctypes.c_char_p, ctypes.c_size_t]
    PG = ctypes.POINTER(Paging)
    lib.dsa_index_score_paged.argtypes = [PP, PG, P, P, P, P, P, P, P]
    lib.dsa_sparse_mla_decode_paged.argtypes = [PP, PG, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.dsa_forward_paged.argtypes = [PP, PG, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P, P]
    for f in (lib.dsa_index_score, lib.dsa_topk, lib.dsa_sparse_mla_decode, lib.dsa_forward,
              lib.dsa_kernel_choice, lib.dsa_index_score_paged, lib.dsa_sparse_mla_decode_paged,
              lib.dsa_forward_paged):
        f.restype = ctypes.c_int
    for f in (lib.dsa_topk_workspace_size, lib.dsa_sparse_mla_workspace_size,
              lib.dsa_forward_workspace_size, lib.dsa_workspace_zero_bytes):
        f.restype = ctypes.c_size_t
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise DsaError(status, load_library().dsa_last_error().decode())


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):  # uint8 = raw E4M3 codes
        return DSA_FP8_E4M3
    raise DsaError(1, f"unsupported tensor dtype {t.dtype}")


def key_dtype_code(k: torch.Tensor, k_scale: Optional[torch.Tensor]) -> int:
    """Index-key format: E4M3 codes with uint8 (E8M0) scales are MXFP8."""
    c = dtype_code(k)
    if c == DSA_FP8_E4M3 and k_scale is not None and k_scale.dtype in (torch.uint8, torch.float8_e8m0fnu):
        return DSA_MXFP8_E4M3
    return c


def kv_dtype_code(kv: torch.Tensor, kv_scale: Optional[torch.Tensor]) -> int:
    """Latent-cache format: E4M3 codes with one more scale dimension than
    rows (one scale per 128-column tile) are FP8_E4M3_T128."""
    c = dtype_code(kv)
    if c == DSA_FP8_E4M3 and kv_scale is not None and kv_scale.dim() == kv.dim():
        return DSA_FP8_E4M3_T128
    return c


def _torch_dtype(code: int) -> torch.dtype:
    return {DSA_F32: torch.float32, DSA_BF16: torch.bfloat16}[code]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise DsaError(1, "tensors must live on the GPU")
    if not t.is_contiguous():
        raise DsaError(1, "tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_problem(*, batch, q_len, max_seq_len, idx_heads=1, idx_dim=1, heads=1, qk_dim=1, v_dim=1,
                 top_k=1, softmax_scale=None, q_idx_dtype=DSA_BF16, idx_key_dtype=DSA_BF16,
                 q_dtype=DSA_BF16, kv_dtype=DSA_BF16, out_dtype=DSA_BF16) -> Problem:
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(qk_dim) if qk_dim > 0 else 1.0
    return Problem(batch, q_len, max_seq_len, idx_heads, idx_dim, heads, qk_dim, v_dim, top_k,
                   softmax_scale, q_idx_dtype, idx_key_dtype, q_dtype, kv_dtype, out_dtype)


def forward_workspace_size(p: Problem) -> int:
    return load_library().dsa_forward_workspace_size(ctypes.byref(p))


def topk_workspace_size(p: Problem) -> int:
    return load_library().dsa_topk_workspace_size(ctypes.byref(p))


def workspace_zero_bytes(p: Problem) -> int:
    """Leading workspace bytes (counters) that must be zero when a call starts;
    every successful call leaves them zero."""
    return load_library().dsa_workspace_zero_bytes(ctypes.byref(p))


def workspace_init(ws: torch.Tensor, stream=None) -> None:
    """Zero a workspace on the device (once per new workspace)."""
    _check(load_library().dsa_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def sparse_mla_workspace_size(p: Problem) -> int:
    return load_library().dsa_sparse_mla_workspace_size(ctypes.byref(p))


def kernel_choice(p: Problem) -> str:
    buf = ctypes.create_string_buffer(256)
    load_library().dsa_kernel_choice(ctypes.byref(p), buf, 256)
    return buf.value.decode()


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return workspace
    if workspace is not None:
        return workspace
    # zeroed: the leading counter region must be zero on the first call
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def _index_problem(q_idx, k_idx, seq_lens, top_k=1, k_scale=None) -> dict:
    B, T, Hi, Di = q_idx.shape
    assert k_idx.dim() == 3 and k_idx.shape[0] == B and k_idx.shape[2] == Di, "k_idx must be [B,Lmax,Di]"
    assert seq_lens.shape == (B,) and seq_lens.dtype == torch.int32, "seq_lens must be int32 [B]"
    return dict(batch=B, q_len=T, max_seq_len=k_idx.shape[1], idx_heads=Hi, idx_dim=Di,
                top_k=top_k, q_idx_dtype=dtype_code(q_idx), idx_key_dtype=key_dtype_code(k_idx, k_scale))


def dsa_index_score(q_idx: torch.Tensor, head_w: torch.Tensor, k_idx: torch.Tensor,
                    seq_lens: torch.Tensor, k_scale: Optional[torch.Tensor] = None,
                    scores: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    lib = load_library()
    d = _index_problem(q_idx, k_idx, seq_lens, k_scale=k_scale)
    p = make_problem(**d)
    if scores is None:
        scores = torch.empty((d["batch"], d["q_len"], d["max_seq_len"]), dtype=torch.float32,
                             device=q_idx.device)
    _check(lib.dsa_index_score(ctypes.byref(p), _ptr(q_idx), _ptr(head_w), _ptr(k_idx), _ptr(k_scale),
                               _ptr(seq_lens), _ptr(scores), _stream(stream)))
    return scores


def dsa_topk(scores: torch.Tensor, seq_lens: torch.Tensor, top_k: int,
             workspace: Optional[torch.Tensor] = None, stream=None):
    lib = load_library()
    B, T, L = scores.shape
    p = make_problem(batch=B, q_len=T, max_seq_len=L, top_k=top_k)
    idx = torch.empty((B, T, top_k), dtype=torch.int32, device=scores.device)
    cnt = torch.empty((B, T), dtype=torch.int32, device=scores.device)
    nbytes = lib.dsa_topk_workspace_size(ctypes.byref(p))
    ws = _workspace(nbytes, scores.device, workspace)
    _check(lib.dsa_topk(ctypes.byref(p), _ptr(scores), _ptr(seq_lens), _ptr(idx), _ptr(cnt), _ptr(ws),
                        nbytes if workspace is None else ws.numel(), _stream(stream)))
    return idx, cnt


def dsa_sparse_mla_decode(q: torch.Tensor, kv: torch.Tensor, topk_idx: torch.Tensor,
                          seq_lens: torch.Tensor, v_dim: int, softmax_scale: Optional[float] = None,
                          kv_scale: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                          return_lse: bool = True, workspace: Optional[torch.Tensor] = None,
                          stream=None):
    lib = load_library()
    B, T, H, Dqk = q.shape
    assert kv.dim() == 3 and kv.shape[0] == B and kv.shape[2] == Dqk, "kv must be [B,Lmax,Dqk]"
    K = topk_idx.shape[-1]
    assert topk_idx.shape == (B, T, K) and topk_idx.dtype == torch.int32
    if out_dtype is None:
        out_dtype = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    p = make_problem(batch=B, q_len=T, max_seq_len=kv.shape[1], heads=H, qk_dim=Dqk, v_dim=v_dim,
                     top_k=K, softmax_scale=softmax_scale, q_dtype=dtype_code(q),
                     kv_dtype=kv_dtype_code(kv, kv_scale), out_dtype=dtype_code(torch.empty(0, dtype=out_dtype)))
    out = torch.empty((B, T, H, v_dim), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = lib.dsa_sparse_mla_workspace_size(ctypes.byref(p))
    ws = _workspace(nbytes, q.device, workspace)
    _check(lib.dsa_sparse_mla_decode(ctypes.byref(p), _ptr(q), _ptr(kv), _ptr(kv_scale), _ptr(topk_idx),
                                     _ptr(seq_lens), _ptr(out), _ptr(lse), _ptr(ws),
                                     0 if ws is None else ws.numel(), _stream(stream)))
    return out, lse


def forward_problem(q_idx, k_idx, q, kv, seq_lens, top_k, v_dim, softmax_scale=None,
                    out_dtype: Optional[torch.dtype] = None, k_scale=None, kv_scale=None) -> Problem:
    d = _index_problem(q_idx, k_idx, seq_lens, top_k, k_scale)
    B, T, H, Dqk = q.shape
    assert (B, T) == (d["batch"], d["q_len"]) and kv.shape == (B, d["max_seq_len"], Dqk)
    if out_dtype is None:
        out_dtype = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    d.update(heads=H, qk_dim=Dqk, v_dim=v_dim, softmax_scale=softmax_scale, q_dtype=dtype_code(q),
             kv_dtype=kv_dtype_code(kv, kv_scale), out_dtype=dtype_code(torch.empty(0, dtype=out_dtype)))
    return make_problem(**d)


def _forward_outputs(p: Problem, dev, top_k: int, v_dim: int, return_scores: bool, return_lse: bool,
                     out: Optional[dict]) -> dict:
    B, T, H = p.batch, p.q_len, p.heads
    o = dict(out or {})
    if "out" not in o:
        o["out"] = torch.empty((B, T, H, v_dim), dtype=_torch_dtype(p.out_dtype), device=dev)
    if return_lse and "lse" not in o:
        o["lse"] = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    if "topk_idx" not in o:
        o["topk_idx"] = torch.empty((B, T, top_k), dtype=torch.int32, device=dev)
    if "topk_count" not in o:
        o["topk_count"] = torch.empty((B, T), dtype=torch.int32, device=dev)
    if return_scores and "scores" not in o:
        o["scores"] = torch.empty((B, T, p.max_seq_len), dtype=torch.float32, device=dev)
    return o


def _events(stage_events):
    if stage_events is None:
        return None
    assert len(stage_events) == FORWARD_STAGES + 1
    return (ctypes.c_void_p * (FORWARD_STAGES + 1))(*[e.cuda_event for e in stage_events])


def dsa_forward_paged(q_idx: torch.Tensor, head_w: torch.Tensor, k_pages: torch.Tensor, q: torch.Tensor,
                      kv_pages: torch.Tensor, seq_lens: torch.Tensor, block_table: torch.Tensor,
                      top_k: int, v_dim: int, max_seq_len: int, softmax_scale: Optional[float] = None,
                      k_scales: Optional[torch.Tensor] = None, kv_scales: Optional[torch.Tensor] = None,
                      out_dtype: Optional[torch.dtype] = None, return_scores: bool = False,
                      return_lse: bool = True, out: Optional[dict] = None,
                      workspace: Optional[torch.Tensor] = None, stage_events: Optional[Sequence] = None,
                      stream=None) -> dict:
    """Whole path over paged caches: k_pages [num_pages, page_size, Di],
    kv_pages [num_pages, page_size, Dqk] (scales [num_pages, page_size]),
    block_table int32 [batch, max_pages] shared by both caches."""
    lib = load_library()
    num_pages, page_size, Di = k_pages.shape
    assert kv_pages.shape[:2] == (num_pages, page_size)
    B, T, Hi, _ = q_idx.shape
    _, _, H, Dqk = q.shape
    if out_dtype is None:
        out_dtype = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    p = make_problem(batch=B, q_len=T, max_seq_len=max_seq_len, idx_heads=Hi, idx_dim=Di, heads=H,
                     qk_dim=Dqk, v_dim=v_dim, top_k=top_k, softmax_scale=softmax_scale,
                     q_idx_dtype=dtype_code(q_idx), idx_key_dtype=key_dtype_code(k_pages, k_scales),
                     q_dtype=dtype_code(q), kv_dtype=kv_dtype_code(kv_pages, kv_scales),
                     out_dtype=dtype_code(torch.empty(0, dtype=out_dtype)))
    pg = make_paging(block_table, page_size, num_pages)
    o = _forward_outputs(p, q.device, top_k, v_dim, return_scores, return_lse, out)
    ws = _workspace(lib.dsa_forward_workspace_size(ctypes.byref(p)), q.device, workspace)
    _check(lib.dsa_forward_paged(ctypes.byref(p), ctypes.byref(pg), _ptr(q_idx), _ptr(head_w), _ptr(k_pages),
                                 _ptr(k_scales), _ptr(q), _ptr(kv_pages), _ptr(kv_scales), _ptr(seq_lens),
                                 _ptr(o.get("scores")), _ptr(o["topk_idx"]), _ptr(o["topk_count"]),
                                 _ptr(o["out"]), _ptr(o.get("lse")), _ptr(ws), ws.numel(), _stream(stream),
                                 _events(stage_events)))
    return o


def dsa_forward(q_idx: torch.Tensor, head_w: torch.Tensor, k_idx: torch.Tensor, q: torch.Tensor,
                kv: torch.Tensor, seq_lens: torch.Tensor, top_k: int, v_dim: int,
                softmax_scale: Optional[float] = None, k_scale: Optional[torch.Tensor] = None,
                kv_scale: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                return_scores: bool = False, return_lse: bool = True,
                out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None,
                stage_events: Optional[Sequence] = None, stream=None) -> dict:
    """Whole path.  ``out`` may hold preallocated 'out', 'lse', 'topk_idx',
    'topk_count', 'scores' tensors (reused as given)."""
    lib = load_library()
    p = forward_problem(q_idx, k_idx, q, kv, seq_lens, top_k, v_dim, softmax_scale, out_dtype, k_scale, kv_scale)
    dev = q.device
    B, T, H = p.batch, p.q_len, p.heads
    o = dict(out or {})
    if "out" not in o:
        o["out"] = torch.empty((B, T, H, v_dim), dtype=_torch_dtype(p.out_dtype), device=dev)
    if return_lse and "lse" not in o:
        o["lse"] = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    if "topk_idx" not in o:
        o["topk_idx"] = torch.empty((B, T, top_k), dtype=torch.int32, device=dev)
    if "topk_count" not in o:
        o["topk_count"] = torch.empty((B, T), dtype=torch.int32, device=dev)
    if return_scores and "scores" not in o:
        o["scores"] = torch.empty((B, T, p.max_seq_len), dtype=torch.float32, device=dev)
    nbytes = lib.dsa_forward_workspace_size(ctypes.byref(p))
    ws = _workspace(nbytes, dev, workspace)
    ev = None
    if stage_events is not None:
        assert len(stage_events) == FORWARD_STAGES + 1
        ev = (ctypes.c_void_p * (FORWARD_STAGES + 1))(*[e.cuda_event for e in stage_events])
    _check(lib.dsa_forward(ctypes.byref(p), _ptr(q_idx), _ptr(head_w), _ptr(k_idx), _ptr(k_scale),
                           _ptr(q), _ptr(kv), _ptr(kv_scale), _ptr(seq_lens), _ptr(o.get("scores")),
                           _ptr(o["topk_idx"]), _ptr(o["topk_count"]), _ptr(o["out"]),
                           _ptr(o.get("lse")), _ptr(ws), ws.numel(), _stream(stream), ev))
    return o
