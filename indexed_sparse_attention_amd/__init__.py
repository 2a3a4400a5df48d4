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
  dsa_forward_noalloc(...)  dsa_forward with the library's own device
                            workspace (for callers that cannot allocate)
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# (DSA_LIBRARY: another build of the same sources, e.g. a sanitised one)
LIB_PATH = os.environ.get("DSA_LIBRARY") or os.path.join(_HERE, "libdsa.so")

DSA_F32, DSA_BF16, DSA_FP8_E4M3, DSA_MXFP8_E4M3, DSA_FP8_E4M3_T128 = 0, 1, 2, 3, 4
FORWARD_STAGES = 3
NOALLOC_WORKSPACE_BYTES = 64 << 20  # DSA_NOALLOC_WORKSPACE_BYTES
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
    lib.dsa_forward_tile_tokens.argtypes = [PP]
    lib.dsa_forward_tile_tokens.restype = ctypes.c_int32
    lib.dsa_set_workgroup_trace.argtypes = [P, ctypes.c_int64]
    lib.dsa_set_workgroup_trace.restype = ctypes.c_int
    lib.dsa_forward.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P, P]
    lib.dsa_kernel_choice.argtypes = [PP, ctypes.c_char_p, ctypes.c_size_t]
    PG = ctypes.POINTER(Paging)
    lib.dsa_index_score_paged.argtypes = [PP, PG, P, P, P, P, P, P, P]
    lib.dsa_sparse_mla_decode_paged.argtypes = [PP, PG, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.dsa_forward_paged.argtypes = [PP, PG, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P, P]
    lib.dsa_forward_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
    for f in (lib.dsa_index_score, lib.dsa_topk, lib.dsa_sparse_mla_decode, lib.dsa_forward,
              lib.dsa_kernel_choice, lib.dsa_index_score_paged, lib.dsa_sparse_mla_decode_paged,
              lib.dsa_forward_paged, lib.dsa_forward_noalloc):
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


def _bad(msg: str):
    raise DsaError(1, msg)


_FLOAT_IN = (torch.float32, torch.bfloat16)
_OUT_CODE = {torch.float32: DSA_F32, torch.bfloat16: DSA_BF16}
_CODE_IN = (torch.float32, torch.bfloat16, torch.float8_e4m3fn, torch.uint8)
_E8M0 = (torch.uint8, torch.float8_e8m0fnu)


def _expect(t: Optional[torch.Tensor], name: str, shape: tuple, dtypes: tuple, device=None) -> None:
    """The C ABI sees raw pointers only, so this layer checks every tensor's
    shape, dtype and device against the problem before a call: a tensor of
    the wrong size would otherwise be read or written out of bounds.  (Kept
    to a few attribute reads per tensor: it runs on every call.)"""
    if (t.__class__ is torch.Tensor or isinstance(t, torch.Tensor)) and t.shape == shape and \
            t.dtype in dtypes and (device is None or t.device == device):
        return
    if t is None:
        _bad(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        _bad(f"{name} must be a torch.Tensor")
    want = tuple(int(x) for x in shape)
    if tuple(t.shape) != want:
        _bad(f"{name} must have shape {want}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        _bad(f"{name} must have dtype in {[str(d) for d in dtypes]}, got {t.dtype}")
    _bad(f"{name} is on {t.device}, expected {device}")


def _expect_none(t, name: str, why: str) -> None:
    if t is not None:
        _bad(f"{name} must be None {why}")


def _key_scale_check(k_scale, key_code: int, rows: tuple, idx_dim: int, device, name="k_scale") -> None:
    if key_code == DSA_FP8_E4M3:
        _expect(k_scale, name, rows, (torch.float32,), device)
    elif key_code == DSA_MXFP8_E4M3:
        _expect(k_scale, name, rows + (-(-idx_dim // 32),), _E8M0, device)
    else:
        _expect_none(k_scale, name, "unless the index keys are E4M3 codes")


def _kv_scale_check(kv_scale, kv_code: int, rows: tuple, qk_dim: int, device, name="kv_scale") -> None:
    if kv_code == DSA_FP8_E4M3:
        _expect(kv_scale, name, rows, (torch.float32,), device)
    elif kv_code == DSA_FP8_E4M3_T128:
        _expect(kv_scale, name, rows + (-(-qk_dim // 128),), (torch.float32,), device)
    else:
        _expect_none(kv_scale, name, "unless the latent cache holds E4M3 codes")


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def make_problem(*, batch, q_len, max_seq_len, idx_heads=1, idx_dim=1, heads=1, qk_dim=1, v_dim=1,
                 top_k=1, softmax_scale=None, q_idx_dtype=DSA_BF16, idx_key_dtype=DSA_BF16,
                 q_dtype=DSA_BF16, kv_dtype=DSA_BF16, out_dtype=DSA_BF16) -> Problem:
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(qk_dim) if qk_dim > 0 else 1.0
    return Problem(batch, q_len, max_seq_len, idx_heads, idx_dim, heads, qk_dim, v_dim, top_k,
                   softmax_scale, q_idx_dtype, idx_key_dtype, q_dtype, kv_dtype, out_dtype)


def forward_workspace_size(p: Problem) -> int:
    return load_library().dsa_forward_workspace_size(ctypes.byref(p))


def forward_tile_tokens(p: Problem) -> int:
    """Query tokens per token tile of dsa_forward on p (0: one pass over the
    whole problem; -1: invalid problem)."""
    return load_library().dsa_forward_tile_tokens(ctypes.byref(p))


TRACE_KINDS = ("scores", "topk_chunk", "topk_emit", "topk_row", "attention", "attention_merge")


def set_workgroup_trace(buf: Optional[torch.Tensor], slots: int = 0) -> None:
    """Per-workgroup clock stamps of every later launch into `buf` (an int64
    device tensor of len(TRACE_KINDS) * slots * 2 values, kept alive while
    set), laid out as [kind, workgroup, start / end] in TRACE_KINDS order;
    None turns tracing off."""
    lib = load_library()
    if buf is None:
        _check(lib.dsa_set_workgroup_trace(None, 0))
        return
    _expect(buf, "buf", (len(TRACE_KINDS) * slots * 2,), (torch.int64,), None)
    if buf.device.type != "cuda" or not buf.is_contiguous():
        _bad("buf must be a contiguous device tensor")
    _check(lib.dsa_set_workgroup_trace(_ptr(buf), slots))


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
    buf = ctypes.create_string_buffer(512)
    load_library().dsa_kernel_choice(ctypes.byref(p), buf, 512)
    return buf.value.decode()


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != device:
            _bad(f"workspace must be a tensor on {device}")
        return workspace
    if nbytes == 0:
        return None
    # zeroed: the leading counter region must be zero on the first call
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def _index_problem(q_idx, head_w, k_idx, seq_lens, top_k=1, k_scale=None, skip_head_w=False) -> dict:
    """Problem fields of the indexer, with every indexer tensor checked
    (head_w may be left out, as None, only where skip_head_w says so)."""
    if not isinstance(q_idx, torch.Tensor) or q_idx.dim() != 4:
        _bad("q_idx must be a [B,T,Hi,Di] tensor")
    B, T, Hi, Di = q_idx.shape
    dev = q_idx.device
    _expect(q_idx, "q_idx", (B, T, Hi, Di), _FLOAT_IN, dev)
    if not isinstance(k_idx, torch.Tensor) or k_idx.dim() != 3:
        _bad("k_idx must be a [B,Lmax,Di] tensor")
    L = k_idx.shape[1]
    _expect(k_idx, "k_idx", (B, L, Di), _CODE_IN, dev)
    if head_w is not None or not skip_head_w:
        _expect(head_w, "head_w", (B, T, Hi), (torch.float32,), dev)
    _expect(seq_lens, "seq_lens", (B,), (torch.int32,), dev)
    key = key_dtype_code(k_idx, k_scale)
    _key_scale_check(k_scale, key, (B, L), Di, dev)
    return dict(batch=B, q_len=T, max_seq_len=L, idx_heads=Hi, idx_dim=Di, top_k=top_k,
                q_idx_dtype=dtype_code(q_idx), idx_key_dtype=key)


def dsa_index_score(q_idx: torch.Tensor, head_w: torch.Tensor, k_idx: torch.Tensor,
                    seq_lens: torch.Tensor, k_scale: Optional[torch.Tensor] = None,
                    scores: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    lib = load_library()
    d = _index_problem(q_idx, head_w, k_idx, seq_lens, k_scale=k_scale)
    p = make_problem(**d)
    shape = (d["batch"], d["q_len"], d["max_seq_len"])
    if scores is None:
        scores = torch.empty(shape, dtype=torch.float32, device=q_idx.device)
    _expect(scores, "scores", shape, (torch.float32,), q_idx.device)
    _check(lib.dsa_index_score(ctypes.byref(p), _ptr(q_idx), _ptr(head_w), _ptr(k_idx), _ptr(k_scale),
                               _ptr(seq_lens), _ptr(scores), _stream(stream)))
    return scores


def dsa_topk(scores: torch.Tensor, seq_lens: torch.Tensor, top_k: int,
             workspace: Optional[torch.Tensor] = None, stream=None):
    lib = load_library()
    if not isinstance(scores, torch.Tensor) or scores.dim() != 3:
        _bad("scores must be a [B,T,Lmax] tensor")
    B, T, L = scores.shape
    dev = scores.device
    _expect(scores, "scores", (B, T, L), (torch.float32,), dev)
    _expect(seq_lens, "seq_lens", (B,), (torch.int32,), dev)
    p = make_problem(batch=B, q_len=T, max_seq_len=L, top_k=top_k)
    idx = torch.empty((B, T, top_k), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, T), dtype=torch.int32, device=dev)
    nbytes = lib.dsa_topk_workspace_size(ctypes.byref(p))
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.dsa_topk(ctypes.byref(p), _ptr(scores), _ptr(seq_lens), _ptr(idx), _ptr(cnt), _ptr(ws),
                        _nbytes(ws), _stream(stream)))
    return idx, cnt


def _mla_checks(q, kv, seq_lens, kv_scale, v_dim, topk_idx=None, top_k=None, kv_rows=None):
    """Checks the attention tensors; returns (B, T, H, Dqk, kv_code)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        _bad("q must be a [B,T,H,Dqk] tensor")
    B, T, H, Dqk = q.shape
    dev = q.device
    _expect(q, "q", (B, T, H, Dqk), _FLOAT_IN, dev)
    if kv_rows is None:
        if not isinstance(kv, torch.Tensor) or kv.dim() != 3:
            _bad("kv must be a [B,Lmax,Dqk] tensor")
        kv_rows = (B, kv.shape[1])
    _expect(kv, "kv", kv_rows + (Dqk,), _CODE_IN, dev)
    _expect(seq_lens, "seq_lens", (B,), (torch.int32,), dev)
    if not 1 <= v_dim <= Dqk:
        _bad(f"v_dim must be in [1, {Dqk}], got {v_dim}")
    code = kv_dtype_code(kv, kv_scale)
    _kv_scale_check(kv_scale, code, kv_rows, Dqk, dev)
    if topk_idx is not None:
        _expect(topk_idx, "topk_idx", (B, T, top_k), (torch.int32,), dev)
    return B, T, H, Dqk, code


def dsa_sparse_mla_decode(q: torch.Tensor, kv: torch.Tensor, topk_idx: torch.Tensor,
                          seq_lens: torch.Tensor, v_dim: int, softmax_scale: Optional[float] = None,
                          kv_scale: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                          return_lse: bool = True, workspace: Optional[torch.Tensor] = None,
                          stream=None):
    lib = load_library()
    if not isinstance(topk_idx, torch.Tensor) or topk_idx.dim() != 3:
        _bad("topk_idx must be a [B,T,K] tensor")
    K = topk_idx.shape[-1]
    B, T, H, Dqk, kv_code = _mla_checks(q, kv, seq_lens, kv_scale, v_dim, topk_idx, K)
    if out_dtype is None:
        out_dtype = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    if out_dtype not in _FLOAT_IN:
        _bad(f"out_dtype must be float32 or bfloat16, got {out_dtype}")
    p = make_problem(batch=B, q_len=T, max_seq_len=kv.shape[1], heads=H, qk_dim=Dqk, v_dim=v_dim,
                     top_k=K, softmax_scale=softmax_scale, q_dtype=dtype_code(q),
                     kv_dtype=kv_code, out_dtype=_OUT_CODE[out_dtype])
    out = torch.empty((B, T, H, v_dim), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = lib.dsa_sparse_mla_workspace_size(ctypes.byref(p))
    ws = _workspace(nbytes, q.device, workspace)
    _check(lib.dsa_sparse_mla_decode(ctypes.byref(p), _ptr(q), _ptr(kv), _ptr(kv_scale), _ptr(topk_idx),
                                     _ptr(seq_lens), _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws),
                                     _stream(stream)))
    return out, lse


def forward_problem(q_idx, k_idx, q, kv, seq_lens, top_k, v_dim, softmax_scale=None,
                    out_dtype: Optional[torch.dtype] = None, k_scale=None, kv_scale=None,
                    head_w=None) -> Problem:
    """dsa_problem of a dsa_forward call (head_w, when given, is checked too)."""
    d = _index_problem(q_idx, head_w, k_idx, seq_lens, top_k, k_scale, skip_head_w=True)
    B, T, H, Dqk, kv_code = _mla_checks(q, kv, seq_lens, kv_scale, v_dim,
                                        kv_rows=(d["batch"], d["max_seq_len"]))
    if (B, T) != (d["batch"], d["q_len"]):
        _bad(f"q is [{B},{T},...] but q_idx is [{d['batch']},{d['q_len']},...]")
    if out_dtype is None:
        out_dtype = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    if out_dtype not in _FLOAT_IN:
        _bad(f"out_dtype must be float32 or bfloat16, got {out_dtype}")
    d.update(heads=H, qk_dim=Dqk, v_dim=v_dim, softmax_scale=softmax_scale, q_dtype=dtype_code(q),
             kv_dtype=kv_code, out_dtype=_OUT_CODE[out_dtype])
    return make_problem(**d)


_OUT_KEYS = ("out", "lse", "topk_idx", "topk_count", "scores")


def _forward_outputs(p: Problem, dev, top_k: int, v_dim: int, return_scores: bool, return_lse: bool,
                     out: Optional[dict]) -> dict:
    """Outputs of a forward call: caller-supplied tensors (checked against the
    problem) or new ones."""
    B, T, H, L = p.batch, p.q_len, p.heads, p.max_seq_len
    spec = {"out": ((B, T, H, v_dim), (_torch_dtype(p.out_dtype),)),
            "lse": ((B, T, H), (torch.float32,)),
            "topk_idx": ((B, T, top_k), (torch.int32,)),
            "topk_count": ((B, T), (torch.int32,)),
            "scores": ((B, T, L), (torch.float32,))}
    o = dict(out or {})
    for k in o:
        if k not in _OUT_KEYS:
            _bad(f"unknown output {k!r} (expected one of {_OUT_KEYS})")
        if o[k] is not None:
            _expect(o[k], k, spec[k][0], spec[k][1], dev)
    for k in ("out", "topk_idx", "topk_count"):
        if o.get(k) is None:
            o[k] = torch.empty(spec[k][0], dtype=spec[k][1][0], device=dev)
    if return_lse and o.get("lse") is None:
        o["lse"] = torch.empty(spec["lse"][0], dtype=torch.float32, device=dev)
    if return_scores and o.get("scores") is None:
        o["scores"] = torch.empty(spec["scores"][0], dtype=torch.float32, device=dev)
    return {k: v for k, v in o.items() if v is not None}


def _events(stage_events):
    if stage_events is None:
        return None
    if len(stage_events) != FORWARD_STAGES + 1:
        _bad(f"stage_events must hold {FORWARD_STAGES + 1} events")
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
    kv_pages [num_pages, page_size, Dqk] (scales [num_pages, page_size] or
    [num_pages, page_size, groups]), block_table int32 [batch, max_pages]
    shared by both caches."""
    lib = load_library()
    if not isinstance(q_idx, torch.Tensor) or q_idx.dim() != 4:
        _bad("q_idx must be a [B,T,Hi,Di] tensor")
    B, T, Hi, Di = q_idx.shape
    dev = q_idx.device
    _expect(q_idx, "q_idx", (B, T, Hi, Di), _FLOAT_IN, dev)
    _expect(head_w, "head_w", (B, T, Hi), (torch.float32,), dev)
    _expect(seq_lens, "seq_lens", (B,), (torch.int32,), dev)
    if not isinstance(k_pages, torch.Tensor) or k_pages.dim() != 3:
        _bad("k_pages must be a [num_pages, page_size, Di] tensor")
    num_pages, page_size = k_pages.shape[:2]
    _expect(k_pages, "k_pages", (num_pages, page_size, Di), _CODE_IN, dev)
    key = key_dtype_code(k_pages, k_scales)
    _key_scale_check(k_scales, key, (num_pages, page_size), Di, dev, "k_scales")
    if not isinstance(block_table, torch.Tensor) or block_table.dim() != 2:
        _bad("block_table must be an int32 [batch, max_pages] tensor")
    _expect(block_table, "block_table", (B, block_table.shape[1]), (torch.int32,), dev)
    if block_table.shape[1] * page_size < max_seq_len:
        _bad(f"block_table covers {block_table.shape[1] * page_size} rows < max_seq_len {max_seq_len}")
    _, _, H, Dqk, kv_code = _mla_checks(q, kv_pages, seq_lens, kv_scales, v_dim,
                                        kv_rows=(num_pages, page_size))
    if tuple(q.shape[:2]) != (B, T):
        _bad(f"q is [{q.shape[0]},{q.shape[1]},...] but q_idx is [{B},{T},...]")
    if out_dtype is None:
        out_dtype = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    if out_dtype not in _FLOAT_IN:
        _bad(f"out_dtype must be float32 or bfloat16, got {out_dtype}")
    p = make_problem(batch=B, q_len=T, max_seq_len=max_seq_len, idx_heads=Hi, idx_dim=Di, heads=H,
                     qk_dim=Dqk, v_dim=v_dim, top_k=top_k, softmax_scale=softmax_scale,
                     q_idx_dtype=dtype_code(q_idx), idx_key_dtype=key, q_dtype=dtype_code(q),
                     kv_dtype=kv_code, out_dtype=_OUT_CODE[out_dtype])
    pg = Paging(_ptr(block_table), page_size, block_table.shape[1], num_pages)
    o = _forward_outputs(p, dev, top_k, v_dim, return_scores, return_lse, out)
    ws = _workspace(lib.dsa_forward_workspace_size(ctypes.byref(p)), dev, workspace)
    _check(lib.dsa_forward_paged(ctypes.byref(p), ctypes.byref(pg), _ptr(q_idx), _ptr(head_w), _ptr(k_pages),
                                 _ptr(k_scales), _ptr(q), _ptr(kv_pages), _ptr(kv_scales), _ptr(seq_lens),
                                 _ptr(o.get("scores")), _ptr(o["topk_idx"]), _ptr(o["topk_count"]),
                                 _ptr(o["out"]), _ptr(o.get("lse")), _ptr(ws), _nbytes(ws), _stream(stream),
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
    'topk_count', 'scores' tensors (checked against the problem, reused as
    given)."""
    lib = load_library()
    p = forward_problem(q_idx, k_idx, q, kv, seq_lens, top_k, v_dim, softmax_scale, out_dtype, k_scale,
                        kv_scale, head_w=head_w)
    dev = q.device
    o = _forward_outputs(p, dev, top_k, v_dim, return_scores, return_lse, out)
    nbytes = lib.dsa_forward_workspace_size(ctypes.byref(p))
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.dsa_forward(ctypes.byref(p), _ptr(q_idx), _ptr(head_w), _ptr(k_idx), _ptr(k_scale),
                           _ptr(q), _ptr(kv), _ptr(kv_scale), _ptr(seq_lens), _ptr(o.get("scores")),
                           _ptr(o["topk_idx"]), _ptr(o["topk_count"]), _ptr(o["out"]),
                           _ptr(o.get("lse")), _ptr(ws), _nbytes(ws), _stream(stream), _events(stage_events)))
    return o


def dsa_forward_noalloc(q_idx: torch.Tensor, head_w: torch.Tensor, k_idx: torch.Tensor, q: torch.Tensor,
                        kv: torch.Tensor, seq_lens: torch.Tensor, top_k: int, v_dim: int,
                        softmax_scale: Optional[float] = None, k_scale: Optional[torch.Tensor] = None,
                        kv_scale: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                        return_scores: bool = False, return_lse: bool = True, out: Optional[dict] = None,
                        stage_events: Optional[Sequence] = None, stream=None) -> dict:
    """dsa_forward with the workspace the library keeps on each GPU (no
    workspace argument, no device allocation by the library).  Every output
    must be preallocated in ``out`` for a call that may allocate nothing at
    all; missing outputs are allocated here with torch.  Calls that overlap on
    one GPU race on that workspace."""
    lib = load_library()
    p = forward_problem(q_idx, k_idx, q, kv, seq_lens, top_k, v_dim, softmax_scale, out_dtype, k_scale,
                        kv_scale, head_w=head_w)
    o = _forward_outputs(p, q.device, top_k, v_dim, return_scores, return_lse, out)
    _check(lib.dsa_forward_noalloc(ctypes.byref(p), _ptr(q_idx), _ptr(head_w), _ptr(k_idx), _ptr(k_scale),
                                   _ptr(q), _ptr(kv), _ptr(kv_scale), _ptr(seq_lens), _ptr(o.get("scores")),
                                   _ptr(o["topk_idx"]), _ptr(o["topk_count"]), _ptr(o["out"]),
                                   _ptr(o.get("lse")), _stream(stream), _events(stage_events)))
    return o
