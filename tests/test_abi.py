"""The C ABI: the library loads without a GPU, exports every symbol that
include/dsa.h declares, and rejects bad arguments before any HIP call
(so every case here runs on a machine with no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import indexed_sparse_attention_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dsa.LIB_PATH), reason="libdsa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for f in ("dsa_index_score", "dsa_topk", "dsa_sparse_mla_decode", "dsa_forward"):
        assert f in names


def test_every_declared_symbol_is_exported():
    out = subprocess.check_output(["nm", "-D", "--defined-only", dsa.LIB_PATH]).decode()
    exported = set(re.findall(r"\bT (dsa_[a-z_0-9]+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    lib = dsa.load_library()
    for n in declared_functions():
        getattr(lib, n)


def test_status_strings_and_version():
    lib = dsa.load_library()
    assert lib.dsa_abi_version() == 6
    assert lib.dsa_status_string(0) == b"DSA_OK"
    assert lib.dsa_status_string(3) == b"DSA_ERR_WORKSPACE_TOO_SMALL"


def good_problem(**kw):
    d = dict(batch=2, q_len=1, max_seq_len=4096, idx_heads=64, idx_dim=128, heads=128, qk_dim=576,
             v_dim=512, top_k=2048)
    d.update(kw)
    return dsa.make_problem(**d)


BAD_PROBLEMS = [
    dict(batch=0), dict(q_len=0), dict(max_seq_len=0), dict(q_len=5000), dict(max_seq_len=2 ** 31),
    dict(idx_heads=0), dict(idx_dim=0), dict(heads=0), dict(qk_dim=0), dict(v_dim=0),
    dict(v_dim=577), dict(top_k=0), dict(softmax_scale=0.0), dict(softmax_scale=-1.0),
    dict(softmax_scale=float("inf")), dict(softmax_scale=float("nan")), dict(q_idx_dtype=2),
    dict(idx_key_dtype=4), dict(idx_key_dtype=5), dict(q_dtype=2), dict(kv_dtype=-1), dict(kv_dtype=3),
    dict(kv_dtype=5), dict(out_dtype=2),
]

FAKE = 0x10000  # a 16-byte aligned non-NULL address: never dereferenced, calls fail validation first


@pytest.mark.parametrize("kw", BAD_PROBLEMS)
def test_invalid_problem_rejected_everywhere(kw):
    lib = dsa.load_library()
    p = good_problem(**kw)
    P = ctypes.byref(p)
    assert lib.dsa_forward_workspace_size(P) == 0
    assert lib.dsa_forward_tile_tokens(P) == -1
    assert lib.dsa_topk_workspace_size(P) == 0
    assert lib.dsa_sparse_mla_workspace_size(P) == 0
    f = FAKE
    assert lib.dsa_index_score(P, f, f, f, None, f, f, None) == 1
    assert lib.dsa_topk(P, f, f, f, f, f, 1 << 40, None) == 1
    assert lib.dsa_sparse_mla_decode(P, f, f, None, f, f, f, f, f, 1 << 40, None) == 1
    assert lib.dsa_forward(P, f, f, f, None, f, f, None, f, None, None, None, f, f, f, 1 << 40, None, None) == 1
    assert lib.dsa_last_error() != b""


def test_null_problem():
    lib = dsa.load_library()
    assert lib.dsa_forward_workspace_size(None) == 0
    assert lib.dsa_index_score(None, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == 1
    assert b"NULL" in lib.dsa_last_error()


def test_pointer_checks():
    lib = dsa.load_library()
    p = good_problem()
    P = ctypes.byref(p)
    f = FAKE
    # NULL or misaligned tensors
    assert lib.dsa_index_score(P, None, f, f, None, f, f, None) == 1
    assert lib.dsa_index_score(P, f + 8, f, f, None, f, f, None) == 1
    assert lib.dsa_index_score(P, f, f, f + 4, None, f, f, None) == 1
    assert lib.dsa_index_score(P, f, f, f, None, f, None, None) == 1
    # scales: required for FP8, forbidden otherwise
    assert lib.dsa_index_score(P, f, f, f, f, f, f, None) == 1
    assert b"k_scale" in lib.dsa_last_error()
    p8 = good_problem(idx_key_dtype=2)
    assert lib.dsa_index_score(ctypes.byref(p8), f, f, f, None, f, f, None) == 1
    assert b"k_scale" in lib.dsa_last_error()
    pk8 = good_problem(kv_dtype=2)
    assert lib.dsa_sparse_mla_decode(ctypes.byref(pk8), f, f, None, f, f, f, f, f, 1 << 40, None) == 1
    assert b"kv_scale" in lib.dsa_last_error()
    # MXFP8 keys need their E8M0 group scales (any alignment); 128-column
    # tile scales of an FP8 cache are fp32 like the per-row ones
    pmx = good_problem(idx_key_dtype=3)
    assert lib.dsa_index_score(ctypes.byref(pmx), f, f, f, None, f, f, None) == 1
    assert b"k_scale" in lib.dsa_last_error()
    pt = good_problem(kv_dtype=4)
    assert lib.dsa_sparse_mla_decode(ctypes.byref(pt), f, f, None, f, f, f, f, f, 1 << 40, None) == 1
    assert b"kv_scale" in lib.dsa_last_error()
    assert lib.dsa_sparse_mla_decode(ctypes.byref(pt), f, f, f + 2, f, f, f, f, f, 1 << 40, None) == 1
    assert b"kv_scale" in lib.dsa_last_error()


def test_workspace_too_small_is_reported_before_launch():
    lib = dsa.load_library()
    p = good_problem()
    P = ctypes.byref(p)
    need = lib.dsa_forward_workspace_size(P)
    assert need > 0
    f = FAKE
    st = lib.dsa_forward(P, f, f, f, None, f, f, None, f, None, None, None, f, f, f, need - 1, None, None)
    assert st == 3 and b"workspace" in lib.dsa_last_error()
    need_t = lib.dsa_topk_workspace_size(P)
    assert lib.dsa_topk(P, f, f, f, None, f, need_t - 1, None) == 3


def test_workspace_sizes_monotone_in_problem_size():
    lib = dsa.load_library()
    sizes = [lib.dsa_forward_workspace_size(ctypes.byref(good_problem(max_seq_len=L)))
             for L in (1024, 4096, 65536, 131072)]
    assert sizes == sorted(sizes) and sizes[0] > 0
    sizes_b = [lib.dsa_forward_workspace_size(ctypes.byref(good_problem(batch=b))) for b in (1, 2, 8, 32)]
    assert sizes_b == sorted(sizes_b)
    # Top-K needs at least the score-key histograms and one candidate slot per position
    p = good_problem()
    assert lib.dsa_topk_workspace_size(ctypes.byref(p)) >= 2 * 1 * (4096 * 4 + 4096 * 4)


def test_token_tiles_keep_the_workspace_under_its_budget():
    lib = dsa.load_library()
    assert dsa.forward_tile_tokens(good_problem(batch=8, max_seq_len=131072)) == 0  # decode: one pass
    # a 4096-token prefill chunk over 64K keys: the largest power-of-two tile
    # whose scratch fits 1 GiB, and the workspace is that tile's
    p = good_problem(batch=1, q_len=4096, max_seq_len=65536)
    n = dsa.forward_tile_tokens(p)
    assert n == 512
    tile = good_problem(batch=1, q_len=n, max_seq_len=65536)
    twice = good_problem(batch=1, q_len=2 * n, max_seq_len=65536)
    ws = lib.dsa_forward_workspace_size(ctypes.byref(p))
    assert ws == lib.dsa_forward_workspace_size(ctypes.byref(tile)) <= 1 << 30
    assert dsa.forward_tile_tokens(tile) == 0 and dsa.forward_tile_tokens(twice) == n  # 2n tokens pass 1 GiB
    # a smaller budget gives smaller tiles, and an odd token count a ragged last tile
    os.environ["DSA_TILE_BUDGET"] = str(64 << 20)
    try:
        p3 = good_problem(batch=3, q_len=100, max_seq_len=65536)
        n3 = dsa.forward_tile_tokens(p3)
        assert 0 < n3 < 100 and n3 & (n3 - 1) == 0
        assert lib.dsa_forward_workspace_size(ctypes.byref(p3)) <= 64 << 20
    finally:
        del os.environ["DSA_TILE_BUDGET"]


def test_workgroup_trace_setting():
    lib = dsa.load_library()
    assert lib.dsa_set_workgroup_trace(FAKE + 4, 16) == 1 and b"aligned" in lib.dsa_last_error()
    # setting and clearing touch no GPU
    assert lib.dsa_set_workgroup_trace(FAKE, 16) == 0
    assert lib.dsa_set_workgroup_trace(None, 0) == 0
    assert lib.dsa_set_workgroup_trace(FAKE, 0) == 0  # no slots: off


def test_workspace_counter_region_and_init_validation():
    lib = dsa.load_library()
    p = good_problem(batch=3, q_len=2)
    z = lib.dsa_workspace_zero_bytes(ctypes.byref(p))
    # one 4096-bin histogram per query, at the start of the workspace
    assert z == 3 * 2 * 4096 * 4
    assert z < lib.dsa_topk_workspace_size(ctypes.byref(p)) <= lib.dsa_forward_workspace_size(ctypes.byref(p))
    assert lib.dsa_workspace_zero_bytes(None) == 0
    # argument checks happen before any HIP call
    assert lib.dsa_workspace_init(None, 64, None) == 1 and b"ws" in lib.dsa_last_error()
    assert lib.dsa_workspace_init(FAKE, 6, None) == 1 and b"multiple of 4" in lib.dsa_last_error()
    assert lib.dsa_workspace_init(FAKE + 2, 64, None) == 1
    assert lib.dsa_workspace_init(None, 0, None) == 0  # nothing to do


def test_stage_events_must_be_non_null():
    lib = dsa.load_library()
    p = good_problem()
    need = lib.dsa_forward_workspace_size(ctypes.byref(p))
    ev = (ctypes.c_void_p * 4)(FAKE, FAKE, None, FAKE)
    f = FAKE
    assert lib.dsa_forward(ctypes.byref(p), f, f, f, None, f, f, None, f, None, None, None, f, f,
                           0x100000, need, None, ev) == 1


def test_kernel_choice_reports_paths():
    p = good_problem()
    s = dsa.kernel_choice(p)
    assert "score=mfma" in s and "mla=mfma" in s
    tiny = dsa.make_problem(batch=1, q_len=1, max_seq_len=256, idx_heads=4, idx_dim=32, heads=4,
                            qk_dim=80, v_dim=64, top_k=32, q_idx_dtype=0, idx_key_dtype=0, q_dtype=0,
                            kv_dtype=0, out_dtype=0)
    s = dsa.kernel_choice(tiny)
    assert "score=generic" in s and "mla=generic" in s
    os.environ["DSA_FORCE_GENERIC"] = "1"
    try:
        assert "score=generic" in dsa.kernel_choice(p) and "mla=generic" in dsa.kernel_choice(p)
    finally:
        del os.environ["DSA_FORCE_GENERIC"]


def test_kernel_choice_names_the_launches():
    """The description follows the launch rules: the score kernel's shape and
    workgroup count, the Top-K mode and the token tile."""
    def prob(B, T, L):
        return dsa.make_problem(batch=B, q_len=T, max_seq_len=L, idx_heads=64, idx_dim=128, heads=128,
                                qk_dim=576, v_dim=512, top_k=2048, q_idx_dtype=1, idx_key_dtype=1, q_dtype=1,
                                kv_dtype=1, out_dtype=1)
    long_decode = dsa.kernel_choice(prob(8, 1, 131072))  # 8 sequences of 128K keys
    assert "1 token, ring 4" in long_decode and "chunks + emit" in long_decode and "tile_tokens=0" in long_decode
    short_decode = dsa.kernel_choice(prob(32, 1, 8192))  # short rows: 8-deep rings, one workgroup per query
    assert "1 token, ring 8" in short_decode and "one workgroup per query" in short_decode
    prefill = dsa.kernel_choice(prob(1, 4096, 65536))  # eight tokens per segment, token tiles of 512
    assert "8 tokens, shared LDS ring" in prefill and "tile_tokens=512" in prefill and "splits=1 " in prefill
    drafts = dsa.kernel_choice(prob(4, 2, 65536))  # two draft tokens: two per segment
    assert "2 tokens, ring 4" in drafts


def _paging(table=FAKE, page_size=64, max_pages=64, num_pages=1024):
    return dsa.Paging(table, page_size, max_pages, num_pages)


@pytest.mark.parametrize("kw,msg", [
    (dict(table=None), b"block_table"),
    (dict(table=FAKE + 2), b"block_table"),
    (dict(page_size=32), b"page_size"),
    (dict(page_size=96), b"page_size"),
    (dict(max_pages=63), b"max_pages"),
    (dict(num_pages=0), b"num_pages"),
    (dict(num_pages=1 << 26, page_size=64), b"2^31"),
])
def test_paging_descriptor_checked_before_launch(kw, msg):
    # 4096 rows = 64 pages of 64; every call fails validation before any HIP call
    lib = dsa.load_library()
    p = good_problem()
    P = ctypes.byref(p)
    pg = _paging(**kw)
    f = FAKE
    need = lib.dsa_forward_workspace_size(P)
    for st in (lib.dsa_index_score_paged(P, ctypes.byref(pg), f, f, f, None, f, f, None),
               lib.dsa_sparse_mla_decode_paged(P, ctypes.byref(pg), f, f, None, f, f, f, f, f, 1 << 40, None),
               lib.dsa_forward_paged(P, ctypes.byref(pg), f, f, f, None, f, f, None, f, None, None, None, f, f,
                                     0x100000, need, None, None)):
        assert st == 1, lib.dsa_last_error()
        assert msg in lib.dsa_last_error(), lib.dsa_last_error()
    assert lib.dsa_forward_paged(P, None, f, f, f, None, f, f, None, f, None, None, None, f, f, 0x100000, need,
                                 None, None) == 1


def test_paging_needs_the_matrix_core_kernels():
    lib = dsa.load_library()
    tiny = dsa.make_problem(batch=1, q_len=1, max_seq_len=256, idx_heads=4, idx_dim=32, heads=4,
                            qk_dim=80, v_dim=64, top_k=32, q_idx_dtype=0, idx_key_dtype=0, q_dtype=0,
                            kv_dtype=0, out_dtype=0)
    pg = _paging(max_pages=4)
    f = FAKE
    assert lib.dsa_index_score_paged(ctypes.byref(tiny), ctypes.byref(pg), f, f, f, None, f, f, None) == 2
    assert lib.dsa_sparse_mla_decode_paged(ctypes.byref(tiny), ctypes.byref(pg), f, f, None, f, f, f, f, f,
                                           1 << 40, None) == 2


def test_missing_library_fails_loudly(tmp_path):
    # no CPU fallback: without libdsa.so every entry point raises DsaError
    import subprocess
    import sys
    code = (
        "import torch, indexed_sparse_attention_amd as dsa\n"
        f"dsa.LIB_PATH = {str(tmp_path / 'absent.so')!r}\n"
        "orig = dsa.load_library\n"
        "dsa.load_library = lambda path=dsa.LIB_PATH: orig(path)\n"
        "t = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16)\n"
        "try:\n"
        "    dsa.dsa_index_score(t, torch.zeros(1, 1, 64), torch.zeros(1, 8, 128, dtype=torch.bfloat16),\n"
        "                        torch.zeros(1, dtype=torch.int32))\n"
        "except dsa.DsaError as e:\n"
        "    print('raised', e)\n"
        "else:\n"
        "    raise SystemExit('no error')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 0 and "raised" in r.stdout and "not built" in r.stdout, r.stdout + r.stderr


# ---------------------------------------------------------------- the binding's tensor checks
# The C ABI takes raw pointers, so the Python layer is what compares every
# tensor with the problem; a wrong shape or dtype must raise DsaError before
# any pointer reaches the library.  CPU tensors suffice: the checks run first.
def _cpu_forward_args(B=2, T=1, L=256, Hi=64, Di=128, H=128, Dqk=576, fp8=None):
    import torch
    a = dict(q_idx=torch.zeros(B, T, Hi, Di, dtype=torch.bfloat16),
             head_w=torch.zeros(B, T, Hi), k_idx=torch.zeros(B, L, Di, dtype=torch.bfloat16),
             q=torch.zeros(B, T, H, Dqk, dtype=torch.bfloat16), kv=torch.zeros(B, L, Dqk, dtype=torch.bfloat16),
             seq_lens=torch.full((B,), L, dtype=torch.int32), top_k=64, v_dim=512)
    if fp8 == "row":
        a.update(k_idx=torch.zeros(B, L, Di, dtype=torch.uint8), k_scale=torch.ones(B, L),
                 kv=torch.zeros(B, L, Dqk, dtype=torch.uint8), kv_scale=torch.ones(B, L))
    elif fp8 == "mx":
        a.update(k_idx=torch.zeros(B, L, Di, dtype=torch.uint8), k_scale=torch.full((B, L, Di // 32), 127, dtype=torch.uint8),
                 kv=torch.zeros(B, L, Dqk, dtype=torch.uint8), kv_scale=torch.ones(B, L, 5))
    return a


def _expect_dsa_error(fn, *args, match, **kw):
    with pytest.raises(dsa.DsaError) as e:
        fn(*args, **kw)
    assert e.value.status == 1 and match in str(e.value), str(e.value)


@pytest.mark.parametrize("field,bad,match", [
    ("head_w", ("shape", (2, 1, 63)), "head_w"),
    ("head_w", ("dtype", "bfloat16"), "head_w"),
    ("seq_lens", ("shape", (3,)), "seq_lens"),
    ("seq_lens", ("dtype", "int64"), "seq_lens"),
    ("k_idx", ("shape", (2, 256, 64)), "k_idx"),
    ("k_idx", ("shape", (3, 256, 128)), "k_idx"),
    ("q", ("shape", (2, 2, 128, 576)), "q"),
    ("kv", ("shape", (2, 255, 576)), "kv"),
    ("kv", ("shape", (2, 256, 512)), "kv"),
])
def test_binding_checks_forward_inputs(field, bad, match):
    import torch
    a = _cpu_forward_args()
    kind, v = bad
    if kind == "shape":
        a[field] = torch.zeros(v, dtype=a[field].dtype)
    else:
        a[field] = a[field].to(getattr(torch, v))
    _expect_dsa_error(dsa.dsa_forward, **a, match=match)


@pytest.mark.parametrize("fp8,field,shape,match", [
    ("row", "k_scale", (2, 255), "k_scale"),
    ("row", "kv_scale", (2, 256, 2), "kv_scale"),
    ("mx", "k_scale", (2, 256, 3), "k_scale"),
    ("mx", "kv_scale", (2, 256, 4), "kv_scale"),
])
def test_binding_checks_scale_layouts(fp8, field, shape, match):
    import torch
    a = _cpu_forward_args(fp8=fp8)
    a[field] = torch.zeros(shape, dtype=a[field].dtype)
    _expect_dsa_error(dsa.dsa_forward, **a, match=match)
    if field == "k_scale":
        _expect_dsa_error(dsa.dsa_index_score, a["q_idx"], a["head_w"], a["k_idx"], a["seq_lens"],
                          k_scale=a[field], match=match)
    else:
        idx = torch.zeros(2, 1, 64, dtype=torch.int32)
        _expect_dsa_error(dsa.dsa_sparse_mla_decode, a["q"], a["kv"], idx, a["seq_lens"], 512,
                          kv_scale=a[field], match=match)


@pytest.mark.parametrize("key,shape,dtype,match", [
    ("out", (2, 1, 128, 511), "bfloat16", "out"),
    ("out", (2, 1, 128, 512), "float32", "out"),       # a bf16 problem with an fp32 buffer
    ("lse", (2, 1, 127), "float32", "lse"),
    ("topk_idx", (2, 1, 63), "int32", "topk_idx"),
    ("topk_idx", (2, 1, 64), "int64", "topk_idx"),
    ("topk_count", (2,), "int32", "topk_count"),
    ("scores", (2, 1, 255), "float32", "scores"),
    ("bogus", (1,), "float32", "bogus"),
])
def test_binding_checks_preallocated_outputs(key, shape, dtype, match):
    import torch
    a = _cpu_forward_args()
    _expect_dsa_error(dsa.dsa_forward, **a, out={key: torch.zeros(shape, dtype=getattr(torch, dtype))}, match=match)


def test_binding_checks_the_other_entry_points():
    import torch
    a = _cpu_forward_args()
    _expect_dsa_error(dsa.dsa_index_score, a["q_idx"], a["head_w"], a["k_idx"], a["seq_lens"],
                      scores=torch.zeros(2, 1, 100), match="scores")
    _expect_dsa_error(dsa.dsa_topk, torch.zeros(2, 1, 256, dtype=torch.bfloat16), a["seq_lens"], 64, match="scores")
    _expect_dsa_error(dsa.dsa_topk, torch.zeros(2, 1, 256), torch.zeros(3, dtype=torch.int32), 64, match="seq_lens")
    _expect_dsa_error(dsa.dsa_sparse_mla_decode, a["q"], a["kv"], torch.zeros(2, 2, 64, dtype=torch.int32),
                      a["seq_lens"], 512, match="topk_idx")
    _expect_dsa_error(dsa.dsa_sparse_mla_decode, a["q"], a["kv"], torch.zeros(2, 1, 64, dtype=torch.int32),
                      a["seq_lens"], 577, match="v_dim")


def test_binding_checks_paged_inputs():
    import torch
    a = _cpu_forward_args()
    pages = dict(k_pages=torch.zeros(10, 64, 128, dtype=torch.bfloat16),
                 kv_pages=torch.zeros(10, 64, 576, dtype=torch.bfloat16),
                 block_table=torch.zeros(2, 4, dtype=torch.int32))
    base = dict(q_idx=a["q_idx"], head_w=a["head_w"], q=a["q"], seq_lens=a["seq_lens"], top_k=64, v_dim=512,
                max_seq_len=256)
    bad = [
        (dict(block_table=torch.zeros(3, 4, dtype=torch.int32)), "block_table"),
        (dict(block_table=torch.zeros(2, 3, dtype=torch.int32)), "max_seq_len"),
        (dict(k_pages=torch.zeros(10, 64, 64, dtype=torch.bfloat16)), "k_pages"),
        (dict(kv_pages=torch.zeros(10, 64, 512, dtype=torch.bfloat16)), "kv"),
        (dict(kv_pages=torch.zeros(9, 64, 576, dtype=torch.bfloat16)), "kv"),
    ]
    for change, match in bad:
        kw = dict(base, **pages)
        kw.update(change)
        _expect_dsa_error(dsa.dsa_forward_paged, match=match, **kw)


def test_noalloc_checks_arguments_and_size_before_any_hip_call():
    lib = dsa.load_library()
    f = FAKE
    # an invalid problem and a NULL pointer: rejected as for dsa_forward
    p = good_problem(top_k=0)
    assert lib.dsa_forward_noalloc(ctypes.byref(p), f, f, f, None, f, f, None, f, None, None, None, f, f,
                                   None, None) == 1
    p = good_problem()
    assert lib.dsa_forward_noalloc(ctypes.byref(p), None, f, f, None, f, f, None, f, None, None, None, f, f,
                                   None, None) == 1
    # a problem whose workspace exceeds the library's fixed one: a clear error
    big = good_problem(batch=8, q_len=2, max_seq_len=1 << 20)
    assert lib.dsa_forward_workspace_size(ctypes.byref(big)) > dsa.NOALLOC_WORKSPACE_BYTES
    assert lib.dsa_forward_noalloc(ctypes.byref(big), f, f, f, None, f, f, None, f, None, None, None, f, f,
                                   None, None) == 3
    assert b"dsa_forward_noalloc" in lib.dsa_last_error() and b"workspace" in lib.dsa_last_error()
