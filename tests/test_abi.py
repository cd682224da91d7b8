"""C-ABI checks that need no GPU: the library loads, exports what include/cpattn.h declares, agrees with the binding on
struct layouts, and refuses bad arguments on the host before anything is enqueued (no compute call is made)."""
import ctypes as C
import os
import re

import pytest

from cp_slot_map_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(c\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for must in ("cp_slot_map", "cp_paged_attn_partial", "cp_own_token_attn", "cp_lse_merge"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} declared in cpattn.h but not exported"
        assert name in _lib.EXPORTS, f"{name} has no binding signature"


def test_struct_layouts_match(lib):
    assert lib.cpattn_struct_size(0) == C.sizeof(_lib.PagedArgs)
    assert lib.cpattn_struct_size(1) == C.sizeof(_lib.OwnArgs)
    assert lib.cpattn_struct_size(2) == C.sizeof(_lib.MergeArgs)
    assert lib.cpattn_struct_size(3) == C.sizeof(_lib.MergeOut)
    assert lib.cpattn_struct_size(7) == -1


def test_merged_call_refusals(lib):
    """cp_paged_attn_merged refuses a stripe subset, a missing or misaligned merged output and an unknown dtype, on
    the host."""
    m = _lib.MergeOut()
    m.out_dtype, m.out = 1, 4096
    a = _paged()
    assert lib.cp_paged_attn_merged(C.byref(a), None, None) == _lib.CPATTN_EINVAL
    b = _paged(stripe_begin=1, stripe_count=3)
    assert lib.cp_paged_attn_merged(C.byref(b), C.byref(m), None) == _lib.CPATTN_EINVAL
    assert "resident stripes" in _err(lib)
    m.out_dtype = 5
    assert lib.cp_paged_attn_merged(C.byref(a), C.byref(m), None) == _lib.CPATTN_EINVAL
    m.out_dtype, m.out = 1, 4104                                 # not 16-byte aligned
    assert lib.cp_paged_attn_merged(C.byref(a), C.byref(m), None) == _lib.CPATTN_EINVAL
    m.out, m.out_stride_head = 4096, 4                           # head stride not a multiple of 8
    assert lib.cp_paged_attn_merged(C.byref(a), C.byref(m), None) == _lib.CPATTN_EINVAL
    m.out_stride_head, m.out = 128, 16                           # the partial buffer itself
    assert lib.cp_paged_attn_merged(C.byref(a), C.byref(m), None) == _lib.CPATTN_EINVAL
    assert "alias" in _err(lib)


def test_version(lib):
    assert re.match(rb"^\d+\.\d+\.\d+$", lib.cpattn_version())


def _err(lib):
    return lib.cpattn_last_error().decode()


def test_slot_map_refusals(lib):
    assert lib.cp_slot_map(None, 4, 16, 3, 1, None, None, None) == _lib.CPATTN_EINVAL
    assert "divide" in _err(lib)
    assert lib.cp_slot_map(None, 4, 16, 0, 1, None, None, None) == _lib.CPATTN_EINVAL
    assert lib.cp_slot_map(None, -1, 16, 4, 1, None, None, None) == _lib.CPATTN_EINVAL
    assert lib.cp_slot_map(None, 4, 16, 4, 1, None, None, None) == _lib.CPATTN_EINVAL   # null pointers
    assert lib.cp_slot_map(None, 0, 16, 4, 1, None, None, None) == _lib.CPATTN_OK      # nothing to do
    assert lib.cp_slot_map(None, 0, 16, 4, 0, None, None, None) == _lib.CPATTN_EINVAL  # interleave < 1
    assert lib.cp_slot_map(None, 0, 16, 4, 8, None, None, None) == _lib.CPATTN_EINVAL  # I * P does not divide 16
    assert "interleave" in _err(lib)
    assert lib.cp_slot_map(None, 0, 16, 4, 4, None, None, None) == _lib.CPATTN_OK      # I * P = 16
    assert lib.cp_slot_map_rank(None, 4, 16, 4, 1, 4, 0, None, None) == _lib.CPATTN_EINVAL
    assert lib.cp_slot_map_rank(None, 4, 16, 4, 1, 1, -2, None, None) == _lib.CPATTN_EINVAL
    assert lib.cp_slot_map_rank(None, 0, 16, 2, 3, 1, 0, None, None) == _lib.CPATTN_EINVAL   # I * P = 6


def _paged(**kw):
    a = _lib.PagedArgs()
    base = dict(kind=0, dtype=1, num_rows=2, num_tokens=2, num_partners=4, stripe_begin=0, stripe_count=4,
                page_size=16, num_pages=10, num_q_heads=32, num_kv_heads=8, head_dim=128, head_dim_v=128, scale=0.1,
                max_ctx_len=100, max_row_tokens=1, max_pages=8, bt_stride=8, q_row_start=8, ctx_len=8,
                block_table=8, q=16, k_pool=16, v_pool=16, out=16, lse=16)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("bad,code", [
    (dict(num_partners=3), _lib.CPATTN_EINVAL),
    (dict(num_q_heads=30), _lib.CPATTN_EINVAL),
    (dict(stripe_begin=2, stripe_count=3), _lib.CPATTN_EINVAL),
    (dict(num_pages=0), _lib.CPATTN_EINVAL),
    (dict(bt_stride=4), _lib.CPATTN_EINVAL),
    (dict(kind=5), _lib.CPATTN_EINVAL),
    (dict(dtype=9), _lib.CPATTN_EINVAL),
    (dict(head_dim=96, head_dim_v=96), _lib.CPATTN_EUNSUPPORTED),
    (dict(head_dim=128, head_dim_v=64), _lib.CPATTN_EUNSUPPORTED),
    (dict(kind=1, num_kv_heads=8), _lib.CPATTN_EINVAL),
    (dict(kind=1, num_kv_heads=1, head_dim=576, head_dim_v=512, v_pool=32), _lib.CPATTN_EINVAL),
    (dict(kind=1, num_kv_heads=1, head_dim=512, head_dim_v=512), _lib.CPATTN_EUNSUPPORTED),
    (dict(q=0), _lib.CPATTN_EINVAL),
    (dict(num_rows=-1), _lib.CPATTN_EINVAL),
    (dict(kv_stride_page=-8), _lib.CPATTN_EINVAL),
    (dict(flags=4), _lib.CPATTN_EINVAL),
    (dict(flags=-1), _lib.CPATTN_EINVAL),
    (dict(interleave=-1), _lib.CPATTN_EINVAL),
    (dict(interleave=8), _lib.CPATTN_EINVAL),          # I * P = 32 does not divide page_size 16
    (dict(kv_format=2), _lib.CPATTN_EINVAL),
    (dict(kv_format=1, k_descale=0.5, v_descale=0.0), _lib.CPATTN_EINVAL),
    (dict(kv_format=1, k_descale=float("inf"), v_descale=0.5), _lib.CPATTN_EINVAL),
    (dict(kv_format=1, dtype=0, k_descale=0.5, v_descale=0.5), _lib.CPATTN_EINVAL),   # fp8 pools need bf16 queries
    (dict(kv_format=1, kind=1, num_kv_heads=1, head_dim=576, head_dim_v=512, k_descale=0.5, v_descale=0.25),
     _lib.CPATTN_EINVAL),                              # MLA latent rows carry one descale
])
def test_paged_refusals(lib, bad, code):
    a = _paged(**bad)
    assert lib.cp_paged_attn_partial(C.byref(a), None) == code
    assert _err(lib)
    assert lib.cp_paged_attn_partial_noalloc(C.byref(a), None) == code
    n = C.c_int64(-1)
    # the workspace-size query looks at shapes only, not at pointers
    assert lib.cp_paged_attn_workspace_size(C.byref(a), C.byref(n)) == (_lib.CPATTN_OK if "q" in bad else code)


def test_mla_over_fp8_passes_host_checks(lib):
    """MLA over an fp8 latent pool with one descale is accepted; the MFMA MLA kernel reads it, with a workspace for its
    split records."""
    a = _paged(kv_format=1, kind=1, num_kv_heads=1, num_q_heads=128, head_dim=576, head_dim_v=512, k_descale=0.5,
               v_descale=0.5)
    n = C.c_int64(-1)
    assert lib.cp_paged_attn_workspace_size(C.byref(a), C.byref(n)) == _lib.CPATTN_OK
    assert n.value > 0


def test_paged_null_args(lib):
    assert lib.cp_paged_attn_partial(None, None) == _lib.CPATTN_EINVAL
    assert lib.cp_paged_attn_partial_noalloc(None, None) == _lib.CPATTN_EINVAL
    assert lib.cp_paged_attn_noalloc_scratch_bytes() == 64 << 20


def test_paged_workspace_size_is_host_only(lib):
    # bf16 D=128 decode with split chunks needs a workspace; fp32 (generic path) needs none
    a = _paged(max_ctx_len=8192, kv_stride_slot=128, kv_stride_head=512, kv_stride_page=4096, kv_stride_stripe=40960,
               q_stride_token=4096, q_stride_head=128, out_stride_stripe=8192, out_stride_token=4096,
               out_stride_head=128, lse_stride_stripe=64, lse_stride_token=32)
    n = C.c_int64(-1)
    assert lib.cp_paged_attn_workspace_size(C.byref(a), C.byref(n)) == _lib.CPATTN_OK
    assert n.value > 0
    # too small a workspace is refused before any launch
    assert lib.cp_paged_attn_partial(C.byref(a), None) == _lib.CPATTN_EINVAL
    assert "workspace" in _err(lib)
    b = _paged(dtype=0)
    assert lib.cp_paged_attn_workspace_size(C.byref(b), C.byref(n)) == _lib.CPATTN_OK and n.value == 0
    # fixed splits: chunks of 64 steps (1024 keys) of a stripe; 4096 context tokens over 4 stripes fit one chunk
    f = _paged(flags=_lib.CPATTN_FLAG_FIXED_SPLITS, max_ctx_len=4096, kv_stride_slot=128, kv_stride_head=512,
               kv_stride_page=4096, kv_stride_stripe=40960, q_stride_token=4096, q_stride_head=128,
               out_stride_stripe=8192, out_stride_token=4096, out_stride_head=128, lse_stride_stripe=64,
               lse_stride_token=32)
    assert lib.cp_paged_attn_workspace_size(C.byref(f), C.byref(n)) == _lib.CPATTN_OK and n.value == 0
    f.max_ctx_len = 4 * 16 * 64 + 1          # one stripe now needs a second chunk
    assert lib.cp_paged_attn_workspace_size(C.byref(f), C.byref(n)) == _lib.CPATTN_OK and n.value > 0


def test_extend_workspace_holds_the_plan(lib):
    """bf16 rows with more than 16 query rows per kv head run the extend kernel, whose plan (one int32 per (row, stripe,
    query block of 128 rows) triple, ranked longest stripe first) lives in the workspace, rounded up to 256 bytes; past
    8192 triples the units run in grid order and need none."""
    strides = dict(kv_stride_slot=128, kv_stride_head=512, kv_stride_page=4096, kv_stride_stripe=40960,
                   q_stride_token=4096, q_stride_head=128, out_stride_stripe=8192, out_stride_token=4096,
                   out_stride_head=128, lse_stride_stripe=64, lse_stride_token=32)
    n = C.c_int64(-1)
    for kw, want in [(dict(max_row_tokens=40, num_tokens=80), 256),                      # 2 rows x 4 stripes x 2 blocks
                     (dict(max_row_tokens=40, num_tokens=80, kv_format=1, k_descale=0.5, v_descale=0.5), 256),
                     (dict(num_rows=1024, max_row_tokens=64, num_tokens=1024), 4 * 8192),  # 8192 triples
                     (dict(num_rows=1024, max_row_tokens=65, num_tokens=1024), 0),         # 12288: grid order
                     (dict(num_rows=1, stripe_count=1, max_row_tokens=20, num_tokens=20), 0)]:  # one triple
        a = _paged(**strides, **kw)
        assert lib.cp_paged_attn_workspace_size(C.byref(a), C.byref(n)) == _lib.CPATTN_OK, _err(lib)
        assert n.value == want, (kw, n.value)


def test_own_token_refusals(lib):
    a = _lib.OwnArgs()
    a.dtype, a.num_rows, a.bucket_tokens, a.num_q_heads, a.num_kv_heads, a.head_dim = 1, 2, 16, 32, 8, 96
    assert lib.cp_own_token_attn(C.byref(a), None) == _lib.CPATTN_EUNSUPPORTED
    a.head_dim, a.num_q_heads = 128, 30
    assert lib.cp_own_token_attn(C.byref(a), None) == _lib.CPATTN_EINVAL
    a.num_q_heads = 32
    assert lib.cp_own_token_attn(C.byref(a), None) == _lib.CPATTN_EINVAL       # null pointers
    a.flags = 4
    assert lib.cp_own_token_attn(C.byref(a), None) == _lib.CPATTN_EINVAL       # unknown flag bits
    assert "flags" in _err(lib)
    a.flags = 0
    a.bucket_tokens = 0
    assert lib.cp_own_token_attn(C.byref(a), None) == _lib.CPATTN_OK
    assert lib.cp_own_token_attn(None, None) == _lib.CPATTN_EINVAL


def test_merge_refusals(lib):
    a = _lib.MergeArgs()
    a.num_partials, a.num_tokens, a.num_heads, a.head_dim_v = 0, 4, 2, 8
    assert lib.cp_lse_merge(C.byref(a), None) == _lib.CPATTN_EINVAL
    a.num_partials = 18
    assert lib.cp_lse_merge(C.byref(a), None) == _lib.CPATTN_EINVAL
    a.num_partials, a.head_dim_v = 2, 6
    assert lib.cp_lse_merge(C.byref(a), None) == _lib.CPATTN_EINVAL
    a.head_dim_v, a.out = 8, 64
    a.part_out[0], a.part_lse[0] = 64, 128
    a.part_out[1], a.part_lse[1] = 256, 512
    assert lib.cp_lse_merge(C.byref(a), None) == _lib.CPATTN_EINVAL           # out aliases partial 0
    assert "alias" in _err(lib)
    a.out_dtype = 7
    assert lib.cp_lse_merge(C.byref(a), None) == _lib.CPATTN_EINVAL
    assert lib.cp_lse_merge(None, None) == _lib.CPATTN_EINVAL


def test_kv_write_refusals(lib):
    args = [None, 4, None, None, 0, 0, 1, 8, 128, 128, None, None, 0, 0, 0, 0, 16, 4, 1, 10, 0, 4, -1, None]
    bad = list(args)
    bad[17] = 3                                                               # P does not divide page_size
    assert lib.cp_kv_write(*bad) == _lib.CPATTN_EINVAL
    bad = list(args)
    bad[18] = 8                                                               # I * P does not divide page_size
    assert lib.cp_kv_write(*bad) == _lib.CPATTN_EINVAL
    bad = list(args)
    bad[18] = 0                                                               # interleave < 1
    assert lib.cp_kv_write(*bad) == _lib.CPATTN_EINVAL
    bad = list(args)
    bad[21] = 5                                                               # stripe range past P
    assert lib.cp_kv_write(*bad) == _lib.CPATTN_EINVAL
    bad = list(args)
    bad[22] = 10 * 4                                                          # sink outside the pool
    assert lib.cp_kv_write(*bad) == _lib.CPATTN_EINVAL
    assert lib.cp_kv_write(*args) == _lib.CPATTN_EINVAL                      # null pointers
    bad = list(args)
    bad[1] = 0
    assert lib.cp_kv_write(*bad) == _lib.CPATTN_OK


def test_debug_gather_refusals(lib):
    n = C.c_int32(-1)
    g = lib.cp_debug_gather_stripe
    assert g(None, 1, 0, 0, 0, 0, 4, None, 10, 16, 4, 1, 4, 1, 8, None, 99, C.byref(n), None) == _lib.CPATTN_EINVAL
    assert g(None, 1, 0, 0, 0, 0, 4, None, 10, 16, 3, 1, 0, 1, 8, None, 99, C.byref(n), None) == _lib.CPATTN_EINVAL
    assert g(None, 1, 0, 0, 0, 0, 4, None, 10, 16, 4, 8, 0, 1, 8, None, 99, C.byref(n), None) == _lib.CPATTN_EINVAL
    assert g(None, 1, 0, 0, 0, 0, 4, None, 0, 16, 4, 1, 1, 1, 8, None, 0, C.byref(n), None) == _lib.CPATTN_OK
    assert n.value == 0
    # stripe 1 of a 10-token row at P = 4 holds positions 1, 5, 9: a destination of two rows is refused
    assert g(None, 1, 0, 0, 0, 0, 4, None, 10, 16, 4, 1, 1, 1, 8, None, 2, C.byref(n), None) == _lib.CPATTN_EINVAL
    assert "room" in _err(lib)
    assert g(None, 1, 0, 0, 0, 0, 4, None, 10, 16, 4, 1, 1, 1, 8, None, 3, None, None) == _lib.CPATTN_EINVAL


def test_stripe_length_matches_the_oracle(lib):
    """cp_stripe_length (the function every kernel uses) against the oracle's count of the positions a stripe holds,
    for plain and interleaved placements."""
    import oracle
    n = C.c_int32(-1)
    for P, I, ps in [(1, 1, 16), (2, 1, 16), (4, 1, 16), (8, 1, 16), (16, 1, 16), (4, 2, 16), (4, 4, 16), (2, 8, 16),
                     (4, 16, 64), (3, 2, 12)]:
        for L in list(range(0, 70)) + [255, 1031, 4096, 8193]:
            for r in range(P):
                assert lib.cp_stripe_length(L, ps, P, I, r, C.byref(n)) == _lib.CPATTN_OK
                assert n.value == oracle.stripe_len(L, P, r, I), (P, I, L, r)
    assert lib.cp_stripe_length(10, 16, 3, 1, 0, C.byref(n)) == _lib.CPATTN_EINVAL      # P does not divide 16
    assert lib.cp_stripe_length(10, 16, 4, 1, 4, C.byref(n)) == _lib.CPATTN_EINVAL      # r outside [0, P)
    assert lib.cp_stripe_length(-1, 16, 4, 1, 0, C.byref(n)) == _lib.CPATTN_EINVAL
    assert lib.cp_stripe_length(10, 16, 4, 1, 0, None) == _lib.CPATTN_EINVAL


def test_stream_read_host_checks(lib):
    """The streaming-read reference kernel refuses what it cannot read; an empty buffer is a no-op."""
    assert lib.cp_debug_stream_read(None, 0, None, 1, None) == _lib.CPATTN_OK
    assert lib.cp_debug_stream_read(None, -16, None, 1, None) == _lib.CPATTN_EINVAL
    assert lib.cp_debug_stream_read(None, 24, None, 1, None) == _lib.CPATTN_EINVAL
    assert lib.cp_debug_stream_read(None, 32, None, 0, None) == _lib.CPATTN_EINVAL
    assert lib.cp_debug_stream_read(None, 32, None, 1, None) == _lib.CPATTN_EINVAL
    assert lib.cp_debug_stream_read(C.c_void_p(8), 32, C.c_void_p(64), 1, None) == _lib.CPATTN_EINVAL  # misaligned


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """With no built library the binding raises at load time: there is no non-HIP fallback."""
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libcpattn.so"))
    with pytest.raises(ImportError, match="not built"):
        _lib.load()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with a message (before touching a device)."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


# ------------------------------------------------------------------ binding checks (before any library call)
# The binding checks shapes and dtypes before it hands pointers to the library, so a mismatched tensor never reaches a
# kernel. CPU tensors serve here: with consistent shapes the binding gets as far as its device check.
def _gqa_tensors(dt=None):
    import torch
    dt = dt or torch.bfloat16
    P, pages, pp, hkv, D, T, Hq, B = 4, 6, 4, 2, 128, 3, 8, 2
    return dict(
        q=torch.zeros(T, Hq, D, dtype=dt), k_pool=torch.zeros(P, pages, pp, hkv, D, dtype=dt),
        v_pool=torch.zeros(P, pages, pp, hkv, D, dtype=dt), q_row_start=torch.tensor([0, 1, 3], dtype=torch.int32),
        ctx_len=torch.tensor([5, 9], dtype=torch.int32), block_table=torch.zeros(B, 3, dtype=torch.int32))


def _partial(**over):
    from cp_slot_map_amd import api
    t = _gqa_tensors()
    t.update(over)
    return api.paged_attn_partial(t["q"], t["k_pool"], t["v_pool"], t["q_row_start"], t["ctx_len"],
                                  t["block_table"], page_size=16, partners=4, scale=0.1, max_ctx_len=9,
                                  max_row_tokens=2, out=over.get("out"), lse=over.get("lse"))


def test_binding_partial_checks():
    import torch
    with pytest.raises(ValueError, match="GPU"):
        _partial()                                                  # consistent shapes reach the device check
    with pytest.raises(ValueError, match="head dim"):
        _partial(q=torch.zeros(3, 8, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="B \\+ 1"):
        _partial(q_row_start=torch.tensor([0, 1], dtype=torch.int32))
    with pytest.raises(ValueError, match="block_table"):
        _partial(block_table=torch.zeros(1, 3, dtype=torch.int32))
    with pytest.raises(ValueError, match="out must be"):
        _partial(out=torch.zeros(4, 3, 8, 64), lse=torch.zeros(4, 3, 8))
    with pytest.raises(ValueError, match="lse must be"):
        _partial(out=torch.zeros(4, 3, 8, 128), lse=torch.zeros(4, 3, 7))
    with pytest.raises(ValueError, match="out must be"):
        _partial(out=torch.zeros(4, 3, 8, 128, dtype=torch.bfloat16), lse=torch.zeros(4, 3, 8))
    with pytest.raises(TypeError):
        _partial(q=torch.zeros(3, 8, 128, dtype=torch.float32))     # q and pools differ
    with pytest.raises(TypeError):
        _partial(ctx_len=torch.tensor([5, 9], dtype=torch.int64))
    with pytest.raises(ValueError, match="stripes"):
        _partial(k_pool=torch.zeros(2, 6, 4, 2, 128, dtype=torch.bfloat16),
                 v_pool=torch.zeros(2, 6, 4, 2, 128, dtype=torch.bfloat16))


def test_binding_kv_write_checks():
    import torch
    from cp_slot_map_amd import api
    t = _gqa_tensors()
    s = torch.arange(5, dtype=torch.int64)
    k = torch.zeros(5, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        api.kv_write(s, k, k, t["k_pool"], t["v_pool"], 16, 4)
    fp8 = torch.zeros(4, 6, 4, 2, 128, dtype=torch.float8_e4m3fn)
    with pytest.raises(TypeError, match="dtype"):
        api.kv_write(s, k, k, fp8, fp8, 16, 4)                      # bf16 rows into an fp8 pool
    with pytest.raises(ValueError, match="heads"):
        api.kv_write(s, torch.zeros(5, 4, 128, dtype=torch.bfloat16), None, t["k_pool"], None, 16, 4)
    with pytest.raises(ValueError, match="rows"):
        api.kv_write(s[:4], k, k, t["k_pool"], t["v_pool"], 16, 4)
    with pytest.raises(ValueError, match="value pool"):
        api.kv_write(s, k, torch.zeros(5, 2, 64, dtype=torch.bfloat16), t["k_pool"], t["v_pool"], 16, 4)
    lat = torch.zeros(4, 6, 16, 576, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="latent"):
        api.kv_write(s, torch.zeros(5, 512, dtype=torch.bfloat16), None, lat, None, 64, 4, kind="mla")


def test_binding_merge_checks():
    import torch
    from cp_slot_map_amd import api
    outs = [torch.zeros(3, 4, 8) for _ in range(2)]
    lses = [torch.zeros(3, 4) for _ in range(2)]
    with pytest.raises(ValueError, match="GPU"):
        api.lse_merge(outs, lses)
    with pytest.raises(ValueError, match="out must be"):
        api.lse_merge(outs, lses, out=torch.zeros(3, 4, 4))
    with pytest.raises(ValueError, match="lse_out"):
        api.lse_merge(outs, lses, lse_out=torch.zeros(4, 3).t())    # heads not contiguous
    with pytest.raises(ValueError, match="lses must be"):
        api.lse_merge(outs, [lses[0], torch.zeros(3, 5)])
    with pytest.raises(TypeError):
        api.lse_merge(outs, lses, token_count=torch.zeros(1, dtype=torch.int64))


def test_binding_own_token_checks():
    import torch
    from cp_slot_map_amd import api
    q = torch.zeros(6, 8, 128, dtype=torch.bfloat16)
    k = torch.zeros(6, 2, 128, dtype=torch.bfloat16)
    cu = torch.tensor([0, 2, 5], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        api.own_token_attn(q, k, k, cu, scale=0.1)
    with pytest.raises(ValueError, match="must be"):
        api.own_token_attn(q, torch.zeros(5, 2, 128, dtype=torch.bfloat16), k, cu, scale=0.1)
    with pytest.raises(ValueError, match="out must be"):
        api.own_token_attn(q, k, k, cu, scale=0.1, out=torch.zeros(6, 8, 64))
    with pytest.raises(ValueError, match="cu_seqlens"):
        api.own_token_attn(q, k, k, cu, scale=0.1, num_rows=3)
    with pytest.raises(TypeError):
        api.own_token_attn(q, k.float(), k, cu, scale=0.1)
