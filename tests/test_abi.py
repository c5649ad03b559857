"""C-ABI checks that need no GPU: the library loads, exports every function
include/fa.h declares, and rejects bad arguments before touching the device.

Every call below carries exactly one defect, so validation returns before any
HIP call; the fake addresses are never dereferenced. No call here has valid
arguments (that would launch a kernel).
"""

import ctypes

import pytest

from exact_attention_120_amd import _lib

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_WORKSPACE, FA_ERR_HIP = (
    0, -1, -2, -3, -4, -5)
FA_ERR_SCRATCH = -6

# Distinct, 256-byte aligned fake addresses far apart (never dereferenced).
Q, K, V, O, LSE, DO, DQ, DK, DV, WS = (0x10_0000_0000 + i * 0x1_0000_0000 for i in range(10))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_functions_are_exported(lib):
    names = _lib.header_functions()
    assert set(names) == {"fa_fwd", "fa_bwd", "fa_fwd_ex", "fa_bwd_ex", "fa_bwd_workspace_size",
                          "fa_fwd_keysplit", "fa_fwd_num_splits",
                          "fa_fwd_splitkv_workspace_size", "fa_fwd_splitkv",
                          "fa_fwd_fp8", "fa_fwd_sparse", "fa_bwd_sparse", "fa_bwd_noalloc",
                          "fa_strerror"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_strerror(lib):
    for st in (FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_WORKSPACE,
               FA_ERR_HIP, FA_ERR_SCRATCH):
        assert lib.fa_strerror(st) and lib.fa_strerror(st) != b"unknown status"
    assert lib.fa_strerror(12345) == b"unknown status"


def fwd(lib, q=Q, k=K, v=V, o=O, lse=LSE, B=1, H=2, N=16, d=64, scale=0.125, causal=0,
        dtype=2):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, None)


FWD_CASES = [
    (dict(q=None), FA_ERR_INVALID_ARG),
    (dict(lse=None), FA_ERR_INVALID_ARG),
    (dict(B=0), FA_ERR_INVALID_ARG),
    (dict(H=-1), FA_ERR_INVALID_ARG),
    (dict(N=0), FA_ERR_INVALID_ARG),
    (dict(dtype=7), FA_ERR_INVALID_ARG),
    (dict(causal=2), FA_ERR_INVALID_ARG),
    (dict(scale=-0.5), FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), FA_ERR_INVALID_ARG),
    (dict(d=32), FA_ERR_UNSUPPORTED),
    (dict(d=96), FA_ERR_UNSUPPORTED),
    (dict(N=1 << 24, d=128), FA_ERR_UNSUPPORTED),          # N*d >= 2^31
    (dict(B=1 << 12, H=1 << 12, N=1 << 16), FA_ERR_UNSUPPORTED),  # total >= 2^40
    (dict(q=Q + 8), FA_ERR_ALIGN),
    (dict(o=O + 2), FA_ERR_ALIGN),
    (dict(lse=LSE + 4), FA_ERR_ALIGN),
    (dict(o=Q), FA_ERR_INVALID_ARG),                        # output aliases input
    (dict(o=K + 1024), FA_ERR_INVALID_ARG),                 # output overlaps input
    (dict(lse=V + 16), FA_ERR_INVALID_ARG),
    (dict(lse=O + 256), FA_ERR_INVALID_ARG),                # lse overlaps o
]


@pytest.mark.parametrize("kw,status", FWD_CASES)
def test_fwd_rejects(lib, kw, status):
    assert fwd(lib, **kw) == status


def test_workspace_size(lib):
    B, H, N, d = 2, 3, 100, 64
    rows = B * H * N
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert lib.fa_bwd_workspace_size(B, H, N, d) == up(rows * 4) + up(2 * rows * d * 4)
    assert lib.fa_bwd_workspace_size(0, H, N, d) == 0
    assert lib.fa_bwd_workspace_size(B, H, N, 80) == 0


def bwd(lib, q=Q, k=K, v=V, o=O, do=DO, lse=LSE, dq=DQ, dk=DK, dv=DV, B=1, H=2, N=16, d=64,
        scale=0.125, causal=1, dtype=1, ws=WS, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_size(B, H, N, d) if d in (64, 128) else 1 << 20
    return lib.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, ws,
                      ws_bytes, None)


BWD_CASES = [
    (dict(do=None), FA_ERR_INVALID_ARG),
    (dict(ws=None), FA_ERR_INVALID_ARG),
    (dict(N=0), FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), FA_ERR_INVALID_ARG),
    (dict(d=256), FA_ERR_UNSUPPORTED),
    (dict(dk=DK + 4), FA_ERR_ALIGN),
    (dict(ws=WS + 16), FA_ERR_ALIGN),                       # workspace needs 256 B
    (dict(ws_bytes=1024), FA_ERR_WORKSPACE),
    (dict(dq=Q), FA_ERR_INVALID_ARG),
    (dict(dv=DK), FA_ERR_INVALID_ARG),                      # two outputs alias
    (dict(ws=DO), FA_ERR_INVALID_ARG),                      # workspace overlaps an input
]


@pytest.mark.parametrize("kw,status", BWD_CASES)
def test_bwd_rejects(lib, kw, status):
    assert bwd(lib, **kw) == status


def bwd_noalloc(lib, q=Q, k=K, v=V, o=O, do=DO, lse=LSE, dq=DQ, dk=DK, dv=DV, B=1, H=2, N=16,
                d=64, scale=0.125, causal=1, dtype=1):
    return lib.fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype,
                              None)


SCRATCH = 64 << 20
BWD_NOALLOC_CASES = [
    (dict(do=None), FA_ERR_INVALID_ARG),
    (dict(dq=None), FA_ERR_INVALID_ARG),
    (dict(N=0), FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), FA_ERR_INVALID_ARG),
    (dict(d=96), FA_ERR_UNSUPPORTED),
    (dict(dk=DK + 4), FA_ERR_ALIGN),
    (dict(dq=Q), FA_ERR_INVALID_ARG),
    (dict(dv=DK), FA_ERR_INVALID_ARG),
    # Too large for the static scratch: D alone (16-bit) or D + the float32
    # dQ accumulator (FA_F32) exceeds 64 MiB. (Sizes are valid otherwise.)
    (dict(B=64, H=64, N=4097, d=64), FA_ERR_SCRATCH),                # 4*B*H*N > 64 MiB
    (dict(B=1, H=2, N=65536, d=128, dtype=0), FA_ERR_SCRATCH),       # fp32: 4*rows*(d+1)
    # ... and a defect earlier in the validation order still wins.
    (dict(B=64, H=64, N=4097, d=64, q=Q + 8), FA_ERR_ALIGN),
]


@pytest.mark.parametrize("kw,status", BWD_NOALLOC_CASES)
def test_bwd_noalloc_rejects(lib, kw, status):
    assert bwd_noalloc(lib, **kw) == status


def test_bwd_noalloc_limit_is_the_scratch_size(lib):
    # 16-bit: 4*B*H*N bytes may be at most 64 MiB, i.e. 2^24 rows; one row
    # group past that is rejected before anything is enqueued. (No call
    # here is valid: a valid one would launch.)
    rows = SCRATCH // 4
    assert bwd_noalloc(lib, B=1, H=256, N=rows // 256 + 1, d=64) == FA_ERR_SCRATCH
    assert bwd_noalloc(lib, B=1, H=256, N=rows // 256, d=64, dk=DK + 2) == FA_ERR_ALIGN


def test_signatures_match_header_argument_counts():
    import re
    text = open(_lib.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    for name, (_, args) in _lib.SIGNATURES.items():
        m = re.search(name + r"\s*\(([^)]*)\)", text)
        assert m, name
        n_params = len([p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"])
        assert n_params == len(args), name


def test_library_is_native_shared_object():
    with open(_lib.LIB_PATH, "rb") as f:
        assert f.read(4) == b"\x7fELF"
    assert isinstance(_lib.load(), ctypes.CDLL)


def fwd_ex(lib, kv_heads=0, wl=-1, wr=-1, opts=True, q=Q, k=K, v=V, o=O, lse=LSE, B=1, H=4,
           N=16, d=64, causal=0, dtype=2):
    op = ctypes.byref(_lib.FaOptions(kv_heads, wl, wr)) if opts else None
    return lib.fa_fwd_ex(q, k, v, o, lse, B, H, N, d, 0.125, causal, dtype, op, None)


def bwd_ex(lib, kv_heads=0, wl=-1, wr=-1, q=Q, k=K, v=V, o=O, dq=DQ, dk=DK, B=1, H=4, N=16,
           d=64, causal=1, dtype=1):
    op = ctypes.byref(_lib.FaOptions(kv_heads, wl, wr))
    ws = lib.fa_bwd_workspace_size(B, H, N, d)
    return lib.fa_bwd_ex(q, k, v, o, DO, LSE, dq, dk, DV, B, H, N, d, 0.125, causal, dtype, op,
                         WS, ws, None)


KV_BYTES_1 = 1 * 1 * 16 * 64 * 2  # one K/V head of the calls above (bf16)

FWD_EX_CASES = [
    (dict(kv_heads=-1), FA_ERR_INVALID_ARG),
    (dict(kv_heads=3), FA_ERR_INVALID_ARG),                 # does not divide H=4
    (dict(kv_heads=8), FA_ERR_INVALID_ARG),                 # more K/V heads than query heads
    (dict(kv_heads=2, q=None), FA_ERR_INVALID_ARG),
    (dict(kv_heads=2, d=80), FA_ERR_UNSUPPORTED),
    (dict(kv_heads=2, causal=3), FA_ERR_INVALID_ARG),
    (dict(wl=5, k=K + 8), FA_ERR_ALIGN),
    # With one K/V head, k spans KV_BYTES_1 bytes: an output starting inside
    # it overlaps, one starting right past it would not.
    (dict(kv_heads=1, o=K + KV_BYTES_1 - 256), FA_ERR_INVALID_ARG),
    (dict(kv_heads=1, lse=V + KV_BYTES_1 - 256), FA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,status", FWD_EX_CASES)
def test_fwd_ex_rejects(lib, kw, status):
    assert fwd_ex(lib, **kw) == status


def fwd_keysplit(lib, kv_heads=0, wl=-1, wr=-1, opts=True, q=Q, k=K, v=V, o=O, lse=LSE, B=1,
                 H=4, N=16, d=64, causal=0, dtype=2):
    op = ctypes.byref(_lib.FaOptions(kv_heads, wl, wr)) if opts else None
    return lib.fa_fwd_keysplit(q, k, v, o, lse, B, H, N, d, 0.125, causal, dtype, op, None)


# fa_fwd_keysplit validates as fa_fwd_ex does, and has no float32 kernel.
FWD_KEYSPLIT_CASES = FWD_EX_CASES + [
    (dict(dtype=0), FA_ERR_UNSUPPORTED),
    (dict(dtype=0, opts=False), FA_ERR_UNSUPPORTED),
    (dict(dtype=0, q=None), FA_ERR_INVALID_ARG),            # argument errors come first
    (dict(dtype=0, d=96), FA_ERR_UNSUPPORTED),
    (dict(dtype=5), FA_ERR_INVALID_ARG),
    (dict(opts=False, o=Q), FA_ERR_INVALID_ARG),
    (dict(N=1 << 24, d=128), FA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,status", FWD_KEYSPLIT_CASES)
def test_fwd_keysplit_rejects(lib, kw, status):
    assert fwd_keysplit(lib, **kw) == status


BWD_EX_CASES = [
    (dict(kv_heads=-2), FA_ERR_INVALID_ARG),
    (dict(kv_heads=3), FA_ERR_INVALID_ARG),
    (dict(kv_heads=2, wl=4, d=32), FA_ERR_UNSUPPORTED),
    (dict(kv_heads=2, dk=DK + 2), FA_ERR_ALIGN),
    (dict(kv_heads=1, dk=K + KV_BYTES_1 - 256), FA_ERR_INVALID_ARG),  # dk overlaps k
    (dict(kv_heads=2, dq=O), FA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,status", BWD_EX_CASES)
def test_bwd_ex_rejects(lib, kw, status):
    assert bwd_ex(lib, **kw) == status


INT_MAX = 2 ** 31 - 1


@pytest.mark.parametrize("wl,wr", [(INT_MAX, 0), (0, INT_MAX), (INT_MAX, INT_MAX),
                                   (15, 15), (1 << 30, -5)])
def test_any_int_window_bound_is_accepted(lib, wl, wr):
    # A bound of N - 1 or more is the unbounded side; every int is valid, so
    # the single defect (a misaligned q) is still the one reported.
    assert fwd_ex(lib, wl=wl, wr=wr, q=Q + 8) == FA_ERR_ALIGN
    assert bwd_ex(lib, wl=wl, wr=wr, dq=DQ + 2) == FA_ERR_ALIGN
    assert bwd_ex(lib, wl=wl, wr=wr, kv_heads=3) == FA_ERR_INVALID_ARG


def test_binding_window_bounds_must_fit_int32():
    import exact_attention_120_amd as fa
    op = fa._options(4, (INT_MAX, None))
    assert (op.kv_heads, op.window_left, op.window_right) == (4, INT_MAX, -1)
    op = fa._options(4, (-7, 3))
    assert (op.window_left, op.window_right) == (-1, 3)
    for window in ((INT_MAX + 1, 0), (0, 2 ** 32 + 5), (2 ** 40, 2 ** 40)):
        with pytest.raises(ValueError):
            fa._options(4, window)


def test_ex_with_null_options_validates_like_plain(lib):
    # NULL options = plain attention; the same single defects are rejected.
    assert fwd_ex(lib, opts=False, q=None) == FA_ERR_INVALID_ARG
    assert fwd_ex(lib, opts=False, d=96) == FA_ERR_UNSUPPORTED
    assert fwd_ex(lib, opts=False, o=O + 2) == FA_ERR_ALIGN


def test_num_splits_choice(lib):
    # B=2, H=8, N=1024, bf16: 2*8*4 = 64 workgroups of 256 rows -> 4 slices
    # of the 16 key tiles give 256 workgroups.
    assert lib.fa_fwd_num_splits(2, 8, 1024, 64, 2) == 4
    # Enough workgroups already: no split.
    assert lib.fa_fwd_num_splits(1, 16, 16384, 128, 2) == 1
    assert lib.fa_fwd_num_splits(4, 16, 4096, 128, 2) == 1
    # Too few key tiles to split (N=128: two tiles).
    assert lib.fa_fwd_num_splits(1, 1, 128, 64, 0) == 1
    # One head, N=4096 (64 key tiles, 16 query tiles): 16 slices.
    assert lib.fa_fwd_num_splits(1, 1, 4096, 128, 1) == 16
    # Invalid arguments.
    assert lib.fa_fwd_num_splits(0, 1, 128, 64, 2) == 0
    assert lib.fa_fwd_num_splits(1, 1, 128, 80, 2) == 0
    assert lib.fa_fwd_num_splits(1, 1, 128, 64, 9) == 0


def test_splitkv_workspace_size(lib):
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    B, H, N, d = 2, 8, 1024, 64
    for s in (2, 3, 64):
        rows = s * B * H * N
        assert lib.fa_fwd_splitkv_workspace_size(B, H, N, d, 2, s) == up(rows * d * 4) + up(rows * 4)
    # 0 = the library's count (4 here).
    assert (lib.fa_fwd_splitkv_workspace_size(B, H, N, d, 2, 0)
            == lib.fa_fwd_splitkv_workspace_size(B, H, N, d, 2, 4))
    assert lib.fa_fwd_splitkv_workspace_size(B, H, N, d, 2, 1) == 0
    assert lib.fa_fwd_splitkv_workspace_size(1, 16, 16384, 128, 2, 0) == 0
    assert lib.fa_fwd_splitkv_workspace_size(B, H, N, d, 2, 65) == 0
    assert lib.fa_fwd_splitkv_workspace_size(B, H, N, d, 2, -1) == 0


def splitkv(lib, num_splits=4, ws=WS, ws_bytes=None, kv_heads=0, q=Q, o=O, lse=LSE, B=2, H=8,
            N=1024, d=64, dtype=2):
    if ws_bytes is None:
        ws_bytes = lib.fa_fwd_splitkv_workspace_size(B, H, N, d, dtype, num_splits)
    op = ctypes.byref(_lib.FaOptions(kv_heads, -1, -1))
    return lib.fa_fwd_splitkv(q, K, V, o, lse, B, H, N, d, 0.125, 1, dtype, op, num_splits, ws,
                              ws_bytes, None)


SPLITKV_CASES = [
    (dict(num_splits=-1), FA_ERR_INVALID_ARG),
    (dict(num_splits=65), FA_ERR_INVALID_ARG),
    (dict(ws=None), FA_ERR_WORKSPACE),
    (dict(ws_bytes=4096), FA_ERR_WORKSPACE),
    (dict(num_splits=0, ws_bytes=4096), FA_ERR_WORKSPACE),  # 0 -> 4 slices need space
    (dict(ws=WS + 64), FA_ERR_ALIGN),
    (dict(ws=Q), FA_ERR_INVALID_ARG),                       # workspace overlaps q
    (dict(ws=O + 512), FA_ERR_INVALID_ARG),                 # workspace overlaps o
    (dict(kv_heads=3), FA_ERR_INVALID_ARG),
    (dict(q=None), FA_ERR_INVALID_ARG),
    (dict(d=32), FA_ERR_UNSUPPORTED),
    (dict(lse=LSE + 4), FA_ERR_ALIGN),
]


@pytest.mark.parametrize("kw,status", SPLITKV_CASES)
def test_splitkv_rejects(lib, kw, status):
    assert splitkv(lib, **kw) == status


def fwd_fp8(lib, q=Q, k=K, v=V, o=O, lse=LSE, B=1, H=4, N=16, d=64, scale=0.125, causal=0,
            dq=0.01, dk=0.02, dv=0.5, out_dtype=2, kv_heads=0, opts=True):
    op = ctypes.byref(_lib.FaOptions(kv_heads, -1, -1)) if opts else None
    return lib.fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, causal, dq, dk, dv, out_dtype, op,
                          None)


QB_FP8 = 1 * 4 * 16 * 64  # bytes of q (one byte per code) in the calls above

FWD_FP8_CASES = [
    (dict(q=None), FA_ERR_INVALID_ARG),
    (dict(v=None), FA_ERR_INVALID_ARG),
    (dict(out_dtype=0), FA_ERR_UNSUPPORTED),   # float32 output is not offered
    (dict(out_dtype=3), FA_ERR_INVALID_ARG),
    (dict(out_dtype=-1), FA_ERR_INVALID_ARG),
    (dict(dq=0.0), FA_ERR_INVALID_ARG),
    (dict(dk=-1.0), FA_ERR_INVALID_ARG),
    (dict(dv=float("nan")), FA_ERR_INVALID_ARG),
    (dict(dv=float("inf")), FA_ERR_INVALID_ARG),
    (dict(scale=3e38, dq=1e10, dk=1e10), FA_ERR_INVALID_ARG),  # score scale overflows
    (dict(scale=-1.0), FA_ERR_INVALID_ARG),
    (dict(causal=5), FA_ERR_INVALID_ARG),
    (dict(d=256), FA_ERR_UNSUPPORTED),
    (dict(B=0), FA_ERR_INVALID_ARG),
    (dict(kv_heads=3), FA_ERR_INVALID_ARG),
    (dict(q=Q + 8), FA_ERR_ALIGN),
    (dict(o=O + 2), FA_ERR_ALIGN),
    # q spans QB_FP8 bytes (1-byte codes): an output starting inside it overlaps.
    (dict(o=Q + QB_FP8 - 256), FA_ERR_INVALID_ARG),
    (dict(lse=Q + QB_FP8 - 16), FA_ERR_INVALID_ARG),
    (dict(lse=O + 256), FA_ERR_INVALID_ARG),   # lse inside o (bf16: twice q's bytes)
    (dict(opts=False, d=32), FA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,status", FWD_FP8_CASES)
def test_fwd_fp8_rejects(lib, kw, status):
    assert fwd_fp8(lib, **kw) == status



MASK = 0x10_0000_0000 + 10 * 0x1_0000_0000  # fake block-mask address (never dereferenced)


def fwd_sparse(lib, mask=MASK, q=Q, o=O, lse=LSE, B=1, H=4, N=16, d=64, causal=0, dtype=2,
               kv_heads=0, opts=True):
    op = ctypes.byref(_lib.FaOptions(kv_heads, -1, -1)) if opts else None
    return lib.fa_fwd_sparse(q, K, V, o, lse, B, H, N, d, 0.125, causal, dtype, op, mask, None)


def bwd_sparse(lib, mask=MASK, dq=DQ, dk=DK, ws=WS, B=1, H=4, N=16, d=64, causal=0, dtype=1,
               kv_heads=0):
    op = ctypes.byref(_lib.FaOptions(kv_heads, -1, -1))
    wsb = lib.fa_bwd_workspace_size(B, H, N, d)
    return lib.fa_bwd_sparse(Q, K, V, O, DO, LSE, dq, dk, DV, B, H, N, d, 0.125, causal, dtype,
                             op, mask, ws, wsb, None)


FWD_SPARSE_CASES = [
    (dict(mask=None), FA_ERR_INVALID_ARG),
    (dict(q=None), FA_ERR_INVALID_ARG),
    (dict(dtype=0), FA_ERR_UNSUPPORTED),          # float32 is not offered
    (dict(dtype=7), FA_ERR_INVALID_ARG),
    (dict(N=65537), FA_ERR_UNSUPPORTED),          # 1025 mask blocks
    (dict(d=96), FA_ERR_UNSUPPORTED),
    (dict(kv_heads=3), FA_ERR_INVALID_ARG),
    (dict(o=O + 8), FA_ERR_ALIGN),
    (dict(mask=O + 4096), FA_ERR_INVALID_ARG),    # the mask inside o
    (dict(mask=LSE + 16), FA_ERR_INVALID_ARG),    # the mask inside lse
    (dict(mask=O - 1, N=100), FA_ERR_INVALID_ARG),  # 2x2 blocks: its last 3 bytes are in o
]


@pytest.mark.parametrize("kw,status", FWD_SPARSE_CASES)
def test_fwd_sparse_rejects(lib, kw, status):
    assert fwd_sparse(lib, **kw) == status


def test_fwd_sparse_mask_extent_is_nmb_squared_bytes(lib):
    # N = 16384: 256 x 256 blocks, 65536 bytes. A mask starting 65535 bytes
    # before lse reaches into it; one 2^16 bytes before would not (not called:
    # that would launch).
    assert fwd_sparse(lib, mask=LSE - 65535, N=16384) == FA_ERR_INVALID_ARG


BWD_SPARSE_CASES = [
    (dict(mask=None), FA_ERR_INVALID_ARG),
    (dict(dtype=0), FA_ERR_UNSUPPORTED),
    (dict(N=70000), FA_ERR_UNSUPPORTED),
    (dict(kv_heads=3), FA_ERR_INVALID_ARG),
    (dict(dk=DK + 4), FA_ERR_ALIGN),
    (dict(mask=DQ + 256), FA_ERR_INVALID_ARG),    # inside dq
    (dict(mask=DK), FA_ERR_INVALID_ARG),          # at dk
    (dict(mask=WS + 100), FA_ERR_INVALID_ARG),    # inside the workspace
    (dict(ws=WS + 1), FA_ERR_ALIGN),
]


@pytest.mark.parametrize("kw,status", BWD_SPARSE_CASES)
def test_bwd_sparse_rejects(lib, kw, status):
    assert bwd_sparse(lib, **kw) == status


def test_missing_library_fails_loudly():
    """No CPU or PyTorch fallback sits behind the binding: without a built
    library loading raises, and CPU tensors are refused before any call."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, FA_LIBRARY="/nonexistent/libfa_missing.so")
    load = subprocess.run([sys.executable, "-c", "import exact_attention_120_amd as fa; fa._lib.load()"],
                          cwd=root, env=env, capture_output=True, text=True, timeout=300)
    assert load.returncode != 0
    assert "RuntimeError" in load.stderr and "no fallback" in load.stderr, load.stderr[-2000:]
    code = ("import torch, exact_attention_120_amd as fa\n"
            "q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)\n"
            "fa.fa_fwd(q, q, q, q.clone(), torch.zeros(1, 1, 64), 0.125, False)\n")
    cpu = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         timeout=300)
    assert cpu.returncode != 0
    assert "must be a GPU tensor" in cpu.stderr, cpu.stderr[-2000:]
