"""The C ABI library on a host without a GPU: it loads, exports what the
header declares, and rejects every bad argument before touching HIP."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_mi355x.h")


@pytest.fixture(scope="module")
def L():
    from io_aware_tiled_08_amd import binding, build
    if not os.path.exists(binding.library_path()):
        build.build_library()
    return binding.lib()


def _header():
    with open(HEADER) as f:
        return f.read()


def test_exports_every_declared_function(L):
    from io_aware_tiled_08_amd import binding
    declared = set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(flash_attn_\w+)\s*\(", _header(), re.M))
    assert declared == set(binding.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_abi_version_matches_header(L):
    m = re.search(r"#define\s+FA_MI355X_ABI_VERSION\s+(\d+)", _header())
    assert int(m.group(1)) == L.flash_attn_abi_version()


def test_status_codes_match_header(L):
    from io_aware_tiled_08_amd import binding
    enum = dict((name, int(val)) for name, val in
                re.findall(r"\b(FA_(?:OK|ERR_\w+))\s*=\s*(\d+)", _header()))
    assert enum == binding.STATUS_CODE
    texts = {L.flash_attn_status_str(c).decode() for c in enum.values()}
    assert len(texts) == len(enum)
    for name, code in enum.items():
        assert L.flash_attn_status_str(code).decode().startswith(name)
    assert L.flash_attn_status_str(999).decode() == "unknown fa_status"
    dt = dict(re.findall(r"\b(FA_(?:F32|F16|BF16))\s*=\s*(\d+)", _header()))
    assert {k: int(v) for k, v in dt.items()} == {
        "FA_F32": binding.FA_F32, "FA_F16": binding.FA_F16, "FA_BF16": binding.FA_BF16}


# Fake, 16-byte aligned, non-overlapping device addresses: every call below
# returns before anything could dereference them.
GiB = 1 << 30
Q, K, V, O, LSE = (0x10000000000 + i * 64 * GiB for i in range(5))


def _call(L, q=Q, k=K, v=V, o=O, lse=LSE, B=2, H=3, N=100, d=64, scale=0.125,
          causal=0, dtype=1):
    st = L.flash_attn_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, None)
    return st, L.flash_attn_last_error().decode()


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse"])
def test_null_pointer(L, field):
    st, msg = _call(L, **{field: None})
    assert st == 1 and "non-NULL" in msg


@pytest.mark.parametrize("shape", [(-1, 1, 1), (1, -2, 1), (1, 1, -3)])
def test_negative_shape(L, shape):
    B, H, N = shape
    assert _call(L, B=B, H=H, N=N)[0] == 2


def test_overflowing_shape(L):
    assert _call(L, B=1 << 40, H=1 << 20, N=1 << 10)[0] == 2


def test_grid_limit(L):
    # 2^31 query blocks cannot be launched on a 32-bit grid.
    assert _call(L, B=1 << 20, H=1 << 11, N=1 << 10)[0] == 2


@pytest.mark.parametrize("d", [0, 32, 96, 100, 256, -64])
def test_head_dim(L, d):
    assert _call(L, d=d)[0] == 3


@pytest.mark.parametrize("dtype", [-1, 3, 42])
def test_dtype(L, dtype):
    assert _call(L, dtype=dtype)[0] == 4


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse"])
def test_misaligned(L, field):
    base = {"q": Q, "k": K, "v": V, "o": O, "lse": LSE}[field]
    assert _call(L, **{field: base + 8})[0] == 5


@pytest.mark.parametrize("scale", [math.nan, math.inf, -math.inf])
def test_scale(L, scale):
    assert _call(L, scale=scale)[0] == 6


@pytest.mark.parametrize("o,lse", [(Q, LSE), (K + 4096, LSE), (O, V + 256), (O, O + 1024)])
def test_alias(L, o, lse):
    assert _call(L, o=o, lse=lse)[0] == 7


def test_inputs_may_alias_each_other(L):
    st, _ = _call(L, k=Q, v=Q)
    assert st != 7


@pytest.mark.parametrize("shape", [(0, 3, 100), (2, 0, 100), (2, 3, 0)])
def test_empty_is_a_no_op(L, shape):
    B, H, N = shape
    assert _call(L, B=B, H=H, N=N) == (0, "")
    assert _call(L, q=None, o=None, lse=None, B=B, H=H, N=N) == (0, "")
    assert _call(L, B=B, H=H, N=N, d=96)[0] == 3


def test_no_device_reported_not_crashed(L):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, msg = _call(L)
    assert st == 8, msg
    assert msg


def test_error_string_cleared_on_success(L):
    assert _call(L, d=96)[0] == 3
    assert L.flash_attn_last_error().decode() != ""
    assert _call(L, N=0) == (0, "")


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    from io_aware_tiled_08_amd import flash_attn_fwd
    x = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        flash_attn_fwd(x, x, x)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from io_aware_tiled_08_amd import binding
    monkeypatch.setenv("FA_MI355X_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        binding.lib()


# ---- flash_attn_fwd_kvcache: argument checks before any HIP call ----------
WS = 0x10000000000 + 5 * 64 * GiB


def _kv(L, q=Q, k=K, v=V, o=O, lse=LSE, B=2, H=3, Nq=4, Nk=1000, d=64, scale=0.125,
        causal=0, splits=0, ws=WS, ws_bytes=1 << 30, dtype=1):
    st = L.flash_attn_fwd_kvcache(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, splits,
                                  ws, ws_bytes, dtype, None)
    return st, L.flash_attn_last_error().decode()


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse"])
def test_kv_null_pointer(L, field):
    st, msg = _kv(L, **{field: None})
    assert st == 1 and "non-NULL" in msg


@pytest.mark.parametrize("shape", [(-1, 1, 1, 1), (1, -1, 1, 1), (1, 1, -1, 1), (1, 1, 1, -1)])
def test_kv_negative_shape(L, shape):
    B, H, Nq, Nk = shape
    assert _kv(L, B=B, H=H, Nq=Nq, Nk=Nk)[0] == 2


def test_kv_no_keys_and_short_causal_cache(L):
    st, msg = _kv(L, Nk=0)
    assert st == 2 and "no key" in msg
    st, msg = _kv(L, Nq=10, Nk=9, causal=1)
    assert st == 2 and "Nk >= Nq" in msg
    # non-causal queries may outnumber the keys
    assert _kv(L, Nq=10, Nk=9, causal=0)[0] not in (2,)


@pytest.mark.parametrize("dtype", [0, 3, -1])
def test_kv_dtype(L, dtype):
    st, msg = _kv(L, dtype=dtype)
    assert st == 4
    if dtype == 0:
        assert "FA_F16 or FA_BF16" in msg


@pytest.mark.parametrize("d", [0, 32, 96, 256])
def test_kv_head_dim(L, d):
    assert _kv(L, d=d)[0] == 3


@pytest.mark.parametrize("scale", [math.inf, -math.inf, math.nan])
def test_kv_scale(L, scale):
    assert _kv(L, scale=scale)[0] == 6


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse", "ws"])
def test_kv_misaligned(L, field):
    base = {"q": Q, "k": K, "v": V, "o": O, "lse": LSE, "ws": WS}[field]
    assert _kv(L, splits=4, **{field: base + 8})[0] == 5


def test_kv_empty_is_a_no_op(L):
    for B, H, Nq in [(0, 3, 4), (2, 0, 4), (2, 3, 0)]:
        assert _kv(L, B=B, H=H, Nq=Nq, q=None, o=None, lse=None, ws=None) == (0, "")


def test_kv_split_count_and_workspace_size(L):
    # one head, one query, 32768 keys: the library splits the keys
    S = L.flash_attn_kvcache_splits(1, 1, 1, 32768, 128, 0)
    assert 1 < S <= 256
    assert L.flash_attn_kvcache_workspace_size(1, 1, 1, 32768, 128, 0) == S * 1 * 1 * 129 * 4
    # a requested count is honoured up to the number of 32-key tiles
    assert L.flash_attn_kvcache_splits(1, 1, 1, 32768, 128, 7) == 7
    assert L.flash_attn_kvcache_splits(1, 1, 1, 100, 128, 50) == 4
    assert L.flash_attn_kvcache_splits(1, 1, 1, 100, 128, 1) == 1
    assert L.flash_attn_kvcache_workspace_size(1, 1, 1, 100, 128, 1) == 0
    # many heads already fill the GPU: no split
    assert L.flash_attn_kvcache_splits(64, 32, 64, 512, 128, 0) == 1
    # invalid sizes need nothing
    assert L.flash_attn_kvcache_workspace_size(0, 1, 1, 100, 64, 0) == 0
    assert L.flash_attn_kvcache_splits(1, 1, 1, 100, 96, 0) == 1
    # every tile of every split count lands in exactly one split
    for nk in (1, 31, 32, 33, 1000, 4097):
        for req in (1, 2, 3, 5, 64, 300):
            S = L.flash_attn_kvcache_splits(1, 1, 1, nk, 64, req)
            tiles = -(-nk // 32)
            assert 1 <= S <= min(tiles, 256)


def test_kv_workspace_missing_or_small(L):
    need = L.flash_attn_kvcache_workspace_size(2, 3, 4, 1000, 64, 4)
    assert need == 4 * 2 * 3 * 4 * 65 * 4
    st, msg = _kv(L, splits=4, ws=None)
    assert st == 11 and "workspace" in msg
    st, msg = _kv(L, splits=4, ws_bytes=need - 1)
    assert st == 11
    # one split needs no workspace at all
    st, msg = _kv(L, splits=1, ws=None, ws_bytes=0)
    assert st not in (11, 1), msg


def test_kv_alias(L):
    assert _kv(L, o=Q)[0] == 7
    assert _kv(L, lse=K + 64)[0] == 7
    assert _kv(L, splits=4, ws=O)[0] == 7
    assert _kv(L, splits=4, ws=LSE)[0] == 7


def test_kv_no_device_reported_not_crashed(L):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, msg = _kv(L, splits=4)
    assert st == 8, msg


def test_dispatch_thread_count_limit(L):
    # 2^20 heads x 8 blocks of 256 rows x 512 threads overflows the 32-bit
    # dispatch size although the workgroup count fits 31 bits.
    assert _call(L, B=1 << 20, H=1, N=2048)[0] == 2
    assert _call(L, B=1 << 20, H=1, N=1792)[0] != 2
    # cache path: 2^23 rows need 2^31 merge threads
    st, _ = _kv(L, B=1 << 23, H=1, Nq=1, Nk=4096, splits=2, ws_bytes=1 << 62)
    assert st == 2


# ---- flash_attn_fwd_fp8: argument checks before any HIP call -------------
def _f8(L, q=Q, k=K, v=V, o=O, lse=LSE, B=2, H=3, N=100, d=64, scale=0.125, causal=0,
        qs=0.01, ks=0.02, vs=0.03):
    st = L.flash_attn_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, causal, qs, ks, vs, None)
    return st, L.flash_attn_last_error().decode()


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse"])
def test_fp8_null_pointer(L, field):
    assert _f8(L, **{field: None})[0] == 1


@pytest.mark.parametrize("bad", [{"qs": 0.0}, {"ks": -1.0}, {"vs": math.inf}, {"qs": math.nan},
                                 {"scale": math.inf}])
def test_fp8_scale_and_descales(L, bad):
    assert _f8(L, **bad)[0] == 6


def test_fp8_shapes_head_dim_alignment_alias(L):
    assert _f8(L, B=-1)[0] == 2
    assert _f8(L, d=96)[0] == 3
    assert _f8(L, k=K + 4)[0] == 5
    assert _f8(L, o=V)[0] == 7
    assert _f8(L, B=0, q=None, o=None) == (0, "")
    assert _f8(L, B=1 << 20, H=1, N=2048)[0] == 2


def test_fp8_no_device_reported_not_crashed(L):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _f8(L)[0] == 8


# ---- persistent schedule -----------------------------------------------------
def _pers(L, q=Q, k=K, v=V, o=O, lse=LSE, B=2, H=3, N=100, d=64, scale=0.125, causal=0,
          nwg=0, dtype=1):
    st = L.flash_attn_fwd_persistent(q, k, v, o, lse, B, H, N, d, scale, causal, nwg, dtype, None)
    return st, L.flash_attn_last_error().decode()


def test_persistent_argument_checks_match_the_forward(L):
    """Same checks, same codes as flash_attn_fwd, before any HIP call."""
    for kw in ({"q": None}, {"lse": None}, {"B": -1}, {"d": 96}, {"dtype": 7}, {"v": V + 8},
               {"scale": math.nan}, {"o": K}, {"B": 1 << 40, "H": 1 << 20, "N": 1 << 10},
               {"B": 1 << 20, "H": 1 << 11, "N": 1 << 10}):
        assert _pers(L, **kw)[0] == _call(L, **kw)[0] != 0, kw


def test_persistent_rejects_fp32_and_negative_grid(L):
    st, msg = _pers(L, dtype=0)
    assert st == 4 and "fp16 and bf16" in msg
    st, msg = _pers(L, nwg=-1)
    assert st == 2 and "num_workgroups" in msg


def test_persistent_empty_is_a_no_op(L):
    assert _pers(L, N=0, q=None, o=None, lse=None) == (0, "")
    assert _pers(L, B=0, nwg=5) == (0, "")


def test_persistent_no_device_reported_not_crashed(L):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _pers(L)[0] == 8
    assert _pers(L, nwg=3, causal=1)[0] == 8


def test_bwd_workspace_size(L):
    """D and LSE * log2(e) per row: 8 bytes per (b, h, row)."""
    assert L.flash_attn_bwd_workspace_size(2, 3, 100) == 2 * 3 * 100 * 8
    assert L.flash_attn_bwd_workspace_size(0, 3, 100) == 0
    assert L.flash_attn_bwd_workspace_size(1 << 30, 1 << 20, 1 << 20) == -1


# ---- backward: workspace contract ---------------------------------------------
# Fake device addresses for the gradients, dO and the workspace, 64 GiB apart.
DQ, DK, DV, DO_, BWS = (0x10000000000 + i * 64 * GiB for i in range(6, 11))


def _bwd(L, ws=BWS, ws_bytes=None, dq=DQ, B=1, H=2, N=100, d=64, dtype=1):
    if ws_bytes is None:
        ws_bytes = L.flash_attn_bwd_workspace_size(B, H, N)
    st = L.flash_attn_bwd(Q, K, V, O, DO_, LSE, dq, DK, DV, B, H, N, d, 0.125, 0,
                          ws, ws_bytes, dtype, None)
    return st, L.flash_attn_last_error().decode()


def test_bwd_workspace_one_byte_short_is_rejected(L):
    """The prep kernel writes D and LSE * log2(e): 8 bytes per row, all required."""
    need = 1 * 2 * 100 * 8
    assert L.flash_attn_bwd_workspace_size(1, 2, 100) == need
    st, msg = _bwd(L, ws_bytes=need - 1)
    assert st == 11 and str(need) in msg
    st, _ = _bwd(L, ws_bytes=need // 2)  # the size of D alone
    assert st == 11


def test_bwd_workspace_of_the_full_size_reaches_the_device_check(L):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _bwd(L)[0] == 8


def test_bwd_workspace_second_half_overlapping_dq_is_an_alias(L):
    """dq starts inside the second half of the workspace (the LSE * log2(e) part)."""
    need = L.flash_attn_bwd_workspace_size(1, 2, 100)
    st, msg = _bwd(L, ws=DQ - need + 16)
    assert st == 7 and "overlap" in msg
    # Just past the end is fine (the device check is what stops it here).
    st, _ = _bwd(L, ws=DQ - need)
    assert st != 7


# ---- flash_attn_fwd_kvcache_noalloc: the same checks, the scratch limit -----

def _kvn(L, q=Q, k=K, v=V, o=O, lse=LSE, B=2, H=3, Nq=4, Nk=1000, d=64, scale=0.125,
         causal=0, splits=0, dtype=1):
    st = L.flash_attn_fwd_kvcache_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal,
                                          splits, dtype, None)
    return st, L.flash_attn_last_error().decode()


def test_noalloc_scratch_size_matches_the_header(L):
    m = re.search(r"#define\s+FA_MI355X_KVCACHE_SCRATCH_BYTES\s+\((\d+) \* (\d+) \* (\d+)\)",
                  _header())
    assert m and int(m.group(1)) * int(m.group(2)) * int(m.group(3)) == 16 << 20


def test_noalloc_argument_checks_match_the_workspace_entry_point(L):
    """Every argument error of flash_attn_fwd_kvcache (other than the
    workspace's own) comes back with the same code, before any HIP call."""
    for kw in ({"q": None}, {"lse": None}, {"B": -1}, {"Nk": -1}, {"d": 96}, {"dtype": 0},
               {"dtype": 7}, {"v": V + 8}, {"scale": math.nan}, {"o": K}, {"lse": K + 64},
               {"Nk": 0}, {"Nq": 10, "Nk": 9, "causal": 1}):
        assert _kvn(L, **kw)[0] == _kv(L, **kw)[0] != 0, kw
    assert _kvn(L, B=0, q=None, o=None, lse=None) == (0, "")


def test_noalloc_rejects_splits_beyond_the_scratch(L):
    """Two splits of one head at d=64 take 2 * Nq * 65 * 4 bytes: 32263 query
    rows fit 16 MiB, 32264 do not."""
    cap = 16 << 20
    assert L.flash_attn_kvcache_workspace_size(1, 1, 32263, 32768, 64, 2) <= cap
    assert L.flash_attn_kvcache_workspace_size(1, 1, 32264, 32768, 64, 2) > cap
    st, msg = _kvn(L, B=1, H=1, Nq=32264, Nk=32768, splits=2)
    assert st == 11 and "scratch" in msg and str(cap) in msg


def test_noalloc_no_device_reported_not_crashed(L):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _kvn(L, B=1, H=1, Nq=32263, Nk=32768, splits=2)[0] == 8
    assert _kvn(L, splits=1)[0] == 8
    assert _kvn(L)[0] == 8
