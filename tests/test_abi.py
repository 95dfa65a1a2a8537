"""The C-ABI library loads and exports every symbol include/mla_attn.h declares.

CPU only: every call below is rejected by the host-side checks (or is an empty
call), so nothing reaches the GPU. Calls that would pass the checks are never
made here.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_attn.h")

SC = 192.0 ** -0.5


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import attention_mla_causal_amd as m
    return m._lib


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted([
        "mla_attn_decode", "mla_attn_decode_workspace_bytes", "mla_attn_prefill", "mla_attn_decode_noalloc",
        "mla_attn_decode_latent", "mla_attn_decode_latent_workspace_bytes",
        "mla_attn_decode_varlen", "mla_attn_decode_varlen_workspace_bytes",
        "mla_attn_decode_paged", "mla_attn_decode_paged_workspace_bytes",
        "mla_attn_prefill_ws", "mla_attn_prefill_workspace_bytes",
        "mla_attn_prefill_varlen",
        "mla_attn_prefill_masked", "mla_attn_decode_masked",
        "mla_rope_table", "mla_rope_table_bytes", "mla_rope_apply", "mla_rope_apply_qk",
        "mla_attn_decode_rope", "mla_attn_decode_paged_rope", "mla_attn_decode_varlen_rope",
        "mla_last_error", "mla_status_string"])


def test_every_declared_symbol_is_exported(lib):
    import attention_mla_causal_amd as m
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert name in m.SIGNATURES, name


def test_status_strings(lib):
    import attention_mla_causal_amd as m
    for code, name in m.STATUS_NAMES.items():
        assert lib.mla_status_string(code).decode() == name
    assert lib.mla_status_string(99).decode() == "unknown status"


ALIGNED = ctypes.c_void_p(0x10000)    # never dereferenced: every call below fails its checks
MISALIGNED = ctypes.c_void_p(0x10002)


def _prefill(lib, ptrs, B, H, T, S, P, scale=SC):
    return lib.mla_attn_prefill(*ptrs, B, H, T, S, P, scale, None)


@pytest.mark.parametrize("B,H,T,S,P", [(1, 4, 16, 17, 0), (1, 4, 16, 20, 5), (-1, 4, 16, 16, 0),
                                       (1, 4, 16, 15, -1), (1, -2, 3, 3, 0),
                                       (1, 1, 1, 8388608, 8388607)])   # S beyond the prefill limit
def test_prefill_shape_errors(lib, B, H, T, S, P):
    assert _prefill(lib, [ALIGNED] * 6, B, H, T, S, P) == 2
    assert "mla_attn_prefill" in lib.mla_last_error().decode()


def test_prefill_null_align_scale_errors(lib):
    for i in range(6):
        ptrs = [ALIGNED] * 6
        ptrs[i] = None
        assert _prefill(lib, ptrs, 1, 2, 3, 3, 0) == 1
        ptrs[i] = MISALIGNED
        assert _prefill(lib, ptrs, 1, 2, 3, 3, 0) == 3
    for bad in (float("nan"), float("inf"), float("-inf"), 3.0e38, -3.0e38):
        assert _prefill(lib, [ALIGNED] * 6, 1, 2, 3, 3, 0, bad) == 4
    assert "softmax_scale" in lib.mla_last_error().decode()


def test_empty_calls_are_ok(lib):
    assert _prefill(lib, [None] * 6, 0, 4, 16, 16, 0) == 0
    assert _prefill(lib, [None] * 6, 1, 4, 0, 9, 9) == 0
    assert lib.mla_attn_decode(*([None] * 7), 0, 0, 64, 10, 9, SC, None) == 0


def test_decode_errors(lib):
    need = lib.mla_attn_decode_workspace_bytes(1, 64, 1001)
    assert need > 0 and need % 256 == 0
    assert lib.mla_attn_decode_workspace_bytes(32, 64, 8192) == 0
    assert lib.mla_attn_decode_workspace_bytes(-1, 64, 8192) == 0
    args = [ALIGNED] * 6
    assert lib.mla_attn_decode(*args, ALIGNED, need - 1, 1, 64, 1001, 1000, SC, None) == 5
    assert lib.mla_attn_decode(*args, None, need, 1, 64, 1001, 1000, SC, None) == 5
    assert lib.mla_attn_decode(*args, MISALIGNED, need, 1, 64, 1001, 1000, SC, None) == 3
    assert lib.mla_attn_decode(*args, ALIGNED, need, 1, 64, 1001, 999, SC, None) == 2
    assert lib.mla_attn_decode(*args, ALIGNED, need, 1, 64, 1001, 1000, float("nan"), None) == 4


def test_binding_has_no_fallback(tmp_path):
    import attention_mla_causal_amd as m
    with pytest.raises(ImportError):
        m.load_library(str(tmp_path / "missing.so"))


def _latent(lib, ptrs, ws, ws_bytes, B, H, S, P, scale=SC):
    return lib.mla_attn_decode_latent(*ptrs, ws, ws_bytes, B, H, S, P, scale, None)


def test_latent_decode_errors(lib):
    need = lib.mla_attn_decode_latent_workspace_bytes(1, 64, 1001)
    assert need > 0 and need % 256 == 0
    ok = [ALIGNED] * 6
    # shapes: S != past_len + 1, negative sizes, H above 64
    assert _latent(lib, ok, ALIGNED, need, 1, 64, 1001, 999) == 2
    assert _latent(lib, ok, ALIGNED, need, -1, 64, 1001, 1000) == 2
    assert _latent(lib, ok, ALIGNED, 1 << 40, 1, 64, 2097152, 2097151) == 2   # S beyond the limit
    assert "exceeds the latent decode limit" in lib.mla_last_error().decode()
    for H in (65, 80):
        ws = lib.mla_attn_decode_latent_workspace_bytes(1, H, 11)
        assert _latent(lib, ok, ALIGNED, ws, 1, H, 11, 10) == 2
    assert "at most 64 heads" in lib.mla_last_error().decode()
    for i in range(6):
        ptrs = list(ok)
        ptrs[i] = None
        assert _latent(lib, ptrs, ALIGNED, need, 1, 64, 1001, 1000) == 1
        ptrs[i] = MISALIGNED
        assert _latent(lib, ptrs, ALIGNED, need, 1, 64, 1001, 1000) == 3
    assert _latent(lib, ok, None, need, 1, 64, 1001, 1000) == 5
    assert _latent(lib, ok, ALIGNED, need - 1, 1, 64, 1001, 1000) == 5
    assert _latent(lib, ok, MISALIGNED, need, 1, 64, 1001, 1000) == 3
    assert _latent(lib, ok, ALIGNED, need, 1, 64, 1001, 1000, float("nan")) == 4
    assert "mla_attn_decode_latent" in lib.mla_last_error().decode()
    assert _latent(lib, [None] * 6, None, 0, 0, 64, 1001, 1000) == 0   # empty batch



def _varlen(lib, ptrs, ws, ws_bytes, B, H, L, M, scale=SC):
    # ptrs: q_nope, q_pe, k_nope_cache, k_pe_cache, v_cache, seq_lens, out
    return lib.mla_attn_decode_varlen(*ptrs, ws, ws_bytes, B, H, L, M, scale, None)


def test_varlen_decode_errors(lib):
    need = lib.mla_attn_decode_varlen_workspace_bytes(1, 64, 1001)
    assert need > 0 and need == lib.mla_attn_decode_workspace_bytes(1, 64, 1001)
    # B*H fills the chip, but long sequences still split into pieces of <= 1024
    # keys; from 2048 (b, h) pairs on, of <= 8192 keys
    assert lib.mla_attn_decode_workspace_bytes(16, 64, 8192) == 0
    assert lib.mla_attn_decode_varlen_workspace_bytes(16, 64, 8192) >= 16 * 64 * 8 * (128 + 4) * 4
    assert lib.mla_attn_decode_varlen_workspace_bytes(32, 64, 8192) == 0
    assert lib.mla_attn_decode_varlen_workspace_bytes(32, 64, 16384) >= 32 * 64 * 2 * (128 + 4) * 4
    assert lib.mla_attn_decode_varlen_workspace_bytes(32, 64, 1024) == 0
    ok = [ALIGNED] * 7
    assert _varlen(lib, ok, ALIGNED, need, 1, 64, 1000, 1001) == 2        # max_seq_len > cache
    assert "exceeds the cache length" in lib.mla_last_error().decode()
    assert _varlen(lib, ok, ALIGNED, need, -1, 64, 1001, 1001) == 2
    assert _varlen(lib, ok, ALIGNED, need, 1, 64, 1001, -1) == 2
    for i in range(7):
        ptrs = list(ok)
        ptrs[i] = None
        assert _varlen(lib, ptrs, ALIGNED, need, 1, 64, 2048, 1001) == 1
        ptrs[i] = MISALIGNED
        assert _varlen(lib, ptrs, ALIGNED, need, 1, 64, 2048, 1001) == 3
    # the length array needs only 4-byte alignment: such a call gets past the
    # alignment checks and stops at the missing workspace
    ptrs = list(ok)
    ptrs[5] = ctypes.c_void_p(0x10004)
    assert _varlen(lib, ptrs, None, need, 1, 64, 2048, 1001) == 5
    ptrs[5] = ctypes.c_void_p(0x10002)
    assert _varlen(lib, ptrs, None, need, 1, 64, 2048, 1001) == 3
    assert _varlen(lib, [None] * 7, None, 0, 0, 64, 2048, 1001) == 0      # empty batch: no-op
    assert _varlen(lib, ok, None, need, 1, 64, 2048, 1001) == 5
    assert _varlen(lib, ok, ALIGNED, need - 1, 1, 64, 2048, 1001) == 5
    assert _varlen(lib, ok, ALIGNED, need, 1, 64, 2048, 1001, float("nan")) == 4
    assert "mla_attn_decode_varlen" in lib.mla_last_error().decode()


def _paged(lib, ptrs, new, ws, ws_bytes, B, H, N, bs, M, L, scale=SC):
    # ptrs: q_nope, q_pe, k_nope_pages, k_pe_pages, v_pages, block_table, seq_lens; then out
    return lib.mla_attn_decode_paged(*ptrs, *new, ALIGNED, ws, ws_bytes, B, H, N, bs, M, L, scale, None)


def test_paged_decode_errors(lib):
    need = lib.mla_attn_decode_paged_workspace_bytes(4, 64, 4096)
    assert need == lib.mla_attn_decode_varlen_workspace_bytes(4, 64, 4096) and need > 0
    ok = [ALIGNED] * 7
    none3 = [None] * 3
    all3 = [ALIGNED] * 3
    # block_size must be a positive multiple of 32; lengths must fit the table
    for bs in (0, 16, 48):
        assert _paged(lib, ok, none3, ALIGNED, need, 4, 64, 100, bs, 64, 1024) == 2
    assert _paged(lib, ok, none3, ALIGNED, need, 4, 64, 100, 64, 63, 4096) == 2   # 63*64 < 4096
    assert _paged(lib, ok, none3, ALIGNED, need, 4, 64, 0, 64, 64, 4096) == 2     # no blocks
    assert _paged(lib, ok, none3, ALIGNED, need, -1, 64, 100, 64, 64, 4096) == 2
    # append needs all three new tensors
    assert _paged(lib, ok, [ALIGNED, None, None], ALIGNED, need, 4, 64, 100, 64, 64, 4096) == 1
    assert "append takes all" in lib.mla_last_error().decode()
    for i in range(7):
        ptrs = list(ok)
        ptrs[i] = None
        assert _paged(lib, ptrs, none3, ALIGNED, need, 4, 64, 100, 64, 64, 4096) == 1
        ptrs[i] = MISALIGNED
        assert _paged(lib, ptrs, none3, ALIGNED, need, 4, 64, 100, 64, 64, 4096) == 3
    for i in range(3):
        new = list(all3)
        new[i] = MISALIGNED
        assert _paged(lib, ok, new, ALIGNED, need, 4, 64, 100, 64, 64, 4096) == 3
    assert _paged(lib, ok, all3, None, need, 4, 64, 100, 64, 64, 4096) == 5
    assert _paged(lib, ok, all3, ALIGNED, need, 4, 64, 100, 64, 64, 4096, float("inf")) == 4
    assert _paged(lib, [None] * 7, none3, None, 0, 0, 64, 0, 0, 0, 0) == 0       # empty batch: no-op
    assert "mla_attn_decode_paged" in lib.mla_last_error().decode()


def test_prefill_ws_errors(lib):
    # a small grid (2 heads, 2 query tiles, 4096 keys) splits its keys; a full one does not
    need = lib.mla_attn_prefill_workspace_bytes(1, 2, 256, 4096)
    assert need >= 2 * 256 * 2 * 128 * 4
    assert lib.mla_attn_prefill_workspace_bytes(1, 64, 4096, 4096) == 0
    assert lib.mla_attn_prefill_workspace_bytes(1, 2, 256, 256) == 0       # too few keys to split
    ok = [ALIGNED] * 6

    def call(ptrs, ws, ws_bytes, B, H, T, S, P, scale=SC):
        return lib.mla_attn_prefill_ws(*ptrs, ws, ws_bytes, B, H, T, S, P, scale, None)

    assert call(ok, ALIGNED, need, 1, 2, 256, 4096, 3839) == 2             # S != past_len + T
    assert call(ok, None, need, 1, 2, 256, 4096, 3840) == 5
    assert call(ok, ALIGNED, need - 1, 1, 2, 256, 4096, 3840) == 5
    assert call(ok, MISALIGNED, need, 1, 2, 256, 4096, 3840) == 3
    assert call(ok, ALIGNED, need, 1, 2, 256, 4096, 3840, float("nan")) == 4
    for i in range(6):
        ptrs = list(ok)
        ptrs[i] = None
        assert call(ptrs, ALIGNED, need, 1, 2, 256, 4096, 3840) == 1
    assert "mla_attn_prefill_ws" in lib.mla_last_error().decode()
    assert call([None] * 6, None, 0, 0, 2, 256, 4096, 3840) == 0           # empty batch


def test_prefill_varlen_errors(lib):
    ok = [ALIGNED] * 8   # q_nope, q_pe, k_nope, k_pe, v, q_lens, past_lens, out

    def call(ptrs, B, H, Tmax, Smax, scale=SC):
        return lib.mla_attn_prefill_varlen(*ptrs, B, H, Tmax, Smax, scale, None)

    assert call(ok, 2, 64, 2049, 2048) == 2                 # a sequence's keys follow its cache
    assert "exceeds max_kv_len" in lib.mla_last_error().decode()
    assert call(ok, -1, 64, 16, 16) == 2
    assert call(ok, 1, 64, 16, 8388608) == 2                # past the 32-bit byte range of a slice
    for i in range(8):
        ptrs = list(ok)
        ptrs[i] = None
        assert call(ptrs, 2, 4, 16, 32) == 1
        ptrs[i] = MISALIGNED
        assert call(ptrs, 2, 4, 16, 32) == 3
    # the length arrays need only 4-byte alignment: the call then stops at the scale
    ptrs = list(ok)
    ptrs[5] = ptrs[6] = ctypes.c_void_p(0x10004)
    assert call(ptrs, 2, 4, 16, 32, float("nan")) == 4
    assert call(ok, 2, 4, 16, 32, float("-inf")) == 4
    assert "mla_attn_prefill_varlen" in lib.mla_last_error().decode()
    assert call([None] * 8, 2, 4, 0, 32) == 0               # no query rows: empty call
    assert call([None] * 8, 0, 4, 16, 32) == 0


def test_masked_errors(lib):
    ok = [ALIGNED] * 7   # q_nope, q_pe, k_nope, k_pe, v, attn_mask, out

    def pre(ptrs, B, H, T, S, P, scale=SC):
        return lib.mla_attn_prefill_masked(*ptrs, B, H, T, S, P, scale, None)

    def dec(ptrs, ws, ws_bytes, B, H, S, P, scale=SC):
        return lib.mla_attn_decode_masked(*ptrs, ws, ws_bytes, B, H, S, P, scale, None)

    assert pre(ok, 1, 4, 16, 20, 3) == 2                       # S != past_len + T
    mask_none = list(ok)
    mask_none[5] = None
    assert pre(mask_none, 1, 4, 16, 20, 4) == 1
    assert "attn_mask is NULL" in lib.mla_last_error().decode()
    odd = list(ok)
    odd[5] = ctypes.c_void_p(0x10003)                           # the mask needs no alignment: stops at the scale
    assert pre(odd, 1, 4, 16, 20, 4, float("inf")) == 4
    assert pre([None] * 7, 0, 4, 16, 20, 4) == 0               # empty call
    need = lib.mla_attn_decode_varlen_workspace_bytes(1, 64, 1001)
    assert dec(ok, ALIGNED, need, 1, 64, 1001, 999) == 2
    # the variable-length split plan: B*H fills the GPU, yet 8192 keys split in pieces
    big = lib.mla_attn_decode_varlen_workspace_bytes(16, 64, 8192)
    assert big > 0 and lib.mla_attn_decode_workspace_bytes(16, 64, 8192) == 0
    assert dec(ok, ALIGNED, big - 1, 16, 64, 8192, 8191) == 5
    assert dec(ok, MISALIGNED, big, 16, 64, 8192, 8191) == 3
    assert dec(mask_none, ALIGNED, need, 1, 64, 1001, 1000) == 1
    assert dec(ok, None, need, 1, 64, 1001, 1000) == 5
    assert dec(odd, ALIGNED, need, 1, 64, 1001, 1000, float("inf")) == 4
    assert "mla_attn_decode_masked" in lib.mla_last_error().decode()
    assert dec([None] * 7, None, 0, 1, 0, 1001, 1000) == 0


def test_rope_errors(lib):
    AL, MIS = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x100008)
    assert lib.mla_rope_table_bytes(4096) == 4096 * 256
    assert lib.mla_rope_table_bytes(0) == 0 and lib.mla_rope_table_bytes(-3) == 0
    assert lib.mla_rope_table(None, 0, 50000.0, 32.0, 4096, 1.0, 1.0, None) == 0      # empty
    assert lib.mla_rope_table(AL, -1, 50000.0, 32.0, 4096, 1.0, 1.0, None) == 2
    assert lib.mla_rope_table(AL, 16, 50000.0, float("nan"), 4096, 1.0, 1.0, None) == 4
    assert lib.mla_rope_table(None, 16, 50000.0, 32.0, 4096, 1.0, 1.0, None) == 1
    assert lib.mla_rope_table(MIS, 16, 50000.0, 32.0, 4096, 1.0, 1.0, None) == 3
    assert "mla_rope_table" in lib.mla_last_error().decode()
    assert lib.mla_rope_apply(AL, None, AL, 4096, 1, 64, 2048, 2049, None) == 2        # past the table
    assert "table" in lib.mla_last_error().decode()
    assert lib.mla_rope_apply(None, None, None, 0, 1, 64, 0, 0, None) == 0            # empty
    assert lib.mla_rope_apply(None, None, AL, 16, 1, 1, 1, 0, None) == 1
    assert lib.mla_rope_apply(MIS, None, AL, 16, 1, 1, 1, 0, None) == 3
    assert lib.mla_rope_apply(AL, ctypes.c_void_p(0x100002), AL, 16, 1, 1, 1, 0, None) == 3
    assert lib.mla_rope_apply_qk(AL, None, None, AL, 4096, 1, 64, 8, 0, None) == 1           # k_pe NULL
    assert lib.mla_rope_apply_qk(AL, MIS, None, AL, 4096, 1, 64, 8, 0, None) == 3
    assert lib.mla_rope_apply_qk(AL, AL, None, AL, 4096, 1, 64, 8, 4089, None) == 2         # past the table
    assert lib.mla_rope_apply_qk(None, None, None, None, 0, 1, 64, 0, 0, None) == 0         # T == 0: no-op
    assert lib.mla_rope_apply_qk(None, None, None, AL, 16, 1, 0, 8, 0, None) == 1           # H == 0: keys still turn
    assert "x is NULL" in lib.mla_last_error().decode()
    assert lib.mla_rope_apply_qk(None, MIS, None, AL, 16, 1, 0, 8, 0, None) == 3            # ... and are checked
    # fused prologue in decode: the table must cover the new token's position
    ok = [AL] * 5
    need = lib.mla_attn_decode_workspace_bytes(1, 64, 1001)
    assert lib.mla_attn_decode_rope(*ok, AL, 1000, AL, AL, need, 1, 64, 1001, 1000, SC, None) == 2
    assert "rope_max_pos" in lib.mla_last_error().decode()
    assert lib.mla_attn_decode_rope(*ok, None, 1001, AL, AL, need, 1, 64, 1001, 1000, SC, None) == 1
    assert lib.mla_attn_decode_rope(*ok, MIS, 1001, AL, AL, need, 1, 64, 1001, 1000, SC, None) == 3
    assert lib.mla_attn_decode_rope(*ok, None, 0, AL, AL, need, 1, 64, 1001, 999, SC, None) == 2  # shape first
    assert lib.mla_attn_decode_rope(*ok, None, 0, None, None, 0, 0, 64, 1001, 1000, SC, None) == 0  # empty
    vw = lib.mla_attn_decode_varlen_workspace_bytes(2, 8, 4096)
    assert lib.mla_attn_decode_varlen_rope(*ok, AL, None, 4096, AL, AL, vw, 2, 8, 4096, 4096, SC, None) == 1
    assert lib.mla_attn_decode_varlen_rope(*ok, AL, AL, 4000, AL, AL, vw, 2, 8, 4096, 4096, SC, None) == 2
    assert "mla_attn_decode_varlen_rope" in lib.mla_last_error().decode()
    pw = lib.mla_attn_decode_paged_workspace_bytes(2, 8, 4096)
    args = [AL, AL, AL, AL, AL, AL, AL, None, None, None]
    assert lib.mla_attn_decode_paged_rope(*args, None, 4096, AL, AL, pw, 2, 8, 64, 64, 64, 4096, SC, None) == 1
    assert lib.mla_attn_decode_paged_rope(*args, AL, 4095, AL, AL, pw, 2, 8, 64, 64, 64, 4096, SC, None) == 2
    assert "mla_attn_decode_paged_rope" in lib.mla_last_error().decode()


def test_product_path_never_touches_the_oracle():
    """The package (binding and HIP sources) names neither the oracle package
    nor any of its modules, and the oracle imports nothing from the package."""
    pkg = os.path.join(ROOT, "attention_mla_causal_amd")
    oracle_dir = os.path.join(ROOT, "oracle")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if not f.endswith((".py", ".hip", ".h", ".cpp")):
                continue
            text = open(os.path.join(dirpath, f), encoding="utf-8").read()
            assert not re.search(r"\b(from|import)\s+oracle\b", text), f
            assert not re.search(r"\boracle[./]", text), f
            assert "importlib" not in text or "oracle" not in text, f
    for f in os.listdir(oracle_dir):
        if f.endswith(".py"):
            text = open(os.path.join(oracle_dir, f), encoding="utf-8").read()
            assert not re.search(r"\b(from|import)\s+attention_mla_causal_amd\b", text), f
            assert "libmla_attn" not in text, f
