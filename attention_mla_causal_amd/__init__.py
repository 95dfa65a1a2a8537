"""Causal multi-head latent attention (MLA) core for AMD Instinct MI355X.

A thin ctypes binding over libmla_attn.so (the C ABI in include/mla_attn.h).
The functions below only check and marshal arguments: torch supplies device
memory and the current HIP stream; every step of the attention, and of the
rotary prologue (the YaRN table, the rotation of new rows, or the rotation
fused into the decode), runs in the library's HIP kernels. There is no fallback path: if the library has not been
built (``python attention_mla_causal_amd/build.py``) importing this package
raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_attn.so")

QK_NOPE_HEAD_DIM = 128
QK_ROPE_HEAD_DIM = 64
V_HEAD_DIM = 128

STATUS_NAMES = {
    0: "MLA_OK",
    1: "MLA_ERR_NULL",
    2: "MLA_ERR_SHAPE",
    3: "MLA_ERR_ALIGN",
    4: "MLA_ERR_SCALE",
    5: "MLA_ERR_WORKSPACE",
    6: "MLA_ERR_DEVICE",
}
MLA_ERR_SHAPE = 2

# Exported C symbols and their signatures (kept in step with include/mla_attn.h).
_VP, _I32, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "mla_attn_prefill": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _F32, _VP]),
    "mla_attn_prefill_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "mla_attn_prefill_ws": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _I32, _I32, _I32, _I32, _I32, _F32, _VP]),
    "mla_attn_prefill_varlen": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _F32, _VP]),
    "mla_attn_prefill_masked": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _F32, _VP]),
    "mla_attn_decode_masked": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _I32, _I32, _I32, _I32, _F32, _VP]),
    "mla_attn_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "mla_attn_decode": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _I32, _I32, _I32, _I32, _F32, _VP]),
    "mla_attn_decode_noalloc": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _F32, _VP]),
    "mla_attn_decode_varlen_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "mla_attn_decode_varlen": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _I32, _I32, _I32, _I32, _F32, _VP]),
    "mla_attn_decode_paged_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "mla_attn_decode_paged": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ,
                                             _I32, _I32, _I32, _I32, _I32, _I32, _F32, _VP]),
    "mla_attn_decode_latent_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "mla_attn_decode_latent": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _I32, _I32, _I32, _I32, _F32, _VP]),
    "mla_rope_table_bytes": (_SZ, [_I32]),
    "mla_rope_table": (ctypes.c_int, [_VP, _I32, ctypes.c_double, ctypes.c_double, _I32, ctypes.c_double,
                                      ctypes.c_double, _VP]),
    "mla_rope_apply": (ctypes.c_int, [_VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP]),
    "mla_rope_apply_qk": (ctypes.c_int, [_VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP]),
    "mla_attn_decode_rope": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _SZ, _I32, _I32, _I32,
                                            _I32, _F32, _VP]),
    "mla_attn_decode_varlen_rope": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _SZ, _I32,
                                                   _I32, _I32, _I32, _F32, _VP]),
    "mla_attn_decode_paged_rope": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32,
                                                  _VP, _VP, _SZ, _I32, _I32, _I32, _I32, _I32, _I32, _F32, _VP]),
    "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_last_error": (ctypes.c_char_p, []),
}


class MLAError(RuntimeError):
    """A non-shape failure reported by the library (status code attached)."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python attention_mla_causal_amd/build.py); there is no non-GPU fallback")
    try:
        import torch  # noqa: F401  (load torch's HIP runtime first so the library binds to it)
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = load_library()


def _raise_for(status: int, where: str):
    if status == 0:
        return
    detail = _lib.mla_last_error().decode(errors="replace")
    name = STATUS_NAMES.get(status, f"status {status}")
    msg = f"{where} failed with {name}: {detail}"
    if status == MLA_ERR_SHAPE:
        raise ValueError(msg)
    raise MLAError(status, msg)


def _check_tensor(t, name: str):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4D, got shape {tuple(t.shape)}")


def _stream_handle(device):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shapes(q_nope, q_pe, k_nope, k_pe, v):
    for t, n in ((q_nope, "q_nope"), (q_pe, "q_pe"), (k_nope, "k_nope"), (k_pe, "k_pe"), (v, "v")):
        _check_tensor(t, n)
    B, H, T, dn = q_nope.shape
    S = k_nope.shape[2]
    want = {
        "q_nope": (B, H, T, QK_NOPE_HEAD_DIM),
        "q_pe": (B, H, T, QK_ROPE_HEAD_DIM),
        "k_nope": (B, H, S, QK_NOPE_HEAD_DIM),
        "k_pe": (B, 1, S, QK_ROPE_HEAD_DIM),
        "v": (B, H, S, V_HEAD_DIM),
    }
    for t, n in ((q_nope, "q_nope"), (q_pe, "q_pe"), (k_nope, "k_nope"), (k_pe, "k_pe"), (v, "v")):
        if tuple(t.shape) != want[n]:
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {want[n]}")
    devs = {t.device for t in (q_nope, q_pe, k_nope, k_pe, v)}
    if len(devs) != 1:
        raise ValueError(f"inputs are on different devices: {devs}")
    return B, H, T, S


def mla_attn_prefill_workspace_bytes(B: int, H: int, T: int, S: int) -> int:
    """Bytes of device scratch the split prefill needs for (B, H, T, S) (0: none)."""
    return int(_lib.mla_attn_prefill_workspace_bytes(int(B), int(H), int(T), int(S)))


def mla_attn_prefill(q_nope, q_pe, k_nope, k_pe, v, past_len: int, softmax_scale: float, out=None,
                     workspace=None, split=True):
    """Causal MLA attention of T new queries over S = past_len + T keys.

    q_nope [B,H,T,128], q_pe [B,H,T,64], k_nope [B,H,S,128], k_pe [B,1,S,64]
    (one rotary key for all heads), v [B,H,S,128]; bf16, contiguous, on one
    GPU. Returns out [B,H,T,128] bf16, enqueued on the current stream.
    When the query tiles alone would leave the GPU part-empty and split is
    true, the keys are split over several workgroups (mla_attn_prefill_ws,
    with `workspace` or one allocated here); otherwise mla_attn_prefill.
    """
    import torch

    B, H, T, S = _shapes(q_nope, q_pe, k_nope, k_pe, v)
    if out is None:
        out = torch.empty((B, H, T, V_HEAD_DIM), dtype=torch.bfloat16, device=q_nope.device)
    else:
        _check_tensor(out, "out")
        if tuple(out.shape) != (B, H, T, V_HEAD_DIM) or out.device != q_nope.device:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, T, V_HEAD_DIM)}")
    need = mla_attn_prefill_workspace_bytes(B, H, T, S) if split else 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q_nope.device)
        if not (workspace.is_cuda and workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous GPU tensor")
        st = _lib.mla_attn_prefill_ws(
            q_nope.data_ptr(), q_pe.data_ptr(), k_nope.data_ptr(), k_pe.data_ptr(), v.data_ptr(),
            out.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            B, H, T, S, int(past_len), float(softmax_scale), _stream_handle(q_nope.device))
        _raise_for(st, "mla_attn_prefill_ws")
        return out
    st = _lib.mla_attn_prefill(
        q_nope.data_ptr(), q_pe.data_ptr(), k_nope.data_ptr(), k_pe.data_ptr(), v.data_ptr(),
        out.data_ptr(), B, H, T, S, int(past_len), float(softmax_scale), _stream_handle(q_nope.device))
    _raise_for(st, "mla_attn_prefill")
    return out


def mla_attn_prefill_varlen(q_nope, q_pe, k_nope, k_pe, v, q_lens, past_lens, softmax_scale: float,
                            out=None):
    """Causal MLA prefill of a right-padded batch with a length per sequence.

    q_nope [B,H,Tmax,128], q_pe [B,H,Tmax,64], k_nope [B,H,Smax,128],
    k_pe [B,1,Smax,64], v [B,H,Smax,128] bf16; q_lens and past_lens int32 GPU
    tensors [B]: sequence b has q_lens[b] new queries (rows [0, q_lens[b]))
    over past_lens[b] cached keys (its keys are rows [0, past_lens[b] +
    q_lens[b])). Both are clamped on the device (q_lens to [0, Tmax],
    past_lens to [0, Smax - q_lens]). Returns out [B,H,Tmax,128] bf16 with
    padded query rows set to 0.
    """
    import torch

    B, H, Tmax, Smax = _shapes(q_nope, q_pe, k_nope, k_pe, v)
    _check_int32(q_lens, "q_lens", (B,), q_nope.device)
    _check_int32(past_lens, "past_lens", (B,), q_nope.device)
    if out is None:
        out = torch.empty((B, H, Tmax, V_HEAD_DIM), dtype=torch.bfloat16, device=q_nope.device)
    else:
        _check_tensor(out, "out")
        if tuple(out.shape) != (B, H, Tmax, V_HEAD_DIM) or out.device != q_nope.device:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, Tmax, V_HEAD_DIM)}")
    st = _lib.mla_attn_prefill_varlen(
        q_nope.data_ptr(), q_pe.data_ptr(), k_nope.data_ptr(), k_pe.data_ptr(), v.data_ptr(),
        q_lens.data_ptr(), past_lens.data_ptr(), out.data_ptr(), B, H, Tmax, Smax,
        float(softmax_scale), _stream_handle(q_nope.device))
    _raise_for(st, "mla_attn_prefill_varlen")
    return out


def _check_mask(attn_mask, B, S, device):
    import torch
    if not (isinstance(attn_mask, torch.Tensor) and attn_mask.dtype in (torch.uint8, torch.bool)
            and attn_mask.is_cuda and attn_mask.is_contiguous() and tuple(attn_mask.shape) == (B, S)
            and attn_mask.device == device):
        raise ValueError(f"attn_mask must be a contiguous uint8 or bool tensor of shape {(B, S)} on {device}")


def mla_attn_prefill_masked(q_nope, q_pe, k_nope, k_pe, v, attn_mask, past_len: int,
                            softmax_scale: float, out=None):
    """mla_attn_prefill under the caller's 2D padding mask attn_mask [B, S]
    (uint8 or bool on the GPU, nonzero keeps key j of sequence b). Query i sees
    key j iff j <= past_len + i and the mask keeps j; a query with no visible
    key gives a zero row."""
    import torch

    B, H, T, S = _shapes(q_nope, q_pe, k_nope, k_pe, v)
    _check_mask(attn_mask, B, S, q_nope.device)
    if out is None:
        out = torch.empty((B, H, T, V_HEAD_DIM), dtype=torch.bfloat16, device=q_nope.device)
    else:
        _check_tensor(out, "out")
        if tuple(out.shape) != (B, H, T, V_HEAD_DIM) or out.device != q_nope.device:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, T, V_HEAD_DIM)}")
    st = _lib.mla_attn_prefill_masked(
        q_nope.data_ptr(), q_pe.data_ptr(), k_nope.data_ptr(), k_pe.data_ptr(), v.data_ptr(),
        attn_mask.data_ptr(), out.data_ptr(), B, H, T, S, int(past_len), float(softmax_scale),
        _stream_handle(q_nope.device))
    _raise_for(st, "mla_attn_prefill_masked")
    return out


def mla_attn_decode_masked(q_nope, q_pe, k_nope, k_pe, v, attn_mask, past_len: int,
                           softmax_scale: float, out=None, workspace=None):
    """mla_attn_decode under the caller's 2D padding mask attn_mask [B, S]
    (uint8 or bool on the GPU, nonzero keeps); a sequence with no visible key
    gives a zero row. workspace: at least
    mla_attn_decode_varlen_workspace_bytes(B, H, S) bytes (allocated here when
    omitted)."""
    import torch

    B, H, T, S = _shapes(q_nope, q_pe, k_nope, k_pe, v)
    if T != 1:
        raise ValueError(f"decode takes one query per sequence, got T={T}")
    _check_mask(attn_mask, B, S, q_nope.device)
    if out is None:
        out = torch.empty((B, H, 1, V_HEAD_DIM), dtype=torch.bfloat16, device=q_nope.device)
    else:
        _check_tensor(out, "out")
        if tuple(out.shape) != (B, H, 1, V_HEAD_DIM) or out.device != q_nope.device:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, 1, V_HEAD_DIM)}")
    need = mla_attn_decode_varlen_workspace_bytes(B, H, S)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_nope.device)
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    st = _lib.mla_attn_decode_masked(
        q_nope.data_ptr(), q_pe.data_ptr(), k_nope.data_ptr(), k_pe.data_ptr(), v.data_ptr(),
        attn_mask.data_ptr(), out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), B, H, S, int(past_len), float(softmax_scale),
        _stream_handle(q_nope.device))
    _raise_for(st, "mla_attn_decode_masked")
    return out


def mla_attn_decode_workspace_bytes(B: int, H: int, S: int) -> int:
    """Bytes of device scratch mla_attn_decode needs for (B, H, S) (0: none)."""
    return int(_lib.mla_attn_decode_workspace_bytes(int(B), int(H), int(S)))


def _check_rope_table(table, device):
    import torch
    if not (isinstance(table, torch.Tensor) and table.dtype == torch.float32 and table.is_contiguous()
            and table.dim() == 3 and tuple(table.shape[1:]) == (32, 2) and table.device == device):
        raise ValueError(f"rope_table must be a contiguous float32 [max_pos, 32, 2] tensor on {device}")


def mla_attn_decode(q_nope, q_pe, k_nope, k_pe, v, past_len: int, softmax_scale: float,
                    out=None, workspace=None, rope_table=None):
    """One new query per sequence (T = 1) against S = past_len + 1 keys.

    workspace: a GPU tensor of at least mla_attn_decode_workspace_bytes(B, H, S)
    bytes of scratch (contents irrelevant, reusable by non-overlapping calls);
    allocated here when omitted. rope_table (from mla_rope_table): q_pe is
    taken before rotation and turned at position past_len in the kernel
    (mla_attn_decode_rope).
    """
    import torch

    B, H, T, S = _shapes(q_nope, q_pe, k_nope, k_pe, v)
    if T != 1:
        raise ValueError(f"decode takes one query per sequence, got T={T}")
    if out is None:
        out = torch.empty((B, H, 1, V_HEAD_DIM), dtype=torch.bfloat16, device=q_nope.device)
    else:
        _check_tensor(out, "out")
        if tuple(out.shape) != (B, H, 1, V_HEAD_DIM) or out.device != q_nope.device:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, 1, V_HEAD_DIM)}")
    need = mla_attn_decode_workspace_bytes(B, H, S)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_nope.device)
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    if rope_table is not None:
        _check_rope_table(rope_table, q_nope.device)
        st = _lib.mla_attn_decode_rope(
            q_nope.data_ptr(), q_pe.data_ptr(), k_nope.data_ptr(), k_pe.data_ptr(), v.data_ptr(),
            rope_table.data_ptr(), int(rope_table.shape[0]), out.data_ptr(), workspace.data_ptr(),
            ws_bytes, B, H, S, int(past_len), float(softmax_scale), _stream_handle(q_nope.device))
        _raise_for(st, "mla_attn_decode_rope")
        return out
    st = _lib.mla_attn_decode(
        q_nope.data_ptr(), q_pe.data_ptr(), k_nope.data_ptr(), k_pe.data_ptr(), v.data_ptr(),
        out.data_ptr(), workspace.data_ptr(), ws_bytes, B, H, S, int(past_len),
        float(softmax_scale), _stream_handle(q_nope.device))
    _raise_for(st, "mla_attn_decode")
    return out


def mla_attn_decode_noalloc(q_nope, q_pe, k_nope, k_pe, v, past_len: int, softmax_scale: float, out=None):
    """mla_attn_decode without a workspace: the library keeps the split
    partials in its own per-device scratch array, so the C call allocates
    nothing (pass `out` to keep this wrapper from allocating it). Calls that
    may overlap on one device share that array and must be ordered."""
    import torch

    B, H, T, S = _shapes(q_nope, q_pe, k_nope, k_pe, v)
    if T != 1:
        raise ValueError(f"decode takes one query per sequence, got T={T}")
    if out is None:
        out = torch.empty((B, H, 1, V_HEAD_DIM), dtype=torch.bfloat16, device=q_nope.device)
    else:
        _check_tensor(out, "out")
        if tuple(out.shape) != (B, H, 1, V_HEAD_DIM) or out.device != q_nope.device:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, 1, V_HEAD_DIM)}")
    st = _lib.mla_attn_decode_noalloc(
        q_nope.data_ptr(), q_pe.data_ptr(), k_nope.data_ptr(), k_pe.data_ptr(), v.data_ptr(), out.data_ptr(),
        B, H, S, int(past_len), float(softmax_scale), _stream_handle(q_nope.device))
    _raise_for(st, "mla_attn_decode_noalloc")
    return out


def mla_attn_decode_varlen_workspace_bytes(B: int, H: int, max_seq_len: int) -> int:
    """Bytes of device scratch mla_attn_decode_varlen needs (0: none)."""
    return int(_lib.mla_attn_decode_varlen_workspace_bytes(int(B), int(H), int(max_seq_len)))


def mla_attn_decode_varlen(q_nope, q_pe, k_nope_cache, k_pe_cache, v_cache, seq_lens,
                           max_seq_len: int, softmax_scale: float, out=None, workspace=None,
                           rope_table=None):
    """Decode over a preallocated, right-padded cache with a length per sequence.

    q_nope [B,H,1,128], q_pe [B,H,1,64]; k_nope_cache [B,H,L,128], k_pe_cache
    [B,1,L,64], v_cache [B,H,L,128] with L the cache length; seq_lens an int32
    GPU tensor [B]: sequence b attends over cache rows [0, seq_lens[b]),
    each length clamped on the device to [0, max_seq_len] (max_seq_len <= L).
    A sequence of length 0 gives a zero row. rope_table (from mla_rope_table):
    q_pe is taken before rotation and turned at position seq_lens[b]-1 in the
    kernel (mla_attn_decode_varlen_rope). Returns out [B,H,1,128] bf16.
    """
    import torch

    B, H, T, L = _shapes(q_nope, q_pe, k_nope_cache, k_pe_cache, v_cache)
    if T != 1:
        raise ValueError(f"decode takes one query per sequence, got T={T}")
    if not (isinstance(seq_lens, torch.Tensor) and seq_lens.dtype == torch.int32 and seq_lens.is_cuda
            and seq_lens.is_contiguous() and tuple(seq_lens.shape) == (B,)
            and seq_lens.device == q_nope.device):
        raise ValueError(f"seq_lens must be a contiguous int32 tensor of shape ({B},) on {q_nope.device}")
    if out is None:
        out = torch.empty((B, H, 1, V_HEAD_DIM), dtype=torch.bfloat16, device=q_nope.device)
    else:
        _check_tensor(out, "out")
        if tuple(out.shape) != (B, H, 1, V_HEAD_DIM) or out.device != q_nope.device:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, 1, V_HEAD_DIM)}")
    need = mla_attn_decode_varlen_workspace_bytes(B, H, max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_nope.device)
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    if rope_table is not None:
        _check_rope_table(rope_table, q_nope.device)
        st = _lib.mla_attn_decode_varlen_rope(
            q_nope.data_ptr(), q_pe.data_ptr(), k_nope_cache.data_ptr(), k_pe_cache.data_ptr(),
            v_cache.data_ptr(), seq_lens.data_ptr(), rope_table.data_ptr(), int(rope_table.shape[0]),
            out.data_ptr(), workspace.data_ptr(), ws_bytes, B, H, L, int(max_seq_len), float(softmax_scale),
            _stream_handle(q_nope.device))
        _raise_for(st, "mla_attn_decode_varlen_rope")
        return out
    st = _lib.mla_attn_decode_varlen(
        q_nope.data_ptr(), q_pe.data_ptr(), k_nope_cache.data_ptr(), k_pe_cache.data_ptr(),
        v_cache.data_ptr(), seq_lens.data_ptr(), out.data_ptr(), workspace.data_ptr(), ws_bytes,
        B, H, L, int(max_seq_len), float(softmax_scale), _stream_handle(q_nope.device))
    _raise_for(st, "mla_attn_decode_varlen")
    return out


def mla_attn_decode_paged_workspace_bytes(B: int, H: int, max_seq_len: int) -> int:
    """Bytes of device scratch mla_attn_decode_paged needs (0: none)."""
    return int(_lib.mla_attn_decode_paged_workspace_bytes(int(B), int(H), int(max_seq_len)))


def _check_int32(t, name, shape, device):
    import torch
    if not (isinstance(t, torch.Tensor) and t.dtype == torch.int32 and t.is_cuda and t.is_contiguous()
            and tuple(t.shape) == tuple(shape) and t.device == device):
        raise ValueError(f"{name} must be a contiguous int32 tensor of shape {tuple(shape)} on {device}")


def mla_attn_decode_paged(q_nope, q_pe, k_nope_pages, k_pe_pages, v_pages, block_table, seq_lens,
                          max_seq_len: int, softmax_scale: float, new=None, out=None, workspace=None,
                          rope_table=None):
    """Decode over a paged cache, optionally appending the new token.

    k_nope_pages / v_pages [N, H, bs, 128], k_pe_pages [N, bs, 64] (bs a
    multiple of 32); block_table int32 [B, M]; seq_lens int32 [B] (keys after
    the call, clamped on the device to [0, max_seq_len]). new: None or
    (k_nope_new [B,H,1,128], k_pe_new [B,1,1,64], v_new [B,H,1,128]), attended
    to as key seq_lens[b]-1 and written into that slot of the pages.
    rope_table (from mla_rope_table): q_pe and k_pe_new are taken before
    rotation and turned at position seq_lens[b]-1 in the kernel, the new key
    stored rotated (mla_attn_decode_paged_rope).
    Returns out [B,H,1,128] bf16 on the current stream.
    """
    import torch

    for t, n in ((q_nope, "q_nope"), (q_pe, "q_pe"), (k_nope_pages, "k_nope_pages"), (v_pages, "v_pages")):
        _check_tensor(t, n)
    if not (isinstance(k_pe_pages, torch.Tensor) and k_pe_pages.dtype == torch.bfloat16 and k_pe_pages.is_cuda
            and k_pe_pages.is_contiguous() and k_pe_pages.dim() == 3):
        raise ValueError("k_pe_pages must be a contiguous 3D bfloat16 GPU tensor")
    B, H = q_nope.shape[0], q_nope.shape[1]
    N, bs = k_pe_pages.shape[0], k_pe_pages.shape[1]
    want = {"q_nope": (B, H, 1, QK_NOPE_HEAD_DIM), "q_pe": (B, H, 1, QK_ROPE_HEAD_DIM),
            "k_nope_pages": (N, H, bs, QK_NOPE_HEAD_DIM), "k_pe_pages": (N, bs, QK_ROPE_HEAD_DIM),
            "v_pages": (N, H, bs, V_HEAD_DIM)}
    for t, n in ((q_nope, "q_nope"), (q_pe, "q_pe"), (k_nope_pages, "k_nope_pages"),
                 (k_pe_pages, "k_pe_pages"), (v_pages, "v_pages")):
        if tuple(t.shape) != want[n] or t.device != q_nope.device:
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {want[n]} on {q_nope.device}")
    if block_table.dim() != 2:
        raise ValueError("block_table must be 2D [B, max_blocks]")
    M = block_table.shape[1]
    _check_int32(block_table, "block_table", (B, M), q_nope.device)
    _check_int32(seq_lens, "seq_lens", (B,), q_nope.device)
    ptr_new = [None, None, None]
    if new is not None:
        kn_new, kp_new, v_new = new
        for t, n, shp in ((kn_new, "k_nope_new", (B, H, 1, QK_NOPE_HEAD_DIM)),
                          (kp_new, "k_pe_new", (B, 1, 1, QK_ROPE_HEAD_DIM)),
                          (v_new, "v_new", (B, H, 1, V_HEAD_DIM))):
            _check_tensor(t, n)
            if tuple(t.shape) != shp or t.device != q_nope.device:
                raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {shp}")
        ptr_new = [kn_new.data_ptr(), kp_new.data_ptr(), v_new.data_ptr()]
    if out is None:
        out = torch.empty((B, H, 1, V_HEAD_DIM), dtype=torch.bfloat16, device=q_nope.device)
    else:
        _check_tensor(out, "out")
        if tuple(out.shape) != (B, H, 1, V_HEAD_DIM) or out.device != q_nope.device:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, 1, V_HEAD_DIM)}")
    need = mla_attn_decode_paged_workspace_bytes(B, H, max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_nope.device)
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    if rope_table is not None:
        _check_rope_table(rope_table, q_nope.device)
        st = _lib.mla_attn_decode_paged_rope(
            q_nope.data_ptr(), q_pe.data_ptr(), k_nope_pages.data_ptr(), k_pe_pages.data_ptr(),
            v_pages.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), *ptr_new,
            rope_table.data_ptr(), int(rope_table.shape[0]), out.data_ptr(), workspace.data_ptr(),
            ws_bytes, B, H, N, bs, M, int(max_seq_len), float(softmax_scale),
            _stream_handle(q_nope.device))
        _raise_for(st, "mla_attn_decode_paged_rope")
        return out
    st = _lib.mla_attn_decode_paged(
        q_nope.data_ptr(), q_pe.data_ptr(), k_nope_pages.data_ptr(), k_pe_pages.data_ptr(),
        v_pages.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), *ptr_new, out.data_ptr(),
        workspace.data_ptr(), ws_bytes, B, H, N, bs, M, int(max_seq_len), float(softmax_scale),
        _stream_handle(q_nope.device))
    _raise_for(st, "mla_attn_decode_paged")
    return out


KV_LORA_RANK = 512


def mla_attn_decode_latent_workspace_bytes(B: int, H: int, S: int) -> int:
    """Bytes of device scratch mla_attn_decode_latent needs for (B, H, S)."""
    return int(_lib.mla_attn_decode_latent_workspace_bytes(int(B), int(H), int(S)))


def mla_attn_decode_latent(q_nope, q_pe, c_kv, k_pe, w_kv_b, past_len: int, softmax_scale: float,
                           out=None, workspace=None):
    """Decode over the compressed cache: one query per sequence against S = past_len + 1 keys.

    q_nope [B,H,1,128], q_pe [B,H,1,64], c_kv [B,S,512] (normalised latent),
    k_pe [B,1,S,64] (shared rotary key), w_kv_b [H*256,512] (kv_b_proj.weight);
    bf16, contiguous, one GPU. Returns out [B,H,1,128] bf16 on the current stream.
    """
    import torch

    for t, n in ((q_nope, "q_nope"), (q_pe, "q_pe"), (k_pe, "k_pe")):
        _check_tensor(t, n)
    for t, n, nd in ((c_kv, "c_kv", 3), (w_kv_b, "w_kv_b", 2)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda \
                or not t.is_contiguous() or t.dim() != nd:
            raise ValueError(f"{n} must be a contiguous {nd}D bfloat16 GPU tensor")
    B, H, T, _ = q_nope.shape
    S = c_kv.shape[1]
    want = {"q_nope": (B, H, 1, QK_NOPE_HEAD_DIM), "q_pe": (B, H, 1, QK_ROPE_HEAD_DIM),
            "c_kv": (B, S, KV_LORA_RANK), "k_pe": (B, 1, S, QK_ROPE_HEAD_DIM),
            "w_kv_b": (H * (QK_NOPE_HEAD_DIM + V_HEAD_DIM), KV_LORA_RANK)}
    for t, n in ((q_nope, "q_nope"), (q_pe, "q_pe"), (c_kv, "c_kv"), (k_pe, "k_pe"), (w_kv_b, "w_kv_b")):
        if tuple(t.shape) != want[n]:
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {want[n]}")
    devs = {t.device for t in (q_nope, q_pe, c_kv, k_pe, w_kv_b)}
    if len(devs) != 1:
        raise ValueError(f"inputs are on different devices: {devs}")
    if out is None:
        out = torch.empty((B, H, 1, V_HEAD_DIM), dtype=torch.bfloat16, device=q_nope.device)
    else:
        _check_tensor(out, "out")
        if tuple(out.shape) != (B, H, 1, V_HEAD_DIM) or out.device != q_nope.device:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, 1, V_HEAD_DIM)}")
    need = mla_attn_decode_latent_workspace_bytes(B, H, S)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_nope.device)
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.mla_attn_decode_latent(
        q_nope.data_ptr(), q_pe.data_ptr(), c_kv.data_ptr(), k_pe.data_ptr(), w_kv_b.data_ptr(),
        out.data_ptr(), workspace.data_ptr(), ws_bytes, B, H, S, int(past_len),
        float(softmax_scale), _stream_handle(q_nope.device))
    _raise_for(st, "mla_attn_decode_latent")
    return out


def mla_rope_table_bytes(max_pos: int) -> int:
    """Bytes of the rotary table for positions 0..max_pos-1 (256 per position)."""
    return int(_lib.mla_rope_table_bytes(int(max_pos)))


def mla_rope_table(max_pos: int, theta: float = 50000.0, factor: float = 32.0,
                   original_max_position: int = 4096, beta_fast: float = 1.0, beta_slow: float = 1.0,
                   device=None, out=None):
    """cos/sin table [max_pos, 32, 2] fp32 of YaRN-scaled RoPE (defaults: the
    released configuration's rope_theta and rope_scaling), built on the GPU."""
    import torch

    if out is None:
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        out = torch.empty((max(int(max_pos), 0), 32, 2), dtype=torch.float32, device=dev)
    if not (out.dtype == torch.float32 and out.is_cuda and out.is_contiguous()
            and tuple(out.shape) == (int(max_pos), 32, 2)):
        raise ValueError(f"out must be a contiguous float32 GPU tensor of shape ({int(max_pos)}, 32, 2)")
    st = _lib.mla_rope_table(out.data_ptr(), int(max_pos), float(theta), float(factor),
                             int(original_max_position), float(beta_fast), float(beta_slow),
                             _stream_handle(out.device))
    _raise_for(st, "mla_rope_table")
    return out


def mla_rope_apply(x, table, past_len: int = 0, past_lens=None):
    """Rotate x [B, R, T, 64] bf16 in place (R = H for q_pe, 1 for the shared
    k_pe): row t of sequence b at position past_len + t, or past_lens[b] + t
    (int32 [B] on the device). Returns x."""
    import torch

    _check_tensor(x, "x")
    B, R, T, D = x.shape
    if D != QK_ROPE_HEAD_DIM:
        raise ValueError(f"x must have {QK_ROPE_HEAD_DIM} rotary dims, got shape {tuple(x.shape)}")
    if not (isinstance(table, torch.Tensor) and table.dtype == torch.float32 and table.is_contiguous()
            and table.dim() == 3 and tuple(table.shape[1:]) == (32, 2) and table.device == x.device):
        raise ValueError(f"table must be a contiguous float32 [max_pos, 32, 2] tensor on {x.device}")
    if past_lens is not None:
        _check_int32(past_lens, "past_lens", (B,), x.device)
    st = _lib.mla_rope_apply(x.data_ptr(), past_lens.data_ptr() if past_lens is not None else None,
                             table.data_ptr(), int(table.shape[0]), B, R, T, int(past_len),
                             _stream_handle(x.device))
    _raise_for(st, "mla_rope_apply")
    return x


def mla_rope_apply_qk(q_pe, k_pe, table, past_len: int = 0, past_lens=None):
    """Rotate q_pe [B, H, T, 64] and the new keys' k_pe [B, 1, T, 64] in place,
    in one launch (positions as mla_rope_apply). Returns (q_pe, k_pe)."""
    import torch

    _check_tensor(q_pe, "q_pe")
    _check_tensor(k_pe, "k_pe")
    B, H, T, D = q_pe.shape
    if D != QK_ROPE_HEAD_DIM or tuple(k_pe.shape) != (B, 1, T, QK_ROPE_HEAD_DIM) or k_pe.device != q_pe.device:
        raise ValueError(f"q_pe {tuple(q_pe.shape)} and k_pe {tuple(k_pe.shape)} must be [B, H, T, 64] and "
                         "[B, 1, T, 64] on one device")
    if not (isinstance(table, torch.Tensor) and table.dtype == torch.float32 and table.is_contiguous()
            and table.dim() == 3 and tuple(table.shape[1:]) == (32, 2) and table.device == q_pe.device):
        raise ValueError(f"table must be a contiguous float32 [max_pos, 32, 2] tensor on {q_pe.device}")
    if past_lens is not None:
        _check_int32(past_lens, "past_lens", (B,), q_pe.device)
    st = _lib.mla_rope_apply_qk(q_pe.data_ptr(), k_pe.data_ptr(),
                                past_lens.data_ptr() if past_lens is not None else None, table.data_ptr(),
                                int(table.shape[0]), B, H, T, int(past_len), _stream_handle(q_pe.device))
    _raise_for(st, "mla_rope_apply_qk")
    return q_pe, k_pe


__all__ = [
    "mla_rope_table",
    "mla_rope_table_bytes",
    "mla_rope_apply",
    "mla_rope_apply_qk",
    "mla_attn_prefill_ws",
    "mla_attn_prefill_workspace_bytes",
    "mla_attn_decode_paged",
    "mla_attn_decode_paged_workspace_bytes",
    "mla_attn_decode_varlen",
    "mla_attn_decode_varlen_workspace_bytes",
    "mla_attn_decode_latent",
    "mla_attn_decode_latent_workspace_bytes",
    "mla_attn_prefill",
    "mla_attn_prefill_varlen",
    "mla_attn_prefill_masked",
    "mla_attn_decode",
    "mla_attn_decode_masked",
    "mla_attn_decode_workspace_bytes",
    "MLAError",
    "LIB_PATH",
    "SIGNATURES",
    "load_library",
]
