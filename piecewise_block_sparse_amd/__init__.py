"""Piecewise block-sparse (PISA) attention for MI355X: Python binding of libpisa.

Thin marshalling layer over the C ABI in include/pisa.h.  Torch supplies the
device memory and the current HIP stream; every step of the computation runs
in libpisa's gfx950 kernels.  If libpisa.so is missing the calls raise.

    stats = precompute(K, V, block)                       # centroids, value sums, Hbar, M
    idx = route(Q, stats, k, lam, block)                  # [b,h,nb,k] int32, ascending
    O = attention(Q, K, V, idx, stats, block, mode="approx")

Modes: "approx" (PISA: exact blocks, zeroth-order blocks, global Hbar
correction), "zeroth" (no correction), "first" (a first-order term per
unselected block; needs precompute(..., store_Ht=True) for bf16 inputs or
store_H=True for fp32 inputs), "drop" (keep-or-drop block-sparse attention).

Q, K, V: contiguous [b, h, L, d] CUDA tensors, bfloat16 or float32, L a
multiple of `block`.  seq_lens (every call, optional): int32 CUDA tensor [b]
with each sequence's valid length inside its padded buffer; the three calls
must get the same lengths.
"""
from __future__ import annotations

import ctypes
import math

from . import _lib

__all__ = ["precompute", "route", "attention", "route_attention", "workspace_size",
           "attention_split_workspace_size", "version", "MODE_APPROX",
           "MODE_DROP", "MODE_ZEROTH", "MODE_FIRST"]

MODE_APPROX = _lib.MODE_APPROX
MODE_DROP = _lib.MODE_DROP
MODE_ZEROTH = _lib.MODE_ZEROTH
MODE_FIRST = _lib.MODE_FIRST
_MODES = {"approx": MODE_APPROX, "drop": MODE_DROP, "zeroth": MODE_ZEROTH, "first": MODE_FIRST}


def _torch():
    import torch
    return torch


def _shape(X, block: int, seq_lens=None) -> _lib.PisaShape:
    torch = _torch()
    if X.dim() != 4:
        raise ValueError("expected a [b, h, L, d] tensor")
    if seq_lens is not None:
        _expect(seq_lens, (X.shape[0],), torch.int32, "seq_lens")
        if seq_lens.device != X.device:
            raise ValueError("seq_lens must be on the device of the inputs")
    if X.dtype == torch.bfloat16:
        dt = _lib.DTYPE_BF16
    elif X.dtype == torch.float32:
        dt = _lib.DTYPE_FP32
    else:
        raise TypeError(f"unsupported dtype {X.dtype}")
    b, h, L, d = X.shape
    return _lib.PisaShape(b, h, L, d, block, dt, _ptr(seq_lens))


def _ptr(t) -> int:
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors must be contiguous device tensors")
    return t.data_ptr()


def _stream(t) -> int:
    return _torch().cuda.current_stream(t.device).cuda_stream


def _expect(t, shape, dtype, name):
    if t is None or tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        got = None if t is None else (tuple(t.shape), t.dtype)
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {got}")


def _same(ref, *others):
    for o in others:
        if o.shape != ref.shape or o.dtype != ref.dtype or o.device != ref.device:
            raise ValueError("Q, K, V (and O) must share shape, dtype and device")


def version() -> int:
    return _lib.load().pisa_version()


def workspace_size(X, block: int) -> int:
    return _lib.load().pisa_workspace_size(ctypes.byref(_shape(X, block)))


def precompute(K, V, block: int, store_H: bool = False, workspace=None, packed: bool = True,
               store_Ht: bool = False, norm: str = "fro", seq_lens=None) -> dict:
    """Block statistics (fp32): centroid, vsum, Hbar, M, and H when store_H.

    norm: "fro" (M_j = Frobenius norm of H_j - Hbar) or "spectral" (its largest
    singular value; with bf16 inputs this also returns H, which it reads).

    For bf16 inputs (and packed=True) also the bf16 pack that the attention
    kernel streams in PISA mode (key "packed"), and with store_Ht the bf16
    H_j^T per block (key "Ht") that mode "first" streams."""
    torch = _torch()
    lib = _lib.load()
    _same(K, V)
    shp = _shape(K, block, seq_lens)
    m_norm = {"fro": _lib.NORM_FROBENIUS, "spectral": _lib.NORM_SPECTRAL}[norm]
    if m_norm == _lib.NORM_SPECTRAL and K.dtype == torch.bfloat16:
        store_H = True
    b, h, L, d = K.shape
    nb = L // block if L % block == 0 else 0
    f32 = dict(dtype=torch.float32, device=K.device)
    out = {
        "centroid": torch.empty((b, h, nb, d), **f32),
        "vsum": torch.empty((b, h, nb, d), **f32),
        "H": torch.empty((b, h, nb, d, d), **f32) if store_H else None,
        "Hbar": torch.empty((b, h, d, d), **f32),
        "M": torch.empty((b, h, nb), **f32),
        "packed": None,
        "Ht": None,
    }
    if store_Ht:
        if K.dtype != torch.bfloat16:
            raise ValueError("store_Ht is for bf16 inputs (fp32 mode 'first' reads H)")
        out["Ht"] = torch.empty((b, h, nb, d, d), dtype=torch.bfloat16, device=K.device)
    npk = lib.pisa_packed_size(ctypes.byref(shp)) if packed else 0
    if npk:
        out["packed"] = torch.empty(npk, dtype=torch.uint8, device=K.device)
    need = lib.pisa_workspace_size(ctypes.byref(shp))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=K.device)
    st = _lib.PisaStats(*(_ptr(out[n]) for n in ("centroid", "vsum", "H", "Hbar", "M", "packed", "Ht")),
                        m_norm)
    _lib.check("pisa_precompute", lib.pisa_precompute(
        ctypes.byref(shp), _ptr(K), _ptr(V), ctypes.byref(st), _ptr(workspace),
        workspace.numel(), _stream(K)))
    return out


def route(Q, stats: dict, k: int, lam: float, block: int, scale: float | None = None,
          seq_lens=None):
    """Top-k exact blocks per query block, int32 [b, h, nb, k], rows ascending
    (with seq_lens: -1 after the last candidate of a short row)."""
    torch = _torch()
    lib = _lib.load()
    shp = _shape(Q, block, seq_lens)
    b, h, L, d = Q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    idx = torch.empty((b, h, max(L // block, 0), max(k, 0)), dtype=torch.int32, device=Q.device)
    nb = L // block if L % block == 0 else 0
    _expect(stats["centroid"], (b, h, nb, d), torch.float32, "stats['centroid']")
    _expect(stats["M"], (b, h, nb), torch.float32, "stats['M']")
    _lib.check("pisa_route", lib.pisa_route(
        ctypes.byref(shp), _ptr(Q), _ptr(stats["centroid"]), _ptr(stats["M"]), int(k), scale,
        float(lam), _ptr(idx), _stream(Q)))
    return idx


def attention(Q, K, V, idx, stats: dict | None, block: int, mode: int | str = "approx",
              scale: float | None = None, out=None, seq_lens=None, split_blocks: int | None = None,
              workspace=None):
    """PISA block-sparse attention; mode "approx", "zeroth", "first" or "drop".

    split_blocks (bf16; not mode "first"): run work items whose exact lists
    hold more than this many blocks as several workgroups and merge them
    (pisa_attention_split), with `workspace` (allocated when None)."""
    torch = _torch()
    lib = _lib.load()
    _same(Q, K, V)
    if isinstance(mode, str):
        mode = _MODES[mode]
    shp = _shape(Q, block, seq_lens)
    d = Q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    b, h, L, _ = Q.shape
    nb = L // block if L % block == 0 else 0
    if idx.dim() != 4:
        raise ValueError("idx must be an int32 [b, h, nb, kmax] tensor")
    _expect(idx, (b, h, nb, idx.shape[-1]), torch.int32, "idx")
    O = torch.empty_like(Q) if out is None else out
    _same(Q, O)
    st = None
    if mode != MODE_DROP:
        if stats is None:
            raise ValueError("modes other than drop need the block statistics")
        _expect(stats["centroid"], (b, h, nb, d), torch.float32, "stats['centroid']")
        _expect(stats["vsum"], (b, h, nb, d), torch.float32, "stats['vsum']")
        if mode == MODE_APPROX:
            _expect(stats["Hbar"], (b, h, d, d), torch.float32, "stats['Hbar']")
        if mode == MODE_FIRST and Q.dtype == torch.bfloat16:
            _expect(stats.get("Ht"), (b, h, nb, d, d), torch.bfloat16, "stats['Ht']")
        if mode == MODE_FIRST and Q.dtype == torch.float32:
            _expect(stats.get("H"), (b, h, nb, d, d), torch.float32, "stats['H']")
    if stats is not None:
        pk = stats.get("packed")
        if pk is not None and pk.numel() != lib.pisa_packed_size(ctypes.byref(shp)):
            raise ValueError("stats['packed'] does not match this shape")
        st = _lib.PisaStats(_ptr(stats["centroid"]), _ptr(stats["vsum"]), _ptr(stats.get("H")),
                            _ptr(stats["Hbar"]), None, _ptr(pk), _ptr(stats.get("Ht")))
    if split_blocks is not None:
        kmax = int(idx.shape[-1])
        need = lib.pisa_attention_split_workspace_size(ctypes.byref(shp), kmax, int(split_blocks))
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
        _lib.check("pisa_attention_split", lib.pisa_attention_split(
            ctypes.byref(shp), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), kmax,
            ctypes.byref(st) if st is not None else None, int(mode), scale, int(split_blocks),
            _ptr(O), _ptr(workspace), workspace.numel(), _stream(Q)))
        return O
    _lib.check("pisa_attention", lib.pisa_attention(
        ctypes.byref(shp), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), int(idx.shape[-1]),
        ctypes.byref(st) if st is not None else None, int(mode), scale, _ptr(O), _stream(Q)))
    return O


def attention_split_workspace_size(X, block: int, kmax: int, split_blocks: int) -> int:
    """Bytes of workspace attention(..., split_blocks=...) needs for idx rows of kmax entries."""
    return _lib.load().pisa_attention_split_workspace_size(ctypes.byref(_shape(X, block)), int(kmax),
                                                           int(split_blocks))


_ROUTE_FORMS = {"auto": _lib.ROUTE_AUTO, "in_kernel": _lib.ROUTE_IN_KERNEL,
                "two_launch": _lib.ROUTE_TWO_LAUNCH}


def route_attention(Q, K, V, stats: dict, k: int, lam: float, block: int,
                    mode: int | str = "approx", scale: float | None = None, out=None,
                    seq_lens=None, return_idx: bool = False, form: str = "auto"):
    """Routing and attention in one call (bf16): the selection of route()
    (bit for bit) followed by attention() on it.  form "in_kernel": each
    attention workgroup routes its own query block(s), no idx round trip;
    "two_launch": route() then attention(); "auto" (default): in-kernel while
    the work fits one round of workgroups, else two launches (the same
    selection and output either way).  Modes "approx", "zeroth" and "drop".
    With return_idx, returns (O, idx)."""
    torch = _torch()
    lib = _lib.load()
    _same(Q, K, V)
    if isinstance(mode, str):
        mode = _MODES[mode]
    shp = _shape(Q, block, seq_lens)
    b, h, L, d = Q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nb = L // block if L % block == 0 else 0
    _expect(stats["centroid"], (b, h, nb, d), torch.float32, "stats['centroid']")
    _expect(stats["M"], (b, h, nb), torch.float32, "stats['M']")
    if mode != MODE_DROP:
        _expect(stats["vsum"], (b, h, nb, d), torch.float32, "stats['vsum']")
    if mode == MODE_APPROX:
        _expect(stats["Hbar"], (b, h, d, d), torch.float32, "stats['Hbar']")
    pk = stats.get("packed")
    if pk is not None and pk.numel() != lib.pisa_packed_size(ctypes.byref(shp)):
        raise ValueError("stats['packed'] does not match this shape")
    if form not in _ROUTE_FORMS:
        raise ValueError(f"unknown form {form!r}")
    # the automatic form may need idx to hold the selection between two launches
    idx = (torch.empty((b, h, nb, max(k, 0)), dtype=torch.int32, device=Q.device)
           if return_idx or form != "in_kernel" else None)
    O = torch.empty_like(Q) if out is None else out
    _same(Q, O)
    st = _lib.PisaStats(_ptr(stats["centroid"]), _ptr(stats.get("vsum")), None,
                        _ptr(stats.get("Hbar")), _ptr(stats["M"]), _ptr(pk), None)
    _lib.check("pisa_route_attention", lib.pisa_route_attention(
        ctypes.byref(shp), _ptr(Q), _ptr(K), _ptr(V), ctypes.byref(st), int(k), float(lam),
        int(mode), scale, _ptr(idx), _ptr(O), _ROUTE_FORMS[form], _stream(Q)))
    return (O, idx) if return_idx else O
