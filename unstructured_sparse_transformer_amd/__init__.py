"""Python binding of libtwell (ReLU-sparse gated FFN with TwELL on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libtwell.so`` (built from ``csrc/`` by ``_build.py``); PyTorch supplies device
memory and the current HIP stream.  There is no CPU fallback: ``load()``
raises when the library is missing, and every call raises on a non-OK status.

The functions carry the C names (``include/twell.h``):
``twell_ffn_forward``, ``twell_ffn_from_gate``, ``twell_pack_gate``, ``twell_gate_dense``, ``twell_pack_gate_stats``, ``twell_partition_overflow``,
``twell_pack_gate_hybrid``,
``twell_ffn_fused``, ``twell_ffn_overflow``, ``twell_ffn_hybrid``,
``twell_workspace_bytes``, ``twell_ffn_decode``,
``twell_ffn_decode_workspace_bytes``, ``twell_ffn_decode_noalloc``, ``twell_dense_to_hybrid``,
``twell_hybrid_to_dense``, ``twell_compact_min_bytes``, ``twell_compact_hybrid``,
``twell_compact_to_dense``, ``twell_ffn_backward``,
``twell_ffn_backward_workspace_bytes``.

One layer's forward pass, bf16 (x [T][d], W_g^T and W_u^T [F][d], W_d [F][d],
all contiguous on the GPU; y [T][d] fp32)::

    import unstructured_sparse_transformer_amd as tw
    hy = tw.Hybrid.empty(T, F, tile_w=256, cap=16, dtype=torch.bfloat16, max_ovf=1024)
    ws = tw.hybrid_workspace(hy, d)
    tw.twell_ffn_forward(x, wg_t, wu_t, wd, hy, y, ws)   # on the current stream
    # hy.ell holds the TwELL of ReLU(x W_g); hy.n_ovf counts the overflow rows.
    # Overflow rows past max_ovf are counted but not computed: after
    # synchronising, check n_ovf <= max_ovf and grow max_ovf otherwise.

For T <= 64 tokens, ``twell_ffn_decode`` with ``decode_workspace(T, F, d,
tile_w)`` computes the same in four short kernels.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtwell.so")

TWELL_F32, TWELL_BF16 = 0, 1
STATUS = {0: "TWELL_OK", -1: "TWELL_E_NULL", -2: "TWELL_E_ALIGN", -3: "TWELL_E_SHAPE",
          -4: "TWELL_E_UNSUPPORTED", -5: "TWELL_E_HIP", -6: "TWELL_E_WORKSPACE", -7: "TWELL_E_SCRATCH"}
EXPORTS = ("twell_ffn_forward", "twell_ffn_from_gate", "twell_pack_gate", "twell_gate_dense", "twell_pack_gate_stats", "twell_partition_overflow", "twell_pack_gate_hybrid",
           "twell_ffn_fused", "twell_workspace_bytes", "twell_ffn_overflow", "twell_ffn_hybrid",
           "twell_ffn_decode_workspace_bytes", "twell_ffn_decode", "twell_ffn_decode_noalloc", "twell_dense_to_hybrid", "twell_hybrid_to_dense",
           "twell_compact_min_bytes", "twell_compact_hybrid", "twell_compact_to_dense",
           "twell_ffn_backward_workspace_bytes", "twell_ffn_backward", "twell_status_str", "twell_version")


class TwellT(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("F", ctypes.c_int32), ("tile_w", ctypes.c_int32),
                ("cap", ctypes.c_int32), ("vdtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("val", ctypes.c_void_p), ("idx", ctypes.c_void_p), ("cnt", ctypes.c_void_p)]


class TwellHybridT(ctypes.Structure):
    _fields_ = [("ell", TwellT), ("max_ovf", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("row_ovf", ctypes.c_void_p), ("ovf_rows", ctypes.c_void_p), ("n_ovf", ctypes.c_void_p),
                ("dense", ctypes.c_void_p), ("order", ctypes.c_void_p)]


class TwellError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.twell_status_str(status).decode() if _lib is not None else ""
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libtwell.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libtwell.so not found at {path}: build it with "
                           "`python -m unstructured_sparse_transformer_amd._build` (no CPU fallback exists)")
    lib = ctypes.CDLL(path)
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    lib.twell_pack_gate.argtypes = [P, P, I32, ctypes.POINTER(TwellT), P]
    lib.twell_pack_gate_stats.argtypes = [P, P, I32, ctypes.POINTER(TwellT), P, P, P]
    lib.twell_gate_dense.argtypes = [P, P, I32, I32, I32, I32, P, P]
    lib.twell_partition_overflow.argtypes = [P, P, I32, ctypes.POINTER(TwellHybridT), P]
    lib.twell_pack_gate_hybrid.argtypes = [P, P, I32, ctypes.POINTER(TwellHybridT), P]
    lib.twell_ffn_fused.argtypes = [ctypes.POINTER(TwellT), P, P, P, P, I32, P, P, ctypes.c_size_t, P]
    lib.twell_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    lib.twell_workspace_bytes.restype = ctypes.c_size_t
    lib.twell_ffn_hybrid.argtypes = [ctypes.POINTER(TwellHybridT), P, P, P, I32, P, P, ctypes.c_size_t, P]
    lib.twell_ffn_overflow.argtypes = [ctypes.POINTER(TwellHybridT), P, P, P, I32, P, P, ctypes.c_size_t, P]
    lib.twell_ffn_forward.argtypes = [P, P, P, P, I32, ctypes.POINTER(TwellHybridT), P, P, ctypes.c_size_t, P]
    lib.twell_ffn_from_gate.argtypes = [P, P, P, P, I32, ctypes.POINTER(TwellHybridT), P, P, ctypes.c_size_t, P]
    lib.twell_ffn_decode_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.twell_ffn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.twell_ffn_decode.argtypes = [P, P, P, P, I32, ctypes.POINTER(TwellHybridT), P, P, ctypes.c_size_t, P]
    lib.twell_ffn_decode_noalloc.argtypes = [P, P, P, P, I32, ctypes.POINTER(TwellHybridT), P, P]
    lib.twell_dense_to_hybrid.argtypes = [P, ctypes.POINTER(TwellHybridT), P]
    lib.twell_hybrid_to_dense.argtypes = [ctypes.POINTER(TwellHybridT), P, P]
    lib.twell_compact_min_bytes.argtypes = [I32]
    lib.twell_compact_min_bytes.restype = ctypes.c_size_t
    lib.twell_compact_hybrid.argtypes = [ctypes.POINTER(TwellHybridT), P, ctypes.c_size_t, P]
    lib.twell_compact_to_dense.argtypes = [P, I32, I32, I32, P, P]
    lib.twell_ffn_backward_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.twell_ffn_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.twell_ffn_backward.argtypes = [ctypes.POINTER(TwellHybridT), P, P, P, P, I32, P, P, P, P, P, I32, P,
                                       ctypes.c_size_t, P]
    lib.twell_status_str.argtypes = [ctypes.c_int]
    lib.twell_status_str.restype = ctypes.c_char_p
    lib.twell_version.restype = ctypes.c_int
    for fn in (lib.twell_pack_gate, lib.twell_gate_dense, lib.twell_pack_gate_stats, lib.twell_partition_overflow, lib.twell_pack_gate_hybrid,
               lib.twell_ffn_fused, lib.twell_ffn_hybrid, lib.twell_ffn_overflow, lib.twell_ffn_forward,
               lib.twell_ffn_from_gate, lib.twell_ffn_decode, lib.twell_ffn_decode_noalloc,
               lib.twell_dense_to_hybrid, lib.twell_hybrid_to_dense, lib.twell_compact_hybrid,
               lib.twell_compact_to_dense, lib.twell_ffn_backward):
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


# ---------------------------------------------------------------- marshalling helpers
def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def vdtype_of(torch_dtype) -> int:
    import torch
    if torch_dtype == torch.bfloat16:
        return TWELL_BF16
    if torch_dtype == torch.float32:
        return TWELL_F32
    raise TypeError(f"unsupported element type {torch_dtype}")


def _check(fn: str, st: int):
    if st != 0:
        raise TwellError(fn, st)


@dataclass
class TwELL:
    """Device buffers of one TwELL (torch tensors) and its C descriptor."""
    T: int
    F: int
    tile_w: int
    cap: int
    dtype: object
    val: object  # [T][n_b][cap] dtype
    idx: object  # [T][n_b][cap] uint8
    cnt: object  # [T][n_b] int32

    @property
    def n_b(self) -> int:
        return self.F // self.tile_w

    @classmethod
    def empty(cls, T, F, tile_w, cap, dtype, device="cuda"):
        import torch
        n_b = F // tile_w
        return cls(T, F, tile_w, cap, dtype,
                   torch.empty((T, n_b, cap), dtype=dtype, device=device),
                   torch.empty((T, n_b, cap), dtype=torch.uint8, device=device),
                   torch.empty((T, n_b), dtype=torch.int32, device=device))

    def desc(self) -> TwellT:
        return TwellT(self.T, self.F, self.tile_w, self.cap, vdtype_of(self.dtype), 0,
                      _ptr(self.val), _ptr(self.idx), _ptr(self.cnt))


@dataclass
class Hybrid:
    """TwELL plus overflow partition and dense backup buffers."""
    ell: TwELL
    max_ovf: int
    row_ovf: object   # [T] int32
    ovf_rows: object  # [max_ovf] int32
    n_ovf: object     # [1] int32
    dense: object     # [max_ovf][F] dtype
    order: object     # [T] int32: the fused step's work order

    @classmethod
    def empty(cls, T, F, tile_w, cap, dtype, max_ovf, device="cuda"):
        import torch
        return cls(TwELL.empty(T, F, tile_w, cap, dtype, device), max_ovf,
                   torch.empty(T, dtype=torch.int32, device=device),
                   torch.empty(max(max_ovf, 1), dtype=torch.int32, device=device),
                   torch.empty(1, dtype=torch.int32, device=device),
                   torch.empty((max(max_ovf, 1), F), dtype=dtype, device=device),
                   torch.empty(T, dtype=torch.int32, device=device))

    def desc(self) -> TwellHybridT:
        return TwellHybridT(self.ell.desc(), self.max_ovf, 0, _ptr(self.row_ovf), _ptr(self.ovf_rows),
                            _ptr(self.n_ovf), _ptr(self.dense), _ptr(self.order))


# ---------------------------------------------------------------- the C entry points
def twell_pack_gate(x, wg_t, tw: TwELL, stream=None):
    lib = load()
    d = ctypes.byref(tw.desc())
    _check("twell_pack_gate", lib.twell_pack_gate(_ptr(x), _ptr(wg_t), int(x.shape[1]), d, _stream(stream)))


def twell_gate_dense(x, wg_t, h, stream=None):
    """h [T][F] (x's dtype) = ReLU(x W_g), the gate with a plain dense store."""
    _check("twell_gate_dense", load().twell_gate_dense(_ptr(x), _ptr(wg_t), int(x.shape[1]), int(x.shape[0]),
                                                       int(wg_t.shape[0]), vdtype_of(x.dtype), _ptr(h),
                                                       _stream(stream)))


def twell_pack_gate_stats(x, wg_t, tw: TwELL, neuron_cnt, l1, stream=None):
    """neuron_cnt: int32 [F] (added to); l1: float32 [T][F // tile_w] (overwritten)."""
    lib = load()
    d = ctypes.byref(tw.desc())
    _check("twell_pack_gate_stats", lib.twell_pack_gate_stats(_ptr(x), _ptr(wg_t), int(x.shape[1]), d,
                                                              _ptr(neuron_cnt), _ptr(l1), _stream(stream)))


def twell_partition_overflow(x, wg_t, hy: Hybrid, stream=None):
    lib = load()
    _check("twell_partition_overflow",
           lib.twell_partition_overflow(_ptr(x), _ptr(wg_t), int(x.shape[1]), ctypes.byref(hy.desc()),
                                        _stream(stream)))


def twell_pack_gate_hybrid(x, wg_t, hy: Hybrid, stream=None):
    lib = load()
    _check("twell_pack_gate_hybrid",
           lib.twell_pack_gate_hybrid(_ptr(x), _ptr(wg_t), int(x.shape[1]), ctypes.byref(hy.desc()),
                                      _stream(stream)))


def twell_ffn_fused(tw: TwELL, x, wu_t, wd, y, workspace, stream=None, order=None):
    lib = load()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("twell_ffn_fused", lib.twell_ffn_fused(ctypes.byref(tw.desc()), _ptr(order), _ptr(x), _ptr(wu_t),
                                                  _ptr(wd), int(x.shape[1]), _ptr(y), _ptr(workspace), nbytes,
                                                  _stream(stream)))


def twell_workspace_bytes(T: int, F: int, tile_w: int, cap: int, max_ovf: int, d: int, dtype) -> int:
    return int(load().twell_workspace_bytes(T, F, tile_w, cap, max_ovf, d, vdtype_of(dtype)))


def twell_ffn_hybrid(hy: Hybrid, x, wu_t, wd, y, workspace, stream=None):
    lib = load()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("twell_ffn_hybrid",
           lib.twell_ffn_hybrid(ctypes.byref(hy.desc()), _ptr(x), _ptr(wu_t), _ptr(wd), int(x.shape[1]),
                                _ptr(y), _ptr(workspace), nbytes, _stream(stream)))


def twell_ffn_forward(x, wg_t, wu_t, wd, hy: Hybrid, y, workspace, stream=None):
    """The whole layer: fills the hybrid `hy` and y [T][d] float in one call."""
    lib = load()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("twell_ffn_forward",
           lib.twell_ffn_forward(_ptr(x), _ptr(wg_t), _ptr(wu_t), _ptr(wd), int(x.shape[1]), ctypes.byref(hy.desc()),
                                 _ptr(y), _ptr(workspace), nbytes, _stream(stream)))


def twell_ffn_from_gate(x, wg_t, wu_t, wd, hy: Hybrid, y, workspace, stream=None):
    """The layer after twell_pack_gate on hy.ell: the rest of the hybrid and y."""
    lib = load()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("twell_ffn_from_gate",
           lib.twell_ffn_from_gate(_ptr(x), _ptr(wg_t), _ptr(wu_t), _ptr(wd), int(x.shape[1]),
                                   ctypes.byref(hy.desc()), _ptr(y), _ptr(workspace), nbytes, _stream(stream)))


def twell_ffn_overflow(hy: Hybrid, x, wu_t, wd, y, workspace, stream=None):
    lib = load()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("twell_ffn_overflow",
           lib.twell_ffn_overflow(ctypes.byref(hy.desc()), _ptr(x), _ptr(wu_t), _ptr(wd), int(x.shape[1]),
                                  _ptr(y), _ptr(workspace), nbytes, _stream(stream)))


def twell_dense_to_hybrid(h, hy: Hybrid, stream=None):
    """h: [T][F] in the hybrid's value dtype."""
    _check("twell_dense_to_hybrid", load().twell_dense_to_hybrid(_ptr(h), ctypes.byref(hy.desc()), _stream(stream)))


def twell_hybrid_to_dense(hy: Hybrid, out, stream=None):
    """out: [T][F] in the hybrid's value dtype (every element written)."""
    _check("twell_hybrid_to_dense", load().twell_hybrid_to_dense(ctypes.byref(hy.desc()), _ptr(out), _stream(stream)))


COMPACT_HEADER = (("T", "i"), ("F", "i"), ("tile_w", "i"), ("vdtype", "i"), ("n_entries", "i"), ("n_ovf", "i"),
                  ("n_dense", "i"), ("fits", "i"), ("off_row_ptr", "q"), ("off_col", "q"), ("off_val", "q"),
                  ("off_ovf", "q"), ("off_dense", "q"), ("bytes", "q"))


def twell_compact_min_bytes(T: int) -> int:
    return int(load().twell_compact_min_bytes(T))


def twell_compact_hybrid(hy: Hybrid, buf, stream=None):
    """buf: a uint8 device tensor (256-byte aligned by the allocator)."""
    _check("twell_compact_hybrid", load().twell_compact_hybrid(ctypes.byref(hy.desc()), _ptr(buf),
                                                               buf.numel() * buf.element_size(), _stream(stream)))


def twell_compact_to_dense(buf, T: int, F: int, dtype, out, stream=None):
    _check("twell_compact_to_dense", load().twell_compact_to_dense(_ptr(buf), T, F, vdtype_of(dtype), _ptr(out),
                                                                   _stream(stream)))


def compact_header(buf) -> dict:
    """The header of a compact buffer, read back to the host (synchronises)."""
    import struct
    fmt = "<" + "".join(f for _, f in COMPACT_HEADER)
    raw = bytes(buf[: struct.calcsize(fmt)].cpu().numpy().tobytes())
    return dict(zip((n for n, _ in COMPACT_HEADER), struct.unpack(fmt, raw)))


def twell_ffn_backward_workspace_bytes(T: int, F: int, d: int, max_entries: int) -> int:
    return int(load().twell_ffn_backward_workspace_bytes(T, F, d, max_entries))


def backward_workspace(T: int, F: int, d: int, max_entries: int, device="cuda"):
    import torch
    n = twell_ffn_backward_workspace_bytes(T, F, d, max_entries)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def twell_ffn_backward(hy: Hybrid, x, wg_t, wu_t, wd, dy, dx, dwg, dwu, dwd, max_entries: int, workspace,
                       stream=None):
    _check("twell_ffn_backward",
           load().twell_ffn_backward(ctypes.byref(hy.desc()), _ptr(x), _ptr(wg_t), _ptr(wu_t), _ptr(wd),
                                     int(wg_t.shape[1]), _ptr(dy), _ptr(dx), _ptr(dwg), _ptr(dwu), _ptr(dwd),
                                     max_entries, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))


def backward_status(workspace) -> tuple:
    """(entries, too_many) from a backward workspace (synchronises)."""
    v = workspace[:8].cpu().numpy().view("<i4")
    return int(v[0]), int(v[1])


def twell_ffn_decode_workspace_bytes(T: int, F: int, d: int, tile_w: int) -> int:
    return int(load().twell_ffn_decode_workspace_bytes(T, F, d, tile_w))


def twell_ffn_decode(x, wg_t, wu_t, wd, hy: Hybrid, y, workspace, stream=None):
    lib = load()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("twell_ffn_decode",
           lib.twell_ffn_decode(_ptr(x), _ptr(wg_t), _ptr(wu_t), _ptr(wd), int(x.shape[1]), ctypes.byref(hy.desc()),
                                _ptr(y), _ptr(workspace), nbytes, _stream(stream)))


def twell_ffn_decode_noalloc(x, wg_t, wu_t, wd, hy: Hybrid, y, stream=None):
    """twell_ffn_decode on the library's static scratch (no workspace argument)."""
    _check("twell_ffn_decode_noalloc",
           load().twell_ffn_decode_noalloc(_ptr(x), _ptr(wg_t), _ptr(wu_t), _ptr(wd), int(x.shape[1]),
                                           ctypes.byref(hy.desc()), _ptr(y), _stream(stream)))


def decode_workspace(T: int, F: int, d: int, tile_w: int, device="cuda"):
    """A workspace tensor of the size twell_ffn_decode needs (256-byte aligned by the allocator)."""
    import torch
    n = twell_ffn_decode_workspace_bytes(T, F, d, tile_w)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def workspace(T: int, F: int, tile_w: int, cap: int, max_ovf: int, d: int, dtype, device="cuda"):
    """A workspace tensor of the size twell_workspace_bytes gives (256-byte
    aligned by the allocator); it serves twell_ffn_fused, twell_ffn_overflow,
    twell_ffn_hybrid, twell_ffn_forward and twell_ffn_from_gate."""
    import torch
    n = twell_workspace_bytes(T, F, tile_w, cap, max_ovf, d, dtype)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def hybrid_workspace(hy: "Hybrid", d: int, device="cuda"):
    """The workspace for the calls on hybrid `hy` with model width d."""
    e = hy.ell
    return workspace(e.T, e.F, e.tile_w, e.cap, hy.max_ovf, d, e.dtype, device)
