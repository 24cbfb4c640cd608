"""Python binding of libduo (include/duo.h): argument marshalling only.

Every step of the hot path runs in the HIP kernels of libduo.so; this module
checks shapes, dtypes and devices of torch tensors, hands their device
pointers and the current HIP stream to the C ABI, and turns error codes into
exceptions.  There is no fallback: if libduo.so is missing this import fails.

Build the library first with ``python head_wise_kv_amd/build.py`` (or
``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libduo.so")

DUO_OK, DUO_EINVAL, DUO_EUNSUPPORTED, DUO_ECAPACITY, DUO_EEMPTY, DUO_EWORKSPACE, DUO_EHIP = 0, -1, -2, -3, -4, -5, -6
DUO_F32, DUO_BF16 = 0, 1
DUO_KV_NATIVE, DUO_KV_FP8, DUO_KV_INT4 = 0, 1, 2
ERROR_NAMES = {DUO_EINVAL: "DUO_EINVAL", DUO_EUNSUPPORTED: "DUO_EUNSUPPORTED", DUO_ECAPACITY: "DUO_ECAPACITY",
               DUO_EEMPTY: "DUO_EEMPTY", DUO_EWORKSPACE: "DUO_EWORKSPACE", DUO_EHIP: "DUO_EHIP"}

# Every entry point declared in include/duo.h.
EXPORTS = ("duo_cache_bytes", "duo_cache_payload_bytes", "duo_cache_init", "duo_append", "duo_decode",
           "duo_decode_append", "duo_prefill_chunk", "duo_cache_seq_len", "duo_cache_head_view", "duo_cache_free",
           "duo_last_error", "duo_gated_attention", "duo_cache_head_scales", "duo_append_row", "duo_prefill_chunk_row",
           "duo_cache_row_len", "duo_cache_reset_row", "duo_cache_fork_row", "duo_cache_free_pages",
           "duo_cache_row_pages", "duo_prefill_workspace_bytes", "duo_decode_append_noalloc",
           "duo_cache_sync", "duo_cache_reserve", "duo_rope_apply", "duo_decode_plan")


class DuoError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


class duo_config(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("B", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32),
                ("d_head", ctypes.c_int32), ("T_cap", ctypes.c_int64), ("sink", ctypes.c_int32),
                ("recent", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("retrieval_mask", ctypes.POINTER(ctypes.c_uint8)), ("kv_format", ctypes.c_int32),
                ("page_rows", ctypes.c_int32), ("n_pages", ctypes.c_int32), ("rope_theta", ctypes.c_float)]


class duo_gated_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("d_head", ctypes.c_int32),
                ("N", ctypes.c_int64), ("sink", ctypes.c_int32), ("recent", ctypes.c_int32), ("dtype", ctypes.c_int32)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libduo.so is not built ({_LIB_PATH}); run `python head_wise_kv_amd/build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(duo_config)
    lib.duo_cache_bytes.argtypes = [cfgp, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.duo_cache_payload_bytes.argtypes = [cfgp, ctypes.POINTER(sz)]
    lib.duo_cache_init.argtypes = [cfgp, vp, sz, vp, ctypes.POINTER(vp)]
    lib.duo_append.argtypes = [vp, i32, vp, vp, i64, vp]
    lib.duo_decode.argtypes = [vp, i32, vp, vp, ctypes.c_float, vp, sz, vp]
    lib.duo_decode_append.argtypes = [vp, i32, vp, vp, vp, vp, ctypes.c_float, vp, sz, vp]
    lib.duo_decode_append_noalloc.argtypes = [vp, i32, vp, vp, vp, vp, ctypes.c_float, vp]
    lib.duo_prefill_chunk.argtypes = [vp, i32, vp, vp, vp, i64, vp, ctypes.c_float, vp, sz, vp]
    lib.duo_cache_seq_len.argtypes = [vp, i32, ctypes.POINTER(i64)]
    lib.duo_cache_head_view.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(vp),
                                        ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(i64),
                                        ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.duo_gated_attention.argtypes = [ctypes.POINTER(duo_gated_shape), vp, vp, vp, vp, vp, ctypes.c_float, vp]
    lib.duo_cache_head_scales.argtypes = [vp, i32, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(i64)]
    lib.duo_append_row.argtypes = [vp, i32, i32, vp, vp, i64, vp]
    lib.duo_prefill_chunk_row.argtypes = [vp, i32, i32, vp, vp, vp, i64, vp, ctypes.c_float, vp, sz, vp]
    lib.duo_cache_row_len.argtypes = [vp, i32, i32, ctypes.POINTER(i64)]
    lib.duo_cache_reset_row.argtypes = [vp, i32, i32]
    lib.duo_cache_fork_row.argtypes = [vp, i32, i32, i32, vp]
    lib.duo_cache_free_pages.argtypes = [vp, i32, ctypes.POINTER(i64)]
    lib.duo_cache_row_pages.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_int32), i64, ctypes.POINTER(i64)]
    lib.duo_prefill_workspace_bytes.argtypes = [vp, i32, i64, ctypes.POINTER(sz)]
    lib.duo_cache_sync.argtypes = [vp, vp]
    lib.duo_cache_reserve.argtypes = [vp, i32, i64, vp]
    lib.duo_decode_plan.argtypes = [vp, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.duo_rope_apply.argtypes = [ctypes.c_float, i32, i32, i32, i64, i32, ctypes.POINTER(i64), vp, vp, vp]
    lib.duo_cache_free.argtypes = [vp]
    lib.duo_cache_free.restype = None
    lib.duo_last_error.argtypes = []
    lib.duo_last_error.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name not in ("duo_cache_free", "duo_last_error"):
            getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load()
LIB_PATH = _LIB_PATH


def _check(rc: int) -> None:
    if rc != DUO_OK:
        raise DuoError(rc, lib.duo_last_error().decode(errors="replace"))


def _dtype_code(dtype) -> int:
    if dtype in ("bf16", torch.bfloat16):
        return DUO_BF16
    if dtype in ("f32", "fp32", torch.float32):
        return DUO_F32
    raise ValueError(f"unsupported dtype {dtype}")


def _kv_code(kv_format) -> int:
    if kv_format in (None, 0, "native"):
        return DUO_KV_NATIVE
    if kv_format in (1, "fp8"):
        return DUO_KV_FP8
    if kv_format in (2, "int4"):
        return DUO_KV_INT4
    if isinstance(kv_format, int):
        return kv_format  # passed through; the library rejects unknown codes
    raise ValueError(f"unknown kv_format {kv_format}")


def make_config(L, B, n_q, n_kv, d_head, T_cap, sink, recent, dtype, mask, kv_format=None, page_rows=0,
                n_pages=0, rope_theta=0.0):
    """(duo_config, keep-alive mask buffer).  page_rows > 0 stores retrieval
    rows in pages of that many rows, n_pages per layer; rope_theta > 0 turns
    on rotary positions with that base."""
    import numpy as np
    m = torch.from_numpy(np.asarray(mask, dtype=np.uint8).reshape(-1).copy())
    if m.numel() != L * n_kv:
        raise ValueError(f"mask must hold L*n_kv = {L * n_kv} entries, got {m.numel()}")
    buf = (ctypes.c_uint8 * m.numel())(*m.tolist())
    cfg = duo_config(L, B, n_q, n_kv, d_head, int(T_cap), sink, recent, _dtype_code(dtype),
                     ctypes.cast(buf, ctypes.POINTER(ctypes.c_uint8)), _kv_code(kv_format), int(page_rows),
                     int(n_pages), float(rope_theta))
    return cfg, buf


def cache_bytes(L, B, n_q, n_kv, d_head, T_cap, sink, recent, dtype, mask, kv_format=None, page_rows=0, n_pages=0,
                rope_theta=0.0):
    """(arena bytes, workspace bytes, K+V payload bytes) -- host-only size query."""
    cfg, _buf = make_config(L, B, n_q, n_kv, d_head, T_cap, sink, recent, dtype, mask, kv_format, page_rows,
                            n_pages, rope_theta)
    a, w, p = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.duo_cache_bytes(ctypes.byref(cfg), ctypes.byref(a), ctypes.byref(w)))
    _check(lib.duo_cache_payload_bytes(ctypes.byref(cfg), ctypes.byref(p)))
    return a.value, w.value, p.value


def _stream_handle(stream: Optional[torch.cuda.Stream]):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class DuoCache:
    """A mixed retrieval/streaming KV cache in one caller-owned device arena.

    Tensors: K/V inputs [B][n_kv][n][d], queries/outputs [B][n_q][d] (decode)
    or [B][n_q][C][d] (prefill), all contiguous in the cache dtype on the
    cache's device.  kv_format "fp8" stores the K/V rows as FP8 codes with one
    scale per row (bf16 caches with d_head 128).  page_rows > 0 stores the
    retrieval rows in pages (n_pages per layer) that rows take as they grow
    and can share (fork_row).  rope_theta > 0 applies rotary positions (keys
    stored rotated, queries rotated by decode and prefill).  kv_format
    "int4" stores 4-bit codes (two per byte) with one scale per row.
    """

    def __init__(self, L: int, B: int, n_q: int, n_kv: int, d_head: int, T_cap: int, sink: int, recent: int,
                 dtype, mask: Sequence, device="cuda", stream: Optional[torch.cuda.Stream] = None, kv_format=None,
                 page_rows: int = 0, n_pages: int = 0, rope_theta: float = 0.0):
        self.L, self.B, self.n_q, self.n_kv, self.d = L, B, n_q, n_kv, d_head
        self.T_cap, self.S, self.W = int(T_cap), sink, recent
        self.page_rows, self.n_pages = int(page_rows), int(n_pages)
        self.rope_theta = float(rope_theta)
        self.torch_dtype = torch.bfloat16 if _dtype_code(dtype) == DUO_BF16 else torch.float32
        self.kv_format = _kv_code(kv_format)
        self.device = torch.device(device)
        self._cfg, self._mask_buf = make_config(L, B, n_q, n_kv, d_head, T_cap, sink, recent, dtype, mask, kv_format,
                                                page_rows, n_pages, rope_theta)
        import numpy as np
        self.mask = torch.from_numpy(np.asarray(mask, dtype=np.uint8).reshape(L, n_kv).copy())
        a, w = ctypes.c_size_t(), ctypes.c_size_t()
        _check(lib.duo_cache_bytes(ctypes.byref(self._cfg), ctypes.byref(a), ctypes.byref(w)))
        self.arena_bytes, self.workspace_bytes = a.value, w.value
        self.arena = torch.empty(self.arena_bytes, dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(max(self.workspace_bytes, 256), dtype=torch.uint8, device=self.device)
        self._h = ctypes.c_void_p()
        self._free = lib.duo_cache_free  # held so teardown at interpreter exit still finds it
        _check(lib.duo_cache_init(ctypes.byref(self._cfg), ctypes.c_void_p(self.arena.data_ptr()),
                                  self.arena_bytes, _stream_handle(stream), ctypes.byref(self._h)))

    def close(self) -> None:
        """Free the host handle (the arena and workspace tensors stay with
        Python's garbage collector)."""
        h = getattr(self, "_h", None)
        free = getattr(self, "_free", None)
        if h is not None and h.value and free is not None:
            free(h)
        self._h = None

    def __del__(self):
        self.close()

    # ------------------------------------------------------------ checks
    def _chk(self, t: torch.Tensor, shape, name: str):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a tensor")
        if t.device != self.device and not (t.is_cuda and self.device.type == "cuda" and self.device.index is None):
            raise ValueError(f"{name} must be on {self.device}, got {t.device}")
        if t.dtype != self.torch_dtype:
            raise ValueError(f"{name} must be {self.torch_dtype}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    # ------------------------------------------------------------ entry points
    def append(self, layer: int, k: torch.Tensor, v: torch.Tensor, stream=None) -> None:
        n = k.shape[2] if k.dim() == 4 else -1
        self._chk(k, (self.B, self.n_kv, n, self.d), "k")
        self._chk(v, (self.B, self.n_kv, n, self.d), "v")
        _check(lib.duo_append(self._h, layer, ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()), n,
                              _stream_handle(stream)))

    def decode(self, layer: int, q: torch.Tensor, out: Optional[torch.Tensor] = None, scale: Optional[float] = None,
               stream=None) -> torch.Tensor:
        self._chk(q, (self.B, self.n_q, self.d), "q")
        if out is None:
            out = torch.empty_like(q)
        self._chk(out, (self.B, self.n_q, self.d), "out")
        sc = float(self.d ** -0.5 if scale is None else scale)
        _check(lib.duo_decode(self._h, layer, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(out.data_ptr()), sc,
                              ctypes.c_void_p(self.workspace.data_ptr()), self.workspace.numel(),
                              _stream_handle(stream)))
        return out

    def decode_append(self, layer: int, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor,
                      out: Optional[torch.Tensor] = None, scale: Optional[float] = None, stream=None) -> torch.Tensor:
        """Append one token (k, v: [B][n_kv][1][d]) and decode q at its
        position, in one launch (duo_decode_append)."""
        self._chk(k, (self.B, self.n_kv, 1, self.d), "k")
        self._chk(v, (self.B, self.n_kv, 1, self.d), "v")
        self._chk(q, (self.B, self.n_q, self.d), "q")
        if out is None:
            out = torch.empty_like(q)
        self._chk(out, (self.B, self.n_q, self.d), "out")
        sc = float(self.d ** -0.5 if scale is None else scale)
        _check(lib.duo_decode_append(self._h, layer, ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                     ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(out.data_ptr()), sc,
                                     ctypes.c_void_p(self.workspace.data_ptr()), self.workspace.numel(),
                                     _stream_handle(stream)))
        return out

    def prefill_chunk(self, layer: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      out: Optional[torch.Tensor] = None, scale: Optional[float] = None, stream=None) -> torch.Tensor:
        C = q.shape[2] if q.dim() == 4 else -1
        self._chk(q, (self.B, self.n_q, C, self.d), "q")
        self._chk(k, (self.B, self.n_kv, C, self.d), "k")
        self._chk(v, (self.B, self.n_kv, C, self.d), "v")
        if out is None:
            out = torch.empty_like(q)
        self._chk(out, (self.B, self.n_q, C, self.d), "out")
        sc = float(self.d ** -0.5 if scale is None else scale)
        self._ensure_prefill_workspace(self.B, C)
        _check(lib.duo_prefill_chunk(self._h, layer, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                     ctypes.c_void_p(v.data_ptr()), C, ctypes.c_void_p(out.data_ptr()), sc,
                                     ctypes.c_void_p(self.workspace.data_ptr()), self.workspace.numel(),
                                     _stream_handle(stream)))
        return out

    def sync(self, stream=None) -> None:
        """Host-side token counts from the device-side ones (after replays of
        captured steps); raises DuoError(DUO_ECAPACITY) if a replayed step
        found no room for its tokens."""
        _check(lib.duo_cache_sync(self._h, _stream_handle(stream)))

    def reserve(self, layer: int, n_tokens: int, stream=None) -> None:
        """Room for n_tokens more tokens in every row of `layer` (pages of a
        paged layer), for replays of captured steps."""
        _check(lib.duo_cache_reserve(self._h, layer, int(n_tokens), _stream_handle(stream)))

    def seq_len(self, layer: int) -> int:
        """Token count of the layer's rows (they must hold equal counts)."""
        x = ctypes.c_int64()
        _check(lib.duo_cache_seq_len(self._h, layer, ctypes.byref(x)))
        return x.value

    def row_len(self, layer: int, row: int) -> int:
        x = ctypes.c_int64()
        _check(lib.duo_cache_row_len(self._h, layer, row, ctypes.byref(x)))
        return x.value

    def _ensure_prefill_workspace(self, rows: int, C: int) -> None:
        """Grow the workspace tensor to what a prefill of `rows` rows and C
        tokens needs (rotary positions need room for the rotated chunk)."""
        if C < 1:
            return
        need = ctypes.c_size_t()
        _check(lib.duo_prefill_workspace_bytes(self._h, rows, C, ctypes.byref(need)))
        if need.value > self.workspace.numel():
            self.workspace = torch.empty(need.value, dtype=torch.uint8, device=self.device)

    def reset_row(self, layer: int, row: int) -> None:
        """Empty batch row `row` of `layer` (its pages return to the pool)."""
        _check(lib.duo_cache_reset_row(self._h, layer, row))

    def fork_row(self, layer: int, src_row: int, dst_row: int, stream=None) -> None:
        """Make empty row dst_row a copy of row src_row (paged: sharing its full pages)."""
        _check(lib.duo_cache_fork_row(self._h, layer, src_row, dst_row, _stream_handle(stream)))

    def decode_plan(self, layer: int) -> tuple:
        """(work items, shared items) a decode of `layer` would launch now."""
        n, sh = ctypes.c_int32(), ctypes.c_int32()
        _check(lib.duo_decode_plan(self._h, layer, ctypes.byref(n), ctypes.byref(sh)))
        return n.value, sh.value

    def free_pages(self, layer: int) -> int:
        x = ctypes.c_int64()
        _check(lib.duo_cache_free_pages(self._h, layer, ctypes.byref(x)))
        return x.value

    def row_pages(self, layer: int, row: int) -> list:
        """Page numbers batch row `row` of a paged layer holds, in position order."""
        n = ctypes.c_int64()
        _check(lib.duo_cache_row_pages(self._h, layer, row, None, 0, ctypes.byref(n)))
        buf = (ctypes.c_int32 * max(n.value, 1))()
        _check(lib.duo_cache_row_pages(self._h, layer, row, buf, n.value, ctypes.byref(n)))
        return list(buf[: n.value])

    def append_row(self, layer: int, row: int, k: torch.Tensor, v: torch.Tensor, stream=None) -> None:
        """Append n tokens (k, v: [1][n_kv][n][d]) to batch row `row` alone."""
        n = k.shape[2] if k.dim() == 4 else -1
        self._chk(k, (1, self.n_kv, n, self.d), "k")
        self._chk(v, (1, self.n_kv, n, self.d), "v")
        _check(lib.duo_append_row(self._h, layer, row, ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                  n, _stream_handle(stream)))

    def prefill_chunk_row(self, layer: int, row: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          out: Optional[torch.Tensor] = None, scale: Optional[float] = None, stream=None) -> torch.Tensor:
        """Chunked prefill of batch row `row` alone (q: [1][n_q][C][d], k, v: [1][n_kv][C][d])."""
        C = q.shape[2] if q.dim() == 4 else -1
        self._chk(q, (1, self.n_q, C, self.d), "q")
        self._chk(k, (1, self.n_kv, C, self.d), "k")
        self._chk(v, (1, self.n_kv, C, self.d), "v")
        if out is None:
            out = torch.empty_like(q)
        self._chk(out, (1, self.n_q, C, self.d), "out")
        sc = float(self.d ** -0.5 if scale is None else scale)
        self._ensure_prefill_workspace(1, C)
        _check(lib.duo_prefill_chunk_row(self._h, layer, row, ctypes.c_void_p(q.data_ptr()),
                                         ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()), C,
                                         ctypes.c_void_p(out.data_ptr()), sc, ctypes.c_void_p(self.workspace.data_ptr()),
                                         self.workspace.numel(), _stream_handle(stream)))
        return out

    def head_view(self, layer: int, kv_head: int) -> dict:
        """Device addresses and strides of one KV head's rows (for layout checks)."""
        ir = ctypes.c_int()
        kb, vb, pp = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        ns, rb, hs, ps = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib.duo_cache_head_view(self._h, layer, kv_head, ctypes.byref(ir), ctypes.byref(kb), ctypes.byref(vb),
                                       ctypes.byref(pp), ctypes.byref(ns), ctypes.byref(rb), ctypes.byref(hs),
                                       ctypes.byref(ps)))
        return dict(is_retrieval=bool(ir.value), k_base=kb.value, v_base=vb.value, pos=pp.value,
                    n_slots=ns.value, row_bytes=rb.value, head_stride_bytes=hs.value, pos_stride=ps.value)

    def head_scales(self, layer: int, kv_head: int):
        """FP8 caches: (K scales [B][n_slots], V scales) of one KV head copied to
        the host as float32 tensors; (None, None) for a native cache."""
        ks, vs, st = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_int64()
        _check(lib.duo_cache_head_scales(self._h, layer, kv_head, ctypes.byref(ks), ctypes.byref(vs), ctypes.byref(st)))
        if not ks.value:
            return None, None
        hv = self.head_view(layer, kv_head)
        base = self.arena.data_ptr()
        if self._paged_head(hv):
            return tuple(self._gather_pages(layer, ptr - base, st.value * 4, 4).view(torch.float32)
                         .reshape(self.B, -1) for ptr in (ks.value, vs.value))
        rows = hv["n_slots"]
        out = []
        for ptr in (ks.value, vs.value):
            off = ptr - base
            seg = torch.stack([self.arena[off + b * st.value * 4: off + (b * st.value + rows) * 4] for b in range(self.B)])
            out.append(seg.cpu().view(torch.float32).reshape(self.B, rows))
        return out[0], out[1]

    def _paged_head(self, hv: dict) -> bool:
        return bool(hv["is_retrieval"]) and self.page_rows > 0

    def _gather_pages(self, layer: int, off: int, page_stride: int, row_bytes: int) -> torch.Tensor:
        """Bytes of one paged head's positions 0 .. ceil(T_cap / page_rows) * page_rows - 1
        for every batch row, [B][positions * row_bytes] on the host, read through
        the row's page table (positions on no page read as zero bytes)."""
        P = self.page_rows
        n_pos = -(-self.T_cap // P) * P
        out = torch.zeros(self.B, n_pos * row_bytes, dtype=torch.uint8)
        for b in range(self.B):
            for i, pg in enumerate(self.row_pages(layer, b)):
                src = off + pg * page_stride
                out[b, i * P * row_bytes:(i + 1) * P * row_bytes] = self.arena[src: src + P * row_bytes].cpu()
        return out

    def read_head(self, layer: int, kv_head: int):
        """Copy one KV head's slots to the host: (K [B][n_slots][d], V, pos [B][n_slots] or None).
        The bytes come from the arena tensor by offset (a plain device copy).
        FP8 caches give the codes as uint8.  A paged retrieval head gives its
        positions 0 .. ceil(T_cap / page_rows) * page_rows - 1 read through each
        row's page table (positions on no page read as zeros)."""
        hv = self.head_view(layer, kv_head)
        base = self.arena.data_ptr()
        es = 2 if self.torch_dtype == torch.bfloat16 else 4
        if self.kv_format in (DUO_KV_FP8, DUO_KV_INT4):
            es = 1  # codes as bytes (INT4: two per byte, d / 2 per row)
        width = hv["row_bytes"] // es
        if self._paged_head(hv):
            kv = [self._gather_pages(layer, hv[key] - base, hv["head_stride_bytes"], hv["row_bytes"])
                  .view(torch.uint8 if es == 1 else self.torch_dtype).reshape(self.B, -1, width)
                  for key in ("k_base", "v_base")]
            return kv[0], kv[1], None
        rows = hv["n_slots"]
        out = []
        for key in ("k_base", "v_base"):
            off = hv[key] - base
            seg = torch.stack([self.arena[off + b * hv["head_stride_bytes"]: off + b * hv["head_stride_bytes"]
                                          + rows * hv["row_bytes"]] for b in range(self.B)])
            out.append(seg.cpu().view(torch.uint8 if es == 1 else self.torch_dtype).reshape(self.B, rows, width))
        pos = None
        if hv["pos"]:
            off = hv["pos"] - base
            seg = torch.stack([self.arena[off + b * hv["pos_stride"] * 4: off + (b * hv["pos_stride"] + rows) * 4]
                               for b in range(self.B)])
            pos = seg.cpu().view(torch.int32).reshape(self.B, rows)
        assert es in (1, 2, 4)
        return out[0], out[1], pos


def gated_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor, sink: int, recent: int,
                    out: Optional[torch.Tensor] = None, scale: Optional[float] = None, stream=None) -> torch.Tensor:
    """Head-gated forward (duo_gated_attention): per query head,
    alpha[kv head] * causal attention + (1 - alpha[kv head]) * sink + window
    attention over one whole sequence.  q: [B][n_q][N][d]; k, v: [B][n_kv][N][d]
    (bf16 or float32, contiguous, one device); alpha: float32 [n_kv] on the
    same device."""
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B][n_q][N][d]; k and v [B][n_kv][N][d]")
    B, n_q, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    n_kv = k.shape[1]
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k and v must share one dtype")
    if alpha.dtype != torch.float32 or tuple(alpha.shape) != (n_kv,):
        raise ValueError(f"alpha must be float32 [{n_kv}]")
    if any(t.device != q.device for t in (k, v, alpha)):
        raise ValueError("q, k, v and alpha must be on one device")
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    shape = duo_gated_shape(B, n_q, n_kv, d, N, sink, recent, _dtype_code(q.dtype))
    sc = float(d ** -0.5 if scale is None else scale)
    _check(lib.duo_gated_attention(ctypes.byref(shape), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                   ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(alpha.data_ptr()),
                                   ctypes.c_void_p(out.data_ptr()), sc, _stream_handle(stream)))
    return out


def rope_apply(x: torch.Tensor, p0, theta: float, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Rotary position embedding as the cache applies it (duo_rope_apply):
    row c of x[b][h] rotated at position p0[b] + c with base theta.
    x: contiguous device [B][H][C][d], bf16 or float32; p0: B ints."""
    if not isinstance(x, torch.Tensor) or not x.is_cuda or not x.is_contiguous() or x.dim() != 4:
        raise ValueError("x must be a contiguous device tensor [B][H][C][d]")
    B, Hh, C, d = x.shape
    p = [int(v) for v in p0]
    if len(p) != B:
        raise ValueError(f"p0 must hold {B} positions")
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or out.device != x.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x")
    arr = (ctypes.c_int64 * B)(*p)
    _check(lib.duo_rope_apply(float(theta), _dtype_code(x.dtype), B, Hh, C, d, arr, ctypes.c_void_p(x.data_ptr()),
                              ctypes.c_void_p(out.data_ptr()), _stream_handle(stream)))
    return out
