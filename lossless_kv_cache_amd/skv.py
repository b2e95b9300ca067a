"""ctypes binding of libskv (argument marshalling only).

Torch tensors provide device memory, and the current torch stream provides
the HIP stream. Every step of the coding runs in the library's HIP
kernels. There is no CPU fallback: a missing library or GPU raises.
"""
from __future__ import annotations

import atexit
import ctypes
import hashlib
import os
import sys
import weakref

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libskv.so")

ABI_VERSION = 1
BF16, E4M3, INT16 = 1, 2, 3
RESIDUAL, CHECKERBOARD, RESIDUAL_EXP, CHECKERBOARD_MAP = 0, 1, 2, 3
OK, ERR_ARG, ERR_SHAPE, ERR_CAPACITY, ERR_CORRUPT, ERR_TABLES, ERR_DEVICE, ERR_NOMEM = 0, -1, -2, -3, -4, -5, -6, -7
ERR_BUSY = -8
BLOCK_TOKENS = 128


class SkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().skv_strerror(status).decode()} ({status})")


class Shape(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("dtype", ctypes.c_uint32), ("mode", ctypes.c_uint32),
                ("layers", ctypes.c_uint32), ("kv", ctypes.c_uint32), ("tokens", ctypes.c_uint32),
                ("channels", ctypes.c_uint32)]


class NbrMap(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_uint32), ("shift_h", ctypes.c_uint32), ("shift_m", ctypes.c_uint32),
                ("V", ctypes.c_void_p), ("U", ctypes.c_void_p)]


class StoreHit(ctypes.Structure):
    _fields_ = [("entry", ctypes.c_uint64), ("matched_blocks", ctypes.c_uint32), ("entry_blocks", ctypes.c_uint32),
                ("container", ctypes.c_void_p), ("container_bytes", ctypes.c_uint64)]


class StoreInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("arena_bytes", "used_bytes", "largest_free", "container_bytes",
                                               "entries", "pinned", "inserts", "evictions", "hits", "misses",
                                               "hit_blocks")]


_lib = None


def lib():
    """Load libskv.so (built in-tree by lossless_kv_cache_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m lossless_kv_cache_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32
        psz = ctypes.POINTER(sz)
        sp = ctypes.POINTER(Shape)
        L.skv_version.restype = u32
        L.skv_version.argtypes = []
        L.skv_strerror.restype = ctypes.c_char_p
        L.skv_strerror.argtypes = [ctypes.c_int]
        L.skv_fit_tables.restype = ctypes.c_int
        L.skv_fit_tables.argtypes = [sp, vp, vp, u32, ctypes.POINTER(vp), psz]
        L.skv_fit_tables_map.restype = ctypes.c_int
        L.skv_fit_tables_map.argtypes = [sp, vp, vp, u32, ctypes.POINTER(NbrMap), ctypes.POINTER(vp), psz]
        L.skv_load_tables.restype = ctypes.c_int
        L.skv_load_tables.argtypes = [vp, sz, ctypes.POINTER(vp)]
        L.skv_encode.restype = ctypes.c_int
        L.skv_encode.argtypes = [vp, sp, vp, vp, vp, sz, psz, vp, psz, vp]
        L.skv_encode_workspace.restype = ctypes.c_int
        L.skv_encode_workspace.argtypes = [sp, ctypes.c_uint64, psz, ctypes.POINTER(u32)]
        L.skv_encode_noalloc.restype = ctypes.c_int
        L.skv_encode_noalloc.argtypes = [vp, sp, vp, vp, vp, sz, psz, vp]
        L.skv_decode.restype = ctypes.c_int
        L.skv_decode.argtypes = [vp, vp, sz, vp, vp, sz, vp, psz, vp]
        L.skv_decode_range.restype = ctypes.c_int
        L.skv_decode_range.argtypes = [vp, vp, sz, u32, u32, vp, vp, sz, vp, psz, vp]
        L.skv_free.restype = None
        L.skv_transfer.argtypes = [vp, sp, u32, vp, vp, vp, sz, psz, ctypes.POINTER(ctypes.c_uint64), vp, vp, sz,
                                   vp, psz, vp]
        L.skv_transfer.restype = ctypes.c_int
        L.skv_free.argtypes = [vp]
        L.skv_kernel_timing.restype = ctypes.c_int
        L.skv_kernel_timing.argtypes = [ctypes.c_int]
        u64 = ctypes.c_uint64
        pu64 = ctypes.POINTER(u64)
        L.skv_store_create.restype = ctypes.c_int
        L.skv_store_create.argtypes = [vp, u64, ctypes.POINTER(vp)]
        L.skv_store_destroy.restype = None
        L.skv_store_destroy.argtypes = [vp]
        L.skv_store_reserve.restype = ctypes.c_int
        L.skv_store_reserve.argtypes = [vp, vp, u32, u64, pu64, ctypes.POINTER(vp)]
        L.skv_store_commit.restype = ctypes.c_int
        L.skv_store_commit.argtypes = [vp, u64, u64]
        L.skv_store_abort.restype = ctypes.c_int
        L.skv_store_abort.argtypes = [vp, u64]
        L.skv_store_put.restype = ctypes.c_int
        L.skv_store_put.argtypes = [vp, vp, u32, vp, sp, vp, vp, vp, psz, vp, pu64, pu64]
        L.skv_store_lookup.restype = ctypes.c_int
        L.skv_store_lookup.argtypes = [vp, vp, u32, ctypes.POINTER(StoreHit)]
        L.skv_store_release.restype = ctypes.c_int
        L.skv_store_release.argtypes = [vp, u64]
        L.skv_store_decode.restype = ctypes.c_int
        L.skv_store_decode.argtypes = [vp, vp, u64, u32, u32, vp, vp, sz, vp, psz, vp]
        L.skv_store_erase.restype = ctypes.c_int
        L.skv_store_erase.argtypes = [vp, u64]
        L.skv_store_stats.restype = ctypes.c_int
        L.skv_store_stats.argtypes = [vp, ctypes.POINTER(StoreInfo)]
        L.skv_kernel_times.restype = ctypes.c_int
        L.skv_kernel_times.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float), ctypes.c_int]
        if L.skv_version() != ABI_VERSION:
            raise RuntimeError("libskv ABI version mismatch")
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != OK:
        raise SkvError(rc, what)


def make_shape(dtype: int, mode: int, layers: int, kv: int, tokens: int, channels: int) -> Shape:
    return Shape(ABI_VERSION, dtype, mode, layers, kv, tokens, channels)


# Every open blob, so that the exit hook below can release them.
_live_tables = weakref.WeakSet()


class Tables:
    """A library-owned table blob (host), uploaded to each device on first use."""

    def __init__(self, ptr: int, nbytes: int):
        self._ptr = ctypes.c_void_p(ptr)
        self.nbytes = nbytes
        _live_tables.add(self)
        b = self.bytes()[:64]
        self.dtype, self.mode = b[6], b[7]
        self.layers = int.from_bytes(b[12:16], "little")
        self.kv = int.from_bytes(b[16:20], "little")
        self.channels = int.from_bytes(b[20:24], "little")

    @property
    def ptr(self):
        return self._ptr

    def bytes(self) -> bytes:
        return ctypes.string_at(self._ptr, self.nbytes)

    def shape(self, tokens: int) -> Shape:
        return make_shape(self.dtype, self.mode, self.layers, self.kv, tokens, self.channels)

    def close(self):
        if self._ptr and self._ptr.value and _lib is not None:
            _lib.skv_free(self._ptr)
        self._ptr = ctypes.c_void_p(None)

    def __del__(self, _finalizing=sys.is_finalizing):
        # During interpreter shutdown the exit hook has already released every
        # blob; a finalizer running later (module globals may be gone by then)
        # must not make HIP calls.
        if _finalizing():
            return
        try:
            self.close()
        except Exception:
            pass


@atexit.register
def _release_tables():
    """Release every open blob and its device tables at interpreter exit,
    while torch and the HIP runtime are still whole: exit hooks run before
    module teardown, and long before the runtime's own static destructors."""
    for t in list(_live_tables):
        try:
            t.close()
        except Exception:
            pass


def _host_ptr(a) -> tuple[int, object]:
    if isinstance(a, torch.Tensor):
        if a.is_cuda:
            raise ValueError("calibration arrays are host arrays")
        a = a.contiguous()
        return a.data_ptr(), a
    a = np.ascontiguousarray(a)
    return a.ctypes.data, a


def fit_tables(dtype: int, mode: int, layers: int, kv: int, channels: int, calib_target, calib_aux,
               calib_tokens: int) -> Tables:
    """Fit the tables once from host calibration arrays (see skv_fit_tables)."""
    s = make_shape(dtype, mode, layers, kv, 0, channels)
    pt, keep_t = _host_ptr(calib_target)
    pa, keep_a = _host_ptr(calib_aux)
    out, nb = ctypes.c_void_p(), ctypes.c_size_t()
    _check(lib().skv_fit_tables(ctypes.byref(s), pt, pa, calib_tokens, ctypes.byref(out), ctypes.byref(nb)),
           "skv_fit_tables")
    return Tables(out.value, nb.value)


def fit_tables_map(channels: int, calib_coef, calib_G, calib_tokens: int, V, U, shift_h: int,
                   shift_m: int) -> Tables:
    """Tables of the checkerboard mode with a decoded-neighbour map (see
    skv_fit_tables_map): V int8 [rank][2 * channels], U int8 [channels][rank]."""
    s = make_shape(INT16, CHECKERBOARD_MAP, 1, 1, 0, channels)
    v = np.ascontiguousarray(V, dtype=np.int8)
    u = np.ascontiguousarray(U, dtype=np.int8)
    if v.ndim != 2 or u.shape != (channels, v.shape[0]) or v.shape[1] != 2 * channels:
        raise ValueError("V must be [rank][2 * channels] and U [channels][rank]")
    m = NbrMap(v.shape[0], shift_h, shift_m, v.ctypes.data, u.ctypes.data)
    pt, keep_t = _host_ptr(calib_coef)
    pa, keep_a = _host_ptr(calib_G)
    out, nb = ctypes.c_void_p(), ctypes.c_size_t()
    _check(lib().skv_fit_tables_map(ctypes.byref(s), pt, pa, calib_tokens, ctypes.byref(m), ctypes.byref(out),
                                    ctypes.byref(nb)), "skv_fit_tables_map")
    return Tables(out.value, nb.value)


def load_tables(blob: bytes) -> Tables:
    buf = ctypes.create_string_buffer(bytes(blob), len(blob))
    out = ctypes.c_void_p()
    _check(lib().skv_load_tables(buf, len(blob), ctypes.byref(out)), "skv_load_tables")
    return Tables(out.value, len(blob))


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def elem_bytes(dtype: int) -> int:
    return 1 if dtype == E4M3 else 2


def is_checkerboard(mode: int) -> bool:
    return mode in (CHECKERBOARD, CHECKERBOARD_MAP)


def _layout(tables: "Tables", tokens: int) -> tuple:
    if is_checkerboard(tables.mode):
        return (tokens, tables.channels)
    return (tables.layers, tables.kv, tokens, tables.channels)


def _check_cache(t: torch.Tensor, name: str, tables: "Tables", tokens: int) -> int:
    """A contiguous device array in the tables' layout with `tokens` tokens and
    elements of the tables' width; the kernels read or write exactly that many
    bytes, so anything else is refused here before the library is called."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a device tensor")
    eb = elem_bytes(tables.dtype)
    if t.element_size() != eb:
        raise ValueError(f"{name}: {t.element_size()}-byte elements, the tables code {eb}-byte elements")
    want = _layout(tables, tokens)
    if tuple(t.shape) != want:
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {want}")
    return _dev(t, name)


def _decode_buffers(aux: torch.Tensor, out: torch.Tensor, tables: "Tables", tokens=None) -> tuple[int, int, int]:
    """Decode: the predictor (or G) in the tables' layout (with `tokens`
    tokens when given) and an output of the same element width.  The library
    checks the capacity it is given against the container header; the
    capacity passed is the smaller of the output's and the predictor's sizes,
    so neither is read or written past its end.  Returns (aux, out, capacity)."""
    nd = len(_layout(tables, 0))
    if not isinstance(aux, torch.Tensor) or aux.dim() != nd:
        raise ValueError(f"aux must be a {nd}-D device tensor in the tables' layout")
    if tokens is None:
        tokens = aux.shape[0] if is_checkerboard(tables.mode) else aux.shape[2]
    if not isinstance(out, torch.Tensor) or out.element_size() != aux.element_size():
        raise ValueError(f"out must be a device tensor of {aux.element_size()}-byte elements")
    pa = _check_cache(aux, "aux", tables, tokens)
    po = _dev(out, "out")
    cap = min(out.numel() * out.element_size(), aux.numel() * aux.element_size())
    return pa, po, cap


def tokens_of(tables: Tables, target: torch.Tensor) -> int:
    if is_checkerboard(tables.mode):
        if target.dim() != 2:
            raise ValueError("checkerboard arrays are [tokens][channels]")
        return target.shape[0]
    if target.dim() != 4:
        raise ValueError("residual arrays are [layers][kv][tokens][channels]")
    return target.shape[2]


def encode_workspace(tables: Tables, tokens: int, max_bytes: int = 0) -> tuple[int, int]:
    """(workspace bytes, passes) of an encode of `tokens` tokens within
    max_bytes of workspace (0: a single pass)."""
    shape = tables.shape(tokens)
    wb, ps = ctypes.c_size_t(), ctypes.c_uint32()
    _check(lib().skv_encode_workspace(ctypes.byref(shape), max_bytes, ctypes.byref(wb), ctypes.byref(ps)),
           "skv_encode_workspace")
    return wb.value, ps.value


class Encoder:
    """Encodes repeatedly with one set of tables, reusing its buffers; with
    max_work_bytes the workspace stays within that budget (the cache is then
    coded in passes)."""

    def __init__(self, tables: Tables, tokens: int, device=None, max_work_bytes: int = 0):
        self.tables = tables
        self.shape = tables.shape(tokens)
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        ob, wb = ctypes.c_size_t(), ctypes.c_size_t()
        _check(lib().skv_encode(tables.ptr, ctypes.byref(self.shape), None, None, None, 0, ctypes.byref(ob), None,
                                ctypes.byref(wb), None), "skv_encode(size query)")
        work_bytes, self.passes = encode_workspace(tables, tokens, max_work_bytes)
        self.out = torch.empty(ob.value, dtype=torch.uint8, device=dev)
        self.work = torch.empty(work_bytes, dtype=torch.uint8, device=dev)

    def __call__(self, target: torch.Tensor, aux: torch.Tensor) -> torch.Tensor:
        """Returns a view of the container (valid until the next call)."""
        pt = _check_cache(target, "target", self.tables, self.shape.tokens)
        pa = _check_cache(aux, "aux", self.tables, self.shape.tokens)
        if target.device != self.out.device or aux.device != self.out.device:
            raise ValueError("target and aux must be on the encoder's device")
        ob = ctypes.c_size_t()
        wb = ctypes.c_size_t(self.work.numel())
        rc = lib().skv_encode(self.tables.ptr, ctypes.byref(self.shape), pt, pa,
                              self.out.data_ptr(), self.out.numel(), ctypes.byref(ob), self.work.data_ptr(),
                              ctypes.byref(wb), _stream())
        _check(rc, "skv_encode")
        return self.out[: ob.value]


def encode(tables: Tables, target: torch.Tensor, aux: torch.Tensor) -> torch.Tensor:
    """Encode a device cache; returns a fresh uint8 device tensor (the container)."""
    enc = Encoder(tables, tokens_of(tables, target), target.device)
    return enc(target, aux).clone()


NOALLOC_WORK_BYTES = 64 << 20


def encode_noalloc(tables: Tables, target: torch.Tensor, aux: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """Encode into the caller's uint8 device tensor `out` through the entry
    point that allocates nothing (its workspace is the library's fixed
    per-device array); returns the view of `out` that holds the container.
    The tables must have been used on this device before (see
    skv_encode_noalloc)."""
    shape = tables.shape(tokens_of(tables, target))
    pt = _check_cache(target, "target", tables, shape.tokens)
    pa = _check_cache(aux, "aux", tables, shape.tokens)
    po = _check_container(out)
    ob = ctypes.c_size_t()
    _check(lib().skv_encode_noalloc(tables.ptr, ctypes.byref(shape), pt, pa, po, out.numel(), ctypes.byref(ob),
                                    _stream()), "skv_encode_noalloc")
    return out[: ob.value]


def encode_noalloc_bound(tables: Tables, tokens: int) -> int:
    """Container bound for encode_noalloc (raises SkvError(ERR_SHAPE) for a
    checkerboard shape whose single-pass workspace exceeds the fixed array)."""
    shape = tables.shape(tokens)
    ob = ctypes.c_size_t()
    _check(lib().skv_encode_noalloc(tables.ptr, ctypes.byref(shape), None, None, None, 0, ctypes.byref(ob), None),
           "skv_encode_noalloc(size query)")
    return ob.value


_decode_work = {}


def _check_container(container: torch.Tensor) -> int:
    ptr = _dev(container, "container")
    if container.element_size() != 1:
        raise ValueError("container must be a uint8 device tensor")
    return ptr


def decode_into(tables: Tables, container: torch.Tensor, aux: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    pc = _check_container(container)
    pa, po, cap = _decode_buffers(aux, out, tables)
    key = container.device
    work = _decode_work.get(key)
    if work is None:
        wb = ctypes.c_size_t()
        _check(lib().skv_decode(tables.ptr, None, 0, None, None, 0, None, ctypes.byref(wb), None), "skv_decode(size)")
        work = _decode_work[key] = torch.empty(wb.value, dtype=torch.uint8, device=key)
    wb = ctypes.c_size_t(work.numel())
    rc = lib().skv_decode(tables.ptr, pc, container.numel(), pa, po, cap, work.data_ptr(), ctypes.byref(wb),
                          _stream())
    _check(rc, "skv_decode")
    return out


def container_tokens(container: torch.Tensor) -> int:
    """Tokens per slab in a container's header (a small device-to-host read)."""
    _check_container(container)
    if container.numel() < 64:
        raise SkvError(ERR_CORRUPT, "container header")
    return int.from_bytes(container[20:24].cpu().numpy().tobytes(), "little")


def range_aux_tokens(tables: Tables, tokens: int, token_begin: int, token_end: int) -> int:
    """Tokens of side input / predictor a range decode reads: the range, and
    for a checkerboard range that stops before the container's `tokens`, the
    256-token block after it (its even tokens are decoded for the range's
    last odd token)."""
    if is_checkerboard(tables.mode):
        return min(tokens, token_end + 256) - token_begin
    return token_end - token_begin


def _range_buffers(tables: Tables, tokens: int | None, token_begin: int, token_end: int, aux, out, what: str,
                   rules_only: bool = False):
    """The library's range rules (same status), then the buffers of the
    range: aux with range_aux_tokens tokens, out of the range's elements."""
    cb = is_checkerboard(tables.mode)
    blk = 256 if cb else 128
    if (not 0 <= token_begin < token_end or token_begin % blk or token_end % blk or
            (tokens is not None and token_end > tokens)):
        raise SkvError(ERR_SHAPE, what)
    if rules_only:
        return None
    if not cb:
        return _decode_buffers(aux, out, tables, token_end - token_begin)
    pa = _check_cache(aux, "aux", tables, range_aux_tokens(tables, tokens, token_begin, token_end))
    if not isinstance(out, torch.Tensor) or out.element_size() != 2:
        raise ValueError("out must be a device tensor of 2-byte elements")
    po = _dev(out, "out")
    cap = min(out.numel(), (token_end - token_begin) * tables.channels) * 2
    return pa, po, cap


def _range_work(tables: Tables, token_begin: int, token_end: int, device) -> torch.Tensor:
    wb = ctypes.c_size_t()
    _check(lib().skv_decode_range(tables.ptr, None, 0, token_begin, token_end, None, None, 0, None, ctypes.byref(wb),
                                  None), "skv_decode_range(size)")
    work = _decode_work.get(device)
    if work is None or work.numel() < wb.value:
        _decode_work[device] = None
        work = _decode_work[device] = torch.empty(wb.value, dtype=torch.uint8, device=device)
    return work


def decode_range_into(tables: Tables, container: torch.Tensor, token_begin: int, token_end: int, aux: torch.Tensor,
                      out: torch.Tensor) -> torch.Tensor:
    """Decode tokens [token_begin, token_end) of every slab; out holds that
    range, aux range_aux_tokens(...) tokens from token_begin."""
    _range_buffers(tables, None, token_begin, token_end, None, None, "skv_decode_range", rules_only=True)
    pc = _check_container(container)
    T = container_tokens(container) if is_checkerboard(tables.mode) else None
    pa, po, cap = _range_buffers(tables, T, token_begin, token_end, aux, out, "skv_decode_range")
    work = _range_work(tables, token_begin, token_end, container.device)
    wb = ctypes.c_size_t(work.numel())
    rc = lib().skv_decode_range(tables.ptr, pc, container.numel(), token_begin, token_end, pa, po, cap,
                                work.data_ptr(), ctypes.byref(wb), _stream())
    _check(rc, "skv_decode_range")
    return out


def decode_range(tables: Tables, container: torch.Tensor, token_begin: int, token_end: int,
                 aux: torch.Tensor) -> torch.Tensor:
    """Decode a token range against its predictor (or side input); returns the range's reconstruction."""
    _range_buffers(tables, None, token_begin, token_end, None, None, "skv_decode_range", rules_only=True)
    out = torch.empty(_layout(tables, token_end - token_begin), dtype=aux.dtype, device=aux.device)
    return decode_range_into(tables, container, token_begin, token_end, aux, out)


class Transfer:
    """Chunked encode -> host -> decode pipeline with reusable buffers: a
    device workspace and a page-locked host wire buffer sized for the bound."""

    def __init__(self, tables: Tables, tokens: int, layers_per_chunk: int, device=None):
        self.tables = tables
        self.shape = tables.shape(tokens)
        self.layers_per_chunk = layers_per_chunk
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        wire, wb = ctypes.c_size_t(), ctypes.c_size_t()
        _check(lib().skv_transfer(tables.ptr, ctypes.byref(self.shape), layers_per_chunk, None, None, None, 0,
                                  ctypes.byref(wire), None, None, None, 0, None, ctypes.byref(wb), None),
               "skv_transfer(size query)")
        self.n_chunks = -(-self.shape.layers // layers_per_chunk)
        self.work = torch.empty(wb.value, dtype=torch.uint8, device=dev)
        self.wire = torch.empty(wire.value, dtype=torch.uint8, pin_memory=True)
        self.offsets = (ctypes.c_uint64 * (self.n_chunks + 1))()

    def __call__(self, target: torch.Tensor, aux_send: torch.Tensor, aux_recv: torch.Tensor,
                 out: torch.Tensor) -> tuple[torch.Tensor, list[int]]:
        """Moves target through the pipeline into out; returns (wire bytes view, chunk offsets)."""
        T = self.shape.tokens
        pt = _check_cache(target, "target", self.tables, T)
        ps = _check_cache(aux_send, "aux_send", self.tables, T)
        pr = _check_cache(aux_recv, "aux_recv", self.tables, T)
        po = _check_cache(out, "out", self.tables, T)
        nbytes = ctypes.c_size_t()
        wb = ctypes.c_size_t(self.work.numel())
        rc = lib().skv_transfer(self.tables.ptr, ctypes.byref(self.shape), self.layers_per_chunk, pt, ps,
                                self.wire.data_ptr(), self.wire.numel(), ctypes.byref(nbytes), self.offsets, pr, po,
                                out.numel() * out.element_size(), self.work.data_ptr(), ctypes.byref(wb), _stream())
        _check(rc, "skv_transfer")
        return self.wire[: nbytes.value], list(self.offsets)


def transfer(tables: Tables, target: torch.Tensor, aux_send: torch.Tensor, aux_recv: torch.Tensor,
             layers_per_chunk: int) -> tuple[torch.Tensor, torch.Tensor, list[int]]:
    """Move a residual-mode cache through the pipeline; returns (reconstruction, wire bytes, chunk offsets)."""
    tr = Transfer(tables, tokens_of(tables, target), layers_per_chunk, target.device)
    out = torch.empty_like(aux_recv)
    wire, offsets = tr(target, aux_send, aux_recv, out)
    return out, wire.clone(), offsets


def kernel_timing(enable: bool) -> None:
    """Enable per-kernel HIP-event timing of the following encode/decode calls."""
    _check(lib().skv_kernel_timing(1 if enable else 0), "skv_kernel_timing")


def kernel_times() -> list[tuple[str, float]]:
    """(kernel name, milliseconds) of the last encode/decode call."""
    cap = 16
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    n = lib().skv_kernel_times(names, ms, cap)
    return [(names[i].decode(), float(ms[i])) for i in range(n)]


def decode(tables: Tables, container: torch.Tensor, aux: torch.Tensor) -> torch.Tensor:
    """Decode a container against the predictor (or G); returns a tensor shaped like aux."""
    out = torch.empty_like(aux)
    return decode_into(tables, container, aux, out)


# ------------------------------------------------------------------ prefix-cache store
def block_hashes(token_ids, block: int = BLOCK_TOKENS) -> np.ndarray:
    """Chained 64-bit hashes of the whole blocks of a token-id sequence: the
    hash of block b covers tokens [0, block * (b + 1)) (BLAKE2b of the
    previous block's hash and the block's ids as int64), so two sequences
    share their first m hashes exactly when they share their first m blocks."""
    ids = np.ascontiguousarray(np.asarray(token_ids, dtype=np.int64).reshape(-1))
    out = np.empty(len(ids) // block, dtype=np.uint64)
    h = b""
    for b in range(len(out)):
        h = hashlib.blake2b(h + ids[b * block:(b + 1) * block].tobytes(), digest_size=8).digest()
        out[b] = int.from_bytes(h, "little")
    return out


def _hash_arg(hashes) -> tuple[int, int, np.ndarray]:
    h = np.ascontiguousarray(np.asarray(hashes, dtype=np.uint64).reshape(-1))
    return h.ctypes.data, len(h), h


class Store:
    """Prefix-cache store (skv_store_*) over an arena tensor the store keeps
    alive.  put / decode need a device arena; reserve, commit, lookup, erase
    and stats are bookkeeping only and take any contiguous uint8 tensor."""

    def __init__(self, arena_bytes: int | None = None, arena: torch.Tensor | None = None, device=None):
        if arena is None:
            dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
            arena = torch.empty(arena_bytes, dtype=torch.uint8, device=dev)
        if not isinstance(arena, torch.Tensor) or arena.dtype != torch.uint8 or not arena.is_contiguous():
            raise ValueError("arena must be a contiguous uint8 tensor")
        self.arena = arena
        self._h = ctypes.c_void_p()
        _check(lib().skv_store_create(arena.data_ptr(), arena.numel(), ctypes.byref(self._h)), "skv_store_create")
        self._work = None
        self._tokens = {}          # entry id -> the container's tokens (ids are never reused)
        self._reserved = {}        # open reservation id -> arena address

    def _handle(self):
        if not self._h.value:
            raise ValueError("store is closed")
        return self._h

    def _view(self, addr: int, nbytes: int) -> torch.Tensor:
        off = addr - self.arena.data_ptr()
        return self.arena[off:off + nbytes]

    def _workspace(self, need: int) -> torch.Tensor:
        if self._work is None or self._work.numel() < need:
            self._work = None
            self._work = torch.empty(need, dtype=torch.uint8, device=self.arena.device)
        return self._work

    def reserve(self, nbytes: int, hashes) -> tuple[int, torch.Tensor]:
        """Room for a container written by the caller: (entry id, arena view of nbytes)."""
        hp, n, _keep = _hash_arg(hashes)
        eid, addr = ctypes.c_uint64(), ctypes.c_void_p()
        _check(lib().skv_store_reserve(self._handle(), hp, n, nbytes, ctypes.byref(eid), ctypes.byref(addr)),
               "skv_store_reserve")
        self._reserved[eid.value] = addr.value
        return eid.value, self._view(addr.value, nbytes)

    def commit(self, entry: int, nbytes: int, tokens: int | None = None) -> None:
        """Make a reservation visible; tokens (read from the container header
        when not given) sizes the checks of later range decodes."""
        _check(lib().skv_store_commit(self._handle(), entry, nbytes), "skv_store_commit")
        addr = self._reserved.pop(entry, None)
        if tokens is None and addr is not None and nbytes >= 64:
            tokens = int.from_bytes(self._view(addr, 24)[20:24].cpu().numpy().tobytes(), "little")
        self._tokens[entry] = tokens

    def abort(self, entry: int) -> None:
        _check(lib().skv_store_abort(self._handle(), entry), "skv_store_abort")
        self._reserved.pop(entry, None)

    def insert(self, container: torch.Tensor, hashes) -> int:
        """Store an existing container (copied into the arena on the current stream)."""
        if not isinstance(container, torch.Tensor) or container.dtype != torch.uint8 or container.dim() != 1:
            raise ValueError("container must be a 1-D uint8 tensor")
        eid, view = self.reserve(container.numel(), hashes)
        try:
            view.copy_(container)
            if view.is_cuda:
                torch.cuda.current_stream().synchronize()
        except Exception:
            self.abort(eid)
            raise
        self.commit(eid, container.numel(), container_tokens(container) if container.is_cuda else None)
        return eid

    def put(self, tables: Tables, target: torch.Tensor, aux: torch.Tensor, hashes) -> tuple[int, int]:
        """Encode target against aux into the store; returns (entry id, container bytes)."""
        if not self.arena.is_cuda:
            raise ValueError("put needs a device arena")
        tokens = tokens_of(tables, target)
        pt = _check_cache(target, "target", tables, tokens)
        pa = _check_cache(aux, "aux", tables, tokens)
        if target.device != self.arena.device or aux.device != self.arena.device:
            raise ValueError("target and aux must be on the arena's device")
        hp, n, _keep = _hash_arg(hashes)
        if tokens % BLOCK_TOKENS or n != tokens // BLOCK_TOKENS:
            raise ValueError(f"{tokens} tokens take {tokens // BLOCK_TOKENS} block hashes of whole 128-token blocks")
        shape = tables.shape(tokens)
        wb = ctypes.c_size_t()
        _check(lib().skv_store_put(self._handle(), None, 0, tables.ptr, ctypes.byref(shape), None, None, None,
                                   ctypes.byref(wb), None, None, None), "skv_store_put(size query)")
        work = self._workspace(wb.value)
        wb = ctypes.c_size_t(work.numel())
        eid, nbytes = ctypes.c_uint64(), ctypes.c_uint64()
        rc = lib().skv_store_put(self._handle(), hp, n, tables.ptr, ctypes.byref(shape), pt, pa, work.data_ptr(),
                                 ctypes.byref(wb), _stream(), ctypes.byref(eid), ctypes.byref(nbytes))
        _check(rc, "skv_store_put")
        self._tokens[eid.value] = tokens
        return eid.value, nbytes.value

    def lookup(self, hashes) -> StoreHit:
        """Entry holding the longest leading run of the hashes (entry 0 on a miss); a hit is pinned until release."""
        hp, n, _keep = _hash_arg(hashes)
        hit = StoreHit()
        _check(lib().skv_store_lookup(self._handle(), hp if n else None, n, ctypes.byref(hit)), "skv_store_lookup")
        return hit

    def container(self, hit: StoreHit) -> torch.Tensor:
        """Arena view of a hit's container (valid while the hit is pinned)."""
        return self._view(hit.container, hit.container_bytes)

    def release(self, entry: int) -> None:
        _check(lib().skv_store_release(self._handle(), entry), "skv_store_release")

    def erase(self, entry: int) -> None:
        _check(lib().skv_store_erase(self._handle(), entry), "skv_store_erase")

    def decode_into(self, tables: Tables, entry: int, aux: torch.Tensor, out: torch.Tensor, token_begin: int = 0,
                    token_end: int = 0) -> torch.Tensor:
        """Decode tokens [token_begin, token_end) of an entry (token_end 0: the whole container)."""
        if token_end:
            T = self._tokens.get(entry)
            if T is None and is_checkerboard(tables.mode):
                raise SkvError(ERR_ARG, "skv_store_decode")
            pa, po, cap = _range_buffers(tables, T, token_begin, token_end, aux, out, "skv_store_decode")
        else:
            if token_begin:
                raise ValueError("a whole-container decode starts at token 0")
            pa, po, cap = _decode_buffers(aux, out, tables)
        if aux.device != self.arena.device or out.device != self.arena.device:
            raise ValueError("aux and out must be on the arena's device")
        wb = ctypes.c_size_t()
        _check(lib().skv_store_decode(self._handle(), tables.ptr, entry, token_begin, token_end, None, None, 0, None,
                                      ctypes.byref(wb), None), "skv_store_decode(size query)")
        work = self._workspace(wb.value)
        wb = ctypes.c_size_t(work.numel())
        rc = lib().skv_store_decode(self._handle(), tables.ptr, entry, token_begin, token_end, pa, po, cap,
                                    work.data_ptr(), ctypes.byref(wb), _stream())
        _check(rc, "skv_store_decode")
        return out

    def decode(self, tables: Tables, entry: int, aux: torch.Tensor, token_begin: int = 0,
               token_end: int = 0) -> torch.Tensor:
        if not token_end:
            return self.decode_into(tables, entry, aux, torch.empty_like(aux))
        _range_buffers(tables, None, token_begin, token_end, None, None, "skv_store_decode", rules_only=True)
        out = torch.empty(_layout(tables, token_end - token_begin), dtype=aux.dtype, device=aux.device)
        return self.decode_into(tables, entry, aux, out, token_begin, token_end)

    def stats(self) -> dict:
        info = StoreInfo()
        _check(lib().skv_store_stats(self._handle(), ctypes.byref(info)), "skv_store_stats")
        return {name: getattr(info, name) for name, _ in StoreInfo._fields_}

    def close(self) -> None:
        if self._h.value and _lib is not None:
            _lib.skv_store_destroy(self._h)
        self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
