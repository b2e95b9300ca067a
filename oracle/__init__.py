"""CPU oracle for lossless KV-cache coding -- TEST INFRASTRUCTURE ONLY.

Plain scalar C (``skv_oracle.c``) behind ctypes.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import this package; the
product library never does, and the two share no code.  See the header of
``skv_oracle.c`` for the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "skv_oracle.c")
_LIB = os.path.join(_HERE, "libskv_oracle.so")

BF16, E4M3, INT16 = 1, 2, 3
RESIDUAL, CHECKERBOARD, RESIDUAL_EXP, CHECKERBOARD_MAP = 0, 1, 2, 3
OK, E_ARG, E_SHAPE, E_CAPACITY, E_CORRUPT, E_TABLES = 0, -1, -2, -3, -4, -5


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-Wall", "-Wno-unused-function",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Shape(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_uint32), ("mode", ctypes.c_uint32), ("layers", ctypes.c_uint32),
                ("kv", ctypes.c_uint32), ("tokens", ctypes.c_uint32), ("channels", ctypes.c_uint32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        u32, i32, u64, i64, vp = ctypes.c_uint32, ctypes.c_int32, ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        sp = ctypes.POINTER(Shape)
        sig = {
            "skvo_ord": (u32, [u32, ctypes.c_int]),
            "skvo_inv_ord": (u32, [u32, ctypes.c_int]),
            "skvo_residual": (i32, [u32, u32, ctypes.c_int]),
            "skvo_zigzag": (u32, [i32]),
            "skvo_unzigzag": (i32, [u32]),
            "skvo_reconstruct": (u32, [u32, i32, ctypes.c_int]),
            "skvo_exp_class": (u32, [u32, ctypes.c_int, u32]),
            "skvo_dckv_split": (None, [i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]),
            "skvo_dckv_symbol": (u32, [i32, i32, ctypes.POINTER(i32)]),
            "skvo_dckv_reconstruct": (i32, [u32, i32]),
            "skvo_dckv_mean": (i32, [vp, vp, u32, u32, u32, u32]),
            "skvo_rans_put": (ctypes.c_int, [ctypes.POINTER(u32), u32, u32, ctypes.POINTER(ctypes.c_uint16)]),
            "skvo_rans_pop": (u32, [ctypes.POINTER(u32), vp, vp, u32]),
            "skvo_cell_mass": (ctypes.c_double, [ctypes.c_double, ctypes.c_double, ctypes.c_double]),
            "skvo_quantize": (None, [vp, ctypes.c_int, vp]),
            "skvo_fnv1a64": (u64, [vp, ctypes.c_size_t]),
            "skvo_blob_bytes": (u64, [sp]),
            "skvo_blob_bytes_map": (u64, [sp, u32]),
            "skvo_dckv_map": (ctypes.c_int, [vp, vp, u32, u32, u32, u32, u32, vp, vp, vp, ctypes.c_int]),
            "skvo_fit_tables_map": (ctypes.c_int, [sp, vp, vp, u32, u32, u32, u32, vp, vp, vp, u64,
                                                   ctypes.POINTER(u64)]),
            "skvo_bound": (u64, [sp]),
            "skvo_n_streams": (u64, [sp]),
            "skvo_fit_tables": (ctypes.c_int, [sp, vp, vp, u32, vp, u64, ctypes.POINTER(u64)]),
            "skvo_encode": (i64, [vp, ctypes.c_size_t, sp, vp, vp, vp, u64, ctypes.POINTER(u64), ctypes.c_int]),
            "skvo_decode": (ctypes.c_int, [vp, ctypes.c_size_t, vp, u64, vp, vp, u64, ctypes.c_int]),
            "skvo_container_shape": (ctypes.c_int, [vp, u64, sp]),
            "skvo_encode_tile": (i64, [vp, ctypes.c_size_t, sp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_int)]),
            "skvo_blob_table": (ctypes.c_int, [vp, ctypes.c_size_t, u64, ctypes.POINTER(u32), vp]),
            "skvo_stream_encode_ext": (i64, [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, u64]),
            "skvo_stream_decode_ext": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, u64, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def make_shape(dtype: int, mode: int, layers: int, kv: int, tokens: int, channels: int) -> Shape:
    return Shape(dtype, mode, layers, kv, tokens, channels)


# ---------------------------------------------------------------- primitives
def ord_(u: int, nbits: int) -> int:
    return lib().skvo_ord(u, nbits)


def inv_ord(o: int, nbits: int) -> int:
    return lib().skvo_inv_ord(o, nbits)


def residual(t: int, p: int, nbits: int) -> int:
    return lib().skvo_residual(t, p, nbits)


def zigzag(r: int) -> int:
    return lib().skvo_zigzag(r)


def exp_class(p: int, dtype: int, base: int) -> int:
    return lib().skvo_exp_class(p, dtype, base)


def blob_bases(blob: bytes) -> np.ndarray:
    """Class bases (one per slab) of an exponent-mode blob."""
    nt = int.from_bytes(blob[8:12], "little")
    return np.frombuffer(blob[64 + 514 * nt:], dtype=np.uint8).copy()


def unzigzag(z: int) -> int:
    return lib().skvo_unzigzag(z)


def reconstruct(p: int, r: int, nbits: int) -> int:
    return lib().skvo_reconstruct(p, r, nbits)


def dckv_split(mu_q: int) -> tuple[int, int]:
    k, f = ctypes.c_int32(), ctypes.c_int32()
    lib().skvo_dckv_split(mu_q, ctypes.byref(k), ctypes.byref(f))
    return k.value, f.value


def dckv_symbol(c: int, mu_q: int) -> tuple[int, int]:
    f = ctypes.c_int32()
    z = lib().skvo_dckv_symbol(c, mu_q, ctypes.byref(f))
    return z, f.value


def dckv_reconstruct(z: int, mu_q: int) -> int:
    return lib().skvo_dckv_reconstruct(z, mu_q)


def dckv_mean(coef: np.ndarray, G: np.ndarray, t: int, comp: int) -> int:
    c = np.ascontiguousarray(coef, dtype=np.int16)
    g = np.ascontiguousarray(G, dtype=np.int16)
    T, C = c.shape
    return lib().skvo_dckv_mean(_ptr(c), _ptr(g), T, C, t, comp)


def rans_put(x: int, f: int, c: int) -> tuple[int, int | None]:
    xs, w = ctypes.c_uint32(x), ctypes.c_uint16()
    out = lib().skvo_rans_put(ctypes.byref(xs), f, c, ctypes.byref(w))
    return xs.value, (w.value if out else None)


def rans_pop(x: int, freq, cum) -> tuple[int, int]:
    fr = np.ascontiguousarray(freq, dtype=np.uint32)
    cu = np.ascontiguousarray(cum, dtype=np.uint32)
    xs = ctypes.c_uint32(x)
    s = lib().skvo_rans_pop(ctypes.byref(xs), _ptr(fr), _ptr(cu), len(fr))
    return s, xs.value


def cell_mass(v: float, m: float, b: float) -> float:
    return lib().skvo_cell_mass(v, m, b)


def quantize(q) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float64)
    f = np.zeros(len(q), dtype=np.uint32)
    lib().skvo_quantize(_ptr(q), len(q), _ptr(f))
    return f


def fnv1a64(b: bytes) -> int:
    a = np.frombuffer(b, dtype=np.uint8).copy()
    return lib().skvo_fnv1a64(_ptr(a), len(a))


# ---------------------------------------------------------------- streams
def _tables_arrays(tables):
    """tables: list of (n, freqs[0..n]) -> flat arrays for the C side."""
    n = np.array([t[0] for t in tables], dtype=np.uint32)
    fr = np.zeros((len(tables), 257), dtype=np.uint32)
    for j, (nn, f) in enumerate(tables):
        fr[j, : nn + 1] = f
    return n, fr


def stream_encode(z, tab_of, tables, steps: int, ebytes: int) -> bytes:
    """Encode one stream of `steps` x 32 symbol values with explicit tables;
    escaped values take `ebytes` bytes each."""
    z = np.ascontiguousarray(z, dtype=np.uint32).reshape(-1)
    tab_of = np.ascontiguousarray(tab_of, dtype=np.uint32).reshape(-1)
    assert z.size == steps * 32 and tab_of.size == steps * 32
    n, fr = _tables_arrays(tables)
    cap = 128 + 4 + 4 * steps * 32 + 4
    out = np.zeros(cap, dtype=np.uint8)
    nb = lib().skvo_stream_encode_ext(steps, ebytes, len(tables), _ptr(n), _ptr(fr), _ptr(tab_of), _ptr(z), _ptr(out), cap)
    return out[:nb].tobytes()


def stream_decode(data: bytes, tab_of, tables, steps: int, ebytes: int):
    """Returns (rc, z) for one stream."""
    tab_of = np.ascontiguousarray(tab_of, dtype=np.uint32).reshape(-1)
    n, fr = _tables_arrays(tables)
    buf = np.frombuffer(data, dtype=np.uint8).copy() if len(data) else np.zeros(1, np.uint8)
    z = np.zeros(steps * 32, dtype=np.uint32)
    rc = lib().skvo_stream_decode_ext(steps, ebytes, len(tables), _ptr(n), _ptr(fr), _ptr(tab_of), _ptr(buf), len(data), _ptr(z))
    return rc, z


# ---------------------------------------------------------------- containers
def fit_tables(shape: Shape, calib_t: np.ndarray, calib_a: np.ndarray, calib_tokens: int) -> bytes:
    need = lib().skvo_blob_bytes(ctypes.byref(shape))
    out = np.zeros(need, dtype=np.uint8)
    nb = ctypes.c_uint64()
    ct = np.ascontiguousarray(calib_t)
    ca = np.ascontiguousarray(calib_a)
    rc = lib().skvo_fit_tables(ctypes.byref(shape), _ptr(ct), _ptr(ca), calib_tokens, _ptr(out), need, ctypes.byref(nb))
    if rc:
        raise RuntimeError(f"oracle fit_tables failed: {rc}")
    return out[: nb.value].tobytes()


def dckv_map(coef: np.ndarray, G: np.ndarray, V: np.ndarray, U: np.ndarray, sh1: int, sh2: int,
             threads: int = 1) -> np.ndarray:
    """Side input with the decoded-neighbour map applied (odd rows G', even
    rows G) for [T][C] int16 coefficients and G; V int8 [k][2C], U int8 [C][k]."""
    c = np.ascontiguousarray(coef, dtype=np.int16)
    g = np.ascontiguousarray(G, dtype=np.int16)
    v = np.ascontiguousarray(V, dtype=np.int8)
    u = np.ascontiguousarray(U, dtype=np.int8)
    T, C = c.shape
    k = v.shape[0]
    assert g.shape == (T, C) and v.shape == (k, 2 * C) and u.shape == (C, k)
    out = np.zeros_like(g)
    rc = lib().skvo_dckv_map(_ptr(c), _ptr(g), T, C, k, sh1, sh2, _ptr(v), _ptr(u), _ptr(out), threads)
    if rc:
        raise RuntimeError(f"oracle dckv_map failed: {rc}")
    return out


def fit_tables_map(shape: Shape, calib_coef: np.ndarray, calib_G: np.ndarray, calib_tokens: int, V: np.ndarray,
                   U: np.ndarray, sh1: int, sh2: int) -> bytes:
    """Tables of the decoded-neighbour-map mode (checkerboard fit on G', then the map)."""
    v = np.ascontiguousarray(V, dtype=np.int8)
    u = np.ascontiguousarray(U, dtype=np.int8)
    k = v.shape[0]
    need = lib().skvo_blob_bytes_map(ctypes.byref(shape), k)
    out = np.zeros(need, dtype=np.uint8)
    nb = ctypes.c_uint64()
    c = np.ascontiguousarray(calib_coef, dtype=np.int16)
    g = np.ascontiguousarray(calib_G, dtype=np.int16)
    rc = lib().skvo_fit_tables_map(ctypes.byref(shape), _ptr(c), _ptr(g), calib_tokens, k, sh1, sh2, _ptr(v), _ptr(u),
                                   _ptr(out), need, ctypes.byref(nb))
    if rc:
        raise RuntimeError(f"oracle fit_tables_map failed: {rc}")
    return out[: nb.value].tobytes()


def blob_table(blob: bytes, j: int) -> tuple[int, np.ndarray]:
    b = np.frombuffer(blob, dtype=np.uint8).copy()
    n = ctypes.c_uint32()
    fr = np.zeros(256, dtype=np.uint32)
    rc = lib().skvo_blob_table(_ptr(b), len(b), j, ctypes.byref(n), _ptr(fr))
    if rc:
        raise RuntimeError(rc)
    return n.value, fr[: n.value + 1].copy()


def n_streams(shape: Shape) -> int:
    return lib().skvo_n_streams(ctypes.byref(shape))


def encode_array(blob: bytes, shape: Shape, target: np.ndarray, aux: np.ndarray, threads: int = 1) -> np.ndarray:
    """The container as a uint8 array (no copy of large outputs)."""
    b = np.frombuffer(blob, dtype=np.uint8).copy()
    t = np.ascontiguousarray(target)
    a = np.ascontiguousarray(aux)
    need = ctypes.c_uint64()
    cap = lib().skvo_bound(ctypes.byref(shape))
    out = np.zeros(cap, dtype=np.uint8)
    rc = lib().skvo_encode(_ptr(b), len(b), ctypes.byref(shape), _ptr(t), _ptr(a), _ptr(out), cap, ctypes.byref(need), threads)
    if rc < 0:
        raise RuntimeError(f"oracle encode failed: {rc}")
    return out[:rc]


def encode(blob: bytes, shape: Shape, target: np.ndarray, aux: np.ndarray, threads: int = 1) -> bytes:
    return encode_array(blob, shape, target, aux, threads).tobytes()


def decode_rc(blob: bytes, container: bytes, aux: np.ndarray, out: np.ndarray, threads: int = 1) -> int:
    b = np.frombuffer(blob, dtype=np.uint8).copy()
    c = np.frombuffer(container, dtype=np.uint8).copy() if len(container) else np.zeros(1, np.uint8)
    a = np.ascontiguousarray(aux)
    return lib().skvo_decode(_ptr(b), len(b), _ptr(c), len(container), _ptr(a), _ptr(out), out.nbytes, threads)


def decode(blob: bytes, container: bytes, aux: np.ndarray, out_like: np.ndarray, threads: int = 1) -> np.ndarray:
    out = np.zeros_like(out_like)
    rc = decode_rc(blob, container, aux, out, threads)
    if rc:
        raise RuntimeError(f"oracle decode failed: {rc}")
    return out


def encode_tile(blob: bytes, shape: Shape, tile_t, tile_a, lane_ids, nb_l=None, nb_r=None) -> tuple[bytes, bool]:
    """One stream from its 4096 gathered inputs ((step, lane) order)."""
    b = np.frombuffer(blob, dtype=np.uint8).copy()
    t = np.ascontiguousarray(tile_t).reshape(-1)
    a = np.ascontiguousarray(tile_a).reshape(-1)
    ids = np.ascontiguousarray(lane_ids, dtype=np.uint32)
    out = np.zeros(8192, dtype=np.uint8)
    raw = ctypes.c_int()
    l = np.ascontiguousarray(nb_l, dtype=np.int16).reshape(-1) if nb_l is not None else None
    r = np.ascontiguousarray(nb_r, dtype=np.int16).reshape(-1) if nb_r is not None else None
    nb = lib().skvo_encode_tile(_ptr(b), len(b), ctypes.byref(shape), _ptr(t), _ptr(a),
                                _ptr(l) if l is not None else None, _ptr(r) if r is not None else None,
                                _ptr(ids), _ptr(out), ctypes.byref(raw))
    if nb < 0:
        raise RuntimeError(f"oracle encode_tile failed: {nb}")
    return out[:nb].tobytes(), bool(raw.value)
