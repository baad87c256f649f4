"""CPU oracle for the lossless KV-cache codec and exact decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  It shares no code with the HIP library
(``decode_attention_calibrate_amd``) and never imports it; the HIP library never imports this.

The arithmetic lives in ``kvc_oracle.c`` (plain C, fp64 for attention).  This module compiles
it with gcc, binds it with ctypes, and adds the plain bookkeeping of a paged cache: a sequence
is a list of finished tiles plus an uncompressed tail, and a full tail is encoded once and
never re-encoded (page "GAAC: Lossless KV Compression ...", §3.3).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvc_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16, E5M2, E4M3 = 0, 1, 2
NARROW, WIDE, RAW = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle into oracle/liboracle.so (gcc, -O2, OpenMP over tiles/rows)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Params(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("T", ctypes.c_int32), ("D", ctypes.c_int32), ("G", ctypes.c_int32),
                ("esc_cap", ctypes.c_int32)]


class _Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "F", "MB", "EB", "has_wide", "n_groups", "plane_bytes", "tag_bytes", "code_bytes", "sm_bytes",
        "tag_off", "code_off", "sm_off", "esc_off", "stride", "raw_bytes")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER
        L.orc_layout_of.argtypes = [P(_Params), P(_Layout)]
        L.orc_calibrate.argtypes = [P(_Params), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_encode_tile.argtypes = [P(_Params), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_void_p, P(ctypes.c_int32), P(ctypes.c_int32), ctypes.c_void_p]
        L.orc_decode_tile.argtypes = [P(_Params), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p]
        L.orc_encode_batch.argtypes = [P(_Params), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
        L.orc_decode_batch.argtypes = [P(_Params), ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int32]
        L.orc_value.argtypes = [ctypes.c_int32, ctypes.c_uint32]
        L.orc_value.restype = ctypes.c_double
        L.orc_attention.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p,
                                    ctypes.c_int32]
        _lib = L
    return _lib


def _threads(n):
    """Thread count: explicit n, else OMP_NUM_THREADS, else min(cpu count, 16)."""
    if n:
        return int(n)
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return min(os.cpu_count() or 1, 16)


@dataclass(frozen=True)
class Params:
    """Codec geometry: fmt (BF16/E5M2/E4M3), T tokens per tile, D channels, G tokens per group,
    esc_cap escape bytes per tile (None -> T*D/16)."""
    fmt: int = BF16
    T: int = 64
    D: int = 128
    G: int = 16
    esc_cap: int | None = None

    @property
    def cap(self) -> int:
        return self.T * self.D // 16 if self.esc_cap is None else self.esc_cap

    def c(self) -> _Params:
        return _Params(self.fmt, self.T, self.D, self.G, self.cap)


def layout(p: Params) -> dict:
    out = _Layout()
    rc = lib().orc_layout_of(ctypes.byref(p.c()), ctypes.byref(out))
    if rc != 0:
        raise ValueError(f"invalid codec parameters {p}")
    return {n: getattr(out, n) for n, _ in _Layout._fields_}


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def calibrate(p: Params, x: np.ndarray):
    """x: [n_tokens][D] element bits (uint16) of one (K|V, head) -> (b3[D], b4[D]) uint8."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    assert x.ndim == 2 and x.shape[1] == p.D
    b3 = np.zeros(p.D, np.uint8)
    b4 = np.zeros(p.D, np.uint8)
    rc = lib().orc_calibrate(ctypes.byref(p.c()), _ptr(x), x.shape[0], _ptr(b3), _ptr(b4))
    if rc != 0:
        raise ValueError("calibrate failed")
    return b3, b4


def encode_tiles(p: Params, tiles: np.ndarray, b3: np.ndarray, b4: np.ndarray, is_v, nthreads=None):
    """tiles: [n][T][D] logical tiles; b3, b4: [n][D]; is_v: [n] (raw layout only).
    Returns (bytes [n][max(stride, raw)], is_raw [n], esc_used [n], mode_counts [n][3])."""
    tiles = np.ascontiguousarray(tiles, dtype=np.uint16)
    n = tiles.shape[0]
    lay = layout(p)
    width = max(lay["stride"], lay["raw_bytes"])
    b3 = np.ascontiguousarray(np.broadcast_to(b3, (n, p.D)), dtype=np.uint8)
    b4 = np.ascontiguousarray(np.broadcast_to(b4, (n, p.D)), dtype=np.uint8)
    isv = np.ascontiguousarray(np.broadcast_to(np.asarray(is_v, np.int32), (n,)), dtype=np.int32)
    out = np.zeros((n, width), np.uint8)
    is_raw = np.zeros(n, np.int32)
    esc = np.zeros(n, np.int32)
    modes = np.zeros((n, 3), np.int32)
    rc = lib().orc_encode_batch(ctypes.byref(p.c()), n, _ptr(tiles), _ptr(b3), _ptr(b4), _ptr(isv), _ptr(out), width,
                                _ptr(is_raw), _ptr(esc), _ptr(modes), _threads(nthreads))
    if rc != 0:
        raise ValueError("encode failed")
    return out, is_raw, esc, modes


def decode_tiles(p: Params, data: np.ndarray, is_raw, is_v, b3: np.ndarray, b4: np.ndarray, nthreads=None):
    """Inverse of encode_tiles.  Returns (tiles [n][T][D] uint16, status [n] int32)."""
    data = np.ascontiguousarray(data, dtype=np.uint8)
    n = data.shape[0]
    b3 = np.ascontiguousarray(np.broadcast_to(b3, (n, p.D)), dtype=np.uint8)
    b4 = np.ascontiguousarray(np.broadcast_to(b4, (n, p.D)), dtype=np.uint8)
    isr = np.ascontiguousarray(np.broadcast_to(np.asarray(is_raw, np.int32), (n,)), dtype=np.int32)
    isv = np.ascontiguousarray(np.broadcast_to(np.asarray(is_v, np.int32), (n,)), dtype=np.int32)
    out = np.zeros((n, p.T, p.D), np.uint16)
    status = np.zeros(n, np.int32)
    lib().orc_decode_batch(ctypes.byref(p.c()), n, _ptr(data), data.shape[1], _ptr(isr), _ptr(isv), _ptr(b3), _ptr(b4),
                           _ptr(out), _ptr(status), _threads(nthreads))
    return out, status


# ---- FORMAT v2: nested precision modes (page §4.7.2), BF16 -----------------------------------

MODE_SETS = {1: (2, 3, 4, 8), 2: (4, 8), 3: (3, 4, 8)}   # exponent widths of each mode, raw last


class _V2Layout(ctypes.Structure):
    _fields_ = [("n_modes", ctypes.c_int32), ("width", ctypes.c_int32 * 4)] + [(n, ctypes.c_int32) for n in (
        "n_groups", "plane_bytes", "tag_bytes", "sm_bytes", "code_cap", "tag_off", "sm_off", "code_off", "stride",
        "raw_bytes")]


def _v2_lib():
    L = lib()
    if not getattr(L, "_v2_bound", False):
        P = ctypes.POINTER
        L.orc_v2_layout_of.argtypes = [P(_Params), ctypes.c_int32, P(_V2Layout)]
        L.orc_v2_calibrate.argtypes = [P(_Params), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        L.orc_v2_encode_batch.argtypes = [P(_Params), ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_int32]
        L.orc_v2_decode_batch.argtypes = [P(_Params), ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
        L._v2_bound = True
    return L


def v2_layout(p: Params, mode_set: int) -> dict:
    out = _V2Layout()
    if _v2_lib().orc_v2_layout_of(ctypes.byref(p.c()), mode_set, ctypes.byref(out)) != 0:
        raise ValueError(f"invalid FORMAT v2 parameters {p}, mode set {mode_set}")
    d = {n: getattr(out, n) for n, _ in _V2Layout._fields_ if n != "width"}
    d["width"] = list(out.width)[:out.n_modes]
    return d


def v2_calibrate(p: Params, x: np.ndarray, w: int) -> np.ndarray:
    """Start of the calibrated window of 2^w exponents per channel: x [n_tokens][D] -> [D] uint8."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    b = np.zeros(p.D, np.uint8)
    if _v2_lib().orc_v2_calibrate(ctypes.byref(p.c()), _ptr(x), x.shape[0], w, _ptr(b)) != 0:
        raise ValueError("calibrate failed")
    return b


def v2_calibrate_layer(p: Params, k_cal: np.ndarray, v_cal: np.ndarray):
    """(b2, b3, b4) each [2 (K, V)][Hkv][D] from calibration rows [n][Hkv][D]."""
    Hkv = k_cal.shape[1]
    out = []
    for w in (2, 3, 4):
        b = np.zeros((2, Hkv, p.D), np.uint8)
        for kv, x in enumerate((k_cal, v_cal)):
            for h in range(Hkv):
                b[kv, h] = v2_calibrate(p, np.ascontiguousarray(x[:, h, :]), w)
        out.append(b)
    return tuple(out)


def v2_encode_tiles(p: Params, mode_set: int, tiles, b2, b3, b4, is_v, nthreads=None):
    """FORMAT v2 encode: tiles [n][T][D]; b2, b3, b4 [n][D] (or broadcastable).  Returns
    (bytes [n][max(stride, raw)], is_raw [n], code_bytes [n], mode_counts [n][4])."""
    tiles = np.ascontiguousarray(tiles, dtype=np.uint16)
    n = tiles.shape[0]
    lay = v2_layout(p, mode_set)
    width = max(lay["stride"], lay["raw_bytes"])
    bs = [np.ascontiguousarray(np.broadcast_to(b, (n, p.D)), dtype=np.uint8) for b in (b2, b3, b4)]
    isv = np.ascontiguousarray(np.broadcast_to(np.asarray(is_v, np.int32), (n,)), dtype=np.int32)
    out = np.zeros((n, width), np.uint8)
    is_raw = np.zeros(n, np.int32)
    used = np.zeros(n, np.int32)
    modes = np.zeros((n, 4), np.int32)
    rc = _v2_lib().orc_v2_encode_batch(ctypes.byref(p.c()), mode_set, n, _ptr(tiles), _ptr(bs[0]), _ptr(bs[1]),
                                       _ptr(bs[2]), _ptr(isv), _ptr(out), width, _ptr(is_raw), _ptr(used),
                                       _ptr(modes), _threads(nthreads))
    if rc != 0:
        raise ValueError("v2 encode failed")
    return out, is_raw, used, modes


def v2_decode_tiles(p: Params, mode_set: int, data, is_raw, is_v, b2, b3, b4, nthreads=None):
    """Inverse of v2_encode_tiles: (tiles [n][T][D], status [n])."""
    data = np.ascontiguousarray(data, dtype=np.uint8)
    n = data.shape[0]
    bs = [np.ascontiguousarray(np.broadcast_to(b, (n, p.D)), dtype=np.uint8) for b in (b2, b3, b4)]
    isr = np.ascontiguousarray(np.broadcast_to(np.asarray(is_raw, np.int32), (n,)), dtype=np.int32)
    isv = np.ascontiguousarray(np.broadcast_to(np.asarray(is_v, np.int32), (n,)), dtype=np.int32)
    out = np.zeros((n, p.T, p.D), np.uint16)
    status = np.zeros(n, np.int32)
    _v2_lib().orc_v2_decode_batch(ctypes.byref(p.c()), mode_set, n, _ptr(data), data.shape[1], _ptr(isr), _ptr(isv),
                                  _ptr(bs[0]), _ptr(bs[1]), _ptr(bs[2]), _ptr(out), _ptr(status), _threads(nthreads))
    return out, status


def window_coverage(p: Params, x: np.ndarray, w: int) -> np.ndarray:
    """Per channel of x [n_tokens][D]: the most exponents inside any window of w consecutive
    exponent values -> [D] int32."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    out = np.zeros(p.D, np.int32)
    L = lib()
    L.orc_window_coverage.argtypes = [ctypes.POINTER(_Params), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p]
    if L.orc_window_coverage(ctypes.byref(p.c()), _ptr(x), x.shape[0], w, _ptr(out)) != 0:
        raise ValueError("window coverage: invalid arguments")
    return out


def value(fmt: int, bits: int) -> float:
    return lib().orc_value(fmt, bits)


def values(fmt: int, bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of element bits (element-wise through orc_value)."""
    flat = np.asarray(bits, np.uint32).ravel()
    f = lib().orc_value
    return np.array([f(fmt, int(b)) for b in flat], np.float64).reshape(np.shape(bits))


def attention(fmt: int, q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, nthreads=None) -> np.ndarray:
    """Exact fp64 decode attention of one sequence: q [Hq][D] BF16 bits, k/v [L][Hkv][D]."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    L, Hkv, D = k.shape
    Hq = q.shape[0]
    out = np.zeros((Hq, D), np.float64)
    rc = lib().orc_attention(fmt, _ptr(q), _ptr(k), _ptr(v), L, Hq, Hkv, D, float(scale), _ptr(out),
                             _threads(nthreads))
    if rc != 0:
        raise ValueError("attention: invalid shapes")
    return out


class Sequence:
    """Plain model of one sequence of one layer: finished tiles keyed by (block, K|V, head),
    each compressed bytes or a raw tile, plus the uncompressed tail (fill-then-finalize)."""

    def __init__(self, p: Params, Hkv: int, bases):
        self.p, self.Hkv = p, Hkv
        self.b3, self.b4 = bases            # each [2][Hkv][D]: index 0 = K, 1 = V
        self.tiles = []                     # per block: dict with data/is_raw/esc/modes [2][Hkv]
        self.tail_k = np.zeros((0, Hkv, p.D), np.uint16)
        self.tail_v = np.zeros((0, Hkv, p.D), np.uint16)
        self.all_k = []                     # every appended row, for the lossless invariant
        self.all_v = []

    @property
    def length(self) -> int:
        return len(self.tiles) * self.p.T + self.tail_k.shape[0]

    def append(self, k_rows: np.ndarray, v_rows: np.ndarray, nthreads=None):
        """k_rows, v_rows: [n][Hkv][D].  Full tails are encoded once."""
        self.all_k.append(np.asarray(k_rows, np.uint16))
        self.all_v.append(np.asarray(v_rows, np.uint16))
        self.tail_k = np.concatenate([self.tail_k, k_rows.astype(np.uint16)])
        self.tail_v = np.concatenate([self.tail_v, v_rows.astype(np.uint16)])
        T = self.p.T
        nfull = self.tail_k.shape[0] // T
        if nfull:
            blocks_k = self.tail_k[:nfull * T].reshape(nfull, T, self.Hkv, self.p.D)
            blocks_v = self.tail_v[:nfull * T].reshape(nfull, T, self.Hkv, self.p.D)
            # tiles ordered (block, kv, head): logical [T][D] each
            tiles = np.stack([blocks_k, blocks_v], axis=1).transpose(0, 1, 3, 2, 4).reshape(-1, T, self.p.D)
            nb = nfull
            b3 = np.broadcast_to(self.b3[None], (nb, 2, self.Hkv, self.p.D)).reshape(-1, self.p.D)
            b4 = np.broadcast_to(self.b4[None], (nb, 2, self.Hkv, self.p.D)).reshape(-1, self.p.D)
            isv = np.broadcast_to(np.array([0, 1], np.int32)[None, :, None], (nb, 2, self.Hkv)).reshape(-1)
            data, is_raw, esc, modes = encode_tiles(self.p, tiles, b3, b4, isv, nthreads)
            per = 2 * self.Hkv
            for b in range(nb):
                sl = slice(b * per, (b + 1) * per)
                self.tiles.append(dict(data=data[sl].reshape(2, self.Hkv, -1), is_raw=is_raw[sl].reshape(2, self.Hkv),
                                       esc=esc[sl].reshape(2, self.Hkv), modes=modes[sl].reshape(2, self.Hkv, 3)))
            self.tail_k = self.tail_k[nfull * T:]
            self.tail_v = self.tail_v[nfull * T:]

    def decoded(self, nthreads=None):
        """Rebuild every token from the stored form: (K, V) [L][Hkv][D]."""
        p, H = self.p, self.Hkv
        ks, vs = [], []
        if self.tiles:
            data = np.stack([t["data"] for t in self.tiles]).reshape(-1, self.tiles[0]["data"].shape[-1])
            is_raw = np.stack([t["is_raw"] for t in self.tiles]).reshape(-1)
            nb = len(self.tiles)
            b3 = np.broadcast_to(self.b3[None], (nb, 2, H, p.D)).reshape(-1, p.D)
            b4 = np.broadcast_to(self.b4[None], (nb, 2, H, p.D)).reshape(-1, p.D)
            isv = np.broadcast_to(np.array([0, 1], np.int32)[None, :, None], (nb, 2, H)).reshape(-1)
            x, status = decode_tiles(p, data, is_raw, isv, b3, b4, nthreads)
            if (status != 0).any():
                raise ValueError("corrupt tile in oracle cache")
            x = x.reshape(nb, 2, H, p.T, p.D).transpose(1, 0, 3, 2, 4).reshape(2, nb * p.T, H, p.D)
            ks.append(x[0])
            vs.append(x[1])
        ks.append(self.tail_k)
        vs.append(self.tail_v)
        return np.concatenate(ks), np.concatenate(vs)

    def original(self):
        return np.concatenate(self.all_k), np.concatenate(self.all_v)


def calibrate_layer(p: Params, k_cal: np.ndarray, v_cal: np.ndarray):
    """Bases for one layer from calibration rows k_cal, v_cal [n][Hkv][D] -> (b3, b4) [2][Hkv][D]."""
    Hkv = k_cal.shape[1]
    b3 = np.zeros((2, Hkv, p.D), np.uint8)
    b4 = np.zeros((2, Hkv, p.D), np.uint8)
    for kv, x in enumerate((k_cal, v_cal)):
        for h in range(Hkv):
            b3[kv, h], b4[kv, h] = calibrate(p, np.ascontiguousarray(x[:, h, :]))
    return b3, b4


def stats(p: Params, seqs) -> dict:
    """Codec ratio (raw bits / stored bits, RAW tiles at raw size) and mode shares."""
    lay = layout(p)
    W = 1 + lay["MB"]
    raw_bits = stored_bits = 0
    modes = np.zeros(3, np.int64)
    n_raw = n_tiles = 0
    esc_total = 0
    for s in seqs:
        for t in s.tiles:
            for kv in range(2):
                for h in range(s.Hkv):
                    n_tiles += 1
                    raw_bits += lay["raw_bytes"] * 8
                    modes += t["modes"][kv, h]
                    if t["is_raw"][kv, h]:
                        n_raw += 1
                        stored_bits += lay["raw_bytes"] * 8
                    else:
                        esc_total += int(t["esc"][kv, h])
                        stored_bits += 2 * lay["n_groups"] + 3 * p.T * p.D + W * p.T * p.D + 8 * int(t["esc"][kv, h])
    return dict(codec_ratio=raw_bits / max(stored_bits, 1), mode_share=(modes / max(modes.sum(), 1)).tolist(),
                raw_tiles=n_raw, tiles=n_tiles, esc_bytes_per_tile=esc_total / max(n_tiles - n_raw, 1))
