"""CPU oracle of the HiSparse decode hot path (RESOLVE + top-k sparse attention).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path never does. It shares
no code with the GPU library. The arithmetic lives in hs_oracle.c (plain C,
fp64 attention, sequential resolve); this module loads it with ctypes and
keeps each unit's state in numpy arrays.

Source: the HiSparse summary page (marsggbo.github.io, 2026-09-23), sections
3-5; see hs_oracle.c for the rules and the readings taken where the page is
silent.

Pins (each checked by the CPU tests, none by re-calling this code):
  resolve   brute-force LRU recency-list simulation on tiny traces, state
            invariants on every step, closed forms (cold step, B = k,
            B >= distinct positions), Belady lower bound, hand-worked cases;
  attention dense softmax attention in numpy fp64 when every position is
            selected, k = 1, equal keys, permutation invariance, and the
            exactness property (buffer rows == pool records at the selection).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# HS_ORACLE_LIB names another build of hs_oracle.c to load (the sanitizer
# test's AddressSanitizer + UndefinedBehaviorSanitizer build)
_BUILT = os.path.join(_HERE, "liboracle.so")
_LIB_PATH = os.environ.get("HS_ORACLE_LIB") or _BUILT
_lib = None

ERR_RANGE = 1
ERR_DUP = 2
ERR_CLOCK = 4

DT_F32 = 0
DT_BF16 = 1


def build(force: bool = False) -> str:
    """Compile hs_oracle.c into liboracle.so with gcc (OpenMP)."""
    src = os.path.join(_HERE, "hs_oracle.c")
    if force or not os.path.exists(_BUILT) or os.path.getmtime(_BUILT) < os.path.getmtime(src):
        tmp = _BUILT + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                               "-fno-fast-math", src, "-o", tmp, "-lm"])
        os.replace(tmp, _BUILT)
    return _BUILT


def build_sanitized(out: str) -> str:
    """hs_oracle.c built with AddressSanitizer and UndefinedBehaviorSanitizer
    (clang, every check fatal) into out/liboracle_san.so, for a process that
    preloads the sanitizer runtime (tests/test_sanitizers.py)."""
    src = os.path.join(_HERE, "hs_oracle.c")
    lib = os.path.join(out, "liboracle_san.so")
    subprocess.check_call([SAN_CC, "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                           "-fno-fast-math", "-fno-omit-frame-pointer", *SAN_FLAGS, src, "-o", lib,
                           "-lm", *SAN_LINK])
    return lib


# The host C compiler of the ROCm LLVM (its sanitizer runtime is the one the
# sanitized HIP library's host code uses too) and the sanitizer flags.
SAN_CC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
# its OpenMP runtime is found next to it
SAN_LINK = ["-Wl,-rpath," + os.path.join(os.path.dirname(os.path.dirname(SAN_CC)), "lib")]


class OracleUnitC(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("k", ctypes.c_int32),
        ("pos", ctypes.c_void_p), ("stamp", ctypes.c_void_p), ("clock", ctypes.c_void_p),
        ("err", ctypes.c_void_p), ("rows", ctypes.c_void_p), ("rec_bytes", ctypes.c_int64),
        ("pool", ctypes.c_void_p), ("pool_len", ctypes.c_int64), ("topk", ctypes.c_void_p),
        ("slots", ctypes.c_void_p), ("miss", ctypes.c_void_p),
        ("kind", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32), ("Dl", ctypes.c_int32), ("Dr", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("q_dtype", ctypes.c_int32), ("sm_scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("out", ctypes.c_void_p),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
        L.oracle_resolve.argtypes = [i32, vp, vp, vp, vp, vp, i64, vp, i64, vp, i32, vp, vp]
        L.oracle_resolve.restype = ctypes.c_int
        L.oracle_attend_mha.argtypes = [i32, i32, i32, i32, i32, vp, vp, i64, i64, vp, i32, f32, vp, vp]
        L.oracle_attend_mha.restype = ctypes.c_int
        L.oracle_attend_latent.argtypes = [i32, i32, i32, i32, i32, vp, vp, i64, i64, vp, i32, f32, vp, vp]
        L.oracle_attend_latent.restype = ctypes.c_int
        L.oracle_append.argtypes = [vp, i64, i64, vp, i64, i64, vp]
        L.oracle_append.restype = ctypes.c_int
        L.oracle_step_batch.argtypes = [i32, ctypes.POINTER(OracleUnitC), i32]
        L.oracle_step_batch.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]) -> Optional[int]:
    return None if a is None else a.ctypes.data


class OracleBuffer:
    """State of one (request, layer) device buffer as the oracle keeps it."""

    def __init__(self, B: int, rec_bytes: int, with_rows: bool = True):
        self.B = int(B)
        self.rec_bytes = int(rec_bytes)
        self.pos = np.full(self.B, -1, dtype=np.int32)
        self.stamp = np.zeros(self.B, dtype=np.uint32)
        self.clock = np.zeros(1, dtype=np.uint32)
        self.err = np.zeros(1, dtype=np.int32)
        self.rows = np.zeros((self.B, self.rec_bytes), dtype=np.uint8) if with_rows else None

    def copy(self) -> "OracleBuffer":
        o = OracleBuffer.__new__(OracleBuffer)
        o.B, o.rec_bytes = self.B, self.rec_bytes
        o.pos, o.stamp, o.clock, o.err = self.pos.copy(), self.stamp.copy(), self.clock.copy(), self.err.copy()
        o.rows = None if self.rows is None else self.rows.copy()
        return o


def grow(buf: OracleBuffer, new_B: int) -> OracleBuffer:
    """The buffer with new_B - B slots added (HiSparse summary, section 8: the
    per-request, per-layer device cache is allocated and grown on demand).
    Reading: growth only adds empty slots after the existing ones; positions,
    stamps, rows, clock and error word of slots [0, B) are unchanged."""
    if new_B < buf.B:
        raise ValueError("a buffer does not shrink")
    g = OracleBuffer(new_B, buf.rec_bytes, with_rows=buf.rows is not None)
    g.pos[: buf.B] = buf.pos
    g.stamp[: buf.B] = buf.stamp
    g.clock[:] = buf.clock
    g.err[:] = buf.err
    if buf.rows is not None:
        g.rows[: buf.B] = buf.rows
    return g


def resolve(buf: OracleBuffer, topk: np.ndarray, pool: Optional[np.ndarray], pool_len: int):
    """Resolve one selection against buf in place.

    pool: the unit's records as uint8 [cap][rec_bytes] (or None when the buffer
    keeps no rows). Returns (slots int32[k], miss int). Raises ValueError for a
    malformed call (k outside [1, B])."""
    topk = np.ascontiguousarray(topk, dtype=np.int32)
    k = topk.size
    slots = np.empty(k, dtype=np.int32)
    miss = np.zeros(1, dtype=np.int32)
    rows = buf.rows if pool is not None else None
    rc = lib().oracle_resolve(buf.B, _p(buf.pos), _p(buf.stamp), _p(buf.clock), _p(buf.err),
                              _p(rows), buf.rec_bytes, _p(pool), int(pool_len), _p(topk), k,
                              _p(slots), _p(miss))
    if rc != 0:
        raise ValueError("malformed resolve call")
    return slots, int(miss[0])


def attend_mha(q: np.ndarray, rows: np.ndarray, slots: np.ndarray, Hkv: int, D: int,
               kv_dtype: int, q_dtype: int, sm_scale: float, want64: bool = False):
    """MHA/GQA attention over rows[slots]. q: [Hq][D] (float32 or uint16 bf16
    bits); rows: uint8 [n_rows][rec_bytes]. Returns out float32 [Hq][D] (and
    fp64 values if want64)."""
    q = np.ascontiguousarray(q)
    rows = np.ascontiguousarray(rows)
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    Hq = q.shape[0]
    out = np.empty((Hq, D), dtype=np.float32)
    out64 = np.empty((Hq, D), dtype=np.float64) if want64 else None
    rc = lib().oracle_attend_mha(Hq, Hkv, D, kv_dtype, q_dtype, _p(q), _p(rows), rows.shape[1],
                                 rows.shape[0], _p(slots), slots.size, float(sm_scale), _p(out),
                                 _p(out64))
    if rc < 0:
        raise ValueError("malformed attention call")
    return (out, out64) if want64 else out


def attend_latent(q: np.ndarray, rows: np.ndarray, slots: np.ndarray, Dl: int, Dr: int,
                  kv_dtype: int, q_dtype: int, sm_scale: float, want64: bool = False):
    """Latent attention over rows[slots]. q: [Hq][Dl+Dr]; out float32 [Hq][Dl]."""
    q = np.ascontiguousarray(q)
    rows = np.ascontiguousarray(rows)
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    Hq = q.shape[0]
    out = np.empty((Hq, Dl), dtype=np.float32)
    out64 = np.empty((Hq, Dl), dtype=np.float64) if want64 else None
    rc = lib().oracle_attend_latent(Hq, Dl, Dr, kv_dtype, q_dtype, _p(q), _p(rows), rows.shape[1],
                                    rows.shape[0], _p(slots), slots.size, float(sm_scale), _p(out),
                                    _p(out64))
    if rc < 0:
        raise ValueError("malformed attention call")
    return (out, out64) if want64 else out


def append(pool: np.ndarray, length: np.ndarray, p: int, src: np.ndarray) -> None:
    """Write-through: records src [n][rec_bytes] into pool at [p, p+n); length
    is a 1-element int64 array updated in place."""
    src = np.ascontiguousarray(src, dtype=np.uint8)
    n = src.shape[0]
    rc = lib().oracle_append(_p(pool), pool.shape[1], pool.shape[0], _p(length), int(p), n, _p(src))
    if rc != 0:
        raise ValueError("append out of range")


def step_batch(units, n_threads: int = 0) -> int:
    """Run resolve + attention for a list of OracleUnitC in parallel; returns
    the thread count used."""
    arr = (OracleUnitC * len(units))(*units)
    return int(lib().oracle_step_batch(len(units), arr, int(n_threads)))
