"""Seeded synthetic inputs for the HiSparse decode path.

This module draws inputs only: workload shapes, top-k drift traces, KV record
values and queries. It holds none of the method's arithmetic (no resolve, no
attention, no replacement policy), so both the CPU oracle's tests and the GPU
path can take their inputs from it without sharing any of the method.

The traces stand in for real indexer selections, whose one property the
HiSparse summary relies on is that consecutive decode steps select heavily
overlapping sets that drift a little (HiSparse blog summary, section 4,
"selection has locality"). The shapes (k = 2048, B in {2048, 4096, 8192},
576-element latent records, per-GPU batch 8) follow the same page's sections 4
and 5.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# HS_INPUTS_LIB names another build of fill.c to load (the sanitizer test's)
_BUILT = os.path.join(_HERE, "libhsinputs.so")
_LIB_PATH = os.environ.get("HS_INPUTS_LIB") or _BUILT
_lib = None

F32 = 0
BF16 = 1

# Stream ids of the counter-based generator.
STREAM_RECORD = 1
STREAM_QUERY = 2


def build_fill_lib(force: bool = False) -> str:
    """Compile fill.c into libhsinputs.so with gcc (OpenMP)."""
    import subprocess

    src = os.path.join(_HERE, "fill.c")
    if force or not os.path.exists(_BUILT) or os.path.getmtime(_BUILT) < os.path.getmtime(src):
        tmp = _BUILT + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", src, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _BUILT)
    return _BUILT


def build_sanitized(out: str, cc: str, flags: Sequence[str], link: Sequence[str] = ()) -> str:
    """fill.c built with the given sanitizer compiler and flags into
    out/libhsinputs_san.so (tests/test_sanitizers.py)."""
    import subprocess

    lib = os.path.join(out, "libhsinputs_san.so")
    subprocess.check_call([cc, "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                           "-fno-omit-frame-pointer", *flags, os.path.join(_HERE, "fill.c"), "-o",
                           lib, "-lm", *link])
    return lib


def _fill():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_fill_lib()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, u64, vp, dbl = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_double
        lib.hsin_fill_positions.argtypes = [vp, i64, vp, i64, i64, ctypes.c_int, u64, u64, i64, i64, dbl]
        lib.hsin_fill_range.argtypes = [vp, i64, i64, i64, i64, ctypes.c_int, u64, u64, i64, i64, dbl]
        lib.hsin_fill_rows.argtypes = [vp, i64, i64, ctypes.c_int, u64, u64, i64, i64, i64, dbl]
        lib.hsin_fill_packed.argtypes = [vp, i64, vp, i64, i64, ctypes.c_int, u64, u64, i64, i64, dbl]
        for f in (lib.hsin_fill_positions, lib.hsin_fill_range, lib.hsin_fill_rows, lib.hsin_fill_packed):
            f.restype = None
        _lib = lib
    return _lib


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------


@dataclass
class Workload:
    """One decode workload: shapes, record layout, trace recipe and seed."""

    name: str
    n_requests: int
    n_layers: int
    kind: str  # "mha" or "latent"
    dtype: int  # F32 or BF16 for records; queries use q_dtype
    q_dtype: int
    n_kv_heads: int
    head_dim: int
    latent_dim: int
    rope_dim: int
    n_q_heads: int
    k: int
    steps: int
    n_new: int  # positions replaced per step after step 0
    mix: Tuple[Tuple[str, float], ...]  # (source, probability); sources below
    rec_sigma: float
    seed: int
    append: bool = False
    ctx: List[int] = field(default_factory=list)  # per request prefill length
    B: List[int] = field(default_factory=list)  # per request buffer slots
    window: int = 512  # width of the "window" source
    zipf_s: float = 1.1  # exponent of the "zipf" source
    share: int = 1  # consecutive layers that reuse one selection (a layer group)

    @property
    def n_units(self) -> int:
        return self.n_requests * self.n_layers

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    @property
    def rec_elems(self) -> int:
        if self.kind == "mha":
            return 2 * self.n_kv_heads * self.head_dim
        return self.latent_dim + self.rope_dim

    @property
    def rec_bytes(self) -> int:
        return self.rec_elems * self.elem_bytes

    @property
    def q_dim(self) -> int:
        return self.head_dim if self.kind == "mha" else self.latent_dim + self.rope_dim

    @property
    def out_dim(self) -> int:
        return self.head_dim if self.kind == "mha" else self.latent_dim

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.q_dim)

    def capacity(self, r: int, steps: Optional[int] = None) -> int:
        s = self.steps if steps is None else steps
        return self.ctx[r] + (s if self.append else 0)

    def unit(self, u: int) -> Tuple[int, int]:
        """(request, layer) of unit u; units are request-major."""
        return u // self.n_layers, u % self.n_layers

    def group_base(self, l: int) -> int:
        """First layer of the group of layers whose selections layer l reuses."""
        return l - l % self.share


def _n_new(frac: float, k: int) -> int:
    return int(round(frac * k))


def workload(idx: int) -> Workload:
    """The five decode workloads, numbered 1..5.

    1 tiny fp32 MHA; 2 GQA 32K bf16 with write-through appends; 3 batch-8 MLA
    latent (the headline); 4 batch 32 x 2 layers, 256K context; 5 miss-heavy
    stress with per-request context and buffer sizes; 6 the batch-8 MLA
    setting over 8 layers in two groups of 4 that each reuse one selection
    (cross-layer index sharing); 7 compressed entries: each record is one
    entry standing for 4 tokens, 512 of the 8192 entries of a 32K context
    selected per step, 32 requests.
    """
    if idx == 1:
        w = Workload("tiny_mha_f32", 1, 1, "mha", F32, F32, 1, 64, 0, 0, 1, 256, 32,
                     _n_new(0.10, 256), (("uniform", 0.5), ("window", 0.5)), 1.0, 1)
        w.ctx, w.B = [4096], [512]
    elif idx == 2:
        w = Workload("gqa32k_bf16_append", 1, 1, "mha", BF16, BF16, 8, 128, 0, 0, 8, 2048, 256,
                     _n_new(0.13, 2048), (("zipf", 1.0),), 1.0, 2, append=True)
        w.ctx, w.B = [32768], [4096]
    elif idx == 3:
        w = Workload("mla_b8_128k", 8, 1, "latent", BF16, BF16, 1, 0, 512, 64, 64, 2048, 128,
                     _n_new(0.13, 2048), (("zipf", 1.0),), 0.5, 3)
        w.ctx, w.B = [131072] * 8, [4096] * 8
    elif idx == 4:
        w = Workload("gqa_b32x2_256k", 32, 2, "mha", BF16, BF16, 8, 128, 0, 0, 8, 2048, 64,
                     _n_new(0.07, 2048), (("uniform", 0.3), ("zipf", 0.7)), 1.0, 4)
        w.ctx, w.B = [262144] * 32, [8192] * 32
    elif idx == 5:
        w = Workload("mla_b64_stress", 64, 1, "latent", BF16, BF16, 1, 0, 512, 64, 64, 2048, 64,
                     _n_new(0.30, 2048), (("uniform", 1.0),), 0.5, 5)
        rng = np.random.default_rng(np.random.SeedSequence([5, 0xC0DE]))
        lo, hi = math.log(16384), math.log(1048576)
        w.ctx = [int(math.floor(math.exp(rng.uniform(lo, hi)))) for _ in range(64)]
        w.B = [int(b) for b in rng.choice(np.array([2048, 4096, 8192]), size=64)]
    elif idx == 6:
        w = Workload("mla_b8_128k_share4", 8, 8, "latent", BF16, BF16, 1, 0, 512, 64, 64, 2048,
                     64, _n_new(0.13, 2048), (("zipf", 1.0),), 0.5, 6, share=4)
        w.ctx, w.B = [131072] * 8, [4096] * 8
    elif idx == 7:
        w = Workload("csa_b32_32k_top512", 32, 1, "latent", BF16, BF16, 1, 0, 512, 64, 64, 512,
                     64, _n_new(0.13, 512), (("zipf", 1.0),), 0.5, 7)
        w.ctx, w.B = [32768 // 4] * 32, [1024] * 32
    else:
        raise ValueError(f"no workload {idx}")
    if w.n_layers % w.share:
        raise ValueError("layer groups must divide the layers")
    return w


# --------------------------------------------------------------------------
# Drift traces
# --------------------------------------------------------------------------

_zipf_cache = {}


def _zipf_cum(s: float, n: int) -> np.ndarray:
    key = s
    cum = _zipf_cache.get(key)
    if cum is None or cum.shape[0] < n:
        m = max(n, 1 << 18)
        d = np.arange(1, m + 1, dtype=np.float64)
        cum = np.cumsum(d ** (-s))
        _zipf_cache[key] = cum
    return cum


def _draw(rng: np.random.Generator, w: Workload, length: int, n: int) -> np.ndarray:
    """n candidate positions in [0, length) from the workload's source mixture."""
    probs = np.array([p for _, p in w.mix], dtype=np.float64)
    src = rng.choice(len(w.mix), size=n, p=probs / probs.sum()) if len(w.mix) > 1 else np.zeros(n, np.int64)
    out = np.empty(n, dtype=np.int64)
    for j, (name, _) in enumerate(w.mix):
        sel = np.nonzero(src == j)[0]
        if sel.size == 0:
            continue
        if name == "uniform":
            out[sel] = rng.integers(0, length, size=sel.size)
        elif name == "window":
            lo = max(0, length - w.window)
            out[sel] = rng.integers(lo, length, size=sel.size)
        elif name == "zipf":
            # distance d = length - pos over [1, length], P(d) ~ d^-s
            cum = _zipf_cum(w.zipf_s, length)
            u = rng.random(sel.size) * cum[length - 1]
            d = np.searchsorted(cum[:length], u, side="right") + 1
            d = np.minimum(d, length)
            out[sel] = length - d
        else:
            raise ValueError(name)
    return out


def gen_trace(w: Workload, r: int, l: int, steps: Optional[int] = None) -> np.ndarray:
    """Top-k positions for one (request, layer) unit: int32 [steps][k].

    Step 0 is k distinct positions drawn uniformly from the prefill. Every
    later step keeps a uniformly random subset of k - n_new positions of the
    previous set and adds n_new distinct positions that were not in it, drawn
    from the workload's source mixture over the current length (prefill plus
    the appends made so far). Each step's set is stored in a random order.
    """
    steps = w.steps if steps is None else steps
    k = w.k
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 0x7ACE, r, l]))
    out = np.empty((steps, k), dtype=np.int32)
    length = w.ctx[r]
    if k > length:
        raise ValueError("k exceeds the context")
    prev = rng.choice(length, size=k, replace=False).astype(np.int64)
    out[0] = prev
    taken = np.zeros(w.capacity(r, steps), dtype=bool)
    for t in range(1, steps):
        if w.append:
            length = w.ctx[r] + t
        keep = rng.choice(prev, size=k - w.n_new, replace=False)
        taken[prev] = True
        new: List[np.ndarray] = []
        need = w.n_new
        while need > 0:
            cand = _draw(rng, w, length, max(2 * need, 64))
            cand = cand[~taken[cand]]
            if cand.size:
                _, first = np.unique(cand, return_index=True)
                cand = cand[np.sort(first)][:need]
                taken[cand] = True
                new.append(cand)
                need -= cand.size
        taken[prev] = False
        for a in new:
            taken[a] = False
        cur = np.concatenate([keep] + new)
        cur = rng.permutation(cur)
        out[t] = cur
        prev = cur
    return out


def gen_traces(w: Workload, steps: Optional[int] = None) -> np.ndarray:
    """All units' traces: int32 [steps][n_units][k] (units request-major).
    Every layer of a group takes its first layer's trace."""
    steps = w.steps if steps is None else steps
    out = np.empty((steps, w.n_units, w.k), dtype=np.int32)
    for u in range(w.n_units):
        r, l = w.unit(u)
        g = w.group_base(l)
        if g != l:
            out[:, u, :] = out[:, r * w.n_layers + g, :]
        else:
            out[:, u, :] = gen_trace(w, r, l, steps)
    return out


# --------------------------------------------------------------------------
# Records and queries
# --------------------------------------------------------------------------


def fill_records(w: Workload, dst_addr: int, r: int, l: int,
                 positions: Optional[np.ndarray] = None,
                 p0: int = 0, p1: Optional[int] = None) -> None:
    """Write the records of unit (r, l) into a record array at host address
    dst_addr (record p at dst_addr + p * rec_bytes). Either a list of positions
    or the range [p0, p1)."""
    lib = _fill()
    if positions is not None:
        pos = np.ascontiguousarray(positions, dtype=np.int64)
        lib.hsin_fill_positions(dst_addr, w.rec_bytes, pos.ctypes.data, pos.size, w.rec_elems,
                                w.dtype, w.seed, STREAM_RECORD, r, l, w.rec_sigma)
    else:
        p1 = w.ctx[r] if p1 is None else p1
        lib.hsin_fill_range(dst_addr, w.rec_bytes, p0, p1, w.rec_elems, w.dtype, w.seed,
                            STREAM_RECORD, r, l, w.rec_sigma)


def record_array(w: Workload, r: int, l: int, positions: Sequence[int]) -> np.ndarray:
    """Records at the given positions as raw bytes uint8 [n][rec_bytes]."""
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    buf = np.empty((pos.size, w.rec_bytes), dtype=np.uint8)
    _fill().hsin_fill_packed(buf.ctypes.data, w.rec_bytes, pos.ctypes.data, pos.size, w.rec_elems,
                             w.dtype, w.seed, STREAM_RECORD, r, l, w.rec_sigma)
    return buf


def gen_queries(w: Workload, step: int) -> np.ndarray:
    """Queries of one decode step, all units: [n_units][Hq][q_dim] as float32
    (F32) or uint16 bfloat16 bits (BF16); N(0, 1)."""
    lib = _fill()
    dt = np.float32 if w.q_dtype == F32 else np.uint16
    out = np.empty((w.n_units, w.n_q_heads, w.q_dim), dtype=dt)
    for u in range(w.n_units):
        r, l = w.unit(u)
        lib.hsin_fill_rows(out[u].ctypes.data, w.n_q_heads, w.q_dim, w.q_dtype, w.seed,
                           STREAM_QUERY, r, l, step * w.n_q_heads, 1.0)
    return out


def touched_positions(traces: np.ndarray, u: int) -> np.ndarray:
    """Sorted distinct positions a unit's trace ever selects."""
    return np.unique(traces[:, u, :].astype(np.int64))


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    return (x.astype(np.uint32) << 16).view(np.float32)
