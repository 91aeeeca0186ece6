"""Run the CPU oracle beside a GPU session and compare (test helper).

The oracle keeps its own pool (generated from the same seeded generators,
never read back from the GPU) and its own buffers, and follows the same step
order: per layer, resolve -> attention -> write-through append.
"""
from __future__ import annotations

import numpy as np

import oracle
from tiered_kv_cache_hs_amd import inputs as I

# attention tolerances: fp32 inputs max abs 1e-5; bf16 inputs max abs 1e-2 and
# relative L2 4e-3 (fp32 accumulation)
TOL_F32_MAX_ABS = 1e-5
TOL_BF16_MAX_ABS = 1e-2
TOL_BF16_REL_L2 = 4e-3


class OracleRun:
    def __init__(self, w: I.Workload, traces: np.ndarray, steps: int, keep_rows: bool = True):
        self.w = w
        self.traces = traces
        self.steps = steps
        self.R, self.L = w.n_requests, w.n_layers
        self.pools, self.lens, self.bufs = {}, {}, {}
        for r in range(self.R):
            for l in range(self.L):
                u = r * self.L + l
                cap = w.capacity(r, steps)
                # zero pages are not materialised until written: only the
                # selected positions (and appends) take memory
                pool = np.zeros((cap, w.rec_bytes), dtype=np.uint8)
                pos = np.unique(traces[:steps, u, :].astype(np.int64))
                pos = pos[(pos >= 0) & (pos < w.ctx[r])]
                I.fill_records(w, pool.ctypes.data, r, l, positions=pos)
                self.pools[(r, l)] = pool
                self.lens[(r, l)] = np.array([w.ctx[r]], dtype=np.int64)
                self.bufs[(r, l)] = oracle.OracleBuffer(w.B[r], w.rec_bytes, with_rows=keep_rows)
        self.queries = {}

    def resolve(self, t: int, r: int, l: int):
        u = r * self.L + l
        buf = self.bufs[(r, l)]
        pool = self.pools[(r, l)] if buf.rows is not None else None
        return oracle.resolve(buf, self.traces[t, u], pool, int(self.lens[(r, l)][0]))

    def attend(self, t: int, r: int, l: int, slots: np.ndarray, want64: bool = False):
        w = self.w
        if t not in self.queries:
            self.queries = {t: I.gen_queries(w, t)}
        q = self.queries[t][r * self.L + l]
        rows = self.bufs[(r, l)].rows
        if w.kind == "mha":
            return oracle.attend_mha(q, rows, slots, w.n_kv_heads, w.head_dim, w.dtype, w.q_dtype,
                                     np.float32(w.sm_scale), want64=want64)
        return oracle.attend_latent(q, rows, slots, w.latent_dim, w.rope_dim, w.dtype, w.q_dtype,
                                    np.float32(w.sm_scale), want64=want64)

    def append(self, t: int, r: int, l: int):
        w = self.w
        p = w.ctx[r] + t
        rec = I.record_array(self.w, r, l, [p])
        oracle.append(self.pools[(r, l)], self.lens[(r, l)], p, rec)


def check_attn(w: I.Workload, got: np.ndarray, want: np.ndarray, what: str = "") -> dict:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, what
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    max_abs = float(err.max())
    rel_l2 = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    if w.dtype == I.F32:
        assert max_abs <= TOL_F32_MAX_ABS, f"{what}: max abs {max_abs:.3e}"
    else:
        assert max_abs <= TOL_BF16_MAX_ABS, f"{what}: max abs {max_abs:.3e}"
        assert rel_l2 <= TOL_BF16_REL_L2, f"{what}: rel L2 {rel_l2:.3e}"
    return {"max_abs": max_abs, "rel_l2": rel_l2}


def small_workload(kind, dtype, B, k, ctx, steps, n_new, R=1, L=1, seed=0, Hkv=1, D=64, Hq=1,
                   share=1):
    """A small synthetic workload (test shapes that span tiles and ragged tails)."""
    if kind == "mha":
        w = I.Workload(f"small_{seed}", R, L, "mha", dtype, dtype, Hkv, D, 0, 0, Hq, k, steps,
                       n_new, (("uniform", 0.5), ("window", 0.5)), 1.0, 1000 + seed)
    else:
        w = I.Workload(f"small_{seed}", R, L, "latent", I.BF16, I.BF16, 1, 0, 512, 64, Hq, k,
                       steps, n_new, (("uniform", 1.0),), 0.5, 1000 + seed)
    w.ctx = [ctx] * R
    w.B = [B] * R
    w.share = share
    return w


def compare_run(w, steps, traces=None, attn_every=1, rows_every=1, attn_units=None,
                graph=False, fill="touched", fused=False, share_mode="prefetch", grow=None,
                **session_kw):
    """Run a GPU session step by step beside the oracle and compare slots,
    miss counts, state, resident rows and attention outputs of every unit.
    The oracle resolves every layer on its own, also where the session runs
    a layer group on one shared state. grow = (step, [new B per request]):
    before that step every buffer grows (hs_buffer_grow on the GPU side,
    oracle.grow on the oracle's)."""
    from tiered_kv_cache_hs_amd.session import Session
    import torch

    sess = Session(w, steps, fill=fill, traces=traces, fused=fused, share_mode=share_mode,
                   **session_kw)
    orc = OracleRun(w, sess.traces, steps)
    if graph:
        sess.capture()
    stats = []
    try:
        for t in range(steps):
            if grow is not None and t == grow[0]:
                sess.grow(grow[1])
                for (r, l), b in list(orc.bufs.items()):
                    orc.bufs[(r, l)] = oracle.grow(b, grow[1][r])
                if graph:
                    sess.capture()
            if graph:
                sess.replay(t)
            else:
                sess.step(t)
            torch.cuda.synchronize()
            slots_g = sess.slots.cpu().numpy()
            miss_g = sess.miss.cpu().numpy()
            out_g = sess.out.cpu().numpy()
            for l in range(w.n_layers):
                gl = sess.resolved_layer(l)
                for r in range(w.n_requests):
                    so, mo = orc.resolve(t, r, l)
                    assert np.array_equal(slots_g[gl, r], so), f"slots t={t} r={r} l={l}"
                    assert int(miss_g[gl, r]) == mo, f"miss t={t} r={r} l={l}"
                    pos, stamp, clock, err = sess.state(l, r)
                    ob = orc.bufs[(r, l)]
                    assert np.array_equal(pos, ob.pos), f"pos t={t} r={r} l={l}"
                    assert np.array_equal(stamp, ob.stamp), f"stamp t={t} r={r} l={l}"
                    assert clock == int(ob.clock[0]) and err == int(ob.err[0])
                    if rows_every and t % rows_every == 0:
                        rows = sess.rows(l, r)
                        occ = ob.pos >= 0
                        assert np.array_equal(rows[occ], ob.rows[occ]), f"rows t={t} r={r} l={l}"
                    if attn_every and t % attn_every == 0 and (attn_units is None or (r, l) in attn_units):
                        want = orc.attend(t, r, l, so)
                        stats.append(check_attn(w, out_g[l, r], want, f"attn t={t} r={r} l={l}"))
                    if w.append:
                        orc.append(t, r, l)
    finally:
        sess.close()
    return stats
