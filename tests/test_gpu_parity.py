"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Slot ids, victim choices, LRU state (page table, stamps, clock), error words,
miss counts and resident row bytes must match bit for bit; attention within
max abs 1e-5 (fp32 records) or max abs 1e-2 and relative L2 4e-3 (bf16).
"""
import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from tests.parity import OracleRun, check_attn, compare_run, small_workload as _small  # noqa: E402,F401
from tiered_kv_cache_hs_amd import hisparse as H  # noqa: E402
from tiered_kv_cache_hs_amd import inputs as I  # noqa: E402
from tiered_kv_cache_hs_amd.session import Session  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.lib()
    H.hs_set_tuning()
    yield
    H.hs_set_tuning()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_tiny_fp32_every_step():
    w = I.workload(1)
    say("workload 1 (tiny fp32), 32 steps")
    st = compare_run(w, w.steps)
    say("worst max abs", max(s["max_abs"] for s in st))


def test_tiny_fp32_graph_replay():
    w = I.workload(1)
    compare_run(w, w.steps, graph=True)


def test_gqa32k_append_prefix():
    w = I.workload(2)
    say("workload 2 (GQA 32K bf16, appends), 48 steps")
    st = compare_run(w, 48, attn_every=4, rows_every=8)
    say("worst", max(s["max_abs"] for s in st), max(s["rel_l2"] for s in st))


def test_mla_b8_prefix():
    w = I.workload(3)
    say("workload 3 (MLA batch 8), 12 steps")
    st = compare_run(w, 12, attn_every=4, rows_every=6, attn_units=[(0, 0), (5, 0)])
    say("worst", max(s["max_abs"] for s in st), max(s["rel_l2"] for s in st))


SMALL = [
    # kind, dtype, B, k, ctx, steps, n_new
    ("mha", I.F32, 1, 1, 5, 6, 1),
    ("mha", I.F32, 7, 7, 40, 8, 3),
    ("mha", I.F32, 33, 17, 100, 10, 9),
    ("mha", I.F32, 1000, 300, 5000, 6, 77),
    ("mha", I.F32, 1024, 1024, 3000, 4, 100),
    ("mha", I.F32, 1025, 1000, 6000, 5, 333),
    ("mha", I.BF16, 3000, 2049, 9000, 5, 500),
    ("mha", I.F32, 16384, 4096, 40000, 4, 1000),
    ("latent", I.BF16, 97, 33, 500, 6, 10),
    ("latent", I.BF16, 2048, 2048, 9000, 4, 614),
    ("latent", I.BF16, 4096, 4096, 9000, 3, 700),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_shapes(case):
    kind, dt, B, k, ctx, steps, n_new = SMALL[case]
    if kind == "mha":
        w = _small(kind, dt, B, k, ctx, steps, n_new, seed=case,
                   Hkv=2 if dt == I.BF16 else 1, D=128 if dt == I.BF16 else 64,
                   Hq=4 if dt == I.BF16 else 1)
    else:
        w = _small(kind, dt, B, k, ctx, steps, n_new, seed=case, Hq=32)
    say(f"small case {case}: {SMALL[case]}")
    compare_run(w, steps, fill="full")


@pytest.mark.parametrize("hpw,splits,fused", [(32, 0, False), (32, 1, False), (32, 3, False),
                                               (64, 0, False), (64, 1, False), (64, 5, False),
                                               (64, 8, False), (32, 2, True), (64, 0, True)])
def test_latent_splits(hpw, splits, fused):
    """Latent attention with 32 and 64 heads per workgroup and several split-k
    factors (each split a run of 32-entry tiles; k = 197 = 6 * 32 + 5, so the
    last tile is ragged and, with 32 heads per workgroup and one split, alone
    in its step) and through the fused entry point."""
    w = _small("latent", I.BF16, 300, 197, 3000, 4, 40, R=2, seed=50 + splits + hpw, Hq=64)
    H.hs_set_tuning(splits, latent_heads_per_wg=hpw)
    try:
        compare_run(w, 4, fill="full", fused=fused)
    finally:
        H.hs_set_tuning()


@pytest.mark.parametrize("k,splits", [(700, 11), (1000, 16), (1100, 20)])
def test_latent_many_splits(k, splits):
    """Latent attention with 11, 16 and 18 splits of 64 entries (ragged last
    splits): the bf16 split partials merged by the one-pass combine (up to
    16 splits) and by the two-phase one (18)."""
    w = _small("latent", I.BF16, k + 100, k, 5000, 3, 60, R=2, seed=70 + splits, Hq=64)
    H.hs_set_tuning(splits)
    try:
        compare_run(w, 3, fill="full")
    finally:
        H.hs_set_tuning()


@pytest.mark.parametrize("hq", [16, 32, 64])
@pytest.mark.parametrize("k", [1, 15, 16, 17, 47, 64, 100, 250])
def test_latent_tile_tails(hq, k):
    """One split over the whole selection: 1 to 8 tiles of 32 entries, with
    ragged last tiles. 16 or 32 query heads take 32 heads per workgroup (two
    tiles per step, so the last step may hold one tile and the stream without
    it merges as an empty state; 16 heads pad the group); 64 heads take 64
    per workgroup (one tile per step, three step buffers)."""
    w = _small("latent", I.BF16, 300, k, 3000, 3, min(30, k), R=2, seed=900 + k + hq, Hq=hq)
    H.hs_set_tuning(1)
    try:
        compare_run(w, 3, fill="full")
    finally:
        H.hs_set_tuning()


@pytest.mark.parametrize("R,fetch", [(4, 2), (5, 2), (2, 1), (1, 1)])
def test_resolve_fetch_forced(R, fetch):
    """hs_tuning.resolve_fetch moves the misses in a gather kernel of its own
    on batches of 4 or more units (2) and inside the resolve kernel on
    smaller ones (1), against the oracle as always."""
    w = _small("latent", I.BF16, 300, 197, 3000, 4, 40, R=R, seed=70 + 10 * R + fetch, Hq=32)
    H.hs_set_tuning(resolve_fetch=fetch)
    try:
        compare_run(w, 4, fill="full")
    finally:
        H.hs_set_tuning()


@pytest.mark.parametrize("R,fetch", [(4, 0), (1, 1)])
def test_large_buffer_inline_fetch(R, fetch):
    """Buffers of more than 8192 slots with the misses fetched inside the
    resolve kernel (16 slots per thread, fewer host reads in flight per lane):
    by default on a batch of 4 units, forced on a single unit."""
    w = _small("mha", I.F32, 16384, 4096, 40000, 3, 1000, R=R, seed=90 + R)
    H.hs_set_tuning(resolve_fetch=fetch)
    try:
        compare_run(w, 3, fill="full")
    finally:
        H.hs_set_tuning()


def test_multi_request_multi_layer_small():
    w = _small("mha", I.BF16, 600, 200, 3000, 6, 50, R=3, L=2, seed=77, Hkv=2, D=128, Hq=16)
    compare_run(w, 6, fill="full")


def test_stamp_ties_break_by_position():
    # hand-made state: every slot holds the same stamp; the victims must be
    # the smallest positions (then ascending slot pairing with the misses)
    w = _small("mha", I.F32, 8, 3, 64, 1, 1, seed=5)
    sess = Session(w, 1, fill="full", traces=np.array([[[60, 61, 62]]], dtype=np.int32))
    try:
        pos = np.array([40, 3, 22, 7, 50, 9, 31, 18], dtype=np.int32)
        stamp = np.full(8, 5, dtype=np.uint32)
        H.hs_buffer_state_set(sess.bufs[0][0], pos, stamp, 3)
        ob = oracle.OracleBuffer(8, w.rec_bytes, with_rows=False)
        ob.pos[:] = pos
        ob.stamp[:] = stamp
        ob.clock[0] = 3
        sess.step(0)
        torch.cuda.synchronize()
        so, mo = oracle.resolve(ob, np.array([60, 61, 62]), None, 64)
        g_pos, g_stamp, g_clock, g_err = sess.state(0, 0)
        assert mo == 3 and int(sess.miss[0, 0]) == 3
        # positions 3, 7, 9 (slots 1, 3, 5) are evicted
        assert sorted(set(pos) - set(g_pos.tolist())) == [3, 7, 9]
        assert np.array_equal(sess.slots[0, 0].cpu().numpy(), so)
        assert np.array_equal(g_pos, ob.pos) and np.array_equal(g_stamp, ob.stamp)
    finally:
        sess.close()


def test_data_errors_leave_state_unchanged():
    w = _small("mha", I.F32, 16, 4, 64, 4, 2, seed=9)
    tr = np.array([[[1, 2, 3, 4]], [[5, 64, 6, 7]], [[8, 9, 8, 10]], [[11, 12, 13, -3]]],
                  dtype=np.int32)
    sess = Session(w, 4, fill="full", traces=tr)
    try:
        sess.step(0)
        torch.cuda.synchronize()
        p0, s0, c0, e0 = sess.state(0, 0)
        out0 = sess.out.cpu().numpy()
        assert e0 == 0 and c0 == 1
        for t, bits in ((1, H.HS_ERR_RANGE), (2, H.HS_ERR_DUP), (3, H.HS_ERR_RANGE)):
            sess.step(t)
            torch.cuda.synchronize()
            p, s, c, e = sess.state(0, 0)
            assert np.array_equal(p, p0) and np.array_equal(s, s0) and c == c0
            assert e & bits and e & H.HS_ERR_SLOT  # attention saw slots of -1
            assert (sess.slots.cpu().numpy() == -1).all() and int(sess.miss[0, 0]) == -1
            assert np.isnan(sess.out.cpu().numpy()).all()
        # a valid selection still resolves; the sticky bits stay
        H.hs_resolve(sess.batches[0], sess.topk[0, 0], 4, sess.slots[0], sess.miss[0])
        torch.cuda.synchronize()
        p, s, c, e = sess.state(0, 0)
        assert c == 2 and int(sess.miss[0, 0]) == 0
        assert e == (H.HS_ERR_RANGE | H.HS_ERR_DUP | H.HS_ERR_SLOT)
        assert np.isfinite(out0).all()
    finally:
        sess.close()


@pytest.mark.parametrize("B", [16, 2048])
def test_restored_state_then_resolves_and_repeats(B):
    """A state restored by hs_buffer_state_set, then resolves checked against
    the oracle step by step (for B > 1024 the resolve classifies positions
    through the inverse page table, which the restore rebuilds), then a
    position repeated among the hits and one repeated among the misses: each
    is refused with the state unchanged, and a valid selection resolves
    after them."""
    k = 4 if B == 16 else 600
    ctx = 64 if B == 16 else 4000
    rng = np.random.default_rng(B)
    held = rng.choice(ctx, size=B // 2, replace=False).astype(np.int32)
    pos = np.full(B, -1, dtype=np.int32)
    at = rng.choice(B, size=B // 2, replace=False)
    pos[at] = held
    clock = 9
    stamp = np.where(pos >= 0, rng.integers(1, 2 * clock + 1, size=B), 0).astype(np.uint32)
    # steps: half from the restored positions (hits), half new (misses)
    def sel(t):
        h = rng.choice(held, size=k // 2, replace=False)
        fresh = np.setdiff1d(np.arange(ctx, dtype=np.int32), held)
        m = rng.choice(fresh, size=k - k // 2, replace=False)
        return rng.permutation(np.concatenate([h, m])).astype(np.int32)
    tr = np.stack([sel(t)[None, :] for t in range(3)])
    hit_dup = tr[2, 0].copy()
    hit_dup[1] = hit_dup[0] = held[0]
    miss_dup = tr[2, 0].copy()
    fresh0 = int(np.setdiff1d(np.arange(ctx), np.concatenate([held, tr[:, 0].ravel()]))[0])
    miss_dup[1] = miss_dup[0] = fresh0
    tr = np.concatenate([tr, hit_dup[None, None], miss_dup[None, None], tr[2:3]])
    w = _small("mha", I.F32, B, k, ctx, tr.shape[0], 1, seed=B + 3)
    sess = Session(w, tr.shape[0], fill="full", traces=tr)
    try:
        H.hs_buffer_state_set(sess.bufs[0][0], pos, stamp, clock)
        ob = oracle.OracleBuffer(B, w.rec_bytes, with_rows=False)
        ob.pos[:] = pos
        ob.stamp[:] = stamp
        ob.clock[0] = clock
        for t in range(3):
            sess.step(t)
            torch.cuda.synchronize()
            so, mo = oracle.resolve(ob, tr[t, 0], None, ctx)
            g_pos, g_stamp, g_clock, g_err = sess.state(0, 0)
            assert g_err == 0 and g_clock == int(ob.clock[0])
            assert np.array_equal(sess.slots[0, 0].cpu().numpy(), so)
            assert int(sess.miss[0, 0]) == mo
            assert np.array_equal(g_pos, ob.pos) and np.array_equal(g_stamp, ob.stamp)
        p0, s0, c0, _ = sess.state(0, 0)
        for t in (3, 4):
            sess.step(t)
            torch.cuda.synchronize()
            p, s, c, e = sess.state(0, 0)
            assert e & H.HS_ERR_DUP
            assert np.array_equal(p, p0) and np.array_equal(s, s0) and c == c0
            assert int(sess.miss[0, 0]) == -1
        sess.step(5)  # the selection of step 2 again: all hits
        torch.cuda.synchronize()
        so, mo = oracle.resolve(ob, tr[5, 0], None, ctx)
        g_pos, g_stamp, g_clock, _ = sess.state(0, 0)
        assert mo == 0 and int(sess.miss[0, 0]) == 0
        assert np.array_equal(sess.slots[0, 0].cpu().numpy(), so)
        assert np.array_equal(g_pos, ob.pos) and np.array_equal(g_stamp, ob.stamp)
    finally:
        sess.close()


def test_clock_exhaustion_and_state_validation():
    w = _small("mha", I.F32, 4, 1, 16, 2, 1, seed=11)
    sess = Session(w, 2, fill="full", traces=np.array([[[1]], [[1]]], dtype=np.int32))
    try:
        buf = sess.bufs[0][0]
        pos = np.array([1, -1, -1, -1], np.int32)
        with pytest.raises(H.HsError):  # stamp must be 0 exactly for empty slots
            H.hs_buffer_state_set(buf, pos, np.array([0, 0, 0, 0], np.uint32), 5)
        with pytest.raises(H.HsError):  # duplicate position
            H.hs_buffer_state_set(buf, np.array([1, 1, -1, -1], np.int32),
                                  np.array([3, 4, 0, 0], np.uint32), 5)
        with pytest.raises(H.HsError):  # position beyond the pool length
            H.hs_buffer_state_set(buf, np.array([16, -1, -1, -1], np.int32),
                                  np.array([3, 0, 0, 0], np.uint32), 5)
        H.hs_buffer_state_set(buf, pos, np.array([9, 0, 0, 0], np.uint32), 0x7FFFFFFE)
        sess.step(0)
        torch.cuda.synchronize()
        p, s, c, e = sess.state(0, 0)
        assert c == 0x7FFFFFFF and e == 0 and s[0] == 2 * 0x7FFFFFFF
        sess.step(1)
        torch.cuda.synchronize()
        p, s, c, e = sess.state(0, 0)
        assert c == 0x7FFFFFFF and e & H.HS_ERR_CLOCK
    finally:
        sess.close()


def test_host_argument_checks():
    w = _small("mha", I.F32, 8, 4, 64, 1, 1, seed=12)
    sess = Session(w, 1, fill="full")
    try:
        b = sess.batches[0]
        with pytest.raises(H.HsError):
            H.hs_resolve(b, sess.topk[0, 0], 9, sess.slots[0], sess.miss[0])  # k > B
        with pytest.raises(H.HsError):
            H.hs_resolve(b, sess.topk[0, 0], 0, sess.slots[0], sess.miss[0])
        with pytest.raises(H.HsError):
            H.hs_pool_append(sess.pool, 0, 0, 70, np.zeros((1, w.rec_bytes), np.uint8))
        with pytest.raises(H.HsError):
            H.hs_pool_append(sess.pool, 1, 0, 0, np.zeros((1, w.rec_bytes), np.uint8))
        with pytest.raises(H.HsError):
            H.hs_sparse_attn(b, sess.q[0, 0], 3, sess.slots[0], 4, 0.1, sess.out[0], sess.ws)
    finally:
        sess.close()


def test_invalid_slot_gives_nan_and_error_bit():
    w = _small("mha", I.BF16, 64, 40, 500, 1, 1, seed=13, Hkv=2, D=128, Hq=4)
    sess = Session(w, 1, fill="full")
    try:
        sess.step(0)
        torch.cuda.synchronize()
        bad = sess.slots.clone()
        bad[0, 0, 17] = 64  # == B
        H.hs_sparse_attn(sess.batches[0], sess.q[0, 0], 4, bad[0], 40, 0.1, sess.out[0], sess.ws)
        torch.cuda.synchronize()
        assert np.isnan(sess.out.cpu().numpy()).all()
        assert sess.state(0, 0)[3] & H.HS_ERR_SLOT
    finally:
        sess.close()


@pytest.mark.parametrize("bad_index,bad_slot", [(0, -1), (37, 96), (95, 10**6)])
def test_latent_invalid_slot_gives_nan_and_error_bit(bad_index, bad_slot):
    w = _small("latent", I.BF16, 96, 96, 700, 1, 1, seed=14, Hq=32)
    sess = Session(w, 1, fill="full")
    try:
        sess.step(0)
        torch.cuda.synchronize()
        assert np.isfinite(sess.out.cpu().numpy()).all()
        assert sess.state(0, 0)[3] == 0
        bad = sess.slots.clone()
        bad[0, 0, bad_index] = bad_slot
        H.hs_sparse_attn(sess.batches[0], sess.q[0, 0], 32, bad[0], 96, 0.1, sess.out[0], sess.ws)
        torch.cuda.synchronize()
        assert np.isnan(sess.out.cpu().numpy()).all()
        assert sess.state(0, 0)[3] & H.HS_ERR_SLOT
    finally:
        sess.close()


@pytest.mark.parametrize("wl", [1, 3])
def test_exactness_against_full_kv_buffer(wl):
    # attention through the resolved slots equals the same kernel over a
    # full-KV buffer (slot = position), bit for bit
    w = I.workload(wl)
    steps = 4
    sess = Session(w, steps, fill="full")
    try:
        full_B = w.ctx[0]
        t_mem = torch.empty(H.hs_buffer_bytes(sess.pool, full_B), dtype=torch.uint8, device="cuda")
        fb = H.hs_buffer_create(sess.pool, 0, 0, full_B, t_mem)
        H.hs_buffer_state_set(fb, np.arange(full_B, dtype=np.int32),
                              np.ones(full_B, dtype=np.uint32), 1)
        fbatch = H.hs_batch_create([fb])
        # single-unit batches on both sides, so the split plans are the same
        b1 = H.hs_batch_create([sess.bufs[0][0]])
        out_res = torch.empty_like(sess.out[0, :1])
        out_full = torch.empty_like(sess.out[0, :1])
        ws = torch.empty(max(256, H.hs_sparse_attn_workspace(fbatch, w.n_q_heads, w.k)),
                         dtype=torch.uint8, device="cuda")
        for t in range(steps):
            sess.step(t)
            H.hs_sparse_attn(b1, sess.q[t, 0, :1], w.n_q_heads, sess.slots[0, :1], w.k,
                             w.sm_scale, out_res, ws)
            H.hs_sparse_attn(fbatch, sess.q[t, 0, :1], w.n_q_heads, sess.topk[t, 0, :1], w.k,
                             w.sm_scale, out_full, ws)
            torch.cuda.synchronize()
            a = out_res.cpu().numpy().view(np.uint32)
            b = out_full.cpu().numpy().view(np.uint32)
            assert np.array_equal(a, b), f"step {t}"
        H.hs_batch_destroy(b1)
        H.hs_batch_destroy(fbatch)
        H.hs_buffer_destroy(fb)
    finally:
        sess.close()


@pytest.mark.parametrize("case", [1, 3, 7, 8, 9])
def test_small_shapes_fused(case):
    kind, dt, B, k, ctx, steps, n_new = SMALL[case]
    if kind == "mha":
        w = _small(kind, dt, B, k, ctx, steps, n_new, seed=case,
                   Hkv=2 if dt == I.BF16 else 1, D=128 if dt == I.BF16 else 64,
                   Hq=4 if dt == I.BF16 else 1)
    else:
        w = _small(kind, dt, B, k, ctx, steps, n_new, seed=case, Hq=32)
    compare_run(w, steps, fill="full", fused=True)


@pytest.mark.parametrize("wl,steps,hq", [(1, 12, None), (2, 10, None), (3, 6, None), (3, 4, 16),
                                         (5, 3, None)])
def test_fused_equals_resolve_then_attention_bitwise(wl, steps, hq):
    """hs_resolve_attn == hs_resolve + hs_sparse_attn: state, rows and outputs
    bit for bit, step by step (workload 5 with its first 8 requests)."""
    w = I.workload(wl)
    if hq is not None:
        w = dataclasses.replace(w, n_q_heads=hq)
    if wl == 5:
        w = dataclasses.replace(w, n_requests=8, ctx=w.ctx[:8], B=w.B[:8])
    a = Session(w, steps, fill="touched", fused=False)
    b = Session(w, steps, fill="touched", fused=True, traces=a.traces)
    try:
        for t in range(steps):
            a.step(t)
            b.step(t)
            torch.cuda.synchronize()
            assert np.array_equal(a.slots.cpu().numpy(), b.slots.cpu().numpy()), t
            assert np.array_equal(a.miss.cpu().numpy(), b.miss.cpu().numpy()), t
            assert np.array_equal(a.out.cpu().numpy().view(np.uint32),
                                  b.out.cpu().numpy().view(np.uint32)), t
            for l in range(w.n_layers):
                for r in range(w.n_requests):
                    sa, sb = a.state(l, r), b.state(l, r)
                    assert all(np.array_equal(x, y) for x, y in zip(sa[:2], sb[:2])) and sa[2:] == sb[2:]
                    assert np.array_equal(a.rows(l, r)[sa[0] >= 0], b.rows(l, r)[sb[0] >= 0])
    finally:
        a.close()
        b.close()


@pytest.mark.parametrize("kind,graph", [("mha", False), ("latent", False), ("mha", True)])
def test_buffer_growth_mid_run(kind, graph):
    """Every buffer grows (B 40 -> 96, and 300 -> 300 + 211 for latent) after
    a few steps; slots, state, rows and outputs keep matching the oracle
    grown the same way, the new empty slots being used first."""
    if kind == "mha":
        w = _small("mha", I.F32, 40, 17, 300, 9, 6, R=2, L=2, seed=400)
        new_B = [96, 60]
    else:
        w = _small("latent", I.BF16, 300, 197, 3000, 6, 40, R=2, seed=401, Hq=32)
        new_B = [511, 300]
    compare_run(w, w.steps, fill="full", graph=graph, grow=(3, new_B))



@pytest.mark.parametrize("kind,fused,page", [("mha", False, 64), ("mha", True, 16),
                                             ("latent", False, 128), ("latent", True, 32)])
def test_paged_pool_small_pages(kind, fused, page):
    """Pool pages much smaller than the context: every host read (resolve's
    fetch, the gather, the attention kernels' fetch) goes through the page
    table across many pages."""
    if kind == "mha":
        w = _small("mha", I.BF16, 600, 200, 3000, 5, 50, R=2, L=2, seed=410, Hkv=2, D=128, Hq=8)
    else:
        w = _small("latent", I.BF16, 300, 197, 3000, 5, 40, R=2, seed=411, Hq=32)
    compare_run(w, 5, fill="full", fused=fused, page_tokens=page)


@pytest.mark.parametrize("graph", [False, True])
def test_paged_pool_grows_with_appends(graph):
    """Write-through appends past the prefill's pages: pages are reserved on
    demand (eagerly step by step, or all before capture), appends cross page
    boundaries, and new tokens come back as misses through the page table."""
    w = _small("mha", I.F32, 48, 24, 200, 40, 6, R=2, L=2, seed=420)
    w.append = True
    compare_run(w, 40, fill="full", graph=graph, page_tokens=16, reserve="prefill")


def test_pool_pages_and_reserve():
    pool = H.hs_pool_create(2, 3, H.HS_KV_MHA, H.HS_F32, [40, 10], n_kv_heads=1, head_dim=8,
                            max_tokens=[100, 10], page_tokens=16)
    try:
        assert H.hs_pool_capacity(pool, 0) == (48, 100, 16)
        assert H.hs_pool_capacity(pool, 1) == (16, 10, 16)  # whole pages
        rec = H.hs_pool_record_bytes(pool)
        a = H.hs_pool_record_ptr(pool, 0, 2, 17)
        b = H.hs_pool_record_ptr(pool, 0, 2, 18)
        assert b - a == rec
        assert H.hs_pool_page_ptr(pool, 0, 2, 1) == H.hs_pool_record_ptr(pool, 0, 2, 16)
        with pytest.raises(H.HsError):
            H.hs_pool_record_ptr(pool, 0, 0, 48)
        with pytest.raises(H.HsError):
            H.hs_pool_page_ptr(pool, 0, 0, 3)
        with pytest.raises(H.HsError):
            H.hs_pool_reserve(pool, 0, 101)
        with pytest.raises(H.HsError):  # append past the allocated pages
            H.hs_pool_append(pool, 0, 0, 0, np.zeros((49, rec), np.uint8))
        # existing records stay where they are when pages are added
        arr = np.arange(40 * rec, dtype=np.uint32).astype(np.uint8).reshape(40, rec)
        H.hs_pool_append(pool, 0, 1, 0, arr)
        H.hs_pool_reserve(pool, 0, 90)
        assert H.hs_pool_capacity(pool, 0)[0] == 96
        assert H.hs_pool_record_ptr(pool, 0, 2, 17) == a
        more = (np.arange(50 * rec, dtype=np.uint32) * 3).astype(np.uint8).reshape(50, rec)
        H.hs_pool_append(pool, 0, 1, 40, more)  # crosses pages 2 -> 5
        assert H.hs_pool_length(pool, 0, 1) == 90
        got = H.pool_read(pool, 0, 1, np.arange(90))
        assert np.array_equal(got[:40], arr) and np.array_equal(got[40:], more)
        # device-side append across a page boundary
        src = torch.from_numpy((np.arange(5 * rec) % 199).astype(np.uint8)).to("cuda")
        H.hs_pool_append(pool, 0, 0, 0, np.zeros((14, rec), np.uint8))
        H.hs_pool_append(pool, 0, 0, 14, src, n=5)
        torch.cuda.synchronize()
        assert np.array_equal(H.pool_read(pool, 0, 0, np.arange(14, 19)).reshape(-1),
                              src.cpu().numpy())
        assert H.hs_pool_length(pool, 0, 0) == 19
    finally:
        torch.cuda.synchronize()
        H.hs_pool_destroy(pool)


def test_batches_made_before_growth_are_refused():
    w = _small("mha", I.F32, 16, 8, 64, 2, 2, R=2, seed=430)
    sess = Session(w, 2, fill="full")
    try:
        sess.step(0)
        old = H.hs_batch_create(sess.bufs[0])
        t = torch.empty(H.hs_buffer_bytes(sess.pool, 32), dtype=torch.uint8, device="cuda")
        H.hs_buffer_grow(sess.bufs[0][0], 32, t)
        sess.mem[0] = t
        with pytest.raises(H.HsError):
            H.hs_resolve(old, sess.topk[1, 0], 8, sess.slots[0], sess.miss[0])
        with pytest.raises(H.HsError):
            H.hs_sparse_attn(old, sess.q[1, 0], 1, sess.slots[0], 8, 0.1, sess.out[0], sess.ws)
        with pytest.raises(H.HsError):
            H.hs_prefetch(old)
        H.hs_batch_destroy(old)
        fresh = H.hs_batch_create(sess.bufs[0])
        H.hs_resolve(fresh, sess.topk[1, 0], 8, sess.slots[0], sess.miss[0])
        torch.cuda.synchronize()
        H.hs_batch_destroy(fresh)
        H.hs_batch_destroy(sess.batches[0])
        sess.batches[0] = H.hs_batch_create(sess.bufs[0])
    finally:
        sess.close()


def test_pool_release_and_reuse_of_a_request_index():
    """A finished request returns its pages. Its buffer is then refused by
    the host until reset; a graph captured before the release (no host
    check) resolves it with range errors and reads nothing. After a new
    reservation, prefill and a buffer reset the request index serves a new
    request like a fresh one; without the reset the resolve is refused."""
    w = _small("mha", I.F32, 40, 17, 300, 6, 5, R=2, seed=440)
    sess = Session(w, 6, fill="full", page_tokens=64)
    try:
        for t in range(3):
            sess.step(t)
        sess.capture()
        torch.cuda.synchronize()
        H.hs_pool_release(sess.pool, 0)
        assert H.hs_pool_capacity(sess.pool, 0)[0] == 0
        assert H.hs_pool_length(sess.pool, 0, 0) == 0
        assert H.hs_pool_capacity(sess.pool, 1)[0] >= 300  # the other request keeps its pages
        with pytest.raises(H.HsError):
            H.hs_pool_record_ptr(sess.pool, 0, 0, 0)
        with pytest.raises(H.HsError, match="reset the buffer"):
            sess.step(3)
        sess.replay()  # captured before the release: every position is out of range now
        torch.cuda.synchronize()
        assert sess.state(0, 0)[3] & H.HS_ERR_RANGE
        assert sess.state(0, 1)[3] == 0  # request 1 unaffected
        st, errs = H.hs_batch_status(sess.batches[0], 2)
        assert st == H.HS_E_DEVICE and errs[0] & H.HS_ERR_RANGE and errs[1] == 0
        # a new request in index 0: pages, prefill, empty buffer
        H.hs_pool_reserve(sess.pool, 0, 300)
        for first, page in H.pool_pages(sess.pool, 0, 0):
            n = min(page.shape[0], 300 - first)
            if n > 0:
                I.fill_records(w, page.ctypes.data - first * w.rec_bytes, 0, 0,
                               positions=np.arange(first, first + n))
        H.hs_pool_set_length(sess.pool, 0, 0, 300)
        with pytest.raises(H.HsError, match="reset the buffer"):
            H.hs_resolve(sess.batches[0], sess.topk[4, 0], w.k, sess.slots[0], sess.miss[0])
        H.hs_buffer_reset(sess.bufs[0][0])
        torch.cuda.synchronize()
        assert H.hs_batch_status(sess.batches[0], 2)[0] == H.HS_OK
        sel = sess.topk[4, 0, 0].cpu().numpy()
        ob = oracle.OracleBuffer(40, w.rec_bytes, with_rows=True)
        pool = np.zeros((300, w.rec_bytes), np.uint8)
        I.fill_records(w, pool.ctypes.data, 0, 0, p0=0, p1=300)
        so, mo = oracle.resolve(ob, sel, pool, 300)
        H.hs_resolve(sess.batches[0], sess.topk[4, 0], w.k, sess.slots[0], sess.miss[0])
        torch.cuda.synchronize()
        assert np.array_equal(sess.slots[0, 0].cpu().numpy(), so) and int(sess.miss[0, 0]) == mo
        pos, stamp, clock, err = sess.state(0, 0)
        assert np.array_equal(pos, ob.pos) and err == 0
        rows = sess.rows(0, 0)
        assert np.array_equal(rows[pos >= 0], ob.rows[ob.pos >= 0])
    finally:
        sess.close()

