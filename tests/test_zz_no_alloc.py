"""GPU: the allocation-free attention entry point (hs_sparse_attn_noalloc)
against hs_sparse_attn with a caller workspace, through the C ABI.

Both run the same kernels with the same plan, so the outputs must be equal
bit for bit, and both within the attention tolerance of the oracle. Two
calls in a row, the second on a smaller input (fewer units, smaller k,
fewer splits), show that the scratch the calls share keeps no state that
matters; a captured graph of the call replayed several times gives the eager
result every time; a call needing more scratch than the library holds is
refused before anything is enqueued.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from tests.parity import OracleRun, check_attn, small_workload  # noqa: E402
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


def _both(sess, batch, q, slots, k, n_units, Hq, dv):
    """(workspace output, allocation-free output) of one attention call."""
    ws_bytes = H.hs_sparse_attn_workspace(batch, Hq, k)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    a = torch.full((n_units, Hq, dv), np.nan, dtype=torch.float32, device="cuda")
    b = torch.full((n_units, Hq, dv), np.nan, dtype=torch.float32, device="cuda")
    H.hs_sparse_attn(batch, q, Hq, slots, k, sess.scale, a, ws)
    H.hs_sparse_attn_noalloc(batch, q, Hq, slots, k, sess.scale, b)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy(), ws_bytes


@pytest.mark.parametrize("kind", ["latent", "mha"])
def test_noalloc_equals_workspace_form_two_calls_second_smaller(kind):
    if kind == "latent":
        w = small_workload("latent", I.BF16, 1024, 768, 4000, 2, 100, R=6, seed=61, Hq=64)
    else:
        w = small_workload("mha", I.BF16, 1024, 768, 4000, 2, 100, R=6, seed=62, Hkv=4, D=128,
                           Hq=16)
    sess = Session(w, 2, fill="touched")
    orc = OracleRun(w, sess.traces, 2)
    try:
        sess.step(0)
        torch.cuda.synchronize()
        for r in range(w.n_requests):
            orc.resolve(0, r, 0)
        # call 1: every unit, the whole selection
        a, b, ws1 = _both(sess, sess.batches[0], sess.q[0, 0], sess.slots[0], w.k, w.n_requests,
                          w.n_q_heads, w.out_dim)
        assert ws1 > 0  # split-k partials go through the scratch
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        for r in range(w.n_requests):
            check_attn(w, b[r], orc.attend(0, r, 0, sess.slots[0, r].cpu().numpy()), f"r={r}")
        # call 2: a smaller input - two units, the first 512 selected slots
        small = H.hs_batch_create(sess.bufs[0][1:3])
        try:
            k2 = 512
            sl = sess.slots[0, 1:3, :k2].contiguous()
            q2 = sess.q[0, 0, 1:3].contiguous()
            a2, b2, ws2 = _both(sess, small, q2, sl, k2, 2, w.n_q_heads, w.out_dim)
            assert 0 < ws2 < ws1
            assert np.array_equal(a2.view(np.uint32), b2.view(np.uint32))
            for j, r in enumerate((1, 2)):
                want = orc.attend(0, r, 0, sl[j].cpu().numpy())
                check_attn(w, b2[j], want, f"small r={r}")
        finally:
            H.hs_batch_destroy(small)
    finally:
        sess.close()


def test_noalloc_in_a_graph_replayed():
    w = small_workload("latent", I.BF16, 512, 512, 3000, 1, 50, R=3, seed=63, Hq=32)
    sess = Session(w, 1, fill="touched")
    try:
        sess.step(0)
        out = torch.zeros((w.n_requests, w.n_q_heads, w.out_dim), dtype=torch.float32,
                          device="cuda")
        H.hs_sparse_attn_noalloc(sess.batches[0], sess.q[0, 0], w.n_q_heads, sess.slots[0], w.k,
                                 sess.scale, out)  # eager, first call on the device
        torch.cuda.synchronize()
        want = out.clone()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            H.hs_sparse_attn_noalloc(sess.batches[0], sess.q[0, 0], w.n_q_heads, sess.slots[0],
                                     w.k, sess.scale, out)
        torch.cuda.current_stream().wait_stream(s)
        for rep in range(4):
            out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int32), want.view(torch.int32)), rep
        del g
    finally:
        sess.close()


def test_noalloc_refuses_more_than_its_scratch():
    # 32 splits of 64 slots (latent splits are whole pairs of 32-row tiles) for
    # 32 latent units of 64 heads: 67 MB of bf16 partials
    w = small_workload("latent", I.BF16, 2048, 2048, 2100, 1, 10, R=32, seed=64, Hq=64)
    sess = Session(w, 1, fill="touched")
    try:
        sess.step(0)
        torch.cuda.synchronize()
        H.hs_set_tuning(attn_splits=64)
        need = H.hs_sparse_attn_workspace(sess.batches[0], w.n_q_heads, w.k)
        assert need > H.HS_NOALLOC_SCRATCH_BYTES
        with pytest.raises(H.HsError, match="scratch"):
            H.hs_sparse_attn_noalloc(sess.batches[0], sess.q[0, 0], w.n_q_heads, sess.slots[0],
                                     w.k, sess.scale, sess.out[0])
    finally:
        H.hs_set_tuning()
        sess.close()
