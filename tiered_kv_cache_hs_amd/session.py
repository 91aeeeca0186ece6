"""Set up one decode workload on the GPU and run its steps.

A Session owns, for one Workload: the pinned host pool (prefill records
written from the seeded generators), one device buffer per (request, layer)
unit, one batch per layer (layers run in sequence within a step, requests of
a layer together), the per-step selections and queries staged in HBM, and
the appended-token records for write-through workloads. A decode step is,
for each layer in order: hs_resolve -> hs_sparse_attn (or the fused
hs_resolve_attn) -> (write-through) append of that layer's new token.

Steps run in one of two ways:
  eager, step(t): every call takes step t's own arrays (any step, any
      order), and the append names its position (hs_pool_append);
  graph, capture() once then replay() every step: one hipGraph
      (torch.cuda.CUDAGraph) holds a whole step. Its first kernel,
      hs_stage_run, copies the next step's selections, queries and new
      records from the per-step arrays into fixed device buffers (the
      stand-in for the indexer and the other producers of a decode step)
      and advances a step counter on the device; the rest reads only those
      fixed buffers, and the append lands at each pool's device-side length
      (hs_pool_append_batch). The same graph is replayed for every step
      with no host synchronisation; replays run the steps in order from
      the counter (reset() sets it back to 0). (Staging the queries on a
      second stream beside the resolve measured slower: a fork and join
      inside a graph cost more than the copy.)

Layer groups that reuse one selection (Workload.share > 1; HiSparse summary,
section 6) run in one of three ways:
  "prefetch" - the group's later layers get buffers sharing the first
      layer's state (hs_buffer_create_shared); per group, hs_resolve of the
      first layer (the plan, and that layer's fetch), then on a second stream
      hs_prefetch of each later layer in order, each layer's attention
      waiting only for its own fetch, so the host-link transfer of layer
      l + 1 overlaps the attention of layer l;
  "serial"   - the same shared buffers, every call on one stream;
  "none"     - every layer has its own state and resolves on its own.

Only the library's entry points do work here; this module allocates and
orders. Unit order inside the session is layer-major: index l * R + r.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import hisparse as H
from . import inputs as I


class Session:
    def __init__(self, w: I.Workload, steps: Optional[int] = None, device: str = "cuda",
                 fill: str = "touched", traces: Optional[np.ndarray] = None,
                 fused: bool = False, share_mode: str = "prefetch", page_tokens: int = 0,
                 reserve: str = "all"):
        self.w = w
        self.fused = fused  # hs_resolve_attn instead of hs_resolve + hs_sparse_attn
        if share_mode not in ("prefetch", "serial", "none"):
            raise ValueError(share_mode)
        self.share_mode = share_mode if w.share > 1 else "none"
        self.grouped = self.share_mode != "none"
        self.steps = w.steps if steps is None else steps
        self.device = torch.device(device)
        R, L, k = w.n_requests, w.n_layers, w.k
        self.R, self.L, self.k = R, L, k
        # traces [steps][n_units (request-major)][k] -> layer-major device copy,
        # each step's entry padded to 16 bytes (a stage ring entry)
        self.traces = I.gen_traces(w, self.steps) if traces is None else traces
        lm = self.traces.reshape(self.steps, R, L, k).transpose(0, 2, 1, 3)
        self.topk = self._ring(torch.from_numpy(np.ascontiguousarray(lm)))  # [T][L][R][k]

        # reserve "all": every record the steps will append is allocated up
        # front; "prefill": only the prefill, the rest with hs_pool_reserve
        kind = H.HS_KV_MHA if w.kind == "mha" else H.HS_KV_LATENT
        cap_all = [w.capacity(r, self.steps) for r in range(R)]
        self.pool = H.hs_pool_create(R, L, kind, w.dtype,
                                     cap_all if reserve == "all" else list(w.ctx),
                                     n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                                     latent_dim=w.latent_dim, rope_dim=w.rope_dim,
                                     max_tokens=cap_all, page_tokens=page_tokens)
        self.rec = H.hs_pool_record_bytes(self.pool)
        self.reserve = reserve
        for r in range(R):
            for l in range(L):
                u = r * L + l
                if fill == "full":
                    want = np.arange(w.ctx[r], dtype=np.int64)
                else:  # only the positions the trace ever selects are written
                    want = np.unique(self.traces[:, u, :].astype(np.int64))
                    want = want[(want >= 0) & (want < w.ctx[r])]
                for first, page in H.pool_pages(self.pool, r, l):
                    sel = want[(want >= first) & (want < first + page.shape[0])]
                    if sel.size:  # record p of this page lies at base + p * rec
                        base = page.ctypes.data - first * self.rec
                        assert base > 0
                        I.fill_records(w, base, r, l, positions=sel)
                H.hs_pool_set_length(self.pool, r, l, w.ctx[r])

        # device buffers, one allocation per unit; in a grouped session the
        # later layers of a group hold rows only and share the first's state
        self.mem: List[torch.Tensor] = []
        self.bufs: List[List[int]] = [[0] * R for _ in range(L)]
        for l in range(L):
            g = w.group_base(l)
            for r in range(R):
                if self.grouped and g != l:
                    nbytes = H.hs_buffer_shared_bytes(self.pool, w.B[r])
                    t = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
                    self.bufs[l][r] = H.hs_buffer_create_shared(self.bufs[g][r], l, t)
                else:
                    nbytes = H.hs_buffer_bytes(self.pool, w.B[r])
                    t = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
                    self.bufs[l][r] = H.hs_buffer_create(self.pool, r, l, w.B[r], t)
                self.mem.append(t)
        self.batches = [H.hs_batch_create(self.bufs[l]) for l in range(L)]
        self.Bs = [list(w.B) for _ in range(L)]  # slots of each buffer [l][r]
        self.side = torch.cuda.Stream(device=self.device) if self.share_mode == "prefetch" else None
        self.fetched = [torch.cuda.Event() for _ in range(w.share)]

        # queries [T][L][R][Hq][qdim] (bf16 bits as int16, or fp32)
        qdt = torch.float32 if w.q_dtype == I.F32 else torch.int16
        q = np.stack([I.gen_queries(w, t) for t in range(self.steps)])  # [T][n(req-major)]...
        q = q.reshape(self.steps, R, L, w.n_q_heads, w.q_dim).transpose(0, 2, 1, 3, 4)
        q = np.ascontiguousarray(q)
        self.q = self._ring(torch.from_numpy(q.view(np.int16) if qdt == torch.int16 else q))

        # appended-token records [T][L][R][rec] (write-through workloads)
        self.app = None
        if w.append:
            app = np.empty((self.steps, L, R, self.rec), dtype=np.uint8)
            for r in range(R):
                for l in range(L):
                    pos = np.array([w.ctx[r] + t for t in range(self.steps)], dtype=np.int64)
                    app[:, l, r, :] = I.record_array(w, r, l, pos)
            self.app = self._ring(torch.from_numpy(app))

        # fixed buffers a captured step reads, filled by its stage kernel from
        # entry t of the rings above
        rings = [self.topk, self.q] + ([] if self.app is None else [self.app])
        fixed = [self._ring(torch.zeros((1,) + tuple(a.shape[1:]), dtype=a.dtype))[0]
                 for a in rings]
        self.topk_cur, self.q_cur = fixed[0], fixed[1]
        self.app_cur = None if self.app is None else fixed[2]
        # whole padded entries: the ring's stride in bytes
        self.stage = H.hs_stage_create(
            [(a, f, self._entry_bytes(a), self._entry_bytes(a)) for a, f in zip(rings, fixed)],
            self.steps)
        self._next = 0  # the step the next replay stages (the device counter)
        self.graph: Optional[torch.cuda.CUDAGraph] = None

        self.slots = torch.empty((L, R, k), dtype=torch.int32, device=self.device)
        self.miss = torch.empty((L, R), dtype=torch.int32, device=self.device)
        self.out = torch.empty((L, R, w.n_q_heads, w.out_dim), dtype=torch.float32,
                               device=self.device)
        wsb = max(H.hs_sparse_attn_workspace(self.batches[l], w.n_q_heads, k) for l in range(L))
        self.ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=self.device)
        self.scale = w.sm_scale
        torch.cuda.synchronize()

    @staticmethod
    def _entry_bytes(a: torch.Tensor) -> int:
        """Bytes of one step's entry of a ring made by _ring (padded to 16)."""
        return -(-a[0].numel() * a.element_size() // 16) * 16

    def _ring(self, a: torch.Tensor) -> torch.Tensor:
        """a [T][...] on the device with every step's entry starting on a
        16-byte boundary (a view of a padded [T][stride] array)."""
        T = a.shape[0]
        per = a[0].numel()
        stride = self._entry_bytes(a) // a.element_size()
        flat = torch.zeros((T, stride), dtype=a.dtype, device=self.device)
        flat[:, :per].copy_(a.reshape(T, per))
        return flat[:, :per].unflatten(1, tuple(a.shape[1:]))

    # -------------------------------------------------------------- steps
    def resolved_layer(self, l: int) -> int:
        """The layer whose resolve produced layer l's slots and misses."""
        return self.w.group_base(l) if self.grouped else l

    def _inputs(self, t: Optional[int]):
        """(selections [L][R][k], queries [L][R][Hq][qdim], new records
        [L][R][rec] or None) of step t, or the fixed staged buffers (t None)."""
        if t is None:
            return self.topk_cur, self.q_cur, self.app_cur
        return self.topk[t], self.q[t], None if self.app is None else self.app[t]

    def _append(self, t: Optional[int], l: int, app) -> None:
        if app is None:
            return
        if t is None:  # at each pool's device-side length
            H.hs_pool_append_batch(self.batches[l], app[l])
            return
        for r in range(self.R):
            H.hs_pool_append(self.pool, r, l, self.w.ctx[r] + t, app[l, r], n=1)

    def _attn(self, l: int, q) -> None:
        g = self.resolved_layer(l)
        H.hs_sparse_attn(self.batches[l], q[l], self.w.n_q_heads, self.slots[g], self.k,
                         self.scale, self.out[l], self.ws)

    def _group(self, t: Optional[int], g: int) -> None:
        """Enqueue the layer group starting at layer g (grouped sessions):
        one resolve for the group, the later layers' fetches from its plan,
        every layer's attention."""
        w = self.w
        topk, q, app = self._inputs(t)
        H.hs_resolve(self.batches[g], topk[g], self.k, self.slots[g], self.miss[g])
        if self.share_mode == "serial":
            self._attn(g, q)
            self._append(t, g, app)
            for l in range(g + 1, g + w.share):
                H.hs_prefetch(self.batches[l])
                self._attn(l, q)
                self._append(t, l, app)
            return
        cur = torch.cuda.current_stream()
        self.side.wait_stream(cur)
        with torch.cuda.stream(self.side):
            for j in range(1, w.share):
                H.hs_prefetch(self.batches[g + j])
                self.fetched[j].record(self.side)
        self._attn(g, q)
        self._append(t, g, app)
        for j in range(1, w.share):
            cur.wait_event(self.fetched[j])
            self._attn(g + j, q)
            self._append(t, g + j, app)

    def _layer(self, t: Optional[int], l: int) -> None:
        w = self.w
        topk, q, app = self._inputs(t)
        if self.fused:
            H.hs_resolve_attn(self.batches[l], topk[l], self.k, self.slots[l], self.miss[l],
                              q[l], w.n_q_heads, self.scale, self.out[l], self.ws)
        else:
            H.hs_resolve(self.batches[l], topk[l], self.k, self.slots[l], self.miss[l])
            H.hs_sparse_attn(self.batches[l], q[l], w.n_q_heads, self.slots[l], self.k,
                             self.scale, self.out[l], self.ws)
        self._append(t, l, app)

    def _run(self, t: Optional[int]) -> None:
        if self.grouped:
            for g in range(0, self.L, self.w.share):
                self._group(t, g)
            return
        for l in range(self.L):
            self._layer(t, l)

    def step(self, t: int) -> None:
        """Enqueue step t eagerly on the current stream (step t's own arrays)."""
        if self.reserve == "prefill" and self.app is not None:
            # pool pages on demand: room for this step's appended records
            for r in range(self.R):
                H.hs_pool_reserve(self.pool, r, self.w.ctx[r] + t + 1)
        self._run(t)

    def staged_step(self) -> None:
        """Enqueue the next step in graph form on the current stream: stage
        its inputs, then the step over the fixed buffers."""
        H.hs_stage_run(self.stage)
        self._run(None)

    def capture(self) -> None:
        """Capture one graph of staged_step(), replayed for every step."""
        if self.reserve == "prefill" and self.app is not None:
            for r in range(self.R):  # pages cannot be allocated inside a graph
                H.hs_pool_reserve(self.pool, r, self.w.capacity(r, self.steps))
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            self.staged_step()
        self.graph = g
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()

    def grow(self, new_B: List[int]) -> None:
        """Grow every buffer of request r to new_B[r] slots (hs_buffer_grow, or
        hs_buffer_grow_group for a layer group) and rebuild the batches; a
        graph captured before must be captured again."""
        torch.cuda.synchronize()
        self.graph = None
        dev = self.device
        for l in range(self.L):
            if self.resolved_layer(l) != l:
                continue  # grown with its group's first layer
            members = [m for m in range(l + 1, self.L) if self.resolved_layer(m) == l]
            for r in range(self.R):
                t = torch.empty(H.hs_buffer_bytes(self.pool, new_B[r]), dtype=torch.uint8,
                                device=dev)
                if members:
                    nb = H.hs_buffer_shared_bytes(self.pool, new_B[r])
                    mts = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in members]
                    H.hs_buffer_grow_group(self.bufs[l][r], [self.bufs[m][r] for m in members],
                                           new_B[r], t, mts)
                    for m, mt in zip(members, mts):
                        self.mem[m * self.R + r] = mt
                        self.Bs[m][r] = new_B[r]
                else:
                    H.hs_buffer_grow(self.bufs[l][r], new_B[r], t)
                self.mem[l * self.R + r] = t
                self.Bs[l][r] = new_B[r]
        # every batch of the pool is made again once all buffers have moved
        for l in range(self.L):
            H.hs_batch_destroy(self.batches[l])
            self.batches[l] = H.hs_batch_create(self.bufs[l])
        wsb = max(H.hs_sparse_attn_workspace(self.batches[l], self.w.n_q_heads, self.k)
                  for l in range(self.L))
        if wsb > self.ws.numel():
            self.ws = torch.empty(wsb, dtype=torch.uint8, device=self.device)
        torch.cuda.synchronize()

    def replay(self, t: Optional[int] = None) -> None:
        """Replay the captured step graph; it runs the step the device
        counter names (t, if given, must be that step)."""
        if t is not None and t != self._next:
            raise ValueError(f"the graph runs step {self._next} next, not {t}")
        if self._next >= self.steps:
            raise ValueError("every step of the trace has run")
        self.graph.replay()
        self._next += 1

    def reset(self) -> None:
        """Every buffer back to empty; pool lengths back to the prefill; the
        staged step counter back to 0."""
        torch.cuda.synchronize()
        H.hs_stage_set_step(self.stage, 0)
        self._next = 0
        for l in range(self.L):
            if self.resolved_layer(l) != l:
                continue  # a shared state is reset through its group's first layer
            for r in range(self.R):
                H.hs_buffer_reset(self.bufs[l][r])
        for r in range(self.R):
            for l in range(self.L):
                H.hs_pool_set_length(self.pool, r, l, self.w.ctx[r])
        torch.cuda.synchronize()

    # -------------------------------------------------------------- state
    def state(self, l: int, r: int):
        return H.hs_buffer_state_get(self.bufs[l][r], self.Bs[l][r])

    def rows(self, l: int, r: int) -> np.ndarray:
        addr, rec = H.hs_buffer_rows(self.bufs[l][r])
        B = self.Bs[l][r]
        t = self.mem[l * self.R + r][: B * rec]
        return t.cpu().numpy().reshape(B, rec)

    def close(self) -> None:
        torch.cuda.synchronize()
        self.graph = None
        H.hs_stage_destroy(self.stage)
        for b in self.batches:
            H.hs_batch_destroy(b)
        for l in reversed(range(self.L)):  # shared buffers before the state they use
            for r in range(self.R):
                H.hs_buffer_destroy(self.bufs[l][r])
        H.hs_pool_destroy(self.pool)
        self.batches, self.bufs, self.pool = [], [], None
