"""Iteration-level (continuous) batching over the paged KV pool: a host-side
scheduler, and an executor that runs its decisions through the kernels one
iteration at a time.

What it follows:

* "What problem does PagedAttention solve, and what is continuous
  batching?" (datarekha), section "What continuous batching changes": a
  static batch runs until its longest request is done; with iteration-level
  batching the active set is revisited at every generation boundary, a
  finished request leaves at once and a queued one takes its place after
  its prompt's prefill has been scheduled, with its KV blocks from the same
  pool.  Section "How the two fit together in production": queue -> prefill
  and block allocation -> decode pool, one token per active sequence per
  iteration -> release on finish -> admit waiting requests when capacity
  allows; long prompts are processed in chunks under a per-step token cap.
  Section "A concrete memory example": a conventional design reserves 4,096
  tokens per request; paged allocation hands out blocks as they fill.
  Section "The senior-level nuance": when the pool is full the server must
  queue, preempt and recompute, offload or reject.
* "PagedAttention & Continuous Batching" (ai-ml-animation-academy),
  "Overview": the memory freed from reservations turns into concurrency.

Readings (the pages fix no policy details):

* An iteration is one generation boundary.  A request's prefill (its whole
  prompt, or the chunks of it that fit under the step's token cap) runs in
  the iterations after its admission; the iteration that completes its
  prompt also yields its first generated token.  Every other running request
  yields one token per iteration; a request that reaches its generation
  length leaves at the end of that iteration.
* Admission is first come, first served: the head of the queue waits until
  it fits, and nothing behind it is admitted first.
* ``static``: a batch of up to ``max_batch`` requests is formed when no batch
  is running and holds its slots until its last member finishes; each member
  reserves ``reserve_tokens`` (the conventional design).
* ``reserved``: iteration-level batching, each request reserving
  ``reserve_tokens`` tokens of the pool for its whole life.
* ``paged``: iteration-level batching over the block manager: a request is
  admitted when the free blocks cover its prompt plus one token; it takes a
  block whenever its last one fills; if the pool cannot supply one, the most
  recently admitted running request is preempted (its blocks freed, its
  progress dropped, back to the front of the queue) until the growth fits.
"""
from collections import deque
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np


@dataclass(eq=False)  # compared by identity: the running list removes by object
class Request:
    rid: int
    arrival: int          # first iteration at which it may be admitted
    prompt_len: int       # >= 1
    gen_len: int          # tokens it generates, >= 1
    # progress
    admitted: Optional[int] = None
    prefilled: int = 0    # prompt tokens whose keys and values are in the pool
    generated: int = 0
    finished: Optional[int] = None   # iteration that yielded its last token
    released: Optional[int] = None   # iteration at whose end its slot was freed
    preemptions: int = 0

    def kv_tokens(self, prefilled=None, generated=None) -> int:
        """Positions whose keys and values are in the pool: the prompt so far,
        then every generated token but the newest (it is fed back, and its
        keys and values appended, in the next iteration)."""
        p = self.prefilled if prefilled is None else prefilled
        g = self.generated if generated is None else generated
        return p + max(0, g - 1) if p == self.prompt_len else p


@dataclass
class StepPlan:
    """What one iteration runs."""
    iteration: int
    prefill: List[tuple] = field(default_factory=list)   # (rid, first prompt token, count)
    decode: List[int] = field(default_factory=list)       # rids yielding a token
    padded: List[int] = field(default_factory=list)       # static: done rows still in the batch
    admitted: List[int] = field(default_factory=list)
    finished: List[int] = field(default_factory=list)
    preempted: List[int] = field(default_factory=list)
    released: List[int] = field(default_factory=list)     # left the running set at the end


class Scheduler:
    """Decides, iteration by iteration, which requests prefill, which decode
    and which wait.  Pure host logic: no device memory."""

    def __init__(self, mode: str, requests, num_blocks: int, block_size: int = 16,
                 max_batch: int = 256, max_step_tokens: int = 2048,
                 reserve_tokens: int = 4096):
        if mode not in ("static", "reserved", "paged"):
            raise ValueError(f"unknown mode {mode!r}")
        self.mode = mode
        self.bs = int(block_size)
        self.num_blocks = int(num_blocks)
        self.max_batch = int(max_batch)
        self.max_step_tokens = int(max_step_tokens)
        self.reserve_tokens = int(reserve_tokens)
        self.slots = self.num_blocks * self.bs // self.reserve_tokens  # reservations that fit
        self.pending = deque(sorted(requests, key=lambda r: (r.arrival, r.rid)))
        self._prompt_len = {r.rid: r.prompt_len for r in self.pending}
        self.queue: deque = deque()
        self.running: List[Request] = []       # admission order
        self.done: List[Request] = []
        self.it = 0
        self.history: List[Dict] = []

    def blocks(self, tokens: int) -> int:
        return -(-tokens // self.bs)

    def active(self) -> int:
        """Requests pending, queued or running."""
        return len(self.pending) + len(self.queue) + len(self.running)

    def prompt_len_of(self, rid: int) -> int:
        return self._prompt_len[rid]

    def blocks_used(self) -> int:
        """Paged: blocks the running requests hold now (Request.kv_tokens
        and blocks() written out: this runs over the running set twice an
        iteration)."""
        bs = self.bs
        n = 0
        for r in self.running:
            p = r.prefilled
            t = p + (r.generated - 1 if r.generated > 0 else 0) if p == r.prompt_len else p
            n += -(-t // bs)
        return n

    # ---- one iteration
    def step(self) -> StepPlan:
        self.it += 1
        plan = StepPlan(self.it)
        while self.pending and self.pending[0].arrival <= self.it:
            self.queue.append(self.pending.popleft())
        self._admit_all(plan)
        self._plan(plan)
        if self.mode == "paged":
            while self._need(plan) > self.num_blocks and len(self.running) > 1:
                self._preempt(self.running[-1], plan)
                self._plan(plan)
        # apply
        pre = {rid: k for rid, _, k in plan.prefill}
        dec = set(plan.decode)
        for r in self.running:
            k = pre.get(r.rid)
            if k is not None:
                r.prefilled += k
            if r.rid in dec:
                r.generated += 1
        for r in list(self.running):
            if r.generated >= r.gen_len and r.finished is None:
                r.finished = self.it
                plan.finished.append(r.rid)
                if self.mode != "static":
                    self._release(r, plan)
        if self.mode == "static" and self.running and all(
                r.finished is not None for r in self.running):
            for r in list(self.running):
                self._release(r, plan)
        self.history.append({"iteration": self.it, "running": len(self.running),
                             "decode": len(plan.decode), "padded": len(plan.padded),
                             "prefill_tokens": sum(k for _, _, k in plan.prefill),
                             "blocks_used": self.blocks_used() if self.mode == "paged" else
                             len(self.running) * self.reserve_tokens // self.bs,
                             "queued": len(self.queue)})
        return plan

    def _admit_all(self, plan: StepPlan):
        if self.mode == "static" and self.running:
            return  # the batch holds its slots until its last member is done
        used = self.blocks_used() if self.mode == "paged" else 0
        while self.queue and len(self.running) < self.max_batch:
            r = self.queue[0]
            if self.mode == "paged":
                need = self.blocks(r.prompt_len + 1)  # the prompt and the first growth
                if used + need > self.num_blocks:
                    break
                used += need
            else:
                if r.prompt_len + r.gen_len > self.reserve_tokens:
                    raise ValueError(f"request {r.rid} is longer than a reservation")
                if len(self.running) >= self.slots:
                    break
            self.queue.popleft()
            r.admitted = self.it
            self.running.append(r)
            plan.admitted.append(r.rid)

    def _plan(self, plan: StepPlan):
        """Prefill chunks under the token cap (admission order) and the
        requests that yield a token this iteration."""
        plan.prefill, plan.decode = [], []
        budget = self.max_step_tokens
        for r in self.running:
            if r.prefilled < r.prompt_len and budget > 0:
                k = min(budget, r.prompt_len - r.prefilled)
                plan.prefill.append((r.rid, r.prefilled, k))
                budget -= k
        pre = {rid: k for rid, _, k in plan.prefill}
        for r in self.running:
            if r.generated < r.gen_len and r.prefilled + pre.get(r.rid, 0) == r.prompt_len:
                plan.decode.append(r.rid)
            elif r.generated >= r.gen_len:
                plan.padded.append(r.rid)  # static: its row still runs, to no use

    def _need(self, plan: StepPlan) -> int:
        """Paged: blocks the running requests hold after this iteration
        (Request.kv_tokens and blocks() written out)."""
        pre = {rid: k for rid, _, k in plan.prefill}
        dec = set(plan.decode)
        bs = self.bs
        n = 0
        for r in self.running:
            p = r.prefilled + pre.get(r.rid, 0)
            g = r.generated + (1 if r.rid in dec else 0)
            t = p + (g - 1 if g > 0 else 0) if p == r.prompt_len else p
            n += -(-t // bs)
        return n

    def _preempt(self, r: Request, plan: StepPlan):
        self.running.remove(r)
        r.prefilled, r.generated = 0, 0
        r.preemptions += 1
        self.queue.appendleft(r)
        plan.preempted.append(r.rid)
        if r.rid in plan.admitted:
            plan.admitted.remove(r.rid)

    def _release(self, r: Request, plan: StepPlan):
        self.running.remove(r)
        r.released = self.it
        self.done.append(r)
        plan.released.append(r.rid)

    def run(self, max_iterations: int = 1_000_000) -> List[Request]:
        while (self.pending or self.queue or self.running) and self.it < max_iterations:
            self.step()
        return self.done

    def summary(self) -> Dict:
        dec = [x["decode"] for x in self.history]
        return {"mode": self.mode, "iterations": self.it, "finished": len(self.done),
                "generated_tokens": int(sum(dec)),
                "mean_decode_batch": float(np.mean(dec)) if dec else 0.0,
                "padded_rows": int(sum(x["padded"] for x in self.history)),
                "max_running": max((x["running"] for x in self.history), default=0),
                "preemptions": int(sum(r.preemptions
                                       for r in self.done + self.running + list(self.queue)))}


class NativeScheduler:
    """The same scheduler in C++ (include/pa_scheduler.h, csrc/scheduler.cpp):
    the same decisions as Scheduler, plan by plan (the tests compare them),
    at a fraction of the host time per iteration.  Same constructor, step(),
    active(), prompt_len_of(), history and summary() as Scheduler; `done`
    holds the released requests' ids."""

    def __init__(self, mode: str, requests, num_blocks: int, block_size: int = 16,
                 max_batch: int = 256, max_step_tokens: int = 2048,
                 reserve_tokens: int = 4096):
        from .binding import NativeSchedulerHandle
        self.mode = mode
        self.bs = int(block_size)
        self.num_blocks = int(num_blocks)
        self.max_batch = int(max_batch)
        self.reserve_tokens = int(reserve_tokens)
        self.slots = self.num_blocks * self.bs // self.reserve_tokens
        self._h = NativeSchedulerHandle(mode, num_blocks, block_size, max_batch,
                                        max_step_tokens, reserve_tokens)
        reqs = list(requests)
        self._prompt_len = {r.rid: r.prompt_len for r in reqs}
        self._rids = [r.rid for r in reqs]
        if reqs:
            self._h.add([r.rid for r in reqs], [r.arrival for r in reqs],
                        [r.prompt_len for r in reqs], [r.gen_len for r in reqs])
        self.it = 0
        self.done: List[int] = []
        self.history: List[Dict] = []

    def step(self) -> StepPlan:
        it, p = self._h.step()
        self.it = it
        plan = StepPlan(it, prefill=p["prefill"], decode=p["decode"], padded=p["padded"],
                        admitted=p["admitted"], finished=p["finished"],
                        preempted=p["preempted"], released=p["released"])
        self.done.extend(plan.released)
        self.history.append({"iteration": it, "running": p["running"],
                             "decode": len(plan.decode), "padded": len(plan.padded),
                             "prefill_tokens": sum(k for _, _, k in plan.prefill),
                             "blocks_used": p["blocks_used"], "queued": p["queued"]})
        return plan

    def active(self) -> int:
        return self._h.active()

    def prompt_len_of(self, rid: int) -> int:
        return self._prompt_len[rid]

    def request(self, rid: int):
        """(admitted, prefilled, generated, finished, released, preemptions)
        of request rid, None for an iteration that has not happened."""
        return tuple(None if (i in (0, 3, 4) and v < 0) else v
                     for i, v in enumerate(self._h.request(rid)))

    def run(self, max_iterations: int = 1_000_000) -> List[int]:
        while self.active() and self.it < max_iterations:
            self.step()
        return self.done

    def summary(self) -> Dict:
        dec = [x["decode"] for x in self.history]
        return {"mode": self.mode, "iterations": self.it, "finished": len(self.done),
                "generated_tokens": int(sum(dec)),
                "mean_decode_batch": float(np.mean(dec)) if dec else 0.0,
                "padded_rows": int(sum(x["padded"] for x in self.history)),
                "max_running": max((x["running"] for x in self.history), default=0),
                "preemptions": int(sum(self._h.request(r)[5] for r in self._rids))}


def seeded_requests(n: int, seed: int, prompt=(64, 1024), gen=(16, 512), rate: float = 4.0):
    """n requests: prompt and generation lengths uniform in the given ranges,
    arrivals a Poisson process of `rate` requests per iteration (seeded)."""
    rng = np.random.default_rng([seed, 9])
    arrivals = np.floor(np.cumsum(rng.exponential(1.0 / rate, size=n))).astype(np.int64) + 1
    p = rng.integers(prompt[0], prompt[1] + 1, size=n)
    g = rng.integers(gen[0], gen[1] + 1, size=n)
    return [Request(i, int(arrivals[i]), int(p[i]), int(g[i])) for i in range(n)]


class Executor:
    """Runs a Scheduler's iterations through the library: the host block
    manager (include/pa_block_manager.h) places every token, and on the GPU
    pa_reshape_and_cache writes the new keys and values, pa_prefill attends
    with the prompt chunks and pa_decode with the running requests' newest
    tokens; one attention layer per iteration.

    Keys, values and queries are rows of seeded tables indexed by (request,
    position), so a request's data does not depend on when it runs; token
    ids (which only key the manager's prefix cache) are distinct per
    request, so no blocks are shared.  A static batch's finished rows stay
    in the decode call (its idle work).  ``observe(it, plan, info)`` is
    called after each iteration with what ran (for tests)."""

    def __init__(self, num_blocks: int, block_size: int = 16, num_q_heads: int = 32,
                 num_kv_heads: int = 8, head_dim: int = 128, dtype: str = "bf16",
                 device: str = "cuda:0", seed: int = 0, table_rows: int = 4096):
        import torch
        from . import binding as pa
        self.torch, self.pa = torch, pa
        td = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
        self.dtype, self.device = td, torch.device(device)
        self.nb, self.bs = int(num_blocks), int(block_size)
        self.hq, self.hkv, self.d = num_q_heads, num_kv_heads, head_dim
        shape = (self.nb, self.hkv, self.bs, self.d)
        self.k_cache = torch.zeros(shape, dtype=td, device=self.device)
        self.v_cache = torch.zeros(shape, dtype=td, device=self.device)
        self.bm = pa.BlockManager(self.nb, self.bs)
        g = torch.Generator().manual_seed(seed)
        self.rows = table_rows
        self.kv_table = torch.randn((table_rows, 2, self.hkv, self.d), generator=g).to(td)
        self.q_table = torch.randn((table_rows, self.hq, self.d), generator=g).to(td)
        self.k_dev = self.kv_table[:, 0].contiguous().to(self.device)
        self.v_dev = self.kv_table[:, 1].contiguous().to(self.device)
        self.q_dev = self.q_table.to(self.device)
        self.scale = float(np.float32(head_dim ** -0.5))
        self.kv_len: Dict[int, int] = {}      # tokens of each live request in the pool
        self.ws = None
        self.timing = False                   # bracket every kernel call with events
        self.events: List = []

    def _timed(self, fn, *a, **k):
        if not self.timing:
            return fn(*a, **k)
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        r = fn(*a, **k)
        e1.record()
        self.events.append((e0, e1))
        return r

    def kernel_ms(self) -> float:
        """Sum of the timed kernel calls since the last call (synchronises)."""
        self.torch.cuda.synchronize()
        t = sum(a.elapsed_time(b) for a, b in self.events)
        self.events = []
        return t

    def row_of(self, rid, pos):
        """Table row of (request, position); either may be an array."""
        return (np.asarray(rid, dtype=np.int64) * 7919 +
                np.asarray(pos, dtype=np.int64) * 104729) % self.rows

    def token_of(self, rid, pos):
        return ((np.asarray(rid, dtype=np.int64) << 16) ^
                np.asarray(pos, dtype=np.int64)) & 0x3FFFFFFF

    def _upload(self, *arrays):
        """Host integer arrays (int32 values) on the device without waiting
        for the GPU: packed into one pinned staging buffer from torch's
        caching host allocator (which keeps it until the copy has run) and
        copied asynchronously on the current stream, so the host can plan
        the next iteration while the kernels run.  Returns int32 device views
        of the arrays' shapes."""
        torch = self.torch
        sizes = [int(np.size(a)) for a in arrays]
        buf = torch.empty(sum(sizes), dtype=torch.int32, pin_memory=True)
        host = buf.numpy()
        o = 0
        for a, n in zip(arrays, sizes):
            host[o:o + n] = np.asarray(a).reshape(-1)
            o += n
        dev = buf.to(self.device, non_blocking=True)
        out, o = [], 0
        for a, n in zip(arrays, sizes):
            out.append(dev[o:o + n].view(np.shape(a)))
            o += n
        return out

    def _write(self, rows, slots):
        """Append the key and value rows `rows` (device int32) of the tables
        at `slots` (device int32)."""
        k = self.k_dev.index_select(0, rows)
        v = self.v_dev.index_select(0, rows)
        self._timed(self.pa.reshape_and_cache, k, v, self.k_cache, self.v_cache, slots)

    def _tables(self, rids):
        mb = max(1, -(-max(self.kv_len[r] for r in rids) // self.bs))
        return self.bm.tables(rids, mb)

    def iteration(self, sched: Scheduler, observe=None):
        """One scheduler step and the kernels it calls; returns the plan."""
        torch = self.torch
        plan = sched.step()
        info = {}
        for rid in plan.preempted:
            if rid in self.kv_len:
                self.bm.free(rid)
                del self.kv_len[rid]
        # prompt chunks: place, write, attend
        if plan.prefill:
            slots, q_rows, qs, prids = [], [], [0], []
            for rid, first, k in plan.prefill:
                pos = np.arange(first, first + k)
                toks = self.token_of(rid, pos).astype(np.int32)
                if first == 0:
                    _, sl = self.bm.add_sequence(rid, toks)
                else:
                    sl, _ = self.bm.append(rid, toks)
                self.kv_len[rid] = first + k
                slots.append(sl)
                q_rows.append(self.row_of(rid, pos))
                qs.append(qs[-1] + k)
                prids.append(rid)
            rows = np.concatenate(q_rows)  # a token's q, key and value share its row
            bt_h, lens_h = self._tables(prids)
            rows_d, sl, bt, lens, qs_d = self._upload(rows, np.concatenate(slots), bt_h, lens_h,
                                                      np.asarray(qs))
            self._write(rows_d, sl)
            q = self.q_dev.index_select(0, rows_d)
            out = self._timed(self.pa.prefill, q, self.k_cache, self.v_cache, bt, lens, qs_d,
                              scale=self.scale)
            info["prefill"] = (prids, q, qs, bt_h, lens_h, out)
        # newest tokens of the running requests: append, then attend
        completes = {rid for rid, first, k in plan.prefill
                     if first + k == sched.prompt_len_of(rid)}
        drids = [rid for rid in plan.decode if rid not in completes]
        new = []
        if drids:
            rid_a = np.asarray(drids, np.int64)
            pos = np.fromiter((self.kv_len[r] for r in drids), np.int64, len(drids))
            sl, cow = self.bm.append_batch(rid_a, self.token_of(rid_a, pos).astype(np.int32))
            assert len(cow) == 0
            for r in drids:
                self.kv_len[r] += 1
            new = [self.row_of(rid_a, pos), sl]
        rows = drids + [rid for rid in plan.padded if rid in self.kv_len]
        if rows:
            last = np.fromiter((self.kv_len[r] - 1 for r in rows), np.int64, len(rows))
            bt_h, lens_h = self._tables(rows)
            up = self._upload(self.row_of(rows, last), bt_h, lens_h, *new)
            if drids:
                self._write(up[3], up[4])
            q = self.q_dev.index_select(0, up[0])
            bt, lens = up[1], up[2]
            need = self.pa.decode_workspace_bytes(len(rows), self.hq, self.d, bt.shape[1], self.bs)
            if self.ws is None or self.ws.numel() < need:
                self.ws = torch.empty(max(need, 1 << 20) * 2, dtype=torch.uint8,
                                      device=self.device)
            out = self._timed(self.pa.decode, q, self.k_cache, self.v_cache, bt, lens,
                              scale=self.scale, workspace=self.ws)
            info["decode"] = (rows, q, bt_h, lens_h, out)
        # slots freed at the end of the iteration
        for r in plan.released:
            if r in self.kv_len:
                self.bm.free(r)
                del self.kv_len[r]
        if observe is not None:
            observe(sched.it, plan, info)
        return plan

    def run(self, sched: Scheduler, iterations: int, observe=None, timed: bool = False) -> Dict:
        """Run `iterations` iterations (or until the scheduler is idle).
        Returns the generated tokens, the host wall time and, with `timed`,
        the summed time of the kernel calls (HIP events around each, on the
        current stream)."""
        import time
        torch = self.torch
        torch.cuda.synchronize()
        self.timing, self.events = timed, []
        t0 = time.perf_counter()
        gen = dec_rows = pre = 0
        n = 0
        while n < iterations and sched.active():
            plan = self.iteration(sched, observe)
            gen += len(plan.decode)
            dec_rows += len(plan.decode) + len(plan.padded)
            pre += sum(k for _, _, k in plan.prefill)
            n += 1
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        out = {"iterations": n, "generated_tokens": gen, "decode_rows": dec_rows,
               "prefill_tokens": pre, "wall_s": wall}
        if timed:
            out["kernel_ms"] = self.kernel_ms()
        self.timing = False
        return out
