"""The serving loop's control side: requests, pages, prefill and batch management in Python, with a
C++ thread of libmk owning the decode loop (P3 "Scheduling and Performance Benchmarks": a Python
control thread handles control, prefill and batch management while a C++ thread owns decode; P1 "From
demo to a full serving system": continuous batching with ragged sequence lengths).

``Server`` wraps the library's decode owner (``mk_server_*``): it admits sequences at step
boundaries, prefills the prompts it is given in chunks that share steps with decoding sequences
(P3 "Limitations and Future Plans": mixed prefill/decode batches are the pages' next step), rebuilds
the schedule when the rows' composition changes and runs steps until told to hold.
``ControlLoop`` is the control side: it collects finished sequences and returns their pages to a
``PagePool``, and refills free batch rows from a request source. Requests either carry their prompt
tokens (the server prefills them, decode never pauses) or come with a ``prefill`` callable that the
loop runs while decode is paused (the pages' arrangement; the callable here writes seeded synthetic
K/V). It can run as a thread of its own (``start`` / ``join``) or one boundary at a time (``boundary``).
"""

import collections
import threading
import time

from . import mk, synth


class PagePool:
    """Free KV-cache pages (ids valid in every layer's cache), handed out first-in first-out."""

    def __init__(self, page_ids):
        self.free = collections.deque(int(p) for p in page_ids)
        self.total = len(self.free)

    def alloc(self, n):
        if n > len(self.free):
            raise RuntimeError(f"page pool exhausted: {n} pages asked, {len(self.free)} free")
        return [self.free.popleft() for _ in range(n)]

    def release(self, pages):
        self.free.extend(int(p) for p in pages)


class Server:
    """The library's decode owner over an ``mk.Engine`` (the engine belongs to it until ``close``)."""

    def __init__(self, engine, max_batch, start_held=False, topk_out=None, router_logits_out=None, hidden_out=None,
                 logits_out=None):
        self.engine = engine
        self._keep = (topk_out, router_logits_out, hidden_out, logits_out)
        self.h = mk.mk_server_create(engine.h, max_batch, start_held, topk_out, router_logits_out, hidden_out,
                                     logits_out)
        self.max_batch = max_batch

    def submit(self, request_id, pages, prompt_len, first_token, max_new_tokens, prompt=None):
        mk.mk_server_submit(self.h, request_id, pages, prompt_len, first_token, max_new_tokens, prompt)

    def pause(self):
        mk.mk_server_pause(self.h)

    def resume(self):
        mk.mk_server_resume(self.h)

    def run(self, n_steps=-1):
        mk.mk_server_run(self.h, n_steps)

    def wait(self):
        mk.mk_server_wait(self.h)

    def poll(self):
        return mk.mk_server_poll(self.h)

    def take(self, request_id):
        return mk.mk_server_take(self.h, request_id)

    def stats(self):
        return mk.mk_server_stats(self.h)

    def last_step(self):
        return mk.mk_server_last_step(self.h)

    def close(self):
        if getattr(self, "h", None):
            st = mk.mk_server_destroy(self.h)
            self.h = None
            if st != mk.MK_OK:
                raise mk.MkError(st, "decode owner failed")


class ControlLoop:
    """Control side of the serving loop over a ``Server``: keeps every batch row busy from ``requests``
    and collects finished sequences (tokens kept in ``results``), with pages from ``pool``.
    With ``prefill`` None, requests are (prompt tokens, max_new_tokens) and the server prefills them.
    Otherwise requests are (prompt_len, max_new_tokens, first_token) and ``prefill(pages, prompt_len,
    seed)`` writes the prompt's K/V while decode is paused. ``page_size`` sizes the allocation."""

    def __init__(self, server, pool, requests, prefill, page_size=16, seed=0, first_id=0):
        self.server, self.pool, self.requests, self.prefill = server, pool, iter(requests), prefill
        self.page_size, self.seed = page_size, seed
        self.next_id = first_id
        self.in_flight = {}                # request id -> (pages, prompt_len, max_new_tokens, first_token)
        self.results = {}                  # request id -> generated tokens
        self.budgets = {}
        self.refills = 0
        self.prefill_seconds = 0.0
        self.exhausted = False
        self.error = None
        self._stop = threading.Event()
        self._thread = None

    def collect(self):
        """Take every finished sequence and return its pages to the pool."""
        n = 0
        for rid, _ in self.server.poll():
            self.results[rid] = self.server.take(rid)
            pages = self.in_flight.pop(rid)[0]
            self.pool.release(pages)
            n += 1
        return n

    def refill(self):
        """Fill free batch rows with new requests: allocate pages, pause decode, prefill, submit, resume."""
        n = 0
        while not self.exhausted and len(self.in_flight) < self.server.max_batch:
            try:
                req = next(self.requests)
            except StopIteration:
                self.exhausted = True
                break
            rid = self.next_id
            if self.prefill is None:                          # the server prefills the prompt
                prompt, max_new = [int(t) for t in req[0]], int(req[1])
                pages = self.pool.alloc((len(prompt) - 1 + max_new + self.page_size - 1) // self.page_size)
                self.next_id += 1
                self.server.submit(rid, pages, len(prompt), 0, max_new, prompt=prompt)
                self.in_flight[rid] = (pages, len(prompt), max_new, prompt[-1])
                self.budgets[rid] = max_new
                self.refills += 1
                n += 1
                continue
            prompt_len, max_new, first = req
            pages = self.pool.alloc((prompt_len + max_new + self.page_size - 1) // self.page_size)
            self.next_id += 1
            t0 = time.perf_counter()
            self.server.pause()                               # decode paused while the prefill runs
            try:
                self.prefill(pages, prompt_len, self.seed * 1_000_003 + rid)
                self.server.submit(rid, pages, prompt_len, first, max_new)
            finally:
                self.server.resume()
            self.prefill_seconds += time.perf_counter() - t0
            self.in_flight[rid] = (pages, prompt_len, max_new, first)
            self.budgets[rid] = max_new
            self.refills += 1
            n += 1
        return n

    def boundary(self):
        """One pass of the control side: collect finished sequences, then refill free rows."""
        return self.collect(), self.refill()

    def done(self):
        return self.exhausted and not self.in_flight

    # ---- as a thread of its own
    def _run(self):
        try:
            while not self._stop.is_set() and not self.done():
                c, r = self.boundary()
                if c == 0 and r == 0:
                    time.sleep(0.0002)
        except Exception as e:                                # surfaced by join()
            self.error = e

    def start(self):
        self._thread = threading.Thread(target=self._run, name="mk-control", daemon=True)
        self._thread.start()

    def join(self, timeout=None):
        self._thread.join(timeout)
        if self._thread.is_alive():
            self._stop.set()
            self._thread.join()
            raise TimeoutError("control loop did not finish")
        if self.error is not None:
            raise self.error


def synthetic_prefill(wl, k, v):
    """A prefill that writes seeded N(0,1) K/V for the prompt's positions (synthetic stand-in)."""
    def run(pages, prompt_len, seed):
        import torch
        synth.prefill_pages(wl, k, v, pages, prompt_len, seed)
        torch.cuda.synchronize()
    return run
