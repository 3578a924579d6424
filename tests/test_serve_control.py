"""The serving loop's control side on the CPU (no GPU): page pool, refills around a decode pause, and
collection of finished sequences, against a fake decode owner that finishes each sequence after its
budget of steps."""

import threading

import pytest

from decode_megakernel_03_amd.serve import ControlLoop, PagePool


class FakeServer:
    """Stands in for the library's decode owner: a step advances every active row by one token."""

    def __init__(self, max_batch):
        self.max_batch = max_batch
        self.active, self.pending, self.done = {}, [], {}
        self.paused = False
        self.events = []
        self.lock = threading.Lock()

    def pause(self):
        self.paused = True
        self.events.append("pause")

    def resume(self):
        self.paused = False
        self.events.append("resume")

    def submit(self, rid, pages, prompt_len, first, max_new, prompt=None):
        if prompt is None:
            assert self.paused, "a prefilled sequence must be submitted while decode is paused (its prefill just ran)"
        else:
            assert not self.paused and prompt_len == len(prompt)
            assert len(pages) * 16 >= prompt_len - 1 + max_new
        self.pending.append([rid, max_new, []])
        self.events.append(("submit", rid))

    def step(self):
        with self.lock:
            while self.pending and len(self.active) < self.max_batch:
                rid, n, out = self.pending.pop(0)
                self.active[rid] = [n, out]
            for rid in list(self.active):
                n, out = self.active[rid]
                out.append(len(out))
                if len(out) == n:
                    self.done[rid] = out
                    del self.active[rid]

    def poll(self):
        with self.lock:
            return [(rid, len(out)) for rid, out in self.done.items()]

    def take(self, rid):
        with self.lock:
            return self.done.pop(rid)


def test_page_pool_is_fifo_and_bounded():
    pool = PagePool(range(10))
    a = pool.alloc(4)
    assert a == [0, 1, 2, 3]
    pool.release(a[:2])
    assert pool.alloc(6) == [4, 5, 6, 7, 8, 9]
    assert pool.alloc(2) == [0, 1]
    with pytest.raises(RuntimeError):
        pool.alloc(3)


def test_control_loop_keeps_rows_busy_and_recycles_pages():
    srv = FakeServer(max_batch=3)
    pool = PagePool(range(40))
    reqs = [(20, 3, 1), (35, 1, 2), (10, 5, 3), (50, 2, 4), (5, 4, 5), (60, 1, 6), (17, 2, 7)]
    prefilled = []
    ctl = ControlLoop(srv, pool, reqs, prefill=lambda pages, n, seed: prefilled.append((tuple(pages), n)), page_size=16)
    steps = 0
    while not ctl.done():
        ctl.boundary()
        assert len(ctl.in_flight) <= 3
        srv.step()
        steps += 1
        assert steps < 100
    assert sorted(ctl.results) == list(range(7))
    assert all(len(ctl.results[r]) == reqs[r][1] for r in range(7))
    assert len(pool.free) == 40                      # every page came back
    assert len(prefilled) == 7
    # every prefill ran inside a pause and was followed by a submit before the resume
    ev = srv.events
    for i, e in enumerate(ev):
        if isinstance(e, tuple):
            assert ev[i - 1] == "pause" and ev[i + 1] == "resume"
    # pages cover prompt + budget
    for (pages, n), (c, o, _) in zip(prefilled, reqs):
        assert len(pages) * 16 >= c + o and n == c


def test_control_loop_as_a_thread():
    srv = FakeServer(max_batch=2)
    pool = PagePool(range(64))
    reqs = [(16 * (i % 3) + 1, 1 + i % 4, i) for i in range(12)]
    ctl = ControlLoop(srv, pool, reqs, prefill=lambda *a: None)
    stop = threading.Event()

    def decode():
        while not stop.is_set():
            srv.step()

    t = threading.Thread(target=decode, daemon=True)
    t.start()
    ctl.start()
    ctl.join(timeout=30)
    stop.set()
    t.join()
    assert sorted(ctl.results) == list(range(12))
    assert all(len(ctl.results[i]) == reqs[i][1] for i in range(12))


def test_control_loop_hands_prompts_to_the_server_without_pausing():
    """Requests that carry their prompts go to the server as they are (it prefills them in steps it
    shares with decode): no pause, pages for prompt_len - 1 + max_new positions, all collected."""
    srv = FakeServer(3)
    pool = PagePool(range(40))
    reqs = [([5] * n, o) for n, o in [(1, 2), (17, 3), (40, 1), (3, 5), (16, 1)]]
    ctl = ControlLoop(srv, pool, reqs, None)
    while not ctl.done():
        ctl.boundary()
        srv.step()
    assert "pause" not in srv.events
    assert sorted(ctl.results) == list(range(5))
    assert [len(ctl.results[i]) for i in range(5)] == [2, 3, 1, 5, 1]
    assert len(pool.free) == 40
