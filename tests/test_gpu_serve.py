"""The serving loop on the GPU: the library's C++ decode owner with the Python control side.

* Small model, three batch rows, twelve requests: the control loop runs as a thread of its own and
  keeps the rows busy (continuous batching, refills while decode is paused); every request's tokens
  equal the oracle's greedy decode of that request alone from the K/V its prefill wrote.
* Small model, four rows, ten requests that carry their prompts: the server prefills them in chunks
  mixed with decoding rows; every request's tokens equal the oracle's prefill + greedy decode.
* The 48-layer model on the ragged Zipf-routed batch of eight, stepped one step at a time: the first
  step, the step right after a finished sequence's row is refilled with a new prompt (schedule rebuilt,
  pages reused), and a step after a sequence left without a replacement are each checked against the
  oracle (teacher-forced on the GPU's tokens and KV cache), with the same gates as the other parity tests.
"""

import sys

import numpy as np
import pytest
import torch

from decode_megakernel_03_amd import synth
from tests import harness

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900),
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_serve_tiny_continuous_batching():
    import oracle
    from decode_megakernel_03_amd import mk, serve
    say("test_serve_tiny_continuous_batching: 3 rows, 12 requests, control loop thread")
    wl = synth.workload("tiny", batch=3)
    w = synth.make_weights(wl, seed=0, device="cuda")
    num_pages, max_pages = 96, 12
    k, v = synth.make_kv(wl, num_pages, device="cuda")
    eng = mk.Engine(wl, w, k, v, num_pages, max_pages, max_batch=3)
    reqs = synth.synthetic_requests(wl, seed=5, n=12, ctx=(1, 150), new_tokens=(1, 9))
    snaps = {}
    prefill = serve.synthetic_prefill(wl, k, v)

    def prefill_and_snapshot(pages, prompt_len, seed):
        prefill(pages, prompt_len, seed)
        snaps[seed] = [(synth.to_u16(k[l][pages]), synth.to_u16(v[l][pages])) for l in range(wl.n_layers)]

    srv = serve.Server(eng, 3)
    ctl = serve.ControlLoop(srv, serve.PagePool(np.random.default_rng(3).permutation(num_pages)), reqs,
                            prefill_and_snapshot, seed=0)
    ctl.start()
    ctl.join(timeout=300)
    st = srv.stats()
    srv.close()
    say(f"  {st.steps} steps, {st.tokens} tokens, {st.rebuilds} schedule rebuilds, {ctl.refills} refills")
    assert sorted(ctl.results) == list(range(12))
    dims = harness.dims_of(wl)
    dw = harness.dense_weights(w)
    for rid, (c, o, first) in enumerate(reqs):
        got = ctl.results[rid]
        assert len(got) == o
        n_pages = len(snaps[rid][0][0])
        kv = oracle.PagedKV(k=[s[0].copy() for s in snaps[rid]], v=[s[1].copy() for s in snaps[rid]])
        bt = np.arange(n_pages, dtype=np.int32)[None, :]
        res = oracle.greedy_decode(dims, dw, kv, [first], [c], bt, [c + 1], o)
        ref = [int(np.argmax(r.logits[0])) for r in res]
        say(f"  request {rid}: prompt {c}, {o} tokens: {got}")
        assert got == ref, f"request {rid}: GPU {got} != oracle {ref}"
    eng.close()


def test_serve_tiny_prompts_prefilled_in_mixed_batches():
    """Requests that carry their prompts: the server prefills them in chunks that share steps with the
    decoding sequences (no pause). Every request's tokens equal the oracle's: its prefill of the prompt
    but the last token, then greedy decode from the last prompt token, alone."""
    import oracle
    import oracle.prefill
    from decode_megakernel_03_amd import mk, serve
    say("test_serve_tiny_prompts_prefilled_in_mixed_batches: 4 rows, 10 prompts of 1..40 tokens")
    wl = synth.workload("tiny", batch=4)
    w = synth.make_weights(wl, seed=0, device="cuda", gains="uniform")
    num_pages, max_pages = 64, 4
    k, v = synth.make_kv(wl, num_pages, device="cuda")
    eng = mk.Engine(wl, w, k, v, num_pages, max_pages, max_batch=4)
    reqs = synth.synthetic_prompts(wl, seed=8, n=10, ctx=(1, 40), new_tokens=(1, 6))
    srv = serve.Server(eng, 4)
    ctl = serve.ControlLoop(srv, serve.PagePool(np.random.default_rng(4).permutation(num_pages)), reqs, None)
    ctl.start()
    ctl.join(timeout=300)
    st = srv.stats()
    srv.close()
    say(f"  {st.steps} steps, {st.tokens} generated, {st.prefill_tokens} prompt positions, {st.rebuilds} rebuilds")
    assert st.prefill_tokens == sum(len(p) - 1 for p, _ in reqs)
    dims = harness.dims_of(wl)
    dw = harness.dense_weights(w)
    for rid, (prompt, o) in enumerate(reqs):
        n = len(prompt)
        kv = oracle.PagedKV(k=[np.zeros((max_pages, wl.n_kv_heads, 16, wl.head_dim), np.uint16) for _ in range(wl.n_layers)],
                            v=[np.zeros((max_pages, wl.n_kv_heads, 16, wl.head_dim), np.uint16) for _ in range(wl.n_layers)])
        bt = np.arange(max_pages, dtype=np.int32)[None, :]
        if n > 1:
            oracle.prefill.prefill(dims, dw, kv, prompt[:-1].astype(np.int64), bt[0], 0)
        res = oracle.greedy_decode(dims, dw, kv, [int(prompt[-1])], [n - 1], bt, [n], o)
        ref = [int(np.argmax(r.logits[0])) for r in res]
        got = ctl.results[rid]
        say(f"  request {rid}: prompt {n}, {o} tokens: {got}")
        assert got == ref, f"request {rid}: GPU {got} != oracle {ref}"
    eng.close()


def test_serve_full_ragged_refill():
    from decode_megakernel_03_amd import mk, serve
    say("test_serve_full_ragged_refill: 48 layers, ragged Zipf batch of 8, refill after step 1")
    wl = synth.workload("ragged")
    bias = synth.zipf_router_bias(wl)
    w = synth.make_weights(wl, seed=0, device="cuda", router_bias=bias)
    ctx = synth.context_lengths(wl)
    budgets = [4, 3, 6, 2, 5, 4, 6, 3]
    need = [int((c + o + 15) // 16) for c, o in zip(ctx, budgets)]
    num_pages = int(sum(need))
    order = np.random.default_rng([1, 5]).permutation(num_pages)      # shuffled page assignment
    k, v = synth.make_kv(wl, num_pages, device="cuda")               # the initial prompts' K/V
    max_pages = max(need)
    eng = mk.Engine(wl, w, k, v, num_pages, max_pages, max_batch=8)
    L, B, K, E, V = wl.n_layers, 8, wl.top_k, wl.n_experts, wl.vocab
    topk = torch.zeros(L, B, K, dtype=torch.int32, device="cuda")
    rlog = torch.zeros(L, B, E, dtype=torch.float32, device="cuda")
    logits = torch.zeros(B, V, dtype=torch.float32, device="cuda")
    srv = serve.Server(eng, 8, start_held=True, topk_out=topk, router_logits_out=rlog, logits_out=logits)
    pool = serve.PagePool(order)
    firsts = synth.first_tokens(wl)
    pages_of = {}
    for b in range(8):
        pages_of[b] = pool.alloc(need[b])
        srv.submit(b, pages_of[b], int(ctx[b]), int(firsts[b]), budgets[b])
    # the refill: a new prompt of 1000 positions in the pages the finished sequence gave back
    refill = [(1000, 3, 777)]
    ctl = serve.ControlLoop(srv, pool, refill, serve.synthetic_prefill(wl, k, v), seed=11, first_id=8)
    for b in range(8):
        ctl.in_flight[b] = (pages_of[b], int(ctx[b]), budgets[b], int(firsts[b]))
    dims = harness.dims_of(wl)
    lw = harness.LazyWeights(w)
    checks = {0: "first step", 2: "after the refill", 3: "after a sequence left"}
    for step in range(4):
        kv0 = harness.host_kv(k, v) if step in checks else None
        say(f"  step {step}: run")
        srv.run(1)
        srv.wait()
        rec = srv.last_step()
        say(f"  step {step}: rows {rec['request_id']} positions {rec['position']} rebuilt {rec['rebuilt']}")
        if step in checks:
            nb = rec["batch"]
            bt = np.full((nb, max_pages), -1, np.int32)
            for i, rid in enumerate(rec["request_id"]):
                pg = ctl.in_flight[rid][0]
                bt[i, :len(pg)] = pg
            assert nb <= 8
            # the per-layer outputs are [L, batch, .] for the step's batch (rows packed with stride nb)
            g_topk = topk.cpu().numpy().reshape(-1)[:L * nb * K].reshape(L, nb, K)
            g_rlog = rlog.cpu().numpy().reshape(-1)[:L * nb * E].reshape(L, nb, E)
            stats = harness.check_full_step(
                dims, lw, kv0, rec["token_in"], rec["position"], bt, g_topk, g_rlog,
                logits.cpu().numpy()[:nb], rec["token_out"], near_tie=2e-4,
                router_tol=1e-4,
                g_kv=lambda l, page, slot: (synth.to_u16(k[l][page, :, slot, :]), synth.to_u16(v[l][page, :, slot, :])),
                kv_floor=1e-4)
            say(f"  step {step} ({checks[step]}): {stats}")
            lw.drop_layers()
        if step == 2:
            assert 8 in rec["request_id"] and rec["rebuilt"], "the refilled sequence joins the batch at step 2"
        if step == 3:      # sequences 1 and 7 (3 tokens each) left after step 2, with no replacement
            assert rec["batch"] == 6 and 1 not in rec["request_id"] and 7 not in rec["request_id"]
        c, r = ctl.boundary()  # the control side between steps: collect, then refill (decode paused)
        say(f"  after step {step}: {c} finished, {r} refilled")
        if step == 1:
            assert c == 1 and r == 1 and 3 in ctl.results and len(ctl.results[3]) == 2
            assert set(ctl.in_flight[8][0]) <= set(pages_of[3]), "the refill reuses the finished sequence's pages"
    srv.close()
    eng.close()
