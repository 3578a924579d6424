"""Prefill through the decode kernel on the GPU, against the oracle.

* Small model (bf16, FP8 and MXFP4 matrices): a 19-position prompt (chunks of 8, 8 and 3 rows of one
  sequence) written by ``mk_prefill`` from position 0 and after 21 cached positions, against ``oracle.prefill``: routing
  (near-tie replay as everywhere), the last position's logits, the K/V of every prompt position; then
  four greedy decode steps from the prompt's K/V equal the oracle's greedy decode.
* Small model, a mixed batch: two decode rows and a five-row chunk of a third sequence's prompt in
  one step, twice on one schedule (the chunk advances five positions per step), each step against
  the oracle's decode step over the same rows (which writes each row's K/V before the next row
  attends, so a chunk row sees the keys of the rows before it).
* The 48-layer model: a 9-position prompt after 1000 cached positions (a chunk of 8 rows, then 1),
  then a decode step from the K/V the prefill wrote.
Gates as in the other parity tests (router sets bit-exact up to replayed near-ties; logits max |d| <=
2e-2 and relative L2 <= 5e-3; identical greedy tokens; K/V within one bf16 step).
"""

import copy
import sys

import numpy as np
import pytest
import torch

from decode_megakernel_03_amd import synth
from tests import harness

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900),
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

MAX_ABS, MAX_REL_L2 = 2e-2, 5e-3
# Router logits of a step whose rows attend to keys other rows wrote in the same step: such a key is
# an fp32 result rounded to bf16, and two correct fp32 results may round one bf16 step apart; every
# later row of the chunk then attends to the flipped entry. On the mixed batch below the oracle's own
# fp32 and fp64 runs differ by 1.8e-5 in layer 1 of the chunk's second row at the second step for
# exactly this reason, so the gate is 5e-5 (half the near-tie band) instead of the decode tests' 1e-5.
ROUTER_TOL_CHUNK = 5e-5
# Likewise the K/V rows the later chunk rows write in the next layer carry that deviation: the same
# fp32 / fp64 comparison puts one entry of that step beyond one bf16 step + 1e-5 (14 entries differ),
# so the chunk test takes the floor of the full-size tests, 1e-4, instead of 1e-5.
KV_FLOOR_CHUNK = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(w):
    out = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in w.items() if k != "layers"}
    out["layers"] = [{k: (v.cuda() if torch.is_tensor(v) else v) for k, v in lw.items()} for lw in w["layers"]]
    return out


def check_logits(g, ref, where):
    d = np.abs(g.astype(np.float64) - ref).max()
    rel = np.linalg.norm(g.astype(np.float64) - ref) / np.linalg.norm(ref)
    assert d <= MAX_ABS and rel <= MAX_REL_L2, f"{where}: logits max|d| {d:.3g} rel L2 {rel:.3g}"
    return float(d), float(rel)


def oracle_prefill(dims, w, kv0, prompt, bt_row, start, g_topk, near_tie):
    """oracle.prefill with the GPU's near-tied routing decisions replayed; returns (result, kv)."""
    import oracle.prefill
    last = {}

    def run(forced):
        kv = copy.deepcopy(kv0)
        last["kv"] = kv
        return oracle.prefill.prefill(dims, w, kv, np.asarray(prompt, np.int64), bt_row, start, forced_topk=forced)

    ref, replay = harness.replay_near_ties(run, g_topk, near_tie)
    return ref, last["kv"], replay


def prompt_rows_check(dims, kd, vd, kv_ref, bt_row, positions, max_frac):
    """The GPU's K/V at the prompt positions against the oracle's: within one bf16 step, few differ."""
    nbad = ndiff = ntot = 0
    for l in range(dims.n_layers):
        for dev, host in ((kd, kv_ref.k), (vd, kv_ref.v)):
            for p in positions:
                page, slot = int(bt_row[p // dims.page_size]), p % dims.page_size
                g16 = synth.to_u16(dev[l][page, :, slot, :])
                h16 = host[l][page, :, slot, :]
                nbad += int(harness.bf16_step_mismatch(g16, h16, floor=1e-4).sum())
                ndiff += int((g16 != h16).sum())
                ntot += g16.size
    assert nbad == 0 and ndiff <= max(2, int(ntot * max_frac)), f"prompt K/V: {nbad} beyond one bf16 step, {ndiff}/{ntot} differ"
    return f"{ndiff}/{ntot}"


@pytest.mark.parametrize("start", [0, 21], ids=["from-position-0", "after-21-cached"])
@pytest.mark.parametrize("name", ["tiny", "tiny_fp8", "tiny_mxfp4"])
def test_tiny_prefill_then_decode(name, start):
    import oracle
    from decode_megakernel_03_amd import mk
    n = 19
    say(f"test_tiny_prefill_then_decode: {name}, prompt of {n} at position {start}, chunks of 8")
    wl = synth.workload(name, steps=n + 8)
    s = harness.tiny_setup(wl, ctx=[start], gains="uniform")
    dims = harness.dims_of(wl)
    dw = harness.dense_weights(s["w"])
    kv0 = harness.host_kv(s["k"], s["v"])
    kd = [t.cuda() for t in s["k"]]
    vd = [t.cuda() for t in s["v"]]
    bt = s["block_tables"]
    eng = mk.Engine(wl, to_dev(s["w"]), kd, vd, s["num_pages"], bt.shape[1], max_batch=8)
    prompt = np.random.default_rng(3).integers(0, wl.vocab, n)
    L, K = wl.n_layers, wl.top_k
    logits = torch.zeros(wl.vocab, dtype=torch.float32, device="cuda")
    topk = torch.zeros(L, n, K, dtype=torch.int32, device="cuda")
    eng.prefill(prompt.tolist(), start, bt[0].tolist(), logits_out=logits, topk_out=topk)
    torch.cuda.synchronize()
    eng.sync()
    ref, kv_ref, replay = oracle_prefill(dims, dw, kv0, prompt, bt[0], start, topk.cpu().numpy(), 1e-4)
    g = logits.cpu().numpy()
    d, rel = check_logits(g, ref.logits, "prefill")
    assert int(np.argmax(g)) == int(np.argmax(ref.logits)), "first generated token differs"
    frac = prompt_rows_check(dims, kd, vd, kv_ref, bt[0], range(start, start + n), 0.02)
    say(f"  prefill: logits max|d| {d:.2e} rel {rel:.2e}, near-tie replays {len(replay)}, prompt K/V differ {frac}")
    # greedy decode from the prompt's K/V, both sides free-running
    steps = 4
    tok = int(np.argmax(g))
    pos = start + n
    eng.build_schedule([pos + 1])
    argmax = torch.zeros(1, dtype=torch.int32, device="cuda")
    eng.set_step_outputs(argmax_out=argmax)
    lg = torch.zeros(1, wl.vocab, dtype=torch.float32, device="cuda")
    btd = torch.from_numpy(bt).cuda()
    got = []
    for i in range(steps):
        eng.step(torch.tensor([tok], dtype=torch.int32, device="cuda"), torch.tensor([pos + i], dtype=torch.int32, device="cuda"),
                 btd, torch.tensor([pos + i + 1], dtype=torch.int32, device="cuda"), lg)
        torch.cuda.synchronize()
        eng.sync()
        tok = int(argmax.cpu().numpy()[0])
        got.append(tok)
    res = oracle.greedy_decode(dims, dw, kv_ref, [int(np.argmax(ref.logits))], [pos], bt, [pos + 1], steps)
    want = [int(np.argmax(r.logits[0])) for r in res]
    say(f"  decode after prefill: GPU {got}, oracle {want}")
    assert got == want
    eng.close()


def test_tiny_mixed_prefill_decode_batch():
    from decode_megakernel_03_amd import mk
    say("test_tiny_mixed_prefill_decode_batch: rows [A, B x5, C], two steps on one schedule")
    wl = synth.workload("tiny", batch=3, steps=16)
    s = harness.tiny_setup(wl, ctx=[40, 13, 7], gains="uniform")
    dims = harness.dims_of(wl)
    dw = harness.dense_weights(s["w"])
    kd = [t.cuda() for t in s["k"]]
    vd = [t.cuda() for t in s["v"]]
    bt3 = s["block_tables"]
    eng = mk.Engine(wl, to_dev(s["w"]), kd, vd, s["num_pages"], bt3.shape[1], max_batch=8)
    rows_of = [0, 1, 1, 1, 1, 1, 2]             # sequence of each row
    B, C, L, K, E = len(rows_of), 5, wl.n_layers, wl.top_k, wl.n_experts
    bt = bt3[rows_of]
    prompt_b = np.random.default_rng(9).integers(0, wl.vocab, 2 * C)
    tok_a, tok_c = int(s["tokens"][0]), int(s["tokens"][2])
    pos = np.array([40, 13, 14, 15, 16, 17, 7], np.int64)
    eng.build_schedule((pos + 1).tolist(), rows_per_seq=C)
    argmax = torch.zeros(8, dtype=torch.int32, device="cuda")
    topk = torch.zeros(L * 8 * K, dtype=torch.int32, device="cuda")
    rlog = torch.zeros(L * 8 * E, dtype=torch.float32, device="cuda")
    eng.set_step_outputs(argmax_out=argmax, topk_out=topk, router_logits_out=rlog)
    logits = torch.zeros(B, wl.vocab, dtype=torch.float32, device="cuda")
    btd = torch.from_numpy(bt).cuda()
    for step in range(2):
        tokens = np.array([tok_a] + prompt_b[step * C:(step + 1) * C].tolist() + [tok_c], np.int64)
        kv0 = harness.host_kv(kd, vd)
        say(f"  step {step}: positions {pos.tolist()}")
        eng.step(torch.from_numpy(tokens.astype(np.int32)).cuda(), torch.from_numpy(pos.astype(np.int32)).cuda(), btd,
                 torch.from_numpy((pos + 1).astype(np.int32)).cuda(), logits)
        torch.cuda.synchronize()
        eng.sync()
        g_arg = argmax.cpu().numpy()[:B]
        stats = harness.check_full_step(
            dims, dw, kv0, tokens, pos, bt, topk.cpu().numpy()[:L * B * K].reshape(L, B, K),
            rlog.cpu().numpy()[:L * B * E].reshape(L, B, E), logits.cpu().numpy(), g_arg, near_tie=1e-4,
            router_tol=ROUTER_TOL_CHUNK, g_kv=lambda l, page, slot: (synth.to_u16(kd[l][page, :, slot, :]), synth.to_u16(vd[l][page, :, slot, :])),
            kv_floor=KV_FLOOR_CHUNK)
        say(f"  step {step}: {stats}")
        assert eng.rebuilds == 0, "the chunk's schedule serves both steps"
        tok_a, tok_c = int(g_arg[0]), int(g_arg[-1])
        pos = pos + np.array([1] + [C] * C + [1])
    eng.close()


def test_full_prefill_then_decode():
    from decode_megakernel_03_amd import mk
    start, n = 1000, 9
    say(f"test_full_prefill_then_decode: 48 layers, prompt of {n} after {start} cached positions")
    wl = synth.workload("full")
    w = synth.make_weights(wl, seed=0, device="cuda")
    ctx = np.array([start], np.int64)
    bt, num_pages = synth.make_block_tables(ctx, 16, wl.page_size)
    k, v = synth.make_kv(wl, num_pages, device="cuda")
    dims = harness.dims_of(wl)
    lw = harness.LazyWeights(w)
    kv0 = harness.host_kv(k, v)
    eng = mk.Engine(wl, w, k, v, num_pages, bt.shape[1], max_batch=8)
    prompt = np.random.default_rng(17).integers(0, wl.vocab, n)
    L, K, E = wl.n_layers, wl.top_k, wl.n_experts
    logits = torch.zeros(wl.vocab, dtype=torch.float32, device="cuda")
    topk = torch.zeros(L, n, K, dtype=torch.int32, device="cuda")
    say("  prefill: launch")
    eng.prefill(prompt.tolist(), start, bt[0].tolist(), logits_out=logits, topk_out=topk)
    torch.cuda.synchronize()
    eng.sync()
    say("  prefill: oracle")
    ref, kv_ref, replay = oracle_prefill(dims, lw, kv0, prompt, bt[0], start, topk.cpu().numpy(), 2e-4)
    g = logits.cpu().numpy()
    d, rel = check_logits(g, ref.logits, "prefill")
    assert int(np.argmax(g)) == int(np.argmax(ref.logits)), "first generated token differs"
    frac = prompt_rows_check(dims, k, v, kv_ref, bt[0], range(start, start + n), 0.02)
    say(f"  prefill: logits max|d| {d:.2e} rel {rel:.2e}, near-tie replays {len(replay)}, prompt K/V differ {frac}")
    lw.drop_layers()
    # a decode step from the K/V the prefill wrote (teacher-forced on the GPU's cache)
    kv1 = harness.host_kv(k, v)
    pos = start + n
    tok = int(np.argmax(g))
    eng.build_schedule([pos + 1])
    argmax = torch.zeros(1, dtype=torch.int32, device="cuda")
    tk = torch.zeros(L, 1, K, dtype=torch.int32, device="cuda")
    rl = torch.zeros(L, 1, E, dtype=torch.float32, device="cuda")
    eng.set_step_outputs(argmax_out=argmax, topk_out=tk, router_logits_out=rl)
    lg = torch.zeros(1, wl.vocab, dtype=torch.float32, device="cuda")
    say("  decode step: launch")
    eng.step(torch.tensor([tok], dtype=torch.int32, device="cuda"), torch.tensor([pos], dtype=torch.int32, device="cuda"),
             torch.from_numpy(bt).cuda(), torch.tensor([pos + 1], dtype=torch.int32, device="cuda"), lg)
    torch.cuda.synchronize()
    eng.sync()
    stats = harness.check_full_step(dims, lw, kv1, [tok], [pos], bt, tk.cpu().numpy(), rl.cpu().numpy(), lg.cpu().numpy(),
                                    argmax.cpu().numpy(), near_tie=2e-4, router_tol=1e-4,
                                    g_kv=lambda l, page, slot: (synth.to_u16(k[l][page, :, slot, :]), synth.to_u16(v[l][page, :, slot, :])),
                                    kv_floor=1e-4)
    say(f"  decode step after prefill: {stats}")
    eng.close()
