"""Pins of the oracle's FP8 weights (``oracle.fp8``): the E4M3 decoder and the packed row layout,
and a whole step with FP8 matrices against the pinned bf16 step.

* The decoder, written from the format's definition, against torch's float8_e4m3fn conversion for
  all 256 codes (a library cross-check), and at the format's landmarks (1, the largest finite value
  448, the smallest normal 2^-6 and subnormal 2^-9, signed zero, the two NaN codes).
* Packing: a row's bytes are its codes, then its float32 scale, then zeros, and dequantizing gives
  code * scale exactly.
* A decode step and a prefill of a model whose matrices are FP8 with power-of-two row scales equal,
  bit for bit, the same model stored as bf16 (E4M3 values times powers of two are exact in bf16), so
  the FP8 path of the oracle is pinned to its bf16 path; the same model with one row scale dropped,
  or with scales applied per column, does not.
"""

import copy

import numpy as np
import pytest
import torch

import oracle
import oracle.prefill
from oracle import fp8
from decode_megakernel_03_amd import synth
from tests import harness

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_decoder_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_decoder_landmarks():
    t = fp8.e4m3_table()
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.isnan(t).sum() == 2
    assert np.nanmax(t) == 448.0


def test_packed_rows_layout_and_dequant():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, (3, 32)).astype(np.uint8)
    codes[codes & 0x7F == 0x7F] = 0x10
    scales = np.array([0.5, 3.25e-3, -7.0], np.float32)
    p = fp8.pack_rows(codes, scales)
    assert p.shape == (3, 48) and p.dtype == np.uint8
    assert np.array_equal(p[:, :32], codes) and not p[:, 36:].any()
    assert np.array_equal(p[:, 32:36].copy().view(np.float32)[:, 0], scales)
    d = fp8.dequant_rows(p, np.float64)
    assert np.array_equal(d, fp8.e4m3_to_f64(codes) * scales.astype(np.float64)[:, None])


def _fp8_twin(dw, seed=5, mutate=None):
    """The model with every matrix replaced by FP8 codes and power-of-two row scales (packed), and
    its bf16 twin holding the same values."""
    rng = np.random.default_rng(seed)
    q = copy.deepcopy(dw)
    b = copy.deepcopy(dw)

    def conv(u16):
        x = oracle.bf16_to_f32(u16).astype(np.float64)
        rows = x.reshape(-1, x.shape[-1])
        k = rng.integers(-9, -5, rows.shape[0]).astype(np.float64)
        sc = np.exp2(k)
        codes = torch.from_numpy((rows / sc[:, None]).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        packed = fp8.pack_rows(codes, sc.astype(np.float32)).reshape(x.shape[:-1] + (x.shape[-1] + 16,))
        vals = fp8.dequant_rows(packed, np.float64)
        if mutate == "drop":
            vals.reshape(-1, x.shape[-1])[0] /= sc[0]          # one row without its scale
        elif mutate == "columns":
            flat = vals.reshape(-1, x.shape[-1])
            flat[:] = fp8.e4m3_to_f64(codes) * np.resize(sc, x.shape[-1])[None, :]
        bf = oracle.f32_to_bf16(vals.astype(np.float32))
        assert np.array_equal(oracle.bf16_to_f32(bf).astype(np.float64), vals), "FP8 * 2^k must be exact in bf16"
        return packed, bf

    for ql, bl in zip(q.layers, b.layers):
        for name in ("w_qkv", "w_o", "w_router", "w_gate", "w_up", "w_down"):
            pk, bf = conv(getattr(ql, name))
            setattr(ql, name, pk)
            setattr(bl, name, bf)
    q.lm_head, b.lm_head = conv(dw.lm_head)
    return q, b


@pytest.fixture(scope="module")
def tiny():
    s = harness.tiny_setup(synth.workload("tiny", batch=2), ctx=[30, 9], gains="uniform")
    s["dims"] = harness.dims_of(s["wl"])
    s["dw"] = harness.dense_weights(s["w"])
    s["kv"] = harness.host_kv(s["k"], s["v"])
    return s


def _step(s, w):
    ctx = s["ctx"]
    return oracle.decode_step(s["dims"], w, copy.deepcopy(s["kv"]), s["tokens"], ctx.copy(), s["block_tables"], ctx + 1)


def test_fp8_step_equals_its_bf16_twin(tiny):
    q, b = _fp8_twin(tiny["dw"])
    rq, rb = _step(tiny, q), _step(tiny, b)
    assert np.array_equal(rq.logits, rb.logits) and np.array_equal(rq.topk, rb.topk)
    assert np.array_equal(rq.x_final, rb.x_final)
    # and the prefill
    bt = tiny["block_tables"][0]
    prompt = np.random.default_rng(2).integers(0, tiny["dims"].vocab, 11)
    pq = oracle.prefill.prefill(tiny["dims"], q, copy.deepcopy(tiny["kv"]), prompt, bt, 30)
    pb = oracle.prefill.prefill(tiny["dims"], b, copy.deepcopy(tiny["kv"]), prompt, bt, 30)
    assert np.array_equal(pq.logits, pb.logits) and np.array_equal(pq.topk, pb.topk)


@pytest.mark.parametrize("mutate", ["drop", "columns"])
def test_fp8_twin_check_catches_misapplied_scales(tiny, mutate):
    q, b = _fp8_twin(tiny["dw"], mutate=mutate)
    rq, rb = _step(tiny, q), _step(tiny, b)
    assert not np.array_equal(rq.logits, rb.logits)
