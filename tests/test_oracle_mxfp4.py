"""Pins of the oracle's MXFP4 weights (``oracle.mxfp4``): the E2M1 and E8M0 decoders, the packed row
layout, and a whole step with MXFP4 matrices against the pinned bf16 step.

* E2M1 against the element table of the OCP Microscaling Formats (MX) v1.0 specification (FP4 E2M1:
  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; largest normal 6, smallest normal 1, the one subnormal 0.5,
  signed zero) - a document of its own, not the definition the decoder was written from.
* E8M0 against torch's float8_e8m0fnu conversion for all 256 codes (a library cross-check).
* Packing: nibble order, scale placement and zero padding byte by byte; the row length's inverse;
  dequantizing gives value(code) * 2^(scale - 127) per block of 32.
* The seeded quantizer that feeds both sides writes the layout the oracle reads, and its codes are
  nearest E2M1 values of the block-scaled inputs.
* A decode step and a prefill of a model whose matrices are MXFP4 equal, bit for bit, the same model
  stored as bf16 (E2M1 values times powers of two are exact in bf16), so the MXFP4 path of the oracle
  is pinned to its bf16 path; swapped nibbles, scales shifted by one block or one dropped block
  scale break the equality.
"""

import copy

import numpy as np
import pytest
import torch

import oracle
import oracle.prefill
from oracle import mxfp4
from decode_megakernel_03_amd import synth
from tests import harness

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

# OCP MX v1.0, FP4 (E2M1) element encodings 0b0000 .. 0b0111 (the sign bit negates them)
MX_SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_matches_the_mx_specification():
    t = mxfp4.e2m1_table()
    assert list(t[:8]) == MX_SPEC_E2M1
    assert list(t[8:]) == [-v for v in MX_SPEC_E2M1]
    assert not np.signbit(t[0]) and np.signbit(t[8])
    assert t.max() == 6.0 and t[0b0010] == 1.0 and t[0b0001] == 0.5 and not np.isnan(t).any()


def test_e8m0_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = mxfp4.e8m0_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_packed_rows_layout_and_dequant():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, (3, 64)).astype(np.uint8)
    scales = np.array([[127, 120], [130, 1], [0, 254]], np.uint8)
    p = mxfp4.pack_rows(codes, scales)
    assert isinstance(p, mxfp4.Mxfp4Rows) and p.k == 64 and p.shape == (3, 48) and p.dtype == np.uint8
    raw = np.asarray(p)
    assert np.array_equal(raw[:, :32] & 0xF, codes[:, 0::2]) and np.array_equal(raw[:, :32] >> 4, codes[:, 1::2])
    assert np.array_equal(raw[:, 32:34], scales) and not raw[:, 34:].any()
    d = mxfp4.dequant_rows(p, np.float64)
    for r in range(3):
        for b in range(2):
            want = [MX_SPEC_E2M1[c & 7] * (-1 if c & 8 else 1) * 2.0 ** (int(scales[r, b]) - 127)
                    for c in codes[r, 32 * b: 32 * b + 32]]
            assert np.array_equal(d[r, 32 * b: 32 * b + 32], want)
    assert p[1].k == 64 and copy.deepcopy(p).k == 64


@pytest.mark.parametrize("k", [32, 128, 256, 768, 2048, 4096])
def test_row_length_and_its_inverse(k):
    n = mxfp4.row_bytes(k)
    assert n % 16 == 0 and k // 2 + k // 32 <= n < k // 2 + k // 32 + 16
    assert mxfp4.k_of_row_bytes(n) == k and synth.mxfp4_row_bytes(k) == n


def test_seeded_quantizer_writes_the_oracle_layout():
    x = synth.normal_bf16((5, 256), 0.02, 0, 7)
    x[0, :32] = 0                                   # a zero block
    x[1, 5] = 0.3                                   # a block with one large entry
    p = synth.quantize_rows_mxfp4(x).numpy()
    assert p.shape == (5, mxfp4.row_bytes(256))
    rows = mxfp4.Mxfp4Rows(p, 256)
    d = mxfp4.dequant_rows(rows, np.float64)
    xs = x.float().double().numpy()
    # scale exponent = floor(log2 amax) - 2 per block, so |x| / scale lies in [0, 8)
    blocks = xs.reshape(5, 8, 32)
    amax = np.abs(blocks).max(-1)
    want = np.where(amax > 0, 127 + np.floor(np.log2(np.where(amax > 0, amax, 1))) - 2, 127)
    assert np.array_equal(p[:, 128:136], want.astype(np.uint8))
    # every code is a nearest E2M1 value of x / scale (below the clamp at 6)
    sc = np.repeat(mxfp4.e8m0_to_f64(p[:, 128:136]), 32, axis=-1)
    y = xs / sc
    grid = np.concatenate([mxfp4.e2m1_table()])
    best = np.abs(y[..., None] - grid).min(-1)
    got = np.abs(y - d / sc)
    inside = np.abs(y) <= 6
    assert np.all(got[inside] <= best[inside] + 1e-12)
    assert np.all(np.abs(d[~inside] / sc[~inside]) == 6)
    assert not d[0, :32].any()


def _nearest_codes(y):
    t = mxfp4.e2m1_table()
    return np.abs(y[..., None] - t).argmin(-1).astype(np.uint8)


def _mx_twin(dw, mutate=None):
    """The model with every matrix replaced by MXFP4 rows (block scales from the bf16 values), and its
    bf16 twin holding the same values."""
    q = copy.deepcopy(dw)
    b = copy.deepcopy(dw)

    def conv(u16):
        x = oracle.bf16_to_f32(u16).astype(np.float64)
        k = x.shape[-1]
        blocks = x.reshape(x.shape[:-1] + (k // 32, 32))
        amax = np.abs(blocks).max(-1)
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1))) - 2, 0)
        codes = _nearest_codes(blocks / np.exp2(e)[..., None]).reshape(x.shape)
        packed = mxfp4.pack_rows(codes, (e + 127).astype(np.uint8))
        vals = mxfp4.dequant_rows(packed, np.float64)
        flat = vals.reshape(-1, k)
        fc = codes.reshape(-1, k)
        fs = np.repeat(np.exp2(e).reshape(-1, k // 32), 32, axis=-1)
        t = mxfp4.e2m1_table()
        if mutate == "nibbles":                      # element 2i read from the high nibble
            sw = fc.copy()
            sw[:, 0::2], sw[:, 1::2] = fc[:, 1::2], fc[:, 0::2]
            flat[:] = t[sw] * fs
        elif mutate == "blocks":                     # each block scaled by its neighbour's scale
            flat[:] = t[fc] * np.roll(fs, 32, axis=-1)
        elif mutate == "drop":                       # one block without its scale
            flat[0, :32] = t[fc[0, :32]]
        bf = oracle.f32_to_bf16(vals.astype(np.float32))
        assert np.array_equal(oracle.bf16_to_f32(bf).astype(np.float64), vals), "E2M1 * 2^k must be exact in bf16"
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


def test_mxfp4_step_equals_its_bf16_twin(tiny):
    q, b = _mx_twin(tiny["dw"])
    rq, rb = _step(tiny, q), _step(tiny, b)
    assert np.array_equal(rq.logits, rb.logits) and np.array_equal(rq.topk, rb.topk)
    assert np.array_equal(rq.x_final, rb.x_final)
    bt = tiny["block_tables"][0]
    prompt = np.random.default_rng(2).integers(0, tiny["dims"].vocab, 11)
    pq = oracle.prefill.prefill(tiny["dims"], q, copy.deepcopy(tiny["kv"]), prompt, bt, 30)
    pb = oracle.prefill.prefill(tiny["dims"], b, copy.deepcopy(tiny["kv"]), prompt, bt, 30)
    assert np.array_equal(pq.logits, pb.logits) and np.array_equal(pq.topk, pb.topk)


@pytest.mark.parametrize("mutate", ["nibbles", "blocks", "drop"])
def test_mxfp4_twin_check_catches_misread_rows(tiny, mutate):
    q, b = _mx_twin(tiny["dw"], mutate=mutate)
    rq, rb = _step(tiny, q), _step(tiny, b)
    assert not np.array_equal(rq.logits, rb.logits)


def test_harness_reads_seeded_mxfp4_weights():
    wl = synth.workload("tiny_mxfp4")
    w = synth.make_weights(wl)
    dw = harness.dense_weights(w)
    assert isinstance(dw.layers[0].w_qkv, mxfp4.Mxfp4Rows) and dw.layers[0].w_qkv.k == wl.hidden
    assert dw.layers[0].w_down.k == wl.expert_ffn and dw.layers[0].w_o.k == wl.n_q_heads * wl.head_dim
    assert dw.lm_head.k == wl.hidden
