"""Pins of the oracle's supporting paths that every full-size parity check runs through.

* ``decode_bf16`` turns the bf16 bit patterns both sides receive into exact fp64 values.  It is
  checked against the bfloat16 format's definition (sign, 8-bit exponent with bias 127, 7-bit
  fraction, subnormals below exponent 1) on every one of the 65,536 patterns, against torch's
  own bf16 -> fp64 conversion, and against hand values.
* ``mean_f64`` (the router's pooled state, summary section 3 "Attention Router") sums rows in
  chunks of 8,192; here more than three chunks are summed and compared with correctly rounded
  sums (``math.fsum``), with a marker row planted in the last chunk so that a dropped or
  repeated chunk cannot pass.
* ``attention(..., workers > 1)`` splits the work over a thread pool; each task writes its own
  rows, so the result must equal the one-thread evaluation bit for bit, on a packed batch with
  full, streaming, block and block-list heads and empty / one-token sequences.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _bf16_by_definition(bits: int) -> float:
    """Value of one bfloat16 pattern from the format's fields (not from a float conversion)."""
    sign = -1.0 if bits >> 15 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return sign * math.inf if f == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)          # subnormal: 0.f x 2^-126
    return sign * math.ldexp(128 + f, e - 127 - 7)      # normal: 1.f x 2^(e - 127)


@pytest.mark.filterwarnings("ignore:invalid value encountered in cast")  # the NaN patterns
def test_decode_bf16_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_bf16(bits)
    want = np.array([_bf16_by_definition(int(b)) for b in bits.tolist()])
    nan = np.isnan(want)
    assert nan.sum() == 2 * 127                          # exponent 255 with a non-zero fraction
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    # the sign of zero survives
    assert math.copysign(1.0, got[0x8000]) == -1.0 and got[0x8000] == 0.0
    # torch's bf16 -> fp64 conversion agrees on every non-NaN pattern
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_decode_bf16_hand_values():
    cases = {0x3F80: 1.0, 0xC020: -2.5, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
             0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x4049: 3.140625, 0xBF00: -0.5,
             0x7F80: math.inf, 0xFF80: -math.inf}
    got = oracle.decode_bf16(np.array(list(cases), dtype=np.uint16))
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    # as_f64 decodes uint16 arrays and keeps float arrays as they are; shapes are kept
    x = np.array([[0x3F80, 0x4000], [0xC000, 0x0000]], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.as_f64(x), [[1.0, 2.0], [-2.0, 0.0]])
    np.testing.assert_array_equal(oracle.as_f64(np.float32([1.5, -3.25])), [1.5, -3.25])


def _round_bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_mean_f64_over_several_chunks():
    n, d = 3 * 8192 + 1234, 24                       # four chunks of the default 8,192 rows
    rng = np.random.default_rng(40)
    bits = _round_bf16(rng.standard_normal((n, d)))
    bits[n - 5] = _round_bf16(np.full(d, 2.0 ** 20))  # a marker in the last chunk
    rows = np.arange(n)
    got = oracle.mean_f64(bits, rows)
    vals = oracle.decode_bf16(bits)
    exact = np.array([math.fsum(vals[:, c]) / n for c in range(d)])
    np.testing.assert_allclose(got, exact, rtol=1e-14, atol=0)
    np.testing.assert_array_equal(oracle.mean_exact(vals), exact)
    # the marker alone moves every column by about 2^20 / n: a dropped last chunk would show
    assert np.all(got > 2.0 ** 20 / n * 0.9)
    # a non-contiguous row subset spanning the chunks, and other chunk sizes
    sub = np.arange(3, n, 7)
    exact_sub = np.array([math.fsum(vals[sub, c]) / len(sub) for c in range(d)])
    for chunk in (8192, 1000, 1 << 30):
        np.testing.assert_allclose(oracle.mean_f64(bits, sub, chunk=chunk), exact_sub, rtol=1e-14, atol=0)
    # and the router's plain path equals its exact path on this input
    w1 = rng.standard_normal((8, d))
    w2 = rng.standard_normal((3, 8))
    a = oracle.route(bits, [0, n], w1, w2)
    b = oracle.route(bits, [0, n], w1, w2, exact=True)
    np.testing.assert_allclose(a["pooled"], b["pooled"], rtol=1e-14, atol=0)
    np.testing.assert_allclose(a["logits"], b["logits"], rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("workers", [2, 8])
def test_threaded_attention_equals_one_thread(workers):
    lens = [70, 0, 1, 300, 129]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, D = int(cu[-1]), 8, 2, 16
    rng = np.random.default_rng(41)
    q = _round_bf16(rng.standard_normal((T, Hq, D)) * 0.5)
    k = _round_bf16(rng.standard_normal((T, Hkv, D)) * 0.5)
    v = _round_bf16(rng.standard_normal((T, Hkv, D)) * 0.5)
    mask = np.array([[1, 0], [0, 1], [0, 0], [0, 1], [1, 1]])
    patterns = [
        {"kind": "streaming", "sink": 3, "window": 20},
        {"kind": "block", "block": 16, "sink_blocks": 1, "local_blocks": 2, "stride_blocks": 5},
    ]
    lists = oracle.block_list_from_pattern(patterns[1], len(lens), Hkv, max(lens))
    # drop one listed block per row so the lists differ from the pattern
    rp = np.asarray(lists["row_ptr"])
    ci = list(lists["col_idx"])
    keep = np.ones(len(ci), dtype=bool)
    for r in range(len(rp) - 1):
        if rp[r + 1] - rp[r] > 1:
            keep[rp[r]] = False
    new_rp = np.concatenate([[0], np.cumsum([keep[rp[r]:rp[r + 1]].sum() for r in range(len(rp) - 1)])])
    patterns.append(dict(lists, row_ptr=new_rp.tolist(), col_idx=np.asarray(ci)[keep].tolist()))
    for sp in patterns:
        o1, l1 = oracle.attention(q, k, v, cu, mask, sp, block_rows=32, workers=1)
        on, ln = oracle.attention(q, k, v, cu, mask, sp, block_rows=32, workers=workers)
        np.testing.assert_array_equal(on, o1, err_msg=sp["kind"])
        np.testing.assert_array_equal(ln, l1, err_msg=sp["kind"])
        # a row and head subset: threads equal one thread bit for bit, and both equal the
        # slice of the whole evaluation up to rounding (the subset changes the operand shapes
        # of the row-block products, hence their summation order)
        rows = np.array([0, 69, 70, 71, 200, 370, T - 1])
        hs = [7, 0, 3]
        s1, t1 = oracle.attention(q, k, v, cu, mask, sp, rows=rows, heads=hs, block_rows=32)
        sn, tn = oracle.attention(q, k, v, cu, mask, sp, rows=rows, heads=hs, block_rows=32,
                                  workers=workers)
        np.testing.assert_array_equal(sn, s1)
        np.testing.assert_array_equal(tn, t1)
        np.testing.assert_allclose(sn, o1[rows][:, hs], rtol=0, atol=1e-14)
        np.testing.assert_allclose(tn, l1[hs][:, rows], rtol=0, atol=1e-14)
