"""Pins of the oracle's fp8-page functions (readings R12-R14) against things other than
themselves: the OCP E4M3 definition's closed forms, torch's own float8_e4m3fn conversions (an
independent library routine), round trips, half-ulp error bounds, and the upper-bound invariant
of the page score. Each check also gets a broken copy of the oracle function (a planted mistake)
and must reject it."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

# ----------------------------------------------------------------------------------------------
# decoding
# ----------------------------------------------------------------------------------------------


def decode_ok(decode):
    codes = np.arange(256)
    v = np.asarray(decode(codes), dtype=np.float64)
    t = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = np.array_equal(np.isnan(v), np.isnan(t)) and np.array_equal(v[~np.isnan(v)], t[~np.isnan(t)])
    one = lambda c: float(np.asarray(decode([c]))[0])  # noqa: E731
    closed = (one(0x7E) == 448.0 and one(0xFE) == -448.0 and one(0x38) == 1.0
              and one(0x08) == 2.0 ** -6 and one(0x07) == 7 * 2.0 ** -9 and one(0x01) == 2.0 ** -9
              and one(0x00) == 0.0 and np.isnan(one(0x7F)) and np.isnan(one(0xFF)))
    return same and closed


def test_decode_every_code():
    assert decode_ok(O.fp8_e4m3_decode)


@pytest.mark.parametrize("mistake", ["bias_8", "no_subnormals", "four_mantissa_bits"])
def test_planted_decode_mistakes_are_caught(mistake):
    def broken(codes):
        c = np.asarray(codes, dtype=np.int64) & 0xFF
        sign = np.where(c & 0x80, -1.0, 1.0)
        if mistake == "four_mantissa_bits":
            e, m = (c >> 4) & 0x7, (c & 0xF) / 16.0
            return sign * (1.0 + m) * np.exp2(e - 3.0)
        e, m = (c >> 3) & 0xF, (c & 7) / 8.0
        bias = 8.0 if mistake == "bias_8" else 7.0
        mag = (1.0 + m) * np.exp2(e - bias)
        if mistake != "no_subnormals":
            mag = np.where(e == 0, m * 2.0 ** (1 - bias), mag)
        return sign * np.where((e == 15) & (c & 7 == 7), np.nan, mag)

    assert not decode_ok(broken)


# ----------------------------------------------------------------------------------------------
# encoding (R12)
# ----------------------------------------------------------------------------------------------


def encode_ok(encode):
    enc = lambda x: np.asarray(encode(np.asarray(x, dtype=np.float64)))  # noqa: E731
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    round_trip = np.array_equal(enc(O.fp8_e4m3_decode(finite)), finite)
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(40000) * np.exp2(rng.integers(-14, 9, 40000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    library = np.array_equal(enc(x), torch.from_numpy(x).to(torch.float8_e4m3fn)
                             .view(torch.uint8).numpy())
    ties = list(enc([1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10])) == [0x38, 0x3A, 0xB8,
                                                                              0x00, 0x02]
    saturation = list(enc([464.0, 1e6, -1e30, 448.0])) == [0x7E, 0x7E, 0xFE, 0x7E]
    zeros = list(enc([0.0, -0.0])) == [0x00, 0x80]
    return round_trip and library and ties and saturation and zeros


def test_encode():
    assert encode_ok(O.fp8_e4m3_encode)


@pytest.mark.parametrize("mistake", ["ties_away", "toward_zero", "nan_on_overflow"])
def test_planted_encode_mistakes_are_caught(mistake):
    table = O.fp8_e4m3_decode(np.arange(127))

    def broken(x):
        a = np.abs(x)
        hi = np.minimum(np.searchsorted(table, np.minimum(a, 448.0), side="left"), 126)
        lo = np.maximum(hi - 1, 0)
        d_lo, d_hi = np.minimum(a, 448.0) - table[lo], table[hi] - np.minimum(a, 448.0)
        if mistake == "ties_away":
            pick = d_hi <= d_lo
        elif mistake == "toward_zero":
            pick = np.zeros_like(d_hi, dtype=bool)
        else:
            pick = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
        code = np.where(table[hi] == np.minimum(a, 448.0), hi, np.where(pick, hi, lo))
        if mistake == "nan_on_overflow":
            code = np.where(a > 448.0, 0x7F, code)
        return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)

    assert not encode_ok(broken)


# ----------------------------------------------------------------------------------------------
# page quantization (R13)
# ----------------------------------------------------------------------------------------------


def quantize_ok(quantize):
    w = W.custom(31, B=2, Hq=4, Hkv=2, D=16, P=8, k=2, lens=[20, 9], dtype="bf16")
    pool = w.k_pool.clone()
    pool[0] = 0  # an all-zero tile
    pool[1, 1] *= 3.0e-3  # a small-valued tile
    codes, sc = quantize(pool)
    X = pool.double().numpy()
    amax = np.abs(X).reshape(X.shape[0], X.shape[1], -1).max(axis=2)
    want = np.where(amax > 0, np.float32(amax) / np.float32(448.0), np.float32(1.0))
    if not np.array_equal(np.asarray(sc, np.float32), want.astype(np.float32)):
        return False
    if not (np.asarray(codes)[0] == 0).all():
        return False
    deq = O.dequantize_pages(codes, sc)
    half_ulp = np.maximum(np.abs(X) * 2.0 ** -4, 2.0 ** -10 * np.asarray(sc)[:, :, None, None])
    if not (np.abs(X - deq) <= half_ulp * (1 + 1e-6)).all():
        return False
    # each tile's largest magnitude codes to +-448 (x / scale is 448 up to one fp32 rounding)
    for p in range(1, X.shape[0]):
        for j in range(X.shape[1]):
            i = np.unravel_index(np.argmax(np.abs(X[p, j])), X[p, j].shape)
            if abs(O.fp8_e4m3_decode([codes[p, j][i]])[0]) != 448.0:
                return False
    return True


def test_quantize_pages():
    assert quantize_ok(O.quantize_pages)


@pytest.mark.parametrize("mistake", ["max_240", "one_scale_per_page", "truncating_codes"])
def test_planted_quantize_mistakes_are_caught(mistake):
    def broken(pool):
        X = O.as_f64(pool).astype(np.float32)
        if mistake == "one_scale_per_page":
            amax = np.abs(X).reshape(X.shape[0], -1).max(axis=1)[:, None].repeat(X.shape[1], 1)
        else:
            amax = np.abs(X).reshape(X.shape[0], X.shape[1], -1).max(axis=2)
        top = np.float32(240.0 if mistake == "max_240" else 448.0)
        sc = np.where(amax > 0, amax / top, np.float32(1.0)).astype(np.float32)
        y = (X / sc[:, :, None, None]).astype(np.float32)
        if mistake == "truncating_codes":
            table = O.fp8_e4m3_decode(np.arange(127))
            idx = np.searchsorted(table, np.minimum(np.abs(y), 448.0), side="right") - 1
            return (idx | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8), sc
        return O.fp8_e4m3_encode(y), sc

    assert not quantize_ok(broken)


# ----------------------------------------------------------------------------------------------
# outward bf16 rounding and fp8 summaries (R14)
# ----------------------------------------------------------------------------------------------


def _bf16_order(x):
    """Orderable integer of each bf16 value (x must be bf16-representable)."""
    b = torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16)
    u = b.numpy().astype(np.int64)
    return np.where(u < 0, -(u & 0x7FFF), u)


def directed_ok(down, up):
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 256, 20000)
    codes = codes[(codes != 0x7F) & (codes != 0xFF)]
    scales = (rng.random(codes.size) * np.exp2(rng.integers(-12, 4, codes.size))).astype(np.float32)
    x = O.fp8_e4m3_decode(codes) * scales.astype(np.float64)  # exact products
    x = np.concatenate([x, [1.0, -3.0, 0.0, 2.0 ** -126 * 3]])
    d, u = np.asarray(down(x)), np.asarray(up(x))
    as_bf16 = lambda v: torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).double().numpy()  # noqa: E731
    if not (np.array_equal(as_bf16(d), d) and np.array_equal(as_bf16(u), u)):
        return False  # not bf16 values
    if not ((d <= x) & (x <= u)).all():
        return False
    exact = d == x
    if not np.array_equal(exact, u == x):
        return False
    gap = _bf16_order(u) - _bf16_order(d)
    return bool((gap[~exact] == 1).all())


def test_outward_bf16_rounding():
    assert directed_ok(O.bf16_round_down, O.bf16_round_up)


@pytest.mark.parametrize("mistake", ["nearest", "toward_zero"])
def test_planted_rounding_mistakes_are_caught(mistake):
    if mistake == "nearest":
        rne = lambda x: torch.from_numpy(np.asarray(x)).to(torch.float32).to(torch.bfloat16).double().numpy()  # noqa: E731
        assert not directed_ok(rne, rne)
    else:
        def tz(x):
            x = np.asarray(x, dtype=np.float64)
            m, e = np.frexp(x)
            return np.ldexp(np.trunc(m * 256.0), e - 8)
        assert not directed_ok(tz, tz)


def fp8_summaries_ok(summaries):
    """Every valid dequantized key lies inside [lo, hi]; lo and hi are within one bf16 step of
    the extremes; a one-hot query on any channel of a single-token page scores at least that
    key's value (the score's upper bound survives the quantization)."""
    w = W.custom(33, B=2, Hq=8, Hkv=2, D=16, P=8, k=3, lens=[37, 20], dtype="bf16")
    kc, ks = O.quantize_pages(w.k_pool)
    summ = summaries(kc, ks, w.page_table, w.seq_lens, w.P)
    deq = O.dequantize_pages(kc, ks)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        for n in range(O.n_pages(L, w.P)):
            p = int(w.page_table[b, n])
            valid = min(w.P, L - n * w.P)
            keys = deq[p, :, :valid, :]  # [Hkv][valid][D]
            lo, hi = summ[p, :, 0, :], summ[p, :, 1, :]
            if not ((lo <= keys.min(axis=1)) & (hi >= keys.max(axis=1))).all():
                return False
            if not (np.abs(_bf16_order(hi) - _bf16_order(O.bf16_round_up(keys.max(axis=1)))) == 0).all():
                return False
    # one-hot queries over single-token pages: the score is hi_d (q_d = 1) and must be >= k_d
    one = W.custom(34, B=1, Hq=2, Hkv=2, D=16, P=8, k=1, lens=[1], dtype="bf16")
    kc1, ks1 = O.quantize_pages(one.k_pool)
    s1 = summaries(kc1, ks1, one.page_table, one.seq_lens, one.P)
    k1 = O.dequantize_pages(kc1, ks1)
    p = int(one.page_table[0, 0])
    for d in range(one.D):
        q = torch.zeros((1, 2, one.D))
        q[0, :, d] = 1.0
        sc = O.page_scores(q, s1, one.page_table, one.seq_lens, one.P)
        if not (sc[0, :, 0] >= k1[p, :, 0, d]).all():
            return False
    return True


def test_fp8_summaries_contain_the_keys():
    assert fp8_summaries_ok(O.page_summaries_fp8)


def test_planted_fp8_summary_mistake_is_caught():
    def nearest(kc, ks, table, lens, P):
        s = O.page_summaries(O.dequantize_pages(kc, ks), table, lens, P)
        out = s.copy()
        ok = ~np.isnan(s)
        out[ok] = torch.from_numpy(s[ok]).to(torch.float32).to(torch.bfloat16).double().numpy()
        return out

    assert not fp8_summaries_ok(nearest)
