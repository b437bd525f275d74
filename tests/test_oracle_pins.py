"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each check is written from the mathematics or the pages, never by retyping the oracle's formula:
brute force on tiny inputs, closed forms, invariants, hand-worked examples (tests/golden/), and
special cases that reduce to a library routine (torch's scaled_dot_product_attention on the CPU,
NumPy complex multiplication). The ``planted`` tests feed each check a deliberately broken copy of
an oracle function and require the check to fail, so a dropped term, a wrong sign or index, or a
transposed operand cannot pass unnoticed.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


# ----------------------------------------------------------------------------------------------
# a1 summaries
# ----------------------------------------------------------------------------------------------

def check_summaries(fn, w):
    """Brute-force Python min/max over the valid slots of every referenced page."""
    summ = fn(w.k_pool, w.page_table, w.seq_lens, w.P)
    K = w.k_pool.to(torch.float64)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        for n in range(-(-L // w.P)):
            p = int(w.page_table[b, n])
            valid = min(w.P, L - n * w.P)
            for j in range(w.Hkv):
                for d in range(w.D):
                    col = [float(K[p, j, s, d]) for s in range(valid)]
                    if summ[p, j, 0, d] != min(col) or summ[p, j, 1, d] != max(col):
                        return False
    return True


def test_summaries_brute_force_ragged():
    w = W.custom(7, B=3, Hq=4, Hkv=2, D=8, P=4, k=2, lens=[7, 1, 12], dtype="bf16",
                 spare_pages=2)
    assert check_summaries(O.page_summaries, w)


def test_summaries_ignore_padding_and_single_token():
    w = W.custom(8, B=1, Hq=2, Hkv=1, D=4, P=4, k=1, lens=[5], dtype="f32", permute=False)
    # slots 1..3 of the last page (logical page 1 -> physical 1) are padding: poison them
    w.k_pool[1, :, 1:, :] = float("nan")
    summ = O.page_summaries(w.k_pool, w.page_table, w.seq_lens, w.P)
    assert np.isfinite(summ[1]).all()
    # a page with one valid token has lo == hi == that key
    np.testing.assert_array_equal(summ[1, 0, 0], w.k_pool[1, 0, 0].double().numpy())
    np.testing.assert_array_equal(summ[1, 0, 1], w.k_pool[1, 0, 0].double().numpy())


@pytest.mark.parametrize("mistake", ["all_slots", "no_min"])
def test_planted_summary_mistakes_are_caught(mistake):
    w = W.custom(7, B=3, Hq=4, Hkv=2, D=8, P=4, k=2, lens=[7, 1, 12], dtype="bf16")

    def broken(k_pool, page_table, seq_lens, P):
        if mistake == "all_slots":  # ignores the valid-slot limit of a partial page
            big = W.custom(7, B=3, Hq=4, Hkv=2, D=8, P=4, k=2, lens=[8, 4, 12], dtype="bf16")
            return O.page_summaries(k_pool, big.page_table, big.seq_lens, P)
        s = O.page_summaries(k_pool, page_table, seq_lens, P)
        s[:, :, 0] = s[:, :, 1]  # lo replaced by hi
        return s

    assert not check_summaries(broken, w)


# ----------------------------------------------------------------------------------------------
# decode-time append
# ----------------------------------------------------------------------------------------------

def check_append(fn, lens):
    """A cache filled one token at a time from empty equals the cache built at once: every valid
    slot holds the reference key and value, nothing else is written, the lengths match, and a
    full table refuses the next token."""
    w = W.custom(17, B=len(lens), Hq=4, Hkv=2, D=8, P=4, k=2, lens=lens, dtype="f32")
    Kref, Vref = w.k_pool.double().numpy(), w.v_pool.double().numpy()
    table = w.page_table.numpy()
    K = np.full_like(Kref, np.nan)
    V = np.full_like(Vref, np.nan)
    cur = np.zeros(w.B, dtype=np.int64)
    Lmax = int(max(lens))
    for t in range(Lmax):
        kn = np.zeros((w.B, w.Hkv, w.D))
        vn = np.zeros((w.B, w.Hkv, w.D))
        for b in range(w.B):
            if t < lens[b]:  # the reference token at position t
                p, sl = int(table[b, t // w.P]), t % w.P
                kn[b], vn[b] = Kref[p, :, sl, :], Vref[p, :, sl, :]
        K2, V2, cur2, rej = fn(K, V, table, cur, kn, vn, w.P)
        for b in range(w.B):  # sequences already complete keep their state
            if t >= lens[b]:
                K2, V2 = K2.copy(), V2.copy()
                if not rej[b]:
                    p, sl = int(table[b, int(cur[b]) // w.P]), int(cur[b]) % w.P
                    K2[p, :, sl, :], V2[p, :, sl, :] = K[p, :, sl, :], V[p, :, sl, :]
                cur2[b] = cur[b]
        K, V, cur = K2, V2, cur2
    if list(cur) != list(lens):
        return False
    for b in range(w.B):
        for t in range(Lmax):
            p, sl = int(table[b, t // w.P]), t % w.P
            if t < lens[b]:
                if not (np.array_equal(K[p, :, sl], Kref[p, :, sl])
                        and np.array_equal(V[p, :, sl], Vref[p, :, sl])):
                    return False
            elif t // w.P < -(-lens[b] // w.P) and not np.isnan(K[p, :, sl]).all():
                return False  # a slot past the length was written
    # a full table takes no further token
    full = np.array([table.shape[1] * w.P] * w.B)
    _, _, cur3, rej = fn(K, V, table, full, np.ones((w.B, w.Hkv, w.D)), np.ones((w.B, w.Hkv, w.D)),
                         w.P)
    return bool(rej.all()) and list(cur3) == list(full)


@pytest.mark.parametrize("lens", [[21, 21], [9, 16, 3], [1, 4, 5]])
def test_append_builds_the_cache_token_by_token(lens):
    assert check_append(O.append_tokens, lens)


@pytest.mark.parametrize("mistake", ["next_slot", "slot_as_page", "keeps_length", "no_bound"])
def test_planted_append_mistakes_are_caught(mistake):
    def broken(k_pool, v_pool, page_table, seq_lens, k_new, v_new, P):
        lens = np.asarray(seq_lens)
        if mistake == "next_slot":  # writes one position too far
            return O.append_tokens(k_pool, v_pool, page_table, lens + 1, k_new, v_new, P)[:2] + \
                O.append_tokens(k_pool, v_pool, page_table, lens, k_new, v_new, P)[2:]
        if mistake == "slot_as_page":  # logical page from the slot instead of the position
            K, V = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
            out = lens.copy()
            for b in range(len(lens)):
                L = int(lens[b])
                p = int(np.asarray(page_table)[b, L % P])
                K[p, :, L % P], V[p, :, L % P] = k_new[b], v_new[b]
                out[b] = L + 1
            return K, V, out, np.zeros(len(lens), dtype=bool)
        if mistake == "keeps_length":
            K, V, _, rej = O.append_tokens(k_pool, v_pool, page_table, lens, k_new, v_new, P)
            return K, V, lens.copy(), rej
        K, V, out, rej = O.append_tokens(k_pool, v_pool, page_table, lens, k_new, v_new, P)
        return K, V, np.where(rej, lens + 1, out), np.zeros_like(rej)  # full tables accepted

    assert not all(check_append(broken, lens) for lens in ([21, 21], [9, 16, 3]))


# ----------------------------------------------------------------------------------------------
# a2 scores
# ----------------------------------------------------------------------------------------------

def check_score_bound(score_fn, w):
    """Invariant: each page's score >= the largest group dot product sum_g q_g.k_t of its keys
    (exact sums; rounding to fp32 is monotone so the rounded bound stays above)."""
    summ = O.page_summaries(w.k_pool, w.page_table, w.seq_lens, w.P)
    sc = score_fn(w.q, summ, w.page_table, w.seq_lens, w.P)
    Q = w.q.to(torch.float64).numpy()
    K = w.k_pool.to(torch.float64).numpy()
    G = w.G
    for b in range(w.B):
        L = int(w.seq_lens[b])
        for n in range(-(-L // w.P)):
            p = int(w.page_table[b, n])
            valid = min(w.P, L - n * w.P)
            for j in range(w.Hkv):
                qsum = Q[b, j * G:(j + 1) * G]
                best = max(math.fsum((qsum @ np.diag(K[p, j, t])).ravel())
                           for t in range(valid))
                if not sc[b, j, n] >= np.float32(best):
                    return False
    return True


def test_score_hand_example():
    g = json.load(open(os.path.join(GOLD, "score_hand_example.json")))
    q = torch.tensor([g["group_queries"]], dtype=torch.float32)  # [1][2][2]
    keys = np.array(g["page_keys"], dtype=np.float32)  # 3 tokens
    pool = torch.zeros(1, 1, 4, 2)
    pool[0, 0, :3] = torch.from_numpy(keys)
    summ = O.page_summaries(pool, torch.zeros(1, 1, dtype=torch.int32), torch.tensor([3]), 4)
    np.testing.assert_array_equal(summ[0, 0, 0], g["lo"])
    np.testing.assert_array_equal(summ[0, 0, 1], g["hi"])
    sc = O.page_scores(q, summ, torch.zeros(1, 1, dtype=torch.int32), torch.tensor([3]), 4)
    assert sc[0, 0, 0] == g["score"]
    assert sc[0, 0, 0] >= g["true_max_group_dot"]


@pytest.mark.parametrize("wl", ["tiny", "bf16"])
def test_score_upper_bounds_every_key(wl):
    if wl == "tiny":
        w = W.tiny_fp32()
        # trim to a few pages to keep the brute force quick
        w = W.Workload(w.name, w.dtype, 1, w.Hq, w.Hkv, w.D, w.P, 4,
                       torch.tensor([8 * w.P + 5], dtype=torch.int32), w.page_table[:, :9],
                       w.k_pool, w.v_pool, w.q)
    else:
        w = W.custom(11, B=2, Hq=8, Hkv=2, D=16, P=8, k=3, lens=[37, 20], dtype="bf16")
    assert check_score_bound(O.page_scores, w)


def test_score_single_token_page_is_tight():
    # one token per page: the bound equals the group dot product exactly (then rounded to fp32)
    w = W.custom(12, B=1, Hq=4, Hkv=1, D=16, P=1, k=2, lens=[6], dtype="bf16")
    summ = O.page_summaries(w.k_pool, w.page_table, w.seq_lens, 1)
    sc = O.page_scores(w.q, summ, w.page_table, w.seq_lens, 1)
    Q = w.q.double().numpy()[0]
    for n in range(6):
        k = w.k_pool[int(w.page_table[0, n]), 0, 0].double().numpy()
        exact = math.fsum((Q * k[None, :]).ravel())
        assert sc[0, 0, n] == np.float32(exact)


def test_score_one_hot_queries():
    # G = 1, q = c * e_d: score = c * hi_d for c > 0 and c * lo_d for c < 0
    w = W.custom(13, B=1, Hq=1, Hkv=1, D=8, P=4, k=1, lens=[16], dtype="f32")
    summ = O.page_summaries(w.k_pool, w.page_table, w.seq_lens, 4)
    for d in range(8):
        for c in (2.0, -3.0):
            q = torch.zeros(1, 1, 8)
            q[0, 0, d] = c
            sc = O.page_scores(q, summ, w.page_table, w.seq_lens, 4)
            for n in range(4):
                p = int(w.page_table[0, n])
                col = w.k_pool[p, 0, :, d].double()
                want = c * (col.max() if c > 0 else col.min())
                assert sc[0, 0, n] == np.float32(float(want))


@pytest.mark.parametrize("mistake", ["hi_only", "one_head", "wrong_bound_per_sign"])
def test_planted_score_mistakes_are_caught(mistake):
    w = W.custom(11, B=2, Hq=8, Hkv=2, D=16, P=8, k=3, lens=[37, 20], dtype="bf16")

    def broken(q, summ, table, lens, P):
        s = np.array(summ, copy=True)
        if mistake == "hi_only":
            s[:, :, 0] = s[:, :, 1]
        elif mistake == "wrong_bound_per_sign":  # lo for q >= 0 and hi for q < 0
            Q = q.double().numpy()
            G = Q.shape[1] // s.shape[1]
            out = np.full((Q.shape[0], s.shape[1], table.shape[1]), np.nan, np.float32)
            for b in range(Q.shape[0]):
                for n in range(-(-int(lens[b]) // P)):
                    p = int(table[b, n])
                    for j in range(s.shape[1]):
                        qg = Q[b, j * G:(j + 1) * G]
                        out[b, j, n] = math.fsum(np.minimum(qg * s[p, j, 0], qg * s[p, j, 1]).ravel())
            return out
        qq = q.clone()
        if mistake == "one_head":  # drops all but the first head of each group
            G = q.shape[1] // s.shape[1]
            for j in range(s.shape[1]):
                qq[:, j * G + 1:(j + 1) * G] = 0
        return O.page_scores(qq, s, table, lens, P)

    assert not check_score_bound(broken, w)


# ----------------------------------------------------------------------------------------------
# a3 top-k
# ----------------------------------------------------------------------------------------------

def brute_topk(scores, k):
    """Subset of size min(k, N) with the largest exact score sum; among equal sums the one whose
    sorted index tuple is lexicographically smallest."""
    N = len(scores)
    kk = min(k, N)
    best = None
    for sub in itertools.combinations(range(N), kk):  # generated in lexicographic order
        s = sum(Fraction(float(scores[i])) for i in sub)
        if best is None or s > best[0]:
            best = (s, sub)
    return list(best[1])


def check_topk(fn, cases):
    for scores, k in cases:
        sc = np.asarray(scores, dtype=np.float32)[None, None, :]
        sel, cnt = fn(sc, torch.tensor([len(scores)]), 1, k)
        got = [int(x) for x in sel[0, 0, :cnt[0, 0]]]
        if got != brute_topk(scores, k):
            return False
        if any(int(x) != -1 for x in sel[0, 0, cnt[0, 0]:]):
            return False
    return True


def _topk_cases():
    rng = np.random.Generator(np.random.PCG64(5))
    cases = []
    for _ in range(60):
        N = int(rng.integers(1, 10))
        vals = rng.choice([-1.5, 0.0, 0.25, 1.0, 2.0, 3.5], size=N)  # many exact ties
        cases.append((list(vals), int(rng.integers(1, 11))))
    for _ in range(20):
        N = int(rng.integers(1, 10))
        cases.append((list(rng.standard_normal(N).astype(np.float32)), int(rng.integers(1, N + 1))))
    cases.append(([-0.0, 0.0, -0.0], 1))  # signed zeros compare equal: lowest index wins
    return cases


def test_topk_matches_brute_force():
    assert check_topk(O.top_pages, _topk_cases())


def test_topk_duplicate_pages_tie_to_lower_index():
    w = W.custom(21, B=1, Hq=4, Hkv=1, D=16, P=4, k=1, lens=[32], dtype="bf16", permute=False)
    w.k_pool[5] = w.k_pool[2]  # identical keys -> identical summaries -> exact tie
    w.q[0] = w.k_pool[2, 0, 0]  # make those pages the best
    summ = O.page_summaries(w.k_pool, w.page_table, w.seq_lens, w.P)
    sc = O.page_scores(w.q, summ, w.page_table, w.seq_lens, w.P)
    assert sc[0, 0, 2] == sc[0, 0, 5] == sc[0, 0].max()
    sel, cnt = O.top_pages(sc, w.seq_lens, w.P, 1)
    assert sel[0, 0, 0] == 2


def test_topk_takes_all_when_few_pages():
    sel, cnt = O.top_pages(np.array([[[3.0, 1.0, 2.0]]], dtype=np.float32), torch.tensor([3]), 1, 5)
    assert cnt[0, 0] == 3 and list(sel[0, 0]) == [0, 1, 2, -1, -1]


@pytest.mark.parametrize("mistake", ["ties_high", "unsorted", "smallest"])
def test_planted_topk_mistakes_are_caught(mistake):
    def broken(sc, lens, P, k):
        sc = np.asarray(sc)
        N = sc.shape[2]
        sel = np.full((1, 1, k), -1, dtype=np.int32)
        s = sc[0, 0].astype(np.float64)
        if mistake == "ties_high":
            order = np.lexsort((-np.arange(N), -s))
        elif mistake == "smallest":
            order = np.lexsort((np.arange(N), s))
        else:
            order = np.lexsort((np.arange(N), -s))
        take = order[:min(k, N)]
        if mistake != "unsorted":
            take = np.sort(take)
        sel[0, 0, :take.size] = take
        return sel, np.array([[take.size]], dtype=np.int32)

    assert not check_topk(broken, _topk_cases())


# The k-boundary margin (selection_margin_ulps) decides which fp32 lists the parity tests compare
# by a band check instead of bit for bit, so it is pinned on its own: the distance between the
# k-th and (k+1)-th best score is counted as np.nextafter steps (an fp32 walk that knows nothing
# of the oracle's integer mapping), with +0 and -0 one value.

def _steps_between(lo, hi):
    """nextafter steps from fp32 lo up to fp32 hi (lo <= hi), -0 and +0 counted as one value."""
    lo, hi = np.float32(lo), np.float32(hi)
    n = 0
    x = lo
    while x != hi:  # -0 == +0 compares equal, so the two zeros are one value
        x = np.nextafter(x, np.float32(np.inf))
        n += 1
        assert n < 10_000
    return n


def brute_margin(scores, k):
    """Steps between the k-th and (k+1)-th largest of a list; None when it has <= k entries."""
    vals = sorted((np.float32(v) for v in scores), key=float, reverse=True)
    if len(vals) <= k:
        return None
    return _steps_between(vals[k], vals[k - 1])


def _margin_cases():
    f = np.float32

    def up(x, n):  # n nextafter steps up from fp32 x
        x = f(x)
        for _ in range(n):
            x = np.nextafter(x, f(np.inf))
        return x

    tiny = np.nextafter(f(0), f(1))  # smallest positive subnormal
    cases = [
        ([1.0, 2.0, 2.0, 0.5], 1),                           # exact tie at the boundary -> 0
        ([f(1.0), up(f(1.0), 1), f(0.0)], 1),               # adjacent floats -> 1
        ([f(3.0), up(f(3.0), 2), f(-1.0)], 1),              # two ulps -> 2
        ([f(-0.0), f(0.0), f(5.0)], 2),                     # -0 against +0 -> a tie
        ([tiny, -tiny, f(9.0)], 2),                         # across zero: -tiny, 0, tiny -> 2
        ([up(f(7.0), 1), up(f(7.0), 6), f(7.0), up(f(7.0), 7), f(1.0)], 2),  # 5 between k and k+1
        ([f(1.0), f(2.0)], 2),                              # N == k: no boundary
        ([f(1.0)], 3),                                      # N < k
    ]
    rng = np.random.Generator(np.random.PCG64(17))
    for _ in range(40):  # random lists a few ulps apart around random bases, either sign
        base = f(rng.standard_normal() * 10.0 ** int(rng.integers(-3, 4)))
        N = int(rng.integers(2, 12))
        vals = [up(base, int(s)) for s in rng.integers(0, 12, size=N)]
        cases.append((vals, int(rng.integers(1, N + 2))))
    return cases


def check_margin(fn):
    for vals, k in _margin_cases():
        sc = np.asarray(vals, dtype=np.float32)[None, None, :]
        got = int(fn(sc, torch.tensor([len(vals)]), 1, k)[0, 0])
        want = brute_margin(vals, k)
        if want is None:
            if got < (1 << 40):
                return False
        elif got != want:
            return False
    return True


def test_selection_margin_matches_nextafter_walk():
    assert check_margin(O.selection_margin_ulps)
    # the hand-built cases alone, by name
    m = lambda vals, k: int(O.selection_margin_ulps(  # noqa: E731
        np.asarray(vals, np.float32)[None, None], torch.tensor([len(vals)]), 1, k)[0, 0])
    assert m([1.0, 2.0, 2.0, 0.5], 1) == 0
    assert m([1.0, float(np.nextafter(np.float32(1), np.float32(2))), 0.0], 1) == 1
    assert m([-0.0, 0.0, 5.0], 2) == 0
    assert m([1.0, 2.0], 2) >= 1 << 40


@pytest.mark.parametrize("mistake", ["k_plus_1", "k_minus_1", "always_0", "raw_bits",
                                     "no_sentinel"])
def test_planted_margin_mistakes_are_caught(mistake):
    def broken(scores, seq_lens, P, k):
        sc = np.asarray(scores, dtype=np.float32)
        N = sc.shape[2]
        out = np.full((1, 1), 1 << 40, dtype=np.int64)
        if N <= k:
            if mistake == "no_sentinel":
                out[0, 0] = 0
            return out
        u = np.where(sc[0, 0] == 0, np.float32(0), sc[0, 0]).view(np.int32).astype(np.int64)
        if mistake != "raw_bits":  # raw_bits: two's-complement order, wrong below zero
            u = np.where(u < 0, -(u & 0x7FFFFFFF), u)
        o = np.sort(u)[::-1]
        if mistake == "k_plus_1":
            out[0, 0] = o[k] - o[k + 1] if k + 1 < N else o[k]
        elif mistake == "k_minus_1":
            out[0, 0] = o[k - 2] - o[k - 1] if k >= 2 else o[0]
        elif mistake == "always_0":
            out[0, 0] = 0
        else:
            out[0, 0] = o[k - 1] - o[k]
        return out

    assert not check_margin(broken)


# ----------------------------------------------------------------------------------------------
# a4 reuse / correction
# ----------------------------------------------------------------------------------------------

def test_similarity_closed_forms():
    rng = np.random.Generator(np.random.PCG64(3))
    q = torch.from_numpy(rng.standard_normal((2, 8, 16)).astype(np.float32))
    assert np.allclose(O.query_similarity(q, q, 2), 1.0, atol=1e-15)
    assert np.allclose(O.query_similarity(q, 4 * q, 2), 1.0, atol=1e-15)
    assert np.allclose(O.query_similarity(q, -q, 2), -1.0, atol=1e-15)
    # group mean: heads of KV head 0 get cosines 1, -1, 1, 0 -> mean 0.25
    qp = q.clone()
    qp[0, 1] = -q[0, 1]
    e = torch.zeros(16)
    e[0] = 1.0
    qa = q.clone()
    qa[0, 3] = e
    qp[0, 3] = torch.zeros(16)
    qp[0, 3, 1] = 1.0  # orthogonal to e
    C = O.query_similarity(qa, qp, 2)
    assert abs(C[0, 0] - 0.25) < 1e-15


def test_correction_special_cases():
    fresh = np.arange(2 * 3 * 4).reshape(2, 3, 4).astype(np.int32)
    prev = fresh + 100
    fc = np.full((2, 3), 4, np.int32)
    pc = np.full((2, 3), 3, np.int32)
    C = np.array([[0.5, 0.8, 0.95], [0.79999, 1.0, -1.0]])
    u, uc, corr = O.speculative_choice(fresh, fc, prev, pc, C, 0.8, first_step=True)
    assert corr.all() and (u == fresh).all()
    u, uc, corr = O.speculative_choice(fresh, fc, prev, pc, C, -np.inf, first_step=False)
    assert not corr.any() and (u == prev).all() and (uc == 3).all()
    u, uc, corr = O.speculative_choice(fresh, fc, prev, pc, C, np.inf, first_step=False)
    assert corr.all() and (u == fresh).all()
    u, uc, corr = O.speculative_choice(fresh, fc, prev, pc, C, 0.8, first_step=False)
    assert corr.tolist() == [[1, 0, 0], [1, 0, 1]]  # strict '<': C == 0.8 is not corrected


# ----------------------------------------------------------------------------------------------
# a5 / a6 attention
# ----------------------------------------------------------------------------------------------

def _dense_tokens(w):
    """[B][Hkv][Lmax][D] keys/values in logical order (fp64), plus lengths."""
    K = w.k_pool.double().numpy()
    V = w.v_pool.double().numpy()
    outK, outV = [], []
    for b in range(w.B):
        L = int(w.seq_lens[b])
        kb = [O.gather_tokens(K, w.page_table, L, b, j, range(-(-L // w.P)), w.P)
              for j in range(w.Hkv)]
        vb = [O.gather_tokens(V, w.page_table, L, b, j, range(-(-L // w.P)), w.P)
              for j in range(w.Hkv)]
        outK.append(np.stack(kb))
        outV.append(np.stack(vb))
    return outK, outV


def check_all_pages_is_sdpa(attn_fn, w, scale):
    """Invariant: selecting every page gives dense softmax attention, checked against torch's
    scaled_dot_product_attention on the CPU in float64."""
    npg = [-(-int(L) // w.P) for L in w.seq_lens]
    kk = max(npg)
    sel = np.full((w.B, w.Hkv, kk), -1, dtype=np.int32)
    cnt = np.zeros((w.B, w.Hkv), dtype=np.int32)
    for b, n in enumerate(npg):
        sel[b, :, :n] = np.arange(n)
        cnt[b, :] = n
    out, lse = attn_fn(w.q, w.k_pool, w.v_pool, w.page_table, w.seq_lens, sel, cnt, w.P, scale)
    Ks, Vs = _dense_tokens(w)
    for b in range(w.B):
        q = w.q[b].double()[None, :, None, :]  # [1][Hq][1][D]
        k = torch.from_numpy(Ks[b]).repeat_interleave(w.G, dim=0)[None]
        v = torch.from_numpy(Vs[b]).repeat_interleave(w.G, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0, :, 0]
        if not np.allclose(out[b], ref.numpy(), rtol=0, atol=1e-12):
            return False
        # lse pinned by its definition via torch.logsumexp
        z = scale * torch.einsum("hd,htd->ht", w.q[b].double(), k[0])
        if not np.allclose(lse[b], torch.logsumexp(z, dim=-1).numpy(), rtol=0, atol=1e-12):
            return False
    return True


@pytest.mark.parametrize("case", ["tiny", "ragged_bf16"])
def test_all_pages_equals_dense_attention(case):
    if case == "tiny":
        w = W.tiny_fp32()
    else:
        w = W.custom(31, B=3, Hq=8, Hkv=2, D=32, P=16, k=4, lens=[50, 16, 1], dtype="bf16")
    scale = float(np.float32(1.0 / math.sqrt(w.D)))
    assert check_all_pages_is_sdpa(O.sparse_decode_attention, w, scale)


@pytest.mark.parametrize("mistake", ["no_scale", "wrong_head_map", "value_transposed_pages"])
def test_planted_attention_mistakes_are_caught(mistake):
    w = W.custom(31, B=3, Hq=8, Hkv=2, D=32, P=16, k=4, lens=[50, 16, 1], dtype="bf16")
    scale = float(np.float32(1.0 / math.sqrt(w.D)))

    def broken(q, kp, vp, table, lens, sel, cnt, P, sc):
        if mistake == "no_scale":
            return O.sparse_decode_attention(q, kp, vp, table, lens, sel, cnt, P, 1.0)
        if mistake == "wrong_head_map":  # interleaved instead of contiguous groups
            Hq, Hkv = q.shape[1], kp.shape[1]
            G = Hq // Hkv
            perm = [(h % Hkv) * G + h // Hkv for h in range(Hq)]
            return O.sparse_decode_attention(q[:, perm], kp, vp, table, lens, sel, cnt, P, sc)
        # values read with K's page order reversed within a sequence
        vp2 = vp.clone()
        vp2 = vp2.flip(0)
        return O.sparse_decode_attention(q, kp, vp2, table, lens, sel, cnt, P, sc)

    assert not check_all_pages_is_sdpa(broken, w, scale)


def check_dense_is_sdpa(dense_fn, w, scale):
    """dense_decode_attention over a sequence's tokens against torch's CPU
    scaled_dot_product_attention (float64), one sequence at a time (lengths differ)."""
    Ks, Vs = _dense_tokens(w)
    for b in range(w.B):
        out, lse = dense_fn(w.q[b:b + 1], Ks[b][None], Vs[b][None], scale)
        q = w.q[b].double()[None, :, None, :]
        k = torch.from_numpy(Ks[b]).repeat_interleave(w.G, dim=0)[None]
        v = torch.from_numpy(Vs[b]).repeat_interleave(w.G, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0, :, 0]
        if not np.allclose(out[0], ref.numpy(), rtol=0, atol=1e-12):
            return False
        z = scale * torch.einsum("hd,htd->ht", w.q[b].double(), k[0])
        if not np.allclose(lse[0], torch.logsumexp(z, dim=-1).numpy(), rtol=0, atol=1e-12):
            return False
    return True


def test_dense_attention_equals_sdpa():
    w = W.custom(32, B=3, Hq=8, Hkv=2, D=32, P=16, k=4, lens=[50, 16, 1], dtype="bf16")
    scale = float(np.float32(1.0 / math.sqrt(w.D)))
    assert check_dense_is_sdpa(O.dense_decode_attention, w, scale)


@pytest.mark.parametrize("mistake", ["no_scale", "wrong_head_map"])
def test_planted_dense_attention_mistakes_are_caught(mistake):
    w = W.custom(32, B=3, Hq=8, Hkv=2, D=32, P=16, k=4, lens=[50, 16, 1], dtype="bf16")
    scale = float(np.float32(1.0 / math.sqrt(w.D)))

    def broken(q, keys, values, sc):
        if mistake == "no_scale":
            return O.dense_decode_attention(q, keys, values, 1.0)
        Hq, Hkv = q.shape[1], keys.shape[1]
        G = Hq // Hkv
        perm = [(h % Hkv) * G + h // Hkv for h in range(Hq)]  # interleaved groups
        return O.dense_decode_attention(q[:, perm], keys, values, sc)

    assert not check_dense_is_sdpa(broken, w, scale)


def check_decode_step_all_pages(step_fn, w, scale):
    """The one-step composition (scores, top-k, attention) with k at least every sequence's page
    count attends over every token: it must equal dense attention on the CPU (torch SDPA)."""
    summ = O.page_summaries(w.k_pool, w.page_table, w.seq_lens, w.P)
    kk = max(-(-int(L) // w.P) for L in w.seq_lens)
    sel, cnt, out, lse = step_fn(w.q, summ, w.k_pool, w.v_pool, w.page_table, w.seq_lens, w.P,
                                 kk, scale)
    Ks, Vs = _dense_tokens(w)
    for b in range(w.B):
        n = -(-int(w.seq_lens[b]) // w.P)
        if not (np.asarray(cnt)[b] == n).all():
            return False
        q = w.q[b].double()[None, :, None, :]
        k = torch.from_numpy(Ks[b]).repeat_interleave(w.G, dim=0)[None]
        v = torch.from_numpy(Vs[b]).repeat_interleave(w.G, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0, :, 0]
        if not np.allclose(out[b], ref.numpy(), rtol=0, atol=1e-12):
            return False
    return True


def test_decode_step_with_every_page_is_dense_attention():
    w = W.custom(33, B=3, Hq=8, Hkv=2, D=32, P=16, k=4, lens=[70, 33, 5], dtype="bf16")
    scale = float(np.float32(1.0 / math.sqrt(w.D)))
    assert check_decode_step_all_pages(O.decode_step, w, scale)

    def broken(q, summ, kp, vp, table, lens, P, k, sc):  # attends over one page too few
        return O.decode_step(q, summ, kp, vp, table, lens, P, k - 1, sc)

    assert not check_decode_step_all_pages(broken, w, scale)


def test_attention_weights_sum_to_one_and_closed_forms():
    w = W.custom(41, B=2, Hq=4, Hkv=2, D=16, P=8, k=3, lens=[29, 9], dtype="bf16")
    sel = np.array([[[0, 2, 3], [1, 3, -1]], [[1, -1, -1], [0, 1, -1]]], dtype=np.int32)
    cnt = np.array([[3, 2], [1, 2]], dtype=np.int32)
    scale = float(np.float32(0.25))
    ones = torch.ones_like(w.v_pool)
    out, _ = O.sparse_decode_attention(w.q, w.k_pool, ones, w.page_table, w.seq_lens, sel, cnt,
                                       w.P, scale)
    assert np.allclose(out, 1.0, atol=1e-14)
    # q = 0: uniform weights -> mean of the selected values
    zq = torch.zeros_like(w.q)
    out, lse = O.sparse_decode_attention(zq, w.k_pool, w.v_pool, w.page_table, w.seq_lens, sel,
                                         cnt, w.P, scale)
    V = w.v_pool.double().numpy()
    for b in range(2):
        for j in range(2):
            rows = O.gather_tokens(V, w.page_table, int(w.seq_lens[b]), b, j,
                                   sel[b, j, :cnt[b, j]], w.P)
            for h in (2 * j, 2 * j + 1):
                assert np.allclose(out[b, h], rows.mean(axis=0), atol=1e-14)
                assert abs(lse[b, h] - math.log(rows.shape[0])) < 1e-12
    # one selected token (sequence 1, page 1 holds a single valid token): o = v exactly
    one = np.array([[[0, -1, -1], [0, -1, -1]], [[1, -1, -1], [1, -1, -1]]], dtype=np.int32)
    c1 = np.array([[1, 1], [1, 1]], dtype=np.int32)
    out, _ = O.sparse_decode_attention(w.q, w.k_pool, w.v_pool, w.page_table, w.seq_lens, one, c1,
                                       w.P, scale)
    p = int(w.page_table[1, 1])
    for h in range(4):
        np.testing.assert_array_equal(out[1, h], w.v_pool[p, h // 2, 0].double().numpy())


def test_attention_page_table_permutation_invariance():
    a = W.custom(51, B=2, Hq=4, Hkv=1, D=16, P=8, k=3, lens=[40, 17], dtype="bf16", permute=False)
    rng = np.random.Generator(np.random.PCG64(9))
    perm = rng.permutation(a.num_phys_pages)
    inv = np.argsort(perm)
    k2 = a.k_pool[torch.from_numpy(perm)]
    v2 = a.v_pool[torch.from_numpy(perm)]
    t2 = torch.from_numpy(inv[a.page_table.numpy()].astype(np.int32))
    sel = np.array([[[0, 2, 4]], [[0, 2, -1]]], dtype=np.int32)
    cnt = np.array([[3], [2]], dtype=np.int32)
    o1, l1 = O.sparse_decode_attention(a.q, a.k_pool, a.v_pool, a.page_table, a.seq_lens, sel, cnt,
                                       8, 0.25)
    o2, l2 = O.sparse_decode_attention(a.q, k2, v2, t2, a.seq_lens, sel, cnt, 8, 0.25)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_tiny_planted_tokens_are_selected():
    w = W.tiny_fp32()
    summ = O.page_summaries(w.k_pool, w.page_table, w.seq_lens, w.P)
    sc = O.page_scores(w.q, summ, w.page_table, w.seq_lens, w.P)
    sel, cnt = O.top_pages(sc, w.seq_lens, w.P, w.k)
    for j in range(w.Hkv):
        for p in w.extra["planted_pages"]:
            assert p in set(sel[0, j].tolist())


# ----------------------------------------------------------------------------------------------
# a7 rotary re-positioning
# ----------------------------------------------------------------------------------------------

def _complex_rotate(x, positions, theta):
    """Rotate-half RoPE as complex multiplication (x_i + i x_{i+D/2}) * exp(i pos theta^(-2i/D)),
    NumPy complex128 -- an independent formulation of the rotation."""
    D = x.shape[-1]
    half = D // 2
    inv = theta ** (-(2.0 * np.arange(half)) / D)
    z = x[..., :half] + 1j * x[..., half:]
    r = z * np.exp(1j * positions[..., None] * inv)
    return np.concatenate([r.real, r.imag], axis=-1)


def test_rope_table_closed_forms():
    cos, sin = O.rope_table(500000.0, 128, 0, 3)
    assert (cos[0] == 1).all() and (sin[0] == 0).all()
    # channel pair 0 has inverse frequency 1: angle = position
    assert cos[2, 0] == np.float32(math.cos(2.0)) and sin[1, 0] == np.float32(math.sin(1.0))
    # pair D/4 has inverse frequency theta^(-1/2)
    c, s = O.rope_table(10000.0, 8, 7, 1)
    assert abs(float(c[0, 2]) - math.cos(7 / 100.0)) < 1e-7
    assert abs(float(s[0, 2]) - math.sin(7 / 100.0)) < 1e-7


def check_rope_matches_complex(rotate_fn, dtype):
    rng = np.random.Generator(np.random.PCG64(17))
    D, P, theta = 16, 4, 500000.0
    x = rng.standard_normal((3, 2, P, D)).astype(np.float32)
    pool = torch.from_numpy(x) if dtype == "f32" else torch.from_numpy(x).to(torch.bfloat16)
    xs = pool.double().numpy()
    cos, sin = O.rope_table(theta, D, 0, 64)
    page_row = np.array([5, -1, 40], dtype=np.int32)
    out = rotate_fn(pool, cos, sin, page_row, 1, dtype)
    for p in range(3):
        if page_row[p] < 0:
            if not np.array_equal(out[p], xs[p]):
                return False
            continue
        pos = (page_row[p] + np.arange(P)).astype(np.float64)
        want = _complex_rotate(xs[p], np.broadcast_to(pos, (2, P)), theta)
        tol = (2.0 ** -7 if dtype == "bf16" else 1e-6) * np.maximum(np.abs(want), 1e-3) + 1e-6
        if not (np.abs(out[p] - want) <= tol).all():
            return False
    return True


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_rotation_matches_complex_multiplication(dtype):
    assert check_rope_matches_complex(O.rope_rotate, dtype)


@pytest.mark.parametrize("mistake", ["sign", "pairing", "no_position_step"])
def test_planted_rope_mistakes_are_caught(mistake):
    def broken(pool, cos, sin, page_row, row_step, dtype):
        if mistake == "sign":
            return O.rope_rotate(pool, cos, -np.asarray(sin), page_row, row_step, dtype)
        if mistake == "no_position_step":
            return O.rope_rotate(pool, cos, sin, page_row, 0, dtype)
        # adjacent pairs (2i, 2i+1) instead of rotate-half pairs (i, i + D/2)
        X = pool.double().numpy()
        D = X.shape[-1]
        perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
        inv = np.argsort(perm)
        Xp = torch.from_numpy(X[..., perm].astype(np.float32))
        if dtype == "bf16":
            Xp = Xp.to(torch.bfloat16)
        return O.rope_rotate(Xp, cos, sin, page_row, row_step, dtype)[..., inv]

    assert not check_rope_matches_complex(broken, "f32")


def test_rope_zero_shift_is_identity_and_composition():
    w = W.custom(61, B=1, Hq=4, Hkv=2, D=32, P=8, k=2, lens=[32], dtype="bf16", permute=False)
    cos, sin = O.rope_table(500000.0, 32, 0, 4097)
    zero = np.zeros(4, dtype=np.int32)
    np.testing.assert_array_equal(O.rope_rotate(w.k_pool, cos, sin, zero, 0, "bf16"),
                                  w.k_pool.float().numpy())
    # shift by 1000 then by 3000 ~ shift by 4000 (within bf16 rounding of the intermediate)
    r1 = O.rope_rotate(w.k_pool, cos, sin, np.full(4, 1000, np.int32), 0, "bf16")
    r2 = O.rope_rotate(torch.from_numpy(r1).to(torch.bfloat16), cos, sin,
                       np.full(4, 3000, np.int32), 0, "bf16")
    r3 = O.rope_rotate(w.k_pool, cos, sin, np.full(4, 4000, np.int32), 0, "bf16")
    assert np.abs(r2 - r3).max() <= 2.0 ** -6 * np.abs(r3).max()
    # pair norms are preserved within bf16 rounding
    n0 = np.hypot(w.k_pool.float().numpy()[..., :16], w.k_pool.float().numpy()[..., 16:])
    n1 = np.hypot(r3[..., :16], r3[..., 16:])
    assert np.abs(n1 - n0).max() <= 2.0 ** -6 * n0.max()


def test_rope_relative_position_property():
    # <R(m) q, R(n) k> depends on m - n only (fp32 rotation, fp64 dot)
    rng = np.random.Generator(np.random.PCG64(71))
    D = 64
    qk = torch.from_numpy(rng.standard_normal((2, 1, 1, D)).astype(np.float32))
    cos, sin = O.rope_table(500000.0, D, 0, 5000)
    def rot(x, pos):
        return O.rope_rotate(x, cos, sin, np.array([pos], np.int32), 0, "f32")[0, 0, 0].astype(np.float64)
    a = rot(qk[0:1], 1234) @ rot(qk[1:2], 1000)
    b = rot(qk[0:1], 4234) @ rot(qk[1:2], 4000)
    assert abs(a - b) < 1e-4


def test_block_shift_equals_direct_encoding():
    # a block encoded at positions 0..T-1 then shifted by delta == encoding at delta..delta+T-1,
    # within two bf16 roundings
    w = W.custom(81, B=1, Hq=4, Hkv=2, D=32, P=8, k=2, lens=[64], dtype="bf16", permute=False)
    cos, sin = O.rope_table(500000.0, 32, 0, 8192)
    enc_rows = (np.arange(8) * 8).astype(np.int32)
    enc = O.rope_rotate(w.k_pool, cos, sin, enc_rows, 1, "bf16")
    shifted = O.rope_rotate(torch.from_numpy(enc).to(torch.bfloat16), cos, sin,
                            np.full(8, 4096, np.int32), 0, "bf16")
    direct = O.rope_rotate(w.k_pool, cos, sin, enc_rows + 4096, 1, "bf16")
    assert np.abs(shifted - direct).max() <= 2.0 ** -6 * np.abs(direct).max()
    assert not np.array_equal(enc, direct)  # the shift does something


# ----------------------------------------------------------------------------------------------
# byte accounting
# ----------------------------------------------------------------------------------------------

def test_kv_bytes_formula_reproduces_kvzap_figure():
    from query_aware_sparse_page_amd.accounting import kv_cache_bytes
    g = json.load(open(os.path.join(GOLD, "kvzap_llama65b_kv_bytes.json")))
    b = kv_cache_bytes(g["num_layers"], g["kv_heads_times_head_dim"], g["tokens"],
                       g["bytes_per_element"])
    assert round(b / 1e9) == g["stated_gb"] + 1 or round(b / 1e9) == g["stated_gb"]
    assert abs(b / 1e9 - g["stated_gb"]) < 1.0
