"""Shared helpers of the GPU parity tests (no GPU work at import time)."""
import math
import sys

import numpy as np
import torch

import oracle as O

BF16_OUT_TOL = 2e-2   # absolute, bf16 attention outputs
F32_OUT_TOL = 1e-5    # absolute, fp32 attention outputs
# bf16 lse (the method's tolerance): lse = m + ln(sum of the fp32 probabilities exp(z - m)),
# taken from the unrounded probabilities (the bf16-rounded ones only feed the P x V product). Its
# error is the fp32 rounding of the logits (exact bf16 products summed in fp32) and of the sum of
# at most a few thousand terms plus the fp32 exp / log: a few 1e-5, under 1e-3.
BF16_LSE_TOL = 1e-3
F32_LSE_TOL = 1e-5


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def kv_of(K, w, dev="cuda"):
    return K.PagedKV(w.k_pool.to(dev), K.device_v_layout(w.v_pool.to(dev)), w.page_table.to(dev),
                     w.seq_lens.to(dev), w.Hq)


def scale_of(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def referenced_pages(w):
    out = []
    for b in range(w.B):
        out.extend(int(x) for x in w.page_table[b, :w.n_pages(b)])
    return sorted(set(out))


def assert_summaries_equal(gpu_summ, ref_summ, w):
    """gpu_summ is sequence-major [B][Hkv][max_pages][2][D]; ref_summ is the oracle's per physical
    page [Npp][Hkv][2][D]: logical page n of sequence b must equal physical page page_table[b][n]."""
    g = gpu_summ.float().cpu().numpy()
    n_bad = 0
    first = None
    for b in range(w.B):
        N = w.n_pages(b)
        pages = w.page_table[b, :N].numpy()
        r = ref_summ[pages].transpose(1, 0, 2, 3)  # [Hkv][N][2][D]
        assert np.isfinite(r).all()
        bad = np.argwhere(g[b, :, :N] != r)  # by value: -0 == +0
        n_bad += len(bad)
        if len(bad) and first is None:
            first = (b, bad[:3].tolist())
    assert n_bad == 0, f"{n_bad} summary values differ, first {first}"


def orderable32(x):
    x = np.where(np.asarray(x, np.float32) == 0, np.float32(0), x).astype(np.float32)
    u = x.view(np.int32).astype(np.int64)
    return np.where(u < 0, -(u & 0x7FFFFFFF), u)


def assert_scores_close(gpu_scores, ref_scores, w, exact):
    g = gpu_scores.cpu().numpy()
    worst = 0
    n_exact = 0
    n = 0
    for b in range(w.B):
        N = w.n_pages(b)
        d = np.abs(orderable32(g[b, :, :N]) - orderable32(ref_scores[b, :, :N]))
        worst = max(worst, int(d.max()) if d.size else 0)
        n_exact += int((d == 0).sum())
        n += d.size
    if exact:
        assert worst == 0, f"scores differ by up to {worst} ulp ({n - n_exact}/{n} inexact)"
    else:
        assert worst <= 1, f"scores differ by up to {worst} ulp"
    return n_exact, n


def fp32_boundary(dtype, scores, seq_lens, P, k):
    """What the selection check needs for an fp32 cache, whose scores may legitimately differ
    from the oracle's by one fp32 ulp (the library sums exact fp64 products in a fixed order, the
    oracle rounds the exact sum once); None for bf16 / fp8, whose scores are exact in any order
    and whose selections are compared bit for bit unconditionally."""
    if dtype != "f32":
        return None
    return dict(scores=np.asarray(scores), lens=np.asarray(seq_lens), P=P, k=k,
                margins=O.selection_margin_ulps(scores, seq_lens, P, k))


def _band_check(row, b, j, fb):
    """A list whose k-boundary margin is <= 2 ulps: with every score within 1 ulp of the
    oracle's, the k-th and (k+1)-th may each move by one ulp and trade places. Let T be the
    oracle's k-th best (as an orderable integer): every chosen page must score >= T - 2 and
    every page left out <= T + 2, so a page may differ from the oracle's list only inside that
    band."""
    L = int(fb["lens"][b])
    N = -(-L // fb["P"])
    o = orderable32(fb["scores"][b, j, :N])
    T = np.sort(o)[::-1][fb["k"] - 1]
    assert (np.diff(row) > 0).all() and row.min() >= 0 and row.max() < N, f"list ({b},{j})"
    chosen = np.zeros(N, bool)
    chosen[row] = True
    assert (o[chosen] >= T - 2).all(), f"list ({b},{j}): a page below the boundary band chosen"
    assert (o[~chosen] <= T + 2).all(), f"list ({b},{j}): a page above the boundary band left out"


def assert_selection_equal(sel, cnt, ref_sel, ref_cnt, fp32=None, gpu_scores=None):
    """Selected pages bit for bit against the oracle's. fp32: fp32_boundary(...) of an fp32
    cache, whose lists with a k-boundary margin <= 2 ulps get the band check instead (logged).
    gpu_scores: the library's own scores, when it returned them; then every list must also be
    exactly the oracle's top-k of those scores (ties to the lower index)."""
    s = sel.cpu().numpy()
    c = cnt.cpu().numpy()
    np.testing.assert_array_equal(c, ref_cnt)
    banded = 0
    for b in range(s.shape[0]):
        for j in range(s.shape[1]):
            if fp32 is not None and fp32["margins"][b, j] <= 2:
                banded += 1
                _band_check(s[b, j, :c[b, j]], b, j, fp32)
                np.testing.assert_array_equal(s[b, j, c[b, j]:], -1)
                continue
            np.testing.assert_array_equal(s[b, j], ref_sel[b, j], err_msg=f"list ({b},{j})")
    if gpu_scores is not None:
        g = gpu_scores.cpu().numpy()
        lens = fp32["lens"] if fp32 is not None else None
        if lens is not None:
            own, own_cnt = O.top_pages(g, lens, fp32["P"], s.shape[2])
            np.testing.assert_array_equal(s, own)
            np.testing.assert_array_equal(c, own_cnt)
    if banded:
        say(f"selection: {banded} of {c.size} fp32 lists within 2 ulps of the boundary, band-checked")
    return banded


def assert_attention_close(out, lse, ref_out, ref_lse, dtype):
    tol = BF16_OUT_TOL if dtype == "bf16" else F32_OUT_TOL
    ltol = BF16_LSE_TOL if dtype == "bf16" else F32_LSE_TOL
    o = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(o - ref_out).max()
    assert err <= tol, f"attention max abs error {err:.3g} > {tol}"
    if lse is not None:
        l = lse.cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref_lse)
        assert (np.isfinite(l) == fin).all()
        if fin.any():
            lerr = np.abs(l[fin] - ref_lse[fin]).max()
            assert lerr <= ltol, f"lse max abs error {lerr:.3g} > {ltol}"
    return err


def oracle_path(w, scale):
    summ = O.page_summaries(w.k_pool, w.page_table, w.seq_lens, w.P)
    sc = O.page_scores(w.q, summ, w.page_table, w.seq_lens, w.P)
    sel, cnt = O.top_pages(sc, w.seq_lens, w.P, w.k)
    out, lse = O.sparse_decode_attention(w.q, w.k_pool, w.v_pool, w.page_table, w.seq_lens, sel,
                                         cnt, w.P, scale)
    return dict(summ=summ, scores=sc, sel=sel, cnt=cnt,
                fp32=fp32_boundary(w.dtype, sc, w.seq_lens, w.P, w.k), out=out, lse=lse)
