"""Shared helpers of the GPU parity tests (no GPU work at import time)."""
import math
import sys

import numpy as np
import torch

import oracle as O

BF16_OUT_TOL = 2e-2   # absolute, bf16 attention outputs
F32_OUT_TOL = 1e-5    # absolute, fp32 attention outputs
# bf16 lse: the kernel rounds each probability exp(z - m) to bf16 (round to nearest even, unit
# roundoff 2^-8) before the P x V product and sums the rounded values, so the sum is off by a
# relative 2^-8 at most and ln of it by -ln(1 - 2^-8) < 3.92e-3; the logits (exact bf16 products,
# fp32 sums) and the fp32 exp / log add well under 1e-4.
BF16_LSE_TOL = 4e-3
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


def assert_selection_equal(sel, cnt, ref_sel, ref_cnt, margins=None):
    s = sel.cpu().numpy()
    c = cnt.cpu().numpy()
    np.testing.assert_array_equal(c, ref_cnt)
    for b in range(s.shape[0]):
        for j in range(s.shape[1]):
            if margins is not None and margins[b, j] <= 1:
                # parity-fragile: a 1-ulp score difference may legitimately swap the boundary
                # page; require a valid sorted list of distinct in-range pages instead
                row = s[b, j, :c[b, j]]
                assert (np.diff(row) > 0).all()
                continue
            np.testing.assert_array_equal(s[b, j], ref_sel[b, j], err_msg=f"list ({b},{j})")


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
    margins = O.selection_margin_ulps(sc, w.seq_lens, w.P, w.k)
    out, lse = O.sparse_decode_attention(w.q, w.k_pool, w.v_pool, w.page_table, w.seq_lens, sel,
                                         cnt, w.P, scale)
    return dict(summ=summ, scores=sc, sel=sel, cnt=cnt, margins=margins, out=out, lse=lse)
