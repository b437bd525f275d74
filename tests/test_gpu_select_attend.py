"""kvsel_select_attend (selection fused into the attention launch) against the two separate calls
(bit for bit) and against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import (assert_attention_close, assert_selection_equal, kv_of, oracle_path,
                        referenced_pages, say, scale_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_page_amd import kvsel as K
    K.lib()  # raises if libkvsel.so is missing: no fallback
    return K


def separate_calls(K, kv, summ, q, k, refresh_tail=False):
    sel, cnt = K.score_topk(kv, summ, q, k, refresh_tail=refresh_tail)
    out, lse = K.sparse_decode_attn(kv, q, sel, cnt, k, pages_per_split=K.step_pages_per_split(kv, k))
    return sel, cnt, out, lse


def assert_same(a, b):
    for x, y, name in zip(a, b, ("sel_idx", "sel_cnt", "out", "lse")):
        assert torch.equal(x, y), f"{name} differs between the fused call and the separate calls"


@pytest.mark.parametrize("name", ["tiny_fp32", "llama8b_32k", "ragged_batch", "qwen4b_128k"])
def test_full_workloads(K, name):
    w = W.make(name)
    say(f"select_attend {name}")
    kv = kv_of(K, w)
    q = w.q.cuda()
    summ = K.build_summaries(kv)
    fused = K.select_attend(kv, summ, q, w.k)
    sep = separate_calls(K, kv, summ, q, w.k)
    torch.cuda.synchronize()
    assert_same(fused, sep)
    ref = oracle_path(w, scale_of(w.D))
    assert_selection_equal(fused[0], fused[1], ref["sel"], ref["cnt"], ref["fp32"])
    err = assert_attention_close(fused[2], fused[3], ref["out"], ref["lse"], w.dtype)
    say(f"{name}: max abs err {err:.3g}")


EDGE = [
    dict(seed=301, B=3, Hq=8, Hkv=2, D=64, P=16, k=3, lens=[0, 1, 47], dtype="bf16"),
    dict(seed=302, B=2, Hq=8, Hkv=8, D=128, P=32, k=4, lens=[200, 31], dtype="bf16"),     # G=1
    dict(seed=303, B=2, Hq=16, Hkv=2, D=128, P=16, k=5, lens=[33, 170], dtype="bf16"),    # G=8
    dict(seed=304, B=2, Hq=4, Hkv=2, D=64, P=32, k=8, lens=[96, 65], dtype="bf16"),       # k >= N
    dict(seed=305, B=2, Hq=8, Hkv=4, D=128, P=32, k=3, lens=[300, 64], dtype="f32"),      # G=2
    dict(seed=306, B=3, Hq=8, Hkv=2, D=64, P=16, k=4, lens=[16, 100, 257], dtype="f32"),
    dict(seed=307, B=1, Hq=32, Hkv=8, D=128, P=32, k=64, lens=[32768 - 5], dtype="bf16"),
    dict(seed=308, B=2, Hq=8, Hkv=2, D=128, P=16, k=40, lens=[16 * 3000 + 3, 16 * 900], dtype="bf16"),
    dict(seed=309, B=2, Hq=8, Hkv=2, D=64, P=32, k=100, lens=[32 * 7000 + 1, 32 * 150], dtype="f32"),
]


@pytest.mark.parametrize("case", EDGE)
def test_edge_cases(K, case):
    w = W.custom(case["seed"], case["B"], case["Hq"], case["Hkv"], case["D"], case["P"], case["k"],
                 case["lens"], case["dtype"], spare_pages=3)
    used = set(referenced_pages(w))
    for p in range(w.num_phys_pages):  # poison everything no sequence may read
        if p not in used:
            w.k_pool[p] = float("nan")
            w.v_pool[p] = float("nan")
    for b in range(w.B):
        L = int(w.seq_lens[b])
        if L % w.P:
            p = int(w.page_table[b, L // w.P])
            w.k_pool[p, :, L % w.P:] = float("nan")
            w.v_pool[p, :, L % w.P:] = float("nan")
    say(f"select_attend edge case {case['seed']}: maxp {w.max_pages}")
    kv = kv_of(K, w)
    q = w.q.cuda()
    summ = K.build_summaries(kv)
    fused = K.select_attend(kv, summ, q, w.k)
    sep = separate_calls(K, kv, summ, q, w.k)
    torch.cuda.synchronize()
    assert_same(fused, sep)
    ref = oracle_path(w, scale_of(w.D))
    assert_selection_equal(fused[0], fused[1], ref["sel"], ref["cnt"], ref["fp32"])
    assert_attention_close(fused[2], fused[3], ref["out"], ref["lse"], w.dtype)


def test_tail_refresh_and_workspace_reuse(K):
    w = W.custom(321, B=3, Hq=32, Hkv=8, D=128, P=32, k=6, lens=[700, 64, 33], dtype="bf16")
    say("select_attend with tail refresh, one workspace")
    kv = kv_of(K, w)
    q = w.q.cuda()
    summ_a = K.build_summaries(kv)
    summ_b = summ_a.clone()
    ws = K.new_workspace(kv, w.k, K.KVSEL_OP_SELECT_ATTEND)
    gen = torch.Generator().manual_seed(7)
    for it in range(3):
        for b in range(w.B):  # a decode step writes into each tail page
            p = int(w.page_table[b, w.n_pages(b) - 1])
            kv.k_pool[p] = (torch.randn(kv.k_pool[p].shape, generator=gen)).to(kv.k_pool.dtype).cuda()
        fused = K.select_attend(kv, summ_a, q, w.k, refresh_tail=True, workspace=ws)
        sep = separate_calls(K, kv, summ_b, q, w.k, refresh_tail=True)
        torch.cuda.synchronize()
        assert_same(fused, sep)
        for b in range(w.B):  # entries past a sequence's pages are never written
            assert torch.equal(summ_a[b, :, :w.n_pages(b)], summ_b[b, :, :w.n_pages(b)])
    ref_summ = O.page_summaries(kv.k_pool.cpu(), w.page_table, w.seq_lens, w.P)
    sc = O.page_scores(w.q, ref_summ, w.page_table, w.seq_lens, w.P)
    ref_sel, ref_cnt = O.top_pages(sc, w.seq_lens, w.P, w.k)
    assert_selection_equal(fused[0], fused[1], ref_sel, ref_cnt)


def _refresh_case(K, w, prep, k, label, stale=True):
    """select_attend with the tail refresh against the separate calls and the oracle, after
    `prep(k_pool)` rewrote keys on the host: with `stale` the summaries were built before (prep
    may then change only the tail pages, whose summaries the refresh rebuilds), else after."""
    kv = kv_of(K, w)
    pool = w.k_pool.clone()
    if stale:
        summ_a = K.build_summaries(kv)
    prep(pool)
    kv.k_pool.copy_(pool.cuda())
    if not stale:
        summ_a = K.build_summaries(kv)
    summ_b = summ_a.clone()
    q = w.q.cuda()
    say(f"select_attend tail merge: {label}")
    fused = K.select_attend(kv, summ_a, q, k, refresh_tail=True)
    sep = separate_calls(K, kv, summ_b, q, k, refresh_tail=True)
    torch.cuda.synchronize()
    assert_same(fused, sep)
    for b in range(w.B):
        assert torch.equal(summ_a[b, :, :w.n_pages(b)], summ_b[b, :, :w.n_pages(b)])
    ref_summ = O.page_summaries(pool, w.page_table, w.seq_lens, w.P)
    sc = O.page_scores(w.q, ref_summ, w.page_table, w.seq_lens, w.P)
    ref_sel, ref_cnt = O.top_pages(sc, w.seq_lens, w.P, k)
    assert_selection_equal(fused[0], fused[1], ref_sel, ref_cnt)
    return fused, ref_sel


def test_tail_merge_cases(K):
    """The fused form selects over all pages but the tail and merges the refreshed tail page in:
    a tail that ties the weakest chosen page stays out (the lower index wins), a tail above it
    displaces it, and lists of at most k pages (or a single page) take the tail as one more."""
    # every page's keys equal: all scores tie, so the first k pages are chosen, never the tail
    w = W.custom(341, B=2, Hq=32, Hkv=8, D=128, P=32, k=8, lens=[32 * 40 - 7, 32 * 25],
                 dtype="bf16")
    tile = w.k_pool[0].clone()

    def all_equal(pool):
        pool[:] = tile

    fused, ref_sel = _refresh_case(K, w, all_equal, w.k, "all scores tie", stale=False)
    assert (ref_sel[:, :, : w.k] == np.arange(w.k)).all()
    # the tail page's keys far above every other page's for the group's queries: it must enter

    def planted(pool):
        for b in range(w.B):
            p = int(w.page_table[b, w.n_pages(b) - 1])
            qg = w.q[b].float().reshape(w.Hkv, -1, w.D).sum(dim=1)  # [Hkv][D]
            pool[p] = (12.0 * torch.sign(qg)[:, None, :]).expand(w.Hkv, w.P, w.D).to(pool.dtype)

    fused, ref_sel = _refresh_case(K, w, planted, w.k, "planted tail")
    for b in range(w.B):
        assert (ref_sel[b, :, w.k - 1] == w.n_pages(b) - 1).all()
    # lists of at most k pages, a one-page sequence and an empty one
    w2 = W.custom(342, B=4, Hq=8, Hkv=2, D=64, P=16, k=12, lens=[16 * 12, 16 * 7 + 3, 5, 0],
                  dtype="bf16")
    _refresh_case(K, w2, lambda pool: None, w2.k, "N <= k, one page, empty")
    # fp32 with many splits
    w3 = W.custom(343, B=2, Hq=16, Hkv=4, D=128, P=32, k=40, lens=[32 * 300 - 1, 32 * 130 + 9],
                  dtype="f32")
    gen = torch.Generator().manual_seed(343)

    def fresh_tails(pool):
        for b in range(w3.B):
            p = int(w3.page_table[b, w3.n_pages(b) - 1])
            pool[p] = 3.0 * torch.randn(pool[p].shape, generator=gen)

    _refresh_case(K, w3, fresh_tails, w3.k, "fp32, fresh tails")


def test_fallback_paths_match(K):
    # k above 1024 needs splits larger than the fused launch's, and a 1500-page table is wider
    # than the fused form is taken for: the separate launches run inside the same call
    w = W.custom(331, B=1, Hq=8, Hkv=2, D=64, P=16, k=1100, lens=[16 * 1500], dtype="bf16")
    say("select_attend fallback: k = 1100")
    kv = kv_of(K, w)
    q = w.q.cuda()
    summ = K.build_summaries(kv)
    fused = K.select_attend(kv, summ, q, w.k)
    sep = separate_calls(K, kv, summ, q, w.k)
    torch.cuda.synchronize()
    assert_same(fused, sep)
    say("select_attend fallback: 1500-page table, k = 64")
    fused = K.select_attend(kv, summ, q, 64)
    sep = separate_calls(K, kv, summ, q, 64)
    torch.cuda.synchronize()
    assert_same(fused, sep)


def test_rotary_gather_fused(K):
    # the fused launch with the rotary gather, bf16 P 16 (2-wave blocks) and fp32 P 32
    for seed, dtype, P, D, lens in ((332, "bf16", 16, 64, [16 * 300, 16 * 200 + 5]),
                                    (333, "f32", 32, 128, [32 * 250 + 7, 32 * 90])):
        w = W.custom(seed, B=2, Hq=8, Hkv=2, D=D, P=P, k=24, lens=lens, dtype=dtype)
        kv = kv_of(K, w)
        q = w.q.cuda()
        n_rows = 4
        cos, sin = K.rope_table(500000.0, w.D, 4096, n_rows, torch.device("cuda"))
        page_row = torch.full((w.num_phys_pages,), -1, dtype=torch.int32)
        half = w.num_phys_pages // 2
        page_row[:half] = torch.arange(half, dtype=torch.int32) % n_rows
        rope = K.Rope(cos, sin, page_row.cuda(), row_step=0)
        say(f"select_attend with the rotary gather ({dtype}, P {P})")
        summ_r = K.build_summaries(kv, rope=rope)
        fused = K.select_attend(kv, summ_r, q, w.k, rope=rope)
        sel, cnt = K.score_topk(kv, summ_r, q, w.k)
        out, lse = K.sparse_decode_attn(kv, q, sel, cnt, w.k, rope=rope,
                                        pages_per_split=K.step_pages_per_split(kv, w.k))
        torch.cuda.synchronize()
        assert_same(fused, (sel, cnt, out, lse))
