"""kvsel_append_kv against the oracle's append, bit for bit: the pools, the lengths, and the tail
summaries it keeps current without a rebuild (checked after every step against the oracle's
summaries of the grown cache); the full-table refusal; and a decode step on the grown cache
against the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import (assert_attention_close, assert_selection_equal, assert_summaries_equal,
                        kv_of, oracle_path, say, scale_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_page_amd import kvsel as K
    K.lib()  # raises if libkvsel.so is missing: no fallback
    return K


def grown_case(seed, dtype, D, P, lens, T, Hq=8, Hkv=2, k=8):
    """A cache with room for T more tokens per sequence: the table is widened and every page the
    appends will open is given a spare physical page up front (the caller's allocator)."""
    extra = sum(-(-(L + T) // P) - -(-L // P) for L in lens)
    w = W.custom(seed, B=len(lens), Hq=Hq, Hkv=Hkv, D=D, P=P, k=k, lens=lens, dtype=dtype,
                 spare_pages=extra)
    width = max(-(-(L + T) // P) for L in lens)
    table = torch.zeros((w.B, width), dtype=torch.int32)
    table[:, : w.max_pages] = w.page_table
    used = {int(w.page_table[b, n]) for b in range(w.B) for n in range(w.n_pages(b))}
    spare = [p for p in range(w.num_phys_pages) if p not in used]
    for b, L in enumerate(lens):
        for n in range(-(-L // P), -(-(L + T) // P)):
            table[b, n] = spare.pop()
    return dataclasses.replace(w, page_table=table)


CASES = [("bf16", 128, 32), ("bf16", 64, 16), ("f32", 128, 16), ("f32", 64, 32)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_append_matches_oracle(K, case):
    dtype, D, P = case
    lens = [2 * P + 8, P - 1, 0, P, 1]
    T = P + 5  # crosses a page boundary in every sequence
    w = grown_case(711, dtype, D, P, lens, T)
    say(f"append {case}: lens {lens}, {T} steps")
    kv = kv_of(K, w)
    summ = K.build_summaries(kv)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    Kc, Vc = w.k_pool.double().numpy(), w.v_pool.double().numpy()
    cur = w.seq_lens.numpy().astype(np.int64)
    gen = torch.Generator().manual_seed(712)
    tdt = w.k_pool.dtype
    for t in range(T):
        kn = torch.randn((w.B, w.Hkv, D), generator=gen).to(tdt)
        vn = torch.randn((w.B, w.Hkv, D), generator=gen).to(tdt)
        K.append_kv(kv, kn.cuda(), vn.cuda(), summ=summ, flags=flags)
        Kc, Vc, cur, rej = O.append_tokens(Kc, Vc, w.page_table, cur, kn.double().numpy(),
                                           vn.double().numpy(), P)
        assert not rej.any()
        torch.cuda.synchronize()
        assert list(kv.seq_lens.cpu().numpy()) == list(cur), f"lengths after step {t}"
        wt = dataclasses.replace(w, seq_lens=torch.from_numpy(cur.astype(np.int32)))
        assert_summaries_equal(summ, O.page_summaries(Kc, w.page_table, wt.seq_lens, P), wt)
    assert int(flags.item()) == 0
    assert np.array_equal(kv.k_pool.double().cpu().numpy(), Kc)
    assert np.array_equal(kv.v_pool.permute(0, 1, 3, 2).double().cpu().numpy(), Vc)
    # a decode step on the grown cache (summaries current: no refresh)
    wg = dataclasses.replace(w, seq_lens=torch.from_numpy(cur.astype(np.int32)),
                             k_pool=torch.from_numpy(Kc).to(tdt), v_pool=torch.from_numpy(Vc).to(tdt))
    ref = oracle_path(wg, scale_of(D))
    sel, cnt, out, lse = K.select_attend(kv, summ, w.q.cuda(), w.k)
    torch.cuda.synchronize()
    assert_selection_equal(sel, cnt, ref["sel"], ref["cnt"], ref["fp32"])
    assert_attention_close(out, lse, ref["out"], ref["lse"], dtype)


def test_append_more_heads_than_waves(K):
    """20 KV heads: the block's 16 waves take heads 16..19 on a second pass."""
    P, T = 16, 20
    lens = [3 * P + 1, P - 1, 0]
    w = grown_case(715, "bf16", 64, P, lens, T, Hq=20, Hkv=20, k=4)
    say(f"append: 20 KV heads, lens {lens}, {T} steps")
    kv = kv_of(K, w)
    summ = K.build_summaries(kv)
    Kc, Vc = w.k_pool.double().numpy(), w.v_pool.double().numpy()
    cur = w.seq_lens.numpy().astype(np.int64)
    gen = torch.Generator().manual_seed(716)
    for t in range(T):
        kn = torch.randn((w.B, w.Hkv, 64), generator=gen).to(torch.bfloat16)
        vn = torch.randn((w.B, w.Hkv, 64), generator=gen).to(torch.bfloat16)
        K.append_kv(kv, kn.cuda(), vn.cuda(), summ=summ)
        Kc, Vc, cur, _ = O.append_tokens(Kc, Vc, w.page_table, cur, kn.double().numpy(),
                                         vn.double().numpy(), P)
    torch.cuda.synchronize()
    assert list(kv.seq_lens.cpu().numpy()) == list(cur)
    wt = dataclasses.replace(w, seq_lens=torch.from_numpy(cur.astype(np.int32)))
    assert_summaries_equal(summ, O.page_summaries(Kc, w.page_table, wt.seq_lens, P), wt)
    assert np.array_equal(kv.k_pool.double().cpu().numpy(), Kc)
    assert np.array_equal(kv.v_pool.permute(0, 1, 3, 2).double().cpu().numpy(), Vc)


def test_append_refuses_a_full_table(K):
    w = W.custom(713, B=2, Hq=8, Hkv=2, D=64, P=16, k=4, lens=[32, 10], dtype="bf16")
    say("append: full table")
    kv = kv_of(K, w)
    summ = K.build_summaries(kv)
    before_k = kv.k_pool.clone()
    before_s = summ.clone()
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    kn = torch.ones((2, 2, 64), dtype=torch.bfloat16, device="cuda")
    out_lens = torch.empty(2, dtype=torch.int32, device="cuda")
    out_lens.copy_(kv.seq_lens)
    K.append_kv(kv, kn, kn, summ=summ, seq_lens_out=out_lens, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & 1
    assert out_lens.tolist() == [32, 11] and kv.seq_lens.tolist() == [32, 10]
    p0 = [int(x) for x in w.page_table[0, :2]]
    assert torch.equal(kv.k_pool[p0], before_k[p0])  # the full sequence's pages untouched
    assert torch.equal(summ[0], before_s[0])
    p1 = int(w.page_table[1, 0])
    assert torch.equal(kv.k_pool[p1, :, 10], kn[1])  # the other sequence took its token


def test_growing_speculative_loop(K):
    """Appends interleaved with speculative steps (the summaries kept current by the appends, no
    refresh): each step's outputs equal the serial calls' bit for bit, and every step's fresh
    selection, similarity, decision and used lists match the oracle on the grown cache, with the
    attention against the oracle's over its own used lists."""
    T, k = 12, 6
    lens = [5 * 16 + 3, 2 * 16, 16 - 2]
    w = grown_case(721, "bf16", 128, 16, lens, T, Hq=16, Hkv=4, k=k)
    say(f"growing speculative loop: lens {lens}, {T} steps")
    kv_a, kv_b = kv_of(K, w), kv_of(K, w)
    summ_a, summ_b = K.build_summaries(kv_a), K.build_summaries(kv_b)
    gen = torch.Generator().manual_seed(722)
    q = w.q.float()
    sel_prev = cnt_prev = None
    o_prev = None
    Kc, Vc = w.k_pool.double().numpy(), w.v_pool.double().numpy()
    cur = w.seq_lens.numpy().astype(np.int64)
    for t in range(T):
        kn = torch.randn((w.B, w.Hkv, 128), generator=gen).to(torch.bfloat16)
        vn = torch.randn((w.B, w.Hkv, 128), generator=gen).to(torch.bfloat16)
        q_prev = q
        q = 0.9 * q + 0.45 * torch.randn(q.shape, generator=gen)
        qt, qp = q.to(torch.bfloat16).cuda(), q_prev.to(torch.bfloat16).cuda()
        for kv, summ in ((kv_a, summ_a), (kv_b, summ_b)):
            K.append_kv(kv, kn.cuda(), vn.cuda(), summ=summ)
        Kc, Vc, cur, _ = O.append_tokens(Kc, Vc, w.page_table, cur, kn.double().numpy(),
                                         vn.double().numpy(), 16)
        first = t == 0
        prev_i = sel_prev if not first else torch.zeros((w.B, w.Hkv, k), dtype=torch.int32, device="cuda")
        prev_c = cnt_prev if not first else torch.zeros((w.B, w.Hkv), dtype=torch.int32, device="cuda")
        reuse = K.Reuse(qp, prev_i, prev_c, 0.8, first_step=first)
        spec = K.speculative_step(kv_a, summ_a, qt, k, reuse)
        sel, cnt, used, ucnt, corr, sim = K.score_topk(kv_b, summ_b, qt, k, reuse=reuse)
        out, lse = K.sparse_decode_attn(kv_b, qt, used, ucnt, k,
                                        pages_per_split=K.step_pages_per_split(kv_b, k))
        torch.cuda.synchronize()
        for x, y, name in zip(spec, (sel, cnt, used, ucnt, corr, sim, out, lse),
                              ("sel", "cnt", "used", "ucnt", "corrected", "similarity", "out", "lse")):
            assert torch.equal(x, y), f"step {t}: {name} differs"
        sel_prev, cnt_prev = spec[0].clone(), spec[1].clone()
        # the oracle on the grown cache
        o_summ = O.page_summaries(Kc, w.page_table, cur, 16)
        sc = O.page_scores(qt.cpu(), o_summ, w.page_table, cur, 16)
        f_sel, f_cnt = O.top_pages(sc, cur, 16, k)
        C = O.query_similarity(qt.cpu(), qp.cpu(), w.Hkv)
        if first:
            o_prev = (f_sel, f_cnt)
        u_sel, u_cnt, o_corr = O.speculative_choice(f_sel, f_cnt, o_prev[0], o_prev[1], C, 0.8,
                                                    first)
        assert_selection_equal(spec[0], spec[1], f_sel, f_cnt)
        assert np.abs(spec[5].cpu().numpy() - C).max() < 1e-12
        np.testing.assert_array_equal(spec[4].cpu().numpy(), o_corr)
        assert_selection_equal(spec[2], spec[3], u_sel, u_cnt)
        o_out, o_lse = O.sparse_decode_attention(qt.cpu(), Kc, Vc, w.page_table, cur, u_sel, u_cnt,
                                                 16, scale_of(128))
        assert_attention_close(spec[6], spec[7], o_out, o_lse, "bf16")
        o_prev = (f_sel, f_cnt)
    assert list(kv_a.seq_lens.cpu().numpy()) == list(cur)


def free_list_case(seed, lens, T, P=16, D=64, Hkv=2, extra_free=3):
    """A cache whose table rows hold junk (-7) past each sequence's pages, and a shuffled free list
    of the spare physical pages: one for every page the T appends will open, plus extra_free."""
    opened = sum(-(-(L + T) // P) - -(-L // P) for L in lens)
    w = W.custom(seed, B=len(lens), Hq=2 * Hkv, Hkv=Hkv, D=D, P=P, k=4, lens=lens, dtype="bf16",
                 spare_pages=opened + extra_free)
    width = max(-(-(L + T) // P) for L in lens)
    table = np.full((w.B, width), -7, np.int32)
    used = set()
    for b in range(w.B):
        n = w.n_pages(b)
        table[b, :n] = w.page_table[b, :n].numpy()
        used.update(int(x) for x in table[b, :n])
    spare = np.array([p for p in range(w.num_phys_pages) if p not in used], np.int32)
    np.random.default_rng(seed).shuffle(spare)
    return dataclasses.replace(w, page_table=torch.from_numpy(table)), spare, opened


def test_append_takes_pages_from_the_free_list(K):
    """Pages opened by the appends come off the top of the free list into the table (which
    sequence gets which of them is unspecified: checked as a set); the pools and summaries then
    equal the oracle's append on the table the appends produced."""
    P, T = 16, 16 + 5
    lens = [2 * P - 1, P, 0, 3 * P + 4, P - 2]
    w, spare, opened = free_list_case(731, lens, T, P=P)
    say(f"append from a free list: lens {lens}, {T} steps, {opened} pages to open")
    kv = kv_of(K, w)
    summ = K.build_summaries(kv)
    fp = K.FreePages(torch.from_numpy(spare).cuda(), torch.tensor([len(spare)], dtype=torch.int32,
                                                                  device="cuda"))
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    gen = torch.Generator().manual_seed(732)
    steps = []
    for t in range(T):
        kn = torch.randn((w.B, w.Hkv, 64), generator=gen).to(torch.bfloat16)
        vn = torch.randn((w.B, w.Hkv, 64), generator=gen).to(torch.bfloat16)
        K.append_kv(kv, kn.cuda(), vn.cuda(), summ=summ, flags=flags, free_pages=fp)
        steps.append((kn, vn))
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    assert int(fp.count.item()) == len(spare) - opened
    table = kv.page_table.cpu().numpy()
    before = w.page_table.numpy()
    taken = []
    for b, L in enumerate(lens):
        n0, n1 = -(-L // P), -(-(L + T) // P)
        assert (table[b, :n0] == before[b, :n0]).all()
        assert (table[b, n1:] == -7).all()
        taken.extend(int(x) for x in table[b, n0:n1])
    assert sorted(taken) == sorted(int(x) for x in spare[len(spare) - opened:])
    Kc, Vc = w.k_pool.double().numpy(), w.v_pool.double().numpy()
    cur = np.asarray(lens, np.int64)
    for kn, vn in steps:
        Kc, Vc, cur, rej = O.append_tokens(Kc, Vc, table, cur, kn.double().numpy(),
                                           vn.double().numpy(), P)
        assert not rej.any()
    assert list(kv.seq_lens.cpu().numpy()) == list(cur)
    assert np.array_equal(kv.k_pool.double().cpu().numpy(), Kc)
    assert np.array_equal(kv.v_pool.permute(0, 1, 3, 2).double().cpu().numpy(), Vc)
    wt = dataclasses.replace(w, page_table=torch.from_numpy(table),
                             seq_lens=torch.from_numpy(cur.astype(np.int32)))
    assert_summaries_equal(summ, O.page_summaries(Kc, table, wt.seq_lens, P), wt)


def test_free_list_runs_out(K):
    """Two sequences open a page with one id on the list: one takes it, the other is left as it
    was (KVSEL_CHECK_NO_FREE_PAGE) and the count stays 0; a sequence that does not open a page is
    unaffected. Then an id outside the pool is consumed and the sequence again left as it was
    (KVSEL_CHECK_PAGE_ID)."""
    P = 16
    lens = [P, 2 * P, P - 1]
    w, spare, _ = free_list_case(741, lens, 1, P=P, extra_free=0)
    say("append: free list runs out")
    kv = kv_of(K, w)
    summ = K.build_summaries(kv)
    fp = K.FreePages(torch.from_numpy(spare).cuda(), torch.ones(1, dtype=torch.int32, device="cuda"))
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    kn = torch.ones((w.B, w.Hkv, 64), dtype=torch.bfloat16, device="cuda")
    K.append_kv(kv, kn, kn, summ=summ, flags=flags, free_pages=fp)
    torch.cuda.synchronize()
    got = kv.seq_lens.cpu().tolist()
    assert int(flags.item()) == K.KVSEL_CHECK_NO_FREE_PAGE and int(fp.count.item()) == 0
    assert got[2] == P and sorted(got[:2]) == sorted([P + 1, 2 * P]) or \
        sorted(got[:2]) == sorted([P, 2 * P + 1]) and got[2] == P
    won = 0 if got[0] == P + 1 else 1
    lost = 1 - won
    table = kv.page_table.cpu().numpy()
    assert table[won, lens[won] // P] == spare[0] and table[lost, lens[lost] // P] == -7
    # an id outside the pool: consumed, the sequence left as it was
    flags.zero_()
    fp.ids[0] = w.num_phys_pages + 5
    fp.count.fill_(1)
    before = kv.seq_lens.clone()
    only = torch.zeros((w.B, w.Hkv, 64), dtype=torch.bfloat16, device="cuda")
    K.append_kv(kv, only, only, summ=summ, flags=flags, free_pages=fp)
    torch.cuda.synchronize()
    assert int(flags.item()) & K.KVSEL_CHECK_PAGE_ID
    assert int(fp.count.item()) == 0
    after = kv.seq_lens.cpu().tolist()
    assert after[lost] == before[lost].item()
    assert kv.page_table[lost, lens[lost] // P].item() == -7
