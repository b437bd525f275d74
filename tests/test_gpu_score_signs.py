"""Page scores of queries whose channels take every sign pattern over a KV head's group, on every
score launch layout, against the oracle bit for bit (bf16 caches).

The score of a page is the sum over the group's heads and channels of q*hi for q >= 0 and q*lo
otherwise ([FreeKV] section 2.1, with the upper-bound reading of the channel summaries). The
library forms it per channel from the group's sums of the non-negative and of the negative query
values. Here every channel follows one of six patterns over the G heads: all +0, all -0, all
positive, all negative, mixed signs, or a single non-zero head. Magnitudes span 2^-16 to 2^5, so
every fp64 sum stays exact. The cases run one, two and four pages per lane group and the
one-launch selection, with and without the decode-time tail refresh.
"""
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import assert_scores_close, assert_selection_equal, kv_of, say

pytestmark = pytest.mark.gpu

LENS16 = [40000, 1280, 5, 1, 33, 4096, 20000, 31999, 777, 64, 65, 50000, 12345, 2, 32, 8000]

# layout -> (B, lens, page-table width or 0 for the natural width)
CASES = {
    "one_page_per_lane_group": (2, [32 * 1000 - 7, 32 * 600], 0),   # 8 lists, <= 1024 pages
    "two_pages_per_lane_group": (2, [32 * 1500 + 3, 32 * 900], 0),  # 8 lists, 1025..8192 pages
    "one_launch_selection": (16, LENS16, 0),                        # 64 lists, <= 2048 pages
    "four_pages_per_lane_group": (16, LENS16, 2100),                # 64 lists, 2100-entry table
}


def sign_pattern_queries(B, Hkv, G, D, seed):
    """bf16 queries [B][Hkv*G][D]: channel d of every KV head's group follows pattern d % 6."""
    gen = torch.Generator().manual_seed(seed)
    shape = (B, Hkv, G, D)
    mag = torch.exp2(torch.randint(-16, 5, shape, generator=gen).float())
    mag = mag * (1.0 + torch.rand(shape, generator=gen))
    sign = torch.where(torch.rand(shape, generator=gen) < 0.5, -1.0, 1.0)
    pat = (torch.arange(D) % 6).view(1, 1, 1, D).expand(shape)
    lone = ((torch.arange(D) // 6) % G).view(1, 1, 1, D).expand(shape)
    head = torch.arange(G).view(1, 1, G, 1).expand(shape)
    q = torch.zeros(shape)
    q = torch.where(pat == 1, torch.full(shape, -0.0), q)
    q = torch.where(pat == 2, mag, q)
    q = torch.where(pat == 3, -mag, q)
    q = torch.where(pat == 4, sign * mag, q)
    q = torch.where((pat == 5) & (head == lone), sign * mag, q)
    return q.reshape(B, Hkv * G, D).to(torch.bfloat16)


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_page_amd import kvsel as K
    K.lib()  # raises if libkvsel.so is missing: no fallback
    return K


def test_sign_patterns_cover_the_six_cases():
    q = sign_pattern_queries(1, 1, 4, 128, 7).view(4, 128)
    bits = q.view(torch.int16)
    assert (bits[:, 0::6] == 0).all()  # +0
    assert (bits[:, 1::6] == torch.tensor(-0.0, dtype=torch.bfloat16).view(torch.int16)).all()
    assert (q[:, 2::6] > 0).all() and (q[:, 3::6] < 0).all()
    assert ((q[:, 4::6] > 0).any(0) & (q[:, 4::6] < 0).any(0)).any()
    assert ((q[:, 5::6] != 0).sum(0) == 1).all()


@pytest.mark.parametrize("case", list(CASES))
def test_sign_pattern_scores_are_exact(K, case):
    B, lens, width = CASES[case]
    w = W.custom(401, B=B, Hq=16, Hkv=4, D=128, P=32, k=24, lens=lens, dtype="bf16")
    w.q = sign_pattern_queries(w.B, w.Hkv, w.Hq // w.Hkv, w.D, 402)
    say(f"sign patterns, {case}: lists={w.B * w.Hkv} max pages={w.max_pages} width={width or w.max_pages}")
    kv = kv_of(K, w)
    if width:
        pt = torch.cat([w.page_table, torch.zeros(w.B, width - w.max_pages, dtype=torch.int32)], 1)
        kv = K.PagedKV(kv.k_pool, kv.v_pool, pt.cuda(), kv.seq_lens, w.Hq)
    q = w.q.cuda()
    summ = K.build_summaries(kv)
    ref_summ = O.page_summaries(w.k_pool, w.page_table, w.seq_lens, w.P)
    ref_sc = O.page_scores(w.q, ref_summ, w.page_table, w.seq_lens, w.P)
    ref_sel, ref_cnt = O.top_pages(ref_sc, w.seq_lens, w.P, w.k)
    for refresh in (False, True):
        sc = torch.full((w.B, w.Hkv, width or w.max_pages), float("nan"), device="cuda")
        sel, cnt = K.score_topk(kv, summ, q, w.k, refresh_tail=refresh, scores=sc)
        torch.cuda.synchronize()
        assert_scores_close(sc[:, :, :w.max_pages], ref_sc, w, exact=True)
        assert_selection_equal(sel, cnt, ref_sel, ref_cnt)
