"""kvsel_check_inputs: the device-side contract check flags exactly the broken contents.

Broken contents are given only to the check (whose reads stay inside the arrays whatever the
values), never to the other entry points."""
import pytest
import torch

import workloads as W
from gpu_common import kv_of, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_page_amd import kvsel as K
    K.lib()
    return K


def test_check_inputs_flags(K):
    w = W.custom(401, B=3, Hq=8, Hkv=2, D=64, P=16, k=6, lens=[300, 17, 0], dtype="bf16")
    kv = kv_of(K, w)
    summ = K.build_summaries(kv)
    sel, cnt = K.score_topk(kv, summ, w.q.cuda(), w.k)
    say("check_inputs: valid inputs")
    f = K.check_inputs(kv, sel, cnt)
    torch.cuda.synchronize()
    assert int(f.item()) == 0

    def flags_of(kvx, s=None, c=None):
        out = K.check_inputs(kvx, s, c, w.k if s is not None else None)
        torch.cuda.synchronize()
        return int(out.item())

    maxp = w.max_pages
    say("check_inputs: sequence length past the table")
    lens = kv.seq_lens.clone()
    lens[1] = maxp * w.P + 1
    assert flags_of(K.PagedKV(kv.k_pool, kv.v_pool, kv.page_table, lens, w.Hq)) == K.KVSEL_CHECK_SEQ_LEN
    lens[1] = -5
    assert flags_of(K.PagedKV(kv.k_pool, kv.v_pool, kv.page_table, lens, w.Hq)) == K.KVSEL_CHECK_SEQ_LEN
    say("check_inputs: page ids outside the pool")
    for bad in (-1, w.num_phys_pages):
        pt = kv.page_table.clone()
        pt[0, 5] = bad
        assert flags_of(K.PagedKV(kv.k_pool, kv.v_pool, pt, kv.seq_lens, w.Hq)) == K.KVSEL_CHECK_PAGE_ID
    pt = kv.page_table.clone()
    pt[1, maxp - 1] = -7  # past sequence 1's pages: not read, not flagged
    assert flags_of(K.PagedKV(kv.k_pool, kv.v_pool, pt, kv.seq_lens, w.Hq)) == 0
    say("check_inputs: broken selections")
    s2 = sel.clone()
    s2[0, 0, 0], s2[0, 0, 1] = s2[0, 0, 1], s2[0, 0, 0]  # not ascending
    assert flags_of(kv, s2, cnt) == K.KVSEL_CHECK_SELECTION
    s2 = sel.clone()
    s2[0, 1, 2] = w.n_pages(0)  # past the sequence
    assert flags_of(kv, s2, cnt) == K.KVSEL_CHECK_SELECTION
    c2 = cnt.clone()
    c2[1, 0] = w.n_pages(1) + 1  # count above min(k, N)
    assert flags_of(kv, sel, c2) == K.KVSEL_CHECK_SELECTION
    say("check_inputs: sticky flags")
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.check_inputs(K.PagedKV(kv.k_pool, kv.v_pool, pt, lens, w.Hq), flags=fl)
    K.check_inputs(kv, sel, cnt, flags=fl)
    torch.cuda.synchronize()
    assert int(fl.item()) == K.KVSEL_CHECK_SEQ_LEN
