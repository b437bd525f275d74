"""kvsel_select_attend_static (scores and split partials in the library's per-GPU device array,
no workspace argument) against kvsel_select_attend with a caller workspace, bit for bit, on two
calls in a row, the second with a smaller input: a batch of 128 (sequence, KV head) lists, which
runs the separate selection and attention launches, then a smaller batch that takes the fused
selection launch (the second call finds the first call's data in the array)."""
import pytest
import torch

import workloads as W
from gpu_common import kv_of, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_page_amd import kvsel as K
    K.lib()  # raises if libkvsel.so is missing: no fallback
    return K


CALLS = [
    dict(seed=951, B=16, Hq=32, Hkv=8, D=128, P=32, k=32, dtype="bf16",
         lens=[4096 + 731 * i for i in range(16)]),
    dict(seed=952, B=2, Hq=16, Hkv=4, D=128, P=16, k=12, dtype="bf16", lens=[3000, 517]),
]


def test_static_scratch_matches_workspace_entry_point(K):
    needs = []
    for c in CALLS:
        w = W.custom(**c)
        kv = kv_of(K, w)
        need = K.workspace_bytes(kv, w.k, K.KVSEL_OP_SELECT_ATTEND)
        needs.append(need)
        say(f"static scratch: B={w.B} Hkv={w.Hkv} k={w.k}, scratch need {need} bytes")
        assert need <= K.KVSEL_STATIC_SCRATCH_BYTES
        q = w.q.cuda()
        summ = K.build_summaries(kv)
        summ_a, summ_b = summ.clone(), summ.clone()  # the tail refresh writes the summaries
        ref = K.select_attend(kv, summ_a, q, w.k, refresh_tail=True)
        sel = torch.full((w.B, w.Hkv, w.k), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((w.B, w.Hkv), -7, dtype=torch.int32, device="cuda")
        out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
        lse = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device="cuda")
        got = K.select_attend_static(kv, summ_b, q, w.k, sel_idx=sel, sel_cnt=cnt, out=out,
                                     lse=lse, refresh_tail=True)
        torch.cuda.synchronize()
        for x, y, name in zip(got, ref, ("sel_idx", "sel_cnt", "out", "lse")):
            assert torch.equal(x, y), f"{name} differs from kvsel_select_attend"
        # bitwise: rows past a sequence's pages are never written and may hold NaN bit patterns
        assert torch.equal(summ_a.view(torch.int16), summ_b.view(torch.int16))
    assert needs[1] < needs[0]  # the second call is the smaller one
