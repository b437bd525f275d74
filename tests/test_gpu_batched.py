"""The batched 32K and 128K workloads (B sequences of the full context, drawn on the device) in
the bench's launch configuration: one kvsel_select_attend call with the tail refresh, at the
default split of a call with this many lists (8 pages per split). Sampled sequences -- the first,
the last and two in between -- are checked against the CPU oracle on their own pages: summaries and
selection bit-exact, attention within the bf16 tolerance."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import assert_attention_close, assert_selection_equal, oracle_path, say, scale_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_page_amd import kvsel as K
    K.lib()  # raises if libkvsel.so is missing: no fallback
    return K


def sequence_on_host(w, b):
    """Sequence b of a device batch as a one-sequence CPU workload over its own pages, in order."""
    pages = w.page_table[b, :w.n_pages(b)].long()
    return W.Workload(w.name, w.dtype, 1, w.Hq, w.Hkv, w.D, w.P, w.k,
                      w.seq_lens[b:b + 1].cpu(),
                      torch.arange(len(pages), dtype=torch.int32).reshape(1, -1),
                      w.k_pool[pages].cpu(), w.v_pool[pages].cpu(), w.q[b:b + 1].cpu())


@pytest.mark.parametrize("name", sorted(W.BATCHED))
def test_batched_workload_sampled_sequences(K, name):
    w = W.batched_device(name, "cuda")
    say(f"batched workload {name}: B {w.B}, context {int(w.seq_lens.max())}, k {w.k}")
    scale = scale_of(w.D)
    kv = K.PagedKV(w.k_pool, K.device_v_layout(w.v_pool), w.page_table, w.seq_lens, w.Hq)
    summ = K.build_summaries(kv)
    sel, cnt, out, lse = K.select_attend(kv, summ, w.q, w.k, refresh_tail=True, scale=scale)
    torch.cuda.synchronize()
    for b in sorted({0, w.B // 3, (2 * w.B) // 3, w.B - 1}):
        ws = sequence_on_host(w, b)
        ref = oracle_path(ws, scale)
        s = summ[b:b + 1].float().cpu().numpy()
        r = ref["summ"].transpose(1, 0, 2, 3)[None]  # [1][Hkv][N][2][D], pages in order
        assert np.array_equal(s[:, :, :ws.n_pages(0)], r), f"sequence {b}: summaries differ"
        assert_selection_equal(sel[b:b + 1], cnt[b:b + 1], ref["sel"], ref["cnt"])
        err = assert_attention_close(out[b:b + 1], lse[b:b + 1], ref["out"], ref["lse"], "bf16")
        say(f"{name} sequence {b}: selection bit-exact, attention max abs err {err:.3g}")
