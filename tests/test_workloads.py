"""The seeded input generators: determinism and the structure each workload promises."""
import numpy as np
import pytest
import torch

import workloads as W


def test_deterministic_and_seed_sensitive():
    a, b = W.tiny_fp32(), W.tiny_fp32()
    assert torch.equal(a.k_pool, b.k_pool) and torch.equal(a.q, b.q)
    c = W.tiny_fp32(seed=77)
    assert not torch.equal(a.k_pool, c.k_pool)


def test_tiny_planted_keys():
    w = W.tiny_fp32()
    assert w.k_pool.shape == (64, 2, 16, 64) and w.dtype == "f32"
    for g, (p, s) in enumerate(zip(w.extra["planted_pages"], w.extra["planted_slots"])):
        for j in range(2):
            key = w.k_pool[p, j, s].double()
            q = w.q[0, j * 4 + g].double()
            assert abs(key.norm().item() - 24.0) < 1e-4
            assert torch.nn.functional.cosine_similarity(key, q, dim=0).item() > 0.99999


def test_ragged_batch_structure():
    w = W.ragged_batch()
    lens = w.seq_lens.numpy()
    assert w.B == 16 and lens.min() >= 4096 and lens.max() <= 16384
    used = np.concatenate([w.page_table[b, :w.n_pages(b)].numpy() for b in range(w.B)])
    assert np.array_equal(np.sort(used), np.arange(w.num_phys_pages))  # a permutation of the pool
    assert not np.array_equal(used, np.arange(w.num_phys_pages))
    assert w.k == 32


@pytest.mark.slow
def test_qwen_needles_align_with_group_query():
    w = W.qwen4b_128k()
    assert w.k_pool.shape == (4096, 8, 32, 128) and w.k == 128
    q = w.q.double()[0]
    for j in range(8):
        u = q[j * 4:(j + 1) * 4].sum(0)
        for p in w.extra["needle_pages"]:
            m = w.k_pool[p, j].double().mean(0)
            cos = torch.nn.functional.cosine_similarity(m, u, dim=0).item()
            assert abs(cos - 0.9) < 0.01


def test_speculative_queries_are_correlated():
    w = W.speculative_rope(steps=8)
    qs = w.extra["q_steps"].double()
    cos = torch.nn.functional.cosine_similarity(qs[1:], qs[:-1], dim=-1)
    assert 0.75 < cos.mean().item() < 0.92
    assert torch.equal(w.q, w.extra["q_steps"][0])


def test_batched_device_structure(monkeypatch):
    """The device-drawn batch generator (run here on the CPU at a small size): shapes, one
    permutation of the pool over all sequences, the outlier channels, determinism per seed."""
    monkeypatch.setitem(W.BATCHED, "small_batch", (3, 4096, 512))
    w = W.batched_device("small_batch", "cpu")
    assert w.k_pool.shape == (384, 8, 32, 128) and w.v_pool.shape == w.k_pool.shape
    assert w.page_table.shape == (3, 128) and w.k == 16 and w.B == 3
    assert w.seq_lens.tolist() == [4096] * 3 and w.q.dtype == torch.bfloat16
    assert torch.equal(torch.sort(w.page_table.flatten().long())[0], torch.arange(384))
    k = w.k_pool.float()
    for j, chans in enumerate(w.extra["outlier_channels"]):
        std = k[:, j].std(dim=(0, 1))
        others = torch.ones(128, dtype=torch.bool)
        others[chans] = False
        assert std[chans].min() > 6.0 and std[others].max() < 1.5
    w2 = W.batched_device("small_batch", "cpu")
    assert torch.equal(w.k_pool, w2.k_pool) and torch.equal(w.page_table, w2.page_table)
    w3 = W.batched_device("small_batch", "cpu", seed=7)
    assert not torch.equal(w.q, w3.q)
