"""Checks of the seeded input generators (no GPU)."""

import numpy as np
import torch

from diffusion_drafted_verification_amd import inputs as I


def test_page_table_is_a_bijection_with_capacity():
    lens = I.draw_ctx_lens("qwen3_8b_ragged16")
    assert lens.min() >= 1024 and lens.max() <= 16384
    table, total = I.make_page_table(lens, 32, 16, shuffle=True, seed=3, extra_pages=5)
    used = table[table >= 0]
    assert len(np.unique(used)) == len(used) and used.max() < total
    for b, L in enumerate(lens):
        assert (table[b] >= 0).sum() * 16 >= L + 32
    assert total == len(used) + 5
    # shuffled: logically adjacent pages are not physically adjacent in general
    assert np.mean(np.diff(table[0][table[0] >= 0]) == 1) < 0.1


def test_identity_pages_for_contiguous_cache():
    a = I.make_attn_inputs("tiny_fp32")
    assert a.q.dtype == torch.float32 and tuple(a.q.shape) == (1, 32, 4, 64)
    assert torch.equal(a.page_table[0], torch.arange(a.page_table.shape[1], dtype=torch.int32))


def test_seeded_and_reproducible():
    a = I.make_attn_inputs("qwen3_1p7b_2k", seed=0)
    b = I.make_attn_inputs("qwen3_1p7b_2k", seed=0)
    c = I.make_attn_inputs("qwen3_1p7b_2k", seed=1)
    assert torch.equal(a.k_cache, b.k_cache) and torch.equal(a.page_table, b.page_table)
    assert not torch.equal(a.q, c.q)
    assert a.q.dtype == torch.bfloat16
    # N(0,1) draws
    x = a.k_cache.float()
    assert abs(x.mean().item()) < 0.01 and abs(x.std().item() - 1) < 0.01


def test_planted_logits_make_the_target_the_unique_max():
    x, t = I.make_logits(2, 32, 5000, seed=2, plant=True)
    top2 = torch.topk(x, 2, dim=-1)
    assert torch.equal(top2.indices[..., 0].int(), t)
    assert bool((top2.values[..., 0] > top2.values[..., 1]).all())


def test_drafts_agree_on_exactly_the_prefix():
    t = np.arange(64).reshape(2, 32) * 3
    pre = [0, 17]
    d = I.make_drafts(t, pre, 1000, seed=1).numpy()
    for b, a in enumerate(pre):
        assert np.array_equal(d[b, :a], t[b, :a]) and d[b, a] != t[b, a]


def test_sample_inputs_shapes_seeds_and_draft_distribution():
    """Seeded and reproducible; drafts follow softmax(draft_logits / T): at a
    tiny vocabulary the empirical draft frequencies of many rows sharing one
    draft row match that softmax."""
    a = I.make_sample_inputs(3, 5, 100, 0.7, seed=4, workload="qwen3_8b_8k")
    b = I.make_sample_inputs(3, 5, 100, 0.7, seed=4, workload="qwen3_8b_8k")
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    ar, dr, d, ua, ur = a
    assert ar.shape == dr.shape == (3, 5, 100) and d.shape == ua.shape == (3, 5) and ur.shape == (3,)
    assert d.dtype == torch.int32 and ua.dtype == ur.dtype == torch.float32
    assert float(ua.min()) >= 0 and float(ua.max()) < 1
    assert 0.1 < float((dr - ar).std()) < 0.3            # draft head near the AR head
    # each draft is a sample of its own row's softmax(draft_logits / T): over
    # many rows the indicator minus the row's probability averages to zero
    n, V, T = 20000, 4, 0.9
    _, dr, d, _, _ = I.make_sample_inputs(1, n, V, T, seed=1, workload="", std=1.0)
    q = torch.softmax(dr[0].double() / T, dim=-1)
    ind = torch.nn.functional.one_hot(d[0].long(), V).double()
    dev_ = (ind - q).mean(0)
    sd = torch.sqrt((q * (1 - q)).mean(0) / n)
    assert (dev_.abs() < 5 * sd).all(), (dev_, sd)
