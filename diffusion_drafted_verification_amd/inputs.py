"""Seeded synthetic inputs for one dual-view decode step.

This module only draws random numbers and lays them out; it contains none of
the step's arithmetic (no attention, no greedy argmax, no acceptance), so the
HIP path and the CPU oracle can both be fed from it.  (Sampled drafts are
drawn from the draft head's own distribution with the Gumbel-max trick: the
drafting that precedes the step, not part of it.)

Workloads (Qwen3-shaped layers; the pages publish no kernel-level workload,
so the shapes are the Qwen3 family the method is evaluated on):

===================  ===================================================
name                 shape
===================  ===================================================
tiny_fp32            B1, Hq4/Hkv1, D64, L256, K32, fp32, identity pages,
                     logits 32 x 1024 ~ N(0, 4^2), 12 agreeing drafts
qwen3_1p7b_2k        B1, Hq16/Hkv8, D128, L2048, bf16, shuffled 16-token
                     pages, logits 32 x 151936, Geometric(11.7) prefix
qwen3_8b_8k          B1, Hq32/Hkv8, D128, L8192, bf16, shuffled pages
qwen3_8b_ragged16    B16, L_b ~ U[1024, 16384], shuffled pages
qwen3_8b_32k_b4      B4, L32768, 36 layers with independent K/V
===================  ===================================================

q, k and v are N(0, 1) fp32 draws rounded to the storage type (RNE).  The
draft/AR agreement prefix is Geometric with mean 11.7 on {0, 1, ...}, capped
at K: the acceptance length the explainer reports on MATH-500 (§4); synthetic
logits stand in for that benchmark.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

PAGE_SIZE = 16
QWEN3_VOCAB = 151936
MEAN_ACCEPT = 11.7

WORKLOADS = {
    "tiny_fp32": dict(batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64, ctx=256, block_k=32,
                      dtype=torch.float32, shuffle=False, vocab=1024, layers=1),
    "qwen3_1p7b_2k": dict(batch=1, n_q_heads=16, n_kv_heads=8, head_dim=128, ctx=2048, block_k=32,
                          dtype=torch.bfloat16, shuffle=True, vocab=QWEN3_VOCAB, layers=1),
    "qwen3_8b_8k": dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, ctx=8192, block_k=32,
                        dtype=torch.bfloat16, shuffle=True, vocab=QWEN3_VOCAB, layers=1),
    "qwen3_8b_ragged16": dict(batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, ctx=(1024, 16384),
                              block_k=32, dtype=torch.bfloat16, shuffle=True, vocab=QWEN3_VOCAB, layers=1),
    "qwen3_8b_32k_b4": dict(batch=4, n_q_heads=32, n_kv_heads=8, head_dim=128, ctx=32768, block_k=32,
                            dtype=torch.bfloat16, shuffle=True, vocab=QWEN3_VOCAB, layers=36),
}

_TENSOR_IDS = {"ctx": 1, "pages": 2, "q": 3, "k_cache": 4, "v_cache": 5, "k_blk": 6, "v_blk": 7,
               "logits": 8, "targets": 9, "prefix": 10, "drafts": 11, "draft_logits": 12, "gumbel": 13,
               "u_accept": 14, "u_resample": 15, "lm_hidden": 16, "lm_weight": 17, "lm_targets": 18}


def _seed(seed, workload, layer, tensor):
    """Independent, reproducible stream id per (seed, workload, layer, tensor)."""
    wl = sorted(WORKLOADS).index(workload) if workload in WORKLOADS else 99
    return ((seed * 1000003 + wl) * 1009 + layer) * 101 + _TENSOR_IDS[tensor]


def _gen(device, s):
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _randn(shape, dtype, device, s, std=1.0):
    x = torch.randn(shape, generator=_gen(device, s), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


@dataclass
class AttnInputs:
    q: torch.Tensor            # [B, K, Hq, D]
    k_cache: torch.Tensor      # [num_pages, Hkv, P, D]
    v_cache: torch.Tensor
    k_blk: torch.Tensor        # [B, K, Hkv, D]
    v_blk: torch.Tensor
    page_table: torch.Tensor   # [B, max_pages] int32, -1 = unused
    ctx_lens: torch.Tensor     # [B] int32
    max_ctx_len: int
    meta: dict = field(default_factory=dict)

    def to(self, device):
        f = lambda t: t.to(device)
        return AttnInputs(f(self.q), f(self.k_cache), f(self.v_cache), f(self.k_blk), f(self.v_blk),
                          f(self.page_table), f(self.ctx_lens), self.max_ctx_len, dict(self.meta))


def draw_ctx_lens(workload, seed=0, batch=None):
    """Per-sequence cached context lengths (uniform, or U[lo, hi] inclusive)."""
    w = WORKLOADS[workload]
    B = w["batch"] if batch is None else batch
    if isinstance(w["ctx"], tuple):
        lo, hi = w["ctx"]
        rng = np.random.default_rng(_seed(seed, workload, 0, "ctx"))
        return rng.integers(lo, hi + 1, size=B).astype(np.int32)
    return np.full(B, w["ctx"], dtype=np.int32)


def make_page_table(ctx_lens, block_k, page_size=PAGE_SIZE, shuffle=True, seed=0, extra_pages=0,
                    max_pages=None):
    """Page table with room for ctx + block_k tokens per sequence.

    Each sequence b owns ceil((L_b + K) / P) physical pages; when `shuffle`
    the physical ids are a seeded uniform permutation of all pages (so
    logically adjacent pages are scattered), otherwise they are consecutive
    (a contiguous cache).  `extra_pages` appends unowned pages to the pool.
    Unused table entries are -1.  Returns (page_table int32 [B, max_pages],
    num_pages).
    """
    lens = np.asarray(ctx_lens, dtype=np.int64)
    need = [-(-(int(L) + block_k) // page_size) for L in lens]
    total = int(sum(need)) + extra_pages
    mp = max(need) if max_pages is None else max_pages
    assert mp >= max(need)
    if shuffle:
        rng = np.random.default_rng([seed, _TENSOR_IDS["pages"]])
        perm = rng.permutation(total)
    else:
        perm = np.arange(total)
    table = np.full((len(lens), mp), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, total


def make_attn_inputs(workload, seed=0, layer=0, device="cpu", ctx_lens=None, batch=None,
                     extra_pages=0, dtype=None):
    """q, paged K/V cache, block K/V, page table and context lengths of one
    layer of `workload`, drawn on `device` from fixed seeds."""
    w = WORKLOADS[workload]
    B = w["batch"] if batch is None else batch
    K, Hq, Hkv, D = w["block_k"], w["n_q_heads"], w["n_kv_heads"], w["head_dim"]
    dt = w["dtype"] if dtype is None else dtype
    lens = draw_ctx_lens(workload, seed, B) if ctx_lens is None else np.asarray(ctx_lens, dtype=np.int32)
    table, num_pages = make_page_table(lens, K, PAGE_SIZE, w["shuffle"], seed=seed + 1000 * layer,
                                       extra_pages=extra_pages)
    s = lambda name: _seed(seed, workload, layer, name)
    q = _randn((B, K, Hq, D), dt, device, s("q"))
    kc = _randn((num_pages, Hkv, PAGE_SIZE, D), dt, device, s("k_cache"))
    vc = _randn((num_pages, Hkv, PAGE_SIZE, D), dt, device, s("v_cache"))
    kb = _randn((B, K, Hkv, D), dt, device, s("k_blk"))
    vb = _randn((B, K, Hkv, D), dt, device, s("v_blk"))
    return AttnInputs(q, kc, vc, kb, vb,
                      torch.from_numpy(table).to(device), torch.from_numpy(lens).to(device),
                      int(lens.max()), dict(workload=workload, seed=seed, layer=layer))


def kv_bytes(ctx_lens, n_kv_heads, head_dim, elem_bytes):
    """Algorithmic bytes of cached K and V one block-attention call reads."""
    return int(np.sum(np.asarray(ctx_lens, dtype=np.int64))) * n_kv_heads * head_dim * 2 * elem_bytes


def make_logits(batch, block_k, vocab, seed=0, workload="", std=4.0, plant=False, device="cpu"):
    """AR logits [B, K, V] fp32 ~ N(0, std^2).

    With `plant`, draws are clipped to +-6 std and one seeded target token per
    row is set to +8 std, so the row's greedy token is that target by
    construction (no argmax is computed here).  Returns (logits, targets or
    None); targets is int32 [B, K].
    """
    x = torch.randn((batch, block_k, vocab), generator=_gen(device, _seed(seed, workload, 0, "logits")),
                    device=device, dtype=torch.float32).mul_(std)
    if not plant:
        return x, None
    x.clamp_(-6.0 * std, 6.0 * std)
    rng = np.random.default_rng(_seed(seed, workload, 0, "targets"))
    t = rng.integers(0, vocab, size=(batch, block_k)).astype(np.int32)
    tt = torch.from_numpy(t).to(device=device, dtype=torch.int64)
    x.scatter_(2, tt.unsqueeze(-1), 8.0 * std)
    return x, torch.from_numpy(t).to(device)


def geometric_prefix(batch, block_k, seed=0, workload="", mean=MEAN_ACCEPT):
    """Draft/AR agreement prefix lengths ~ Geometric(mean) on {0, 1, ...},
    capped at block_k (p = 1 / (1 + mean))."""
    rng = np.random.default_rng(_seed(seed, workload, 0, "prefix"))
    a = rng.geometric(1.0 / (1.0 + mean), size=batch) - 1
    return np.minimum(a, block_k).astype(np.int32)


def make_drafts(targets, prefix_lens, vocab, seed=0, workload=""):
    """Draft tokens that agree with `targets` on exactly the first
    prefix_lens[b] positions: equal there, a different token at the prefix
    end (when it is < K), uniform tokens after it."""
    t = np.asarray(targets.cpu() if hasattr(targets, "cpu") else targets, dtype=np.int64)
    B, K = t.shape
    rng = np.random.default_rng(_seed(seed, workload, 0, "drafts"))
    d = rng.integers(0, vocab, size=(B, K))
    for b in range(B):
        a = int(prefix_lens[b])
        d[b, :a] = t[b, :a]
        if a < K:
            d[b, a] = (t[b, a] + 1 + rng.integers(0, vocab - 1)) % vocab
    return torch.from_numpy(d.astype(np.int32))


def block_kv_bytes_per_step(block_k, layers, n_kv_heads, head_dim, elem_bytes=2):
    """Size of one block's transient K/V over all layers (the method's O(1)
    memory overhead: the block rows are a K-row buffer, not a second cache)."""
    return block_k * layers * n_kv_heads * head_dim * 2 * elem_bytes


def make_sample_inputs(batch, block_k, vocab, temperature, seed=0, workload="", std=4.0, draft_noise=0.2,
                       device="cpu"):
    """Inputs of the sampled consensus at temperature T.

    AR logits ~ N(0, std^2); the draft head approximates them:
    draft_logits = ar_logits + N(0, draft_noise^2) (draft_noise = 0 gives
    equal heads).  Draft tokens are samples of softmax(draft_logits / T),
    drawn as argmax(draft_logits / T + Gumbel noise); u_accept [B, K] and
    u_resample [B] are U[0, 1) fp32.  Returns
    (ar_logits, draft_logits, draft_tokens int32, u_accept, u_resample).
    """
    ar, _ = make_logits(batch, block_k, vocab, seed=seed, workload=workload, std=std, device=device)
    noise = torch.randn((batch, block_k, vocab), generator=_gen(device, _seed(seed, workload, 0, "draft_logits")),
                        device=device, dtype=torch.float32)
    dr = ar + noise.mul_(draft_noise)
    u = torch.rand((batch, block_k, vocab), generator=_gen(device, _seed(seed, workload, 0, "gumbel")),
                   device=device, dtype=torch.float64).clamp_(min=1e-300)
    gumbel = -torch.log(-torch.log(u))
    drafts = torch.argmax(dr.double() / temperature + gumbel, dim=-1).to(torch.int32)
    ua = torch.rand((batch, block_k), generator=_gen(device, _seed(seed, workload, 0, "u_accept")),
                    device=device, dtype=torch.float32)
    ur = torch.rand((batch,), generator=_gen(device, _seed(seed, workload, 0, "u_resample")),
                    device=device, dtype=torch.float32)
    return ar, dr, drafts, ua, ur


QWEN3_8B_HIDDEN = 4096


def make_lm_head_inputs(rows, hidden, vocab, seed=0, workload="", planted=False, device="cpu"):
    """Final hidden states [rows, hidden] and an LM-head weight [vocab, hidden],
    both bf16.

    Default: hidden ~ N(0, 1), weight ~ N(0, (3 / sqrt(hidden))^2), so logits
    have a standard deviation of about 3.  With `planted`, weight rows are
    random +-1 and hidden row m is a copy of weight row targets[m] (drawn
    uniformly): every logit is an integer of magnitude <= hidden (exact in
    fp32 and bf16 products) and, the rows being distinct, targets[m] is the
    unique maximum by Cauchy-Schwarz.  Returns (hidden, weight, targets or
    None); targets is int32 [rows].
    """
    gen = _gen(device, _seed(seed, workload, 0, "lm_weight"))
    if not planted:
        w = torch.randn((vocab, hidden), generator=gen, device=device, dtype=torch.float32)
        w = w.mul_(3.0 / math.sqrt(hidden)).to(torch.bfloat16)
        h = torch.randn((rows, hidden), generator=_gen(device, _seed(seed, workload, 0, "lm_hidden")),
                        device=device, dtype=torch.float32).to(torch.bfloat16)
        return h, w, None
    bits = torch.randint(0, 2, (vocab, hidden), generator=gen, device=device, dtype=torch.int8)
    w = (bits.to(torch.bfloat16) * 2 - 1).to(torch.bfloat16)
    t = torch.randint(0, vocab, (rows,), generator=_gen(device, _seed(seed, workload, 0, "lm_targets")),
                      device=device, dtype=torch.int64)
    h = w[t].clone()
    return h, w, t.to(torch.int32)


def make_prefill_inputs(ctx_lens, prompt_lens, n_q_heads, n_kv_heads, head_dim, dtype=torch.bfloat16, seed=0,
                        device="cpu", shuffle=True):
    """A prompt of prompt_lens[b] rows after ctx_lens[b] cached tokens: q
    [B, S, Hq, D] and the prompt's k, v [B, S, Hkv, D] with S = max prompt
    rounded up to 32 (rows past the prompt are padding), a paged cache
    [num_pages, Hkv, 16, D] whose pages hold N(0, 1) values everywhere (the
    positions the prompt will occupy start with stale values), and a page
    table with room for L_b + S tokens.  Returns a dict of tensors plus
    `max_prompt` and `max_ctx_len`."""
    lens = np.asarray(ctx_lens, dtype=np.int32)
    plens = np.asarray(prompt_lens, dtype=np.int32)
    B = len(lens)
    mp = int(plens.max())
    S = (mp + 31) // 32 * 32
    table, num_pages = make_page_table(lens, S, PAGE_SIZE, shuffle, seed=seed + 77)
    s = lambda name: _seed(seed, "prefill", 0, name)
    return dict(q=_randn((B, S, n_q_heads, head_dim), dtype, device, s("q")),
                k=_randn((B, S, n_kv_heads, head_dim), dtype, device, s("k_blk")),
                v=_randn((B, S, n_kv_heads, head_dim), dtype, device, s("v_blk")),
                k_cache=_randn((num_pages, n_kv_heads, PAGE_SIZE, head_dim), dtype, device, s("k_cache")),
                v_cache=_randn((num_pages, n_kv_heads, PAGE_SIZE, head_dim), dtype, device, s("v_cache")),
                page_table=torch.from_numpy(table).to(device), ctx_lens=torch.from_numpy(lens).to(device),
                prompt_lens=torch.from_numpy(plens).to(device), max_prompt=mp, max_ctx_len=int(lens.max()))
