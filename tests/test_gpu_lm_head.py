"""Parity of the LM head with fused argmax (and the greedy accept fed by it)
through the C ABI with the fp64 CPU oracle.

Tokens are integers, so the bar is equality.  Two kinds of input:

* planted: weight rows +-1 and each hidden row a copy of its target row, so
  every logit is an integer of magnitude <= H (exact in fp32 whatever the
  summation order) and the target is the unique maximum (Cauchy-Schwarz).
  Tokens must equal the targets bit-exactly at every size, including the
  Qwen3-8B head (H 4096, V 151936); duplicated winner rows test the
  lowest-index tie rule exactly;
* random (N(0, 1) hidden, N(0, 9/H) weights): the kernel accumulates in
  fp32, the oracle in fp64.  A row whose fp64 gap between the two largest
  logits is within the accumulation bound 1e-5 * max_v sum_k |h_k w_vk| may
  resolve either way; such rows are checked to pick a logit within that bound
  of the maximum, and at most one per case may be excused.  max_logits is
  within the bound of the fp64 maximum.
"""

import numpy as np
import pytest
import torch

from diffusion_drafted_verification_amd import inputs as I
from oracle import orthrus_oracle as O

pytestmark = pytest.mark.gpu

REL = 1e-5


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def ob():
    from diffusion_drafted_verification_amd import orthrus
    return orthrus


def say(*a):
    print("[case]", *a, flush=True)


def oracle_logits(h, w, vslice=16384):
    """fp64 logits of the oracle, called on slices of the vocabulary (each
    logit is still one whole dot product) to bound host memory."""
    return np.concatenate([O.lm_head_logits(h, w[v0:v0 + vslice]) for v0 in range(0, w.shape[0], vslice)], axis=-1)


def abs_bound(h, w, vslice=16384):
    ha = np.abs(O._f64(h))
    return REL * np.max(np.concatenate([ha @ np.abs(O._f64(w[v0:v0 + vslice])).T
                                        for v0 in range(0, w.shape[0], vslice)], axis=-1), axis=-1)


def check_random(rows, H, V, seed, sample=None):
    """GPU argmax of all rows; the oracle checks every row, or the rows in
    `sample` (a row's token depends on that row alone)."""
    d = dev()
    h, w, _ = I.make_lm_head_inputs(rows, H, V, seed=seed)
    tok, mx = ob().lm_head_argmax(h.to(d), ob().PackedLmHead(w.to(d)), want_max=True)
    torch.cuda.synchronize()
    tok, mx = tok.cpu().numpy(), mx.cpu().numpy().astype(np.float64)
    if sample is not None:
        tok, mx, h = tok[sample], mx[sample], h[sample]
    lg = oracle_logits(h, w)
    ref = O.greedy_argmax(lg)
    eb = abs_bound(h, w)
    top = lg.max(axis=-1)
    assert np.all(np.abs(mx - top) <= eb), (np.abs(mx - top).max(), eb.min())
    bad = np.flatnonzero(tok != ref)
    for m in bad:
        assert 0 <= tok[m] < V
        assert lg[m, tok[m]] >= top[m] - 2 * eb[m], (m, tok[m], ref[m], lg[m, tok[m]], top[m])
    assert len(bad) <= 1, bad
    return tok


@pytest.mark.parametrize("rows,H,V", [(1, 256, 1000), (7, 512, 5003), (32, 1024, 20000), (33, 256, 777),
                                      (64, 2048, 10007), (100, 512, 3001), (130, 256, 4099), (257, 512, 2000),
                                      (600, 256, 1500)])
def test_lm_head_random_vs_oracle(rows, H, V):
    """Row counts 1..600 cover every kernel and row grouping: one 32-row
    group, one 64-row group, the many-row kernel's 128 x 128 tiles (100
    rows), 256 x 256 tiles in one row group (130 rows) and in two (257 rows:
    a one-row second group), and three 256-row groups with ordinary weight
    loads (600 rows); vocabularies from 777 to 20000 cover ragged 128- and
    256-row tiles."""
    say("lm_head random", rows, H, V)
    check_random(rows, H, V, seed=rows + V)


def test_lm_head_qwen3_8b_random():
    say("lm_head qwen3-8b random")
    check_random(32, I.QWEN3_8B_HIDDEN, I.QWEN3_VOCAB, seed=1)


@pytest.mark.parametrize("rows", [128, 512])
def test_lm_head_qwen3_8b_random_wide_rows_sampled(rows):
    """The benchmark's B4 and B16 row counts at the Qwen3-8B head (the
    many-row kernel: 128 rows in one work-group; 512 rows in two 256-row
    groups): the oracle checks rows on both sides of 32-row accumulator-tile
    boundaries (every 64 rows at 512, including the groups' boundary at 256)
    and the last row."""
    say("lm_head qwen3-8b random wide", rows)
    step = 32 if rows <= 128 else 64
    sample = sorted({0} | {m for k in range(step, rows, step) for m in (k - 1, k)} | {rows - 1})
    check_random(rows, I.QWEN3_8B_HIDDEN, I.QWEN3_VOCAB, seed=rows, sample=sample)


@pytest.mark.parametrize("rows", [1, 32, 64, 96, 512, 1100])
def test_lm_head_planted_qwen3_8b(rows):
    """Planted targets at the Qwen3-8B head, bit-exact; the maximum is H."""
    say("lm_head planted", rows)
    d = dev()
    h, w, t = I.make_lm_head_inputs(rows, I.QWEN3_8B_HIDDEN, I.QWEN3_VOCAB, seed=rows, planted=True, device=d)
    tok, mx = ob().lm_head_argmax(h, ob().PackedLmHead(w), want_max=True)
    torch.cuda.synchronize()
    assert torch.equal(tok, t)
    assert torch.all(mx == float(I.QWEN3_8B_HIDDEN))


def test_lm_head_planted_ties_resolve_to_lowest_index():
    """A copy of the winner row placed before it (in another tile, in the
    same 128-row tile, in the same 32-row wave slice, in the other lane half
    of the same accumulator) or after it: the token is the lower index of the
    pair, exactly, and the maximum is H."""
    say("lm_head ties")
    d = dev()
    H, V = 1024, 10000
    _, w, _ = I.make_lm_head_inputs(1, H, V, seed=5, planted=True, device=d)
    cases = [(5000, 17), (5000, 4990), (5000, 4997), (5000, 4996), (5000, 6000), (9999, 9998), (130, 129),
             (0, 9999)]
    for winner, copy in cases:
        wi = w.clone()
        wi[copy] = w[winner]
        h = w[winner:winner + 1].clone()
        tok, mx = ob().lm_head_argmax(h, ob().PackedLmHead(wi), want_max=True)
        torch.cuda.synchronize()
        assert tok.item() == min(winner, copy) and mx.item() == float(H), (winner, copy, tok.item())


@pytest.mark.parametrize("rows", [96, 200, 300])
def test_lm_head_planted_ties_many_rows(rows):
    """The same ties with more than 64 hidden rows, in each tiling of the
    many-row kernel: 96 rows (128-row key tiles, one weight slice per wave),
    200 rows (256-row key tiles, two slices per wave, four vocabulary parts
    merged in LDS) and 300 rows (256-row key tiles, four slices per wave, two
    parts; two row groups).  Copies in the same 32-row slice, in the other
    lane half, in another slice of the same wave, in another vocabulary part
    of the same tile, and in another tile, before or after the winner.  Every
    row must give the lower index of the pair, exactly."""
    say("lm_head ties, many rows", rows)
    d = dev()
    H, V = 1024, 10000
    _, w, _ = I.make_lm_head_inputs(1, H, V, seed=6, planted=True, device=d)
    # 128-row tiles: 5000 and 5030 sit in different waves' slices of one
    # tile.  256-row tiles (4864 .. 5119): 5000 (slice 4) and 5030 (slice 5)
    # share a wave; 4990 (slice 3) is in another vocabulary part; 5100
    # (slice 7) shares the wave at four slices per wave and not at two;
    # 4863 and 5200 are in the neighbouring tiles
    cases = [(5030, 5000), (5000, 5030), (5000, 4997), (5000, 4990), (5000, 5100), (5000, 4863), (5000, 5200),
             (9999, 9998), (300, 44)]
    for winner, copy in cases:
        wi = w.clone()
        wi[copy] = w[winner]
        h = w[winner:winner + 1].repeat(rows, 1).contiguous()
        tok, mx = ob().lm_head_argmax(h, ob().PackedLmHead(wi), want_max=True)
        torch.cuda.synchronize()
        assert torch.all(tok == min(winner, copy)) and torch.all(mx == float(H)), (winner, copy, tok.unique())


def test_lm_head_greedy_accept_planted():
    """The AR view's hidden states planted at known greedy tokens; drafts
    agree on a geometric prefix: accept_len, next_token and ar_tokens equal
    the planted values and the oracle's."""
    say("lm_head accept planted")
    d = dev()
    B, K, H, V = 4, 32, 2048, 30011
    h, w, t = I.make_lm_head_inputs(B * K, H, V, seed=9, planted=True, device=d)
    t = t.view(B, K).cpu()
    pre = np.array([0, 11, 32, 5])
    drafts = I.make_drafts(t, pre, V, seed=9).to(d)
    acc, nxt, g = ob().lm_head_greedy_accept(h.view(B, K, H), ob().PackedLmHead(w), drafts)
    torch.cuda.synchronize()
    assert torch.equal(g.cpu(), t) and acc.cpu().tolist() == pre.tolist()
    ra, rn, rg = O.lm_head_greedy_accept(h.view(B, K, H).cpu(), w.cpu(), drafts.cpu())
    assert np.array_equal(acc.cpu().numpy(), ra) and np.array_equal(nxt.cpu().numpy(), rn)
    assert np.array_equal(g.cpu().numpy(), rg)


def test_lm_head_greedy_accept_matches_argmax_then_accept():
    """At the Qwen3-8B head with random inputs, the fused accept equals
    orthrus_lm_head_argmax followed by the same prefix rule (on the GPU's own
    tokens: the fused path must take identical decisions)."""
    say("lm_head accept random")
    d = dev()
    B, K = 2, 32
    h, w, _ = I.make_lm_head_inputs(B * K, I.QWEN3_8B_HIDDEN, I.QWEN3_VOCAB, seed=3, device=d)
    head = ob().PackedLmHead(w)
    tok, _ = ob().lm_head_argmax(h, head)
    g0 = tok.view(B, K).cpu()
    drafts = I.make_drafts(g0, np.array([7, 32]), I.QWEN3_VOCAB, seed=3).to(d)
    acc, nxt, g = ob().lm_head_greedy_accept(h.view(B, K, -1), head, drafts)
    torch.cuda.synchronize()
    assert torch.equal(g.cpu(), g0) and acc.cpu().tolist() == [7, 32]
    assert nxt.cpu().tolist() == [g0[0, 7].item(), g0[1, 31].item()]


def test_lm_head_workspace_reuse_and_determinism():
    say("lm_head workspace reuse")
    d = dev()
    ws = torch.full((ob().lib().orthrus_lm_head_workspace_bytes(130, 512, 20000),), 0x5A, dtype=torch.uint8,
                    device=d)
    for rows, H, V, s in [(130, 512, 20000, 1), (3, 256, 900, 2), (64, 1024, 20000, 3)]:
        h, w, _ = I.make_lm_head_inputs(rows, H, V, seed=s, device=d)
        head = ob().PackedLmHead(w)
        a, am = ob().lm_head_argmax(h, head, want_max=True, ws=ws)
        b, bm = ob().lm_head_argmax(h, head, want_max=True)
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(am, bm)


@pytest.mark.parametrize("V,H", [(1, 256), (33, 256), (1000, 512), (4099, 1024)])
def test_lm_head_pack_layout(V, H):
    """The packed weight is bit-exactly the layout the header defines: tile t,
    k-step s, lane l hold weight[32 t + l % 32][16 s + 8 (l / 32) + j], zero
    past the vocabulary (built here with numpy reshapes)."""
    say("lm_head pack", V, H)
    d = dev()
    _, w, _ = I.make_lm_head_inputs(1, H, V, seed=V, device=d)
    got = ob().PackedLmHead(w).packed.cpu().view(torch.int16).numpy()
    T = (V + 31) // 32
    wp = np.zeros((T * 32, H), dtype=np.int16)
    wp[:V] = w.cpu().view(torch.int16).numpy()
    want = wp.reshape(T, 32, H // 16, 2, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
    assert got.shape == want.shape and np.array_equal(got, want)
