"""Parity of the multi-step denoising update fused into the LM head
(orthrus_lm_head_denoise_step) through the C ABI with the fp64 CPU oracle.

Tokens and masks are integers: the bar is equality.  The kernel takes its
decisions in fp32 and the oracle in fp64, so
* a row whose fp64 top-2 logit gap is within the fp32 accumulation bound
  (1e-5 * max sum |h w|) may pick either token; it must pick a logit within
  the bound of the maximum;
* confidences are within 1e-4 (relative) of the oracle's;
* the unmasked set may differ only where the n-th and (n+1)-th confidences
  of the masked rows are within 1e-4 (relative); it must then still be
  min(n, #masked) masked rows, each at least as confident as every row left
  masked, to that margin.
Each test bounds how many rows or sequences are excused.
"""

import numpy as np
import pytest
import torch

from diffusion_drafted_verification_amd import inputs as I
from oracle import orthrus_oracle as O

pytestmark = pytest.mark.gpu

REL = 1e-5
CREL = 1e-4


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def ob():
    from diffusion_drafted_verification_amd import orthrus
    return orthrus


def say(*a):
    print("[case]", *a, flush=True)


def masks_and_counts(B, K, seed):
    rng = np.random.default_rng(seed)
    masked = (rng.random((B, K)) < 0.75).astype(np.uint8)
    n = rng.integers(0, K + 3, size=B).astype(np.int32)
    return torch.from_numpy(masked), torch.from_numpy(n)


def check_step(h, w, masked, n, head=None, max_excused=1, seqs=None):
    """GPU step over every sequence; the oracle checks every sequence, or
    those in `seqs` (a sequence's tokens, confidences and unmasking depend
    on its own rows alone)."""
    d = dev()
    head = head or ob().PackedLmHead(w.to(d))
    tok, conf, nm = ob().lm_head_denoise_step(h.to(d), head, masked.to(d), n.to(d))
    torch.cuda.synchronize()
    tok, conf, nm = tok.cpu().numpy(), conf.cpu().numpy().astype(np.float64), nm.cpu().numpy().astype(bool)
    if seqs is not None:
        tok, conf, nm, h, masked, n = tok[seqs], conf[seqs], nm[seqs], h[seqs], masked[seqs], n[seqs]
    B, K, H = h.shape
    lg = np.concatenate([O.lm_head_logits(h, w[v0:v0 + 16384]) for v0 in range(0, w.shape[0], 16384)], axis=-1)
    rtok, rconf = O.denoise_confidence(lg)
    rnm = O.denoise_select(rconf, masked.numpy().astype(bool), n.numpy())
    # tokens
    eb = REL * np.max(np.concatenate([np.abs(O._f64(h)) @ np.abs(O._f64(w[v0:v0 + 16384])).T
                                      for v0 in range(0, w.shape[0], 16384)], axis=-1), axis=-1)
    top = lg.max(axis=-1)
    bad = np.argwhere(tok != rtok)
    for b, i in bad:
        assert lg[b, i, tok[b, i]] >= top[b, i] - 2 * eb[b, i]
    assert len(bad) <= max_excused
    # confidences
    assert np.all(np.abs(conf - rconf) <= CREL * rconf), np.abs(conf / rconf - 1).max()
    # selection
    mk = masked.numpy().astype(bool)
    excused = 0
    for b in range(B):
        if np.array_equal(nm[b], rnm[b]):
            continue
        excused += 1
        un = mk[b] & ~nm[b]
        assert not (nm[b] & ~mk[b]).any()
        assert un.sum() == min(int(n[b]), int(mk[b].sum()))
        left = mk[b] & nm[b]
        if un.any() and left.any():
            assert rconf[b][un].min() >= rconf[b][left].max() * (1 - 2 * CREL)
    assert excused <= max_excused
    return tok, conf, nm


@pytest.mark.parametrize("B,K,H,V", [(1, 32, 256, 1000), (4, 32, 1024, 20011), (3, 7, 512, 5000), (2, 1, 256, 300),
                                     (7, 32, 512, 5000), (10, 32, 256, 3001)])
def test_denoise_random_vs_oracle(B, K, H, V):
    """Up to 32 rows (the tile kernel), 128 rows (the many-row kernel's
    128 x 128 tiles), 224 rows (256 x 256 tiles, four vocabulary parts merge
    their softmax statistics in LDS) and 320 rows (two 256-row groups, two
    parts), ragged vocabularies."""
    say("denoise random", B, K, H, V)
    h, w, _ = I.make_lm_head_inputs(B * K, H, V, seed=B * K + V)
    masked, n = masks_and_counts(B, K, seed=V)
    check_step(h.view(B, K, H), w, masked, n)


def test_denoise_qwen3_8b_head():
    say("denoise qwen3-8b")
    B, K = 2, 32
    h, w, _ = I.make_lm_head_inputs(B * K, I.QWEN3_8B_HIDDEN, I.QWEN3_VOCAB, seed=7)
    masked, n = masks_and_counts(B, K, seed=7)
    check_step(h.view(B, K, -1), w, masked, n)


def test_denoise_qwen3_8b_head_b16_sampled():
    """The benchmark's B16 rows (512: two 256-row groups of the many-row
    kernel) at the Qwen3-8B head; the oracle checks sequences at both ends
    and on both sides of the groups' boundary at row 256."""
    say("denoise qwen3-8b B16 sampled")
    B, K = 16, 32
    h, w, _ = I.make_lm_head_inputs(B * K, I.QWEN3_8B_HIDDEN, I.QWEN3_VOCAB, seed=16)
    masked, n = masks_and_counts(B, K, seed=16)
    check_step(h.view(B, K, -1), w, masked, n, seqs=[0, 1, 7, 8, 15])


def test_denoise_planted_sharpness_orders_the_unmasking():
    """Planted +-1 weights with hidden row i = s_i * weight[t_i]: the token is
    t_i exactly, and larger scales s_i give sharper softmaxes; the rows are
    unmasked in the oracle's confidence order, exactly (the scales are far
    apart)."""
    say("denoise planted")
    d = dev()
    B, K, H, V = 2, 32, 512, 4096
    _, w, _ = I.make_lm_head_inputs(1, H, V, seed=11, planted=True)
    g = torch.Generator().manual_seed(11)
    t = torch.randint(0, V, (B, K), generator=g)
    scales = torch.tensor([2.0 ** (-6 + (7 * i) % 9) for i in range(B * K)]).view(B, K, 1)   # powers of two: exact
    h = (w[t.view(-1)].float().view(B, K, H) * scales / 64).to(torch.bfloat16)
    masked = torch.ones((B, K), dtype=torch.uint8)
    n = torch.tensor([5, 20], dtype=torch.int32)
    tok, conf, nm = check_step(h, w, masked, n, max_excused=0)
    assert np.array_equal(tok, t.numpy())


def test_denoise_loop_unmasks_every_position():
    """T = 4 steps with a linear schedule (8 per step) on fresh hidden states
    each step, the new mask fed back in place: every position is unmasked at
    the end, and each step unmasks exactly its count."""
    say("denoise loop")
    d = dev()
    B, K, H, V = 3, 32, 1024, 20000
    _, w, _ = I.make_lm_head_inputs(1, H, V, seed=13, device=d)
    head = ob().PackedLmHead(w)
    masked = torch.ones((B, K), dtype=torch.uint8, device=d)
    n = torch.full((B,), 8, dtype=torch.int32, device=d)
    for step in range(4):
        h, _, _ = I.make_lm_head_inputs(B * K, H, 1, seed=100 + step, device=d)
        before = int(masked.sum())
        _, _, masked = ob().lm_head_denoise_step(h.view(B, K, H), head, masked, n, new_masked=masked)
        torch.cuda.synchronize()
        assert before - int(masked.sum()) == 8 * B
    assert int(masked.sum()) == 0
