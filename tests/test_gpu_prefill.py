"""Parity of the prompt prefill (orthrus_prefill: cache write plus causal
attention over the paged cache) through the C ABI with the fp64 CPU oracle.

Bars: the cache after the call is bit-exactly the oracle's kv_write (the
prompt rows at L + r, every other byte unchanged) and new_ctx_lens is exact;
attention rows i < prompt_len are within 2e-2 * max|V| of the oracle (the
stated tolerance) and within 2e-2 of the largest |oracle output| of each
(sequence, head) slice; padding rows are not compared.
"""

import numpy as np
import pytest
import torch

from diffusion_drafted_verification_amd import inputs as I
from oracle import orthrus_oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-2


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def ob():
    from diffusion_drafted_verification_amd import orthrus
    return orthrus


def say(*a):
    print("[case]", *a, flush=True)


def run_prefill(x, split=0, heads=None, rows=None):
    d = dev()
    g = {k: (v.to(d) if hasattr(v, "to") else v) for k, v in x.items()}
    kc0, vc0 = x["k_cache"].clone(), x["v_cache"].clone()
    out, nl = ob().prefill(g["q"], g["k"], g["v"], g["k_cache"], g["v_cache"], g["page_table"], g["ctx_lens"],
                           g["prompt_lens"], x["max_prompt"], max_ctx_len=x["max_ctx_len"], split_tokens=split)
    torch.cuda.synchronize()
    # cache writes: bit-exact
    rk, rv, rl = O.kv_write(kc0, vc0, x["k"], x["v"], x["page_table"], x["ctx_lens"], x["prompt_lens"])
    assert np.array_equal(g["k_cache"].cpu().view(torch.int16 if kc0.dtype == torch.bfloat16 else torch.int32)
                          .numpy(), rk.view(np.int16) if kc0.dtype == torch.bfloat16 else rk.view(np.int32))
    assert np.array_equal(g["v_cache"].cpu().view(torch.int16 if vc0.dtype == torch.bfloat16 else torch.int32)
                          .numpy(), rv.view(np.int16) if vc0.dtype == torch.bfloat16 else rv.view(np.int32))
    assert np.array_equal(nl.cpu().numpy(), rl)
    # attention: the oracle reads the cache as it was before the prompt
    ref = O.prefill_attn(x["q"], kc0, vc0, x["k"], x["v"], x["page_table"], x["ctx_lens"], x["prompt_lens"],
                         heads=heads)
    got = out.float().cpu().numpy().astype(np.float64)
    vmax = max(float(vc0.float().abs().max()), float(x["v"].float().abs().max()))
    B, S, Hq, D = ref.shape
    plens = x["prompt_lens"].numpy()
    for b in range(B):
        for h in (range(Hq) if heads is None else heads):
            n = int(plens[b])
            sel = slice(0, n) if rows is None else [r for r in rows if r < n]
            r_, g_ = ref[b, sel, h], got[b, sel, h]
            if np.size(r_) == 0:
                continue
            assert np.isfinite(g_).all()
            err = np.abs(g_ - r_).max()
            assert err <= TOL * vmax, (b, h, err, vmax)
            assert err <= TOL * np.abs(r_).max(), (b, h, err, np.abs(r_).max())
    return out


@pytest.mark.parametrize("L,n", [(0, 1), (0, 31), (0, 32), (100, 33), (5, 64), (1000, 100), (17, 257)])
def test_prefill_lengths(L, n):
    """Prompt lengths around the 32-row chunk, with and without context."""
    say("prefill", L, n)
    x = I.make_prefill_inputs([L], [n], 8, 2, 128, seed=L + n)
    run_prefill(x)


def test_prefill_ragged_batch():
    """Sequences with different contexts and prompt lengths in one call;
    padding chunks of the shorter prompts are skipped."""
    say("prefill ragged")
    x = I.make_prefill_inputs([0, 700, 33, 4096], [100, 257, 1, 64], 32, 8, 128, seed=3)
    run_prefill(x, heads=[0, 7, 13, 31])


@pytest.mark.parametrize("G,D,dtype", [(1, 64, torch.bfloat16), (2, 128, torch.bfloat16), (4, 64, torch.bfloat16),
                                       (8, 128, torch.bfloat16), (4, 128, torch.float32), (1, 64, torch.float32)])
def test_prefill_group_sizes_head_dims_dtypes(G, D, dtype):
    say("prefill G D dtype", G, D, dtype)
    x = I.make_prefill_inputs([300, 0], [77, 130], 4 * G if G < 8 else 16, 4 if G < 8 else 2, D, dtype=dtype,
                              seed=G * D)
    run_prefill(x)


@pytest.mark.parametrize("split", [64, 256, 1024])
def test_prefill_split_lengths(split):
    say("prefill split", split)
    x = I.make_prefill_inputs([2000], [200], 16, 4, 128, seed=split)
    run_prefill(x, split=split)


def run_prefill_pairs(x, split):
    """run_prefill on a shape that takes the pair kernel (two chunks per
    attention work-group)."""
    assert ob().prefill_chunks_per_workgroup(x["q"], x["k_cache"], x["page_table"], x["max_prompt"],
                                             max_ctx_len=x["max_ctx_len"], split_tokens=split) == 2
    return run_prefill(x, split=split)


@pytest.mark.parametrize("split,G,D", [(64, 4, 128), (128, 4, 128), (64, 2, 128), (128, 1, 128), (64, 4, 64)])
def test_prefill_split_boundary_at_chunk_pair(split, G, D):
    """Contexts L_b + 64 j that are multiples of the split: chunk 2j's last
    split ends at its block while chunk 2j + 1 (32 positions more context)
    needs one more split, so a work-group serving both chunks computes one
    chunk's split alone or masks the other's range.  Four sequences and 8 KV
    heads make the grid large enough for the pair kernel."""
    say("prefill pairs, split boundary", split, G, D)
    x = I.make_prefill_inputs([0, split, 2 * split, 3 * split], [200, 200, 171, 200], 8 * G, 8, D,
                              seed=split + G + D)
    run_prefill_pairs(x, split)


def test_prefill_pairs_ragged_batch_short_splits():
    """Odd chunk counts in a batch (no chunk may pair with the next
    sequence's first chunk) with many splits per chunk, on the pair kernel."""
    say("prefill pairs, ragged short splits")
    x = I.make_prefill_inputs([0, 700, 33], [100, 257, 1], 16, 8, 128, seed=13)
    run_prefill_pairs(x, 64)


def test_prefill_qwen3_8b_2k_prompt_sampled():
    """A 2048-token prompt at the Qwen3-8B attention shape after 4096 cached
    tokens, compared on sampled heads and rows (the oracle is slow)."""
    say("prefill qwen3-8b 2k")
    x = I.make_prefill_inputs([4096], [2048], 32, 8, 128, seed=11)
    run_prefill(x, heads=[0, 9, 31], rows=[0, 1, 31, 32, 33, 500, 1023, 1024, 2047])


@pytest.mark.parametrize("L,S", [(8192, 2048), (0, 8192)])
def test_prefill_qwen3_8b_benchmark_shapes_sampled(L, S):
    """The two larger prompts the benchmark times at the Qwen3-8B attention
    shape (a 2048-token prompt after 8192 cached tokens; an 8192-token prompt
    on an empty cache), in the launch configuration it times (automatic
    split), compared on sampled heads and rows."""
    say("prefill qwen3-8b benchmark shape", L, S)
    x = I.make_prefill_inputs([L], [S], 32, 8, 128, seed=L + S)
    assert ob().prefill_chunks_per_workgroup(x["q"], x["k_cache"], x["page_table"], x["max_prompt"],
                                             max_ctx_len=x["max_ctx_len"]) == 2
    run_prefill(x, heads=[0, 14, 31], rows=[0, 31, 32, S // 2 - 1, S // 2, S - 33, S - 1])


def test_prefill_in_two_calls_equals_one():
    """Chunked prefill through the ABI: the prompt's second part after the
    first part's call (its rows now cached, new_ctx_lens as the context)
    matches the one-call output within the attention tolerance, and both
    leave the same cache bytes."""
    say("prefill two calls")
    d = dev()
    x = I.make_prefill_inputs([50], [96], 8, 2, 128, seed=5, device=d)
    k1, v1 = x["k_cache"].clone(), x["v_cache"].clone()
    whole, nl = ob().prefill(x["q"], x["k"], x["v"], k1, v1, x["page_table"], x["ctx_lens"], x["prompt_lens"], 96,
                             max_ctx_len=50)
    k2, v2 = x["k_cache"].clone(), x["v_cache"].clone()
    p1 = torch.tensor([40], dtype=torch.int32, device=d)
    _, mid = ob().prefill(x["q"][:, :64].contiguous(), x["k"][:, :64].contiguous(), x["v"][:, :64].contiguous(),
                          k2, v2, x["page_table"], x["ctx_lens"], p1, 40, max_ctx_len=50)
    p2 = torch.tensor([56], dtype=torch.int32, device=d)
    pad = lambda t: torch.cat([t[:, 40:96], torch.zeros_like(t[:, :8])], dim=1).contiguous()   # 56 -> 64 rows
    part2, nl2 = ob().prefill(pad(x["q"]), pad(x["k"]), pad(x["v"]), k2, v2, x["page_table"], mid, p2, 56,
                              max_ctx_len=90)
    torch.cuda.synchronize()
    assert torch.equal(k1, k2) and torch.equal(v1, v2) and torch.equal(nl, nl2)
    vmax = max(float(x["v_cache"].float().abs().max()), float(x["v"].float().abs().max()))
    assert (whole[:, 40:96].float() - part2[:, :56].float()).abs().max().item() <= TOL * vmax
