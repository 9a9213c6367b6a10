"""The entry point that allocates nothing (orthrus_block_attn_noalloc) gives
the same bits as orthrus_block_attn with a caller workspace, on two calls in
a row (the second one smaller, so it runs on the scratch array the first one
left behind), and rejects a call whose partials would not fit that array."""

import ctypes

import pytest
import torch

from diffusion_drafted_verification_amd import inputs as I

pytestmark = pytest.mark.gpu


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def test_noalloc_matches_workspace_entry_point():
    d = dev()
    from diffusion_drafted_verification_amd import orthrus as ob
    cases = [("qwen3_8b_8k B1 ctx 8192 (26 splits)", "qwen3_8b_8k", dict(ctx_lens=[8192]), 0, 8192),
             ("qwen3_8b_8k B3 ragged, split 256", "qwen3_8b_8k", dict(batch=3, ctx_lens=[3001, 17, 1200]), 256, 3001),
             ("qwen3_8b_ragged16, balanced split (two rounds)", "qwen3_8b_ragged16", {}, ob.SPLIT_BALANCED, None)]
    for name, workload, kw, split, mx in cases:
        x = I.make_attn_inputs(workload, device=d, **kw)
        mx = x.max_ctx_len if mx is None else mx
        desc = ob.make_desc(x.q, x.k_cache, x.page_table, mx, None, split)
        need = ob.block_attn_workspace_bytes(desc)
        assert 0 < need <= ob.STATIC_SCRATCH_BYTES, need
        for mode in (ob.DIFF_BIDIR, ob.AR_CAUSAL):
            print("[case] no-alloc entry point:", name, "mode", mode, "workspace bytes", need, flush=True)
            ws = torch.full((need,), 0x3c, dtype=torch.uint8, device=d)
            ref = ob.block_attn(x.q, x.k_cache, x.v_cache, x.k_blk, x.v_blk, x.page_table, x.ctx_lens, mode,
                                max_ctx_len=mx, split_tokens=split, ws=ws)
            out = torch.full_like(x.q, 7.0)
            ob.block_attn_noalloc(x.q, x.k_cache, x.v_cache, x.k_blk, x.v_blk, x.page_table, x.ctx_lens, mode, out,
                                  max_ctx_len=mx, split_tokens=split)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), (name, mode)


def test_noalloc_rejects_oversized_calls():
    d = dev()
    from diffusion_drafted_verification_amd import orthrus as ob
    x = I.make_attn_inputs("qwen3_8b_8k", device=d, batch=4, ctx_lens=[8192] * 4)
    desc = ob.make_desc(x.q, x.k_cache, x.page_table, 8192, None, 64)     # 128 splits per sequence
    assert ob.block_attn_workspace_bytes(desc) > ob.STATIC_SCRATCH_BYTES
    out = torch.empty_like(x.q)
    with pytest.raises(ob.OrthrusError, match="ERR_WORKSPACE"):
        ob.block_attn_noalloc(x.q, x.k_cache, x.v_cache, x.k_blk, x.v_blk, x.page_table, x.ctx_lens,
                              ob.AR_CAUSAL, out, max_ctx_len=8192, split_tokens=64)
