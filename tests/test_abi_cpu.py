"""The C-ABI library loads, exports every entry point the header declares,
and rejects invalid arguments on the host (no GPU needed: every call here
fails validation before any HIP call)."""

import ctypes
import os
import re

import pytest

from diffusion_drafted_verification_amd import orthrus as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "orthrus.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="library not built")


def declared_entry_points():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(orthrus_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_entry_points()
    assert len(names) == 24
    assert set(names) == set(B.SIGNATURES)
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_one_hip_runtime_in_process():
    B.lib()
    maps = open("/proc/self/maps").read()
    runtimes = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(runtimes) == 1, runtimes


def test_version_and_status_strings():
    lib = B.lib()
    assert lib.orthrus_abi_version() == 1
    for s in range(6):
        assert lib.orthrus_status_str(s)


def good_desc(**kw):
    d = dict(batch=1, block_k=32, n_q_heads=32, n_kv_heads=8, head_dim=128, page_size=16,
             max_pages_per_seq=514, num_pages=514, max_ctx_len=8192, dtype=0, softmax_scale=0.0, split_tokens=0)
    d.update(kw)
    return B.AttnDesc(**d)


FAKE = ctypes.c_void_p(4096)   # never dereferenced: validation fails first


def attn(desc, ws=None, ws_bytes=0, mode=0, null_q=False):
    return B.lib().orthrus_block_attn(None if null_q else FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, mode, FAKE,
                                      ctypes.byref(desc), ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(block_k=0), 2), (dict(block_k=33), 2), (dict(batch=0), 2), (dict(n_q_heads=12), 2),
    (dict(n_q_heads=48), 3), (dict(head_dim=96), 3), (dict(page_size=32), 3), (dict(dtype=7), 3),
    (dict(max_ctx_len=8193 - 32 + 16 * 514), 2), (dict(split_tokens=100), 2), (dict(split_tokens=16384), 2),
    (dict(split_tokens=-2), 2),
    (dict(num_pages=0), 2), (dict(max_ctx_len=-1), 2)])
def test_block_attn_rejects_bad_descriptors(kw, status):
    assert attn(good_desc(**kw)) == status
    assert B.lib().orthrus_block_attn_workspace_bytes(ctypes.byref(good_desc(**kw))) == 0


def test_block_attn_rejects_null_mode_and_workspace():
    d = good_desc()
    assert attn(d, null_q=True) == 1
    need = B.lib().orthrus_block_attn_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert attn(d, mode=2, ws=FAKE, ws_bytes=need) == 2
    assert attn(d) == 4                                   # workspace missing
    assert attn(d, ws=FAKE, ws_bytes=need - 1) == 4       # too small
    assert attn(d, ws=ctypes.c_void_p(4100), ws_bytes=need) == 4   # misaligned


def test_prefill_chunks_per_workgroup():
    """The pair kernel (two 32-row chunks per work-group) runs where its grid
    fills two rounds of 256 work-groups: the Qwen3-8B 8192-token prompt (128
    pairs x 8 KV heads) and the 2048-token prompt after 8192 cached tokens (two
    splits), not the 2048-token prompt alone (one round); never for fp32 or
    G = 8 (no streaming kernel); 0 for an invalid shape."""
    f = lambda d, mp: B.lib().orthrus_prefill_chunks_per_workgroup(ctypes.byref(d), mp)
    pages = lambda n: dict(max_pages_per_seq=n, num_pages=n)
    assert f(good_desc(max_ctx_len=0, **pages(512)), 8192) == 2
    assert f(good_desc(max_ctx_len=0, **pages(128)), 2048) == 1
    assert f(good_desc(max_ctx_len=8192, **pages(640)), 2048) == 2
    assert f(good_desc(max_ctx_len=0, dtype=1, **pages(512)), 8192) == 1
    assert f(good_desc(max_ctx_len=0, n_q_heads=64, **pages(512)), 8192) == 1
    assert f(good_desc(max_ctx_len=0, **pages(512)), 0) == 0
    assert f(good_desc(max_ctx_len=0, split_tokens=B.SPLIT_BALANCED, **pages(512)), 8192) == 1


def test_split_and_workspace_arithmetic():
    lib = B.lib()
    d = good_desc()
    split = lib.orthrus_block_attn_split_tokens(ctypes.byref(d))
    assert split % 64 == 0 and 64 <= split <= 8192
    s_max = -(-8192 // split)           # splits partition the cached context
    rows = 1 * 32 * s_max * 32
    up = lambda x: -(-x // 256) * 256
    # bf16, 4 query heads per KV head: bf16 partials, then row stats
    bf16_bytes = up(rows * 128 * 2) + rows * 8
    assert lib.orthrus_block_attn_workspace_bytes(ctypes.byref(d)) == bf16_bytes
    # fp32 storage: fp32 partials and row stats
    d32 = good_desc(dtype=1)
    split32 = lib.orthrus_block_attn_split_tokens(ctypes.byref(d32))
    rows32 = 32 * -(-8192 // split32) * 32
    assert lib.orthrus_block_attn_workspace_bytes(ctypes.byref(d32)) == rows32 * 128 * 4 + rows32 * 8
    d1 = good_desc(split_tokens=8192, max_ctx_len=100)      # one split: no workspace
    assert lib.orthrus_block_attn_workspace_bytes(ctypes.byref(d1)) == 0


@pytest.mark.parametrize("batch,hq,hkv,max_ctx,split,units", [
    (2, 32, 8, 8192, 512, 64),      # 2 x 16 splits fill one 32-slot round per KV head; slots for two rounds
    (4, 32, 8, 8192, 1024, 64),
    (16, 32, 8, 8192, 4096, 64),
    (3, 32, 8, 8192, 832, 64),      # 3 x 10 splits fit one 32-slot round (a 768 split would need 33)
    (16, 32, 8, 16379, 8192, 64),   # the ragged batch's bound: its lengths pick the split on the device
    (16, 32, 8, 200000, 8192, 400),  # 25 splits of 8192 each: more than two rounds
    (64, 8, 2, 8192, 4096, 256)])
def test_balanced_split_plan(batch, hq, hkv, max_ctx, split, units):
    """Balanced split requested, several sequences, bf16 with Hq/Hkv <= 4:
    the split that a batch with every length at max_ctx gets (the smallest
    multiple of 64 in [320, 8192] giving at most ceil(256 / Hkv) work-groups
    per KV head), and partial slots for `units` work-groups per KV head: two
    rounds of ceil(256 / Hkv) (a poorly balanced batch may take the second),
    or every split of every sequence at the longest split if that is more."""
    lib = B.lib()
    pages = -(-(max_ctx + 32) // 16)
    d = good_desc(batch=batch, n_q_heads=hq, n_kv_heads=hkv, max_ctx_len=max_ctx, max_pages_per_seq=pages,
                  num_pages=pages, split_tokens=B.SPLIT_BALANCED)
    assert lib.orthrus_block_attn_split_tokens(ctypes.byref(d)) == split
    rows = hq * units * 32
    up = lambda x: -(-x // 256) * 256
    # bf16 partials, row statistics, then one (splits, first slot) pair per sequence
    assert lib.orthrus_block_attn_workspace_bytes(ctypes.byref(d)) == up(up(rows * 128 * 2) + rows * 8) + batch * 8


def test_fixed_split_outside_the_balanced_case():
    lib = B.lib()
    up = lambda x: -(-x // 256) * 256
    bal = B.SPLIT_BALANCED
    for kw, split in [(dict(batch=16, split_tokens=1024), 1024),   # explicit split
                      (dict(batch=16, split_tokens=0), 4096),      # automatic: 2 splits each, one round
                      (dict(batch=3, split_tokens=0), 832),        # 10 splits each (11 would need 33 slots)
                      (dict(batch=1, split_tokens=0), 320),        # the shortest automatic split
                      (dict(batch=16, split_tokens=bal, dtype=1), 4096),   # fp32: no balanced split
                      (dict(batch=1, split_tokens=bal), 320),      # one sequence
                      (dict(batch=65, n_q_heads=8, n_kv_heads=2, max_ctx_len=4096, split_tokens=bal), 4096),
                      (dict(batch=32, max_ctx_len=8192, split_tokens=bal), 8192),   # one split each
                      (dict(batch=4, max_ctx_len=1000000, max_pages_per_seq=62503, num_pages=62503), 8192)]:
        d = good_desc(**kw)
        assert lib.orthrus_block_attn_split_tokens(ctypes.byref(d)) == split
        s_max = -(-d.max_ctx_len // split)
        rows = d.batch * d.n_q_heads * s_max * 32
        want = 0 if s_max <= 1 else up(rows * 128 * (2 if d.dtype == 0 else 4)) + rows * 8
        assert lib.orthrus_block_attn_workspace_bytes(ctypes.byref(d)) == want


def test_accept_and_append_validation():
    lib = B.lib()
    assert lib.orthrus_greedy_accept(None, FAKE, FAKE, FAKE, None, 1, 32, 100, FAKE, 1 << 20, None) == 1
    assert lib.orthrus_greedy_accept(FAKE, FAKE, FAKE, FAKE, None, 1, 33, 100, FAKE, 1 << 20, None) == 2
    assert lib.orthrus_greedy_accept(FAKE, FAKE, FAKE, FAKE, None, 1, 32, 0, FAKE, 1 << 20, None) == 2
    need = lib.orthrus_greedy_accept_workspace_bytes(2, 32, 151936)
    # one 8-byte key per (row, chunk): 64 rows take 4096-logit chunks (38),
    # more rows 8192-logit ones (19)
    assert need == 64 * 38 * 8
    assert lib.orthrus_greedy_accept_workspace_bytes(16, 32, 151936) == 512 * 19 * 8
    assert lib.orthrus_greedy_accept_workspace_bytes(1, 32, 1024) == 32 * 1 * 8
    assert lib.orthrus_greedy_accept(FAKE, FAKE, FAKE, FAKE, None, 2, 32, 151936, FAKE, need - 1, None) == 4
    assert lib.orthrus_greedy_accept(FAKE, FAKE, FAKE, FAKE, None, 2, 32, 151936, None, need, None) == 4
    d = good_desc()
    assert lib.orthrus_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, ctypes.byref(d), None) == 1
    assert lib.orthrus_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                 ctypes.byref(good_desc(head_dim=80)), None) == 3
    assert lib.orthrus_kv_append_layers(FAKE, FAKE, FAKE, None, 36, FAKE, FAKE, FAKE, None, None,
                                        ctypes.byref(d), None) == 1
    assert lib.orthrus_kv_append_layers(FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None, None,
                                        ctypes.byref(d), None) == 2
    assert lib.orthrus_copy_probe(FAKE, FAKE, 17, None) == 2
    assert lib.orthrus_copy_probe(None, FAKE, 16, None) == 1
    assert lib.orthrus_read_probe(FAKE, 17, FAKE, 4 << 20, None) == 2
    assert lib.orthrus_read_probe(FAKE, 16, FAKE, (4 << 20) - 1, None) == 4
    assert lib.orthrus_read_probe(None, 16, FAKE, 4 << 20, None) == 1


def test_sample_accept_validation():
    lib = B.lib()
    args = lambda **kw: dict(dict(ar=FAKE, dr=FAKE, d=FAKE, ua=FAKE, ur=FAKE, t=0.7, acc=FAKE, nxt=FAKE, b=2,
                                   k=32, v=151936, ws=FAKE, wsb=1 << 20), **kw)

    def call(**kw):
        a = args(**kw)
        return lib.orthrus_sample_accept(a["ar"], a["dr"], a["d"], a["ua"], a["ur"], a["t"], a["acc"], a["nxt"],
                                         a["b"], a["k"], a["v"], a["ws"], a["wsb"], None)

    for ptr in ("ar", "dr", "d", "ua", "ur", "acc", "nxt"):
        assert call(**{ptr: None}) == 1, ptr
    assert call(k=33) == 2 and call(k=0) == 2 and call(v=0) == 2 and call(b=0) == 2
    for t in (0.0, -1.0, float("inf"), float("nan"), 1e-45):   # 1e-45: log2(e) / T overflows
        assert call(t=t) == 2, t
    # per (row, chunk) one 16-byte pair for each head pair; per sequence the
    # row normalisers, the decision and one residual sum per chunk (each
    # region rounded up to 256 bytes)
    up = lambda x: -(-x // 256) * 256
    need = lib.orthrus_sample_accept_workspace_bytes(2, 32, 151936)
    assert need == up(64 * 38 * 16) + up(2 * 16) + up(2 * 4) + up(2 * 38 * 4)   # 4096-logit chunks
    need16 = lib.orthrus_sample_accept_workspace_bytes(16, 32, 151936)          # 8192-logit chunks
    assert need16 == up(512 * 19 * 16) + up(16 * 16) + up(16 * 4) + up(16 * 19 * 4)
    assert lib.orthrus_sample_accept_workspace_bytes(1, 33, 100) == 0
    assert call(wsb=need - 1) == 4
    assert call(ws=None, wsb=need) == 4
    assert call(ws=ctypes.c_void_p(4096 + 8), wsb=need) == 4   # 16-byte alignment


def test_lm_head_validation():
    lib = B.lib()
    A16 = ctypes.c_void_p(4096 * 16)
    ok = dict(h=A16, w=A16, tok=FAKE, rows=32, H=4096, V=151936, ws=FAKE, wsb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.orthrus_lm_head_argmax(a["h"], a["w"], a["tok"], None, a["rows"], a["H"], a["V"], a["ws"],
                                          a["wsb"], None)

    assert call(h=None) == 1 and call(w=None) == 1 and call(tok=None) == 1
    assert call(H=4000) == 2 and call(H=0) == 2 and call(H=128) == 2 and call(rows=0) == 2 and call(V=0) == 2
    assert call(h=ctypes.c_void_p(4096 * 16 + 8)) == 2          # 16-byte alignment
    # one 8-byte key per (row, 128-entry vocabulary tile)
    need = lib.orthrus_lm_head_workspace_bytes(32, 4096, 151936)
    assert need == 32 * 1187 * 8
    assert lib.orthrus_lm_head_workspace_bytes(32, 4000, 151936) == 0
    assert call(wsb=need - 1) == 4 and call(ws=None) == 4
    assert lib.orthrus_lm_head_packed_bytes(4096, 151936) == 151936 * 4096 * 2
    assert lib.orthrus_lm_head_packed_bytes(256, 33) == 64 * 256 * 2          # padded to 32-row tiles
    assert lib.orthrus_lm_head_packed_bytes(100, 33) == 0
    assert lib.orthrus_lm_head_pack_weight(None, A16, 4096, 100, None) == 1
    assert lib.orthrus_lm_head_pack_weight(A16, A16, 4000, 100, None) == 2
    assert lib.orthrus_lm_head_pack_weight(A16, ctypes.c_void_p(4096 * 16 + 4), 4096, 100, None) == 2
    dn = lib.orthrus_lm_head_denoise_workspace_bytes(64, 4096, 151936)
    assert dn == 64 * 1187 * 16                                               # key + (max, sum) per tile
    den = lib.orthrus_lm_head_denoise_step
    assert den(A16, A16, FAKE, FAKE, FAKE, None, None, 2, 32, 4096, 151936, FAKE, dn, None) == 1
    assert den(A16, A16, FAKE, FAKE, FAKE, None, FAKE, 2, 33, 4096, 151936, FAKE, dn, None) == 2
    assert den(A16, A16, FAKE, FAKE, FAKE, None, FAKE, 2, 32, 4096, 151936, FAKE, dn - 1, None) == 4
    acc = lib.orthrus_lm_head_greedy_accept
    assert acc(A16, A16, None, FAKE, FAKE, None, 1, 32, 4096, 151936, FAKE, need, None) == 1
    assert acc(A16, A16, FAKE, FAKE, FAKE, None, 1, 33, 4096, 151936, FAKE, need, None) == 2
    assert acc(A16, A16, FAKE, FAKE, FAKE, None, 2, 32, 4096, 151936, FAKE, need, None) == 4   # needs 64 rows


def test_prefill_validation():
    lib = B.lib()
    d = good_desc(max_ctx_len=4096, max_pages_per_seq=514)      # capacity 8224 positions
    wsb = lib.orthrus_prefill_workspace_bytes(ctypes.byref(d), 4096)
    # 128 virtual sequences: their page-table rows and lengths, each region
    # rounded up to 256 bytes, then the block-attention workspace of the
    # virtual batch (automatic split: 8192 positions)
    vd = good_desc(batch=128, block_k=32, max_ctx_len=4096 + 4096 - 32, max_pages_per_seq=514, split_tokens=8192)
    up = lambda x: -(-x // 256) * 256
    assert wsb == up(128 * 514 * 4) + up(128 * 4) + lib.orthrus_block_attn_workspace_bytes(ctypes.byref(vd))
    assert lib.orthrus_prefill_workspace_bytes(ctypes.byref(d), 4200) == 0      # 4096 + 4224 > 8224
    assert lib.orthrus_prefill_workspace_bytes(ctypes.byref(d), 0) == 0
    W = ctypes.c_void_p(4096 * 256)
    call = lambda desc, mp, ws=W, wsb=wsb, q=FAKE: lib.orthrus_prefill(
        q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, mp, FAKE, None, ctypes.byref(desc), ws, wsb, None)
    assert call(d, 4096, q=None) == 1
    assert call(d, 4200) == 2 and call(d, 0) == 2
    assert call(good_desc(head_dim=80, max_ctx_len=0), 32) == 3
    assert call(d, 4096, wsb=wsb - 1) == 4 and call(d, 4096, ws=None) == 4
    assert call(d, 4096, ws=ctypes.c_void_p(4096 * 256 + 16)) == 4          # 256-byte alignment


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 32, 4, 64)
    with pytest.raises(B.OrthrusError):
        B.block_attn(q, q, q, q, q, torch.zeros(1, 1, dtype=torch.int32), torch.zeros(1, dtype=torch.int32), 0)


def test_misaligned_pointers_are_rejected():
    """Tensors moved as 16-byte units must be 16-byte aligned, device-address
    arrays 8-byte aligned and int32 arrays 4-byte aligned: a misaligned
    pointer gives ERR_SHAPE (2) before anything is launched."""
    lib = B.lib()
    d = good_desc()
    need = lib.orthrus_block_attn_workspace_bytes(ctypes.byref(d))
    W = ctypes.c_void_p(4096 * 256)
    A = FAKE
    M8 = ctypes.c_void_p(4096 + 8)      # 8-byte but not 16-byte aligned
    M2 = ctypes.c_void_p(4096 + 2)      # 2-byte aligned only
    for slot in range(9):               # q, k_cache, v_cache, k_blk, v_blk, page_table, ctx_lens, (mode), out
        if slot == 7:
            continue
        ptrs = [A] * 9
        ptrs[slot] = M2 if slot in (5, 6) else M8
        assert lib.orthrus_block_attn(*ptrs[:7], 0, ptrs[8], ctypes.byref(d), W, need, None) == 2, slot
    # int32 arrays need only 4-byte alignment: the call gets past that check
    # and fails on the (too small) workspace instead
    assert lib.orthrus_block_attn(A, A, A, A, A, ctypes.c_void_p(4096 + 4), A, 0, A, ctypes.byref(d), W, need - 1,
                                  None) == 4
    for slot in range(4):
        ptrs = [A] * 4
        ptrs[slot] = M8
        assert lib.orthrus_kv_append(*ptrs, A, A, A, None, None, ctypes.byref(d), None) == 2, slot
    assert lib.orthrus_kv_append(A, A, A, A, M2, A, A, None, None, ctypes.byref(d), None) == 2
    assert lib.orthrus_kv_append(A, A, A, A, A, A, A, None, M2, ctypes.byref(d), None) == 2
    assert lib.orthrus_kv_append_layers(A, A, A, ctypes.c_void_p(4096 + 4), 36, A, A, A, None, None,
                                        ctypes.byref(d), None) == 2
    pd = good_desc(max_ctx_len=4096, max_pages_per_seq=514)
    pw = lib.orthrus_prefill_workspace_bytes(ctypes.byref(pd), 4096)
    P = ctypes.c_void_p(4096 * 256)
    for slot in (0, 1, 2, 3, 4, 9):     # q, k, v, k_cache, v_cache, out
        ptrs = [A] * 10
        ptrs[slot] = M8
        assert lib.orthrus_prefill(*ptrs[:8], 4096, ptrs[9], None, ctypes.byref(pd), P, pw, None) == 2, slot
    assert lib.orthrus_prefill(A, A, A, A, A, A, A, M2, 4096, A, None, ctypes.byref(pd), P, pw, None) == 2


def test_noalloc_validation():
    """The entry point without a workspace validates like orthrus_block_attn
    and refuses, before any HIP call, a descriptor whose partials exceed the
    library's fixed scratch array."""
    lib = B.lib()
    d = good_desc()
    call = lambda desc, q=FAKE, mode=0: lib.orthrus_block_attn_noalloc(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, mode,
                                                                       FAKE, ctypes.byref(desc), None)
    assert call(d, q=None) == 1
    assert call(d, mode=2) == 2
    assert call(good_desc(head_dim=96)) == 3
    assert call(d, q=ctypes.c_void_p(4096 + 8)) == 2
    big = good_desc(batch=4, split_tokens=64)             # 4 x 128 splits: about 138 MB of partials
    assert lib.orthrus_block_attn_workspace_bytes(ctypes.byref(big)) > 32 << 20
    assert call(big) == 4


def test_binding_makes_no_workspace_during_capture(monkeypatch):
    """The binding's cached workspaces are per (device, kind, stream), are
    replaced (never freed) when they must grow, and are never made while a
    stream is capturing a graph (the zero fill would become a graph node):
    such a call raises and asks for a warm-up or an explicit ws=."""
    import torch

    class FakeStream:
        cuda_stream = 0xabc

    made = []
    monkeypatch.setattr(torch, "zeros", lambda n, dtype=None, device=None: made.append(n) or torch.empty(n, dtype=dtype))
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: False)
    B._workspaces.clear()
    s = FakeStream()
    w1 = B.workspace("cuda:0", 1000, "attn", s)
    assert B.workspace("cuda:0", 900, "attn", s) is w1            # cached per stream
    w2 = B.workspace("cuda:0", 1500, "attn", s)                   # grows at least twofold
    assert w2.numel() == 2000 and made == [1000, 2000] and w1 in B._retired
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
    assert B.workspace("cuda:0", 1800, "attn", s) is w2           # big enough: fine while capturing
    with pytest.raises(B.OrthrusError, match="capturing stream"):
        B.workspace("cuda:0", 5000, "attn", s)
    other = FakeStream()
    other.cuda_stream = 0xdef
    with pytest.raises(B.OrthrusError, match="capturing stream"):
        B.workspace("cuda:0", 100, "attn", other)                 # another stream has none yet
    B._workspaces.clear()
    B._retired.clear()
