"""Plain fp64 CPU oracle for one Orthrus dual-view decode step.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously correct
definition that the HIP kernels are checked against.  Only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import it; the
product path never does, and this module imports nothing from the product
package (it shares no code, tables or helpers with it).

Source of the definitions: the explainer page for "Orthrus: Memory-Efficient
Parallel Token Generation via Dual-View Diffusion" (gist.science, arXiv
2605.12825), technical summary:

* §2.1 -- the frozen AR head and the diffusion head both read ONE shared
  cache of AR keys/values (K_AR, V_AR); there is no second cache.
* §2.2 -- the diffusion view's block mask M_diff: (rule 1) every position in
  the block attends to the clean AR context that precedes the block anchor;
  (rule 2) positions inside the same block attend to each other in both
  directions.
* §2.3 -- inference: the diffusion head projects K candidates from
  [anchor, K-1 masks] in one pass; the frozen AR head then sees the filled
  block and computes exact targets for all K positions in one (causal) pass;
  drafts are accepted strictly left to right while they equal the AR greedy
  prediction; at the first divergence j the prefix up to j-1 is committed
  together with the AR correction token, and the cache is truncated to the
  committed positions.

Everything is written as the definition, in fp64, with numpy primitives
(fancy indexing, matmul, exp) as steps and no blocking or fusion.

Readings of points the pages leave open:

* rows of the two views are aligned by position: row i of either view is the
  prediction for the token after block position i; drafts[i] is compared
  with argmax(ar_logits[i]);
* accept_len a counts accepted drafts (0..K); the step commits
  n = min(a + 1, K) tokens (the correction exists only on a divergence; with
  a == K no bonus token exists because no AR row past K-1 is computed);
* next_token = g[min(a, K - 1)], the last committed token (next anchor);
* the appended K/V are the AR verify pass's block rows 0..n-1 (anchor plus
  accepted drafts), written at cache positions L .. L+n-1;
* grouped-query attention maps query head h to KV head h * Hkv // Hq; the
  softmax scale defaults to 1/sqrt(D); no soft-cap, window or bias;
* argmax ties go to the lowest index; -0.0 equals +0.0 (IEEE compare);
* the LM head is a plain linear map hidden @ weight^T with weight stored as
  [V, H] (no bias, no logit scaling or soft-cap);
* multi-step denoising (a variant the pages name without its re-mask rule)
  uses low-confidence remasking: each step unmasks the most confident
  still-masked positions, confidence = the greedy token's softmax
  probability;
* at temperature T > 0 a draft is accepted when u * q[x] < p[x] (p, q the
  AR and diffusion softmaxes at T; u a given uniform), and the correction at
  the first rejection is drawn from max(p - q, 0) by inverse CDF with a
  second given uniform (the standard lossless rejection rule; the pages name
  temperature settings without the rule).

Pins: every function here is pinned in tests/test_oracle_pins.py against
closed forms, invariants and brute force (see each docstring).
"""

from __future__ import annotations

import numpy as np

DIFF_BIDIR = 0
AR_CAUSAL = 1


def _f64(x):
    """Exact widening to fp64 (bf16/fp16/fp32 all embed exactly in fp64)."""
    if hasattr(x, "detach"):  # a torch tensor: go through float32 exactly
        x = x.detach().cpu()
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.int64)


def _raw(x):
    """Element storage as numpy without any value conversion (bf16 tensors
    are viewed as their int16 bit patterns), for bit-exact copies."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            import torch
            x = x.view(torch.int16)
        x = x.numpy()
    return np.asarray(x)


def gather_context(cache, page_table_row, n_tokens, kv_head, page_size):
    """The cached key (or value) rows of one sequence and one KV head.

    Cache layout [num_pages, Hkv, P, D]; logical position p of the sequence
    lives in physical page page_table_row[p // P], slot p % P.  Returns the
    [n_tokens, D] fp64 rows in logical order.
    """
    n_pages = -(-n_tokens // page_size)
    pages = _i64(page_table_row)[:n_pages]
    if hasattr(cache, "detach"):                  # index before widening a large cache
        import torch
        rows = _f64(cache[torch.as_tensor(pages, device=cache.device), kv_head])
    else:
        rows = _f64(np.asarray(cache)[pages, kv_head])   # [n_pages, P, D]
    return rows.reshape(n_pages * page_size, rows.shape[-1])[:n_tokens]


def visible_keys(mode, L, K, i):
    """Logical key positions visible to block row i (0-based) of a block of K
    rows placed after L cached tokens.

    Cached context 0..L-1 is always visible (§2.2 rule 1).  Block key L+j is
    visible for every j < K in DIFF_BIDIR (§2.2 rule 2, bidirectional block),
    and only for j <= i in AR_CAUSAL (§2.3, the AR head's causal verify pass).
    """
    if mode == DIFF_BIDIR:
        blk = list(range(K))
    elif mode == AR_CAUSAL:
        blk = list(range(i + 1))
    else:
        raise ValueError("mode must be DIFF_BIDIR or AR_CAUSAL")
    return list(range(L)) + [L + j for j in blk]


def block_attn(q, k_cache, v_cache, k_blk, v_blk, page_table, ctx_lens, mode,
               softmax_scale=None, page_size=16, batches=None, heads=None):
    """Block attention of one decode step over the shared paged KV cache.

    Shapes: q [B, K, Hq, D]; k_cache/v_cache [num_pages, Hkv, P, D];
    k_blk/v_blk [B, K, Hkv, D]; page_table [B, max_pages]; ctx_lens [B].
    Returns fp64 [B, K, Hq, D]; rows/heads outside `batches`/`heads` (when
    given) are left NaN.

    For sequence b, query head h (KV head g = h*Hkv//Hq) and block row i:
    keys are the L cached keys followed by the K block keys, the visible set
    is visible_keys(mode, L, K, i), scores s_p = scale * <q, k_p>, and the
    output is sum_p softmax(s)_p v_p over the visible set.  Every visible set
    holds at least the row's own block key, so no softmax is empty.
    """
    q = _f64(q)
    kb = _f64(k_blk)
    vb = _f64(v_blk)
    pt = _i64(page_table)
    lens = _i64(ctx_lens)
    B, K, Hq, D = q.shape
    Hkv = kb.shape[2]
    scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)
    out = np.full((B, K, Hq, D), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(lens[b])
        ctx = {}
        for h in (range(Hq) if heads is None else heads):
            g = h * Hkv // Hq
            if g not in ctx:
                ctx[g] = (gather_context(k_cache, pt[b], L, g, page_size),
                          gather_context(v_cache, pt[b], L, g, page_size))
            keys_c, vals_c = ctx[g]
            # scores of every block row against the cached keys and the block keys
            s_c = scale * (keys_c @ q[b, :, h].T)           # [L, K]
            s_b = scale * (kb[b, :, g] @ q[b, :, h].T)      # [K(keys), K(rows)]
            for i in range(K):
                vis_b = [p - L for p in visible_keys(mode, L, K, i) if p >= L]
                s = np.concatenate([s_c[:, i], s_b[vis_b, i]])
                w = np.exp(s - s.max())
                num = w[:L] @ vals_c + w[L:] @ vb[b, vis_b, g]
                out[b, i, h] = num / w.sum()
    return out


def prefill_attn(q, k_cache, v_cache, k, v, page_table, ctx_lens, prompt_lens, softmax_scale=None,
                 page_size=16, batches=None, heads=None):
    """Causal attention of a prompt by the frozen AR head (§2.1: its keys and
    values are what fill the shared cache; the prompt is processed causally,
    as any AR prefill).

    Shapes: q [B, S, Hq, D]; k, v [B, S, Hkv, D] (the prompt's own keys and
    values); k_cache/v_cache [num_pages, Hkv, P, D] holding the L_b =
    ctx_lens[b] positions already cached before the prompt; page_table
    [B, max_pages]; prompt_lens [B] <= S.  Returns fp64 [B, S, Hq, D]: for
    sequence b, query head h (KV head h*Hkv//Hq) and prompt row i <
    prompt_lens[b], the softmax-weighted sum over cached positions 0..L_b-1
    and prompt rows 0..i.  Rows i >= prompt_lens[b] (padding) and rows or
    heads outside `batches`/`heads` are NaN.
    """
    q = _f64(q)
    kp = _f64(k)
    vp = _f64(v)
    pt = _i64(page_table)
    lens = _i64(ctx_lens)
    plens = _i64(prompt_lens)
    B, S, Hq, D = q.shape
    Hkv = kp.shape[2]
    scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)
    out = np.full((B, S, Hq, D), np.nan)
    for b in (range(B) if batches is None else batches):
        L, n = int(lens[b]), int(plens[b])
        for h in (range(Hq) if heads is None else heads):
            g = h * Hkv // Hq
            keys = np.concatenate([gather_context(k_cache, pt[b], L, g, page_size), kp[b, :n, g]])
            vals = np.concatenate([gather_context(v_cache, pt[b], L, g, page_size), vp[b, :n, g]])
            for i in range(n):
                s = scale * (keys[:L + i + 1] @ q[b, i, h])
                w = np.exp(s - s.max())
                out[b, i, h] = (w @ vals[:L + i + 1]) / w.sum()
    return out


def greedy_argmax(logits):
    """g[..., ] = the lowest vocabulary index attaining the row maximum.

    The AR head's greedy prediction per block position (§2.3 "greedy
    prediction"); ties resolve to the lowest index.  Written as its
    definition: find the maximum, then the first position equal to it.
    """
    x = _f64(logits)
    flat = x.reshape(-1, x.shape[-1])
    g = np.empty(flat.shape[0], dtype=np.int64)
    for r in range(flat.shape[0]):
        m = flat[r].max()
        g[r] = np.flatnonzero(flat[r] == m)[0]
    return g.reshape(x.shape[:-1])


def accept_prefix(draft_row, g_row):
    """Number of leading positions where the draft equals the AR greedy token
    (strict left-to-right evaluation, §2.3)."""
    a = 0
    for d, t in zip(draft_row, g_row):
        if int(d) != int(t):
            break
        a += 1
    return a


def greedy_accept(ar_logits, draft_tokens):
    """Greedy consensus of one step.

    Returns (accept_len [B], next_token [B], g [B, K]) with
    accept_len = accepted drafts a in [0, K] and next_token = g[min(a, K-1)],
    the AR correction token on a divergence (or the last accepted token when
    all K agree).  The committed tokens of the step are g[0 .. n-1] with
    n = commit_count(a, K).
    """
    g = greedy_argmax(ar_logits)
    drafts = _i64(draft_tokens)
    B, K = g.shape
    acc = np.array([accept_prefix(drafts[b], g[b]) for b in range(B)], dtype=np.int64)
    nxt = np.array([g[b, min(acc[b], K - 1)] for b in range(B)], dtype=np.int64)
    return acc, nxt, g


def lm_head_logits(hidden, weight):
    """Logits of the language-model head: logits[m, v] = sum_k hidden[m, k] *
    weight[v, k], in fp64 (products of bf16 values are exact in fp64).

    hidden [..., H] (the final hidden states of the block rows), weight
    [V, H] (one row per vocabulary entry, the usual linear-layer layout).
    The LM head turns each view's block rows into the token distributions
    that §2.3 compares (diffusion drafts, AR targets).
    """
    h = _f64(hidden)
    w = _f64(weight)
    return h @ w.T


def lm_head_argmax(hidden, weight):
    """Greedy token of each row: greedy_argmax of lm_head_logits (lowest
    index on ties)."""
    return greedy_argmax(lm_head_logits(hidden, weight))


def lm_head_greedy_accept(hidden, weight, draft_tokens):
    """Greedy consensus straight from the AR view's final hidden states
    [B, K, H]: greedy_accept of lm_head_logits.  Returns (accept_len [B],
    next_token [B], g [B, K])."""
    return greedy_accept(lm_head_logits(hidden, weight), draft_tokens)


def denoise_confidence(logits):
    """Greedy token and its confidence per row: the token is greedy_argmax
    and the confidence is its softmax probability,
    max_v softmax(x)_v = 1 / sum_v exp(x_v - max x)."""
    x = _f64(logits)
    m = x.max(axis=-1, keepdims=True)
    return greedy_argmax(x), 1.0 / np.exp(x - m).sum(axis=-1)


def denoise_select(confidence, masked, n_unmask):
    """One step of low-confidence remasking over a block: among the
    positions still masked, the n_unmask[b] most confident are unmasked (ties
    go to the lower position); every other masked position stays masked and
    unmasked positions stay unmasked.  Returns the new mask [B, K] (bool)."""
    c = _f64(confidence)
    m = np.asarray(masked, dtype=bool)
    n = _i64(n_unmask)
    out = m.copy()
    for b in range(c.shape[0]):
        cand = [i for i in range(c.shape[1]) if m[b, i]]
        order = sorted(cand, key=lambda i: (-c[b, i], i))
        for i in order[:max(int(n[b]), 0)]:
            out[b, i] = False
    return out


def lm_head_denoise_step(hidden, weight, masked, n_unmask):
    """One multi-step-denoising update from the diffusion view's final hidden
    states [B, K, H]: the LM-head logits give every position's greedy token
    and confidence, then denoise_select unmasks the n_unmask[b] most confident
    masked positions.  Returns (tokens [B, K], confidence [B, K],
    new_mask [B, K])."""
    tok, conf = denoise_confidence(lm_head_logits(hidden, weight))
    return tok, conf, denoise_select(conf, masked, n_unmask)


def softmax_t(logits, temperature):
    """Row-wise softmax of logits / T in fp64 (the sampling distribution of
    a head at temperature T > 0)."""
    x = _f64(logits) / float(temperature)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def sample_accept(ar_logits, draft_logits, draft_tokens, u_accept, u_resample, temperature):
    """Lossless acceptance of sampled drafts at temperature T > 0 (the
    stochastic form of the consensus step: the pages name temperature
    settings; this is the standard rejection rule that keeps the AR head's
    distribution exact).

    For each sequence b, rows i = 0 .. K-1 in order, with p = softmax(ar/T),
    q = softmax(draft/T) of row i and x = draft_tokens[b, i]:
      accept x when u_accept[b, i] * q[x] < p[x] (probability min(1, p/q));
      at the first rejection i: accept_len = i and next_token is drawn from
      the residual r = max(p - q, 0) / sum(r) by inverse CDF,
      next = min{v : cumsum(r)[v] > u_resample[b] * sum(r)}.
    With no rejection: accept_len = K, next_token = x of row K - 1.  A draft
    outside [0, V) has probability zero under both heads and is rejected.
    The step commits min(accept_len + 1, K) tokens, as in the greedy case.
    Returns (accept_len [B], next_token [B]).
    """
    drafts = _i64(draft_tokens)
    ua = _f64(u_accept)
    ur = _f64(u_resample)
    p_all = softmax_t(ar_logits, temperature)
    q_all = softmax_t(draft_logits, temperature)
    B, K = drafts.shape
    acc = np.full(B, K, dtype=np.int64)
    nxt = drafts[:, K - 1].copy()
    V = p_all.shape[-1]
    for b in range(B):
        for i in range(K):
            p, q, x = p_all[b, i], q_all[b, i], drafts[b, i]
            # a token outside the vocabulary has p = q = 0: never accepted
            if 0 <= x < V and ua[b, i] * q[x] < p[x]:
                continue
            r = np.maximum(p - q, 0.0)
            total = r.sum()
            if total <= 0.0:  # p == q: cannot reject; kept for completeness
                r, total = p, 1.0
            c = np.cumsum(r)
            acc[b] = i
            nxt[b] = int(np.flatnonzero(c > ur[b] * total)[0])
            break
    return acc, nxt


def commit_count(accept_len, K):
    """Tokens committed by one step: the accepted prefix plus the correction
    token, capped at the block size (§2.3)."""
    return min(int(accept_len) + 1, K)


def kv_append(k_cache, v_cache, k_blk, v_blk, page_table, ctx_lens, accept_len, page_size=16):
    """Commit the accepted block rows into the shared cache.

    Rows r < n = commit_count(a_b, K) of the AR pass's block K/V go to
    logical position L_b + r, i.e. physical page page_table[b][(L_b+r)//P],
    slot (L_b+r) % P, for every KV head.  Nothing else in the cache changes
    (the cache is "truncated" to the committed positions, §2.3).

    Returns (k_cache', v_cache', new_ctx_lens [B], slots [B, K]) where the
    caches are fresh numpy copies of the element storage (bf16 as int16 bit
    patterns), new_ctx_lens = L + n, and
    slots[b, r] = page * P + slot for the written rows and -1 otherwise.
    """
    kc = _raw(k_cache).copy()
    vc = _raw(v_cache).copy()
    kb = _raw(k_blk)
    vb = _raw(v_blk)
    pt = _i64(page_table)
    lens = _i64(ctx_lens)
    acc = _i64(accept_len)
    B, K = kb.shape[0], kb.shape[1]
    slots = np.full((B, K), -1, dtype=np.int64)
    new_lens = np.empty(B, dtype=np.int64)
    for b in range(B):
        L = int(lens[b])
        n = commit_count(acc[b], K)
        for r in range(n):
            pos = L + r
            page = int(pt[b, pos // page_size])
            slot = pos % page_size
            kc[page, :, slot, :] = kb[b, r]
            vc[page, :, slot, :] = vb[b, r]
            slots[b, r] = page * page_size + slot
        new_lens[b] = L + n
    return kc, vc, new_lens, slots


def kv_write(k_cache, v_cache, k, v, page_table, ctx_lens, n_rows, page_size=16):
    """Write a prompt's keys and values into the shared cache (the prefill
    that builds K_AR, V_AR, §2.1): rows r < n_rows[b] of k/v [B, S, Hkv, D] go
    to logical position L_b + r, i.e. page page_table[b][(L_b+r)//P], slot
    (L_b+r) % P, for every KV head; nothing else changes.

    Returns (k_cache', v_cache', new_ctx_lens = L + n) with the caches as
    fresh numpy copies of the element storage (bf16 as int16 bit patterns).
    """
    kc = _raw(k_cache).copy()
    vc = _raw(v_cache).copy()
    kr = _raw(k)
    vr = _raw(v)
    pt = _i64(page_table)
    lens = _i64(ctx_lens)
    n = _i64(n_rows)
    for b in range(kr.shape[0]):
        L = int(lens[b])
        for r in range(int(n[b])):
            pos = L + r
            page = int(pt[b, pos // page_size])
            kc[page, :, pos % page_size, :] = kr[b, r]
            vc[page, :, pos % page_size, :] = vr[b, r]
    return kc, vc, lens + n
