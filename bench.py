#!/usr/bin/env python3
"""Benchmark of one Orthrus dual-view decode step on one MI355X.

Workload (Qwen3-8B attention shape, batch 1, 8192 cached tokens, K = 32):
one decode step of the whole 36-layer model's hot path =
  36 x block attention in the diffusion view (DIFF_BIDIR)
  36 x block attention in the AR verify view (AR_CAUSAL)
   1 x greedy accept over 32 x 151936 fp32 logits
   1 x KV append of the accepted rows into all 36 layers (one launch)
Every layer has its own synthetic paged K/V (N(0,1) bf16, shuffled 16-token
pages), so each attention call reads its 32 MiB of KV cold (1.2 GB per view
per step, several times the 256 MB Infinity Cache).  The step is captured once
in a HIP graph and replayed; inputs are resident in HBM before timing starts.

Output: one JSON line.  `value` = block-attention KV bytes read per step /
step time (GB/s).  The step's accept replays one 19.4 MB logits buffer, so it
reads it warm from the Infinity Cache (under 1 % of the step); the
`greedy_accept` field times it alone both warm and cold.  `roofline` = the block-attention call (main + combine
kernels) timed alone with HIP events on its stream, against the 8 TB/s HBM
peak.  `cpu_baseline` = the fp64 oracle on a bounded sample of the same step
on the host cores.  `sample_accept` = the sampled consensus at temperature 1
(orthrus_sample_accept over both heads' [B, 32, 151936] fp32 logits) timed
on its own at B = 1 and 16; it is not part of the greedy step above.
`lm_head` = the LM head with fused argmax and greedy accept at the Qwen3-8B
head (B = 1, 4, 16); `prefill` = the prompt prefill of one layer (2k and 8k
prompts).  Neither is part of the step above either.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "block-attn KV-read GB/s (% of HBM peak), Qwen3-8B K=32 ctx 8k, bs 1–16"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--batch", type=int, default=1)
    p.add_argument("--ctx", type=int, default=8192)
    p.add_argument("--layers", type=int, default=36)
    p.add_argument("--split-tokens", type=int, default=0,
                   help="context positions per work-group: 0 automatic, -1 balanced, else a multiple of 64")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a graph")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-sample", action="store_true", help="skip the sampled-consensus timing")
    p.add_argument("--no-lm-head", action="store_true", help="skip the LM-head timing")
    p.add_argument("--no-prefill", action="store_true", help="skip the prompt-prefill timing")
    p.add_argument("--no-config2", action="store_true", help="skip the Qwen3-1.7B attention-shape leg")
    p.add_argument("--no-long-context", action="store_true",
                   help="skip the 36-layer step at batch 4, 32768 cached tokens")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="run one plain device copy of this size first (calibrates HBM byte counters)")
    return p.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Step:
    """Buffers and calls of one decode step (all layers)."""

    def __init__(self, ob, I, torch, batch, ctx, layers, split_tokens, seed=0, workload="qwen3_8b_8k"):
        self.ob, self.torch = ob, torch
        d = torch.device("cuda:0")
        w = I.WORKLOADS[workload]
        self.B, self.K, self.Hq, self.Hkv, self.D = batch, w["block_k"], w["n_q_heads"], w["n_kv_heads"], w["head_dim"]
        self.layers, self.split = layers, split_tokens
        lens = [int(c) for c in ctx] if hasattr(ctx, "__len__") else [ctx] * batch
        table, n_pages = I.make_page_table(lens, self.K, 16, shuffle=True, seed=seed)
        self.page_table = torch.from_numpy(table).to(d)
        self.ctx_lens = torch.tensor(lens, dtype=torch.int32, device=d)
        self.max_ctx = max(lens)
        self.L = []
        for l in range(layers):
            a = I.make_attn_inputs(workload, seed=seed, layer=l, device=d, ctx_lens=lens, batch=batch)
            q_ar = I._randn(a.q.shape, torch.bfloat16, d, I._seed(seed + 1, workload, l, "q"))
            kb_ar = I._randn(a.k_blk.shape, torch.bfloat16, d, I._seed(seed + 1, workload, l, "k_blk"))
            vb_ar = I._randn(a.v_blk.shape, torch.bfloat16, d, I._seed(seed + 1, workload, l, "v_blk"))
            self.L.append(dict(k_cache=a.k_cache, v_cache=a.v_cache, q_diff=a.q, kb_diff=a.k_blk, vb_diff=a.v_blk,
                               q_ar=q_ar, kb_ar=kb_ar, vb_ar=vb_ar, out_diff=torch.empty_like(a.q),
                               out_ar=torch.empty_like(a.q)))
        self.logits, t = I.make_logits(batch, self.K, I.QWEN3_VOCAB, seed=seed, workload=workload, plant=True,
                                       device=d)
        self.prefix = I.geometric_prefix(batch, self.K, seed=seed, workload=workload)
        self.drafts = I.make_drafts(t.cpu(), self.prefix, I.QWEN3_VOCAB, seed=seed).to(d)
        self.new_ctx = torch.empty(batch, dtype=torch.int32, device=d)
        self.append_ptrs = ob.LayerPointers([x["k_cache"] for x in self.L], [x["v_cache"] for x in self.L],
                                            [x["kb_ar"] for x in self.L], [x["vb_ar"] for x in self.L])
        self.kv_bytes_call = I.kv_bytes(lens, self.Hkv, self.D, 2)

    def attn(self, l, mode):
        x = self.L[l]
        q, kb, vb, out = ((x["q_diff"], x["kb_diff"], x["vb_diff"], x["out_diff"]) if mode == self.ob.DIFF_BIDIR
                          else (x["q_ar"], x["kb_ar"], x["vb_ar"], x["out_ar"]))
        self.ob.block_attn(q, x["k_cache"], x["v_cache"], kb, vb, self.page_table, self.ctx_lens, mode, out,
                           max_ctx_len=self.max_ctx, split_tokens=self.split)

    def run(self):
        ob = self.ob
        for l in range(self.layers):
            self.attn(l, ob.DIFF_BIDIR)
        for l in range(self.layers):
            self.attn(l, ob.AR_CAUSAL)
        self.acc, self.nxt, self.tok = ob.greedy_accept(self.logits, self.drafts)
        ob.kv_append_layers(self.append_ptrs, self.page_table, self.ctx_lens, self.acc, new_ctx_lens=self.new_ctx,
                            max_ctx_len=self.max_ctx)


def capture(torch, fn):
    """Capture fn() in a HIP graph on a side stream, after one eager run on
    that same stream so that the binding's per-stream workspaces exist before
    capture (and no zero fill of a new workspace lands in the graph); returns
    a replay callable."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g.replay


def time_region(torch, fn, iters, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(iters):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters  # ms


def attn_only_ms(torch, step, mode, use_graph, iters=20, warmup=3, min_calls=16, spread=None):
    """Average time of one block-attention call (main + combine kernels).
    One replay runs at least `min_calls` calls, cycling through the layers
    (the other layers' KV read between two calls on one layer exceeds the
    256 MB Infinity Cache, so every call reads its KV cold), and the replay
    boundary is amortised over those calls."""
    n = max(step.layers, min_calls)
    fn = lambda: [step.attn(c % step.layers, mode) for c in range(n)]
    rep = capture(torch, fn) if use_graph else fn
    ms = time_region(torch, rep, iters, warmup) / n
    if spread is not None:   # per-call time of each replay, timed on its own
        st = torch.cuda.current_stream()
        for _ in range(iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            rep()
            e1.record(st)
            torch.cuda.synchronize()
            spread.append(e0.elapsed_time(e1) / n)
    return ms


TRAFFIC_FILE = os.path.join("diffusion_drafted_verification_amd", "traffic_counters.json")
ATTN_SOURCES = ("block_attn.hip", "orthrus_device.h", "orthrus_host.h")


def attn_source_sha(root):
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(root, "diffusion_drafted_verification_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(root, batch, ctx):
    """HBM bytes per block-attention call from the committed FETCH_SIZE /
    WRITE_SIZE counter runs, if they were taken on the current kernel
    sources at this workload; else None."""
    path = os.path.join(root, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("attn_source_sha256") != attn_source_sha(root):
        return None
    w = d.get("workloads", {}).get(f"b{batch}_ctx{ctx}")
    return None if w is None else int(w["hbm_bytes_per_call"])


def achievable_gbs(torch, ob, mib=1024):
    """Measured achievable HBM rates over `mib` MiB (4x the Infinity Cache):
    the library's read-only streaming probe (bytes read / time) and its
    plain streaming copy (bytes read + written / time)."""
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    sink = torch.empty(4 << 20, dtype=torch.uint8, device="cuda:0")
    ms_read = time_region(torch, lambda: ob.read_probe(src, sink), 10, 3)
    ms_copy = time_region(torch, lambda: ob.copy_probe(dst, src), 10, 3)
    del src, dst, sink
    torch.cuda.empty_cache()
    return round(n / (ms_read * 1e-3) / 1e9, 1), round(2 * n / (ms_copy * 1e-3) / 1e9, 1)


def sample_accept_timing(torch, ob, I, use_graph, temperature=1.0):
    """Sampled consensus (orthrus_sample_accept) over both heads' fp32 logits
    [B, 32, 151936] at B = 1 and 16.  Each graph replay cycles through enough
    input copies (>= 600 MB) that every call reads its logits from HBM, not
    from the 256 MB Infinity Cache.  Algorithmic bytes per call: both heads'
    logits once, 2 * B * K * V * 4."""
    d = torch.device("cuda:0")
    V, K = I.QWEN3_VOCAB, 32
    out = {}
    for bs in (1, 16):
        args = I.make_sample_inputs(bs, K, V, temperature, seed=bs, workload="qwen3_8b_8k", device=d)
        nbytes = 2 * bs * K * V * 4
        n = max(2, math.ceil(600e6 / nbytes))
        sets = [args] + [tuple(t.clone() for t in args) for _ in range(n - 1)]
        ws = torch.empty(ob.lib().orthrus_sample_accept_workspace_bytes(bs, K, V), dtype=torch.uint8, device=d)
        acc, _ = ob.sample_accept(*args, temperature, ws=ws)
        mean_acc = float(acc.float().mean().item())
        fn = lambda: [ob.sample_accept(*c, temperature, ws=ws) for c in sets]
        rep = capture(torch, fn) if use_graph else fn
        ms = time_region(torch, rep, 10, 2) / n
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[f"bs{bs}"] = {"us_per_call": round(ms * 1e3, 2), "bytes_per_call": nbytes, "gbs": round(gbs, 1),
                          "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "mean_accept_len": round(mean_acc, 2),
                          "input_copies": n}
        del sets, args, rep, ws
        torch.cuda.empty_cache()
    return {"kernel": "orthrus_sample_accept (sample_stats + sample_resid + sample_pick)",
            "temperature": temperature, "vocab": V, "block_k": K, **out}


def lm_head_timing(torch, ob, I, use_graph):
    """LM head with fused argmax (orthrus_lm_head_greedy_accept) over the
    Qwen3-8B head: bf16 weight [151936, 4096], packed once (1.24 GB, larger than the
    256 MB Infinity Cache, so every call streams it from HBM) and the AR
    view's hidden states [B, 32, 4096], at B = 1, 4 and 16.  Algorithmic
    bytes per call: the weight once plus the hidden states; flops:
    2 * B * 32 * 4096 * 151936."""
    d = torch.device("cuda:0")
    H, V, K = I.QWEN3_8B_HIDDEN, I.QWEN3_VOCAB, 32
    _, w, _ = I.make_lm_head_inputs(1, H, V, seed=0, workload="qwen3_8b_8k", device=d)
    head = ob.PackedLmHead(w)   # packed once, as at model load
    del w
    out = {}
    for bs in (1, 4, 16):
        h, _, _ = I.make_lm_head_inputs(bs * K, H, 1, seed=bs, workload="qwen3_8b_8k", device=d)
        h = h.view(bs, K, H)
        drafts = torch.zeros((bs, K), dtype=torch.int32, device=d)
        ws = torch.empty(ob.lib().orthrus_lm_head_workspace_bytes(bs * K, H, V), dtype=torch.uint8, device=d)
        n = 4
        fn = lambda: [ob.lm_head_greedy_accept(h, head, drafts, ws=ws) for _ in range(n)]
        fn()
        rep = capture(torch, fn) if use_graph else fn
        ms = time_region(torch, rep, 5, 2) / n
        nbytes = V * H * 2 + bs * K * H * 2
        flops = 2.0 * bs * K * H * V
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[f"bs{bs}"] = {"us_per_call": round(ms * 1e3, 2), "bytes_per_call": nbytes, "gbs": round(gbs, 1),
                          "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                          "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                          "frac_mfma_bf16": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        # the multi-step denoising update on the same rows (argmax plus the
        # softmax statistics in the epilogue, then the remasking)
        masked = torch.ones((bs, K), dtype=torch.uint8, device=d)
        nun = torch.full((bs,), 8, dtype=torch.int32, device=d)
        nm = torch.empty_like(masked)
        wsd = torch.empty(ob.lib().orthrus_lm_head_denoise_workspace_bytes(bs * K, H, V), dtype=torch.uint8,
                          device=d)
        fnd = lambda: [ob.lm_head_denoise_step(h, head, masked, nun, new_masked=nm, ws=wsd) for _ in range(n)]
        fnd()
        repd = capture(torch, fnd) if use_graph else fnd
        msd = time_region(torch, repd, 5, 2) / n
        out[f"bs{bs}"]["denoise_step_us"] = round(msd * 1e3, 2)
        del h, ws, rep, repd, wsd
    del head
    torch.cuda.empty_cache()
    return {"kernel": "orthrus_lm_head_greedy_accept (lm_head_tiles + lm_head_finish); denoise_step_us: "
                      "orthrus_lm_head_denoise_step on the same rows", "hidden": H,
            "vocab": V, "block_k": K, **out}


def prefill_timing(torch, ob, I, use_graph):
    """Prompt prefill (orthrus_prefill: cache write plus causal attention) of
    one layer at the Qwen3-8B attention shape (Hq 32, Hkv 8, D 128, bf16),
    B = 1: a 2048-token prompt with an empty cache, a 2048-token prompt after
    8192 cached tokens, and an 8192-token prompt.  Algorithmic flops: QK^T
    and PV over the causal set, 4 * Hq * D * sum_i (L + i + 1)."""
    d = torch.device("cuda:0")
    Hq, Hkv, D = 32, 8, 128
    out = {}
    for L, S in ((0, 2048), (8192, 2048), (0, 8192)):
        x = I.make_prefill_inputs([L], [S], Hq, Hkv, D, seed=1, device=d)
        ws = torch.empty(max(256, ob.lib().orthrus_prefill_workspace_bytes(
            ctypes.byref(ob.make_desc(x["q"][:, :32], x["k_cache"], x["page_table"], L)), S)),
            dtype=torch.uint8, device=d)
        o = torch.empty_like(x["q"])
        nl = torch.empty(1, dtype=torch.int32, device=d)
        fn = lambda: ob.prefill(x["q"], x["k"], x["v"], x["k_cache"], x["v_cache"], x["page_table"], x["ctx_lens"],
                                x["prompt_lens"], S, o, new_ctx_lens=nl, max_ctx_len=L, ws=ws)
        fn()
        rep = capture(torch, fn) if use_graph else fn
        ms = time_region(torch, rep, 10, 2)
        flops = 4.0 * Hq * D * sum(L + i + 1 for i in range(S))
        tf = flops / (ms * 1e-3) / 1e12
        out[f"L{L}_S{S}"] = {"us_per_call": round(ms * 1e3, 1), "tflops": round(tf, 1),
                             "frac_mfma_bf16": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                             "prompt_tokens_per_s": round(S / (ms * 1e-3), 1)}
        del x, ws, o, rep
        torch.cuda.empty_cache()
    return {"kernel": "orthrus_prefill (prefill_setup + prefill_kv_write + attn_stream AR_CAUSAL)",
            "shape": "B1 Hq32/Hkv8 D128 bf16, one layer", **out}


def config2_timing(torch, ob, I, use_graph):
    """The Qwen3-1.7B attention shape (Hq 16, Hkv 8, D 128: two query heads
    per KV head), one sequence with 2048 cached tokens, K = 32: the block
    attention call of both views timed alone, cycling over enough layers
    (1 GiB of K/V) that every call reads its K/V cold.  Algorithmic bytes per
    call: 2048 x 8 x 128 x 2 x 2 = 8 MiB."""
    layers = max(2, math.ceil(1.0 * 2**30 / (2048 * 4096)))
    s2 = Step(ob, I, torch, 1, 2048, layers, 0, seed=1, workload="qwen3_1p7b_2k")
    spread = []
    ms_diff = attn_only_ms(torch, s2, ob.DIFF_BIDIR, use_graph, iters=10, spread=spread)
    ms_ar = attn_only_ms(torch, s2, ob.AR_CAUSAL, use_graph, iters=10, spread=spread)
    ms = 0.5 * (ms_diff + ms_ar)
    gbs = s2.kv_bytes_call / (ms * 1e-3) / 1e9
    split = ob.lib().orthrus_block_attn_split_tokens(
        ob.make_desc(s2.L[0]["q_diff"], s2.L[0]["k_cache"], s2.page_table, s2.max_ctx, None, 0))
    flops = 2 * 2 * 1 * 32 * 16 * 128 * (2048 + 32)
    out = {"workload": "qwen3_1p7b_2k: B1 Hq16/Hkv8 D128 ctx2048 K32 (block attention, both views)",
           "us_per_call": round(ms * 1e3, 3), "us_diff": round(ms_diff * 1e3, 3), "us_ar": round(ms_ar * 1e3, 3),
           "bytes_per_call": s2.kv_bytes_call, "kv_gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
           "split_tokens": split, "mfma_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "us_per_call_p10_p50_p90": [round(sorted(spread)[int(q * (len(spread) - 1))] * 1e3, 3)
                                       for q in (0.1, 0.5, 0.9)]}
    del s2
    torch.cuda.empty_cache()
    return out


def accept_timing(torch, ob, I, use_graph, step):
    """The step's greedy accept (32 x 151936 fp32 logits per sequence) timed
    alone, warm (the same 19.4 MB each call, as the step replays it: the
    logits stay in the 256 MB Infinity Cache) and cold (cycling over input
    copies of at least 600 MB)."""
    B, K, V = step.B, step.K, I.QWEN3_VOCAB
    ws = torch.empty(ob.lib().orthrus_greedy_accept_workspace_bytes(B, K, V), dtype=torch.uint8, device="cuda:0")
    n = max(2, math.ceil(600e6 / (B * K * V * 4)))
    sets = [step.logits] + [step.logits.clone() for _ in range(n - 1)]
    out = {}
    for name, calls in (("warm", [step.logits] * n), ("cold", sets)):
        fn = lambda calls=calls: [ob.greedy_accept(c, step.drafts, ws=ws) for c in calls]
        fn()
        rep = capture(torch, fn) if use_graph else fn
        out[f"us_per_call_{name}"] = round(time_region(torch, rep, 10, 2) / n * 1e3, 2)
    del sets
    torch.cuda.empty_cache()
    nbytes = B * K * V * 4
    out.update({"kernel": "orthrus_greedy_accept (argmax_chunks + accept_rows)", "bytes_per_call": nbytes,
                "gbs_cold": round(nbytes / (out["us_per_call_cold"] * 1e-6) / 1e9, 1),
                "note": "the step replays one logits buffer, so its accept reads them warm"})
    return out


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline_long(I, torch):
    """The fp64 oracle, as is, on ONE layer of the long-context step (B4,
    32768 cached tokens: DIFF and AR block attention, greedy accept over
    4 x 32 x 151936 logits, append), run once; a step is 36 such layers."""
    from oracle import orthrus_oracle as O
    x = I.make_attn_inputs("qwen3_8b_32k_b4", layer=0)
    logits, t = I.make_logits(4, 32, I.QWEN3_VOCAB, seed=0, workload="qwen3_8b_32k_b4", plant=True)
    prefix = I.geometric_prefix(4, 32, seed=0, workload="qwen3_8b_32k_b4")
    drafts = I.make_drafts(t, prefix, I.QWEN3_VOCAB, seed=0).numpy()
    t0 = time.perf_counter()
    O.block_attn(x.q, x.k_cache, x.v_cache, x.k_blk, x.v_blk, x.page_table, x.ctx_lens, O.DIFF_BIDIR)
    O.block_attn(x.q, x.k_cache, x.v_cache, x.k_blk, x.v_blk, x.page_table, x.ctx_lens, O.AR_CAUSAL)
    acc, _, _ = O.greedy_accept(logits.numpy(), drafts)
    O.kv_append(x.k_cache, x.v_cache, x.k_blk, x.v_blk, x.page_table, x.ctx_lens, acc)
    el = time.perf_counter() - t0
    kv = 2 * I.kv_bytes([32768] * 4, 8, 128, 2)
    return {"workload": "qwen3_8b_32k_b4 step", "s_per_layer_step": round(el, 2),
            "s_per_step_x36": round(36 * el, 1), "kv_gbs": round(kv / el / 1e9, 4), "cores": int(_threads()),
            "sample": "one layer of the B4 x 32768-token step (both views over 4 sequences, accept over "
                      "4x32x151936, append), run once; x36 for the 36-layer step"}


def cpu_baseline(step, I, seconds):
    """The fp64 oracle, as is, on one layer of the step (both views, accept,
    append) at the same shapes; repeated for about `seconds`."""
    import numpy as np
    from oracle import orthrus_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    x = step.L[0]
    cpu = {k: v.cpu() for k, v in x.items()}
    pt, cl = step.page_table.cpu(), step.ctx_lens.cpu()
    logits, drafts = step.logits.cpu().numpy(), step.drafts.cpu().numpy()
    reps, t0 = 0, time.perf_counter()
    kv = 0
    while True:
        O.block_attn(cpu["q_diff"], cpu["k_cache"], cpu["v_cache"], cpu["kb_diff"], cpu["vb_diff"], pt, cl, O.DIFF_BIDIR)
        O.block_attn(cpu["q_ar"], cpu["k_cache"], cpu["v_cache"], cpu["kb_ar"], cpu["vb_ar"], pt, cl, O.AR_CAUSAL)
        acc, nxt, g = O.greedy_accept(logits, drafts)
        O.kv_append(cpu["k_cache"], cpu["v_cache"], cpu["kb_ar"], cpu["vb_ar"], pt, cl, acc)
        kv += 2 * step.kv_bytes_call
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
    except Exception:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join(sorted({f"{t.get('internal_api')} {t.get('version')}" for t in threadpool_info()}))
    except Exception:
        blas = "unknown"
    return {"value": round(kv / el / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model, "blas": blas,
            "sample": f"{reps} x one layer of the step (DIFF + AR block attention over {step.max_ctx} cached "
                      f"tokens x B{step.B}, accept over 32x151936, append) in {el:.1f} s; "
                      f"same shapes and inputs as the GPU step",
            "s_per_layer_step": round(el / reps, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    ROOT = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, ROOT)
    from diffusion_drafted_verification_amd import inputs as I
    from diffusion_drafted_verification_amd import orthrus as ob
    ob.lib()
    use_graph = not args.no_graph

    log("building inputs")
    step = Step(ob, I, torch, args.batch, args.ctx, args.layers, args.split_tokens)
    split = ob.lib().orthrus_block_attn_split_tokens(
        ob.make_desc(step.L[0]["q_diff"], step.L[0]["k_cache"], step.page_table, step.max_ctx, None,
                     args.split_tokens))
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
        dst = torch.empty_like(src)
        ob.copy_probe(dst, src)
        torch.cuda.synchronize()
        del src, dst
    step.run()
    torch.cuda.synchronize()
    rep = capture(torch, step.run) if use_graph else step.run
    log("timing step")
    ms = time_region(torch, rep, args.steps, args.warmup)
    kv_step = 2 * args.layers * step.kv_bytes_call
    value = kv_step / (ms * 1e-3) / 1e9

    log("timing attention calls")
    spread = []
    ms_diff = attn_only_ms(torch, step, ob.DIFF_BIDIR, use_graph, spread=spread)
    ms_ar = attn_only_ms(torch, step, ob.AR_CAUSAL, use_graph, spread=spread)
    ms_call = 0.5 * (ms_diff + ms_ar)
    achieved = step.kv_bytes_call / (ms_call * 1e-3) / 1e9
    pct = lambda q: round(sorted(spread)[min(len(spread) - 1, int(q * len(spread)))] * 1e3, 3)
    log("greedy accept, warm and cold")
    accept = accept_timing(torch, ob, I, use_graph, step)
    log("achievable read and copy rates")
    read_gbs, copy_gbs = achievable_gbs(torch, ob)
    flops = 2 * 2 * step.B * step.K * step.Hq * step.D * (args.ctx + step.K)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(ROOT, args.batch, args.ctx),
            "kernel": "block_attn call (attn_stream + attn_combine)", "us_per_call": round(ms_call * 1e3, 3),
            "us_diff": round(ms_diff * 1e3, 3), "us_ar": round(ms_ar * 1e3, 3),
            "bytes_per_call": step.kv_bytes_call, "split_tokens": split,
            "mfma_tflops": round(flops / (ms_call * 1e-3) / 1e12, 1),
            "us_per_call_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
            "achievable_read_gbs": read_gbs, "achievable_copy_gbs": copy_gbs,
            "frac_of_achievable_read": round(achieved / read_gbs, 4)}

    sweep = {}
    if not args.no_sweep:
        log("batch sweep")
        del step
        torch.cuda.empty_cache()
        for bs in (1, 2, 4, 8, 16):
            layers = max(2, math.ceil(1.0 * 2**30 / (bs * args.ctx * 4096)))
            s2 = Step(ob, I, torch, bs, args.ctx, layers, 0, seed=1)
            t = 0.5 * (attn_only_ms(torch, s2, ob.DIFF_BIDIR, use_graph, iters=10) +
                       attn_only_ms(torch, s2, ob.AR_CAUSAL, use_graph, iters=10))
            gbs = s2.kv_bytes_call / (t * 1e-3) / 1e9
            sweep[f"bs{bs}"] = {"us_per_call": round(t * 1e3, 2), "kv_gbs": round(gbs, 1),
                                "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
            del s2
            torch.cuda.empty_cache()
        # the ragged batch: 16 sequences with L_b ~ U[1024, 16384], with the
        # balanced split (chosen on the device from the lengths) and, for
        # comparison, the automatic split sized from the longest context
        lens = I.draw_ctx_lens("qwen3_8b_ragged16", seed=0, batch=16)
        layers = max(2, math.ceil(1.0 * 2**30 / (int(sum(lens)) * 4096)))
        ts = {}
        for name, sp in (("balanced", ob.SPLIT_BALANCED), ("automatic", 0)):
            s2 = Step(ob, I, torch, 16, lens, layers, sp, seed=1)
            ts[name] = 0.5 * (attn_only_ms(torch, s2, ob.DIFF_BIDIR, use_graph, iters=10) +
                              attn_only_ms(torch, s2, ob.AR_CAUSAL, use_graph, iters=10))
            kv = s2.kv_bytes_call
            del s2
            torch.cuda.empty_cache()
        t = ts["balanced"]
        gbs = kv / (t * 1e-3) / 1e9
        sweep["ragged16"] = {"us_per_call": round(t * 1e3, 2), "kv_gbs": round(gbs, 1),
                             "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "cached_tokens": int(sum(lens)),
                             "max_ctx": int(max(lens)), "split": "balanced",
                             "automatic_split_us_per_call": round(ts["automatic"] * 1e3, 2)}
        step = None

    longctx = None
    if not args.no_long_context:
        log("long-context step")
        step = None
        torch.cuda.empty_cache()
        s5 = Step(ob, I, torch, 4, 32768, 36, 0, seed=0, workload="qwen3_8b_32k_b4")
        s5.run()
        torch.cuda.synchronize()
        committed = int(torch.clamp(s5.acc + 1, max=s5.K).sum().item())
        rep5 = capture(torch, s5.run) if use_graph else s5.run
        ms5 = time_region(torch, rep5, 5, 2)
        kv5 = 2 * 36 * s5.kv_bytes_call
        longctx = {"workload": "qwen3_8b_32k_b4 step: B4 Hq32/Hkv8 D128 ctx32768 K32, 36 layers x (DIFF_BIDIR + "
                               "AR_CAUSAL) + accept(V=151936) + kv_append into 36 layers",
                   "us_per_step": round(ms5 * 1e3, 1), "kv_bytes_per_step": kv5,
                   "kv_gbs": round(kv5 / (ms5 * 1e-3) / 1e9, 1),
                   "frac_hbm": round(kv5 / (ms5 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "committed_tokens_per_step": committed,
                   "committed_tokens_per_s": round(committed / (ms5 * 1e-3), 1)}
        del s5, rep5
        torch.cuda.empty_cache()

    conf2 = None
    if not args.no_config2:
        log("config 2 (Qwen3-1.7B attention shape)")
        step = None
        torch.cuda.empty_cache()
        conf2 = config2_timing(torch, ob, I, use_graph)

    sample = None
    if not args.no_sample:
        log("sampled consensus")
        step = None
        torch.cuda.empty_cache()
        sample = sample_accept_timing(torch, ob, I, use_graph)

    lmhead = None
    if not args.no_lm_head:
        log("lm head")
        step = None
        torch.cuda.empty_cache()
        lmhead = lm_head_timing(torch, ob, I, use_graph)

    pre = None
    if not args.no_prefill:
        log("prefill")
        step = None
        torch.cuda.empty_cache()
        pre = prefill_timing(torch, ob, I, use_graph)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline")
        s1 = step if step is not None else Step(ob, I, torch, args.batch, args.ctx, 1, args.split_tokens)
        cpu = cpu_baseline(s1, I, args.cpu_seconds)
        if not args.no_long_context:
            log("cpu baseline: one layer of the long-context step")
            cpu["long_context_step"] = cpu_baseline_long(I, torch)

    line = {"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"qwen3_8b_8k step: B{args.batch} Hq32/Hkv8 D128 ctx{args.ctx} K32, "
                                   f"{args.layers} layers x (DIFF_BIDIR + AR_CAUSAL) + accept(V=151936) + "
                                   f"kv_append into {args.layers} layers",
                       "batch": args.batch, "ctx": args.ctx, "block_k": 32, "layers": args.layers,
                       "graph": use_graph, "parallelism": "none (1 GPU)"},
            "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "roofline": roof, "cpu_baseline": cpu, "sweep": sweep or None, "long_context_step": longctx,
            "config2": conf2, "greedy_accept": accept,
            "sample_accept": sample, "lm_head": lmhead, "prefill": pre}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
