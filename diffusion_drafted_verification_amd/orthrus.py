"""Python binding of the gfx950 C-ABI library (include/orthrus.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of liborthrus_gfx950.so.  PyTorch provides device memory and the
current stream.  There is no CPU fallback: if the library is missing or the
tensors are not on a GPU, the calls raise.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch  # imported before the library so both share torch's HIP runtime

DIFF_BIDIR = 0
AR_CAUSAL = 1
BF16 = 0
F32 = 1
SPLIT_BALANCED = -1   # split_tokens: chosen on the device from ctx_lens (ragged batches)
PAGE_SIZE = 16

LIB_NAME = "liborthrus_gfx950.so"
# the in-tree library; ORTHRUS_LIBRARY may name another build of it (the
# sanitized host-only build that the CPU validation tests run against)
LIB_PATH = os.environ.get("ORTHRUS_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

STATUS = {0: "ok", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_UNSUPPORTED", 4: "ERR_WORKSPACE", 5: "ERR_LAUNCH"}

# every entry point include/orthrus.h declares, with its ctypes signature
_vp, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float


class AttnDesc(ctypes.Structure):
    """orthrus_attn_desc"""
    _fields_ = [("batch", _i32), ("block_k", _i32), ("n_q_heads", _i32), ("n_kv_heads", _i32),
                ("head_dim", _i32), ("page_size", _i32), ("max_pages_per_seq", _i32), ("num_pages", _i32),
                ("max_ctx_len", _i32), ("dtype", _i32), ("softmax_scale", _f32), ("split_tokens", _i32)]


_DESC_P = ctypes.POINTER(AttnDesc)
SIGNATURES = {
    "orthrus_abi_version": (_i32, []),
    "orthrus_status_str": (ctypes.c_char_p, [_i32]),
    "orthrus_block_attn_workspace_bytes": (_sz, [_DESC_P]),
    "orthrus_block_attn_split_tokens": (_i32, [_DESC_P]),
    "orthrus_block_attn": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _DESC_P, _vp, _sz, _vp]),
    "orthrus_block_attn_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _DESC_P, _vp]),
    "orthrus_greedy_accept_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "orthrus_greedy_accept": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "orthrus_sample_accept_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "orthrus_sample_accept": (_i32, [_vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "orthrus_lm_head_packed_bytes": (_sz, [_i32, _i32]),
    "orthrus_lm_head_pack_weight": (_i32, [_vp, _vp, _i32, _i32, _vp]),
    "orthrus_lm_head_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "orthrus_lm_head_denoise_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "orthrus_lm_head_denoise_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz,
                                            _vp]),
    "orthrus_lm_head_argmax": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "orthrus_lm_head_greedy_accept": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz, _vp]),
    "orthrus_kv_append": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _DESC_P, _vp]),
    "orthrus_kv_append_layers": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _DESC_P, _vp]),
    "orthrus_prefill_workspace_bytes": (_sz, [_DESC_P, _i32]),
    "orthrus_prefill_chunks_per_workgroup": (_i32, [_DESC_P, _i32]),
    "orthrus_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _DESC_P, _vp, _sz, _vp]),
    "orthrus_copy_probe": (_i32, [_vp, _vp, _sz, _vp]),
    "orthrus_read_probe": (_i32, [_vp, _sz, _vp, _sz, _vp]),
}

_lib = None
_lock = threading.Lock()


class OrthrusError(RuntimeError):
    pass


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise OrthrusError(f"{LIB_PATH} is missing: build it with "
                                       "`python -m diffusion_drafted_verification_amd.build`")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def _check(status, what):
    if status != 0:
        msg = lib().orthrus_status_str(status).decode()
        raise OrthrusError(f"{what}: {STATUS.get(status, status)} ({msg})")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _gpu(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise OrthrusError("tensors must be on a GPU (there is no CPU path)")
        if not t.is_contiguous():
            raise OrthrusError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise OrthrusError("tensors must be on one device")
    return dev


_DTYPES = {torch.bfloat16: BF16, torch.float32: F32}


def make_desc(q, k_cache, page_table, max_ctx_len=None, softmax_scale=None, split_tokens=0):
    """orthrus_attn_desc for tensors q [B,K,Hq,D], k_cache [pages,Hkv,P,D] and
    page_table [B, max_pages].  max_ctx_len defaults to the table capacity
    minus K (always a valid bound; pass the true maximum to size the launch
    tightly)."""
    B, K, Hq, D = q.shape
    n_pages, Hkv, P, D2 = k_cache.shape
    if D2 != D or P != PAGE_SIZE:
        raise OrthrusError("k_cache must be [num_pages, Hkv, 16, D]")
    if q.dtype not in _DTYPES:
        raise OrthrusError(f"unsupported dtype {q.dtype}")
    max_pages = page_table.shape[1]
    if max_ctx_len is None:
        max_ctx_len = max_pages * P - K
    return AttnDesc(B, K, Hq, Hkv, D, P, max_pages, n_pages, int(max_ctx_len), _DTYPES[q.dtype],
                    float(softmax_scale) if softmax_scale else 0.0, int(split_tokens))


_workspaces = {}   # (device, kind, stream) -> the cached workspace of that stream
_retired = []      # workspaces replaced by larger ones: a graph captured earlier may still address them


def workspace(device, nbytes, kind, stream=None):
    """A workspace of at least nbytes for calls of one kind on one stream,
    zero-filled when it is made.

    Calls that share a workspace must be ordered on one stream, so the cache
    is per (device, kind, stream).  A workspace that has to grow is replaced
    but never freed: a HIP graph captured earlier may still hold its address.
    Sizes grow at least twofold, so few buffers are ever retired.  No
    workspace is made during graph capture (the zero fill would become part
    of the graph): run the call once on the capturing stream before capture,
    or pass ws= explicitly."""
    s = torch.cuda.current_stream(device) if stream is None else stream
    key = (str(device), kind, s.cuda_stream)
    ws = _workspaces.get(key)
    if ws is not None and ws.numel() >= nbytes:
        return ws
    if torch.cuda.is_current_stream_capturing():
        raise OrthrusError(f"no {kind} workspace of {nbytes} bytes for the capturing stream: run the call once "
                           "on that stream before capture, or pass ws=")
    size = max(nbytes, 256, 2 * ws.numel() if ws is not None else 0)
    new = torch.zeros(size, dtype=torch.uint8, device=device)
    if ws is not None:
        _retired.append(ws)
    _workspaces[key] = new
    return new


def block_attn_workspace_bytes(desc):
    return lib().orthrus_block_attn_workspace_bytes(ctypes.byref(desc))


def block_attn(q, k_cache, v_cache, k_blk, v_blk, page_table, ctx_lens, mode, out=None, *, max_ctx_len=None,
               softmax_scale=None, split_tokens=0, ws=None, stream=None):
    """orthrus_block_attn: out [B, K, Hq, D] in q's dtype.

    split_tokens: 0 sizes the context split from max_ctx_len (equal lengths),
    SPLIT_BALANCED lets the kernels choose it from ctx_lens (ragged batches),
    and a multiple of 64 in [64, 8192] fixes it."""
    dev = _gpu(q, k_cache, v_cache, k_blk, v_blk, page_table, ctx_lens, out)
    if not (q.dtype == k_cache.dtype == v_cache.dtype == k_blk.dtype == v_blk.dtype):
        raise OrthrusError("q, caches and block K/V must share one dtype")
    if page_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32:
        raise OrthrusError("page_table and ctx_lens must be int32")
    B, K, Hq, D = q.shape
    if tuple(k_blk.shape) != (B, K, k_cache.shape[1], D) or v_blk.shape != k_blk.shape \
            or v_cache.shape != k_cache.shape or tuple(ctx_lens.shape) != (B,) or page_table.shape[0] != B:
        raise OrthrusError("inconsistent shapes")
    desc = make_desc(q, k_cache, page_table, max_ctx_len, softmax_scale, split_tokens)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise OrthrusError("out must match q")
    need = lib().orthrus_block_attn_workspace_bytes(ctypes.byref(desc))
    if ws is None and need:
        ws = workspace(dev, need, "attn", stream)
    st = lib().orthrus_block_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_blk), _ptr(v_blk),
                                  _ptr(page_table), _ptr(ctx_lens), int(mode), _ptr(out), ctypes.byref(desc),
                                  _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream))
    _check(st, "orthrus_block_attn")
    return out


STATIC_SCRATCH_BYTES = 32 << 20   # ORTHRUS_STATIC_SCRATCH_BYTES


def block_attn_noalloc(q, k_cache, v_cache, k_blk, v_blk, page_table, ctx_lens, mode, out, *, max_ctx_len=None,
                       softmax_scale=None, split_tokens=0, stream=None):
    """orthrus_block_attn_noalloc: block_attn into a caller-provided `out`,
    with the split partials in the library's fixed per-GPU scratch array
    (nothing is allocated)."""
    _gpu(q, k_cache, v_cache, k_blk, v_blk, page_table, ctx_lens, out)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise OrthrusError("out must match q")
    desc = make_desc(q, k_cache, page_table, max_ctx_len, softmax_scale, split_tokens)
    st = lib().orthrus_block_attn_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_blk), _ptr(v_blk),
                                          _ptr(page_table), _ptr(ctx_lens), int(mode), _ptr(out),
                                          ctypes.byref(desc), _stream(stream))
    _check(st, "orthrus_block_attn_noalloc")
    return out


def greedy_accept(ar_logits, draft_tokens, *, want_ar_tokens=True, ws=None, stream=None):
    """orthrus_greedy_accept: returns (accept_len [B], next_token [B],
    ar_tokens [B, K] or None), int32 on the logits' device."""
    dev = _gpu(ar_logits, draft_tokens)
    if ar_logits.dtype != torch.float32 or draft_tokens.dtype != torch.int32:
        raise OrthrusError("ar_logits must be fp32 and draft_tokens int32")
    B, K, V = ar_logits.shape
    if tuple(draft_tokens.shape) != (B, K):
        raise OrthrusError("draft_tokens must be [B, K]")
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    g = torch.empty((B, K), dtype=torch.int32, device=dev) if want_ar_tokens else None
    need = lib().orthrus_greedy_accept_workspace_bytes(B, K, V)
    if ws is None:
        ws = workspace(dev, need, "accept", stream)
    st = lib().orthrus_greedy_accept(_ptr(ar_logits), _ptr(draft_tokens), _ptr(acc), _ptr(nxt), _ptr(g),
                                     B, K, V, _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "orthrus_greedy_accept")
    return acc, nxt, g


def sample_accept(ar_logits, draft_logits, draft_tokens, u_accept, u_resample, temperature, *, ws=None,
                  stream=None):
    """orthrus_sample_accept: returns (accept_len [B], next_token [B]), int32
    on the logits' device."""
    dev = _gpu(ar_logits, draft_logits, draft_tokens, u_accept, u_resample)
    if (ar_logits.dtype != torch.float32 or draft_logits.dtype != torch.float32
            or u_accept.dtype != torch.float32 or u_resample.dtype != torch.float32
            or draft_tokens.dtype != torch.int32):
        raise OrthrusError("logits and uniforms must be fp32, draft_tokens int32")
    B, K, V = ar_logits.shape
    if tuple(draft_logits.shape) != (B, K, V) or tuple(draft_tokens.shape) != (B, K) \
            or tuple(u_accept.shape) != (B, K) or tuple(u_resample.shape) != (B,):
        raise OrthrusError("draft_logits [B, K, V], draft_tokens and u_accept [B, K], u_resample [B]")
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    need = lib().orthrus_sample_accept_workspace_bytes(B, K, V)
    if ws is None:
        ws = workspace(dev, need, "sample", stream)
    st = lib().orthrus_sample_accept(_ptr(ar_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(u_accept),
                                     _ptr(u_resample), float(temperature), _ptr(acc), _ptr(nxt), B, K, V,
                                     _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "orthrus_sample_accept")
    return acc, nxt


class PackedLmHead:
    """An LM-head weight [V, H] bf16 repacked once (orthrus_lm_head_pack_weight)
    into the layout the LM-head calls stream."""

    def __init__(self, weight, stream=None):
        dev = _gpu(weight)
        if weight.dtype != torch.bfloat16 or weight.dim() != 2:
            raise OrthrusError("weight must be bf16 [V, H]")
        self.vocab, self.hidden = int(weight.shape[0]), int(weight.shape[1])
        nbytes = lib().orthrus_lm_head_packed_bytes(self.hidden, self.vocab)
        if nbytes == 0:
            raise OrthrusError("unsupported LM-head shape (H must be a multiple of 256 in [256, 65536])")
        self.packed = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev)
        st = lib().orthrus_lm_head_pack_weight(_ptr(weight), _ptr(self.packed), self.hidden, self.vocab,
                                               _stream(stream))
        _check(st, "orthrus_lm_head_pack_weight")


def _lm_check(hidden, head):
    if not isinstance(head, PackedLmHead):
        raise OrthrusError("the LM-head calls take a PackedLmHead")
    if hidden.dtype != torch.bfloat16 or hidden.shape[-1] != head.hidden:
        raise OrthrusError("hidden must be bf16 [..., H] with the head's H")


def lm_head_argmax(hidden, head, *, want_max=False, ws=None, stream=None):
    """orthrus_lm_head_argmax over hidden [..., H] with a PackedLmHead:
    returns (tokens [...] int32, max_logits [...] fp32 or None)."""
    dev = _gpu(hidden, head.packed)
    _lm_check(hidden, head)
    H, V = head.hidden, head.vocab
    weight = head.packed
    rows = hidden.numel() // H
    tok = torch.empty(hidden.shape[:-1], dtype=torch.int32, device=dev)
    mx = torch.empty(hidden.shape[:-1], dtype=torch.float32, device=dev) if want_max else None
    need = lib().orthrus_lm_head_workspace_bytes(rows, H, V)
    if ws is None:
        ws = workspace(dev, need, "lm_head", stream)
    st = lib().orthrus_lm_head_argmax(_ptr(hidden), _ptr(weight), _ptr(tok), _ptr(mx), rows, H, V, _ptr(ws),
                                      ws.numel(), _stream(stream))
    _check(st, "orthrus_lm_head_argmax")
    return tok, mx


def lm_head_greedy_accept(hidden, head, draft_tokens, *, want_ar_tokens=True, ws=None, stream=None):
    """orthrus_lm_head_greedy_accept over the AR view's hidden states
    [B, K, H] with a PackedLmHead: returns (accept_len [B], next_token [B],
    ar_tokens [B, K] or None)."""
    dev = _gpu(hidden, head.packed, draft_tokens)
    _lm_check(hidden, head)
    if hidden.dim() != 3 or draft_tokens.dtype != torch.int32 or tuple(draft_tokens.shape) != hidden.shape[:2]:
        raise OrthrusError("hidden must be [B, K, H] and draft_tokens int32 [B, K]")
    B, K, H = hidden.shape
    V = head.vocab
    weight = head.packed
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    g = torch.empty((B, K), dtype=torch.int32, device=dev) if want_ar_tokens else None
    need = lib().orthrus_lm_head_workspace_bytes(B * K, H, V)
    if ws is None:
        ws = workspace(dev, need, "lm_head", stream)
    st = lib().orthrus_lm_head_greedy_accept(_ptr(hidden), _ptr(weight), _ptr(draft_tokens), _ptr(acc), _ptr(nxt),
                                             _ptr(g), B, K, H, V, _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "orthrus_lm_head_greedy_accept")
    return acc, nxt, g


def kv_append(k_cache, v_cache, k_blk, v_blk, page_table, ctx_lens, accept_len, *, new_ctx_lens=None,
              slots=None, want_outputs=True, max_ctx_len=None, stream=None):
    """orthrus_kv_append (in place on the caches): returns (new_ctx_lens [B],
    slots [B, K]) or (None, None) when want_outputs is False."""
    dev = _gpu(k_cache, v_cache, k_blk, v_blk, page_table, ctx_lens, accept_len)
    B, K, Hkv, D = k_blk.shape
    if want_outputs:
        if new_ctx_lens is None:
            new_ctx_lens = torch.empty(B, dtype=torch.int32, device=dev)
        if slots is None:
            slots = torch.empty((B, K), dtype=torch.int32, device=dev)
    qlike = torch.empty((B, K, Hkv, D), dtype=k_blk.dtype, device="meta")
    desc = make_desc(qlike, k_cache, page_table, max_ctx_len)
    st = lib().orthrus_kv_append(_ptr(k_cache), _ptr(v_cache), _ptr(k_blk), _ptr(v_blk), _ptr(page_table),
                                 _ptr(ctx_lens), _ptr(accept_len), _ptr(new_ctx_lens), _ptr(slots),
                                 ctypes.byref(desc), _stream(stream))
    _check(st, "orthrus_kv_append")
    return new_ctx_lens, slots


class LayerPointers:
    """Device arrays of per-layer cache and block K/V addresses for
    kv_append_layers (built once per set of tensors)."""

    def __init__(self, k_caches, v_caches, k_blks, v_blks):
        self.tensors = (list(k_caches), list(v_caches), list(k_blks), list(v_blks))
        n = len(self.tensors[0])
        if not all(len(t) == n for t in self.tensors) or n == 0:
            raise OrthrusError("one tensor of each kind per layer")
        dev = _gpu(*[t for ts in self.tensors for t in ts])
        ref = self.tensors[0][0]
        for ts in self.tensors[:2]:
            if any(t.shape != ref.shape or t.dtype != ref.dtype for t in ts):
                raise OrthrusError("all layer caches must share one shape and dtype")
        kb = self.tensors[2][0]
        for ts in self.tensors[2:]:
            if any(t.shape != kb.shape or t.dtype != ref.dtype for t in ts):
                raise OrthrusError("all layer block K/V must share one shape and the cache dtype")
        self.n_layers = n
        self.ptrs = [torch.tensor([t.data_ptr() for t in ts], dtype=torch.int64, device=dev)
                     for ts in self.tensors]


def kv_append_layers(layers, page_table, ctx_lens, accept_len, *, new_ctx_lens=None, slots=None,
                     want_outputs=True, max_ctx_len=None, stream=None):
    """orthrus_kv_append_layers over a LayerPointers set: one launch appends
    the accepted rows of every layer."""
    k0, kb0 = layers.tensors[0][0], layers.tensors[2][0]
    dev = _gpu(k0, page_table, ctx_lens, accept_len)
    B, K, Hkv, D = kb0.shape
    if want_outputs:
        if new_ctx_lens is None:
            new_ctx_lens = torch.empty(B, dtype=torch.int32, device=dev)
        if slots is None:
            slots = torch.empty((B, K), dtype=torch.int32, device=dev)
    qlike = torch.empty((B, K, Hkv, D), dtype=kb0.dtype, device="meta")
    desc = make_desc(qlike, k0, page_table, max_ctx_len)
    kp, vp, kbp, vbp = layers.ptrs
    st = lib().orthrus_kv_append_layers(_ptr(kp), _ptr(vp), _ptr(kbp), _ptr(vbp), layers.n_layers, _ptr(page_table),
                                        _ptr(ctx_lens), _ptr(accept_len), _ptr(new_ctx_lens), _ptr(slots),
                                        ctypes.byref(desc), _stream(stream))
    _check(st, "orthrus_kv_append_layers")
    return new_ctx_lens, slots


def lm_head_denoise_step(hidden, head, masked, n_unmask, *, new_masked=None, ws=None, stream=None):
    """orthrus_lm_head_denoise_step over the diffusion view's hidden states
    [B, K, H] with a PackedLmHead; masked uint8 [B, K], n_unmask int32 [B].
    Returns (tokens [B, K] int32, confidence [B, K] fp32, new_masked [B, K]
    uint8; new_masked may be `masked` itself)."""
    dev = _gpu(hidden, head.packed, masked, n_unmask, new_masked)
    _lm_check(hidden, head)
    if hidden.dim() != 3 or masked.dtype != torch.uint8 or tuple(masked.shape) != hidden.shape[:2] \
            or n_unmask.dtype != torch.int32 or tuple(n_unmask.shape) != hidden.shape[:1]:
        raise OrthrusError("hidden [B, K, H], masked uint8 [B, K], n_unmask int32 [B]")
    B, K, H = hidden.shape
    V = head.vocab
    tok = torch.empty((B, K), dtype=torch.int32, device=dev)
    conf = torch.empty((B, K), dtype=torch.float32, device=dev)
    if new_masked is None:
        new_masked = torch.empty_like(masked)
    need = lib().orthrus_lm_head_denoise_workspace_bytes(B * K, H, V)
    if ws is None:
        ws = workspace(dev, need, "lm_head_denoise", stream)
    st = lib().orthrus_lm_head_denoise_step(_ptr(hidden), _ptr(head.packed), _ptr(masked), _ptr(n_unmask),
                                            _ptr(tok), _ptr(conf), _ptr(new_masked), B, K, H, V, _ptr(ws),
                                            ws.numel(), _stream(stream))
    _check(st, "orthrus_lm_head_denoise_step")
    return tok, conf, new_masked


def prefill(q, k, v, k_cache, v_cache, page_table, ctx_lens, prompt_lens, max_prompt, out=None, *,
            new_ctx_lens=None, max_ctx_len=None, softmax_scale=None, split_tokens=0, ws=None, stream=None):
    """orthrus_prefill (writes the prompt rows into the caches in place):
    q [B, S, Hq, D], k/v [B, S, Hkv, D] with S = max_prompt rounded up to a
    multiple of 32.  Returns (out [B, S, Hq, D], new_ctx_lens [B])."""
    dev = _gpu(q, k, v, k_cache, v_cache, page_table, ctx_lens, prompt_lens, out, new_ctx_lens)
    B, S = q.shape[0], q.shape[1]
    if S != (int(max_prompt) + 31) // 32 * 32 or tuple(k.shape[:2]) != (B, S) or tuple(v.shape) != tuple(k.shape):
        raise OrthrusError("q/k/v must be [B, S, ...] with S = max_prompt rounded up to a multiple of 32")
    if page_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32 or prompt_lens.dtype != torch.int32:
        raise OrthrusError("page_table, ctx_lens and prompt_lens must be int32")
    if out is None:
        out = torch.empty_like(q)
    if new_ctx_lens is None:
        new_ctx_lens = torch.empty(B, dtype=torch.int32, device=dev)
    if max_ctx_len is None:   # the largest context the table leaves room for before the prompt
        max_ctx_len = page_table.shape[1] * PAGE_SIZE - S
    desc = make_desc(q[:, :32], k_cache, page_table, max_ctx_len, softmax_scale, split_tokens)
    need = lib().orthrus_prefill_workspace_bytes(ctypes.byref(desc), int(max_prompt))
    if ws is None:
        ws = workspace(dev, need, "prefill", stream)
    st = lib().orthrus_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                               _ptr(ctx_lens), _ptr(prompt_lens), int(max_prompt), _ptr(out), _ptr(new_ctx_lens),
                               ctypes.byref(desc), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "orthrus_prefill")
    return out, new_ctx_lens


def prefill_chunks_per_workgroup(q, k_cache, page_table, max_prompt, *, max_ctx_len=None, split_tokens=0):
    """orthrus_prefill_chunks_per_workgroup for the shape `prefill` would
    get with these arguments: 2 when one attention work-group serves two
    32-row chunks, else 1."""
    S = q.shape[1]
    if max_ctx_len is None:
        max_ctx_len = page_table.shape[1] * PAGE_SIZE - S
    desc = make_desc(q[:, :32], k_cache, page_table, max_ctx_len, None, split_tokens)
    n = lib().orthrus_prefill_chunks_per_workgroup(ctypes.byref(desc), int(max_prompt))
    if n == 0:
        raise OrthrusError("orthrus_prefill_chunks_per_workgroup: invalid shape")
    return n


def copy_probe(dst, src, stream=None):
    _gpu(dst, src)
    n = src.numel() * src.element_size()
    _check(lib().orthrus_copy_probe(_ptr(dst), _ptr(src), n, _stream(stream)), "orthrus_copy_probe")


def read_probe(src, sink, stream=None):
    """orthrus_read_probe: reads all of src once (sink >= 4 MiB receives
    meaningless XOR folds)."""
    _gpu(src, sink)
    n = src.numel() * src.element_size()
    m = sink.numel() * sink.element_size()
    _check(lib().orthrus_read_probe(_ptr(src), n, _ptr(sink), m, _stream(stream)), "orthrus_read_probe")
