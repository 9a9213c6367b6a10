"""MI355X (gfx950) hot path of Orthrus-style dual-view diffusion decoding.

One decode step = block attention of K block rows over a shared paged KV
cache (diffusion view: bidirectional block; AR verify view: causal block),
greedy consensus (vocab argmax + longest-prefix accept) and KV append.  The
work runs in hand-written HIP kernels behind the C ABI of include/orthrus.h;
this package holds those sources (csrc/), their build script and a thin
ctypes binding.
"""

from .orthrus import (AR_CAUSAL, DIFF_BIDIR, AttnDesc, LayerPointers, OrthrusError, block_attn,
                      block_attn_workspace_bytes, copy_probe, greedy_accept, kv_append, kv_append_layers, lib,
                      make_desc)

__all__ = ["AR_CAUSAL", "DIFF_BIDIR", "AttnDesc", "LayerPointers", "OrthrusError", "block_attn",
           "block_attn_workspace_bytes", "copy_probe", "greedy_accept", "kv_append", "kv_append_layers", "lib",
           "make_desc"]
