// Host-side argument checks shared by the C entry points.  They run before
// any HIP call, so every error status can be produced without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "orthrus.h"

namespace orthrus {

// Every tensor the kernels move as 16-byte units (q, out, caches, block K/V)
// must start on a 16-byte boundary, arrays of device addresses on an 8-byte
// one and every int32 array on a 4-byte one.  NULL pointers pass (optional
// outputs).
template <size_t N, typename... P>
inline bool aligned_to(P... p) {
  return ((reinterpret_cast<uintptr_t>(p) % N == 0) && ...);
}
template <typename... P>
inline bool aligned16(P... p) {
  return aligned_to<16>(p...);
}
template <typename... P>
inline bool aligned4(P... p) {
  return aligned_to<4>(p...);
}

inline orthrus_status validate_desc(const orthrus_attn_desc* d) {
  if (!d) return ORTHRUS_ERR_NULL;
  if (d->batch < 1 || d->block_k < 1 || d->block_k > 32 || d->n_q_heads < 1 || d->n_kv_heads < 1 ||
      d->max_pages_per_seq < 1 || d->num_pages < 1 || d->max_ctx_len < 0)
    return ORTHRUS_ERR_SHAPE;
  if (d->n_q_heads % d->n_kv_heads != 0) return ORTHRUS_ERR_SHAPE;
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return ORTHRUS_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return ORTHRUS_ERR_UNSUPPORTED;
  if (d->page_size != 16) return ORTHRUS_ERR_UNSUPPORTED;
  if (d->dtype != ORTHRUS_BF16 && d->dtype != ORTHRUS_F32) return ORTHRUS_ERR_UNSUPPORTED;
  if ((long)d->max_ctx_len + d->block_k > (long)d->max_pages_per_seq * d->page_size) return ORTHRUS_ERR_SHAPE;
  if ((long)d->max_ctx_len + d->block_k > (1L << 30)) return ORTHRUS_ERR_SHAPE;
  if (d->split_tokens != ORTHRUS_SPLIT_BALANCED &&
      (d->split_tokens < 0 || d->split_tokens % 64 != 0 || d->split_tokens > 8192))
    return ORTHRUS_ERR_SHAPE;
  if (d->softmax_scale != d->softmax_scale) return ORTHRUS_ERR_SHAPE;  // NaN
  return ORTHRUS_OK;
}

// orthrus_block_attn with the cache policy of the context K/V stream chosen
// by the caller: kv_read_once streams it with the nontemporal hint (a decode
// call reads each byte once); callers that re-read the same K/V across
// launches in quick succession (the chunks of a prefill) pass false.  mode
// is checked here (an orthrus_mode value, else ORTHRUS_ERR_SHAPE).
// pair_chunks > 0 marks a prefill's virtual batch (pair_chunks 32-row chunks
// per sequence, chunk j after L_b + 32 j cached tokens, the prompt as the
// block keys): on the streaming path its AR_CAUSAL call runs the pair
// kernel, one work-group per two consecutive chunks.
orthrus_status block_attn_run(const void* q, const void* k_cache, const void* v_cache, const void* k_blk,
                              const void* v_blk, const int32_t* page_table, const int32_t* ctx_lens,
                              int32_t mode, void* out, const orthrus_attn_desc* desc, void* workspace,
                              size_t workspace_bytes, void* stream, bool kv_read_once, int pair_chunks = 0);

}  // namespace orthrus
