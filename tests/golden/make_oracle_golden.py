"""Write tests/golden/tiny_fp32_oracle.txt: the oracle's results on the
seeded tiny fp32 workload (both attention modes, the greedy consensus with
drafts agreeing on 12 positions, and the append), so that a later change to
the oracle's arithmetic shows up as a difference.  Calls only the oracle and
the seeded input generators.

    python tests/golden/make_oracle_golden.py
"""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from diffusion_drafted_verification_amd import inputs as I  # noqa: E402
from oracle import orthrus_oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32_oracle.txt")


def summarise():
    """Name -> value lines of the tiny workload's oracle results."""
    inp = I.make_attn_inputs("tiny_fp32")
    lines = {}
    for name, mode in (("diff", O.DIFF_BIDIR), ("ar", O.AR_CAUSAL)):
        out = O.block_attn(inp.q, inp.k_cache, inp.v_cache, inp.k_blk, inp.v_blk, inp.page_table, inp.ctx_lens, mode)
        lines[f"attn_{name}_sum"] = f"{out.sum():.12e}"
        lines[f"attn_{name}_abs_sum"] = f"{np.abs(out).sum():.12e}"
        lines[f"attn_{name}_row0_head0_first4"] = " ".join(f"{x:.12e}" for x in out[0, 0, 0, :4])
    logits, _ = I.make_logits(1, 32, 1024, seed=0, workload="tiny_fp32")
    g = O.greedy_argmax(logits.numpy())
    drafts = I.make_drafts(g, [12], 1024, seed=0, workload="tiny_fp32")
    acc, nxt, g2 = O.greedy_accept(logits.numpy(), drafts.numpy())
    lines["greedy_tokens"] = " ".join(str(int(t)) for t in g2[0])
    lines["accept_len"] = str(int(acc[0]))
    lines["next_token"] = str(int(nxt[0]))
    kc, vc, nl, slots = O.kv_append(inp.k_cache, inp.v_cache, inp.k_blk, inp.v_blk, inp.page_table, inp.ctx_lens, acc)
    lines["append_new_ctx_len"] = str(int(nl[0]))
    lines["append_slots"] = " ".join(str(int(x)) for x in slots[0])
    return lines


def main():
    with open(OUT, "w") as fh:
        fh.write("# Oracle results on the seeded tiny fp32 workload (written by make_oracle_golden.py).\n")
        for k, v in summarise().items():
            fh.write(f"{k} = {v}\n")


if __name__ == "__main__":
    main()
