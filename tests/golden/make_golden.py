"""Writes the oracle regression fixtures in this folder.  It calls only ``oracle/`` and the
seeded input generator; run it (``python tests/golden/make_golden.py``) only after a change
to the oracle's arithmetic that a passage of the pages justifies.

The pages print no worked numeric example of the attention core, so nothing here is a
page-printed value: the fixtures freeze what the pinned oracle computes on the tiny
workload (two packed sequences) and on one row of 8-bit quantisation, so that a later,
unintended change to the oracle fails ``tests/test_golden.py``."""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from transformer_prefill_attention_amd import workloads as wl  # noqa: E402

ROWS = (0, 6, 7, 8, 39)   # first, last of sequence 0; first, ..., last of sequence 1


def tiny_case():
    w = wl.CONFIGS["tiny"].with_(seq_lens=(7, 33))
    return w, wl.make_inputs(w)


def tiny_qk_prep_attn():
    w, x = tiny_case()
    return oracle.qk_prep_attn(x.q, x.k, x.v, x.wq, x.wk, n_head=w.n_head,
                               n_head_kv=w.n_head_kv, head_dim=w.head_dim,
                               rope_dim=w.rope_dim, rope_freq_base=w.rope_freq_base,
                               rms_eps=float(np.float32(w.rms_eps)), scale=w.softmax_scale,
                               seq_offsets=w.seq_offsets, rows=np.array(ROWS))


def quant_row():
    x = np.linspace(-3.0, 2.0, 64).astype(np.float32) ** 3
    return x, oracle.quant_rows(x, 64)


def main():
    out = tiny_qk_prep_attn()
    with open(os.path.join(HERE, "tiny_qk_prep_attn.txt"), "w") as f:
        f.write("# oracle.qk_prep_attn on the tiny workload with sequences (7, 33): QK-norm,\n"
                "# NeoX RoPE and causal GQA attention (memra-engine 0.130.0 src/forward.rs,\n"
                "# Model::forward, QK-norm, RoPE and SDPA blocks), f64.  Rows of the output\n"
                f"# [T, n_head*head_dim], one per line: {ROWS}.  Written by make_golden.py.\n")
        for r in out:
            f.write(" ".join(f"{v:.17g}" for v in r) + "\n")
    x, (codes, scales, deq) = quant_row()
    with open(os.path.join(HERE, "quant_row.txt"), "w") as f:
        f.write("# oracle.quant_rows of one 64-value row, x = linspace(-3, 2, 64)^3 in f32\n"
                "# (needle-core v3/model.rs, quant_rows / quantize_rows): the scale, then the\n"
                "# 64 codes.  Written by make_golden.py.\n")
        f.write(f"{float(scales[0]):.9g}\n")
        f.write(" ".join(str(int(c)) for c in codes) + "\n")


if __name__ == "__main__":
    main()
