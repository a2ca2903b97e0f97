"""fp64 CPU oracle for exact attention -- test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package. The product path (the HIP library and its Python binding) never imports,
calls or falls back to it, and this package imports nothing from the product path.

What it computes, with the passages it follows:

* ``attention``: the definition of self-attention, O = softmax(scale * Q K^T) V, evaluated the
  slow, materialising way (score matrix S, then the row softmax P, then P V) in float64.
  Pages: "Flash Attention" (14cs17 notes), sections "Prerequisites" and "Standard Attention
  Memory Analysis" (steps 1-3 and Theorem 1); xspy "FlashAttention and chunked prefill
  mechanics", section 1.
* ``attention_rows``: the same definition for selected query rows only, for full-size checks.
* ``flash_forward`` / ``merge``: the tiled algorithm of the "Flash Attention Algorithm" section
  with the online-softmax update of Theorem 2 (equations (1)-(3), lost from the extracted page
  and reconstructed from the proof sentence and the xspy update rule), in float64. It exists to
  pin the definition against the pages' claim that tiling is exact.
* ``scalar``: pure-Python (math.fsum) brute force and the two-pass online normaliser of the xspy
  page's section 3, for tiny inputs.
* ``rope``: rotary position embedding in front of the definition (the RoPE of the notes'
  "Flash Attention 2 Improvements" list): the standard tables, the exact rotation, the rounded
  fp32 rotation of the reading, per-sequence positions, and ``attention_rope``.
* ``attention_backward``: the exact gradients dQ, dK, dV of the definition (the chain rule through
  the materialised softmax), which the recomputing backward pass of the notes' Pitfall 3 and
  the FromZero2AI page's mechanism 3 must reproduce.

Every function here is pinned by tests under ``-m "not gpu"`` (worked examples, closed forms,
invariants, a library routine, brute force); none is "parity unpinned". One constant is an
empirical reading: the FP8 matrix instruction's summation error in ``fp8`` (its docstring says
how it was measured), which the FP8 score and LSE bounds scale with.
"""
from .definition import (attention, attention_rows, kv_head, score_matrix_bytes,
                        softmax_rows_with_lse)
from .online import flash_forward, merge
from .backward import (attention_backward, attention_backward_dq_rows,
                       attention_backward_kv_rows, output_gradient_rowsum,
                       softmax_jacobian_product)
from . import rope, scalar

__all__ = [
    "attention",
    "attention_rows",
    "kv_head",
    "score_matrix_bytes",
    "softmax_rows_with_lse",
    "flash_forward",
    "merge",
    "scalar",
    "rope",
    "attention_backward",
    "attention_backward_dq_rows",
    "attention_backward_kv_rows",
    "output_gradient_rowsum",
    "softmax_jacobian_product",
]
