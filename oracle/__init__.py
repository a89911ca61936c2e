"""CPU oracle for the per-step batched sampler (float64, NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything here: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use it.  It shares no code with the HIP
library under ``decode_step_token_amd/``.

Pins (each in ``tests/test_oracle_pins.py``):

* ``philox``: equals ``numpy.random.Philox`` (Philox-4x64-10) block outputs.
* ``row_params``/``sample_row``: the pages' worked example (closed forms and
  draw frequency), argmax identities, the full-softmax identity against
  ``scipy.special.softmax``, exact rational top-p cut-offs, the top-k set
  against ``heapq.nsmallest``, the draw against ``numpy.searchsorted`` and a
  brute-force sweep of ``u``, the filter-order counterexample.
* ``write_tokens``: NumPy fancy-index assignment.
* ``gather_tokens`` / ``input_tuple``: NumPy fancy indexing, a write-then-gather
  round trip, and the packed positions of a hand-worked prefill + decode batch.
* ``prepare``: hand-worked batches (clamps and the None rules), and that the
  per-row routing of the prepared tensors equals that of the raw parameters.
* ``min_p_count`` (min_p in ``sample_row``): the pages' worked logits give
  the closed forms of top-k 2 at min_p 0.2; min_p 1 is argmax (all ties at
  the maximum kept); the prefix-minimum equals the literal intersection of
  the masks by brute force; the count equals the logit-space threshold
  ``x >= m + T ln(min_p)``; min_p 0 changes nothing.
* ``PagePool`` / ``paged_info`` / ``page_to_token`` / ``write_page_table``:
  the pages' page-aligned allocation test (row [0..7], free pages 6, 6, 5, a
  new page starting at a multiple of 4), their worked page count (page size
  4, cached 6, device 9: one page), and brute force over random batches
  (every position holds its own page's location plus its offset, no location
  twice).
"""
from .philox import philox4x64, request_uniform, request_word, uniform24
from .sampler_ref import (CUT_BAND, DRAW_BAND, MIN_P, MIN_P_BAND, MIN_T, RowParams, RowResult,
                          descending_order, filter_sorted, gather_tokens, input_tuple,
                          inverse_cdf, min_p_count, PagePool, page_to_token, paged_info,
                          prepare,
                          row_params, sample_batch, sample_row, widen_logits,
                          write_page_table, write_tokens)

__all__ = [
    "philox4x64", "request_uniform", "request_word", "uniform24", "CUT_BAND", "DRAW_BAND",
    "MIN_P_BAND", "min_p_count",
    "MIN_P", "MIN_T", "RowParams", "RowResult", "descending_order", "filter_sorted",
    "gather_tokens", "input_tuple", "inverse_cdf", "PagePool", "page_to_token", "paged_info",
    "prepare", "write_page_table", "row_params", "sample_batch", "sample_row", "widen_logits", "write_tokens",
]
