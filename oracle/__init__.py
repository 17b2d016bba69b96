"""CPU float64 oracle for decode attention over a compressed KV cache.

TEST INFRASTRUCTURE ONLY: tests/, the package's smoke check and the CPU
baseline leg of bench.py are the only code that may import it.  It shares no
code with the HIP library and never calls it.

Parity status of each function (what pins it is in tests/test_oracle_*.py):
  share_map       pinned (exhaustive enumeration, page's memory figures)
  attention       pinned (closed forms, brute force, invariants)
  decode_attention pinned (GQA grouping, all-leaders reduction)
  value_range     pinned (hand values, invariances, torch float32 rounding)
  window_score    pinned (closed-form causal case, row sums, brute force)
  philox4         pinned (64-bit instance equals numpy's Philox4x64-10)
  exp_variate     pinned (end points, exponential law)
  select          pinned (invariants, top-K reduction, exact 8-token law)
  compact         pinned (gather identity, restricted attention)
  run_decode      pinned through the functions above and the schedule count
  dkv.gaussian_bf16  pinned (Box-Muller word roles in closed form, bf16
                  round-to-nearest-even cases, normal law)
  dkv.dkv_score   pinned (QR and SVD leverage, closed two-row form,
                  subspace invariance, rank deficiency, isolated rows)
  quant.*         pinned (hand values with half-even rounding, the rounding
                  bound, power-of-two scalings, the protection rule, exact
                  cases equal to plain attention, the large-range-row claim)
  ragged.*        pinned (short-window scores by brute force and row sums,
                  reduction to the uniform trajectory and to a batch of one,
                  sequence independence, the length schedule)
  xkv.*           pinned (the page's storage formula, exact reconstruction at
                  full rank and for shared cross-layer structure, a closed
                  rank-1 case, optimality against other subspaces, landmarks
                  and chunk scores by brute force, the selection rule, the
                  exact merge of two attention parts)
End-to-end model quality (does the eviction keep accuracy?) is parity
unpinned: it needs trained weights and datasets that are not available.
"""
from .philox import philox4, philox4x32_10, seed_key, mulhilo
from . import dkv, quant, ragged, xkv
from .kvc_oracle import (
    share_map, append_row, attention, decode_attention, value_range,
    window_score, philox_word0, exp_variate, select, select_detail, compact,
    eviction_due, run_decode,
)

__all__ = [
    "philox4", "philox4x32_10", "seed_key", "mulhilo", "share_map",
    "append_row", "attention", "decode_attention", "value_range",
    "window_score", "philox_word0", "exp_variate", "select", "select_detail",
    "compact", "eviction_due", "run_decode", "dkv", "quant", "ragged", "xkv",
]
