"""CPU oracle for paged extend attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library never reaches it, and it
shares no code with the library.

Parity status of each function (what pins it is listed in the tests):
  extend_metadata   pinned: closed-form indptrs of the ragged batch
  append_kv         pinned: gather after chunk-by-chunk append returns the
                    contiguous sequence; untouched slots keep their canary bytes
  gather_kv         pinned: same round trip, under shuffled page tables
  extend_attention  pinned: zero-score closed forms (the PR's [1,2,3,4]),
                    torch scaled_dot_product_attention on the full sequence
                    (causal, GQA, band mask), W=1 and single-key identities,
                    bitwise partition invariance; non-causal: SDPA without a
                    mask, zero-score mean of all values; explicit mask: an
                    all-keep mask and the causal mask written out reproduce the
                    unmasked results, SDPA with the same bool mask, broadcast
                    axes, rows that keep nothing give 0
  rope_rows         pinned: identity, quarter and half turns (exact), the
                    hand-worked adjacent-pair example, complex multiplication,
                    norm preservation, angle composition and the relative-
                    position identity of the dot product; the bf16 rounding
                    agrees with float32 round-to-nearest-even references
  rope_append       pinned: V copied bit for bit, K equal to rope_rows at the
                    absolute position, chunk-by-chunk equal to one full call
"""
from .paged_attention import (append_kv, extend_attention, extend_metadata, gather_kv,  # noqa: F401
                               visible_range)
from .rope import positions_of, rope_append, rope_rows, rotate_pairs, round_to_bf16_bits  # noqa: F401
