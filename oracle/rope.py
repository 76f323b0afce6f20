"""CPU oracle for rotary position embedding fused with the KV append.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports, links or runs this
module; only the tests do. It shares no code with the HIP path.

What it computes, from the pages:

* AstrAI compare v1.3.12..925cbed, ``csrc/kernels/rotary_emb.cu``
  (``rotary_emb``): bf16 rows laid out [batch, seq_len, heads, head_dim] are
  rotated with an fp32 table ``freqs_cis`` of shape [batch, seq_len,
  head_dim/2, 2] that holds (cos, sin) for each pair of head dimensions; the
  output has the input's type and shape.
* Same page, the CUDA backend's prefill path: the new K/V rows of a step are
  written into the cache slots of their positions, as the attention oracle's
  ``append_kv`` does.
* AReno PR #642, "What does this PR do?": a later chunk's rows sit at absolute
  positions P + i behind the request's cached prefix.

Readings where the pages are silent (each also listed in the design notes):

* The kernel body is not on the page. Pair j is elements 2j and 2j+1 of a head
  row, read as the complex number x[2j] + i x[2j+1] and multiplied by
  cos + i sin of table entry j: (a, b) -> (a cos - b sin, a sin + b cos). The
  table's [head_dim/2][2] layout and its name (cos + i sin per pair) fix one
  angle per adjacent pair.
* The table is indexed by absolute position (row P + i for chunk row i of a
  request with prefix P), so every chunk of a prompt rotates its rows exactly
  as a single full prefill would; every query head and every KV head of a
  token uses the same table row.
* V rows are not rotated. The result is rounded once to the storage type
  (round to nearest, ties to even).

Arithmetic is in float64; rounding to bf16 is written out here (no shared
helper).
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np


def rotate_pairs(x: np.ndarray, cs: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs of the last axis of ``x`` (float64, even length D)
    by ``cs`` (float64 [..., D/2, 2] = cos, sin), broadcast over leading axes."""
    a, b = x[..., 0::2], x[..., 1::2]
    c, s = cs[..., 0], cs[..., 1]
    out = np.empty(x.shape, dtype=np.float64)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 (8 significant bits, ties to even) of float64 values, as
    uint16 bit patterns. Finite inputs only (the rotation of finite data)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.float64)
    nz = x != 0
    mant, exp = np.frexp(x[nz])                 # x = mant * 2**exp, 0.5 <= |mant| < 1
    q = np.maximum(exp - 8, -133)                # spacing 2**q of bf16 values near x (subnormals: 2**-133)
    step = np.ldexp(1.0, q)
    out[nz] = np.rint(x[nz] / step) * step       # np.rint rounds halves to even
    bits32 = out.astype(np.float32).view(np.uint32)   # exact: out holds a bf16 value
    return (bits32 >> 16).astype(np.uint16) | np.where(np.signbit(x), np.uint16(0x8000), np.uint16(0))


def _to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (stored.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return stored.astype(np.float64)


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16_bits(x)
    return x.astype(np.float32)


def rope_rows(x: np.ndarray, positions: Sequence[int], table: np.ndarray, dtype: str) -> np.ndarray:
    """Rotate rows ``x`` [T, heads, D] (storage: bf16 bits or float32) at
    absolute ``positions`` [T] with ``table`` [table_len, D/2, 2] (float32
    cos, sin). Returns the rotated rows in storage form."""
    pos = np.asarray(positions, dtype=np.int64)
    cs = np.asarray(table, dtype=np.float64)[pos][:, None, :, :]   # [T, 1, D/2, 2]: one row per token
    return _to_storage(rotate_pairs(_to_f64(x, dtype), cs), dtype)


def positions_of(prefix_lens: Sequence[int], chunk_lens: Sequence[int]) -> np.ndarray:
    """Absolute position P_b + i of every new row, in request order."""
    return np.concatenate([np.arange(int(p), int(p) + int(l), dtype=np.int64)
                           for p, l in zip(prefix_lens, chunk_lens)] or [np.zeros(0, np.int64)])


def rope_append(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, table: np.ndarray,
                k_pool: np.ndarray, v_pool: np.ndarray, page_table: np.ndarray,
                prefix_lens: Sequence[int], chunk_lens: Sequence[int], dtype: str,
                req_pool_indices: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Rotated q [total_q, Hq, D] and copies of the pools with each new token's
    rotated K and unrotated V written to the slot of its position (page
    P_b+i // ps of the request's page-table row, offset P_b+i % ps)."""
    pos = positions_of(prefix_lens, chunk_lens)
    q_rot = rope_rows(q, pos, table, dtype)
    k_rot = rope_rows(k_new, pos, table, dtype)
    k_out, v_out = k_pool.copy(), v_pool.copy()
    ps = k_pool.shape[1]
    t = 0
    for b in range(len(chunk_lens)):
        row = page_table[int(req_pool_indices[b]) if req_pool_indices is not None else b]
        for i in range(int(chunk_lens[b])):
            p = int(prefix_lens[b]) + i
            page, off = int(row[p // ps]), p % ps
            k_out[page, off] = k_rot[t]
            v_out[page, off] = v_new[t]
            t += 1
    return q_rot, k_out, v_out

