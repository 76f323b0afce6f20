"""Every output row of the two largest configurations against the CPU oracle,
at full size, in the launch configuration the bench times:

* 8 requests of 6000 cached + 1000 new tokens, window 4096 (32 query / 8 KV
  heads, D = 128, 16-token pages), with prefixes of 6000 and, so that every
  append continues inside a page, 6001 + 2b;
* one mixed step: 64 one-token rows (KV 2048..32768, 8 splits) and 2 prefill
  rows of 16384 cached + 2048 new tokens (64 query / 8 KV heads).

The GPU runs each batch once (module fixture); the oracle, as it is, computes
every row of every request, in blocks of rows on a thread pool
(pkv_testlib.oracle_rows_parallel). Bar: |gpu - ref| <= 2e-2 + 1e-2 |ref|
(bf16 inputs, fp32 accumulation) on every element."""
import numpy as np
import pytest
import torch

import workloads as wl
from pkv_testlib import assert_parity, oracle_rows_parallel

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_chunked_prefill_amd as pkv
    from gpu_harness import prefill_and_attend, values_of


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    assert pkv.device_supported(torch.cuda.current_device()), "not a gfx950 device"


_OUT = {}


def gpu_out(name):
    """GPU output (float32 values) of a whole batch, computed once."""
    if name not in _OUT:
        w = {"window": lambda: wl.config4(False), "window_mid_page": lambda: wl.config4(True),
             "mixed": wl.config5}[name]()
        print(f"[full-size] GPU run of {name}: B={w.batch} total_q={w.total_q}", flush=True)
        out, cache, plan = prefill_and_attend(w)
        torch.cuda.synchronize()
        assert pkv.read_status(plan) == 0
        if name == "mixed":
            assert plan.plan.n_split_rows == 64 and plan.plan.max_splits == 8
        _OUT[name] = (w, values_of(out))
        del cache
        torch.cuda.empty_cache()
    return _OUT[name]


def compare(name, b, rows=None):
    w, got = gpu_out(name)
    qo = np.concatenate([[0], np.cumsum(w.chunk_lens)])
    L = int(w.chunk_lens[b])
    rows = list(range(L)) if rows is None else list(rows)
    ref = oracle_rows_parallel(w, b, rows)
    g = got[qo[b] + np.array(rows)]
    assert not np.isnan(g).any(), f"{name} request {b}: NaN in output"
    rep = assert_parity(g, ref, w.dtype, f"{name} request {b} rows {rows[0]}..{rows[-1]}")
    print(f"[parity] full-size {name} request {b} rows {rows[0]}..{rows[-1]} ({len(rows)} rows x {w.num_q_heads} "
          f"heads): max_abs={rep['max_abs']:.3e} max_rel={rep['max_rel']:.3e}", flush=True)


@pytest.mark.parametrize("req", range(8))
@pytest.mark.parametrize("variant", ["window", "window_mid_page"])
def test_window_every_row(variant, req):
    compare(variant, req)


@pytest.mark.parametrize("first", range(0, 64, 16))
def test_mixed_one_token_rows(first):
    for b in range(first, first + 16):
        compare("mixed", b)


@pytest.mark.parametrize("rows", [(a, a + 512) for a in range(0, 2048, 512)], ids=lambda r: f"{r[0]}-{r[1]}")
@pytest.mark.parametrize("req", [64, 65])
def test_mixed_prefill_rows(req, rows):
    compare("mixed", req, range(*rows))
