"""paged_extend_attn_noalloc keeps the split partials in the library's static
per-device scratch instead of a caller workspace. Two calls in a row, the
second with a smaller batch, each against paged_extend_attn with a workspace
on the same plan and inputs: the outputs must be equal bit for bit (same
kernels), and the smaller batch is also held to the oracle's bar."""
import numpy as np
import pytest
import torch

import workloads as wl
from pkv_testlib import assert_parity, oracle_out, oracle_pools

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_chunked_prefill_amd as pkv
    from gpu_harness import DeviceCache, upload_q, values_of


def _step(w):
    cache = DeviceCache(w)
    cache.fill_prefix(w)
    plan = cache.append_step(w, decode_splits=w.decode_splits)
    return cache, plan, upload_q(w)


def test_noalloc_matches_workspace_call():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    assert pkv.device_supported(torch.cuda.current_device()), "not a gfx950 device"
    big = wl.config3(4097).with_lengths([3584], [512])     # 32 tiles split up to 8 ways over KV
    small = wl.config2()                                    # ragged batch: long tiles split, one-token row
    for name, w in (("3584+512", big), ("ragged", small)):
        print(f"[noalloc] {name}: P={list(w.prefix_lens)} L={list(w.chunk_lens)}", flush=True)
        cache, plan, q = _step(w)
        assert 0 < plan.plan.workspace_bytes <= pkv.PKV_NOALLOC_SCRATCH_BYTES and plan.plan.n_split_rows > 0
        ref = pkv.paged_extend_attn(q, cache.k_pool, cache.v_pool, cache.page_table, plan)
        out = torch.full_like(q, float("nan"))
        pkv.paged_extend_attn_noalloc(q, cache.k_pool, cache.v_pool, cache.page_table, plan, out)
        torch.cuda.synchronize()
        assert pkv.read_status(plan) == 0
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{name}: differs from the workspace call"
        if w is small:
            rep = assert_parity(values_of(out), oracle_out(w, oracle_pools(w)), w.dtype, "noalloc ragged")
            print(f"[parity] noalloc ragged: max_abs={rep['max_abs']:.3e}", flush=True)
