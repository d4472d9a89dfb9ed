"""pkv_paged_decode_step_noalloc (the fused step with the library's static scratch as its
workspace) on the GPU, through the C ABI: outputs and pools bitwise equal to
pkv_paged_decode_step with a caller workspace, and within the bars of the oracle, on two
calls in a row, the second with a smaller input (the scratch keeps the first call's
records, which must not matter)."""

import numpy as np
import pytest
import torch

from oracle import pkv_oracle as orc
from paged_kv_cache_26_amd import pkv
from paged_kv_cache_26_amd import workload as wlm
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available()
    pkv.load_library()


def same_bits(x, y):
    return torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))


def _compare(wl, what):
    print(f"no-alloc step: {what}", flush=True)
    need = pkv.pkv_decode_workspace_bytes(wl.batch, wl.spec.n_heads, wl.spec.n_kv_heads,
                                          wl.spec.d_head, wl.max_context_len, 0)
    assert 0 < need <= 32 << 20, need            # the call does use the scratch
    ta = wlm.to_torch(wl, DEV)
    out_a = torch.empty_like(ta["q"])
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    pkv.pkv_paged_decode_step(out_a, ta["q"], ta["k_pool"], ta["v_pool"], ta["k_new"],
                              ta["v_new"], ta["block_tables"], ta["context_lens"],
                              wl.max_context_len, wl.scale, 0, ws)
    tb = wlm.to_torch(wl, DEV)
    out_b = torch.empty_like(tb["q"])
    torch.cuda.synchronize()
    reserved = torch.cuda.memory_reserved()
    pkv.pkv_paged_decode_step_noalloc(out_b, tb["q"], tb["k_pool"], tb["v_pool"], tb["k_new"],
                                      tb["v_new"], tb["block_tables"], tb["context_lens"],
                                      wl.max_context_len, wl.scale)
    torch.cuda.synchronize()
    assert torch.cuda.memory_reserved() == reserved     # nothing taken from torch either
    assert same_bits(out_a, out_b)
    assert same_bits(ta["k_pool"], tb["k_pool"]) and same_bits(ta["v_pool"], tb["v_pool"])
    kp, vp = orc.kv_append(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.block_tables,
                           wl.positions, 16)
    ref = orc.paged_decode_attention(wl.q, kp, vp, wl.block_tables, wl.context_lens, 16,
                                     wl.scale, wl.dtype)
    e = assert_close(out_b.double().cpu().numpy(), ref, wl.dtype, what)
    print(f"  errors {e}", flush=True)


def test_noalloc_step_equals_the_workspace_step_on_two_calls():
    # first call: the GQA workload at full size (64 sequences of 4096-8192 tokens, 18 MB
    # of records in the scratch); second call: a smaller batch of the same shape
    _compare(wlm.make_workload(3), "gqa-bf16, full size")
    spec = wlm.Spec("noalloc-small-bf16", "bf16", 3, 32, 8, 128, "gqa",
                    lengths=(600, 900, 1300))
    _compare(wlm.make_workload(spec, seed=31), "3 sequences of 600-1300 tokens")
