"""The fused multi-query step (q_len new tokens appended and attended in one launch) on the
GPU: pools and outputs bitwise equal to pkv_kv_append_tokens followed by
pkv_paged_multi_query_attention, pools bit-exact against the oracle's appends and outputs
within the bars of the oracle."""

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


def mq_workload(q_len, dtype="bf16", H=32, Hkv=8, d=128, B=6, lengths=None, lo=0, hi=900,
                seed=0):
    kw = dict(lengths=lengths) if lengths else dict(len_range=(lo, hi))
    spec = wlm.Spec(f"mqs-{dtype}-{q_len}-{H}-{Hkv}-{d}", dtype, B, H, Hkv, d, "gqa",
                    q_len=q_len, **kw)
    return wlm.make_workload(spec, seed=seed)


def fused(wl, ptok=0, t=None):
    if t is None:
        t = wlm.to_torch(wl, DEV)
    out = torch.empty_like(t["q"])
    pkv.pkv_paged_multi_query_step(out, t["q"], t["k_pool"], t["v_pool"], t["k_new"],
                                   t["v_new"], t["block_tables"], t["context_lens"],
                                   wl.max_context_len, wl.scale, partition_tokens=ptok)
    torch.cuda.synchronize()
    return out, t


def separate(wl, ptok=0):
    t = wlm.to_torch(wl, DEV)
    pkv.pkv_kv_append_tokens(t["k_pool"], t["v_pool"], t["k_new"], t["v_new"],
                             t["block_tables"], t["positions"])
    out = torch.empty_like(t["q"])
    pkv.pkv_paged_multi_query_attention(out, t["q"], t["k_pool"], t["v_pool"], t["block_tables"],
                                        t["context_lens"], wl.max_context_len, wl.scale,
                                        partition_tokens=ptok)
    torch.cuda.synchronize()
    return out, t


def oracle_pools(wl):
    kp, vp = wl.k_pool, wl.v_pool
    for i in range(wl.spec.q_len):
        kp, vp = orc.kv_append(kp, vp, np.ascontiguousarray(wl.k_new[:, i]),
                               np.ascontiguousarray(wl.v_new[:, i]), wl.block_tables,
                               wl.positions + i, 16)
    return kp, vp


def check_against_separate(wl, ptok):
    a, ta = fused(wl, ptok)
    b, tb = separate(wl, ptok)
    assert same_bits(ta["k_pool"], tb["k_pool"]) and same_bits(ta["v_pool"], tb["v_pool"])
    assert same_bits(a, b)
    return a, ta


@pytest.mark.parametrize("q_len,dtype,H,Hkv,d", [
    (2, "bf16", 32, 8, 128), (4, "bf16", 32, 8, 128), (16, "f16", 32, 32, 128),
    (8, "bf16", 16, 8, 64), (4, "f32", 8, 2, 64), (3, "f16", 32, 8, 128),
])
@pytest.mark.parametrize("ptok", [0, 128])
def test_mq_step_matches_the_two_calls_and_the_oracle(q_len, dtype, H, Hkv, d, ptok):
    # lengths put the new tokens at the start, the middle and across the end of a block
    lengths = (0, 14, 16, 29, 300, 1000 - q_len // 2)
    wl = mq_workload(q_len, dtype, H, Hkv, d, lengths=lengths, seed=q_len * 5 + H)
    out, t = check_against_separate(wl, ptok)
    kp, vp = oracle_pools(wl)
    assert np.array_equal(wlm.from_torch(t["k_pool"], dtype).view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(wlm.from_torch(t["v_pool"], dtype).view(np.uint8), vp.view(np.uint8))
    ref = orc.paged_multi_query_attention(wl.q, kp, vp, wl.block_tables, wl.context_lens, 16,
                                          wl.scale, dtype)
    assert_close(out.double().cpu().numpy(), ref, dtype, f"mq step q_len {q_len} P {ptok}")


def test_new_tokens_of_long_sequences_split_over_workgroups():
    """Long contexts whose new tokens straddle a block boundary: the two blocks can fall
    into different segments of the balanced split."""
    wl = mq_workload(4, B=3, lengths=(9006, 20014, 126), seed=9)
    check_against_separate(wl, 0)


def test_q_len_one_is_the_single_token_step():
    wl = mq_workload(1, lengths=(0, 15, 16, 700, 1601), B=5, seed=4)
    ta = wlm.to_torch(wl, DEV)                    # single-token layout: q [B, H, d]
    a = torch.empty((wl.batch, 1, 32, 128), dtype=torch.bfloat16, device=DEV)
    pkv.pkv_paged_multi_query_step(a, ta["q"].unsqueeze(1).contiguous(), ta["k_pool"],
                                   ta["v_pool"], ta["k_new"].unsqueeze(1).contiguous(),
                                   ta["v_new"].unsqueeze(1).contiguous(), ta["block_tables"],
                                   ta["context_lens"], wl.max_context_len, wl.scale)
    t = wlm.to_torch(wl, DEV)
    out = torch.empty_like(t["q"])
    pkv.pkv_paged_decode_step(out, t["q"], t["k_pool"], t["v_pool"], t["k_new"], t["v_new"],
                              t["block_tables"], t["context_lens"], wl.max_context_len, wl.scale)
    torch.cuda.synchronize()
    assert same_bits(a[:, 0], out)
    assert same_bits(ta["k_pool"], t["k_pool"]) and same_bits(ta["v_pool"], t["v_pool"])


def test_bad_entries_skip_the_append_and_give_nan():
    wl = mq_workload(4, B=5, lengths=(14, 300, 700, 40, 900), seed=7)
    t = wlm.to_torch(wl, DEV)
    prev_k = t["k_pool"].clone()
    n2 = int(wl.context_lens[2])
    t["block_tables"][2, (n2 - 1) // 16] = wl.num_blocks + 3       # block of the last new token
    t["context_lens"][4] = wl.max_context_len + 1                    # invalid length
    out, t = fused(wl, 0, t)
    got = out.double().cpu().numpy()
    assert np.isnan(got[2]).all() and np.isnan(got[4]).all()
    kp, _ = oracle_pools(wl)
    after = wlm.from_torch(t["k_pool"], "bf16")
    prev = wlm.from_torch(prev_k, "bf16")
    for b in range(wl.batch):
        for i in range(4):
            p = int(wl.positions[b]) + i
            blk, off = int(wl.block_tables[b, p // 16]), p % 16
            skipped = b == 4 or (b == 2 and p // 16 == (n2 - 1) // 16)
            want = prev[blk, off] if skipped else kp[blk, off]
            assert np.array_equal(after[blk, off], want), (b, i)


def test_many_rows_use_the_wave_per_row_merge():
    """20 sequences x 4 new tokens x 32 heads = 2560 output rows: the merge runs one wave
    per row (from 1024 rows on); the result must still match the oracle."""
    wl = mq_workload(4, B=20, lo=600, hi=2500, seed=21)
    out, t = check_against_separate(wl, 0)
    kp, vp = oracle_pools(wl)
    ref = orc.paged_multi_query_attention(wl.q, kp, vp, wl.block_tables, wl.context_lens, 16,
                                          wl.scale, "bf16")
    assert_close(out.double().cpu().numpy(), ref, "bf16", "many rows")


@pytest.mark.slow
def test_full_size_gqa_verify4():
    """The benchmark's multi-query shape: the GQA workload (64 sequences of 4096-8192
    tokens, 32 / 8 heads, d 128, bf16) with 4 new tokens per sequence, fused step bitwise
    equal to the two calls, pools bit-exact, every output against the oracle."""
    import dataclasses
    print("multi-query full size, q_len 4", flush=True)
    spec = dataclasses.replace(wlm.SPECS[3], name="gqa-bf16-verify4", q_len=4)
    wl = wlm.make_workload(spec, seed=3)
    out, t = check_against_separate(wl, 0)
    kp, vp = oracle_pools(wl)
    for name, ref_pool in (("k_pool", kp), ("v_pool", vp)):
        ref_dev = torch.from_numpy(ref_pool.view(np.int16)).to(DEV)
        assert torch.equal(t[name].view(torch.int16), ref_dev), name
        del ref_dev
    ref = orc.paged_multi_query_attention(wl.q, kp, vp, wl.block_tables, wl.context_lens, 16,
                                          wl.scale, "bf16")
    e = assert_close(out.double().cpu().numpy(), ref, "bf16", "verify4 full size")
    print(f"  errors {e}", flush=True)
