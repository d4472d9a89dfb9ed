"""Pins of the multi-query (several new tokens per sequence) oracle, CPU only."""

import math

import numpy as np
import pytest
import torch

from oracle import pkv_oracle as orc
from paged_kv_cache_26_amd import workload as wlm
from tests.parity import within


def mq_spec(q_len, dtype="bf16", H=32, Hkv=8, B=5, lo=20, hi=700, **kw):
    return wlm.Spec(f"mq-{dtype}-{q_len}", dtype, B, H, Hkv, 128, "gqa", len_range=(lo, hi),
                    q_len=q_len, **kw)


def append_all(wl):
    """The q_len new tokens written one position after another (the oracle's append)."""
    kp, vp = wl.k_pool, wl.v_pool
    ql = wl.spec.q_len
    for i in range(ql):
        kn = wl.k_new if ql == 1 else wl.k_new[:, i]
        vn = wl.v_new if ql == 1 else wl.v_new[:, i]
        kp, vp = orc.kv_append(kp, vp, kn, vn, wl.block_tables, wl.positions + i, 16)
    return kp, vp


def test_one_query_equals_decode():
    wl = wlm.make_workload(3, small=True)
    kp, vp = append_all(wl)
    one = orc.paged_decode_attention(wl.q, kp, vp, wl.block_tables, wl.context_lens, 16,
                                     wl.scale, wl.dtype)
    mq = orc.paged_multi_query_attention(wl.q[:, None], kp, vp, wl.block_tables,
                                         wl.context_lens, 16, wl.scale, wl.dtype)
    assert np.array_equal(mq[:, 0], one)


@pytest.mark.parametrize("q_len", [2, 4])
def test_each_query_equals_a_decode_step_on_its_prefix(q_len):
    """Verifying q_len tokens in one pass equals q_len single-token steps."""
    wl = wlm.make_workload(mq_spec(q_len), seed=30 + q_len)
    kp, vp = append_all(wl)
    mq = orc.paged_multi_query_attention(wl.q, kp, vp, wl.block_tables, wl.context_lens, 16,
                                         wl.scale, wl.dtype)
    for i in range(q_len):
        lens_i = wl.context_lens - q_len + i + 1
        step = orc.paged_decode_attention(np.ascontiguousarray(wl.q[:, i]), kp, vp,
                                          wl.block_tables, lens_i, 16, wl.scale, wl.dtype)
        assert np.array_equal(mq[:, i], step)


def _sdpa_masked(wl, kp, vp):
    """torch SDPA (fp64, CPU) with the causal mask built as in the KV Cache section:
    triu(ones(q_len, K), diagonal = K - q_len + 1) hides a key from a query."""
    B, ql, H, d = wl.q.shape
    out = np.empty((B, ql, H, d))
    for b in range(B):
        n = int(wl.context_lens[b])
        k = orc.storage_to_f64(orc.gather_kv(kp, wl.block_tables[b], n, 16), wl.dtype)
        v = orc.storage_to_f64(orc.gather_kv(vp, wl.block_tables[b], n, 16), wl.dtype)
        kt = torch.from_numpy(k).permute(1, 0, 2).unsqueeze(0).contiguous()
        vt = torch.from_numpy(v).permute(1, 0, 2).unsqueeze(0).contiguous()
        qt = torch.from_numpy(orc.storage_to_f64(wl.q[b], wl.dtype)).permute(1, 0, 2)
        qt = qt.unsqueeze(0).contiguous()                                   # [1, H, ql, d]
        hidden = torch.triu(torch.ones(ql, n), diagonal=n - ql + 1).bool()
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=~hidden,
                                                             enable_gqa=True)
        out[b] = o[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("q_len,H,Hkv", [(2, 32, 8), (4, 32, 8), (16, 8, 8)])
def test_multi_query_equals_library_masked_attention(q_len, H, Hkv):
    wl = wlm.make_workload(mq_spec(q_len, H=H, Hkv=Hkv, lo=1), seed=40 + q_len)
    kp, vp = append_all(wl)
    got = orc.paged_multi_query_attention(wl.q, kp, vp, wl.block_tables, wl.context_lens, 16,
                                          wl.scale, wl.dtype)
    ref = _sdpa_masked(wl, kp, vp)
    assert np.isfinite(got).all()
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 1e-12


def test_hand_worked_two_queries():
    """Tokens t0, t1 cached; t2, t3 are the two new tokens. K rows (1,0), (0,1), (-1,0),
    (0,-1); V rows (1,0), (0,1), (1,1), (0,0); q0 = (sqrt2, 0) sees t0..t2, q1 = (0, sqrt2)
    sees t0..t3. Scale 1/sqrt2."""
    k = np.full((3, 2, 1, 2), np.nan, np.float32)
    v = np.full((3, 2, 1, 2), np.nan, np.float32)
    rows_k = [(1, 0), (0, 1), (-1, 0), (0, -1)]
    rows_v = [(1, 0), (0, 1), (1, 1), (0, 0)]
    table = np.array([[2, 0]], np.int32)           # tokens 0,1 in block 2; 2,3 in block 0
    for t in range(4):
        k[table[0, t // 2], t % 2, 0] = rows_k[t]
        v[table[0, t // 2], t % 2, 0] = rows_v[t]
    r2 = math.sqrt(2)
    q = np.array([[[[r2, 0]], [[0, r2]]]], np.float32)   # [1, 2, 1, 2]
    out = orc.paged_multi_query_attention(q, k, v, table, np.array([4], np.int32), 2,
                                          1 / r2, "f32")
    e = math.e
    z0 = e + 1 + 1 / e                             # scores (1, 0, -1)
    z1 = 1 + e + 1 + 1 / e                         # scores (0, 1, 0, -1)
    want = np.array([[(e + 1 / e) / z0, (1 + 1 / e) / z0], [(1 + 1) / z1, (e + 1) / z1]])
    np.testing.assert_allclose(out[0, :, 0], want, rtol=1e-6)


def test_planted_causal_off_by_one_is_caught(monkeypatch):
    wl = wlm.make_workload(mq_spec(4, B=3), seed=50)
    kp, vp = append_all(wl)
    ref = _sdpa_masked(wl, kp, vp)
    real = orc.softmax_two_pass
    # hide one more key than the definition does: the last visible score of every query
    monkeypatch.setattr(orc, "softmax_two_pass",
                        lambda s: np.concatenate([real(s[:-1]), [0.0]]) if s.size > 1 else real(s))
    got = orc.paged_multi_query_attention(wl.q, kp, vp, wl.block_tables, wl.context_lens, 16,
                                          wl.scale, wl.dtype)
    assert not within(got, ref, "bf16")[0]
