"""Pins for the oracle's multi-token decode (speculative verification) (CPU only).

Pinned against: torch's float64 scaled-dot-product attention with an explicit
boolean mask that lets query i of the last q_len tokens see positions up to
L - q_len + i (a library routine given the mask written from the definition),
the q_len = 1 case (plain decode), the sharding identity over the
brute-force ownership for every dcp_size and interleave, and a planted
off-by-one in the causal boundary that the torch pin must catch.
"""

import numpy as np
import pytest
import torch

from oracle import attention, layout


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa_causal_tail(q, k, v, scale):
    """torch reference: q [q_len, Hq, Dk] at the last q_len positions of k / v [L, Hkv, D]."""
    q_len, Hq, _ = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    kq = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)              # [Hq, L, Dk]
    vq = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)
    qq = torch.from_numpy(q).permute(1, 0, 2)                                      # [Hq, q_len, Dk]
    pos_q = torch.arange(L - q_len, L)[:, None]
    mask = torch.arange(L)[None, :] <= pos_q                                       # [q_len, L]
    o = torch.nn.functional.scaled_dot_product_attention(qq, kq, vq, attn_mask=mask, scale=scale)
    s = (qq @ kq.transpose(1, 2)) * scale
    s = s.masked_fill(~mask, float("-inf"))
    return o.permute(1, 0, 2).numpy(), torch.logsumexp(s, dim=-1).permute(1, 0).numpy()


@pytest.mark.parametrize("q_len,Hq,Hkv,Dk,Dv,L", [(2, 8, 2, 64, 64, 37), (4, 8, 8, 16, 16, 5), (8, 16, 1, 40, 32, 300),
                                                  (3, 4, 4, 8, 8, 3), (1, 8, 2, 16, 16, 20)])
def test_matches_masked_torch_sdpa(q_len, Hq, Hkv, Dk, Dv, L):
    q, k, v = _rand((q_len, Hq, Dk), 1), _rand((L, Hkv, Dk), 2), _rand((L, Hkv, Dv), 3)
    scale = 1 / np.sqrt(Dk)
    o, lse = attention.verify_attention(q, k, v, scale)
    o_ref, lse_ref = _sdpa_causal_tail(q, k, v, scale)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_one_token_is_decode():
    q, k, v = _rand((1, 8, 16), 4), _rand((30, 2, 16), 5), _rand((30, 2, 16), 6)
    o, lse = attention.verify_attention(q, k, v, 0.25, sink=np.linspace(-1, 1, 8))
    o1, lse1 = attention.decode_attention(q[0], k, v, 0.25, sink=np.linspace(-1, 1, 8))
    np.testing.assert_array_equal(o[0], o1)
    np.testing.assert_array_equal(lse[0], lse1)


def test_queries_beyond_the_cache_are_rejected():
    with pytest.raises(ValueError):
        attention.verify_attention(_rand((4, 2, 8), 1), _rand((3, 1, 8), 2), _rand((3, 1, 8), 3), 1.0)


@pytest.mark.parametrize("bs,D,I", [(4, 2, 2), (16, 4, 1), (16, 3, 16), (8, 8, 4), (2, 1, 1)])
def test_sharded_merge_equals_unsharded(bs, D, I):
    q_len, Hq, Hkv, Dk, L = 5, 6, 3, 16, 41
    q, k, v = _rand((q_len, Hq, Dk), 7), _rand((L, Hkv, Dk), 8), _rand((L, Hkv, Dk), 9)
    sink = np.linspace(-2, 2, Hq)
    owner = layout.owners(L, bs, D, I)
    po, pl = attention.verify_rank_partials(q, k, v, 0.3, owner, D)
    o_ref, lse_ref = attention.verify_attention(q, k, v, 0.3, sink)
    for i in range(q_len):
        o, lse = attention.lse_merge(po[:, i], pl[:, i], sink)
        np.testing.assert_allclose(o, o_ref[i], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, lse_ref[i], rtol=1e-12, atol=1e-12)


def test_early_queries_can_be_empty_on_a_rank():
    # 4 tokens, 2 ranks, interleave 1: rank 1 owns positions 1 and 3; with q_len = 3 the
    # first query (position 1) sees position 1 on rank 1, the tail query sees both
    q, k, v = _rand((3, 2, 8), 10), _rand((4, 1, 8), 11), _rand((4, 1, 8), 12)
    owner = layout.owners(4, 2, 2, 1)
    po, pl = attention.verify_rank_partials(q[:1], k[:2], v[:2], 1.0, owner[:2], 2)
    assert np.isfinite(pl).all()
    # a rank that owns nothing at or before the query's position gives O = 0, LSE = -inf
    po, pl = attention.verify_rank_partials(q[:1], k[:1], v[:1], 1.0, owner[:1], 2)
    assert np.all(pl[1] == -np.inf) and np.all(po[1] == 0)


def test_planted_causal_off_by_one_is_caught(monkeypatch):
    real = attention.decode_attention
    calls = []

    def leaky(q, k, v, scale, sink=None):       # sees one position too many (where it exists)
        calls.append(k.shape[0])
        return real(q, full_k[:k.shape[0] + 1], full_v[:k.shape[0] + 1], scale, sink)

    q, full_k, full_v = _rand((3, 4, 8), 13), _rand((20, 2, 8), 14), _rand((20, 2, 8), 15)
    monkeypatch.setattr(attention, "decode_attention", leaky)
    o, _ = attention.verify_attention(q, full_k, full_v, 0.5)
    o_ref, _ = _sdpa_causal_tail(q, full_k, full_v, 0.5)
    assert calls == [18, 19, 20]
    assert not np.allclose(o[:2], o_ref[:2], rtol=1e-6, atol=1e-6)
