"""Pins for the oracle's float64 attention and LSE merge (CPU only).

Pinned against: torch's float64 scaled-dot-product attention on the CPU (a
library routine), closed forms (q = 0, one token, identical keys), the
sharding identity (merge of per-rank partials over the brute-force ownership
equals the unsharded result for every dcp_size and interleave), associativity
of the merge, and the sink identities.
"""

import numpy as np
import pytest
import torch

from oracle import attention, layout


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, scale):
    # torch reference, float64, GQA expanded by repeating each KV head G times
    Hq, Hkv = q.shape[0], k.shape[1]
    G = Hq // Hkv
    kq = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)    # [Hq, L, Dk]
    vq = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)
    qq = torch.from_numpy(q)[:, None, :]                                  # [Hq, 1, Dk]
    o = torch.nn.functional.scaled_dot_product_attention(qq, kq, vq, scale=scale)
    s = (qq @ kq.transpose(1, 2))[:, 0, :] * scale
    return o[:, 0, :].numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("Hq,Hkv,Dk,Dv,L", [(8, 2, 64, 64, 37), (8, 8, 16, 16, 5), (16, 1, 40, 32, 300), (4, 4, 8, 8, 1)])
def test_matches_torch_sdpa(Hq, Hkv, Dk, Dv, L):
    q, k, v = _rand((Hq, Dk), 1), _rand((L, Hkv, Dk), 2), _rand((L, Hkv, Dv), 3)
    scale = 1 / np.sqrt(Dk)
    o, lse = attention.decode_attention(q, k, v, scale)
    o_ref, lse_ref = _sdpa(q, k, v, scale)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_closed_forms():
    Hq, Hkv, D, L = 6, 3, 16, 50
    k, v = _rand((L, Hkv, D), 4), _rand((L, Hkv, D), 5)
    # q = 0: uniform weights -> mean of the values, LSE = ln L
    o, lse = attention.decode_attention(np.zeros((Hq, D)), k, v, 0.3)
    for h in range(Hq):
        np.testing.assert_allclose(o[h], v[:, h // 2, :].mean(axis=0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(L), rtol=1e-14)
    # one token: O = v_0, LSE = s_0
    q = _rand((Hq, D), 6)
    o, lse = attention.decode_attention(q, k[:1], v[:1], 0.3)
    for h in range(Hq):
        np.testing.assert_allclose(o[h], v[0, h // 2], rtol=1e-14)
        np.testing.assert_allclose(lse[h], 0.3 * q[h] @ k[0, h // 2], rtol=1e-13)
    # identical keys: mean of values, LSE = s + ln L
    kk = np.repeat(k[:1], L, axis=0)
    o, lse = attention.decode_attention(q, kk, v, 0.3)
    for h in range(Hq):
        np.testing.assert_allclose(o[h], v[:, h // 2].mean(axis=0), rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(lse[h], 0.3 * q[h] @ k[0, h // 2] + np.log(L), rtol=1e-12)


def test_nonpositive_scales():
    """Scale 0: uniform weights whatever q is (mean of the values, LSE = ln L);
    scale -c: the same result as scale c with q negated; both against torch."""
    Hq, Hkv, D, L = 6, 3, 16, 50
    q, k, v = _rand((Hq, D), 8), _rand((L, Hkv, D), 9), _rand((L, Hkv, D), 10)
    o, lse = attention.decode_attention(q, k, v, 0.0)
    for h in range(Hq):
        np.testing.assert_allclose(o[h], v[:, h // 2, :].mean(axis=0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(L), rtol=1e-14)
    o, lse = attention.decode_attention(q, k, v, -0.2)
    o2, lse2 = attention.decode_attention(-q, k, v, 0.2)
    np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13)
    o_ref, lse_ref = _sdpa(q, k, v, -0.2)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_empty_and_sink_edge_cases():
    Hq, D = 4, 8
    q = _rand((Hq, D), 7)
    k, v = np.zeros((0, 2, D)), np.zeros((0, 2, D))
    o, lse = attention.decode_attention(q, k, v, 1.0)
    assert np.all(o == 0) and np.all(lse == -np.inf)
    sink = np.array([0.5, -1.0, 2.0, 0.0])
    o, lse = attention.decode_attention(q, k, v, 1.0, sink)
    assert np.all(o == 0) and np.array_equal(lse, sink)
    # merge of empty parts
    mo, ml = attention.lse_merge(np.zeros((3, Hq, D)), np.full((3, Hq), -np.inf))
    assert np.all(mo == 0) and np.all(ml == -np.inf)
    mo, ml = attention.lse_merge(np.zeros((3, Hq, D)), np.full((3, Hq), -np.inf), sink)
    assert np.all(mo == 0) and np.array_equal(ml, sink)


@pytest.mark.parametrize("bs,D,I", [(bs, D, I) for bs in (1, 4, 16) for D in (1, 2, 3, 4, 8)
                                     for I in (1, 2, 4, 16) if bs % I == 0])
def test_sharded_merge_equals_unsharded(bs, D, I):
    Hq, Hkv, Dk, Dv = 8, 2, 16, 12
    L = 5 * bs * D + 3
    q, k, v = _rand((Hq, Dk), 8), _rand((L, Hkv, Dk), 9), _rand((L, Hkv, Dv), 10)
    own = layout.owners(L, bs, D, I)
    po, pl = attention.rank_partials(q, k, v, 0.25, own, D)
    mo, ml = attention.lse_merge(po, pl)
    o, lse = attention.decode_attention(q, k, v, 0.25)
    np.testing.assert_allclose(mo, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ml, lse, rtol=1e-13)
    # with a sink, applied once in the merge
    sink = _rand((Hq,), 11) + 2.0
    mo, ml = attention.lse_merge(po, pl, sink)
    o, lse = attention.decode_attention(q, k, v, 0.25, sink)
    np.testing.assert_allclose(mo, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ml, lse, rtol=1e-13)


def test_merge_associative_and_sink_identities():
    Hq, Dk, L = 4, 8, 60
    q, k, v = _rand((Hq, Dk), 12), _rand((L, 1, Dk), 13), _rand((L, 1, Dk), 14)
    own = np.arange(L) % 3
    po, pl = attention.rank_partials(q, k, v, 0.5, own, 3)
    ab_o, ab_l = attention.lse_merge(po[:2], pl[:2])
    two_o, two_l = attention.lse_merge(np.stack([ab_o, po[2]]), np.stack([ab_l, pl[2]]))
    all_o, all_l = attention.lse_merge(po, pl)
    np.testing.assert_allclose(two_o, all_o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(two_l, all_l, rtol=1e-14)
    # sink -> -inf reduces to the no-sink result
    so, sl = attention.lse_merge(po, pl, np.full(Hq, -1e300))
    np.testing.assert_allclose(so, all_o, rtol=1e-14)
    np.testing.assert_allclose(sl, all_l, rtol=1e-14)
    # O_sink = O * exp(LSE - LSE_sink), LSE_sink = logaddexp(LSE, sink)
    sink = _rand((Hq,), 15) + 2.0
    so, sl = attention.lse_merge(po, pl, sink)
    np.testing.assert_allclose(sl, np.logaddexp(all_l, sink), rtol=1e-14)
    np.testing.assert_allclose(so, all_o * np.exp(all_l - sl)[:, None], rtol=1e-12, atol=1e-15)


def test_sink_as_extra_zero_value_token():
    # A sink logit behaves like one more token whose score is the sink and
    # whose value row is zero; compare against torch SDPA over L + 1 tokens.
    Hq, Dk, L = 4, 16, 20
    q, k, v = _rand((Hq, Dk), 16), _rand((L, Hq, Dk), 17), _rand((L, Hq, Dk), 18)
    scale = 0.25
    sink = _rand((Hq,), 19)
    extra_k = (q * (sink / (scale * (q * q).sum(axis=1)))[:, None])[None]   # score == sink
    k2 = np.concatenate([k, extra_k], axis=0)
    v2 = np.concatenate([v, np.zeros((1, Hq, Dk))], axis=0)
    o_ref, lse_ref = _sdpa(q, k2, v2, scale)
    o, lse = attention.decode_attention(q, k, v, scale, sink)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)


def test_planted_mistake_dropped_group_mapping(monkeypatch):
    # If the oracle used KV head h % Hkv instead of h // G, the SDPA pin fails.
    q, k, v = _rand((8, 16), 20), _rand((9, 2, 16), 21), _rand((9, 2, 16), 22)
    o_ref, _ = _sdpa(q, k, v, 0.25)
    k_wrong = k[:, ::-1, :]
    o_wrong, _ = attention.decode_attention(q, k_wrong, v[:, ::-1, :], 0.25)
    assert not np.allclose(o_wrong, o_ref)
