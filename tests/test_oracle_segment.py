"""Pins for the oracle's replicated segment (a sliding-window cache kept on
every rank that exactly one rank counts) (CPU only).

Pinned against: torch's float64 SDPA over the sharded sequence and the
segment concatenated (the plain definition), the sharding identity for every
layout and every choice of the designated rank, the empty segment (plain
decode), and a planted mistake (the segment counted on every rank) that the
identity must catch.
"""

import numpy as np
import pytest
import torch

from oracle import attention, layout


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa_with_sink(q, k, v, scale, sink):
    Hq, Hkv = q.shape[0], k.shape[1]
    G = Hq // Hkv
    kq = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)
    vq = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)
    s = (torch.from_numpy(q)[:, None, :] @ kq.transpose(1, 2))[:, 0, :] * scale      # [Hq, L]
    s = torch.cat([s, torch.from_numpy(sink)[:, None]], dim=1)                       # sink: zero value
    p = torch.softmax(s, dim=1)
    o = (p[:, None, :-1] @ vq)[:, 0, :]
    return o.numpy(), torch.logsumexp(s, dim=1).numpy()


@pytest.mark.parametrize("bs,D,I,seg_rank", [(4, 2, 2, 0), (16, 4, 1, 3), (16, 3, 16, 1), (8, 8, 4, 5), (2, 1, 1, 0)])
def test_one_rank_counts_the_segment(bs, D, I, seg_rank):
    Hq, Hkv, Dk, L, W = 8, 2, 16, 57, 9
    q, k, v = _rand((Hq, Dk), 1), _rand((L, Hkv, Dk), 2), _rand((L, Hkv, Dk), 3)
    ks, vs = _rand((W, Hkv, Dk), 4), _rand((W, Hkv, Dk), 5)
    sink = np.linspace(-1, 2, Hq)
    po, pl = attention.segment_rank_partials(q, k, v, 0.3, layout.owners(L, bs, D, I), D, ks, vs, seg_rank)
    o, lse = attention.lse_merge(po, pl, sink)
    o_ref, lse_ref = _sdpa_with_sink(q, np.concatenate([k, ks]), np.concatenate([v, vs]), 0.3, sink)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_empty_segment_is_plain_decode():
    q, k, v = _rand((4, 8), 6), _rand((20, 1, 8), 7), _rand((20, 1, 8), 8)
    own = layout.owners(20, 4, 2, 1)
    po, pl = attention.segment_rank_partials(q, k, v, 0.5, own, 2, k[:0], v[:0], 1)
    po2, pl2 = attention.rank_partials(q, k, v, 0.5, own, 2)
    np.testing.assert_array_equal(po, po2)
    np.testing.assert_array_equal(pl, pl2)


def test_segment_alone_on_an_empty_rank():
    # 2 tokens on 4 ranks: rank 3 owns nothing and takes the segment
    q, k, v = _rand((2, 8), 9), _rand((2, 1, 8), 10), _rand((2, 1, 8), 11)
    ks, vs = _rand((3, 1, 8), 12), _rand((3, 1, 8), 13)
    po, pl = attention.segment_rank_partials(q, k, v, 0.5, layout.owners(2, 4, 4, 1), 4, ks, vs, 3)
    o_seg, l_seg = attention.decode_attention(q, ks, vs, 0.5)
    np.testing.assert_array_equal(po[3], o_seg)
    np.testing.assert_array_equal(pl[3], l_seg)
    assert np.all(pl[2] == -np.inf)


def test_planted_double_count_is_caught():
    Hq, Hkv, Dk, L, W, D = 4, 1, 8, 30, 5, 4
    q, k, v = _rand((Hq, Dk), 14), _rand((L, Hkv, Dk), 15), _rand((L, Hkv, Dk), 16)
    ks, vs = _rand((W, Hkv, Dk), 17), _rand((W, Hkv, Dk), 18)
    own = layout.owners(L, 4, D, 1)
    # every rank adds the segment (the mistake the designated rank avoids)
    parts = [attention.segment_rank_partials(q, k, v, 0.5, own, D, ks, vs, r) for r in range(D)]
    po = np.stack([parts[r][0][r] for r in range(D)])
    pl = np.stack([parts[r][1][r] for r in range(D)])
    o_bad, _ = attention.lse_merge(po, pl)
    o_ref, _ = attention.decode_attention(q, np.concatenate([k, ks]), np.concatenate([v, vs]), 0.5)
    assert not np.allclose(o_bad, o_ref, rtol=1e-6, atol=1e-6)
