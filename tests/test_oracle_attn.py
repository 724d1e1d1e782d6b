"""Pins of the oracle's causal GQA attention.

Causal attention with the diagonal included (page "训练3.8B LLM至0.384
CORE，成本998美元 – Hugo Vergnes", section 无效的方法; the m.nxbn.cn
build-an-LLM page, section 3.1), query heads in groups sharing one KV head
(page "750美元从零训练3个LLM：一位开发者的实战复盘", section V2).  The oracle
is pinned to torch's float64 SDPA, to literal loops on tiny shapes, to closed
forms and to invariants.
"""
import math

import pytest
import torch
import torch.nn.functional as F

import oracle
from rope_gqa_causal_amd import synth


def _cache_from_bshd(k):
    """[B,S,H,D] -> a [B,H,S,D] view (strided stand-in for a cache)."""
    return k.transpose(1, 2)


def _rand(shape, seed, dtype=torch.float32):
    return synth.normal(shape, synth.generator(seed), dtype)


@pytest.mark.parametrize("B,S,Hq,Hkv,D", [(1, 1, 1, 1, 4), (2, 17, 4, 2, 32), (1, 33, 6, 2, 16),
                                          (2, 9, 8, 1, 8), (1, 12, 3, 3, 64)])
def test_matches_torch_sdpa_float64(B, S, Hq, Hkv, D):
    q = _rand((B, S, Hq, D), 100 + S)
    k = _rand((B, S, Hkv, D), 200 + S)
    v = _rand((B, S, Hkv, D), 300 + S)
    o = oracle.attn(q, _cache_from_bshd(k), _cache_from_bshd(v))
    ref = F.scaled_dot_product_attention(
        q.double().transpose(1, 2), k.double().transpose(1, 2), v.double().transpose(1, 2),
        is_causal=True, enable_gqa=True).transpose(1, 2)
    assert (o - ref).abs().max().item() < 1e-12


def test_bottom_right_alignment_with_q_start():
    # Rows sit at absolute slots q_start + s; SDPA gets the explicit mask.
    B, Sk, Sq, Hq, Hkv, D = 2, 20, 5, 4, 2, 16
    q = _rand((B, Sq, Hq, D), 1)
    k = _rand((B, Sk, Hkv, D), 2)
    v = _rand((B, Sk, Hkv, D), 3)
    q_start = torch.tensor([15, 4], dtype=torch.int32)
    o = oracle.attn(q, _cache_from_bshd(k), _cache_from_bshd(v), q_start=q_start)
    for b in range(B):
        p = q_start[b].item() + torch.arange(Sq)
        mask = torch.arange(Sk)[None, :] <= p[:, None]
        ref = F.scaled_dot_product_attention(
            q[b:b + 1].double().transpose(1, 2), k[b:b + 1].double().transpose(1, 2),
            v[b:b + 1].double().transpose(1, 2), attn_mask=mask, enable_gqa=True).transpose(1, 2)
        assert (o[b:b + 1] - ref).abs().max().item() < 1e-12


def _brute(q, k, v, q_start, scale):
    """Literal loops: scores, max, exp, sum, weighted values."""
    B, Sq, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    out = [[[[0.0] * D for _ in range(Hq)] for _ in range(Sq)] for _ in range(B)]
    for b in range(B):
        for s in range(Sq):
            p = q_start[b] + s
            for h in range(Hq):
                kh = h // g
                z = []
                for j in range(p + 1):
                    acc = 0.0
                    for d in range(D):
                        acc += float(q[b, s, h, d]) * float(k[b, j, kh, d])
                    z.append(scale * acc)
                m = max(z)
                e = [math.exp(t - m) for t in z]
                tot = sum(e)
                for d in range(D):
                    out[b][s][h][d] = sum(e[j] * float(v[b, j, kh, d]) for j in range(p + 1)) / tot
    return torch.tensor(out, dtype=torch.float64)


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,D", [(1, 4, 4, 2, 1, 2), (2, 3, 7, 4, 2, 4), (1, 6, 6, 3, 3, 8)])
def test_matches_brute_force_loops(B, Sq, Sk, Hq, Hkv, D):
    q = _rand((B, Sq, Hq, D), 7)
    k = _rand((B, Sk, Hkv, D), 8)
    v = _rand((B, Sk, Hkv, D), 9)
    q_start = [Sk - Sq] * B
    scale = 0.37
    o = oracle.attn(q, _cache_from_bshd(k), _cache_from_bshd(v),
                    q_start=torch.tensor(q_start, dtype=torch.int32), scale=scale)
    ref = _brute(q, k, v, q_start, scale)
    assert (o - ref).abs().max().item() < 1e-12


def test_gqa_equals_mha_on_repeated_kv_and_group_one_is_mha():
    B, S, Hq, Hkv, D = 2, 11, 6, 2, 16
    q = _rand((B, S, Hq, D), 21)
    k = _rand((B, S, Hkv, D), 22)
    v = _rand((B, S, Hkv, D), 23)
    o = oracle.attn(q, _cache_from_bshd(k), _cache_from_bshd(v))
    kr = k.repeat_interleave(Hq // Hkv, dim=2)
    vr = v.repeat_interleave(Hq // Hkv, dim=2)
    o_mha = oracle.attn(q, _cache_from_bshd(kr), _cache_from_bshd(vr))
    assert torch.equal(o, o_mha)
    # MQA (one KV head) is the other extreme.
    o_mqa = oracle.attn(q, _cache_from_bshd(k[:, :, :1]), _cache_from_bshd(v[:, :, :1]))
    o_ref = oracle.attn(q, _cache_from_bshd(k[:, :, :1].expand(B, S, Hq, D)),
                        _cache_from_bshd(v[:, :, :1].expand(B, S, Hq, D)))
    assert torch.equal(o_mqa, o_ref)


def test_rows_sum_to_one_and_lse_is_logsumexp():
    B, S, Hq, Hkv, D = 1, 13, 4, 2, 8
    q = _rand((B, S, Hq, D), 31) * 3
    k = _rand((B, S, Hkv, D), 32)
    ones = torch.ones((B, S, Hkv, D))
    o, lse = oracle.attn(q, _cache_from_bshd(k), _cache_from_bshd(ones), want_lse=True)
    assert (o - 1.0).abs().max().item() < 1e-14
    scale = D ** -0.5
    kk = k.double().repeat_interleave(Hq // Hkv, dim=2)
    z = torch.einsum("bshd,bjhd->bhsj", q.double(), kk) * scale
    causal = torch.ones(S, S, dtype=torch.bool).tril()
    z = z.masked_fill(~causal, float("-inf"))
    assert (lse - torch.logsumexp(z, dim=-1)).abs().max().item() < 1e-12


def test_zero_query_averages_the_visible_values():
    # q = 0 makes every visible score equal: row p is the mean of v_0..v_p.
    B, S, Hq, Hkv, D = 2, 10, 2, 1, 8
    q = torch.zeros((B, S, Hq, D))
    k = _rand((B, S, Hkv, D), 41)
    v = _rand((B, S, Hkv, D), 42)
    o = oracle.attn(q, _cache_from_bshd(k), _cache_from_bshd(v))
    mean = v.double().cumsum(dim=1) / torch.arange(1, S + 1, dtype=torch.float64)[None, :, None, None]
    assert (o - mean.expand(B, S, Hq, D)).abs().max().item() < 1e-14


def test_one_hot_values_return_the_weight_rows():
    # V_j = e_j turns o into the softmax row itself; compare with torch.softmax.
    S, D, Hq, Hkv = 8, 8, 2, 1
    q = _rand((1, S, Hq, D), 51) * 2
    k = _rand((1, S, Hkv, D), 52)
    v = torch.eye(S, D)[None, :, None, :].contiguous()
    o = oracle.attn(q, _cache_from_bshd(k), _cache_from_bshd(v), scale=0.5)
    z = torch.einsum("shd,jd->hsj", q[0].double(), k[0, :, 0].double()) * 0.5
    z = z.masked_fill(~torch.ones(S, S, dtype=torch.bool).tril(), float("-inf"))
    w = torch.softmax(z, dim=-1).permute(1, 0, 2)       # [s, h, j]
    assert (o[0] - w).abs().max().item() < 1e-14


def test_future_keys_and_values_cannot_change_a_row():
    B, S, Hq, Hkv, D = 1, 12, 4, 2, 16
    q = _rand((B, S, Hq, D), 61)
    k = _rand((B, S, Hkv, D), 62)
    v = _rand((B, S, Hkv, D), 63)
    o = oracle.attn(q, _cache_from_bshd(k), _cache_from_bshd(v))
    k2, v2 = k.clone(), v.clone()
    k2[:, 7:] = _rand((B, S - 7, Hkv, D), 64) * 10
    v2[:, 7:] = _rand((B, S - 7, Hkv, D), 65) * 10
    o2 = oracle.attn(q, _cache_from_bshd(k2), _cache_from_bshd(v2))
    assert torch.equal(o[:, :7], o2[:, :7])
    assert not torch.equal(o[:, 7:], o2[:, 7:])


def test_output_stays_inside_the_values_hull():
    B, S, Hq, Hkv, D = 1, 16, 2, 2, 8
    q = _rand((B, S, Hq, D), 71) * 4
    k = _rand((B, S, Hkv, D), 72)
    v = _rand((B, S, Hkv, D), 73)
    o = oracle.attn(q, _cache_from_bshd(k), _cache_from_bshd(v))
    vmin = v.double().cummin(dim=1).values
    vmax = v.double().cummax(dim=1).values
    assert (o >= vmin - 1e-14).all() and (o <= vmax + 1e-14).all()


def test_shift_of_all_positions_leaves_attention_unchanged():
    # RoPE's relative property carried through attention: rotating q and k at
    # positions p + 1000 instead of p gives the same output.
    B, S, Hq, Hkv, D = 1, 9, 4, 2, 32
    q = _rand((B, S, Hq, D), 81)
    k = _rand((B, S, Hkv, D), 82)
    v = _rand((B, S, Hkv, D), 83)
    outs = []
    for shift in (0, 1000):
        p0 = torch.tensor([shift], dtype=torch.int32)
        qr = oracle.rope_f64(q, p0).float()
        kr = oracle.rope_f64(k, p0).float()
        outs.append(oracle.attn(qr, _cache_from_bshd(kr), _cache_from_bshd(v)))
    # float32 storage of the rotated inputs bounds the agreement.
    assert (outs[0] - outs[1]).abs().max().item() < 1e-5


def test_bf16_inputs_are_read_exactly():
    B, S, Hq, Hkv, D = 1, 7, 2, 1, 16
    q = _rand((B, S, Hq, D), 91, torch.bfloat16)
    k = _rand((B, S, Hkv, D), 92, torch.bfloat16)
    v = _rand((B, S, Hkv, D), 93, torch.bfloat16)
    o = oracle.attn(q, _cache_from_bshd(k), _cache_from_bshd(v))
    o32 = oracle.attn(q.float(), _cache_from_bshd(k.float()), _cache_from_bshd(v.float()))
    assert torch.equal(o, o32)


def test_group_divisibility_and_capacity_are_checked():
    q = _rand((1, 4, 3, 8), 1)
    k = _rand((1, 4, 2, 8), 2)
    with pytest.raises(oracle.OracleError):
        oracle.attn(q, _cache_from_bshd(k), _cache_from_bshd(k))
    q = _rand((1, 4, 2, 8), 1)
    with pytest.raises(oracle.OracleError):
        oracle.attn(q, _cache_from_bshd(k), _cache_from_bshd(k), q_start=torch.tensor([1], dtype=torch.int32))
