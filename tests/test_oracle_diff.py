"""Pins of the oracle's differential attention.

Page "750美元从零训练3个LLM：一位开发者的实战复盘", section V2: DiffAttn
computes two attention maps and takes their difference so that noise common
to both cancels.  Reading taken: o = sum_j (w1_j - lambda * w2_j) v_j with a
constant lambda.  Pinned by the cases that reduce it to plain attention and
by literal loops.
"""
import math

import torch

import oracle
from rope_gqa_causal_amd import synth


def _inputs(B, S, Hq, Hkv, D, seed, dtype=torch.float32):
    g = synth.generator(seed)
    q1 = synth.normal((B, S, Hq, D), g, dtype)
    q2 = synth.normal((B, S, Hq, D), g, dtype)
    k1 = synth.normal((B, S, Hkv, D), g, dtype).transpose(1, 2)
    k2 = synth.normal((B, S, Hkv, D), g, dtype).transpose(1, 2)
    v = synth.normal((B, S, Hkv, D), g, dtype).transpose(1, 2)
    return q1, q2, k1, k2, v


def test_lambda_zero_is_plain_attention():
    q1, q2, k1, k2, v = _inputs(2, 9, 4, 2, 16, 1)
    o = oracle.diff_attn(q1, q2, k1, k2, v, 0.0)
    assert (o - oracle.attn(q1, k1, v)).abs().max().item() < 1e-14


def test_identical_maps_scale_by_one_minus_lambda():
    q1, _, k1, _, v = _inputs(1, 11, 4, 2, 16, 2)
    o = oracle.diff_attn(q1, q1, k1, k1, v, 0.8)
    assert (o - 0.2 * oracle.attn(q1, k1, v)).abs().max().item() < 1e-14


def test_weight_rows_sum_to_one_minus_lambda():
    q1, q2, k1, k2, _ = _inputs(1, 10, 2, 1, 8, 3)
    ones = torch.ones((1, 1, 10, 8))
    o = oracle.diff_attn(q1, q2, k1, k2, ones, 0.8)
    assert (o - 0.2).abs().max().item() < 1e-14


def test_matches_literal_loops():
    B, S, Hq, Hkv, D, lam, scale = 1, 5, 4, 2, 4, 0.8, 0.5
    q1, q2, k1, k2, v = _inputs(B, S, Hq, Hkv, D, 4)
    o = oracle.diff_attn(q1, q2, k1, k2, v, lam, scale=scale)
    g = Hq // Hkv
    for s in range(S):
        for h in range(Hq):
            kh = h // g
            def weights(q, k):
                z = [scale * sum(float(q[0, s, h, d]) * float(k[0, kh, j, d]) for d in range(D))
                     for j in range(s + 1)]
                m = max(z)
                e = [math.exp(t - m) for t in z]
                return [t / sum(e) for t in e]
            w1, w2 = weights(q1, k1), weights(q2, k2)
            for d in range(D):
                want = sum((w1[j] - lam * w2[j]) * float(v[0, kh, j, d]) for j in range(s + 1))
                assert abs(o[0, s, h, d].item() - want) < 1e-12
