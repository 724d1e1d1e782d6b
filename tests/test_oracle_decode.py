"""Pins of the oracle's cache append and cached decode.

Page "750美元从零训练3个LLM：一位开发者的实战复盘", section V3: the cache
stores each step's K and V, the new token computes only its own q, k, v and
attends over the cache, and outputs with and without the cache agree.  Page
"从零手训LLaMa：125M模型11小时训练全记录" (core-architecture section): the
per-layer cache grows by one row per step, and generation becomes linear per
step.  Decode is therefore pinned to the uncached recompute.
"""
import pytest
import torch

import oracle
from rope_gqa_causal_amd import synth


def test_append_is_an_exact_copy_at_the_right_slots_and_nothing_else():
    B, Hkv, S_max, D, S_new = 3, 2, 12, 8, 4
    g = synth.generator(5)
    kc, vc = synth.nan_cache(B, Hkv, S_max, D)
    k_new = synth.normal((B, S_new, Hkv, D), g)
    v_new = synth.normal((B, S_new, Hkv, D), g)
    pos0 = torch.tensor([0, 5, 8], dtype=torch.int32)
    assert oracle.kv_cache_append_(kc, vc, k_new, v_new, pos0) == 0
    for b in range(B):
        p = pos0[b].item()
        want_k = torch.full((Hkv, S_max, D), float("nan"), dtype=torch.bfloat16)
        want_k[:, p:p + S_new] = k_new[b].transpose(0, 1)
        assert torch.equal(kc[b].view(torch.int16), want_k.view(torch.int16))
        want_v = torch.full((Hkv, S_max, D), float("nan"), dtype=torch.bfloat16)
        want_v[:, p:p + S_new] = v_new[b].transpose(0, 1)
        assert torch.equal(vc[b].view(torch.int16), want_v.view(torch.int16))


def test_append_refuses_slots_beyond_capacity():
    kc, vc = synth.nan_cache(1, 1, 4, 8)
    new = synth.normal((1, 3, 1, 8), synth.generator(6))
    st = oracle.kv_cache_append_(kc, vc, new, new, torch.tensor([2], dtype=torch.int32))
    assert st == -7  # capacity: the two valid rows are copied, the third is refused
    assert torch.equal(kc[0, 0, 2:4].view(torch.int16), new[0, :2, 0].view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_cached_decode_equals_uncached_recompute(dtype):
    # Prefill P tokens, then append one token per step and decode it; each
    # decode output must equal the last row of attention recomputed from
    # scratch over the whole prefix (no cache).
    B, Hq, Hkv, D, P, T = 2, 6, 2, 16, 5, 6
    S_max = P + T
    g = synth.generator(7)
    q_all, k_all, v_all = synth.qkv(B, P + T, Hq, Hkv, D, g, dtype)
    kc, vc = synth.nan_cache(B, Hkv, S_max, D, dtype)
    lens = torch.zeros(B, dtype=torch.int32)
    oracle.kv_cache_append_(kc, vc, k_all[:, :P], v_all[:, :P], lens)
    lens += P
    for t in range(T):
        s = P + t
        oracle.kv_cache_append_(kc, vc, k_all[:, s:s + 1], v_all[:, s:s + 1], lens)
        lens += 1
        o_dec = oracle.attn_decode(q_all[:, s], kc, vc, lens)
        full = oracle.attn(q_all[:, :s + 1], k_all[:, :s + 1].transpose(1, 2),
                           v_all[:, :s + 1].transpose(1, 2))
        assert (o_dec - full[:, -1]).abs().max().item() < 1e-12


def test_ragged_batch_equals_one_sequence_at_a_time():
    B, Hq, Hkv, D, S_max = 4, 4, 2, 32, 40
    g = synth.generator(8)
    kc, vc = synth.filled_cache(B, Hkv, S_max, D, g, torch.float32)
    q = synth.normal((B, Hq, D), g, torch.float32)
    lens = synth.lengths(B, 1, S_max, g)
    o = oracle.attn_decode(q, kc, vc, lens)
    for b in range(B):
        ob = oracle.attn_decode(q[b:b + 1], kc[b:b + 1], vc[b:b + 1], lens[b:b + 1])
        assert torch.equal(o[b:b + 1], ob)


def test_decode_never_reads_slots_at_or_beyond_the_length():
    B, Hq, Hkv, D, S_max = 2, 2, 1, 8, 16
    g = synth.generator(9)
    kc, vc = synth.nan_cache(B, Hkv, S_max, D)
    lens = torch.tensor([3, 16], dtype=torch.int32)
    for b in range(B):
        L = lens[b].item()
        kc[b, :, :L] = synth.normal((Hkv, L, D), g)
        vc[b, :, :L] = synth.normal((Hkv, L, D), g)
    q = synth.normal((B, Hq, D), g)
    o = oracle.attn_decode(q, kc, vc, lens)
    assert torch.isfinite(o).all()


def test_decode_rejects_lengths_outside_the_cache():
    kc, vc = synth.filled_cache(1, 1, 8, 8, synth.generator(10))
    q = synth.normal((1, 1, 8), synth.generator(11))
    for bad in (0, 9):
        with pytest.raises(oracle.OracleError):
            oracle.attn_decode(q, kc, vc, torch.tensor([bad], dtype=torch.int32))
