"""GPU parity on the named workloads, end to end (RoPE -> append -> attention).

* tiny (fp32): the whole path, every output element, at 1e-5.
* llama125m (bf16): two of the twelve independent layers, prefill 512 then
  100 cached decode steps, every output element; a third layer with every
  step as one gqa_attn_decode_rope_append call.
* prefill3p8b and ragged_decode at full size, in the launch configuration
  the benchmark times: sampled rows checked against the oracle row by row.
"""
import pytest
import torch

import oracle
import rope_gqa_causal_amd as rgc
from rope_gqa_causal_amd import synth
from _util import assert_close

pytestmark = pytest.mark.gpu


def _oracle_chain(w, q, k, v, S_max):
    """Oracle: rope q,k (rounded once), append, prefill, then decode steps."""
    q, k = q.clone(), k.clone()
    oracle.rope_apply_(q, None, synth.BASE)
    oracle.rope_apply_(k, None, synth.BASE)
    kc = torch.zeros((w.B, w.Hkv, S_max, w.D), dtype=w.dtype)
    vc = torch.zeros_like(kc)
    oracle.kv_cache_append_(kc, vc, k[:, :w.S], v[:, :w.S], torch.zeros(w.B, dtype=torch.int32))
    pre = oracle.attn(q[:, :w.S], kc, vc)
    dec = []
    lens = torch.full((w.B,), w.S, dtype=torch.int32)
    for t in range(w.steps):
        s = w.S + t
        oracle.kv_cache_append_(kc, vc, k[:, s:s + 1], v[:, s:s + 1], lens)
        lens += 1
        dec.append(oracle.attn_decode(q[:, s], kc, vc, lens))
    return pre, torch.stack(dec, dim=1)


def _gpu_chain(w, q, k, v, S_max):
    """GPU: the same steps through the C ABI, one call per step."""
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    T = w.S + w.steps
    pos0 = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    rgc.rope_apply(q[:, :w.S], pos0)
    rgc.rope_apply(k[:, :w.S], pos0)
    kc = torch.zeros((w.B, w.Hkv, S_max, w.D), dtype=w.dtype, device="cuda")
    vc = torch.zeros_like(kc)
    rgc.kv_cache_append(kc, vc, k[:, :w.S], v[:, :w.S], pos0)
    pre = rgc.gqa_attn_prefill(q[:, :w.S], kc, vc, pos0)
    lens = torch.full((w.B,), w.S, dtype=torch.int32, device="cuda")
    ws = rgc.decode_workspace(w.B, w.Hq, w.Hkv, w.D, T)
    dec = []
    for t in range(w.steps):
        s = w.S + t
        qs, ks = q[:, s:s + 1], k[:, s:s + 1]
        rgc.rope_apply(qs, lens)
        rgc.rope_apply(ks, lens)
        rgc.kv_cache_append(kc, vc, ks, v[:, s:s + 1], lens)
        lens += 1
        dec.append(rgc.gqa_attn_decode(qs[:, 0], kc, vc, lens, T, ws))
    return pre, torch.stack(dec, dim=1)


def _gpu_chain_one_launch(w, q, k, v, S_max):
    """GPU: the prompt as above, then each new token's RoPE, append and
    decode in one gqa_attn_decode_rope_append call (q and k unrotated)."""
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    T = w.S + w.steps
    pos0 = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    qp, kp = q[:, :w.S].clone(), k[:, :w.S].clone()
    rgc.rope_apply(qp, pos0)
    rgc.rope_apply(kp, pos0)
    kc = torch.zeros((w.B, w.Hkv, S_max, w.D), dtype=w.dtype, device="cuda")
    vc = torch.zeros_like(kc)
    rgc.kv_cache_append(kc, vc, kp, v[:, :w.S], pos0)
    pre = rgc.gqa_attn_prefill(qp, kc, vc, pos0)
    lens = torch.full((w.B,), w.S, dtype=torch.int32, device="cuda")
    ws = rgc.decode_workspace(w.B, w.Hq, w.Hkv, w.D, T)
    dec = []
    for t in range(w.steps):
        s = w.S + t
        lens += 1
        dec.append(rgc.gqa_attn_decode_rope_append(q[:, s], k[:, s], v[:, s], kc, vc, lens, T, ws))
    return pre, torch.stack(dec, dim=1)


def test_tiny_workload_end_to_end_fp32():
    w = synth.WORKLOADS["tiny"]
    T = w.S + w.steps
    q, k, v = synth.qkv(w.B, T, w.Hq, w.Hkv, w.D, synth.generator(w.seed), w.dtype)
    ref_pre, ref_dec = _oracle_chain(w, q, k, v, T)
    pre, dec = _gpu_chain(w, q, k, v, T)
    assert_close(pre, ref_pre, torch.float32, "tiny prefill")
    assert_close(dec, ref_dec, torch.float32, "tiny decode")


@pytest.mark.parametrize("layer", [0, 11])
def test_llama125m_layer_end_to_end_bf16(layer):
    w = synth.WORKLOADS["llama125m"]
    T = w.S + w.steps
    g = synth.generator(w.seed * 1000 + layer)
    q, k, v = synth.qkv(w.B, T, w.Hq, w.Hkv, w.D, g, w.dtype)
    ref_pre, ref_dec = _oracle_chain(w, q, k, v, T)
    pre, dec = _gpu_chain(w, q, k, v, T)
    assert_close(pre, ref_pre, torch.bfloat16, "125m prefill")
    assert_close(dec, ref_dec, torch.bfloat16, "125m decode")


def test_llama125m_layer_end_to_end_one_launch_steps():
    w = synth.WORKLOADS["llama125m"]
    T = w.S + w.steps
    g = synth.generator(w.seed * 1000 + 5)
    q, k, v = synth.qkv(w.B, T, w.Hq, w.Hkv, w.D, g, w.dtype)
    ref_pre, ref_dec = _oracle_chain(w, q, k, v, T)
    pre, dec = _gpu_chain_one_launch(w, q, k, v, T)
    assert_close(pre, ref_pre, torch.bfloat16, "125m prefill")
    assert_close(dec, ref_dec, torch.bfloat16, "125m one-launch decode steps")


@pytest.mark.parametrize("seed_off", [0, 100, 200])
def test_prefill3p8b_full_size_sampled_rows(seed_off):
    w = synth.WORKLOADS["prefill3p8b"]
    g = synth.generator(w.seed + seed_off)
    q, k, v = synth.qkv(w.B, w.S, w.Hq, w.Hkv, w.D, g, w.dtype)
    kc = k.transpose(1, 2).contiguous()
    vc = v.transpose(1, 2).contiguous()
    o = rgc.gqa_attn_prefill(q.cuda(), kc.cuda(), vc.cuda()).cpu()
    sg = synth.generator(99 + seed_off)
    for b in range(w.B):
        s0 = int(torch.randint(0, w.S - 16, (1,), generator=sg))
        for lo in (s0, w.S - 16):
            rows = slice(lo, lo + 16)
            ref = oracle.attn(q[b:b + 1, rows], kc[b:b + 1], vc[b:b + 1],
                              torch.tensor([lo], dtype=torch.int32))
            assert_close(o[b:b + 1, rows], ref, torch.bfloat16, f"3.8B b={b} rows {lo}")


@pytest.mark.parametrize("seed_off", [0, 100, 200])
def test_ragged_decode_full_size_sampled_sequences(seed_off):
    w = synth.WORKLOADS["ragged_decode"]
    g = synth.generator(w.seed + seed_off)
    lens0 = synth.lengths(w.B, w.len_lo, w.len_hi, g)
    S_max = w.len_hi + w.steps
    kc, vc = synth.filled_cache(w.B, w.Hkv, S_max, w.D, g, w.dtype)
    q = synth.normal((w.B, w.Hq, w.D), g, w.dtype)
    lens = lens0 + 1
    kg, vg = kc.cuda(), vc.cuda()
    ws = rgc.decode_workspace(w.B, w.Hq, w.Hkv, w.D, S_max)
    o = rgc.gqa_attn_decode(q.cuda(), kg, vg, lens.cuda(), S_max, ws).cpu()
    for b in [0, 1, 17, 33, 63] + [int(torch.argmax(lens)), int(torch.argmin(lens))]:
        ref = oracle.attn_decode(q[b:b + 1], kc[b:b + 1], vc[b:b + 1], lens[b:b + 1])
        assert_close(o[b:b + 1], ref, torch.bfloat16, f"ragged decode b={b} L={int(lens[b])}")
