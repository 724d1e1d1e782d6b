"""GPU parity: causal GQA over packed documents against the fp64 oracle."""
import math

import pytest
import torch

import oracle
import rope_gqa_causal_amd as rgc
from rope_gqa_causal_amd import synth
from _util import assert_close

pytestmark = pytest.mark.gpu

LSE_TOL_BF16 = math.log1p(2.0 ** -9) + 1e-4


def _packed(T, Hq, Hkv, D, seed):
    g = synth.generator(seed)
    return (synth.normal((T, Hq, D), g), synth.normal((T, Hkv, D), g), synth.normal((T, Hkv, D), g))


VARLEN_CASES = [
    # Hq, Hkv, D, document lengths
    (6, 2, 128, [300, 1, 0, 256, 257, 77]),   # empty and one-token documents, tile edges
    (8, 8, 64, [1000, 24]),                   # g = 1
    (4, 1, 32, [5, 5, 5, 5, 5, 5, 5]),        # many tiny documents, MQA
    (24, 8, 128, [700, 513, 64, 33]),         # the 3.8B head layout
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"H{c[0]}/{c[1]}D{c[2]}n{len(c[3])}")
def test_varlen_prefill_bf16(case):
    Hq, Hkv, D, lens = case
    cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0)), dtype=torch.int32)
    T = int(cu[-1])
    q, k, v = _packed(T, Hq, Hkv, D, T + D)
    ref, ref_lse = oracle.attn_varlen(q, k, v, cu, want_lse=True)
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = rgc.gqa_attn_prefill_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), max(lens), lse=lse, err_flag=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert_close(o, ref, torch.bfloat16, "varlen prefill")
    assert (lse.cpu().double() - ref_lse).abs().max().item() < LSE_TOL_BF16


def test_one_document_equals_the_padded_prefill_bit_for_bit():
    T, Hq, Hkv, D = 333, 6, 2, 128
    q, k, v = [t.cuda() for t in _packed(T, Hq, Hkv, D, 5)]
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    a = rgc.gqa_attn_prefill_varlen(q, k, v, cu, T)
    b = rgc.gqa_attn_prefill(q[None], k.transpose(0, 1)[None], v.transpose(0, 1)[None])[0]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_malformed_offsets_are_flagged_and_other_documents_still_computed():
    Hq, Hkv, D = 4, 2, 64
    lens = [40, 30, 20]
    T = sum(lens)
    q, k, v = _packed(T, Hq, Hkv, D, 9)
    bad = torch.tensor([0, 40, 30, 90], dtype=torch.int32)   # document 1 runs backwards
    o = torch.full((T, Hq, D), 7.0, dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rgc.gqa_attn_prefill_varlen(q.cuda(), k.cuda(), v.cuda(), bad.cuda(), 60, out=o, err_flag=err)
    assert err.item() == 1
    # Document 2 (tokens 30..89) overlaps document 0's last rows; rows 0..29
    # belong to document 0 alone.
    good = torch.tensor([0, 40], dtype=torch.int32)
    ref = oracle.attn_varlen(q[:40], k[:40], v[:40], good)
    assert_close(o[:30], ref[:30], torch.bfloat16, "document before the malformed one")
    # A document longer than max_seqlen is flagged, not truncated silently.
    err.zero_()
    rgc.gqa_attn_prefill_varlen(q.cuda(), k.cuda(), v.cuda(), torch.tensor([0, 90], dtype=torch.int32,
                                device="cuda"), 64, out=o, err_flag=err)
    assert err.item() == 1


def test_varlen_workload_full_size_sampled_documents():
    # The packed workload (16384 tokens in documents of 64..4096 tokens, 24 q /
    # 8 KV heads, D 128) launched as the bench times it; the oracle checks the
    # shortest documents whole and row blocks of the longest.
    w = synth.WORKLOADS["varlen"]
    g = synth.generator(w.seed)
    lens = synth.document_lengths(w.S, w.len_lo, w.len_hi, g)
    cu = torch.cat([torch.zeros(1, dtype=torch.int32), lens.cumsum(0).to(torch.int32)])
    q = synth.normal((w.S, w.Hq, w.D), g)
    k = synth.normal((w.S, w.Hkv, w.D), g)
    v = synth.normal((w.S, w.Hkv, w.D), g)
    o = rgc.gqa_attn_prefill_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), int(lens.max())).cpu()
    order = torch.argsort(lens)
    for i in order[:3].tolist():                      # shortest documents, whole
        a, b = int(cu[i]), int(cu[i + 1])
        ref = oracle.attn_varlen(q[a:b], k[a:b], v[a:b], torch.tensor([0, b - a], dtype=torch.int32))
        assert_close(o[a:b], ref, torch.bfloat16, f"document {i}")
    i = int(order[-1])                                 # longest document, sampled row blocks
    a, b = int(cu[i]), int(cu[i + 1])
    kc, vc = k[a:b].transpose(0, 1)[None], v[a:b].transpose(0, 1)[None]
    for s0, s1 in ((0, 32), ((b - a) // 2, (b - a) // 2 + 32), (b - a - 32, b - a)):
        ref = oracle.attn(q[a + s0:a + s1][None], kc, vc, torch.tensor([s0], dtype=torch.int32))[0]
        assert_close(o[a + s0:a + s1], ref, torch.bfloat16, f"document {i} rows {s0}..{s1}")
