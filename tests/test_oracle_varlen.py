"""Pins of the oracle's packed-document (varlen) causal attention.

Document masking (page "训练3.8B LLM至0.384 CORE，成本998美元 – Hugo Vergnes",
section 无效的方法): with several documents packed into one token sequence,
each token attends only to the tokens of its own document, causally.  The
oracle runs one plain causal attention per document; these tests pin it to
torch float64 scaled_dot_product_attention with an explicit block-diagonal
causal mask, and to the invariances of the definition.
"""
import torch
import torch.nn.functional as F

import oracle
from rope_gqa_causal_amd import synth


def _packed(T, Hq, Hkv, D, seed, dtype=torch.bfloat16):
    g = synth.generator(seed)
    return (synth.normal((T, Hq, D), g, dtype), synth.normal((T, Hkv, D), g, dtype),
            synth.normal((T, Hkv, D), g, dtype))


def _doc_mask(cu, T):
    doc = torch.empty(T, dtype=torch.int64)
    for i, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        doc[a:b] = i
    pos = torch.arange(T)
    return (doc[:, None] == doc[None, :]) & (pos[None, :] <= pos[:, None])


def test_matches_sdpa_with_block_diagonal_causal_mask():
    Hq, Hkv, D = 6, 2, 32
    cu = [0, 5, 5, 17, 18, 40]          # includes an empty and a one-token document
    T = cu[-1]
    q, k, v = _packed(T, Hq, Hkv, D, 31)
    ours, lse = oracle.attn_varlen(q, k, v, torch.tensor(cu, dtype=torch.int32), want_lse=True)
    g = Hq // Hkv
    qd = q.to(torch.float64).transpose(0, 1)[None]                     # [1,Hq,T,D]
    kd = k.to(torch.float64).repeat_interleave(g, dim=1).transpose(0, 1)[None]
    vd = v.to(torch.float64).repeat_interleave(g, dim=1).transpose(0, 1)[None]
    ref = F.scaled_dot_product_attention(qd, kd, vd, attn_mask=_doc_mask(cu, T))[0].transpose(0, 1)
    assert torch.allclose(ours, ref, atol=1e-12, rtol=0)
    s = (qd @ kd.transpose(-1, -2))[0] * D ** -0.5
    s = s.masked_fill(~_doc_mask(cu, T), float("-inf"))
    assert torch.allclose(lse, torch.logsumexp(s, dim=-1), atol=1e-12, rtol=0)


def test_one_document_is_plain_causal_attention():
    T, Hq, Hkv, D = 23, 4, 4, 16
    q, k, v = _packed(T, Hq, Hkv, D, 32, torch.float32)
    ours = oracle.attn_varlen(q, k, v, torch.tensor([0, T], dtype=torch.int32))
    plain = oracle.attn(q[None], k.transpose(0, 1)[None], v.transpose(0, 1)[None])[0]
    assert torch.equal(ours, plain)


def test_other_documents_cannot_change_a_row():
    T, Hq, Hkv, D = 30, 2, 1, 16
    cu = torch.tensor([0, 10, 22, 30], dtype=torch.int32)
    q, k, v = _packed(T, Hq, Hkv, D, 33, torch.float32)
    a = oracle.attn_varlen(q, k, v, cu)
    k2, v2 = k.clone(), v.clone()
    k2[:10] += 5.0
    v2[22:] -= 3.0            # documents 0 and 2 change; document 1 must not
    b = oracle.attn_varlen(q, k2, v2, cu)
    assert torch.equal(a[10:22], b[10:22])
    assert not torch.equal(a[:10], b[:10])
