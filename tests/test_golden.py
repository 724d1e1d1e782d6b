"""Stored facts: the pages' printed numbers, and the oracle's regression record."""
import json
import os

import torch

from rope_gqa_causal_amd import synth

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)


def test_large_workload_heads_follow_the_3p8b_parameter_table():
    # The 3.8B page prints 24 query / 8 KV heads and a parameter table; the
    # token embedding (vocab x d_model) and the 14 value-embedding tables
    # (vocab x kv_dim) fix d_model = 3072 = 24 x 128 and kv_dim = 1024 = 8 x 128.
    facts = _load("pages_facts.json")
    heads = facts["little_lm_3p8b_heads"]
    table = facts["little_lm_3p8b_param_table"]
    d_model = table["token_embedding_params_M"] * 1e6 / table["padded_vocab"]
    kv_dim = table["value_embedding_params_M"] * 1e6 / table["value_embedding_tables"] / table["padded_vocab"]
    for name in ("prefill3p8b", "ragged_decode"):
        w = synth.WORKLOADS[name]
        assert (w.Hq, w.Hkv) == (heads["query_heads"], heads["kv_heads"])
        assert abs(d_model - w.Hq * w.D) < 3072 * 0.002
        assert abs(kv_dim - w.Hkv * w.D) < 1024 * 0.002


def test_generation_workload_follows_the_cached_generation_experiment():
    facts = _load("pages_facts.json")["cached_generation"]
    w = synth.WORKLOADS["llama125m"]
    assert (w.S, w.steps) == (facts["prompt_tokens"], facts["new_tokens"])


def test_oracle_regression_record():
    import sys
    sys.path.insert(0, HERE)
    import make_tiny_fixture
    rec = _load("tiny_oracle.json")
    pre, dec = make_tiny_fixture.run()
    assert torch.equal(pre.reshape(-1)[::17], torch.tensor(rec["prefill_every17"], dtype=torch.float64))
    assert torch.equal(dec.reshape(-1)[::17], torch.tensor(rec["decode_every17"], dtype=torch.float64))
