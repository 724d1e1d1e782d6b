"""Write tests/golden/tiny_oracle.json: a regression record of the oracle.

Runs the fp64 oracle (and nothing else) on the seeded ``tiny`` workload: RoPE
on q and k at positions 0..23, the 16-token causal prefill and the 8 cached
decode steps, then stores every 17th output value.  The test-suite re-runs
the oracle and compares, so any later change to the oracle's arithmetic shows.
"""
import json
import os
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from rope_gqa_causal_amd import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")


def run():
    w = synth.WORKLOADS["tiny"]
    g = synth.generator(w.seed)
    T = w.S + w.steps
    q, k, v = synth.qkv(w.B, T, w.Hq, w.Hkv, w.D, g, w.dtype)
    oracle.rope_apply_(q, None, synth.BASE)
    oracle.rope_apply_(k, None, synth.BASE)
    kc = torch.zeros((w.B, w.Hkv, T, w.D), dtype=w.dtype)
    vc = torch.zeros_like(kc)
    zero = torch.zeros(w.B, dtype=torch.int32)
    oracle.kv_cache_append_(kc, vc, k[:, :w.S], v[:, :w.S], zero)
    pre = oracle.attn(q[:, :w.S], kc, vc)
    dec = []
    lens = torch.full((w.B,), w.S, dtype=torch.int32)
    for t in range(w.steps):
        s = w.S + t
        oracle.kv_cache_append_(kc, vc, k[:, s:s + 1], v[:, s:s + 1], lens)
        lens += 1
        dec.append(oracle.attn_decode(q[:, s], kc, vc, lens))
    dec = torch.stack(dec, dim=1)
    return pre, dec


def main():
    pre, dec = run()
    rec = {
        "_about": "fp64 oracle on the seeded tiny workload (seed 1); every 17th value. "
                  "Written by tests/golden/make_tiny_fixture.py, which calls only oracle/.",
        "prefill_every17": pre.reshape(-1)[::17].tolist(),
        "decode_every17": dec.reshape(-1)[::17].tolist(),
    }
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=0)


if __name__ == "__main__":
    main()
