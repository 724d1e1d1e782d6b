"""Benchmark of the causal GQA + RoPE path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  prefill phase  (24 query / 8 KV heads, head dim 128, batch 8 x 2048 tokens):
                 fused RoPE on q and k + cache append, causal GQA prefill;
  decode phase   (64 sequences, cache lengths uniform on {256..2048}, same
                 heads): 32 generation steps, each one launch of the cached
                 GQA decode with the new token's RoPE (q and k) and the
                 append of its k and v inside, plus the chunk merge (the
                 lengths of every step are precomputed once, as a serving
                 loop knows them).
`value` is the decode phase's KV-read rate (cache bytes every decode call
must read / decode-phase time, GB/s); the prefill phase's attention rate is
reported beside it (TFLOP/s over unmasked query-key pairs).  Both are also
given per kernel against the MI355X peaks (HBM 8 TB/s; dense bf16 MFMA
2.5 PFLOP/s), from HIP events recorded on the stream the kernels run on: the
decode's dominant kernel (the split-K kernel that streams the cache) is timed
by the library's per-kernel events, and the whole decode op (split + merge)
is reported beside it.
The differential-attention variant (`diff_attn`), the packed-document prefill
(`varlen_prefill`), the fused prologue with and without QK normalisation
(`prologue`), the attention backward (`backward`) and the 125M-shaped cached
versus recomputed generation (`generation_125m`) are timed apart on their own
workloads.  The fp64 CPU oracle is timed on a bounded sample of the same
decode workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GQA decode KV-read GB/s + prefill attn TFLOP/s, % of MI355X roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the CPU-oracle sample")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the variant lines (diff, varlen, prologue, backward, generation)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration runs)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, WRITE_SIZE; both "
                         "with --copy-calibration) into profiles/counters_*.json and exit")
    return ap.parse_args()


def kernel_sha(name):
    with open(os.path.join(ROOT, "rope_gqa_causal_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic(kind, src, launches_bytes):
    """HBM bytes per launch from committed counter runs, if the kernel is unchanged."""
    path = os.path.join(PROFILES, f"counters_{kind}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    if rec.get("kernel_sha") != kernel_sha(src):
        return None
    return rec.get("traffic_bytes_per_launch")


def _pmc_per_dispatch(run_dir, counter):
    """{kernel short name: [value summed over the dispatch's instances, ...]} from a rocpd database."""
    import glob
    import sqlite3
    dbs = glob.glob(os.path.join(run_dir, "**", "*.db"), recursive=True)
    if not dbs:
        raise SystemExit(f"no rocpd database under {run_dir}")
    per = {}
    for path in dbs:
        rows = sqlite3.connect(path).execute(
            "select dispatch_id, kernel_name, counter_name, value from counters_collection").fetchall()
        for did, kname, cname, val in rows:
            if cname != counter:
                continue
            short = kname.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            short = short.split("<")[0].split("::")[-1]
            per.setdefault(short, {}).setdefault((path, did), 0.0)
            per[short][(path, did)] += val
    return {k: [v for _, v in sorted(d.items())] for k, d in per.items()}


def summarize_pmc(fetch_dir, write_dir):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the decode and prefill kernels,
    scaled by what the same counters read for a plain 1 GiB device copy."""
    copy_bytes = float(1 << 30)
    out = {}
    cal = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _pmc_per_dispatch(d, counter)
        copies = [v for k, vs in per.items() if "copy" in k.lower() for v in vs]
        if not copies:
            raise SystemExit(f"{counter}: no copy kernel in {d} (run with --copy-calibration)")
        cal[counter] = copy_bytes / (max(copies) * 1024.0)
        avg = {k: sum(vs) / len(vs) for k, vs in per.items()}
        out[counter] = avg
    kib = lambda c, k: out[c].get(k, 0.0)
    def record(kind, src, kernels, note):
        fetch = sum(kib("FETCH_SIZE", k) for k in kernels)
        write = sum(kib("WRITE_SIZE", k) for k in kernels)
        rec = {
            "kernel": " + ".join(kernels), "kernel_sha": kernel_sha(src),
            "fetch_kib_per_launch": round(fetch, 1), "write_kib_per_launch": round(write, 1),
            "copy_scale": {"FETCH_SIZE": round(cal["FETCH_SIZE"], 4), "WRITE_SIZE": round(cal["WRITE_SIZE"], 4)},
            "traffic_bytes_per_launch": round(fetch * 1024 * cal["FETCH_SIZE"] + write * 1024 * cal["WRITE_SIZE"]),
            "note": note,
        }
        with open(os.path.join(PROFILES, f"counters_{kind}.json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(kind, json.dumps(rec))
    record("decode", "decode.hip", ["decode_split_kernel"],
           "the decode's dominant kernel (with the token's RoPE and append inside), average over the 32 "
           "decode calls of one bench step (cache lengths grow by one per call)")
    record("decode_op", "decode.hip", ["decode_split_kernel", "decode_combine_kernel"],
           "the whole one-launch decode step (split + merge), average over the 32 decode calls of one bench step")
    record("prefill", "prefill.hip", ["prefill_kernel"], "one prefill launch of the bench step")


class Prefill:
    def __init__(self, rgc, synth):
        w = synth.WORKLOADS["prefill3p8b"]
        self.w = w
        g = synth.generator(w.seed)
        q, k, v = synth.qkv(w.B, w.S, w.Hq, w.Hkv, w.D, g, w.dtype)
        self.q, self.k, self.v = q.cuda(), k.cuda(), v.cuda()
        self.kc = torch.empty((w.B, w.Hkv, w.S, w.D), dtype=w.dtype, device="cuda")
        self.vc = torch.empty_like(self.kc)
        self.o = torch.empty_like(self.q)
        self.pos0 = torch.zeros(w.B, dtype=torch.int32, device="cuda")
        self.rgc = rgc
        self.flops = 4.0 * w.D * w.B * w.Hq * w.S * (w.S + 1) / 2  # unmasked pairs x 4D
        self.events = []

    def run(self, record):
        r = self.rgc
        # RoPE on q and k and the cache append in one fused pass.
        r.rope_append(self.q, self.k, self.v, self.kc, self.vc, self.pos0)
        if record:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        r.gqa_attn_prefill(self.q, self.kc, self.vc, self.pos0, out=self.o)
        if record:
            e1.record()
            self.events.append((e0, e1))


class Decode:
    def __init__(self, rgc, synth):
        w = synth.WORKLOADS["ragged_decode"]
        self.w = w
        g = synth.generator(w.seed)
        self.lens0_cpu = synth.lengths(w.B, w.len_lo, w.len_hi, g)
        self.S_max = w.len_hi + w.steps
        kc, vc = synth.filled_cache(w.B, w.Hkv, self.S_max, w.D, g, w.dtype)
        self.kc_cpu, self.vc_cpu = kc, vc
        self.kc, self.vc = kc.cuda(), vc.cuda()
        q, k, v = synth.qkv(w.B * w.steps, 1, w.Hq, w.Hkv, w.D, g, w.dtype)
        self.q = q.view(w.steps, w.B, 1, w.Hq, w.D).cuda()
        self.k = k.view(w.steps, w.B, 1, w.Hkv, w.D).cuda()
        self.v = v.view(w.steps, w.B, 1, w.Hkv, w.D).cuda()
        # Lengths of every step, computed once: step t appends at slot
        # lens0 + t and then attends over lens0 + t + 1 rows.
        steps = torch.arange(w.steps, dtype=torch.int32)[:, None]
        self.slots = (self.lens0_cpu[None, :] + steps).contiguous().cuda()
        self.lens = (self.lens0_cpu[None, :] + steps + 1).contiguous().cuda()
        self.o = torch.empty((w.B, w.Hq, w.D), dtype=w.dtype, device="cuda")
        self.ws = rgc.decode_workspace(w.B, w.Hq, w.Hkv, w.D, self.S_max)
        self.rgc = rgc
        # KV bytes the t-th decode call must read: every cached row of every
        # sequence, new token included (lengths lens0 + t + 1).
        per_token = w.Hkv * w.D * 2 * 2
        self.bytes_per_call = [per_token * float((self.lens0_cpu + t + 1).sum()) for t in range(w.steps)]

    def run(self, fused=False):
        r, w = self.rgc, self.w
        for t in range(w.steps):
            if not fused:
                # the two-launch form: RoPE (q, k at position lens0 + t) and
                # cache append, then the decode of the rotated q
                r.rope_append(self.q[t], self.k[t], self.v[t], self.kc, self.vc, self.slots[t])
                r.gqa_attn_decode(self.q[t][:, 0], self.kc, self.vc, self.lens[t], self.S_max, self.ws,
                                  out=self.o)
            else:
                # one launch (plus the chunk merge): RoPE of q and k at
                # position lens0 + t, append of k and v, attention
                r.gqa_attn_decode_rope_append(self.q[t][:, 0], self.k[t][:, 0], self.v[t][:, 0], self.kc,
                                              self.vc, self.lens[t], self.S_max, self.ws, out=self.o)


class Diff:
    """Differential attention on its own workload (B 4 x 1024 tokens, 16 q /
    8 KV heads, two maps of head dim 64, lambda 0.8); timed apart from the
    step, since it is a variant of the prefill rather than a stage of it."""

    def __init__(self, rgc, synth):
        w = synth.WORKLOADS["diff"]
        self.w = w
        g = synth.generator(w.seed)
        self.q1 = synth.normal((w.B, w.S, w.Hq, w.D), g).cuda()
        self.q2 = synth.normal((w.B, w.S, w.Hq, w.D), g).cuda()
        self.k1, self.k2, self.v = (synth.normal((w.B, w.Hkv, w.S, w.D), g).cuda() for _ in range(3))
        self.o = torch.empty_like(self.q1)
        self.rgc = rgc
        self.flops = 2 * 4.0 * w.D * w.B * w.Hq * w.S * (w.S + 1) / 2  # two maps x unmasked pairs x 4D

    def run(self):
        self.rgc.diff_attn_prefill(self.q1, self.q2, self.k1, self.k2, self.v, self.w.lam, out=self.o)

    def time(self, iters):
        for _ in range(3):
            self.run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            self.run()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / iters * 1e3
        tflops = self.flops / (us * 1e-6) / 1e12
        return {"bound": "mfma", "kernel": "diff_attn_prefill", "achieved": round(tflops, 2),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                "algorithmic_flops_per_launch": self.flops, "avg_launch_us": round(us, 3),
                "workload": "differential attention B4 x 1024, 16q/8kv, two maps of D64, lambda 0.8, bf16",
                "note": "timed apart from the step; FLOPs count both maps' unmasked pairs x 4D"}


class Varlen:
    """Document-masked prefill on the 3.8B-shaped token count: 16384 tokens
    packed as documents of 64..4096 tokens, 24 q / 8 KV heads, D 128."""

    def __init__(self, rgc, synth):
        w = synth.WORKLOADS["varlen"]
        g = synth.generator(w.seed)
        self.lens = synth.document_lengths(w.S, w.len_lo, w.len_hi, g)
        self.cu = torch.cat([torch.zeros(1, dtype=torch.int32), self.lens.cumsum(0).to(torch.int32)]).cuda()
        self.q = synth.normal((w.S, w.Hq, w.D), g).cuda()
        self.k = synth.normal((w.S, w.Hkv, w.D), g).cuda()
        self.v = synth.normal((w.S, w.Hkv, w.D), g).cuda()
        self.o = torch.empty_like(self.q)
        self.max_len = int(self.lens.max())
        n = self.lens.to(torch.float64)
        self.flops = float((n * (n + 1) / 2).sum()) * w.Hq * 4.0 * w.D
        self.rgc, self.w = rgc, w

    def time(self, iters):
        run = lambda: self.rgc.gqa_attn_prefill_varlen(self.q, self.k, self.v, self.cu, self.max_len, out=self.o)
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            run()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / iters * 1e3
        tf = self.flops / (us * 1e-6) / 1e12
        return {"bound": "mfma", "kernel": "gqa_attn_prefill_varlen", "achieved": round(tf, 2),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                "algorithmic_flops_per_launch": self.flops, "avg_launch_us": round(us, 3),
                "documents": int(self.lens.numel()),
                "workload": "16384 tokens packed as documents of U{64..4096} tokens, 24q/8kv, D128, bf16"}


class Generation:
    """Attention side of the 125M-shaped cached generation (12 layers with
    their own caches, 12 q / 4 KV heads, D 64, bf16; a 512-token prompt,
    then 100 new tokens), cached versus recomputed: the attention analogue
    of the cached-generation experiment (278 s -> 28 s for the whole model,
    hardware not stated) on page "750美元从零训练3个LLM：一位开发者的实战复盘",
    section V3."""

    def __init__(self, rgc, synth):
        w = synth.WORKLOADS["llama125m"]
        self.w, self.rgc = w, rgc
        self.total = w.S + w.steps
        g = synth.generator(w.seed)
        self.layers = []
        for _ in range(w.layers):
            q, k, v = (t.cuda() for t in synth.qkv(1, self.total, w.Hq, w.Hkv, w.D, g, w.dtype))
            kc = torch.empty((1, w.Hkv, self.total, w.D), dtype=w.dtype, device="cuda")
            self.layers.append((q, k, v, kc, torch.empty_like(kc)))
        self.qs = torch.empty_like(self.layers[0][0])
        self.o = torch.empty_like(self.layers[0][0])
        self.o1 = torch.empty((1, w.Hq, w.D), dtype=w.dtype, device="cuda")
        self.ws = rgc.decode_workspace(1, w.Hq, w.Hkv, w.D, self.total)
        steps = torch.arange(w.steps, dtype=torch.int32)
        self.slots = (w.S + steps).view(-1, 1).cuda()
        self.lens = (w.S + steps + 1).view(-1, 1).cuda()
        self.zero = torch.zeros(1, dtype=torch.int32, device="cuda")

    def cached(self):
        """Each new token's step in one decode launch (RoPE, append and attention)."""
        r, w, P = self.rgc, self.w, self.w.S
        self._prompt()
        for t in range(w.steps):
            for q, k, v, kc, vc in self.layers:
                r.gqa_attn_decode_rope_append(q[:, P + t], k[:, P + t], v[:, P + t], kc, vc, self.lens[t],
                                              self.total, self.ws, out=self.o1)

    def cached_two_launch(self):
        """The same steps as a RoPE/append launch followed by the decode."""
        r, w, P = self.rgc, self.w, self.w.S
        self._prompt()
        for t in range(w.steps):
            for q, k, v, kc, vc in self.layers:
                qt = self.qs[:, P + t:P + t + 1]
                qt.copy_(q[:, P + t:P + t + 1])
                r.rope_append(qt, k[:, P + t:P + t + 1], v[:, P + t:P + t + 1], kc, vc, self.slots[t])
                r.gqa_attn_decode(qt[:, 0], kc, vc, self.lens[t], self.total, self.ws, out=self.o1)

    def _prompt(self):
        r, P = self.rgc, self.w.S
        for q, k, v, kc, vc in self.layers:
            self.qs[:, :P].copy_(q[:, :P])
            r.rope_append(self.qs[:, :P], k[:, :P], v[:, :P], kc, vc, self.zero)
            r.gqa_attn_prefill(self.qs[:, :P], kc, vc, self.zero, out=self.o[:, :P])

    def uncached(self):
        r, w, P = self.rgc, self.w, self.w.S
        for t in range(w.steps):
            n = P + t + 1
            for q, k, v, kc, vc in self.layers:
                self.qs[:, :n].copy_(q[:, :n])
                r.rope_append(self.qs[:, :n], k[:, :n], v[:, :n], kc, vc, self.zero)
                r.gqa_attn_prefill(self.qs[:, :n], kc, vc, self.zero, out=self.o[:, :n])

    def time(self):
        # Each variant is thousands of small launches; replaying it from a HIP
        # graph times the GPU work instead of the host's launch loop.  One
        # replay's last decode output is checked against the eager run.
        res, ok = {}, True
        for name, fn in (("cached", self.cached), ("cached_two_launch", self.cached_two_launch),
                         ("uncached", self.uncached)):
            fn()
            torch.cuda.synchronize()
            ref = self.o1.clone() if name != "uncached" else self.o.clone()
            if name == "cached":
                fused_out = ref
            elif name == "cached_two_launch":
                ok = ok and torch.equal(ref, fused_out)  # one-launch and two-launch steps agree bit for bit
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn()
            graph.replay()
            torch.cuda.synchronize()
            out = self.o1 if name != "uncached" else self.o
            ok = ok and torch.equal(out, ref)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) / 3
            del graph
        return {"cached_ms": round(res["cached"], 3), "uncached_ms": round(res["uncached"], 3),
                "speedup": round(res["uncached"] / res["cached"], 2), "launch": "HIP graph replay",
                "cached_two_launch_ms": round(res["cached_two_launch"], 3),
                "cached_step": "one gqa_attn_decode_rope_append per layer and token (two-launch form: "
                               "rope_append + gqa_attn_decode, timed for comparison)",
                "graph_matches_eager": bool(ok),
                "workload": "12 layers, 12q/4kv, D64, bf16: 512-token prompt then 100 new tokens; uncached "
                            "recomputes RoPE, append and prefill over the whole prefix for every new token",
                "pages": "278 s -> 28 s (9.9x) for the whole model, 100 tokens after a 512-token prompt, "
                         "hardware not stated"}


def time_backward(rgc, synth, iters):
    """Attention backward (dq, dk, dv) on the 3.8B-shaped batch (B 8 x 2048,
    24 q / 8 KV, D 128), from the forward's output and lse."""
    w = synth.WORKLOADS["prefill3p8b"]
    g = synth.generator(w.seed + 100)
    q, k, v = (t.cuda() for t in synth.qkv(w.B, w.S, w.Hq, w.Hkv, w.D, g, w.dtype))
    d_o = synth.normal((w.B, w.S, w.Hq, w.D), g, w.dtype).cuda()
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device="cuda")
    o = rgc.gqa_attn_prefill(q, k.transpose(1, 2), v.transpose(1, 2), lse=lse)
    ws = rgc.backward_workspace(w.B, w.S, w.Hq)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    run = lambda: rgc.gqa_attn_backward(q, k, v, o, d_o, lse, workspace=ws, dq=dq, dk=dk, dv=dv)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        run()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / iters * 1e3
    flops = 10.0 * w.D * w.B * w.Hq * w.S * (w.S + 1) / 2  # five products per unmasked pair x 2D
    tf = flops / (us * 1e-6) / 1e12
    return {"bound": "mfma", "kernel": "gqa_attn_backward (dQ with Dlt, then dK/dV)", "achieved": round(tf, 2),
            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "algorithmic_flops_per_launch": flops, "avg_launch_us": round(us, 3),
            "workload": "B8 x 2048, 24q/8kv, D128, bf16; FLOPs count S, dP, dV, dK, dQ (2D each) per unmasked pair"}


def time_prologues(pre, iters):
    """The fused prologue on the 3.8B-shaped prefill batch, plain and with QK
    normalisation (HBM-bound: q, k, v read once; q and the cache rows written
    once)."""
    w = pre.w
    byts = 2.0 * 2 * w.B * w.S * (w.Hq + 2 * w.Hkv) * w.D  # bf16 read + write
    out = {}
    for name, fn in (("rope_append", lambda: pre.rgc.rope_append(pre.q, pre.k, pre.v, pre.kc, pre.vc, pre.pos0)),
                     ("norm_rope_append", lambda: pre.rgc.norm_rope_append(pre.q, pre.k, pre.v, pre.kc, pre.vc,
                                                                          pre.pos0, eps=1e-6))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / iters * 1e3
        out[name] = {"avg_launch_us": round(us, 3), "achieved": round(byts / (us * 1e-6) / 1e9, 1), "unit": "GB/s",
                     "frac": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    out["bound"] = "hbm"
    out["algorithmic_bytes_per_launch"] = byts
    out["workload"] = "B8 x 2048 tokens, 24 q / 8 kv heads, D128, bf16 (q rotated in place; k, v into the cache)"
    return out


def cpu_baseline(dec, seconds):
    """Time the fp64 oracle's decode on the host: passes over the workload's
    decode calls (lengths growing by one per call, as on the GPU) until about
    ``seconds`` of CPU time have been spent."""
    import oracle
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", threads))
    w = dec.w
    q = dec.q.cpu()
    done_bytes, t_total, calls = 0.0, 0.0, 0
    while calls == 0 or t_total < seconds:
        t = calls % w.steps
        lens = dec.lens0_cpu + (t + 1)
        t0 = time.perf_counter()
        oracle.attn_decode(q[t][:, 0], dec.kc_cpu, dec.vc_cpu, lens, nthreads=threads)
        t_total += time.perf_counter() - t0
        done_bytes += dec.bytes_per_call[t]
        calls += 1
    return {"value": done_bytes / t_total / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{calls} decode calls ({calls / w.steps:.1f} passes over the {w.steps} steps) of the "
                      f"ragged-decode workload (64 sequences, all heads), fp64, {t_total:.1f} s"}


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import rope_gqa_causal_amd as rgc
    from rope_gqa_causal_amd import synth

    print("[bench] setting up inputs", file=sys.stderr, flush=True)
    pre = Prefill(rgc, synth)
    dec = Decode(rgc, synth)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        pre.run(False)
        dec.run(fused=True)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    phase = []
    torch.cuda.synchronize()
    t_start.record()
    rgc.timing_report()  # clear
    for i in range(args.steps):
        a = torch.cuda.Event(enable_timing=True)
        m = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        a.record()
        pre.run(True)
        m.record()
        # Events between the decode kernels break their back-to-back issue
        # (a few us per call), so only the last timed step carries them: the
        # library brackets each kernel it launches there, and the decode
        # roofline averages that step's 32 launches.
        last = i == args.steps - 1
        if last:
            rgc.timing_enable(True)
        dec.run(fused=True)
        if last:
            rgc.timing_enable(False)
        z.record()
        phase.append((a, m, z))
    t_end.record()
    torch.cuda.synchronize()
    ktimes = rgc.timing_report()
    print(f"[bench] timed {args.steps} steps", file=sys.stderr, flush=True)

    total_ms = t_start.elapsed_time(t_end)
    pre_ms = sum(a.elapsed_time(m) for a, m, _ in phase)
    dec_ms = sum(m.elapsed_time(z) for _, m, z in phase)
    dec_bytes = sum(dec.bytes_per_call) * args.steps
    value = dec_bytes / (dec_ms * 1e-3) / 1e9
    prefill_tflops = pre.flops * args.steps / (pre_ms * 1e-3) / 1e12

    # Per-launch kernel durations: the prefill from HIP events around each
    # call (one kernel per call), the decode kernels from the library's own
    # per-kernel events in the last timed step.
    pk_ms = [e0.elapsed_time(e1) for e0, e1 in pre.events]
    pk_avg = sum(pk_ms) / len(pk_ms)
    n_split, split_us = ktimes["decode_split_kernel"]
    n_comb, comb_us = ktimes.get("decode_combine_kernel", (n_split, 0.0))
    if n_split != dec.w.steps or n_comb != dec.w.steps:
        raise SystemExit(f"expected {dec.w.steps} decode launches per kernel, got {ktimes}")
    dk_avg = split_us / n_split * 1e-3               # ms
    op_avg = dk_avg + comb_us / n_comb * 1e-3        # ms, kernel time of split + merge
    dk_bytes_avg = sum(dec.bytes_per_call) / len(dec.bytes_per_call)
    dec_achieved = dk_bytes_avg / (dk_avg * 1e-3) / 1e9
    op_achieved = dk_bytes_avg / (op_avg * 1e-3) / 1e9
    pre_achieved = pre.flops / (pk_avg * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "prefill 3.8B-shaped (B8 x 2048, 24q/8kv, D128) + ragged decode "
                        "(64 seqs, L~U{256..2048}, 24q/8kv, D128, 32 steps); bf16, fp32 accumulate",
            "global_batch": dec.w.B,
            "seq_len": pre.w.S,
            "parallelism": "single GPU",
        },
        "prefill": {
            "tflops": round(prefill_tflops, 2),
            "phase_ms_per_step": round(pre_ms / args.steps, 4),
            "note": "fused RoPE q,k + append, then causal prefill; FLOPs count unmasked pairs x 4D",
        },
        "decode_phase_ms_per_step": round(dec_ms / args.steps, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_split_kernel with the token's RoPE and append inside (the decode's dominant "
                      "kernel: streams the cache)",
            "achieved": round(dec_achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_achieved / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic("decode", "decode.hip", dk_bytes_avg),
            "algorithmic_bytes_per_launch": round(dk_bytes_avg),
            "avg_launch_us": round(dk_avg * 1e3, 3),
            "op": {
                "kernels": "decode_split_kernel + decode_combine_kernel (gqa_attn_decode_rope_append)",
                "avg_kernel_us": round(op_avg * 1e3, 3),
                "achieved": round(op_achieved, 2),
                "frac": round(op_achieved / HBM_PEAK_GBS, 4),
                "traffic": stored_traffic("decode_op", "decode.hip", dk_bytes_avg),
            },
        },
        "roofline_prefill": {
            "bound": "mfma",
            "kernel": "gqa_attn_prefill",
            "achieved": round(pre_achieved, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre_achieved / BF16_PEAK_TFLOPS, 4),
            "traffic": stored_traffic("prefill", "prefill.hip", None),
            "algorithmic_flops_per_launch": pre.flops,
            "avg_launch_us": round(pk_avg * 1e3, 3),
        },
    }
    if not args.no_extras:
        result["diff_attn"] = Diff(rgc, synth).time(max(args.steps, 5))
        result["prologue"] = time_prologues(pre, max(args.steps, 5))
        result["varlen_prefill"] = Varlen(rgc, synth).time(max(args.steps, 5))
        result["backward"] = time_backward(rgc, synth, max(args.steps, 3))
        result["generation_125m"] = Generation(rgc, synth).time()
        print("[bench] timed the variant lines", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(dec, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
