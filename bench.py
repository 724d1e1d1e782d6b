"""Benchmark of the causal GQA + RoPE path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  prefill phase  (24 query / 8 KV heads, head dim 128, batch 8 x 2048 tokens):
                 fused RoPE on q and k + cache append, causal GQA prefill;
  decode phase   (64 sequences, cache lengths uniform on {256..2048}, same
                 heads): 32 generation steps, each one launch of the cached
                 GQA decode with the new token's RoPE (q and k) and the
                 append of its k and v inside, plus the chunk merge (the
                 lengths of every step are precomputed once, as a serving
                 loop knows them).  Successive decode calls rotate over
                 several independent cache sets (3 by default, 545 MB each),
                 so no call finds the cache rows of the previous one in the
                 256 MB last-level (MALL) cache: the rate is HBM bandwidth.
`value` is the decode phase's KV-read rate (cache bytes every decode call
must read / decode-phase time, GB/s); the prefill phase's attention rate is
reported beside it (TFLOP/s over unmasked query-key pairs).  `roofline` is
the whole decode op (split kernel + merge kernel) per call, from HIP events
recorded around each decode call of the last timed step on the stream the
library launches on; the split kernel alone is reported beside it, timed by
the instrumented build of the library in an extra, untimed decode phase.
`roofline_prefill` is the prefill kernel against the bf16 MFMA peak.
The differential-attention variant (`diff_attn`), the packed-document prefill
(`varlen_prefill`), the fused prologue with and without QK normalisation
(`prologue`), the attention backward (`backward`), the 125M-shaped cached
versus recomputed generation (`generation_125m`), a decode length sweep with
a linear fit of time against cache length (`decode_length_sweep`) and the
measured ceilings of this GPU (`ceilings`: a streaming read, a matrix-core
loop) are timed apart on their own workloads.  The fp64 CPU oracle is timed
on bounded samples of the decode and prefill workloads (`cpu_baseline`).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import hashlib
import json
import os
import re
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
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="target wall time of each CPU-oracle sample (decode, prefill)")
    ap.add_argument("--cache-sets", type=int, default=3,
                    help="independent decode cache sets rotated call by call (1 = no rotation)")
    ap.add_argument("--phase", choices=("all", "prefill", "decode"), default="all",
                    help="time only one phase (for counter runs); the JSON line then carries that phase only")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the variant lines (diff, varlen, prologue, backward, generation, sweep, ceilings)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration runs)")
    ap.add_argument("--with-ceilings", action="store_true",
                    help="run the ceiling kernels even with --no-extras (counter calibration runs)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="RUN_DIR",
                    help="turn rocprofv3 --pmc runs of `--phase prefill --with-ceilings` into "
                         "profiles/counters_prefill_mfma.json and exit")
    ap.add_argument("--variants-only", action="store_true",
                    help="time only the matrix-core variant lines (differential prefill and decode, "
                         "packed-document prefill, backward) and exit: the counter runs of "
                         "profiles/counters_variants.md")
    ap.add_argument("--summarize-variant-counters", nargs="+", metavar="RUN_DIR",
                    help="turn rocprofv3 --pmc runs of `--variants-only` into profiles/counters_variants.json")
    ap.add_argument("--summarize-trace", metavar="RUN_DIR",
                    help="print the per-kernel table of a rocprofv3 --kernel-trace run and exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, WRITE_SIZE; both "
                         "with --copy-calibration) into profiles/counters_*.json and exit")
    return ap.parse_args()


def _code_text(name, seen):
    """The code of csrc/<name> and of the local headers it includes, with
    comments and whitespace removed (so that a comment edit keeps the stored
    counters, and a change to a header the kernel includes does not)."""
    if name in seen:
        return ""
    seen.add(name)
    path = os.path.join(ROOT, "rope_gqa_causal_amd", "csrc", name)
    if not os.path.exists(path):
        return ""
    with open(path) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    parts = [re.sub(r"\s+", " ", src).strip()]
    for inc in re.findall(r'#include\s+"([^"]+)"', src):
        parts.append(_code_text(inc, seen))
    return "\n".join(parts)


def kernel_sha(name):
    """Hash of a kernel source's code (see _code_text), recorded with the
    counters taken on it."""
    return hashlib.sha256(_code_text(name, set()).encode()).hexdigest()[:16]


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


def stored_mfma_util():
    """Matrix-core utilisation of the prefill kernel from committed counter
    runs, if the kernel is unchanged since they were taken."""
    path = os.path.join(PROFILES, "counters_prefill_mfma.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    if rec.get("kernel_sha") != kernel_sha("prefill.hip"):
        return None
    return rec.get("derived")


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


def summarize_trace(run_dir, top=40):
    """Per kernel and launch shape (workgroups x threads, LDS bytes, VGPRs):
    calls and average / min / max duration in us, from the database of a
    rocprofv3 --kernel-trace run, as a markdown table ordered by total time."""
    import glob
    import sqlite3
    groups = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*.db"), recursive=True):
        rows = sqlite3.connect(path).execute(
            "select name, grid_x, grid_y, grid_z, workgroup_x, workgroup_y, workgroup_z, lds_size, vgpr_count, "
            "duration from kernels").fetchall()
        for name, gx, gy, gz, wx, wy, wz, lds, vgpr, dur in rows:
            short = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            short = short.split("<")[0].split("::")[-1]
            wgs = (gx // max(wx, 1)) * (gy // max(wy, 1)) * (gz // max(wz, 1))
            key = (short, wgs, wx * wy * wz, lds, vgpr)
            groups.setdefault(key, []).append(dur / 1e3)
    print("| kernel | workgroups x threads | LDS bytes | VGPRs (trace field) | calls | avg us | min us | max us |")
    print("|---|---|---|---|---|---|---|---|")
    for (k, wg, wx, lds, vgpr), d in sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:top]:
        print(f"| {k} | {wg} x {wx} | {lds} | {vgpr} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | {max(d):.1f} |")


VARIANT_KERNELS = ("diff_kernel", "diff_decode_kernel", "diff_combine_kernel", "prefill_kernel", "dq_kernel",
                   "dkdv_kernel")


def summarize_variant_counters(run_dirs):
    """Per-dispatch averages of every counter found in the rocpd databases of
    `--variants-only` runs, per kernel at its largest grid (the timed launch
    shape), with the derived ratios of summarize_counters."""
    import glob
    import sqlite3
    per = {}
    for d in run_dirs:
        for path in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
            rows = sqlite3.connect(path).execute(
                "select dispatch_id, kernel_name, grid_size, counter_name, value from counters_collection").fetchall()
            for did, kname, grid, cname, val in rows:
                short = kname.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
                short = short.split("<")[0].split("::")[-1]
                if short not in VARIANT_KERNELS:
                    continue
                dd = per.setdefault((short, grid), {}).setdefault(cname, {})
                key = (path, did)
                if cname.startswith("GRBM_"):
                    dd[key] = max(dd.get(key, 0.0), val)
                else:
                    dd[key] = dd.get(key, 0.0) + val
    out = {}
    for name in VARIANT_KERNELS:
        grids = [g for (k, g) in per if k == name]
        if not grids:
            continue
        cs = per[(name, max(grids))]
        avg = {c: sum(v.values()) / len(v) for c, v in cs.items()}
        mfma = avg.get("SQ_INSTS_MFMA", 0.0)
        rec = {"grid_threads": max(grids), "counters_per_dispatch": {k: round(v, 1) for k, v in sorted(avg.items())}}
        der = {}
        if "MfmaUtil" in avg:
            der["mfma_util"] = round(avg["MfmaUtil"] / 100.0, 4)
        if "VALUBusy" in avg:
            der["valu_busy"] = round(avg["VALUBusy"] / 100.0, 4)
        if mfma and "SQ_INSTS_VALU" in avg:
            der["other_valu_per_mfma"] = round((avg["SQ_INSTS_VALU"] - mfma) / mfma, 3)
        if avg.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
            der["valu_coexec_per_mfma_busy"] = round(avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / avg["SQ_VALU_MFMA_BUSY_CYCLES"], 4)
        if avg.get("SQ_LDS_IDX_ACTIVE"):
            der["lds_conflict_per_active"] = round(avg.get("SQ_LDS_BANK_CONFLICT", 0.0) / avg["SQ_LDS_IDX_ACTIVE"], 4)
        rec["derived"] = der
        src = {"diff_kernel": "diff.hip", "diff_decode_kernel": "diff_decode.hip", "diff_combine_kernel": "diff_decode.hip",
               "prefill_kernel": "prefill.hip", "dq_kernel": "backward_dq.hip", "dkdv_kernel": "backward.hip"}[name]
        rec["kernel_sha"] = kernel_sha(src)
        out[name] = rec
    out["runs"] = list(run_dirs)
    with open(os.path.join(PROFILES, "counters_variants.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def summarize_counters(run_dirs):
    """Per-dispatch averages of every counter found in the rocpd databases of
    the given runs, for the prefill kernel and for the matrix-core loop of
    ceilings/ceilings.hip (the calibration: a kernel that does nothing but
    back-to-back MFMA), and the ratios derived from them:
      mfma_util       the profiler's MfmaUtil (MFMA-busy cycles over active
                      cycles of all SIMDs), beside the calibration loop's;
      executed_flops  SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (flops per MOP);
      other_valu_per_mfma  (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA;
      valu_coexec_per_mfma_busy  cycles a plain VALU op issued while the
                      matrix core was busy, over the matrix-core busy cycles;
      lds_conflict    SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE."""
    per = {}
    for d in run_dirs:
        import glob
        import sqlite3
        for path in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
            rows = sqlite3.connect(path).execute(
                "select dispatch_id, kernel_name, counter_name, value from counters_collection").fetchall()
            for did, kname, cname, val in rows:
                short = kname.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
                short = short.split("<")[0].split("::")[-1]
                if short not in ("prefill_kernel", "mfma_bf16_kernel"):
                    continue
                key = (path, did)
                d = per.setdefault(short, {}).setdefault(cname, {})
                # GRBM counters repeat one GPU-wide count per XCD: take the
                # largest (as the profiler's own derived formulas do); SQ
                # counters are summed over their instances.
                if cname.startswith("GRBM_"):
                    d[key] = max(d.get(key, 0.0), val)
                else:
                    d[key] = d.get(key, 0.0) + val
    avg = {k: {c: sum(v.values()) / len(v) for c, v in cs.items()} for k, cs in per.items()}
    # The calibration loop runs in several sizes (a warm-up launch among
    # them): keep the dispatches of the largest, in every pass.
    cal_d = per.get("mfma_bf16_kernel", {})
    if cal_d:
        keep = {}
        for cname, d in cal_d.items():
            top = max(d.values())
            keep[cname] = [v for v in d.values() if v >= 0.9 * top]
        avg["mfma_bf16_kernel"] = {c: sum(v) / len(v) for c, v in keep.items()}
    pre = avg.get("prefill_kernel", {})
    cal = avg.get("mfma_bf16_kernel", {})

    derived = {}
    if "MfmaUtil" in pre:
        derived["mfma_util"] = pre["MfmaUtil"] / 100.0  # the profiler's formula
    if "MfmaUtil" in cal:
        derived["mfma_util_calibration_loop"] = cal["MfmaUtil"] / 100.0
    if "VALUBusy" in pre:
        derived["valu_busy"] = pre["VALUBusy"] / 100.0
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in pre:
        derived["executed_mfma_flops"] = pre["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    if pre.get("SQ_INSTS_MFMA") and "SQ_INSTS_VALU" in pre:
        # SQ_INSTS_VALU counts the MFMAs too
        derived["other_valu_per_mfma"] = (pre["SQ_INSTS_VALU"] - pre["SQ_INSTS_MFMA"]) / pre["SQ_INSTS_MFMA"]
    if pre.get("SQ_INSTS_MFMA") and "SQ_VALU_MFMA_BUSY_CYCLES" in pre:
        derived["mfma_busy_cycles_per_mfma"] = pre["SQ_VALU_MFMA_BUSY_CYCLES"] / pre["SQ_INSTS_MFMA"]
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in pre and pre.get("SQ_VALU_MFMA_BUSY_CYCLES"):
        derived["valu_coexec_per_mfma_busy"] = pre["SQ_VALU_MFMA_COEXEC_CYCLES"] / pre["SQ_VALU_MFMA_BUSY_CYCLES"]
    if pre.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in pre:
        derived["lds_conflict_per_active"] = pre["SQ_LDS_BANK_CONFLICT"] / pre["SQ_LDS_IDX_ACTIVE"]
    derived = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in derived.items()}
    rec = {"kernel": "prefill_kernel", "kernel_sha": kernel_sha("prefill.hip"),
           "counters_per_dispatch": {k: round(v, 1) for k, v in sorted(pre.items())},
           "calibration_loop_counters_per_dispatch": {k: round(v, 1) for k, v in sorted(cal.items())},
           "derived": derived,
           "runs": [os.path.relpath(d, ROOT) for d in run_dirs]}
    with open(os.path.join(PROFILES, "counters_prefill_mfma.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


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
    def __init__(self, rgc, synth, cache_sets=3):
        w = synth.WORKLOADS["ragged_decode"]
        self.w = w
        g = synth.generator(w.seed)
        self.lens0_cpu = synth.lengths(w.B, w.len_lo, w.len_hi, g)
        self.S_max = w.len_hi + w.steps
        kc, vc = synth.filled_cache(w.B, w.Hkv, self.S_max, w.D, g, w.dtype)
        self.kc_cpu, self.vc_cpu = kc, vc
        # Independent cache sets at their own addresses, rotated call by call:
        # a set is read again only after (sets - 1) other calls have streamed
        # about 289 MB each through the 256 MB MALL.
        first = (kc.cuda(), vc.cuda())
        self.sets = [first] + [(first[0].clone(), first[1].clone()) for _ in range(max(cache_sets, 1) - 1)]
        self.calls = 0
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

    def run(self, fused=True, events=None):
        """The 32 decode calls of one step; with ``events`` (a list), each call
        is bracketed by HIP events on the current stream (the library's)."""
        r, w = self.rgc, self.w
        for t in range(w.steps):
            kc, vc = self.sets[self.calls % len(self.sets)]
            self.calls += 1
            if events is not None:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
            if not fused:
                # the two-launch form: RoPE (q, k at position lens0 + t) and
                # cache append, then the decode of the rotated q
                r.rope_append(self.q[t], self.k[t], self.v[t], kc, vc, self.slots[t])
                r.gqa_attn_decode(self.q[t][:, 0], kc, vc, self.lens[t], self.S_max, self.ws, out=self.o)
            else:
                # one launch (plus the chunk merge): RoPE of q and k at
                # position lens0 + t, append of k and v, attention
                r.gqa_attn_decode_rope_append(self.q[t][:, 0], self.k[t][:, 0], self.v[t][:, 0], kc, vc,
                                              self.lens[t], self.S_max, self.ws, out=self.o)
            if events is not None:
                e1.record()
                events.append((e0, e1))


def decode_length_sweep(rgc, iters=20, cache_sets=3, lengths=(256, 512, 1024, 2048, 4096, 8192)):
    """Decode time against cache length at a fixed batch (64 sequences, all
    of length L, 24 q / 8 KV heads, D 128, bf16), over rotated cache sets.
    Cached decode reads each cached row once per step, so its time should be
    linear in L (the O(N)-per-step cost of cached generation on page
    "750美元从零训练3个LLM：一位开发者的实战复盘", section V3); a least-squares
    line t = a + b L and its r^2 are reported."""
    B, Hq, Hkv, D = 64, 24, 8, 128
    S_max = max(lengths)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(404)
    sets = []
    for _ in range(cache_sets):
        pair = []
        for _ in range(2):
            pair.append(torch.randn((B, Hkv, S_max, D), generator=gen, device="cuda").to(torch.bfloat16))
        sets.append(tuple(pair))
    q = torch.randn((B, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    ws = rgc.decode_workspace(B, Hq, Hkv, D, S_max)
    o = torch.empty_like(q)
    rows = []
    for L in lengths:
        lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
        run = lambda i: rgc.gqa_attn_decode(q, sets[i % cache_sets][0], sets[i % cache_sets][1], lens, L, ws, out=o)
        for i in range(10):
            run(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            run(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / iters * 1e3
        byts = float(B) * L * Hkv * D * 2 * 2
        rows.append({"L": L, "us_per_call": round(us, 3), "GB/s": round(byts / (us * 1e-6) / 1e9, 1)})
    del sets
    xs = [float(r["L"]) for r in rows]
    ys = [r["us_per_call"] for r in rows]
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    sxy = sum((x - mx) * (y - my) for x, y in zip(xs, ys))
    slope = sxy / sxx
    icept = my - slope * mx
    ss_res = sum((y - (icept + slope * x)) ** 2 for x, y in zip(xs, ys))
    ss_tot = sum((y - my) ** 2 for y in ys)
    return {"points": rows, "fit_us": {"intercept": round(icept, 3), "us_per_1k_tokens": round(slope * 1e3, 4),
                                        "r2": round(1.0 - ss_res / ss_tot, 6)},
            "cache_sets": cache_sets,
            "workload": "64 sequences all of cache length L, 24q/8kv, D128, bf16, gqa_attn_decode (max_len = L)",
            "pages": "cached generation costs O(N) per new token where recomputing costs O(N^2)"}


def ceilings(iters=10):
    """What this GPU delivers to a hand-written kernel: a streaming read of
    2 GiB with 16-byte loads, back-to-back bf16 MFMA (32x32x16) on four
    accumulators per wave, and the same MFMA loop with every operand read
    from LDS just before its use (ceilings/ceilings.hip)."""
    import ctypes
    path = os.path.join(ROOT, "ceilings", "libceil.so")
    if not os.path.exists(path):
        return {"error": "ceilings/libceil.so is not built"}
    lib = ctypes.CDLL(path)
    lib.ceil_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p]
    lib.ceil_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.ceil_lds_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    best_read = 0.0
    read_rows = []
    modes = {0: "grid-stride, 4 loads in flight", 1: "contiguous slices, 8 in flight",
             2: "contiguous slices, 16 in flight", 3: "contiguous slices, 8 in flight, nontemporal"}
    for mode, wgs in ((0, 2048), (1, 1024), (1, 2048), (1, 4096), (2, 1024), (2, 2048), (3, 2048)):
        out = torch.empty(wgs * 256, dtype=torch.int32, device="cuda")
        args = (ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()), wgs, mode, stream)
        if lib.ceil_stream_read(*args):
            return {"error": "ceil_stream_read refused"}
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            lib.ceil_stream_read(*args)
        e1.record()
        torch.cuda.synchronize()
        gbs = nbytes * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9
        read_rows.append({"form": modes[mode], "workgroups": wgs, "GB/s": round(gbs, 1)})
        best_read = max(best_read, gbs)
    del buf
    mf_rows, best_mf = [], 0.0
    for wgs, loop in ((512, 2048), (1024, 2048)):
        out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
        lib.ceil_mfma_bf16(ctypes.c_void_p(out.data_ptr()), wgs, 64, stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            lib.ceil_mfma_bf16(ctypes.c_void_p(out.data_ptr()), wgs, loop, stream)
        e1.record()
        torch.cuda.synchronize()
        flops = float(wgs) * 4 * loop * 4 * 32768 * iters
        tf = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
        mf_rows.append({"workgroups": wgs, "waves_per_simd": wgs * 4 // 1024, "TFLOP/s": round(tf, 1)})
        best_mf = max(best_mf, tf)
    # LDS-fed matrix loop: 8 waves per workgroup (two per SIMD), each MFMA's
    # B operand (16 bytes per lane, 1 KiB per wave) read from LDS; mode 0 is
    # the same reads without the MFMAs (LDS read bandwidth).
    lds_rows = {}
    for mode in (0, 1):
        wgs, loop = 512, 4096
        out = torch.empty(wgs * 512, dtype=torch.float32, device="cuda")
        if lib.ceil_lds_mfma(ctypes.c_void_p(out.data_ptr()), wgs, 64, mode, stream):
            return {"error": "ceil_lds_mfma refused"}
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            lib.ceil_lds_mfma(ctypes.c_void_p(out.data_ptr()), wgs, loop, mode, stream)
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3
        lds_bytes = float(wgs) * 8 * loop * 4 * 1024 * iters
        if mode:
            lds_rows["mfma_TFLOPs"] = round(float(wgs) * 8 * loop * 4 * 32768 * iters / sec / 1e12, 1)
            lds_rows["lds_TBs_with_mfma"] = round(lds_bytes / sec / 1e12, 2)
        else:
            lds_rows["lds_TBs_reads_only"] = round(lds_bytes / sec / 1e12, 2)
    return {"hbm_read_GBs": round(best_read, 1), "hbm_read_frac_of_spec": round(best_read / HBM_PEAK_GBS, 4),
            "hbm_read_runs": read_rows,
            "mfma_bf16_TFLOPs": round(best_mf, 1), "mfma_bf16_frac_of_spec": round(best_mf / BF16_PEAK_TFLOPS, 4),
            "mfma_runs": mf_rows,
            "lds_fed_mfma": dict(lds_rows, workgroups=512, waves_per_workgroup=8,
                                 form="every MFMA's B operand read from LDS (16 B per lane) just before it"),
            "kernels": "ceilings/ceilings.hip: 16-byte reads of a 2 GiB buffer (8x the MALL) in several forms, "
                       "the best reported; v_mfma_f32_32x32x16_bf16 back to back on 4 accumulators per wave, no "
                       "memory traffic"}


def warm_up(run, min_ms=25.0, min_calls=10):
    """Untimed calls before a variant line's timed ones: at least min_calls
    and at least min_ms of GPU work, about what the step's own ten warm-up
    steps give (the shader clock rises over the first tens of milliseconds
    of load, so a line timed after a few calls of a short kernel reads its
    ramp rather than its settled rate).  run(i) takes the call index."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while i < min_calls or (time.perf_counter() - t0) * 1e3 < min_ms:
        run(i)
        i += 1
        if i % 5 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


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
        warm_up(lambda i: self.run())
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


class DiffDecode:
    """Cached decode of differential attention: 64 sequences with cache
    lengths uniform on {256..2048}, the differential workload's heads (16 q /
    8 KV, two maps of head dim 64, value dim 64, lambda 0.8), bf16; calls
    rotate over independent cache sets (k1, k2, v: 3 x 201 MB each) like the
    main decode.  HBM-bound: 3 x 8 x 64 x 2 B of cache per token."""

    def __init__(self, rgc, synth, cache_sets=3):
        w = synth.WORKLOADS["diff"]
        self.w, self.rgc = w, rgc
        g = synth.generator(w.seed + 1000)
        self.B, self.S_max = 64, 2048
        self.lens = synth.lengths(self.B, 256, 2048, g).cuda()
        gen = torch.Generator(device="cuda")
        gen.manual_seed(w.seed + 1000)
        self.sets = [tuple(torch.randn((self.B, w.Hkv, self.S_max, w.D), generator=gen, device="cuda")
                           .to(torch.bfloat16) for _ in range(3)) for _ in range(max(cache_sets, 1))]
        self.q1 = torch.randn((self.B, w.Hq, w.D), generator=gen, device="cuda").to(torch.bfloat16)
        self.q2 = torch.randn((self.B, w.Hq, w.D), generator=gen, device="cuda").to(torch.bfloat16)
        self.o = torch.empty_like(self.q1)
        self.ws = rgc.diff_decode_workspace(self.B, w.Hq, w.Hkv, w.D, self.S_max)
        self.bytes = float(self.lens.sum().item()) * w.Hkv * w.D * 3 * 2

    def time(self, iters):
        run = lambda i: self.rgc.diff_attn_decode(self.q1, self.q2, *self.sets[i % len(self.sets)], self.lens,
                                                  self.w.lam, self.S_max, self.ws, out=self.o)
        warm_up(run)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            run(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / iters * 1e3
        gbs = self.bytes / (us * 1e-6) / 1e9
        return {"bound": "hbm", "kernel": "diff_attn_decode (split + merge)", "achieved": round(gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                "algorithmic_bytes_per_launch": self.bytes, "avg_launch_us": round(us, 3),
                "cache_sets": len(self.sets),
                "workload": "64 sequences, cache lengths U{256..2048}, 16q/8kv, k1, k2, v of D64, lambda 0.8, bf16"}


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
        warm_up(lambda i: run())
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
    warm_up(lambda i: run(), min_calls=5)
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
        warm_up(lambda i: fn())
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


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(pre, dec, seconds):
    """Time the fp64 oracle (as it stands) on the host cores, on bounded
    samples of the two workloads of the step:
      decode  passes over the ragged-decode calls (lengths growing by one per
              call, as on the GPU) until about ``seconds`` have been spent;
      prefill row blocks of 16 query rows at random slots of the 3.8B-shaped
              batch (all 8 sequences and 24 heads), until about ``seconds``;
    plus one-thread figures for the tiny fp32 workload (its whole prefill and
    decode chain) and for sampled rows of the differential workload."""
    import oracle
    from rope_gqa_causal_amd import synth
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", threads))
    # decode
    w = dec.w
    q = dec.q.cpu()
    done_bytes, t_dec, calls = 0.0, 0.0, 0
    while calls == 0 or t_dec < seconds:
        t = calls % w.steps
        lens = dec.lens0_cpu + (t + 1)
        t0 = time.perf_counter()
        oracle.attn_decode(q[t][:, 0], dec.kc_cpu, dec.vc_cpu, lens, nthreads=threads)
        t_dec += time.perf_counter() - t0
        done_bytes += dec.bytes_per_call[t]
        calls += 1
    dec_gbs = done_bytes / t_dec / 1e9
    # prefill: row blocks of the (rotated) q over the cache the bench filled
    pw = pre.w
    pq, pk, pv = pre.q.cpu(), pre.kc.cpu(), pre.vc.cpu()
    g = torch.Generator().manual_seed(303)
    flops, t_pre, blocks = 0.0, 0.0, 0
    while blocks == 0 or t_pre < seconds:
        s0 = int(torch.randint(0, pw.S - 16 + 1, (1,), generator=g))
        qs = torch.full((pw.B,), s0, dtype=torch.int32)
        t0 = time.perf_counter()
        oracle.attn(pq[:, s0:s0 + 16], pk, pv, qs, nthreads=threads)
        t_pre += time.perf_counter() - t0
        flops += 4.0 * pw.D * pw.B * pw.Hq * sum(s0 + i + 1 for i in range(16))
        blocks += 1
    pre_gfs = flops / t_pre / 1e9
    # one thread: the tiny fp32 workload's whole chain
    tw = synth.WORKLOADS["tiny"]
    T = tw.S + tw.steps
    tq, tk, tv = synth.qkv(tw.B, T, tw.Hq, tw.Hkv, tw.D, synth.generator(tw.seed), tw.dtype)
    tiny_flops = 4.0 * tw.D * tw.Hq * (sum(i + 1 for i in range(tw.S)) + sum(tw.S + i + 1 for i in range(tw.steps)))
    n_tiny, t_tiny = 0, 0.0
    while n_tiny == 0 or t_tiny < 1.0:
        t0 = time.perf_counter()
        qo, ko = tq.clone(), tk.clone()
        oracle.rope_apply_(qo, None)
        oracle.rope_apply_(ko, None)
        kco = torch.zeros((tw.B, tw.Hkv, T, tw.D), dtype=tw.dtype)
        vco = torch.zeros_like(kco)
        oracle.kv_cache_append_(kco, vco, ko, tv, torch.zeros(tw.B, dtype=torch.int32))
        oracle.attn(qo[:, :tw.S], kco, vco, nthreads=1)
        for i in range(tw.steps):
            oracle.attn_decode(qo[:, tw.S + i], kco, vco, torch.full((tw.B,), tw.S + i + 1, dtype=torch.int32),
                               nthreads=1)
        t_tiny += time.perf_counter() - t0
        n_tiny += 1
    # one thread: sampled rows of the differential workload
    dw = synth.WORKLOADS["diff"]
    dg = synth.generator(dw.seed)
    q1 = synth.normal((dw.B, dw.S, dw.Hq, dw.D), dg)
    q2 = synth.normal((dw.B, dw.S, dw.Hq, dw.D), dg)
    k1, k2, dv = (synth.normal((dw.B, dw.Hkv, dw.S, dw.D), dg) for _ in range(3))
    dflops, t_diff, dblocks = 0.0, 0.0, 0
    while dblocks == 0 or t_diff < 2.0:
        s0 = int(torch.randint(0, dw.S - 4 + 1, (1,), generator=g))
        qs = torch.full((dw.B,), s0, dtype=torch.int32)
        t0 = time.perf_counter()
        oracle.diff_attn(q1[:, s0:s0 + 4], q2[:, s0:s0 + 4], k1, k2, dv, dw.lam, qs, nthreads=1)
        t_diff += time.perf_counter() - t0
        dflops += 2 * 4.0 * dw.D * dw.B * dw.Hq * sum(s0 + i + 1 for i in range(4))
        dblocks += 1
    return {"value": round(dec_gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"decode: {calls} calls ({calls / w.steps:.1f} passes over the {w.steps} steps) of the "
                      f"ragged-decode workload (64 sequences, all heads), fp64, {t_dec:.1f} s",
            "prefill": {"value": round(pre_gfs, 3), "unit": "GFLOP/s", "cores": threads,
                        "sample": f"{blocks} blocks of 16 query rows at random slots of the 8 x 2048, 24q/8kv, "
                                  f"D128 batch (all sequences and heads), fp64, {t_pre:.1f} s"},
            "one_thread": {
                "tiny": {"us_per_run": round(t_tiny / n_tiny * 1e6, 1),
                         "GFLOP/s": round(tiny_flops * n_tiny / t_tiny / 1e9, 4),
                         "sample": f"{n_tiny} runs of the tiny fp32 chain (RoPE, append, 16-row prefill, 8 decode "
                                   "steps; 4q/2kv, D32)"},
                "diff": {"GFLOP/s": round(dflops / t_diff / 1e9, 4),
                         "sample": f"{dblocks} blocks of 4 query rows at random slots of the differential workload "
                                   f"(B4 x 1024, 16q/8kv, two maps of D64), {t_diff:.1f} s"}},
            "note": "fp64 CPU oracle as it stands: a baseline, not a target"}


PAGES_CONTEXT = {
    "cached_generation": "278 s -> 28 s for 100 new tokens after a 512-token prompt, whole model, hardware "
                         "not stated (page '750美元从零训练3个LLM：一位开发者的实战复盘', section V3)",
    "training_throughput": "about 480,000 tokens/s in steady state on 8x B200 (DDP, bf16 with FP8 GEMMs), "
                           "whole-model training of the 24q/8kv 3.8B model at 1024 context (page "
                           "'训练3.8B LLM至0.384 CORE，成本998美元 – Hugo Vergnes', sections 结果 and 提高吞吐量)",
    "note": "context only: whole-model figures on other hardware, not comparable with these kernel rates",
}


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_variant_counters:
        summarize_variant_counters(args.summarize_variant_counters)
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

    if args.variants_only:
        res = {"diff_attn": Diff(rgc, synth).time(5),
               "diff_attn_decode": DiffDecode(rgc, synth, args.cache_sets).time(10),
               "varlen_prefill": Varlen(rgc, synth).time(5),
               "backward": time_backward(rgc, synth, 3)}
        print(json.dumps(res, ensure_ascii=False), flush=True)
        return
    do_pre = args.phase in ("all", "prefill")
    do_dec = args.phase in ("all", "decode")
    t_run = time.perf_counter()
    print("[bench] setting up inputs", file=sys.stderr, flush=True)
    pre = Prefill(rgc, synth) if do_pre else None
    dec = Decode(rgc, synth, args.cache_sets) if do_dec else None
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        if do_pre:
            pre.run(False)
        if do_dec:
            dec.run()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps) ({time.perf_counter() - t_run:.1f} s)", file=sys.stderr, flush=True)

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    phase = []
    call_events = []
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        a = torch.cuda.Event(enable_timing=True)
        m = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        a.record()
        if do_pre:
            pre.run(True)
        m.record()
        if do_dec:
            dec.run()
        z.record()
        phase.append((a, m, z))
    t_end.record()
    torch.cuda.synchronize()
    # Events between the decode calls break their back-to-back issue (a few
    # us per call): one more, untimed decode phase carries them.
    if do_dec:
        dec.run(events=call_events)
        torch.cuda.synchronize()
    print(f"[bench] timed {args.steps} steps ({time.perf_counter() - t_run:.1f} s)", file=sys.stderr, flush=True)

    total_ms = t_start.elapsed_time(t_end)
    result = {
        "metric": METRIC,
        "value": None,
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
            "global_batch": synth.WORKLOADS["ragged_decode"].B,
            "seq_len": synth.WORKLOADS["prefill3p8b"].S,
            "parallelism": "single GPU",
            "cache_sets": args.cache_sets if do_dec else None,
            "phase": args.phase,
        },
    }
    if do_dec:
        dec_ms = sum(m.elapsed_time(z) for _, m, z in phase)
        dec_bytes = sum(dec.bytes_per_call) * args.steps
        result["value"] = round(dec_bytes / (dec_ms * 1e-3) / 1e9, 2)
        result["decode_phase_ms_per_step"] = round(dec_ms / args.steps, 4)
        # The whole decode op per call (split + merge kernels, and the gap
        # between them): the decode phase of the timed steps over its calls
        # (issued back to back, as in a generation loop).  The average of
        # events around each call of one more phase is reported beside it.
        op_avg = dec_ms / args.steps / dec.w.steps
        op_ms = [e0.elapsed_time(e1) for e0, e1 in call_events]
        ev_avg = sum(op_ms) / len(op_ms)
        bytes_avg = sum(dec.bytes_per_call) / len(dec.bytes_per_call)
        op_achieved = bytes_avg / (op_avg * 1e-3) / 1e9
        # The split kernel alone: the instrumented build times each kernel
        # of one more (untimed) decode phase.
        # The first phase through the instrumented build loads its code
        # objects; it is run once and its record dropped.
        for _ in range(2):
            rgc.timing_report()  # clear
            with rgc.kernel_timing():
                dec.run()
            torch.cuda.synchronize()
        kt = rgc.timing_report()
        n_split, split_us = kt["decode_split_kernel"]
        n_comb, comb_us = kt.get("decode_combine_kernel", (n_split, 0.0))
        if n_split != dec.w.steps or n_comb != dec.w.steps:
            raise SystemExit(f"expected {dec.w.steps} decode launches per kernel, got {kt}")
        split_avg = split_us / n_split * 1e-3
        split_achieved = bytes_avg / (split_avg * 1e-3) / 1e9
        result["roofline"] = {
            "bound": "hbm",
            "kernel": "gqa_attn_decode_rope_append: decode_split_kernel (with the token's RoPE and append "
                      "inside) + decode_combine_kernel, per call",
            "achieved": round(op_achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(op_achieved / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic("decode_op", "decode.hip", bytes_avg),
            "algorithmic_bytes_per_launch": round(bytes_avg),
            "avg_launch_us": round(op_avg * 1e3, 3),
            "timing": "HIP events around the decode phase (32 calls back to back) of each timed step, on the "
                      "stream the library launches on, per call",
            "avg_launch_us_with_call_events": round(ev_avg * 1e3, 3),
            "achieved_with_call_events": round(bytes_avg / (ev_avg * 1e-3) / 1e9, 2),
            "cache_sets": args.cache_sets,
            "split_kernel": {
                "kernel": "decode_split_kernel (streams the cache; carries all the algorithmic bytes)",
                "avg_launch_us": round(split_avg * 1e3, 3),
                "achieved": round(split_achieved, 2),
                "frac": round(split_achieved / HBM_PEAK_GBS, 4),
                "merge_avg_us": round(comb_us / n_comb, 3),
                "traffic": stored_traffic("decode", "decode.hip", bytes_avg),
                "timing": "instrumented build (librgc_timed.so): HIP events around each kernel, one extra "
                          "untimed decode phase on the same rotated cache sets",
            },
        }
    if do_pre:
        pre_ms = sum(a.elapsed_time(m) for a, m, _ in phase)
        pk_ms = [e0.elapsed_time(e1) for e0, e1 in pre.events]
        pk_avg = sum(pk_ms) / len(pk_ms)
        pre_achieved = pre.flops / (pk_avg * 1e-3) / 1e12
        result["prefill"] = {
            "tflops": round(pre.flops * args.steps / (pre_ms * 1e-3) / 1e12, 2),
            "phase_ms_per_step": round(pre_ms / args.steps, 4),
            "note": "fused RoPE q,k + append, then causal prefill; FLOPs count unmasked pairs x 4D",
        }
        result["roofline_prefill"] = {
            "bound": "mfma",
            "kernel": "gqa_attn_prefill",
            "achieved": round(pre_achieved, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre_achieved / BF16_PEAK_TFLOPS, 4),
            "traffic": stored_traffic("prefill", "prefill.hip", None),
            "algorithmic_flops_per_launch": pre.flops,
            "avg_launch_us": round(pk_avg * 1e3, 3),
            "mfma_util": stored_mfma_util(),
        }
        if result["value"] is None:
            result["value"] = round(pre_achieved, 2)
            result["unit"] = "TFLOP/s"
    if not args.no_extras and args.phase == "all":
        result["diff_attn"] = Diff(rgc, synth).time(max(args.steps, 5))
        result["diff_attn_decode"] = DiffDecode(rgc, synth, args.cache_sets).time(max(args.steps, 30))
        result["prologue"] = time_prologues(pre, max(args.steps, 5))
        result["varlen_prefill"] = Varlen(rgc, synth).time(max(args.steps, 5))
        result["backward"] = time_backward(rgc, synth, max(args.steps, 3))
        result["generation_125m"] = Generation(rgc, synth).time()
        print(f"[bench] timed the variant lines ({time.perf_counter() - t_run:.1f} s)", file=sys.stderr, flush=True)
        result["decode_length_sweep"] = decode_length_sweep(rgc, cache_sets=max(args.cache_sets, 1))
        result["ceilings"] = ceilings()
        print(f"[bench] timed the length sweep and the ceilings ({time.perf_counter() - t_run:.1f} s)", file=sys.stderr, flush=True)
    elif args.with_ceilings:
        result["ceilings"] = ceilings(iters=2)
    result["pages_context"] = PAGES_CONTEXT
    if not args.no_cpu_baseline and args.phase == "all":
        print(f"[bench] timing the CPU oracle ({time.perf_counter() - t_run:.1f} s)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(pre, dec, args.cpu_seconds)
    print(f"[bench] done ({time.perf_counter() - t_run:.1f} s)", file=sys.stderr, flush=True)
    print(json.dumps(result, ensure_ascii=False), flush=True)


if __name__ == "__main__":
    main()
