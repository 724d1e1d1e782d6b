"""CPU: the bench's host logic that decides what it reports -- the one-GPU
guard, and the code hash that keeps stored counter figures attached only to
the kernel source they were taken on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def _tree(tmp_path, kernel, header):
    csrc = tmp_path / "rope_gqa_causal_amd" / "csrc"
    csrc.mkdir(parents=True, exist_ok=True)
    (csrc / "k.hip").write_text(kernel)
    (csrc / "h.h").write_text(header)


def test_kernel_hash_ignores_comments_and_whitespace_but_not_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _tree(tmp_path, '#include "h.h"\n// a comment\nint f(int x) { return x + 1; }\n', "int g();\n")
    base = bench.kernel_sha("k.hip")
    _tree(tmp_path, '#include "h.h"\n/* another\n comment */\nint  f(int x)\n{ return x + 1; }  // note\n',
          "int g();  // header comment\n")
    assert bench.kernel_sha("k.hip") == base
    _tree(tmp_path, '#include "h.h"\nint f(int x) { return x + 2; }\n', "int g();\n")
    assert bench.kernel_sha("k.hip") != base
    _tree(tmp_path, '#include "h.h"\n// a comment\nint f(int x) { return x + 1; }\n', "int g(int);\n")
    assert bench.kernel_sha("k.hip") != base  # a local header the kernel includes is part of its code


def test_stored_traffic_is_reported_only_for_the_kernel_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    _tree(tmp_path, "int f() { return 1; }\n", "")
    rec = {"kernel_sha": bench.kernel_sha("k.hip"), "traffic_bytes_per_launch": 12345}
    (tmp_path / "counters_x.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("x", "k.hip", 0) == 12345
    _tree(tmp_path, "int f() { return 2; }\n", "")
    assert bench.stored_traffic("x", "k.hip", 0) is None
    assert bench.stored_traffic("missing", "k.hip", 0) is None
