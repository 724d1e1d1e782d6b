"""The C ABI library loads, exports what include/rgc.h declares, and checks
its arguments on the host before any HIP call (no GPU needed: every call here
is rejected or is a no-op before a launch)."""
import ctypes
import os
import re

import pytest

import rope_gqa_causal_amd as rgc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rgc.h")

# Status codes from include/rgc.h
OK, NULL, SHAPE, GROUP, DTYPE, HEADDIM, LAYOUT, CAPACITY, WORKSPACE = 0, -1, -2, -3, -4, -5, -6, -7, -8
BF16, F32 = 1, 0
A = 0x10000  # a 16-byte-aligned fake device address; never dereferenced by a rejected call


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(rgc_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_are_exported():
    lib = rgc.library()
    names = _declared()
    assert {"rgc_rope_apply", "rgc_kv_cache_append", "rgc_rope_append", "rgc_norm_rope_append",
            "rgc_gqa_attn_prefill",
            "rgc_gqa_attn_decode", "rgc_gqa_attn_decode_workspace_size", "rgc_gqa_attn_decode_rope_append",
            "rgc_diff_attn_prefill", "rgc_gqa_attn_prefill_varlen", "rgc_rope_backward",
            "rgc_gqa_attn_backward", "rgc_gqa_attn_backward_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    lib = rgc.library()
    assert lib.rgc_abi_version() == 1
    for st in range(-10, 1):
        assert lib.rgc_status_string(st)
    assert lib.rgc_status_string(GROUP).decode() == "Hq is not a multiple of Hkv"


def _prefill(**kw):
    a = dict(o=A, q=A, k=A, v=A, dt=BF16, B=1, Sq=4, Hq=4, Hkv=2, D=128, S_max=16,
             q_sb=4 * 4 * 128, q_ss=4 * 128, q_sh=128, o_sb=4 * 4 * 128, o_ss=4 * 128, o_sh=128,
             kv_sb=2 * 16 * 128, kv_sh=16 * 128, kv_ss=128, q_start=None, scale=0.1, lse=None, err=None)
    a.update(kw)
    return rgc.library().rgc_gqa_attn_prefill(
        a["o"], a["q"], a["k"], a["v"], a["dt"], a["B"], a["Sq"], a["Hq"], a["Hkv"], a["D"], a["S_max"],
        a["q_sb"], a["q_ss"], a["q_sh"], a["o_sb"], a["o_ss"], a["o_sh"], a["kv_sb"], a["kv_sh"],
        a["kv_ss"], a["q_start"], a["scale"], a["lse"], a["err"], None)


def test_prefill_rejects_bad_arguments_before_launch():
    assert _prefill(Hq=3, Hkv=2) == GROUP          # configuration assertion: Hq % Hkv
    assert _prefill(dt=7) == DTYPE
    assert _prefill(D=96) == HEADDIM
    assert _prefill(Sq=-1) == SHAPE
    assert _prefill(Hkv=0) == SHAPE
    assert _prefill(q=None) == NULL
    assert _prefill(o=A + 2) == LAYOUT
    assert _prefill(q_ss=4 * 128 + 1) == LAYOUT
    assert _prefill(kv_ss=1 << 24) == LAYOUT       # bf16 token stride past 2^24 elements
    assert _prefill(kv_ss=-128) == LAYOUT
    assert _prefill(Sq=17) == CAPACITY
    assert _prefill(scale=float("nan")) == -10
    assert _prefill(B=0) == OK                      # empty batch: a no-op
    assert _prefill(Sq=0) == OK


def _diff(**kw):
    a = dict(o=A, q1=A, q2=A, k1=A, k2=A, v=A, dt=BF16, B=2, Sq=16, Hq=4, Hkv=2, D=64, S_max=16,
             q_sb=16 * 4 * 64, q_ss=4 * 64, q_sh=64, o_sb=16 * 4 * 64, o_ss=4 * 64, o_sh=64,
             kv_sb=2 * 16 * 64, kv_sh=16 * 64, kv_ss=64, q_start=None, lam=0.8, scale=0.125, err=None)
    a.update(kw)
    return rgc.library().rgc_diff_attn_prefill(
        a["o"], a["q1"], a["q2"], a["k1"], a["k2"], a["v"], a["dt"], a["B"], a["Sq"], a["Hq"], a["Hkv"],
        a["D"], a["S_max"], a["q_sb"], a["q_ss"], a["q_sh"], a["o_sb"], a["o_ss"], a["o_sh"],
        a["kv_sb"], a["kv_sh"], a["kv_ss"], a["q_start"], a["lam"], a["scale"], a["err"], None)


def test_diff_rejects_bad_arguments_before_launch():
    assert _diff(Hq=3) == GROUP
    assert _diff(dt=F32) == DTYPE        # bf16 only
    assert _diff(D=96) == HEADDIM        # head dims 32, 64, 128
    assert _diff(q2=None) == NULL
    assert _diff(k2=A + 8) == LAYOUT
    assert _diff(kv_ss=1 << 24) == LAYOUT
    assert _diff(Sq=17) == CAPACITY
    assert _diff(lam=float("inf")) == -10
    assert _diff(B=0) == OK
    assert _diff(Sq=0) == OK


def _varlen(**kw):
    a = dict(o=A, q=A, k=A, v=A, dt=BF16, n=3, cu=A, maxlen=16, T=40, Hq=4, Hkv=2, D=64, q_ts=256, q_hs=64,
             o_ts=256, o_hs=64, kv_ts=128, kv_hs=64, scale=0.125, lse=None, err=None)
    a.update(kw)
    return rgc.library().rgc_gqa_attn_prefill_varlen(
        a["o"], a["q"], a["k"], a["v"], a["dt"], a["n"], a["cu"], a["maxlen"], a["T"], a["Hq"], a["Hkv"], a["D"],
        a["q_ts"], a["q_hs"], a["o_ts"], a["o_hs"], a["kv_ts"], a["kv_hs"], a["scale"], a["lse"], a["err"], None)


def test_varlen_rejects_bad_arguments_before_launch():
    assert _varlen(Hq=3) == GROUP
    assert _varlen(dt=F32) == DTYPE
    assert _varlen(D=96) == HEADDIM
    assert _varlen(cu=None) == NULL
    assert _varlen(maxlen=41) == CAPACITY
    assert _varlen(kv_ts=127) == LAYOUT
    assert _varlen(kv_ts=1 << 24) == LAYOUT
    assert _varlen(n=0) == OK
    assert _varlen(T=0, maxlen=0) == OK


def _bwd(**kw):
    a = dict(dq=A, dk=A, dv=A, q=A, k=A, v=A, o=A, do=A, lse=A, dt=BF16, B=2, S=16, Hq=4, Hkv=2, D=64,
             q_sb=16 * 4 * 64, q_ss=4 * 64, q_sh=64, kv_sb=16 * 2 * 64, kv_ss=2 * 64, kv_sh=64, scale=0.125,
             ws=A, ws_bytes=1 << 20)
    a.update(kw)
    return rgc.library().rgc_gqa_attn_backward(
        a["dq"], a["dk"], a["dv"], a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dt"], a["B"], a["S"],
        a["Hq"], a["Hkv"], a["D"], a["q_sb"], a["q_ss"], a["q_sh"], a["kv_sb"], a["kv_ss"], a["kv_sh"],
        a["scale"], a["ws"], a["ws_bytes"], None)


def test_backward_rejects_bad_arguments_before_launch():
    assert _bwd(Hq=3) == GROUP
    assert _bwd(dt=F32) == DTYPE
    assert _bwd(D=96) == HEADDIM
    assert _bwd(lse=None) == NULL
    assert _bwd(dk=A + 4) == LAYOUT
    assert _bwd(ws_bytes=16) == WORKSPACE
    assert _bwd(ws=A + 16) == LAYOUT
    assert _bwd(q_ss=1 << 24) == LAYOUT  # row offsets are 32-bit inside the kernels
    assert _bwd(q_ss=-4 * 64) == LAYOUT
    assert _bwd(kv_ss=1 << 24) == LAYOUT
    assert _bwd(B=0) == OK
    assert rgc.library().rgc_gqa_attn_backward_workspace_size(2, 16, 4) >= 2 * 16 * 4 * 4


def _decode(**kw):
    a = dict(o=A, q=A, k=A, v=A, dt=BF16, B=2, Hq=4, Hkv=2, D=64, S_max=32, q_sb=256, q_sh=64,
             o_sb=256, o_sh=64, kv_sb=2 * 32 * 64, kv_sh=32 * 64, kv_ss=64, lens=A, max_len=32,
             scale=0.125, ws=A, ws_bytes=1 << 20, lse=None, err=None)
    a.update(kw)
    return rgc.library().rgc_gqa_attn_decode(
        a["o"], a["q"], a["k"], a["v"], a["dt"], a["B"], a["Hq"], a["Hkv"], a["D"], a["S_max"],
        a["q_sb"], a["q_sh"], a["o_sb"], a["o_sh"], a["kv_sb"], a["kv_sh"], a["kv_ss"], a["lens"],
        a["max_len"], a["scale"], a["ws"], a["ws_bytes"], a["lse"], a["err"], None)


def test_decode_rejects_bad_arguments_before_launch():
    assert _decode(Hq=6, Hkv=4) == GROUP
    assert _decode(lens=None) == NULL
    assert _decode(max_len=33) == CAPACITY
    assert _decode(max_len=0) == CAPACITY
    assert _decode(ws=None) == WORKSPACE
    assert _decode(ws_bytes=16) == WORKSPACE
    assert _decode(ws=A + 16) == LAYOUT
    assert _decode(kv_ss=68) == LAYOUT
    assert _decode(D=48) == HEADDIM
    assert _decode(B=0) == OK


ARG = -10


def _decode_rope(**kw):
    a = dict(o=A, q=A, kn=A, vn=A, k=A, v=A, dt=BF16, B=2, Hq=4, Hkv=2, D=64, S_max=32, q_sb=256, q_sh=64,
             n_sb=128, n_sh=64, o_sb=256, o_sh=64, kv_sb=2 * 32 * 64, kv_sh=32 * 64, kv_ss=64, lens=A,
             max_len=32, base=10000.0, style=0, scale=0.125, ws=A, ws_bytes=1 << 20, lse=None, err=None)
    a.update(kw)
    return rgc.library().rgc_gqa_attn_decode_rope_append(
        a["o"], a["q"], a["kn"], a["vn"], a["k"], a["v"], a["dt"], a["B"], a["Hq"], a["Hkv"], a["D"],
        a["S_max"], a["q_sb"], a["q_sh"], a["n_sb"], a["n_sh"], a["o_sb"], a["o_sh"], a["kv_sb"], a["kv_sh"],
        a["kv_ss"], a["lens"], a["max_len"], a["base"], a["style"], a["scale"], a["ws"], a["ws_bytes"],
        a["lse"], a["err"], None)


def test_fused_decode_step_rejects_bad_arguments_before_launch():
    assert _decode_rope(dt=F32) == DTYPE  # the fused step is bf16 only
    assert _decode_rope(dt=7) == DTYPE
    assert _decode_rope(style=2) == ARG
    assert _decode_rope(base=0.0) == ARG
    assert _decode_rope(base=float("inf")) == ARG
    assert _decode_rope(scale=float("nan")) == ARG
    assert _decode_rope(Hq=6, Hkv=4) == GROUP
    assert _decode_rope(D=48) == HEADDIM
    assert _decode_rope(kn=None) == NULL
    assert _decode_rope(vn=None) == NULL
    assert _decode_rope(lens=None) == NULL
    assert _decode_rope(kn=A + 2) == LAYOUT
    assert _decode_rope(n_sh=60) == LAYOUT
    assert _decode_rope(max_len=33) == CAPACITY
    assert _decode_rope(ws=None) == WORKSPACE
    assert _decode_rope(ws_bytes=16) == WORKSPACE
    assert _decode_rope(ws=A + 16) == LAYOUT
    assert _decode_rope(B=0) == OK


def test_decode_workspace_size_grows_with_the_split_count():
    lib = rgc.library()
    one = lib.rgc_gqa_attn_decode_workspace_size(64, 24, 8, 128, 256)
    many = lib.rgc_gqa_attn_decode_workspace_size(64, 24, 8, 128, 2080)
    assert 0 < one < many
    assert lib.rgc_gqa_attn_decode_workspace_size(64, 24, 8, 100, 2080) == 0


def test_rope_and_append_reject_bad_arguments_before_launch():
    lib = rgc.library()
    rope = lambda **kw: lib.rgc_rope_apply(kw.get("x", A), kw.get("dt", BF16), 1, 4, 2, kw.get("D", 64),
                                           512, 128, 64, None, kw.get("base", 10000.0),
                                           kw.get("style", 0), None)
    assert rope(D=3) == HEADDIM
    assert rope(D=258) == HEADDIM
    assert rope(style=2) == -10
    assert rope(base=-1.0) == -10
    assert rope(x=None) == NULL
    assert rope(x=A + 1) == LAYOUT
    app = lambda **kw: lib.rgc_kv_cache_append(A, A, BF16, 1, 2, kw.get("D", 64), kw.get("S_max", 8),
                                               1024, 512, 64, A, A, kw.get("S_new", 4), 512, 128, 64,
                                               kw.get("pos0", A), None, None)
    assert app(S_new=9) == CAPACITY
    assert app(pos0=None) == NULL
    assert app(D=40) == HEADDIM
    assert app(S_new=0) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rgc.rope_apply(x)


def test_product_library_has_no_timing_state_and_the_timed_build_exports_all():
    lib = rgc.library()
    assert not hasattr(lib, "rgc_timing_enable") and not hasattr(lib, "rgc_timing_report")
    timed = rgc.timed_library()
    timing_names = sorted(set(re.findall(r"\b(rgc_[a-z0-9_]+)\s*\(", open(os.path.join(ROOT, "include", "rgc_timing.h")).read())))
    assert timing_names == ["rgc_timing_enable", "rgc_timing_report"]
    for n in _declared() + timing_names:
        assert hasattr(timed, n), n


def test_timing_switch_and_empty_report():
    lib = rgc.timed_library()
    assert lib.rgc_timing_enable(1) == OK
    assert lib.rgc_timing_enable(0) == OK
    assert rgc.timing_report() == {}  # nothing launched: no lines
    buf = ctypes.create_string_buffer(16)
    assert lib.rgc_timing_report(buf, len(buf)) == 0 and buf.value == b""
    assert lib.rgc_timing_report(None, 16) == -10  # RGC_ERR_ARG
    assert lib.rgc_timing_report(buf, 0) == -10


@pytest.mark.parametrize("scale", [0.0, -0.125, float("inf"), float("nan")])
def test_attention_entries_reject_a_scale_that_is_not_positive_and_finite(scale):
    # The bf16 kernels mask a score by setting it to -inf before it is
    # multiplied by the scale, which is only the mask a positive scale needs;
    # every attention entry therefore takes the same rule: scale > 0, finite.
    assert _prefill(scale=scale) == ARG
    assert _prefill(scale=scale, dt=F32) == ARG
    assert _diff(scale=scale) == ARG
    assert _varlen(scale=scale) == ARG
    assert _bwd(scale=scale) == ARG
    assert _decode(scale=scale) == ARG
    assert _decode_rope(scale=scale) == ARG


def _decode_static(**kw):
    a = dict(o=A, q=A, kn=A, vn=A, k=A, v=A, dt=BF16, B=2, Hq=4, Hkv=2, D=64, S_max=32, q_sb=256, q_sh=64,
             n_sb=128, n_sh=64, o_sb=256, o_sh=64, kv_sb=2 * 32 * 64, kv_sh=32 * 64, kv_ss=64, lens=A,
             max_len=32, base=10000.0, style=0, scale=0.125, lse=None, err=None)
    a.update(kw)
    return rgc.library().rgc_gqa_attn_decode_rope_append_static(
        a["o"], a["q"], a["kn"], a["vn"], a["k"], a["v"], a["dt"], a["B"], a["Hq"], a["Hkv"], a["D"],
        a["S_max"], a["q_sb"], a["q_sh"], a["n_sb"], a["n_sh"], a["o_sb"], a["o_sh"], a["kv_sb"], a["kv_sh"],
        a["kv_ss"], a["lens"], a["max_len"], a["base"], a["style"], a["scale"], a["lse"], a["err"], None)


def test_allocation_free_decode_step_checks_its_arguments_and_its_array_size():
    lib = rgc.library()
    assert _decode_static(dt=F32) == DTYPE
    assert _decode_static(scale=0.0) == ARG
    assert _decode_static(kn=None) == NULL
    assert _decode_static(max_len=33) == CAPACITY
    assert _decode_static(B=0) == OK
    # partials beyond the 16 MiB array: refused before anything is launched
    big = dict(B=64, Hq=64, Hkv=8, D=128, S_max=8192, max_len=8192, q_sb=64 * 128, o_sb=64 * 128,
               n_sb=8 * 128, kv_sb=8 * 8192 * 128, kv_sh=8192 * 128, kv_ss=128, q_sh=128, o_sh=128, n_sh=128)
    assert lib.rgc_gqa_attn_decode_workspace_size(64, 64, 8, 128, 8192) > 16 << 20
    assert _decode_static(**big) == WORKSPACE
    # the ragged-decode shape fits
    assert lib.rgc_gqa_attn_decode_workspace_size(64, 24, 8, 128, 2080) <= 16 << 20


def _diff_decode(**kw):
    a = dict(o=A, q1=A, q2=A, k1=A, k2=A, v=A, dt=BF16, B=2, Hq=4, Hkv=2, D=64, S_max=32, q_sb=256, q_sh=64,
             o_sb=256, o_sh=64, kv_sb=2 * 32 * 64, kv_sh=32 * 64, kv_ss=64, lens=A, max_len=32, lam=0.8,
             scale=0.125, ws=A, ws_bytes=1 << 20, err=None)
    a.update(kw)
    return rgc.library().rgc_diff_attn_decode(
        a["o"], a["q1"], a["q2"], a["k1"], a["k2"], a["v"], a["dt"], a["B"], a["Hq"], a["Hkv"], a["D"],
        a["S_max"], a["q_sb"], a["q_sh"], a["o_sb"], a["o_sh"], a["kv_sb"], a["kv_sh"], a["kv_ss"], a["lens"],
        a["max_len"], a["lam"], a["scale"], a["ws"], a["ws_bytes"], a["err"], None)


def test_diff_decode_rejects_bad_arguments_before_launch():
    lib = rgc.library()
    assert _diff_decode(Hq=3) == GROUP
    assert _diff_decode(dt=F32) == DTYPE
    assert _diff_decode(D=96) == HEADDIM
    assert _diff_decode(q2=None) == NULL
    assert _diff_decode(lens=None) == NULL
    assert _diff_decode(k2=A + 8) == LAYOUT
    assert _diff_decode(kv_ss=68) == LAYOUT
    assert _diff_decode(max_len=33) == CAPACITY
    assert _diff_decode(lam=float("nan")) == ARG
    assert _diff_decode(scale=0.0) == ARG
    assert _diff_decode(ws=None) == WORKSPACE
    assert _diff_decode(ws_bytes=16) == WORKSPACE
    assert _diff_decode(ws=A + 16) == LAYOUT
    assert _diff_decode(B=0) == OK
    assert 0 < lib.rgc_diff_attn_decode_workspace_size(4, 16, 8, 64, 128) < \
        lib.rgc_diff_attn_decode_workspace_size(4, 16, 8, 64, 1024)
