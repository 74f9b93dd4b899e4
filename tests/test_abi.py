"""C ABI checks that need no GPU: every symbol the header declares is
exported, and argument errors are reported before any device work."""
import math
import re
import os

import numpy as np
import pytest

import bf16_attention_forward_amd as pkg
from bf16_attention_forward_amd import attn_fwd_bf16_raw, load_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s+(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(pkg.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    assert pkg.attn_version() >= 10000
    for code in range(-12, 1):
        assert pkg.attn_status_string(code)
    assert pkg.attn_status_string(-999) == "unknown status"


FAKE = 1 << 40   # 16-byte aligned, never dereferenced: validation fails first


def call(**kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), o=FAKE + (3 << 30), layout=0, B=1, H=2,
             Sq=64, Skv=64, scale=0.088, mode=0, stream=0, splits=0, order=0, waves=0, grid=0)
    a.update(kw)
    return attn_fwd_bf16_raw(a["q"], a["k"], a["v"], a["o"], a["layout"], a["B"], a["H"], a["Sq"], a["Skv"],
                             a["scale"], a["mode"], a["stream"], a["splits"], a["order"], a["waves"], a["grid"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), -1), (dict(o=0), -1), (dict(layout=2), -2), (dict(layout=-1), -2),
    (dict(mode=3), -3), (dict(mode=0x100 | 3), -3), (dict(mode=0x200), -3), (dict(mode=0x101 | 0x10000), -3),
    (dict(B=0), -4), (dict(H=0), -4), (dict(Sq=0), -4), (dict(Skv=0), -4),
    (dict(Skv=-5), -4), (dict(Sq=1 << 40), -4), (dict(scale=math.nan), -5), (dict(scale=math.inf), -5),
    (dict(q=FAKE + 8), -6), (dict(o=FAKE + (3 << 30) + 2), -6), (dict(o=FAKE), -7),
    (dict(o=FAKE + 64 * 2 * 128 * 2 - 16), -7), (dict(splits=65), -11), (dict(order=3), -11),
    (dict(waves=3), -11), (dict(waves=16), -11), (dict(waves=-4), -11), (dict(waves=2), -11), (dict(grid=-1), -11),
])
def test_argument_errors_before_device(kw, code):
    assert call(**kw) == code


def test_key_extent_limit_edge():
    """A head's K/V rows are addressed with 32-bit byte offsets: the last
    row must start below 2^31 - 256.  BSHD with 16 heads (4096-byte rows):
    524288 keys are accepted (they reach the device probe), 524289 are not."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    G = 1 << 33
    kw = dict(q=FAKE, k=FAKE + G, v=FAKE + 2 * G, o=FAKE + 3 * G, layout=0, H=16, Sq=300)
    assert call(Skv=524288, **kw) == -8
    assert call(Skv=524289, **kw) == -4
    # BHSD rows are 256 bytes: 2^23 - 1 keys per head
    kw.update(layout=1, H=1)
    assert call(Skv=(1 << 23) - 1, **kw) == -8
    assert call(Skv=1 << 23, **kw) == -4


def test_valid_arguments_reach_device_check():
    # without a GPU a valid call stops at the device probe (-8); with one this test is skipped
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call() == -8
    for m in (0x100, 0x101, 0x102):   # ATTN_ROUND_WEIGHTS with each output mode is valid
        assert call(mode=m) == -8
    for w in (4, 8):                  # both work-group sizes are valid for any length
        assert call(waves=w) == -8 and call(waves=w, Skv=5000) == -8


def call_gqa(**kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), o=FAKE + (3 << 30), lse=None, layout=1, B=1, Hq=8,
             Hkv=2, Sq=64, Skv=64, scale=0.088, causal=1, mode=0, stream=0)
    a.update(kw)
    return load_library().attn_fwd_bf16_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["layout"], a["B"], a["Hq"],
                                            a["Hkv"], a["Sq"], a["Skv"], a["scale"], a["causal"], a["mode"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), -1), (dict(layout=5), -2), (dict(mode=-1), -3), (dict(Hkv=0), -4), (dict(Hkv=3), -4),
    (dict(Hq=2, Hkv=4), -4), (dict(scale=-math.inf), -5), (dict(v=FAKE + (2 << 30) + 4), -6),
    (dict(o=FAKE + (2 << 30) + 64 * 2 * 128 * 2 - 16), -7), (dict(causal=2), -11), (dict(causal=-1), -11),
    (dict(lse=FAKE + (4 << 30) + 2), -6), (dict(lse=FAKE + (3 << 30) + 64), -7), (dict(lse=FAKE + 4), -7),
])
def test_gqa_argument_errors_before_device(kw, code):
    assert call_gqa(**kw) == code


def call_hd(**kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), o=FAKE + (3 << 30), lse=None, layout=0, B=1, Hq=4,
             Hkv=2, Sq=64, Skv=64, hd=64, scale=0.125, causal=0, mode=0, stream=0)
    a.update(kw)
    return load_library().attn_fwd_bf16_hd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["layout"], a["B"], a["Hq"],
                                           a["Hkv"], a["Sq"], a["Skv"], a["hd"], a["scale"], a["causal"], a["mode"],
                                           a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(hd=96), -4), (dict(hd=0), -4), (dict(hd=256), -4), (dict(hd=-64), -4), (dict(q=0), -1),
    (dict(Hkv=3), -4), (dict(mode=5), -3), (dict(causal=3), -11), (dict(v=FAKE + (2 << 30) + 8), -6),
    # with head_dim 64, o overlaps q only if it starts inside q's 64*4*64*2 bytes
    (dict(o=FAKE + 64 * 4 * 64 * 2 - 16), -7),
])
def test_hd_argument_errors_before_device(kw, code):
    assert call_hd(**kw) == code


def test_hd_valid_arguments_reach_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call_hd() == -8
    assert call_hd(hd=128) == -8
    assert call_hd(o=FAKE + 64 * 4 * 64 * 2) == -8    # just past q (64-dim rows): no overlap


def test_gqa_valid_arguments_reach_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call_gqa() == -8
    assert call_gqa(causal=0, Hkv=8) == -8
    assert call_gqa(lse=FAKE + (4 << 30)) == -8
    assert call_gqa(mode=0x102) == -8


def call_bwd(**kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), o=FAKE + (3 << 30), do=FAKE + (4 << 30),
             lse=FAKE + (5 << 30), dq=FAKE + (6 << 30), dk=FAKE + (7 << 30), dv=FAKE + (8 << 30), layout=1,
             B=1, H=2, Hkv=2, Sq=64, Skv=64, hd=128, scale=0.088, causal=0, stream=0)
    a.update(kw)
    return load_library().attn_bwd_bf16(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                                        a["dv"], a["layout"], a["B"], a["H"], a["Hkv"], a["Sq"], a["Skv"],
                                        a["hd"], a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(do=0), -1), (dict(lse=0), -1), (dict(dv=0), -1), (dict(layout=3), -2), (dict(Sq=0), -4),
    (dict(Skv=-1), -4), (dict(scale=math.nan), -5), (dict(dq=FAKE + (6 << 30) + 8), -6),
    (dict(lse=FAKE + (5 << 30) + 2), -6),
    (dict(dq=FAKE + 64), -7),                           # dq overlaps q
    (dict(dk=FAKE + (6 << 30) + 16), -7),               # dk overlaps dq
    (dict(dv=FAKE + (5 << 30)), -7),                    # dv overlaps lse
    (dict(causal=2), -11), (dict(causal=-1), -11),
    (dict(Hkv=0), -4), (dict(Hkv=3), -4), (dict(H=4, Hkv=3), -4), (dict(hd=96), -4), (dict(hd=256), -4),
])
def test_bwd_argument_errors_before_device(kw, code):
    assert call_bwd(**kw) == code


def test_bwd_valid_arguments_reach_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call_bwd() == -8
    assert call_bwd(causal=1) == -8
    assert call_bwd(H=4, Hkv=1) == -8 and call_bwd(H=4, Hkv=2, causal=1) == -8
    assert call_bwd(hd=64) == -8


def call_paged(**kw):
    a = dict(q=FAKE, kc=FAKE + (1 << 30), vc=FAKE + (2 << 30), bt=FAKE + (4 << 30), kl=FAKE + (5 << 30),
             o=FAKE + (3 << 30), lse=None, layout=0, B=2, Hq=4, Hkv=2, Sq=64, max_kv=300, ps=64, pps=5, npages=10,
             hd=128, scale=0.0883883, causal=0, mode=0, stream=0)
    a.update(kw)
    return load_library().attn_fwd_bf16_paged(a["q"], a["kc"], a["vc"], a["bt"], a["kl"], a["o"], a["lse"],
                                              a["layout"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["max_kv"],
                                              a["ps"], a["pps"], a["npages"], a["hd"], a["scale"], a["causal"],
                                              a["mode"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(bt=0), -1), (dict(kl=0), -1), (dict(kc=0), -1), (dict(q=0), -1),
    (dict(ps=0), -4), (dict(npages=0), -4), (dict(pps=4), -4),          # 4 pages of 64 do not cover 300 keys
    (dict(max_kv=0), -4), (dict(hd=96), -4), (dict(Hkv=3), -4), (dict(max_kv=1 << 31), -4),
    (dict(kc=FAKE + (1 << 30) + 8), -6), (dict(bt=FAKE + (4 << 30) + 2), -6), (dict(kl=FAKE + (5 << 30) + 1), -6),
    (dict(o=FAKE + (1 << 30) + 64), -7),                                # o inside the key cache
    (dict(mode=5), -3), (dict(causal=2), -11), (dict(layout=7), -2), (dict(scale=float("nan")), -5),
])
def test_paged_argument_errors_before_device(kw, code):
    assert call_paged(**kw) == code


def test_paged_valid_arguments_reach_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call_paged() == -8
    assert call_paged(causal=1, hd=64, layout=1) == -8
    assert call_paged(pps=5, max_kv=320) == -8                          # exactly covered


def call_varlen(**kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), o=FAKE + (3 << 30), lse=None,
             cq=FAKE + (4 << 30), ck=FAKE + (5 << 30), B=3, Hq=4, Hkv=2, tq=500, tk=700, mq=300, mk=400,
             hd=128, scale=0.0883883, causal=0, mode=0, stream=0)
    a.update(kw)
    return load_library().attn_fwd_bf16_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"],
                                               a["B"], a["Hq"], a["Hkv"], a["tq"], a["tk"], a["mq"], a["mk"],
                                               a["hd"], a["scale"], a["causal"], a["mode"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(cq=0), -1), (dict(ck=0), -1), (dict(q=0), -1), (dict(o=0), -1),
    (dict(B=0), -4), (dict(tq=0), -4), (dict(tk=0), -4), (dict(mq=0), -4), (dict(mk=0), -4),
    (dict(hd=96), -4), (dict(Hkv=3), -4), (dict(tq=1 << 31), -4), (dict(mk=1 << 31), -4),
    (dict(cq=FAKE + (4 << 30) + 2), -6), (dict(ck=FAKE + (5 << 30) + 1), -6), (dict(q=FAKE + 8), -6),
    (dict(o=FAKE + (1 << 30) + 64), -7),                                  # o inside k
    (dict(lse=FAKE + (3 << 30) + 16), -7),                                # lse inside o
    (dict(mode=5), -3), (dict(causal=2), -11), (dict(scale=float("nan")), -5),
])
def test_varlen_argument_errors_before_device(kw, code):
    assert call_varlen(**kw) == code


def test_varlen_valid_arguments_reach_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call_varlen() == -8
    assert call_varlen(causal=1, hd=64, lse=FAKE + (6 << 30)) == -8
