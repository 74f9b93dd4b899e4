"""GPU test of the allocation-free entry point attn_fwd_bf16_hd_noalloc,
through the C ABI: its output (and log-sum-exp) equals attn_fwd_bf16_hd's
bit for bit on shapes whose plan splits the key range (so the fixed scratch
array carries the partials), on consecutive calls with a smaller second
input, and when the call is captured into a HIP graph without any eager
call of that shape before (nothing to allocate)."""
import ctypes

import numpy as np
import pytest
import torch

from bf16_attention_forward_amd import load_library
from bf16_attention_forward_amd import workloads as wl
from tests.helpers import say, to_dev

pytestmark = pytest.mark.gpu

LAYOUT = {"bshd": 0, "bhsd": 1}


def call(fn, q, k, v, o, lse, layout, Hkv, causal, mode):
    if layout == "bshd":
        B, Sq, Hq, D = q.shape
        Skv = k.shape[1]
    else:
        B, Hq, Sq, D = q.shape
        Skv = k.shape[2]
    stream = torch.cuda.current_stream().cuda_stream
    return fn(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
              ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()), LAYOUT[layout], B, Hq, Hkv, Sq, Skv,
              D, ctypes.c_float(float(np.float32(1.0 / np.sqrt(D)))), 1 if causal else 0, mode,
              ctypes.c_void_p(stream))


# (layout, B, Hq, Hkv, Sq, Skv, D, causal): each call's plan splits the keys
# (few query tiles) except the causal one, which never splits.  The second
# call is smaller than the first, so it runs on an array that still holds a
# larger call's partials beyond its own.
CALLS = [
    ("bhsd", 1, 3, 3, 300, 1000, 128, False),    # 4-wave groups, 9 tiles split 8 ways
    ("bshd", 1, 2, 1, 200, 700, 128, False),     # smaller: 4 tiles split 5 ways, grouped heads
    ("bhsd", 1, 2, 2, 260, 1500, 128, False),    # 8-wave groups, 4 tiles split
    ("bshd", 2, 2, 2, 90, 640, 64, False),       # head dimension 64
    ("bhsd", 1, 4, 2, 300, 300, 128, True),      # causal: no split, the array unused
]


def test_noalloc_matches_the_allocating_entry_point():
    lib = load_library()
    for n, (layout, B, Hq, Hkv, Sq, Skv, D, causal) in enumerate(CALLS):
        say(f"[case] noalloc call {n}: {layout} B{B} Hq{Hq} Hkv{Hkv} {Sq}x{Skv} d{D} causal={causal}")
        q, k, v = wl.random_qkv(layout, B, Hq, Sq, Skv, 5100 + n, 1.0, 2.0, 1.0, Hkv=Hkv, D=D)
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        for mode in (0, 2):
            oa, ob = torch.empty_like(qd), torch.empty_like(qd)
            la = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
            lb = torch.empty_like(la)
            assert call(lib.attn_fwd_bf16_hd_noalloc, qd, kd, vd, oa, la, layout, Hkv, causal, mode) == 0
            assert call(lib.attn_fwd_bf16_hd, qd, kd, vd, ob, lb, layout, Hkv, causal, mode) == 0
            torch.cuda.synchronize()
            assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), (n, mode)
            assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), (n, mode)


def test_noalloc_call_captured_without_warm_up():
    """Captured into a graph with no eager call of the shape before it, the
    allocation-free call replays to the allocating entry point's result, replay
    after replay, with other work on the GPU between replays."""
    lib = load_library()
    layout, B, Hq, Hkv, Sq, Skv, D = "bhsd", 1, 3, 3, 333, 1111, 128
    q, k, v = wl.random_qkv(layout, B, Hq, Sq, Skv, 5200, 1.0, 2.0, 1.0, D=D)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = torch.empty_like(qd)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rc = call(lib.attn_fwd_bf16_hd_noalloc, qd, kd, vd, o, lse, layout, Hkv, False, 0)
    assert rc == 0
    ref, lref = torch.empty_like(qd), torch.empty_like(lse)
    assert call(lib.attn_fwd_bf16_hd, qd, kd, vd, ref, lref, layout, Hkv, False, 0) == 0
    torch.cuda.synchronize()
    for r in range(3):
        o.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), r
        assert torch.equal(lse.view(torch.int32), lref.view(torch.int32)), r
        # other work between replays
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()
