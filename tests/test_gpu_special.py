"""GPU exactness cases, memory-safety checks and device-side error codes."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from bf16_attention_forward_amd import workloads as wl
from bf16_attention_forward_amd import attn_fwd_bf16, attn_fwd_bf16_raw, load_library
from tests.helpers import assert_gates, check, run_hip, say

pytestmark = pytest.mark.gpu
MODES = ("rtne", "rtna", "rtz")


def bf(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("mode", MODES)
def test_single_key_returns_value_row_bitwise(mode):
    q, k, v = wl.random_qkv("bshd", 1, 3, 200, 1, 31)
    o = run_hip(q, k, v, "bshd", mode).reshape(1, 200, 3, 128)
    assert np.array_equal(o, np.broadcast_to(wl.bits(v)[:, :1], o.shape))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("how", ["zero_q", "zero_scale"])
def test_equal_scores_tie_cases_bitwise(mode, how):
    skv = 64
    q, k, _ = wl.random_qkv("bhsd", 1, 2, 40, skv, 32)
    vals = np.where(np.arange(skv) % 2 == 0, 1.0, 1.0 + 2.0 ** -7)
    v = bf(np.broadcast_to(vals[None, None, :, None], (1, 2, skv, 128)).copy())
    scale = wl.DEFAULT_SCALE
    if how == "zero_q":
        q = torch.zeros_like(q)
    else:
        scale = 0.0
    o = run_hip(q, k, v, "bhsd", mode, scale=scale)
    expect = {"rtne": 0x3F80, "rtna": 0x3F81, "rtz": 0x3F80}[mode]
    assert np.all(o == expect)
    res = oracle.attention(wl.bits(q), wl.bits(k), wl.bits(v), layout="bhsd", scale=scale, method=False)
    assert np.array_equal(o.reshape(-1, 128), res.rounded(mode))


@pytest.mark.parametrize("j0", [0, 37, 99])
def test_one_hot_dominant_score_selects_row_bitwise(j0):
    skv = 100
    _, _, v = wl.random_qkv("bshd", 1, 1, 1, skv, 33)
    qv = np.zeros((1, 4, 1, 128)); qv[..., 0] = 128.0
    kv = np.zeros((1, skv, 1, 128)); kv[0, j0, 0, 0] = 128.0; kv[0, :, 0, 1] = 1.0
    for mode in MODES:
        o = run_hip(bf(qv), bf(kv), v, "bshd", mode)
        assert np.array_equal(o.reshape(4, 128), np.broadcast_to(wl.bits(v)[0, j0, 0], (4, 128)))


@pytest.mark.parametrize("scale", [-0.0883883461356163, 0.5, 1e-3])
def test_other_scales_match_oracle(scale):
    q, k, v = wl.random_qkv("bhsd", 1, 2, 150, 270, 34)
    for mode in MODES:
        o = run_hip(q, k, v, "bhsd", mode, scale=scale)
        st, _ = check(o, q, k, v, "bhsd", mode, scale=scale, label=f"scale={scale}")
        assert_gates(st)


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
def test_poison_tails_are_never_read(layout):
    """Rows past Sq / Skv hold NaN; a call with the true lengths must ignore them."""
    Sq, Skv, pad = 131, 97, 64
    q, k, v = wl.random_qkv(layout, 1, 1, Sq + pad, Skv + pad, 35)
    sl = (slice(None), slice(None), slice(None), slice(None))

    def cut(t, n):
        return t[:, :n] if layout == "bshd" else t[:, :, :n]
    for t, n in ((q, Sq), (k, Skv), (v, Skv)):
        if layout == "bshd":
            t[:, n:] = float("nan")
        else:
            t[:, :, n:] = float("nan")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    qv, kv_, vv = cut(qd, Sq), cut(kd, Skv), cut(vd, Skv)   # contiguous prefixes (B = H = 1)
    assert qv.is_contiguous() and kv_.is_contiguous()
    for splits in (0, 2):
        o = attn_fwd_bf16(qv, kv_, vv, layout=layout, kv_splits=splits)
        torch.cuda.synchronize()
        ob = wl.bits(o.cpu())
        assert not np.isnan((ob.astype(np.uint32) << 16).view(np.float32)).any()
        clean = run_hip(cut(q, Sq).contiguous(), cut(k, Skv).contiguous(), cut(v, Skv).contiguous(), layout,
                        kv_splits=splits)
        assert np.array_equal(ob, clean)


def test_output_canaries_untouched():
    B, H, Sq, Skv = 1, 3, 77, 120
    q, k, v = wl.random_qkv("bshd", B, H, Sq, Skv, 36)
    n = B * Sq * H * 128
    guard = 2048   # elements (4 KiB) on each side
    buf = torch.full((n + 2 * guard,), 12345, dtype=torch.int16, device="cuda")
    o = buf[guard:guard + n].view(torch.bfloat16).view(B, Sq, H, 128)
    for splits in (0, 2):
        attn_fwd_bf16(q.cuda(), k.cuda(), v.cuda(), o, layout="bshd", kv_splits=splits)
        torch.cuda.synchronize()
        host = buf.cpu().numpy()
        assert np.all(host[:guard] == 12345) and np.all(host[guard + n:] == 12345)
        assert np.array_equal(wl.bits(o.cpu()), run_hip(q, k, v, "bshd", kv_splits=splits))


def test_device_side_argument_errors():
    q, k, v = (t.cuda() for t in wl.random_qkv("bshd", 1, 2, 64, 64, 37))
    o = torch.empty_like(q)
    st = torch.cuda.current_stream().cuda_stream
    args = lambda qp, op: (qp, k.data_ptr(), v.data_ptr(), op, 0, 1, 2, 64, 64, 0.088, 0, st)
    assert attn_fwd_bf16_raw(*args(q.data_ptr() + 2, o.data_ptr())) == -6     # misaligned
    assert attn_fwd_bf16_raw(*args(q.data_ptr(), q.data_ptr())) == -7         # o aliases q
    assert attn_fwd_bf16_raw(*args(q.data_ptr(), o.data_ptr())) == 0
    torch.cuda.synchronize()
    # forced split larger than the number of key tiles is rejected
    assert attn_fwd_bf16_raw(*args(q.data_ptr(), o.data_ptr()), kv_splits=2) == -11


def ramp_inputs(layout, B, H, Sq, Skv, seed, t_max=470.0):
    """Scores that grow along the keys (for queries with a positive component
    along a shared direction, shrink for the others): later key tiles keep
    outgrowing the softmax offset, which exercises the offset moves."""
    q, _, v = wl.random_qkv(layout, B, H, Sq, Skv, seed)
    g = torch.Generator().manual_seed(seed)
    u = torch.randn(128, generator=g)
    u = u / u.norm()
    t = torch.linspace(0.0, t_max, Skv)
    noise = torch.randn(B, Skv, H, 128, generator=g)
    k = t[None, :, None, None] * u + noise
    if layout == "bhsd":
        k = k.permute(0, 2, 1, 3)
    return q, k.contiguous().to(torch.bfloat16), v


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_growing_scores_move_the_offset(layout, splits):
    q, k, v = ramp_inputs(layout, 1, 2, 300, 1000, 71)
    say(f"[case] growing scores {layout} splits={splits}")
    for mode in MODES:
        o = run_hip(q, k, v, layout, mode, kv_splits=splits)
        st, _ = check(o, q, k, v, layout, mode, label=f"ramp {layout} {splits}")
        assert_gates(st)


def test_growing_scores_causal():
    from tests.helpers import run_hip_gqa
    q, k, v = ramp_inputs("bhsd", 1, 2, 700, 700, 72)
    o = run_hip_gqa(q, k, v, "bhsd", "rtne", causal=True)
    st, _ = check(o, q, k, v, "bhsd", "rtne", label="ramp causal", causal=True)
    assert_gates(st)


def test_graph_capture_replays_match_eager():
    """A launch captured into a HIP graph (torch.cuda.graph) replays to the
    eager result, replay after replay, with eager work in between; the split
    path's workspace is allocated before capture by the eager warm-up call."""
    q, k, v = wl.random_qkv("bhsd", 1, 4, 700, 900, 81)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for splits in (0, 3):
        eager = attn_fwd_bf16(qd, kd, vd, layout="bhsd", kv_splits=splits)
        torch.cuda.synchronize()
        ref = eager.clone()
        out = torch.empty_like(qd)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            attn_fwd_bf16(qd, kd, vd, out, layout="bhsd", kv_splits=splits, stream=s)   # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            attn_fwd_bf16(qd, kd, vd, out, layout="bhsd", kv_splits=splits, stream=s)
        for rep in range(4):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"splits={splits} replay {rep}"
            attn_fwd_bf16(qd, kd, vd, layout="bhsd")   # eager work between replays
            torch.cuda.synchronize()


def test_largest_key_extent_reads_the_last_rows():
    """The largest key extent the 32-bit offsets allow (BSHD, 16 heads,
    524288 keys: 2 GiB each of K and V).  Head h's one dominant key sits
    among the last rows (the last one for head 0), every other score is 0,
    so every output row is that key's V row bitwise -- through the planner's
    split and unsplit."""
    B, H, Sq, Skv = 1, 16, 130, 524288
    say(f"[case] largest key extent bshd B{B} H{H} Sq{Sq} Skv{Skv}")
    dev = torch.device("cuda")
    k = torch.zeros((B, Skv, H, 128), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    q = torch.zeros((B, Sq, H, 128), dtype=torch.bfloat16, device=dev)
    q[..., 0] = 128.0
    j0 = [Skv - 1 - 37 * h for h in range(H)]
    rows = wl.random_qkv("bshd", 1, H, 1, 1, 41)[2]          # [1, 1, H, 128] random bf16 rows
    for h in range(H):
        k[0, j0[h], h, 0] = 128.0
        v[0, j0[h], h] = rows[0, 0, h].to(dev)
    expect = np.broadcast_to(wl.bits(rows)[0, 0][None, :, :], (Sq, H, 128))
    for splits in (0, 1):
        for mode in ("rtne", "rtz"):
            o = attn_fwd_bf16(q, k, v, layout="bshd", round_mode=mode, kv_splits=splits)
            torch.cuda.synchronize()
            got = wl.bits(o.cpu()).reshape(Sq, H, 128)
            assert np.array_equal(got, expect), (splits, mode, int((got != expect).sum()))

