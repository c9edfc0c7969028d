"""GPU parity of the align-free path (fused_moe_lora_naive) through the C ABI.

Against the CPU oracle: |gpu - oracle| <= 1e-2 * (1 + |oracle|) elementwise,
rows of pairs in no slot bit-identical to the input.  Against the sorted
path (moe_lora_align + fused_moe_lora) with the same variant and block_m:
bit-identical, since both hand the same blocks to the same kernel.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import moe_lora_adapter_amd as mla  # noqa: E402
from moe_lora_adapter_amd import synth  # noqa: E402
import gpu_helpers as gh  # noqa: E402

DECODE = ["tiny"] + [f"oss20b_decode_w13_a{a}" for a in range(1, 7)] + \
    ["oss120b_decode_w13", "oss120b_decode_w2"]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def _ref(orc, c):
    s = c.shape
    return orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                     c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)


def _variants(s, block_m):
    """The variants the align-free path takes for these sizes (MFMA needs
    r % 8 == 0 and blocks of at least 16 pairs)."""
    ok = s.r % 8 == 0 and block_m >= 16
    return ["valu"] + (["mfma"] if ok else [])


def _check(orc, c, dc, block_m, what, variant="auto", ref=None):
    s = c.shape
    y = dc.naive(block_m=block_m, variant=variant)
    got = gh.bf16_host_f64(y).reshape(s.numel, s.N)
    gh.assert_fused_close(got, _ref(orc, c) if ref is None else ref, f"{what}/{variant}")
    base = gh.bf16_host_f64(dc.y_in).reshape(s.numel, s.N)
    inval = ~gh.valid_pairs(c)
    assert np.array_equal(got[inval], base[inval]), f"{what}: rows of unmapped pairs changed"
    if block_m in (16, 32, 64, 128):
        dc.s = s.replace(block_m=block_m)
        ys = dc.fused(variant=variant)
        dc.s = s
        assert torch.equal(y.view(torch.int16), ys.view(torch.int16)), \
            f"{what}/{variant}: differs from the sorted path"
    return y


@pytest.mark.parametrize("dist", ["literal", "stress"])
@pytest.mark.parametrize("name", DECODE)
def test_naive_decode_workloads(orc, name, dist):
    s = synth.shape(name, dist=dist)
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    ref = _ref(orc, c)
    for bm in (s.block_m, 1):
        for v in ["auto"] + _variants(s, bm):
            _log(f"naive {name} {dist} block_m={bm} {v}")
            _check(orc, c, dc, bm, f"{name}/{dist}/B{bm}", v, ref)


NAIVE_EDGE = [
    # every block size, both kernels (r = 64: stream; r = 8: register batches)
    dict(K=256, Ns=136, r=64, block_m=2, M=48, E=3, topk=2, L=2, active=2),
    dict(K=256, Ns=136, r=8, block_m=4, M=48, E=3, topk=2, L=2, active=2),
    dict(K=200, Ns=72, r=32, block_m=8, M=40, E=2, topk=2, L=1, active=1, p_neg=0.0),
    dict(K=200, Ns=72, r=128, block_m=32, M=40, E=2, topk=2, L=1, active=1, p_neg=0.0),
    dict(K=136, Ns=64, r=16, block_m=64, M=100, E=2, topk=1, L=1, active=1, p_neg=0.0),
    dict(K=136, Ns=64, r=5, block_m=128, M=300, E=2, topk=1, L=1, active=1, p_neg=0.0),
    # the most pairs: one group of 1024 (64 blocks of 16), and up to 1024 groups
    # (L * E = 8192, the largest key space: 13-bit keys, a full hash table)
    dict(K=64, Ns=64, r=32, block_m=16, M=1024, E=1, topk=1, L=1, active=1, p_neg=0.0),
    dict(K=64, Ns=64, r=16, block_m=16, M=1024, E=1024, topk=1, L=8, active=8, p_neg=0.1),
    # 2^20 and 65536 (slot, expert) keys: the align in passes over slot ranges,
    # 20- and 16-bit keys in the grouping
    # K = 3072 (the eight-row build option's largest), 17- and 21-row groups
    dict(K=3072, Ns=520, r=64, block_m=16, M=38, E=2, topk=1, L=1, active=1, p_neg=0.0),
    # (K, Ns and r small: the weights of every slot are drawn, zero for inactive ones)
    dict(K=8, Ns=8, r=2, block_m=16, M=256, E=1024, topk=2, L=1024, active=40, p_neg=0.1),
    dict(K=8, Ns=16, r=4, block_m=16, M=128, E=1024, topk=4, L=64, active=64, p_neg=0.1),
    dict(K=64, Ns=64, r=64, block_m=1, M=256, E=64, topk=4, L=4, active=4, p_neg=0.1),
    # just past one wavefront of pairs, and a dense decode batch (MFMA by AUTO)
    dict(K=128, Ns=64, r=32, block_m=16, M=65, E=4, topk=1, L=2, active=2, p_neg=0.1),
    dict(K=256, Ns=192, r=16, block_m=32, M=200, E=1, topk=1, L=3, active=3, p_neg=0.0),
    # L * E = 1: zero key bits
    dict(K=72, Ns=40, r=24, block_m=16, M=30, E=1, topk=1, L=1, active=1, p_neg=0.3),
    # keys whose bits are all ones (L * E a power of two) next to invalid pairs
    dict(K=96, Ns=48, r=32, block_m=16, M=64, E=4, topk=2, L=2, active=2, p_neg=0.3),
    # w2 style: X per pair and routed weights; three slices
    dict(K=136, Ns=64, r=56, block_m=16, M=50, E=3, topk=2, L=2, active=2, x_per_pair=True,
         mul=True),
    dict(K=1032, Ns=136, r=64, block_m=16, S=3, M=20, E=8, topk=2, L=3, active=3),
    # overwrite instead of add
    dict(K=256, Ns=128, r=64, block_m=16, M=16, E=8, topk=4, L=2, active=2, add=False),
    # K beyond the stream kernel's X staging: register batches at r = 64
    dict(K=4104, Ns=136, r=64, block_m=16, M=24, E=2, topk=2, L=2, active=2),
]


@pytest.mark.parametrize("i", range(len(NAIVE_EDGE)))
def test_naive_edge_shapes(orc, i):
    s = synth.shape("tiny", dist="stress", seed=9500 + i, **NAIVE_EDGE[i])
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    ref = _ref(orc, c)
    for v in _variants(s, s.block_m):
        _log(f"naive edge {i} {NAIVE_EDGE[i]} {v}")
        _check(orc, c, dc, s.block_m, f"edge {i}", v, ref)


def test_naive_out_of_range_ids_and_duplicates(orc):
    s = synth.shape("tiny", dist="stress", seed=9601, M=40, E=6, topk=4, L=3, active=3,
                    r=32, K=128, Ns=64)
    c = synth.draw(s)
    c.token_lora_mapping[::5] = -2          # below -1
    c.token_lora_mapping[1::7] = s.L        # one past the last slot
    c.topk_ids[::4, 2] = -1
    c.topk_ids[1::6, 0] = s.E
    c.topk_ids[:, 3] = c.topk_ids[:, 1]     # the same expert twice in a token
    dc = gh.DeviceCase(c)
    ref = _ref(orc, c)
    for bm in (1, 16):
        for v in _variants(s, bm):
            _log(f"naive out-of-range ids block_m={bm} {v}")
            _check(orc, c, dc, bm, f"out-of-range/B{bm}", v, ref)


def test_naive_no_valid_pair_and_empty_batch():
    s = synth.shape("tiny", p_neg=1.0, r=64, K=256, Ns=128)
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    for bm in (1, 16):
        for v in _variants(s, bm):
            y = dc.naive(block_m=bm, variant=v)
            assert torch.equal(y.view(torch.int16), dc.y_in.view(torch.int16))
    d0 = gh.DeviceCase(synth.draw(synth.shape("tiny", M=0)))
    mla.fused_moe_lora_naive(d0.x, d0.a, d0.b, d0.topk_ids, d0.mapping, d0.w, d0.y_in,
                             mul_routed_weight=True, add_inputs=True)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["tiny", "oss20b_decode_w13_a6", "oss120b_decode_w2"])
def test_naive_metamorphic(name):
    s = synth.shape(name, dist="stress")
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    valid = torch.from_numpy(gh.valid_pairs(c)).to(gh.DEV)
    _log(f"naive metamorphic {name}")
    y = dc.naive(add=True, a=torch.zeros_like(dc.a))
    assert torch.equal(y.view(torch.int16), dc.y_in.view(torch.int16)), "zero adapter, add"
    d1 = dc.naive(add=False).view(s.numel, s.N)[valid].float()
    d2 = dc.naive(add=False, b=dc.b * 2).view(s.numel, s.N)[valid].float()
    assert torch.equal(d2, 2 * d1), "B -> 2B"
    ya, yb = dc.naive(), dc.naive()
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)), "run to run"
    # on the stream kernel a row's arithmetic does not depend on the other
    # rows of its block, so the block size changes nothing; the register-batch
    # kernel folds lane partials in an order set by its 2- or 4-row groups
    y1, y16 = dc.naive(block_m=1, variant="valu"), dc.naive(block_m=16, variant="valu")
    kernel = mla.fused_kernel_name(s.M, s.topk, s.K, s.Ns, s.S, s.E, s.L, s.r, s.block_m,
                                   s.x_per_pair, "valu")
    if kernel == "fused_stream_kernel":
        assert torch.equal(y1.view(torch.int16), y16.view(torch.int16)), "block_m 1 vs 16"
    else:
        gh.assert_fused_close(gh.bf16_host_f64(y1), gh.bf16_host_f64(y16), "block_m 1 vs 16")


@pytest.mark.parametrize("name", ["tiny", "oss20b_decode_w13_a6"])
def test_naive_graph_replay_matches_eager(name):
    s = synth.shape(name, dist="stress")
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    eager = dc.naive()
    y = dc.y_in.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dc.naive(y=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mla.fused_moe_lora_naive(dc.x, dc.a, dc.b, dc.topk_ids, dc.mapping, dc.w, y,
                                 mul_routed_weight=s.mul, add_inputs=s.add,
                                 block_m=s.block_m, x_per_pair=s.x_per_pair)
    for rep in range(3):
        _log(f"naive graph replay {name} {rep}")
        y.copy_(dc.y_in)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
