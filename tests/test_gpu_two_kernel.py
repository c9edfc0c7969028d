"""GPU parity of the two-kernel path (fused_moe_lora_two_kernel) through the C ABI.

Against the CPU oracle: |gpu - oracle| <= 1e-2 * (1 + |oracle|) elementwise,
rows of pairs in no slot bit-identical to the input; ranks up to 512 (past the
fused kernels' 128); run-to-run bit identity; with add_inputs = 0 the output
differs from the exact delta by output rounding only.
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

SMALL = ["tiny"] + [f"oss20b_decode_w13_a{a}" for a in (1, 3, 6)] + \
    ["oss120b_decode_w13", "oss120b_decode_w2"]
LARGE = ["oss120b_prefill_w13", "qwen3_prefill", "dense_o"]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def _two(dc, align=None, y=None, add=None, max_active=None):
    s = dc.s
    align = align if align is not None else dc.align()
    y = dc.y_in.clone() if y is None else y
    mla.fused_moe_lora_two_kernel(dc.x, dc.a, dc.b, align, dc.w, y, mul_routed_weight=s.mul,
                                  add_inputs=s.add if add is None else add,
                                  x_per_pair=s.x_per_pair, max_active_loras=max_active)
    torch.cuda.synchronize()
    return y


def _full(orc, s, what):
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    y = _two(dc)
    got = gh.bf16_host_f64(y).reshape(s.numel, s.N)
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)
    gh.assert_fused_close(got, ref, what)
    base = gh.bf16_host_f64(dc.y_in).reshape(s.numel, s.N)
    inval = ~gh.valid_pairs(c)
    assert np.array_equal(got[inval], base[inval]), f"{what}: rows of unmapped pairs changed"
    return c, dc, y, ref


@pytest.mark.parametrize("dist", ["literal", "stress"])
@pytest.mark.parametrize("name", SMALL)
def test_two_kernel_small_full(orc, name, dist):
    s = synth.shape(name, dist=dist)
    _log(f"two-kernel {name} {dist}")
    _full(orc, s, f"{name}/{dist}")


TWO_EDGE = [
    # ranks past the fused kernels' limit, with rank and K tails
    dict(K=264, Ns=136, r=256, block_m=16, M=40, E=3, topk=2, L=2, active=2),
    dict(K=200, Ns=72, r=512, block_m=16, M=24, E=2, topk=2, L=1, active=1, p_neg=0.0),
    dict(K=136, Ns=64, r=200, block_m=64, M=150, E=2, topk=1, L=1, active=1, p_neg=0.0),
    dict(K=72, Ns=40, r=384, block_m=32, M=40, E=2, topk=2, L=2, active=2, mul=True),
    dict(K=512, Ns=256, r=129, block_m=128, M=300, E=2, topk=1, L=1, active=1, p_neg=0.0),
    # ranks the fused kernels take too, odd ones included
    dict(K=264, Ns=776, r=5, block_m=32),
    dict(K=8, Ns=8, r=1, block_m=16),
    dict(K=1032, Ns=136, r=64, block_m=16, S=3),
    dict(K=256, Ns=128, r=96, block_m=64, M=300, E=4, topk=3, x_per_pair=True, mul=True),
    dict(K=4104, Ns=136, r=64, block_m=16, M=24, E=2, topk=2, L=2, active=2),
    dict(K=2880, Ns=4096, r=32, block_m=32, M=48, E=3, topk=2, L=2, active=2, p_neg=0.0),
    dict(K=256, Ns=128, r=128, block_m=16, M=16, E=8, topk=4, L=2, active=2, add=False),
    dict(K=64, Ns=64, r=16, block_m=16, M=70, E=3, L=100, active=70, p_neg=0.1),
]


@pytest.mark.parametrize("i", range(len(TWO_EDGE)))
def test_two_kernel_edge_shapes(orc, i):
    s = synth.shape("tiny", dist="stress", seed=9700 + i, **TWO_EDGE[i])
    _log(f"two-kernel edge {i} {TWO_EDGE[i]}")
    _full(orc, s, f"edge {i}")


def test_two_kernel_max_active_loras(orc):
    """Bounded by the active-slot count: the same bits as bounded by L; 0
    launches nothing."""
    s = synth.shape("tiny", dist="stress", seed=9760, K=264, Ns=136, r=256, M=64, E=4,
                    topk=2, L=6, active=6)
    c = synth.draw(s)
    m = c.token_lora_mapping
    c.token_lora_mapping = np.where(m >= 0, 5 * (m % 2), m).astype(m.dtype)  # slots 0 and 5 of 6
    dc = gh.DeviceCase(c)
    al = dc.align()
    torch.cuda.synchronize()
    nact = int(al.num_active_loras.item())
    full = _two(dc, align=al)
    bound = _two(dc, align=al, max_active=nact)
    assert torch.equal(full.view(torch.int16), bound.view(torch.int16))
    none = _two(dc, align=al, max_active=0)
    assert torch.equal(none.view(torch.int16), dc.y_in.view(torch.int16))
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)
    gh.assert_fused_close(gh.bf16_host_f64(bound).reshape(s.numel, s.N), ref, "max_active")


@pytest.mark.parametrize("dist", ["literal", "stress"])
@pytest.mark.parametrize("name", LARGE)
def test_two_kernel_full_size(orc, name, dist):
    """Every element of Y against the oracle at the configured full sizes."""
    s = synth.shape(name, dist=dist)
    _log(f"two-kernel full-size {name} {dist}: drawing inputs")
    _log(f"two-kernel full-size {name} {dist}")
    _full(orc, s, f"{name}/{dist}")


@pytest.mark.parametrize("name,kw", [("oss20b_decode_w13_a6", {}),
                                     ("tiny", dict(r=512, K=512, Ns=256))])
def test_two_kernel_precision_and_determinism(orc, name, kw):
    s = synth.shape(name, dist="stress", add=False, **kw)
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    v = gh.valid_pairs(c)
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)[v]
    ya, yb = _two(dc), _two(dc)
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)), "run to run"
    got = gh.bf16_host_f64(ya).reshape(s.numel, s.N)[v]
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * np.sqrt(np.mean(ref ** 2))
    assert (err <= bound).all(), f"{name}: worst err {np.max(err - bound):.3e} above bound"


def test_two_kernel_matches_fused_on_literal_inputs(orc):
    """Same function as the one-shot kernels: on the 20b-like decode shape both stay within
    the tolerance of the oracle and of each other."""
    s = synth.shape("oss20b_decode_w13_a6")
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    al = dc.align()
    y1 = gh.bf16_host_f64(dc.fused(align=al, variant="valu"))
    y2 = gh.bf16_host_f64(_two(dc, align=al))
    gh.assert_fused_close(y2.reshape(s.numel, s.N), y1.reshape(s.numel, s.N), "two vs one-shot")


def test_two_kernel_no_valid_pair_and_empty_batch():
    s = synth.shape("tiny", p_neg=1.0, r=256, K=256, Ns=128)
    dc = gh.DeviceCase(synth.draw(s))
    y = _two(dc)
    assert torch.equal(y.view(torch.int16), dc.y_in.view(torch.int16))
    d0 = gh.DeviceCase(synth.draw(synth.shape("tiny", M=0)))
    al = d0.align()
    mla.fused_moe_lora_two_kernel(d0.x, d0.a, d0.b, al, d0.w, d0.y_in, mul_routed_weight=True,
                                  add_inputs=True)
    torch.cuda.synchronize()
