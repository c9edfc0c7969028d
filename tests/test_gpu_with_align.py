"""GPU parity of fused_moe_lora_with_align (align + fused in one launch) through the C ABI.

The align outputs come from one extra workgroup running the one-wavefront
align beside the fused workgroups, which form their blocks on chip.  Checked:
the align outputs bit for bit against the oracle and against moe_lora_align;
y bit for bit against fused_moe_lora_naive with the same block_m (the same
fused work) and within tolerance of the oracle; rows of pairs in no slot
untouched; the empty batch; one captured graph across active-slot counts.
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

DECODE = ["tiny"] + [f"oss20b_decode_w13_a{a}" for a in (1, 3, 6)] + \
    ["oss120b_decode_w13", "oss120b_decode_w2"]

EDGE = [
    # 64 pairs, 64 slots (both limits), many slots inactive
    dict(M=32, topk=2, E=4, L=64, active=40, K=64, Ns=64, r=16, block_m=16),
    # one token, block sizes above the rows present
    dict(M=1, topk=4, E=8, L=2, active=2, K=256, Ns=128, r=32, block_m=64),
    # routed weights, per-pair X, overwrite
    dict(M=16, topk=4, E=8, L=2, active=2, K=264, Ns=776, r=64, block_m=16, x_per_pair=True,
         mul=True, add=False),
    # the MFMA kernel's align-free instantiation (r a multiple of 8, rank 128)
    dict(M=16, topk=4, E=8, L=1, active=1, K=512, Ns=256, r=128, block_m=32, p_neg=0.0),
]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def _with_align(dc, variant="auto", y=None):
    s = dc.s
    y = dc.y_in.clone() if y is None else y
    out = mla.fused_moe_lora_with_align(dc.topk_ids, dc.mapping, dc.x, dc.a, dc.b, dc.w, y,
                                        E=s.E, L=s.L, block_m=s.block_m,
                                        mul_routed_weight=s.mul, add_inputs=s.add,
                                        x_per_pair=s.x_per_pair, variant=variant)
    torch.cuda.synchronize()
    return out, y


def _check(orc, s, what, variant="auto"):
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    out, y = _with_align(dc, variant)
    ref_al = orc.align(c.topk_ids, c.token_lora_mapping, s.E, s.L, s.block_m)
    got_al = gh.align_to_host(out)
    gh.assert_align_equal(got_al, ref_al, s.block_m)
    sep = gh.align_to_host(dc.align())  # the align kernel on the same inputs
    gh.assert_align_equal(got_al, sep, s.block_m)
    y_naive = dc.naive(block_m=s.block_m, variant=variant)
    assert torch.equal(y.view(torch.int16), y_naive.view(torch.int16)), f"{what}: y vs align-free"
    got = gh.bf16_host_f64(y).reshape(s.numel, s.N)
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)
    gh.assert_fused_close(got, ref, what)
    base = gh.bf16_host_f64(dc.y_in).reshape(s.numel, s.N)
    inval = ~gh.valid_pairs(c)
    assert np.array_equal(got[inval], base[inval]), f"{what}: rows of unmapped pairs changed"


@pytest.mark.parametrize("dist", ["literal", "stress"])
@pytest.mark.parametrize("name", DECODE)
def test_with_align_decode(orc, name, dist):
    s = synth.shape(name, dist=dist)
    _log(f"with-align {name} {dist}")
    _check(orc, s, f"{name}/{dist}")


@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_with_align_variants(orc, variant):
    s = synth.shape("oss20b_decode_w13_a6", dist="stress")
    _log(f"with-align a6 {variant}")
    _check(orc, s, f"a6/{variant}", variant=variant)


@pytest.mark.parametrize("i", range(len(EDGE)))
def test_with_align_edge_shapes(orc, i):
    s = synth.shape("tiny", dist="stress", seed=9900 + i, **EDGE[i])
    _log(f"with-align edge {i} {EDGE[i]}")
    _check(orc, s, f"edge {i}")


def test_with_align_empty_batch(orc):
    s = synth.shape("tiny", M=0)
    dc = gh.DeviceCase(synth.draw(s))
    out = mla.alloc_align_output(0, s.topk, s.E, s.L, s.block_m, gh.DEV)
    out.num_tokens_post_padded.fill_(-5)
    out.lora_ids.fill_(7)
    mla.fused_moe_lora_with_align(dc.topk_ids, dc.mapping, dc.x, dc.a, dc.b, dc.w, dc.y_in,
                                  E=s.E, L=s.L, block_m=s.block_m, mul_routed_weight=False,
                                  add_inputs=True, out=out)
    torch.cuda.synchronize()
    assert (out.num_tokens_post_padded.cpu().numpy() == 0).all()
    assert (out.lora_ids.cpu().numpy() == -1).all()
    assert int(out.num_active_loras.cpu().numpy()[0]) == 0


def test_with_align_one_graph_across_active_counts(orc):
    s = synth.shape("oss20b_decode_w13_a6", dist="stress")
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    rng = np.random.default_rng(4545)
    a = rng.standard_normal((s.S, s.L, s.E, s.r, s.K), dtype=np.float32) / np.sqrt(s.K)
    b = rng.standard_normal((s.S, s.L, s.E, s.Ns, s.r), dtype=np.float32) / np.sqrt(s.r)
    dc.a = torch.from_numpy(a).to(gh.DEV).to(torch.bfloat16)
    dc.b = torch.from_numpy(b).to(gh.DEV).to(torch.bfloat16)
    out = mla.alloc_align_output(s.M, s.topk, s.E, s.L, s.block_m, gh.DEV)
    y = dc.y_in.clone()

    def call():
        mla.fused_moe_lora_with_align(dc.topk_ids, dc.mapping, dc.x, dc.a, dc.b, dc.w, y,
                                      E=s.E, L=s.L, block_m=s.block_m, mul_routed_weight=s.mul,
                                      add_inputs=s.add, out=out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    a_host = dc.a.view(torch.int16).cpu().numpy().view(np.uint16)
    b_host = dc.b.view(torch.int16).cpu().numpy().view(np.uint16)
    for n_active in [1, 3, s.L]:
        slots = np.sort(rng.choice(s.L, size=n_active, replace=False))
        m = slots[rng.integers(0, n_active, size=s.M)].astype(np.int32)
        m[rng.random(s.M) < 0.1] = -1
        _log(f"with-align graph: {n_active} active slots")
        dc.mapping.copy_(torch.from_numpy(m))
        y.copy_(dc.y_in)
        torch.cuda.synchronize()
        call()
        torch.cuda.synchronize()
        eager = y.clone()
        eager_al = gh.align_to_host(out)
        for rep in range(3):
            y.copy_(dc.y_in)
            out.num_tokens_post_padded.fill_(-3)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), \
                f"{n_active} active, replay {rep}"
            gh.assert_align_equal(gh.align_to_host(out), eager_al, s.block_m)
        ref_al = orc.align(c.topk_ids, m, s.E, s.L, s.block_m)
        gh.assert_align_equal(eager_al, ref_al, s.block_m)
        ref = orc.fused(c.x, a_host, b_host, c.topk_ids, m, c.topk_weights, c.y_in, s.mul, s.add,
                        x_per_pair=s.x_per_pair)
        gh.assert_fused_close(gh.bf16_host_f64(y).reshape(s.numel, s.N), ref, f"graph/{n_active}")


@pytest.mark.parametrize("variant", ["valu", "auto"])
def test_with_align_no_spare_workgroup(orc, variant):
    """64 pairs on 64 distinct experts over 4 slices: 256 (block, slice) units,
    one per workgroup of a 256-workgroup grid, so no workgroup is left spare and
    workgroup 0 runs the align before its own unit."""
    s = synth.shape("tiny", dist="stress", seed=9950, M=16, topk=4, E=64, L=1, active=1,
                    S=4, K=256, Ns=256, r=64, block_m=16, p_neg=0.0)
    c = synth.draw(s)
    c.topk_ids[:] = np.arange(s.numel, dtype=np.int32).reshape(s.M, s.topk)
    c.token_lora_mapping[:] = 0
    _log(f"with-align, no spare workgroup, {variant}")
    dc = gh.DeviceCase(c)
    out, y = _with_align(dc, variant)
    ref_al = orc.align(c.topk_ids, c.token_lora_mapping, s.E, s.L, s.block_m)
    gh.assert_align_equal(gh.align_to_host(out), ref_al, s.block_m)
    assert int(out.num_tokens_post_padded.cpu().numpy()[0]) == 64 * s.block_m
    y_naive = dc.naive(block_m=s.block_m, variant=variant)
    assert torch.equal(y.view(torch.int16), y_naive.view(torch.int16))
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)
    gh.assert_fused_close(gh.bf16_host_f64(y).reshape(s.numel, s.N), ref, f"no spare/{variant}")
