"""GPU parity of the K split of the decode kernels (fused_moe_lora_ws) through the C ABI.

The workgroups that share a (block, slice) -- one per column range of the
expand -- each multiply an equal share of A's K range and meet through the
workspace, adding the partial rank vectors in the same order (the decode
stream kernel, ranks 32, 64, 128).  Checked here:

- against the CPU oracle with fused_moe_lora's tolerance, rows of pairs in
  no slot untouched;
- the precision bound of the rank vector (hi/lo split) still holds;
- peer_wait = 0, where every workgroup computes every partial itself from A
  in memory (the path taken when a peer is late), gives the same bytes as
  the exchange: published and recomputed partials are the same bits;
- a workspace reused after calls on other inputs gives the same bytes as a
  fresh zero-filled one (the area's layout depends on its size alone and
  every stale word carries an older tag);
- one workspace reused by calls of different sizes (M = 16, 15, 16, and
  ranks 64, 32, 128), each result equal bit for bit to peer_wait = 0 on
  that workspace;
- one captured graph, replayed with the slot mapping rewritten in place
  between replays, matches eager calls bit for bit;
- a launch bounded by max_active_loras equals the one bounded by L;
- the workspace checks of the entry point.
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

DECODE = [f"oss20b_decode_w13_a{a}" for a in (1, 2, 3, 6)]

# shapes the stream kernel takes (r in {32, 64, 128}, 4 K <= 16384), with
# K stage counts that do not divide by the split count, fewer K stages than
# workgroups sharing a block (empty shares), blocks of several 4-row passes,
# per-pair X, routed weights and overwrite
EDGE = [
    dict(K=264, Ns=2880, r=64, block_m=16, M=16, E=4, topk=2, L=2, active=2),
    dict(K=2880, Ns=1032, r=32, block_m=16, M=24, E=3, topk=2, L=2, active=2),
    dict(K=1000, Ns=4096, r=128, block_m=16, M=12, E=4, topk=2, L=1, active=1),
    dict(K=4096, Ns=2048, r=64, block_m=32, M=48, E=2, topk=2, L=2, active=2, p_neg=0.0),
    dict(K=256, Ns=2184, r=64, block_m=16, M=64, E=2, topk=1, L=1, active=1, p_neg=0.0),
    dict(K=2880, Ns=2880, r=64, block_m=16, M=16, E=8, topk=4, L=2, active=2, x_per_pair=True,
         mul=True),
    dict(K=136, Ns=1544, r=32, block_m=64, M=40, E=2, topk=2, L=3, active=3, add=False),
    dict(K=8, Ns=776, r=128, block_m=16, M=8, E=2, topk=2, L=1, active=1),
]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def _ksplit_kernel(s):
    return mla.fused_kernel_name(s.M, s.topk, s.K, s.Ns, s.S, s.E, s.L, s.r, s.block_m,
                                 s.x_per_pair, "valu") == "fused_stream_kernel"


def _ws(dc, align, ws, y=None, peer_wait=-1, add=None, stream=None, max_active=None):
    s = dc.s
    y = dc.y_in.clone() if y is None else y
    mla.fused_moe_lora_ws(dc.x, dc.a, dc.b, align, dc.w, y, mul_routed_weight=s.mul,
                          add_inputs=s.add if add is None else add, workspace=ws,
                          x_per_pair=s.x_per_pair, variant="valu", peer_wait=peer_wait,
                          max_active_loras=max_active, stream=stream)
    return y


def _workspace(s):
    return mla.alloc_fused_workspace(s.M, s.topk, s.K, s.Ns, s.S, s.E, s.L, s.r, s.block_m,
                                     gh.DEV, x_per_pair=s.x_per_pair, variant="valu")


def _check_case(orc, s, what):
    assert _ksplit_kernel(s), f"{what}: the stream kernel does not take this shape"
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    al = dc.align()
    ws = _workspace(s)
    y1 = _ws(dc, al, ws)
    # the same workspace after a call on other inputs (x scaled: other partials)
    x_keep = dc.x
    dc.x = (x_keep.float() * -3.0).to(torch.bfloat16)
    _ws(dc, al, ws)
    dc.x = x_keep
    y2 = _ws(dc, al, ws)
    y0 = _ws(dc, al, ws, peer_wait=0)  # every workgroup computes every partial
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), f"{what}: reused workspace"
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16)), \
        f"{what}: exchanged and recomputed partials differ"
    got = gh.bf16_host_f64(y1).reshape(s.numel, s.N)
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)
    gh.assert_fused_close(got, ref, what)
    base = gh.bf16_host_f64(dc.y_in).reshape(s.numel, s.N)
    inval = ~gh.valid_pairs(c)
    assert np.array_equal(got[inval], base[inval]), f"{what}: rows of unmapped pairs changed"


@pytest.mark.parametrize("dist", ["literal", "stress"])
@pytest.mark.parametrize("name", DECODE)
def test_k_split_decode(orc, name, dist):
    s = synth.shape(name, dist=dist)
    _log(f"k-split {name} {dist}")
    _check_case(orc, s, f"{name}/{dist}")


@pytest.mark.parametrize("i", range(len(EDGE)))
def test_k_split_edge_shapes(orc, i):
    s = synth.shape("tiny", dist="stress", seed=9800 + i, **EDGE[i])
    _log(f"k-split edge {i} {EDGE[i]}")
    _check_case(orc, s, f"edge {i}")


@pytest.mark.parametrize("name", ["oss20b_decode_w13_a6", "oss20b_decode_w13_a3"])
def test_k_split_max_active_loras(orc, name):
    """A launch bounded by the active-slot count uses fewer exchange slots of
    the same workspace and writes the same bits as the one bounded by L."""
    s = synth.shape(name, dist="stress")
    c = synth.draw(s)
    m = c.token_lora_mapping
    keep = (c.active_slots[0], c.active_slots[-1])   # two of the filled slots only
    c.token_lora_mapping = np.where(m >= 0, np.where(m % 2 == 0, keep[0], keep[1]),
                                    m).astype(m.dtype)
    dc = gh.DeviceCase(c)
    al = dc.align()
    ws = _workspace(s)
    torch.cuda.synchronize()
    nact = int(al.num_active_loras.item())
    _log(f"k-split max_active {name} nact={nact}")
    full = _ws(dc, al, ws)
    bound = _ws(dc, al, ws, max_active=nact)
    none = _ws(dc, al, ws, max_active=0)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), bound.view(torch.int16))
    assert torch.equal(none.view(torch.int16), dc.y_in.view(torch.int16))
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)
    gh.assert_fused_close(gh.bf16_host_f64(bound).reshape(s.numel, s.N), ref, name)


def test_k_split_rank_vector_precision(orc):
    """With add_inputs = 0, Y differs from the exact delta by the output's bf16
    rounding and a small absolute term, as for fused_moe_lora."""
    s = synth.shape("oss20b_decode_w13_a6", dist="stress", add=False)
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    v = gh.valid_pairs(c)
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)[v]
    y = _ws(dc, dc.align(), _workspace(s))
    torch.cuda.synchronize()
    got = gh.bf16_host_f64(y).reshape(s.numel, s.N)[v]
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * np.sqrt(np.mean(ref ** 2))
    assert (err <= bound).all(), f"worst err {np.max(err - bound):.3e} above bound"


def test_k_split_one_graph_across_active_counts(orc):
    s = synth.shape("oss20b_decode_w13_a6", dist="stress")
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    rng = np.random.default_rng(4343)
    a = rng.standard_normal((s.S, s.L, s.E, s.r, s.K), dtype=np.float32) / np.sqrt(s.K)
    b = rng.standard_normal((s.S, s.L, s.E, s.Ns, s.r), dtype=np.float32) / np.sqrt(s.r)
    dc.a = torch.from_numpy(a).to(gh.DEV).to(torch.bfloat16)
    dc.b = torch.from_numpy(b).to(gh.DEV).to(torch.bfloat16)
    mapping = dc.mapping
    al = mla.alloc_align_output(s.M, s.topk, s.E, s.L, s.block_m, gh.DEV)
    aws = torch.empty(max(16, mla.align_workspace_size(s.M, s.topk, s.E, s.L, s.block_m)),
                      dtype=torch.uint8, device=gh.DEV)
    ws = _workspace(s)
    y = dc.y_in.clone()

    def call():
        mla.moe_lora_align(dc.topk_ids, mapping, s.E, s.L, s.block_m, out=al, workspace=aws)
        _ws(dc, al, ws, y=y)

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
        _log(f"k-split graph: {n_active} active slots")
        mapping.copy_(torch.from_numpy(m))
        y.copy_(dc.y_in)
        torch.cuda.synchronize()
        call()
        torch.cuda.synchronize()
        eager = y.clone()
        for rep in range(3):
            y.copy_(dc.y_in)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), \
                f"{n_active} active, replay {rep}"
        ref = orc.fused(c.x, a_host, b_host, c.topk_ids, m, c.topk_weights, c.y_in, s.mul, s.add,
                        x_per_pair=s.x_per_pair)
        gh.assert_fused_close(gh.bf16_host_f64(y).reshape(s.numel, s.N), ref,
                              f"graph/{n_active}")


def test_k_split_workspace_checks():
    s = synth.shape("oss20b_decode_w13_a6")
    dc = gh.DeviceCase(synth.draw(s))
    al = dc.align()
    need = mla.fused_moe_lora_workspace_bytes(s.M, s.topk, s.K, s.Ns, s.S, s.E, s.L, s.r,
                                              s.block_m, s.x_per_pair, "valu")
    assert need > 0
    small = torch.zeros(need - 16, dtype=torch.uint8, device=gh.DEV)
    with pytest.raises(mla.MoeLoraError) as ei:
        _ws(dc, al, small)
    assert ei.value.status == mla.ERR_WORKSPACE
    with pytest.raises(mla.MoeLoraError) as ei:
        _ws(dc, al, None)
    assert ei.value.status == mla.ERR_WORKSPACE
    # misaligned
    big = torch.zeros(need + 64, dtype=torch.uint8, device=gh.DEV)
    with pytest.raises(mla.MoeLoraError) as ei:
        _ws(dc, al, big[4:])
    assert ei.value.status == mla.ERR_WORKSPACE
    # a shape whose kernel needs none (an odd rank: register batches): the
    # workspace may be absent
    t = synth.shape("tiny", r=5)
    assert mla.fused_moe_lora_workspace_bytes(t.M, t.topk, t.K, t.Ns, t.S, t.E, t.L, t.r,
                                              t.block_m, t.x_per_pair, "valu") == 0
    dt = gh.DeviceCase(synth.draw(t))
    y = _ws(dt, dt.align(), None)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), dt.fused(variant="valu").view(torch.int16))


@pytest.mark.parametrize("name,calls", [
    ("oss20b_decode_w13_a6", (dict(M=16), dict(M=15), dict(M=16))),
    ("oss20b_decode_w13_a3", (dict(M=16, r=64), dict(M=12, r=32), dict(M=16, r=128)))])
def test_k_split_workspace_reused_across_sizes(orc, name, calls):
    """One workspace, sized for the largest call, serves calls of other sizes
    in a row: each result equals peer_wait = 0 (every partial computed in
    place) bit for bit, and the oracle within tolerance."""
    shapes = [synth.shape(name, dist="stress", seed=5000 + 17 * i, **kw) for i, kw in enumerate(calls)]
    need_max = max(mla.fused_moe_lora_workspace_bytes(t.M, t.topk, t.K, t.Ns, t.S, t.E, t.L, t.r,
                                                      t.block_m, t.x_per_pair, "valu") for t in shapes)
    ws = torch.zeros(need_max, dtype=torch.uint8, device=gh.DEV)
    for i, s in enumerate(shapes):
        M = s.M
        assert _ksplit_kernel(s)
        need = mla.fused_moe_lora_workspace_bytes(s.M, s.topk, s.K, s.Ns, s.S, s.E, s.L, s.r,
                                                  s.block_m, s.x_per_pair, "valu")
        assert 0 < need <= ws.numel()
        _log(f"k-split workspace reuse {name} call {i}: M={M} r={s.r}")
        c = synth.draw(s)
        dc = gh.DeviceCase(c)
        al = dc.align()
        y = _ws(dc, al, ws)
        y0 = _ws(dc, al, ws, peer_wait=0)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), f"{name} M={M} r={s.r}"
        ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping,
                        c.topk_weights, c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)
        gh.assert_fused_close(gh.bf16_host_f64(y).reshape(s.numel, s.N), ref, f"{name} M={M}")
