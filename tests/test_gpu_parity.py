"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Align outputs must match bit for bit.  Y must satisfy
|gpu - oracle| <= 1e-2 * (1 + |oracle|) elementwise; rows of pairs in no slot
must be bit-identical to the input.  Every workload, the full-size ones
included, is compared element by element over all of Y.
"""
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from moe_lora_adapter_amd import synth  # noqa: E402
import gpu_helpers as gh  # noqa: E402

SMALL = ["tiny"] + [f"oss20b_decode_w13_a{a}" for a in range(1, 7)] + \
    ["oss120b_decode_w13", "oss120b_decode_w2"]
LARGE = ["oss120b_prefill_w13", "oss120b_prefill_w2", "qwen3_prefill", "dense_qkv", "dense_o"]
ALIGN_ALL = SMALL + LARGE + ["align_stress", "align_stress_neg"]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def _variants(s):
    return ["valu"] + (["mfma"] if _mfma_ok(s) else [])


def _mfma_ok(s):
    import moe_lora_adapter_amd as mla
    import ctypes
    # probe with a zero-sized call: MOE_LORA_ERR_UNSUPPORTED means not available
    rc = mla.lib().fused_moe_lora(ctypes.c_void_p(16), 0, ctypes.c_void_p(16), ctypes.c_void_p(16),
                                  ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16),
                                  s.L, None, 0, 1, 0, s.topk, s.K, s.Ns, s.S, s.E, s.L, s.r,
                                  s.block_m, ctypes.c_void_p(16), 2, None)
    return rc == 0


# ------------------------------------------------------------------ align
@pytest.mark.parametrize("name", ALIGN_ALL)
def test_align_matches_oracle(orc, name):
    s = synth.shape(name)
    _log(f"align parity {name} M={s.M} topk={s.topk} E={s.E} L={s.L} B={s.block_m}")
    c = synth.draw(s, with_tensors=False)
    ref = orc.align(c.topk_ids, c.token_lora_mapping, s.E, s.L, s.block_m)
    gpu = gh.align_to_host(gh.run_align(c.topk_ids, c.token_lora_mapping, s.E, s.L, s.block_m))
    gh.assert_align_equal(gpu, ref, s.block_m)


def _random_align_case(rng):
    M = int(rng.choice([0, 1, 3, 64, 65, 1000, 4095, 4096, 4097, 9000, 20000]))
    topk = int(rng.integers(1, 9))
    E = int(rng.choice([1, 2, 7, 64, 129, 1024]))
    L = int(rng.choice([1, 2, 5, 8, 9, 64, 1024]))
    B = int(rng.choice([16, 32, 64, 128]))
    # bounded output (L rows of capacity) for the oracle; past 8192 keys the
    # library aligns in passes over slot ranges
    while L > 1 and L * (M * topk + min(E, M * topk) * (B - 1)) > 1 << 23:
        L //= 2
    topk_ids = rng.integers(-1, E + 1, size=(M, topk)).astype(np.int32)
    mapping = rng.integers(-2, L + 1, size=M).astype(np.int32)
    return topk_ids, mapping, E, L, B


@pytest.mark.parametrize("seed", range(16))
def test_align_edge_cases(orc, seed):
    rng = np.random.default_rng(100 + seed)
    topk_ids, mapping, E, L, B = _random_align_case(rng)
    _log(f"align edge seed={seed} M={len(mapping)} topk={topk_ids.shape[1]} E={E} L={L} B={B}")
    ref = orc.align(topk_ids, mapping, E, L, B)
    gpu = gh.align_to_host(gh.run_align(topk_ids, mapping, E, L, B))
    gh.assert_align_equal(gpu, ref, B)


def test_align_max_experts_and_many_slots(orc):
    rng = np.random.default_rng(7)
    for (M, topk, E, L, B) in ((3000, 8, 1024, 8, 64), (500, 2, 2, 1024, 16),
                               (40000, 4, 8, 1024, 128)):
        _log(f"align limits M={M} topk={topk} E={E} L={L} B={B}")
        topk_ids = rng.integers(0, E, size=(M, topk)).astype(np.int32)
        mapping = rng.integers(-1, L, size=M).astype(np.int32)
        ref = orc.align(topk_ids, mapping, E, L, B)
        gpu = gh.align_to_host(gh.run_align(topk_ids, mapping, E, L, B))
        gh.assert_align_equal(gpu, ref, B)


@pytest.mark.parametrize("M,topk,E,L,B,lo", [
    (256, 8, 256, 64, 64, 0),      # 16384 keys: two passes of 32 slots (tile path)
    (256, 8, 256, 64, 64, 40),     # every pair in the second pass's slots
    (9000, 2, 100, 100, 32, 0),    # 10000 keys: passes of 81 and 19 slots
    (512, 4, 1024, 1024, 16, 0),   # 2^20 keys: 128 passes of 8 slots
    (512, 4, 1024, 1024, 16, 1000),
    (0, 4, 1024, 64, 16, 0),       # no pairs: every slot empty, no active slot
])
@pytest.mark.parametrize("noalloc", [False, True])
def test_align_key_spaces_in_passes(orc, M, topk, E, L, B, lo, noalloc):
    """Key spaces beyond one pass's 8192 (slot, expert) keys, up to 2^20:
    bit-exact against the oracle, lora_ids and num_active_loras included,
    through moe_lora_align and moe_lora_align_noalloc."""
    rng = np.random.default_rng(M + 7 * L + lo)
    topk_ids = rng.integers(-1, E + 1, size=(M, topk)).astype(np.int32)
    topk_ids[::4] = rng.integers(0, max(1, E // 8), size=topk_ids[::4].shape)  # repeated keys
    mapping = rng.integers(lo - 1, L + 1, size=M).astype(np.int32)
    _log(f"align passes M={M} topk={topk} E={E} L={L} B={B} slots from {lo} noalloc={noalloc}")
    ref = orc.align(topk_ids, mapping, E, L, B)
    if noalloc:
        import moe_lora_adapter_amd as mla
        out = mla.alloc_align_output(M, topk, E, L, B, gh.DEV)
        mla.moe_lora_align_noalloc(gh.i32_dev(topk_ids), gh.i32_dev(mapping), E, L, B, out=out)
        torch.cuda.synchronize()
    else:
        out = gh.run_align(topk_ids, mapping, E, L, B)
    gh.assert_align_equal(gh.align_to_host(out), ref, B)


@pytest.mark.parametrize("M,topk,E,L,B", [
    (64, 1, 7, 3, 16), (16, 4, 32, 6, 16), (21, 3, 5, 64, 32), (63, 1, 2, 1, 128),
    (8, 8, 1024, 8, 64), (1, 1, 1, 1, 16), (0, 4, 32, 6, 16),
    # just past the one-wavefront path: 65 pairs, 65 slots
    (65, 1, 7, 3, 16), (16, 4, 32, 65, 16)])
def test_align_one_wavefront_boundaries(orc, M, topk, E, L, B):
    rng = np.random.default_rng(M * 131 + L)
    topk_ids = rng.integers(-1, E + 1, size=(M, topk)).astype(np.int32)
    topk_ids[::3] = rng.integers(0, max(1, E // 4), size=topk_ids[::3].shape)  # repeated keys
    mapping = rng.integers(-2, L + 1, size=M).astype(np.int32)
    _log(f"align boundary M={M} topk={topk} E={E} L={L} B={B}")
    ref = orc.align(topk_ids, mapping, E, L, B)
    gpu = gh.align_to_host(gh.run_align(topk_ids, mapping, E, L, B))
    gh.assert_align_equal(gpu, ref, B)


def test_align_deterministic():
    s = synth.shape("align_stress")
    c = synth.draw(s, with_tensors=False)
    a = gh.align_to_host(gh.run_align(c.topk_ids, c.token_lora_mapping, s.E, s.L, s.block_m))
    b = gh.align_to_host(gh.run_align(c.topk_ids, c.token_lora_mapping, s.E, s.L, s.block_m))
    for k in ("sorted_token_ids", "num_tokens_post_padded", "lora_ids"):
        for l, n in enumerate(a["num_tokens_post_padded"]):
            if k == "sorted_token_ids":
                assert np.array_equal(a[k][l, :n], b[k][l, :n])
        assert np.array_equal(a["num_tokens_post_padded"], b["num_tokens_post_padded"])


# ------------------------------------------------------------------ fused, full compare
def _full_compare(orc, s, variant):
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    y = dc.fused(variant=variant)
    got = gh.bf16_host_f64(y).reshape(s.numel, s.N)
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)
    gh.assert_fused_close(got, ref, f"{s.name}/{variant}/{s.dist}")
    base = gh.bf16_host_f64(dc.y_in).reshape(s.numel, s.N)
    inval = ~gh.valid_pairs(c)
    assert np.array_equal(got[inval], base[inval]), "rows of unmapped pairs changed"
    return c, dc, got, ref


@pytest.mark.parametrize("dist", ["literal", "stress"])
@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_fused_small_full(orc, name, dist, variant):
    s = synth.shape(name, dist=dist)
    if variant == "mfma" and not _mfma_ok(s):
        pytest.skip("MFMA kernel not available for this shape")
    _log(f"fused full {name} {dist} {variant}")
    _full_compare(orc, s, variant)


@pytest.mark.parametrize("name", ["tiny", "oss20b_decode_w13_a3"])
def test_fused_overwrite_delta(orc, name):
    """add_inputs = 0 writes the delta itself: checked elementwise and normwise."""
    s = synth.shape(name, add=False)
    for variant in _variants(s):
        _log(f"fused overwrite {name} {variant}")
        c, dc, got, ref = _full_compare(orc, s, variant)
        v = gh.valid_pairs(c)
        gh.assert_delta_close(got[v], ref[v], np.zeros_like(ref[v]), f"{name}/{variant}")


PRECISION = [
    ("oss20b_decode_w13_a6", {}, "valu"),          # stream kernel
    ("oss20b_decode_w13_a6", {}, "mfma"),          # MFMA kernel, one row tile
    ("tiny", dict(M=256, E=2, topk=2, L=1, active=1, p_neg=0.0, r=128, K=512, Ns=256,
                  block_m=64), "mfma"),            # MFMA kernel, 64-row passes, r = 128
    ("oss120b_decode_w13", {}, "valu"),            # register-batch kernel (fp32 v)
]


@pytest.mark.parametrize("i", range(len(PRECISION)))
def test_fused_rank_vector_precision(orc, i):
    """The rank vector enters the expand with about 16 significant bits: with
    add_inputs = 0, Y differs from the exact delta by the bf16 rounding of the
    output (at most 2^-8 relative) and a small absolute term.  A rank vector
    rounded once to bf16 misses this bound by about 0.01 of the rms delta."""
    name, kw, variant = PRECISION[i]
    s = synth.shape(name, dist="stress", add=False, **kw)
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    v = gh.valid_pairs(c)
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)[v]
    paths = [("sorted", dc.fused(variant=variant))]
    if s.numel <= 1024:
        paths.append(("align-free", dc.naive(variant=variant)))
    for path, y in paths:
        _log(f"precision {name} {variant} {path}")
        got = gh.bf16_host_f64(y).reshape(s.numel, s.N)[v]
        err = np.abs(got - ref)
        bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * np.sqrt(np.mean(ref ** 2))
        worst = np.argmax(err - bound)
        assert (err <= bound).all(), (f"{name}/{variant}/{path}: err {err.flat[worst]:.3e} > "
                                      f"{bound.flat[worst]:.3e} at |ref| {abs(ref.flat[worst]):.3e}")


# ------------------------------------------------------------------ fused, full size, every row
@pytest.mark.parametrize("dist", ["literal", "stress"])
@pytest.mark.parametrize("name", LARGE)
def test_fused_full_size(orc, name, dist):
    """Every element of Y against the oracle, at the configured full sizes, for
    every kernel that takes the shape; unmapped rows bit-identical."""
    s = synth.shape(name, dist=dist)
    _log(f"fused full-size {name} {dist}: drawing inputs")
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    align = dc.align()
    _log(f"fused full-size {name} {dist}: oracle over all {int(gh.valid_pairs(c).sum())} pairs")
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)
    inval = ~gh.valid_pairs(c)
    base_inval = dc.y_in.view(s.numel, s.N).view(torch.int16).cpu().numpy()[inval]
    for variant in _variants(s):
        _log(f"fused full-size {name} {dist} {variant}")
        y = dc.fused(align=align, variant=variant)
        got = gh.bf16_host_f64(y).reshape(s.numel, s.N)
        gh.assert_fused_close(got, ref, f"{name}/{dist}/{variant}")
        got_inval = y.view(s.numel, s.N).view(torch.int16).cpu().numpy()[inval]
        assert np.array_equal(got_inval, base_inval), "rows of unmapped pairs changed"
        del y, got


# ------------------------------------------------------------------ metamorphic, bit-exact
@pytest.mark.parametrize("name", ["tiny", "oss20b_decode_w13_a6", "oss120b_decode_w2"])
def test_fused_metamorphic(name):
    s = synth.shape(name, dist="stress")
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    align = dc.align()
    for variant in _variants(s):
        _log(f"fused metamorphic {name} {variant}")
        zero_a = torch.zeros_like(dc.a)
        y = dc.fused(align, variant, add=True, a=zero_a)
        assert torch.equal(y.view(torch.int16), dc.y_in.view(torch.int16)), "zero adapter, add"
        y = dc.fused(align, variant, add=False, a=zero_a)
        valid = torch.from_numpy(gh.valid_pairs(c)).to(gh.DEV)
        assert bool((y.view(s.numel, s.N)[valid].float() == 0).all()), "zero adapter, overwrite"
        # routed weights of one equal no routed weight
        ones = torch.ones_like(dc.w)
        w_saved, dc.w = dc.w, ones
        y1 = dc.fused(align, variant, mul=True)
        dc.w = w_saved
        y0 = dc.fused(align, variant, mul=False)
        assert torch.equal(y1.view(torch.int16), y0.view(torch.int16)), "w = 1 vs no weight"
        # doubling B doubles the overwritten delta exactly
        d1 = dc.fused(align, variant, add=False).view(s.numel, s.N)[valid].float()
        d2 = dc.fused(align, variant, add=False, b=dc.b * 2).view(s.numel, s.N)[valid].float()
        assert torch.equal(d2, 2 * d1), "B -> 2B"
        # add onto zeros equals overwrite
        yz = dc.fused(align, variant, add=True, y=torch.zeros_like(dc.y_in))
        yo = dc.fused(align, variant, add=False, y=torch.zeros_like(dc.y_in))
        assert torch.equal(yz.view(torch.int16), yo.view(torch.int16)), "add onto 0"
        # deterministic
        ya = dc.fused(align, variant)
        yb = dc.fused(align, variant)
        assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)), "run to run"


# ------------------------------------------------------------------ shapes and edge cases
EDGE = [
    dict(K=264, Ns=776, r=8, block_m=16),
    dict(K=264, Ns=776, r=5, block_m=32),
    dict(K=8, Ns=8, r=1, block_m=16),
    dict(K=128, Ns=64, r=4, block_m=64),
    dict(K=256, Ns=128, r=24, block_m=128),
    dict(K=512, Ns=256, r=128, block_m=64),
    dict(K=1032, Ns=136, r=64, block_m=16, S=3),
    dict(K=256, Ns=128, r=16, block_m=64, M=300, E=4, topk=3, x_per_pair=True, mul=True),
    dict(K=256, Ns=128, r=32, block_m=16, M=200, E=1024, topk=8, L=2, active=2),
    dict(K=64, Ns=64, r=16, block_m=16, M=70, E=3, L=100, active=70, p_neg=0.1),
    # full decode blocks: many valid rows per block (4-row and looped passes)
    dict(K=256, Ns=2184, r=64, block_m=16, M=64, E=2, topk=1, L=1, active=1, p_neg=0.0),
    dict(K=512, Ns=256, r=128, block_m=16, M=40, E=2, topk=1, L=1, active=1, p_neg=0.0),
    dict(K=2880, Ns=4096, r=32, block_m=32, M=48, E=3, topk=2, L=2, active=2, p_neg=0.0),
    # MFMA passes of 1, 2 and 4 row tiles; K and column tails; odd rank tiles
    # (r = 40: three tiles, one idle wavefront when they are split by rank)
    dict(K=200, Ns=200, r=40, block_m=64, M=256, E=2, topk=1, L=1, active=1, p_neg=0.0),
    # block_m = 128: two passes of 64 rows, rank 24 and 128
    dict(K=136, Ns=72, r=24, block_m=128, M=400, E=2, topk=1, L=1, active=1, p_neg=0.0),
    dict(K=256, Ns=136, r=128, block_m=128, M=300, E=2, topk=1, L=1, active=1, p_neg=0.0),
    # small ranks with few rows per block: K split over the wavefronts
    dict(K=392, Ns=104, r=8, block_m=32, M=40, E=4, topk=2, L=2, active=2),
    dict(K=328, Ns=88, r=32, block_m=64, M=24, E=2, topk=2, L=2, active=2),
    # ranks that are not a multiple of 16 / 32
    dict(K=320, Ns=96, r=96, block_m=32, M=64, E=2, topk=2, L=1, active=1, p_neg=0.0),
    # key spaces beyond one align pass (8192 keys): 16384 and 2^20 (slot, expert) keys
    # (K, Ns and r small: the weights of every slot are drawn, zero for inactive ones)
    dict(K=64, Ns=64, r=16, block_m=16, M=96, E=1024, topk=4, L=16, active=12),
    dict(K=8, Ns=8, r=2, block_m=32, M=40, E=1024, topk=2, L=1024, active=30),
    dict(K=128, Ns=48, r=120, block_m=64, M=100, E=2, topk=1, L=1, active=1, mul=True),
    dict(K=136, Ns=64, r=56, block_m=16, M=50, E=3, topk=2, L=2, active=2, x_per_pair=True),
    # K beyond what the decode stream kernel stages in LDS (4 rows x K):
    # the register-batch vector kernel takes it
    dict(K=4104, Ns=136, r=64, block_m=16, M=24, E=2, topk=2, L=2, active=2),
    # the stream kernel at its limits: the largest K it stages (4096), rank
    # 128, and enough units that the split count is the fewest that keep a
    # workgroup's columns within its Y buffer (4096 columns: two of 2048)
    dict(K=4096, Ns=4096, S=2, r=128, block_m=16, M=160, E=16, topk=4, L=2, active=2),
    # the stream kernel's largest blocks: 128 rows in 32 passes of 4
    dict(K=1024, Ns=1024, r=64, block_m=128, M=200, E=2, topk=1, L=1, active=1, p_neg=0.0),
    # around K = 3072, the largest K of the eight-row build option; full 16-row
    # blocks and tail blocks of 1 and 5 rows (several passes per block)
    dict(K=3072, Ns=520, r=64, block_m=16, M=38, E=2, topk=1, L=1, active=1, p_neg=0.0),
    dict(K=3080, Ns=520, r=32, block_m=16, M=38, E=2, topk=1, L=1, active=1, p_neg=0.0),
    # the block lookup on either side of 64 slots (one wavefront up to 64,
    # every wavefront beyond), stream and register-batch kernels
    dict(K=256, Ns=256, r=64, block_m=16, M=96, E=2, topk=1, L=64, active=40, p_neg=0.1),
    dict(K=256, Ns=256, r=32, block_m=16, M=96, E=2, topk=1, L=65, active=50, p_neg=0.1),
    dict(K=256, Ns=256, r=16, block_m=16, M=96, E=2, topk=1, L=65, active=50, p_neg=0.1),
]


@pytest.mark.parametrize("i", range(len(EDGE)))
def test_fused_edge_shapes(orc, i):
    s = synth.shape("tiny", dist="stress", seed=9000 + i, **EDGE[i])
    for variant in _variants(s):
        _log(f"fused edge {i} {EDGE[i]} {variant}")
        _full_compare(orc, s, variant)


def test_fused_duplicate_experts_in_token(orc):
    s = synth.shape("tiny", dist="stress", seed=77, topk=4)
    c = synth.draw(s)
    c.topk_ids[:, 1] = c.topk_ids[:, 0]     # the same expert twice per token
    c.topk_ids[::3, 3] = c.topk_ids[::3, 0]
    dc = gh.DeviceCase(c)
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, s.add)
    for variant in _variants(s):
        got = gh.bf16_host_f64(dc.fused(variant=variant)).reshape(s.numel, s.N)
        gh.assert_fused_close(got, ref, f"duplicates/{variant}")


def test_fused_no_mapped_token_and_empty_batch():
    s = synth.shape("tiny", p_neg=1.0)
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    for variant in _variants(s):
        y = dc.fused(variant=variant)
        assert torch.equal(y.view(torch.int16), dc.y_in.view(torch.int16))
    import moe_lora_adapter_amd as mla
    s0 = synth.shape("tiny", M=0)
    c0 = synth.draw(s0)
    d0 = gh.DeviceCase(c0)
    al = d0.align()
    torch.cuda.synchronize()
    assert int(al.num_active_loras.item()) == 0
    assert bool((al.num_tokens_post_padded == 0).all())
    mla.fused_moe_lora(d0.x, d0.a, d0.b, al, d0.w, d0.y_in, mul_routed_weight=True,
                       add_inputs=True)


@pytest.mark.parametrize("name", ["tiny", "oss20b_decode_w13_a6", "oss120b_decode_w13",
                                  "qwen3_prefill"])
def test_fused_max_active_loras(orc, name):
    """A batch that uses two of the L slots: the launch bounded by
    max_active_loras = 2 writes the same bits as the one bounded by L (and
    matches the oracle); max_active_loras = 0 launches nothing."""
    s = synth.shape(name)
    c = synth.draw(s)
    m = c.token_lora_mapping
    keep = (c.active_slots[0], c.active_slots[-1])   # two of the filled slots only
    c.token_lora_mapping = np.where(m >= 0, np.where(m % 2 == 0, keep[0], keep[1]), m).astype(m.dtype)
    dc = gh.DeviceCase(c)
    al = dc.align()
    torch.cuda.synchronize()
    nact = int(al.num_active_loras.item())
    assert nact <= 2
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, s.add, x_per_pair=s.x_per_pair)
    for variant in _variants(s):
        _log(f"fused max_active {name} {variant} nact={nact}")
        full = dc.fused(align=al, variant=variant)
        bound = dc.fused(align=al, variant=variant, max_active=nact)
        assert torch.equal(full.view(torch.int16), bound.view(torch.int16)), variant
        got = gh.bf16_host_f64(bound).reshape(s.numel, s.N)
        gh.assert_fused_close(got, ref, f"{name}/{variant}/max_active={nact}")
        none = dc.fused(align=al, variant=variant, max_active=0)
        assert torch.equal(none.view(torch.int16), dc.y_in.view(torch.int16))


# ------------------------------------------------------------------ graph capture
@pytest.mark.parametrize("name", ["tiny", "oss20b_decode_w13_a6", "qwen3_prefill"])
def test_graph_replay_matches_eager(name):
    """align + fused captured in a HIP graph: every replay equals the eager run."""
    import moe_lora_adapter_amd as mla
    s = synth.shape(name, dist="stress")
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    variants = _variants(s)
    eager = {v: dc.fused(variant=v) for v in variants}
    al = mla.alloc_align_output(s.M, s.topk, s.E, s.L, s.block_m, gh.DEV)
    ws = torch.empty(max(16, mla.align_workspace_size(s.M, s.topk, s.E, s.L, s.block_m)),
                     dtype=torch.uint8, device=gh.DEV)
    for v in variants:
        _log(f"graph replay {name} {v}")
        y = dc.y_in.clone()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            mla.moe_lora_align(dc.topk_ids, dc.mapping, s.E, s.L, s.block_m, out=al, workspace=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            mla.moe_lora_align(dc.topk_ids, dc.mapping, s.E, s.L, s.block_m, out=al, workspace=ws)
            mla.fused_moe_lora(dc.x, dc.a, dc.b, al, dc.w, y, mul_routed_weight=s.mul,
                               add_inputs=s.add, x_per_pair=s.x_per_pair, variant=v)
        for rep in range(3):
            y.copy_(dc.y_in)                       # eager work between replays
            al.sorted_token_ids.fill_(-7)
            al.num_tokens_post_padded.fill_(-7)
            al.expert_ids.fill_(-7)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), eager[v].view(torch.int16)), f"replay {rep}"
