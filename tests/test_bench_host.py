"""Host-side logic of bench.py (no GPU): the algorithmic work the roofline is
computed from, the one-GPU rule, the traffic records, the CPU baseline leg."""
import json
import os
import re

import numpy as np
import pytest

import bench
from moe_lora_adapter_amd import synth


def _brute_work(c):
    """The algorithmic bytes and flops, pair by pair (an independent count)."""
    s = c.shape
    groups, xrows, P, padded = set(), set(), 0, {}
    for p in range(s.numel):
        m, k = divmod(p, s.topk)
        l, e = int(c.token_lora_mapping[m]), int(c.topk_ids[m, k])
        if not (0 <= l < s.L and 0 <= e < s.E):
            continue
        P += 1
        groups.add((l, e))
        xrows.add(p if s.x_per_pair else m)
        padded[(l, e)] = padded.get((l, e), 0) + 1
    pad = sum(-(-n // s.block_m) * s.block_m for n in padded.values())
    w = len(groups) * s.S * (s.r * s.K + s.Ns * s.r) * 2
    x = len(xrows) * s.K * 2
    y = P * s.S * s.Ns * 2 * (2 if s.add else 1)
    meta = pad * 4 + pad // s.block_m * 4 + (P * 4 if s.mul else 0)
    return dict(valid_pairs=P, active_groups=len(groups), fused_bytes=w + x + y + meta,
                weight_bytes=w, fused_flops=2.0 * P * s.S * s.r * (s.K + s.Ns),
                naive_bytes=w + x + y + s.numel * 4 + s.M * 4 + (P * 4 if s.mul else 0))


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("oss20b_decode_w13_a3", {}),
                                     ("oss120b_decode_w2", {}),
                                     ("tiny", dict(add=False, x_per_pair=True, M=40, topk=3))])
def test_algorithmic_work_matches_a_pair_by_pair_count(name, kw):
    c = synth.draw(synth.shape(name, **kw), with_tensors=False)
    got, ref = bench.algorithmic_work(c), _brute_work(c)
    for k, v in ref.items():
        assert got[k] == v, k


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_traffic_record_goes_stale_with_the_kernel_sources(tmp_path, monkeypatch):
    for kernel in bench.KERNEL_SOURCES:
        for f in bench.kernel_source_files(kernel):
            assert os.path.exists(os.path.join(bench.ROOT, "moe_lora_adapter_amd", "csrc", f)), f
    rec = {"fused_stream_kernel/w": {"src_sha": bench.kernel_sources_sha("fused_stream_kernel"),
                                     "traffic_bytes_per_launch": 123},
           "fused_mfma_kernel/w": {"src_sha": "0" * 16, "traffic_bytes_per_launch": 456}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic("fused_stream_kernel", "w")[0] == 123
    assert bench.load_traffic("fused_mfma_kernel", "w")[0] is None      # sources changed since
    assert bench.load_traffic("fused_valu_kernel", "w")[0] is None      # never recorded


def test_traffic_record_covers_every_included_source():
    """A kernel's record key covers the headers its file includes, directly or
    through another header: the device code of every file that reaches it."""
    csrc = os.path.join(bench.ROOT, "moe_lora_adapter_amd", "csrc")
    for kernel, own in bench.KERNEL_SOURCES.items():
        files = bench.kernel_source_files(kernel)
        for f in own:
            with open(os.path.join(csrc, f)) as fh:
                for inc in re.findall(r'^#include "([^"]+)"', fh.read(), re.M):
                    assert os.path.normpath(inc) in files, (kernel, inc)
    assert "align_wave.h" in bench.kernel_source_files("fused_stream_kernel")
    assert "groups.h" in bench.kernel_source_files("fused_mfma_kernel")
    assert "common.h" in bench.kernel_source_files("fused_valu_kernel")  # through every header


def test_cpu_baseline_leg_reports_the_oracle():
    c = synth.draw(synth.shape("tiny"))
    out = bench.cpu_baseline(c, 0.2)
    assert out["kind"] == "oracle" and out["unit"] == "us/call"
    assert out["value"] > 0 and out["cores"] >= 1
    assert out["value"] == pytest.approx(out["align_us"] + out["fused_us"], abs=0.2)


def test_step_path_resolution():
    """--path auto times the whole path in one launch for decode batches (at
    most 64 pairs and slots) and as align + fused otherwise; the limits are the
    library's."""
    import moe_lora_adapter_amd as mla
    assert (mla.WITH_ALIGN_MAX_PAIRS, mla.WITH_ALIGN_MAX_SLOTS) == (64, 64)
    for name, want in [("oss20b_decode_w13_a6", "with_align"), ("oss120b_decode_w13", "with_align"),
                       ("tiny", "with_align"), ("qwen3_prefill", "sorted"),
                       ("oss120b_prefill_w13", "sorted"), ("dense_qkv", "sorted")]:
        assert bench.resolve_path("auto", synth.shape(name)) == want, name
    assert bench.resolve_path("auto", synth.shape("tiny", M=17, topk=4)) == "sorted"  # 68 pairs
    assert bench.resolve_path("auto", synth.shape("tiny", L=65, E=2, active=2)) == "sorted"
    assert bench.resolve_path("sorted", synth.shape("tiny")) == "sorted"


@pytest.mark.parametrize("name", ["oss20b_decode_w13_a6", "oss20b_decode_w13_a2",
                                  "oss120b_decode_w13"])
def test_draw_layer_shares_the_routing(name):
    """The w2 case of a layer takes the w13 case's routing, and its adapters
    sit in exactly the slots that routing uses."""
    c13, c2 = synth.draw_layer(name)
    s13, s2 = c13.shape, c2.shape
    assert s2.x_per_pair and s2.K == s13.Ns and s2.name == synth.w2_partner(name)
    for k in ("active_slots", "token_lora_mapping", "topk_ids", "topk_weights"):
        assert np.array_equal(getattr(c13, k), getattr(c2, k)), k
    filled = [l for l in range(s2.L) if c2.lora_a[:, l].any() or c2.lora_b[:, l].any()]
    assert filled == sorted(c13.active_slots.tolist())
    # the moved adapters are c2's own draw, not zeros and not w13's
    own = synth.draw(s2)
    assert np.array_equal(c2.lora_a[:, c13.active_slots], own.lora_a[:, own.active_slots])
    with pytest.raises(KeyError):
        synth.w2_partner("qwen3_prefill")


def test_active_count_buckets():
    from moe_lora_adapter_amd import graphs
    assert graphs.active_count_buckets(1) == [0, 1]
    assert graphs.active_count_buckets(4) == [0, 1, 2, 4]
    assert graphs.active_count_buckets(6) == [0, 1, 2, 4, 6]
    assert graphs.active_count_buckets(8) == [0, 1, 2, 4, 8]
    # key count for L = 4 and two batch sizes: 4 buckets x 2
    assert 2 * len(graphs.active_count_buckets(4)) == 8
    assert [graphs.bucket_for(n, 6) for n in range(7)] == [0, 1, 2, 4, 4, 6, 6]
    with pytest.raises(ValueError):
        graphs.bucket_for(7, 6)
    with pytest.raises(ValueError):
        graphs.active_count_buckets(0)


@pytest.mark.parametrize("name,kw", [("tiny", dict(dist="stress")),
                                     ("oss20b_decode_w13_a6", dict(K=256, Ns=256)),
                                     ("align_stress", {}),
                                     ("qwen3_prefill", dict(M=64, K=64, Ns=64, r=8))])
def test_generator_is_deterministic(name, kw):
    """The same seed draws the same bytes; another seed draws other routing.
    The drawn routing has the recipe's structure: the mapping names only the
    drawn active slots (or -1), every token's top-k experts are distinct and in
    range, and the routing weights of a token sum to one."""
    s = synth.shape(name, **kw)
    c1, c2 = synth.draw(s), synth.draw(s)
    for k in ("active_slots", "token_lora_mapping", "topk_ids", "topk_weights",
              "x", "lora_a", "lora_b", "y_in"):
        a, b = getattr(c1, k), getattr(c2, k)
        assert (a is None) == (b is None), k
        if a is not None:
            assert a.dtype == b.dtype and a.tobytes() == b.tobytes(), k
    other = synth.draw(s.replace(seed=s.seed + 1), with_tensors=False)
    assert not np.array_equal(other.topk_ids, c1.topk_ids)
    assert len(c1.active_slots) == s.active == len(set(c1.active_slots.tolist()))
    used = set(c1.token_lora_mapping.tolist()) - {-1}
    assert used <= set(c1.active_slots.tolist())
    ids = c1.topk_ids
    assert ids.shape == (s.M, s.topk) and ids.min() >= 0 and ids.max() < s.E
    if s.topk <= s.E:
        assert all(len(set(row)) == s.topk for row in ids.tolist())
    np.testing.assert_allclose(c1.topk_weights.sum(axis=1), 1.0, rtol=1e-5)
