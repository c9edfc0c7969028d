"""One captured HIP graph serves every active-slot count.

The fused kernels find their blocks on the device (from
num_tokens_post_padded, or from topk_ids and the mapping on the align-free
path), and the launch size depends on M alone, so a graph captured once
replays correctly whatever number of slots the current batch uses: no
per-count graphs and no device-to-host read of the active count.  Each
replay below runs after the mapping has been rewritten in place to activate
a different number of slots (none, one, some, all) and is compared with the
eager result for the same inputs, bit for bit.
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


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _mappings(s, rng):
    """Token -> slot mappings with 0, 1, 2, ..., L active slots (and -1 tokens)."""
    out = []
    for n_active in [0, 1, 2, s.L // 2, s.L]:
        if n_active == 0:
            m = np.full(s.M, -1, dtype=np.int32)
        else:
            slots = np.sort(rng.choice(s.L, size=n_active, replace=False))
            m = slots[rng.integers(0, n_active, size=s.M)].astype(np.int32)
            m[rng.random(s.M) < 0.1] = -1
        out.append((n_active, m))
    return out


def _full_adapters(s, rng):
    """lora_a / lora_b with every slot filled (the drawn case fills only its active slots)."""
    a = rng.standard_normal((s.S, s.L, s.E, s.r, s.K), dtype=np.float32) / np.sqrt(s.K)
    b = rng.standard_normal((s.S, s.L, s.E, s.Ns, s.r), dtype=np.float32) / np.sqrt(s.r)
    to16 = lambda v: torch.from_numpy(v).to(gh.DEV).to(torch.bfloat16)  # noqa: E731
    return to16(a), to16(b)


@pytest.mark.parametrize("path", ["sorted", "naive", "two_kernel"])
@pytest.mark.parametrize("name", ["tiny", "oss20b_decode_w13_a6", "oss120b_decode_w2"])
def test_one_graph_all_active_counts(name, path):
    s = synth.shape(name, dist="stress")
    rng = np.random.default_rng(4242)
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    dc.a, dc.b = _full_adapters(s, rng)
    mapping = dc.mapping            # rewritten in place between replays
    y = dc.y_in.clone()
    al = mla.alloc_align_output(s.M, s.topk, s.E, s.L, s.block_m, gh.DEV)
    ws = torch.empty(max(16, mla.align_workspace_size(s.M, s.topk, s.E, s.L, s.block_m)),
                     dtype=torch.uint8, device=gh.DEV)
    ws2 = torch.empty(max(16, mla.two_kernel_workspace_bytes(s.M, s.topk, s.K, s.Ns, s.S, s.E,
                                                             s.L, s.r, s.block_m, s.x_per_pair)),
                      dtype=torch.uint8, device=gh.DEV)

    def call():
        if path == "two_kernel":
            mla.moe_lora_align(dc.topk_ids, mapping, s.E, s.L, s.block_m, out=al, workspace=ws)
            mla.fused_moe_lora_two_kernel(dc.x, dc.a, dc.b, al, dc.w, y, mul_routed_weight=s.mul,
                                          add_inputs=s.add, x_per_pair=s.x_per_pair,
                                          workspace=ws2)
        elif path == "sorted":
            mla.moe_lora_align(dc.topk_ids, mapping, s.E, s.L, s.block_m, out=al, workspace=ws)
            mla.fused_moe_lora(dc.x, dc.a, dc.b, al, dc.w, y, mul_routed_weight=s.mul,
                               add_inputs=s.add, x_per_pair=s.x_per_pair)
        else:
            mla.fused_moe_lora_naive(dc.x, dc.a, dc.b, dc.topk_ids, mapping, dc.w, y,
                                     mul_routed_weight=s.mul, add_inputs=s.add,
                                     block_m=s.block_m, x_per_pair=s.x_per_pair)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()

    orc = oracle.load()
    for n_active, m in _mappings(s, rng):
        _log(f"graph {name} {path}: {n_active} active slots")
        mapping.copy_(torch.from_numpy(m))
        y.copy_(dc.y_in)
        torch.cuda.synchronize()
        call()                      # eager reference on the same inputs
        torch.cuda.synchronize()
        eager = y.clone()
        y.copy_(dc.y_in)
        al.num_tokens_post_padded.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"{n_active} active"
        if n_active == 0:
            assert torch.equal(y.view(torch.int16), dc.y_in.view(torch.int16))
        # and the replay is the right answer, not only a repeatable one
        a_host = dc.a.view(torch.int16).cpu().numpy().view(np.uint16)
        b_host = dc.b.view(torch.int16).cpu().numpy().view(np.uint16)
        ref = orc.fused(c.x, a_host, b_host, c.topk_ids, m, c.topk_weights, c.y_in, s.mul,
                        s.add, x_per_pair=s.x_per_pair)
        gh.assert_fused_close(gh.bf16_host_f64(y).reshape(s.numel, s.N), ref,
                              f"{name}/{path}/{n_active}")


@pytest.mark.parametrize("name", ["tiny", "oss20b_decode_w13_a6", "qwen3_prefill"])
def test_graph_per_active_count_bucket(name):
    """The per-bucket scheme: one graph per bound on the active slots
    (max_active_loras = bucket), the host choosing the bucket from the batch's
    adapters; each replay equals the eager launch bounded by L, bit for bit."""
    from moe_lora_adapter_amd import graphs
    s = synth.shape(name, dist="stress")
    rng = np.random.default_rng(4343)
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    dc.a, dc.b = _full_adapters(s, rng)
    mapping = dc.mapping
    y = dc.y_in.clone()
    al = mla.alloc_align_output(s.M, s.topk, s.E, s.L, s.block_m, gh.DEV)
    ws = torch.empty(max(16, mla.align_workspace_size(s.M, s.topk, s.E, s.L, s.block_m)),
                     dtype=torch.uint8, device=gh.DEV)

    def call(bound):
        mla.moe_lora_align(dc.topk_ids, mapping, s.E, s.L, s.block_m, out=al, workspace=ws)
        mla.fused_moe_lora(dc.x, dc.a, dc.b, al, dc.w, y, mul_routed_weight=s.mul,
                           add_inputs=s.add, x_per_pair=s.x_per_pair, max_active_loras=bound)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(s.L)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    per_bucket = {}
    for bk in graphs.active_count_buckets(s.L):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(bk)
        per_bucket[bk] = g
    orc = oracle.load()
    a_host = dc.a.view(torch.int16).cpu().numpy().view(np.uint16)
    b_host = dc.b.view(torch.int16).cpu().numpy().view(np.uint16)
    for n_active, m in _mappings(s, rng):
        bk = graphs.bucket_for(len(np.unique(m[m >= 0])), s.L)
        _log(f"bucket graphs {name}: {n_active} active -> bucket {bk}")
        mapping.copy_(torch.from_numpy(m))
        y.copy_(dc.y_in)
        torch.cuda.synchronize()
        call(s.L)
        torch.cuda.synchronize()
        eager = y.clone()
        for rep in range(2):
            y.copy_(dc.y_in)
            al.num_tokens_post_padded.fill_(-7)
            torch.cuda.synchronize()
            per_bucket[bk].replay()
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), \
                f"{n_active} active, bucket {bk}, replay {rep}"
        ref = orc.fused(c.x, a_host, b_host, c.topk_ids, m, c.topk_weights, c.y_in, s.mul,
                        s.add, x_per_pair=s.x_per_pair)
        gh.assert_fused_close(gh.bf16_host_f64(y).reshape(s.numel, s.N), ref,
                              f"{name}/bucket {bk}/{n_active}")
