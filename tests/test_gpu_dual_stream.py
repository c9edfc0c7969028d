"""The dual-stream path: LoRA delta on an auxiliary stream, joined onto the base output.

The base output is produced on the default stream while the aligned LoRA delta
(fused_moe_lora with add_inputs = 0 into a zero-filled buffer) runs on an
auxiliary stream; an event joins them and moe_lora_accumulate adds the delta.
Checked against the oracle (Y_in + delta, tolerance 1e-2 (1 + |oracle|)),
eagerly and captured in one graph; moe_lora_accumulate itself bit for bit
against an fp32 add rounded to nearest even on the host.

Also: the base MoE align (one slot, every token in it) and the LoRA align on
two streams in one graph, both bit-exact against the oracle; and one MoE
layer's w13 -> activation -> w2 chain with four events (moe_lora_adapter_amd.
streams), each LoRA step against the oracle and the dual-stream run equal bit
for bit to the serial one.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import moe_lora_adapter_amd as mla  # noqa: E402
from moe_lora_adapter_amd import synth  # noqa: E402
import gpu_helpers as gh  # noqa: E402


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 4096, 100003, 5 * 2 ** 20 + 3])
def test_accumulate_bit_exact(n):
    g = torch.Generator().manual_seed(n)
    y = (torch.randn(n, generator=g) * 3).to(torch.bfloat16)
    d = (torch.randn(n, generator=g) * 0.01).to(torch.bfloat16)
    if n > 4:  # exact cancellation, infinities away, subnormal-free edges
        d[:2] = -y[:2]
    ref = (y.float() + d.float()).to(torch.bfloat16)  # fp32 sum, one rounding to nearest even
    yd, dd = y.to(gh.DEV), d.to(gh.DEV)
    mla.moe_lora_accumulate(yd, dd)
    torch.cuda.synchronize()
    assert torch.equal(yd.cpu().view(torch.int16), ref.view(torch.int16))


def test_accumulate_rounding_edges():
    """The one rounding of every kernel's output, through moe_lora_accumulate:
    sums that fall exactly halfway between two bf16 values (ties to even, both
    directions, both signs), subnormal sums, sums past the largest bf16 (to
    infinity), cancellation to zero, against an fp32 add rounded to nearest
    even on the host."""
    bf = torch.bfloat16
    ulp_at_1 = 2.0 ** -7
    tiny = 2.0 ** -133                     # a bf16 subnormal
    big = float(torch.finfo(bf).max)
    pairs = [
        (1.0, ulp_at_1 / 2),               # tie: 1 (even) stays
        (1.0 + ulp_at_1, ulp_at_1 / 2),    # tie: odd rounds up to even
        (-1.0, -ulp_at_1 / 2),
        (-(1.0 + ulp_at_1), -ulp_at_1 / 2),
        (1.0, ulp_at_1 / 4),               # below the tie: down
        (1.0, 3 * ulp_at_1 / 4),           # above the tie: up
        (tiny, tiny),                      # subnormal + subnormal
        (3 * tiny, -tiny),
        (2.0 ** -126, -2.0 ** -127),       # normal - subnormal -> subnormal
        (big, big),                        # overflow -> inf
        (-big, -big),
        (2.5, -2.5),                       # exact cancellation
        (0.0, -0.0),
    ]
    y = torch.tensor([a for a, _ in pairs], dtype=torch.float32).to(bf)
    d = torch.tensor([b for _, b in pairs], dtype=torch.float32).to(bf)
    # the inputs are exact in bf16
    assert torch.equal(y.float(), torch.tensor([a for a, _ in pairs], dtype=torch.float32))
    assert torch.equal(d.float(), torch.tensor([b for _, b in pairs], dtype=torch.float32))
    ref = (y.float() + d.float()).to(bf)
    yd, dd = y.to(gh.DEV), d.to(gh.DEV)
    mla.moe_lora_accumulate(yd, dd)
    torch.cuda.synchronize()
    got = yd.cpu()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (got, ref)
    assert got[0].item() == 1.0 and got[1].item() == 1.0 + 2 * ulp_at_1
    assert got[9].item() == float("inf") and got[10].item() == float("-inf")


def _dual(dc, al, y, delta, aux, ev):
    """Base output (here: Y_in) on the current stream, the LoRA delta on `aux`, then the join."""
    s = dc.s
    main = torch.cuda.current_stream()
    aux.wait_stream(main)
    with torch.cuda.stream(aux):
        delta.zero_()
        mla.moe_lora_align(dc.topk_ids, dc.mapping, s.E, s.L, s.block_m, out=al)
        mla.fused_moe_lora(dc.x, dc.a, dc.b, al, dc.w, delta, mul_routed_weight=s.mul,
                           add_inputs=False, x_per_pair=s.x_per_pair)
        ev.record(aux)
    y.copy_(dc.y_in)          # stands for the base GEMM's output
    main.wait_event(ev)
    mla.moe_lora_accumulate(y, delta)


@pytest.mark.parametrize("name", ["tiny", "oss20b_decode_w13_a6", "oss120b_decode_w2",
                                  "oss120b_prefill_w13"])
def test_dual_stream_matches_oracle_eager_and_in_a_graph(name):
    s = synth.shape(name, dist="stress")
    c = synth.draw(s)
    dc = gh.DeviceCase(c)
    orc = oracle.load()
    ref = orc.fused(c.x, c.lora_a, c.lora_b, c.topk_ids, c.token_lora_mapping, c.topk_weights,
                    c.y_in, s.mul, True, x_per_pair=s.x_per_pair)
    al = mla.alloc_align_output(s.M, s.topk, s.E, s.L, s.block_m, gh.DEV)
    y = torch.empty_like(dc.y_in)
    delta = torch.empty_like(dc.y_in)
    aux = torch.cuda.Stream()
    ev = torch.cuda.Event()

    def check(what):
        got = gh.bf16_host_f64(y).reshape(s.numel, s.N)
        gh.assert_fused_close(got, ref, f"{name}/{what}")

    _dual(dc, al, y, delta, aux, ev)
    torch.cuda.synchronize()
    check("eager")
    eager = y.clone()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _dual(dc, al, y, delta, aux, ev)       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _dual(dc, al, y, delta, aux, ev)
    for rep in range(3):
        y.fill_(7.0)
        delta.fill_(-3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
    check("graph")


# ------------------------------------------------------------------ two-stream align
def _host_i32(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("name", ["oss20b_decode_w13_a6", "oss120b_prefill_w13", "qwen3_prefill",
                                  "align_stress", "align_stress_neg"])
def test_two_stream_align_in_one_graph(name):
    """The base MoE align (one slot, every token mapped to it) on an auxiliary
    stream beside the LoRA align on the main one, each with its own output and
    workspace, captured in one graph: every replay writes both results bit for
    bit as the oracle defines them."""
    s = synth.shape(name)
    c = synth.draw(s, with_tensors=False)
    orc = oracle.load()
    topk_ids = gh.i32_dev(c.topk_ids)
    mapping = gh.i32_dev(c.token_lora_mapping)
    zero_map = torch.zeros(s.M, dtype=torch.int32, device=gh.DEV)  # plain MoE: slot 0 for all
    ref_lora = orc.align(c.topk_ids, c.token_lora_mapping, s.E, s.L, s.block_m)
    ref_base = orc.align(c.topk_ids, np.zeros(s.M, np.int32), s.E, 1, s.block_m)
    outs, wss = [], []
    for L in (s.L, 1):
        outs.append(mla.alloc_align_output(s.M, s.topk, s.E, L, s.block_m, gh.DEV))
        nb = mla.align_workspace_size(s.M, s.topk, s.E, L, s.block_m)
        wss.append(torch.empty(max(16, nb), dtype=torch.uint8, device=gh.DEV))
    lora_out, base_out = outs
    aux = torch.cuda.Stream()
    fork, join = torch.cuda.Event(), torch.cuda.Event()

    def both():
        main = torch.cuda.current_stream()
        fork.record(main)
        aux.wait_event(fork)
        with torch.cuda.stream(aux):
            mla.moe_lora_align(topk_ids, zero_map, s.E, 1, s.block_m, out=base_out,
                               workspace=wss[1])
            join.record(aux)
        mla.moe_lora_align(topk_ids, mapping, s.E, s.L, s.block_m, out=lora_out,
                           workspace=wss[0])
        main.wait_event(join)

    def poison():
        for o in outs:
            for t in (o.sorted_token_ids, o.expert_ids, o.num_tokens_post_padded, o.lora_ids,
                      o.num_active_loras):
                t.fill_(-7)
        torch.cuda.synchronize()

    def check(what):
        gh.assert_align_equal(gh.align_to_host(lora_out), ref_lora, s.block_m)
        gh.assert_align_equal(gh.align_to_host(base_out), ref_base, s.block_m)

    print(f"two-stream align {name}", flush=True)
    poison()
    both()
    torch.cuda.synchronize()
    check("eager")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        both()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        both()
    for rep in range(3):
        poison()
        g.replay()
        torch.cuda.synchronize()
        check(f"replay {rep}")
        both()                                     # eager work between replays
        torch.cuda.synchronize()
        check(f"eager after replay {rep}")


# ------------------------------------------------------------------ one MoE layer, four events
class _Layer:
    """One MoE layer's w13 -> activation -> w2 with the LoRA side forked off.

    The base GEMMs are dense stand-ins (one shared matrix instead of one per
    expert; the base MoE is the caller's, not this library's).  The w13 fork
    also runs the base MoE align (one slot) beside the LoRA align."""

    def __init__(self, c13, c2, seed=123):
        from moe_lora_adapter_amd.streams import LoraStreams
        s13, s2 = c13.shape, c2.shape
        self.s13, self.s2 = s13, s2
        self.d13, self.d2 = gh.DeviceCase(c13), gh.DeviceCase(c2)
        dev = gh.DEV
        M, topk, numel = s13.M, s13.topk, s13.numel
        self.zero_map = torch.zeros(M, dtype=torch.int32, device=dev)
        self.al = mla.alloc_align_output(M, topk, s13.E, s13.L, s13.block_m, dev)
        self.al_ws = torch.empty(max(16, mla.align_workspace_size(M, topk, s13.E, s13.L,
                                                                  s13.block_m)),
                                 dtype=torch.uint8, device=dev)
        self.base_al = mla.alloc_align_output(M, topk, s13.E, 1, s13.block_m, dev)
        self.base_al_ws = torch.empty(max(16, mla.align_workspace_size(M, topk, s13.E, 1,
                                                                       s13.block_m)),
                                      dtype=torch.uint8, device=dev)
        gen = torch.Generator().manual_seed(seed)
        self.w13b = (torch.randn(s13.K, s13.N, generator=gen) / s13.K ** 0.5).to(torch.bfloat16).to(dev)
        self.w2b = (torch.randn(s2.K, s2.N, generator=gen) / s2.K ** 0.5).to(torch.bfloat16).to(dev)
        self.base1 = torch.empty(M, s13.N, dtype=torch.bfloat16, device=dev)
        self.y1 = torch.empty(M, topk, s13.N, dtype=torch.bfloat16, device=dev)
        self.delta1 = torch.empty_like(self.y1)
        self.h = torch.empty(numel, s2.K, dtype=torch.bfloat16, device=dev)
        self.base2 = torch.empty(numel, s2.N, dtype=torch.bfloat16, device=dev)
        self.y2 = torch.empty(M, topk, s2.N, dtype=torch.bfloat16, device=dev)
        self.delta2 = torch.empty_like(self.y2)
        self.streams = LoraStreams()

    def base13(self):
        s = self.s13
        mla.moe_lora_align(self.d13.topk_ids, self.zero_map, s.E, 1, s.block_m,
                           out=self.base_al, workspace=self.base_al_ws)
        torch.matmul(self.d13.x, self.w13b, out=self.base1)
        self.y1.copy_(self.base1[:, None, :].expand(s.M, s.topk, s.N))

    def lora13(self):
        s, d = self.s13, self.d13
        self.delta1.zero_()
        mla.moe_lora_align(d.topk_ids, d.mapping, s.E, s.L, s.block_m, out=self.al,
                           workspace=self.al_ws)
        mla.fused_moe_lora(d.x, d.a, d.b, self.al, d.w, self.delta1, mul_routed_weight=s.mul,
                           add_inputs=False)

    def act(self):
        s = self.s13
        y = self.y1.view(s.numel, s.N)
        if s.S == 2:       # gate and up slices (a stand-in SwiGLU)
            torch.mul(torch.nn.functional.silu(y[:, :s.Ns]), y[:, s.Ns:], out=self.h)
        else:
            self.h.copy_(torch.nn.functional.silu(y))

    def base2_fn(self):
        torch.matmul(self.h, self.w2b, out=self.base2)
        self.y2.view(self.s2.numel, self.s2.N).copy_(self.base2)

    def lora2(self):
        s, d = self.s2, self.d2
        self.delta2.zero_()
        mla.fused_moe_lora(self.h, d.a, d.b, self.al, d.w, self.delta2, mul_routed_weight=s.mul,
                           add_inputs=False, x_per_pair=True)

    def dual(self):
        from moe_lora_adapter_amd.streams import W13, W2
        self.streams.fork_join(W13, self.base13, self.lora13, self.y1, self.delta1)
        self.act()
        self.streams.fork_join(W2, self.base2_fn, self.lora2, self.y2, self.delta2)

    def serial(self):
        self.base13()
        self.lora13()
        mla.moe_lora_accumulate(self.y1, self.delta1)
        self.act()
        self.base2_fn()
        self.lora2()
        mla.moe_lora_accumulate(self.y2, self.delta2)

    def results(self):
        return [t.clone() for t in (self.y1, self.h, self.y2)]

    def poison(self):
        for t in (self.y1, self.delta1, self.h, self.y2, self.delta2, self.base1, self.base2):
            t.fill_(5.0)
        for o in (self.al, self.base_al):
            o.sorted_token_ids.fill_(-7)
            o.num_tokens_post_padded.fill_(-7)
        torch.cuda.synchronize()


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _same(a, b):
    return all(torch.equal(x.view(torch.int16), y.view(torch.int16)) for x, y in zip(a, b))


@pytest.mark.parametrize("name", ["oss20b_decode_w13_a6", "oss120b_decode_w13",
                                  "oss120b_prefill_w13"])
def test_layer_chain_four_events(name):
    """w13 (LoRA ‖ base, join) -> activation -> w2 (LoRA with per-pair X ‖ base,
    join), the LoRA side on an auxiliary stream: each LoRA step against the
    oracle on the inputs it actually saw, both aligns bit-exact, and the
    dual-stream run equal bit for bit to the serial one, eagerly and on every
    replay of one captured graph."""
    c13, c2 = synth.draw_layer(name, dist="stress")
    s13, s2 = c13.shape, c2.shape
    lay = _Layer(c13, c2)
    orc = oracle.load()
    print(f"layer chain {name}", flush=True)
    lay.poison()
    lay.serial()
    torch.cuda.synchronize()
    serial = lay.results()

    # the LoRA align and the base MoE align
    gh.assert_align_equal(gh.align_to_host(lay.al),
                          orc.align(c13.topk_ids, c13.token_lora_mapping, s13.E, s13.L,
                                    s13.block_m), s13.block_m)
    gh.assert_align_equal(gh.align_to_host(lay.base_al),
                          orc.align(c13.topk_ids, np.zeros(s13.M, np.int32), s13.E, 1,
                                    s13.block_m), s13.block_m)
    # w13: Y1 = base + LoRA delta
    y1_in = np.broadcast_to(_bits(lay.base1)[:, None, :], (s13.M, s13.topk, s13.N)).copy()
    ref1 = orc.fused(c13.x, c13.lora_a, c13.lora_b, c13.topk_ids, c13.token_lora_mapping,
                     c13.topk_weights, y1_in, s13.mul, True)
    gh.assert_fused_close(gh.bf16_host_f64(serial[0]).reshape(s13.numel, s13.N), ref1, "w13")
    # w2: Y2 = base + LoRA delta of the activation (one X row per pair)
    y2_in = _bits(lay.base2).reshape(s2.M, s2.topk, s2.N)
    ref2 = orc.fused(_bits(serial[1]), c2.lora_a, c2.lora_b, c2.topk_ids, c2.token_lora_mapping,
                     c2.topk_weights, y2_in, s2.mul, True, x_per_pair=True)
    gh.assert_fused_close(gh.bf16_host_f64(serial[2]).reshape(s2.numel, s2.N), ref2, "w2")

    lay.poison()
    lay.dual()
    torch.cuda.synchronize()
    assert _same(lay.results(), serial), "dual-stream eager run differs from the serial one"

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lay.dual()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        lay.dual()
    for rep in range(3):
        lay.poison()
        g.replay()
        torch.cuda.synchronize()
        assert _same(lay.results(), serial), f"replay {rep}"
        lay.serial()                               # eager work between replays
        torch.cuda.synchronize()
