"""The dual-stream path: LoRA delta on an auxiliary stream, joined onto the base output.

The base output is produced on the default stream while the aligned LoRA delta
(fused_moe_lora with add_inputs = 0 into a zero-filled buffer) runs on an
auxiliary stream; an event joins them and moe_lora_accumulate adds the delta.
Checked against the oracle (Y_in + delta, tolerance 1e-2 (1 + |oracle|)),
eagerly and captured in one graph; moe_lora_accumulate itself bit for bit
against an fp32 add rounded to nearest even on the host.
"""
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
