"""The no-allocation align (moe_lora_align_noalloc) against moe_lora_align.

moe_lora_align_noalloc takes no workspace: the multi-workgroup path's scratch
is a static device array of the library.  Its outputs must equal those of
moe_lora_align with a caller-owned workspace, bit for bit, on two calls in a
row on the same GPU, the second smaller than the first (the array keeps the
first call's contents), and both must equal the oracle.
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


def _case(M, topk, E, L, B, seed):
    rng = np.random.default_rng(seed)
    topk_ids = rng.integers(-1, E + 1, size=(M, topk)).astype(np.int32)
    mapping = rng.integers(-2, L + 1, size=M).astype(np.int32)
    return topk_ids, mapping


def _noalloc(topk_ids, mapping, E, L, B):
    M, topk = topk_ids.shape
    out = mla.alloc_align_output(M, topk, E, L, B, gh.DEV)
    for t in (out.sorted_token_ids, out.expert_ids, out.num_tokens_post_padded, out.lora_ids,
              out.num_active_loras):
        t.fill_(-7)
    mla.moe_lora_align_noalloc(gh.i32_dev(topk_ids), gh.i32_dev(mapping), E, L, B, out=out)
    torch.cuda.synchronize()
    return gh.align_to_host(out)


def test_noalloc_align_matches_workspace_align_twice_shrinking():
    orc = oracle.load()
    s = synth.shape("align_stress")
    c = synth.draw(s, with_tensors=False)
    cases = [(c.topk_ids, c.token_lora_mapping, s.E, s.L, s.block_m),
             (*_case(5003, 4, 64, 4, 32, 11), 64, 4, 32)]
    for i, (topk_ids, mapping, E, L, B) in enumerate(cases):
        M, topk = topk_ids.shape
        assert mla.align_workspace_size(M, topk, E, L, B) > 0, "the case must use the scratch"
        _log(f"no-alloc align call {i}: M={M} topk={topk} E={E} L={L} B={B}")
        got = _noalloc(topk_ids, mapping, E, L, B)
        ref_ws = gh.align_to_host(gh.run_align(topk_ids, mapping, E, L, B))
        gh.assert_align_equal(got, ref_ws, B)
        gh.assert_align_equal(got, orc.align(topk_ids, mapping, E, L, B), B)


def test_noalloc_align_single_workgroup_and_wave_paths():
    orc = oracle.load()
    for (M, topk, E, L, B) in ((16, 4, 32, 6, 16), (1000, 4, 64, 4, 64), (0, 4, 32, 6, 16)):
        topk_ids, mapping = _case(M, topk, E, L, B, M + 3)
        _log(f"no-alloc align small M={M} topk={topk} E={E} L={L} B={B}")
        got = _noalloc(topk_ids, mapping, E, L, B)
        gh.assert_align_equal(got, orc.align(topk_ids, mapping, E, L, B), B)
