"""The C ABI library on the host: it loads, exports every declared symbol,
and rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import moe_lora_adapter_amd as mla
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_lora.h")

V = ctypes.c_void_p
P16 = V(16)  # a non-null, 16-byte aligned stand-in; never dereferenced


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"MOE_LORA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert set(names) == set(mla.SIGNATURES), names
    lib = mla.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert mla.status_string(0) == "ok"
    for st in (-1, -2, -3, -4):
        assert mla.status_string(st) not in ("ok", "unknown status")
    assert mla.status_string(5) == "unknown status"


def test_capacity_matches_oracle_and_bound():
    o = oracle.load()
    for M, topk, E, B in ((16, 2, 8, 16), (16, 4, 32, 16), (8192, 8, 128, 64),
                          (0, 4, 32, 16), (3, 1, 2, 4 * 4), (65536, 8, 256, 64)):
        assert mla.align_capacity(M, topk, E, B) == o.capacity(M, topk, E, B)


def test_workspace_query():
    assert mla.align_workspace_size(16, 4, 32, 6, 16) == 0          # one workgroup
    # tiles: the per-tile counts (tiles of >= 512 pairs, at most 2^20 / (L E)
    # of them) and the key totals, int32
    assert mla.align_workspace_size(65536, 8, 256, 16, 64) == (256 + 1) * 4096 * 4
    assert mla.align_workspace_size(8192, 8, 128, 8, 64) == (128 + 1) * 1024 * 4
    assert mla.align_workspace_size(0, 4, 32, 6, 16) == 0


def align_call(**kw):
    args = dict(topk_ids=P16, mapping=P16, M=16, topk=4, E=32, L=6, B=16, sorted=P16,
                eids=P16, ntpp=P16, lora_ids=None, nact=None, ws=None, ws_bytes=0)
    args.update(kw)
    a = args
    return mla.lib().moe_lora_align(a["topk_ids"], a["mapping"], a["M"], a["topk"], a["E"],
                                    a["L"], a["B"], a["sorted"], a["eids"], a["ntpp"],
                                    a["lora_ids"], a["nact"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(topk_ids=None), mla.ERR_INVALID),
    (dict(M=0, ntpp=None), mla.ERR_INVALID),
    (dict(mapping=None), mla.ERR_INVALID),
    (dict(sorted=None), mla.ERR_INVALID),
    (dict(eids=None), mla.ERR_INVALID),
    (dict(ntpp=None), mla.ERR_INVALID),
    (dict(M=-1), mla.ERR_INVALID),
    (dict(topk=0), mla.ERR_INVALID),
    (dict(E=0), mla.ERR_INVALID),
    (dict(L=0), mla.ERR_INVALID),
    (dict(E=1025), mla.ERR_UNSUPPORTED),
    (dict(L=1025, E=1), mla.ERR_UNSUPPORTED),
    (dict(B=8), mla.ERR_UNSUPPORTED),
    (dict(B=48), mla.ERR_UNSUPPORTED),
    (dict(M=2 ** 31, topk=1), mla.ERR_UNSUPPORTED),
    (dict(M=65536, topk=8, E=256, L=16, B=64), mla.ERR_WORKSPACE),
    (dict(M=65536, topk=8, E=256, L=16, B=64, ws=P16, ws_bytes=100), mla.ERR_WORKSPACE),
    (dict(ws_bytes=-1), mla.ERR_INVALID),
])
def test_align_rejects(kw, status):
    assert align_call(**kw) == status


def align_noalloc_call(**kw):
    args = dict(topk_ids=P16, mapping=P16, M=16, topk=4, E=32, L=6, B=16, sorted=P16,
                eids=P16, ntpp=P16, lora_ids=None, nact=None)
    args.update(kw)
    a = args
    return mla.lib().moe_lora_align_noalloc(a["topk_ids"], a["mapping"], a["M"], a["topk"],
                                            a["E"], a["L"], a["B"], a["sorted"], a["eids"],
                                            a["ntpp"], a["lora_ids"], a["nact"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(topk_ids=None), mla.ERR_INVALID),
    (dict(ntpp=None), mla.ERR_INVALID),
    (dict(sorted=None), mla.ERR_INVALID),
    (dict(M=-1), mla.ERR_INVALID),
    (dict(E=1025), mla.ERR_UNSUPPORTED),
    (dict(B=48), mla.ERR_UNSUPPORTED),
    (dict(L=1025, E=1), mla.ERR_UNSUPPORTED),
])
def test_align_noalloc_rejects(kw, status):
    assert align_noalloc_call(**kw) == status


def test_align_noalloc_scratch_covers_every_accepted_size():
    """The static scratch of the no-allocation align holds the workspace of the largest
    problems the limits admit (the tile path's per-tile counts are capped)."""
    assert mla.ALIGN_NOALLOC_SCRATCH_BYTES == 8 * 1024 * 1024
    for M, topk, E, L, B in ((65536, 8, 256, 16, 64), (2 ** 22, 8, 1024, 8, 128),
                             (2 ** 20, 1, 1, 1024, 16), (10 ** 6, 1, 1024, 8, 16),
                             (5000, 4, 2, 1, 16), (8192, 8, 1024, 1024, 128),
                             (65536, 8, 256, 64, 64)):
        assert mla.align_workspace_size(M, topk, E, L, B) <= mla.ALIGN_NOALLOC_SCRATCH_BYTES


def test_align_takes_every_key_space_in_passes():
    """Every L <= 1024 and E <= 1024 is accepted (up to 2^20 (slot, expert)
    keys).  Key spaces beyond the 8192 keys of one pass's LDS tables are
    aligned in passes over slot ranges, each sized like a call with that many
    slots: the workspace of a call with L slots is that of a call with
    8192 / E slots."""
    ws = mla.align_workspace_size
    assert ws(65536, 8, 256, 64, 64) == ws(65536, 8, 256, 32, 64)
    assert ws(65536, 8, 1024, 1024, 64) == ws(65536, 8, 1024, 8, 64)
    assert ws(8192, 8, 1024, 1024, 128) == ws(8192, 8, 1024, 8, 128)
    # one pass up to 8192 keys: unchanged
    assert ws(65536, 8, 256, 32, 64) == (128 + 1) * 8192 * 4   # 2^20 / 8192 tiles
    # decode batches (at most 64 pairs and 64 slots) take the one-wavefront path at any E
    assert ws(16, 4, 1024, 64, 16) == 0


def fused_call(**kw):
    a = dict(x=P16, xpp=0, la=P16, lb=P16, sorted=P16, eids=P16, ntpp=P16, w=None, mul=0,
             add=1, M=16, topk=4, K=2880, Ns=2880, S=2, E=32, L=6, r=64, B=16, y=P16,
             variant=0, act=None)
    a.update(kw)
    act = a["L"] if a["act"] is None else a["act"]
    return mla.lib().fused_moe_lora(a["x"], a["xpp"], a["la"], a["lb"], a["sorted"], a["eids"],
                                    a["ntpp"], act, a["w"], a["mul"], a["add"], a["M"],
                                    a["topk"], a["K"], a["Ns"], a["S"], a["E"], a["L"], a["r"],
                                    a["B"], a["y"], a["variant"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), mla.ERR_INVALID),
    (dict(la=None), mla.ERR_INVALID),
    (dict(lb=None), mla.ERR_INVALID),
    (dict(y=None), mla.ERR_INVALID),
    (dict(sorted=None), mla.ERR_INVALID),
    (dict(mul=1, w=None), mla.ERR_INVALID),
    (dict(mul=2), mla.ERR_INVALID),
    (dict(add=-1), mla.ERR_INVALID),
    (dict(xpp=3), mla.ERR_INVALID),
    (dict(variant=7), mla.ERR_INVALID),
    (dict(K=2884), mla.ERR_INVALID),
    (dict(Ns=2881), mla.ERR_INVALID),
    (dict(K=0), mla.ERR_INVALID),
    (dict(S=0), mla.ERR_INVALID),
    (dict(r=0), mla.ERR_INVALID),
    (dict(r=129), mla.ERR_UNSUPPORTED),
    (dict(E=1025), mla.ERR_UNSUPPORTED),
    (dict(B=24), mla.ERR_UNSUPPORTED),
    (dict(x=V(24)), mla.ERR_INVALID),
    (dict(y=V(18)), mla.ERR_INVALID),
    (dict(M=0), mla.OK),
    (dict(M=0, x=None, y=None, sorted=None, eids=None), mla.OK),
    (dict(act=-1), mla.ERR_INVALID),
    (dict(act=7), mla.ERR_INVALID),
    # no active slot: nothing is launched or read, not even the pointers
    (dict(act=0), mla.OK),
    (dict(act=0, x=None, la=None, lb=None, y=None, sorted=None, eids=None, ntpp=None), mla.OK),
])
def test_fused_rejects(kw, status):
    assert fused_call(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(r=0), mla.ERR_INVALID),
    (dict(r=129), mla.ERR_UNSUPPORTED),
    (dict(E=1025), mla.ERR_UNSUPPORTED),
    (dict(B=24), mla.ERR_UNSUPPORTED),
    (dict(K=2884), mla.ERR_INVALID),
    (dict(xpp=2), mla.ERR_INVALID),
    (dict(variant=3), mla.ERR_INVALID),
    (dict(variant=mla.VARIANT_MFMA, r=12), mla.ERR_UNSUPPORTED),
    # x above 2 GiB: M * K * 2 = 2^31 + 2^14 bytes
    (dict(variant=mla.VARIANT_MFMA, M=262145, K=4096), mla.ERR_UNSUPPORTED),
    (dict(S=0), mla.ERR_INVALID),
])
def test_variant_query_rejects_like_fused(kw, status):
    a = dict(M=16, topk=4, K=2880, Ns=2880, S=2, E=32, L=6, r=64, B=16, xpp=0, variant=0)
    a.update(kw)
    assert status != mla.OK  # fused_call below must not reach a launch
    assert mla.lib().fused_moe_lora_variant(a["M"], a["topk"], a["K"], a["Ns"], a["S"], a["E"],
                                            a["L"], a["r"], a["B"], a["xpp"],
                                            a["variant"]) == status
    assert fused_call(**a) == status


def naive_call(**kw):
    a = dict(x=P16, xpp=0, la=P16, lb=P16, ids=P16, mapping=P16, w=None, mul=0, add=1, M=16,
             topk=4, K=2880, Ns=2880, S=2, E=32, L=6, r=64, B=16, y=P16, variant=0)
    a.update(kw)
    return mla.lib().fused_moe_lora_naive(a["x"], a["xpp"], a["la"], a["lb"], a["ids"],
                                          a["mapping"], a["w"], a["mul"], a["add"], a["M"],
                                          a["topk"], a["K"], a["Ns"], a["S"], a["E"], a["L"],
                                          a["r"], a["B"], a["y"], a["variant"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), mla.ERR_INVALID),
    (dict(la=None), mla.ERR_INVALID),
    (dict(lb=None), mla.ERR_INVALID),
    (dict(ids=None), mla.ERR_INVALID),
    (dict(mapping=None), mla.ERR_INVALID),
    (dict(y=None), mla.ERR_INVALID),
    (dict(mul=1, w=None), mla.ERR_INVALID),
    (dict(mul=2), mla.ERR_INVALID),
    (dict(add=3), mla.ERR_INVALID),
    (dict(xpp=-1), mla.ERR_INVALID),
    (dict(K=2884), mla.ERR_INVALID),
    (dict(Ns=4), mla.ERR_INVALID),
    (dict(S=0), mla.ERR_INVALID),
    (dict(r=0), mla.ERR_INVALID),
    (dict(M=-1), mla.ERR_INVALID),
    (dict(topk=0), mla.ERR_INVALID),
    (dict(r=129), mla.ERR_UNSUPPORTED),
    (dict(E=1025), mla.ERR_UNSUPPORTED),
    (dict(L=1025, E=1), mla.ERR_UNSUPPORTED),
    # block sizes: powers of two from 1 to 128
    (dict(B=0), mla.ERR_UNSUPPORTED),
    (dict(B=3), mla.ERR_UNSUPPORTED),
    (dict(B=24), mla.ERR_UNSUPPORTED),
    (dict(B=256), mla.ERR_UNSUPPORTED),
    # more pairs than one workgroup groups
    (dict(M=257, topk=4), mla.ERR_UNSUPPORTED),
    (dict(M=1025, topk=1), mla.ERR_UNSUPPORTED),
    (dict(x=V(24)), mla.ERR_INVALID),
    (dict(la=V(40)), mla.ERR_INVALID),
    (dict(variant=3), mla.ERR_INVALID),
    (dict(variant=-1), mla.ERR_INVALID),
    # the MFMA kernel: r a multiple of 8, blocks of at least 16 pairs
    (dict(variant=mla.VARIANT_MFMA, r=12), mla.ERR_UNSUPPORTED),
    (dict(variant=mla.VARIANT_MFMA, B=8), mla.ERR_UNSUPPORTED),
    (dict(M=0), mla.OK),
    (dict(M=0, x=None, y=None, ids=None, mapping=None), mla.OK),
])
def test_naive_rejects(kw, status):
    assert naive_call(**kw) == status


def test_naive_binding_checks_before_calling():
    torch = pytest.importorskip("torch")
    bf = dict(dtype=torch.bfloat16)
    x, y = torch.zeros((4, 64), **bf), torch.zeros((4, 2, 32), **bf)
    a, b = torch.zeros((1, 2, 8, 8, 64), **bf), torch.zeros((1, 2, 8, 32, 8), **bf)
    ids, mp = torch.zeros((4, 2), dtype=torch.int32), torch.zeros(4, dtype=torch.int32)
    with pytest.raises(TypeError):
        mla.fused_moe_lora_naive(x, a, b, ids.long(), mp, None, y, mul_routed_weight=False,
                                 add_inputs=True)
    with pytest.raises(ValueError):
        mla.fused_moe_lora_naive(x, a, b, ids[:, :1].contiguous(), mp, None, y,
                                 mul_routed_weight=False, add_inputs=True)
    with pytest.raises(ValueError):
        mla.fused_moe_lora_naive(x, a, b, ids, mp[:3].contiguous(), None, y,
                                 mul_routed_weight=False, add_inputs=True)


def wa_call(**kw):
    a = dict(ids=P16, mp=P16, M=16, topk=4, E=32, L=6, B=16, sorted=P16, eids=P16, ntpp=P16,
             lids=P16, nact=P16, x=P16, xpp=0, la=P16, lb=P16, w=None, mul=0, add=1, K=2880,
             Ns=2880, S=2, r=64, y=P16, variant=0)
    a.update(kw)
    return mla.lib().fused_moe_lora_with_align(
        a["ids"], a["mp"], a["M"], a["topk"], a["E"], a["L"], a["B"], a["sorted"], a["eids"],
        a["ntpp"], a["lids"], a["nact"], a["x"], a["xpp"], a["la"], a["lb"], a["w"], a["mul"],
        a["add"], a["K"], a["Ns"], a["S"], a["r"], a["y"], a["variant"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=17), mla.ERR_UNSUPPORTED),            # 68 pairs: beyond the one-wavefront align
    (dict(L=65, E=2), mla.ERR_UNSUPPORTED),       # 65 slots
    (dict(B=8), mla.ERR_UNSUPPORTED),             # block_m as moe_lora_align takes it
    (dict(ntpp=None), mla.ERR_INVALID),
    (dict(sorted=None), mla.ERR_INVALID),
    (dict(x=None), mla.ERR_INVALID),
    (dict(ids=None), mla.ERR_INVALID),
    (dict(y=V(18)), mla.ERR_INVALID),
    (dict(mul=1, w=None), mla.ERR_INVALID),
    (dict(mul=2), mla.ERR_INVALID),
    (dict(K=2884), mla.ERR_INVALID),
    (dict(r=129), mla.ERR_UNSUPPORTED),
    (dict(variant=5), mla.ERR_INVALID),
])
def test_with_align_rejects(kw, status):
    assert wa_call(**kw) == status


def ws_call(**kw):
    a = dict(x=P16, xpp=0, la=P16, lb=P16, sorted=P16, eids=P16, ntpp=P16, w=None, mul=0,
             add=1, M=16, topk=4, K=2880, Ns=2880, S=2, E=32, L=6, r=64, B=16, y=P16,
             variant=1, ws=P16, ws_bytes=1 << 40, wait=-1, act=None)
    a.update(kw)
    act = a["L"] if a["act"] is None else a["act"]
    return mla.lib().fused_moe_lora_ws(a["x"], a["xpp"], a["la"], a["lb"], a["sorted"],
                                       a["eids"], a["ntpp"], act, a["w"], a["mul"], a["add"],
                                       a["M"], a["topk"], a["K"], a["Ns"], a["S"], a["E"], a["L"],
                                       a["r"], a["B"], a["y"], a["variant"], a["ws"],
                                       a["ws_bytes"], a["wait"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), mla.ERR_INVALID),
    (dict(sorted=None), mla.ERR_INVALID),
    (dict(y=V(18)), mla.ERR_INVALID),
    (dict(r=129), mla.ERR_UNSUPPORTED),
    (dict(K=2884), mla.ERR_INVALID),
    (dict(variant=3), mla.ERR_INVALID),
    (dict(ws_bytes=-1), mla.ERR_INVALID),
    # the decode stream kernel takes this shape and needs the exchange area
    (dict(ws=None), mla.ERR_WORKSPACE),
    (dict(ws_bytes=4096), mla.ERR_WORKSPACE),
    (dict(ws=V(24)), mla.ERR_WORKSPACE),
    (dict(M=0), mla.OK),
    (dict(M=0, x=None, y=None, sorted=None, ws=None, ws_bytes=0), mla.OK),
    (dict(act=-1), mla.ERR_INVALID),
    (dict(act=7), mla.ERR_INVALID),
    (dict(act=7, ws=None), mla.ERR_WORKSPACE),
    (dict(act=0, x=None, y=None, sorted=None, ntpp=None, ws=None, ws_bytes=0), mla.OK),
])
def test_fused_ws_rejects(kw, status):
    assert ws_call(**kw) == status


def test_fused_workspace_query():
    q = mla.fused_moe_lora_workspace_bytes
    # the decode stream kernel's K split: one slot per (unit, 4-row pass) bound;
    # a slot holds 8 peers x 4 rows x 128 ranks of 8-byte words whatever the
    # rank, after the slots' tag words (8 peers x 4 bytes each)
    slot = 8 * 4 * 128 * 8

    def area(n):
        return (32 * n + 15) // 16 * 16 + n * slot
    b = q(16, 4, 2880, 2880, 2, 32, 6, 64, 16, False, "valu")       # stream kernel
    units = (64 + 64 * 15) // 16 * 2                                  # block bound x slices
    assert b == area(units * 4)
    assert q(16, 4, 2880, 2880, 2, 32, 6, 128, 16, False, "valu") == b  # rank-free layout
    assert q(16, 4, 2880, 2880, 2, 32, 6, 64, 32, False, "valu") > b    # more passes per block
    assert q(8, 4, 2880, 2880, 2, 128, 4, 32, 16, False, "valu") == area((32 + 32 * 15) // 16 * 2 * 4)
    # kernels without the K split need none
    assert q(16, 2, 256, 128, 1, 8, 2, 8, 16) == 0                    # register-batch kernel
    assert q(16, 4, 2880, 2880, 2, 32, 6, 64, 16, False, "mfma") == 0
    assert q(8192, 8, 2048, 768, 2, 128, 8, 128, 64) == 0            # MFMA prefill
    assert q(0, 4, 2880, 2880, 2, 32, 6, 64, 16) == 0
    with pytest.raises(mla.MoeLoraError):
        q(16, 4, 2880, 2880, 2, 32, 6, 129, 16)


def two_call(**kw):
    a = dict(x=P16, xpp=0, la=P16, lb=P16, sorted=P16, eids=P16, ntpp=P16, w=None, mul=0,
             add=1, M=16, topk=4, K=2880, Ns=2880, S=2, E=32, L=6, r=256, B=16, y=P16,
             ws=P16, ws_bytes=1 << 40, act=None)
    a.update(kw)
    act = a["L"] if a["act"] is None else a["act"]
    return mla.lib().fused_moe_lora_two_kernel(a["x"], a["xpp"], a["la"], a["lb"], a["sorted"],
                                               a["eids"], a["ntpp"], act, a["w"], a["mul"],
                                               a["add"], a["M"], a["topk"], a["K"], a["Ns"],
                                               a["S"], a["E"], a["L"], a["r"], a["B"], a["y"],
                                               a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), mla.ERR_INVALID),
    (dict(la=None), mla.ERR_INVALID),
    (dict(lb=None), mla.ERR_INVALID),
    (dict(sorted=None), mla.ERR_INVALID),
    (dict(y=None), mla.ERR_INVALID),
    (dict(mul=1, w=None), mla.ERR_INVALID),
    (dict(add=2), mla.ERR_INVALID),
    (dict(xpp=5), mla.ERR_INVALID),
    (dict(K=2884), mla.ERR_INVALID),
    (dict(r=0), mla.ERR_INVALID),
    (dict(S=0), mla.ERR_INVALID),
    (dict(ws_bytes=-1), mla.ERR_INVALID),
    (dict(r=513), mla.ERR_UNSUPPORTED),
    (dict(E=1025), mla.ERR_UNSUPPORTED),
    (dict(B=8), mla.ERR_UNSUPPORTED),
    # an A matrix above 2 GiB: r * K * 2 = 2^31 + 2^13
    (dict(r=512, K=2 ** 21 + 8, Ns=64), mla.ERR_UNSUPPORTED),
    (dict(ws=None), mla.ERR_WORKSPACE),
    (dict(ws_bytes=1024), mla.ERR_WORKSPACE),
    (dict(ws=V(24)), mla.ERR_WORKSPACE),
    (dict(x=V(24)), mla.ERR_INVALID),
    (dict(M=0), mla.OK),
    (dict(M=0, x=None, y=None, sorted=None, ws=None), mla.OK),
    (dict(act=-1), mla.ERR_INVALID),
    (dict(act=7), mla.ERR_INVALID),
    (dict(act=0, x=None, la=None, y=None, ntpp=None, ws=None), mla.OK),
])
def test_two_kernel_rejects(kw, status):
    assert two_call(**kw) == status


def test_two_kernel_workspace_query():
    q = mla.two_kernel_workspace_bytes
    # fp32 rank vectors of every pair and slice, once per K split
    b = q(16, 4, 2880, 2880, 2, 32, 6, 256, 16)
    assert b > 0 and b % (2 * 64 * 256 * 4) == 0 and b // (2 * 64 * 256 * 4) <= 8
    # a large batch needs no K split
    assert q(8192, 8, 2048, 768, 2, 128, 8, 128, 64) == 2 * 65536 * 128 * 4
    assert q(0, 4, 2880, 2880, 2, 32, 6, 64, 16) == 0
    with pytest.raises(mla.MoeLoraError):
        q(16, 4, 2880, 2880, 2, 32, 6, 513, 16)


@pytest.mark.parametrize("args,status", [
    ((None, P16, 8), mla.ERR_INVALID),
    ((P16, None, 8), mla.ERR_INVALID),
    ((P16, P16, -1), mla.ERR_INVALID),
    ((V(24), P16, 8), mla.ERR_INVALID),
    ((P16, V(40), 8), mla.ERR_INVALID),
    ((P16, P16, 0), mla.OK),
    ((None, None, 0), mla.OK),
])
def test_accumulate_rejects(args, status):
    y, d, n = args
    assert mla.lib().moe_lora_accumulate(y, d, n, None) == status


def test_variant_query_resolves_auto():
    fv = mla.fused_variant
    # decode: about two rows per (slot, expert) group -> vector kernel
    assert fv(16, 4, 2880, 2880, 2, 32, 6, 64, 16) == "valu"
    # dense prefill blocks with a large rank -> MFMA kernel
    assert fv(8192, 8, 2048, 768, 2, 128, 8, 128, 64) == "mfma"
    # MFMA needs r % 8 == 0, so AUTO never picks it otherwise
    assert fv(8192, 8, 2048, 768, 2, 128, 8, 100, 64) == "valu"
    # from half a row per (slot, expert) group on, small ranks take MFMA too
    assert fv(2048, 4, 2880, 2880, 2, 128, 4, 8, 64) == "mfma"
    assert fv(64, 4, 2880, 2880, 2, 128, 4, 8, 64) == "mfma"
    assert fv(63, 4, 2880, 2880, 2, 128, 4, 8, 64) == "valu"
    # rank 16 (512-thread vector kernel) above two rows per group
    assert fv(2048, 4, 2880, 2880, 2, 128, 4, 16, 64) == "mfma"
    assert fv(257, 4, 2880, 2880, 2, 128, 4, 16, 64) == "mfma"
    assert fv(256, 4, 2880, 2880, 2, 128, 4, 16, 64) == "valu"
    # an x above 2 GiB keeps AUTO on the vector kernel
    assert fv(262145, 8, 4096, 768, 2, 128, 8, 128, 64) == "valu"
    # so does a y above 2 GiB (M * topk * S * Ns * 2 = 2^31 + 2^16 bytes)
    assert fv(65537, 8, 256, 1024, 2, 128, 8, 128, 64) == "valu"
    assert fv(16, 4, 2880, 2880, 2, 32, 6, 64, 16, variant="mfma") == "mfma"
    assert fv(8192, 8, 2048, 768, 2, 128, 8, 128, 64, variant="valu") == "valu"


def test_kernel_name_query():
    kn = mla.fused_kernel_name
    # 20b-like decode (r = 64, K = 2880): the stream kernel
    assert kn(16, 4, 2880, 2880, 2, 32, 6, 64, 16) == "fused_stream_kernel"
    # r = 16 decode and K past the stream kernel's X staging: register batches
    assert kn(8, 4, 2880, 2880, 2, 128, 4, 16, 16) == "fused_valu_kernel"
    assert kn(16, 4, 4104, 2880, 2, 32, 6, 64, 16) == "fused_valu_kernel"
    assert kn(8192, 8, 2048, 768, 2, 128, 8, 128, 64) == "fused_mfma_kernel"
    assert mla.lib().fused_moe_lora_kernel_name(16, 4, 2880, 2880, 2, 32, 6, 129, 16, 0, 0) is None


def test_binding_checks_dtypes_before_calling():
    torch = pytest.importorskip("torch")
    with pytest.raises(TypeError):
        mla.moe_lora_align(torch.zeros((4, 2), dtype=torch.int64), torch.zeros(4, dtype=torch.int32),
                           8, 2, 16)
    with pytest.raises(ValueError):
        mla.moe_lora_align(torch.zeros((4, 2), dtype=torch.int32)[:, :1],
                           torch.zeros(4, dtype=torch.int32), 8, 2, 16)


def test_missing_library_fails_loudly(tmp_path):
    saved = mla._lib
    try:
        mla._lib = None
        with pytest.raises(RuntimeError, match="no fallback"):
            mla.lib(str(tmp_path / "nope.so"))
    finally:
        mla._lib = saved


def test_product_package_does_not_import_oracle():
    pkg = os.path.join(ROOT, "moe_lora_adapter_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "oracle.c" not in text, f
