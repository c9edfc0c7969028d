"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C ABI binding, compare with the oracle."""

from __future__ import annotations

import numpy as np
import torch

import moe_lora_adapter_amd as mla
from moe_lora_adapter_amd.synth import bf16_bits_to_f32

DEV = torch.device("cuda:0")

# |gpu - oracle| <= TOL * (1 + |oracle|), elementwise, on the bf16 output
TOL = 1e-2


def bf16_dev(a: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(DEV).view(torch.bfloat16)


def i32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def bf16_host_f64(t: torch.Tensor) -> np.ndarray:
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return bf16_bits_to_f32(bits).astype(np.float64)


def run_align(topk_ids, mapping, E, L, B):
    out = mla.moe_lora_align(i32_dev(topk_ids), i32_dev(mapping), E, L, B)
    torch.cuda.synchronize()
    return out


def align_to_host(out):
    return {"sorted_token_ids": out.sorted_token_ids.cpu().numpy(),
            "expert_ids": out.expert_ids.cpu().numpy(),
            "num_tokens_post_padded": out.num_tokens_post_padded.cpu().numpy(),
            "lora_ids": out.lora_ids.cpu().numpy(),
            "num_active": int(out.num_active_loras.cpu().numpy()[0]),
            "cap": out.cap}


def assert_align_equal(gpu, ref, B):
    """Bit-exact on everything the align step defines (each slot's prefix)."""
    assert gpu["cap"] == ref["cap"]
    np.testing.assert_array_equal(gpu["num_tokens_post_padded"], ref["num_tokens_post_padded"])
    for l, n in enumerate(ref["num_tokens_post_padded"]):
        np.testing.assert_array_equal(gpu["sorted_token_ids"][l, :n], ref["sorted_token_ids"][l, :n],
                                      err_msg=f"sorted_token_ids slot {l}")
        np.testing.assert_array_equal(gpu["expert_ids"][l, :n // B], ref["expert_ids"][l, :n // B],
                                      err_msg=f"expert_ids slot {l}")
    np.testing.assert_array_equal(gpu["lora_ids"], ref["lora_ids"])
    assert gpu["num_active"] == ref["num_active"]


class DeviceCase:
    """A drawn Case moved to the device."""

    def __init__(self, case):
        s = case.shape
        self.case = case
        self.s = s
        self.topk_ids = i32_dev(case.topk_ids)
        self.mapping = i32_dev(case.token_lora_mapping)
        self.w = f32_dev(case.topk_weights)
        self.x = bf16_dev(case.x)
        self.a = bf16_dev(case.lora_a)
        self.b = bf16_dev(case.lora_b)
        self.y_in = bf16_dev(case.y_in)

    def align(self):
        s = self.s
        return mla.moe_lora_align(self.topk_ids, self.mapping, s.E, s.L, s.block_m)

    def fused(self, align=None, variant="auto", y=None, add=None, mul=None, b=None, a=None,
              max_active=None):
        s = self.s
        align = align if align is not None else self.align()
        y = self.y_in.clone() if y is None else y
        mla.fused_moe_lora(self.x, self.a if a is None else a, self.b if b is None else b, align,
                           self.w, y, mul_routed_weight=s.mul if mul is None else mul,
                           add_inputs=s.add if add is None else add,
                           x_per_pair=s.x_per_pair, variant=variant,
                           max_active_loras=max_active)
        torch.cuda.synchronize()
        return y


    def naive(self, block_m=None, y=None, add=None, mul=None, b=None, a=None, variant="auto"):
        """The align-free path (fused_moe_lora_naive) on the same inputs."""
        s = self.s
        y = self.y_in.clone() if y is None else y
        mla.fused_moe_lora_naive(self.x, self.a if a is None else a, self.b if b is None else b,
                                 self.topk_ids, self.mapping, self.w, y,
                                 mul_routed_weight=s.mul if mul is None else mul,
                                 add_inputs=s.add if add is None else add,
                                 block_m=s.block_m if block_m is None else block_m,
                                 x_per_pair=s.x_per_pair, variant=variant)
        torch.cuda.synchronize()
        return y


def valid_pairs(case) -> np.ndarray:
    s = case.shape
    slot = np.repeat(case.token_lora_mapping, s.topk)
    e = case.topk_ids.reshape(-1)
    return (slot >= 0) & (slot < s.L) & (e >= 0) & (e < s.E)


def assert_fused_close(gpu_rows: np.ndarray, ref_rows: np.ndarray, what: str = ""):
    err = np.abs(gpu_rows - ref_rows)
    bound = TOL * (1.0 + np.abs(ref_rows))
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first {idx.tolist()}: "
            f"gpu {gpu_rows[bad][:5]} oracle {ref_rows[bad][:5]}")


def assert_delta_close(gpu_rows, ref_rows, base_rows, what="", rel=1e-2):
    """Stricter, normwise check on the delta itself (gpu - base vs oracle - base)."""
    dg = gpu_rows - base_rows
    dr = ref_rows - base_rows
    num = np.linalg.norm(dg - dr)
    den = np.linalg.norm(dr)
    assert den > 0, what
    assert num <= rel * den, f"{what}: delta rel error {num / den:.3e}"
