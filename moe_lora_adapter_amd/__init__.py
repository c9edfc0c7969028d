"""MI355X-native MoE-LoRA hot path: Python binding of libmoelora.so.

The binding only marshals arguments: every step of the path runs in the HIP
kernels behind the C ABI declared in include/moe_lora.h.  PyTorch provides
device memory and the current stream.  If the library is not built the calls
raise; there is no fallback implementation.

    out = moe_lora_align(topk_ids, token_lora_mapping, E, L, block_m)
    fused_moe_lora(x, lora_a, lora_b, out, topk_weights, y,
                   mul_routed_weight=..., add_inputs=..., x_per_pair=...)
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoelora.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
VARIANT_AUTO, VARIANT_VALU, VARIANT_MFMA = 0, 1, 2
VARIANTS = {"auto": VARIANT_AUTO, "valu": VARIANT_VALU, "mfma": VARIANT_MFMA}

# symbol -> (restype, argtypes); mirrors include/moe_lora.h
_P = ctypes.c_void_p
_I32, _I64 = ctypes.c_int32, ctypes.c_int64
SIGNATURES = {
    "moe_lora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_lora_align_capacity": (_I64, [_I64, _I32, _I32, _I32]),
    "moe_lora_align_workspace_size": (_I64, [_I64, _I32, _I32, _I32, _I32]),
    "moe_lora_align": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P,
                                      _P, _P, _P, _I64, _P]),
    "moe_lora_align_noalloc": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P,
                                              _P, _P, _P, _P]),
    "fused_moe_lora": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _I64,
                                      _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P,
                                      _I32, _P]),
    "fused_moe_lora_with_align": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P,
                                                 _P, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32,
                                                 _I32, _I32, _I32, _I32, _P, _I32, _P]),
    "fused_moe_lora_ws": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32,
                                         _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                         _P, _I32, _P, _I64, _I32, _P]),
    "fused_moe_lora_workspace_bytes": (_I64, [_I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                              _I32, _I32, _I32]),
    "fused_moe_lora_variant": (ctypes.c_int, [_I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                              _I32, _I32, _I32]),
    "fused_moe_lora_kernel_name": (ctypes.c_char_p, [_I64, _I32, _I32, _I32, _I32, _I32, _I32,
                                                     _I32, _I32, _I32, _I32]),
    "fused_moe_lora_naive": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _P, _I32, _I32, _I64,
                                            _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P,
                                            _I32, _P]),
    "fused_moe_lora_two_kernel_workspace_bytes": (_I64, [_I64, _I32, _I32, _I32, _I32, _I32, _I32,
                                                         _I32, _I32, _I32]),
    "fused_moe_lora_two_kernel": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _P, _I32, _P, _I32,
                                                 _I32, _I64, _I32, _I32, _I32, _I32, _I32, _I32,
                                                 _I32, _I32, _P, _P, _I64, _P]),
    "moe_lora_accumulate": (ctypes.c_int, [_P, _P, _I64, _P]),
}

NAIVE_MAX_PAIRS = 1024        # MOE_LORA_NAIVE_MAX_PAIRS
WITH_ALIGN_MAX_PAIRS = 64     # MOE_LORA_WITH_ALIGN_MAX_PAIRS
WITH_ALIGN_MAX_SLOTS = 64     # MOE_LORA_WITH_ALIGN_MAX_SLOTS
TWO_KERNEL_MAX_RANK = 512     # MOE_LORA_TWO_KERNEL_MAX_RANK


class MoeLoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def lib(path: str = LIB_PATH) -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m moe_lora_adapter_amd.build` "
                "(or __graft_entry__.build()); there is no fallback path")
        handle = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().moe_lora_status_string(int(status)).decode()


def align_capacity(M: int, topk: int, E: int, block_m: int) -> int:
    v = lib().moe_lora_align_capacity(M, topk, E, block_m)
    if v < 0:
        raise MoeLoraError(v, "moe_lora_align_capacity")
    return int(v)


def align_workspace_size(M: int, topk: int, E: int, L: int, block_m: int) -> int:
    v = lib().moe_lora_align_workspace_size(M, topk, E, L, block_m)
    if v < 0:
        raise MoeLoraError(v, "moe_lora_align_workspace_size")
    return int(v)


def fused_variant(M: int, topk: int, K: int, Ns: int, S: int, E: int, L: int, r: int,
                  block_m: int, x_per_pair: bool = False, variant: str | int = "auto") -> str:
    """Name of the kernel ("valu" or "mfma") fused_moe_lora runs for these sizes."""
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    rc = lib().fused_moe_lora_variant(M, topk, K, Ns, S, E, L, r, block_m, int(bool(x_per_pair)),
                                      v)
    if rc < 0:
        raise MoeLoraError(rc, "fused_moe_lora_variant")
    return {VARIANT_VALU: "valu", VARIANT_MFMA: "mfma"}[rc]


def fused_kernel_name(M: int, topk: int, K: int, Ns: int, S: int, E: int, L: int, r: int,
                      block_m: int, x_per_pair: bool = False, variant: str | int = "auto") -> str:
    """Name of the GPU kernel fused_moe_lora launches for these sizes."""
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    args = (M, topk, K, Ns, S, E, L, r, block_m, int(bool(x_per_pair)), v)
    name = lib().fused_moe_lora_kernel_name(*args)
    if name is None:
        raise MoeLoraError(lib().fused_moe_lora_variant(*args), "fused_moe_lora_kernel_name")
    return name.decode()


@dataclass
class AlignOutput:
    sorted_token_ids: "object"        # int32 [L, cap]
    expert_ids: "object"              # int32 [L, cap // block_m]
    num_tokens_post_padded: "object"  # int32 [L]
    lora_ids: "object"                # int32 [L]
    num_active_loras: "object"        # int32 [1]
    block_m: int
    cap: int


def _dptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(t, name, dtype, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def alloc_align_output(M, topk, E, L, block_m, device):
    import torch
    cap = align_capacity(M, topk, E, block_m)
    i32 = dict(dtype=torch.int32, device=device)
    return AlignOutput(torch.empty((L, cap), **i32), torch.empty((L, cap // block_m), **i32),
                       torch.empty(L, **i32), torch.empty(L, **i32), torch.empty(1, **i32),
                       block_m, cap)


def moe_lora_align(topk_ids, token_lora_mapping, E: int, L: int, block_m: int, *,
                   out: AlignOutput | None = None, workspace=None, stream=None) -> AlignOutput:
    """Group the (token, k) pairs of every LoRA slot by expert; see moe_lora.h."""
    import torch
    dev = topk_ids.device
    _check(topk_ids, "topk_ids", torch.int32, dev)
    _check(token_lora_mapping, "token_lora_mapping", torch.int32, dev)
    if topk_ids.dim() != 2 or token_lora_mapping.shape != (topk_ids.shape[0],):
        raise ValueError("topk_ids must be [M, topk] and token_lora_mapping [M]")
    M, topk = topk_ids.shape
    if out is None:
        out = alloc_align_output(M, topk, E, L, block_m, dev)
    ws_bytes = align_workspace_size(M, topk, E, L, block_m)
    if ws_bytes > 0 and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    rc = lib().moe_lora_align(
        _dptr(topk_ids), _dptr(token_lora_mapping), M, topk, E, L, block_m,
        _dptr(out.sorted_token_ids), _dptr(out.expert_ids), _dptr(out.num_tokens_post_padded),
        _dptr(out.lora_ids), _dptr(out.num_active_loras), _dptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream_ptr(stream))
    if rc != OK:
        raise MoeLoraError(rc, "moe_lora_align")
    return out


ALIGN_NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024   # MOE_LORA_ALIGN_NOALLOC_SCRATCH_BYTES


def moe_lora_align_noalloc(topk_ids, token_lora_mapping, E: int, L: int, block_m: int, *,
                           out: AlignOutput, stream=None) -> AlignOutput:
    """moe_lora_align with the library's own per-GPU scratch instead of a workspace: the
    call allocates nothing (out must be given).  Calls that may overlap on one GPU race;
    see moe_lora.h."""
    import torch
    dev = topk_ids.device
    _check(topk_ids, "topk_ids", torch.int32, dev)
    _check(token_lora_mapping, "token_lora_mapping", torch.int32, dev)
    if topk_ids.dim() != 2 or token_lora_mapping.shape != (topk_ids.shape[0],):
        raise ValueError("topk_ids must be [M, topk] and token_lora_mapping [M]")
    M, topk = topk_ids.shape
    rc = lib().moe_lora_align_noalloc(
        _dptr(topk_ids), _dptr(token_lora_mapping), M, topk, E, L, block_m,
        _dptr(out.sorted_token_ids), _dptr(out.expert_ids), _dptr(out.num_tokens_post_padded),
        _dptr(out.lora_ids), _dptr(out.num_active_loras), _stream_ptr(stream))
    if rc != OK:
        raise MoeLoraError(rc, "moe_lora_align_noalloc")
    return out


def _fused_shapes(x, lora_a, lora_b, topk_weights, y, x_per_pair):
    """Checks the tensors of a fused call; returns (M, topk, K, Ns, S, E, L, r)."""
    import torch
    dev = y.device
    _check(x, "x", torch.bfloat16, dev)
    _check(lora_a, "lora_a", torch.bfloat16, dev)
    _check(lora_b, "lora_b", torch.bfloat16, dev)
    _check(y, "y", torch.bfloat16, dev)
    if topk_weights is not None:
        _check(topk_weights, "topk_weights", torch.float32, dev)
    if lora_a.dim() != 5 or lora_b.dim() != 5 or y.dim() != 3:
        raise ValueError("lora_a [S,L,E,r,K], lora_b [S,L,E,Ns,r], y [M,topk,S*Ns]")
    S, L, E, r, K = lora_a.shape
    Ns = lora_b.shape[3]
    if tuple(lora_b.shape) != (S, L, E, Ns, r):
        raise ValueError("lora_b shape does not match lora_a")
    M, topk, N = y.shape
    if N != S * Ns:
        raise ValueError("y's last dim must be S*Ns")
    rows = M * topk if x_per_pair else M
    if tuple(x.shape) != (rows, K):
        raise ValueError(f"x must be [{rows}, {K}]")
    if topk_weights is not None and tuple(topk_weights.shape) != (M, topk):
        raise ValueError("topk_weights must be [M, topk]")
    return M, topk, K, Ns, S, E, L, r


def fused_moe_lora(x, lora_a, lora_b, align: AlignOutput, topk_weights, y, *,
                   mul_routed_weight: bool, add_inputs: bool, x_per_pair: bool = False,
                   variant: str | int = "auto", max_active_loras: int | None = None,
                   stream=None):
    """Y (+)= (X A^T) B^T per routed pair and slice, in place on y; see moe_lora.h.
    max_active_loras: host-side bound on the active slots (None: L; 0: no launch)."""
    M, topk, K, Ns, S, E, L, r = _fused_shapes(x, lora_a, lora_b, topk_weights, y, x_per_pair)
    if align.sorted_token_ids.shape[0] != L:
        raise ValueError("align output was made for another L")
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    rc = lib().fused_moe_lora(
        _dptr(x), int(bool(x_per_pair)), _dptr(lora_a), _dptr(lora_b),
        _dptr(align.sorted_token_ids), _dptr(align.expert_ids),
        _dptr(align.num_tokens_post_padded), L if max_active_loras is None else int(max_active_loras),
        _dptr(topk_weights),
        int(bool(mul_routed_weight)), int(bool(add_inputs)), M, topk, K, Ns, S, E, L, r,
        align.block_m, _dptr(y), v, _stream_ptr(stream))
    if rc != OK:
        raise MoeLoraError(rc, "fused_moe_lora")
    return y


def fused_moe_lora_workspace_bytes(M: int, topk: int, K: int, Ns: int, S: int, E: int, L: int,
                                   r: int, block_m: int, x_per_pair: bool = False,
                                   variant: str | int = "auto") -> int:
    """Bytes of the workspace fused_moe_lora_ws uses for these sizes (0: none)."""
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    n = lib().fused_moe_lora_workspace_bytes(M, topk, K, Ns, S, E, L, r, block_m,
                                             int(bool(x_per_pair)), v)
    if n < 0:
        raise MoeLoraError(int(n), "fused_moe_lora_workspace_bytes")
    return int(n)


def alloc_fused_workspace(M: int, topk: int, K: int, Ns: int, S: int, E: int, L: int, r: int,
                          block_m: int, device, x_per_pair: bool = False,
                          variant: str | int = "auto"):
    """A zero-filled workspace for fused_moe_lora_ws (at least 16 bytes)."""
    import torch
    n = fused_moe_lora_workspace_bytes(M, topk, K, Ns, S, E, L, r, block_m, x_per_pair, variant)
    return torch.zeros(max(16, n), dtype=torch.uint8, device=device)


def fused_moe_lora_ws(x, lora_a, lora_b, align: AlignOutput, topk_weights, y, *,
                      mul_routed_weight: bool, add_inputs: bool, workspace,
                      x_per_pair: bool = False, variant: str | int = "auto",
                      peer_wait: int = -1, max_active_loras: int | None = None, stream=None):
    """fused_moe_lora with a K-split workspace (zero-filled before first use); see moe_lora.h."""
    M, topk, K, Ns, S, E, L, r = _fused_shapes(x, lora_a, lora_b, topk_weights, y, x_per_pair)
    if align.sorted_token_ids.shape[0] != L:
        raise ValueError("align output was made for another L")
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().fused_moe_lora_ws(
        _dptr(x), int(bool(x_per_pair)), _dptr(lora_a), _dptr(lora_b),
        _dptr(align.sorted_token_ids), _dptr(align.expert_ids),
        _dptr(align.num_tokens_post_padded), L if max_active_loras is None else int(max_active_loras),
        _dptr(topk_weights),
        int(bool(mul_routed_weight)), int(bool(add_inputs)), M, topk, K, Ns, S, E, L, r,
        align.block_m, _dptr(y), v, _dptr(workspace), nbytes, int(peer_wait),
        _stream_ptr(stream))
    if rc != OK:
        raise MoeLoraError(rc, "fused_moe_lora_ws")
    return y


def fused_moe_lora_with_align(topk_ids, token_lora_mapping, x, lora_a, lora_b, topk_weights, y,
                              *, E: int, L: int, block_m: int, mul_routed_weight: bool,
                              add_inputs: bool, out: "AlignOutput | None" = None,
                              x_per_pair: bool = False, variant: str | int = "auto",
                              stream=None) -> "AlignOutput":
    """moe_lora_align and fused_moe_lora in one launch (at most WITH_ALIGN_MAX_PAIRS pairs
    and WITH_ALIGN_MAX_SLOTS slots); returns the align outputs; see moe_lora.h."""
    import torch
    M, topk, K, Ns, S, E2, L2, r = _fused_shapes(x, lora_a, lora_b, topk_weights, y, x_per_pair)
    if (E2, L2) != (E, L):
        raise ValueError("E and L must match lora_a / lora_b")
    _check(topk_ids, "topk_ids", torch.int32, y.device)
    _check(token_lora_mapping, "token_lora_mapping", torch.int32, y.device)
    if tuple(topk_ids.shape) != (M, topk) or tuple(token_lora_mapping.shape) != (M,):
        raise ValueError("topk_ids must be [M, topk] and token_lora_mapping [M]")
    if out is None:
        out = alloc_align_output(M, topk, E, L, block_m, y.device)
    rc = lib().fused_moe_lora_with_align(
        _dptr(topk_ids), _dptr(token_lora_mapping), M, topk, E, L, block_m,
        _dptr(out.sorted_token_ids), _dptr(out.expert_ids), _dptr(out.num_tokens_post_padded),
        _dptr(out.lora_ids), _dptr(out.num_active_loras), _dptr(x), int(bool(x_per_pair)),
        _dptr(lora_a), _dptr(lora_b), _dptr(topk_weights), int(bool(mul_routed_weight)),
        int(bool(add_inputs)), K, Ns, S, r, _dptr(y),
        VARIANTS[variant] if isinstance(variant, str) else int(variant), _stream_ptr(stream))
    if rc != OK:
        raise MoeLoraError(rc, "fused_moe_lora_with_align")
    return out


def fused_moe_lora_naive(x, lora_a, lora_b, topk_ids, token_lora_mapping, topk_weights, y, *,
                         mul_routed_weight: bool, add_inputs: bool, block_m: int = 16,
                         x_per_pair: bool = False, variant: str | int = "auto", stream=None):
    """fused_moe_lora without the align step (M * topk <= NAIVE_MAX_PAIRS); see moe_lora.h."""
    import torch
    M, topk, K, Ns, S, E, L, r = _fused_shapes(x, lora_a, lora_b, topk_weights, y, x_per_pair)
    _check(topk_ids, "topk_ids", torch.int32, y.device)
    _check(token_lora_mapping, "token_lora_mapping", torch.int32, y.device)
    if tuple(topk_ids.shape) != (M, topk) or tuple(token_lora_mapping.shape) != (M,):
        raise ValueError("topk_ids must be [M, topk] and token_lora_mapping [M]")
    rc = lib().fused_moe_lora_naive(
        _dptr(x), int(bool(x_per_pair)), _dptr(lora_a), _dptr(lora_b), _dptr(topk_ids),
        _dptr(token_lora_mapping), _dptr(topk_weights), int(bool(mul_routed_weight)),
        int(bool(add_inputs)), M, topk, K, Ns, S, E, L, r, block_m, _dptr(y),
        VARIANTS[variant] if isinstance(variant, str) else int(variant), _stream_ptr(stream))
    if rc != OK:
        raise MoeLoraError(rc, "fused_moe_lora_naive")
    return y


def two_kernel_workspace_bytes(M: int, topk: int, K: int, Ns: int, S: int, E: int, L: int, r: int,
                               block_m: int, x_per_pair: bool = False) -> int:
    v = lib().fused_moe_lora_two_kernel_workspace_bytes(M, topk, K, Ns, S, E, L, r, block_m,
                                                        int(bool(x_per_pair)))
    if v < 0:
        raise MoeLoraError(v, "fused_moe_lora_two_kernel_workspace_bytes")
    return int(v)


def fused_moe_lora_two_kernel(x, lora_a, lora_b, align: AlignOutput, topk_weights, y, *,
                              mul_routed_weight: bool, add_inputs: bool, x_per_pair: bool = False,
                              workspace=None, max_active_loras: int | None = None, stream=None):
    """fused_moe_lora as shrink + expand with the rank vectors in `workspace` (ranks up to
    TWO_KERNEL_MAX_RANK); see moe_lora.h."""
    import torch
    M, topk, K, Ns, S, E, L, r = _fused_shapes(x, lora_a, lora_b, topk_weights, y, x_per_pair)
    if align.sorted_token_ids.shape[0] != L:
        raise ValueError("align output was made for another L")
    nbytes = two_kernel_workspace_bytes(M, topk, K, Ns, S, E, L, r, align.block_m, x_per_pair)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=y.device)
    _check(workspace, "workspace", workspace.dtype, y.device)
    rc = lib().fused_moe_lora_two_kernel(
        _dptr(x), int(bool(x_per_pair)), _dptr(lora_a), _dptr(lora_b),
        _dptr(align.sorted_token_ids), _dptr(align.expert_ids),
        _dptr(align.num_tokens_post_padded), L if max_active_loras is None else int(max_active_loras),
        _dptr(topk_weights),
        int(bool(mul_routed_weight)), int(bool(add_inputs)), M, topk, K, Ns, S, E, L, r,
        align.block_m, _dptr(y), _dptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_ptr(stream))
    if rc != OK:
        raise MoeLoraError(rc, "fused_moe_lora_two_kernel")
    return y


def moe_lora_accumulate(y, delta, stream=None):
    """y += delta (bf16, elementwise, one rounding): the join of the dual-stream path; see
    moe_lora.h.  Ordering the two streams is the caller's."""
    import torch
    _check(y, "y", torch.bfloat16, y.device)
    _check(delta, "delta", torch.bfloat16, y.device)
    if y.numel() != delta.numel():
        raise ValueError("y and delta must have the same number of elements")
    rc = lib().moe_lora_accumulate(_dptr(y), _dptr(delta), y.numel(), _stream_ptr(stream))
    if rc != OK:
        raise MoeLoraError(rc, "moe_lora_accumulate")
    return y
