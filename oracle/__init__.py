"""CPU oracle of the MoE-LoRA hot path (plain C, double precision).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark; never by the product package.  It shares no
source, header, table or helper with the HIP library.  See ``oracle.c`` for
the definitions it follows and the readings it takes.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_i32p = ctypes.POINTER(ctypes.c_int32)


def build(src: str = SRC, out: str = LIB, extra: tuple = ()) -> str:
    """Compile the oracle with gcc into a shared library; return its path."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", *extra, src, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else ctypes.c_void_p(0)


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, path: str = LIB):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_capacity.restype = ctypes.c_int64
        lib.oracle_capacity.argtypes = [ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_align.restype = ctypes.c_int
        lib.oracle_align.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
        lib.oracle_fused.restype = ctypes.c_int
        lib.oracle_fused.argtypes = [
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p]
        self.lib = lib

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def capacity(self, M, topk, E, block_m) -> int:
        return int(self.lib.oracle_capacity(M, topk, E, block_m))

    def align(self, topk_ids, token_lora_mapping, E, L, block_m):
        """Returns dict: sorted_token_ids [L, cap], expert_ids [L, cap/B],
        num_tokens_post_padded [L], lora_ids [L], num_active (int).
        Entries past a slot's padded length are left at -7 (never written)."""
        topk_ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
        mapping = np.ascontiguousarray(token_lora_mapping, dtype=np.int32)
        M, topk = topk_ids.shape
        cap = self.capacity(M, topk, E, block_m)
        sorted_ids = np.full((L, cap), -7, dtype=np.int32)
        expert_ids = np.full((L, cap // block_m), -7, dtype=np.int32)
        ntpp = np.zeros(L, dtype=np.int32)
        lora_ids = np.zeros(L, dtype=np.int32)
        nact = np.zeros(1, dtype=np.int32)
        rc = self.lib.oracle_align(_ptr(topk_ids), _ptr(mapping), M, topk, E, L,
                                   block_m, cap, _ptr(sorted_ids), _ptr(expert_ids),
                                   _ptr(ntpp), _ptr(lora_ids), _ptr(nact))
        if rc != 0:
            raise MemoryError("oracle_align failed")
        return {"sorted_token_ids": sorted_ids, "expert_ids": expert_ids,
                "num_tokens_post_padded": ntpp, "lora_ids": lora_ids,
                "num_active": int(nact[0]), "cap": cap}

    def fused(self, x, lora_a, lora_b, topk_ids, token_lora_mapping, topk_weights,
              y_in, mul_routed_weight, add_inputs, x_per_pair=False, pairs=None):
        """Y as float64 [numel, S*Ns] (or [len(pairs), S*Ns] for a pair list)."""
        topk_ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
        mapping = np.ascontiguousarray(token_lora_mapping, dtype=np.int32)
        w = np.ascontiguousarray(topk_weights, dtype=np.float32)
        x = np.ascontiguousarray(x, dtype=np.uint16)
        lora_a = np.ascontiguousarray(lora_a, dtype=np.uint16)
        lora_b = np.ascontiguousarray(lora_b, dtype=np.uint16)
        y_in = np.ascontiguousarray(y_in, dtype=np.uint16)
        M, topk = topk_ids.shape
        S, L, E, r, K = lora_a.shape
        Ns = lora_b.shape[3]
        assert lora_b.shape == (S, L, E, Ns, r)
        assert x.shape == ((M * topk) if x_per_pair else M, K)
        assert y_in.size == M * topk * S * Ns
        if pairs is not None:
            pairs = np.ascontiguousarray(pairs, dtype=np.int64)
            n = len(pairs)
        else:
            n = M * topk
        out = np.empty((n, S * Ns), dtype=np.float64)
        rc = self.lib.oracle_fused(
            _ptr(x), int(bool(x_per_pair)), _ptr(lora_a), _ptr(lora_b),
            _ptr(topk_ids), _ptr(mapping), _ptr(w), int(bool(mul_routed_weight)),
            int(bool(add_inputs)), M, topk, K, Ns, S, E, L, r, _ptr(y_in),
            _ptr(pairs), n if pairs is not None else 0, _ptr(out))
        if rc != 0:
            raise MemoryError("oracle_fused failed")
        return out


_default = None


def load(rebuild: bool = False) -> Oracle:
    """The oracle built from ``oracle.c`` (compiled on first use)."""
    global _default
    if _default is None or rebuild:
        if rebuild or not os.path.exists(LIB) or \
                os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _default = Oracle(LIB)
    return _default
