"""Seeded synthetic inputs for the MoE-LoRA hot path.

This module only draws random numbers and lays them out; it holds none of the
arithmetic of the method itself.  Both the CPU oracle tests and the HIP path
take their inputs from here, so the two sides see identical bytes.

Workload shapes follow the serving setups the pages describe (vLLM PR #29257
"Lora MoE Align Improvements", Test Result: gpt-oss-120b at concurrency 8;
vLLM PR #29708, Benchmark: gpt-oss-20b with max-loras 6 and rank 64; vLLM
#13096, Llama-2-7b with max-loras 4 and rank 8; the prhub summary of vLLM PR
#42290 names a Qwen3-MoE preset for its one-shot benchmark).  No dataset item
is used: token routing, adapter assignment and weights are all drawn here.

Recipe (fixed order, one ``numpy.random.default_rng(seed)`` per case):
  1. the set of active adapter slots (seeded subset of the L slots),
  2. ``token_lora_mapping`` (-1 with probability ``p_neg``, else uniform over
     the active slots),
  3. ``topk_ids`` (distinct experts per token; uniform, or Zipf(s) popularity
     through Gumbel-top-k on log-probabilities with a seeded rank->expert
     permutation),
  4. router logits -> ``topk_weights`` (softmax over the top-k, fp32),
  5. X, 6. lora_a, 7. lora_b (bf16; only the active slots are filled, the
     others stay zero and are never read), 8. Y_in (bf16 N(0,1) when
     ``add_inputs``, zeros otherwise).

bf16 values are produced by round-to-nearest-even from float32 samples and
are carried as raw ``uint16`` bit patterns.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Shape:
    """One synthetic workload: sizes, flags and the input distribution."""

    name: str
    M: int            # tokens
    K: int            # input width of the adapter (contracted in the shrink)
    Ns: int           # width of one output slice
    S: int            # number of slices (gate+up = 2, qkv = 3, ...)
    E: int            # experts
    topk: int         # experts per token
    L: int            # adapter slots
    r: int            # adapter rank
    block_m: int      # BLOCK_M
    active: int       # number of active slots (seeded subset of the L)
    p_neg: float      # probability that a token has no adapter (-1)
    routing: str = "uniform"   # "uniform" | "zipf"
    zipf_s: float = 1.2
    x_per_pair: bool = False   # w2-style input: one X row per (token, k)
    mul: bool = False          # multiply the delta by the routed weight
    add: bool = True           # accumulate into Y (else overwrite)
    dist: str = "literal"      # "literal": X ~ N(0,1)/sqrt(K); "stress": X ~ N(0,1)
    seed: int = 0
    align_only: bool = False

    @property
    def numel(self) -> int:
        return self.M * self.topk

    @property
    def N(self) -> int:
        return self.S * self.Ns

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


# The five workload families (plus the align-only stress case).  Seeds are
# 1000 * family + sub-case so every case draws its own stream.
def _catalog() -> dict:
    c = {}
    c["tiny"] = Shape("tiny", M=16, K=256, Ns=128, S=1, E=8, topk=2, L=2, r=8,
                      block_m=16, active=2, p_neg=0.25, mul=True, add=True,
                      seed=1000)
    for a in range(1, 7):
        c[f"oss20b_decode_w13_a{a}"] = Shape(
            f"oss20b_decode_w13_a{a}", M=16, K=2880, Ns=2880, S=2, E=32, topk=4,
            L=6, r=64, block_m=16, active=a, p_neg=0.0, mul=False, add=True,
            seed=2000 + a)
        # the same layer's down projection: X is the activation of the w13
        # output, one row per pair, K = the w13 slice width
        c[f"oss20b_decode_w2_a{a}"] = Shape(
            f"oss20b_decode_w2_a{a}", M=16, K=2880, Ns=2880, S=1, E=32, topk=4,
            L=6, r=64, block_m=16, active=a, p_neg=0.0, x_per_pair=True, mul=True,
            add=True, seed=2010 + a)
    for i, (M, bm, tag) in enumerate(((8, 16, "decode"), (2048, 64, "prefill"))):
        c[f"oss120b_{tag}_w13"] = Shape(
            f"oss120b_{tag}_w13", M=M, K=2880, Ns=2880, S=2, E=128, topk=4, L=4,
            r=16, block_m=bm, active=4, p_neg=0.2, mul=False, add=True,
            seed=3000 + 2 * i)
        c[f"oss120b_{tag}_w2"] = Shape(
            f"oss120b_{tag}_w2", M=M, K=2880, Ns=2880, S=1, E=128, topk=4, L=4,
            r=16, block_m=bm, active=4, p_neg=0.2, x_per_pair=True, mul=True,
            add=True, seed=3001 + 2 * i)
    c["qwen3_prefill"] = Shape(
        "qwen3_prefill", M=8192, K=2048, Ns=768, S=2, E=128, topk=8, L=8, r=128,
        block_m=64, active=3, p_neg=0.2, routing="zipf", zipf_s=1.2, mul=False,
        add=True, seed=4000)
    c["dense_qkv"] = Shape(
        "dense_qkv", M=4096, K=4096, Ns=4096, S=3, E=1, topk=1, L=4, r=8,
        block_m=64, active=4, p_neg=0.0, mul=False, add=True, seed=5000)
    c["dense_o"] = Shape(
        "dense_o", M=4096, K=4096, Ns=4096, S=1, E=1, topk=1, L=4, r=8,
        block_m=64, active=4, p_neg=0.0, mul=False, add=True, seed=5001)
    c["align_stress"] = Shape(
        "align_stress", M=65536, K=8, Ns=8, S=1, E=256, topk=8, L=16, r=1,
        block_m=64, active=16, p_neg=0.0, align_only=True, seed=5002)
    c["align_stress_neg"] = c["align_stress"].replace(
        name="align_stress_neg", p_neg=0.2, seed=5003)
    return c


CATALOG = _catalog()


def shape(name: str, **overrides) -> Shape:
    """Look up a named workload, optionally overriding fields."""
    s = CATALOG[name]
    return s.replace(**overrides) if overrides else s


@dataclass
class Case:
    """The drawn inputs of one workload (numpy, host memory)."""

    shape: Shape
    active_slots: np.ndarray          # int32 [active]
    token_lora_mapping: np.ndarray    # int32 [M]
    topk_ids: np.ndarray              # int32 [M, topk]
    topk_weights: np.ndarray          # float32 [M, topk]
    x: np.ndarray | None = None       # uint16 bf16 [M or M*topk, K]
    lora_a: np.ndarray | None = None  # uint16 bf16 [S, L, E, r, K]
    lora_b: np.ndarray | None = None  # uint16 bf16 [S, L, E, Ns, r]
    y_in: np.ndarray | None = None    # uint16 bf16 [M, topk, S*Ns]
    extra: dict = field(default_factory=dict)


def _topk_uniform(rng, M, E, topk):
    if E == 1:
        return np.zeros((M, topk), dtype=np.int32)
    keys = rng.random((M, E), dtype=np.float32)
    # first `topk` entries of a uniformly random permutation per token
    idx = np.argpartition(keys, topk - 1, axis=1)[:, :topk] if topk < E else np.argsort(keys, axis=1)
    sub = np.take_along_axis(keys, idx, axis=1)
    order = np.argsort(sub, axis=1, kind="stable")
    return np.take_along_axis(idx, order, axis=1).astype(np.int32)


def _topk_zipf(rng, M, E, topk, s):
    perm = rng.permutation(E)                      # popularity rank -> expert id
    logp_rank = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    logp = np.empty(E, dtype=np.float64)
    logp[perm] = logp_rank
    keys = logp[None, :] + rng.gumbel(size=(M, E))
    idx = np.argpartition(-keys, topk - 1, axis=1)[:, :topk]
    sub = np.take_along_axis(keys, idx, axis=1)
    order = np.argsort(-sub, axis=1, kind="stable")
    return np.take_along_axis(idx, order, axis=1).astype(np.int32)


def _normal_bf16(rng, size, scale):
    a = rng.standard_normal(size, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return f32_to_bf16_bits(a)


def w2_partner(name: str) -> str:
    """The down-projection (w2) workload of a w13 workload's layer."""
    if "_w13" not in name or name.replace("_w13", "_w2") not in CATALOG:
        raise KeyError(f"{name} has no w2 partner")
    return name.replace("_w13", "_w2")


def draw_layer(name13: str, **overrides) -> tuple:
    """Both projections of one MoE layer: the w13 case and its w2 partner,
    the latter with the w13 case's routing (slots, mapping, top-k ids and
    weights) so that one align serves both.  The w2 case's X is drawn but a
    layer feeds w2 the activation of the w13 output instead."""
    s13 = shape(name13, **overrides)
    s2 = shape(w2_partner(name13), **overrides)
    if (s2.M, s2.topk, s2.E, s2.L, s2.block_m) != (s13.M, s13.topk, s13.E, s13.L, s13.block_m):
        raise ValueError("w13 and w2 workloads of one layer must share the routing sizes")
    if s2.active != s13.active:
        raise ValueError("w13 and w2 workloads of one layer must have the same active count")
    c13, c2 = draw(s13), draw(s2)
    # the w2 adapters drawn into c2's own active slots move to c13's
    src, dst = c2.active_slots, c13.active_slots
    for name in ("lora_a", "lora_b"):
        arr = getattr(c2, name)
        moved = np.zeros_like(arr)
        moved[:, dst] = arr[:, src]
        setattr(c2, name, moved)
    c2.active_slots = dst.copy()
    c2.token_lora_mapping = c13.token_lora_mapping.copy()
    c2.topk_ids = c13.topk_ids.copy()
    c2.topk_weights = c13.topk_weights.copy()
    return c13, c2


def draw(s: Shape, with_tensors: bool = True) -> Case:
    """Draw every input of workload ``s`` from ``default_rng(s.seed)``."""
    rng = np.random.default_rng(s.seed)
    active = np.sort(rng.choice(s.L, size=s.active, replace=False)).astype(np.int32)
    neg = rng.random(s.M) < s.p_neg
    pick = rng.integers(0, s.active, size=s.M)
    mapping = np.where(neg, -1, active[pick]).astype(np.int32)
    if s.routing == "zipf":
        topk_ids = _topk_zipf(rng, s.M, s.E, s.topk, s.zipf_s)
    else:
        topk_ids = _topk_uniform(rng, s.M, s.E, s.topk)
    logits = rng.standard_normal((s.M, s.topk))
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    case = Case(s, active, mapping, np.ascontiguousarray(topk_ids), w)
    if not with_tensors or s.align_only:
        return case
    rows = s.numel if s.x_per_pair else s.M
    xs = 1.0 if s.dist == "stress" else 1.0 / np.sqrt(s.K)
    case.x = _normal_bf16(rng, (rows, s.K), xs)
    a = np.zeros((s.S, s.L, s.E, s.r, s.K), dtype=np.uint16)
    a[:, active] = _normal_bf16(rng, (s.S, s.active, s.E, s.r, s.K), 1.0 / np.sqrt(s.K))
    case.lora_a = a
    b = np.zeros((s.S, s.L, s.E, s.Ns, s.r), dtype=np.uint16)
    b[:, active] = _normal_bf16(rng, (s.S, s.active, s.E, s.Ns, s.r), 1.0 / np.sqrt(s.r))
    case.lora_b = b
    if s.add:
        case.y_in = _normal_bf16(rng, (s.M, s.topk, s.N), 1.0)
    else:
        case.y_in = np.zeros((s.M, s.topk, s.N), dtype=np.uint16)
    return case
