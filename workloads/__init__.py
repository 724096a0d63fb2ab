"""Seeded synthetic inputs for the tensor-parallel MLP shard.

This module only draws random numbers and stores them as bfloat16 bit
patterns.  It holds none of the MLP's arithmetic, and both the CPU oracle and
the GPU path consume exactly the bits it returns.

The MLP block is Y = GeLU(X·A)·B with A of shape [d, 4d] and B of shape
[4d, d] ("Megatron architecture and 6D parallel guide", §3.1 tensor-parallel
principle).  Rank i of an N-way tensor-parallel group holds the column block
A_i and the matching row block B_i.

Recipe (the same for every workload):
  rng = numpy.random.default_rng(seed)          (PCG64)
  X = rng.standard_normal((M, d))                drawn first, float64
  A = sigma * rng.standard_normal((d, H))        drawn second
  B = sigma * rng.standard_normal((H, d))        drawn third
each then rounded float64 -> float32 (IEEE, round to nearest even) and
float32 -> bfloat16 (round to nearest even).  H is 4d for a full weight, or
the shard width F when a workload draws one rank's shard directly.

The backward's output gradient comes from a generator of its own, so that
the forward inputs of a workload stay the same bits:
  dY = grad_sigma * default_rng([seed, 1]).standard_normal((M, d))
rounded the same way.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_random", "make_output_grad",
           "AttnWorkload", "ATTN_WORKLOADS", "make_attn_inputs",
           "bf16_bits_from_f32", "bf16_bits_to_f32"]


@dataclass(frozen=True)
class Workload:
    """One MLP shape.  H is the column count of the drawn A (4d, or F)."""
    name: str
    M: int            # tokens (rows of X)
    d: int            # model width
    H: int            # columns of the drawn A / rows of the drawn B
    N: int            # tensor-parallel degree the drawn A/B are split over
    sigma: float      # std-dev of A and B entries
    seed: int
    description: str = ""
    fp8: bool = False  # the workload runs the e4m3 variant of the path
    grad_sigma: float = 1.0  # std-dev of the output gradient dY (backward workloads)
    tags: tuple = field(default_factory=tuple)

    @property
    def F(self) -> int:
        return self.H // self.N

    @property
    def backward(self) -> bool:
        return "backward" in self.tags

    def flops_per_shard(self) -> int:
        """Forward: two GEMMs of 2·M·d·F flops each. Backward: five (S
        recomputed, dZ, dX_i, dA_i, dB_i)."""
        return (10 if self.backward else 4) * self.M * self.d * self.F


WORKLOADS = {
    # Tiny MLP at TP=2, both ranks run.
    "tiny_tp2": Workload("tiny_tp2", M=32, d=64, H=256, N=2, sigma=0.02, seed=0,
                         description="X[32x64], A[64x256], B[256x64], TP N=2, both ranks"),
    # GPT-2-small width, unsharded (N=1): 8 sequences x 1024 tokens.
    "gpt2s_n1": Workload("gpt2s_n1", M=8192, d=768, H=3072, N=1, sigma=0.02, seed=1,
                         description="X[8192x768], A[768x3072], B[3072x768], N=1"),
    # 7B-class width d=4096 at TP=8: 4 sequences x 2048 tokens; full A, B drawn
    # and sliced into 8 shards A_i[4096x2048], B_i[2048x4096].
    "7b_tp8": Workload("7b_tp8", M=8192, d=4096, H=16384, N=8, sigma=0.02, seed=2,
                       description="X[8192x4096], A[4096x16384] -> A_i[4096x2048], "
                                   "B[16384x4096] -> B_i[2048x4096], TP N=8, all ranks"),
    # 175B-class width d=12288 at TP=8: one 2048-token micro-batch; one rank's
    # shard drawn directly at its shape (every rank is statistically alike).
    "175b_tp8": Workload("175b_tp8", M=2048, d=12288, H=6144, N=1, sigma=0.006, seed=3,
                         description="X[2048x12288], A_i[12288x6144], B_i[6144x12288], "
                                     "one TP=8 rank's shard"),
    # The same shard in fp8 e4m3 with per-tensor amax scales.
    "175b_tp8_e4m3": Workload("175b_tp8_e4m3", M=2048, d=12288, H=6144, N=1, sigma=0.006,
                              seed=3, fp8=True,
                              description="175b_tp8 shard quantised to e4m3, per-tensor "
                                          "scale 448/amax, bf16 output"),
    # The same fp8 shard with delayed scaling of Z: Z quantised in the column
    # GEMM's epilogue with the scale predicted from the recorded amaxes.
    "175b_tp8_e4m3_delayed": Workload("175b_tp8_e4m3_delayed", M=2048, d=12288, H=6144, N=1,
                                      sigma=0.006, seed=3, fp8=True, tags=("delayed",),
                                      description="175b_tp8_e4m3 with delayed scaling of Z "
                                                  "(amax history of 1024 steps)"),
    # Backward of every rank's shard of 7b_tp8 for an output gradient dY, and
    # the sum of the ranks' input gradients.
    "7b_tp8_bwd": Workload("7b_tp8_bwd", M=8192, d=4096, H=16384, N=8, sigma=0.02, seed=2,
                           tags=("backward",),
                           description="backward of 7b_tp8: dY[8192x4096]; per rank S, dS, "
                                       "dX_i, dA_i[4096x2048], dB_i[2048x4096]; sum of dX_i"),
    # The same backward with fp8 GEMMs in the hybrid formats (E4M3 activations
    # and weights, E5M2 gradients, current amax scales).
    "7b_tp8_bwd_fp8": Workload("7b_tp8_bwd_fp8", M=8192, d=4096, H=16384, N=8, sigma=0.02,
                               seed=2, fp8=True, tags=("backward",),
                               description="7b_tp8_bwd with fp8 GEMMs: X, A_i, B_i, Z in e4m3, "
                                           "dY, dS in e5m2; sum of dX_i"),
}


@dataclass(frozen=True)
class AttnWorkload:
    """One attention-block shape: B sequences of S tokens, width d, `heads`
    heads of width d/heads split over N ranks."""
    name: str
    B: int
    S: int
    d: int
    heads: int
    N: int
    sigma: float      # std-dev of W_qkv and W_o entries
    seed: int
    causal: bool = True
    description: str = ""

    @property
    def M(self) -> int:
        return self.B * self.S

    @property
    def dh(self) -> int:
        return self.d // self.heads

    @property
    def F(self) -> int:
        return self.d // self.N

    def flops_per_shard(self) -> int:
        """QKV projection 2·M·d·3F, output projection 2·M·F·d, and per head
        QKᵀ and P·V, 4·S²·dh per sequence (half of it with the causal mask)."""
        hr = self.heads // self.N
        att = 4 * self.S * self.S * self.dh * hr * self.B
        if self.causal:
            att //= 2
        return 2 * self.M * self.d * 3 * self.F + 2 * self.M * self.F * self.d + att


ATTN_WORKLOADS = {
    # Two sequences of 40 tokens (a ragged tail for 64-key blocks), d = 1024,
    # 8 heads of 128 split over 2 ranks.
    "attn_tiny": AttnWorkload("attn_tiny", B=2, S=40, d=1024, heads=8, N=2, sigma=0.03, seed=10,
                              description="X[80x1024], W_qkv[1024x3072], W_o[1024x1024], "
                                          "8 heads of 128, TP N=2, causal"),
    # 7B-class attention block at TP=8: 32 heads of 128, 4 per rank
    # ("Megatron architecture and 6D parallel guide", §3.2: 32 heads at TP=8),
    # 4 sequences of 2048 tokens, causal.
    "7b_tp8_attn": AttnWorkload("7b_tp8_attn", B=4, S=2048, d=4096, heads=32, N=8, sigma=0.02,
                                seed=4,
                                description="X[8192x4096] (4 x 2048 tokens), W_qkv[4096x12288], "
                                            "W_o[4096x4096], 32 heads of 128, TP N=8 (4 heads "
                                            "per rank), causal, all ranks + sum"),
}


def make_attn_inputs(name_or_wl) -> tuple:
    """(X, W_qkv, W_o) bfloat16 bits: rng = default_rng(seed); X = N(0,1)
    [B·S, d], then W_qkv = σ·N(0,1) [d, 3d] (head-major: columns
    [h·3dh, (h+1)·3dh) are head h's query, key and value columns), then
    W_o = σ·N(0,1) [d, d]; rounded as the MLP inputs are."""
    wl = ATTN_WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    rng = np.random.default_rng(wl.seed)
    X = _draw_bf16(rng, (wl.M, wl.d), 1.0)
    Wqkv = _draw_bf16(rng, (wl.d, 3 * wl.d), wl.sigma)
    Wo = _draw_bf16(rng, (wl.d, wl.d), wl.sigma)
    return X, Wqkv, Wo


def bf16_bits_from_f32(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    x = rng.standard_normal(shape)
    if sigma != 1.0:
        x *= sigma
    return bf16_bits_from_f32(x.astype(np.float32))


def make_random(M: int, d: int, H: int, seed: int, sigma: float = 0.02,
                x_sigma: float = 1.0):
    """(X, A, B) as uint16 bfloat16 bit arrays of shapes [M,d], [d,H], [H,d]."""
    rng = np.random.default_rng(seed)
    X = _draw_bf16(rng, (M, d), x_sigma)
    A = _draw_bf16(rng, (d, H), sigma)
    B = _draw_bf16(rng, (H, d), sigma)
    return X, A, B


def make_output_grad(M: int, d: int, seed: int, sigma: float = 1.0) -> np.ndarray:
    """dY [M, d] as bfloat16 bits, from its own generator default_rng([seed, 1])."""
    return _draw_bf16(np.random.default_rng([seed, 1]), (M, d), sigma)


def make_bias(n: int, seed: int, sigma: float = 0.5) -> np.ndarray:
    """A bias vector [n] as bfloat16 bits, from its own generator default_rng([seed, 2])."""
    return _draw_bf16(np.random.default_rng([seed, 2]), (n,), sigma)


def make_inputs(name_or_wl) -> tuple:
    """Inputs of a named workload: (X, A, B) bfloat16 bit arrays (uint16)."""
    wl = WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    return make_random(wl.M, wl.d, wl.H, wl.seed, wl.sigma)


def make_integer_valued(M: int, d: int, H: int, seed: int, lo: int = -4, hi: int = 4):
    """Small-integer-valued bfloat16 inputs (every value exact in bf16).

    With |x| <= 4 and sums far below 2**24 every fp32 dot product is exact, so
    integer GEMM results can be compared bit for bit.
    """
    rng = np.random.default_rng(seed)
    X = rng.integers(lo, hi + 1, size=(M, d)).astype(np.float32)
    A = rng.integers(lo, hi + 1, size=(d, H)).astype(np.float32)
    B = rng.integers(lo, hi + 1, size=(H, d)).astype(np.float32)
    return bf16_bits_from_f32(X), bf16_bits_from_f32(A), bf16_bits_from_f32(B)


def tile_rows(M: int, seed: int = 4321, tile: int = 256, per_tile: int = 4) -> np.ndarray:
    """Sorted distinct row indices in [0, M) that hit every `tile`-row block of
    the output: one row at a random offset inside each of its `per_tile` equal
    parts (so every 256-, 128- and 64-row M-tile of the GEMM tilings is
    sampled, at offsets that differ from block to block), plus rows 0 and M-1."""
    rng = np.random.default_rng(seed)
    part = tile // per_tile
    rows = {0, M - 1}
    for start in range(0, M, part):
        n = min(part, M - start)
        rows.add(start + int(rng.integers(0, n)))
    return np.array(sorted(rows), dtype=np.int64)


def sample_rows(M: int, count: int, seed: int = 1234) -> np.ndarray:
    """Sorted distinct row indices in [0, M), always including 0 and M-1."""
    rng = np.random.default_rng(seed)
    count = min(count, M)
    rows = set([0, M - 1])
    if count > len(rows):
        rows.update(rng.choice(M, size=count, replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)
