"""Every tile instantiation of the two GEMM engines against the oracle, element
by element.

The launchers pick a tile shape from the problem size, so the moderate shapes
of the other parity tests mostly run the 128x128 tile, and the large tiles the
full-size workloads run (256x256 for the 7B-class GEMMs, 256x192 for the
GPT-2-small column GEMM and the 175B-class ones, 128x192 for the GPT-2-small
row GEMM) would otherwise only be checked there. Here the environment variable TPMLP_TILE forces each shape in
turn on shapes that span several tiles with ragged edges in M and N, with and
without a K tail (K not a multiple of the 64-element bf16 or 128-byte fp8
k-slice), and every output element is compared with the oracle by the same
checks as the untiled tests (one ulp plus the accumulation bound on Z, the
1e-2 / 6e-2 bar on Y, bit-exact integer GEMMs, the backward's bounds).
"""
import numpy as np
import pytest

import oracle
import test_gpu_backward as bwd
import test_gpu_backward_fp8 as bwd8
import test_gpu_bias as bias
import test_gpu_linear_layout as lin
import test_gpu_parity as par
from helpers import dev_bf16, host_bf16_bits, host_f64, log
from workloads import make_integer_valued

pytestmark = pytest.mark.gpu

BF16_TILES = ["256x256", "256x192", "256x128", "128x192", "128x128"]
FP8_TILES = ["256x256", "256x192", "128x128"]


@pytest.fixture(scope="module")
def tpm():
    import torch
    import megatron_tensor_transformer_shard_amd as m
    assert torch.cuda.is_available()
    return m


@pytest.fixture
def tile(request, monkeypatch):
    monkeypatch.setenv("TPMLP_TILE", request.param)
    log(f"tile {request.param}")
    return request.param


# M, d, H, N, out dtype; F = H/N. K1 is [M, d]·[d, F], K2 [M, F]·[F, d].
# The main loop takes six 64-k slices per iteration when the slice count is a
# multiple of 6 (not at 256x256), two when it is even, one otherwise: the
# shapes cover all three, with and without a K tail.
SHAPES = [
    (600, 512, 1280, 2, "f32"),    # no K tail in either GEMM (d = 512, F = 640: 8 and 10 slices); M, N ragged
    (600, 576, 2560, 4, "bf16"),   # no K tail, an odd slice count in K1 (d = 576: 9 slices)
    (600, 768, 1536, 2, "f32"),    # no K tail, 12 slices in both GEMMs
    (520, 328, 912, 2, "bf16"),    # K tails in both (328 = 5·64 + 8, F = 456 = 7·64 + 8)
    (1030, 520, 4160, 8, "bf16"),  # 8 ranks, K tails with 9 slices, ragged everywhere
    (333, 200, 2400, 3, "f32"),    # F = 800 (13 slices with a tail)
]


@pytest.mark.parametrize("tile", BF16_TILES, indirect=True)
@pytest.mark.parametrize("M,d,H,N,odt", SHAPES)
def test_forward_every_element(tpm, tile, M, d, H, N, odt):
    # every rank: Z_i against the oracle's Z_i (bound + 95% bit-identical), Y_i
    # and the sum of the ranks against the oracle at the bf16 bar
    par.test_ragged_shapes_all_ranks(tpm, M, d, H, N, odt)


@pytest.mark.parametrize("tile", BF16_TILES, indirect=True)
@pytest.mark.parametrize("M,F,d", [(600, 640, 576), (333, 520, 264)])
def test_row_partial_integer_bit_exact(tpm, tile, M, F, d):
    # small integers: every fp32 sum is exact, so Y_i must equal Z_i·B_i to the bit
    import torch
    Zi, Bi, _ = make_integer_valued(M, F, d, seed=M + F)
    Zd, Bd = dev_bf16(Zi), dev_bf16(Bi)
    Y = tpm.tp_mlp_row_partial(Zd, Bd)
    Yb = tpm.tp_mlp_row_partial(Zd, Bd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.bf16_decode(Zi) @ oracle.bf16_decode(Bi)
    assert np.array_equal(host_f64(Y), ref)
    assert np.array_equal(host_bf16_bits(Yb), oracle.bf16_encode(ref))


@pytest.mark.parametrize("tile", BF16_TILES, indirect=True)
def test_col_gelu_strided_view_and_identity(tpm, tile):
    par.test_col_gelu_on_strided_column_view(tpm)
    par.test_identity_weights_give_elementwise_gelu(tpm)


@pytest.mark.parametrize("tile", BF16_TILES, indirect=True)
@pytest.mark.parametrize("M,d,H,N", [(296, 136, 528, 2), (520, 512, 2560, 4)])
def test_backward_every_element(tpm, tile, M, d, H, N):
    # the backward's layouts (K-major Q, M-major P) and the GeLU' epilogue
    bwd.test_backward_vs_oracle(tpm, M, d, H, N)


@pytest.mark.parametrize("tile", BF16_TILES, indirect=True)
def test_transposed_weights_and_biases(tpm, tile):
    lin.test_transposed_weights_vs_oracle_and_math_layout(tpm, 513, 264, 1056, 4, "bf16")
    bias.test_col_gelu_bias_vs_oracle_both_layouts(tpm, 300, 136, 544, 2)
    bias.test_backward_with_bias_vs_oracle(tpm, 520, 136, 1088, 4)


# fp8: d, F multiples of 16; k-slices of 128 bytes. (300, 272, 800, 1): K tails
# in both GEMMs (272 = 2·128 + 16, 800 = 6·128 + 32); (520, 512, 2048, 4): none.
@pytest.mark.parametrize("tile", FP8_TILES, indirect=True)
@pytest.mark.parametrize("M,d,H,N", [(300, 272, 800, 1), (520, 512, 2048, 4), (384, 768, 1536, 2)])
def test_fp8_forward_every_element(tpm, tile, M, d, H, N):
    # 128-byte slices: 3 and 7 with K tails, 4, and 6 (six per iteration)
    par.test_fp8_shard_vs_oracle(tpm, M, d, H, N)


@pytest.mark.parametrize("tile", FP8_TILES, indirect=True)
def test_fp8_steps_and_delayed_scaling(tpm, tile):
    par.test_fp8_steps_individually(tpm)
    par.test_col_gelu_e4m3_delayed_equals_current_path_at_the_current_scale(tpm, 257, 512, 2048)
    par.test_col_gelu_e4m3_delayed_with_a_predicted_scale(tpm, 3.5)


@pytest.mark.parametrize("tile", FP8_TILES, indirect=True)
@pytest.mark.parametrize("M,d,H,N", [(272, 144, 576, 2), (528, 512, 2048, 4)])
def test_fp8_backward_every_element(tpm, tile, M, d, H, N):
    bwd8.test_backward_fp8_vs_oracle(tpm, M, d, H, N)
