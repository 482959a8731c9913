"""Parity of the MFMA GEMM (every operand layout, both storage types, ragged
and multi-tile shapes) against the oracle's dense product (GPU).

Every element must lie within the product's rounding-error bound
(oracle.compare.product_bound: fp32 accumulation over K terms plus one
rounding of the stored output), which is stricter than the layer gate."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tensor_transformer_layer_03_amd import binding as B

pytestmark = pytest.mark.gpu

# (dtype, a_kmajor, b_kmajor, M, N, K, bias)
CASES = [
    ("bf16", 1, 1, 300, 264, 136, True), ("bf16", 1, 0, 300, 264, 136, False), ("bf16", 0, 0, 264, 136, 300, False),
    ("f32", 1, 1, 300, 264, 136, True), ("f32", 1, 0, 300, 264, 136, False), ("f32", 0, 0, 264, 136, 300, False),
    ("bf16", 1, 1, 1024, 1024, 1024, False), ("bf16", 1, 1, 2048, 768, 520, True),
    ("bf16", 1, 0, 4096, 1024, 512, False), ("bf16", 0, 0, 1024, 512, 4000, False),
    ("bf16", 1, 1, 1, 8, 8, False), ("bf16", 0, 0, 8, 8, 1, False),
    # width a multiple of 192 whose 256x256 grid leaves a half-empty last round: 256x192 tiles
    ("bf16", 1, 1, 8000, 3072, 520, True),
]


def _dev(a, dtype):
    a = np.ascontiguousarray(a, np.float32)
    if dtype == "bf16":
        return torch.from_numpy(synth.bf16_bits(a)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_gemm(case):
    dtype, ak, bk, M, N, K, use_bias = case
    g = np.random.default_rng(M * 7 + N * 3 + K)
    rnd = (lambda a: synth.round_to_bf16(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    A = rnd(g.standard_normal((M, K)).astype(np.float32))    # logical A[m][k]
    Bm = rnd(g.standard_normal((N, K)).astype(np.float32))   # logical B[n][k]
    bias = rnd(g.standard_normal(N).astype(np.float32)) if use_bias else None
    dA = _dev(A if ak else A.T, dtype)
    dB = _dev(Bm if bk else Bm.T, dtype)
    c_f32 = (not ak) and (not bk)
    C = torch.full((M, N), float("nan"), dtype=torch.float32 if c_f32 else dA.dtype, device="cuda")
    B.tpl_gemm(B.TPL_BF16 if dtype == "bf16" else B.TPL_F32, ak, bk, M, N, K, dA, K if ak else M, dB,
               K if bk else N, None if bias is None else _dev(bias, dtype), C, N, c_f32)
    torch.cuda.synchronize()
    ref = O.linear(A, Bm, bias)
    mag = np.abs(A.astype(np.float64)) @ np.abs(Bm.astype(np.float64)).T
    if bias is not None:
        mag += np.abs(bias.astype(np.float64))
    got = C.float().cpu().numpy()
    out_dtype = "f32" if c_f32 or dtype == "f32" else "bf16"
    bound = O.compare.product_bound(ref, mag, K, out_dtype)
    err = np.abs(got - ref)
    ratio = err / np.maximum(bound, 1e-300)
    print(case, f"worst err/bound {ratio.max():.3g}, elements out of bound {(~(err <= bound)).sum()}")
    assert np.all(err <= bound), (case, float(ratio.max()))


TILE_CASES = [(lay, tile) for lay in ((1, 1), (1, 0), (0, 0))
              for tile in ("256x256", "256x256w8", "256x256w8t", "256x128", "256x128w8", "256x128w8t", "128x128", "256x256w8s4",
                           "256x192w8t")]


@pytest.mark.parametrize("lay,tile", TILE_CASES, ids=lambda c: str(c))
def test_gemm_every_tile_shape(lay, tile, monkeypatch):
    """Force each workgroup tile shape on a ragged multi-tile product."""
    monkeypatch.setenv("TPL_GEMM_TILE", tile)
    ak, bk = lay
    test_gemm(("bf16", ak, bk, 520, 776, 328, ak and bk))


@pytest.mark.parametrize("shape", [(4200, 4200, 96), (4104, 4296, 32), (2056, 8200, 1064)], ids=lambda c: str(c))
def test_gemm_multistage(shape, monkeypatch):
    """The four-stage forward kernel on more tiles than workgroups, with fewer
    K-tiles than pipeline stages, a ragged K tail and ragged M and N."""
    monkeypatch.setenv("TPL_GEMM_TILE", "256x256w8s4")
    M, N, K = shape
    test_gemm(("bf16", 1, 1, M, N, K, True))


@pytest.mark.parametrize("shape", [(16600, 1000, 3000), (16640, 1024, 4096), (51200, 1024, 1024)],
                         ids=lambda c: str(c))
def test_gemm_tail_split(shape):
    """fp32 weight-gradient products whose 256x256 tiles fill the CUs for whole
    rounds and leave a short last round: those tile rows run first, split over
    K, their partials parked in output rows that the whole rounds overwrite
    (the output starts as NaN, so a row left unwritten fails). Ragged M, N and
    K tails included."""
    M, N, K = shape
    test_gemm(("bf16", 0, 0, M, N, K, False))
