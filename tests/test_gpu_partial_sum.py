"""shard_partial_sum through the C ABI (GPU): the sum of n partials plus the
row-parallel bias and the residual, against the oracle within the dtype's
tolerance and bit for bit against the documented order (fp32 accumulation
of residual, bias, partials 0..n-1, rounded once to the storage type), for
partial counts from 1 to 16 (the kernel has one instantiation per count),
ragged row counts (a thread's second chunk past the end) and an output that
aliases the residual."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tensor_transformer_layer_03_amd import binding as B

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(synth.bf16_bits(a)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def _stored(a, dtype):
    a = np.asarray(a, np.float32)
    return synth.round_to_bf16(a) if dtype == "bf16" else a


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("rows,cols,with_bias,with_res,alias", [
    (37, 104, True, True, False),      # 481 16-B chunks (bf16): ragged against 512 per workgroup
    (300, 1024, False, True, True),    # out aliases the residual
    (8, 8, True, False, False),        # one chunk per row
])
def test_partial_sum(dtype, n, rows, cols, with_bias, with_res, alias):
    g = np.random.default_rng(1000 * n + rows)
    parts = [_stored(g.standard_normal((rows, cols)), dtype) for _ in range(n)]
    bias = _stored(g.standard_normal(cols), dtype) if with_bias else None
    res = _stored(g.standard_normal((rows, cols)), dtype) if with_res else None
    desc = B.make_desc(64, 1, 64, 64, 1, 0, 1, 1, 8, True, dtype)
    d_parts = [_dev(p, dtype) for p in parts]
    d_res = _dev(res, dtype) if with_res else None
    out = d_res if alias else torch.full((rows, cols), float("nan"), device="cuda",
                                         dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    B.shard_partial_sum(desc, d_parts, _dev(bias, dtype) if with_bias else None, d_res, out, rows, cols)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    rep = O.compare.compare_tensor(got, O.partial_sum(parts, bias, res), dtype)
    assert rep["ok"], rep
    acc = np.zeros((rows, cols), np.float32)
    if with_res:
        acc += res
    if with_bias:
        acc += bias[None, :]
    for p in parts:
        acc += p
    assert np.array_equal(got, _stored(acc, dtype))
