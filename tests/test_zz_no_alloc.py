"""w4_gptq_quantize_noalloc -- the GPTQ column loop for callers that cannot allocate -- against
w4_gptq_quantize (the same kernels with a caller workspace), through the C ABI: two calls in a
row, the second on a smaller matrix (the library's device array keeps the first call's
contents), each bit-identical to the workspace call. Also the size limit."""
import numpy as np
import pytest
import torch

import int4_weight_only_amd as w4
import workloads
from tests.gpu_helpers import dev_bf16, host, host_bits

pytestmark = pytest.mark.gpu


def _calib(seed, N, d_in):
    rng = np.random.default_rng(seed)
    lat = rng.normal(size=(N, max(1, d_in // 4)))
    x = lat @ (rng.normal(size=(lat.shape[1], d_in)) / 2.0) + 0.3 * rng.normal(size=(N, d_in))
    return workloads.to_bf16_bits(x.astype(np.float32))


def _bits(t):
    return None if t is None else (host_bits(t) if t.dtype == torch.bfloat16 else host(t))


def test_noalloc_column_loop_matches_the_workspace_call():
    cases = ((1000, 600, 32, w4.W4_ASYM), (130, 200, 128, w4.W4_SYM))  # the second is smaller
    for i, (d_out, d_in, g, mode) in enumerate(cases):
        print("[case] gptq noalloc", d_out, d_in, g, mode, flush=True)
        w = workloads.weight(81, i, d_out, d_in)
        h = w4.gptq_hessian(dev_bf16(_calib(81 + i, 256, d_in)))
        u, dead = w4.gptq_factor(h, 0.01)
        wd = torch.from_numpy(w).cuda()
        ref = w4.gptq_quantize(wd.clone(), u, dead, g, mode)
        row_loss = torch.full((d_out,), float("nan"), dtype=torch.float32, device="cuda")
        got = w4.gptq_quantize_noalloc(wd.clone(), u, dead, g, mode, row_loss=row_loss)
        torch.cuda.synchronize()
        for name, a, b in zip(("qweight", "scales", "zeros", "row_loss"), ref, got):
            if a is None:
                assert b is None
                continue
            assert np.array_equal(_bits(a), _bits(b)), f"case {i}: {name} differs"


def test_noalloc_rejects_more_rows_than_its_array():
    d_out, d_in = (1 << 16) + 1, 32
    w = torch.zeros((d_out, d_in), dtype=torch.float32, device="cuda")
    u = torch.eye(d_in, dtype=torch.float32, device="cuda")
    with pytest.raises(w4.W4Error) as err:
        w4.gptq_quantize_noalloc(w, u, None, 32, w4.W4_SYM)
    assert err.value.status == 5  # W4_ERR_RANGE: nothing was launched
