"""mx_gemm_scratch (the allocation-free variant of mx_gemm_ws, for callers
that cannot allocate) through the C ABI: two calls in a row, the second
smaller, each equal bit for bit to mx_gemm_ws with a caller workspace of
mx_gemm_workspace_bytes, and within the oracle's bound; the scratch keeps the
last call's partials, so the second call must not depend on them. Both plans
split K, so the scratch is in use."""
import numpy as np
import pytest
import torch

from block_scaled_precision_mx_amd import _lib, api
from block_scaled_precision_mx_amd import workloads as W
from oracle import gemm as G
from oracle import quantize as Q
from gpu_util import Guarded, f64_of, log, quantize_guarded, to_device_bf16

pytestmark = pytest.mark.gpu


def scratch_and_ws(m, n, k, fmt, bias_bits, seed):
    a = W.np_activation((m, k), seed=seed)
    b = W.np_normal((n, k), seed=seed + 1, std=W.W_STD)
    qa, qb = quantize_guarded(to_device_bf16(a), fmt), quantize_guarded(to_device_bf16(b), fmt)
    bias = None if bias_bits is None else to_device_bf16(bias_bits.reshape(1, -1)).reshape(-1)
    need = api.gemm_workspace_bytes(m, n, k, fmt)
    plan = api.gemm_ws_plan(m, n, k, fmt, need)
    assert "+splitk" in plan and 0 < need <= _lib.SCRATCH_BYTES, (plan, need)
    log(f"mx_gemm_scratch {fmt} {m}x{n}x{k} plan={plan}")
    gc = Guarded(m * n * 2)
    got = api.mx_gemm_scratch(qa, qb, bias, "bf16", gc.typed(torch.bfloat16, (m, n)))
    gc.check("C")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ref = api.mx_gemm_ws(qa, qb, bias, "bf16", ws)
    g, r = f64_of(got), f64_of(ref)
    assert np.array_equal(g, r), f"{(g != r).sum()} outputs differ from mx_gemm_ws"
    qa_o, qb_o = Q.quantize(a, fmt), Q.quantize(b, fmt)
    c, s = G.gemm_ref(qa_o, qb_o, bias_bits)
    rr, cc = np.nonzero(np.ones_like(c, dtype=bool))
    assert G.accept_entries(g[rr, cc], c[rr, cc], s[rr, cc], "bf16", qa_o, qb_o, rr, cc).all()


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_scratch_gemm_two_calls(fmt):
    # the larger problem first, then a smaller one over the same scratch
    scratch_and_ws(1024, 1024, 11235, fmt, W.np_normal((1024,), seed=3, std=W.BIAS_STD), seed=11)
    scratch_and_ws(300, 264, 7000, fmt, None, seed=12)
