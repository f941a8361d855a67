"""Host-side checks of the C ABI (no GPU compute): the library loads, exports
every function include/mx.h declares, reports the buffer sizes the oracle's
layout implies, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

from block_scaled_precision_mx_amd import _lib
from oracle import quantize as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mx.h")
FMTS = {"mxfp8": 1, "mxfp4": 2, "nvfp4": 3}
AXES = {"row": 0, "col": 1}


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_declared_function(L):
    names = header_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(L, n)


def test_version_and_kpad(L):
    assert L.mx_version() >= 10000
    assert [L.mx_k_pad(n) for n in (1, 127, 128, 129, 11235)] == [128, 128, 128, 256, 11264]
    assert L.mx_k_pad(0) == 0


@pytest.mark.parametrize("shape", [(1, 1), (3, 70), (256, 768), (11235, 1024), (4096, 11235)])
def test_sizes_match_oracle_layout(L, shape):
    for fmt, f in FMTS.items():
        for axis, a in AXES.items():
            assert L.mx_codes_bytes(*shape, f, a) == Q.codes_bytes(*shape, fmt, axis)
            assert L.mx_scales_bytes(*shape, f, a) == Q.scales_bytes(*shape, fmt, axis)


def test_size_queries_reject_bad_args(L):
    assert L.mx_codes_bytes(0, 5, 1, 0) == 0
    assert L.mx_codes_bytes(5, 5, 9, 0) == 0
    assert L.mx_scales_bytes(5, 5, 1, 7) == 0


ALIGNED = 1 << 20      # fake, never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,status,msg", [
    ((ALIGNED, 4, 4, 4, ALIGNED, ALIGNED, 7, 0), 1, "unknown format"),
    ((ALIGNED, 4, 4, 4, ALIGNED, ALIGNED, 1, 3), 1, "unknown axis"),
    ((ALIGNED, 0, 4, 4, ALIGNED, ALIGNED, 1, 0), 1, "empty"),
    ((ALIGNED, 4, 8, 4, ALIGNED, ALIGNED, 1, 0), 1, "ld"),
    ((None, 4, 4, 4, ALIGNED, ALIGNED, 1, 0), 1, "null"),
    ((ALIGNED + 1, 4, 4, 4, ALIGNED, ALIGNED, 1, 0), 3, "2-byte"),
    ((ALIGNED, 4, 4, 4, ALIGNED + 8, ALIGNED, 1, 0), 3, "16-byte"),
    ((ALIGNED, 1 << 20, 1 << 12, 1 << 12, ALIGNED, ALIGNED, 1, 0), 2, "2 GiB"),
    # a column quantization of one column of 3e9 rows: one stored row of
    # K_pad ~ 3e9 elements (1.5 GB of fp4 codes) would overflow the kernels' int counts
    ((ALIGNED, 3_000_000_000, 1, 1, ALIGNED, ALIGNED, 2, 1), 2, "below 2^31"),
    ((ALIGNED, 3_000_000_000, 1, 1, ALIGNED, ALIGNED, 3, 1), 2, "below 2^31"),
    ((ALIGNED, 1, (1 << 31) - 200, (1 << 31) - 200, ALIGNED, ALIGNED, 2, 0), 2, "below 2^31"),
])
def test_quantize_validation(L, args, status, msg):
    assert L.mx_quantize(*args, None) == status
    assert msg in L.mx_last_error().decode()


@pytest.mark.parametrize("args,status,msg", [
    ((ALIGNED,) * 5 + (4, 4, 32, 9, None, 0), 1, "unknown format"),
    ((ALIGNED,) * 5 + (4, 4, 32, 1, None, 5), 1, "output dtype"),
    ((ALIGNED,) * 5 + (0, 4, 32, 1, None, 0), 1, ">= 1"),
    ((ALIGNED,) * 5 + (4, 4, 0, 1, None, 0), 1, ">= 1"),
    ((ALIGNED, None, ALIGNED, ALIGNED, ALIGNED, 4, 4, 32, 1, None, 0), 1, "null"),
    ((ALIGNED, ALIGNED, ALIGNED + 4, ALIGNED, ALIGNED, 4, 4, 32, 1, None, 0), 3, "16-byte"),
    ((ALIGNED,) * 5 + (4, 4, 32, 1, ALIGNED + 1, 0), 3, "bias"),
    ((ALIGNED,) * 5 + (1 << 22, 4, 1024, 1, None, 0), 2, "2 GiB"),
    # one fp4 row of K >= 2^31 elements is only 1 GiB of codes: rejected by the count bound
    ((ALIGNED,) * 5 + (1, 1, 1 << 31, 2, None, 0), 2, "below 2^31"),
    ((ALIGNED,) * 5 + (1, 1, (1 << 31) - 200, 3, None, 0), 2, "below 2^31"),
])
def test_gemm_validation(L, args, status, msg):
    assert L.mx_gemm(*args, None) == status
    assert msg in L.mx_last_error().decode()


@pytest.mark.parametrize("args,status,msg", [
    ((ALIGNED, 4, 4, 4) + (ALIGNED,) * 4 + (7, None, 32.0), 1, "unknown format"),
    ((ALIGNED, 4, 0, 4) + (ALIGNED,) * 4 + (1, None, 32.0), 1, "empty"),
    ((ALIGNED, 4, 8, 4) + (ALIGNED,) * 4 + (1, None, 32.0), 1, "ld"),
    ((ALIGNED, 4, 4, 4, ALIGNED, ALIGNED, None, ALIGNED, 1, None, 32.0), 1, "null"),
    ((ALIGNED, 4, 4, 4) + (ALIGNED,) * 4 + (3, ALIGNED, 0.0), 1, "headroom"),
    ((ALIGNED, 4, 4, 4) + (ALIGNED,) * 4 + (3, ALIGNED, float("inf")), 1, "headroom"),
    ((ALIGNED, 4, 4, 4) + (ALIGNED,) * 4 + (3, ALIGNED + 2, 32.0), 3, "amax_prev"),
    ((ALIGNED + 1, 4, 4, 4) + (ALIGNED,) * 4 + (1, None, 32.0), 3, "2-byte"),
    ((ALIGNED, 4, 4, 4, ALIGNED, ALIGNED, ALIGNED, ALIGNED + 8, 1, None, 32.0), 3, "16-byte"),
    ((ALIGNED, 1 << 20, 1 << 12, 1 << 12) + (ALIGNED,) * 4 + (1, None, 32.0), 2, "2 GiB"),
    ((ALIGNED, 3_000_000_000, 1, 1) + (ALIGNED,) * 4 + (2, None, 32.0), 2, "below 2^31"),
])
def test_quantize_dual_validation(L, args, status, msg):
    assert L.mx_quantize_dual(*args, None) == status
    assert msg in L.mx_last_error().decode()


def _items(*specs):
    arr = (_lib.QuantItem * max(1, len(specs)))()
    for i, (src, rows, cols, ld, codes, scales) in enumerate(specs):
        arr[i] = _lib.QuantItem(src, rows, cols, ld, codes, scales)
    return arr


GOOD = (ALIGNED, 4, 4, 4, ALIGNED, ALIGNED)


@pytest.mark.parametrize("specs,n,fmt,status,msg", [
    ((GOOD,), 1, 3, 2, "NVFP4"),
    ((GOOD,), 1, 9, 1, "unknown format"),
    ((GOOD,), 0, 1, 1, "outside [1, 32]"),
    ((GOOD,), 33, 1, 1, "outside [1, 32]"),
    ((GOOD, (ALIGNED, 0, 4, 4, ALIGNED, ALIGNED)), 2, 1, 1, "item 1: empty"),
    ((GOOD, (ALIGNED, 1, (1 << 31) - 200, (1 << 31) - 200, ALIGNED, ALIGNED)), 2, 2, 2, "item 1: rows and cols"),
    ((GOOD, GOOD, (ALIGNED, 4, 8, 4, ALIGNED, ALIGNED)), 3, 2, 1, "item 2: ld"),
    (((None, 4, 4, 4, ALIGNED, ALIGNED),), 1, 1, 1, "item 0: null"),
    (((ALIGNED + 1, 4, 4, 4, ALIGNED, ALIGNED),), 1, 1, 3, "item 0: src must be 2-byte"),
    ((GOOD, (ALIGNED, 4, 4, 4, ALIGNED, ALIGNED + 4)), 2, 1, 3, "item 1: codes and scales"),
    (((ALIGNED, 1 << 20, 1 << 12, 1 << 12, ALIGNED, ALIGNED),), 1, 1, 2, "item 0: output larger"),
    (((ALIGNED, 1 << 19, 4096, 4096, ALIGNED, ALIGNED),), 1, 2, 2, "item 0: input too large"),
])
def test_quantize_batch_validation(L, specs, n, fmt, status, msg):
    """Every item is checked before anything is launched; the message names
    the first bad item."""
    assert L.mx_quantize_batch(_items(*specs), n, fmt, None) == status
    assert msg in L.mx_last_error().decode()


def test_quantize_batch_null_items(L):
    assert L.mx_quantize_batch(None, 1, 1, None) == 1
    assert "null item array" in L.mx_last_error().decode()


@pytest.mark.parametrize("specs,n,fmt,amax,status,msg", [
    ((GOOD,), 1, 1, None, 1, "null amax"),
    ((GOOD,), 1, 1, ALIGNED + 2, 3, "amax must be 4-byte"),
    ((GOOD,), 1, 3, ALIGNED, 2, "NVFP4"),
    ((GOOD,), 0, 1, ALIGNED, 1, "outside [1, 32]"),
    ((GOOD, (ALIGNED, 0, 4, 4, ALIGNED, ALIGNED)), 2, 2, ALIGNED, 1, "item 1: empty"),
])
def test_quantize_batch_amax_validation(L, specs, n, fmt, amax, status, msg):
    """mx_quantize_batch_amax checks its accumulator pointer and every item as
    mx_quantize_batch does, and names itself in the message."""
    assert L.mx_quantize_batch_amax(_items(*specs), n, fmt, amax, None) == status
    err = L.mx_last_error().decode()
    assert msg in err and err.startswith("mx_quantize_batch_amax")


@pytest.mark.parametrize("args,status,msg", [
    ((ALIGNED, 4, 4, 4, ALIGNED, ALIGNED, 1, 0, ALIGNED, 8), 2, "only NVFP4"),
    ((ALIGNED, 4, 4, 4, ALIGNED, ALIGNED, 7, 0, ALIGNED, 8), 1, "unknown format"),
    ((ALIGNED, 4, 4, 4, ALIGNED, ALIGNED, 3, 0, None, 8), 1, "null amax"),
    ((ALIGNED, 4, 4, 4, ALIGNED, ALIGNED, 3, 0, ALIGNED + 2, 8), 3, "amax must be 4-byte"),
    ((ALIGNED, 4, 4, 4, ALIGNED, ALIGNED, 3, 0, ALIGNED, 0), 1, "nslots = 0"),
    ((ALIGNED, 4, 4, 4, ALIGNED, ALIGNED, 3, 0, ALIGNED, 257), 1, "nslots = 257"),
    ((ALIGNED, 4, 4, 4, ALIGNED, ALIGNED, 3, 3, ALIGNED, 8), 1, "unknown axis"),
    ((ALIGNED, 4, 8, 4, ALIGNED, ALIGNED, 3, 1, ALIGNED, 8), 1, "ld"),
    ((ALIGNED, 4, 4, 4, ALIGNED + 8, ALIGNED, 3, 1, ALIGNED, 8), 3, "16-byte"),
    ((ALIGNED, 3_000_000_000, 1, 1, ALIGNED, ALIGNED, 3, 1, ALIGNED, 1), 2, "below 2^31"),
])
def test_quantize_amax_validation(L, args, status, msg):
    assert L.mx_quantize_amax(*args, None) == status
    err = L.mx_last_error().decode()
    assert msg in err and err.startswith("mx_quantize_amax")


@pytest.mark.parametrize("args,status,msg", [
    ((ALIGNED, 4, 8, 8) + (ALIGNED,) * 4 + (1, None, 32.0), 2, "NVFP4 only"),
    ((ALIGNED, 4, 8, 8) + (ALIGNED,) * 4 + (9, None, 32.0), 1, "unknown format"),
    ((ALIGNED, 4, 12, 12) + (ALIGNED,) * 4 + (3, None, 32.0), 2, "multiple of 8"),
    ((ALIGNED, 0, 8, 8) + (ALIGNED,) * 4 + (3, None, 32.0), 1, "empty"),
    ((ALIGNED, 4, 8, 8, ALIGNED, None, ALIGNED, ALIGNED, 3, None, 32.0), 1, "null"),
    ((ALIGNED, 4, 8, 8) + (ALIGNED,) * 4 + (3, ALIGNED, -1.0), 1, "headroom"),
    ((ALIGNED, 4, 8, 8) + (ALIGNED,) * 3 + (ALIGNED + 4, 3, None, 32.0), 3, "16-byte"),
    ((ALIGNED, 1 << 21, 1 << 12, 1 << 12) + (ALIGNED,) * 4 + (3, None, 32.0), 2, "2 GiB"),
    ((ALIGNED, 3_000_000_000, 8, 8) + (ALIGNED,) * 4 + (3, None, 32.0), 2, "below 2^31"),
])
def test_quantize_dual_sr_validation(L, args, status, msg):
    assert L.mx_quantize_dual_sr(*args, 1, 2, None) == status
    assert msg in L.mx_last_error().decode()


@pytest.mark.parametrize("args,status,msg", [
    ((ALIGNED,) * 4 + (4, 8, 32, 3, None, ALIGNED, ALIGNED), 2, "MXFP8 and MXFP4 only"),
    ((ALIGNED,) * 4 + (4, 8, 32, 9, None, ALIGNED, ALIGNED), 1, "unknown format"),
    ((ALIGNED,) * 4 + (4, 12, 32, 1, None, ALIGNED, ALIGNED), 2, "multiple of 8"),
    ((ALIGNED,) * 4 + (0, 8, 32, 1, None, ALIGNED, ALIGNED), 1, ">= 1"),
    ((ALIGNED,) * 4 + (4, 8, 32, 1, None, None, ALIGNED), 1, "null"),
    ((ALIGNED,) * 4 + (4, 8, 32, 1, None, ALIGNED, ALIGNED + 8), 3, "16-byte"),
    ((ALIGNED,) * 4 + (4, 8, 32, 2, ALIGNED + 1, ALIGNED, ALIGNED), 3, "bias"),
    ((ALIGNED,) * 4 + (1 << 22, 1 << 10, 32, 1, None, ALIGNED, ALIGNED), 2, "output larger"),
    ((ALIGNED,) * 4 + (1, 8, 1 << 31, 2, None, ALIGNED, ALIGNED), 2, "below 2^31"),
])
def test_gemm_gelu_quantize_validation(L, args, status, msg):
    assert L.mx_gemm_gelu_quantize(*args, None) == status
    assert msg in L.mx_last_error().decode()


# mx_layernorm_quantize(x, rows, cols, ld, gamma, beta, eps, codes, scales, fmt)
@pytest.mark.parametrize("args,status,msg", [
    ((ALIGNED, 4, 8, 8, ALIGNED, ALIGNED, 1e-6, ALIGNED, ALIGNED, 3), 2, "NVFP4"),
    ((ALIGNED, 4, 8, 8, ALIGNED, ALIGNED, 1e-6, ALIGNED, ALIGNED, 9), 1, "unknown format"),
    ((ALIGNED, 0, 8, 8, ALIGNED, ALIGNED, 1e-6, ALIGNED, ALIGNED, 1), 1, "empty"),
    ((ALIGNED, 4, 8, 7, ALIGNED, ALIGNED, 1e-6, ALIGNED, ALIGNED, 1), 1, "ld"),
    ((ALIGNED, 4, 8, 8, None, ALIGNED, 1e-6, ALIGNED, ALIGNED, 1), 1, "null"),
    ((ALIGNED, 4, 8, 8, ALIGNED, ALIGNED, -1.0, ALIGNED, ALIGNED, 1), 1, "eps"),
    ((ALIGNED, 4, 8, 8, ALIGNED, ALIGNED, float("nan"), ALIGNED, ALIGNED, 2), 1, "eps"),
    ((ALIGNED, 4, 8, 8, ALIGNED, ALIGNED, 0.0, ALIGNED, ALIGNED, 1), 1, "eps"),
    ((ALIGNED + 2, 4, 8, 8, ALIGNED, ALIGNED, 1e-6, ALIGNED, ALIGNED, 1), 3, "4-byte"),
    ((ALIGNED, 4, 8, 8, ALIGNED, ALIGNED, 1e-6, ALIGNED + 4, ALIGNED, 1), 3, "16-byte"),
    ((ALIGNED, 1 << 22, 1 << 10, 1 << 10, ALIGNED, ALIGNED, 1e-6, ALIGNED, ALIGNED, 1), 2, "2 GiB"),
    # rows longer than the stated accuracy covers
    ((ALIGNED, 4, 8193, 8193, ALIGNED, ALIGNED, 1e-6, ALIGNED, ALIGNED, 1), 2, "8192 columns"),
])
def test_layernorm_quantize_validation(L, args, status, msg):
    assert L.mx_layernorm_quantize(*args, None) == status
    assert msg in L.mx_last_error().decode()


def test_quantize_dual_ignores_headroom_for_mx(L):
    """MX formats never read amax_prev / headroom: a bad headroom is not an
    error there (the call then fails later on the 2 GiB check, still before
    any launch)."""
    args = (ALIGNED, 1 << 20, 1 << 12, 1 << 12) + (ALIGNED,) * 4 + (1, ALIGNED, 0.0)
    assert L.mx_quantize_dual(*args, None) == 2


def test_last_error_is_per_thread(L):
    import threading
    L.mx_quantize(None, 4, 4, 4, ALIGNED, ALIGNED, 1, 0, None)
    seen = {}

    def other():
        L.mx_gemm(*((ALIGNED,) * 5 + (4, 4, 32, 9, None, 0)), None)
        seen["msg"] = L.mx_last_error().decode()
    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert "unknown format" in seen["msg"]
    assert "null" in L.mx_last_error().decode()


def test_gemm_plan_names(L):
    assert L.mx_gemm_plan(11235, 4096, 1024, 1).decode() == "gemm_mx_kernel<mxfp8, 256x256>"
    assert L.mx_gemm_plan(11235, 3072, 1024, 1).decode() == "gemm_mx_kernel<mxfp8, 192x256>"
    # at least 32 K-stages of 128 (fp8): the L2-prefetching variant of the tile
    assert L.mx_gemm_plan(11235, 1024, 4096, 1).decode() == "gemm_mx_kernel<mxfp8, 192x256, l2pf>"
    assert L.mx_gemm_plan(11235, 1024, 3968, 1).decode() == "gemm_mx_kernel<mxfp8, 192x256>"
    assert L.mx_gemm_plan(11235, 1024, 4096, 2).decode() == "gemm_mx_kernel<mxfp4, 192x256>"
    assert L.mx_gemm_plan(11235, 4096, 1024, 2).decode() == "gemm_mx_kernel<mxfp4, 192x256>"
    assert L.mx_gemm_plan(256, 768, 768, 1).decode() == "gemm_mx_kernel<mxfp8, 128x128>"
    # NVFP4: weight-gradient shapes (few output tiles) take 128x128; the
    # token-major shapes keep the large tiles.
    assert L.mx_gemm_plan(4096, 1024, 11235, 3).decode() == "gemm_mx_kernel<nvfp4, 128x128>"
    assert L.mx_gemm_plan(1024, 4096, 11235, 3).decode() == "gemm_mx_kernel<nvfp4, 128x128>"
    assert L.mx_gemm_plan(11235, 4096, 1024, 3).decode() == "gemm_mx_kernel<nvfp4, 192x256>"
    assert L.mx_gemm_plan(4160, 4096, 384, 3).decode() == "gemm_mx_kernel<nvfp4, 192x256>"
    assert L.mx_gemm_plan(0, 4, 4, 1) is None
    assert L.mx_gemm_plan(4, 4, 4, 9) is None



def test_bench_workloads_are_defined():
    """Every workload bench.py offers is a stack, a training pair or a
    block-training workload of the workloads module, and each names its own
    format; the default line measures the headline and every other
    configuration."""
    import bench
    from block_scaled_precision_mx_amd import workloads as W
    assert set(bench.WORKLOADS) == set(W.STACKS) | set(W.TRAIN_PAIRS) | set(W.BLOCK_TRAINS)
    for name in bench.WORKLOADS:
        wl = W.STACKS.get(name) or W.TRAIN_PAIRS.get(name)
        if wl is not None:
            assert wl.fmt in name
        else:
            bt = W.BLOCK_TRAINS[name]
            assert (bt.bwd_fmt in name) or ("p3" in name and bt.bwd_fmt == "nvfp4" and bt.sr_grads)
    assert set(bench.EXTRA_CONFIGS) <= set(bench.WORKLOADS) and bench.HEADLINE not in bench.EXTRA_CONFIGS
    # the five configurations: single layer, ViT-B MXFP8, ViT-L MXFP8 (headline), ViT-L MXFP4, NVFP4 pair
    for name in ("single_mxfp8_256x768x768", "vitb16_mxfp8_fwd_stack", "vitl16_mxfp4_fwd_stack",
                 "vitl16_nvfp4_fc1fc2_train"):
        assert name in bench.EXTRA_CONFIGS


@pytest.mark.parametrize("args,status,msg", [
    ((ALIGNED,) * 5 + (4, 4, 32, 1, None, 0, ALIGNED + 4, 1 << 20), 3, "workspace must be 16-byte aligned"),
    ((ALIGNED,) * 5 + (4, 4, 32, 9, None, 0, ALIGNED, 1 << 20), 1, "unknown format"),
    ((ALIGNED,) * 5 + (0, 4, 32, 1, None, 0, ALIGNED, 1 << 20), 1, ">= 1"),
    ((ALIGNED,) * 5 + (1, 1, 1 << 31, 2, None, 0, ALIGNED, 1 << 20), 2, "below 2^31"),
])
def test_gemm_ws_validation(L, args, status, msg):
    assert L.mx_gemm_ws(*args, None) == status
    assert msg in L.mx_last_error().decode()
    assert L.mx_last_error().decode().startswith("mx_gemm_ws")


def test_gemm_ws_plans_follow_the_workspace():
    """The weight-gradient shapes split K when the workspace holds the
    partials; less workspace gives fewer splits or none; the forward shapes
    never split; mx_gemm_workspace_bytes is S M N 4 of the preferred plan."""
    from block_scaled_precision_mx_amd import api
    for fmt in ("mxfp8", "nvfp4"):
        need = api.gemm_workspace_bytes(3072, 1024, 11235, fmt)
        plan = api.gemm_ws_plan(3072, 1024, 11235, fmt, need)
        s = int(plan.split("+splitk")[1])
        assert need == s * 3072 * 1024 * 4
        assert api.gemm_ws_plan(3072, 1024, 11235, fmt, 0) == api.gemm_plan(3072, 1024, 11235, fmt)
        fewer = api.gemm_ws_plan(3072, 1024, 11235, fmt, need - 1)
        assert "+splitk" not in fewer or int(fewer.split("+splitk")[1]) < s
    for (m, n, k) in [(11235, 3072, 1024), (11235, 1024, 4096), (11235, 4096, 1024), (22470, 768, 3072)]:
        for fmt in ("mxfp8", "mxfp4", "nvfp4"):
            assert api.gemm_workspace_bytes(m, n, k, fmt) == 0
            assert api.gemm_ws_plan(m, n, k, fmt, 1 << 30) == api.gemm_plan(m, n, k, fmt)
    assert api.gemm_workspace_bytes(0, 4, 4, "mxfp8") == 0
