"""Every GEMM the benchmark launches runs a kernel configuration that the GPU
parity tests check (host-side: plans come from the library's own tile
choice, no GPU needed). A configuration is the kernel instantiation
(mx_gemm_plan) together with its epilogue, output dtype and whether N is a
multiple of 8 (which selects the LDS-staged or the register store path)."""
import bench
from block_scaled_precision_mx_amd import api
import test_gpu_gemm
import test_gpu_gemm_fused
import test_gpu_gemm_splitk


def config_key(m, n, k, fmt, out, epilogue, ws=0):
    """The configuration a GEMM runs: plan (for mx_gemm_ws, with ws bytes of
    workspace), epilogue, output dtype, N % 8 == 0."""
    return (api.gemm_ws_plan(m, n, k, fmt, ws), epilogue, out, n % 8 == 0)


def parity_cases():
    return test_gpu_gemm.parity_cases() + test_gpu_gemm_fused.parity_cases() + test_gpu_gemm_splitk.parity_cases()


def bench_specs(names):
    for name in names:
        for s in bench.workload_gemms(name):
            yield name, s


def test_every_benchmarked_configuration_has_gpu_parity():
    covered = {config_key(*c) for c in parity_cases()}
    missing = set()
    for name, s in bench_specs(bench.WORKLOADS):
        key = config_key(s.m, s.n, s.k, s.fmt, s.out, s.epilogue, bench.WORKSPACE_BYTES if s.ws else 0)
        if key not in covered:
            missing.add((name, s.label, key))
    assert not missing, sorted(missing)


def test_every_measured_shape_has_full_size_gpu_parity():
    """The headline and every configuration in the default benchmark line:
    each distinct GEMM shape is itself a GPU parity case (full or sampled)."""
    shapes = {c[:4] + (c[5],) for c in parity_cases()}
    missing = set()
    for name, s in bench_specs([bench.HEADLINE] + bench.EXTRA_CONFIGS):
        if (s.m, s.n, s.k, s.fmt, s.epilogue) not in shapes:
            missing.add((name, s.label, s.m, s.n, s.k, s.fmt))
    assert not missing, sorted(missing)


def test_workload_gemm_lists():
    """The GEMM lists are what the workloads define: four linears per block for
    the stacks, six GEMMs for the fc1/fc2 pair, twelve per block for the
    block-training workloads (four fprop, then dgrad and wgrad per linear)."""
    from block_scaled_precision_mx_amd import workloads as W
    st = W.VITL_MXFP8
    specs = bench.workload_gemms(st.name)
    assert len(specs) == 4 * st.blocks
    assert sum(2 * s.m * s.n * s.k for s in specs) == st.gemm_flops()
    tp = W.TRAIN_PAIR
    specs = bench.workload_gemms(tp.name)
    assert len(specs) == 6 and sum(2 * s.m * s.n * s.k for s in specs) == tp.gemm_flops()
    for bt in W.BLOCK_TRAINS.values():
        specs = bench.workload_gemms(bt.name)
        assert len(specs) == 12 * bt.blocks
        assert sum(2 * s.m * s.n * s.k for s in specs) == bt.gemm_flops()
        first = specs[:12]
        assert [s.label for s in first[:4]] == [f"gemm_{l}_fprop" for l in ("qkv", "proj", "fc1", "fc2")]
        assert all(s.fmt == bt.fwd_fmt for s in first[:4]) and all(s.fmt == bt.bwd_fmt for s in first[4:])
        # wgrad contracts over the tokens
        assert all(s.k == bt.m for s in first if s.label.endswith("wgrad"))


def test_kernel_families_aggregate():
    """The roofline's kernel: a format's tile configurations summed (flops
    over time), each family priced against its own matrix-core peak."""
    kernels = {
        "gemm_mx_kernel<mxfp8, 192x256>": {"launches_per_step": 2, "ms_per_step": 0.1, "flops_per_launch_avg": 5e10},
        "gemm_mx_kernel<mxfp8, 192x256, l2pf>": {"launches_per_step": 1, "ms_per_step": 0.05,
                                                 "flops_per_launch_avg": 9e10},
        "gemm_mx_kernel<nvfp4, 128x256>+splitk2": {"launches_per_step": 1, "ms_per_step": 0.2,
                                                   "flops_per_launch_avg": 9e10},
    }
    fam = bench.kernel_families(kernels)
    f8 = fam["gemm_mx_kernel<mxfp8>"]
    assert f8["launches_per_step"] == 3 and abs(f8["ms_per_step"] - 0.15) < 1e-12
    assert abs(f8["flops_per_launch_avg"] - (2 * 5e10 + 9e10) / 3) < 1.0
    assert abs(f8["avg_launch_us"] - 50.0) < 1e-9
    assert f8["configurations"] == ["gemm_mx_kernel<mxfp8, 192x256, l2pf>", "gemm_mx_kernel<mxfp8, 192x256>"]
    assert fam["gemm_mx_kernel<nvfp4>"]["launches_per_step"] == 1
    assert set(bench.FAMILY_PEAK) >= set(fam)
