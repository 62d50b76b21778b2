"""Host-side logic of bench.py (CPU only): which traced kernels count as the
workload's fused kernel in the counter summary, the algorithmic byte counts,
and the refusal of multi-GPU runs."""
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PLAIN = "void ng::gemm_kernel<ng::Tile<128, 128, 4, 1, true, 2, false, 0, 64, true>, 0>(ng::GemmParams)"
ROW_LN = "void ng::gemm_kernel<ng::Tile<128, 128, 4, 1, true, 2, false, 0, 64, true>, 3>(ng::GemmParams)"
LAZY = "void ng::gemm_persistent_kernel<ng::Tile<256, 256, 4, 2, true, 4, false, 0, 32, false>, 1>(ng::GemmParams)"
XWG = ("void ng::gemm_xwg_kernel<ng::Tile<256, 256, 4, 2, true, 4, false, 0, 32, false>, false, "
       "false, false>(ng::GemmParams)")


def test_every_workload_label_names_a_known_epilogue():
    for w in workloads.WORKLOADS + workloads.NEXT_WORKLOADS:
        label = bench.kernel_label(w)
        epi = label.rstrip(">").rsplit("<", 1)[-1].rsplit(", ", 1)[-1]
        assert epi in bench.EPI_NUMBER, (w.name, label)


def test_fused_dispatch_excludes_the_unfused_gemm():
    w = workloads.WORKLOAD_BY_NAME["gemm_ln_65536x512x128"]
    assert bench.is_fused_dispatch(ROW_LN, w)
    assert bench.is_fused_dispatch(ROW_LN.replace("void ng::", "").replace("(ng::GemmParams)", ""), w)
    assert not bench.is_fused_dispatch(PLAIN, w)
    assert not bench.is_fused_dispatch("void ng::norm_kernel<16, 1, false>(ng::NormParams)", w)


def test_fused_dispatch_large_shapes():
    lazy = workloads.WORKLOAD_BY_NAME["lazy_rms_32768x4096x4096"]
    assert bench.is_fused_dispatch(LAZY, lazy)
    assert not bench.is_fused_dispatch(LAZY.replace(", 1>(", ", 0>("), lazy)
    rms = workloads.WORKLOAD_BY_NAME["gemm_rms_16384x4096x8192"]
    assert bench.is_fused_dispatch(XWG, rms)
    assert not bench.is_fused_dispatch(LAZY.replace(", 1>(", ", 0>("), rms)
    # the persistent grids' symbols carry the k-walk flag after the epilogue
    assert bench.is_fused_dispatch(LAZY.replace(", 1>(", ", 1, false>("), lazy)
    assert not bench.is_fused_dispatch(LAZY.replace(", 1>(", ", 0, true>("), lazy)
    assert not bench.is_fused_dispatch(LAZY.replace(", 1>(", ", 0, false>("), lazy)


def test_algorithmic_bytes_of_the_default_workload():
    w = workloads.WORKLOAD_BY_NAME["gemm_ln_65536x512x128"]
    # A 65536x512, B 512x128, C 65536x128, bf16
    assert bench.algorithmic_bytes(w) == 2 * (65536 * 512 + 512 * 128 + 65536 * 128) == 84017152


def test_more_than_one_gpu_is_refused():
    env = dict(os.environ)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
