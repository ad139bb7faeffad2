"""CPU checks of bench.py's host side: the one-GPU refusal, the byte model
of the headline step, and that the committed HBM-counter summary was taken on
the current kernel sources (so the bench line reports `roofline.traffic`)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_headline_bytes_per_step():
    # inputs x and residual, residual write, e4m3 codes, fp32 scales, gamma once
    M, d = 8192, 2816
    assert bench.case_bytes_8192() == M * (2 * d + 2 * d + 2 * d + d + 4) + 4 * d == 161_524_736


def test_counter_summary_matches_the_kernel_sources():
    t = bench.read_traffic()
    assert t is not None, ("profiles/rmsnorm_fp8_m8192_d2816_hbm_counters.md was taken on other kernel "
                           "sources: profile the current kernel again")
    assert 0.99 < t / bench.case_bytes_8192() < 1.05


def test_workload_byte_model_without_a_gpu():
    """The byte model the counter summaries compare against, by workload
    name: each configuration's bytes per call as the pages' model gives them
    (inputs + residual write + codes + scales, shared vectors once)."""
    assert bench.workload_rw("rms_2816_m8192") == (92_285_952, 69_238_784)
    assert sum(bench.workload_rw("group_m32768_fp32")) == 406_847_488
    assert sum(bench.workload_rw("layernorm_m16384")) == 201_359_364
    assert sum(bench.workload_rw("nvfp4_7168_m8192")) == 385_380_356
    assert sum(bench.workload_rw("nvfp4_slice_m8192")) == 32_249_860
    assert sum(bench.workload_rw("rms_small")) == 115_968
    for w in bench.HBM_WORKLOADS:
        rd, wr = bench.workload_rw(w)
        assert rd > 0 and wr > 0, w


def test_every_configuration_workload_is_a_suite_workload():
    import inspect
    src = inspect.getsource(bench.suite_cases)
    names = ({w for ws in bench.CONFIG_WORKLOADS.values() for w in ws} | set(bench.HBM_WORKLOADS)
             | set(bench.M1_WORKLOADS))
    for w in names:
        assert f'("{w}"' in src, w
    assert sorted(bench.CONFIG_WORKLOADS) == ["1", "2", "3", "4", "5"]
