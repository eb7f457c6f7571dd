"""Host-side tests of bench.py and workloads.py (no GPU needed): the
single-GPU guard, the rocprofv3 summary readers, the traffic lookup and the
FLOP convention."""
import csv
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_summarize_pmc_scales_by_the_copy_kernel(tmp_path):
    mib = 1 << 20
    # the copy of 512 MiB reads as half its bytes on FETCH_SIZE, exactly on WRITE_SIZE
    fetch = [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE", "Counter_Value": 512 * 1024 / 2},
             {"Kernel_Name": "fwd_bf16_kernel", "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000.0},
             {"Kernel_Name": "fwd_bf16_kernel", "Counter_Name": "FETCH_SIZE", "Counter_Value": 3000.0}]
    write = [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE", "Counter_Value": 512 * 1024},
             {"Kernel_Name": "fwd_bf16_kernel", "Counter_Name": "WRITE_SIZE", "Counter_Value": 500.0}]
    _write_csv(str(tmp_path / "f" / "run_counter_collection.csv"), fetch)
    _write_csv(str(tmp_path / "w" / "run_counter_collection.csv"), write)
    out = tmp_path / "summary.txt"
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), 512 * mib, str(out), "cmd")
    text = out.read_text().splitlines()
    assert text[0] == "command: cmd"
    assert text[1] == f"source_hash {bench.kernel_source_hash()}"
    assert "fetch_scale 2.0000 write_scale 1.0000" in text[2]
    line = next(l for l in text if "fwd_bf16_kernel" in l)
    parts = line.split()
    # average 2000 KiB per dispatch, scaled by 2: 4096000 bytes; write 500 KiB
    assert float(parts[parts.index("fetch_bytes") + 1]) == 2000 * 1024 * 2
    assert float(parts[parts.index("write_bytes") + 1]) == 500 * 1024


def test_traffic_lookup_needs_matching_sources(tmp_path, monkeypatch):
    summ = tmp_path / "hbm.txt"
    summ.write_text("command: x\nsource_hash {}\ncopy_bytes 1 fetch_scale 2 write_scale 1\n"
                    "kernel 'k_bwd_dkdv_kernel' fetch_bytes 100 write_bytes 20\n".format(bench.kernel_source_hash()))
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(summ))
    assert bench.traffic_from_summary("bwd_dkdv") == 120.0
    assert bench.traffic_from_summary("nothing_like_it") is None
    summ.write_text(summ.read_text().replace(bench.kernel_source_hash(), "0000000000000000"))
    assert bench.traffic_from_summary("bwd_dkdv") is None


def test_counter_lookup_needs_matching_sources(tmp_path, monkeypatch):
    summ = tmp_path / "sq.txt"
    summ.write_text("command: x\nsource_hash {}\nvalues: average\n"
                    "kernel 'k_fwd_bf16_kernel'\n  MfmaUtil 48.5\n  VALUBusy 40\n"
                    "kernel 'k_bwd_dkdv_kernel'\n  MfmaUtil 50.25\n".format(bench.kernel_source_hash()))
    monkeypatch.setattr(bench, "SQ_SUMMARY", str(summ))
    assert bench.counter_from_summary("fwd_bf16", "MfmaUtil") == 48.5
    assert bench.counter_from_summary("bwd_dkdv", "MfmaUtil") == 50.25
    assert bench.counter_from_summary("bwd_dkdv", "VALUBusy") is None
    assert bench.counter_from_summary("bwd_dq_kernel", "MfmaUtil") is None
    summ.write_text(summ.read_text().replace(bench.kernel_source_hash(), "0000000000000000"))
    assert bench.counter_from_summary("fwd_bf16", "MfmaUtil") is None


def test_summary_lookups_on_the_committed_profiles():
    # the committed summaries name every bench kernel (when they match the sources)
    if bench.counter_from_summary(bench.KERNEL_KEYS["fwd"], "MfmaUtil") is None:
        pytest.skip("committed counter summary predates the kernel sources")
    for key in bench.KERNEL_KEYS.values():
        assert bench.counter_from_summary(key, "MfmaUtil") is not None, key
        assert bench.traffic_from_summary(key) is not None, key


def test_summarize_stats_and_counters(tmp_path):
    stats = [{"Name": "bwd_dkdv_kernel", "Calls": "3", "TotalDurationNs": "3000000", "AverageNs": "1000000",
              "MinNs": "900000", "MaxNs": "1100000", "Percentage": "75.0"},
             {"Name": "fwd_bf16_kernel", "Calls": "3", "TotalDurationNs": "1000000", "AverageNs": "333333",
              "MinNs": "300000", "MaxNs": "400000", "Percentage": "25.0"}]
    _write_csv(str(tmp_path / "s" / "run_kernel_stats.csv"), stats)
    out = tmp_path / "stats.txt"
    bench.summarize_stats(str(tmp_path / "s"), str(out), "cmd")
    lines = out.read_text().splitlines()
    assert lines[3].startswith("bwd_dkdv_kernel") and "1000.00" in lines[3]
    cnt = [{"Kernel_Name": "fwd_bf16_kernel", "Counter_Name": "MfmaUtil", "Counter_Value": 40.0},
           {"Kernel_Name": "fwd_bf16_kernel", "Counter_Name": "MfmaUtil", "Counter_Value": 60.0}]
    _write_csv(str(tmp_path / "c" / "run_counter_collection.csv"), cnt)
    out2 = tmp_path / "cnt.txt"
    bench.summarize_counters([str(tmp_path / "c")], str(out2), "cmd")
    body = out2.read_text()
    assert "MfmaUtil" in body and " 50" in body


@pytest.mark.parametrize("n_q,n_k,causal", [(37, 37, True), (50, 130, True), (130, 50, True),
                                            (50, 130, "bottom_right"), (130, 50, "bottom_right"),
                                            (64, 64, False), (1, 9, "bottom_right")])
def test_forward_flop_convention(n_q, n_k, causal):
    w = workloads.custom(2, 3, n_q, n_k, 16, "bf16", causal)
    per_pair = 4 * 16 * 2 * 3
    if not causal:
        want = per_pair * n_q * n_k
    elif n_q == n_k:
        want = per_pair * n_q * n_k / 2          # the usual convention for square causal
    else:
        off = n_k - n_q if causal == "bottom_right" else 0
        want = per_pair * np.clip(np.arange(n_q) + off + 1, 0, n_k).sum()
    assert w.fwd_flop() == want
    assert w.fwd_bwd_flop() == 3.5 * want


def test_headline_workload_flops():
    w = workloads.WORKLOADS[workloads.HEADLINE]
    assert (w.batch, w.heads, w.n_q, w.n_k, w.d, w.dtype, w.causal) == (2, 32, 4096, 4096, 128, "bf16", True)
    assert w.fwd_flop() == 4 * 4096 * 4096 * 128 * 64 / 2


def test_amd_smi_parse():
    text = ("GPU: 0\n    POWER:\n        SOCKET_POWER: 1385 W\n    CLOCK:\n        GFX_0:\n"
            "            CLK: 1855 MHz\n            MIN_CLK: 500 MHz\n        GFX_1:\n            CLK: 1700 MHz\n")
    assert bench.parse_amd_smi(text) == (1385.0, 1855.0)
    assert bench.parse_amd_smi("nothing") == (None, None)


def test_stats_median_and_min():
    assert bench._stats([3.0, 1.0, 2.0]) == {"median": 2.0, "min": 1.0, "mean": 2.0}
    assert bench._stats([4.0, 1.0, 2.0, 3.0])["median"] == 2.5


def test_oracle_sample_is_bounded_and_whole_heads():
    for name, w in workloads.WORKLOADS.items():
        heads = bench.oracle_sample(w)
        assert 1 <= len(heads) <= w.batch * w.heads
        assert len(set(heads)) == len(heads)
        assert all(0 <= b < w.batch and 0 <= h < w.heads for b, h in heads)
        # a bounded amount of fp64 work, or a single head
        assert len(heads) == 1 or bench.oracle_flop_per_head(w) * len(heads) <= bench.ORACLE_SAMPLE_FLOP


def test_cpu_oracle_pool_matches_whole_heads():
    # the pool's chunked tasks compute the same per-head results the oracle
    # gives for the whole head (timing entry point, small workload)
    import torch
    w = workloads.custom(1, 2, 700, 300, 32, "f32", True)
    q, k, v, do = workloads.make_inputs(w, seed=3)
    t = bench.cpu_oracle_times(w, q, k, v, do, [(0, 0), (0, 1)])
    assert t["fwd_s"] > 0 and t["fwd_bwd_s"] > 0 and 1 <= t["workers"] <= bench.CPU_SHARE
    e = bench.cpu_baseline_entry(w, q, k, v, do, [(0, 1)], gpu_fwd_ms=0.01, gpu_step_ms=0.03)
    assert e["oracle_flop_fwd_bwd"] == 12.0 * 700 * 300 * 32
    assert e["gpu_over_oracle_fwd_bwd"] > 0 and e["cores"] >= 1


def test_rocminfo_parse(monkeypatch):
    import subprocess as sp
    text = ("Agent 1\n  Name: cpu\nAgent 2\n  Name:                    gfx950\n  Marketing Name:          AMD Instinct MI355X\n"
            "  Vendor Name:             AMD\n  Compute Unit:            256\n  Max Clock Freq. (MHz):   2400\n")

    class R:
        stdout = text
    monkeypatch.setattr(sp, "run", lambda *a, **k: R())
    info = bench.device_info()
    assert info == {"rocminfo_compute_units": 256, "rocminfo_max_clock_mhz": 2400,
                    "name": "AMD Instinct MI355X"}


def test_summarize_io_per_path_and_scaled(tmp_path, monkeypatch):
    # one path per process; FETCH_SIZE of the 512 MiB copy reads half its
    # bytes (scale 2), WRITE_SIZE all of them; three calls per path
    mib = 1 << 20
    copy_f = {"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE", "Counter_Value": 512 * 1024 / 2}
    copy_w = {"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE", "Counter_Value": 512 * 1024}

    def rows(counter, spec):
        return [{"Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v} for k, v in spec]
    gemm, soft = "Cijk_Alik_Bljk_BBS", "cunn_SoftMaxForward"
    pp, merge = "_ZN2fa12_GLOBAL__N_113fwd_pp_kernelIL", "_ZN2fa12_GLOBAL__N_116fwd_merge_kernelIL"
    other = "at::native::reduce_kernel"
    runs = {
        "materialising": ([copy_f] + rows("FETCH_SIZE", [(gemm, 300.0)] * 6 + [(soft, 600.0)] * 3 + [(other, 1e6)]),
                          [copy_w] + rows("WRITE_SIZE", [(gemm, 100.0)] * 6 + [(soft, 300.0)] * 3)),
        "fused": ([copy_f] + rows("FETCH_SIZE", [(pp, 10.0)] * 3), [copy_w] + rows("WRITE_SIZE", [(pp, 5.0)] * 3)),
        "fused_split": ([copy_f] + rows("FETCH_SIZE", [(pp, 4.0)] * 12 + [(merge, 20.0)] * 3),
                        [copy_w] + rows("WRITE_SIZE", [(pp, 4.0)] * 12 + [(merge, 5.0)] * 3)),
    }
    for path, (f, w) in runs.items():
        _write_csv(str(tmp_path / "io" / f"f4096_{path}" / "run_counter_collection.csv"), f)
        _write_csv(str(tmp_path / "io" / f"w4096_{path}" / "run_counter_collection.csv"), w)
    out = tmp_path / "io.txt"
    bench.summarize_io(str(tmp_path / "io"), str(out), "cmd", copy_bytes=512 * mib)
    monkeypatch.setattr(bench, "IO_SUMMARY", str(out))
    t = bench.io_traffic_from_summary(4096)
    # per call: fetch KiB x 2 + write KiB, over the 3 calls the anchor kernel counts
    assert t["materialising"] == ((6 * 300 + 3 * 600) * 2 + 6 * 100 + 3 * 300) * 1024 / 3
    assert t["fused"] == (3 * 10 * 2 + 3 * 5) * 1024 / 3
    assert t["fused_split"] == ((12 * 4 + 3 * 20) * 2 + 12 * 4 + 3 * 5) * 1024 / 3
    assert bench.io_traffic_from_summary(1024) == {}
    out.write_text(out.read_text().replace(bench.kernel_source_hash(), "0000000000000000"))
    assert bench.io_traffic_from_summary(4096) == {}
