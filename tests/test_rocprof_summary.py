"""The rocprofv3 summarizer that turns traces and counter files into the
tables under profiles/ (CPU; synthetic CSV files in a temporary directory)."""

import csv

from precision_rl_rollout_amd import rocprof_summary as rs


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_groups_by_kernel_and_launch_shape(tmp_path):
    hdr = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size", "VGPR_Count",
           "Workgroup_Size_X", "Grid_Size_X"]
    rows = [["void prr::gemm_decode_kernel<4, 4, false>(unsigned char const*)", 0, 30000, 73728,
             96, 512, 131072],
            ["void prr::gemm_decode_kernel<4, 4, false>(unsigned char const*)", 50000, 84000, 73728,
             96, 512, 131072],
            ["prr::fp8_weight_block_kernel(unsigned short const*)", 0, 70000, 512, 40, 256,
             2121728]]
    _write(tmp_path / "run_kernel_trace.csv", hdr, rows)
    out = rs.trace_table(str(tmp_path)).splitlines()
    assert out[2] == "| `gemm_decode_kernel` | 256 | 73728 | 96 | 2 | 32.00 | 30.00 | 34.00 |"
    assert out[3] == "| `fp8_weight_block_kernel` | 8288 | 512 | 40 | 1 | 70.00 | 70.00 | 70.00 |"


def test_counters_report_the_copy_calibration(tmp_path):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value", "Grid_Size", "Workgroup_Size",
           "LDS_Block_Size", "VGPR_Count"]
    rows = [["__amd_rocclr_copyBuffer", "FETCH_SIZE", 262144.0, 65536, 256, 0, 8],
            ["prr::kv_cache_write_kernel(x)", "FETCH_SIZE", 100.0, 524288, 256, 0, 24],
            ["prr::kv_cache_write_kernel(x)", "FETCH_SIZE", 200.0, 524288, 256, 0, 24],
            ["prr::kv_cache_write_kernel(x)", "WRITE_SIZE", 999.0, 524288, 256, 0, 24]]
    _write(tmp_path / "run_counter_collection.csv", hdr, rows)
    out = rs.counter_table(str(tmp_path), "FETCH_SIZE").splitlines()
    assert out[0] == "calibration copy: 262144.0 KiB -> scale 2.0000"
    assert out[-1] == "| `kv_cache_write_kernel` | 2048 | 0 | 24 | 2 | 150.0 |"


def test_trace_split_by_dispatch_order(tmp_path):
    hdr = ["Kernel_Name", "Dispatch_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
           "VGPR_Count", "Workgroup_Size_X", "Grid_Size_X"]
    k = "void prr::gemm_decode_kernel<4, 4, false>(unsigned char const*)"
    rows = [[k, 3, 0, 40000, 73728, 96, 512, 131072],     # dispatch order 1, 2, 3, 4
            [k, 1, 0, 10000, 73728, 96, 512, 131072],
            ["prr::fp8_act_group_kernel(x)", 2, 0, 5000, 0, 12, 256, 28672],
            [k, 2, 0, 20000, 73728, 96, 512, 131072],
            [k, 4, 0, 50000, 73728, 96, 512, 131072]]
    _write(tmp_path / "run_kernel_trace.csv", hdr, rows)
    out = rs.trace_table(str(tmp_path), "gemm_decode_kernel=1,2").splitlines()
    assert out[2] == "| `gemm_decode_kernel #1` | 256 | 73728 | 96 | 1 | 10.00 | 10.00 | 10.00 |"
    assert out[3] == "| `gemm_decode_kernel #2` | 256 | 73728 | 96 | 2 | 30.00 | 20.00 | 40.00 |"
    assert out[4] == "| `gemm_decode_kernel #3` | 256 | 73728 | 96 | 1 | 50.00 | 50.00 | 50.00 |"
    assert out[5].startswith("| `fp8_act_group_kernel` | 112 |")


def test_counters_other_than_bytes_carry_no_kib_unit(tmp_path):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value", "Grid_Size", "Workgroup_Size",
           "LDS_Block_Size", "VGPR_Count"]
    rows = [["__amd_rocclr_copyBuffer", "MfmaUtil", 0.0, 65536, 256, 0, 8],
            ["prr::gemm_prefill_kernel(x)", "MfmaUtil", 50.0, 1703936, 512, 135168, 124],
            ["prr::gemm_prefill_kernel(x)", "MfmaUtil", 55.0, 1703936, 512, 135168, 124]]
    _write(tmp_path / "run_counter_collection.csv", hdr, rows)
    out = rs.counter_table(str(tmp_path), "MfmaUtil").splitlines()
    assert not any(line.startswith("calibration copy") for line in out)
    assert out[0] == "| kernel | workgroups | LDS bytes | VGPRs | dispatches | MfmaUtil (mean) |"
    assert out[-1] == "| `gemm_prefill_kernel` | 3328 | 135168 | 124 | 2 | 52.5 |"
