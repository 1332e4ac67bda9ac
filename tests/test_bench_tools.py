"""The measurement tooling of bench.py on small rocprofv3-shaped CSV fixtures (CPU only): the kernel
trace summary (statistics table and per-grid grouping), the counter summary (the copy calibration
scales FETCH_SIZE and WRITE_SIZE, bytes per dispatch, MFMA figures) and the traffic file, whose
source hash must match the fused kernel's sources for the bench to report it."""
import csv
import json
import os

import pytest

import bench


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


FUSED = "void fdl::attn_mha_kernel<128, false, false, true, false, false>(fdl::MhaParams)"
COPY = "void at::native::vectorized_elementwise_kernel<8, at::native::neg_kernel_cuda(at::TensorIterator&)>"


def test_summarize_trace(tmp_path):
    d = str(tmp_path / "kt")
    _write(os.path.join(d, "kt_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
           [[FUSED, 3, 69000, 23000, 75.0, 22000, 24000, 800], ["other", 1, 23000, 23000, 25.0, 23000, 23000, 0]])
    _write(os.path.join(d, "kt_kernel_trace.csv"),
           ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z",
            "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z"],
           [[FUSED, 0, 22000, 131072, 1, 1, 512, 1, 1], [FUSED, 50000, 74000, 131072, 1, 1, 512, 1, 1],
            [FUSED, 90000, 113000, 65536, 1, 1, 512, 1, 1], ["other", 0, 1000, 64, 1, 1, 64, 1, 1]])
    text = bench.summarize_trace(d, "fixture", "rocprofv3 ... -- python3 bench.py")
    lines = text.splitlines()
    assert lines[0] == "# Kernel trace: fixture" and "    rocprofv3 ... -- python3 bench.py" in lines
    assert f"| `{FUSED}` | 3 | 69.0 | 23.000 | 22.000 | 24.000 | 75.00 |" in lines
    # the fused kernel's two grids are kept apart; 'other' is no fdl:: kernel and is left out there
    assert f"| `{FUSED}` | (131072, 1, 1) / (512, 1, 1) | 2 | 23.000 | 22.000 | 24.000 |" in lines
    assert f"| `{FUSED}` | (65536, 1, 1) / (512, 1, 1) | 1 | 23.000 | 23.000 | 23.000 |" in lines
    assert not any(l.startswith("| `other` | (") for l in lines)


def _counters(d, name, counter_rows):
    _write(os.path.join(d, f"{name}_counter_collection.csv"),
           ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], counter_rows)


def test_summarize_counters_scaling_and_traffic_file(tmp_path):
    f, w, m = str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "m")
    # a 4 MiB copy reads as 2048 KiB of FETCH_SIZE (x 2.0) and 4096 KiB of WRITE_SIZE (x 1.0); the fused
    # kernel's two dispatches each sum two counter instances (per-XCD rows of one dispatch)
    _counters(f, "f", [[1, COPY, "FETCH_SIZE", 2048.0],
                       [2, FUSED, "FETCH_SIZE", 30000.0], [2, FUSED, "FETCH_SIZE", 10000.0],
                       [3, FUSED, "FETCH_SIZE", 25000.0], [3, FUSED, "FETCH_SIZE", 15000.0]])
    _counters(w, "w", [[1, COPY, "WRITE_SIZE", 4096.0], [2, FUSED, "WRITE_SIZE", 4600.0],
                       [3, FUSED, "WRITE_SIZE", 4600.0]])
    _counters(m, "m", [[2, FUSED, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 4.0e6], [2, FUSED, "SQ_VALU_MFMA_BUSY_CYCLES", 2.0e6],
                       [2, FUSED, "SQ_BUSY_CU_CYCLES", 1.0e8], [2, FUSED, "GRBM_GUI_ACTIVE", 6.4e5]])
    out = tmp_path / "traffic.json"
    text = bench.summarize_counters(f, w, 4, ["cmd-f", "cmd-w", "cmd-m"], m, str(out))
    assert "scale factors fetch x2.0000, write x1.0000" in text
    d = json.loads(out.read_text())
    assert d["fetch_kib_per_dispatch"] == pytest.approx(40000.0)
    assert d["write_kib_per_dispatch"] == pytest.approx(4600.0)
    assert d["hbm_bytes_per_dispatch"] == pytest.approx((40000.0 * 2 + 4600.0) * 1024)
    assert d["mfma_bf16_flop_per_dispatch"] == pytest.approx(4.0e6 * 512)
    assert d["mfma_busy_frac"] == pytest.approx(2.0e6 / (6.4e5 / 8 * 1024))
    assert d["commands"] == ["cmd-f", "cmd-w", "cmd-m"]
    # the hash is that of the kernel's current sources, so the bench would report this figure
    real = bench.TRAFFIC_FILE
    try:
        bench.TRAFFIC_FILE = str(out)
        assert bench.measured_traffic() == pytest.approx((40000.0 * 2 + 4600.0) * 1024)
        d["source_sha256"] = "0" * 64   # sources changed since: no figure
        out.write_text(json.dumps(d))
        assert bench.measured_traffic() is None and bench.mfma_figures(23.0) is None
    finally:
        bench.TRAFFIC_FILE = real



def test_algorithmic_bytes_of_the_32k_layer_and_step():
    """The byte counts behind the roofline, term by term for the 32K layer with 65 blocks kept per
    head (the sink block and the top 64): K and V of 2080 selected 64-token blocks, Q and O and the
    decode block's own K and V (bf16), the selection indices and counts, the pooled keys (float32)
    and the scores written."""
    from synth import get_config
    cfg = get_config(3)
    units = 32 * 65
    terms = {"selected K+V": units * 64 * 128 * 2 * 2, "Q+O": 32 * 32 * 128 * 2 * 2,
             "own K+V": 32 * 32 * 128 * 2 * 2, "indices": units * 4 + 32 * 4,
             "pooled keys": 32 * 512 * 128 * 4, "scores": 32 * 512 * 4}
    assert terms["selected K+V"] == 68_157_440 and terms["pooled keys"] == 8_388_608
    assert bench.sparse_launch_bytes(cfg, units) == sum(terms.values()) == 77_668_608
    sb = bench.step_bytes(cfg, units)
    kv = 32 * 32768 * 128 * 2   # one layer's cached K (or V)
    assert sb["dense_layer"] == 2 * kv + 2 * 524_288
    assert sb["source_layer"] == 77_668_608 + kv + 32 * 32 * 128 * 2   # the scan reads every K and the block's own
    assert sb["step"] == 2 * sb["dense_layer"] + sb["source_layer"] + 29 * 77_668_608 == 3_674_594_816
