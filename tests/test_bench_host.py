"""bench.py's host-side pieces: the traffic figures written from rocprofv3
counter collections (scaled by the calibration copy in the same run)."""
import csv
import json

import bench

HEADER = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(at::TensorIteratorBase&)>"
GATHER = "mla::(anonymous namespace)::gather_kernel(HIP_vector_type<unsigned int, 4u> const*, int)"
# a function template's instance demangles with its return type and arguments
GATHER_T = "void mla::(anonymous namespace)::gather_kernel<false>(HIP_vector_type<unsigned int, 4u> const*, int)"
ATTN = "mla::(anonymous namespace)::chunk_attention_kernel(mla::(anonymous namespace)::AttnArgs)"
OTHER = "void at::native::vectorized_gather_kernel<16, long>(char*, char*)"


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEADER)
        for d, name, v in rows:
            # rocprofv3 may split one dispatch's counter over several rows
            w.writerow([d, name, counter, v / 2])
            w.writerow([d, name, counter, v / 2])


def test_write_traffic_scales_by_the_calibration_copy(tmp_path):
    # the 1 GiB copy reads FETCH_SIZE = 512 Mi KiB units and WRITE_SIZE = 1 Mi:
    # fetch counts 2 bytes per KiB unit read, write 1
    _csv(tmp_path / "f.csv", "FETCH_SIZE",
         [(1, GATHER, 1000.0), (2, GATHER_T, 3000.0), (3, ATTN, 500.0), (4, NEG, 524288.0), (5, OTHER, 7.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE",
         [(1, GATHER, 2000.0), (2, GATHER_T, 2000.0), (3, ATTN, 100.0), (4, NEG, 1048576.0), (5, OTHER, 9.0)])
    out = tmp_path / "t.json"
    res = bench.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "demo", out_path=str(out))
    assert json.load(open(out)) == res
    assert res["fetch_scale"] == 2.0 and res["write_scale"] == 1.0
    k = res["kernels"]
    assert set(k) == {"gather_kernel", "chunk_attention_kernel"}
    assert k["gather_kernel"]["launches_profiled"] == 2
    assert k["gather_kernel"]["fetch_bytes_per_launch"] == 2000 * 1024 * 2
    assert k["gather_kernel"]["write_bytes_per_launch"] == 2000 * 1024
    assert k["chunk_attention_kernel"]["fetch_bytes_per_launch"] == 500 * 1024 * 2
    assert k["chunk_attention_kernel"]["sources"][0].endswith("attention.hip")
    assert k["gather_kernel"]["sources"][0].endswith("memory_ops.hip")


def test_cpu_baseline_reports_host_and_labels_extrapolation():
    import workloads as W
    wl = W.named_workloads()[1]
    b = W.make_batch(wl, canary=False)
    full = bench.cpu_baseline(b, wl)
    assert full["kind"] == "oracle" and full["oracle_ms_kind"] == "measured"
    assert full["cores"] >= 1 and full["machine_cpus"] >= full["cores"] and full["cpu_model"]
    assert abs(full["oracle_ms_per_step"] - full["seconds"] * 1e3) < 1.0  # both rounded
    part = bench.cpu_baseline(b, wl, sample_heads=2, sample_queries=3)
    assert part["oracle_ms_kind"] == "extrapolated" and "2 of 8 heads" in part["sample"]
    assert part["oracle_ms_per_step"] > part["seconds"] * 1e3
