"""Host logic of the rocprofv3 summaries: calibration arithmetic and the digest guard."""
import json
import os

from exact_io_aware_20_amd import profile_summary as ps


def _pmc_csv(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "p_counter_collection.csv"), "w") as f:
        f.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        for k, v in rows:
            f.write(f'"{k}","{counter}",{v}\n')


def test_traffic_calibration(tmp_path):
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)"
    dk = "void fa::fa_bwd_dkdv_kernel<128>(fa::BwdParams)"
    # the copy of 64 MiB reads as 32 MiB of FETCH_SIZE (scale 2) and 64 MiB of WRITE_SIZE
    _pmc_csv(tmp_path / "f", "FETCH_SIZE", [(neg, 32 * 1024), (dk, 100.0), (dk, 300.0)])
    _pmc_csv(tmp_path / "w", "WRITE_SIZE", [(neg, 64 * 1024), (dk, 50.0), (dk, 50.0)])
    t = ps.traffic(str(tmp_path / "f"), str(tmp_path / "w"), 64)
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["kernels"]["fa_bwd_dkdv_kernel<128>"]["bytes"] == 200.0 * 1024 * 2 + 50.0 * 1024


def test_committed_traffic_needs_matching_sources(tmp_path):
    md = tmp_path / "t.md"
    data = {"kernels": {"k": {"bytes": 123.0}}, "source_digest": ps.source_digest()}
    md.write_text("# x\n" + ps.TRAFFIC_TAG + " " + json.dumps(data) + "\n")
    assert ps.committed_traffic(str(md), "k") == 123.0
    assert ps.committed_traffic(str(md), "other") is None
    data["source_digest"] = "0" * 16
    md.write_text(ps.TRAFFIC_TAG + " " + json.dumps(data) + "\n")
    assert ps.committed_traffic(str(md), "k") is None
    assert ps.committed_traffic(str(tmp_path / "missing.md"), "k") is None


def test_short_name():
    assert ps.short_name("void fa::fa_bwd_dkdv_kernel<128>(fa::BwdParams)") == "fa_bwd_dkdv_kernel<128>"
