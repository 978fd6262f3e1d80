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


def test_mfma_busy_fraction(tmp_path):
    fw = "void fa::fa_fwd_bf16_kernel<128, false>(fa::FwdParams)"
    d = tmp_path / "m"
    os.makedirs(d)
    with open(d / "p_agent_info.csv", "w") as f:
        f.write("Agent_Type,Simd_Count,Num_Xcc\nCPU,0,0\nGPU,1024,8\n")
    with open(d / "p_counter_collection.csv", "w") as f:
        f.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        # GRBM_GUI_ACTIVE summed over 8 XCDs: 1000 cycles each; the 1024 SIMDs' matrix
        # pipes busy 400 and 600 of them in the two dispatches
        for busy in (1024 * 400, 1024 * 600):
            f.write(f'"{fw}","SQ_VALU_MFMA_BUSY_CYCLES",{busy}\n')
            f.write(f'"{fw}","GRBM_GUI_ACTIVE",8000\n')
        f.write('"other_kernel","SQ_VALU_MFMA_BUSY_CYCLES",5\n"other_kernel","GRBM_GUI_ACTIVE",5\n')
    m = ps.mfma_busy(str(d))
    assert m["agent"] == {"simds": 1024, "xcc": 8}
    assert list(m["kernels"]) == ["fa_fwd_bf16_kernel<128, false>"]
    assert abs(m["kernels"]["fa_fwd_bf16_kernel<128, false>"]["frac"] - 0.5) < 1e-12


def test_digest_ignores_comments_only():
    code = "int f(int x) {\n    return x + 1;   // one more\n}\n/* block\n comment */\n"
    assert ps.code_text(code) == ps.code_text("int f(int x) { return x + 1; }")
    assert ps.code_text(code) != ps.code_text("int f(int x) { return x + 2; }")


def _counter_dir(tmp_path, name, rows):
    d = tmp_path / name
    os.makedirs(d)
    with open(d / "p_agent_info.csv", "w") as f:
        f.write("Agent_Type,Simd_Count,Num_Xcc\nCPU,0,0\nGPU,1024,8\n")
    with open(d / "p_counter_collection.csv", "w") as f:
        f.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        for k, c, v in rows:
            f.write(f'"{k}","{c}",{v}\n')
    return str(d)


def test_wave_state_shares(tmp_path):
    k = "void fa::fa_bwd_dq_kernel<128, false>(fa::BwdParams)"
    vals = {"SQ_WAVE_CYCLES": 1000, "SQ_ACTIVE_INST_ANY": 300, "SQ_WAIT_ANY": 350, "SQ_WAIT_INST_ANY": 350,
            "SQ_ACTIVE_INST_VALU": 200, "SQ_ACTIVE_INST_LDS": 50, "SQ_WAIT_INST_LDS": 30, "SQ_ACTIVE_INST_MISC": 10}
    rows = [(k, c, v) for c, v in vals.items()] + [("other_kernel", "SQ_WAVE_CYCLES", 7)]
    m = ps.wave_states(_counter_dir(tmp_path, "w", rows))
    assert list(m) == ["fa_bwd_dq_kernel<128, false>"]
    s = m["fa_bwd_dq_kernel<128, false>"]
    assert abs(s["SQ_ACTIVE_INST_ANY"] + s["SQ_WAIT_ANY"] + s["SQ_WAIT_INST_ANY"] - 1.0) < 1e-12
    assert abs(s["SQ_ACTIVE_INST_VALU"] - 0.2) < 1e-12


def test_lds_use_per_cu(tmp_path):
    k = "void fa::fa_fwd_bf16_kernel<128, false>(fa::FwdParams)"
    # 8 XCDs x 1000 cycles; 256 CUs; LDS busy 250 cycles per CU; 64 B/clk per CU loaded
    rows = [(k, "GRBM_GUI_ACTIVE", 8000), (k, "SQ_LDS_IDX_ACTIVE", 256 * 250),
            (k, "SQ_INSTS_LDS_LOAD_BANDWIDTH", 256 * 1000), (k, "SQ_LDS_BANK_CONFLICT", 0),
            (k, "SQ_LDS_DATA_FIFO_FULL", 0)]
    m = ps.lds_use(_counter_dir(tmp_path, "l", rows))
    v = m["kernels"]["fa_fwd_bf16_kernel<128, false>"]
    assert abs(v["busy"] - 0.25) < 1e-12
    assert abs(v["load_bytes_per_clk_cu"] - 64.0) < 1e-12


def test_valu_issue_share(tmp_path):
    k = "void fa::fa_fwd_persist_kernel<64, false>(fa::FwdParams)"
    # 8 XCDs x 1000 cycles on 1024 SIMDs; per SIMD 100 vector instructions (20 of them
    # exp) besides 10 MFMAs: (80 x 4 + 20 x 10) / 1000 = 0.52 of the cycles
    rows = [(k, "GRBM_GUI_ACTIVE", 8000), (k, "SQ_INSTS_VALU", 1024 * 110), (k, "SQ_INSTS_MFMA", 1024 * 10),
            (k, "SQ_INSTS_VALU_TRANS_F32", 1024 * 20), (k, "SQ_ACTIVE_INST_VALU", 0)]
    m = ps.valu_load(_counter_dir(tmp_path, "v", rows))
    v = m["kernels"]["fa_fwd_persist_kernel<64, false>"]
    assert abs(v["valu_issue_frac"] - 0.52) < 1e-12
    assert abs(v["valu_per_mfma"] - 10.0) < 1e-12
    md = tmp_path / "valu.md"
    ps._write_valu_md(m, str(md), "cmd")
    assert ps.committed_valu(str(md), "fa_fwd_persist_kernel<64, false>")["valu"] == 1024 * 100
    assert ps.committed_valu(str(md), "missing") is None
