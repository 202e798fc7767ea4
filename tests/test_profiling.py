"""The HBM traffic record: copy-kernel scaling, staleness by source hash, and
the committed record's fields (host logic only)."""

import os

from tree_attention_verification_ancestor_amd import profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_record_scales_counters_by_the_copy_kernel(tmp_path):
    copy_bytes = 1 << 20
    # the counters read half of the fetched bytes and all of the written ones
    copy_fetch = {"copy": {"FETCH_SIZE": copy_bytes / 1024 / 2}}
    copy_write = {"copy": {"WRITE_SIZE": copy_bytes / 1024}}
    fetch = {"tree_attn_kernel": {"FETCH_SIZE": 100.0}, "tree_attn_combine_kernel": {"FETCH_SIZE": 10.0}}
    write = {"tree_attn_kernel": {"WRITE_SIZE": 20.0}, "tree_attn_combine_kernel": {"WRITE_SIZE": 5.0}}
    out = tmp_path / "rec.txt"
    rec = profiling.write_record(str(out), fetch, write, copy_fetch, copy_write, copy_bytes, "a ;; b")
    assert float(rec["fetch_factor"]) == 0.5 and float(rec["write_factor"]) == 1.0
    expect = (100 / 0.5 + 20) * 1024 + (10 / 0.5 + 5) * 1024
    assert int(rec["traffic_bytes_per_launch"]) == int(expect)
    assert profiling.current_traffic(str(out)) == int(expect)   # same source as now
    text = out.read_text()
    assert "#   a" in text and "#   b" in text


def test_stale_or_missing_record_gives_none(tmp_path, monkeypatch):
    out = tmp_path / "rec.txt"
    out.write_text("kernel_source_sha256 = 00\ntraffic_bytes_per_launch = 5\n")
    assert profiling.current_traffic(str(out)) is None
    assert profiling.current_traffic(str(tmp_path / "missing.txt")) is None
    monkeypatch.setattr(profiling, "source_sha256", lambda path=None: "00")
    assert profiling.current_traffic(str(out)) == 5


def test_committed_record_is_well_formed():
    path = os.path.join(ROOT, "profiles", "tree_attn_llama70b_hbm_traffic.txt")
    rec = profiling.read_record(path)
    for key in ("kernel_source_sha256", "fetch_factor", "write_factor", "traffic_bytes_per_launch",
                "tree_attn_kernel.fetch_kib", "tree_attn_kernel.write_kib"):
        assert key in rec, key
    assert int(float(rec["traffic_bytes_per_launch"])) > 0


def test_kernel_names_map_to_short_names():
    assert profiling.short_name("void tav::(anonymous namespace)::tree_attn_kernel<128, 8>(x)") == \
        "tree_attn_kernel"
    assert profiling.short_name("void tav::(anonymous namespace)::tree_attn_combine_kernel<128>(x)") == \
        "tree_attn_combine_kernel"
    assert profiling.short_name(
        "void at::native::vectorized_elementwise_kernel<4, at::native::CUDAFunctorOnSelf_add<float>, "
        "std::array<char*, 2ul> >(int)") == "copy"


def test_counter_summary_derives_ratios(tmp_path):
    # 2 XCDs of 1000 active cycles each, 4 SIMDs: 1000 SIMD-cycles per SIMD
    c = {"GRBM_GUI_ACTIVE": 2000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1000.0, "SQ_WAVE_CYCLES": 400.0,
         "SQ_WAIT_INST_ANY": 100.0, "SQ_LDS_IDX_ACTIVE": 50.0, "SQ_LDS_BANK_CONFLICT": 5.0,
         "SQ_INSTS_VALU_MFMA_MOPS_BF16": 3.0, "SQ_INSTS_VALU_MFMA_MOPS_F16": 1.0}
    d = profiling.derived_counters(c, xcds=2, simds=4)
    vals = {k.split(" = ")[0]: v for k, v in d.items()}
    assert vals["mfma_busy"] == 0.25
    assert d["SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES"] == 0.25
    assert d["SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE"] == 0.1
    assert vals["mfma_flops"] == 4 * 512
    out = tmp_path / "sq.txt"
    res = profiling.write_counter_summary(str(out), [{"tree_attn_kernel": c}], ["tree_attn_kernel"],
                                          2, 4, "x ;; y")
    text = out.read_text()
    assert "[tree_attn_kernel]" in text and "#   x" in text and "#   y" in text
    assert res["tree_attn_kernel"]["SQ_WAVE_CYCLES"] == 400.0
