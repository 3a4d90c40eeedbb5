"""The rocprof harness's parser and report writer on a small committed fixture
(tests/golden/rocprof/: rows cut from real rocprofv3 --output-format csv runs
on an MI355X -- kernel trace, FETCH_SIZE, WRITE_SIZE and MFMA counter passes of
the bench step, including the 1 GiB calibration copy, and a pass of the eight
stall counters over the GA and SWA prefill and the GA decode split kernel).  CPU only; the
expected figures are worked out by hand from the fixture rows quoted here."""
import json
import os

import pytest

from global_attention_mimo_amd import prof

FIX = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rocprof")
PREFILL = "void mimo::(anonymous namespace)::prefill_kernel<8, 1, 64, false, 2, false, false>"


def full(rows, short):
    return next(k for k in rows if prof.short_name(k) == short)


def test_short_names():
    assert prof.short_name("void mimo::(anonymous namespace)::ga_split_kernel<false>(unsigned short const*, int)") == \
        "ga_split_kernel<false>"
    assert prof.short_name("mimo::(anonymous namespace)::ga_combine_kernel(long long const*, float const*)") == \
        "ga_combine_kernel"
    assert prof.short_name(PREFILL + "(unsigned short const*, float)") == \
        "prefill_kernel<8, 1, 64, false, 2, false, false>"
    assert prof.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_ga_prefill_instantiation_is_recognised():
    assert prof.is_ga_prefill("prefill_kernel<8, 1, 64, false, 2, false, false>")
    assert prof.is_ga_prefill("prefill_kernel<8, 1, 64, false, 2, false, false, false>")
    assert not prof.is_ga_prefill("prefill_kernel<4, 1, 32, true, 2, false, false, false>")  # SWA
    assert not prof.is_ga_prefill("prefill_kernel<8, 1, 64, false, 2, true, false, false>")  # chunked
    assert not prof.is_ga_prefill("prefill_kernel<8, 1, 64, false, 2, true, false, true>")  # FP8 chunk
    assert not prof.is_ga_prefill("swa_stream_kernel<false, false>")


def test_trace_stats_from_fixture():
    st = prof.trace_stats(prof._csv_rows(os.path.join(FIX, "trace"), "kernel_trace.csv"))
    p = st[full(st, "prefill_kernel<8, 1, 64, false, 2, false, false>")]
    # dispatches 323, 332, 341: 21067042, 21428832, 19101666 ns
    assert p["dispatches"] == 3
    assert p["median_us"] == pytest.approx(21067.042)
    assert p["avg_us"] == pytest.approx((21067042 + 21428832 + 19101666) / 3e3)
    assert p["min_us"] == pytest.approx(19101.666) and p["max_us"] == pytest.approx(21428.832)
    g = st[full(st, "ga_split_kernel<false>")]  # 7479959 and 7433923 ns
    assert g["dispatches"] == 2 and g["median_us"] == pytest.approx((7479.959 + 7433.923) / 2)
    assert st[full(st, "ga_combine_kernel")]["total_ms"] == pytest.approx(0.013198)


def test_calibration_and_bytes_from_fixture():
    fetch = prof._csv_rows(os.path.join(FIX, "fetch"), "counter_collection.csv")
    write = prof._csv_rows(os.path.join(FIX, "write"), "counter_collection.csv")
    fs, ws = prof.calibration_scales(fetch, write)
    # The copy whose WRITE_SIZE is nearest 1 GiB is dispatch 315: WRITE 1048576 KiB, FETCH 524308.0625 KiB
    # (the 2 GiB copy 318 and the 512 MiB ones are farther).
    assert ws == pytest.approx(1.0)
    assert fs == pytest.approx(1048576 / 524308.0625)
    res = prof.summarize(FIX)
    kern = {prof.short_name(k): v for k, v in res["traffic"]["kernels"].items()}
    p = kern["prefill_kernel<8, 1, 64, false, 2, false, false>"]
    assert p["fetch_kib"] == pytest.approx(1908619.375) and p["write_kib"] == pytest.approx(532705.09375)
    assert p["read_bytes"] == pytest.approx(1908619.375 * 1024 * 1048576 / 524308.0625)
    assert p["write_bytes"] == pytest.approx(532705.09375 * 1024)
    assert kern["ga_split_kernel<false>"]["read_bytes"] / 1e9 == pytest.approx(44.478, abs=1e-3)
    assert not any("copy" in k for k in kern), "only library kernels are reported"


def test_mfma_busy_from_fixture():
    res = prof.summarize(FIX)
    m = {prof.short_name(k): v for k, v in res["mfma"].items()}
    # dispatch 325: SQ_VALU_MFMA_BUSY_CYCLES 21516779520, GRBM_GUI_ACTIVE 292159803 over 8 XCDs, 1024 SIMDs
    assert m["prefill_kernel<8, 1, 64, false, 2, false, false>"]["busy"] == \
        pytest.approx(21516779520 / (1024 * 292159803 / 8))
    assert m["prefill_kernel<8, 1, 64, false, 2, false, false>"]["insts_mfma"] == 672399360
    # effective clock: 292159803 / 8 cycles over the trace's median 21067.042 us
    assert m["prefill_kernel<8, 1, 64, false, 2, false, false>"]["clock_ghz"] == \
        pytest.approx(292159803 / 8 / 21067042)
    assert m["ga_combine_kernel"]["clock_ghz"] is None  # 13 us: too short for a clock estimate


def test_report_files(tmp_path):
    res = prof.summarize(FIX)
    md = tmp_path / "step.md"
    prof.write_markdown("step", FIX, res, str(md))
    text = md.read_text()
    assert "| `prefill_kernel<8, 1, 64, false, 2, false, false>` | 3 |" in text
    assert "rocprofv3 --pmc FETCH_SIZE --output-format csv" in text
    assert "-- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-next-rows --copy-calibration" in text
    rec = prof.write_traffic_record(res, str(tmp_path / "traffic.json"))
    on_disk = json.loads((tmp_path / "traffic.json").read_text())
    assert on_disk == rec
    assert rec["code_sha256"] == prof.code_digest(prof.TRAFFIC_SOURCES)
    assert rec["read_bytes"] + rec["write_bytes"] == pytest.approx(
        1908619.375 * 1024 * 1048576 / 524308.0625 + 532705.09375 * 1024)


def test_pass_commands_put_the_program_right_after_the_separator():
    for which in prof.PASSES:
        cmd = prof.pass_command("step", which, "/tmp/out", "python3")
        i = cmd.index("--")
        assert cmd[0] == "rocprofv3" and cmd[i + 1] == "python3" and cmd[i + 2].endswith("bench.py")
        pmc = which != "trace"
        assert ("--pmc" in cmd) == pmc and ("--copy-calibration" in cmd) == pmc
        assert not any(f in cmd for f in ("-s", "--sys-trace", "-r", "--runtime-trace"))


def test_bench_reads_the_committed_traffic_record():
    """bench.py's roofline traffic comes from the record prof.py writes, and
    only while the GA prefill sources still match its digest."""
    import bench
    rec = json.load(open(os.path.join(prof.ROOT, "profiles", "prefill_ga_1x32768_traffic.json")))
    assert rec["sources"] == prof.TRAFFIC_SOURCES
    if rec["code_sha256"] == prof.code_digest(rec["sources"]):
        assert bench.measured_traffic() == pytest.approx(rec["read_bytes"] + rec["write_bytes"])
    else:
        assert bench.measured_traffic() is None


def test_stall_fractions_from_fixture():
    """tests/golden/rocprof/stalls: one dispatch each of the GA prefill, the streaming SWA prefill and the GA
    split kernel (rows of a real --pmc run of the eight stall counters), plus a torch copy that is not reported."""
    res = prof.summarize(FIX)
    s = {prof.short_name(k): v for k, v in res["stalls"].items()}
    assert set(s) == {"prefill_kernel<8, 1, 64, false, 2, false, false, false>", "swa_stream_kernel<false, false>",
                      "ga_split_kernel<false>"}
    p = s["prefill_kernel<8, 1, 64, false, 2, false, false, false>"]
    # dispatch 15: SQ_WAVE_CYCLES 16968076230, SQ_WAIT_ANY 4509090417, SQ_WAIT_INST_ANY 6215074302,
    # SQ_ACTIVE_INST_ANY 6243911511, SQ_ACTIVE_INST_VALU 3961405721
    assert p["wave_cycles"] == 16968076230
    assert p["SQ_WAIT_ANY"] == pytest.approx(4509090417 / 16968076230)
    assert p["SQ_WAIT_INST_ANY"] == pytest.approx(6215074302 / 16968076230)
    assert p["SQ_ACTIVE_INST_ANY"] == pytest.approx(6243911511 / 16968076230)
    assert p["SQ_ACTIVE_INST_VALU"] == pytest.approx(3961405721 / 16968076230)
    g = s["ga_split_kernel<false>"]  # dispatch 97: 58552621 of 73456964 wave cycles ready but not issued
    assert g["SQ_WAIT_INST_ANY"] == pytest.approx(58552621 / 73456964)


def test_report_writes_the_stall_table(tmp_path):
    res = prof.summarize(FIX)
    md = tmp_path / "r.md"
    prof.write_markdown("step", FIX, res, str(md))
    text = md.read_text()
    assert "## Where the waves' cycles go" in text
    assert "| `swa_stream_kernel<false, false>` | 38.4% |" in text  # 133432366 / 347661741
