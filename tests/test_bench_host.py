"""Host-side logic of bench.py (no GPU): the algorithmic byte counts the
roofline fractions are quoted with, and the counter-traffic record (scaling by
the device copy, and withheld once the kernel sources change)."""
import json

import pytest

import bench


def test_head_bytes_match_the_stated_per_launch_figures():
    # B=64 fp32 fused-norm decode: 64 KiB tile read + written, q and k of the
    # key head shared by 3 value heads, v, alpha, beta, z and the fp32 output
    per_head = 2 * 128 * 128 * 4 + 2 * 128 * 4 / 3 + 128 * 4 + 8 + 128 * 4 + 128 * 4
    assert bench.head_bytes(128, 48, 16, 4, 4, True) == pytest.approx(per_head)
    assert round(64 * 48 * bench.head_bytes(128, 48, 16, 4, 4, True)) == 408_444_928
    # B=256 binary16 state with a bf16 output
    assert round(256 * 48 * bench.head_bytes(128, 48, 16, 2, 2, True)) == 825_327_616
    # raw output: no z
    assert bench.head_bytes(128, 48, 16, 4, 4, False) == pytest.approx(per_head - 128 * 4)


def _counter_csv(path, counter, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, value) in enumerate(rows):
            f.write(f'{i + 1},"{name}",{counter},{value}\n')


def test_pmc_record_scaling_and_hash_gate(tmp_path, monkeypatch):
    kernel = "void gdn::decode_kernel<128, float, 1, 16, 1>(gdn::StepArgs)"
    verify = "void gdn::verify_kernel<128, true>(gdn::StepArgs, float*, long)"
    copy = "__amd_rocclr_copyBuffer"
    root = tmp_path / "passes"
    # the 1 GiB copy reads 512 Ki KiB of FETCH_SIZE (factor 2) and writes
    # 1 Mi KiB of WRITE_SIZE (factor 1); a smaller copy must not be taken
    _counter_csv(root / "fetch" / "fetch_counter_collection.csv", "FETCH_SIZE",
                 [(copy, 1000.0), (copy, 524288.0), (kernel, 100000.0), (kernel, 100002.0),
                  (verify, 1000.0), (verify, 1000.0), (verify, 3000.0), (verify, 3000.0)])
    _counter_csv(root / "write" / "write_counter_collection.csv", "WRITE_SIZE",
                 [(copy, 2000.0), (copy, 1048576.0), (kernel, 200000.0), (kernel, 200000.0),
                  (verify, 0.0), (verify, 0.0), (verify, 0.0), (verify, 0.0)])
    _counter_csv(root / "insts" / "insts_counter_collection.csv", "SQ_WAVES",
                 [(kernel, 49152.0), (kernel, 49152.0)])
    _counter_csv(root / "insts2" / "insts2_counter_collection.csv", "SQ_INSTS_VALU",
                 [(kernel, 49152.0 * 240), (kernel, 49152.0 * 240)])
    out = tmp_path / "pmc.json"
    monkeypatch.setattr(bench, "PMC_FILE", str(out))
    monkeypatch.setattr(bench, "PMC_DETAIL_FILE", str(tmp_path / "detail.json"))
    monkeypatch.setattr(bench, "PMC_TABLE_FILE", str(tmp_path / "table.md"))
    bench.pmc_summarize(str(root))
    rec = json.loads(out.read_text())
    assert rec["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["calibration"]["write_factor"] == pytest.approx(1.0)
    assert rec["fetch_bytes_per_launch"] == int(100001.0 * 1024 * 2)
    assert rec["write_bytes_per_launch"] == int(200000.0 * 1024)
    assert abs(rec["bytes_per_launch"] - rec["fetch_bytes_per_launch"] - rec["write_bytes_per_launch"]) <= 1
    assert rec["kernel_hash"] == bench.kernel_hash()
    assert bench.pmc_traffic(408_444_928) == rec["bytes_per_launch"]
    detail = json.loads((tmp_path / "detail.json").read_text())["kernels"]
    assert detail[kernel]["valu_insts_per_wave"] == pytest.approx(240.0)
    # verify: the first half of its dispatches is T = 2, the second T = 4
    v2, v4 = detail[verify + " [T=2]"], detail[verify + " [T=4]"]
    t2 = 64 * 3 * 48 * 128 * 128 * 4.0 + 64 * 2 * 48 * (bench.head_bytes(128, 48, 16, 4, 4, True)
                                                          - 2 * 128 * 128 * 4)
    assert v2["algorithmic_bytes_per_launch"][0] == int(t2)
    assert v4["algorithmic_bytes_per_launch"][0] > v2["algorithmic_bytes_per_launch"][0]
    assert v2["FETCH_SIZE"] == pytest.approx(1000.0) and v4["FETCH_SIZE"] == pytest.approx(3000.0)
    assert "verify_kernel" in (tmp_path / "table.md").read_text()
    # a record taken on other kernel sources is not reported
    rec["kernel_hash"] = "0" * 16
    out.write_text(json.dumps(rec))
    assert bench.pmc_traffic(408_444_928) is None


def test_committed_record_names_the_timed_kernel():
    with open(bench.PMC_FILE) as f:
        rec = json.load(f)
    assert rec["kernel"] == "void gdn::decode_kernel<128, float, 1, 16, 1>(gdn::StepArgs)"
    assert rec["algorithmic_bytes_per_launch"] == 408_444_928
    assert rec["kernel_sources"] == list(bench.KERNEL_SOURCES)


def test_cpu_model_is_a_string():
    assert isinstance(bench.cpu_model(), str)


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_code_hash_ignores_comments_only():
    a = b"// header\nint f(int x) {  /* inline\n comment */\n  return x + 1;  // tail\n}\n"
    b = b"// a different header\n\nint f(int x) {\n  return x + 1;\n}\n"
    c = b"int f(int x) {\n  return x + 2;\n}\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
