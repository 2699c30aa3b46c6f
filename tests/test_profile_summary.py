"""profile_summary.py's arithmetic on synthetic rocprofv3 CSV files (no GPU): kernel
durations and the timed tail, calibrated traffic and its ratio to the algorithmic bytes,
the per-XCD GRBM cycles, MFMA-busy and LDS ratios, and the traffic.json entry with the
hash of the kernel sources."""
import csv
import hashlib
import json
import os

import pytest

import profile_summary as P


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


@pytest.fixture
def fake(tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    (csrc / "k.hip").write_text("kernel source\n")
    profiles = tmp_path / "profiles"
    profiles.mkdir()
    traffic = profiles / "traffic.json"
    traffic.write_text(json.dumps({"_calibration": {"fetch": 2.0, "write": 1.0}}))
    monkeypatch.setattr(P, "CSRC", str(csrc))
    monkeypatch.setattr(P, "PROFILES", str(profiles))
    monkeypatch.setattr(P, "TRAFFIC", str(traffic))
    case = dict(title="synthetic", bench=["--workload", "x"], steps=3, timed=2,
                pmc=[["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
                      "SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE"]],
                kernels={"k_fake": ("fake_key", ["k.hip"], 1_000_000, 4.0e12)})
    monkeypatch.setattr(P, "CASES", {"fake": case})
    out = tmp_path / "out"
    # kernel trace: durations 10, 20, 30 us (ns timestamps), plus an unrelated kernel
    trace = [{"Kernel_Name": "void k_fake<8>(...)", "Start_Timestamp": s, "End_Timestamp": s + d}
             for s, d in ((1000, 10000), (50000, 20000), (90000, 30000))]
    trace.append({"Kernel_Name": "other", "Start_Timestamp": 5, "End_Timestamp": 7})
    _write_csv(str(out / "fake" / "trace" / "run_kernel_trace.csv"), trace)

    def counters(tag, values):
        rows = []
        for disp, v in enumerate(values):
            for name, val in v.items():
                rows.append({"Kernel_Name": "k_fake<8>", "Dispatch_Id": disp, "Counter_Name": name,
                             "Counter_Value": val, "Start_Timestamp": 0, "End_Timestamp": 1_000_000})
        _write_csv(str(out / "fake" / tag / "run_counter_collection.csv"), rows)

    counters("FETCH_SIZE", [{"FETCH_SIZE": 400.0}, {"FETCH_SIZE": 500.0}, {"FETCH_SIZE": 600.0}])
    counters("WRITE_SIZE", [{"WRITE_SIZE": 100.0}] * 3)
    counters("pmc1", [{"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 500.0, "SQ_INSTS_MFMA": 1000.0, "SQ_LDS_BANK_CONFLICT": 25.0,
                       "SQ_LDS_IDX_ACTIVE": 100.0, "SQ_ACTIVE_INST_VALU": 1024 * 100.0,
                       "GRBM_GUI_ACTIVE": 8 * 1000.0}] * 3)
    return out, profiles, traffic


def test_summary_arithmetic(fake):
    out, profiles, traffic = fake
    P.summarize("fake", str(out))
    text = (profiles / "fake.txt").read_text()
    # durations: all three dispatches (avg 20, min 10, max 30), the last two timed (avg 25)
    line = next(l for l in text.splitlines() if l.strip().startswith("k_fake") and "dispatches" not in l
                and "FETCH" not in l)
    assert line.split()[1:] == ["3", "20.0", "10.0", "30.0", "25.0"]
    # traffic: median FETCH 500 KiB x 2.0 + WRITE 100 KiB x 1.0 = 1,126,400 B against 1,000,000
    assert "traffic        1.1 MB" in text and "ratio 1.13" in text
    # GRBM summed over 8 XCDs -> 1000 cycles; MFMA busy 500 / 1000; LDS conflicts 25 %
    assert "GRBM_GUI_ACTIVE / 8 XCDs = 1000 cycles" in text
    assert "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs) = 50.0 %" in text
    assert "LDS bank conflict / LDS active = 25.0 %" in text
    assert "VALU active = SQ_ACTIVE_INST_VALU / (cycles x 1024 SIMDs) = 10.0 %" in text
    assert "MFMA instructions per dispatch 1000 (expected 30517578 of 32x32x64)" in text   # 4e12 / 131072
    entry = json.loads(traffic.read_text())["fake_key"]
    assert entry["bytes"] == 500 * 1024 * 2 + 100 * 1024
    assert entry["sources"] == ["k.hip"]
    assert entry["source_sha"] == hashlib.sha256(b"kernel source\0").hexdigest()[:16]
    assert entry["profile"] == "profiles/fake.txt"


def test_code_text_drops_comments_and_layout_only():
    src = ('int a = 1; // note "x"\n/* block\n comment */ const char* s = "a // kept";\n'
           "char c = '/';  int   b;\n")
    assert P.code_text(src) == 'int a = 1; const char* s = "a // kept"; char c = \'/\'; int b;'
    assert P.code_text('x = "q \\" // in the string"; // gone\n') == 'x = "q \\" // in the string";'


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    """A traffic entry stays valid across comment and layout edits of its kernel sources and
    is voided by a change of code; bench.py and profile_summary.py hash alike."""
    import bench
    k = tmp_path / "k.hip"
    monkeypatch.setattr(P, "CSRC", str(tmp_path))
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    k.write_text("__global__ void f(int* p) { p[0] = 1; }\n")
    h0 = P.source_sha(["k.hip"])
    assert bench.source_sha(["k.hip"]) == h0
    k.write_text("// what f does\n__global__ void f(int* p) {\n  p[0] = 1;  /* one */\n}\n")
    assert P.source_sha(["k.hip"]) == h0
    k.write_text("__global__ void f(int* p) { p[0] = 2; }\n")
    assert P.source_sha(["k.hip"]) != h0


def test_bench_traffic_entry_follows_its_sources(tmp_path, monkeypatch):
    """bench.py reports an entry's calibrated bytes while the kernel code matches the hash
    it was measured with, keeps them across a comment edit, and reports None after a code
    change or when the entry is missing."""
    import bench
    (tmp_path / "csrc").mkdir()
    k = tmp_path / "csrc" / "k.hip"
    k.write_text("__global__ void f(int* p) { p[0] = 1; }\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path / "csrc"))
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    (tmp_path / "traffic.json").write_text(json.dumps(
        {"k": {"bytes": 1234, "sources": ["k.hip"], "source_sha": bench.source_sha(["k.hip"])}}))
    assert bench._traffic("k") == 1234
    k.write_text("// f stores one\n__global__ void f(int* p) { p[0] = 1; }\n")
    assert bench._traffic("k") == 1234
    k.write_text("__global__ void f(int* p) { p[0] = 2; }\n")
    assert bench._traffic("k") is None
    assert bench._traffic("missing") is None


def test_source_hash_of_every_kernel_source_list():
    """The hash reads every source list the profiles name (UTF-8 comments included)."""
    import bench
    entries = json.load(open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                          "profiles", "traffic.json")))
    for key, e in entries.items():
        if isinstance(e, dict) and "sources" in e:
            h = bench.source_sha(e["sources"])
            assert len(h) == 16 and h == P.source_sha(e["sources"]), key
