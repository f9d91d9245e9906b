"""Host-side checks of the rocprofv3 summary helpers (no GPU)."""

import csv
import json
import re

from soft_lsh_sparse_amd import profiling

FIELDS = ["Kernel_Name", "Counter_Name", "Counter_Value"]


def _pmc(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})
    return str(path)


ATTN = ("void socket_lsh::(anonymous namespace)::sparse_attn_kernel<socket_lsh::BF16, "
        "128, 64>(int)")
SCORE = "void socket_lsh::(anonymous namespace)::score_kernel_rot<4, 8>(ScoreArgs)"


def test_traffic_summary_scales_by_the_copy_and_round_trips(tmp_path):
    fetch = _pmc(tmp_path / "f.csv", "FETCH_SIZE",
                 [(ATTN, 100.0), (ATTN, 300.0), (SCORE, 50.0), ("other", 9.0)])
    write = _pmc(tmp_path / "w.csv", "WRITE_SIZE", [(ATTN, 10.0), (ATTN, 10.0), (SCORE, 40.0)])
    cfetch = _pmc(tmp_path / "cf.csv", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 512.0)])
    cwrite = _pmc(tmp_path / "cw.csv", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1024.0)])
    out = tmp_path / "t.md"
    data = profiling.write_traffic_summary(fetch, write, cfetch, cwrite, 1 << 20, str(out),
                                           "cmd", "copy cmd", "t")
    assert data["f_fetch"] == 2.0 and data["f_write"] == 1.0
    # mean FETCH 200 KiB x 2 + mean WRITE 10 KiB x 1
    assert data["kernels"]["sparse_attn_kernel"]["traffic_bytes"] == (400 + 10) * 1024
    assert data["kernels"]["score_kernel"]["traffic_bytes"] == (100 + 40) * 1024
    assert profiling.load_traffic(str(out), "sparse_attn_kernel") == 410 * 1024
    assert profiling.load_traffic(str(out), "score_kernel") == 140 * 1024
    assert profiling.load_traffic(str(out), "topk_filter_kernel") is None
    assert profiling.load_traffic(str(tmp_path / "missing.md"), "score_kernel") is None


def test_stale_counters_are_not_reported(tmp_path):
    fetch = _pmc(tmp_path / "f.csv", "FETCH_SIZE", [(ATTN, 100.0)])
    write = _pmc(tmp_path / "w.csv", "WRITE_SIZE", [(ATTN, 10.0)])
    cfetch = _pmc(tmp_path / "cf.csv", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 1.0)])
    cwrite = _pmc(tmp_path / "cw.csv", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1.0)])
    out = tmp_path / "t.md"
    profiling.write_traffic_summary(fetch, write, cfetch, cwrite, 1024, str(out), "c", "c", "t")
    text = out.read_text()
    block = re.search(r"```json\n(.*?)\n```", text, re.S).group(1)
    data = json.loads(block)
    data["kernels"]["sparse_attn_kernel"]["source_sha256"] = "0" * 64
    out.write_text(text.replace(block, json.dumps(data)))
    assert profiling.load_traffic(str(out), "sparse_attn_kernel") is None


def test_short_names():
    assert profiling.short_name(ATTN) == "sparse_attn_kernel"
    assert profiling.canonical(profiling.short_name(SCORE)) == "score_kernel"
    assert profiling.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
    assert profiling.short_name("at::native::foo") is None


def test_counter_summary_means_per_kernel(tmp_path):
    path = tmp_path / "c.csv"
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for name, counter, value in [(SCORE, "SQ_INSTS_LDS", 10), (SCORE, "SQ_INSTS_LDS", 30),
                                     (SCORE, "SQ_INSTS_VALU", 7), (SCORE, "SQ_INSTS_VALU", 9),
                                     (ATTN, "SQ_INSTS_LDS", 4), ("other", "SQ_INSTS_LDS", 1)]:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})
    out = tmp_path / "c.md"
    data = profiling.write_counter_summary(str(path), str(out), "cmd", "t")
    assert data["kernels"]["score_kernel_rot<4, 8>"] == {"dispatches": 2, "SQ_INSTS_LDS": 20.0,
                                                         "SQ_INSTS_VALU": 8.0}
    assert data["kernels"]["sparse_attn_kernel<socket_lsh::BF16, 128, 64>"]["dispatches"] == 1
    assert len(data["kernels"]) == 2
    text = out.read_text()
    assert "| `score_kernel_rot<4, 8>` | 2 |" in text


def test_counter_summary_keeps_template_instances_apart(tmp_path):
    path = tmp_path / "c.csv"
    other = SCORE.replace("<4, 8>", "<4, 16>")
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for name, value in [(SCORE, 10), (SCORE, 30), (other, 100)]:
            w.writerow({"Kernel_Name": name, "Counter_Name": "SQ_WAVES", "Counter_Value": value})
    data = profiling.write_counter_summary(str(path), str(tmp_path / "c.md"), "cmd", "t")
    assert data["kernels"]["score_kernel_rot<4, 8>"]["SQ_WAVES"] == 20.0
    assert data["kernels"]["score_kernel_rot<4, 16>"]["SQ_WAVES"] == 100.0
