"""Host-side logic of the benchmark and the traffic converter (no GPU needed)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from online_softmax_attention_pass_amd import traffic  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_counters(path, counter, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


SP = "void rf::attention_bf16_sp_kernel<{}>(unsigned short const*)"


def test_traffic_scales_by_the_copy_calibration(tmp_path):
    copy = "void at::native::vectorized_elementwise_kernel<4, AUnaryFunctor<MulFunctor<float> > >(int)"
    names = {
        "softmax": "void rf::softmax_rows_reg<float, 4, 512, 16>(float const*)",
        "layernorm": "void rf::layernorm_rows_reg<float, 4, 512, 16>(float const*)",
        "prefill": SP.format("128, 4, 2, false, false, 0, false"),
        "sparse": SP.format("64, 2, 2, false, false, 0, true"),
        "bitmap": SP.format("64, 2, 2, true, false, 0, true"),
        "decode": "void rf::decode_partial_kernel<128, 8>(unsigned short const*)",
        "attn_f32": "void rf::attention_f32_kernel<64>(float const*)",
    }
    # the fetch counter reads half of the copy's 1 GiB, the write counter all of it
    fetch = [(copy, 524288.0), (copy, 524288.0)] + [(n, 1000.0 * (i + 1)) for i, n in enumerate(names.values())]
    fetch += [(names["prefill"], 5000.0)]                         # second dispatch: mean is 4000
    write = [(copy, 1048576.0)] + [(n, 10.0 * (i + 1)) for i, n in enumerate(names.values())]
    fcsv, wcsv, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    _write_counters(fcsv, "FETCH_SIZE", fetch)
    _write_counters(wcsv, "WRITE_SIZE", write)
    traffic.main([str(out), f"copy,{','.join(names)}:{fcsv}:{wcsv}"])
    t = json.load(open(out))
    assert t["calibration"]["fetch_bytes_per_kib"] == pytest.approx(2048.0)
    assert t["calibration"]["write_bytes_per_kib"] == pytest.approx(1024.0)
    assert t["softmax"]["fetch_bytes"] == 1000 * 2048
    assert t["prefill"]["fetch_bytes"] == 4000 * 2048          # (3000 + 5000) / 2
    assert t["prefill"]["write_bytes"] == 30 * 1024
    assert t["decode"]["bytes_per_launch"] == 6000 * 2048 + 60 * 1024
    assert t["bitmap"]["fetch_bytes"] == 5000 * 2048
    assert t["layernorm"]["write_bytes"] == 20 * 1024
    assert t["prefill"]["source_sha"] == traffic.source_sha("attention_bf16.hip")


def test_traffic_keeps_shared_kernels_apart_by_run(tmp_path):
    """The ALiBi and window legs use one kernel instance: they are measured in
    different runs, and a run that holds both is rejected. Grouped-query
    decode (8 query heads per key/value head, 32-row tiles) and shared-cache
    decode (128-row tiles) use different instances."""
    copy = "vectorized_elementwise_kernel<MulFunctor>"
    gqa_k, split = SP.format("128, 1, 1, false, true, 0, false"), SP.format("128, 4, 2, false, true, 0, false")
    mod1 = SP.format("128, 4, 2, false, false, 1, false")
    runs = []
    for r, (wl, kn, kf) in enumerate((("copy,gqa,alibi", gqa_k, 100.0), ("mla,window", split, 300.0))):
        rows = ([(copy, 524288.0)] if r == 0 else []) + [(kn, kf), (mod1, kf + 1)]
        wrows = ([(copy, 1048576.0)] if r == 0 else []) + [(kn, kf), (mod1, kf + 1)]
        f, w = tmp_path / f"f{r}.csv", tmp_path / f"w{r}.csv"
        _write_counters(f, "FETCH_SIZE", rows)
        _write_counters(w, "WRITE_SIZE", wrows)
        runs.append(f"{wl}:{f}:{w}")
    out = tmp_path / "t.json"
    traffic.main([str(out)] + runs)
    t = json.load(open(out))
    assert t["gqa"]["fetch_bytes"] == 100 * 2048 and t["alibi"]["fetch_bytes"] == 101 * 2048
    assert t["mla"]["fetch_bytes"] == 300 * 2048 and t["window"]["write_bytes"] == 301 * 1024
    with pytest.raises(SystemExit):                    # one run may not hold both users of a kernel
        traffic.main([str(out), runs[0].replace("copy,gqa,alibi", "copy,gqa,alibi,window")])


def test_traffic_rejects_an_ambiguous_kernel(tmp_path):
    copy = "vectorized_elementwise_kernel<MulFunctor>"
    rows = [(copy, 1.0), ("softmax_rows_reg<float, 4>", 1.0), ("softmax_rows_stream<float>", 1.0)]
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_counters(fcsv, "FETCH_SIZE", rows)
    _write_counters(wcsv, "WRITE_SIZE", rows)
    with pytest.raises(SystemExit):
        traffic.main([str(tmp_path / "t.json"), f"copy,softmax:{fcsv}:{wcsv}"])


def test_bench_reports_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    import bench
    os.makedirs(tmp_path / "profiles")
    sha = bench.source_sha("softmax_rows.hip")
    json.dump({"softmax": {"source_sha": sha, "bytes_per_launch": 123},
               "decode": {"source_sha": "0" * 16, "bytes_per_launch": 456}},
              open(tmp_path / "profiles" / "traffic.json", "w"))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha", lambda name: sha if name == "softmax_rows.hip" else "f" * 16)
    assert bench.measured_traffic("softmax") == 123
    assert bench.measured_traffic("decode") is None      # kernel changed since the counters were taken
    assert bench.measured_traffic("prefill") is None     # never measured
    assert bench.measured_traffic("copy") is None        # calibration only


def test_source_sha_ignores_comments_but_not_code(tmp_path):
    """The staleness hash follows the code of a kernel and its local headers:
    comment and whitespace edits keep it, a code edit or a header's code edit
    changes it."""
    from online_softmax_attention_pass_amd import traffic
    (tmp_path / "h.h").write_text("int f() { return 1; }\n")
    (tmp_path / "k.hip").write_text('#include "h.h"\n// a kernel\nint g() { return f(); }\n')
    base = traffic.source_sha("k.hip", str(tmp_path))
    (tmp_path / "k.hip").write_text('#include "h.h"\n/* another\n comment */\nint g()  {\n return f();  }  // end\n')
    assert traffic.source_sha("k.hip", str(tmp_path)) == base
    (tmp_path / "k.hip").write_text('#include "h.h"\nint g() { return f() + 1; }\n')
    changed = traffic.source_sha("k.hip", str(tmp_path))
    assert changed != base
    (tmp_path / "h.h").write_text("int f() { return 2; }\n")
    assert traffic.source_sha("k.hip", str(tmp_path)) != changed


def test_cpu_baseline_plan_covers_every_workload():
    """Every benchmark workload (the calibration copy aside) has a bounded
    oracle sample on the CPU, with its work in the leg's own unit."""
    import bench
    import workloads as W
    for name in bench.SETUPS:
        if name == "copy":
            continue
        kind, tasks, work, unit, sample = bench.cpu_baseline_plan(name, W, 4)
        assert kind in ("attention", "decode", "softmax", "ext_attention", "layernorm", "gqa", "moe"), name
        assert 4 <= len(tasks) <= 4 * 1000 and work > 0 and unit in ("GB/s", "TFLOP/s") and sample, name


def test_cpu_baseline_prefill_work_is_the_causal_pairs():
    import bench
    import workloads as W
    c = W.CONFIGS["prefill"]
    _, tasks, work, _, _ = bench.cpu_baseline_plan("prefill", W, 4)
    pairs = sum(sum(i + 1 for i in range(r0, r1)) for _, _, _, r0, r1 in tasks)
    assert work == 4 * c["d"] * pairs
