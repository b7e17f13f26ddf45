"""Host-side checks of the rocprofv3 summary helper (no GPU)."""
import json
import os

from tree_causal_draft_parent_amd import profsum


def test_short_name():
    assert profsum.short_name("void jf::(anonymous namespace)::k_fuse_gemm_bf16<256>("
                              "jf::(anonymous namespace)::FuseArgs)") == "k_fuse_gemm_bf16<256>"
    assert profsum.short_name("jf::(anonymous namespace)::k_tree_attn_split("
                              "jf::(anonymous namespace)::AttnArgs)") == "k_tree_attn_split"
    assert profsum.short_name("void jf::(anonymous namespace)::k_topk_stage1<unsigned short, true>("
                              "unsigned short const*, long)") == "k_topk_stage1<unsigned short, true>"


def _counter_csv(path, rows):
    cols = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w") as f:
        f.write(",".join(f'"{c}"' for c in cols) + "\n")
        for i, (k, c, v) in enumerate(rows):
            f.write(f'{i},{i},"{k}","{c}",{v}\n')


def test_traffic_scaling(tmp_path):
    d = {n: tmp_path / n for n in ("f", "w", "cf", "cw")}
    for p in d.values():
        p.mkdir()
    g = "void jf::(anonymous namespace)::k_fuse_gemm_bf16<256>(jf::(anonymous namespace)::FuseArgs)"
    _counter_csv(d["f"] / "r_counter_collection.csv", [(g, "FETCH_SIZE", 1000.0), (g, "FETCH_SIZE", 1200.0)])
    _counter_csv(d["w"] / "r_counter_collection.csv", [(g, "WRITE_SIZE", 10.0)])
    copy = "void at::native::copy_kernel(int)"
    # the copy reads and writes 2048 KiB; the counters read 1024 / 4096 KiB
    _counter_csv(d["cf"] / "r_counter_collection.csv", [(copy, "FETCH_SIZE", 1024.0)])
    _counter_csv(d["cw"] / "r_counter_collection.csv", [(copy, "WRITE_SIZE", 4096.0)])
    out = tmp_path / "t.json"
    profsum.main(["traffic", "--fetch", str(d["f"]), "--write", str(d["w"]), "--copy-fetch", str(d["cf"]),
                  "--copy-write", str(d["cw"]), "--copy-bytes", str(2048 * 1024), "--workload", "x",
                  "--out", str(out)])
    rec = json.loads(out.read_text())
    k = rec["kernels"]["k_fuse_gemm_bf16<256>"]
    assert k["launches"] == 2
    assert k["fetch_bytes"] == round(1100.0 * 1024 * 2.0)
    assert k["write_bytes"] == round(10.0 * 1024 * 0.5)
    assert rec["sources_sha256"] == profsum.sources_hash()
    assert rec["file_sha256"] == profsum.file_hashes()
    assert "k_fuse.hip" in rec["file_sha256"] and "jf_internal.h" in rec["file_sha256"]
    assert os.path.exists(out)


def test_traffic_freshness_follows_the_calls_kernel_file(tmp_path, monkeypatch):
    # a changed unrelated source leaves a call's counters valid; a changed
    # kernel file of that call makes them stale
    import bench
    cur = profsum.file_hashes()
    rec = {"workload": "w", "sources_sha256": "x", "file_sha256": dict(cur),
           "kernels": {"k_fuse_gemm_bf16<256>": {"fetch_bytes": 10, "write_bytes": 5},
                       "k_fuse_reduce": {"fetch_bytes": 3, "write_bytes": 1}}}
    rec["file_sha256"]["k_tree.hip"] = "changed"
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(path))
    total, src = bench.measured_traffic("fuse", "w")
    assert total == 19 and "k_fuse.hip sha256" in src and "traffic.json" in src
    assert bench.measured_traffic("fuse", "other")[0] is None
    rec["file_sha256"]["k_fuse.hip"] = "changed"
    path.write_text(json.dumps(rec))
    total, src = bench.measured_traffic("fuse", "w")
    assert total is None and "changed" in src


def test_trace_split_by_grid(tmp_path, capsys):
    d = tmp_path / "trace"
    d.mkdir()
    hdr = '"Kind","Kernel_Name","Start_Timestamp","End_Timestamp","Grid_Size_X"\n'
    rows = ['"KERNEL_DISPATCH","void jf::(anonymous namespace)::k_fuse_gemm_bf16<256>(jf::FuseArgs)",100,2100,131072\n',
            '"KERNEL_DISPATCH","void jf::(anonymous namespace)::k_fuse_gemm_bf16<256>(jf::FuseArgs)",5000,9000,131072\n',
            '"KERNEL_DISPATCH","void jf::(anonymous namespace)::k_fuse_gemm_bf16<256>(jf::FuseArgs)",10000,410000,607744\n']
    (d / "run_kernel_trace.csv").write_text(hdr + "".join(rows))
    per = profsum.read_trace_by_grid(str(d))
    assert per[("k_fuse_gemm_bf16<256>", 131072)] == [2.0, 4.0]
    assert per[("k_fuse_gemm_bf16<256>", 607744)] == [400.0]
    profsum.main(["stats", str(d), "--by-grid"])
    out = capsys.readouterr().out
    assert "607744" in out and "131072" in out


def test_flushed_and_warm_launches_are_told_apart(tmp_path, capsys):
    # fill, A, B, A, fill, A, B, B: A's 1st and 3rd launches and B's 1st and
    # 3rd follow a fill; A's 2nd and B's 2nd do not
    cols = ["Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"]
    a = "void jf::(anonymous namespace)::k_a(int)"
    b = "void jf::(anonymous namespace)::k_b(int)"
    fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float> >(int)"
    seq = [(fill, 1), (a, 10), (b, 20), (a, 30), (fill, 1), (a, 50), (b, 60), (b, 70)]
    with open(tmp_path / "r_kernel_trace.csv", "w") as f:
        f.write(",".join(f'"{c}"' for c in cols) + "\n")
        t = 0
        for name, dur in seq:
            f.write(f'"{name}",64,{t},{t + dur * 1000}\n')
            t += 100000
    per = profsum.read_trace_split(str(tmp_path), "FillFunctor")
    assert per[("k_a", 64)] == ([10.0, 50.0], [30.0])
    assert per[("k_b", 64)] == ([20.0, 60.0], [70.0])
    profsum.main(["stats", str(tmp_path), "--cold-after", "FillFunctor"])
    assert "| `k_a` | 64 | 2 | 30.00 | 1 | 30.00 |" in capsys.readouterr().out
