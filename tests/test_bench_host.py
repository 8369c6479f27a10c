"""Host logic of bench.py, on the CPU: the algorithmic byte counts behind
every GB/s figure (against the per-workload totals stated with the
workloads: read the BF16 input, write codes, scales and optional dequant),
the comment-blind source digest that guards the HBM traffic figures, and
the one-GPU-only exit."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_workloads():
    # moe_act 8192 x 7168, 4/6 + dequant: 4.5631 B per element
    assert bench.nvfp4_bytes(8192, 7168) == 267_943_936
    # expert weights 65536 x 7168 with dequant
    assert bench.nvfp4_bytes(65536, 7168) == 2_143_551_488
    # ragged routed 65536 x 2048, no dequant, 64 groups (65 int64 offsets)
    assert bench.nvfp4_bytes(65536, 2048, dequant=False, groups=64) == 344_195_592
    # tiny 256 x 2048, per mode
    assert bench.nvfp4_bytes(256, 2048) == 2_393_088
    # MXFP4 Rollout-ResQ 8192 x 7168: codes, E8M0, kept residual codes,
    # 2:4 metadata, residual E8M0
    assert bench.mx_bytes(8192, 7168) == 172_490_752
    # standalone dequant reads codes, scales and token scales, writes BF16
    assert bench.dequant_bytes(8192, 7168) == 8192 * 7168 * (2 + 0.5 + 1 / 16) + 8192 * 4


def test_code_only_drops_comments_keeps_strings():
    src = ('int a = 1;  // trailing\n'
           '/* a block\n   comment */\n'
           'const char* s = "not // a comment /* either */";\n'
           '\n'
           'char c = \'/\'; char q = \'"\';  int b = a / 2;\n')
    got = bench._code_only(src)
    lines = got.split("\n")
    assert lines[0] == "int a = 1;"
    assert "trailing" not in got and "block" not in got
    assert 'const char* s = "not // a comment /* either */";' in lines
    assert "char c = '/'; char q = '\"';  int b = a / 2;" in lines
    # a comment-only edit keeps the text; a code edit changes it
    assert bench._code_only(src.replace("trailing", "other words")) == got
    assert bench._code_only(src.replace("a / 2", "a / 3")) != got


def test_source_digest_is_stable():
    assert bench.source_digest() == bench.source_digest()
    assert len(bench.source_digest()) == 16


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_more_byte_counts():
    n = 8192 * 7168
    # dense residual: primary and residual codes (1/2 B each), two E8M0
    assert bench.mx_dense_bytes(8192, 7168) == n * 2 + n + n // 16
    # S2:4 reconstruction reads 1/2 + 1/32 + 1/4 + 1/8 + 1/32 B, writes 4 B
    assert bench.reconstruct_bytes(8192, 7168) == n * (0.5 + 1 / 32 + 0.25 + 0.125 + 1 / 32 + 4)
    # guided: x, guide codes, scales, token scales in; codes out
    assert bench.guided_bytes(8192, 7168) == n * (2 + 0.5 + 1 / 16 + 0.5) + 8192 * 4
    assert bench.guided_bytes(8192, 7168, guide=False) == n * (2 + 1 / 16 + 0.5) + 8192 * 4


def test_rotating_sets_span_a_gib():
    for per_set in (bench.nvfp4_bytes(8192, 7168), bench.nvfp4_bytes(256, 2048),
                    bench.mx_bytes(8192, 7168), bench.reconstruct_bytes(8192, 7168),
                    bench.nvfp4_bytes(65536, 2048, dequant=False, groups=64)):
        k = bench.n_sets(per_set)
        assert k >= 4 and k * per_set >= 1 << 30, (per_set, k)


def test_dispatch_labels():
    lab = bench._label
    q = "fp4q::(anonymous namespace)::nvfp4_quantize_split<%s>(HIP_vector_type<unsigned int, 4u> const*)"
    assert lab(q % "1, true, 2, false", 8192 * 256) == bench.HEADLINE_KEY
    assert lab(q % "1, true, 2, true", 8192 * 256).startswith("nvfp4_quantize_global")
    assert lab(q.replace("fp4q::", "fp4q_standin::") % "1, true, 2, false",
               8192 * 256).startswith("stand-in")
    assert lab(q % "1, false, 2, false", 65536 * 64).endswith("ragged_routed 65536x2048")
    k0 = "void (anonymous namespace)::k0_read<%s, %s>(x)"
    assert lab(k0 % ("unsigned char", "false"), 1) == "K0 read 1B 256 MiB"
    assert lab(k0 % ("unsigned short", "false"), 1) == "K0 read 2B 256 MiB"
    assert lab(k0 % ("unsigned int", "false"), 1) == "K0 read 4B 256 MiB"
    assert lab(k0 % ("unsigned int __vector(2)", "false"), 1) == "K0 read 8B 256 MiB"
    assert lab(k0 % ("unsigned int __vector(4)", "true"), 1) == "K0 read 16B nt 256 MiB"
    assert lab("(anonymous namespace)::k0_copy<1>(x)", 1) == bench.COPY_CAL_KEY
    assert lab("(anonymous namespace)::k0_copy<0>(x)", 1) == "K0 copy 256 MiB"
    assert lab("(anonymous namespace)::k0_copy<2>(x)", 1) == "K0 copy nt sc1 256 MiB"
    assert lab("(anonymous namespace)::k0_write<2>(x)", 1) == "K0 write nt sc1 256 MiB"
    assert lab("(anonymous namespace)::k0_copy_stream<1>(x)", 1) is None
    assert lab("void (anonymous namespace)::k0_mix<4, 1>(x)", 1) == \
        "K0 mix read 4 KiB, write 4/4 KiB nt 256 MiB"
    # the exact-decision build, the FP16 decision on routed tokens, and the
    # guided kernels (two template arguments: nearest or guided, dequant)
    ex = q.replace("fp4q::", "fp4q_exactdecision::")
    assert lab(ex % "1, true, 2, false", 8192 * 256).startswith("exact-error decision")
    assert lab(ex % "1, false, 2, false", 65536 * 64).startswith("exact-error decision")
    assert lab(q % "2, false, 2, false", 65536 * 64) == \
        "nvfp4_quantize_split<fp16-decision> ragged_routed 65536x2048"
    g = "fp4q::(anonymous namespace)::nvfp4_guided_units<%s>(HIP_vector_type<unsigned int, 4u> const*)"
    assert lab(g % "false, false", 1) == "nvfp4_quantize_guided moe_act 8192x7168"
    assert lab(g % "true, false", 1) == "nvfp4_quantize_guided (no guide: nearest) moe_act 8192x7168"
    # every labelled kernel has algorithmic bytes
    algo = bench.algorithmic_rw()
    assert bench.HEADLINE_KEY in algo and bench.COPY_CAL_KEY in algo
    for name in (ex % "1, true, 2, false", q % "2, false, 2, false", g % "false, false",
                 g % "true, false"):
        key = lab(name, 8192 * 256 if "true, 2" in name else 65536 * 64)
        assert key in algo, key


def test_host_cpu_description():
    d = bench.host_cpu()
    assert d["cpus_usable_by_this_process"] >= 1 and d["host_logical_cpus"] >= 1
    assert isinstance(d["cpu_model"], str)
    assert d["cpuid"] is None or d["cpuid"].startswith("family ")
    assert isinstance(d["vector_extensions"], list)


def test_profile_summary_splits_the_dequant_layouts(tmp_path):
    # a synthetic rocprofv3 output: the copy that calibrates the counters,
    # then two bursts of dequant dispatches a pause apart (the bench's two
    # layouts of the same sets); the summary keeps them as two rows
    import csv

    def write_csv(path, header, rows):
        path.parent.mkdir(parents=True, exist_ok=True)
        with open(path, "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(header)
            w.writerows(rows)

    dq = "fp4q::(anonymous namespace)::nvfp4_dequantize_rows(unsigned int const*)"
    copy = "void (anonymous namespace)::k0_copy<1>(x)"
    disp = [(copy, 1, 0, 80_000)]
    t = 1_000_000
    for i in range(5):                      # separate allocations: 25 us each
        disp.append((dq, 1, t, t + 25_000)); t += 30_000
    t += 5_000_000                          # the second layout's set-up
    for i in range(5):                      # one allocation per kind: 22 us
        disp.append((dq, 1, t, t + 22_000)); t += 30_000
    trace = [(k, g, d, a, b) for d, (k, g, a, b) in enumerate(disp)]
    write_csv(tmp_path / "tr" / "run_kernel_trace.csv",
              ["Kernel_Name", "Grid_Size", "Dispatch_Id", "Start_Timestamp", "End_Timestamp"], trace)
    write_csv(tmp_path / "tr" / "run_kernel_stats.csv",
              ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"], [(dq, 10, 1, 1, 1)])
    for cname, val in (("FETCH_SIZE", 131072.0), ("WRITE_SIZE", 262144.0)):
        rows = [(k, g, d, cname, val) for d, (k, g, a, b) in enumerate(disp)]
        write_csv(tmp_path / cname / "run_counter_collection.csv",
                  ["Kernel_Name", "Grid_Size", "Dispatch_Id", "Counter_Name", "Counter_Value"], rows)
    out = tmp_path / "out"
    bench.summarize_profiles(str(tmp_path / "tr"), str(tmp_path / "FETCH_SIZE"),
                             str(tmp_path / "WRITE_SIZE"), str(out))
    text = (out / "kernel_trace_bench_default.md").read_text()
    row = {ln.split("|")[1].strip(): ln.split("|")[2:4] for ln in text.splitlines()
           if ln.startswith("| nvfp4_dequantize")}
    assert row[bench.DQ_KEY][0].strip() == "5" and row[bench.DQ_KEY][1].strip() == "25.00"
    assert row[bench.DQ_PACKED_KEY][0].strip() == "5" and row[bench.DQ_PACKED_KEY][1].strip() == "22.00"
