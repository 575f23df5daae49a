"""Host-side logic of bench.py (CPU only): the kernel code digest that ties
the committed counter figures to the code they were taken on, the statistics
of the measurement build's per-workgroup records (store spans, shader clock),
the +-2% DVFS flag on a timing, and the refusal of more than one GPU."""
import bench


def test_code_text_drops_comments_and_keeps_literals():
    src = ('// header\n'
           'int a = 1; /* block\n comment */ int b = 2;\n'
           '\n'
           'asm volatile("s_waitcnt vmcnt(0)\\n\\ts_barrier" ::: "memory");  // trailing\n'
           'const char *u = "a // not a comment";\n'
           "char q = '\"';\n")
    code = bench.code_text(src)
    assert "header" not in code and "block" not in code and "trailing" not in code
    assert 'asm volatile("s_waitcnt vmcnt(0)\\n\\ts_barrier" ::: "memory");' in code
    assert '"a // not a comment"' in code
    assert "char q = '\"';" in code
    assert "\n\n" not in code


def test_digest_ignores_comment_edits_but_not_code_edits(tmp_path, monkeypatch):
    k = tmp_path / "k.hip"
    k.write_text("// v1\nint f() { return 2; }\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(k))
    d0 = bench.source_digest()
    k.write_text("// v2, reworded\n\nint f() { return 2; }   \n/* note */\n")
    assert bench.source_digest() == d0
    k.write_text("// v1\nint f() { return 3; }\n")
    assert bench.source_digest() != d0



def test_traffic_figures_apply_only_to_their_workload():
    # the committed counter summary covers one workload; any other reports null
    assert bench.measured_traffic("tiny") is None
    assert bench.measured_traffic("no_such_workload") is None


def test_trace_stats_on_a_hand_made_trace():
    # four workgroups on the 100 MHz clock: start, rows ready, stores done,
    # shader cycles.  Three store 1 MB each in 2 us after 10 us of work, at
    # 2000 MHz; the fourth is a split part merged elsewhere ([1] == [2]),
    # at 1000 MHz.
    rec = [[0, 1000, 1200, 24000],
           [100, 1100, 1300, 24000],
           [50, 1050, 1250, 24000],
           [0, 600, 600, 6000]]
    st = bench.trace_stats(rec, 3_000_000)
    assert st["trace_work_units"] == 4
    assert st["epilogue_span_us_mean"] == 2.0 and st["epilogue_span_us_p90"] == 2.0
    assert st["epilogue_unit_GBs_mean"] == 500.0            # 1 MB in 2 us
    # clock: all cycles over all lifetimes, 78000 cycles in 42 us
    assert st["sclk_mhz_trace"] == round(78000 / 42.0, 1)
    assert st["epilogue_share_of_unit_time"] == round(6.0 / 42.0, 4)
    lo, hi = st["sclk_mhz_trace_p10_p90"]
    assert 1000.0 < lo < 2000.0 and hi == 2000.0


def test_clock_flags_mark_drift_and_spread_beyond_two_percent():
    steady = [1.0] * 20
    f = bench.clock_flags(2000.0, 1980.0, steady)
    assert f["sclk_drift_pct"] == -1.01 and f["launch_spread_pct"] == 0.0 and not f["outside_dvfs_band"]
    f = bench.clock_flags(2000.0, 1950.0, steady)               # -2.53%
    assert f["outside_dvfs_band"]
    f = bench.clock_flags(1950.0, 2000.0, steady)               # +2.53%
    assert f["outside_dvfs_band"]
    # half the launches 10% slower: spread (p90 - p10) / 2 / median = 4.8%
    f = bench.clock_flags(2000.0, 2000.0, [1.0] * 10 + [1.1] * 10)
    assert f["launch_spread_pct"] == 4.76 and f["outside_dvfs_band"]
    # a clock that could not be read counts as outside
    assert bench.clock_flags(0.0, 0.0, steady)["outside_dvfs_band"]


def test_more_than_one_gpu_is_refused_with_a_message():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
