"""Host-side logic of bench.py (CPU only): the kernel code digest that ties
the committed counter figures to the code they were taken on."""
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
