"""Host-side pieces of bench.py: the code hash that ties the committed HBM
counter record to the kernel source it was measured on."""
import bench


def test_code_text_drops_comments_and_layout_but_keeps_literals():
    src = 'int a = 1; // note\n/* block\n comment */ int   b =\n 2; const char *s = "// not /* a comment";\n'
    assert bench.code_text(src) == 'int a = 1; int b = 2; const char *s = "// not /* a comment";'
    assert bench.code_text("x = '\\'' ; // q") == "x = '\\'' ;"


def test_code_hash_ignores_comments_but_not_code():
    a = "int f() { return 1; } // one\n"
    b = "/* the same code */\nint   f() {\n  return 1;\n}\n"
    c = "int f() { return 2; }\n"
    h = lambda t: bench.hashlib.sha256(bench.code_text(t).encode()).hexdigest()
    assert h(a) == h(b) != h(c)


def test_counter_record_parses():
    rec = bench.read_counters()
    # None only when the kernel code changed since the counters were taken
    if rec is not None:
        assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
        assert rec["hbm_bytes_per_launch"] == int((rec["fetch_kib_per_launch"] * 2.0 +
                                                   rec["write_kib_per_launch"]) * 1024)
