"""Host-side pieces of bench.py: the code hash that ties the committed HBM
counter record to the kernel source it was measured on, and the kernel names
it reports from a host plan."""
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


def test_plan_kernel_names(detfold_lib):
    df = detfold_lib
    base, cu = 0x7F0000000000, 256
    name = lambda out, st, W, n, scaled=False: bench.plan_kernel_name(
        df, df.plan_fold_ranks(out, st, W, n, cu), W, scaled)
    assert name(base, base + (1 << 34), 8, 1 << 24) == \
        "k_fold_rows<8,1,false> grid=32768 block=512 tile=128 xcd_group=1"
    assert name(base, base + (1 << 34), 8, 1 << 23).startswith("k_fold_rows<8,2,false>")
    assert name(base, base + (1 << 34), 8, 10_000_000).endswith("block=512 tile=128 xcd_group=32")
    assert name(base, base + (1 << 34), 7, 1 << 22).startswith("k_fold_rows<7,2,false> grid=16384 block=256")
    assert name(base, base + (1 << 34) + 4, 7, 1 << 20).startswith("k_fold_rows<7,2,false> grid=4096 block=256")
    assert name(base, base + (1 << 34), 14, 1 << 20).startswith("k_fold_rows<14,2,false> grid=4096 block=512")
    assert name(base, base + (1 << 34), 4, 100_000_000, True) == \
        "k_fold_rows<4,1,true> grid=390625 block=256 tile=64 xcd_group=8"
    assert name(base, base + (1 << 34) + 4, 16, 10_000_019).startswith("k_fold_rows<16,2,false> grid=39063 block=512")
    assert name(base, base + (1 << 34), 32, 1 << 20).startswith("k_fold_rows_wide<8,2,1,false>")
    assert name(base, base + (1 << 34) + 4, 32, 1 << 20).startswith("k_fold_rows_wide<16,1,4,false>")


def test_output_set_spans_twice_the_memory_side_cache():
    import torch
    for n, count in ((1 << 24, 8), (100_000_000, 2), (10_000_019, 14), (8_000_001, 17), (4096, 32768)):
        out = torch.empty(0).new_empty((n,), device="meta")
        outs = bench.output_set(torch, out)
        assert len(outs) == count and outs[0] is out
        assert len(outs) * n * 4 >= 2 * bench.MEMORY_SIDE_CACHE_BYTES
        assert (len(outs) - 1) * n * 4 < 2 * bench.MEMORY_SIDE_CACHE_BYTES or len(outs) == 2
        assert all(o.shape == out.shape and o.dtype == out.dtype for o in outs)


def test_rotating_step_takes_the_buffers_in_turn():
    seen = []
    step = bench.rotating(["a", "b", "c"], seen.append)
    for _ in range(7):
        step()
    assert seen == ["a", "b", "c", "a", "b", "c", "a"]
