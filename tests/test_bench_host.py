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


def test_fold_step_takes_arenas_and_outputs_in_turn():
    seen = []

    class Lib:
        def fold_ranks(self, o, s):
            seen.append(("plain", o, s))

        def fold_ranks_scaled(self, o, s, inv_w):
            seen.append((inv_w, o, s))

    step = bench.fold_step(Lib(), ["o0", "o1", "o2"], ["a0", "a1"], None)
    for _ in range(6):
        step()
    assert seen == [("plain", "o0", "a0"), ("plain", "o1", "a1"), ("plain", "o2", "a0"),
                    ("plain", "o0", "a1"), ("plain", "o1", "a0"), ("plain", "o2", "a1")]
    seen.clear()
    step = bench.fold_step(Lib(), ["o0"], ["a0"], 0.25)
    step()
    assert seen == [(0.25, "o0", "a0")]


def test_arena_set_copies_keep_the_phase_and_the_contents(monkeypatch):
    import torch
    monkeypatch.setattr(bench, "MEMORY_SIDE_CACHE_BYTES", 1024)
    W, n, offset = 8, 100, 1
    alloc = torch.empty(W * n + offset, dtype=torch.float32)
    stacked = alloc[offset:].view(W, n)
    stacked.copy_(torch.arange(W * n, dtype=torch.float32).view(W, n))
    copies = bench.arena_set(torch, stacked, offset)
    # 1 + ceil(4 * 1024 / 3200) copies: at least 4x the cache of other copies between reuses
    assert len(copies) == 3 and copies[0] is stacked
    for c in copies[1:]:
        assert c.shape == (W, n) and c.data_ptr() != stacked.data_ptr()
        assert c.data_ptr() % 16 == stacked.data_ptr() % 16
        assert torch.equal(c, stacked)
    monkeypatch.setattr(bench, "MEMORY_SIDE_CACHE_BYTES", 256 << 20)
    meta = torch.empty((8, 1 << 24), dtype=torch.float32, device="meta")
    assert len(bench.arena_set(torch, meta, 0)) == 3      # W=8 x 2^24: 512 MiB per copy
    meta = torch.empty((4, 100_000_000), dtype=torch.float32, device="meta")
    assert len(bench.arena_set(torch, meta, 0)) == 2      # W=4 x 1e8: 1.6 GB per copy


def test_fill_outputs_takes_every_arena_copy(monkeypatch):
    seen = []

    class Lib:
        def fold_ranks(self, o, s):
            seen.append((o, s))

    class Torch:
        class cuda:
            @staticmethod
            def synchronize():
                seen.append("sync")

    bench.fill_outputs(Torch, Lib(), ["o0", "o1", "o2", "o3", "o4"], ["a0", "a1", "a2"], None)
    assert seen == [("o0", "a0"), ("o1", "a1"), ("o2", "a2"), ("o3", "a0"), ("o4", "a1"), "sync"]
