"""The benchmark's algorithmic work figures and bound choice (CPU only)."""
import numpy as np

import bench


def test_headline_figures():
    # 64 sequences of 4096 rows, 128 heads: 1152 B per cache row and per Q row,
    # 1024 B of out and 4 B of lse per (b, h); 2 * 128 * (576 + 512) flop per row.
    flops, kv, total = bench.workload_figures([4096] * 64, 128)
    assert kv == 64 * 4096 * 1152
    assert total == kv + 64 * 128 * (1152 + 1024 + 4)
    assert flops == 2 * 128 * 1088 * 64 * 4096


def test_several_tokens_visible_rows():
    # Two tokens of 16 heads each over 5 rows: token 0 sees 4 rows, token 1 sees 5.
    flops, kv, total = bench.workload_figures([5], 32, seqlen_q=2)
    assert flops == 2 * 16 * 1088 * (4 + 5)
    assert kv == 5 * 1152
    # Negative lengths count as empty sequences.
    f0, kv0, _ = bench.workload_figures([-3, 0], 8)
    assert f0 == 0 and kv0 == 0


def test_bound_follows_intensity():
    # One token per sequence at H = 128 sits below the ridge (2.5 PF / 8 TB/s = 312.5
    # flop/B): HBM binds.  Two tokens double the flops per row: MFMA binds.
    for s, want in [(1, "hbm"), (2, "mfma")]:
        flops, _, total = bench.workload_figures([4096] * 64, 128 * s, seqlen_q=s)
        first, other = bench.split_bounds(flops, total, 0.1, None)
        assert first["bound"] == want and other["bound"] != want
        hbm = first if want == "hbm" else other
        mfma = other if want == "hbm" else first
        assert np.isclose(hbm["achieved"], total / 1e-4 / 1e9, rtol=1e-4)
        assert np.isclose(mfma["achieved"], flops / 1e-4 / 1e12, rtol=1e-4)
        assert np.isclose(hbm["frac"], hbm["achieved"] / 8000.0, atol=1e-4)
    # No launch time: no figures, but the bound is still named.
    first, _ = bench.split_bounds(1.0, 1.0, 0.0, 123)
    assert first["achieved"] is None and first["frac"] is None and first["traffic"] == 123


def test_code_hash_ignores_comments_only():
    src = "int f(int a) {\n  return a + 1;\n}\n"
    commented = ("// header\n/* block\n   comment */\nint f(int a) {   \n\n"
                 "  return a + 1;  // trailing\n}\n\n")
    assert bench.code_sha256(src) == bench.code_sha256(commented)
    assert bench.code_sha256(src) != bench.code_sha256(src.replace("+ 1", "+ 2"))
    assert bench.code_sha256(src) != bench.code_sha256(src.replace("  return", "  return 0 *"))


def test_measured_counters_follow_the_code_hash(tmp_path):
    """Counter lines are used for their own workload and only while their code
    hash is the one asked for."""
    import json
    rec = {"workload": "w1", "code_sha256": "abc", "fetch_bytes": 100, "write_bytes": 20}
    busy = {"workload": "w1", "code_sha256": "abc", "mfma_busy": 0.5}
    other = {"workload": "w2", "code_sha256": "abc", "fetch_bytes": 7, "write_bytes": 1}
    (tmp_path / "p.md").write_text("# summary\n"
                                   f"traffic-json: {json.dumps(rec)}\n"
                                   f"counters-json: {json.dumps(busy)}\n"
                                   f"traffic-json: {json.dumps(other)}\n")
    t, b, src = bench.measured_counters("w1", str(tmp_path), sha="abc")
    assert t == 120 and b == 0.5 and src.endswith("p.md")
    assert bench.measured_counters("w1", str(tmp_path), sha="def") == (None, None, None)
    assert bench.measured_counters("w3", str(tmp_path), sha="abc") == (None, None, None)
    assert bench.measured_counters("w2", str(tmp_path), sha="abc")[:2] == (8, None)


def test_committed_profiles_parse():
    """Every machine-readable line in profiles/ is JSON with the fields bench.py
    reads; each workload's counter lines name one code hash."""
    import glob
    import json
    import os
    seen = {}
    for f in glob.glob(os.path.join(bench.ROOT, "profiles", "*.md")):
        for line in open(f):
            for tag, keys in (("traffic-json:", ("fetch_bytes", "write_bytes")), ("counters-json:", ("mfma_busy",))):
                if line.startswith(tag):
                    rec = json.loads(line.split(":", 1)[1])
                    assert all(k in rec for k in ("workload", "code_sha256") + keys), (f, line)
                    seen.setdefault(rec["workload"], set()).add(rec["code_sha256"])
    assert seen, "no counter lines under profiles/"
    assert all(len(v) == 1 for v in seen.values()), seen


def test_cpu_baseline_cycles_through_the_workload():
    """The oracle baseline keeps decoding the workload's sequences, from the
    first again, until its budget is spent, and counts the flops of exactly
    the sequences it decoded."""
    import re
    import mla_inputs as mi
    inp = mi.make_config(0)   # B=2, H=16, L=256: a few ms per sequence
    rec = bench.cpu_baseline(inp, 0.3)
    m = re.match(r"(\d+) sequence decodes? \((\d+) passes over all (\d+) sequences \+ (\d+);", rec["sample"])
    assert m, rec["sample"]
    done, passes, batch, rest = map(int, m.groups())
    assert batch == inp.batch and done == passes * batch + rest and passes >= 1
    wall = float(re.search(r"([0-9.]+) s wall", rec["sample"]).group(1))
    full, _, _ = bench.workload_figures(inp.cache_seqlens, inp.heads)
    part, _, _ = bench.workload_figures(inp.cache_seqlens[:rest], inp.heads)
    assert np.isclose(rec["value"] * 1e12 * wall, passes * full + part, rtol=0.2)
    assert rec["kind"] == "oracle" and rec["cores"] >= 1
