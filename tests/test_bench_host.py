"""Host logic of bench.py (no GPU): the algorithmic work the roofline divides
by, the kernel-trace table, the counter summaries and their calibration, and
the gate that drops HBM traffic taken on other kernel sources.

The attention work is pinned by counting, per query row, the keys it may see
(the prefix plus its own root path, walked through the parents here), not by
re-running bench.py's formula; the logit bytes by the array's own size."""
import importlib.util
import json
import os
import sqlite3

import pytest

from tests import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _visible_keys(parents, P):
    """Keys query row i sees: the P prefix rows and every node on its root path."""
    out = []
    for i in range(len(parents)):
        n, j = 0, i
        while j >= 0:
            n += 1
            j = int(parents[j])
        out.append(P + n)
    return out


@pytest.mark.parametrize("tree,dtype", [("random", "f32"), ("chain", "bf16"), ("star", "bf16")])
def test_attention_work_counts_visible_keys(tree, dtype):
    b = _bench()
    wl = W.make_custom("w", R=2, B=23, V=300, Hq=6, Hkv=2, D=64, P=37, dtype=dtype, tree=tree, n_uniform=1)
    e = 2 if dtype == "bf16" else 4
    work = b.algorithmic_work(wl)
    # each visible (query row, key) pair: a D-long dot product and a D-long
    # weighted sum, 2 FLOP per multiply-add, for every q head
    pairs = sum(sum(_visible_keys(wl.parents[r], wl.P)) for r in range(wl.R))
    assert work["attn_flops"] == 4 * wl.D * wl.Hq * pairs
    # K and V of every kv head once, Q once, the f32 output once
    kv_rows = wl.R * wl.Hkv * (wl.P + wl.B)
    assert work["attn_bytes"] == 2 * kv_rows * wl.D * e + wl.R * wl.B * wl.Hq * wl.D * (e + 4)
    assert work["exit_law_bytes"] == wl.logits.nbytes == wl.R * wl.B * wl.V * e


def test_qwen3_4b_work_matches_the_stated_figures():
    """The Qwen3-4B-shaped round: 18,612,224 attention bytes, 19.45 MB of logits."""
    b = _bench()
    wl = W.make_config("qwen3_4b", n_uniform=1)
    work = b.algorithmic_work(wl)
    assert work["attn_bytes"] == 2 * 8 * (4096 + 64) * 128 * 2 + 64 * 32 * 128 * (2 + 4) == 18_612_224
    assert work["exit_law_bytes"] == 64 * 151936 * 2
    pairs = sum(_visible_keys(wl.parents[0], 4096))
    assert work["attn_flops"] == 4 * 128 * 32 * pairs


def _trace_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table kernels (id integer, kernel_name text, start integer, end integer)")
    con.executemany("insert into kernels values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_summarize_trace_table(tmp_path, capsys):
    b = _bench()
    db = str(tmp_path / "t.db")
    # durations in ns: kernel a 1000, 3000, 2000 (three calls), kernel b 9000
    _trace_db(db, [(1, "a", 0, 1000), (2, "a", 5000, 8000), (3, "a", 9000, 11000), (4, "b", 0, 9000)])
    b.summarize_trace(db)
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("| `")]
    assert lines[0] == "| `b` | 1 | 9.0 | 9.000 | 9.000 | 9.000 | 60.0% |"
    assert lines[1] == "| `a` | 3 | 6.0 | 2.000 | 2.000 | 1.000 | 40.0% |"


def _pmc_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, dispatch_id integer, "
                "counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_summarize_pmc_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    copy = "__amd_rocclr_copyBuffer"
    kern = "void tev::(anonymous namespace)::k_demo<1>(int)"
    # the calibration copy reads FETCH_SIZE = half its bytes in KiB and writes
    # them all; a small copy dispatch of the same kernel must not be taken as
    # the calibration; the kernel's counters are averaged over its dispatches
    half_kib = (b.COPY_BYTES // 2) / 1024
    rows = [(copy, 1, "FETCH_SIZE", 4.0), (copy, 1, "WRITE_SIZE", 8.0),
            (copy, 2, "FETCH_SIZE", half_kib), (copy, 2, "WRITE_SIZE", 2 * half_kib),
            (kern, 3, "FETCH_SIZE", 1000.0), (kern, 4, "FETCH_SIZE", 3000.0),
            (kern, 3, "GRBM_GUI_ACTIVE", 8 * 1000.0), (kern, 4, "GRBM_GUI_ACTIVE", 8 * 1000.0),
            (kern, 3, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 500.0), (kern, 4, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 500.0),
            (kern, 3, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 10.0), (kern, 4, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 10.0)]
    db = str(tmp_path / "p.db")
    _pmc_db(db, rows)
    b.summarize_pmc("demo", [db])
    out = json.load(open(tmp_path / "profiles" / "pmc_demo.json"))
    k = out["kernels"]["k_demo<1>"]
    assert k["cycles"] == 1000.0                       # GRBM_GUI_ACTIVE summed over 8 XCDs
    assert k["mfma_busy_frac"] == pytest.approx(0.5)   # over 1024 SIMDs
    assert k["mfma_flop"] == 10 * 512
    # mean FETCH_SIZE 2000 KiB, scaled so that the copy's reading is its byte count
    assert k["fetch_bytes"] == pytest.approx(2000.0 * b.COPY_BYTES / half_kib)


def test_summarize_pmc_averages_a_counter_over_the_passes(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    kern = "void tev::(anonymous namespace)::k_demo<1>(int)"
    # two passes of the same run, dispatch ids restarting at 1 in each; each
    # collects GRBM_GUI_ACTIVE (two rows per dispatch, one per XCD group),
    # which must be summed within a pass and averaged over the passes
    sq = [(kern, 1, "GRBM_GUI_ACTIVE", 4 * 900.0), (kern, 1, "GRBM_GUI_ACTIVE", 4 * 900.0),
          (kern, 1, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 450.0)]
    wave = [(kern, 1, "GRBM_GUI_ACTIVE", 4 * 1100.0), (kern, 1, "GRBM_GUI_ACTIVE", 4 * 1100.0),
            (kern, 1, "SQ_WAVE_CYCLES", 200.0), (kern, 1, "SQ_WAIT_ANY", 50.0),
            (kern, 1, "SQ_WAIT_INST_ANY", 30.0), (kern, 1, "SQ_ACTIVE_INST_ANY", 120.0)]
    dbs = [str(tmp_path / "sq.db"), str(tmp_path / "wave.db")]
    _pmc_db(dbs[0], sq)
    _pmc_db(dbs[1], wave)
    b.summarize_pmc("demo", dbs)
    k = json.load(open(tmp_path / "profiles" / "pmc_demo.json"))["kernels"]["k_demo<1>"]
    assert k["cycles"] == pytest.approx(1000.0)        # (900 + 1100) / 2, not their sum
    assert k["mfma_busy_frac"] == pytest.approx(0.45)
    ws = k["wave_state"]
    assert ws["wait_any"] == pytest.approx(0.25)
    assert ws["wait_inst_any"] == pytest.approx(0.15)
    assert ws["active_inst_any"] == pytest.approx(0.6)
    assert "active_inst_lds" not in ws                # not collected


def test_traffic_is_dropped_when_the_sources_changed(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    with open(tmp_path / "profiles" / "traffic_demo.json", "w") as f:
        json.dump({"kernel_source_hash": "abc", "k_round_attn": {"bytes": 1}}, f)
    assert b.load_traffic("demo", "abc")["k_round_attn"]["bytes"] == 1
    assert b.load_traffic("demo", "other") is None
    assert b.load_traffic("missing", "abc") is None


def test_committed_counters_match_the_current_sources():
    """The committed counter summaries carry the hash of the round kernels'
    sources they were taken on; they must be the current ones."""
    b = _bench()
    h = b.kernel_source_hash()
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        if name.endswith(".json"):
            with open(os.path.join(ROOT, "profiles", name)) as f:
                assert json.load(f).get("kernel_source_hash") == h, name


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
