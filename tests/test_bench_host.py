"""Host-side logic of bench.py (no GPU): the algorithmic byte counts it reports against,
the gating of counter-measured traffic by the kernel sources' digest, and the refusal of
more than one GPU.

The byte counts are pinned to figures worked out independently of bench.py from the
per-call formulas (x read once, every placed row written or read once, 4 bytes of slot
map per route, 8 with the route weight): the dispatch + combine bytes and bytes per token
of the three dropless workloads, and the backward bytes of the Zipf workload.
"""
import subprocess
import sys

import pytest

import bench
import workloads as W


@pytest.mark.parametrize("name,total,per_token", [
    ("dropless_top8_h2816", 415_629_312, 101_472),
    ("zipf_skew_h4096", 1_208_745_984, 147_552),
    ("checkpoint_replay_h2816", 3_325_034_496, 101_472),
])
def test_dispatch_combine_bytes_of_the_dropless_workloads(name, total, per_token):
    w = W.WORKLOADS[name]
    ab = bench.algorithmic_bytes(w, kept_routes=w.s * w.k)  # dropless: every route placed
    assert ab["dispatch"] + ab["combine"] == total
    assert total // w.s == per_token


def test_backward_bytes_of_the_zipf_workload():
    w = W.WORKLOADS["zipf_skew_h4096"]
    ab = bench.algorithmic_bytes(w, kept_routes=w.s * w.k)
    # combine backward: grad_y once, every expert row read, every buffer row written, and
    # per route its slot, weight and weight gradient
    assert ab["combine_bwd"] == 1_141_637_120
    assert ab["dispatch_bwd"] == 604_241_920


def test_dropped_routes_are_not_counted_as_read():
    w = W.WORKLOADS["gshard_capacity_drop"]
    full = bench.algorithmic_bytes(w, kept_routes=w.s * w.k)
    part = bench.algorithmic_bytes(w, kept_routes=w.s * w.k - 100)
    row = w.m * W.ELEM_BYTES[w.dtype]
    assert full["combine"] - part["combine"] == 100 * row
    assert full["dispatch"] == part["dispatch"]  # the [e, c, m] buffer is written whole


def _write_traffic(root, digest):
    prof = root / "profiles"
    prof.mkdir()
    (prof / "traffic_zipf_skew_h4096.txt").write_text(
        "# summary\n\ntraffic dispatch 606666937\ntraffic combine 606132834\n"
        f"source_digest {digest}\n")


def test_traffic_is_reported_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _write_traffic(tmp_path, bench.kernel_source_digest())
    assert bench.measured_traffic("zipf_skew_h4096") == {"dispatch": 606666937, "combine": 606132834}
    assert bench.measured_traffic("zipf_skew_h4096", "expert_gemm") == {}  # no such summary


def test_gemm_sources_only_change_the_gemm_variant_digest(monkeypatch):
    from combine_moe_gate_amd import _build
    real_open = open

    def edited_gemm(path, mode="r", *a, **k):
        f = real_open(path, mode, *a, **k)
        if path.endswith("gemm.hip") and "b" in mode:
            data = f.read() + b"\nstatic int digest_probe;\n"
            f.close()
            import io
            return io.BytesIO(data)
        return f

    before = (bench.kernel_source_digest(), bench.kernel_source_digest("expert_gemm"))
    monkeypatch.setattr("builtins.open", edited_gemm)
    after = (bench.kernel_source_digest(), bench.kernel_source_digest("expert_gemm"))
    assert before[0] == after[0] and before[1] != after[1]
    assert any(p.endswith("gemm.hip") for p in _build.SOURCES)


def test_traffic_of_other_sources_is_dropped(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _write_traffic(tmp_path, "0123456789abcdef")
    assert bench.measured_traffic("zipf_skew_h4096") == {}


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_cold_pair_summary_quotes_the_median_pair():
    # three pairs of 100 + 110, 120 + 130 and 200 + 200 microseconds over 1.2e9 bytes:
    # pairs of 210, 250 and 400 us, median 250 us (the mean, 286.7, is not quoted), so
    # 4800 GB/s and 0.6 of 8 TB/s; p10 = 210 + 0.2 * 40, p90 = 250 + 0.8 * 150
    s = bench.cold_pair_summary(8192, [100.0, 120.0, 200.0], [110.0, 130.0, 200.0], 1_200_000_000)
    assert s["pairs"] == 3
    assert s["us_median"] == 250.0 and s["us_min"] == 210.0 and s["us_mean"] == 286.67
    assert s["us_p10"] == 218.0 and s["us_p90"] == 370.0
    assert s["dispatch_us_median"] == 120.0 and s["combine_us_median"] == 130.0
    assert s["GBps"] == 4800.0 and s["frac_of_hbm_peak"] == 0.6
    assert s["tokens_per_s"] == round(8192 / 250e-6, 1)


def test_expert_gemm_bytes_count_only_the_experts_that_receive_rows():
    w = W.WORKLOADS["zipf_skew_h4096"]
    K = w.s * w.k
    row, wrow = w.m * 2, W.EXPERT_WIDTH * w.m * 2  # bf16: one token row, one expert's weights
    all_e = bench.algorithmic_bytes(w, K, variant="expert_gemm")
    some = bench.algorithmic_bytes(w, K, variant="expert_gemm", active_experts=43)
    assert all_e["expert_gemm"] - some["expert_gemm"] == (w.e - 43) * wrow
    assert all_e["expert_gemm_dgrad"] - some["expert_gemm_dgrad"] == (w.e - 43) * wrow
    # x once, 43 experts' weights once, [rows, n] output and its row map
    assert some["expert_gemm"] == w.s * row + 43 * wrow + K * W.EXPERT_WIDTH * 2 + K * 4
    # the weight gradient writes every expert's (zeros for the idle ones)
    assert all_e["expert_gemm_wgrad"] == some["expert_gemm_wgrad"]


def test_loop_oracle_sample_times_the_first_tokens_with_the_capacity_scaled():
    w = W.WORKLOADS["tiny_capacity_top2"]
    r = bench._loop_oracle_sample(w, 4)
    assert r["tokens_per_s"] > 0 and r["seconds"] > 0
    # capacity 80 of 256 tokens, scaled to 4 tokens: ceil(80 * 4 / 256) = 2
    assert r["sample"] == "first 4 of 256 tokens (m=64, e=8, k=2, f32, capacity scaled to 2)"


def test_host_only_sources_do_not_change_the_digest(monkeypatch):
    real_open = open

    def edited_host(path, mode="r", *a, **k):
        f = real_open(path, mode, *a, **k)
        if (path.endswith("api.hip") or path.endswith("moe_gate.h")) and "b" in mode:
            data = f.read() + b"\nstatic int digest_probe;\n"
            f.close()
            import io
            return io.BytesIO(data)
        return f

    before = (bench.kernel_source_digest(), bench.kernel_source_digest("expert_gemm"))
    monkeypatch.setattr("builtins.open", edited_host)
    assert (bench.kernel_source_digest(), bench.kernel_source_digest("expert_gemm")) == before


def _digests_with_gate_edit(monkeypatch, tail: bytes):
    real_open = open

    def edited(path, mode="r", *a, **k):
        f = real_open(path, mode, *a, **k)
        if path.endswith("gate.hip") and "b" in mode:
            data = f.read() + tail
            f.close()
            import io
            return io.BytesIO(data)
        return f

    monkeypatch.setattr("builtins.open", edited)
    out = (bench.kernel_source_digest(), bench.kernel_source_digest("expert_gemm"))
    monkeypatch.undo()
    return out


def test_comments_and_layout_do_not_change_the_digest_but_code_does(monkeypatch):
    before = (bench.kernel_source_digest(), bench.kernel_source_digest("expert_gemm"))
    assert _digests_with_gate_edit(monkeypatch, b"\n// a note\n/* and a\n block */\n\n") == before
    code = _digests_with_gate_edit(monkeypatch, b"\nstatic int digest_probe;\n")
    assert code[0] != before[0] and code[1] != before[1]


def test_source_code_bytes_drops_comments_and_folds_whitespace():
    src = b"int a; // one\n/* two\n three */  int\tb;\n"
    assert bench.source_code_bytes(src) == b"int a; int b;"
