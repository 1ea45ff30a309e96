"""Host-side checks of bench.py's bookkeeping (no GPU): its work accounting against the
oracle's pair counts, and the counter summary it derives HBM traffic from."""
import random

import bench
from oracle import accounting


def test_bench_work_accounting_matches_oracle_counts():
    rng = random.Random(0)
    cases = [(131072, 2048, 131072), (200001, 2048, 1), (1048576, 2048, 4096), (1024, 64, 1024),
             (10, 2048, 10), (3000, 2048, 5)]
    cases += [(L, rng.randint(1, 3000), rng.randint(1, L)) for L in (rng.randint(1, 9000) for _ in range(500))]
    for L, k, Lq in cases:
        assert bench.Work.causal_pairs(L, Lq) == accounting.causal_pairs(L, Lq)
        assert bench.Work.selected_pairs(L, k, Lq) == accounting.selected_pairs(L, k, Lq)
    assert bench.Work.indexer_flops(10, 64, 128) == accounting.indexer_flops(10, 64, 128)
    assert bench.Work.attention_flops(10, 32, 576, 512) == accounting.attention_flops(10, 32, 576, 512)


def _csv(path, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for d, name, cn, v in rows:
            f.write(f'{d},"{name}",{cn},{v}\n')


def test_counter_summary_scales_by_the_calibration_copy(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    k = "void dsa::mla_attn32_kernel<false>(dsa::MlaParams)"
    _csv(fetch, [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 99.0),
                 (5, k, "FETCH_SIZE", 1000.0), (6, k, "FETCH_SIZE", 3000.0),
                 (9, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0)])
    _csv(write, [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 50.0),
                 (5, k, "WRITE_SIZE", 10.0), (6, k, "WRITE_SIZE", 30.0),
                 (9, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)])
    text = bench.summarize_counters(str(fetch), str(write), "mla_attn32_kernel", "<false>", "w")
    fields = dict(l.split(":", 1) for l in text.splitlines() if ":" in l and not l.startswith("#"))
    assert float(fields["read_scale"]) == 2.0 and float(fields["write_scale"]) == 1.0
    assert int(fields["launches"]) == 2
    # mean fetch 2000 KiB read twice over, mean write 20 KiB
    assert int(fields["traffic_bytes_per_launch"]) == 2000 * 1024 * 2 + 20 * 1024


def test_counter_summary_leaves_out_dispatches_that_do_no_work(tmp_path):
    """A dispatch reading under 1% of the largest (the fused indexer's recompute pass when
    no item failed) does not dilute the per-launch figures."""
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    k = "void dsa::indexer_topk_kernel<2, 4>(dsa::FusedParams)"
    _csv(fetch, [(3, k, "FETCH_SIZE", 4000.0), (4, k, "FETCH_SIZE", 2.0),
                 (9, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0)])
    _csv(write, [(3, k, "WRITE_SIZE", 100.0), (4, k, "WRITE_SIZE", 1.0),
                 (9, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)])
    text = bench.summarize_counters(str(fetch), str(write), "indexer_topk_kernel", "<2, 4>", "w")
    fields = dict(l.split(":", 1) for l in text.splitlines() if ":" in l and not l.startswith("#"))
    assert int(fields["dispatches"]) == 2 and int(fields["launches"]) == 1
    assert int(fields["traffic_bytes_per_launch"]) == 4000 * 1024 * 2 + 100 * 1024


def test_main_roofline_follows_the_workload():
    import synth
    # prefill128k: the attention of four layers outweighs the indexer; bf16 MFMA peak
    cfg = synth.get_config("prefill128k")
    roof, extra = bench.main_roofline(cfg, cfg.L, 55.0, 28.0, 140.7e12, 18.5e12, 306.8)
    assert (roof["kernel"], roof["bound"], roof["unit"], roof["peak"]) == ("sparse_attn", "mfma", "TFLOP/s", 2500.0)
    assert abs(roof["achieved"] - 18.5e12 / 28e-3 / 1e12) < 0.01 and extra is None
    # an indexer that outweighs the layers is priced on its own type's peak (fp8)
    roof, _ = bench.main_roofline(cfg, cfg.L, 200.0, 28.0, 140.7e12, 18.5e12, 306.8)
    assert (roof["kernel"], roof["bound"], roof["peak"]) == ("indexer_topk", "mfma", 5000.0)
    # decode: HBM bytes, the k^I codes plus one fp32 scale per key
    cfg = synth.get_config("decode200k")
    roof, extra = bench.main_roofline(cfg, cfg.L, 0.35, 0.046, 2.1e11, 9e9, 0.151)
    kI = 64 * 200001 * (128 + 4) / 1e9
    assert (roof["kernel"], roof["bound"], roof["unit"], roof["peak"]) == ("indexer_topk", "hbm", "GB/s", 8000.0)
    assert abs(roof["achieved"] - kI / 0.35e-3) < 0.1 and extra["hbm_gb"] == round(kI, 3)
    roof, _ = bench.main_roofline(cfg, cfg.L, 0.10, 0.046, 2.1e11, 9e9, 0.151)
    assert (roof["kernel"], roof["bound"]) == ("sparse_attn", "hbm")
    assert abs(roof["achieved"] - 0.151 / 0.046e-3) < 0.1
    # fp32 MHA: the vector ALU peak
    cfg = synth.get_config("tiny")
    roof, _ = bench.main_roofline(cfg, cfg.L, 0.01, 0.06, 1e9, 2e9, 0.01)
    assert (roof["kernel"], roof["bound"], roof["peak"]) == ("sparse_attn", "alu", 157.3)


def test_more_than_one_gpu_is_refused_with_a_message():
    import json, os, subprocess, sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for argv, env in ((["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *argv], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2
        msg = json.loads(r.stdout.strip().splitlines()[-1])
        assert "one GPU" in msg["error"]
