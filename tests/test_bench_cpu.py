"""bench.py's contract checks that need no GPU: one GPU only, and the argument defaults."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout.strip() == ""


def test_defaults_time_the_largest_single_gpu_workload():
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'ap.add_argument("--config", type=int, default=2,' in src  # the 32k latent prefill
    assert 'ap.add_argument("--gpus", type=int, default=1)' in src


def test_stage_rooflines_price_each_stage_on_its_own_bound():
    sys.path.insert(0, ROOT)
    import bench

    t = dict(indexer_score=0.088, topk=0.05, select=0.13, sparse_attn=0.066)
    dec = dict(decode=True, idx_scan_bytes=3.7e8, pairs=2.9e6, topk_bytes=1.2e7, gather_bytes=1.69e8,
               attn_flops=3.65e10, idx_flops=4.7e10)
    r = bench.stage_rooflines({}, dec, t)
    # decode: HBM for the scan, the select and the attention, with the attention's matrix-core view beside
    assert r["indexer_score"]["bound"] == "hbm" and r["sparse_attn"]["bound"] == "hbm"
    assert abs(r["sparse_attn"]["achieved"] - 1.69e8 / 0.066e-3 / 1e9) < 0.1
    mv = r["sparse_attn"]["mfma_view"]
    assert mv["unit"] == "TFLOP/s" and abs(mv["achieved"] - 3.65e10 / 0.066e-3 / 1e12) < 0.01
    pre = dict(dec, decode=False)
    r = bench.stage_rooflines({}, pre, t)
    # prefill: the matrix cores for the indexer and the attention, the logical gather rate beside it
    assert r["indexer_score"]["bound"] == "mfma" and r["sparse_attn"]["bound"] == "mfma"
    assert "gather_gbs_logical" in r["sparse_attn"] and "mfma_view" not in r["sparse_attn"]
