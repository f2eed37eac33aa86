"""bench.py checks that need no GPU: the one-GPU guard, and the algorithmic byte counts behind its
roofline objects, recomputed here from the sizes of the 1M-context decode configurations (1M
tokens, CSA every 4 and HCA every 128 tokens, 4 indexer heads x 128 FP4 values + one E8M0 scale
per 32, 576-byte rows, 64 heads x 512, top-1024, a 128-token window)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


def test_algorithmic_bytes_of_the_decode_kernels():
    import bench
    ctx = 1 << 20
    keys = ctx // 4                          # CSA / indexer entries per sequence
    key_bytes = 128 // 2 + 128 // 32         # FP4 codes + E8M0 scales
    assert bench.SCAN_BYTES_PER_SEQ == keys * key_bytes == 17_825_792
    q, out, lse = 64 * 512 * 2, 64 * 512 * 4, 64 * 4
    csa_seq = (1024 + 128) * 576 + 1024 * 4 + q + out + lse
    hca_seq = (ctx // 128 + 128) * 576 + q + out + lse
    assert bench.CSA_SEQ_BYTES == csa_seq == 864_512
    assert bench.KERNELS["index_scan"]["bytes"] == 16 * 17_825_792
    assert bench.KERNELS["csa_attend"]["bytes"] == 16 * csa_seq + 64 * 4
    assert bench.KERNELS["hca_attend"]["bytes"] == 16 * hca_seq + 64 * 4 == 16 * 4_989_184 + 256
    assert bench.CSA4_BYTES == 4 * (17_825_792 + 864_512) + 256 == 74_761_472


def test_roofline_reports_the_kernel_with_most_hbm_bytes():
    import bench
    dom = max(bench.KERNELS, key=lambda k: bench.KERNELS[k]["per_step"] * bench.KERNELS[k]["bytes"])
    assert dom == "index_scan"
    spec = bench.KERNELS[dom]
    # HBM-bound: its bytes at 8 TB/s take longer than its arithmetic at the FP4 MFMA peak
    assert spec["bytes"] / 8e12 > spec["flops"] / spec["peak_flops"]
