"""Host-side logic of bench.py (no GPU): the byte counts the roofline
fraction is built on, the kernel-source hash that keys the committed
counter runs, and the one-GPU contract."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_headline_algorithmic_bytes():
    """64 064 x 2560 NVFP4 at batch 1: 82 001 920 code bytes + 10 250 240
    scale bytes + 5120 bytes of h + the global scale, the winning dh_idx
    entry and the out id (4 bytes each) = 92 257 292 bytes."""
    assert bench.weight_bytes("nvfp4", 64064, 2560) == 82001920 + 10250240
    assert bench.algorithmic_bytes("nvfp4", 64064, 2560, 1, "top",
                                   248320) == 92257292


def test_other_algorithmic_bytes():
    # the 98K head at batch 16: codes + scales + h + scale + 16 (id, entry)
    assert bench.algorithmic_bytes("nvfp4", 98304, 2560, 16, "top", 248320) \
        == 98304 * 1280 + 98304 * 160 + 16 * 5120 + 4 + 16 * 8
    # the W8A8 step moves what the W8A16 step moves (its quantized tokens
    # are an intermediate)
    assert bench.algorithmic_bytes("w8a8", 98304, 2560, 16, "top", 248320) \
        == bench.algorithmic_bytes("e4m3", 98304, 2560, 16, "top", 248320)
    # logits: the dh_idx column and the full fp32 (or BF16) output
    base = bench.weight_bytes("nvfp4", 64064, 5120) + 8 * 5120 * 2 + 4
    assert bench.algorithmic_bytes("nvfp4", 64064, 5120, 8, "logits",
                                   248320) == base + 64064 * 4 + 8 * 248320 * 4
    assert bench.algorithmic_bytes("nvfp4", 64064, 5120, 8, "logits_bf16",
                                   248320) == base + 64064 * 4 + 8 * 248320 * 2
    # the linear: weights, h, the scale and the dense output
    assert bench.algorithmic_bytes("nvfp4", 2560, 5120, 1, "linear", 2560) \
        == 2560 * 2560 + 2560 * 320 + 5120 * 2 + 4 + 2560 * 4


def test_kernel_hash_ignores_comments_but_not_code(tmp_path):
    src = os.path.join(ROOT, "reduced_vocab_nvfp4_amd", "csrc")
    copy = tmp_path / "csrc"
    shutil.copytree(src, copy)
    h0 = bench.kernel_source_hash(str(copy))
    assert h0 == bench.kernel_source_hash()
    p = copy / "gemv_b1.hip"
    text = p.read_text()
    p.write_text("// a new comment line\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_source_hash(str(copy)) == h0
    code = "constexpr int B1_BLOCKS_PER_CU = 2;"
    assert code in text
    p.write_text(text.replace(code, "constexpr int B1_BLOCKS_PER_CU = 3;"))
    assert bench.kernel_source_hash(str(copy)) != h0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_a_negative_seed_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--seed", "-1"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2
    assert "--seed" in r.stderr
