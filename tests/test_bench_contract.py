"""Host-side parts of bench.py: the one-GPU refusal, the algorithmic byte
count it divides by the launch time, and the stored HBM counter figures it
reports as traffic.  No GPU needed."""
import json
import os
import subprocess
import sys

import numpy as np

import lossless_entropy_coded_huffman_amd as dfh
from lossless_entropy_coded_huffman_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                           capture_output=True, text=True, timeout=120,
                           env=dict(os.environ, **env))
        assert r.returncode == 2
        assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_per_kind():
    # bytes read: the stream rounded up to bytes, 5 gap bits per thread, one
    # u64 offset per tile plus one, and for BF16 one sign|mantissa byte per
    # weight; bytes written: the decoded output
    x = synth.bf16_rne(np.random.default_rng(1).normal(0, 0.02, 300_001).astype(np.float32))
    c = dfh.compress(dfh.KIND_BF16, x)
    inf = c.info()
    sb = inf["section_bytes"]
    stream = (inf["total_bits"] + 7) // 8
    assert sb["bitstream"] >= stream                       # stored with padding
    expect = stream + (5 * inf["n_threads"] + 7) // 8 + 8 * (inf["n_tiles"] + 1) + 300_001 + 2 * 300_001
    assert bench.algorithmic_bytes(inf) == expect
    # about 3.36 bytes per weight at the exponent's ~2.6-bit codes
    assert 3.2 < bench.algorithmic_bytes(inf) / 300_001 < 3.5
    q = synth.quantize_u8(np.random.default_rng(2).normal(0, 0.02, 70_000).astype(np.float32), False)
    inf = dfh.compress(dfh.KIND_U8, q).info()
    assert bench.algorithmic_bytes(inf) == (inf["total_bits"] + 7) // 8 + (5 * inf["n_threads"] + 7) // 8 \
        + 8 * (inf["n_tiles"] + 1) + 70_000
    p = synth.pack_u4(synth.quantize_u4(np.random.default_rng(3).normal(0, 0.02, 70_001).astype(np.float32), True))
    inf = dfh.compress(dfh.KIND_U4, p, n=70_001).info()
    assert bench.algorithmic_bytes(inf) == (inf["total_bits"] + 7) // 8 + (5 * inf["n_threads"] + 7) // 8 \
        + 8 * (inf["n_tiles"] + 1) + 35_001


def test_stored_traffic_figures_are_consistent():
    prof = json.load(open(bench.PROFILE_COUNTERS))
    assert "llama3_8b_block_bf16" in prof
    for name, e in prof.items():
        assert name in bench.WORKLOADS
        # FETCH_SIZE counts half the bytes read, WRITE_SIZE all bytes written
        # (the copy calibration), both in KiB per dispatch
        assert (e["fetch_scale"], e["write_scale"]) == (2.0, 1.0)
        total = e["fetch_size_kib"] * 1024 * 2 + e["write_size_kib"] * 1024
        assert abs(e["bytes_per_launch"] - total) < 2 * 1024 * 0.1 + 1
        src = os.path.join(ROOT, e["source"])
        assert os.path.exists(src)
        assert e["kernel_source_sha"] in open(src).read()
        assert len(e["kernel_source_sha"]) == 16


def test_kernel_sha_is_the_decoder_source():
    import hashlib
    p = os.path.join(ROOT, "lossless_entropy_coded_huffman_amd", "csrc", "dfh_decode.hip")
    assert bench.kernel_sha() == hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]
