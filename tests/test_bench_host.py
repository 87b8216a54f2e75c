"""Host-side pieces of bench.py that need no GPU: the algorithmic byte and flop counts behind the
roofline figures, the source-hash gate on recorded HBM traffic, and the one-GPU refusal."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_algorithmic_bytes():
    # per token-head: q, k (2 x 128) and v (128) bf16, g 128 float32, beta bf16, o 128 bf16
    per_th = (2 * 128 + 128) * 2 + 128 * 4 + 2 + 128 * 2
    assert per_th == 1538
    states = 2 * 4 * 32 * 128 * 128 * 4                    # S0 read, S_T written, float32
    assert bench.prefill_alg_bytes(4, 32768, 32, 128, 128, 4) == 4 * 32768 * 32 * per_th + states
    assert bench.prefill_alg_bytes(4, 32768, 32, 128, 128, 4) == 6_467_616_768


def test_prefill_gate_algorithmic_bytes():
    # bf16 logits z (128) replace the float32 g (512 B): 1282 B per token-head, plus H log-scales
    assert bench.prefill_gate_alg_bytes(4, 32768, 32, 128, 128, 4) == \
        4 * 32768 * 32 * 1282 + 2 * 4 * 32 * 128 * 128 * 4 + 32 * 4


def test_decode_algorithmic_bytes():
    unit = 2 * 128 * 128 * 4 + 1538                          # state in and out, one token
    assert bench.decode_alg_bytes(1024, 32, 128, 128) == 1024 * 32 * unit == 4_345_364_480
    assert bench.decode_alg_bytes(1024, 32, 128, 128, K=4) == \
        1024 * 32 * (2 * 128 * 128 * 4 + 4 * 1538)


def test_prefill_algorithmic_flops_per_token_head():
    # C = 32, d = 128, causal 16x16 tiles only: 24,576 intra-chunk + 104,448 inter-chunk flops
    assert bench.prefill_alg_flops(1, 1, 1, 128, 128) == 129_024
    # C = 64 grows the intra-chunk share (more causal tiles per token)
    assert bench.prefill_alg_flops(1, 1, 1, 128, 128, C=64) == 149_504


def test_recorded_traffic_is_gated_by_the_kernel_source():
    assert bench.measured_traffic("no such kernel", "kda_prefill.hip") is None
    rec = json.load(open(os.path.join(ROOT, "profiles", "kernel_counters.json")))
    for key, src in (("prefill_kernel<128,bf16,bf16>", "kda_prefill.hip"),
                     ("decode_kernel<128,128,bf16,bf16>", "kda_decode.hip")):
        t = bench.measured_traffic(key, src)
        if rec[key]["source_sha256_16"] == bench.kernel_source_hash(src):
            assert t is not None and t > 0
        else:
            assert t is None
        # the other kernel's source never validates this record
        other = "kda_decode.hip" if src == "kda_prefill.hip" else "kda_prefill.hip"
        assert bench.measured_traffic(key, other) is None
        assert bench.measured_mfma_busy(key, other) is None


def test_more_than_one_gpu_is_refused_before_any_device_use():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
