"""CPU checks of bench.py's command-line contract (no GPU needed): more than
one GPU is refused with a message and a non-zero exit, and the algorithmic
byte counts the roofline uses follow from the expert format."""
import json
import os
import subprocess
import sys

import oracle as orc
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_algorithmic_bytes_match_the_expert_format():
    sys.path.insert(0, ROOT)
    import bench
    d, f, E, k, L = synth.D_MODEL, synth.D_FF, synth.N_EXPERTS, synth.TOP_K, synth.N_LAYERS
    assert bench.blob_bytes() == orc.blob_bytes(d, f) == 3345408
    per_layer, _, _ = bench.decode_bytes()
    # router (fp32 E x d), RMSNorm weight, k expert blobs per layer
    assert per_layer == E * d * 4 + d * 4 + k * orc.blob_bytes(d, f)
    assert L * per_layer == 846489600
