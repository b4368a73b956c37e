"""bench.py's contract checks that need no GPU: more than one GPU is refused with a message
before anything else runs, and the committed HBM-traffic record parses (CPU only)."""
import json
import os
import re
import subprocess
import sys

from tests.conftest import ROOT


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode != 0
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""             # no JSON line


def test_traffic_record_is_well_formed():
    path = os.path.join(ROOT, "profiles", "decode_kernel_hbm_traffic.md")
    text = open(path).read()
    rec = json.loads(re.search(r"```json\n(.*?)\n```", text, flags=re.S).group(1))
    assert re.fullmatch(r"[0-9a-f]{16}", rec["decode_source_sha256_16"])
    assert rec["fetch_scale"] > 0 and rec["write_scale"] > 0
    # the fetched bytes cover at least the KV + Q the decode must read (75.57 MB at batch 1)
    assert rec["bytes_per_launch"]["b1_h128_l131072"] >= 75_571_200
    assert rec["bytes_per_launch"]["b16_h128_l131072_contig"] >= 1_209_139_200
