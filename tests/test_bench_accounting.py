"""Host-side accounting of bench.py (CPU only): the algorithmic bytes and updates per launch that
the roofline figures divide by, checked against independently worked figures for the 721x1440 and
181x360 workloads (bytes = inputs + outputs once + 8 bytes per psi entry + 4 per CSR row pointer;
updates = B * C * Wo * nnz), and the rule that measured traffic is reported only for the kernel
source the counters were taken on."""
import hashlib
import json
import os

import pytest

import bench
from disco_inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name,op,nnz,mb", [
    ("fwd_bf16_721x1440", "fwd", 1_842_128, 413.8),   # x 132.9 MB + out 266.2 MB + psi 14.7 MB
    ("bwd_bf16_721x1440", "bwd", 1_842_128, 413.8),
    ("fwdbwd_f32_181x360", "fwd", 23_309, 67.1),      # x 33.4 MB + out 33.5 MB + psi 0.19 MB
    ("fused_bf16_721x1440", "fused", 3_417_372, 2156.0),  # x 1063 + W 2.1 + y 1063 + psi 27.4 MB
])
def test_algorithmic_bytes(name, op, nnz, mb):
    w = WORKLOADS[name]
    assert bench.op_bytes(op, w, nnz, w.Co) / 1e6 == pytest.approx(mb, rel=2e-3)


def test_updates_and_einsum_macs():
    w = WORKLOADS["fwd_bf16_721x1440"]
    assert bench.op_updates(w, 1_842_128) == 1 * 64 * 720 * 1_842_128  # 84.89 G
    u = WORKLOADS["fused_bf16_721x1440"]
    assert bench.op_updates(u, 3_417_372) / 1e9 == pytest.approx(2519.6, rel=1e-4)
    assert u.B * u.Ho * u.Wo * u.Co * u.C * u.K == 2_177_347_092_480


def test_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "sparse_gather_contraction_amd", "csrc", bench.KERNEL_SOURCES["fused"])
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (tmp_path / "sparse_gather_contraction_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "sparse_gather_contraction_amd" / "csrc" / bench.KERNEL_SOURCES["fused"]).write_bytes(
        open(src, "rb").read())
    rec = {"kernel": "fused", "read_bytes": 100, "write_bytes": 20, "source_sha256": digest}
    summary = prof / "disco_step_721x1440_hbm_counters.md"
    summary.write_text("text\n\ntraffic-record: " + json.dumps(rec) + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic("fused") == 120
    assert bench.counter_traffic("fwd") is None                   # no record for this kernel
    rec["source_sha256"] = "0" * 64
    summary.write_text("traffic-record: " + json.dumps(rec) + "\n")
    assert bench.counter_traffic("fused") is None                 # counters of another source
