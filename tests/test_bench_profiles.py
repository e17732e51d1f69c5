"""CPU checks of the committed profile summaries that bench.py reads into its roofline line.

Each workload's default step has HBM-traffic and SQ-counter summaries under profiles/, keyed by
the kernel sources' digest.  The digest a file states must be the one its machine-readable lines
carry; while it is the digest of the current sources, every kernel of the step (forward, dq and
dkdv of each variant) must find its measured traffic and issue shares there."""
import os
import re

import pytest

import bench
from quantized_softmax_attention_kia_amd.inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("wl", ["gpt2", "wide", "1b", "long"])
@pytest.mark.parametrize("kind", ["hbm_traffic", "sq_counters"])
def test_profile_lines_match_their_digest_and_cover_the_step(wl, kind):
    path = os.path.join(ROOT, "profiles", f"{kind}_{wl}_fwd_bwd.md")
    text = open(path).read()
    stated = re.search(r"Kernel sources digest \(bench.py `sources_digest`\): `([0-9a-f]{16})`", text).group(1)
    tag = "traffic" if kind == "hbm_traffic" else "issue"
    lines = [ln.split() for ln in text.splitlines() if ln.strip().startswith(tag + " ")]
    assert lines, "no machine-readable lines"
    assert {ln[-1] for ln in lines} == {stated}
    if stated != bench.sources_digest():
        pytest.skip("the kernel sources changed since these counters were taken: bench reports null")
    read = bench.read_traffic if kind == "hbm_traffic" else bench.read_issue
    for var in WORKLOADS[wl].variants:
        for stage in ("fwd", "dq", "dkdv"):
            got = read(f"{stage}:{var.name}", wl)
            assert got is not None, (stage, var.name)
            if kind == "sq_counters":
                assert 0.0 < got["valu_busy"] < 1.0 and 0.0 < got["mfma_busy"] < 1.0
                assert got["limiter"] in ("valu", "mfma")
            else:
                assert got > 0.0
