"""The device-check build (build.py --device-checks) on the GPU: valid decode
steps and attention calls count no violation; planted faults -- selected
entries outside the visible range, pages of selected entries outside the pool
-- are each counted once.  The debug library runs in a child process
(tests/device_checks_child.py) so that this process keeps the release build."""
import json
import os
import subprocess
import sys

import pytest

from long_context_attention_14_amd import build as lca_build

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_device_checks_count_planted_faults_only():
    assert os.path.exists(lca_build.DBG_LIB), "build the device-check library first (__graft_entry__.build)"
    env = dict(os.environ, LCA_LIB=lca_build.DBG_LIB)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "device_checks_child.py")],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    print(r.stderr[-3000:], flush=True)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-3000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    print(res, flush=True)
    for case in ("csa_fused", "csa_lds", "csa_paged", "hca", "mqa_valid"):
        assert res[case] == 0, f"{case}: {res[case]} violations on valid inputs"
    assert res["mqa_bad_idx_planted"] == 3 and res["mqa_bad_idx"] == 3, res
    assert res["mqa_bad_pages_planted"] >= 2 and res["mqa_bad_pages"] == res["mqa_bad_pages_planted"], res
