"""Host logic of bench.py without a GPU: its launch schedule and byte counts
agree with the oracle's pass schedule (the pass the metric is defined on),
the GDN state-stream byte count follows its definition, and a request for
more than one GPU is refused with a message."""
import importlib.util
import os
import subprocess
import sys

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_schedule_matches_the_oracle_pass():
    B = _bench()
    ours = B.schedule()
    ref = O.pass_schedule()
    assert len(ours) == len(ref) == 257
    for (k1, f1, n1, kk1), (k2, f2, n2, kk2) in zip(ours, ref):
        assert k1 == k2 and kk1 == kk2
        # the fused [gate; up] launch is listed by its output width (half the weight rows)
        assert (2 * n1 if f1 == "nvfp4_silu" else n1) == n2
        assert (f1 == "fp8") == (f2 == "fp8")
    total = sum(B.weight_bytes(f, n, k) for _, f, n, k in ours)
    assert total == 17_555_292_160
    assert total == sum(O.bytes_nvfp4(n, k) if f == "nvfp4" else O.bytes_fp8(n, k) for _, f, n, k in ref)


def test_gdn_state_bytes():
    B = _bench()
    state = 48 * 48 * 128 * 128 * 4            # one slot, one lane: 150,994,944 B
    assert state == 150_994_944
    rows = 8 * (16 * 128 * 4 * 2 + 48 * 128 * 4 * 2 + 48 * 4 * 2)   # q, k, v, o, a, b of 8 rows, one layer
    assert B.gdn_bytes(48, 1, 8) == 2 * state + 48 * rows
    # the commit reads no queries and writes no outputs
    commit_rows = 4 * (16 * 128 * 4 + 48 * 128 * 4 + 48 * 4 * 2)
    assert B.gdn_bytes(48, 1, 4, read_q=False, write_o=False) == 2 * state + 48 * commit_rows
    assert B.gdn_bytes(48, 4, 8) == 4 * B.gdn_bytes(48, 1, 8)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
