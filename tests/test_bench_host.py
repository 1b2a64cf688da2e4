"""Host-side checks of bench.py: the one-GPU guard and the timing loop."""
import os
import subprocess
import sys
import time
import types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


class _Event:
    def __init__(self, log, enable_timing=False):
        self.log = log
        self.t = None

    def record(self):
        self.t = len(self.log)
        self.log.append("event")

    def elapsed_time(self, other):
        # one "millisecond" per step launched between the two records
        return float(sum(1 for x in self.log[self.t:other.t] if x == "step"))


def _fake_torch(log):
    cuda = types.SimpleNamespace(Event=lambda enable_timing=False: _Event(log, enable_timing),
                                 synchronize=lambda: log.append("sync"))
    return types.SimpleNamespace(cuda=cuda)


def test_time_steps_brackets_exactly_the_timed_steps():
    log = []
    wall, ev, warm_steps, warm_ms = bench.time_steps(lambda: log.append("step"), steps=7,
                                                     warmup=3, torch=_fake_torch(log))
    assert warm_steps == 3 and warm_ms >= 0.0
    assert log.count("step") == 10
    assert log.count("event") == 2
    first = log.index("event")
    # warm-up steps all come before the first event, the timed ones between the two
    assert log[:first].count("step") == 3
    assert log[first:].count("step") == 7
    assert ev == 1.0
    assert wall >= 0.0


def test_time_steps_warms_for_the_minimum_time():
    log = []

    def step():
        log.append("step")
        time.sleep(0.002)

    _, _, warm_steps, warm_ms = bench.time_steps(step, steps=2, warmup=2, torch=_fake_torch(log),
                                                 min_warm_ms=30.0)
    first = log.index("event")
    # the warm-up ran on past its 2 steps until 30 ms had passed (each step
    # sleeps at least 2 ms, often more on a busy host, so no exact count)
    assert log[:first].count("step") > 2
    assert warm_steps == log[:first].count("step") and warm_ms >= 30.0
    assert log[first:].count("step") == 2


def test_decode_work_counts_each_key_once():
    """Algorithmic bytes of a multi-token decode: the K/V of the keys any of
    a sequence's queries sees, once, plus q/out and the bias entries used."""
    import types as _t
    sp = _t.SimpleNamespace(head_dim=128, num_q_heads=32, num_kv_heads=8, window=0,
                            rel_extent=1024)
    one = _t.SimpleNamespace(spec=sp, seq_lens=[5000], q_len=1)
    four = _t.SimpleNamespace(spec=sp, seq_lens=[5000], q_len=4)
    f1, b1 = bench.decode_work(one)
    f4, b4 = bench.decode_work(four)
    kv = 5000 * 8 * 128 * 2 * 2
    assert b1 == kv + 32 * 1024 * 2 + 32 * 128 * 2 * 2
    assert b4 == kv + 4 * 32 * 1024 * 2 + 4 * 32 * 128 * 2 * 2
    assert f4 == 4 * 128 * 32 * (4997 + 4998 + 4999 + 5000)
    loc = _t.SimpleNamespace(head_dim=128, num_q_heads=32, num_kv_heads=16, window=512,
                             rel_extent=512)
    f, b = bench.decode_work(_t.SimpleNamespace(spec=loc, seq_lens=[5000], q_len=4))
    assert b == (512 + 3) * 16 * 128 * 2 * 2 + 4 * 32 * 512 * 2 + 4 * 32 * 128 * 2 * 2
    assert f == 4 * 128 * 32 * 512 * 4
