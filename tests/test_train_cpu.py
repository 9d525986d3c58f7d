"""Host logic of the training driver: the learning-rate schedule against the
oracle's, the resumable data cursor, and the supervisor's relaunch and marker
rules (forced from the host with stub child processes; no GPU)."""
import json
import os
import sys

import numpy as np
import pytest

import oracle
from transformer_lm_pretraining_amd import synth, train


def test_lr_schedule_matches_oracle():
    for t in [1, 2, 350, 699, 700, 701, 1000, 5000, 9782, 18000, 18864, 18865]:
        assert train.lr_at(t) == pytest.approx(oracle.lr_at(t), rel=1e-12, abs=1e-18), t
    assert train.lr_at(18865) == pytest.approx(0.0, abs=1e-12)


def test_token_stream_resumes_exactly():
    a = synth.TokenStream(50257, seed=5)
    first = [a.micro_batch(2, 64) for _ in range(3)]
    b = synth.TokenStream.from_state(json.loads(json.dumps(a.state())))
    rest = [b.micro_batch(2, 64) for _ in range(4)]
    ref = [synth.TokenStream(50257, seed=5).micro_batch(2, 64)]
    c = synth.TokenStream(50257, seed=5)
    ref = [c.micro_batch(2, 64) for _ in range(7)]
    for (t1, g1), (t2, g2) in zip(first + rest, ref):
        np.testing.assert_array_equal(t1, t2)
        np.testing.assert_array_equal(g1, g2)
    tok, tgt = ref[0]
    assert tok[0, 0] == 50256  # the stream opens with end-of-text
    np.testing.assert_array_equal(tok.ravel()[1:], tgt.ravel()[:-1])  # targets are the next ids
    assert ref[1][0].ravel()[0] == ref[0][1].ravel()[-1]  # consecutive micro-batches share one id


def _stub(tmp_path, body):
    """A child process that keeps a launch counter in tmp_path and then runs `body`."""
    script = tmp_path / "child.py"
    script.write_text(
        "import os, sys\n"
        f"d = {str(tmp_path)!r}\n"
        "c = os.path.join(d, 'count')\n"
        "n = int(open(c).read()) + 1 if os.path.exists(c) else 1\n"
        "open(c, 'w').write(str(n))\n" + body)
    return [sys.executable, str(script)]


def test_supervisor_relaunches_after_a_crash_until_complete(tmp_path):
    cmd = _stub(tmp_path, "if n == 1: sys.exit(7)\nopen(os.path.join(d, 'COMPLETE'), 'w').write('done')\n")
    assert train.supervise(cmd, str(tmp_path), log=lambda s: None) == 2
    assert (tmp_path / "count").read_text() == "2"


def test_supervisor_does_not_launch_past_a_halt_marker(tmp_path):
    (tmp_path / "HALT").write_text("gate")
    cmd = _stub(tmp_path, "")
    assert train.supervise(cmd, str(tmp_path), log=lambda s: None) == 0
    assert not (tmp_path / "count").exists()


def test_supervisor_stops_when_the_child_halts(tmp_path):
    cmd = _stub(tmp_path, "open(os.path.join(d, 'HALT'), 'w').write('gate')\nsys.exit(3)\n")
    assert train.supervise(cmd, str(tmp_path), log=lambda s: None) == 1


def test_supervisor_gives_up_after_max_restarts(tmp_path):
    cmd = _stub(tmp_path, "sys.exit(1)\n")
    assert train.supervise(cmd, str(tmp_path), max_restarts=2, log=lambda s: None) == 3
