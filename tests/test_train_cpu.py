"""Host logic of the training driver: the learning-rate schedule against the
oracle's, the resumable data cursor, the supervisor's relaunch and marker
rules, and the halting gate (forced from the host with stub child processes;
no GPU)."""
import json
import os
import sys
import threading
import time

import numpy as np
import pytest

import oracle
from transformer_lm_pretraining_amd import supervisor, synth, train


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
    assert supervisor.supervise(cmd, str(tmp_path), log=lambda s: None) == 2
    assert (tmp_path / "count").read_text() == "2"


def test_supervisor_does_not_launch_past_a_halt_marker(tmp_path):
    (tmp_path / "HALT").write_text("gate")
    cmd = _stub(tmp_path, "")
    assert supervisor.supervise(cmd, str(tmp_path), log=lambda s: None) == 0
    assert not (tmp_path / "count").exists()


def test_supervisor_stops_when_the_child_halts(tmp_path):
    cmd = _stub(tmp_path, "open(os.path.join(d, 'HALT'), 'w').write('gate')\nsys.exit(3)\n")
    assert supervisor.supervise(cmd, str(tmp_path), log=lambda s: None) == 1


def test_supervisor_gives_up_after_max_restarts(tmp_path):
    cmd = _stub(tmp_path, "sys.exit(1)\n")
    assert supervisor.supervise(cmd, str(tmp_path), max_restarts=2, log=lambda s: None) == 3


def test_gate_halts_on_three_consecutive_evaluations_above_the_margin():
    ref = {250: 4.0, 500: 3.8, 750: 3.6, 1000: 3.5, 1250: 3.4}
    g = supervisor.gate
    assert g([], ref)[0] == "waiting"
    assert g([(250, 4.1)], ref)[0] == "normal"  # 2.5% above: inside the margin
    assert g([(250, 4.3)], ref)[0] == "alert"  # 7.5% above
    assert g([(250, 4.3), (500, 4.1)], ref)[0] == "alert"
    assert g([(250, 4.3), (500, 4.1), (750, 3.9)], ref)[0] == "halt"
    # a normal evaluation breaks the streak
    assert g([(250, 4.3), (500, 3.9), (750, 3.9), (1000, 3.7)], ref)[0] == "alert"
    # exactly 5% above is not above the margin
    assert g([(250, 4.0 * 1.05)], ref)[0] == "normal"
    # steps the reference lacks are not judged and keep the streak
    assert g([(250, 4.3), (300, 9.0), (500, 4.1), (600, 1.0), (750, 3.9)], ref)[0] == "halt"
    assert g([(300, 9.0)], ref)[0] == "normal"
    # after a relaunch the last loss at a repeated step counts
    assert g([(250, 4.3), (500, 4.1), (500, 3.8), (750, 3.9)], ref)[0] == "alert"


def test_sidecar_halts_a_supervised_run_and_the_supervisor_stops(tmp_path):
    """The stub trainer logs three evaluations 10% above the reference and then
    hangs; the sidecar must write the halt marker and end the trainer's process
    group, and the supervisor must not relaunch it."""
    recs = [{"step": s, "loss": 5.0, "eval_loss": 1.1 * r} for s, r in ((250, 4.0), (500, 3.8), (750, 3.6))]
    body = ("import json, time\n"
            "with open(os.path.join(d, 'log.jsonl'), 'a') as f:\n"
            f"    for r in {recs!r}:\n"
            "        f.write(json.dumps(r) + '\\n')\n"
            "time.sleep(60)\n")
    cmd = _stub(tmp_path, body)
    ref = {250: 4.0, 500: 3.8, 750: 3.6}
    verdicts = []
    t = threading.Thread(target=lambda: verdicts.append(
        supervisor.sidecar(str(tmp_path), ref, interval=0.05, max_checks=400, log=lambda s: None)))
    t.start()
    t0 = time.time()
    launches = supervisor.supervise(cmd, str(tmp_path), log=lambda s: None)
    t.join()
    assert time.time() - t0 < 30  # the hanging trainer was ended, not waited out
    assert launches == 1 and verdicts == ["halt"]
    assert "step 750" in (tmp_path / "HALT").read_text()
    gate_log = [json.loads(x)["verdict"] for x in (tmp_path / "gate.jsonl").read_text().splitlines()]
    assert gate_log[-1] == "halt"
    assert not (tmp_path / "trainer.pgid").exists()


def test_sidecar_stops_when_the_run_completes(tmp_path):
    (tmp_path / "COMPLETE").write_text("6")
    assert supervisor.sidecar(str(tmp_path), {}, interval=0.01, log=lambda s: None) == "complete"
