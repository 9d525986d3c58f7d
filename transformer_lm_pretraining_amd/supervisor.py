"""Run supervision after Pretraining and adapting a language model on a
dependency-free stack (supervision paragraphs of the pretraining section):

* the supervisor relaunches a crashed trainer, which resumes from its latest
  checkpoint, and stops for good once a completion or a halt marker exists;
* the sidecar gate reads the run's held-out losses from disk every few
  minutes, compares each against a reference curve at the same step, and after
  three consecutive evaluations more than 5% above the reference writes a halt
  marker and signals the trainer's whole process group.  The marker is what lets
  the supervisor tell a deliberate stop from a crash.

Host logic only: no GPU work happens here.
"""
from __future__ import annotations

import json
import os
import signal
import subprocess
import time

COMPLETE_MARKER = "COMPLETE"
HALT_MARKER = "HALT"
PGID_FILE = "trainer.pgid"
GATE_LOG = "gate.jsonl"
GATE_MARGIN = 0.05
GATE_PATIENCE = 3


def read_evals(run_dir: str):
    """[(step, held-out loss)] in log order from run_dir/log.jsonl (a missing log is empty;
    a torn last line is skipped)."""
    path = os.path.join(run_dir, "log.jsonl")
    out = []
    if not os.path.exists(path):
        return out
    with open(path) as f:
        for line in f:
            try:
                rec = json.loads(line)
            except json.JSONDecodeError:
                continue
            if "eval_loss" in rec:
                out.append((int(rec["step"]), float(rec["eval_loss"])))
    return out


def gate(evals, reference: dict, margin: float = GATE_MARGIN, patience: int = GATE_PATIENCE):
    """Verdict on a run's evaluations so far: (verdict, detail).

    verdict is "waiting" before the first evaluation, "halt" once the last
    `patience` evaluations that have a reference point at their step are all more
    than `margin` (relative) above it, "alert" while the latest such evaluation is
    above but the streak is shorter, else "normal".  An evaluation at a step the
    reference lacks is not judged and does not break a streak.  A relaunched run
    repeats steps: the last loss logged at a step counts, and steps are judged in
    step order."""
    if not evals:
        return "waiting", "no evaluation yet"
    latest = {}
    for step, loss in evals:
        latest[step] = loss
    streak = 0
    last = None
    for step in sorted(latest):
        loss, ref = latest[step], reference.get(step)
        if ref is None:
            continue
        last = (step, loss, ref)
        streak = streak + 1 if loss > ref * (1.0 + margin) else 0
    if last is None:
        return "normal", "no reference at the evaluated steps"
    step, loss, ref = last
    detail = f"step {step}: held-out {loss:.4f} vs reference {ref:.4f} ({streak} above in a row)"
    if streak >= patience:
        return "halt", detail
    return ("alert" if streak else "normal"), detail


def load_reference(path: str) -> dict:
    """Reference curve from a JSON object {step: held-out loss}."""
    with open(path) as f:
        return {int(k): float(v) for k, v in json.load(f).items()}


def halt(run_dir: str, reason: str, log=print) -> bool:
    """Writes the halt marker, then sends SIGTERM to the process group recorded in
    run_dir/trainer.pgid (if any).  Returns whether a group was signalled."""
    with open(os.path.join(run_dir, HALT_MARKER), "w") as f:
        f.write(reason + "\n")
    try:
        with open(os.path.join(run_dir, PGID_FILE)) as f:
            pgid = int(f.read().strip())
    except (OSError, ValueError):
        return False
    try:
        os.killpg(pgid, signal.SIGTERM)
    except ProcessLookupError:
        return False
    log(f"sidecar: halted process group {pgid}: {reason}")
    return True


def sidecar(run_dir: str, reference: dict, interval: float = 300.0, margin: float = GATE_MARGIN,
            patience: int = GATE_PATIENCE, max_checks: int | None = None, log=print) -> str:
    """Checks the run every `interval` seconds until it completes, is halted, or
    `max_checks` checks have run; appends each verdict to run_dir/gate.jsonl and
    halts the run on a "halt" verdict.  Returns the last verdict."""
    checks = 0
    verdict = "waiting"
    while max_checks is None or checks < max_checks:
        if os.path.exists(os.path.join(run_dir, COMPLETE_MARKER)):
            return "complete"
        if os.path.exists(os.path.join(run_dir, HALT_MARKER)):
            return "halted"
        verdict, detail = gate(read_evals(run_dir), reference, margin, patience)
        with open(os.path.join(run_dir, GATE_LOG), "a") as f:
            f.write(json.dumps({"time": time.time(), "verdict": verdict, "detail": detail}) + "\n")
        if verdict == "halt":
            halt(run_dir, detail, log)
            return verdict
        checks += 1
        if max_checks is None or checks < max_checks:
            time.sleep(interval)
    return verdict


def supervise(cmd, run_dir: str, max_restarts: int = 10, log=print) -> int:
    """Runs `cmd` (a list) until it leaves the completion marker in run_dir; relaunches it
    after a failure (the trainer resumes from run_dir/latest itself); stops for good,
    without launching, once a halt or completion marker exists.  Each launch runs in a
    process group of its own, recorded in run_dir/trainer.pgid for the sidecar.
    Returns the number of launches."""
    os.makedirs(run_dir, exist_ok=True)
    launches = 0
    while True:
        for marker in (HALT_MARKER, COMPLETE_MARKER):
            if os.path.exists(os.path.join(run_dir, marker)):
                log(f"supervisor: {marker} marker present, stopping after {launches} launch(es)")
                return launches
        if launches > max_restarts:
            log(f"supervisor: giving up after {launches} launches")
            return launches
        launches += 1
        child = subprocess.Popen(cmd, start_new_session=True)
        tmp = os.path.join(run_dir, PGID_FILE + ".tmp")
        with open(tmp, "w") as f:
            f.write(str(child.pid))
        os.replace(tmp, os.path.join(run_dir, PGID_FILE))
        rc = child.wait()
        os.remove(os.path.join(run_dir, PGID_FILE))  # the group is gone; its id may be reused
        log(f"supervisor: launch {launches} exited with {rc}")
