"""Resume from a state written by a process that then died (yfxerp page,
section 1.2: the recurrent call takes an initial state and returns the final
one).  A first process runs the first part of a sequence, writes its final
state to disk and (on the oracle) is killed with SIGKILL; a fresh process
resumes from that file.  The resumed run must equal one uninterrupted run exactly: bit for bit
on the oracle (fp64, the same operations in the same order) and on the GPU
(a split at a multiple of 64 tokens keeps the chunk schedule and the fp32
state carry)."""
import os
import signal
import subprocess
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
WORKER = os.path.join(HERE, "resume_worker.py")


def _run(args, tmp, timeout=600):
    r = subprocess.run([sys.executable, WORKER, *args], capture_output=True, text=True, timeout=timeout, cwd=tmp)
    return r


def _resume_case(mode, tmp, seed, t_split, t_total, die=True):
    a_state, a_o = str(tmp / "a_state.npy"), str(tmp / "a_o.npy")
    b_state, b_o = str(tmp / "b_state.npy"), str(tmp / "b_o.npy")
    w_state, w_o = str(tmp / "w_state.npy"), str(tmp / "w_o.npy")
    r = _run([mode, str(seed), str(t_total), "0", str(t_split), "-", a_state, a_o] + (["--die"] if die else []), tmp)
    assert r.returncode == (-signal.SIGKILL if die else 0), (r.returncode, r.stderr[-2000:])
    r = _run([mode, str(seed), str(t_total), str(t_split), str(t_total), a_state, b_state, b_o], tmp)
    assert r.returncode == 0, r.stderr[-2000:]
    r = _run([mode, str(seed), str(t_total), "0", str(t_total), "-", w_state, w_o], tmp)
    assert r.returncode == 0, r.stderr[-2000:]
    whole_o, whole_s = np.load(w_o), np.load(w_state)
    parts_o = np.concatenate([np.load(a_o), np.load(b_o)], axis=1)
    assert np.array_equal(np.load(b_state), whole_s), "resumed final state differs"
    assert np.array_equal(parts_o, whole_o), "resumed outputs differ"


def test_oracle_resume_after_kill(tmp_path):
    _resume_case("oracle", tmp_path, seed=91, t_split=40, t_total=96)


@pytest.mark.gpu
def test_gpu_resume_in_fresh_process(tmp_path):
    from helpers import say
    say("resume in a fresh process: GPU, 4096 + 4096 tokens")
    # the first process exits normally here: no process is killed while it
    # holds the GPU; the kill itself is exercised by the oracle case
    _resume_case("gpu", tmp_path, seed=92, t_split=4096, t_total=8192, die=False)
