"""The oracle's pins must catch plausible mistakes in the oracle itself.

Each case plants one mistake in a copy of oracle/hils_oracle.py (a dropped
term, a wrong sign, an off-by-one, a swapped tie-break, ...), runs the pin
tests (tests/test_oracle_pins.py) against that copy in a fresh process, and
requires at least one pin to fail.  The unmodified copy must pass, so a
failure can only come from the planted mistake.  CPU only; the GPU path is not
involved.
"""
import os
import shutil
import subprocess
import sys
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in the oracle, replacement)
MUTATIONS = [
    ("tie_break_highest_id", "order = np.lexsort((cand, -g32))", "order = np.lexsort((-cand, -g32))"),
    ("group_score_max", "gbar = s_all.mean(axis=0)", "gbar = s_all.max(axis=0)"),
    ("bias_dropped", "s_all = s_all + bias[cand][None, :]", "s_all = s_all + 0.0 * bias[cand][None, :]"),
    ("retrieval_unscaled", "s_all = scale * (qr @ lmk[cand].T)", "s_all = (qr @ lmk[cand].T)"),
    ("own_chunk_is_candidate", "cand = np.arange(0, max(0, min(first_local, NC)))",
     "cand = np.arange(0, max(0, min(first_local + 1, NC)))"),
    ("own_chunk_misses_self", "own_rng = (own * S, t + 1)", "own_rng = (own * S, t)"),
    ("window_score_zero", "s_c = lse_c ", "s_c = 0.0 * lse_c "),
    ("token_logits_unscaled", "logits = scale * (k_blk @ q)", "logits = (k_blk @ q)"),
    ("fusion_unnormalised", "w = np.exp(s_vec - LSE)", "w = np.exp(s_vec - np.max(s_vec))"),
    ("ds_sign", "ds = wc * (Dc - D)", "ds = wc * (D - Dc)"),
    ("dl_without_Dc", "dl = wc * p * (u - Dc)", "dl = wc * p * u"),
    ("dv_unweighted", "np.outer(wc * p, g)", "np.outer(p, g)"),
    ("entropy_sign", "bias[b, g, c] = -float(np.sum(p[nz] * np.log(p[nz])))",
     "bias[b, g, c] = float(np.sum(p[nz] * np.log(p[nz])))"),
    # (dropping the "+ 1" of d(-p log p)/dp would be an equivalent mutant: the
    # softmax backward removes any constant added to every dp_j)
    ("landmark_bwd_uncentred", "dl = p * (dp - float(p @ dp))", "dl = p * dp"),
    ("landmark_bwd_entropy_sign", "dp = kb @ dm - db * (logp + 1.0)", "dp = kb @ dm + db * (logp + 1.0)"),
    ("query_position_shift", "t = Lkv - Lq + i", "t = Lkv - Lq + i - 1"),
    ("window_gap", "first_local = own - max(w - 1, 0)", "first_local = own - w"),
    ("window_chunk_short", "else (c * S, c * S + S)", "else (c * S, c * S + S - 1)"),
    ("one_selection_short", "order[:min(K, len(cand))]", "order[:min(K - 1, len(cand))]"),
    ("dq_without_score_term", 'res["dq"][h] = dq + dqr', 'res["dq"][h] = dq'),
    ("dk_unscaled", "scale * np.outer(dl, q)", "np.outer(dl, q)"),
    ("dlmk_unscaled", 'res["dlmk"].append((c, scale * ds * qr[h]))', 'res["dlmk"].append((c, ds * qr[h]))'),
]


def _copy_tree(dst):
    for name in ("oracle",):
        shutil.copytree(os.path.join(ROOT, name), os.path.join(dst, name),
                        ignore=shutil.ignore_patterns("__pycache__", "*.so", "*.o"))
    os.makedirs(os.path.join(dst, "tests"))
    for name in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", name), os.path.join(dst, "tests", name))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), os.path.join(dst, "pytest.ini"))


def _pins_cmd(dst):
    env = dict(os.environ, PYTHONPATH=dst, PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           "tests/test_oracle_pins.py"]
    return cmd, env


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    """Return code of the pin run for every mutation (and for the pristine copy),
    four pin runs at a time."""
    base = tmp_path_factory.mktemp("mutations")
    jobs = {}
    for name, old, new in [("pristine", None, None)] + MUTATIONS:
        dst = str(base / name)
        _copy_tree(dst)
        if old is not None:
            path = os.path.join(dst, "oracle", "hils_oracle.py")
            src = open(path).read()
            assert src.count(old) >= 1, f"mutation site for {name} not found"
            open(path, "w").write(src.replace(old, new, 1))
        jobs[name] = dst
    results, running, queue = {}, {}, list(jobs.items())
    deadline = time.monotonic() + 900
    try:
        while queue or running:
            assert time.monotonic() < deadline, "pin runs did not finish in 900 s"
            while queue and len(running) < 4:
                name, dst = queue.pop(0)
                cmd, env = _pins_cmd(dst)
                log = open(os.path.join(dst, "pins.log"), "w")
                running[name] = (subprocess.Popen(cmd, cwd=dst, env=env, stdout=log,
                                                  stderr=subprocess.STDOUT), log)
            for name in list(running):
                proc, log = running[name]
                if proc.poll() is not None:
                    log.close()
                    results[name] = (proc.returncode,
                                     open(os.path.join(jobs[name], "pins.log")).read())
                    del running[name]
            time.sleep(0.2)
    finally:
        for proc, log in running.values():
            proc.kill()
            proc.wait()
            log.close()
    return results


def test_pristine_copy_passes(outcomes):
    code, out = outcomes["pristine"]
    assert code == 0, "the unmodified copy must pass its pins:\n" + out[-2000:]


@pytest.mark.parametrize("name", [m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(outcomes, name):
    assert outcomes["pristine"][0] == 0
    code, out = outcomes[name]
    assert code != 0, f"no pin failed with the mistake '{name}' planted:\n" + out[-1000:]
