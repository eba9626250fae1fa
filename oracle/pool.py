"""Runs the oracle's per-group solver over many groups in P single-threaded processes.

Test infrastructure, like the rest of this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it. Groups are independent, so a tensor's groups are cut
into contiguous ranges and worker processes run the unchanged single-threaded C oracle on
them; results are identical to one ``Oracle.solve_groups`` call over the whole tensor.
Inputs and outputs pass through memory-mapped files in a temporary directory.

Each worker is a child process (``python -m oracle.pool``) that reads one task per line on
its standard input and answers each with a line starting "@@ok" on its standard output.
"""
from __future__ import annotations

import json
import os
import queue
import shutil
import subprocess
import sys
import tempfile
import threading

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# per-group outputs of Oracle.solve_groups and their element types
_FIELDS = (("scale", np.uint16), ("zero_f32", np.float32), ("s", np.float32),
           ("passes", np.uint8), ("last_change", np.uint8), ("shrink_active", np.uint8),
           ("stopped", np.uint8))

_worker_oracle = None


def _solve_range(task):
    """Worker: solves groups [a, b) of the memory-mapped input into the output maps."""
    global _worker_oracle
    if _worker_oracle is None:
        from oracle.hqq_oracle import Oracle
        _worker_oracle = Oracle()
    d, n_groups, g, nbits, params, a, b = task
    w = np.memmap(os.path.join(d, "w"), np.uint16, "r", shape=(n_groups * g,))
    r = _worker_oracle.solve_groups(np.array(w[a * g:b * g]), g, nbits, **params)
    codes = np.memmap(os.path.join(d, "codes"), np.uint8, "r+", shape=(n_groups * g,))
    codes[a * g:b * g] = r["codes"]
    codes.flush()
    for name, t in _FIELDS:
        m = np.memmap(os.path.join(d, name), t, "r+", shape=(n_groups,))
        m[a:b] = r[name]
        m.flush()
    return b - a


def default_procs() -> int:
    """Worker count: the host's cores, at most 16 (a GPU machine's CPU share)."""
    return max(1, min(16, os.cpu_count() or 1))


class OraclePool:
    """P worker processes, each with its own loaded oracle."""

    def __init__(self, procs: int | None = None):
        from oracle.hqq_oracle import build
        build(force=False)                 # the workers load the library, never build it
        self.procs = procs or default_procs()
        env = dict(os.environ)
        env["PYTHONPATH"] = _ROOT + os.pathsep + env.get("PYTHONPATH", "")
        self._w = [subprocess.Popen([sys.executable, "-m", "oracle.pool"], cwd=_ROOT, env=env,
                                    stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True)
                   for _ in range(self.procs)]

    def close(self):
        for p in self._w:
            if p.poll() is None:
                p.stdin.close()
        for p in self._w:
            try:
                p.wait(timeout=30)
            except subprocess.TimeoutExpired:
                p.kill()
                p.wait()
        self._w = []

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _run(self, tasks):
        """Hands the tasks to the workers, each taking the next one when it is free."""
        todo = queue.Queue()
        for t in tasks:
            todo.put(t)
        errors = []

        def feed(p):
            while not errors:
                try:
                    t = todo.get_nowait()
                except queue.Empty:
                    return
                p.stdin.write(json.dumps(t) + "\n")
                p.stdin.flush()
                while True:
                    line = p.stdout.readline()
                    if not line:
                        errors.append(f"oracle worker {p.pid} ended (status {p.poll()})")
                        return
                    if line.startswith("@@"):
                        break
                if not line.startswith("@@ok"):
                    errors.append(line.strip())
                    return

        threads = [threading.Thread(target=feed, args=(p,)) for p in self._w]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        if errors:
            raise RuntimeError("; ".join(errors))

    def solve_groups(self, w16, g, nbits, p=0.7, beta=1.0, kappa=1.01, iters=20,
                     early_stop=1, parts: int | None = None):
        """Same result as ``Oracle.solve_groups`` (codes, scale, zero_f32, s, passes,
        last_change, shrink_active, stopped, evals_needed), computed in parallel."""
        w16 = np.ascontiguousarray(w16, np.uint16).reshape(-1)
        assert w16.size % g == 0
        ng = w16.size // g
        d = tempfile.mkdtemp(prefix="hqq_oracle_")
        try:
            np.memmap(os.path.join(d, "w"), np.uint16, "w+", shape=(max(w16.size, 1),))[
                :w16.size] = w16
            np.memmap(os.path.join(d, "codes"), np.uint8, "w+", shape=(max(w16.size, 1),))
            for name, t in _FIELDS:
                np.memmap(os.path.join(d, name), t, "w+", shape=(max(ng, 1),))
            parts = parts or 4 * self.procs
            edges = np.linspace(0, ng, min(parts, max(ng, 1)) + 1).astype(np.int64)
            params = dict(p=p, beta=beta, kappa=kappa, iters=iters, early_stop=early_stop)
            tasks = [(d, ng, g, nbits, params, int(a), int(b))
                     for a, b in zip(edges[:-1], edges[1:]) if b > a]
            self._run(tasks)
            out = {"codes": np.array(np.memmap(os.path.join(d, "codes"), np.uint8, "r",
                                               shape=(max(w16.size, 1),))[:w16.size])}
            for name, t in _FIELDS:
                out[name] = np.array(np.memmap(os.path.join(d, name), t, "r",
                                               shape=(max(ng, 1),))[:ng])
        finally:
            shutil.rmtree(d, ignore_errors=True)
        out["evals_needed"] = np.where(out["stopped"] == 1, out["passes"],
                                       out["last_change"].astype(np.int32) + 1).astype(np.uint8)
        return out


def _worker_main():
    for line in sys.stdin:
        try:
            _solve_range(json.loads(line))
            print("@@ok", flush=True)
        except Exception as e:  # reported to the parent, which raises
            print(f"@@error {type(e).__name__}: {e}", flush=True)


if __name__ == "__main__":
    _worker_main()
