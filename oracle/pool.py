"""Runs the oracle over many independent cases on all host cores.

TEST INFRASTRUCTURE ONLY (see the package docstring). This module adds no
arithmetic of its own: every job below only slices its inputs and calls
functions of oracle.rswa, one (sequence, head), query row or key set at a
time, exactly as a single-threaded loop would. It exists because checking
full-size workloads element by element (every (sequence, head) of a 40-page
decode step, thousands of rows of a 32K pack, the gradients of reference keys
that every later row sees) takes minutes on one core.

Workers are fresh interpreters (multiprocessing "spawn"): they import numpy,
this package and the input generator only, never the GPU library, and each
runs BLAS on one thread. Large inputs travel once through POSIX shared memory
(`SharedArrays`), not per task.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time
import weakref
from multiprocessing import shared_memory

import numpy as np

from . import rswa as orc

_SHARED: dict = {}
_SEGMENTS: list = []
_RETIRED: list = []
_LIMITS = None


def workers() -> int:
    """Host cores this process may use, at most 16 (one GPU's share of the host's cores)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


class SharedArrays:
    """Named numpy arrays in POSIX shared memory, visible to the pool's workers.

    `new(name, shape, dtype)` returns a writable array the caller fills;
    `put(name, array)` copies an existing one. Close with `release()` (or use
    as a context manager)."""

    def __init__(self):
        self._segs = {}
        self.specs = {}

    def new(self, name: str, shape, dtype) -> np.ndarray:
        dtype = np.dtype(dtype)
        nbytes = max(1, int(np.prod(shape)) * dtype.itemsize)
        seg = shared_memory.SharedMemory(create=True, size=nbytes)
        self.specs[name] = (seg.name, tuple(int(s) for s in shape), dtype.str)
        a = np.ndarray(shape, dtype=dtype, buffer=seg.buf)
        self._segs[name] = (seg, weakref.ref(a))   # views of `a` keep it alive
        return a

    def put(self, name: str, a: np.ndarray) -> np.ndarray:
        view = self.new(name, a.shape, a.dtype)
        view[...] = a
        return view

    def release(self):
        """Removes the segments' names and unmaps them; a segment the caller still
        holds a view of stays mapped (until a later release finds it unused)."""
        global _RETIRED
        for seg, ref in self._segs.values():
            seg.unlink()
            _RETIRED.append((seg, ref))
        keep = []
        for seg, ref in _RETIRED:
            if ref() is None:
                seg.close()
            else:
                keep.append((seg, ref))
        _RETIRED = keep
        self._segs.clear()
        self.specs.clear()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.release()


def _init(specs):
    global _LIMITS
    try:
        from threadpoolctl import threadpool_limits
        _LIMITS = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        pass
    for name, (seg_name, shape, dtype) in (specs or {}).items():
        seg = shared_memory.SharedMemory(name=seg_name)
        _SEGMENTS.append(seg)
        _SHARED[name] = np.ndarray(shape, dtype=np.dtype(dtype), buffer=seg.buf)


def shared(name: str) -> np.ndarray:
    """A shared array inside a worker (read-only by convention)."""
    return _SHARED[name]


class OraclePool:
    """A spawn-context process pool whose workers see `arrays` (BLAS on one
    thread each). Use as a context manager; `map` keeps the task order."""

    def __init__(self, arrays: SharedArrays | None = None, processes: int | None = None):
        self.processes = processes or workers()
        self._pool = mp.get_context("spawn").Pool(
            self.processes, initializer=_init, initargs=(arrays.specs if arrays else None,))

    def map(self, fn, tasks, progress: str | None = None, task_timeout: float = 900.0):
        """[fn(t) for t in tasks]. Raises TimeoutError if any result is more than
        task_timeout seconds in coming (a worker that died, e.g. in its start-up,
        is replaced by the pool and its task would otherwise never return). With
        `progress`, prints a line (flushed) as every tenth of the tasks completes,
        so a long oracle run shows it is alive."""
        tasks = list(tasks)
        out, t0, mark = [], time.perf_counter(), 1
        it = self._pool.imap(fn, tasks, chunksize=1)
        for _ in range(len(tasks)):
            out.append(it.next(task_timeout))
            if progress is not None and len(out) * 10 >= mark * len(tasks):
                print(f"[oracle] {progress}: {len(out)}/{len(tasks)} tasks, "
                      f"{time.perf_counter() - t0:.0f} s", flush=True)
                while len(out) * 10 >= mark * len(tasks):
                    mark += 1
        return out

    def close(self):
        self._pool.close()
        self._pool.join()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        if exc[0] is not None:
            self._pool.terminate()   # a failed map: do not wait on workers still busy
        else:
            self.close()


def pool_map(fn, tasks, arrays: SharedArrays | None = None, processes: int | None = None,
             progress: str | None = None):
    """[fn(t) for t in tasks] on a fresh OraclePool, order kept."""
    tasks = list(tasks)
    if not tasks:
        return []
    with OraclePool(arrays, min(processes or workers(), len(tasks))) as pool:
        return pool.map(fn, tasks, progress)


def ready(_=None):
    """A no-op job: mapping it over the workers waits until every one has started."""
    return os.getpid()


# ----------------------------------------------------------------------- jobs
def _f64(a, dtype):
    import workloads as wl
    return wl.to_f64(a, dtype)


def decode_sequence_job(task):
    """Decode outputs of one sequence at several steps, every listed head.

    task = (dtype, L_m, n, scale, b, heads, steps) with steps a list of T.
    Shared arrays: "kref", "vref" [B][H][L_m][d] and "q", "k", "v"
    [S][B][H][d] holding outputs 1..S (storage form). Returns {T: [len(heads)][d]}."""
    dtype, L_m, n, scale, b, heads, steps = task
    kref, vref = shared("kref"), shared("vref")
    qs, ks, vs = shared("q"), shared("k"), shared("v")
    res = {}
    for T in steps:
        first = max(1, T - n + 1)
        rows = []
        for h in heads:
            rows.append(orc.decode_output(
                _f64(qs[T - 1, b, h], dtype), _f64(kref[b, h], dtype), _f64(vref[b, h], dtype),
                _f64(ks[first - 1:T, b, h], dtype), _f64(vs[first - 1:T, b, h], dtype),
                first, L_m, n, T, scale))
        res[T] = np.asarray(rows)
    return res


def masked_rows_job(task):
    """Packed-forward oracle rows: task = (rows, L_m, n, scale, prefix_mode).
    Shared arrays "Q", "K", "V" [N][H][d] with exact values (float32 or float64)."""
    rows, L_m, n, scale, mode = task
    return orc.masked_attention_rows(shared("Q"), shared("K"), shared("V"), rows, L_m, n, scale, mode)


def masked_bwd_keys_job(task):
    """Gradients of selected keys from a run of query rows.

    task = (rows, keys, heads, L_m, n, scale, prefix_mode). Shared arrays "Q",
    "K", "V", "dO" [N][H][d] (exact values). Runs the oracle's backward over the
    listed heads with the contributions of `rows` only, and returns
    (dK[keys], dV[keys]) of shape [len(keys)][len(heads)][d]; summing the
    results of runs that partition every row that sees the keys gives their
    full gradients."""
    rows, keys, heads, L_m, n, scale, mode = task
    hs = list(heads)
    Q, K, V, G = (np.asarray(shared(x)[:, hs], np.float64) for x in ("Q", "K", "V", "dO"))
    _, dK, dV = orc.masked_attention_backward(Q, K, V, G, L_m, n, scale, mode, rows=rows)
    return dK[list(keys)], dV[list(keys)]
