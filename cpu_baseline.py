"""CPU baseline leg of bench.py: the oracle, as it stands, timed on the host.

The oracle (numpy float64) quantizes and packs a bounded sample of the
workload -- every (KV head, K|V) plane of the first `layers` layers -- and runs
one decode step of attention over those layers, in a pool of worker
processes, one plane or KV head per task.  bench.py scales the measured time
to the full step (all layers, all decode steps) and says so.
"""
from __future__ import annotations

import math
import multiprocessing as mp
import os
import time

import numpy as np


def _quantize_plane(args):
    import oracle as O
    rows, perm, k, Lh, Ll = args
    rh = rows[perm[:k]]
    rl = rows[perm[k:]]
    ch, sh, mh = O.quantize_rows(rh, Lh)
    cl, sl, ml = O.quantize_rows(rl, Ll)
    return (O.pack_rows(ch, Lh), O.fp16_bits(sh), O.fp16_bits(mh),
            O.pack_rows(cl, Ll), O.fp16_bits(sl), O.fp16_bits(ml))


def _decode_head(args):
    import oracle as O
    q, packed, Lh, Ll, sm = args          # q [group][128]; packed: K and V planes
    (kh, ksh, kmh, kl, ksl, kml), (vh, vsh, vmh, vl, vsl, vml) = packed
    def deq(codes, s, m, L):
        return O.dequantize_rows(O.unpack_rows(codes, L), s.view(np.float16), m.view(np.float16))
    keys = np.concatenate([deq(kh, ksh, kmh, Lh), deq(kl, ksl, kml, Ll)])
    vals = np.concatenate([deq(vh, vsh, vmh, Lh), deq(vl, vsl, vml, Ll)])
    return np.stack([O.attention(q[h].astype(np.float64), keys, vals, sm) for h in range(q.shape[0])])


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (or the platform string)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def available_cores():
    """CPU cores this process may run on (its affinity set)."""
    return len(os.sched_getaffinity(0))


def time_oracle(K, V, perm, k, Lh, Ll, q, sm, workers=None):
    """K, V fp16 [layers_s][kv][n][128] (the sample); perm int32 [n]; q fp16
    [layers_s][Hq][128].  Returns (quantize seconds, decode seconds, workers).

    One single-threaded worker process per core, at most 16 (one GPU's share
    of the host), so that `workers` is the number of threads that run."""
    workers = workers or min(16, available_cores())
    ls, kv = K.shape[0], K.shape[1]
    group = q.shape[1] // kv
    threads_env = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {v: os.environ.get(v) for v in threads_env}
    for v in threads_env:
        os.environ[v] = "1"                        # inherited by the spawned workers
    ctx = mp.get_context("spawn")
    try:
        return _time_in_pool(ctx, workers, K, V, perm, k, Lh, Ll, q, sm, ls, kv, group)
    finally:
        for v, old in saved.items():
            if old is None:
                os.environ.pop(v, None)
            else:
                os.environ[v] = old


def _time_in_pool(ctx, workers, K, V, perm, k, Lh, Ll, q, sm, ls, kv, group):
    with ctx.Pool(workers) as pool:
        pool.map(math.sqrt, range(workers))          # start the workers before timing
        tasks = [(np.ascontiguousarray(X[l, g]), perm, k, Lh, Ll)
                 for l in range(ls) for g in range(kv) for X in (K, V)]
        t0 = time.perf_counter()
        planes = pool.map(_quantize_plane, tasks, chunksize=1)
        tq = time.perf_counter() - t0
        dtasks = []
        for l in range(ls):
            for g in range(kv):
                i = (l * kv + g) * 2
                dtasks.append((q[l, g * group:(g + 1) * group], (planes[i], planes[i + 1]),
                               Lh, Ll, sm))
        t0 = time.perf_counter()
        pool.map(_decode_head, dtasks, chunksize=1)
        td = time.perf_counter() - t0
    return tq, td, workers
