"""Oracle references for the full-size parity tests, computed in worker
processes that start when the session collects those tests, so that the
oracle's minutes of CPU work overlap the other GPU tests.

Each job is a plain call of the oracle on one workload item (or, for the
encoder item, one of its frame windows widened by the stack's reach, whose
interior equals the full encode: pinned bitwise in test_oracle_pins.py).
Workers import only numpy, the oracle and the seeded input generators; they
never touch the GPU.
"""

from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import time

HOP = 800
C3 = (2, 1200)                # B, N latents
C4 = (2, 256, 30000)          # stage-1 AMP set input
E3 = (2, 960000, 7)           # B, samples, waveform seed
E3_WINDOWS = ((0, 300), (300, 600), (600, 900), (900, 1200))  # frames of item 0


def _limit_threads(n):
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(n)
    except Exception:
        pass


def c3_item(item):
    import oracle as O
    from neural_audio_vae_amd import synth
    t = time.time()
    z = synth.make_latents(*C3)
    y = O.decode_item(synth.make_params(), z[item], clamp=False)
    return y, time.time() - t


def c4_item(item):
    import oracle as O
    from neural_audio_vae_amd import synth
    t = time.time()
    x = synth.make_signal(C4, seed=0)
    y = O.stage_amp(x[item], synth.make_params(), 1)
    return y, time.time() - t


def e3_window(k):
    import oracle as O
    from neural_audio_vae_amd import synth
    from tests.conftest import encoder_margin_frames
    t = time.time()
    batch, samples, seed = E3
    frames = samples // HOP
    wave = synth.make_waveform(batch, samples, seed=seed)
    f0, f1 = E3_WINDOWS[k]
    m = encoder_margin_frames(O.DEFAULT_CONFIG["encoder_rates"])
    w0, w1 = max(0, f0 - m), min(frames, f1 + m)
    h = O.encode_hidden(synth.make_encoder_params(seed=0), wave[0:1, :, w0 * HOP:w1 * HOP])
    return h[0, :, f0 - w0:f1 - w0], time.time() - t


JOBS = {
    **{f"c4/{i}": (c4_item, i) for i in range(C4[0])},
    **{f"c3/{i}": (c3_item, i) for i in range(C3[0])},
    **{f"e3/0/{k}": (e3_window, k) for k in range(len(E3_WINDOWS))},
}


class Pool:
    """The session's oracle workers and their pending results."""

    def __init__(self, names):
        cores = min(16, len(os.sched_getaffinity(0)))
        workers = max(1, min(4, cores // 2, len(names)))
        self.ex = cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                                         initializer=_limit_threads, initargs=(max(1, cores // workers),))
        self.futures = {n: self.ex.submit(JOBS[n][0], JOBS[n][1]) for n in names}
        self.t0 = time.time()

    def result(self, name, timeout=900):
        y, dt = self.futures[name].result(timeout=timeout)
        print(f"[oracle] {name}: {dt:.1f} s of oracle time, ready {time.time() - self.t0:.0f} s after the "
              "session started", flush=True)
        return y

    def close(self):
        for f in self.futures.values():
            f.cancel()
        procs = list(getattr(self.ex, "_processes", {}).values())
        self.ex.shutdown(wait=False, cancel_futures=True)
        for p in procs:
            if p.is_alive():
                p.terminate()
