"""One plan shared by several host threads, each on its own HIP stream.

The plan is immutable after creation and may be shared between threads
(the C ABI's promise); stream objects are per thread. Four threads run
offline batches and stream pushes concurrently, each on its own torch
stream (default priority), and every output must equal, bit for bit, the
same call made alone beforehand."""

import sys
import threading

import numpy as np
import pytest

import logmel_synth as S

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests.libload import load_binding
    lm = load_binding()
    plan = lm.logmel_plan_create(0)
    return lm, plan, torch


def _batch(torch, t):
    """Thread t's ragged batch: 6 speech-like clips of 0.5 to 40 s."""
    rng = np.random.default_rng(500 + t)
    lens = rng.integers(8000, 640000, 6)
    return S.pack(lens, lambda i, v: S.speech_like(600 + 10 * t + i, int(lens[i]), "cuda", out=v),
                  "cuda")


def _stream_run(lm, plan, torch, streams_x, pushes, push_len):
    n = streams_x.shape[0]
    s = lm.logmel_stream_create(plan, n, push_len)
    got = []
    for c in range(pushes):
        new = streams_x[:, c * push_len:(c + 1) * push_len].contiguous().reshape(-1)
        o, f = lm.logmel_stream_push(s, new, [push_len] * n)
        got.append(o.clone())
    s.close()
    return torch.cat(got)


def test_threads_share_a_plan(env):
    lm, plan, torch = env
    n_threads, reps, pushes, push_len = 4, 4, 12, 1280
    say("threads: inputs and single-threaded references")
    inputs, ref_off, ref_str = [], [], []
    for t in range(n_threads):
        x, so = _batch(torch, t)
        sx = torch.stack([S.speech_like(900 + 40 * t + j, pushes * push_len, "cuda")
                          for j in range(32)])
        inputs.append((x, so, sx))
        out, _ = lm.log_mel(plan, x, so)
        ref_off.append(out.clone())
        ref_str.append(_stream_run(lm, plan, torch, sx, pushes, push_len))
    torch.cuda.synchronize()

    results = [None] * n_threads
    errors = []

    def work(t):
        try:
            hs = torch.cuda.Stream()
            x, so, sx = inputs[t]
            outs = []
            with torch.cuda.stream(hs):
                hs.wait_stream(torch.cuda.default_stream())
                for _ in range(reps):
                    out, _ = lm.log_mel(plan, x, so, stream=hs)
                    outs.append(out)
                    outs.append(_stream_run(lm, plan, torch, sx, pushes, push_len))
            hs.synchronize()
            results[t] = outs
        except Exception as e:  # reported in the main thread
            errors.append((t, repr(e)))

    say(f"threads: {n_threads} threads x {reps} offline calls and {reps} x {pushes} pushes")
    th = [threading.Thread(target=work, args=(t,)) for t in range(n_threads)]
    for h in th:
        h.start()
    for h in th:
        h.join(timeout=100)
    assert not any(h.is_alive() for h in th), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for t in range(n_threads):
        for r in range(reps):
            assert torch.equal(results[t][2 * r], ref_off[t]), (t, r, "offline")
            assert torch.equal(results[t][2 * r + 1], ref_str[t]), (t, r, "stream")
    say("threads: every output equals its single-threaded reference")
