"""logmel_stream_push_static, the push for callers that cannot allocate:
through the C ABI, on two pushes in a row (the second smaller), its frames
equal a stream object's (logmel_stream_push) bit for bit, and the oracle's
frames of the concatenated streams within the parity rule; reset starts the
streams afresh; sizes beyond the stated limits are refused on the host."""

import sys

import numpy as np
import pytest

import oracle as O
import logmel_synth as S
from tests.parity import assert_parity

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


def _rows_cap(pl):
    return int(sum(-(-int(p) // 160) for p in pl))


def test_static_push_equals_stream_object(env):
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    n1, p1 = 64, 1280          # first push: 64 streams of 1280 samples
    n2, p2 = 40, 700           # second push: 40 streams of 700 samples
    N = p1 + p2
    streams = torch.stack([S.speech_like(500 + j, N, dev) for j in range(n1)])
    say("static push 1: 64 streams x 1280 (reset)")
    pl1 = np.full(n1, p1, dtype=np.int64)
    new1 = streams[:, :p1].contiguous().reshape(-1)
    out_s1 = torch.full((_rows_cap(pl1), 128), float("nan"), device=dev)
    fo_s1 = lm.logmel_stream_push_static(plan, new1, pl1, out_s1, reset=True)
    say("static push 2: 40 streams x 700")
    pl2 = np.full(n2, p2, dtype=np.int64)
    new2 = streams[:n2, p1:].contiguous().reshape(-1)
    out_s2 = torch.full((_rows_cap(pl2), 128), float("nan"), device=dev)
    fo_s2 = lm.logmel_stream_push_static(plan, new2, pl2, out_s2)
    torch.cuda.synchronize()

    say("stream object: the same two pushes")
    s = lm.logmel_stream_create(plan, n1, p1)
    out_o1, fo_o1 = lm.logmel_stream_push(s, new1, pl1)
    pl2o = np.zeros(n1, dtype=np.int64)
    pl2o[:n2] = p2
    out_o2, fo_o2 = lm.logmel_stream_push(s, new2, pl2o)
    torch.cuda.synchronize()
    s.close()

    assert np.array_equal(fo_s1, fo_o1)
    assert np.array_equal(fo_s2, fo_o2[:n2 + 1])
    assert fo_s1[-1] == n1 * 6 and fo_s2[-1] == n2 * 4
    assert torch.equal(out_s1[:int(fo_s1[-1])], out_o1)
    assert torch.equal(out_s2[:int(fo_s2[-1])], out_o2[:int(fo_o2[n2])])
    # rows past the push's frames are untouched
    assert torch.isnan(out_s2[int(fo_s2[-1]):]).all()

    say("oracle: the first 40 streams' 1980 samples")
    xs = streams[:n2].cpu().numpy()
    got = np.concatenate([
        np.concatenate([out_s1[fo_s1[j]:fo_s1[j + 1]].cpu().numpy(),
                        out_s2[fo_s2[j]:fo_s2[j + 1]].cpu().numpy()]) for j in range(n2)])
    Ls, Es = [], []
    for j in range(n2):
        L, E = O.logmel_clip(xs[j])
        Ls.append(L)
        Es.append(E)
    assert got.shape[0] == n2 * O.num_frames(N)
    assert_parity(got, np.concatenate(Ls), np.concatenate(Es), "static streams")


def test_static_push_reset_and_limits(env):
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    x = torch.stack([S.speech_like(900 + j, 2 * 2560, dev) for j in range(3)])
    pl = np.full(3, 2560, dtype=np.int64)
    out = torch.empty((3 * 16, 128), device=dev)
    say("static reset: 3 streams, 2 pushes of 2560, then a reset push")
    lm.logmel_stream_push_static(plan, x[:, :2560].contiguous().reshape(-1), pl, out, reset=True)
    lm.logmel_stream_push_static(plan, x[:, 2560:].contiguous().reshape(-1), pl, out)
    fo = lm.logmel_stream_push_static(plan, x[:, :2560].contiguous().reshape(-1), pl, out,
                                      reset=True)
    torch.cuda.synchronize()
    # after the reset the streams hold only this push: 14 frames each
    assert np.array_equal(fo, np.arange(4) * 14)
    ref, _ = lm.log_mel(plan, x[:, :2560].contiguous().reshape(-1), np.arange(4) * 2560)
    assert torch.equal(out[:42], ref)
    say("static limits (host checks only)")
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_stream_push_static(plan, torch.zeros(2561, device=dev),
                                     np.array([2561]), out)
    assert e.value.status == lm.LOGMEL_ERR_INPUT_TOO_LONG
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_stream_push_static(plan, torch.zeros(513, device=dev),
                                     np.ones(513, dtype=np.int64), out)
    assert e.value.status == lm.LOGMEL_ERR_INPUT_TOO_LONG
    small = torch.empty((1, 128), device=dev)
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_stream_push_static(plan, torch.zeros(800, device=dev), np.array([800]), small,
                                     reset=True)
    assert e.value.status == lm.LOGMEL_ERR_INVALID_ARGUMENT
