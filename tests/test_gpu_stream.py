"""Streaming push: frames emitted over all pushes equal the offline frames of
the concatenated stream, bit for bit; snapshot and restore; counters."""

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


def offline(env, streams):
    """Offline frames of each row of streams [n, N] (torch, cuda)."""
    lm, plan, torch = env
    n, N = streams.shape
    so = np.arange(n + 1, dtype=np.int64) * N
    out, fo = lm.log_mel(plan, streams.reshape(-1).contiguous(), so)
    return out, fo


def run_pushes(env, s, streams, schedule, collect):
    """schedule: list of push-length arrays; collect[j] gets stream j's rows."""
    lm, plan, torch = env
    n = streams.shape[0]
    pos = np.zeros(n, dtype=np.int64)
    for pl in schedule:
        pl = np.asarray(pl, dtype=np.int64)
        chunks = [streams[j, pos[j]:pos[j] + pl[j]] for j in range(n)]
        new = torch.cat(chunks).contiguous()
        out, fo = lm.logmel_stream_push(s, new, pl)
        for j in range(n):
            if fo[j + 1] > fo[j]:
                collect[j].append(out[fo[j]:fo[j + 1]])
        pos += pl
    return pos


def test_config3_stream_equals_offline(env):
    """512 streams, 375 pushes of 1280 samples (80 ms): 6 frames on the
    first push, then 8; 2998 per stream; bitwise equal to offline."""
    lm, plan, torch = env
    say("config3 generate")
    streams = S.config3_streams(device="cuda")
    n = streams.shape[0]
    s = lm.logmel_stream_create(plan, n, 1280)
    first = lm.logmel_stream_frames_for_push(s, np.full(n, 1280))
    assert np.all(np.diff(first) == 6)
    say("config3 pushes")
    collect = [[] for _ in range(n)]
    new_all = streams.reshape(n, 375, 1280)
    fo_seen = []
    for c in range(375):
        new = new_all[:, c, :].contiguous().reshape(-1)
        out, fo = lm.logmel_stream_push(s, new, np.full(n, 1280))
        fo_seen.append(int(fo[1] - fo[0]))
        for j in range(n):
            collect[j].append(out[fo[j]:fo[j + 1]])
    assert fo_seen[0] == 6 and all(v == 8 for v in fo_seen[1:])
    streamed = torch.stack([torch.cat(collect[j]) for j in range(n)])
    torch.cuda.synchronize()
    assert streamed.shape == (n, 2998, 128)
    say("config3 offline")
    ref, fo = offline(env, streams)
    assert torch.equal(streamed.reshape(-1, 128), ref), "stream != offline"
    for j in (0, 511):
        assert lm.logmel_stream_counters(s, j) == (480000, 2998)
    # and the offline frames against the oracle on two streams
    x = streams[[0, 511]].cpu().numpy()
    for k, j in enumerate((0, 511)):
        L, E = O.logmel_clip(x[k])
        assert_parity(streamed[j].cpu().numpy(), L, E, f"config3 stream {j}")
    s.close()


def test_random_push_lengths(env):
    lm, plan, torch = env
    say("random push lengths")
    rng = np.random.default_rng(31)
    n, N = 13, 20000
    streams = torch.from_numpy(rng.uniform(-1, 1, (n, N)).astype(np.float32)).cuda()
    s = lm.logmel_stream_create(plan, n, 3000)
    collect = [[] for _ in range(n)]
    pos = np.zeros(n, dtype=np.int64)
    while np.any(pos < N):
        pl = np.minimum(rng.choice([0, 1, 7, 159, 160, 161, 399, 400, 1280, 3000], n), N - pos)
        chunks = [streams[j, pos[j]:pos[j] + pl[j]] for j in range(n)]
        out, fo = lm.logmel_stream_push(s, torch.cat(chunks).contiguous(), pl)
        for j in range(n):
            if fo[j + 1] > fo[j]:
                collect[j].append(out[fo[j]:fo[j + 1]])
        pos += pl
    ref, fo = offline(env, streams)
    got = torch.cat([torch.cat(c) for c in collect])
    assert torch.equal(got, ref)
    s.close()


def test_push_too_long_is_an_error(env):
    lm, plan, torch = env
    say("push too long")
    s = lm.logmel_stream_create(plan, 2, 100)
    new = torch.zeros(202, dtype=torch.float32, device="cuda")
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_stream_push(s, new, [101, 101])
    assert e.value.status == lm.LOGMEL_ERR_INPUT_TOO_LONG
    assert lm.logmel_stream_counters(s, 0) == (0, 0)
    s.close()


def test_snapshot_restore(env):
    """Snapshot after some pushes, destroy, restore into a new object and
    continue: identical to an uninterrupted run."""
    lm, plan, torch = env
    say("snapshot restore")
    rng = np.random.default_rng(32)
    n, N, P = 5, 16000, 1000
    streams = torch.from_numpy(rng.uniform(-1, 1, (n, N)).astype(np.float32)).cuda()
    sched = [np.full(n, P)] * (N // P)
    a = lm.logmel_stream_create(plan, n, P)
    ca = [[] for _ in range(n)]
    run_pushes(env, a, streams, sched, ca)
    b = lm.logmel_stream_create(plan, n, P)
    cb = [[] for _ in range(n)]
    half = len(sched) // 2 + 1
    run_pushes(env, b, streams[:, :half * P], sched[:half], cb)
    state = lm.logmel_stream_get_state(b)
    b.close()
    c = lm.logmel_stream_create(plan, n, P)
    lm.logmel_stream_set_state(c, state)
    assert lm.logmel_stream_counters(c, 0) == (half * P, O.num_frames(half * P))
    rest = streams[:, half * P:].contiguous()
    run_pushes(env, c, rest, sched[half:], cb)
    for j in range(n):
        assert torch.equal(torch.cat(ca[j]), torch.cat(cb[j]))
    a.close()
    c.close()


def test_reset(env):
    lm, plan, torch = env
    say("reset")
    n = 3
    rng = np.random.default_rng(33)
    x = torch.from_numpy(rng.uniform(-1, 1, (n, 4000)).astype(np.float32)).cuda()
    s = lm.logmel_stream_create(plan, n, 4000)
    o1, _ = lm.logmel_stream_push(s, x.reshape(-1).contiguous(), [4000] * n)
    lm.logmel_stream_reset(s)
    o2, _ = lm.logmel_stream_push(s, x.reshape(-1).contiguous(), [4000] * n)
    assert torch.equal(o1, o2)
    s.close()


@pytest.mark.parametrize("push,first,steady", [(1920, 10, 12), (2560, 14, 16)])
def test_other_clocks_equal_offline(env, push, first, steady):
    """The 120 and 160 ms audio clocks (1920- and 2560-sample pushes): the
    page-5 clocks other than 80 ms. 64 speech-like 30 s streams; the last
    push of the 160 ms clock is the 1280-sample remainder."""
    lm, plan, torch = env
    say(f"clock {push} samples: generate")
    streams = S.config3_streams(device="cuda", n_streams=64)
    n, N = streams.shape
    s = lm.logmel_stream_create(plan, n, push)
    collect = [[] for _ in range(n)]
    per_push = []
    pos = 0
    say(f"clock {push} samples: pushes")
    while pos < N:
        p = min(push, N - pos)
        new = streams[:, pos:pos + p].contiguous().reshape(-1)
        out, fo = lm.logmel_stream_push(s, new, np.full(n, p))
        per_push.append(int(fo[1] - fo[0]))
        for j in range(n):
            collect[j].append(out[fo[j]:fo[j + 1]])
        pos += p
    full = N // push
    assert per_push[0] == first and all(v == steady for v in per_push[1:full])
    assert sum(per_push) == 2998
    streamed = torch.stack([torch.cat(collect[j]) for j in range(n)])
    ref, fo = offline(env, streams)
    torch.cuda.synchronize()
    assert torch.equal(streamed.reshape(-1, 128), ref), "stream != offline"
    assert lm.logmel_stream_counters(s, 0) == (N, 2998)
    s.close()


def test_int16_and_fp16_streams_equal_offline(env):
    """int16 PCM pushes and fp16 output: the streamed frames equal the offline
    frames of the same samples and types bit for bit; a stream fed int16 and
    fp32 pushes of the same values in turn equals the fp32 offline result."""
    lm, plan, torch = env
    say("int16 / fp16 streams: 24 streams x 4 s, pushes of 1280 and ragged")
    dev = torch.device("cuda", 0)
    n, N = 24, 64000
    x = torch.stack([S.speech_like(700 + j, N, "cuda") for j in range(n)])
    s16 = torch.clamp(torch.round(x * 32768.0), -32768, 32767).to(torch.int16)
    x32 = s16.to(torch.float32) / 32768.0
    so = np.arange(n + 1, dtype=np.int64) * N
    fo = lm.logmel_frame_offsets(so)
    so_d = torch.from_numpy(so).to(dev)
    fo_d = torch.from_numpy(fo).to(dev)
    T = int(fo[-1])
    ref32 = lm.logmel_compute_ex(plan, x32.reshape(-1).contiguous(), so_d, fo_d, T)
    ref16 = lm.logmel_compute_ex(plan, x32.reshape(-1).contiguous(), so_d, fo_d, T,
                                 out_dtype=torch.float16)
    rng = np.random.default_rng(9)
    for case, (inp, odt, ref) in {"int16 in": (s16, torch.float32, ref32),
                                  "fp16 out": (x32, torch.float16, ref16),
                                  "int16 in, fp16 out": (s16, torch.float16, ref16),
                                  "int16 and fp32 pushes": (None, torch.float32, ref32)}.items():
        s = lm.logmel_stream_create(plan, n, 2000)
        got = [[] for _ in range(n)]
        pos = np.zeros(n, dtype=np.int64)
        k = 0
        while (pos < N).any():
            pl = np.minimum(rng.integers(0, 2001, n) if k % 3 == 2 else np.full(n, 1280), N - pos)
            src = inp if inp is not None else (s16 if k % 2 == 0 else x32)
            new = torch.cat([src[j, pos[j]:pos[j] + pl[j]] for j in range(n)]).contiguous()
            out, f = lm.logmel_stream_push(s, new, pl, out_dtype=odt)
            for j in range(n):
                if f[j + 1] > f[j]:
                    got[j].append(out[f[j]:f[j + 1]])
            pos += pl
            k += 1
        torch.cuda.synchronize()
        for j in range(n):
            g = torch.cat(got[j])
            assert g.dtype == odt
            assert torch.equal(g, ref[fo[j]:fo[j + 1]]), (case, j)
        s.close()
        say(f"{case}: equal to offline")


def test_stream_push_ex_rejects_types(env):
    lm, plan, torch = env
    s = lm.logmel_stream_create(plan, 2, 100)
    pl = np.array([0, 0], dtype=np.int64)
    assert lm._stream_push_ex(s.handle, None, 7, lm._ptr64(pl), None, lm.LOGMEL_F32, None,
                              None) == lm.LOGMEL_ERR_UNSUPPORTED
    assert lm._stream_push_ex(s.handle, None, lm.LOGMEL_F32, lm._ptr64(pl), None, 9, None,
                              None) == lm.LOGMEL_ERR_UNSUPPORTED
    s.close()


def resampled_streams_case(env, rate, n, seconds, seed, in_dtype="f32", out_dtype="f32",
                           uniform=False):
    """Streams at `rate`: ragged pushes around 80 ms, then a flush; each
    stream's frames equal, bit for bit, logmel_resample of the whole input
    followed by logmel_compute. With uniform, every stream is `seconds` long
    and every push is 80 ms (the last one shorter, the same for all), so
    the streams stay in one state and each push, the flush included, takes
    the records that follow from the prep kernel's arguments."""
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(seed)
    if uniform:
        lens = [int(seconds * rate) + 123] * n
    else:
        lens = [int(rng.integers(int(0.2 * rate), int(seconds * rate))) for _ in range(n)]
        lens[0] = 0
        lens[1] = 37
    clips = [S.speech_like(900 + j, max(L, 1), "cuda", fs=rate)[:L] for j, L in enumerate(lens)]
    if in_dtype == "i16":
        clips = [torch.clamp(torch.round(c * 32768.0), -32768, 32767).to(torch.int16) for c in clips]
    odt = torch.float16 if out_dtype == "f16" else torch.float32
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    packed = torch.cat(clips).contiguous() if sum(lens) else torch.zeros(0, device=dev)
    r = lm.logmel_resampler_create(plan, rate)
    y, oo = lm.resample(r, packed, so)
    fo = lm.logmel_frame_offsets(oo)
    ref = lm.logmel_compute_ex(plan, y, torch.from_numpy(oo).to(dev), torch.from_numpy(fo).to(dev),
                               int(fo[-1]), out_dtype=odt)
    push = rate * 80 // 1000
    s = lm.logmel_stream_create(plan, n, push + push // 2, in_rate=rate)
    got = [[] for _ in range(n)]
    pos = np.zeros(n, dtype=np.int64)
    k = 0
    while (pos < np.array(lens)).any():
        if uniform:
            pl = np.full(n, push)
        else:
            pl = np.full(n, push) if k % 3 else rng.integers(0, push + push // 2 + 1, n)
        pl = np.minimum(pl, np.array(lens) - pos)
        new = torch.cat([clips[j][pos[j]:pos[j] + pl[j]] for j in range(n)]).contiguous()
        fo_pred = lm.logmel_stream_frames_for_push(s, pl)
        out, f = lm.logmel_stream_push(s, new, pl, out_dtype=odt)
        assert np.array_equal(f, fo_pred)
        for j in range(n):
            if f[j + 1] > f[j]:
                got[j].append(out[f[j]:f[j + 1]])
        pos += pl
        k += 1
    out, f = lm.logmel_stream_flush(s, out_dtype=odt)
    for j in range(n):
        if f[j + 1] > f[j]:
            got[j].append(out[f[j]:f[j + 1]])
    torch.cuda.synchronize()
    for j in range(n):
        g = torch.cat(got[j]) if got[j] else torch.zeros((0, 128), dtype=odt, device=dev)
        assert g.shape[0] == fo[j + 1] - fo[j], (rate, j, g.shape[0], fo[j + 1] - fo[j])
        assert torch.equal(g, ref[fo[j]:fo[j + 1]]), (rate, j)
    # after the flush the streams start again from nothing
    assert lm.logmel_stream_counters(s, 2) == (0, 0)
    s.close()
    return k


# 96 kHz: super-periods staged with pad floats
@pytest.mark.parametrize("rate", [48000, 44100, 8000, 22050, 96000])
def test_resampling_streams_equal_offline(env, rate):
    say(f"resampling streams at {rate} Hz")
    pushes = resampled_streams_case(env, rate, 10, 3.0, rate)
    say(f"{rate} Hz: {pushes} pushes and a flush equal offline")


def test_resampling_streams_int16_fp16(env):
    say("resampling streams at 48 kHz, int16 in, fp16 out")
    resampled_streams_case(env, 48000, 6, 2.0, 5, in_dtype="i16", out_dtype="f16")


@pytest.mark.parametrize("rate,in_dtype,out_dtype", [(48000, "f32", "f32"), (44100, "f32", "f32"),
                                                     (8000, "f32", "f32"), (48000, "i16", "f16")])
def test_resampling_streams_uniform_pushes(env, rate, in_dtype, out_dtype):
    """Streams in one state pushing one length (a fixed audio clock): the
    prep kernel builds every record from its arguments, for the input
    segments, the resampler's segment arrays, the 16 kHz carries and the
    transform's offsets; the frames still equal offline resampling then
    log-mel bit for bit."""
    say(f"resampling streams at {rate} Hz, uniform pushes, {in_dtype} in, {out_dtype} out")
    pushes = resampled_streams_case(env, rate, 24, 1.5, 3, in_dtype=in_dtype,
                                    out_dtype=out_dtype, uniform=True)
    say(f"{rate} Hz uniform: {pushes} pushes and a flush equal offline")


def test_resampling_stream_limits(env):
    lm, plan, torch = env
    s = lm.logmel_stream_create(plan, 2, 1000, in_rate=48000)
    r = lm.logmel_resampler_create(plan, 48000)
    taps = lm.logmel_resampler_info(r)[1]
    r.close()
    # per stream: 6 int64, 400 carry words, 2J input carry words
    assert lm.logmel_stream_state_bytes(s) == 2 * (12 + 400 + (taps - 1)) * 4
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_stream_push(s, torch.zeros(2002, device="cuda"), [1001, 1001])
    assert e.value.status == lm.LOGMEL_ERR_INPUT_TOO_LONG
    s.close()
    with pytest.raises(lm.LogmelError):
        lm.logmel_stream_create(plan, 2, 1000, in_rate=44101)
    # a 16 kHz stream's flush emits nothing and resets it
    s = lm.logmel_stream_create(plan, 3, 1280)
    lm.logmel_stream_push(s, torch.zeros(3 * 1000, device="cuda"), [1000] * 3)
    out, f = lm.logmel_stream_flush(s)
    assert out.shape[0] == 0 and list(f) == [0, 0, 0, 0]
    assert lm.logmel_stream_counters(s, 0) == (0, 0)
    s.close()


def _resampling_pushes(rate, lens, seed):
    """A fixed schedule of ragged pushes around 80 ms covering every stream."""
    rng = np.random.default_rng(seed)
    push = rate * 80 // 1000
    pos = np.zeros(len(lens), dtype=np.int64)
    sched = []
    k = 0
    while (pos < np.array(lens)).any():
        pl = np.full(len(lens), push) if k % 3 else rng.integers(0, push + push // 2 + 1, len(lens))
        pl = np.minimum(pl, np.array(lens) - pos)
        sched.append(pl)
        pos += pl
        k += 1
    return sched, push + push // 2


def _run_resampling(lm, s, clips, sched, got, start):
    pos = start.copy()
    for pl in sched:
        new = torch_cat([clips[j][pos[j]:pos[j] + pl[j]] for j in range(len(clips))])
        out, f = lm.logmel_stream_push(s, new, pl)
        for j in range(len(clips)):
            if f[j + 1] > f[j]:
                got[j].append(out[f[j]:f[j + 1]])
        pos += pl
    return pos


def torch_cat(parts):
    import torch
    return torch.cat(parts).contiguous()


@pytest.mark.parametrize("rate", [48000, 44100])
def test_resampling_snapshot_restore(env, rate):
    """A stream at another input rate: snapshot after half its pushes,
    destroy, restore into a new object, continue and flush: bit for bit the
    uninterrupted run, and the offline resample-then-log-mel frames. A state
    whose counters disagree, or one of another rate, is refused."""
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    say(f"resampling stream snapshot/restore at {rate} Hz")
    rng = np.random.default_rng(rate + 7)
    n = 6
    lens = [int(rng.integers(rate, 3 * rate)) for _ in range(n)]
    clips = [S.speech_like(950 + j, L, "cuda", fs=rate) for j, L in enumerate(lens)]
    sched, max_push = _resampling_pushes(rate, lens, rate)
    half = len(sched) // 2 + 1

    def flush_into(s, got):
        out, f = lm.logmel_stream_flush(s)
        for j in range(n):
            if f[j + 1] > f[j]:
                got[j].append(out[f[j]:f[j + 1]])

    a = lm.logmel_stream_create(plan, n, max_push, in_rate=rate)
    ga = [[] for _ in range(n)]
    _run_resampling(lm, a, clips, sched, ga, np.zeros(n, dtype=np.int64))
    flush_into(a, ga)
    a.close()

    b = lm.logmel_stream_create(plan, n, max_push, in_rate=rate)
    gb = [[] for _ in range(n)]
    pos = _run_resampling(lm, b, clips, sched[:half], gb, np.zeros(n, dtype=np.int64))
    state = lm.logmel_stream_get_state(b)
    counters = [lm.logmel_stream_counters(b, j) for j in range(n)]
    b.close()
    c = lm.logmel_stream_create(plan, n, max_push, in_rate=rate)
    # a state whose input carry length disagrees with its counters is refused
    # and changes nothing (word 5 of stream 0's record)
    bad = bytearray(state)
    v = int.from_bytes(bad[40:48], "little", signed=True)
    bad[40:48] = (v + 1).to_bytes(8, "little", signed=True)
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_stream_set_state(c, bytes(bad))
    assert e.value.status == lm.LOGMEL_ERR_INVALID_ARGUMENT
    assert lm.logmel_stream_counters(c, 0) == (0, 0)
    lm.logmel_stream_set_state(c, state)
    assert [lm.logmel_stream_counters(c, j) for j in range(n)] == counters
    assert all(counters[j][0] == pos[j] for j in range(n))
    _run_resampling(lm, c, clips, sched[half:], gb, pos)
    flush_into(c, gb)
    c.close()
    torch.cuda.synchronize()

    packed = torch.cat(clips).contiguous()
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    r = lm.logmel_resampler_create(plan, rate)
    y, oo = lm.resample(r, packed, so)
    r.close()
    fo = lm.logmel_frame_offsets(oo)
    ref = lm.logmel_compute(plan, y, torch.from_numpy(oo).to(dev), torch.from_numpy(fo).to(dev),
                            int(fo[-1]))
    for j in range(n):
        ra, rb = torch.cat(ga[j]), torch.cat(gb[j])
        assert torch.equal(ra, rb), (rate, j)
        assert torch.equal(rb, ref[fo[j]:fo[j + 1]]), (rate, j)

    # another rate's state does not fit this stream
    other = lm.logmel_stream_create(plan, n, max_push, in_rate=22050 if rate != 22050 else 8000)
    with pytest.raises((ValueError, lm.LogmelError)):
        lm.logmel_stream_set_state(other, state)
    other.close()


def test_push_into_larger_buffer_and_slot_groups(env):
    """A push into a buffer with spare rows writes exactly its own rows (the
    rest stay untouched) and returns a view of them, equal bit for bit to the
    same push into a buffer of its size. Stream objects closed after 1 to 13
    pushes (inside and at the ends of the staging slots' groups of four)
    leave the next object's pushes intact, and every frame so far equals the
    offline frame of the stream's audio."""
    lm, plan, torch = env
    n, P, K = 6, 1280, 13
    streams = S.config3_streams(device="cuda", n_streams=n, n_samples=K * P)
    ref, fo_ref = offline(env, streams)
    torch.cuda.synchronize()
    for k in (1, 3, 4, 5, 8, 9, 13):
        say(f"slot groups: {k} pushes")
        s = lm.logmel_stream_create(plan, n, P)
        t = lm.logmel_stream_create(plan, n, P)
        big = torch.empty((n * 10, 128), dtype=torch.float32, device="cuda")
        got = [[] for _ in range(n)]
        for c in range(k):
            new = streams[:, c * P:(c + 1) * P].contiguous().reshape(-1)
            o1, f1 = lm.logmel_stream_push(s, new, [P] * n)
            big.fill_(float("nan"))
            o2, f2 = lm.logmel_stream_push(t, new, np.full(n, P), out=big)
            torch.cuda.synchronize()
            total = int(f1[-1])
            assert np.array_equal(f1, f2)
            assert tuple(o2.shape) == (total, 128) and o2.data_ptr() == big.data_ptr()
            assert torch.equal(o1, o2), (k, c)
            assert bool(torch.isnan(big[total:]).all()), (k, c)
            for j in range(n):
                got[j].append(o1[f1[j]:f1[j + 1]].clone())
        with pytest.raises(ValueError):
            lm.logmel_stream_push(t, streams[:, :P].contiguous().reshape(-1), [P] * n,
                                  out=big[:4])
        with pytest.raises(ValueError):
            lm.logmel_stream_push(t, streams[:, :P].contiguous().reshape(-1), [P] * (n - 1) + [P, 0])
        s.close()
        t.close()
        for j in range(n):
            m = sum(int(x.shape[0]) for x in got[j])
            assert m == lm.logmel_num_frames(k * P)
            assert torch.equal(torch.cat(got[j]), ref[fo_ref[j]:fo_ref[j] + m]), (k, j)
