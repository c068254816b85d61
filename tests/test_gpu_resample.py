"""Resampling to 16 kHz on the GPU against the fp64 oracle.

The kernel forms each output as an fp32 dot product of its T taps
(T = 2 ceil(H) + 1) with fp32 taps, accumulated on the matrix cores four
products per step in fp32 (the other products of a step have zero taps and
add exactly nothing); the standard bound for such a sum is
|y - y_exact| <= (T + 2) u sum_k |x_k h_k| with u = 2^-24 (taps rounded
once, each product and each addition of a nonzero term rounded at most
once). The test allows (T + 4) u a[n], a[n] being the oracle's sum of
|x_k h_k|.
int16 input must give the fp32 result of s / 32768 bit for bit, 16 kHz input
must come back unchanged, and the resampled batch must feed the log-mel path
(checked against the oracle's log-mel of the same buffer)."""

import sys

import numpy as np
import pytest

import oracle as O
import logmel_synth as S
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
RATES = [4800, 8000, 9600, 11025, 12000, 22050, 24000, 32000, 44100, 48000, 88200, 96000, 176400,
         192000]


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


def batch_at(rate, seed):
    """Ragged clips at ``rate``: speech-like clips made at that rate plus a
    tone above 8 kHz (where the rate allows one) and light noise; clips of
    0, 1, 2 and a few samples, shorter than the kernel, and up to 1.5 s."""
    rng = np.random.default_rng(seed)
    lens = [0, 1, 2, 5, 37, 0] + list(rng.integers(0, rate // 20, 6)) + \
        list(rng.integers(rate // 4, 3 * rate // 2, 5))
    rng.shuffle(lens)
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = np.zeros(int(so[-1]), dtype=np.float64)
    for i, n in enumerate(lens):
        if n == 0:
            continue
        v = S.speech_like(300 + i, int(n), fs=rate).numpy().astype(np.float64)
        k = np.arange(n)
        if rate > 20000:
            v += 0.2 * np.sin(2 * np.pi * 0.45 * rate * k / rate + i)
        v += 0.01 * rng.standard_normal(n)
        x[so[i]:so[i + 1]] = 0.8 * v / max(1.0, np.abs(v).max())
    return x.astype(np.float32), so


def check(y_gpu, y_ref, a_ref, T, what):
    bound = (T + 4) * U * a_ref + 1e-30
    err = np.abs(np.asarray(y_gpu, dtype=np.float64) - y_ref)
    bad = err > bound
    ratio = float(np.max(err / bound)) if err.size else 0.0
    say(f"{what}: {err.size} outputs, max |err| {err.max(initial=0):.3g}, "
        f"max err/bound {ratio:.3f}, over bound {int(bad.sum())}")
    assert not bad.any(), what


@pytest.mark.parametrize("rate", RATES)
def test_resample_parity(env, rate):
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    x, so = batch_at(rate, rate)
    say(f"resample {rate} Hz: {len(so) - 1} clips, {int(so[-1])} samples")
    r = lm.logmel_resampler_create(plan, rate)
    L, T = lm.logmel_resampler_info(r)
    y, oo = lm.resample(r, torch.from_numpy(x).to(dev), so)
    torch.cuda.synchronize()
    y_ref, oo_ref, a_ref = O.resample_packed(x, so, rate)
    assert np.array_equal(oo, oo_ref)
    assert T == 2 * int(np.ceil(O.resample_halfwidth(rate))) + 1
    check(y.cpu().numpy(), y_ref, a_ref, T, f"{rate} Hz (L {L}, T {T})")


def test_resample_16k_is_identity_and_int16_bitwise(env):
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    say("16 kHz identity; int16 == fp32 at 44.1, 48, 11.025, 9.6, 176.4 and 32 kHz")
    x, so = batch_at(16000, 7)
    r = lm.logmel_resampler_create(plan, 16000)
    y, oo = lm.resample(r, torch.from_numpy(x).to(dev), so)
    torch.cuda.synchronize()
    assert np.array_equal(oo, so)
    assert np.array_equal(y.cpu().numpy(), x)
    # every staging form and workgroup shape the kernel picks: 44.1 and 11.025 kHz
    # wide staging, 8 wavefronts; 48 kHz narrow, 4; 9.6 kHz narrow, 8; 176.4 kHz
    # wide, one row block per item; 32 kHz super-periods padded with zeros
    for rate in (44100, 48000, 11025, 9600, 176400, 32000):
        x, so = batch_at(rate, rate + 1)
        s16 = np.clip(np.round(x.astype(np.float64) * 32768), -32768, 32767).astype(np.int16)
        x32 = s16.astype(np.float32) / np.float32(32768.0)
        r = lm.logmel_resampler_create(plan, rate)
        y16, _ = lm.resample(r, torch.from_numpy(s16).to(dev), so)
        y32, _ = lm.resample(r, torch.from_numpy(x32).to(dev), so)
        torch.cuda.synchronize()
        assert torch.equal(y16, y32), rate
        y_ref, _, a_ref = O.resample_packed(x32, so, rate)
        check(y16.cpu().numpy(), y_ref, a_ref, lm.logmel_resampler_info(r)[1], f"int16 {rate} Hz")


def test_resampled_batch_feeds_log_mel(env):
    """44.1 kHz clips -> 16 kHz -> log-mel: the log-mel of the GPU's
    resampled buffer matches the oracle's log-mel of that same buffer."""
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    say("44.1 kHz -> 16 kHz -> log-mel")
    x, so = batch_at(44100, 9)
    r = lm.logmel_resampler_create(plan, 44100)
    y, oo = lm.resample(r, torch.from_numpy(x).to(dev), so)
    L, fo = lm.log_mel(plan, y, oo)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    Lr, Er, fo_ref = O.logmel_packed(yh, oo)
    assert np.array_equal(fo, fo_ref)
    rep = assert_parity(L.cpu().numpy(), Lr, Er, "log-mel of the resampled batch")
    say(f"log-mel of the resampled batch: {rep}")


def test_resample_full_size_sampled(env):
    """The benchmark's batch: 64 clips x 30 s at 44.1 kHz (84.7 M samples),
    resampled in one launch; 4096 outputs spread over the batch against
    the oracle, computed one by one."""
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    say("64 x 30 s at 44.1 kHz, sampled outputs")
    x, so = S.config2_at(44100, device=dev)
    r = lm.logmel_resampler_create(plan, 44100)
    y, oo = lm.resample(r, x, so)
    torch.cuda.synchronize()
    assert int(oo[-1]) == 64 * 480000
    rng = np.random.default_rng(12)
    rows = np.sort(np.concatenate([rng.integers(0, int(oo[-1]), 4000),
                                   oo[:-1], oo[1:] - 1, oo[1:-1] + 3]))
    xh = x.cpu().numpy()
    y_ref, a_ref = O.resample_selected(xh, so, 44100, rows)
    check(y.cpu().numpy()[rows], y_ref, a_ref, lm.logmel_resampler_info(r)[1],
          "64 x 30 s at 44.1 kHz (sampled)")



def test_resample_past_2_31_input_samples(env):
    """30 speech-like clips of 75,000,017 samples at 44.1 kHz (28 minutes
    each, 2,250,000,510 samples: input positions pass 2**31), resampled in
    one launch; outputs at the clips' edges, around input sample 2**31 and
    3000 random ones against the oracle, computed one by one."""
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    n = 75_000_017
    say("30 x 75e6 samples at 44.1 kHz (past 2**31), sampled outputs")
    x, so = S.pack([n] * 30, lambda i, v: S.speech_like(700 + i, n, dev, out=v, fs=44100), dev)
    assert int(so[-1]) > 2**31
    r = lm.logmel_resampler_create(plan, 44100)
    y, oo = lm.resample(r, x, so)
    torch.cuda.synchronize()
    c = int(np.searchsorted(so, 2**31, side="right")) - 1
    m = int(oo[c]) + ((2**31 - int(so[c])) * 16000) // 44100     # output at input 2**31
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([rng.integers(0, int(oo[-1]), 3000),
                                     oo[:-1], oo[1:] - 1, np.arange(m - 40, m + 40)]))
    xh = x.cpu().numpy()
    del x
    torch.cuda.empty_cache()
    y_ref, a_ref = O.resample_selected(xh, so, 44100, rows)
    check(y.cpu().numpy()[rows], y_ref, a_ref, lm.logmel_resampler_info(r)[1],
          "30 x 75e6 samples at 44.1 kHz (sampled)")
    del y
    torch.cuda.empty_cache()

def test_resample_validate_empty_and_unsupported(env, monkeypatch):
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    say("resample: validate mode, empty calls, unsupported rates")
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_resampler_create(plan, 44101)     # 16000 phases: table beyond LDS
    assert e.value.status == lm.LOGMEL_ERR_UNSUPPORTED
    with pytest.raises(lm.LogmelError):
        lm.logmel_resampler_create(plan, 999)
    r = lm.logmel_resampler_create(plan, 48000)
    x = torch.zeros(4800, dtype=torch.float32, device=dev)
    so = torch.tensor([0, 4800], dtype=torch.int64, device=dev)
    bad = torch.tensor([0, 1601], dtype=torch.int64, device=dev)
    monkeypatch.setenv("LOGMEL_VALIDATE", "1")
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_resample(r, x, so, bad, 1601)
    assert e.value.status == lm.LOGMEL_ERR_INVALID_ARGUMENT
    good = torch.tensor([0, 1600], dtype=torch.int64, device=dev)
    y = lm.logmel_resample(r, x, so, good, 1600)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
    monkeypatch.delenv("LOGMEL_VALIDATE")
    empty = torch.empty(0, dtype=torch.float32, device=dev)
    z = torch.tensor([0], dtype=torch.int64, device=dev)
    assert lm.logmel_resample(r, empty, z, z, 0).numel() == 0
    zz = torch.tensor([0, 0, 0], dtype=torch.int64, device=dev)
    assert lm.logmel_resample(r, empty, zz, zz, 0).numel() == 0
