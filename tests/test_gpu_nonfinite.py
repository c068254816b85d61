"""Non-finite input. A NaN sample makes NaN exactly the frames whose 400
samples hold it, in all 128 bands (the oracle's sums, empty filters'
included, are NaN there), offline and streamed; every other frame keeps the
parity rule. The resampler's NaN reach is bounded by its stated geometry.
Offsets that overstate the resampler's output write nothing past it."""

import math
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


def _check_nan_rows(got, L_ref, E_ref, what):
    """Rows the oracle gives NaN are NaN in every band on the GPU; the other
    rows hold the parity rule (and so have no NaN)."""
    bad = np.isnan(L_ref).any(axis=1)
    assert np.isnan(L_ref[bad]).all(), what
    assert np.isnan(got[bad]).all(), f"{what}: NaN rows not all NaN"
    assert_parity(got[~bad], L_ref[~bad], E_ref[~bad], what)
    return int(bad.sum())


# clip lengths: a 30 s clip (tiles inside one clip), short and 1-frame clips
# (tiles across clips, staged as pieces), 12 clips of 450 samples in a row
# (more than 8 pieces in a tile: per-lane gathers), a 5 s clip
LENS = [480000, 2000, 600] + [450] * 12 + [80000]
# (clip, sample index in the clip) of each NaN
NANS = [(0, 100000), (0, 479999), (1, 700), (2, 0), (5, 449), (8, 200), (15, 79999)]


def _batch(torch, dev):
    so = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int64)
    x = torch.empty(int(so[-1]), dtype=torch.float32, device=dev)
    for i, n in enumerate(LENS):
        x[so[i]:so[i + 1]] = S.speech_like(700 + i, n, dev)
    for c, k in NANS:
        x[so[c] + k] = float("nan")
    return x, so


def test_nan_offline_frames(env):
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    x, so = _batch(torch, dev)
    say(f"offline NaN batch: {len(LENS)} clips, {len(NANS)} NaN samples")
    out, fo = lm.log_mel(plan, x, so)
    torch.cuda.synchronize()
    xh = x.cpu().numpy()
    L, E, fo_ref = O.logmel_packed(xh, so)
    assert np.array_equal(fo, fo_ref)
    n_bad = _check_nan_rows(out.cpu().numpy(), L, E, "offline NaN")
    # the frames holding each NaN: ceil-window count per sample position
    expect = 0
    for c, k in NANS:
        F = O.num_frames(LENS[c])
        expect += sum(1 for f in range(F) if 160 * f <= k < 160 * f + 400)
    assert n_bad == expect


def test_nan_streamed_frames(env):
    """Streams fed the same clips in pushes of 1280: the same NaN rows as
    offline, every other row bit for bit the offline row."""
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    n, N = 4, 25600
    x = torch.stack([S.speech_like(800 + j, N, dev) for j in range(n)])
    x[0, 5000] = float("nan")
    x[1, 0] = float("nan")
    x[3, N - 1] = float("nan")
    x[3, 12345] = float("nan")
    say("streamed NaN: 4 streams x 25600 in pushes of 1280")
    s = lm.logmel_stream_create(plan, n, 1280)
    got = [[] for _ in range(n)]
    for c in range(N // 1280):
        new = x[:, c * 1280:(c + 1) * 1280].contiguous().reshape(-1)
        o, f = lm.logmel_stream_push(s, new, [1280] * n)
        for j in range(n):
            got[j].append(o[f[j]:f[j + 1]])
    torch.cuda.synchronize()
    s.close()
    streamed = torch.cat([torch.cat(g) for g in got]).cpu().numpy()
    so = np.arange(n + 1, dtype=np.int64) * N
    ref, _ = lm.log_mel(plan, x.reshape(-1).contiguous(), so)
    ref = ref.cpu().numpy()
    assert streamed.shape == ref.shape
    assert np.array_equal(np.isnan(streamed), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(streamed[ok], ref[ok])
    L, E, _ = O.logmel_packed(x.reshape(-1).cpu().numpy(), so)
    _check_nan_rows(streamed, L, E, "streamed NaN")


def _reach(rate):
    """4 KS - 2J - 1, the stated bound on how far past an output's own window
    a non-finite sample can reach: the kernel stages, for each group of 16
    consecutive outputs, a window of 4 KS positions, KS the smallest multiple
    of 8 with 4 KS >= 2J + 1 plus the spread of the group's windows (plus two
    pad positions per super-period at rates where 32 divides its input span)."""
    g = math.gcd(rate, 16000)
    L, M = 16000 // g, rate // g
    J = math.ceil(O.resample_halfwidth(rate))
    T = 2 * J + 1
    Sp = L // math.gcd(L, 16) * 16
    S_in = Sp // L * M
    P = S_in + 2 if S_in % 32 == 0 else S_in

    def lds(u):
        return u // S_in * P + u % S_in
    t_max = 0
    for gm in range(Sp // 16):
        gb = (16 * gm * M) // L
        dd = ((16 * gm + 15) * M) // L - gb
        t_max = max(t_max, lds(gb + dd + T - 1) + 1 - lds(gb))
    KS = ((t_max + 3) // 4 + 7) // 8 * 8
    return 4 * KS - T, J


@pytest.mark.parametrize("rate,reach", [(44100, 53), (48000, 73), (32000, None)])
def test_resample_nan_reach(env, rate, reach):
    """A NaN sample makes NaN every output whose 2J + 1 window holds it (the
    oracle's definition); the kernel's other NaN outputs lie within the
    stated reach of the sample, inside its clip."""
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    R, J = _reach(rate)
    if reach is not None:
        assert R == reach
    lens = [3 * rate, rate, 2 * rate]
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    rng = np.random.default_rng(rate)
    xh = rng.uniform(-0.5, 0.5, int(so[-1])).astype(np.float32)
    k0 = rate // 2 + 37                 # in clip 1
    xh[so[1] + k0] = np.nan
    say(f"resampler NaN reach at {rate} Hz (bound {R})")
    r = lm.logmel_resampler_create(plan, rate)
    oo = lm.logmel_resample_offsets(so, rate)
    x = torch.from_numpy(xh).to(dev)
    y = lm.logmel_resample(r, x, torch.from_numpy(so).to(dev), torch.from_numpy(oo).to(dev),
                           int(oo[-1])).cpu().numpy()
    r.close()
    nan_out = np.flatnonzero(np.isnan(y))
    assert nan_out.size > 0
    # only in clip 1
    assert nan_out.min() >= oo[1] and nan_out.max() < oo[2]
    n = nan_out - oo[1]
    q = (n * rate) // 16000
    # oracle: outputs whose window [q - J, q + J] holds k0 are NaN
    n_all = np.arange(oo[2] - oo[1])
    q_all = (n_all * rate) // 16000
    must = n_all[(q_all - J <= k0) & (k0 <= q_all + J)]
    assert np.isin(must, n).all()
    # beyond the own window by at most the stated reach
    dist = np.maximum(np.maximum(q - J - k0, k0 - (q + J)), 0)
    assert dist.max() <= R, (rate, int(dist.max()), R)
    say(f"  {rate} Hz: {must.size} outputs by definition, {n.size} NaN, "
        f"furthest {int(dist.max())} past its window (bound {R})")


def test_resample_overstated_offsets_write_nothing_past_output(env):
    """Output offsets whose last entry overstates the total: the kernel
    writes no element past total_out (a sentinel tail stays untouched) and
    the earlier clips' outputs are unchanged."""
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    rate = 44100
    lens = [rate, rate // 3]
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    oo = lm.logmel_resample_offsets(so, rate)
    total = int(oo[-1])
    bad = oo.copy()
    bad[-1] += 4000                      # non-decreasing, past the buffer
    x = S.speech_like(5, int(so[-1]), dev)
    so_d = torch.from_numpy(so).to(dev)
    r = lm.logmel_resampler_create(plan, rate)
    say("resampler: overstated output offsets, sentinel tail")
    good = lm.logmel_resample(r, x, so_d, torch.from_numpy(oo).to(dev), total)
    buf = torch.full((total + 8192,), 12345.0, dtype=torch.float32, device=dev)
    bad_d = torch.from_numpy(bad).to(dev)
    # the raw C call: the binding sizes the output from total_out
    lm._check(lm._resample(r.handle, lm._dev_ptr(x, torch.float32, "x"), lm.LOGMEL_F32,
                           lm._dev_ptr(so_d, torch.int64, "so"),
                           lm._dev_ptr(bad_d, torch.int64, "oo"),
                           len(lens), total, lm._dev_ptr(buf, torch.float32, "y"),
                           lm._stream_handle(None, dev)), "logmel_resample")
    torch.cuda.synchronize()
    r.close()
    assert (buf[total:] == 12345.0).all()
    assert torch.equal(buf[:int(oo[1])], good[:int(oo[1])])
