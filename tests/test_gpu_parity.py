"""Offline HIP path against the fp64 oracle, element by element.

Every case prints its name before touching the GPU. Inputs are seeded and
synthetic (logmel_synth); the same fp32 buffer goes to both sides. The rule
is in tests/parity.py; frame offsets are compared exactly.
"""

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


def run_gpu(env, samples, so):
    """samples: torch fp32 (any device); so: numpy int64 offsets."""
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    x = samples.to(dev)
    out, fo = lm.log_mel(plan, x, so)
    torch.cuda.synchronize()
    return out.cpu().numpy(), fo


def check_against_oracle(env, samples, so, what):
    say(what)
    Lg, fo = run_gpu(env, samples, so)
    x = samples.cpu().numpy()
    L, E, fo_ref = O.logmel_packed(x, so)
    assert np.array_equal(fo, fo_ref), "frame offsets differ"
    rep = assert_parity(Lg, L, E, what)
    say(f"{what}: {rep}")
    return Lg, L, E


def test_config0_three_tone(env):
    import torch
    x, so = S.config0()
    Lg, L, E = check_against_oracle(env, x, so, "config0 three tones, 1 clip x 16000")
    assert Lg.shape == (98, 128)


def test_config1_speech_30s(env):
    x, so = S.config1()
    Lg, L, E = check_against_oracle(env, x, so, "config1 speech 30 s")
    assert Lg.shape == (2998, 128)


def test_edge_lengths_and_misaligned_starts(env):
    import torch
    lens = [0, 399, 400, 401, 559, 560, 561, 719, 720, 1000, 16001, 3, 7, 65 * 160 + 240]
    rng = np.random.default_rng(21)
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = torch.from_numpy(rng.uniform(-1, 1, int(so[-1])).astype(np.float32))
    check_against_oracle(env, x, so, "edge lengths, odd starts")


def test_many_boundaries_in_one_tile(env):
    """More than 64 clip boundaries inside one 64-frame tile (runs of empty
    clips) and tiles made of one-frame clips."""
    import torch
    lens = [400] * 10 + [0] * 150 + [560] * 70 + [100] * 80 + [1000] + [0] * 5 + [401] * 90
    rng = np.random.default_rng(22)
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = torch.from_numpy(rng.uniform(-1, 1, int(so[-1])).astype(np.float32))
    check_against_oracle(env, x, so, "many boundaries per tile")


def short_clip_lengths(rng):
    """Clips of 0 to 40 frames: runs of 2, 3, 4 and 8-frame clips (tiles of
    up to 8 clip pieces are staged in LDS, more gather per lane), random
    mixes with odd leftovers, empty and sub-frame clips between them."""
    def clip(frames):
        return 0 if frames == 0 else 160 * (frames - 1) + 400 + int(rng.integers(0, 160))
    lens = []
    for frames, count in [(4, 40), (3, 40), (8, 20), (2, 30), (1, 10)]:
        lens += [clip(frames) for _ in range(count)]
    lens += [clip(int(f)) for f in rng.integers(0, 13, 80)]
    lens += [int(n) for n in rng.integers(0, 400, 10)]
    lens += [clip(int(f)) for f in rng.integers(30, 41, 10)]
    order = rng.permutation(len(lens) - 50)
    return [lens[i] for i in order] + lens[-50:]


def test_short_clips_staged_across_clips(env):
    """Tiles across many short clips: every frame against the oracle, and bit
    for bit the frames of the same clip computed alone (a one-clip call)."""
    import torch
    rng = np.random.default_rng(26)
    lens = short_clip_lengths(rng)
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = torch.from_numpy((0.5 * rng.normal(size=int(so[-1]))).clip(-1, 1).astype(np.float32))
    Lg, L, E = check_against_oracle(env, x, so, f"{len(lens)} short clips")
    fo = O.frame_offsets(so)
    say("short clips, each alone")
    for i in range(len(lens)):
        if fo[i + 1] == fo[i]:
            continue
        alone, _ = run_gpu(env, x[so[i]:so[i + 1]], np.array([0, lens[i]], dtype=np.int64))
        assert np.array_equal(alone, Lg[fo[i]:fo[i + 1]]), f"clip {i} ({lens[i]} samples)"


def test_random_ragged_batch(env):
    import torch
    rng = np.random.default_rng(23)
    lens = rng.integers(0, 40000, 97)
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = torch.from_numpy((0.5 * rng.normal(size=int(so[-1]))).clip(-1, 1).astype(np.float32))
    check_against_oracle(env, x, so, "random ragged batch of 97 clips")


def test_silence_is_floor(env):
    import torch
    say("silence")
    x = torch.zeros(16000 * 3, dtype=torch.float32)
    Lg, fo = run_gpu(env, x, np.array([0, 16000, 48000], dtype=np.int64))
    assert Lg.shape == (98 + 198, 128)
    assert np.all(np.abs(Lg - math.log(1e-10)) < 1e-5)


def test_scale_of_outputs_matches_tone_closed_form(env):
    """A bin-25 (1000 Hz) tone of amplitude A: the two filters around 1000 Hz
    carry (A sum w / 2)^2 times their weights at bin 25, plus neighbours."""
    import torch
    n = np.arange(16000)
    x = torch.from_numpy((0.3 * np.sin(2 * np.pi * 1000 * n / 16000)).astype(np.float32))
    check_against_oracle(env, x, np.array([0, 16000], dtype=np.int64), "pure 1000 Hz tone")


def test_batch_invariance(env):
    """A clip alone and the same clip inside a packed batch give the same
    bits."""
    import torch
    say("batch invariance")
    a = S.speech_like(5, 100_003)
    b = S.speech_like(6, 77_777)
    c = S.speech_like(7, 50_001)
    alone, _ = run_gpu(env, b, np.array([0, b.numel()], dtype=np.int64))
    packed = torch.cat([a, b, c])
    so = np.array([0, a.numel(), a.numel() + b.numel(), packed.numel()], dtype=np.int64)
    Lp, fo = run_gpu(env, packed, so)
    assert np.array_equal(alone, Lp[fo[1]:fo[2]])


def test_config2_full(env):
    """64 x 30 s packed batch, every element against the oracle."""
    import torch
    say("config2 generate on GPU")
    x, so = S.config2(device="cuda")
    check_against_oracle(env, x, so, "config2 64 x 480000")


def test_inconsistent_offsets_give_nan_rows(env):
    """Frame offsets promising more frames than a clip holds: those rows are
    NaN (the kernel's own bounds check), the others are right."""
    import torch
    lm, plan, torch = env
    say("inconsistent offsets")
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(24)
    x = torch.from_numpy(rng.uniform(-1, 1, 1060).astype(np.float32)).to(dev)
    so = torch.tensor([0, 500, 1060], dtype=torch.int64, device=dev)   # 1 and 2 frames
    fo = torch.tensor([0, 3, 5], dtype=torch.int64, device=dev)        # claims 3 and 2
    out = lm.logmel_compute(plan, x, so, fo, 5)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(np.isnan(o[1:3]))
    assert not np.any(np.isnan(o[[0, 3, 4]]))
    L, E, _ = O.logmel_packed(x.cpu().numpy(), [0, 500, 1060])
    assert_parity(o[[0, 3, 4]], L, E, "rows that are valid")


@pytest.mark.gpu
@pytest.mark.parametrize("in_i16,out_f16", [(False, True), (True, False), (True, True)])
def test_inconsistent_offsets_nan_rows_all_types(env, in_i16, out_f16):
    """The same NaN rows with int16 PCM input and with fp16 output (a NaN
    sample marks the frame before the transform, so the row is NaN in every
    output type), and the other rows equal to the fp32 path's, rounded once
    to fp16 for fp16 output."""
    lm, plan, torch = env
    say(f"inconsistent offsets, int16 in {in_i16}, fp16 out {out_f16}")
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(25)
    s16 = rng.integers(-32768, 32768, 1060).astype(np.int16)
    x32 = s16.astype(np.float32) / np.float32(32768.0)
    so = torch.tensor([0, 500, 1060], dtype=torch.int64, device=dev)   # 1 and 2 frames
    fo = torch.tensor([0, 3, 5], dtype=torch.int64, device=dev)        # claims 3 and 2
    xin = torch.from_numpy(s16 if in_i16 else x32).to(dev)
    got = lm.logmel_compute_ex(plan, xin, so, fo, 5,
                               out_dtype=torch.float16 if out_f16 else torch.float32)
    ref = lm.logmel_compute_ex(plan, torch.from_numpy(x32).to(dev), so, fo, 5)
    torch.cuda.synchronize()
    g = got.float().cpu().numpy()
    r = ref.cpu().numpy()
    assert np.all(np.isnan(g[1:3]))
    assert not np.any(np.isnan(g[[0, 3, 4]]))
    want = r[[0, 3, 4]].astype(np.float16).astype(np.float32) if out_f16 else r[[0, 3, 4]]
    assert np.array_equal(g[[0, 3, 4]], want)


def test_validate_mode_rejects(env, monkeypatch):
    lm, plan, torch = env
    say("validate mode")
    dev = torch.device("cuda", 0)
    x = torch.zeros(1060, dtype=torch.float32, device=dev)
    so = torch.tensor([0, 500, 1060], dtype=torch.int64, device=dev)
    fo = torch.tensor([0, 3, 5], dtype=torch.int64, device=dev)
    monkeypatch.setenv("LOGMEL_VALIDATE", "1")
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_compute(plan, x, so, fo, 5)
    assert e.value.status == lm.LOGMEL_ERR_INVALID_ARGUMENT
    fo_ok = torch.tensor([0, 1, 3], dtype=torch.int64, device=dev)
    lm.logmel_compute(plan, x, so, fo_ok, 3)
    torch.cuda.synchronize()


def test_empty_calls(env):
    lm, plan, torch = env
    say("empty calls")
    dev = torch.device("cuda", 0)
    x = torch.zeros(300, dtype=torch.float32, device=dev)
    out, fo = lm.log_mel(plan, x, [0, 300])
    assert out.shape == (0, 128) and fo.tolist() == [0, 0]
    out, fo = lm.log_mel(plan, x, [0])
    assert out.shape == (0, 128)


def test_config4_ragged_long_sampled(env):
    """200 log-uniform clips up to 87 min (about 2e9 samples), in the launch
    configuration the benchmark times; the oracle checks every clip's first
    and last three frames plus 20000 random rows, each from its own 400
    samples, and the frame offsets exactly."""
    lm, plan, torch = env
    say("config4 generate on GPU")
    x, so = S.config4(device="cuda")
    say(f"config4 samples={int(so[-1])}")
    fo_ref = O.frame_offsets(so)
    out, fo = lm.log_mel(plan, x, so)
    torch.cuda.synchronize()
    assert np.array_equal(fo, fo_ref)
    total = int(fo[-1])
    rng = np.random.default_rng(25)
    edge = []
    for i in range(len(so) - 1):
        a, b = int(fo[i]), int(fo[i + 1])
        edge += list(range(a, min(b, a + 3))) + list(range(max(a, b - 3), b))
    rows = np.unique(np.concatenate([np.array(edge, dtype=np.int64),
                                     rng.integers(0, total, 20000)]))
    clip = np.searchsorted(fo, rows, side="right") - 1
    start = so[clip] + 160 * (rows - fo[clip])
    idx = torch.from_numpy(start).cuda()[:, None] + torch.arange(400, device="cuda")[None, :]
    frames = x[idx].cpu().numpy()
    L, E = O.logmel_frames(frames)
    Lg = out[torch.from_numpy(rows).cuda()].cpu().numpy()
    rep = assert_parity(Lg, L, E, "config4 sampled rows")
    say(f"config4: {rep}")
    del x, out
    torch.cuda.empty_cache()



def _sampled_rows_parity(torch, x, so, fo, out, rows, what):
    """Rows ``rows`` of ``out`` against the oracle on each row's own 400
    samples of ``x`` (fp32 on the GPU)."""
    clip = np.searchsorted(fo, rows, side="right") - 1
    start = so[clip] + 160 * (rows - fo[clip])
    idx = torch.from_numpy(start).cuda()[:, None] + torch.arange(400, device="cuda")[None, :]
    frames = x[idx].cpu().numpy()
    L, E = O.logmel_frames(frames)
    Lg = out[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    return assert_parity(Lg, L, E, what)


def test_config4_recipe_past_2_31_samples(env):
    """The ragged long batch's recipe with seed 20009, whose 200 clips hold
    2,167,173,778 samples: sample indices pass 2**31, so every sample
    position must be carried in 64 bits. fp32 input, then the same samples
    as int16 PCM (read two bytes per sample, another address computation).
    The oracle checks every clip's first and last three frames, the frames
    whose 400 samples lie around sample 2**31, 5000 random rows and 2000
    random rows past sample 2**31, each from its own samples; the frame
    offsets exactly."""
    lm, plan, torch = env
    say("config4 recipe, seed 20009: generate on GPU")
    x, so = S.config4(device="cuda", seed=20009)
    assert int(so[-1]) == 2_167_173_778 and int(so[-1]) > 2**31
    fo = O.frame_offsets(so)
    total = int(fo[-1])
    rng = np.random.default_rng(26)
    rows = []
    for i in range(len(so) - 1):
        a, b = int(fo[i]), int(fo[i + 1])
        rows += list(range(a, min(b, a + 3))) + list(range(max(a, b - 3), b))
    c = int(np.searchsorted(so, 2**31, side="right")) - 1
    f0 = int(fo[c]) + (2**31 - int(so[c])) // 160
    rows += [r for r in range(f0 - 4, f0 + 4) if fo[c] <= r < fo[c + 1]]
    rows = np.unique(np.concatenate([np.array(rows, dtype=np.int64),
                                     rng.integers(0, total, 5000),
                                     rng.integers(f0 + 1, total, 2000)]))
    clip = np.searchsorted(fo, rows, side="right") - 1
    start = so[clip] + 160 * (rows - fo[clip])
    assert int((start > 2**31).sum()) > 1000     # rows that read samples past 2**31
    so_d = torch.from_numpy(so).cuda()
    fo_d = torch.from_numpy(fo).cuda()
    say(f"config4 seed 20009 fp32: samples={int(so[-1])} frames={total}")
    out = lm.logmel_compute(plan, x, so_d, fo_d, total)
    torch.cuda.synchronize()
    rep = _sampled_rows_parity(torch, x, so, fo, out, rows, "past 2**31, fp32 in")
    say(f"config4 seed 20009 fp32: {rep}")
    say("config4 seed 20009 int16")
    x16 = torch.round(x * 32767.0).to(torch.int16)
    del x
    torch.cuda.empty_cache()
    out.fill_(0.0)
    lm.logmel_compute_ex(plan, x16, so_d, fo_d, total, out=out)
    torch.cuda.synchronize()
    xs = x16.to(torch.float32) * (1.0 / 32768.0)
    del x16
    torch.cuda.empty_cache()
    rep = _sampled_rows_parity(torch, xs, so, fo, out, rows, "past 2**31, int16 in")
    say(f"config4 seed 20009 int16: {rep}")
    del xs, out
    torch.cuda.empty_cache()