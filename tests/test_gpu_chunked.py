"""30-s chunk layout [chunks, 3000, 128] of the HIP path: against the
offline HIP output (the same frames, bit for bit) and against the fp64
oracle's chunked layout (the parity rule of tests/parity.py)."""

import math
import sys

import numpy as np
import pytest

import oracle as O
import logmel_synth as S
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

# Padding rows hold the value of a silent frame: ln(1e-10) as the kernel's
# fp32 log gives it (silent_value checks it against ln(1e-10)).


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


def run_both(env, x_host, so):
    """Offline and chunked HIP outputs of one packed batch."""
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    x = torch.from_numpy(x_host).to(dev)
    fo = lm.logmel_frame_offsets(so)
    co = lm.logmel_chunk_offsets(so)
    so_d = torch.from_numpy(so).to(dev)
    fo_d = torch.from_numpy(fo).to(dev)
    co_d = torch.from_numpy(co).to(dev)
    off = lm.logmel_compute(plan, x, so_d, fo_d, int(fo[-1]))
    # poison the chunk output so that an unwritten row shows
    ch = torch.full((int(co[-1]), 3000, 128), float("nan"), dtype=torch.float32, device=dev)
    lm.logmel_compute_chunked(plan, x, so_d, fo_d, co_d, int(fo[-1]), int(co[-1]), out=ch)
    torch.cuda.synchronize()
    return off.cpu().numpy(), ch.cpu().numpy(), fo, co


def silent_value(env):
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    x = torch.zeros(400, dtype=torch.float32, device=dev)
    out, _ = lm.log_mel(plan, x, [0, 400])
    torch.cuda.synchronize()
    v = out.cpu().numpy()
    assert np.all(v == v[0, 0])
    assert abs(float(v[0, 0]) - math.log(1e-10)) < 1e-5
    return v[0, 0]


def check_layout(off, ch, fo, co, so, lm, pad):
    cf = lm.logmel_chunk_frames(so, int(co[-1]))
    for i in range(len(fo) - 1):
        F = int(fo[i + 1] - fo[i])
        assert int(co[i + 1] - co[i]) == -(-F // 3000)
        for j in range(int(co[i + 1] - co[i])):
            n = int(cf[co[i] + j])
            assert n == min(3000, F - 3000 * j)
            np.testing.assert_array_equal(ch[co[i] + j, :n], off[fo[i] + 3000 * j: fo[i] + 3000 * j + n])
            assert np.all(ch[co[i] + j, n:] == pad), (i, j)


def test_chunked_edges_equal_offline(env):
    lm = env[0]
    say("chunked: edge clip lengths, bitwise against the offline output")
    lens = [0, 399, 400, 3000 * 160 + 240, 3000 * 160 + 400, 6000 * 160 + 240, 480000,
            12345, 0, 9000 * 160 + 241, 77]
    rng = np.random.default_rng(8)
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = rng.uniform(-0.5, 0.5, int(so[-1])).astype(np.float32)
    off, ch, fo, co = run_both(env, x, so)
    assert [O.num_frames(n) for n in lens] == [0, 0, 1, 3000, 3001, 6000, 2998, 75, 0, 9000, 0]
    assert list(np.diff(co)) == [0, 0, 1, 1, 2, 2, 1, 1, 0, 3, 0]
    check_layout(off, ch, fo, co, so, lm, silent_value(env))


def test_chunked_parity_vs_oracle(env):
    say("chunked: parity against the oracle's chunk layout")
    lens = [16000, 3000 * 160 + 400, 0, 5000]
    rng = np.random.default_rng(9)
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = (0.2 * rng.standard_normal(int(so[-1]))).astype(np.float32)
    off, ch, fo, co = run_both(env, x, so)
    ref, co_ref = O.logmel_chunked(x, so)
    assert np.array_equal(co, co_ref)
    # energies of the oracle in the same layout (padding rows: the floor)
    _, E, _ = O.logmel_packed(x, so)
    Ech = np.full(ref.shape, 1e-10)
    for i in range(len(lens)):
        F = int(fo[i + 1] - fo[i])
        for j in range(int(co[i + 1] - co[i])):
            n = min(3000, F - 3000 * j)
            Ech[co[i] + j, :n] = E[fo[i] + 3000 * j: fo[i] + 3000 * j + n]
    rep = assert_parity(ch.reshape(-1, 128), ref.reshape(-1, 128), Ech.reshape(-1, 128),
                        "chunked small batch")
    say(f"chunked small batch: {rep}")


def test_chunked_config2(env):
    lm = env[0]
    say("chunked: config2, 64 x 30 s, bitwise against the offline output")
    import torch
    x, so = S.config2(device=torch.device("cuda", 0))
    off, ch, fo, co = run_both(env, x.cpu().numpy(), so)
    assert ch.shape == (64, 3000, 128)
    check_layout(off, ch, fo, co, so, lm, silent_value(env))



def test_chunked_past_2_31_samples(env):
    """The ragged long batch's recipe with seed 20009 (2,167,173,778
    samples, 4,641 chunks) in the chunk layout: every frame row of every
    chunk equals the offline row bit for bit and every padding row holds
    the silent frame's value, compared on the GPU (the layouts are 7 GB
    each)."""
    lm, plan, torch = env
    say("chunked: config4 recipe seed 20009, past 2**31 samples")
    dev = torch.device("cuda", 0)
    x, so = S.config4(device=dev, seed=20009)
    assert int(so[-1]) > 2**31
    fo = lm.logmel_frame_offsets(so)
    co = lm.logmel_chunk_offsets(so)
    so_d = torch.from_numpy(so).to(dev)
    fo_d = torch.from_numpy(fo).to(dev)
    co_d = torch.from_numpy(co).to(dev)
    total, chunks = int(fo[-1]), int(co[-1])
    off = lm.logmel_compute(plan, x, so_d, fo_d, total)
    ch = torch.full((chunks, 3000, 128), float("nan"), dtype=torch.float32, device=dev)
    lm.logmel_compute_chunked(plan, x, so_d, fo_d, co_d, total, chunks, out=ch)
    torch.cuda.synchronize()
    del x
    torch.cuda.empty_cache()
    # flat chunk row of every frame: co[clip] * 3000 + (frame - fo[clip])
    clip = torch.from_numpy(np.repeat(np.arange(len(so) - 1), np.diff(fo))).to(dev)
    frame = torch.arange(total, device=dev)
    flat = co_d[clip] * 3000 + (frame - fo_d[clip])
    chf = ch.view(-1, 128)
    same = torch.zeros(total, dtype=torch.bool, device=dev)
    for a in range(0, total, 1 << 22):
        b = min(total, a + (1 << 22))
        same[a:b] = (chf[flat[a:b]] == off[a:b]).all(dim=1)
    assert bool(same.all()), int((~same).sum())
    is_frame = torch.zeros(chunks * 3000, dtype=torch.bool, device=dev)
    is_frame[flat] = True
    pad = chf[~is_frame]
    assert pad.shape[0] == chunks * 3000 - total
    assert bool((pad == silent_value(env)).all())
    say(f"chunked past 2**31: {total} frame rows equal offline, {pad.shape[0]} padding rows")
    del off, ch, chf, pad, same, is_frame, flat
    torch.cuda.empty_cache()

def test_chunked_validate_and_empty(env, monkeypatch):
    lm, plan, torch = env
    say("chunked: validate mode, empty calls")
    dev = torch.device("cuda", 0)
    x = torch.zeros(1060, dtype=torch.float32, device=dev)
    so = torch.tensor([0, 500, 1060], dtype=torch.int64, device=dev)
    fo = torch.tensor([0, 1, 3], dtype=torch.int64, device=dev)
    co_bad = torch.tensor([0, 1, 1], dtype=torch.int64, device=dev)
    co = torch.tensor([0, 1, 2], dtype=torch.int64, device=dev)
    monkeypatch.setenv("LOGMEL_VALIDATE", "1")
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_compute_chunked(plan, x, so, fo, co_bad, 3, 1)
    assert e.value.status == lm.LOGMEL_ERR_INVALID_ARGUMENT
    out = lm.logmel_compute_chunked(plan, x, so, fo, co, 3, 2)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    pad = silent_value(env)
    # padding rows and the silent frames hold the same value
    assert np.all(o == pad)
    monkeypatch.delenv("LOGMEL_VALIDATE")
    empty = torch.zeros(0, 3000, 128, dtype=torch.float32, device=dev)
    so0 = torch.tensor([0, 300], dtype=torch.int64, device=dev)
    z = torch.tensor([0, 0], dtype=torch.int64, device=dev)
    lm.logmel_compute_chunked(plan, x, so0, z, z, 0, 0, out=empty)
    torch.cuda.synchronize()
