"""int16 PCM ingest and fp16 output of the HIP path.

int16 sample s means s / 32768, exact in fp32: an int16 batch must give the
fp32 batch's result bit for bit, in both layouts, and match the oracle on
the same values. fp16 output must be the fp32 output rounded once to
nearest (bit for bit), and within the parity rule widened by half an fp16
spacing of the oracle's value."""

import math
import sys

import numpy as np
import pytest

import oracle as O
import logmel_synth as S
from tests.parity import assert_parity, parity_report

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


def offsets(env, so):
    lm, plan, torch = env
    dev = torch.device("cuda", 0)
    fo = lm.logmel_frame_offsets(so)
    co = lm.logmel_chunk_offsets(so)
    return (fo, co, torch.from_numpy(so).to(dev), torch.from_numpy(fo).to(dev),
            torch.from_numpy(co).to(dev))


def int16_batch(lens, seed):
    rng = np.random.default_rng(seed)
    n = int(sum(lens))
    s = rng.integers(-32768, 32768, n).astype(np.int16)
    # full-scale values and silence somewhere
    s[: min(n, 50)] = -32768
    s[min(n, 50): min(n, 100)] = 32767
    s[min(n, 100): min(n, 900)] = 0
    return s


def test_int16_equals_fp32_and_oracle(env):
    lm, plan, torch = env
    say("int16: edge lengths (odd and even clip starts), both layouts")
    lens = [0, 399, 400, 401, 559, 560, 561, 3, 7, 1000, 3000 * 160 + 400, 16001,
            65 * 160 + 240, 480000 + 1]
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    s16 = int16_batch(lens, 41)
    x32 = s16.astype(np.float32) / np.float32(32768.0)
    assert np.array_equal((x32 * 32768).astype(np.int16), s16)
    fo, co, so_d, fo_d, co_d = offsets(env, so)
    dev = torch.device("cuda", 0)
    a16 = torch.from_numpy(s16).to(dev)
    a32 = torch.from_numpy(x32).to(dev)
    T = int(fo[-1])
    C = int(co[-1])
    o16 = lm.logmel_compute_ex(plan, a16, so_d, fo_d, T)
    o32 = lm.logmel_compute_ex(plan, a32, so_d, fo_d, T)
    c16 = lm.logmel_compute_ex(plan, a16, so_d, fo_d, T, chunk_offsets=co_d, total_chunks=C)
    c32 = lm.logmel_compute_ex(plan, a32, so_d, fo_d, T, chunk_offsets=co_d, total_chunks=C)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32), "int16 != fp32 (frames)"
    assert torch.equal(c16, c32), "int16 != fp32 (chunks)"
    L, E, _ = O.logmel_packed(x32, so)
    rep = assert_parity(o16.cpu().numpy(), L, E, "int16 edge batch")
    say(f"int16 edge batch: {rep}")


def test_int16_short_clips(env):
    """Tiles across short clips (odd and even starts) staged from int16."""
    lm, plan, torch = env
    say("int16: short clips")
    rng = np.random.default_rng(43)
    lens = [0 if f == 0 else 160 * (int(f) - 1) + 400 + int(rng.integers(0, 160))
            for f in rng.integers(0, 10, 300)]
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    s16 = int16_batch(lens, 44)
    x32 = s16.astype(np.float32) / np.float32(32768.0)
    fo, co, so_d, fo_d, co_d = offsets(env, so)
    dev = torch.device("cuda", 0)
    T = int(fo[-1])
    o16 = lm.logmel_compute_ex(plan, torch.from_numpy(s16).to(dev), so_d, fo_d, T)
    o32 = lm.logmel_compute_ex(plan, torch.from_numpy(x32).to(dev), so_d, fo_d, T)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32), "int16 != fp32"
    L, E, _ = O.logmel_packed(x32, so)
    rep = assert_parity(o16.cpu().numpy(), L, E, "int16 short clips")
    say(f"int16 short clips: {rep}")


def test_int16_config2_quantised(env):
    lm, plan, torch = env
    say("int16: config2 quantised to 16 bits, bitwise against fp32")
    dev = torch.device("cuda", 0)
    x, so = S.config2(device=dev)
    s16 = torch.clamp(torch.round(x * 32768.0), -32768, 32767).to(torch.int16)
    x32 = s16.to(torch.float32) / 32768.0
    fo, co, so_d, fo_d, co_d = offsets(env, so)
    T = int(fo[-1])
    o16 = lm.logmel_compute_ex(plan, s16, so_d, fo_d, T)
    o32 = lm.logmel_compute_ex(plan, x32, so_d, fo_d, T)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32)


def half_rule(L16, L, E):
    """The parity rule of tests/parity.py for a value rounded once more, to
    fp16: the fp32 result is within the rule, and rounding to nearest moves
    it by at most half the fp16 spacing of the binade it lies in (taken at the
    larger magnitude of result and oracle, so a value just past a power of
    two gets that binade's spacing). Both the 1e-3 bound and the quiet
    ceiling widen by that."""
    L16 = np.asarray(L16, dtype=np.float64)
    loud = E >= 1e-7
    # fp16 spacing of the binade holding the larger of the two magnitudes
    mag = np.maximum(np.abs(L), np.abs(L16)) + 1e-3
    sp = np.exp2(np.floor(np.log2(np.maximum(mag, 2.0 ** -14))) - 10)
    err = np.abs(L16 - L)
    bad_loud = loud & ~(err <= 1e-3 + sp / 2)
    bad_quiet = ~loud & ~(L16 < math.log(1e-7) + 1 + sp / 2)
    for idx in np.argwhere(bad_loud | bad_quiet)[:8]:
        t = tuple(idx)
        say(f"  fp16 miss at {t}: oracle {L[t]:.9g} (E {E[t]:.3g}) fp16 {L16[t]:.9g} "
            f"err {err[t]:.3g} spacing {sp[t]:.3g}")
    return int(bad_loud.sum()), int(bad_quiet.sum()), float(err[loud].max(initial=0.0))


def test_fp16_output(env):
    lm, plan, torch = env
    say("fp16 output: fp32 rounded once, and the widened parity rule")
    x, so = S.config1()
    dev = torch.device("cuda", 0)
    xd = x.to(dev)
    fo, co, so_d, fo_d, co_d = offsets(env, so)
    T = int(fo[-1])
    C = int(co[-1])
    h = lm.logmel_compute_ex(plan, xd, so_d, fo_d, T, out_dtype=torch.float16)
    f = lm.logmel_compute_ex(plan, xd, so_d, fo_d, T)
    hc = lm.logmel_compute_ex(plan, xd, so_d, fo_d, T, chunk_offsets=co_d, total_chunks=C,
                              out_dtype=torch.float16)
    fc = lm.logmel_compute_ex(plan, xd, so_d, fo_d, T, chunk_offsets=co_d, total_chunks=C)
    s16 = torch.clamp(torch.round(xd * 32768.0), -32768, 32767).to(torch.int16)
    h16 = lm.logmel_compute_ex(plan, s16, so_d, fo_d, T, out_dtype=torch.float16)
    f16in = lm.logmel_compute_ex(plan, s16, so_d, fo_d, T)
    torch.cuda.synchronize()
    assert h.dtype == torch.float16 and h.shape == (T, 128)
    assert torch.equal(h, f.half()), "fp16 output is not the fp32 output rounded"
    assert torch.equal(hc, fc.half()), "fp16 chunks are not the fp32 chunks rounded"
    assert torch.equal(h16, f16in.half())
    L, E, _ = O.logmel_packed(x.numpy(), so)
    bl, bq, mx = half_rule(h.float().cpu().numpy(), L, E)
    say(f"fp16 config1: bad_loud={bl} bad_quiet={bq} max_err_loud={mx:.3g}")
    assert bl == 0 and bq == 0



def test_fp16_config2_is_fp32_rounded(env):
    """The 64 x 30 s batch (24.6 M values), fp32 and int16 input: the fp16
    output is the fp32 output rounded once, bit for bit. The two kernels
    split the bands between a pair's lanes differently (alternate runs of 4
    bands for fp32 output, of 8 for fp16), so a band whose bins lie in both
    halves is added up by different lanes; its energy must not depend on
    that."""
    lm, plan, torch = env
    say("fp16 output: config2, fp16 = fp32 rounded, bit for bit")
    dev = torch.device("cuda", 0)
    x, so = S.config2(device=dev)
    fo, co, so_d, fo_d, co_d = offsets(env, so)
    T = int(fo[-1])
    f = lm.logmel_compute_ex(plan, x, so_d, fo_d, T)
    h = lm.logmel_compute_ex(plan, x, so_d, fo_d, T, out_dtype=torch.float16)
    torch.cuda.synchronize()
    diff = int((h != f.half()).sum())
    s16 = torch.clamp(torch.round(x * 32768.0), -32768, 32767).to(torch.int16)
    f16in = lm.logmel_compute_ex(plan, s16, so_d, fo_d, T)
    h16 = lm.logmel_compute_ex(plan, s16, so_d, fo_d, T, out_dtype=torch.float16)
    torch.cuda.synchronize()
    diff16 = int((h16 != f16in.half()).sum())
    say(f"fp16 config2: {diff} and {diff16} values differ from the rounded fp32 output")
    assert diff == 0 and diff16 == 0

def test_unsupported_types(env):
    lm, plan, torch = env
    say("unsupported sample and output types")
    dev = torch.device("cuda", 0)
    x = torch.zeros(1000, dtype=torch.float32, device=dev)
    so = torch.tensor([0, 1000], dtype=torch.int64, device=dev)
    fo = torch.tensor([0, 4], dtype=torch.int64, device=dev)
    out = torch.empty((4, 128), dtype=torch.float32, device=dev)
    for it, ot in ((7, lm.LOGMEL_F32), (lm.LOGMEL_F16, lm.LOGMEL_F32), (lm.LOGMEL_F32, lm.LOGMEL_I16)):
        r = lm._compute_ex(plan.handle, ctypes_ptr(x), it, ctypes_ptr(so), ctypes_ptr(fo), None, 1, 4,
                           0, ctypes_ptr(out), ot, None)
        assert r == lm.LOGMEL_ERR_UNSUPPORTED, (it, ot)


def ctypes_ptr(t):
    import ctypes
    return ctypes.c_void_p(t.data_ptr())


def test_misaligned_sample_buffer_rejected(env):
    lm, plan, torch = env
    say("int16 buffer starting 2 bytes into an allocation is rejected")
    dev = torch.device("cuda", 0)
    base = torch.zeros(2001, dtype=torch.int16, device=dev)
    x = base[1:]
    assert x.data_ptr() % 4 == 2
    so = torch.tensor([0, 2000], dtype=torch.int64, device=dev)
    fo = torch.tensor([0, 10], dtype=torch.int64, device=dev)
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_compute_ex(plan, x, so, fo, 10)
    assert e.value.status == lm.LOGMEL_ERR_INVALID_ARGUMENT
