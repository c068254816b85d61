"""Python binding of liblogmel.so, the MI355X (gfx950) 128-bin log-mel front end.

Argument marshalling only: every step of the front end runs in the HIP
kernels behind the C ABI declared in include/logmel.h. Functions carry the C
names. Device buffers are torch tensors on a ROCm device (torch provides the
memory and the stream); the library is loaded from this directory and there
is no fallback: without the built library, importing this package raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblogmel.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python log_mel_spectrogram_amd/build.py` "
        "(hipcc for gfx950). There is no CPU fallback.")

_lib = ctypes.CDLL(LIB_PATH)

LOGMEL_OK = 0
LOGMEL_ERR_INVALID_ARGUMENT = -1
LOGMEL_ERR_UNSUPPORTED = -2
LOGMEL_ERR_OUT_OF_MEMORY = -3
LOGMEL_ERR_DEVICE = -4
LOGMEL_ERR_INPUT_TOO_LONG = -5

N_MELS = 128
CHUNK_FRAMES = 3000   # LOGMEL_CHUNK_FRAMES
LOGMEL_F32 = 0
LOGMEL_I16 = 1
LOGMEL_F16 = 2
N_FFT = 400
HOP = 160
SAMPLE_RATE = 16000

_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_i64p = ctypes.POINTER(ctypes.c_int64)


class logmel_config(ctypes.Structure):
    _fields_ = [("sample_rate", ctypes.c_int32), ("n_fft", ctypes.c_int32),
                ("hop", ctypes.c_int32), ("n_mels", ctypes.c_int32),
                ("f_min", ctypes.c_double), ("f_max", ctypes.c_double),
                ("log_floor", ctypes.c_double), ("device", ctypes.c_int32)]


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_default_config = _sig("logmel_default_config", None, ctypes.POINTER(logmel_config))
_abi_version = _sig("logmel_abi_version", ctypes.c_int)
_status_string = _sig("logmel_status_string", ctypes.c_char_p, ctypes.c_int)
_plan_create = _sig("logmel_plan_create", ctypes.c_int, ctypes.POINTER(logmel_config),
                    ctypes.POINTER(_p))
_plan_destroy = _sig("logmel_plan_destroy", None, _p)
_num_frames = _sig("logmel_num_frames", _i64, _i64)
_frame_offsets = _sig("logmel_frame_offsets", ctypes.c_int, _i64p, _i64, _i64p)
_compute = _sig("logmel_compute", ctypes.c_int, _p, _p, _p, _p, _i64, _i64, _p, _p)
_chunk_offsets = _sig("logmel_chunk_offsets", ctypes.c_int, _i64p, _i64, _i64p)
_chunk_frames = _sig("logmel_chunk_frames", ctypes.c_int, _i64p, _i64, _i64, _i64p)
_compute_chunked = _sig("logmel_compute_chunked", ctypes.c_int, _p, _p, _p, _p, _p, _i64, _i64,
                        _i64, _p, _p)
_compute_ex = _sig("logmel_compute_ex", ctypes.c_int, _p, _p, ctypes.c_int, _p, _p, _p, _i64, _i64,
                   _i64, _p, ctypes.c_int, _p)
_stream_create = _sig("logmel_stream_create", ctypes.c_int, _p, _i64, _i64, ctypes.POINTER(_p))
_stream_create_ex = _sig("logmel_stream_create_ex", ctypes.c_int, _p, _i64, _i64, ctypes.c_int32,
                         ctypes.POINTER(_p))
_stream_frames_for_flush = _sig("logmel_stream_frames_for_flush", ctypes.c_int, _p, _i64p)
_stream_flush = _sig("logmel_stream_flush", ctypes.c_int, _p, _p, ctypes.c_int, _i64p, _p)
_stream_destroy = _sig("logmel_stream_destroy", None, _p)
_stream_reset = _sig("logmel_stream_reset", ctypes.c_int, _p)
_stream_frames_for_push = _sig("logmel_stream_frames_for_push", ctypes.c_int, _p, _i64p, _i64p)
_stream_push = _sig("logmel_stream_push", ctypes.c_int, _p, _p, _i64p, _p, _i64p, _p)
_stream_push_ex = _sig("logmel_stream_push_ex", ctypes.c_int, _p, _p, ctypes.c_int, _i64p, _p,
                       ctypes.c_int, _i64p, _p)
_stream_counters = _sig("logmel_stream_counters", ctypes.c_int, _p, _i64, _i64p, _i64p)
_stream_push_static = _sig("logmel_stream_push_static", ctypes.c_int, _p, _i64, _p, _i64p,
                           ctypes.c_int, _p, _i64, _i64p, _p)
_stream_state_bytes = _sig("logmel_stream_state_bytes", _i64, _p)
_stream_get_state = _sig("logmel_stream_get_state", ctypes.c_int, _p, _p, _p)
_stream_set_state = _sig("logmel_stream_set_state", ctypes.c_int, _p, _p, _p)
_resample_length = _sig("logmel_resample_length", _i64, _i64, ctypes.c_int32)
_resample_offsets = _sig("logmel_resample_offsets", ctypes.c_int, ctypes.c_int32, _i64p, _i64,
                         _i64p)
_resampler_create = _sig("logmel_resampler_create", ctypes.c_int, _p, ctypes.c_int32,
                         ctypes.POINTER(_p))
_resampler_destroy = _sig("logmel_resampler_destroy", None, _p)
_resampler_info = _sig("logmel_resampler_info", ctypes.c_int, _p, _i64p, _i64p)
_resample = _sig("logmel_resample", ctypes.c_int, _p, _p, ctypes.c_int, _p, _p, _i64, _i64, _p,
                 _p)

EXPORTED = [
    "logmel_default_config", "logmel_abi_version", "logmel_status_string",
    "logmel_plan_create", "logmel_plan_destroy", "logmel_num_frames",
    "logmel_frame_offsets", "logmel_compute", "logmel_chunk_offsets", "logmel_chunk_frames",
    "logmel_compute_chunked", "logmel_compute_ex", "logmel_stream_create",
    "logmel_stream_destroy", "logmel_stream_reset", "logmel_stream_frames_for_push",
    "logmel_stream_push", "logmel_stream_push_ex", "logmel_stream_counters",
    "logmel_stream_create_ex", "logmel_stream_frames_for_flush", "logmel_stream_flush", "logmel_stream_state_bytes",
    "logmel_stream_get_state", "logmel_stream_set_state", "logmel_resample_length",
    "logmel_resample_offsets", "logmel_resampler_create", "logmel_resampler_destroy",
    "logmel_resampler_info", "logmel_resample", "logmel_stream_push_static",
]

STATIC_MAX_STREAMS = 512   # LOGMEL_STATIC_MAX_STREAMS
STATIC_MAX_PUSH = 2560     # LOGMEL_STATIC_MAX_PUSH


class LogmelError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {logmel_status_string(status)} ({status})")


def _check(status: int, what: str):
    if status != LOGMEL_OK:
        raise LogmelError(status, what)


def _i64_array(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64).reshape(-1))


def _ptr64(a: np.ndarray):
    return a.ctypes.data_as(_i64p)


# ------------------------------------------------------------------ basics

def logmel_abi_version() -> int:
    return int(_abi_version())


def logmel_status_string(status: int) -> str:
    return _status_string(int(status)).decode()


def logmel_default_config(device: int = 0) -> logmel_config:
    cfg = logmel_config()
    _default_config(ctypes.byref(cfg))
    cfg.device = int(device)
    return cfg


def logmel_num_frames(n_samples: int) -> int:
    return int(_num_frames(int(n_samples)))


def logmel_frame_offsets(sample_offsets) -> np.ndarray:
    so = _i64_array(sample_offsets)
    if so.size < 1:
        raise LogmelError(LOGMEL_ERR_INVALID_ARGUMENT, "logmel_frame_offsets")
    fo = np.zeros(so.size, dtype=np.int64)
    _check(_frame_offsets(_ptr64(so), so.size - 1, _ptr64(fo)), "logmel_frame_offsets")
    return fo


def logmel_chunk_offsets(sample_offsets) -> np.ndarray:
    """Exclusive prefix sum of the clips' 30-s chunk counts (int64, n_clips + 1)."""
    so = _i64_array(sample_offsets)
    if so.size < 1:
        raise LogmelError(LOGMEL_ERR_INVALID_ARGUMENT, "logmel_chunk_offsets")
    co = np.zeros(so.size, dtype=np.int64)
    _check(_chunk_offsets(_ptr64(so), so.size - 1, _ptr64(co)), "logmel_chunk_offsets")
    return co


def logmel_chunk_frames(sample_offsets, total_chunks: int) -> np.ndarray:
    """Frames held by each 30-s chunk (int64, total_chunks)."""
    so = _i64_array(sample_offsets)
    if so.size < 1:
        raise LogmelError(LOGMEL_ERR_INVALID_ARGUMENT, "logmel_chunk_frames")
    cf = np.zeros(max(int(total_chunks), 1), dtype=np.int64)
    _check(_chunk_frames(_ptr64(so), so.size - 1, int(total_chunks), _ptr64(cf)),
           "logmel_chunk_frames")
    return cf[:int(total_chunks)]


class Plan:
    """Owns a logmel_plan handle."""

    def __init__(self, cfg: logmel_config):
        h = _p()
        _check(_plan_create(ctypes.byref(cfg), ctypes.byref(h)), "logmel_plan_create")
        self.handle = h
        self.device = int(cfg.device)
        # kept on the object: at interpreter exit the module's globals may be
        # gone before __del__ runs
        self._destroy = _plan_destroy

    def close(self):
        if getattr(self, "handle", None):
            self._destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()


def logmel_plan_create(device: int = 0, cfg: logmel_config | None = None) -> Plan:
    return Plan(cfg if cfg is not None else logmel_default_config(device))


def logmel_plan_destroy(plan: Plan):
    plan.close()


# ----------------------------------------------------------- device glue

def _torch():
    import torch
    return torch


def _dev_ptr(t, dtype, what):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a torch tensor on a ROCm device")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def logmel_compute(plan: Plan, samples, sample_offsets, frame_offsets, total_frames: int,
                   out=None, stream=None):
    """Offline log-mel of a packed ragged batch; returns out [total_frames, 128].

    samples fp32, sample_offsets / frame_offsets int64 [n_clips + 1], all on
    the plan's device; the call is asynchronous on ``stream`` (default: the
    current torch stream)."""
    torch = _torch()
    n_clips = int(sample_offsets.numel()) - 1
    if out is None:
        out = torch.empty((int(total_frames), N_MELS), dtype=torch.float32,
                          device=samples.device)
    if tuple(out.shape) != (int(total_frames), N_MELS):
        raise ValueError(f"out must be [{total_frames}, {N_MELS}]")
    if frame_offsets.numel() != n_clips + 1:
        raise ValueError("frame_offsets must have n_clips + 1 entries")
    st = _stream_handle(stream, samples.device)
    _check(_compute(plan.handle, _dev_ptr(samples, torch.float32, "samples"),
                    _dev_ptr(sample_offsets, torch.int64, "sample_offsets"),
                    _dev_ptr(frame_offsets, torch.int64, "frame_offsets"),
                    n_clips, int(total_frames), _dev_ptr(out, torch.float32, "out"), st),
           "logmel_compute")
    return out


def logmel_compute_chunked(plan: Plan, samples, sample_offsets, frame_offsets, chunk_offsets,
                           total_frames: int, total_chunks: int, out=None, stream=None):
    """logmel_compute into the 30-s chunk layout; returns out
    [total_chunks, 3000, 128] (frame f of clip i at flat row
    chunk_offsets[i] * 3000 + f, the rest of a clip's last chunk ln(1e-10))."""
    torch = _torch()
    n_clips = int(sample_offsets.numel()) - 1
    if out is None:
        out = torch.empty((int(total_chunks), CHUNK_FRAMES, N_MELS), dtype=torch.float32,
                          device=samples.device)
    if tuple(out.shape) != (int(total_chunks), CHUNK_FRAMES, N_MELS):
        raise ValueError(f"out must be [{total_chunks}, {CHUNK_FRAMES}, {N_MELS}]")
    if frame_offsets.numel() != n_clips + 1 or chunk_offsets.numel() != n_clips + 1:
        raise ValueError("frame_offsets and chunk_offsets must have n_clips + 1 entries")
    st = _stream_handle(stream, samples.device)
    _check(_compute_chunked(plan.handle, _dev_ptr(samples, torch.float32, "samples"),
                            _dev_ptr(sample_offsets, torch.int64, "sample_offsets"),
                            _dev_ptr(frame_offsets, torch.int64, "frame_offsets"),
                            _dev_ptr(chunk_offsets, torch.int64, "chunk_offsets"),
                            n_clips, int(total_frames), int(total_chunks),
                            _dev_ptr(out, torch.float32, "out"), st),
           "logmel_compute_chunked")
    return out


def logmel_compute_ex(plan: Plan, samples, sample_offsets, frame_offsets, total_frames: int,
                      chunk_offsets=None, total_chunks: int = 0, out=None, out_dtype=None,
                      stream=None):
    """The general offline call: samples fp32 or int16 (s / 32768), output
    fp32 or fp16 (out_dtype, default fp32), frame layout [total_frames, 128]
    or, with chunk_offsets, the 30-s chunk layout [total_chunks, 3000, 128]."""
    torch = _torch()
    n_clips = int(sample_offsets.numel()) - 1
    if samples.dtype == torch.float32:
        st_in = LOGMEL_F32
    elif samples.dtype == torch.int16:
        st_in = LOGMEL_I16
    else:
        raise TypeError(f"samples must be float32 or int16, got {samples.dtype}")
    out_dtype = out_dtype or (out.dtype if out is not None else torch.float32)
    if out_dtype == torch.float32:
        st_out = LOGMEL_F32
    elif out_dtype == torch.float16:
        st_out = LOGMEL_F16
    else:
        raise TypeError(f"output must be float32 or float16, got {out_dtype}")
    shape = ((int(total_chunks), CHUNK_FRAMES, N_MELS) if chunk_offsets is not None
             else (int(total_frames), N_MELS))
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=samples.device)
    if tuple(out.shape) != shape:
        raise ValueError(f"out must be {list(shape)}")
    if frame_offsets.numel() != n_clips + 1:
        raise ValueError("frame_offsets must have n_clips + 1 entries")
    if chunk_offsets is not None and chunk_offsets.numel() != n_clips + 1:
        raise ValueError("chunk_offsets must have n_clips + 1 entries")
    st = _stream_handle(stream, samples.device)
    _check(_compute_ex(plan.handle, _dev_ptr(samples, samples.dtype, "samples"), st_in,
                       _dev_ptr(sample_offsets, torch.int64, "sample_offsets"),
                       _dev_ptr(frame_offsets, torch.int64, "frame_offsets"),
                       (None if chunk_offsets is None
                        else _dev_ptr(chunk_offsets, torch.int64, "chunk_offsets")),
                       n_clips, int(total_frames), int(total_chunks),
                       _dev_ptr(out, out_dtype, "out"), st_out, st),
           "logmel_compute_ex")
    return out


def log_mel(plan: Plan, samples, sample_offsets_host, stream=None):
    """Convenience: host int64 sample offsets in, [frames, 128] out.

    Computes the frame offsets with the C helper and uploads both offset
    arrays with torch."""
    torch = _torch()
    so = _i64_array(sample_offsets_host)
    fo = logmel_frame_offsets(so)
    dev = samples.device
    so_d = torch.from_numpy(so).to(dev)
    fo_d = torch.from_numpy(fo).to(dev)
    return logmel_compute(plan, samples, so_d, fo_d, int(fo[-1]), stream=stream), fo


# --------------------------------------------------------------- streaming

class Stream:
    """Owns a logmel_stream handle (n_streams independent streams)."""

    def __init__(self, plan: Plan, n_streams: int, max_push: int, in_rate: int = SAMPLE_RATE):
        h = _p()
        _check(_stream_create_ex(plan.handle, int(n_streams), int(max_push), int(in_rate),
                                 ctypes.byref(h)),
               "logmel_stream_create_ex")
        self.handle = h
        self.plan = plan
        self.n_streams = int(n_streams)
        self.max_push = int(max_push)
        self.in_rate = int(in_rate)
        self._destroy = _stream_destroy
        # Host arrays a push reuses (push lengths, frame offsets) and their
        # addresses, so that a push marshals no new numpy or ctypes objects.
        self._pl = np.zeros(self.n_streams, dtype=np.int64)
        self._fo = np.zeros(self.n_streams + 1, dtype=np.int64)
        self._pl_p = _ptr64(self._pl)
        self._fo_p = _ptr64(self._fo)

    def close(self):
        if getattr(self, "handle", None):
            self._destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()


def logmel_stream_create(plan: Plan, n_streams: int, max_push: int,
                         in_rate: int = SAMPLE_RATE) -> Stream:
    """n_streams streams taking up to max_push samples per push at in_rate
    (other rates than 16 kHz are resampled on the device)."""
    return Stream(plan, n_streams, max_push, in_rate)


def logmel_stream_frames_for_flush(s: Stream) -> np.ndarray:
    fo = np.zeros(s.n_streams + 1, dtype=np.int64)
    _check(_stream_frames_for_flush(s.handle, _ptr64(fo)), "logmel_stream_frames_for_flush")
    return fo


def logmel_stream_flush(s: Stream, out=None, out_dtype=None, stream=None, device=None):
    """Ends every stream (emitting what only the end of the input completes)
    and resets them; returns (out [frames, 128], frame offsets)."""
    torch = _torch()
    out_dtype = out_dtype or (out.dtype if out is not None else torch.float32)
    if out_dtype == torch.float32:
        st_out = LOGMEL_F32
    elif out_dtype == torch.float16:
        st_out = LOGMEL_F16
    else:
        raise TypeError(f"output must be float32 or float16, got {out_dtype}")
    fo = logmel_stream_frames_for_flush(s)
    total = int(fo[-1])
    dev = device if device is not None else torch.device("cuda", s.plan.device)
    if out is None:
        out = torch.empty((total, N_MELS), dtype=out_dtype, device=dev)
    if tuple(out.shape) != (total, N_MELS):
        raise ValueError(f"out must be [{total}, {N_MELS}]")
    st = _stream_handle(stream, dev)
    fo2 = np.zeros(s.n_streams + 1, dtype=np.int64)
    ptr = _dev_ptr(out, out_dtype, "out") if out.numel() else None
    _check(_stream_flush(s.handle, ptr, st_out, _ptr64(fo2), st), "logmel_stream_flush")
    return out, fo2


def logmel_stream_destroy(s: Stream):
    s.close()


def logmel_stream_reset(s: Stream):
    _check(_stream_reset(s.handle), "logmel_stream_reset")


def logmel_stream_frames_for_push(s: Stream, push_len) -> np.ndarray:
    pl = _i64_array(push_len)
    if pl.size != s.n_streams:
        raise ValueError("push_len must have n_streams entries")
    fo = np.zeros(s.n_streams + 1, dtype=np.int64)
    _check(_stream_frames_for_push(s.handle, _ptr64(pl), _ptr64(fo)),
           "logmel_stream_frames_for_push")
    return fo


def logmel_stream_push_static(plan, new_samples, push_len, out, reset=False, stream=None):
    """Pushes fp32 samples to the first len(push_len) streams kept in the
    library's fixed device array (no stream object, nothing allocated by the
    call). ``out`` is a caller-provided fp32 [rows, 128] buffer with room for
    every frame of the push (at most ceil(push_len / 160) per stream); the
    push writes its first fo[-1] rows. Returns the frame offsets fo."""
    torch = _torch()
    pl = _i64_array(push_len)
    if int(pl.sum()) != int(new_samples.numel()):
        raise ValueError("new_samples must hold sum(push_len) samples")
    if out.dim() != 2 or out.shape[1] != N_MELS:
        raise ValueError(f"out must be [rows, {N_MELS}]")
    st = _stream_handle(stream, new_samples.device)
    fo = np.zeros(pl.size + 1, dtype=np.int64)
    _check(_stream_push_static(plan.handle, pl.size,
                               _dev_ptr(new_samples, torch.float32, "new_samples"), _ptr64(pl),
                               1 if reset else 0, _dev_ptr(out, torch.float32, "out"),
                               int(out.shape[0]), _ptr64(fo), st),
           "logmel_stream_push_static")
    return fo


def logmel_stream_push(s: Stream, new_samples, push_len, out=None, stream=None, out_dtype=None):
    """Pushes packed new samples; returns (out [frames, 128], frame offsets).

    new_samples fp32 or int16 (s / 32768); output fp32 or fp16 (out_dtype,
    default fp32, or out's dtype). ``out`` may have more rows than the push
    emits (a buffer sized once for the largest push): the push writes its
    first fo[-1] rows and returns a view of them."""
    torch = _torch()
    pl = s._pl
    try:
        ok = len(push_len) == s.n_streams
    except TypeError:
        ok = False
    if not ok:
        raise ValueError("push_len must have n_streams entries")
    pl[...] = push_len
    if int(pl.sum()) != new_samples.numel():
        raise ValueError("new_samples must hold sum(push_len) samples")
    dt = new_samples.dtype
    if dt == torch.float32:
        st_in = LOGMEL_F32
    elif dt == torch.int16:
        st_in = LOGMEL_I16
    else:
        raise TypeError(f"new_samples must be float32 or int16, got {dt}")
    out_dtype = out_dtype or (out.dtype if out is not None else torch.float32)
    if out_dtype == torch.float32:
        st_out = LOGMEL_F32
    elif out_dtype == torch.float16:
        st_out = LOGMEL_F16
    else:
        raise TypeError(f"output must be float32 or float16, got {out_dtype}")
    _check(_stream_frames_for_push(s.handle, s._pl_p, s._fo_p), "logmel_stream_frames_for_push")
    total = int(s._fo[-1])
    if out is None:
        out = torch.empty((total, N_MELS), dtype=out_dtype, device=new_samples.device)
    if out.dim() != 2 or out.shape[1] != N_MELS or out.shape[0] < total:
        raise ValueError(f"out must be [rows >= {total}, {N_MELS}]")
    st = _stream_handle(stream, new_samples.device)
    d_new = _dev_ptr(new_samples, dt, "new_samples")
    d_out = _dev_ptr(out, out_dtype, "out")
    if st_in == LOGMEL_F32 and st_out == LOGMEL_F32:
        _check(_stream_push(s.handle, d_new, s._pl_p, d_out, s._fo_p, st), "logmel_stream_push")
    else:
        _check(_stream_push_ex(s.handle, d_new, st_in, s._pl_p, d_out, st_out, s._fo_p, st),
               "logmel_stream_push_ex")
    return (out if out.shape[0] == total else out[:total]), s._fo.copy()


def logmel_stream_counters(s: Stream, j: int):
    a, b = _i64(), _i64()
    _check(_stream_counters(s.handle, int(j), ctypes.byref(a), ctypes.byref(b)),
           "logmel_stream_counters")
    return int(a.value), int(b.value)


def logmel_stream_state_bytes(s: Stream) -> int:
    return int(_stream_state_bytes(s.handle))


def logmel_stream_get_state(s: Stream, stream=None) -> bytes:
    buf = ctypes.create_string_buffer(logmel_stream_state_bytes(s))
    st = _stream_handle(stream, None)
    _check(_stream_get_state(s.handle, ctypes.cast(buf, _p), st), "logmel_stream_get_state")
    return buf.raw


def logmel_stream_set_state(s: Stream, state: bytes, stream=None):
    if len(state) != logmel_stream_state_bytes(s):
        raise ValueError("state blob has the wrong size")
    buf = ctypes.create_string_buffer(state, len(state))
    st = _stream_handle(stream, None)
    _check(_stream_set_state(s.handle, ctypes.cast(buf, _p), st), "logmel_stream_set_state")


# ------------------------------------------------------- resampling to 16 kHz

def logmel_resample_length(n_samples: int, in_rate: int) -> int:
    """ceil(16000 n / in_rate); -1 for an unsupported rate or length."""
    return int(_resample_length(int(n_samples), int(in_rate)))


def logmel_resample_offsets(sample_offsets, in_rate: int) -> np.ndarray:
    """Exclusive prefix sum of the clips' 16 kHz output lengths (int64)."""
    so = _i64_array(sample_offsets)
    if so.size < 1:
        raise LogmelError(LOGMEL_ERR_INVALID_ARGUMENT, "logmel_resample_offsets")
    oo = np.zeros(so.size, dtype=np.int64)
    _check(_resample_offsets(int(in_rate), _ptr64(so), so.size - 1, _ptr64(oo)),
           "logmel_resample_offsets")
    return oo


class Resampler:
    """Owns a logmel_resampler handle (one input rate)."""

    def __init__(self, plan: Plan, in_rate: int):
        h = _p()
        _check(_resampler_create(plan.handle, int(in_rate), ctypes.byref(h)),
               "logmel_resampler_create")
        self.handle = h
        self.plan = plan
        self.rate = int(in_rate)
        self._destroy = _resampler_destroy

    def close(self):
        if getattr(self, "handle", None):
            self._destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()


def logmel_resampler_create(plan: Plan, in_rate: int) -> Resampler:
    return Resampler(plan, in_rate)


def logmel_resampler_destroy(r: Resampler):
    r.close()


def logmel_resampler_info(r: Resampler):
    """(phases L, taps per phase)."""
    a, b = _i64(), _i64()
    _check(_resampler_info(r.handle, ctypes.byref(a), ctypes.byref(b)), "logmel_resampler_info")
    return int(a.value), int(b.value)


def logmel_resample(r: Resampler, samples, sample_offsets, out_offsets, total_out: int,
                    out=None, stream=None):
    """Resamples a packed batch (fp32 or int16 samples, int64 offsets on the
    device) to 16 kHz; returns out fp32 [total_out]."""
    torch = _torch()
    n_clips = int(sample_offsets.numel()) - 1
    if samples.dtype == torch.float32:
        st_in = LOGMEL_F32
    elif samples.dtype == torch.int16:
        st_in = LOGMEL_I16
    else:
        raise TypeError(f"samples must be float32 or int16, got {samples.dtype}")
    if out is None:
        out = torch.empty(int(total_out), dtype=torch.float32, device=samples.device)
    if tuple(out.shape) != (int(total_out),):
        raise ValueError(f"out must be [{total_out}]")
    if out_offsets.numel() != n_clips + 1:
        raise ValueError("out_offsets must have n_clips + 1 entries")
    st = _stream_handle(stream, samples.device)
    _check(_resample(r.handle, _dev_ptr(samples, samples.dtype, "samples"), st_in,
                     _dev_ptr(sample_offsets, torch.int64, "sample_offsets"),
                     _dev_ptr(out_offsets, torch.int64, "out_offsets"), n_clips, int(total_out),
                     _dev_ptr(out, torch.float32, "out"), st),
           "logmel_resample")
    return out


def resample(r: Resampler, samples, sample_offsets_host, stream=None):
    """Convenience: host int64 sample offsets in; returns (16 kHz samples,
    their host offsets)."""
    torch = _torch()
    so = _i64_array(sample_offsets_host)
    oo = logmel_resample_offsets(so, r.rate)
    dev = samples.device
    y = logmel_resample(r, samples, torch.from_numpy(so).to(dev), torch.from_numpy(oo).to(dev),
                        int(oo[-1]), stream=stream)
    return y, oo
