// C-ABI layer of the log-mel library: argument checks, integer frame
// arithmetic, the stream objects' host shadow state, and kernel launches.
// The declarations and their contracts are in include/logmel.h.
#include "logmel.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "logmel_launch.h"
#include "logmel_resample_launch.h"
#include "logmel_slots.h"

namespace {

constexpr int kNFFT = 400;
constexpr int kHop = 160;
constexpr int kMels = 128;
constexpr int64_t kChunkFrames = LOGMEL_CHUNK_FRAMES;   // 30 s of 10 ms frames
constexpr int kRing = 400;  // carry capacity in front of each workspace row

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

bool env_validate() {
  const char* v = std::getenv("LOGMEL_VALIDATE");
  return v && v[0] && v[0] != '0';
}

int64_t frames_of(int64_t n) { return n < kNFFT ? 0 : (n - kNFFT) / kHop + 1; }

}  // namespace

// fp64 tables, computed by gen_tables.py from the definitions.
static const double kHostWindow[200] = {
#include "logmel_window.inc"
};
static const double kHostRot400[200] = {
#include "logmel_rot400.inc"
};

struct logmel_plan {
  logmel_config cfg;
  double* tables = nullptr;  // device, kTabBytes
  int resident_waves = 0;    // wavefronts of the transform kernel resident at once: one per SIMD
};

// ---------------------------------------------------------------------------
// Resampling to 16 kHz: a Kaiser-windowed sinc (the reading and its
// parameters are stated in logmel.h).
// ---------------------------------------------------------------------------

namespace {

constexpr int kResZeros = LOGMEL_RESAMPLE_ZEROS;
constexpr double kResRolloff = 0.96;
constexpr double kResBeta = 9.0;
constexpr int32_t kResMinRate = 1000;
constexpr int32_t kResMaxRate = 384000;

int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Modified Bessel function of the first kind, order 0, by its power series
// sum_k ((x / 2)^k / k!)^2 (all terms positive; converges for any x).
double bessel_i0(double x) {
  const double h = 0.5 * x;
  double term = 1.0, sum = 1.0;
  for (int k = 1; k < 500; ++k) {
    term *= (h / k) * (h / k);
    sum += term;
    if (term < 1e-17 * sum) break;
  }
  return sum;
}

struct ResGeometry {
  int64_t L, M;   // 16000 / R = L / M in lowest terms
  int J;          // taps j = 0 .. 2J cover input samples q - J .. q + J
  int Tp;         // 2J + 1 rounded up to a multiple of 16 (host table row length)
  double fc, H;   // cutoff (Hz) and half-width (input samples)
  RsmGeometry k;  // the matrix-core kernel's geometry; k.NT == 0: unsupported
  std::vector<int> gbase;   // per column group, floor(16 g M / L)
  std::vector<int> abase;   // its LDS offset from its super-period's first float
};

// The tile shape for NT row blocks (the other fields of k set; abase_max:
// the last column group's window offset in LDS floats).
void rsm_set_tiles(RsmGeometry& k, int64_t abase_max, int64_t NT, bool pair_blocks = true) {
  k.NT = (int)NT;
  // two row blocks per item share one read of the taps, when that still
  // leaves an item for each of the four wavefronts
  k.RB = pair_blocks && NT % 2 == 0 && k.C * NT / 2 >= 4 ? 2 : 1;
  k.span = (int)((16 * NT - 1) * k.P + abase_max + 4 * k.KS);
  k.TB = NT * 16 * k.S;
}

ResGeometry res_geometry(int32_t rate) {
  ResGeometry g;
  const int64_t d = gcd64(rate, 16000);
  g.L = 16000 / d;
  g.M = rate / d;
  g.fc = kResRolloff * (rate < 16000 ? rate : 16000) / 2.0;
  g.H = kResZeros * (double)rate / (2.0 * g.fc);
  g.J = rate == 16000 ? 0 : (int)std::ceil(g.H);
  g.Tp = (2 * g.J + 1 + 15) / 16 * 16;
  RsmGeometry& k = g.k;
  k = RsmGeometry{0, 0, 0, 0, 0, 1, g.J, 0, 0, 0};
  // super-periods of S = lcm(L, 16) outputs, S M / L input samples apart
  const int64_t S = g.L / gcd64(g.L, 16) * 16;
  const int64_t S_in = S / g.L * g.M;
  const int64_t C = S / 16;
  if (S > (1 << 20) || S_in > kRsmLdsMax) return g;   // too many phases, or too sparse
  // staged super-periods P floats apart: with 32 | S_in the 16 rows of an
  // MFMA operand would all start in one of the 32 banks (32, 64, 96 and
  // 192 kHz); two zero floats after each make P = 2 mod 4, 16 distinct even
  // banks (32 kHz 285 -> 195 us, 96 kHz 749 -> 478 us on the 64 x 30 s
  // batch). Where 32 does not divide S_in the conflicts are milder and the
  // pad floats' staging costs more than they save (8 kHz 83 -> 118 us).
  const int64_t P = S_in % 32 == 0 ? S_in + 2 : S_in;
  auto lds_of = [&](int64_t u) { return u / S_in * P + u % S_in; };
  const int64_t T = 2 * g.J + 1;
  g.gbase.resize((size_t)C);
  g.abase.resize((size_t)C);
  int64_t t_max = 0;
  for (int64_t gm = 0; gm < C; ++gm) {
    const int64_t gb = (16 * gm * g.M) / g.L;
    const int64_t dd = ((16 * gm + 15) * g.M) / g.L - gb;
    g.gbase[(size_t)gm] = (int)gb;
    g.abase[(size_t)gm] = (int)lds_of(gb);
    const int64_t t_end = lds_of(gb + dd + T - 1) + 1 - lds_of(gb);   // the group's window in LDS
    if (t_end > t_max) t_max = t_end;
  }
  // K / 4 MFMA steps cover every group's window (2J + 1 + its spread, plus
  // pad floats), padded to whole chunks of 8 steps
  const int64_t KS = ((t_max + 3) / 4 + 7) / 8 * 8;
  const int64_t abase_max = g.abase.back();
  auto span_of = [&](int64_t nt) { return (16 * nt - 1) * P + abase_max + 4 * KS; };
  int64_t NT = 1;
  if (span_of(1) > kRsmLdsMax) return g;
  while (NT < 8 && span_of(2 * NT) <= kRsmLdsSmall) NT *= 2;   // 1, 2, 4 or 8 row blocks
  k.S = (int)S;
  k.S_in = (int)S_in;
  k.C = (int)C;
  k.KS = (int)KS;
  k.P = (int)P;
  rsm_set_tiles(k, abase_max, NT);
  return g;
}

// Taps table [L][Tp]: row phi, tap j < 2J + 1 is h(phi / L + J - j); the
// row's last Tp - 2J - 1 entries are zero.
std::vector<float> res_taps(int32_t rate, const ResGeometry& g) {
  const int T = 2 * g.J + 1;
  std::vector<float> t((size_t)(g.L * g.Tp), 0.0f);
  if (rate == 16000) {   // no resampling: the output is the input
    t[0] = 1.0f;
    return t;
  }
  const double i0b = bessel_i0(kResBeta);
  const double pi = 3.14159265358979323846;
  for (int64_t phi = 0; phi < g.L; ++phi) {
    for (int j = 0; j < T; ++j) {
      const double dd = ((double)phi / (double)g.L + g.J) - j;   // p - k, input samples
      const double r = dd / g.H;
      double h = 0.0;
      if (std::fabs(r) < 1.0) {
        const double u = 2.0 * g.fc * dd / rate;
        const double sinc = u == 0.0 ? 1.0 : std::sin(pi * u) / (pi * u);
        h = (2.0 * g.fc / rate) * sinc * bessel_i0(kResBeta * std::sqrt(1.0 - r * r)) / i0b;
      }
      t[(size_t)(phi * g.Tp + j)] = (float)h;
    }
  }
  return t;
}

// The matrix cores' B operand, [C][KS][64]: for column group g and step s,
// lane l holds W_g[4 s + l / 16][l % 16]. W_g[t][c] multiplies LDS float
// abase_g + t of a row: the tap of output r = 16 g + c (phase r M mod L) for
// the sample that float holds, i.e. the output's tap row shifted right by
// floor(r M / L) - floor(16 g M / L) samples; zero for pad floats and for
// samples outside the output's window.
std::vector<float> res_btab(const ResGeometry& g, const std::vector<float>& t) {
  const RsmGeometry& k = g.k;
  const int T = 2 * g.J + 1;
  std::vector<float> b((size_t)k.C * k.KS * 64, 0.0f);
  for (int64_t gm = 0; gm < k.C; ++gm)
    for (int c = 0; c < 16; ++c) {
      const int64_t r = 16 * gm + c;
      const int64_t phi = (r * g.M) % g.L;
      const int64_t d = (r * g.M) / g.L - g.gbase[(size_t)gm];
      for (int64_t tt = 0; tt < 4 * (int64_t)k.KS; ++tt) {
        const int64_t a = g.abase[(size_t)gm] + tt;   // LDS float of the row
        if (a % k.P >= k.S_in) continue;               // a pad float
        const int64_t u = a / k.P * k.S_in + a % k.P;   // its sample, from the row's first
        const int64_t j = u - g.gbase[(size_t)gm] - d;
        if (j < 0 || j >= T) continue;
        b[(size_t)((gm * k.KS + tt / 4) * 64 + (tt % 4) * 16 + c)] = t[(size_t)(phi * g.Tp + j)];
      }
    }
  return b;
}

// Largest taps table accepted (floats, device memory).
constexpr int64_t kResMaxTableFloats = int64_t(1) << 24;

bool res_rate_ok(int32_t rate) { return rate >= kResMinRate && rate <= kResMaxRate; }

}  // namespace

struct logmel_resampler {
  const logmel_plan* plan;
  int32_t rate;
  ResGeometry geo;
  float* btab = nullptr;   // device: the B operand [C][KS][64], then abase [C] int32
  int* abase = nullptr;    // inside the btab allocation
};

struct logmel_stream {
  const logmel_plan* plan;
  int64_t n;
  int64_t max_push;
  int64_t stride;              // floats per workspace row
  float* ws = nullptr;         // device [n][stride]
  int64_t* meta_dev = nullptr; // device [7n + 1]
  // Pinned staging ring for the per-push metadata, taken in order and
  // reused in groups of kSlotGroup: one event, recorded after the prep
  // kernel of a group's last slot, tells the host that the group's slots
  // have all been read (an event per push would put a packet of its own
  // between the kernels of every push).
  static constexpr int kSlots = 8;
  static constexpr int kSlotGroup = 4;
  static constexpr int kGroups = kSlots / kSlotGroup;
  int64_t* meta_host[kSlots] = {};
  int64_t* meta_host_dev[kSlots] = {};   // their device addresses
  hipEvent_t slot_done[kGroups] = {};
  int slot = 0;
  // host shadow, per stream
  std::vector<int64_t> seen, emitted, carry_len, carry_src;

  // Streams at another input rate: each push is resampled to 16 kHz first,
  // straight into the workspace rows above, whose frames are then
  // transformed as for a 16 kHz push. Per stream, the input
  // samples the next outputs' windows still need (at most 2J) are kept as a
  // carry, in one of two packed input buffers that alternate from push to
  // push.
  int32_t in_rate = 16000;
  logmel_resampler* rs = nullptr;
  RsmGeometry rs_k{};                   // its kernel's geometry for pushes (smaller tiles)
  int64_t in_max_push = 0;              // input samples per push and stream
  int64_t in_stride = 0;                // a stream's room in an input buffer
  float* in_buf[2] = {nullptr, nullptr};
  int in_cur = 0;                       // the buffer holding the carries
  int64_t* rmeta_dev = nullptr;         // [9n + 1], layout in rs_push
  int64_t* rmeta_host[kSlots] = {};      // the same ring for the resampling prep
  int64_t* rmeta_host_dev[kSlots] = {};
  hipEvent_t rslot_done[kGroups] = {};
  int rslot = 0;
  std::vector<int64_t> rs_in, rs_out, rcarry_len, rcarry_src;
};

namespace {

// Outputs of a clip whose whole window lies in its first n_in samples:
// the n with floor(n M / L) + J <= n_in - 1.
int64_t res_final(const ResGeometry& g, int64_t n_in) {
  const int64_t x = n_in - g.J;   // floor(n M / L) < x
  return x >= 1 ? ((x * g.L - 1) / g.M) + 1 : 0;
}

// 16 kHz outputs a push of p samples (or, with flush, the end of the stream)
// completes for stream j.
int64_t res_new_outputs(const logmel_stream* s, int64_t j, int64_t p, bool flush) {
  const int64_t n_in = s->rs_in[j] + p;
  const int64_t end = flush ? (n_in * 16000 + s->in_rate - 1) / s->in_rate
                            : res_final(s->rs->geo, n_in);
  return end - s->rs_out[j];
}

}  // namespace

extern "C" {

void logmel_default_config(logmel_config* cfg) {
  if (!cfg) return;
  cfg->sample_rate = 16000;
  cfg->n_fft = kNFFT;
  cfg->hop = kHop;
  cfg->n_mels = kMels;
  cfg->f_min = 0.0;
  cfg->f_max = 8000.0;
  cfg->log_floor = 1e-10;
  cfg->device = 0;
}

int logmel_abi_version(void) { return 1; }

const char* logmel_status_string(int status) {
  switch (status) {
    case LOGMEL_OK: return "ok";
    case LOGMEL_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LOGMEL_ERR_UNSUPPORTED: return "unsupported configuration";
    case LOGMEL_ERR_OUT_OF_MEMORY: return "out of memory";
    case LOGMEL_ERR_DEVICE: return "HIP runtime error";
    case LOGMEL_ERR_INPUT_TOO_LONG: return "input too long";
    default: return "unknown status";
  }
}

int logmel_plan_create(const logmel_config* cfg, logmel_plan** out) {
  if (!cfg || !out) return LOGMEL_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (cfg->sample_rate != 16000 || cfg->n_fft != kNFFT || cfg->hop != kHop ||
      cfg->n_mels != kMels || cfg->f_min != 0.0 || cfg->f_max != 8000.0 ||
      cfg->log_floor != 1e-10)
    return LOGMEL_ERR_UNSUPPORTED;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return LOGMEL_ERR_DEVICE;
  if (cfg->device < 0 || cfg->device >= ndev) return LOGMEL_ERR_INVALID_ARGUMENT;
  logmel_plan* p = new (std::nothrow) logmel_plan;
  if (!p) return LOGMEL_ERR_OUT_OF_MEMORY;
  p->cfg = *cfg;
  DeviceGuard g(cfg->device);
  if (!g.ok) {
    delete p;
    return LOGMEL_ERR_DEVICE;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, cfg->device) !=
          hipSuccess || cus <= 0) {
    delete p;
    return LOGMEL_ERR_DEVICE;
  }
  p->resident_waves = 4 * cus;   // 4 SIMDs per compute unit
  double host[kTabDoubles];
  std::memcpy(host + kTabWindow, kHostWindow, sizeof(kHostWindow));
  std::memcpy(host + kTabRot400, kHostRot400, sizeof(kHostRot400));
  if (hipMalloc(&p->tables, kTabBytes) != hipSuccess) {
    delete p;
    return LOGMEL_ERR_OUT_OF_MEMORY;
  }
  if (hipMemset(p->tables, 0, kTabBytes) != hipSuccess ||
      hipMemcpy(p->tables, host, sizeof(host), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(p->tables);
    delete p;
    return LOGMEL_ERR_DEVICE;
  }
  *out = p;
  return LOGMEL_OK;
}

void logmel_plan_destroy(logmel_plan* plan) {
  if (!plan) return;
  if (plan->tables) {
    DeviceGuard g(plan->cfg.device);
    (void)hipFree(plan->tables);
  }
  delete plan;
}

int64_t logmel_num_frames(int64_t n_samples) { return frames_of(n_samples); }

int logmel_frame_offsets(const int64_t* so, int64_t n_clips, int64_t* fo) {
  if (!so || !fo || n_clips < 0) return LOGMEL_ERR_INVALID_ARGUMENT;
  if (so[0] != 0) return LOGMEL_ERR_INVALID_ARGUMENT;
  for (int64_t i = 0; i < n_clips; ++i)
    if (so[i + 1] < so[i]) return LOGMEL_ERR_INVALID_ARGUMENT;
  int64_t acc = 0;
  fo[0] = 0;
  for (int64_t i = 0; i < n_clips; ++i) {
    acc += frames_of(so[i + 1] - so[i]);
    fo[i + 1] = acc;
  }
  return LOGMEL_OK;
}

int logmel_chunk_offsets(const int64_t* so, int64_t n_clips, int64_t* co) {
  if (!so || !co || n_clips < 0) return LOGMEL_ERR_INVALID_ARGUMENT;
  if (so[0] != 0) return LOGMEL_ERR_INVALID_ARGUMENT;
  for (int64_t i = 0; i < n_clips; ++i)
    if (so[i + 1] < so[i]) return LOGMEL_ERR_INVALID_ARGUMENT;
  int64_t acc = 0;
  co[0] = 0;
  for (int64_t i = 0; i < n_clips; ++i) {
    acc += (frames_of(so[i + 1] - so[i]) + kChunkFrames - 1) / kChunkFrames;
    co[i + 1] = acc;
  }
  return LOGMEL_OK;
}

int logmel_chunk_frames(const int64_t* so, int64_t n_clips, int64_t total_chunks, int64_t* cf) {
  if (!so || !cf || n_clips < 0 || total_chunks < 0) return LOGMEL_ERR_INVALID_ARGUMENT;
  std::vector<int64_t> co(n_clips + 1);
  const int r = logmel_chunk_offsets(so, n_clips, co.data());
  if (r != LOGMEL_OK) return r;
  if (co[n_clips] != total_chunks) return LOGMEL_ERR_INVALID_ARGUMENT;
  for (int64_t i = 0; i < n_clips; ++i) {
    const int64_t F = frames_of(so[i + 1] - so[i]);
    for (int64_t j = co[i]; j < co[i + 1]; ++j) {
      const int64_t left = F - (j - co[i]) * kChunkFrames;
      cf[j] = left < kChunkFrames ? left : kChunkFrames;
    }
  }
  return LOGMEL_OK;
}

namespace {

// Reads offsets back (one synchronisation) and checks them against the
// sample offsets; for LOGMEL_VALIDATE=1.
int validate_offsets(const int64_t* d_so, const int64_t* d_fo, const int64_t* d_co,
                     int64_t n_clips, int64_t total_frames, int64_t total_chunks,
                     hipStream_t st) {
  std::vector<int64_t> so(n_clips + 1), fo(n_clips + 1), co(n_clips + 1), ref(n_clips + 1);
  if (hipMemcpyAsync(so.data(), d_so, (n_clips + 1) * 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(fo.data(), d_fo, (n_clips + 1) * 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
      (d_co && hipMemcpyAsync(co.data(), d_co, (n_clips + 1) * 8, hipMemcpyDeviceToHost, st) !=
                   hipSuccess) ||
      hipStreamSynchronize(st) != hipSuccess)
    return LOGMEL_ERR_DEVICE;
  if (logmel_frame_offsets(so.data(), n_clips, ref.data()) != LOGMEL_OK)
    return LOGMEL_ERR_INVALID_ARGUMENT;
  if (ref != fo || fo[n_clips] != total_frames) return LOGMEL_ERR_INVALID_ARGUMENT;
  if (d_co) {
    if (logmel_chunk_offsets(so.data(), n_clips, ref.data()) != LOGMEL_OK)
      return LOGMEL_ERR_INVALID_ARGUMENT;
    if (ref != co || co[n_clips] != total_chunks) return LOGMEL_ERR_INVALID_ARGUMENT;
  }
  return LOGMEL_OK;
}

}  // namespace

int logmel_compute_ex(const logmel_plan* plan, const void* d_samples, int sample_type,
                      const int64_t* d_sample_offsets, const int64_t* d_frame_offsets,
                      const int64_t* d_chunk_offsets, int64_t n_clips, int64_t total_frames,
                      int64_t total_chunks, void* d_out, int out_type, void* hip_stream) {
  if (!plan || n_clips < 0 || total_frames < 0) return LOGMEL_ERR_INVALID_ARGUMENT;
  if (sample_type != LOGMEL_F32 && sample_type != LOGMEL_I16) return LOGMEL_ERR_UNSUPPORTED;
  if (out_type != LOGMEL_F32 && out_type != LOGMEL_F16) return LOGMEL_ERR_UNSUPPORTED;
  const bool chunked = d_chunk_offsets != nullptr;
  int64_t out_rows = total_frames;
  if (chunked) {
    if (total_chunks < 0) return LOGMEL_ERR_INVALID_ARGUMENT;
    if (total_chunks > INT64_MAX / (kChunkFrames * kMels)) return LOGMEL_ERR_INPUT_TOO_LONG;
    if (total_frames > total_chunks * kChunkFrames) return LOGMEL_ERR_INVALID_ARGUMENT;
    out_rows = total_chunks * kChunkFrames;
  } else if (total_frames > INT64_MAX / kMels) {
    return LOGMEL_ERR_INPUT_TOO_LONG;
  }
  if (n_clips == 0 || out_rows == 0) return LOGMEL_OK;
  if (!d_samples || !d_sample_offsets || !d_frame_offsets || !d_out)
    return LOGMEL_ERR_INVALID_ARGUMENT;
  // the kernels read samples with 4-byte aligned loads from the buffer start
  if (reinterpret_cast<uintptr_t>(d_samples) % 4 != 0) return LOGMEL_ERR_INVALID_ARGUMENT;
  DeviceGuard g(plan->cfg.device);
  if (!g.ok) return LOGMEL_ERR_DEVICE;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (env_validate()) {
    const int r = validate_offsets(d_sample_offsets, d_frame_offsets, d_chunk_offsets, n_clips,
                                   total_frames, total_chunks, st);
    if (r != LOGMEL_OK) return r;
  }
  const int out_f16 = out_type == LOGMEL_F16;
  if (chunked && logmel_launch_chunk_pad(d_out, out_f16, d_frame_offsets, d_chunk_offsets,
                                         n_clips, out_rows, st) != hipSuccess)
    return LOGMEL_ERR_DEVICE;
  const hipError_t e = logmel_launch_tiles(
      plan->tables, d_samples, sample_type == LOGMEL_I16, d_sample_offsets, d_sample_offsets + 1,
      d_frame_offsets, n_clips, total_frames, d_out, out_f16,
      chunked ? d_chunk_offsets : d_frame_offsets, chunked ? kChunkFrames : 1, out_rows,
      plan->resident_waves, st);
  return e == hipSuccess ? LOGMEL_OK : LOGMEL_ERR_DEVICE;
}

int logmel_compute(const logmel_plan* plan, const float* d_samples,
                   const int64_t* d_sample_offsets, const int64_t* d_frame_offsets,
                   int64_t n_clips, int64_t total_frames, float* d_out, void* hip_stream) {
  return logmel_compute_ex(plan, d_samples, LOGMEL_F32, d_sample_offsets, d_frame_offsets, nullptr,
                           n_clips, total_frames, 0, d_out, LOGMEL_F32, hip_stream);
}

int logmel_compute_chunked(const logmel_plan* plan, const float* d_samples,
                           const int64_t* d_sample_offsets, const int64_t* d_frame_offsets,
                           const int64_t* d_chunk_offsets, int64_t n_clips,
                           int64_t total_frames, int64_t total_chunks, float* d_out,
                           void* hip_stream) {
  if (!d_chunk_offsets) return LOGMEL_ERR_INVALID_ARGUMENT;
  return logmel_compute_ex(plan, d_samples, LOGMEL_F32, d_sample_offsets, d_frame_offsets,
                           d_chunk_offsets, n_clips, total_frames, total_chunks, d_out,
                           LOGMEL_F32, hip_stream);
}

// ---------------------------------------------------------------- streaming

int logmel_stream_create(const logmel_plan* plan, int64_t n_streams, int64_t max_push,
                         logmel_stream** out) {
  if (!plan || !out || n_streams < 1 || max_push < 1) return LOGMEL_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (n_streams > (1LL << 31) - 1) return LOGMEL_ERR_INPUT_TOO_LONG;
  int64_t stride = kRing + max_push;
  stride = (stride + 63) / 64 * 64;  // 256-byte aligned rows
  if (stride > INT64_MAX / n_streams / 4) return LOGMEL_ERR_INPUT_TOO_LONG;
  DeviceGuard g(plan->cfg.device);
  if (!g.ok) return LOGMEL_ERR_DEVICE;
  logmel_stream* s = new (std::nothrow) logmel_stream;
  if (!s) return LOGMEL_ERR_OUT_OF_MEMORY;
  s->plan = plan;
  s->n = n_streams;
  s->max_push = max_push;
  s->stride = stride;
  const size_t meta_words = 7 * (size_t)n_streams + 1;
  const size_t slot_words = kStreamMetaRec * (size_t)n_streams;
  bool ok = hipMalloc(&s->ws, (size_t)n_streams * stride * sizeof(float)) == hipSuccess &&
            hipMalloc(&s->meta_dev, meta_words * 8) == hipSuccess;
  for (int i = 0; ok && i < logmel_stream::kSlots; ++i)
    ok = hipHostMalloc(&s->meta_host[i], slot_words * 8, hipHostMallocDefault) == hipSuccess &&
         hipHostGetDevicePointer(reinterpret_cast<void**>(&s->meta_host_dev[i]), s->meta_host[i],
                                 0) == hipSuccess;
  for (int i = 0; ok && i < logmel_stream::kGroups; ++i)
    ok = hipEventCreateWithFlags(&s->slot_done[i], hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    logmel_stream_destroy(s);
    return LOGMEL_ERR_OUT_OF_MEMORY;
  }
  s->seen.assign(n_streams, 0);
  s->emitted.assign(n_streams, 0);
  s->carry_len.assign(n_streams, 0);
  s->carry_src.assign(n_streams, 0);
  for (int64_t j = 0; j < n_streams; ++j) s->carry_src[j] = j * stride + kRing;
  *out = s;
  return LOGMEL_OK;
}

void logmel_stream_destroy(logmel_stream* s) {
  if (!s) return;
  DeviceGuard g(s->plan->cfg.device);
  // The pushes of a group not yet closed by its event may still be reading
  // their slots: wait for the device before freeing them.
  if (s->slot % logmel_stream::kSlotGroup != 0 || s->rslot % logmel_stream::kSlotGroup != 0)
    (void)hipDeviceSynchronize();
  for (int i = 0; i < logmel_stream::kGroups; ++i) {
    if (s->slot_done[i]) {
      (void)hipEventSynchronize(s->slot_done[i]);
      (void)hipEventDestroy(s->slot_done[i]);
    }
    if (s->rslot_done[i]) {
      (void)hipEventSynchronize(s->rslot_done[i]);
      (void)hipEventDestroy(s->rslot_done[i]);
    }
  }
  for (int i = 0; i < logmel_stream::kSlots; ++i) {
    if (s->meta_host[i]) (void)hipHostFree(s->meta_host[i]);
    if (s->rmeta_host[i]) (void)hipHostFree(s->rmeta_host[i]);
  }
  if (s->ws) (void)hipFree(s->ws);
  if (s->meta_dev) (void)hipFree(s->meta_dev);
  for (int i = 0; i < 2; ++i)
    if (s->in_buf[i]) (void)hipFree(s->in_buf[i]);
  if (s->rmeta_dev) (void)hipFree(s->rmeta_dev);
  if (s->rs) logmel_resampler_destroy(s->rs);
  delete s;
}

int logmel_stream_create_ex(const logmel_plan* plan, int64_t n_streams, int64_t max_push,
                            int32_t in_rate, logmel_stream** out) {
  if (in_rate == 16000) return logmel_stream_create(plan, n_streams, max_push, out);
  if (!plan || !out || n_streams < 1 || max_push < 1) return LOGMEL_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  logmel_resampler* r = nullptr;
  int e = logmel_resampler_create(plan, in_rate, &r);
  if (e != LOGMEL_OK) return e;
  const ResGeometry& geo = r->geo;
  // 16 kHz samples one push can complete: those of its new input, one more
  // for rounding, and at the end of the stream those of the retained 2J.
  if (max_push > (INT64_MAX / 16) / geo.L) {
    logmel_resampler_destroy(r);
    return LOGMEL_ERR_INPUT_TOO_LONG;
  }
  const int64_t by_push = (max_push * geo.L + geo.M - 1) / geo.M + 2;
  const int64_t by_end = ((2 * geo.J + 2) * geo.L + geo.M - 1) / geo.M + 2;
  const int64_t max16 = by_push > by_end ? by_push : by_end;
  logmel_stream* s = nullptr;
  e = logmel_stream_create(plan, n_streams, max16, &s);
  if (e != LOGMEL_OK) {
    logmel_resampler_destroy(r);
    return e;
  }
  s->in_rate = in_rate;
  s->rs = r;
  // A push forms about max_push outputs per stream, mostly in partial tiles
  // at its segments' edges: tiles of half the offline height (where the
  // offline tiles have 4 or more row blocks) stage and work less for them
  // (48 kHz, 80 ms pushes: 70.6 -> 61.0 us; at 44.1 kHz, 2 -> 1 row blocks
  // cost more than they save), and one row block per item lets the kernel
  // skip the row blocks a push does not reach. An output's sum is the same
  // in any tile (same taps, same samples, same order of steps), so pushes
  // still equal offline resampling.
  s->rs_k = geo.k;
  rsm_set_tiles(s->rs_k, geo.abase.back(), geo.k.NT >= 4 ? geo.k.NT / 2 : geo.k.NT, false);
  s->in_max_push = max_push;
  s->in_stride = 2 * (int64_t)geo.J + 2 + max_push;
  if (s->in_stride > INT64_MAX / n_streams / 4) {
    logmel_stream_destroy(s);
    return LOGMEL_ERR_INPUT_TOO_LONG;
  }
  DeviceGuard g(plan->cfg.device);
  if (!g.ok) {
    logmel_stream_destroy(s);
    return LOGMEL_ERR_DEVICE;
  }
  const size_t rmeta_words = 9 * (size_t)n_streams + 1;
  bool ok = true;
  for (int i = 0; ok && i < 2; ++i)
    ok = hipMalloc(&s->in_buf[i], (size_t)n_streams * s->in_stride * sizeof(float)) == hipSuccess;
  ok = ok && hipMalloc(&s->rmeta_dev, rmeta_words * 8) == hipSuccess;
  for (int i = 0; ok && i < logmel_stream::kSlots; ++i)
    ok = hipHostMalloc(&s->rmeta_host[i], kRStreamMetaRec * (size_t)n_streams * 8,
                       hipHostMallocDefault) == hipSuccess &&
         hipHostGetDevicePointer(reinterpret_cast<void**>(&s->rmeta_host_dev[i]),
                                 s->rmeta_host[i], 0) == hipSuccess;
  for (int i = 0; ok && i < logmel_stream::kGroups; ++i)
    ok = hipEventCreateWithFlags(&s->rslot_done[i], hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    logmel_stream_destroy(s);
    return LOGMEL_ERR_OUT_OF_MEMORY;
  }
  s->rs_in.assign(n_streams, 0);
  s->rs_out.assign(n_streams, 0);
  s->rcarry_len.assign(n_streams, 0);
  s->rcarry_src.assign(n_streams, 0);
  *out = s;
  return LOGMEL_OK;
}

int logmel_stream_reset(logmel_stream* s) {
  if (!s) return LOGMEL_ERR_INVALID_ARGUMENT;
  for (int64_t j = 0; j < s->n; ++j) {
    s->seen[j] = 0;
    s->emitted[j] = 0;
    s->carry_len[j] = 0;
    s->carry_src[j] = j * s->stride + kRing;
  }
  for (size_t j = 0; j < s->rs_in.size(); ++j) {
    s->rs_in[j] = 0;
    s->rs_out[j] = 0;
    s->rcarry_len[j] = 0;
    s->rcarry_src[j] = 0;
  }
  return LOGMEL_OK;
}

int logmel_stream_frames_for_push(const logmel_stream* s, const int64_t* push_len,
                                  int64_t* fo) {
  if (!s || !push_len || !fo) return LOGMEL_ERR_INVALID_ARGUMENT;
  fo[0] = 0;
  for (int64_t j = 0; j < s->n; ++j) {
    if (push_len[j] < 0) return LOGMEL_ERR_INVALID_ARGUMENT;
    const int64_t p = s->rs ? res_new_outputs(s, j, push_len[j], false) : push_len[j];
    fo[j + 1] = fo[j] + frames_of(s->carry_len[j] + p);
  }
  return LOGMEL_OK;
}

int logmel_stream_frames_for_flush(const logmel_stream* s, int64_t* fo) {
  if (!s || !fo) return LOGMEL_ERR_INVALID_ARGUMENT;
  fo[0] = 0;
  for (int64_t j = 0; j < s->n; ++j) {
    const int64_t p = s->rs ? res_new_outputs(s, j, 0, true) : 0;
    fo[j + 1] = fo[j] + (s->rs ? frames_of(s->carry_len[j] + p) : 0);
  }
  return LOGMEL_OK;
}

int logmel_stream_push(logmel_stream* s, const float* d_new, const int64_t* push_len,
                       float* d_out, int64_t* fo_out, void* hip_stream) {
  return logmel_stream_push_ex(s, d_new, LOGMEL_F32, push_len, d_out, LOGMEL_F32, fo_out,
                               hip_stream);
}

namespace {

// The 16 kHz part of a push once its segments are in place (each stream's
// carry, then its push_len[j] new samples, from row j's float 400 - carry
// on, and the transform kernel's offsets in meta_dev): the transform of
// every completed frame into d_out (frame offsets fo), then the host shadow.
int lm_transform(logmel_stream* s, const int64_t* push_len, const std::vector<int64_t>& fo,
                 void* d_out, int out_type, int64_t* fo_out, hipStream_t st) {
  const int64_t n = s->n;
  const int64_t total_frames = fo[n];
  if (logmel_launch_tiles(s->plan->tables, s->ws, 0, s->meta_dev + 4 * n, s->meta_dev + 5 * n,
                          s->meta_dev + 6 * n, n, total_frames, d_out, out_type == LOGMEL_F16,
                          s->meta_dev + 6 * n, 1, total_frames, s->plan->resident_waves, st) !=
      hipSuccess)
    return LOGMEL_ERR_DEVICE;
  // Advance the host shadow.
  for (int64_t j = 0; j < n; ++j) {
    const int64_t c = s->carry_len[j], p = push_len[j];
    const int64_t F = frames_of(c + p);
    const int64_t seg0 = j * s->stride + kRing - c;
    s->carry_src[j] = seg0 + kHop * F;
    s->carry_len[j] = c + p - kHop * F;
    s->seen[j] += p;
    s->emitted[j] += F;
  }
  if (fo_out) std::memcpy(fo_out, fo.data(), (n + 1) * sizeof(int64_t));
  return LOGMEL_OK;
}

// The 16 kHz part of a push: push_len[j] <= max_push new samples per stream
// (checked by the caller), the device on.
int lm_push(logmel_stream* s, const void* d_new, int sample_type, const int64_t* push_len,
            void* d_out, int out_type, int64_t* fo_out, hipStream_t st) {
  const int64_t n = s->n;
  // Fill the next staging slot; at the first slot of a group, once the
  // group's previous pushes have read it.
  const int slot = s->slot, grp = slot / logmel_stream::kSlotGroup;
  const bool first = slot % logmel_stream::kSlotGroup == 0;
  const bool last = slot % logmel_stream::kSlotGroup == logmel_stream::kSlotGroup - 1;
  if (first && hipEventSynchronize(s->slot_done[grp]) != hipSuccess) return LOGMEL_ERR_DEVICE;
  // One record of kStreamMetaRec words per stream (a stream's fields in one
  // line of the pinned slot, read by its prep workgroup in one load):
  // carry index, carry length, offset and number of new samples, segment
  // start and end in the workspace, frame offset after the stream.
  int64_t* m = s->meta_host[slot];
  int64_t off = 0;
  std::vector<int64_t> fo(n + 1);
  fo[0] = 0;
  for (int64_t j = 0; j < n; ++j) {
    const int64_t c = s->carry_len[j];
    const int64_t p = push_len[j];
    const int64_t base = j * s->stride;
    int64_t* r = m + j * kStreamMetaRec;
    fo[j + 1] = fo[j] + frames_of(c + p);
    r[0] = s->carry_src[j];
    r[1] = c;
    r[2] = off;
    r[3] = p;
    r[4] = base + kRing - c;
    r[5] = base + kRing + p;
    r[6] = fo[j + 1];
    off += p;
  }
  const int64_t total_frames = fo[n];
  if (total_frames > INT64_MAX / kMels) return LOGMEL_ERR_INPUT_TOO_LONG;
  if (total_frames > 0 && !d_out) return LOGMEL_ERR_INVALID_ARGUMENT;
  // Every stream in the same state and pushing the same number of samples
  // (a fixed audio clock): the prep kernel derives the records from its
  // arguments and reads no host memory.
  StreamUniform uni{1, push_len[0], s->carry_len[0], s->carry_src[0], 0};
  for (int64_t j = 1; j < n && uni.on; ++j)
    uni.on = push_len[j] == uni.P && s->carry_len[j] == uni.c &&
             s->carry_src[j] - j * s->stride == uni.d;
  uni.F = frames_of(uni.c + uni.P);
  // Otherwise the prep kernel reads the slot in place (no copy engine in the
  // push's path). It hands the transform kernel its offsets in meta_dev.
  if (logmel_launch_stream_prep(s->ws, s->stride, d_new, sample_type == LOGMEL_I16,
                                s->meta_host_dev[slot], s->meta_dev, n, uni, st) != hipSuccess ||
      (last && hipEventRecord(s->slot_done[grp], st) != hipSuccess))
    return LOGMEL_ERR_DEVICE;
  s->slot = (slot + 1) % logmel_stream::kSlots;
  return lm_transform(s, push_len, fo, d_out, out_type, fo_out, st);
}

// The resampling part of a push (or, with flush, of the end of the
// streams): builds each stream's segment (carry, then the new samples) in
// the other input buffer and moves each stream's 16 kHz carry in its
// workspace row (one prep kernel), resamples every output the segment
// completes straight into the rows after those carries, and transforms the
// completed frames (lm_transform). Slot layout: one record of
// kRStreamMetaRec int64 per stream (one line of the pinned slot):
//   0 carry index in the carry buffer    1 carry length
//   2 offset of the new samples in d_new  3 number of new samples
//   4 segment start in the new buffer     5 buffer index of the clip's sample 0
//   6 segment end                         7 number of the first output
//   8 output offset after the stream      9 16 kHz carry index in the workspace
//  10 16 kHz carry length                11 16 kHz samples of the push
//  12 frame offset after the stream
static_assert(kRStreamMetaRec >= 13, "a resampling push's record has 13 fields");
int rs_push(logmel_stream* s, const void* d_new, int sample_type, const int64_t* push_len,
            void* d_out, int out_type, int64_t* fo_out, hipStream_t st, bool flush) {
  const int64_t n = s->n;
  const ResGeometry& geo = s->rs->geo;
  const int slot = s->rslot, grp = slot / logmel_stream::kSlotGroup;
  const bool first = slot % logmel_stream::kSlotGroup == 0;
  const bool last = slot % logmel_stream::kSlotGroup == logmel_stream::kSlotGroup - 1;
  if (first && hipEventSynchronize(s->rslot_done[grp]) != hipSuccess) return LOGMEL_ERR_DEVICE;
  int64_t* m = s->rmeta_host[slot];
  std::vector<int64_t> k(n), fo(n + 1);
  fo[0] = 0;
  int64_t seg = 0, noff = 0, total_k = 0;
  for (int64_t j = 0; j < n; ++j) {
    const int64_t c = s->rcarry_len[j];
    const int64_t p = flush ? 0 : push_len[j];
    int64_t* r = m + j * kRStreamMetaRec;
    k[j] = res_new_outputs(s, j, p, flush);
    if (k[j] < 0 || k[j] > s->max_push) return LOGMEL_ERR_INVALID_ARGUMENT;   // not reached
    total_k += k[j];
    r[0] = s->rcarry_src[j];
    r[1] = c;
    r[2] = noff;
    r[3] = p;
    r[4] = seg;
    r[5] = seg - (s->rs_in[j] - c);
    r[6] = seg + c + p;
    r[7] = s->rs_out[j];
    r[8] = total_k;
    fo[j + 1] = fo[j] + frames_of(s->carry_len[j] + k[j]);
    r[9] = s->carry_src[j];
    r[10] = s->carry_len[j];
    r[11] = k[j];
    r[12] = fo[j + 1];
    seg += c + p;
    noff += p;
  }
  const int64_t total_frames = fo[n];
  if (total_frames > INT64_MAX / kMels) return LOGMEL_ERR_INPUT_TOO_LONG;
  if (total_frames > 0 && !d_out) return LOGMEL_ERR_INVALID_ARGUMENT;
  float* src = s->in_buf[s->in_cur];
  float* dst = s->in_buf[1 - s->in_cur];
  // Every stream in the same state and pushing the same number of samples
  // (a fixed audio clock): the prep kernel derives the records from its
  // arguments (the carries then lie src_step apart, as they were cut from
  // equal segments) and reads no host memory.
  RStreamUniform uni{1, s->rcarry_len[0], flush ? 0 : push_len[0], s->rcarry_src[0],
                     n > 1 ? s->rcarry_src[1] - s->rcarry_src[0] : 0, s->rs_in[0], s->rs_out[0],
                     k[0]};
  for (int64_t j = 1; j < n && uni.on; ++j)
    uni.on = s->rcarry_len[j] == uni.c && (flush ? 0 : push_len[j]) == uni.p &&
             s->rcarry_src[j] == uni.src0 + j * uni.src_step && s->rs_in[j] == uni.rs_in &&
             s->rs_out[j] == uni.rs_out && k[j] == uni.k;
  // and the 16 kHz carries of one length at one place in their rows
  StreamUniform uni16{uni.on, k[0], s->carry_len[0], s->carry_src[0], 0};
  for (int64_t j = 1; j < n && uni16.on; ++j)
    uni16.on = s->carry_len[j] == uni16.c && s->carry_src[j] - j * s->stride == uni16.d;
  uni16.F = frames_of(uni16.c + uni16.P);
  uni.on = uni16.on;
  // Otherwise the prep kernel reads the slot in place. It hands the
  // resampling kernel its segment arrays in rmeta_dev and the transform
  // kernel its offsets in meta_dev.
  if (logmel_launch_rstream_prep(dst, src, flush ? nullptr : d_new, sample_type == LOGMEL_I16,
                                 s->rmeta_host_dev[slot], s->rmeta_dev, n, uni, s->ws, s->stride,
                                 s->meta_dev, uni16, st) != hipSuccess ||
      (last && hipEventRecord(s->rslot_done[grp], st) != hipSuccess))
    return LOGMEL_ERR_DEVICE;
  s->rslot = (slot + 1) % logmel_stream::kSlots;
  // stream j's k[j] <= max_push outputs go to its workspace row from float
  // 400 on, which holds them (stride >= 400 + max_push)
  if (total_k > 0 &&
      logmel_launch_resample(dst, 0, s->rmeta_dev + 5 * n, s->rmeta_dev + 6 * n,
                             s->rmeta_dev + 7 * n, s->rmeta_dev + 8 * n, n, total_k, s->ws,
                             s->stride, kRing, s->rs->btab, s->rs->abase, s->rs_k, st) !=
          hipSuccess)
    return LOGMEL_ERR_DEVICE;
  const int r = lm_transform(s, k.data(), fo, d_out, out_type, fo_out, st);
  if (r != LOGMEL_OK) return r;
  // Advance the host shadow: keep the input from the first window the next
  // outputs need.
  for (int64_t j = 0; j < n; ++j) {
    const int64_t c = s->rcarry_len[j];
    const int64_t p = flush ? 0 : push_len[j];
    const int64_t n_in = s->rs_in[j] + p;
    const int64_t n_out = s->rs_out[j] + k[j];
    int64_t a = (n_out * geo.M) / geo.L - geo.J;        // first sample still needed
    const int64_t kept = s->rs_in[j] - c;                // first sample in the segment
    if (a < kept) a = kept;
    if (a > n_in) a = n_in;
    s->rcarry_src[j] = m[j * kRStreamMetaRec + 4] + (a - kept);   // segment start + offset
    s->rcarry_len[j] = n_in - a;
    s->rs_in[j] = n_in;
    s->rs_out[j] = n_out;
  }
  s->in_cur = 1 - s->in_cur;
  return LOGMEL_OK;
}

}  // namespace

int logmel_stream_push_ex(logmel_stream* s, const void* d_new, int sample_type,
                          const int64_t* push_len, void* d_out, int out_type, int64_t* fo_out,
                          void* hip_stream) {
  if (!s || !push_len) return LOGMEL_ERR_INVALID_ARGUMENT;
  if (sample_type != LOGMEL_F32 && sample_type != LOGMEL_I16) return LOGMEL_ERR_UNSUPPORTED;
  if (out_type != LOGMEL_F32 && out_type != LOGMEL_F16) return LOGMEL_ERR_UNSUPPORTED;
  const int64_t n = s->n;
  const int64_t limit = s->rs ? s->in_max_push : s->max_push;
  int64_t total_new = 0;
  for (int64_t j = 0; j < n; ++j) {
    if (push_len[j] < 0) return LOGMEL_ERR_INVALID_ARGUMENT;
    if (push_len[j] > limit) return LOGMEL_ERR_INPUT_TOO_LONG;
    total_new += push_len[j];
  }
  if (total_new > 0 && !d_new) return LOGMEL_ERR_INVALID_ARGUMENT;
  DeviceGuard g(s->plan->cfg.device);
  if (!g.ok) return LOGMEL_ERR_DEVICE;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (s->rs) return rs_push(s, d_new, sample_type, push_len, d_out, out_type, fo_out, st, false);
  return lm_push(s, d_new, sample_type, push_len, d_out, out_type, fo_out, st);
}

int logmel_stream_flush(logmel_stream* s, void* d_out, int out_type, int64_t* fo_out,
                        void* hip_stream) {
  if (!s) return LOGMEL_ERR_INVALID_ARGUMENT;
  if (out_type != LOGMEL_F32 && out_type != LOGMEL_F16) return LOGMEL_ERR_UNSUPPORTED;
  int r = LOGMEL_OK;
  if (s->rs) {
    DeviceGuard g(s->plan->cfg.device);
    if (!g.ok) return LOGMEL_ERR_DEVICE;
    r = rs_push(s, nullptr, LOGMEL_F32, nullptr, d_out, out_type, fo_out,
                static_cast<hipStream_t>(hip_stream), true);
  } else if (fo_out) {
    for (int64_t j = 0; j <= s->n; ++j) fo_out[j] = 0;   // partial frames are dropped
  }
  if (r != LOGMEL_OK) return r;
  return logmel_stream_reset(s);
}

// ------------------------------------------- streams in the fixed device array

namespace {

static_assert(kStreamMetaRec == 8, "kStaticRecBytes assumes 8 words per stream");
static_assert(kStaticMaxStreams == LOGMEL_STATIC_MAX_STREAMS &&
                  kStaticMaxPush == LOGMEL_STATIC_MAX_PUSH,
              "the header states the limits of the fixed array");

// Host shadow of the streams of logmel_stream_push_static, one set per
// device, in static storage (the entry point allocates nothing): each
// stream's carry (where it sits in its workspace row and how long it is),
// and the records and frame offsets of the push being issued.
struct StaticStreams {
  int64_t carry_len[kStaticMaxStreams];
  int64_t carry_src[kStaticMaxStreams];
  int64_t rec[kStaticMaxStreams * kStreamMetaRec];
  int64_t fo[kStaticMaxStreams + 1];
};
static StaticStreams g_static_streams[kStaticMaxDevices];

}  // namespace

int logmel_stream_push_static(const logmel_plan* plan, int64_t n_streams, const float* d_new,
                              const int64_t* push_len, int reset, float* d_out, int64_t out_rows,
                              int64_t* fo_out, void* hip_stream) {
  if (!plan || !push_len || n_streams < 1 || out_rows < 0) return LOGMEL_ERR_INVALID_ARGUMENT;
  if (n_streams > kStaticMaxStreams) return LOGMEL_ERR_INPUT_TOO_LONG;
  const int dev = plan->cfg.device;
  if (dev < 0 || dev >= kStaticMaxDevices) return LOGMEL_ERR_UNSUPPORTED;
  int64_t fresh = 0;
  for (int64_t j = 0; j < n_streams; ++j) {
    if (push_len[j] < 0) return LOGMEL_ERR_INVALID_ARGUMENT;
    if (push_len[j] > kStaticMaxPush) return LOGMEL_ERR_INPUT_TOO_LONG;
    fresh += push_len[j];
  }
  if (fresh > 0 && !d_new) return LOGMEL_ERR_INVALID_ARGUMENT;
  StaticStreams& S = g_static_streams[dev];
  // Frame offsets of this push (a reset push starts every stream empty).
  S.fo[0] = 0;
  for (int64_t j = 0; j < n_streams; ++j)
    S.fo[j + 1] = S.fo[j] + frames_of((reset ? 0 : S.carry_len[j]) + push_len[j]);
  const int64_t total_frames = S.fo[n_streams];
  if (total_frames > out_rows) return LOGMEL_ERR_INVALID_ARGUMENT;
  if (total_frames > 0 && !d_out) return LOGMEL_ERR_INVALID_ARGUMENT;
  DeviceGuard g(dev);
  if (!g.ok) return LOGMEL_ERR_DEVICE;
  void* scratch = nullptr;
  if (logmel_static_scratch(dev, &scratch) != hipSuccess) return LOGMEL_ERR_DEVICE;
  if (reset)
    for (int64_t j = 0; j < kStaticMaxStreams; ++j) S.carry_len[j] = 0;
  float* ws = static_cast<float*>(scratch);
  int64_t* rec_dev = reinterpret_cast<int64_t*>(static_cast<unsigned char*>(scratch) +
                                                kStaticWsBytes);
  int64_t* meta_dev = reinterpret_cast<int64_t*>(static_cast<unsigned char*>(scratch) +
                                                 kStaticWsBytes + kStaticRecBytes);
  // One record per stream, as for a stream object's push (layout in
  // logmel_stream.hip), copied into the array on the caller's stream.
  int64_t off = 0;
  for (int64_t j = 0; j < n_streams; ++j) {
    const int64_t c = S.carry_len[j], p = push_len[j];
    const int64_t base = j * kStaticStride;
    int64_t* r = S.rec + j * kStreamMetaRec;
    r[0] = c > 0 ? S.carry_src[j] : base + kRing;
    r[1] = c;
    r[2] = off;
    r[3] = p;
    r[4] = base + kRing - c;
    r[5] = base + kRing + p;
    r[6] = S.fo[j + 1];
    r[7] = 0;
    off += p;
  }
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (hipMemcpyAsync(rec_dev, S.rec, (size_t)n_streams * kStreamMetaRec * 8,
                     hipMemcpyHostToDevice, st) != hipSuccess ||
      logmel_launch_stream_prep(ws, kStaticStride, d_new, 0, rec_dev, meta_dev, n_streams,
                                StreamUniform{0, 0, 0, 0, 0}, st) !=
          hipSuccess ||
      logmel_launch_tiles(plan->tables, ws, 0, meta_dev + 4 * n_streams, meta_dev + 5 * n_streams,
                          meta_dev + 6 * n_streams, n_streams, total_frames, d_out, 0,
                          meta_dev + 6 * n_streams, 1, total_frames, plan->resident_waves, st) !=
          hipSuccess)
    return LOGMEL_ERR_DEVICE;
  // Advance the host shadow.
  for (int64_t j = 0; j < n_streams; ++j) {
    const int64_t c = S.carry_len[j], p = push_len[j];
    const int64_t F = frames_of(c + p);
    const int64_t seg0 = j * kStaticStride + kRing - c;
    S.carry_src[j] = seg0 + kHop * F;
    S.carry_len[j] = c + p - kHop * F;
  }
  if (fo_out) std::memcpy(fo_out, S.fo, (n_streams + 1) * sizeof(int64_t));
  return LOGMEL_OK;
}

int logmel_stream_counters(const logmel_stream* s, int64_t j, int64_t* seen, int64_t* emitted) {
  if (!s || j < 0 || j >= s->n) return LOGMEL_ERR_INVALID_ARGUMENT;
  if (seen) *seen = s->rs ? s->rs_in[j] : s->seen[j];
  if (emitted) *emitted = s->emitted[j];
  return LOGMEL_OK;
}

static constexpr int64_t kStateWords = 3 * 2 + kRing;  // 3 int64 + 400 fp32, in 4-byte words

namespace {

// A resampling stream's record: 6 int64 (16 kHz samples seen, frames
// emitted, 16 kHz carry length, input samples seen, 16 kHz samples formed,
// input carry length), the 400-word 16 kHz carry, then the input carry of
// at most 2J samples (every input sample before the next output's window has
// been used), in 4-byte words.
int64_t rs_state_words(const logmel_stream* s) { return 6 * 2 + kRing + 2 * (int64_t)s->rs->geo.J; }

// The input carry a stream holds after rs_in input samples and rs_out
// outputs: from the first sample of output rs_out's window on.
int64_t rs_expected_carry(const ResGeometry& geo, int64_t rs_in, int64_t rs_out) {
  int64_t a = (rs_out * geo.M) / geo.L - geo.J;
  if (a < 0) a = 0;
  if (a > rs_in) a = rs_in;
  return rs_in - a;
}

// The 16 kHz carry after `seen` samples: from the start of the next frame on.
int64_t expected_carry(int64_t seen) { return seen < kNFFT ? seen : seen - kHop * frames_of(seen); }

}  // namespace

int64_t logmel_stream_state_bytes(const logmel_stream* s) {
  if (!s) return 0;
  return s->n * (s->rs ? rs_state_words(s) : kStateWords) * 4;
}

int logmel_stream_get_state(logmel_stream* s, void* state_host, void* hip_stream) {
  if (!s || !state_host) return LOGMEL_ERR_INVALID_ARGUMENT;
  DeviceGuard g(s->plan->cfg.device);
  if (!g.ok) return LOGMEL_ERR_DEVICE;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  char* b = static_cast<char*>(state_host);
  const int64_t words = s->rs ? rs_state_words(s) : kStateWords;
  const int64_t hdr_bytes = s->rs ? 48 : 24;
  for (int64_t j = 0; j < s->n; ++j) {
    char* r = b + j * words * 4;
    std::memset(r, 0, words * 4);
    if (s->rs) {
      const int64_t hdr[6] = {s->seen[j],  s->emitted[j], s->carry_len[j],
                              s->rs_in[j], s->rs_out[j],  s->rcarry_len[j]};
      std::memcpy(r, hdr, sizeof(hdr));
    } else {
      const int64_t hdr[3] = {s->seen[j], s->emitted[j], s->carry_len[j]};
      std::memcpy(r, hdr, sizeof(hdr));
    }
    // both carries are read on hip_stream, after the pushes that wrote them
    if (s->carry_len[j] > 0 &&
        hipMemcpyAsync(r + hdr_bytes, s->ws + s->carry_src[j], s->carry_len[j] * 4,
                       hipMemcpyDeviceToHost, st) != hipSuccess)
      return LOGMEL_ERR_DEVICE;
    if (s->rs && s->rcarry_len[j] > 0 &&
        hipMemcpyAsync(r + hdr_bytes + kRing * 4, s->in_buf[s->in_cur] + s->rcarry_src[j],
                       s->rcarry_len[j] * 4, hipMemcpyDeviceToHost, st) != hipSuccess)
      return LOGMEL_ERR_DEVICE;
  }
  return hipStreamSynchronize(st) == hipSuccess ? LOGMEL_OK : LOGMEL_ERR_DEVICE;
}

int logmel_stream_set_state(logmel_stream* s, const void* state_host, void* hip_stream) {
  if (!s || !state_host) return LOGMEL_ERR_INVALID_ARGUMENT;
  const char* b = static_cast<const char*>(state_host);
  const int64_t words = s->rs ? rs_state_words(s) : kStateWords;
  const int64_t hdr_bytes = s->rs ? 48 : 24;
  // The state must be one a stream can reach: carries and counters agree.
  for (int64_t j = 0; j < s->n; ++j) {
    int64_t hdr[6] = {0, 0, 0, 0, 0, 0};
    std::memcpy(hdr, b + j * words * 4, hdr_bytes);
    const int64_t seen = hdr[0], emitted = hdr[1], c = hdr[2];
    if (seen < 0 || emitted != frames_of(seen) || c != expected_carry(seen) || c < 0 ||
        c >= kRing)
      return LOGMEL_ERR_INVALID_ARGUMENT;
    if (s->rs) {
      const int64_t rs_in = hdr[3], rs_out = hdr[4], rc = hdr[5];
      if (rs_in < 0 || rs_in > INT64_MAX / 16000 || rs_out != res_final(s->rs->geo, rs_in) ||
          seen != rs_out || rc != rs_expected_carry(s->rs->geo, rs_in, rs_out) ||
          rc > 2 * (int64_t)s->rs->geo.J)
        return LOGMEL_ERR_INVALID_ARGUMENT;
    }
  }
  DeviceGuard g(s->plan->cfg.device);
  if (!g.ok) return LOGMEL_ERR_DEVICE;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  int64_t rpos = 0;   // input carries, packed stream by stream in the carry buffer
  for (int64_t j = 0; j < s->n; ++j) {
    const char* r = b + j * words * 4;
    int64_t hdr[6] = {0, 0, 0, 0, 0, 0};
    std::memcpy(hdr, r, hdr_bytes);
    const int64_t c = hdr[2];
    const int64_t dst = j * s->stride + kRing - c;
    if (c > 0 && hipMemcpyAsync(s->ws + dst, r + hdr_bytes, c * 4, hipMemcpyHostToDevice, st) !=
                     hipSuccess)
      return LOGMEL_ERR_DEVICE;
    s->seen[j] = hdr[0];
    s->emitted[j] = hdr[1];
    s->carry_len[j] = c;
    s->carry_src[j] = dst;
    if (s->rs) {
      const int64_t rc = hdr[5];
      if (rc > 0 && hipMemcpyAsync(s->in_buf[s->in_cur] + rpos, r + hdr_bytes + kRing * 4,
                                   rc * 4, hipMemcpyHostToDevice, st) != hipSuccess)
        return LOGMEL_ERR_DEVICE;
      s->rs_in[j] = hdr[3];
      s->rs_out[j] = hdr[4];
      s->rcarry_len[j] = rc;
      s->rcarry_src[j] = rpos;
      rpos += rc;
    }
  }
  // The host buffer is the caller's: finish the copies before returning.
  return hipStreamSynchronize(st) == hipSuccess ? LOGMEL_OK : LOGMEL_ERR_DEVICE;
}

}  // extern "C"

extern "C" {

int64_t logmel_resample_length(int64_t n_samples, int32_t in_rate) {
  if (n_samples < 0 || !res_rate_ok(in_rate)) return -1;
  if (n_samples > INT64_MAX / 16000) return -1;
  return (n_samples * 16000 + in_rate - 1) / in_rate;
}

int logmel_resample_offsets(int32_t in_rate, const int64_t* so, int64_t n_clips, int64_t* oo) {
  if (!so || !oo || n_clips < 0) return LOGMEL_ERR_INVALID_ARGUMENT;
  if (!res_rate_ok(in_rate)) return LOGMEL_ERR_UNSUPPORTED;
  if (so[0] != 0) return LOGMEL_ERR_INVALID_ARGUMENT;
  for (int64_t i = 0; i < n_clips; ++i)
    if (so[i + 1] < so[i]) return LOGMEL_ERR_INVALID_ARGUMENT;
  if (so[n_clips] > INT64_MAX / 16000) return LOGMEL_ERR_INPUT_TOO_LONG;
  int64_t acc = 0;
  oo[0] = 0;
  for (int64_t i = 0; i < n_clips; ++i) {
    acc += logmel_resample_length(so[i + 1] - so[i], in_rate);
    oo[i + 1] = acc;
  }
  return LOGMEL_OK;
}

int logmel_resampler_create(const logmel_plan* plan, int32_t in_rate, logmel_resampler** out) {
  if (!plan || !out) return LOGMEL_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (!res_rate_ok(in_rate)) return LOGMEL_ERR_UNSUPPORTED;
  const ResGeometry geo = res_geometry(in_rate);
  if (geo.k.NT < 1 || (int64_t)geo.k.C * geo.k.KS * 64 + geo.k.C > kResMaxTableFloats ||
      geo.L * geo.Tp > kResMaxTableFloats)
    return LOGMEL_ERR_UNSUPPORTED;   // a tile's input beyond LDS, or too many phases
  const std::vector<float> taps = res_taps(in_rate, geo);
  const std::vector<float> btab = res_btab(geo, taps);
  logmel_resampler* r = new (std::nothrow) logmel_resampler;
  if (!r) return LOGMEL_ERR_OUT_OF_MEMORY;
  r->plan = plan;
  r->rate = in_rate;
  r->geo = geo;
  DeviceGuard g(plan->cfg.device);
  if (!g.ok) {
    delete r;
    return LOGMEL_ERR_DEVICE;
  }
  const size_t bbytes = btab.size() * sizeof(float);
  const size_t gbytes = geo.abase.size() * sizeof(int);
  if (hipMalloc(&r->btab, bbytes + gbytes) != hipSuccess) {
    delete r;
    return LOGMEL_ERR_OUT_OF_MEMORY;
  }
  r->abase = reinterpret_cast<int*>(reinterpret_cast<char*>(r->btab) + bbytes);
  if (hipMemcpy(r->btab, btab.data(), bbytes, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(r->abase, geo.abase.data(), gbytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(r->btab);
    delete r;
    return LOGMEL_ERR_DEVICE;
  }
  *out = r;
  return LOGMEL_OK;
}

void logmel_resampler_destroy(logmel_resampler* r) {
  if (!r) return;
  if (r->btab) {
    DeviceGuard g(r->plan->cfg.device);
    (void)hipFree(r->btab);
  }
  delete r;
}

int logmel_resampler_info(const logmel_resampler* r, int64_t* phases, int64_t* taps_per_phase) {
  if (!r) return LOGMEL_ERR_INVALID_ARGUMENT;
  if (phases) *phases = r->geo.L;
  if (taps_per_phase) *taps_per_phase = 2 * r->geo.J + 1;
  return LOGMEL_OK;
}

int logmel_resample(const logmel_resampler* r, const void* d_samples, int sample_type,
                    const int64_t* d_sample_offsets, const int64_t* d_out_offsets,
                    int64_t n_clips, int64_t total_out, float* d_out, void* hip_stream) {
  if (!r || n_clips < 0 || total_out < 0) return LOGMEL_ERR_INVALID_ARGUMENT;
  if (sample_type != LOGMEL_F32 && sample_type != LOGMEL_I16) return LOGMEL_ERR_UNSUPPORTED;
  if (n_clips == 0 || total_out == 0) return LOGMEL_OK;
  if (!d_samples || !d_sample_offsets || !d_out_offsets || !d_out)
    return LOGMEL_ERR_INVALID_ARGUMENT;
  DeviceGuard g(r->plan->cfg.device);
  if (!g.ok) return LOGMEL_ERR_DEVICE;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (env_validate()) {
    std::vector<int64_t> so(n_clips + 1), oo(n_clips + 1), ref(n_clips + 1);
    if (hipMemcpyAsync(so.data(), d_sample_offsets, (n_clips + 1) * 8, hipMemcpyDeviceToHost,
                       st) != hipSuccess ||
        hipMemcpyAsync(oo.data(), d_out_offsets, (n_clips + 1) * 8, hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return LOGMEL_ERR_DEVICE;
    if (logmel_resample_offsets(r->rate, so.data(), n_clips, ref.data()) != LOGMEL_OK ||
        ref != oo || oo[n_clips] != total_out)
      return LOGMEL_ERR_INVALID_ARGUMENT;
  }
  if (logmel_launch_resample(d_samples, sample_type == LOGMEL_I16, d_sample_offsets,
                             d_sample_offsets + 1, nullptr, d_out_offsets, n_clips, total_out,
                             d_out, 0, 0, r->btab, r->abase, r->geo.k, st) !=
      hipSuccess)
    return LOGMEL_ERR_DEVICE;
  return LOGMEL_OK;
}

}  // extern "C"
