/* logmel.h -- C ABI of the MI355X (gfx950) 128-bin log-mel front end.
 *
 * What is computed (page "从零理解 ASR：音频基础、Qwen3-ASR 架构，以及离线 vs
 * 流式推理原理", marsggbo blog, §2.3 "Log-Mel Spectrogram 提取流水线",
 * steps 1-5, and the preprocessor-config list after them): 16 kHz mono fp32
 * PCM is cut into 400-sample frames every 160 samples with no centring or
 * padding, floor((N - 400) / 160) + 1 frames for N >= 400 and none below;
 * each frame is multiplied by the symmetric Hamming window
 * 0.54 - 0.46 cos(2 pi n / 399), transformed by a 400-point real FFT to 201
 * bins, squared in magnitude, projected onto 128 triangular filters evenly
 * spaced on mel = 2595 log10(1 + f/700) over 0..8000 Hz (peak 1, no
 * normalisation; end vertices exactly 0 and 8000 Hz; triangles linear in
 * Hz), and compressed by ln(max(E, 1e-10)). The output is frame-major
 * [frames][128] fp32 (the page's shape table after step 5).
 *
 * Conventions of every call:
 *  - Return value: LOGMEL_OK (0) or a negative LOGMEL_ERR_* code. Arguments
 *    are checked on the host before anything is launched, so an error means
 *    nothing was written. logmel_status_string() names a code.
 *  - "d_" pointers are device pointers on the plan's device; "_host" pointers
 *    are host memory. The caller owns every buffer it passes; the library
 *    never keeps a pointer past the call. The plan owns nothing on the
 *    device; a stream object owns its workspace.
 *  - hip_stream is a hipStream_t (NULL = the null stream). Compute calls are
 *    asynchronous on it: no host synchronisation, no read-back.
 *  - Input values are not checked or clamped; [-1, 1] is the expected range
 *    (page 1, §2.1). A NaN in a frame gives NaN in its outputs.
 *  - Over-long input is an error (LOGMEL_ERR_INPUT_TOO_LONG), never a silent
 *    truncation (the transcribe.cpp Qwen3-ASR page, §四, states the same
 *    convention for its length limit).
 */
#ifndef LOGMEL_H_
#define LOGMEL_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  LOGMEL_OK = 0,
  LOGMEL_ERR_INVALID_ARGUMENT = -1, /* null pointer, negative size, bad offsets */
  LOGMEL_ERR_UNSUPPORTED = -2,      /* a configuration other than the one below */
  LOGMEL_ERR_OUT_OF_MEMORY = -3,    /* device or pinned host allocation failed */
  LOGMEL_ERR_DEVICE = -4,           /* a HIP runtime call failed */
  LOGMEL_ERR_INPUT_TOO_LONG = -5    /* sizes beyond int64 indexing or a stream's push limit */
};

/* The front-end configuration. Only the values of page 1 (§2.3 and the
 * preprocessor-config list) are supported: sample_rate 16000, n_fft 400,
 * hop 160, n_mels 128, f_min 0, f_max 8000, log_floor 1e-10. Any other value
 * gives LOGMEL_ERR_UNSUPPORTED (a sample rate other than 16 kHz is rejected,
 * as the page's processor call requires 16 kHz input). */
typedef struct logmel_config {
  int32_t sample_rate;
  int32_t n_fft;
  int32_t hop;
  int32_t n_mels;
  double f_min;
  double f_max;
  double log_floor;
  int32_t device; /* HIP device ordinal */
} logmel_config;

/* Fills *cfg with the supported configuration on device 0. */
void logmel_default_config(logmel_config* cfg);

typedef struct logmel_plan logmel_plan;     /* immutable, shareable across threads */
typedef struct logmel_stream logmel_stream; /* state of n streams; not thread-safe */

/* Validates cfg and creates a plan for cfg->device. */
int logmel_plan_create(const logmel_config* cfg, logmel_plan** out);
void logmel_plan_destroy(logmel_plan* plan);

/* Frames of an n_samples clip (page 1, §2.3 step 1): 0 if n_samples < 400,
 * else floor((n_samples - 400) / 160) + 1. Negative n gives 0. */
int64_t logmel_num_frames(int64_t n_samples);

/* Host helper (page 1, §2.3 step 1: each clip's frame count, as
 * logmel_num_frames, summed clip by clip). Clip i holds samples
 * [sample_offsets_host[i], sample_offsets_host[i+1]) of a packed buffer
 * (n_clips + 1 non-decreasing int64, first 0). Writes
 * frame_offsets_host[0..n_clips] = exclusive prefix sum of the clips' frame
 * counts, in exact int64 arithmetic: clip i's frames are output rows
 * [frame_offsets[i], frame_offsets[i+1]). Errors: INVALID_ARGUMENT for null
 * pointers, n_clips < 0, a non-zero first offset or decreasing offsets. */
int logmel_frame_offsets(const int64_t* sample_offsets_host, int64_t n_clips,
                         int64_t* frame_offsets_host);

/* Offline log-mel of a packed ragged batch (page 1, §2.3 steps 1-5).
 *   d_samples          fp32, clip i = d_samples[d_sample_offsets[i] ..
 *                      d_sample_offsets[i+1]), packed with no padding
 *   d_sample_offsets   int64[n_clips + 1], as for logmel_frame_offsets
 *   d_frame_offsets    int64[n_clips + 1], what logmel_frame_offsets returns
 *                      for those sample offsets
 *   total_frames       d_frame_offsets[n_clips]
 *   d_out              fp32 [total_frames][128], row-major; row
 *                      d_frame_offsets[i] + f is frame f of clip i
 * The offsets are a precondition the device does not read back: a frame
 * whose 400 samples do not lie inside its clip is written as a row of NaN
 * rather than read out of bounds. With the environment variable
 * LOGMEL_VALIDATE=1 the call copies the offsets to the host first (one
 * synchronisation) and returns INVALID_ARGUMENT if they disagree.
 * n_clips == 0 or total_frames == 0 is a valid empty call.
 * INPUT_TOO_LONG if total_frames * 128 overflows int64. */
int logmel_compute(const logmel_plan* plan, const float* d_samples,
                   const int64_t* d_sample_offsets, const int64_t* d_frame_offsets,
                   int64_t n_clips, int64_t total_frames, float* d_out,
                   void* hip_stream);

/* 30-s chunks for the encoder input [chunks][3000][128] (page 1: the
 * preprocessor-config list after §2.3 gives chunk_length 30 s -> 3000
 * frames, and §4 says the encoder takes a fixed [B, 3000, 128] with every
 * input padded to 3000 frames; page 3, §二 stage 1: the front end cuts at
 * 30 s). Chunk j of a clip holds the clip's frames 3000 j .. 3000 j + 2999
 * (the frames that start in seconds 30 j .. 30 j + 30), so a chunked frame
 * is the offline frame bit for bit; the rows of a clip's last chunk past its
 * last frame hold ln(1e-10), bit for bit the value of a silent frame; a clip
 * with no frame has no chunk. */
#define LOGMEL_CHUNK_FRAMES 3000

/* Host helper. Writes chunk_offsets_host[0..n_clips] = exclusive prefix sum
 * of the clips' chunk counts ceil(F_i / 3000): clip i's chunks are
 * [chunk_offsets[i], chunk_offsets[i+1]). Same errors as
 * logmel_frame_offsets. */
int logmel_chunk_offsets(const int64_t* sample_offsets_host, int64_t n_clips,
                         int64_t* chunk_offsets_host);

/* Host helper. Writes, for each of the total_chunks chunks in order, the
 * number of frames it holds (1..3000; the rest of its rows are padding), for
 * an encoder's attention mask or ragged-tail trimming. total_chunks must be
 * what logmel_chunk_offsets gives (INVALID_ARGUMENT otherwise). */
int logmel_chunk_frames(const int64_t* sample_offsets_host, int64_t n_clips,
                        int64_t total_chunks, int64_t* chunk_frames_host);

/* logmel_compute into the chunk layout.
 *   d_chunk_offsets    int64[n_clips + 1], what logmel_chunk_offsets returns
 *   total_chunks       d_chunk_offsets[n_clips]
 *   d_out              fp32 [total_chunks][3000][128], row-major; frame f of
 *                      clip i is row d_chunk_offsets[i] * 3000 + f
 * Everything else as logmel_compute (LOGMEL_VALIDATE=1 also checks the chunk
 * offsets). INPUT_TOO_LONG if total_chunks * 3000 * 128 overflows int64. */
int logmel_compute_chunked(const logmel_plan* plan, const float* d_samples,
                           const int64_t* d_sample_offsets, const int64_t* d_frame_offsets,
                           const int64_t* d_chunk_offsets, int64_t n_clips,
                           int64_t total_frames, int64_t total_chunks, float* d_out,
                           void* hip_stream);

/* Sample and output types of logmel_compute_ex. */
#define LOGMEL_F32 0 /* fp32 */
#define LOGMEL_I16 1 /* int16 PCM, input only: sample s means s / 32768 (page 1, §2.1 gives
                        samples as floats in [-1.0, 1.0]; s / 32768 is exact in fp32, so an int16
                        batch gives the fp32 batch's result bit for bit) */
#define LOGMEL_F16 2 /* IEEE half, output only: each fp32 log-mel value rounded once to
                        nearest; padding and the NaN rows of inconsistent offsets as in fp32 */

/* The general offline call; logmel_compute and logmel_compute_chunked are
 * this call with fp32 in and out.
 *   d_samples          sample_type LOGMEL_F32 (float) or LOGMEL_I16 (int16_t);
 *                      the buffer start must be 4-byte aligned (INVALID_ARGUMENT
 *                      otherwise); clips may start at any sample
 *   d_chunk_offsets    NULL: the frame layout [total_frames][128]
 *                      (total_chunks unused); else the 30-s chunk layout
 *                      [total_chunks][3000][128] as in logmel_compute_chunked
 *   d_out              out_type LOGMEL_F32 (float) or LOGMEL_F16 (half)
 * Other types: UNSUPPORTED. Everything else as logmel_compute. */
int logmel_compute_ex(const logmel_plan* plan, const void* d_samples, int sample_type,
                      const int64_t* d_sample_offsets, const int64_t* d_frame_offsets,
                      const int64_t* d_chunk_offsets, int64_t n_clips, int64_t total_frames,
                      int64_t total_chunks, void* d_out, int out_type, void* hip_stream);

/* Streaming (the 80 ms audio clock of the Audio8-ASR-Infinite page gives the
 * 1280-sample push). A stream object holds n_streams independent streams.
 * Each push appends new samples to every stream and emits every frame that
 * is now complete on the offline grid of that stream: the frames emitted
 * over all pushes are exactly logmel_compute's frames of the concatenated
 * stream, bit for bit. Between pushes a stream keeps only its carry: the
 * samples from the start of its next frame on, at most 399 (240 plus the
 * stream length minus 400, modulo 160, once 400 samples have arrived).
 *
 * logmel_stream_create allocates, on the plan's device, a workspace of
 * n_streams rows of (400 + max_push) fp32 and a small pinned host staging
 * area; pushes allocate nothing. max_push >= 1 is the most new samples one
 * stream may receive in one push. */
int logmel_stream_create(const logmel_plan* plan, int64_t n_streams, int64_t max_push,
                         logmel_stream** out);
void logmel_stream_destroy(logmel_stream* s);

/* Forgets every stream's history (carry and counters). Host-side only. */
int logmel_stream_reset(logmel_stream* s);

/* Frames each stream will emit if push_len_host[j] new samples are pushed
 * to stream j: writes out_frame_offsets_host[0..n_streams] (exclusive
 * prefix sum). Stream j emits logmel_num_frames(total after the push) minus
 * the frames it has already emitted: the offline count of page 1, §2.3
 * step 1, applied to the stream's audio so far (the pushes are the audio
 * clock of the Audio8-ASR-Infinite page). Computed from the stream object's
 * host-side counters; does not change the state and reads nothing back. */
int logmel_stream_frames_for_push(const logmel_stream* s, const int64_t* push_len_host,
                                  int64_t* out_frame_offsets_host);

/* Pushes push_len_host[j] (0..max_push) new samples to every stream j.
 *   d_new   fp32, the new samples packed stream by stream, stream j's at
 *           offset sum_{i<j} push_len_host[i]
 *   d_out   fp32 [total][128]: stream j's new frames are rows
 *           [fo[j], fo[j+1]) with fo = logmel_stream_frames_for_push()
 *   out_frame_offsets_host  optional (may be NULL): receives fo
 * Two kernel launches on hip_stream; the per-push offsets go up through the
 * stream object's pinned staging area. INPUT_TOO_LONG if a push_len exceeds
 * max_push. The new samples are copied before the call returns its work to
 * the queue, so d_new may be reused once hip_stream has passed this call.
 * A push reads the carry the previous push of the same stream object wrote:
 * successive pushes must run in order on the device (one hip_stream, or
 * streams the caller orders). */
int logmel_stream_push(logmel_stream* s, const float* d_new, const int64_t* push_len_host,
                       float* d_out, int64_t* out_frame_offsets_host, void* hip_stream);

/* logmel_stream_push with the sample and output types of logmel_compute_ex:
 * d_new fp32 or int16 PCM (sample_type LOGMEL_F32 / LOGMEL_I16; s means
 * s / 32768, exact), d_out fp32 or fp16 (out_type LOGMEL_F32 / LOGMEL_F16,
 * each value the fp32 result rounded once to nearest). A stream may mix
 * types from push to push: its carry is kept as fp32 values. UNSUPPORTED for
 * other types. */
int logmel_stream_push_ex(logmel_stream* s, const void* d_new, int sample_type,
                          const int64_t* push_len_host, void* d_out, int out_type,
                          int64_t* out_frame_offsets_host, void* hip_stream);

/* Streams at another input rate (the resampling reading below: Kaiser-
 * windowed sinc to 16 kHz): in_rate 16000 is logmel_stream_create; other
 * rates resample every push to 16 kHz on the device before framing.
 * max_push counts input samples. A stream's frames over all its pushes and
 * its flush are, bit for bit, the offline frames of logmel_resample of the
 * concatenated input followed by logmel_compute: each 16 kHz sample is
 * formed once its whole window has arrived, and the last ones (whose windows
 * reach past the input) at logmel_stream_flush. UNSUPPORTED for rates the
 * resampler does not take. logmel_stream_counters reports input samples for
 * them. */
int logmel_stream_create_ex(const logmel_plan* plan, int64_t n_streams, int64_t max_push,
                            int32_t in_rate, logmel_stream** out);

/* Ends every stream: emits the frames that only the end of the input
 * completes (for 16 kHz streams none: a partial frame is dropped, as
 * offline), then resets the streams. d_out and the offsets as for a push;
 * logmel_stream_frames_for_flush gives the offsets beforehand. */
int logmel_stream_frames_for_flush(const logmel_stream* s, int64_t* out_frame_offsets_host);
int logmel_stream_flush(logmel_stream* s, void* d_out, int out_type,
                        int64_t* out_frame_offsets_host, void* hip_stream);

/* Total samples pushed and frames emitted so far for stream j. */
int logmel_stream_counters(const logmel_stream* s, int64_t j, int64_t* samples_seen,
                           int64_t* frames_emitted);

/* Snapshot / restore of all streams (a stream's state is its carry and
 * counters, so a restored stream continues bit for bit as the uninterrupted
 * one). State blob layout (int64 and fp32 words, size from
 * logmel_stream_state_bytes), per stream:
 *   16 kHz streams: int64 samples_seen, int64 frames_emitted, int64
 *     carry_len, then 400 fp32 carry samples (the first carry_len used);
 *   streams at another input rate: int64 samples_seen (16 kHz samples),
 *     frames_emitted, carry_len, input samples seen, 16 kHz samples formed,
 *     input carry length, then the 400 fp32 carry words as above, then 2J
 *     fp32 input carry samples (the first input-carry-length used; J the
 *     resampler's half width in input samples, logmel_resampler_info).
 * get_state and set_state synchronise hip_stream (get_state reads the
 * carries after the pushes queued on it). set_state accepts only a state a
 * stream of this object's kind (rate) can reach: counters and carry lengths
 * that agree, else INVALID_ARGUMENT with nothing changed. */
int64_t logmel_stream_state_bytes(const logmel_stream* s);
int logmel_stream_get_state(logmel_stream* s, void* state_host, void* hip_stream);
int logmel_stream_set_state(logmel_stream* s, const void* state_host, void* hip_stream);

/* Streams without a stream object, for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same push as logmel_stream_push (fp32 in and out, the
 * frames bit for bit those of logmel_stream_push and of offline log-mel on
 * the concatenated streams), with the streams' workspace in a fixed device
 * array of the library (one per GPU, 6.2 MB, held until the process ends)
 * and their carry counters in static host memory. The call allocates
 * nothing, device or host.
 *   n_streams        1..LOGMEL_STATIC_MAX_STREAMS; stream j is the same
 *                    stream from call to call, whatever n_streams
 *   push_len_host    n_streams new-sample counts, 0..LOGMEL_STATIC_MAX_PUSH
 *   reset            non-zero: every stream forgets its history first
 *   d_out, out_rows  fp32 [out_rows][128]; the push writes rows
 *                    [0, fo[n_streams]) with fo as for logmel_stream_push
 *                    (a push emits at most ceil(push_len / 160) frames per
 *                    stream); INVALID_ARGUMENT if out_rows is too small
 *   out_frame_offsets_host  optional: receives fo[0..n_streams]
 * INPUT_TOO_LONG for more streams or samples than the limits. Calls on one
 * GPU share its array and counters: they must not overlap (two threads, or
 * two HIP streams in flight at once, race). The per-stream records of a push
 * go to the device with an asynchronous host-to-device copy on hip_stream. */
#define LOGMEL_STATIC_MAX_STREAMS 512
#define LOGMEL_STATIC_MAX_PUSH 2560
int logmel_stream_push_static(const logmel_plan* plan, int64_t n_streams, const float* d_new,
                              const int64_t* push_len_host, int reset, float* d_out,
                              int64_t out_rows, int64_t* out_frame_offsets_host,
                              void* hip_stream);

/* ---------------------------------------------------------------------------
 * Resampling to 16 kHz, the step before the front end for audio at another
 * rate. The pages require 16 kHz input (page 1, §6, the offline example in
 * "可运行代码示例": other rates are refused, with a library resampler named
 * for real use; page 1, §2.1: 16 kHz because speech content of interest lies
 * below 8 kHz). They name no method; this library's reading is band-limited
 * interpolation with a Kaiser-windowed sinc (J. O. Smith's bandlimited
 * interpolation): output sample n of a clip sits at input position
 * p = n R / 16000 (R the input rate) and is
 *   y[n] = sum_k x[k] h(p - k) over the clip's samples (zero outside it),
 *   h(d) = (2 fc / R) sinc(2 fc d / R) I0(9 sqrt(1 - (d/H)^2)) / I0(9), |d| < H,
 * with cutoff fc = 0.96 min(R, 16000) / 2 Hz and half-width
 * H = 24 R / (2 fc) input samples (24 zero crossings each side). A clip of
 * N samples gives ceil(16000 N / R) outputs. At R = 16000 the output is the
 * input. The taps are computed in fp64 and rounded to fp32; each output is
 * an fp32 dot product of its 2 ceil(H) + 1 terms, accumulated in fp32 on the
 * matrix cores four products per step (the kernel forms 16 consecutive
 * outputs at once over the union of their windows, with zero taps outside
 * each output's own window; an output gets the same value whichever call
 * forms it, but a non-finite sample also reaches the outputs of its group of
 * 16 whose staged window holds it: 4 KS positions of the staged input, KS the
 * smallest multiple of 8 with 4 KS >= 2J + 1 plus the spread of the group's
 * windows, so at most 4 KS - 2J - 1 positions beyond an output's own window
 * (53 at 44.1 kHz, 73 at 48 kHz; at rates whose staged input carries two pad
 * positions per super-period, 32, 64, 96 and 192 kHz, fewer samples), within
 * its clip). Output offsets that overstate total_out write nothing past
 * d_out[total_out - 1].
 * --------------------------------------------------------------------------- */
#define LOGMEL_RESAMPLE_ZEROS 24

/* Output length for n_samples at in_rate Hz: ceil(16000 n / in_rate); -1 for
 * a negative length, a rate outside [1000, 384000], or n above INT64_MAX / 16000. */
int64_t logmel_resample_length(int64_t n_samples, int32_t in_rate);

/* Exclusive prefix sum of per-clip output lengths (host arrays of
 * n_clips + 1 int64). INVALID_ARGUMENT for offsets that do not start at 0 or
 * decrease; UNSUPPORTED for a rate outside [1000, 384000]. */
int logmel_resample_offsets(int32_t in_rate, const int64_t* sample_offsets_host, int64_t n_clips,
                            int64_t* out_offsets_host);

/* A resampler for one input rate: owns the device taps table (fp32: the
 * 2J + 1 taps of each of the L phases, 16000 / R = L / M in lowest terms,
 * arranged per group of 16 consecutive outputs as the matrix cores read
 * them). UNSUPPORTED for rates outside [1000, 384000] and for rates with so
 * many phases, or samples so far apart, that a tile's input does not fit the
 * kernel's LDS (it holds every common rate: 8000, 11025, 12000, 16000,
 * 22050, 24000, 32000, 44100, 48000, 88200, 96000, 176400, 192000). */
typedef struct logmel_resampler logmel_resampler;
int logmel_resampler_create(const logmel_plan* plan, int32_t in_rate, logmel_resampler** out);
void logmel_resampler_destroy(logmel_resampler* r);
/* Phase count L and taps per phase (2J + 1) of a resampler. */
int logmel_resampler_info(const logmel_resampler* r, int64_t* phases, int64_t* taps_per_phase);

/* Resamples a packed batch of clips to 16 kHz.
 *   d_samples          fp32 or int16 PCM (sample_type LOGMEL_F32 / LOGMEL_I16;
 *                      int16 s means s / 32768), clips packed back to back
 *   d_sample_offsets   int64 [n_clips + 1], clip i = [so[i], so[i+1])
 *   d_out_offsets      int64 [n_clips + 1] from logmel_resample_offsets()
 *   d_out              fp32 [total_out], clip i's output at [oo[i], oo[i+1]);
 *                      it is itself a packed 16 kHz batch for logmel_compute
 *                      with d_out_offsets as its sample offsets
 * One kernel launch on hip_stream; the offsets are a precondition, checked
 * only with LOGMEL_VALIDATE=1 (one synchronisation). */
int logmel_resample(const logmel_resampler* r, const void* d_samples, int sample_type,
                    const int64_t* d_sample_offsets, const int64_t* d_out_offsets,
                    int64_t n_clips, int64_t total_out, float* d_out, void* hip_stream);

/* Names a status code (a static string; "unknown status" for codes this
 * library does not return). Every failure is an explicit negative code and
 * over-long input is an error, never a silent truncation: the convention
 * the transcribe.cpp Qwen3-ASR page (§四) states for its input-length limit. */
const char* logmel_status_string(int status);

/* Version of this ABI, for binding checks. */
int logmel_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LOGMEL_H_ */
