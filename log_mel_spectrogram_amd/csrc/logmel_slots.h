// Streaming pushes: the records of the pinned host staging slots that the
// prep kernels read in place (layouts in logmel_stream.hip). One record per
// stream, so that a prep workgroup's fields come in one line of host memory.
#pragma once

// Words (int64) per stream in a 16 kHz push's slot (64 bytes).
static constexpr int kStreamMetaRec = 8;

// Words (int64) per stream in a resampling push's slot (one 128-byte line).
static constexpr int kRStreamMetaRec = 16;
