// engine_internal.h -- what static_step.hip (the allocation-free entry
// point) needs from engine.cpp. Internal to libmoshi.so.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/moshi.h"

namespace moshi_internal {

// static_step.hip: the device address of this device's static step scratch
// (looked up once per device, with that device current) and its size; null
// if the lookup failed.
void* static_scratch_setup(int device, size_t* bytes);

// engine.cpp: the device a context runs on (< 0 on a NULL context).
int ctx_device(const moshi_ctx* c);

// engine.cpp: moshi_step_enqueue's one-session step kernel with its
// synchronisation scratch (grid-barrier counters and the flagged hand-off
// arena) in the static scratch instead of the context's buffers. `seq` is
// this device's launch sequence number (never 0); its low bit picks the
// barrier counter set.
int enqueue_static(moshi_ctx* c, const int32_t* d_frames, int32_t* d_text_token,
                   int32_t* d_audio_codes, uint32_t seq);

}  // namespace moshi_internal
