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

// static_step.hip: for a launch that uses the static scratch on `device`,
// its sequence number (unique on the device, never 0) and the barrier
// counter set it uses; static_launch_done (after the launch was queued)
// hands the other set to the next launch on the device.
void static_launch_ids(int device, uint32_t* seq, int* parity);
void static_launch_done(int device);

// engine.cpp: moshi_step_enqueue's one-session step kernel with its
// synchronisation scratch (grid-barrier counters and the flagged hand-off
// arena) in the static scratch instead of the context's buffers.
int enqueue_static(moshi_ctx* c, const int32_t* d_frames, int32_t* d_text_token,
                   int32_t* d_audio_codes);

}  // namespace moshi_internal
