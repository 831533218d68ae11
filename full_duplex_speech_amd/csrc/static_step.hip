// static_step.hip -- moshi_step_enqueue_noalloc: the device-resident step
// for callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc). The one-session step
// kernel's synchronisation scratch -- two sets of grid-barrier counters and
// the arena of flagged vectors the operations hand on -- lives in the
// file-scope array `scratch` below instead of buffers the context allocated.
//
// Every call on one GPU shares that GPU's array and finds the last call's
// contents there. Nothing has to be cleared per call: each launch clears the
// barrier counter set the next launch on the device uses (the array starts
// zeroed; the sets alternate per launch on the device, not per call, since a
// call with no live session launches nothing), and a flagged word only
// counts when its flag equals the launch's sequence number, which is unique
// per device (a host counter per device that skips 0), so a word another
// context or an earlier call left behind is never taken as current. Calls
// that overlap on one GPU (two streams, two threads) race and are not
// supported.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/moshi.h"
#include "engine_internal.h"

namespace {

// 40 MiB: the barrier counters (136 KiB) and the flagged arena of the
// PersonaPlex-shape step (29.7 MB), with room to spare.
constexpr size_t kScratchBytes = (size_t)40 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];      // device address of `scratch`, per device
uint32_t g_seq[kMaxDevices];   // last launch sequence number, per device
int g_par[kMaxDevices];        // barrier counter set of the next launch, per device

}  // namespace

void* moshi_internal::static_scratch_setup(int device, size_t* bytes) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[device] == nullptr) {
    // In host code `scratch` names a host-side stand-in; the array's address
    // on this device (the caller made it current) comes from the runtime.
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_ptr[device] = p;
  }
  *bytes = kScratchBytes;
  return g_ptr[device];
}

void moshi_internal::static_launch_ids(int device, uint32_t* seq, int* parity) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (++g_seq[device] == 0) g_seq[device] = 1;  // 0 is the zeroed arena's flag
  *seq = g_seq[device];
  *parity = g_par[device];
}

void moshi_internal::static_launch_done(int device) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_par[device] ^= 1;
}

extern "C" int moshi_step_enqueue_noalloc(moshi_ctx* ctx, const int32_t* d_frames,
                                          int32_t* d_text_token, int32_t* d_audio_codes) {
  const int dev = moshi_internal::ctx_device(ctx);
  if (dev < 0 || dev >= kMaxDevices) return MOSHI_E_INVALID;
  return moshi_internal::enqueue_static(ctx, d_frames, d_text_token, d_audio_codes);
}
