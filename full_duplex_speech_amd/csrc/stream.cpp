// stream.cpp -- the delayed-stream wrapper of libmoshi.so: per-codebook
// acoustic delays around moshi_step_forced, with initial tokens, delayed
// output collection and teacher forcing (mobius PR #368, "P3 - ONNX Runtime
// example": the LMGen.step port keeps a ring cache with per-codebook delays
// [0,0,1,1,1,1,1,1,1,0,1,1,1,1,1,1,1] and collects the outputs delayed; the
// persona/voice commit teacher-forces the agent audio and the text stream for
// priming). Host code only: it calls the library's C ABI.
//
// Reading of the timeline (the pages give the delays, not the bookkeeping):
//  * channel k (0 text, 1..A agent audio, A+1..S user audio) has delay d_k;
//    stream column c of channel k carries that channel's token of acoustic
//    frame c - d_k, and the initial token (the embedding tables' last row:
//    Vt for text, card for audio) where c - d_k < 0;
//  * step t feeds column t to the model and writes what it generates (text
//    and the agent codes) into column t+1; the user's frame t goes to column
//    t + d_k of each user channel;
//  * column 0 of a generated channel holds the initial token (nothing was
//    generated before step 0);
//  * after step t the acoustic frame tau = t + 1 - max_k d_k is complete
//    (its channel k sits in column tau + d_k <= t + 1); it is returned once
//    tau >= 1 (frame 0 of a generated channel is only initial tokens). With
//    the pages' delays (max 1), n steps return n - 1 frames;
//  * forcing acts on what step t generates, in stream coordinates: a forced
//    text token is column t+1's text (and depformer substep 0's input), a
//    forced agent code k is column t+1's channel k (and substep k's input).
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "../../include/moshi.h"

namespace {

constexpr int kMaxDelay = 8;

}  // namespace

struct moshi_stream {
  moshi_ctx* ctx = nullptr;
  int B = 0, S = 0, A = 0, NCH = 0;  // slots, substeps, agent channels, channels
  int Vt = 0, Va = 0, S_run = 0;
  std::vector<int> delay;  // [NCH]
  int D = 0;               // max delay
  int C = 0;               // ring columns
  // per slot: ring of columns [C][NCH], frames stepped since the reset, the
  // context position at the reset
  std::vector<int32_t> ring;
  std::vector<int64_t> t, base;
  std::vector<char> reset_done;
  std::vector<int32_t> frames, forced, text, codes;  // staging for one step
  std::string err;
};

namespace {

int32_t* col(moshi_stream* s, int b, int64_t c) {
  return s->ring.data() + ((size_t)b * s->C + (size_t)(c % s->C)) * s->NCH;
}

int initial_token(const moshi_stream* s, int k) { return k == 0 ? s->Vt : s->Va; }

}  // namespace

extern "C" {

int moshi_stream_create(moshi_ctx* ctx, int32_t n_agent, const int32_t* delays,
                        moshi_stream** out) {
  if (!out) return MOSHI_E_INVALID;
  *out = nullptr;
  moshi_config c;
  const moshi_config* cfg = &c;
  if (!ctx || moshi_get_config(ctx, &c) != MOSHI_OK) return MOSHI_E_INVALID;
  const int S = cfg->n_substeps;
  const int S_run = (cfg->dep_q > 0 && cfg->dep_q < S) ? cfg->dep_q : S;
  if (n_agent < 1 || n_agent >= S || n_agent > S_run) return MOSHI_E_INVALID;
  moshi_stream* s = new (std::nothrow) moshi_stream();
  if (!s) return MOSHI_E_OOM;
  s->ctx = ctx;
  s->B = cfg->max_sessions;
  s->S = S;
  s->A = n_agent;
  s->NCH = 1 + S;
  s->Vt = cfg->text_vocab;
  s->Va = cfg->audio_card;
  s->S_run = S_run;
  s->delay.assign(s->NCH, 0);
  for (int k = 0; k < s->NCH; ++k) {
    int d;
    if (delays) {
      d = delays[k];
    } else {  // the pages' pattern: text 0; in each half, first codebook 0, the rest 1
      d = (k == 0 || k == 1 || k == n_agent + 1) ? 0 : 1;
    }
    if (d < 0 || d > kMaxDelay) {
      delete s;
      return MOSHI_E_INVALID;
    }
    s->delay[k] = d;
    s->D = d > s->D ? d : s->D;
  }
  s->C = 2 * s->D + 2;
  s->ring.assign((size_t)s->B * s->C * s->NCH, 0);
  s->t.assign(s->B, 0);
  s->base.assign(s->B, 0);
  s->reset_done.assign(s->B, 0);
  s->frames.assign((size_t)s->B * s->NCH, 0);
  s->forced.assign((size_t)s->B * s->NCH, -1);
  s->text.assign(s->B, -1);
  s->codes.assign((size_t)s->B * S, -1);
  *out = s;
  return MOSHI_OK;
}

int moshi_stream_destroy(moshi_stream* s) {
  delete s;
  return MOSHI_OK;
}

int moshi_stream_reset(moshi_stream* s, int32_t slot) {
  if (!s) return MOSHI_E_INVALID;
  int64_t pos = 0;
  int rc = moshi_session_info(s->ctx, slot, &pos, nullptr, nullptr);
  if (rc) {
    s->err = "slot not live";
    return rc;
  }
  s->t[slot] = 0;
  s->base[slot] = pos;
  s->reset_done[slot] = 1;
  std::fill(col(s, slot, 0), col(s, slot, 0) + (size_t)s->C * s->NCH, 0);
  return MOSHI_OK;
}

int moshi_stream_step(moshi_stream* s, const int32_t* user, const int32_t* forced,
                      int32_t* out_frames, int32_t* out_ready, int32_t* step_text,
                      int32_t* step_codes) {
  if (!s || !user || !out_frames || !out_ready) return MOSHI_E_INVALID;
  const int B = s->B, A = s->A, NU = s->S - s->A, NCH = s->NCH;
  // validate everything before any state moves
  std::vector<char> live(B, 0);
  for (int b = 0; b < B; ++b) {
    int64_t pos;
    if (moshi_session_info(s->ctx, b, &pos, nullptr, nullptr) != MOSHI_OK) continue;
    live[b] = 1;
    if (!s->reset_done[b] || pos != s->base[b] + s->t[b]) {
      s->err = "slot " + std::to_string(b) + ": its stream was not reset since the session joined";
      return MOSHI_E_INVALID;
    }
    for (int j = 0; j < NU; ++j) {
      const int32_t u = user[(size_t)b * NU + j];
      if (u < 0 || u >= s->Va) {
        s->err = "user code out of range";
        return MOSHI_E_INVALID;
      }
    }
    if (forced) {
      const int32_t* f = forced + (size_t)b * (1 + A);
      if (f[0] < -1 || f[0] >= s->Vt) {
        s->err = "forced text token out of range";
        return MOSHI_E_INVALID;
      }
      for (int k = 1; k <= A; ++k)
        if (f[k] < -1 || f[k] >= s->Va) {
          s->err = "forced code out of range";
          return MOSHI_E_INVALID;
        }
    }
  }
  // the user's frame t into column t + d_k; the input column t
  for (int b = 0; b < B; ++b) {
    int32_t* fr = s->frames.data() + (size_t)b * NCH;
    int32_t* fc = s->forced.data() + (size_t)b * NCH;
    std::fill(fc, fc + NCH, -1);
    if (!live[b]) {
      std::fill(fr, fr + NCH, 0);
      continue;
    }
    const int64_t t = s->t[b];
    for (int j = 0; j < NU; ++j) {
      const int k = A + 1 + j;
      col(s, b, t + s->delay[k])[k] = user[(size_t)b * NU + j];
    }
    for (int k = 0; k < NCH; ++k) {
      const bool generated = k <= A;
      if (t < s->delay[k] || (generated && t == 0))
        fr[k] = initial_token(s, k);
      else
        fr[k] = col(s, b, t)[k];
    }
    if (forced) {
      const int32_t* f = forced + (size_t)b * (1 + A);
      for (int k = 0; k <= A; ++k) fc[k] = f[k];
    }
  }
  int rc = moshi_step_forced(s->ctx, s->frames.data(), forced ? s->forced.data() : nullptr,
                             s->text.data(), s->codes.data());
  if (rc) {
    s->err = "step failed";
    return rc;
  }
  // column t+1 of the generated channels, then the frame that is complete
  for (int b = 0; b < B; ++b) {
    out_ready[b] = 0;
    for (int k = 0; k <= A; ++k) out_frames[(size_t)b * (1 + A) + k] = -1;
    if (step_text) step_text[b] = s->text[b];
    if (step_codes)
      memcpy(step_codes + (size_t)b * s->S, s->codes.data() + (size_t)b * s->S,
             sizeof(int32_t) * s->S);
    if (!live[b]) continue;
    const int64_t t = s->t[b];
    int32_t* nx = col(s, b, t + 1);
    nx[0] = s->text[b];
    for (int k = 1; k <= A; ++k) nx[k] = s->codes[(size_t)b * s->S + (k - 1)];
    s->t[b] = t + 1;
    const int64_t tau = t + 1 - s->D;
    if (tau >= 1) {
      for (int k = 0; k <= A; ++k)
        out_frames[(size_t)b * (1 + A) + k] = col(s, b, tau + s->delay[k])[k];
      out_ready[b] = 1;
    }
  }
  return MOSHI_OK;
}

const char* moshi_stream_last_error(const moshi_stream* s) { return s ? s->err.c_str() : ""; }

}  // extern "C"
