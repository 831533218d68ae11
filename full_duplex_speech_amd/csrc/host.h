// host.h -- the host-only logic of libmoshi.so that needs no GPU: config
// validation, the weight-tensor count, frame validation and the session slot
// table. Plain C++ (no HIP types), so it also builds into the CPU sanitizer
// checks under tests/sanitize/.
//
// Slots: sessions join the lowest free slot, a full engine refuses joins, a
// recycled slot starts like a fresh one ("vLLM-Omni recipe: PersonaPlex",
// "Notes"). A slot's position is the number of frames it has consumed (the
// RoPE position, which mobius PR #368 "P2 - Moshi LM" derives from the cache
// length); fill = min(pos, W), write index = pos mod W.
#pragma once

#include <stdint.h>

#include <vector>

#include "../../include/moshi.h"

namespace moshi_host {

// Depformer substeps a config runs (dep_q, 0 = all n_substeps).
inline int dep_steps(const moshi_config* c) {
  return (c->dep_q > 0 && c->dep_q < c->n_substeps) ? c->dep_q : c->n_substeps;
}

inline bool valid_head_dim(int hd) { return hd == 32 || hd == 64 || hd == 128; }

// Weight tensors moshi_create expects (include/moshi.h lists the order).
inline int32_t tensor_count(const moshi_config* c) {
  const int S = c->n_substeps, L = c->n_layers, Ld = c->dep_layers;
  const int extra = (c->flags & MOSHI_FLAG_DEP_FINAL_NORM) ? 1 : 0;
  return 1 + S + 6 * L + 2 + S + S + 2 * Ld + 4 * S * Ld + S + extra;
}

constexpr uint32_t kKnownFlags = MOSHI_FLAG_MASK_OLDEST | MOSHI_FLAG_DEP_FINAL_NORM |
                                 MOSHI_FLAG_DEP_REF_RING | MOSHI_FLAG_SAMPLING;
// Largest vocabulary the sampling kernel takes (1024 threads x 32 values).
constexpr int kMaxSampledVocab = 32768;

// Largest window the attention kernels accept (64-key spans, 512 of them).
constexpr int kMaxWindow = 64 * 512;

// nullptr if the config is usable, else what is wrong with it.
inline const char* config_error(const moshi_config* c) {
  if (!c) return "config is NULL";
  if (c->dtype != MOSHI_F32 && c->dtype != MOSHI_BF16) return "dtype must be MOSHI_F32 or MOSHI_BF16";
  const int vec = c->dtype == MOSHI_BF16 ? 8 : 4;
  if (c->dim <= 0 || c->n_heads <= 0 || c->dim % c->n_heads) return "dim must be a positive multiple of n_heads";
  if (!valid_head_dim(c->dim / c->n_heads)) return "temporal head_dim must be 32, 64 or 128";
  if (c->dep_dim <= 0 || c->dep_heads <= 0 || c->dep_dim % c->dep_heads) return "dep_dim must be a positive multiple of dep_heads";
  if (!valid_head_dim(c->dep_dim / c->dep_heads)) return "depformer head_dim must be 32, 64 or 128";
  if (c->n_layers < 1 || c->dep_layers < 1) return "n_layers and dep_layers must be >= 1";
  if (c->n_substeps < 1 || c->n_substeps > 64) return "n_substeps must be in [1, 64]";
  if (c->dep_q < 0 || c->dep_q > c->n_substeps) return "dep_q must be in [0, n_substeps]";
  if (c->ffn_hidden <= 0 || c->dep_ffn_hidden <= 0) return "ffn widths must be positive";
  if (c->dim % vec || c->ffn_hidden % vec || c->dep_dim % vec || c->dep_ffn_hidden % vec)
    return "widths must be multiples of 8 (bf16) / 4 (fp32)";
  if (c->window < 1 || c->window > kMaxWindow) return "window must be in [1, 32768]";
  {
    const int esz = c->dtype == MOSHI_BF16 ? 2 : 4;
    const int kmax = c->ffn_hidden > c->dim ? c->ffn_hidden : c->dim;
    if ((long)kmax * esz > 49152 || (long)c->dep_ffn_hidden * esz > 49152)
      return "projection inputs must fit 48 KB of LDS (ffn_hidden * element size)";
  }
  if ((c->flags & MOSHI_FLAG_MASK_OLDEST) && c->window < 2) return "mask-oldest needs window >= 2";
  if ((c->flags & MOSHI_FLAG_DEP_REF_RING) && dep_steps(c) < 2)
    return "the depformer ring reading needs at least 2 substeps";
  if (c->flags & ~kKnownFlags) return "unknown flag bits";
  if ((c->flags & MOSHI_FLAG_SAMPLING) &&
      (c->text_vocab > kMaxSampledVocab || c->audio_card > kMaxSampledVocab))
    return "sampling takes vocabularies of at most 32768 entries";
  if (c->text_vocab < 2 || c->audio_card < 2) return "vocabularies must have >= 2 entries";
  if (c->max_sessions < 1 || c->max_sessions > 64) return "max_sessions must be in [1, 64]";
  if (!(c->rope_theta > 0.0) || !(c->norm_eps >= 0.0)) return "rope_theta must be > 0 and norm_eps >= 0";
  return nullptr;
}

// The per-slot bookkeeping the host keeps (the device holds a mirror of
// liveness and positions, refreshed when `dirty`).
struct SlotTable {
  std::vector<int> live;
  std::vector<int64_t> pos;
  bool dirty = true;

  void init(int B) {
    live.assign(B, 0);
    pos.assign(B, 0);
    dirty = true;
  }
  int capacity() const { return (int)live.size(); }
  bool is_live(int slot) const { return slot >= 0 && slot < capacity() && live[slot]; }
  int live_count() const {
    int n = 0;
    for (int v : live) n += v;
    return n;
  }
  // Lowest free slot, or -1 when every slot is live.
  int join() {
    for (int b = 0; b < capacity(); ++b)
      if (!live[b]) {
        live[b] = 1;
        pos[b] = 0;
        dirty = true;
        return b;
      }
    return -1;
  }
  bool leave(int slot) {
    if (!is_live(slot)) return false;
    live[slot] = 0;
    pos[slot] = 0;
    dirty = true;
    return true;
  }
  // A prefill of n positions: the next frame is at position n.
  bool set_pos(int slot, int64_t n) {
    if (!is_live(slot) || n < 0) return false;
    pos[slot] = n;
    dirty = true;
    return true;
  }
  // After a step: every live slot consumed one frame (the device advanced
  // its own copy, so the mirror stays clean).
  void advance() {
    for (int b = 0; b < capacity(); ++b)
      if (live[b]) pos[b] += 1;
  }
  void info(int slot, int window, int64_t* p, int32_t* fill, int32_t* widx) const {
    const int64_t q = pos[slot];
    if (p) *p = q;
    if (fill) *fill = (int32_t)(q < window ? q : window);
    if (widx) *widx = (int32_t)(q % window);
  }
};

// nullptr if every live row of frames [B][1+S] holds codes in range (text in
// [0, Vt], audio in [0, Va]); else what is wrong.
inline const char* frames_error(const SlotTable& t, const int32_t* frames, int n_ch, int Vt, int Va) {
  if (!frames) return "frames is NULL";
  for (int b = 0; b < t.capacity(); ++b) {
    if (!t.live[b]) continue;
    const int32_t* f = frames + (size_t)b * n_ch;
    if (f[0] < 0 || f[0] > Vt) return "text code out of range";
    for (int k = 1; k < n_ch; ++k)
      if (f[k] < 0 || f[k] > Va) return "audio code out of range";
  }
  return nullptr;
}

// nullptr if every live row of forced [B][1+S] is -1 (not forced) or a valid
// token: text in [0, Vt), code s in [0, Va).
inline const char* forced_error(const SlotTable& t, const int32_t* forced, int n_ch, int Vt, int Va) {
  if (!forced) return nullptr;
  for (int b = 0; b < t.capacity(); ++b) {
    if (!t.live[b]) continue;
    const int32_t* f = forced + (size_t)b * n_ch;
    if (f[0] < -1 || f[0] >= Vt) return "forced text token out of range";
    for (int k = 1; k < n_ch; ++k)
      if (f[k] < -1 || f[k] >= Va) return "forced code out of range";
  }
  return nullptr;
}

}  // namespace moshi_host
