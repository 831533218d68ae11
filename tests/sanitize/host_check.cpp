// CPU check of libmoshi.so's host-only logic (config validation, weight
// count, slot table, frame and forced-token validation), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitize.py.
// Exits 0 when every expectation holds; prints the first failure otherwise.
#include <stdio.h>
#include <string.h>

#include <vector>

#include "host.h"

using namespace moshi_host;

static int failures = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                 \
    }                                                             \
  } while (0)

static moshi_config good() {
  moshi_config c;
  memset(&c, 0, sizeof(c));
  c.dim = 384; c.n_layers = 2; c.n_heads = 3; c.ffn_hidden = 1000; c.window = 37;
  c.dep_dim = 192; c.dep_layers = 2; c.dep_heads = 3; c.dep_ffn_hidden = 520; c.n_substeps = 16;
  c.text_vocab = 1000; c.audio_card = 300; c.rope_theta = 1e4; c.norm_eps = 1e-8;
  c.dtype = MOSHI_BF16; c.max_sessions = 4; c.flags = 0; c.dep_q = 0;
  return c;
}

static void check_config() {
  moshi_config c = good();
  EXPECT(config_error(&c) == nullptr);
  EXPECT(config_error(nullptr) != nullptr);
  EXPECT(tensor_count(&c) == 1 + 16 + 12 + 2 + 16 + 16 + 4 + 128 + 16);
  c.flags = MOSHI_FLAG_DEP_FINAL_NORM;
  EXPECT(config_error(&c) == nullptr && tensor_count(&c) == 212);
  struct Bad {
    void (*edit)(moshi_config&);
  } bad[] = {
      {[](moshi_config& x) { x.dtype = 7; }},
      {[](moshi_config& x) { x.dim = 385; }},
      {[](moshi_config& x) { x.n_heads = 0; }},
      {[](moshi_config& x) { x.n_heads = 2; }},  // head dim 192
      {[](moshi_config& x) { x.dep_heads = 5; }},
      {[](moshi_config& x) { x.n_layers = 0; }},
      {[](moshi_config& x) { x.n_substeps = 65; }},
      {[](moshi_config& x) { x.dep_q = 17; }},
      {[](moshi_config& x) { x.dep_q = -1; }},
      {[](moshi_config& x) { x.ffn_hidden = 1004; }},  // not a multiple of 8
      {[](moshi_config& x) { x.window = 0; }},
      {[](moshi_config& x) { x.window = kMaxWindow + 1; }},
      {[](moshi_config& x) { x.ffn_hidden = 24576 + 8; }},
      {[](moshi_config& x) { x.flags = 1u << 9; }},
      {[](moshi_config& x) { x.flags = MOSHI_FLAG_MASK_OLDEST; x.window = 1; }},
      {[](moshi_config& x) { x.flags = MOSHI_FLAG_DEP_REF_RING; x.dep_q = 1; }},
      {[](moshi_config& x) { x.text_vocab = 1; }},
      {[](moshi_config& x) { x.max_sessions = 65; }},
      {[](moshi_config& x) { x.max_sessions = 0; }},
      {[](moshi_config& x) { x.rope_theta = 0.0; }},
      {[](moshi_config& x) { x.norm_eps = -1.0; }},
  };
  for (auto& b : bad) {
    moshi_config x = good();
    b.edit(x);
    EXPECT(config_error(&x) != nullptr);
  }
  c = good();
  c.dep_q = 8;
  EXPECT(config_error(&c) == nullptr && dep_steps(&c) == 8);
  c.dep_q = 0;
  EXPECT(dep_steps(&c) == 16);
}

static void check_slots() {
  SlotTable t;
  t.init(3);
  EXPECT(t.capacity() == 3 && t.live_count() == 0);
  EXPECT(t.join() == 0 && t.join() == 1 && t.join() == 2);
  EXPECT(t.join() == -1);  // full
  EXPECT(t.leave(1) && !t.leave(1) && !t.leave(-1) && !t.leave(3));
  EXPECT(t.join() == 1);  // lowest free slot, fresh
  EXPECT(t.pos[1] == 0);
  EXPECT(t.set_pos(2, 37) && !t.set_pos(2, -1) && !t.set_pos(5, 1));
  t.dirty = false;
  t.advance();
  EXPECT(!t.dirty && t.pos[0] == 1 && t.pos[1] == 1 && t.pos[2] == 38);
  int64_t p = 0;
  int32_t fill = 0, widx = 0;
  t.info(2, 37, &p, &fill, &widx);
  EXPECT(p == 38 && fill == 37 && widx == 1);
  t.info(0, 37, &p, &fill, &widx);
  EXPECT(p == 1 && fill == 1 && widx == 1);
  EXPECT(t.leave(0));
  t.advance();
  EXPECT(t.pos[0] == 0);  // free slots do not move
  EXPECT(!t.is_live(0) && t.is_live(2) && !t.is_live(-4) && !t.is_live(99));
}

static void check_frames() {
  SlotTable t;
  t.init(2);
  t.join();  // slot 0 live, slot 1 free
  const int n_ch = 17, Vt = 1000, Va = 300;
  std::vector<int32_t> f(2 * n_ch, 0);
  EXPECT(frames_error(t, f.data(), n_ch, Vt, Va) == nullptr);
  EXPECT(frames_error(t, nullptr, n_ch, Vt, Va) != nullptr);
  f[0] = Vt;  // the initial text token is a valid input
  f[16] = Va;
  EXPECT(frames_error(t, f.data(), n_ch, Vt, Va) == nullptr);
  f[0] = Vt + 1;
  EXPECT(frames_error(t, f.data(), n_ch, Vt, Va) != nullptr);
  f[0] = 0;
  f[5] = -1;
  EXPECT(frames_error(t, f.data(), n_ch, Vt, Va) != nullptr);
  f[5] = 0;
  f[n_ch + 3] = -77;  // a free row is ignored
  EXPECT(frames_error(t, f.data(), n_ch, Vt, Va) == nullptr);
  std::vector<int32_t> g(2 * n_ch, -1);
  EXPECT(forced_error(t, nullptr, n_ch, Vt, Va) == nullptr);
  EXPECT(forced_error(t, g.data(), n_ch, Vt, Va) == nullptr);
  g[0] = Vt - 1;
  g[16] = Va - 1;
  EXPECT(forced_error(t, g.data(), n_ch, Vt, Va) == nullptr);
  g[0] = Vt;  // the initial token is not a token the head can produce
  EXPECT(forced_error(t, g.data(), n_ch, Vt, Va) != nullptr);
  g[0] = -1;
  g[3] = -2;
  EXPECT(forced_error(t, g.data(), n_ch, Vt, Va) != nullptr);
  g[3] = -1;
  g[n_ch + 1] = 12345;  // free row
  EXPECT(forced_error(t, g.data(), n_ch, Vt, Va) == nullptr);
}

int main() {
  check_config();
  check_slots();
  check_frames();
  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("host checks ok\n");
  return 0;
}
