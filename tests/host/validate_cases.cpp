// Cases for libblock's host-side checks, workspace layout and rotary table
// (validate.cpp), built with the host compiler under the address and
// undefined-behaviour sanitizers by tests/test_host_sanitizers.py.  The
// pointers handed to the checks are addresses only: nothing dereferences them.
#include <limits.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "../../transformer_decoder_block_amd/csrc/validate.h"

static int g_cases = 0, g_failed = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    ++g_cases;                                                         \
    if (!(cond)) {                                                     \
      ++g_failed;                                                      \
      fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
    }                                                                  \
  } while (0)

// a status and a non-empty message
#define EXPECT_ST(expr, want)                                                    \
  do {                                                                           \
    const blk_status st_ = (expr);                                               \
    ++g_cases;                                                                   \
    if (st_ != (want) || (st_ != BLK_OK && blkv::last_error()[0] == 0)) {        \
      ++g_failed;                                                                \
      fprintf(stderr, "%s:%d: %s gave %s, want %s (%s)\n", __FILE__, __LINE__,   \
              #expr, blkv::status_str(st_), blkv::status_str(want),              \
              blkv::last_error());                                               \
    }                                                                            \
  } while (0)

static const void* A = (const void*)0x10000;   // a 16-byte aligned address
static const void* MIS = (const void*)0x10008; // not 16-byte aligned

static blk_config llama() {
  blk_config c;
  memset(&c, 0, sizeof(c));
  c.dtype = BLK_BF16;
  c.hidden = 4096;
  c.num_heads = 32;
  c.num_kv_heads = 32;
  c.head_dim = 128;
  c.mlp_kind = BLK_MLP_SWIGLU;
  c.intermediate = 11008;
  c.rms_eps = 1e-5f;
  c.rope_theta = 10000.f;
  c.use_rope = 1;
  c.max_batch = 4;
  c.max_seq = 2048;
  return c;
}

static blk_config afmoe() {
  blk_config c = llama();
  c.hidden = 2048;
  c.num_heads = 32;
  c.num_kv_heads = 4;
  c.head_dim = 64;
  c.mlp_kind = BLK_MLP_MOE;
  c.intermediate = 0;
  c.qk_norm = 1;
  c.sandwich_norm = 1;
  c.sliding_window = 2048;
  c.head_gate_dim = 32;
  c.num_experts = 128;
  c.top_k = 8;
  c.moe_intermediate = 1024;
  c.num_shared_experts = 1;
  c.route_scale = 2.5f;
  return c;
}

static blk_weights all_weights(const void* p) {
  blk_weights w;
  memset(&w, 0, sizeof(w));
  const void** f[] = {&w.w_in_norm, &w.w_post_attn_norm, &w.w_mlp_norm, &w.w_post_mlp_norm,
                      &w.wq, &w.wk, &w.wv, &w.wo, &w.w_q_norm, &w.w_k_norm, &w.w_head_gate,
                      &w.w_gate, &w.w_up, &w.w_down, &w.w_router, &w.w_e_gate, &w.w_e_up,
                      &w.w_e_down, &w.w_sh_gate, &w.w_sh_up, &w.w_sh_down};
  for (auto q : f) *q = p;
  w.expert_bias = (const float*)p;
  return w;
}

static void config_cases() {
  blk_config c = llama();
  EXPECT_ST(blkv::check_config(&c), BLK_OK);
  EXPECT_ST(blkv::check_config(nullptr), BLK_E_NULL);
  blk_config m = afmoe();
  EXPECT_ST(blkv::check_config(&m), BLK_OK);
  for (int kind : {BLK_MLP_RELU2, BLK_MLP_XIELU}) {
    blk_config d = llama();
    d.mlp_kind = kind;
    EXPECT_ST(blkv::check_config(&d), BLK_OK);
  }
  struct Bad {
    void (*set)(blk_config&);
  };
  const Bad dense_bad[] = {
      {[](blk_config& c) { c.dtype = 7; }},
      {[](blk_config& c) { c.dtype = BLK_I32; }},
      {[](blk_config& c) { c.hidden = 0; }},
      {[](blk_config& c) { c.hidden = -8; }},
      {[](blk_config& c) { c.hidden = 4100; }},
      {[](blk_config& c) { c.hidden = 8200; }},
      {[](blk_config& c) { c.hidden = INT_MAX; }},
      {[](blk_config& c) { c.hidden = INT_MIN; }},
      {[](blk_config& c) { c.num_heads = 0; }},
      {[](blk_config& c) { c.num_kv_heads = 0; }},
      {[](blk_config& c) { c.num_kv_heads = -1; }},
      {[](blk_config& c) { c.num_kv_heads = 5; }},
      {[](blk_config& c) { c.num_heads = INT_MIN; c.num_kv_heads = -1; }},
      {[](blk_config& c) { c.head_dim = 96; }},
      {[](blk_config& c) { c.head_dim = 0; }},
      {[](blk_config& c) { c.rms_eps = 0.f; }},
      {[](blk_config& c) { c.rms_eps = -1e-5f; }},
      {[](blk_config& c) { c.rms_eps = NAN; }},
      {[](blk_config& c) { c.rope_theta = 0.f; }},
      {[](blk_config& c) { c.rope_theta = NAN; }},
      {[](blk_config& c) { c.sliding_window = -1; }},
      {[](blk_config& c) { c.head_gate_dim = 7; }},
      // num_heads * head_dim overflows int32: the check must not overflow
      {[](blk_config& c) { c.num_heads = INT_MAX; c.num_kv_heads = 1; c.head_gate_dim = 5; }},
      {[](blk_config& c) { c.max_batch = 0; }},
      {[](blk_config& c) { c.max_seq = -3; }},
      {[](blk_config& c) { c.mlp_kind = 9; }},
      {[](blk_config& c) { c.intermediate = 0; }},
      {[](blk_config& c) { c.intermediate = 11007; }},
      // operand sizes past 32-bit byte offsets, products past int32 and int64
      {[](blk_config& c) { c.max_batch = 64; c.max_seq = 8192; }},
      {[](blk_config& c) { c.max_batch = INT_MAX; c.max_seq = INT_MAX; }},
      {[](blk_config& c) { c.intermediate = INT_MAX - 7; }},
      {[](blk_config& c) { c.num_heads = INT_MAX; c.num_kv_heads = 1; }},
  };
  for (const auto& b : dense_bad) {
    blk_config d = llama();
    b.set(d);
    EXPECT_ST(blkv::check_config(&d), BLK_E_CONFIG);
  }
  const Bad moe_bad[] = {
      {[](blk_config& c) { c.num_experts = 0; }},
      {[](blk_config& c) { c.num_experts = 257; }},
      {[](blk_config& c) { c.top_k = 0; }},
      {[](blk_config& c) { c.top_k = 17; }},
      {[](blk_config& c) { c.num_experts = 4; c.top_k = 5; }},
      {[](blk_config& c) { c.moe_intermediate = 0; }},
      {[](blk_config& c) { c.moe_intermediate = 12; }},
      {[](blk_config& c) { c.num_shared_experts = -1; }},
      {[](blk_config& c) { c.num_shared_experts = INT_MAX; }},
      {[](blk_config& c) { c.moe_intermediate = INT_MAX - 7; }},
      {[](blk_config& c) { c.head_gate_dim = 32 * 64 + 1; }},
  };
  for (const auto& b : moe_bad) {
    blk_config d = afmoe();
    b.set(d);
    EXPECT_ST(blkv::check_config(&d), BLK_E_CONFIG);
  }
  // one long sequence, well inside the 4e9-byte operand bound
  blk_config big = llama();
  big.max_batch = 1;
  big.max_seq = 40000;
  EXPECT_ST(blkv::check_config(&big), BLK_OK);
  blk_config gate = afmoe();
  gate.head_gate_dim = 32 * 64;  // per channel
  EXPECT_ST(blkv::check_config(&gate), BLK_OK);
}

static void io_cases() {
  const blk_config c = llama();
  blk_io io;
  memset(&io, 0, sizeof(io));
  io.x = A;
  io.y = (void*)0x20000;
  io.batch = 4;
  io.seq = 2048;
  EXPECT_ST(blkv::check_io(c, &io), BLK_OK);
  EXPECT_ST(blkv::check_io(c, nullptr), BLK_E_NULL);
  blk_io t = io;
  t.x = nullptr;
  EXPECT_ST(blkv::check_io(c, &t), BLK_E_NULL);
  t = io;
  t.y = nullptr;
  EXPECT_ST(blkv::check_io(c, &t), BLK_E_NULL);
  t = io;
  t.y = (void*)A;
  EXPECT_ST(blkv::check_io(c, &t), BLK_E_CONFIG);
  t = io;
  t.x = MIS;
  EXPECT_ST(blkv::check_io(c, &t), BLK_E_ALIGN);
  t = io;
  t.y = (void*)MIS;
  EXPECT_ST(blkv::check_io(c, &t), BLK_E_ALIGN);
  for (int b : {0, -1, 5, INT_MIN, INT_MAX}) {
    t = io;
    t.batch = b;
    EXPECT_ST(blkv::check_io(c, &t), BLK_E_SHAPE);
  }
  for (int s : {0, 2049, INT_MIN, INT_MAX}) {
    t = io;
    t.seq = s;
    EXPECT_ST(blkv::check_io(c, &t), BLK_E_SHAPE);
  }
  t = io;
  t.batch = 1;
  t.seq = 1;
  EXPECT_ST(blkv::check_io(c, &t), BLK_OK);
}

// every weight a configuration needs, one missing or misaligned at a time
static void weight_cases(const blk_config& c, int needed) {
  blk_weights w = all_weights(A);
  EXPECT_ST(blkv::check_weights(c, &w), BLK_OK);
  EXPECT_ST(blkv::check_weights(c, nullptr), BLK_E_NULL);
  const size_t nptr = offsetof(blk_weights, w_sh_down) / sizeof(void*) + 1;
  int n_null = 0, n_align = 0;
  for (size_t i = 0; i < nptr; ++i) {
    const size_t off = i * sizeof(void*);
    if (off == offsetof(blk_weights, xielu_alpha_p_raw) ||
        off == offsetof(blk_weights, xielu_alpha_n_raw))
      continue;
    blk_weights v = w;
    memset((char*)&v + off, 0, sizeof(void*));
    const blk_status s0 = blkv::check_weights(c, &v);
    EXPECT(s0 == BLK_OK || s0 == BLK_E_NULL);
    n_null += s0 == BLK_E_NULL;
    v = w;
    memcpy((char*)&v + off, &MIS, sizeof(void*));
    const blk_status s1 = blkv::check_weights(c, &v);
    EXPECT(s1 == BLK_OK || s1 == BLK_E_ALIGN);
    n_align += s1 == BLK_E_ALIGN;
    EXPECT((s0 == BLK_OK) == (s1 == BLK_OK));
  }
  EXPECT(n_null == needed);
  EXPECT(n_align == needed);
}

static void tap_cases(const blk_config& c, bool moe) {
  EXPECT_ST(blkv::check_taps(c, nullptr), BLK_OK);
  blk_taps t;
  memset(&t, 0, sizeof(t));
  EXPECT_ST(blkv::check_taps(c, &t), BLK_OK);
  const size_t ntap = sizeof(blk_taps) / sizeof(blk_tap);
  blk_tap* taps = (blk_tap*)&t;
  int allowed = 0;
  for (size_t i = 0; i < ntap; ++i) {
    // find the dtype this tap accepts (if it exists for this block)
    int ok_dtype = -1;
    for (int dt : {BLK_F32, BLK_BF16, BLK_I32}) {
      memset(&t, 0, sizeof(t));
      taps[i].ptr = (void*)A;
      taps[i].dtype = dt;
      if (blkv::check_taps(c, &t) == BLK_OK) {
        EXPECT(ok_dtype == -1);  // exactly one dtype
        ok_dtype = dt;
      }
    }
    if (ok_dtype < 0) {
      taps[i].dtype = BLK_F32;
      const blk_status s = blkv::check_taps(c, &t);
      EXPECT(s == BLK_E_CONFIG || s == BLK_E_DTYPE);
      continue;
    }
    ++allowed;
    memset(&t, 0, sizeof(t));
    taps[i].ptr = (void*)MIS;
    taps[i].dtype = ok_dtype;
    EXPECT_ST(blkv::check_taps(c, &t), BLK_E_ALIGN);
    taps[i].ptr = (void*)A;
    taps[i].dtype = ok_dtype == BLK_F32 ? BLK_I32 : BLK_F32;
    EXPECT_ST(blkv::check_taps(c, &t), BLK_E_DTYPE);
  }
  // dense: 17 taps (no router, expert or shared taps); MoE with a shared
  // expert: 21 (no dense neuron/activation taps)
  EXPECT(allowed == (moe ? 21 : 17));
  // every tap at once
  memset(&t, 0, sizeof(t));
  EXPECT_ST(blkv::check_forward(c, nullptr, nullptr, &t), BLK_E_NULL);
}

static void layout_cases(const blk_config& c, size_t hist_ints, size_t split) {
  blkv::WsLayout L;
  blkv::ws_layout(c, hist_ints, split, &L);
  // parts 256-byte aligned, disjoint and inside the total
  std::vector<std::pair<size_t, size_t>> parts;
  for (int p = 0; p < blkv::WS_NPARTS; ++p) {
    if (L.off[p] == blkv::WS_ABSENT) {
      EXPECT(L.bytes[p] == 0);
      continue;
    }
    EXPECT(L.off[p] % 256 == 0);
    parts.push_back({L.off[p], L.bytes[p]});
  }
  std::sort(parts.begin(), parts.end());
  size_t end = 0;
  for (const auto& q : parts) {
    EXPECT(q.first >= end);
    end = q.first + q.second;
    EXPECT(end <= L.total);
  }
  const int present = (int)parts.size();
  EXPECT(L.total % 256 == 0);
  EXPECT(L.total - end < 256);
  const size_t T = (size_t)c.max_batch * c.max_seq, es = blkv::esize(c.dtype);
  EXPECT(L.bytes[blkv::WS_A] == T * c.hidden * es);
  EXPECT(L.bytes[blkv::WS_MID] == T * c.hidden * 4);
  EXPECT(L.bytes[blkv::WS_SPLIT] == split);
  const bool moe = c.mlp_kind == BLK_MLP_MOE;
  EXPECT((L.off[blkv::WS_LOGITS] != blkv::WS_ABSENT) == moe);
  EXPECT((L.off[blkv::WS_ROPE_COS] != blkv::WS_ABSENT) == (bool)c.use_rope);
  EXPECT((L.off[blkv::WS_GATE] != blkv::WS_ABSENT) == (c.head_gate_dim > 0));
  if (moe) {
    EXPECT(L.bytes[blkv::WS_HIST] == hist_ints * 4);
    EXPECT(L.bytes[blkv::WS_NEUR] == T * c.top_k * c.moe_intermediate * es);
  } else {
    EXPECT(L.bytes[blkv::WS_NEUR] == T * blkv::neuron_ld(c.intermediate) * es);
    EXPECT(blkv::neuron_ld(c.intermediate) % 64 == 0);
    EXPECT(blkv::neuron_ld(c.intermediate) >= (size_t)c.intermediate);
  }
  EXPECT(present >= 10);
}

static void rope_cases() {
  blk_config c = llama();
  c.head_dim = 64;
  const int S = 37, half = 32;
  // exact-size buffers: an index past the table trips the address sanitizer
  std::vector<float> cs(S * half), sn(S * half);
  blkv::rope_table(c, S, cs.data(), sn.data());
  for (int s = 0; s < S; ++s)
    for (int i = 0; i < half; ++i) {
      const double ang = s / pow(10000.0, (2.0 * i) / 64.0);
      EXPECT(fabs(cs[s * half + i] - cos(ang)) < 1e-6);
      EXPECT(fabs(sn[s * half + i] - sin(ang)) < 1e-6);
    }
  EXPECT(cs[0] == 1.f && sn[0] == 0.f);
  blkv::rope_table(c, 0, nullptr, nullptr);  // no positions: touches nothing
}

int main() {
  config_cases();
  io_cases();
  blk_config d = llama();
  weight_cases(d, 9);  // norms 2, q/k/v/o 4, gate/up/down 3
  blk_config m = afmoe();
  weight_cases(m, 19);  // norms 4, q/k/v/o 4, q/k norm 2, gate 1, router + bias +
                        // experts 5, shared expert 3
  blk_config r = llama();
  r.mlp_kind = BLK_MLP_RELU2;
  weight_cases(r, 8);
  tap_cases(d, false);
  tap_cases(m, true);
  for (int rope = 0; rope < 2; ++rope) {
    blk_config a = llama();
    a.use_rope = rope;
    layout_cases(a, 0, 0);
    layout_cases(a, 0, 128 * 2 * 256 * 256 * 4);
    blk_config b = afmoe();
    b.use_rope = rope;
    layout_cases(b, 128 * 128, 0);
    b.num_shared_experts = 0;
    b.head_gate_dim = 0;
    layout_cases(b, 7, 1000);
  }
  for (int s : {BLK_OK, BLK_E_NULL, BLK_E_CONFIG, BLK_E_SHAPE, BLK_E_ALIGN, BLK_E_DTYPE,
                BLK_E_OOM, BLK_E_HIP})
    EXPECT(strncmp(blkv::status_str((blk_status)s), "BLK_", 4) == 0);
  EXPECT(strcmp(blkv::status_str((blk_status)12345), "BLK_E_UNKNOWN") == 0);
  rope_cases();
  printf("%d cases, %d failed\n", g_cases, g_failed);
  return g_failed ? 1 : 0;
}
