// Host-side argument checks, workspace layout and rotary table of libblock
// (no HIP: see validate.h).
#include "validate.h"

#include <math.h>

namespace blkv {

namespace {
thread_local std::string g_err;
}  // namespace

blk_status fail(blk_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

const char* last_error() { return g_err.c_str(); }

const char* status_str(blk_status s) {
  switch (s) {
    case BLK_OK: return "BLK_OK";
    case BLK_E_NULL: return "BLK_E_NULL";
    case BLK_E_CONFIG: return "BLK_E_CONFIG";
    case BLK_E_SHAPE: return "BLK_E_SHAPE";
    case BLK_E_ALIGN: return "BLK_E_ALIGN";
    case BLK_E_DTYPE: return "BLK_E_DTYPE";
    case BLK_E_OOM: return "BLK_E_OOM";
    case BLK_E_HIP: return "BLK_E_HIP";
  }
  return "BLK_E_UNKNOWN";
}

size_t esize(int dtype) { return dtype == BLK_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

size_t neuron_ld(int I) { return ((size_t)I + 63) & ~(size_t)63; }

blk_status check_config(const blk_config* c) {
  if (!c) return fail(BLK_E_NULL, "cfg must not be NULL");
  if (c->dtype != BLK_F32 && c->dtype != BLK_BF16)
    return fail(BLK_E_CONFIG, "dtype must be BLK_F32 or BLK_BF16");
  if (c->hidden <= 0 || c->hidden % 8 || c->hidden > 8192)
    return fail(BLK_E_CONFIG, "hidden must be a positive multiple of 8, at most 8192");
  if (c->num_heads <= 0 || c->num_kv_heads <= 0 || c->num_heads % c->num_kv_heads)
    return fail(BLK_E_CONFIG, "num_heads must be a positive multiple of num_kv_heads");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(BLK_E_CONFIG, "head_dim must be 64 or 128");
  if (!(c->rms_eps > 0.f)) return fail(BLK_E_CONFIG, "rms_eps must be > 0");
  if (c->use_rope && !(c->rope_theta > 0.f))
    return fail(BLK_E_CONFIG, "rope_theta must be > 0");
  if (c->sliding_window < 0) return fail(BLK_E_CONFIG, "sliding_window must be >= 0");
  const int64_t G = c->head_gate_dim;
  if (G != 0 && G != c->num_heads && G != (int64_t)c->num_heads * c->head_dim)
    return fail(BLK_E_CONFIG, "head_gate_dim must be 0, num_heads or num_heads*head_dim");
  if (c->max_batch <= 0 || c->max_seq <= 0)
    return fail(BLK_E_CONFIG, "max_batch and max_seq must be >= 1");
  switch (c->mlp_kind) {
    case BLK_MLP_SWIGLU:
    case BLK_MLP_RELU2:
    case BLK_MLP_XIELU:
      if (c->intermediate <= 0 || c->intermediate % 8)
        return fail(BLK_E_CONFIG, "intermediate must be a positive multiple of 8");
      break;
    case BLK_MLP_MOE:
      if (c->num_experts <= 0 || c->num_experts > 256)
        return fail(BLK_E_CONFIG, "num_experts must be in [1, 256]");
      if (c->top_k <= 0 || c->top_k > 16 || c->top_k > c->num_experts)
        return fail(BLK_E_CONFIG, "top_k must be in [1, min(16, num_experts)]");
      if (c->moe_intermediate <= 0 || c->moe_intermediate % 8)
        return fail(BLK_E_CONFIG, "moe_intermediate must be a positive multiple of 8");
      if (c->num_shared_experts < 0)
        return fail(BLK_E_CONFIG, "num_shared_experts must be >= 0");
      break;
    default:
      return fail(BLK_E_CONFIG, "unknown mlp_kind");
  }
  // every GEMM operand is addressed with 32-bit byte offsets (products in
  // double: the factors are ints that may be as large as INT_MAX)
  const double T = (double)c->max_batch * c->max_seq;
  const double es = (double)esize(c->dtype);
  double big = T * c->hidden * es;
  big = fmax(big, T * c->num_heads * c->head_dim * es);
  if (c->mlp_kind == BLK_MLP_MOE) {
    big = fmax(big, T * c->top_k * c->moe_intermediate * es);
    big = fmax(big, T * c->moe_intermediate * c->num_shared_experts * es);
    big = fmax(big, (double)c->num_experts * c->moe_intermediate * c->hidden * es);
  } else {
    big = fmax(big, T * c->intermediate * es);
    big = fmax(big, (double)c->intermediate * c->hidden * es);
  }
  if (big > 4.0e9)
    return fail(BLK_E_CONFIG, "an operand would exceed 4e9 bytes; lower max_batch*max_seq");
  return BLK_OK;
}

blk_status check_io(const blk_config& c, const blk_io* io) {
  if (!io) return fail(BLK_E_NULL, "io must not be NULL");
  if (!io->x || !io->y) return fail(BLK_E_NULL, "io.x and io.y must not be NULL");
  if (io->x == io->y) return fail(BLK_E_CONFIG, "io.y must not alias io.x");
  if (!aligned16(io->x) || !aligned16(io->y))
    return fail(BLK_E_ALIGN, "io.x and io.y must be 16-byte aligned");
  if (io->batch < 1 || io->seq < 1 || io->batch > c.max_batch || io->seq > c.max_seq)
    return fail(BLK_E_SHAPE, "batch/seq must be in [1, max_batch] x [1, max_seq]");
  return BLK_OK;
}

namespace {

struct WNeed {
  const char* name;
  const void* p;
  bool needed;
};

struct TapCheck {
  const char* name;
  const blk_tap* tap;
  int want;  // required dtype
  bool allowed;
};

}  // namespace

blk_status check_weights(const blk_config& c, const blk_weights* w) {
  if (!w) return fail(BLK_E_NULL, "weights must not be NULL");
  const int k = c.mlp_kind;
  const bool moe = k == BLK_MLP_MOE;
  const bool shared = moe && c.num_shared_experts > 0;
  const WNeed list[] = {
      {"w_in_norm", w->w_in_norm, true},
      {"w_post_attn_norm", w->w_post_attn_norm, (bool)c.sandwich_norm},
      {"w_mlp_norm", w->w_mlp_norm, true},
      {"w_post_mlp_norm", w->w_post_mlp_norm, (bool)c.sandwich_norm},
      {"wq", w->wq, true},
      {"wk", w->wk, true},
      {"wv", w->wv, true},
      {"wo", w->wo, true},
      {"w_q_norm", w->w_q_norm, (bool)c.qk_norm},
      {"w_k_norm", w->w_k_norm, (bool)c.qk_norm},
      {"w_head_gate", w->w_head_gate, c.head_gate_dim > 0},
      {"w_gate", w->w_gate, k == BLK_MLP_SWIGLU},
      {"w_up", w->w_up, k == BLK_MLP_SWIGLU || k == BLK_MLP_RELU2 || k == BLK_MLP_XIELU},
      {"w_down", w->w_down, !moe},
      {"w_router", w->w_router, moe},
      {"expert_bias", w->expert_bias, moe},
      {"w_e_gate", w->w_e_gate, moe},
      {"w_e_up", w->w_e_up, moe},
      {"w_e_down", w->w_e_down, moe},
      {"w_sh_gate", w->w_sh_gate, shared},
      {"w_sh_up", w->w_sh_up, shared},
      {"w_sh_down", w->w_sh_down, shared},
  };
  for (const auto& n : list) {
    if (!n.needed) continue;
    if (!n.p) return fail(BLK_E_NULL, std::string("weight ") + n.name + " is NULL");
    if (!aligned16(n.p))
      return fail(BLK_E_ALIGN, std::string("weight ") + n.name + " is not 16-byte aligned");
  }
  return BLK_OK;
}

blk_status check_taps(const blk_config& c, const blk_taps* t) {
  if (!t) return BLK_OK;
  const int md = c.dtype;
  const bool moe = c.mlp_kind == BLK_MLP_MOE;
  const TapCheck list[] = {
      {"layer_input", &t->layer_input, md, true},
      {"attention_norm_output", &t->attention_norm_output, md, true},
      {"attention_scores", &t->attention_scores, BLK_F32, true},
      {"layer_mid", &t->layer_mid, BLK_F32, true},
      {"mlp_input", &t->mlp_input, md, true},
      {"layer_output", &t->layer_output, BLK_F32, true},
      {"attention_output", &t->attention_output, BLK_F32, true},
      {"mlp_output", &t->mlp_output, BLK_F32, true},
      {"router_logits", &t->router_logits, md, moe},
      {"expert_indices", &t->expert_indices, BLK_I32, moe},
      {"expert_weights", &t->expert_weights, BLK_F32, moe},
      {"attention_queries", &t->attention_queries, md, true},
      {"attention_keys", &t->attention_keys, md, true},
      {"attention_values", &t->attention_values, md, true},
      {"attention_probabilities", &t->attention_probabilities, BLK_F32, true},
      {"attention_head_outputs", &t->attention_head_outputs, md, true},
      {"attention_premix", &t->attention_premix, md, true},
      {"mlp_neurons", &t->mlp_neurons, md, !moe},
      {"mlp_activation", &t->mlp_activation, md, !moe},
      {"mlp_norm_output", &t->mlp_norm_output, md, true},
      {"expert_outputs", &t->expert_outputs, md, moe},
      {"routed_output", &t->routed_output, BLK_F32, moe},
      {"shared_expert_output", &t->shared_expert_output, BLK_F32,
       moe && c.num_shared_experts > 0},
  };
  for (const auto& e : list) {
    if (!e.tap->ptr) continue;
    if (!e.allowed)
      return fail(BLK_E_CONFIG, std::string("tap ") + e.name +
                                    " does not exist for this block's mlp_kind");
    if (e.tap->dtype != e.want)
      return fail(BLK_E_DTYPE, std::string("tap ") + e.name + " must be requested as dtype " +
                                   std::to_string(e.want));
    if (!aligned16(e.tap->ptr))
      return fail(BLK_E_ALIGN, std::string("tap ") + e.name + " is not 16-byte aligned");
  }
  return BLK_OK;
}

blk_status check_forward(const blk_config& c, const blk_io* io, const blk_weights* w,
                         const blk_taps* t) {
  if (!io || !w) return fail(BLK_E_NULL, "handle, io and weights must not be NULL");
  blk_status st = check_io(c, io);
  if (st != BLK_OK) return st;
  st = check_weights(c, w);
  if (st != BLK_OK) return st;
  return check_taps(c, t);
}

void ws_layout(const blk_config& c, size_t hist_ints, size_t split_bytes, WsLayout* L) {
  for (int i = 0; i < WS_NPARTS; ++i) {
    L->off[i] = WS_ABSENT;
    L->bytes[i] = 0;
  }
  const size_t es = esize(c.dtype);
  const size_t T = (size_t)c.max_batch * c.max_seq;
  const size_t H = c.hidden, nh = c.num_heads, nkv = c.num_kv_heads, hd = c.head_dim;
  const size_t Sp = ((size_t)c.max_seq + 63) & ~(size_t)63;
  const bool moe = c.mlp_kind == BLK_MLP_MOE;
  const size_t kk = moe ? c.top_k : 0;
  size_t off = 0;
  auto add = [&](WsPart part, size_t bytes) {
    L->off[part] = off;
    L->bytes[part] = bytes;
    off += (bytes + 255) & ~(size_t)255;
  };
  add(WS_A, T * H * es);
  add(WS_Q, T * nh * hd * es);
  add(WS_K, T * nkv * hd * es);
  add(WS_VT, (size_t)c.max_batch * nkv * hd * Sp * es);
  if (c.head_gate_dim) add(WS_GATE, T * c.head_gate_dim * 4);
  add(WS_PREMIX, T * nh * hd * es);
  if (c.sandwich_norm) add(WS_O, T * H * 4);
  add(WS_MID, T * H * 4);
  add(WS_M, T * H * es);
  add(WS_LAYER_OUT, T * H * es);
  if (!moe) {
    add(WS_NEUR, T * neuron_ld(c.intermediate) * es);
    if (c.sandwich_norm) add(WS_MLP_RAW, T * H * 4);
  } else {
    const size_t E = c.num_experts;
    add(WS_LOGITS, T * E * es);
    add(WS_EIDX, T * kk * 4);
    add(WS_EW, T * kk * 4);
    add(WS_GCNT, E * 4);
    add(WS_GOFF, E * 4);
    add(WS_HIST, hist_ints * 4);
    add(WS_ROW_TOKEN, T * kk * 4);
    add(WS_PAIR_ROW, T * kk * 4);
    add(WS_ROW_WEIGHT, T * kk * 4);
    add(WS_NEUR, T * kk * c.moe_intermediate * es);
    add(WS_STAGE, T * kk * H * es);
    if (c.num_shared_experts > 0) {
      add(WS_NSH, T * (size_t)c.moe_intermediate * c.num_shared_experts * es);
      add(WS_MLP_RAW, T * H * 4);
    }
  }
  if (c.use_rope) {
    add(WS_ROPE_COS, (size_t)c.max_seq * (hd / 2) * 4);
    add(WS_ROPE_SIN, (size_t)c.max_seq * (hd / 2) * 4);
  }
  add(WS_SPLIT, split_bytes);
  L->total = off;
}

void rope_table(const blk_config& c, int S, float* cs, float* sn) {
  const size_t hd = c.head_dim, half = hd / 2;
  for (size_t s = 0; s < (size_t)S; ++s)
    for (size_t i = 0; i < half; ++i) {
      const double inv_freq = pow((double)c.rope_theta, -2.0 * (double)i / (double)hd);
      const double phi = (double)s * inv_freq;
      cs[s * half + i] = (float)cos(phi);
      sn[s * half + i] = (float)sin(phi);
    }
}

}  // namespace blkv
