// libblock runtime: configuration checks, workspace, rotary table and the
// kernel sequence of one decoder block, behind the C ABI of libblock.h.
//
// The sequence (granite sheet "LlamaForCausalLM 32L-4096d", section
// "Implementing it"; nnterp arcee/afmoe/apertus pages, section 03):
//   rmsnorm -> fused Q/K/V(/gate) GEMM with q/k norm + rotary epilogue ->
//   flash attention (+ head gate) -> o_proj GEMM (+ residual, or afmoe
//   post-norm + residual + pre-MLP norm) -> MLP norm -> MLP GEMMs with the
//   activation fused into the first and the residual into the last (afmoe:
//   router, top-k, dispatch, grouped expert GEMMs, shared expert, combine
//   with post-MLP norm and residual).
// The residual stream (layer_mid, the pre-rounding layer_output) is kept in
// float32 inside the block; GEMM operands are in the model dtype.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/libblock.h"
#include "kernels.h"

using namespace blk;

namespace {

thread_local std::string g_err;

blk_status fail(blk_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

size_t esize(int dtype) { return dtype == BLK_BF16 ? 2 : 4; }

}  // namespace

struct blk_handle {
  blk_config cfg;
  int device = 0;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  // workspace views
  void *a = nullptr, *q = nullptr, *k = nullptr, *vt = nullptr, *premix = nullptr,
       *m = nullptr, *neur = nullptr, *logits = nullptr, *stage = nullptr, *nsh = nullptr,
       *layer_out = nullptr;  // blk_forward_layers: outputs of the layers before the last
  float* split = nullptr;  // GEMM tail-split partial tiles
  size_t split_bytes = 0;
  float *gate = nullptr, *o = nullptr, *mid = nullptr, *mlp_raw = nullptr, *ew = nullptr,
        *rope_cos = nullptr, *rope_sin = nullptr;
  int *eidx = nullptr, *gcnt = nullptr, *goff = nullptr, *row_token = nullptr,
      *pair_row = nullptr, *hist = nullptr;
  float* row_weight = nullptr;  // slot weight of each expert-ordered row
  // optional per-kernel event timing (blk_profile_begin / blk_profile_end)
  std::vector<hipEvent_t> pev;
  std::vector<const char*> pname;  // name of the span each mark opens
  int pmax = 0, pfwd = 0, pmarks = 0;
};

static constexpr int PROF_MARKS = 32;  // marks per forward

// Scratch for the GEMMs' tail split: up to 128 float32 tiles of 256 x 256,
// two K halves each.
static constexpr size_t SPLIT_WS_BYTES = (size_t)128 * 2 * 256 * 256 * 4;

// Record a timing mark on the stream: the span from this mark to the next
// one is charged to `name`.
static void prof_mark(blk_handle* h, const char* name, hipStream_t s) {
  if (h->pmax == 0 || h->pfwd >= h->pmax || h->pmarks >= PROF_MARKS) return;
  const int i = h->pfwd * PROF_MARKS + h->pmarks;
  hipEventRecord(h->pev[i], s);
  if (h->pfwd == 0) h->pname[h->pmarks] = name;
  ++h->pmarks;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Row stride of the dense MLP's neuron buffer: the width rounded up to 64
// elements, so that every 128-byte K stage of the down projection's A rows
// is one cache line (the pad columns are never read: K stays the width).
static size_t neuron_ld(int I) { return ((size_t)I + 63) & ~(size_t)63; }

// Lay the workspace of h->cfg (sized for max_batch * max_seq tokens) out
// from `base` and return its size in bytes; with base == nullptr only the
// size is computed.  Every part starts on a 256-byte boundary.  The GEMMs'
// K-split scratch gets split_bytes.  Allocates nothing.
static size_t carve(blk_handle* h, char* base, size_t split_bytes) {
  const blk_config& c = h->cfg;
  const size_t es = esize(c.dtype);
  const size_t T = (size_t)c.max_batch * c.max_seq;
  const size_t H = c.hidden, nh = c.num_heads, nkv = c.num_kv_heads, hd = c.head_dim;
  const size_t Sp = ((size_t)c.max_seq + 63) & ~(size_t)63;
  const bool moe = c.mlp_kind == BLK_MLP_MOE;
  const size_t kk = moe ? c.top_k : 0;
  size_t off = 0;
  auto add = [&](void** dst, size_t bytes) {
    *dst = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
  };
  add(&h->a, T * H * es);
  add(&h->q, T * nh * hd * es);
  add(&h->k, T * nkv * hd * es);
  add(&h->vt, (size_t)c.max_batch * nkv * hd * Sp * es);
  if (c.head_gate_dim) add((void**)&h->gate, T * c.head_gate_dim * 4);
  add(&h->premix, T * nh * hd * es);
  if (c.sandwich_norm) add((void**)&h->o, T * H * 4);
  add((void**)&h->mid, T * H * 4);
  add(&h->m, T * H * es);
  add(&h->layer_out, T * H * es);
  if (!moe) {
    add(&h->neur, T * neuron_ld(c.intermediate) * es);
    if (c.sandwich_norm) add((void**)&h->mlp_raw, T * H * 4);
  } else {
    const size_t E = c.num_experts;
    add(&h->logits, T * E * es);
    add((void**)&h->eidx, T * kk * 4);
    add((void**)&h->ew, T * kk * 4);
    add((void**)&h->gcnt, E * 4);
    add((void**)&h->goff, E * 4);
    add((void**)&h->hist, (size_t)dispatch_hist_ints(T, (int)E) * 4);
    add((void**)&h->row_token, T * kk * 4);
    add((void**)&h->pair_row, T * kk * 4);
    add((void**)&h->row_weight, T * kk * 4);
    add(&h->neur, T * kk * c.moe_intermediate * es);
    add(&h->stage, T * kk * H * es);
    if (c.num_shared_experts > 0) {
      add(&h->nsh, T * (size_t)c.moe_intermediate * c.num_shared_experts * es);
      add((void**)&h->mlp_raw, T * H * 4);
    }
  }
  if (c.use_rope) {
    add((void**)&h->rope_cos, (size_t)c.max_seq * (hd / 2) * 4);
    add((void**)&h->rope_sin, (size_t)c.max_seq * (hd / 2) * 4);
  }
  add((void**)&h->split, split_bytes);
  h->split_bytes = split_bytes;
  return off;
}

static blk_status check_config(const blk_config* c) {
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
  const int G = c->head_gate_dim;
  if (G != 0 && G != c->num_heads && G != c->num_heads * c->head_dim)
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
  // every GEMM operand is addressed with 32-bit byte offsets
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

extern "C" {

int32_t blk_abi_version(void) { return BLK_ABI_VERSION; }

const char* blk_status_str(blk_status s) {
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

const char* blk_last_error(void) { return g_err.c_str(); }

size_t blk_workspace_bytes(const blk_handle* h) { return h ? h->ws_bytes : 0; }

blk_status blk_create(const blk_config* cfg, blk_handle** out) {
  if (!cfg || !out) return fail(BLK_E_NULL, "cfg and out must not be NULL");
  *out = nullptr;
  blk_status st = check_config(cfg);
  if (st != BLK_OK) return st;
  const blk_config& c = *cfg;
  blk_handle* h = new blk_handle();
  h->cfg = c;
  const size_t total = carve(h, nullptr, SPLIT_WS_BYTES);
  hipGetDevice(&h->device);
  if (hipMalloc((void**)&h->ws, total) != hipSuccess) {
    hipGetLastError();
    delete h;
    return fail(BLK_E_OOM, "hipMalloc of " + std::to_string(total) + " workspace bytes failed");
  }
  h->ws_bytes = total;
  carve(h, h->ws, SPLIT_WS_BYTES);
  if (c.use_rope) {
    // rotary angles phi[s, i] = s * theta^(-2i/hd), computed in double
    const size_t hd = c.head_dim, half = hd / 2;
    std::vector<float> cs(c.max_seq * half), sn(c.max_seq * half);
    for (size_t s = 0; s < (size_t)c.max_seq; ++s)
      for (size_t i = 0; i < half; ++i) {
        const double inv_freq = pow((double)c.rope_theta, -2.0 * (double)i / (double)hd);
        const double phi = (double)s * inv_freq;
        cs[s * half + i] = (float)cos(phi);
        sn[s * half + i] = (float)sin(phi);
      }
    if (hipMemcpy(h->rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(h->rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice) != hipSuccess) {
      hipFree(h->ws);
      delete h;
      return fail(BLK_E_HIP, "copying the rotary table failed");
    }
  }
  *out = h;
  return BLK_OK;
}

void blk_destroy(blk_handle* h) {
  if (!h) return;
  for (auto e : h->pev) hipEventDestroy(e);
  if (h->ws) hipFree(h->ws);
  delete h;
}

blk_status blk_profile_begin(blk_handle* h, int32_t max_forwards) {
  if (!h) return fail(BLK_E_NULL, "handle is NULL");
  if (max_forwards < 1) return fail(BLK_E_CONFIG, "max_forwards must be >= 1");
  for (auto e : h->pev) hipEventDestroy(e);
  h->pev.assign((size_t)max_forwards * PROF_MARKS, nullptr);
  for (auto& e : h->pev)
    if (hipEventCreate(&e) != hipSuccess) return fail(BLK_E_HIP, "hipEventCreate failed");
  h->pname.assign(PROF_MARKS, nullptr);
  h->pmax = max_forwards;
  h->pfwd = 0;
  h->pmarks = 0;
  return BLK_OK;
}

int32_t blk_profile_end(blk_handle* h, int32_t max_entries, const char** names,
                        double* total_ms, int32_t* calls) {
  if (!h || h->pmax == 0) return -1;
  hipDeviceSynchronize();
  int n = 0;
  const int nfwd = h->pfwd;
  std::vector<double> tot(PROF_MARKS, 0.0);
  int marks = 0;
  for (int m = 0; m < PROF_MARKS && h->pname[m]; ++m) marks = m + 1;
  for (int f = 0; f < nfwd; ++f)
    for (int m = 0; m + 1 < marks; ++m) {
      float ms = 0.f;
      hipEventElapsedTime(&ms, h->pev[f * PROF_MARKS + m], h->pev[f * PROF_MARKS + m + 1]);
      tot[m] += ms;
    }
  for (int m = 0; m + 1 < marks && n < max_entries; ++m, ++n) {
    names[n] = h->pname[m];
    total_ms[n] = tot[m];
    calls[n] = nfwd;
  }
  for (auto e : h->pev) hipEventDestroy(e);
  h->pev.clear();
  h->pmax = 0;
  return n;
}

}  // extern "C"

// ------------------------------------------------------------- forward

namespace {

struct TapCheck {
  const char* name;
  const blk_tap* tap;
  int want;  // required dtype
  bool allowed;
};

blk_status check_taps(const blk_handle* h, const blk_taps* t) {
  if (!t) return BLK_OK;
  const int md = h->cfg.dtype;
  const bool moe = h->cfg.mlp_kind == BLK_MLP_MOE;
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
       moe && h->cfg.num_shared_experts > 0},
  };
  for (const auto& c : list) {
    if (!c.tap->ptr) continue;
    if (!c.allowed)
      return fail(BLK_E_CONFIG, std::string("tap ") + c.name +
                                    " does not exist for this block's mlp_kind");
    if (c.tap->dtype != c.want)
      return fail(BLK_E_DTYPE, std::string("tap ") + c.name + " must be requested as dtype " +
                                   std::to_string(c.want));
    if (!aligned16(c.tap->ptr))
      return fail(BLK_E_ALIGN, std::string("tap ") + c.name + " is not 16-byte aligned");
  }
  return BLK_OK;
}

struct WNeed {
  const char* name;
  const void* p;
  bool needed;
};

blk_status check_weights(const blk_handle* h, const blk_weights* w) {
  const blk_config& c = h->cfg;
  const int k = c.mlp_kind;
  const bool moe = k == BLK_MLP_MOE;
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
      {"w_sh_gate", w->w_sh_gate, moe && c.num_shared_experts > 0},
      {"w_sh_up", w->w_sh_up, moe && c.num_shared_experts > 0},
      {"w_sh_down", w->w_sh_down, moe && c.num_shared_experts > 0},
  };
  for (const auto& n : list) {
    if (!n.needed) continue;
    if (!n.p) return fail(BLK_E_NULL, std::string("weight ") + n.name + " is NULL");
    if (!aligned16(n.p))
      return fail(BLK_E_ALIGN, std::string("weight ") + n.name + " is not 16-byte aligned");
  }
  return BLK_OK;
}

#define HIP_TRY(expr, what)                                                        \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess)                                                         \
      return fail(BLK_E_HIP, std::string(what) + ": " + hipGetErrorString(e_));   \
  } while (0)

GemmParams gp0(const blk_handle* h) {
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.split_ws = h->split;
  p.split_ws_bytes = h->split_bytes;
  return p;
}

uint32_t bytes32(size_t n) { return (uint32_t)n; }

}  // namespace

// Every check of a forward call, before anything is enqueued.
static blk_status check_forward(const blk_handle* h, const blk_io* io, const blk_weights* w,
                                const blk_taps* taps) {
  if (!h || !io || !w) return fail(BLK_E_NULL, "handle, io and weights must not be NULL");
  const blk_config& c = h->cfg;
  if (!io->x || !io->y) return fail(BLK_E_NULL, "io.x and io.y must not be NULL");
  if (io->x == io->y) return fail(BLK_E_CONFIG, "io.y must not alias io.x");
  if (!aligned16(io->x) || !aligned16(io->y))
    return fail(BLK_E_ALIGN, "io.x and io.y must be 16-byte aligned");
  if (io->batch < 1 || io->seq < 1 || io->batch > c.max_batch || io->seq > c.max_seq)
    return fail(BLK_E_SHAPE, "batch/seq must be in [1, max_batch] x [1, max_seq]");
  blk_status st = check_weights(h, w);
  if (st != BLK_OK) return st;
  return check_taps(h, taps);
}

// The kernel sequence of one forward (the call has been checked).
static blk_status enqueue_forward(blk_handle* h, const blk_io* io, const blk_weights* w,
                                  const blk_taps* taps, void* stream_) {
  const blk_config& c = h->cfg;
  hipStream_t s = (hipStream_t)stream_;
  const DType dt = c.dtype == BLK_BF16 ? DType::BF16 : DType::F32;
  const int es = (int)esize(c.dtype);
  const int B = io->batch, S = io->seq, T = B * S;
  const int H = c.hidden, nh = c.num_heads, nkv = c.num_kv_heads, hd = c.head_dim;
  const int G = c.head_gate_dim;
  const float eps = c.rms_eps;
  const bool moe = c.mlp_kind == BLK_MLP_MOE;
  const bool sandwich = c.sandwich_norm != 0;
  blk_taps none;
  memset(&none, 0, sizeof(none));
  const blk_taps& tp = taps ? *taps : none;

  if (tp.layer_input.ptr)
    HIP_TRY(hipMemcpyAsync(tp.layer_input.ptr, io->x, (size_t)T * H * es,
                           hipMemcpyDeviceToDevice, s), "layer_input tap");

  h->pmarks = 0;
  // (1) attention-input RMSNorm
  prof_mark(h, "rmsnorm_in", s);
  HIP_TRY(rmsnorm(dt, 0, io->x, w->w_in_norm, h->a, T, H, eps, s), "input rmsnorm");
  if (tp.attention_norm_output.ptr)
    HIP_TRY(hipMemcpyAsync(tp.attention_norm_output.ptr, h->a, (size_t)T * H * es,
                           hipMemcpyDeviceToDevice, s), "attention_norm_output tap");

  // (2) fused Q/K/V(/gate) projection with q/k norm + rotary epilogue
  {
    GemmParams p = gp0(h);
    p.M = T;
    p.K = H;
    p.A = h->a;
    p.lda = H;
    p.a_bytes = bytes32((size_t)T * H * es);
    p.B[0] = w->wq;
    p.B[1] = w->wk;
    p.B[2] = w->wv;
    p.seg_end[0] = nh * hd;
    p.seg_end[1] = nh * hd + nkv * hd;
    p.seg_end[2] = nh * hd + 2 * nkv * hd;
    p.b_bytes[0] = bytes32((size_t)nh * hd * H * es);
    p.b_bytes[1] = p.b_bytes[2] = bytes32((size_t)nkv * hd * H * es);
    p.nseg = 3;
    if (G) {
      p.B[3] = w->w_head_gate;
      p.seg_end[3] = p.seg_end[2] + G;
      p.b_bytes[3] = bytes32((size_t)G * H * es);
      p.nseg = 4;
    }
    p.N = p.seg_end[p.nseg - 1];
    p.ldb = H;
    p.q = h->q;
    p.k = h->k;
    p.vt = h->vt;
    p.gate = h->gate;
    p.S = S;
    p.nh = nh;
    p.nkv = nkv;
    p.hd = hd;
    p.G = G;
    p.qk_norm = c.qk_norm;
    p.use_rope = c.use_rope;
    p.q_norm_w = w->w_q_norm;
    p.k_norm_w = w->w_k_norm;
    p.rope_cos = h->rope_cos;
    p.rope_sin = h->rope_sin;
    p.eps = eps;
    prof_mark(h, "gemm_qkv", s);
    HIP_TRY(gemm(dt, EPI_QKV, p, T, s), "qkv gemm");
  }

  // (3) attention (+ head gate) -> premix [T, nh*hd]
  AttnParams ap;
  memset(&ap, 0, sizeof(ap));
  ap.q = h->q;
  ap.k = h->k;
  ap.vt = h->vt;
  ap.gate = G ? h->gate : nullptr;
  ap.mask = io->attention_mask;
  ap.out = h->premix;
  ap.B = B;
  ap.S = S;
  ap.nh = nh;
  ap.nkv = nkv;
  ap.hd = hd;
  ap.window = c.sliding_window;
  ap.G = G;
  ap.scale = (float)(1.0 / sqrt((double)hd));
  prof_mark(h, "attention", s);
  HIP_TRY(attention(dt, ap, s), "attention");
  if (tp.attention_scores.ptr)
    HIP_TRY(attention_scores(dt, ap, (float*)tp.attention_scores.ptr, s), "scores tap");
  if (tp.attention_probabilities.ptr)
    HIP_TRY(attention_probs(dt, ap, (float*)tp.attention_probabilities.ptr, s), "probs tap");
  if (tp.attention_queries.ptr)
    HIP_TRY(hipMemcpyAsync(tp.attention_queries.ptr, h->q, (size_t)T * nh * hd * es,
                           hipMemcpyDeviceToDevice, s), "queries tap");
  if (tp.attention_keys.ptr)
    HIP_TRY(hipMemcpyAsync(tp.attention_keys.ptr, h->k, (size_t)T * nkv * hd * es,
                           hipMemcpyDeviceToDevice, s), "keys tap");
  if (tp.attention_values.ptr)
    HIP_TRY(attention_values(dt, ap, tp.attention_values.ptr, s), "values tap");
  if (tp.attention_premix.ptr)
    HIP_TRY(hipMemcpyAsync(tp.attention_premix.ptr, h->premix, (size_t)T * nh * hd * es,
                           hipMemcpyDeviceToDevice, s), "premix tap");
  if (tp.attention_head_outputs.ptr) {
    if (G) {  // the same attention without the head gate
      AttnParams hp = ap;
      hp.gate = nullptr;
      hp.G = 0;
      hp.out = tp.attention_head_outputs.ptr;
      HIP_TRY(attention(dt, hp, s), "head outputs tap");
    } else {
      HIP_TRY(hipMemcpyAsync(tp.attention_head_outputs.ptr, h->premix,
                             (size_t)T * nh * hd * es, hipMemcpyDeviceToDevice, s),
              "head outputs tap");
    }
  }

  // (4) o_proj (+ residual) and the MLP-input norm
  {
    GemmParams p = gp0(h);
    p.M = T;
    p.N = H;
    p.K = nh * hd;
    p.A = h->premix;
    p.lda = nh * hd;
    p.a_bytes = bytes32((size_t)T * nh * hd * es);
    p.B[0] = w->wo;
    p.seg_end[0] = H;
    p.nseg = 1;
    p.ldb = nh * hd;
    p.b_bytes[0] = bytes32((size_t)H * nh * hd * es);
    p.ldo = H;
    if (!sandwich) {
      p.resid = io->x;
      p.resid_f32 = 0;
      p.out_f32p = h->mid;
      p.out_raw = (float*)tp.attention_output.ptr;
      prof_mark(h, "gemm_o", s);
      HIP_TRY(gemm(dt, EPI_RESID, p, T, s), "o_proj gemm");
      prof_mark(h, "rmsnorm_mlp", s);
      HIP_TRY(rmsnorm(dt, 1, h->mid, w->w_mlp_norm, h->m, T, H, eps, s), "mlp rmsnorm");
    } else {
      p.out = h->o;
      p.out_f32 = 1;
      prof_mark(h, "gemm_o", s);
      HIP_TRY(gemm(dt, EPI_STORE, p, T, s), "o_proj gemm");
      prof_mark(h, "norm_add_norm", s);
      HIP_TRY(norm_add_norm(dt, h->o, io->x, w->w_post_attn_norm, w->w_mlp_norm,
                            (float*)tp.attention_output.ptr, h->mid, h->m, T, H, eps, s),
              "post-attention norm");
    }
  }
  if (tp.layer_mid.ptr)
    HIP_TRY(hipMemcpyAsync(tp.layer_mid.ptr, h->mid, (size_t)T * H * 4,
                           hipMemcpyDeviceToDevice, s), "layer_mid tap");
  if (tp.mlp_input.ptr)
    HIP_TRY(hipMemcpyAsync(tp.mlp_input.ptr, h->m, (size_t)T * H * es,
                           hipMemcpyDeviceToDevice, s), "mlp_input tap");
  if (tp.mlp_norm_output.ptr)
    HIP_TRY(hipMemcpyAsync(tp.mlp_norm_output.ptr, h->m, (size_t)T * H * es,
                           hipMemcpyDeviceToDevice, s), "mlp_norm_output tap");

  // (5) MLP
  if (!moe) {
    const int I = c.intermediate;
    GemmParams p = gp0(h);
    p.M = T;
    p.N = I;
    p.K = H;
    p.A = h->m;
    p.lda = H;
    p.a_bytes = bytes32((size_t)T * H * es);
    p.ldb = H;
    p.out = h->neur;
    p.ldo = (int64_t)neuron_ld(I);
    EpiKind epi;
    if (c.mlp_kind == BLK_MLP_SWIGLU) {
      p.B[0] = w->w_gate;
      p.B[1] = w->w_up;
      p.b_bytes[0] = p.b_bytes[1] = bytes32((size_t)I * H * es);
      p.nseg = 2;
      p.seg_end[0] = p.seg_end[1] = I;
      epi = EPI_SWIGLU;
    } else {
      p.B[0] = w->w_up;
      p.b_bytes[0] = bytes32((size_t)I * H * es);
      p.nseg = 1;
      p.seg_end[0] = I;
      epi = c.mlp_kind == BLK_MLP_RELU2 ? EPI_RELU2 : EPI_XIELU;
      if (epi == EPI_XIELU) {
        auto softplus = [](double z) { return log1p(exp(-fabs(z))) + fmax(z, 0.0); };
        p.xbeta = c.xielu_beta;
        p.xeps = c.xielu_eps;
        p.xa_p = (float)softplus(w->xielu_alpha_p_raw);
        p.xa_n = (float)(c.xielu_beta + softplus(w->xielu_alpha_n_raw));
      }
    }
    prof_mark(h, "gemm_up", s);
    HIP_TRY(gemm(dt, epi, p, T, s), "mlp up gemm");
    if (tp.mlp_neurons.ptr)
      HIP_TRY(hipMemcpy2DAsync(tp.mlp_neurons.ptr, (size_t)I * es, h->neur,
                               neuron_ld(I) * es, (size_t)I * es, T, hipMemcpyDeviceToDevice, s),
              "neurons tap");
    if (tp.mlp_activation.ptr) {
      if (c.mlp_kind == BLK_MLP_SWIGLU) {
        // act_fn's output is silu(gate), which the fused gate/up GEMM never
        // stores: the gate projection again, with a silu epilogue
        GemmParams a = p;
        a.B[0] = w->w_gate;
        a.nseg = 1;
        a.seg_end[0] = I;
        a.out = tp.mlp_activation.ptr;
        a.ldo = I;
        HIP_TRY(gemm(dt, EPI_SILU, a, T, s), "activation tap gemm");
      } else {
        HIP_TRY(hipMemcpy2DAsync(tp.mlp_activation.ptr, (size_t)I * es, h->neur,
                                 neuron_ld(I) * es, (size_t)I * es, T,
                                 hipMemcpyDeviceToDevice, s),
                "activation tap");
      }
    }

    GemmParams d = gp0(h);
    d.M = T;
    d.N = H;
    d.K = I;
    d.A = h->neur;
    d.lda = (int64_t)neuron_ld(I);
    d.a_bytes = bytes32((size_t)T * neuron_ld(I) * es);
    d.B[0] = w->w_down;
    d.seg_end[0] = H;
    d.nseg = 1;
    d.ldb = I;
    d.b_bytes[0] = bytes32((size_t)H * I * es);
    d.ldo = H;
    if (!sandwich) {
      d.resid = h->mid;
      d.resid_f32 = 1;
      d.out_f32p = (float*)tp.layer_output.ptr;
      d.out_model = io->y;
      d.out_raw = (float*)tp.mlp_output.ptr;
      prof_mark(h, "gemm_down", s);
      HIP_TRY(gemm(dt, EPI_RESID, d, T, s), "mlp down gemm");
    } else {
      d.out = h->mlp_raw;
      d.out_f32 = 1;
      prof_mark(h, "gemm_down", s);
      HIP_TRY(gemm(dt, EPI_STORE, d, T, s), "mlp down gemm");
      prof_mark(h, "post_mlp_norm", s);
      HIP_TRY(moe_combine(dt, nullptr, nullptr, h->mlp_raw, h->mid, w->w_post_mlp_norm, 0,
                          (float*)tp.mlp_output.ptr, (float*)tp.layer_output.ptr, io->y, T,
                          H, eps, 1, s),
              "post-mlp norm");
    }
    prof_mark(h, "end", s);
    if (h->pmax) ++h->pfwd;
    return BLK_OK;
  }

  // afmoe mixture
  const int E = c.num_experts, kk = c.top_k, Ie = c.moe_intermediate;
  const int Ish = Ie * c.num_shared_experts;
  // router: logits in the model dtype, then sigmoid + bias, top-k and the
  // weights; when one GEMM tile holds every expert of its tokens that all
  // runs in the GEMM's epilogue, which also counts the dispatch histogram
  const int rtpc = router_tile_tokens(dt, E);
  {
    GemmParams p = gp0(h);  // router.gate
    p.M = T;
    p.N = E;
    p.K = H;
    p.A = h->m;
    p.lda = H;
    p.a_bytes = bytes32((size_t)T * H * es);
    p.B[0] = w->w_router;
    p.seg_end[0] = E;
    p.nseg = 1;
    p.ldb = H;
    p.b_bytes[0] = bytes32((size_t)E * H * es);
    p.out = h->logits;
    p.out_f32 = 0;
    p.ldo = E;
    if (rtpc) {
      p.bias = w->expert_bias;
      p.top_k = kk;
      p.route_scale = c.route_scale;
      p.eidx = h->eidx;
      p.ew = h->ew;
      p.hist = h->hist;
      p.hist_nchunks = (T + rtpc - 1) / rtpc;
      prof_mark(h, "gemm_router_topk", s);
      HIP_TRY(gemm(dt, EPI_ROUTER, p, T, s), "router gemm + top-k");
    } else {
      prof_mark(h, "gemm_router", s);
      HIP_TRY(gemm(dt, EPI_STORE, p, T, s), "router gemm");
      prof_mark(h, "topk", s);
      HIP_TRY(moe_topk(dt, h->logits, w->expert_bias, T, E, kk, c.route_scale, h->eidx, h->ew,
                       s),
              "router top-k");
    }
  }
  if (tp.router_logits.ptr)
    HIP_TRY(hipMemcpyAsync(tp.router_logits.ptr, h->logits, (size_t)T * E * es,
                           hipMemcpyDeviceToDevice, s), "router_logits tap");
  if (tp.expert_indices.ptr)
    HIP_TRY(hipMemcpyAsync(tp.expert_indices.ptr, h->eidx, (size_t)T * kk * 4,
                           hipMemcpyDeviceToDevice, s), "expert_indices tap");
  if (tp.expert_weights.ptr)
    HIP_TRY(hipMemcpyAsync(tp.expert_weights.ptr, h->ew, (size_t)T * kk * 4,
                           hipMemcpyDeviceToDevice, s), "expert_weights tap");
  prof_mark(h, "dispatch", s);
  HIP_TRY(moe_dispatch(h->eidx, h->ew, T, kk, E, h->gcnt, h->goff, h->row_token,
                       h->pair_row, h->row_weight, h->hist, rtpc ? rtpc : DISPATCH_TOKENS,
                       rtpc != 0, s),
          "dispatch");
  {
    GemmParams p = gp0(h);  // routed experts: gate/up + SwiGLU
    p.M = T * kk;
    p.N = Ie;
    p.K = H;
    p.A = h->m;
    p.lda = H;
    p.a_bytes = bytes32((size_t)T * H * es);
    p.a_gather = h->row_token;
    p.B[0] = w->w_e_gate;
    p.B[1] = w->w_e_up;
    p.nseg = 2;
    p.seg_end[0] = p.seg_end[1] = Ie;
    p.ldb = H;
    p.b_bytes[0] = p.b_bytes[1] = bytes32((size_t)Ie * H * es);
    p.gcnt = h->gcnt;
    p.goff = h->goff;
    p.ngroups = E;
    p.b_group_stride = (int64_t)Ie * H;
    p.out = h->neur;
    p.ldo = Ie;
    prof_mark(h, "gemm_expert_up", s);
    HIP_TRY(gemm(dt, EPI_SWIGLU, p, T * kk, s), "expert gate/up gemm");
  }
  {
    GemmParams p = gp0(h);  // routed experts: down, scaled by the slot weight; the
                            // rows stay in expert order (the combine gathers them)
    p.M = T * kk;
    p.N = H;
    p.K = Ie;
    p.A = h->neur;
    p.lda = Ie;
    p.a_bytes = bytes32((size_t)T * kk * Ie * es);
    p.B[0] = w->w_e_down;
    p.seg_end[0] = H;
    p.nseg = 1;
    p.ldb = Ie;
    p.b_bytes[0] = bytes32((size_t)H * Ie * es);
    p.gcnt = h->gcnt;
    p.goff = h->goff;
    p.ngroups = E;
    p.b_group_stride = (int64_t)H * Ie;
    p.out = h->stage;
    p.ldo = H;
    p.row_weight = h->row_weight;
    prof_mark(h, "gemm_expert_down", s);
    HIP_TRY(gemm(dt, EPI_MOE_DOWN, p, T * kk, s), "expert down gemm");
  }
  if (Ish > 0) {
    GemmParams p = gp0(h);  // shared expert
    p.M = T;
    p.N = Ish;
    p.K = H;
    p.A = h->m;
    p.lda = H;
    p.a_bytes = bytes32((size_t)T * H * es);
    p.B[0] = w->w_sh_gate;
    p.B[1] = w->w_sh_up;
    p.nseg = 2;
    p.seg_end[0] = p.seg_end[1] = Ish;
    p.ldb = H;
    p.b_bytes[0] = p.b_bytes[1] = bytes32((size_t)Ish * H * es);
    p.out = h->nsh;
    p.ldo = Ish;
    prof_mark(h, "gemm_shared_up", s);
    HIP_TRY(gemm(dt, EPI_SWIGLU, p, T, s), "shared gate/up gemm");
    GemmParams d = gp0(h);
    d.M = T;
    d.N = H;
    d.K = Ish;
    d.A = h->nsh;
    d.lda = Ish;
    d.a_bytes = bytes32((size_t)T * Ish * es);
    d.B[0] = w->w_sh_down;
    d.seg_end[0] = H;
    d.nseg = 1;
    d.ldb = Ish;
    d.b_bytes[0] = bytes32((size_t)H * Ish * es);
    d.out = h->mlp_raw;
    d.out_f32 = 1;
    d.ldo = H;
    prof_mark(h, "gemm_shared_down", s);
    HIP_TRY(gemm(dt, EPI_STORE, d, T, s), "shared down gemm");
  }
  if (tp.expert_outputs.ptr)
    HIP_TRY(moe_gather_slots(dt, h->stage, h->pair_row, tp.expert_outputs.ptr, T * kk, H, s),
            "expert outputs tap");
  if (tp.routed_output.ptr)
    HIP_TRY(moe_sum_slots(dt, h->stage, h->pair_row, kk, (float*)tp.routed_output.ptr, T, H,
                          s),
            "routed output tap");
  if (tp.shared_expert_output.ptr)
    HIP_TRY(hipMemcpyAsync(tp.shared_expert_output.ptr, h->mlp_raw, (size_t)T * H * 4,
                           hipMemcpyDeviceToDevice, s), "shared expert output tap");
  prof_mark(h, "combine", s);
  HIP_TRY(moe_combine(dt, h->stage, h->pair_row, Ish > 0 ? h->mlp_raw : nullptr, h->mid,
                      w->w_post_mlp_norm, kk, (float*)tp.mlp_output.ptr,
                      (float*)tp.layer_output.ptr, io->y, T, H, eps, sandwich ? 1 : 0, s),
          "combine");
  prof_mark(h, "end", s);
  if (h->pmax) ++h->pfwd;
  return BLK_OK;
}

extern "C" blk_status blk_forward(blk_handle* h, const blk_io* io, const blk_weights* w,
                                  const blk_taps* taps, void* stream) {
  const blk_status st = check_forward(h, io, w, taps);
  if (st != BLK_OK) return st;
  return enqueue_forward(h, io, w, taps, stream);
}

extern "C" blk_status blk_forward_layers(blk_handle* h, const blk_io* io,
                                         const blk_weights* const* layers, int32_t n_layers,
                                         void* stream) {
  if (!h || !io || !layers) return fail(BLK_E_NULL, "handle, io and layers must not be NULL");
  if (n_layers < 1) return fail(BLK_E_CONFIG, "n_layers must be >= 1");
  if (!io->x || !io->y) return fail(BLK_E_NULL, "io.x and io.y must not be NULL");
  if (io->x == io->y) return fail(BLK_E_CONFIG, "io.y must not alias io.x");
  if (!aligned16(io->x) || !aligned16(io->y))
    return fail(BLK_E_ALIGN, "io.x and io.y must be 16-byte aligned");
  const blk_config& c = h->cfg;
  if (io->batch < 1 || io->seq < 1 || io->batch > c.max_batch || io->seq > c.max_seq)
    return fail(BLK_E_SHAPE, "batch/seq must be in [1, max_batch] x [1, max_seq]");
  for (int32_t l = 0; l < n_layers; ++l) {
    if (!layers[l]) return fail(BLK_E_NULL, "layer " + std::to_string(l) + " weights are NULL");
    const blk_status st = check_weights(h, layers[l]);
    if (st != BLK_OK) return st;
  }
  // layer l writes y when n_layers - 1 - l is even, else the workspace
  // buffer, so the last layer writes y and no layer reads what it writes
  const void* src = io->x;
  for (int32_t l = 0; l < n_layers; ++l) {
    blk_io lio = *io;
    lio.x = src;
    lio.y = ((n_layers - 1 - l) % 2 == 0) ? io->y : h->layer_out;
    const blk_status st = blk_forward(h, &lio, layers[l], nullptr, stream);
    if (st != BLK_OK) return st;
    src = lio.y;
  }
  return BLK_OK;
}

// ------------------------------------------------- forward without allocation

// The workspace of blk_forward_noalloc: one copy of this array on every GPU
// the library runs on, held until the process ends.  In host code its name
// is only a host-side stand-in; the device address comes from
// hipGetSymbolAddress, once per device (scratch_base), and only that
// address is ever handed to kernels.
static __device__ __align__(256) char scratch[BLK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
void* g_scratch[MAX_DEVICES];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`, looked up on
// the first call on that device with that device current.
blk_status scratch_base(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
    return fail(BLK_E_HIP, "no current HIP device (or more than 64 devices)");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(BLK_E_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                 hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = (char*)g_scratch[dev];
  return BLK_OK;
}

// Rotary table of S positions, the same angles as blk_create's host table:
// phi[s, i] = s * theta^(-2i/hd) in double, cos and sin rounded to float.
__global__ void __launch_bounds__(256) rope_table_kernel(float* cs, float* sn, int S, int hd,
                                                         double theta) {
  const int half = hd / 2;
  const int64_t n = (int64_t)S * half;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * 256) {
    const int pos = (int)(e / half), i = (int)(e % half);
    const double inv_freq = pow(theta, -2.0 * (double)i / (double)hd);
    const double phi = (double)pos * inv_freq;
    cs[e] = (float)cos(phi);
    sn[e] = (float)sin(phi);
  }
}

}  // namespace

extern "C" blk_status blk_forward_noalloc(const blk_config* cfg, const blk_io* io,
                                          const blk_weights* w, const blk_taps* taps,
                                          void* stream) {
  if (!cfg || !io || !w) return fail(BLK_E_NULL, "cfg, io and weights must not be NULL");
  if (io->batch < 1 || io->seq < 1)
    return fail(BLK_E_SHAPE, "batch and seq must be >= 1");
  // a handle on the stack, sized for this call's batch and sequence, whose
  // workspace is the device's scratch array
  blk_handle h;
  h.cfg = *cfg;
  h.cfg.max_batch = io->batch;
  h.cfg.max_seq = io->seq;
  blk_status st = check_config(&h.cfg);
  if (st != BLK_OK) return st;
  const size_t need = carve(&h, nullptr, 0);
  if (need > BLK_NOALLOC_SCRATCH_BYTES)
    return fail(BLK_E_SHAPE, "this batch and sequence need " + std::to_string(need) +
                                 " bytes of workspace; blk_forward_noalloc holds " +
                                 std::to_string((size_t)BLK_NOALLOC_SCRATCH_BYTES) +
                                 " (use blk_create / blk_forward)");
  st = check_forward(&h, io, w, taps);
  if (st != BLK_OK) return st;
  char* base = nullptr;
  st = scratch_base(&base);
  if (st != BLK_OK) return st;
  // what the workspace leaves of the array serves the GEMMs' K split, up
  // to the handle path's size
  const size_t split = std::min(SPLIT_WS_BYTES, (BLK_NOALLOC_SCRATCH_BYTES - need) & ~(size_t)255);
  carve(&h, base, split);
  h.ws = base;
  h.ws_bytes = need + split;
  hipStream_t s = (hipStream_t)stream;
  if (h.cfg.use_rope) {
    const int64_t n = (int64_t)io->seq * (h.cfg.head_dim / 2);
    const int grid = (int)std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(rope_table_kernel, dim3(grid), dim3(256), 0, s, h.rope_cos, h.rope_sin,
                       io->seq, h.cfg.head_dim, (double)h.cfg.rope_theta);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return fail(BLK_E_HIP, std::string("rotary table: ") + hipGetErrorString(e));
  }
  st = enqueue_forward(&h, io, w, taps, stream);
  h.ws = nullptr;  // the scratch array is not the handle's to free
  return st;
}
