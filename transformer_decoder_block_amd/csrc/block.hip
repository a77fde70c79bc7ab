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
#include "validate.h"

using namespace blk;

using blkv::aligned16;
using blkv::esize;
using blkv::fail;
using blkv::neuron_ld;

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

// Point the handle's workspace views into `base` (laid out for h->cfg:
// max_batch * max_seq tokens, every part on a 256-byte boundary, the GEMMs'
// K-split scratch last with split_bytes) and return the workspace size; with
// base == nullptr only the size is computed.  Allocates nothing.
static size_t carve(blk_handle* h, char* base, size_t split_bytes) {
  const blk_config& c = h->cfg;
  const int64_t T = (int64_t)c.max_batch * c.max_seq;
  const size_t hist = c.mlp_kind == BLK_MLP_MOE ? (size_t)dispatch_hist_ints(T, c.num_experts) : 0;
  blkv::WsLayout L;
  blkv::ws_layout(c, hist, split_bytes, &L);
  auto at = [&](blkv::WsPart part) -> char* {
    return (base && L.off[part] != blkv::WS_ABSENT) ? base + L.off[part] : nullptr;
  };
  h->a = at(blkv::WS_A);
  h->q = at(blkv::WS_Q);
  h->k = at(blkv::WS_K);
  h->vt = at(blkv::WS_VT);
  h->gate = (float*)at(blkv::WS_GATE);
  h->premix = at(blkv::WS_PREMIX);
  h->o = (float*)at(blkv::WS_O);
  h->mid = (float*)at(blkv::WS_MID);
  h->m = at(blkv::WS_M);
  h->layer_out = at(blkv::WS_LAYER_OUT);
  h->neur = at(blkv::WS_NEUR);
  h->mlp_raw = (float*)at(blkv::WS_MLP_RAW);
  h->logits = at(blkv::WS_LOGITS);
  h->eidx = (int*)at(blkv::WS_EIDX);
  h->ew = (float*)at(blkv::WS_EW);
  h->gcnt = (int*)at(blkv::WS_GCNT);
  h->goff = (int*)at(blkv::WS_GOFF);
  h->hist = (int*)at(blkv::WS_HIST);
  h->row_token = (int*)at(blkv::WS_ROW_TOKEN);
  h->pair_row = (int*)at(blkv::WS_PAIR_ROW);
  h->row_weight = (float*)at(blkv::WS_ROW_WEIGHT);
  h->stage = at(blkv::WS_STAGE);
  h->nsh = at(blkv::WS_NSH);
  h->rope_cos = (float*)at(blkv::WS_ROPE_COS);
  h->rope_sin = (float*)at(blkv::WS_ROPE_SIN);
  h->split = (float*)at(blkv::WS_SPLIT);
  h->split_bytes = split_bytes;
  return L.total;
}

extern "C" {

int32_t blk_abi_version(void) { return BLK_ABI_VERSION; }

const char* blk_status_str(blk_status s) { return blkv::status_str(s); }

const char* blk_last_error(void) { return blkv::last_error(); }

size_t blk_workspace_bytes(const blk_handle* h) { return h ? h->ws_bytes : 0; }

blk_status blk_create(const blk_config* cfg, blk_handle** out) {
  if (!cfg || !out) return fail(BLK_E_NULL, "cfg and out must not be NULL");
  *out = nullptr;
  blk_status st = blkv::check_config(cfg);
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
    const size_t half = c.head_dim / 2;
    std::vector<float> cs(c.max_seq * half), sn(c.max_seq * half);
    blkv::rope_table(c, c.max_seq, cs.data(), sn.data());
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
  if (!h) return fail(BLK_E_NULL, "handle, io and weights must not be NULL");
  return blkv::check_forward(h->cfg, io, w, taps);
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
  blk_status st = blkv::check_io(h->cfg, io);
  if (st != BLK_OK) return st;
  for (int32_t l = 0; l < n_layers; ++l) {
    if (!layers[l]) return fail(BLK_E_NULL, "layer " + std::to_string(l) + " weights are NULL");
    st = blkv::check_weights(h->cfg, layers[l]);
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
  blk_status st = blkv::check_config(&h.cfg);
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
