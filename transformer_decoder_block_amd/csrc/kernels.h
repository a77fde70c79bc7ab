// Internal interface between the libblock runtime (block.cpp) and the
// kernel translation units.  Every launcher enqueues on `stream` and
// returns the hipError_t of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace blk {

enum class DType : int { F32 = 0, BF16 = 1 };

// ---------------------------------------------------------------- GEMM
// C[M, N] = A[M, K] . B[N, K]^T with an epilogue.  A and B in the model
// dtype, float32 accumulation.
enum EpiKind : int {
  EPI_STORE = 0,     // out = acc (float32 or model dtype, see out_f32)
  EPI_RESID = 1,     // out_f32 = resid + acc; out_model = model(resid + acc);
                     // out_raw = acc
  EPI_SWIGLU = 2,    // paired gate/up rows; out = model(silu(g) * u)
  EPI_RELU2 = 3,     // out = model(relu(acc)^2)
  EPI_XIELU = 4,     // out = model(xielu(acc))
  EPI_QKV = 5,       // q/k/v head-major scatter, q/k norm, rotary, gate
  EPI_MOE_DOWN = 6,  // out[r] = model(row_weight[r] * acc), rows in expert order
  EPI_SILU = 7,      // out = model(silu(acc)): the gated MLP's activation tap
  EPI_ROUTER = 8     // out = model(acc), the router logits [M, N = experts];
                     // then, per token, sigmoid + bias, top-k, weights, and
                     // the tile's expert histogram for the dispatch
};

struct GemmParams {
  int M, N, K;           // N: output columns (SWIGLU: neurons; B has 2N rows)
  const void* A;         // [*, lda]
  int64_t lda;
  const int* a_gather;   // optional: logical row r reads A row a_gather[r]
  uint32_t a_bytes;      // byte size of the A allocation (< 4 GiB)
  // B: up to four row segments stacked along N (QKV: q, k, v, gate).
  // Segment s holds rows [seg_end[s-1], seg_end[s]); SWIGLU: seg 0 = gate,
  // seg 1 = up, both [N, K].
  const void* B[4];
  int seg_end[4];
  int nseg;
  int64_t ldb;
  uint32_t b_bytes[4];   // byte size of each segment (of one group)
  // grouped (MoE): group g owns logical rows [goff[g], goff[g] + gcnt[g])
  // and reads B[s] + g * b_group_stride.
  const int* gcnt;
  const int* goff;
  int ngroups;
  int64_t b_group_stride;
  // epilogue outputs
  void* out;             // EPI_STORE/SWIGLU/RELU2/XIELU/MOE_DOWN output
  int64_t ldo;
  int out_f32;           // EPI_STORE: 1 = float32 output, 0 = model dtype
  float* out_f32p;       // EPI_RESID: float32 result (may be null)
  void* out_model;       // EPI_RESID: model-dtype result (may be null)
  float* out_raw;        // EPI_RESID: the product alone (may be null)
  const void* resid;     // EPI_RESID: residual [M, ldo]
  int resid_f32;         //   1 = float32 residual, 0 = model dtype
  // EPI_XIELU
  float xa_p, xa_n, xbeta, xeps;
  // EPI_MOE_DOWN
  const float* row_weight;  // the slot weight of each grouped row
  // EPI_ROUTER: expert bias [N] (float32), top_k, route_scale; outputs the
  // chosen experts eidx [M, top_k], their weights ew [M, top_k], and
  // hist[e * hist_nchunks + tile] = pairs of the tile's tokens routed to e
  const float* bias;
  int top_k;
  float route_scale;
  int* eidx;
  float* ew;
  int* hist;
  int hist_nchunks;
  // EPI_QKV
  void* q; void* k; void* vt;   // [B,nh,S,hd], [B,nkv,S,hd], [B,nkv,hd,Sp]
                                // with Sp = S rounded up to 64
  float* gate;                  // [M, G] sigmoid of the gate columns
  int S, nh, nkv, hd, G;
  int qk_norm, use_rope;
  const void* q_norm_w; const void* k_norm_w;
  const float* rope_cos; const float* rope_sin;   // [S_max, hd/2]
  float eps;
  // K split (chosen by gemm(); the caller only provides the scratch): the
  // last split_tiles tiles of the grid are each computed as split_parts K
  // ranges whose float32 partial tiles go to split_ws; a fixup kernel adds
  // the parts in a fixed order and applies the epilogue.  Used for the
  // tail of a large grid (two parts) and for grids that fill few CUs.
  float* split_ws;
  size_t split_ws_bytes;
  int split_tiles;
  int split_parts;
  // EPI_QKV only (set by gemm() for the last round of a large grid): the
  // grid covers output columns [n_base, N); column indices stay global, so
  // the segments and heads are found as for the whole product
  int n_base;
};

hipError_t gemm(DType dt, EpiKind epi, const GemmParams& p, int max_rows,
                hipStream_t stream);

// Tokens per tile of the router GEMM with the fused top-k (EPI_ROUTER) for
// E experts, or 0 when one tile cannot hold every expert of a token (then
// the logits are stored and moe_topk / moe_dispatch run separately).  The
// dispatch histogram is kept per chunk of this many tokens.
int router_tile_tokens(DType dt, int E);

// --------------------------------------------------------------- norms
// out[t] = model(g * x[t] / sqrt(mean(x[t]^2) + eps)); x float32 or model.
hipError_t rmsnorm(DType dt, int x_f32, const void* x, const void* g,
                   void* out, int rows, int H, float eps, hipStream_t s);

// afmoe attention tail: attn = norm_post(o) (o float32), mid = x + attn,
// m = model(norm_pre(mid)).  attn_out may be null.
hipError_t norm_add_norm(DType dt, const float* o, const void* x,
                         const void* g_post, const void* g_pre,
                         float* attn_out, float* mid, void* m, int rows,
                         int H, float eps, hipStream_t s);

// MoE tail.  stage holds the weighted expert outputs in expert order; the
// output of slot s of token t is stage row pair_row[t*k + s].
// raw = sum_k stage[pair_row[t, k]] + shared[t]; mo = norm_post(raw);
// out = mid + mo -> out_f32 (may be null), y (model dtype).
// routed[t] = sum over slots 0..k-1 (in that order) of token t's slot rows
// (the routed_output tap)
hipError_t moe_sum_slots(DType dt, const void* stage, const int* pair_row, int top_k,
                         float* routed, int rows, int H, hipStream_t s);

// out[p] = stage[pair_row[p]] for the T*k (token, slot) pairs (the
// expert_outputs tap, token-major)
hipError_t moe_gather_slots(DType dt, const void* stage, const int* pair_row, void* out,
                            int npairs, int H, hipStream_t s);

hipError_t moe_combine(DType dt, const void* stage, const int* pair_row, const float* shared,
                       const float* mid, const void* g_post, int top_k,
                       float* mlp_out, float* out_f32, void* y, int rows,
                       int H, float eps, int sandwich, hipStream_t s);

// ----------------------------------------------------------- attention
struct AttnParams {
  const void* q; const void* k; const void* vt;   // see EPI_QKV layouts
  const float* gate;      // [B*S, G] or null
  const int* mask;        // [B, S] or null
  void* out;              // [B*S, nh*hd] model dtype
  int B, S, nh, nkv, hd, window, G;
  float scale;            // 1/sqrt(hd)
};
hipError_t attention(DType dt, const AttnParams& p, hipStream_t s);

// probs[b,h,i,:] = softmax of row i's visible scores, 0 elsewhere (tap only)
hipError_t attention_probs(DType dt, const AttnParams& p, float* probs, hipStream_t s);
// v[b,kvh,s,:] from the transposed V^T (tap only)
hipError_t attention_values(DType dt, const AttnParams& p, void* v, hipStream_t s);

// scores[b,h,i,j] = q.k/sqrt(hd) or -inf (tap only)
hipError_t attention_scores(DType dt, const AttnParams& p, float* scores,
                            hipStream_t s);

// ----------------------------------------------------------------- MoE
// logits [T, E] model dtype -> idx [T, k] int32, w [T, k] float32.
hipError_t moe_topk(DType dt, const void* logits, const float* bias, int T,
                    int E, int k, float route_scale, int* idx, float* w,
                    hipStream_t s);
// Stable token-major dispatch of the T*k (token, slot) pairs by expert:
// gcnt[E], goff[E]; for each grouped row r, row_token[r] (its token) and
// row_weight[r] (its pair's slot weight w[pair]); for each pair p,
// pair_row[p] (its grouped row).  hist is scratch of
// dispatch_hist_ints(T*k, E) ints.
// The (token, slot) pairs are counted per chunk of `tpc` tokens (tpc * k
// pairs): hist[e * nchunks + c].  With `counted`, hist already holds those
// counts (the router GEMM's fused epilogue wrote them) and only the scan
// and the write pass run.
hipError_t moe_dispatch(const int* idx, const float* w, int T, int k, int E, int* gcnt,
                        int* goff, int* row_token, int* pair_row, float* row_weight,
                        int* hist, int tpc, bool counted, hipStream_t s);
constexpr int DISPATCH_TOKENS = 64;  // tokens per dispatch chunk (at least)
inline int64_t dispatch_hist_ints(int64_t T, int E) {
  return ((T + DISPATCH_TOKENS - 1) / DISPATCH_TOKENS) * E;
}

}  // namespace blk
