/*
 * libblock -- forward pass of one Llama-family decoder block on an MI355X
 * (gfx950), as a C ABI.
 *
 * The block (sources: safebydesign granite sheet "LlamaForCausalLM
 * 32L-4096d", section "Implementing it"; nnterp encyclopedia pages arcee,
 * afmoe and apertus, sections 02 "support()" and 03 "The Notes"):
 *
 *   a   = rmsnorm(x, w_in_norm)
 *   q,k,v = a Wq^T, a Wk^T, a Wv^T      (per-head q/k RMSNorm if qk_norm,
 *                                        then rotary if use_rope)
 *   h   = softmax(q k^T / sqrt(hd), causal [, window] [, key mask]) v
 *         (grouped-query: query head j reads KV head j / (nh/nkv))
 *   h  *= sigmoid(a Wgate^T)             (if head_gate_dim > 0)
 *   o   = h Wo^T                         (post_attn rmsnorm if sandwich_norm)
 *   mid = x + o
 *   m   = rmsnorm(mid, w_mlp_norm)
 *   y   = mid + mlp(m)                   (post_mlp rmsnorm of mlp(m) if sandwich_norm)
 *
 * mlp: SwiGLU (Llama), squared ReLU (arcee), xIELU (apertus) or the
 * sigmoid-routed mixture with a shared expert (afmoe).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous,
 *    16-byte aligned, owned by the caller; libblock never frees them.
 *  - Weights use the Linear layout [out_features, in_features], no bias.
 *  - Model-dtype tensors (x, y, weights, operand taps) are BLK_F32 (IEEE
 *    float) or BLK_BF16 (bfloat16 bit patterns) as set by blk_config.dtype.
 *  - Errors are returned as blk_status; no exception crosses the ABI.  A
 *    call refused by validation enqueues nothing; a BLK_E_HIP from a
 *    forward leaves the launches before the failing one enqueued (see
 *    blk_forward).  blk_last_error() gives a readable reason for the
 *    calling thread's last failure.
 *  - Results are bitwise deterministic for identical inputs (no floating
 *    point atomics anywhere).
 */
#ifndef LIBBLOCK_H
#define LIBBLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BLK_ABI_VERSION 6

typedef enum blk_status {
  BLK_OK = 0,
  BLK_E_NULL = 1,    /* a required pointer is NULL                         */
  BLK_E_CONFIG = 2,  /* the configuration is invalid or unsupported        */
  BLK_E_SHAPE = 3,   /* batch/seq exceed the created maxima or are < 1     */
  BLK_E_ALIGN = 4,   /* a pointer is not 16-byte aligned                   */
  BLK_E_DTYPE = 5,   /* a tap asks for a dtype it does not support         */
  BLK_E_OOM = 6,     /* device allocation failed in blk_create             */
  BLK_E_HIP = 7      /* the HIP runtime reported an error                  */
} blk_status;

typedef enum blk_dtype { BLK_F32 = 0, BLK_BF16 = 1, BLK_I32 = 2 } blk_dtype;

typedef enum blk_mlp_kind {
  BLK_MLP_SWIGLU = 0, /* Llama: down(silu(gate(m)) * up(m))                 */
  BLK_MLP_RELU2 = 1,  /* arcee: down(relu(up(m))^2)                         */
  BLK_MLP_XIELU = 2,  /* apertus: down(xielu(up(m)))                        */
  BLK_MLP_MOE = 3     /* afmoe: routed SwiGLU experts + shared SwiGLU expert */
} blk_mlp_kind;

/*
 * Block configuration.  Field names follow the config tables of the nnterp
 * pages (hidden_size, num_attention_heads, num_key_value_heads, head_dim,
 * intermediate_size, rms_norm_eps, sliding_window, num_experts,
 * num_experts_per_tok, moe_intermediate_size, num_shared_experts,
 * route_scale).
 *
 * Supported: head_dim 64 or 128; hidden, intermediate, moe_intermediate
 * multiples of 8 and hidden <= 8192; num_heads a multiple of num_kv_heads;
 * head_gate_dim 0, num_heads or num_heads*head_dim; num_experts <= 256,
 * 1 <= top_k <= min(16, num_experts).
 */
typedef struct blk_config {
  int32_t dtype;              /* blk_dtype: BLK_F32 or BLK_BF16            */
  int32_t hidden;             /* H                                         */
  int32_t num_heads;          /* nh                                        */
  int32_t num_kv_heads;       /* nkv                                       */
  int32_t head_dim;           /* hd                                        */
  int32_t mlp_kind;           /* blk_mlp_kind                              */
  int32_t intermediate;       /* dense MLP width (SWIGLU/RELU2/XIELU)      */
  float rms_eps;              /* every RMSNorm's eps (1e-5 on the pages)   */
  float rope_theta;           /* 10000 on the pages' plain rotary          */
  int32_t use_rope;           /* 0 on an afmoe full-attention block        */
  int32_t qk_norm;            /* per-head q/k RMSNorm before the rotary    */
  int32_t sandwich_norm;      /* afmoe: post-attention and post-MLP norms  */
  int32_t sliding_window;     /* W keys incl. the query's own; 0 = off     */
  int32_t head_gate_dim;      /* 0, nh (one gate per head), nh*hd          */
  int32_t num_experts;        /* E (MOE)                                   */
  int32_t top_k;              /* experts per token (MOE)                   */
  int32_t moe_intermediate;   /* width of one expert (MOE)                 */
  int32_t num_shared_experts; /* shared width = moe_intermediate * this   */
  float route_scale;          /* expert weights sum to this (MOE)          */
  float xielu_beta;           /* 0.5 on the apertus page                   */
  float xielu_eps;            /* -1e-6 on the apertus page                 */
  int32_t max_batch;          /* workspace is sized for max_batch*max_seq  */
  int32_t max_seq;
} blk_config;

/*
 * Weights: caller-owned device pointers in the model dtype unless noted.
 * Pointers a configuration does not use may be NULL.
 */
typedef struct blk_weights {
  const void* w_in_norm;        /* [H]   input_layernorm (attention_layernorm) */
  const void* w_post_attn_norm; /* [H]   afmoe post_attention_layernorm        */
  const void* w_mlp_norm;       /* [H]   post_attention_layernorm (Llama,
                                         arcee), feedforward_layernorm
                                         (apertus), pre_mlp_layernorm (afmoe)  */
  const void* w_post_mlp_norm;  /* [H]   afmoe post_mlp_layernorm              */
  const void* wq;               /* [nh*hd, H]                                  */
  const void* wk;               /* [nkv*hd, H]                                 */
  const void* wv;               /* [nkv*hd, H]                                 */
  const void* wo;               /* [H, nh*hd]                                  */
  const void* w_q_norm;         /* [hd]  one gain shared by every query head   */
  const void* w_k_norm;         /* [hd]                                        */
  const void* w_head_gate;      /* [head_gate_dim, H]  afmoe gate_proj         */
  const void* w_gate;           /* [I, H]  SWIGLU                              */
  const void* w_up;             /* [I, H]                                      */
  const void* w_down;           /* [H, I]                                      */
  double xielu_alpha_p_raw;     /* host value, before softplus (XIELU)         */
  double xielu_alpha_n_raw;     /* host value, before beta + softplus          */
  const void* w_router;         /* [E, H]  router.gate                         */
  const float* expert_bias;     /* [E]     float32 selection bias              */
  const void* w_e_gate;         /* [E, I_e, H]                                 */
  const void* w_e_up;           /* [E, I_e, H]                                 */
  const void* w_e_down;         /* [E, H, I_e]                                 */
  const void* w_sh_gate;        /* [I_sh, H]  shared expert                    */
  const void* w_sh_up;          /* [I_sh, H]                                   */
  const void* w_sh_down;        /* [H, I_sh]                                   */
} blk_weights;

/* One optional output of a named interior value: NULL ptr = not requested. */
typedef struct blk_tap {
  void* ptr;
  int32_t dtype; /* blk_dtype; each tap accepts the dtype listed below */
} blk_tap;

/*
 * Taps, named as in the support() tables of the nnterp pages.  Each is
 * [batch, seq, ...] with the dtype it must be requested in:
 *  layer_input           [B,S,H]        model dtype (a copy of x)
 *  attention_norm_output [B,S,H]        model dtype: the exact operand of
 *                                       the Q/K/V projections
 *  attention_scores      [B,nh,S,S]     F32, scaled by 1/sqrt(hd), after q/k
 *                                       norm and rotary, -inf where masked
 *  layer_mid             [B,S,H]        F32 (the block keeps it in float32)
 *  mlp_input             [B,S,H]        model dtype: the exact MLP operand
 *  layer_output          [B,S,H]        F32, before the rounding to y
 *  attention_output      [B,S,H]        F32 (what attention adds)
 *  mlp_output            [B,S,H]        F32 (what the MLP adds)
 *  router_logits         [B,S,E]        model dtype (MOE)
 *  expert_indices        [B,S,top_k]    I32, slots in descending biased
 *                                       score, ties to the lower index (MOE)
 *  expert_weights        [B,S,top_k]    F32 (MOE)
 * Interior values of the attention and the MLP (support() tables, the
 * attention and mlp rows):
 *  attention_queries     [B,nh,S,hd]    model dtype: the queries the
 *                                       attention reads (after q norm and
 *                                       rotary)
 *  attention_keys        [B,nkv,S,hd]   model dtype (after k norm, rotary)
 *  attention_values      [B,nkv,S,hd]   model dtype
 *  attention_probabilities [B,nh,S,S]   F32, softmax rows, 0 where masked
 *                                       (a row with no visible key is 0)
 *  attention_head_outputs [B,S,nh,hd]   model dtype, before the head gate
 *  attention_premix      [B,S,nh*hd]    model dtype: the o_proj operand
 *                                       (after the head gate)
 *  mlp_neurons           [B,S,I]        model dtype: the down projection's
 *                                       operand (SWIGLU, RELU2, XIELU)
 *  mlp_norm_output       [B,S,H]        model dtype: the normed stream
 *                                       entering the MLP (the same values
 *                                       as mlp_input: the MLP is called
 *                                       with the norm's output)
 *  mlp_activation        [B,S,I]        model dtype: the activation
 *                                       function's output, silu(gate) on
 *                                       SWIGLU (an extra GEMM), the neurons
 *                                       on RELU2 and XIELU
 *  expert_outputs        [B,S,top_k,H]  model dtype: each slot's expert
 *                                       output times its weight (MOE)
 *  routed_output         [B,S,H]        F32: the sum of the slots (MOE)
 *  shared_expert_output  [B,S,H]        F32 (MOE with a shared expert)
 * The interior taps are produced by extra copies or kernels on the same
 * stream (the probabilities and the ungated head outputs recompute the
 * attention); requesting them slows the call down.
 */
typedef struct blk_taps {
  blk_tap layer_input;
  blk_tap attention_norm_output;
  blk_tap attention_scores;
  blk_tap layer_mid;
  blk_tap mlp_input;
  blk_tap layer_output;
  blk_tap attention_output;
  blk_tap mlp_output;
  blk_tap router_logits;
  blk_tap expert_indices;
  blk_tap expert_weights;
  blk_tap attention_queries;
  blk_tap attention_keys;
  blk_tap attention_values;
  blk_tap attention_probabilities;
  blk_tap attention_head_outputs;
  blk_tap attention_premix;
  blk_tap mlp_neurons;
  blk_tap expert_outputs;
  blk_tap routed_output;
  blk_tap shared_expert_output;
  blk_tap mlp_activation;
  blk_tap mlp_norm_output;
} blk_taps;

/* The residual stream in and out. */
typedef struct blk_io {
  const void* x;                  /* [B,S,H] layer_input, model dtype        */
  const int32_t* attention_mask;  /* [B,S] 1 = token, 0 = padding; NULL =
                                     all ones.  Masks keys only.            */
  int32_t batch;                  /* 1 <= B <= max_batch                     */
  int32_t seq;                    /* 1 <= S <= max_seq                       */
  void* y;                        /* [B,S,H] layer_output, model dtype;
                                     required, must not alias x             */
} blk_io;

typedef struct blk_handle blk_handle;

/*
 * Validate cfg, precompute the rotary table, choose the kernels and
 * allocate the device workspace for max_batch*max_seq tokens on the
 * current HIP device.  *out receives the handle (owned by libblock; free it
 * with blk_destroy).  Errors: BLK_E_NULL, BLK_E_CONFIG, BLK_E_OOM,
 * BLK_E_HIP.
 */
blk_status blk_create(const blk_config* cfg, blk_handle** out);

/*
 * Enqueue one forward pass of the block on `stream` (a hipStream_t; NULL =
 * the default stream) and return.  No host synchronisation, no allocation,
 * no weight copies.  Success means "enqueued"; device-side faults surface
 * at the caller's next synchronisation.  `taps` may be NULL.  Validation
 * (pointers, alignment, sizes, tap dtypes) happens before any launch, so a
 * validation error (BLK_E_NULL, BLK_E_CONFIG, BLK_E_SHAPE, BLK_E_ALIGN,
 * BLK_E_DTYPE) enqueues nothing and leaves y untouched.  BLK_E_HIP is
 * different: it reports a launch (or tap copy) that the HIP runtime refused
 * part-way through the sequence, and the kernels enqueued before it stay
 * enqueued and run; y and the taps are then undefined, the handle stays
 * usable, and blk_last_error() names the step that failed.
 * A handle must not be used by two forwards that may run concurrently (the
 * workspace is shared).  With taps NULL the call enqueues kernels only (no
 * memset, copy or synchronisation), so it may be captured into a HIP graph
 * and replayed while the pointers it was given stay valid.
 */
blk_status blk_forward(blk_handle* h, const blk_io* io, const blk_weights* w,
                       const blk_taps* taps, void* stream);

/*
 * A stack of n_layers blocks of this handle's configuration, layers[0]
 * first, each with its own weights: the model loop of the granite sheet
 * "LlamaForCausalLM 32L-4096d", section "Implementing it", where each
 * layer's output is the next layer's input.  io->x is the first layer's
 * input and io->y receives the last layer's output; io->attention_mask
 * (may be NULL) applies to every layer.  The outputs of the layers before
 * the last alternate between io->y and a buffer of the handle's workspace
 * (max_batch*max_seq*hidden in the model dtype), so nothing is allocated.
 * Same contract as blk_forward, without taps; io and every layer's
 * weights are validated before the first launch, so a validation error
 * enqueues nothing.  A BLK_E_HIP in layer l leaves layers 0 .. l-1 and the
 * kernels of layer l before the failing one enqueued; y is then undefined.
 * Errors: BLK_E_NULL, BLK_E_CONFIG (n_layers < 1, io.y aliasing io.x),
 * BLK_E_SHAPE, BLK_E_ALIGN, BLK_E_HIP.
 */
blk_status blk_forward_layers(blk_handle* h, const blk_io* io,
                              const blk_weights* const* layers, int32_t n_layers,
                              void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  One
 * forward pass exactly as blk_forward (same kernels, same taps, same
 * checks, same errors), but with no handle: the configuration comes with
 * the call, and the workspace is a static device array of
 * BLK_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  cfg->max_batch and cfg->max_seq are ignored;
 * the workspace is laid out for io->batch x io->seq, and a call whose
 * workspace would not fit is refused with BLK_E_SHAPE (the message gives
 * the bytes it would need) before anything is enqueued.  The rotary table
 * is rebuilt on `stream` by each call (angles in double, as blk_create).
 * The call allocates no device memory, and no host memory unless it fails
 * (the error text).  The first call on a device looks the array's address
 * up once (hipGetSymbolAddress).  Every call on one GPU shares that GPU's
 * array, which keeps the last call's contents (nothing in it needs to
 * start at zero): calls that may overlap on one GPU -- two streams, or two
 * host threads -- race and must be serialised by the caller.
 */
#define BLK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
blk_status blk_forward_noalloc(const blk_config* cfg, const blk_io* io, const blk_weights* w,
                               const blk_taps* taps, void* stream);

/* Free the workspace and the handle (NULL is ignored). */
void blk_destroy(blk_handle* h);

/* Static name of a status code. */
const char* blk_status_str(blk_status s);

/* Readable detail of the calling thread's last failed call ("" if none). */
const char* blk_last_error(void);

/* BLK_ABI_VERSION of the loaded library. */
int32_t blk_abi_version(void);

/* Bytes of device workspace the handle holds. */
size_t blk_workspace_bytes(const blk_handle* h);

/*
 * Measurement.  blk_profile_begin creates max_forwards * 32 HIP events;
 * each following blk_forward (up to max_forwards of them) records an event
 * on its stream before every kernel of the block and one after the last.
 * blk_profile_end synchronises the device, sums the elapsed time of every
 * span over the recorded forwards, writes at most max_entries
 * (name, total milliseconds, number of forwards) triples -- names are
 * static strings owned by libblock, e.g. "gemm_qkv", "attention",
 * "gemm_up" -- frees the events and returns the number of entries (-1 if
 * profiling was not begun).  Without blk_profile_begin no event is recorded.
 */
blk_status blk_profile_begin(blk_handle* h, int32_t max_forwards);
int32_t blk_profile_end(blk_handle* h, int32_t max_entries, const char** names,
                        double* total_ms, int32_t* calls);

#ifdef __cplusplus
}
#endif

#endif /* LIBBLOCK_H */
