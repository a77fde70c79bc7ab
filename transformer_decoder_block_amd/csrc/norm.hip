// Row kernels of the block: RMSNorm, the afmoe norm-add-norm tail of the
// attention, and the afmoe combine of the mixture's slots.
//
// RMSNorm (granite sheet "LlamaForCausalLM 32L-4096d", section
// "Implementing it": rmsnorm(x, w, eps)): out = g * x / sqrt(mean(x^2) + eps),
// float32 arithmetic, one rounding to the model dtype at the end.
//
// One wavefront per row: each lane owns 16-byte chunks lane, lane+64, ...
// of the row, keeps them in registers between the reduction and the
// scaling, and the sum of squares is reduced across the 64 lanes.  These
// kernels are HBM-bound: every row is read once and written once.
#include "common.h"
#include "kernels.h"

namespace blk {

template <typename Tx, typename T, int MAXCH>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const Tx* __restrict__ x,
                                                      const T* __restrict__ g,
                                                      T* __restrict__ out, int rows,
                                                      int H, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const Tx* xr = x + (int64_t)row * H;
  float v[MAXCH][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const int c = (lane + 64 * j) * 8;
    if (c < H) {
      load8(xr + c, v[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += v[j][i] * v[j][i];
    }
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);
  T* orow = out + (int64_t)row * H;
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const int c = (lane + 64 * j) * 8;
    if (c < H) {
      float gv[8], o[8];
      load8(g + c, gv);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = gv[i] * (v[j][i] * inv);
      store8(orow + c, o);
    }
  }
}

template <typename T, int MAXCH>
__global__ void __launch_bounds__(256) norm_add_norm_kernel(
    const float* __restrict__ o, const T* __restrict__ x, const T* __restrict__ g_post,
    const T* __restrict__ g_pre, float* __restrict__ attn_out, float* __restrict__ mid,
    T* __restrict__ m, int rows, int H, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t base = (int64_t)row * H;
  float v[MAXCH][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const int c = (lane + 64 * j) * 8;
    if (c < H) {
      load8(o + base + c, v[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += v[j][i] * v[j][i];
    }
  }
  ss = wave_sum(ss);
  const float inv1 = 1.0f / sqrtf(ss / (float)H + eps);
  float ss2 = 0.f;
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const int c = (lane + 64 * j) * 8;
    if (c < H) {
      float gv[8], xv[8];
      load8(g_post + c, gv);
      load8(x + base + c, xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a = gv[i] * (v[j][i] * inv1);
        v[j][i] = a;
      }
      if (attn_out) store8(attn_out + base + c, v[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[j][i] = xv[i] + v[j][i];
        ss2 += v[j][i] * v[j][i];
      }
      store8(mid + base + c, v[j]);
    }
  }
  ss2 = wave_sum(ss2);
  const float inv2 = 1.0f / sqrtf(ss2 / (float)H + eps);
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const int c = (lane + 64 * j) * 8;
    if (c < H) {
      float gv[8], r[8];
      load8(g_pre + c, gv);
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = gv[i] * (v[j][i] * inv2);
      store8(m + base + c, r);
    }
  }
}

// Eight consecutive elements kept as loaded (bf16: 16 bytes) until added.
template <typename T>
struct Raw8;
template <>
struct Raw8<bf16> {
  uint4 r;
  __device__ __forceinline__ void load(const bf16* p) { r = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void add_to(float* f) const {
    float t[8];
    unpack8(r, t);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] += t[i];
  }
};
template <>
struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void add_to(float* f) const {
    f[0] += a.x; f[1] += a.y; f[2] += a.z; f[3] += a.w;
    f[4] += b.x; f[5] += b.y; f[6] += b.z; f[7] += b.w;
  }
};

// raw = shared[t] + the slots 0..k-1 in that order (slot s is stage row
// pair_row[t*k + s]).  The slot loads of a row go out several slots at a
// time for all of the lane's chunks before any is added, so a wave keeps
// many loads in flight; the sum order is fixed.
template <typename T, int MAXCH>
__global__ void __launch_bounds__(256) moe_combine_kernel(
    const T* __restrict__ stage, const int* __restrict__ pair_row,
    const float* __restrict__ shared,
    const float* __restrict__ mid, const T* __restrict__ g_post, int top_k,
    float* __restrict__ mlp_out, float* __restrict__ out_f32, T* __restrict__ y,
    int rows, int H, float eps, int sandwich) {
  // slots per batch of loads; the residual row is loaded up front when
  // the registers allow
  constexpr int SU = MAXCH >= 16 ? 1 : (MAXCH >= 8 ? 2 : 4);
  constexpr bool PRE_MID = MAXCH <= 4;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t base = (int64_t)row * H;
  // lane s < top_k holds the stage row of slot s (top_k <= 64)
  const int srow = lane < top_k ? pair_row[(int64_t)row * top_k + lane] : 0;
  float v[MAXCH][8], mv[PRE_MID ? MAXCH : 1][8];
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const int c = (lane + 64 * j) * 8;
    if (c < H) {
      if constexpr (PRE_MID) load8(mid + base + c, mv[j]);
      if (shared) {
        load8(shared + base + c, v[j]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[j][i] = 0.f;
      }
    }
  }
  for (int s0 = 0; s0 < top_k; s0 += SU) {
    Raw8<T> t[MAXCH][SU];
    int64_t sb[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u)
      sb[u] = (int64_t)__builtin_amdgcn_readlane(srow, s0 + u < top_k ? s0 + u : 0) * H;
#pragma unroll
    for (int j = 0; j < MAXCH; ++j) {
      const int c = (lane + 64 * j) * 8;
#pragma unroll
      for (int u = 0; u < SU; ++u)
        if (c < H && s0 + u < top_k) t[j][u].load(stage + sb[u] + c);
    }
#pragma unroll
    for (int j = 0; j < MAXCH; ++j) {
      const int c = (lane + 64 * j) * 8;
#pragma unroll
      for (int u = 0; u < SU; ++u)
        if (c < H && s0 + u < top_k) t[j][u].add_to(v[j]);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const int c = (lane + 64 * j) * 8;
    if (c < H) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += v[j][i] * v[j][i];
    }
  }
  float inv = 1.0f;
  if (sandwich) {
    ss = wave_sum(ss);
    inv = 1.0f / sqrtf(ss / (float)H + eps);
  }
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const int c = (lane + 64 * j) * 8;
    if (c < H) {
      if (sandwich) {
        float gv[8];
        load8(g_post + c, gv);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[j][i] = gv[i] * (v[j][i] * inv);
      }
      if (mlp_out) store8(mlp_out + base + c, v[j]);
      float m8[8];
      if constexpr (PRE_MID) {
#pragma unroll
        for (int i = 0; i < 8; ++i) m8[i] = mv[j][i];
      } else {
        load8(mid + base + c, m8);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) v[j][i] = m8[i] + v[j][i];
      if (out_f32) store8(out_f32 + base + c, v[j]);
      store8(y + base + c, v[j]);
    }
  }
}

template <int MAXCH>
static hipError_t rmsnorm_dispatch(DType dt, int x_f32, const void* x, const void* g,
                                   void* out, int rows, int H, float eps,
                                   hipStream_t s) {
  dim3 grid((rows + 3) / 4), block(256);
  if (dt == DType::BF16) {
    if (x_f32)
      hipLaunchKernelGGL((rmsnorm_kernel<float, bf16, MAXCH>), grid, block, 0, s,
                         (const float*)x, (const bf16*)g, (bf16*)out, rows, H, eps);
    else
      hipLaunchKernelGGL((rmsnorm_kernel<bf16, bf16, MAXCH>), grid, block, 0, s,
                         (const bf16*)x, (const bf16*)g, (bf16*)out, rows, H, eps);
  } else {
    hipLaunchKernelGGL((rmsnorm_kernel<float, float, MAXCH>), grid, block, 0, s,
                       (const float*)x, (const float*)g, (float*)out, rows, H, eps);
  }
  return hipGetLastError();
}

#define BLK_BY_WIDTH(H, CALL)        \
  do {                               \
    if ((H) <= 1024) { CALL(2); }    \
    else if ((H) <= 2048) { CALL(4); } \
    else if ((H) <= 4096) { CALL(8); } \
    else { CALL(16); }               \
  } while (0)

hipError_t rmsnorm(DType dt, int x_f32, const void* x, const void* g, void* out,
                   int rows, int H, float eps, hipStream_t s) {
#define C_(n) return rmsnorm_dispatch<n>(dt, x_f32, x, g, out, rows, H, eps, s)
  BLK_BY_WIDTH(H, C_);
#undef C_
}

template <int MAXCH>
static hipError_t nan_dispatch(DType dt, const float* o, const void* x, const void* gp,
                               const void* gq, float* ao, float* mid, void* m, int rows,
                               int H, float eps, hipStream_t s) {
  dim3 grid((rows + 3) / 4), block(256);
  if (dt == DType::BF16)
    hipLaunchKernelGGL((norm_add_norm_kernel<bf16, MAXCH>), grid, block, 0, s, o,
                       (const bf16*)x, (const bf16*)gp, (const bf16*)gq, ao, mid,
                       (bf16*)m, rows, H, eps);
  else
    hipLaunchKernelGGL((norm_add_norm_kernel<float, MAXCH>), grid, block, 0, s, o,
                       (const float*)x, (const float*)gp, (const float*)gq, ao, mid,
                       (float*)m, rows, H, eps);
  return hipGetLastError();
}

hipError_t norm_add_norm(DType dt, const float* o, const void* x, const void* g_post,
                         const void* g_pre, float* attn_out, float* mid, void* m,
                         int rows, int H, float eps, hipStream_t s) {
#define C_(n) return nan_dispatch<n>(dt, o, x, g_post, g_pre, attn_out, mid, m, rows, H, eps, s)
  BLK_BY_WIDTH(H, C_);
#undef C_
}

template <int MAXCH>
static hipError_t comb_dispatch(DType dt, const void* stage, const int* pair_row,
                                const float* shared,
                                const float* mid, const void* g_post, int top_k,
                                float* mlp_out, float* out_f32, void* y, int rows, int H,
                                float eps, int sandwich, hipStream_t s) {
  dim3 grid((rows + 3) / 4), block(256);
  if (dt == DType::BF16)
    hipLaunchKernelGGL((moe_combine_kernel<bf16, MAXCH>), grid, block, 0, s,
                       (const bf16*)stage, pair_row, shared, mid, (const bf16*)g_post, top_k,
                       mlp_out, out_f32, (bf16*)y, rows, H, eps, sandwich);
  else
    hipLaunchKernelGGL((moe_combine_kernel<float, MAXCH>), grid, block, 0, s,
                       (const float*)stage, pair_row, shared, mid, (const float*)g_post, top_k,
                       mlp_out, out_f32, (float*)y, rows, H, eps, sandwich);
  return hipGetLastError();
}

template <typename T>
__global__ void __launch_bounds__(256) sum_slots_kernel(const T* __restrict__ stage,
                                                        const int* __restrict__ pair_row,
                                                        int top_k, float* __restrict__ routed,
                                                        int rows, int H) {
  const int64_t n = (int64_t)rows * H;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / H, c = e % H;
    float acc = 0.f;
    for (int s = 0; s < top_k; ++s)
      acc += to_f32(stage[(int64_t)pair_row[r * top_k + s] * H + c]);
    routed[e] = acc;
  }
}

hipError_t moe_sum_slots(DType dt, const void* stage, const int* pair_row, int top_k,
                         float* routed, int rows, int H, hipStream_t s) {
  const int64_t n = (int64_t)rows * H;
  const int blocks = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  if (dt == DType::BF16)
    hipLaunchKernelGGL((sum_slots_kernel<bf16>), dim3(blocks), dim3(256), 0, s,
                       (const bf16*)stage, pair_row, top_k, routed, rows, H);
  else
    hipLaunchKernelGGL((sum_slots_kernel<float>), dim3(blocks), dim3(256), 0, s,
                       (const float*)stage, pair_row, top_k, routed, rows, H);
  return hipGetLastError();
}

// One 256-thread block per (token, slot) pair: its stage row copied in
// 4-byte words (H * sizeof(T) is a multiple of 16).
__global__ void __launch_bounds__(256) gather_rows_kernel(const uint32_t* __restrict__ stage,
                                                          const int* __restrict__ pair_row,
                                                          uint32_t* __restrict__ out,
                                                          int words) {
  const int64_t p = blockIdx.x;
  const uint32_t* src = stage + (int64_t)pair_row[p] * words;
  uint32_t* dst = out + p * words;
  for (int i = threadIdx.x; i < words; i += 256) dst[i] = src[i];
}

hipError_t moe_gather_slots(DType dt, const void* stage, const int* pair_row, void* out,
                            int npairs, int H, hipStream_t s) {
  const int words = H * (dt == DType::BF16 ? 2 : 4) / 4;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(npairs), dim3(256), 0, s,
                     (const uint32_t*)stage, pair_row, (uint32_t*)out, words);
  return hipGetLastError();
}

hipError_t moe_combine(DType dt, const void* stage, const int* pair_row, const float* shared,
                       const float* mid, const void* g_post, int top_k, float* mlp_out,
                       float* out_f32, void* y, int rows, int H, float eps, int sandwich,
                       hipStream_t s) {
#define C_(n) return comb_dispatch<n>(dt, stage, pair_row, shared, mid, g_post, top_k, mlp_out, out_f32, y, rows, H, eps, sandwich, s)
  BLK_BY_WIDTH(H, C_);
#undef C_
}

}  // namespace blk
