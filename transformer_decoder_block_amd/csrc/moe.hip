// Router top-k and token dispatch of the afmoe mixture (nnterp afmoe page,
// section 03 "The Notes": the router's logits are in the model's dtype and
// are cast to float32 before the sigmoid and the bias add; the bias only
// chooses the experts; the weights are the chosen unbiased sigmoids
// renormalised to sum to route_scale; no expert groups).
//
// topk: one wavefront per token; lane j owns experts j, j+64, ...  The
// sigmoid is evaluated in double precision and rounded once to float32, so
// it is the correctly rounded float32 sigmoid of the logit; the biased
// score is the float32 sum of that and the float32 bias.  k rounds of a
// wave-wide arg-max (larger score first, lower expert index on ties) pick
// the slots in descending order.
//
// dispatch: the T*k (token, slot) pairs are grouped by expert in token-major
// order (a stable counting sort), with no atomics: per-chunk histograms,
// one scan over (expert, chunk), and a per-chunk write pass.
#include "common.h"
#include "kernels.h"

namespace blk {

template <typename T>
__global__ void __launch_bounds__(256) topk_kernel(const T* __restrict__ logits,
                                                   const float* __restrict__ bias,
                                                   int ntok, int E, int k, float rs,
                                                   int* __restrict__ idx,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  constexpr int MAXE = 4;  // experts per lane (E <= 256)
  float sg[MAXE], sc[MAXE];
#pragma unroll
  for (int j = 0; j < MAXE; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      const double l = (double)to_f32(logits[(int64_t)t * E + e]);
      sg[j] = (float)(1.0 / (1.0 + exp(-l)));
      sc[j] = sg[j] + bias[e];
    } else {
      sg[j] = 0.f;
      sc[j] = -INFINITY;
    }
  }
  unsigned taken = 0;
  float wsum = 0.f;
  int my_slot_e = -1;
  float my_slot_s = 0.f;
  for (int slot = 0; slot < k; ++slot) {
    // lane-local best: largest score, lowest expert on ties
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < MAXE; ++j) {
      const int e = lane + 64 * j;
      if (e < E && !(taken & (1u << j))) {
        if (sc[j] > bv || (sc[j] == bv && e < be)) { bv = sc[j]; be = e; }
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    // the owner marks it taken and publishes its unbiased sigmoid
    float s_sel = 0.f;
    if ((be & 63) == lane) {
      const int j = be >> 6;
#pragma unroll
      for (int jj = 0; jj < MAXE; ++jj)
        if (jj == j) { taken |= 1u << jj; s_sel = sg[jj]; }
    }
    s_sel = __shfl(s_sel, be & 63, 64);
    wsum += s_sel;
    if (lane == slot) { my_slot_e = be; my_slot_s = s_sel; }
  }
  if (lane < k) {
    idx[(int64_t)t * k + lane] = my_slot_e;
    w[(int64_t)t * k + lane] = my_slot_s / wsum * rs;
  }
}

hipError_t moe_topk(DType dt, const void* logits, const float* bias, int T, int E, int k,
                    float route_scale, int* idx, float* w, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  if (dt == DType::BF16)
    hipLaunchKernelGGL((topk_kernel<bf16>), grid, block, 0, s, (const bf16*)logits, bias,
                       T, E, k, route_scale, idx, w);
  else
    hipLaunchKernelGGL((topk_kernel<float>), grid, block, 0, s, (const float*)logits,
                       bias, T, E, k, route_scale, idx, w);
  return hipGetLastError();
}

constexpr int DCHUNK = 1024;  // pairs per dispatch chunk

// hist[c * E + e] = number of pairs of chunk c routed to expert e.
__global__ void __launch_bounds__(256) dispatch_count(const int* __restrict__ idx, int npairs,
                                                      int E, int* __restrict__ hist) {
  __shared__ int sidx[DCHUNK];
  const int c = blockIdx.x;
  const int p0 = c * DCHUNK;
  const int n = min(DCHUNK, npairs - p0);
  for (int i = threadIdx.x; i < n; i += 256) sidx[i] = idx[p0 + i];
  __syncthreads();
  const int e = threadIdx.x;
  if (e < E) {
    int cnt = 0;
    for (int i = 0; i < n; ++i) cnt += (sidx[i] == e);
    hist[c * E + e] = cnt;
  }
}

// gcnt[e] = total; goff[e] = exclusive scan of gcnt; hist[c*E+e] becomes the
// first output row of chunk c's pairs of expert e.
__global__ void __launch_bounds__(256) dispatch_scan(int* __restrict__ hist, int nchunks,
                                                     int E, int* __restrict__ gcnt,
                                                     int* __restrict__ goff) {
  __shared__ int tot[256];
  const int e = threadIdx.x;
  int t = 0;
  if (e < E)
    for (int c = 0; c < nchunks; ++c) t += hist[c * E + e];
  tot[e] = (e < E) ? t : 0;
  __syncthreads();
  if (e < E) {
    int off = 0;
    for (int j = 0; j < e; ++j) off += tot[j];
    gcnt[e] = t;
    goff[e] = off;
    for (int c = 0; c < nchunks; ++c) {
      const int h = hist[c * E + e];
      hist[c * E + e] = off;
      off += h;
    }
  }
}

__global__ void __launch_bounds__(256) dispatch_write(const int* __restrict__ idx, int npairs,
                                                      int k, int E,
                                                      const int* __restrict__ hist,
                                                      int* __restrict__ row_token,
                                                      int* __restrict__ row_pair) {
  __shared__ int sidx[DCHUNK];
  const int c = blockIdx.x;
  const int p0 = c * DCHUNK;
  const int n = min(DCHUNK, npairs - p0);
  for (int i = threadIdx.x; i < n; i += 256) sidx[i] = idx[p0 + i];
  __syncthreads();
  const int e = threadIdx.x;
  if (e < E) {
    int pos = hist[c * E + e];
    for (int i = 0; i < n; ++i) {
      if (sidx[i] == e) {
        row_pair[pos] = p0 + i;
        row_token[pos] = (p0 + i) / k;
        ++pos;
      }
    }
  }
}

hipError_t moe_dispatch(const int* idx, int T, int k, int E, int* gcnt, int* goff,
                        int* row_token, int* row_pair, int* hist, hipStream_t s) {
  const int npairs = T * k;
  const int nchunks = (npairs + DCHUNK - 1) / DCHUNK;
  hipLaunchKernelGGL(dispatch_count, dim3(nchunks), dim3(256), 0, s, idx, npairs, E, hist);
  hipLaunchKernelGGL(dispatch_scan, dim3(1), dim3(256), 0, s, hist, nchunks, E, gcnt, goff);
  hipLaunchKernelGGL(dispatch_write, dim3(nchunks), dim3(256), 0, s, idx, npairs, k, E, hist,
                     row_token, row_pair);
  return hipGetLastError();
}

}  // namespace blk
