// Router top-k and token dispatch of the afmoe mixture (nnterp afmoe page,
// section 03 "The Notes": the router's logits are in the model's dtype and
// are cast to float32 before the sigmoid and the bias add; the bias only
// chooses the experts; the weights are the chosen unbiased sigmoids
// renormalised to sum to route_scale; no expert groups).
//
// The router GEMM's epilogue does the sigmoid, bias and top-k itself when
// one tile holds every expert (gemm.hip, EPI_ROUTER); topk_kernel below
// serves the wider expert counts.
//
// topk: one wavefront per token; lane j owns experts j, j+64, ...  The
// sigmoid is evaluated in double precision and rounded once to float32, so
// it is the correctly rounded float32 sigmoid of the logit; the biased
// score is the float32 sum of that and the float32 bias.  k rounds of a
// wave-wide arg-max (larger score first, lower expert index on ties) pick
// the slots in descending order.
//
// dispatch: the T*k (token, slot) pairs are grouped by expert in token-major
// order (a stable counting sort), with no float atomics: per-chunk
// histograms (a chunk is the pairs of one router tile's tokens; the fused
// router epilogue counts them), a per-expert scan over the chunks, and a
// per-chunk write pass.
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

// hist[e * nchunks + c] = number of pairs of chunk c routed to expert e
// (integer LDS atomics: the count does not depend on their order).  Chunk c
// holds the pairs of tokens [c tpc, (c + 1) tpc).
__global__ void __launch_bounds__(256) dispatch_count(const int* __restrict__ idx, int npairs,
                                                      int E, int nchunks, int chunk_pairs,
                                                      int* __restrict__ hist) {
  __shared__ int cnt[256];
  const int c = blockIdx.x, t = threadIdx.x;
  const int p0 = c * chunk_pairs;
  const int n = min(chunk_pairs, npairs - p0);
  cnt[t] = 0;
  __syncthreads();
  for (int i = t; i < n; i += 256) atomicAdd(&cnt[idx[p0 + i]], 1);
  __syncthreads();
  if (t < E) hist[t * nchunks + c] = cnt[t];
}

// One block per expert: exclusive scan of its chunk counts in place (the
// row of the expert's group where chunk c's pairs start) and its total.
__global__ void __launch_bounds__(256) dispatch_scan(int* __restrict__ hist, int nchunks,
                                                     int* __restrict__ gcnt) {
  __shared__ int part[256];
  const int e = blockIdx.x, t = threadIdx.x;
  int* h = hist + (int64_t)e * nchunks;
  int carry = 0;
  for (int base = 0; base < nchunks; base += 256) {
    const int v = (base + t < nchunks) ? h[base + t] : 0;
    part[t] = v;
    __syncthreads();
    // Hillis-Steele inclusive scan over the 256 values
    for (int o = 1; o < 256; o <<= 1) {
      const int add = (t >= o) ? part[t - o] : 0;
      __syncthreads();
      part[t] += add;
      __syncthreads();
    }
    if (base + t < nchunks) h[base + t] = carry + part[t] - v;
    carry += part[255];
    __syncthreads();
  }
  if (t == 0) gcnt[e] = carry;
}

// One workgroup of eight waves per chunk writes the chunk's pairs in
// token-major order: expert e's pairs of chunk c go to rows
// goff[e] + hist[e][c] + their rank among the chunk's earlier pairs of e.
// Wave q takes the q-th eighth of the chunk's pairs.  Each wave first counts
// its part per expert (integer LDS atomics: order-free), so wave q's pairs
// of e start after those of waves 0 .. q-1; then it walks its part in
// rounds of 64 consecutive pairs, where a pair's rank inside its round is
// the number of lower lanes holding the same expert.  (The whole dispatch
// at the afmoe shape, scan and write: 26 us with one wave per chunk, which
// left the write latency-bound, 15 with four waves, 13.5 with eight, 14.7
// with sixteen.)
constexpr int DW_WAVES = 8;
__global__ void __launch_bounds__(64 * DW_WAVES) dispatch_write(
    const int* __restrict__ idx, const float* __restrict__ w, int npairs, int k, int E,
    int nchunks, int chunk_pairs, const int* __restrict__ hist, const int* __restrict__ gcnt,
    int* __restrict__ goff, int* __restrict__ row_token, int* __restrict__ pair_row,
    float* __restrict__ row_weight) {
  __shared__ int base[256];
  __shared__ int wpos[DW_WAVES][256];  // counts, then each wave's next row per expert
  const int c = blockIdx.x, t = threadIdx.x, l = t & 63, q = t >> 6;
  const int p0 = c * chunk_pairs;
  const int n = min(chunk_pairs, npairs - p0);
  const int qlen = (n + DW_WAVES - 1) / DW_WAVES;
  const int q0 = min(n, q * qlen), q1 = min(n, q0 + qlen);  // this wave's pairs
  for (int i = t; i < DW_WAVES * 256; i += 64 * DW_WAVES) (&wpos[0][0])[i] = 0;
  // first row of each expert's group: exclusive scan of the totals (wave
  // 0, lane l owns experts 4l .. 4l+3), plus this chunk's offset inside the
  // group
  if (q == 0) {
    int cnt[4], sum = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = 4 * l + r;
      cnt[r] = e < E ? gcnt[e] : 0;
      sum += cnt[r];
    }
    int inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (l >= o) inc += v;
    }
    int ex = inc - sum;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = 4 * l + r;
      if (e < E) {
        if (c == 0) goff[e] = ex;
        base[e] = ex + hist[e * nchunks + c];
      }
      ex += cnt[r];
    }
  }
  __syncthreads();
  for (int i = q0 + l; i < q1; i += 64) atomicAdd(&wpos[q][idx[p0 + i]], 1);
  __syncthreads();
  if (t < E) {  // thread e: the row where each wave's pairs of e start
    int run = base[t];
#pragma unroll
    for (int r = 0; r < DW_WAVES; ++r) {
      const int v = wpos[r][t];
      wpos[r][t] = run;
      run += v;
    }
  }
  __syncthreads();
  int* next = wpos[q];
  for (int r0 = q0; r0 < q1; r0 += 64) {
    const int i = r0 + l;
    const bool ok = i < q1;
    const int e = ok ? idx[p0 + i] : -1;
    int rank = 0;
    for (int j = 0; j < 64; ++j) {
      const int ej = __builtin_amdgcn_readlane(e, j);
      rank += (j < l && ej == e) ? 1 : 0;
    }
    if (ok) {
      const int pos = next[e] + rank;
      pair_row[p0 + i] = pos;
      row_token[pos] = (p0 + i) / k;
      row_weight[pos] = w[p0 + i];
    }
    // every lane has read its expert's next row before any lane moves it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (ok) atomicAdd(&next[e], 1);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

hipError_t moe_dispatch(const int* idx, const float* w, int T, int k, int E, int* gcnt,
                        int* goff, int* row_token, int* pair_row, float* row_weight,
                        int* hist, int tpc, bool counted, hipStream_t s) {
  const int npairs = T * k;
  const int nchunks = (T + tpc - 1) / tpc;
  const int chunk_pairs = tpc * k;
  if (!counted)
    hipLaunchKernelGGL(dispatch_count, dim3(nchunks), dim3(256), 0, s, idx, npairs, E, nchunks,
                       chunk_pairs, hist);
  hipLaunchKernelGGL(dispatch_scan, dim3(E), dim3(256), 0, s, hist, nchunks, gcnt);
  hipLaunchKernelGGL(dispatch_write, dim3(nchunks), dim3(64 * DW_WAVES), 0, s, idx, w, npairs,
                     k, E,
                     nchunks, chunk_pairs, hist, gcnt, goff, row_token, pair_row, row_weight);
  return hipGetLastError();
}

}  // namespace blk
