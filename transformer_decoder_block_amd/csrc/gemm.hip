// NT GEMM on gfx950 matrix cores with the block's fused epilogues.
//
//   C[M, N] = A[M, K] . B[N, K]^T        (both operands K-contiguous, the
//                                         Linear layout [out, in] for B)
//
// One workgroup of WGM x WGN wavefronts (4: one per SIMD, or 8: two per
// SIMD) computes a BM x BN tile; each wave owns a (BM/WGM) x (BN/WGN)
// sub-tile made of 32x32 MFMA blocks.  K is consumed in
// tiles of 128 bytes per row (64 bf16 / 32 fp32; the router's narrow tile
// takes 512).  Operand tiles go from
// global memory straight into LDS (buffer_load ... lds: no VGPR staging),
// double-buffered: the loads of K-tile k+1 are issued right after the
// barrier that opens K-tile k and land while its MFMAs run, so one barrier
// per K-tile suffices.  Raw buffer loads return zeros at or past the
// resource size, which covers ragged M/N edges and the K tail.
//
// LDS layout: row r of a tile is 128 contiguous bytes = eight 16-byte
// chunks; chunk c is stored in slot c ^ ((r >> 1) & 7) (rows of 256 bytes
// or more: c ^ (r & 15)).  A direct-to-LDS
// load writes 64 lanes x 16 bytes contiguously, so each lane fetches the
// global chunk that belongs in its slot.  With 64 four-byte banks, a
// 16-byte read by 16 lanes of 16 consecutive rows at one k touches every
// bank once: even rows fill banks 0-31, odd rows 32-63, and within a
// parity the 8 rows sit in 8 different slots.
//
// bf16: v_mfma_f32_16x16x32_bf16 (lane l holds row l%16, k 8*(l/16)..+7 of
//       a 32-wide k-step; 64 lanes x 16 bytes = one fragment).
// f32 : v_mfma_f32_32x32x2f32 with the K order inside a 32-wide K tile
//       permuted so every lane reads 4 consecutive floats per LDS access
//       (half h of the wave takes k = 16h + 4g + s at step (g, s)); A and B
//       use the same permutation, so the sum is unchanged.
// The B fragment is the MFMA's first operand, so each accumulator block
// holds C^T: a lane owns "quads", four consecutive columns of one row of C,
// stored with one vector write (16x16 blocks: one quad per lane, row l%16,
// columns 4*(l/16)..+3; 32x32 blocks: four quads, row l%32, columns
// 8*q + 4*(l/32)..+3).
// Fragments of k-step s+1 are read from LDS while the MFMAs of step s run.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace blk {

// Tile shape: BM x BN outputs per workgroup of WGM x WGN waves (4: one per
// SIMD; 8: two per SIMD), KB bytes of K per row per pipeline stage, NS
// stages in LDS (NS - 1 in flight).
template <typename T, int BM_, int BN_, int WGM_, int WGN_, int KB_, int NS_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int KB = KB_, NS = NS_;
  static constexpr int BK = KB / sizeof(T);   // K elements per stage
  static constexpr int CH = 16 / sizeof(T);   // elements per 16-byte chunk
  static constexpr int CPR = KB / 16;         // chunks per tile row
  static constexpr int RPI = 1024 / KB;       // rows per direct-load instruction
  static constexpr int LD = BK;               // LDS row (KB bytes, swizzled)
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int NW = WGM * WGN;        // waves per workgroup
  static constexpr int NT = 64 * NW;          // threads per workgroup
  static constexpr int WPE = NW / 4;          // waves per SIMD
  static constexpr int AL = BM / RPI / NW;    // A load instructions per wave
  static constexpr int BL = BN / RPI / NW;    // B load instructions per wave
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(FM >= 1 && FN >= 1, "wave tile >= 32x32");
  static_assert(AL >= 1 && BL >= 1, "every wave loads");
};

// Blocks are dealt to the 8 XCDs round-robin (block i runs on XCD i % 8).
// Renumber them so that each XCD receives one contiguous run of tile ids,
// which the grouped ordering below turns into a compact patch of C: the
// A and B panels of that patch are then shared through the XCD's own L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int nblk) {
  const int per = nblk / 8, rem = nblk % 8;
  const int xcd = bid % 8, local = bid / 8;
  return (xcd < rem) ? xcd * (per + 1) + local
                     : rem * (per + 1) + (xcd - rem) * per + local;
}

// Tile id -> (mt, nt): GROUP_M rows of tiles are walked column by column,
// so the tiles in flight share their A and B panels.
__device__ __forceinline__ void tile_coords(int id, int num_m, int num_n, int& mt, int& nt) {
  constexpr int GROUP_M = 8;
  const int width = GROUP_M * num_n;
  const int first_m = (id / width) * GROUP_M;
  const int gsz = min(num_m - first_m, GROUP_M);
  mt = first_m + (id % width) % gsz;
  nt = (id % width) / gsz;
}

// One direct-to-LDS load per lane: 16 bytes at byte offset voff of the
// buffer land at lds + 16 * lane (lds is the wave's uniform base).
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t r, const void* lds,
                                              uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Address (in elements) of 16-byte chunk c of tile row r, rows of KB bytes.
// 64 four-byte banks span 256 bytes = 256/KB rows; the slot of chunk c is
// c xor'ed with the row's index among the rows that share banks.
// Rows of 256 bytes or more span every bank: the slot is then c xor'ed with
// the row's low four bits (16 rows, 16 distinct 16-byte slots).
template <int KB>
__device__ __forceinline__ int swz_key(int r) {
  constexpr int CPR = KB / 16, RPB = KB >= 256 ? 1 : 256 / KB;
  constexpr int MASK = (CPR < 16 ? CPR : 16) - 1;
  return (r / RPB) & MASK;
}
template <typename T, int KB>
__device__ __forceinline__ int swz(int r, int c) {
  constexpr int CH = 16 / sizeof(T), CPR = KB / 16;
  return r * (CPR * CH) + ((c ^ swz_key<KB>(r)) * CH);
}

// Accumulator layout of a wave's WM x WN sub-tile: AM x AN blocks, QPB
// quads per lane per block; quad q of block (i, j) is row row(lane, i),
// columns col(lane, j, q) .. +3 of the sub-tile, values acc[i][j][4q .. 4q+3].
template <typename T, int WM, int WN>
struct AccL;
template <int WM, int WN>
struct AccL<bf16, WM, WN> {
  static constexpr int BR = 16, AM = WM / 16, AN = WN / 16, QPB = 1;
  typedef f32x4 Blk;
  static __device__ __forceinline__ int row(int lane, int i) { return 16 * i + (lane & 15); }
  static __device__ __forceinline__ int col(int lane, int j, int q) {
    return 16 * j + 4 * (lane >> 4);
  }
  // sum over the four lanes that hold the columns of one row
  static __device__ __forceinline__ float row_sum(float v) {
    v += __shfl_xor(v, 16, 64);
    return v + __shfl_xor(v, 32, 64);
  }
};
template <int WM, int WN>
struct AccL<float, WM, WN> {
  static constexpr int BR = 32, AM = WM / 32, AN = WN / 32, QPB = 4;
  typedef f32x16 Blk;
  static __device__ __forceinline__ int row(int lane, int i) { return 32 * i + (lane & 31); }
  static __device__ __forceinline__ int col(int lane, int j, int q) {
    return 32 * j + 8 * q + 4 * (lane >> 5);
  }
  static __device__ __forceinline__ float row_sum(float v) { return v + __shfl_xor(v, 32, 64); }
};

template <typename T, int AM, int AN, int KB>
struct Frags;
template <int AM, int AN, int KB>
struct Frags<bf16, AM, AN, KB> {
  static constexpr int STEPS = KB / 64;  // 32-wide k-steps per stage
  typedef f32x4 Blk;
  bf16x8 a[AM], b[AN];
  // k-step ks: lane quarter q (= lane / 16) reads chunk 4 ks + q of its row.
  // Read order follows the MFMA order (row block i outer, column block j
  // inner): b[0], a[0], the other b, then the other a, so the first MFMA
  // waits for two reads rather than for all of a.
  __device__ __forceinline__ void load(const bf16* As, const bf16* Bs, int arow0,
                                       int brow0, int lane, int ks) {
    const int r = lane & 15, c = 4 * ks + (lane >> 4);
    b[0] = *reinterpret_cast<const bf16x8*>(Bs + swz<bf16, KB>(brow0 + r, c));
    a[0] = *reinterpret_cast<const bf16x8*>(As + swz<bf16, KB>(arow0 + r, c));
#pragma unroll
    for (int j = 1; j < AN; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(Bs + swz<bf16, KB>(brow0 + j * 16 + r, c));
#pragma unroll
    for (int i = 1; i < AM; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(As + swz<bf16, KB>(arow0 + i * 16 + r, c));
  }
  __device__ __forceinline__ void mma(f32x4 (&acc)[AM][AN]) const {
#pragma unroll
    for (int i = 0; i < AM; ++i)
#pragma unroll
      for (int j = 0; j < AN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
  }
};
template <int FM, int FN, int KB>
struct Frags<float, FM, FN, KB> {
  static constexpr int STEPS = KB / 32;  // groups of 4 k per lane half
  typedef f32x16 Blk;
  f32x4 a[FM], b[FN];
  // group g: lane half hf reads chunk hf * STEPS + g
  __device__ __forceinline__ void load(const float* As, const float* Bs, int arow0,
                                       int brow0, int lane, int g) {
    const int r = lane & 31, c = STEPS * (lane >> 5) + g;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      a[i] = *reinterpret_cast<const f32x4*>(As + swz<float, KB>(arow0 + i * 32 + r, c));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      b[j] = *reinterpret_cast<const f32x4*>(Bs + swz<float, KB>(brow0 + j * 32 + r, c));
  }
  __device__ __forceinline__ void mma(f32x16 (&acc)[FM][FN]) const {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(b[j][s], a[i][s], acc[i][j], 0, 0, 0);
  }
};

// All MFMAs of one stage, the next step's fragments read while the current
// step's MFMAs run.
template <typename T, int FM, int FN, int KB>
__device__ __forceinline__ void compute_tile(typename Frags<T, FM, FN, KB>::Blk (&acc)[FM][FN],
                                             const T* As, const T* Bs, int arow0, int brow0,
                                             int lane) {
  using F = Frags<T, FM, FN, KB>;
  constexpr int NSTEP = F::STEPS;
  F f[2];
  f[0].load(As, Bs, arow0, brow0, lane, 0);
#pragma unroll
  for (int ks = 0; ks < NSTEP; ++ks) {
    if (ks + 1 < NSTEP) f[(ks + 1) & 1].load(As, Bs, arow0, brow0, lane, ks + 1);
    f[ks & 1].mma(acc);
  }
  // Schedule: the first step's fragment reads, then each step's MFMAs with
  // the next step's fragment reads spread between them (without this the
  // scheduler sinks every read next to its first use and the LDS latency
  // shows up before each group of MFMAs).
  constexpr int NMMA = FM * FN * (sizeof(T) == 2 ? 1 : 4);  // MFMAs per step
  constexpr int NRD = FM + FN;                             // reads per step
  __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
#pragma unroll
  for (int ks = 0; ks < NSTEP; ++ks) {
    if (ks + 1 < NSTEP) {
#pragma unroll
      for (int r = 0; r < NRD; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, NMMA / NRD > 0 ? NMMA / NRD : 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if (NMMA > NRD * (NMMA / NRD))
        __builtin_amdgcn_sched_group_barrier(0x008, NMMA - NRD * (NMMA / NRD), 0);
    } else {
      __builtin_amdgcn_sched_group_barrier(0x008, NMMA, 0);
    }
  }
}

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt left alone), n < 64
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// ------------------------------------------------------------ epilogues

__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

__device__ __forceinline__ float xielu_f(float z, float ap, float an, float beta,
                                         float eps) {
  if (z > 0.0f) return ap * z * z + beta * z;
  return an * (expm1f(fminf(z, eps)) - z) + beta * z;
}

// Make this wave's LDS writes visible to its own later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Four consecutive elements of T <-> floats (8-byte bf16, 16-byte fp32).
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  uint2 w;
  w.x = pack2_bf16(a, b);
  w.y = pack2_bf16(c, d);
  *reinterpret_cast<uint2*>(p) = w;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <typename T>
__device__ __forceinline__ void load4(const T* p, float* v);
template <>
__device__ __forceinline__ void load4<bf16>(const bf16* p, float* v) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(w.x << 16);
  v[1] = __uint_as_float(w.x & 0xffff0000u);
  v[2] = __uint_as_float(w.y << 16);
  v[3] = __uint_as_float(w.y & 0xffff0000u);
}
template <>
__device__ __forceinline__ void load4<float>(const float* p, float* v) {
  const float4 w = *reinterpret_cast<const float4*>(p);
  v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
}

// One quad (four consecutive columns col..col+3 of one output row, values
// v) through the elementwise epilogue EPI; orow is the row's element offset
// in the output(s).  Columns at or past N are not written.
template <typename T, int EPI>
__device__ __forceinline__ void epi_quad(const GemmParams& p, int64_t orow, int col,
                                         const float (&v)[4], float wrow) {
  const int64_t o = orow + col;
  const bool full = col + 3 < p.N;
  if constexpr (EPI == EPI_STORE) {
    if (full) {
      if (p.out_f32) store4((float*)p.out + o, v[0], v[1], v[2], v[3]);
      else store4((T*)p.out + o, v[0], v[1], v[2], v[3]);
    } else {
      for (int e = 0; e < 4 && col + e < p.N; ++e) {
        if (p.out_f32) ((float*)p.out)[o + e] = v[e];
        else ((T*)p.out)[o + e] = from_f32<T>(v[e]);
      }
    }
  } else if constexpr (EPI == EPI_RESID) {
    float res[4], sum[4];
    if (full) {
      if (p.resid_f32) load4((const float*)p.resid + o, res);
      else load4((const T*)p.resid + o, res);
    } else {
      for (int e = 0; e < 4; ++e)
        res[e] = (col + e < p.N) ? (p.resid_f32 ? ((const float*)p.resid)[o + e]
                                                : to_f32(((const T*)p.resid)[o + e]))
                                 : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sum[e] = res[e] + v[e];
    if (full) {
      if (p.out_f32p) store4(p.out_f32p + o, sum[0], sum[1], sum[2], sum[3]);
      if (p.out_model) store4((T*)p.out_model + o, sum[0], sum[1], sum[2], sum[3]);
      if (p.out_raw) store4(p.out_raw + o, v[0], v[1], v[2], v[3]);
    } else {
      for (int e = 0; e < 4 && col + e < p.N; ++e) {
        if (p.out_f32p) p.out_f32p[o + e] = sum[e];
        if (p.out_model) ((T*)p.out_model)[o + e] = from_f32<T>(sum[e]);
        if (p.out_raw) p.out_raw[o + e] = v[e];
      }
    }
  } else {
    float w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (EPI == EPI_RELU2) {
        const float rl = fmaxf(v[e], 0.f);
        w[e] = rl * rl;
      } else if constexpr (EPI == EPI_XIELU) {
        w[e] = xielu_f(v[e], p.xa_p, p.xa_n, p.xbeta, p.xeps);
      } else if constexpr (EPI == EPI_SILU) {
        w[e] = silu_f(v[e]);
      } else {  // EPI_MOE_DOWN
        w[e] = wrow * v[e];
      }
    }
    if (full) {
      store4((T*)p.out + o, w[0], w[1], w[2], w[3]);
    } else {
      for (int e = 0; e < 4 && col + e < p.N; ++e) ((T*)p.out)[o + e] = from_f32<T>(w[e]);
    }
  }
}

// Residual epilogue of a wave sub-tile whose columns all exist: the
// residual quads of row block i + 1 are loaded before the sums of block i
// are stored, so the loads of a block overlap the stores of the one before
// (every residual element is loaded before the same element is stored,
// which also holds when the output is the residual buffer).
template <typename T, typename R, class L, class ACC>
__device__ __forceinline__ void resid_tile(const GemmParams& p, const ACC& acc,
                                           const int64_t (&orow)[L::AM],
                                           const bool (&rok)[L::AM], int col0, int lane) {
  constexpr int AM = L::AM, NQ = L::AN * L::QPB;
  float res[2][NQ][4];
  auto load_blk = [&](int i, float (&r)[NQ][4]) {
#pragma unroll
    for (int j = 0; j < L::AN; ++j)
#pragma unroll
      for (int q = 0; q < L::QPB; ++q)
        load4((const R*)p.resid + orow[i] + col0 + L::col(lane, j, q), r[j * L::QPB + q]);
  };
  load_blk(0, res[0]);
#pragma unroll
  for (int i = 0; i < AM; ++i) {
    if (i + 1 < AM) load_blk(i + 1, res[(i + 1) & 1]);
    if (!rok[i]) continue;
#pragma unroll
    for (int j = 0; j < L::AN; ++j)
#pragma unroll
      for (int q = 0; q < L::QPB; ++q) {
        const int64_t o = orow[i] + col0 + L::col(lane, j, q);
        const float* r = res[i & 1][j * L::QPB + q];
        float sum[4], v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[i][j][4 * q + e];
          sum[e] = r[e] + v[e];
        }
        if (p.out_f32p) store4(p.out_f32p + o, sum[0], sum[1], sum[2], sum[3]);
        if (p.out_model) store4((T*)p.out_model + o, sum[0], sum[1], sum[2], sum[3]);
        if (p.out_raw) store4(p.out_raw + o, v[0], v[1], v[2], v[3]);
      }
  }
}

// SwiGLU quad: neurons col..col+3 of one row from their gate and up values.
template <typename T>
__device__ __forceinline__ void swiglu_quad(const GemmParams& p, T* orow, int col,
                                            const float (&g)[4], const float (&u)[4]) {
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = silu_f(g[e]) * u[e];
  if (col + 3 < p.N) {
    store4(orow + col, v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (col + e < p.N) orow[col + e] = from_f32<T>(v[e]);
  }
}

// Q/K/V(/gate) epilogue.  A wave owns WM rows (tokens) x WN columns; its
// columns hold whole heads.  A lane holds quads (four consecutive columns)
// of its rows; per head: optional RMSNorm over the head (sum of squares in
// the lane, then across the lanes that share the row), rotary on the pairs
// (d, d + HD/2), which sit in the same lane and register, then the head is
// staged through this wave's slice of LDS so that the global stores are
// 16 bytes and coalesced: q/k rows [token][d] go to [b, head, s, :], v goes
// transposed to V^T [b, head, d, s] (keys contiguous, the layout the
// attention kernel's P.V product reads).
template <typename T, int HD, int WM, int WN, typename ACC>
__device__ __forceinline__ void qkv_epilogue(ACC& acc, const GemmParams& p, int row0,
                                             int col0, int lane, T* lds) {
  using L = AccL<T, WM, WN>;
  constexpr int AM = L::AM, AN = L::AN, QPB = L::QPB;
  constexpr int HB = HD / L::BR;    // accumulator blocks per head
  constexpr int CH = 16 / sizeof(T);
  constexpr int QLD = HD + CH;      // staged q/k row   [WM][QLD]
  constexpr int VLD = WM + CH;      // staged v^T row   [HD][VLD]
  static_assert(AN % HB == 0, "wave columns must hold whole heads");
  const int Sp = (p.S + 63) & ~63;  // V^T rows are padded to 64 keys
#pragma unroll
  for (int hh = 0; hh < AN / HB; ++hh) {
    const int c0 = col0 + hh * HD;
    if (c0 >= p.N) continue;
    int seg = 0;
    while (seg < p.nseg - 1 && c0 >= p.seg_end[seg]) ++seg;
    const int start = seg ? p.seg_end[seg - 1] : 0;
    if (seg == 3) {  // gate columns: sigmoid, float32 [M, G]
#pragma unroll
      for (int i = 0; i < AM; ++i) {
        const int row = row0 + L::row(lane, i);
        if (row >= p.M) continue;
#pragma unroll
        for (int jb = 0; jb < HB; ++jb)
#pragma unroll
          for (int q = 0; q < QPB; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int col = c0 + L::col(lane, jb, q) + e;
              if (col < p.N)
                p.gate[(int64_t)row * p.G + (col - start)] =
                    1.0f / (1.0f + expf(-acc[i][hh * HB + jb][4 * q + e]));
            }
      }
      continue;
    }
    const int head = (c0 - start) / HD;
    if (seg < 2) {
      // Per row: optional RMSNorm over the head, then rotary on the pairs
      // (d, d + HD/2), each output computed from acc and written straight
      // into the staging rows [row][d] (acc itself is never modified: an
      // in-place update under a condition makes the compiler keep a second
      // copy of the accumulators).  Where norm or rotary is off, the value
      // is passed through unchanged.
      const bool do_norm = p.qk_norm != 0, do_rope = p.use_rope != 0;
      const T* gw = (const T*)(seg == 0 ? p.q_norm_w : p.k_norm_w);
      // the norm gains of the lane's columns (the same on every row), read
      // once per head
      float glo[HB / 2][QPB][4], ghi[HB / 2][QPB][4];
#pragma unroll
      for (int jb = 0; jb < HB / 2; ++jb)
#pragma unroll
        for (int q = 0; q < QPB; ++q) {
          const int d = L::col(lane, jb, q);
          if (do_norm) {
            load4(gw + d, glo[jb][q]);
            load4(gw + d + HD / 2, ghi[jb][q]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) glo[jb][q][e] = ghi[jb][q][e] = 1.f;
          }
        }
      // Rotary factors: when the wave's WM rows are consecutive positions of
      // one sequence, row block i + 1 sits 16 positions after row block i,
      // so its factors follow from the angle-addition rule with the factors
      // of 16 positions (table row 16, the same for every row block): one
      // table read for the first row block instead of one dependent read
      // per row block.
      const int pos0 = row0 % p.S;
      const bool rec = do_rope && (row0 + WM <= p.M) && (pos0 + WM <= p.S) && (p.S > 16);
      float c[HB / 2][QPB][4], sn[HB / 2][QPB][4];
#pragma unroll
      for (int i = 0; i < AM; ++i) {
        float inv = 1.0f;
        if (do_norm) {
          float ss = 0.f;
#pragma unroll
          for (int jb = 0; jb < HB; ++jb)
#pragma unroll
            for (int r = 0; r < 4 * QPB; ++r) {
              const float v = acc[i][hh * HB + jb][r];
              ss += v * v;
            }
          ss = L::row_sum(ss);
          inv = 1.0f / sqrtf(ss * (1.0f / HD) + p.eps);
        }
        const int lr = L::row(lane, i);
        const int row = row0 + lr;
        const int pos = (row < p.M) ? row % p.S : 0;
        const float* cr = p.rope_cos + (int64_t)pos * (HD / 2);
        const float* sr = p.rope_sin + (int64_t)pos * (HD / 2);
        T* srow = lds + lr * QLD;
        if (rec && i > 0) {
          // (c, s) <- (c c16 - s s16, s c16 + c s16)
          const float* c16 = p.rope_cos + 16 * (HD / 2);
          const float* s16 = p.rope_sin + 16 * (HD / 2);
#pragma unroll
          for (int jb = 0; jb < HB / 2; ++jb)
#pragma unroll
            for (int q = 0; q < QPB; ++q) {
              const int d = L::col(lane, jb, q);
              float cd[4], sd[4];
              load4(c16 + d, cd);
              load4(s16 + d, sd);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float cn = c[jb][q][e] * cd[e] - sn[jb][q][e] * sd[e];
                sn[jb][q][e] = sn[jb][q][e] * cd[e] + c[jb][q][e] * sd[e];
                c[jb][q][e] = cn;
              }
              // one group's step factors live at a time
              __builtin_amdgcn_sched_barrier(0);
            }
        } else {
          // the row's rotary factors for all of the lane's columns, loaded
          // together so their latencies overlap
#pragma unroll
          for (int jb = 0; jb < HB / 2; ++jb)
#pragma unroll
            for (int q = 0; q < QPB; ++q) {
              const int d = L::col(lane, jb, q);  // low member of the pairs
              if (do_rope) {
                load4(cr + d, c[jb][q]);
                load4(sr + d, sn[jb][q]);
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) { c[jb][q][e] = 1.f; sn[jb][q][e] = 0.f; }
              }
            }
        }
#pragma unroll
        for (int jb = 0; jb < HB / 2; ++jb)
#pragma unroll
          for (int q = 0; q < QPB; ++q) {
            const int d = L::col(lane, jb, q);
            float olo[4], ohi[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float lo = glo[jb][q][e] * (acc[i][hh * HB + jb][4 * q + e] * inv);
              const float hi = ghi[jb][q][e] * (acc[i][hh * HB + jb + HB / 2][4 * q + e] * inv);
              olo[e] = do_rope ? lo * c[jb][q][e] - hi * sn[jb][q][e] : lo;
              ohi[e] = do_rope ? hi * c[jb][q][e] + lo * sn[jb][q][e] : hi;
            }
            store4(srow + d, olo[0], olo[1], olo[2], olo[3]);
            store4(srow + d + HD / 2, ohi[0], ohi[1], ohi[2], ohi[3]);
          }
        // keep the next row block's table loads from being hoisted here
        // (their registers would be live together with these)
        __builtin_amdgcn_sched_barrier(0);
      }
      wave_lds_sync();
      T* base = (T*)(seg == 0 ? p.q : p.k);
      const int nheads = seg == 0 ? p.nh : p.nkv;
      constexpr int CPRW = HD / CH;  // 16-byte chunks per row
#pragma unroll 4
      for (int it = 0; it < WM * CPRW / 64; ++it) {
        const int idx = it * 64 + lane;
        const int rr = idx / CPRW, ch = idx % CPRW;
        const int row = row0 + rr;
        if (row < p.M) {
          const int b = row / p.S, sp = row % p.S;
          T* dst = base + (((int64_t)b * nheads + head) * p.S + sp) * HD + ch * CH;
          *reinterpret_cast<uint4*>(dst) =
              *reinterpret_cast<const uint4*>(lds + rr * QLD + ch * CH);
        }
      }
    } else {
      // stage transposed [d][row], then store key-contiguous runs of V^T
#pragma unroll
      for (int i = 0; i < AM; ++i)
#pragma unroll
        for (int jb = 0; jb < HB; ++jb)
#pragma unroll
          for (int q = 0; q < QPB; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int d = L::col(lane, jb, q) + e;
              lds[d * VLD + L::row(lane, i)] = from_f32<T>(acc[i][hh * HB + jb][4 * q + e]);
            }
      wave_lds_sync();
      // bf16: within each aligned group of 16 keys the row holds keys
      // 0-3, 8-11, 4-7, 12-15 (position and key differ by a swap of bits
      // 2 and 3), the order in which the attention kernel's P.V step
      // consumes them; float rows keep the natural order.
      constexpr bool PERM = sizeof(T) == 2;
      T* base = (T*)p.vt;
      constexpr int RCH = WM / CH;  // chunks of CH positions per d
      const bool s_aligned = PERM ? (p.S % 16) == 0 : (p.S % CH) == 0;
#pragma unroll 4
      for (int it = 0; it < HD * RCH / 64; ++it) {
        const int idx = it * 64 + lane;
        const int d = idx / RCH, rc = idx % RCH;
        const int r0 = row0 + rc * CH;
        const T* src = lds + d * VLD + rc * CH;
        const int b0 = r0 / p.S;
        if (s_aligned && r0 + CH <= p.M && (r0 + CH - 1) / p.S == b0) {
          T* dst = base + (((int64_t)b0 * p.nkv + head) * HD + d) * Sp + (r0 % p.S);
          if constexpr (PERM) {
            // positions rc*8 .. +7 hold keys (local) rc*8 + {0..3, 8..11}
            // for even rc and rc*8 + {-4..-1, 4..7} for odd rc
            const int odd = rc & 1;
            const uint2 lo = *reinterpret_cast<const uint2*>(src - 4 * odd);
            const uint2 hi = *reinterpret_cast<const uint2*>(src + 8 - 4 * odd);
            *reinterpret_cast<uint4*>(dst) = make_uint4(lo.x, lo.y, hi.x, hi.y);
          } else {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
          }
        } else {
          for (int e = 0; e < CH; ++e) {
            const int row = r0 + e;
            if (row >= p.M) break;
            const int b = row / p.S, sk = row % p.S;
            const int pos = PERM ? ((sk & ~12) | ((sk & 4) << 1) | ((sk & 8) >> 1)) : sk;
            base[(((int64_t)b * p.nkv + head) * HD + d) * Sp + pos] = src[e];
          }
        }
      }
    }
    wave_lds_sync();  // the next head reuses this wave's LDS slice
  }
}

// Register epilogue of one tile (every EPI but the q/k/v one): each lane
// stores its quads (four consecutive columns) of the rows it holds.
template <typename T, class TL, int EPI, class ACC>
__device__ __forceinline__ void tile_epilogue(const GemmParams& p, ACC& acc, int mt, int nt,
                                              int row_begin, int row_count, int wm, int wn,
                                              int lane) {
  constexpr int BM = TL::BM, BN = TL::BN, WM = TL::WM, WN = TL::WN;
  constexpr bool PAIRED = (EPI == EPI_SWIGLU);
  using L = AccL<T, WM, WN>;
  constexpr int AM = L::AM, AN = L::AN, QPB = L::QPB;
  const int lrow0 = mt * BM + wm * WM;  // tile-local (group-local) row base
  if constexpr (PAIRED) {
    // gate columns are the first half of the wave's columns, up the second
    const int ncol0 = nt * (BN / 2) + wn * (WN / 2);
#pragma unroll
    for (int i = 0; i < AM; ++i) {
      const int lr = lrow0 + L::row(lane, i);
      if (lr >= row_count) continue;
      T* orow = (T*)p.out + (int64_t)(row_begin + lr) * p.ldo;
#pragma unroll
      for (int j = 0; j < AN / 2; ++j)
#pragma unroll
        for (int q = 0; q < QPB; ++q) {
          float g[4], u[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            g[e] = acc[i][j][4 * q + e];
            u[e] = acc[i][j + AN / 2][4 * q + e];
          }
          swiglu_quad<T>(p, orow, ncol0 + L::col(lane, j, q), g, u);
        }
    }
    return;
  } else {
    // The lane's rows: output offsets (and for the MoE down projection the
    // rows' slot weights) are all computed before the first store, so a
    // load's latency is paid once.  Rows past the tile's end are clamped
    // to a valid row for the loads and never stored.
    int64_t orow[AM];
    float wrow[AM];
    bool rok[AM];
#pragma unroll
    for (int i = 0; i < AM; ++i) {
      const int lr = lrow0 + L::row(lane, i);
      rok[i] = lr < row_count;
      const int64_t row = row_begin + (rok[i] ? lr : 0);
      orow[i] = row * p.ldo;
      wrow[i] = 1.0f;
      if constexpr (EPI == EPI_MOE_DOWN) wrow[i] = p.row_weight[row];
    }
    const int col0 = nt * BN + wn * WN;
    if (col0 + WN <= p.N) {
      // every column of the wave's sub-tile exists: no per-quad tests
      if constexpr (EPI == EPI_RESID) {
        if (p.resid_f32)
          resid_tile<T, float, L>(p, acc, orow, rok, col0, lane);
        else
          resid_tile<T, T, L>(p, acc, orow, rok, col0, lane);
      } else {
#pragma unroll
        for (int i = 0; i < AM; ++i) {
          if (!rok[i]) continue;
#pragma unroll
          for (int j = 0; j < AN; ++j)
#pragma unroll
            for (int q = 0; q < QPB; ++q) {
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
              epi_quad<T, EPI>(p, orow[i], col0 + L::col(lane, j, q), v, wrow[i]);
            }
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < AM; ++i) {
      if (!rok[i]) continue;
#pragma unroll
      for (int j = 0; j < AN; ++j)
#pragma unroll
        for (int q = 0; q < QPB; ++q) {
          const int col = col0 + L::col(lane, j, q);
          if (col >= p.N) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          epi_quad<T, EPI>(p, orow[i], col, v, wrow[i]);
        }
    }
  }
}

// Epilogue stores through LDS.  In the accumulator layout one store
// instruction writes sixteen separate pieces of 32 bytes (bf16) or 64 bytes
// (float32), four lanes per row, and the memory pipeline drains those far
// more slowly than whole lines: per-tile timestamps put the epilogue at
// 9-14 us of a 27-103 us tile.  Here each wave writes its 128 x 64
// sub-tile, already in the output type SE, into an 8 KiB slice of the stage
// buffer that the tile's last k-stage freed, 8 KiB of rows per pass; then it
// reads the slice back by rows, so that every global store covers whole
// row segments of 128 or 256 bytes.  The rows' 16-byte chunks are
// XOR-swizzled (by (r / 2) mod 8 for 128-byte rows, r mod 16 for 256-byte
// rows), which keeps the accumulator writes and the row reads free of bank
// conflicts.  The slice is the wave's own and LDS operations of one wave
// complete in order, so the passes need no barrier.
//   pre(i):          called before row block i is written (loads for it)
//   val(i, j, v):    the four values of quad (i, j) to stage
//   emit(rr, ch, d): the 16 bytes d of chunk ch of sub-tile row rr
template <typename SE, int AM, int AN, class PRE, class VAL, class EMIT>
__device__ __forceinline__ void stage_rows(char* stage, int lane, PRE&& pre, VAL&& val,
                                           EMIT&& emit) {
  constexpr int ES = sizeof(SE), RB = 64 * ES, CPR = RB / 16, RP = 8192 / RB;
  constexpr int PB = RP / 16, RPI = 64 / CPR, NRD = RP / RPI;
  static_assert(AN == 4 && AM % PB == 0, "64-column wave tiles");
  auto sw = [](int r) { return ES == 2 ? (r >> 1) & 7 : r & 15; };
  const int l15 = lane & 15;
  int woff[AN];
#pragma unroll
  for (int j = 0; j < AN; ++j) {
    const int byte = (16 * j + 4 * (lane >> 4)) * ES;
    woff[j] = l15 * RB + (((byte >> 4) ^ sw(l15)) << 4) + (byte & 15);
  }
  const int rsub = lane / CPR, ch = lane % CPR;
#pragma unroll
  for (int h = 0; h < AM / PB; ++h) {
#pragma unroll
    for (int ib = 0; ib < PB; ++ib) {
      const int i = h * PB + ib;
      pre(i);
#pragma unroll
      for (int j = 0; j < AN; ++j) {
        float v[4];
        val(i, j, v);
        char* dst = stage + ib * 16 * RB + woff[j];
        if constexpr (ES == 2) {
          uint2 w;
          w.x = pack2_bf16(v[0], v[1]);
          w.y = pack2_bf16(v[2], v[3]);
          *reinterpret_cast<uint2*>(dst) = w;
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NRD; ++k) {
      const int r = RPI * k + rsub;
      const uint4 d = *reinterpret_cast<const uint4*>(stage + r * RB + ((ch ^ sw(r)) << 4));
      emit(16 * PB * h + r, ch, d);
    }
  }
}

// The staged epilogue of a plain (model dtype or float32), MoE-down or
// residual tile; false when the wave's sub-tile is not one it handles
// (columns past N, an unaligned row stride, the residual's raw-product tap),
// which then takes tile_epilogue.
template <typename T, class TL, int EPI, class ACC>
__device__ __forceinline__ bool staged_epilogue(const GemmParams& p, const ACC& acc, int mt,
                                                int nt, int row_begin, int row_count, int wm,
                                                int wn, int lane_in, char* stage) {
  static_assert(sizeof(T) == 2 && TL::WN == 64, "bf16, 64-wide wave tiles");
  using L = AccL<T, TL::WM, TL::WN>;
  constexpr int AM = L::AM, AN = L::AN;
  const int col0 = nt * TL::BN + wn * TL::WN;
  if (col0 + TL::WN > p.N || (p.ldo % 8) != 0) return false;
  if (EPI == EPI_RESID && p.out_raw) return false;
  // the lane's offsets are recomputed here rather than kept live across
  // the tile loop
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  const int lrow0 = mt * TL::BM + wm * TL::WM;
  auto none = [](int) {};
  if constexpr (EPI == EPI_STORE || EPI == EPI_MOE_DOWN) {
    float wrow[AM];
#pragma unroll
    for (int i = 0; i < AM; ++i) {
      wrow[i] = 1.0f;
      if constexpr (EPI == EPI_MOE_DOWN) {
        const int lr = lrow0 + L::row(lane, i);
        wrow[i] = p.row_weight[row_begin + (lr < row_count ? lr : 0)];
      }
    }
    auto val = [&](int i, int j, float (&v)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = wrow[i] * acc[i][j][e];
    };
    if (EPI == EPI_STORE && p.out_f32) {
      float* out = (float*)p.out + (int64_t)(row_begin + lrow0) * p.ldo + col0;
      stage_rows<float, AM, AN>(stage, lane, none, val, [&](int rr, int ch, const uint4& d) {
        if (lrow0 + rr < row_count)
          *reinterpret_cast<uint4*>(out + (int64_t)rr * p.ldo + ch * 4) = d;
      });
    } else {
      T* out = (T*)p.out + (int64_t)(row_begin + lrow0) * p.ldo + col0;
      stage_rows<T, AM, AN>(stage, lane, none, val, [&](int rr, int ch, const uint4& d) {
        if (lrow0 + rr < row_count)
          *reinterpret_cast<uint4*>(out + (int64_t)rr * p.ldo + ch * 8) = d;
      });
    }
  } else if constexpr (EPI == EPI_RESID) {
    // residual quads in the accumulator layout, row block i + 1 loaded
    // while block i is staged; the sums are staged as float32
    float res[2][AN][4];
    auto load_blk = [&](int i) {
      const int lr = lrow0 + L::row(lane, i);
      const int64_t o = (int64_t)(row_begin + (lr < row_count ? lr : 0)) * p.ldo + col0;
#pragma unroll
      for (int j = 0; j < AN; ++j) {
        if (p.resid_f32) load4((const float*)p.resid + o + L::col(lane, j, 0), res[i & 1][j]);
        else load4((const T*)p.resid + o + L::col(lane, j, 0), res[i & 1][j]);
      }
    };
    load_blk(0);
    auto pre = [&](int i) {
      if (i + 1 < AM) load_blk(i + 1);
    };
    auto val = [&](int i, int j, float (&v)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = res[i & 1][j][e] + acc[i][j][e];
    };
    const int64_t obase = (int64_t)(row_begin + lrow0) * p.ldo + col0;
    stage_rows<float, AM, AN>(stage, lane, pre, val, [&](int rr, int ch, const uint4& d) {
      if (lrow0 + rr >= row_count) return;
      const int64_t o = obase + (int64_t)rr * p.ldo + ch * 4;
      if (p.out_f32p) *reinterpret_cast<uint4*>(p.out_f32p + o) = d;
      if (p.out_model)
        store4((T*)p.out_model + o, __uint_as_float(d.x), __uint_as_float(d.y),
               __uint_as_float(d.z), __uint_as_float(d.w));
    });
  }
  return true;
}

// Router epilogue (afmoe page, section 03, on the router): the tile holds
// every expert of BM tokens.  The logits are rounded to the model dtype
// (stored: the router_logits value) and kept in LDS as floats; then one
// lane per token takes the sigmoid of each rounded logit in double
// precision, rounded once to float32 (the correctly rounded float32
// sigmoid), adds the float32 selection bias, and keeps the K largest
// biased scores by insertion in expert order (ties: the lower expert
// first); the slot weights are the chosen unbiased sigmoids over their sum
// (summed in slot order) times route_scale.  The tile's expert counts go to
// the dispatch histogram.
// Four lanes per token (lanes 4t .. 4t+3 of a wave): lane `part` keeps the
// K best of experts part, part + 4, ... by insertion in expert order, then
// the four sorted lists are merged slot by slot (larger biased score first,
// the lower expert on ties).  Lane part 0 writes the token's slots and
// counts them into the tile histogram hcnt.
template <int K>
__device__ __forceinline__ void router_select(const GemmParams& p, const float* srow, int tok,
                                              bool live, int part, int* hcnt) {
  float bc[K], bs[K];
  int be[K];
#pragma unroll
  for (int j = 0; j < K; ++j) { bc[j] = -INFINITY; bs[j] = 0.f; be[j] = 0x7fffffff; }
  if (live) {
    for (int e = part; e < p.N; e += 4) {
      const double l = (double)srow[e];
      const float sg = (float)(1.0 / (1.0 + exp(-l)));
      const float c = sg + p.bias[e];
      // insert (c, e) after every kept score >= c
#pragma unroll
      for (int j = K - 1; j >= 1; --j) {
        const bool up = c > bc[j - 1];     // the entry above moves down
        const bool here = !up && c > bc[j];
        bc[j] = up ? bc[j - 1] : (here ? c : bc[j]);
        bs[j] = up ? bs[j - 1] : (here ? sg : bs[j]);
        be[j] = up ? be[j - 1] : (here ? e : be[j]);
      }
      if (c > bc[0]) { bc[0] = c; bs[0] = sg; be[0] = e; }
    }
  }
  float sel_s[K];
  int sel_e[K];
#pragma unroll
  for (int slot = 0; slot < K; ++slot) {
    float v = bc[0], sv = bs[0];
    int ev = be[0];
#pragma unroll
    for (int o = 1; o <= 2; o <<= 1) {
      const float ov = __shfl_xor(v, o, 64), os = __shfl_xor(sv, o, 64);
      const int oe = __shfl_xor(ev, o, 64);
      if (ov > v || (ov == v && oe < ev)) { v = ov; sv = os; ev = oe; }
    }
    if (be[0] == ev) {  // this lane's head was taken: the next one moves up
#pragma unroll
      for (int j = 0; j + 1 < K; ++j) { bc[j] = bc[j + 1]; bs[j] = bs[j + 1]; be[j] = be[j + 1]; }
      bc[K - 1] = -INFINITY;
      bs[K - 1] = 0.f;
      be[K - 1] = 0x7fffffff;
    }
    sel_s[slot] = sv;
    sel_e[slot] = ev;
  }
  if (!live || part != 0) return;
  float wsum = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j)
    if (j < p.top_k) wsum += sel_s[j];
#pragma unroll
  for (int j = 0; j < K; ++j)
    if (j < p.top_k) {
      p.eidx[(int64_t)tok * p.top_k + j] = sel_e[j];
      p.ew[(int64_t)tok * p.top_k + j] = sel_s[j] / wsum * p.route_scale;
      atomicAdd(&hcnt[sel_e[j]], 1);
    }
}

template <typename T, class TL, class ACC>
__device__ __forceinline__ void router_epilogue(const GemmParams& p, const ACC& acc, int mt,
                                                int wm, int wn, int lane, int tid,
                                                float* sc, int* hcnt) {
  using L = AccL<T, TL::WM, TL::WN>;
  constexpr int BM = TL::BM, SP = TL::BN + 1;
#pragma unroll
  for (int i = 0; i < L::AM; ++i) {
    const int r = wm * TL::WM + L::row(lane, i);
    const int64_t grow = (int64_t)mt * BM + r;
#pragma unroll
    for (int j = 0; j < L::AN; ++j)
#pragma unroll
      for (int q = 0; q < L::QPB; ++q) {
        const int c = wn * TL::WN + L::col(lane, j, q);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[i][j][4 * q + e];
          sc[r * SP + c + e] = to_f32(from_f32<T>(v[e]));
        }
        if (grow < p.M && c < p.N) epi_quad<T, EPI_STORE>(p, grow * p.ldo, c, v, 1.0f);
      }
  }
  for (int e = tid; e < 256; e += TL::NT) hcnt[e] = 0;
  __syncthreads();
  for (int t0 = 0; t0 < BM; t0 += TL::NT / 4) {
    const int tl = t0 + tid / 4;
    const int tok = mt * BM + tl;
    const bool live = tok < p.M;  // uniform over the token's four lanes
    if (p.top_k <= 8) router_select<8>(p, sc + tl * SP, tok, live, tid & 3, hcnt);
    else router_select<16>(p, sc + tl * SP, tok, live, tid & 3, hcnt);
  }
  __syncthreads();
  for (int e = tid; e < p.N; e += TL::NT) p.hist[(int64_t)e * p.hist_nchunks + mt] = hcnt[e];
}

// ---------------------------------------------------------------- kernel

template <typename T, class TL, int EPI, bool GROUPED, int HDQ = 0>
__global__ void __attribute__((amdgpu_flat_work_group_size(TL::NT, TL::NT),
                               amdgpu_waves_per_eu(TL::WPE, TL::WPE)))
gemm_kernel(const GemmParams p) {
  constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, CH = TL::CH,
                CPR = TL::CPR, LD = TL::LD, WM = TL::WM, WN = TL::WN,
                FM = TL::FM, FN = TL::FN, AL = TL::AL, BL = TL::BL, NS = TL::NS,
                RPI = TL::RPI, KB = TL::KB;
  constexpr int RPB = KB >= 256 ? 1 : 256 / KB;  // rows that share the 64 banks
  constexpr bool PAIRED = (EPI == EPI_SWIGLU);
  constexpr int CHT = 16 / sizeof(T);
  // q/k/v epilogue: each wave stages one head in its own LDS slice
  constexpr int SLICE = (WM * (128 + CHT) > 128 * (WM + CHT)) ? WM * (128 + CHT)
                                                               : 128 * (WM + CHT);
  constexpr int MAIN = NS * (BM + BN) * LD;
  // router epilogue: float scores [BM][BN + 1] and 256 int counts
  constexpr int RSTAGE = (BM * (BN + 1) + 256) * 4 / (int)sizeof(T);
  constexpr int SMEM0 = (EPI == EPI_QKV && TL::NW * SLICE > MAIN) ? TL::NW * SLICE
                        : (EPI == EPI_ROUTER && RSTAGE > MAIN) ? RSTAGE
                                                               : MAIN;
  // grouped: 257 ints of tile prefix sums after the operand tiles
  constexpr int SMEM = GROUPED ? SMEM0 + 257 * 4 / (int)sizeof(T) + 4 : SMEM0;
  __shared__ __attribute__((aligned(1024))) T smem[SMEM];
  auto As = [&](int b) { return smem + b * (BM * LD); };
  auto Bs = [&](int b) { return smem + NS * BM * LD + b * (BN * LD); };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
  const int n_per_tile = PAIRED ? BN / 2 : BN;
  const int nb0 = (EPI == EPI_QKV) ? p.n_base : 0;  // first output column
  const int num_n = (p.N - nb0 + n_per_tile - 1) / n_per_tile;

  // ---- which tile
  int mt, nt, row_begin = 0, row_count = p.M, group = 0;
  int split_slot = -1;  // >= 0: this block computes K part split_slot % split_parts of a split tile
  if constexpr (GROUPED) {
    // M tiles per group, exclusive prefix sums in LDS (the first wave: lane
    // j owns groups 4j .. 4j+3, at most 256 groups); the group of a tile is
    // then found by a binary search
    int* tpre = reinterpret_cast<int*>(smem + SMEM0);
    if (wave == 0) {
      int c[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = 4 * lane + q;
        c[q] = g < p.ngroups ? (p.gcnt[g] + BM - 1) / BM : 0;
        sum += c[q];
      }
      int inc = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o, 64);
        if (lane >= o) inc += v;
      }
      int ex = inc - sum;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        tpre[4 * lane + q] = ex;
        ex += c[q];
      }
      if (lane == 63) tpre[256] = inc;
    }
    __syncthreads();
    // one dimension over the real tiles (the grid is sized for the worst
    // case): consecutive ids, which the renumbering keeps on one XCD, are
    // the N tiles of one M tile, so the gathered A rows are read once and an
    // expert's weights are shared by its M tiles in that L2.  The surplus
    // workgroups are the highest block numbers, spread evenly over the XCDs.
    const int real = tpre[256] * num_n;
    if ((int)blockIdx.x >= real) return;
    const int id = xcd_contiguous(blockIdx.x, real);
    const int t = id / num_n;
    nt = id % num_n;
    int lo = 0, hi = p.ngroups;  // tpre[lo] <= t < tpre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tpre[mid] <= t) lo = mid;
      else hi = mid;
    }
    group = lo;
    mt = t - tpre[lo];
    row_begin = p.goff[lo];
    row_count = p.gcnt[lo];
  } else {
    const int num_m = (p.M + BM - 1) / BM;
    // blocks [0, F) are whole tiles; with a K split, blocks F + u are K
    // part (u % split_parts) of tile F + u / split_parts (dispatched last)
    const int F = num_m * num_n - p.split_tiles;
    int id;
    if (p.split_tiles > 0 && (int)blockIdx.x >= F) {
      const int u = blockIdx.x - F;
      id = F + u / p.split_parts;
      split_slot = u;
    } else {
      id = xcd_contiguous(blockIdx.x, p.split_tiles > 0 ? F : gridDim.x);
    }
    tile_coords(id, num_m, num_n, mt, nt);
  }

  // ---- direct-to-LDS loads.  Load instruction i of wave w fills tile rows
  // [RPI (4 i + w), +RPI): lane L writes slot L % CPR of row
  // RPI (4i+w) + L / CPR and so fetches the global chunk the swizzle puts
  // there.  A chunk at or past the resource size reads as zeros (rows past
  // M/N, the K tail).
  const int lrowi = lane / CPR;
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, p.a_bytes, 0x00020000);
  uint32_t a_off[AL];
  int a_k[AL];  // first k of the chunk this lane fetches
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int lrow = (TL::NW * i + wave) * RPI + lrowi;
    const int kch = (lane % CPR) ^ swz_key<KB>(lrow);
    a_k[i] = kch * CH;
    const int r = mt * BM + lrow;
    int src = row_begin + (r < row_count ? r : 0);
    if (p.a_gather) src = p.a_gather[src];
    a_off[i] = (r < row_count)
                   ? (uint32_t)(((int64_t)src * p.lda + kch * CH) * sizeof(T))
                   : p.a_bytes;
  }
  // B: the segment (QKV: q/k/v/gate; SWIGLU: gate/up) of one load is the
  // same for the whole wave, since segments are 32-row aligned.
  const int64_t gofs = GROUPED ? (int64_t)group * p.b_group_stride : 0;
  __amdgpu_buffer_rsrc_t rB[BL];
  uint32_t b_off[BL];
  int b_k[BL];
#pragma unroll
  for (int i = 0; i < BL; ++i) {
    const int lbase = (TL::NW * i + wave) * RPI;
    const int lrow = lbase + lrowi;
    const int kch = (lane % CPR) ^ swz_key<KB>(lrow);
    b_k[i] = kch * CH;
    int seg, n;
    bool ok;
    if constexpr (PAIRED) {
      constexpr int half = WN / 2;
      seg = (lbase % WN) / half;
      n = nt * (BN / 2) + (lbase / WN) * half + (lrow % WN) % half;
      ok = n < p.N;
    } else {
      const int nb = nb0 + nt * BN + lbase;
      seg = 0;
      while (seg < p.nseg - 1 && nb >= p.seg_end[seg]) ++seg;
      n = nb0 + nt * BN + lrow;
      ok = n < p.N;
      n -= seg ? p.seg_end[seg - 1] : 0;
    }
    seg = __builtin_amdgcn_readfirstlane(seg);
    rB[i] = __builtin_amdgcn_make_buffer_rsrc((void*)((const T*)p.B[seg] + gofs),
                                              (short)0, p.b_bytes[seg], 0x00020000);
    b_off[i] = ok ? (uint32_t)(((int64_t)n * p.ldb + kch * CH) * sizeof(T))
                  : p.b_bytes[seg];
  }
  // When the swizzle repeats every NW*RPI rows, the k of this lane's chunk
  // is the same in every load instruction and one K-tail test covers a
  // stage; otherwise (rows of 512 bytes) each load tests its own k.
  constexpr bool K_UNIFORM = (TL::NW * RPI) % 16 == 0 || KB <= 256;
  static_assert(!K_UNIFORM || KB > 256 || (TL::NW * RPI / RPB) % CPR == 0,
                "swizzle period divides the load stride");
  const int k_lane = a_k[0];
  // Dense A rows without a gather: offsets are base + i * stride (rows past
  // M read whatever the resource holds or zeros, and are never stored).
  const bool a_dense = !GROUPED && p.a_gather == nullptr;
  const uint32_t a_stride = (uint32_t)((int64_t)TL::NW * RPI * p.lda * sizeof(T));
  auto issue = [&](int kt, int buf) {
    const uint32_t ko = kt * BK * sizeof(T);
    const bool kin = kt * BK + k_lane < p.K;
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const bool ki = K_UNIFORM ? kin : kt * BK + a_k[i] < p.K;
      load16_to_lds(rA, As(buf) + (TL::NW * i + wave) * RPI * LD,
                    !ki ? p.a_bytes : (a_dense && K_UNIFORM ? a_off[0] + i * a_stride : a_off[i]) + ko);
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const bool ki = K_UNIFORM ? kin : kt * BK + b_k[i] < p.K;
      load16_to_lds(rB[i], Bs(buf) + (TL::NW * i + wave) * RPI * LD,
                    ki ? b_off[i] + ko : 0xffffffffu);
    }
  };

  using L = AccL<T, WM, WN>;
  constexpr int AM = L::AM, AN = L::AN, QPB = L::QPB;
  typename L::Blk acc[AM][AN];
#pragma unroll
  for (int i = 0; i < AM; ++i)
#pragma unroll
    for (int j = 0; j < AN; ++j)
#pragma unroll
      for (int r = 0; r < 4 * QPB; ++r) acc[i][j][r] = 0.f;

  const int nk_all = (p.K + BK - 1) / BK;
  // Whole tiles of odd rounds run K downwards.  A round is the 256
  // workgroups that fill the chip's 256 CUs once (the large tiles hold one
  // per CU); an XCD's consecutive rounds share their A panels, so a tile of
  // an odd round starts on the stages the round before ended on, still in
  // L2.  The sum runs in the other order on those tiles (float32).
  const bool rev = split_slot < 0 && ((blockIdx.x / 256) & 1);
  auto kphys = [&](int k) { return rev ? nk_all - 1 - k : k; };
  // K stages [k0, k0 + nk): all of them, or part q of S (S <= nk_all)
  const int sp_q = split_slot >= 0 ? split_slot % p.split_parts : 0;
  const int sp_n = split_slot >= 0 ? p.split_parts : 1;
  const int k0 = sp_q * nk_all / sp_n;
  const int nk = (sp_q + 1) * nk_all / sp_n - k0;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) issue(kphys(k0 + st), st);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt % NS;
    // this thread's loads of stage kt have landed (the loads of the later
    // stages may stay in flight); after the barrier all threads' have, and
    // every wave is done reading the buffer stage kt + NS - 1 refills
    if (nk - 1 - kt >= NS - 2)
      wait_vmcnt<(NS - 2) * (AL + BL)>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (kt + NS - 1 < nk) issue(kphys(k0 + kt + NS - 1), (kt + NS - 1) % NS);
    compute_tile<T, AM, AN, KB>(acc, As(cur), Bs(cur), wm * WM, wn * WN, lane);
  }
  __syncthreads();  // LDS is free for the epilogue

  if constexpr (!GROUPED && EPI != EPI_QKV && EPI != EPI_ROUTER) {
    if (split_slot >= 0) {
      // raw float32 partial tile [BM][BN] (tile-local), finished by the fixup
      float* ws = p.split_ws + (size_t)split_slot * BM * BN;
#pragma unroll
      for (int i = 0; i < AM; ++i)
#pragma unroll
        for (int j = 0; j < AN; ++j)
#pragma unroll
          for (int q = 0; q < QPB; ++q) {
            const int r = wm * WM + L::row(lane, i), c = wn * WN + L::col(lane, j, q);
            store4(ws + r * BN + c, acc[i][j][4 * q], acc[i][j][4 * q + 1],
                   acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          }
      return;
    }
  }

  // ---- epilogue: each lane stores its quads (four consecutive columns)
  if constexpr (EPI == EPI_ROUTER) {
    float* sc = reinterpret_cast<float*>(smem);
    int* hcnt = reinterpret_cast<int*>(sc + BM * (BN + 1));
    router_epilogue<T, TL>(p, acc, mt, wm, wn, lane, tid, sc, hcnt);
    return;
  } else if constexpr (EPI == EPI_QKV) {
    // each wave stages its heads in its own slice of the (now idle) LDS
    const int lrow0 = mt * BM + wm * WM;
    T* slice = smem + wave * SLICE;
    qkv_epilogue<T, HDQ, WM, WN>(acc, p, lrow0, nb0 + nt * BN + wn * WN, lane, slice);
    return;
  } else {
    tile_epilogue<T, TL, EPI>(p, acc, mt, nt, row_begin, row_count, wm, wn, lane);
  }
}

// Persistent form for the register epilogues (every EPI but q/k/v) of the
// 256x256 tile without a K split.  One workgroup per CU walks the tile ids
// b, b + G, b + 2G, ... (G = the grid); ids stay on the XCD the block runs
// on, as in the one-tile-per-block launch.  The first stage of the next
// tile is issued while the last stage of the current one computes, and its
// epilogue stores run while that load lands, so a tile boundary does not
// drain the load pipeline.
template <typename T, class TL, int EPI, bool GROUPED>
__global__ void __attribute__((amdgpu_flat_work_group_size(TL::NT, TL::NT),
                               amdgpu_waves_per_eu(TL::WPE, TL::WPE)))
gemm_persistent_kernel(const GemmParams p) {
  constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, CH = TL::CH,
                CPR = TL::CPR, LD = TL::LD, WM = TL::WM, WN = TL::WN,
                AL = TL::AL, BL = TL::BL, NS = TL::NS, RPI = TL::RPI, KB = TL::KB;
  static_assert(NS == 2 && EPI != EPI_QKV, "two stages, register epilogue");
  constexpr int RPB = 256 / KB;
  constexpr bool PAIRED = (EPI == EPI_SWIGLU);
  // epilogue stores staged through LDS (8 waves, each with an 8 KiB slice
  // of one 64 KiB stage buffer)
  constexpr bool STAGED = sizeof(T) == 2 && TL::NW == 8 && WN == 64 &&
                          BM * LD * (int)sizeof(T) == 32768 && BN * LD * (int)sizeof(T) == 32768 &&
                          (EPI == EPI_STORE || EPI == EPI_MOE_DOWN || EPI == EPI_RESID);
  constexpr int MAIN = NS * (BM + BN) * LD;
  // grouped: the tile prefix (257 ints), then each group's row offset and
  // row count (256 each), so that looking up a tile reads LDS only
  constexpr int SMEM = GROUPED ? MAIN + (257 + 512) * 4 / (int)sizeof(T) + 4 : MAIN;
  __shared__ __attribute__((aligned(1024))) T smem[SMEM];
  auto As = [&](int b) { return smem + b * (BM * LD); };
  auto Bs = [&](int b) { return smem + NS * BM * LD + b * (BN * LD); };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
  const int n_per_tile = PAIRED ? BN / 2 : BN;
  const int num_n = (p.N + n_per_tile - 1) / n_per_tile;
  const int num_m = (p.M + BM - 1) / BM;

  // ---- the tiles: grouped M tiles per expert as in gemm_kernel
  int* tpre = reinterpret_cast<int*>(smem + MAIN);
  int* sgoff = tpre + 257;
  int* sgcnt = sgoff + 256;
  int total;
  if constexpr (GROUPED) {
    if (wave == 0) {
      int c[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = 4 * lane + q;
        const int cnt = g < p.ngroups ? p.gcnt[g] : 0;
        sgcnt[g] = cnt;
        sgoff[g] = g < p.ngroups ? p.goff[g] : 0;
        c[q] = (cnt + BM - 1) / BM;
        sum += c[q];
      }
      int inc = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o, 64);
        if (lane >= o) inc += v;
      }
      int ex = inc - sum;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        tpre[4 * lane + q] = ex;
        ex += c[q];
      }
      if (lane == 63) tpre[256] = inc;
    }
    __syncthreads();
    total = tpre[256] * num_n;
  } else {
    total = num_m * num_n;
  }
  auto select = [&](int item, int& mt, int& nt, int& rb, int& rc, int& grp) {
    const int id = xcd_contiguous(item, total);
    if constexpr (GROUPED) {
      const int t = id / num_n;
      nt = id % num_n;
      int lo = 0, hi = p.ngroups;  // tpre[lo] <= t < tpre[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tpre[mid] <= t) lo = mid;
        else hi = mid;
      }
      grp = lo;
      mt = t - tpre[lo];
      rb = sgoff[lo];
      rc = sgcnt[lo];
    } else {
      tile_coords(id, num_m, num_n, mt, nt);
      rb = 0;
      rc = p.M;
      grp = 0;
    }
  };

  // ---- direct-to-LDS load offsets of a tile (as in gemm_kernel)
  const int lrowi = lane / CPR;
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, p.a_bytes, 0x00020000);
  static_assert((TL::NW * RPI / RPB) % CPR == 0, "swizzle period divides the load stride");
  const int k_lane = ((lane % CPR) ^ (((wave * RPI + lrowi) / RPB) & (CPR - 1))) * CH;
  const bool a_dense = !GROUPED && p.a_gather == nullptr;
  const uint32_t a_stride = (uint32_t)((int64_t)TL::NW * RPI * p.lda * sizeof(T));
  // Only a grouped gate/up GEMM gathers its A rows.  The gathered row of
  // each of the thread's A loads is fetched when the tile is looked up and
  // consumed when its first stage is issued, a whole tile later.  With
  // LATE, every other offset of the next tile is computed from its scalars
  // when its first stage is issued, so nothing per lane stays live across
  // the k-loop: the grouped and activation kernels spill otherwise (up to
  // 30 VGPRs, reloaded behind the epilogue's stores).  The others compute
  // the offsets up front, which measured slightly faster for them.
  constexpr bool GATHER = GROUPED && PAIRED;
  constexpr bool LATE = GROUPED || EPI == EPI_RELU2 || EPI == EPI_XIELU || EPI == EPI_SILU;
  auto src_row = [&](int mt, int rb, int rc, int i) {
    const int r = mt * BM + (TL::NW * i + wave) * RPI + lrowi;
    return rb + (r < rc ? r : 0);
  };
  auto gather = [&](int mt, int rb, int rc, int (&g)[AL]) {
#pragma unroll
    for (int i = 0; i < AL; ++i) g[i] = (GATHER && p.a_gather) ? p.a_gather[src_row(mt, rb, rc, i)] : 0;
  };
  auto setup = [&](int mt, int nt, int rb, int rc, int grp, const int (&g)[AL],
                   uint32_t (&a_off)[AL], uint32_t (&b_off)[BL],
                   __amdgpu_buffer_rsrc_t (&rB)[BL]) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int lrow = (TL::NW * i + wave) * RPI + lrowi;
      const int kch = (lane % CPR) ^ ((lrow / RPB) & (CPR - 1));
      const int r = mt * BM + lrow;
      const int src = (GATHER && p.a_gather) ? g[i] : src_row(mt, rb, rc, i);
      a_off[i] = (r < rc) ? (uint32_t)(((int64_t)src * p.lda + kch * CH) * sizeof(T))
                          : p.a_bytes;
    }
    const int64_t gofs = GROUPED ? (int64_t)grp * p.b_group_stride : 0;
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int lbase = (TL::NW * i + wave) * RPI;
      const int lrow = lbase + lrowi;
      const int kch = (lane % CPR) ^ ((lrow / RPB) & (CPR - 1));
      int seg, n;
      bool ok;
      if constexpr (PAIRED) {
        constexpr int half = WN / 2;
        seg = (lbase % WN) / half;
        n = nt * (BN / 2) + (lbase / WN) * half + (lrow % WN) % half;
        ok = n < p.N;
      } else {
        const int nb = nt * BN + lbase;
        seg = 0;
        while (seg < p.nseg - 1 && nb >= p.seg_end[seg]) ++seg;
        n = nt * BN + lrow;
        ok = n < p.N;
        n -= seg ? p.seg_end[seg - 1] : 0;
      }
      seg = __builtin_amdgcn_readfirstlane(seg);
      rB[i] = __builtin_amdgcn_make_buffer_rsrc((void*)((const T*)p.B[seg] + gofs), (short)0,
                                                p.b_bytes[seg], 0x00020000);
      b_off[i] = ok ? (uint32_t)(((int64_t)n * p.ldb + kch * CH) * sizeof(T)) : p.b_bytes[seg];
    }
  };
  auto issue = [&](int kt, int buf, const uint32_t (&a_off)[AL], const uint32_t (&b_off)[BL],
                   const __amdgpu_buffer_rsrc_t (&rB)[BL]) {
    const uint32_t ko = kt * BK * sizeof(T);
    const bool kin = kt * BK + k_lane < p.K;
#pragma unroll
    for (int i = 0; i < AL; ++i)
      load16_to_lds(rA, As(buf) + (TL::NW * i + wave) * RPI * LD,
                    !kin ? p.a_bytes : (a_dense ? a_off[0] + i * a_stride : a_off[i]) + ko);
#pragma unroll
    for (int i = 0; i < BL; ++i)
      load16_to_lds(rB[i], Bs(buf) + (TL::NW * i + wave) * RPI * LD,
                    kin ? b_off[i] + ko : 0xffffffffu);
  };

  using L = AccL<T, WM, WN>;
  constexpr int AM = L::AM, AN = L::AN, QPB = L::QPB;
  typename L::Blk acc[AM][AN];
  const int nk = (p.K + BK - 1) / BK;

  int item = blockIdx.x;
  if (item >= total) return;
  int mt, nt, rb, rc, grp;
  select(item, mt, nt, rb, rc, grp);
  int g[AL];
  gather(mt, rb, rc, g);
  uint32_t a_off[AL], b_off[BL];
  __amdgpu_buffer_rsrc_t rB[BL];
  setup(mt, nt, rb, rc, grp, g, a_off, b_off, rB);
#ifndef GEMM_SNAKE
#define GEMM_SNAKE 1
#endif
  // K runs up on a block's even tiles and down on its odd ones: a block's
  // consecutive tiles share their A rows (or, grouped, their expert's B
  // rows), so a new tile starts on the stage the tiles before it just read
  // (still in L2) instead of a stage every block of the XCD misses at once
  auto kphys = [&](int kt, int dir) { return (GEMM_SNAKE && dir) ? nk - 1 - kt : kt; };
  int dir = 0;
  int buf = 0;
  issue(kphys(0, dir), 0, a_off, b_off, rB);
  while (true) {
#pragma unroll
    for (int i = 0; i < AM; ++i)
#pragma unroll
      for (int j = 0; j < AN; ++j)
#pragma unroll
        for (int r = 0; r < 4 * QPB; ++r) acc[i][j][r] = 0.f;
    // the next tile, looked up while this one computes
    const int nitem = item + (int)gridDim.x;
    const bool more = nitem < total;
    int mt2 = 0, nt2 = 0, rb2 = 0, rc2 = 0, grp2 = 0;
    int g2[AL];
    uint32_t a2[AL], b2[BL];
    __amdgpu_buffer_rsrc_t rB2[BL];
    if (more) {
      select(nitem, mt2, nt2, rb2, rc2, grp2);
      mt2 = __builtin_amdgcn_readfirstlane(mt2);
      nt2 = __builtin_amdgcn_readfirstlane(nt2);
      rb2 = __builtin_amdgcn_readfirstlane(rb2);
      rc2 = __builtin_amdgcn_readfirstlane(rc2);
      grp2 = __builtin_amdgcn_readfirstlane(grp2);
      gather(mt2, rb2, rc2, g2);
      if constexpr (!LATE) setup(mt2, nt2, rb2, rc2, grp2, g2, a2, b2, rB2);
    }
    for (int kt = 0; kt < nk; ++kt) {
      // this thread's loads of stage kt (and the stores of the previous
      // tile's epilogue) are done; after the barrier all threads' are, and
      // every wave is done with the buffer the next stage refills
      wait_vmcnt<0>();
      __syncthreads();
      if (kt + 1 < nk) {
        issue(kphys(kt + 1, dir), buf ^ 1, a_off, b_off, rB);
      } else if (more) {
        if constexpr (LATE) setup(mt2, nt2, rb2, rc2, grp2, g2, a2, b2, rB2);
        issue(kphys(0, dir ^ 1), buf ^ 1, a2, b2, rB2);
      }
      compute_tile<T, AM, AN, KB>(acc, As(buf), Bs(buf), wm * WM, wn * WN, lane);
      buf ^= 1;
    }
    dir ^= 1;
    if constexpr (STAGED) {
      // every wave is done with the last stage's buffer (buf ^ 1): it holds
      // the staging slices until the next tile's first barrier
      __syncthreads();
      char* st = wave < 4 ? (char*)As(buf ^ 1) + wave * 8192
                          : (char*)Bs(buf ^ 1) + (wave - 4) * 8192;
      if (!staged_epilogue<T, TL, EPI>(p, acc, mt, nt, rb, rc, wm, wn, lane, st))
        tile_epilogue<T, TL, EPI>(p, acc, mt, nt, rb, rc, wm, wn, lane);
    } else {
      tile_epilogue<T, TL, EPI>(p, acc, mt, nt, rb, rc, wm, wn, lane);
    }
    if (!more) break;
    item = nitem;
    mt = mt2;
    nt = nt2;
    rb = rb2;
    rc = rc2;
    grp = grp2;
    if constexpr (LATE) {
      setup(mt, nt, rb, rc, grp, g2, a_off, b_off, rB);
    } else {
#pragma unroll
      for (int i = 0; i < AL; ++i) a_off[i] = a2[i];
#pragma unroll
      for (int i = 0; i < BL; ++i) {
        b_off[i] = b2[i];
        rB[i] = rB2[i];
      }
    }
  }
}

// K-split fixup: split tile j is tile F + j of the grid (F = whole tiles);
// its S = split_parts K parts are float32 [BM][BN] tiles at
// split_ws[S j + q].  Their sum, added in part order, goes through the same
// epilogue as a whole tile.
template <typename T, int EPI, int BM, int BN, int WN>
__global__ void __launch_bounds__(256) split_fixup_kernel(const GemmParams p) {
  constexpr bool PAIRED = (EPI == EPI_SWIGLU);
  const int n_per_tile = PAIRED ? BN / 2 : BN;
  const int num_n = (p.N + n_per_tile - 1) / n_per_tile;
  const int num_m = (p.M + BM - 1) / BM;
  const int j = blockIdx.x;
  int mt, nt;
  tile_coords(num_m * num_n - p.split_tiles + j, num_m, num_n, mt, nt);
  const int S = p.split_parts;
  const float* w0 = p.split_ws + (size_t)(S * j) * BM * BN;
  auto sum4 = [&](int off, float (&v)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = w0[off + e];
    for (int q = 1; q < S; ++q) {
      const float* wq = w0 + (size_t)q * BM * BN + off;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += wq[e];
    }
  };
  for (int qd = threadIdx.x; qd < BM * BN / 4; qd += 256) {
    const int r = qd / (BN / 4), c = (qd % (BN / 4)) * 4;
    const int row = mt * BM + r;
    if (row >= p.M) continue;
    if constexpr (PAIRED) {
      const int cc = c % WN;
      if (cc >= WN / 2) continue;
      float g[4], u[4];
      sum4(r * BN + c, g);
      sum4(r * BN + c + WN / 2, u);
      swiglu_quad<T>(p, (T*)p.out + (int64_t)row * p.ldo, nt * (BN / 2) + (c / WN) * (WN / 2) + cc,
                     g, u);
    } else {
      const int col = nt * BN + c;
      if (col >= p.N) continue;
      float v[4];
      sum4(r * BN + c, v);
      epi_quad<T, EPI>(p, (int64_t)row * p.ldo, col, v, 1.0f);
    }
  }
}

// ------------------------------------------------------------ launchers

static int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      n = v;
    if (n <= 0) n = 256;
  }
  return n;
}

// 256 x 128 tiles (8 waves of 64 x 64, the wave width of the staged
// epilogues) for the last round of a persistent launch.
using TileH = Tile<bf16, 256, 128, 4, 2, 128, 2>;
// the q/k/v form: 8 waves of 32 x 128, whole heads per wave
using TileQH = Tile<bf16, 256, 128, 8, 1, 128, 2>;

// The same product restricted to output columns [n0, N): the first nb B
// segments (those that hold output columns) start n0 rows later, and every
// output and the residual start n0 columns later.
template <typename T>
static GemmParams column_window(const GemmParams& p, int n0, int nb) {
  GemmParams q = p;
  q.N = p.N - n0;
  const int64_t skip = (int64_t)n0 * p.ldb;
  for (int s = 0; s < nb; ++s) {
    q.B[s] = (const T*)p.B[s] + skip;
    q.b_bytes[s] = p.b_bytes[s] - (uint32_t)(skip * (int64_t)sizeof(T));
    q.seg_end[s] = p.seg_end[s] - n0;
  }
  if (p.out)
    q.out = p.out_f32 ? (void*)((float*)p.out + n0) : (void*)((T*)p.out + n0);
  if (p.out_f32p) q.out_f32p = p.out_f32p + n0;
  if (p.out_model) q.out_model = (T*)p.out_model + n0;
  if (p.out_raw) q.out_raw = p.out_raw + n0;
  if (p.resid)
    q.resid = p.resid_f32 ? (const void*)((const float*)p.resid + n0)
                          : (const void*)((const T*)p.resid + n0);
  return q;
}

template <typename T, class TL, int EPI, bool GROUPED, int HDQ = 0>
static hipError_t launch(const GemmParams& p0, int max_rows, hipStream_t s) {
  const int n_per_tile = (EPI == EPI_SWIGLU) ? TL::BN / 2 : TL::BN;
  const int num_n = (p0.N + n_per_tile - 1) / n_per_tile;
  constexpr bool PERSIST = TL::BM == 256 && TL::BN == 256 && TL::NS == 2 && TL::WGM == 2 &&
                           sizeof(T) == 2 && EPI != EPI_QKV;
  if (GROUPED && !PERSIST) {
    const int max_tiles = (max_rows + TL::BM - 1) / TL::BM + p0.ngroups;
    hipLaunchKernelGGL((gemm_kernel<T, TL, EPI, GROUPED, HDQ>), dim3(max_tiles * num_n),
                       dim3(TL::NT), 0, s, p0);
    return hipGetLastError();
  }
  if constexpr (PERSIST && GROUPED) {
    const int max_tiles = (max_rows + TL::BM - 1) / TL::BM + p0.ngroups;
    const int grid = std::min(max_tiles * num_n, cu_count());
    hipLaunchKernelGGL((gemm_persistent_kernel<T, TL, EPI, GROUPED>), dim3(grid),
                       dim3(TL::NT), 0, s, p0);
    return hipGetLastError();
  }
  GemmParams p = p0;
  p.split_tiles = 0;
  p.split_parts = 1;
  const int num_m = (p.M + TL::BM - 1) / TL::BM;
  const int tiles = num_m * num_n;
  if constexpr (EPI != EPI_QKV && EPI != EPI_ROUTER) {
    const int cus = cu_count();
    const int rem = tiles % cus;
    const int nk = (p.K + TL::BK - 1) / TL::BK;
    const size_t tile_bytes = (size_t)TL::BM * TL::BN * sizeof(float);
    if (tiles > cus && rem > 0 && rem <= cus / 2 && nk >= 128 && p.split_ws != nullptr &&
        (size_t)rem * 2 * tile_bytes <= p.split_ws_bytes) {
      // tail split: the last wave would leave more than half of the CUs
      // idle.  The partial tiles and the fixup cost a roughly fixed ~30 us,
      // so only long K (>= 128 stages; measured: 288 stages gain 10%, 40
      // and 64 lose)
      p.split_tiles = rem;
      p.split_parts = 2;
    } else if (4 * tiles <= cus && nk >= 16 && p.split_ws != nullptr) {
      // a grid on at most a quarter of the CUs: every tile in S K parts of
      // at least 4 stages, so that the grid's stage-by-stage latency is
      // paid on S times fewer stages (measured on the tiny float32 block:
      // 22 stages in 5 parts 52 -> 29 us; 8 stages in 2 parts gain or lose
      // about 2 us, so shorter K stays whole)
      int S = std::min(std::min(nk / 4, cus / tiles), 16);
      while (S >= 2 && (size_t)tiles * S * tile_bytes > p.split_ws_bytes) --S;
      if (S >= 2) {
        p.split_tiles = tiles;
        p.split_parts = S;
      }
    }
  }
  if constexpr (PERSIST && !GROUPED) {
    if (p.split_tiles == 0) {
      const int cus = cu_count();
      const int rem = tiles % cus;
      const int c = rem / num_m;  // whole tile columns in the last round
      if (tiles > cus && rem > 0 && rem <= cus / 2 && rem % num_m == 0 &&
          p.nseg == (EPI == EPI_SWIGLU ? 2 : 1)) {
        // The last round would leave half the CUs idle or more.  Its tiles
        // are the last c tile columns: run them as twice as many 256 x 128
        // tiles in a launch of their own, so every CU has one.
        const int n0 = (num_n - c) * n_per_tile;
        GemmParams head = p;
        head.N = n0;
        hipLaunchKernelGGL((gemm_persistent_kernel<T, TL, EPI, GROUPED>),
                           dim3(std::min(tiles - rem, cus)), dim3(TL::NT), 0, s, head);
        const GemmParams tail = column_window<T>(p, n0, EPI == EPI_SWIGLU ? 2 : 1);
        const int tn = (EPI == EPI_SWIGLU) ? TileH::BN / 2 : TileH::BN;
        hipLaunchKernelGGL((gemm_kernel<T, TileH, EPI, GROUPED>),
                           dim3(num_m * ((tail.N + tn - 1) / tn)), dim3(TileH::NT), 0, s,
                           tail);
        return hipGetLastError();
      }
      hipLaunchKernelGGL((gemm_persistent_kernel<T, TL, EPI, GROUPED>),
                         dim3(std::min(tiles, cus)), dim3(TL::NT), 0, s, p);
      return hipGetLastError();
    }
  }
  if constexpr (EPI == EPI_QKV && TL::BM == 256 && TL::BN == 256) {
    const int cus = cu_count();
    const int rem = tiles % cus;
    if (tiles > cus && rem > 0 && rem <= cus / 2 && rem % num_m == 0) {
      // the last round as 256 x 128 tiles of the same heads, one per CU
      const int n0 = (num_n - rem / num_m) * TL::BN;
      GemmParams head = p;
      head.N = n0;
      hipLaunchKernelGGL((gemm_kernel<T, TL, EPI, GROUPED, HDQ>), dim3(tiles - rem),
                         dim3(TL::NT), 0, s, head);
      GemmParams tail = p;
      tail.n_base = n0;
      hipLaunchKernelGGL((gemm_kernel<T, TileQH, EPI, GROUPED, HDQ>),
                         dim3(num_m * ((p.N - n0 + TileQH::BN - 1) / TileQH::BN)),
                         dim3(TileQH::NT), 0, s, tail);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kernel<T, TL, EPI, GROUPED, HDQ>),
                     dim3(tiles + p.split_tiles * (p.split_parts - 1)), dim3(TL::NT), 0, s, p);
  if constexpr (EPI != EPI_QKV && EPI != EPI_ROUTER) {
    if (p.split_tiles > 0)
      hipLaunchKernelGGL((split_fixup_kernel<T, EPI, TL::BM, TL::BN, TL::WN>),
                         dim3(p.split_tiles), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

// 128-byte K stages, two in LDS (a deeper pipeline of 64-byte stages
// measured slower: the extra barriers cost more than the latency it hides).
using TileL = Tile<bf16, 256, 256, 2, 4, 128, 2>;
using TileQ = Tile<bf16, 256, 256, 4, 2, 128, 2>;  // 64x128 wave tiles: whole heads per wave
using TileS = Tile<bf16, 128, 128, 4, 1, 128, 2>;
// narrow outputs (the router): 64 x 64 tiles, 512-byte K rows per stage.
// The router reads its 67 MB operand once, one 64-row block per
// workgroup; longer rows per stage read faster at the afmoe shape (128-byte
// rows 48 us, 256-byte 37.6, 512-byte 35.0), where 4 or 8 stages of
// 128-byte rows gained nothing.
using TileR = Tile<bf16, 64, 64, 2, 2, 512, 2>;
using TileF = Tile<float, 128, 128, 4, 1, 128, 2>;

template <typename T, class TL>
static hipError_t dispatch_epi(EpiKind epi, bool grouped, const GemmParams& p,
                               int max_rows, hipStream_t s) {
  if (grouped) {
    switch (epi) {
      case EPI_SWIGLU: return launch<T, TL, EPI_SWIGLU, true>(p, max_rows, s);
      case EPI_MOE_DOWN: return launch<T, TL, EPI_MOE_DOWN, true>(p, max_rows, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (epi) {
    case EPI_STORE: return launch<T, TL, EPI_STORE, false>(p, max_rows, s);
    case EPI_RESID: return launch<T, TL, EPI_RESID, false>(p, max_rows, s);
    case EPI_SWIGLU: return launch<T, TL, EPI_SWIGLU, false>(p, max_rows, s);
    case EPI_RELU2: return launch<T, TL, EPI_RELU2, false>(p, max_rows, s);
    case EPI_XIELU: return launch<T, TL, EPI_XIELU, false>(p, max_rows, s);
    case EPI_SILU: return launch<T, TL, EPI_SILU, false>(p, max_rows, s);
    case EPI_QKV:
      if constexpr (TL::FM <= 2 && TL::WN >= 128) {
        if (p.hd == 64) return launch<T, TL, EPI_QKV, false, 64>(p, max_rows, s);
        return launch<T, TL, EPI_QKV, false, 128>(p, max_rows, s);
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

int router_tile_tokens(DType dt, int E) {
  if (dt == DType::F32) return E <= TileF::BN ? TileF::BM : 0;
  return E <= TileR::BN ? TileR::BM : 0;
}

hipError_t gemm(DType dt, EpiKind epi, const GemmParams& p, int max_rows,
                hipStream_t s) {
  const bool grouped = p.gcnt != nullptr;
  if (epi == EPI_ROUTER) {
    if (grouped || router_tile_tokens(dt, p.N) == 0) return hipErrorInvalidValue;
    if (dt == DType::F32) return launch<float, TileF, EPI_ROUTER, false>(p, max_rows, s);
    return launch<bf16, TileR, EPI_ROUTER, false>(p, max_rows, s);
  }
  if (dt == DType::F32) return dispatch_epi<float, TileF>(epi, grouped, p, max_rows, s);
  // Large tiles when they still give the chip at least one full wave of
  // workgroups; the 128x128 tile otherwise.
  const int n_per = (epi == EPI_SWIGLU) ? 128 : 256;
  if (epi == EPI_QKV) {
    // the q/k norm + rotary epilogue needs whole heads in a wave: 64 x 128
    // wave tiles
    const long tiles_q = (long)((max_rows + 255) / 256) * ((p.N + 255) / 256);
    if (tiles_q >= 256) return dispatch_epi<bf16, TileQ>(epi, grouped, p, max_rows, s);
    return dispatch_epi<bf16, TileS>(epi, grouped, p, max_rows, s);
  }
  const long tiles_l = (long)((max_rows + 255) / 256) * ((p.N + n_per - 1) / n_per);
  if (tiles_l >= 256) return dispatch_epi<bf16, TileL>(epi, grouped, p, max_rows, s);
  const long tiles_s = (long)((max_rows + 127) / 128) * ((p.N + n_per / 2 - 1) / (n_per / 2));
  if (tiles_s >= 256 || grouped || epi != EPI_STORE)
    return dispatch_epi<bf16, TileS>(epi, grouped, p, max_rows, s);
  return launch<bf16, TileR, EPI_STORE, false>(p, max_rows, s);
}

}  // namespace blk
