// NT GEMM on gfx950 matrix cores with the block's fused epilogues.
//
//   C[M, N] = A[M, K] . B[N, K]^T        (both operands K-contiguous, the
//                                         Linear layout [out, in] for B)
//
// One workgroup = 4 wavefronts computes a BM x BN tile; each wave owns a
// (BM/WGM) x (BN/WGN) sub-tile made of 32x32 MFMA blocks.  Operand tiles of
// 128 bytes of K per row are staged through LDS, double-buffered: the
// global loads of step k+1 are issued before the MFMAs of step k and land
// in the other LDS buffer afterwards, so one barrier per K-step suffices.
// LDS rows are padded by 16 bytes so the 16-byte fragment reads of 16 (or
// 8) consecutive rows hit distinct banks.
//
// bf16: v_mfma_f32_32x32x16_bf16 (lane l holds row l%32, k 8*(l/32)..+7).
// f32 : v_mfma_f32_32x32x2f32 with the K order inside a 32-wide K tile
//       permuted so every lane reads 4 consecutive floats per LDS access
//       (half h of the wave takes k = 16h + 4g + s at step (g, s)); A and B
//       use the same permutation, so the sum is unchanged.
// Accumulator layout (both): lane l holds column l%32 and rows
//       8*(r/4) + 4*(l/32) + r%4 of its 32x32 block, r = 0..15.
#include "common.h"
#include "kernels.h"

namespace blk {

template <typename T> struct KTile;
template <> struct KTile<bf16> { static constexpr int BK = 64; };
template <> struct KTile<float> { static constexpr int BK = 32; };

template <typename T, int BM_, int BN_, int WGM_, int WGN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int BK = KTile<T>::BK;
  static constexpr int CH = 16 / sizeof(T);   // elements per 16-byte chunk
  static constexpr int CPR = BK / CH;         // chunks per tile row (8)
  static constexpr int LD = BK + CH;          // padded LDS row (144 bytes)
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int AL = BM * CPR / 256;   // A chunks per thread
  static constexpr int BL = BN * CPR / 256;   // B chunks per thread
  static_assert(WGM * WGN == 4, "4 waves");
  static_assert(FM >= 1 && FN >= 1, "wave tile >= 32x32");
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

template <typename T, int FM, int FN, int LD, int BK>
__device__ __forceinline__ void compute_tile(f32x16 (&acc)[FM][FN],
                                             const T* As, const T* Bs,
                                             int arow0, int brow0, int lane);

#define BLK_COMPUTE_BF16(FM_, FN_)                                            \
  template <>                                                                 \
  __device__ __forceinline__ void compute_tile<bf16, FM_, FN_, 72, 64>(       \
      f32x16(&acc)[FM_][FN_], const bf16* As, const bf16* Bs, int arow0,      \
      int brow0, int lane) {                                                  \
    const int r = lane & 31, kh = (lane >> 5) * 8;                            \
    _Pragma("unroll") for (int ks = 0; ks < 4; ++ks) {                        \
      bf16x8 af[FM_], bfr[FN_];                                               \
      _Pragma("unroll") for (int i = 0; i < FM_; ++i) af[i] =                 \
          *reinterpret_cast<const bf16x8*>(As + (arow0 + i * 32 + r) * 72 +   \
                                           ks * 16 + kh);                     \
      _Pragma("unroll") for (int j = 0; j < FN_; ++j) bfr[j] =                \
          *reinterpret_cast<const bf16x8*>(Bs + (brow0 + j * 32 + r) * 72 +   \
                                           ks * 16 + kh);                     \
      _Pragma("unroll") for (int i = 0; i < FM_; ++i)                         \
          _Pragma("unroll") for (int j = 0; j < FN_; ++j) acc[i][j] =         \
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j],          \
                                                      acc[i][j], 0, 0, 0);    \
    }                                                                         \
  }

BLK_COMPUTE_BF16(4, 4)
BLK_COMPUTE_BF16(1, 4)
BLK_COMPUTE_BF16(2, 2)
BLK_COMPUTE_BF16(2, 4)

#define BLK_COMPUTE_F32(FM_, FN_)                                             \
  template <>                                                                 \
  __device__ __forceinline__ void compute_tile<float, FM_, FN_, 36, 32>(      \
      f32x16(&acc)[FM_][FN_], const float* As, const float* Bs, int arow0,    \
      int brow0, int lane) {                                                  \
    const int r = lane & 31, kh = (lane >> 5) * 16;                           \
    _Pragma("unroll") for (int g = 0; g < 4; ++g) {                           \
      f32x4 af[FM_], bfr[FN_];                                                \
      _Pragma("unroll") for (int i = 0; i < FM_; ++i) af[i] =                 \
          *reinterpret_cast<const f32x4*>(As + (arow0 + i * 32 + r) * 36 +    \
                                          kh + g * 4);                        \
      _Pragma("unroll") for (int j = 0; j < FN_; ++j) bfr[j] =                \
          *reinterpret_cast<const f32x4*>(Bs + (brow0 + j * 32 + r) * 36 +    \
                                          kh + g * 4);                        \
      _Pragma("unroll") for (int s = 0; s < 4; ++s)                           \
          _Pragma("unroll") for (int i = 0; i < FM_; ++i)                     \
              _Pragma("unroll") for (int j = 0; j < FN_; ++j) acc[i][j] =     \
                  __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][s], bfr[j][s],   \
                                                       acc[i][j], 0, 0, 0);   \
    }                                                                         \
  }

BLK_COMPUTE_F32(1, 4)

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

// Q/K/V(/gate) epilogue.  A wave owns WM rows (tokens) x FN*32 columns; its
// columns hold whole heads.  Per head: optional per-head RMSNorm (sum of
// squares over the head's HD columns, reduced across the 32 lanes that
// hold them), rotary on the pairs (d, d + HD/2), which sit in the same
// lane, then the head is staged through this wave's slice of LDS so that
// the global stores are 16-byte and coalesced: q/k rows [token][d] go to
// [b, head, s, :], v goes transposed to V^T [b, head, d, s] (keys
// contiguous, the layout the attention kernel's P.V product reads).
template <typename T, int HD, int FM, int FN, int WM>
__device__ __forceinline__ void qkv_epilogue(f32x16 (&acc)[FM][FN],
                                             const GemmParams& p, int row0,
                                             int col0, int lane, T* lds) {
  constexpr int HB = HD / 32;       // 32-wide blocks per head
  constexpr int CH = 16 / sizeof(T);
  constexpr int QLD = HD + CH;      // staged q/k row   [WM][QLD]
  constexpr int VLD = WM + CH;      // staged v^T row   [HD][VLD]
  static_assert(FN % HB == 0, "wave columns must hold whole heads");
  const int cl = lane & 31, hi4 = (lane >> 5) * 4;
  const int Sp = (p.S + 63) & ~63;  // V^T rows are padded to 64 keys
#pragma unroll
  for (int hh = 0; hh < FN / HB; ++hh) {
    const int c0 = col0 + hh * HD;
    if (c0 >= p.N) continue;
    int seg = 0;
    while (seg < p.nseg - 1 && c0 >= p.seg_end[seg]) ++seg;
    const int start = seg ? p.seg_end[seg - 1] : 0;
    if (seg == 3) {  // gate columns: sigmoid, float32 [M, G]
#pragma unroll
      for (int fb = 0; fb < HB; ++fb) {
        const int col = c0 + fb * 32 + cl;
        if (col >= p.N) continue;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row0 + fm * 32 + (r >> 2) * 8 + hi4 + (r & 3);
            if (row < p.M)
              p.gate[(int64_t)row * p.G + (col - start)] =
                  1.0f / (1.0f + expf(-acc[fm][hh * HB + fb][r]));
          }
      }
      continue;
    }
    const int head = (c0 - start) / HD;
    if (seg < 2 && p.qk_norm) {
      const T* gw = (const T*)(seg == 0 ? p.q_norm_w : p.k_norm_w);
      float gv[HB];
#pragma unroll
      for (int fb = 0; fb < HB; ++fb) gv[fb] = to_f32(gw[fb * 32 + cl]);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float ss = 0.f;
#pragma unroll
          for (int fb = 0; fb < HB; ++fb) {
            const float v = acc[fm][hh * HB + fb][r];
            ss += v * v;
          }
          ss = half_sum(ss);
          const float inv = 1.0f / sqrtf(ss * (1.0f / HD) + p.eps);
#pragma unroll
          for (int fb = 0; fb < HB; ++fb)
            acc[fm][hh * HB + fb][r] = gv[fb] * (acc[fm][hh * HB + fb][r] * inv);
        }
    }
    if (seg < 2 && p.use_rope) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + fm * 32 + (r >> 2) * 8 + hi4 + (r & 3);
          const int pos = (row < p.M) ? row % p.S : 0;
#pragma unroll
          for (int fb = 0; fb < HB / 2; ++fb) {
            const int d = fb * 32 + cl;
            const float c = p.rope_cos[pos * (HD / 2) + d];
            const float s = p.rope_sin[pos * (HD / 2) + d];
            const float lo = acc[fm][hh * HB + fb][r];
            const float hi = acc[fm][hh * HB + fb + HB / 2][r];
            acc[fm][hh * HB + fb][r] = lo * c - hi * s;
            acc[fm][hh * HB + fb + HB / 2][r] = hi * c + lo * s;
          }
        }
    }
    if (seg < 2) {
      // stage [row][d], then store rows of the head contiguously
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fb = 0; fb < HB; ++fb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = fm * 32 + (r >> 2) * 8 + hi4 + (r & 3);
            lds[rr * QLD + fb * 32 + cl] = from_f32<T>(acc[fm][hh * HB + fb][r]);
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
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fb = 0; fb < HB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            T* dstl = lds + (fb * 32 + cl) * VLD + fm * 32 + i * 8 + hi4;
#pragma unroll
            for (int j = 0; j < 4; ++j) dstl[j] = from_f32<T>(acc[fm][hh * HB + fb][i * 4 + j]);
          }
      wave_lds_sync();
      T* base = (T*)p.vt;
      constexpr int RCH = WM / CH;  // chunks of CH rows per d
      const bool s_aligned = (p.S % CH) == 0;
#pragma unroll 4
      for (int it = 0; it < HD * RCH / 64; ++it) {
        const int idx = it * 64 + lane;
        const int d = idx / RCH, rc = idx % RCH;
        const int r0 = row0 + rc * CH;
        const T* src = lds + d * VLD + rc * CH;
        const int b0 = r0 / p.S;
        if (s_aligned && r0 + CH <= p.M && (r0 + CH - 1) / p.S == b0) {
          T* dst = base + (((int64_t)b0 * p.nkv + head) * HD + d) * Sp + (r0 % p.S);
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
          for (int e = 0; e < CH; ++e) {
            const int row = r0 + e;
            if (row >= p.M) break;
            const int b = row / p.S;
            base[(((int64_t)b * p.nkv + head) * HD + d) * Sp + (row % p.S)] = src[e];
          }
        }
      }
    }
    wave_lds_sync();  // the next head reuses this wave's LDS slice
  }
}

// ---------------------------------------------------------------- kernel

template <typename T, class TL, int EPI, bool GROUPED>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256),
                               amdgpu_waves_per_eu(1, 1)))
gemm_kernel(const GemmParams p) {
  constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, CH = TL::CH,
                CPR = TL::CPR, LD = TL::LD, WM = TL::WM, WN = TL::WN,
                FM = TL::FM, FN = TL::FN, AL = TL::AL, BL = TL::BL;
  constexpr bool PAIRED = (EPI == EPI_SWIGLU);
  __shared__ __attribute__((aligned(16))) T smem[2 * (BM + BN) * LD];
  auto As = [&](int b) { return smem + b * (BM * LD); };
  auto Bs = [&](int b) { return smem + 2 * BM * LD + b * (BN * LD); };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
  const int n_per_tile = PAIRED ? BN / 2 : BN;
  const int num_n = (p.N + n_per_tile - 1) / n_per_tile;

  // ---- which tile
  int mt, nt, row_begin = 0, row_count = p.M, group = 0;
  if constexpr (GROUPED) {
    int t = blockIdx.x;
    nt = blockIdx.y;
    int g = 0;
    for (; g < p.ngroups; ++g) {
      const int tiles = (p.gcnt[g] + BM - 1) / BM;
      if (t < tiles) break;
      t -= tiles;
    }
    if (g >= p.ngroups) return;  // idle tile of the worst-case grid
    group = g;
    mt = t;
    row_begin = p.goff[g];
    row_count = p.gcnt[g];
  } else {
    const int num_m = (p.M + BM - 1) / BM;
    const int id = xcd_contiguous(blockIdx.x, gridDim.x);
    constexpr int GROUP_M = 8;
    const int width = GROUP_M * num_n;
    const int first_m = (id / width) * GROUP_M;
    const int gsz = min(num_m - first_m, GROUP_M);
    mt = first_m + (id % width) % gsz;
    nt = (id % width) / gsz;
  }

  // ---- per-thread global sources.  Operands are read with raw buffer
  // loads: an offset at or past the resource's byte size returns zeros,
  // which covers rows past M/N (ragged tiles); the K tail is masked the
  // same way.  Each thread always reads the same 16-byte column chunk kc
  // of CPR-chunk rows tid/CPR + 32 i.
  const int kc = tid % CPR;
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, p.a_bytes, 0x00020000);
  uint32_t a_off[AL];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int lrow = tid / CPR + i * (256 / CPR);
    const int r = mt * BM + lrow;
    int src = row_begin + (r < row_count ? r : 0);
    if (p.a_gather) src = p.a_gather[src];
    a_off[i] = (r < row_count)
                   ? (uint32_t)(((int64_t)src * p.lda + kc * CH) * sizeof(T))
                   : p.a_bytes;
  }
  // B: the segment (QKV: q/k/v/gate; SWIGLU: gate/up) of chunk i is the
  // same for the whole workgroup, since segments are 32-row aligned.
  const int64_t gofs = GROUPED ? (int64_t)group * p.b_group_stride : 0;
  __amdgpu_buffer_rsrc_t rB[BL];
  uint32_t b_off[BL];
#pragma unroll
  for (int i = 0; i < BL; ++i) {
    // rows [lbase, lbase + 32) of the tile are loaded by chunk i; segment
    // boundaries are multiples of 32 rows, so the segment (and with it the
    // buffer resource) is uniform across the workgroup.
    const int lbase = i * (256 / CPR);
    const int lrow = tid / CPR + lbase;
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
    rB[i] = __builtin_amdgcn_make_buffer_rsrc((void*)((const T*)p.B[seg] + gofs),
                                              (short)0, p.b_bytes[seg], 0x00020000);
    b_off[i] = ok ? (uint32_t)(((int64_t)n * p.ldb + kc * CH) * sizeof(T))
                  : p.b_bytes[seg];
  }

  uint4 ra[AL], rb[BL];
  auto gload = [&](int kt) {
    const bool kval = kt * BK + kc * CH < p.K;
    const uint32_t ko = kt * BK * sizeof(T);
#pragma unroll
    for (int i = 0; i < AL; ++i)
      ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rA, kval ? a_off[i] + ko : p.a_bytes, 0, 0));
#pragma unroll
    for (int i = 0; i < BL; ++i)
      rb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rB[i], kval ? b_off[i] + ko : 0xffffffffu, 0, 0));
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int lrow = tid / CPR + i * (256 / CPR);
      *reinterpret_cast<uint4*>(As(buf) + lrow * LD + kc * CH) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int lrow = tid / CPR + i * (256 / CPR);
      *reinterpret_cast<uint4*>(Bs(buf) + lrow * LD + kc * CH) = rb[i];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (p.K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    compute_tile<T, FM, FN, LD, BK>(acc, As(cur), Bs(cur), wm * WM, wn * WN,
                                    lane);
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  const int cl = lane & 31, hi4 = (lane >> 5) * 4;
  const int lrow0 = mt * BM + wm * WM;  // tile-local (group-local) row base
  if constexpr (EPI == EPI_QKV) {
    // each wave stages its heads in its own slice of the (now idle) LDS
    constexpr int CHT = 16 / sizeof(T);
    constexpr int SLICE = (WM * (128 + CHT) > 128 * (WM + CHT)) ? WM * (128 + CHT)
                                                                 : 128 * (WM + CHT);
    static_assert(4 * SLICE <= 2 * (BM + BN) * LD, "LDS slices fit");
    T* slice = smem + wave * SLICE;
    if (p.hd == 64)
      qkv_epilogue<T, 64, FM, FN, WM>(acc, p, lrow0, nt * BN + wn * WN, lane, slice);
    else
      qkv_epilogue<T, 128, FM, FN, WM>(acc, p, lrow0, nt * BN + wn * WN, lane, slice);
    return;
  } else if constexpr (PAIRED) {
    const int ncol0 = nt * (BN / 2) + wn * (WN / 2);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN / 2; ++fn) {
        const int col = ncol0 + fn * 32 + cl;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = lrow0 + fm * 32 + (r >> 2) * 8 + hi4 + (r & 3);
          if (lr < row_count && col < p.N) {
            const float g = acc[fm][fn][r], u = acc[fm][fn + FN / 2][r];
            ((T*)p.out)[(int64_t)(row_begin + lr) * p.ldo + col] =
                from_f32<T>(silu_f(g) * u);
          }
        }
      }
    return;
  } else {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = nt * BN + wn * WN + fn * 32 + cl;
        if (col >= p.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = lrow0 + fm * 32 + (r >> 2) * 8 + hi4 + (r & 3);
          if (lr >= row_count) continue;
          const int64_t row = row_begin + lr;
          const float v = acc[fm][fn][r];
          if constexpr (EPI == EPI_STORE) {
            if (p.out_f32)
              ((float*)p.out)[row * p.ldo + col] = v;
            else
              ((T*)p.out)[row * p.ldo + col] = from_f32<T>(v);
          } else if constexpr (EPI == EPI_RESID) {
            const int64_t o = row * p.ldo + col;
            const float res = p.resid_f32 ? ((const float*)p.resid)[o]
                                          : to_f32(((const T*)p.resid)[o]);
            const float s = res + v;
            if (p.out_f32p) p.out_f32p[o] = s;
            if (p.out_model) ((T*)p.out_model)[o] = from_f32<T>(s);
            if (p.out_raw) p.out_raw[o] = v;
          } else if constexpr (EPI == EPI_RELU2) {
            const float rl = fmaxf(v, 0.f);
            ((T*)p.out)[row * p.ldo + col] = from_f32<T>(rl * rl);
          } else if constexpr (EPI == EPI_XIELU) {
            ((T*)p.out)[row * p.ldo + col] =
                from_f32<T>(xielu_f(v, p.xa_p, p.xa_n, p.xbeta, p.xeps));
          } else if constexpr (EPI == EPI_MOE_DOWN) {
            const int pair = p.row_pair[row];
            ((T*)p.out)[(int64_t)pair * p.ldo + col] =
                from_f32<T>(p.pair_weight[pair] * v);
          }
        }
      }
  }
}

// ------------------------------------------------------------ launchers

template <typename T, class TL, int EPI, bool GROUPED>
static hipError_t launch(const GemmParams& p, int max_rows, hipStream_t s) {
  const int n_per_tile = (EPI == EPI_SWIGLU) ? TL::BN / 2 : TL::BN;
  const int num_n = (p.N + n_per_tile - 1) / n_per_tile;
  if (GROUPED) {
    const int max_tiles = (max_rows + TL::BM - 1) / TL::BM + p.ngroups;
    dim3 grid(max_tiles, num_n);
    hipLaunchKernelGGL((gemm_kernel<T, TL, EPI, GROUPED>), grid, dim3(256), 0,
                       s, p);
  } else {
    const int num_m = (p.M + TL::BM - 1) / TL::BM;
    hipLaunchKernelGGL((gemm_kernel<T, TL, EPI, GROUPED>),
                       dim3(num_m * num_n), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

using TileL = Tile<bf16, 256, 256, 2, 2>;
using TileQ = Tile<bf16, 128, 256, 2, 2>;
using TileS = Tile<bf16, 128, 128, 4, 1>;
using TileF = Tile<float, 128, 128, 4, 1>;

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
    case EPI_QKV:
      if constexpr (TL::FM <= 2) return launch<T, TL, EPI_QKV, false>(p, max_rows, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm(DType dt, EpiKind epi, const GemmParams& p, int max_rows,
                hipStream_t s) {
  const bool grouped = p.gcnt != nullptr;
  if (dt == DType::F32) return dispatch_epi<float, TileF>(epi, grouped, p, max_rows, s);
  // Large tiles when they still give the chip at least one full wave of
  // workgroups; the 128x128 tile otherwise.
  const int n_per = (epi == EPI_SWIGLU) ? 128 : 256;
  if (epi == EPI_QKV) {
    // the q/k norm + rotary epilogue needs the register room of a
    // 64-row wave tile
    const long tiles_q = (long)((max_rows + 127) / 128) * ((p.N + 255) / 256);
    if (tiles_q >= 256) return dispatch_epi<bf16, TileQ>(epi, grouped, p, max_rows, s);
    return dispatch_epi<bf16, TileS>(epi, grouped, p, max_rows, s);
  }
  const long tiles_l = (long)((max_rows + 255) / 256) * ((p.N + n_per - 1) / n_per);
  if (tiles_l >= 256) return dispatch_epi<bf16, TileL>(epi, grouped, p, max_rows, s);
  return dispatch_epi<bf16, TileS>(epi, grouped, p, max_rows, s);
}

}  // namespace blk
