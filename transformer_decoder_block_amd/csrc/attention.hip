// Causal grouped-query softmax attention on gfx950 matrix cores
// (granite sheet "LlamaForCausalLM 32L-4096d", section "Implementing it":
// softmax(q k^T / sqrt(hd), mask=causal) v; GQA head map of the nnterp
// arcee/apertus notes: query head h reads KV head h / (nh/nkv); sliding
// window of the afmoe notes; key padding of the support() tables).
//
// Flash formulation.  One workgroup = 4 waves = 256 queries of one head;
// wave w owns 64 queries as two 32-query blocks.  Key tiles of 64 keys (K
// rows and the matching V^T rows) go from global memory straight into LDS
// (buffer_load ... lds), double-buffered and XOR-swizzled like the GEMM
// tiles, and are shared by the 4 waves; every K and V fragment a wave
// reads from LDS feeds the MFMAs of both of its query blocks.
//
// Each wave computes the TRANSPOSED score block S^T = K Q^T with 32x32
// MFMAs, so a lane holds one query (column l%32) and 32 of the 64 keys of
// the tile; the row max needs one exchange with lane l^32 and the
// online-softmax state (m, l) is a per-lane scalar.  The probabilities feed
// O^T += V^T P^T straight from registers: the keys a lane holds become the
// K index of that MFMA and the V^T fragment is read in the same key order.
// exp2 with the 1/sqrt(hd) scale folded into log2(e); the per-key mask
// (causal edge, window edge, padded keys, keys past the sequence) is
// applied only on tiles that need it, and the O rescale is skipped when no
// lane's running max moved.
//
// Workgroups are numbered so that the query heads sharing one KV head and
// one query block are consecutive and land on the same XCD (shared K/V in
// its L2), and the heaviest (latest) query blocks start first.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace blk {

constexpr int QW = 64;        // queries per wave (two 32-query blocks)
constexpr int QB = 4 * QW;    // queries per workgroup
constexpr int KT = 64;        // keys per tile

template <typename T, int HD>
struct AttnCfg {
  static constexpr int CH = 16 / sizeof(T);         // elements per 16 bytes
  static constexpr int KROW = HD * sizeof(T);       // bytes per K tile row
  static constexpr int VROW = KT * sizeof(T);       // bytes per V^T tile row
  static constexpr int KELEMS = KT * HD, VELEMS = HD * KT;
  static constexpr int KLOADS = KT * KROW / 1024 / 4;   // per wave
  static constexpr int VLOADS = HD * VROW / 1024 / 4;   // per wave
  static constexpr int DB = HD / 32;                // 32-row blocks of O^T
};

__device__ __forceinline__ int xcd_contiguous_a(int bid, int nblk) {
  const int per = nblk / 8, rem = nblk % 8;
  const int xcd = bid % 8, local = bid / 8;
  return (xcd < rem) ? xcd * (per + 1) + local
                     : rem * (per + 1) + (xcd - rem) * per + local;
}

// Work id of a block.  Ids are group-major, ((b * nkv + KV head) * nqb +
// qbr) * g + head of the group, where qbr = 0 is the last (heaviest) query
// block under the causal mask.  Each XCD receives a contiguous range of ids.
// When the (b, KV head) groups divide evenly over the 8 XCDs, that range is
// whole groups, and its blocks are dealt heaviest query block first across
// all of them, a longest-first list schedule; the query heads of one KV head
// stay consecutive, so they stream the same K/V tiles together.  Otherwise
// the heavy-first order holds within each group.
__device__ __forceinline__ int attn_work_id(int bid, int nblk, int ngroups, int g, int nqb) {
  int id = xcd_contiguous_a(bid, nblk);
  if (ngroups % 8 == 0) {
    const int gx = ngroups / 8, per = gx * g * nqb;
    const int x = id / per, l = id - x * per;
    const int qbr = l / (gx * g), r = l - qbr * (gx * g);
    id = x * per + ((r / g) * nqb + qbr) * g + r % g;
  }
  return id;
}

// element offset of 16-byte chunk c of row r in a swizzled tile whose rows
// hold CPR chunks
template <typename T, int CPR>
__device__ __forceinline__ int aswz(int r, int c) {
  constexpr int CH = 16 / sizeof(T);
  return r * (CPR * CH) + ((c ^ (r & 7)) * CH);
}

__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, const void* lds,
                                           uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

template <typename T, int HD>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256),
                               amdgpu_waves_per_eu(1, 1)))
attn_kernel(const AttnParams p) {
  using C = AttnCfg<T, HD>;
  constexpr int CH = C::CH, DB = C::DB;
  constexpr int KCPR = HD / CH, VCPR = KT / CH;
  __shared__ __attribute__((aligned(16))) T smem[2 * (C::KELEMS + C::VELEMS)];
  auto Ks = [&](int b) { return smem + b * C::KELEMS; };
  auto Vs = [&](int b) { return smem + 2 * C::KELEMS + b * C::VELEMS; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cl = lane & 31, hf = lane >> 5;
  const int g = p.nh / p.nkv;
  const int nqb = (p.S + QB - 1) / QB;

  // ---- which (b, head, query block)
  const int id = attn_work_id(blockIdx.x, gridDim.x, p.B * p.nkv, g, nqb);
  const int hg = id % g;
  const int qbr = (id / g) % nqb;
  const int kvh = (id / (g * nqb)) % p.nkv;
  const int b = id / (g * nqb * p.nkv);
  const int qb = nqb - 1 - qbr;  // heavy blocks first
  const int h = kvh * g + hg;
  const int q0 = qb * QB;
  const int qw = q0 + wave * QW;  // this wave's first query

  const T* Qh = (const T*)p.q + ((int64_t)b * p.nh + h) * p.S * HD;
  const T* Kh = (const T*)p.k + ((int64_t)b * p.nkv + kvh) * p.S * HD;
  const int Sp = (p.S + 63) & ~63;  // padded row length of V^T
  const T* Vh = (const T*)p.vt + ((int64_t)b * p.nkv + kvh) * HD * Sp;
  const int* mrow = p.mask ? p.mask + (int64_t)b * p.S : nullptr;
  const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Kh, (short)0, (uint32_t)((int64_t)p.S * HD * sizeof(T)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Vh, (short)0, (uint32_t)((int64_t)HD * Sp * sizeof(T)), 0x00020000);

  // ---- Q fragments (B operand of S^T = K Q^T) of both query blocks
  constexpr int NKS = (sizeof(T) == 2) ? HD / 16 : HD / 8;
  typedef typename std::conditional<sizeof(T) == 2, bf16x8, f32x4>::type QFrag;
  QFrag qf[2][NKS];
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int q = qw + qi * 32 + cl;
    const bool ok = q < p.S;
    const T* qr = Qh + (int64_t)(ok ? q : 0) * HD;
#pragma unroll
    for (int i = 0; i < NKS; ++i) {
      if constexpr (sizeof(T) == 2)  // step i: d = 16 i + 8 hf .. +7
        qf[qi][i] = ok ? *reinterpret_cast<const bf16x8*>(qr + i * 16 + hf * 8) : QFrag{};
      else                           // group i: d = hf HD/2 + 4 i .. +3
        qf[qi][i] = ok ? *reinterpret_cast<const f32x4*>(qr + hf * (HD / 2) + i * 4) : QFrag{};
    }
  }

  // ---- key tiles of the workgroup
  const int qlast = min(q0 + QB, p.S) - 1;
  const int kt_hi = qlast / KT;
  int kt_lo = 0;
  if (p.window > 0) kt_lo = max(0, q0 - p.window + 1) / KT;

  // direct-to-LDS: instruction j of wave w fills bytes [(4j+w) KiB, +1 KiB)
  // of the tile; lane L writes slot L % (row/16) of its row and fetches the
  // global chunk that the swizzle puts there
  auto issue = [&](int kt, int buf) {
    const int k0 = kt * KT;
#pragma unroll
    for (int j = 0; j < C::KLOADS; ++j) {
      constexpr int RPI = 1024 / C::KROW;  // rows per instruction
      const int row = (4 * j + wave) * RPI + lane / (C::KROW / 16);
      const int c = (lane % (C::KROW / 16)) ^ (row & 7);
      lds_load16(rK, Ks(buf) + (4 * j + wave) * 1024 / sizeof(T),
                 (uint32_t)(((int64_t)(k0 + row) * HD + c * CH) * sizeof(T)));
    }
#pragma unroll
    for (int j = 0; j < C::VLOADS; ++j) {
      constexpr int RPI = 1024 / C::VROW;
      const int d = (4 * j + wave) * RPI + lane / (C::VROW / 16);
      const int c = (lane % (C::VROW / 16)) ^ (d & 7);
      lds_load16(rV, Vs(buf) + (4 * j + wave) * 1024 / sizeof(T),
                 (uint32_t)(((int64_t)d * Sp + k0 + c * CH) * sizeof(T)));
    }
  };

  f32x16 o[2][DB];
#pragma unroll
  for (int qi = 0; qi < 2; ++qi)
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qi][i][r] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  const float sl2 = p.scale * 1.4426950408889634f;

  issue(kt_lo, 0);
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int cur = (kt - kt_lo) & 1;
    const int k0 = kt * KT;
    // keys of the tile that exist and are not padding, one bit per key
    bool kv = k0 + lane < p.S;
    if (kv && mrow) kv = mrow[k0 + lane] != 0;
    const uint64_t kvalid = __ballot(kv);
    const bool all_valid = kvalid == ~0ull;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's tile loads
    __syncthreads();
    if (k0 + KT > p.S) {
      // keys past the sequence: zero their V^T columns (the padded rows of
      // V^T hold no data)
      const int nval = p.S - k0;
      T* V = Vs(cur);
      for (int e = tid; e < HD * KT; e += 256) {
        const int d = e / KT, key = e % KT;
        if (key >= nval) V[aswz<T, VCPR>(d, key / CH) + key % CH] = from_f32<T>(0.f);
      }
      __syncthreads();
    }
    if (kt < kt_hi) issue(kt + 1, cur ^ 1);

    // skip the tile when neither of this wave's query blocks sees a key of it
    {
      const int qa = qw, qz = qw + 63;  // first and last query of the wave
      const bool any = (qa < p.S) && (k0 <= qz) &&
                       (p.window <= 0 || k0 + KT - 1 > qa - p.window);
      if (!any) continue;
    }
    const T* Kt = Ks(cur);
    const T* Vt = Vs(cur);

    // ---- S^T = K Q^T for both query blocks, K fragments shared
    f32x16 s[2][2];
#pragma unroll
    for (int qi = 0; qi < 2; ++qi)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qi][kb][r] = 0.f;
#pragma unroll
    for (int i = 0; i < NKS; ++i)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = kb * 32 + cl;
        if constexpr (sizeof(T) == 2) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kt + aswz<T, KCPR>(key, 2 * i + hf));
#pragma unroll
          for (int qi = 0; qi < 2; ++qi)
            s[qi][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qi][i], s[qi][kb], 0, 0, 0);
        } else {
          const f32x4 a = *reinterpret_cast<const f32x4*>(
              Kt + aswz<T, KCPR>(key, hf * (HD / 8) + i));
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int qi = 0; qi < 2; ++qi)
              s[qi][kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], qf[qi][i][t], s[qi][kb], 0, 0, 0);
        }
      }

    // ---- mask where needed, online softmax (per lane = per query).  The
    // probabilities go to a separate register array x; the MFMA results in
    // s are only read.
    float x[2][32];
#pragma unroll
    for (int qi = 0; qi < 2; ++qi) {
      const int myq = qw + qi * 32 + cl;
      // key kl of the tile is visible iff lo <= kl <= hi (causal edge and
      // window edge, relative to k0) and it exists and is not padding
      const int hi = myq - k0;
      const int lo = (p.window > 0) ? myq - p.window + 1 - k0 : -KT;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = kb * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
          bool vis = (kl <= hi) && (kl >= lo);
          if (!all_valid) vis = vis && ((kvalid >> kl) & 1ull);
          x[qi][kb * 16 + r] = vis ? s[qi][kb][r] : -INFINITY;
        }
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 32; ++e) tmax = fmaxf(tmax, x[qi][e]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run[qi], tmax * sl2);
      const float msub = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[qi] - msub);  // exp2(-inf) = 0
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float pe = fast_exp2(fmaf(x[qi][e], sl2, -msub));
        x[qi][e] = pe;
        psum += pe;
      }
      l_run[qi] = l_run[qi] * alpha + psum;
      const bool moved = m_new != m_run[qi];
      m_run[qi] = m_new;
      if (__ballot(moved) != 0ull) {
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[qi][i][r] *= alpha;
      }
    }

    // ---- O^T += V^T P^T over the 64 keys, V fragments shared
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int kb = st >> 1, i0 = (st & 1) * 2;
        bf16x8 pb[2];
#pragma unroll
        for (int qi = 0; qi < 2; ++qi)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pb[qi][j] = (bf16)x[qi][kb * 16 + i0 * 4 + j];
            pb[qi][4 + j] = (bf16)x[qi][kb * 16 + (i0 + 1) * 4 + j];
          }
        const int c = kb * 4 + i0;  // chunk of keys kb*32 + i0*8 .. +7
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 32 + cl;
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(Vt + aswz<T, VCPR>(d, c) + hf * 4);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(Vt + aswz<T, VCPR>(d, c + 1) + hf * 4);
          const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int qi = 0; qi < 2; ++qi)
            o[qi][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qi], o[qi][db], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = kb * 8 + 2 * i + hf;  // keys kb*32 + 8 i + 4 hf .. +3
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const f32x4 va = *reinterpret_cast<const f32x4*>(Vt + aswz<T, VCPR>(db * 32 + cl, c));
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int qi = 0; qi < 2; ++qi)
                o[qi][db] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[j], x[qi][kb * 16 + i * 4 + j],
                                                                 o[qi][db], 0, 0, 0);
          }
        }
    }
  }

  // ---- normalise, gate, store premix [B*S, nh*hd]
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int myq = qw + qi * 32 + cl;
    const float l_tot = l_run[qi] + __shfl_xor(l_run[qi], 32, 64);
    if (myq >= p.S) continue;
    const float inv_l = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
    const int64_t tok = (int64_t)b * p.S + myq;
    T* orow = (T*)p.out + tok * ((int64_t)p.nh * HD) + h * HD;
    // gate factors read before the first store (see the bf16 kernel)
    const bool per_channel = p.gate && p.G != p.nh;
    const float gh = (p.gate && !per_channel) ? p.gate[tok * p.G + h] : 1.0f;
    float gv[DB * 16];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 g4 = make_float4(gh, gh, gh, gh);
        if (per_channel)
          g4 = *reinterpret_cast<const float4*>(p.gate + tok * p.G + h * HD + db * 32 + i * 8 +
                                                 hf * 4);
        gv[(db * 4 + i) * 4 + 0] = g4.x;
        gv[(db * 4 + i) * 4 + 1] = g4.y;
        gv[(db * 4 + i) * 4 + 2] = g4.z;
        gv[(db * 4 + i) * 4 + 3] = g4.w;
      }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + i * 8 + hf * 4;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = o[qi][db][i * 4 + j] * inv_l * gv[(db * 4 + i) * 4 + j];
        if constexpr (sizeof(T) == 2) {
          uint2 w;
          w.x = pack2_bf16(v[0], v[1]);
          w.y = pack2_bf16(v[2], v[3]);
          *reinterpret_cast<uint2*>(orow + d0) = w;
        } else {
          *reinterpret_cast<float4*>(orow + d0) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel.  One workgroup = 4 waves = 128 queries of one head; wave w
// owns 32 queries.  Registers are capped so that two workgroups (head_dim
// 128) or four (head_dim 64) share a CU and one's softmax overlaps the
// others' MFMAs.
//
// Per 64-key tile a wave computes S^T = K Q^T (lane = query l%32, 32 of the
// 64 keys), then the online softmax, then O^T += V^T P^T with P taken
// straight from the registers.  For that the V^T rows hold the keys of each
// aligned group of 16 in the order 0-3, 8-11, 4-7, 12-15 (the QKV epilogue
// writes them so): the 8 keys a lane holds for one 16-key MFMA step are then
// one 16-byte chunk of the row.
//
// Masking is decided per wave and tile from scalars: a tile that every query
// of the wave sees whole (below the causal edge, inside the window, no
// padding) takes no mask at all; the others compare each key against the
// lane's bounds and the tile's padding bits, branch-free.  The running
// maximum is raised only when a tile's maximum exceeds it by more than
// 2^TAU_L2 in the exp2 domain (probabilities stay <= 2^TAU_L2), so the O
// rescale is rare.
constexpr int BQW = 32;           // queries per wave
constexpr int BNW = 4;            // waves per workgroup
constexpr int BQB = BQW * BNW;    // queries per workgroup
constexpr float TAU_L2 = 8.0f;

template <int HD>
struct BCfg {
  static constexpr int KBYTES = KT * HD * 2;       // K tile, rows = keys
  static constexpr int VBYTES = HD * KT * 2;       // V^T tile, rows = d
  static constexpr int KLD = KBYTES / 1024 / BNW;  // direct loads per wave
  static constexpr int VLD = VBYTES / 1024 / BNW;
  static constexpr int NKS = HD / 16;              // QK k-steps
  static constexpr int DB = HD / 32;               // 32-row blocks of O^T
};

// LDS slot of 16-byte chunk c of row r.  K rows of 256 bytes span all 64
// banks, so 16 consecutive rows need 16 different slots; rows of 128 bytes
// (K at hd 64, V^T) pair up as even/odd halves of the banks.
template <int ROWBYTES>
__device__ __forceinline__ int bslot(int r, int c) {
  if constexpr (ROWBYTES == 256) return c ^ (r & 15);
  else return c ^ ((r >> 1) & 7);
}

// (v of this lane) op (v of lane l^32), in every lane
__device__ __forceinline__ float xhalf_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// head_dim 64 needs fewer registers (at most 128) and half the LDS (32 KiB
// per workgroup): four workgroups per CU
template <int HD>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256),
                               amdgpu_waves_per_eu(HD == 64 ? 4 : 2, HD == 64 ? 4 : 2)))
attn_bf16_kernel(const AttnParams p) {
  using C = BCfg<HD>;
  constexpr int NKS = C::NKS, DB = C::DB;
  constexpr int KRB = HD * 2;  // K row bytes
  __shared__ __attribute__((aligned(1024))) char smem[2 * (C::KBYTES + C::VBYTES)];
  auto Kb = [&](int b) { return smem + b * C::KBYTES; };
  auto Vb = [&](int b) { return smem + 2 * C::KBYTES + b * C::VBYTES; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cl = lane & 31, hf = lane >> 5;
  const int g = p.nh / p.nkv;
  const int nqb = (p.S + BQB - 1) / BQB;

  // ---- which (b, KV head, query block, head of the group)
  const int id = attn_work_id(blockIdx.x, gridDim.x, p.B * p.nkv, g, nqb);
  const int hg = id % g;
  const int qbr = (id / g) % nqb;
  const int kvh = (id / (g * nqb)) % p.nkv;
  const int b = id / (g * nqb * p.nkv);
  const int qb = nqb - 1 - qbr;  // heavy blocks first
  const int h = kvh * g + hg;
  const int q0 = qb * BQB;
  const int qw = q0 + wave * BQW;           // the wave's first query
  const int qz = min(qw + BQW, p.S) - 1;    // its last real query
  const int myq = qw + cl;

  const bf16* Qh = (const bf16*)p.q + ((int64_t)b * p.nh + h) * p.S * HD;
  const bf16* Kh = (const bf16*)p.k + ((int64_t)b * p.nkv + kvh) * p.S * HD;
  const int Sp = (p.S + 63) & ~63;
  const bf16* Vh = (const bf16*)p.vt + ((int64_t)b * p.nkv + kvh) * HD * Sp;
  const int* mrow = p.mask ? p.mask + (int64_t)b * p.S : nullptr;
  const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Kh, (short)0, (uint32_t)((int64_t)p.S * HD * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Vh, (short)0, (uint32_t)((int64_t)HD * Sp * 2), 0x00020000);

  // ---- Q fragments: step i holds d = 16 i + 8 hf .. +7 of the lane's query
  bf16x8 qf[NKS];
  {
    const bool ok = myq < p.S;
    const bf16* qr = Qh + (int64_t)(ok ? myq : 0) * HD + hf * 8;
#pragma unroll
    for (int i = 0; i < NKS; ++i)
      qf[i] = ok ? *reinterpret_cast<const bf16x8*>(qr + i * 16) : bf16x8{};
  }

  // ---- key tiles of the workgroup
  const int kt_hi = (min(q0 + BQB, p.S) - 1) / KT;
  const int kt_lo = (p.window > 0) ? max(0, q0 - p.window + 1) / KT : 0;

  // direct-to-LDS: instruction j of wave w fills bytes [(BNW j + w) KiB, +1)
  // of the tile; lane L writes slot L % (row/16) of its row and fetches the
  // global chunk the swizzle puts there.  The padding mask of the tile's
  // 64 keys is fetched alongside (lane = key).
  int mnext = 1;
  auto issue = [&](int kt, int buf) {
    const int k0 = kt * KT;
#pragma unroll
    for (int j = 0; j < C::KLD; ++j) {
      constexpr int RPI = 1024 / KRB;
      const int blk = BNW * j + wave;
      const int row = blk * RPI + lane / (KRB / 16);
      const int c = bslot<KRB>(row, lane % (KRB / 16));
      lds_load16(rK, Kb(buf) + blk * 1024, (uint32_t)(((k0 + row) * HD + c * 8) * 2));
    }
#pragma unroll
    for (int j = 0; j < C::VLD; ++j) {
      const int blk = BNW * j + wave;
      const int d = blk * 8 + lane / 8;
      const int c = bslot<128>(d, lane % 8);
      lds_load16(rV, Vb(buf) + blk * 1024, (uint32_t)((d * Sp + k0 + c * 8) * 2));
    }
    if (mrow) mnext = (k0 + lane < p.S) ? mrow[k0 + lane] : 1;
  };

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  // Head width 64 leaves the matrix pipe half idle while the lanes run the
  // softmax, so there the row sums come from one 16x16x32 MFMA per 16-key
  // step instead of 32 adds per tile: D = Sel P^T, with P^T (16 keys x 32
  // queries) read as B (32 k x 16 columns; column j holds queries j and
  // j + 16, each in two 8-key blocks of k).  Row i of Sel selects the
  // blocks of query j (rows 0, 8) or of query j + 16 (rows 4, 12), the
  // rows that D places in element 0 of lanes j, j + 16, j + 32, j + 48: so
  // lacc[0] of every lane is its own query's sum of the probabilities as
  // rounded for P V^T.  The other rows of Sel are 0.
  constexpr bool MSUM = HD == 64;
  bf16x8 sel;
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
  {
    const int i16 = lane & 15, kb = lane >> 4;
    const bool on = ((i16 == 0 || i16 == 8) && !(kb & 1)) || ((i16 == 4 || i16 == 12) && (kb & 1));
#pragma unroll
    for (int t = 0; t < 8; ++t) sel[t] = on ? (bf16)1.0f : (bf16)0.0f;
  }
  const float sl2 = p.scale * 1.4426950408889634f;

  issue(kt_lo, 0);
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int cur = (kt - kt_lo) & 1;
    const int k0 = kt * KT;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's tile loads
    __syncthreads();
    const uint64_t kvalid = mrow ? __ballot(mnext != 0) : ~0ull;
    if (k0 + KT > p.S) {
      // keys past the sequence: zero their (permuted) V^T columns
      const int nval = p.S - k0;
      char* V = Vb(cur);
      for (int e = tid; e < HD * KT; e += 256) {
        const int d = e / KT, pos = e % KT;
        // position -> key within an aligned group of 16: swap bits 2 and 3
        const int key = (pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1);
        if (key >= nval) {
          const int c = bslot<128>(d, pos / 8);
          *reinterpret_cast<bf16*>(V + d * 128 + c * 16 + (pos % 8) * 2) = (bf16)0.f;
        }
      }
      __syncthreads();
    }
    if (kt < kt_hi) issue(kt + 1, cur ^ 1);

    // wave-uniform tile class
    const bool any = (qw < p.S) && (k0 <= qz) &&
                     (p.window <= 0 || k0 + KT - 1 >= qw - p.window + 1);
    if (!any) continue;
    const bool full = (k0 + KT - 1 <= qw) &&
                      (p.window <= 0 || k0 >= qz - p.window + 1) && (kvalid == ~0ull);

    // ---- S^T = K Q^T: two 32-key blocks
    const char* Kt = Kb(cur);
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
    for (int i = 0; i < NKS; ++i) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(
          Kt + cl * KRB + bslot<KRB>(cl, 2 * i + hf) * 16);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(
          Kt + (32 + cl) * KRB + bslot<KRB>(32 + cl, 2 * i + hf) * 16);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[i], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[i], s1, 0, 0, 0);
    }
    // lane holds keys kb*32 + 8 (r/4) + 4 hf + r%4 of its query
    float x[32];
#pragma unroll
    for (int r = 0; r < 16; ++r) { x[r] = s0[r]; x[16 + r] = s1[r]; }
    if (!full) {
      // bit kl of vis: key k0 + kl is visible to the lane's query (causal
      // bound hi, window bound lo, padding); shifted so that each score's
      // bit sits at a constant position
      const int hi = myq - k0;
      const int lo = (p.window > 0) ? myq - p.window + 1 - k0 : 0;
      uint64_t vis = kvalid;
      vis &= hi < 0 ? 0ull : (hi >= 63 ? ~0ull : (2ull << hi) - 1);
      vis &= lo <= 0 ? ~0ull : (lo > 63 ? 0ull : ~((1ull << lo) - 1));
      vis >>= 4 * hf;
      const uint32_t w0 = (uint32_t)vis, w1 = (uint32_t)(vis >> 32);
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int r = e & 15;
        const uint32_t m = 1u << ((r >> 2) * 8 + (r & 3));
        x[e] = ((e < 16 ? w0 : w1) & m) ? x[e] : -INFINITY;
      }
    }

    // ---- online softmax, one query per lane (keys split with lane l^32)
    float tmax = x[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) tmax = fmaxf(tmax, x[e]);
    const float mt = xhalf_max(tmax) * sl2;
    if (__ballot(mt > m_run + TAU_L2) != 0ull) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
      if constexpr (MSUM) lacc[0] *= alpha;
      else l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      m_run = m_new;
    }
    const float msub = (m_run == -INFINITY) ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      x[e] = fast_exp2(fmaf(x[e], sl2, -msub));
      if constexpr (!MSUM) psum += x[e];
    }
    if constexpr (!MSUM) l_run += psum;

    // ---- O^T += V^T P^T, 16 keys per step
    const char* Vt = Vb(cur);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 pb;
#pragma unroll
      for (int t = 0; t < 8; ++t) pb[t] = (bf16)x[j * 8 + t];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 32 + cl;
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(
            Vt + d * 128 + bslot<128>(d, 2 * j + hf) * 16);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
      }
      if constexpr (MSUM) lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb, lacc, 0, 0, 0);
    }
  }

  // ---- normalise, gate, store premix [B*S, nh*hd]
  const float l_tot = MSUM ? lacc[0] : xhalf_sum(l_run);
  if (myq >= p.S) return;
  const float inv_l = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
  const int64_t tok = (int64_t)b * p.S + myq;
  bf16* orow = (bf16*)p.out + tok * ((int64_t)p.nh * HD) + h * HD;
  // The gate factor of each value the lane stores (one per head, or one per
  // channel), all read before the first store: a load between the stores
  // would make every store wait for the ones before it.
  float gv[DB * 16];
  if (p.gate && p.G != p.nh) {
    const float* gr = p.gate + tok * p.G + h * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 g4 = *reinterpret_cast<const float4*>(gr + db * 32 + i * 8 + hf * 4);
        gv[(db * 4 + i) * 4 + 0] = g4.x;
        gv[(db * 4 + i) * 4 + 1] = g4.y;
        gv[(db * 4 + i) * 4 + 2] = g4.z;
        gv[(db * 4 + i) * 4 + 3] = g4.w;
      }
  } else {
    const float gh = p.gate ? p.gate[tok * p.G + h] : 1.0f;
#pragma unroll
    for (int e = 0; e < DB * 16; ++e) gv[e] = gh;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = db * 32 + i * 8 + hf * 4;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = o[db][i * 4 + j] * inv_l * gv[(db * 4 + i) * 4 + j];
      uint2 w;
      w.x = pack2_bf16(v[0], v[1]);
      w.y = pack2_bf16(v[2], v[3]);
      *reinterpret_cast<uint2*>(orow + d0) = w;
    }
}

// The attention_scores tap: q.k / sqrt(hd) where visible, -inf elsewhere.
template <typename T, int HD>
__global__ void __launch_bounds__(256) scores_kernel(const AttnParams p, float* scores) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int i = blockIdx.y;
  const int bh = blockIdx.z;
  const int b = bh / p.nh, h = bh % p.nh;
  if (j >= p.S) return;
  const int kvh = h / (p.nh / p.nkv);
  const T* qr = (const T*)p.q + (((int64_t)b * p.nh + h) * p.S + i) * HD;
  const T* kr = (const T*)p.k + (((int64_t)b * p.nkv + kvh) * p.S + j) * HD;
  bool vis = j <= i;
  if (p.mask && p.mask[(int64_t)b * p.S + j] == 0) vis = false;
  if (p.window > 0 && i - j >= p.window) vis = false;
  float acc = 0.f;
  if (vis) {
#pragma unroll 8
    for (int d = 0; d < HD; ++d) acc += to_f32(qr[d]) * to_f32(kr[d]);
  }
  scores[(((int64_t)b * p.nh + h) * p.S + i) * p.S + j] = vis ? acc * p.scale : -INFINITY;
}

// The attention_probabilities tap: softmax over each query row of the
// visible keys' scores (q.k / sqrt(hd)), 0 at masked keys and on rows with
// no visible key.  One workgroup per row; the output row holds the scores,
// then their exponentials, then the probabilities.
template <typename T, int HD>
__global__ void __launch_bounds__(256) probs_kernel(const AttnParams p, float* probs) {
  __shared__ float red[4];
  const int i = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / p.nh, h = bh % p.nh;
  const int kvh = h / (p.nh / p.nkv);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const T* qr = (const T*)p.q + (((int64_t)b * p.nh + h) * p.S + i) * HD;
  float* row = probs + (((int64_t)b * p.nh + h) * p.S + i) * p.S;
  float mx = -INFINITY;
  for (int j = tid; j < p.S; j += 256) {
    const T* kr = (const T*)p.k + (((int64_t)b * p.nkv + kvh) * p.S + j) * HD;
    bool vis = j <= i;
    if (p.mask && p.mask[(int64_t)b * p.S + j] == 0) vis = false;
    if (p.window > 0 && i - j >= p.window) vis = false;
    float acc = -INFINITY;
    if (vis) {
      acc = 0.f;
      for (int d = 0; d < HD; ++d) acc += to_f32(qr[d]) * to_f32(kr[d]);
      acc *= p.scale;
    }
    row[j] = acc;
    mx = fmaxf(mx, acc);
  }
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (int j = tid; j < p.S; j += 256) {
    const float e = (mx == -INFINITY) ? 0.f : expf(row[j] - mx);
    row[j] = e;
    sum += e;
  }
  sum = wave_sum(sum);
  if (lane == 0) red[wv] = sum;
  __syncthreads();
  sum = red[0] + red[1] + red[2] + red[3];
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  for (int j = tid; j < p.S; j += 256) row[j] *= inv;
}

// The attention_values tap: [B, nkv, S, hd] from the transposed V^T rows
// (bf16 rows hold each aligned group of 16 keys in the order 0-3, 8-11,
// 4-7, 12-15).
template <typename T, int HD>
__global__ void __launch_bounds__(256) values_kernel(const AttnParams p, T* v) {
  const int64_t n = (int64_t)p.B * p.nkv * p.S * HD;
  const int Sp = (p.S + 63) & ~63;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int d = (int)(e % HD);
    const int64_t r = e / HD;
    const int sk = (int)(r % p.S);
    const int64_t bk = r / p.S;  // b * nkv + kv head
    const int pos = (sizeof(T) == 2) ? ((sk & ~12) | ((sk & 4) << 1) | ((sk & 8) >> 1)) : sk;
    v[e] = ((const T*)p.vt)[(bk * HD + d) * Sp + pos];
  }
}

template <typename T, int HD>
static hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  const int nqb = (p.S + QB - 1) / QB;
  const int nblk = p.B * p.nh * nqb;
  hipLaunchKernelGGL((attn_kernel<T, HD>), dim3(nblk), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int HD>
static hipError_t launch_attn_bf16(const AttnParams& p, hipStream_t s) {
  const int nqb = (p.S + BQB - 1) / BQB;
  const int nblk = p.B * p.nh * nqb;
  hipLaunchKernelGGL((attn_bf16_kernel<HD>), dim3(nblk), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t attention(DType dt, const AttnParams& p, hipStream_t s) {
  if (dt == DType::BF16)
    return p.hd == 64 ? launch_attn_bf16<64>(p, s) : launch_attn_bf16<128>(p, s);
  return p.hd == 64 ? launch_attn<float, 64>(p, s) : launch_attn<float, 128>(p, s);
}

hipError_t attention_scores(DType dt, const AttnParams& p, float* scores, hipStream_t s) {
  dim3 grid((p.S + 255) / 256, p.S, p.B * p.nh);
  if (dt == DType::BF16) {
    if (p.hd == 64) hipLaunchKernelGGL((scores_kernel<bf16, 64>), grid, dim3(256), 0, s, p, scores);
    else hipLaunchKernelGGL((scores_kernel<bf16, 128>), grid, dim3(256), 0, s, p, scores);
  } else {
    if (p.hd == 64) hipLaunchKernelGGL((scores_kernel<float, 64>), grid, dim3(256), 0, s, p, scores);
    else hipLaunchKernelGGL((scores_kernel<float, 128>), grid, dim3(256), 0, s, p, scores);
  }
  return hipGetLastError();
}

}  // namespace blk

namespace blk {

hipError_t attention_probs(DType dt, const AttnParams& p, float* probs, hipStream_t s) {
  dim3 grid(p.S, p.B * p.nh);
  if (dt == DType::BF16) {
    if (p.hd == 64) hipLaunchKernelGGL((probs_kernel<bf16, 64>), grid, dim3(256), 0, s, p, probs);
    else hipLaunchKernelGGL((probs_kernel<bf16, 128>), grid, dim3(256), 0, s, p, probs);
  } else {
    if (p.hd == 64) hipLaunchKernelGGL((probs_kernel<float, 64>), grid, dim3(256), 0, s, p, probs);
    else hipLaunchKernelGGL((probs_kernel<float, 128>), grid, dim3(256), 0, s, p, probs);
  }
  return hipGetLastError();
}

hipError_t attention_values(DType dt, const AttnParams& p, void* v, hipStream_t s) {
  const int64_t n = (int64_t)p.B * p.nkv * p.S * p.hd;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 65536);
  if (dt == DType::BF16) {
    if (p.hd == 64) hipLaunchKernelGGL((values_kernel<bf16, 64>), dim3(blocks), dim3(256), 0, s, p, (bf16*)v);
    else hipLaunchKernelGGL((values_kernel<bf16, 128>), dim3(blocks), dim3(256), 0, s, p, (bf16*)v);
  } else {
    if (p.hd == 64) hipLaunchKernelGGL((values_kernel<float, 64>), dim3(blocks), dim3(256), 0, s, p, (float*)v);
    else hipLaunchKernelGGL((values_kernel<float, 128>), dim3(blocks), dim3(256), 0, s, p, (float*)v);
  }
  return hipGetLastError();
}

}  // namespace blk
