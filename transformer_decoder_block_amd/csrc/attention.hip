// Causal grouped-query softmax attention on gfx950 matrix cores
// (granite sheet "LlamaForCausalLM 32L-4096d", section "Implementing it":
// softmax(q k^T / sqrt(hd), mask=causal) v; GQA head map of the nnterp
// arcee/apertus notes: query head h reads KV head h / (nh/nkv); sliding
// window of the afmoe notes; key padding of the support() tables).
//
// Flash formulation: one workgroup = 4 waves = 128 queries of one head;
// wave w owns 32 queries.  Key tiles of 64 keys (K rows and the matching
// V^T columns) are staged through LDS, double-buffered, and shared by the
// 4 waves.  Each wave computes the TRANSPOSED score block S^T = K Q^T with
// 32x32 MFMAs, so a lane holds one query (column l%32) and 32 of the 64
// keys of the tile in registers; the row max needs one exchange with lane
// l^32 and the online-softmax state (m, l) is a per-lane scalar.  The
// probabilities feed O^T += V^T P^T directly from registers: the keys a
// lane holds become the K index of that MFMA, and the V^T fragment is
// read from LDS in the same key order.  Softmax uses exp2 with the
// 1/sqrt(hd) scale folded into log2(e).
//
// Workgroups are numbered so that the query heads sharing one KV head and
// one query block are consecutive and land on the same XCD (shared K/V in
// its L2), and the heaviest (latest) query blocks start first.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace blk {

constexpr int QB = 128;  // queries per workgroup
constexpr int KT = 64;   // keys per tile

template <typename T, int HD>
struct AttnCfg {
  static constexpr int CH = 16 / sizeof(T);          // elements per 16 bytes
  static constexpr int KLD = HD + CH;                // K tile row (keys)
  static constexpr int VLD = KT + CH;                // V^T tile row (dims)
  static constexpr int KCH = KT * HD / CH / 256;     // K chunks per thread
  static constexpr int VCH = HD * KT / CH / 256;     // V^T chunks per thread
  static constexpr int DB = HD / 32;                 // 32-row blocks of O^T
};

__device__ __forceinline__ int xcd_contiguous_a(int bid, int nblk) {
  const int per = nblk / 8, rem = nblk % 8;
  const int xcd = bid % 8, local = bid / 8;
  return (xcd < rem) ? xcd * (per + 1) + local
                     : rem * (per + 1) + (xcd - rem) * per + local;
}

template <typename T, int HD>
__global__ void __launch_bounds__(256) attn_kernel(const AttnParams p) {
  using C = AttnCfg<T, HD>;
  constexpr int CH = C::CH, KLD = C::KLD, VLD = C::VLD, KCH = C::KCH,
                VCH = C::VCH, DB = C::DB;
  __shared__ __attribute__((aligned(16))) T Ks[2][KT * KLD];
  __shared__ __attribute__((aligned(16))) T Vs[2][HD * VLD];
  __shared__ int Ms[2][KT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cl = lane & 31, hf = lane >> 5;
  const int g = p.nh / p.nkv;
  const int nqb = (p.S + QB - 1) / QB;

  // ---- which (b, head, query block)
  const int id = xcd_contiguous_a(blockIdx.x, gridDim.x);
  const int hg = id % g;
  const int qbr = (id / g) % nqb;
  const int kvh = (id / (g * nqb)) % p.nkv;
  const int b = id / (g * nqb * p.nkv);
  const int qb = nqb - 1 - qbr;  // heavy blocks first
  const int h = kvh * g + hg;
  const int q0 = qb * QB;
  const int qw = q0 + wave * 32;  // this wave's first query
  const int myq = qw + cl;        // this lane's query

  const T* Qh = (const T*)p.q + ((int64_t)b * p.nh + h) * p.S * HD;
  const T* Kh = (const T*)p.k + ((int64_t)b * p.nkv + kvh) * p.S * HD;
  const int Sp = (p.S + 63) & ~63;  // padded row length of V^T
  const T* Vh = (const T*)p.vt + ((int64_t)b * p.nkv + kvh) * HD * Sp;
  const int* mrow = p.mask ? p.mask + (int64_t)b * p.S : nullptr;

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers
  constexpr int QREGS = (sizeof(T) == 2) ? HD / 16 : HD / 8;
  typedef typename std::conditional<sizeof(T) == 2, bf16x8, f32x4>::type QFrag;
  QFrag qf[QREGS];
  {
    const bool ok = myq < p.S;
    const T* qr = Qh + (int64_t)(ok ? myq : 0) * HD;
#pragma unroll
    for (int i = 0; i < QREGS; ++i) {
      if constexpr (sizeof(T) == 2) {
        // step i covers d = 16 i + 8 hf .. +7
        qf[i] = ok ? *reinterpret_cast<const bf16x8*>(qr + i * 16 + hf * 8) : QFrag{};
      } else {
        // group i covers d = hf*HD/2 + 4 i .. +3 (permuted K order)
        qf[i] = ok ? *reinterpret_cast<const f32x4*>(qr + hf * (HD / 2) + i * 4) : QFrag{};
      }
    }
  }

  // ---- key tile range of the workgroup
  const int qlast = min(q0 + QB, p.S) - 1;
  const int kt_hi = qlast / KT;
  int kt_lo = 0;
  if (p.window > 0) kt_lo = max(0, q0 - p.window + 1) / KT;

  uint4 rk[KCH], rv[VCH];
  int rm = 1;
  auto gload = [&](int kt) {
    const int k0 = kt * KT;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * 256;
      const int key = c / (HD / CH), dc = c % (HD / CH);
      rk[i] = (k0 + key < p.S)
                  ? *reinterpret_cast<const uint4*>(Kh + (int64_t)(k0 + key) * HD + dc * CH)
                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + i * 256;
      const int d = c / (KT / CH), kc = c % (KT / CH);
      const int key = k0 + kc * CH;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (key < p.S) {
        v = *reinterpret_cast<const uint4*>(Vh + (int64_t)d * Sp + key);
        if (key + CH > p.S) {  // zero the padding past the sequence
          uint32_t w[4] = {v.x, v.y, v.z, v.w};
          const int valid = p.S - key;  // 1..CH-1 elements
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (sizeof(T) == 2) {
              if (2 * e >= valid) w[e] = 0;
              else if (2 * e + 1 >= valid) w[e] &= 0xffffu;
            } else {
              if (e >= valid) w[e] = 0;
            }
          }
          v = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
      rv[i] = v;
    }
    if (tid < KT) {
      const int key = k0 + tid;
      rm = (key < p.S) && (!mrow || mrow[key] != 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * 256;
      const int key = c / (HD / CH), dc = c % (HD / CH);
      *reinterpret_cast<uint4*>(&Ks[buf][key * KLD + dc * CH]) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + i * 256;
      const int d = c / (KT / CH), kc = c % (KT / CH);
      *reinterpret_cast<uint4*>(&Vs[buf][d * VLD + kc * CH]) = rv[i];
    }
    if (tid < KT) Ms[buf][tid] = rm;
  };

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale * 1.4426950408889634f;

  gload(kt_lo);
  sstore(0);
  __syncthreads();
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int cur = (kt - kt_lo) & 1;
    if (kt < kt_hi) gload(kt + 1);
    const int k0 = kt * KT;
    // does this wave see any key of the tile?
    const bool active = (qw < p.S) && (k0 <= qw + 31) &&
                        (p.window <= 0 || k0 + KT - 1 > qw - p.window);
    if (active) {
      const T* Kt = Ks[cur];
      const T* Vt = Vs[cur];
      // ---- S^T blocks: keys kb*32.. x this wave's 32 queries
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        const T* krow = Kt + (kb * 32 + cl) * KLD;
#pragma unroll
        for (int i = 0; i < QREGS; ++i) {
          if constexpr (sizeof(T) == 2) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + i * 16 + hf * 8);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[i], s[kb], 0, 0, 0);
          } else {
            const f32x4 a = *reinterpret_cast<const f32x4*>(krow + hf * (HD / 2) + i * 4);
#pragma unroll
            for (int t = 0; t < 4; ++t)
              s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], qf[i][t], s[kb], 0, 0, 0);
          }
        }
      }
      // ---- mask, scale, online softmax (per lane = per query)
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = kb * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
          const int key = k0 + kl;
          const bool vis = (key <= myq) && Ms[cur][kl] &&
                           (p.window <= 0 || myq - key < p.window);
          const float v = vis ? s[kb][r] * sl2 : -INFINITY;
          s[kb][r] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
      const float msub = (m_new == -INFINITY) ? 0.f : m_new;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(s[kb][r] - msub);  // exp2(-inf) = 0
          s[kb][r] = e;
          psum += e;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      // ---- O^T += V^T P^T over the 64 keys of the tile
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int kb = st >> 1, i0 = (st & 1) * 2;
          bf16x8 pb;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pb[j] = (bf16)s[kb][i0 * 4 + j];
            pb[4 + j] = (bf16)s[kb][(i0 + 1) * 4 + j];
          }
          const int key_a = kb * 32 + i0 * 8 + hf * 4;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const T* vrow = Vt + (db * 32 + cl) * VLD;
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow + key_a);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + key_a + 8);
            const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key_a = kb * 32 + i * 8 + hf * 4;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const f32x4 va = *reinterpret_cast<const f32x4*>(Vt + (db * 32 + cl) * VLD + key_a);
#pragma unroll
              for (int j = 0; j < 4; ++j)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[j], s[kb][i * 4 + j], o[db], 0, 0, 0);
            }
          }
      }
    }
    if (kt < kt_hi) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- normalise, gate, store premix [B*S, nh*hd]
  if (myq >= p.S) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv_l = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
  const int64_t tok = (int64_t)b * p.S + myq;
  float gh = 1.0f;
  if (p.gate && p.G == p.nh) gh = p.gate[tok * p.G + h];
  T* orow = (T*)p.out + tok * ((int64_t)p.nh * HD) + h * HD;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = db * 32 + i * 8 + hf * 4;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float gv = gh;
        if (p.gate && p.G != p.nh) gv = p.gate[tok * p.G + h * HD + d0 + j];
        v[j] = o[db][i * 4 + j] * inv_l * gv;
      }
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

template <typename T, int HD>
static hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  const int nqb = (p.S + QB - 1) / QB;
  const int nblk = p.B * p.nh * nqb;
  hipLaunchKernelGGL((attn_kernel<T, HD>), dim3(nblk), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t attention(DType dt, const AttnParams& p, hipStream_t s) {
  if (dt == DType::BF16)
    return p.hd == 64 ? launch_attn<bf16, 64>(p, s) : launch_attn<bf16, 128>(p, s);
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
