// Non-causal local-Q / global-KV multi-head attention, bf16 in/out, for gfx950.
//
// The problem is the one an AllGather-KV rank hands to its attention backend
// (vllm-omni PR #7641, "Compose Ulysses with AllGather-KV as a 2D diffusion
// SP", commit message): this rank's query rows against every key row of the
// same heads, with an optional per-batch key-validity mask (that PR's review-fix
// commits: a [B, K] mask, True = attend).  Head dims 64 and 128.
//
// Design (one workgroup = 4 waves = 128 query rows of one (batch, head)):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16.  With keys as the MFMA row
//    dimension, each lane owns one query column and 16 key rows per 32x32
//    block, so the softmax row max and row sum are in-lane reductions plus one
//    swap with lane^32.  Q stays in registers (the B operand) for the whole
//    key loop.
//  * O^T = V^T P^T on the same MFMA.  The probabilities leave the S^T
//    accumulators already in B-operand position; the 16 keys of each MFMA step
//    are taken in the order the accumulator layout delivers them, and V is
//    written into LDS transposed ([d][key]) in that same key order, so every
//    operand is one 16-byte LDS read.
//  * K and V tiles of 64 keys are double-buffered in LDS: tile t+1 is fetched
//    from HBM into registers while tile t is in the MFMAs, then stored to the
//    other buffer; one barrier per tile.
//  * Online softmax in fp32 with exp2 (scale * log2 e folded into one FMA).
//    The running max is only raised when a tile's max exceeds it by more than
//    2^8 in probability terms, so the O rescale is rare; the quotient is
//    unchanged because numerator and denominator share the stale max.
//  * Key tail and key mask: a per-tile additive bias row (0 or -inf) in LDS,
//    applied only to tiles that need it.
//  * Workgroups are numbered so that all query tiles of one (batch, head) land
//    on the same XCD, whose L2 then serves that head's K/V to all of them.

#include <hip/hip_runtime.h>

#include <cmath>

#include "cp_common.hpp"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kNumXcd = 8;

template <int D>
struct Cfg {
  static constexpr int BM = 32 * kWaves;     // query rows per workgroup
  static constexpr int BN = 64;              // keys per tile
  static constexpr int KP = D + 8;           // K row pitch in LDS (elements); +16 B vs bank conflicts
  static constexpr int VP = BN + 8;          // V^T row pitch in LDS (elements)
  static constexpr int K_ELEMS = BN * KP;
  static constexpr int V_ELEMS = D * VP;
  static constexpr int VD = D / 8;           // 16-byte vectors per head row
  static constexpr int LOADS = BN * VD / kThreads;   // K (and V) vectors per thread per tile
  static constexpr int KPT = LOADS;          // keys per thread in the V transpose
  static constexpr int GROUPS = BN / KPT;    // key groups per 16-byte column of V
  static constexpr int DB = D / 32;          // 32-row blocks of O^T
  static constexpr int KS = D / 16;          // 16-wide reduction steps of Q K^T
  static_assert(LOADS * kThreads == BN * VD, "tile must split evenly");
  static_assert(GROUPS * VD == kThreads, "V transpose mapping must cover the tile");
  static_assert(KPT == 2 || KPT == 4, "V transpose writes 2 or 4 keys per store");
};

// Position of key offset `ko` (0..BN-1) inside a V^T row: bits 2 and 3 swapped,
// which is the order in which a lane's accumulator rows enter one MFMA step.
__device__ __forceinline__ int vt_pos(int ko) {
  return (ko & ~12) | ((ko & 4) << 1) | ((ko & 8) >> 1);
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}
__device__ __forceinline__ uint32_t dword_of(const uint4& v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

struct AttnArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const uint8_t* mask;
  __bf16* o;
  int B, Sq, Skv, H;
  int m_tiles;       // ceil(Sq / BM)
  int n_work;        // B * H * m_tiles
  float sc;          // scale * log2(e)
};

template <int D>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd_kernel(AttnArgs a) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (C::K_ELEMS + C::V_ELEMS)];
  __shared__ __attribute__((aligned(16))) float kbias[2][C::BN];

  // ---- XCD-aware work numbering: consecutive logical tiles share an XCD.
  const int pid = blockIdx.x;
  const int n = a.n_work;
  const int per = n / kNumXcd, rem = n % kNumXcd;
  const int xcd = pid % kNumXcd, local = pid / kNumXcd;
  const int work = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int mt = work % a.m_tiles;
  const int bh = work / a.m_tiles;
  const int h = bh % a.H;
  const int b = bh / a.H;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;  // which half of the wave: selects 8-wide k slices

  const size_t row_stride = size_t(a.H) * D;  // elements between consecutive sequence rows
  const __bf16* kbase = a.k + (size_t(b) * a.Skv * a.H + h) * D;
  const __bf16* vbase = a.v + (size_t(b) * a.Skv * a.H + h) * D;
  const uint8_t* mbase = a.mask ? a.mask + size_t(b) * a.Skv : nullptr;

  // ---- Q fragment (B operand of S^T = K Q^T): query row q_row, d = ks*16 + 8*hi .. +8
  const int q_row = mt * C::BM + wave * 32 + l32;
  bf16x8 qf[C::KS];
  {
    const bool ok = q_row < a.Sq;
    const __bf16* qp = a.q + (size_t(b) * a.Sq + (ok ? q_row : 0)) * row_stride + size_t(h) * D;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      bf16x8 t = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + 8 * hi);
      if (!ok) t = bf16x8{};
      qf[ks] = t;
    }
  }

  const int n_tiles = (a.Skv + C::BN - 1) / C::BN;

  // ---- global -> register staging of one K/V tile
  uint4 kreg[C::LOADS], vreg[C::LOADS];
  float breg = 0.f;  // this thread's key bias (threads < BN)
  const int vgrp = tid % C::GROUPS;   // V: key group (KPT consecutive keys)
  const int vcol = tid / C::GROUPS;   // V: 16-byte column (8 head-dim values)

  auto load_tile = [&](int t) {
    const int key0 = t * C::BN;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int vec = tid + kThreads * i;
      const int kr = vec / C::VD, kc = vec % C::VD;
      const int key = key0 + kr;
      uint4 x = {0u, 0u, 0u, 0u};
      if (key < a.Skv) x = *reinterpret_cast<const uint4*>(kbase + size_t(key) * row_stride + kc * 8);
      kreg[i] = x;
    }
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int key = key0 + vgrp * C::KPT + i;
      uint4 x = {0u, 0u, 0u, 0u};
      if (key < a.Skv) x = *reinterpret_cast<const uint4*>(vbase + size_t(key) * row_stride + vcol * 8);
      vreg[i] = x;
    }
    if (tid < C::BN) {
      const int key = key0 + tid;
      bool valid = key < a.Skv;
      if (valid && mbase) valid = mbase[key] != 0;
      breg = valid ? 0.f : -INFINITY;
    }
  };

  auto store_tile = [&](int buf) {
    __bf16* ks = smem + buf * (C::K_ELEMS + C::V_ELEMS);
    __bf16* vs = ks + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int vec = tid + kThreads * i;
      const int kr = vec / C::VD, kc = vec % C::VD;
      *reinterpret_cast<uint4*>(ks + kr * C::KP + kc * 8) = kreg[i];
    }
    const int pos = vt_pos(vgrp * C::KPT);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      __bf16* dst = vs + (vcol * 8 + e) * C::VP + pos;
      if constexpr (C::KPT == 4) {
        uint2 pr;
        if (e & 1) {
          pr.x = hi_pair(dword_of(vreg[0], w), dword_of(vreg[1], w));
          pr.y = hi_pair(dword_of(vreg[2], w), dword_of(vreg[3], w));
        } else {
          pr.x = lo_pair(dword_of(vreg[0], w), dword_of(vreg[1], w));
          pr.y = lo_pair(dword_of(vreg[2], w), dword_of(vreg[3], w));
        }
        *reinterpret_cast<uint2*>(dst) = pr;
      } else {
        const uint32_t x = (e & 1) ? hi_pair(dword_of(vreg[0], w), dword_of(vreg[1], w))
                                   : lo_pair(dword_of(vreg[0], w), dword_of(vreg[1], w));
        *reinterpret_cast<uint32_t*>(dst) = x;
      }
    }
    if (tid < C::BN) kbias[buf][tid] = breg;
  };

  // ---- accumulators
  f32x16 acc_o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc_o[db] = f32x16{};
  float m_run = -INFINITY;  // running max, in scaled log2 units
  float l_run = 0.f;        // this lane's partial row sum (its 32 of each 64 keys)

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);

    const __bf16* ks = smem + cur * (C::K_ELEMS + C::V_ELEMS);
    const __bf16* vs = ks + C::K_ELEMS;

    // S^T[key][query] for the two 32-key blocks of the tile.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + l32) * C::KP + kk * 16 + 8 * hi);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], acc, 0, 0, 0);
      }
      s[kb] = acc;
    }

    // Tail / mask bias.  Accumulator row r of block kb is key kb*32 + 8*(r/4) + 4*hi + r%4.
    const bool need_bias = (a.mask != nullptr) || ((t + 1) * C::BN > a.Skv);
    if (need_bias) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 bb = *reinterpret_cast<const float4*>(&kbias[cur][kb * 32 + 8 * g + 4 * hi]);
          s[kb][4 * g + 0] += bb.x;
          s[kb][4 * g + 1] += bb.y;
          s[kb][4 * g + 2] += bb.z;
          s[kb][4 * g + 3] += bb.w;
        }
    }

    // Tile max over this query's 64 keys (32 here, 32 in lane ^ 32).
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt_scaled = mx * a.sc;

    const bool raise = mt_scaled > m_run + 8.0f;
    if (__any(raise)) {
      const float m_new = raise ? mt_scaled : m_run;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;

    // Probabilities, in B-operand order: step m uses block m/2, rows 8*(m%2) .. +8.
    bf16x8 pf[4];
    float lsum = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[m >> 1][8 * (m & 1) + kk], a.sc, -m_use));
        lsum += p;
        pf[m][kk] = (__bf16)p;
      }
    }
    l_run += lsum;

    // O^T[d][query] += V^T[d][keys] P^T[keys][query]
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const bf16x8 vf =
            *reinterpret_cast<const bf16x8*>(vs + (db * 32 + l32) * C::VP + 16 * m + 8 * hi);
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[m], acc_o[db], 0, 0, 0);
      }

    if (t + 1 < n_tiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- normalise and store.  Accumulator row r of block db is d = db*32 + 8*(r/4) + 4*hi + r%4.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (q_row < a.Sq) {
    __bf16* op = a.o + (size_t(b) * a.Sq + q_row) * row_stride + size_t(h) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 w;
        w[0] = (__bf16)(acc_o[db][4 * g + 0] * inv);
        w[1] = (__bf16)(acc_o[db][4 * g + 1] * inv);
        w[2] = (__bf16)(acc_o[db][4 * g + 2] * inv);
        w[3] = (__bf16)(acc_o[db][4 * g + 3] * inv);
        *reinterpret_cast<bf16x4*>(op + db * 32 + 8 * g + 4 * hi) = w;
      }
  }
}

}  // namespace
}  // namespace cpattn

using namespace cpattn;

extern "C" int cp_attn_localq_globalkv(const void* q, const void* k, const void* v,
                                       const uint8_t* key_mask, void* o, int64_t B, int64_t Sq,
                                       int64_t Skv, int64_t H, int64_t D, float scale,
                                       int causal, cp_stream_t stream) {
  if (!q || !k || !v || !o) return CP_ERR_NULL;
  if (B < 1 || Sq < 1 || Skv < 1 || H < 1) return CP_ERR_SHAPE;
  if (D != 64 && D != 128) return CP_ERR_HEAD_DIM;
  if (!std::isfinite(scale) || !(scale > 0.f)) return CP_ERR_SCALE;
  if (causal != 0) return CP_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return CP_ERR_ALIGNMENT;
  // Extents: element offsets fit size_t easily; the work count and per-dimension
  // sizes are kept in int.
  constexpr int64_t kIntMax = 0x7fffffff;
  if (B > kIntMax || Sq > kIntMax || Skv > kIntMax || H > kIntMax) return CP_ERR_SHAPE;
  const int64_t bm = 32 * kWaves;
  const int64_t m_tiles = (Sq + bm - 1) / bm;
  int64_t bh, n_work, qe, ke;
  if (!mul_capped(B, H, kIntMax, &bh) || !mul_capped(bh, m_tiles, kIntMax, &n_work)) return CP_ERR_SHAPE;
  if (!mul_capped(B * Sq, H * D, int64_t(1) << 60, &qe) || !mul_capped(B * Skv, H * D, int64_t(1) << 60, &ke))
    return CP_ERR_SHAPE;
  const size_t qb = size_t(qe) * 2, kb = size_t(ke) * 2;
  if (overlaps(o, qb, q, qb) || overlaps(o, qb, k, kb) || overlaps(o, qb, v, kb)) return CP_ERR_ALIAS;
  if (key_mask && overlaps(o, qb, key_mask, size_t(B * Skv))) return CP_ERR_ALIAS;

  AttnArgs args;
  args.q = static_cast<const __bf16*>(q);
  args.k = static_cast<const __bf16*>(k);
  args.v = static_cast<const __bf16*>(v);
  args.mask = key_mask;
  args.o = static_cast<__bf16*>(o);
  args.B = int(B);
  args.Sq = int(Sq);
  args.Skv = int(Skv);
  args.H = int(H);
  args.m_tiles = int(m_tiles);
  args.n_work = int(n_work);
  args.sc = scale * 1.4426950408889634f;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (D == 128)
    hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3(unsigned(n_work)), dim3(kThreads), 0, s, args);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3(unsigned(n_work)), dim3(kThreads), 0, s, args);
  return hip_status(hipGetLastError());
}
