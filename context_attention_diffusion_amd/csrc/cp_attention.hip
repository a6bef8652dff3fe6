// Non-causal local-Q / global-KV multi-head attention, bf16 in/out, for gfx950.
//
// The problem is the one an AllGather-KV rank hands to its attention backend
// (vllm-omni PR #7641, "Compose Ulysses with AllGather-KV as a 2D diffusion
// SP", commit message): this rank's query rows against every key row of the
// same heads, with an optional per-batch key-validity mask (that PR's review-fix
// commits: a [B, K] mask, True = attend).  Head dims 64 and 128.
//
// Design.  One workgroup = 8 waves = 128 query rows of one (batch, head).  The
// waves form two groups of four; group g takes the key tiles t = 2i + g, so the
// two groups walk the keys side by side, each with its own double-buffered
// LDS tiles, and every SIMD runs one wave of each group.  At the end the two
// partial softmax states are merged through LDS.
//
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16.  With keys as the MFMA row
//    dimension, each lane owns one query column and 16 key rows per 32x32
//    block, so the row max and row sum are in-lane reductions plus one
//    permlane32 swap.  Q stays in registers (the B operand) for the whole loop.
//  * O^T = V^T P^T on the same MFMA.  The probabilities leave the S^T
//    accumulators already in B-operand position; the 16 keys of each MFMA step
//    are taken in the order the accumulator layout delivers them, and V is
//    written to LDS transposed ([d][key]) in that same key order, so every
//    operand is one 16-byte LDS read.
//  * Software pipeline per wave: iteration i issues the Q K^T MFMAs of its
//    next tile while the VALU turns the current tile's scores into
//    probabilities, then the P V MFMAs of the current tile while the VALU takes
//    the next tile's row max.  K therefore runs one tile ahead of V in LDS.
//  * Online softmax in fp32 with exp2 (scale * log2 e folded into one FMA).  The
//    running max is only raised when a tile's max exceeds it by more than 8 (a
//    factor 2^8 in probability), so the O rescale is rare; numerator and
//    denominator share the stale max, so the quotient is unchanged.  The row sum
//    adds the bf16-rounded probabilities pairwise with v_dot2, i.e. exactly the
//    values that enter the P V product.
//  * Key tail and key mask: a per-tile additive bias row (0 or -inf) in LDS,
//    applied only to tiles that need it.
//  * Workgroups are numbered so that all query tiles of one (batch, head) land
//    on the same XCD, whose L2 then serves that head's K/V to all of them.

#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "cp_common.hpp"

namespace cpattn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGroupWaves = 4;
constexpr int kGroups = 2;
constexpr int kGroupThreads = 64 * kGroupWaves;
constexpr int kThreads = kGroupThreads * kGroups;
constexpr int kNumXcd = 8;

template <int D>
struct Cfg {
  static constexpr int BM = 32 * kGroupWaves;  // query rows per workgroup
  static constexpr int BN = 64;                // keys per tile
  static constexpr int KP = D + 8;             // K row pitch in LDS (elements); +16 B vs bank conflicts
  static constexpr int VP = BN + 8;            // V^T row pitch in LDS (elements)
  static constexpr int K_ELEMS = BN * KP;
  static constexpr int V_ELEMS = D * VP;
  static constexpr int VD = D / 8;             // 16-byte vectors per head row
  static constexpr int LOADS = BN * VD / kGroupThreads;  // K (and V) vectors per thread per tile
  static constexpr int KPT = LOADS;            // keys per thread in the V transpose
  static constexpr int VGROUPS = BN / KPT;     // key groups per 16-byte column of V
  static constexpr int DB = D / 32;            // 32-row blocks of O^T
  static constexpr int KS = D / 16;            // 16-wide reduction steps of Q K^T
  static constexpr int NCOMB = DB * 16 + 2;    // floats per lane in the group merge
  static_assert(LOADS * kGroupThreads == BN * VD, "tile must split evenly");
  static_assert(VGROUPS * VD == kGroupThreads, "V transpose mapping must cover the tile");
  static_assert(KPT == 2 || KPT == 4, "V transpose writes 2 or 4 keys per store");
  static_assert(kGroupWaves * 64 * NCOMB * 4 <= kGroups * 2 * K_ELEMS * 2,
                "group merge must fit in the K buffers");
};

// Position of key offset `ko` (0..BN-1) inside a V^T row: bits 2 and 3 swapped,
// which is the order in which a lane's accumulator rows enter one MFMA step.
__device__ __forceinline__ int vt_pos(int ko) {
  return (ko & ~12) | ((ko & 4) << 1) | ((ko & 8) >> 1);
}

// Two-element transposes of bf16 pairs: lo_pair(a, b) = {a.lo, b.lo}, hi_pair(a, b) = {a.hi, b.hi},
// one v_perm_b32 each.
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }
__device__ __forceinline__ uint32_t dword_of(const uint4& v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

// max / sum of x over lanes l and l ^ 32
__device__ __forceinline__ float pair_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float pair_sum(float x) { return x + __shfl_xor(x, 32); }

struct AttnArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const uint8_t* mask;
  __bf16* o;
  int B, Sq, Skv, H;
  int m_tiles;  // ceil(Sq / BM)
  int n_work;   // B * H * m_tiles
  float sc;     // scale * log2(e)
};

template <int D>
__global__ void __launch_bounds__(kThreads) attn_fwd_kernel(AttnArgs a) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 kbuf[kGroups][2][C::K_ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 vbuf[kGroups][2][C::V_ELEMS];
  __shared__ __attribute__((aligned(16))) float kbias[kGroups][2][C::BN];

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
  // Wave-uniform indices go through readfirstlane so that the compiler keeps
  // them (and the buffer descriptors built from them) in scalar registers.
  const int grp = __builtin_amdgcn_readfirstlane(tid / kGroupThreads);  // key-tile group
  const int gt = tid % kGroupThreads;                                   // thread index inside the group
  const int gw = __builtin_amdgcn_readfirstlane(gt >> 6);               // wave index inside the group
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;                // which half of the wave: selects 8-wide k slices

  const size_t row_stride = size_t(a.H) * D;  // elements between consecutive sequence rows
  const __bf16* kbase = a.k + (size_t(b) * a.Skv * a.H + h) * D;
  const __bf16* vbase = a.v + (size_t(b) * a.Skv * a.H + h) * D;
  const uint8_t* mbase = a.mask ? a.mask + size_t(b) * a.Skv : nullptr;

  // ---- Q fragment (B operand of S^T = K Q^T): query row q_row, d = ks*16 + 8*hi .. +8
  const int q_row = mt * C::BM + gw * 32 + l32;
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
  const int n_iter = (n_tiles + 1) / 2;              // iterations of every wave
  const int n_g = (n_tiles - grp + 1) / 2;           // tiles of this group
  auto tile_of = [&](int i) { return 2 * i + grp; };

  // ---- global -> register staging through buffer resources.  One descriptor
  // per tile (base advanced to the tile's first key, scalar registers); fixed
  // per-lane byte offsets; rows past the last key fall outside the descriptor's
  // range and read as zero, so the loads need no bounds arithmetic.
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  uint4 kreg[C::LOADS], vreg[C::KPT];
  float breg = 0.f;
  const int vgrp = gt % C::VGROUPS;   // V: key group (KPT consecutive keys)
  const int vcol = gt / C::VGROUPS;   // V: 16-byte column (8 head-dim values)
  const uint32_t rs_bytes = uint32_t(row_stride) * 2u;
  const uint32_t valid_end = uint32_t(a.Skv - 1) * rs_bytes + uint32_t(D) * 2u;
  uint32_t koff[C::LOADS], voff[C::KPT];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int vec = gt + kGroupThreads * i;
    koff[i] = uint32_t(vec / C::VD) * rs_bytes + uint32_t(vec % C::VD) * 16u;
  }
#pragma unroll
  for (int i = 0; i < C::KPT; ++i) voff[i] = uint32_t(vgrp * C::KPT + i) * rs_bytes + uint32_t(vcol) * 16u;
  auto tile_rsrc = [&](const __bf16* base, int t) {
    const uint32_t off = uint32_t(t) * uint32_t(C::BN) * rs_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(base)) + off, (short)0, int(valid_end - off),
        0x00020000);
  };
  auto as_uint4 = [](u32x4 x) { return uint4{x.x, x.y, x.z, x.w}; };

  auto load_k = [&](int t) {
    const auto rk = tile_rsrc(kbase, t);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) kreg[i] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rk, koff[i], 0, 0));
    if (gt < C::BN) {
      const int key = t * C::BN + gt;
      bool valid = key < a.Skv;
      if (mbase) valid = valid && mbase[valid ? key : 0] != 0;
      breg = valid ? 0.f : -INFINITY;
    }
  };
  auto load_v = [&](int t) {
    const auto rv = tile_rsrc(vbase, t);
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) vreg[i] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rv, voff[i], 0, 0));
  };
  auto store_k = [&](int buf) {
    __bf16* ks = kbuf[grp][buf];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int vec = gt + kGroupThreads * i;
      const int kr = vec / C::VD, kc = vec % C::VD;
      *reinterpret_cast<uint4*>(ks + kr * C::KP + kc * 8) = kreg[i];
    }
    if (gt < C::BN) kbias[grp][buf][gt] = breg;
  };
  auto store_v = [&](int buf) {
    __bf16* vs = vbuf[grp][buf];
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
  };

  // S^T[key][query] of one tile (two 32-key blocks) from K in LDS.
  auto qk = [&](int buf, f32x16* s) {
    const __bf16* ks = kbuf[grp][buf];
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
  };
  // Bias (tail / mask) and the scaled tile max over this query's 64 keys.
  // Accumulator row r of block kb is key kb*32 + 8*(r/4) + 4*hi + r%4.
  auto bias_max = [&](int buf, int t, f32x16* s) -> float {
    if (a.mask != nullptr || (t + 1) * C::BN > a.Skv) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 bb = *reinterpret_cast<const float4*>(&kbias[grp][buf][kb * 32 + 8 * g + 4 * hi]);
          s[kb][4 * g + 0] += bb.x;
          s[kb][4 * g + 1] += bb.y;
          s[kb][4 * g + 2] += bb.z;
          s[kb][4 * g + 3] += bb.w;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    return pair_max(mx) * a.sc;
  };
  // Probabilities in B-operand order (step m uses block m/2, rows 8*(m%2) .. +8)
  // and their bf16 sum.
  auto softmax = [&](const f32x16* s, float m_use, bf16x8* pf) -> float {
    float lsum = 0.f;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        pf[m][kk] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[m >> 1][8 * (m & 1) + kk], a.sc, -m_use));
#pragma unroll
      for (int j = 0; j < 4; ++j)
      {
        const bf16x2 pr = {pf[m][2 * j], pf[m][2 * j + 1]};
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
      }
    }
    return lsum;
  };
  f32x16 acc_o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc_o[db] = f32x16{};
  // O^T[d][query] += V^T[d][keys] P^T[keys][query]
  auto pv = [&](int buf, const bf16x8* pf) {
    const __bf16* vs = vbuf[grp][buf];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vs + (db * 32 + l32) * C::VP + 16 * m + 8 * hi);
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[m], acc_o[db], 0, 0, 0);
      }
  };

  float m_run = -INFINITY;  // running max, scaled log2 units (shared by lanes l, l^32)
  float l_run = 0.f;        // this lane's partial row sum
  f32x16 s_cur[2], s_nxt[2];

  // ---- prologue: K of local tiles 0 and 1, V of tile 0, scores of tile 0
  if (n_g > 0) {
    load_k(tile_of(0));
    store_k(0);
    if (n_g > 1) {
      load_k(tile_of(1));
      store_k(1);
    }
    load_v(tile_of(0));
    store_v(0);
  }
  __syncthreads();
  if (n_g > 0) {
    qk(0, s_cur);
    m_run = bias_max(0, tile_of(0), s_cur);
  }

  // ---- main loop; every wave runs n_iter iterations so that barriers match
  auto iteration = [&](int i, auto load_next_k, auto has_next) {
    constexpr bool LK = decltype(load_next_k)::value;
    constexpr bool NX = decltype(has_next)::value;
    if constexpr (LK) load_k(tile_of(i + 2));
    if constexpr (NX) load_v(tile_of(i + 1));
    // Keep the loads at the top: their latency is covered by this iteration's MFMAs.
    __builtin_amdgcn_sched_barrier(0);
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    if constexpr (NX) qk((i + 1) & 1, s_nxt);
    bf16x8 pf[4];
    const float lsum = softmax(s_cur, m_use, pf);
    pv(i & 1, pf);
    l_run += lsum;
    if constexpr (NX) {
      const float mt_next = bias_max((i + 1) & 1, tile_of(i + 1), s_nxt);
      const bool raise = mt_next > m_run + 8.0f;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = raise ? mt_next : m_run;
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
        m_run = m_new;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (LK) store_k(i & 1);
    if constexpr (NX) store_v((i + 1) & 1);
  };

  for (int i = 0; i < n_iter; ++i) {
    if (i + 2 < n_g) {
      iteration(i, std::true_type{}, std::true_type{});
    } else if (i + 1 < n_g) {
      iteration(i, std::false_type{}, std::true_type{});
    } else if (i < n_g) {
      iteration(i, std::false_type{}, std::false_type{});
    }
    __syncthreads();
    s_cur[0] = s_nxt[0];
    s_cur[1] = s_nxt[1];
  }

  // ---- merge the two groups' softmax states through LDS (reusing the K buffers)
  float* comb = reinterpret_cast<float*>(&kbuf[0][0][0]);
  auto slot = [&](int k) { return (gw * C::NCOMB + k) * 64 + lane; };
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) comb[slot(db * 16 + r)] = acc_o[db][r];
    comb[slot(C::DB * 16)] = m_run;
    comb[slot(C::DB * 16 + 1)] = l_run;
  }
  __syncthreads();
  if (grp == 0) {
    const float m1 = comb[slot(C::DB * 16)];
    const float l1 = comb[slot(C::DB * 16 + 1)];
    const float mm = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
    const float l_tot = pair_sum(a0 * l_run + a1 * l1);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float c0 = a0 * inv, c1 = a1 * inv;
    if (q_row < a.Sq) {
      __bf16* op = a.o + (size_t(b) * a.Sq + q_row) * row_stride + size_t(h) * D;
      // Accumulator row r of block db is d = db*32 + 8*(r/4) + 4*hi + r%4.
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            w[e] = (__bf16)(acc_o[db][r] * c0 + comb[slot(db * 16 + r)] * c1);
          }
          *reinterpret_cast<bf16x4*>(op + db * 32 + 8 * g + 4 * hi) = w;
        }
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
  // Per-dimension sizes and the work count are kept in int on the device.
  constexpr int64_t kIntMax = 0x7fffffff;
  if (B > kIntMax || Sq > kIntMax || Skv > kIntMax - 64 || H > kIntMax) return CP_ERR_SHAPE;
  // K/V of one batch are addressed with 32-bit byte offsets.
  if (Skv * H * D * 2 > kIntMax) return CP_ERR_SHAPE;
  const int64_t bm = 32 * kGroupWaves;
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
