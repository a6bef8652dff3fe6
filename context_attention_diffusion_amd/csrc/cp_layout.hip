// Ulysses layout exchange for one rank: destination-major pack of Q/K/V, the
// simulated chunk exchange, the receive-side unpack and the output reverse.
//
// Every map here moves whole 16-byte vectors (8 two-byte elements) without
// touching their bits, so results are bit-exact for bf16 and fp16 alike.  The
// maps are the ones of the sglang PR #33667 summary ("Key source snippets",
// usp.py excerpt of _usp_input_all_to_all_qkv and the unit-test excerpt); the
// output reverse is read as the inverse of the forward exchange.
//
// Kernel shape (all four maps): HBM-bound permutations of contiguous runs.  Each
// thread owns kVecPerThread output vectors spaced one block apart, issues all
// their loads before any store (bytes in flight), and writes the output in
// order so stores are fully coalesced; reads come in runs of D*2 bytes (pack,
// unpack) or H_local*D*2 bytes (reverse), >= 128 B for every supported shape.

#include <hip/hip_runtime.h>

#include "cp_common.hpp"

namespace cpattn {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;
constexpr int kVecPerBlock = kThreads * kVecPerThread;

typedef uint32_t vec_t __attribute__((ext_vector_type(4)));  // 16 bytes

__device__ __forceinline__ vec_t ld(const vec_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st(vec_t* p, vec_t v) { __builtin_nontemporal_store(v, p); }

// ------------------------------------------------------------------ pack
// Output order (j, row, hl, c, dv); VD = D/8 vectors per head row.
template <int VD>
__global__ void __launch_bounds__(kThreads)
pack_kernel(const vec_t* __restrict__ q, const vec_t* __restrict__ k,
            const vec_t* __restrict__ v, vec_t* __restrict__ out, uint32_t n_vec,
            uint32_t vd_rt, FastDiv div_vd, FastDiv div_hl, FastDiv div_rows,
            uint32_t H_local, uint32_t H) {
  const uint32_t vd = VD > 0 ? uint32_t(VD) : vd_rt;
  const uint32_t base = blockIdx.x * kVecPerBlock + threadIdx.x;
  vec_t buf[kVecPerThread];
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const uint32_t o = base + u * kThreads;
    if (o < n_vec) {
      uint32_t t, dv;
      if (VD > 0) { dv = o % VD; t = o / VD; } else { div_vd.divmod(o, t, dv); }
      const uint32_t c = t % 3u;
      t /= 3u;
      uint32_t rj, hl, j, row;
      div_hl.divmod(t, rj, hl);
      div_rows.divmod(rj, j, row);
      const vec_t* src = c == 0 ? q : (c == 1 ? k : v);
      buf[u] = ld(src + (size_t(row) * H + j * H_local + hl) * vd + dv);
    }
  }
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const uint32_t o = base + u * kThreads;
    if (o < n_vec) st(out + o, buf[u]);
  }
}

// ------------------------------------------------------------------ unpack
// Output order (c, b, t, hl, dv) over the three outputs, t = r*S_local + s.
template <int VD>
__global__ void __launch_bounds__(kThreads)
unpack_kernel(const vec_t* __restrict__ recv, vec_t* __restrict__ q, vec_t* __restrict__ k,
              vec_t* __restrict__ v, uint32_t n_vec_per_out, uint32_t vd_rt,
              FastDiv div_inner, FastDiv div_wsl, FastDiv div_sl, FastDiv div_b,
              uint32_t rows, uint32_t H_local) {
  const uint32_t vd = VD > 0 ? uint32_t(VD) : vd_rt;
  const uint32_t n_vec = 3u * n_vec_per_out;
  const uint32_t base = blockIdx.x * kVecPerBlock + threadIdx.x;
  vec_t buf[kVecPerThread];
  vec_t* dst[kVecPerThread];
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const uint32_t o = base + u * kThreads;
    dst[u] = nullptr;
    if (o < n_vec) {
      uint32_t run, inner;
      div_inner.divmod(o, run, inner);                 // inner over (hl, dv)
      uint32_t hl, dv;
      if (VD > 0) { hl = inner / VD; dv = inner % VD; } else { hl = inner / vd; dv = inner % vd; }
      uint32_t bc, t, r, s, c, b;
      div_wsl.divmod(run, bc, t);                      // run = bc * (W*S_l) + t
      div_sl.divmod(t, r, s);
      div_b.divmod(bc, c, b);
      const uint32_t row = b * div_sl.d + s;
      buf[u] = ld(recv + ((size_t(r) * rows + row) * H_local + hl) * (3u * vd) + c * vd + dv);
      vec_t* base_out = c == 0 ? q : (c == 1 ? k : v);
      dst[u] = base_out + (o - c * n_vec_per_out);
    }
  }
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u)
    if (dst[u]) st(dst[u], buf[u]);
}

// ------------------------------------------------------------------ reverse
// Both phases copy runs of `run` vectors (H_local * D / 8).
//   SEND : out (r, b, s)  <- src (b, r*S_l + s)
//   MERGE: out (b, s, j)  <- src (j, b, s)
template <int PHASE>
__global__ void __launch_bounds__(kThreads)
reverse_kernel(const vec_t* __restrict__ src, vec_t* __restrict__ out, uint32_t n_vec,
               FastDiv div_run, FastDiv div_a, FastDiv div_b, uint32_t W, uint32_t B,
               uint32_t S_local) {
  const uint32_t base = blockIdx.x * kVecPerBlock + threadIdx.x;
  const uint32_t run = div_run.d;
  vec_t buf[kVecPerThread];
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const uint32_t o = base + u * kThreads;
    if (o < n_vec) {
      uint32_t idx, inner;
      div_run.divmod(o, idx, inner);
      size_t src_run;
      if (PHASE == 0) {
        // idx = (r * B + b) * S_l + s ; div_a = S_l, div_b = B
        uint32_t rb, s, r, b;
        div_a.divmod(idx, rb, s);
        div_b.divmod(rb, r, b);
        src_run = (size_t(b) * W + r) * S_local + s;
      } else {
        // idx = (b * S_l + s) * W + j ; div_a = W, div_b = S_l
        uint32_t bs, j, b, s;
        div_a.divmod(idx, bs, j);
        div_b.divmod(bs, b, s);
        src_run = (size_t(j) * B + b) * S_local + s;
      }
      buf[u] = ld(src + src_run * run + inner);
    }
  }
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const uint32_t o = base + u * kThreads;
    if (o < n_vec) st(out + o, buf[u]);
  }
}

// ------------------------------------------------------------------ simulated exchange
constexpr int kMaxRanks = 64;
struct SendPtrs {
  const vec_t* p[kMaxRanks];
};

__global__ void __launch_bounds__(kThreads)
exchange_kernel(SendPtrs sends, vec_t* __restrict__ recv, uint32_t n_vec, FastDiv div_chunk,
                uint32_t rank) {
  const uint32_t base = blockIdx.x * kVecPerBlock + threadIdx.x;
  const uint32_t chunk = div_chunk.d;
  vec_t buf[kVecPerThread];
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const uint32_t o = base + u * kThreads;
    if (o < n_vec) {
      uint32_t r, e;
      div_chunk.divmod(o, r, e);
      buf[u] = ld(sends.p[r] + size_t(rank) * chunk + e);
    }
  }
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const uint32_t o = base + u * kThreads;
    if (o < n_vec) st(recv + o, buf[u]);
  }
}

inline unsigned grid_for(uint32_t n_vec) { return (n_vec + kVecPerBlock - 1) / kVecPerBlock; }

// Shared checks of the layout entry points: sizes >= 1, D a multiple of 8.
int check_layout_dims(int64_t B, int64_t S_local, int64_t H, int64_t D, int64_t W, int dtype) {
  if (!layout_dtype_ok(dtype)) return CP_ERR_DTYPE;
  if (B < 1 || S_local < 1 || H < 1 || W < 1) return CP_ERR_SHAPE;
  if (D < 8 || D % 8 != 0) return CP_ERR_HEAD_DIM;
  return CP_OK;
}

}  // namespace
}  // namespace cpattn

using namespace cpattn;

extern "C" int cp_pack_qkv_dst_major(const void* q, const void* k, const void* v, void* staging,
                                     int64_t B, int64_t S_local, int64_t H, int64_t D,
                                     int64_t W, int dtype, cp_stream_t stream) {
  if (!q || !k || !v || !staging) return CP_ERR_NULL;
  int st = check_layout_dims(B, S_local, H, D, W, dtype);
  if (st) return st;
  if (H % W != 0) return CP_ERR_DIVISIBILITY;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(staging))
    return CP_ERR_ALIGNMENT;
  int64_t rows, per_tensor, n_vec;
  if (!mul_capped(B, S_local, kMaxVectors, &rows) || !mul_capped(rows, H * (D / 8), kMaxVectors, &per_tensor) ||
      !mul_capped(per_tensor, 3, kMaxVectors, &n_vec))
    return CP_ERR_SHAPE;
  const size_t tb = size_t(per_tensor) * 16;
  if (overlaps(staging, 3 * tb, q, tb) || overlaps(staging, 3 * tb, k, tb) ||
      overlaps(staging, 3 * tb, v, tb))
    return CP_ERR_ALIAS;
  const uint32_t H_local = uint32_t(H / W);
  const uint32_t vd = uint32_t(D / 8);
  FastDiv dvd{vd}, dhl{H_local}, drows{uint32_t(rows)};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const auto* qv = static_cast<const vec_t*>(q);
  const auto* kv = static_cast<const vec_t*>(k);
  const auto* vv = static_cast<const vec_t*>(v);
  auto* out = static_cast<vec_t*>(staging);
  const dim3 grid(grid_for(uint32_t(n_vec))), block(kThreads);
  if (vd == 16)
    hipLaunchKernelGGL(pack_kernel<16>, grid, block, 0, s, qv, kv, vv, out, uint32_t(n_vec), vd,
                       dvd, dhl, drows, H_local, uint32_t(H));
  else if (vd == 8)
    hipLaunchKernelGGL(pack_kernel<8>, grid, block, 0, s, qv, kv, vv, out, uint32_t(n_vec), vd,
                       dvd, dhl, drows, H_local, uint32_t(H));
  else
    hipLaunchKernelGGL(pack_kernel<0>, grid, block, 0, s, qv, kv, vv, out, uint32_t(n_vec), vd,
                       dvd, dhl, drows, H_local, uint32_t(H));
  return hip_status(hipGetLastError());
}

extern "C" int cp_unpack_head_sharded(const void* recv, void* q_out, void* k_out, void* v_out,
                                      int64_t B, int64_t S_local, int64_t H_local, int64_t D,
                                      int64_t W, int dtype, cp_stream_t stream) {
  if (!recv || !q_out || !k_out || !v_out) return CP_ERR_NULL;
  int st = check_layout_dims(B, S_local, H_local, D, W, dtype);
  if (st) return st;
  if (!aligned16(recv) || !aligned16(q_out) || !aligned16(k_out) || !aligned16(v_out))
    return CP_ERR_ALIGNMENT;
  int64_t rows, wsl, per_out, n_vec, bw;
  if (!mul_capped(B, S_local, kMaxVectors, &rows) || !mul_capped(W, S_local, kMaxVectors, &wsl) ||
      !mul_capped(rows, W, kMaxVectors, &bw) ||
      !mul_capped(bw, H_local * (D / 8), kMaxVectors, &per_out) ||
      !mul_capped(per_out, 3, kMaxVectors, &n_vec))
    return CP_ERR_SHAPE;
  const size_t ob = size_t(per_out) * 16;
  if (overlaps(recv, 3 * ob, q_out, ob) || overlaps(recv, 3 * ob, k_out, ob) ||
      overlaps(recv, 3 * ob, v_out, ob) || overlaps(q_out, ob, k_out, ob) ||
      overlaps(q_out, ob, v_out, ob) || overlaps(k_out, ob, v_out, ob))
    return CP_ERR_ALIAS;
  const uint32_t vd = uint32_t(D / 8);
  FastDiv dinner{uint32_t(H_local) * vd}, dwsl{uint32_t(wsl)}, dsl{uint32_t(S_local)},
      db{uint32_t(B)};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const auto* rv = static_cast<const vec_t*>(recv);
  auto* qo = static_cast<vec_t*>(q_out);
  auto* ko = static_cast<vec_t*>(k_out);
  auto* vo = static_cast<vec_t*>(v_out);
  const dim3 grid(grid_for(uint32_t(n_vec))), block(kThreads);
  if (vd == 16)
    hipLaunchKernelGGL(unpack_kernel<16>, grid, block, 0, s, rv, qo, ko, vo, uint32_t(per_out), vd,
                       dinner, dwsl, dsl, db, uint32_t(rows), uint32_t(H_local));
  else if (vd == 8)
    hipLaunchKernelGGL(unpack_kernel<8>, grid, block, 0, s, rv, qo, ko, vo, uint32_t(per_out), vd,
                       dinner, dwsl, dsl, db, uint32_t(rows), uint32_t(H_local));
  else
    hipLaunchKernelGGL(unpack_kernel<0>, grid, block, 0, s, rv, qo, ko, vo, uint32_t(per_out), vd,
                       dinner, dwsl, dsl, db, uint32_t(rows), uint32_t(H_local));
  return hip_status(hipGetLastError());
}

extern "C" int cp_output_reverse(int phase, const void* src, void* dst, int64_t B,
                                 int64_t S_local, int64_t H_local, int64_t D, int64_t W,
                                 int dtype, cp_stream_t stream) {
  if (!src || !dst) return CP_ERR_NULL;
  int st = check_layout_dims(B, S_local, H_local, D, W, dtype);
  if (st) return st;
  if (phase != 0 && phase != 1) return CP_ERR_UNSUPPORTED;
  if (!aligned16(src) || !aligned16(dst)) return CP_ERR_ALIGNMENT;
  int64_t run, rows, bw, n_vec;
  if (!mul_capped(H_local, D / 8, kMaxVectors, &run) || !mul_capped(B, S_local, kMaxVectors, &rows) ||
      !mul_capped(rows, W, kMaxVectors, &bw) || !mul_capped(bw, run, kMaxVectors, &n_vec))
    return CP_ERR_SHAPE;
  if (overlaps(src, size_t(n_vec) * 16, dst, size_t(n_vec) * 16)) return CP_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const auto* sv = static_cast<const vec_t*>(src);
  auto* dv = static_cast<vec_t*>(dst);
  const dim3 grid(grid_for(uint32_t(n_vec))), block(kThreads);
  FastDiv drun{uint32_t(run)};
  if (phase == 0)
    hipLaunchKernelGGL(reverse_kernel<0>, grid, block, 0, s, sv, dv, uint32_t(n_vec), drun,
                       FastDiv(uint32_t(S_local)), FastDiv(uint32_t(B)), uint32_t(W), uint32_t(B),
                       uint32_t(S_local));
  else
    hipLaunchKernelGGL(reverse_kernel<1>, grid, block, 0, s, sv, dv, uint32_t(n_vec), drun,
                       FastDiv(uint32_t(W)), FastDiv(uint32_t(S_local)), uint32_t(W), uint32_t(B),
                       uint32_t(S_local));
  return hip_status(hipGetLastError());
}

extern "C" int cp_sim_exchange(const void* const* sends, void* recv, int64_t W, int64_t rank,
                               int64_t bytes_per_rank, cp_stream_t stream) {
  if (!sends || !recv) return CP_ERR_NULL;
  if (W < 1 || bytes_per_rank < 1) return CP_ERR_SHAPE;
  if (W > kMaxRanks) return CP_ERR_UNSUPPORTED;
  if (rank < 0 || rank >= W) return CP_ERR_SHAPE;
  if (bytes_per_rank % (16 * W) != 0) return CP_ERR_DIVISIBILITY;
  if (bytes_per_rank / 16 > kMaxVectors) return CP_ERR_SHAPE;
  if (!aligned16(recv)) return CP_ERR_ALIGNMENT;
  SendPtrs p{};
  for (int64_t r = 0; r < W; ++r) {
    if (!sends[r]) return CP_ERR_NULL;
    if (!aligned16(sends[r])) return CP_ERR_ALIGNMENT;
    if (overlaps(sends[r], size_t(bytes_per_rank), recv, size_t(bytes_per_rank)))
      return CP_ERR_ALIAS;
    p.p[r] = static_cast<const vec_t*>(sends[r]);
  }
  const uint32_t n_vec = uint32_t(bytes_per_rank / 16);
  const uint32_t chunk = n_vec / uint32_t(W);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(exchange_kernel, dim3(grid_for(n_vec)), dim3(kThreads), 0, s, p,
                     static_cast<vec_t*>(recv), n_vec, FastDiv(chunk), uint32_t(rank));
  return hip_status(hipGetLastError());
}
