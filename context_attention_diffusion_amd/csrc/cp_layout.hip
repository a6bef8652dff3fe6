// Ulysses layout exchange for one rank: destination-major pack of Q/K/V, the
// simulated chunk exchange, the receive-side unpack and the output reverse.
//
// Every map here moves whole 16-byte vectors (8 two-byte elements) without
// touching their bits, so results are bit-exact for bf16 and fp16 alike.  The
// maps are the ones of the sglang PR #33667 summary ("Key source snippets",
// usp.py excerpt of _usp_input_all_to_all_qkv and the unit-test excerpt); the
// output reverse is read as the inverse of the forward exchange.
//
// Kernel shape: all four maps are HBM-bound permutations of contiguous runs and
// share one persistent kernel.  A map object gives the source and destination
// of each 16-byte vector; blocks (8 per CU) stride over tiles of 1024 vectors
// and each thread loads its 4 vectors of the next tile before storing those of
// the current one, so reads and writes stay in flight together.  Pack, reverse
// and exchange enumerate the output in order (coalesced stores, reads in runs of
// D*2 or H_local*D*2 bytes); unpack enumerates its input in order (sequential
// reads, writes in D*2-byte runs).  Loads use the default cache policy (the
// sources are usually still cache-resident).  Stores are nontemporal where the
// result leaves for the collective (pack staging, reverse send layout) and for
// the unpacked Q/K/V (cold, the unpack then matches or beats a plain device copy
// of the same bytes, and the attention reading them next is slowed by well
// under 1%); the receive buffer and the merged output use the default policy.

#include <hip/hip_runtime.h>

#include "cp_common.hpp"

namespace cpattn {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;
constexpr int kVecPerBlock = kThreads * kVecPerThread;
constexpr int kBlocksPerCu = 8;

typedef uint32_t vec_t __attribute__((ext_vector_type(4)));  // 16 bytes

__device__ __forceinline__ vec_t ld(const vec_t* p) { return *p; }
template <bool NT>
__device__ __forceinline__ void st(vec_t* p, vec_t v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// ------------------------------------------------------------------ the one kernel
// Every layout map is a permutation of 16-byte vectors given by a map object:
// m.src(o) / m.dst(o) for output-ordered index o.  Blocks stride over tiles of
// kVecPerBlock vectors; each thread loads its 4 vectors of the next tile before
// storing those of the current one, so reads and writes stay in flight together.
// A map with kZeroFill set may return nullptr from src(o): that output vector is
// zero (padding).
template <class Map, bool NT_STORE>
__global__ void __launch_bounds__(kThreads) permute_kernel(Map m, uint32_t n_vec) {
  const uint32_t n_tiles = (n_vec + kVecPerBlock - 1) / kVecPerBlock;
  uint32_t tile = blockIdx.x;
  if (tile >= n_tiles) return;
  vec_t cur[kVecPerThread];
  auto load = [&](uint32_t t, vec_t* buf) {
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const uint32_t o = t * kVecPerBlock + u * kThreads + threadIdx.x;
      if (o < n_vec) {
        if constexpr (Map::kZeroFill) {
          const vec_t* p = m.src(o);
          buf[u] = p ? ld(p) : vec_t{0u, 0u, 0u, 0u};
        } else {
          buf[u] = ld(m.src(o));
        }
      }
    }
  };
  auto store = [&](uint32_t t, const vec_t* buf) {
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const uint32_t o = t * kVecPerBlock + u * kThreads + threadIdx.x;
      if (o < n_vec) st<NT_STORE>(m.dst(o), buf[u]);
    }
  };
  load(tile, cur);
  for (;;) {
    const uint32_t nxt = tile + gridDim.x;
    vec_t nb[kVecPerThread];
    if (nxt < n_tiles) load(nxt, nb);
    store(tile, cur);
    if (nxt >= n_tiles) break;
    tile = nxt;
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) cur[u] = nb[u];
  }
}

// ------------------------------------------------------------------ maps
// pack: output order (j, row, hl, c, dv); VD = D/8 vectors per head row (0 = runtime vd).
template <int VD>
struct PackMap {
  // the staging buffer goes to the collective, not to another kernel on this GPU
  static constexpr bool kNontemporalStore = true;
  static constexpr bool kZeroFill = false;
  const vec_t *q, *k, *v;
  vec_t* out;
  uint32_t vd, H_local, H;
  FastDiv div_vd, div_hl, div_rows;
  __device__ __forceinline__ const vec_t* src(uint32_t o) const {
    uint32_t t, dv;
    if (VD > 0) { dv = o % VD; t = o / VD; } else { div_vd.divmod(o, t, dv); }
    const uint32_t c = t % 3u;
    t /= 3u;
    uint32_t rj, hl, j, row;
    div_hl.divmod(t, rj, hl);
    div_rows.divmod(rj, j, row);
    const vec_t* base = c == 0 ? q : (c == 1 ? k : v);
    const uint32_t w = VD > 0 ? uint32_t(VD) : vd;
    return base + (size_t(row) * H + j * H_local + hl) * w + dv;
  }
  __device__ __forceinline__ vec_t* dst(uint32_t o) const { return out + o; }
};

// unpack: input order (r, row = b*S_l + s, hl, c, dv) over the receive buffer, so reads
// are sequential; the vector goes to out_c[b][r*S_l + s][hl][dv].
template <int VD>
struct UnpackMap {
  // Streaming stores: the unpack then runs near copy speed from HBM; the attention
  // that reads these rows next loses well under 1% (its K/V reuse is served by L2).
  static constexpr bool kNontemporalStore = true;
  static constexpr bool kZeroFill = false;
  const vec_t* recv;
  vec_t *q, *k, *v;
  uint32_t vd, H_local, wsl;                  // wsl = W * S_local output rows per batch
  FastDiv div_3vd, div_hl, div_sl, div_rows;
  __device__ __forceinline__ const vec_t* src(uint32_t o) const { return recv + o; }
  __device__ __forceinline__ vec_t* dst(uint32_t o) const {
    const uint32_t w = VD > 0 ? uint32_t(VD) : vd;
    uint32_t t, e;
    div_3vd.divmod(o, t, e);  // e = c*w + dv
    const uint32_t c = e / w, dv = e % w;
    uint32_t rr, hl, r, row, b, s;
    div_hl.divmod(t, rr, hl);  // rr = r*rows + row
    div_rows.divmod(rr, r, row);
    div_sl.divmod(row, b, s);
    vec_t* base = c == 0 ? q : (c == 1 ? k : v);
    return base + ((size_t(b) * wsl + r * div_sl.d + s) * H_local + hl) * w + dv;
  }
};

// reverse: runs of `run` vectors.  SEND: out (r, b, s) <- src (b, r*S_l + s);
// MERGE: out (b, s, j) <- src (j, b, s).
template <int PHASE>
struct ReverseMap {
  static constexpr bool kNontemporalStore = PHASE == 0;  // send layout goes to the collective
  static constexpr bool kZeroFill = false;
  const vec_t* src_;
  vec_t* out;
  uint32_t W, B, S_local;
  FastDiv div_run, div_a, div_b;
  __device__ __forceinline__ const vec_t* src(uint32_t o) const {
    uint32_t idx, inner;
    div_run.divmod(o, idx, inner);
    size_t src_run;
    if (PHASE == 0) {
      uint32_t rb, s, r, b;  // idx = (r * B + b) * S_l + s
      div_a.divmod(idx, rb, s);
      div_b.divmod(rb, r, b);
      src_run = (size_t(b) * W + r) * S_local + s;
    } else {
      uint32_t bs, j, b, s;  // idx = (b * S_l + s) * W + j
      div_a.divmod(idx, bs, j);
      div_b.divmod(bs, b, s);
      src_run = (size_t(j) * B + b) * S_local + s;
    }
    return src_ + src_run * div_run.d + inner;
  }
  __device__ __forceinline__ vec_t* dst(uint32_t o) const { return out + o; }
};

// pack with head padding: as PackMap over H_pad = W * H_local heads, of which
// heads >= H (the source's head count and row stride) are zeros.
template <int VD>
struct PackPadMap {
  static constexpr bool kNontemporalStore = true;
  static constexpr bool kZeroFill = true;
  const vec_t *q, *k, *v;
  vec_t* out;
  uint32_t vd, H_local, H;
  FastDiv div_vd, div_hl, div_rows;
  __device__ __forceinline__ const vec_t* src(uint32_t o) const {
    uint32_t t, dv;
    if (VD > 0) { dv = o % VD; t = o / VD; } else { div_vd.divmod(o, t, dv); }
    const uint32_t c = t % 3u;
    t /= 3u;
    uint32_t rj, hl, j, row;
    div_hl.divmod(t, rj, hl);
    div_rows.divmod(rj, j, row);
    const uint32_t g = j * H_local + hl;
    if (g >= H) return nullptr;
    const vec_t* base = c == 0 ? q : (c == 1 ? k : v);
    const uint32_t w = VD > 0 ? uint32_t(VD) : vd;
    return base + (size_t(row) * H + g) * w + dv;
  }
  __device__ __forceinline__ vec_t* dst(uint32_t o) const { return out + o; }
};

// merge with the padded heads dropped: output order (b, s, g, dv) over the H
// real heads; head g = j * H_local + hl comes from rank j's chunk.
struct MergeCropMap {
  static constexpr bool kNontemporalStore = false;
  static constexpr bool kZeroFill = false;
  const vec_t* src_;
  vec_t* out;
  uint32_t B, S_local, H_local;
  FastDiv div_vd, div_h, div_hl;
  __device__ __forceinline__ const vec_t* src(uint32_t o) const {
    uint32_t t, dv, bs, g, j, hl;
    div_vd.divmod(o, t, dv);
    div_h.divmod(t, bs, g);
    div_hl.divmod(g, j, hl);
    // [W][B][S_local][H_local][D]: rank j's chunk holds B * S_local rows
    return src_ + ((size_t(j) * B * S_local + bs) * H_local + hl) * div_vd.d + dv;
  }
  __device__ __forceinline__ vec_t* dst(uint32_t o) const { return out + o; }
};

// simulated exchange: recv chunk r <- chunk `rank` of sends[r].
constexpr int kMaxRanks = 64;
struct ExchangeMap {
  static constexpr bool kNontemporalStore = false;  // the receive buffer is unpacked next
  static constexpr bool kZeroFill = false;
  const vec_t* p[kMaxRanks];
  vec_t* recv;
  uint32_t rank;
  FastDiv div_chunk;
  __device__ __forceinline__ const vec_t* src(uint32_t o) const {
    uint32_t r, e;
    div_chunk.divmod(o, r, e);
    return p[r] + size_t(rank) * div_chunk.d + e;
  }
  __device__ __forceinline__ vec_t* dst(uint32_t o) const { return recv + o; }
};

inline unsigned grid_for(uint32_t n_vec) {
  const unsigned tiles = (n_vec + kVecPerBlock - 1) / kVecPerBlock;
  const unsigned cap = unsigned(num_cus()) * kBlocksPerCu;
  return tiles < cap ? tiles : cap;
}

template <class Map>
int launch_permute(const Map& m, uint32_t n_vec, hipStream_t s) {
  hipLaunchKernelGGL((permute_kernel<Map, Map::kNontemporalStore>), dim3(grid_for(n_vec)), dim3(kThreads), 0, s,
                     m, n_vec);
  return hip_status(hipGetLastError());
}

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
  if (vd == 16)
    return launch_permute(PackMap<16>{qv, kv, vv, out, vd, H_local, uint32_t(H), dvd, dhl, drows},
                          uint32_t(n_vec), s);
  if (vd == 8)
    return launch_permute(PackMap<8>{qv, kv, vv, out, vd, H_local, uint32_t(H), dvd, dhl, drows},
                          uint32_t(n_vec), s);
  return launch_permute(PackMap<0>{qv, kv, vv, out, vd, H_local, uint32_t(H), dvd, dhl, drows},
                        uint32_t(n_vec), s);
}

extern "C" int cp_pack_qkv_dst_major_padded(const void* q, const void* k, const void* v, void* staging,
                                            int64_t B, int64_t S_local, int64_t H, int64_t H_pad, int64_t D,
                                            int64_t W, int dtype, cp_stream_t stream) {
  if (!q || !k || !v || !staging) return CP_ERR_NULL;
  int st = check_layout_dims(B, S_local, H, D, W, dtype);
  if (st) return st;
  if (H_pad < H) return CP_ERR_SHAPE;
  if (H_pad % W != 0) return CP_ERR_DIVISIBILITY;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(staging))
    return CP_ERR_ALIGNMENT;
  int64_t rows, per_in, per_out, n_vec;
  if (!mul_capped(B, S_local, kMaxVectors, &rows) || !mul_capped(rows, H * (D / 8), kMaxVectors, &per_in) ||
      !mul_capped(rows, H_pad * (D / 8), kMaxVectors, &per_out) ||
      !mul_capped(per_out, 3, kMaxVectors, &n_vec))
    return CP_ERR_SHAPE;
  const size_t ib = size_t(per_in) * 16, sb = size_t(n_vec) * 16;
  if (overlaps(staging, sb, q, ib) || overlaps(staging, sb, k, ib) || overlaps(staging, sb, v, ib))
    return CP_ERR_ALIAS;
  const uint32_t H_local = uint32_t(H_pad / W);
  const uint32_t vd = uint32_t(D / 8);
  FastDiv dvd{vd}, dhl{H_local}, drows{uint32_t(rows)};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const auto* qv = static_cast<const vec_t*>(q);
  const auto* kv = static_cast<const vec_t*>(k);
  const auto* vv = static_cast<const vec_t*>(v);
  auto* out = static_cast<vec_t*>(staging);
  if (vd == 16)
    return launch_permute(PackPadMap<16>{qv, kv, vv, out, vd, H_local, uint32_t(H), dvd, dhl, drows},
                          uint32_t(n_vec), s);
  if (vd == 8)
    return launch_permute(PackPadMap<8>{qv, kv, vv, out, vd, H_local, uint32_t(H), dvd, dhl, drows},
                          uint32_t(n_vec), s);
  return launch_permute(PackPadMap<0>{qv, kv, vv, out, vd, H_local, uint32_t(H), dvd, dhl, drows},
                        uint32_t(n_vec), s);
}

extern "C" int cp_output_merge_cropped(const void* src, void* dst, int64_t B, int64_t S_local, int64_t H_local,
                                       int64_t H, int64_t D, int64_t W, int dtype, cp_stream_t stream) {
  if (!src || !dst) return CP_ERR_NULL;
  int st = check_layout_dims(B, S_local, H_local, D, W, dtype);
  if (st) return st;
  if (H < 1 || H > W * H_local) return CP_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return CP_ERR_ALIGNMENT;
  int64_t rows, in_vec, n_vec;
  if (!mul_capped(B, S_local, kMaxVectors, &rows) ||
      !mul_capped(rows, W * H_local * (D / 8), kMaxVectors, &in_vec) ||
      !mul_capped(rows, H * (D / 8), kMaxVectors, &n_vec))
    return CP_ERR_SHAPE;
  if (overlaps(src, size_t(in_vec) * 16, dst, size_t(n_vec) * 16)) return CP_ERR_ALIAS;
  const uint32_t vd = uint32_t(D / 8);
  MergeCropMap m{static_cast<const vec_t*>(src), static_cast<vec_t*>(dst), uint32_t(B), uint32_t(S_local),
                 uint32_t(H_local), FastDiv(vd), FastDiv(uint32_t(H)), FastDiv(uint32_t(H_local))};
  return launch_permute(m, uint32_t(n_vec), reinterpret_cast<hipStream_t>(stream));
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
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const auto* rv = static_cast<const vec_t*>(recv);
  auto* qo = static_cast<vec_t*>(q_out);
  auto* ko = static_cast<vec_t*>(k_out);
  auto* vo = static_cast<vec_t*>(v_out);
  const FastDiv d3vd{3u * vd}, dhl{uint32_t(H_local)}, dsl{uint32_t(S_local)}, drows{uint32_t(rows)};
  const uint32_t hl32 = uint32_t(H_local), wsl32 = uint32_t(wsl);
  if (vd == 16)
    return launch_permute(UnpackMap<16>{rv, qo, ko, vo, vd, hl32, wsl32, d3vd, dhl, dsl, drows},
                          uint32_t(n_vec), s);
  if (vd == 8)
    return launch_permute(UnpackMap<8>{rv, qo, ko, vo, vd, hl32, wsl32, d3vd, dhl, dsl, drows},
                          uint32_t(n_vec), s);
  return launch_permute(UnpackMap<0>{rv, qo, ko, vo, vd, hl32, wsl32, d3vd, dhl, dsl, drows},
                        uint32_t(n_vec), s);
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
  FastDiv drun{uint32_t(run)};
  if (phase == 0)
    return launch_permute(ReverseMap<0>{sv, dv, uint32_t(W), uint32_t(B), uint32_t(S_local), drun,
                                        FastDiv(uint32_t(S_local)), FastDiv(uint32_t(B))},
                          uint32_t(n_vec), s);
  return launch_permute(ReverseMap<1>{sv, dv, uint32_t(W), uint32_t(B), uint32_t(S_local), drun,
                                      FastDiv(uint32_t(W)), FastDiv(uint32_t(S_local))},
                        uint32_t(n_vec), s);
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
  ExchangeMap p{};
  for (int64_t r = 0; r < W; ++r) {
    if (!sends[r]) return CP_ERR_NULL;
    if (!aligned16(sends[r])) return CP_ERR_ALIGNMENT;
    if (overlaps(sends[r], size_t(bytes_per_rank), recv, size_t(bytes_per_rank)))
      return CP_ERR_ALIAS;
    p.p[r] = static_cast<const vec_t*>(sends[r]);
  }
  const uint32_t n_vec = uint32_t(bytes_per_rank / 16);
  const uint32_t chunk = n_vec / uint32_t(W);
  p.recv = static_cast<vec_t*>(recv);
  p.rank = uint32_t(rank);
  p.div_chunk = FastDiv(chunk);
  return launch_permute(p, n_vec, reinterpret_cast<hipStream_t>(stream));
}
