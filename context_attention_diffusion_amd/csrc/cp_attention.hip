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
//  * K and V tiles (64 keys) go from HBM straight into LDS with buffer loads
//    that write LDS directly (no VGPR staging), row-major, with the 16-byte
//    chunks of each row XOR-swizzled so that both readers below are free of
//    bank conflicts.  Rows past the last key fall outside the buffer
//    descriptor's range and arrive as zeros.  Each (operand, group, buffer)
//    tile is its own LDS object, so the compiler can tell that the reads of one
//    buffer do not wait on the in-flight fills of another.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16.  With keys as the MFMA row
//    dimension, each lane owns one query column and 16 key rows per 32x32
//    block, so the row max and row sum are in-lane reductions plus one
//    exchange with lane ^ 32.  Q stays in registers (the B operand).
//  * O^T = V^T P^T on the same MFMA.  The probabilities leave the S^T
//    accumulators already in B-operand position.  The V^T operand comes from
//    the row-major V tile through ds_read_b64_tr_b16, which hands each lane
//    four consecutive keys of one head-dim column; two such reads cover the
//    eight keys a lane contributes to one MFMA step, in the order the
//    accumulator layout delivers the matching probabilities.
//  * Schedule: each SIMD runs one wave of each group, phase-shifted.  Group 0's
//    iteration i runs tile i's Q K^T as two interleaved MFMA chains, with the
//    HBM->LDS fills of the next tiles (of both groups) issued between its steps,
//    then the tile max, then softmax and P V in two 32-key halves.  Group 1 runs
//    one K tile ahead: its iteration i takes tile i's max (scores computed the
//    iteration before), softmax and P V in halves, then tile i+1's Q K^T.  After
//    each barrier group 0 is in MFMAs while group 1 is in VALU work, and the
//    roles alternate.  One barrier per iteration publishes the fills and frees
//    the buffers they overwrite.
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
//  * Wide blocks (compile-time bit 64): 256 query rows, the two groups on rows
//    0-127 and 128-255, both walking every key tile (group 1 still one Q K^T
//    ahead), so that each tile brought into LDS serves 256 rows: half the L2 ->
//    LDS traffic per flop, which the chip turns into clock when it runs at its
//    power limit.  K tiles rotate over four LDS buffers and V tiles over two.  A
//    call splits its heads between a launch of wide blocks and one of 128-row
//    blocks so that each launch fills whole rounds of the compute units.
//
// Variants (compile-time MODE bits, so that the dense path carries none of the
// others' scalar state): 1 = operands addressed through strided views whose
// rows may come in chunks (Q/K/V read from a received Ulysses buffer, O written
// in the send layout); 4 = with chunks whose length is not a multiple of the
// 64-key tile (tiles spanning chunks take per-lane row offsets); 2 = keys in two
// segments with masks of their own (joint text/image keys, or the other
// AllGather rank's K/V); 8 = a second segment with a row stride of its own;
// 16 = packed documents (varlen: query document i against key document i, the
// boundaries read from device memory); 32 = split-KV (the key range of each
// query block cut over nsplit workgroups, whose partial states a separate
// kernel merges); 64 = wide blocks (with 0, 1, 5, 2, 10, 11 and 15).  The
// partial / accumulating outputs are run-time paths of the 128-row and wide
// blocks alike.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>
#include <utility>

#include "cp_common.hpp"

// Scratch memory of cp_attn_localq_globalkv_noalloc, for callers that cannot
// allocate: the split-KV partial states (one 128 x (D + 2) fp32 slot per part,
// at most one part per compute unit), sized for D = 128 on up to 256 compute
// units.  Every device the library runs on holds its own copy until the process
// ends.  Host code never uses this name as an address: it asks each device for
// the array's address once (scratch_on_device below).
static __device__ __align__(256) unsigned char scratch[CP_ATTN_NOALLOC_SCRATCH_BYTES];

namespace cpattn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kGroupWaves = 4;
constexpr int kGroups = 2;
constexpr int kGroupThreads = 64 * kGroupWaves;
constexpr int kThreads = kGroupThreads * kGroups;
constexpr int kNumXcd = 8;

template <int D>
struct Cfg {
  static constexpr int BM = 32 * kGroupWaves;   // query rows per workgroup
  static constexpr int BN = 64;                 // keys per tile
  static constexpr int RB = 2 * D;              // bytes per K/V row
  static constexpr int TILE = BN * RB;          // bytes per K or V tile
  static constexpr int SPT = TILE / 16 / kGroupThreads;  // 16-byte slots per thread per tile
  static constexpr int CHUNKS = RB / 16;        // 16-byte chunks per row
  static constexpr int RPL = 256 / RB;          // rows per 256-byte LDS line
  static constexpr int DB = D / 32;             // 32-row blocks of O^T
  static constexpr int KS = D / 16;             // 16-wide reduction steps of Q K^T
  static constexpr int NCOMB = DB * 16 + 2;     // floats per lane in the group merge
  static_assert(SPT * kGroupThreads * 16 == TILE, "tile must split evenly into slots");
  static_assert(64 * DB * 16 * 4 <= TILE, "a wave's O must fit in one tile array for the merge");
  static_assert(kGroupWaves * 2 * 64 * 4 <= TILE, "m and l of the merge must fit in one tile array");
  // Chunk swizzle of a row (the 16-byte chunk index is XORed with it).  LDS
  // serves 16 lanes of a 16-byte read, or 32 lanes of an 8-byte read, per pass
  // over its 256 bytes of banks; the swizzle makes both passes conflict-free:
  //  * K reads: 16 consecutive rows at one chunk -> 16 distinct 16-byte slots;
  //  * V^T transpose reads: 4 consecutive rows x 4 consecutive chunks -> 16
  //    distinct slots (bits 2-3 of the swizzle separate the 4 rows).
  static __device__ __forceinline__ int swz(int key) {
    return 4 * ((key / RPL) % (4 / RPL)) + (key / 4) % 4;
  }
};

// Reductions over the lane pair (l, l ^ 32) that holds one query: v_permlane32_swap
// of x with itself leaves x in one result and the partner lane's x in the other.
__device__ __forceinline__ void pair_of(float x, float& u, float& w) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  u = __uint_as_float(r[0]);
  w = __uint_as_float(r[1]);
}
// Maximum of scores, which are finite or -inf (never NaN): the instructions
// themselves, without the canonicalisation fmaxf needs for signalling NaNs.
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Maximum of the 32 scores of two accumulator blocks, as two instruction blocks (the
// compiler pads every inline-assembly boundary with a wait state, so it sees two
// boundaries instead of one per v_max3).
__device__ __forceinline__ float max_of_32(const f32x16& x, const f32x16& y) {
  float m;
  asm("v_max3_f32 %0, %1, %2, %3\n\t"
      "v_max3_f32 %0, %0, %4, %5\n\t"
      "v_max3_f32 %0, %0, %6, %7\n\t"
      "v_max3_f32 %0, %0, %8, %9\n\t"
      "v_max3_f32 %0, %0, %10, %11\n\t"
      "v_max3_f32 %0, %0, %12, %13\n\t"
      "v_max3_f32 %0, %0, %14, %15\n\t"
      "v_max3_f32 %0, %0, %16, %17"
      : "=&v"(m)
      : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]),
        "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]), "v"(y[0]));
  asm("v_max3_f32 %0, %0, %1, %2\n\t"
      "v_max3_f32 %0, %0, %3, %4\n\t"
      "v_max3_f32 %0, %0, %5, %6\n\t"
      "v_max3_f32 %0, %0, %7, %8\n\t"
      "v_max3_f32 %0, %0, %9, %10\n\t"
      "v_max3_f32 %0, %0, %11, %12\n\t"
      "v_max3_f32 %0, %0, %13, %14\n\t"
      "v_max_f32 %0, %0, %15"
      : "+v"(m)
      : "v"(y[1]), "v"(y[2]), "v"(y[3]), "v"(y[4]), "v"(y[5]), "v"(y[6]), "v"(y[7]), "v"(y[8]), "v"(y[9]),
        "v"(y[10]), "v"(y[11]), "v"(y[12]), "v"(y[13]), "v"(y[14]), "v"(y[15]));
  return m;
}
__device__ __forceinline__ float pair_max(float x) {
  float u, w;
  pair_of(x, u, w);
  return max2(u, w);
}
__device__ __forceinline__ float pair_sum(float x) {
  float u, w;
  pair_of(x, u, w);
  return u + w;
}

// Row addressing of one operand: element (b, i, h, d) of a [B][S][H][D] view
// lies at  b * bs + row_off(i) + h * hs + d  elements from the base, with
// row_off(i) = (i / L) * cs + (i % L) * rs  for a chunked view (rows come in
// chunks of L, e.g. one chunk per source rank of an all-to-all buffer) and
// i * rs  otherwise.
struct View {
  long long bs;    // batch stride
  long long cs;    // chunk stride (chunked views)
  int rs;          // row stride
  int hs;          // head stride
  int chunked;     // 0: row_off(i) = i * rs
  FastDiv L;       // rows per chunk
};

// Kernel variants (compile-time): chunked row views, a second key segment, and
// (with chunked views only) K/V chunks whose row count is not a multiple of the
// 64-key tile, so that a tile can span chunks.
constexpr int kModeChunked = 1;
constexpr int kModeTwoSeg = 2;
constexpr int kModeCross = 4;
constexpr int kModeSeg1Rows = 8;  // segment 1 has a view (row stride) of its own
constexpr int kModeVarlen = 16;   // packed documents: batch index b is document b
constexpr int kModeSplit = 32;    // the key range of each query block split over nsplit workgroups
constexpr int kModeWide = 64;     // 256-row blocks: the two groups take different rows and share every tile

// CHUNKED = false: every view of the kernel is plain.  CHUNKED = true: a view may
// be chunked (each view says whether it is).
template <bool CHUNKED>
__device__ __forceinline__ long long row_off_t(const View& v, int i) {
  if (!CHUNKED || !v.chunked) return (long long)i * v.rs;
  uint32_t c, r;
  v.L.divmod(uint32_t(i), c, r);
  return (long long)c * v.cs + (long long)r * v.rs;
}

struct AttnArgs {
  View qv, kv, ov;  // Q, K and V (one view for both), O
  View kv1;         // K and V of segment 1
  // Keys come in up to two segments, attended as one sequence in this order:
  // segment 0 = k, v, mask through kv (Skv keys, tiles [0, nt0)), segment 1 =
  // k1, v1, mask1 through kv1 (Skv1 keys, tiles from nt0 on).  Each segment's
  // last tile may be partial.
  const __bf16* k1;
  const __bf16* v1;
  const uint8_t* mask1;
  int Skv1;         // 0: one segment
  int nt0;          // ceil(Skv / BN)
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const uint8_t* mask;
  __bf16* o;
  int B, Sq, Skv, H;
  int m_tiles;  // ceil(Sq / BM)
  int n_work;   // B * H * m_tiles  (query blocks)
  float sc;     // scale * log2(e)
  // Split-KV: with nsplit > 1, workgroup w takes part j = w % nsplit of the key
  // iterations of query block w / nsplit, [n_iter * j / nsplit, n_iter * (j + 1) / nsplit),
  // and writes its partial state to workspace slot w.
  int nsplit;          // 1: one workgroup per query block
  int n_iter_blk;      // iterations per query block: ceil(ceil(Skv / BN) / 2)
  float* ws;           // partial states, slot = query block * nsplit + part:
                       // O [n_work * nsplit][BM][D] fp32, then (m, l) [n_work * nsplit][BM][2]
  // Partial-attention output (instead of o): normalised O [B][Sq][H][D] fp32 and
  // lse = ln(sum of exp(scale q.k) over the valid keys) [B][H][Sq] fp32, over all
  // H_all heads of the call; this launch's head h is head h_base + h there (a call
  // may split its heads between two launches).
  float* o_part;
  float* lse;
  int H_all;
  int h_base;
  // Running state of an attention over earlier key chunks (same format as
  // o_part / lse), folded into this call's result; NULL: none.
  const float* st_o;
  const float* st_lse;
  // Packed documents (varlen variant only): document b takes query rows
  // [cu_q[b], cu_q[b+1]) of the Sq packed rows and key rows [cu_k[b], cu_k[b+1])
  // of the Skv packed keys; B is the document count.  A query block is a BM-row
  // tile of the packed rows (m_tiles = ceil(Sq / BM) per head) and runs every
  // document that has rows in it, one after the other.
  const int* cu_q;
  const int* cu_k;
};

// The body is a device function behind a thin kernel: the LDS address-space
// casts it needs are device-only, and keeping them out of the kernel itself lets
// the host pass emit the kernel's launch stub.
template <int D, int MODE>
__device__ __forceinline__ void attn_fwd_body(const AttnArgs& a) {
  constexpr bool kChunked = (MODE & kModeChunked) != 0;
  constexpr bool kTwoSeg = (MODE & kModeTwoSeg) != 0;
  constexpr bool kCross = (MODE & kModeCross) != 0;
  static_assert(!kCross || kChunked, "tiles cross chunks only in chunked views");
  // Segment 1 with a view of its own (its row stride may differ from segment 0's):
  // it has lane offsets of its own.  Otherwise both segments share K/V's stride.
  constexpr bool kSeg1Rows = (MODE & kModeSeg1Rows) != 0;
  static_assert(!kSeg1Rows || kTwoSeg, "a view of its own for segment 1 needs two segments");
  constexpr bool kVarlen = (MODE & kModeVarlen) != 0;
  static_assert(!kVarlen || MODE == kModeVarlen, "packed documents use plain views and one key segment");
  constexpr bool kSplit = (MODE & kModeSplit) != 0;
  // Wide block: 256 query rows, group g on rows [128 g, 128 g + 128), both groups on
  // every key tile (group 1 one Q K^T ahead, as in the 128-row block), so each K/V
  // tile brought into LDS serves twice the rows.  Not for packed documents or
  // split-KV parts; each wave writes its own rows (bf16 O, or the partial output).
  constexpr bool kWide = (MODE & kModeWide) != 0;
  static_assert(!kWide || (!kVarlen && !kSplit), "the wide block has no packed-document or split-KV form");
  using C = Cfg<D>;
  constexpr int BMB = kWide ? 2 * C::BM : C::BM;  // query rows per workgroup
  // K and V tiles: one array per (operand, key group, buffer).  Separate objects
  // let the compiler see that a fill of one buffer does not alias the reads of
  // another, so no wait for the in-flight fills is inserted before those reads.
  // The compiler lays __shared__ arrays out in name order: the V tiles come first,
  // inside the 64 KB that a ds_read's 16-bit offset reaches, so every transposed V
  // read takes its tile base as an immediate instead of an address add.
  __shared__ __attribute__((aligned(1024))) char lds0_v00[C::TILE], lds0_v01[C::TILE], lds0_v10[C::TILE], lds0_v11[C::TILE];
  __shared__ __attribute__((aligned(1024))) char lds1_k00[C::TILE], lds1_k01[C::TILE], lds1_k10[C::TILE], lds1_k11[C::TILE];
  __shared__ __attribute__((aligned(16))) float lds2_bias[6 * C::BN];
  // Group 1's first K tile, read by its first Q K^T right after the prologue
  // barrier.  It has a buffer of its own because group 0's first in-loop fills,
  // issued in the same interval, overwrite group 1's K buffer 0 with its third
  // tile; nothing orders those writes after that read.
  __shared__ __attribute__((aligned(1024))) char lds3_k1first[C::TILE];
  // Wide block: V tile i in buffer i % 2, K tile i in buffer i % 4 (group 0 reads K
  // tile i and group 1 K tile i + 1 while tile i + 2 is being filled).  The V
  // buffers again come first, below the K buffers.
  __shared__ __attribute__((aligned(1024))) char lds0_w_v0[C::TILE], lds0_w_v1[C::TILE];
  __shared__ __attribute__((aligned(1024))) char lds1_w_k0[C::TILE], lds1_w_k1[C::TILE], lds1_w_k2[C::TILE],
      lds1_w_k3[C::TILE];

  const int tid = threadIdx.x;
  // Wave-uniform indices go through readfirstlane so that the compiler keeps
  // them (and the buffer descriptors and LDS bases built from them) scalar.
  const int grp = __builtin_amdgcn_readfirstlane(tid / kGroupThreads);  // key-tile group
  const int gt = tid % kGroupThreads;                                   // thread index in the group
  const int gw = __builtin_amdgcn_readfirstlane(gt >> 6);               // wave index in the group
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;  // half of the wave: selects the 8-wide k slice of an MFMA operand

  // One segment: query block `work`, iterations [i0, i1) of it.  slot_idx < 0:
  // the segment is the whole block and writes O; otherwise it writes its
  // partial state to workspace slot slot_idx.
  // vdoc: the document a packed-documents block runs (varlen variant only).
  auto process = [&](int work, int i0, int i1, int slot_idx, int vdoc) {
  // Packed documents: query block = (head, BM-row tile of the packed rows), numbered
  // head-major so that one head's blocks stay on one XCD.
  const int mt = kVarlen ? 0 : work % a.m_tiles;
  const int bh = work / a.m_tiles;
  const int h = kVarlen ? bh : bh % a.H;
  const int b = kVarlen ? vdoc : bh / a.H;
  // Query rows [q_lo, Sq) of the block (relative to q_boff) and keys of its batch row.
  int q_lo = 0, Sq = a.Sq, Skv = a.Skv;
  long long q_boff = (long long)b * a.qv.bs, kv_boff = (long long)b * a.kv.bs, o_boff = (long long)b * a.ov.bs;
  if constexpr (kVarlen) {
    // The boundaries are read from device memory: clamp them into the packed
    // buffers so that malformed ones cannot address outside them.
    const int r0 = (work % a.m_tiles) * C::BM;  // packed row of the tile's first row
    const int q0 = min(max(a.cu_q[b], 0), a.Sq), q1 = min(max(a.cu_q[b + 1], q0), a.Sq);
    const int k0 = min(max(a.cu_k[b], 0), a.Skv), k1 = min(max(a.cu_k[b + 1], k0), a.Skv);
    q_lo = __builtin_amdgcn_readfirstlane(q0 - r0);
    Sq = __builtin_amdgcn_readfirstlane(q1 - r0);
    Skv = __builtin_amdgcn_readfirstlane(k1 - k0);
    q_boff = (long long)r0 * a.qv.rs;
    o_boff = (long long)r0 * a.ov.rs;
    kv_boff = (long long)__builtin_amdgcn_readfirstlane(k0) * a.kv.rs;
    if (Skv == 0) {
      // no key: the document's rows in this tile are zero
      constexpr int kVec = D / 8;
      for (int e = tid; e < C::BM * kVec; e += kThreads) {
        const int row = e / kVec;
        if (row >= q_lo && row < Sq)
          *reinterpret_cast<uint4*>(a.o + o_boff + (long long)row * a.ov.rs + h * a.ov.hs + (e % kVec) * 8) =
              make_uint4(0u, 0u, 0u, 0u);
      }
      return;
    }
  }
  const __bf16* kbase = a.k + kv_boff + h * a.kv.hs;
  const __bf16* vbase = a.v + kv_boff + h * a.kv.hs;
  const uint8_t* mbase = a.mask ? a.mask + size_t(b) * a.Skv : nullptr;
  const __bf16* kbase1 = kbase;  // segment 1 (two-segment variant only)
  const __bf16* vbase1 = vbase;
  const uint8_t* mbase1 = nullptr;
  if constexpr (kTwoSeg) {
    const size_t seg1_off = size_t(b) * a.kv1.bs + size_t(h) * a.kv1.hs;
    kbase1 = a.k1 + seg1_off;
    vbase1 = a.v1 + seg1_off;
    mbase1 = a.mask1 ? a.mask1 + size_t(b) * a.Skv1 : nullptr;
  }
  // Segment of tile t and its first key there (one segment: tile t, key t * BN).
  auto seg_of = [&](int t, bool& s1, int& key0, int& len) {
    if constexpr (kTwoSeg) {
      s1 = t >= a.nt0;
      key0 = (s1 ? t - a.nt0 : t) * C::BN;
      len = s1 ? a.Skv1 : a.Skv;
    } else {
      s1 = false;
      key0 = t * C::BN;
      len = Skv;
    }
  };

  // ---- Q fragment (B operand of S^T = K Q^T): query row q_row, d = ks*16 + 8*hi .. +8
  const int q_row = mt * BMB + (kWide ? grp * C::BM : 0) + gw * 32 + l32;
  // A wave whose 32 rows all lie past the last query row (the last block of a
  // head when Sq is not a multiple of the block) only issues its share of the
  // fills and bias rows and meets every barrier: its MFMA and softmax work would
  // go to rows that are never stored.
  const bool idle = !kVarlen && __builtin_amdgcn_readfirstlane(q_row - l32) >= Sq;
  bf16x8 qf[C::KS];
  {
    const bool ok = q_row < Sq && q_row >= q_lo;
    const __bf16* qp = a.q + q_boff + row_off_t<kChunked>(a.qv, ok ? q_row : 0) + h * a.qv.hs;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      bf16x8 t = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + 8 * hi);
      if (!ok) t = bf16x8{};
      qf[ks] = t;
    }
  }

  const int n_tiles = kTwoSeg ? a.nt0 + (a.Skv1 + C::BN - 1) / C::BN : (Skv + C::BN - 1) / C::BN;
  // iterations of every wave in this segment (a document: all of its key tiles)
  const int n_iter = kVarlen ? (n_tiles + 1) / 2 : i1 - i0;
  // tiles of key group g in the segment: global tiles 2 (i0 + j) + g < n_tiles (wide
  // block: both groups take every tile, i0 + j < n_tiles)
  auto tiles_of_group = [&](int g) {
    return kWide ? min(n_iter, max(0, n_tiles - i0)) : min(n_iter, max(0, (n_tiles - g + 1) / 2 - i0));
  };
  const int n_g = tiles_of_group(grp);
  auto tile_of = [&](int i) { return kWide ? i0 + i : 2 * (i0 + i) + grp; };

  // ---- HBM -> LDS fill.  Slot s of a tile (16 bytes) holds chunk
  // (s % CHUNKS) ^ swz(key) of row key = s / CHUNKS; instruction j of wave gw
  // fills slots [(gw*SPT + j)*64, +64), lane-ordered.  The SPT instructions of a
  // wave share one LDS base (the M0 register): instruction j carries its 1 KB step
  // as the immediate offset, which the hardware adds to both the LDS and the
  // global address, so the lane offsets are stored 1 KB * j low.
  const uint32_t rs_bytes = uint32_t(a.kv.rs) * 2u;
  uint32_t goff[C::SPT];
#pragma unroll
  for (int j = 0; j < C::SPT; ++j) {
    const int slot = (gw * C::SPT + j) * 64 + lane;
    const int key = slot / C::CHUNKS;
    const int chunk = (slot % C::CHUNKS) ^ C::swz(key);
    goff[j] = uint32_t(key) * rs_bytes + uint32_t(chunk) * 16u - uint32_t(j) * 1024u;
  }
  const uint32_t rs1_bytes = uint32_t(a.kv1.rs) * 2u;
  uint32_t goff1[C::SPT];
#pragma unroll
  for (int j = 0; j < C::SPT; ++j) {
    if constexpr (kSeg1Rows) {
      const int slot = (gw * C::SPT + j) * 64 + lane;
      const int key = slot / C::CHUNKS;
      const int chunk = (slot % C::CHUNKS) ^ C::swz(key);
      goff1[j] = uint32_t(key) * rs1_bytes + uint32_t(chunk) * 16u - uint32_t(j) * 1024u;
    } else {
      goff1[j] = 0u;
    }
  }
  static_assert(C::SPT == 2 || C::SPT == 4, "fill instructions per wave");
  // off: the lane offset of instruction j (goff[j], or xoff for a tile that
  // spans chunks).
  auto fill_j = [&](int j, __amdgpu_buffer_rsrc_t rs, char* dst, uint32_t off) {
    lds_void* const d = (lds_void*)(dst + gw * C::SPT * 1024);
    switch (j) {
      case 0: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, off, 0, 0, 0); break;
      case 1: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, off, 0, 1024, 0); break;
      case 2: if constexpr (C::SPT > 2) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, off, 0, 2048, 0); break;
      default: if constexpr (C::SPT > 3) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, off, 0, 3072, 0); break;
    }
  };
  // A tile of a chunked view whose chunks are not a multiple of 64 rows can span
  // two or more chunks: its rows are then not at one stride from the tile's first
  // row.  Such a tile takes per-lane offsets row_off(key0 + key) - row_off(key0)
  // (rows past the last key get an offset outside the range and read as zero) and
  // a range up to its last row.
  auto crosses = [&](const View& v, int key0, int rows) -> bool {
    if constexpr (!kCross) {
      (void)v;
      (void)key0;
      (void)rows;
      return false;
    } else {
      if (kSeg1Rows && !v.chunked) return false;
      uint32_t c, r;
      v.L.divmod(uint32_t(key0), c, r);
      return int(r) + rows > int(v.L.d);
    }
  };
  auto xoff = [&](const View& v, int j, int key0, int rows) -> uint32_t {
    const int slot = (gw * C::SPT + j) * 64 + lane;
    const int key = slot / C::CHUNKS;
    const int chunk = (slot % C::CHUNKS) ^ C::swz(key);
    if (key >= rows) return 0x80000000u;
    const long long dr = row_off_t<true>(v, key0 + key) - row_off_t<true>(v, key0);
    return uint32_t(dr) * 2u + uint32_t(chunk) * 16u - uint32_t(j) * 1024u;
  };
  auto tile_bytes = [&](const View& v, int key0, int rows, bool cr) -> int {
    if (kCross && cr) {
      const long long last = row_off_t<true>(v, key0 + rows - 1) - row_off_t<true>(v, key0);
      return int(uint32_t(last) * 2u + uint32_t(D) * 2u);
    }
    return int(uint32_t(rows - 1) * (kSeg1Rows ? uint32_t(v.rs) * 2u : rs_bytes) + uint32_t(D) * 2u);
  };
  // The source of tile t (which: 0 = K, 1 = V): its buffer descriptor, and for a
  // tile that spans chunks its first key and row count.  The 64 rows of a tile are
  // otherwise contiguous at stride rs; rows past the last key are outside the range.
  struct FillSrc {
    __amdgpu_buffer_rsrc_t rs;
    int key0, rows;
    bool seg1, cross;
  };
  // segc: the segment of tile t when the caller knows it at compile time (0 or 1),
  // so that the choice of base, view and lane offsets folds away; -1: from t.
  auto fill_src_in = [&](auto segc, int which, int t) -> FillSrc {
    constexpr int SG = decltype(segc)::value;
    bool s1;
    int key0, len;
    if constexpr (kTwoSeg && SG >= 0) {
      s1 = SG == 1;
      key0 = (SG == 1 ? t - a.nt0 : t) * C::BN;
      len = SG == 1 ? a.Skv1 : a.Skv;
    } else {
      seg_of(t, s1, key0, len);
    }
    const int rows = min(C::BN, len - key0);
    // (plain two-segment calls share K/V's row stride: segment 1 only changes the base)
    const View& v = (kSeg1Rows && s1) ? a.kv1 : a.kv;
    const bool cr = crosses(v, key0, rows);
    const __bf16* src = (s1 ? (which ? vbase1 : kbase1) : (which ? vbase : kbase)) + row_off_t<kChunked>(v, key0);
    return {__builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(src), (short)0, tile_bytes(v, key0, rows, cr),
                                              0x00020000),
            key0, rows, s1, cr};
  };
  using SegDyn = std::integral_constant<int, -1>;
  using Seg0 = std::integral_constant<int, 0>;
  using Seg1 = std::integral_constant<int, 1>;
  auto fill_src = [&](int which, int t) -> FillSrc { return fill_src_in(SegDyn{}, which, t); };
  // Instruction j of a tile's fill into the tile array dst.
  auto fill_one = [&](const FillSrc& f, int j, char* dst) {
    fill_j(j, f.rs, dst,
           (kCross && f.cross) ? xoff((kSeg1Rows && f.seg1) ? a.kv1 : a.kv, j, f.key0, f.rows)
                               : ((kSeg1Rows && f.seg1) ? goff1[j] : goff[j]));
  };
  // A whole tile.
  auto fill = [&](int which, int t, char* dst) {
    const FillSrc f = fill_src(which, t);
#pragma unroll
    for (int j = 0; j < C::SPT; ++j) fill_one(f, j, dst);
  };
  // Tile arrays of key group G, buffer B (both compile-time).
  auto ktile = [&](auto g, auto bf) -> char* {
    constexpr int G = decltype(g)::value, B = decltype(bf)::value;
    return G == 0 ? (B == 0 ? lds1_k00 : lds1_k01) : (B == 0 ? lds1_k10 : lds1_k11);
  };
  auto vtile = [&](auto g, auto bf) -> char* {
    constexpr int G = decltype(g)::value, B = decltype(bf)::value;
    return G == 0 ? (B == 0 ? lds0_v00 : lds0_v01) : (B == 0 ? lds0_v10 : lds0_v11);
  };
  // Wide block: K tile buffer B (0..3), V tile buffer B (0..1).
  auto wktile = [&](auto bf) -> char* {
    constexpr int B = decltype(bf)::value;
    return B == 0 ? lds1_w_k0 : B == 1 ? lds1_w_k1 : B == 2 ? lds1_w_k2 : lds1_w_k3;
  };
  auto wvtile = [&](auto bf) -> char* {
    constexpr int B = decltype(bf)::value;
    return B == 0 ? lds0_w_v0 : lds0_w_v1;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  const int n_g1 = tiles_of_group(1);  // tiles of group 1 (local tile i is global tile 2(i0 + i) + 1)
  // Bias rows: group 0 keeps tile i's row in slot i % 2, group 1 in slot i % 4 (it
  // reads a row one iteration later, at the top of the iteration that uses it, so a
  // row is rewritten only after a barrier has followed its last read).
  // (wide block: one row per tile, slot i % 2, written by group 0 and read by both)
  float* bias_row = lds2_bias + (kWide ? 0 : grp * 2 * C::BN);

  // Key validity of tile t as an additive bias, one key per lane.  The mask byte
  // is loaded here and only compared when the bias row is stored, late in the
  // iteration, so its load latency is never waited on early.  Wave 0 of the
  // group writes the row; with a mask every wave also keeps, per bias slot, a bit
  // that says whether the tile has an invalid key (mflags), so that a tile whose
  // keys are all valid skips the bias (most tiles of a padding mask).
  const bool has_mask = mbase != nullptr || mbase1 != nullptr;
  bool kvalid = true;
  uint32_t mraw = 1;
  uint32_t mflags = 0;
  auto bias_of = [&](int t) {
    if (gt < C::BN || has_mask) {
      bool s1;
      int key0, len;
      seg_of(t, s1, key0, len);
      const int key = key0 + lane;
      kvalid = key < len;
      const uint8_t* mb = s1 ? mbase1 : mbase;
      mraw = mb ? uint32_t(mb[kvalid ? key : 0]) : 1u;
    }
  };
  auto note_bias = [&](int buf) {
    if (has_mask) {
      const uint32_t bit = 1u << buf;
      mflags = __builtin_amdgcn_ballot_w64(!(kvalid && mraw != 0)) != 0 ? (mflags | bit) : (mflags & ~bit);
    }
  };
  auto store_bias = [&](int buf) {
    if (gt < C::BN) bias_row[buf * C::BN + gt] = (kvalid && mraw != 0) ? 0.f : -INFINITY;
    note_bias(buf);
  };

  // ---- LDS readers
  // K operand of S^T: row kb*32 + l32, chunk 2*kk + hi  ->  byte kb*32*RB + (kaddr ^ (kk * 32))
  const int kswz = C::swz(l32);
  const int kaddr = l32 * C::RB + ((hi ^ (kswz & 1)) * 16) + (kswz & ~1) * 16;
  // With D = 128 the K tiles lie above the 64 KB that a ds_read offset reaches
  // (the V tiles fill it): the per-step lane addresses are kept kKHigh bytes high,
  // opaque to the optimiser so it cannot fold the constant back, and reads address
  // from tile - kKHigh, so the tile base and the 32-key block fit the offset field.
  constexpr int kKHigh = kWide ? (6 * C::TILE > 65536 ? 2 * C::TILE : 0) : (4 * C::TILE >= 65536 ? 65536 : 0);
  uint32_t kx[C::KS];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) {
    kx[kk] = uint32_t(kaddr ^ (kk * 32)) + uint32_t(kKHigh);
    asm volatile("" : "+v"(kx[kk]));
  }
  // V^T operand: lane (G = lane/16, i = lane%16) reads row 16m + 8r + 4hi + i/4, head-dim
  // 32db + 16(G%2) + 4(i%4) .. +4  ->  byte (16m + 8r) * RB + (vaddr_r ^ (db * 64))
  // (r = 0 / 1 for the first / second four keys of the step).
  const int vG = lane >> 4, vi = lane & 15;
  const int vrow = 4 * hi + vi / 4;
  const int vj = 2 * (vG & 1) + ((vi & 3) >> 1);  // chunk within the 4-chunk group of this db
  auto vaddr_of = [&](int r) {
    const int f = C::swz(8 * r + vrow);
    return vrow * C::RB + (vi & 1) * 8 + (vj ^ (f & 3)) * 16 + (f >> 2) * 64;
  };
  const int vaddr0 = vaddr_of(0), vaddr1 = vaddr_of(1);

  // S^T[key][query] of one tile (two 32-key blocks).  The two blocks' MFMA chains
  // are interleaved step by step, so each chain's dependent MFMA and each K read
  // have the other chain's MFMA to hide behind.
  auto qk = [&](const char* kt, f32x16* s) {
    f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) {
      const bf16x8 kf0 = *reinterpret_cast<const bf16x8*>(kt - kKHigh + kx[kk]);
      const bf16x8 kf1 = *reinterpret_cast<const bf16x8*>(kt - kKHigh + 32 * C::RB + kx[kk]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[kk], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf1, qf[kk], acc1, 0, 0, 0);
    }
    s[0] = acc0;
    s[1] = acc1;
  };
  // Bias (tail / mask) and the scaled tile max over this query's 64 keys.
  // Accumulator row r of block kb is key kb*32 + 8*(r/4) + 4*hi + r%4.
  auto bias_max = [&](int buf, int t, f32x16* s) -> float {
    bool s1;
    int key0, len;
    seg_of(t, s1, key0, len);
    if (key0 + C::BN > len || ((s1 ? mbase1 : mbase) != nullptr && ((mflags >> buf) & 1u) != 0)) {
      const float* br = bias_row + buf * C::BN;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 bb = *reinterpret_cast<const float4*>(br + kb * 32 + 8 * g + 4 * hi);
          s[kb][4 * g + 0] += bb.x;
          s[kb][4 * g + 1] += bb.y;
          s[kb][4 * g + 2] += bb.z;
          s[kb][4 * g + 3] += bb.w;
        }
    }
    return pair_max(max_of_32(s[0], s[1])) * a.sc;
  };
  f32x16 acc_o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc_o[db] = f32x16{};

  float m_run = -INFINITY;  // running max, scaled log2 units (shared by lanes l, l^32)
  float nm_use = 0.f;       // -m_run, or 0 while m_run is -inf (the softmax's offset)
  float l_run = 0.f;        // this lane's partial row sum
  f32x16 sc[2];             // scores of one tile

  // Raise the running max to a tile max that exceeds it by more than 8.
  auto rescale = [&](float mt_tile) {
    const bool raise = mt_tile > m_run + 8.0f;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float m_new = raise ? mt_tile : m_run;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
      m_run = m_new;
      nm_use = m_run == -INFINITY ? 0.f : -m_run;
    }
  };
  // Half-tile pieces (keys 32*kb .. 32*kb + 31) of the softmax and the P V
  // product; both groups run each half's P V right after that half's softmax.
  // Probabilities go to B-operand order (step m uses block m/2, rows 8*(m%2) .. +8),
  // and the bf16 values are summed; O^T[d][query] += V^T[d][keys] P^T[keys][query].
  auto softmax_part = [&](const f32x16* s, int kb, bf16x8* pf) -> float {
    float lsum = 0.f;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int m = 2 * kb; m < 2 * kb + 2; ++m) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        pf[m][kk] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][8 * (m & 1) + kk], a.sc, nm_use));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x2 pr = {pf[m][2 * j], pf[m][2 * j + 1]};
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
      }
    }
    return lsum;
  };
  auto pv_part = [&](const char* vt, const bf16x8* pf, int kb) {
#pragma unroll
    for (int m = 2 * kb; m < 2 * kb + 2; ++m)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const i16x4 lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + 16 * m * C::RB + (vaddr0 ^ (db * 64))));
        const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vt + (16 * m + 8) * C::RB + (vaddr1 ^ (db * 64))));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[m], acc_o[db], 0, 0, 0);
      }
  };
  // Q K^T whose steps are interleaved with up to 16 fill instructions: after step
  // kk, fills 3kk .. 3kk+2 of the list (tile f / SPT, instruction f % SPT), so the
  // last ones go out by two thirds of the chain.  Scheduling fences keep the fills
  // in place while MFMAs and LDS reads move freely.
  auto qk_fills = [&](const char* kt, f32x16* s, const FillSrc* fs, char* const* dst, int n_fill_tiles) {
    f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) {
      const bf16x8 kf0 = *reinterpret_cast<const bf16x8*>(kt - kKHigh + kx[kk]);
      const bf16x8 kf1 = *reinterpret_cast<const bf16x8*>(kt - kKHigh + 32 * C::RB + kx[kk]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[kk], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf1, qf[kk], acc1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0x078F);
#pragma unroll
      for (int f = 3 * kk; f < 3 * kk + 3 && f < 4 * C::SPT; ++f) {
        const int tile = f / C::SPT, j = f % C::SPT;
        if (tile < n_fill_tiles) fill_one(fs[tile], j, dst[tile]);
      }
      __builtin_amdgcn_sched_barrier(0x078F);
    }
    s[0] = acc0;
    s[1] = acc1;
  };

  // Partial output of this wave's rows: the call's normalised output and lse over
  // its keys, folded into the running state when there is one: L = ln(e^lse_s +
  // e^lse_k), O = e^(lse_s - L) O_s + e^(lse_k - L) O_k.  Output: fp32 O and L
  // (o_part, lse), or bf16 O (o).  The state is acc_o scaled by c0, plus (merged:
  // the 128-row block) the other group's accumulators cb scaled by c1; mm and l_tot
  // are its max and row sum, in the kernel's log2 units.
  float4 cb[C::DB][4];  // the other group's O (128-row block, group 0 after the merge)
  auto emit_partial = [&](auto merged, float mm, float l_tot, float c0, float c1) {
    constexpr bool kMerged = decltype(merged)::value;
    if (q_row >= a.Sq) return;
    const int hh = a.h_base + h;
    const size_t orow = ((size_t(b) * a.Sq + q_row) * a.H_all + hh) * D;
    const size_t lidx = (size_t(b) * a.H_all + hh) * a.Sq + q_row;
    // sum_j e^{z_j} = 2^mm * l_tot
    const float lse_k = l_tot > 0.f ? (mm + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    float L = lse_k, wk = 1.f, ws = 0.f;
    const float* sp = nullptr;
    if (a.st_o != nullptr) {
      const float lse_s = a.st_lse[lidx];
      if (lse_s != -INFINITY) {
        sp = a.st_o + orow;
        if (lse_k == -INFINITY) {
          L = lse_s;
          ws = 1.f;
          wk = 0.f;
        } else {
          L = fmaxf(lse_s, lse_k) + log1pf(expf(-fabsf(lse_s - lse_k)));
          ws = expf(lse_s - L);
          wk = expf(lse_k - L);
        }
      }
    }
    const float k0 = c0 * wk, k1 = c1 * wk;
    float4 out[C::DB][4];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 w;
        w.x = acc_o[db][4 * g + 0] * k0;
        w.y = acc_o[db][4 * g + 1] * k0;
        w.z = acc_o[db][4 * g + 2] * k0;
        w.w = acc_o[db][4 * g + 3] * k0;
        if constexpr (kMerged) {
          w.x += cb[db][g].x * k1;
          w.y += cb[db][g].y * k1;
          w.z += cb[db][g].z * k1;
          w.w += cb[db][g].w * k1;
        } else {
          (void)k1;
        }
        if (sp != nullptr) {
          const float4 sv = *reinterpret_cast<const float4*>(sp + db * 32 + 8 * g + 4 * hi);
          w.x += ws * sv.x;
          w.y += ws * sv.y;
          w.z += ws * sv.z;
          w.w += ws * sv.w;
        }
        out[db][g] = w;
      }
    if (a.o_part != nullptr) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(a.o_part + orow + db * 32 + 8 * g + 4 * hi) = out[db][g];
      if (hi == 0) a.lse[lidx] = L;
    } else {
      __bf16* op = a.o + b * a.ov.bs + row_off_t<kChunked>(a.ov, q_row) + h * a.ov.hs;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 w;
          w[0] = (__bf16)out[db][g].x;
          w[1] = (__bf16)out[db][g].y;
          w[2] = (__bf16)out[db][g].z;
          w[3] = (__bf16)out[db][g].w;
          *reinterpret_cast<bf16x4*>(op + db * 32 + 8 * g + 4 * hi) = w;
        }
    }
  };

  if constexpr (!kWide) {
  // ---- prologue.  Group 0 consumes K and V of tile i in iteration i; group 1
  // runs one K tile ahead (its iteration i ends with the scores of tile i+1, whose
  // max it takes at the top of iteration i+1, while group 0 is in its Q K^T).
  // Only group 0 issues HBM->LDS fills, for both groups' buffers: fill
  // instructions stall at issue while the texture path drains, and group 1 is
  // the one on the critical path.
  if (grp == 0) {
    if (n_g > 0) {
      fill(0, 2 * (i0 + 0) + 0, ktile(I0{}, I0{}));
      fill(1, 2 * (i0 + 0) + 0, vtile(I0{}, I0{}));
    }
    if (n_g1 > 0) {
      fill(0, 2 * (i0 + 0) + 1, lds3_k1first);
      fill(1, 2 * (i0 + 0) + 1, vtile(I1{}, I0{}));
    }
    if (n_g1 > 1) fill(0, 2 * (i0 + 1) + 1, ktile(I1{}, I1{}));
  }
  if (n_g > 0) {
    bias_of(tile_of(0));
    store_bias(0);
  }
  if (grp == 1 && n_g > 1) {
    bias_of(tile_of(1));
    store_bias(1);
  }
  if (grp == 1 && n_g > 2) {
    bias_of(tile_of(2));
    store_bias(2);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's LDS fills have landed
  __syncthreads();

  // ---- main loop; every wave runs n_iter iterations so that barriers match.
  // On each SIMD one wave of each group runs; right after every barrier group 0
  // is in its Q K^T MFMAs while group 1 is in its softmax VALU work, then the
  // roles swap, so the matrix pipe and the VALU overlap across the two waves.
  // Iterations come in pairs so that every buffer choice is compile-time.
  if (grp == 0 && idle) {
    // the fills and bias rows of iter0 below, without its MFMA and softmax work
    auto iter0_idle = [&](auto par, int i) {
      constexpr int P = decltype(par)::value;
      using BP = std::integral_constant<int, P>;
      using BQ = std::integral_constant<int, 1 - P>;
      if (i < n_g) {
        const bool nx = i + 1 < n_g;
        const bool want[4] = {nx, nx, i + 2 < n_g1, i + 1 < n_g1};
        const int tc = 2 * (i0 + i);
        const int tl[4] = {want[0] ? 2 * (i0 + i + 1) : tc, want[1] ? 2 * (i0 + i + 1) : tc,
                           want[2] ? 2 * (i0 + i + 2) + 1 : tc, want[3] ? 2 * (i0 + i + 1) + 1 : tc};
        const FillSrc fs[4] = {fill_src(1, tl[3]), fill_src(0, tl[0]), fill_src(1, tl[1]), fill_src(0, tl[2])};
        char* const dst[4] = {vtile(I1{}, BQ{}), ktile(I0{}, BQ{}), vtile(I0{}, BQ{}), ktile(I1{}, BP{})};
#pragma unroll
        for (int f = 0; f < 4 * C::SPT; ++f) fill_one(fs[f / C::SPT], f % C::SPT, dst[f / C::SPT]);
        if (nx) {
          bias_of(tile_of(i + 1));
          store_bias(1 - P);
        }
      }
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
    };
    for (int i = 0; i < n_iter; i += 2) {
      iter0_idle(I0{}, i);
      if (i + 1 < n_iter) iter0_idle(I1{}, i + 1);
    }
  } else if (grp == 0) {
    auto iter0 = [&](auto par, auto segc, int i) {
      constexpr int P = decltype(par)::value;
      using BP = std::integral_constant<int, P>;
      using BQ = std::integral_constant<int, 1 - P>;
      if (i < n_g) {
        const bool nx = i + 1 < n_g;
        // the fills of the next tiles (both groups) go out three at a time between
        // the Q K^T steps: issued at the top of the iteration they held back the first
        // MFMAs (a fill can stall at issue while the texture path drains); spread
        // over the chain, their stalls overlap MFMA execution.  Group 1's V tile,
        // which it reads first in the next iteration, goes first.  They are issued
        // unconditionally (no branches in the chain): a tile past the end of its
        // group is replaced by this iteration's tile, re-read into a buffer that
        // nothing reads before the next fill of it.
        {
          const bool want[4] = {nx, nx, i + 2 < n_g1, i + 1 < n_g1};
          const int tc = 2 * (i0 + i);
          const int tl[4] = {want[0] ? 2 * (i0 + i + 1) : tc, want[1] ? 2 * (i0 + i + 1) : tc,
                             want[2] ? 2 * (i0 + i + 2) + 1 : tc, want[3] ? 2 * (i0 + i + 1) + 1 : tc};
          const FillSrc fs[4] = {fill_src_in(segc, 1, tl[3]), fill_src_in(segc, 0, tl[0]),
                                 fill_src_in(segc, 1, tl[1]), fill_src_in(segc, 0, tl[2])};
          char* const dst[4] = {vtile(I1{}, BQ{}), ktile(I0{}, BQ{}), vtile(I0{}, BQ{}), ktile(I1{}, BP{})};
          qk_fills(ktile(I0{}, BP{}), sc, fs, dst, 4);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (nx) bias_of(tile_of(i + 1));
        rescale(bias_max(P, tile_of(i), sc));
        {
          bf16x8 pf[4];
          float lsum = softmax_part(sc, 0, pf);
          pv_part(vtile(I0{}, BP{}), pf, 0);
          lsum += softmax_part(sc, 1, pf);
          pv_part(vtile(I0{}, BP{}), pf, 1);
          l_run += lsum;
        }
        if (nx) store_bias(1 - P);
      }
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
    };
    // Two key segments: the pairs of iterations whose fills (tiles 2(i0+i) ..
    // 2(i0+i+3)+1) all lie in segment 0, then those that straddle the boundary,
    // then those in segment 1, each run as a loop of its own with the fills'
    // segment fixed where it is known.
    auto pair = [&](auto segc, int i) {
      iter0(I0{}, segc, i);
      if (i + 1 < n_iter) iter0(I1{}, segc, i + 1);
    };
    int i = 0;
    if constexpr (kTwoSeg) {
      for (; i < n_iter && 2 * (i0 + i + 3) + 1 < a.nt0; i += 2) pair(Seg0{}, i);
      for (; i < n_iter && 2 * (i0 + i) < a.nt0; i += 2) pair(SegDyn{}, i);
      for (; i < n_iter; i += 2) pair(Seg1{}, i);
    } else {
      for (; i < n_iter; i += 2) pair(SegDyn{}, i);
    }
  } else if (idle) {
    // the bias rows of iter1 below, without its MFMA and softmax work
    for (int i = 0; i < n_iter; ++i) {
      if (i < n_g && i + 3 < n_g) {
        bias_of(tile_of(i + 3));
        store_bias((i + 3) & 3);
      }
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
    }
  } else {
    if (n_g > 0) {
      qk(lds3_k1first, sc);
    }
    auto iter1 = [&](auto par, int i) {
      constexpr int P = decltype(par)::value;
      using BP = std::integral_constant<int, P>;
      using BQ = std::integral_constant<int, 1 - P>;
      if (i < n_g) {
        const bool nk = i + 3 < n_g;
        if (nk) bias_of(tile_of(i + 3));
        // tile i's max: its scores were finished by the previous iteration; taken
        // here, after the barrier, it overlaps group 0's Q K^T instead of delaying
        // this group's arrival at the barrier
        rescale(bias_max(i & 3, tile_of(i), sc));
        __builtin_amdgcn_sched_barrier(0);
        // tile i's softmax and P V in two halves, then tile i+1's Q K^T as two
        // interleaved chains (none after the group's last tile).  The second half's
        // softmax then runs while group 0 is in its P V MFMAs, and this group's
        // Q K^T while group 0 waits for its fills.
        {
          bf16x8 pf[4];
          float lsum = softmax_part(sc, 0, pf);
          pv_part(vtile(I1{}, BP{}), pf, 0);
          lsum += softmax_part(sc, 1, pf);
          pv_part(vtile(I1{}, BP{}), pf, 1);
          if (i + 1 < n_g) qk(ktile(I1{}, BQ{}), sc);
          l_run += lsum;
        }
        __builtin_amdgcn_sched_barrier(0);
        if (nk) store_bias((i + 3) & 3);
      }
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
    };
    for (int i = 0; i < n_iter; i += 2) {
      iter1(I0{}, i);
      if (i + 1 < n_iter) iter1(I1{}, i + 1);
    }
  }
  } else {
  // ---- wide block.  Iteration i: group 0 runs Q K^T of tile i (K buffer i % 4) with
  // the fills of V tile i + 1 and K tile i + 2 between its steps, then the max,
  // softmax and P V (V buffer i % 2); group 1 takes the max, softmax and P V of
  // tile i (scores from the previous iteration), then Q K^T of tile i + 1.  During
  // iteration i the buffers being filled held V tile i - 1 and K tile i - 2, last
  // read no later than iteration i - 1.  Group 0 issues every fill and writes the
  // bias rows (tile i in slot i % 2), which both groups read in iteration i.
  if (grp == 0) {
    if (n_g > 0) {
      fill(0, tile_of(0), wktile(I0{}));
      fill(1, tile_of(0), wvtile(I0{}));
      bias_of(tile_of(0));
      store_bias(0);
    }
    if (n_g > 1) fill(0, tile_of(1), wktile(I1{}));
  } else if (has_mask && n_g > 0) {
    // group 1 keeps its own mask bits (group 0 writes the rows)
    bias_of(tile_of(0));
    note_bias(0);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's LDS fills have landed
  __syncthreads();
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  if (grp == 0 && idle) {
    // the fills and bias rows of iterw0 below, without its MFMA and softmax work
    for (int i = 0; i < n_iter; ++i) {
      if (i < n_g) {
        const bool nx = i + 1 < n_g;
        const int tc = tile_of(i);
        const FillSrc fv = fill_src(1, nx ? tc + 1 : tc), fk = fill_src(0, i + 2 < n_g ? tc + 2 : tc);
        char* const dv = (i & 1) ? wvtile(I0{}) : wvtile(I1{});
        char* const dk = (i & 3) == 0 ? wktile(I2{}) : (i & 3) == 1 ? wktile(I3{}) : (i & 3) == 2 ? wktile(I0{})
                                                                                                  : wktile(I1{});
#pragma unroll
        for (int j = 0; j < C::SPT; ++j) fill_one(fv, j, dv);
#pragma unroll
        for (int j = 0; j < C::SPT; ++j) fill_one(fk, j, dk);
        if (nx) {
          bias_of(tile_of(i + 1));
          store_bias((i + 1) & 1);
        }
      }
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
    }
  } else if (grp == 0) {
    auto iterw0 = [&](auto par, auto segc, int i) {
      constexpr int P = decltype(par)::value;  // i % 4
      using V0 = std::integral_constant<int, P % 2>;
      using V1 = std::integral_constant<int, (P + 1) % 2>;
      using K0 = std::integral_constant<int, P>;
      using K2 = std::integral_constant<int, (P + 2) % 4>;
      if (i < n_g) {
        const bool nx = i + 1 < n_g;
        {
          // past the last tile the current one is re-read into a buffer whose
          // contents nothing reads before its next fill
          const int tc = tile_of(i);
          const FillSrc fs[2] = {fill_src_in(segc, 1, nx ? tc + 1 : tc), fill_src_in(segc, 0, i + 2 < n_g ? tc + 2 : tc)};
          char* const dst[2] = {wvtile(V1{}), wktile(K2{})};
          qk_fills(wktile(K0{}), sc, fs, dst, 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (nx) bias_of(tile_of(i + 1));
        rescale(bias_max(P % 2, tile_of(i), sc));
        {
          bf16x8 pf[4];
          float lsum = softmax_part(sc, 0, pf);
          pv_part(wvtile(V0{}), pf, 0);
          lsum += softmax_part(sc, 1, pf);
          pv_part(wvtile(V0{}), pf, 1);
          l_run += lsum;
        }
        if (nx) store_bias((P + 1) % 2);
      }
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
    };
    // (two key segments: runs of four iterations whose fills, tiles i0+i ..
    // i0+i+5, all lie in segment 0, then those straddling the boundary, then
    // those in segment 1, as loops of their own)
    auto quad = [&](auto segc, int i) {
      iterw0(I0{}, segc, i);
      if (i + 1 < n_iter) iterw0(I1{}, segc, i + 1);
      if (i + 2 < n_iter) iterw0(I2{}, segc, i + 2);
      if (i + 3 < n_iter) iterw0(I3{}, segc, i + 3);
    };
    int i = 0;
    if constexpr (kTwoSeg) {
      for (; i < n_iter && i0 + i + 5 < a.nt0; i += 4) quad(Seg0{}, i);
      for (; i < n_iter && i0 + i < a.nt0; i += 4) quad(SegDyn{}, i);
      for (; i < n_iter; i += 4) quad(Seg1{}, i);
    } else {
      for (; i < n_iter; i += 4) quad(SegDyn{}, i);
    }
  } else if (idle) {
    for (int i = 0; i < n_iter; ++i) {
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
    }
  } else {
    if (n_g > 0) qk(wktile(I0{}), sc);
    auto iterw1 = [&](auto par, int i) {
      constexpr int P = decltype(par)::value;  // i % 4
      using V0 = std::integral_constant<int, P % 2>;
      using K1 = std::integral_constant<int, (P + 1) % 4>;
      if (i < n_g) {
        const bool nb = has_mask && i + 1 < n_g;
        if (nb) bias_of(tile_of(i + 1));
        rescale(bias_max(P % 2, tile_of(i), sc));
        __builtin_amdgcn_sched_barrier(0);
        {
          bf16x8 pf[4];
          float lsum = softmax_part(sc, 0, pf);
          pv_part(wvtile(V0{}), pf, 0);
          lsum += softmax_part(sc, 1, pf);
          pv_part(wvtile(V0{}), pf, 1);
          if (i + 1 < n_g) qk(wktile(K1{}), sc);
          l_run += lsum;
        }
        __builtin_amdgcn_sched_barrier(0);
        if (nb) note_bias((P + 1) % 2);
      }
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
    };
    for (int i = 0; i < n_iter; i += 4) {
      iterw1(I0{}, i);
      if (i + 1 < n_iter) iterw1(I1{}, i + 1);
      if (i + 2 < n_iter) iterw1(I2{}, i + 2);
      if (i + 3 < n_iter) iterw1(I3{}, i + 3);
    }
  }
  // Each wave owns whole rows: normalise and store (lanes l and l + 32 hold the two
  // halves of each 8-element run, as in the merged store below).
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (a.o_part != nullptr || a.st_o != nullptr) {
    emit_partial(std::false_type{}, m_run, l_tot, inv, 0.f);
    return;
  }
  const bool o_ok = q_row < Sq && q_row >= q_lo;
  __bf16* op = a.o + o_boff + row_off_t<kChunked>(a.ov, o_ok ? q_row : 0) + h * a.ov.hs;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      bf16x4 w0, w1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0[e] = (__bf16)(acc_o[db][8 * k + e] * inv);
        w1[e] = (__bf16)(acc_o[db][8 * k + 4 + e] * inv);
      }
      const uint2 x = __builtin_bit_cast(uint2, w0), y = __builtin_bit_cast(uint2, w1);
      const auto s0 = __builtin_amdgcn_permlane32_swap(x.x, y.x, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(x.y, y.y, false, false);
      const uint4 out = make_uint4(s0[0], s1[0], s0[1], s1[1]);
      if (o_ok) *reinterpret_cast<uint4*>(op + db * 32 + 8 * (2 * k + hi)) = out;
    }
  return;
  }

  // ---- merge the two groups' softmax states through LDS (reusing the K tile
  // arrays: O of group-1 wave gw in one array each, as float4 columns that
  // consecutive lanes read at consecutive 16-byte slots; m and l in the first V
  // array).  Group 0 issues all its reads before using any.
  float4* comb4 = reinterpret_cast<float4*>(gw == 0 ? lds1_k00 : gw == 1 ? lds1_k01 : gw == 2 ? lds1_k10 : lds1_k11);
  float* comb_ml = reinterpret_cast<float*>(lds0_v00) + gw * 2 * 64;
  auto slot = [&](int k) { return k * 64 + lane; };
  auto cslot = [&](int db, int g) { return (db * 4 + g) * 64 + lane; };
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        comb4[cslot(db, g)] =
            make_float4(acc_o[db][4 * g], acc_o[db][4 * g + 1], acc_o[db][4 * g + 2], acc_o[db][4 * g + 3]);
    comb_ml[slot(0)] = m_run;
    comb_ml[slot(1)] = l_run;
  }
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) cb[db][g] = comb4[cslot(db, g)];
    const float m1 = comb_ml[slot(0)];
    const float l1 = comb_ml[slot(1)];
    const float mm = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
    const float l_tot = pair_sum(a0 * l_run + a1 * l1);
    if (kSplit && slot_idx >= 0) {
      // partial state of this segment: unnormalized O (relative to mm), mm, l
      const size_t prow = size_t(slot_idx) * C::BM + gw * 32 + l32;
      float* wp = a.ws + prow * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float4 w;
          w.x = acc_o[db][4 * g + 0] * a0 + cb[db][g].x * a1;
          w.y = acc_o[db][4 * g + 1] * a0 + cb[db][g].y * a1;
          w.z = acc_o[db][4 * g + 2] * a0 + cb[db][g].z * a1;
          w.w = acc_o[db][4 * g + 3] * a0 + cb[db][g].w * a1;
          *reinterpret_cast<float4*>(wp + db * 32 + 8 * g + 4 * hi) = w;
        }
      if (hi == 0) {
        float* ml = a.ws + size_t(a.n_work) * a.nsplit * C::BM * D + prow * 2;
        ml[0] = mm;
        ml[1] = l_tot;
      }
      return;
    }
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float c0 = a0 * inv, c1 = a1 * inv;
    if (a.o_part != nullptr || a.st_o != nullptr) {
      emit_partial(std::true_type{}, mm, l_tot, c0, c1);
      return;
    }
    // Accumulator row r of block db is d = db*32 + 8*(r/4) + 4*hi + r%4: lanes l and
    // l + 32 hold the two 4-element halves of each 8-element run.  One swap per
    // dword pair hands lane l the run of g = 2k and lane l + 32 that of g = 2k + 1,
    // so each lane stores 16 contiguous bytes.  (Both lanes of a pair hold the same
    // query row, so they are valid or not together.)
    const bool o_ok = q_row < Sq && q_row >= q_lo;
    __bf16* op = a.o + o_boff + row_off_t<kChunked>(a.ov, o_ok ? q_row : 0) + h * a.ov.hs;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        bf16x4 w0, w1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w0[e] = (__bf16)(acc_o[db][8 * k + e] * c0 + cb[db][2 * k][e] * c1);
          w1[e] = (__bf16)(acc_o[db][8 * k + 4 + e] * c0 + cb[db][2 * k + 1][e] * c1);
        }
        const uint2 x = __builtin_bit_cast(uint2, w0), y = __builtin_bit_cast(uint2, w1);
        const auto s0 = __builtin_amdgcn_permlane32_swap(x.x, y.x, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x.y, y.y, false, false);
        const uint4 out = make_uint4(s0[0], s1[0], s0[1], s1[1]);
        if (o_ok) *reinterpret_cast<uint4*>(op + db * 32 + 8 * (2 * k + hi)) = out;
      }
  }
  };  // process

  const int n_iter_blk = a.n_iter_blk;
  // XCD-aware numbering: consecutive logical indices (query blocks, or the
  // parts of one block) run on one XCD and its L2.
  // Packed documents: blocks [0, n_work), numbered as usual, run the first document
  // with rows in each (head, tile); the blocks after them, one per (head,
  // document), run a document on the tile where it starts when an earlier document
  // has rows there too, so that two documents sharing a tile run side by side.
  const bool vslot1 = kVarlen && int(blockIdx.x) >= a.n_work;
  const int pid = vslot1 ? int(blockIdx.x) - a.n_work : int(blockIdx.x);
  const int n = kSplit ? a.n_work * a.nsplit : a.n_work;
  const int per = n / kNumXcd, rem = n % kNumXcd;
  const int xcd = pid % kNumXcd, local = pid / kNumXcd;
  const int logical =
      vslot1 ? pid : xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  if constexpr (kVarlen) {
    auto end_of = [&](int d) { return min(max(a.cu_q[d + 1], 0), a.Sq); };
    auto start_of = [&](int d) { return min(max(a.cu_q[d], 0), a.Sq); };
    if (vslot1) {
      const int d = pid / a.H, h = pid % a.H;
      const int s0 = start_of(d);
      if (end_of(d) <= s0) return;  // no rows
      const int t = s0 / C::BM;
      // rows of earlier documents in the tile: the packed rows [max(cu_q[0], tile start), s0)
      if (max(start_of(0), t * C::BM) >= s0) return;  // the tile's first document: run below
      process(h * a.m_tiles + t, 0, 0, -1, d);
    } else {
      // The tile's first document with rows in it: the first whose end lies past the
      // tile's first row (binary search; the boundaries are non-decreasing), past
      // empty ones.
      const int r0 = (logical % a.m_tiles) * C::BM;
      int lo = 0, hi = a.B;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (end_of(mid) > r0) hi = mid;
        else lo = mid + 1;
      }
      while (lo < a.B && end_of(lo) <= start_of(lo) && start_of(lo) < r0 + C::BM) ++lo;
      if (lo < a.B && start_of(lo) < r0 + C::BM && end_of(lo) > start_of(lo)) process(logical, 0, 0, -1, lo);
    }
  } else if constexpr (!kSplit) {
    process(logical, 0, n_iter_blk, -1, 0);
  } else {
    const int j = logical % a.nsplit;
    process(logical / a.nsplit, n_iter_blk * j / a.nsplit, n_iter_blk * (j + 1) / a.nsplit, logical, 0);
  }
}

// Merges the nsplit partial states of each query block:
// O = sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k per row, M = max_k m_k (0 when
// no key of the row is valid).  A thread owns four consecutive head-dim columns
// of one row, so a wave reads whole rows of every partial O.
template <int D>
__global__ void __launch_bounds__(256) attn_combine_kernel(AttnArgs a) {
  constexpr int BM = Cfg<D>::BM;
  constexpr int TPR = D / 4;                 // threads per row
  constexpr int RPW = 256 / TPR;             // rows per workgroup
  constexpr int WPB = BM / RPW;              // workgroups per query block
  const int blk = blockIdx.x / WPB;
  const int row = (blockIdx.x % WPB) * RPW + threadIdx.x / TPR;
  const int c4 = (threadIdx.x % TPR) * 4;
  const int mt = blk % a.m_tiles, bh = blk / a.m_tiles, h = bh % a.H, b = bh / a.H;
  const int q_row = mt * BM + row;
  if (q_row >= a.Sq) return;
  const size_t slot0 = size_t(blk) * a.nsplit;
  const float* ml = a.ws + size_t(a.n_work) * a.nsplit * BM * D;
  float M = -INFINITY;
  for (int j = 0; j < a.nsplit; ++j) M = fmaxf(M, ml[((slot0 + j) * BM + row) * 2]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
  for (int j = 0; j < a.nsplit; ++j) {
    const size_t prow = (slot0 + j) * BM + row;
    const float mk = ml[prow * 2], lk = ml[prow * 2 + 1];
    const float f = mk == -INFINITY ? 0.f : exp2f(mk - M);
    const float4 x = *reinterpret_cast<const float4*>(a.ws + prow * D + c4);
    L += f * lk;
    acc.x += f * x.x;
    acc.y += f * x.y;
    acc.z += f * x.z;
    acc.w += f * x.w;
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  bf16x4 w;
  w[0] = (__bf16)(acc.x * inv);
  w[1] = (__bf16)(acc.y * inv);
  w[2] = (__bf16)(acc.z * inv);
  w[3] = (__bf16)(acc.w * inv);
  *reinterpret_cast<bf16x4*>(a.o + b * a.ov.bs + row_off_t<true>(a.ov, q_row) + h * a.ov.hs + c4) = w;
}

// Merge of N partial attentions of the same queries over disjoint key sets:
// O = sum_k e^{lse_k - L} O_k with L = ln sum_k e^{lse_k}; rows with no valid key
// in any part (every lse_k = -inf) get zeros.  One thread per four columns.
struct MergeArgs {
  const float* o_parts;  // [N][B][Sq][H][D]
  const float* lses;     // [N][B][H][Sq]
  __bf16* o;             // [B][Sq][H][D]
  int N, B, Sq, H, D;
  long long rows;        // B * Sq * H
};

__global__ void __launch_bounds__(256) attn_merge_kernel(MergeArgs a) {
  const int tpr = a.D / 4;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long r = t / tpr;
  if (r >= a.rows) return;
  const int c4 = int(t % tpr) * 4;
  const int h = int(r % a.H);
  const long long bi = r / a.H;
  const int i = int(bi % a.Sq), b = int(bi / a.Sq);
  const long long lse_stride = (long long)a.B * a.H * a.Sq;
  const long long lse0 = ((long long)b * a.H + h) * a.Sq + i;
  const long long o_stride = a.rows * a.D;
  float M = -INFINITY;
  for (int k = 0; k < a.N; ++k) M = fmaxf(M, a.lses[k * lse_stride + lse0]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
  if (M != -INFINITY) {
    for (int k = 0; k < a.N; ++k) {
      const float lk = a.lses[k * lse_stride + lse0];
      const float f = lk == -INFINITY ? 0.f : expf(lk - M);
      const float4 x = *reinterpret_cast<const float4*>(a.o_parts + k * o_stride + r * a.D + c4);
      L += f;
      acc.x += f * x.x;
      acc.y += f * x.y;
      acc.z += f * x.z;
      acc.w += f * x.w;
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  bf16x4 w;
  w[0] = (__bf16)(acc.x * inv);
  w[1] = (__bf16)(acc.y * inv);
  w[2] = (__bf16)(acc.z * inv);
  w[3] = (__bf16)(acc.w * inv);
  *reinterpret_cast<bf16x4*>(a.o + r * a.D + c4) = w;
}

template <int D, int MODE>
__global__ void __launch_bounds__(kThreads) attn_fwd_kernel(AttnArgs a) {
  attn_fwd_body<D, MODE>(a);
}

}  // namespace
}  // namespace cpattn

using namespace cpattn;

namespace {

// Local boundary i of an AllGather-KV rank whose query span is [s0, s0 + S_local):
// the global boundary clamped into the span and shifted to it.  Document i's local
// rows [local[i], local[i+1]) are then its intersection with the span, empty
// when the two do not meet.
__global__ void __launch_bounds__(256) remap_cu_kernel(const int* cu, int* local, int n, long long s0,
                                                       long long S_local) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    const long long x = (long long)cu[i] - s0;
    local[i] = int(x < 0 ? 0 : (x > S_local ? S_local : x));
  }
}

View plain_view(int64_t S, int64_t H, int64_t D) {
  View v;
  v.bs = S * H * D;
  v.cs = 0;
  v.rs = int(H * D);
  v.hs = int(D);
  v.chunked = 0;
  return v;
}

// Rows of S = W * L in W chunks of L rows: batch b, row i at
// (i / L) * cs + b * bs + (i % L) * rs.  With one batch the chunks are
// consecutive and the view is a plain strided one.
View chunked_view(int64_t B, int64_t L, int64_t H, int64_t hs, int64_t rs) {
  View v;
  v.bs = L * rs;
  v.cs = B * L * rs;
  v.rs = int(rs);
  v.hs = int(hs);
  v.chunked = B > 1;
  v.L = FastDiv(uint32_t(L));
  (void)H;
  return v;
}

// Heads of a call to run in 256-row blocks (the rest run in 128-row blocks): the
// split of the H heads between the two launches that takes the fewest rounds of
// `cus` workgroups, a round of 256-row blocks counted as 1.9 rounds of 128-row
// blocks (twice the work in the same cycles per tile, at a clock about 4% higher
// under the power limit for the halved L2 -> LDS traffic per flop; measured on the
// video share).  0 unless the split beats 128-row blocks alone.
int64_t wide_heads(int64_t B, int64_t Sq, int64_t H, int64_t cus) {
  constexpr double kWideRound = 1.9;
  const int64_t m128 = (Sq + 127) / 128, m256 = (Sq + 255) / 256;
  auto rounds = [&](int64_t n) { return double((n + cus - 1) / cus); };
  double best = rounds(B * H * m128);
  int64_t best_x = 0;
  // (every split for up to 4096 heads; beyond that only all heads in 256-row blocks)
  for (int64_t x = H <= 4096 ? 1 : H; x <= H; ++x) {
    const double t = kWideRound * rounds(B * x * m256) + rounds(B * (H - x) * m128);
    if (t < best - 0.05) {
      best = t;
      best_x = x;
    }
  }
  return best_x;
}

// Split plan and launch.  Every argument has been validated; ext_* are the byte
// extents of the operands, for the workspace overlap check.
int attn_launch(const __bf16* q, const View& qv, const __bf16* k, const __bf16* v, const View& kv,
                const uint8_t* key_mask, __bf16* o, const View& ov, int64_t B, int64_t Sq, int64_t Skv,
                int64_t H, int64_t D, float scale, void* ws, size_t ws_bytes, size_t ext_q, size_t ext_kv,
                size_t ext_o, cp_stream_t stream, float* o_part = nullptr, float* lse = nullptr,
                const float* st_o = nullptr, const float* st_lse = nullptr,
                const __bf16* k1 = nullptr, const __bf16* v1 = nullptr, const uint8_t* mask1 = nullptr,
                int64_t Skv1 = 0, const View* kv1 = nullptr, const int* cu_q = nullptr,
                const int* cu_k = nullptr) {
  const int64_t bm = 32 * kGroupWaves;
  const int64_t m_tiles = (Sq + bm - 1) / bm;
  // packed documents: B documents, one block per (head, tile of the packed rows)
  const int64_t n_work = (cu_q ? 1 : B) * H * m_tiles;
  AttnArgs args;
  args.qv = qv;
  args.kv = kv;
  args.ov = ov;
  args.q = q;
  args.k = k;
  args.v = v;
  args.mask = key_mask;
  args.o = o;
  args.B = int(B);
  args.Sq = int(Sq);
  args.Skv = int(Skv);
  args.H = int(H);
  args.m_tiles = int(m_tiles);
  args.n_work = int(n_work);
  args.sc = scale * 1.4426950408889634f;
  args.k1 = k1;
  args.v1 = v1;
  args.mask1 = mask1;
  args.Skv1 = int(Skv1);
  // segment 1: its own view, else dense [B][Skv1][H][D] with K/V's strides
  if (kv1) {
    args.kv1 = *kv1;
  } else {
    args.kv1 = kv;
    args.kv1.bs = (long long)Skv1 * kv.rs;
    args.kv1.chunked = 0;
  }
  args.nt0 = int((Skv + 63) / 64);
  const int64_t n_tiles = args.nt0 + (Skv1 + 63) / 64;
  args.n_iter_blk = int((n_tiles + 1) / 2);
  args.nsplit = 1;
  args.ws = nullptr;
  args.o_part = o_part;
  args.lse = lse;
  args.H_all = int(H);
  args.h_base = 0;
  args.st_o = st_o;
  args.st_lse = st_lse;
  args.cu_q = cu_q;
  args.cu_k = cu_k;
  // Split the key range of every query block into nsplit parts when the query
  // blocks alone would occupy at most half of the compute units; each part
  // keeps at least kMinSplitIters iterations.
  constexpr int64_t kMinSplitIters = 4;
  if (ws && !cu_q) {
    const int64_t cus = num_cus();
    const int64_t nsplit = std::min<int64_t>(cus / n_work, args.n_iter_blk / kMinSplitIters);
    if (2 * n_work <= cus && nsplit >= 2) {
      const size_t need = size_t(n_work * nsplit) * size_t(bm) * size_t(D + 2) * sizeof(float);
      if (ws_bytes < need) return CP_ERR_WORKSPACE;
      const size_t ext1 = size_t(B * Skv1 * H * D) * 2;
      if (overlaps(ws, need, q, ext_q) || overlaps(ws, need, k, ext_kv) || overlaps(ws, need, v, ext_kv) ||
          overlaps(ws, need, o, ext_o) || (key_mask && overlaps(ws, need, key_mask, size_t(B * Skv))) ||
          (k1 && overlaps(ws, need, k1, ext1)) || (v1 && overlaps(ws, need, v1, ext1)) ||
          (mask1 && overlaps(ws, need, mask1, size_t(B * Skv1))))
        return CP_ERR_ALIAS;
      args.nsplit = int(nsplit);
      args.ws = static_cast<float*>(ws);
    }
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 block{unsigned(kThreads)};
  // The chunked variants address rows through the views at run time (a view that
  // is not chunked is plain there too).  Segment 1 takes a view of its own when it
  // is chunked or its row stride differs from segment 0's.
  const bool seg1 = Skv1 > 0;
  const bool chunked = kv.chunked || qv.chunked || ov.chunked || (seg1 && args.kv1.chunked);
  const bool seg1_rows = seg1 && (args.kv1.chunked || kv.chunked || args.kv1.rs != kv.rs);
  const int mode = (chunked ? kModeChunked : 0) | (seg1 ? kModeTwoSeg : 0) |
                   ((kv.chunked && kv.L.d % 64 != 0) || (seg1 && args.kv1.chunked && args.kv1.L.d % 64 != 0)
                        ? kModeCross : 0) |
                   (seg1_rows ? kModeSeg1Rows : 0) | (cu_q ? kModeVarlen : 0) | (args.nsplit > 1 ? kModeSplit : 0);
  // Calls without packed documents or split-KV (D = 128): heads [0, wh) run in
  // 256-row blocks (one launch), the rest below in 128-row blocks.
  if (D == 128 && !cu_q && args.nsplit == 1) {
    const int64_t wh = wide_heads(B, Sq, H, num_cus());
    if (wh > 0) {
      AttnArgs w = args;
      w.H = int(wh);
      w.m_tiles = int((Sq + 2 * bm - 1) / (2 * bm));
      w.n_work = int(B * wh * w.m_tiles);
      w.n_iter_blk = int(n_tiles);  // both groups take every tile
      const dim3 wgrid{unsigned(w.n_work)};
      auto launch_w = [&](auto kern) { hipLaunchKernelGGL(kern, wgrid, block, 0, s, w); };
      switch (mode) {
        case 0: launch_w(attn_fwd_kernel<128, kModeWide>); break;
        case kModeChunked: launch_w(attn_fwd_kernel<128, kModeWide + kModeChunked>); break;
        case kModeChunked + kModeCross: launch_w(attn_fwd_kernel<128, kModeWide + kModeChunked + kModeCross>); break;
        case kModeTwoSeg: launch_w(attn_fwd_kernel<128, kModeWide + kModeTwoSeg>); break;
        case kModeTwoSeg + kModeSeg1Rows:
          launch_w(attn_fwd_kernel<128, kModeWide + kModeTwoSeg + kModeSeg1Rows>);
          break;
        case kModeChunked + kModeTwoSeg + kModeSeg1Rows:
          launch_w(attn_fwd_kernel<128, kModeWide + kModeChunked + kModeTwoSeg + kModeSeg1Rows>);
          break;
        case kModeChunked + kModeTwoSeg + kModeCross + kModeSeg1Rows:
          launch_w(attn_fwd_kernel<128, kModeWide + kModeChunked + kModeTwoSeg + kModeCross + kModeSeg1Rows>);
          break;
        default: return CP_ERR_UNSUPPORTED;
      }
      if (wh == H) return hip_status(hipGetLastError());
      args.q += wh * qv.hs;
      args.k += wh * kv.hs;
      args.v += wh * kv.hs;
      if (args.o) args.o += wh * ov.hs;
      args.h_base = int(wh);  // partial outputs index the call's heads
      if (seg1) {
        args.k1 += wh * args.kv1.hs;
        args.v1 += wh * args.kv1.hs;
      }
      args.H = int(H - wh);
      args.n_work = int(B * (H - wh) * m_tiles);
    }
  }
  // combine: BM * D / 4 threads of 256 per query block
  const int64_t n_blocks = args.n_work;
  const dim3 grid{unsigned(n_blocks * args.nsplit + (cu_q ? H * B : 0))}, cblock{256u},
      cgrid{unsigned(n_blocks * (D / 8))};
  auto launch_fwd = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, s, args); };
  if (D == 128) {
    if (mode == 0) launch_fwd(attn_fwd_kernel<128, 0>);
    else if (mode == kModeSplit) launch_fwd(attn_fwd_kernel<128, kModeSplit>);
    else if (mode == kModeChunked + kModeSplit) launch_fwd(attn_fwd_kernel<128, kModeChunked + kModeSplit>);
    else if (mode == kModeChunked + kModeCross + kModeSplit) launch_fwd(attn_fwd_kernel<128, kModeChunked + kModeCross + kModeSplit>);
    else if (mode == kModeTwoSeg + kModeSplit) launch_fwd(attn_fwd_kernel<128, kModeTwoSeg + kModeSplit>);
    else if (mode == kModeTwoSeg + kModeSeg1Rows + kModeSplit) launch_fwd(attn_fwd_kernel<128, kModeTwoSeg + kModeSeg1Rows + kModeSplit>);
    else if (mode == kModeChunked + kModeTwoSeg + kModeSeg1Rows + kModeSplit)
      launch_fwd(attn_fwd_kernel<128, kModeChunked + kModeTwoSeg + kModeSeg1Rows + kModeSplit>);
    else if (mode == kModeChunked + kModeTwoSeg + kModeCross + kModeSeg1Rows + kModeSplit)
      launch_fwd(attn_fwd_kernel<128, kModeChunked + kModeTwoSeg + kModeCross + kModeSeg1Rows + kModeSplit>);
    else if (mode == kModeVarlen) launch_fwd(attn_fwd_kernel<128, kModeVarlen>);
    else if (mode == kModeChunked) launch_fwd(attn_fwd_kernel<128, kModeChunked>);
    else if (mode == kModeChunked + kModeCross) launch_fwd(attn_fwd_kernel<128, kModeChunked + kModeCross>);
    else if (mode == kModeTwoSeg) launch_fwd(attn_fwd_kernel<128, kModeTwoSeg>);
    else if (mode == kModeTwoSeg + kModeSeg1Rows) launch_fwd(attn_fwd_kernel<128, kModeTwoSeg + kModeSeg1Rows>);
    else if (mode == kModeChunked + kModeTwoSeg + kModeSeg1Rows)
      launch_fwd(attn_fwd_kernel<128, kModeChunked + kModeTwoSeg + kModeSeg1Rows>);
    else if (mode == kModeChunked + kModeTwoSeg + kModeCross + kModeSeg1Rows)
      launch_fwd(attn_fwd_kernel<128, kModeChunked + kModeTwoSeg + kModeCross + kModeSeg1Rows>);
    else return CP_ERR_UNSUPPORTED;
    if (args.nsplit > 1) hipLaunchKernelGGL(attn_combine_kernel<128>, cgrid, cblock, 0, s, args);
  } else {
    if (mode == 0) launch_fwd(attn_fwd_kernel<64, 0>);
    else if (mode == kModeSplit) launch_fwd(attn_fwd_kernel<64, kModeSplit>);
    else if (mode == kModeChunked + kModeSplit) launch_fwd(attn_fwd_kernel<64, kModeChunked + kModeSplit>);
    else if (mode == kModeChunked + kModeCross + kModeSplit) launch_fwd(attn_fwd_kernel<64, kModeChunked + kModeCross + kModeSplit>);
    else if (mode == kModeTwoSeg + kModeSplit) launch_fwd(attn_fwd_kernel<64, kModeTwoSeg + kModeSplit>);
    else if (mode == kModeTwoSeg + kModeSeg1Rows + kModeSplit) launch_fwd(attn_fwd_kernel<64, kModeTwoSeg + kModeSeg1Rows + kModeSplit>);
    else if (mode == kModeChunked + kModeTwoSeg + kModeSeg1Rows + kModeSplit)
      launch_fwd(attn_fwd_kernel<64, kModeChunked + kModeTwoSeg + kModeSeg1Rows + kModeSplit>);
    else if (mode == kModeChunked + kModeTwoSeg + kModeCross + kModeSeg1Rows + kModeSplit)
      launch_fwd(attn_fwd_kernel<64, kModeChunked + kModeTwoSeg + kModeCross + kModeSeg1Rows + kModeSplit>);
    else if (mode == kModeVarlen) launch_fwd(attn_fwd_kernel<64, kModeVarlen>);
    else if (mode == kModeChunked) launch_fwd(attn_fwd_kernel<64, kModeChunked>);
    else if (mode == kModeChunked + kModeCross) launch_fwd(attn_fwd_kernel<64, kModeChunked + kModeCross>);
    else if (mode == kModeTwoSeg) launch_fwd(attn_fwd_kernel<64, kModeTwoSeg>);
    else if (mode == kModeTwoSeg + kModeSeg1Rows) launch_fwd(attn_fwd_kernel<64, kModeTwoSeg + kModeSeg1Rows>);
    else if (mode == kModeChunked + kModeTwoSeg + kModeSeg1Rows)
      launch_fwd(attn_fwd_kernel<64, kModeChunked + kModeTwoSeg + kModeSeg1Rows>);
    else if (mode == kModeChunked + kModeTwoSeg + kModeCross + kModeSeg1Rows)
      launch_fwd(attn_fwd_kernel<64, kModeChunked + kModeTwoSeg + kModeCross + kModeSeg1Rows>);
    else return CP_ERR_UNSUPPORTED;
    if (args.nsplit > 1) hipLaunchKernelGGL(attn_combine_kernel<64>, cgrid, cblock, 0, s, args);
  }
  return hip_status(hipGetLastError());
}

// Checks shared by every attention entry point.
int attn_check(int64_t B, int64_t Sq, int64_t Skv, int64_t H, int64_t D, float scale) {
  if (B < 1 || Sq < 1 || Skv < 1 || H < 1) return CP_ERR_SHAPE;
  if (D != 64 && D != 128) return CP_ERR_HEAD_DIM;
  if (!std::isfinite(scale) || !(scale > 0.f)) return CP_ERR_SCALE;
  return CP_OK;
}

// Device address of the scratch array on the current device, looked up once per
// device (with that device current) and kept.
int scratch_on_device(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CP_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return CP_ERR_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return CP_OK;
}

// Local-Q / global-KV attention on dense [B][S][H][D] operands.  static_scratch:
// the split-KV partial states go to the library's scratch array (ws unused).
int attn_run(const void* q, const void* k, const void* v, const uint8_t* key_mask, void* o, int64_t B,
             int64_t Sq, int64_t Skv, int64_t H, int64_t D, float scale, void* ws, size_t ws_bytes,
             cp_stream_t stream, bool static_scratch = false) {
  if (!q || !k || !v || !o) return CP_ERR_NULL;
  if (const int st = attn_check(B, Sq, Skv, H, D, scale)) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return CP_ERR_ALIGNMENT;
  if (ws && !aligned16(ws)) return CP_ERR_ALIGNMENT;
  // Per-dimension sizes and the work count are kept in int on the device.
  constexpr int64_t kIntMax = 0x7fffffff;
  if (B > kIntMax || Sq > kIntMax || Skv > kIntMax - 64 || H > kIntMax) return CP_ERR_SHAPE;
  // Rows of a K/V tile are addressed with 32-bit byte offsets.
  if (H * D * 2 * 64 > kIntMax) return CP_ERR_SHAPE;
  const int64_t bm = 32 * kGroupWaves;
  const int64_t m_tiles = (Sq + bm - 1) / bm;
  int64_t bh, n_work, qe, ke;
  if (!mul_capped(B, H, kIntMax, &bh) || !mul_capped(bh, m_tiles, kIntMax, &n_work)) return CP_ERR_SHAPE;
  if (!mul_capped(B * Sq, H * D, int64_t(1) << 60, &qe) || !mul_capped(B * Skv, H * D, int64_t(1) << 60, &ke))
    return CP_ERR_SHAPE;
  const size_t qb = size_t(qe) * 2, kb = size_t(ke) * 2;
  if (overlaps(o, qb, q, qb) || overlaps(o, qb, k, kb) || overlaps(o, qb, v, kb)) return CP_ERR_ALIAS;
  if (key_mask && overlaps(o, qb, key_mask, size_t(B * Skv))) return CP_ERR_ALIAS;
  if (static_scratch) {
    if (const int st = scratch_on_device(&ws)) return st;
    ws_bytes = CP_ATTN_NOALLOC_SCRATCH_BYTES;
  }
  const int st = attn_launch(static_cast<const __bf16*>(q), plain_view(Sq, H, D), static_cast<const __bf16*>(k),
                             static_cast<const __bf16*>(v), plain_view(Skv, H, D), key_mask,
                             static_cast<__bf16*>(o), plain_view(Sq, H, D), B, Sq, Skv, H, D, scale, ws, ws_bytes,
                             qb, kb, qb, stream);
  return static_scratch && st == CP_ERR_WORKSPACE ? CP_ERR_SCRATCH : st;
}

}  // namespace

extern "C" int cp_attn_localq_globalkv(const void* q, const void* k, const void* v,
                                       const uint8_t* key_mask, void* o, int64_t B, int64_t Sq,
                                       int64_t Skv, int64_t H, int64_t D, float scale,
                                       cp_stream_t stream) {
  return attn_run(q, k, v, key_mask, o, B, Sq, Skv, H, D, scale, nullptr, 0, stream);
}

extern "C" int cp_attn_localq_globalkv_ws(const void* q, const void* k, const void* v,
                                          const uint8_t* key_mask, void* o, int64_t B, int64_t Sq,
                                          int64_t Skv, int64_t H, int64_t D, float scale,
                                          void* workspace, size_t workspace_bytes, cp_stream_t stream) {
  return attn_run(q, k, v, key_mask, o, B, Sq, Skv, H, D, scale, workspace, workspace_bytes, stream);
}

extern "C" int cp_attn_localq_globalkv_noalloc(const void* q, const void* k, const void* v,
                                               const uint8_t* key_mask, void* o, int64_t B, int64_t Sq,
                                               int64_t Skv, int64_t H, int64_t D, float scale,
                                               cp_stream_t stream) {
  return attn_run(q, k, v, key_mask, o, B, Sq, Skv, H, D, scale, nullptr, 0, stream, true);
}

extern "C" int cp_varlen_remap_cu_seqlens_q(const int32_t* cu_q_global, int32_t* cu_q_local, int64_t n_docs,
                                            int64_t rank, int64_t S_local, cp_stream_t stream) {
  if (!cu_q_global || !cu_q_local) return CP_ERR_NULL;
  constexpr int64_t kIntMax = 0x7fffffff;
  if (n_docs < 1 || n_docs >= kIntMax || rank < 0 || S_local < 1 || S_local > kIntMax ||
      rank > kIntMax / S_local)
    return CP_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(cu_q_global) | reinterpret_cast<uintptr_t>(cu_q_local)) & 3u)
    return CP_ERR_ALIGNMENT;
  const size_t bytes = size_t(n_docs + 1) * 4;
  if (overlaps(cu_q_local, bytes, cu_q_global, bytes)) return CP_ERR_ALIAS;
  const unsigned n = unsigned(n_docs + 1);
  hipLaunchKernelGGL(remap_cu_kernel, dim3((n + 255) / 256), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     cu_q_global, cu_q_local, int(n), (long long)(rank * S_local), (long long)S_local);
  return hip_status(hipGetLastError());
}

extern "C" int cp_attn_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int64_t n_docs, void* o,
                              int64_t Sq, int64_t Skv, int64_t H, int64_t D, float scale,
                              cp_stream_t stream) {
  if (!q || !k || !v || !o || !cu_seqlens_q || !cu_seqlens_k) return CP_ERR_NULL;
  if (const int st = attn_check(1, Sq, Skv, H, D, scale)) return st;
  constexpr int64_t kIntMax = 0x7fffffff;
  if (n_docs < 1 || n_docs >= kIntMax) return CP_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return CP_ERR_ALIGNMENT;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) | reinterpret_cast<uintptr_t>(cu_seqlens_k)) & 3u)
    return CP_ERR_ALIGNMENT;
  if (Sq > kIntMax || Skv > kIntMax - 64 || H > kIntMax) return CP_ERR_SHAPE;
  if (H * D * 2 * 64 > kIntMax) return CP_ERR_SHAPE;
  const int64_t bm = 32 * kGroupWaves;
  int64_t bh, n_work, qe, ke;
  // one block per (head, tile) and one per (head, document)
  if (!mul_capped(H, (Sq + bm - 1) / bm + n_docs, kIntMax, &n_work)) return CP_ERR_SHAPE;
  (void)bh;
  if (!mul_capped(Sq, H * D, int64_t(1) << 60, &qe) || !mul_capped(Skv, H * D, int64_t(1) << 60, &ke))
    return CP_ERR_SHAPE;
  const size_t qb = size_t(qe) * 2, kb = size_t(ke) * 2, cb = size_t(n_docs + 1) * 4;
  if (overlaps(o, qb, q, qb) || overlaps(o, qb, k, kb) || overlaps(o, qb, v, kb) ||
      overlaps(o, qb, cu_seqlens_q, cb) || overlaps(o, qb, cu_seqlens_k, cb))
    return CP_ERR_ALIAS;
  return attn_launch(static_cast<const __bf16*>(q), plain_view(Sq, H, D), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), plain_view(Skv, H, D), nullptr, static_cast<__bf16*>(o),
                     plain_view(Sq, H, D), n_docs, Sq, Skv, H, D, scale, nullptr, 0, qb, kb, qb, stream, nullptr,
                     nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, cu_seqlens_q, cu_seqlens_k);
}

extern "C" int cp_attn_joint(const void* q, const void* k_img, const void* v_img, const uint8_t* img_mask,
                             const void* k_joint, const void* v_joint, const uint8_t* joint_mask, int joint_front,
                             void* o, int64_t B, int64_t Sq, int64_t S_img, int64_t T, int64_t H, int64_t D,
                             float scale, void* workspace, size_t workspace_bytes, cp_stream_t stream) {
  if (!q || !k_img || !v_img || !o) return CP_ERR_NULL;
  if (T > 0 && (!k_joint || !v_joint)) return CP_ERR_NULL;
  if (T < 0 || S_img < 1) return CP_ERR_SHAPE;
  if (joint_front != 0 && joint_front != 1) return CP_ERR_UNSUPPORTED;
  constexpr int64_t kIntMax = 0x7fffffff;
  if (S_img > kIntMax / 2 || T > kIntMax / 2) return CP_ERR_SHAPE;
  if (const int st = attn_check(B, Sq, S_img + T, H, D, scale)) return st;
  if (!aligned16(q) || !aligned16(k_img) || !aligned16(v_img) || !aligned16(o)) return CP_ERR_ALIGNMENT;
  if (T > 0 && (!aligned16(k_joint) || !aligned16(v_joint))) return CP_ERR_ALIGNMENT;
  if (workspace && !aligned16(workspace)) return CP_ERR_ALIGNMENT;
  if (B > kIntMax || Sq > kIntMax || S_img + T > kIntMax - 64 || H > kIntMax) return CP_ERR_SHAPE;
  if (H * D * 2 * 64 > kIntMax) return CP_ERR_SHAPE;
  const int64_t bm = 32 * kGroupWaves;
  int64_t bh, n_work, qe, ie, je;
  if (!mul_capped(B, H, kIntMax, &bh) || !mul_capped(bh, (Sq + bm - 1) / bm, kIntMax, &n_work)) return CP_ERR_SHAPE;
  if (!mul_capped(B * Sq, H * D, int64_t(1) << 60, &qe) || !mul_capped(B * S_img, H * D, int64_t(1) << 60, &ie) ||
      !mul_capped(B * (T > 0 ? T : 1), H * D, int64_t(1) << 60, &je))
    return CP_ERR_SHAPE;
  const size_t qb = size_t(qe) * 2, ib = size_t(ie) * 2, jb = size_t(je) * 2;
  if (overlaps(o, qb, q, qb) || overlaps(o, qb, k_img, ib) || overlaps(o, qb, v_img, ib)) return CP_ERR_ALIAS;
  if (T > 0 && (overlaps(o, qb, k_joint, jb) || overlaps(o, qb, v_joint, jb))) return CP_ERR_ALIAS;
  if (img_mask && overlaps(o, qb, img_mask, size_t(B * S_img))) return CP_ERR_ALIAS;
  if (T > 0 && joint_mask && overlaps(o, qb, joint_mask, size_t(B * T))) return CP_ERR_ALIAS;
  const auto* qp = static_cast<const __bf16*>(q);
  const auto* ki = static_cast<const __bf16*>(k_img);
  const auto* vi = static_cast<const __bf16*>(v_img);
  const auto* kj = static_cast<const __bf16*>(k_joint);
  const auto* vj = static_cast<const __bf16*>(v_joint);
  auto* op = static_cast<__bf16*>(o);
  if (T == 0)
    return attn_launch(qp, plain_view(Sq, H, D), ki, vi, plain_view(S_img, H, D), img_mask, op, plain_view(Sq, H, D),
                       B, Sq, S_img, H, D, scale, workspace, workspace_bytes, qb, ib, qb, stream);
  if (joint_front)
    return attn_launch(qp, plain_view(Sq, H, D), kj, vj, plain_view(T, H, D), joint_mask, op, plain_view(Sq, H, D),
                       B, Sq, T, H, D, scale, workspace, workspace_bytes, qb, jb, qb, stream, nullptr, nullptr, nullptr,
                       nullptr, ki, vi, img_mask, S_img);
  return attn_launch(qp, plain_view(Sq, H, D), ki, vi, plain_view(S_img, H, D), img_mask, op, plain_view(Sq, H, D),
                     B, Sq, S_img, H, D, scale, workspace, workspace_bytes, qb, ib, qb, stream, nullptr, nullptr, nullptr,
                     nullptr, kj, vj, joint_mask, T);
}

extern "C" int cp_attn_recv_to_send(const void* recv, const uint8_t* key_mask, void* send, int64_t B,
                                    int64_t S_local, int64_t H_local, int64_t D, int64_t W, float scale,
                                    void* workspace, size_t workspace_bytes, cp_stream_t stream) {
  if (!recv || !send) return CP_ERR_NULL;
  if (W < 1) return CP_ERR_SHAPE;
  constexpr int64_t kIntMax = 0x7fffffff;
  if (S_local < 1 || S_local > kIntMax / W) return CP_ERR_SHAPE;
  const int64_t S = W * S_local;
  if (const int st = attn_check(B, S, S, H_local, D, scale)) return st;
  if (!aligned16(recv) || !aligned16(send)) return CP_ERR_ALIGNMENT;
  if (workspace && !aligned16(workspace)) return CP_ERR_ALIGNMENT;
  if (B > kIntMax || S > kIntMax - 64 || H_local > kIntMax) return CP_ERR_SHAPE;
  if (H_local * 3 * D * 2 * 64 > kIntMax) return CP_ERR_SHAPE;
  // With several batches the received rows of one batch come in W chunks of
  // S_local rows.  When S_local is not a multiple of 64 a K/V tile can span
  // chunks; its lane offsets are then 32-bit differences of row offsets, so the
  // received buffer must stay below 2 GB.
  const int64_t bm = 32 * kGroupWaves;
  int64_t bh, n_work, re, se;
  if (!mul_capped(B, H_local, kIntMax, &bh) || !mul_capped(bh, (S + bm - 1) / bm, kIntMax, &n_work))
    return CP_ERR_SHAPE;
  if (!mul_capped(B * S, H_local * 3 * D, int64_t(1) << 60, &re)) return CP_ERR_SHAPE;
  se = re / 3;
  const size_t rb = size_t(re) * 2, sb = size_t(se) * 2;
  if (B > 1 && S_local % 64 != 0 && rb > size_t(kIntMax)) return CP_ERR_SHAPE;
  if (overlaps(send, sb, recv, rb)) return CP_ERR_ALIAS;
  if (key_mask && overlaps(send, sb, key_mask, size_t(B * S))) return CP_ERR_ALIAS;
  const View in = chunked_view(B, S_local, H_local, 3 * D, H_local * 3 * D);
  const View out = chunked_view(B, S_local, H_local, D, H_local * D);
  const __bf16* r = static_cast<const __bf16*>(recv);
  return attn_launch(r, in, r + D, r + 2 * D, in, key_mask, static_cast<__bf16*>(send), out, B, S, S, H_local,
                     D, scale, workspace, workspace_bytes, rb, rb, sb, stream);
}

extern "C" int cp_attn_recv_to_send_2d(const void* recv, const void* k_other, const void* v_other, int64_t S_other,
                                       int other_first, const uint8_t* own_mask, const uint8_t* other_mask,
                                       void* send, int64_t B, int64_t S_local, int64_t H_local, int64_t D,
                                       int64_t W, float scale, void* workspace,
                                       size_t workspace_bytes, cp_stream_t stream) {
  if (!recv || !send || !k_other || !v_other) return CP_ERR_NULL;
  if (W < 1 || S_other < 1) return CP_ERR_SHAPE;
  if (other_first != 0 && other_first != 1) return CP_ERR_UNSUPPORTED;
  constexpr int64_t kIntMax = 0x7fffffff;
  if (S_local < 1 || S_local > kIntMax / W) return CP_ERR_SHAPE;
  const int64_t S = W * S_local;
  if (S > kIntMax / 2 || S_other > kIntMax / 2) return CP_ERR_SHAPE;
  if (const int st = attn_check(B, S, S + S_other, H_local, D, scale)) return st;
  if (!aligned16(recv) || !aligned16(send) || !aligned16(k_other) || !aligned16(v_other)) return CP_ERR_ALIGNMENT;
  if (workspace && !aligned16(workspace)) return CP_ERR_ALIGNMENT;
  if (B > kIntMax || S + S_other > kIntMax - 64 || H_local > kIntMax) return CP_ERR_SHAPE;
  if (H_local * 3 * D * 2 * 64 > kIntMax) return CP_ERR_SHAPE;
  const int64_t bm = 32 * kGroupWaves;
  int64_t bh, n_work, re, oe;
  if (!mul_capped(B, H_local, kIntMax, &bh) || !mul_capped(bh, (S + bm - 1) / bm, kIntMax, &n_work))
    return CP_ERR_SHAPE;
  if (!mul_capped(B * S, H_local * 3 * D, int64_t(1) << 60, &re) ||
      !mul_capped(B * S_other, H_local * D, int64_t(1) << 60, &oe))
    return CP_ERR_SHAPE;
  const size_t rb = size_t(re) * 2, sb = size_t(re / 3) * 2, ob = size_t(oe) * 2;
  // tiles that span the received chunks use 32-bit differences of row offsets
  if (B > 1 && S_local % 64 != 0 && rb > size_t(kIntMax)) return CP_ERR_SHAPE;
  if (overlaps(send, sb, recv, rb) || overlaps(send, sb, k_other, ob) || overlaps(send, sb, v_other, ob))
    return CP_ERR_ALIAS;
  if (own_mask && overlaps(send, sb, own_mask, size_t(B * S))) return CP_ERR_ALIAS;
  if (other_mask && overlaps(send, sb, other_mask, size_t(B * S_other))) return CP_ERR_ALIAS;
  // the workspace must not overlap any operand (checked here over its whole extent)
  if (workspace && workspace_bytes &&
      (overlaps(workspace, workspace_bytes, recv, rb) || overlaps(workspace, workspace_bytes, k_other, ob) ||
       overlaps(workspace, workspace_bytes, v_other, ob) || overlaps(workspace, workspace_bytes, send, sb) ||
       (own_mask && overlaps(workspace, workspace_bytes, own_mask, size_t(B * S))) ||
       (other_mask && overlaps(workspace, workspace_bytes, other_mask, size_t(B * S_other)))))
    return CP_ERR_ALIAS;
  const View in = chunked_view(B, S_local, H_local, 3 * D, H_local * 3 * D);
  const View out = chunked_view(B, S_local, H_local, D, H_local * D);
  const View oth = plain_view(S_other, H_local, D);
  const __bf16* r = static_cast<const __bf16*>(recv);
  const auto* ko = static_cast<const __bf16*>(k_other);
  const auto* vo = static_cast<const __bf16*>(v_other);
  auto* sp = static_cast<__bf16*>(send);
  if (other_first)
    return attn_launch(r, in, ko, vo, oth, other_mask, sp, out, B, S, S_other, H_local, D, scale, workspace,
                       workspace_bytes, rb, ob, sb, stream, nullptr, nullptr, nullptr, nullptr, r + D, r + 2 * D,
                       own_mask, S, &in);
  return attn_launch(r, in, r + D, r + 2 * D, in, own_mask, sp, out, B, S, S, H_local, D, scale, workspace,
                     workspace_bytes, rb, rb, sb, stream, nullptr, nullptr, nullptr, nullptr, ko, vo, other_mask,
                     S_other, &oth);
}

namespace {

// Checks and launch shared by cp_attn_partial and cp_attn_partial_accum.
// out_o / out_lse: fp32 outputs (may be the state itself); o_final: bf16 output.
int partial_run(const void* q, const void* k, const void* v, const uint8_t* key_mask, void* out_o,
                void* out_lse, const void* st_o, const void* st_lse, void* o_final, int64_t B, int64_t Sq,
                int64_t Skv, int64_t H, int64_t D, float scale, cp_stream_t stream) {
  if (const int st = attn_check(B, Sq, Skv, H, D, scale)) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return CP_ERR_ALIGNMENT;
  if ((out_o && !aligned16(out_o)) || (st_o && !aligned16(st_o)) || (o_final && !aligned16(o_final)))
    return CP_ERR_ALIGNMENT;
  if ((reinterpret_cast<uintptr_t>(out_lse) & 3u) != 0 || (reinterpret_cast<uintptr_t>(st_lse) & 3u) != 0)
    return CP_ERR_ALIGNMENT;
  constexpr int64_t kIntMax = 0x7fffffff;
  if (B > kIntMax || Sq > kIntMax || Skv > kIntMax - 64 || H > kIntMax) return CP_ERR_SHAPE;
  if (H * D * 2 * 64 > kIntMax) return CP_ERR_SHAPE;
  const int64_t bm = 32 * kGroupWaves;
  int64_t bh, n_work, qe, ke;
  if (!mul_capped(B, H, kIntMax, &bh) || !mul_capped(bh, (Sq + bm - 1) / bm, kIntMax, &n_work))
    return CP_ERR_SHAPE;
  if (!mul_capped(B * Sq, H * D, int64_t(1) << 59, &qe) || !mul_capped(B * Skv, H * D, int64_t(1) << 60, &ke))
    return CP_ERR_SHAPE;
  const size_t qb = size_t(qe) * 2, kb = size_t(ke) * 2, pb = size_t(qe) * 4, lb = size_t(B * H * Sq) * 4;
  const size_t mb = key_mask ? size_t(B * Skv) : 0;
  // every buffer this call writes or keeps must be disjoint from the inputs it reads
  struct Range { const void* p; size_t n; };
  const Range writes[] = {{out_o, pb}, {out_lse, lb}, {o_final, qb}, {st_o, pb}, {st_lse, lb}};
  for (const Range& w : writes) {
    if (!w.p) continue;
    if (overlaps(w.p, w.n, q, qb) || overlaps(w.p, w.n, k, kb) || overlaps(w.p, w.n, v, kb) ||
        (key_mask && overlaps(w.p, w.n, key_mask, mb)))
      return CP_ERR_ALIAS;
  }
  if (out_o && out_lse && overlaps(out_o, pb, out_lse, lb)) return CP_ERR_ALIAS;
  if (st_o && st_lse && overlaps(st_o, pb, st_lse, lb)) return CP_ERR_ALIAS;
  if (o_final && ((st_o && overlaps(o_final, qb, st_o, pb)) || (st_lse && overlaps(o_final, qb, st_lse, lb))))
    return CP_ERR_ALIAS;
  return attn_launch(static_cast<const __bf16*>(q), plain_view(Sq, H, D), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), plain_view(Skv, H, D), key_mask,
                     static_cast<__bf16*>(o_final), plain_view(Sq, H, D), B, Sq, Skv, H, D, scale, nullptr, 0,
                     qb, kb, o_final ? qb : pb, stream, static_cast<float*>(out_o), static_cast<float*>(out_lse),
                     static_cast<const float*>(st_o), static_cast<const float*>(st_lse));
}

}  // namespace

extern "C" int cp_attn_partial(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                               void* o_part, void* lse, int64_t B, int64_t Sq, int64_t Skv, int64_t H,
                               int64_t D, float scale, cp_stream_t stream) {
  if (!q || !k || !v || !o_part || !lse) return CP_ERR_NULL;
  return partial_run(q, k, v, key_mask, o_part, lse, nullptr, nullptr, nullptr, B, Sq, Skv, H, D, scale,
                     stream);
}

extern "C" int cp_attn_partial_accum(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                                     void* state_o, void* state_lse, void* o_final, int64_t B, int64_t Sq,
                                     int64_t Skv, int64_t H, int64_t D, float scale,
                                     cp_stream_t stream) {
  if (!q || !k || !v || !state_o || !state_lse) return CP_ERR_NULL;
  if (o_final)
    return partial_run(q, k, v, key_mask, nullptr, nullptr, state_o, state_lse, o_final, B, Sq, Skv, H, D, scale,
                       stream);
  return partial_run(q, k, v, key_mask, state_o, state_lse, state_o, state_lse, nullptr, B, Sq, Skv, H, D, scale,
                     stream);
}

extern "C" int cp_attn_merge(const void* o_parts, const void* lses, int64_t N, void* o, int64_t B, int64_t Sq,
                             int64_t H, int64_t D, cp_stream_t stream) {
  if (!o_parts || !lses || !o) return CP_ERR_NULL;
  if (N < 1 || B < 1 || Sq < 1 || H < 1) return CP_ERR_SHAPE;
  if (D != 64 && D != 128) return CP_ERR_HEAD_DIM;
  if (!aligned16(o_parts) || !aligned16(o)) return CP_ERR_ALIGNMENT;
  if ((reinterpret_cast<uintptr_t>(lses) & 3u) != 0) return CP_ERR_ALIGNMENT;
  constexpr int64_t kIntMax = 0x7fffffff;
  int64_t rows, total;
  if (N > kIntMax || B > kIntMax || Sq > kIntMax || H > kIntMax) return CP_ERR_SHAPE;
  if (!mul_capped(B * Sq, H, int64_t(1) << 40, &rows) || !mul_capped(rows, N * D, int64_t(1) << 58, &total))
    return CP_ERR_SHAPE;
  const size_t ob = size_t(rows * D) * 2, pb = size_t(total) * 4, lb = size_t(rows * N) * 4;
  if (overlaps(o, ob, o_parts, pb) || overlaps(o, ob, lses, lb)) return CP_ERR_ALIAS;
  MergeArgs m;
  m.o_parts = static_cast<const float*>(o_parts);
  m.lses = static_cast<const float*>(lses);
  m.o = static_cast<__bf16*>(o);
  m.N = int(N);
  m.B = int(B);
  m.Sq = int(Sq);
  m.H = int(H);
  m.D = int(D);
  m.rows = rows;
  const int64_t threads = rows * (D / 4);
  const dim3 grid{unsigned((threads + 255) / 256)}, block{256u};
  hipLaunchKernelGGL(attn_merge_kernel, grid, block, 0, reinterpret_cast<hipStream_t>(stream), m);
  return hip_status(hipGetLastError());
}

extern "C" size_t cp_attn_workspace_bytes(int64_t B, int64_t Sq, int64_t Skv, int64_t H, int64_t D) {
  if (D != 64 && D != 128) return 0;
  if (B < 1 || Sq < 1 || Skv < 1 || H < 1) return 0;
  // at most one partial slot of BM x (D + 2) floats per compute unit
  return size_t(num_cus()) * size_t(32 * kGroupWaves) * size_t(D + 2) * sizeof(float);
}
