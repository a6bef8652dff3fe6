/*
 * cp_attn.h -- C ABI of libcpattn.so: one GPU's share of context-parallel
 * diffusion-transformer attention on AMD MI355X (gfx950).
 *
 * The library covers the per-rank hot path of Ulysses / AllGather-KV context
 * parallelism:
 *   1. cp_pack_qkv_dst_major   -- Ulysses input exchange, send side
 *   2. cp_sim_exchange         -- the W-way chunk exchange, simulated on one GPU
 *   3. cp_unpack_head_sharded  -- Ulysses input exchange, receive side
 *   4. cp_attn_localq_globalkv -- non-causal local-Q / global-KV attention
 *   5. cp_output_reverse       -- Ulysses output exchange (send layout, merge)
 *
 * Sources, by page and section:
 *   [sglang#33667]   prhub summary of sglang PR #33667 (pack the Ulysses QKV
 *                    all-to-all into one collective and reuse staging buffers):
 *                    "Implementation breakdown", "Key source snippets".
 *   [vllm-omni#7641] vllm-omni PR #7641, "[Feature] Compose Ulysses with
 *                    AllGather-KV as a 2D diffusion SP": commit message and
 *                    review-fix commits.
 *   [chitu-fastcp]   ChituDiffusion docs, "Install and enable Fast CP":
 *                    "Support scope".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every pointer argument is DEVICE memory allocated and owned by the
 * caller; the library never allocates, frees or retains a pointer past the call.
 * Tensors are dense, row-major ("contiguous BSHD") and must start on a 16-byte
 * boundary.  Outputs are fully overwritten; nothing stale is read from them.
 *
 * Streams.  `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 * call only enqueues work on that stream and returns; results are visible to
 * later work on the same stream.  A staging buffer reused across calls is safe
 * under in-order use on one stream (or with explicit events); using one buffer
 * from two streams without synchronisation is a data race.  The library keeps
 * no state and may be called from several host threads at once.
 *
 * Errors.  Every entry point returns 0 (CP_OK) or a CP_ERR_* code.  All argument
 * checks run on the host before anything is enqueued, so a rejected call writes
 * nothing.  There is no fallback path: an unsupported request fails.  A fault
 * inside a kernel surfaces at the caller's next synchronisation.  The message for
 * a code comes from cp_status_string().
 *
 * Dtypes.  The layout entry points move 2-byte elements bit-exactly and accept
 * CP_DTYPE_BF16 and CP_DTYPE_FP16 (the packed path of [sglang#33667] is limited
 * to those).  Attention is bf16 only.
 */
#ifndef CP_ATTN_H
#define CP_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CP_ABI_VERSION 11

typedef struct ihipStream_t* cp_stream_t; /* == hipStream_t */

enum cp_status {
  CP_OK = 0,
  CP_ERR_NULL = 1,         /* a required pointer is NULL */
  CP_ERR_DTYPE = 2,        /* dtype code not supported by this entry point */
  CP_ERR_SHAPE = 3,        /* a size is < 1, or the problem exceeds the supported extent */
  CP_ERR_DIVISIBILITY = 4, /* H % W != 0, or a chunk does not divide evenly */
  CP_ERR_HEAD_DIM = 5,     /* D not supported (layout: D % 8 != 0; attention: D not 64/128) */
  CP_ERR_ALIGNMENT = 6,    /* a pointer is not 16-byte aligned */
  CP_ERR_ALIAS = 7,        /* an output overlaps an input or another output */
  CP_ERR_SCALE = 8,        /* softmax scale is not finite or not > 0 */
  CP_ERR_UNSUPPORTED = 9,  /* a valid but unsupported request (bad phase or layout flag, W too large) */
  CP_ERR_HIP = 10,         /* the HIP runtime rejected the launch */
  CP_ERR_WORKSPACE = 11,   /* the workspace is too small (see cp_attn_workspace_bytes) */
  CP_ERR_SCRATCH = 12      /* the problem needs more than the library's static scratch array */
};

enum cp_dtype { CP_DTYPE_BF16 = 0, CP_DTYPE_FP16 = 1 };

/* Version of this ABI (CP_ABI_VERSION). */
int cp_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* cp_status_string(int status);

/*
 * Ulysses input exchange, send side: destination-major pack of Q, K and V into
 * one staging buffer, so that a single all-to-all moves all three tensors
 * ([sglang#33667], implementation breakdown items 2-3 and the usp.py excerpt of
 * _usp_input_all_to_all_qkv).
 *
 *   q, k, v : [B][S_local][H][D]            (this rank's sequence shard, all heads)
 *   staging : [W][B*S_local][H/W][3*D]      (chunk j goes to rank j)
 *   staging[j][b*S_local+s][hl][c*D+d] = X_c[b][s][j*(H/W)+hl][d],  X_0..2 = q, k, v
 *
 * Requires B, S_local, H, W >= 1, H % W == 0, D % 8 == 0 (rows of whole 16-byte
 * vectors), all four pointers 16-byte aligned, staging disjoint from q, k, v.
 */
int cp_pack_qkv_dst_major(const void* q, const void* k, const void* v, void* staging,
                          int64_t B, int64_t S_local, int64_t H, int64_t D, int64_t W,
                          int dtype, cp_stream_t stream);

/*
 * Destination-major pack with head padding, for head counts that the Ulysses
 * degree does not divide (the UAA padding of [vllm-omni#7641]'s attention
 * benchmark: 14 heads over 4 ranks padded to 16, +14.3% attention work).  The
 * head axis is read as padded with zero heads up to H_pad, then packed as by
 * cp_pack_qkv_dst_major:
 *
 *   staging[j][b*S_local+s][hl][c*D+d] = X_c[b][s][j*H_local+hl][d]  if j*H_local+hl < H,
 *                                        0                            otherwise,
 *   H_local = H_pad / W.
 *
 *   q, k, v : [B][S_local][H][D];  staging : [W][B*S_local][H_pad/W][3*D]
 *
 * Requires H <= H_pad, H_pad % W == 0 (CP_ERR_DIVISIBILITY), and the conditions
 * of cp_pack_qkv_dst_major.  H_pad == H is the plain pack.
 */
int cp_pack_qkv_dst_major_padded(const void* q, const void* k, const void* v, void* staging,
                                 int64_t B, int64_t S_local, int64_t H, int64_t H_pad, int64_t D,
                                 int64_t W, int dtype, cp_stream_t stream);

/*
 * Output merge of a padded Ulysses layout: as cp_output_reverse phase 1, keeping
 * only the first H of the W*H_local heads (the padding heads are dropped):
 *
 *   dst[b][s][g][d] = src[g / H_local][b][s][g % H_local][d],  g < H.
 *
 *   src : [W][B][S_local][H_local][D];  dst : [B][S_local][H][D]
 *
 * Requires 1 <= H <= W*H_local and the conditions of cp_output_reverse.
 */
int cp_output_merge_cropped(const void* src, void* dst, int64_t B, int64_t S_local, int64_t H_local,
                            int64_t H, int64_t D, int64_t W, int dtype, cp_stream_t stream);

/*
 * Simulated W-way all-to-all, receive side of one rank (the single-GPU stand-in
 * for the collective in [sglang#33667]'s unit-test excerpt): the chunk `rank`
 * of every sender's buffer becomes chunk r of this rank's receive buffer,
 *
 *   recv[r*C .. (r+1)*C) = sends[r][rank*C .. (rank+1)*C),  C = bytes_per_rank / W.
 *
 *   sends : host array of W device pointers, each to bytes_per_rank bytes
 *   recv  : device buffer of bytes_per_rank bytes
 *
 * Requires 1 <= W <= 64, 0 <= rank < W, bytes_per_rank % (16*W) == 0, every
 * pointer 16-byte aligned, recv disjoint from every send buffer.
 */
int cp_sim_exchange(const void* const* sends, void* recv, int64_t W, int64_t rank,
                    int64_t bytes_per_rank, cp_stream_t stream);

/*
 * Ulysses input exchange, receive side: split the received staging buffer into
 * head-sharded Q, K, V with the source-rank axis placed in front of the
 * sequence axis ([sglang#33667], usp.py excerpt: a view for B == 1, a
 * rank/batch permute for B > 1, then a split of the last axis by D).
 *
 *   recv             : [W][B*S_local][H_local][3*D]
 *   q_out/k_out/v_out: [B][W*S_local][H_local][D]
 *   X_c[b][r*S_local+s][hl][d] = recv[r][b*S_local+s][hl][c*D+d]
 *
 * Requires sizes >= 1, D % 8 == 0, 16-byte aligned pointers, the three outputs
 * pairwise disjoint and disjoint from recv.
 */
int cp_unpack_head_sharded(const void* recv, void* q_out, void* k_out, void* v_out,
                           int64_t B, int64_t S_local, int64_t H_local, int64_t D,
                           int64_t W, int dtype, cp_stream_t stream);

/*
 * Non-causal multi-head attention of local queries against global keys, the
 * plain problem an AllGather-KV rank hands to its backend ([vllm-omni#7641],
 * commit message; MHA, BF16, D 128 in [chitu-fastcp] "Support scope"):
 *
 *   o[b,i,h,:] = sum_{j valid} softmax_j(scale * q[b,i,h,:] . k[b,j,h,:]) v[b,j,h,:]
 *
 *   q, o     : [B][Sq][H][D]  bf16
 *   k, v     : [B][Skv][H][D] bf16
 *   key_mask : NULL, or [B][Skv] uint8 key-validity mask, nonzero = attend (the
 *              2D key mask of [vllm-omni#7641]'s review fixes; any alignment)
 *   scale    : softmax scale, finite and > 0 (1/sqrt(D) for standard attention)
 *
 * Non-causal is the only mode: the pages attend every query to every valid key
 * ([chitu-fastcp] "Support scope" lists non-causal attention only), so there is
 * no causal flag.
 *
 * Softmax statistics and accumulation are fp32; probabilities are rounded to
 * bf16 before the P.V product; o is rounded to nearest-even bf16.  A query row
 * whose batch has no valid key gets zeros.  Requires B, Sq, Skv, H >= 1,
 * D in {64, 128}, q/k/v/o 16-byte aligned, o disjoint from q, k, v.
 */
int cp_attn_localq_globalkv(const void* q, const void* k, const void* v,
                            const uint8_t* key_mask, void* o,
                            int64_t B, int64_t Sq, int64_t Skv, int64_t H, int64_t D,
                            float scale, cp_stream_t stream);

/*
 * The same attention with a caller-owned workspace, which lets the library
 * split the key range of each query block (128 query rows) over several
 * workgroups, with the partial softmax states merged by their log-sum-exp as
 * split-KV / FlashDecoding do, when the query blocks alone would occupy at
 * most half of the GPU.  The
 * [vllm-omni#7641] "Recommended follow-up" note on attention over arriving
 * K/V chunks is the same merge.  The split is deterministic for a given
 * problem and device, so results are reproducible run to run.
 *
 *   workspace       : NULL (never split; identical to cp_attn_localq_globalkv),
 *                     or device memory of workspace_bytes, 16-byte aligned,
 *                     disjoint from q, k, v, o and key_mask.  Contents on
 *                     entry are ignored; the library never allocates.
 *   workspace_bytes : at least cp_attn_workspace_bytes(B, Sq, Skv, H, D)
 *                     for the current device, else CP_ERR_WORKSPACE.
 *
 * The workspace is used by the kernels enqueued on `stream`; reusing it on
 * another stream without ordering is a race.
 */
int cp_attn_localq_globalkv_ws(const void* q, const void* k, const void* v,
                               const uint8_t* key_mask, void* o,
                               int64_t B, int64_t Sq, int64_t Skv, int64_t H, int64_t D,
                               float scale, void* workspace, size_t workspace_bytes,
                               cp_stream_t stream);

/*
 * The same attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * split-KV partial states live in a static device array of
 * CP_ATTN_NOALLOC_SCRATCH_BYTES bytes inside the library (one 128 x 130 fp32
 * slot per compute unit for up to 256 compute units), of which each device holds
 * its own copy from the first call on it until the process ends.  Arguments,
 * results and conditions are those of cp_attn_localq_globalkv_ws, and the
 * results are bit-identical to it.  The call allocates and frees nothing.
 *
 * A problem whose split would need more scratch than the array holds (only on a
 * device with more than 256 compute units) is rejected with CP_ERR_SCRATCH
 * before anything is enqueued.  All calls on one device share that device's
 * array and leave their partial states in it (nothing in it needs to start
 * cleared: every slot a call reads it has written first), so two calls that
 * can overlap on one device -- on two streams without ordering, or from two
 * host threads -- race.  Calls on one stream are safe.
 */
#define CP_ATTN_NOALLOC_SCRATCH_BYTES (256u * 128u * 130u * 4u)
int cp_attn_localq_globalkv_noalloc(const void* q, const void* k, const void* v,
                                    const uint8_t* key_mask, void* o,
                                    int64_t B, int64_t Sq, int64_t Skv, int64_t H, int64_t D,
                                    float scale, cp_stream_t stream);

/*
 * Bytes of workspace cp_attn_localq_globalkv_ws may use for this problem on
 * the current device (an upper bound: one partial slot of 128 x (D + 2) floats
 * per compute unit).  0 for an unsupported D.  No GPU work, no allocation.
 */
size_t cp_attn_workspace_bytes(int64_t B, int64_t Sq, int64_t Skv, int64_t H, int64_t D);

/*
 * Joint text/image attention of the composed Ulysses x AllGather-KV layout
 * ([vllm-omni#7641]: the Ulysses step keeps the head-sliced joint (text) K/V
 * aside, the AllGather-KV step gathers the image K/V and re-attaches the joint
 * tensors in front of or behind them; the review-fix commits merge the 2D key
 * masks against that final key layout, filling a missing side with "attend").
 * The keys are the two segments in that order, each with its own optional
 * mask, attended as one sequence without building the concatenation:
 *
 *   keys = joint_front ? [joint | image] : [image | joint]
 *   mask = the same concatenation of img_mask and joint_mask (NULL = all valid)
 *   o[b,i,h,:] = sum_{j valid} softmax_j(scale * q[b,i,h,:] . key_j) value_j
 *
 *   q, o              : [B][Sq][H][D] bf16
 *   k_img, v_img      : [B][S_img][H][D] bf16;  img_mask   : NULL or [B][S_img] uint8
 *   k_joint, v_joint  : [B][T][H][D] bf16;      joint_mask : NULL or [B][T] uint8
 *   joint_front       : 1 = joint keys first, 0 = image keys first
 *   workspace         : as for cp_attn_localq_globalkv_ws (sized for Skv = S_img + T), or NULL
 *
 * T == 0 (no joint tokens; k_joint/v_joint may be NULL) is plain attention over
 * the image keys.  Requires S_img >= 1, T >= 0, the attention's conditions, and
 * o disjoint from every input.  The result equals cp_attn_localq_globalkv on
 * the concatenated keys, values and mask up to the order of summation.
 */
int cp_attn_joint(const void* q, const void* k_img, const void* v_img, const uint8_t* img_mask,
                  const void* k_joint, const void* v_joint, const uint8_t* joint_mask, int joint_front,
                  void* o, int64_t B, int64_t Sq, int64_t S_img, int64_t T, int64_t H, int64_t D,
                  float scale, void* workspace, size_t workspace_bytes, cp_stream_t stream);

/*
 * Attention over keys that arrive in chunks: a forward pass over one K/V chunk
 * that also returns the log-sum-exp, and a merge of such partial results (the
 * forward / merge split of [chitu-fastcp] FAQ and section 5; the
 * [vllm-omni#7641] "Recommended follow-up" note on attending to gathered K/V
 * as it arrives).  With z_ij = scale * q_i . k_j over the chunk's valid keys:
 *
 *   lse[b][h][i]     = ln sum_j exp(z_ij)           (-inf if the chunk has no valid key)
 *   o_part[b][i][h]  = sum_j exp(z_ij - lse) v_j     (zeros if no valid key)
 *
 *   q            : [B][Sq][H][D] bf16;  k, v : [B][Skv][H][D] bf16 (this chunk)
 *   key_mask     : NULL or [B][Skv] uint8 for this chunk, nonzero = attend
 *   o_part       : [B][Sq][H][D] fp32, 16-byte aligned
 *   lse          : [B][H][Sq] fp32, 4-byte aligned
 *
 * Same arithmetic and conditions as cp_attn_localq_globalkv (bf16
 * probabilities, fp32 accumulation); o_part and lse must not overlap each
 * other or any input.
 */
int cp_attn_partial(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                    void* o_part, void* lse, int64_t B, int64_t Sq, int64_t Skv, int64_t H,
                    int64_t D, float scale, cp_stream_t stream);

/*
 * Attention over the next key chunk folded into a running state, for K/V that
 * arrive chunk by chunk (same definitions as cp_attn_partial and cp_attn_merge;
 * the merge happens in this call's epilogue, so no partial buffers and no merge
 * launch are needed).  The state is a partial result in cp_attn_partial's
 * format: state_o [B][Sq][H][D] fp32 (normalised) and state_lse [B][H][Sq]
 * fp32; a row whose state_lse is -inf has no contribution yet (its state_o is
 * not read).  With L = ln(e^state_lse + e^lse_chunk):
 *
 *   merged = e^(state_lse - L) state_o + e^(lse_chunk - L) o_chunk
 *
 *   o_final == NULL : the state is updated in place (state_o = merged, state_lse = L)
 *   o_final != NULL : merged is written to o_final [B][Sq][H][D] as bf16 (RNE) and
 *                     the state is left unchanged (the last chunk)
 *
 * A sequence: cp_attn_partial on the first chunk (or a state with lse = -inf),
 * then cp_attn_partial_accum on each further chunk, o_final given on the last.
 * The state must not overlap q, k, v or key_mask; o_final must not overlap
 * anything.  Other conditions as for cp_attn_partial.
 */
int cp_attn_partial_accum(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                          void* state_o, void* state_lse, void* o_final, int64_t B, int64_t Sq, int64_t Skv,
                          int64_t H, int64_t D, float scale, cp_stream_t stream);

/*
 * Merge of N partial results of the same queries over disjoint key sets:
 *
 *   L = ln sum_k exp(lse_k),   o = sum_k exp(lse_k - L) o_part_k   (bf16, RNE)
 *
 * Rows whose lse is -inf in every part (no valid key anywhere) get zeros.
 *
 *   o_parts : [N][B][Sq][H][D] fp32, 16-byte aligned
 *   lses    : [N][B][H][Sq] fp32, 4-byte aligned
 *   o       : [B][Sq][H][D] bf16, 16-byte aligned, disjoint from both inputs
 *
 * Requires N, B, Sq, H >= 1 and D in {64, 128}.
 */
int cp_attn_merge(const void* o_parts, const void* lses, int64_t N, void* o,
                  int64_t B, int64_t Sq, int64_t H, int64_t D, cp_stream_t stream);

/*
 * Ulysses attention fused with the steps on either side of it: the attention
 * of this rank's H_local heads over the whole sequence S = W * S_local reads
 * Q, K and V straight out of the received staging buffer (the unpack of
 * cp_unpack_head_sharded becomes addressing, as the B == 1 "view, no copy"
 * case of [sglang#33667]'s usp.py excerpt already is for the sequence axis),
 * and writes O straight into the send layout of cp_output_reverse phase 0.
 * The result equals
 *
 *   cp_unpack_head_sharded(recv) -> cp_attn_localq_globalkv(q, k, v) with
 *   Sq = Skv = S, H = H_local -> cp_output_reverse(SEND)
 *
 * bit for bit, without the intermediate Q/K/V and O buffers.
 *
 *   recv      : [W][B*S_local][H_local][3*D] bf16 (q, k, v concatenated per head)
 *   key_mask  : NULL, or [B][S] uint8 over the global key index r*S_local + s
 *   send      : [W][B][S_local][H_local][D] bf16
 *   workspace : as for cp_attn_localq_globalkv_ws (sized by
 *               cp_attn_workspace_bytes(B, S, S, H_local, D)), or NULL
 *
 * Requires the attention's conditions (D in {64, 128}, scale),
 * W >= 1, 16-byte aligned pointers, send disjoint from recv and key_mask.  With
 * B > 1 a batch's rows arrive in W chunks of S_local rows; when S_local is not a
 * multiple of 64, key tiles that span chunks are addressed row by row, which
 * needs recv to be smaller than 2 GB (CP_ERR_SHAPE otherwise).
 */
int cp_attn_recv_to_send(const void* recv, const uint8_t* key_mask, void* send,
                         int64_t B, int64_t S_local, int64_t H_local, int64_t D, int64_t W,
                         float scale, void* workspace, size_t workspace_bytes,
                         cp_stream_t stream);

/*
 * The same for the 2D layout ([vllm-omni#7641]: Ulysses groups of W ranks inside
 * AllGather-KV groups): the rank's keys are its own Ulysses group's sequence,
 * received in recv, and the sequence of the other AllGather rank, whose
 * head-sharded K and V (the same heads) are already resident.  The two key
 * ranges are attended as one sequence, the other rank's first when other_first
 * is 1 (it holds the earlier sequence region), else after the rank's own.  The
 * result equals
 *
 *   cp_unpack_head_sharded(recv) -> cp_attn_joint(q, own K/V, other K/V, in the
 *   order above) with Sq = W*S_local, H = H_local -> cp_output_reverse(SEND)
 *
 * bit for bit, without the intermediate Q/K/V and O buffers.
 *
 *   recv       : [W][B*S_local][H_local][3*D] bf16 (q, k, v concatenated per head)
 *   k_other,
 *   v_other    : [B][S_other][H_local][D] bf16
 *   own_mask   : NULL, or [B][W*S_local] uint8 over the rank's own keys
 *   other_mask : NULL, or [B][S_other] uint8 over the other rank's keys
 *   send       : [W][B][S_local][H_local][D] bf16
 *   workspace  : as for cp_attn_localq_globalkv_ws (sized by
 *                cp_attn_workspace_bytes(B, W*S_local, W*S_local + S_other, H_local, D)),
 *                or NULL; it must not overlap any operand
 *
 * Requires what cp_attn_recv_to_send requires, S_other >= 1, other_first in
 * {0, 1} (CP_ERR_UNSUPPORTED otherwise), k_other / v_other 16-byte aligned and
 * disjoint from send.
 */
int cp_attn_recv_to_send_2d(const void* recv, const void* k_other, const void* v_other, int64_t S_other,
                            int other_first, const uint8_t* own_mask, const uint8_t* other_mask,
                            void* send, int64_t B, int64_t S_local, int64_t H_local, int64_t D,
                            int64_t W, float scale, void* workspace, size_t workspace_bytes,
                            cp_stream_t stream);

/*
 * Ulysses output exchange ([sglang#33667] names _usp_output_all_to_all in its
 * implementation breakdown; [vllm-omni#7641] ends each attention with the
 * reverse Ulysses step).  Read as the exact inverse of the input exchange with
 * the same flat-chunk collective, it has a send phase and a merge phase:
 *
 *   phase 0 (SEND) : src [B][W*S_local][H_local][D] -> dst [W][B][S_local][H_local][D]
 *                    dst[r][b][s][hl][d] = src[b][r*S_local+s][hl][d]
 *                    (the identity on memory when B == 1)
 *   phase 1 (MERGE): src [W][B][S_local][H_local][D] -> dst [B][S_local][W*H_local][D]
 *                    dst[b][s][j*H_local+hl][d] = src[j][b][s][hl][d]
 *
 * Requires sizes >= 1, D % 8 == 0, 16-byte aligned pointers, dst disjoint from
 * src, phase in {0, 1}.
 */
int cp_output_reverse(int phase, const void* src, void* dst,
                      int64_t B, int64_t S_local, int64_t H_local, int64_t D, int64_t W,
                      int dtype, cp_stream_t stream);

/*
 * Packed query boundaries of one AllGather-KV rank ([vllm-omni#7641], review-fix
 * commit on packed query metadata).  Packed documents (requests) share one
 * sequence; cu_seqlens holds their n_docs + 1 cumulative boundaries.  After the
 * K/V gather a rank keeps only the query rows [rank*S_local, (rank+1)*S_local),
 * so every global query document is intersected with that span: entry i of the
 * result is boundary i clamped into the span and shifted to it,
 *
 *   cu_q_local[i] = min(max(cu_q_global[i] - rank*S_local, 0), S_local),
 *
 * which keeps exactly one, possibly empty, local entry per document (query
 * document i still pairs with key document i; the key boundaries stay global).
 * The remap runs on the device, in stream order, with no host synchronisation.
 *
 *   cu_q_global : [n_docs + 1] int32, device, non-decreasing
 *   cu_q_local  : [n_docs + 1] int32, device, output; disjoint from cu_q_global
 *
 * Requires n_docs >= 1, rank >= 0, S_local >= 1 with rank*S_local and
 * S_local within int32 (CP_ERR_SHAPE), 4-byte aligned pointers.
 */
int cp_varlen_remap_cu_seqlens_q(const int32_t* cu_q_global, int32_t* cu_q_local, int64_t n_docs,
                                 int64_t rank, int64_t S_local, cp_stream_t stream);

/*
 * Packed variable-length attention (the packed backend of [vllm-omni#7641]'s
 * review-fix commit on packed query metadata, on the AllGather-KV rank's local
 * query rows).  One packed batch row: query document i takes rows
 * [cu_seqlens_q[i], cu_seqlens_q[i+1]) of q and attends, non-causally, to the
 * key rows [cu_seqlens_k[i], cu_seqlens_k[i+1]) of k and v only:
 * softmax(scale q k^T) v per document and head.
 *
 *   q, o           : [Sq][H][D] bf16 (o disjoint from every input)
 *   k, v           : [Skv][H][D] bf16
 *   cu_seqlens_q/k : [n_docs + 1] int32, device, non-decreasing, within
 *                    [0, Sq] and [0, Skv] (read by the kernel and not checked on
 *                    the host; out-of-range values are clamped into the buffers,
 *                    so a malformed array gives wrong rows, never an access
 *                    outside them)
 *
 * The work is one block per (head, 128-row tile of the packed query rows), which
 * finds the tile's first document by binary search on cu_seqlens_q, and one per
 * (head, document), which runs the document on the tile where it starts when an
 * earlier document has rows there too; no max_seqlen_q is needed.  A document with query rows and no key
 * rows gets zero outputs.  Rows of o outside every document are not written (the
 * one exception to "outputs are fully overwritten").  No key mask, no split; D in
 * {64, 128}, 16-byte aligned q, k, v, o and 4-byte aligned boundary
 * arrays; n_docs >= 1.
 */
int cp_attn_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                   const int32_t* cu_seqlens_k, int64_t n_docs, void* o,
                   int64_t Sq, int64_t Skv, int64_t H, int64_t D, float scale,
                   cp_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CP_ATTN_H */
