/*
 * ulysses.h -- C ABI of the MI355X (gfx950) per-rank hot path of
 * DeepSpeed-Ulysses sequence parallelism: the local halves of the two
 * all-to-alls and the head-sharded attention between them.
 *
 * Pages cited (title, then section):
 *   [ATLAS] "02 · DeepSpeed-Ulysses" (llm-infra-atlas, parallel/04_cp),
 *           §1 attention is parallel over heads, §2 the all-to-all as a
 *           transpose, §3 the head-count constraint.
 *   [DSU]   "DeepSpeed-Ulysses 深度解析：用 All-to-All 序列并行撑起百万 Token
 *           超长序列训练", core design steps 1-5 and the DistributedAttention
 *           signature (scatter_idx, gather_idx, sp_stream, num_kv_heads).
 *   [CMP]   "Ulysses vs Ring Attention：序列并行深度对比", §三 (Q, K and V take
 *           the same all-to-all; Ulysses' degree is capped by num_kv_heads).
 *   [SPCP]  "长上下文训练中的 SP 与 CP：从 Megatron 到分布式 Attention",
 *           the Ulysses section (P must divide the KV head count under GQA)
 *           and the Ring section (online softmax, scale 1/sqrt(d_h)), USP.
 *
 * General conventions
 *   - Every tensor pointer is a DEVICE pointer to a contiguous row-major
 *     array (last axis fastest) and must be 16-byte aligned.  The caller owns
 *     every buffer; the library allocates nothing and keeps no state between
 *     calls, so the entry points are thread-safe -- except that
 *     ulys_attn_fwd_noalloc works in one fixed device array per GPU, so its
 *     calls that overlap in time on one GPU race (see there).
 *   - s, h and h_kv are GLOBAL sizes (whole sequence, all heads); P is the
 *     number of ranks of the sequence-parallel group.  Shapes below use
 *     sl = s/P, hp = h/P, and hkvp = h_kv/P, or hkvp = 1 when h_kv < P and
 *     h_kv | P (KV heads replicated, see ulys_pack_seq2head_kv).
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Each
 *     entry only enqueues kernels on it and never synchronizes.
 *   - Arguments are validated on the host first; on any error the entry
 *     point returns a negative ULYS_ERR_* code and launches nothing.  A
 *     launch failure returns ULYS_ERR_HIP.  No entry prints, throws or sets
 *     errno.
 *   - Outputs are written out of place: the byte ranges of inputs and
 *     outputs must not overlap (ULYS_ERR_ALIAS).
 */
#ifndef ULYSSES_H_
#define ULYSSES_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
typedef enum { ULYS_F32 = 0, ULYS_BF16 = 1 } ulys_dtype;

/* Status codes. */
enum {
  ULYS_OK = 0,
  ULYS_ERR_NULL = -1,         /* a required pointer is NULL                      */
  ULYS_ERR_DIM = -2,          /* a size is <= 0 or too large                      */
  ULYS_ERR_DIVISIBILITY = -3, /* P !| s, P !| h, h_kv !| h, or neither of P and  */
                              /* h_kv divides the other                          */
  ULYS_ERR_UNSUPPORTED = -4,  /* dtype or head size not supported by the kernel   */
  ULYS_ERR_ALIGNMENT = -5,    /* a pointer is not 16-byte aligned                 */
  ULYS_ERR_ALIAS = -6,        /* an output overlaps an input or another output    */
  ULYS_ERR_HIP = -7           /* the HIP runtime reported a launch error          */
};

/*
 * Seq->head all-to-all, send side (pack), one rank.
 * [ATLAS] §2: the local [sl, heads, d] is split along the head axis into P
 * equal groups and group r is sent to rank r; [DSU] step 3 (the exchange of
 * Q, K and V before attention, scatter_idx=2).  For K and V pass h = h_kv.
 *
 *   x : input  [sl, b, h, d_h]        the rank's sequence shard
 *   y : output [P, sl, b, hp, d_h]    send buffer; block r is for rank r,
 *                                     y[r] = x[:, :, r*hp:(r+1)*hp, :]
 * The receive side needs no kernel: rank r's P received blocks, stored in
 * source-rank order, are exactly its [s, b, hp, d_h] share (the sequence
 * axis is outermost).  The move is bit-exact for every bit pattern.
 * Errors: NULL pointers, sizes <= 0, P !| s or P !| h, dtype not F32/BF16,
 * misaligned or overlapping buffers.
 */
int ulys_pack_seq2head(const void* x, void* y, int64_t s, int64_t b, int64_t h,
                       int64_t d_h, int32_t P, int32_t dtype, void* stream);

/*
 * Seq->head send side for K or V when the model may have fewer KV heads than
 * ranks.  [CMP] §三: Q, K and V take the same all-to-all, so a plain split of
 * h_kv < P heads leaves some ranks with no KV head (one head on four ranks:
 * [1, 0, 0, 0]); [SPCP] (Ulysses section): replicating KV heads lifts the
 * requirement that P divide h_kv, at a cost in memory and traffic; [DSU]:
 * num_kv_heads is given when heads do not divide evenly.
 *
 *   x : input  [sl, b, h_kv, d_h]                 the rank's K or V shard
 *   y : output [P, sl, b, max(1, h_kv/P), d_h]    send buffer, block r for rank r
 * With P | h_kv this is ulys_pack_seq2head.  With h_kv < P and h_kv | P,
 * block r is KV head floor(r*h_kv/P) -- the head that rank r's query heads
 * [r*hp, (r+1)*hp) use under the contiguous GQA grouping -- so after the
 * exchange every rank holds one KV head for the whole sequence, and
 * ulys_attn_fwd / ulys_attn_bwd take the model's h_kv unchanged.  Bit-exact.
 * Errors: as ulys_pack_seq2head, with ULYS_ERR_DIVISIBILITY unless P | s and
 * (P | h_kv or h_kv | P); ULYS_ERR_DIM for more than 2^31 elements with
 * replication.
 */
int ulys_pack_seq2head_kv(const void* x, void* y, int64_t s, int64_t b, int64_t h_kv,
                          int64_t d_h, int32_t P, int32_t dtype, void* stream);

/*
 * The send sides of Q, K and V in one call: the same results as
 * ulys_pack_seq2head(xq -> yq, h) followed by ulys_pack_seq2head_kv(xk -> yk,
 * h_kv) and ulys_pack_seq2head_kv(xv -> yv, h_kv) ([DSU] step 3: Q, K and V
 * each go through the seq->head exchange; [CMP] §三: all three take the same
 * path), done by a single kernel launch when every run is a whole number of
 * 16-byte vectors (else the three packs in turn).  Shapes, validation and
 * errors as the single packs; no output may overlap any input or another
 * output.
 */
int ulys_pack_seq2head_qkv(const void* xq, const void* xk, const void* xv, void* yq, void* yk,
                           void* yv, int64_t s, int64_t b, int64_t h, int64_t h_kv, int64_t d_h,
                           int32_t P, int32_t dtype, void* stream);

/*
 * Backward of ulys_pack_seq2head_kv, receive side: the gradients of K or V
 * sent back by the P ranks (block r from rank r) into the rank's
 * [sl, b, h_kv, d_h] shard.  With P | h_kv this is ulys_unpack_head2seq.  With
 * replication the gradient of a KV head is the sum of its copies' gradients
 * ([SPCP]: a K/V row used by many queries receives the sum of their
 * gradients): x[:, :, g, :] = sum over j < P/h_kv of y[g*P/h_kv + j],
 * accumulated in fp32 in ascending j and rounded once (nearest-even) to the
 * dtype.
 *   y : input  [P, sl, b, max(1, h_kv/P), d_h]
 *   x : output [sl, b, h_kv, d_h]
 * Errors: as ulys_pack_seq2head_kv.
 */
int ulys_unpack_head2seq_kv(const void* y, void* x, int64_t s, int64_t b, int64_t h_kv,
                            int64_t d_h, int32_t P, int32_t dtype, void* stream);

/*
 * Head->seq all-to-all, receive side (unpack), one rank.
 * [ATLAS] §2: the second all-to-all inverts the first: the P blocks received
 * (block r holds head group r of this rank's sequence segment) are
 * concatenated along the head axis; [DSU] step 5 (gather_idx=2 for the
 * output).  It is the exact inverse of ulys_pack_seq2head.
 *
 *   y : input  [P, sl, b, hp, d_h]    received blocks, block r = head group r
 *   x : output [sl, b, h, d_h]        x[:, :, r*hp:(r+1)*hp, :] = y[r]
 * Errors: as ulys_pack_seq2head.
 */
int ulys_unpack_head2seq(const void* y, void* x, int64_t s, int64_t b, int64_t h,
                         int64_t d_h, int32_t P, int32_t dtype, void* stream);

/*
 * Head-sharded attention on one rank's share (forward).
 * [ATLAS] §1 and [DSU] step 4: with the whole sequence for hp heads, each
 * head computes softmax(Q K^T / sqrt(d_h)) V independently; the scale is
 * fixed at 1/sqrt(d_h) ([SPCP], Ring section).  causal != 0 lets query t see
 * keys j <= t (global positions; the received blocks are in sequence order).
 * GQA: query head i of the share reads KV head i / (h/h_kv), i.e. contiguous
 * groups ([DSU] num_kv_heads; [SPCP] requires P | h_kv).  With h_kv < P
 * (h_kv | P) the share holds the one replicated KV head that all its query
 * heads read (ulys_pack_seq2head_kv).
 *
 *   q   : [s, b, hp, d_h]      o : [s, b, hp, d_h]   (same dtype as q)
 *   k,v : [s, b, hkvp, d_h]
 *   lse : [b, hp, s] fp32 natural-log sum of exp of the scaled scores,
 *         or NULL to skip it.
 * O is accumulated in fp32 and rounded once (nearest-even) to the dtype.
 * Supported: ULYS_BF16 with d_h in {64, 128} (MFMA kernel); ULYS_F32 with
 * d_h in {64, 128} (fp32 kernel, b * h/P at most 65535).  s may be any
 * positive multiple of P.
 * Errors: as above, plus h_kv !| h, neither of P and h_kv dividing the other,
 * unsupported d_h/dtype, and o or lse overlapping q, k, v or each other.
 */
int ulys_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  int64_t s, int64_t b, int64_t h, int64_t h_kv, int64_t d_h, int32_t P,
                  int32_t causal, int32_t dtype, void* stream);

/*
 * ulys_attn_fwd with a caller-owned workspace, used to balance the work.
 * When a causal share has too few query blocks (256 queries of one head, or
 * fewer queries of several heads of one GQA group) to fill the GPU's resident
 * workgroups twice (e.g. s = 32768 with 2 heads), one block's keys would set
 * the run time; with a workspace of ulys_attn_fwd_workspace_size() bytes the
 * keys of every block are split into two halves computed by separate
 * workgroups, each leaving its partial (m, l, O) state in the workspace, and a
 * second kernel merges the halves with the online-softmax rescaling
 * ([SPCP] Ring section: partial results over disjoint key ranges combine by
 * rescaling with the running max).  The result equals ulys_attn_fwd's up to
 * fp32 rounding order.  When a share is four or more rounds of workgroups
 * (e.g. s = 131072 with 4 heads), the workspace instead holds a counter from
 * which every workgroup takes the next block, so that XCDs running at
 * different clocks share the blocks by speed (one atomic add per workgroup,
 * on the counter only; every block is still computed by the same code), so
 * the result is then identical to ulys_attn_fwd's, bit for bit.
 *
 *   workspace       : device pointer, 16-byte aligned, or NULL (then this call
 *                     is ulys_attn_fwd); must not overlap q, k, v, o or lse.
 *                     Contents on entry are ignored; on return undefined.
 *   workspace_bytes : its size; a smaller workspace than required disables the
 *                     split or the counter (still correct).
 * Errors: as ulys_attn_fwd, plus ULYS_ERR_DIM for workspace_bytes < 0,
 * ULYS_ERR_ALIGNMENT / ULYS_ERR_ALIAS for the workspace.  Calls that share one
 * workspace must be ordered (same stream).
 */
int ulys_attn_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t s, int64_t b, int64_t h, int64_t h_kv, int64_t d_h, int32_t P,
                     int32_t causal, int32_t dtype, void* workspace, int64_t workspace_bytes,
                     void* stream);

/* Size of the fixed device scratch of ulys_attn_fwd_noalloc, in bytes. */
#define ULYS_NOALLOC_SCRATCH_BYTES (96LL << 20)

/*
 * ulys_attn_fwd_ws without caller memory, for callers that cannot allocate
 * device memory (work captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results, bit for
 * bit, as ulys_attn_fwd_ws with a workspace of
 * ulys_attn_fwd_workspace_size() bytes, the workspace being a fixed array of
 * ULYS_NOALLOC_SCRATCH_BYTES (96 MiB) in the library's device memory.  The
 * array is part of the library's device code, so every GPU on which any of
 * the library's kernels has run holds its own copy until the process ends;
 * the call allocates nothing.
 *   Arguments, layouts and errors as ulys_attn_fwd, plus ULYS_ERR_DIM when the
 *   workspace the call would use exceeds the array (a causal share with too
 *   few blocks to fill the GPU twice, whose split partial states need more
 *   than 96 MiB; e.g. s = 51200 with 2 heads of 128), ULYS_ERR_HIP when the
 *   array's device address cannot be resolved.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (two streams, two host threads) race on it and give undefined
 * results; calls ordered on one stream are safe.
 */
int ulys_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                          int64_t s, int64_t b, int64_t h, int64_t h_kv, int64_t d_h, int32_t P,
                          int32_t causal, int32_t dtype, void* stream);

/*
 * Workspace bytes ulys_attn_fwd_ws uses for these arguments on the current
 * device: the split's partial states, 256 for the block counter, or 0.  Negative ULYS_ERR_* for arguments
 * ulys_attn_fwd would reject on size, divisibility or dtype grounds.
 */
int64_t ulys_attn_fwd_workspace_size(int64_t s, int64_t b, int64_t h, int64_t h_kv, int64_t d_h,
                                     int32_t P, int32_t causal, int32_t dtype);

/*
 * Backward of the head-sharded attention on one rank's share.
 * [ATLAS] §5: both all-to-alls are linear and their backward is the same
 * exchange with the split and concatenation axes swapped, so the gradient of
 * the layer's output is brought to head-sharded form with
 * ulys_pack_seq2head (plus the exchange) and dq, dk, dv go back with
 * ulys_unpack_head2seq; the local attention's backward is the ordinary
 * attention backward, i.e. the gradient of ulys_attn_fwd's result:
 *   P = exp(S - lse) with S = q k^T / sqrt(d_h) (causal: keys j <= t),
 *   dP = dout v^T, D = rowsum(dout * o), dS = P * (dP - D),
 *   dq = dS k / sqrt(d_h), dk = dS^T q / sqrt(d_h), dv = P^T dout,
 * with dk and dv summed over the query heads of each GQA group (contiguous
 * groups, as in ulys_attn_fwd; [SPCP] notes that a K/V row used by many
 * queries receives the sum of their gradients).
 *
 *   q, o, dout : [s, b, hp, d_h]; o and lse are ulys_attn_fwd's outputs for
 *                the same q, k, v
 *   k, v       : [s, b, hkvp, d_h]
 *   lse        : [b, hp, s] fp32 (required)
 *   dq         : [s, b, hp, d_h]   dk, dv : [s, b, hkvp, d_h]   (dtype of q)
 *   workspace  : device, 16-byte aligned, at least
 *                ulys_attn_bwd_workspace_size() bytes (per-row statistics;
 *                for bf16 also partial sums when a causal share is split and,
 *                on shares of four or more rounds of dQ work, a counter from
 *                which the dQ workgroups take their blocks); contents ignored
 *                on entry, undefined on return.
 * Gradients are accumulated in fp32 and rounded once (nearest-even) to the
 * dtype.  No
 * gradient is accumulated with atomics: every output element is summed by
 * one workgroup in a fixed order (split halves are added by a merge kernel in
 * a fixed order), so the result does not depend on scheduling.  The only
 * atomic is the dQ kernel's unit counter on long shares: each workgroup takes
 * the index of the next query block from it, and that block is then computed
 * by the same code whichever workgroup runs it, so the values are the same
 * bit for bit as with the static block order.
 * Supported: ULYS_BF16 with d_h in {64, 128} (MFMA kernels); ULYS_F32 with
 * d_h in {64, 128} (fp32 kernels: one group of d_h/32 lanes per query row for
 * dq and per key row for dk and dv, b * h/P at most 65535).
 * Errors: as ulys_attn_fwd, plus ULYS_ERR_NULL for any missing pointer
 * (lse and workspace included), ULYS_ERR_UNSUPPORTED for another dtype or
 * head size, ULYS_ERR_DIM for a workspace smaller than required, and
 * ULYS_ERR_ALIAS when an output or the workspace overlaps an input or
 * another output.
 */
int ulys_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, int64_t s, int64_t b, int64_t h,
                  int64_t h_kv, int64_t d_h, int32_t P, int32_t causal, int32_t dtype,
                  void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Workspace bytes ulys_attn_bwd needs for these arguments; negative
 * ULYS_ERR_* for arguments it would reject on size, divisibility, dtype or
 * head size.
 */
int64_t ulys_attn_bwd_workspace_size(int64_t s, int64_t b, int64_t h, int64_t h_kv, int64_t d_h,
                                     int32_t P, int32_t causal, int32_t dtype);

/* Largest P the push entry points take (the destination table size). */
#define ULYS_MAX_RANKS 64

/*
 * Seq->head exchange as pushes, the send side of one rank writing straight
 * into every rank's receive buffer.  [ATLAS] §2: rank `rank` splits its
 * [sl, b, h, d_h] shard along heads and sends group r to rank r, which
 * concatenates what it receives along the sequence in source order; here the
 * sender places its block at rows [rank*sl, (rank+1)*sl) of rank r's share,
 * so neither the send buffer of ulys_pack_seq2head nor a receive-side step
 * exists.  On a node the P destinations are the ranks' share buffers mapped
 * into this process (hipIpcOpenMemHandle); on one GPU any P buffers.
 *
 *   x       : [sl, b, h, d_h]        this rank's shard (device)
 *   y_ranks : HOST array of P device pointers; y_ranks[r] is rank r's share
 *             [s, b, hp, d_h]; this call writes its rows [rank*sl, (rank+1)*sl)
 *   rank    : this rank, 0 <= rank < P <= ULYS_MAX_RANKS
 * After every rank's call (and the streams' ordering across ranks), share r
 * equals what ulys_pack_seq2head + an all-to-all + the source-ordered receive
 * gives.  Bit-exact.  Errors: as ulys_pack_seq2head, plus ULYS_ERR_DIM for P
 * or rank out of range, ULYS_ERR_NULL / ULYS_ERR_ALIGNMENT for any
 * destination, ULYS_ERR_ALIAS when a written range overlaps x or another
 * destination's.
 */
int ulys_seq2head_push(const void* x, void* const* y_ranks, int32_t rank, int64_t s, int64_t b,
                       int64_t h, int64_t d_h, int32_t P, int32_t dtype, void* stream);

/*
 * Head->seq exchange as pushes, from rank `rank` holding head group `rank`
 * ([ATLAS] §2: the reverse exchange splits along the sequence and the
 * receiver concatenates along heads): rank j's shard x_ranks[j]
 * [sl, b, h, d_h] receives rows [j*sl, (j+1)*sl) of this rank's output o
 * [s, b, hp, d_h] at heads [rank*hp, (rank+1)*hp).  Replaces the send of O's
 * blocks and ulys_unpack_head2seq.  Bit-exact.  Errors: as
 * ulys_seq2head_push.
 */
int ulys_head2seq_push(const void* o, void* const* x_ranks, int32_t rank, int64_t s, int64_t b,
                       int64_t h, int64_t d_h, int32_t P, int32_t dtype, void* stream);

/*
 * Attention of one rank's share with the head->seq exchange fused into its
 * epilogue: the result of ulys_attn_fwd_ws followed by ulys_head2seq_push,
 * without the output tensor in between.  Query row t of the share (global
 * position t) is written, rounded once to bf16, into rank j = t / sl's shard
 * x_ranks[j] [sl, b, h, d_h] at token t % sl, heads [rank*hp, (rank+1)*hp)
 * ([ATLAS] §2: the reverse exchange sends by sequence segment, the receiver
 * concatenates along heads; [ATLAS] §1 / [DSU] step 4 for the attention).
 * On a node the destinations are the ranks' shards mapped into this process,
 * so the output crosses xGMI once, straight from the attention kernel.
 *
 *   q, k, v, lse, s, b, h, h_kv, d_h, P, causal, workspace: as
 *             ulys_attn_fwd_ws (lse [b, hp, s] stays local; may be NULL)
 *   x_ranks : HOST array of P device pointers, rank j's shard; only this
 *             rank's head columns are written
 *   rank    : this rank, 0 <= rank < P <= ULYS_MAX_RANKS
 *   dtype   : ULYS_BF16 only (ULYS_ERR_UNSUPPORTED otherwise)
 * Same values, bit for bit, as ulys_attn_fwd_ws with the same workspace
 * followed by ulys_head2seq_push.  Errors: as ulys_attn_fwd_ws and
 * ulys_head2seq_push (a written range of a destination overlapping q, k, v,
 * lse, the workspace or another destination's is ULYS_ERR_ALIAS).
 */
int ulys_attn_fwd_push(const void* q, const void* k, const void* v, void* const* x_ranks,
                       int32_t rank, float* lse, int64_t s, int64_t b, int64_t h, int64_t h_kv,
                       int64_t d_h, int32_t P, int32_t causal, int32_t dtype, void* workspace,
                       int64_t workspace_bytes, void* stream);

/*
 * Attention backward with the gradients' head->seq exchange fused into its
 * epilogues: the result of ulys_attn_bwd followed by ulys_head2seq_push of
 * dQ (h heads) and of dK, dV (h_kv heads), without the dq, dk, dv tensors
 * in between.  [ATLAS] §5: the exchanges' backward is the same all-to-all
 * with its axes swapped, so the gradient of a share goes back by sequence
 * segment and the receiver concatenates along heads ([ATLAS] §2).
 *
 *   q, k, v, o, dout, lse, s, b, h, h_kv, d_h, P, causal, workspace: as
 *             ulys_attn_bwd
 *   dq_ranks, dk_ranks, dv_ranks : HOST arrays of P device pointers; rank
 *             j's shards [s/P, b, h, d_h] (dQ) and [s/P, b, h_kv, d_h] (dK,
 *             dV); only this rank's head columns are written
 *   rank    : this rank, 0 <= rank < P <= ULYS_MAX_RANKS
 *   dtype   : ULYS_BF16 only (ULYS_ERR_UNSUPPORTED otherwise)
 * Same values, bit for bit, as the separate calls.  Errors: as
 * ulys_attn_bwd and ulys_head2seq_push; ULYS_ERR_UNSUPPORTED when the KV
 * heads would be replicated (h_kv < P: the copies' gradients have to be
 * summed, which ulys_unpack_head2seq_kv does after the exchange).
 */
int ulys_attn_bwd_push(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* const* dq_ranks,
                       void* const* dk_ranks, void* const* dv_ranks, int32_t rank, int64_t s,
                       int64_t b, int64_t h, int64_t h_kv, int64_t d_h, int32_t P, int32_t causal,
                       int32_t dtype, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Merge of two partial attention results of one share over disjoint key sets.
 * [SPCP] (Ring section): each query row's online-softmax state -- running
 * max, scaled sum, scaled weighted sum of values -- is brought to a common max
 * and added when a block from another key range arrives; a finished partial
 * result carries that state as its log-sum-exp and normalised output, so
 *   lse = ln(e^lse_a + e^lse_b),  O = e^(lse_a - lse) O_a + e^(lse_b - lse) O_b
 * per query row.  This combines a rank's Ulysses share with key blocks that
 * arrive around a ring: [ATLAS] §4 (all-to-all inside a node, ring across
 * nodes) and [SPCP] (USP: Ulysses groups whose same-head ranks exchange K/V).
 * Partials come from ulys_attn_fwd with lse (dense for a key block wholly
 * before the queries, causal for the block that holds them).
 *
 *   o_a, o_b, o       : [s, b, hp, d_h]  (dtype; hp = query heads of the share)
 *   lse_a, lse_b, lse : [b, hp, s] fp32, natural log; -inf marks an empty
 *                       partial, which contributes nothing (both empty: O = 0,
 *                       lse = -inf)
 * o may be o_a and lse may be lse_a (in-place accumulation); every other
 * overlap is ULYS_ERR_ALIAS.  Arithmetic in fp32, O rounded once
 * (nearest-even).  Supported: F32 and BF16 with d_h in {64, 128}.
 * Errors: NULL pointers, sizes <= 0, unsupported dtype or d_h, misaligned
 * buffers, overlaps other than the in-place pair.
 */
int ulys_attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                    void* o, float* lse, int64_t s, int64_t b, int64_t hp, int64_t d_h,
                    int32_t dtype, void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* ulys_status_string(int status);

/* ABI version of this header: (major << 16) | minor. */
int ulys_abi_version(void);

#define ULYS_ABI_VERSION ((1 << 16) | 12)

#ifdef __cplusplus
}
#endif

#endif /* ULYSSES_H_ */
