// attn_bwd_bf16.hip -- backward of the head-sharded attention on gfx950.
//
// What it computes: the gradients dq, dk, dv of one rank's share of
// softmax(Q K^T / sqrt(d_h)) V given the output gradient dout, the forward
// output o and its log-sum-exp ("02 · DeepSpeed-Ulysses", §5: the exchanges'
// backward is the same all-to-all with its axes swapped, so the layout
// kernels serve it unchanged, and the local attention's backward is the
// ordinary attention backward).  With P = exp(S - lse) (S the scaled
// scores), dP = dout V^T and D = rowsum(dout * o):
//   dS = P * (dP - D),  dq = dS K / sqrt(d_h),  dk = dS^T Q / sqrt(d_h),
//   dv = P^T dout,
// dk and dv summed over the query heads of each GQA group (contiguous
// groups, as in the forward).
//
// Kernels.  No gradient is accumulated with atomics: every output element is
// summed by one workgroup in a fixed order, so the result does not depend on
// scheduling.  The one atomic is the dq kernel's unit counter on long shares
// (each workgroup takes the index of its query block from it; the block is
// computed by the same code wherever it runs):
//  * prep: -D and -lse * sqrt(d_h) per query row, into the caller's
//    workspace (both kernels start their dP accumulators from -D, so that
//    dP - D comes out of the MFMA, and the dkv kernel its S accumulators
//    from -lse * sqrt(d_h), so that exp2(c S) is P);
//  * dq: a workgroup of 8 waves owns 256 queries (as the forward: up to 8
//    query heads of one KV group), streaming 64-key K/V tiles through LDS:
//    S^T = K Q^T and dP^T = V dout^T with the wave's Q^T and dout^T
//    fragments in registers (dP^T accumulated from -D, so it ends as
//    dP^T - D), dS^T = P^T (dP^T - D), dq^T += K^T dS^T with K^T read
//    transposed from LDS;
//  * dkv: a workgroup of 8 waves owns 256 keys of one KV head (32 per wave,
//    K^T and V^T fragments in registers for the whole loop), streaming
//    64-query tiles of Q, dout and their statistics through LDS for every
//    query head of the group: S = Q K^T, dP = dout V^T, then dv^T += dout^T P
//    and dk^T += Q^T dS with dout^T and Q^T read transposed.  S comes first,
//    so that its exponentials run beside the dP products, and dV, which needs
//    only P, beside dS;
//  * merge (dq, dkv): when a causal share has too few work items to fill the
//    GPU twice, every item is run as two halves (keys for dq, queries for
//    dkv) that leave fp32 partial sums in the workspace, and a merge adds the
//    two halves in a fixed order, scales and rounds.
// S and dP are computed by both kernels.  The dq kernel has a branch-free
// fast path for tiles with no masked entry and a masked path for diagonal and
// tail tiles; the dkv kernel masks by starting the masked entries' S and dP
// accumulators at -inf and 0, so every tile then runs the same code.
//
// Every tile read both row-wise (16-byte MFMA operand reads of 16
// consecutive rows) and transposed (ds_read_b64_tr_b16 over 4 consecutive
// rows x 64 bytes) stores chunk c of row r at c ^ g(r) with
// g(4a + i) = (0, 4, 10, 14)[i] ^ a (r mod 16): both patterns are then free
// of bank conflicts on the 64-bank LDS.
#include <math.h>

#include <type_traits>

#include "cdna4.h"
#include "internal.h"

namespace ulys {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxPushRanks = 64;  // destinations of the pushing epilogues
constexpr int kBN = 64;            // dq: keys per tile
constexpr int kKB = 32 * kWaves;   // dkv: keys per workgroup
constexpr int kQT = 64;            // dkv: queries per step
constexpr int kStatBuf = 2048;     // dkv: nlse (first 256 bytes of 1 KiB) then ndelta

// Sizes that follow from the head size D (64 or 128).
template <int D>
struct Geo {
  static constexpr int ROW = D * 2;        // bytes of one bf16 row
  static constexpr int CHUNKS = ROW / 16;  // 16-byte chunks per row
  static constexpr int RPL = 64 / CHUNKS;  // rows filled by one 64-lane 16-byte load
  // dq
  static constexpr int kTile = kBN * ROW;                         // one K or V tile
  static constexpr int kQLoads = kBN * CHUNKS / (64 * kWaves);    // loads per lane per tensor
  static constexpr int kDqPart = kWaves * 64 * (D / 2);           // floats of one split unit
  // dkv
  static constexpr int kQTile = kQT * ROW;                        // one Q or dout tile
  static constexpr int kKLoads = kQT * CHUNKS / (64 * kWaves);    // loads per lane per tensor
  static constexpr int kDkvPart = kWaves * 64 * D;                // floats of one split unit
  static constexpr int kDkvLds = 4 * kQTile + 2 * kStatBuf;
};

// Chunk swizzle g(r) of row r (the tile layout above).
template <int D>
__device__ __forceinline__ int dswz(int r) {
  const int i = r & 3;
  if constexpr (D == 128)
    return ((4 * i) ^ ((i >> 1) << 1)) ^ ((r >> 2) & 3);
  else
    return (4 * (i >> 1)) ^ ((r >> 2) & 3);
}

// ------------------------------------------------------------------ prep
// D / 8 lanes per query row (8 bf16 each); rows enumerated in memory order
// r = (t * b + be) * hp + i of the [s, b, hp, d] tensors.  Writes
// ndelta = -D and nlse = -lse * sqrt(d_h): with c = log2(e) / sqrt(d_h),
// P = exp2(c (q.k + nlse)).
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ o,
                                                       const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ ndelta,
                                                       float* __restrict__ nlse, int rows,
                                                       int s, int s_pad, int bhp, float sqrt_d,
                                                       unsigned* q_tickets) {
  constexpr int LPR = D / 8, SH = (D == 128) ? 4 : 3;  // lanes per row, log2
  static_assert(LPR == 1 << SH, "head size");
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int r = gid >> SH, part = gid & (LPR - 1);
  if (q_tickets && gid == 0) __builtin_nontemporal_store(0u, q_tickets);  // for the dq kernel
  float acc = 0.f;
  if (r < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + (int64_t)r * D + part * 8);
    const u32x4 g = *reinterpret_cast<const u32x4*>(dout + (int64_t)r * D + part * 8);
    const bf16x8 av = as_bf16x8(a), gv = as_bf16x8(g);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)av[e], (float)gv[e], acc);
  }
#pragma unroll
  for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, LPR);
  if (r < rows && part == 0) {
    const int t = r / bhp, rem = r - t * bhp;  // rem = be * hp + i
    ndelta[(int64_t)rem * s_pad + t] = -acc;
    nlse[(int64_t)rem * s_pad + t] = -lse[(int64_t)rem * s + t] * sqrt_d;
  }
}

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* ndelta;  // [b, hp, s_pad], -D
  const float* nlse;    // [b, hp, s_pad], -lse * sqrt(d_h)
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* part;         // partial sums of split units (fp32), when a split is used
  int s, b, hp, hkvp, G;
  int s_pad;  // row length of ndelta and nlse: s rounded up to 4 (16-byte rows)
  int q_tok_bytes, kv_tok_bytes, q_bytes, kv_bytes, stat_bytes;
  float c;       // log2(e) / sqrt(d_h)
  float inv_sd;  // 1 / sqrt(d_h)
  // dq kernel: items = n_qblk * b * hkvp * nsub (as the forward)
  int QH, QB, n_qblk, nsub;
  int q_split;   // 1: every dq item runs as two halves of its key tiles
  // dkv kernel: items = n_kblk * b * hkvp
  int n_kblk;
  int kv_split;  // 1: every dkv item runs as two halves of its query steps
  int kv_units;  // dkv work units: items << kv_split
  int kv_xcd;    // 1: dkv units dispatched in the XCD-aware order (see xcd_unit)
  int rev_q, rev_kv;  // dq / dkv workgroups below these run first_round_slot
  unsigned* q_tickets;  // non-null: dq workgroups take their units from this counter
  // push (non-zero): the gradient rows go to the shards of the head->seq
  // exchange instead of to dq, dk, dv (see store_t_push)
  int push, sl;
  int q_ptok, q_pbe, q_phead, q_pbytes;      // dQ shards [s/P, b, h, d]
  int kv_ptok, kv_pbe, kv_phead, kv_pbytes;  // dK, dV shards [s/P, b, h_kv, d]
  uint16_t* dq_rank[kMaxPushRanks];
  uint16_t* dk_rank[kMaxPushRanks];
  uint16_t* dv_rank[kMaxPushRanks];
};

// XCD-aware order of the dkv units.  The dispatcher sends workgroup b to XCD
// b % 8 (each XCD has its own L2) and each XCD starts its workgroups in order
// of b.  Causal dkv units are ranked longest first and neighbouring units read
// nearly the same query tiles at nearly the same time, but the round-robin
// spreads neighbours over all eight L2s.  Here the ranked list is cut into 16
// equal chunks and XCD x runs chunk x, then chunk 15 - x: the units it runs
// together are neighbours (their Q / dout tiles are shared in its L2), and a
// long chunk paired with the mirrored short one gives every XCD the same
// amount of work under the linear causal profile.  Needs N % 16 == 0.
__device__ __forceinline__ int xcd_unit(int b, int n) {
  const int c = n >> 4, x = b & 7, j = b >> 3;
  return j < c ? x * c + j : (15 - x) * c + (j - c);
}

// Slot of workgroup b in the ranked order.  Within an XCD the dispatcher hands
// workgroups, in order, to its four shader engines in a fixed rotation, each
// waiting for a free CU in its own engine.  In the first round (one workgroup
// per CU) a run of four consecutive workgroups of an XCD holds units ranked
// longest first, which free their CUs in the reverse of the rotation, so every
// second-round workgroup would wait for the last of the four.  Reversing each
// run (32 consecutive workgroups: 4 per XCD, the XCD b % 8 unchanged) in the
// first round frees the CUs in rotation order.
__device__ __forceinline__ int first_round_slot(int b, int rev) {
  if (b >= rev) return b;
  const int r = b & 31;
  return (b & ~31) | ((3 - (r >> 3)) << 3) | (r & 7);
}

// Transposed 32 x 32 accumulator (rows = features, column = lane % 32) scaled
// and rounded once to bf16, stored at row `col` of a [tokens, heads, d] tensor
// with token stride tok_bytes and head offset head_off (bytes).
template <int D>
__device__ __forceinline__ void store_t(__amdgpu_buffer_rsrc_t r, const f32x16* acc, float scale,
                                        int col, int tok_bytes, int head_off, int hh) {
  const int off = col * tok_bytes + head_off + hh * 8;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const __bf16 x0 = (__bf16)(acc[db][4 * g4 + 0] * scale);
      const __bf16 x1 = (__bf16)(acc[db][4 * g4 + 1] * scale);
      const __bf16 x2 = (__bf16)(acc[db][4 * g4 + 2] * scale);
      const __bf16 x3 = (__bf16)(acc[db][4 * g4 + 3] * scale);
      const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, x0) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16);
      const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, x2) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, x3) << 16);
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, r, off + (db * 32 + 8 * g4) * 2, 0,
                                            0);
    }
}

// store_t's rows pushed to their place after the head->seq exchange
// ("02 · DeepSpeed-Ulysses" §2, §5: the gradients go back by sequence
// segment and the receiver concatenates along heads): row `row` of the share
// goes to shard table[row / sl] at token row % sl, `col_off` bytes into the
// token (batch, this rank's head columns, the head).  A wave's 32 rows may
// span several segments; it takes them one uniform segment at a time, so
// every destination pointer is a scalar load.
template <int D>
__device__ __forceinline__ void store_t_push(uint16_t* const* table, int dst_bytes,
                                             const f32x16* acc, float scale, int row, int s,
                                             int sl, int tok_bytes, int col_off, int hh) {
  u32x2 w[D / 32][4];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const __bf16 x0 = (__bf16)(acc[db][4 * g4 + 0] * scale);
      const __bf16 x1 = (__bf16)(acc[db][4 * g4 + 1] * scale);
      const __bf16 x2 = (__bf16)(acc[db][4 * g4 + 2] * scale);
      const __bf16 x3 = (__bf16)(acc[db][4 * g4 + 3] * scale);
      w[db][g4] = u32x2{(uint32_t)__builtin_bit_cast(uint16_t, x0) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16),
                        (uint32_t)__builtin_bit_cast(uint16_t, x2) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, x3) << 16)};
    }
  const int j = (row < s) ? row / sl : -1;
  uint64_t todo = __ballot(j >= 0);
  while (todo) {
    const int jj = __builtin_amdgcn_readlane(j, (int)__builtin_ctzll(todo));
    const bool mine = j == jj;
    todo &= ~__ballot(mine);
    if (mine) {
      const __amdgpu_buffer_rsrc_t r = rsrc(table[jj], dst_bytes);
      const int off = (row - jj * sl) * tok_bytes + col_off + hh * 8;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          __builtin_amdgcn_raw_buffer_store_b64(w[db][g4], r, off + (db * 32 + 8 * g4) * 2, 0, 0);
    }
  }
}
// The three outputs' stores: to dq / dk / dv, or pushed (PUSH, a separate
// instantiation of every kernel, so the plain kernels compile as if the
// pushing epilogue did not exist)
template <int D, bool PUSH>
__device__ __forceinline__ void store_dq(const BwdParams& p, const f32x16* acc, int row, int be,
                                         int head, int hh) {
  constexpr int ROW = Geo<D>::ROW;
  if constexpr (PUSH)
    store_t_push<D>(p.dq_rank, p.q_pbytes, acc, p.inv_sd, row, p.s, p.sl, p.q_ptok,
                 be * p.q_pbe + p.q_phead + head * ROW, hh);
  else
    store_t<D>(rsrc(p.dq, p.q_bytes), acc, p.inv_sd, row, p.q_tok_bytes, (be * p.hp + head) * ROW,
            hh);
}
template <int D, bool PUSH>
__device__ __forceinline__ void store_dkv(const BwdParams& p, const f32x16* acc, bool is_dk,
                                          int row, int be, int kvg, int hh) {
  constexpr int ROW = Geo<D>::ROW;
  const float scale = is_dk ? p.inv_sd : 1.f;
  if constexpr (PUSH)
    store_t_push<D>(is_dk ? p.dk_rank : p.dv_rank, p.kv_pbytes, acc, scale, row, p.s, p.sl,
                 p.kv_ptok, be * p.kv_pbe + p.kv_phead + kvg * ROW, hh);
  else
    store_t<D>(rsrc(is_dk ? p.dk : p.dv, p.kv_bytes), acc, scale, row, p.kv_tok_bytes,
            (be * p.hkvp + kvg) * ROW, hh);
}

// Partial sums of a split unit: n accumulator blocks per lane, stored lane
// contiguous ([wave][slot][lane]) so both writes and reads coalesce.
template <int N>
__device__ __forceinline__ void store_part(float* unit_base, const f32x16* acc, int wave,
                                           int lane) {
  float* dst = unit_base + wave * (N * 16 * 64) + lane;
#pragma unroll
  for (int n = 0; n < N; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[(n * 16 + r) * 64] = acc[n][r];
}
template <int N>
__device__ __forceinline__ void add_parts(const float* u0, const float* u1, f32x16* acc, int wave,
                                          int lane) {
  const float* a = u0 + wave * (N * 16 * 64) + lane;
  const float* b = u1 + wave * (N * 16 * 64) + lane;
#pragma unroll
  for (int n = 0; n < N; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = a[(n * 16 + r) * 64] + b[(n * 16 + r) * 64];
}

// Lane parts of the LDS addresses into a swizzled tile of ROW-byte rows.
//  row reads (A operand of 32 rows x 16 features): row l%32 of a 32-row
//  block, logical chunk 2 dk + hh;
//  transposed reads (A operand of 32 features x 16 rows), feature block db,
//  16-row step: rows 4 hh + (l%16)/4 (lo) and + 8 (hi), byte column
//  64 db + 32 ((l/16)%2) + 8 (l%4).  Row offsets that are multiples of 16
//  leave the swizzle unchanged.
//  Since 2 dk has bit 0 clear, (2 dk + hh) ^ g = 2 (dk ^ (g >> 1)) + ((hh ^ g) & 1),
//  so the row read of step dk is at row_base ^ (32 dk): one register (the
//  XOR stays below bit 8 for D = 128 and below bit 7 for D = 64, where g < 8).
template <int D>
struct TileAddr {
  int row_base;
  int tr_lo[D / 32], tr_hi[D / 32];
  __device__ __forceinline__ int row_rd(int dk) const { return row_base ^ (dk << 5); }
};
template <int D>
__device__ __forceinline__ TileAddr<D> tile_addr(int lane) {
  constexpr int ROW = Geo<D>::ROW;
  TileAddr<D> a;
  const int l32 = lane & 31, hh = lane >> 5;
  a.row_base = l32 * ROW + ((hh ^ dswz<D>(l32)) << 4);
  const int vr = 4 * hh + ((lane & 15) >> 2);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int c = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    a.tr_lo[db] = vr * ROW + ((c ^ dswz<D>(vr)) << 4) + 8 * (lane & 1);
    a.tr_hi[db] = (vr + 8) * ROW + ((c ^ dswz<D>(vr + 8)) << 4) + 8 * (lane & 1);
  }
  return a;
}

// A operand of a transposed read at 16-row step base `tile + 16 ks * ROW`.
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const uint8_t* tile, const TileAddr<D>& a, int ks,
                                          int db) {
  constexpr int ROW = Geo<D>::ROW;
  const u32x2 lo = lds_read_tr(reinterpret_cast<const uint16_t*>(tile + ks * 16 * ROW + a.tr_lo[db]));
  const u32x2 hi = lds_read_tr(reinterpret_cast<const uint16_t*>(tile + ks * 16 * ROW + a.tr_hi[db]));
  return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// ------------------------------------------------------------------ dq
struct QItem {
  int qblk, be, kvg, head, q0;
};
__device__ __forceinline__ QItem decode_q_item(const BwdParams& p, int rank, int wave, bool causal) {
  QItem it;
  const int per_q = p.b * p.hkvp * p.nsub;
  const int qi = rank / per_q;
  int rest = rank - qi * per_q;
  it.qblk = causal ? (p.n_qblk - 1 - qi) : qi;  // longest first
  const int sub = rest % p.nsub;
  rest /= p.nsub;
  it.kvg = rest % p.hkvp;
  it.be = rest / p.hkvp;
  const int wph = kWaves / p.QH;
  it.head = it.kvg * p.G + sub * p.QH + wave / wph;
  it.q0 = it.qblk * p.QB + (wave % wph) * 32;
  return it;
}

template <int D, bool CAUSAL, bool PUSH>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdParams p) {
  constexpr int ROW = Geo<D>::ROW, CHUNKS = Geo<D>::CHUNKS, RPL = Geo<D>::RPL;
  constexpr int kTile = Geo<D>::kTile, kQLoads = Geo<D>::kQLoads;
  // LDS: K0 K1 V0 V1
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kTile];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l32 = lane & 31, hh = lane >> 5;
  int unit;
  if (p.q_tickets) {
    // the next unit in ranked order, whichever XCD this workgroup runs on;
    // broadcast through K buffer 1, which the first step's loads write only
    // after the prologue's barrier
    int* slot = reinterpret_cast<int*>(lds + kTile);
    if (threadIdx.x == 0)
      *slot = (int)__hip_atomic_fetch_add(p.q_tickets, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    unit = __builtin_amdgcn_readfirstlane(*slot);
  } else {
    unit = first_round_slot(blockIdx.x, p.rev_q);
  }
  int rank = unit, half = 0;
  if (p.q_split) {
    half = rank & 1;
    rank >>= 1;
  }
  const QItem it = decode_q_item(p, rank, wave, CAUSAL);
  const int my_q = it.q0 + l32;
  const __amdgpu_buffer_rsrc_t rq = rsrc(p.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rdo = rsrc(p.dout, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(p.v, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t rst = rsrc(p.nlse, p.stat_bytes);
  const __amdgpu_buffer_rsrc_t rde = rsrc(p.ndelta, p.stat_bytes);
  const int q_head_off = (it.be * p.hp + it.head) * ROW;
  const int kv_head_off = (it.be * p.hkvp + it.kvg) * ROW;

  // Q^T and dout^T fragments (B operands): query my_q, features 16 dk + 8 hh .. +7
  bf16x8 qf[D / 16], gf[D / 16];
  {
    const int off = my_q * p.q_tok_bytes + q_head_off + hh * 16;
#pragma unroll
    for (int dk = 0; dk < D / 16; ++dk) {
      qf[dk] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rq, off + dk * 32, 0, 0));
      gf[dk] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rdo, off + dk * 32, 0, 0));
    }
  }
  // statistics of query my_q (rows past s read whatever lies there: their
  // results are never stored)
  const int stat = (it.be * p.hp + it.head) * p.s_pad + my_q;
  const float clse = p.c * __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rst, stat * 4, 0, 0));
  const float ndlt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rde, stat * 4, 0, 0));
  // complete these loads before the loop, so that no wait in the loop is on
  // anything but the tile loads
#pragma unroll
  for (int dk = 0; dk < D / 16; ++dk) asm volatile("" ::"v"(qf[dk]), "v"(gf[dk]));
  asm volatile("" ::"v"(clse), "v"(ndlt));

  const int q_hi = min(p.s, (it.qblk + 1) * p.QB);
  const int n_item = CAUSAL ? (q_hi + kBN - 1) / kBN : (p.s + kBN - 1) / kBN;
  const int t_mid = (n_item + 1) >> 1;
  const int t_lo = (p.q_split && half == 1) ? t_mid : 0;
  const int t_hi = (p.q_split && half == 0) ? t_mid : n_item;
  const int wave_last_q = min(it.q0 + 32, p.s) - 1;
  const int wave_tiles = (it.q0 >= p.s) ? 0 : (CAUSAL ? wave_last_q / kBN + 1 : n_item);

  // direct loads: wave w, load i fills rows (w*kQLoads + i)*RPL .. +RPL-1 of a tile
  int src[kQLoads];
#pragma unroll
  for (int i = 0; i < kQLoads; ++i) {
    const int row = (wave * kQLoads + i) * RPL + lane / CHUNKS;
    src[i] = row * p.kv_tok_bytes + kv_head_off + (((lane % CHUNKS) ^ dswz<D>(row)) << 4);
  }
  auto load_tile = [&](int t, int buf) {
    const int koff = t * kBN * p.kv_tok_bytes;
#pragma unroll
    for (int i = 0; i < kQLoads; ++i) {
      const int dst = (wave * kQLoads + i) * 1024;
      load_lds16(rk, lds + buf * kTile + dst, src[i] + koff);
      load_lds16(rv, lds + (2 + buf) * kTile + dst, src[i] + koff);
    }
  };
  const TileAddr<D> ta = tile_addr<D>(lane);

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  if (t_lo < t_hi) load_tile(t_lo, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // one key tile t in buffer CUR
  auto dq_step = [&](int t, auto cur_tag) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_tag)::value;
    if (t + 1 < t_hi) load_tile(t + 1, cur ^ 1);
    if (t < wave_tiles) {
      const uint8_t* kl = lds + cur * kTile;
      const uint8_t* vl = lds + (2 + cur) * kTile;
      const int k0 = t * kBN;
      // the tile's two 32-key halves in turn.
      // S^T and dP^T of half kb: keys k0 + 32 kb + (8 (r/4) + 4 hh + r%4),
      // query my_q
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint8_t* kh = kl + kb * 32 * ROW;
        // dP^T starts from -D (this lane's query), so it ends as dP - D
        f32x16 sc, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[r] = 0.f;
          dp[r] = ndlt;
        }
#pragma unroll
        for (int dk = 0; dk < D / 16; ++dk) {
          const bf16x8 ka = *(const bf16x8*)(kh + ta.row_rd(dk));
          const bf16x8 va = *(const bf16x8*)(vl + kb * 32 * ROW + ta.row_rd(dk));
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[dk], sc, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gf[dk], dp, 0, 0, 0);
        }
        const int kh0 = k0 + 32 * kb;
        const bool need_mask = (kh0 + 32 > p.s) || (CAUSAL && kh0 + 31 > it.q0);
        if (!need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pr = __builtin_amdgcn_exp2f(fmaf(sc[r], p.c, clse));
            sc[r] = pr * dp[r];
          }
        } else {
          // masked entries are set to zero, not multiplied by it
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pr = __builtin_amdgcn_exp2f(fmaf(sc[r], p.c, clse));
            const int key = kh0 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const float ds = pr * dp[r];
            sc[r] = (key >= p.s || (CAUSAL && key > my_q)) ? 0.f : ds;
          }
        }
        bf16x8 dsb[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) dsb[ks][e] = (__bf16)sc[ks * 8 + e];
        // dq^T += K^T dS^T, K^T read transposed from the K tile
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(kh, ta, ks, db), dsb[ks],
                                                              acc[db], 0, 0, 0);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  // unrolled by two so every buffer index is a compile-time constant
  for (int t = t_lo; t < t_hi; t += 2) {
    dq_step(t, std::integral_constant<int, 0>{});
    if (t + 1 < t_hi) dq_step(t + 1, std::integral_constant<int, 1>{});
  }
  if (p.q_split) {
    store_part<D / 32>(p.part + (int64_t)unit * Geo<D>::kDqPart, acc, wave, lane);
    return;
  }
  store_dq<D, PUSH>(p, acc, my_q, it.be, it.head, hh);
}

// The two halves of every dq item: added in a fixed order, scaled, rounded.
template <int D, bool CAUSAL, bool PUSH>
__global__ __launch_bounds__(kThreads) void bwd_dq_merge_kernel(BwdParams p) {
  constexpr int kDqPart = Geo<D>::kDqPart;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const QItem it = decode_q_item(p, blockIdx.x, wave, CAUSAL);
  const float* u0 = p.part + (int64_t)(2 * blockIdx.x) * kDqPart;
  f32x16 acc[D / 32];
  add_parts<D / 32>(u0, u0 + kDqPart, acc, wave, lane);
  store_dq<D, PUSH>(p, acc, it.q0 + l32, it.be, it.head, hh);
}

// ------------------------------------------------------------------ dk, dv
struct KItem {
  int kblk, be, kvg;
};
__device__ __forceinline__ KItem decode_k_item(const BwdParams& p, int rank) {
  // key block (lowest first when causal: the longest), then batch, KV head
  KItem it;
  const int per_k = p.b * p.hkvp;
  it.kblk = rank / per_k;
  it.kvg = (rank - it.kblk * per_k) % p.hkvp;
  it.be = (rank - it.kblk * per_k) / p.hkvp;
  return it;
}

template <int D, bool CAUSAL, bool PUSH>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkv_kernel(BwdParams p) {
  constexpr int ROW = Geo<D>::ROW, CHUNKS = Geo<D>::CHUNKS, RPL = Geo<D>::RPL;
  constexpr int kQTile = Geo<D>::kQTile;
  constexpr int kKLoads = Geo<D>::kKLoads;
  constexpr int kDkvPart = Geo<D>::kDkvPart;
  // LDS: Q0 Q1 | dout0 dout1 | stats0 stats1.  The tiles first:
  // with the buffer and half indices compile-time constants, every tile read
  // is one lane register plus an offset that fits the instruction's 16 bits.
  __shared__ __attribute__((aligned(16))) uint8_t lds[Geo<D>::kDkvLds];
  uint8_t* qt = lds;
  uint8_t* gt = qt + 2 * kQTile;
  uint8_t* stt = gt + 2 * kQTile;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l32 = lane & 31, hh = lane >> 5;
  const int slot = first_round_slot(blockIdx.x, p.rev_kv);
  const int unit = p.kv_xcd ? xcd_unit(slot, p.kv_units) : slot;
  int rank = unit, half = 0;
  if (p.kv_split) {
    half = rank & 1;
    rank >>= 1;
  }
  const KItem it = decode_k_item(p, rank);
  const int kw0 = it.kblk * kKB + wave * 32;  // this wave's first key
  const int my_key = kw0 + l32;

  const __amdgpu_buffer_rsrc_t rq = rsrc(p.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rdo = rsrc(p.dout, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(p.v, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t rst = rsrc(p.nlse, p.stat_bytes);
  const __amdgpu_buffer_rsrc_t rde = rsrc(p.ndelta, p.stat_bytes);
  const int kv_head_off = (it.be * p.hkvp + it.kvg) * ROW;

  // K^T and V^T fragments (B operands of S = Q K^T and dP = dout V^T): key
  // my_key, features 16 dk + 8 hh .. +7
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const int off = my_key * p.kv_tok_bytes + kv_head_off + hh * 16;
#pragma unroll
    for (int dk = 0; dk < D / 16; ++dk) {
      kf[dk] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rk, off + dk * 32, 0, 0));
      vf[dk] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rv, off + dk * 32, 0, 0));
    }
  }
#pragma unroll
  for (int dk = 0; dk < D / 16; ++dk) asm volatile("" ::"v"(kf[dk]), "v"(vf[dk]));

  // steps: (query head of the group, 64-query tile); causal tiles start at
  // the workgroup's first key
  const int t_first = CAUSAL ? (it.kblk * kKB) / kQT : 0;
  const int n_qt = (p.s + kQT - 1) / kQT;
  const int per_head = n_qt - t_first;
  const int n_steps = (it.kblk * kKB < p.s) ? p.G * per_head : 0;
  const int st_mid = (n_steps + 1) >> 1;
  const int st_lo = (p.kv_split && half == 1) ? st_mid : 0;
  const int st_hi = (p.kv_split && half == 0) ? st_mid : n_steps;

  int src[kKLoads];
#pragma unroll
  for (int i = 0; i < kKLoads; ++i) {
    const int row = (wave * kKLoads + i) * RPL + lane / CHUNKS;
    src[i] = row * p.q_tok_bytes + (((lane % CHUNKS) ^ dswz<D>(row)) << 4);
  }
  // statistics: lanes 0..15 of waves 0 (nlse) and 1 (ndelta) fetch the 64
  // rows of the step, 16 bytes each; the other lanes read past the
  // resource, which lands zeros in the rest of the 1 KiB slot
  const __amdgpu_buffer_rsrc_t rstat = (wave == 0) ? rst : rde;
  const int stat_lane = (lane < 16) ? lane * 16 : p.stat_bytes;
  auto step_head = [&](int st) { return it.kvg * p.G + st / per_head; };
  auto step_q0 = [&](int st) { return (t_first + st % per_head) * kQT; };
  auto load_step = [&](int st, int buf) {
    const int head = step_head(st), q0 = step_q0(st);
    const int off = q0 * p.q_tok_bytes + (it.be * p.hp + head) * ROW;
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int dst = (wave * kKLoads + i) * 1024;
      load_lds16(rq, qt + buf * kQTile + dst, src[i] + off);
      load_lds16(rdo, gt + buf * kQTile + dst, src[i] + off);
    }
    if (wave < 2) {
      const int soff = (lane < 16) ? ((it.be * p.hp + head) * p.s_pad + q0) * 4 + stat_lane
                                   : stat_lane;
      load_lds16(rstat, stt + buf * kStatBuf + wave * 1024, soff);
    }
  };
  const TileAddr<D> ta = tile_addr<D>(lane);

  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[db][r] = dva[db][r] = 0.f;

  if (st_lo < st_hi) load_step(st_lo, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // one step: query tile st in buffer CUR, its two 32-query halves
  auto dkv_step = [&](int st, auto cur_tag) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_tag)::value;
    if (st + 1 < st_hi) load_step(st + 1, cur ^ 1);
    const int q0 = step_q0(st);
#pragma unroll
    for (int hq = 0; hq < kQT / 32; ++hq) {
      const int qr = q0 + 32 * hq;  // first query of this 32-query half
      // the wave's keys all come after these queries (causal), or either
      // side lies past the sequence: nothing to add
      if ((CAUSAL && qr + 31 < kw0) || kw0 >= p.s || qr >= p.s) continue;
      const uint8_t* ql = qt + cur * kQTile + hq * 32 * ROW;
      const uint8_t* gl = gt + cur * kQTile + hq * 32 * ROW;
      const float* sl = reinterpret_cast<const float*>(stt + cur * kStatBuf) + 32 * hq + 4 * hh;
      // S (queries x keys) and dP: rows qr + 8 (r/4) + 4 hh + r%4, column
      // my_key.  The accumulators start from the rows' statistics (broadcast
      // reads), so they end as q.k - lse sqrt(d_h) and dP - D.  Entries
      // above the diagonal or past the sequence start from -inf and 0
      // instead, so that P and dS come out as 0 from the same code as every
      // other entry (statistics of rows past the sequence are not defined,
      // and the Q, dout and K rows past it read as zero).
      const bool need_mask = (CAUSAL && qr < kw0 + 31) || (qr + 32 > p.s) || (kw0 + 32 > p.s);
      f32x16 sc, dp;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(sl + 8 * j);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(sl + 256 + 8 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[4 * j + i] = l4[i];
          dp[4 * j + i] = d4[i];
        }
      }
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qq = qr + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool off = qq >= p.s || my_key >= p.s || (CAUSAL && my_key > qq);
          sc[r] = off ? -INFINITY : sc[r];
          dp[r] = off ? 0.f : dp[r];
        }
      }
      // S first, so that its exponentials run beside the dP products; then
      // dV, which needs only P, beside dS = P (dP - D); then dK
#pragma unroll
      for (int dk = 0; dk < D / 16; ++dk) {
        const bf16x8 qa = *(const bf16x8*)(ql + ta.row_rd(dk));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[dk], sc, 0, 0, 0);
      }
#pragma unroll
      for (int dk = 0; dk < D / 16; ++dk) {
        const bf16x8 ga = *(const bf16x8*)(gl + ta.row_rd(dk));
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[dk], dp, 0, 0, 0);
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = __builtin_amdgcn_exp2f(sc[r] * p.c);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[ks][e] = (__bf16)sc[ks * 8 + e];
      // dv^T += dout^T P (dout^T read transposed)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(gl, ta, ks, db), pb[ks],
                                                            dva[db], 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = sc[r] * dp[r];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) dsb[ks][e] = (__bf16)dp[ks * 8 + e];
      // dk^T += Q^T dS (Q^T read transposed)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(ql, ta, ks, db), dsb[ks],
                                                            dka[db], 0, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  // unrolled by two so every buffer index is a compile-time constant
  for (int st = st_lo; st < st_hi; st += 2) {
    dkv_step(st, std::integral_constant<int, 0>{});
    if (st + 1 < st_hi) dkv_step(st + 1, std::integral_constant<int, 1>{});
  }
  if (p.kv_split) {
    float* base = p.part + (int64_t)unit * kDkvPart;
    store_part<D / 32>(base, dka, wave, lane);
    store_part<D / 32>(base + kDkvPart / 2, dva, wave, lane);
    return;
  }
  store_dkv<D, PUSH>(p, dka, true, my_key, it.be, it.kvg, hh);
  store_dkv<D, PUSH>(p, dva, false, my_key, it.be, it.kvg, hh);
}

// The two halves of every dkv item: added in a fixed order, scaled, rounded.
template <int D, bool PUSH>
__global__ __launch_bounds__(kThreads) void bwd_dkv_merge_kernel(BwdParams p) {
  constexpr int kDkvPart = Geo<D>::kDkvPart;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const KItem it = decode_k_item(p, blockIdx.x);
  const int my_key = it.kblk * kKB + wave * 32 + l32;
  const float* u0 = p.part + (int64_t)(2 * blockIdx.x) * kDkvPart;
  const float* u1 = u0 + kDkvPart;
  f32x16 acc[D / 32];
  add_parts<D / 32>(u0, u1, acc, wave, lane);
  store_dkv<D, PUSH>(p, acc, true, my_key, it.be, it.kvg, hh);
  add_parts<D / 32>(u0 + kDkvPart / 2, u1 + kDkvPart / 2, acc, wave, lane);
  store_dkv<D, PUSH>(p, acc, false, my_key, it.be, it.kvg, hh);
}

// Work layout for one call: statistics, split decisions, partial-sum bytes.
struct BwdPlan {
  int64_t s_pad, stat_floats;  // per statistic: b * hp * s_pad
  int QH, QB, n_qblk, nsub, n_kblk;
  int64_t q_items, k_items;
  int q_split, kv_split;
  int64_t part_offset, part_bytes;  // in the workspace
  int q_tickets;                    // 1: dq units from a counter at ticket_offset
  int64_t ticket_offset;
};

int64_t device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return (int64_t)cus;
}

template <int D>
BwdPlan plan(const AttnBwdArgs& a) {
  BwdPlan pl;
  pl.s_pad = (a.s + 3) / 4 * 4;
  pl.stat_floats = a.b * a.hp * pl.s_pad;
  const int G = (int)(a.hp / a.hkvp);
  pl.QH = (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  pl.QB = 32 * (kWaves / pl.QH);
  pl.n_qblk = (int)((a.s + pl.QB - 1) / pl.QB);
  pl.nsub = G / pl.QH;
  pl.n_kblk = (int)((a.s + kKB - 1) / kKB);
  pl.q_items = (int64_t)pl.n_qblk * a.b * a.hkvp * pl.nsub;
  pl.k_items = (int64_t)pl.n_kblk * a.b * a.hkvp;
  // one 8-wave workgroup per CU: causal work with fewer than two items per
  // CU is split, or the longest item alone would set the run time
  const int64_t cus = device_cus();
  pl.q_split = (a.causal && cus > 0 && pl.q_items < 2 * cus) ? 1 : 0;
  pl.kv_split = (a.causal && cus > 0 && pl.k_items < 2 * cus) ? 1 : 0;
  // the dq partials are consumed by their merge before the dkv kernel runs,
  // so both use the same region
  const int64_t qpart = pl.q_split ? pl.q_items * 2 * Geo<D>::kDqPart * 4 : 0;
  const int64_t kpart = pl.kv_split ? pl.k_items * 2 * Geo<D>::kDkvPart * 4 : 0;
  pl.part_offset = (2 * pl.stat_floats * 4 + 255) / 256 * 256;
  pl.part_bytes = qpart > kpart ? qpart : kpart;
  // dq work of four or more rounds takes its units from a counter (cleared by
  // the prep kernel), so that XCDs running at different clocks share them by
  // speed; the dkv units keep their XCD-aware order, which the L2 needs
  pl.q_tickets = (cus > 0 && pl.q_items >= 4 * cus) ? 1 : 0;
  pl.ticket_offset = pl.part_offset + pl.part_bytes;
  return pl;
}

template <int D, bool CAUSAL, bool PUSH>
void launch_kernels(const BwdParams& p, const BwdPlan& pl, unsigned q_grid, unsigned k_grid,
                    hipStream_t stream) {
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, PUSH>), dim3(q_grid), dim3(kThreads), 0, stream,
                     p);
  if (pl.q_split)
    hipLaunchKernelGGL((bwd_dq_merge_kernel<D, CAUSAL, PUSH>), dim3((unsigned)pl.q_items),
                       dim3(kThreads), 0, stream, p);
  hipLaunchKernelGGL((bwd_dkv_kernel<D, CAUSAL, PUSH>), dim3(k_grid), dim3(kThreads), 0, stream,
                     p);
  if (pl.kv_split)
    hipLaunchKernelGGL((bwd_dkv_merge_kernel<D, PUSH>), dim3((unsigned)pl.k_items),
                       dim3(kThreads), 0, stream, p);
}

template <int D>
hipError_t launch_d(const AttnBwdArgs& a, hipStream_t stream) {
  constexpr int ROW = Geo<D>::ROW;
  const BwdPlan pl = plan<D>(a);
  float* ndelta = static_cast<float*>(a.workspace);
  float* nlse = ndelta + pl.stat_floats;
  unsigned* q_tickets =
      pl.q_tickets ? reinterpret_cast<unsigned*>(static_cast<uint8_t*>(a.workspace) +
                                                 pl.ticket_offset)
                   : nullptr;
  const int64_t rows = a.s * a.b * a.hp;
  if (rows <= 0) return hipSuccess;
  if (pl.q_items > 0x3FFFFFFF || pl.k_items > 0x3FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)((rows * (D / 8) + 255) / 256)),
                     dim3(256), 0, stream, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.lse,
                     ndelta, nlse, (int)rows, (int)a.s, (int)pl.s_pad, (int)(a.b * a.hp),
                     (float)sqrt((double)D), q_tickets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  BwdParams p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.dout = (const uint16_t*)a.dout;
  p.ndelta = ndelta;
  p.nlse = nlse;
  p.dq = (uint16_t*)a.dq;
  p.dk = (uint16_t*)a.dk;
  p.dv = (uint16_t*)a.dv;
  p.part = pl.part_bytes > 0
               ? reinterpret_cast<float*>(static_cast<uint8_t*>(a.workspace) + pl.part_offset)
               : nullptr;
  p.s = (int)a.s;
  p.b = (int)a.b;
  p.hp = (int)a.hp;
  p.hkvp = (int)a.hkvp;
  p.G = (int)(a.hp / a.hkvp);
  p.q_tok_bytes = (int)(a.b * a.hp * ROW);
  p.kv_tok_bytes = (int)(a.b * a.hkvp * ROW);
  p.q_bytes = (int)(a.s * a.b * a.hp * ROW);
  p.kv_bytes = (int)(a.s * a.b * a.hkvp * ROW);
  p.s_pad = (int)pl.s_pad;
  p.stat_bytes = (int)(pl.stat_floats * 4);
  p.c = (float)(1.4426950408889634 / sqrt((double)D));
  p.inv_sd = (float)(1.0 / sqrt((double)D));
  p.push = a.dq_ranks != nullptr;
  p.sl = p.q_ptok = p.q_pbe = p.q_phead = p.q_pbytes = 0;
  p.kv_ptok = p.kv_pbe = p.kv_phead = p.kv_pbytes = 0;
  for (int r = 0; r < kMaxPushRanks; ++r) p.dq_rank[r] = p.dk_rank[r] = p.dv_rank[r] = nullptr;
  if (p.push) {
    if (!a.dk_ranks || !a.dv_ranks || a.ranks <= 0 || a.ranks > kMaxPushRanks || a.rank < 0 ||
        a.rank >= a.ranks || a.s % a.ranks != 0)
      return hipErrorInvalidValue;
    const int64_t h = a.hp * a.ranks, h_kv = a.hkvp * a.ranks;
    p.sl = (int)(a.s / a.ranks);
    p.q_pbe = (int)(h * ROW);
    p.q_ptok = (int)(a.b * h * ROW);
    p.q_phead = (int)(a.rank * a.hp * ROW);
    p.q_pbytes = (int)((int64_t)p.sl * p.q_ptok);
    p.kv_pbe = (int)(h_kv * ROW);
    p.kv_ptok = (int)(a.b * h_kv * ROW);
    p.kv_phead = (int)(a.rank * a.hkvp * ROW);
    p.kv_pbytes = (int)((int64_t)p.sl * p.kv_ptok);
    for (int r = 0; r < a.ranks; ++r) {
      p.dq_rank[r] = static_cast<uint16_t*>(a.dq_ranks[r]);
      p.dk_rank[r] = static_cast<uint16_t*>(a.dk_ranks[r]);
      p.dv_rank[r] = static_cast<uint16_t*>(a.dv_ranks[r]);
    }
  }
  p.QH = pl.QH;
  p.QB = pl.QB;
  p.n_qblk = pl.n_qblk;
  p.nsub = pl.nsub;
  p.n_kblk = pl.n_kblk;
  p.q_split = pl.q_split;
  p.kv_split = pl.kv_split;
  p.kv_units = (int)(pl.k_items << pl.kv_split);
  p.kv_xcd = (a.causal && p.kv_units % 16 == 0) ? 1 : 0;
  const unsigned q_grid = (unsigned)(pl.q_items << pl.q_split);
  const unsigned k_grid = (unsigned)(pl.k_items << pl.kv_split);
  {
    // the first round: one workgroup per CU, whole runs of 32 only
    const int64_t slots = device_cus();
    p.rev_q = (int)(((int64_t)q_grid < slots ? (int64_t)q_grid : slots) & ~int64_t(31));
    p.rev_kv = (int)(((int64_t)k_grid < slots ? (int64_t)k_grid : slots) & ~int64_t(31));
  }
  p.q_tickets = q_tickets;
  if (a.causal && p.push)
    launch_kernels<D, true, true>(p, pl, q_grid, k_grid, stream);
  else if (a.causal)
    launch_kernels<D, true, false>(p, pl, q_grid, k_grid, stream);
  else if (p.push)
    launch_kernels<D, false, true>(p, pl, q_grid, k_grid, stream);
  else
    launch_kernels<D, false, false>(p, pl, q_grid, k_grid, stream);
  return hipGetLastError();
}

int64_t workspace_bytes(const BwdPlan& pl) {
  if (pl.q_tickets) return pl.ticket_offset + 256;
  return pl.part_bytes > 0 ? pl.part_offset + pl.part_bytes : 2 * pl.stat_floats * 4;
}

}  // namespace

int64_t attn_bwd_bf16_workspace_size(const AttnBwdArgs& a) {
  if (a.d == 64) return workspace_bytes(plan<64>(a));
  return workspace_bytes(plan<128>(a));
}

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_d<128>(a, stream);
  if (a.d == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ulys
