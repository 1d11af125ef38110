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
// Three kernels, no atomics (the result does not depend on scheduling):
//  * prep: D and lse * log2(e) per query row, into the caller's workspace;
//  * dq: one workgroup of 8 waves per 256 queries (as the forward), looping
//    over 64-key K/V tiles in LDS: S^T = K Q^T and dP^T = V dout^T with the
//    wave's Q^T and dout^T fragments in registers, dS^T = P^T (dP^T - D),
//    dq^T += K^T dS^T with K^T read transposed from LDS;
//  * dkv: one workgroup of 4 waves per 128 keys of one KV head, each wave
//    owning 32 keys, looping over the group's query heads and 32-query tiles
//    of Q and dout in LDS: S = Q K^T (K^T fragments in registers),
//    dP = dout V^T (V^T from the workgroup's V block in LDS), then
//    dv^T += dout^T P and dk^T += Q^T dS with dout^T and Q^T read transposed.
// S and dP are therefore computed twice (once per kernel).
//
// Every tile read both row-wise (16-byte MFMA operand reads of 16
// consecutive rows) and transposed (ds_read_b64_tr_b16 over 4 consecutive
// rows x 64 bytes) stores chunk c of row r at c ^ g(r) with
// g(4a + i) = (0, 4, 10, 14)[i] ^ a (r mod 16): both patterns are then free
// of bank conflicts on the 64-bank LDS.
#include <math.h>

#include "cdna4.h"
#include "internal.h"

namespace ulys {
namespace {

constexpr int D = 128;               // head size served here
constexpr int ROW = D * 2;           // bytes of one bf16 row
constexpr int CHUNKS = ROW / 16;     // 16-byte chunks per row
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int dswz(int r) {
  const int i = r & 3;
  return ((4 * i) ^ ((i >> 1) << 1)) ^ ((r >> 2) & 3);
}

// ------------------------------------------------------------------ prep
// 16 lanes per query row (8 bf16 each); rows enumerated in memory order
// r = (t * b + be) * hp + i of the [s, b, hp, d] tensors.
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ o,
                                                       const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ delta,
                                                       float* __restrict__ lse2, int rows,
                                                       int s, int s_pad, int bhp) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int r = gid >> 4, part = gid & 15;
  float acc = 0.f;
  if (r < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + (int64_t)r * D + part * 8);
    const u32x4 g = *reinterpret_cast<const u32x4*>(dout + (int64_t)r * D + part * 8);
    const bf16x8 av = as_bf16x8(a), gv = as_bf16x8(g);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)av[e], (float)gv[e], acc);
  }
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, 16);
  if (r < rows && part == 0) {
    const int t = r / bhp, rem = r - t * bhp;  // rem = be * hp + i
    delta[(int64_t)rem * s_pad + t] = acc;
    lse2[(int64_t)rem * s_pad + t] = lse[(int64_t)rem * s + t] * kLog2e;
  }
}

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* delta;  // [b, hp, s_pad]
  const float* lse2;   // [b, hp, s_pad], lse * log2(e)
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int s, b, hp, hkvp, G;
  int s_pad;  // row length of delta and lse2: s rounded up to 4 (16-byte rows)
  int q_tok_bytes, kv_tok_bytes, q_bytes, kv_bytes, stat_bytes;
  float c;       // log2(e) / sqrt(d_h)
  float inv_sd;  // 1 / sqrt(d_h)
  // dq kernel: items = n_qblk * b * hkvp * nsub (as the forward)
  int QH, QB, n_qblk, nsub;
  // dkv kernel: items = n_kblk * b * hkvp; pairing of the first resident wave
  int n_kblk, slots;
};

// Transposed 32 x 32 accumulator (rows = features, column = lane % 32) scaled
// and rounded once to bf16, stored at row `col` of a [tokens, heads, d] tensor
// with token stride tok_bytes and head offset head_off (bytes).
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

// Lane parts of the LDS addresses into a swizzled tile of 256-byte rows.
//  row reads (A operand of 32 rows x 16 features): row l%32 of a 32-row
//  block, logical chunk 2 dk + hh;
//  transposed reads (A operand of 32 features x 16 rows), feature block db,
//  16-row step: rows 4 hh + (l%16)/4 (lo) and + 8 (hi), byte column
//  64 db + 32 ((l/16)%2) + 8 (l%4).  Row offsets that are multiples of 16
//  leave the swizzle unchanged; +8 rows flips bit 1 of g.
struct TileAddr {
  int row_rd[D / 16];
  int tr_lo[D / 32], tr_hi[D / 32];
};
__device__ __forceinline__ TileAddr tile_addr(int lane) {
  TileAddr a;
  const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int dk = 0; dk < D / 16; ++dk) a.row_rd[dk] = l32 * ROW + (((2 * dk + hh) ^ dswz(l32)) << 4);
  const int vr = 4 * hh + ((lane & 15) >> 2);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int c = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    a.tr_lo[db] = vr * ROW + ((c ^ dswz(vr)) << 4) + 8 * (lane & 1);
    a.tr_hi[db] = (vr + 8) * ROW + ((c ^ dswz(vr + 8)) << 4) + 8 * (lane & 1);
  }
  return a;
}

// A operand of a transposed read at 16-row step base `tile + 16 ks * ROW`.
__device__ __forceinline__ bf16x8 read_tr(const uint8_t* tile, const TileAddr& a, int ks, int db) {
  const u32x2 lo = lds_read_tr(reinterpret_cast<const uint16_t*>(tile + ks * 16 * ROW + a.tr_lo[db]));
  const u32x2 hi = lds_read_tr(reinterpret_cast<const uint16_t*>(tile + ks * 16 * ROW + a.tr_hi[db]));
  return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// ------------------------------------------------------------------ dq
constexpr int kQWaves = 8;
constexpr int kQThreads = 64 * kQWaves;
constexpr int kBN = 64;              // keys per tile
constexpr int kTile = kBN * ROW;     // one K or V tile
constexpr int kQLoads = kBN * CHUNKS / (64 * kQWaves);  // 16-byte loads per lane per tensor

struct QItem {
  int qblk, be, kvg, head, q0;
};
__device__ __forceinline__ QItem decode_q_item(const BwdParams& p, int rank, int wave, bool causal) {
  QItem it;
  const int per_q = p.b * p.hkvp * p.nsub;
  const int qi = rank / per_q;
  int rest = rank - qi * per_q;
  it.qblk = causal ? (p.n_qblk - 1 - qi) : qi;
  const int sub = rest % p.nsub;
  rest /= p.nsub;
  it.kvg = rest % p.hkvp;
  it.be = rest / p.hkvp;
  const int wph = kQWaves / p.QH;
  it.head = it.kvg * p.G + sub * p.QH + wave / wph;
  it.q0 = it.qblk * p.QB + (wave % wph) * 32;
  return it;
}

template <bool CAUSAL>
__global__ __launch_bounds__(kQThreads, 1) void bwd_dq_kernel(BwdParams p) {
  // LDS: K0 K1 V0 V1
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kTile];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const QItem it = decode_q_item(p, blockIdx.x, wave, CAUSAL);
  const int my_q = it.q0 + l32;
  const __amdgpu_buffer_rsrc_t rq = rsrc(p.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rdo = rsrc(p.dout, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(p.v, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t rst = rsrc(p.lse2, p.stat_bytes);
  const __amdgpu_buffer_rsrc_t rde = rsrc(p.delta, p.stat_bytes);
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
  const int stat = (it.be * p.hp + it.head) * p.s_pad + my_q;
  const float lse2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rst, stat * 4, 0, 0));
  const float dlt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rde, stat * 4, 0, 0));
#pragma unroll
  for (int dk = 0; dk < D / 16; ++dk) asm volatile("" ::"v"(qf[dk]), "v"(gf[dk]));
  asm volatile("" ::"v"(lse2), "v"(dlt));

  const int q_hi = min(p.s, (it.qblk + 1) * p.QB);
  const int n_tiles = CAUSAL ? (q_hi + kBN - 1) / kBN : (p.s + kBN - 1) / kBN;
  const int wave_last_q = min(it.q0 + 32, p.s) - 1;
  const int wave_tiles = (it.q0 >= p.s) ? 0 : (CAUSAL ? wave_last_q / kBN + 1 : n_tiles);

  // direct loads: wave w, load i fills rows (w*kQLoads + i)*4 .. +3 of a tile
  int src[kQLoads];
#pragma unroll
  for (int i = 0; i < kQLoads; ++i) {
    const int row = (wave * kQLoads + i) * 4 + lane / CHUNKS;
    src[i] = row * p.kv_tok_bytes + kv_head_off + (((lane % CHUNKS) ^ dswz(row)) << 4);
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
  const TileAddr ta = tile_addr(lane);

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  if (n_tiles > 0) load_tile(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1, cur ^ 1);
    if (t < wave_tiles) {
      const uint8_t* kl = lds + cur * kTile;
      const uint8_t* vl = lds + (2 + cur) * kTile;
      const int k0 = t * kBN;
      // S^T and dP^T blocks kb: keys k0 + 32 kb + (8 (r/4) + 4 hh + r%4), query my_q
      f32x16 sc[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][r] = dp[kb][r] = 0.f;
#pragma unroll
      for (int dk = 0; dk < D / 16; ++dk)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 ka = *(const bf16x8*)(kl + kb * 32 * ROW + ta.row_rd[dk]);
          const bf16x8 va = *(const bf16x8*)(vl + kb * 32 * ROW + ta.row_rd[dk]);
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[dk], sc[kb], 0, 0, 0);
          dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gf[dk], dp[kb], 0, 0, 0);
        }
      const bool need_mask = (k0 + kBN > p.s) || (CAUSAL && k0 + kBN - 1 > it.q0);
      bf16x8 dsb[kBN / 16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], p.c, -lse2));
          float ds = pr * (dp[kb][r] - dlt);
          if (need_mask) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= p.s || (CAUSAL && key > my_q)) ds = 0.f;
          }
          sc[kb][r] = ds;
        }
#pragma unroll
      for (int ks = 0; ks < kBN / 16; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) dsb[ks][e] = (__bf16)sc[ks >> 1][(ks & 1) * 8 + e];
      // dq^T += K^T dS^T, K^T read transposed from the K tile
#pragma unroll
      for (int ks = 0; ks < kBN / 16; ++ks)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr(kl, ta, ks, db), dsb[ks],
                                                            acc[db], 0, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  store_t(rsrc(p.dq, p.q_bytes), acc, p.inv_sd, my_q, p.q_tok_bytes, q_head_off, hh);
}

// ------------------------------------------------------------------ dk, dv
constexpr int kKWaves = 4;
constexpr int kKThreads = 64 * kKWaves;
constexpr int kKB = 32 * kKWaves;      // keys per workgroup
constexpr int kQT = 32;                // queries per tile
constexpr int kQTile = kQT * ROW;      // one Q or dout tile
constexpr int kVBlock = kKB * ROW;     // the workgroup's V rows
constexpr int kKLoads = kQT * CHUNKS / (64 * kKWaves);  // 16-byte loads per lane per tile tensor

template <bool CAUSAL>
__global__ __launch_bounds__(kKThreads, 2) void bwd_dkv_kernel(BwdParams p) {
  // LDS: V block, then Q0 Q1 dout0 dout1
  __shared__ __attribute__((aligned(16))) uint8_t lds[kVBlock + 4 * kQTile];
  uint8_t* vblk = lds;
  uint8_t* qt = lds + kVBlock;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  // item: key block (lowest first when causal: the longest), then batch, KV
  // head.  The first `slots` workgroups are resident together and the
  // dispatcher gives workgroups p and p + slots/2 the same CU, so the second
  // half of that first wave takes its ranks in reverse (longest with shortest).
  int rank = blockIdx.x;
  if (CAUSAL && p.slots > 0 && rank < p.slots && rank >= p.slots / 2)
    rank = p.slots + p.slots / 2 - 1 - rank;
  const int per_k = p.b * p.hkvp;
  const int kblk = rank / per_k;
  const int kvg = (rank - kblk * per_k) % p.hkvp;
  const int be = (rank - kblk * per_k) / p.hkvp;
  const int kw0 = kblk * kKB + wave * 32;  // this wave's first key
  const int my_key = kw0 + l32;

  const __amdgpu_buffer_rsrc_t rq = rsrc(p.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rdo = rsrc(p.dout, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(p.v, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t rst = rsrc(p.lse2, p.stat_bytes);
  const __amdgpu_buffer_rsrc_t rde = rsrc(p.delta, p.stat_bytes);
  const int kv_head_off = (be * p.hkvp + kvg) * ROW;

  // K^T fragments (B operand of S = Q K^T): key my_key, features 16 dk + 8 hh .. +7
  bf16x8 kf[D / 16];
  {
    const int off = my_key * p.kv_tok_bytes + kv_head_off + hh * 16;
#pragma unroll
    for (int dk = 0; dk < D / 16; ++dk)
      kf[dk] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rk, off + dk * 32, 0, 0));
  }
  // the workgroup's V rows into LDS (swizzled like the tiles): 32 KiB, 8 loads per wave
#pragma unroll
  for (int i = 0; i < kVBlock / (1024 * kKWaves); ++i) {
    const int row = (wave * (kVBlock / (1024 * kKWaves)) + i) * 4 + lane / CHUNKS;
    load_lds16(rv, vblk + (wave * (kVBlock / (1024 * kKWaves)) + i) * 1024,
               (kblk * kKB + row) * p.kv_tok_bytes + kv_head_off +
                   (((lane % CHUNKS) ^ dswz(row)) << 4));
  }
#pragma unroll
  for (int dk = 0; dk < D / 16; ++dk) asm volatile("" ::"v"(kf[dk]));

  // steps: (query head of the group, 32-query tile); causal tiles start at the
  // workgroup's first key
  const int t_first = CAUSAL ? (kblk * kKB) / kQT : 0;
  const int n_qt = (p.s + kQT - 1) / kQT;
  const int per_head = n_qt - t_first;
  const int n_steps = (kblk * kKB < p.s) ? p.G * per_head : 0;

  int src[kKLoads];
#pragma unroll
  for (int i = 0; i < kKLoads; ++i) {
    const int row = (wave * kKLoads + i) * 4 + lane / CHUNKS;
    src[i] = row * p.q_tok_bytes + (((lane % CHUNKS) ^ dswz(row)) << 4);
  }
  auto step_head = [&](int st) { return kvg * p.G + st / per_head; };
  auto step_q0 = [&](int st) { return (t_first + st % per_head) * kQT; };
  auto load_step = [&](int st, int buf) {
    const int off = step_q0(st) * p.q_tok_bytes + (be * p.hp + step_head(st)) * ROW;
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int dst = (wave * kKLoads + i) * 1024;
      load_lds16(rq, qt + buf * kQTile + dst, src[i] + off);
      load_lds16(rdo, qt + (2 + buf) * kQTile + dst, src[i] + off);
    }
  };
  const TileAddr ta = tile_addr(lane);

  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[db][r] = dva[db][r] = 0.f;

  if (n_steps > 0) load_step(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int st = 0; st < n_steps; ++st) {
    const int cur = st & 1;
    if (st + 1 < n_steps) load_step(st + 1, cur ^ 1);
    const int head = step_head(st), q0 = step_q0(st);
    // the wave's keys are all above this tile's queries: nothing to add
    if (!(CAUSAL && q0 + kQT - 1 < kw0) && kw0 < p.s) {
      const uint8_t* ql = qt + cur * kQTile;
      const uint8_t* gl = qt + (2 + cur) * kQTile;
      // lse2 and D of the 16 queries this lane's accumulator rows hold:
      // q0 + 8 j + 4 hh + (0..3), j = 0..3
      const int stat = ((be * p.hp + head) * p.s_pad + q0 + 4 * hh) * 4;
      f32x4 l4[4], d4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        l4[j] = as_f32x4(__builtin_amdgcn_raw_buffer_load_b128(rst, stat + 32 * j, 0, 0));
        d4[j] = as_f32x4(__builtin_amdgcn_raw_buffer_load_b128(rde, stat + 32 * j, 0, 0));
      }
      // S (queries x keys) and dP: rows q0 + 8 (r/4) + 4 hh + r%4, column my_key
      f32x16 sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = dp[r] = 0.f;
#pragma unroll
      for (int dk = 0; dk < D / 16; ++dk) {
        const bf16x8 qa = *(const bf16x8*)(ql + ta.row_rd[dk]);
        const bf16x8 ga = *(const bf16x8*)(gl + ta.row_rd[dk]);
        // V^T fragment of this lane's key from the V block (row-read addressing)
        const bf16x8 vb = *(const bf16x8*)(vblk + wave * 32 * ROW + ta.row_rd[dk]);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[dk], sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vb, dp, 0, 0, 0);
      }
      const bool need_mask = (q0 + kQT > p.s) || (CAUSAL && q0 < kw0 + 31) || (kw0 + 32 > p.s);
      bf16x8 pb[kQT / 16], dsb[kQT / 16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float l2 = l4[r >> 2][r & 3];
        const float dl = d4[r >> 2][r & 3];
        // masked entries are set to zero, not multiplied by it: the statistics
        // of query rows past the sequence are not defined
        float pr = __builtin_amdgcn_exp2f(fmaf(sc[r], p.c, -l2));
        float ds = pr * (dp[r] - dl);
        if (need_mask) {
          const int qq = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (qq >= p.s || my_key >= p.s || (CAUSAL && my_key > qq)) pr = ds = 0.f;
        }
        sc[r] = pr;
        dp[r] = ds;
      }
#pragma unroll
      for (int ks = 0; ks < kQT / 16; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[ks][e] = (__bf16)sc[ks * 8 + e];
          dsb[ks][e] = (__bf16)dp[ks * 8 + e];
        }
      // dv^T += dout^T P, dk^T += Q^T dS (tiles read transposed)
#pragma unroll
      for (int ks = 0; ks < kQT / 16; ++ks)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr(gl, ta, ks, db), pb[ks],
                                                            dva[db], 0, 0, 0);
          dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr(ql, ta, ks, db), dsb[ks],
                                                            dka[db], 0, 0, 0);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  store_t(rsrc(p.dk, p.kv_bytes), dka, p.inv_sd, my_key, p.kv_tok_bytes, kv_head_off, hh);
  store_t(rsrc(p.dv, p.kv_bytes), dva, 1.f, my_key, p.kv_tok_bytes, kv_head_off, hh);
}

int64_t bwd_slots() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return (int64_t)cus * 2;  // two 4-wave dkv workgroups per CU
}

}  // namespace

int64_t attn_bwd_bf16_workspace_size(const AttnBwdArgs& a) {
  const int64_t s_pad = (a.s + 3) / 4 * 4;
  return 2 * a.b * a.hp * s_pad * (int64_t)sizeof(float);
}

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream) {
  if (a.d != D) return hipErrorInvalidValue;
  const int64_t s_pad = (a.s + 3) / 4 * 4;
  float* delta = static_cast<float*>(a.workspace);
  float* lse2 = delta + a.b * a.hp * s_pad;
  const int64_t rows = a.s * a.b * a.hp;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0,
                     stream, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.lse, delta, lse2,
                     (int)rows, (int)a.s, (int)s_pad, (int)(a.b * a.hp));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  BwdParams p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.dout = (const uint16_t*)a.dout;
  p.delta = delta;
  p.lse2 = lse2;
  p.dq = (uint16_t*)a.dq;
  p.dk = (uint16_t*)a.dk;
  p.dv = (uint16_t*)a.dv;
  p.s = (int)a.s;
  p.b = (int)a.b;
  p.hp = (int)a.hp;
  p.hkvp = (int)a.hkvp;
  p.G = (int)(a.hp / a.hkvp);
  p.q_tok_bytes = (int)(a.b * a.hp * ROW);
  p.kv_tok_bytes = (int)(a.b * a.hkvp * ROW);
  p.q_bytes = (int)(a.s * a.b * a.hp * ROW);
  p.kv_bytes = (int)(a.s * a.b * a.hkvp * ROW);
  p.s_pad = (int)s_pad;
  p.stat_bytes = (int)(a.b * a.hp * s_pad * 4);
  p.c = (float)(1.4426950408889634 / sqrt((double)D));
  p.inv_sd = (float)(1.0 / sqrt((double)D));
  p.QH = (p.G % 8 == 0) ? 8 : (p.G % 4 == 0) ? 4 : (p.G % 2 == 0) ? 2 : 1;
  p.QB = 32 * (kQWaves / p.QH);
  p.n_qblk = (p.s + p.QB - 1) / p.QB;
  p.nsub = p.G / p.QH;
  p.n_kblk = (p.s + kKB - 1) / kKB;
  const int64_t q_items = (int64_t)p.n_qblk * p.b * p.hkvp * p.nsub;
  const int64_t k_items = (int64_t)p.n_kblk * p.b * p.hkvp;
  const int64_t slots = bwd_slots();
  p.slots = (slots > 0 && k_items >= slots && (slots % 2) == 0) ? (int)slots : 0;
  if (a.causal) {
    hipLaunchKernelGGL(bwd_dq_kernel<true>, dim3((unsigned)q_items), dim3(kQThreads), 0, stream, p);
    hipLaunchKernelGGL(bwd_dkv_kernel<true>, dim3((unsigned)k_items), dim3(kKThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(bwd_dq_kernel<false>, dim3((unsigned)q_items), dim3(kQThreads), 0, stream, p);
    hipLaunchKernelGGL(bwd_dkv_kernel<false>, dim3((unsigned)k_items), dim3(kKThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace ulys
