// attn_bf16.hip -- bf16 head-sharded attention on CDNA4 matrix cores.
//
// What it computes: for each query head of the share, softmax(Q K^T/sqrt(d_h)) V
// over the whole sequence ("DeepSpeed-Ulysses 深度解析", core design step 4;
// "02 · DeepSpeed-Ulysses", §1 -- heads are independent), dense or causal
// (key j visible to query t iff j <= t), GQA by contiguous groups.  K/V tiles
// are folded in with the online softmax ("长上下文训练中的 SP 与 CP", Ring
// section: running max m, rescaled sum l and accumulator A, start m = -inf,
// l = 0, A = 0, finish O = A / l), so the s x s score matrix never exists.
//
// How it maps onto gfx950:
//  * A workgroup is 8 waves (one per CU; two per SIMD) and each wave owns 32
//    queries of one head, so every K/V tile brought into LDS serves 256
//    queries.  For GQA the waves may cover up to 8 query heads of one KV
//    group, so a K/V tile is fetched once for all of them.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand and the wave's
//    Q^T (kept in registers for the whole loop) the B operand.  In the 32x32
//    result each lane then holds 16 keys of ONE query, so the row max and row
//    sum are lane-local; only one exchange with the partner lane (l ^ 32) is
//    needed per tile for the max, and one at the end for the sum.
//  * The probabilities stay in registers and become the B operand of
//    O^T += V^T P^T with the same instruction.  V stays row-major in LDS; its
//    A operand comes from ds_read_b64_tr_b16, which transposes 4x4 blocks of
//    16-bit values across lanes as it reads.
//  * K and V tiles of 64 keys are double-buffered in LDS and filled by direct
//    global->LDS buffer loads (no staging registers).  The loop is software
//    pipelined: step t issues the loads of K_{t+2} and V_{t+1}, the MFMAs of
//    S_{t+1}, the softmax of S_t and the MFMAs of V_t^T P_t^T, so the score
//    MFMAs of the next tile overlap the exp work of this one.  Loads go
//    through raw buffer resources, so rows past the sequence read as zero
//    and the ragged tail needs no branch.  Tile rows are unpadded with
//    XOR-swizzled 16-byte chunks chosen so the MFMA K reads and the
//    transposing V reads are free of bank conflicts.
//  * exp2 with log2(e)/sqrt(d_h) folded into one FMA per score; causal tiles
//    above a wave's diagonal are skipped and only diagonal / tail tiles are
//    masked.
//  * The row max is taken only on a unit's first tile and on masked tiles.
//    Every other tile's probabilities are taken against the row's current
//    reference max, and only their sum is checked afterwards: a row whose
//    sum passed 2^8 moves its reference up by log2 of that sum (an upper
//    bound of the tile's max) and rescales.  Scores that jump so far within
//    one tile that the sum passes 2^64 flag the wave, which then redoes its
//    rows with the row max on every tile, reading K and V from global memory.
//  * Work items are ordered longest-first (causal), which the dispatcher turns
//    into a longest-processing-time-first schedule (with the first round's
//    order adapted to how it hands workgroups to shader engines, see
//    first_round_unit).  With a workspace, causal shares with few items split
//    every item's keys in two halves that a second kernel merges, and shares
//    of many rounds hand out units from a counter (see
//    attn_bf16_workspace_bytes).
#include <math.h>

#include "cdna4.h"
#include "internal.h"

namespace ulys {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;  // keys per tile
constexpr int kQW = 32;  // queries per wave
constexpr int kMaxPushRanks = 64;  // destinations of the pushing epilogue

template <int D>
struct Cfg {
  static constexpr int ROW_BYTES = D * 2;             // one key row of K or V
  static constexpr int CHUNKS = ROW_BYTES / 16;       // 16-byte chunks per row
  static constexpr int TILE_BYTES = kBN * ROW_BYTES;  // one K or V tile, unpadded
  // LDS: V0 V1 K0 K1, so every read offset fits the 16-bit immediate field
  static constexpr int V_BASE = 0;
  static constexpr int K_BASE = 2 * TILE_BYTES;
  static constexpr int LDS_BYTES = 4 * TILE_BYTES;
  // direct global->LDS loads: one wave instruction fills 1 KiB = ROWS_PER_LOAD rows
  static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;
  static constexpr int LOADS = kBN / (ROWS_PER_LOAD * kWaves);  // per wave per tensor
  // one partial state of a work unit: per wave and lane, the D/2 O^T
  // accumulator slots, the running max m and the lane's running sum l
  static constexpr int PART_SLOTS = D / 2 + 2;
  static constexpr int PART_FLOATS = kWaves * 64 * PART_SLOTS;
  static_assert(LOADS * ROWS_PER_LOAD * kWaves == kBN, "tile split");
};

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int s, b, hp, hkvp;
  int G;       // query heads per KV head
  int QH;      // query heads per workgroup (divides G, <= 8)
  int QB;      // queries per head per workgroup = 32 * 8 / QH
  int n_qblk;  // ceil(s / QB)
  int nsub;    // G / QH
  int nsplit;  // 1: one unit per item; 2: each item's key tiles split in two halves
  int rev_units;  // workgroups below this index (the first round) run first_round_unit
  unsigned* tickets;  // non-null: every workgroup takes its unit from this counter (zeroed first)
  float* ws;   // nsplit == 2: partial states, PART_FLOATS per (item, half)
  int q_tok_bytes, kv_tok_bytes;  // bytes between consecutive tokens
  int q_bytes, kv_bytes;  // tensor sizes in bytes (bounds of the buffer resources)
  float c;     // log2(e) / sqrt(d_h)
  float lazy;  // 8 / c: margin (raw score units) by which a row max may pass m_run
  // push (o_rank set): row t of the share goes to shard o_rank[t / sl] at
  // token t % sl, this rank's head columns, instead of to o
  int push, sl;
  int push_tok_bytes, push_be_bytes, push_head_off, push_bytes;
  uint16_t* o_rank[kMaxPushRanks];
};

// LDS tiles are unpadded, with the 16-byte chunks of row r XOR-swizzled so
// that reads are free of bank conflicts on gfx950's LDS, which serves 256
// bytes (64 banks) per clock: 16 lanes of a 16-byte read, 32 lanes of an
// 8-byte read.
//  * K: the QK MFMA operand read takes 16 consecutive rows at one logical
//    chunk per clock.  With 256-byte rows (D = 128) chunk c is stored at
//    c ^ (r & 15): 16 distinct chunks.  With 128-byte rows (D = 64) rows pair
//    up in one 256-byte bank line, so even rows use c ^ (r/2 & 7) and odd rows
//    c ^ ((r/2 & 7) ^ 4): 16 distinct (half-line, chunk) slots.
//  * V: a transposing read takes 4 consecutive rows x 64 bytes per 32 lanes
//    (4 chunks 4 db .. 4 db + 3).  With 256-byte rows chunk c is stored at
//    c ^ (10 (r & 3) mod 16): the 4 rows' chunk groups land on 4 different
//    64-byte quarters of the bank line, and on different 32-byte halves of
//    128 bytes too.  With 128-byte rows c ^ 2 (r & 3) does the same.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  if constexpr (D == 128) return r & 15;
  else return ((r >> 1) ^ ((r & 1) << 2)) & 7;
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  if constexpr (D == 128) return (10 * (r & 3)) & 15;
  else return 2 * (r & 3);
}

// Work item `rank` (longest causal q-block first, then batch, KV head, head
// subgroup) as seen by one wave: its batch, KV head, query head and first query.
struct Item {
  int qblk, be, kvg, head, q0;
};
__device__ __forceinline__ Item decode_item(const Params& p, int rank, int wave, bool causal) {
  Item it;
  const int per_q = p.b * p.hkvp * p.nsub;
  const int qi = rank / per_q;
  int rest = rank - qi * per_q;
  it.qblk = causal ? (p.n_qblk - 1 - qi) : qi;
  const int sub = rest % p.nsub;
  rest /= p.nsub;
  it.kvg = rest % p.hkvp;
  it.be = rest / p.hkvp;
  const int wph = kWaves / p.QH;  // waves per query head
  it.head = it.kvg * p.G + sub * p.QH + wave / wph;
  it.q0 = it.qblk * p.QB + (wave % wph) * kQW;
  return it;
}

// O = A / l rounded once to bf16, and lse in natural log, for this lane's
// query (rows past s fall outside the buffer resource and are dropped).
// With push set, the row goes straight to its place after the head->seq
// exchange ("02 · DeepSpeed-Ulysses" §2: the output is sent by sequence
// segment and the receiver concatenates along heads): shard o_rank[j] of the
// rank that owns segment j = my_q / sl, token my_q % sl, this rank's head
// columns.  A wave's 32 rows may span several segments; the wave takes them
// one uniform segment at a time, so every destination pointer is a scalar.
// PUSH is a separate instantiation of the kernels, so the plain ones compile
// as if the pushing epilogue did not exist.
template <int D, bool PUSH>
__device__ __forceinline__ void store_output(const Params& p, const f32x16* oacc, float m_run,
                                             float l_run, int be, int head, int my_q, int hh) {
  const float l_tot = xsum32(l_run);
  const float inv = 1.f / l_tot;
  u32x2 w[D / 32][4];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const __bf16 x0 = (__bf16)(oacc[db][4 * g4 + 0] * inv);
      const __bf16 x1 = (__bf16)(oacc[db][4 * g4 + 1] * inv);
      const __bf16 x2 = (__bf16)(oacc[db][4 * g4 + 2] * inv);
      const __bf16 x3 = (__bf16)(oacc[db][4 * g4 + 3] * inv);
      w[db][g4] = u32x2{(uint32_t)__builtin_bit_cast(uint16_t, x0) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16),
                        (uint32_t)__builtin_bit_cast(uint16_t, x2) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, x3) << 16)};
    }
  if constexpr (!PUSH) {
    const __amdgpu_buffer_rsrc_t ro = rsrc(p.o, p.q_bytes);
    const int ooff = my_q * p.q_tok_bytes + (be * p.hp + head) * D * 2 + hh * 8;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        __builtin_amdgcn_raw_buffer_store_b64(w[db][g4], ro, ooff + (db * 32 + 8 * g4) * 2, 0,
                                              0);
  } else {
    const int j = (my_q < p.s) ? my_q / p.sl : -1;
    uint64_t todo = __ballot(j >= 0);
    while (todo) {
      const int jj = __builtin_amdgcn_readlane(j, (int)__builtin_ctzll(todo));
      const bool mine = j == jj;
      todo &= ~__ballot(mine);
      if (mine) {
        const __amdgpu_buffer_rsrc_t rd = rsrc(p.o_rank[jj], p.push_bytes);
        const int off = (my_q - jj * p.sl) * p.push_tok_bytes + be * p.push_be_bytes +
                        p.push_head_off + head * D * 2 + hh * 8;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            __builtin_amdgcn_raw_buffer_store_b64(w[db][g4], rd, off + (db * 32 + 8 * g4) * 2, 0,
                                                  0);
      }
    }
  }
  if (p.lse && hh == 0 && my_q < p.s)
    p.lse[(int64_t)(be * p.hp + head) * p.s + my_q] =
        (m_run * p.c + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
}

// Unit run by workgroup b.  The dispatcher sends workgroup b to XCD b % 8 and
// hands each XCD's workgroups, in order, to its four shader engines in a fixed
// rotation, each waiting for a free CU in its own engine.  Units are ranked
// longest first, so in the first round (one workgroup per CU) each run of four
// consecutive workgroups of an XCD would free its CUs in the reverse of the
// rotation, and every second-round workgroup would wait for the last of the
// four.  Reversing each such run (32 consecutive workgroups: 4 per XCD) in the
// first round frees the CUs in rotation order; later rounds keep the ranked
// order, so the longest remaining unit still goes to the first free CU.
__device__ __forceinline__ int first_round_unit(int b, int rev_units) {
  if (b >= rev_units) return b;
  const int r = b & 31;
  return (b & ~31) | ((3 - (r >> 3)) << 3) | (r & 7);
}

template <int D, bool CAUSAL, bool PUSH>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(Params p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  // ---- work unit.  With nsplit == 2, unit u is half u % 2 of item u / 2.
  // Items are ranked longest first, so unit sizes never increase and the
  // dispatcher, which hands the next unit to the first CU that frees up,
  // schedules longest-processing-time first.
  int unit;
  if (p.tickets) {
    // the next unit in ranked order, whichever XCD this workgroup runs on;
    // broadcast through the second V buffer, which the first step's loads
    // write only after the prologue's barriers
    int* slot = reinterpret_cast<int*>(lds + C::V_BASE + C::TILE_BYTES);
    if (tid == 0)
      *slot = (int)__hip_atomic_fetch_add(p.tickets, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    unit = __builtin_amdgcn_readfirstlane(*slot);
  } else {
    unit = first_round_unit(blockIdx.x, p.rev_units);
  }
  int rank = unit;
  int half_id = 0;
  if (p.nsplit == 2) {
    half_id = rank & 1;
    rank >>= 1;
  }
  const Item item = decode_item(p, rank, wave, CAUSAL);
  const int qblk = item.qblk, be = item.be, kvg = item.kvg, head = item.head, q0 = item.q0;
  const int my_q = q0 + l32;

  const __amdgpu_buffer_rsrc_t rq = rsrc(p.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(p.v, p.kv_bytes);
  const int q_head_off = (be * p.hp + head) * D * 2;     // bytes
  const int kv_head_off = (be * p.hkvp + kvg) * D * 2;   // bytes

  // ---- Q^T fragments (B operand): lane holds query my_q, d = 16*dk + 8*hh .. +7
  bf16x8 qf[D / 16];
  {
    const int qoff = my_q * p.q_tok_bytes + q_head_off + hh * 16;
#pragma unroll
    for (int dk = 0; dk < D / 16; ++dk)
      qf[dk] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rq, qoff + dk * 32, 0, 0));
    // consume Q here so its loads are complete before the key loop: otherwise
    // the loop inherits them as outstanding and every tile waits on the vector
    // memory counter, i.e. on the next tile's K/V loads
#pragma unroll
    for (int dk = 0; dk < D / 16; ++dk) asm volatile("" ::"v"(qf[dk]));
  }

  const int q_hi = min(p.s, (qblk + 1) * p.QB);
  const int n_item_tiles = CAUSAL ? (q_hi + kBN - 1) / kBN : (p.s + kBN - 1) / kBN;
  // key tiles [t_lo, n_tiles) of this unit
  const int t_split = (n_item_tiles + 1) >> 1;
  const int t_lo = (p.nsplit == 2 && half_id == 1) ? t_split : 0;
  const int n_tiles = (p.nsplit == 2 && half_id == 0) ? t_split : n_item_tiles;
  const int wave_last_q = min(q0 + kQW, p.s) - 1;
  const int wave_tiles = (q0 >= p.s) ? 0 : (CAUSAL ? wave_last_q / kBN + 1 : n_tiles);

  // ---- global -> LDS loads of one K/V tile (rows past s read as 0).  Wave w,
  // load i fills LDS rows R0 = (w*LOADS + i)*ROWS_PER_LOAD .. +ROWS_PER_LOAD-1;
  // lane j lands at byte 16 j of that KiB: row R0 + j / CHUNKS, stored chunk
  // j % CHUNKS, so it fetches the logical chunk that the swizzle puts there.
  int k_src[C::LOADS], v_src[C::LOADS];  // per-lane global byte offsets at key 0
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int row = (wave * C::LOADS + i) * C::ROWS_PER_LOAD + lane / C::CHUNKS;
    const int pc = lane % C::CHUNKS;
    k_src[i] = row * p.kv_tok_bytes + kv_head_off + ((pc ^ k_swz<D>(row)) << 4);
    v_src[i] = row * p.kv_tok_bytes + kv_head_off + ((pc ^ v_swz<D>(row)) << 4);
  }
  f32x16 oacc[D / 32];
  float m_run;  // reference max of raw scores (q.k) the exponents subtract
  float l_run;  // this lane's share of the running sum
  bool overflow = false;  // a fast step's probabilities got too large

  // K tile t goes to K buffer (t - t_lo) % 2 and V tile t to V buffer
  // (t - t_lo) % 2.  Past the unit's last tile the source is clamped to it
  // while the buffer stays that of t, which no later step reads.
  const int t_last = n_tiles - 1;
  auto load_k = [&](int t) {
    const int koff = min(t, t_last) * kBN * p.kv_tok_bytes;
    uint8_t* dst = lds + C::K_BASE + ((t - t_lo) & 1) * C::TILE_BYTES + wave * C::LOADS * 1024;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) load_lds16(rk, dst + i * 1024, k_src[i] + koff);
  };
  auto load_v = [&](int t) {
    const int koff = min(t, t_last) * kBN * p.kv_tok_bytes;
    uint8_t* dst = lds + C::V_BASE + ((t - t_lo) & 1) * C::TILE_BYTES + wave * C::LOADS * 1024;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) load_lds16(rv, dst + i * 1024, v_src[i] + koff);
  };
  // lane parts of the LDS read addresses (bytes), one per operand column
  // block.  K, step dk: row kb*32 + l32 (kb*32 leaves the swizzle unchanged),
  // logical chunk 2 dk + hh.
  int k_rd[D / 16];
#pragma unroll
  for (int dk = 0; dk < D / 16; ++dk)
    k_rd[dk] = l32 * C::ROW_BYTES + (((2 * dk + hh) ^ k_swz<D>(l32)) << 4);
  // V (transposing reads), feature block db: row 4 hh + (l%16)/4 of a 16-key
  // step (the keys this lane's P^T registers hold; 16 ks and +8 leave the
  // swizzle unchanged), byte column 64 db + 32 ((l/16)%2) + 8 (l%4)
  const int vr = 4 * hh + ((lane & 15) >> 2);
  int v_rd[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int c = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    v_rd[db] = vr * C::ROW_BYTES + ((c ^ v_swz<D>(vr)) << 4) + 8 * (lane & 1);
  }

  // S^T block kb of tile t: keys 64 t + 32 kb + (8 (r/4) + 4 hh + r%4), query
  // my_q.  The two blocks' MFMA chains are interleaved.
  auto qk = [&](int t, f32x16* sc) {
    const uint8_t* kl = lds + C::K_BASE + ((t - t_lo) & 1) * C::TILE_BYTES;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
    for (int dk = 0; dk < D / 16; ++dk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *(const bf16x8*)(kl + kb * 32 * C::ROW_BYTES + k_rd[dk]);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dk], sc[kb], 0, 0, 0);
      }
  };
  // O^T += V^T P^T for tile t.  Key step ks: this lane's P^T registers hold
  // keys 16 ks + 8 j + 4 hh + (0..3) in slots 4 j .. 4 j + 3 (j = 0, 1).  The
  // feature blocks' MFMA chains are interleaved.
  auto pv = [&](int t, const bf16x8* pb) {
    const uint8_t* vl = lds + C::V_BASE + ((t - t_lo) & 1) * C::TILE_BYTES;
#pragma unroll
    for (int ks = 0; ks < kBN / 16; ++ks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint8_t* vb = vl + (ks * 16) * C::ROW_BYTES + v_rd[db];
        const u32x2 lo = lds_read_tr(reinterpret_cast<const uint16_t*>(vb));
        const u32x2 hi = lds_read_tr(reinterpret_cast<const uint16_t*>(vb + 8 * C::ROW_BYTES));
        const bf16x8 a = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], oacc[db], 0, 0, 0);
      }
  };
  // S^T blocks of tile t read straight from global memory (rows past the
  // sequence read as zero, as in the LDS loads)
  auto qk_global = [&](int t, f32x16* sc) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
      const int off = (t * kBN + kb * 32 + l32) * p.kv_tok_bytes + kv_head_off + hh * 16;
#pragma unroll
      for (int dk = 0; dk < D / 16; ++dk) {
        const bf16x8 a = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rk, off + dk * 32, 0, 0));
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dk], sc[kb], 0, 0, 0);
      }
    }
  };
  // scores of tile t past the sequence end or above the causal diagonal -> -inf
  auto needs_mask = [&](int t) {
    const int k0 = t * kBN;
    return (k0 + kBN > p.s) || (CAUSAL && k0 + kBN - 1 > q0);
  };
  auto mask = [&](int t, f32x16* sc) {
    const int k0 = t * kBN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= p.s || (CAUSAL && key > my_q)) sc[kb][r] = -INFINITY;
      }
  };
  // online-softmax step on the scores of one tile.  The reference max m_run
  // that the exponents subtract moves only when a row's tile max exceeds it
  // by more than p.lazy (8 in log2 units): any m_run at least the true max
  // minus that margin gives the same softmax (the factor cancels between the
  // sum and the accumulator) and keeps every exponent at most 8, far from
  // overflow.  After the first tiles of a row the rescale of the running sum
  // and accumulator then almost never runs.  Returns m_run * c.
  auto update_max = [&](const f32x16* sc) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    mx = xmax32(mx);
    const bool grow = mx > m_run + p.lazy;  // m_run = -inf: any finite max
    if (__ballot(grow) != 0) {
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * p.c) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
    }
    return (m_run == -INFINITY) ? 0.f : m_run * p.c;
  };
  // probabilities exp2(s c - m c) of one tile, packed to bf16 as the P^T
  // operands (16-key step ks uses registers 8 (ks%2) .. +7 of block ks/2);
  // returns their fp32 sum over this lane's 32 keys
  auto probs = [&](f32x16* sc, float base, bf16x8* pb) -> float {
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], p.c, -base));
        sc[kb][r] = e;
        ps += e;
      }
#pragma unroll
    for (int ks = 0; ks < kBN / 16; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[ks][e] = (__bf16)sc[ks >> 1][(ks & 1) * 8 + e];
    return ps;
  };
  // After a fast step (probabilities against the current reference, no row
  // max): a row whose tile sum -- over both partner lanes -- passed 2^8 had
  // a score more than 8 (log2 units) above the reference, or many near it.
  // Its reference moves up by log2 of that sum, which bounds the tile's max
  // from above (the sum is at least its largest term), and the running sum
  // and accumulator are scaled by its inverse -- the same rescale a max
  // would give, with another valid reference.  A sum beyond 2^64 (or not a
  // number) flags the unit: its accumulator may have lost range, and it is
  // redone with the row max on every tile.
  auto settle = [&](float ps) {
    const float pair = xsum32(ps);
    overflow |= !(pair <= 0x1p64f);
    if (pair > 256.f && pair <= 0x1p64f) {
      const float alpha = __builtin_amdgcn_rcpf(pair);
      m_run += __builtin_amdgcn_logf(pair) * (p.lazy * 0.125f);  // log2(pair) / c
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
  };

  // O^T += V^T P^T for tile t with V^T read from global memory: the A operand
  // slot e of lane (feature f, half hh) is key 16 ks + 8 (e/4) + 4 hh + e%4,
  // the key the P^T slot e of the same half holds (rows past the sequence
  // read as zero).
  auto pv_global = [&](int t, const bf16x8* pb) {
#pragma unroll
    for (int ks = 0; ks < kBN / 16; ++ks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        bf16x8 a;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = t * kBN + 16 * ks + 8 * (e >> 2) + 4 * hh + (e & 3);
          const int off = key * p.kv_tok_bytes + kv_head_off + (db * 32 + l32) * 2;
          a[e] = __builtin_bit_cast(__bf16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rv, off, 0, 0));
        }
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], oacc[db], 0, 0, 0);
      }
  };
  auto redo_from_global = [&]() {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;
    const int t_end = min(wave_tiles, n_tiles);
#pragma unroll 1
    for (int t = t_lo; t < t_end; ++t) {
      f32x16 sc[2];
      qk_global(t, sc);
      if (needs_mask(t)) mask(t, sc);
      const float base = update_max(sc);
      bf16x8 pb[kBN / 16];
      l_run += probs(sc, base, pb);
      pv_global(t, pb);
    }
  };

  // ---- software pipeline over the unit's key tiles [t_lo, n_tiles).  On
  // entry to step t the scores S_t are in sacc, K_{t+1} and V_t are in LDS.
  // Step t issues the loads of K_{t+2} (into the buffer K_t used) and V_{t+1}
  // (into the buffer V_{t-1} used), computes S_{t+1} = K_{t+1} Q^T, turns S_t
  // into probabilities and accumulates V_t^T P_t^T; the next step starts after
  // its loads landed and every wave passed the barrier.  The MFMAs of S_{t+1}
  // are independent of the exp / sum / convert work on S_t, so the two
  // interleave.  Buffer reuse: K_{t+2} overwrites K_t, last read by step
  // t - 1 (or, for the first step, by the prologue, hence its barrier), and
  // V_{t+1} overwrites V_{t-1}, last read by step t - 1.
  // one step; cur holds S_t on entry, nxt receives S_{t+1}
  auto step = [&](int t, f32x16* cur, f32x16* nxt) {
    const int k0 = t * kBN;
    const bool need_mask = (k0 + kBN > p.s) || (CAUSAL && k0 + kBN - 1 > q0);
    if (t > t_lo && t < wave_tiles && !need_mask && t + 1 < wave_tiles) {
      // steady state, fast: no row max.  The probabilities of S_t are taken
      // against the reference max as it stands (every row has seen visible
      // keys in tile t_lo, so it is finite), and the rule that bounds them
      // is applied afterwards (settle).  One basic block up to that test.
      qk(t + 1, nxt);
      bf16x8 pb[kBN / 16];
      const float ps = probs(cur, m_run * p.c, pb);
      load_k(t + 2);
      load_v(t + 1);
      pv(t, pb);
      l_run += ps;
      if (__ballot(ps > 256.f) != 0) settle(ps);
    } else {
      load_k(t + 2);
      load_v(t + 1);
      if (t < wave_tiles) {
        if (need_mask) mask(t, cur);
        const float base = update_max(cur);
        bf16x8 pb[kBN / 16];
        l_run += probs(cur, base, pb);
        if (t + 1 < wave_tiles) qk(t + 1, nxt);
        pv(t, pb);
      }
    }
    // this step's loads must have landed before anyone reads them
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  m_run = -INFINITY;
  l_run = 0.f;
  f32x16 sa[2], sb[2];
  if (t_lo < n_tiles) {
    load_k(t_lo);
    load_v(t_lo);
    load_k(t_lo + 1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (t_lo < wave_tiles) qk(t_lo, sa);
  __syncthreads();  // every wave's reads of K_{t_lo} precede the first step's loads
  // unrolled by two so the score registers swap roles instead of being
  // copied, and every buffer parity is a compile-time constant
  for (int i = 0; t_lo + 2 * i < n_tiles; ++i) {
    const int t = t_lo + 2 * i;
    step(t, sa, sb);
    if (t + 1 < n_tiles) step(t + 1, sb, sa);
  }
  // Only if a fast step flagged an overflow (scores that jump by more than
  // ~64 log2 units past a row's reference within one tile, so that the
  // accumulator may have lost range): this wave's rows again, every tile with
  // the row max, K and V read from global memory (the other waves have
  // moved on, so the LDS tiles and barriers are not available).
  if (__ballot(overflow) != 0) redo_from_global();

  if (p.nsplit == 2) {
    // partial state of this half, lanes contiguous: [wave][slot][lane]
    float* part = p.ws + (int64_t)unit * C::PART_FLOATS + wave * (C::PART_SLOTS * 64) + lane;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[(db * 16 + r) * 64] = oacc[db][r];
    part[(D / 2) * 64] = m_run;
    part[(D / 2 + 1) * 64] = l_run;
    return;
  }
  store_output<D, PUSH>(p, oacc, m_run, l_run, be, head, my_q, hh);
}

// Workgroups of this kernel resident at once on the current device: one per
// CU (8 waves of up to 256 VGPRs fill a CU's register file), or 0 if unknown.
int64_t resident_slots() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return (int64_t)cus;
}

int64_t count_items(const AttnArgs& a) {
  const int64_t G = a.hp / a.hkvp;
  const int64_t QH = (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int64_t QB = kQW * (kWaves / QH);
  return (a.s + QB - 1) / QB * a.b * a.hkvp * (G / QH);
}

// Bytes of workspace the call can use (0: none):
//  * causal work with too few items to fill the resident slots twice (the
//    longest item alone would set the run time) is split into two halves per
//    item, whose partial states the workspace holds;
//  * work of four or more rounds of workgroups takes its units from a counter
//    in the workspace instead of from the workgroup index.  The dispatcher
//    binds workgroup b to XCD b % 8, and the XCDs of one GPU run at somewhat
//    different clocks, so a fixed mapping leaves the slowest XCD finishing
//    last; with the counter each workgroup, wherever it starts, takes the
//    longest unit left.
int64_t attn_bf16_workspace_bytes(const AttnArgs& a) {
  const int64_t items = count_items(a);
  const int64_t slots = resident_slots();
  if (slots > 0 && items >= 4 * slots) return 256;
  if (!a.causal || slots <= 0 || items >= 2 * slots) return 0;
  const int64_t part = (int64_t)kWaves * 64 * (a.d / 2 + 2) * 4;
  return items * 2 * part;
}

// Merge of the two halves of every item: the same rescaling as the online
// softmax, applied once to two partial states over disjoint key ranges.
template <int D, bool CAUSAL, bool PUSH>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(Params p) {
  using C = Cfg<D>;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const Item item = decode_item(p, blockIdx.x, wave, CAUSAL);
  const float* p0 = p.ws + (int64_t)(2 * blockIdx.x) * C::PART_FLOATS +
                    wave * (C::PART_SLOTS * 64) + lane;
  const float* p1 = p0 + C::PART_FLOATS;
  const float m0 = p0[(D / 2) * 64], m1 = p1[(D / 2) * 64];
  const float m = fmaxf(m0, m1);
  // the first half always holds key 0, so m is finite for every real query
  const float a0 = __builtin_amdgcn_exp2f((m0 - m) * p.c);
  const float a1 = __builtin_amdgcn_exp2f((m1 - m) * p.c);
  const float l = p0[(D / 2 + 1) * 64] * a0 + p1[(D / 2 + 1) * 64] * a1;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      oacc[db][r] = p0[(db * 16 + r) * 64] * a0 + p1[(db * 16 + r) * 64] * a1;
  store_output<D, PUSH>(p, oacc, m, l, item.be, item.head, item.q0 + l32, hh);
}

__global__ void clear_tickets(unsigned* t) {
  if (threadIdx.x == 0) __builtin_nontemporal_store(0u, t);
}

// The unit counter cleared first, then the attention; with a split, the merge.
template <int D, bool CAUSAL, bool PUSH>
void launch_kernels(const Params& p, unsigned units, unsigned items, int nsplit,
                    hipStream_t stream) {
  if (p.tickets) hipLaunchKernelGGL(clear_tickets, dim3(1), dim3(64), 0, stream, p.tickets);
  hipLaunchKernelGGL((attn_bf16_kernel<D, CAUSAL, PUSH>), dim3(units), dim3(kThreads), 0, stream,
                     p);
  if (nsplit == 2)
    hipLaunchKernelGGL((attn_merge_kernel<D, CAUSAL, PUSH>), dim3(items), dim3(kThreads), 0,
                       stream, p);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  Params p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.o = (uint16_t*)a.o;
  p.lse = a.lse;
  p.s = (int)a.s;
  p.b = (int)a.b;
  p.hp = (int)a.hp;
  p.hkvp = (int)a.hkvp;
  p.G = (int)(a.hp / a.hkvp);
  p.QH = (p.G % 8 == 0) ? 8 : (p.G % 4 == 0) ? 4 : (p.G % 2 == 0) ? 2 : 1;
  p.QB = kQW * (kWaves / p.QH);
  p.n_qblk = (p.s + p.QB - 1) / p.QB;
  p.nsub = p.G / p.QH;
  p.q_tok_bytes = (int)(a.b * a.hp * D * 2);
  p.kv_tok_bytes = (int)(a.b * a.hkvp * D * 2);
  p.q_bytes = (int)(a.s * a.b * a.hp * D * 2);
  p.kv_bytes = (int)(a.s * a.b * a.hkvp * D * 2);
  p.c = (float)(1.4426950408889634 / sqrt((double)D));
  p.lazy = 8.f / p.c;
  p.push = a.o_ranks != nullptr;
  p.sl = p.push_tok_bytes = p.push_be_bytes = p.push_head_off = p.push_bytes = 0;
  for (int r = 0; r < kMaxPushRanks; ++r) p.o_rank[r] = nullptr;
  if (p.push) {
    if (a.ranks <= 0 || a.ranks > kMaxPushRanks || a.rank < 0 || a.rank >= a.ranks ||
        a.s % a.ranks != 0)
      return hipErrorInvalidValue;
    const int64_t h = a.hp * a.ranks;
    p.sl = (int)(a.s / a.ranks);
    p.push_be_bytes = (int)(h * D * 2);
    p.push_tok_bytes = (int)(a.b * h * D * 2);
    p.push_head_off = (int)(a.rank * a.hp * D * 2);
    p.push_bytes = (int)((int64_t)p.sl * p.push_tok_bytes);
    for (int r = 0; r < a.ranks; ++r) p.o_rank[r] = static_cast<uint16_t*>(a.o_ranks[r]);
  }
  const int64_t items = (int64_t)p.n_qblk * p.b * p.hkvp * p.nsub;
  if (items <= 0) return hipSuccess;
  if (items > 0x7FFFFFFF) return hipErrorInvalidValue;
  // split halves or the unit counter (see attn_bf16_workspace_bytes) when the
  // caller gave room
  const int64_t ws_need = attn_bf16_workspace_bytes(a);
  const bool room = ws_need > 0 && a.workspace && a.workspace_bytes >= ws_need;
  const int nsplit = (room && ws_need > 256) ? 2 : 1;
  p.nsplit = nsplit;
  p.tickets = (room && ws_need == 256) ? static_cast<unsigned*>(a.workspace) : nullptr;
  {
    // the first round: one workgroup per CU, whole runs of 32 only
    const int64_t units = items * nsplit, slots = resident_slots();
    p.rev_units = (int)((units < slots ? units : slots) & ~int64_t(31));
  }
  p.ws = nsplit == 2 ? (float*)a.workspace : nullptr;
  const unsigned units = (unsigned)(items * nsplit);
  if (a.causal && p.push)
    launch_kernels<D, true, true>(p, units, (unsigned)items, nsplit, stream);
  else if (a.causal)
    launch_kernels<D, true, false>(p, units, (unsigned)items, nsplit, stream);
  else if (p.push)
    launch_kernels<D, false, true>(p, units, (unsigned)items, nsplit, stream);
  else
    launch_kernels<D, false, false>(p, units, (unsigned)items, nsplit, stream);
  return hipGetLastError();
}

}  // namespace

int64_t attn_bf16_workspace_size(const AttnArgs& a) { return attn_bf16_workspace_bytes(a); }

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_d<128>(a, stream);
  if (a.d == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ulys
