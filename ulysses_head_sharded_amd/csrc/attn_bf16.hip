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
//  * A workgroup is 4 waves; each wave owns 32 queries of one head.  For GQA
//    the 4 waves may cover up to 4 query heads of one KV group, so a K/V tile
//    is fetched once for all of them.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand and the wave's
//    Q^T (kept in registers for the whole loop) the B operand.  In the 32x32
//    result each lane then holds 16 keys of ONE query, so the row max and row
//    sum are lane-local; only one exchange with the partner lane (l ^ 32) is
//    needed per tile for the max, and one at the end for the sum.
//  * The probabilities stay in registers and become the B operand of
//    O^T += V^T P^T with the same instruction; V^T (the A operand) is read
//    from LDS, where V is stored transposed ([d][key]) with the keys of each
//    16-key step permuted so every lane reads 16 contiguous bytes that match
//    the keys its P^T registers hold.
//  * K and V^T tiles of 64 keys are double-buffered in LDS; the next tile's
//    global loads are in flight during the current tile's MFMAs.  Rows are
//    padded so the 16-byte LDS reads of 8 consecutive rows hit distinct banks.
//  * exp2 with log2(e)/sqrt(d_h) folded into one FMA per score; causal tiles
//    above a wave's diagonal are skipped, the diagonal tile is masked.
//  * Work items are ordered longest-first (causal) so short items fill the
//    tail of the grid.
#include <math.h>

#include "internal.h"

namespace ulys {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;  // keys per tile
constexpr int kQW = 32;  // queries per wave

template <int D>
struct Cfg {
  static constexpr int KP = D + 8;    // K row pitch in bf16 elements (odd multiple of 16 B)
  static constexpr int VP = kBN + 8;  // V^T row pitch in bf16 elements (odd multiple of 16 B)
  static constexpr int K_ELEMS = kBN * KP;
  static constexpr int V_ELEMS = D * VP;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int KCH = D / 8;                         // 16-byte chunks per row
  static constexpr int K_LOADS = kBN * KCH / kThreads;      // 16-byte K loads per thread
  static constexpr int V_KPT = kBN * D / (kThreads * 8);    // V keys per thread (x 8 d)
  static_assert(K_LOADS * kThreads == kBN * KCH, "K tile split");
  static_assert(V_KPT == 2 || V_KPT == 4, "V tile split");
};

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int s, b, hp, hkvp;
  int G;       // query heads per KV head
  int QH;      // query heads per workgroup (divides G, <= 4)
  int QB;      // queries per head per workgroup = 32 * 4 / QH
  int n_qblk;  // ceil(s / QB)
  int nsub;    // G / QH
  int64_t q_tok, kv_tok;  // elements between consecutive tokens
  float c;                // log2(e) / sqrt(d_h)
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Column of key kk (0..63) inside a V^T row: inside each 16-key step the
// 4-key chunks are stored in the order 0, 2, 1, 3, which puts the keys a lane
// pair (l, l+32) holds in P^T next to each other.
__device__ __forceinline__ int vt_col(int kk) {
  const int c = (kk >> 2) & 3;
  const int pc = ((c & 1) << 1) | (c >> 1);
  return (kk & ~15) | (pc << 2) | (kk & 3);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(Params p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * C::BUF_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  // ---- work item: longest causal q-block first, then batch, KV head, head subgroup
  const int per_q = p.b * p.hkvp * p.nsub;
  const int qi = blockIdx.x / per_q;
  int rest = blockIdx.x - qi * per_q;
  const int qblk = CAUSAL ? (p.n_qblk - 1 - qi) : qi;
  const int sub = rest % p.nsub;
  rest /= p.nsub;
  const int kvg = rest % p.hkvp;
  const int be = rest / p.hkvp;
  const int wph = kWaves / p.QH;  // waves per query head
  const int head = kvg * p.G + sub * p.QH + wave / wph;
  const int q0 = qblk * p.QB + (wave % wph) * kQW;  // first query of this wave
  const int my_q = q0 + l32;

  const uint16_t* qbase = p.q + (int64_t)(be * p.hp + head) * D;
  const uint16_t* kbase = p.k + (int64_t)(be * p.hkvp + kvg) * D;
  const uint16_t* vbase = p.v + (int64_t)(be * p.hkvp + kvg) * D;

  // ---- Q^T fragments (B operand): lane holds query my_q, d = 16*dk + 8*hh .. +7
  bf16x8 qf[D / 16];
#pragma unroll
  for (int dk = 0; dk < D / 16; ++dk) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (my_q < p.s) x = *(const u32x4*)(qbase + (int64_t)my_q * p.q_tok + dk * 16 + hh * 8);
    qf[dk] = as_bf16x8(x);
  }

  const int q_hi = min(p.s, (qblk + 1) * p.QB);
  const int n_tiles = CAUSAL ? (q_hi + kBN - 1) / kBN : (p.s + kBN - 1) / kBN;
  const int wave_last_q = min(q0 + kQW, p.s) - 1;
  const int wave_tiles = (q0 >= p.s) ? 0 : (CAUSAL ? wave_last_q / kBN + 1 : n_tiles);

  // ---- global -> register staging of one K/V tile
  u32x4 kreg[C::K_LOADS];
  u32x4 vreg[C::V_KPT];
  const int v_dc = tid % C::KCH;           // d chunk of this thread's V block
  const int v_kg = tid / C::KCH;           // key group of this thread's V block
  auto load_tile = [&](int t) {
    const int k0 = t * kBN;
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int ch = tid + i * kThreads;
      const int row = ch / C::KCH, col = ch % C::KCH;
      const int key = k0 + row;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < p.s) x = *(const u32x4*)(kbase + (int64_t)key * p.kv_tok + col * 8);
      kreg[i] = x;
    }
#pragma unroll
    for (int j = 0; j < C::V_KPT; ++j) {
      const int key = k0 + v_kg * C::V_KPT + j;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < p.s) x = *(const u32x4*)(vbase + (int64_t)key * p.kv_tok + v_dc * 8);
      vreg[j] = x;
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* kl = lds + buf * C::BUF_ELEMS;
    uint16_t* vl = kl + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int ch = tid + i * kThreads;
      const int row = ch / C::KCH, col = ch % C::KCH;
      *(u32x4*)(kl + row * C::KP + col * 8) = kreg[i];
    }
    // transpose the V_KPT x 8 block in registers: row d gets V_KPT consecutive keys
    const int col = vt_col(v_kg * C::V_KPT);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t w[C::V_KPT / 2];
#pragma unroll
      for (int jj = 0; jj < C::V_KPT / 2; ++jj) {
        const uint32_t a = vreg[2 * jj][e >> 1], bq = vreg[2 * jj + 1][e >> 1];
        w[jj] = (e & 1) ? ((a >> 16) | (bq & 0xFFFF0000u)) : ((a & 0xFFFFu) | (bq << 16));
      }
      uint16_t* dst = vl + (v_dc * 8 + e) * C::VP + col;
      if constexpr (C::V_KPT == 4) {
        *(u32x2*)dst = u32x2{w[0], w[1]};
      } else {
        *(uint32_t*)dst = w[0];
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY;  // running max of raw scores (q.k)
  float l_run = 0.f;        // this lane's share of the running sum

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);

    if (t < wave_tiles) {
      const uint16_t* kl = lds + cur * C::BUF_ELEMS;
      const uint16_t* vl = kl + C::K_ELEMS;
      const int k0 = t * kBN;

      // S^T block kb: keys k0 + 32 kb + (8 (r/4) + 4 hh + r%4), query my_q
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
        for (int dk = 0; dk < D / 16; ++dk) {
          const bf16x8 a = *(const bf16x8*)(kl + (kb * 32 + l32) * C::KP + dk * 16 + hh * 8);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dk], sacc[kb], 0, 0, 0);
        }
      }

      const bool need_mask = (k0 + kBN > p.s) || (CAUSAL && k0 + kBN - 1 > q0);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sacc[kb][r];
          if (need_mask) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= p.s || (CAUSAL && key > my_q)) x = -INFINITY;
          }
          sacc[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float base = (m_new == -INFINITY) ? 0.f : m_new * p.c;
      // rescale the running sum and accumulator only when some row's max grew;
      // rows whose max is unchanged keep a factor of exactly 1
      if (__ballot(m_new > m_run) != 0) {
        const float alpha = (m_new > m_run) ? __builtin_amdgcn_exp2f(m_run * p.c - base) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      m_run = m_new;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], p.c, -base));
          sacc[kb][r] = e;
          ps += e;
        }
      l_run += ps;

      // P^T operands: 16-key step ks uses registers 8 (ks%2) .. +7 of block ks/2
      bf16x8 pb[kBN / 16];
#pragma unroll
      for (int ks = 0; ks < kBN / 16; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[ks][e] = (__bf16)sacc[ks >> 1][(ks & 1) * 8 + e];

#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int ks = 0; ks < kBN / 16; ++ks) {
          const bf16x8 a = *(const bf16x8*)(vl + (db * 32 + l32) * C::VP + ks * 16 + hh * 8);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], oacc[db], 0, 0, 0);
        }
    }

    if (t + 1 < n_tiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = A / l, rounded once to bf16; lse in natural log
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_q < p.s) {
    const float inv = 1.f / l_tot;
    uint16_t* obase = p.o + (int64_t)my_q * p.q_tok + (int64_t)(be * p.hp + head) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const __bf16 x0 = (__bf16)(oacc[db][4 * g4 + 0] * inv);
        const __bf16 x1 = (__bf16)(oacc[db][4 * g4 + 1] * inv);
        const __bf16 x2 = (__bf16)(oacc[db][4 * g4 + 2] * inv);
        const __bf16 x3 = (__bf16)(oacc[db][4 * g4 + 3] * inv);
        const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, x0) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16);
        const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, x2) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, x3) << 16);
        *(u32x2*)(obase + db * 32 + 8 * g4 + 4 * hh) = u32x2{w0, w1};
      }
    if (p.lse && hh == 0)
      p.lse[(int64_t)(be * p.hp + head) * p.s + my_q] =
          (m_run * p.c + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
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
  p.QH = (p.G % 4 == 0) ? 4 : (p.G % 2 == 0) ? 2 : 1;
  p.QB = kQW * (kWaves / p.QH);
  p.n_qblk = (p.s + p.QB - 1) / p.QB;
  p.nsub = p.G / p.QH;
  p.q_tok = a.b * a.hp * D;
  p.kv_tok = a.b * a.hkvp * D;
  p.c = (float)(1.4426950408889634 / sqrt((double)D));
  const int64_t items = (int64_t)p.n_qblk * p.b * p.hkvp * p.nsub;
  if (items <= 0) return hipSuccess;
  if (items > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (a.causal)
    hipLaunchKernelGGL((attn_bf16_kernel<D, true>), dim3((unsigned)items), dim3(kThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, false>), dim3((unsigned)items), dim3(kThreads), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_d<128>(a, stream);
  if (a.d == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ulys
