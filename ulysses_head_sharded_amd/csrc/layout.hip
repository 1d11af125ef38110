// layout.hip -- the local halves of the two Ulysses all-to-alls on gfx950.
//
// Pack (seq->head send side) and unpack (head->seq receive side) are both a
// transpose of a 2-D grid of contiguous runs ("02 · DeepSpeed-Ulysses", §2:
// split along heads and send group j to rank j; the reverse exchange is the
// inverse).  With sl = s/P and a run = the hp*d_h elements of one head group
// of one (token, batch) row:
//   pack   in [sl*b][P] runs  -> out [P][sl*b] runs
//   unpack in [P][sl*b] runs  -> out [sl*b][P] runs
// Every run is >= 256 bytes in the target workloads, so each 16-byte lane
// access is already fully coalesced on both sides.  Threads walk the OUTPUT
// in order (consecutive lanes -> consecutive 16-byte vectors), one vector per
// thread with non-temporal loads and stores: on MI355X that streams at the
// rate of a plain device copy (~5.9 TB/s from HBM at 128 MiB), while keeping
// several vectors per thread in flight was slower (4 per thread: ~4.9 TB/s).
// An LDS-staged tile transpose (transpose_runs_lds: a workgroup reads a tile
// of input rows into LDS and writes it out as contiguous output segments) was
// measured against it from HBM: 13-16% slower for the 128 MiB shards with
// 1 KiB runs and 22% slower for 256-byte runs over 8 ranks, but 11% faster
// for the pack of 256-byte runs over 64 ranks, where the output-order walk
// reads 256 bytes out of every 16 KiB input row; it serves that case (runs
// of at most 256 bytes, input rows of at least 8 KiB, the pack direction).
#include "internal.h"

namespace ulys {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kUnroll = 1;

template <typename Vec>
__global__ __launch_bounds__(kThreads) void transpose_runs32(
    const Vec* __restrict__ in, Vec* __restrict__ out, uint32_t total, FastDiv vpr,
    FastDiv rows_a, uint32_t cols_b) {
  // out is [B][A] runs of vpr vectors; in is [A][B] runs.
  const uint32_t base = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  Vec v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t g = base + u * kThreads;
    if (g < total) {
      const uint32_t run = fast_div(g, vpr);          // output run index = bb*A + a
      const uint32_t c = g - run * vpr.div;           // vector inside the run
      const uint32_t bb = fast_div(run, rows_a);
      const uint32_t a = run - bb * rows_a.div;
      v[u] = __builtin_nontemporal_load(&in[(a * cols_b + bb) * vpr.div + c]);
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t g = base + u * kThreads;
    if (g < total) __builtin_nontemporal_store(v[u], &out[g]);
  }
}

// LDS-staged variant of the same map: a workgroup moves a tile of TR input
// rows x TC input columns of runs.  It reads the tile's TR row segments (TC*V
// contiguous vectors each) into LDS in input order, then writes the TC output
// row segments (TR*V contiguous vectors each) from LDS in output order.
//   in [R][Cc] runs -> out [Cc][R] runs, V vectors per run;
//   R % TR == 0, Cc % TC == 0, TR*TC*V <= kLdsTile, R*Cc*V < 2^31 (host checks).
constexpr int kLdsTile = 1024;  // vectors: 16 KiB of LDS per workgroup
__global__ __launch_bounds__(kThreads) void transpose_runs_lds(
    const u32x4* __restrict__ in, u32x4* __restrict__ out, uint32_t R, uint32_t Cc, uint32_t V,
    uint32_t TR, uint32_t TC, FastDiv tiles_c, FastDiv seg_in, FastDiv seg_out) {
  __shared__ u32x4 tile[kLdsTile];
  const uint32_t tr = fast_div(blockIdx.x, tiles_c);
  const uint32_t tc = blockIdx.x - tr * tiles_c.div;
  const uint32_t r0 = tr * TR, c0 = tc * TC;
  const uint32_t n = TR * TC * V;
  for (uint32_t e = threadIdx.x; e < n; e += kThreads) {
    const uint32_t i = fast_div(e, seg_in);  // input row r0 + i
    const uint32_t w = e - i * seg_in.div;   // vector within its TC runs
    tile[e] = __builtin_nontemporal_load(&in[((r0 + i) * Cc + c0) * V + w]);
  }
  __syncthreads();
  for (uint32_t e = threadIdx.x; e < n; e += kThreads) {
    const uint32_t j = fast_div(e, seg_out);  // output row c0 + j
    const uint32_t w = e - j * seg_out.div;   // vector within its TR runs
    const uint32_t i = w / V, c = w - i * V;
    __builtin_nontemporal_store(tile[(i * TC + j) * V + c], &out[((c0 + j) * R + r0) * V + w]);
  }
}

// Same map with 64-bit indices, for grids of 2^32 vectors or more.
template <typename Vec>
__global__ __launch_bounds__(kThreads) void transpose_runs64(
    const Vec* __restrict__ in, Vec* __restrict__ out, uint64_t total, uint64_t vpr,
    uint64_t rows_a, uint64_t cols_b) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t g = (uint64_t)blockIdx.x * kThreads + threadIdx.x; g < total; g += stride) {
    const uint64_t run = g / vpr, c = g % vpr;
    const uint64_t bb = run / rows_a, a = run % rows_a;
    out[g] = in[(a * cols_b + bb) * vpr + c];
  }
}

// The tile of transpose_runs_lds for an [A][B] grid of runs of vpr 16-byte
// vectors, or false where the output-order walk is the faster kernel (see the
// file comment).  The walk reads one input run out of every B-run input row
// before it moves to the next row, and comes back B times: with runs of at
// most 256 bytes and rows of at least 8 KiB that reopens every row B times.
// The LDS tile serves that case in the pack direction (at least as many rows
// as columns; the unpack's few rows are read as that many sequential
// streams), with whole 8 x TC tiles.
bool lds_tile(uint64_t A, uint64_t B, uint64_t vpr, uint64_t* TR, uint64_t* TC) {
  if (vpr > 16 || B * vpr * 16 < 8192 || A < B || A * B * vpr >= (1ull << 31)) return false;
  *TR = 8;
  *TC = 8;
  while (*TR * *TC * vpr > (uint64_t)kLdsTile && *TC > 1) *TC >>= 1;
  return *TR * *TC * vpr <= (uint64_t)kLdsTile && A % *TR == 0 && B % *TC == 0;
}

template <typename Vec>
hipError_t launch_vec(const void* in, void* out, uint64_t A, uint64_t B, uint64_t run_bytes,
                      hipStream_t stream) {
  const uint64_t vpr = run_bytes / sizeof(Vec);
  uint64_t TR = 0, TC = 0;
  if (sizeof(Vec) == 16 && lds_tile(A, B, vpr, &TR, &TC)) {
    const uint32_t tiles = (uint32_t)((A / TR) * (B / TC));
    hipLaunchKernelGGL(transpose_runs_lds, dim3(tiles), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(in), static_cast<u32x4*>(out), (uint32_t)A,
                       (uint32_t)B, (uint32_t)vpr, (uint32_t)TR, (uint32_t)TC,
                       make_fastdiv((uint32_t)(B / TC)), make_fastdiv((uint32_t)(TC * vpr)),
                       make_fastdiv((uint32_t)(TR * vpr)));
    return hipGetLastError();
  }
  const uint64_t total = A * B * vpr;
  if (total == 0) return hipSuccess;
  if (total < (1ull << 32) - (uint64_t)kThreads * kUnroll) {
    const uint32_t blocks = (uint32_t)((total + kThreads * kUnroll - 1) / (kThreads * kUnroll));
    hipLaunchKernelGGL(transpose_runs32<Vec>, dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const Vec*>(in), static_cast<Vec*>(out), (uint32_t)total,
                       make_fastdiv((uint32_t)vpr), make_fastdiv((uint32_t)A), (uint32_t)B);
  } else {
    const uint32_t blocks = 65536;
    hipLaunchKernelGGL(transpose_runs64<Vec>, dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const Vec*>(in), static_cast<Vec*>(out), total, vpr, A, B);
  }
  return hipGetLastError();
}

// ---- fewer KV heads than ranks ("Ulysses vs Ring Attention" §三: Q, K and V
// take the same all-to-all, so with h_kv < P some ranks would get no KV head;
// the SP/CP page's Ulysses section: replicating KV heads lifts P | h_kv).
// Rank r's block is KV head r*C/P, the head its query heads use; the backward
// sums the gradient copies of each head.  Both walk the output in order, one
// vector per thread, like the transpose.
template <typename Vec>
__global__ __launch_bounds__(kThreads) void replicate_runs(
    const Vec* __restrict__ in, Vec* __restrict__ out, uint32_t total, FastDiv vpr,
    FastDiv rows_a, uint32_t C, FastDiv ranks) {
  const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  if (g >= total) return;
  const uint32_t run = fast_div(g, vpr);  // r*A + a
  const uint32_t c = g - run * vpr.div;
  const uint32_t r = fast_div(run, rows_a);
  const uint32_t a = run - r * rows_a.div;
  const uint32_t head = fast_div(r * C, ranks);
  __builtin_nontemporal_store(__builtin_nontemporal_load(&in[(a * C + head) * vpr.div + c]),
                              &out[g]);
}

// One thread per 16-byte output vector (8 bf16 or 4 fp32 elements).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void sum_runs16(
    const u32x4* __restrict__ in, u32x4* __restrict__ out, uint32_t total, FastDiv vpr,
    FastDiv heads_c, uint32_t A, uint32_t R) {
  const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  if (g >= total) return;
  const uint32_t run = fast_div(g, vpr);  // a*C + head
  const uint32_t c = g - run * vpr.div;
  const uint32_t a = fast_div(run, heads_c);
  const uint32_t head = run - a * heads_c.div;
  constexpr int N = BF16 ? 8 : 4;
  float acc[N];
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = 0.f;
  for (uint32_t j = 0; j < R; ++j) {
    const u32x4 v = __builtin_nontemporal_load(&in[((head * R + j) * A + a) * vpr.div + c]);
    // whole-vector casts (a bit_cast of a single vector element is miscompiled)
    if (BF16) {
      const f32x4 lo = __builtin_bit_cast(f32x4, v << 16);          // even elements
      const f32x4 hi = __builtin_bit_cast(f32x4, v & 0xFFFF0000u);  // odd elements
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc[2 * w] += lo[w];
        acc[2 * w + 1] += hi[w];
      }
    } else {
      const f32x4 f = __builtin_bit_cast(f32x4, v);
#pragma unroll
      for (int w = 0; w < 4; ++w) acc[w] += f[w];
    }
  }
  u32x4 o;
  if (BF16) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)acc[e];  // nearest-even
    o = __builtin_bit_cast(u32x4, r);
  } else {
    const f32x4 f = {acc[0], acc[1], acc[2], acc[3]};
    o = __builtin_bit_cast(u32x4, f);
  }
  __builtin_nontemporal_store(o, &out[g]);
}

// One thread per element, for runs that are not a whole number of vectors.
template <typename T>
__global__ __launch_bounds__(kThreads) void sum_runs1(const T* __restrict__ in,
                                                      T* __restrict__ out, uint32_t total,
                                                      FastDiv epr, FastDiv heads_c, uint32_t A,
                                                      uint32_t R) {
  const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  if (g >= total) return;
  const uint32_t run = fast_div(g, epr);
  const uint32_t c = g - run * epr.div;
  const uint32_t a = fast_div(run, heads_c);
  const uint32_t head = run - a * heads_c.div;
  float acc = 0.f;
  for (uint32_t j = 0; j < R; ++j) acc += (float)in[((head * R + j) * A + a) * epr.div + c];
  out[g] = (T)acc;
}

template <typename Vec>
hipError_t launch_replicate_vec(const void* in, void* out, uint32_t A, uint32_t C, uint32_t P,
                                uint32_t run_bytes, hipStream_t stream) {
  const uint32_t vpr = run_bytes / sizeof(Vec);
  const uint64_t total = (uint64_t)P * A * vpr;
  if (total == 0) return hipSuccess;
  if (total >= (1ull << 32) - kThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(replicate_runs<Vec>, dim3((uint32_t)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, static_cast<const Vec*>(in),
                     static_cast<Vec*>(out), (uint32_t)total, make_fastdiv(vpr),
                     make_fastdiv(A), C, make_fastdiv(P));
  return hipGetLastError();
}

// ---- Q, K and V packed by one launch.  Each segment is a pack whose output
// run r*A + a (rank r, token-batch row a) comes from input run
// a*C + r*C/P: C = P is the plain pack (run = the rank's head group), C = h_kv
// < P the replicating one (run = one KV head).  Every segment starts at a
// multiple of the workgroup size, so a workgroup finds its segment from its
// first thread index (uniform: the segment's fields become scalar loads),
// then each thread walks that output in order.
struct PackSeg {
  const u32x4* in;
  u32x4* out;
  uint32_t start;    // first global vector index of this segment (a multiple of kThreads)
  uint32_t n;        // vectors of this segment
  FastDiv vpr;       // vectors per run
  FastDiv rows_a;    // A = s/P * b
  uint32_t cols_c;   // input runs per token-batch row
};
struct PackSegs {
  PackSeg seg[3];
  FastDiv ranks;     // P
  uint32_t total;
};

__global__ __launch_bounds__(kThreads) void pack_segments(PackSegs ps) {
  const uint32_t g0 = blockIdx.x * kThreads;
  const int k = (g0 >= ps.seg[2].start) ? 2 : (g0 >= ps.seg[1].start) ? 1 : 0;
  const PackSeg& sg = ps.seg[k];
  const uint32_t gl = g0 - sg.start + threadIdx.x;
  if (gl >= sg.n) return;  // the padding up to the next segment's start
  const uint32_t run = fast_div(gl, sg.vpr);  // r*A + a
  const uint32_t c = gl - run * sg.vpr.div;
  const uint32_t r = fast_div(run, sg.rows_a);
  const uint32_t a = run - r * sg.rows_a.div;
  const uint32_t col = fast_div(r * sg.cols_c, ps.ranks);
  __builtin_nontemporal_store(
      __builtin_nontemporal_load(&sg.in[(a * sg.cols_c + col) * sg.vpr.div + c]), &sg.out[gl]);
}

// ---- the exchange as pushes: the sender writes each block straight into its
// destination's final layout ("02 · DeepSpeed-Ulysses" §2: send by head
// group, the receiver concatenates along the sequence; the reverse exchange
// sends by sequence segment and the receiver concatenates along heads), so
// neither a local send buffer nor an unpack is needed.  The destinations are
// P device pointers -- on a node, the ranks' receive buffers mapped into this
// process; on one GPU, P regions of its own memory.  Output order walk, one
// vector per thread; the pointer table travels in the kernel arguments.
constexpr int kMaxRanks = 64;
template <typename Vec>
struct RankPtrs {
  Vec* p[kMaxRanks];
};

// seq->head, from rank `src`: y_ranks[r][(src*A + a)*V + c] = x[(a*P + r)*V + c]
// (A = s/P * b token-batch rows, V = vectors per run of hp*d elements)
// head->seq, from rank `src`: x_ranks[j][(a*P + src)*V + c] = o[(j*A + a)*V + c]
template <typename Vec, bool SEQ2HEAD>
__global__ __launch_bounds__(kThreads) void push_runs(const Vec* __restrict__ in,
                                                      RankPtrs<Vec> dst, uint32_t total,
                                                      FastDiv vpr, FastDiv rows_a, uint32_t P,
                                                      uint32_t src) {
  const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  if (g >= total) return;
  const uint32_t run = fast_div(g, vpr);  // m*A + a: destination rank m, row a
  const uint32_t c = g - run * vpr.div;
  const uint32_t m = fast_div(run, rows_a);
  const uint32_t a = run - m * rows_a.div;
  const uint32_t V = vpr.div, A = rows_a.div;
  if (SEQ2HEAD) {
    __builtin_nontemporal_store(__builtin_nontemporal_load(&in[(a * P + m) * V + c]),
                                &dst.p[m][(src * A + a) * V + c]);
  } else {
    __builtin_nontemporal_store(__builtin_nontemporal_load(&in[(m * A + a) * V + c]),
                                &dst.p[m][(a * P + src) * V + c]);
  }
}

template <typename Vec>
hipError_t launch_push_vec(const void* in, void* const* dst, uint32_t A, uint32_t P, uint32_t src,
                           uint32_t run_bytes, bool seq2head, hipStream_t stream) {
  RankPtrs<Vec> ptrs;
  for (uint32_t r = 0; r < P; ++r) ptrs.p[r] = static_cast<Vec*>(dst[r]);
  for (uint32_t r = P; r < (uint32_t)kMaxRanks; ++r) ptrs.p[r] = nullptr;
  const uint32_t vpr = run_bytes / sizeof(Vec);
  const uint64_t total = (uint64_t)P * A * vpr;
  if (total == 0) return hipSuccess;
  if (total >= (1ull << 32) - kThreads) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)((total + kThreads - 1) / kThreads));
  if (seq2head)
    hipLaunchKernelGGL((push_runs<Vec, true>), grid, dim3(kThreads), 0, stream,
                       static_cast<const Vec*>(in), ptrs, (uint32_t)total, make_fastdiv(vpr),
                       make_fastdiv(A), P, src);
  else
    hipLaunchKernelGGL((push_runs<Vec, false>), grid, dim3(kThreads), 0, stream,
                       static_cast<const Vec*>(in), ptrs, (uint32_t)total, make_fastdiv(vpr),
                       make_fastdiv(A), P, src);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_push(const void* in, void* const* dst, uint32_t A, uint32_t P, uint32_t src,
                       uint32_t run_bytes, bool seq2head, hipStream_t stream) {
  if (P == 0 || P > (uint32_t)kMaxRanks || src >= P) return hipErrorInvalidValue;
  if (run_bytes % 16 == 0)
    return launch_push_vec<u32x4>(in, dst, A, P, src, run_bytes, seq2head, stream);
  if (run_bytes % 4 == 0)
    return launch_push_vec<uint32_t>(in, dst, A, P, src, run_bytes, seq2head, stream);
  return launch_push_vec<uint16_t>(in, dst, A, P, src, run_bytes, seq2head, stream);
}

hipError_t launch_pack_qkv(const void* const in[3], void* const out[3], uint32_t A, uint32_t P,
                           const uint32_t cols[3], const uint32_t run_bytes[3],
                           hipStream_t stream) {
  PackSegs ps;
  uint64_t start = 0;
  for (int k = 0; k < 3; ++k) {
    if (run_bytes[k] % 16 != 0 || cols[k] == 0) return hipErrorInvalidValue;
    const uint32_t vpr = run_bytes[k] / 16;
    ps.seg[k].in = static_cast<const u32x4*>(in[k]);
    ps.seg[k].out = static_cast<u32x4*>(out[k]);
    const uint64_t n = (uint64_t)P * A * vpr;
    if (n >= (1ull << 32)) return hipErrorInvalidValue;
    ps.seg[k].start = (uint32_t)start;
    ps.seg[k].n = (uint32_t)n;
    ps.seg[k].vpr = make_fastdiv(vpr);
    ps.seg[k].rows_a = make_fastdiv(A);
    ps.seg[k].cols_c = cols[k];
    start += (n + kThreads - 1) / kThreads * kThreads;
    if (start >= (1ull << 32) - kThreads) return hipErrorInvalidValue;
  }
  ps.ranks = make_fastdiv(P);
  ps.total = (uint32_t)start;
  if (ps.total == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_segments, dim3((ps.total + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, ps);
  return hipGetLastError();
}

hipError_t launch_replicate_runs(const void* in, void* out, uint32_t A, uint32_t C, uint32_t P,
                                 uint32_t run_bytes, hipStream_t stream) {
  if (run_bytes % 16 == 0) return launch_replicate_vec<u32x4>(in, out, A, C, P, run_bytes, stream);
  if (run_bytes % 8 == 0) return launch_replicate_vec<u32x2>(in, out, A, C, P, run_bytes, stream);
  if (run_bytes % 4 == 0) return launch_replicate_vec<uint32_t>(in, out, A, C, P, run_bytes, stream);
  return launch_replicate_vec<uint16_t>(in, out, A, C, P, run_bytes, stream);
}

hipError_t launch_sum_runs(const void* in, void* out, uint32_t A, uint32_t C, uint32_t P,
                           uint32_t run_bytes, int elt, hipStream_t stream) {
  if (C == 0 || P % C != 0 || (elt != 2 && elt != 4)) return hipErrorInvalidValue;
  const uint32_t R = P / C;
  if (run_bytes % 16 == 0) {
    const uint32_t vpr = run_bytes / 16;
    const uint64_t total = (uint64_t)A * C * vpr;
    if (total == 0) return hipSuccess;
    if (total >= (1ull << 32) - kThreads) return hipErrorInvalidValue;
    const dim3 grid((uint32_t)((total + kThreads - 1) / kThreads));
    if (elt == 2)
      hipLaunchKernelGGL(sum_runs16<true>, grid, dim3(kThreads), 0, stream,
                         static_cast<const u32x4*>(in), static_cast<u32x4*>(out), (uint32_t)total,
                         make_fastdiv(vpr), make_fastdiv(C), A, R);
    else
      hipLaunchKernelGGL(sum_runs16<false>, grid, dim3(kThreads), 0, stream,
                         static_cast<const u32x4*>(in), static_cast<u32x4*>(out), (uint32_t)total,
                         make_fastdiv(vpr), make_fastdiv(C), A, R);
    return hipGetLastError();
  }
  const uint32_t epr = run_bytes / elt;
  const uint64_t total = (uint64_t)A * C * epr;
  if (total == 0) return hipSuccess;
  if (total >= (1ull << 32) - kThreads) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)((total + kThreads - 1) / kThreads));
  if (elt == 2)
    hipLaunchKernelGGL(sum_runs1<__bf16>, grid, dim3(kThreads), 0, stream,
                       static_cast<const __bf16*>(in), static_cast<__bf16*>(out), (uint32_t)total,
                       make_fastdiv(epr), make_fastdiv(C), A, R);
  else
    hipLaunchKernelGGL(sum_runs1<float>, grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(in), static_cast<float*>(out), (uint32_t)total,
                       make_fastdiv(epr), make_fastdiv(C), A, R);
  return hipGetLastError();
}

hipError_t launch_transpose_runs(const void* in, void* out, uint64_t A, uint64_t B,
                                 uint64_t run_bytes, hipStream_t stream) {
  // widest vector that divides the run; the base pointers are 16-byte aligned
  if (run_bytes % 16 == 0) return launch_vec<u32x4>(in, out, A, B, run_bytes, stream);
  if (run_bytes % 8 == 0) return launch_vec<u32x2>(in, out, A, B, run_bytes, stream);
  if (run_bytes % 4 == 0) return launch_vec<uint32_t>(in, out, A, B, run_bytes, stream);
  return launch_vec<uint16_t>(in, out, A, B, run_bytes, stream);
}

}  // namespace ulys
