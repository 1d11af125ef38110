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
// access is already fully coalesced on both sides; staging through LDS would
// add a round trip without removing any HBM transaction.  Threads walk the
// OUTPUT in order (consecutive lanes -> consecutive 16-byte vectors), one
// vector per thread with non-temporal loads and stores: on MI355X that
// streams at the rate of a plain device copy (measured ~5.9 TB/s from HBM at
// 128 MiB), while keeping several vectors per thread in flight was slower
// (4 per thread: ~4.9 TB/s).
#include "internal.h"

namespace ulys {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

template <typename Vec>
hipError_t launch_vec(const void* in, void* out, uint64_t A, uint64_t B, uint64_t run_bytes,
                      hipStream_t stream) {
  const uint64_t vpr = run_bytes / sizeof(Vec);
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

}  // namespace

hipError_t launch_transpose_runs(const void* in, void* out, uint64_t A, uint64_t B,
                                 uint64_t run_bytes, hipStream_t stream) {
  // widest vector that divides the run; the base pointers are 16-byte aligned
  if (run_bytes % 16 == 0) return launch_vec<u32x4>(in, out, A, B, run_bytes, stream);
  if (run_bytes % 8 == 0) return launch_vec<u32x2>(in, out, A, B, run_bytes, stream);
  if (run_bytes % 4 == 0) return launch_vec<uint32_t>(in, out, A, B, run_bytes, stream);
  return launch_vec<uint16_t>(in, out, A, B, run_bytes, stream);
}

}  // namespace ulys
