// merge.hip -- merge of two partial attention results of one share over
// disjoint key sets, on gfx950.
//
// What it computes ("长上下文训练中的 SP 与 CP", Ring section: every query row's
// online-softmax state -- running max, scaled sum, scaled weighted sum -- is
// brought to a common max and added when a block from another key range
// arrives; a finished partial result carries the same state as its
// log-sum-exp and normalised output): per query row,
//   lse = ln(e^lse_a + e^lse_b),  O = e^(lse_a - lse) O_a + e^(lse_b - lse) O_b,
// with an empty partial (lse = -inf) contributing nothing and two empties
// giving O = 0, lse = -inf.  This is the step that combines a rank's
// Ulysses-sharded attention with the key blocks a ring delivers in the
// hierarchical scheme ("02 · DeepSpeed-Ulysses" §4) and in USP.
//
// Layout: O [s, b, hp, d] (bf16 or fp32), lse [b, hp, s] fp32, as the forward
// writes them.  A row's d*elt bytes are covered by consecutive lanes of one
// wave, one 16-byte vector each; every lane of the row loads its two lse
// values (the same address for all of them) and the row's first lane stores
// the merged lse.  All loads of a row are complete before any of its stores,
// so the merge may accumulate in place (o = o_a, lse = lse_a; hence no
// restrict qualifier on those two).  HBM-bound:
// 3 * (row bytes + 4) per row.
#include <math.h>

#include "cdna4.h"
#include "internal.h"

namespace ulys {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

template <bool BF16>
__global__ __launch_bounds__(kThreads) void attn_merge_rows(
    const u32x4* o_a, const float* lse_a, const u32x4* __restrict__ o_b,
    const float* __restrict__ lse_b, u32x4* o, float* lse, uint32_t total, FastDiv lanes_per_row,
    FastDiv heads, FastDiv batch, uint32_t s) {
  const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  if (g >= total) return;
  const uint32_t row = fast_div(g, lanes_per_row);  // (t * b + be) * hp + i
  const uint32_t part = g - row * lanes_per_row.div;
  const uint32_t ti = fast_div(row, heads);          // t * b + be
  const uint32_t i = row - ti * heads.div;
  const uint32_t t = fast_div(ti, batch);
  const uint32_t be = ti - t * batch.div;
  const uint32_t li = (be * heads.div + i) * s + t;  // this row's lse
  const float la = lse_a[li], lb = lse_b[li];
  const u32x4 va = o_a[g], vb = o_b[g];
  const float m = fmaxf(la, lb);
  u32x4 out;
  float l_new;
  if (m == -INFINITY) {
    out = u32x4{0u, 0u, 0u, 0u};
    l_new = -INFINITY;
  } else {
    const float wa = __builtin_amdgcn_exp2f((la - m) * kLog2e);  // exp2(-inf) = 0
    const float wb = __builtin_amdgcn_exp2f((lb - m) * kLog2e);
    const float l = wa + wb;
    const float inv = 1.f / l;
    const float ca = wa * inv, cb = wb * inv;
    if (BF16) {
      const bf16x8 xa = as_bf16x8(va), xb = as_bf16x8(vb);
      bf16x8 r;
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = (__bf16)fmaf(ca, (float)xa[e], cb * (float)xb[e]);
      out = __builtin_bit_cast(u32x4, r);
    } else {
      const f32x4 xa = as_f32x4(va), xb = as_f32x4(vb);
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = fmaf(ca, xa[e], cb * xb[e]);
      out = __builtin_bit_cast(u32x4, r);
    }
    l_new = m + __builtin_amdgcn_logf(l) * kLn2;
  }
  o[g] = out;
  if (part == 0) lse[li] = l_new;
}

}  // namespace

hipError_t launch_attn_merge(const void* o_a, const float* lse_a, const void* o_b,
                             const float* lse_b, void* o, float* lse, uint32_t s, uint32_t b,
                             uint32_t hp, uint32_t row_bytes, int elt, hipStream_t stream) {
  if (row_bytes % 16 != 0 || row_bytes / 16 > 64 || (elt != 2 && elt != 4))
    return hipErrorInvalidValue;
  const uint32_t lanes = row_bytes / 16;
  const uint64_t total = (uint64_t)s * b * hp * lanes;
  if (total == 0) return hipSuccess;
  if (total >= (1ull << 32) - kThreads) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)((total + kThreads - 1) / kThreads));
  if (elt == 2)
    hipLaunchKernelGGL(attn_merge_rows<true>, grid, dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(o_a), lse_a, static_cast<const u32x4*>(o_b),
                       lse_b, static_cast<u32x4*>(o), lse, (uint32_t)total, make_fastdiv(lanes),
                       make_fastdiv(hp), make_fastdiv(b), s);
  else
    hipLaunchKernelGGL(attn_merge_rows<false>, grid, dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(o_a), lse_a, static_cast<const u32x4*>(o_b),
                       lse_b, static_cast<u32x4*>(o), lse, (uint32_t)total, make_fastdiv(lanes),
                       make_fastdiv(hp), make_fastdiv(b), s);
  return hipGetLastError();
}

}  // namespace ulys
