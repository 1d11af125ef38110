// internal.h -- declarations shared by the host-side ABI and the kernel files
// of the HIP library.  Not installed; the public surface is include/ulysses.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ulys {

// Division of 32-bit unsigned numerators by a runtime-invariant divisor with a
// multiply-high and a shift (Granlund & Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994, round-up variant).
struct FastDiv {
  uint32_t div;    // the divisor d >= 1
  uint32_t mul;    // m = floor(2^32 * (2^l - d) / d) + 1
  uint32_t shift;  // l = ceil(log2 d)
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.div = d;
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  f.shift = l;
  f.mul = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
  uint32_t t = __umulhi(n, f.mul);
  return (uint32_t)(((uint64_t)t + n) >> f.shift);
}

// Layout kernels: out[bb][a] = in[a][bb] over an [A][B] grid of runs of
// run_bytes bytes each (a run is hp*d_h contiguous elements).
hipError_t launch_transpose_runs(const void* in, void* out, uint64_t A, uint64_t B,
                                 uint64_t run_bytes, hipStream_t stream);

// KV replication (fewer KV heads C than ranks P, C | P), runs of one head:
//   replicate: out[r][a] = in[a][r*C/P]            in [A][C], out [P][A]
//   sum:       out[a][g] = sum_{j<P/C} in[g*P/C+j][a] in [P][A], out [A][C]
// The sum accumulates in fp32 in ascending j and rounds once to the element
// type (elt 4: fp32, 2: bf16).  Grids must stay below 2^32 vectors.
hipError_t launch_replicate_runs(const void* in, void* out, uint32_t A, uint32_t C, uint32_t P,
                                 uint32_t run_bytes, hipStream_t stream);
// Q, K and V packs in one launch: segment k maps input [A][cols[k]] runs to
// output [P][A] runs with run r*A + a <- a*cols[k] + r*cols[k]/P (cols = P:
// the plain pack; cols = h_kv < P: the replicating one).  Every run_bytes
// a multiple of 16 and fewer than 2^32 vectors in all.
hipError_t launch_pack_qkv(const void* const in[3], void* const out[3], uint32_t A, uint32_t P,
                           const uint32_t cols[3], const uint32_t run_bytes[3],
                           hipStream_t stream);
// The exchange as pushes from one rank `src` to P destination pointers (runs
// of run_bytes = hp*d*elt, A = s/P*b rows):
//   seq2head: dst[r][src*A + a] = in[a*P + r]      (in: the rank's shard)
//   head2seq: dst[j][a*P + src] = in[j*A + a]      (in: the rank's output share)
// P <= 64.
hipError_t launch_push(const void* in, void* const* dst, uint32_t A, uint32_t P, uint32_t src,
                       uint32_t run_bytes, bool seq2head, hipStream_t stream);
hipError_t launch_sum_runs(const void* in, void* out, uint32_t A, uint32_t C, uint32_t P,
                           uint32_t run_bytes, int elt, hipStream_t stream);

// Merge of two partial attention results of one share (O [s, b, hp, d],
// lse [b, hp, s] fp32); o/lse may be o_a/lse_a.  row_bytes = d * elt, a
// multiple of 16 up to 1 KiB.
hipError_t launch_attn_merge(const void* o_a, const float* lse_a, const void* o_b,
                             const float* lse_b, void* o, float* lse, uint32_t s, uint32_t b,
                             uint32_t hp, uint32_t row_bytes, int elt, hipStream_t stream);

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;       // may be null
  int64_t s;        // sequence length of the share
  int64_t b;        // batch
  int64_t hp;       // query heads of the share
  int64_t hkvp;     // KV heads of the share
  int64_t d;        // head size
  int causal;
  void* workspace;          // may be null
  int64_t workspace_bytes;
  // non-null (bf16 only): the output rows are pushed into these `ranks`
  // shards [s/ranks, b, hp*ranks, d] at head columns of rank `rank`, not to o
  void* const* o_ranks = nullptr;
  int ranks = 0, rank = 0;
};

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream);
// workspace bytes launch_attn_bf16 would use to balance causal work (0: none)
int64_t attn_bf16_workspace_size(const AttnArgs& a);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream);

struct AttnBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int64_t s, b, hp, hkvp, d;
  int causal;
  void* workspace;
  int64_t workspace_bytes;
  // non-null: dQ, dK, dV rows are pushed into these `ranks` shards each
  // ([s/ranks, b, heads*ranks, d], head columns of rank `rank`), not stored
  // to dq, dk, dv (the KV heads must not be replicated)
  void* const* dq_ranks = nullptr;
  void* const* dk_ranks = nullptr;
  void* const* dv_ranks = nullptr;
  int ranks = 0, rank = 0;
};

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream);
int64_t attn_bwd_bf16_workspace_size(const AttnBwdArgs& a);
// fp32 inputs (no pushing epilogue): the workspace holds D = rowsum(dout * o)
hipError_t launch_attn_bwd_f32(const AttnBwdArgs& a, hipStream_t stream);
int64_t attn_bwd_f32_workspace_size(const AttnBwdArgs& a);

}  // namespace ulys
