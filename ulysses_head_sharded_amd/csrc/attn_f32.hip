// attn_f32.hip -- fp32 head-sharded attention (the fp32 path of the share).
//
// Per head, softmax(Q K^T / sqrt(d_h)) V over the whole sequence, dense or
// causal (key j visible to query t iff j <= t), GQA by contiguous groups
// ("DeepSpeed-Ulysses 深度解析", core design step 4; "02 · DeepSpeed-Ulysses",
// §1).  The key loop folds tiles in with the online softmax (running max m,
// rescaled sum l, rescaled accumulator; start m = -inf, l = 0, end O = A/l --
// "长上下文训练中的 SP 与 CP", Ring section).
//
// This path serves fp32 inputs, which the workloads use only at tiny sizes,
// so it favours plainness: one lane owns one query row and keeps q and its
// accumulator in registers; a 64-lane workgroup stages 32-key K/V tiles of
// its head in LDS.  All arithmetic is fp32 (FMA dot products, exp2 with
// log2(e)/sqrt(d_h) folded into the scores).
#include <math.h>

#include "internal.h"

namespace ulys {
namespace {

constexpr int kRows = 64;   // query rows per workgroup (one per lane)
constexpr int kKeys = 32;   // keys per LDS tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int s, int b, int hp, int hkvp,
    float scale_log2) {
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];

  const int lane = threadIdx.x;
  const int bh = blockIdx.y;        // = beta * hp + i
  const int be = bh / hp, i = bh % hp;
  const int g = i / (hp / hkvp);    // KV head of this query head
  const int t = blockIdx.x * kRows + lane;
  const bool valid = t < s;
  const int64_t q_tok = (int64_t)b * hp * D, kv_tok = (int64_t)b * hkvp * D;
  const int64_t q_off = (int64_t)(be * hp + i) * D, kv_off = (int64_t)(be * hkvp + g) * D;

  float qr[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qr[e] = valid ? q[(int64_t)t * q_tok + q_off + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const int t_last = min(s, (int)(blockIdx.x + 1) * kRows) - 1;  // last row of the block
  const int key_end = CAUSAL ? t_last + 1 : s;
  for (int k0 = 0; k0 < key_end; k0 += kKeys) {
    __syncthreads();
    for (int idx = lane; idx < kKeys * D; idx += kRows) {
      const int j = idx / D, e = idx % D;
      const int key = k0 + j;
      const bool in = key < s;
      ks[j][e] = in ? k[(int64_t)key * kv_tok + kv_off + e] : 0.f;
      vs[j][e] = in ? v[(int64_t)key * kv_tok + kv_off + e] : 0.f;
    }
    __syncthreads();

    float sc[kKeys];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(qr[e], ks[j][e], dot);
      const int key = k0 + j;
      const bool vis = key < s && (!CAUSAL || key <= t);
      sc[j] = vis ? dot * scale_log2 : -INFINITY;   // log2-domain score
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float base = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m - base);
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      sc[j] = exp2f(sc[j] - base);
      psum += sc[j];
    }
    l = l * alpha + psum;
#pragma unroll
    for (int e = 0; e < D; ++e) {
      float a = acc[e] * alpha;
#pragma unroll
      for (int j = 0; j < kKeys; ++j) a = fmaf(sc[j], vs[j][e], a);
      acc[e] = a;
    }
    m = m_new;
  }

  if (!valid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < D; ++e) o[(int64_t)t * q_tok + q_off + e] = acc[e] * inv;
  if (lse) {
    // m and the scores are in log2 units: ln-sum-exp = (m + log2 l) * ln 2
    lse[(int64_t)bh * s + t] = (l > 0.f) ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.s + kRows - 1) / kRows), (unsigned)(a.b * a.hp));
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  if (a.causal)
    hipLaunchKernelGGL((attn_f32_kernel<D, true>), grid, dim3(kRows), 0, stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o,
                       a.lse, (int)a.s, (int)a.b, (int)a.hp, (int)a.hkvp, scale_log2);
  else
    hipLaunchKernelGGL((attn_f32_kernel<D, false>), grid, dim3(kRows), 0, stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o,
                       a.lse, (int)a.s, (int)a.b, (int)a.hp, (int)a.hkvp, scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream) {
  if (a.d == 64) return launch_d<64>(a, stream);
  if (a.d == 128) return launch_d<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ulys
