// attn_bwd_f32.hip -- fp32 backward of the head-sharded attention.
//
// The gradients of one rank's share for fp32 inputs, the same quantities as
// the bf16 backward ("02 · DeepSpeed-Ulysses", §5: the local attention's
// backward is the ordinary attention backward).  With the scaled scores
// S = q k^T / sqrt(d_h), P = exp(S - lse), dP = dout v^T, D = rowsum(dout * o):
//   dS = P * (dP - D),  dq = dS k / sqrt(d_h),  dk = dS^T q / sqrt(d_h),
//   dv = P^T dout,
// dk and dv summed over the query heads of each GQA group (contiguous groups,
// as in the forward).  Everything is fp32.
//
// Like the fp32 forward this path favours plainness over speed (the fp32
// workloads are tiny).  A head row of D features is held by D/32 neighbouring
// lanes, 32 features each, and the dot products q.k and dout.v are finished
// with xor shuffles inside that lane group:
//  * prep: D = rowsum(dout * o) per query row, into the workspace [b, hp, s];
//  * dq: a lane group per query row; 32-key K and V tiles of its head staged
//    in LDS; for every visible key, p, dp, ds and dq += ds k, in key order;
//  * dkv: a lane group per key row of a KV head; 32-query tiles of every query
//    head of its group (q, dout, lse and D) staged in LDS; dv += p dout and
//    dk += ds q, query head by query head, in query order.
// Every output element is summed by one lane group in a fixed order, so the
// result does not depend on scheduling.
#include <math.h>

#include "internal.h"

namespace ulys {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;  // keys (dq) or queries (dkv) per LDS tile
constexpr int kFeat = 32;  // features per lane

// Sum of x over the LPR lanes of a row's lane group (aligned, contiguous).
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int w = LPR / 2; w >= 1; w >>= 1) x += __shfl_xor(x, w, LPR);
  return x;
}

// D = rowsum(dout * o): one lane group per (token, batch, head) row in memory
// order r = (t * b + be) * hp + i, written to dl[(be * hp + i) * s + t].
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_f32(const float* __restrict__ o,
                                                         const float* __restrict__ dout,
                                                         float* __restrict__ dl, int64_t rows,
                                                         int s, int bhp) {
  constexpr int LPR = D / kFeat;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t r = gid / LPR;
  const int part = (int)(gid % LPR);
  float acc = 0.f;
  if (r < rows) {
    const float* a = o + r * D + part * kFeat;
    const float* g = dout + r * D + part * kFeat;
#pragma unroll
    for (int e = 0; e < kFeat; ++e) acc = fmaf(a[e], g[e], acc);
  }
  acc = group_sum<LPR>(acc);
  if (r < rows && part == 0) {
    const int64_t t = r / bhp, rem = r - t * bhp;  // rem = be * hp + i
    dl[rem * s + t] = acc;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_dq_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dl,
    float* __restrict__ dq, int s, int b, int hp, int hkvp, float scale) {
  constexpr int LPR = D / kFeat, RPB = kThreads / LPR;
  __shared__ float ks[kTile][D];
  __shared__ float vs[kTile][D];
  const int tid = threadIdx.x;
  const int part = tid % LPR, f0 = part * kFeat;
  const int bh = blockIdx.y, be = bh / hp, i = bh % hp;
  const int g = i / (hp / hkvp);
  const int t = blockIdx.x * RPB + tid / LPR;
  const bool valid = t < s;
  const int64_t q_tok = (int64_t)b * hp * D, kv_tok = (int64_t)b * hkvp * D;
  const int64_t q_off = (int64_t)(be * hp + i) * D + f0, kv_off = (int64_t)(be * hkvp + g) * D;

  float qr[kFeat], gr[kFeat], acc[kFeat];
#pragma unroll
  for (int e = 0; e < kFeat; ++e) {
    qr[e] = valid ? q[(int64_t)t * q_tok + q_off + e] : 0.f;
    gr[e] = valid ? dout[(int64_t)t * q_tok + q_off + e] : 0.f;
    acc[e] = 0.f;
  }
  const float lse_t = valid ? lse[(int64_t)bh * s + t] : 0.f;
  const float d_t = valid ? dl[(int64_t)bh * s + t] : 0.f;

  const int last_row = min(s, (int)(blockIdx.x + 1) * RPB) - 1;
  const int k_end = CAUSAL ? last_row + 1 : s;
  for (int k0 = 0; k0 < k_end; k0 += kTile) {
    for (int idx = tid; idx < kTile * D; idx += kThreads) {
      const int j = idx / D, e = idx % D, key = k0 + j;
      ks[j][e] = key < s ? k[(int64_t)key * kv_tok + kv_off + e] : 0.f;
      vs[j][e] = key < s ? v[(int64_t)key * kv_tok + kv_off + e] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < kTile; ++j) {
      float sd = 0.f, pd = 0.f;
#pragma unroll
      for (int e = 0; e < kFeat; ++e) {
        sd = fmaf(qr[e], ks[j][f0 + e], sd);
        pd = fmaf(gr[e], vs[j][f0 + e], pd);
      }
      sd = group_sum<LPR>(sd);
      pd = group_sum<LPR>(pd);
      const int key = k0 + j;
      const bool vis = valid && key < s && (!CAUSAL || key <= t);
      const float p = vis ? expf(sd * scale - lse_t) : 0.f;
      const float ds = p * (pd - d_t);
#pragma unroll
      for (int e = 0; e < kFeat; ++e) acc[e] = fmaf(ds, ks[j][f0 + e], acc[e]);
    }
    __syncthreads();
  }
  if (!valid) return;
#pragma unroll
  for (int e = 0; e < kFeat; ++e) dq[(int64_t)t * q_tok + q_off + e] = acc[e] * scale;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_dkv_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dl,
    float* __restrict__ dk, float* __restrict__ dv, int s, int b, int hp, int hkvp,
    float scale) {
  constexpr int LPR = D / kFeat, RPB = kThreads / LPR;
  __shared__ float qs[kTile][D];
  __shared__ float gs[kTile][D];
  __shared__ float ls[kTile];
  __shared__ float ds_[kTile];
  const int tid = threadIdx.x;
  const int part = tid % LPR, f0 = part * kFeat;
  const int bg = blockIdx.y, be = bg / hkvp, g = bg % hkvp;
  const int G = hp / hkvp;
  const int j = blockIdx.x * RPB + tid / LPR;  // this lane group's key
  const bool valid = j < s;
  const int64_t q_tok = (int64_t)b * hp * D, kv_tok = (int64_t)b * hkvp * D;
  const int64_t kv_off = (int64_t)(be * hkvp + g) * D + f0;

  float kr[kFeat], vr[kFeat], ak[kFeat], av[kFeat];
#pragma unroll
  for (int e = 0; e < kFeat; ++e) {
    kr[e] = valid ? k[(int64_t)j * kv_tok + kv_off + e] : 0.f;
    vr[e] = valid ? v[(int64_t)j * kv_tok + kv_off + e] : 0.f;
    ak[e] = 0.f;
    av[e] = 0.f;
  }
  // causal: no query before the block's first key sees any of its keys
  const int t_begin = CAUSAL ? (int)blockIdx.x * RPB / kTile * kTile : 0;
  for (int hi = 0; hi < G; ++hi) {
    const int i = g * G + hi;
    const int64_t q_off = (int64_t)(be * hp + i) * D;
    const int64_t st_off = (int64_t)(be * hp + i) * s;
    for (int t0 = t_begin; t0 < s; t0 += kTile) {
      for (int idx = tid; idx < kTile * D; idx += kThreads) {
        const int u = idx / D, e = idx % D, t = t0 + u;
        qs[u][e] = t < s ? q[(int64_t)t * q_tok + q_off + e] : 0.f;
        gs[u][e] = t < s ? dout[(int64_t)t * q_tok + q_off + e] : 0.f;
      }
      if (tid < kTile) {
        const int t = t0 + tid;
        ls[tid] = t < s ? lse[st_off + t] : 0.f;
        ds_[tid] = t < s ? dl[st_off + t] : 0.f;
      }
      __syncthreads();
      for (int u = 0; u < kTile; ++u) {
        float sd = 0.f, pd = 0.f;
#pragma unroll
        for (int e = 0; e < kFeat; ++e) {
          sd = fmaf(qs[u][f0 + e], kr[e], sd);
          pd = fmaf(gs[u][f0 + e], vr[e], pd);
        }
        sd = group_sum<LPR>(sd);
        pd = group_sum<LPR>(pd);
        const int t = t0 + u;
        const bool vis = valid && t < s && (!CAUSAL || j <= t);
        const float p = vis ? expf(sd * scale - ls[u]) : 0.f;
        const float dsv = p * (pd - ds_[u]);
#pragma unroll
        for (int e = 0; e < kFeat; ++e) {
          av[e] = fmaf(p, gs[u][f0 + e], av[e]);
          ak[e] = fmaf(dsv, qs[u][f0 + e], ak[e]);
        }
      }
      __syncthreads();
    }
  }
  if (!valid) return;
#pragma unroll
  for (int e = 0; e < kFeat; ++e) {
    dk[(int64_t)j * kv_tok + kv_off + e] = ak[e] * scale;
    dv[(int64_t)j * kv_tok + kv_off + e] = av[e];
  }
}

template <int D>
hipError_t launch_d(const AttnBwdArgs& a, hipStream_t stream) {
  constexpr int LPR = D / kFeat, RPB = kThreads / LPR;
  const int s = (int)a.s, b = (int)a.b, hp = (int)a.hp, hkvp = (int)a.hkvp;
  const float scale = (float)(1.0 / sqrt((double)D));
  const float* q = (const float*)a.q;
  const float* k = (const float*)a.k;
  const float* v = (const float*)a.v;
  const float* o = (const float*)a.o;
  const float* g = (const float*)a.dout;
  float* dl = (float*)a.workspace;
  const int64_t rows = a.s * a.b * a.hp;
  const int64_t prep_threads = rows * LPR;
  hipLaunchKernelGGL(bwd_prep_f32<D>, dim3((unsigned)((prep_threads + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, o, g, dl, rows, s, b * hp);
  const dim3 gq((unsigned)((a.s + RPB - 1) / RPB), (unsigned)(a.b * a.hp));
  const dim3 gkv((unsigned)((a.s + RPB - 1) / RPB), (unsigned)(a.b * a.hkvp));
  if (a.causal) {
    hipLaunchKernelGGL((bwd_dq_f32<D, true>), gq, dim3(kThreads), 0, stream, q, k, v, g, a.lse,
                       dl, (float*)a.dq, s, b, hp, hkvp, scale);
    hipLaunchKernelGGL((bwd_dkv_f32<D, true>), gkv, dim3(kThreads), 0, stream, q, k, v, g,
                       a.lse, dl, (float*)a.dk, (float*)a.dv, s, b, hp, hkvp, scale);
  } else {
    hipLaunchKernelGGL((bwd_dq_f32<D, false>), gq, dim3(kThreads), 0, stream, q, k, v, g, a.lse,
                       dl, (float*)a.dq, s, b, hp, hkvp, scale);
    hipLaunchKernelGGL((bwd_dkv_f32<D, false>), gkv, dim3(kThreads), 0, stream, q, k, v, g,
                       a.lse, dl, (float*)a.dk, (float*)a.dv, s, b, hp, hkvp, scale);
  }
  return hipGetLastError();
}

}  // namespace

int64_t attn_bwd_f32_workspace_size(const AttnBwdArgs& a) {
  return (a.b * a.hp * a.s * 4 + 255) / 256 * 256;
}

hipError_t launch_attn_bwd_f32(const AttnBwdArgs& a, hipStream_t stream) {
  if (a.dq_ranks || a.dk_ranks || a.dv_ranks) return hipErrorInvalidValue;
  if (a.d == 64) return launch_d<64>(a, stream);
  if (a.d == 128) return launch_d<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ulys
