// abi.cpp -- the extern "C" entry points declared in include/ulysses.h.
//
// Each entry validates everything on the host (sizes, divisibility, dtype,
// alignment, aliasing) and returns before touching the HIP runtime when an
// argument is bad; only then does it enqueue its kernel on the caller's
// stream.  Nothing here allocates, synchronizes or keeps state.
#include <stdint.h>
#include <string.h>

#include "internal.h"
#include "ulysses.h"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 40;    // per-argument sanity bound
constexpr int64_t kMaxBytes = int64_t(1) << 46;  // 64 TiB: any real buffer is smaller

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

int elt_size(int32_t dtype) {
  if (dtype == ULYS_F32) return 4;
  if (dtype == ULYS_BF16) return 2;
  return 0;
}

// Product of positive sizes with an overflow guard; -1 when too large.
int64_t checked_product(std::initializer_list<int64_t> xs) {
  int64_t r = 1;
  for (int64_t x : xs) {
    if (x <= 0 || x > kMaxDim) return -1;
    if (r > kMaxBytes / x) return -1;
    r *= x;
  }
  return r;
}

// KV heads in one rank's share: h_kv/P, or 1 when there are fewer KV heads
// than ranks and each is replicated to the ranks whose query heads use it
// (then rank r's query heads all map to KV head floor(r*h_kv/P)).
int64_t kv_per_rank(int64_t h_kv, int64_t P) { return h_kv % P == 0 ? h_kv / P : 1; }

// Shared validation of the two layout entry points.
int check_layout(const void* in, const void* out, int64_t s, int64_t b, int64_t h, int64_t d_h,
                 int32_t P, int32_t dtype, int64_t* bytes) {
  if (!in || !out) return ULYS_ERR_NULL;
  if (s <= 0 || b <= 0 || h <= 0 || d_h <= 0 || P <= 0) return ULYS_ERR_DIM;
  if (s > kMaxDim || b > kMaxDim || h > kMaxDim || d_h > kMaxDim) return ULYS_ERR_DIM;
  if (s % P != 0 || h % P != 0) return ULYS_ERR_DIVISIBILITY;
  const int elt = elt_size(dtype);
  if (elt == 0) return ULYS_ERR_UNSUPPORTED;
  const int64_t n = checked_product({s / P, b, h, d_h, (int64_t)elt});
  if (n < 0) return ULYS_ERR_DIM;
  if (!aligned16(in) || !aligned16(out)) return ULYS_ERR_ALIGNMENT;
  if (overlaps(in, n, out, n)) return ULYS_ERR_ALIAS;
  *bytes = n;
  return ULYS_OK;
}

}  // namespace

extern "C" {

int ulys_pack_seq2head(const void* x, void* y, int64_t s, int64_t b, int64_t h, int64_t d_h,
                       int32_t P, int32_t dtype, void* stream) {
  int64_t bytes = 0;
  const int rc = check_layout(x, y, s, b, h, d_h, P, dtype, &bytes);
  if (rc != ULYS_OK) return rc;
  const int64_t run = (h / P) * d_h * elt_size(dtype);
  // x is [sl*b][P] runs, y is [P][sl*b] runs
  const hipError_t e = ulys::launch_transpose_runs(x, y, (uint64_t)((s / P) * b), (uint64_t)P,
                                                   (uint64_t)run, (hipStream_t)stream);
  return e == hipSuccess ? ULYS_OK : ULYS_ERR_HIP;
}

int ulys_unpack_head2seq(const void* y, void* x, int64_t s, int64_t b, int64_t h, int64_t d_h,
                         int32_t P, int32_t dtype, void* stream) {
  int64_t bytes = 0;
  const int rc = check_layout(y, x, s, b, h, d_h, P, dtype, &bytes);
  if (rc != ULYS_OK) return rc;
  const int64_t run = (h / P) * d_h * elt_size(dtype);
  // y is [P][sl*b] runs, x is [sl*b][P] runs
  const hipError_t e = ulys::launch_transpose_runs(y, x, (uint64_t)P, (uint64_t)((s / P) * b),
                                                   (uint64_t)run, (hipStream_t)stream);
  return e == hipSuccess ? ULYS_OK : ULYS_ERR_HIP;
}

}  // extern "C"

namespace {

// Size, divisibility and dtype checks of the attention entry points.
int check_attn_shape(int64_t s, int64_t b, int64_t h, int64_t h_kv, int64_t d_h, int32_t P,
                     int32_t dtype, int64_t* nq, int64_t* nkv, int64_t* nl) {
  if (s <= 0 || b <= 0 || h <= 0 || h_kv <= 0 || d_h <= 0 || P <= 0) return ULYS_ERR_DIM;
  if (s > kMaxDim || b > kMaxDim || h > kMaxDim || h_kv > kMaxDim || d_h > kMaxDim)
    return ULYS_ERR_DIM;
  if (s % P != 0 || h % P != 0 || h % h_kv != 0) return ULYS_ERR_DIVISIBILITY;
  if (h_kv % P != 0 && P % h_kv != 0) return ULYS_ERR_DIVISIBILITY;
  const int elt = elt_size(dtype);
  if (elt == 0) return ULYS_ERR_UNSUPPORTED;
  if (d_h != 64 && d_h != 128) return ULYS_ERR_UNSUPPORTED;
  const int64_t hp = h / P, hkvp = kv_per_rank(h_kv, P);
  *nq = checked_product({s, b, hp, d_h, (int64_t)elt});
  *nkv = checked_product({s, b, hkvp, d_h, (int64_t)elt});
  *nl = checked_product({b, hp, s, (int64_t)sizeof(float)});
  if (*nq < 0 || *nkv < 0 || *nl < 0) return ULYS_ERR_DIM;
  // the kernels index tokens and work items with 32-bit integers
  if (s > 0x7FFFFFFF || b * hp > 0x7FFFFFFF || b * hp * s > (int64_t(1) << 40))
    return ULYS_ERR_DIM;
  // the fp32 kernels put (batch, head) on the grid's second dimension
  if (dtype == ULYS_F32 && b * hp > 65535) return ULYS_ERR_DIM;
  // the bf16 kernels address each tensor with 32-bit byte offsets, up to one
  // 256-row workgroup block past the end (read as zero, stores dropped)
  if (dtype == ULYS_BF16 && (*nq + 256 * b * hp * d_h * 2 >= (int64_t(1) << 31) ||
                             *nkv + 256 * b * hkvp * d_h * 2 >= (int64_t(1) << 31)))
    return ULYS_ERR_DIM;
  return ULYS_OK;
}

ulys::AttnArgs make_args(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t s, int64_t b, int64_t h, int64_t h_kv, int64_t d_h, int32_t P,
                         int32_t causal) {
  ulys::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.s = s;
  a.b = b;
  a.hp = h / P;
  a.hkvp = kv_per_rank(h_kv, P);
  a.d = d_h;
  a.causal = causal != 0;
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  return a;
}

}  // namespace

extern "C" {

int ulys_attn_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t s, int64_t b, int64_t h, int64_t h_kv, int64_t d_h, int32_t P,
                     int32_t causal, int32_t dtype, void* workspace, int64_t workspace_bytes,
                     void* stream) {
  if (!q || !k || !v || !o) return ULYS_ERR_NULL;
  int64_t nq = 0, nkv = 0, nl = 0;
  const int rc = check_attn_shape(s, b, h, h_kv, d_h, P, dtype, &nq, &nkv, &nl);
  if (rc != ULYS_OK) return rc;
  if (workspace && workspace_bytes < 0) return ULYS_ERR_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ULYS_ERR_ALIGNMENT;
  if (lse && !aligned16(lse)) return ULYS_ERR_ALIGNMENT;
  if (workspace && !aligned16(workspace)) return ULYS_ERR_ALIGNMENT;
  if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv))
    return ULYS_ERR_ALIAS;
  if (lse && (overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) ||
              overlaps(lse, nl, v, nkv) || overlaps(lse, nl, o, nq)))
    return ULYS_ERR_ALIAS;
  if (workspace && workspace_bytes > 0) {
    const int64_t w = workspace_bytes;
    if (overlaps(workspace, w, q, nq) || overlaps(workspace, w, k, nkv) ||
        overlaps(workspace, w, v, nkv) || overlaps(workspace, w, o, nq) ||
        (lse && overlaps(workspace, w, lse, nl)))
      return ULYS_ERR_ALIAS;
  }
  ulys::AttnArgs a = make_args(q, k, v, o, lse, s, b, h, h_kv, d_h, P, causal);
  if (workspace && workspace_bytes > 0) {
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
  }
  const hipError_t e = (dtype == ULYS_BF16) ? ulys::launch_attn_bf16(a, (hipStream_t)stream)
                                            : ulys::launch_attn_f32(a, (hipStream_t)stream);
  return e == hipSuccess ? ULYS_OK : ULYS_ERR_HIP;
}

int ulys_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t s,
                  int64_t b, int64_t h, int64_t h_kv, int64_t d_h, int32_t P, int32_t causal,
                  int32_t dtype, void* stream) {
  return ulys_attn_fwd_ws(q, k, v, o, lse, s, b, h, h_kv, d_h, P, causal, dtype, nullptr, 0,
                          stream);
}

int64_t ulys_attn_fwd_workspace_size(int64_t s, int64_t b, int64_t h, int64_t h_kv, int64_t d_h,
                                     int32_t P, int32_t causal, int32_t dtype) {
  int64_t nq = 0, nkv = 0, nl = 0;
  const int rc = check_attn_shape(s, b, h, h_kv, d_h, P, dtype, &nq, &nkv, &nl);
  if (rc != ULYS_OK) return rc;
  if (dtype != ULYS_BF16) return 0;
  const ulys::AttnArgs a = make_args(nullptr, nullptr, nullptr, nullptr, nullptr, s, b, h, h_kv,
                                     d_h, P, causal);
  return ulys::attn_bf16_workspace_size(a);
}

int64_t ulys_attn_bwd_workspace_size(int64_t s, int64_t b, int64_t h, int64_t h_kv, int64_t d_h,
                                     int32_t P, int32_t causal, int32_t dtype) {
  int64_t nq = 0, nkv = 0, nl = 0;
  const int rc = check_attn_shape(s, b, h, h_kv, d_h, P, dtype, &nq, &nkv, &nl);
  if (rc != ULYS_OK) return rc;
  ulys::AttnBwdArgs a;
  a.s = s;
  a.b = b;
  a.hp = h / P;
  a.hkvp = kv_per_rank(h_kv, P);
  a.d = d_h;
  a.causal = causal != 0;
  if (dtype == ULYS_F32) return ulys::attn_bwd_f32_workspace_size(a);
  const int64_t need = ulys::attn_bwd_bf16_workspace_size(a);
  // the kernels address the per-row statistics with 32-bit byte offsets
  if (need >= (int64_t(1) << 31)) return ULYS_ERR_DIM;
  return need;
}

int ulys_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, int64_t s, int64_t b, int64_t h,
                  int64_t h_kv, int64_t d_h, int32_t P, int32_t causal, int32_t dtype,
                  void* workspace, int64_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
    return ULYS_ERR_NULL;
  const int64_t need = ulys_attn_bwd_workspace_size(s, b, h, h_kv, d_h, P, causal, dtype);
  if (need < 0) return (int)need;
  if (workspace_bytes < need) return ULYS_ERR_DIM;
  int64_t nq = 0, nkv = 0, nl = 0;
  const int rc = check_attn_shape(s, b, h, h_kv, d_h, P, dtype, &nq, &nkv, &nl);
  if (rc != ULYS_OK) return rc;
  const void* ins[] = {q, k, v, o, dout, lse};
  const int64_t in_bytes[] = {nq, nkv, nkv, nq, nq, nl};
  void* outs[] = {dq, dk, dv, workspace};
  const int64_t out_bytes[] = {nq, nkv, nkv, need};
  for (const void* p : ins)
    if (!aligned16(p)) return ULYS_ERR_ALIGNMENT;
  for (const void* p : outs)
    if (!aligned16(p)) return ULYS_ERR_ALIGNMENT;
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return ULYS_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return ULYS_ERR_ALIAS;
  }
  ulys::AttnBwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.s = s;
  a.b = b;
  a.hp = h / P;
  a.hkvp = kv_per_rank(h_kv, P);
  a.d = d_h;
  a.causal = causal != 0;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  const hipError_t e = (dtype == ULYS_BF16) ? ulys::launch_attn_bwd_bf16(a, (hipStream_t)stream)
                                            : ulys::launch_attn_bwd_f32(a, (hipStream_t)stream);
  return e == hipSuccess ? ULYS_OK : ULYS_ERR_HIP;
}

int ulys_attn_bwd_push(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* const* dq_ranks,
                       void* const* dk_ranks, void* const* dv_ranks, int32_t rank, int64_t s,
                       int64_t b, int64_t h, int64_t h_kv, int64_t d_h, int32_t P, int32_t causal,
                       int32_t dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq_ranks || !dk_ranks || !dv_ranks ||
      !workspace)
    return ULYS_ERR_NULL;
  const int64_t need = ulys_attn_bwd_workspace_size(s, b, h, h_kv, d_h, P, causal, dtype);
  if (need < 0) return (int)need;
  // the pushing epilogues exist in the bf16 kernels only
  if (dtype != ULYS_BF16) return ULYS_ERR_UNSUPPORTED;
  if (workspace_bytes < need) return ULYS_ERR_DIM;
  int64_t nq = 0, nkv = 0, nl = 0;
  const int rc = check_attn_shape(s, b, h, h_kv, d_h, P, dtype, &nq, &nkv, &nl);
  if (rc != ULYS_OK) return rc;
  // replicated KV heads: the copies' gradients must be summed across ranks
  if (h_kv % P != 0) return ULYS_ERR_UNSUPPORTED;
  if (P > ULYS_MAX_RANKS || rank < 0 || rank >= P) return ULYS_ERR_DIM;
  void* const* tables[] = {dq_ranks, dk_ranks, dv_ranks};
  for (void* const* t : tables)
    for (int32_t r = 0; r < P; ++r) {
      if (!t[r]) return ULYS_ERR_NULL;
      if (!aligned16(t[r])) return ULYS_ERR_ALIGNMENT;
    }
  const void* ins[] = {q, k, v, o, dout, lse, workspace};
  const int64_t in_bytes[] = {nq, nkv, nkv, nq, nq, nl, need};
  for (const void* p : ins)
    if (!aligned16(p)) return ULYS_ERR_ALIGNMENT;
  if (overlaps(workspace, need, q, nq) || overlaps(workspace, need, k, nkv) ||
      overlaps(workspace, need, v, nkv) || overlaps(workspace, need, o, nq) ||
      overlaps(workspace, need, dout, nq) || overlaps(workspace, need, lse, nl))
    return ULYS_ERR_ALIAS;
  // written span of each destination: head group `rank` of every row of a
  // shard of the share's bytes (dQ: nq; dK, dV: nkv)
  const int64_t run_q = (h / P) * d_h * 2, run_kv = (h_kv / P) * d_h * 2;
  const int64_t span[] = {nq - (int64_t)(P - 1) * run_q, nkv - (int64_t)(P - 1) * run_kv,
                          nkv - (int64_t)(P - 1) * run_kv};
  const int64_t run[] = {run_q, run_kv, run_kv};
  for (int t = 0; t < 3; ++t)
    for (int32_t r = 0; r < P; ++r) {
      const char* lo = static_cast<const char*>(tables[t][r]) + (int64_t)rank * run[t];
      for (int i = 0; i < 7; ++i)
        if (overlaps(lo, span[t], ins[i], in_bytes[i])) return ULYS_ERR_ALIAS;
      for (int t2 = 0; t2 <= t; ++t2)
        for (int32_t r2 = 0; r2 < (t2 == t ? r : P); ++r2)
          if (overlaps(lo, span[t],
                       static_cast<const char*>(tables[t2][r2]) + (int64_t)rank * run[t2],
                       span[t2]))
            return ULYS_ERR_ALIAS;
    }
  ulys::AttnBwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = a.dk = a.dv = nullptr;
  a.s = s;
  a.b = b;
  a.hp = h / P;
  a.hkvp = h_kv / P;
  a.d = d_h;
  a.causal = causal != 0;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.dq_ranks = dq_ranks;
  a.dk_ranks = dk_ranks;
  a.dv_ranks = dv_ranks;
  a.ranks = P;
  a.rank = rank;
  const hipError_t e = ulys::launch_attn_bwd_bf16(a, (hipStream_t)stream);
  return e == hipSuccess ? ULYS_OK : ULYS_ERR_HIP;
}

// Shared validation of the two KV layout entry points; *rep is set when the
// heads are replicated (h_kv < P), else the plain layout applies.
static int check_layout_kv(const void* in, const void* out, int64_t s, int64_t b, int64_t h_kv,
                           int64_t d_h, int32_t P, int32_t dtype, int* rep, int64_t* shard,
                           int64_t* blocks) {
  if (!in || !out) return ULYS_ERR_NULL;
  if (s <= 0 || b <= 0 || h_kv <= 0 || d_h <= 0 || P <= 0) return ULYS_ERR_DIM;
  if (s > kMaxDim || b > kMaxDim || h_kv > kMaxDim || d_h > kMaxDim) return ULYS_ERR_DIM;
  if (s % P != 0 || (h_kv % P != 0 && P % h_kv != 0)) return ULYS_ERR_DIVISIBILITY;
  const int elt = elt_size(dtype);
  if (elt == 0) return ULYS_ERR_UNSUPPORTED;
  *rep = h_kv % P != 0;
  *shard = checked_product({s / P, b, h_kv, d_h, (int64_t)elt});
  *blocks = checked_product({(int64_t)P, s / P, b, kv_per_rank(h_kv, P), d_h, (int64_t)elt});
  if (*shard < 0 || *blocks < 0) return ULYS_ERR_DIM;
  // the replication kernels index with 32-bit integers
  if (*rep && *blocks / elt >= (int64_t(1) << 31)) return ULYS_ERR_DIM;
  if (!aligned16(in) || !aligned16(out)) return ULYS_ERR_ALIGNMENT;
  return ULYS_OK;
}

int ulys_pack_seq2head_kv(const void* x, void* y, int64_t s, int64_t b, int64_t h_kv,
                          int64_t d_h, int32_t P, int32_t dtype, void* stream) {
  int rep = 0;
  int64_t shard = 0, blocks = 0;
  const int rc = check_layout_kv(x, y, s, b, h_kv, d_h, P, dtype, &rep, &shard, &blocks);
  if (rc != ULYS_OK) return rc;
  if (overlaps(x, shard, y, blocks)) return ULYS_ERR_ALIAS;
  if (!rep) return ulys_pack_seq2head(x, y, s, b, h_kv, d_h, P, dtype, stream);
  const hipError_t e = ulys::launch_replicate_runs(
      x, y, (uint32_t)((s / P) * b), (uint32_t)h_kv, (uint32_t)P,
      (uint32_t)(d_h * elt_size(dtype)), (hipStream_t)stream);
  return e == hipSuccess ? ULYS_OK : ULYS_ERR_HIP;
}

int ulys_unpack_head2seq_kv(const void* y, void* x, int64_t s, int64_t b, int64_t h_kv,
                            int64_t d_h, int32_t P, int32_t dtype, void* stream) {
  int rep = 0;
  int64_t shard = 0, blocks = 0;
  const int rc = check_layout_kv(y, x, s, b, h_kv, d_h, P, dtype, &rep, &shard, &blocks);
  if (rc != ULYS_OK) return rc;
  if (overlaps(y, blocks, x, shard)) return ULYS_ERR_ALIAS;
  if (!rep) return ulys_unpack_head2seq(y, x, s, b, h_kv, d_h, P, dtype, stream);
  const hipError_t e = ulys::launch_sum_runs(y, x, (uint32_t)((s / P) * b), (uint32_t)h_kv,
                                             (uint32_t)P, (uint32_t)(d_h * elt_size(dtype)),
                                             elt_size(dtype), (hipStream_t)stream);
  return e == hipSuccess ? ULYS_OK : ULYS_ERR_HIP;
}

int ulys_pack_seq2head_qkv(const void* xq, const void* xk, const void* xv, void* yq, void* yk,
                           void* yv, int64_t s, int64_t b, int64_t h, int64_t h_kv, int64_t d_h,
                           int32_t P, int32_t dtype, void* stream) {
  int64_t nq = 0;
  int rc = check_layout(xq, yq, s, b, h, d_h, P, dtype, &nq);
  if (rc != ULYS_OK) return rc;
  int rep = 0;
  int64_t shard_kv = 0, blocks_kv = 0;
  rc = check_layout_kv(xk, yk, s, b, h_kv, d_h, P, dtype, &rep, &shard_kv, &blocks_kv);
  if (rc != ULYS_OK) return rc;
  rc = check_layout_kv(xv, yv, s, b, h_kv, d_h, P, dtype, &rep, &shard_kv, &blocks_kv);
  if (rc != ULYS_OK) return rc;
  const void* ins[] = {xq, xk, xv};
  const int64_t in_bytes[] = {nq, shard_kv, shard_kv};
  void* outs[] = {yq, yk, yv};
  const int64_t out_bytes[] = {nq, blocks_kv, blocks_kv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return ULYS_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return ULYS_ERR_ALIAS;
  }
  const int elt = elt_size(dtype);
  const int64_t hkv_runs = rep ? h_kv : P;  // input runs per token-batch row
  const int64_t run_q = (h / P) * d_h * elt, run_kv = kv_per_rank(h_kv, P) * d_h * elt;
  const int64_t vecs = (nq + 2 * blocks_kv) / 16;
  if (run_q % 16 != 0 || run_kv % 16 != 0 || vecs >= (int64_t(1) << 31)) {
    // not a whole number of 16-byte vectors per run, or too large for one
    // launch's 32-bit indices: the three packs one after another
    rc = ulys_pack_seq2head(xq, yq, s, b, h, d_h, P, dtype, stream);
    if (rc == ULYS_OK) rc = ulys_pack_seq2head_kv(xk, yk, s, b, h_kv, d_h, P, dtype, stream);
    if (rc == ULYS_OK) rc = ulys_pack_seq2head_kv(xv, yv, s, b, h_kv, d_h, P, dtype, stream);
    return rc;
  }
  const void* in3[3] = {xq, xk, xv};
  void* out3[3] = {yq, yk, yv};
  const uint32_t cols[3] = {(uint32_t)P, (uint32_t)hkv_runs, (uint32_t)hkv_runs};
  const uint32_t runs[3] = {(uint32_t)run_q, (uint32_t)run_kv, (uint32_t)run_kv};
  const hipError_t e = ulys::launch_pack_qkv(in3, out3, (uint32_t)((s / P) * b), (uint32_t)P, cols,
                                             runs, (hipStream_t)stream);
  return e == hipSuccess ? ULYS_OK : ULYS_ERR_HIP;
}

// Shared validation of the two push entry points: `local` is the rank's own
// tensor (x [sl,b,h,d] or o [s,b,hp,d]), `remote` the P destination pointers;
// the bytes each destination receives are checked against `local` and
// against every other destination's.
static int check_push(const void* local, void* const* remote, int32_t rank, int64_t s, int64_t b,
                      int64_t h, int64_t d_h, int32_t P, int32_t dtype, bool seq2head) {
  if (!local || !remote) return ULYS_ERR_NULL;
  if (s <= 0 || b <= 0 || h <= 0 || d_h <= 0 || P <= 0) return ULYS_ERR_DIM;
  if (s > kMaxDim || b > kMaxDim || h > kMaxDim || d_h > kMaxDim) return ULYS_ERR_DIM;
  if (P > ULYS_MAX_RANKS || rank < 0 || rank >= P) return ULYS_ERR_DIM;
  if (s % P != 0 || h % P != 0) return ULYS_ERR_DIVISIBILITY;
  const int elt = elt_size(dtype);
  if (elt == 0) return ULYS_ERR_UNSUPPORTED;
  const int64_t n = checked_product({s / P, b, h, d_h, (int64_t)elt});  // shard = share bytes
  if (n < 0 || n / elt >= (int64_t(1) << 31)) return ULYS_ERR_DIM;
  if (!aligned16(local)) return ULYS_ERR_ALIGNMENT;
  for (int32_t r = 0; r < P; ++r) {
    if (!remote[r]) return ULYS_ERR_NULL;
    if (!aligned16(remote[r])) return ULYS_ERR_ALIGNMENT;
  }
  // the byte range this call writes in destination r
  const int64_t blk = n / P;
  auto written = [&](int32_t r, const char** lo, int64_t* len) {
    if (seq2head) {  // rows [rank*sl, (rank+1)*sl) of share r
      *lo = static_cast<const char*>(remote[r]) + (int64_t)rank * blk;
      *len = blk;
    } else {  // head group `rank` of every row of shard r: the span from its first to last run
      const int64_t run = (h / P) * d_h * elt;
      *lo = static_cast<const char*>(remote[r]) + (int64_t)rank * run;
      *len = n - (int64_t)(P - 1) * run;
    }
  };
  for (int32_t r = 0; r < P; ++r) {
    const char* lo = nullptr;
    int64_t len = 0;
    written(r, &lo, &len);
    if (overlaps(lo, len, local, n)) return ULYS_ERR_ALIAS;
    for (int32_t q = 0; q < r; ++q) {
      const char* lo2 = nullptr;
      int64_t len2 = 0;
      written(q, &lo2, &len2);
      if (overlaps(lo, len, lo2, len2)) return ULYS_ERR_ALIAS;
    }
  }
  return ULYS_OK;
}

int ulys_seq2head_push(const void* x, void* const* y_ranks, int32_t rank, int64_t s, int64_t b,
                       int64_t h, int64_t d_h, int32_t P, int32_t dtype, void* stream) {
  const int rc = check_push(x, y_ranks, rank, s, b, h, d_h, P, dtype, true);
  if (rc != ULYS_OK) return rc;
  const hipError_t e = ulys::launch_push(x, y_ranks, (uint32_t)((s / P) * b), (uint32_t)P,
                                         (uint32_t)rank, (uint32_t)((h / P) * d_h * elt_size(dtype)),
                                         true, (hipStream_t)stream);
  return e == hipSuccess ? ULYS_OK : ULYS_ERR_HIP;
}

int ulys_head2seq_push(const void* o, void* const* x_ranks, int32_t rank, int64_t s, int64_t b,
                       int64_t h, int64_t d_h, int32_t P, int32_t dtype, void* stream) {
  const int rc = check_push(o, x_ranks, rank, s, b, h, d_h, P, dtype, false);
  if (rc != ULYS_OK) return rc;
  const hipError_t e = ulys::launch_push(o, x_ranks, (uint32_t)((s / P) * b), (uint32_t)P,
                                         (uint32_t)rank, (uint32_t)((h / P) * d_h * elt_size(dtype)),
                                         false, (hipStream_t)stream);
  return e == hipSuccess ? ULYS_OK : ULYS_ERR_HIP;
}

int ulys_attn_fwd_push(const void* q, const void* k, const void* v, void* const* x_ranks,
                       int32_t rank, float* lse, int64_t s, int64_t b, int64_t h, int64_t h_kv,
                       int64_t d_h, int32_t P, int32_t causal, int32_t dtype, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !x_ranks) return ULYS_ERR_NULL;
  int64_t nq = 0, nkv = 0, nl = 0;
  const int rc = check_attn_shape(s, b, h, h_kv, d_h, P, dtype, &nq, &nkv, &nl);
  if (rc != ULYS_OK) return rc;
  if (dtype != ULYS_BF16) return ULYS_ERR_UNSUPPORTED;
  if (P > ULYS_MAX_RANKS || rank < 0 || rank >= P) return ULYS_ERR_DIM;
  if (workspace && workspace_bytes < 0) return ULYS_ERR_DIM;
  for (int32_t r = 0; r < P; ++r)
    if (!x_ranks[r]) return ULYS_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return ULYS_ERR_ALIGNMENT;
  if ((lse && !aligned16(lse)) || (workspace && !aligned16(workspace))) return ULYS_ERR_ALIGNMENT;
  for (int32_t r = 0; r < P; ++r)
    if (!aligned16(x_ranks[r])) return ULYS_ERR_ALIGNMENT;
  // a destination shard [s/P, b, h, d_h] has the share's bytes; this call
  // writes head group `rank` of each of its rows: the span from the first
  // to the last such run
  const int64_t n = nq;
  const int64_t run = (h / P) * d_h * 2;
  const int64_t span = n - (int64_t)(P - 1) * run;
  const int64_t w = (workspace && workspace_bytes > 0) ? workspace_bytes : 0;
  if (lse && (overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) || overlaps(lse, nl, v, nkv)))
    return ULYS_ERR_ALIAS;
  if (w && (overlaps(workspace, w, q, nq) || overlaps(workspace, w, k, nkv) ||
            overlaps(workspace, w, v, nkv) || (lse && overlaps(workspace, w, lse, nl))))
    return ULYS_ERR_ALIAS;
  for (int32_t r = 0; r < P; ++r) {
    const char* lo = static_cast<const char*>(x_ranks[r]) + (int64_t)rank * run;
    if (overlaps(lo, span, q, nq) || overlaps(lo, span, k, nkv) || overlaps(lo, span, v, nkv) ||
        (lse && overlaps(lo, span, lse, nl)) || (w && overlaps(lo, span, workspace, w)))
      return ULYS_ERR_ALIAS;
    for (int32_t j = 0; j < r; ++j)
      if (overlaps(lo, span, static_cast<const char*>(x_ranks[j]) + (int64_t)rank * run, span))
        return ULYS_ERR_ALIAS;
  }
  ulys::AttnArgs a = make_args(q, k, v, nullptr, lse, s, b, h, h_kv, d_h, P, causal);
  if (w) {
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
  }
  a.o_ranks = x_ranks;
  a.ranks = P;
  a.rank = rank;
  const hipError_t e = ulys::launch_attn_bf16(a, (hipStream_t)stream);
  return e == hipSuccess ? ULYS_OK : ULYS_ERR_HIP;
}

int ulys_attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                    void* o, float* lse, int64_t s, int64_t b, int64_t hp, int64_t d_h,
                    int32_t dtype, void* stream) {
  if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse) return ULYS_ERR_NULL;
  if (s <= 0 || b <= 0 || hp <= 0 || d_h <= 0) return ULYS_ERR_DIM;
  if (s > kMaxDim || b > kMaxDim || hp > kMaxDim || d_h > kMaxDim) return ULYS_ERR_DIM;
  const int elt = elt_size(dtype);
  if (elt == 0 || (d_h != 64 && d_h != 128)) return ULYS_ERR_UNSUPPORTED;
  const int64_t no = checked_product({s, b, hp, d_h, (int64_t)elt});
  const int64_t nl = checked_product({s, b, hp, (int64_t)sizeof(float)});
  if (no < 0 || nl < 0) return ULYS_ERR_DIM;
  // one 16-byte vector per thread, 32-bit indices
  if (no / 16 >= (int64_t(1) << 31)) return ULYS_ERR_DIM;
  const void* ptrs[] = {o_a, lse_a, o_b, lse_b, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ULYS_ERR_ALIGNMENT;
  // o may be exactly o_a and lse exactly lse_a (in-place accumulation);
  // any other overlap between an output and an input or the other output is
  // rejected
  const void* ins[] = {o_a, lse_a, o_b, lse_b};
  const int64_t in_bytes[] = {no, nl, no, nl};
  const void* outs[] = {o, lse};
  const int64_t out_bytes[] = {no, nl};
  const void* same[] = {o_a, lse_a};
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 4; ++j)
      if (!(j == i && outs[i] == same[i]) && overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j]))
        return ULYS_ERR_ALIAS;
  if (overlaps(o, no, lse, nl)) return ULYS_ERR_ALIAS;
  const hipError_t e = ulys::launch_attn_merge(o_a, lse_a, o_b, lse_b, o, lse, (uint32_t)s,
                                               (uint32_t)b, (uint32_t)hp,
                                               (uint32_t)(d_h * elt), elt, (hipStream_t)stream);
  return e == hipSuccess ? ULYS_OK : ULYS_ERR_HIP;
}

const char* ulys_status_string(int status) {
  switch (status) {
    case ULYS_OK: return "ok";
    case ULYS_ERR_NULL: return "a required pointer is NULL";
    case ULYS_ERR_DIM: return "a size is non-positive or too large";
    case ULYS_ERR_DIVISIBILITY:
      return "P must divide s and h, P and h_kv must divide one another, and h_kv must divide h";
    case ULYS_ERR_UNSUPPORTED: return "unsupported dtype or head size";
    case ULYS_ERR_ALIGNMENT: return "a pointer is not 16-byte aligned";
    case ULYS_ERR_ALIAS: return "an output overlaps an input or another output";
    case ULYS_ERR_HIP: return "the HIP runtime reported a launch error";
    default: return "unknown status";
  }
}

int ulys_abi_version(void) { return ULYS_ABI_VERSION; }

}  // extern "C"
