/*
 * abi_chain.c -- the per-rank path driven from plain C through the C ABI of
 * include/ulysses.h, with no Python and no torch: HIP runtime calls for
 * device memory, the library's entry points for every step, and the CPU
 * oracle (oracle/ulys_oracle.c, test infrastructure) for the expected values.
 *
 * One layer of P emulated ranks on one GPU ("02 · DeepSpeed-Ulysses" §2; the
 * DSU page's core design steps 3-5): every rank packs its sequence shard of
 * Q, K and V (ulys_pack_seq2head), block r of every sender is routed to rank
 * r (device-to-device copies stand in for the all-to-all), every rank runs
 * the attention over the whole sequence for its heads (ulys_attn_fwd), the
 * output goes back by sequence segment and is unpacked
 * (ulys_unpack_head2seq).  Checked: every pack bit for bit against orc_pack,
 * the layer's output against orc_attn of unsharded attention over all heads
 * (max-abs 2e-2, bf16 inputs), and a few status codes.
 *
 * Inputs: uniform in [-2, 2) from SplitMix64 (Steele, Lea & Flood, OOPSLA
 * 2014; draw i of stream seed = mix(seed + (i + 1) * 0x9E3779B97F4A7C15)),
 * rounded to bf16 (nearest, ties to even).
 *
 * Usage: abi_chain [s b h h_kv d P causal]; exit status 0 when every check
 * passes.  Build: gcc -std=c11 -D__HIP_PLATFORM_AMD__ -I include
 * -I /opt/rocm/include abi_chain.c -L <dir of libulysses.so> -lulysses
 * -L <dir of libulys_oracle.so> -lulys_oracle -L /opt/rocm/lib -lamdhip64.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ulysses.h"

/* the oracle's entry points used here (it has no header of its own) */
int orc_pack(const void *x, void *y, int64_t s, int64_t b, int64_t h, int64_t d, int64_t P,
             int64_t elt);
int orc_attn(const void *q, const void *k, const void *v, double *o, double *lse, int64_t s,
             int64_t b, int64_t h, int64_t h_kv, int64_t d, int64_t P, int causal, int dtype,
             int nthreads);

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static float bf16_to_f32(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static void fill(uint16_t *a, int64_t n, uint64_t seed) {
  for (int64_t i = 0; i < n; ++i) {
    const double u = (double)(mix64(seed + (uint64_t)(i + 1) * 0x9E3779B97F4A7C15ull) >> 11) *
                     (1.0 / 9007199254740992.0);
    a[i] = bf16_rne((float)(4.0 * u - 2.0));
  }
}

static int failures = 0;

#define HIP_OK(call)                                                              \
  do {                                                                            \
    const hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s:%d: %s -> %s\n", __FILE__, __LINE__, #call,            \
              hipGetErrorString(e_));                                             \
      exit(2);                                                                    \
    }                                                                             \
  } while (0)

static void expect(int cond, const char *what) {
  if (!cond) {
    fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

/* seq->head exchange of one tensor with `heads` heads: pack every rank's shard
 * of the global [s, b, heads, d] host array, check each pack against the
 * oracle, route block r of sender j to rows [j*sl, (j+1)*sl) of rank r's
 * share.  Returns the P device shares [s, b, heads/P, d]. */
static uint16_t **exchange(const uint16_t *glob, int64_t s, int64_t b, int64_t heads, int64_t d,
                           int P) {
  const int64_t sl = s / P, hp = heads / P;
  const int64_t shard = sl * b * heads * d, block = sl * b * hp * d;
  uint16_t **share = (uint16_t **)calloc((size_t)P, sizeof(uint16_t *));
  for (int r = 0; r < P; ++r) HIP_OK(hipMalloc((void **)&share[r], (size_t)(s * b * hp * d * 2)));
  uint16_t *x_d, *y_d;
  HIP_OK(hipMalloc((void **)&x_d, (size_t)(shard * 2)));
  HIP_OK(hipMalloc((void **)&y_d, (size_t)(shard * 2)));
  uint16_t *y_h = (uint16_t *)malloc((size_t)(shard * 2));
  uint16_t *y_ref = (uint16_t *)malloc((size_t)(shard * 2));
  for (int j = 0; j < P; ++j) {
    const uint16_t *x_h = glob + (int64_t)j * shard;
    HIP_OK(hipMemcpy(x_d, x_h, (size_t)(shard * 2), hipMemcpyHostToDevice));
    const int rc = ulys_pack_seq2head(x_d, y_d, s, b, heads, d, P, ULYS_BF16, NULL);
    expect(rc == ULYS_OK, "ulys_pack_seq2head status");
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(y_h, y_d, (size_t)(shard * 2), hipMemcpyDeviceToHost));
    expect(orc_pack(x_h, y_ref, s, b, heads, d, P, 2) == 0, "orc_pack status");
    expect(memcmp(y_h, y_ref, (size_t)(shard * 2)) == 0, "pack equals the oracle bit for bit");
    for (int r = 0; r < P; ++r)
      HIP_OK(hipMemcpy(share[r] + (int64_t)j * block, y_d + (int64_t)r * block,
                       (size_t)(block * 2), hipMemcpyDeviceToDevice));
  }
  free(y_h);
  free(y_ref);
  HIP_OK(hipFree(x_d));
  HIP_OK(hipFree(y_d));
  return share;
}

int main(int argc, char **argv) {
  int64_t s = 512, b = 2, h = 8, h_kv = 4, d = 128;
  int P = 4, causal = 1;
  if (argc == 8) {
    s = atoll(argv[1]);
    b = atoll(argv[2]);
    h = atoll(argv[3]);
    h_kv = atoll(argv[4]);
    d = atoll(argv[5]);
    P = atoi(argv[6]);
    causal = atoi(argv[7]);
  }
  const int64_t sl = s / P, hp = h / P;
  printf("abi_chain: s=%lld b=%lld h=%lld h_kv=%lld d=%lld P=%d causal=%d\n", (long long)s,
         (long long)b, (long long)h, (long long)h_kv, (long long)d, P, causal);
  fflush(stdout);
  expect(ulys_abi_version() == ULYS_ABI_VERSION, "ulys_abi_version");

  const int64_t nq = s * b * h * d, nkv = s * b * h_kv * d;
  uint16_t *qg = (uint16_t *)malloc((size_t)(nq * 2));
  uint16_t *kg = (uint16_t *)malloc((size_t)(nkv * 2));
  uint16_t *vg = (uint16_t *)malloc((size_t)(nkv * 2));
  fill(qg, nq, 501);
  fill(kg, nkv, 502);
  fill(vg, nkv, 503);

  uint16_t **qs = exchange(qg, s, b, h, d, P);
  uint16_t **ks = exchange(kg, s, b, h_kv, d, P);
  uint16_t **vs = exchange(vg, s, b, h_kv, d, P);

  /* every rank's attention over the whole sequence for its heads */
  uint16_t **os = (uint16_t **)calloc((size_t)P, sizeof(uint16_t *));
  for (int r = 0; r < P; ++r) {
    HIP_OK(hipMalloc((void **)&os[r], (size_t)(s * b * hp * d * 2)));
    const int rc = ulys_attn_fwd(qs[r], ks[r], vs[r], os[r], NULL, s, b, h, h_kv, d, P, causal,
                                 ULYS_BF16, NULL);
    expect(rc == ULYS_OK, "ulys_attn_fwd status");
  }
  /* a rejected call launches nothing and says why */
  expect(ulys_attn_fwd(qs[0], ks[0], vs[0], os[0], NULL, s + 1, b, h, h_kv, d, P, causal,
                       ULYS_BF16, NULL) == ULYS_ERR_DIVISIBILITY,
         "s not divisible by P is refused");
  expect(ulys_attn_fwd(qs[0], ks[0], vs[0], qs[0], NULL, s, b, h, h_kv, d, P, causal, ULYS_BF16,
                       NULL) == ULYS_ERR_ALIAS,
         "an output over an input is refused");

  /* head->seq: rank j receives segment j of every rank's output, in rank
   * order, and unpacks it into its [sl, b, h, d] output shard */
  const int64_t block = sl * b * hp * d, shard = sl * b * h * d;
  uint16_t *recv_d, *x_d;
  HIP_OK(hipMalloc((void **)&recv_d, (size_t)(shard * 2)));
  HIP_OK(hipMalloc((void **)&x_d, (size_t)(shard * 2)));
  uint16_t *out = (uint16_t *)malloc((size_t)(nq * 2));
  for (int j = 0; j < P; ++j) {
    for (int r = 0; r < P; ++r)
      HIP_OK(hipMemcpy(recv_d + (int64_t)r * block, os[r] + (int64_t)j * block,
                       (size_t)(block * 2), hipMemcpyDeviceToDevice));
    const int rc = ulys_unpack_head2seq(recv_d, x_d, s, b, h, d, P, ULYS_BF16, NULL);
    expect(rc == ULYS_OK, "ulys_unpack_head2seq status");
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(out + (int64_t)j * shard, x_d, (size_t)(shard * 2), hipMemcpyDeviceToHost));
  }

  /* the layer's output against unsharded attention over all heads */
  double *o_ref = (double *)malloc((size_t)(nq * sizeof(double)));
  double *lse_ref = (double *)malloc((size_t)(b * h * s * sizeof(double)));
  expect(orc_attn(qg, kg, vg, o_ref, lse_ref, s, b, h, h_kv, d, 1, causal, 1, 8) == 0,
         "orc_attn status");
  double err = 0.0;
  for (int64_t i = 0; i < nq; ++i) {
    const double e = fabs((double)bf16_to_f32(out[i]) - o_ref[i]);
    if (!(e <= err)) err = e; /* also catches NaN */
  }
  printf("abi_chain: max |O - O_ref| = %.3e over %lld elements\n", err, (long long)nq);
  expect(err <= 2e-2, "layer output within 2e-2 of the oracle");

  for (int r = 0; r < P; ++r) {
    HIP_OK(hipFree(qs[r]));
    HIP_OK(hipFree(ks[r]));
    HIP_OK(hipFree(vs[r]));
    HIP_OK(hipFree(os[r]));
  }
  HIP_OK(hipFree(recv_d));
  HIP_OK(hipFree(x_d));
  free(qs);
  free(ks);
  free(vs);
  free(os);
  free(qg);
  free(kg);
  free(vg);
  free(out);
  free(o_ref);
  free(lse_ref);
  printf("abi_chain: %s\n", failures ? "FAILED" : "ok");
  return failures ? 1 : 0;
}
