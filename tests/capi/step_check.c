/* The fused step from plain C on the GPU, through the C ABI only: zero_adam_shard_step on device
 * buffers must equal zero_reduce_shard (device) followed by zero_host_adam_step (host) on the same
 * inputs, bit for bit: master, m, v and the bf16 slot. Then the clipped path with nothing read
 * back between its calls (zero_shard_sqnorm, zero_clip_scale, zero_adam_shard_step_dev_scale):
 * the device's grad scale must equal C's own double evaluation of the clip rule on the device's
 * norm, and the update must equal the host update with that scale; so must the same update with
 * t on the device (zero_adam_shard_step_dev_t), which also advances the counter. Last, the reduce
 * pass with no workspace (zero_reduce_shard_static) against the one with a caller's partials.
 * The offloaded step (zero_offload_step: host state, pinned staging, the caller's four events) must
 * equal the fused device step too, with the gradient chunks copied from device staging and with
 * the reduce kernel writing them into pinned host memory; pageable memory for the latter must be
 * refused before anything is enqueued. And the ZeRO-3 gather (zero_gather_params) of a range across
 * the replica buffers taken as rank shards must equal the host's concatenation of them, and the
 * fused step with all its arrays in one arena (zero_arena_layout, zero_arena_alloc) must equal the
 * step on separate allocations. Exits 0 when all match. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zero_shard.h"

#define N 100003u /* several tiles and a ragged end */
#define R 3u

static uint64_t state = 0x9e3779b97f4a7c15ull;
static float uniform(void) { /* [-1, 1), 24 random bits */
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((int32_t)(state >> 40) - (1 << 23)) / (float)(1 << 23);
}

#define HIP(x)                                                                  \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      return 2;                                                                 \
    }                                                                           \
  } while (0)
#define ZS(x)                                                                        \
  do {                                                                               \
    zero_status s_ = (x);                                                            \
    if (s_ != ZERO_OK) {                                                             \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, zero_status_str(s_),   \
              zero_last_error());                                                    \
      return 2;                                                                      \
    }                                                                                \
  } while (0)

static uint16_t bf16_trunc(float x) { /* an input recipe: replicas as truncated fp32 draws */
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}

int main(void) {
  static uint16_t reps[R][N], out_dev[N], out_host[N];
  static float p0[N], m0[N], v0[N], p_dev[N], m_dev[N], v_dev[N], p_host[N], m_host[N], v_host[N], g[N],
      g2[N];
  void* d_reps[R];
  const void* d_rep_ptrs[R];
  float *d_p, *d_m, *d_v, *d_g;
  uint16_t* d_out;
  zero_grad_src src;
  zero_adam_hparams hp;
  uint32_t i, k, bad = 0;
  const float gs = 0.5f;

  for (k = 0; k < R; ++k)
    for (i = 0; i < N; ++i) reps[k][i] = bf16_trunc(uniform() * 1e-3f);
  for (i = 0; i < N; ++i) {
    p0[i] = uniform() * 0.02f;
    m0[i] = uniform() * 1e-4f;
    v0[i] = (uniform() + 1.0f) * 1e-8f;
  }
  for (k = 0; k < R; ++k) {
    HIP(hipMalloc(&d_reps[k], N * 2));
    HIP(hipMemcpy(d_reps[k], reps[k], N * 2, hipMemcpyHostToDevice));
    d_rep_ptrs[k] = d_reps[k];
  }
  HIP(hipMalloc((void**)&d_p, N * 4));
  HIP(hipMalloc((void**)&d_m, N * 4));
  HIP(hipMalloc((void**)&d_v, N * 4));
  HIP(hipMalloc((void**)&d_g, N * 4));
  HIP(hipMalloc((void**)&d_out, N * 2));
  HIP(hipMemcpy(d_p, p0, N * 4, hipMemcpyHostToDevice));
  HIP(hipMemcpy(d_m, m0, N * 4, hipMemcpyHostToDevice));
  HIP(hipMemcpy(d_v, v0, N * 4, hipMemcpyHostToDevice));

  src.ptrs = d_rep_ptrs;
  src.count = R;
  src.dtype = ZERO_BF16;
  memset(&hp, 0, sizeof hp);
  hp.lr = 1e-3; hp.beta1 = 0.9; hp.beta2 = 0.999; hp.eps = 1e-8; hp.weight_decay = 0.01;
  hp.wd_mode = ZERO_ADAMW; hp.step = 4;

  /* device: fused step; and the reduce pass alone into d_g */
  ZS(zero_adam_shard_step(&src, N, gs, d_p, d_m, d_v, &hp, d_out, ZERO_BF16, NULL, NULL));
  ZS(zero_reduce_shard(&src, N, d_g, NULL, NULL, 1.0, NULL));
  HIP(hipDeviceSynchronize());
  HIP(hipMemcpy(p_dev, d_p, N * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(m_dev, d_m, N * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(v_dev, d_v, N * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(out_dev, d_out, N * 2, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(g, d_g, N * 4, hipMemcpyDeviceToHost));

  /* host: the same update on the reduced gradient */
  memcpy(p_host, p0, sizeof p0);
  memcpy(m_host, m0, sizeof m0);
  memcpy(v_host, v0, sizeof v0);
  ZS(zero_host_adam_step(g, N, gs, p_host, m_host, v_host, &hp, out_host, ZERO_BF16, 4));

  for (i = 0; i < N; ++i) {
    if (memcmp(&p_dev[i], &p_host[i], 4) || memcmp(&m_dev[i], &m_host[i], 4) ||
        memcmp(&v_dev[i], &v_host[i], 4) || out_dev[i] != out_host[i]) {
      if (bad < 5) fprintf(stderr, "element %u differs\n", i);
      ++bad;
    }
  }

  /* the fused step with every array in one arena placed by zero_arena_layout */
  {
    static float pa[N], ma[N], va[N];
    static uint16_t oa[N];
    zero_arena_array arr[R + 4];
    uint64_t off[R + 4], total = 0;
    const void* a_reps[R];
    zero_grad_src src_a;
    char* base = NULL;
    int32_t contiguous = -1;
    for (k = 0; k < R + 4; ++k) {
      arr[k].bytes = (uint64_t)N * (k <= R ? 2 : 4); /* R replicas and the slot, then master, m, v */
      arr[k].hot_offset = 0;
      arr[k].group = k <= R ? 0 : 1;
      arr[k].elem_bytes = k <= R ? 2 : 4;
    }
    ZS(zero_arena_layout(arr, R + 4, off, &total));
    ZS(zero_arena_alloc(total, (void**)&base, &contiguous));
    for (k = 0; k < R; ++k) {
      HIP(hipMemcpy(base + off[k], reps[k], N * 2, hipMemcpyHostToDevice));
      a_reps[k] = base + off[k];
    }
    HIP(hipMemcpy(base + off[R + 1], p0, N * 4, hipMemcpyHostToDevice));
    HIP(hipMemcpy(base + off[R + 2], m0, N * 4, hipMemcpyHostToDevice));
    HIP(hipMemcpy(base + off[R + 3], v0, N * 4, hipMemcpyHostToDevice));
    src_a.ptrs = a_reps;
    src_a.count = R;
    src_a.dtype = ZERO_BF16;
    ZS(zero_adam_shard_step(&src_a, N, gs, (float*)(base + off[R + 1]), (float*)(base + off[R + 2]),
                            (float*)(base + off[R + 3]), &hp, base + off[R], ZERO_BF16, NULL, NULL));
    HIP(hipDeviceSynchronize());
    HIP(hipMemcpy(pa, base + off[R + 1], N * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(ma, base + off[R + 2], N * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(va, base + off[R + 3], N * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(oa, base + off[R], N * 2, hipMemcpyDeviceToHost));
    ZS(zero_arena_free(base));
    if (contiguous != 0 && contiguous != 1) {
      fprintf(stderr, "zero_arena_alloc: contiguous flag %d\n", (int)contiguous);
      ++bad;
    }
    if (memcmp(pa, p_dev, sizeof pa) || memcmp(ma, m_dev, sizeof ma) || memcmp(va, v_dev, sizeof va) ||
        memcmp(oa, out_dev, sizeof oa)) {
      fprintf(stderr, "the step in an arena differs from the step on separate allocations\n");
      ++bad;
    }
  }

  /* the ZeRO-3 gather: flat [N - 100, 2N + 50) of the replica buffers laid end to end */
  {
    enum { GB = N - 100, GC = N + 150 };
    static uint16_t g_out[GC];
    uint16_t* d_gout;
    HIP(hipMalloc((void**)&d_gout, GC * 2));
    ZS(zero_gather_params(d_rep_ptrs, R, N, 2, GB, GC, d_gout, NULL));
    HIP(hipMemcpy(g_out, d_gout, GC * 2, hipMemcpyDeviceToHost));
    for (i = 0; i < GC; ++i) {
      const uint32_t j = GB + i;
      if (g_out[i] != reps[j / N][j % N]) {
        if (bad < 5) fprintf(stderr, "gather element %u differs\n", i);
        ++bad;
      }
    }
    HIP(hipFree(d_gout));
  }

  /* the offloaded step against the fused device step, both stagings */
  {
    enum { CH = 4096 }; /* 25 chunks, the last one short */
    static float p_off[N], m_off[N], v_off[N];
    static uint16_t out_off[N];
    float *d_stage, *h_grad, *pageable;
    uint16_t *h_param, *d_out2;
    hipEvent_t ev[4];
    zero_offload_buffers ob;
    zero_status st;
    int pass;
    HIP(hipMalloc((void**)&d_stage, 2 * CH * 4));
    HIP(hipMalloc((void**)&d_out2, N * 2));
    HIP(hipHostMalloc((void**)&h_grad, 2 * CH * 4, hipHostMallocDefault));
    HIP(hipHostMalloc((void**)&h_param, 2 * CH * 2, hipHostMallocDefault));
    for (k = 0; k < 4; ++k) HIP(hipEventCreateWithFlags(&ev[k], hipEventDisableTiming));
    memset(&ob, 0, sizeof ob);
    ob.h_grad = h_grad;
    ob.h_param = h_param;
    ob.chunk_elems = CH;
    ob.threads = 3;
    for (k = 0; k < 4; ++k) ob.events[k] = ev[k];
    for (pass = 0; pass < 2; ++pass) {
      ob.d_grad = pass == 0 ? d_stage : NULL; /* NULL: the reduce kernel writes h_grad itself */
      memcpy(p_off, p0, sizeof p0);
      memcpy(m_off, m0, sizeof m0);
      memcpy(v_off, v0, sizeof v0);
      HIP(hipMemset(d_out2, 0, N * 2));
      ZS(zero_offload_step(&src, N, gs, p_off, m_off, v_off, &hp, d_out2, ZERO_BF16, &ob, NULL));
      HIP(hipMemcpy(out_off, d_out2, N * 2, hipMemcpyDeviceToHost));
      for (i = 0; i < N; ++i) {
        if (memcmp(&p_off[i], &p_dev[i], 4) || memcmp(&m_off[i], &m_dev[i], 4) ||
            memcmp(&v_off[i], &v_dev[i], 4) || out_off[i] != out_dev[i]) {
          if (bad < 5) fprintf(stderr, "offload (%s) element %u differs\n", pass ? "direct" : "copy", i);
          ++bad;
        }
      }
    }
    pageable = malloc(2 * CH * 4);
    if (!pageable) return 2;
    ob.d_grad = NULL;
    ob.h_grad = pageable;
    memcpy(p_off, p0, sizeof p0);
    st = zero_offload_step(&src, N, gs, p_off, m_off, v_off, &hp, d_out2, ZERO_BF16, &ob, NULL);
    if (st != ZERO_E_INVAL || memcmp(p_off, p0, sizeof p0)) {
      fprintf(stderr, "direct staging into pageable memory: status %d (%s)\n", (int)st, zero_last_error());
      ++bad;
    }
    free(pageable);
    for (k = 0; k < 4; ++k) HIP(hipEventDestroy(ev[k]));
    HIP(hipHostFree(h_grad));
    HIP(hipHostFree(h_param));
    HIP(hipFree(d_stage));
    HIP(hipFree(d_out2));
  }

  /* the clipped path: squared norm of the reduced gradient, clip scale and update on the device */
  {
    const double max_norm = 1e-3, clip_eps = 1e-6, inv_scale = 0.5;
    double *d_parts, *d_sq, sq, q, coef;
    float *d_gs, gs_dev, gs_c;
    HIP(hipMalloc((void**)&d_parts, zero_sq_partials_len(N) * 8));
    HIP(hipMalloc((void**)&d_sq, 8));
    HIP(hipMalloc((void**)&d_gs, 4));
    HIP(hipMemcpy(d_p, p0, N * 4, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_m, m0, N * 4, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_v, v0, N * 4, hipMemcpyHostToDevice));
    ZS(zero_shard_sqnorm(d_g, N, 1.0, d_parts, d_sq, NULL));
    ZS(zero_clip_scale(d_sq, max_norm, clip_eps, inv_scale, d_gs, NULL));
    ZS(zero_adam_shard_step_dev_scale(&src, N, d_gs, d_p, d_m, d_v, &hp, d_out, ZERO_BF16, NULL,
                                      NULL));
    HIP(hipDeviceSynchronize());
    HIP(hipMemcpy(&sq, d_sq, 8, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(&gs_dev, d_gs, 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(p_dev, d_p, N * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(m_dev, d_m, N * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(v_dev, d_v, N * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(out_dev, d_out, N * 2, hipMemcpyDeviceToHost));
    q = max_norm / (sqrt(sq) + clip_eps);
    coef = q < 1.0 ? q : 1.0;
    gs_c = (float)(coef * inv_scale);
    if (!(coef < 1.0) || memcmp(&gs_c, &gs_dev, 4)) {
      fprintf(stderr, "clip scale: device %.9g, C %.9g (coef %.17g)\n", gs_dev, gs_c, coef);
      ++bad;
    }
    memcpy(p_host, p0, sizeof p0);
    memcpy(m_host, m0, sizeof m0);
    memcpy(v_host, v0, sizeof v0);
    ZS(zero_host_adam_step(g, N, gs_dev, p_host, m_host, v_host, &hp, out_host, ZERO_BF16, 4));
    for (i = 0; i < N; ++i) {
      if (memcmp(&p_dev[i], &p_host[i], 4) || memcmp(&m_dev[i], &m_host[i], 4) ||
          memcmp(&v_dev[i], &v_host[i], 4) || out_dev[i] != out_host[i]) {
        if (bad < 5) fprintf(stderr, "clipped step: element %u differs\n", i);
        ++bad;
      }
    }

    /* the same clipped update with t on the device: a table of the constants of steps 1..8 built
     * by zero_adam_derive_table, the counter at hp.step, advanced by the call */
    {
      zero_adam_scalars table[8];
      zero_adam_scalars* d_table;
      int64_t t = hp.step, *d_t;
      int32_t status = -1, *d_status;
      ZS(zero_adam_derive_table(&hp, 8, table));
      HIP(hipMalloc((void**)&d_table, sizeof table));
      HIP(hipMalloc((void**)&d_t, 8));
      HIP(hipMalloc((void**)&d_status, 4));
      HIP(hipMemset(d_status, 0, 4));
      HIP(hipMemcpy(d_table, table, sizeof table, hipMemcpyHostToDevice));
      HIP(hipMemcpy(d_t, &t, 8, hipMemcpyHostToDevice));
      HIP(hipMemcpy(d_p, p0, N * 4, hipMemcpyHostToDevice));
      HIP(hipMemcpy(d_m, m0, N * 4, hipMemcpyHostToDevice));
      HIP(hipMemcpy(d_v, v0, N * 4, hipMemcpyHostToDevice));
      ZS(zero_adam_shard_step_dev_t(&src, N, d_gs, d_table, 8, d_t, d_status, ZERO_ADAMW, d_p, d_m,
                                    d_v, d_out, ZERO_BF16, NULL, NULL));
      HIP(hipDeviceSynchronize());
      HIP(hipMemcpy(&t, d_t, 8, hipMemcpyDeviceToHost));
      HIP(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost));
      if (status != 0) {
        fprintf(stderr, "status word %d after a step inside the table\n", (int)status);
        ++bad;
      }
      HIP(hipMemcpy(p_dev, d_p, N * 4, hipMemcpyDeviceToHost));
      HIP(hipMemcpy(m_dev, d_m, N * 4, hipMemcpyDeviceToHost));
      HIP(hipMemcpy(v_dev, d_v, N * 4, hipMemcpyDeviceToHost));
      HIP(hipMemcpy(out_dev, d_out, N * 2, hipMemcpyDeviceToHost));
      if (t != hp.step + 1) {
        fprintf(stderr, "step counter: %lld after the call, %lld expected\n", (long long)t,
                (long long)(hp.step + 1));
        ++bad;
      }
      for (i = 0; i < N; ++i) {
        if (memcmp(&p_dev[i], &p_host[i], 4) || memcmp(&m_dev[i], &m_host[i], 4) ||
            memcmp(&v_dev[i], &v_host[i], 4) || out_dev[i] != out_host[i]) {
          if (bad < 5) fprintf(stderr, "device-step update: element %u differs\n", i);
          ++bad;
        }
      }
      HIP(hipFree(d_table));
      HIP(hipFree(d_t));
      HIP(hipFree(d_status));
    }

    /* the reduce pass and its norm with no workspace (zero_reduce_shard_static, the partials in
     * the library's own scratch) against zero_reduce_shard and zero_shard_sqnorm with a caller's
     * partials: the gradient and the norm bit for bit, twice in a row */
    {
      double sq_ws, sq_static;
      int32_t *d_flag, flag = -1;
      float* d_g2;
      int rep_i;
      HIP(hipMalloc((void**)&d_flag, 4));
      HIP(hipMalloc((void**)&d_g2, N * 4));
      ZS(zero_reduce_shard(&src, N, NULL, NULL, d_parts, 0.25, NULL));
      ZS(zero_shard_sqnorm(NULL, N, 0.25, d_parts, d_sq, NULL));
      HIP(hipDeviceSynchronize());
      HIP(hipMemcpy(&sq_ws, d_sq, 8, hipMemcpyDeviceToHost));
      for (rep_i = 0; rep_i < 2; ++rep_i) {
        HIP(hipMemset(d_flag, 0, 4));
        HIP(hipMemset(d_sq, 0, 8));
        ZS(zero_reduce_shard_static(&src, N, d_g2, d_flag, 0.25, d_sq, NULL));
        HIP(hipDeviceSynchronize());
        HIP(hipMemcpy(&sq_static, d_sq, 8, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(&flag, d_flag, 4, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(g2, d_g2, N * 4, hipMemcpyDeviceToHost));
        if (memcmp(&sq_ws, &sq_static, 8) || flag != 0 || memcmp(g, g2, sizeof g)) {
          fprintf(stderr, "static reduce: norm %.17g against %.17g, flag %d, gradient %s\n", sq_static,
                  sq_ws, (int)flag, memcmp(g, g2, sizeof g) ? "differs" : "equal");
          ++bad;
        }
      }
      HIP(hipFree(d_flag));
      HIP(hipFree(d_g2));
    }
    HIP(hipFree(d_parts));
    HIP(hipFree(d_sq));
    HIP(hipFree(d_gs));
  }
  for (k = 0; k < R; ++k) HIP(hipFree(d_reps[k]));
  HIP(hipFree(d_p));
  HIP(hipFree(d_m));
  HIP(hipFree(d_v));
  HIP(hipFree(d_g));
  HIP(hipFree(d_out));
  printf("%u of %u elements differ\n", bad, N);
  return bad ? 1 : 0;
}
