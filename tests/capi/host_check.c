/* The host entry points of libzero_shard called from plain C99: prints one line per result for the
 * test to compare with the oracle. Exits non-zero on an unexpected status. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "zero_shard.h"

static int fails = 0;
static void expect(int ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "unexpected: %s (%s)\n", what, zero_last_error());
    ++fails;
  }
}

int main(void) {
  const uint64_t ns[4] = {1000003ull, 124356864ull, 6738415616ull, 7ull};
  const uint32_t nds[4] = {4u, 8u, 8u, 16u};
  const uint32_t aligns[4] = {1u, 8u, 1u, 4u};
  int i;
  for (i = 0; i < 4; ++i) {
    zero_plan p;
    uint32_t r;
    expect(zero_partition_plan(ns[i], nds[i], aligns[i], &p) == ZERO_OK, "plan");
    printf("plan %llu %u %u -> %llu %llu %llu\n", (unsigned long long)ns[i], nds[i], aligns[i],
           (unsigned long long)p.shard_elems, (unsigned long long)p.padded_n, (unsigned long long)p.pad);
    for (r = 0; r < p.nd; ++r) {
      uint64_t b, v;
      expect(zero_shard_range(&p, r, &b, &v) == ZERO_OK, "range");
      printf("range %llu %u %u %u -> %llu %llu\n", (unsigned long long)ns[i], nds[i], aligns[i], r,
             (unsigned long long)b, (unsigned long long)v);
    }
    {
      uint32_t st;
      for (st = 0; st <= 3; ++st) {
        uint64_t by[4];
        expect(zero_stage_bytes(&p, st, 2, 2, 12, by) == ZERO_OK, "stage bytes");
        printf("stage %llu %u %u %u -> %llu %llu %llu %llu\n", (unsigned long long)ns[i], nds[i],
               aligns[i], st, (unsigned long long)by[0], (unsigned long long)by[1],
               (unsigned long long)by[2], (unsigned long long)by[3]);
        expect(zero_stage_comm_bytes(&p, st, 2, 2, by) == ZERO_OK, "stage comm bytes");
        printf("comm %llu %u %u %u -> %llu %llu %llu\n", (unsigned long long)ns[i], nds[i],
               aligns[i], st, (unsigned long long)by[0], (unsigned long long)by[1],
               (unsigned long long)by[2]);
      }
    }
  }
  {
    zero_adam_hparams hp;
    zero_adam_scalars k;
    memset(&hp, 0, sizeof hp);
    hp.lr = 1e-3; hp.beta1 = 0.9; hp.beta2 = 0.999; hp.eps = 1e-8; hp.weight_decay = 0.01;
    hp.wd_mode = ZERO_ADAMW; hp.step = 11;
    expect(zero_adam_derive(&hp, &k) == ZERO_OK, "derive");
    printf("scalars %a %a %a %a %a %a %a %a %a\n", (double)k.b1, (double)k.b2, (double)k.c1,
           (double)k.c2, (double)k.ss, (double)k.bc, (double)k.e, (double)k.dec, (double)k.w);
    hp.step = 0;
    expect(zero_adam_derive(&hp, &k) == ZERO_E_INVAL, "derive rejects step 0");
  }
  {
    zero_arena_array a[3];
    uint64_t off[3], total;
    a[0].bytes = 1000; a[0].hot_offset = 0; a[0].group = 0; a[0].elem_bytes = 2;
    a[1].bytes = 4000; a[1].hot_offset = 400; a[1].group = 0; a[1].elem_bytes = 2;
    a[2].bytes = 4000; a[2].hot_offset = 0; a[2].group = 1; a[2].elem_bytes = 4;
    expect(zero_arena_layout(a, 3, off, &total) == ZERO_OK, "arena layout");
    printf("arena %llu %llu %llu %llu\n", (unsigned long long)off[0], (unsigned long long)off[1],
           (unsigned long long)off[2], (unsigned long long)total);
  }
  expect(zero_partition_plan(5, 0, 1, NULL) == ZERO_E_INVAL, "plan rejects NULL");
  printf("status %s\n", zero_status_str(ZERO_E_OVERFLOW));
  return fails ? 1 : 0;
}
