// Drives every host-only entry point of the library under AddressSanitizer and UBSan: the
// partition plan, shard ranges, per-stage bytes, the stage choice, the arena layout, the Adam
// constants and the host update (all sizes from 0 up, unaligned arrays, every thread count, both
// 16-bit outputs, the error paths). Built with a plain host compiler from the sources that make no HIP calls.
// Exits non-zero on a wrong status or a result that differs between thread counts.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "zero_host_adam.h"
#include "zero_shard.h"

static int failures = 0;
#define EXPECT(cond)                                                    \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

static uint32_t lcg(uint64_t* s) {
  *s = *s * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(*s >> 33);
}

static void plans() {
  const uint64_t ns[] = {0, 1, 2, 7, 63, 64, 1000003, 6738415616ull, 174604259328ull, ~0ull - 5};
  const uint32_t nds[] = {1, 2, 3, 8, 16, 64, 4096};
  const uint32_t aligns[] = {1, 2, 8, 256};
  for (uint64_t n : ns)
    for (uint32_t nd : nds)
      for (uint32_t al : aligns) {
        zero_plan p;
        const zero_status s = zero_partition_plan(n, nd, al, &p);
        EXPECT(s == ZERO_OK || s == ZERO_E_OVERFLOW);
        if (s != ZERO_OK) continue;
        uint64_t covered = 0;
        for (uint32_t r = 0; r < nd; ++r) {
          uint64_t b, v;
          EXPECT(zero_shard_range(&p, r, &b, &v) == ZERO_OK);
          EXPECT(b == (uint64_t)r * p.shard_elems && v <= p.shard_elems);
          covered += v;
        }
        EXPECT(covered == n);
        uint64_t by[4];
        for (uint32_t st = 0; st <= 4; ++st) {
          const zero_status bs = zero_stage_bytes(&p, st, 2, 2, 12, by);
          EXPECT(st == 4 ? bs == ZERO_E_INVAL : (bs == ZERO_OK || bs == ZERO_E_OVERFLOW));
          const zero_status cb = zero_stage_comm_bytes(&p, st, 2, 2, by);
          EXPECT(st == 4 ? cb == ZERO_E_INVAL : (cb == ZERO_OK || cb == ZERO_E_OVERFLOW));
          if (st < 4 && cb == ZERO_OK) EXPECT(by[2] == by[0] + by[1]);
        }
        zero_stage_choice c;
        const zero_status cs = zero_choose_stage(&p, 80000000000ull, 2, 2, 12, &c);
        EXPECT(cs == ZERO_OK || cs == ZERO_E_OVERFLOW);
        if (cs == ZERO_OK) EXPECT(c.stage >= 1 && c.stage <= 3);
      }
  zero_plan p;
  EXPECT(zero_partition_plan(5, 0, 1, &p) == ZERO_E_INVAL);
  EXPECT(zero_partition_plan(5, 1, 0, &p) == ZERO_E_INVAL);
  EXPECT(zero_partition_plan(5, 1, 1, NULL) == ZERO_E_INVAL);
  EXPECT(zero_partition_plan(~0ull, 2, 1, &p) == ZERO_E_OVERFLOW);  // S = 2^63, P = 2^64
  EXPECT(zero_partition_plan(~0ull, 3, 1, &p) == ZERO_OK);           // 2^64 - 1 = 3 * S exactly
  EXPECT(zero_partition_plan(10, 4, 1, &p) == ZERO_OK);
  uint64_t b, v;
  EXPECT(zero_shard_range(&p, 4, &b, &v) == ZERO_E_INVAL);
  p.pad += 1;
  EXPECT(zero_shard_range(&p, 0, &b, &v) == ZERO_E_INVAL);
  EXPECT(zero_status_str((zero_status)77) != NULL && zero_last_error() != NULL);
}

static void derive() {
  zero_adam_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.01, ZERO_ADAMW, 0, 1};
  zero_adam_scalars k;
  for (int64_t t : {1ll, 2ll, 1000ll, 1ll << 40}) {
    hp.step = t;
    EXPECT(zero_adam_derive(&hp, &k) == ZERO_OK);
  }
  hp.step = 0;
  EXPECT(zero_adam_derive(&hp, &k) == ZERO_E_INVAL);
  hp.step = 1;
  hp.beta1 = 1.0;
  EXPECT(zero_adam_derive(&hp, &k) == ZERO_E_INVAL);
  hp.beta1 = 0.9;
  hp.wd_mode = 7;
  EXPECT(zero_adam_derive(&hp, &k) == ZERO_E_INVAL);
  EXPECT(zero_adam_derive(NULL, &k) == ZERO_E_INVAL);
  // the per-step table: every entry equals the single-step call, on a heap array sized exactly
  hp.wd_mode = ZERO_ADAMW;
  const uint32_t count = 3000;
  zero_adam_scalars* tab = new zero_adam_scalars[count];
  EXPECT(zero_adam_derive_table(&hp, count, tab) == ZERO_OK);
  for (uint32_t t = 1; t <= count; t += 37) {
    hp.step = t;
    EXPECT(zero_adam_derive(&hp, &k) == ZERO_OK);
    EXPECT(memcmp(&k, &tab[t - 1], sizeof k) == 0);
  }
  EXPECT(zero_adam_derive_table(&hp, 0, tab) == ZERO_E_INVAL);
  EXPECT(zero_adam_derive_table(NULL, 1, tab) == ZERO_E_INVAL);
  EXPECT(zero_adam_derive_table(&hp, 1, NULL) == ZERO_E_INVAL);
  hp.beta2 = -1.0;
  EXPECT(zero_adam_derive_table(&hp, count, tab) == ZERO_E_INVAL);
  delete[] tab;
}

static void host_updates() {
  const uint64_t sizes[] = {0, 1, 3, 63, 64, 65, 4099, 70001, 300007};
  const uint32_t threads[] = {1, 2, 3, 16};
  uint64_t seed = 42;
  for (uint64_t n : sizes)
    for (int off = 0; off < 2; ++off)
      for (int odt : {(int)ZERO_BF16, (int)ZERO_F16, -1})
        for (int mode : {(int)ZERO_ADAMW, (int)ZERO_ADAM_L2}) {
          std::vector<float> g(n + off), p0(n + off), m0(n + off), v0(n + off);
          for (uint64_t i = 0; i < n + off; ++i) {
            g[i] = ((int)(lcg(&seed) % 2001) - 1000) * 1e-6f;
            p0[i] = ((int)(lcg(&seed) % 2001) - 1000) * 2e-5f;
            m0[i] = ((int)(lcg(&seed) % 2001) - 1000) * 1e-7f;
            v0[i] = (lcg(&seed) % 1000) * 1e-10f;
          }
          zero_adam_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.01, mode, 0, 3};
          std::vector<float> ref_p;
          std::vector<uint16_t> ref_o;
          for (uint32_t t : threads) {
            std::vector<float> p = p0, m = m0, v = v0;
            std::vector<uint16_t> o(n + off, 0xABCD);
            const zero_status s = zero_host_adam_step(g.data() + off, n, 0.5f, p.data() + off, m.data() + off,
                                                      v.data() + off, &hp, odt < 0 ? NULL : o.data() + off,
                                                      odt < 0 ? ZERO_BF16 : odt, t);
            EXPECT(s == ZERO_OK);
            for (int i = 0; i < off; ++i) EXPECT(memcmp(&p[i], &p0[i], 4) == 0 && o[i] == 0xABCD);
            if (ref_p.empty()) {
              ref_p = p;
              ref_o = o;
            } else {
              EXPECT(memcmp(ref_p.data(), p.data(), p.size() * 4) == 0);
              EXPECT(memcmp(ref_o.data(), o.data(), o.size() * 2) == 0);
            }
          }
        }
  // error paths: overlaps, NULLs, unsupported output
  std::vector<float> a(64), b2(64), c(64), d(64);
  std::vector<uint16_t> o(64);
  zero_adam_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.0, ZERO_ADAMW, 0, 1};
  EXPECT(zero_host_adam_step(a.data(), 64, 1.f, b2.data(), b2.data() + 10, c.data(), &hp, NULL, 0, 1) == ZERO_E_INVAL);
  EXPECT(zero_host_adam_step(a.data(), 64, 1.f, a.data(), c.data(), d.data(), &hp, NULL, 0, 1) == ZERO_E_INVAL);
  EXPECT(zero_host_adam_step(NULL, 64, 1.f, b2.data(), c.data(), d.data(), &hp, NULL, 0, 1) == ZERO_E_INVAL);
  EXPECT(zero_host_adam_step(a.data(), 64, 1.f, b2.data(), c.data(), d.data(), &hp, o.data(), ZERO_F32, 1) ==
         ZERO_E_UNSUPPORTED);
  EXPECT(zero_host_adam_step(NULL, 0, 1.f, NULL, NULL, NULL, &hp, NULL, ZERO_BF16, 0) == ZERO_OK);
  EXPECT(zero_host_adam_step(a.data(), ~0ull / 4, 1.f, b2.data(), c.data(), d.data(), &hp, NULL, 0, 1) ==
         ZERO_E_OVERFLOW);
}

// the offloaded step's thread team: consecutive jobs of different sizes on one team (as the step's
// chunks run) give the same bits as the per-call threads, for every team size
static void teams() {
  const uint64_t sizes[] = {0, 1, 70001, 300007, 5, 131072, 65536 * 3 + 1};
  uint64_t seed = 9;
  const uint64_t nmax = 300007;
  std::vector<float> g(nmax), p0(nmax), m0(nmax), v0(nmax);
  for (uint64_t i = 0; i < nmax; ++i) {
    g[i] = ((int)(lcg(&seed) % 2001) - 1000) * 1e-6f;
    p0[i] = ((int)(lcg(&seed) % 2001) - 1000) * 2e-5f;
    m0[i] = ((int)(lcg(&seed) % 2001) - 1000) * 1e-7f;
    v0[i] = (lcg(&seed) % 1000) * 1e-10f;
  }
  zero_adam_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.01, ZERO_ADAMW, 0, 5};
  zero_adam_scalars k;
  EXPECT(zero_adam_derive(&hp, &k) == ZERO_OK);
  for (uint32_t t : {1u, 2u, 3u, 16u}) {
    zero::HostTeam team(t);
    EXPECT(team.size() >= 1 && team.size() <= t);
    for (int rep = 0; rep < 2; ++rep)
      for (uint64_t n : sizes) {
        std::vector<float> pa = p0, ma = m0, va = v0, pb = p0, mb = m0, vb = v0;
        std::vector<uint16_t> oa(nmax, 0x1111), ob(nmax, 0x1111);
        EXPECT(zero::host_step(g.data(), n, 0.5f, pa.data(), ma.data(), va.data(), k, false, oa.data(),
                               ZERO_BF16, t, &team) == ZERO_OK);
        EXPECT(zero::host_step(g.data(), n, 0.5f, pb.data(), mb.data(), vb.data(), k, false, ob.data(),
                               ZERO_BF16, t) == ZERO_OK);
        EXPECT(memcmp(pa.data(), pb.data(), nmax * 4) == 0 && memcmp(va.data(), vb.data(), nmax * 4) == 0);
        EXPECT(memcmp(oa.data(), ob.data(), nmax * 2) == 0);
      }
  }
}

static void arenas() {
  uint64_t seed = 7;
  for (int trial = 0; trial < 200; ++trial) {
    const uint32_t count = 1 + lcg(&seed) % ZERO_ARENA_MAX_ARRAYS;
    std::vector<zero_arena_array> a(count);
    for (auto& x : a) {
      x.elem_bytes = (lcg(&seed) & 1) ? 4 : 2;
      const uint64_t n = lcg(&seed) % (1u << (lcg(&seed) % 31));
      x.bytes = n * x.elem_bytes;
      x.hot_offset = n ? (lcg(&seed) % (n + 1)) * x.elem_bytes : 0;
      x.group = lcg(&seed) % 5;
    }
    std::vector<uint64_t> off(count);
    uint64_t total = 0;
    EXPECT(zero_arena_layout(a.data(), count, off.data(), &total) == ZERO_OK);
    uint64_t end = 0;
    for (uint32_t i = 0; i < count; ++i) {
      EXPECT(off[i] >= end && off[i] - end < ZERO_ARENA_GRANULE);
      EXPECT((off[i] + a[i].hot_offset) % 2048 == 0);
      end = off[i] + a[i].bytes;
    }
    EXPECT(total == end);
  }
  zero_arena_array big[2] = {{1ull << 63, 0, 0, 2}, {1ull << 63, 0, 1, 2}};
  uint64_t off[ZERO_ARENA_MAX_ARRAYS + 1], total;
  EXPECT(zero_arena_layout(big, 2, off, &total) == ZERO_E_OVERFLOW);
  zero_arena_array bad = {1024, 0, 0, 3};
  EXPECT(zero_arena_layout(&bad, 1, off, &total) == ZERO_E_INVAL);
  EXPECT(zero_arena_layout(big, 0, off, &total) == ZERO_E_INVAL);
  EXPECT(zero_arena_layout(NULL, 1, off, &total) == ZERO_E_INVAL);
  std::vector<zero_arena_array> many(ZERO_ARENA_MAX_ARRAYS + 1, zero_arena_array{64, 0, 0, 2});
  EXPECT(zero_arena_layout(many.data(), ZERO_ARENA_MAX_ARRAYS + 1, off, &total) == ZERO_E_INVAL);
}

int main() {
  plans();
  arenas();
  derive();
  host_updates();
  teams();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host driver ok\n");
  return 0;
}
