/* Drives the CPU oracle through random traces, invalid rows, appends and
 * window loads so that an AddressSanitizer/UBSan build can check its memory
 * and integer behaviour.  Built and run by test_oracle_sanitizers.py (gcc). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t C, R;
  int64_t l_cap, row_bytes;
  int32_t *pos2slot, *slot2pos, *last_use, *t;
  uint8_t *slots, *host;
} hso_stream;

uint32_t hso_resolve(const hso_stream*, const int32_t*, int32_t, int64_t, uint32_t, int32_t*,
                     int32_t*, int32_t*, int64_t*);
int hso_seed_window(const hso_stream*, int64_t);
int hso_append(const hso_stream*, const uint8_t*, int64_t);

static uint64_t rng_state = 88172645463325252ull;
static uint64_t rnd(void) { /* xorshift64 */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}

int main(void) {
  for (int trial = 0; trial < 200; ++trial) {
    int32_t k = 1 + (int32_t)(rnd() % 40);
    int32_t C = k + (int32_t)(rnd() % 20);
    int32_t R = (int32_t)(rnd() % 5);
    int64_t L = k + 10 + (int64_t)(rnd() % 200);
    int steps = 2 + (int)(rnd() % 30);
    int64_t l_cap = L + steps;
    int64_t rb = 16 * (1 + (int64_t)(rnd() % 4));
    hso_stream st = {C, R, l_cap, rb, NULL, NULL, NULL, NULL, NULL, NULL};
    st.pos2slot = malloc(sizeof(int32_t) * l_cap);
    st.slot2pos = malloc(sizeof(int32_t) * C);
    st.last_use = calloc(C, sizeof(int32_t));
    st.t = calloc(1, sizeof(int32_t));
    st.slots = calloc((size_t)(C + R) * rb, 1);
    st.host = malloc((size_t)l_cap * rb);
    for (int64_t i = 0; i < l_cap; ++i) st.pos2slot[i] = -1;
    for (int32_t i = 0; i < C; ++i) st.slot2pos[i] = -1;
    for (int64_t i = 0; i < l_cap * rb; ++i) st.host[i] = (uint8_t)rnd();
    hso_seed_window(&st, L);
    int32_t *sel = malloc(sizeof(int32_t) * k), *out = malloc(sizeof(int32_t) * k);
    int32_t *ls = malloc(sizeof(int32_t) * k), *lo = malloc(sizeof(int32_t) * k);
    uint8_t* used = calloc((size_t)l_cap, 1);
    uint8_t* row = malloc((size_t)rb);
    int64_t cnt[6];
    int64_t ctx = L;
    for (int s = 0; s < steps; ++s) {
      memset(used, 0, (size_t)l_cap);
      for (int32_t i = 0; i < k; ++i) {
        if (rnd() % 10 == 0) { sel[i] = -1; continue; }
        int64_t p;
        do { p = (int64_t)(rnd() % (uint64_t)ctx); } while (used[p]);
        used[p] = 1;
        sel[i] = (int32_t)p;
      }
      if (rnd() % 20 == 0) sel[rnd() % k] = (int32_t)(ctx + (int64_t)(rnd() % 3));
      if (rnd() % 20 == 0 && k > 1) sel[1] = sel[0] >= 0 ? sel[0] : sel[1];
      hso_resolve(&st, sel, k, ctx, (uint32_t)(rnd() % 2), out, ls, lo, cnt);
      for (int64_t i = 0; i < rb; ++i) row[i] = (uint8_t)rnd();
      if (ctx < l_cap) { hso_append(&st, row, ctx); ++ctx; }
    }
    free(sel); free(out); free(ls); free(lo); free(used); free(row);
    free(st.pos2slot); free(st.slot2pos); free(st.last_use); free(st.t); free(st.slots);
    free(st.host);
  }
  printf("sanitized oracle run: ok\n");
  return 0;
}
