/* A plain C caller of libhisparse (no Python, no torch): replays the
 * hand-derived LRU example of tests/golden/lru_hand_example.txt through the
 * C ABI and checks every step's slot map, the slot-to-position table and the
 * last-use stamps (read back through hisparse_meta_layout_of), and that every
 * served slot holds its host row.  Device buffers come from hipMalloc, the
 * host history from hisparse_host_alloc.
 *
 * usage: c_abi_example <golden file>; exit status 0 when every check passes.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hisparse.h"

#define MAX_STEPS 16
#define ROW 16 /* bytes per history row */

#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      fprintf(stderr, __VA_ARGS__);       \
      fprintf(stderr, "\n");              \
      exit(1);                            \
    }                                     \
  } while (0)

#define HIP(call) CHECK((call) == hipSuccess, "HIP call failed: %s", #call)
#define LIB(call) CHECK((call) == HISPARSE_OK, "%s: %s", #call, hisparse_last_error())

typedef struct {
  int t, ctx;
  int sel[2], out[2], slot2pos[3], last_use[3];
} Step;

/* the integers after `key` in one '|'-separated field */
static int ints_after(const char* line, const char* key, int* v, int n) {
  const char* p = strstr(line, key);
  if (!p) return 0;
  p += strlen(key);
  int got = 0;
  while (got < n) {
    char* end;
    long x = strtol(p, &end, 10);
    if (end == p) break;
    v[got++] = (int)x;
    p = end;
  }
  return got;
}

int main(int argc, char** argv) {
  CHECK(argc == 2, "usage: %s <golden file>", argv[0]);
  FILE* f = fopen(argv[1], "r");
  CHECK(f, "cannot open %s", argv[1]);
  Step steps[MAX_STEPS];
  int n = 0, C = 0, R = 0, L = 0;
  char line[512];
  while (fgets(line, sizeof line, f)) {
    if (line[0] == 'C' && line[1] == ' ') C = atoi(line + 2);
    else if (line[0] == 'R' && line[1] == ' ') R = atoi(line + 2);
    else if (line[0] == 'L' && line[1] == ' ') L = atoi(line + 2);
    else if (!strncmp(line, "step ", 5)) {
      CHECK(n < MAX_STEPS, "too many steps");
      Step* s = &steps[n++];
      CHECK(ints_after(line, "step ", &s->t, 1) == 1 && ints_after(line, "ctx ", &s->ctx, 1) == 1 &&
                ints_after(line, "sel ", s->sel, 2) == 2 && ints_after(line, "out ", s->out, 2) == 2 &&
                ints_after(line, "slot2pos ", s->slot2pos, 3) == 3 &&
                ints_after(line, "last_use ", s->last_use, 3) == 3,
            "cannot parse: %s", line);
    }
  }
  fclose(f);
  CHECK(n > 0 && C == 3 && R == 0 && L > 0, "unexpected example (C %d, R %d, L %d)", C, R, L);

  hisparse_config cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.num_requests = 1;
  cfg.num_layers = 1;
  cfg.max_positions = L;
  cfg.row_bytes = ROW;
  cfg.cache_slots = C;
  cfg.resident_window = R;
  cfg.top_k = 2;
  size_t cache_bytes = 0, meta_bytes = 0;
  LIB(hisparse_workspace_bytes(&cfg, &cache_bytes, &meta_bytes));
  hisparse_meta_layout lay;
  LIB(hisparse_meta_layout_of(&cfg, &lay));

  void* host = NULL;
  LIB(hisparse_host_alloc((size_t)L * ROW, HISPARSE_NUMA_DEVICE, HISPARSE_HOST_COHERENT, &host));
  unsigned char* rows = (unsigned char*)host;
  for (int p = 0; p < L; ++p)
    for (int j = 0; j < ROW; ++j) rows[p * ROW + j] = (unsigned char)(7 * p + j + 1);

  void *cache = NULL, *meta = NULL;
  int32_t *d_sel = NULL, *d_ctx = NULL, *d_out = NULL;
  HIP(hipMalloc(&cache, cache_bytes));
  HIP(hipMalloc(&meta, meta_bytes));
  HIP(hipMalloc((void**)&d_sel, 2 * sizeof(int32_t)));
  HIP(hipMalloc((void**)&d_ctx, sizeof(int32_t)));
  HIP(hipMalloc((void**)&d_out, 2 * sizeof(int32_t)));
  hisparse_t h = NULL;
  void* hosts[1] = {host};
  LIB(hisparse_create(&cfg, hosts, cache, meta, &h));

  unsigned char* slots = (unsigned char*)malloc(cache_bytes);
  unsigned char* m = (unsigned char*)malloc(meta_bytes);
  CHECK(slots && m, "malloc");
  for (int i = 0; i < n; ++i) {
    const Step* s = &steps[i];
    int32_t ctx = s->ctx, out[2];
    HIP(hipMemcpy(d_sel, s->sel, sizeof s->sel, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_ctx, &ctx, sizeof ctx, hipMemcpyHostToDevice));
    LIB(hisparse_resolve(h, NULL, d_sel, d_ctx, 0, d_out));
    HIP(hipDeviceSynchronize());
    HIP(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(slots, cache, cache_bytes, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(m, meta, meta_bytes, hipMemcpyDeviceToHost));
    const unsigned char* st = m + lay.stream_base; /* stream (request 0, layer 0) */
    const int32_t* hdr = (const int32_t*)(st + lay.hdr);
    const int32_t* s2p = (const int32_t*)(st + lay.slot2pos);
    const int32_t* lu = (const int32_t*)(st + lay.last_use);
    CHECK(hdr[0] == s->t, "step %d: clock %d", s->t, hdr[0]);
    for (int e = 0; e < 2; ++e) {
      CHECK(out[e] == s->out[e], "step %d: out[%d] = %d, expected %d", s->t, e, out[e], s->out[e]);
      CHECK(!memcmp(slots + (size_t)out[e] * ROW, rows + (size_t)s->sel[e] * ROW, ROW),
            "step %d: slot %d does not hold host row %d", s->t, out[e], s->sel[e]);
    }
    for (int c = 0; c < C; ++c) {
      CHECK(s2p[c] == s->slot2pos[c], "step %d: slot2pos[%d] = %d, expected %d", s->t, c, s2p[c],
            s->slot2pos[c]);
      CHECK(lu[c] == s->last_use[c], "step %d: last_use[%d] = %d, expected %d", s->t, c, lu[c],
            s->last_use[c]);
    }
  }
  uint32_t status = 1;
  LIB(hisparse_get_status(h, &status, 0));
  CHECK(status == 0, "status word 0x%x", status);
  LIB(hisparse_destroy(h));
  free(slots);
  free(m);
  HIP(hipFree(cache));
  HIP(hipFree(meta));
  HIP(hipFree(d_sel));
  HIP(hipFree(d_ctx));
  HIP(hipFree(d_out));
  LIB(hisparse_host_free(host));
  printf("c_abi_example: %d steps of the hand example match through the C ABI\n", n);
  return 0;
}
