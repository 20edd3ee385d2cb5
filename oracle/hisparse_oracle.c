/* CPU oracle for the per-layer selection resolution of a two-tier KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
 * statement of what the GPU path computes; only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * Sources (pages, cited by title and section):
 *   [P3] "HiSparse: Scaling Sparse-Attention Decoding with Hierarchical KV
 *        Cache Management" -- Abstract: each request keeps its full KV history
 *        in host memory and a small fixed-size GPU cache; per layer, the
 *        selected positions are resolved by hit detection, LRU replacement and
 *        host-to-device fetches of the missing rows; only placement changes,
 *        so attention outputs are unchanged.  AI Summary: hit detection,
 *        eviction and migration happen in one pass.
 *   [P2] "Hybrid HiSparse" -- Timeline: rows are classified as resident, hot
 *        or missing in a single pass.
 *   [P1] "HiSparse" -- Timeline: only the missing rows that the top-k hits are
 *        copied back into the request's hot buffer.
 *
 * Where the pages are silent the following readings are used (each is stated
 * again at the line that implements it):
 *   - one cache per (request, layer) = one "stream";
 *   - the LRU clock is a per-stream step counter t, advanced once per call;
 *   - victims are the slots not referenced this step, ordered by
 *     (last_use ascending, slot ascending);
 *   - the j-th miss in ascending selection index takes the j-th victim;
 *   - empty slots have last_use 0 and hold position -1; they are "victims"
 *     without an eviction;
 *   - "resident" rows are the last R positions of the context, kept in a ring
 *     of R extra slots at slot C + (p mod R), outside the LRU;
 *   - -1 is padding; a position outside [0, ctx) or a repeated position makes
 *     the call a no-op for that stream, with every output -1 and a status bit.
 *
 * Parity of slot numbering and victim order is pinned only by these readings
 * (hand-derived examples, closed forms and an independent brute force in the
 * tests); the data-level exactness is pinned by the pages' claim that outputs
 * are unchanged.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HSO_STATUS_SEL_RANGE 1u /* a selection outside [-1, ctx) */
#define HSO_STATUS_SEL_DUP 2u   /* a non-negative selection repeated */
#define HSO_STATUS_CTX_RANGE 4u /* ctx outside [0, l_cap] */
#define HSO_STATUS_CAPACITY 8u  /* more selections than LRU slots (k > C) */

#define HSO_FLAG_NO_IO 1u /* metadata only: skip the row copies */

/* One stream = one (request, layer).  All arrays are owned by the caller. */
typedef struct {
  int32_t C;           /* LRU slots, numbered [0, C) */
  int32_t R;           /* resident ring slots, numbered [C, C+R) */
  int64_t l_cap;       /* host rows */
  int64_t row_bytes;   /* bytes per row */
  int32_t* pos2slot;   /* [l_cap]: LRU slot holding position p, or -1 */
  int32_t* slot2pos;   /* [C]: position held by LRU slot s, or -1 */
  int32_t* last_use;   /* [C]: step at which slot s was last referenced */
  int32_t* t;          /* [1]: step counter */
  uint8_t* slots;      /* [(C+R) * row_bytes] or NULL (metadata only) */
  uint8_t* host;       /* [l_cap * row_bytes] or NULL (metadata only) */
} hso_stream;

/* Counters returned by hso_resolve, in this order. */
enum { HSO_N_PAD, HSO_N_RES, HSO_N_HIT, HSO_N_MISS, HSO_N_EVICT, HSO_BYTES, HSO_NCOUNT };

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

typedef struct {
  int32_t last_use;
  int32_t slot;
} lru_key;

/* LRU order: older stamp first; equal stamps by ascending slot number. */
static int cmp_lru(const void* a, const void* b) {
  const lru_key* x = (const lru_key*)a;
  const lru_key* y = (const lru_key*)b;
  if (x->last_use != y->last_use) return (x->last_use > y->last_use) - (x->last_use < y->last_use);
  return (x->slot > y->slot) - (x->slot < y->slot);
}

static void copy_row(const hso_stream* st, int64_t slot, int64_t pos) {
  memcpy(st->slots + slot * st->row_bytes, st->host + pos * st->row_bytes,
         (size_t)st->row_bytes);
}

/* Resolve one stream's k selections for one step at context length ctx.
 *
 * Outputs: out[k] (slot per selection, -1 for padding), the eviction log
 * (log_slot[j], log_old[j]) for the j-th miss (old = -1 when the slot was
 * empty), and counters[HSO_NCOUNT].  Returns 0 or a status bit set; on a
 * status the stream is left untouched and every out[i] is -1.
 */
uint32_t hso_resolve(const hso_stream* st, const int32_t* sel, int32_t k, int64_t ctx,
                     uint32_t flags, int32_t* out, int32_t* log_slot, int32_t* log_old,
                     int64_t* counters) {
  const int32_t C = st->C, R = st->R;
  uint32_t status = 0;
  for (int c = 0; c < HSO_NCOUNT; ++c) counters[c] = 0;

  /* Step 1: validate the whole row before touching any state. */
  if (k > C) status |= HSO_STATUS_CAPACITY;
  if (ctx < 0 || ctx > st->l_cap) status |= HSO_STATUS_CTX_RANGE;
  for (int32_t i = 0; i < k; ++i) {
    int32_t p = sel[i];
    if (p < -1 || (p >= 0 && (int64_t)p >= ctx)) status |= HSO_STATUS_SEL_RANGE;
  }
  if (status == 0 && k > 0) {
    int32_t* sorted = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    int32_t n = 0;
    for (int32_t i = 0; i < k; ++i)
      if (sel[i] >= 0) sorted[n++] = sel[i];
    qsort(sorted, (size_t)n, sizeof(int32_t), cmp_i32);
    for (int32_t i = 1; i < n; ++i)
      if (sorted[i] == sorted[i - 1]) status |= HSO_STATUS_SEL_DUP;
    free(sorted);
  }
  if (status != 0) {
    for (int32_t i = 0; i < k; ++i) out[i] = -1;
    return status;
  }

  /* Step 2: advance this stream's LRU clock (once per call). */
  const int32_t t = ++st->t[0];

  /* Step 3: one pass over the selections in index order.
   *   padding        -> -1
   *   resident row   -> its ring slot C + (p mod R); the resident test comes
   *                     before the lookup
   *   cached (hit)   -> its slot, stamped with t
   *   otherwise      -> remembered as a miss, in ascending selection index */
  int32_t* miss_idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
  int32_t n_miss = 0;
  for (int32_t i = 0; i < k; ++i) {
    int32_t p = sel[i];
    if (p == -1) {
      out[i] = -1;
      counters[HSO_N_PAD]++;
    } else if (R > 0 && (int64_t)p >= ctx - R) {
      out[i] = C + (p % R);
      counters[HSO_N_RES]++;
    } else if (st->pos2slot[p] >= 0) {
      int32_t s = st->pos2slot[p];
      out[i] = s;
      st->last_use[s] = t;
      counters[HSO_N_HIT]++;
    } else {
      miss_idx[n_miss++] = i;
    }
  }

  /* Step 4: the slots not referenced this step, in LRU order
   * (last_use ascending, then slot ascending). */
  lru_key* order = (lru_key*)malloc(sizeof(lru_key) * (size_t)C);
  int32_t n_free = 0;
  for (int32_t s = 0; s < C; ++s) {
    if (st->last_use[s] != t) {
      order[n_free].last_use = st->last_use[s];
      order[n_free].slot = s;
      n_free++;
    }
  }
  qsort(order, (size_t)n_free, sizeof(lru_key), cmp_lru);
  /* n_free >= n_miss holds because k <= C: every referenced slot is a hit. */

  /* Step 5: the j-th miss takes the j-th slot of that order. */
  for (int32_t j = 0; j < n_miss; ++j) {
    int32_t i = miss_idx[j];
    int32_t p = sel[i];
    int32_t s = order[j].slot;
    int32_t q = st->slot2pos[s];
    log_slot[j] = s;
    log_old[j] = q;
    if (q >= 0) {
      st->pos2slot[q] = -1;
      counters[HSO_N_EVICT]++;
    }
    st->pos2slot[p] = s;
    st->slot2pos[s] = p;
    st->last_use[s] = t;
    if (!(flags & HSO_FLAG_NO_IO) && st->slots && st->host) copy_row(st, s, p);
    out[i] = s;
  }
  counters[HSO_N_MISS] = n_miss;
  counters[HSO_BYTES] = (flags & HSO_FLAG_NO_IO) ? 0 : (int64_t)n_miss * st->row_bytes;

  free(order);
  free(miss_idx);
  return 0;
}

/* Load the resident window of a context of length ctx from the host rows:
 * ring slot C + (p mod R) holds row p for p in [max(0, ctx-R), ctx). */
int hso_seed_window(const hso_stream* st, int64_t ctx) {
  if (st->R <= 0) return 0;
  if (ctx < 0 || ctx > st->l_cap || !st->slots || !st->host) return -1;
  int64_t lo = ctx - st->R > 0 ? ctx - st->R : 0;
  for (int64_t p = lo; p < ctx; ++p) copy_row(st, st->C + p % st->R, p);
  return 0;
}

/* Append the row of position ctx (the context grows by one): the host history
 * gets the row and, when there is a resident window, so does ring slot
 * C + (ctx mod R), which drops position ctx - R out of the window. */
int hso_append(const hso_stream* st, const uint8_t* row, int64_t ctx) {
  if (ctx < 0 || ctx >= st->l_cap || !st->host) return -1;
  memcpy(st->host + ctx * st->row_bytes, row, (size_t)st->row_bytes);
  if (st->R > 0 && st->slots)
    memcpy(st->slots + (st->C + ctx % st->R) * st->row_bytes, row, (size_t)st->row_bytes);
  return 0;
}
