// gfx950 kernels of the top-k selection step that feeds the resolver: per
// row of indexer scores (one request of one layer; one score per token for
// DSA-style selection, per page for Quest-style selection), the k positions
// with the largest scores among [0, ctx), equal scores going to the lower
// position, written in ascending position order and padded with -1.
//
// Source: "HiSparse: Scaling Sparse-Attention Decoding with Hierarchical KV
// Cache Management" (Abstract): decoding attends to the top-k positions an
// indexer picks, and the cache does not depend on which indexer; the tie and
// order rules are this library's readings (the pages give none).
//
// Design for CDNA4.  The step reads one float per position and is bound by
// HBM; the answer needs no sort.  Three launches (kernel boundaries are the
// only cross-workgroup synchronization: on this multi-XCD part a device-scope
// release fence inside a kernel writes back the XCD's L2, which costs far
// more per workgroup than a launch):
//   1. histogram: workgroups of 256 threads over 4096-position chunks build
//      an LDS histogram of the top 12 bits of an order-preserving key and
//      add its non-zero bins to the row's global histogram;
//   2. filter: every workgroup finds the bin where the count from the top
//      reaches k (a block scan over the 4096 bins), re-reads its chunk (same
//      grid shape, so the same XCD and, mostly, its L2), sets the bits of
//      the positions above that bin in a per-row bitmap and appends the
//      positions inside it to a candidate list (one global counter update
//      per workgroup), counting them by the next 12 key bits (the level-2
//      histogram);
//   3. finish (one workgroup of 1024 threads per row): one crossing search
//      over the level-2 histogram; a level-2 bin needed whole is taken
//      whole, else its candidates (at most 512) rank themselves by direct
//      counting over (remaining key bits, inverted position), and larger
//      ties fall back to a radix select over those bits; marks go to an LDS
//      copy of the bitmap, which becomes the ascending position list through
//      one block scan of per-thread popcounts.
// The histogram and the candidate counter are zero on entry and zeroed again
// by the finish kernel, so the three launches capture into a HIP graph with
// no memset nodes and replay any number of times.
#include <hip/hip_runtime.h>

#include "hisparse_device.h"
#include "hisparse_topk_internal.h"

namespace hsp {
namespace {

constexpr int kTkPerThread = kTopkChunk / kTopkThreads;  // 16 scores per thread
constexpr int kTkWords = kTopkChunk / 32;                // bitmap words per chunk
constexpr int kTkFinishThreads = 1024;                   // finish: one workgroup per row
constexpr int kTkRankMax = 512;                          // last-bin candidates ranked directly
constexpr int kTkOverlayWords = 8192;                    // LDS bitmap overlay (rows <= 256 Ki)
constexpr int kTkWordsReg = kTkOverlayWords / kTkFinishThreads;  // bitmap words per thread
constexpr int kTkCandReg = 2;                            // candidates per thread loaded up front
static_assert(kTkCandReg == 2, "the rank loop picks cr[0] or cr[1]");
constexpr int kCwCand = 0;                               // per-row counter words: candidates,
constexpr int kCwT = 1;                                  // threshold bin (-1: take every position),
constexpr int kCwAbove = 2;                              // positions in the bins above it

// Order-preserving key of a finite or infinite float: a larger score gives a
// larger unsigned key; -0 and +0 map to the same key (they are equal scores).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Key of a candidate inside its level-1 bin: the key's low 20 bits, then the
// position inverted so that a lower position ranks higher.  Unique per row.
__device__ __forceinline__ uint64_t cand_key(uint2 c) {
  return ((uint64_t)(c.x & 0xFFFFFu) << 32) | (uint64_t)(0xFFFFFFFFu - c.y);
}

__device__ __forceinline__ uint32_t load_l2(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int64_t row_ctx(const TopkArgs& a, int b) {
  int64_t c = a.ctx_len[b];
  return c < 0 ? 0 : (c > a.max_len ? a.max_len : c);
}

// The scores of one chunk: thread tid holds positions chunk0 + 1024 j +
// 4 tid + e (j, e < 4), loaded as 16-byte vectors where the whole vector is
// inside [0, ctx).
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int64_t chunk0,
                                           int64_t ctx, int tid, float (&v)[kTkPerThread]) {
  if (chunk0 + kTopkChunk <= ctx) {
    // a whole chunk (every chunk of a row but its last): four 16-byte loads
    // with no branch between them, so all four are in flight at once (behind
    // per-lane branches the compiler waits for each before the next)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 x =
          *reinterpret_cast<const float4*>(row + chunk0 + j * (4 * kTopkThreads) + 4 * tid);
      v[4 * j + 0] = x.x;
      v[4 * j + 1] = x.y;
      v[4 * j + 2] = x.z;
      v[4 * j + 3] = x.w;
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t p0 = chunk0 + j * (4 * kTopkThreads) + 4 * tid;
    if (p0 + 4 <= ctx) {
      const float4 x = *reinterpret_cast<const float4*>(row + p0);
      v[4 * j + 0] = x.x;
      v[4 * j + 1] = x.y;
      v[4 * j + 2] = x.z;
      v[4 * j + 3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * j + e] = (p0 + e < ctx) ? row[p0 + e] : 0.f;
    }
  }
}

__device__ __forceinline__ int64_t chunk_pos(int64_t chunk0, int tid, int i) {
  return chunk0 + (i >> 2) * (4 * kTopkThreads) + 4 * tid + (i & 3);
}

// Over 4096 bins taken from the top, for a block of BD threads: the
// bin where the running count reaches `need`, into sh[0], the count in the
// bins above it, into sh[1], and the count in that bin, into sh[2]; when all
// bins hold fewer than `need`, sh[0] = -1, sh[1] = the total and sh[2] = 0.
// sh[3 ..] holds per-wave sums.  Starts and ends with a barrier.
template <int BD, typename Load>
__device__ void find_crossing(Load load, int need, int* sh, int tid) {
  constexpr int P = kTopkBins / BD;
  const int lane = tid & 63, wave = tid >> 6;
  const int top = kTopkBins - 1 - tid * P;  // this thread: bins top, top-1, ..
  uint32_t c[P];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    c[i] = load(top - i);
    sum += (int)c[i];
  }
  const int incl = wave_inclusive_scan(sum);
  int* wsum = sh + 3;
  __syncthreads();
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < BD / 64; ++w) {
    const int x = wsum[w];
    before += w < wave ? x : 0;
    total += x;
  }
  const int excl = before + incl - sum;
  if (total >= need && excl < need && excl + sum >= need) {  // exactly one thread
    int cc = excl;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (cc + (int)c[i] >= need) {
        sh[0] = top - i;
        sh[1] = cc;
        sh[2] = (int)c[i];
        break;
      }
      cc += (int)c[i];
    }
  }
  if (total < need && tid == 0) {
    sh[0] = -1;
    sh[1] = total;
    sh[2] = 0;
  }
  __syncthreads();
}

// ---- 1. level-1 histogram -------------------------------------------------
__global__ void __launch_bounds__(kTopkThreads) topk_hist_kernel(TopkArgs a) {
  __shared__ uint32_t h[kTopkBins];
  const int b = blockIdx.y, tid = threadIdx.x;
  const int64_t ctx = row_ctx(a, b);
  const int64_t chunk0 = (int64_t)blockIdx.x * kTopkChunk;
  if (chunk0 >= ctx) return;
  for (int i = tid; i < kTopkBins; i += kTopkThreads) h[i] = 0u;
  float v[kTkPerThread];
  load_chunk(a.scores + (int64_t)b * a.row_stride, chunk0, ctx, tid, v);
  lds_barrier();
#pragma unroll
  for (int i = 0; i < kTkPerThread; ++i)
    if (chunk_pos(chunk0, tid, i) < ctx) atomicAdd(&h[order_key(v[i]) >> 20], 1u);
  lds_barrier();
  uint32_t* gh = a.hist + (int64_t)b * kTopkBins;
  for (int i = tid; i < kTopkBins; i += kTopkThreads) {
    const uint32_t c = h[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// ---- 3. finish: exact boundary among the candidates, then the bitmap as an
// ascending position list; leaves the row's histograms and counter zero.
//
// The candidates share the top 12 key bits (bin t).  The filter also counted
// them by the next 12 bits (the level-2 histogram), so one crossing search
// over it gives the level-2 bin and how many of its candidates are needed.
// If the bin is needed whole, every candidate at or above it is taken; if it
// holds at most kTkRankMax candidates, each of them counts the bin's
// candidates with a larger (score bits, inverted position) key and is taken
// when fewer than the needed number outrank it; otherwise (a very large tie)
// a radix select goes on over the remaining 8 score bits and the inverted
// position (8, 12, 12, 8 bits), stopping once a digit bin is taken whole.
// Marks go to an LDS overlay of the bitmap for rows of up to 256 Ki
// positions, to the global bitmap otherwise.  Everything the kernel reads
// from memory that does not depend on another read -- the row's counters,
// the level-2 histogram, the thread's bitmap words and its first
// candidates -- is requested at once at the start, so the kernel waits for
// one memory round trip before its LDS work.
__global__ void __launch_bounds__(kTkFinishThreads) topk_finish_kernel(TopkArgs a) {
  constexpr int BD = kTkFinishThreads;
  constexpr int kShift[4] = {32, 20, 8, 0};
  constexpr int kWidth[4] = {8, 12, 12, 8};
  __shared__ uint32_t dh[kTopkBins];
  __shared__ uint32_t ov[kTkOverlayWords + kTkOverlayWords / 8];  // word w at w + w/8
  __shared__ uint64_t rk[kTkRankMax];
  __shared__ int sh[3 + BD / 64];
  __shared__ int wtot[BD / 64];
  __shared__ int nrank;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t ctx = row_ctx(a, b);
  uint32_t* gh = a.hist + (int64_t)b * kTopkBins;
  uint32_t* gh2 = a.hist2 + (int64_t)b * kTopkBins;
  uint32_t* cw = a.cnt + (int64_t)b * kTopkCntStride;
  uint32_t* bmap = a.bitmap + (int64_t)b * a.bm_words;
  const uint2* cand = reinterpret_cast<const uint2*>(a.cand) + (int64_t)b * a.max_len;
  const int nw = (int)((ctx + 31) >> 5);
  const bool overlay = nw <= kTkOverlayWords;
  // words per thread: 4 or 8 with the overlay (aligned 16-byte loads), else
  // an even share
  const int wpt = overlay ? (nw <= 4 * BD ? 4 : kTkWordsReg) : (nw + BD - 1) / BD;
  const int w0 = tid * wpt < nw ? tid * wpt : nw;
  const int w1 = w0 + wpt < nw ? w0 + wpt : nw;
  // threshold bin and count above it, published by the row's first filter
  // workgroup (a row with ctx = 0 has no filter workgroups and takes nothing)
  const int t_raw = (int)cw[kCwT];
  const int above_raw = (int)cw[kCwAbove];
  const int64_t nc_raw = (int64_t)cw[kCwCand];
  uint2 cr[kTkCandReg];
#pragma unroll
  for (int j = 0; j < kTkCandReg; ++j) {
    const int i = tid + j * BD;
    cr[j] = i < a.max_len ? cand[i] : make_uint2(0u, 0u);
  }
  uint32_t wv[kTkWordsReg];
  if (overlay && w0 + wpt <= w1) {
    const uint4 x = reinterpret_cast<const uint4*>(bmap + w0)[0];
    const uint4 y = wpt == 8 ? reinterpret_cast<const uint4*>(bmap + w0)[1] : make_uint4(0, 0, 0, 0);
    wv[0] = x.x; wv[1] = x.y; wv[2] = x.z; wv[3] = x.w;
    wv[4] = y.x; wv[5] = y.y; wv[6] = y.z; wv[7] = y.w;
  } else {
#pragma unroll
    for (int j = 0; j < kTkWordsReg; ++j) wv[j] = (overlay && w0 + j < w1) ? bmap[w0 + j] : 0u;
  }
  auto ovi = [](int w) { return w + (w >> 3); };
  if (overlay)
    for (int i = tid; i < nw; i += BD) ov[ovi(i)] = 0u;
  if (tid == 0) nrank = 0;
  const int t = ctx > 0 ? t_raw : -1;
  const int above = ctx > 0 ? above_raw : 0;
  const int nc = t >= 0 ? (int)(nc_raw < ctx ? nc_raw : ctx) : 0;  // <= ctx unless not zero-filled
  const int need0 = a.k - above;                                     // t >= 0: 1 <= need0
  // the level-2 crossing, computed whether or not it is needed (its loads
  // join the others; its barriers also publish the overlay clearing)
  find_crossing<BD>([&](int i) { return gh2[i]; }, need0, sh, tid);
  // body(c) for this thread's candidates: the first ones from registers
  auto for_cands = [&](auto&& body) {
#pragma unroll
    for (int j = 0; j < kTkCandReg; ++j)
      if (tid + j * BD < nc) body(cr[j]);
    for (int i = tid + kTkCandReg * BD; i < nc; i += BD) body(cand[i]);
  };
  auto mark = [&](uint32_t p) {
    if ((int64_t)p >= ctx) return;
    if (overlay)
      atomicOr(&ov[ovi((int)(p >> 5))], 1u << (p & 31));
    else
      atomicOr(&bmap[p >> 5], 1u << (p & 31));
  };
  if (t >= 0) {
    if (need0 >= nc) {  // the whole boundary bin is taken
      for_cands([&](uint2 c) { mark(c.y); });
    } else {
      const int d2 = sh[0] < 0 ? 0 : sh[0];  // (-1 only if the workspace was not zero-filled)
      const int need2 = need0 - sh[1];
      const int in2 = sh[2];
      if (in2 == need2 || in2 <= kTkRankMax) {
        // take everything above level-2 bin d2; inside it, all of it when
        // it is needed whole, else the need2 best-ranked candidates
        const bool whole = in2 == need2;
        // (uniform trip counts: every lane takes part in the ballots)
        const uint64_t below = (1ull << lane) - 1ull;
        for (int i0 = 0; i0 < nc; i0 += BD) {
          const int i = i0 + tid;
          const int j = (i - tid) / BD;
          const bool have = i < nc;
          const uint2 c = !have ? make_uint2(0u, 0u) : (j < kTkCandReg ? (j == 0 ? cr[0] : cr[1]) : cand[i]);
          const int d = (int)((c.x >> 8) & 0xFFFu);
          if (have && (d > d2 || (whole && d == d2))) mark(c.y);
          const bool put = have && !whole && d == d2;
          const uint64_t m = __ballot(put);
          if (m) {  // one LDS counter update per wave
            int base = 0;
            if (lane == 0) base = atomicAdd(&nrank, __popcll(m));
            base = __shfl(base, 0);
            const int slot = base + __popcll(m & below);
            if (put && slot < kTkRankMax) rk[slot] = cand_key(c);
          }
        }
        __syncthreads();
        const int g = nrank < kTkRankMax ? nrank : kTkRankMax;
        for (int i = tid; i < g; i += BD) {
          const uint64_t key = rk[i];
          int rank = 0;
          int j = 0;
          for (; j + 8 <= g; j += 8) {  // eight independent LDS reads in flight
#pragma unroll
            for (int q = 0; q < 8; ++q) rank += rk[j + q] > key;
          }
          for (; j < g; ++j) rank += rk[j] > key;
          if (rank < need2) mark(0xFFFFFFFFu - (uint32_t)key);
        }
      } else {
        uint64_t prefix = (uint64_t)d2 << 40, pmask = 0xFFFull << 40;
        int need = need2;
        for (int pass = 0; pass < 4; ++pass) {
          const int shift = kShift[pass];
          const uint64_t dmask = (1ull << kWidth[pass]) - 1ull;
          for (int i = tid; i < kTopkBins; i += BD) dh[i] = 0u;
          __syncthreads();
          for_cands([&](uint2 c) {
            const uint64_t key = cand_key(c);
            if ((key & pmask) == prefix) atomicAdd(&dh[(int)((key >> shift) & dmask)], 1u);
          });
          __syncthreads();  // digit histogram complete
          find_crossing<BD>([&](int i) { return dh[i]; }, need, sh, tid);
          const int d = sh[0];
          if (d < 0) break;  // only if the workspace was not zero-filled
          need -= sh[1];
          prefix |= (uint64_t)d << shift;
          pmask |= dmask << shift;
          const bool whole = sh[2] == need;
          __syncthreads();  // dh and sh are rewritten by the next pass
          if (whole) break;
        }
        for_cands([&](uint2 c) {
          if (cand_key(c) >= prefix) mark(c.y);
        });
      }
    }
  }
  // Global marks are device-scope atomics, performed in L2, and read back
  // below with L1-bypassing loads: a workgroup barrier (which waits for this
  // workgroup's outstanding atomics) orders them, as it orders the LDS
  // marks.  An agent-scope fence would also write back the XCD's L2.
  __syncthreads();

  // bitmap -> ascending positions: contiguous words per thread, block scan
  // of the popcounts
  int mine = 0;
  if (overlay) {
#pragma unroll
    for (int j = 0; j < kTkWordsReg; ++j)
      if (w0 + j < w1) mine += __popc(wv[j] | ov[ovi(w0 + j)]);
  } else {
    for (int w = w0; w < w1; ++w) mine += __popc(load_l2(&bmap[w]));
  }
  const int incl = wave_inclusive_scan(mine);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < BD / 64; ++w) {
    const int x = wtot[w];
    before += w < wave ? x : 0;
    total += x;
  }
  int o = before + incl - mine;
  int32_t* out = a.out + (int64_t)b * a.k;
  auto emit = [&](uint32_t word, int w) {
    while (word) {
      const int bit = __ffs(word) - 1;
      if (o < a.k) out[o] = w * 32 + bit;
      ++o;
      word &= word - 1u;
    }
  };
  if (overlay) {
#pragma unroll
    for (int j = 0; j < kTkWordsReg; ++j)
      if (w0 + j < w1) emit(wv[j] | ov[ovi(w0 + j)], w0 + j);
  } else {
    for (int w = w0; w < w1; ++w) emit(load_l2(&bmap[w]), w);
  }
  for (int i = total + tid; i < a.k; i += BD) out[i] = -1;
  for (int i = tid; i < kTopkBins; i += BD) {
    gh[i] = 0u;
    gh2[i] = 0u;
  }
  if (tid == 0) cw[kCwCand] = 0u;
}

// ---- 2. filter: bitmap of sure picks, list of boundary-bin candidates -----
__global__ void __launch_bounds__(kTopkThreads) topk_filter_kernel(TopkArgs a) {
  __shared__ uint32_t bm[kTkWords];
  __shared__ int sh[3 + kTopkThreads / 64];
  __shared__ int wg_cnt, wg_base;
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int64_t ctx = row_ctx(a, b);
  const int64_t chunk0 = (int64_t)blockIdx.x * kTopkChunk;
  uint32_t* cw = a.cnt + (int64_t)b * kTopkCntStride;
  if (chunk0 >= ctx) return;
  {
    float v[kTkPerThread];
    load_chunk(a.scores + (int64_t)b * a.row_stride, chunk0, ctx, tid, v);
    for (int i = tid; i < kTkWords; i += kTopkThreads) bm[i] = 0u;
    if (tid == 0) wg_cnt = 0;
    const uint32_t* gh = a.hist + (int64_t)b * kTopkBins;
    find_crossing<kTopkThreads>([&](int i) { return gh[i]; }, a.k, sh, tid);
    const int t = sh[0];
    if (blockIdx.x == 0 && tid == 0) {  // every workgroup of the row finds the same
      cw[kCwT] = (uint32_t)t;
      cw[kCwAbove] = (uint32_t)sh[1];
    }
    bool is_cand[kTkPerThread];
    int n_wave = 0;
#pragma unroll
    for (int i = 0; i < kTkPerThread; ++i) {
      const int64_t p = chunk_pos(chunk0, tid, i);
      const bool valid = p < ctx;
      const int bin = (int)(order_key(v[i]) >> 20);
      if (valid && bin > t) atomicOr(&bm[(int)(p - chunk0) >> 5], 1u << (p & 31));
      is_cand[i] = valid && bin == t;
      n_wave += __popcll(__ballot(is_cand[i]));
    }
    int woff = 0;
    if (lane == 0 && n_wave) woff = atomicAdd(&wg_cnt, n_wave);
    woff = __shfl(woff, 0);
    lds_barrier();  // bm complete, wg_cnt final
    if (tid == 0) wg_base = wg_cnt ? (int)atomicAdd(&cw[kCwCand], (uint32_t)wg_cnt) : 0;
    uint32_t* gbm = a.bitmap + (int64_t)b * a.bm_words + (int64_t)blockIdx.x * kTkWords;
    for (int i = tid; i < kTkWords; i += kTopkThreads) gbm[i] = bm[i];
    __syncthreads();  // wg_base
    if (n_wave) {
      uint2* cand = reinterpret_cast<uint2*>(a.cand) + (int64_t)b * a.max_len;
      uint32_t* gh2 = a.hist2 + (int64_t)b * kTopkBins;
      const uint64_t below = (1ull << lane) - 1ull;
      int64_t run = (int64_t)wg_base + woff;
#pragma unroll
      for (int i = 0; i < kTkPerThread; ++i) {
        const uint64_t m = __ballot(is_cand[i]);
        const int64_t slot = run + __popcll(m & below);
        if (is_cand[i] && slot < a.max_len) {
          const uint32_t key = order_key(v[i]);
          cand[slot] = make_uint2(key, (uint32_t)chunk_pos(chunk0, tid, i));
          atomicAdd(&gh2[(key >> 8) & 0xFFFu], 1u);
        }
        run += __popcll(m);
      }
    }
  }
}

}  // namespace

TopkLayout topk_layout(int rows, int64_t max_len) {
  TopkLayout l{};
  const int64_t chunks = (max_len + kTopkChunk - 1) / kTopkChunk;
  l.bm_words = chunks * (kTopkChunk / 32);
  l.hist = 0;
  l.hist2 = align256((size_t)rows * kTopkBins * 4);
  l.cnt = l.hist2 + align256((size_t)rows * kTopkBins * 4);
  l.bitmap = l.cnt + align256((size_t)rows * kTopkCntStride * 4);
  l.cand = l.bitmap + align256((size_t)rows * (size_t)l.bm_words * 4);
  l.total = l.cand + align256((size_t)rows * (size_t)max_len * 8);
  return l;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  const int chunks = (int)((a.max_len + kTopkChunk - 1) / kTopkChunk);
  const dim3 grid(chunks, a.rows);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kTopkThreads), 0, s, a);
  hipLaunchKernelGGL(topk_filter_kernel, grid, dim3(kTopkThreads), 0, s, a);
  hipLaunchKernelGGL(topk_finish_kernel, dim3(a.rows), dim3(kTkFinishThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hsp
