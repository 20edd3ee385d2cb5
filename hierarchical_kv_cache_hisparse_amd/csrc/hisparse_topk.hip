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
// HBM; the answer needs no sort.  Three launches:
//   1. histogram: workgroups of 256 threads over 4096-position chunks build
//      an LDS histogram of the top 12 bits of an order-preserving key and
//      add its non-zero bins to the row's global histogram;
//   2. filter: every workgroup finds the bin where the count from the top
//      reaches k (a block scan over the 4096 bins), re-reads its chunk (same
//      grid shape, so the same XCD and, mostly, its L2), sets the bits of
//      the positions above that bin in a per-row bitmap and appends the
//      positions inside it to a candidate list;
//   3. finish (one workgroup per row): a radix select over the candidates'
//      remaining key bits and position picks exactly the missing count, sets
//      their bits, and the bitmap is turned into the ascending position list
//      with one block scan of per-thread popcounts.
// The histogram and candidate counters are zero on entry and zeroed again by
// the finish kernel, so the three launches capture into a HIP graph with no
// memset nodes and replay any number of times.
#include <hip/hip_runtime.h>

#include "hisparse_device.h"
#include "hisparse_internal.h"

namespace hsp {
namespace {

constexpr int kTkPerThread = kTopkChunk / kTopkThreads;  // 16 scores per thread
constexpr int kTkWords = kTopkChunk / 32;                // bitmap words per chunk

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

__device__ __forceinline__ int64_t row_ctx(const TopkArgs& a, int b) {
  int64_t c = a.ctx_len[b];
  return c < 0 ? 0 : (c > a.max_len ? a.max_len : c);
}

// The scores of one chunk: thread tid holds positions chunk0 + 1024 j +
// 4 tid + e (j, e < 4), loaded as 16-byte vectors where the whole vector is
// inside [0, ctx).
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int64_t chunk0,
                                           int64_t ctx, int tid, float (&v)[kTkPerThread]) {
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

// Level-1 threshold of a row from its histogram, for a block of BD threads:
// sh[0] = the bin where the count from the top reaches k (-1 when the row
// has at most k positions: all of them are taken), sh[1] = the count in the
// bins above it.  sh[2 ..] holds the per-wave sums.  Ends with a barrier.
template <int BD>
__device__ void find_threshold(const uint32_t* __restrict__ gh, int k, int* sh, int tid) {
  constexpr int P = kTopkBins / BD;
  const int lane = tid & 63, wave = tid >> 6;
  const int top = kTopkBins - 1 - tid * P;  // this thread: bins top, top-1, ..
  uint32_t c[P];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    c[i] = gh[top - i];
    sum += (int)c[i];
  }
  const int incl = wave_inclusive_scan(sum);
  int* wsum = sh + 2;
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
  if (total > k && excl < k && excl + sum >= k) {  // exactly one thread
    int cc = excl;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (cc + (int)c[i] >= k) {
        sh[0] = top - i;
        sh[1] = cc;
        break;
      }
      cc += (int)c[i];
    }
  }
  if (total <= k && tid == 0) {
    sh[0] = -1;
    sh[1] = total;
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

// ---- 2. filter: bitmap of sure picks, list of boundary-bin candidates -----
__global__ void __launch_bounds__(kTopkThreads) topk_filter_kernel(TopkArgs a) {
  __shared__ uint32_t bm[kTkWords];
  __shared__ int sh[2 + kTopkThreads / 64];
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int64_t ctx = row_ctx(a, b);
  const int64_t chunk0 = (int64_t)blockIdx.x * kTopkChunk;
  if (chunk0 >= ctx) return;
  float v[kTkPerThread];
  load_chunk(a.scores + (int64_t)b * a.row_stride, chunk0, ctx, tid, v);
  for (int i = tid; i < kTkWords; i += kTopkThreads) bm[i] = 0u;
  find_threshold<kTopkThreads>(a.hist + (int64_t)b * kTopkBins, a.k, sh, tid);
  const int t = sh[0];
  uint32_t* cnt = a.cnt + (int64_t)b * kTopkCntStride;
  uint2* cand = reinterpret_cast<uint2*>(a.cand) + (int64_t)b * a.max_len;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int i = 0; i < kTkPerThread; ++i) {
    const int64_t p = chunk_pos(chunk0, tid, i);
    const bool valid = p < ctx;
    const uint32_t key = order_key(v[i]);
    const int bin = (int)(key >> 20);
    if (valid && bin > t) atomicOr(&bm[(int)(p - chunk0) >> 5], 1u << (p & 31));
    const bool is_cand = valid && bin == t;
    const uint64_t m = __ballot(is_cand);
    if (m) {  // one counter update per wave and round
      const int leader = __ffsll((unsigned long long)m) - 1;
      int base = 0;
      if (lane == leader) base = (int)atomicAdd(cnt, (uint32_t)__popcll(m));
      base = __shfl(base, leader);
      const int64_t slot = (int64_t)base + __popcll(m & below);
      if (is_cand && slot < a.max_len) cand[slot] = make_uint2(key, (uint32_t)p);
    }
  }
  lds_barrier();
  uint32_t* gbm = a.bitmap + (int64_t)b * a.bm_words + (int64_t)blockIdx.x * kTkWords;
  for (int i = tid; i < kTkWords; i += kTopkThreads) gbm[i] = bm[i];
}

// ---- 3. finish: exact boundary by radix select, emit ascending positions --
__global__ void __launch_bounds__(kTopkFinishThreads) topk_finish_kernel(TopkArgs a) {
  constexpr int BD = kTopkFinishThreads;
  __shared__ int sh[2 + BD / 64];
  __shared__ uint32_t dh[256];
  __shared__ int pick[2];
  __shared__ int wtot[BD / 64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t ctx = row_ctx(a, b);
  uint32_t* gh = a.hist + (int64_t)b * kTopkBins;
  uint32_t* cnt = a.cnt + (int64_t)b * kTopkCntStride;
  uint32_t* bmap = a.bitmap + (int64_t)b * a.bm_words;
  const uint2* cand = reinterpret_cast<const uint2*>(a.cand) + (int64_t)b * a.max_len;
  find_threshold<BD>(gh, a.k, sh, tid);
  const int t = sh[0];
  const int64_t nc_raw = t >= 0 ? (int64_t)*cnt : 0;
  const int nc = (int)(nc_raw < ctx ? nc_raw : ctx);  // <= ctx unless the workspace was not zeroed
  const int need0 = a.k - sh[1];  // candidates to take (t >= 0: 1 <= need0)
  if (t >= 0) {
    uint64_t T = 0;  // take the candidates whose key is >= T
    if (need0 < nc) {
      // MSD radix select of the need0-th largest candidate key (52 bits:
      // six 8-bit digits, then 4 bits).  Keys are unique, so exactly need0
      // candidates have a key >= the result.
      uint64_t prefix = 0, pmask = 0;
      int need = need0;
      for (int pass = 0; pass < 7; ++pass) {
        const int shift = pass < 6 ? 44 - 8 * pass : 0;
        const uint64_t dmask = pass < 6 ? 0xFFull : 0xFull;
        for (int i = tid; i < 256; i += BD) dh[i] = 0u;
        __syncthreads();
        for (int i = tid; i < nc; i += BD) {
          const uint64_t key = cand_key(cand[i]);
          if ((key & pmask) == prefix) atomicAdd(&dh[(int)((key >> shift) & dmask)], 1u);
        }
        __syncthreads();
        if (wave == 0) {  // digits from the top: lane l holds 255-4l .. 252-4l
          uint32_t c4[4];
          int s = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            c4[q] = dh[255 - 4 * lane - q];
            s += (int)c4[q];
          }
          const int incl = wave_inclusive_scan(s);
          const int excl = incl - s;
          if (excl < need && excl + s >= need) {
            int cc = excl;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (cc + (int)c4[q] >= need) {
                pick[0] = 255 - 4 * lane - q;
                pick[1] = cc;
                break;
              }
              cc += (int)c4[q];
            }
          }
        }
        __syncthreads();
        need -= pick[1];
        prefix |= (uint64_t)pick[0] << shift;
        pmask |= dmask << shift;
        __syncthreads();  // pick and dh are rewritten by the next pass
      }
      T = prefix;
    }
    for (int i = tid; i < nc; i += BD) {
      const uint2 c = cand[i];
      if (cand_key(c) >= T && (int64_t)c.y < ctx) atomicOr(&bmap[c.y >> 5], 1u << (c.y & 31));
    }
  }
  __threadfence();
  __syncthreads();

  // bitmap -> ascending positions: contiguous words per thread, block scan
  const int nw = (int)((ctx + 31) >> 5);
  const int wpt = (nw + BD - 1) / BD;
  const int w0 = tid * wpt;
  const int w1 = w0 + wpt < nw ? w0 + wpt : nw;
  int mine = 0;
  for (int w = w0; w < w1; ++w)
    mine += __popc(__hip_atomic_load(&bmap[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
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
  for (int w = w0; w < w1; ++w) {
    uint32_t word = __hip_atomic_load(&bmap[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (word) {
      const int bit = __ffs(word) - 1;
      if (o < a.k) out[o] = w * 32 + bit;
      ++o;
      word &= word - 1u;
    }
  }
  for (int i = total + tid; i < a.k; i += BD) out[i] = -1;
  // leave the histogram and the candidate counter zero for the next call
  for (int i = tid; i < kTopkBins; i += BD) gh[i] = 0u;
  if (tid == 0) *cnt = 0u;
}

}  // namespace

TopkLayout topk_layout(int rows, int64_t max_len) {
  TopkLayout l{};
  const int64_t chunks = (max_len + kTopkChunk - 1) / kTopkChunk;
  l.bm_words = chunks * (kTopkChunk / 32);
  l.hist = 0;
  l.cnt = align256((size_t)rows * kTopkBins * 4);
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
  hipLaunchKernelGGL(topk_finish_kernel, dim3(a.rows), dim3(kTopkFinishThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hsp
