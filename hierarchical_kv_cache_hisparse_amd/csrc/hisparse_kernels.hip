// gfx950 kernels of libhisparse: per-layer selection resolution of a two-tier
// (host + GPU) KV cache, the miss fetch over the host link, and the small
// state-management kernels around them.
//
// Sources (pages, cited by title and section):
//   [P3] "HiSparse: Scaling Sparse-Attention Decoding with Hierarchical KV
//        Cache Management" -- Abstract: per layer, the selections are resolved
//        by hit detection, LRU replacement and host-to-device fetches inside
//        the decode graph; AI Summary: the three happen in a single pass.
//   [P2] "Hybrid HiSparse" -- Timeline: rows are resident, hot or missing,
//        told apart in one pass by one graph-capturable kernel.
//   [P1] "HiSparse" -- Timeline: only missing rows the top-k hits are copied.
//
// Design for CDNA4 (not a translation of the pages' CUDA kernel):
//   * one workgroup per stream (request, layer); the work is latency-bound
//     (two dependent HBM round trips: selections, then the position->slot
//     gathers), so everything else stays in LDS and registers;
//   * each thread owns `IPT` selections and `IPT` LRU-order entries, strided
//     by the workgroup size, so every global load is coalesced except the
//     position->slot gathers;
//   * three ordered compactions (misses by selection index, unreferenced
//     slots by LRU order, referenced slots by slot number) use 64-lane
//     ballots plus per-(round, wave) counts in LDS, one barrier each;
//   * LRU victim order without a sort: each stream keeps its slots in
//     (last_use, slot) order.  Slots referenced in a step all get the newest
//     stamp, so the next order is "unreferenced, not evicted, in old order"
//     followed by "referenced or refilled, by slot number"; the victims are
//     the first M unreferenced entries of the old order.  O(C) per step;
//   * the miss fetch is a separate launch fanned out over the whole chip:
//     16-byte non-temporal loads straight from mapped host memory, written to
//     the slot rows in HBM.  No MFMA anywhere: nothing here is a contraction.
#include <hip/hip_runtime.h>

#include "hisparse_internal.h"

namespace hsp {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

enum Cls : int { kNone = 0, kPad = 1, kRes = 2, kHit = 3, kMiss = 4, kBad = 5 };

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

struct StreamPtrs {
  int32_t* hdr;
  int32_t* pos2slot;
  int32_t* slot2pos;
  int32_t* last_use;
  int32_t* order;
  int32_t* evict;
  int32_t* miss;
};

__device__ __forceinline__ StreamPtrs stream_ptrs(const StreamView& v, int layer, int b) {
  uint8_t* blk = v.meta + v.stream_base + (int64_t)(layer * v.B + b) * v.stream_stride;
  StreamPtrs s;
  s.hdr = (int32_t*)(blk + v.off_hdr);
  s.pos2slot = (int32_t*)(blk + v.off_pos2slot);
  s.slot2pos = (int32_t*)(blk + v.off_slot2pos);
  s.last_use = (int32_t*)(blk + v.off_last_use);
  s.order = (int32_t*)(blk + v.off_order);
  s.evict = (int32_t*)(blk + v.off_evict);
  s.miss = (int32_t*)(blk + v.off_miss);
  return s;
}

__device__ __forceinline__ uint32_t* status_word(const StreamView& v) {
  return (uint32_t*)v.meta;
}

// Ordered compaction, part 1: per round r, the lane's rank among the flagged
// lanes of its wave, and (lane 0) the wave's count into cnt[r*W + wave].
template <int IPT>
__device__ __forceinline__ void ballot_counts(const bool (&flag)[IPT], int* cnt, int W, int wave,
                                              int lane, int (&pre)[IPT]) {
  const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < IPT; ++r) {
    const uint64_t m = __ballot(flag[r]);
    pre[r] = __popcll(m & lt);
    if (lane == 0) cnt[r * W + wave] = __popcll(m);
  }
}

// Ordered compaction, part 2 (after a barrier): off[r] = number of flagged
// items before (round r, this wave); returns the total.  Every wave computes
// its own offsets, so no extra barrier is needed.
template <int IPT>
__device__ __forceinline__ int wave_offsets(const int* cnt, int W, int wave, int lane,
                                            int (&off)[IPT]) {
#pragma unroll
  for (int r = 0; r < IPT; ++r) {
    const int lim = r * W + wave;
    int s = 0;
    for (int e = lane; e < lim; e += 64) s += cnt[e];
    off[r] = wave_sum(s);
  }
  int s = 0;
  for (int e = lane; e < IPT * W; e += 64) s += cnt[e];
  return wave_sum(s);
}

__device__ __forceinline__ bool test_bit(const uint32_t* bm, int s) {
  return (bm[s >> 5] >> (s & 31)) & 1u;
}

// ---------------------------------------------------------------------------
// Resolve: one workgroup per stream (request b of `layer`).
// ---------------------------------------------------------------------------
template <int IPT>
__global__ void __launch_bounds__(kMaxThreads)
    resolve_kernel(StreamView v, int layer, const int32_t* __restrict__ sel_all,
                   const int32_t* __restrict__ ctx_len, int32_t* __restrict__ out_all,
                   int32_t* __restrict__ sel_copy) {
  extern __shared__ int lds[];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int BD = blockDim.x;
  const int W = BD >> 6;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int C = v.C, R = v.R, k = v.k;
  const bool debug = (v.flags & HISPARSE_DEBUG_VALIDATE) != 0;
  const StreamPtrs st = stream_ptrs(v, layer, b);
  const int32_t* sel = sel_all + (int64_t)b * k;
  int32_t* out = out_all + (int64_t)b * k;

  // LDS: [bitmap C bits][slot2pos C][victims k][3 x count tables][misc 8][hash]
  const int nbm = (C + 31) >> 5;
  uint32_t* bitmap = (uint32_t*)lds;
  int* s2p = lds + nbm;
  int* victim = s2p + C;
  int* cntA = victim + k;
  int* cntB = cntA + IPT * W;
  int* cntC = cntB + IPT * W;
  int* misc = cntC + IPT * W;  // 0 status, 1 pad, 2 res, 3 hit, 4 evict
  int* hash = misc + 8;

  // ---- Phase A: independent loads, then the position->slot gathers -------
  const int32_t ctx = ctx_len[b];
  const int32_t t = st.hdr[kHdrT] + 1;  // one clock tick per resolve
  const bool ctx_ok = ctx >= 0 && ctx <= v.l_cap;
  if (tid < 8) misc[tid] = 0;
  for (int w = tid; w < nbm; w += BD) bitmap[w] = 0;

  int32_t p[IPT], o[IPT], slot[IPT];
  int cls[IPT];
#pragma unroll
  for (int r = 0; r < IPT; ++r) {
    const int i = r * BD + tid;
    p[r] = (i < k) ? sel[i] : -1;
    cls[r] = (i < k) ? kPad : kNone;
  }
#pragma unroll
  for (int r = 0; r < IPT; ++r) {
    const int x = r * BD + tid;
    if (x < C) {
      o[r] = st.order[x];
      s2p[x] = st.slot2pos[x];
    } else {
      o[r] = 0;
    }
  }
  uint32_t bad = ctx_ok ? 0u : (uint32_t)HISPARSE_STATUS_CTX_RANGE;
#pragma unroll
  for (int r = 0; r < IPT; ++r) {
    slot[r] = -1;
    if (cls[r] == kNone) continue;
    const int32_t q = p[r];
    if (q == -1) continue;  // padding
    if (q < -1 || q >= ctx) {
      bad |= HISPARSE_STATUS_SEL_RANGE;
      cls[r] = kBad;
    } else if (!ctx_ok) {
      cls[r] = kBad;
    } else if (R > 0 && q >= ctx - R) {
      cls[r] = kRes;  // resident window: tested before the cache lookup
    } else {
      cls[r] = kMiss;
      slot[r] = st.pos2slot[q];
    }
  }
  if (debug) {  // repeated positions: LDS open-addressing set of size H
    const int H = 2 << (31 - __clz(k));  // power of two > k... >= 2k
    for (int w = tid; w < H; w += BD) hash[w] = -1;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < IPT; ++r) {
      if (cls[r] == kNone || p[r] < 0) continue;
      uint32_t h = ((uint32_t)p[r] * 2654435761u) & (uint32_t)(H - 1);
      while (true) {
        const int prev = atomicCAS(&hash[h], -1, p[r]);
        if (prev == -1) break;
        if (prev == p[r]) {
          bad |= HISPARSE_STATUS_SEL_DUP;
          break;
        }
        h = (h + 1) & (uint32_t)(H - 1);
      }
    }
  }
  if (__syncthreads_or(bad != 0u)) {
    // Rejected row: leave the stream untouched, serve -1 everywhere.
    if (bad) atomicOr((uint32_t*)&misc[0], bad);
    __syncthreads();
    uint32_t err = (uint32_t)misc[0];
    if (err & (HISPARSE_STATUS_SEL_RANGE | HISPARSE_STATUS_CTX_RANGE))
      err &= ~(uint32_t)HISPARSE_STATUS_SEL_DUP;
#pragma unroll
    for (int r = 0; r < IPT; ++r) {
      const int i = r * BD + tid;
      if (i < k) {
        out[i] = -1;
        if (sel_copy) sel_copy[(int64_t)b * k + i] = p[r];
      }
    }
    if (tid == 0) {
      atomicOr(status_word(v), err);
      st.hdr[kHdrStatus] = (int32_t)err;
      for (int c = kHdrPad; c <= kHdrBytes; ++c) st.hdr[c] = 0;
    }
    return;
  }

  // ---- Phase B: serve padding, resident rows and hits; rank the misses -----
#pragma unroll
  for (int r = 0; r < IPT; ++r) {
    const int i = r * BD + tid;
    if (cls[r] == kMiss && slot[r] >= 0) cls[r] = kHit;
    if (cls[r] == kPad) {
      out[i] = -1;
    } else if (cls[r] == kRes) {
      out[i] = C + p[r] % R;
    } else if (cls[r] == kHit) {
      const int s = slot[r];
      out[i] = s;
      st.last_use[s] = t;
      atomicOr(&bitmap[s >> 5], 1u << (s & 31));
    }
    if (sel_copy && cls[r] != kNone) sel_copy[(int64_t)b * k + i] = p[r];
  }
#pragma unroll
  for (int r = 0; r < IPT; ++r) {
    const int np = __popcll(__ballot(cls[r] == kPad));
    const int nr = __popcll(__ballot(cls[r] == kRes));
    const int nh = __popcll(__ballot(cls[r] == kHit));
    if (lane == 0) {
      if (np) atomicAdd(&misc[1], np);
      if (nr) atomicAdd(&misc[2], nr);
      if (nh) atomicAdd(&misc[3], nh);
    }
  }
  bool flag[IPT];
  int pre[IPT], off[IPT], jm[IPT];
#pragma unroll
  for (int r = 0; r < IPT; ++r) flag[r] = cls[r] == kMiss;
  ballot_counts<IPT>(flag, cntA, W, wave, lane, pre);
  __syncthreads();  // hits marked, miss counts and class counters complete
  const int M = wave_offsets<IPT>(cntA, W, wave, lane, off);
  const int n_hit = misc[3];
#pragma unroll
  for (int r = 0; r < IPT; ++r) jm[r] = off[r] + pre[r];  // miss index j (ascending i)

  // ---- Phase C: victims = first M unreferenced slots in LRU order ----------
#pragma unroll
  for (int r = 0; r < IPT; ++r) {
    const int x = r * BD + tid;
    flag[r] = (x < C) && !test_bit(bitmap, o[r]);
  }
  ballot_counts<IPT>(flag, cntB, W, wave, lane, pre);
  __syncthreads();
  wave_offsets<IPT>(cntB, W, wave, lane, off);
#pragma unroll
  for (int r = 0; r < IPT; ++r) {
    if (!flag[r]) continue;
    const int u = off[r] + pre[r];
    if (u < M) {
      victim[u] = o[r];
      atomicOr(&bitmap[o[r] >> 5], 1u << (o[r] & 31));
    } else {
      st.order[u - M] = o[r];  // kept: old relative order, at the front
    }
  }
  __syncthreads();  // victims and the referenced-or-refilled bitmap complete

  // ---- Phase D: the j-th miss takes the j-th victim; update the maps -------
  int nev = 0;
#pragma unroll
  for (int r = 0; r < IPT; ++r) {
    if (cls[r] != kMiss) continue;
    const int i = r * BD + tid;
    const int j = jm[r];
    const int s = victim[j];
    const int q = s2p[s];
    reinterpret_cast<int2*>(st.evict)[j] = make_int2(s, q);
    if (q >= 0) {
      st.pos2slot[q] = -1;
      ++nev;
    }
    st.pos2slot[p[r]] = s;
    st.slot2pos[s] = p[r];
    st.last_use[s] = t;
    out[i] = s;
    reinterpret_cast<int2*>(st.miss)[j] = make_int2(s, p[r]);
  }
  nev = wave_sum(nev);
  if (lane == 0 && nev) atomicAdd(&misc[4], nev);

  // ---- Phase E: referenced-or-refilled slots go to the back, by slot -------
#pragma unroll
  for (int r = 0; r < IPT; ++r) {
    const int x = r * BD + tid;
    flag[r] = (x < C) && test_bit(bitmap, x);
  }
  ballot_counts<IPT>(flag, cntC, W, wave, lane, pre);
  __syncthreads();
  wave_offsets<IPT>(cntC, W, wave, lane, off);
  const int base = C - (n_hit + M);
#pragma unroll
  for (int r = 0; r < IPT; ++r)
    if (flag[r]) st.order[base + off[r] + pre[r]] = r * BD + tid;

  if (tid == 0) {
    st.hdr[kHdrT] = t;
    st.hdr[kHdrStatus] = 0;
    st.hdr[kHdrPad] = misc[1];
    st.hdr[kHdrRes] = misc[2];
    st.hdr[kHdrHit] = n_hit;
    st.hdr[kHdrMiss] = M;
    st.hdr[kHdrEvict] = misc[4];
    st.hdr[kHdrBytes] = (v.flags & HISPARSE_NO_IO) ? 0 : (int32_t)(M * v.row_bytes);
    *reinterpret_cast<int64_t*>(st.hdr + kHdrTotalMiss) += M;
    *reinterpret_cast<int64_t*>(st.hdr + kHdrTotalEvict) += misc[4];
    *reinterpret_cast<int64_t*>(st.hdr + kHdrTotalHit) += n_hit;
  }
}

// ---------------------------------------------------------------------------
// Miss fetch: copy every listed row from the host history into its slot.
// grid = (grid_x, B); each workgroup strides over its stream's 16-byte chunks.
// ---------------------------------------------------------------------------
template <int U>
__global__ void __launch_bounds__(kFetchThreads) fetch_kernel(StreamView v, int layer) {
  const int b = blockIdx.y;
  const StreamPtrs st = stream_ptrs(v, layer, b);
  const int M = st.hdr[kHdrMiss];
  const uint32_t cpr = (uint32_t)(v.row_bytes >> 4);
  const uint32_t total = (uint32_t)M * cpr;
  const uint32_t first = blockIdx.x * (kFetchThreads * U);
  if (first >= total) return;
  const int2* ml = reinterpret_cast<const int2*>(st.miss);
  const uint8_t* host = v.host[layer * v.B + b];
  uint8_t* dst = v.cache + (int64_t)(layer * v.B + b) * (v.C + v.R) * v.row_bytes;
  const uint32_t stride = gridDim.x * (kFetchThreads * U);
  for (uint32_t g0 = first + threadIdx.x; g0 < total; g0 += stride) {
    u32x4 val[U];
    int2 e[U];
    uint32_t c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t g = g0 + u * kFetchThreads;
      if (g < total) {
        const uint32_t j = g / cpr;
        c[u] = g - j * cpr;
        e[u] = ml[j];
        val[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(host + (int64_t)e[u].y * v.row_bytes) + c[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t g = g0 + u * kFetchThreads;
      if (g < total)
        reinterpret_cast<u32x4*>(dst + (int64_t)e[u].x * v.row_bytes)[c[u]] = val[u];
    }
  }
}

// ---------------------------------------------------------------------------
// State reset: every slot empty, clock 0, LRU order 0..C-1.
// grid = (chunks, requests, layers)
// ---------------------------------------------------------------------------
__global__ void init_kernel(StreamView v, int layer0, int b0, int clear_status) {
  const int b = b0 + blockIdx.y;
  const int layer = layer0 + blockIdx.z;
  const StreamPtrs st = stream_ptrs(v, layer, b);
  const int stride = gridDim.x * blockDim.x;
  const int first = blockIdx.x * blockDim.x + threadIdx.x;
  for (int x = first; x < v.l_cap; x += stride) st.pos2slot[x] = -1;
  for (int x = first; x < v.C; x += stride) {
    st.slot2pos[x] = -1;
    st.last_use[x] = 0;
    st.order[x] = x;
  }
  if (first < kHdrWords) st.hdr[first] = 0;
  if (clear_status && first == 0 && blockIdx.y == 0 && blockIdx.z == 0) *status_word(v) = 0u;
}

// ---------------------------------------------------------------------------
// Resident window load: ring slot C + (p mod R) <- host row p, for p in
// [max(0, ctx-R), ctx).  grid = (chunks, B, layers)
// ---------------------------------------------------------------------------
__global__ void load_window_kernel(StreamView v, int layer0, const int32_t* __restrict__ ctx_len) {
  const int b = blockIdx.y;
  const int layer = layer0 + blockIdx.z;
  const int32_t ctx = ctx_len[b];
  if (ctx < 0 || ctx > v.l_cap) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(status_word(v), HISPARSE_STATUS_CTX_RANGE);
    return;
  }
  const int32_t lo = ctx - v.R > 0 ? ctx - v.R : 0;
  const uint32_t cpr = (uint32_t)(v.row_bytes >> 4);
  const uint32_t total = (uint32_t)(ctx - lo) * cpr;
  const uint8_t* host = v.host[layer * v.B + b];
  uint8_t* dst = v.cache + (int64_t)(layer * v.B + b) * (v.C + v.R) * v.row_bytes;
  for (uint32_t g = blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += gridDim.x * blockDim.x) {
    const uint32_t r = g / cpr, c = g - r * cpr;
    const int32_t pos = lo + (int32_t)r;
    const u32x4 val = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(host + (int64_t)pos * v.row_bytes) + c);
    reinterpret_cast<u32x4*>(dst + (int64_t)(v.C + pos % v.R) * v.row_bytes)[c] = val;
  }
}

// ---------------------------------------------------------------------------
// Append: host row pos <- rows[b] and, with a window, ring slot C + pos mod R.
// grid = (chunks, B)
// ---------------------------------------------------------------------------
__global__ void append_kernel(StreamView v, int layer, const uint8_t* __restrict__ rows,
                              const int32_t* __restrict__ pos_arr) {
  const int b = blockIdx.y;
  const int32_t pos = pos_arr[b];
  if (pos < 0) return;
  if (pos >= v.l_cap) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(status_word(v), HISPARSE_STATUS_CTX_RANGE);
    return;
  }
  const uint32_t cpr = (uint32_t)(v.row_bytes >> 4);
  uint8_t* host = v.host[layer * v.B + b];
  uint8_t* dst = v.cache + (int64_t)(layer * v.B + b) * (v.C + v.R) * v.row_bytes;
  const u32x4* src = reinterpret_cast<const u32x4*>(rows + (int64_t)b * v.row_bytes);
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < cpr; c += gridDim.x * blockDim.x) {
    const u32x4 val = src[c];
    reinterpret_cast<u32x4*>(host + (int64_t)pos * v.row_bytes)[c] = val;
    if (v.R > 0) reinterpret_cast<u32x4*>(dst + (int64_t)(v.C + pos % v.R) * v.row_bytes)[c] = val;
  }
}

// ---------------------------------------------------------------------------
// Prefetch join: copy the prefetched slot map, check the selections match.
// grid = B
// ---------------------------------------------------------------------------
__global__ void prefetch_join_kernel(StreamView v, const int32_t* __restrict__ sel,
                                     const int32_t* __restrict__ sel_copy,
                                     const int32_t* __restrict__ pf_out, int32_t* __restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * v.k;
  int mismatch = 0;
  for (int i = threadIdx.x; i < v.k; i += blockDim.x) {
    mismatch |= sel[base + i] != sel_copy[base + i];
    out[base + i] = pf_out[base + i];
  }
  if (__syncthreads_or(mismatch) && threadIdx.x == 0)
    atomicOr(status_word(v), HISPARSE_STATUS_PREFETCH_MISMATCH);
}

// ---------------------------------------------------------------------------
// Link probe: contiguous 16-byte zero-copy reads of host memory.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) probe_host_read_kernel(const u32x4* __restrict__ host,
                                                              u32x4* __restrict__ dev, size_t n) {
  constexpr int U = 4;
  const size_t stride = (size_t)gridDim.x * blockDim.x * U;
  for (size_t g0 = (size_t)blockIdx.x * blockDim.x * U + threadIdx.x; g0 < n; g0 += stride) {
    u32x4 val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t g = g0 + (size_t)u * blockDim.x;
      if (g < n) val[u] = __builtin_nontemporal_load(host + g);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t g = g0 + (size_t)u * blockDim.x;
      if (g < n) dev[g] = val[u];
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
ResolveShape resolve_shape(int k, int C, bool debug_validate) {
  const int n = k > C ? k : C;
  ResolveShape s{0, 0, 0};
  for (int items = 1; items <= kMaxItems; items *= 2) {
    int threads = (n + items - 1) / items;
    threads = ((threads + 63) / 64) * 64;
    if (threads <= kMaxThreads) {
      s.items = items;
      s.threads = threads;
      break;
    }
  }
  if (s.items == 0) return s;
  const int W = s.threads / 64;
  size_t words = (size_t)((C + 31) / 32) + C + k + 3 * (size_t)s.items * W + 8;
  if (debug_validate) words += (size_t)(2 << (31 - __builtin_clz((unsigned)k)));
  s.lds_bytes = 4 * words;
  return s;
}

hipError_t launch_resolve(const StreamView& v, hipStream_t s, int layer, const int32_t* sel,
                          const int32_t* ctx_len, int32_t* out, int32_t* sel_copy) {
  const ResolveShape sh = resolve_shape(v.k, v.C, (v.flags & HISPARSE_DEBUG_VALIDATE) != 0);
  const dim3 grid(v.B), block(sh.threads);
  switch (sh.items) {
    case 1:
      hipLaunchKernelGGL(resolve_kernel<1>, grid, block, sh.lds_bytes, s, v, layer, sel, ctx_len,
                         out, sel_copy);
      break;
    case 2:
      hipLaunchKernelGGL(resolve_kernel<2>, grid, block, sh.lds_bytes, s, v, layer, sel, ctx_len,
                         out, sel_copy);
      break;
    case 4:
      hipLaunchKernelGGL(resolve_kernel<4>, grid, block, sh.lds_bytes, s, v, layer, sel, ctx_len,
                         out, sel_copy);
      break;
    case 8:
      hipLaunchKernelGGL(resolve_kernel<8>, grid, block, sh.lds_bytes, s, v, layer, sel, ctx_len,
                         out, sel_copy);
      break;
    case 16:
      hipLaunchKernelGGL(resolve_kernel<16>, grid, block, sh.lds_bytes, s, v, layer, sel, ctx_len,
                         out, sel_copy);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fetch(const StreamView& v, hipStream_t s, int layer, int grid_x) {
  hipLaunchKernelGGL(fetch_kernel<4>, dim3(grid_x, v.B), dim3(kFetchThreads), 0, s, v, layer);
  return hipGetLastError();
}

hipError_t launch_init(const StreamView& v, hipStream_t s, int layer, int request,
                       bool clear_status) {
  const int nl = layer < 0 ? v.L : 1, l0 = layer < 0 ? 0 : layer;
  const int nb = request < 0 ? v.B : 1, b0 = request < 0 ? 0 : request;
  const int n = v.l_cap > v.C ? v.l_cap : v.C;
  int gx = (n + 255) / 256;
  if (gx > 64) gx = 64;
  hipLaunchKernelGGL(init_kernel, dim3(gx, nb, nl), dim3(256), 0, s, v, l0, b0,
                     clear_status ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_load_window(const StreamView& v, hipStream_t s, int layer,
                              const int32_t* ctx_len) {
  if (v.R <= 0) return hipSuccess;
  const int nl = layer < 0 ? v.L : 1, l0 = layer < 0 ? 0 : layer;
  const int64_t chunks = (int64_t)v.R * (v.row_bytes >> 4);
  int gx = (int)((chunks + 255) / 256);
  if (gx > 256) gx = 256;
  hipLaunchKernelGGL(load_window_kernel, dim3(gx, v.B, nl), dim3(256), 0, s, v, l0, ctx_len);
  return hipGetLastError();
}

hipError_t launch_append(const StreamView& v, hipStream_t s, int layer, const uint8_t* rows,
                         const int32_t* pos) {
  const int64_t cpr = v.row_bytes >> 4;
  int gx = (int)((cpr + 255) / 256);
  hipLaunchKernelGGL(append_kernel, dim3(gx, v.B), dim3(256), 0, s, v, layer, rows, pos);
  return hipGetLastError();
}

hipError_t launch_prefetch_join(const StreamView& v, hipStream_t s, const int32_t* sel,
                                const int32_t* sel_copy, const int32_t* pf_out, int32_t* out) {
  hipLaunchKernelGGL(prefetch_join_kernel, dim3(v.B), dim3(256), 0, s, v, sel, sel_copy, pf_out,
                     out);
  return hipGetLastError();
}

hipError_t launch_probe_host_read(hipStream_t s, const void* host, void* dev, size_t bytes,
                                  int workgroups) {
  hipLaunchKernelGGL(probe_host_read_kernel, dim3(workgroups), dim3(256), 0, s,
                     static_cast<const u32x4*>(host), static_cast<u32x4*>(dev), bytes / 16);
  return hipGetLastError();
}

}  // namespace hsp
