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
//   * each thread owns `IPS` selections and `IPO` LRU-order entries, strided
//     by the workgroup size (sized for the C order entries; the k <= C
//     selections take as few items per thread as cover them), so every
//     global load is coalesced except the position->slot gathers;
//   * three ordered compactions (misses by selection index, unreferenced
//     slots by LRU order, referenced slots by slot number) use 64-lane
//     ballots plus per-(round, wave) counts in LDS, one barrier each;
//   * LRU victim order without a sort: each stream keeps its slots in
//     (last_use, slot) order.  Slots referenced in a step all get the newest
//     stamp, so the next order is "unreferenced, not evicted, in old order"
//     followed by "referenced or refilled, by slot number"; the victims are
//     the first M unreferenced entries of the old order.  O(C) per step;
//   * the miss fetch: 16-byte non-temporal loads straight from mapped host
//     memory (through the global address space, so they count in vmcnt
//     only), written to the slot rows in HBM.  With >= 8 streams per call the
//     resolve workgroups copy their own misses (the first chunks are
//     requested before the victims are chosen); with fewer, a separate launch
//     fans the copies out over ~64 workgroups;
//   * the new row of a growing context can be appended in the same launch
//     (a separate instantiation), since with a resident window it is never
//     looked up or fetched by the resolution.
//   No MFMA anywhere: nothing here is a contraction.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "hisparse_device.h"
#include "hisparse_internal.h"

namespace hsp {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

enum Cls : int { kNone = 0, kPad = 1, kRes = 2, kHit = 3, kMiss = 4, kBad = 5, kRepeat = 6 };

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

// Quotient and remainder of p < 2^31 by d >= 1, given magic = floor(2^32/d)
// (2^32 - 1 for d = 1): the estimate umulhi(p, magic) is q or q - 1.
__device__ __forceinline__ uint32_t fast_div(uint32_t p, uint32_t d, uint32_t magic,
                                             uint32_t* rem) {
  uint32_t q = __umulhi(p, magic);
  uint32_t r = p - q * d;
  if (r >= d) {
    r -= d;
    ++q;
  }
  *rem = r;
  return q;
}

__device__ __forceinline__ uint32_t fast_mod(uint32_t p, uint32_t d, uint32_t magic) {
  uint32_t r;
  fast_div(p, d, magic, &r);
  return r;
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

// Ordered compaction, part 2: one wave-wide scan over the IPT*W counts
// (count(e) for e = r*W + w, in that order); off[r] = number of flagged items
// before (round r, this wave).  Returns the total.  Every wave computes its
// own offsets, so no barrier is needed after it.
template <int IPT, typename CountFn>
__device__ __forceinline__ int scan_offsets(CountFn count, int W, int wave, int lane,
                                            int (&off)[IPT]) {
  const int n = IPT * W;
  int carry = 0;
  for (int c = 0; c < n; c += 64) {
    const int e = c + lane;
    const int v = e < n ? count(e) : 0;
    const int incl = wave_inclusive_scan(v);
    const int excl = incl - v + carry;
#pragma unroll
    for (int r = 0; r < IPT; ++r) {
      const int idx = r * W + wave;  // wave-uniform
      if (idx >= c && idx < c + 64) off[r] = __builtin_amdgcn_readlane(excl, idx - c);
    }
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  return carry;
}

__device__ __forceinline__ bool test_bit(const uint32_t* bm, int s) {
  return (bm[s >> 5] >> (s & 31)) & 1u;
}

// ---------------------------------------------------------------------------
// Resolve: one workgroup per stream (request b of `layer`).
//
// The stream's work runs on one CU, so the kernel is bound by how many
// scattered (one cache line per lane) global accesses it issues.  Only the
// position->slot gathers and the two position->slot updates per miss are
// scattered; last_use and slot2pos are rewritten densely in slot order.
//
// Barriers (LDS only): Z after clearing LDS; 1 after classification (hit
// bitmap, class counters, miss counts, error bits); 2 after the misses are
// staged and the unreferenced slots counted; 3 after the victims are taken.
// No write to the stream's state happens before barrier 1, so a rejected
// row leaves the stream untouched.
//
// Fused append (`app_rows` not NULL; the host calls it only with a resident
// window, R >= 1): the request's new row goes to host history row
// pos = app_pos[b] and to ring slot C + pos mod R, as the separate append
// does.  Nothing in the resolution reads either: pos is the
// last position of the context, hence resident (never looked up, never
// fetched), and misses are fetched into LRU slots only; so the stores run
// alongside the resolution and the launch's end orders them before any later
// reader.
//
// Several query tokens per request (`ke` > 0): the row holds ke entries (the
// queries' selections one after another) and may repeat positions.  The step
// resolves their union once: an LDS hash keyed by position keeps each
// position's first entry index (atomicMin; one more barrier, D), the first
// entry is classified as usual and the later ones are set aside as repeats
// (counted with the padding).  Misses then come in first-entry order, as in
// the union written in first-occurrence order.  The first entries leave
// their slot in LDS, and after barrier 3 every repeat is served that slot.
// ---------------------------------------------------------------------------
template <int IPS, int IPO, bool kAppend>
__global__ void __launch_bounds__(kMaxThreads)
    resolve_kernel(StreamView v, int layer, const int32_t* __restrict__ sel_all,
                   const int32_t* __restrict__ ctx_len, int32_t* __restrict__ out_all,
                   int32_t* __restrict__ sel_copy, int ke_multi,
                   const uint8_t* __restrict__ app_rows, const int32_t* __restrict__ app_pos) {
  extern __shared__ int lds[];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int BD = blockDim.x;
  const int W = BD >> 6;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int C = v.C, R = v.R, k = v.k;
  const bool multi = ke_multi > 0;
  const int ke = multi ? ke_multi : k;  // entries per row (ke <= k)
  const bool debug = !multi && (v.flags & HISPARSE_DEBUG_VALIDATE) != 0;
  const StreamPtrs st = stream_ptrs(v, layer, b);
  const int32_t* sel = sel_all + (int64_t)b * ke;
  int32_t* out = out_all + (int64_t)b * ke;

  // LDS: [bitmap C bits][slot2pos C][miss pos k][miss idx k][cntA][cntB][misc 8][hash]
  // hash: debug: H position keys; several queries: H keys, then H first-entry
  // indices (the key words are reused for the first entries' slots once the
  // first entries are known).
  const int nbm = (C + 31) >> 5;
  uint32_t* bitmap = (uint32_t*)lds;
  int* s2p = lds + nbm;
  int* missp = s2p + C;
  int* missi = missp + k;
  int* cntA = missi + k;
  int* cntB = cntA + IPS * W;
  int* misc = cntB + IPO * W;  // 0 error bits, 1 pad, 2 res, 3 hit, 4 evictions
  const int H = multi ? (2 << (31 - __clz(2 * ke - 1)))   // power of two >= 2 ke
                      : debug ? (2 << (31 - __clz(k)))    // power of two > k
                              : 0;
  int* hash = misc + 8;
  int* first = hash + (multi ? H : 0);
  int* eslot = hash;

  // ---- Phase A: independent loads; clear LDS ------------------------------
  int32_t p[IPS], slot[IPS], o[IPO], q2[IPO];
  int cls[IPS];
#pragma unroll
  for (int r = 0; r < IPS; ++r) {
    const int i = r * BD + tid;
    p[r] = (i < ke) ? sel[i] : -1;
    cls[r] = (i < ke) ? kPad : kNone;
  }
#pragma unroll
  for (int r = 0; r < IPO; ++r) {
    const int x = r * BD + tid;
    o[r] = (x < C) ? st.order[x] : 0;
    q2[r] = (x < C) ? st.slot2pos[x] : -1;
  }
  const int32_t ctx = ctx_len[b];
  const int32_t t = st.hdr[kHdrT] + 1;  // one clock tick per resolve
  // the stream's host history (read here, so that the first host reads of the
  // fused copy do not wait for this pointer)
  const uint8_t* host = v.host[layer * v.B + b];
  const int64_t tot_miss = *reinterpret_cast<const int64_t*>(st.hdr + kHdrTotalMiss);
  const int64_t tot_evict = *reinterpret_cast<const int64_t*>(st.hdr + kHdrTotalEvict);
  const int64_t tot_hit = *reinterpret_cast<const int64_t*>(st.hdr + kHdrTotalHit);
  const bool ctx_ok = ctx >= 0 && ctx <= v.l_cap;
  for (int w = tid; w < nbm; w += BD) bitmap[w] = 0;
  for (int w = tid; w < H; w += BD) hash[w] = -1;
  if (multi)
    for (int w = tid; w < H; w += BD) first[w] = 0x7fffffff;
  if (tid < 8) misc[tid] = 0;

  // ---- fused append (see above): host row and ring slot of the new position
  // (a separate instantiation, so that the plain resolve carries none of it).
  // Issued after the resolution's own loads, so that its two round trips
  // (position, then row) overlap them instead of delaying them.
  if (kAppend && R > 0) {
    const int32_t pos = app_pos[b];
    if (pos >= v.l_cap) {
      if (tid == 0) atomicOr(status_word(v), HISPARSE_STATUS_CTX_RANGE);
    } else if (pos >= 0) {
      const int cpr = v.row_bytes >> 4;
      const u32x4* src = reinterpret_cast<const u32x4*>(app_rows + (int64_t)b * v.row_bytes);
      auto hrow = global_ptr(
          reinterpret_cast<u32x4*>(v.host[layer * v.B + b] + (int64_t)pos * v.row_bytes));
      auto ring = global_ptr(reinterpret_cast<u32x4*>(
          v.cache + ((int64_t)(layer * v.B + b) * (C + R) + C + pos % R) * v.row_bytes));
      for (int c = tid; c < cpr; c += BD) {
        const u32x4 val = src[c];
        hrow[c] = val;
        ring[c] = val;
      }
    }
  }
  lds_barrier();  // Z: LDS cleared (global loads stay in flight)

  // ---- classify; the position->slot gathers -------------------------------
  uint32_t bad = ctx_ok ? 0u : (uint32_t)HISPARSE_STATUS_CTX_RANGE;
#pragma unroll
  for (int r = 0; r < IPS; ++r) {
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
#pragma unroll
  for (int r = 0; r < IPO; ++r) {
    const int x = r * BD + tid;
    if (x < C) s2p[x] = q2[r];
  }
  int hs[IPS];  // several queries: the entry's hash cell, -1 if none
  if (multi) {
    // Open addressing with linear probing; H >= 2 ke > number of distinct
    // positions, so every probe sequence ends at its key or a free cell.
#pragma unroll
    for (int r = 0; r < IPS; ++r) {
      hs[r] = -1;
      if (cls[r] != kRes && cls[r] != kMiss) continue;
      uint32_t h = ((uint32_t)p[r] * 2654435761u) & (uint32_t)(H - 1);
      while (true) {
        const int prev = atomicCAS(&hash[h], -1, p[r]);
        if (prev == -1 || prev == p[r]) break;
        h = (h + 1) & (uint32_t)(H - 1);
      }
      atomicMin(&first[h], r * BD + tid);
      hs[r] = (int)h;
    }
    lds_barrier();  // D: the first entry of every position is known
#pragma unroll
    for (int r = 0; r < IPS; ++r)
      if (hs[r] >= 0 && first[hs[r]] != r * BD + tid) cls[r] = kRepeat;
  } else if (debug) {  // repeated positions: LDS open-addressing set of size H
#pragma unroll
    for (int r = 0; r < IPS; ++r) {
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
  // compaction flags, in-wave ranks and offsets: selections (s), LRU order (o)
  bool fs[IPS], fo[IPO];
  int ps[IPS], os_[IPS], po[IPO], oo[IPO];
  int npad = 0, nres = 0, nhit = 0;
#pragma unroll
  for (int r = 0; r < IPS; ++r) {
    if (cls[r] == kMiss && slot[r] >= 0) {
      cls[r] = kHit;
      atomicOr(&bitmap[slot[r] >> 5], 1u << (slot[r] & 31));
    }
    npad += __popcll(__ballot(cls[r] == kPad || cls[r] == kRepeat));
    nres += __popcll(__ballot(cls[r] == kRes));
    nhit += __popcll(__ballot(cls[r] == kHit));
    fs[r] = cls[r] == kMiss;
  }
  ballot_counts<IPS>(fs, cntA, W, wave, lane, ps);
  if (bad) atomicOr((uint32_t*)&misc[0], bad);
  if (lane == 0) {
    if (npad) atomicAdd(&misc[1], npad);
    if (nres) atomicAdd(&misc[2], nres);
    if (nhit) atomicAdd(&misc[3], nhit);
  }
  lds_barrier();  // 1: hit bitmap, class counters, miss counts, error bits

  uint32_t err = (uint32_t)misc[0];
  if (err) {
    // Rejected row: leave the stream untouched, serve -1 everywhere.
    if (err & (HISPARSE_STATUS_SEL_RANGE | HISPARSE_STATUS_CTX_RANGE))
      err &= ~(uint32_t)HISPARSE_STATUS_SEL_DUP;
#pragma unroll
    for (int r = 0; r < IPS; ++r) {
      const int i = r * BD + tid;
      if (i < ke) {
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
  const int n_hit = misc[3];

  // ---- serve padding, resident rows and hits; stage the misses -------------
  const int M = scan_offsets<IPS>([&](int e) { return cntA[e]; }, W, wave, lane, os_);
#pragma unroll
  for (int r = 0; r < IPS; ++r) {
    const int i = r * BD + tid;
    if (cls[r] == kMiss) {  // j-th miss in ascending selection index
      const int j = os_[r] + ps[r];
      missp[j] = p[r];
      missi[j] = i;
    } else if (cls[r] == kPad) {
      out[i] = -1;
    } else if (cls[r] == kRes) {
      const int s = C + (int)fast_mod((uint32_t)p[r], (uint32_t)R, v.r_magic);
      out[i] = s;
      if (multi) eslot[i] = s;
    } else if (cls[r] == kHit) {
      out[i] = slot[r];
      if (multi) eslot[i] = slot[r];
    }
    if (sel_copy && cls[r] != kNone) sel_copy[(int64_t)b * k + i] = p[r];
  }
#pragma unroll
  for (int r = 0; r < IPO; ++r) {
    const int x = r * BD + tid;
    fo[r] = (x < C) && !test_bit(bitmap, o[r]);  // unreferenced, in LRU order
  }
  ballot_counts<IPO>(fo, cntB, W, wave, lane, po);
  lds_barrier();  // 2: misses staged, unreferenced-slot counts

  // ---- fused fetch, first chunks: the missing positions are known, their --
  // slots are not yet.  Start the first kPre 16-byte host reads per thread
  // now, so the host link is busy while the victims are chosen and the LRU
  // order is rebuilt; they are stored once the slots are known.
  constexpr int kPre = IPO <= 8 ? 4 : 0;
  const bool fuse = v.fuse_fetch && !(v.flags & HISPARSE_NO_IO);
  const uint32_t cpr = (uint32_t)(v.row_bytes >> 4);
  const uint32_t total = fuse ? (uint32_t)M * cpr : 0u;
  u32x4 pre_val[kPre > 0 ? kPre : 1];
  uint32_t pre_c[kPre > 0 ? kPre : 1];
  int pre_j[kPre > 0 ? kPre : 1];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const uint32_t g = tid + u * BD;
    pre_j[u] = -1;
    if (g < total) {
      pre_j[u] = (int)fast_div(g, cpr, v.cpr_magic, &pre_c[u]);
      pre_val[u] = __builtin_nontemporal_load(global_ptr(
          reinterpret_cast<const u32x4*>(host + (int64_t)missp[pre_j[u]] * v.row_bytes) + pre_c[u]));
    }
  }

  // ---- victims = first M unreferenced slots in LRU order; the j-th miss ----
  // takes the j-th victim.  The victim's owner thread applies the whole miss.
  scan_offsets<IPO>([&](int e) { return cntB[e]; }, W, wave, lane, oo);
  int nev = 0;
#pragma unroll
  for (int r = 0; r < IPO; ++r) {
    if (!fo[r]) continue;
    const int u = oo[r] + po[r];
    const int s = o[r];
    if (u < M) {
      const int pos = missp[u];
      const int q = s2p[s];
      reinterpret_cast<int2*>(st.evict)[u] = make_int2(s, q);
      reinterpret_cast<int2*>(st.miss)[u] = make_int2(s, pos);
      if (q >= 0) {
        st.pos2slot[q] = -1;
        ++nev;
      }
      st.pos2slot[pos] = s;
      s2p[s] = pos;
      out[missi[u]] = s;
      if (multi) eslot[missi[u]] = s;
      missi[u] = s;  // from here on: the slot the j-th miss is fetched into
      atomicOr(&bitmap[s >> 5], 1u << (s & 31));
    } else {
      st.order[u - M] = s;  // kept: old relative order, at the front
    }
  }
  nev = wave_inclusive_scan(nev);  // lane 63 holds the wave's total
  if (lane == 63 && nev) atomicAdd(&misc[4], nev);
  lds_barrier();  // 3: bitmap = referenced or refilled slots; s2p updated

  // ---- referenced-or-refilled slots go to the back of the LRU order, by ----
  // slot number; their last_use and slot2pos are written densely.  Chunk
  // e = r*W + w covers slots [64e, 64e + 64) = bitmap words 2e and 2e + 1.
  const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < IPO; ++r) {
    const int x = r * BD + tid;
    fo[r] = (x < C) && test_bit(bitmap, x);
    po[r] = __popcll(__ballot(fo[r]) & lt);
  }
  scan_offsets<IPO>(
      [&](int e) {
        const int w0 = 2 * e;
        return (w0 < nbm ? __popc(bitmap[w0]) : 0) + (w0 + 1 < nbm ? __popc(bitmap[w0 + 1]) : 0);
      },
      W, wave, lane, oo);
  const int base = C - (n_hit + M);
#pragma unroll
  for (int r = 0; r < IPO; ++r) {
    if (!fo[r]) continue;
    const int x = r * BD + tid;
    st.order[base + oo[r] + po[r]] = x;
    st.last_use[x] = t;
    st.slot2pos[x] = s2p[x];
  }
  if (multi) {  // repeats: the slot of the position's first entry
#pragma unroll
    for (int r = 0; r < IPS; ++r)
      if (cls[r] == kRepeat) out[r * BD + tid] = eslot[first[hs[r]]];
  }

  if (tid == 0) {
    const int n_evict = misc[4];
    st.hdr[kHdrT] = t;
    st.hdr[kHdrStatus] = 0;
    st.hdr[kHdrPad] = misc[1];
    st.hdr[kHdrRes] = misc[2];
    st.hdr[kHdrHit] = n_hit;
    st.hdr[kHdrMiss] = M;
    st.hdr[kHdrEvict] = n_evict;
    st.hdr[kHdrBytes] = (v.flags & HISPARSE_NO_IO) ? 0 : (int32_t)(M * v.row_bytes);
    *reinterpret_cast<int64_t*>(st.hdr + kHdrTotalMiss) = tot_miss + M;
    *reinterpret_cast<int64_t*>(st.hdr + kHdrTotalEvict) = tot_evict + n_evict;
    *reinterpret_cast<int64_t*>(st.hdr + kHdrTotalHit) = tot_hit + n_hit;
  }

  // ---- fused miss fetch: the workgroup copies its own missing rows ---------
  // (enough in flight to saturate the host link once a layer call has >= 8
  // streams; with fewer, the separate fan-out fetch kernel is used instead)
  if (fuse) {
    constexpr int U = 4;
    uint8_t* dst = v.cache + (int64_t)(layer * v.B + b) * (C + R) * v.row_bytes;
#pragma unroll
    for (int u = 0; u < kPre; ++u)
      if (pre_j[u] >= 0)
        reinterpret_cast<u32x4*>(dst + (int64_t)missi[pre_j[u]] * v.row_bytes)[pre_c[u]] =
            pre_val[u];
    for (uint32_t g0 = tid + kPre * BD; g0 < total; g0 += BD * U) {
      u32x4 val[U];
      int sl[U];
      uint32_t c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t g = g0 + u * BD;
        if (g < total) {
          const uint32_t j = fast_div(g, cpr, v.cpr_magic, &c[u]);
          sl[u] = missi[j];
          val[u] = __builtin_nontemporal_load(
              global_ptr(reinterpret_cast<const u32x4*>(host + (int64_t)missp[j] * v.row_bytes) + c[u]));
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t g = g0 + u * BD;
        if (g < total) reinterpret_cast<u32x4*>(dst + (int64_t)sl[u] * v.row_bytes)[c[u]] = val[u];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Miss fetch: copy every listed row of every stream of `layer` from the host
// history into its slot.  The 16-byte chunks of all streams' misses form one
// flat index space, split evenly over the grid, so no stream's tail is left
// to a few CUs (one CU pulls only ~1/5 of the link).  grid = (G); LDS holds
// the per-stream chunk prefix.
// ---------------------------------------------------------------------------
template <int U>
__global__ void __launch_bounds__(kFetchThreads) fetch_kernel(StreamView v, int layer) {
  extern __shared__ int lds[];
  uint32_t* pre = reinterpret_cast<uint32_t*>(lds);  // [B + 1] chunk prefix
  const int B = v.B;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint32_t cpr = (uint32_t)(v.row_bytes >> 4);
  if (tid < 64) {  // one wave scans the per-stream miss counts
    uint32_t carry = 0;
    for (int c = 0; c < B; c += 64) {
      const int bb = c + lane;
      const int m = bb < B ? stream_ptrs(v, layer, bb).hdr[kHdrMiss] : 0;
      const int incl = wave_inclusive_scan(m);
      if (bb < B) pre[bb + 1] = carry + (uint32_t)incl * cpr;
      carry += (uint32_t)__builtin_amdgcn_readlane(incl, 63) * cpr;
    }
    if (tid == 0) pre[0] = 0;
  }
  lds_barrier();
  const uint32_t total = pre[B];
  const uint32_t per = (total + gridDim.x - 1) / gridDim.x;
  const uint32_t start = blockIdx.x * per;
  const uint32_t end = start + per < total ? start + per : total;
  for (uint32_t g0 = start + tid; g0 < end; g0 += kFetchThreads * U) {
    u32x4 val[U];
    uint8_t* dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t g = g0 + u * kFetchThreads;
      dst[u] = nullptr;
      if (g < end) {
        int lo = 0, hi = B;  // largest b with pre[b] <= g
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (pre[mid] <= g) lo = mid; else hi = mid;
        }
        const StreamPtrs st = stream_ptrs(v, layer, lo);
        uint32_t c;
        const uint32_t j = fast_div(g - pre[lo], cpr, v.cpr_magic, &c);
        const int2 e = reinterpret_cast<const int2*>(st.miss)[j];
        const uint8_t* host = v.host[layer * B + lo];
        dst[u] = v.cache + ((int64_t)(layer * B + lo) * (v.C + v.R) + e.x) * v.row_bytes + 16 * c;
        val[u] = __builtin_nontemporal_load(
            global_ptr(reinterpret_cast<const u32x4*>(host + (int64_t)e.y * v.row_bytes) + c));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (dst[u]) *global_ptr(reinterpret_cast<u32x4*>(dst[u])) = val[u];
  }
}

// ---------------------------------------------------------------------------
// Miss fetch for calls of few streams: a slice of the grid per stream
// (blockIdx.y).  A thread's chunks, and so the miss-list entries it copies,
// follow from its index alone, so the first list entries are requested
// together with the stream's miss count rather than after it (entries past
// the count are stale but in bounds: the list holds k); then the host reads,
// then the stores -- one dependent round trip fewer than the flat kernel
// above, which needs every stream's count before it can place a chunk.
//
// The host reads and the slot stores are buffer instructions over the
// stream's host history and slot rows: a chunk past the count gets an offset
// beyond the buffer's range, which the hardware drops without a memory
// request (a load returns zeros).  The code has no branch around any memory
// instruction; branches around each load made the compiler wait for every
// earlier memory operation, stores included, before the next load, and
// plain loads at a dummy address would cost link traffic.  The host calls it
// only when the history and the slot rows of a stream span < 4 GiB (32-bit
// buffer offsets).
// grid = (G, B)
// ---------------------------------------------------------------------------
constexpr uint32_t kBufferFormat = 0x00020000u;  // resource word 3 of a raw gfx9 buffer
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;    // past every resource's range (the host
                                                 // checks each spans at most this), and
                                                 // its four dwords do not wrap
constexpr int kBufferNT = 2;                     // cache policy: non-temporal

// `off` when `ok`, else kOutOfRange, by masks (no branch, no select chain)
__device__ __forceinline__ uint32_t in_range(uint32_t off, bool ok) {
  const uint32_t m = 0u - (uint32_t)ok;   // all ones when ok
  return (off & m) | (kOutOfRange & ~m);
}

template <int U>
__global__ void __launch_bounds__(kFetchThreads) fetch_stream_kernel(StreamView v, int layer) {
  const int b = blockIdx.y;
  const StreamPtrs st = stream_ptrs(v, layer, b);
  const uint32_t rb = (uint32_t)v.row_bytes;
  const uint32_t cpr = rb >> 4;
  const uint32_t last = (uint32_t)v.k * cpr - 1;   // last chunk the miss list can name
  const uint32_t stride = gridDim.x * kFetchThreads;
  const int2* list = reinterpret_cast<const int2*>(st.miss);
  const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(v.host[layer * v.B + b]), 0, (int)((uint32_t)v.l_cap * rb),
      (int)kBufferFormat);
  const __amdgpu_buffer_rsrc_t dst = __builtin_amdgcn_make_buffer_rsrc(
      v.cache + (int64_t)(layer * v.B + b) * (v.C + v.R) * v.row_bytes, 0,
      (int)((uint32_t)(v.C + v.R) * rb), (int)kBufferFormat);
  // The first batch is straight-line code, so the count is waited for only
  // after its list reads are issued (in a loop the wait was hoisted above
  // them); the rest (a cold step's misses) follows batch by batch.  A chunk
  // past the count gets offset kOutOfRange by arithmetic, not by a branch.
  const uint32_t g0 = blockIdx.x * kFetchThreads + threadIdx.x;
  int2 e[U];
  uint32_t c[U];
  u32x4 val[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t g = min(g0 + u * stride, last);
    e[u] = list[fast_div(g, cpr, v.cpr_magic, &c[u])];
  }
  const uint32_t total = (uint32_t)st.hdr[kHdrMiss] * cpr;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    val[u] = __builtin_amdgcn_raw_buffer_load_b128(
        src, in_range((uint32_t)e[u].y * rb + 16 * c[u], g0 + u * stride < total), 0, kBufferNT);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    __builtin_amdgcn_raw_buffer_store_b128(
        val[u], dst, in_range((uint32_t)e[u].x * rb + 16 * c[u], g0 + u * stride < total), 0, 0);
  }
  for (uint32_t gb = g0 + stride * U; gb < total; gb += stride * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t g = min(gb + u * stride, last);
      e[u] = list[fast_div(g, cpr, v.cpr_magic, &c[u])];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      val[u] = __builtin_amdgcn_raw_buffer_load_b128(
          src, in_range((uint32_t)e[u].y * rb + 16 * c[u], gb + u * stride < total), 0,
          kBufferNT);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      __builtin_amdgcn_raw_buffer_store_b128(
          val[u], dst, in_range((uint32_t)e[u].x * rb + 16 * c[u], gb + u * stride < total), 0, 0);
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
    uint32_t c;
    const uint32_t r = fast_div(g, cpr, v.cpr_magic, &c);
    const int32_t pos = lo + (int32_t)r;
    const u32x4 val = __builtin_nontemporal_load(
        global_ptr(reinterpret_cast<const u32x4*>(host + (int64_t)pos * v.row_bytes) + c));
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
    global_ptr(reinterpret_cast<u32x4*>(host + (int64_t)pos * v.row_bytes))[c] = val;
    if (v.R > 0) reinterpret_cast<u32x4*>(dst + (int64_t)(v.C + pos % v.R) * v.row_bytes)[c] = val;
  }
}

// ---------------------------------------------------------------------------
// Prefetch join: copy the prefetched slot map (unless it was written to the
// joining call's own buffer), check the selections match.
// One load round trip: every thread handles kJoinItems consecutive entries of
// one request row (4 consecutive int32 per load when the row allows it).
// grid = (ceil(k / (256 * kJoinItems)), B)
// ---------------------------------------------------------------------------
constexpr int kJoinItems = 4;

__global__ void __launch_bounds__(256)
    prefetch_join_kernel(StreamView v, const int32_t* __restrict__ sel,
                         const int32_t* __restrict__ sel_copy,
                         const int32_t* pf_out, int32_t* out, int vec) {
  const int64_t base = (int64_t)blockIdx.y * v.k;
  const int i0 = (blockIdx.x * 256 + threadIdx.x) * kJoinItems;
  int mismatch = 0;
  if (vec && i0 < v.k) {   // k % 4 == 0, so i0 + 3 < k; every row start 16-byte aligned
    const int4 a = *reinterpret_cast<const int4*>(sel + base + i0);
    const int4 c = *reinterpret_cast<const int4*>(sel_copy + base + i0);
    const int4 o = *reinterpret_cast<const int4*>(pf_out + base + i0);
    mismatch = (a.x != c.x) | (a.y != c.y) | (a.z != c.z) | (a.w != c.w);
    if (pf_out != out) *reinterpret_cast<int4*>(out + base + i0) = o;
  } else {
#pragma unroll
    for (int u = 0; u < kJoinItems; ++u) {
      const int i = i0 + u;
      if (i < v.k) {
        mismatch |= sel[base + i] != sel_copy[base + i];
        if (pf_out != out) out[base + i] = pf_out[base + i];
      }
    }
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
namespace {
// A launch whose duration is timed by events attached to the kernel's own
// dispatch (start and end of the kernel, as a profiler sees it) when ev0 or
// ev1 is given; a plain launch otherwise (e.g. under graph capture).
template <typename K, typename... Args>
hipError_t launch_timed(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, hipEvent_t ev0,
                        hipEvent_t ev1, Args... args) {
  if (ev0 || ev1)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, ev0, ev1, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  return hipGetLastError();
}
}  // namespace

ResolveShape resolve_shape(int k, int C, bool debug_validate, int multi_entries) {
  // Fewest order items per thread that fit 1024 threads; then the fewest
  // 64-lane waves that cover max(k, C) with that many items each; then the
  // fewest selection items (1, 2, 4 or the order items) that cover k with
  // those threads.
  const int n = k > C ? k : C;
  ResolveShape s{0, 0, 0, 0};
  static const int kItems[] = {1, 2, 3, 4, 6, 8, 12, 16};
  for (int items : kItems) {
    int threads = (n + items - 1) / items;
    threads = ((threads + 63) / 64) * 64;
    if (threads <= kMaxThreads) {
      s.items = items;
      s.threads = threads;
      break;
    }
  }
  if (s.items == 0) return s;
  // instantiated selection counts: 1, 2, 4 and the order count itself
  const int need = (k + s.threads - 1) / s.threads;
  s.sel_items = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 && s.items >= 4 ? 4 : s.items;
  if (s.sel_items > s.items) s.sel_items = s.items;
  const int W = s.threads / 64;
  size_t words = (size_t)((C + 31) / 32) + C + 2 * (size_t)k + (size_t)(s.items + s.sel_items) * W + 8;
  if (multi_entries > 0)
    words += 2 * (size_t)(2 << (31 - __builtin_clz((unsigned)(2 * multi_entries - 1))));
  else if (debug_validate)
    words += (size_t)(2 << (31 - __builtin_clz((unsigned)k)));
  s.lds_bytes = 4 * words;
  return s;
}

hipError_t launch_resolve(const StreamView& v, hipStream_t s, int layer, const int32_t* sel,
                          const int32_t* ctx_len, int32_t* out, int32_t* sel_copy,
                          int multi_entries, const uint8_t* app_rows, const int32_t* app_pos,
                          hipEvent_t ev0, hipEvent_t ev1) {
  const ResolveShape sh =
      resolve_shape(v.k, v.C, (v.flags & HISPARSE_DEBUG_VALIDATE) != 0, multi_entries);
  const dim3 grid(v.B), block(sh.threads);
  switch (sh.sel_items * 32 + sh.items) {
#define HSP_RESOLVE_CASE(S, O)                                                                 \
  case S * 32 + O:                                                                             \
    return app_rows ? launch_timed(resolve_kernel<S, O, true>, grid, block, sh.lds_bytes, s,    \
                                   ev0, ev1, v, layer, sel, ctx_len, out, sel_copy,             \
                                   multi_entries, app_rows, app_pos)                            \
                    : launch_timed(resolve_kernel<S, O, false>, grid, block, sh.lds_bytes, s,   \
                                   ev0, ev1, v, layer, sel, ctx_len, out, sel_copy,             \
                                   multi_entries, app_rows, app_pos);
    HSP_RESOLVE_CASE(1, 1)
    HSP_RESOLVE_CASE(1, 2)
    HSP_RESOLVE_CASE(2, 2)
    HSP_RESOLVE_CASE(1, 3)
    HSP_RESOLVE_CASE(2, 3)
    HSP_RESOLVE_CASE(3, 3)
    HSP_RESOLVE_CASE(1, 4)
    HSP_RESOLVE_CASE(2, 4)
    HSP_RESOLVE_CASE(4, 4)
    HSP_RESOLVE_CASE(1, 6)
    HSP_RESOLVE_CASE(2, 6)
    HSP_RESOLVE_CASE(4, 6)
    HSP_RESOLVE_CASE(1, 8)
    HSP_RESOLVE_CASE(2, 8)
    HSP_RESOLVE_CASE(4, 8)
    HSP_RESOLVE_CASE(1, 12)
    HSP_RESOLVE_CASE(2, 12)
    HSP_RESOLVE_CASE(4, 12)
    HSP_RESOLVE_CASE(1, 16)
    HSP_RESOLVE_CASE(2, 16)
    HSP_RESOLVE_CASE(4, 16)
    HSP_RESOLVE_CASE(6, 6)
    HSP_RESOLVE_CASE(8, 8)
    HSP_RESOLVE_CASE(12, 12)
    HSP_RESOLVE_CASE(16, 16)
#undef HSP_RESOLVE_CASE
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_fetch(const StreamView& v, hipStream_t s, int layer, int grid, hipEvent_t ev0,
                        hipEvent_t ev1) {
  const uint64_t host_span = (uint64_t)v.l_cap * (uint64_t)v.row_bytes;
  const uint64_t slot_span = (uint64_t)(v.C + v.R) * (uint64_t)v.row_bytes;
  if (v.B < kFetchStreamSlices && host_span <= kOutOfRange && slot_span <= kOutOfRange) {
    // few streams: a grid slice per stream (32-bit buffer offsets)
    const int gx = grid / v.B > 1 ? grid / v.B : 1;
    return launch_timed(fetch_stream_kernel<4>, dim3(gx, v.B), dim3(kFetchThreads), 0, s, ev0, ev1,
                        v, layer);
  }
  return launch_timed(fetch_kernel<4>, dim3(grid), dim3(kFetchThreads), sizeof(int) * (v.B + 1), s,
                      ev0, ev1, v, layer);
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
  // 16-byte vector accesses need every row start 16-byte aligned: k % 4 == 0
  // and 16-byte aligned base pointers (the library's own buffers are)
  const bool vec = (v.k & 3) == 0 &&
                   ((reinterpret_cast<uintptr_t>(sel) | reinterpret_cast<uintptr_t>(sel_copy) |
                     reinterpret_cast<uintptr_t>(pf_out) | reinterpret_cast<uintptr_t>(out)) &
                    15) == 0;
  const int per = 256 * kJoinItems;
  const dim3 grid((v.k + per - 1) / per, v.B);
  hipLaunchKernelGGL(prefetch_join_kernel, grid, dim3(256), 0, s, v, sel, sel_copy, pf_out, out,
                     vec ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_probe_host_read(hipStream_t s, const void* host, void* dev, size_t bytes,
                                  int workgroups) {
  hipLaunchKernelGGL(probe_host_read_kernel, dim3(workgroups), dim3(256), 0, s,
                     static_cast<const u32x4*>(host), static_cast<u32x4*>(dev), bytes / 16);
  return hipGetLastError();
}

}  // namespace hsp
