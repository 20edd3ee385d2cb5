// Sparse MLA decode attention over the slot map (gfx950).
//
// The consumer of the resolution step: for every request, attention of H
// query heads over the rows the slot map points at, read from the HBM slot
// cache.  Because resolution only changes where rows live, this equals
// attention over the same positions of the full host history ("HiSparse:
// Scaling Sparse-Attention Decoding with Hierarchical KV Cache Management",
// Abstract: outputs unchanged; "Hybrid HiSparse", Timeline: the method sits
// under sparse MLA decoding).
//
// Several query tokens per request (multi-token prediction): attention row
// r = b * Qn + q is query token q of request b; it has its own queries and
// slot-map entries (row r of the multi-query slot map) and reads request b's
// slot rows.
//
// Row format: a token row is 576 bf16, 512 compressed-latent values (shared
// by keys and values) followed by 64 rope values (key only).  A slot holds
// T = row_bytes / 1152 token rows (T = 16 for Quest-style pages); every token
// row of every selected slot is attended, padding (-1) is skipped.
//
//   score[h, i] = scale * q[h, :] . row_i[:576]
//   out[h, :]   = sum_i softmax_i(score[h, i]) * row_i[:512]
//   lse[h]      = log sum_i exp(score[h, i])
//
// CDNA4 mapping:
//   * grid = (requests x head blocks of 16) x splits of the token rows, up to
//     two workgroups per CU (78 KiB of LDS each, so one computes while the
//     other waits for its rows); a workgroup (4 waves) walks its split in
//     tiles of 64 rows, each row read once from HBM (16-byte loads, all in
//     flight, the next tile's requested while the current one is finished);
//   * rows are read with whole 128-byte lines per request (8 rows x 128
//     contiguous bytes per load instruction: half-line requests cost a
//     quarter of the gather bandwidth) into an LDS copy of the tile, from
//     which both MFMA operands of the rows are read;
//   * scores: wave w takes rows 16w .. 16w+15 of the tile, S^T (16 rows x 16
//     heads) = K . Q^T with v_mfma_f32_16x16x32_bf16, the 16 query heads'
//     fragments held in registers;
//   * online softmax in fp32 with one running max per head for the whole
//     workgroup (the waves exchange their tile maxima through LDS), so every
//     wave scales its rows the same way;
//   * values: P^T (hi and lo bf16 parts, so the products keep ~16 more bits
//     than a plain bf16 P) goes to LDS next to the rows, and
//     wave w accumulates O^T for output dims 128w .. 128w+127 over the 64 rows
//     with v_mfma_f32_16x16x32_bf16: the waves own disjoint dims, so nothing
//     is combined across waves but the softmax sums.  The V^T operand (one
//     output dim, eight consecutive rows per lane) comes from the row-major
//     tile through gfx950's transposing LDS read, ds_read_b64_tr_b16: within
//     each 16-lane group, element j of lane i's result is element i % 4 of
//     the 8 bytes addressed by lane 4 j + i / 4, so lane 4 j + q points at
//     row j, dims 4 q .. 4 q + 3 of the block and every lane receives four
//     rows of its own dim;
//   * each split writes its partial (max, sum, unnormalised output) to a
//     workspace, and a second kernel (8 workgroups per request and head
//     block, coalesced over the partials' register order) merges the splits.
#include <hip/hip_runtime.h>

#include <math.h>

#include "hisparse_device.h"
#include "hisparse_mla_internal.h"

namespace hsp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kKSteps = kMlaDqk / 32;  // 18 steps of 32 dims for the scores
constexpr int kTile = 16 * kMlaWaves;   // 64 rows per tile
constexpr int kKRowPitch = kMlaDqk + 8;  // bf16 per LDS row: 1168 B (16-byte aligned, and
                                         // 16 consecutive rows start on distinct bank quads)
constexpr int kPPitch = kTile + 8;        // shorts per head in the P^T tile: 144 B, so the 16
                                         // heads' 16-byte operand reads hit distinct banks
constexpr size_t kMlaKbufBytes = sizeof(uint16_t) * kTile * kKRowPitch;     // 73 KiB
constexpr size_t kMlaPBytes = 2 * sizeof(uint16_t) * kMlaHB * kPPitch;      // 4.5 KiB (hi, lo)
constexpr size_t kMlaRedBytes = sizeof(float) * 2 * kMlaWaves * kMlaHB;     // 0.5 KiB
constexpr int kDBlocks = kMlaDv / 16;                 // 32 blocks of 16 output dims
constexpr int kWaveDB = kDBlocks / kMlaWaves;         // 8 blocks (128 dims) per wave
constexpr int kWgPerCu = 2;                           // workgroups resident per CU
constexpr int kMlaMergeParts = 8;                     // merge workgroups per (request, head block)
constexpr int kXcds = 8;                              // MI355X: 8 XCDs, 32 CUs each

__device__ __forceinline__ short bf16_bits(__bf16 x) {
  return __builtin_bit_cast(short, x);
}

// Transposing LDS read of 4 x 16-bit values (ds_read_b64_tr_b16).
__device__ __forceinline__ short4_t lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4*)(__attribute__((address_space(3))) void*)(p));
}

__global__ void __launch_bounds__(kMlaThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
mla_decode_kernel(MlaArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* kt = reinterpret_cast<__bf16*>(smem);                       // [64 rows][pitch]
  short* phi_t = reinterpret_cast<short*>(smem + kMlaKbufBytes);       // [16 heads][kPPitch]
  short* plo_t = phi_t + kMlaHB * kPPitch;
  float* red = reinterpret_cast<float*>(smem + kMlaKbufBytes + kMlaPBytes);
  float* red_m = red;                      // [waves][16] tile maxima
  float* red_l = red + kMlaWaves * kMlaHB;  // [waves][16] softmax sums

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane & 15;  // head (B-operand and D column)
  const int g = lane >> 4;  // lane group: k sub-range of the operands, D rows 4g..4g+3

  // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs
  // (XCD = id mod 8), so the head blocks of one (request, split) -- which
  // read the same rows -- get ids 8 apart: one XCD, dispatched together,
  // sharing its L2.
  const int id = blockIdx.x;
  const int xc = id % kXcds;
  const int qd = id / kXcds;
  const int hb = qd % a.HBn;
  const int unit = (qd / a.HBn) * kXcds + xc;  // b * S + split
  if (unit >= a.B * a.S) return;
  const int split = unit % a.S;
  const int b = unit / a.S;

  const int n_tok = a.k * a.T;
  const int r_begin = split * a.rows_per_split;
  const int r_end = min(n_tok, r_begin + a.rows_per_split);
  const int32_t* slots = a.slots + (int64_t)b * a.k;
  const uint8_t* cbase = a.cache + (int64_t)(b / a.Qn) * a.stream_bytes;  // the row's request
  const bf16x8 zero8 = {};

  // The wave's 16 rows of a tile are read with whole 128-byte lines per
  // request: load j (0 .. 17) covers rows 8 (j & 1) + lane / 8, bytes
  // 128 (j >> 1) + 16 (lane % 8) .. +15 of each, i.e. 8 rows x 128 contiguous
  // bytes, and goes to the LDS copy of the tile; the MFMA operands are read
  // from there.  A lane needs three slot-map entries per tile: the rows of
  // its two lines (m = lane / 8, 8 + lane / 8) and its MFMA row
  // (m = lane % 16).  They are read one tile ahead, so that no dependent
  // index load sits between a tile's rows and their use, and the loads are
  // unconditional (clamped, in-bounds addresses; rows outside the split or
  // padding are replaced by zeros when stored), so that the compiler's
  // wait counts follow the software pipeline exactly.
  const int m0 = lane >> 3, m1 = 8 + (lane >> 3), mv = lane & 15;
  auto slot_raw = [&](int tile0, int m) {
    const int r = min(tile0 + 16 * wave + m, n_tok - 1);
    return slots[r / a.T];
  };
  auto slot_ok = [&](int raw, int tile0, int m) {  // -1: outside the split, or padding
    const int r = tile0 + 16 * wave + m;
    return (r < r_end && raw >= 0 && raw < a.slots_total) ? raw : -1;
  };
  bf16x8 kf[kKSteps];
  bool ok0 = false, ok1 = false;  // the lines in kf belong to rows that are attended
  auto load_rows = [&](int tile0, int sl0, int sl1) {
    const uint8_t* rp[2];
    const int sls[2] = {sl0, sl1};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int r = tile0 + 16 * wave + (half ? m1 : m0);
      rp[half] = cbase + (int64_t)(sls[half] >= 0 ? sls[half] : 0) * a.row_bytes +
                 (int64_t)(r % a.T) * (2 * kMlaDqk) + 16 * (lane & 7);
    }
    ok0 = sl0 >= 0;
    ok1 = sl1 >= 0;
#pragma unroll
    for (int j = 0; j < kKSteps; ++j)
      kf[j] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(rp[j & 1] + 128 * (j >> 1)));
  };
  auto store_rows = [&]() {  // the loaded lines into the wave's 16 rows of the tile
#pragma unroll
    for (int j = 0; j < kKSteps; ++j) {
      const int m = (j & 1) ? m1 : m0;
      *reinterpret_cast<bf16x8*>(kt + (16 * wave + m) * kKRowPitch + 64 * (j >> 1) + 8 * (lane & 7)) =
          ((j & 1) ? ok1 : ok0) ? kf[j] : zero8;
    }
  };

  // the first tile's rows are requested with the queries; each later tile's
  // rows while the previous tile is finished (software pipeline)
  int raw0 = slot_raw(r_begin, m0), raw1 = slot_raw(r_begin, m1), rawv = slot_raw(r_begin, mv);
  load_rows(r_begin, slot_ok(raw0, r_begin, m0), slot_ok(raw1, r_begin, m1));
  bool valid = slot_ok(rawv, r_begin, mv) >= 0;  // the MFMA row of this lane
  // B-operand fragments of Q^T: head h, dims 32 ks + 8 g .. +7
  bf16x8 qf[kKSteps];
  {
    const __bf16* qh = a.q + ((int64_t)b * a.H + hb * kMlaHB + h) * kMlaDqk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qh + 32 * ks);
  }
  raw0 = slot_raw(r_begin + kTile, m0);
  raw1 = slot_raw(r_begin + kTile, m1);
  rawv = slot_raw(r_begin + kTile, mv);
  // Everything above has landed before the loop (s_waitcnt vmcnt(0)): the
  // compiler then knows the query fragments are not pending, and does not
  // make the score MFMAs wait for the next tile's loads.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  float m_run = -INFINITY, l_run = 0.f;  // m_run: the workgroup's; l_run: this wave's rows
  float4_t acc[kWaveDB];
#pragma unroll
  for (int db = 0; db < kWaveDB; ++db) acc[db] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (int tile0 = r_begin; tile0 < r_end; tile0 += kTile) {
    const int t1 = tile0 + kTile;
    const int sl0_next = slot_ok(raw0, t1, m0);
    const int sl1_next = slot_ok(raw1, t1, m1);
    const bool valid_next = slot_ok(rawv, t1, mv) >= 0;
    const bool valid_now = valid;
    store_rows();
    // the registers are free: request the next tile's rows, and the slot-map
    // entries of the tile after it
    if (t1 < r_end) {
      load_rows(t1, sl0_next, sl1_next);
      raw0 = slot_raw(t1 + kTile, m0);
      raw1 = slot_raw(t1 + kTile, m1);
      rawv = slot_raw(t1 + kTile, mv);
    }
    valid = valid_next;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");  // the wave's rows in LDS
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    // S^T[i][h] for rows i = 4g + j of the wave's 16 (A fragments from LDS)
    float4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(
          kt + (16 * wave + (lane & 15)) * kKRowPitch + 32 * ks + 8 * g);
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[ks], st, 0, 0, 0);
    }
    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vj = __shfl(valid_now ? 1 : 0, 4 * g + j);
      sc[j] = vj ? st[j] * a.scale : -INFINITY;
    }
    float tm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    tm = fmaxf(tm, __shfl_xor(tm, 16));
    tm = fmaxf(tm, __shfl_xor(tm, 32));
    if (g == 0) red_m[wave * kMlaHB + h] = tm;
    lds_barrier();  // A: tile maxima (and the V tile) written
    float m_tile = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMlaWaves; ++w) m_tile = fmaxf(m_tile, red_m[w * kMlaHB + h]);
    const float m_new = fmaxf(m_run, m_tile);
    float p[4], alpha;
    if (m_new == -INFINITY) {
      alpha = 1.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = 0.f;
    } else {
      alpha = expf(m_run - m_new);
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = expf(sc[j] - m_new);
    }
    float ps = (p[0] + p[1]) + (p[2] + p[3]);
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    // P^T of the wave's rows 4g .. 4g+3 for head h: four consecutive entries
    short4_t phi, plo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const __bf16 hi = (__bf16)p[j];
      const __bf16 lo = (__bf16)(p[j] - (float)hi);
      phi[j] = bf16_bits(hi);
      plo[j] = bf16_bits(lo);
    }
    *reinterpret_cast<short4_t*>(phi_t + h * kPPitch + 16 * wave + 4 * g) = phi;
    *reinterpret_cast<short4_t*>(plo_t + h * kPPitch + 16 * wave + 4 * g) = plo;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < kWaveDB; ++db) acc[db] *= alpha;
    }
    lds_barrier();  // B: P tile written
    // O^T[128 wave + 16 db + 4g + j][h] += sum over the tile's 64 rows, 32 at a
    // time: this lane's k range is rows 32 rc + 8 g .. +7.  Its two transposing
    // reads point at row 32 rc + 8 g + (lane & 15) / 4 (+ 4), dims
    // 4 (lane & 3) .. +3 of the 16-dim block.
    const __bf16* vrow = kt + (8 * g + ((lane & 15) >> 2)) * kKRowPitch + 4 * (lane & 3) +
                         16 * kWaveDB * wave;
#pragma unroll
    for (int rc = 0; rc < kTile / 32; ++rc) {
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(phi_t + h * kPPitch + 32 * rc + 8 * g);
      const bf16x8 bl = *reinterpret_cast<const bf16x8*>(plo_t + h * kPPitch + 32 * rc + 8 * g);
#pragma unroll
      for (int db = 0; db < kWaveDB; ++db) {
        const __bf16* vp = vrow + 32 * rc * kKRowPitch + 16 * db;
        const short4_t v0 = lds_read_tr16(vp);
        const short4_t v1 = lds_read_tr16(vp + 4 * kKRowPitch);
        const bf16x8 va = __builtin_bit_cast(
            bf16x8, short8_t{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bh, acc[db], 0, 0, 0);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bl, acc[db], 0, 0, 0);
      }
    }
    lds_barrier();  // C: the tile buffers are free for the next tile
  }

  // ---- softmax sums of the waves; the partial result --------------------------
  if (g == 0) red_l[wave * kMlaHB + h] = l_run;
  lds_barrier();
  float l_wg = 0.f;
#pragma unroll
  for (int w = 0; w < kMlaWaves; ++w) l_wg += red_l[w * kMlaHB + h];
  const int pid = (b * a.HBn + hb) * a.S + split;
  float* part = a.part + (int64_t)pid * kMlaHB * kMlaDv;
#pragma unroll
  for (int db = 0; db < kWaveDB; ++db)
    reinterpret_cast<float4_t*>(part)[(kWaveDB * wave + db) * 64 + lane] = acc[db];
  if (wave == 0 && g == 0) {
    a.part_ml[(int64_t)pid * kMlaHB * 2 + h * 2 + 0] = m_run;
    a.part_ml[(int64_t)pid * kMlaHB * 2 + h * 2 + 1] = l_wg;
  }
}

// Merge the splits of one (request, head block): per head, weights
// w_s = exp(m_s - m) from the partial maxima; out = sum_s w_s O_s / sum_s w_s l_s,
// lse = m + log(sum).  The partials keep the split kernel's register order
// (float4 (db, lane) = dims 16 db + 4 (lane >> 4) + 0..3 of head lane & 15), so
// the reads here are fully coalesced.  grid = B * HBn * kMlaMergeParts,
// 256 threads, one float4 of the 16 x 512 block per thread.  With up to
// kMergeRegSplits splits the thread's partials are requested at the start,
// with the maxima and sums, so the weights are computed while they arrive
// (one memory round trip instead of three), and the weights of the 16 heads
// x S splits are computed by one thread each (shuffle reductions over a
// head's 16-lane group) instead of one serial loop per head.
constexpr int kMergeRegSplits = 16;

__global__ void __launch_bounds__(256) mla_combine_kernel(MlaArgs a) {
  extern __shared__ float wsh[];  // [16 heads][S] weights, [16] 1/L, [16 heads][S] sums
  const int id = blockIdx.x;
  const int part_no = id % kMlaMergeParts;
  const int bhb = id / kMlaMergeParts;  // b * HBn + hb
  const int b = bhb / a.HBn;
  const int hb = bhb - b * a.HBn;
  const int pid0 = bhb * a.S;
  const int tid = threadIdx.x;
  constexpr int kF4 = kMlaHB * kMlaDv / 4;  // 2048 float4 per split
  static_assert(kF4 / kMlaMergeParts == 256, "one float4 per thread");
  const int f = part_no * (kF4 / kMlaMergeParts) + tid;
  const float4_t* pbase = reinterpret_cast<const float4_t*>(a.part + (int64_t)pid0 * kMlaHB * kMlaDv) + f;
  const bool in_regs = a.S <= kMergeRegSplits;
  float4_t pv[kMergeRegSplits];
  if (in_regs) {
#pragma unroll
    for (int sp = 0; sp < kMergeRegSplits; ++sp)
      if (sp < a.S) pv[sp] = pbase[(int64_t)sp * kF4];
  }
  float* sums = wsh + kMlaHB * a.S + kMlaHB;
  if (in_regs) {
    // thread (head tid / 16, split tid % 16): maximum and weighted sum over
    // the head's splits with shuffles inside its 16-lane group
    const int h2 = tid >> 4, sp2 = tid & 15;
    float ms = -INFINITY, ls = 0.f;
    if (sp2 < a.S) {
      ms = a.part_ml[((int64_t)(pid0 + sp2) * kMlaHB + h2) * 2];
      ls = a.part_ml[((int64_t)(pid0 + sp2) * kMlaHB + h2) * 2 + 1];
    }
    float m = ms;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float w = (ms == -INFINITY) ? 0.f : expf(ms - m);
    float L = w * ls;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) L += __shfl_xor(L, o);
    if (sp2 < a.S) wsh[h2 * a.S + sp2] = w;
    if (sp2 == 0) {
      wsh[kMlaHB * a.S + h2] = L > 0.f ? 1.f / L : 0.f;
      if (part_no == 0) a.lse[(int64_t)b * a.H + hb * kMlaHB + h2] = L > 0.f ? m + logf(L) : -INFINITY;
    }
  } else {
    for (int x = tid; x < kMlaHB * a.S; x += 256) {
      const int hh = x / a.S, sp = x - hh * a.S;
      wsh[x] = a.part_ml[((int64_t)(pid0 + sp) * kMlaHB + hh) * 2];
      sums[x] = a.part_ml[((int64_t)(pid0 + sp) * kMlaHB + hh) * 2 + 1];
    }
  }
  __syncthreads();
  if (!in_regs && tid < kMlaHB) {
    float m = -INFINITY;
    for (int sp = 0; sp < a.S; ++sp) m = fmaxf(m, wsh[tid * a.S + sp]);
    float L = 0.f;
    for (int sp = 0; sp < a.S; ++sp) {
      const float ms = wsh[tid * a.S + sp];
      const float w = (ms == -INFINITY) ? 0.f : expf(ms - m);
      wsh[tid * a.S + sp] = w;
      L += w * sums[tid * a.S + sp];
    }
    wsh[kMlaHB * a.S + tid] = L > 0.f ? 1.f / L : 0.f;
    if (part_no == 0) a.lse[(int64_t)b * a.H + hb * kMlaHB + tid] = L > 0.f ? m + logf(L) : -INFINITY;
  }
  __syncthreads();
  const int lane = f & 63, db = f >> 6;
  const int hh = lane & 15, g = lane >> 4;
  float4_t o = {0.f, 0.f, 0.f, 0.f};
  if (in_regs) {
#pragma unroll
    for (int sp = 0; sp < kMergeRegSplits; ++sp)
      if (sp < a.S) o += wsh[hh * a.S + sp] * pv[sp];
  } else {
    for (int sp = 0; sp < a.S; ++sp) o += wsh[hh * a.S + sp] * pbase[(int64_t)sp * kF4];
  }
  o *= wsh[kMlaHB * a.S + hh];
  *reinterpret_cast<float4_t*>(a.out + ((int64_t)b * a.H + hb * kMlaHB + hh) * kMlaDv + 16 * db + 4 * g) = o;
}

}  // namespace

MlaShape mla_shape(int B, int H, int k, int T) {
  // Whole 64-row tiles (4 waves x 16 rows, all in flight at once) per
  // split.  Every split costs a 32 KiB partial written and read back by the
  // merge, so two workgroups per CU (256 CUs) are used only while a split
  // keeps at least kMinRows rows (partials <= ~22 % of the row bytes);
  // otherwise one per CU.
  constexpr int kMinRows = 256;
  MlaShape s{};
  s.HBn = H / kMlaHB;
  const int n_tok = k * T;
  const int tile = 16 * kMlaWaves;
  int S = (256 * kWgPerCu + B * s.HBn - 1) / (B * s.HBn);
  if (S > 1 && n_tok / S < kMinRows) S = (256 + B * s.HBn - 1) / (B * s.HBn);
  const int max_s = (n_tok + tile - 1) / tile;
  if (S > max_s) S = max_s;
  if (S > kMlaMaxSplits) S = kMlaMaxSplits;
  if (S < 1) S = 1;
  int rows = (n_tok + S - 1) / S;
  rows = ((rows + tile - 1) / tile) * tile;
  s.rows_per_split = rows;
  s.S = (n_tok + rows - 1) / rows;
  if (s.S < 1) s.S = 1;
  s.lds_bytes = kMlaKbufBytes + kMlaPBytes + kMlaRedBytes;
  s.part_floats = (size_t)B * s.HBn * s.S * kMlaHB * kMlaDv;
  s.ml_floats = (size_t)B * s.HBn * s.S * kMlaHB * 2;
  s.counters = 0;
  return s;
}

hipError_t launch_mla(const MlaArgs& a, hipStream_t s, size_t lds_bytes) {
  const int units = a.B * a.S;
  const int grid = (units + kXcds - 1) / kXcds * kXcds * a.HBn;
  hipLaunchKernelGGL(mla_decode_kernel, dim3(grid), dim3(kMlaThreads), lds_bytes, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(a.B * a.HBn * kMlaMergeParts), dim3(256),
                     sizeof(float) * (2 * kMlaHB * a.S + kMlaHB), s, a);
  return hipGetLastError();
}

}  // namespace hsp
