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
//   * grid = (requests x head blocks of 16) x splits of the token rows, about
//     one workgroup per CU; each workgroup (8 waves, 16 rows each, all row
//     loads in flight at once) streams its split's rows once from HBM;
//   * per wave, 16 rows at a time: S^T (16 rows x 16 heads) = K . Q^T with
//     v_mfma_f32_16x16x32_bf16, the row fragments loaded straight from the
//     slot rows (16-byte loads), the 16 query heads read from LDS;
//   * online softmax in fp32 per head; P^T (rows x heads) is already in the
//     B-operand layout of v_mfma_f32_16x16x16_bf16, so O^T += V^T . P^T needs
//     only V transposed: the wave's rows go through a private LDS buffer;
//     P is split into bf16 hi + lo parts (two MFMAs) so the products keep
//     ~16 more bits than a plain bf16 P;
//   * the 8 waves combine through a fixed-order tree in LDS (bit-reproducible,
//     reusing the V-tile space); wave 0 writes the split's partial; each split
//     writes its partial (max, sum, unnormalised output) to a workspace, and a
//     second kernel (8 workgroups per request and head block, coalesced over
//     the partials' register order) merges the splits.
#include <hip/hip_runtime.h>

#include <math.h>

#include "hisparse_internal.h"

namespace hsp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kKSteps = kMlaDqk / 32;  // 18 steps of 32 dims for the scores
constexpr int kVRowPitch = kMlaDv + 8;  // bf16 per LDS row (padding against bank conflicts)
constexpr size_t kMlaVbufBytes = sizeof(uint16_t) * kMlaWaves * 16 * kVRowPitch;  // 133 KiB
constexpr size_t kMlaQBytes = sizeof(uint16_t) * kMlaHB * kMlaDqk;               // 18 KiB
static_assert(kMlaVbufBytes >= sizeof(float) * (kMlaWaves / 2) * kMlaHB * kMlaDv,
              "the tree-combine buffers alias the V tiles");
constexpr int kDBlocks = kMlaDv / 16;  // 32 blocks of 16 output dims
constexpr int kMlaMergeParts = 8;      // merge workgroups per (request, head block)

__device__ __forceinline__ short bf16_bits(__bf16 x) {
  return __builtin_bit_cast(short, x);
}

__global__ void __launch_bounds__(kMlaThreads) mla_decode_kernel(MlaArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  // [kMlaWaves][16 rows][kVRowPitch] bf16 V tiles; after the row loop the same
  // space holds the tree-combine buffers ([4][16 heads][512] fp32)
  __bf16* vbuf = reinterpret_cast<__bf16*>(smem);
  float* tree = reinterpret_cast<float*>(smem);
  __bf16* qs = reinterpret_cast<__bf16*>(smem + kMlaVbufBytes);      // [16 heads][576]
  float* wml = reinterpret_cast<float*>(smem + kMlaVbufBytes + kMlaQBytes);  // [waves][16][2]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane & 15;  // head (B-operand column, D column)
  const int g = lane >> 4;  // lane group: k sub-range of the operands, D rows 4g..4g+3

  const int id = blockIdx.x;
  const int split = id % a.S;
  const int rest = id / a.S;
  const int hb = rest % a.HBn;
  const int b = rest / a.HBn;

  // this wave's 16 rows: slot lookups first (they gate the row loads)
  const int n_tok = a.k * a.T;
  const int r_begin = split * a.rows_per_split;
  const int r_end = min(n_tok, r_begin + a.rows_per_split);
  const int32_t* slots = a.slots + (int64_t)b * a.k;
  const uint8_t* cbase = a.cache + (int64_t)b * a.stream_bytes;

  // the block's 16 query heads into LDS (16-byte chunks)
  {
    const __bf16* qblk = a.q + ((int64_t)b * a.H + hb * kMlaHB) * kMlaDqk;
    for (int c = tid; c < kMlaHB * kMlaDqk / 8; c += kMlaThreads)
      reinterpret_cast<bf16x8*>(qs)[c] = reinterpret_cast<const bf16x8*>(qblk)[c];
  }

  float m_run = -INFINITY, l_run = 0.f;
  float4_t acc[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db) acc[db] = float4_t{0.f, 0.f, 0.f, 0.f};
  __bf16* vb = vbuf + wave * 16 * kVRowPitch;
  const bf16x8 zero8 = {};
  __syncthreads();  // queries in LDS

  for (int r0 = r_begin + 16 * wave; r0 < r_end; r0 += 16 * kMlaWaves) {
    // this lane's row (A-operand row m = lane & 15)
    const int r = r0 + (lane & 15);
    bool valid = false;
    const uint8_t* rowp = cbase;
    if (r < r_end) {
      const int j = r / a.T;
      const int t = r - j * a.T;
      const int sl = slots[j];
      if (sl >= 0 && sl < a.slots_total) {
        valid = true;
        rowp = cbase + (int64_t)sl * a.row_bytes + (int64_t)t * (2 * kMlaDqk);
      }
    }
    bf16x8 kf[kKSteps];
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      kf[ks] = valid ? __builtin_nontemporal_load(
                           reinterpret_cast<const bf16x8*>(rowp + 2 * (32 * ks + 8 * g)))
                     : zero8;
    // value dims [0, 512) of the 16 rows into the wave's LDS buffer
#pragma unroll
    for (int ks = 0; ks < kMlaDv / 32; ++ks)
      *reinterpret_cast<bf16x8*>(vb + (lane & 15) * kVRowPitch + 32 * ks + 8 * g) = kf[ks];

    // S^T[i][h] for rows i = 4g + j of the tile; Q^T fragments from LDS
    float4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const bf16x8 qf = *reinterpret_cast<const bf16x8*>(qs + h * kMlaDqk + 32 * ks + 8 * g);
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf, st, 0, 0, 0);
    }

    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vj = __shfl(valid ? 1 : 0, 4 * g + j);
      sc[j] = vj ? st[j] * a.scale : -INFINITY;
    }
    float tm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    tm = fmaxf(tm, __shfl_xor(tm, 16));
    tm = fmaxf(tm, __shfl_xor(tm, 32));
    const float m_new = fmaxf(m_run, tm);
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
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) acc[db] *= alpha;
    }

    // P^T as the B operand (k = rows 4g..4g+3, n = head), split hi + lo
    short4_t phi, plo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const __bf16 hi = (__bf16)p[j];
      const __bf16 lo = (__bf16)(p[j] - (float)hi);
      phi[j] = bf16_bits(hi);
      plo[j] = bf16_bits(lo);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");  // V tile written
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) {
      short4_t va;  // A operand: V^T[d = 16 db + (lane & 15)][rows 4g..4g+3]
#pragma unroll
      for (int t = 0; t < 4; ++t)
        va[t] = bf16_bits(vb[(4 * g + t) * kVRowPitch + 16 * db + (lane & 15)]);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, phi, acc[db], 0, 0, 0);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, plo, acc[db], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");  // V tile consumed
  }

  // ---- combine the waves: common max, then a fixed-order tree in LDS -------
  if (g == 0) {
    wml[(wave * kMlaHB + h) * 2 + 0] = m_run;
    wml[(wave * kMlaHB + h) * 2 + 1] = l_run;
  }
  __syncthreads();  // also: every wave is done with its V tile
  float m_wg = -INFINITY, l_wg = 0.f;
#pragma unroll
  for (int w = 0; w < kMlaWaves; ++w) m_wg = fmaxf(m_wg, wml[(w * kMlaHB + h) * 2]);
#pragma unroll
  for (int w = 0; w < kMlaWaves; ++w) {
    const float mw = wml[(w * kMlaHB + h) * 2];
    if (mw != -INFINITY) l_wg += expf(mw - m_wg) * wml[(w * kMlaHB + h) * 2 + 1];
  }
  const float fac = (m_run == -INFINITY) ? 0.f : expf(m_run - m_wg);
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db) acc[db] *= fac;
  for (int half = kMlaWaves / 2; half >= 1; half /= 2) {
    if (wave >= half && wave < 2 * half) {
      float4_t* dst = reinterpret_cast<float4_t*>(tree + (wave - half) * kMlaHB * kMlaDv);
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) dst[db * 64 + lane] = acc[db];
    }
    __syncthreads();
    if (wave < half) {
      const float4_t* src = reinterpret_cast<const float4_t*>(tree + wave * kMlaHB * kMlaDv);
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) acc[db] += src[db * 64 + lane];
    }
    __syncthreads();
  }

  // ---- wave 0 writes the split's partial result ------------------------------
  if (wave == 0) {
    const int pid = (b * a.HBn + hb) * a.S + split;
    float* part = a.part + (int64_t)pid * kMlaHB * kMlaDv;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) reinterpret_cast<float4_t*>(part)[db * 64 + lane] = acc[db];
    if (g == 0) {
      a.part_ml[(int64_t)pid * kMlaHB * 2 + h * 2 + 0] = m_wg;
      a.part_ml[(int64_t)pid * kMlaHB * 2 + h * 2 + 1] = l_wg;
    }
  }
}

// Merge the splits of one (request, head block): per head, weights
// w_s = exp(m_s - m) from the partial maxima; out = sum_s w_s O_s / sum_s w_s l_s,
// lse = m + log(sum).  The partials keep the split kernel's register order
// (float4 (db, lane) = dims 16 db + 4 (lane >> 4) + 0..3 of head lane & 15), so
// the reads here are fully coalesced.  grid = B * HBn * kMlaMergeParts,
// 256 threads, one float4 of the 16 x 512 block per thread.
__global__ void __launch_bounds__(256) mla_combine_kernel(MlaArgs a) {
  extern __shared__ float wsh[];  // [16 heads][S] weights, [16] 1/L, [16 heads][S] sums
  const int id = blockIdx.x;
  const int part_no = id % kMlaMergeParts;
  const int bhb = id / kMlaMergeParts;  // b * HBn + hb
  const int b = bhb / a.HBn;
  const int hb = bhb - b * a.HBn;
  const int pid0 = bhb * a.S;
  const int tid = threadIdx.x;
  float* sums = wsh + kMlaHB * a.S + kMlaHB;
  for (int x = tid; x < kMlaHB * a.S; x += 256) {
    const int hh = x / a.S, sp = x - hh * a.S;
    wsh[x] = a.part_ml[((int64_t)(pid0 + sp) * kMlaHB + hh) * 2];
    sums[x] = a.part_ml[((int64_t)(pid0 + sp) * kMlaHB + hh) * 2 + 1];
  }
  __syncthreads();
  if (tid < kMlaHB) {
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
  constexpr int kF4 = kMlaHB * kMlaDv / 4;  // 2048 float4 per split
  for (int f = part_no * (kF4 / kMlaMergeParts) + tid; f < (part_no + 1) * (kF4 / kMlaMergeParts);
       f += 256) {
    const int lane = f & 63, db = f >> 6;
    const int hh = lane & 15, g = lane >> 4;
    float4_t o = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < a.S; ++sp)
      o += wsh[hh * a.S + sp] *
           reinterpret_cast<const float4_t*>(a.part + (int64_t)(pid0 + sp) * kMlaHB * kMlaDv)[f];
    o *= wsh[kMlaHB * a.S + hh];
    *reinterpret_cast<float4_t*>(a.out + ((int64_t)b * a.H + hb * kMlaHB + hh) * kMlaDv + 16 * db +
                                 4 * g) = o;
  }
}

}  // namespace

MlaShape mla_shape(int B, int H, int k, int T) {
  // About one workgroup per CU (256 CUs), each covering whole 128-row tiles
  // (8 waves x 16 rows, all in flight at once).
  MlaShape s{};
  s.HBn = H / kMlaHB;
  const int n_tok = k * T;
  const int tile = 16 * kMlaWaves;
  int S = (256 + B * s.HBn - 1) / (B * s.HBn);
  const int max_s = (n_tok + tile - 1) / tile;
  if (S > max_s) S = max_s;
  if (S > kMlaMaxSplits) S = kMlaMaxSplits;
  if (S < 1) S = 1;
  int rows = (n_tok + S - 1) / S;
  rows = ((rows + tile - 1) / tile) * tile;
  s.rows_per_split = rows;
  s.S = (n_tok + rows - 1) / rows;
  if (s.S < 1) s.S = 1;
  s.lds_bytes = kMlaVbufBytes + kMlaQBytes + sizeof(float) * kMlaWaves * kMlaHB * 2;
  s.part_floats = (size_t)B * s.HBn * s.S * kMlaHB * kMlaDv;
  s.ml_floats = (size_t)B * s.HBn * s.S * kMlaHB * 2;
  s.counters = 0;
  return s;
}

hipError_t launch_mla(const MlaArgs& a, hipStream_t s, size_t lds_bytes, int grid) {
  hipLaunchKernelGGL(mla_decode_kernel, dim3(grid), dim3(kMlaThreads), lds_bytes, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(a.B * a.HBn * kMlaMergeParts), dim3(256),
                     sizeof(float) * (2 * kMlaHB * a.S + kMlaHB), s, a);
  return hipGetLastError();
}

}  // namespace hsp
