// Index selection (CRISP summary page, Methodology).
//
// VS heads, sink-aware noise floor (Eq. 3 and Eq. 4, Alg. 3): per direction
// keep the first and last block and every middle block with
// p_b > alpha * mu, mu = max(T - p_first - p_last, 0) / (N_b - 2), tested as
// alpha_den (N_b - 2) p_b > alpha_num M in exact integers, compacted into
// ascending lists with wave ballots.
//
// VS heads, cumulative coverage (the FlexPrefill-style rule the pages contrast
// with Eq. 4; selectable for comparison): per direction the shortest prefix of
// the blocks ordered by (mass desc, index asc) whose mass reaches gamma of the
// total, plus the first and last block; found by a radix select over the 48-bit
// masses inside one workgroup per (head, direction).
//
// PE heads, GlobalAdaptive (Alg. 4): block means of Q and K (sequential fp32
// sums), pooled scores zbar = fl(fma-chain(Qbar, Kbar) c) for kb <= qb, row
// softmax with exp_crisp and int64 sums, quantised map Abar_q, total Tbar.
// The gamma-cumsum prefix under the order (Abar_q desc, flat index asc) is
// found by a radix select over the 41-bit values with (count, mass)
// histograms, then ties at the cut value are taken in index order; every
// diagonal block is added; rows are written as CSR.
#include "common.h"
#include "kernels.h"

namespace crisp {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void vs_select_kernel(Dims dm, SelectArgs sa, IndexOut io) {
  __shared__ int wave_cnt[4];
  const int bh = blockIdx.x, tid = threadIdx.x, nb = dm.nb;
  if (!io.route[bh]) {
    if (tid < 2) io.vs_count[bh * 2 + tid] = 0;
    return;
  }
  if (sa.cumulative) return;  // vs_cumulative_kernel
  const long long T = io.mass_total[bh];
  for (int dir = 0; dir < 2; ++dir) {
    const long long* p = (dir == 0 ? io.mass_v : io.mass_s) + (size_t)bh * nb;
    int* list = (dir == 0 ? io.vs_vertical : io.vs_slash) + (size_t)bh * nb;
    const bool all = sa.keep_all || nb <= 2;
    long long M = all ? 0 : T - p[0] - p[nb - 1];
    if (M < 0) M = 0;
    const unsigned __int128 rhs = (unsigned __int128)sa.alpha_num * (unsigned __int128)M;
    int cnt = 0;
    for (int base = 0; base < nb; base += kThreads) {
      const int b = base + tid;
      bool flag = false;
      if (b < nb) {
        if (all || b == 0 || b == nb - 1) {
          flag = true;
        } else {
          const unsigned __int128 lhs = (unsigned __int128)sa.alpha_den *
                                        (unsigned __int128)(nb - 2) * (unsigned __int128)p[b];
          flag = lhs > rhs;
        }
      }
      int tot;
      const int pos = block_compact(flag, wave_cnt, &tot);
      if (flag) list[cnt + pos] = b;
      cnt += tot;
    }
    if (tid == 0) io.vs_count[bh * 2 + dir] = cnt;
    __syncthreads();
  }
}

// Cumulative coverage for VS heads: one workgroup per (head, direction).
constexpr int kCumThreads = 1024;
constexpr int kCumBins = 4096;  // 12-bit digits: four passes cover the 48-bit masses

__global__ __launch_bounds__(kCumThreads) void vs_cumulative_kernel(Dims dm, SelectArgs sa, IndexOut io) {
  __shared__ unsigned int cnt[kCumBins];
  __shared__ unsigned long long mass[kCumBins];
  __shared__ long long part[kCumThreads];
  __shared__ long long cut[2];  // remaining mass, value prefix
  __shared__ int wave_cnt[kCumThreads / 64];
  const int bh = blockIdx.x >> 1, dir = blockIdx.x & 1, tid = threadIdx.x, nb = dm.nb;
  if (!io.route[bh]) return;  // PE head: counts written by vs_select_kernel
  const long long* p = (dir == 0 ? io.mass_v : io.mass_s) + (size_t)bh * nb;
  int* list = (dir == 0 ? io.vs_vertical : io.vs_slash) + (size_t)bh * nb;
  const long long T = io.mass_total[bh];
  // target: the smallest integer cum with gamma_den cum >= gamma_num T
  const unsigned __int128 num = (unsigned __int128)sa.gamma_num * (unsigned __int128)T;
  const long long tgt = (long long)((num + sa.gamma_den - 1) / sa.gamma_den);
  constexpr long long kNone = 0x7fffffffffffffffLL;
  long long vstar = kNone, rties = 0;  // cut value and the number of ties at it to take
  if (tgt > 0 && nb > 2) {
    long long R = tgt, prefix = 0;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 36 - 12 * pass;
      for (int i = tid; i < kCumBins; i += kCumThreads) cnt[i] = 0, mass[i] = 0;
      __syncthreads();
      for (int b = tid; b < nb; b += kCumThreads) {
        const long long v = p[b];
        if ((v >> (shift + 12)) == (prefix >> (shift + 12))) {
          const int dg = (int)((v >> shift) & (kCumBins - 1));
          atomicAdd(&cnt[dg], 1u);
          atomicAdd(&mass[dg], (unsigned long long)v);
        }
      }
      __syncthreads();
      // thread t owns digits 4095 - 4t .. 4095 - 4t - 3 (largest first)
      long long mine = 0;
      for (int k2 = 0; k2 < 4; ++k2) mine += (long long)mass[kCumBins - 1 - (4 * tid + k2)];
      part[tid] = mine;
      __syncthreads();
      for (int off = 1; off < kCumThreads; off <<= 1) {
        const long long v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
      }
      const long long before = part[tid] - mine;
      if (before < R && R <= before + mine) {  // the digit where the running mass reaches R
        long long c = before;
        for (int k2 = 0; k2 < 4; ++k2) {
          const int dg = kCumBins - 1 - (4 * tid + k2);
          const long long m = (long long)mass[dg];
          if (c + m >= R) {
            cut[0] = R - c;
            cut[1] = prefix | ((long long)dg << shift);
            break;
          }
          c += m;
        }
      }
      __syncthreads();
      R = cut[0];
      prefix = cut[1];
      __syncthreads();
    }
    vstar = prefix;                  // > 0: the remaining mass R > 0 lies in this value
    rties = (R + vstar - 1) / vstar;  // ties at v* needed, lowest indices first
  }
  int cnt_out = 0;
  long long tcur = 0;
  for (int base = 0; base < nb; base += kCumThreads) {
    const int b = base + tid;
    const bool in = b < nb;
    const long long v = in ? p[b] : 0;
    const bool tie = in && v == vstar;
    int ntie;
    const int tpos = block_compact(tie, wave_cnt, &ntie);
    const bool flag = in && (nb <= 2 || b == 0 || b == nb - 1 || v > vstar || (tie && tcur + tpos < rties));
    tcur += ntie;
    int tot;
    const int pos = block_compact(flag, wave_cnt, &tot);
    if (flag) list[cnt_out + pos] = b;
    cnt_out += tot;
  }
  if (tid == 0) io.vs_count[bh * 2 + dir] = cnt_out;
}

// ------------------------------------------------------------- PE path ----
__device__ __forceinline__ bool group_has_pe(const IndexOut& io, const Dims& dm, int kvh) {
  const int b = kvh / dm.hkv, g = kvh % dm.hkv;
  for (int t = 0; t < dm.group; ++t)
    if (!io.route[b * dm.hq + g * dm.group + t]) return true;
  return false;
}

// Block means: Qbar[qb][k] = fl(sum over rows ascending) / cnt; same for K.
// Unit u = y * nb + qb: query head y < bh (PE heads only) or KV head y - bh
// (groups with a PE head); a thread owns eight columns of one unit, so the
// d / 8 threads of a unit read each row as contiguous 16-byte pieces.
template <typename T>
__global__ __launch_bounds__(256) void pe_pool_kernel(Dims dm, const T* __restrict__ q, const T* __restrict__ k,
                                                      IndexOut io, float* __restrict__ qbar,
                                                      float* __restrict__ kbar) {
  const int tpu = dm.d / 8;
  const long long units = (long long)(dm.bh + dm.bkv) * dm.nb;
  const long long u = (long long)blockIdx.x * (256 / tpu) + threadIdx.x / tpu;
  if (u >= units) return;
  const int y = (int)(u / dm.nb), qb = (int)(u % dm.nb);
  const T* src;
  float* dst;
  if (y < dm.bh) {
    if (io.route[y]) return;
    src = q + (size_t)y * dm.n * dm.d;
    dst = qbar + ((size_t)y * dm.nb + qb) * dm.d;
  } else {
    const int kvh = y - dm.bh;
    if (!group_has_pe(io, dm, kvh)) return;
    src = k + (size_t)kvh * dm.n * dm.d;
    dst = kbar + ((size_t)kvh * dm.nb + qb) * dm.d;
  }
  const int r0 = qb * dm.B;
  const int c0 = (threadIdx.x % tpu) * 8;
  float out[8];
  mean8(src + (size_t)r0 * dm.d + c0, dm.d, min(dm.B, dm.n - r0), out);
  float4* o4 = reinterpret_cast<float4*>(dst + c0);
  o4[0] = make_float4(out[0], out[1], out[2], out[3]);
  o4[1] = make_float4(out[4], out[5], out[6], out[7]);
}

// Pooled scores zbar[qb][kb] = fl(fma-chain(Qbar_qb, Kbar_kb) c) for kb <= qb, one
// 128 x 128 tile of (query block, key block) per workgroup (tiles on or below the
// diagonal only), 8 x 8 per thread.  The head dimension is staged through LDS in
// 32-wide chunks: each thread reads 16-byte pieces of the rows, held in registers
// while the previous chunk is computed, and stores them dim-major so that a thread
// reads its 8 rows (and 8 keys) of one dimension as two 16-byte LDS loads.  Every
// accumulator keeps its fma chain over the dimensions in ascending order.
constexpr int kPsTile = 128, kPsTm = 8, kPsKc = 32, kPsLd = kPsTile + 4;

template <int D>
__global__ __launch_bounds__(kThreads) void pe_scores_kernel(Dims dm, IndexOut io,
                                                             const float* __restrict__ qbar,
                                                             const float* __restrict__ kbar,
                                                             float* __restrict__ zbar) {
  __shared__ __align__(16) float Qs[kPsKc * kPsLd];
  __shared__ __align__(16) float Ks[kPsKc * kPsLd];
  // tile t of the lower triangle (row tile rt, column tile ct <= rt, row-major)
  const int t = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  int rt = (int)((__builtin_sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((rt + 1) * (rt + 2) / 2 <= t) ++rt;
  while (rt * (rt + 1) / 2 > t) --rt;
  const int ct = t - rt * (rt + 1) / 2;
  if (io.route[bh]) return;
  // tx: the 8 keys of a thread (consecutive lanes, consecutive keys: each row of the
  // tile is written as one contiguous 512-byte run by 16 lanes); ty: its 8 rows
  const int tx = tid & 15, ty = tid >> 4;
  const int b = bh / dm.hq;
  const int kvh = b * dm.hkv + (bh % dm.hq) / dm.group;
  const float* qs = qbar + ((size_t)bh * dm.nb + (size_t)rt * kPsTile) * D;
  const float* ks = kbar + ((size_t)kvh * dm.nb + (size_t)ct * kPsTile) * D;
  const int qrows = min(kPsTile, dm.nb - rt * kPsTile), krows = min(kPsTile, dm.nb - ct * kPsTile);
  float acc[kPsTm][kPsTm];
#pragma unroll
  for (int i = 0; i < kPsTm; ++i)
#pragma unroll
    for (int j = 0; j < kPsTm; ++j) acc[i][j] = 0.0f;
  // a chunk of one operand is 128 rows x 8 pieces of 4 dims: piece g has row g % 128
  // and dims 4 (g / 128) .. + 3 of the chunk
  constexpr int kPieces = kPsTile * kPsKc / 4 / kThreads;  // 4 per thread and operand
  float4 qv[kPieces], kv[kPieces];
  auto fetch = [&](int dc) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int g = tid + kThreads * i, r = g % kPsTile, d4 = (g / kPsTile) * 4;
      qv[i] = r < qrows ? *reinterpret_cast<const float4*>(qs + (size_t)r * D + dc + d4) : make_float4(0, 0, 0, 0);
      kv[i] = r < krows ? *reinterpret_cast<const float4*>(ks + (size_t)r * D + dc + d4) : make_float4(0, 0, 0, 0);
    }
  };
  fetch(0);
  for (int dc = 0; dc < D; dc += kPsKc) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int g = tid + kThreads * i, r = g % kPsTile, d4 = (g / kPsTile) * 4;
      Qs[(d4 + 0) * kPsLd + r] = qv[i].x;
      Qs[(d4 + 1) * kPsLd + r] = qv[i].y;
      Qs[(d4 + 2) * kPsLd + r] = qv[i].z;
      Qs[(d4 + 3) * kPsLd + r] = qv[i].w;
      Ks[(d4 + 0) * kPsLd + r] = kv[i].x;
      Ks[(d4 + 1) * kPsLd + r] = kv[i].y;
      Ks[(d4 + 2) * kPsLd + r] = kv[i].z;
      Ks[(d4 + 3) * kPsLd + r] = kv[i].w;
    }
    __syncthreads();
    if (dc + kPsKc < D) fetch(dc + kPsKc);
#pragma unroll 4
    for (int kk = 0; kk < kPsKc; ++kk) {
      float a[kPsTm], bb[kPsTm];
#pragma unroll
      for (int i = 0; i < kPsTm; i += 4) {
        const float4 va = *reinterpret_cast<const float4*>(&Qs[kk * kPsLd + ty * kPsTm + i]);
        const float4 vb = *reinterpret_cast<const float4*>(&Ks[kk * kPsLd + tx * kPsTm + i]);
        a[i] = va.x, a[i + 1] = va.y, a[i + 2] = va.z, a[i + 3] = va.w;
        bb[i] = vb.x, bb[i + 1] = vb.y, bb[i + 2] = vb.z, bb[i + 3] = vb.w;
      }
#pragma unroll
      for (int i = 0; i < kPsTm; ++i)
#pragma unroll
        for (int j = 0; j < kPsTm; ++j) acc[i][j] = __builtin_fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
  const float c = (float)(1.0 / __builtin_sqrt((double)D));
  const int kb0 = ct * kPsTile + tx * kPsTm;
#pragma unroll
  for (int i = 0; i < kPsTm; ++i) {
    const int qb = rt * kPsTile + ty * kPsTm + i;
    if (qb >= dm.nb) continue;
    float* dst = zbar + ((size_t)bh * dm.nb + qb) * dm.nb + kb0;
    float z[kPsTm];
#pragma unroll
    for (int j = 0; j < kPsTm; ++j) z[j] = acc[i][j] * c;
    if (kb0 + kPsTm - 1 <= qb && ((uintptr_t)dst & 15) == 0) {
      reinterpret_cast<float4*>(dst)[0] = make_float4(z[0], z[1], z[2], z[3]);
      reinterpret_cast<float4*>(dst)[1] = make_float4(z[4], z[5], z[6], z[7]);
    } else {
#pragma unroll
      for (int j = 0; j < kPsTm; ++j)
        if (kb0 + j <= qb) dst[j] = z[j];
    }
  }
}

// Row softmax of the pooled map in fixed point: Abar_q row, row total.  One
// wave per query block (four rows per workgroup), so every reduction is a
// wave reduction; rows are assigned longest first (row nb - 1 - r).
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float o = __shfl_xor(v, m);
    v = o > v ? o : v;
  }
  return v;
}
// The passes over a row read kRowUnroll chunks of 64 entries before using any of
// them, so a wave keeps that many loads in flight (one chunk at a time left the
// kernel waiting on memory latency, not bandwidth).
constexpr int kRowUnroll = 8;

__global__ __launch_bounds__(kThreads) void pe_rowsoft_kernel(Dims dm, IndexOut io,
                                                              const float* __restrict__ zbar,
                                                              long long* __restrict__ abar,
                                                              long long* __restrict__ rowtot) {
  const int bh = blockIdx.y, lane = threadIdx.x & 63;
  const int qb = dm.nb - 1 - (blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6));
  if (qb < 0 || io.route[bh]) return;
  const float* z = zbar + ((size_t)bh * dm.nb + qb) * dm.nb;
  constexpr int kStep = 64 * kRowUnroll;
  float m = -__builtin_inff();
  for (int base = 0; base <= qb; base += kStep) {
    float zz[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int kb = base + 64 * u + lane;
      zz[u] = kb <= qb ? z[kb] : -__builtin_inff();
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) m = zz[u] > m ? zz[u] : m;
  }
  m = wave_max_f32(m);
  long long L = 0;
  for (int base = 0; base <= qb; base += kStep) {
    float zz[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int kb = base + 64 * u + lane;
      zz[u] = kb <= qb ? z[kb] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u)
      if (base + 64 * u + lane <= qb) L += fix_rne(exp_crisp(zz[u] - m));
  }
  L = wave_sum_i64(L);
  const float l = fix_to_float(L), rl = 1.0f / l;
  long long* out = abar + (size_t)bh * dm.ntri + (size_t)qb * (qb + 1) / 2;
  long long tot = 0;
  for (int base = 0; base <= qb; base += kStep) {
    float zz[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int kb = base + 64 * u + lane;
      zz[u] = kb <= qb ? z[kb] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int kb = base + 64 * u + lane;
      if (kb <= qb) {
        const long long aq = fix_rne(quot_rn(exp_crisp(zz[u] - m), l, rl));
        out[kb] = aq;
        tot += aq;
      }
    }
  }
  tot = wave_sum_i64(tot);
  if (lane == 0) rowtot[(size_t)bh * dm.nb + qb] = tot;
}

// Radix-select state per head (int64 slots):
//   0 remaining mass R still to cover inside the current prefix
//   1 value prefix found so far
//   2 cut value v* (set after the last pass; -1 = keep all; INT64_MAX = keep none)
//   3 number of ties at v* to take (in index order)
//   4 active flag
constexpr int kPassShift[4] = {30, 20, 10, 0};
constexpr int kPassWidth[4] = {11, 10, 10, 10};
constexpr int kHistBins = 2048;

__global__ __launch_bounds__(kThreads) void pe_radix_init_kernel(Dims dm, SelectArgs sa, IndexOut io,
                                                                 const long long* __restrict__ rowtot,
                                                                 unsigned long long* __restrict__ hist,
                                                                 long long* __restrict__ state) {
  __shared__ long long red[4];
  const int bh = blockIdx.x, tid = threadIdx.x;
  long long* st = state + (size_t)bh * 8;
  if (io.route[bh]) return;
  if (sa.keep_all) {
    if (tid == 0) st[0] = 0, st[1] = 0, st[2] = -1, st[3] = 0, st[4] = 0;
    return;
  }
  unsigned long long* h = hist + (size_t)bh * 4 * kHistBins * 2;
  for (int i = tid; i < 4 * kHistBins * 2; i += kThreads) h[i] = 0;
  long long T = 0;
  for (int qb = tid; qb < dm.nb; qb += kThreads) T += rowtot[(size_t)bh * dm.nb + qb];
  T = block_sum_i64(T, red);
  if (tid == 0) {
    // target: smallest integer cum with gamma_den cum >= gamma_num T
    const unsigned __int128 num = (unsigned __int128)sa.gamma_num * (unsigned __int128)T;
    const unsigned __int128 tgt = (num + sa.gamma_den - 1) / sa.gamma_den;
    st[0] = (long long)tgt;
    st[1] = 0;
    st[2] = tgt == 0 ? 0x7fffffffffffffffLL : 0;
    st[3] = 0;
    st[4] = tgt == 0 ? 0 : 1;
  }
}

__global__ __launch_bounds__(kThreads) void pe_radix_hist_kernel(Dims dm, IndexOut io, int pass,
                                                                 const long long* __restrict__ abar,
                                                                 unsigned long long* __restrict__ hist,
                                                                 const long long* __restrict__ state,
                                                                 long long chunk) {
  __shared__ unsigned int cnt[kHistBins];
  __shared__ unsigned long long mass[kHistBins];
  const int bh = blockIdx.y, tid = threadIdx.x;
  if (io.route[bh] || !state[(size_t)bh * 8 + 4]) return;
  const long long begin = (long long)blockIdx.x * chunk;
  if (begin >= dm.ntri) return;
  const long long end = min(begin + chunk, dm.ntri);
  const int shift = kPassShift[pass], width = kPassWidth[pass];
  const long long prefix = state[(size_t)bh * 8 + 1];
  const int hi = shift + width;
  for (int i = tid; i < kHistBins; i += kThreads) cnt[i] = 0, mass[i] = 0;
  __syncthreads();
  // a thread scans runs of 16 consecutive values and adds each run of equal
  // digits to LDS once: neighbouring entries of a row of the pooled map are
  // close in value, so most runs collapse (pass 0 puts most of the map in one bin)
  const long long* a = abar + (size_t)bh * dm.ntri;
  constexpr int kRun = 16;
  int cur = -1;
  unsigned ccnt = 0;
  unsigned long long cmass = 0;
  auto add = [&](long long v) {
    if ((v >> hi) != (prefix >> hi)) return;
    const int dg = (int)((v >> shift) & ((1 << width) - 1));
    if (dg != cur) {
      if (ccnt) {
        atomicAdd(&cnt[cur], ccnt);
        atomicAdd(&mass[cur], cmass);
      }
      cur = dg, ccnt = 0, cmass = 0;
    }
    ++ccnt;
    cmass += (unsigned long long)v;
  };
  for (long long e0 = begin + (long long)tid * kRun; e0 < end; e0 += (long long)kThreads * kRun) {
    if (e0 + kRun <= end && (((size_t)(a + e0)) & 15) == 0) {
      longlong2 w[kRun / 2];
#pragma unroll
      for (int j = 0; j < kRun / 2; ++j) w[j] = reinterpret_cast<const longlong2*>(a + e0)[j];
#pragma unroll
      for (int j = 0; j < kRun / 2; ++j) add(w[j].x), add(w[j].y);
    } else {
      for (long long e = e0; e < end && e < e0 + kRun; ++e) add(a[e]);
    }
  }
  if (ccnt) {
    atomicAdd(&cnt[cur], ccnt);
    atomicAdd(&mass[cur], cmass);
  }
  __syncthreads();
  unsigned long long* h = hist + ((size_t)bh * 4 + pass) * kHistBins * 2;
  for (int i = tid; i < (1 << width); i += kThreads) {
    if (cnt[i]) {
      atomicAdd(&h[2 * i], (unsigned long long)cnt[i]);
      atomicAdd(&h[2 * i + 1], mass[i]);
    }
  }
}

// Find the digit where the running mass (from the largest values down) first
// reaches the remaining target R; everything in higher buckets is inside the
// prefix.  After the last pass the full cut value v* is known.
__global__ __launch_bounds__(kThreads) void pe_radix_scan_kernel(IndexOut io, int pass,
                                                                 const unsigned long long* __restrict__ hist,
                                                                 long long* __restrict__ state) {
  __shared__ long long part[kThreads];
  const int bh = blockIdx.x, tid = threadIdx.x;
  long long* st = state + (size_t)bh * 8;
  if (io.route[bh] || !st[4]) return;
  const int shift = kPassShift[pass], width = kPassWidth[pass];
  const int bins = 1 << width;
  const int per = bins / kThreads;  // 8 or 4 digits per thread, highest digits to thread 0
  const unsigned long long* h = hist + ((size_t)bh * 4 + pass) * kHistBins * 2;
  const long long R = st[0];
  long long mine = 0;
  for (int t = 0; t < per; ++t) mine += (long long)h[2 * (bins - 1 - (tid * per + t)) + 1];
  part[tid] = mine;
  __syncthreads();
  // exclusive prefix (Hillis-Steele) over threads in descending-digit order
  for (int off = 1; off < kThreads; off <<= 1) {
    long long v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const long long before = part[tid] - mine;
  if (before < R && R <= before + mine) {
    long long cum = before;
    for (int t = 0; t < per; ++t) {
      const int dg = bins - 1 - (tid * per + t);
      const long long s = (long long)h[2 * dg + 1];
      if (cum + s >= R) {
        const long long prefix = st[1] | ((long long)dg << shift);
        const long long Rn = R - cum;
        st[0] = Rn;
        st[1] = prefix;
        if (pass == 3) {
          st[2] = prefix;                  // v* (> 0 since Rn > 0)
          st[3] = (Rn + prefix - 1) / prefix;  // ties at v* needed, lowest indices first
        }
        break;
      }
      cum += s;
    }
  }
}

// Per query-block row: values above v*, ties at v*.
__global__ __launch_bounds__(kThreads) void pe_count_kernel(Dims dm, IndexOut io,
                                                            const long long* __restrict__ abar,
                                                            const long long* __restrict__ state,
                                                            int* __restrict__ gtcnt, int* __restrict__ tiecnt) {
  // one wave per query block, longest rows first
  const int bh = blockIdx.y, lane = threadIdx.x & 63;
  const int qb = dm.nb - 1 - (blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6));
  if (qb < 0 || io.route[bh]) return;
  const long long vstar = state[(size_t)bh * 8 + 2];
  const long long* a = abar + (size_t)bh * dm.ntri + (size_t)qb * (qb + 1) / 2;
  int gt = 0, tie = 0;
  if (vstar >= 0 && vstar != 0x7fffffffffffffffLL)
    for (int base = 0; base <= qb; base += 64 * kRowUnroll) {
      long long v[kRowUnroll];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int kb = base + 64 * u + lane;
        v[u] = kb <= qb ? a[kb] : -1;  // -1 is below every value and never equals v*
      }
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        gt += v[u] > vstar;
        tie += v[u] == vstar;
      }
    }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    gt += __shfl_xor(gt, m);
    tie += __shfl_xor(tie, m);
  }
  if (lane == 0) {
    gtcnt[(size_t)bh * dm.nb + qb] = gt;
    tiecnt[(size_t)bh * dm.nb + qb] = tie;
  }
}
// Row pointers: exclusive scans over query blocks of the tie counts and the
// row sizes (values above v*, the first ties, plus the diagonal if not in).
__global__ __launch_bounds__(1024) void pe_scan_kernel(Dims dm, IndexOut io,
                                                       const long long* __restrict__ abar,
                                                       const long long* __restrict__ state,
                                                       const int* __restrict__ gtcnt,
                                                       const int* __restrict__ tiecnt,
                                                       int* __restrict__ tiepre) {
  __shared__ long long sa[1024], sb[1024];
  const int bh = blockIdx.x, tid = threadIdx.x, nb = dm.nb;
  int* rowptr = io.pe_rowptr + (size_t)bh * (nb + 1);
  if (io.route[bh]) {
    for (int i = tid; i <= nb; i += 1024) rowptr[i] = 0;
    return;
  }
  const long long* st = state + (size_t)bh * 8;
  const long long vstar = st[2], rties = st[3];
  const bool all = vstar < 0;
  const int per = (nb + 1023) / 1024;
  const int lo = min(tid * per, nb), hi = min(lo + per, nb);
  long long tsum = 0, rsum = 0;
  for (int qb = lo; qb < hi; ++qb) {
    tsum += all ? 0 : tiecnt[(size_t)bh * nb + qb];
  }
  sa[tid] = tsum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    long long v = tid >= off ? sa[tid - off] : 0;
    __syncthreads();
    sa[tid] += v;
    __syncthreads();
  }
  long long tp = sa[tid] - tsum;  // ties in rows before lo
  // row sizes
  long long tcur = tp;
  for (int qb = lo; qb < hi; ++qb) {
    long long sz;
    if (all) {
      sz = qb + 1;
    } else {
      const int tc = tiecnt[(size_t)bh * nb + qb];
      long long take = rties - tcur;
      take = take < 0 ? 0 : (take > tc ? tc : take);
      const long long vd = abar[(size_t)bh * dm.ntri + (size_t)qb * (qb + 1) / 2 + qb];
      // the diagonal is the last element of its row: if it ties, it has the row's last tie rank
      const bool diag_in = vd > vstar || (vd == vstar && tcur + tc - 1 < rties);
      sz = gtcnt[(size_t)bh * nb + qb] + take + (diag_in ? 0 : 1);
      tiepre[(size_t)bh * nb + qb] = (int)tcur;
      tcur += tc;
    }
    rsum += sz;
  }
  sb[tid] = rsum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    long long v = tid >= off ? sb[tid - off] : 0;
    __syncthreads();
    sb[tid] += v;
    __syncthreads();
  }
  long long rp = sb[tid] - rsum;
  tcur = tp;
  for (int qb = lo; qb < hi; ++qb) {
    rowptr[qb] = (int)rp;
    long long sz;
    if (all) {
      sz = qb + 1;
    } else {
      const int tc = tiecnt[(size_t)bh * nb + qb];
      long long take = rties - tcur;
      take = take < 0 ? 0 : (take > tc ? tc : take);
      const long long vd = abar[(size_t)bh * dm.ntri + (size_t)qb * (qb + 1) / 2 + qb];
      const bool diag_in = vd > vstar || (vd == vstar && tcur + tc - 1 < rties);
      sz = gtcnt[(size_t)bh * nb + qb] + take + (diag_in ? 0 : 1);
      tcur += tc;
    }
    rp += sz;
  }
  if (tid == 1023) rowptr[nb] = (int)rp;
}

__global__ __launch_bounds__(kThreads) void pe_write_kernel(Dims dm, IndexOut io,
                                                            const long long* __restrict__ abar,
                                                            const long long* __restrict__ state,
                                                            const int* __restrict__ tiepre) {
  // one wave per query block, longest rows first; ascending compaction by ballots
  const int bh = blockIdx.y, lane = threadIdx.x & 63;
  const int qb = dm.nb - 1 - (blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6));
  if (qb < 0 || io.route[bh]) return;
  const long long* st = state + (size_t)bh * 8;
  const long long vstar = st[2], rties = st[3];
  const bool all = vstar < 0;
  const long long* a = abar + (size_t)bh * dm.ntri + (size_t)qb * (qb + 1) / 2;
  int* out = io.pe_col + (size_t)bh * io.pe_cap + io.pe_rowptr[(size_t)bh * (dm.nb + 1) + qb];
  long long tcur = all ? 0 : tiepre[(size_t)bh * dm.nb + qb];
  const unsigned long long below = (1ull << lane) - 1ull;
  int cnt = 0;
  for (int base0 = 0; base0 <= qb; base0 += 64 * kRowUnroll) {
    long long vv[kRowUnroll];  // the loads of kRowUnroll chunks first, then the chunks in order
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int kb = base0 + 64 * u + lane;
      vv[u] = (kb <= qb && !all) ? a[kb] : 0;
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int kb = base0 + 64 * u + lane;
      const bool in = kb <= qb;
      const long long v = vv[u];
      const bool tie = in && !all && v == vstar;
      const unsigned long long tmask = __ballot(tie);
      const int tpos = __popcll(tmask & below);
      const bool flag = in && (all || v > vstar || kb == qb || (tie && tcur + tpos < rties));
      tcur += __popcll(tmask);
      const unsigned long long fmask = __ballot(flag);
      if (flag) out[cnt + __popcll(fmask & below)] = kb;
      cnt += __popcll(fmask);
    }
  }
}
template <typename T>
void launch_pool(const Dims& dm, const void* q, const void* k, const IndexOut& io, float* qbar,
                 float* kbar, hipStream_t st) {
  const int upb = 256 / (dm.d / 8);  // units per workgroup
  const long long units = (long long)(dm.bh + dm.bkv) * dm.nb;
  pe_pool_kernel<T><<<(unsigned)((units + upb - 1) / upb), 256, 0, st>>>(
      dm, static_cast<const T*>(q), static_cast<const T*>(k), io, qbar, kbar);
}

}  // namespace

hipError_t launch_select(const Dims& dm, const SelectArgs& sa, const void* q, const void* k,
                         const SelectScratch& ws, const IndexOut& io, hipStream_t st) {
  const dim3 rows((dm.nb + kThreads / 64 - 1) / (kThreads / 64), dm.bh);  // one wave per query block
  vs_select_kernel<<<dm.bh, kThreads, 0, st>>>(dm, sa, io);
  if (sa.cumulative) vs_cumulative_kernel<<<dm.bh * 2, kCumThreads, 0, st>>>(dm, sa, io);
  if (!sa.keep_all) {
    if (dm.dtype == 1)
      launch_pool<bf16_t>(dm, q, k, io, ws.qbar, ws.kbar, st);
    else
      launch_pool<float>(dm, q, k, io, ws.qbar, ws.kbar, st);
    const int nt = (dm.nb + kPsTile - 1) / kPsTile, ntri_t = nt * (nt + 1) / 2;
    if (dm.d == 128)
      pe_scores_kernel<128><<<dim3(ntri_t, dm.bh), kThreads, 0, st>>>(dm, io, ws.qbar, ws.kbar, ws.zbar);
    else
      pe_scores_kernel<64><<<dim3(ntri_t, dm.bh), kThreads, 0, st>>>(dm, io, ws.qbar, ws.kbar, ws.zbar);
    pe_rowsoft_kernel<<<rows, kThreads, 0, st>>>(dm, io, ws.zbar, ws.abar, ws.rowtot);
  }
  pe_radix_init_kernel<<<dm.bh, kThreads, 0, st>>>(dm, sa, io, ws.rowtot, ws.hist, ws.state);
  if (!sa.keep_all) {
    const long long chunk = 16384;
    const int nchunks = (int)((dm.ntri + chunk - 1) / chunk);
    for (int pass = 0; pass < 4; ++pass) {
      pe_radix_hist_kernel<<<dim3(nchunks, dm.bh), kThreads, 0, st>>>(dm, io, pass, ws.abar, ws.hist,
                                                                        ws.state, chunk);
      pe_radix_scan_kernel<<<dm.bh, kThreads, 0, st>>>(io, pass, ws.hist, ws.state);
    }
    pe_count_kernel<<<rows, kThreads, 0, st>>>(dm, io, ws.abar, ws.state, ws.gtcnt, ws.tiecnt);
  }
  pe_scan_kernel<<<dm.bh, 1024, 0, st>>>(dm, io, ws.abar, ws.state, ws.gtcnt, ws.tiecnt, ws.tiepre);
  pe_write_kernel<<<rows, kThreads, 0, st>>>(dm, io, ws.abar, ws.state, ws.tiepre);
  return hipGetLastError();
}

}  // namespace crisp
