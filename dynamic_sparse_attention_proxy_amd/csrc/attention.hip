// Sparse and dense causal prefill attention (CRISP summary page, "Algorithm
// Overview", Alg. 1: attention over the selected index set).
//
// Work item = (head, query block of B rows).  Its key tiles (key block kb,
// mask mode) come from a per-item list (sparse) or are 0..qb (dense):
//   VS head : kb in V (whole tile), kb = qb - s for s in S (lower triangle
//             r >= c of the tile: offsets in block s), kb = qb - s - 1
//             (upper triangle r < c: the same offset block from the tile
//             below the diagonal); a selected slash block is the band of
//             diagonals [sB, sB + B).
//   PE head : the CSR row of query block qb.
//   Every tile is intersected with causality (diagonal tile: r >= c).
//
// bf16, d = 128, B = 128: matrix-core engine.  Each of the 4 waves owns 32
// query rows.  S^T = K Q^T is computed with v_mfma_f32_32x32x16_bf16 so that a
// lane holds one query's scores: the softmax max / sum need one cross-half
// exchange only, and the probabilities are already laid out as the B operand
// of O^T = V^T P^T (the key order inside each 32-key group is permuted on the
// K side to make that layout line up).  K is staged in LDS row-major, V is
// transposed in registers (8 x 8 bf16 blocks) while being staged, so every
// LDS read feeding a matrix instruction is one 16-byte vector.
#include "common.h"
#include "kernels.h"

namespace crisp {

namespace {

#ifndef CRISP_ATTN_QG
#define CRISP_ATTN_QG 1
#endif

constexpr int kModeLower = 1;  // r >= c inside the tile
constexpr int kModeUpper = 2;  // r <  c inside the tile
constexpr int kModeFull = 3;

// ------------------------------------------------------------ tile lists --
__global__ void build_tiles_kernel(Dims dm, IndexOut io, int* __restrict__ tiles,
                                   int* __restrict__ tile_cnt) {
  const int qb = blockIdx.x * blockDim.x + threadIdx.x;
  const int bh = blockIdx.y;
  if (qb >= dm.nb) return;
  int* out = tiles + (size_t)bh * dm.ntri + (size_t)qb * (qb + 1) / 2;
  int cnt = 0;
  if (io.route[bh]) {
    const int nv = io.vs_count[bh * 2], ns = io.vs_count[bh * 2 + 1];
    const int* V = io.vs_vertical + (size_t)bh * dm.nb;
    const int* S = io.vs_slash + (size_t)bh * dm.nb;
    int a = 0;
    int sb = ns - 1;
    while (sb >= 0 && S[sb] > qb) --sb;
    int sc = sb;
    while (sc >= 0 && S[sc] > qb - 1) --sc;
    const int inf = 0x7fffffff;
    while (true) {
      const int ka = (a < nv && V[a] <= qb) ? V[a] : inf;
      const int kl = sb >= 0 ? qb - S[sb] : inf;
      const int ku = sc >= 0 ? qb - 1 - S[sc] : inf;
      int kbv = ka < kl ? ka : kl;
      kbv = kbv < ku ? kbv : ku;
      if (kbv == inf) break;
      int mode = 0;
      if (ka == kbv) mode |= kModeFull, ++a;
      if (kl == kbv) mode |= kModeLower, --sb;
      if (ku == kbv) mode |= kModeUpper, --sc;
      if (kbv == qb) mode &= kModeLower;
      if (kbv >= 0 && mode) out[cnt++] = kbv | (mode << 28);
    }
  } else {
    const int* rp = io.pe_rowptr + (size_t)bh * (dm.nb + 1);
    const int* col = io.pe_col + (size_t)bh * io.pe_cap;
    for (int p = rp[qb]; p < rp[qb + 1]; ++p) {
      const int kbv = col[p];
      if (kbv >= 0 && kbv <= qb) out[cnt++] = kbv | ((kbv == qb ? kModeLower : kModeFull) << 28);
    }
  }
  tile_cnt[(size_t)bh * dm.nb + qb] = cnt;
}

// Heaviest query blocks first: item L -> (qb descending, head).
__device__ __forceinline__ void work_item(const Dims& dm, int L, int* qb, int* bh) {
  *qb = dm.nb - 1 - L / dm.bh;
  *bh = L % dm.bh;
}

__device__ __forceinline__ bool tile_keep(int mode, bool diag, int r, int c) {
  const bool lower = r >= c;
  const bool in_mode = lower ? (mode & kModeLower) != 0 : (mode & kModeUpper) != 0;
  return in_mode && (lower || !diag);
}

// ------------------------------------------------------- matrix engine ----
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
}

// sum of a packed bf16 pair added to acc (v_dot2 with (1, 1))
__device__ __forceinline__ float sum_bf16x2(unsigned pr, float acc) {
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pr), one, acc, false);
}

// key row inside a 32-key group that feeds matrix row rho (swap of bits 2 and 3)
__device__ __forceinline__ int key_perm(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

// Work item of the matrix engine: (KV head g, pair w of its query heads, query
// block qb).  Items are ordered by query block, heaviest first; inside a level
// the pairs of one KV head are 8 items apart so they land on the same XCD
// (shared K/V in its L2), and the KV head served by an XCD rotates with the
// level so that cheap (VS) and expensive (PE) groups alternate on every XCD.
__device__ __forceinline__ void pair_item(const Dims& dm, int pairs, int L, int* qb, int* g, int* w) {
  const int U = dm.bkv * pairs;
  const int level = L / U, p = L % U;
  *w = p / dm.bkv;
  *g = (p % dm.bkv + level) % dm.bkv;
  *qb = dm.nb - 1 - level;
}

// LDS layout of one K / V^T tile pair.  Rows are padded to 272 bytes so that
// every fragment address is a per-lane base plus a compile-time offset; V^T
// rows get a further 16-byte skew per group of 8 rows so the transposing
// stores of 16 lanes spread over the banks.
constexpr int kRowK = 136;                                  // bf16 per K row (256 B + 16 B pad)
constexpr int kTileK = 128 * kRowK;                         // 17408 bf16
constexpr int kRowV = 136;
__device__ __forceinline__ int v_off(int row) { return row * kRowV + (row >> 3) * 8; }
constexpr int kTileV = 128 * kRowV + 16 * 8;                // 17536 bf16
constexpr int kBuf = kTileK + kTileV;                       // one stage: 69888 bytes

// Matrix engine.  A workgroup serves 256 query rows that share every K/V tile:
// the two query heads of a pair x the 128 rows of query block qb.  Each wave
// owns QG groups of 32 query rows of one head (QG = 1: 8 waves, two per SIMD;
// QG = 2: 4 waves, one per SIMD, every K or V fragment read from LDS feeding
// two matrix instructions).  A 128-key tile is processed as two halves of 64
// keys.  K and V of tile t + 2 are fetched into registers while tile t is
// computed, and written to the other LDS stage before the barrier that ends
// the iteration.
template <bool kDense, int QG>
__global__ __launch_bounds__(512 / QG, 1) void attn_mfma_kernel(const bf16_t* __restrict__ q,
                                                                const bf16_t* __restrict__ k,
                                                                const bf16_t* __restrict__ v,
                                                                bf16_t* __restrict__ o, Dims dm, BiasArgs bias,
                                                                const int* __restrict__ ulist,
                                                                const int* __restrict__ ucnt, int pairs) {
  constexpr int B = 128, D = 128;
  constexpr int NT = 512 / QG;            // threads per workgroup
  constexpr int WPH = 4 / QG;             // waves per head
  constexpr int CH = (2 * 128 * 16) / NT; // 16-byte chunks of K (and of V) each thread stages
  __shared__ __align__(16) bf16_t lds[2 * kBuf];

  int qb, g, w;
  pair_item(dm, pairs, blockIdx.x, &qb, &g, &w);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = wave / WPH, wr = wave % WPH;
  const int hl = lane >> 5, ql = lane & 31;
  const int bidx = g / dm.hkv, gh = g % dm.hkv;
  const int hin = 2 * w + slot;
  const bool slot_on = hin < dm.group;
  const int bh = bidx * dm.hq + gh * dm.group + (slot_on ? hin : 0);
  const bf16_t* qp = q + (size_t)bh * dm.n * D;
  const bf16_t* kp = k + (size_t)g * dm.n * D;
  const bf16_t* vp = v + (size_t)g * dm.n * D;
  int r_in_blk[QG], qrow[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    r_in_blk[qg] = wr * 32 * QG + qg * 32 + ql;
    qrow[qg] = qb * B + r_in_blk[qg];
  }

  bf16x8_t qreg[QG][8];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (slot_on && qrow[qg] < dm.n)
        u = *reinterpret_cast<const uint4*>(qp + (size_t)qrow[qg] * D + 16 * kc + 8 * hl);
      qreg[qg][kc] = as_bf16x8(u);
    }
  f32x16 oacc[QG][4];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[qg][t][e] = 0.0f;
  float m_run[QG], l_run[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) m_run[qg] = -__builtin_inff(), l_run[qg] = 0.0f;
  const float log2e = 1.4426950408889634f;
  const float sl2 = (float)(1.0 / __builtin_sqrt(128.0)) * log2e;
  // per-lane fragment bases (elements); everything else is a constant offset
  const int kfrag = key_perm(ql) * kRowK + 8 * hl;
  const int vfrag = v_off(ql) + 8 * hl;

  const int item = g * pairs + w;
  const int ntile = kDense ? qb + 1 : ucnt[(size_t)item * dm.nb + qb];
  const int* tl = kDense ? nullptr : ulist + (size_t)item * dm.ntri + (size_t)qb * (qb + 1) / 2;

  // staging.  QG = 2: every thread moves 8 chunks of K and an 8 x 8 block of V.
  // QG = 1: threads 0..255 move K (8 chunks each), threads 256..511 the V blocks.
  const int st = tid & 255;
  const bool do_k = QG == 2 || tid < 256;
  const bool do_v = QG == 2 || tid >= 256;
  const int kg = st >> 4, dg = st & 15;
  uint4 pk[QG == 2 ? 8 : 8], pv[QG == 2 ? 8 : 1];
  (void)CH;
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (QG == 2) {
        const int id = st + 256 * i;
        const int key = kb * B + (id >> 4);
        pk[i] = make_uint4(0, 0, 0, 0);
        if (key < dm.n) pk[i] = *reinterpret_cast<const uint4*>(kp + (size_t)key * D + (id & 15) * 8);
        const int vkey = kb * B + kg * 8 + i;
        pv[QG == 2 ? i : 0] = make_uint4(0, 0, 0, 0);
        if (vkey < dm.n) pv[QG == 2 ? i : 0] = *reinterpret_cast<const uint4*>(vp + (size_t)vkey * D + dg * 8);
      } else if (do_k) {
        const int id = st + 256 * i;
        const int key = kb * B + (id >> 4);
        pk[i] = make_uint4(0, 0, 0, 0);
        if (key < dm.n) pk[i] = *reinterpret_cast<const uint4*>(kp + (size_t)key * D + (id & 15) * 8);
      } else {
        const int vkey = kb * B + kg * 8 + i;
        pk[i] = make_uint4(0, 0, 0, 0);
        if (vkey < dm.n) pk[i] = *reinterpret_cast<const uint4*>(vp + (size_t)vkey * D + dg * 8);
      }
    }
  };
  auto store_v = [&](bf16_t* Vt, const uint4* src) {
    // 8 keys x 8 dims -> 8 dims x 8 keys: dword w of key row e holds dims (2w, 2w+1)
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      unsigned lo[4], hi[4];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const uint4 a0 = src[2 * pp], a1 = src[2 * pp + 1];
        const unsigned ev = wd == 0 ? a0.x : wd == 1 ? a0.y : wd == 2 ? a0.z : a0.w;
        const unsigned od = wd == 0 ? a1.x : wd == 1 ? a1.y : wd == 2 ? a1.z : a1.w;
        lo[pp] = __builtin_amdgcn_perm(od, ev, 0x05040100u);  // low halves: dim 2w of keys 2pp, 2pp+1
        hi[pp] = __builtin_amdgcn_perm(od, ev, 0x07060302u);  // high halves: dim 2w+1
      }
      const int r0 = dg * 8 + 2 * wd;
      *reinterpret_cast<uint4*>(Vt + v_off(r0) + kg * 8) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      *reinterpret_cast<uint4*>(Vt + v_off(r0 + 1) + kg * 8) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    }
  };
  auto store_tile = [&](int buf) {
    bf16_t* Kt = lds + buf * kBuf;
    bf16_t* Vt = Kt + kTileK;
    if (do_k) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int id = st + 256 * i;
        *reinterpret_cast<uint4*>(Kt + (id >> 4) * kRowK + (id & 15) * 8) = pk[i];
      }
    }
    if (do_v) store_v(Vt, QG == 2 ? pv : pk);
  };
  auto entry = [&](int t) -> int { return kDense ? (t | (kModeFull << 24) | (kModeFull << 26)) : tl[t]; };

  if (ntile > 0) {
    load_tile(entry(0) & 0xffffff);
    store_tile(0);
    if (ntile > 1) load_tile(entry(1) & 0xffffff);
  }
  __syncthreads();

  for (int t = 0; t < ntile; ++t) {
    const int e = entry(t);
    const int kb = e & 0xffffff;
    const int mode = slot_on ? (e >> (24 + 2 * slot)) & 3 : 0;
    const bool diag = kb == qb;
    const bf16_t* Kt = lds + (t & 1) * kBuf;
    const bf16_t* Vt = Kt + kTileK;
    if (mode) {
      bool tile_bias = false;
      {
        const int base = (qb - kb) * B;
        for (int t2 = 0; t2 < bias.count; ++t2) {
          const int off = bias.offsets[(size_t)bh * bias.count + t2];
          tile_bias |= off > base - B && off < base + B;
        }
      }
      const bool masked = diag || mode != kModeFull || (kb + 1) * B > dm.n;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {  // 64-key halves of the tile
        f32x16 sacc[QG][2];
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2) {
#pragma unroll
          for (int qg = 0; qg < QG; ++qg)
#pragma unroll
            for (int x = 0; x < 16; ++x) sacc[qg][a2][x] = 0.0f;
          const int a = 2 * kh + a2;
#pragma unroll
          for (int kc = 0; kc < 8; ++kc) {
            const bf16x8_t A =
                as_bf16x8(*reinterpret_cast<const uint4*>(Kt + kfrag + 32 * a * kRowK + 16 * kc));
#pragma unroll
            for (int qg = 0; qg < QG; ++qg)
              sacc[qg][a2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qreg[qg][kc], sacc[qg][a2], 0, 0, 0);
          }
        }
        const bool slow = masked || tile_bias;
        unsigned pk2[QG][2][8];  // probabilities as packed bf16 pairs, per (a2, x / 2)
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          // element (a2, x) of this lane is key column c = C + 8 hl of the tile with the
          // compile-time C = 32 (2 kh + a2) + 16 (x >> 3) + (x & 7); its query row is r
          if (slow) {
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
              for (int x = 0; x < 16; ++x) sacc[qg][a2][x] *= sl2;
            int rr = r_in_blk[qg] - 8 * hl;  // r >= c  <=>  rr >= C
            // keep the per-element compares inside the loop (hoisting them costs 256 SGPRs)
            asm volatile("" : "+v"(rr));
            if (tile_bias) {
              for (int t2 = 0; t2 < bias.count; ++t2) {
                const int off = bias.offsets[(size_t)bh * bias.count + t2];
                const float bv = bias.values[(size_t)bh * bias.count + t2] * log2e;
                const int cstar = rr - (off - (qb - kb) * B);  // r - c == off  <=>  C == cstar
#pragma unroll
                for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
                  for (int x = 0; x < 16; ++x)
                    if (32 * (2 * kh + a2) + 16 * (x >> 3) + (x & 7) == cstar) sacc[qg][a2][x] += bv;
              }
            }
            if (masked) {
              const bool lower_ok = (mode & kModeLower) != 0;
              const bool upper_ok = (mode & kModeUpper) != 0 && !diag;
              const int nl = dm.n - kb * B - 8 * hl;  // key inside the sequence  <=>  C < nl
#pragma unroll
              for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                  const int C = 32 * (2 * kh + a2) + 16 * (x >> 3) + (x & 7);
                  const bool keep = (rr >= C ? lower_ok : upper_ok) && C < nl;
                  if (!keep) sacc[qg][a2][x] = -__builtin_inff();
                }
            }
          }
          // row max of this half (raw scores on the fast path: the scale is positive)
          float mx = -__builtin_inff();
#pragma unroll
          for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
            for (int x = 0; x < 16; x += 2) mx = fmaxf(mx, fmaxf(sacc[qg][a2][x], sacc[qg][a2][x + 1]));
          const float ksc = slow ? 1.0f : sl2;  // multiplier from stored scores to log2 units
          mx *= ksc;
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          // lazy rescaling: the running max moves (and O, l are rescaled) only when
          // some row of the wave grows by more than 2^8; else p = 2^(s - m_run) <= 256
          if (__any(mx > m_run[qg] + 8.0f)) {
            const float m_new = mx > m_run[qg] ? mx : m_run[qg];
            const float alpha =
                m_run[qg] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run[qg] - m_new);
            m_run[qg] = m_new;
            l_run[qg] *= alpha;
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
              for (int x = 0; x < 16; ++x) oacc[qg][t2][x] *= alpha;
          }
          const float m_use = m_run[qg] == -__builtin_inff() ? 0.0f : m_run[qg];
          float psum = l_run[qg];
#pragma unroll
          for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
            for (int x = 0; x < 16; x += 2) {
              const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qg][a2][x], ksc, -m_use));
              const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qg][a2][x + 1], ksc, -m_use));
              pk2[qg][a2][x >> 1] = pack_bf16x2(p0, p1);
              psum = sum_bf16x2(pk2[qg][a2][x >> 1], psum);
            }
          l_run[qg] = psum;
        }
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2) {
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            bf16x8_t P[QG];
#pragma unroll
            for (int qg = 0; qg < QG; ++qg)
              P[qg] = as_bf16x8(make_uint4(pk2[qg][a2][4 * s2 + 0], pk2[qg][a2][4 * s2 + 1], pk2[qg][a2][4 * s2 + 2],
                                           pk2[qg][a2][4 * s2 + 3]));
            const int a = 2 * kh + a2;
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2) {
              // V^T rows 32 t2 + ql, keys 32 a + 16 s2 + 8 hl .. + 7
              const bf16x8_t A = as_bf16x8(*reinterpret_cast<const uint4*>(
                  Vt + vfrag + t2 * (32 * kRowV + 4 * 8) + 32 * a + 16 * s2));
#pragma unroll
              for (int qg = 0; qg < QG; ++qg)
                oacc[qg][t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, P[qg], oacc[qg][t2], 0, 0, 0);
            }
          }
        }
      }
    }
    if (t + 1 < ntile) {
      store_tile((t + 1) & 1);
      if (t + 2 < ntile) load_tile(entry(t + 2) & 0xffffff);
    }
    __syncthreads();
  }

  if (!slot_on) return;
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    if (qrow[qg] >= dm.n) continue;
    const float l_tot = l_run[qg] + __shfl_xor(l_run[qg], 32);
    const float inv = 1.0f / l_tot;
    bf16_t* op = o + ((size_t)bh * dm.n + qrow[qg]) * D;
#pragma unroll
    for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int d0 = 32 * t2 + 8 * gg + 4 * hl;
        uint2 wv;
        wv.x = pack_bf16x2(oacc[qg][t2][4 * gg + 0] * inv, oacc[qg][t2][4 * gg + 1] * inv);
        wv.y = pack_bf16x2(oacc[qg][t2][4 * gg + 2] * inv, oacc[qg][t2][4 * gg + 3] * inv);
        *reinterpret_cast<uint2*>(op + d0) = wv;
      }
  }
}

// Union of the tile lists of the two query heads of a pair (same KV head,
// same query block): ascending kb, with each head's mask mode (0 = absent).
__global__ void union_tiles_kernel(Dims dm, int pairs, const int* __restrict__ tiles,
                                   const int* __restrict__ tile_cnt, int* __restrict__ ulist,
                                   int* __restrict__ ucnt) {
  const int qb = blockIdx.x * blockDim.x + threadIdx.x;
  const int item = blockIdx.y;
  if (qb >= dm.nb) return;
  const int g = item / pairs, w = item % pairs;
  const int bidx = g / dm.hkv, gh = g % dm.hkv;
  const size_t tri = (size_t)qb * (qb + 1) / 2;
  int na = 0, nbb = 0;
  const int* la = nullptr;
  const int* lb = nullptr;
  if (2 * w < dm.group) {
    const int bh = bidx * dm.hq + gh * dm.group + 2 * w;
    la = tiles + (size_t)bh * dm.ntri + tri;
    na = tile_cnt[(size_t)bh * dm.nb + qb];
  }
  if (2 * w + 1 < dm.group) {
    const int bh = bidx * dm.hq + gh * dm.group + 2 * w + 1;
    lb = tiles + (size_t)bh * dm.ntri + tri;
    nbb = tile_cnt[(size_t)bh * dm.nb + qb];
  }
  int* out = ulist + (size_t)item * dm.ntri + tri;
  int ia = 0, ib = 0, cnt = 0;
  while (ia < na || ib < nbb) {
    const int ka = ia < na ? (la[ia] & 0x0fffffff) : 0x7fffffff;
    const int kbb = ib < nbb ? (lb[ib] & 0x0fffffff) : 0x7fffffff;
    const int kk = ka < kbb ? ka : kbb;
    int e = kk;
    if (ka == kk) e |= (la[ia++] >> 28) << 24;
    if (kbb == kk) e |= (lb[ib++] >> 28) << 26;
    out[cnt++] = e;
  }
  ucnt[(size_t)item * dm.nb + qb] = cnt;
}

// ----------------------------------------------------------- vector engine --
// One thread per query row; keys staged 32 at a time through LDS in fp32.
template <typename T, int D>
__global__ __launch_bounds__(128) void attn_generic_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ v, T* __restrict__ o,
                                                           Dims dm, BiasArgs bias, const int* __restrict__ tiles,
                                                           const int* __restrict__ tile_cnt, int dense) {
  constexpr int KCH = 32;
  __shared__ float Kc[KCH * D];
  __shared__ float Vc[KCH * D];
  int qb, bh;
  work_item(dm, blockIdx.x, &qb, &bh);
  const int B = dm.B;
  const int r = threadIdx.x;
  const int i = qb * B + r;
  const int b = bh / dm.hq;
  const int kvh = b * dm.hkv + (bh % dm.hq) / dm.group;
  const T* kp = k + (size_t)kvh * dm.n * D;
  const T* vp = v + (size_t)kvh * dm.n * D;
  float qv[D], acc[D];
#pragma unroll
  for (int t = 0; t < D; ++t) {
    qv[t] = i < dm.n ? load_f32(q + ((size_t)bh * dm.n + i) * D + t) : 0.0f;
    acc[t] = 0.0f;
  }
  const float c = (float)(1.0 / __builtin_sqrt((double)D));
  float m = -__builtin_inff(), l = 0.0f;
  const int ntile = dense ? qb + 1 : tile_cnt[(size_t)bh * dm.nb + qb];
  const int* tl = dense ? nullptr : tiles + (size_t)bh * dm.ntri + (size_t)qb * (qb + 1) / 2;
  for (int t = 0; t < ntile; ++t) {
    int kb, mode;
    if (dense) {
      kb = t;
      mode = kModeFull;
    } else {
      kb = tl[t] & 0x0fffffff;
      mode = tl[t] >> 28;
    }
    const bool diag = kb == qb;
    for (int sub = 0; sub < B; sub += KCH) {
      __syncthreads();
      for (int e = threadIdx.x; e < KCH * D; e += blockDim.x) {
        const int kk = e / D, dd = e % D;
        const int key = kb * B + sub + kk;
        Kc[e] = key < dm.n ? load_f32(kp + (size_t)key * D + dd) : 0.0f;
        Vc[e] = key < dm.n ? load_f32(vp + (size_t)key * D + dd) : 0.0f;
      }
      __syncthreads();
      float s[KCH];
      float cmax = -__builtin_inff();
      for (int kk = 0; kk < KCH; ++kk) {
        const int cc = sub + kk;
        const int j = kb * B + cc;
        float dot = 0.0f;
#pragma unroll
        for (int t2 = 0; t2 < D; ++t2) dot = __builtin_fmaf(qv[t2], Kc[kk * D + t2], dot);
        float z = dot * c;
        for (int t2 = 0; t2 < bias.count; ++t2)
          if (bias.offsets[(size_t)bh * bias.count + t2] == i - j) z += bias.values[(size_t)bh * bias.count + t2];
        const bool ok = j < dm.n && j <= i && tile_keep(mode, diag, r, cc);
        s[kk] = ok ? z : -__builtin_inff();
        cmax = s[kk] > cmax ? s[kk] : cmax;
      }
      if (cmax == -__builtin_inff()) continue;
      const float m_new = cmax > m ? cmax : m;
      const float alpha = expf(m - m_new);
      l *= alpha;
#pragma unroll
      for (int t2 = 0; t2 < D; ++t2) acc[t2] *= alpha;
      for (int kk = 0; kk < KCH; ++kk) {
        const float p = expf(s[kk] - m_new);
        l += p;
#pragma unroll
        for (int t2 = 0; t2 < D; ++t2) acc[t2] = __builtin_fmaf(p, Vc[kk * D + t2], acc[t2]);
      }
      m = m_new;
    }
  }
  if (i < dm.n) {
    const float inv = 1.0f / l;
    T* op = o + ((size_t)bh * dm.n + i) * D;
#pragma unroll
    for (int t2 = 0; t2 < D; ++t2) {
      const float val = acc[t2] * inv;
      if constexpr (sizeof(T) == 4) {
        op[t2] = val;
      } else {
        unsigned u = __float_as_uint(val);
        op[t2] = (bf16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
      }
    }
  }
}

template <typename T, int D>
void launch_generic(const Dims& dm, const BiasArgs& bias, const void* q, const void* k, const void* v,
                    void* o, const int* tiles, const int* tile_cnt, hipStream_t st) {
  const int items = dm.bh * dm.nb;
  attn_generic_kernel<T, D><<<items, dm.B, 0, st>>>(static_cast<const T*>(q), static_cast<const T*>(k),
                                                   static_cast<const T*>(v), static_cast<T*>(o), dm, bias,
                                                   tiles, tile_cnt, tiles == nullptr);
}

}  // namespace

bool use_matrix_engine(const Dims& dm) { return dm.dtype == 1 && dm.d == 128 && dm.B == 128; }

hipError_t launch_build_tiles(const Dims& dm, const IndexOut& io, int* tiles, int* tile_cnt, int* ulist,
                              int* ucnt, hipStream_t st) {
  build_tiles_kernel<<<dim3((dm.nb + 127) / 128, dm.bh), 128, 0, st>>>(dm, io, tiles, tile_cnt);
  if (use_matrix_engine(dm)) {
    const int pairs = (dm.group + 1) / 2;
    union_tiles_kernel<<<dim3((dm.nb + 127) / 128, dm.bkv * pairs), 128, 0, st>>>(dm, pairs, tiles, tile_cnt,
                                                                                 ulist, ucnt);
  }
  return hipGetLastError();
}

hipError_t launch_attention(const Dims& dm, const BiasArgs& bias, const void* q, const void* k,
                            const void* v, void* o, const int* tiles, const int* tile_cnt, const int* ulist,
                            const int* ucnt, hipStream_t st) {
  if (use_matrix_engine(dm)) {
    const bf16_t* qq = static_cast<const bf16_t*>(q);
    const bf16_t* kk = static_cast<const bf16_t*>(k);
    const bf16_t* vv = static_cast<const bf16_t*>(v);
    bf16_t* oo = static_cast<bf16_t*>(o);
    const int pairs = (dm.group + 1) / 2;
    const int items = dm.bkv * pairs * dm.nb;
    constexpr int QG = CRISP_ATTN_QG;
    if (tiles == nullptr)
      attn_mfma_kernel<true, QG><<<items, 512 / QG, 0, st>>>(qq, kk, vv, oo, dm, bias, nullptr, nullptr, pairs);
    else
      attn_mfma_kernel<false, QG><<<items, 512 / QG, 0, st>>>(qq, kk, vv, oo, dm, bias, ulist, ucnt, pairs);
  } else if (dm.dtype == 1) {
    if (dm.d == 128) launch_generic<bf16_t, 128>(dm, bias, q, k, v, o, tiles, tile_cnt, st);
    else launch_generic<bf16_t, 64>(dm, bias, q, k, v, o, tiles, tile_cnt, st);
  } else {
    if (dm.d == 128) launch_generic<float, 128>(dm, bias, q, k, v, o, tiles, tile_cnt, st);
    else launch_generic<float, 64>(dm, bias, q, k, v, o, tiles, tile_cnt, st);
  }
  return hipGetLastError();
}

}  // namespace crisp
