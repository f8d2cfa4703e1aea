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

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  // round to nearest even (finite inputs)
  unsigned a = __float_as_uint(lo), b = __float_as_uint(hi);
  a = (a + 0x7fffu + ((a >> 16) & 1u)) >> 16;
  b = (b + 0x7fffu + ((b >> 16) & 1u)) & 0xffff0000u;
  return a | b;
}

// key row inside a 32-key group that feeds matrix row rho (swap of bits 2 and 3)
__device__ __forceinline__ int key_perm(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

template <bool kDense>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(const bf16_t* __restrict__ q,
                                                           const bf16_t* __restrict__ k,
                                                           const bf16_t* __restrict__ v,
                                                           bf16_t* __restrict__ o, Dims dm, BiasArgs bias,
                                                           const int* __restrict__ tiles,
                                                           const int* __restrict__ tile_cnt) {
  constexpr int B = 128, D = 128, LDK = D + 8;
  __shared__ __align__(16) bf16_t Ks[B * LDK];  // [key][d]
  __shared__ __align__(16) bf16_t Vt[D * LDK];  // [d][key]

  int qb, bh;
  work_item(dm, blockIdx.x, &qb, &bh);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  const int b = bh / dm.hq;
  const int kvh = b * dm.hkv + (bh % dm.hq) / dm.group;
  const bf16_t* qp = q + (size_t)bh * dm.n * D;
  const bf16_t* kp = k + (size_t)kvh * dm.n * D;
  const bf16_t* vp = v + (size_t)kvh * dm.n * D;
  const int r_in_blk = wave * 32 + ql;
  const int qrow = qb * B + r_in_blk;

  bf16x8_t qreg[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qrow < dm.n) u = *reinterpret_cast<const uint4*>(qp + (size_t)qrow * D + 16 * kc + 8 * hl);
    qreg[kc] = as_bf16x8(u);
  }

  f32x16 oacc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[t][e] = 0.0f;
  float m_run = -__builtin_inff(), l_run = 0.0f;
  const float log2e = 1.4426950408889634f;
  const float sl2 = (float)(1.0 / __builtin_sqrt(128.0)) * log2e;

  const int ntile = kDense ? qb + 1 : tile_cnt[(size_t)bh * dm.nb + qb];
  const int* tl = kDense ? nullptr : tiles + (size_t)bh * dm.ntri + (size_t)qb * (qb + 1) / 2;
  const int kg = tid >> 4, dg = tid & 15;  // V staging: keys 8kg.., d 8dg..
  const int prow = key_perm(ql);

  for (int t = 0; t < ntile; ++t) {
    int kb, mode;
    if (kDense) {
      kb = t;
      mode = kModeFull;
    } else {
      const int e = tl[t];
      kb = e & 0x0fffffff;
      mode = e >> 28;
    }
    const bool diag = kb == qb;
    __syncthreads();
    // stage K (row-major) and V (transposed) for keys kb*B .. kb*B + 127
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = tid + 256 * i;
      const int row = id >> 4, cc = id & 15;
      const int key = kb * B + row;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (key < dm.n) val = *reinterpret_cast<const uint4*>(kp + (size_t)key * D + cc * 8);
      *reinterpret_cast<uint4*>(Ks + row * LDK + cc * 8) = val;
    }
    {
      uint4 vv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kb * B + kg * 8 + e;
        vv[e] = make_uint4(0, 0, 0, 0);
        if (key < dm.n) vv[e] = *reinterpret_cast<const uint4*>(vp + (size_t)key * D + dg * 8);
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        unsigned lo[4], hi[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const unsigned ev = (&vv[2 * p].x)[w], od = (&vv[2 * p + 1].x)[w];
          lo[p] = (ev & 0xffffu) | (od << 16);
          hi[p] = (ev >> 16) | (od & 0xffff0000u);
        }
        *reinterpret_cast<uint4*>(Vt + (dg * 8 + 2 * w) * LDK + kg * 8) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        *reinterpret_cast<uint4*>(Vt + (dg * 8 + 2 * w + 1) * LDK + kg * 8) =
            make_uint4(hi[0], hi[1], hi[2], hi[3]);
      }
    }
    __syncthreads();

    // S^T = K Q^T for the 128 keys of the tile, 4 groups of 32
    f32x16 sacc[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[a][e] = 0.0f;
      const bf16_t* krow = Ks + (32 * a + prow) * LDK + 8 * hl;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const bf16x8_t A = as_bf16x8(*reinterpret_cast<const uint4*>(krow + 16 * kc));
        sacc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qreg[kc], sacc[a], 0, 0, 0);
      }
    }

    // logits in log2 units, bias, masks
    bool tile_bias = false;
    {
      const int base = (qb - kb) * B;
      for (int t2 = 0; t2 < bias.count; ++t2) {
        const int off = bias.offsets[(size_t)bh * bias.count + t2];
        tile_bias |= off > base - B && off < base + B;
      }
    }
    const bool masked = diag || mode != kModeFull || (kb + 1) * B > dm.n;
    float mx = -__builtin_inff();
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = 32 * a + 16 * (e >> 3) + 8 * hl + (e & 7);
        float s = sacc[a][e] * sl2;
        if (tile_bias) {
          const int off = (qb - kb) * B + r_in_blk - c;
          for (int t2 = 0; t2 < bias.count; ++t2)
            if (bias.offsets[(size_t)bh * bias.count + t2] == off)
              s += bias.values[(size_t)bh * bias.count + t2] * log2e;
        }
        if (masked && !(tile_keep(mode, diag, r_in_blk, c) && kb * B + c < dm.n)) s = -__builtin_inff();
        sacc[a][e] = s;
        mx = s > mx ? s : mx;
      }
    }
    {
      const float ot = __shfl_xor(mx, 32);
      mx = ot > mx ? ot : mx;
    }
    const float m_new = mx > m_run ? mx : m_run;
    const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.0f;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(sacc[a][e] - m_use);
        sacc[a][e] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[t2][e] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        uint4 pu;
        pu.x = pack_bf16x2(sacc[a][8 * s2 + 0], sacc[a][8 * s2 + 1]);
        pu.y = pack_bf16x2(sacc[a][8 * s2 + 2], sacc[a][8 * s2 + 3]);
        pu.z = pack_bf16x2(sacc[a][8 * s2 + 4], sacc[a][8 * s2 + 5]);
        pu.w = pack_bf16x2(sacc[a][8 * s2 + 6], sacc[a][8 * s2 + 7]);
        const bf16x8_t P = as_bf16x8(pu);
#pragma unroll
        for (int t2 = 0; t2 < 4; ++t2) {
          const bf16x8_t A = as_bf16x8(
              *reinterpret_cast<const uint4*>(Vt + (32 * t2 + ql) * LDK + 32 * a + 16 * s2 + 8 * hl));
          oacc[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, P, oacc[t2], 0, 0, 0);
        }
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (qrow < dm.n) {
    bf16_t* op = o + ((size_t)bh * dm.n + qrow) * D;
#pragma unroll
    for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * t2 + 8 * g + 4 * hl;
        uint2 w;
        w.x = pack_bf16x2(oacc[t2][4 * g + 0] * inv, oacc[t2][4 * g + 1] * inv);
        w.y = pack_bf16x2(oacc[t2][4 * g + 2] * inv, oacc[t2][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(op + d0) = w;
      }
  }
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

hipError_t launch_build_tiles(const Dims& dm, const IndexOut& io, int* tiles, int* tile_cnt,
                              hipStream_t st) {
  build_tiles_kernel<<<dim3((dm.nb + 127) / 128, dm.bh), 128, 0, st>>>(dm, io, tiles, tile_cnt);
  return hipGetLastError();
}

hipError_t launch_attention(const Dims& dm, const BiasArgs& bias, const void* q, const void* k,
                            const void* v, void* o, const int* tiles, const int* tile_cnt,
                            hipStream_t st) {
  const int items = dm.bh * dm.nb;
  if (dm.dtype == 1 && dm.d == 128 && dm.B == 128) {
    const bf16_t* qq = static_cast<const bf16_t*>(q);
    const bf16_t* kk = static_cast<const bf16_t*>(k);
    const bf16_t* vv = static_cast<const bf16_t*>(v);
    bf16_t* oo = static_cast<bf16_t*>(o);
    if (tiles == nullptr)
      attn_mfma_kernel<true><<<items, 256, 0, st>>>(qq, kk, vv, oo, dm, bias, nullptr, nullptr);
    else
      attn_mfma_kernel<false><<<items, 256, 0, st>>>(qq, kk, vv, oo, dm, bias, tiles, tile_cnt);
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
