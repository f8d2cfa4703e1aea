// Proxy map, block masses and C_struct routing (CRISP summary page,
// Methodology: Eq. 2 and Alg. 2; the column / diagonal block pooling of Alg. 3).
//
// Four streaming kernels over the proxy scores of the last query block:
//   proxy_scores : z = fl(fma-chain(q, k) * c) (+ bias) on the fp32 vector ALU,
//                  written tile-contiguous; row max by ordered-int atomicMax
//   proxy_rowsum : L_i = sum_j rne(exp_crisp(z - m_i) 2^40)  (int64 atomics)
//   proxy_mass   : A = fl(e / l_i), A_q = rne(A 2^40); per key block the
//                  vertical mass, the two slash-block parts and the anchor mass
//   route_finish : assemble mass_v / mass_s / total, C_struct test
// Every sum that feeds a decision is an int64 fixed-point sum, so the result
// does not depend on the order in which blocks or threads add.
#include "common.h"
#include "kernels.h"

namespace crisp {

namespace {

constexpr int kThreads = 256;

__global__ void route_init_kernel(int* m_enc, long long* L, int total) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < total) {
    m_enc[t] = float_to_ordered(-__builtin_inff());
    L[t] = 0;
  }
}

// Proxy scores of one (head, key block) tile: B query rows x B keys.
// Each thread owns a TM x TM register tile (rows ty*TM.., keys tx*TM..); every
// accumulator runs its own fma chain over the head dimension in ascending
// order, chunked through LDS.
template <typename T, int B, int D>
__global__ __launch_bounds__(kThreads) void proxy_scores_kernel(const T* __restrict__ q,
                                                                const T* __restrict__ k, Dims dm,
                                                                BiasArgs bias, float* __restrict__ S,
                                                                int* __restrict__ m_enc) {
  constexpr int TM = B / 16;
  constexpr int KC = 32;
  constexpr int LD = B + 4;
  __shared__ __align__(16) float Qs[KC * LD];
  __shared__ __align__(16) float Ks[KC * LD];
  __shared__ float red[4][B];

  const int kb = blockIdx.x;
  const int bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int ty = tid & 15;
  const int tx = tid >> 4;
  const int b = bh / dm.hq;
  const int kvh = b * dm.hkv + (bh % dm.hq) / dm.group;
  const T* qbase = q + ((size_t)bh * dm.n + dm.q0) * D;
  const T* kbase = k + ((size_t)kvh * dm.n + (size_t)kb * B) * D;
  const int krows = min(B, dm.n - kb * B);

  float acc[TM][TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = 0.0f;

  // Staging: a 32-dim chunk of Q and K is B x 4 pieces of 8 dims; piece g has
  // row g % B and dims 8 (g / B) ..; it is read with one 16-byte (bf16) load,
  // held in registers while the previous chunk is computed, and stored
  // transposed (dim-major) so that the lanes of a wave write consecutive rows.
  constexpr int kPieces = B * KC / 8 / kThreads;  // pieces per thread and operand
  float qv[kPieces][8], kv[kPieces][8];
  auto fetch = [&](int dc) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int g = tid + kThreads * i, r = g % B, d8 = (g / B) * 8;
      if (r < dm.qrows) load8(qbase + (size_t)r * D + dc + d8, qv[i]);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) qv[i][j] = 0.0f;
      if (r < krows) load8(kbase + (size_t)r * D + dc + d8, kv[i]);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) kv[i][j] = 0.0f;
    }
  };
  fetch(0);
  for (int dc = 0; dc < D; dc += KC) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int g = tid + kThreads * i, r = g % B, d8 = (g / B) * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        Qs[(d8 + j) * LD + r] = qv[i][j];
        Ks[(d8 + j) * LD + r] = kv[i][j];
      }
    }
    __syncthreads();
    if (dc + KC < D) fetch(dc + KC);
#pragma unroll 4
    for (int kk = 0; kk < KC; ++kk) {
      float a[TM], bb[TM];
#pragma unroll
      for (int i = 0; i < TM; i += 4) {
        float4 va = *reinterpret_cast<const float4*>(&Qs[kk * LD + ty * TM + i]);
        float4 vb = *reinterpret_cast<const float4*>(&Ks[kk * LD + tx * TM + i]);
        a[i] = va.x, a[i + 1] = va.y, a[i + 2] = va.z, a[i + 3] = va.w;
        bb[i] = vb.x, bb[i + 1] = vb.y, bb[i + 2] = vb.z, bb[i + 3] = vb.w;
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = __builtin_fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }

  // scale, bias, causal validity; write the tile [key c][row r]
  const float c = (float)(1.0 / __builtin_sqrt((double)D));
  const long long tile_off = ((long long)bh * dm.nb + kb) * (long long)(B * B);
  // bias can only touch this tile if some offset lies in its diagonal range
  const int omin = dm.q0 - kb * B - (B - 1), omax = dm.q0 + (B - 1) - kb * B;
  bool tile_bias = false;
  for (int t = 0; t < bias.count; ++t) {
    const int o = bias.offsets[(size_t)bh * bias.count + t];
    tile_bias |= o >= omin && o <= omax;
  }
  float rmax[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) rmax[i] = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int cc = tx * TM + j;
    const int jj = kb * B + cc;
    float out[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = ty * TM + i;
      const int ii = dm.q0 + r;
      float z = acc[i][j] * c;
      if (tile_bias)
        for (int t = 0; t < bias.count; ++t)
          if (bias.offsets[(size_t)bh * bias.count + t] == ii - jj) z = z + bias.values[(size_t)bh * bias.count + t];
      const bool valid = (r < dm.qrows) && (jj <= ii);
      out[i] = valid ? z : -__builtin_inff();
      if (valid && z > rmax[i]) rmax[i] = z;
    }
    float* dst = S + tile_off + (size_t)cc * B + ty * TM;
#pragma unroll
    for (int i = 0; i < TM; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(out[i], out[i + 1], out[i + 2], out[i + 3]);
  }
  // row max: across tx within the wave (lanes ty, ty+16, ty+32, ty+48), then across waves
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float v = rmax[i];
    float o = __shfl_xor(v, 16);
    v = o > v ? o : v;
    o = __shfl_xor(v, 32);
    v = o > v ? o : v;
    rmax[i] = v;
  }
  const int wave = tid >> 6;
  if ((tid & 63) < 16) {
#pragma unroll
    for (int i = 0; i < TM; ++i) red[wave][ty * TM + i] = rmax[i];
  }
  __syncthreads();
  if (tid < B && tid < dm.qrows) {
    float v = red[0][tid];
    for (int w = 1; w < 4; ++w) v = red[w][tid] > v ? red[w][tid] : v;
    if (v != -__builtin_inff()) atomicMax(&m_enc[bh * B + tid], float_to_ordered(v));
  }
}

// Thread layout of the streaming passes over one (head, key block) tile stored
// [key c][row r]: each thread owns 4 consecutive rows and visits keys
// c = cp, cp + CP, ... ; float4 loads are contiguous across the row groups.
constexpr int kRowsumTiles = 4;  // key blocks per workgroup of proxy_rowsum_kernel

template <int B>
struct StreamLayout {
  static constexpr int RG = B / 4;
  static constexpr int CP = kThreads / RG;
  static constexpr int IT = B / CP;
};

template <int B>
__global__ __launch_bounds__(kThreads) void proxy_rowsum_kernel(Dims dm, const float* __restrict__ S,
                                                                const int* __restrict__ m_enc,
                                                                long long* __restrict__ L) {
  using Lay = StreamLayout<B>;
  __shared__ long long red[Lay::CP][B];
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int rg = tid % Lay::RG, cp = tid / Lay::RG;
  float m[4];
  long long acc[4] = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < 4; ++e) m[e] = ordered_to_float(m_enc[bh * B + rg * 4 + e]);
  // kRowsumTiles consecutive key blocks per workgroup; full tiles accumulate
  // integer-valued terms in fp64 (at most kRowsumTiles * IT terms of <= 2^40
  // each, exact)
  double accd[4] = {0.0, 0.0, 0.0, 0.0};
  const int kb0 = blockIdx.x * kRowsumTiles, kb1 = min(kb0 + kRowsumTiles, dm.nb);
  for (int kb = kb0; kb < kb1; ++kb) {
    const long long tile_off = ((long long)bh * dm.nb + kb) * (long long)(B * B);
    if (kb < dm.nb - 1 && dm.qrows == B) {
#pragma unroll 4
      for (int it = 0; it < Lay::IT; ++it) {
        const int c = cp + Lay::CP * it;
        const float4 z4 = *reinterpret_cast<const float4*>(S + tile_off + (size_t)c * B + rg * 4);
        const float z[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) accd[e] += (double)fix_rne_f(exp_crisp(z[e] - m[e]));
      }
    } else {
#pragma unroll 4
      for (int it = 0; it < Lay::IT; ++it) {
        const int c = cp + Lay::CP * it;
        const int jj = kb * B + c;
        const float4 z4 = *reinterpret_cast<const float4*>(S + tile_off + (size_t)c * B + rg * 4);
        const float z[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = rg * 4 + e;
          if (r < dm.qrows && jj <= dm.q0 + r) acc[e] += fix_rne(exp_crisp(z[e] - m[e]));
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) red[cp][rg * 4 + e] = acc[e] + (long long)accd[e];
  __syncthreads();
  if (tid < B && tid < dm.qrows) {
    long long s = 0;
    for (int p = 0; p < Lay::CP; ++p) s += red[p][tid];
    if (s) atomicAdd(reinterpret_cast<unsigned long long*>(&L[bh * B + tid]), (unsigned long long)s);
  }
}

template <int B>
__global__ __launch_bounds__(kThreads) void proxy_mass_kernel(Dims dm, RouteArgs ra,
                                                              const float* __restrict__ S,
                                                              const int* __restrict__ m_enc,
                                                              const long long* __restrict__ L,
                                                              long long* __restrict__ part) {
  using Lay = StreamLayout<B>;
  __shared__ long long red[3][4];
  const int kb = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int rg = tid % Lay::RG, cp = tid / Lay::RG;
  const long long tile_off = ((long long)bh * dm.nb + kb) * (long long)(B * B);
  float m[4], l[4], rl[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m[e] = ordered_to_float(m_enc[bh * B + rg * 4 + e]);
    l[e] = fix_to_float(L[bh * B + rg * 4 + e]);
    rl[e] = 1.0f / l[e];
  }
  long long lo = 0, up = 0, an = 0;
  const bool plain = kb < dm.nb - 1 && dm.qrows == B && kb * B >= ra.w_sink &&
                     dm.q0 - (kb * B + B - 1) >= ra.w_local;
  if (plain) {
    // every (row, key) is valid and none is an anchor: integer-valued terms summed
    // in fp64 (at most 4 IT terms of <= 2^40 each, exact); upper = all - lower
    double alld = 0.0, lod = 0.0;
#pragma unroll 8
    for (int it = 0; it < Lay::IT; ++it) {
      const int c = cp + Lay::CP * it;
      const float4 z4 = *reinterpret_cast<const float4*>(S + tile_off + (size_t)c * B + rg * 4);
      const float z[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double aq = (double)fix_rne_f(quot_rn(exp_crisp(z[e] - m[e]), l[e], rl[e]));
        alld += aq;
        lod += rg * 4 + e >= c ? aq : 0.0;
      }
    }
    lo = (long long)lod;
    up = (long long)alld - lo;
  } else
#pragma unroll 4
  for (int it = 0; it < Lay::IT; ++it) {
    const int c = cp + Lay::CP * it;
    const int jj = kb * B + c;
    const float4 z4 = *reinterpret_cast<const float4*>(S + tile_off + (size_t)c * B + rg * 4);
    const float z[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = rg * 4 + e;
      const int ii = dm.q0 + r;
      if (r < dm.qrows && jj <= ii) {
        const float ev = exp_crisp(z[e] - m[e]);
        const long long aq = fix_rne(quot_rn(ev, l[e], rl[e]));
        // slash block (i - j) / B is (nb - 1 - kb) when r >= c, one less when r < c
        if (r >= c)
          lo += aq;
        else
          up += aq;
        if (jj < ra.w_sink || ii - jj < ra.w_local) an += aq;
      }
    }
  }
  lo = wave_sum_i64(lo);
  up = wave_sum_i64(up);
  an = wave_sum_i64(an);
  const int wave = tid >> 6;
  if ((tid & 63) == 0) {
    red[0][wave] = lo;
    red[1][wave] = up;
    red[2][wave] = an;
  }
  __syncthreads();
  if (tid == 0) {
    long long s0 = 0, s1 = 0, s2 = 0;
    for (int w = 0; w < 4; ++w) s0 += red[0][w], s1 += red[1][w], s2 += red[2][w];
    const size_t stride = (size_t)dm.bh * dm.nb;
    const size_t at = (size_t)bh * dm.nb + kb;
    part[at] = s0 + s1;
    part[stride + at] = s0;
    part[2 * stride + at] = s1;
    part[3 * stride + at] = s2;
  }
}

__global__ __launch_bounds__(kThreads) void route_finish_kernel(Dims dm, RouteArgs ra,
                                                                const long long* __restrict__ part,
                                                                IndexOut io) {
  __shared__ long long red[16];
  const int bh = blockIdx.x, tid = threadIdx.x, nb = dm.nb;
  const size_t stride = (size_t)dm.bh * nb;
  const long long* pv = part + (size_t)bh * nb;
  const long long* plo = part + stride + (size_t)bh * nb;
  const long long* pup = part + 2 * stride + (size_t)bh * nb;
  const long long* pan = part + 3 * stride + (size_t)bh * nb;
  long long T = 0, cn = 0;
  for (int b = tid; b < nb; b += kThreads) {
    T += pv[b];
    cn += pan[b];
    io.mass_v[(size_t)bh * nb + b] = pv[b];
    // slash block s collects the lower part of key block nb-1-s and the upper part of nb-2-s
    long long s = plo[nb - 1 - b];
    if (b <= nb - 2) s += pup[nb - 2 - b];
    io.mass_s[(size_t)bh * nb + b] = s;
  }
  T = block_sum_i64(T, red);
  cn = block_sum_i64(cn, red + 8);
  if (tid == 0) {
    io.mass_total[bh] = T;
    io.cstruct_num[bh] = cn;
    // C_struct = cn / (qrows 2^40) >= tau_num / tau_den, as integers
    const unsigned __int128 lhs = (unsigned __int128)ra.tau_den * (unsigned __int128)cn;
    const unsigned __int128 rhs =
        ((unsigned __int128)ra.tau_num * (unsigned __int128)dm.qrows) << kFixShift;
    io.route[bh] = lhs >= rhs ? 1 : 0;
  }
}

template <typename T, int B, int D>
void launch_scores(const Dims& dm, const BiasArgs& bias, const void* q, const void* k, float* S,
                   int* m_enc, hipStream_t st) {
  proxy_scores_kernel<T, B, D><<<dim3(dm.nb, dm.bh), kThreads, 0, st>>>(
      static_cast<const T*>(q), static_cast<const T*>(k), dm, bias, S, m_enc);
}

}  // namespace

hipError_t launch_route(const Dims& dm, const RouteArgs& ra, const BiasArgs& bias, const void* q,
                        const void* k, const RouteScratch& ws, const IndexOut& io, hipStream_t st) {
  const int rows = dm.bh * dm.B;
  route_init_kernel<<<(rows + 255) / 256, 256, 0, st>>>(ws.m_enc, ws.L, rows);
#define CRISP_SCORES(T, BB, DD) launch_scores<T, BB, DD>(dm, bias, q, k, ws.S, ws.m_enc, st)
  if (dm.dtype == 1) {
    if (dm.B == 128 && dm.d == 128) CRISP_SCORES(bf16_t, 128, 128);
    else if (dm.B == 128) CRISP_SCORES(bf16_t, 128, 64);
    else if (dm.d == 128) CRISP_SCORES(bf16_t, 64, 128);
    else CRISP_SCORES(bf16_t, 64, 64);
  } else {
    if (dm.B == 128 && dm.d == 128) CRISP_SCORES(float, 128, 128);
    else if (dm.B == 128) CRISP_SCORES(float, 128, 64);
    else if (dm.d == 128) CRISP_SCORES(float, 64, 128);
    else CRISP_SCORES(float, 64, 64);
  }
#undef CRISP_SCORES
  if (dm.B == 128) {
    proxy_rowsum_kernel<128><<<dim3((dm.nb + kRowsumTiles - 1) / kRowsumTiles, dm.bh), kThreads, 0, st>>>(
        dm, ws.S, ws.m_enc, ws.L);
    proxy_mass_kernel<128><<<dim3(dm.nb, dm.bh), kThreads, 0, st>>>(dm, ra, ws.S, ws.m_enc, ws.L, ws.part);
  } else {
    proxy_rowsum_kernel<64><<<dim3((dm.nb + kRowsumTiles - 1) / kRowsumTiles, dm.bh), kThreads, 0, st>>>(
        dm, ws.S, ws.m_enc, ws.L);
    proxy_mass_kernel<64><<<dim3(dm.nb, dm.bh), kThreads, 0, st>>>(dm, ra, ws.S, ws.m_enc, ws.L, ws.part);
  }
  route_finish_kernel<<<dm.bh, kThreads, 0, st>>>(dm, ra, ws.part, io);
  return hipGetLastError();
}

}  // namespace crisp
