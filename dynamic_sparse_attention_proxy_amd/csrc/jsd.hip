// Jensen-Shannon divergence router: the routing signal that C_struct replaces
// (CRISP summary page, Motivation and Key Contributions), built on the same
// proxy so the two routers can be compared decision by decision and timed.
//
//   per-query estimate  P_b = p^v_b / T: the column block masses of the proxy
//                       map (softmax per query first, then pooled; crisp_route)
//   pooled estimate     Q_b: pool first (block mean of the last query block
//                       against the block means of every key block), one row
//                       of scores, softmax in the fixed point of the pooled
//                       estimation path (Alg. 4)
//   divergence          JSD = (KL(P||M) + KL(Q||M)) / 2, M = (P + Q) / 2;
//                       VS iff JSD >= tau_jsd
// Three kernels: jsd_pool (block means), jsd_scores (one pooled row per head),
// jsd_finish (softmax, divergence terms, routing decision).  Every sum that
// feeds the decision is an int64 sum (block masses at 2^40, divergence terms
// at 2^52), so the result does not depend on the order of the reduction.
#include "common.h"
#include "kernels.h"

namespace crisp {

namespace {

constexpr int kJsdShift = 52;  // divergence terms: rne(t 2^52); JSD = J 2^-53

// Block means, sequential fp32 sums over rows in ascending order, then one
// division by the row count.  Unit u < bh: the last query block of query head
// u; otherwise key block (u - bh) % nb of KV head (u - bh) / nb.  A thread owns
// eight columns of one unit, so one row of a unit is read as d / 8 16-byte
// (bf16) or 32-byte (fp32) pieces by neighbouring lanes.
template <typename T>
__global__ __launch_bounds__(256) void jsd_pool_kernel(Dims dm, const T* __restrict__ q,
                                                       const T* __restrict__ k, float* __restrict__ qbar,
                                                       float* __restrict__ kbar) {
  const int tpu = dm.d / 8;  // threads per unit
  const long long units = (long long)dm.bh + (long long)dm.bkv * dm.nb;
  const long long u = (long long)blockIdx.x * (256 / tpu) + threadIdx.x / tpu;
  if (u >= units) return;
  const int c0 = (threadIdx.x % tpu) * 8;
  const T* src;
  float* dst;
  int r0, cnt;
  if (u < dm.bh) {
    src = q + (size_t)u * dm.n * dm.d;
    dst = qbar + (size_t)u * dm.d;
    r0 = dm.q0;
    cnt = dm.qrows;
  } else {
    const long long v = u - dm.bh;
    const int kvh = (int)(v / dm.nb), b = (int)(v % dm.nb);
    src = k + (size_t)kvh * dm.n * dm.d;
    dst = kbar + ((size_t)kvh * dm.nb + b) * dm.d;
    r0 = b * dm.B;
    cnt = min(dm.B, dm.n - r0);
  }
  float out[8];
  mean8(src + (size_t)r0 * dm.d + c0, dm.d, cnt, out);
  float4* o4 = reinterpret_cast<float4*>(dst + c0);
  o4[0] = make_float4(out[0], out[1], out[2], out[3]);
  o4[1] = make_float4(out[4], out[5], out[6], out[7]);
}

// One pooled row per query head: z_b = fl(fma-chain(Qbar, Kbar_b) c) over the
// head dimension in ascending order, for every key block b.
template <int D>
__global__ __launch_bounds__(256) void jsd_scores_kernel(Dims dm, const float* __restrict__ qbar,
                                                         const float* __restrict__ kbar,
                                                         float* __restrict__ zbar) {
  __shared__ __align__(16) float qs[D];
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int kvh = (bh / dm.hq) * dm.hkv + (bh % dm.hq) / dm.group;
  for (int i = tid; i < D; i += 256) qs[i] = qbar[(size_t)bh * D + i];
  __syncthreads();
  const int b = blockIdx.x * 256 + tid;
  if (b >= dm.nb) return;
  const float4* kr = reinterpret_cast<const float4*>(kbar + ((size_t)kvh * dm.nb + b) * D);
  float acc = 0.0f;
#pragma unroll 8
  for (int i = 0; i < D / 4; ++i) {
    const float4 kv = kr[i];
    acc = __builtin_fmaf(qs[4 * i], kv.x, acc);
    acc = __builtin_fmaf(qs[4 * i + 1], kv.y, acc);
    acc = __builtin_fmaf(qs[4 * i + 2], kv.z, acc);
    acc = __builtin_fmaf(qs[4 * i + 3], kv.w, acc);
  }
  const float c = (float)(1.0 / __builtin_sqrt((double)D));
  zbar[(size_t)bh * dm.nb + b] = acc * c;
}

// ln x for positive normal x in fp64: x = 2^e m with m in (sqrt(1/2), sqrt(2)],
// ln m = 2 atanh(s), s = (m - 1) / (m + 1), by the odd series to s^23 in Horner
// form in s^2, plus e ln2 with ln2 as a 32-bit head and a tail.
__device__ __forceinline__ double log_crisp(double x) {
  const double sqrt2 = 0x1.6a09e667f3bcdp+0;
  const double ln2_hi = 0x1.62e42ff000000p-1;
  const double ln2_lo = -0x1.718432a1b0e26p-35;
  unsigned long long bits = (unsigned long long)__double_as_longlong(x);
  int e = (int)((bits >> 52) & 0x7ff) - 1023;
  bits = (bits & 0x000fffffffffffffULL) | 0x3ff0000000000000ULL;
  double m = __longlong_as_double((long long)bits);
  if (m > sqrt2) {
    m = m * 0.5;
    e += 1;
  }
  const double s = (m - 1.0) / (m + 1.0);
  const double s2 = s * s;
  double p = 1.0 / 23.0;
  p = __builtin_fma(p, s2, 1.0 / 21.0);
  p = __builtin_fma(p, s2, 1.0 / 19.0);
  p = __builtin_fma(p, s2, 1.0 / 17.0);
  p = __builtin_fma(p, s2, 1.0 / 15.0);
  p = __builtin_fma(p, s2, 1.0 / 13.0);
  p = __builtin_fma(p, s2, 1.0 / 11.0);
  p = __builtin_fma(p, s2, 1.0 / 9.0);
  p = __builtin_fma(p, s2, 1.0 / 7.0);
  p = __builtin_fma(p, s2, 1.0 / 5.0);
  p = __builtin_fma(p, s2, 1.0 / 3.0);
  p = __builtin_fma(p, s2, 1.0);
  const double lm = (2.0 * s) * p;
  const double r = __builtin_fma((double)e, ln2_lo, lm);
  return __builtin_fma((double)e, ln2_hi, r);
}

constexpr int kFinThreads = 1024;

// Softmax of the pooled row in fixed point, the divergence from p^v / T and
// the routing decision; one workgroup per query head.
__global__ __launch_bounds__(kFinThreads) void jsd_finish_kernel(Dims dm, unsigned tau_num, unsigned tau_den,
                                                                 const float* __restrict__ zbar,
                                                                 const long long* __restrict__ mass_v,
                                                                 const long long* __restrict__ mass_total,
                                                                 long long* __restrict__ abar,
                                                                 long long* __restrict__ pooled,
                                                                 uint8_t* __restrict__ route_jsd,
                                                                 long long* __restrict__ jsd) {
  __shared__ float redf[kFinThreads / 64];
  __shared__ long long redi[kFinThreads / 64];
  const int bh = blockIdx.x, tid = threadIdx.x, nb = dm.nb;
  const float* z = zbar + (size_t)bh * nb;
  long long* a = abar + (size_t)bh * nb;
  float m = -__builtin_inff();
  for (int b = tid; b < nb; b += kFinThreads) m = z[b] > m ? z[b] : m;
  m = block_max_f32(m, redf);
  long long L = 0;
  for (int b = tid; b < nb; b += kFinThreads) L += fix_rne(exp_crisp(z[b] - m));
  L = block_sum_i64(L, redi);
  const float l = fix_to_float(L);
  long long ta = 0;
  for (int b = tid; b < nb; b += kFinThreads) {
    const long long aq = fix_rne(exp_crisp(z[b] - m) / l);
    a[b] = aq;
    if (pooled) pooled[(size_t)bh * nb + b] = aq;
    ta += aq;
  }
  ta = block_sum_i64(ta, redi);  // the barrier inside also orders the writes of a[] before the reads below
  const double dT = (double)mass_total[bh], dTa = (double)ta;
  const long long* pv = mass_v + (size_t)bh * nb;
  long long J = 0;
  for (int b = tid; b < nb; b += kFinThreads) {
    const double P = (double)pv[b] / dT;
    const double Q = (double)a[b] / dTa;
    const double M = 0.5 * (P + Q);
    const double tp = P > 0.0 ? P * log_crisp(P / M) : 0.0;
    const double tq = Q > 0.0 ? Q * log_crisp(Q / M) : 0.0;
    const double t = tp + tq;
    J += (long long)__builtin_rint(__builtin_ldexp(t, kJsdShift));
  }
  J = block_sum_i64(J, redi);
  if (tid == 0) {
    jsd[bh] = J;
    // JSD = J 2^-53 >= tau_num / tau_den, as integers
    const __int128 lhs = (__int128)tau_den * (__int128)J;
    const __int128 rhs = (__int128)tau_num << (kJsdShift + 1);
    route_jsd[bh] = lhs >= rhs ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_route_jsd(const Dims& dm, unsigned tau_num, unsigned tau_den, const void* q, const void* k,
                            const JsdScratch& ws, const long long* mass_v, const long long* mass_total,
                            uint8_t* route_jsd, long long* jsd, long long* pooled, hipStream_t st) {
  const int upb = 256 / (dm.d / 8);
  const long long units = (long long)dm.bh + (long long)dm.bkv * dm.nb;
  const unsigned grid = (unsigned)((units + upb - 1) / upb);
  if (dm.dtype == 1)
    jsd_pool_kernel<bf16_t><<<grid, 256, 0, st>>>(dm, static_cast<const bf16_t*>(q),
                                                  static_cast<const bf16_t*>(k), ws.qbar, ws.kbar);
  else
    jsd_pool_kernel<float><<<grid, 256, 0, st>>>(dm, static_cast<const float*>(q), static_cast<const float*>(k),
                                                 ws.qbar, ws.kbar);
  const dim3 sg((dm.nb + 255) / 256, dm.bh);
  if (dm.d == 128)
    jsd_scores_kernel<128><<<sg, 256, 0, st>>>(dm, ws.qbar, ws.kbar, ws.zbar);
  else
    jsd_scores_kernel<64><<<sg, 256, 0, st>>>(dm, ws.qbar, ws.kbar, ws.zbar);
  jsd_finish_kernel<<<dm.bh, kFinThreads, 0, st>>>(dm, tau_num, tau_den, ws.zbar, mass_v, mass_total, ws.abar,
                                                   pooled, route_jsd, jsd);
  return hipGetLastError();
}

}  // namespace crisp
