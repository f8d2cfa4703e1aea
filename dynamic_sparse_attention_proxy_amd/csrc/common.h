// Device-side helpers shared by the CRISP HIP kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace crisp {

constexpr int kFixShift = 40;  // fixed-point scale 2^40 for every decision sum

typedef unsigned short bf16_t;  // storage of bfloat16 values

struct bf16x8 {
  uint4 v;
};

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

template <typename T>
__device__ __forceinline__ float load_f32(const T* p);
template <>
__device__ __forceinline__ float load_f32<float>(const float* p) {
  return *p;
}
template <>
__device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p) {
  return bf16_to_f32(*p);
}

// Eight consecutive columns of one row as fp32 (16-byte aligned source).
__device__ __forceinline__ void load8(const bf16_t* p, float* x) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* x) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w;
  x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
}

// Column means of cnt consecutive rows (row stride d): eight columns starting at
// p, each an fp32 sum over the rows in ascending order, then one division by
// the row count.
template <typename T>
__device__ __forceinline__ void mean8(const T* p, int d, int cnt, float* out) {
  float s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = 0.0f;
  int r = 0;
  // eight rows' loads in flight before their (sequential) sums
  for (; r + 8 <= cnt; r += 8) {
    float x[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) load8(p + (size_t)(r + j) * d, x[j]);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = s[i] + x[j][i];
  }
  for (; r < cnt; ++r) {
    float x[8];
    load8(p + (size_t)r * d, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = s[i] + x[i];
  }
  const float fc = (float)cnt;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = s[i] / fc;
}

// e^x for x <= 0 in fp32, bit-identical by construction to the reference
// definition: Cody-Waite reduction x = k ln2 + r (k = rint(x log2 e), ln2 in a
// 15-bit head and a tail), Taylor polynomial of degree 7 in Horner form with
// coefficients 1/j! rounded to fp32, result p 2^k; 0 below -80.
__device__ __forceinline__ float exp_crisp(float x) {
  if (x < -80.0f) return 0.0f;
  const float log2e = 1.44269502f;         // 0x3FB8AA3B
  const float ln2_hi = 0.693145751953125f; // 0x3F317200
  const float ln2_lo = 1.42860677e-06f;    // 0x35BFBE8E
  float t = x * log2e;
  float kf = __builtin_rintf(t);
  float r = __builtin_fmaf(-kf, ln2_hi, x);
  r = __builtin_fmaf(-kf, ln2_lo, r);
  float p = 1.0f / 5040.0f;
  p = __builtin_fmaf(p, r, 1.0f / 720.0f);
  p = __builtin_fmaf(p, r, 1.0f / 120.0f);
  p = __builtin_fmaf(p, r, 1.0f / 24.0f);
  p = __builtin_fmaf(p, r, 1.0f / 6.0f);
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, (int)kf);
}

// rne(v * 2^40) for 0 <= v <= 1: exact scaling, round half to even, exact conversion.
__device__ __forceinline__ long long fix_rne(float v) {
  return (long long)__builtin_rintf(__builtin_ldexpf(v, kFixShift));
}

// The same value as an integer-valued fp32 (<= 2^40): sums of up to 2^13 such
// terms are exact in fp64, which is cheaper to accumulate than int64.
__device__ __forceinline__ float fix_rne_f(float v) {
  return __builtin_rintf(__builtin_ldexpf(v, kFixShift));
}

// e / l rounded to nearest even, from r = 1 / l (itself an IEEE division, once per
// row): q0 = e r is within about an ulp of the quotient, the remainder e - q0 l is
// exact in one fma, and q0 + rem r, rounded once, is the correctly rounded quotient
// (the correction step of Markstein's FMA division, IBM J. Res. Dev. 34, 1990).
// Three instructions instead of an IEEE division's ten.  For e in [0, 1] and
// l >= 1 it gives the same bits as e / l whenever the quotient is a normal
// number, checked exhaustively over e for sampled l, on random pairs and on
// quotients next to rounding midpoints (tests/test_quotient.py); below 2^-126
// its last bits may differ, and every caller scales the quotient by 2^40 and
// rounds it to an integer, which is 0 there either way.
__device__ __forceinline__ float quot_rn(float e, float l, float r) {
  const float q0 = e * r;
  const float rem = __builtin_fmaf(-q0, l, e);
  return __builtin_fmaf(rem, r, q0);
}

// fl32(L) * 2^-40 (int64 -> fp32 rounds to nearest even).
__device__ __forceinline__ float fix_to_float(long long L) {
  return __builtin_ldexpf((float)L, -kFixShift);
}

// Order-preserving map of fp32 onto int32 (for atomicMax of floats).
__device__ __forceinline__ int float_to_ordered(float f) {
  int b = __float_as_int(f);
  return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float ordered_to_float(int o) {
  return __int_as_float(o ^ ((o >> 31) & 0x7fffffff));
}

// A 64-bit value moved across lanes by one DPP pattern (both halves with the same
// control; lanes the pattern or the row mask does not feed read 0).
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ long long dpp_i64(long long v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(v & 0xffffffff), kCtrl, kRowMask, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(v >> 32), kCtrl, kRowMask, 0xf, true);
  return ((long long)hi << 32) | (unsigned int)lo;
}

// Sum over the 64 lanes of a wave (all lanes active), returned in every lane.
// Integer addition is exact, so the order is free: DPP row shifts by 1, 2, 4, 8
// leave each 16-lane row's sum in its lane 15; row broadcast 15 adds row 0 into
// row 1 and row 2 into row 3, row broadcast 31 adds lane 31 into rows 2 and 3;
// lane 63 then holds the total, which readlane hands to the whole wave.
__device__ __forceinline__ long long wave_sum_i64(long long v) {
  v += dpp_i64<0x111>(v);        // row_shr:1
  v += dpp_i64<0x112>(v);        // row_shr:2
  v += dpp_i64<0x114>(v);        // row_shr:4
  v += dpp_i64<0x118>(v);        // row_shr:8
  v += dpp_i64<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_i64<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  const int lo = __builtin_amdgcn_readlane((int)(v & 0xffffffff), 63);
  const int hi = __builtin_amdgcn_readlane((int)(v >> 32), 63);
  return ((long long)hi << 32) | (unsigned int)lo;
}

// Sum / max over one workgroup (every thread gets the result); red holds one
// slot per wave.  The trailing barrier lets the caller reuse red at once.
__device__ __forceinline__ long long block_sum_i64(long long v, long long* red) {
  v = wave_sum_i64(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  long long s = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += red[w];
  __syncthreads();
  return s;
}

__device__ __forceinline__ float block_max_f32(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    float o = __shfl_xor(v, m);
    v = o > v ? o : v;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = red[w] > r ? red[w] : r;
  __syncthreads();
  return r;
}

// Ascending compaction of flags over one block of threads.  Returns the
// position of this thread's element (valid if flag) and the block total.
__device__ __forceinline__ int block_compact(bool flag, int* wave_cnt, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const unsigned long long mask = __ballot(flag);
  const int before = __popcll(mask & ((1ull << lane) - 1ull));
  __syncthreads();
  if (lane == 0) wave_cnt[wave] = __popcll(mask);
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    if (w < wave) off += wave_cnt[w];
    tot += wave_cnt[w];
  }
  *total = tot;
  return off + before;
}

}  // namespace crisp
