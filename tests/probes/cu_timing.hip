// Timing probes of one CDNA4 (gfx950) compute unit (test support, not part of the
// library), each reported in shader clocks from the per-wave clock counter with
// per-workgroup windows (first wave start to last wave end), one workgroup per CU:
//   issue : two independent chains of v_mfma_f32_32x32x16_bf16 per wave with K
//           independent vector instructions (FMA, or FMA and v_exp_f32 mixed)
//           scheduled after each matrix instruction; one or two waves per SIMD;
//   chain : a chain of dependent matrix instructions (each accumulating into the
//           previous result) against independent ones;
//   lds   : ds_read_b128 throughput of 4 or 8 waves, conflict-free addresses.
// Only registers and LDS are touched in the timed loops; the output arrays are
// indexed by thread and wave inside their sizes.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <cstdio>
#include <string>
#include <vector>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int K, int MIX>
__global__ __launch_bounds__(512) void issue_probe(float* out, long long* cyc, int iters) {
  bf16x8 a, b;
  for (int i = 0; i < 8; i++) { a[i] = (__bf16)(threadIdx.x * 0.001f); b[i] = (__bf16)(i * 0.01f); }
  f32x16 acc0 = {}, acc1 = {};
  float x[16];
  for (int j = 0; j < 16; j++) x[j] = -(float)(threadIdx.x + j) * 1e-3f;
  const float y = 0.999f, z = -0.001f;
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < K; j++) {
      float& v = x[j % 16];
      if (MIX && (j & 1)) v = __builtin_amdgcn_exp2f(v);
      else v = __builtin_fmaf(v, y, z);
    }
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc1, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < K; j++) {
      float& v = x[(j + 8) % 16];
      if (MIX && (j & 1)) v = __builtin_amdgcn_exp2f(v);
      else v = __builtin_fmaf(v, y, z);
    }
    if constexpr (K > 0) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, K, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, K, 0);
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int j = 0; j < 16; j++) s += acc0[j] + acc1[j] + x[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) {
    const int w = (blockIdx.x * blockDim.x + threadIdx.x) / 64;
    cyc[2 * w] = t0;
    cyc[2 * w + 1] = t1;
  }
}

template <int CHAINS>
__global__ __launch_bounds__(512) void chain_probe(float* out, long long* cyc, int iters) {
  bf16x8 a, b;
  for (int i = 0; i < 8; i++) { a[i] = (__bf16)(threadIdx.x * 0.001f); b[i] = (__bf16)(i * 0.01f); }
  f32x16 acc[CHAINS];
  for (int c = 0; c < CHAINS; ++c) acc[c] = f32x16{};
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int r = 0; r < 8 / CHAINS; ++r)
#pragma unroll
      for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  const long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int c = 0; c < CHAINS; ++c)
    for (int j = 0; j < 16; j++) s += acc[c][j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) {
    const int w = (blockIdx.x * blockDim.x + threadIdx.x) / 64;
    cyc[2 * w] = t0;
    cyc[2 * w + 1] = t1;
  }
}

__global__ __launch_bounds__(512) void lds_probe(float* out, long long* cyc, int iters) {
  __shared__ __align__(16) unsigned char lds[65536];
  for (int i = threadIdx.x; i < 65536 / 16; i += blockDim.x) reinterpret_cast<u32x4*>(lds)[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  typedef const __attribute__((address_space(3))) u32x4 lds_u4;
  lds_u4* base = (lds_u4*)(lds + ((lane * 16 + wave * 4096) & 65535));
  u32x4 acc = {0, 0, 0, 0};
  __syncthreads();
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = base[((it * 8 + j) * 64) & 4095];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j];
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc.x ^ acc.y ^ acc.z ^ acc.w);
  if (lane == 0) {
    const int w = (blockIdx.x * blockDim.x + threadIdx.x) / 64;
    cyc[2 * w] = t0;
    cyc[2 * w + 1] = t1;
  }
}

namespace {
const int kGrid = 256;
float* g_out;
long long* g_cyc;

// mean over workgroups of (last end - first start) of their waves
double window(int threads) {
  const int wpb = threads / 64;
  std::vector<long long> h(2 * kGrid * wpb);
  (void)hipMemcpy(h.data(), g_cyc, h.size() * sizeof(long long), hipMemcpyDeviceToHost);
  double win = 0;
  for (int g = 0; g < kGrid; ++g) {
    long long lo = h[2 * g * wpb], hi = h[2 * g * wpb + 1];
    for (int w = 0; w < wpb; ++w) {
      lo = std::min(lo, h[2 * (g * wpb + w)]);
      hi = std::max(hi, h[2 * (g * wpb + w) + 1]);
    }
    win += hi - lo;
  }
  return win / kGrid;
}

template <typename F>
double timed(F launch, int threads) {
  for (int rep = 0; rep < 2; ++rep) {
    launch();
    (void)hipDeviceSynchronize();
  }
  return window(threads);
}
}  // namespace

extern "C" int crisp_probe_cu_timing(char* report, size_t cap) {
  if (hipMalloc(&g_out, kGrid * 512 * sizeof(float)) != hipSuccess) return -1;
  if (hipMalloc(&g_cyc, kGrid * 16 * sizeof(long long)) != hipSuccess) return -1;
  std::string out;
  char line[160];
  const int iters = 2048;
  for (int th : {256, 512}) {
    const double mf = 2.0 * iters * (th / 256);  // matrix instructions per SIMD
#define ISSUE(K, MIX)                                                                                         \
  {                                                                                                          \
    const double w = timed([&] { issue_probe<K, MIX><<<kGrid, th>>>(g_out, g_cyc, iters); }, th);            \
    snprintf(line, sizeof line, "issue waves_per_simd %d valu_per_mfma %d mix_exp %d clocks_per_mfma %.1f\n", \
             th / 256, K, MIX, w / mf);                                                                      \
    out += line;                                                                                             \
  }
    ISSUE(0, 0) ISSUE(2, 0) ISSUE(4, 0) ISSUE(6, 0) ISSUE(8, 0) ISSUE(4, 1) ISSUE(6, 1)
#undef ISSUE
    const double mc = 8.0 * iters * (th / 256);
    {
      const double w = timed([&] { chain_probe<1><<<kGrid, th>>>(g_out, g_cyc, iters); }, th);
      snprintf(line, sizeof line, "chain waves_per_simd %d chains 1 clocks_per_mfma %.1f\n", th / 256, w / mc);
      out += line;
    }
    {
      const double w = timed([&] { chain_probe<4><<<kGrid, th>>>(g_out, g_cyc, iters); }, th);
      snprintf(line, sizeof line, "chain waves_per_simd %d chains 4 clocks_per_mfma %.1f\n", th / 256, w / mc);
      out += line;
    }
    {
      const double w = timed([&] { lds_probe<<<kGrid, th>>>(g_out, g_cyc, iters); }, th);
      snprintf(line, sizeof line, "lds waves_per_cu %d bytes_per_clock %.1f\n", th / 64, (th / 64) * iters * 8.0 * 1024 / w);
      out += line;
    }
  }
  (void)hipFree(g_out);
  (void)hipFree(g_cyc);
  snprintf(report, cap, "%s", out.c_str());
  return hipDeviceSynchronize() == hipSuccess && out.size() < cap ? 0 : 1;
}
