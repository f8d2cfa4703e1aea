// Black-box probe of the numerics of the bf16 matrix instruction
// v_mfma_f32_32x32x16_bf16 (test support, not part of the library): D = C + A B for
// many 32x32x16 blocks with seeded inputs of six kinds (Gaussian like the proxy's
// inputs, a wide exponent spread, cancelling product pairs, C much larger or much
// smaller than the products, C = 0).  The host compares every output bit for bit with
// candidate models of the accumulation, each computed exactly in int128 fixed point
// and rounded as the model says.  It reads outputs only.  A bit-exact proxy score on
// the matrix cores needs a model that matches every output; the report says whether
// one does.  Every device index stays inside the arrays it addresses: problem p reads
// A[p], B[p], C[p] and writes D[p].
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <cmath>
#include <vector>
#include <random>
#include <string>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// layout probe + compute: lane l holds A[l%32][8(l/32)+e], B[8(l/32)+e][l%32]; C/D in the
// accumulator layout, written back per (lane, x)
__global__ void mfma_blocks(const uint16_t* A, const uint16_t* B, const float* C, float* D, int np) {
  const int p = blockIdx.x;
  if (p >= np) return;
  const int l = threadIdx.x;
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    const int k = 8 * (l / 32) + e;
    uint16_t av = A[(size_t)p * 512 + (l % 32) * 16 + k];
    uint16_t bv = B[(size_t)p * 512 + k * 32 + (l % 32)];
    a[e] = __builtin_bit_cast(__bf16, av);
    b[e] = __builtin_bit_cast(__bf16, bv);
  }
  f32x16 acc;
  for (int x = 0; x < 16; ++x) acc[x] = C[(size_t)p * 1024 + l * 16 + x];
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  for (int x = 0; x < 16; ++x) D[(size_t)p * 1024 + l * 16 + x] = acc[x];
}

static float bf2f(uint16_t h) { uint32_t u = (uint32_t)h << 16; float f; memcpy(&f, &u, 4); return f; }
static uint16_t f2bf(float f) { uint32_t u; memcpy(&u, &f, 4); u += 0x7fff + ((u >> 16) & 1); return (uint16_t)(u >> 16); }
static uint32_t fbits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

// exact value as int128 at scale 2^-S
const int S = 90;
// double -> int128 at scale 2^S exactly (v must be a multiple of 2^-S)
static __int128 to_fix(double v) {
  int ex;
  double m = std::frexp(v, &ex);  // v = m 2^ex, 0.5 <= |m| < 1
  long long mi = (long long)std::ldexp(m, 53);  // exact
  int sh = ex - 53 + S;
  __int128 r = (__int128)mi;
  if (sh >= 0) r <<= sh; else r >>= -sh;  // inputs chosen so no bits are lost
  return r;
}
// round int128 at scale 2^-S to fp32 with round-to-nearest-even (or toward zero)
static float fix_to_f32(__int128 x, bool rz = false) {
  if (x == 0) return 0.0f;
  bool neg = x < 0;
  unsigned __int128 ux = neg ? (unsigned __int128)(-x) : (unsigned __int128)x;
  int msb = 127;
  while (!((ux >> msb) & 1)) --msb;
  int drop = msb - 23;  // keep 24 bits
  unsigned __int128 q = drop > 0 ? ux >> drop : ux << (-drop);
  if (drop > 0 && !rz) {
    unsigned __int128 rem = ux & (((unsigned __int128)1 << drop) - 1);
    unsigned __int128 half = (unsigned __int128)1 << (drop - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    if (q >> 24) { q >>= 1; ++drop; }
  }
  double v = std::ldexp((double)(uint64_t)q, drop - S);
  return neg ? -(float)v : (float)v;
}

extern "C" int crisp_probe_mfma_numerics(char* report, size_t cap) {
  std::string out;
  char line[256];
  const int np = 6144;
  std::mt19937_64 rng(12345);
  std::uniform_real_distribution<double> U(0, 1);
  std::normal_distribution<double> N(0, 1);
  std::vector<uint16_t> A(np * 512), B(np * 512);
  std::vector<float> C(np * 1024), D(np * 1024);
  // kinds: 0 Gaussian like the proxy inputs (C from a previous chunk), 1 wide exponent
  // spread, 2 cancellation (products in +- pairs of nearly equal size), 3 large C vs small
  // products, 4 small C vs large products, 5 C = 0
  auto gen_bf = [&](int kind) -> uint16_t {
    double v;
    if (kind == 0) v = N(rng) / std::sqrt(128.0) * (U(rng) < 0.1 ? 8.0 : 1.0);
    else if (kind == 1 || kind == 2) v = std::ldexp(1.0 + U(rng), (int)(U(rng) * 24) - 12) * (U(rng) < 0.5 ? -1 : 1);
    else v = N(rng);
    return f2bf((float)v);
  };
  for (int p = 0; p < np; ++p) {
    const int kind = p % 6;
    for (int i = 0; i < 512; ++i) A[(size_t)p * 512 + i] = gen_bf(kind), B[(size_t)p * 512 + i] = gen_bf(kind);
    if (kind == 2)  // make k = 2m+1 products cancel k = 2m ones in every row / column
      for (int r = 0; r < 32; ++r)
        for (int k = 1; k < 16; k += 2) {
          A[(size_t)p * 512 + r * 16 + k] = A[(size_t)p * 512 + r * 16 + k - 1] ^ 0x8000;
          B[(size_t)p * 512 + k * 32 + r] = B[(size_t)p * 512 + (k - 1) * 32 + r] ^ (U(rng) < 0.5 ? 0x0001 : 0x0000);
        }
    for (int i = 0; i < 1024; ++i) {
      double c;
      if (kind == 3) c = std::ldexp(1.0 + U(rng), 12) * (U(rng) < 0.5 ? -1 : 1);
      else if (kind == 4) c = std::ldexp(1.0 + U(rng), -14) * (U(rng) < 0.5 ? -1 : 1);
      else if (kind == 5) c = 0.0;
      else c = N(rng) * (kind == 1 ? 16.0 : 0.5);
      C[(size_t)p * 1024 + i] = (float)c;
    }
  }
  uint16_t *dA, *dB;
  float *dC, *dD;
  (void)hipMalloc(&dA, A.size() * 2); (void)hipMalloc(&dB, B.size() * 2);
  (void)hipMalloc(&dC, C.size() * 4); (void)hipMalloc(&dD, D.size() * 4);
  (void)hipMemcpy(dA, A.data(), A.size() * 2, hipMemcpyHostToDevice);
  (void)hipMemcpy(dB, B.data(), B.size() * 2, hipMemcpyHostToDevice);
  // layout discovery: C = 0, A[i][0] = i + 1, B[0][j] = 1 (others 0) gives D[i][j] = i + 1
  {
    std::vector<uint16_t> a(512, 0), b(512, 0);
    std::vector<float> c(1024, 0.0f), d(1024);
    for (int i = 0; i < 32; ++i) a[i * 16 + 0] = f2bf((float)(i + 1));
    for (int j = 0; j < 32; ++j) b[0 * 32 + j] = f2bf(1.0f);
    (void)hipMemcpy(dA, a.data(), 1024, hipMemcpyHostToDevice);
    (void)hipMemcpy(dB, b.data(), 1024, hipMemcpyHostToDevice);
    (void)hipMemcpy(dC, c.data(), 4096, hipMemcpyHostToDevice);
    mfma_blocks<<<1, 64>>>(dA, dB, dC, dD, 1);
    (void)hipMemcpy(d.data(), dD, 4096, hipMemcpyDeviceToHost);
    out += "layout lane 0 rows:";
    for (int x = 0; x < 16; ++x) { snprintf(line, sizeof line, " %g", d[x] - 1); out += line; }
    out += "\nlayout lane 32 rows:";
    for (int x = 0; x < 16; ++x) { snprintf(line, sizeof line, " %g", d[32 * 16 + x] - 1); out += line; }
    out += "\n";
    (void)hipMemcpy(dA, A.data(), A.size() * 2, hipMemcpyHostToDevice);
    (void)hipMemcpy(dB, B.data(), B.size() * 2, hipMemcpyHostToDevice);
  }
  // row of output (lane l, element x), column l % 32: discovered above; assume the usual
  // 32x32 accumulator layout and check it against the discovery
  auto row_of = [](int l, int x) { return 8 * (x / 4) + 4 * (l / 32) + (x % 4); };
  (void)hipMemcpy(dC, C.data(), C.size() * 4, hipMemcpyHostToDevice);
  mfma_blocks<<<np, 64>>>(dA, dB, dC, dD, np);
  (void)hipMemcpy(D.data(), dD, D.size() * 4, hipMemcpyDeviceToHost);
  const char* names[] = {"exact dot + C, one RNE", "RNE(exact dot) + C, RNE", "sequential fp32 adds k=0..15",
                         "exact dot + C, truncate", "pairwise fp32 tree, then + C"};
  const int NM = 5;
  long long match[6][NM] = {}, total[6] = {};
  long long maxulp[6][NM] = {};
  for (int p = 0; p < np; ++p) {
    const int kind = p % 6;
    for (int l = 0; l < 64; ++l)
      for (int x = 0; x < 16; ++x) {
        const int i = row_of(l, x), j = l % 32;
        const float c = C[(size_t)p * 1024 + l * 16 + x];
        double prod[16];
        __int128 sum = 0;
        for (int k = 0; k < 16; ++k) {
          prod[k] = (double)bf2f(A[(size_t)p * 512 + i * 16 + k]) * (double)bf2f(B[(size_t)p * 512 + k * 32 + j]);
          sum += to_fix(prod[k]);
        }
        float m[NM];
        m[0] = fix_to_f32(sum + to_fix((double)c));
        m[1] = (float)((double)fix_to_f32(sum) + (double)c);
        { float acc = c; for (int k = 0; k < 16; ++k) acc = acc + (float)prod[k]; m[2] = acc; }
        m[3] = fix_to_f32(sum + to_fix((double)c), true);
        { float t[16]; for (int k = 0; k < 16; ++k) t[k] = (float)prod[k];
          for (int w = 8; w >= 1; w >>= 1) for (int k = 0; k < w; ++k) t[k] = t[k] + t[k + w];
          m[4] = t[0] + c; }
        const float g = D[(size_t)p * 1024 + l * 16 + x];
        ++total[kind];
        for (int q = 0; q < NM; ++q) {
          if (fbits(m[q]) == fbits(g)) ++match[kind][q];
          long long du = std::llabs((long long)(int32_t)fbits(m[q]) - (long long)(int32_t)fbits(g));
          if (du > maxulp[kind][q]) maxulp[kind][q] = du;
        }
      }
  }
  const char* kinds[] = {"gaussian", "wide exponents", "cancellation", "large C", "small C", "C = 0"};
  for (int kind = 0; kind < 6; ++kind) {
    snprintf(line, sizeof line, "kind %s outputs %lld\n", kinds[kind], total[kind]);
    out += line;
    for (int q = 0; q < NM; ++q) {
      snprintf(line, sizeof line, "  model %d %s | match %.6f | max ulp diff %lld\n", q, names[q],
               (double)match[kind][q] / total[kind], maxulp[kind][q]);
      out += line;
    }
  }
  (void)hipFree(dA);
  (void)hipFree(dB);
  (void)hipFree(dC);
  (void)hipFree(dD);
  if (hipDeviceSynchronize() != hipSuccess) return -1;
  snprintf(report, cap, "%s", out.c_str());
  return out.size() < cap ? 0 : 1;
}
