// Sparse and dense causal prefill attention (CRISP summary page, "Algorithm
// Overview", Alg. 1: attention over the selected index set).
//
// The key tiles of a (head, query block qb) -- key block kb and a mask mode --
// come from the index sets (sparse) or are 0..qb (dense):
//   VS head : kb in V (whole tile), kb = qb - s for s in S (lower triangle
//             r >= c of the tile: offsets in block s), kb = qb - s - 1
//             (upper triangle r < c: the same offset block from the tile
//             below the diagonal); a selected slash block is the band of
//             diagonals [sB, sB + B).
//   PE head : the CSR row of query block qb.
//   Every tile is intersected with causality (diagonal tile: r >= c).
//
// bf16, d = 128, B = 128: matrix-core engine (attn_mfma_kernel).  A persistent
// workgroup per CU takes work items (KV head, pair of its query heads, query
// block) from per-XCD queues; its 8 waves each own 32 query rows of one of the
// two heads, so every K / V^T tile brought into LDS serves 256 query rows.
// S^T = K Q^T is computed with v_mfma_f32_32x32x16_bf16 so that a lane holds
// one query's scores (the softmax needs one cross-half exchange at most), and
// the probabilities are already laid out as the B operand of O^T = V^T P^T
// (the key order inside each 32-key group is permuted on the K side to make
// that layout line up).  V^T is written to the workspace once per call, so
// both tiles reach LDS by direct global-to-LDS loads and every LDS read that
// feeds a matrix instruction is one 16-byte vector.
// Other shapes (fp32, d = 64, B = 64): attn_generic_kernel, one thread per
// query row on the fp32 vector ALU, same tile lists and masks.
#include <type_traits>

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
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

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

// max / sum over the two 32-lane halves of the wave (v_permlane32_swap exchanges them)
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// key row inside a 32-key group that feeds matrix row rho (swap of bits 2 and 3)
__device__ __forceinline__ int key_perm(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes lds_base + 16 i.  Written as inline assembly so that the compiler does
// not treat the asynchronous LDS write as aliasing the LDS reads of the tile
// being computed (it would wait for the prefetch before every read); the
// kernel itself waits for completion (vmcnt) and synchronises (s_barrier)
// before a tile is read.  base and lds_base are uniform over the wave.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// lds_wave + kBufImm addresses the slot: lds_wave is a per-wave scalar, the
// constant part is encoded in the instruction stream.  The LDS destination goes
// through m0; nothing else in these kernels uses m0 (checked in the generated
// code), so the compiler's treatment of m0 as reserved does not matter here.  A
// scalar write of m0 needs one wait state before an LDS DMA reads it (the
// compiler keeps that distance for its own DMA instructions but cannot see inside
// an asm block), hence the s_nop.
template <unsigned kLdsConst>
__device__ __forceinline__ void dma16(const unsigned char* base, unsigned voff, unsigned lds_wave) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds_wave), "n"(kLdsConst)
               : "memory", "m0");
}
// the same with a per-lane 64-bit address
template <unsigned kLdsConst>
__device__ __forceinline__ void dma16_lane(const unsigned char* addr, unsigned lds_wave) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(addr), "s"(lds_wave), "n"(kLdsConst)
               : "memory", "m0");
}

// keeps a value materialised at this point (no sinking past later branches)
__device__ __forceinline__ void pin(unsigned x) { asm volatile("" ::"v"(x)); }

// 16-byte LDS reads through address-space-3 pointers: a per-lane base pointer plus a
// constant element offset folds into the instruction's offset field
typedef const __attribute__((address_space(3))) u32x4_t lds_u4;
__device__ __forceinline__ lds_u4* lds_u4_ptr(const void* p) { return (lds_u4*)p; }

// Work items of the matrix engine are (KV head g, pair w of its query heads,
// query block qb).  The combos c = g * pairs + w are split into 8 contiguous
// runs, one per XCD queue, so that the workgroups of an XCD share the K/V
// stream of one KV head in that XCD's L2.  A queue lists its items by query
// block, heaviest first.  A workgroup takes items from the queue of its own XCD
// and, once that is empty, from the others (load balance between cheap and
// expensive heads).
// Queue i owns combos combos * i / 8 .. combos * (i + 1) / 8 - 1.
__device__ __forceinline__ int queue_begin(int combos, int i) { return (int)((long long)combos * i / 8); }

// LDS tiles are 128 rows of 256 bytes; the sixteen 16-byte chunks of a row are
// stored XOR-swizzled so that the 16 lanes of a matrix-operand read (16
// different rows, one chunk column) hit 16 different chunk positions:
//   K tile   : row = key, chunk c (8 dims)    stored at c ^ key_perm(row & 15)
//   V^T tile : row = dim, chunk c (8 keys)    stored at c ^ (row & 15)
// Tiles are written by direct global-to-LDS loads: one wave instruction fills
// 4 rows (1 KiB), lane i writing slot (i & 15) of row i >> 4, so the swizzle is
// applied by choosing which global chunk each lane fetches.
constexpr int kTileBytes = 128 * 256;

// Matrix engine.  A workgroup of 8 waves serves 256 query rows that share every
// K/V tile: the two query heads of a pair x the 128 rows of query block qb;
// wave w owns 32 rows of head w / 4 (two waves per SIMD).  A 128-key tile is
// processed in four 32-key quarters: the softmax of quarter a runs on the
// vector ALU while the matrix core computes the scores of quarter a + 1 and the
// P V product of quarter a - 1.  Scores are computed transposed, S^T = K Q^T, so
// a lane holds one query's scores; O^T = V^T P^T takes the probabilities
// straight from registers.  K and V^T tiles are double-buffered in LDS: tile
// t + 1 is in flight while tile t is computed.
template <bool kDense>
__global__ __launch_bounds__(512, 1) void attn_mfma_kernel(const bf16_t* __restrict__ q,
                                                           const bf16_t* __restrict__ k,
                                                           const bf16_t* __restrict__ vt,
                                                           bf16_t* __restrict__ o, Dims dm, BiasArgs bias,
                                                           const int* __restrict__ ulist,
                                                           const int* __restrict__ ucnt, int pairs, int npad,
                                                           int* __restrict__ counters) {
  constexpr int B = 128, D = 128;
  // four tile buffers: K of even / odd tiles, then V^T of even / odd tiles
  __shared__ __align__(1024) unsigned char smem[4 * kTileBytes];
  __shared__ int s_item;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps wave-level addresses scalar
  const int slot = wave >> 2;
  const int hl = lane >> 5, ql = lane & 31, l15 = lane & 15;
  const float log2e = 1.4426950408889634f;
  const float sl2 = (float)(1.0 / __builtin_sqrt(128.0)) * log2e;
  const int r_in_blk = (wave & 3) * 32 + ql;

  // per-lane byte offsets of the matrix operands inside a tile
  // (LDS byte addresses in the first buffer of each kind; the other buffer and the
  // 32-row groups are constant offsets)
  lds_u4* koff[8];
  lds_u4* voff[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) koff[kc] = lds_u4_ptr(smem) + key_perm(ql) * 16 + ((2 * kc + hl) ^ l15);
#pragma unroll
  for (int j = 0; j < 8; ++j)  // j = 2 a + s2
    voff[j] = lds_u4_ptr(smem + 2 * kTileBytes) + ql * 16 + ((2 * j + hl) ^ l15);
  // per-lane source offsets of the direct loads: instruction i of the wave fills
  // rows 4 m .. 4 m + 3 of a tile, m = 4 wave + i
  unsigned dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 4 * i + (lane >> 4);
    const unsigned m = 4 * wave + i;
    dk[i] = m * 1024 + (lane >> 4) * 256 + (((lane & 15) ^ key_perm(rr)) << 4);
    dv[i] = m * 4 * npad * 2 + (lane >> 4) * npad * 2 + (((lane & 15) ^ rr) << 4);
  }
  const unsigned lds_wave = __builtin_amdgcn_readfirstlane(lds_addr(smem) + wave * 4096);
  const int xcd = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 7;  // hardware XCC id (4 bits)
  int ones_bits;  // (1, 1) in bf16, in a scalar register for the row-sum dot products
  asm volatile("s_mov_b32 %0, 0x3f803f80" : "=s"(ones_bits));
  const int combos = dm.bkv * pairs;

  for (;;) {
    // next item: own queue first, then the others in turn
    if (tid == 0) {
      int it = -1;
      for (int k2 = 0; k2 < 8 && it < 0; ++k2) {
        const int qi = (xcd + k2) & 7;
        const int n_items = (queue_begin(combos, qi + 1) - queue_begin(combos, qi)) * dm.nb;
        if (n_items == 0 || __hip_atomic_load(&counters[qi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n_items)
          continue;
        const int v = atomicAdd(&counters[qi], 1);
        if (v < n_items) it = (qi << 24) | v;
      }
      s_item = it;
    }
    __syncthreads();
    const int it = __builtin_amdgcn_readfirstlane(s_item);
    __syncthreads();
    if (it < 0) break;
    const int qi = it >> 24, v = it & 0xffffff;
    const int c0 = queue_begin(combos, qi), ncomb = queue_begin(combos, qi + 1) - c0;
    const int comb = c0 + v % ncomb;
    const int qb = dm.nb - 1 - v / ncomb, g = comb / pairs, w = comb % pairs;

    const int bidx = g / dm.hkv, gh = g % dm.hkv;
    const int hin = 2 * w + slot;
    const bool slot_on = hin < dm.group;
    const int bh = bidx * dm.hq + gh * dm.group + (slot_on ? hin : 0);
    const bf16_t* qp = q + (size_t)bh * dm.n * D;
    const unsigned char* kp = reinterpret_cast<const unsigned char*>(k + (size_t)g * dm.n * D);
    const unsigned char* vp = reinterpret_cast<const unsigned char*>(vt + (size_t)g * D * npad);
    const int qrow = qb * B + r_in_blk;

    bf16x8_t qreg[8];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (slot_on && qrow < dm.n) u = *reinterpret_cast<const uint4*>(qp + (size_t)qrow * D + 16 * kc + 8 * hl);
      qreg[kc] = as_bf16x8(u);
    }
    f32x16 oacc[4];
#pragma unroll
    for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[t2][e] = 0.0f;
    float m_run = -__builtin_inff(), l_run = 0.0f;

    // this head's relative-position bias (at most 8 offsets)
    int boff[8];
    float bval[8];
#pragma unroll
    for (int t2 = 0; t2 < 8; ++t2) {
      boff[t2] = t2 < bias.count ? __builtin_amdgcn_readfirstlane(bias.offsets[(size_t)bh * bias.count + t2]) : -1;
      bval[t2] = t2 < bias.count ? bias.values[(size_t)bh * bias.count + t2] * log2e : 0.0f;
    }

    int bias_dmax = -1;  // largest query-block minus key-block distance a bias offset reaches
#pragma unroll
    for (int t2 = 0; t2 < 8; ++t2)
      if (boff[t2] >= 0) bias_dmax = max(bias_dmax, (boff[t2] + B - 1) / B);

    const int item = g * pairs + w;
    const int ntile = kDense ? qb + 1 : ucnt[(size_t)item * dm.nb + qb];
    const int* tl = kDense ? nullptr : ulist + (size_t)item * dm.ntri + (size_t)qb * (qb + 1) / 2;
    // Sparse lists are read 64 entries at a time into a register (lane i holds entry
    // 64 c + i) and taken out with readlane: no scalar load, whose latency the wave
    // would wait out after every barrier.  The chunk after the current one is loaded
    // when the current one is entered, 64 tiles before it is needed.
    int chunk_cur = 0, chunk_nxt = 0;
    auto load_chunk = [&](int c) -> int {
      const int i = 64 * c + lane;
      return i < ntile ? tl[i] : 0;
    };
    if (!kDense) {
      chunk_cur = load_chunk(0);
      chunk_nxt = load_chunk(1);
    }
    auto entry = [&](int t) -> int {
      if constexpr (kDense) return t | (kModeFull << 24) | (kModeFull << 26);
      else return __builtin_amdgcn_readlane(chunk_cur, t & 63);
    };
    // called once per tile with the next tile's index, after the barrier (every
    // earlier load of this wave has completed there)
    auto advance = [&](int t) {
      if constexpr (!kDense) {
        if ((t & 63) == 0 && t > 0) {
          chunk_cur = chunk_nxt;
          chunk_nxt = load_chunk((t >> 6) + 1);
        }
      }
    };

    // K tile -> buffer KI, V^T tile -> buffer 2 + KI (KI a compile-time 0 / 1)
    auto load_tile = [&](int kb, auto KI) {
      constexpr unsigned kK = decltype(KI)::value * kTileBytes, kV = (2 + decltype(KI)::value) * kTileBytes;
      const unsigned char* kt = kp + (size_t)kb * B * 256;
      const unsigned char* vtile = vp + (size_t)kb * 256;
      if ((kb + 1) * B <= dm.n) {
        dma16<kK + 0 * 1024>(kt, dk[0], lds_wave);
        dma16<kK + 1 * 1024>(kt, dk[1], lds_wave);
        dma16<kK + 2 * 1024>(kt, dk[2], lds_wave);
        dma16<kK + 3 * 1024>(kt, dk[3], lds_wave);
      } else {  // ragged last tile: rows past the end re-read the last key (their scores are masked)
        const unsigned char* a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * (4 * wave + i) + (lane >> 4);
          const int key = min(kb * B + r, dm.n - 1);
          a[i] = kp + (size_t)key * 256 + (((lane & 15) ^ key_perm(r & 15)) << 4);
        }
        dma16_lane<kK + 0 * 1024>(a[0], lds_wave);
        dma16_lane<kK + 1 * 1024>(a[1], lds_wave);
        dma16_lane<kK + 2 * 1024>(a[2], lds_wave);
        dma16_lane<kK + 3 * 1024>(a[3], lds_wave);
      }
      dma16<kV + 0 * 1024>(vtile, dv[0], lds_wave);
      dma16<kV + 1 * 1024>(vtile, dv[1], lds_wave);
      dma16<kV + 2 * 1024>(vtile, dv[2], lds_wave);
      dma16<kV + 3 * 1024>(vtile, dv[3], lds_wave);
    };

    int e_next = 0;  // the entry of the tile the next step computes

    // One tile: wait for its loads (issued during the previous tile), compute it,
    // and start the loads of the next tile into the other buffer on the way.  Called
    // with the buffers as constants so every LDS address is a per-lane base plus an
    // immediate.
    auto tile_step = [&](int t, auto KI) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's share of tile t has landed in LDS
      __builtin_amdgcn_s_barrier();         // every wave's share too; all waves are done with tile t - 1
      const int e = e_next;
      int e_dma = -1;
      if (t + 1 < ntile) {
        advance(t + 1);
        e_next = entry(t + 1);
        e_dma = e_next;
      }
      // the next tile's direct loads into the other buffer (free since the barrier);
      // issued in the second quarter step rather than right after the barrier: 0.9 %
      // faster on the sparse launch (same bits), the loads still land long before
      // the next tile
      auto issue_next = [&]() {
        if (e_dma >= 0) load_tile(e_dma & 0xffffff, std::integral_constant<int, 1 - decltype(KI)::value>());
      };
      constexpr int kbo = decltype(KI)::value * kTileBytes / 16, vbo = kbo;
      const int kb = e & 0xffffff;
      const int mode = slot_on ? (e >> (24 + 2 * slot)) & 3 : 0;
      if (mode) {
        const bool diag = kb == qb;
        bool tile_bias = false;
        if (qb - kb <= bias_dmax) {
          const int base = (qb - kb) * B;
#pragma unroll
          for (int t2 = 0; t2 < 8; ++t2) tile_bias |= boff[t2] > base - B && boff[t2] < base + B;
        }
        const bool masked = diag || mode != kModeFull || (kb + 1) * B > dm.n;
        const bool slow = masked || tile_bias;
        // multiplier from stored scores to log2 units, tile-uniform: kept in a scalar
        // register so the score FMA reads it directly
        const float ksc = __builtin_bit_cast(
            float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, slow ? 1.0f : sl2)));

        f32x16 S[2];       // scores of quarters a and a + 1 (by parity)
        unsigned P[2][8];  // packed bf16 probabilities of quarters a - 1 and a (by parity), [4 s2 + j]
        // operand fragments: K of the next quarter's scores is read one step ahead,
        // V^T of the quarter whose P V product runs in this step at the step start;
        // pinf forces a read to complete (one wait per group rather than per
        // instruction)
        u32x4_t kf[8], vf[8];
        auto kload = [&](int a) {
#pragma unroll
          for (int kc = 0; kc < 8; ++kc) kf[kc] = koff[kc][kbo + a * 32 * 16];
        };
        auto vload = [&](int a) {
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2) vf[4 * s2 + t2] = voff[2 * a + s2][vbo + t2 * 32 * 16];
        };
        auto pinf = [&](u32x4_t* f) {
#pragma unroll
          for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(f[j]));
        };
        auto qk = [&](int a) {
          f32x16 acc;
#pragma unroll
          for (int x = 0; x < 16; ++x) acc[x] = 0.0f;
#pragma unroll
          for (int kc = 0; kc < 8; ++kc)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[kc]), qreg[kc], acc, 0, 0, 0);
          S[a & 1] = acc;
        };
        auto pv = [&](int a) {
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const bf16x8_t Pb = as_bf16x8(make_uint4(P[a & 1][4 * s2 + 0], P[a & 1][4 * s2 + 1],
                                                     P[a & 1][4 * s2 + 2], P[a & 1][4 * s2 + 3]));
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2)
              oacc[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[4 * s2 + t2]), Pb, oacc[t2], 0, 0, 0);
          }
        };
        // masks and bias of quarter a (tiles that need them only), in log2 units
        auto soft_mask = [&](int a) {
          f32x16& s = S[a & 1];
          if (slow) {
#pragma unroll
            for (int x = 0; x < 16; ++x) s[x] *= sl2;
            int rr = r_in_blk - 8 * hl;  // r >= c  <=>  rr >= C
            asm volatile("" : "+v"(rr));
            if (tile_bias) {
#pragma unroll
              for (int t2 = 0; t2 < 8; ++t2) {
                if (boff[t2] < 0) continue;
                const int cstar = rr - (boff[t2] - (qb - kb) * B);  // r - c == off  <=>  C == cstar
#pragma unroll
                for (int x = 0; x < 16; ++x)
                  if (32 * a + 16 * (x >> 3) + (x & 7) == cstar) s[x] += bval[t2];
              }
            }
            if (masked) {
              // the kept keys of a row form one range lo <= C <= hi: C <= rr (lower
              // part) and / or C > rr (upper part), and C < nl (inside the sequence)
              const bool lower_ok = (mode & kModeLower) != 0;
              const bool upper_ok = (mode & kModeUpper) != 0 && !diag;
              const int nl = dm.n - kb * B - 8 * hl;
              const int lo = lower_ok ? 0 : rr + 1;
              const int hi = upper_ok ? nl - 1 : min(rr, nl - 1);
              // kept columns of this quarter as a bit mask over C - 32 a (bits lo .. hi;
              // 0 when the range is empty or misses the quarter), then one signed bit
              // extract (0 or all ones) and one bit select per score
              const int lj = min(max(lo - 32 * a, 0), 32), hj = min(max(hi - 32 * a, -1), 31);
              const unsigned keep = (lj < 32 ? ~0u << lj : 0u) & (hj >= 0 ? ~0u >> (31 - hj) : 0u);
              const unsigned ninf = __float_as_uint(-__builtin_inff());
#pragma unroll
              for (int x = 0; x < 16; ++x) {
                const unsigned sel = (unsigned)__builtin_amdgcn_sbfe((int)keep, 16 * (x >> 3) + (x & 7), 1);
                s[x] = __uint_as_float((sel & __float_as_uint(s[x])) | (~sel & ninf));
              }
            }
          }
        };
        // probabilities 2^(s - m_run) of quarter a as packed bf16 and their sum
        // (from the same bf16 values, in two interleaved partial sums so that the
        // dot instructions do not form one dependent chain)
        auto soft_exp = [&](int a, float m_use) -> float {
          float qs[2];
#pragma unroll
          for (int x = 0; x < 16; x += 2) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[a & 1][x], ksc, -m_use));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[a & 1][x + 1], ksc, -m_use));
            P[a & 1][x >> 1] = pack_bf16x2(p0, p1);
            if (x < 4) {
              // first term of each partial sum: the three-operand dot with a zero
              // addend (the two-operand form the compiler picks accumulates in place
              // and would need the zero moved in first)
              float r;
              asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(P[a & 1][x >> 1]), "s"(ones_bits));
              qs[(x >> 1) & 1] = r;
            } else {
              qs[(x >> 1) & 1] = sum_bf16x2(P[a & 1][x >> 1], qs[(x >> 1) & 1]);
            }
          }
          return qs[0] + qs[1];
        };
        // Lazy softmax: the reference m_run moves only when a quarter's probability
        // sum leaves [0, 2^64) (or is not a number: the first quarter, where m_run is
        // still -inf).  Then the quarter is redone against the row maximum and O and
        // l are rescaled to it.  Every p then stays below 2^64, so O and l cannot
        // overflow, and the result equals the one with any other reference.
        auto soft = [&](int a) {
          float qsum = soft_exp(a, m_run);
#pragma unroll
          for (int j = 0; j < 8; ++j) pin(P[a & 1][j]);
          if (__any(__float_as_uint(qsum) >= 0x5f800000u)) {
            const f32x16& s = S[a & 1];
            float mx = s[0];
#pragma unroll
            for (int x = 1; x < 16; ++x) mx = fmaxf(mx, s[x]);
            mx = half_swap_max(mx * ksc);
            const float m_new = mx > m_run ? mx : m_run;
            const float alpha = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
              for (int x = 0; x < 16; ++x) oacc[t2][x] *= alpha;
            qsum = soft_exp(a, m_run == -__builtin_inff() ? 0.0f : m_run);
          }
          l_run += qsum;
        };

        // Wave priority by progress through the tile: 3 until the first quarter step,
        // then 2, 1, 0.  The two waves of a SIMD (one per head of the pair) otherwise
        // run oldest-first: the older finished its tile about 1500 clocks before the
        // younger (per-wave clock counters, 32K dense), then idled at the barrier
        // while the younger ran alone without a partner to overlap with.  Issuing the
        // wave that is behind first keeps them level (the barrier wait fell from 15 %
        // to 6 % of the tile; 1.6 % and 1.9 % off the 128K sparse and dense launches,
        // same bits).
        __builtin_amdgcn_s_setprio(3);
        kload(0);
        qk(0);
        kload(1);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          if (a == 1) __builtin_amdgcn_s_setprio(2);
          if (a == 2) __builtin_amdgcn_s_setprio(1);
          if (a == 3) __builtin_amdgcn_s_setprio(0);
          if (a > 0) vload(a - 1);
          if (a < 3) pinf(kf);
          soft_mask(a);
          // the compiler's small-GEMM interleaving strategy for this region (matrix
          // instructions spread between the LDS reads and the softmax): 1-2 % faster
          // than its default schedule on both the sparse and the dense launch
          __builtin_amdgcn_iglp_opt(0);
          if (a < 3) qk(a + 1);
          if (a < 2) kload(a + 2);
          if (a == 1) issue_next();
          if (a > 0) { pinf(vf); pv(a - 1); }
          soft(a);
        }
        vload(3);
        pinf(vf);
        pv(3);
      } else {
        issue_next();
      }
    };

    e_next = ntile > 0 ? entry(0) : 0;
    if (ntile > 0) load_tile(e_next & 0xffffff, std::integral_constant<int, 0>());
    for (int t = 0; t < ntile; t += 2) {
      tile_step(t, std::integral_constant<int, 0>());
      if (t + 1 < ntile) tile_step(t + 1, std::integral_constant<int, 1>());
    }

    const float l_tot = half_swap_sum(l_run);
    if (slot_on && qrow < dm.n) {
      const float inv = 1.0f / l_tot;
      bf16_t* op = o + ((size_t)bh * dm.n + qrow) * D;
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int d0 = 32 * t2 + 8 * gg + 4 * hl;
          uint2 wv;
          wv.x = pack_bf16x2(oacc[t2][4 * gg + 0] * inv, oacc[t2][4 * gg + 1] * inv);
          wv.y = pack_bf16x2(oacc[t2][4 * gg + 2] * inv, oacc[t2][4 * gg + 3] * inv);
          *reinterpret_cast<uint2*>(op + d0) = wv;
        }
    }
  }  // items
}

// V^T of one KV head with keys padded to npad (a multiple of B) with zeros:
// vt[kvh][dim][key].  Block = 64 keys x 128 dims.
__global__ __launch_bounds__(256) void transpose_v_kernel(const bf16_t* __restrict__ v, bf16_t* __restrict__ vt,
                                                          int n, int npad) {
  __shared__ unsigned short tile[64][130];
  const int kvh = blockIdx.y, k0 = blockIdx.x * 64, tid = threadIdx.x;
  const bf16_t* src = v + (size_t)kvh * n * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;  // 1024 chunks of 8 dims
    const int key = id >> 4, c = id & 15;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (k0 + key < n) u = *reinterpret_cast<const uint4*>(src + (size_t)(k0 + key) * 128 + c * 8);
    const unsigned w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[key][c * 8 + 2 * j] = (unsigned short)(w4[j] & 0xffffu);
      tile[key][c * 8 + 2 * j + 1] = (unsigned short)(w4[j] >> 16);
    }
  }
  __syncthreads();
  bf16_t* dst = vt + (size_t)kvh * 128 * npad + k0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;  // 1024 chunks of 8 keys
    const int dim = id >> 3, c = id & 7;
    unsigned w4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w4[j] = (unsigned)tile[c * 8 + 2 * j][dim] | ((unsigned)tile[c * 8 + 2 * j + 1][dim] << 16);
    *reinterpret_cast<uint4*>(dst + (size_t)dim * npad + c * 8) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
}

// Tile list of a work item of the matrix engine (KV head g, query-head pair w,
// query block qb): ascending kb with each head's mask mode (bits 24-25 for the
// first head of the pair, 26-27 for the second; 0 = not in that head's set).
// One workgroup per (item, qb) marks the modes of key blocks in LDS, 4096 at a
// time, from the heads' index sets, then compacts them in order.
__global__ __launch_bounds__(256) void pair_tiles_kernel(Dims dm, int pairs, IndexOut io, int* __restrict__ ulist,
                                                         int* __restrict__ ucnt) {
  constexpr int kChunk = 4096;  // 256 threads x 16 key blocks
  // one byte per key block: bits 0-1 first head, 2-3 second
  __shared__ __align__(16) unsigned int modes[kChunk / 4];
  __shared__ int stage[kChunk];  // one chunk's entries in order, then copied out
  __shared__ int wave_tot[4];
  const int qb = blockIdx.x, item = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = item / pairs, w = item % pairs;
  const int bidx = g / dm.hkv, gh = g % dm.hkv;
  int* out = ulist + (size_t)item * dm.ntri + (size_t)qb * (qb + 1) / 2;
  int cnt = 0;
  for (int c0 = 0; c0 <= qb; c0 += kChunk) {
    const int c1 = min(c0 + kChunk, qb + 1);
    for (int i = tid; i < kChunk / 4; i += 256) modes[i] = 0;
    __syncthreads();
    for (int s2 = 0; s2 < 2; ++s2) {
      const int hin = 2 * w + s2;
      if (hin >= dm.group) continue;
      const int bh = bidx * dm.hq + gh * dm.group + hin;
      auto mark = [&](int kb, int mode) {
        if (kb >= c0 && kb < c1) {
          if (kb == qb) mode &= kModeLower;  // diagonal tile: causal part only
          if (mode) atomicOr(&modes[(kb - c0) >> 2], (unsigned)mode << (8 * ((kb - c0) & 3) + 2 * s2));
        }
      };
      // the route picks the head's lists; each list is read eight entries per thread
      // ahead of their marks, so a thread waits on one round of loads per 2048 entries
      // instead of one per 256
      const bool vs = io.route[bh] != 0;
      const int nv = io.vs_count[bh * 2], ns = io.vs_count[bh * 2 + 1];
      const int* rp = io.pe_rowptr + (size_t)bh * (dm.nb + 1);
      const int p0 = rp[qb], p1 = rp[qb + 1];
      auto mark_list = [&](const int* src, int count, bool slash) {
        for (int base = 0; base < count; base += 8 * 256) {
          int e[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = base + 256 * u + tid;
            e[u] = i < count ? src[i] : -1;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            if (e[u] < 0) continue;
            if (slash) {
              // slash block s: lower triangle of tile qb - s, upper triangle of tile qb - s - 1
              mark(qb - e[u], kModeLower);
              mark(qb - e[u] - 1, kModeUpper);
            } else {
              mark(e[u], kModeFull);  // vertical block or PE key block: whole tile
            }
          }
        }
      };
      if (vs) {
        mark_list(io.vs_vertical + (size_t)bh * dm.nb, nv, false);
        mark_list(io.vs_slash + (size_t)bh * dm.nb, ns, true);
      } else {
        mark_list(io.pe_col + (size_t)bh * io.pe_cap + p0, p1 - p0, false);
      }
    }
    __syncthreads();
    // thread tid compacts key blocks c0 + 16 tid .. + 15 (four words; blocks at or past
    // c1 were never marked): one block-wide prefix of the per-thread counts, the
    // entries staged in LDS in ascending order, then one coalesced copy
    const uint4 mw = reinterpret_cast<const uint4*>(modes)[tid];
    const unsigned wd[4] = {mw.x, mw.y, mw.z, mw.w};
    int n = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      unsigned nz = wd[j] | (wd[j] >> 1);
      nz |= nz >> 2;
      n += __popc(nz & 0x01010101u);
    }
    int incl = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int pos = incl - n, tot = 0;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      if (w2 < wave) pos += wave_tot[w2];
      tot += wave_tot[w2];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const unsigned m = (wd[j >> 2] >> (8 * (j & 3))) & 15u;
      if (m) stage[pos++] = (c0 + 16 * tid + j) | (int)((m & 3u) << 24) | (int)((m >> 2) << 26);
    }
    __syncthreads();
    for (int i = tid; i < tot; i += 256) out[cnt + i] = stage[i];
    cnt += tot;
    __syncthreads();  // modes, stage and wave_tot are reused by the next chunk
  }
  if (tid == 0) ucnt[(size_t)item * dm.nb + qb] = cnt;
}

// ----------------------------------------------------------- vector engine --
// One thread per query row; keys staged 32 at a time through LDS in fp32.
//
// A (head, query block) item is served by S workgroups of G groups of B
// threads; group g of workgroup s takes the item's tiles t with
// t mod (S G) = s G + g.  Each thread keeps one query row's running max, sum
// and output; the groups of a workgroup merge their partial results at the end
// in group order.  With S = 1 the workgroup writes the output row; otherwise it
// writes its partial (max, sum, output) to part and attn_generic_merge_kernel
// combines the S partials in workgroup order.  S > 1 is used when there are
// too few items to fill the chip (generic_splits); workgroup s only exists
// for an item with more than s G tiles.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void attn_generic_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ v, T* __restrict__ o,
                                                           Dims dm, BiasArgs bias, const int* __restrict__ tiles,
                                                           const int* __restrict__ tile_cnt, int dense, int S,
                                                           float* __restrict__ part) {
  constexpr int KCH = 32;
  constexpr float kLazy = 16.0f;
  // key and value chunks of every group; once the key loop is done the merge
  // buffer for the groups' outputs reuses the same memory (two workgroups fit
  // one CU's LDS)
  static_assert(G == 1 || G * KCH >= 64, "merge buffer must fit the chunk buffers");
  __shared__ float KV[2 * G * KCH * D];
  __shared__ float Cm[G > 1 ? 128 : 1], Cl[G > 1 ? 128 : 1];
  float (*Kc)[KCH * D] = reinterpret_cast<float (*)[KCH * D]>(KV);
  float (*Vc)[KCH * D] = reinterpret_cast<float (*)[KCH * D]>(KV + G * KCH * D);
  float* Ca = KV;
  const int item = blockIdx.x / S, split = blockIdx.x % S;
  int qb, bh;
  work_item(dm, item, &qb, &bh);
  const int B = dm.B;
  const int g = threadIdx.x / B, r = threadIdx.x % B;
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
  int boff[8];
  float bval[8];
#pragma unroll
  for (int t2 = 0; t2 < 8; ++t2) {
    boff[t2] = t2 < bias.count ? bias.offsets[(size_t)bh * bias.count + t2] : -1;
    bval[t2] = t2 < bias.count ? bias.values[(size_t)bh * bias.count + t2] : 0.0f;
  }
  const float c = (float)(1.0 / __builtin_sqrt((double)D));
  float m = -__builtin_inff(), l = 0.0f;
  const int ntile = dense ? qb + 1 : tile_cnt[(size_t)bh * dm.nb + qb];
  const int* tl = dense ? nullptr : tiles + (size_t)bh * dm.ntri + (size_t)qb * (qb + 1) / 2;
  // every group of the workgroup runs the same number of rounds (block barriers)
  const int stride = S * G, first = split * G;
  const int rounds = ntile > first ? (ntile - first + stride - 1) / stride : 0;
  // a workgroup beyond the item's tiles has nothing to add (the merge skips its
  // partial) and frees its CU at once, so a launch costs what its tiles cost
  if (rounds == 0 && S > 1) return;
  for (int rd = 0; rd < rounds; ++rd) {
    const int t = rd * stride + first + g;
    const bool active = t < ntile;
    int kb = 0, mode = kModeFull;
    if (active) {
      if (dense) {
        kb = t;
      } else {
        kb = tl[t] & 0x0fffffff;
        mode = tl[t] >> 28;
      }
    }
    const bool diag = kb == qb;
    for (int sub = 0; sub < B; sub += KCH) {
      __syncthreads();
      if (active)
        for (int e = r; e < KCH * D; e += B) {
          const int kk = e / D, dd = e % D;
          const int key = kb * B + sub + kk;
          Kc[g][e] = key < dm.n ? load_f32(kp + (size_t)key * D + dd) : 0.0f;
          Vc[g][e] = key < dm.n ? load_f32(vp + (size_t)key * D + dd) : 0.0f;
        }
      __syncthreads();
      if (!active) continue;
      // online softmax with a lazy reference: m moves only when a score exceeds
      // it by more than kLazy nats, so probabilities stay below e^kLazy and the
      // output and sum need rescaling only then
      for (int kk = 0; kk < KCH; ++kk) {
        const int cc = sub + kk;
        const int j = kb * B + cc;
        float dot = 0.0f;
#pragma unroll
        for (int t2 = 0; t2 < D; ++t2) dot = __builtin_fmaf(qv[t2], Kc[g][kk * D + t2], dot);
        float z = dot * c;
#pragma unroll
        for (int t2 = 0; t2 < 8; ++t2)
          if (boff[t2] == i - j) z += bval[t2];
        const bool ok = j < dm.n && j <= i && tile_keep(mode, diag, r, cc);
        if (!ok) continue;
        if (z > m + kLazy) {
          const float alpha = expf(m - z);  // 0 for the first key (m = -inf)
          l *= alpha;
#pragma unroll
          for (int t2 = 0; t2 < D; ++t2) acc[t2] *= alpha;
          m = z;
        }
        const float p = expf(z - m);
        l += p;
#pragma unroll
        for (int t2 = 0; t2 < D; ++t2) acc[t2] = __builtin_fmaf(p, Vc[g][kk * D + t2], acc[t2]);
      }
    }
  }
  // merge the groups' partial results into group 0, in group order
  for (int w = 1; w < G; ++w) {
    __syncthreads();
    if (g == w) {
      Cm[r] = m;
      Cl[r] = l;
#pragma unroll
      for (int t2 = 0; t2 < D; ++t2) Ca[r * D + t2] = acc[t2];
    }
    __syncthreads();
    if (g == 0) {
      const float mw = Cm[r];
      const float m_new = mw > m ? mw : m;
      if (m_new != -__builtin_inff()) {
        const float a0 = expf(m - m_new), a1 = expf(mw - m_new);
        l = l * a0 + Cl[r] * a1;
#pragma unroll
        for (int t2 = 0; t2 < D; ++t2) acc[t2] = acc[t2] * a0 + Ca[r * D + t2] * a1;
        m = m_new;
      }
    }
  }
  if (S > 1) {
    if (g == 0) {
      // partial of row r: [max, sum, output[D]]
      float* pp = part + (((size_t)item * S + split) * B + r) * (D + 2);
      pp[0] = m;
      pp[1] = l;
#pragma unroll
      for (int t2 = 0; t2 < D; ++t2) pp[2 + t2] = acc[t2];
    }
    return;
  }
  if (g == 0 && i < dm.n) {
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

// Combines the S partials of each row of an item in workgroup order (the same
// pairwise rescaling as the in-workgroup merge) and writes the output row.
template <typename T, int D>
__global__ __launch_bounds__(128) void attn_generic_merge_kernel(T* __restrict__ o, Dims dm, int S, int G,
                                                                 const int* __restrict__ tile_cnt, int dense,
                                                                 const float* __restrict__ part) {
  const int item = blockIdx.x, r = threadIdx.x;
  if (r >= dm.B) return;
  int qb, bh;
  work_item(dm, item, &qb, &bh);
  const int i = qb * dm.B + r;
  if (i >= dm.n) return;
  const int ntile = dense ? qb + 1 : tile_cnt[(size_t)bh * dm.nb + qb];
  const int used = min(S, (ntile + G - 1) / G);  // workgroups that had tiles
  float m = -__builtin_inff(), l = 0.0f, acc[D];
#pragma unroll
  for (int t2 = 0; t2 < D; ++t2) acc[t2] = 0.0f;
  for (int sp = 0; sp < used; ++sp) {
    const float* pp = part + (((size_t)item * S + sp) * dm.B + r) * (D + 2);
    const float mw = pp[0];
    const float m_new = mw > m ? mw : m;
    if (m_new == -__builtin_inff()) continue;
    const float a0 = expf(m - m_new), a1 = expf(mw - m_new);
    l = l * a0 + pp[1] * a1;
#pragma unroll
    for (int t2 = 0; t2 < D; ++t2) acc[t2] = acc[t2] * a0 + pp[2 + t2] * a1;
    m = m_new;
  }
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

template <typename T, int D>
void launch_generic(const Dims& dm, const BiasArgs& bias, const void* q, const void* k, const void* v,
                    void* o, const int* tiles, const int* tile_cnt, float* part, hipStream_t st) {
  const int S = generic_splits(dm);
  const int items = dm.bh * dm.nb, grid = items * S;
  // d = 64: 256 threads split each item's key tiles (4 groups at B = 64, 2 at B = 128);
  // d = 128 keeps one group (two accumulators of 128 floats per thread)
  if constexpr (D == 64) {
    if (dm.B == 64)
      attn_generic_kernel<T, D, 4><<<grid, 256, 0, st>>>(static_cast<const T*>(q), static_cast<const T*>(k),
                                                          static_cast<const T*>(v), static_cast<T*>(o), dm, bias,
                                                          tiles, tile_cnt, tiles == nullptr, S, part);
    else
      attn_generic_kernel<T, D, 2><<<grid, 256, 0, st>>>(static_cast<const T*>(q), static_cast<const T*>(k),
                                                          static_cast<const T*>(v), static_cast<T*>(o), dm, bias,
                                                          tiles, tile_cnt, tiles == nullptr, S, part);
  } else {
    attn_generic_kernel<T, D, 1><<<grid, dm.B, 0, st>>>(static_cast<const T*>(q), static_cast<const T*>(k),
                                                        static_cast<const T*>(v), static_cast<T*>(o), dm, bias,
                                                        tiles, tile_cnt, tiles == nullptr, S, part);
  }
  if (S > 1)
    attn_generic_merge_kernel<T, D><<<items, 128, 0, st>>>(static_cast<T*>(o), dm, S, generic_groups(dm), tile_cnt,
                                                         tiles == nullptr, part);
}

}  // namespace

bool use_matrix_engine(const Dims& dm) { return dm.dtype == 1 && dm.d == 128 && dm.B == 128; }

int generic_groups(const Dims& dm) { return dm.d == 64 ? (dm.B == 64 ? 4 : 2) : 1; }

int generic_splits(const Dims& dm) {
  const long long items = (long long)dm.bh * dm.nb;
  if (items >= kSplitItems) return 1;
  // about kSplitItems workgroups in all, at most kMaxSplits per item and no
  // more than the longest item has groups' worth of tiles
  long long s = (kSplitItems + items - 1) / items;
  const long long most = (dm.nb + generic_groups(dm) - 1) / generic_groups(dm);
  if (s > most) s = most;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : (int)s;
}

hipError_t launch_build_tiles(const Dims& dm, const IndexOut& io, int* tiles, int* tile_cnt, int* ulist,
                              int* ucnt, hipStream_t st) {
  if (use_matrix_engine(dm)) {
    const int pairs = (dm.group + 1) / 2;
    pair_tiles_kernel<<<dim3(dm.nb, dm.bkv * pairs), 256, 0, st>>>(dm, pairs, io, ulist, ucnt);
  } else {
    build_tiles_kernel<<<dim3((dm.nb + 127) / 128, dm.bh), 128, 0, st>>>(dm, io, tiles, tile_cnt);
  }
  return hipGetLastError();
}

__global__ void zero_counters_kernel(int* counters) {
  if (threadIdx.x < 8) counters[threadIdx.x] = 0;
}

hipError_t launch_attention(const Dims& dm, const BiasArgs& bias, const void* q, const void* k,
                            const void* v, void* o, const int* tiles, const int* tile_cnt, const int* ulist,
                            const int* ucnt, void* vt, int* counters, float* part, hipStream_t st) {
  if (use_matrix_engine(dm)) {
    const bf16_t* qq = static_cast<const bf16_t*>(q);
    const bf16_t* kk = static_cast<const bf16_t*>(k);
    bf16_t* vvt = static_cast<bf16_t*>(vt);
    bf16_t* oo = static_cast<bf16_t*>(o);
    const int npad = dm.nb * dm.B;
    transpose_v_kernel<<<dim3(npad / 64, dm.bkv), 256, 0, st>>>(static_cast<const bf16_t*>(v), vvt, dm.n, npad);
    const int pairs = (dm.group + 1) / 2;
    const long long combos = (long long)dm.bkv * pairs;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const long long items = combos * dm.nb;
    const int grid = (int)(items < cus ? items : cus);  // one persistent workgroup per CU
    zero_counters_kernel<<<1, 64, 0, st>>>(counters);
    if (tiles == nullptr)
      attn_mfma_kernel<true><<<grid, 512, 0, st>>>(qq, kk, vvt, oo, dm, bias, nullptr, nullptr, pairs, npad,
                                                    counters);
    else
      attn_mfma_kernel<false><<<grid, 512, 0, st>>>(qq, kk, vvt, oo, dm, bias, ulist, ucnt, pairs, npad,
                                                     counters);
  } else if (dm.dtype == 1) {
    if (dm.d == 128) launch_generic<bf16_t, 128>(dm, bias, q, k, v, o, tiles, tile_cnt, part, st);
    else launch_generic<bf16_t, 64>(dm, bias, q, k, v, o, tiles, tile_cnt, part, st);
  } else {
    if (dm.d == 128) launch_generic<float, 128>(dm, bias, q, k, v, o, tiles, tile_cnt, part, st);
    else launch_generic<float, 64>(dm, bias, q, k, v, o, tiles, tile_cnt, part, st);
  }
  return hipGetLastError();
}

}  // namespace crisp
