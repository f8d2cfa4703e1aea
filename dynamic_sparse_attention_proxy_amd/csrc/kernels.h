// Internal launch interface between the C-ABI host code and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace crisp {

// Problem geometry shared by every kernel.
struct Dims {
  int batch, hq, hkv, group;  // query heads per batch, kv heads per batch, hq / hkv
  int bh, bkv;                // batch * hq, batch * hkv
  int n, d, B, nb;            // sequence length, head dim, block size, ceil(n / B)
  int q0, qrows;              // first row and row count of the last query block
  int dtype;                  // 0 = fp32, 1 = bf16
  long long ntri;             // nb (nb + 1) / 2
};

struct BiasArgs {
  int count;  // 0..8
  const int* offsets;
  const float* values;
};

struct RouteArgs {
  int w_sink, w_local;
  unsigned tau_num, tau_den;
};

struct SelectArgs {
  unsigned alpha_num, alpha_den, gamma_num, gamma_den;
  int keep_all;    // every head keeps its full causal set
  int cumulative;  // VS heads use the cumulative-coverage rule instead of Eq. 3-4
};

// Scratch regions (device pointers carved from the caller's workspace).
struct RouteScratch {
  float* S;           // [bh][nb][B (key)][B (row)] proxy scores, tile-contiguous
  int* m_enc;         // [bh][B] row max (order-preserving int encoding)
  long long* L;       // [bh][B] fixed-point row sums
  long long* part;    // [4][bh][nb] per key block: vertical, slash-lower, slash-upper, anchor
};

struct SelectScratch {
  float* qbar;         // [bh][nb][d]
  float* kbar;         // [bkv][nb][d]
  float* zbar;         // [bh][nb][nb] pooled scores (lower triangle used)
  long long* abar;     // [bh][ntri] quantised pooled map, row-major triangle
  long long* rowtot;   // [bh][nb]
  unsigned long long* hist;  // [bh][4][2048][2] radix histogram (count, mass)
  long long* state;    // [bh][8] radix-select state
  int* gtcnt;          // [bh][nb]
  int* tiecnt;         // [bh][nb]
  int* tiepre;         // [bh][nb]
};

struct JsdScratch {
  float* qbar;      // [bh][d] block mean of the last query block
  float* kbar;      // [bkv][nb][d] block means of every key block
  float* zbar;      // [bh][nb] pooled scores of the last query block
  long long* abar;  // [bh][nb] quantised pooled estimate
};

struct IndexOut {
  uint8_t* route;
  long long* cstruct_num;
  long long* mass_v;
  long long* mass_s;
  long long* mass_total;
  int* vs_count;
  int* vs_vertical;
  int* vs_slash;
  int* pe_rowptr;
  int* pe_col;
  long long pe_cap;
};

// route.hip
hipError_t launch_route(const Dims& dm, const RouteArgs& ra, const BiasArgs& bias, const void* q,
                        const void* k, const RouteScratch& ws, const IndexOut& io, hipStream_t st);
// select.hip
hipError_t launch_select(const Dims& dm, const SelectArgs& sa, const void* q, const void* k,
                         const SelectScratch& ws, const IndexOut& io, hipStream_t st);
// jsd.hip: the divergence router; reads mass_v / mass_total written by launch_route
hipError_t launch_route_jsd(const Dims& dm, unsigned tau_num, unsigned tau_den, const void* q, const void* k,
                            const JsdScratch& ws, const long long* mass_v, const long long* mass_total,
                            uint8_t* route_jsd, long long* jsd, long long* pooled, hipStream_t st);
// attention.hip
bool use_matrix_engine(const Dims& dm);  // bf16, d = 128, B = 128
// Vector engine: groups of B threads per workgroup (generic_groups), and
// workgroups per (head, query block) item (generic_splits): launches with fewer
// than kSplitItems items split each item over up to kMaxSplits workgroups.
// With S > 1 the partial results take bh * nb * S * B * (d + 2) floats of
// scratch (below kSplitItems * kMaxSplits * B * (d + 2)).
constexpr long long kSplitItems = 1024;
constexpr long long kMaxSplits = 8;
int generic_groups(const Dims& dm);
int generic_splits(const Dims& dm);
// tile lists: for the matrix engine the lists of query-head pairs [bkv * pairs][ntri]
// + counts [bkv * pairs][nb] (ulist / ucnt), else per-head lists [bh][ntri] + counts
// [bh][nb] (tiles / tile_cnt)
hipError_t launch_build_tiles(const Dims& dm, const IndexOut& io, int* tiles, int* tile_cnt, int* ulist,
                              int* ucnt, hipStream_t st);
// tiles == nullptr: dense causal.  Scratch used by the matrix engine: vt holds V^T of
// every KV head with keys padded to nb * B (bkv * d * nb * B elements); counters
// holds the 8 work-queue counters.  Scratch used by the vector engine: part holds
// the split partial results (generic_splits).
hipError_t launch_attention(const Dims& dm, const BiasArgs& bias, const void* q, const void* k,
                            const void* v, void* o, const int* tiles, const int* tile_cnt, const int* ulist,
                            const int* ucnt, void* vt, int* counters, float* part, hipStream_t st);

}  // namespace crisp
