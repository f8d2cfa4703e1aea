// C-ABI of the CRISP sparse-prefill library: argument validation, workspace
// carve-up and launch sequencing on the caller's stream.  No allocation, no
// host synchronisation.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/crisp.h"
#include "kernels.h"

using namespace crisp;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxSeq = 1 << 23;  // keeps every int64 fixed-point row sum below 2^63
// N_b (N_b + 1) / 2 (PE CSR offsets, flat indices of the pooled map) must fit int32
constexpr int kMaxBlocks = 65535;
// (head, query block) items: one-dimensional grids of up to 256-thread
// workgroups over them stay below 2^32 work-items, and the matrix engine's
// queue positions fit in 24 bits
constexpr long long kMaxItems = (1 << 24) - 1;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Layout {
  // route
  size_t r_S, r_m, r_L, r_part, r_end;
  // select
  size_t s_qbar, s_kbar, s_zbar, s_abar, s_rowtot, s_hist, s_state, s_gt, s_tie, s_tiep, s_end;
  // attention
  size_t a_tiles, a_cnt, a_ulist, a_ucnt, a_vt, a_part, a_qcnt, a_end;
  // divergence router
  size_t j_qbar, j_kbar, j_zbar, j_abar, j_end;
  size_t total;
};

crisp_status make_dims(const crisp_shape* sh, const crisp_config* cfg, Dims* dm) {
  if (!sh || !cfg) return CRISP_ERR_NULL;
  if (sh->dtype != CRISP_F32 && sh->dtype != CRISP_BF16) return CRISP_ERR_DTYPE;
  if (sh->batch < 1 || sh->n_q_heads < 1 || sh->n_kv_heads < 1 || sh->n_q_heads % sh->n_kv_heads)
    return CRISP_ERR_SHAPE;
  if (sh->seq_len < 1 || sh->seq_len > kMaxSeq) return CRISP_ERR_SHAPE;
  if (sh->head_dim != 64 && sh->head_dim != 128) return CRISP_ERR_SHAPE;
  if ((long long)sh->batch * sh->n_q_heads > 65535) return CRISP_ERR_SHAPE;
  if (cfg->block != 64 && cfg->block != 128) return CRISP_ERR_CONFIG;
  if (cfg->w_sink < 1 || cfg->w_local < 1) return CRISP_ERR_CONFIG;
  if (cfg->tau_den == 0 || cfg->alpha_den == 0 || cfg->gamma_den == 0) return CRISP_ERR_CONFIG;
  if (cfg->gamma_num > cfg->gamma_den) return CRISP_ERR_CONFIG;
  if (cfg->select_mode != CRISP_SELECT_NOISE_FLOOR && cfg->select_mode != CRISP_SELECT_KEEP_ALL &&
      cfg->select_mode != CRISP_SELECT_CUMULATIVE)
    return CRISP_ERR_CONFIG;
  Dims d;
  d.batch = sh->batch;
  d.hq = sh->n_q_heads;
  d.hkv = sh->n_kv_heads;
  d.group = d.hq / d.hkv;
  d.bh = sh->batch * d.hq;
  d.bkv = sh->batch * d.hkv;
  d.n = sh->seq_len;
  d.d = sh->head_dim;
  d.B = cfg->block;
  d.nb = (d.n + d.B - 1) / d.B;
  d.q0 = (d.nb - 1) * d.B;
  d.qrows = d.n - d.q0;
  d.dtype = sh->dtype;
  d.ntri = (long long)d.nb * (d.nb + 1) / 2;
  if (d.nb > kMaxBlocks || (long long)d.bh * d.nb > kMaxItems) return CRISP_ERR_SHAPE;
  *dm = d;
  return CRISP_OK;
}

Layout layout(const Dims& d) {
  Layout L;
  size_t o = 0;
  L.r_S = o;
  o = align_up(o + (size_t)d.bh * d.nb * d.B * d.B * sizeof(float));
  L.r_m = o;
  o = align_up(o + (size_t)d.bh * d.B * sizeof(int));
  L.r_L = o;
  o = align_up(o + (size_t)d.bh * d.B * sizeof(long long));
  L.r_part = o;
  o = align_up(o + (size_t)4 * d.bh * d.nb * sizeof(long long));
  L.r_end = o;

  o = 0;
  L.s_qbar = o;
  o = align_up(o + (size_t)d.bh * d.nb * d.d * sizeof(float));
  L.s_kbar = o;
  o = align_up(o + (size_t)d.bkv * d.nb * d.d * sizeof(float));
  L.s_zbar = o;
  o = align_up(o + (size_t)d.bh * d.nb * d.nb * sizeof(float));
  L.s_abar = o;
  o = align_up(o + (size_t)d.bh * d.ntri * sizeof(long long));
  L.s_rowtot = o;
  o = align_up(o + (size_t)d.bh * d.nb * sizeof(long long));
  L.s_hist = o;
  o = align_up(o + (size_t)d.bh * 4 * 2048 * 2 * sizeof(unsigned long long));
  L.s_state = o;
  o = align_up(o + (size_t)d.bh * 8 * sizeof(long long));
  L.s_gt = o;
  o = align_up(o + (size_t)d.bh * d.nb * sizeof(int));
  L.s_tie = o;
  o = align_up(o + (size_t)d.bh * d.nb * sizeof(int));
  L.s_tiep = o;
  o = align_up(o + (size_t)d.bh * d.nb * sizeof(int));
  L.s_end = o;

  o = 0;
  const bool mat = use_matrix_engine(d);
  const size_t pairs = (size_t)d.bkv * ((d.group + 1) / 2);
  L.a_tiles = o;  // per-head lists (vector engine)
  if (!mat) o = align_up(o + (size_t)d.bh * d.ntri * sizeof(int));
  L.a_cnt = o;
  if (!mat) o = align_up(o + (size_t)d.bh * d.nb * sizeof(int));
  L.a_ulist = o;  // pair lists (matrix engine)
  if (mat) o = align_up(o + pairs * d.ntri * sizeof(int));
  L.a_ucnt = o;
  if (mat) o = align_up(o + pairs * d.nb * sizeof(int));
  L.a_vt = o;
  if (mat) o = align_up(o + (size_t)d.bkv * d.d * d.nb * d.B * 2);  // V^T, bf16
  L.a_part = o;  // split partials (vector engine)
  if (!mat && generic_splits(d) > 1)
    o = align_up(o + (size_t)d.bh * d.nb * generic_splits(d) * d.B * (d.d + 2) * sizeof(float));
  L.a_qcnt = o;
  o = align_up(o + 8 * sizeof(int));  // work-queue counters
  L.a_end = o;

  o = 0;
  L.j_qbar = o;
  o = align_up(o + (size_t)d.bh * d.d * sizeof(float));
  L.j_kbar = o;
  o = align_up(o + (size_t)d.bkv * d.nb * d.d * sizeof(float));
  L.j_zbar = o;
  o = align_up(o + (size_t)d.bh * d.nb * sizeof(float));
  L.j_abar = o;
  o = align_up(o + (size_t)d.bh * d.nb * sizeof(long long));
  L.j_end = o;

  L.total = L.r_end;
  if (L.s_end > L.total) L.total = L.s_end;
  if (L.a_end > L.total) L.total = L.a_end;
  if (L.j_end > L.total) L.total = L.j_end;
  return L;
}

crisp_status check_bias(const crisp_rel_bias* bias, BiasArgs* out) {
  out->count = 0;
  out->offsets = nullptr;
  out->values = nullptr;
  if (!bias || bias->count == 0) return CRISP_OK;
  if (bias->count < 0 || bias->count > 8) return CRISP_ERR_CONFIG;
  if (!bias->offsets || !bias->values) return CRISP_ERR_NULL;
  if (!aligned(bias->offsets, 4) || !aligned(bias->values, 4)) return CRISP_ERR_ALIGN;
  out->count = bias->count;
  out->offsets = bias->offsets;
  out->values = bias->values;
  return CRISP_OK;
}

IndexOut index_out(const crisp_index_sets* idx) {
  IndexOut io;
  io.route = idx->route;
  io.cstruct_num = reinterpret_cast<long long*>(idx->cstruct_num);
  io.mass_v = reinterpret_cast<long long*>(idx->mass_v);
  io.mass_s = reinterpret_cast<long long*>(idx->mass_s);
  io.mass_total = reinterpret_cast<long long*>(idx->mass_total);
  io.vs_count = idx->vs_count;
  io.vs_vertical = idx->vs_vertical;
  io.vs_slash = idx->vs_slash;
  io.pe_rowptr = idx->pe_rowptr;
  io.pe_col = idx->pe_col;
  io.pe_cap = idx->pe_cap;
  return io;
}

crisp_status check_tensor(const void* p) {
  if (!p) return CRISP_ERR_NULL;
  if (!aligned(p, 16)) return CRISP_ERR_ALIGN;
  return CRISP_OK;
}

crisp_status check_routing_fields(const crisp_index_sets* idx) {
  if (!idx || !idx->route || !idx->cstruct_num || !idx->mass_v || !idx->mass_s || !idx->mass_total)
    return CRISP_ERR_NULL;
  if (!aligned(idx->cstruct_num, 8) || !aligned(idx->mass_v, 8) || !aligned(idx->mass_s, 8) ||
      !aligned(idx->mass_total, 8))
    return CRISP_ERR_ALIGN;
  return CRISP_OK;
}

crisp_status check_list_fields(const crisp_index_sets* idx, const Dims& d) {
  if (!idx->vs_count || !idx->vs_vertical || !idx->vs_slash || !idx->pe_rowptr || !idx->pe_col)
    return CRISP_ERR_NULL;
  if (!aligned(idx->vs_count, 4) || !aligned(idx->vs_vertical, 4) || !aligned(idx->vs_slash, 4) ||
      !aligned(idx->pe_rowptr, 4) || !aligned(idx->pe_col, 4))
    return CRISP_ERR_ALIGN;
  if (idx->pe_cap < d.ntri) return CRISP_ERR_CAPACITY;
  return CRISP_OK;
}

// Launch failures of one call: every entry point resets the last-error state
// right before its launches (documented in the header) and reads it after them.
crisp_status hip_status() {
  return hipGetLastError() == hipSuccess ? CRISP_OK : CRISP_ERR_HIP;
}

#define CRISP_TRY(x)                 \
  do {                               \
    crisp_status s_ = (x);           \
    if (s_ != CRISP_OK) return s_;   \
  } while (0)

// Argument checks shared by the two sparse-prefill entry points.
crisp_status check_sparse_args(const crisp_shape* shape, const crisp_config* cfg, const void* q, const void* k,
                               const void* v, const crisp_rel_bias* bias, const crisp_index_sets* idx,
                               const void* o, Dims* d, BiasArgs* ba) {
  CRISP_TRY(make_dims(shape, cfg, d));
  CRISP_TRY(check_tensor(q));
  CRISP_TRY(check_tensor(k));
  CRISP_TRY(check_tensor(v));
  CRISP_TRY(check_tensor(o));
  if (!idx || !idx->route) return CRISP_ERR_NULL;
  CRISP_TRY(check_list_fields(idx, *d));
  CRISP_TRY(check_bias(bias, ba));
  return CRISP_OK;
}

// Tile lists, then attention, with the scratch regions carved from w.
crisp_status run_sparse(const Dims& d, const Layout& L, const BiasArgs& ba, const void* q, const void* k,
                        const void* v, const crisp_index_sets* idx, char* w, void* o, void* stream) {
  int* tiles = reinterpret_cast<int*>(w + L.a_tiles);
  int* cnt = reinterpret_cast<int*>(w + L.a_cnt);
  int* ulist = reinterpret_cast<int*>(w + L.a_ulist);
  int* ucnt = reinterpret_cast<int*>(w + L.a_ucnt);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (launch_build_tiles(d, index_out(idx), tiles, cnt, ulist, ucnt, st) != hipSuccess) return CRISP_ERR_HIP;
  if (launch_attention(d, ba, q, k, v, o, tiles, cnt, ulist, ucnt, w + L.a_vt,
                       reinterpret_cast<int*>(w + L.a_qcnt), reinterpret_cast<float*>(w + L.a_part),
                       st) != hipSuccess)
    return CRISP_ERR_HIP;
  return hip_status();
}

// Scratch of crisp_sparse_prefill_noalloc: a static device array, one copy per
// GPU the library runs on.  Host code never passes the array's name to a
// kernel (on the host it only names the symbol): the device address of each
// GPU's copy is looked up once per device with hipGetSymbolAddress, with that
// device current, and kept in g_scratch.
constexpr size_t kScratchBytes = size_t(128) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

crisp_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CRISP_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CRISP_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CRISP_OK;
}

}  // namespace

extern "C" {

size_t crisp_workspace_size(const crisp_shape* shape, const crisp_config* cfg) {
  Dims d;
  if (make_dims(shape, cfg, &d) != CRISP_OK) return 0;
  return layout(d).total;
}

int64_t crisp_index_capacity(const crisp_shape* shape, const crisp_config* cfg) {
  Dims d;
  if (make_dims(shape, cfg, &d) != CRISP_OK) return -1;
  return d.ntri;
}

crisp_status crisp_route(const crisp_shape* shape, const crisp_config* cfg, const void* q, const void* k,
                         const crisp_rel_bias* bias, void* ws, size_t ws_bytes, crisp_index_sets* idx,
                         void* stream) {
  Dims d;
  CRISP_TRY(make_dims(shape, cfg, &d));
  CRISP_TRY(check_tensor(q));
  CRISP_TRY(check_tensor(k));
  CRISP_TRY(check_tensor(ws));
  CRISP_TRY(check_routing_fields(idx));
  BiasArgs ba;
  CRISP_TRY(check_bias(bias, &ba));
  const Layout L = layout(d);
  if (ws_bytes < L.total) return CRISP_ERR_WORKSPACE;
  char* w = static_cast<char*>(ws);
  RouteScratch rs;
  rs.S = reinterpret_cast<float*>(w + L.r_S);
  rs.m_enc = reinterpret_cast<int*>(w + L.r_m);
  rs.L = reinterpret_cast<long long*>(w + L.r_L);
  rs.part = reinterpret_cast<long long*>(w + L.r_part);
  RouteArgs ra;
  ra.w_sink = cfg->w_sink;
  ra.w_local = cfg->w_local;
  ra.tau_num = cfg->tau_num;
  ra.tau_den = cfg->tau_den;
  (void)hipGetLastError();
  if (launch_route(d, ra, ba, q, k, rs, index_out(idx), static_cast<hipStream_t>(stream)) != hipSuccess)
    return CRISP_ERR_HIP;
  return hip_status();
}

crisp_status crisp_select_indices(const crisp_shape* shape, const crisp_config* cfg, const void* q,
                                  const void* k, void* ws, size_t ws_bytes, crisp_index_sets* idx,
                                  void* stream) {
  Dims d;
  CRISP_TRY(make_dims(shape, cfg, &d));
  CRISP_TRY(check_tensor(q));
  CRISP_TRY(check_tensor(k));
  CRISP_TRY(check_tensor(ws));
  CRISP_TRY(check_routing_fields(idx));
  CRISP_TRY(check_list_fields(idx, d));
  const Layout L = layout(d);
  if (ws_bytes < L.total) return CRISP_ERR_WORKSPACE;
  char* w = static_cast<char*>(ws);
  SelectScratch ss;
  ss.qbar = reinterpret_cast<float*>(w + L.s_qbar);
  ss.kbar = reinterpret_cast<float*>(w + L.s_kbar);
  ss.zbar = reinterpret_cast<float*>(w + L.s_zbar);
  ss.abar = reinterpret_cast<long long*>(w + L.s_abar);
  ss.rowtot = reinterpret_cast<long long*>(w + L.s_rowtot);
  ss.hist = reinterpret_cast<unsigned long long*>(w + L.s_hist);
  ss.state = reinterpret_cast<long long*>(w + L.s_state);
  ss.gtcnt = reinterpret_cast<int*>(w + L.s_gt);
  ss.tiecnt = reinterpret_cast<int*>(w + L.s_tie);
  ss.tiepre = reinterpret_cast<int*>(w + L.s_tiep);
  SelectArgs sa;
  sa.alpha_num = cfg->alpha_num;
  sa.alpha_den = cfg->alpha_den;
  sa.gamma_num = cfg->gamma_num;
  sa.gamma_den = cfg->gamma_den;
  sa.keep_all = cfg->select_mode == CRISP_SELECT_KEEP_ALL;
  sa.cumulative = cfg->select_mode == CRISP_SELECT_CUMULATIVE;
  (void)hipGetLastError();
  if (launch_select(d, sa, q, k, ss, index_out(idx), static_cast<hipStream_t>(stream)) != hipSuccess)
    return CRISP_ERR_HIP;
  return hip_status();
}

crisp_status crisp_sparse_prefill(const crisp_shape* shape, const crisp_config* cfg, const void* q,
                                  const void* k, const void* v, const crisp_rel_bias* bias,
                                  const crisp_index_sets* idx, void* ws, size_t ws_bytes, void* o,
                                  void* stream) {
  Dims d;
  BiasArgs ba;
  CRISP_TRY(check_sparse_args(shape, cfg, q, k, v, bias, idx, o, &d, &ba));
  CRISP_TRY(check_tensor(ws));
  const Layout L = layout(d);
  if (ws_bytes < L.total) return CRISP_ERR_WORKSPACE;
  return run_sparse(d, L, ba, q, k, v, idx, static_cast<char*>(ws), o, stream);
}

crisp_status crisp_sparse_prefill_noalloc(const crisp_shape* shape, const crisp_config* cfg, const void* q,
                                          const void* k, const void* v, const crisp_rel_bias* bias,
                                          const crisp_index_sets* idx, void* o, void* stream) {
  Dims d;
  BiasArgs ba;
  CRISP_TRY(check_sparse_args(shape, cfg, q, k, v, bias, idx, o, &d, &ba));
  const Layout L = layout(d);
  // the attention regions of the layout start at offset 0 and end at a_end
  if (L.a_end > kScratchBytes) return CRISP_ERR_SCRATCH;
  void* sp = nullptr;
  CRISP_TRY(device_scratch(&sp));
  return run_sparse(d, L, ba, q, k, v, idx, static_cast<char*>(sp), o, stream);
}

crisp_status crisp_dense_prefill(const crisp_shape* shape, const crisp_config* cfg, const void* q,
                                 const void* k, const void* v, const crisp_rel_bias* bias, void* ws,
                                 size_t ws_bytes, void* o, void* stream) {
  Dims d;
  CRISP_TRY(make_dims(shape, cfg, &d));
  CRISP_TRY(check_tensor(q));
  CRISP_TRY(check_tensor(k));
  CRISP_TRY(check_tensor(v));
  CRISP_TRY(check_tensor(o));
  CRISP_TRY(check_tensor(ws));
  BiasArgs ba;
  CRISP_TRY(check_bias(bias, &ba));
  const Layout L = layout(d);
  if (ws_bytes < L.total) return CRISP_ERR_WORKSPACE;
  char* w = static_cast<char*>(ws);
  (void)hipGetLastError();
  if (launch_attention(d, ba, q, k, v, o, nullptr, nullptr, nullptr, nullptr, w + L.a_vt,
                       reinterpret_cast<int*>(w + L.a_qcnt), reinterpret_cast<float*>(w + L.a_part),
                       static_cast<hipStream_t>(stream)) != hipSuccess)
    return CRISP_ERR_HIP;
  return hip_status();
}

crisp_status crisp_route_jsd(const crisp_shape* shape, const crisp_config* cfg, uint32_t tau_num,
                             uint32_t tau_den, const void* q, const void* k, const crisp_index_sets* idx,
                             void* ws, size_t ws_bytes, uint8_t* route_jsd, int64_t* jsd, int64_t* pooled,
                             void* stream) {
  Dims d;
  CRISP_TRY(make_dims(shape, cfg, &d));
  if (tau_den == 0) return CRISP_ERR_CONFIG;
  CRISP_TRY(check_tensor(q));
  CRISP_TRY(check_tensor(k));
  CRISP_TRY(check_tensor(ws));
  if (!idx || !idx->mass_v || !idx->mass_total || !route_jsd || !jsd) return CRISP_ERR_NULL;
  if (!aligned(idx->mass_v, 8) || !aligned(idx->mass_total, 8) || !aligned(jsd, 8) ||
      (pooled && !aligned(pooled, 8)))
    return CRISP_ERR_ALIGN;
  const Layout L = layout(d);
  if (ws_bytes < L.total) return CRISP_ERR_WORKSPACE;
  char* w = static_cast<char*>(ws);
  JsdScratch js;
  js.qbar = reinterpret_cast<float*>(w + L.j_qbar);
  js.kbar = reinterpret_cast<float*>(w + L.j_kbar);
  js.zbar = reinterpret_cast<float*>(w + L.j_zbar);
  js.abar = reinterpret_cast<long long*>(w + L.j_abar);
  (void)hipGetLastError();
  if (launch_route_jsd(d, tau_num, tau_den, q, k, js, reinterpret_cast<const long long*>(idx->mass_v),
                       reinterpret_cast<const long long*>(idx->mass_total), route_jsd,
                       reinterpret_cast<long long*>(jsd), reinterpret_cast<long long*>(pooled),
                       static_cast<hipStream_t>(stream)) != hipSuccess)
    return CRISP_ERR_HIP;
  return hip_status();
}

crisp_status crisp_tile_layout_of(const crisp_shape* shape, const crisp_config* cfg, crisp_tile_layout* out) {
  Dims d;
  CRISP_TRY(make_dims(shape, cfg, &d));
  if (!out) return CRISP_ERR_NULL;
  const Layout L = layout(d);
  const bool mat = use_matrix_engine(d);
  out->list_offset = (int64_t)(mat ? L.a_ulist : L.a_tiles);
  out->count_offset = (int64_t)(mat ? L.a_ucnt : L.a_cnt);
  out->list_stride = d.ntri;
  out->n_lists = mat ? d.bkv * ((d.group + 1) / 2) : d.bh;
  out->pair_lists = mat ? 1 : 0;
  return CRISP_OK;
}

const char* crisp_status_string(crisp_status s) {
  switch (s) {
    case CRISP_OK: return "ok";
    case CRISP_ERR_NULL: return "a required pointer is NULL";
    case CRISP_ERR_SHAPE: return "unsupported or inconsistent shape";
    case CRISP_ERR_DTYPE: return "unsupported dtype";
    case CRISP_ERR_CONFIG: return "invalid configuration";
    case CRISP_ERR_WORKSPACE: return "workspace too small";
    case CRISP_ERR_CAPACITY: return "index capacity too small";
    case CRISP_ERR_HIP: return "HIP launch failed";
    case CRISP_ERR_ALIGN: return "pointer not aligned";
    case CRISP_ERR_SCRATCH: return "problem needs more scratch than the allocation-free entry point holds (128 MiB)";
  }
  return "unknown status";
}

}  // extern "C"
