/*
 * crisp.h - C interface of the CRISP sparse-prefill library for AMD MI355X (gfx950).
 *
 * The operation (CRISP summary page, picx.dev, "Algorithm Overview", Alg. 1):
 * for each attention head of one prefill layer, build a proxy attention map
 * from a query subset (Alg. 2), route the head to the Vertical-Slash (VS) or
 * the pooled-estimation (PE) path with the structural proxy C_struct (Eq. 2),
 * select a sparse index set (Alg. 3 with the sink-aware noise floor of Eq. 3
 * and Eq. 4, or Alg. 4), and compute causal attention restricted to it.
 *
 * Four calls, in this order for one layer, all asynchronous on `stream`:
 *   crisp_route           proxy map of the last query block, C_struct, route bits
 *   crisp_select_indices  VS vertical/slash block lists or the PE block set
 *   crisp_sparse_prefill  attention over the selected blocks
 *   crisp_dense_prefill   full causal attention with the same tile engine
 * and, for comparison, crisp_route_jsd: the Jensen-Shannon divergence router
 * that C_struct replaces, evaluated on the same proxy after crisp_route.
 *
 * Conventions shared by every call
 *   - Tensors are caller-owned device memory, contiguous, row-major:
 *       q, o : [batch][n_q_heads][seq_len][head_dim]
 *       k, v : [batch][n_kv_heads][seq_len][head_dim]
 *     element type from crisp_shape.dtype (fp32 or bf16); query head h of a
 *     batch entry reads KV head h / (n_q_heads / n_kv_heads).  Attention is
 *     always causal.
 *   - "Heads" below means batch * n_q_heads flattened heads (BH); N_b =
 *     ceil(seq_len / block).  The proxy query subset is the last query block,
 *     rows (N_b - 1) * block .. seq_len - 1 (qrows rows).
 *   - The library never allocates or frees device memory and keeps no state:
 *     `ws` is scratch for the duration of one call (no call reads what an
 *     earlier call left in it; results pass between calls in idx).  Calls that
 *     can run at the same time (on different streams) need separate
 *     workspaces.  Pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *     kernels and return; results are valid once the stream has completed.
 *     No call synchronises with the host.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     failure a negative crisp_status is returned and nothing is written.
 *     A failed kernel launch returns CRISP_ERR_HIP.  To tell its own launch
 *     failures apart, each call resets HIP's last-error state before its
 *     launches: an error that earlier work of the caller left there is
 *     dropped, so check it before calling.
 *   - Supported: head_dim in {64, 128}, block in {64, 128}, n_q_heads a
 *     multiple of n_kv_heads, seq_len >= 1.  The bf16 MFMA attention engine
 *     serves head_dim 128 with block 128; other shapes use a vector-ALU engine.
 *   - Size limits (CRISP_ERR_SHAPE beyond them): seq_len <= 2^23 (int64
 *     fixed-point sums), N_b <= 65535 (int32 CSR offsets), batch * n_q_heads
 *     <= 65535 and batch * n_q_heads * N_b < 2^24 (launch grids over
 *     (head, query block) items).  Any shape whose workspace fits in one
 *     GPU's memory is inside them.
 *
 * Numerics of the decision steps (route and index sets) are exactly specified
 * so results are reproducible bit for bit: fp32 proxy scores with a fixed
 * fused-multiply-add order over the head dimension, a fixed fp32 exponential,
 * int64 fixed-point (2^40) sums and integer threshold tests.  Attention uses
 * bf16 matrix cores with fp32 accumulation (fp32 vector ALU for fp32 inputs).
 */
#ifndef CRISP_H
#define CRISP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CRISP_OK = 0,
  CRISP_ERR_NULL = -1,      /* a required pointer is NULL */
  CRISP_ERR_SHAPE = -2,     /* unsupported or inconsistent shape */
  CRISP_ERR_DTYPE = -3,     /* dtype not CRISP_F32 / CRISP_BF16 */
  CRISP_ERR_CONFIG = -4,    /* block not 64/128, windows < 1, zero denominators, bad mode, bias count > 8 */
  CRISP_ERR_WORKSPACE = -5, /* ws_bytes < crisp_workspace_size() */
  CRISP_ERR_CAPACITY = -6,  /* pe_cap < crisp_index_capacity() */
  CRISP_ERR_HIP = -7,       /* a HIP launch failed */
  CRISP_ERR_ALIGN = -8,     /* a pointer is not 16-byte aligned */
  CRISP_ERR_SCRATCH = -9    /* crisp_sparse_prefill_noalloc: the problem exceeds its static scratch */
} crisp_status;

typedef enum { CRISP_F32 = 0, CRISP_BF16 = 1 } crisp_dtype;

typedef enum {
  CRISP_SELECT_NOISE_FLOOR = 0, /* the method: Eq. 3-4 for VS heads, Alg. 4 for PE heads */
  CRISP_SELECT_KEEP_ALL = 1,    /* every head keeps its complete causal index set (dense check) */
  CRISP_SELECT_CUMULATIVE = 2   /* comparison: VS heads keep, per direction, the shortest prefix of
                                   blocks by (mass desc, index asc) covering gamma of the total mass,
                                   plus the first and last block (the cumulative-coverage rule the
                                   summary page's Introduction contrasts with Eq. 4); PE as mode 0 */
} crisp_select_mode;

typedef struct {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t seq_len;
  int32_t head_dim;
  int32_t dtype; /* crisp_dtype */
} crisp_shape;

/* Hyper-parameters (summary page, Methodology).  Rationals are num/den. */
typedef struct {
  int32_t block;     /* B: block size of the partition (Sink-Aware Thresholding; 128 on the pages) */
  int32_t w_sink;    /* anchor sinks: keys j < w_sink (Eq. 2; 128 on the pages) */
  int32_t w_local;   /* anchor local window: i - j < w_local (Eq. 2; 128 on the pages) */
  uint32_t tau_num, tau_den;     /* routing threshold tau_proxy: VS iff C_struct >= tau */
  uint32_t alpha_num, alpha_den; /* Eq. 4 multiplier alpha (1 is the calibration-free default) */
  uint32_t gamma_num, gamma_den; /* Alg. 4 coverage gamma of the PE index */
  int32_t select_mode;           /* crisp_select_mode */
} crisp_config;

/* Optional relative-position bias added to the attention logits of the proxy,
 * the sparse and the dense attention (not to the pooled PE map):
 * logit(i, j) += values[h][t] when i - j == offsets[h][t].  Device arrays
 * [BH][count]; count 0..8; offsets of one head should be distinct, negative
 * offsets never match.  Pass NULL (or count 0) for none. */
typedef struct {
  int32_t count;
  const int32_t* offsets;
  const float* values;
} crisp_rel_bias;

/* Routing results and index sets, all caller-owned device memory.
 * crisp_route writes route, cstruct_num, mass_v, mass_s and mass_total;
 * crisp_select_indices reads those and writes the lists;
 * crisp_sparse_prefill reads route and the lists. */
typedef struct {
  uint8_t* route;       /* [BH] 1 = VS, 0 = PE */
  int64_t* cstruct_num; /* [BH] anchor mass in fixed point: C_struct = cstruct_num / (qrows * 2^40) */
  int64_t* mass_v;      /* [BH][N_b] vertical mass of key block b (Alg. 3 column scores, block-pooled) */
  int64_t* mass_s;      /* [BH][N_b] slash mass of offset block b = (i - j) / B (diagonal scores, pooled) */
  int64_t* mass_total;  /* [BH] total proxy mass (= sum of mass_v = sum of mass_s) */
  int32_t* vs_count;    /* [BH][2] number of vertical and slash blocks (0, 0 for PE heads) */
  int32_t* vs_vertical; /* [BH][N_b] selected key blocks, ascending */
  int32_t* vs_slash;    /* [BH][N_b] selected offset blocks, ascending */
  int32_t* pe_rowptr;   /* [BH][N_b + 1] CSR row pointers per query block (all 0 for VS heads) */
  int32_t* pe_col;      /* [BH][pe_cap] CSR key blocks, ascending within each query block */
  int64_t pe_cap;       /* per-head capacity of pe_col, >= crisp_index_capacity() */
} crisp_index_sets;

/* Scratch bytes needed by crisp_route, crisp_select_indices,
 * crisp_sparse_prefill, crisp_dense_prefill and crisp_route_jsd for this
 * shape (0 if the arguments are invalid). */
size_t crisp_workspace_size(const crisp_shape* shape, const crisp_config* cfg);

/* Per-head capacity pe_col needs: N_b (N_b + 1) / 2 (-1 if invalid). */
int64_t crisp_index_capacity(const crisp_shape* shape, const crisp_config* cfg);

/* Alg. 2 with Eq. 2.  Proxy scores z = (q . k) / sqrt(d) (+ bias) of the last
 * query block against keys j <= i, post-softmax map A, block masses by column
 * (j / B) and by diagonal ((i - j) / B), C_struct over the anchor set
 * {j < w_sink} U {i - j < w_local}, and route = VS iff C_struct >= tau.
 * Reads q, k, bias; writes idx->route, cstruct_num, mass_v, mass_s, mass_total. */
crisp_status crisp_route(const crisp_shape* shape, const crisp_config* cfg, const void* q, const void* k,
                         const crisp_rel_bias* bias, void* ws, size_t ws_bytes, crisp_index_sets* idx,
                         void* stream);

/* Alg. 3 / Eq. 3-4 for VS heads: per direction, keep blocks 0 and N_b - 1 and
 * every middle block whose mass exceeds alpha times the mean middle mass.
 * Alg. 4 for PE heads: block means of Q and K, softmax of their scores over
 * key blocks kb <= qb, flatten, normalise, order by (mass desc, index
 * qb * N_b + kb asc), keep the shortest prefix covering gamma of the total,
 * plus every diagonal block (qb, qb).  Reads q, k (PE heads) and the routing
 * outputs in idx; writes vs_count, vs_vertical, vs_slash, pe_rowptr, pe_col. */
crisp_status crisp_select_indices(const crisp_shape* shape, const crisp_config* cfg, const void* q,
                                  const void* k, void* ws, size_t ws_bytes, crisp_index_sets* idx,
                                  void* stream);

/* Alg. 1 attention step: o = softmax over the allowed keys of (q . k)/sqrt(d)
 * + bias, times v.  Allowed (i, j), always with j <= i:
 *   VS head: key block j / B in vs_vertical, or offset block (i - j) / B in vs_slash;
 *   PE head: key block j / B listed in the PE row of query block i / B.
 * idx may come from crisp_select_indices or from the caller; either way its lists
 * must be ascending with entries in [0, N_b), vs_count at most N_b, pe_rowptr
 * non-decreasing from 0 with pe_rowptr[N_b] <= pe_cap, and every query row needs at
 * least one allowed key (the selection always keeps offset block 0 of a VS head and
 * the diagonal block of every PE row).  These device-side contents are read as
 * given, not checked.
 * Reads q, k, v, bias, idx; writes o. */
crisp_status crisp_sparse_prefill(const crisp_shape* shape, const crisp_config* cfg, const void* q,
                                  const void* k, const void* v, const crisp_rel_bias* bias,
                                  const crisp_index_sets* idx, void* ws, size_t ws_bytes, void* o,
                                  void* stream);

/* Full causal attention: the dense baseline the sparse path is measured
 * against.  On the CRISP summary page the comparator is exact full attention
 * computed with FlashAttention (Results: the legend of Table 2, and the
 * attention-only latencies of Latency Scaling, Table 4, quoted as speedups
 * over it).  Here it is the same tile engine as crisp_sparse_prefill with every
 * causal key tile listed, so the two differ only in the tiles they visit.
 * Reads q, k, v, bias; uses ws as scratch; writes o. */
crisp_status crisp_dense_prefill(const crisp_shape* shape, const crisp_config* cfg, const void* q,
                                 const void* k, const void* v, const crisp_rel_bias* bias, void* ws,
                                 size_t ws_bytes, void* o, void* stream);

/* crisp_sparse_prefill without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory around the call (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same operation, arguments, kernels and results (bit for bit) as
 * crisp_sparse_prefill; its scratch (key-tile lists, V^T, work-queue counters)
 * lives in a static device array of 128 MiB that the library holds on every
 * GPU it runs on until the process ends.  Problems whose attention scratch
 * exceeds 128 MiB are refused with CRISP_ERR_SCRATCH before anything is
 * enqueued: with bf16, head_dim 128 and block 128 the scratch is about
 * 2 * n_kv_heads * head_dim * seq_len bytes (V^T) plus the tile lists, so
 * 8 KV heads fit up to about 60K tokens.  The array keeps the last call's
 * contents; every call writes all it reads.  Calls share the one array per
 * GPU: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.  The first call on a
 * device looks up that device's copy of the array (no allocation). */
crisp_status crisp_sparse_prefill_noalloc(const crisp_shape* shape, const crisp_config* cfg, const void* q,
                                          const void* k, const void* v, const crisp_rel_bias* bias,
                                          const crisp_index_sets* idx, void* o, void* stream);

/* Where crisp_sparse_prefill keeps, inside ws, the key-tile lists it builds
 * from the index sets: the per-query-block tile iterator of Alg. 1's attention
 * step (summary page, Algorithm Overview), with the band rule of the selected
 * slash blocks (Methodology, Alg. 3).  After the call's stream has completed
 * the lists stay in ws until the next call that uses ws; this lets a caller
 * inspect them.  For query block qb the list holds the key blocks kb <= qb
 * that the attention visits, ascending, each with a mask mode:
 *   1 lower triangle of the tile (r >= c: offsets (qb - kb) B + r - c in
 *     slash block qb - kb, or the causal part of the diagonal tile),
 *   2 upper triangle (r < c: slash block qb - kb - 1),
 *   3 the whole tile (a vertical block, or a PE block below the diagonal).
 * Layout: list_offset is the byte offset in ws of int32 [n_lists][list_stride]
 * with the list of query block qb starting at element qb (qb + 1) / 2;
 * count_offset the byte offset of int32 [n_lists][N_b], the list lengths.
 * pair_lists = 1 (bf16, head_dim 128, block 128): one list per pair of query
 * heads of a KV group, list l = kv * ceil(G / 2) + w for flattened KV head kv
 * (batch * n_kv_heads + kv head) and pair w = query heads 2w, 2w + 1 of the
 * group; entry = kb | mode(2w) << 24 | mode(2w + 1) << 26, a mode 0 where that
 * head does not visit the tile (and for the missing second head of an odd G).
 * pair_lists = 0 (other shapes): one list per flattened query head, entry =
 * kb | mode << 28. */
typedef struct {
  int64_t list_offset;
  int64_t count_offset;
  int64_t list_stride; /* N_b (N_b + 1) / 2 */
  int32_t n_lists;
  int32_t pair_lists;
} crisp_tile_layout;

crisp_status crisp_tile_layout_of(const crisp_shape* shape, const crisp_config* cfg, crisp_tile_layout* out);

/* The divergence router the pages contrast with C_struct (summary page,
 * Motivation: a second, pooled estimate of the head's attention, its
 * Jensen-Shannon divergence from the per-query one, VS above a threshold).
 * Run after crisp_route on the same idx: it reads idx->mass_v and
 * idx->mass_total (the per-query estimate P_b = mass_v[b] / mass_total, the
 * proxy map pooled after the softmax) and q, k.  The pooled estimate Q is the
 * softmax over key blocks of fl(Qbar . Kbar_b) * c, with Qbar the mean of the
 * last query block's rows and Kbar_b the mean of key block b (fp32 sums in
 * row order; the last row of the PE path's pooled map), in the same 2^40
 * fixed point.  JSD = (KL(P||M) + KL(Q||M)) / 2, M = (P + Q) / 2, natural log,
 * with per-block terms t_b computed in fp64 and summed as rne(t_b 2^52).
 * Writes, per head (BH entries):
 *   jsd[h]       int64 J with JSD = J * 2^-53 (nats)
 *   route_jsd[h] 1 (VS) iff tau_den * J >= tau_num * 2^53, i.e. JSD >= tau
 *   pooled[h][b] optional ([BH][N_b] int64, may be NULL): the quantised pooled
 *                estimate rne(Q_b 2^40)
 * Uses ws as scratch (it may overwrite what crisp_route left there; the
 * routing outputs live in idx).  tau_den = 0 gives CRISP_ERR_CONFIG; jsd and
 * pooled must be 8-byte aligned. */
crisp_status crisp_route_jsd(const crisp_shape* shape, const crisp_config* cfg, uint32_t tau_num,
                             uint32_t tau_den, const void* q, const void* k, const crisp_index_sets* idx,
                             void* ws, size_t ws_bytes, uint8_t* route_jsd, int64_t* jsd, int64_t* pooled,
                             void* stream);

/* Static description of a status code. */
const char* crisp_status_string(crisp_status status);

#ifdef __cplusplus
}
#endif

#endif /* CRISP_H */
