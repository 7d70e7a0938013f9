// C ABI of the MoBA prefill library: argument checks, the per-call plan,
// workspace carving, stage ordering and optional per-stage HIP-event timing.
// The library allocates no device memory; every launch goes on the caller's
// stream and nothing here synchronises the device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "moba_plan.h"

namespace moba {

// The selection when every row keeps all of its past blocks (pool_gate.hip).
hipError_t launch_forced_sel(const Plan& p, const int32_t* cu_dev, const Work& w, int32_t* sel,
                             hipStream_t s);

static thread_local char g_err[512] = "";

static moba_status_t fail(moba_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int gcd_int(int a, int b) {
  while (b) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

int64_t max_grid_items(const Plan& p, bool backward) {
  int64_t m = 256;                                          // set-up
  auto take = [&](int64_t groups, int threads) { m = std::max(m, groups * threads); };
  if (p.block == 0) {                                       // dense causal attention
    take(pad8(dense_tile_count(p)), kAttnThreads);
    return m;
  }
  const bool w4 = p.dtype == MOBA_DTYPE_BF16 && p.d == 128;
  take((p.nb + 255) / 256, 256);                            // block table
  take(p.nb * p.hkv, 256);                                  // pool
  if (p.ks > 0) {
    take(pad8(gate_tile_count(p)), 64 * kGateWaves);        // gate passes
    take((int64_t)p.nseq * p.hkv, 256);                     // gate bound
    take(pad8(p.nb) * p.hkv, 512);                          // route count / scatter
    take((p.nlists + 3) / 4, 256);                          // route list scans
    take(pad8(tile_bound(p, p.sel_rows)), w4 ? 64 * kSelWaves : kAttnThreads);
  }
  take(w4 ? pad8(self4_tile_count(p)) : pad8(self8_tile_count(p)),
       w4 ? 64 * kSelWaves : kAttnThreads);
  if (backward) {
    const int64_t rows = p.T * p.hq;
    take((rows + 256 / (p.d / 8) - 1) / (256 / (p.d / 8)), 256);            // Delta
    if (p.ks > 0)                                                           // dQ selected
      take(pad8(tile_bound(p, p.sel_rows)), w4 ? 64 * kSelWaves : kAttnThreads);
    take(w4 ? pad8(self4_tile_count(p)) : pad8(self8_tile_count(p)),        // dQ self
         w4 ? 64 * kSelWaves : kAttnThreads);
    if (w4)
      take(pad8(p.nb * p.hkv) * tiles_per_block(p, kDkvWaves * 32), 64 * kDkvWaves);
    else
      take(p.nb * p.hkv * tiles_per_block(p, kBkvWaves * 32), 64 * kBkvWaves);
  }
  return m;
}

moba_status_t make_plan(const int32_t* cu, int32_t nseq, const moba_shape_t* shape,
                        int32_t block, int32_t topk, bool need_block, Plan* p, char* err,
                        size_t errlen) {
  (void)err;
  (void)errlen;
  if (!shape) return fail(MOBA_ERR_INVALID_ARG, "shape is NULL");
  if (!cu) return fail(MOBA_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
  if (nseq < 0) return fail(MOBA_ERR_INVALID_ARG, "num_seqs < 0");
  if (cu[0] != 0) return fail(MOBA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
  for (int32_t n = 0; n < nseq; ++n)
    if (cu[n + 1] < cu[n]) return fail(MOBA_ERR_INVALID_ARG, "cu_seqlens decreases at %d", n);
  if (shape->num_q_heads < 1 || shape->num_kv_heads < 1)
    return fail(MOBA_ERR_INVALID_ARG, "head counts must be >= 1");
  if (shape->num_q_heads % shape->num_kv_heads)
    return fail(MOBA_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (shape->head_dim != 64 && shape->head_dim != 128)
    return fail(MOBA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", shape->head_dim);
  if (shape->dtype != MOBA_DTYPE_F32 && shape->dtype != MOBA_DTYPE_BF16)
    return fail(MOBA_ERR_UNSUPPORTED, "dtype %d not supported", shape->dtype);
  if (need_block) {
    if (block < 1) return fail(MOBA_ERR_INVALID_ARG, "block_size must be >= 1");
    if (block % 64) return fail(MOBA_ERR_UNSUPPORTED, "block_size must be a multiple of 64");
    if (topk < 1) return fail(MOBA_ERR_INVALID_ARG, "topk must be >= 1");
    if (topk - 1 > kMaxSelected)
      return fail(MOBA_ERR_UNSUPPORTED, "topk - 1 must be <= %d", kMaxSelected);
  }
  Plan& P = *p;
  P = Plan();
  P.nseq = nseq;
  P.T = cu[nseq];
  P.hq = shape->num_q_heads;
  P.hkv = shape->num_kv_heads;
  P.d = shape->head_dim;
  P.dtype = shape->dtype;
  P.group = P.hq / P.hkv;
  P.hg = gcd_int(P.group, kGateWaves);
  P.block = need_block ? block : 0;
  P.topk = need_block ? topk : 1;
  P.ks = P.topk - 1;
  float sc = shape->softmax_scale;
  P.scale = (sc > 0.f && isfinite(sc)) ? sc : 1.0f / sqrtf((float)P.d);
  if (P.T * P.hq >= (int64_t(1) << 31))
    return fail(MOBA_ERR_UNSUPPORTED, "T * num_q_heads must be < 2^31");
  if (P.T * P.hq * (int64_t)P.ks >= (int64_t(1) << 31))
    return fail(MOBA_ERR_UNSUPPORTED, "T * num_q_heads * (topk - 1) must be < 2^31");
  for (int32_t n = 0; n < nseq; ++n) {
    const int64_t len = (int64_t)cu[n + 1] - cu[n];
    if (len > P.max_len) P.max_len = len;
    if (!need_block) continue;
    const int64_t nbn = (len + block - 1) / block;
    P.nb += nbn;
    if (nbn > P.max_nb) P.max_nb = (int32_t)nbn;
    P.tri += (int64_t)P.hkv * nbn * (nbn - 1) / 2;
    for (int64_t i = 0; i < nbn; ++i) {
      const int64_t li = std::min((int64_t)block, len - i * block);
      P.nentries += li * P.hq * std::min((int64_t)P.ks, i);
    }
  }
  if (need_block && P.ks > 0) {
    if (P.max_nb > kMaxBlocksPerSeq)
      return fail(MOBA_ERR_UNSUPPORTED, "a sequence has more than %d blocks", kMaxBlocksPerSeq);
    if (P.tri >= (int64_t(1) << 31))
      return fail(MOBA_ERR_UNSUPPORTED, "routing histogram too large");
  }
  P.nlists = P.nb * P.hkv;
  P.sel_rows = (P.dtype == MOBA_DTYPE_BF16 && P.d == 128) ? kSelRowsPerTile : kRowsPerTile;
  P.span = need_block ? std::min((int64_t)P.block, P.max_len) : P.max_len;
  if (max_grid_items(P, false) > kMaxGridItems)
    return fail(MOBA_ERR_UNSUPPORTED, "this batch needs a launch grid of %lld work-items, more "
                "than HIP allows (many short sequences with a long one?)",
                (long long)max_grid_items(P, false));

  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const int64_t rows = P.T * P.hq;
  P.off_blk_base = take(sizeof(int32_t) * (nseq + 1));
  P.off_tri_base = take(sizeof(int32_t) * (nseq + 1));
  P.off_blk_seq = take(sizeof(int32_t) * P.nb);
  P.off_blk_local = take(sizeof(int32_t) * P.nb);
  P.off_kbar = take(sizeof(float) * P.nb * P.hkv * P.d);
  P.off_kbar_split =
      take(P.dtype == MOBA_DTYPE_BF16 ? sizeof(bf16) * 3 * P.nb * P.hkv * P.d : 0);
  P.off_kbar_err = take(sizeof(float) * P.nb * P.hkv);
  P.off_gate_bound = take(sizeof(float) * nseq * P.hkv);
  // the gate's tiling: 8 waves x 32 rows, HG heads of one group side by side
  P.gate_tiles = need_block ? gate_tile_count(P) : 0;
  P.off_gate_flags = take(P.gate_tiles);
  if (P.ks > 0) {
    P.off_sel = take(sizeof(int32_t) * rows * P.ks);
    P.off_hist = take(sizeof(int32_t) * P.tri);
    P.off_chunk_off = take(sizeof(int32_t) * P.tri);
    P.off_list_count = take(sizeof(int32_t) * P.nlists);
    P.off_list_offsets = take(sizeof(int32_t) * (P.nlists + 1));
    P.off_tile_offsets = take(sizeof(int32_t) * (P.nlists + 1));
    P.off_entries = take(sizeof(int32_t) * P.nentries);
    const size_t part = (P.dtype == MOBA_DTYPE_BF16) ? sizeof(f16) : sizeof(float);
    P.off_o_sel = take(part * rows * P.ks * P.d);
    P.off_lse_sel = take(sizeof(float) * rows * P.ks);
  }
  P.total = off;
  return MOBA_OK;
}

Work carve(const Plan& p, void* base) {
  char* b = (char*)base;
  Work w = {};
  w.blk_base = (int32_t*)(b + p.off_blk_base);
  w.tri_base = (int32_t*)(b + p.off_tri_base);
  w.blk_seq = (int32_t*)(b + p.off_blk_seq);
  w.blk_local = (int32_t*)(b + p.off_blk_local);
  w.kbar = (float*)(b + p.off_kbar);
  w.kbar_split = (bf16*)(b + p.off_kbar_split);
  w.kbar_err = (float*)(b + p.off_kbar_err);
  w.gate_bound = (float*)(b + p.off_gate_bound);
  w.gate_flags = (uint8_t*)(b + p.off_gate_flags);
  if (p.ks > 0) {
    w.sel = (int32_t*)(b + p.off_sel);
    w.hist = (int32_t*)(b + p.off_hist);
    w.chunk_off = (int32_t*)(b + p.off_chunk_off);
    w.list_count = (int32_t*)(b + p.off_list_count);
    w.list_offsets = (int32_t*)(b + p.off_list_offsets);
    w.tile_offsets = (int32_t*)(b + p.off_tile_offsets);
    w.entries = (int32_t*)(b + p.off_entries);
    w.o_sel = (void*)(b + p.off_o_sel);
    w.lse_sel = (float*)(b + p.off_lse_sel);
  }
  return w;
}

// ---------------------------------------------------------------------------
// Optional per-stage timing.
enum { ST_POOL = 0, ST_GATE, ST_ROUTE, ST_SELF, ST_SELECTED, ST_MERGE, ST_DENSE, ST_DECODE,
       ST_KBAR, ST_BACKWARD, ST_SLAB, ST_COUNT };
static const char* kStageNames[ST_COUNT] = {"pool",       "gate",   "route",
                                            "attn_self",  "attn_selected", "merge",
                                            "attn_dense", "decode", "kbar_append",
                                            "backward",   "slab_copy"};
constexpr int kMaxTimed = 4096;

struct Timing {
  std::mutex mu;
  bool enabled = false;
  bool created = false;
  hipEvent_t ev0[kMaxTimed], ev1[kMaxTimed];
  int stage[kMaxTimed];
  int used = 0;
};
static Timing g_timing;

struct StageScope {
  int slot = -1;
  hipStream_t s;
  StageScope(int st, hipStream_t stream) : s(stream) {
    if (!g_timing.enabled) return;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (!g_timing.enabled || g_timing.used >= kMaxTimed) return;
    slot = g_timing.used++;
    g_timing.stage[slot] = st;
    (void)hipEventRecord(g_timing.ev0[slot], s);
  }
  ~StageScope() {
    if (slot >= 0) (void)hipEventRecord(g_timing.ev1[slot], s);
  }
};

static moba_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOBA_OK;
  return fail(MOBA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Checks shared by the decode entry points: shape, block size, top-k, the
// cache lengths cu_k and the new-row counts cu_q (each new row is one of the
// last tokens of its sequence's cache), and the pooled-key cache capacity.
struct DecodePlan {
  int64_t Tq = 0, rows = 0;
  int ks = 0, nseg = 0;
  size_t off_sel = 0, off_part_o = 0, off_part_lse = 0, total = 0;
};

static moba_status_t check_shape(const moba_shape_t* shape) {
  if (!shape) return fail(MOBA_ERR_INVALID_ARG, "shape is NULL");
  if (shape->num_q_heads < 1 || shape->num_kv_heads < 1)
    return fail(MOBA_ERR_INVALID_ARG, "head counts must be >= 1");
  if (shape->num_q_heads % shape->num_kv_heads)
    return fail(MOBA_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (shape->head_dim != 64 && shape->head_dim != 128)
    return fail(MOBA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", shape->head_dim);
  if (shape->dtype != MOBA_DTYPE_F32 && shape->dtype != MOBA_DTYPE_BF16)
    return fail(MOBA_ERR_UNSUPPORTED, "dtype %d not supported", shape->dtype);
  return MOBA_OK;
}

static moba_status_t check_cu(const int32_t* cu, int32_t nseq, const char* name) {
  if (!cu) return fail(MOBA_ERR_INVALID_ARG, "%s (host) is NULL", name);
  if (cu[0] != 0) return fail(MOBA_ERR_INVALID_ARG, "%s[0] must be 0", name);
  for (int32_t n = 0; n < nseq; ++n)
    if (cu[n + 1] < cu[n]) return fail(MOBA_ERR_INVALID_ARG, "%s decreases at %d", name, n);
  return MOBA_OK;
}

static moba_status_t check_block(int32_t block, int32_t max_blocks, const int32_t* cu_k,
                                 int32_t nseq) {
  if (block < 1) return fail(MOBA_ERR_INVALID_ARG, "block_size must be >= 1");
  if (block % 64) return fail(MOBA_ERR_UNSUPPORTED, "block_size must be a multiple of 64");
  if (max_blocks < 0) return fail(MOBA_ERR_INVALID_ARG, "max_blocks < 0");
  for (int32_t n = 0; n < nseq; ++n) {
    const int64_t len = (int64_t)cu_k[n + 1] - cu_k[n];
    if ((len + block - 1) / block > max_blocks)
      return fail(MOBA_ERR_INVALID_ARG, "sequence %d has %lld cached tokens, more than max_blocks "
                  "* block_size", n, (long long)len);
  }
  return MOBA_OK;
}

static moba_status_t make_decode_plan(const int32_t* cu_q, const int32_t* cu_k, int32_t nseq,
                                      const moba_shape_t* shape, int32_t block, int32_t topk,
                                      int32_t max_blocks, DecodePlan* dp) {
  if (nseq < 0) return fail(MOBA_ERR_INVALID_ARG, "num_seqs < 0");
  moba_status_t st = check_shape(shape);
  if (st != MOBA_OK) return st;
  if ((st = check_cu(cu_q, nseq, "cu_q")) != MOBA_OK) return st;
  if ((st = check_cu(cu_k, nseq, "cu_k")) != MOBA_OK) return st;
  if ((st = check_block(block, max_blocks, cu_k, nseq)) != MOBA_OK) return st;
  if (topk < 1) return fail(MOBA_ERR_INVALID_ARG, "topk must be >= 1");
  if (topk - 1 > kMaxSelected)
    return fail(MOBA_ERR_UNSUPPORTED, "topk - 1 must be <= %d", kMaxSelected);
  for (int32_t n = 0; n < nseq; ++n)
    if (cu_q[n + 1] - cu_q[n] > cu_k[n + 1] - cu_k[n])
      return fail(MOBA_ERR_INVALID_ARG, "sequence %d has more new rows than cached tokens", n);
  DecodePlan& P = *dp;
  P = DecodePlan();
  P.Tq = cu_q[nseq];
  P.rows = P.Tq * shape->num_q_heads;
  P.ks = topk - 1;
  P.nseg = decode_segments(block);
  const int64_t items = P.rows * (P.ks + 1) * P.nseg;
  if (items * shape->head_dim >= ((int64_t)1 << 40))
    return fail(MOBA_ERR_UNSUPPORTED, "too many new rows for one call");
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  P.off_sel = take(sizeof(int32_t) * P.rows * (P.ks > 0 ? P.ks : 1));
  P.off_part_o = take(sizeof(float) * items * shape->head_dim);
  P.off_part_lse = take(sizeof(float) * items);
  P.total = off;
  return MOBA_OK;
}

// Backward workspace: the forward's block tables and routing buffers (the
// lists are rebuilt from the forward's selection), then the selected-block dQ
// parts in place of the forward's partial outputs (fp32, indexed like them by
// row * ks + slot) and Delta per row.
struct BwdLayout {
  size_t off_delta = 0, off_lse2 = 0, off_dq_sel = 0, total = 0;
};

static BwdLayout backward_layout(const Plan& p) {
  BwdLayout l;
  size_t off = p.ks > 0 ? p.off_o_sel : p.total;
  l.off_dq_sel = off;
  off = align256(off + sizeof(float) * (size_t)(p.T * p.hq) * p.ks * p.d);
  l.off_delta = off;
  off = align256(off + sizeof(float) * (size_t)(p.T * p.hq));
  l.off_lse2 = off;                                // the forward's LSE times log2(e)
  off = align256(off + sizeof(float) * (size_t)(p.T * p.hq));
  l.total = std::max(off, p.total);
  return l;
}

// The stages of one forward call on a validated plan and a workspace of at
// least plan.total bytes (nothing in it needs to start at zero: every word a
// kernel reads is written earlier in the same call).
static moba_status_t forward_enqueue(const Plan& p, const void* q, const void* k, const void* v,
                                     const int32_t* cu_dev, void* out, void* workspace,
                                     int32_t* sel_out, float* lse_out, hipStream_t s) {
  (void)hipGetLastError();
  Work w = carve(p, workspace);
  int32_t* sel = sel_out ? sel_out : w.sel;
  hipError_t e = hipSuccess;
  if (p.max_nb <= p.topk && pad8(dense_tile_count(p)) * kAttnThreads <= kMaxGridItems) {
    // No sequence has more than topk blocks, so no row has more than topk - 1 past
    // blocks and every row keeps all of them: the attended set is the own block up
    // to the row plus every earlier key, which is causal attention over the whole
    // sequence. That runs as the dense causal kernel, and the selection is the
    // forced one (MoBA README, FAQ of issue #27: moba_topk - 1 capped by the number
    // of complete past blocks). Pool, gate and route have nothing to decide; the
    // block table is built only to write the selection when it is asked for.
    if (sel_out && p.ks > 0) {
      e = launch_setup(p, cu_dev, w, s);
      if (e != hipSuccess) return hip_status(e, "setup");
      StageScope t(ST_GATE, s);
      e = launch_forced_sel(p, cu_dev, w, sel_out, s);
    }
    if (e != hipSuccess) return hip_status(e, "forced selection");
    {
      StageScope t(ST_DENSE, s);
      e = launch_attn_dense(p, q, k, v, cu_dev, out, lse_out, s);
    }
    if (e != hipSuccess) return hip_status(e, "causal attention");
    g_err[0] = 0;
    return MOBA_OK;
  }
  e = launch_setup(p, cu_dev, w, s);
  if (e != hipSuccess) return hip_status(e, "setup");
  {
    StageScope t(ST_POOL, s);
    e = launch_pool(p, k, cu_dev, w, w.kbar, s);
  }
  if (e != hipSuccess) return hip_status(e, "pool");
  if (p.ks > 0) {
    {
      StageScope t(ST_GATE, s);
      e = launch_gate(p, q, cu_dev, w, sel, s);
    }
    if (e != hipSuccess) return hip_status(e, "gate");
    {
      StageScope t(ST_ROUTE, s);
      e = launch_route(p, sel, cu_dev, w, p.sel_rows, w.list_offsets, w.entries, s);
    }
    if (e != hipSuccess) return hip_status(e, "route");
    {
      StageScope t(ST_SELECTED, s);
      e = launch_attn_selected(p, q, k, v, cu_dev, w, s);
    }
    if (e != hipSuccess) return hip_status(e, "selected-block attention");
  }
  {
    StageScope t(ST_SELF, s);
    e = launch_attn_self(p, q, k, v, cu_dev, w, out, lse_out, s);
  }
  if (e != hipSuccess) return hip_status(e, "self-block attention");
  g_err[0] = 0;
  return MOBA_OK;
}

// ---------------------------------------------------------------------------
// kv-group mode of the forward: one kv group (its G q heads and its k/v head) at a
// time. Every step of the method is independent per kv group (a row reads only
// its own kv head), so running the groups one after another computes the same
// rows; the group's heads are gathered into contiguous slabs, the usual stages
// run on a [T, G, D] / [T, 1, D] batch, and the slab's outputs are scattered
// back. The workspace then holds one group's buffers plus the slabs.
struct SlabLayout {
  Plan p;                       // the plan of one group's batch (G q heads, 1 kv head)
  size_t off_q = 0, off_k = 0, off_v = 0, off_out = 0, off_sel = 0, off_lse = 0, off_ws = 0;
  size_t total = 0;
};

static moba_status_t make_slab(const int32_t* cu, int32_t nseq, const moba_shape_t* shape,
                               int32_t block, int32_t topk, SlabLayout* L) {
  moba_shape_t one = *shape;
  one.num_q_heads = shape->num_q_heads / shape->num_kv_heads;
  one.num_kv_heads = 1;
  moba_status_t st = make_plan(cu, nseq, &one, block, topk, true, &L->p, nullptr, 0);
  if (st != MOBA_OK) return st;
  const Plan& p = L->p;
  const size_t e = p.dtype == MOBA_DTYPE_BF16 ? 2 : 4;
  const size_t T = (size_t)p.T;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L->off_q = take(T * p.hq * p.d * e);
  L->off_k = take(T * p.d * e);
  L->off_v = take(T * p.d * e);
  L->off_out = take(T * p.hq * p.d * e);
  L->off_sel = take(T * p.hq * (size_t)p.ks * 4);
  L->off_lse = take(T * p.hq * 4);
  L->off_ws = take(p.total);
  L->total = off;
  return MOBA_OK;
}

// The kv groups one after another: gather, forward, scatter (all on stream s).
static moba_status_t forward_by_group(const SlabLayout& L, const moba_shape_t* shape,
                                      const void* q, const void* k, const void* v,
                                      const int32_t* cu_dev, void* out, void* workspace,
                                      int32_t* sel_out, float* lse_out, hipStream_t s) {
  const Plan& p = L.p;
  const int G = p.hq, hkv = shape->num_kv_heads, hq = shape->num_q_heads;
  const int64_t e = p.dtype == MOBA_DTYPE_BF16 ? 2 : 4;
  const int64_t T = p.T, D = p.d;
  char* b = (char*)workspace;
  char *qs = b + L.off_q, *ks = b + L.off_k, *vs = b + L.off_v, *os = b + L.off_out;
  int32_t* sels = (int32_t*)(b + L.off_sel);
  float* lses = (float*)(b + L.off_lse);
  for (int g = 0; g < hkv; ++g) {
    hipError_t e1;
    {
      StageScope t(ST_SLAB, s);
      e1 = launch_copy_rows((const char*)q + g * G * D * e, hq * D * e, qs, G * D * e, T, G * D * e, s);
      if (e1 == hipSuccess)
        e1 = launch_copy_rows((const char*)k + g * D * e, hkv * D * e, ks, D * e, T, D * e, s);
      if (e1 == hipSuccess)
        e1 = launch_copy_rows((const char*)v + g * D * e, hkv * D * e, vs, D * e, T, D * e, s);
    }
    if (e1 != hipSuccess) return hip_status(e1, "kv-group gather");
    moba_status_t st = forward_enqueue(p, qs, ks, vs, cu_dev, os, b + L.off_ws,
                                       (sel_out && p.ks > 0) ? sels : nullptr,
                                       lse_out ? lses : nullptr, s);
    if (st != MOBA_OK) return st;
    {
      StageScope t(ST_SLAB, s);
      e1 = launch_copy_rows(os, G * D * e, (char*)out + g * G * D * e, hq * D * e, T, G * D * e, s);
      if (e1 == hipSuccess && sel_out && p.ks > 0)
        e1 = launch_copy_rows(sels, (int64_t)G * p.ks * 4, sel_out + (int64_t)g * G * p.ks,
                              (int64_t)hq * p.ks * 4, T, (int64_t)G * p.ks * 4, s);
      if (e1 == hipSuccess && lse_out)
        e1 = launch_copy_rows(lses, (int64_t)G * 4, lse_out + (int64_t)g * G, (int64_t)hq * 4,
                              T, (int64_t)G * 4, s);
    }
    if (e1 != hipSuccess) return hip_status(e1, "kv-group scatter");
  }
  g_err[0] = 0;
  return MOBA_OK;
}

// ---------------------------------------------------------------------------
// Static scratch for moba_forward_noalloc: a device array in this code object,
// one copy per GPU, alive until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// the device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is handed to the kernels.
constexpr size_t kScratchBytes = MOBA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static moba_status_t scratch_pointer(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOBA_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p || (uintptr_t)p % 256)
      return fail(MOBA_ERR_HIP, "static scratch has an unusable address %p", p);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOBA_OK;
}

}  // namespace moba

using namespace moba;

extern "C" {

int32_t moba_abi_version(void) { return MOBA_ABI_VERSION; }

const char* moba_last_error(void) { return g_err; }

size_t moba_workspace_bytes(const int32_t* cu_seqlens_host, int32_t num_seqs,
                            const moba_shape_t* shape, int32_t block_size, int32_t topk) {
  Plan p;
  if (make_plan(cu_seqlens_host, num_seqs, shape, block_size, topk, true, &p, nullptr, 0) !=
      MOBA_OK)
    return 0;
  g_err[0] = 0;
  return p.total;
}

size_t moba_workspace_bytes_min(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                const moba_shape_t* shape, int32_t block_size, int32_t topk) {
  Plan p;
  const moba_status_t st =
      make_plan(cu_seqlens_host, num_seqs, shape, block_size, topk, true, &p, nullptr, 0);
  char msg[sizeof g_err];
  snprintf(msg, sizeof msg, "%s", g_err);
  size_t best = st == MOBA_OK ? p.total : 0;
  if (shape && shape->num_kv_heads > 1 && (st == MOBA_OK || st == MOBA_ERR_UNSUPPORTED)) {
    SlabLayout L;
    if (make_slab(cu_seqlens_host, num_seqs, shape, block_size, topk, &L) == MOBA_OK &&
        (best == 0 || L.total < best))
      best = L.total;
  }
  if (best == 0) {
    snprintf(g_err, sizeof g_err, "%s", msg);
    return 0;
  }
  g_err[0] = 0;
  return best;
}

moba_status_t moba_forward(const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                           int32_t num_seqs, const moba_shape_t* shape, int32_t block_size,
                           int32_t topk, void* out, void* workspace, size_t workspace_bytes,
                           int32_t* sel_out, float* lse_out, void* stream) {
  Plan p;
  moba_status_t st =
      make_plan(cu_seqlens_host, num_seqs, shape, block_size, topk, true, &p, nullptr, 0);
  // a batch over the size limits of one pass over all heads may still run by kv group
  const bool by_group_possible =
      (st == MOBA_OK || st == MOBA_ERR_UNSUPPORTED) && shape && shape->num_kv_heads > 1;
  if (st != MOBA_OK && !by_group_possible) return st;
  if (st == MOBA_OK && p.T == 0) {
    g_err[0] = 0;
    return MOBA_OK;
  }
  if (!q || !k || !v || !out || !cu_seqlens_dev)
    return fail(MOBA_ERR_INVALID_ARG, "q, k, v, out and cu_seqlens_dev must be non-NULL");
  if (!workspace) return fail(MOBA_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)workspace % 256) return fail(MOBA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  if (st == MOBA_OK && workspace_bytes >= p.total)
    return forward_enqueue(p, q, k, v, cu_seqlens_dev, out, workspace, sel_out, lse_out,
                           (hipStream_t)stream);
  char msg[sizeof g_err];
  snprintf(msg, sizeof msg, "%s", g_err);
  const moba_status_t full_st = st;
  const size_t full_total = st == MOBA_OK ? p.total : 0;
  if (by_group_possible) {
    SlabLayout L;
    if (make_slab(cu_seqlens_host, num_seqs, shape, block_size, topk, &L) == MOBA_OK) {
      if (workspace_bytes >= L.total)
        return forward_by_group(L, shape, q, k, v, cu_seqlens_dev, out, workspace, sel_out,
                                lse_out, (hipStream_t)stream);
      if (full_st == MOBA_OK)
        return fail(MOBA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu (all heads at once) "
                    "or %zu (one kv group at a time)", workspace_bytes, full_total, L.total);
      return fail(MOBA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu (one kv group at a "
                  "time)", workspace_bytes, L.total);
    }
  }
  if (full_st != MOBA_OK) {
    snprintf(g_err, sizeof g_err, "%s", msg);
    return full_st;
  }
  return fail(MOBA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
              full_total);
}

moba_status_t moba_forward_noalloc(const void* q, const void* k, const void* v,
                                   const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                                   int32_t num_seqs, const moba_shape_t* shape,
                                   int32_t block_size, int32_t topk, void* out,
                                   int32_t* sel_out, float* lse_out, void* stream) {
  Plan p;
  moba_status_t st =
      make_plan(cu_seqlens_host, num_seqs, shape, block_size, topk, true, &p, nullptr, 0);
  if (st != MOBA_OK) return st;
  if (p.total > kScratchBytes)
    return fail(MOBA_ERR_WORKSPACE, "this batch needs %zu bytes of workspace, more than the "
                "%zu bytes of the library's static scratch; use moba_forward", p.total,
                (size_t)kScratchBytes);
  if (p.T == 0) {
    g_err[0] = 0;
    return MOBA_OK;
  }
  if (!q || !k || !v || !out || !cu_seqlens_dev)
    return fail(MOBA_ERR_INVALID_ARG, "q, k, v, out and cu_seqlens_dev must be non-NULL");
  void* ws = nullptr;
  st = scratch_pointer(&ws);
  if (st != MOBA_OK) return st;
  return forward_enqueue(p, q, k, v, cu_seqlens_dev, out, ws, sel_out, lse_out,
                         (hipStream_t)stream);
}

moba_status_t moba_dense_causal_forward(const void* q, const void* k, const void* v,
                                        const int32_t* cu_seqlens_dev,
                                        const int32_t* cu_seqlens_host, int32_t num_seqs,
                                        const moba_shape_t* shape, void* out, float* lse_out,
                                        void* stream) {
  Plan p;
  moba_status_t st = make_plan(cu_seqlens_host, num_seqs, shape, 0, 1, false, &p, nullptr, 0);
  if (st != MOBA_OK) return st;
  if (p.T == 0) {
    g_err[0] = 0;
    return MOBA_OK;
  }
  if (!q || !k || !v || !out || !cu_seqlens_dev)
    return fail(MOBA_ERR_INVALID_ARG, "q, k, v, out and cu_seqlens_dev must be non-NULL");
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  hipError_t e;
  {
    StageScope t(ST_DENSE, s);
    e = launch_attn_dense(p, q, k, v, cu_seqlens_dev, out, lse_out, s);
  }
  if (e != hipSuccess) return hip_status(e, "dense causal attention");
  g_err[0] = 0;
  return MOBA_OK;
}

moba_status_t moba_attention_forward(int32_t mode, const void* q, const void* k, const void* v,
                                     const int32_t* cu_seqlens_dev,
                                     const int32_t* cu_seqlens_host, int32_t num_seqs,
                                     const moba_shape_t* shape, int32_t block_size,
                                     int32_t topk, void* out, void* workspace,
                                     size_t workspace_bytes, int32_t* sel_out, float* lse_out,
                                     void* stream) {
  if (mode == MOBA_MODE_SPARSE)
    return moba_forward(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs, shape, block_size,
                        topk, out, workspace, workspace_bytes, sel_out, lse_out, stream);
  if (mode == MOBA_MODE_FULL)
    return moba_dense_causal_forward(q, k, v, cu_seqlens_dev, cu_seqlens_host, num_seqs, shape,
                                     out, lse_out, stream);
  return fail(MOBA_ERR_INVALID_ARG, "mode %d is neither MOBA_MODE_SPARSE nor MOBA_MODE_FULL",
              mode);
}

size_t moba_decode_workspace_bytes(const int32_t* cu_q_host, const int32_t* cu_k_host,
                                   int32_t num_seqs, const moba_shape_t* shape,
                                   int32_t block_size, int32_t topk, int32_t max_blocks) {
  DecodePlan dp;
  if (make_decode_plan(cu_q_host, cu_k_host, num_seqs, shape, block_size, topk, max_blocks,
                       &dp) != MOBA_OK)
    return 0;
  g_err[0] = 0;
  return dp.total;
}

moba_status_t moba_kbar_append(const void* k_cache, const int32_t* cu_k_dev,
                               const int32_t* cu_k_host, const int32_t* prev_len_dev,
                               const int32_t* prev_len_host, int32_t num_seqs,
                               const moba_shape_t* shape, int32_t block_size, int32_t max_blocks,
                               float* kbar_cache, void* stream) {
  if (num_seqs < 0) return fail(MOBA_ERR_INVALID_ARG, "num_seqs < 0");
  moba_status_t st = check_shape(shape);
  if (st != MOBA_OK) return st;
  if ((st = check_cu(cu_k_host, num_seqs, "cu_k")) != MOBA_OK) return st;
  if ((st = check_block(block_size, max_blocks, cu_k_host, num_seqs)) != MOBA_OK) return st;
  if (!prev_len_host) return fail(MOBA_ERR_INVALID_ARG, "prev_len_host is NULL");
  int new_max = 0;
  for (int32_t n = 0; n < num_seqs; ++n) {
    const int64_t len = (int64_t)cu_k_host[n + 1] - cu_k_host[n];
    if (prev_len_host[n] < 0 || prev_len_host[n] > len)
      return fail(MOBA_ERR_INVALID_ARG, "prev_len[%d] = %d outside [0, %lld]", n,
                  prev_len_host[n], (long long)len);
    new_max = std::max(new_max, (int)(len / block_size - prev_len_host[n] / block_size));
  }
  if (new_max == 0) {
    g_err[0] = 0;
    return MOBA_OK;
  }
  if (!k_cache || !cu_k_dev || !prev_len_dev || !kbar_cache)
    return fail(MOBA_ERR_INVALID_ARG, "k_cache, cu_k_dev, prev_len_dev and kbar_cache must be "
                "non-NULL");
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  hipError_t e;
  {
    StageScope t(ST_KBAR, s);
    e = launch_kbar_append(k_cache, cu_k_dev, prev_len_dev, num_seqs, shape->num_kv_heads,
                           shape->head_dim, shape->dtype, block_size, max_blocks, new_max,
                           kbar_cache, s);
  }
  if (e != hipSuccess) return hip_status(e, "pooled-key append");
  g_err[0] = 0;
  return MOBA_OK;
}

moba_status_t moba_decode_forward(const void* q_new, const void* k_cache, const void* v_cache,
                                  const int32_t* cu_q_dev, const int32_t* cu_q_host,
                                  const int32_t* cu_k_dev, const int32_t* cu_k_host,
                                  int32_t num_seqs, const moba_shape_t* shape,
                                  int32_t block_size, int32_t topk, const float* kbar_cache,
                                  int32_t max_blocks, void* out, void* workspace,
                                  size_t workspace_bytes, int32_t* sel_out, float* lse_out,
                                  void* stream) {
  DecodePlan dp;
  moba_status_t st = make_decode_plan(cu_q_host, cu_k_host, num_seqs, shape, block_size, topk,
                                      max_blocks, &dp);
  if (st != MOBA_OK) return st;
  if (dp.rows == 0) {
    g_err[0] = 0;
    return MOBA_OK;
  }
  if (!q_new || !k_cache || !v_cache || !cu_q_dev || !cu_k_dev || !out ||
      (dp.ks > 0 && !kbar_cache))
    return fail(MOBA_ERR_INVALID_ARG, "q_new, k_cache, v_cache, cu_q_dev, cu_k_dev, out and "
                "(topk > 1) kbar_cache must be non-NULL");
  if (!workspace) return fail(MOBA_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)workspace % 256) return fail(MOBA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  if (workspace_bytes < dp.total)
    return fail(MOBA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                dp.total);
  char* b = (char*)workspace;
  DecodeArgs a = {};
  a.q = q_new;
  a.k = k_cache;
  a.v = v_cache;
  a.cu_q = cu_q_dev;
  a.cu_k = cu_k_dev;
  a.kbar = kbar_cache;
  a.max_blocks = max_blocks;
  a.nseq = num_seqs;
  a.hq = shape->num_q_heads;
  a.hkv = shape->num_kv_heads;
  a.block = block_size;
  a.ks = dp.ks;
  a.nseg = dp.nseg;
  a.rows = dp.rows;
  const float sc = shape->softmax_scale;
  const float scale = (sc > 0.f && isfinite(sc)) ? sc : 1.0f / sqrtf((float)shape->head_dim);
  a.scale_log2 = scale * kLog2e;
  a.sel = (dp.ks > 0 && sel_out) ? sel_out : (int32_t*)(b + dp.off_sel);
  a.part_o = (float*)(b + dp.off_part_o);
  a.part_lse = (float*)(b + dp.off_part_lse);
  a.out = out;
  a.lse_out = lse_out;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  hipError_t e;
  {
    StageScope t(ST_DECODE, s);
    e = launch_decode(a, shape->head_dim, shape->dtype, s);
  }
  if (e != hipSuccess) return hip_status(e, "decode");
  g_err[0] = 0;
  return MOBA_OK;
}

size_t moba_backward_workspace_bytes(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                     const moba_shape_t* shape, int32_t block_size,
                                     int32_t topk) {
  Plan p;
  if (make_plan(cu_seqlens_host, num_seqs, shape, block_size, topk, true, &p, nullptr, 0) !=
      MOBA_OK)
    return 0;
  g_err[0] = 0;
  return backward_layout(p).total;
}

moba_status_t moba_backward(const void* q, const void* k, const void* v, const void* out,
                            const float* lse, const void* dout, const int32_t* sel,
                            const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                            int32_t num_seqs, const moba_shape_t* shape, int32_t block_size,
                            int32_t topk, void* dq, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, void* stream) {
  Plan p;
  moba_status_t st =
      make_plan(cu_seqlens_host, num_seqs, shape, block_size, topk, true, &p, nullptr, 0);
  if (st != MOBA_OK) return st;
  if (p.T == 0) {
    g_err[0] = 0;
    return MOBA_OK;
  }
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !cu_seqlens_dev)
    return fail(MOBA_ERR_INVALID_ARG, "q, k, v, out, lse, dout, dq, dk, dv and cu_seqlens_dev "
                "must be non-NULL");
  if (p.ks > 0 && !sel) return fail(MOBA_ERR_INVALID_ARG, "sel is NULL (topk > 1)");
  if (max_grid_items(p, true) > kMaxGridItems)
    return fail(MOBA_ERR_UNSUPPORTED, "this batch needs a backward launch grid of %lld "
                "work-items, more than HIP allows", (long long)max_grid_items(p, true));
  if (!workspace) return fail(MOBA_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)workspace % 256) return fail(MOBA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  const BwdLayout bl = backward_layout(p);
  if (workspace_bytes < bl.total)
    return fail(MOBA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                bl.total);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  Work w = carve(p, workspace);
  char* b = (char*)workspace;
  float* delta = (float*)(b + bl.off_delta);
  float* lse2 = (float*)(b + bl.off_lse2);
  float* dq_sel = (float*)(b + bl.off_dq_sel);
  hipError_t e = launch_setup(p, cu_seqlens_dev, w, s);
  if (e != hipSuccess) return hip_status(e, "setup");
  if (p.ks > 0) {
    StageScope t(ST_ROUTE, s);
    e = launch_route(p, sel, cu_seqlens_dev, w, p.sel_rows, w.list_offsets, w.entries, s);
  }
  if (e != hipSuccess) return hip_status(e, "route");
  {
    StageScope t(ST_BACKWARD, s);
    e = launch_backward(p, q, k, v, out, lse, dout, cu_seqlens_dev, w, delta, lse2, dq_sel, dq,
                        dk, dv, s);
  }
  if (e != hipSuccess) return hip_status(e, "backward");
  g_err[0] = 0;
  return MOBA_OK;
}

moba_status_t moba_block_pool(const void* k, const int32_t* cu_seqlens_dev,
                              const int32_t* cu_seqlens_host, int32_t num_seqs,
                              const moba_shape_t* shape, int32_t block_size, float* kbar_out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  moba_status_t st =
      make_plan(cu_seqlens_host, num_seqs, shape, block_size, 1, true, &p, nullptr, 0);
  if (st != MOBA_OK) return st;
  if (p.T == 0) {
    g_err[0] = 0;
    return MOBA_OK;
  }
  if (!k || !kbar_out || !cu_seqlens_dev || !workspace)
    return fail(MOBA_ERR_INVALID_ARG, "k, kbar_out, cu_seqlens_dev and workspace must be non-NULL");
  if ((uintptr_t)workspace % 256) return fail(MOBA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  if (workspace_bytes < p.total)
    return fail(MOBA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                p.total);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  Work w = carve(p, workspace);
  hipError_t e = launch_setup(p, cu_seqlens_dev, w, s);
  if (e != hipSuccess) return hip_status(e, "setup");
  {
    StageScope t(ST_POOL, s);
    e = launch_pool(p, k, cu_seqlens_dev, w, kbar_out, s);
  }
  if (e != hipSuccess) return hip_status(e, "pool");
  g_err[0] = 0;
  return MOBA_OK;
}

moba_status_t moba_route_sizes(const int32_t* cu_seqlens_host, int32_t num_seqs,
                               const moba_shape_t* shape, int32_t block_size, int32_t topk,
                               int64_t* num_lists, int64_t* num_entries) {
  Plan p;
  moba_status_t st =
      make_plan(cu_seqlens_host, num_seqs, shape, block_size, topk, true, &p, nullptr, 0);
  if (st != MOBA_OK) return st;
  if (!num_lists || !num_entries) return fail(MOBA_ERR_INVALID_ARG, "output pointer is NULL");
  *num_lists = p.nlists;
  *num_entries = p.nentries;
  g_err[0] = 0;
  return MOBA_OK;
}

moba_status_t moba_route(const int32_t* sel_dev, const int32_t* cu_seqlens_dev,
                         const int32_t* cu_seqlens_host, int32_t num_seqs,
                         const moba_shape_t* shape, int32_t block_size, int32_t topk,
                         int32_t* list_offsets, int32_t* entries, void* workspace,
                         size_t workspace_bytes, void* stream) {
  Plan p;
  moba_status_t st =
      make_plan(cu_seqlens_host, num_seqs, shape, block_size, topk, true, &p, nullptr, 0);
  if (st != MOBA_OK) return st;
  if (p.ks < 1) return fail(MOBA_ERR_INVALID_ARG, "moba_route needs topk >= 2");
  if (p.T == 0) {
    g_err[0] = 0;
    return MOBA_OK;
  }
  if (!sel_dev || !cu_seqlens_dev || !list_offsets || (!entries && p.nentries > 0) || !workspace)
    return fail(MOBA_ERR_INVALID_ARG, "NULL device pointer");
  if ((uintptr_t)workspace % 256) return fail(MOBA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  if (workspace_bytes < p.total)
    return fail(MOBA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                p.total);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  Work w = carve(p, workspace);
  hipError_t e = launch_setup(p, cu_seqlens_dev, w, s);
  if (e != hipSuccess) return hip_status(e, "setup");
  {
    StageScope t(ST_ROUTE, s);
    e = launch_route(p, sel_dev, cu_seqlens_dev, w, p.sel_rows, list_offsets, entries, s);
  }
  if (e != hipSuccess) return hip_status(e, "route");
  g_err[0] = 0;
  return MOBA_OK;
}

moba_status_t moba_timing_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (enable && !g_timing.created) {
    for (int i = 0; i < kMaxTimed; ++i) {
      hipError_t e0 = hipEventCreate(&g_timing.ev0[i]);
      hipError_t e1 = hipEventCreate(&g_timing.ev1[i]);
      if (e0 != hipSuccess || e1 != hipSuccess) return hip_status(e0 != hipSuccess ? e0 : e1, "hipEventCreate");
    }
    g_timing.created = true;
  }
  g_timing.enabled = enable != 0;
  g_timing.used = 0;
  g_err[0] = 0;
  return MOBA_OK;
}

int32_t moba_timing_read(double* stage_ms, int32_t* stage_launches, int32_t max_stages) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  const int n = max_stages < ST_COUNT ? max_stages : ST_COUNT;
  for (int i = 0; i < n; ++i) {
    if (stage_ms) stage_ms[i] = 0.0;
    if (stage_launches) stage_launches[i] = 0;
  }
  for (int i = 0; i < g_timing.used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_timing.ev1[i]) != hipSuccess) continue;
    if (hipEventElapsedTime(&ms, g_timing.ev0[i], g_timing.ev1[i]) != hipSuccess) continue;
    const int st = g_timing.stage[i];
    if (st < n) {
      if (stage_ms) stage_ms[st] += ms;
      if (stage_launches) stage_launches[st] += 1;
    }
  }
  g_timing.used = 0;
  return n;
}

const char* moba_stage_name(int32_t stage) {
  if (stage < 0 || stage >= ST_COUNT) return "";
  return kStageNames[stage];
}

}  // extern "C"
