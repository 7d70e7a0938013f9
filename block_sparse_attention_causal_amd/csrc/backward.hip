// NEXT-1: backward of the MoBA attention (dQ, dK, dV through the own block and
// the selected blocks; the selection is held fixed — top-k is piecewise
// constant, so no gradient reaches the gate: MoBA README, "Trainable Block
// Sparse Attention").
//
// For a row r with attended set A_r, p_s = exp(c q_r.k_s - lse_r) (lse_r from
// the forward, over the whole set A_r), dO_r the incoming gradient:
//   Delta_r = dO_r . O_r                   (k_bwd_delta)
//   dS_s    = p_s (dO_r . v_s - Delta_r)
//   dQ_r    = c sum_s dS_s k_s             (query-major: k_bwd_dq, one pass per part)
//   dK_s    = c sum_r dS_s q_r             (key-major: k_bwd_dkdv, all rows that
//   dV_s    =   sum_r p_s dO_r              attend the key, own block and routed)
// Both passes reuse the forward's routing lists (rebuilt from the forward's
// selection): the selected-block dQ pass walks the lists' tiles like the
// forward, and the dK/dV pass walks, for each key tile of a block, the block's
// own later rows and then the rows routed to it — so every key's gradient is
// summed by one workgroup, without atomics, and the result is deterministic.
//
// Matrix-core layout as in the forward (32x32x16 MFMA; fp32 inputs feed the
// same data to eight 32x32x2 MFMAs): a register operand from the accumulator
// layout (dS^T, P, dS) pairs with an LDS operand transposed with the row order
// of vt_pos_of_group4.
#include <type_traits>

#include "moba_plan.h"

namespace moba {

enum { BWD_SELF = 0, BWD_SELECTED = 1 };
constexpr int BKC = 64;       // keys per chunk (dQ pass)
constexpr int BRC = 32;       // rows per chunk (dK/dV pass)
constexpr int BDQ_WAVES = 8;  // dQ pass: 8 waves x 32 rows, the forward's tiles
constexpr int BKV_WAVES = kBkvWaves;  // dK/dV pass: 4 waves x 32 keys = 128 keys per tile

// ---------------------------------------------------------------------------
// Delta_r = sum_d dO_r[d] O_r[d] in fp32, D/8 lanes per row.
template <typename T, int D>
__global__ void __launch_bounds__(256) k_bwd_delta(const T* __restrict__ out,
                                                   const T* __restrict__ dout, int64_t rows,
                                                   const float* __restrict__ lse,
                                                   float* __restrict__ delta,
                                                   float* __restrict__ lse2) {
  constexpr int TPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const T* o = out + row * D + 8 * c;
    const T* g = dout + row * D + 8 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(to_f32(o[e]), to_f32(g[e]), acc);
  }
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && c == 0) {
    delta[row] = acc;
    lse2[row] = lse[row] * kLog2e;   // the dK/dV pass's exponent offset, in the log2 domain
  }
}

// ---------------------------------------------------------------------------
// Staging of R rows of a [*, D] matrix into LDS twice: row-major (row stride
// LD) and transposed (column stride TLD, rows permuted by vt_pos_of_group4).
// Each thread of NT moves 16-byte pieces; `rowptr(r)` gives row r's global
// address or nullptr (zeros).
template <typename T, int D, int R, int NT>
struct RowStage {
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int LD = D + VEC;
  static constexpr int TLD = R + VEC;
  static constexpr int PIECES = R * (D / VEC);
  static constexpr int PPT = (PIECES + NT - 1) / NT;
  typedef T vec_t __attribute__((ext_vector_type(VEC)));
  vec_t x[PPT];

  template <typename F>
  __device__ __forceinline__ void load(F rowptr) {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int pc = (int)threadIdx.x + u * NT;
      const int r = pc / (D / VEC), c = pc % (D / VEC);
      const T* src = (pc < PIECES) ? rowptr(r) : nullptr;
      if (src) {
        x[u] = *reinterpret_cast<const vec_t*>(src + c * VEC);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[u][e] = (T)0.0f;
      }
    }
  }
  __device__ __forceinline__ void store_rows(T* rows_lds) const {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int pc = (int)threadIdx.x + u * NT;
      if (pc >= PIECES) break;
      const int r = pc / (D / VEC), c = pc % (D / VEC);
      *reinterpret_cast<vec_t*>(rows_lds + r * LD + c * VEC) = x[u];
    }
  }
  __device__ __forceinline__ void store(T* rows_lds, T* trans_lds) const {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int pc = (int)threadIdx.x + u * NT;
      if (pc >= PIECES) break;
      const int r = pc / (D / VEC), c = pc % (D / VEC);
      *reinterpret_cast<vec_t*>(rows_lds + r * LD + c * VEC) = x[u];
      const int pos = vt_pos_of_group4(r >> 2) + (r & 3);
#pragma unroll
      for (int e = 0; e < VEC; ++e) trans_lds[(c * VEC + e) * TLD + pos] = x[u][e];
    }
  }
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;       // forward log-sum-exp per row (natural log)
  const float* delta;     // [T * hq]
  const float* lse2;      // [T * hq] lse * log2(e)
  const int32_t* cu;
  const int32_t* blk_seq;
  const int32_t* blk_local;
  const int32_t* blk_base;
  const int32_t* list_offsets;
  const int32_t* tile_offsets;
  const int32_t* entries;
  float* dq_sel;          // [T * hq * ks, D] selected-block dQ parts (scaled), by entry value:
                          // fp32, or bf16 (the first half of the buffer) for 16-bit D = 128
  void* dq;               // [T, hq, D]
  void* dk;               // [T, hkv, D]
  void* dv;
  int64_t nb, nlists, ntiles, padded;
  int nseq, hq, hkv, hg, block, ks, nu, kvt;   // kvt = key tiles per block
  float scale, scale_log2;
  FastDiv div_ks, div_g;   // entry value -> row (/ ks), own row -> token (/ G)
};

// ---------------------------------------------------------------------------
// dQ, query-major. SELF tiles: up to 256 rows of one block (32 consecutive
// tokens per wave, the HG heads of one kv group side by side), keys from the
// block start to the tile's last token, causal. SELECTED tiles: up to 256
// routed (row, slot) entries of one list, keys = the whole block. Per wave and
// 64-key chunk: S^T = K Q^T and dP^T = V dO^T (K, V row-major in LDS, Q^T and
// dO^T in registers), P^T = exp2(S^T c log2e - lse log2e), dS^T = P^T (dP^T -
// Delta), dQ^T += K^T dS^T (K^T transposed in LDS). SELECTED writes the
// scaled part per entry; SELF, which runs after, adds the row's parts.
template <typename T, int D, int MODE>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_bwd_dq(BwdArgs a) {
  typedef typename Frag<T>::type frag_t;
  typedef RowStage<T, D, BKC, 512> Stage;
  __shared__ __attribute__((aligned(16))) T smem[2 * BKC * Stage::LD + D * Stage::TLD];
  T* const k_rows = smem;
  T* const v_rows = smem + BKC * Stage::LD;
  T* const k_trans = smem + 2 * BKC * Stage::LD;
  const int64_t logical = xcd_logical(blockIdx.x, a.padded);
  if (logical >= a.ntiles) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int half = lane >> 5, r32 = lane & 31;
  const int group = a.hq / a.hkv;
  const T* __restrict__ q = (const T*)a.q;
  const T* __restrict__ k = (const T*)a.k;
  const T* __restrict__ v = (const T*)a.v;
  const T* __restrict__ dout = (const T*)a.dout;

  int g;
  int64_t kbeg, kend;
  int64_t row = -1, dst_index = -1, wtok0 = 0;
  int blk_i = 0;
  if (MODE == BWD_SELECTED) {
    const int64_t tile = logical;
    const int32_t* toffs = a.tile_offsets;
    if (tile >= toffs[a.nlists]) return;
    const int L = upper_index_wave(toffs, (int)a.nlists, tile, lane);
    const int64_t b = L / a.hkv;
    g = L % a.hkv;
    const int n = a.blk_seq[b], j = a.blk_local[b];
    kbeg = (int64_t)a.cu[n] + (int64_t)j * a.block;
    kend = kbeg + a.block;
    const int64_t e0 = (int64_t)a.list_offsets[L] + (tile - toffs[L]) * kRowsPerTile +
                       (int64_t)w * kRowsPerWave;
    const int64_t e1 = a.list_offsets[L + 1];
    if (e0 + r32 < e1) {
      const int32_t ev = a.entries[e0 + r32];
      dst_index = ev;
      row = ev / a.ks;
    }
  } else {
    const int tt = 32 * (8 / a.hg);
    const int nhs = a.hq / a.hg;
    const int u = a.nu - 1 - (int)(logical % a.nu);
    const int64_t rest = logical / a.nu;
    const int hs = (int)(rest % nhs);
    const int64_t b = a.nb - 1 - rest / nhs;
    const int n = a.blk_seq[b], i = a.blk_local[b];
    blk_i = i;
    const int64_t blk_start = (int64_t)a.cu[n] + (int64_t)i * a.block;
    const int64_t blk_end = min(blk_start + a.block, (int64_t)a.cu[n + 1]);
    const int64_t tok0 = blk_start + (int64_t)u * tt;
    if (tok0 >= blk_end) return;
    const int h = hs * a.hg + (w % a.hg);
    g = h / group;
    wtok0 = tok0 + (int64_t)(w / a.hg) * 32;
    kbeg = blk_start;
    kend = min(tok0 + tt, blk_end);
    if (wtok0 + r32 < blk_end) {
      row = (wtok0 + r32) * a.hq + h;
      dst_index = row;
    }
  }

  frag_t qf[D / 16], gf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qf[kk] = (row >= 0) ? load8(q + row * D + 16 * kk + 8 * half) : zero8<frag_t>();
    gf[kk] = (row >= 0) ? load8(dout + row * D + 16 * kk + 8 * half) : zero8<frag_t>();
  }
  const float lse_l2 = (row >= 0) ? a.lse[row] * kLog2e : 0.f;
  const float dlt = (row >= 0) ? a.delta[row] : 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;

  const int nch = (int)((kend - kbeg + BKC - 1) / BKC);
  const int64_t kstride = (int64_t)a.hkv * D;
  Stage sk, sv;
  for (int c = 0; c < nch; ++c) {
    const int64_t c0 = kbeg + (int64_t)c * BKC;
    sk.load([&](int r) -> const T* { return (c0 + r < kend) ? k + (c0 + r) * kstride + g * D : nullptr; });
    sv.load([&](int r) -> const T* { return (c0 + r < kend) ? v + (c0 + r) * kstride + g * D : nullptr; });
    __syncthreads();                       // the previous chunk is consumed
    sk.store(k_rows, k_trans);
    sv.store_rows(v_rows);
    __syncthreads();
    const bool needed = (MODE == BWD_SELECTED) || (c0 <= wtok0 + 31);
    if (!needed) continue;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) { s[kt][e] = 0.f; dp[kt][e] = 0.f; }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const frag_t kf = load8(k_rows + (32 * kt + r32) * Stage::LD + 16 * kk + 8 * half);
        const frag_t vf = load8(v_rows + (32 * kt + r32) * Stage::LD + 16 * kk + 8 * half);
        s[kt] = mma_k16(kf, qf[kk], s[kt]);
        dp[kt] = mma_k16(vf, gf[kk], dp[kt]);
      }
    }
    float dsv[2][16];
    const int64_t tok = wtok0 + r32;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t key = c0 + 32 * kt + 8 * (e >> 2) + 4 * half + (e & 3);
        const bool masked = (key >= kend) || (MODE == BWD_SELF && key > tok);
        const float p = masked ? 0.f : fast_exp2(fmaf(s[kt][e], a.scale_log2, -lse_l2));
        dsv[kt][e] = p * (dp[kt][e] - dlt);
      }
    frag_t df[4];
    df[0] = pack8<T>(&dsv[0][0]);
    df[1] = pack8<T>(&dsv[0][8]);
    df[2] = pack8<T>(&dsv[1][0]);
    df[3] = pack8<T>(&dsv[1][8]);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const frag_t kf = load8(k_trans + (32 * dt + r32) * Stage::TLD + 16 * qq + 8 * half);
        acc[dt] = mma_k16(kf, df[qq], acc[dt]);
      }
  }

  // epilogue: lane holds dQ^T[32dt + 8(i/4) + 4half + i%4][row r32]
  if (dst_index < 0) return;
  if (MODE == BWD_SELECTED) {
    float* dst = a.dq_sel + dst_index * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        float4 val = make_float4(acc[dt][4 * aa] * a.scale, acc[dt][4 * aa + 1] * a.scale,
                                 acc[dt][4 * aa + 2] * a.scale, acc[dt][4 * aa + 3] * a.scale);
        *reinterpret_cast<float4*>(dst + 32 * dt + 8 * aa + 4 * half) = val;
      }
  } else {
    const int nsel = min(a.ks, blk_i);
    typedef T vec4_t __attribute__((ext_vector_type(4)));
    T* dst = (T*)a.dq + dst_index * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const int d0 = 32 * dt + 8 * aa + 4 * half;
        float x[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) x[b] = acc[dt][4 * aa + b] * a.scale;
        for (int sl = 0; sl < nsel; ++sl) {
          const float4 pt = *reinterpret_cast<const float4*>(
              a.dq_sel + (dst_index * a.ks + sl) * D + d0);
          x[0] += pt.x;
          x[1] += pt.y;
          x[2] += pt.z;
          x[3] += pt.w;
        }
        vec4_t r;
#pragma unroll
        for (int b = 0; b < 4; ++b) r[b] = from_f32<T>(x[b]);
        *reinterpret_cast<vec4_t*>(dst + d0) = r;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV, key-major. Tile = 128 keys of one block and kv head (4 waves x 32
// keys). Rows: the block's own rows from the tile's first token on (the G q
// heads of the group; causal mask), then the rows routed to the block. Per 32-
// row chunk (Q, dO staged in LDS row-major and transposed, lse and Delta per
// row) and wave: S = Q K_w^T, dP = dO V_w^T (K_w^T, V_w^T register operands),
// P = exp2(S c log2e - lse log2e), dS = P (dP - Delta), dV_w^T += dO^T P,
// dK_w^T += Q^T dS.
template <typename T, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
k_bwd_dkdv(BwdArgs a) {
  typedef typename Frag<T>::type frag_t;
  typedef RowStage<T, D, BRC, 256> Stage;
  __shared__ __attribute__((aligned(16))) T smem[2 * BRC * Stage::LD + 2 * D * Stage::TLD];
  __shared__ float lse_s[BRC], dlt_s[BRC];
  __shared__ int tok_s[BRC];
  T* const q_rows = smem;
  T* const g_rows = smem + BRC * Stage::LD;
  T* const q_trans = smem + 2 * BRC * Stage::LD;
  T* const g_trans = q_trans + D * Stage::TLD;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int half = lane >> 5, r32 = lane & 31;
  const int G = a.hq / a.hkv;
  // tile -> (global block b, kv head g, key tile kt)
  const int64_t tile = blockIdx.x;
  const int kt = (int)(tile % a.kvt);
  const int g = (int)((tile / a.kvt) % a.hkv);
  const int64_t b = tile / a.kvt / a.hkv;
  const int n = a.blk_seq[b], i = a.blk_local[b];
  const int64_t blk_start = (int64_t)a.cu[n] + (int64_t)i * a.block;
  const int64_t blk_end = min(blk_start + a.block, (int64_t)a.cu[n + 1]);
  const int64_t t0 = blk_start + (int64_t)kt * (BKV_WAVES * 32);
  if (t0 >= blk_end) return;
  const int64_t key = t0 + 32 * w + r32;          // this lane's key (as a B column)
  const bool key_ok = key < blk_end;
  const int64_t kstride = (int64_t)a.hkv * D;
  const T* __restrict__ q = (const T*)a.q;
  const T* __restrict__ dout = (const T*)a.dout;

  frag_t kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    kf[kk] = key_ok ? load8((const T*)a.k + key * kstride + g * D + 16 * kk + 8 * half)
                    : zero8<frag_t>();
    vf[kk] = key_ok ? load8((const T*)a.v + key * kstride + g * D + 16 * kk + 8 * half)
                    : zero8<frag_t>();
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) { dk[dt][e] = 0.f; dv[dt][e] = 0.f; }

  // rows: own block tokens t0 .. blk_end-1 (x G heads), then list (b, g) entries
  const int64_t nself = (blk_end - t0) * G;
  int64_t e_beg = 0, nsel_rows = 0;
  if (a.ks > 0 && a.list_offsets) {
    const int64_t L = b * a.hkv + g;
    e_beg = a.list_offsets[L];
    nsel_rows = a.list_offsets[L + 1] - e_beg;
  }
  const int64_t nrows = nself + nsel_rows;
  auto row_of = [&](int64_t rr, int64_t& tokv) -> int64_t {
    if (rr < nself) {
      tokv = t0 + rr / G;
      return tokv * a.hq + g * G + (int)(rr % G);
    }
    const int64_t rowid = a.entries[e_beg + (rr - nself)] / a.ks;
    tokv = rowid / a.hq;
    return rowid;
  };
  Stage sq, sg;
  for (int64_t c0 = 0; c0 < nrows; c0 += BRC) {
    sq.load([&](int r) -> const T* {
      if (c0 + r >= nrows) return nullptr;
      int64_t tv;
      return q + row_of(c0 + r, tv) * D;
    });
    sg.load([&](int r) -> const T* {
      if (c0 + r >= nrows) return nullptr;
      int64_t tv;
      return dout + row_of(c0 + r, tv) * D;
    });
    __syncthreads();
    sq.store(q_rows, q_trans);
    sg.store(g_rows, g_trans);
    if (threadIdx.x < BRC) {
      const int64_t rr = c0 + threadIdx.x;
      if (rr < nrows) {
        int64_t tv;
        const int64_t rowid = row_of(rr, tv);
        lse_s[threadIdx.x] = a.lse[rowid] * kLog2e;
        dlt_s[threadIdx.x] = a.delta[rowid];
        tok_s[threadIdx.x] = (rr < nself) ? (int)(tv - t0) : -1;   // own-block rows only
      } else {
        lse_s[threadIdx.x] = 0.f;
        dlt_s[threadIdx.x] = 0.f;
        tok_s[threadIdx.x] = -2;                                   // no row
      }
    }
    __syncthreads();
    f32x16 s, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) { s[e] = 0.f; dp[e] = 0.f; }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const frag_t qa = load8(q_rows + r32 * Stage::LD + 16 * kk + 8 * half);
      const frag_t ga = load8(g_rows + r32 * Stage::LD + 16 * kk + 8 * half);
      s = mma_k16(qa, kf[kk], s);
      dp = mma_k16(ga, vf[kk], dp);
    }
    // lane: key column r32 of wave w; items: rows 8(e/4) + 4half + e%4
    float pv[16], dsv[16];
    const int keyrel = (int)(key - t0);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rr = 8 * (e >> 2) + 4 * half + (e & 3);
      const int tr = tok_s[rr];
      const bool masked = !key_ok || tr == -2 || (tr >= 0 && keyrel > tr);
      const float p = masked ? 0.f : fast_exp2(fmaf(s[e], a.scale_log2, -lse_s[rr]));
      pv[e] = p;
      dsv[e] = p * (dp[e] - dlt_s[rr]);
    }
    frag_t pf[2], df[2];
    pf[0] = pack8<T>(&pv[0]);
    pf[1] = pack8<T>(&pv[8]);
    df[0] = pack8<T>(&dsv[0]);
    df[1] = pack8<T>(&dsv[8]);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const frag_t ga = load8(g_trans + (32 * dt + r32) * Stage::TLD + 16 * qq + 8 * half);
        const frag_t qa = load8(q_trans + (32 * dt + r32) * Stage::TLD + 16 * qq + 8 * half);
        dv[dt] = mma_k16(ga, pf[qq], dv[dt]);
        dk[dt] = mma_k16(qa, df[qq], dk[dt]);
      }
    __syncthreads();                       // before the next chunk overwrites LDS
  }

  // epilogue: lane holds d{K,V}^T[32dt + 8(i/4) + 4half + i%4][key]
  if (!key_ok) return;
  typedef T vec4_t __attribute__((ext_vector_type(4)));
  T* dkp = (T*)a.dk + key * kstride + g * D;
  T* dvp = (T*)a.dv + key * kstride + g * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      const int d0 = 32 * dt + 8 * aa + 4 * half;
      vec4_t rk, rv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rk[e] = from_f32<T>(dk[dt][4 * aa + e] * a.scale);
        rv[e] = from_f32<T>(dv[dt][4 * aa + e]);
      }
      *reinterpret_cast<vec4_t*>(dkp + d0) = rk;
      *reinterpret_cast<vec4_t*>(dvp + d0) = rv;
    }
}

// ---------------------------------------------------------------------------
// dK, dV for 16-bit inputs with D = 128: the same products as k_bwd_dkdv, 8
// waves x 32 keys = 256 keys per tile, with the rows streamed through LDS by
// direct loads. Per 32-row chunk every wave issues exactly four direct loads:
// the list entries of chunk c+5 (row ids of the routed rows, 4 bytes a lane),
// then for chunk c+3 its four rows of Q and of dO (16 bytes a lane, the
// forward's swizzled row layout) and the chunk's lse and Delta (4 bytes a
// lane, a private copy per wave). "Chunk c+1 and the entries of chunk c+4 have
// landed" is then exactly vmcnt(7) at the end of iteration c. Q^T and dO^T
// fragments come from the row-major copies through ds_read_b64_tr_b16, in the
// row order of the score accumulators, so no transposed copy is written.
// Tiles are dealt to the XCDs list by list (all key tiles of one list on one
// XCD, which then shares the list's rows in its L2; consecutive lists on
// different XCDs, which spreads the long lists of the much-selected blocks).
// For that sharing the key tiles of a list stream the same rows in the same
// order at the same time: first the routed rows, then the block's own rows from
// its last token down, each tile stopping below its first key. (Own rows first,
// from each tile's first key up, would start the tiles thousands of rows apart
// and every tile would fetch every row from HBM.)
constexpr int DKV_WAVES = kDkvWaves;

__device__ __forceinline__ bf16x8 tr_frag(const bf16* rows, int r0, int dt, int vrow, int vx0,
                                          int vx1, int vbyte) {
  // rows r0 + {4h .. 4h+3} and r0 + 8 + {4h .. 4h+3} of column 32 dt + (lane % 32)
  const bf16* b = rows + (r0 + vrow) * 128;
  const bf16* p0 = b + 8 * ((4 * dt) ^ vx0) + vbyte;
  const bf16* p1 = b + 8 * 128 + 8 * ((4 * dt) ^ vx1) + vbyte;
  const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 r;
  r[0] = x0[0]; r[1] = x0[1]; r[2] = x0[2]; r[3] = x0[3];
  r[4] = x1[0]; r[5] = x1[1]; r[6] = x1[2]; r[7] = x1[3];
  return __builtin_bit_cast(bf16x8, r);
}

__global__ void __launch_bounds__(64 * DKV_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_bwd_dkdv_dma(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int D = 128;
  constexpr int CH = BRC * D;       // elements of one 32-row block
  constexpr int RBUF = 2 * CH;      // Q rows then dO rows
  __shared__ __attribute__((aligned(16))) bf16 rows_lds[4 * RBUF];
  __shared__ __attribute__((aligned(16))) float meta_lds[4][DKV_WAVES][64];
  __shared__ __attribute__((aligned(16))) int32_t ent_lds[8][DKV_WAVES][64];
  __shared__ __attribute__((aligned(16))) bf16 v_lds[DKV_WAVES * 32 * D];   // the tile's V rows
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // scalar wave index
  const int half = lane >> 5, r32 = lane & 31;
  const int G = a.hq / a.hkv;
  // dispatch id -> (list, key tile): list 8 (j / kvt) + xcd, key tile j % kvt
  const int64_t j = blockIdx.x >> 3;
  const int64_t L = 8 * (j / a.kvt) + (blockIdx.x & 7);
  if (L >= a.nb * a.hkv) return;
  const int kt = (int)(j % a.kvt);
  const int g = (int)(L % a.hkv);
  const int64_t b = L / a.hkv;
  const int n = a.blk_seq[b], i = a.blk_local[b];
  const int64_t blk_start = (int64_t)a.cu[n] + (int64_t)i * a.block;
  const int64_t blk_end = min(blk_start + a.block, (int64_t)a.cu[n + 1]);
  const int64_t t0 = blk_start + (int64_t)kt * (DKV_WAVES * 32);
  if (t0 >= blk_end) return;
  const int keyrel = 32 * w + r32;
  const int64_t key = t0 + keyrel;
  const bool key_ok = key < blk_end;
  const bool wave_live = t0 + 32 * w < blk_end;
  const int64_t kstride = (int64_t)a.hkv * D;
  const bf16* __restrict__ q = (const bf16*)a.q;
  const bf16* __restrict__ dout = (const bf16*)a.dout;

  // K fragments in registers; the wave's 32 V rows in LDS (swizzled like the
  // streamed rows), both of keys clamped into the block
  bf16x8 kf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    kf[kk] = key_ok ? load8((const bf16*)a.k + key * kstride + g * D + 16 * kk + 8 * half)
                    : zero8<bf16x8>();
  {
    const uint32_t vdst = lds_addr(v_lds) + (uint32_t)(32 * w * D * 2);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = 4 * u + (lane >> 4);
      const int64_t kv = min(t0 + 32 * w + r, blk_end - 1);
      dma16((const bf16*)a.v + kv * kstride + g * D + 8 * ((lane & 15) ^ swz(r)),
            vdst + (uint32_t)(u * 1024));
    }
  }
  const bf16* vw = v_lds + 32 * w * D;
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) { dk[dt][e] = 0.f; dv[dt][e] = 0.f; }

  // rows: the list's routed rows, then the block's own tokens blk_end-1 down to t0
  // (G heads each); row counts and row ids fit 32 bits: T * hq < 2^31
  const int nself = (int)(blk_end - t0) * G;
  int e_beg = 0, nsel_rows = 0;
  if (a.ks > 0 && a.list_offsets) {
    e_beg = a.list_offsets[L];
    nsel_rows = a.list_offsets[L + 1] - e_beg;
  }
  const int nrows = nsel_rows + nself;
  const int nch = (nrows + BRC - 1) / BRC;
  const int rowl = (int)(blk_end - 1) * a.hq + g * G;   // row id of own row 0 (last token)

  const uint32_t rows_base = lds_addr(rows_lds);
  auto issue_ent = [&](int c) __attribute__((always_inline)) {
    const int cc = min(c, nch - 1);
    const int idx = cc * BRC + (lane & 31);
    const int32_t* src =
        (nsel_rows > 0) ? a.entries + e_beg + min(max(idx, 0), nsel_rows - 1) : a.cu;
    dma4(src, lds_addr(&ent_lds[c & 7][w][0]));
  };
  // branch-free: both candidates, then a select (entries past the list are
  // clamped copies of valid ones, so the unused candidate is harmless)
  auto rowid_of = [&](int c, int r) __attribute__((always_inline)) -> int {
    const int rr = min(c, nch - 1) * BRC + r;
    const int sel = (int)fdiv((uint32_t)ent_lds[c & 7][w][r], a.div_ks);
    const uint32_t o = (uint32_t)max(rr - nsel_rows, 0);
    const uint32_t tb = fdiv(o, a.div_g);
    const int own = rowl - (int)tb * a.hq + (int)(o - tb * (uint32_t)G);
    return (rr < nsel_rows) ? sel : (rr < nrows) ? own : 0;   // padding: any valid row
  };
  const int rA = 4 * w + (lane >> 4);
  const int offA = 8 * ((lane & 15) ^ swz(rA));
  auto issue_rows = [&](int c) __attribute__((always_inline)) {
    const int buf = c & 3;
    const int ridA = rowid_of(c, rA);
    const int ridM = rowid_of(c, lane & 31);
    const uint32_t dst = rows_base + (uint32_t)((buf * RBUF + 4 * w * D) * 2);
    dma16(q + (int64_t)ridA * D + offA, dst);
    dma16(dout + (int64_t)ridA * D + offA, dst + (uint32_t)(CH * 2));
    dma4((lane < 32) ? a.lse2 + ridM : a.delta + ridM, lds_addr(&meta_lds[buf][w][0]));
  };

  const int hx = half ^ swz(r32);
  const int ml = lane & 15;
  const int vrow = 4 * half + (ml >> 2);
  const int vp = 2 * ((lane >> 4) & 1) + ((ml & 3) >> 1);
  const int vx0 = vp ^ swz(vrow), vx1 = vp ^ swz(vrow + 8);
  const int vbyte = (ml & 1) * 4;
  // own rows from rr = lim on come before the key (and rr >= nrows is padding)
  const int lim = nsel_rows + (int)(blk_end - key) * G;
  const int lim_wave = nsel_rows + (int)(blk_end - t0 - 32 * w) * G;   // of the wave's first key

  auto compute = [&](int c) __attribute__((always_inline)) {
    if (!wave_live) return;
    const int rr0 = c * BRC;
    // a chunk of own rows whose tokens all precede the wave's first key
    if (rr0 >= lim_wave) return;
    const bf16* qb = rows_lds + (c & 3) * RBUF;
    const bf16* gb = qb + CH;
    f32x16 s, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) { s[e] = 0.f; dp[e] = 0.f; }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8 qa = load8(qb + r32 * D + 8 * ((2 * kk) ^ hx));
      const bf16x8 ga = load8(gb + r32 * D + 8 * ((2 * kk) ^ hx));
      const bf16x8 vb = load8(vw + r32 * D + 8 * ((2 * kk) ^ hx));
      s = mma_k16(qa, kf[kk], s);
      dp = mma_k16(ga, vb, dp);
    }
    // lane: key column r32 of wave w; item e: row 8(e/4) + 4half + e%4 of the chunk.
    // P overwrites s, dS overwrites dp.
    const float* mt = meta_lds[c & 3][w];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float4 l4 = *reinterpret_cast<const float4*>(mt + 8 * jj + 4 * half);
      const float4 d4 = *reinterpret_cast<const float4*>(mt + 32 + 8 * jj + 4 * half);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
      const float dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = 4 * jj + u;
        const int rr = rr0 + 8 * jj + 4 * half + u;
        // masked: exp2(-inf) = 0, no branch around the exponential
        const float x = fmaf(s[e], a.scale_log2, -lv[u]);
        const float p = fast_exp2((rr >= lim) ? -INFINITY : x);
        s[e] = p;
        dp[e] = p * (dp[e] - dl[u]);
      }
    }
    bf16x8 pf[2], df[2];
    {
      float t[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) t[e] = s[e];
      pf[0] = pack8<bf16>(&t[0]);
      pf[1] = pack8<bf16>(&t[8]);
#pragma unroll
      for (int e = 0; e < 16; ++e) t[e] = dp[e];
      df[0] = pack8<bf16>(&t[0]);
      df[1] = pack8<bf16>(&t[8]);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const bf16x8 ga = tr_frag(gb, 16 * qq, dt, vrow, vx0, vx1, vbyte);
        dv[dt] = mma_k16(ga, pf[qq], dv[dt]);
        const bf16x8 qa = tr_frag(qb, 16 * qq, dt, vrow, vx0, vx1, vbyte);
        dk[dt] = mma_k16(qa, df[qq], dk[dt]);
      }
  };

  // the K fragments (compiler-visible loads) and the V rows land first
  MOBA_WAIT_VM_LGKM0(0);
  for (int c = 0; c < 5; ++c) issue_ent(c);
  MOBA_WAIT_VM_LGKM0(0);
  bare_barrier();
  issue_rows(0);
  issue_rows(1);
  issue_rows(2);
  MOBA_WAIT_VM_LGKM0(6);
  bare_barrier();
  for (int c = 0; c < nch; ++c) {
    issue_ent(c + 5);
    issue_rows(c + 3);
    compute(c);
    MOBA_WAIT_VM_LGKM0(7);
    bare_barrier();
  }
  MOBA_WAIT_VM_LGKM0(0);

  // epilogue: lane holds d{K,V}^T[32dt + 8(i/4) + 4half + i%4][key]
  if (!key_ok) return;
  typedef bf16 vec4_t __attribute__((ext_vector_type(4)));
  bf16* dkp = (bf16*)a.dk + key * kstride + g * D;
  bf16* dvp = (bf16*)a.dv + key * kstride + g * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      const int d0 = 32 * dt + 8 * aa + 4 * half;
      vec4_t rk, rv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rk[e] = (bf16)(dk[dt][4 * aa + e] * a.scale);
        rv[e] = (bf16)dv[dt][4 * aa + e];
      }
      *reinterpret_cast<vec4_t*>(dkp + d0) = rk;
      *reinterpret_cast<vec4_t*>(dvp + d0) = rv;
    }
#endif
}

// ---------------------------------------------------------------------------
// dQ for 16-bit inputs with D = 128: k_bwd_dq's products, with the forward's
// 4-wave tiles and key pipeline (64-key chunks of K and V by direct loads into
// two swizzled 32 KB LDS buffers, one chunk in flight, vmcnt(0) and a barrier
// per chunk; two workgroups per CU, so one's tile prologue, epilogue and
// barrier waits overlap the other's products). K and V rows are the A operands
// of S^T and dP^T; K^T fragments for dQ^T come from the same K rows through
// ds_read_b64_tr_b16 in the key order of the dS^T registers.
//   SELECTED: a tile is 128 routed rows (4 waves x 32) of one (block, kv head)
//     list; writes one bf16 part per (row, slot).
//   SELF: a tile is 4 / hw groups of 32 consecutive tokens of one block for hw
//     q heads of one kv group (hw = gcd(G, 4)), with the causal mask; adds the
//     row's parts and writes dQ.
template <int MODE>
__global__ void __launch_bounds__(64 * kSelWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_bwd_dq_dma(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int D = 128;
  constexpr int NW = kSelWaves;                  // waves per workgroup
  constexpr int DBUF = 2 * BKC * D;              // K rows then V rows
  static_assert(NW * 32 * (D + 8) <= 2 * DBUF, "part staging must fit in the LDS buffers");
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * DBUF];
  const int64_t logical = xcd_logical(blockIdx.x, a.padded);
  if (logical >= a.ntiles) return;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // scalar wave index
  const int half = lane >> 5, r32 = lane & 31;
  const int group = a.hq / a.hkv;
  const bf16* __restrict__ q = (const bf16*)a.q;
  const bf16* __restrict__ k = (const bf16*)a.k;
  const bf16* __restrict__ v = (const bf16*)a.v;
  const bf16* __restrict__ dout = (const bf16*)a.dout;

  int g;
  int64_t kbeg, kend;
  int64_t row = -1, dst_index = -1, wtok0 = 0;
  bool wave_live;
  int blk_i = 0;
  if (MODE == BWD_SELECTED) {
    const int64_t tile = logical;
    const int32_t* toffs = a.tile_offsets;
    if (tile >= toffs[a.nlists]) return;
    const int L = upper_index_wave(toffs, (int)a.nlists, tile, lane);
    const int64_t b = L / a.hkv;
    g = L % a.hkv;
    const int n = a.blk_seq[b], j = a.blk_local[b];
    kbeg = (int64_t)a.cu[n] + (int64_t)j * a.block;
    kend = kbeg + a.block;
    const int64_t e0 = (int64_t)a.list_offsets[L] + (tile - toffs[L]) * (kRowsPerWave * NW) +
                       (int64_t)w * kRowsPerWave;
    const int64_t e1 = a.list_offsets[L + 1];
    wave_live = e0 < e1;
    if (e0 + r32 < e1) {
      const int32_t ev = a.entries[e0 + r32];
      dst_index = ev;
      row = fdiv((uint32_t)ev, a.div_ks);
    }
  } else {
    const int hw = (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
    const int tt = 32 * (NW / hw);
    const int nhs = a.hq / hw;
    const int u = a.nu - 1 - (int)(logical % a.nu);
    const int64_t rest = logical / a.nu;
    const int hs = (int)(rest % nhs);
    const int64_t b = a.nb - 1 - rest / nhs;
    const int n = a.blk_seq[b], i = a.blk_local[b];
    blk_i = i;
    const int64_t blk_start = (int64_t)a.cu[n] + (int64_t)i * a.block;
    const int64_t blk_end = min(blk_start + a.block, (int64_t)a.cu[n + 1]);
    const int64_t tok0 = blk_start + (int64_t)u * tt;
    if (tok0 >= blk_end) return;
    const int h = hs * hw + (w % hw);
    g = h / group;
    wtok0 = tok0 + (int64_t)(w / hw) * 32;
    wave_live = wtok0 < blk_end;
    kbeg = blk_start;
    kend = min(tok0 + tt, blk_end);
    if (wtok0 + r32 < blk_end) {
      row = (wtok0 + r32) * a.hq + h;
      dst_index = row;
    }
  }

  // cached loads: each instruction takes 32 bytes of every row, and the row's
  // other pieces, read by the next instructions, must still be in L2 (with
  // non-temporal loads the kernel read 1.5x the Q and dO bytes from DRAM)
  bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qf[kk] = (row >= 0) ? load8(q + row * D + 16 * kk + 8 * half) : zero8<bf16x8>();
    gf[kk] = (row >= 0) ? load8(dout + row * D + 16 * kk + 8 * half) : zero8<bf16x8>();
  }
  const float lse_l2 = (row >= 0) ? a.lse[row] * kLog2e : 0.f;
  const float dlt = (row >= 0) ? a.delta[row] : 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;

  const int hx = half ^ swz(r32);
  const int ml = lane & 15;
  const int vrow = 4 * half + (ml >> 2);
  const int vp = 2 * ((lane >> 4) & 1) + ((ml & 3) >> 1);
  const int vx0 = vp ^ swz(vrow), vx1 = vp ^ swz(vrow + 8);
  const int vbyte = (ml & 1) * 4;

  auto compute = [&](int buf, int64_t c0) __attribute__((always_inline)) {
    const bool needed = (MODE == BWD_SELECTED) ? wave_live : (wave_live && c0 <= wtok0 + 31);
    if (!needed) return;
    const bf16* kb = smem + buf * DBUF;
    const bf16* vb = kb + BKC * D;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) { s[kt][e] = 0.f; dp[kt][e] = 0.f; }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 kf = load8(kb + (32 * kt + r32) * D + 8 * ((2 * kk) ^ hx));
        s[kt] = mma_k16(kf, qf[kk], s[kt]);
        const bf16x8 vf = load8(vb + (32 * kt + r32) * D + 8 * ((2 * kk) ^ hx));
        dp[kt] = mma_k16(vf, gf[kk], dp[kt]);
      }
    // SELECTED: a past block is whole 64-key chunks (the block size is a
    // multiple of 64), nothing to mask. SELF: keys after the row's token (this
    // covers the clamped keys past the tile's range, which follow every row of
    // the tile); masked scores become -inf, so exp2 gives 0 without a branch.
    const bool need_mask = (MODE == BWD_SELF) && (c0 + BKC - 1 > wtok0);
    const int krel0 = (int)(c0 - wtok0) - r32 + 4 * half;   // key - token at e = 0, kt = 0
    bf16x8 df[4];
    auto grads = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float dsv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = fmaf(s[kt][e], a.scale_log2, -lse_l2);
          if constexpr (decltype(masked)::value)
            x = (krel0 + 32 * kt + 8 * (e >> 2) + (e & 3) > 0) ? -INFINITY : x;
          const float p = fast_exp2(x);
          dsv[e] = p * (dp[kt][e] - dlt);
        }
        df[2 * kt] = pack8<bf16>(&dsv[0]);
        df[2 * kt + 1] = pack8<bf16>(&dsv[8]);
      }
    };
    if (need_mask)
      grads(std::true_type{});
    else
      grads(std::false_type{});
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const bf16x8 kt_f = tr_frag(kb, 16 * qq, dt, vrow, vx0, vx1, vbyte);
        acc[dt] = mma_k16(kt_f, df[qq], acc[dt]);
      }
  };

  const int nch = (int)((kend - kbeg + BKC - 1) / BKC);
  const int row_stride = a.hkv * D;
  const uint32_t smem_lds = lds_addr(smem);
  // chunk c (clamped to the last) into LDS buffer `buf`: each wave loads 16 rows
  // of K and of V. Keys past the tile's range (the last chunk of a causal tile)
  // read the range's last key: in bounds, and masked.
  constexpr int WR = BKC / NW;                   // chunk rows per wave
  auto issue = [&](int c, int buf) __attribute__((always_inline)) {
    const int cc = min(c, nch - 1);
    const int64_t c0 = kbeg + (int64_t)cc * BKC;
    const int last = (int)min((int64_t)(BKC - 1), kend - 1 - c0);
    const bf16* kp = k + (c0 * a.hkv + g) * D;
    const bf16* vp2 = v + (c0 * a.hkv + g) * D;
    const uint32_t dst = smem_lds + (uint32_t)(buf * DBUF * 2 + WR * w * 256);
#pragma unroll
    for (int i = 0; i < WR / 4; ++i) {
      const int r = WR * w + 4 * i + (lane >> 4);
      // byte offset from the chunk's (wave-uniform) first key
      const uint32_t off = (uint32_t)(min(r, last) * row_stride + 8 * ((lane & 15) ^ swz(r))) * 2u;
      if (i == 0) {                                // first loads from the chunk's bases
        dma16s<true>(kp, off, dst);
        dma16s<true>(vp2, off, dst + (uint32_t)(BKC * D * 2));
      } else {
        dma16s<false>(kp, off, dst + (uint32_t)(1024 * i));
        dma16s<false>(vp2, off, dst + (uint32_t)(BKC * D * 2 + 1024 * i));
      }
    }
  };
  // the Q and dO fragments (compiler-visible loads) land before any direct load
  MOBA_WAIT_VM_LGKM0(0);
  issue(0, 0);
  MOBA_WAIT_VM_LGKM0(0);
  bare_barrier();
  // two chunks per trip, buffers 0 then 1, and an odd last chunk after the loop
  int c = 0;
  for (; c + 1 < nch; c += 2) {
    issue(c + 1, 1);
    compute(0, kbeg + (int64_t)c * BKC);
    MOBA_WAIT_VM_LGKM0(0);
    bare_barrier();
    issue(c + 2, 0);                               // (clamped past the end)
    compute(1, kbeg + (int64_t)(c + 1) * BKC);
    MOBA_WAIT_VM_LGKM0(0);
    bare_barrier();
  }
  if (c < nch) {
    compute(0, kbeg + (int64_t)c * BKC);
  }

  // epilogue: lane holds dQ^T[32dt + 8(i/4) + 4half + i%4][row r32]
  if (MODE == BWD_SELECTED) {
    // bf16 parts (half the bytes of fp32 each way, and within the gradients'
    // 2e-2 bar: a part is rounded once, relative 2^-9) through LDS, so every
    // store writes whole 256-byte rows (written 8 bytes per row at a time, the
    // parts had cost as many DRAM bytes again in reads)
    typedef bf16 b4 __attribute__((ext_vector_type(4)));
    typedef bf16 b8 __attribute__((ext_vector_type(8)));
    constexpr int SLD = D + 8;                     // padded staging row (bf16)
    bf16* stage = reinterpret_cast<bf16*>(smem) + w * 32 * SLD;
    bf16* parts = reinterpret_cast<bf16*>(a.dq_sel);
    __syncthreads();     // every wave's direct loads have landed and its products are done
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        b4 v;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) v[bb] = (bf16)(acc[dt][4 * aa + bb] * a.scale);
        *reinterpret_cast<b4*>(stage + r32 * SLD + 32 * dt + 8 * aa + 4 * half) = v;
      }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int rr = 4 * it + (lane >> 4), pc = lane & 15;
      const int64_t di = __shfl(dst_index, rr, 64);
      if (di >= 0)
        __builtin_nontemporal_store(*reinterpret_cast<const b8*>(stage + rr * SLD + 8 * pc),
                                    reinterpret_cast<b8*>(parts + di * D + 8 * pc));
    }
    return;
  }
  if (dst_index < 0) return;
  {
    const int nsel = min(a.ks, blk_i);
    typedef bf16 vec4_t __attribute__((ext_vector_type(4)));
    bf16* dst = (bf16*)a.dq + dst_index * D;
    float x[D / 32][4][4];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) x[dt][aa][bb] = acc[dt][4 * aa + bb] * a.scale;
    // the selected pass's bf16 parts of this row
    typedef bf16 b4 __attribute__((ext_vector_type(4)));
    const bf16* parts = reinterpret_cast<const bf16*>(a.dq_sel);
    if (a.ks <= 2) {
      // every part load of the row at once (a missing part reads entry 0, always
      // allocated, and is dropped), so the epilogue pays one memory latency
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const bool valid = sl < nsel;
        const int64_t e = valid ? dst_index * a.ks + sl : 0;
        b4 pt[D / 32][4];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int aa = 0; aa < 4; ++aa)
            pt[dt][aa] = *reinterpret_cast<const b4*>(parts + e * D + 32 * dt + 8 * aa + 4 * half);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int aa = 0; aa < 4; ++aa)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) x[dt][aa][bb] += valid ? (float)pt[dt][aa][bb] : 0.f;
      }
    } else {
      for (int sl = 0; sl < nsel; ++sl) {
        const bf16* src = parts + (dst_index * a.ks + sl) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int aa = 0; aa < 4; ++aa) {
            const b4 pt = *reinterpret_cast<const b4*>(src + 32 * dt + 8 * aa + 4 * half);
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) x[dt][aa][bb] += (float)pt[bb];
          }
      }
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        vec4_t r;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) r[bb] = (bf16)x[dt][aa][bb];
        *reinterpret_cast<vec4_t*>(dst + 32 * dt + 8 * aa + 4 * half) = r;
      }
  }
#endif
}

// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t bwd_launch(const BwdArgs& base, const Plan& p, const void* out,
                             float* delta, float* lse2, hipStream_t s) {
  const int64_t rows = p.T * p.hq;
  {
    const int rpw = 256 / (D / 8);
    hipLaunchKernelGGL((k_bwd_delta<T, D>), dim3((unsigned)((rows + rpw - 1) / rpw)), dim3(256),
                       0, s, (const T*)out, (const T*)base.dout, rows, base.lse, delta, lse2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdArgs a = base;
  if (p.ks > 0 && p.nentries > 0) {
    a.ntiles = tile_bound(p, p.sel_rows);            // the lists were routed in these tiles
    a.padded = pad8(a.ntiles);
    if constexpr (sizeof(T) == 2 && D == 128)
      hipLaunchKernelGGL(k_bwd_dq_dma<BWD_SELECTED>, dim3((unsigned)a.padded),
                         dim3(64 * kSelWaves), 0, s, a);
    else
      hipLaunchKernelGGL((k_bwd_dq<T, D, BWD_SELECTED>), dim3((unsigned)a.padded), dim3(512), 0,
                         s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (sizeof(T) == 2 && D == 128) {
    a.nu = tiles_per_block(p, attn4_tokens(p));
    a.ntiles = self4_tile_count(p);
    a.padded = pad8(a.ntiles);
    hipLaunchKernelGGL(k_bwd_dq_dma<BWD_SELF>, dim3((unsigned)a.padded), dim3(64 * kSelWaves), 0,
                       s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    a.nu = tiles_per_block(p, tile_tokens8(p));
    a.ntiles = self8_tile_count(p);
    a.padded = pad8(a.ntiles);
    hipLaunchKernelGGL((k_bwd_dq<T, D, BWD_SELF>), dim3((unsigned)a.padded), dim3(512), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (sizeof(T) == 2 && D == 128) {
    a.kvt = tiles_per_block(p, DKV_WAVES * 32);
    const int64_t lists8 = pad8(p.nb * p.hkv);
    hipLaunchKernelGGL(k_bwd_dkdv_dma, dim3((unsigned)(lists8 * a.kvt)), dim3(64 * DKV_WAVES), 0,
                       s, a);
  } else {
    a.kvt = tiles_per_block(p, BKV_WAVES * 32);
    const int64_t tiles = p.nb * p.hkv * a.kvt;
    hipLaunchKernelGGL((k_bwd_dkdv<T, D>), dim3((unsigned)tiles), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_backward(const Plan& p, const void* q, const void* k, const void* v,
                           const void* out, const float* lse, const void* dout,
                           const int32_t* cu_dev, const Work& w, float* delta, float* lse2,
                           float* dq_sel,
                           void* dq, void* dk, void* dv, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  BwdArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.lse2 = lse2;
  a.cu = cu_dev;
  a.blk_seq = w.blk_seq;
  a.blk_local = w.blk_local;
  a.blk_base = w.blk_base;
  a.list_offsets = (p.ks > 0) ? w.list_offsets : nullptr;
  a.tile_offsets = (p.ks > 0) ? w.tile_offsets : nullptr;
  a.entries = (p.ks > 0) ? w.entries : nullptr;
  a.dq_sel = dq_sel;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.nb = p.nb;
  a.nlists = p.nlists;
  a.nseq = p.nseq;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.hg = p.hg;
  a.block = p.block;
  a.ks = p.ks;
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  a.div_ks = make_fastdiv((uint32_t)(p.ks > 0 ? p.ks : 1));
  a.div_g = make_fastdiv((uint32_t)(p.hq / p.hkv));
  if (p.dtype == MOBA_DTYPE_BF16)
    return p.d == 128 ? bwd_launch<bf16, 128>(a, p, out, delta, lse2, s)
                      : bwd_launch<bf16, 64>(a, p, out, delta, lse2, s);
  return p.d == 128 ? bwd_launch<float, 128>(a, p, out, delta, lse2, s)
                    : bwd_launch<float, 64>(a, p, out, delta, lse2, s);
}

}  // namespace moba
