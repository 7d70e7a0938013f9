// a4a / a4b / a5 / a6: flash attention on the matrix cores, with the merge of
// the parts in the self-block kernel's epilogue.
//
// Kimi发布MoBA突破性实现无限上下文, "PyTorch实现关键要点": flash attention runs
// separately over each query's own block (causal) and over the blocks the gate
// selected, and the parts are then combined with an online-softmax merge.
// MoBA README FAQ (issue #27): the own block is attended with a causal mask.
// The selected-block kernel runs first and leaves its parts in the workspace;
// the self-block kernel merges them into its own result as it writes the rows.
//
// One kernel template serves three tile kinds:
//   SELF     tile = up to 256 rows of one block: 32 consecutive tokens per wave,
//            the HG q-heads of one kv group side by side (GQA: the waves share
//            the K/V tiles). Keys = block start .. last token of the tile, causal.
//   SELECTED tile = up to 256 routed (row, slot) entries of one list (block j,
//            kv-head g); keys = the B keys of block j, no mask. Rows of every
//            q-head of the group mix freely in a tile (GQA sharing again).
//   DENSE    SELF with the whole sequence as one block (the comparison kernel).
//
// Per wave (32 rows) and per 64-key chunk staged in LDS:
//   S^T[key, row] = K . Q^T  (A = K from LDS, B = Q^T held in registers)
//   online softmax per row in the log2 domain; lane l owns row l % 32 and half
//   of its keys, lane l ^ 32 the other half, so only the running max is
//   exchanged per chunk;
//   O^T[d, row] += V^T . P^T (A = V^T from a transposed LDS copy, B = P^T
//   straight from the score registers; the LDS key order is permuted so each
//   lane's eight keys are contiguous).
// K and V chunks are double-buffered in LDS; the next chunk is loaded into
// registers while the current one is multiplied.
#include "moba_plan.h"

namespace moba {

enum { MODE_SELF = 0, MODE_SELECTED = 1, MODE_DENSE = 2 };
constexpr int KC = 64;  // keys per chunk

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu;
  const int32_t* blk_seq;
  const int32_t* blk_local;
  const int32_t* list_offsets;
  const int32_t* tile_offsets;
  const int32_t* entries;
  void* o_part;       // SELF with ks > 0: [T*hq, D]; SELECTED: [T*hq*ks, D] (PartType<T>)
  float* lse_part;
  void* out;          // DENSE and SELF: final output [T*hq, D]
  float* lse_out;     // optional with `out`
  const void* sel_o;        // SELF with ks > 0: selected-block partials to merge
  const float* sel_lse;     //   [T*hq*ks, D] (PartType<T>) and their lse
  int64_t nb, nlists, ntiles, padded;
  int nseq, hq, hkv, hg, block, ks, nu;
  float scale_log2;
};


template <typename T, int D>
struct KVStage {
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int KPAD = 16 / (int)sizeof(T);
  static constexpr int VPAD = 16 / (int)sizeof(T);
  static constexpr int KLD = D + KPAD;
  static constexpr int VLD = KC + VPAD;
  static constexpr int KPIECES = KC * (D / VEC) / 512;   // 16-byte K pieces per thread
  static constexpr int VTASKS = (KC / 4) * (D / 4);      // 4 keys x 4 dims tasks
  typedef T vec_t __attribute__((ext_vector_type(VEC)));
  typedef T vec4_t __attribute__((ext_vector_type(4)));
  vec_t kr[KPIECES];
  vec4_t vr[4];

  // One branch-free load path. Keys past the range end (only in the last,
  // partial chunk of a causal tile) are clamped to the last valid key: those
  // rows are finite data that the causal mask gives zero weight (every such key
  // lies after every row of the tile). Selected-block ranges are whole blocks,
  // a multiple of 64 keys, and never clamp. (Separate full/partial paths made
  // the compiler wait for each prefetch right after issuing it.)
  __device__ __forceinline__ void load(const T* __restrict__ k, const T* __restrict__ v,
                                       int64_t c0, int64_t kend, int hkv, int g) {
    const int tid = threadIdx.x;
    const int row_stride = hkv * D;
    const int last = (int)min((int64_t)(KC - 1), kend - 1 - c0);
    const T* kb = k + (c0 * hkv + g) * D;
    const T* vb = v + (c0 * hkv + g) * D;
#pragma unroll
    for (int r = 0; r < KPIECES; ++r) {
      const int pc = tid + 512 * r;
      const int key = min(pc / (D / VEC), last), col = pc % (D / VEC);
      kr[r] = *reinterpret_cast<const vec_t*>(kb + (key * row_stride + col * VEC));
    }
    if (tid < VTASKS) {
      const int kg = tid % (KC / 4), dg = tid / (KC / 4);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        vr[b] = *reinterpret_cast<const vec4_t*>(vb + (min(4 * kg + b, last) * row_stride + 4 * dg));
    }
  }

  __device__ __forceinline__ void store(T* __restrict__ ks_lds, T* __restrict__ vt_lds) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int r = 0; r < KPIECES; ++r) {
      const int pc = tid + 512 * r;
      const int key = pc / (D / VEC), col = pc % (D / VEC);
      *reinterpret_cast<vec_t*>(ks_lds + key * KLD + col * VEC) = kr[r];
    }
    if (tid < VTASKS) {
      const int kg = tid % (KC / 4), dg = tid / (KC / 4);
      const int pos = vt_pos_of_group4(kg);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vec4_t col;
        col[0] = vr[0][e];
        col[1] = vr[1][e];
        col[2] = vr[2][e];
        col[3] = vr[3][e];
        *reinterpret_cast<vec4_t*>(vt_lds + (4 * dg + e) * VLD + pos) = col;
      }
    }
  }
};



// Writes the 32 normalised output rows of every wave. The accumulator layout
// gives each lane 4-value slivers of one row, so a direct store would touch 32
// scattered rows 16 bytes at a time. Instead each wave transposes its rows
// through LDS (the key loop is over, the arena is free) and then stores whole
// rows: consecutive lanes cover one row's bytes contiguously.
template <typename O, int D>
__device__ __forceinline__ void store_rows(O* __restrict__ dst, char* smem, const f32x16 (&o)[D / 32],
                                           float inv, int64_t dst_index, int w, int lane) {
  constexpr int V = 16 / (int)sizeof(O);          // elements per 16-byte piece
  constexpr int SLD = D + V;                       // padded staging row
  constexpr int PPR = D / V;                       // pieces per row
  constexpr int RPI = 64 / PPR;                    // rows per wave-wide store
  typedef O vec4_t __attribute__((ext_vector_type(4)));
  typedef O vec_t __attribute__((ext_vector_type(V)));
  O* stage = reinterpret_cast<O*>(smem) + w * 32 * SLD;
  const int half = lane >> 5, r32 = lane & 31;
  __syncthreads();                                 // every wave is done with K/V
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      vec4_t val;
#pragma unroll
      for (int b = 0; b < 4; ++b) val[b] = from_f32<O>(o[dt][4 * aa + b] * inv);
      *reinterpret_cast<vec4_t*>(stage + r32 * SLD + 32 * dt + 8 * aa + 4 * half) = val;
    }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int rr = it * RPI + lane / PPR, pc = lane % PPR;
    const int64_t di = __shfl(dst_index, rr, 64);
    if (di >= 0)
      __builtin_nontemporal_store(*reinterpret_cast<const vec_t*>(stage + rr * SLD + pc * V),
                                  reinterpret_cast<vec_t*>(dst + di * D + pc * V));
  }
}

// Self-block epilogue with the merge of the parts (a5) folded in: the selected
// blocks' parts were written by the selected-block kernel, which runs first.
// Kimi发布MoBA突破性实现无限上下文, "PyTorch实现关键要点": the parts of a row are
// combined with an online softmax. Each part p is a normalised output o_p with
// the log-sum-exp lse_p of its disjoint key set, so over their union
//   out = sum_p exp(lse_p - m) o_p / sum_p exp(lse_p - m),  m = max_p lse_p,
//   lse = m + log(sum_p exp(lse_p - m)).
// The own part is rounded to the partials' type first (as a stored partial
// would be); a row of query block i has min(ks, i) selected parts. The rows are
// staged through LDS so each lane combines and stores 16 contiguous bytes.
template <typename T, int D>
__device__ __forceinline__ void merge_rows(const AttnArgs& a, char* smem,
                                           const f32x16 (&o)[D / 32], float inv, float lse_own,
                                           int64_t dst_index, int nsel, int w, int lane) {
  typedef typename PartType<T>::type P;
  constexpr int V = 16 / (int)sizeof(P);          // elements per 16-byte piece
  constexpr int SLD = D + V;                       // padded staging row
  constexpr int PPR = D / V;                       // pieces per row
  constexpr int RPI = 64 / PPR;                    // rows per wave-wide pass
  typedef P pvec4_t __attribute__((ext_vector_type(4)));
  typedef P pvec_t __attribute__((ext_vector_type(V)));
  typedef T tvec_t __attribute__((ext_vector_type(V)));
  P* stage = reinterpret_cast<P*>(smem) + w * 32 * SLD;
  const int half = lane >> 5, r32 = lane & 31;
  const P* __restrict__ o_sel = (const P*)a.sel_o;
  __syncthreads();                                 // every wave is done with K/V
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      pvec4_t val;
#pragma unroll
      for (int b = 0; b < 4; ++b) val[b] = from_f32<P>(o[dt][4 * aa + b] * inv);
      *reinterpret_cast<pvec4_t*>(stage + r32 * SLD + 32 * dt + 8 * aa + 4 * half) = val;
    }
  __syncthreads();
  // Each lane handles one 16-byte piece of rows rr = it * RPI + lane / PPR.
  // Up to two selected parts (top-3 and below) every load of all of the lane's
  // rows is issued before any is used, so the epilogue pays one memory latency
  // instead of one per row and part.
  constexpr int NIT = 32 / RPI;
  const int pc = lane % PPR;
  int64_t di[NIT];
  float ls[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    di[it] = __shfl(dst_index, it * RPI + lane / PPR, 64);
    ls[it] = __shfl(lse_own, it * RPI + lane / PPR, 64);
  }
  auto finish = [&](int it, float m, float den, const float (&acc)[V])
      __attribute__((always_inline)) {
    const float rinv = 1.f / den;
    tvec_t r;
#pragma unroll
    for (int b = 0; b < V; ++b) r[b] = from_f32<T>(acc[b] * rinv);
    __builtin_nontemporal_store(r, reinterpret_cast<tvec_t*>((T*)a.out + di[it] * D + pc * V));
    if (a.lse_out && pc == 0) a.lse_out[di[it]] = m + fast_log2(den) * kLn2;
  };
  auto own_part = [&](int it, float wgt, float (&acc)[V]) __attribute__((always_inline)) {
    const int rr = it * RPI + lane / PPR;
    const pvec_t x = *reinterpret_cast<const pvec_t*>(stage + rr * SLD + pc * V);
#pragma unroll
    for (int b = 0; b < V; ++b) acc[b] = to_f32(x[b]) * wgt;
  };
  if (a.ks <= 2) {
    float lsel[NIT][2];
    pvec_t px[NIT][2];
#pragma unroll
    for (int it = 0; it < NIT; ++it)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        lsel[it][sl] = -INFINITY;
        px[it][sl] = pvec_t{};
        if (di[it] >= 0 && sl < nsel) {
          const int64_t e = di[it] * a.ks + sl;
          lsel[it][sl] = a.sel_lse[e];
          px[it][sl] = __builtin_nontemporal_load(
              reinterpret_cast<const pvec_t*>(o_sel + e * D + pc * V));
        }
      }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (di[it] < 0) continue;
      const float m = fmaxf(fmaxf(ls[it], lsel[it][0]), lsel[it][1]);
      float wgt = fast_exp2((ls[it] - m) * kLog2e);
      float den = wgt;
      float acc[V];
      own_part(it, wgt, acc);
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        if (sl >= nsel) break;
        wgt = fast_exp2((lsel[it][sl] - m) * kLog2e);
        den += wgt;
#pragma unroll
        for (int b = 0; b < V; ++b) acc[b] += to_f32(px[it][sl][b]) * wgt;
      }
      finish(it, m, den, acc);
    }
  } else if constexpr (NIT <= 8) {
    // More parts (16-bit partials): part by part, two at a time, each step
    // loading those parts for all of the lane's rows at once, so that it pays
    // one memory latency for NIT rows. First the maximum LSE of every row, then
    // the weighted sum.
    float m[NIT], den[NIT], acc[NIT][V];
#pragma unroll
    for (int it = 0; it < NIT; ++it) m[it] = ls[it];
    for (int sl = 0; sl < nsel; ++sl) {
      float l[NIT];
#pragma unroll
      for (int it = 0; it < NIT; ++it)
        l[it] = (di[it] >= 0) ? a.sel_lse[di[it] * a.ks + sl] : -INFINITY;
#pragma unroll
      for (int it = 0; it < NIT; ++it) m[it] = fmaxf(m[it], l[it]);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const float wgt = fast_exp2((ls[it] - m[it]) * kLog2e);
      den[it] = wgt;
      own_part(it, wgt, acc[it]);
    }
    for (int sl = 0; sl < nsel; sl += 2) {
      const bool two = sl + 1 < nsel;
      float l[NIT][2];
      pvec_t x[NIT][2];
#pragma unroll
      for (int it = 0; it < NIT; ++it)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          l[it][j] = -INFINITY;
          x[it][j] = pvec_t{};
          if (di[it] >= 0 && (j == 0 || two)) {
            const int64_t e = di[it] * a.ks + sl + j;
            l[it][j] = a.sel_lse[e];
            x[it][j] = __builtin_nontemporal_load(
                reinterpret_cast<const pvec_t*>(o_sel + e * D + pc * V));
          }
        }
#pragma unroll
      for (int it = 0; it < NIT; ++it)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (j == 1 && !two) break;
          const float wgt = fast_exp2((l[it][j] - m[it]) * kLog2e);
          den[it] += wgt;
#pragma unroll
          for (int b = 0; b < V; ++b) acc[it][b] += to_f32(x[it][j][b]) * wgt;
        }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it)
      if (di[it] >= 0) finish(it, m[it], den[it], acc[it]);
  } else {
    // fp32 partials (twice the registers per piece): row by row
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (di[it] < 0) continue;
      float m = ls[it];
      for (int sl = 0; sl < nsel; ++sl) m = fmaxf(m, a.sel_lse[di[it] * a.ks + sl]);
      float wgt = fast_exp2((ls[it] - m) * kLog2e);
      float den = wgt;
      float acc[V];
      own_part(it, wgt, acc);
      for (int sl = 0; sl < nsel; ++sl) {
        const int64_t e = di[it] * a.ks + sl;
        wgt = fast_exp2((a.sel_lse[e] - m) * kLog2e);
        den += wgt;
        const pvec_t x = __builtin_nontemporal_load(
            reinterpret_cast<const pvec_t*>(o_sel + e * D + pc * V));
#pragma unroll
        for (int b = 0; b < V; ++b) acc[b] += to_f32(x[b]) * wgt;
      }
      finish(it, m, den, acc);
    }
  }
}

template <typename T, int D, int MODE>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) k_attn(AttnArgs a) {
  // The host pass only needs this kernel's signature (for its launch stub); the
  // body uses device-only builtins and is compiled in the device pass alone.
#if defined(__HIP_DEVICE_COMPILE__)
  typedef KVStage<T, D> Stage;
  typedef typename Frag<T>::type frag_t;
  // One LDS arena: two K buffers and two transposed-V buffers during the key
  // loop, then the output staging area of the epilogue.
  constexpr int KBUF = KC * Stage::KLD, VBUF = D * Stage::VLD;
  constexpr int ARENA_REG = (2 * KBUF + 2 * VBUF) * (int)sizeof(T);
  constexpr int ARENA_DMA = 4 * 2 * KC * D * (int)sizeof(T);      // four K+V buffers
  constexpr int ARENA = ((sizeof(T) == 2 && D == 128 && kAttnWaves == 8) && ARENA_DMA > ARENA_REG)
                            ? ARENA_DMA : ARENA_REG;
  __shared__ __attribute__((aligned(16))) char smem[ARENA];
  static_assert(8 * 32 * (D + 16 / sizeof(typename PartType<T>::type)) *
                        sizeof(typename PartType<T>::type) <= ARENA &&
                    8 * 32 * (D + 16 / sizeof(T)) * sizeof(T) <= ARENA,
                "output staging must fit in the LDS arena");
  T* const ks_base = reinterpret_cast<T*>(smem);
  T* const vt_base = ks_base + 2 * KBUF;

  const int64_t logical = xcd_logical(blockIdx.x, a.padded);
  if (logical >= a.ntiles) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int half = lane >> 5, r32 = lane & 31;
  const int group = a.hq / a.hkv;
  const T* __restrict__ q = (const T*)a.q;
  const T* __restrict__ k = (const T*)a.k;
  const T* __restrict__ v = (const T*)a.v;

  int g;                      // kv-head of the tile
  int64_t kbeg, kend;         // key range of the tile
  int64_t row = -1;           // this lane's row (token * hq + head), -1 if none
  int64_t dst_index = -1;     // where this lane's result goes (row or entry)
  int64_t wtok0 = 0;          // first token of the wave (causal modes)
  bool wave_live;             // the wave has at least one row
  int blk_i = 0;              // SELF: the tile's block index inside its sequence

  if (MODE == MODE_SELECTED) {
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
    wave_live = e0 < e1;
    if (e0 + r32 < e1) {
      const int32_t ev = a.entries[e0 + r32];
      dst_index = ev;
      row = ev / a.ks;
    }
  } else {
    const int tt = 32 * (8 / a.hg);
    const int nhs = a.hq / a.hg;
    int64_t blk_start, blk_end;
    int u, hs;
    if (MODE == MODE_SELF) {
      u = a.nu - 1 - (int)(logical % a.nu);
      const int64_t rest = logical / a.nu;
      hs = (int)(rest % nhs);
      const int64_t b = a.nb - 1 - rest / nhs;
      const int n = a.blk_seq[b], i = a.blk_local[b];
      blk_i = i;
      blk_start = (int64_t)a.cu[n] + (int64_t)i * a.block;
      blk_end = min(blk_start + a.block, (int64_t)a.cu[n + 1]);
    } else {
      const int n = (int)(logical % a.nseq);
      const int64_t rest = logical / a.nseq;
      u = a.nu - 1 - (int)(rest % a.nu);
      hs = (int)(rest / a.nu);
      blk_start = a.cu[n];
      blk_end = a.cu[n + 1];
    }
    const int64_t tok0 = blk_start + (int64_t)u * tt;
    if (tok0 >= blk_end) return;
    const int h = hs * a.hg + (w % a.hg);
    g = h / group;
    wtok0 = tok0 + (int64_t)(w / a.hg) * 32;
    wave_live = wtok0 < blk_end;
    kbeg = blk_start;
    kend = min(tok0 + tt, blk_end);
    if (wtok0 + r32 < blk_end) {
      row = (wtok0 + r32) * a.hq + h;
      dst_index = row;
    }
  }

  frag_t qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qf[kk] = (row >= 0) ? load8_stream(q + row * D + 16 * kk + 8 * half) : zero8<frag_t>();

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // ---- fragment fetchers for the two LDS layouts ----------------------------
  // DMA layout (16-bit inputs): per buffer K then V, each KC rows x D elements.
  constexpr bool kDMA = (sizeof(T) == 2) && (D == 128) && (kAttnWaves == 8);
  constexpr int DBUF = 2 * KC * D;                 // elements per DMA buffer (K + V)
  const int hx = half ^ swz(r32);                  // K piece xor for this lane's rows
  const int ml = lane & 15;
  const int vrow = 4 * half + (ml >> 2);           // V row (within 16) of this lane's tr reads
  const int vp = 2 * ((lane >> 4) & 1) + ((ml & 3) >> 1);
  const int vx0 = vp ^ swz(vrow), vx1 = vp ^ swz(vrow + 8);
  const int vbyte = (ml & 1) * 4;                  // element offset inside the 16-byte piece
  auto kfrag = [&](int buf, int kt, int kk) __attribute__((always_inline)) -> frag_t {
    if constexpr (kDMA) {
      const T* kb = ks_base + buf * DBUF + (32 * kt + r32) * D;
      return load8(kb + 8 * ((2 * kk) ^ hx));
    } else {
      return load8(ks_base + buf * KBUF + (32 * kt + r32) * Stage::KLD + 16 * kk + 8 * half);
    }
  };
  auto vfrag = [&](int buf, int dt, int qq) __attribute__((always_inline)) -> frag_t {
    if constexpr (kDMA) {
      // keys 32kt + 16mm + {4h .. 4h+3} and the same + 8; head dim 32dt + r32
      const int kt = qq >> 1, mm = qq & 1;
      const T* vb = ks_base + buf * DBUF + KC * D + (32 * kt + 16 * mm + vrow) * D;
      const T* p0 = vb + 8 * ((4 * dt) ^ vx0) + vbyte;
      const T* p1 = vb + 8 * D + 8 * ((4 * dt) ^ vx1) + vbyte;
      const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
      const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      i16x8 r;
      r[0] = x0[0]; r[1] = x0[1]; r[2] = x0[2]; r[3] = x0[3];
      r[4] = x1[0]; r[5] = x1[1]; r[6] = x1[2]; r[7] = x1[3];
      return __builtin_bit_cast(frag_t, r);
    } else {
      return load8(vt_base + buf * VBUF + (32 * dt + r32) * Stage::VLD + 16 * qq + 8 * half);
    }
  };

  // Multiply one staged chunk (LDS buffer `buf`, keys c0 .. c0+63) into the
  // wave's running softmax state.
  auto compute = [&](int buf, int64_t c0) __attribute__((always_inline)) {
    // Does this wave need the chunk at all (causal: some key <= some row), and
    // does any key of it lie after one of the wave's rows (then mask)?
    const bool wave_needs = (MODE == MODE_SELECTED) ? wave_live : (wave_live && c0 <= wtok0 + 31);
    const bool need_mask = (MODE != MODE_SELECTED) && (c0 + KC - 1 > wtok0);
    if (!wave_needs) return;
    // S^T for the chunk's two 32-key tiles: two independent MFMA chains, the
    // LDS fragments read two steps ahead of their use
    f32x16 s0, s1;
#pragma unroll
    for (int e = 0; e < 16; ++e) { s0[e] = 0.f; s1[e] = 0.f; }
    {
      frag_t ring[4];
      ring[0] = kfrag(buf, 0, 0);
      ring[1] = kfrag(buf, 1, 0);
      ring[2] = kfrag(buf, 0, 1);
      ring[3] = kfrag(buf, 1, 1);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        s0 = mma_k16(ring[(2 * kk) & 3], qf[kk], s0);
        if (kk + 2 < D / 16) ring[(2 * kk) & 3] = kfrag(buf, 0, kk + 2);
        s1 = mma_k16(ring[(2 * kk + 1) & 3], qf[kk], s1);
        if (kk + 2 < D / 16) ring[(2 * kk + 1) & 3] = kfrag(buf, 1, kk + 2);
      }
    }
    if (need_mask) {
      const int64_t tok = wtok0 + r32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t key = c0 + 8 * (e >> 2) + 4 * half + (e & 3);
        if (key > tok) s0[e] = -INFINITY;
        if (key + 32 > tok) s1[e] = -INFINITY;
      }
    }
    // running max on the raw scores (the scale is positive), then one fma + exp2
    float mx = vmax(s0[0], s1[0]);
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = vmax(vmax(mx, s0[e]), s1[e]);
    mx = vmax(mx, swap_half(mx));
    // m_run is each row's reference max (log2 domain). It is raised only when
    // some row's max exceeds it by more than 8: until then p <= 2^8, harmless
    // in fp32 sums and bf16 P, and O and l share the reference, so the result
    // is the same softmax. This removes most O rescales.
    const float m_cand = vmax(m_run, mx * a.scale_log2);
    if (__ballot(m_cand > m_run + 8.f)) {
      const float alpha = fast_exp2(m_run - m_cand);   // 0 while m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
      m_run = m_cand;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float p0[16], p1[16];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p0[e] = fast_exp2(fmaf(s0[e], a.scale_log2, -m_use));
      p1[e] = fast_exp2(fmaf(s1[e], a.scale_log2, -m_use));
      psum += p0[e] + p1[e];
    }
    l_run += psum;
    // O^T += V^T P^T; P^T comes straight from the score registers
    frag_t pf[4];
    pf[0] = pack8<T>(&p0[0]);
    pf[1] = pack8<T>(&p0[8]);
    pf[2] = pack8<T>(&p1[0]);
    pf[3] = pack8<T>(&p1[8]);
    {
      constexpr int NF = (D / 32) * 4;   // V^T fragments per chunk, step f = 4 * dt + qq
      frag_t ring[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) ring[f] = vfrag(buf, f >> 2, f & 3);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        o[f >> 2] = mma_k16(ring[f & 3], pf[f & 3], o[f >> 2]);
        if (f + 4 < NF) ring[f & 3] = vfrag(buf, (f + 4) >> 2, f & 3);
      }
    }
  };

  const int nch = (int)((kend - kbeg + KC - 1) / KC);
  if constexpr (kDMA) {
    // Four LDS buffers, three chunks in flight. Every wave issues 4 direct
    // loads per chunk (2 of K, 2 of V), always, with the chunk index clamped at
    // the end, so "chunk c+1 has landed" is exactly vmcnt(8) at the end of
    // iteration c. The barrier is a bare s_barrier after that explicit wait
    // (the compiler would otherwise wait for every load in flight).
    const int row_stride = a.hkv * D;
    const uint32_t smem_lds = lds_addr(ks_base);
    const int rowA = 8 * w + (lane >> 4), rowB = rowA + 4;
    const int pieceA = (lane & 15) ^ swz(rowA), pieceB = (lane & 15) ^ swz(rowB);
    auto issue = [&](int c) __attribute__((always_inline)) {
      const int cc = min(c, nch - 1);
      const int64_t c0 = kbeg + (int64_t)cc * KC;
      const int last = (int)min((int64_t)(KC - 1), kend - 1 - c0);
      const T* kb = k + (c0 * a.hkv + g) * D;
      const T* vb = v + (c0 * a.hkv + g) * D;
      const uint32_t dst = smem_lds + (uint32_t)((c & 3) * DBUF * 2 + 128 * w * 16);
      const int offA = min(rowA, last) * row_stride + 8 * pieceA;
      const int offB = min(rowB, last) * row_stride + 8 * pieceB;
      dma16(kb + offA, dst);
      dma16(kb + offB, dst + 1024u);
      dma16(vb + offA, dst + (uint32_t)(KC * D * 2));
      dma16(vb + offB, dst + (uint32_t)(KC * D * 2) + 1024u);
    };
    // The direct loads are invisible to the compiler's wait bookkeeping, so
    // the Q fragments are waited for here, explicitly, before any is issued.
    MOBA_WAIT_VM_LGKM0(0);
    issue(0);
    issue(1);
    issue(2);
    MOBA_WAIT_VM_LGKM0(8);
    bare_barrier();
    for (int c = 0; c < nch; ++c) {
      issue(c + 3);
      compute(c & 3, kbeg + (int64_t)c * KC);
      MOBA_WAIT_VM_LGKM0(8);
      bare_barrier();
    }
    // the clamped tail loads must land before the epilogue reuses the arena
    MOBA_WAIT_VM_LGKM0(0);
    bare_barrier();
  } else {
    // Two register sets hold chunks in flight: the loads of chunk c+2 are
    // issued before chunk c is multiplied and land in LDS only after chunk c+1
    // has been multiplied, so each load has two compute phases to arrive.
    Stage st0, st1;
    st0.load(k, v, kbeg, kend, a.hkv, g);
    st1.load(k, v, kbeg + (int64_t)min(1, nch - 1) * KC, kend, a.hkv, g);
    st0.store(ks_base, vt_base);
    __syncthreads();
    for (int c = 0; c < nch; c += 2) {
      const int64_t c0 = kbeg + (int64_t)c * KC;
      // Prefetches are issued unconditionally (past the end: the last chunk
      // again, unused) so that every path has the same loads in flight and the
      // wait before each LDS store only covers the older set.
      st0.load(k, v, kbeg + (int64_t)min(c + 2, nch - 1) * KC, kend, a.hkv, g);
      compute(0, c0);
      if (c + 1 < nch) st1.store(ks_base + KBUF, vt_base + VBUF);
      __syncthreads();
      if (c + 1 >= nch) break;
      st1.load(k, v, kbeg + (int64_t)min(c + 3, nch - 1) * KC, kend, a.hkv, g);
      compute(1, c0 + KC);
      if (c + 2 < nch) st0.store(ks_base, vt_base);
      __syncthreads();
    }
  }

  // epilogue: combine the two half-row sums, normalise, write
  const float l_tot = l_run + swap_half(l_run);
  const float inv = (row >= 0) ? 1.f / l_tot : 0.f;
  const float lse = (m_run + fast_log2(l_tot)) * kLn2;
  if (MODE == MODE_SELF && a.ks > 0) {
    merge_rows<T, D>(a, smem, o, inv, lse, dst_index, min(a.ks, blk_i), w, lane);
  } else if (MODE == MODE_SELECTED) {
    if (row >= 0 && half == 0) a.lse_part[dst_index] = lse;
    store_rows<typename PartType<T>::type, D>((typename PartType<T>::type*)a.o_part, smem, o,
                                              inv, dst_index, w, lane);
  } else {
    if (row >= 0 && half == 0 && a.lse_out) a.lse_out[dst_index] = lse;
    store_rows<T, D>((T*)a.out, smem, o, inv, dst_index, w, lane);
  }
#endif
}

// ---------------------------------------------------------------------------
// Selected-block and own-block attention for 16-bit inputs with D = 128, in
// 4-wave workgroups. The keys stream through two LDS buffers (K then V rows of
// a KCH-key chunk, the same swizzled layout and fragment reads as k_attn's
// direct-load path), one chunk in flight. Several workgroups share a CU, and
// one's tile prologue, epilogue and barrier waits overlap the others'
// products, which matters most when tiles are short (block 512: 16 chunks per
// selected tile; the own-block tiles of the causal triangle: 1 to B/64
// chunks). Every wave issues KCH/8 direct loads per chunk (KCH/4 rows of K and
// of V), so "chunk c+1 landed" is vmcnt(0) at the end of iteration c.
//   SELECTED (KCH = 32): a tile is 128 routed rows (4 waves x 32) of one
//     (block, kv head) list over the block's B keys; writes fp16 parts and their
//     LSE. Two 16 KB buffers, 34 KB with the output staging: three workgroups
//     per CU (three waves per SIMD, within the 168 registers that allows),
//     which measured 3 to 4 % faster than two workgroups on 64-key chunks.
//   SELF: a tile is 4 / hw groups of 32 consecutive tokens of one block for hw
//     q heads of one kv group (hw = gcd(G, 4), one wave per head and token
//     group, the heads sharing the K/V chunks), over the block's keys up to the
//     tile's last token with the causal mask; the epilogue merges the row's
//     selected parts (or, with no selection, writes the output). KCH = 32
//     (three workgroups per CU) stages one part at a time in the 32 KB the two
//     buffers span, each wave in its own 8 KB, with a memory latency per part;
//     KCH = 64 (two 32 KB buffers, two workgroups per CU) stages two parts at
//     a time and loads the first during the last chunk. The launch takes 32
//     while the parts are few for the block (k-1 <= B/128): at 1M tokens,
//     block 2048, top-3, the own-block kernel measured 23.4 -> 21.6 ms; with
//     block 512 the 64-key form is ahead from about six parts on.
template <int MODE, int KCH>
__global__ void __launch_bounds__(64 * kSelWaves)
__attribute__((amdgpu_waves_per_eu(KCH == 32 ? 3 : 2, KCH == 32 ? 3 : 2)))
k_attn4(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef bf16 T;
  constexpr int D = 128;
  typedef bf16x8 frag_t;
  typedef typename PartType<T>::type PT;
  static_assert((MODE == MODE_SELECTED || MODE == MODE_SELF) && (KCH == 32 || KCH == 64),
                "chunks of 32 or 64 keys");
  static_assert(sizeof(PT) == sizeof(T), "output staging sized for 16-bit outputs");
  constexpr int NT = KCH / 32;                     // 32-key score tiles per chunk
  constexpr int DBUF = 2 * KCH * D;                // K rows then V rows of one chunk
  constexpr int STAGE = kSelWaves * 32 * (D + 8);  // output staging (elements)
  constexpr int LDS_ELEMS = (STAGE > 2 * DBUF) ? STAGE : 2 * DBUF;
  __shared__ __attribute__((aligned(16))) T lds[LDS_ELEMS];
  const int64_t logical = xcd_logical(blockIdx.x, a.padded);
  if (logical >= a.ntiles) return;
  const int lane = threadIdx.x & 63;
  // the wave index in a scalar register: everything derived from it (heads,
  // token groups, row bases) stays scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, r32 = lane & 31;
  const T* __restrict__ q = (const T*)a.q;
  const T* __restrict__ k = (const T*)a.k;
  const T* __restrict__ v = (const T*)a.v;

  int g;
  int64_t kbeg, kend, row = -1, dst_index = -1;
  int64_t wtok0 = 0;          // SELF: the wave's first token
  bool wave_live = true;      // SELF: the wave has rows
  int blk_i = 0;              // SELF: the tile's block index in its sequence
  int64_t wrow0 = 0;          // SELF: output row of the wave's first token
  int wrows = 0;              // SELF: rows of the wave inside the block (0 .. 32)
  if constexpr (MODE == MODE_SELECTED) {
    const int64_t tile = logical;
    const int32_t* toffs = a.tile_offsets;
    if (tile >= toffs[a.nlists]) return;
    const int L = upper_index_wave(toffs, (int)a.nlists, tile, lane);
    const int64_t b = L / a.hkv;
    g = L % a.hkv;
    const int n = a.blk_seq[b], j = a.blk_local[b];
    kbeg = (int64_t)a.cu[n] + (int64_t)j * a.block;
    kend = kbeg + a.block;                         // a past block is full
    const int64_t e0 = (int64_t)a.list_offsets[L] + (tile - toffs[L]) * kSelRowsPerTile +
                       (int64_t)w * kRowsPerWave;
    const int64_t e1 = a.list_offsets[L + 1];
    if (e0 + r32 < e1) {
      const int32_t ev = a.entries[e0 + r32];
      dst_index = ev;
      row = ev / a.ks;
    }
  } else {
    const int group = a.hq / a.hkv;
    const int hw = (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
    const int tt = 32 * (kSelWaves / hw);
    const int u = a.nu - 1 - (int)(logical % a.nu);
    const int64_t rest = logical / a.nu;
    const int nhs = a.hq / hw;
    const int hs = (int)(rest % nhs);
    const int64_t b = a.nb - 1 - rest / nhs;
    const int n = a.blk_seq[b];
    blk_i = a.blk_local[b];
    const int64_t blk_start = (int64_t)a.cu[n] + (int64_t)blk_i * a.block;
    const int64_t blk_end = min(blk_start + a.block, (int64_t)a.cu[n + 1]);
    const int64_t tok0 = blk_start + (int64_t)u * tt;
    if (tok0 >= blk_end) return;
    const int h = hs * hw + (w % hw);
    g = h / group;
    wtok0 = tok0 + (int64_t)(w / hw) * 32;
    wave_live = wtok0 < blk_end;
    wrow0 = wtok0 * a.hq + h;
    wrows = (int)max((int64_t)0, min((int64_t)32, blk_end - wtok0));
    kbeg = blk_start;
    kend = min(tok0 + tt, blk_end);
    if (wtok0 + r32 < blk_end) {
      row = (wtok0 + r32) * a.hq + h;
      dst_index = row;
    }
  }
  frag_t qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qf[kk] = (row >= 0) ? load8_stream(q + row * D + 16 * kk + 8 * half) : zero8<frag_t>();
  // SELF with selected blocks: the epilogue merges the row's parts from LDS.
  // Part 0 is loaded during the last chunk into the buffer that chunk leaves
  // free, the others after the loop; the LSE of parts 0 and 1 come with Q.
  const int nsel = (MODE == MODE_SELF) ? min(a.ks, blk_i) : 0;
  const bool pref = MODE == MODE_SELF && nsel > 0;
  float lsel0 = -INFINITY, lsel1 = -INFINITY;
  if (KCH == 64 && pref && row >= 0) {
    lsel0 = a.sel_lse[dst_index * a.ks];
    if (nsel > 1) lsel1 = a.sel_lse[dst_index * a.ks + 1];
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int hx = half ^ swz(r32);
  const int ml = lane & 15;
  const int vrow = 4 * half + (ml >> 2);
  const int vp = 2 * ((lane >> 4) & 1) + ((ml & 3) >> 1);
  const int vx0 = vp ^ swz(vrow), vx1 = vp ^ swz(vrow + 8);
  const int vbyte = (ml & 1) * 4;
  auto kfrag = [&](int buf, int kt, int kk) __attribute__((always_inline)) -> frag_t {
    const T* kb = lds + buf * DBUF + (32 * kt + r32) * D;
    return load8(kb + 8 * ((2 * kk) ^ hx));
  };
  auto vfrag = [&](int buf, int dt, int qq) __attribute__((always_inline)) -> frag_t {
    // keys 32kt + 16mm + {4h .. 4h+3} and the same + 8; head dim 32dt + r32
    const int kt = qq >> 1, mm = qq & 1;
    const T* vb = lds + buf * DBUF + KCH * D + (32 * kt + 16 * mm + vrow) * D;
    const T* p0 = vb + 8 * ((4 * dt) ^ vx0) + vbyte;
    const T* p1 = vb + 8 * D + 8 * ((4 * dt) ^ vx1) + vbyte;
    const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
    const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 r;
    r[0] = x0[0]; r[1] = x0[1]; r[2] = x0[2]; r[3] = x0[3];
    r[4] = x1[0]; r[5] = x1[1]; r[6] = x1[2]; r[7] = x1[3];
    return __builtin_bit_cast(frag_t, r);
  };
  // one staged chunk (keys c0 .. c0+KCH-1) into the wave's running softmax
  // state (as in k_attn)
  auto compute = [&](int buf, int64_t c0) __attribute__((always_inline)) {
    if constexpr (MODE == MODE_SELF) {
      if (!wave_live || c0 > wtok0 + 31) return;   // every key after every row
    }
    f32x16 s[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[t][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int t = 0; t < NT; ++t) s[t] = mma_k16(kfrag(buf, t, kk), qf[kk], s[t]);
    if constexpr (MODE == MODE_SELF) {
      if (c0 + KCH - 1 > wtok0) {                   // some key after some row
        const int64_t tok = wtok0 + r32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t key = c0 + 8 * (e >> 2) + 4 * half + (e & 3);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if (key + 32 * t > tok) s[t][e] = -INFINITY;
        }
      }
    }
    float mx = s[0][0];
#pragma unroll
    for (int t = 1; t < NT; ++t) mx = vmax(mx, s[t][0]);
#pragma unroll
    for (int e = 1; e < 16; ++e)
#pragma unroll
      for (int t = 0; t < NT; ++t) mx = vmax(mx, s[t][e]);
    mx = vmax(mx, swap_half_valu(mx, lane));
    const float m_cand = vmax(m_run, mx * a.scale_log2);
    if (__ballot(m_cand > m_run + 8.f)) {
      const float alpha = fast_exp2(m_run - m_cand);   // 0 while m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
      m_run = m_cand;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float pr[NT][16];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float pe = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        pr[t][e] = fast_exp2(fmaf(s[t][e], a.scale_log2, -m_use));
        pe = (t == 0) ? pr[t][e] : pe + pr[t][e];
      }
      psum += pe;
    }
    l_run += psum;
    frag_t pf[2 * NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      pf[2 * t] = pack8<T>(&pr[t][0]);
      pf[2 * t + 1] = pack8<T>(&pr[t][8]);
    }
#pragma unroll
    for (int f = 0; f < (D / 32) * 2 * NT; ++f)
      o[f / (2 * NT)] =
          mma_k16(vfrag(buf, f / (2 * NT), f % (2 * NT)), pf[f % (2 * NT)], o[f / (2 * NT)]);
  };

  const int nch = (int)((kend - kbeg + KCH - 1) / KCH);
  const int row_stride = a.hkv * D;
  const uint32_t lds0 = lds_addr(lds);
  // chunk c into LDS buffer `buf` (the loop passes both as known constants
  // parities, so every LDS address of a chunk is a loop-invariant register plus
  // an immediate offset)
  auto issue = [&](int c, int buf) __attribute__((always_inline)) {
    const int64_t c0 = kbeg + (int64_t)min(c, nch - 1) * KCH;
    const T* kb = k + (c0 * a.hkv + g) * D;
    const T* vb = v + (c0 * a.hkv + g) * D;
    // SELF: keys past the tile's range (the last chunk of a causal tile) read
    // the range's last key: in bounds, and masked. (A selected block is whole
    // chunks: the block size is a multiple of 64.)
    const int last = (MODE == MODE_SELF) ? (int)min((int64_t)(KCH - 1), kend - 1 - c0) : KCH - 1;
    constexpr int WR = KCH / 4;                    // chunk rows per wave
    const uint32_t dst = lds0 + (uint32_t)(buf * DBUF * 2 + WR * w * 256);
#pragma unroll
    for (int i = 0; i < WR / 4; ++i) {
      const int r = WR * w + 4 * i + (lane >> 4);  // rows WR w .. WR w + WR - 1 of the chunk
      const int off = ((MODE == MODE_SELF) ? min(r, last) : r) * row_stride +
                      8 * ((lane & 15) ^ swz(r));
      if (i == 0) {                                // first loads from the chunk's bases
        dma16s<true>(kb, (uint32_t)off * 2u, dst);
        dma16s<true>(vb, (uint32_t)off * 2u, dst + (uint32_t)(KCH * D * 2));
      } else {
        dma16s<false>(kb, (uint32_t)off * 2u, dst + (uint32_t)(1024 * i));
        dma16s<false>(vb, (uint32_t)off * 2u, dst + (uint32_t)(KCH * D * 2 + 1024 * i));
      }
    }
  };
  // Part `part` of the wave's 32 rows into LDS buffer `buf`: the wave's 8 KB
  // quarter, row r at 256 r, piece p of the row at position p ^ swz(r) (the
  // 16-byte pieces of a row spread over the banks, so that the epilogue's reads
  // of one piece of 16 rows hit distinct banks). Rows past the block repeat its
  // last row; a wave without rows loads nothing.
  auto issue_part = [&](int part, int buf) __attribute__((always_inline)) {
    if (!wave_live) return;
    const char* pb = (const char*)a.sel_o + (((wrow0 * a.ks) + part) << 8);
    const uint32_t rbytes = (uint32_t)(a.hq * a.ks) << 8;   // one token to the next
    const uint32_t dst = lds0 + (uint32_t)(buf * DBUF * 2 + w * 8192);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4);
      const uint32_t off = (uint32_t)min(r, wrows - 1) * rbytes + 16u * ((lane & 15) ^ swz(r));
      if (i == 0) dma16s<true>(pb, off, dst);
      else dma16s<false>(pb, off, dst + (uint32_t)(1024 * i));
    }
  };
  // the Q fragments (compiler-visible loads) land before any direct load
  MOBA_WAIT_VM_LGKM0(0);
  issue(0, 0);
  MOBA_WAIT_VM_LGKM0(0);
  bare_barrier();
  // two chunks per trip, buffers 0 then 1, and an odd last chunk after the loop
  // (no exit in the middle of a trip: the compiler then keeps one register
  // assignment for the running state)
  int c = 0;
  for (; c + 1 < nch; c += 2) {
    issue(c + 1, 1);
    compute(0, kbeg + (int64_t)c * KCH);
    MOBA_WAIT_VM_LGKM0(0);
    bare_barrier();
    if (KCH == 64 && pref && c + 2 >= nch) issue_part(0, 0);   // the last chunk: part 0
    else issue(c + 2, 0);                          // (clamped past the end)
    compute(1, kbeg + (int64_t)(c + 1) * KCH);
    MOBA_WAIT_VM_LGKM0(0);
    bare_barrier();
  }
  if (c < nch) {
    if (KCH == 64 && pref) issue_part(0, 1);
    else issue(c + 1, 1);                          // clamped: the last chunk again
    compute(0, kbeg + (int64_t)c * KCH);
    MOBA_WAIT_VM_LGKM0(0);
    bare_barrier();
  }
  const float l_tot = l_run + swap_half(l_run);
  const float inv = (row >= 0) ? 1.f / l_tot : 0.f;
  const float lse = (m_run + fast_log2(l_tot)) * kLn2;
  if constexpr (MODE == MODE_SELECTED) {
    if (row >= 0 && half == 0) a.lse_part[dst_index] = lse;
    store_rows<PT, D>((PT*)a.o_part, (char*)lds, o, inv, dst_index, w, lane);
  } else {
    if (pref) {
      // Kimi发布MoBA突破性实现无限上下文, "PyTorch实现关键要点": the parts (own
      // block and the selected blocks, disjoint key sets) combine with the
      // online-softmax rule, out = sum_p e^(lse_p - m) o_p / sum_p e^(lse_p - m)
      // with m the largest lse_p. Each lane combines its own accumulator slivers
      // with the same slivers of the parts, read from LDS, two parts at a time
      // (one per buffer), rescaling what it holds when the maximum grows. Every
      // wave reads only the quarter of each buffer that it loaded itself.
      const int pb0 = nch & 1;                     // buffer holding part 0
      typedef PT pvec4_t __attribute__((ext_vector_type(4)));
      const char* rp = (const char*)lds + w * 8192 + r32 * 256 + 8 * half;
      float m = lse, den = 1.f, sc = inv;
      // 32-key chunks: the wave's 8 KB region of the 32 KB that the two
      // buffers span holds one part at a time
      for (int sl = 0; KCH == 32 && sl < nsel; ++sl) {
        MOBA_WAIT_VM_LGKM0(0);                     // the wave's reads of the region are done
        issue_part(sl, 0);
        const float la = (row >= 0) ? a.sel_lse[dst_index * a.ks + sl] : -INFINITY;
        MOBA_WAIT_VM_LGKM0(0);
        const float mn = fmaxf(m, la);
        const float alpha = fast_exp2((m - mn) * kLog2e);
        const float wa = fast_exp2((la - mn) * kLog2e);
        den = den * alpha + wa;
        const float so = sc * alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int aa = 0; aa < 4; ++aa) {
            const int pos = 16 * ((4 * dt + aa) ^ swz(r32));
            const pvec4_t xa = *(const pvec4_t*)(rp + pos);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              o[dt][4 * aa + e] = o[dt][4 * aa + e] * so + to_f32(xa[e]) * wa;
          }
        m = mn;
        sc = 1.f;
      }
      for (int sl = 0; KCH == 64 && sl < nsel; sl += 2) {
        const bool two = sl + 1 < nsel;
        float la = lsel0, lb = lsel1;
        if (sl > 0) {
          issue_part(sl, pb0);
          la = (row >= 0) ? a.sel_lse[dst_index * a.ks + sl] : -INFINITY;
          lb = (row >= 0 && two) ? a.sel_lse[dst_index * a.ks + sl + 1] : -INFINITY;
        }
        if (two) issue_part(sl + 1, pb0 ^ 1);      // (part 1: the last chunk's buffer)
        MOBA_WAIT_VM_LGKM0(0);
        bare_barrier();
        const float mn = fmaxf(fmaxf(m, la), lb);
        const float alpha = fast_exp2((m - mn) * kLog2e);
        const float wa = fast_exp2((la - mn) * kLog2e);
        const float wb = two ? fast_exp2((lb - mn) * kLog2e) : 0.f;
        den = den * alpha + wa + wb;
        const float so = sc * alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int aa = 0; aa < 4; ++aa) {
            const int pos = 16 * ((4 * dt + aa) ^ swz(r32));
            const pvec4_t xa = *(const pvec4_t*)(rp + pb0 * DBUF * 2 + pos);
            pvec4_t xb = pvec4_t{};
            if (two) xb = *(const pvec4_t*)(rp + (pb0 ^ 1) * DBUF * 2 + pos);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              o[dt][4 * aa + e] = o[dt][4 * aa + e] * so + to_f32(xa[e]) * wa + to_f32(xb[e]) * wb;
          }
        m = mn;
        sc = 1.f;
      }
      if (row >= 0 && half == 0 && a.lse_out) a.lse_out[dst_index] = m + fast_log2(den) * kLn2;
      store_rows<T, D>((T*)a.out, (char*)lds, o, 1.f / den, dst_index, w, lane);
    } else {
      if (row >= 0 && half == 0 && a.lse_out) a.lse_out[dst_index] = lse;
      store_rows<T, D>((T*)a.out, (char*)lds, o, inv, dst_index, w, lane);
    }
  }
#endif
}

template <int MODE>
static hipError_t attn_dispatch(const Plan& p, const AttnArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.padded), blk(512);
  if (p.dtype == MOBA_DTYPE_BF16) {
    if (p.d == 128) hipLaunchKernelGGL((k_attn<bf16, 128, MODE>), grid, blk, 0, s, a);
    else hipLaunchKernelGGL((k_attn<bf16, 64, MODE>), grid, blk, 0, s, a);
  } else {
    if (p.d == 128) hipLaunchKernelGGL((k_attn<float, 128, MODE>), grid, blk, 0, s, a);
    else hipLaunchKernelGGL((k_attn<float, 64, MODE>), grid, blk, 0, s, a);
  }
  return hipGetLastError();
}

static AttnArgs base_args(const Plan& p, const void* q, const void* k, const void* v,
                          const int32_t* cu) {
  AttnArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu = cu;
  a.nb = p.nb;
  a.nseq = p.nseq;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.hg = p.hg;
  a.block = p.block;
  a.ks = p.ks;
  a.scale_log2 = p.scale * kLog2e;
  return a;
}

hipError_t launch_attn_selected(const Plan& p, const void* q, const void* k, const void* v,
                                const int32_t* cu_dev, const Work& w, hipStream_t s) {
  if (p.ks == 0 || p.nentries == 0) return hipSuccess;
  AttnArgs a = base_args(p, q, k, v, cu_dev);
  a.blk_seq = w.blk_seq;
  a.blk_local = w.blk_local;
  a.list_offsets = w.list_offsets;
  a.tile_offsets = w.tile_offsets;
  a.entries = w.entries;
  a.nlists = p.nlists;
  a.o_part = w.o_sel;
  a.lse_part = w.lse_sel;
  a.ntiles = tile_bound(p, p.sel_rows);
  a.padded = pad8(a.ntiles);
  if (p.sel_rows == kSelRowsPerTile) {             // bf16, D = 128
    hipLaunchKernelGGL((k_attn4<MODE_SELECTED, 32>), dim3((unsigned)a.padded), dim3(64 * kSelWaves), 0,
                       s, a);
    return hipGetLastError();
  }
  return attn_dispatch<MODE_SELECTED>(p, a, s);
}

hipError_t launch_attn_self(const Plan& p, const void* q, const void* k, const void* v,
                            const int32_t* cu_dev, const Work& w, void* out, float* lse_out,
                            hipStream_t s) {
  if (p.nb == 0) return hipSuccess;
  AttnArgs a = base_args(p, q, k, v, cu_dev);
  a.blk_seq = w.blk_seq;
  a.blk_local = w.blk_local;
  a.sel_o = w.o_sel;
  a.sel_lse = w.lse_sel;
  a.out = out;
  a.lse_out = lse_out;
  if (p.dtype == MOBA_DTYPE_BF16 && p.d == 128) {
    // 4-wave tiles: hw = gcd(G, 4) heads x 4 / hw groups of 32 tokens
    a.nu = tiles_per_block(p, attn4_tokens(p));
    a.ntiles = self4_tile_count(p);
    a.padded = pad8(a.ntiles);
    // 32-key chunks (three workgroups per CU) unless the merge has many parts
    // for a short block: that form stages one part at a time
    if (p.ks * 128 <= p.block)
      hipLaunchKernelGGL((k_attn4<MODE_SELF, 32>), dim3((unsigned)a.padded), dim3(64 * kSelWaves),
                         0, s, a);
    else
      hipLaunchKernelGGL((k_attn4<MODE_SELF, 64>), dim3((unsigned)a.padded), dim3(64 * kSelWaves),
                         0, s, a);
    return hipGetLastError();
  }
  a.nu = tiles_per_block(p, tile_tokens8(p));
  a.ntiles = self8_tile_count(p);
  a.padded = pad8(a.ntiles);
  return attn_dispatch<MODE_SELF>(p, a, s);
}

hipError_t launch_attn_dense(const Plan& p, const void* q, const void* k, const void* v,
                             const int32_t* cu_dev, void* out, float* lse_out, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  AttnArgs a = base_args(p, q, k, v, cu_dev);
  a.out = out;
  a.lse_out = lse_out;
  a.nu = dense_tiles_per_seq(p);
  a.ntiles = dense_tile_count(p);
  a.padded = pad8(a.ntiles);
  return attn_dispatch<MODE_DENSE>(p, a, s);
}

}  // namespace moba
