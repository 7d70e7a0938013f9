// NEXT-2: gated decode and chunked-prefill continuation against a KV cache.
//
// MoBA README FAQ (issue #27, the entry on decoding): MoBA's gate also applies
// when tokens are generated one at a time against a KV cache. A new row at
// position p of sequence n attends exactly what the prefill's row p attends —
// its own block up to p, causally, plus the top-(topk-1) past blocks by the
// score of q against the mean-pooled keys ("Parameter-less Gating Mechanism";
// Kimi发布MoBA突破性实现无限上下文, "MoBA：基于块的混合注意力机制") — so the
// result is the prefill's row p. Past blocks are complete, so their pooled
// keys are cached once (k_kbar_append) and reused by every later step.
//
// Rows are few and each (row, head) attends its own key set, so these kernels
// are bound by HBM bytes, not by the matrix cores: VALU dot products, 16-byte
// coalesced K/V rows, and enough independent work items (row, head, part,
// 512-key segment) to fill the chip even for a single sequence.
#include "moba_plan.h"

namespace moba {

constexpr int kSeg = 512;   // keys per attention work item

// Sum over aligned groups of LANES (4, 8 or 16) lanes with DPP lane moves on
// the vector ALU (quad permutations, then the half-row and row mirrors)
// instead of LDS permutes: every lane of a group ends with the group's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                CTRL, 0xF, 0xF, true));
}
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 4 || LANES == 8 || LANES == 16, "groups of 4, 8 or 16 lanes");
  x += dpp_move<0xB1>(x);                        // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_move<0x4E>(x);                        // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LANES >= 8) x += dpp_move<0x141>(x);   // row_half_mirror: the other quad
  if constexpr (LANES >= 16) x += dpp_move<0x140>(x);  // row_mirror: the other half-row
  return x;
}

// Sequence and in-sequence position of new row r.
__device__ __forceinline__ void decode_row(const DecodeArgs& a, int64_t r, int& n, int64_t& p) {
  n = seq_of_token(a.cu_q, a.nseq, r);
  const int64_t len = (int64_t)a.cu_k[n + 1] - a.cu_k[n];
  const int64_t nq = (int64_t)a.cu_q[n + 1] - a.cu_q[n];
  p = len - nq + (r - a.cu_q[n]);
}

// ---------------------------------------------------------------------------
// Gate: one wave per (new row, q head). Lane l scores past blocks l, l+64, ...
// (fp32 dot products against the cached pooled keys, dimensions in ascending
// order) and keeps its best KM in a sorted register list; equal scores keep
// the earlier (lower) block. The wave then takes the best remaining candidate
// of all lanes min(topk-1, i) times — ties again to the lower block — and
// writes the kept blocks in ascending order, padded with -1.
template <typename T, int D, int KM>
__global__ void __launch_bounds__(256) k_dec_gate(DecodeArgs a) {
  __shared__ float qs[4][D];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t rh = (int64_t)blockIdx.x * 4 + wv;
  const bool live = rh < a.rows;
  const int64_t r = live ? rh / a.hq : 0;
  const int h = live ? (int)(rh % a.hq) : 0;
  if (live)
    for (int d = lane; d < D; d += 64) qs[wv][d] = to_f32(((const T*)a.q)[rh * D + d]);
  __syncthreads();
  if (!live) return;
  int n;
  int64_t p;
  decode_row(a, r, n, p);
  const int i = (int)(p / a.block);
  const int g = h / (a.hq / a.hkv);
  const int nk = min(a.ks, i);

  float bs[KM];
  int bj[KM];
#pragma unroll
  for (int t = 0; t < KM; ++t) {
    bs[t] = -INFINITY;
    bj[t] = 0x7fffffff;
  }
  for (int j = lane; j < i; j += 64) {
    const float4* kb = reinterpret_cast<const float4*>(
        a.kbar + (((int64_t)n * a.max_blocks + j) * a.hkv + g) * D);
    float sc = 0.f;
#pragma unroll 8
    for (int d4 = 0; d4 < D / 4; ++d4) {
      const float4 x = kb[d4];
      sc = fmaf(qs[wv][4 * d4 + 0], x.x, sc);
      sc = fmaf(qs[wv][4 * d4 + 1], x.y, sc);
      sc = fmaf(qs[wv][4 * d4 + 2], x.z, sc);
      sc = fmaf(qs[wv][4 * d4 + 3], x.w, sc);
    }
    // insertion by swaps: the candidate moves past every entry it beats strictly
    float ns = sc;
    int nj = j;
#pragma unroll
    for (int t = 0; t < KM; ++t) {
      const bool gt = ns > bs[t];
      const float ts = bs[t];
      const int tj = bj[t];
      bs[t] = gt ? ns : ts;
      bj[t] = gt ? nj : tj;
      ns = gt ? ts : ns;
      nj = gt ? tj : nj;
    }
  }
  int kept[KM];
#pragma unroll
  for (int s = 0; s < KM; ++s) {
    kept[s] = -1;
    if (s < nk) {
      float best = bs[0];
      int bjj = bj[0];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ob = __shfl_xor(best, off, 64);
        const int oj = __shfl_xor(bjj, off, 64);
        if (ob > best || (ob == best && oj < bjj)) {
          best = ob;
          bjj = oj;
        }
      }
      kept[s] = bjj;
      if (bj[0] == bjj) {   // the owning lane pops its head
#pragma unroll
        for (int t = 0; t + 1 < KM; ++t) {
          bs[t] = bs[t + 1];
          bj[t] = bj[t + 1];
        }
        bs[KM - 1] = -INFINITY;
        bj[KM - 1] = 0x7fffffff;
      }
    }
  }
  // ascending block order (nk <= KM, a few compare-exchanges)
#pragma unroll
  for (int x = 0; x < KM; ++x)
#pragma unroll
    for (int y = 0; y + 1 < KM; ++y) {
      const bool sw = (y + 1 < nk) && kept[y] > kept[y + 1];
      const int lo = sw ? kept[y + 1] : kept[y];
      const int hi = sw ? kept[y] : kept[y + 1];
      kept[y] = lo;
      kept[y + 1] = hi;
    }
  if (lane < a.ks) {
    int v = -1;
#pragma unroll
    for (int s = 0; s < KM; ++s) v = (lane == s) ? kept[s] : v;
    a.sel[rh * a.ks + lane] = (lane < nk) ? v : -1;
  }
}

// ---------------------------------------------------------------------------
// Attention parts: one wave per (row-head, part, segment). Part 0 is the own
// block up to the row (causal), part t >= 1 the t-th kept block. LPK lanes
// share one key row (16 bytes each, coalesced), KPS keys per step; scores are
// in the log2 domain (q pre-scaled by scale * log2 e) with an online softmax
// over 64-key chunks. Writes the segment's normalised output and its natural
// log-sum-exp (-inf for an empty segment).
// Items run in (row, head, part, segment) order, and each XCD takes one
// contiguous range of them (the grid is a multiple of 8 workgroups): the q heads
// of one kv group, which read the same own block and often the same selected
// blocks, then run at the same time on one XCD and fetch those keys and values
// from HBM once, through its L2. Dealt round-robin over the XCDs, each head
// fetched its blocks again.
template <typename T, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 3))) k_dec_part(DecodeArgs a) {
  constexpr int LPK = D / 8;      // lanes per key row, 8 values each
  constexpr int KPS = 64 / LPK;   // keys per step
  constexpr int NS = 64 / KPS;    // steps per 64-key chunk
  typedef T vec8 __attribute__((ext_vector_type(8)));
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nparts = a.ks + 1;
  const int64_t item = xcd_logical(blockIdx.x, gridDim.x) * 4 + wv;
  if (item >= a.rows * nparts * a.nseg) return;
  const int sg = (int)(item % a.nseg);
  const int t = (int)((item / a.nseg) % nparts);
  const int64_t rh = item / a.nseg / nparts;
  const int64_t r = rh / a.hq;
  const int h = (int)(rh % a.hq);
  int n;
  int64_t p;
  decode_row(a, r, n, p);
  const int i = (int)(p / a.block);
  const int g = h / (a.hq / a.hkv);
  int64_t kb, ke;
  if (t == 0) {
    kb = (int64_t)i * a.block;
    ke = p + 1;
  } else {
    const int j = a.sel[rh * a.ks + (t - 1)];
    kb = (int64_t)max(j, 0) * a.block;
    ke = (j >= 0) ? kb + a.block : kb;
  }
  const int64_t s0 = kb + (int64_t)sg * kSeg;
  const int64_t len = min(ke, s0 + kSeg) - s0;   // keys of this segment (may be <= 0)
  float* po = a.part_o + item * D;
  if (len <= 0) {
    if (lane == 0) a.part_lse[item] = -INFINITY;
    return;
  }
  const int kl = lane / LPK, dl = lane % LPK;
  float qv[8];
  {
    const vec8 x = *reinterpret_cast<const vec8*>((const T*)a.q + rh * D + 8 * dl);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = to_f32(x[e]) * a.scale_log2;
  }
  const int64_t stride = (int64_t)a.hkv * D;
  const T* kbase = (const T*)a.k + (((int64_t)a.cu_k[n] + s0) * a.hkv + g) * D + 8 * dl;
  const T* vbase = (const T*)a.v + (((int64_t)a.cu_k[n] + s0) * a.hkv + g) * D + 8 * dl;
  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int64_t c0 = 0; c0 < len; c0 += 64) {
    // all of the chunk's K and V pieces of this lane in flight at once (keys
    // past the segment end are clamped, always in range, and masked below)
    vec8 kx[NS], vx[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int64_t kk = min(c0 + kl + KPS * s, len - 1);
      kx[s] = *reinterpret_cast<const vec8*>(kbase + kk * stride);
      vx[s] = *reinterpret_cast<const vec8*>(vbase + kk * stride);
    }
    // keep the loads ahead of their uses (16-bit inputs; fp32 pieces are twice
    // the registers, so there the compiler keeps its own order)
    if constexpr (sizeof(T) == 2) __builtin_amdgcn_sched_barrier(0);
    float sc[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int64_t key = c0 + kl + KPS * s;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(qv[e], to_f32(kx[s][e]), dot);
      dot = group_sum<LPK>(dot);
      sc[s] = (key < len) ? dot : -INFINITY;
    }
    float cm = sc[0];
#pragma unroll
    for (int s = 1; s < NS; ++s) cm = fmaxf(cm, sc[s]);
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) cm = fmaxf(cm, __shfl_xor(cm, off, 64));
    const float mn = fmaxf(m, cm);
    const float alpha = fast_exp2(m - mn);   // 0 while m = -inf
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    m = mn;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float pk = fast_exp2(sc[s] - m);   // 0 for keys past the end
      l += pk;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(pk, to_f32(vx[s][e]), acc[e]);
    }
  }
  // sum over the key groups of the wave (lanes with the same dl)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    l += __shfl_xor(l, off, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
  }
  if (kl == 0) {
    const float inv = 1.f / l;
    float4 o0 = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    float4 o1 = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    reinterpret_cast<float4*>(po + 8 * dl)[0] = o0;
    reinterpret_cast<float4*>(po + 8 * dl)[1] = o1;
    if (dl == 0) a.part_lse[item] = (m + fast_log2(l)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Merge of a row's parts and segments through their log-sum-exp (Kimi发布MoBA
// 突破性实现无限上下文, "PyTorch实现关键要点": online-softmax combination):
// out = sum w_s o_s / sum w_s, w_s = exp(lse_s - m), m = max_s lse_s. One wave
// per row-head.
template <typename T, int D>
__global__ void __launch_bounds__(256) k_dec_merge(DecodeArgs a) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t rh = (int64_t)blockIdx.x * 4 + wv;
  if (rh >= a.rows) return;
  const int np = (a.ks + 1) * a.nseg;
  const int64_t base = rh * np;
  float m = -INFINITY;
  for (int s = 0; s < np; ++s) m = fmaxf(m, a.part_lse[base + s]);
  float den = 0.f;
  float acc[D / 64];
#pragma unroll
  for (int c = 0; c < D / 64; ++c) acc[c] = 0.f;
  for (int s = 0; s < np; ++s) {
    const float ls = a.part_lse[base + s];
    if (ls == -INFINITY) continue;
    const float w = fast_exp2((ls - m) * kLog2e);
    den += w;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) acc[c] += w * a.part_o[(base + s) * D + lane + 64 * c];
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int c = 0; c < D / 64; ++c)
    ((T*)a.out)[rh * D + lane + 64 * c] = from_f32<T>(acc[c] * inv);
  if (a.lse_out && lane == 0) a.lse_out[rh] = m + fast_log2(den) * kLn2;
}

template <int D, typename T>
static hipError_t decode_launch(const DecodeArgs& a, hipStream_t s) {
  const unsigned g_rows = (unsigned)((a.rows + 3) / 4);
  const int64_t items = a.rows * (a.ks + 1) * a.nseg;
  if (a.ks > 0) {
    if (a.ks <= 2)
      hipLaunchKernelGGL((k_dec_gate<T, D, 2>), dim3(g_rows), dim3(256), 0, s, a);
    else if (a.ks <= 4)
      hipLaunchKernelGGL((k_dec_gate<T, D, 4>), dim3(g_rows), dim3(256), 0, s, a);
    else if (a.ks <= 8)
      hipLaunchKernelGGL((k_dec_gate<T, D, 8>), dim3(g_rows), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_dec_gate<T, D, 16>), dim3(g_rows), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t part_wgs = ((items + 3) / 4 + 7) / 8 * 8;
  hipLaunchKernelGGL((k_dec_part<T, D>), dim3((unsigned)part_wgs), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_dec_merge<T, D>), dim3(g_rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

int decode_segments(int block) { return (block + kSeg - 1) / kSeg; }

hipError_t launch_decode(const DecodeArgs& a, int d, int dtype, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (dtype == MOBA_DTYPE_BF16)
    return d == 128 ? decode_launch<128, bf16>(a, s) : decode_launch<64, bf16>(a, s);
  return d == 128 ? decode_launch<128, float>(a, s) : decode_launch<64, float>(a, s);
}

}  // namespace moba
