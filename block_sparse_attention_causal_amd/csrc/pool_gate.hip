// Block table set-up, block mean-pool (a1) and gate + causal block mask + top-k (a2).
//
// Pool: one mean-pooled key per (block, kv-head) (Kimi发布MoBA突破性实现无限上下文,
// "PyTorch实现关键要点"; MoBA终极指南, "MoBA核心技术原理深度解析": pooling
// comes after the rotary embedding, which the caller has already applied).
// Gate: for every (token, q-head) row, score = q . Kbar[j] for each past block j
// of the row's sequence, keep the best topk-1 (MoBA README, "Parameter-less
// Gating Mechanism"; FAQ from issue #27: the own block is forced and not gated,
// so topk-1 past blocks are chosen and the final block is never a candidate).
#include "moba_plan.h"

namespace moba {

// ---------------------------------------------------------------------------
// Set-up: per-sequence first global block id and first histogram slot.
// One workgroup; each thread scans a contiguous slice of sequences.
__global__ void __launch_bounds__(256) k_setup(const int32_t* __restrict__ cu, int nseq,
                                               int block, int hkv, int32_t* blk_base,
                                               int32_t* tri_base) {
  __shared__ int64_t part_b[256], part_t[256];
  const int t = threadIdx.x;
  const int per = (nseq + 255) / 256;
  const int n0 = min(nseq, t * per), n1 = min(nseq, n0 + per);
  int64_t sb = 0, st = 0;
  for (int n = n0; n < n1; ++n) {
    int64_t nb = ((int64_t)cu[n + 1] - cu[n] + block - 1) / block;
    sb += nb;
    st += (int64_t)hkv * nb * (nb - 1) / 2;
  }
  part_b[t] = sb;
  part_t[t] = st;
  __syncthreads();
  if (t == 0) {
    int64_t ab = 0, at = 0;
    for (int i = 0; i < 256; ++i) {
      int64_t xb = part_b[i], xt = part_t[i];
      part_b[i] = ab;
      part_t[i] = at;
      ab += xb;
      at += xt;
    }
  }
  __syncthreads();
  int64_t ab = part_b[t], at = part_t[t];
  for (int n = n0; n < n1; ++n) {
    blk_base[n] = (int32_t)ab;
    tri_base[n] = (int32_t)at;
    int64_t nb = ((int64_t)cu[n + 1] - cu[n] + block - 1) / block;
    ab += nb;
    at += (int64_t)hkv * nb * (nb - 1) / 2;
  }
  if (n1 == nseq && n0 < n1) {
    blk_base[nseq] = (int32_t)ab;
    tri_base[nseq] = (int32_t)at;
  }
  if (nseq == 0 && t == 0) {
    blk_base[0] = 0;
    tri_base[0] = 0;
  }
}

// Sequence and in-sequence index of every global block.
__global__ void __launch_bounds__(256) k_block_info(const int32_t* __restrict__ blk_base, int nseq,
                                                    int64_t nb, int32_t* blk_seq,
                                                    int32_t* blk_local) {
  int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nb) return;
  int n = upper_index(blk_base, nseq, b);
  // skip empty sequences that share the same base
  while (n + 1 < nseq && blk_base[n + 1] <= b) ++n;
  blk_seq[b] = n;
  blk_local[b] = (int32_t)(b - blk_base[n]);
}

// The selection when no block has more than topk - 1 past blocks: a row of block i
// keeps every past block, so its list is 0 .. i - 1 (ascending) padded with -1.
// One workgroup per global block; the block's rows are contiguous in sel.
__global__ void __launch_bounds__(256) k_forced_sel(const int32_t* __restrict__ cu,
                                                    const int32_t* __restrict__ blk_seq,
                                                    const int32_t* __restrict__ blk_local,
                                                    int block, int hq, int ks,
                                                    int32_t* __restrict__ sel) {
  const int64_t b = blockIdx.x;
  const int n = blk_seq[b], i = blk_local[b];
  const int64_t s0 = (int64_t)cu[n] + (int64_t)i * block;
  const int64_t len = min((int64_t)block, (int64_t)cu[n + 1] - s0);
  const int64_t total = len * hq * ks;               // below T * hq * ks < 2^31
  int32_t* dst = sel + s0 * hq * ks;
  for (int64_t e = threadIdx.x; e < total; e += 256) {
    const int slot = (int)(e % ks);
    dst[e] = (slot < i) ? slot : -1;
  }
}

hipError_t launch_forced_sel(const Plan& p, const int32_t* cu_dev, const Work& w, int32_t* sel,
                             hipStream_t s) {
  if (p.ks == 0 || p.nb == 0) return hipSuccess;
  hipLaunchKernelGGL(k_forced_sel, dim3((unsigned)p.nb), dim3(256), 0, s, cu_dev, w.blk_seq,
                     w.blk_local, p.block, p.hq, p.ks, sel);
  return hipGetLastError();
}

hipError_t launch_setup(const Plan& p, const int32_t* cu_dev, const Work& w, hipStream_t s) {
  hipLaunchKernelGGL(k_setup, dim3(1), dim3(256), 0, s, cu_dev, p.nseq, p.block, p.hkv,
                     w.blk_base, w.tri_base);
  if (p.nb > 0)
    hipLaunchKernelGGL(k_block_info, dim3((unsigned)((p.nb + 255) / 256)), dim3(256), 0, s,
                       w.blk_base, p.nseq, p.nb, w.blk_seq, w.blk_local);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a1: block mean-pool. One workgroup per (block, kv-head); each thread owns 16
// bytes of columns and sums a strided subset of the block's rows in fp32; the
// row-lanes are then added in a fixed order, so the result is deterministic.
// Also writes the pooled key split into three bf16 terms (hi + mid + lo equals
// the fp32 value exactly for normal numbers), used by the bf16 gate.
// Mean of `len` key rows starting at token s0 for kv head g, by one
// 256-thread workgroup: 16-byte row slices per thread, four rows in flight,
// then a fixed-order reduction over the row lanes (the same order wherever a
// block is pooled). Threads c < D return the mean of column c; the rest NaN.
template <typename T, int D>
__device__ __forceinline__ float block_mean(const T* __restrict__ k, int64_t s0, int64_t len,
                                            int hkv, int g, float (&red)[256 / (D / (16 / sizeof(T)))][D + 1]) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CPR = D / VEC;          // threads per row
  constexpr int RL = 256 / CPR;         // row lanes
  const int cg = threadIdx.x % CPR, rl = threadIdx.x / CPR;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  const T* src = k + (s0 * hkv + g) * D + cg * VEC;
  const int64_t stride = (int64_t)hkv * D;
  typedef T vec_t __attribute__((ext_vector_type(VEC)));
  int64_t r = rl;
  for (; r + 3 * RL < len; r += 4 * RL) {
    vec_t x0 = *reinterpret_cast<const vec_t*>(src + r * stride);
    vec_t x1 = *reinterpret_cast<const vec_t*>(src + (r + RL) * stride);
    vec_t x2 = *reinterpret_cast<const vec_t*>(src + (r + 2 * RL) * stride);
    vec_t x3 = *reinterpret_cast<const vec_t*>(src + (r + 3 * RL) * stride);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += to_f32(x0[e]);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += to_f32(x1[e]);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += to_f32(x2[e]);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += to_f32(x3[e]);
  }
  for (; r < len; r += RL) {
    vec_t x0 = *reinterpret_cast<const vec_t*>(src + r * stride);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += to_f32(x0[e]);
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[rl][cg * VEC + e] = acc[e];
  __syncthreads();
  float mean = __builtin_nanf("");
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    float sum = 0.f;
    for (int l = 0; l < RL; ++l) sum += red[l][c];
    mean = sum / (float)len;
  }
  return mean;
}

template <typename T, int D>
__global__ void __launch_bounds__(256) k_pool(const T* __restrict__ k,
                                              const int32_t* __restrict__ cu,
                                              const int32_t* __restrict__ blk_seq,
                                              const int32_t* __restrict__ blk_local, int hkv,
                                              int block, int64_t nb, float* __restrict__ kbar,
                                              bf16* __restrict__ kbar_split,
                                              float* __restrict__ kbar_err) {
  __shared__ float red[256 / (D / (16 / sizeof(T)))][D + 1];
  __shared__ float err_part[2][D / 64];
  const int64_t b = blockIdx.x / hkv;
  const int g = blockIdx.x % hkv;
  const int n = blk_seq[b];
  const int i = blk_local[b];
  const int64_t s0 = (int64_t)cu[n] + (int64_t)i * block;
  const int64_t len = min((int64_t)block, (int64_t)cu[n + 1] - s0);
  const float mean = block_mean<T, D>(k, s0, len, hkv, g, red);
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    const int64_t o = (b * hkv + g) * D + c;
    kbar[o] = mean;
    if (kbar_split) {
      bf16 hi = (bf16)mean;
      float r1 = mean - (float)hi;
      bf16 mid = (bf16)r1;
      float r2 = r1 - (float)mid;
      const int64_t part = nb * hkv * D;
      kbar_split[o] = hi;
      kbar_split[part + o] = mid;
      kbar_split[2 * part + o] = (bf16)r2;
      // |mean - hi|^2 and |mean|^2 over the head dimension, per wave then
      // across the D / 64 waves that hold channels
      float e2 = r1 * r1, m2 = mean * mean;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        e2 += __shfl_xor(e2, off, 64);
        m2 += __shfl_xor(m2, off, 64);
      }
      if ((c & 63) == 0) {
        err_part[0][c >> 6] = e2;
        err_part[1][c >> 6] = m2;
      }
    }
  }
  if (kbar_split) {
    __syncthreads();
    if (threadIdx.x == 0) {
      float e2 = 0.f, m2 = 0.f;
#pragma unroll
      for (int u = 0; u < D / 64; ++u) { e2 += err_part[0][u]; m2 += err_part[1][u]; }
      // the hi term's error |mean - hi| plus a bound of the fp32 accumulation
      // of a D-term product (D 2^-24 relative, covered by 2^-16)
      kbar_err[b * hkv + g] = sqrtf(e2) * (1.f + 0x1p-10f) + sqrtf(m2) * 0x1p-16f;
    }
  }
}

hipError_t launch_pool(const Plan& p, const void* k, const int32_t* cu_dev, const Work& w,
                       float* kbar, hipStream_t s) {
  if (p.nb == 0) return hipSuccess;
  dim3 grid((unsigned)(p.nb * p.hkv));
  bf16* split = (p.dtype == MOBA_DTYPE_BF16) ? w.kbar_split : nullptr;
  float* err = w.kbar_err;
  if (p.dtype == MOBA_DTYPE_BF16) {
    if (p.d == 128)
      hipLaunchKernelGGL((k_pool<bf16, 128>), grid, dim3(256), 0, s, (const bf16*)k, cu_dev,
                         w.blk_seq, w.blk_local, p.hkv, p.block, p.nb, kbar, split, err);
    else
      hipLaunchKernelGGL((k_pool<bf16, 64>), grid, dim3(256), 0, s, (const bf16*)k, cu_dev,
                         w.blk_seq, w.blk_local, p.hkv, p.block, p.nb, kbar, split, err);
  } else {
    if (p.d == 128)
      hipLaunchKernelGGL((k_pool<float, 128>), grid, dim3(256), 0, s, (const float*)k, cu_dev,
                         w.blk_seq, w.blk_local, p.hkv, p.block, p.nb, kbar, split, err);
    else
      hipLaunchKernelGGL((k_pool<float, 64>), grid, dim3(256), 0, s, (const float*)k, cu_dev,
                         w.blk_seq, w.blk_local, p.hkv, p.block, p.nb, kbar, split, err);
  }
  return hipGetLastError();
}

// Pooled-key cache for decoding (NEXT-2): the blocks that became complete
// when sequence n grew from prev_len[n] to its cache length are pooled into
// kbar[(n * max_blocks + j) * hkv + g]. Same summation as k_pool, so a cached
// mean equals the one a prefill over the whole sequence computes.
template <typename T, int D>
__global__ void __launch_bounds__(256) k_kbar_append(const T* __restrict__ k,
                                                     const int32_t* __restrict__ cu,
                                                     const int32_t* __restrict__ prev_len,
                                                     int hkv, int block, int max_blocks,
                                                     int new_max, float* __restrict__ kbar) {
  __shared__ float red[256 / (D / (16 / sizeof(T)))][D + 1];
  const int g = blockIdx.x % hkv;
  const int jj = (blockIdx.x / hkv) % new_max;
  const int n = blockIdx.x / hkv / new_max;
  const int64_t len = (int64_t)cu[n + 1] - cu[n];
  const int j = prev_len[n] / block + jj;
  if ((int64_t)(j + 1) * block > len) return;     // not complete (uniform per workgroup)
  const int64_t s0 = (int64_t)cu[n] + (int64_t)j * block;
  const float mean = block_mean<T, D>(k, s0, block, hkv, g, red);
  if (threadIdx.x < D) kbar[(((int64_t)n * max_blocks + j) * hkv + g) * D + threadIdx.x] = mean;
}

hipError_t launch_kbar_append(const void* k, const int32_t* cu_dev, const int32_t* prev_dev,
                              int nseq, int hkv, int d, int dtype, int block, int max_blocks,
                              int new_max, float* kbar, hipStream_t s) {
  if (nseq == 0 || new_max == 0) return hipSuccess;
  dim3 grid((unsigned)((int64_t)nseq * new_max * hkv)), blk(256);
  if (dtype == MOBA_DTYPE_BF16) {
    if (d == 128)
      hipLaunchKernelGGL((k_kbar_append<bf16, 128>), grid, blk, 0, s, (const bf16*)k, cu_dev,
                         prev_dev, hkv, block, max_blocks, new_max, kbar);
    else
      hipLaunchKernelGGL((k_kbar_append<bf16, 64>), grid, blk, 0, s, (const bf16*)k, cu_dev,
                         prev_dev, hkv, block, max_blocks, new_max, kbar);
  } else {
    if (d == 128)
      hipLaunchKernelGGL((k_kbar_append<float, 128>), grid, blk, 0, s, (const float*)k, cu_dev,
                         prev_dev, hkv, block, max_blocks, new_max, kbar);
    else
      hipLaunchKernelGGL((k_kbar_append<float, 64>), grid, blk, 0, s, (const float*)k, cu_dev,
                         prev_dev, hkv, block, max_blocks, new_max, kbar);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a2: gate + causal block mask + top-(topk-1).
//
// Workgroup = 8 waves = (8/HG token sub-tiles of 32) x (HG q-heads of one kv
// group), all inside one block of one sequence, so they share one candidate
// range [0, i) and one kv-head's pooled keys. Pooled keys are staged through
// LDS 32 blocks at a time. Scores S^T = Kbar . Q^T come from the matrix cores
// (bf16: three passes over the hi/mid/lo split of Kbar, products exact, fp32
// accumulation; fp32: fp32 matrix ops). Lane l owns row l % 32 and sees 16 of
// every 32 candidate blocks; its running best list is kept sorted by (score
// descending, block ascending) in registers, then merged with the lane that
// holds the other 16 (lane l ^ 32). Ties therefore go to the lower block.
__device__ __forceinline__ bool better(float s1, int j1, float s2, int j2) {
  return s1 > s2 || (s1 == s2 && j1 < j2);
}

// Inserts (s, j) into the sorted list of ks entries; returns the score that
// ends up outside the list (the evicted last entry, or s itself).
template <int KB>
__device__ __forceinline__ float list_insert(float (&bs)[KB], int (&bj)[KB], int ks, float s,
                                             int j) {
#pragma unroll
  for (int p = 0; p < KB; ++p) {
    if (p < ks) {
      const bool b = better(s, j, bs[p], bj[p]);
      const float ts = bs[p];
      const int tj = bj[p];
      bs[p] = b ? s : ts;
      bj[p] = b ? j : tj;
      s = b ? ts : s;
      j = b ? tj : j;
    }
  }
  return s;
}

constexpr int kNoBlock = 0x7fffffff;

template <typename T, int D, int NP, int KB>
__global__ void __launch_bounds__(512) k_gate(const T* __restrict__ q,
                                              const int32_t* __restrict__ cu,
                                              const int32_t* __restrict__ blk_base,
                                              const int32_t* __restrict__ blk_seq,
                                              const int32_t* __restrict__ blk_local,
                                              const T* __restrict__ kparts, int64_t nb, int hq,
                                              int hkv, int hg, int block, int nu, int ks,
                                              int64_t ntiles, int64_t padded,
                                              const uint8_t* __restrict__ flags,
                                              int32_t* __restrict__ sel) {
  constexpr int PAD = 16 / sizeof(T);
  constexpr int LD = D + PAD;
  constexpr int VEC = 16 / sizeof(T);
  __shared__ __attribute__((aligned(16))) T kb[2][NP][32][LD];

  const int64_t logical = xcd_logical(blockIdx.x, padded);
  if (logical >= ntiles) return;
  if (flags && flags[logical] == 0) return;   // the screened selection is already exact
  const int tt = 32 * (8 / hg);                       // tokens per workgroup tile
  const int nhs = hq / hg;
  const int u = (int)(logical % nu);
  const int64_t rest = logical / nu;
  const int64_t b = nb - 1 - (rest % nb);
  const int hs = (int)(rest / nb);
  const int n = blk_seq[b];
  const int i = blk_local[b];
  const int64_t seq0 = cu[n];
  const int64_t blk_end = min(seq0 + (int64_t)(i + 1) * block, (int64_t)cu[n + 1]);
  const int64_t tok0 = seq0 + (int64_t)i * block + (int64_t)u * tt;
  if (tok0 >= blk_end || hs >= nhs) return;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int half = lane >> 5, r32 = lane & 31;
  const int h = hs * hg + (w % hg);
  const int g = h / (hq / hkv);
  const int64_t tok = tok0 + (int64_t)(w / hg) * 32 + r32;
  bool row_ok = tok < blk_end;
  int64_t row = tok * hq + h;
  bool wave_has = true;                               // the wave has rows to score
  if (flags) {
    // After the screened pass only the rows it left unsettled (their first
    // slot holds -2) are scored again, packed into the leading waves of the
    // tile; every row of a tile has the same candidates and kv head, so any
    // wave can take any of them. The waves left without rows still stage keys.
    __shared__ int64_t crow[256];
    __shared__ int ccount[8];
    const bool fl = row_ok && sel[row * ks] == -2;
    const uint64_t bal = __ballot(fl) & 0xffffffffull;   // one bit per row (half 0)
    if (lane == 0) ccount[w] = __popcll(bal);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int cv = ccount[v];
      before += (v < w) ? cv : 0;
      total += cv;
    }
    if (fl && half == 0) crow[before + __popcll(bal & ((1ull << r32) - 1))] = row;
    __syncthreads();
    const int ci = 32 * w + r32;
    row_ok = ci < total;
    row = row_ok ? crow[ci] : 0;
    wave_has = 32 * w < total;
  }

  float bs[KB];
  int bj[KB];
#pragma unroll
  for (int p = 0; p < KB; ++p) { bs[p] = -INFINITY; bj[p] = kNoBlock; }

  if (i > 0) {
    typedef typename Frag<T>::type frag_t;
    frag_t qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[kk] = row_ok ? load8(q + row * D + 16 * kk + 8 * half) : zero8<frag_t>();
    const int64_t gbase = blk_base[n];
    const int64_t part_stride = nb * hkv * D;
    float ws = -INFINITY;
    int wj = kNoBlock;
    // Pooled keys of 32 candidate blocks x NP parts per chunk, double-buffered
    // in LDS; the next chunk is fetched into registers while this one is used.
    constexpr int PIECES = NP * 32 * (D / VEC);
    constexpr int PPT = (PIECES + 511) / 512;             // pieces per thread
    typedef T vec_t __attribute__((ext_vector_type(VEC)));
    vec_t pre[PPT];
    auto fetch = [&](int j0) {
#pragma unroll
      for (int r = 0; r < PPT; ++r) {
        const int pc = threadIdx.x + 512 * r;
        if (PIECES % 512 == 0 || pc < PIECES) {
          const int part = pc / (32 * (D / VEC));
          const int rr = (pc / (D / VEC)) % 32;
          const int col = pc % (D / VEC);
          // blocks >= i (last chunk only) are clamped to block i-1 and their
          // scores discarded below; one branch-free load path
          const int jj = min(j0 + rr, i - 1);
          pre[r] = *reinterpret_cast<const vec_t*>(kparts + part * part_stride +
                                                   ((gbase + jj) * hkv + g) * D + col * VEC);
        }
      }
    };
    auto stash = [&](int buf) {
#pragma unroll
      for (int r = 0; r < PPT; ++r) {
        const int pc = threadIdx.x + 512 * r;
        if (PIECES % 512 == 0 || pc < PIECES) {
          const int part = pc / (32 * (D / VEC));
          const int rr = (pc / (D / VEC)) % 32;
          const int col = pc % (D / VEC);
          *reinterpret_cast<vec_t*>(&kb[buf][part][rr][col * VEC]) = pre[r];
        }
      }
    };
    fetch(0);
    stash(0);
    __syncthreads();
    int buf = 0;
    for (int j0 = 0; j0 < i; j0 += 32) {
      if (j0 + 32 < i) fetch(j0 + 32);
      if (wave_has) {
        f32x16 acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
        for (int part = 0; part < NP; ++part) {
#pragma unroll
          for (int kk = 0; kk < D / 16; ++kk) {
            frag_t a = load8(&kb[buf][part][r32][16 * kk + 8 * half]);
            acc = mma_k16(a, qf[kk], acc);
          }
        }
        // Candidates of this lane arrive in increasing block order, and every
        // block already in the list is lower, so a candidate enters only with a
        // strictly larger score than the list's worst (a tie keeps the lower
        // block). Blocks >= i (last chunk only) are not candidates.
        if (j0 + 32 > i) {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (j0 + 8 * (e >> 2) + 4 * half + (e & 3) >= i) acc[e] = -INFINITY;
        }
        // Insert the lane's scores above the cut best first, one per trip (a lane
        // rarely has more than one): the element equal to the maximum with the
        // lowest block, then its score is taken out and the maximum recomputed.
        // The wave runs as many trips as its busiest lane needs, rather than one
        // insertion for every position at which any lane has a candidate.
        auto max16 = [&]() __attribute__((always_inline)) {
          float m = acc[0];
#pragma unroll
          for (int e = 1; e < 16; e += 2)
            m = (e + 1 < 16) ? vmax(vmax(m, acc[e]), acc[e + 1]) : vmax(m, acc[e]);
          return m;
        };
        float mx = max16();
        while (mx > ws) {
          int eb = 15;
#pragma unroll
          for (int e = 15; e >= 0; --e) eb = (acc[e] == mx) ? e : eb;
          list_insert<KB>(bs, bj, ks, mx, j0 + 8 * (eb >> 2) + 4 * half + (eb & 3));
#pragma unroll
          for (int p = 0; p < KB; ++p)
            if (p == ks - 1) { ws = bs[p]; wj = bj[p]; }
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] = (e == eb) ? -INFINITY : acc[e];
          mx = max16();
        }
      }
      if (j0 + 32 < i) stash(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
    (void)wj;
    // merge with the partner lane's list (same row, the other 16 of each 32)
    float os[KB];
    int oj[KB];
#pragma unroll
    for (int p = 0; p < KB; ++p) { os[p] = swap_half(bs[p]); oj[p] = swap_half(bj[p]); }
#pragma unroll
    for (int p = 0; p < KB; ++p)
      if (p < ks && oj[p] != kNoBlock) list_insert<KB>(bs, bj, ks, os[p], oj[p]);
  }
  if (!row_ok || half != 0) return;
  // ascending block order; missing entries (kNoBlock) sort last and become -1
  int sj[KB];
#pragma unroll
  for (int p = 0; p < KB; ++p) sj[p] = kNoBlock;
#pragma unroll
  for (int p = 0; p < KB; ++p) {
    if (p < ks) {
      int j = bj[p];
#pragma unroll
      for (int r = 0; r < KB; ++r) {
        if (r < ks) {
          const bool lt = j < sj[r];
          const int t = sj[r];
          sj[r] = lt ? j : t;
          j = lt ? t : j;
        }
      }
    }
  }
  int32_t* dst = sel + row * ks;
#pragma unroll
  for (int p = 0; p < KB; ++p)
    if (p < ks) dst[p] = (sj[p] == kNoBlock) ? -1 : sj[p];
}

// Screened gate (bf16): one matrix-core pass over the hi term of the pooled
// keys gives s~_j = q . hi(Kbar_j) with |s_j - s~_j| <= |q| * err_j, err_j the
// bound the pool kernel stored (|Kbar_j - hi_j| plus the fp32 accumulation
// term). With E = |q| * max_j err_j over the sequence, if the k-th best and
// the (k+1)-th best s~ differ by more than 2E, then every kept block's exact
// score exceeds every other block's, and the kept set is exactly that of the
// exact scores. Rows where this fails (or where two s~ tie across the cut)
// flag their tile, and the exact three-pass kernel recomputes flagged tiles
// only. Tiles, lists and outputs as in k_gate; lists hold ks + 1 entries.
__global__ void __launch_bounds__(256) k_gate_bound(const int32_t* __restrict__ blk_base,
                                                    const float* __restrict__ kbar_err, int hkv,
                                                    float* __restrict__ bound) {
  __shared__ float red[4];
  const int n = blockIdx.x / hkv, g = blockIdx.x % hkv;
  const int b0 = blk_base[n], b1 = blk_base[n + 1];
  float m = 0.f;
  for (int b = b0 + (int)threadIdx.x; b < b1; b += 256) m = vmax(m, kbar_err[(int64_t)b * hkv + g]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = vmax(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) bound[blockIdx.x] = vmax(vmax(red[0], red[1]), vmax(red[2], red[3]));
}

// The low code bits of a packed score: (bits & ~m) | (code & m) in one
// bitfield insert (v_bfi_b32), the mask in a VGPR and the wave-uniform code in an
// SGPR (an and plus an or3, or a byte permute, otherwise).
__device__ __forceinline__ uint32_t insert_code(uint32_t m, uint32_t code, uint32_t bits) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "s"(code), "v"(bits));
  return r;
}

// max(a, b) of two values that are never NaN, in one full-rate v_max_f32 (the
// compiler's two-operand maximum is a half-rate v_maximum3_f32, and fmaxf would
// first canonicalise a value built from bits). The packed scores are finite (a
// score's exponent is never changed; masked places hold the lowest finite value)
// and the list starts at -inf.
__device__ __forceinline__ float max_not_nan(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// (four waves per SIMD: two workgroups per CU, as the LDS ring allows)
template <int D, int KB, int CB, int R>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4)))
k_gate_fast(const bf16* __restrict__ q, const int32_t* __restrict__ cu,
            const int32_t* __restrict__ blk_base, const int32_t* __restrict__ blk_seq,
            const int32_t* __restrict__ blk_local, const bf16* __restrict__ khi,
            const float* __restrict__ bound, int64_t nb, int hq, int hkv, int hg, int block,
            int nu, int nuf, int ks, int64_t ntiles, int64_t padded,
            uint8_t* __restrict__ flags, int32_t* __restrict__ sel) {
  // A workgroup covers R consecutive tiles of the exact gate (same block, same
  // heads): each wave holds R row sets of 32, one per tile, and every key
  // fragment read from LDS feeds R matrix products. Pooled hi keys stream
  // through an LDS ring of GB buffers (32 blocks each, rows of D bf16 in
  // 16-byte pieces, piece p of row r at p ^ swz(r) as in the attention kernels)
  // by direct loads. The ring turns in groups of GRP chunks with one barrier per
  // group (the waves' list upkeep differs from chunk to chunk; within a group
  // they drift instead of meeting at every chunk): a trip issues the group
  // GB / GRP - 1 ahead into the buffers the previous trip used, then works on
  // its own group. Each thread issues exactly one 16-byte load per chunk
  // (clamped past the end; with D = 64 the upper half of a buffer holds unused
  // rows), so "the next group has landed" is vmcnt(GB - 2 GRP) at a trip's end.
  constexpr int GB = 8;
  constexpr int GRP = 4;
  constexpr int KBUF = 512 * 8;                       // bf16 per buffer: 512 16-byte slots
  __shared__ __attribute__((aligned(16))) bf16 kb[GB][KBUF];

  const int64_t logical = xcd_logical(blockIdx.x, padded);
  if (logical >= ntiles) return;
  const int tt = 32 * (8 / hg);
  const int nhs = hq / hg;
  const int uf = (int)(logical % nuf);
  const int64_t rest = logical / nuf;
  const int64_t b = nb - 1 - (rest % nb);
  const int hs = (int)(rest / nb);
  const int n = blk_seq[b];
  const int i = blk_local[b];
  const int64_t seq0 = cu[n];
  const int64_t blk_end = min(seq0 + (int64_t)(i + 1) * block, (int64_t)cu[n + 1]);
  // exact-gate tile R uf + r is set r; its flag sits at (R uf + r) + nu rest
  const int64_t tok0 = seq0 + (int64_t)i * block + (int64_t)(R * uf) * tt;
  if (tok0 >= blk_end || hs >= nhs) {
    if (threadIdx.x < R && R * uf + (int)threadIdx.x < nu)
      flags[R * uf + threadIdx.x + nu * rest] = 0;
    return;
  }

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // scalar wave index
  const int half = lane >> 5, r32 = lane & 31;
  const int h = hs * hg + (w % hg);
  const int g = h / (hq / hkv);
  int64_t row[R];
  bool row_ok[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    // a set past the block's end (or past the last tile) has no valid rows
    const int64_t tok = tok0 + (int64_t)r * tt + (int64_t)(w / hg) * 32 + r32;
    row_ok[r] = tok < blk_end;
    row[r] = tok * hq + h;
  }

  // per set: the top-ks list as in k_gate, plus the best score left out of it
  float bs[R][KB];
  int bj[R][KB];
  float out_max[R];
  bool unsure[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int p = 0; p < KB; ++p) { bs[r][p] = -INFINITY; bj[r][p] = kNoBlock; }
    out_max[r] = -INFINITY;
    unsure[r] = false;
  }

  if (i > 0) {
    bf16x8 qf[R][D / 16];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        qf[r][kk] = row_ok[r] ? load8(q + row[r] * D + 16 * kk + 8 * half) : zero8<bf16x8>();
    const int64_t gbase = blk_base[n];
    const int nsteps = (i + 31) / 32;
    const uint32_t kb_lds = lds_addr(&kb[0][0]);
    constexpr int PIECES_ROW = D / 8;
    const int slot = threadIdx.x;                        // 16-byte slot in a buffer
    const int srow = slot / PIECES_ROW;
    const int spiece = (slot % PIECES_ROW) ^ (swz(srow) & (PIECES_ROW - 1));
    // the lane's piece of block srow, and the last block it may read: chunk st
    // reads block min(32 st + srow, i - 1) (chunks past the end repeat in-range
    // blocks, never used). (A running pointer instead of this multiply measured
    // the same and spilled registers in the loop of the four-entry lists.)
    const char* kpiece = (const char*)(khi + ((gbase + srow) * hkv + g) * D + 8 * spiece);
    const int kmax = i - 1 - srow;                       // may be negative: then block i - 1
    const int64_t kstride = (int64_t)hkv * D * (int64_t)sizeof(bf16);
    auto issue = [&](int st) __attribute__((always_inline)) {
      dma16(kpiece + (int64_t)min(32 * st, kmax) * kstride,
            kb_lds + (uint32_t)(((st % GB) * KBUF + 8 * (threadIdx.x - lane)) * 2));
    };
    const int rx = swz(r32) & (PIECES_ROW - 1);
    // blocks >= i score the lowest finite value (packing the low mantissa bits of
    // an infinity would make a NaN)
    constexpr float kMasked = -3.4028234663852886e38f;
    // S~^T of chunk st for every set (the LDS buffer holds it), blocks >= i masked
    auto scores = [&](int st, f32x16 (&acc)[R]) __attribute__((always_inline)) {
      const bf16* kr = &kb[st % GB][r32 * D];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[r][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a = load8(kr + 8 * (((2 * kk) | half) ^ rx));
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = mma_k16(a, qf[r][kk], acc[r]);
      }
      const int j0 = st * 32;
      if (j0 + 32 > i) {
        const int lim = i - j0 - 4 * half;               // positions >= lim are past i
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (8 * (e >> 2) + (e & 3) >= lim) acc[r][e] = kMasked;
      }
    };
    // Every score either enters the list (and whatever it evicts is left out)
    // or is left out at once, so out_max ends as the best score not kept.
    float tl[R][KB];                       // the packed chain's sorted values
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int p = 0; p < KB; ++p) tl[r][p] = -INFINITY;
    MOBA_WAIT_VM_LGKM0(0);                 // Q before any direct load
    for (int st = 0; st < GB - GRP; ++st) issue(st);
    MOBA_WAIT_VM_LGKM0(GB - 2 * GRP);
    bare_barrier();
    for (int st0 = 0; st0 < nsteps; st0 += GRP) {
#pragma unroll
      for (int x = 0; x < GRP; ++x) issue(st0 + GB - GRP + x);
#pragma unroll
      for (int x = 0; x < GRP; ++x) {
        const int st = st0 + x;
        if (GRP > 1 && st >= nsteps) break;
        f32x16 acc[R];
        scores(st, acc);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          // Every score passes through the lane's list without a branch. The
          // score carries its place in the lane's stream in its CB low mantissa
          // bits (chunk st, position e: code 16 st + e, put in with one bitfield
          // insert), so the list is a list of values and the block comes back
          // from the bits at the end. With the
          // values t sorted descending, admitting s gives t'_0 = max(t_0, s) and
          // t'_p = med3(t_{p-1}, t_p, s); the value that falls off the end,
          // min(t_last, s), is left out, and since nothing left out exceeds
          // t_last the best of them updates as med3(out, t_last, s). Replacing
          // CB low bits moves a score by less than 2^(CB-23) of itself; the
          // screen below adds that to its error bound, so the selection it
          // accepts is still the exact-score selection. Every packed value of a
          // lane is distinct (distinct codes).
          const uint32_t cbase = 16u * (uint32_t)st;
          const uint32_t cmask = (1u << CB) - 1u;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float sc = __uint_as_float(
                insert_code(cmask, cbase + (uint32_t)e, __float_as_uint(acc[r][e])));
            out_max[r] = __builtin_amdgcn_fmed3f(out_max[r], tl[r][KB - 1], sc);
#pragma unroll
            for (int p = KB - 1; p > 0; --p)
              tl[r][p] = __builtin_amdgcn_fmed3f(tl[r][p - 1], tl[r][p], sc);
            tl[r][0] = max_not_nan(tl[r][0], sc);
          }
        }
      }
      MOBA_WAIT_VM_LGKM0(GB - 2 * GRP);
      bare_barrier();
    }
    MOBA_WAIT_VM_LGKM0(0);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // codes to blocks; entries past ks are left out too, and entries below
      // every finite score never held a block (masked or never filled)
#pragma unroll
      for (int p = 0; p < KB; ++p) {
        const uint32_t cd = __float_as_uint(tl[r][p]) & ((1u << CB) - 1u);
        const bool real = tl[r][p] > -1e38f;
        if (p < ks) {
          bs[r][p] = real ? tl[r][p] : -INFINITY;
          bj[r][p] = real ? 32 * (int)(cd >> 4) + 8 * (int)((cd & 15) >> 2) + 4 * half +
                                (int)(cd & 3)
                          : kNoBlock;
        } else if (real) {
          out_max[r] = vmax(out_max[r], tl[r][p]);
        }
      }
      if (!(out_max[r] > -1e38f)) out_max[r] = -INFINITY;
      float os[KB];
      int oj[KB];
#pragma unroll
      for (int p = 0; p < KB; ++p) { os[p] = swap_half(bs[r][p]); oj[p] = swap_half(bj[r][p]); }
      out_max[r] = vmax(out_max[r], swap_half(out_max[r]));
#pragma unroll
      for (int p = 0; p < KB; ++p)
        if (p < ks && oj[p] != kNoBlock)
          out_max[r] = vmax(out_max[r], list_insert<KB>(bs[r], bj[r], ks, os[p], oj[p]));
      // the cut: the last kept entry against the best score left out
      if (row_ok[r] && i > ks) {
        float s_in = 0.f;
#pragma unroll
        for (int p = 0; p < KB; ++p)
          if (p == ks - 1) s_in = bs[r][p];
        // |q|^2 from packed bf16 pairs (products exact; the screen's bound has
        // room for the rounding of the sum)
        float qq = 0.f;
#pragma unroll
        for (int e = 0; e < D / 16; ++e) {
          typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
          typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
          const bf16x8_t v8 = __builtin_bit_cast(bf16x8_t, qf[r][e]);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const bf16x2_t v2 = {v8[2 * x], v8[2 * x + 1]};
            qq = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, qq, false);
          }
        }
        const float qnorm = sqrtf(qq + swap_half(qq));
        float e2 = 2.f * qnorm * bound[(int64_t)n * hkv + g] * (1.f + 0x1p-10f);
        // packed values sit within 2^(CB-23) of their score (twice that here)
        e2 += (float)(1u << CB) * 0x1p-22f * (fabsf(s_in) + fabsf(out_max[r]));
        unsure[r] = !(s_in - out_max[r] > e2);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int any = __syncthreads_or(unsure[r] ? 1 : 0);
    if (threadIdx.x == 0 && R * uf + r < nu) flags[R * uf + r + nu * rest] = any ? 1 : 0;
  }
  if (half != 0) return;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (!row_ok[r]) continue;
    int sj[KB];
#pragma unroll
    for (int p = 0; p < KB; ++p) sj[p] = kNoBlock;
#pragma unroll
    for (int p = 0; p < KB; ++p) {
      if (p < ks) {
        int j = bj[r][p];
#pragma unroll
        for (int x = 0; x < KB; ++x) {
          if (x < ks) {
            const bool lt = j < sj[x];
            const int t = sj[x];
            sj[x] = lt ? j : t;
            j = lt ? t : j;
          }
        }
      }
    }
    int32_t* dst = sel + row[r] * ks;
    // a row the screen cannot settle is marked -2 in its first slot: the exact
    // gate scores those rows only (its tile is flagged too)
#pragma unroll
    for (int p = 0; p < KB; ++p)
      if (p < ks) dst[p] = (p == 0 && unsure[r]) ? -2 : (sj[p] == kNoBlock) ? -1 : sj[p];
  }
}

template <typename T, int D, int NP>
static void gate_dispatch_kb(const Plan& p, const T* q, const int32_t* cu, const Work& w,
                             const T* parts, const uint8_t* flags, int32_t* sel, hipStream_t s,
                             int64_t ntiles, int64_t padded) {
  dim3 grid((unsigned)padded), blk(512);
#define MOBA_GATE(KBV)                                                                        \
  hipLaunchKernelGGL((k_gate<T, D, NP, KBV>), grid, blk, 0, s, q, cu, w.blk_base, w.blk_seq,  \
                     w.blk_local, parts, p.nb, p.hq, p.hkv, p.hg, p.block,                   \
                     tiles_per_block(p, tile_tokens8(p)), p.ks, ntiles, padded, flags, sel)
  if (p.ks <= 2) MOBA_GATE(2);
  else if (p.ks <= 4) MOBA_GATE(4);
  else if (p.ks <= 8) MOBA_GATE(8);
  else MOBA_GATE(16);
#undef MOBA_GATE
}

// Code bits of the screened pass's packed chain: 16 codes per chunk of 32 blocks.
// Sequences of up to 512 blocks take 8 bits, longer ones 12 (up to 8,192 blocks)
// or 13 bits; any topk - 1 <= 16.
static int gate_code_bits(const Plan& p) {
  if (p.max_nb <= 512) return 8;
  return p.max_nb <= 8192 ? 12 : 13;
}

// Row sets per wave in the screened pass: two halve the LDS reads per product and
// the tile set-up per row where the lists are short (few registers each).
template <int KB>
constexpr int gate_sets() { return KB <= 4 ? 2 : 1; }

template <int D>
static void gate_fast_dispatch(const Plan& p, const bf16* q, const int32_t* cu, const Work& w,
                               int32_t* sel, hipStream_t s) {
  const int nu = tiles_per_block(p, tile_tokens8(p));
  const int64_t rest = p.nb * (p.hq / p.hg);
#define MOBA_GATE_FAST(KBV, CBV)                                                              \
  do {                                                                                        \
    constexpr int R = gate_sets<KBV>();                                                       \
    const int nuf = (nu + R - 1) / R;                                                         \
    const int64_t nt = rest * nuf, pd = pad8(nt);                                             \
    hipLaunchKernelGGL((k_gate_fast<D, KBV, CBV, R>), dim3((unsigned)pd), dim3(512), 0, s, q, \
                       cu, w.blk_base, w.blk_seq, w.blk_local, w.kbar_split, w.gate_bound,    \
                       p.nb, p.hq, p.hkv, p.hg, p.block, nu, nuf, p.ks, nt, pd, w.gate_flags, \
                       sel);                                                                  \
  } while (0)
  const int cb = gate_code_bits(p);
  if (cb == 8) {
    if (p.ks <= 2) MOBA_GATE_FAST(2, 8);
    else if (p.ks <= 4) MOBA_GATE_FAST(4, 8);
    else if (p.ks <= 8) MOBA_GATE_FAST(8, 8);
    else if (p.ks <= 12) MOBA_GATE_FAST(12, 8);
    else MOBA_GATE_FAST(16, 8);
  } else if (cb == 12) {
    if (p.ks <= 2) MOBA_GATE_FAST(2, 12);
    else if (p.ks <= 4) MOBA_GATE_FAST(4, 12);
    else if (p.ks <= 8) MOBA_GATE_FAST(8, 12);
    else if (p.ks <= 12) MOBA_GATE_FAST(12, 12);
    else MOBA_GATE_FAST(16, 12);
  } else {
    if (p.ks <= 2) MOBA_GATE_FAST(2, 13);
    else if (p.ks <= 4) MOBA_GATE_FAST(4, 13);
    else if (p.ks <= 8) MOBA_GATE_FAST(8, 13);
    else if (p.ks <= 12) MOBA_GATE_FAST(12, 13);
    else MOBA_GATE_FAST(16, 13);
  }
#undef MOBA_GATE_FAST
}

hipError_t launch_gate(const Plan& p, const void* q, const int32_t* cu_dev, const Work& w,
                       int32_t* sel, hipStream_t s) {
  if (p.ks == 0 || p.nb == 0) return hipSuccess;
  const int64_t ntiles = gate_tile_count(p);
  const int64_t padded = pad8(ntiles);
  if (p.dtype == MOBA_DTYPE_BF16) {
    // Screened single bf16 pass, then the exact three-pass gate on flagged tiles
    // only.
    const bool screen = gate_code_bits(p) != 0;
    if (screen) {
      hipLaunchKernelGGL(k_gate_bound, dim3((unsigned)(p.nseq * p.hkv)), dim3(256), 0, s,
                         w.blk_base, w.kbar_err, p.hkv, w.gate_bound);
      if (p.d == 128)
        gate_fast_dispatch<128>(p, (const bf16*)q, cu_dev, w, sel, s);
      else
        gate_fast_dispatch<64>(p, (const bf16*)q, cu_dev, w, sel, s);
    }
    const uint8_t* flags = screen ? w.gate_flags : nullptr;
    if (p.d == 128)
      gate_dispatch_kb<bf16, 128, 3>(p, (const bf16*)q, cu_dev, w, w.kbar_split, flags, sel, s,
                                     ntiles, padded);
    else
      gate_dispatch_kb<bf16, 64, 3>(p, (const bf16*)q, cu_dev, w, w.kbar_split, flags, sel, s,
                                    ntiles, padded);
  } else {
    if (p.d == 128)
      gate_dispatch_kb<float, 128, 1>(p, (const float*)q, cu_dev, w, w.kbar, nullptr, sel, s,
                                      ntiles, padded);
    else
      gate_dispatch_kb<float, 64, 1>(p, (const float*)q, cu_dev, w, w.kbar, nullptr, sel, s,
                                     ntiles, padded);
  }
  return hipGetLastError();
}

}  // namespace moba
