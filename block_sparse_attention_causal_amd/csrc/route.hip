// a3: MoE-style routing. Inverts the query -> block selection into one list of
// (row, slot) entries per (global block, kv-head), so that the selected-block
// attention can run each block's keys against all the queries that chose it
// (MoBA README, abstract: MoE principles applied to attention; Kimi发布MoBA突破性
// 实现无限上下文, "PyTorch实现关键要点": data is organised by selected block
// before the attention).
//
// Counting sort without global atomics:
//   1. count:   per "chunk" (query block i, kv-head g) an LDS histogram over the
//               chunk's candidate blocks j < i;
//   2. lists:   per list (j, g), one wave: an exclusive scan over the chunks
//               i > j that can feed it -> each chunk's start inside the list,
//               and the list size;
//   3. offsets: one exclusive scan over list sizes (and over tiles of 256 rows);
//   4. scatter: per chunk, one wave walks its entries in row order and ranks
//               equal block ids with ballots, so rows ascend inside every list.
// The result is identical on every run.
#include "moba_plan.h"

namespace moba {

__device__ __forceinline__ int64_t tri_index(const int32_t* tri_base, int n, int nbn, int g,
                                             int i, int j) {
  return (int64_t)tri_base[n] + (int64_t)g * ((int64_t)nbn * (nbn - 1) / 2) +
         (int64_t)i * (i - 1) / 2 + j;
}

__global__ void __launch_bounds__(256) k_route_count(const int32_t* __restrict__ sel,
                                                     const int32_t* __restrict__ cu,
                                                     const int32_t* __restrict__ blk_base,
                                                     const int32_t* __restrict__ tri_base,
                                                     const int32_t* __restrict__ blk_seq,
                                                     const int32_t* __restrict__ blk_local,
                                                     int hq, int hkv, int block, int ks,
                                                     int32_t* __restrict__ hist) {
  extern __shared__ int32_t cnt[];
  const int64_t c = blockIdx.x;
  const int64_t b = c / hkv;
  const int g = (int)(c % hkv);
  const int n = blk_seq[b], i = blk_local[b];
  if (i == 0) return;
  const int group = hq / hkv;
  for (int j = threadIdx.x; j < i; j += 256) cnt[j] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)cu[n] + (int64_t)i * block;
  const int64_t len = min((int64_t)block, (int64_t)cu[n + 1] - s0);
  const int per_tok = group * ks;
  const int total = (int)len * per_tok;            // below T * hq * ks < 2^31
  const int nvalid = min(ks, i);
  const int32_t* base = sel + (s0 * hq + (int64_t)g * group) * ks;
  for (int e = threadIdx.x; e < total; e += 256) {
    const int t = e / per_tok;
    const int r = e % per_tok;
    const int j = base[t * hq * ks + r];
    // only ids a row can hold: at most min(ks, i) valid slots, each in [0, i)
    if (j >= 0 && j < i && (r % ks) < nvalid) atomicAdd(&cnt[j], 1);
  }
  __syncthreads();
  const int nbn = blk_base[n + 1] - blk_base[n];
  const int64_t dst = tri_index(tri_base, n, nbn, g, i, 0);
  for (int j = threadIdx.x; j < i; j += 256) hist[dst + j] = cnt[j];
}

// One wave per list (j, g): the lanes take 64 consecutive feeding chunks i at a
// time (independent loads), and a wave-wide inclusive scan turns their counts
// into each chunk's start inside the list.
__global__ void __launch_bounds__(256) k_route_lists(const int32_t* __restrict__ hist,
                                                     const int32_t* __restrict__ blk_base,
                                                     const int32_t* __restrict__ tri_base,
                                                     const int32_t* __restrict__ blk_seq,
                                                     const int32_t* __restrict__ blk_local,
                                                     int hkv, int64_t nlists,
                                                     int32_t* __restrict__ chunk_off,
                                                     int32_t* __restrict__ list_count) {
  const int64_t L = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (L >= nlists) return;
  const int lane = threadIdx.x & 63;
  const int64_t b = L / hkv;
  const int g = (int)(L % hkv);
  const int n = blk_seq[b], j = blk_local[b];
  const int nbn = blk_base[n + 1] - blk_base[n];
  int32_t run = 0;
  for (int i0 = j + 1; i0 < nbn; i0 += 64) {
    const int i = i0 + lane;
    int64_t idx = 0;
    int32_t h = 0;
    if (i < nbn) {
      idx = tri_index(tri_base, n, nbn, g, i, j);
      h = hist[idx];
    }
    int32_t x = h;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (i < nbn) chunk_off[idx] = run + x - h;
    run += __shfl(x, 63, 64);
  }
  if (lane == 0) list_count[L] = run;
}

// One workgroup of 1024 threads: exclusive scans of list sizes and tile counts.
__global__ void __launch_bounds__(1024) k_route_offsets(const int32_t* __restrict__ list_count,
                                                        int64_t nlists, int rows_per_tile,
                                                        int32_t* __restrict__ list_offsets,
                                                        int32_t* __restrict__ tile_offsets) {
  __shared__ int64_t pe[1024], pt[1024];
  const int t = threadIdx.x;
  const int64_t per = (nlists + 1023) / 1024;
  const int64_t a = min(nlists, (int64_t)t * per), z = min(nlists, a + per);
  int64_t se = 0, st = 0;
  for (int64_t L = a; L < z; ++L) {
    se += list_count[L];
    st += (list_count[L] + rows_per_tile - 1) / rows_per_tile;
  }
  pe[t] = se;
  pt[t] = st;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partial sums
  for (int off = 1; off < 1024; off <<= 1) {
    int64_t xe = (t >= off) ? pe[t - off] : 0, xt = (t >= off) ? pt[t - off] : 0;
    __syncthreads();
    pe[t] += xe;
    pt[t] += xt;
    __syncthreads();
  }
  int64_t re = pe[t] - se, rt = pt[t] - st;
  for (int64_t L = a; L < z; ++L) {
    list_offsets[L] = (int32_t)re;
    tile_offsets[L] = (int32_t)rt;
    re += list_count[L];
    rt += (list_count[L] + rows_per_tile - 1) / rows_per_tile;
  }
  if (t == 1023) {
    list_offsets[nlists] = (int32_t)pe[1023];
    tile_offsets[nlists] = (int32_t)pt[1023];
  }
}

// One wave per chunk (query block i, kv-head g).
__global__ void __launch_bounds__(64) k_route_scatter(const int32_t* __restrict__ sel,
                                                      const int32_t* __restrict__ cu,
                                                      const int32_t* __restrict__ blk_base,
                                                      const int32_t* __restrict__ tri_base,
                                                      const int32_t* __restrict__ blk_seq,
                                                      const int32_t* __restrict__ blk_local,
                                                      const int32_t* __restrict__ chunk_off,
                                                      const int32_t* __restrict__ list_offsets,
                                                      int hq, int hkv, int block, int ks,
                                                      int32_t* __restrict__ entries) {
  extern __shared__ int32_t next[];
  const int64_t c = blockIdx.x;
  const int64_t b = c / hkv;
  const int g = (int)(c % hkv);
  const int n = blk_seq[b], i = blk_local[b];
  if (i == 0) return;
  const int lane = threadIdx.x;
  const int group = hq / hkv;
  const int nbn = blk_base[n + 1] - blk_base[n];
  const int64_t gb0 = blk_base[n];
  const int64_t tri0 = tri_index(tri_base, n, nbn, g, i, 0);
  for (int j = lane; j < i; j += 64)
    next[j] = list_offsets[(gb0 + j) * hkv + g] + chunk_off[tri0 + j];
  __syncthreads();
  const int64_t s0 = (int64_t)cu[n] + (int64_t)i * block;
  const int64_t len = min((int64_t)block, (int64_t)cu[n + 1] - s0);
  const int per_tok = group * ks;
  const int total = (int)len * per_tok;            // below T * hq * ks < 2^31
  const int nbits = (i <= 1) ? 0 : 32 - __clz(i - 1);
  const int nvalid = min(ks, i);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // entry e of the chunk: its row, slot and block id (-1 past the end)
  auto fetch = [&](int e, int64_t& row, int& slot) __attribute__((always_inline)) -> int {
    row = 0;
    slot = 0;
    if (e >= total) return -1;
    const int t = e / per_tok;
    const int r = e % per_tok;
    slot = r % ks;
    row = (s0 + t) * hq + (int64_t)g * group + r / ks;
    return sel[row * ks + slot];
  };
  int64_t row_n;
  int slot_n;
  int j_n = fetch(lane, row_n, slot_n);
  // The workgroup is one wave: its LDS accesses take effect in program order,
  // so the counters need no barrier between steps (only the compiler must keep
  // the order), and the next step's ids are loaded before this step ranks.
  for (int e0 = 0; e0 < total; e0 += 64) {
    const int j = j_n;
    const int64_t row = row_n;
    const int slot = slot_n;
    j_n = fetch(e0 + 64 + lane, row_n, slot_n);
    const bool act = j >= 0 && j < i && slot < nvalid;
    uint64_t peers = __ballot(act);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = act && ((j >> bit) & 1);
      const uint64_t m = __ballot(on);
      peers &= on ? m : ~m;
    }
    if (act) {
      const int rank = __popcll(peers & below);
      const int32_t base = next[j];
      entries[base + rank] = (int32_t)(row * ks + slot);
      if ((peers & below) == 0) next[j] = base + __popcll(peers);
    }
    asm volatile("" ::: "memory");
  }
}

hipError_t launch_route(const Plan& p, const int32_t* sel, const int32_t* cu_dev, const Work& w,
                        int rows_per_tile,
                        int32_t* list_offsets, int32_t* entries, hipStream_t s) {
  if (p.ks == 0 || p.nb == 0) return hipSuccess;
  const unsigned nchunks = (unsigned)(p.nb * p.hkv);
  const size_t lds = (size_t)p.max_nb * sizeof(int32_t);
  hipLaunchKernelGGL(k_route_count, dim3(nchunks), dim3(256), lds, s, sel, cu_dev, w.blk_base,
                     w.tri_base, w.blk_seq, w.blk_local, p.hq, p.hkv, p.block, p.ks, w.hist);
  hipLaunchKernelGGL(k_route_lists, dim3((unsigned)((p.nlists + 3) / 4)), dim3(256), 0, s,
                     w.hist, w.blk_base, w.tri_base, w.blk_seq, w.blk_local, p.hkv, p.nlists,
                     w.chunk_off, w.list_count);
  hipLaunchKernelGGL(k_route_offsets, dim3(1), dim3(1024), 0, s, w.list_count, p.nlists,
                     rows_per_tile, list_offsets, w.tile_offsets);
  hipLaunchKernelGGL(k_route_scatter, dim3(nchunks), dim3(64), lds, s, sel, cu_dev, w.blk_base,
                     w.tri_base, w.blk_seq, w.blk_local, w.chunk_off, list_offsets, p.hq, p.hkv,
                     p.block, p.ks, entries);
  return hipGetLastError();
}

}  // namespace moba
