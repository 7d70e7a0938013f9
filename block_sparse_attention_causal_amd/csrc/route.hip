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
//   4. scatter: per chunk, a few waves each take a slice of its entries in row
//               order, count them per block, take their first places from a
//               prefix over the waves, and rank equal block ids with ballots, so
//               rows ascend inside every list.
// The result is identical on every run.
#include "moba_plan.h"

namespace moba {

// Chunk (query block b, kv head g) of workgroup id x, for the count and scatter
// grids of 8 * ceil(nb / 8) * hkv workgroups: ids go round-robin over the 8
// XCDs, so block b goes to XCD b mod 8 and its hkv chunks run there one after
// another. Those chunks read the same 256-byte rows of sel (32 bytes each) and
// share them in that XCD's L2, while consecutive blocks still spread over the
// XCDs. (With b * hkv + g the kv heads of a block went to eight XCDs, each
// fetching whole rows: four times sel's bytes from DRAM at 1M tokens.)
__device__ __forceinline__ int64_t chunk_block(int64_t x, int hkv) {
  return ((x >> 3) / hkv) * 8 + (x & 7);
}
__device__ __forceinline__ int chunk_head(int64_t x, int hkv) { return (int)((x >> 3) % hkv); }

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
                                                     int64_t nb, int hq, int hkv, int block,
                                                     int ks, FastDiv div_pt, FastDiv div_ks,
                                                     int32_t* __restrict__ hist) {
  extern __shared__ int32_t cnt[];
  const int64_t b = chunk_block(blockIdx.x, hkv);
  if (b >= nb) return;
  const int g = chunk_head(blockIdx.x, hkv);
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
  // eight loads in flight before their counts go to LDS: the loads take a
  // clamped index (entry total-1 stands in past the end) so that none sits
  // under a branch, which would make the compiler wait for each. A lane counts
  // a run of equal ids in a register and adds the run to LDS when the id
  // changes: with a stride that G (k-1) divides, a lane keeps one head and slot,
  // whose rows often choose the same block, and the lanes of a wave that add to
  // one LDS word at once would otherwise be serialised.
  constexpr int NL = 8;
  int run_j = -1, run_n = 0;
  for (int e0 = threadIdx.x; e0 < total; e0 += 256 * NL) {
    int jv[NL];
    bool ok[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int e = e0 + 256 * u;
      const int ec = min(e, total - 1);
      const int t = (int)fdiv((uint32_t)ec, div_pt);
      const int r = ec - t * per_tok;
      jv[u] = base[t * hq * ks + r];
      // only ids a row can hold: at most min(ks, i) valid slots, each in [0, i)
      ok[u] = e < total && (r - (int)fdiv((uint32_t)r, div_ks) * ks) < nvalid;
    }
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int j = (ok[u] && jv[u] >= 0 && jv[u] < i) ? jv[u] : -1;
      if (j != run_j) {
        if (run_j >= 0) atomicAdd(&cnt[run_j], run_n);
        run_j = j;
        run_n = 0;
      }
      ++run_n;
    }
  }
  if (run_j >= 0) atomicAdd(&cnt[run_j], run_n);
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

// One workgroup of W waves per chunk (query block i, kv-head g). The chunk's
// entries (in row order) are cut into W consecutive slices, one per wave. Each
// wave counts its slice's entries per block into LDS, a prefix over the waves
// gives every wave its first place in each block's segment of the list, and each
// wave then walks its slice 64 entries at a time, ranking equal block ids with
// ballots: rows ascend within every list, as with one wave walking the chunk.
__global__ void __launch_bounds__(512) k_route_scatter(const int32_t* __restrict__ sel,
                                                      const int32_t* __restrict__ cu,
                                                      const int32_t* __restrict__ blk_base,
                                                      const int32_t* __restrict__ tri_base,
                                                      const int32_t* __restrict__ blk_seq,
                                                      const int32_t* __restrict__ blk_local,
                                                      const int32_t* __restrict__ chunk_off,
                                                      const int32_t* __restrict__ list_offsets,
                                                      int64_t nb, int hq, int hkv, int block,
                                                      int ks, FastDiv div_pt, FastDiv div_ks,
                                                      int32_t* __restrict__ entries) {
  extern __shared__ int32_t next[];                // [W][i]: per wave, per block
  const int64_t b = chunk_block(blockIdx.x, hkv);
  if (b >= nb) return;
  const int g = chunk_head(blockIdx.x, hkv);
  const int n = blk_seq[b], i = blk_local[b];
  if (i == 0) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, W = blockDim.x >> 6;
  const int group = hq / hkv;
  const int nbn = blk_base[n + 1] - blk_base[n];
  const int64_t gb0 = blk_base[n];
  const int64_t tri0 = tri_index(tri_base, n, nbn, g, i, 0);
  const int64_t s0 = (int64_t)cu[n] + (int64_t)i * block;
  const int64_t len = min((int64_t)block, (int64_t)cu[n + 1] - s0);
  const int per_tok = group * ks;
  const int total = (int)len * per_tok;            // below T * hq * ks < 2^31
  const int nbits = (i <= 1) ? 0 : 32 - __clz(i - 1);
  const int nvalid = min(ks, i);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // the wave's slice [e_lo, e_hi) of the chunk's entries, whole steps of 64
  const int slice = (total + 64 * W - 1) / (64 * W) * 64;
  const int e_lo = min(total, w * slice), e_hi = min(total, e_lo + slice);
  // entry e of the chunk: its row, slot and block id (-1 outside the slice).
  // The load takes a clamped index (e_hi - 1 >= 0: every chunk has entries),
  // so it never sits under a branch and several stay in flight.
  auto fetch = [&](int e, int64_t& row, int& slot) __attribute__((always_inline)) -> int {
    const int ec = min(e, e_hi - 1);
    const int t = (int)fdiv((uint32_t)ec, div_pt);
    const int r = ec - t * per_tok;
    const int h = (int)fdiv((uint32_t)r, div_ks);
    slot = r - h * ks;
    row = (s0 + t) * hq + (int64_t)g * group + h;
    // -1 past the slice by an or, not a select: a select lets the compiler move
    // the load under a branch again
    return sel[row * ks + slot] | -(int)(e >= e_hi);
  };
  int32_t* mine = next + w * i;
  for (int j = threadIdx.x; j < W * i; j += blockDim.x) next[j] = 0;
  __syncthreads();
  // (loads in flight and runs counted in registers as in k_route_count)
  constexpr int NL = 8;
  int run_j = -1, run_n = 0;
  for (int e0 = e_lo + lane; e0 < e_hi; e0 += 64 * NL) {
    int jv[NL];
    bool ok[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      int64_t row;
      int slot;
      jv[u] = fetch(e0 + 64 * u, row, slot);
      ok[u] = slot < nvalid;
    }
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int j = (ok[u] && jv[u] >= 0 && jv[u] < i) ? jv[u] : -1;
      if (j != run_j) {
        if (run_j >= 0) atomicAdd(&mine[run_j], run_n);
        run_j = j;
        run_n = 0;
      }
      ++run_n;
    }
  }
  if (run_j >= 0) atomicAdd(&mine[run_j], run_n);
  __syncthreads();
  // counts -> first places: the list's segment for this chunk, then wave by wave
  for (int j = threadIdx.x; j < i; j += blockDim.x) {
    int32_t at = list_offsets[(gb0 + j) * hkv + g] + chunk_off[tri0 + j];
    for (int v = 0; v < W; ++v) {
      const int32_t cnt = next[v * i + j];
      next[v * i + j] = at;
      at += cnt;
    }
  }
  __syncthreads();
  // Rank pass, in batches of RB steps of 64 entries: the next batch's ids are
  // loaded while this batch ranks, the ranking touches only LDS (per-wave
  // counters) and ballots, and the batch's entry stores go out together at its
  // end, so a wave pays about one memory round trip per batch rather than one
  // per step (a store between a step's load and its use makes the compiler
  // wait for both). A wave's own LDS accesses take effect in program order, so
  // its counters need no barrier between steps. An id is -1 for entries past
  // the slice and for slots a row cannot hold.
  constexpr int RB = 8;
  auto fetch_id = [&](int e, int& val) __attribute__((always_inline)) -> int {
    int64_t row;
    int slot;
    const int jv = fetch(e, row, slot);
    val = (int)(row * ks + slot);
    return jv | -(int)(slot >= nvalid);
  };
  int jq[RB], vq[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) jq[u] = fetch_id(e_lo + 64 * u + lane, vq[u]);
  // the previous step's ids and peer masks: when no lane's id changed (a lane
  // keeps one head and slot from step to step when G (k-1) divides 64, and a
  // head's rows often choose the same blocks), the peers are the same too
  int j_prev = -2;
  uint64_t peers_prev = 0;
  for (int e00 = e_lo; e00 < e_hi; e00 += 64 * RB) {
    int jc[RB], vc[RB], at[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      jc[u] = jq[u];
      vc[u] = vq[u];
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) jq[u] = fetch_id(e00 + 64 * (RB + u) + lane, vq[u]);
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      at[u] = -1;
      if (e00 + 64 * u >= e_hi) continue;          // wave-uniform
      const int j0 = jc[u];
      const bool act = j0 >= 0 && j0 < i;
      const int j = act ? j0 : -1;
      uint64_t peers;
      if (__ballot(j != j_prev) == 0) {
        peers = peers_prev;
      } else {
        peers = __ballot(act);
        for (int bit = 0; bit < nbits; ++bit) {
          const bool on = act && ((j >> bit) & 1);
          const uint64_t m = __ballot(on);
          peers &= on ? m : ~m;
        }
      }
      j_prev = j;
      peers_prev = peers;
      if (act) {
        const int32_t base = mine[j];
        at[u] = base + __popcll(peers & below);
        if ((peers & below) == 0) mine[j] = base + __popcll(peers);
      }
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int u = 0; u < RB; ++u)
      if (at[u] >= 0) entries[at[u]] = vc[u];
  }
}

hipError_t launch_route(const Plan& p, const int32_t* sel, const int32_t* cu_dev, const Work& w,
                        int rows_per_tile,
                        int32_t* list_offsets, int32_t* entries, hipStream_t s) {
  if (p.ks == 0 || p.nb == 0) return hipSuccess;
  const unsigned nchunks = (unsigned)(pad8(p.nb) * p.hkv);
  const size_t lds = (size_t)p.max_nb * sizeof(int32_t);
  // entry e of a chunk: token e / (G ks), head and slot from e mod (G ks)
  const FastDiv div_pt = make_fastdiv((uint32_t)((p.hq / p.hkv) * p.ks));
  const FastDiv div_ks = make_fastdiv((uint32_t)p.ks);
  hipLaunchKernelGGL(k_route_count, dim3(nchunks), dim3(256), lds, s, sel, cu_dev, w.blk_base,
                     w.tri_base, w.blk_seq, w.blk_local, p.nb, p.hq, p.hkv, p.block, p.ks,
                     div_pt, div_ks, w.hist);
  hipLaunchKernelGGL(k_route_lists, dim3((unsigned)((p.nlists + 3) / 4)), dim3(256), 0, s,
                     w.hist, w.blk_base, w.tri_base, w.blk_seq, w.blk_local, p.hkv, p.nlists,
                     w.chunk_off, w.list_count);
  hipLaunchKernelGGL(k_route_offsets, dim3(1), dim3(1024), 0, s, w.list_count, p.nlists,
                     rows_per_tile, list_offsets, w.tile_offsets);
  // as many waves per chunk as the per-wave counters fit in 64 KB of LDS (8 for
  // sequences of up to 2048 blocks)
  int waves = 8;
  while (waves > 1 && (size_t)waves * p.max_nb * sizeof(int32_t) > 65536) waves >>= 1;
  hipLaunchKernelGGL(k_route_scatter, dim3(nchunks), dim3(64 * waves), lds * waves, s, sel,
                     cu_dev, w.blk_base, w.tri_base, w.blk_seq, w.blk_local, w.chunk_off,
                     list_offsets, p.nb, p.hq, p.hkv, p.block, p.ks, div_pt, div_ks, entries);
  return hipGetLastError();
}

}  // namespace moba
