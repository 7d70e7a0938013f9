// Host-side plan of one MoBA forward call: sizes, workspace carving, launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moba.h"
#include "moba_device.h"

namespace moba {

constexpr int kRowsPerWave = 32;           // one 32-row MFMA tile per wave
constexpr int kGateWaves = 8;              // gate workgroups: 512 threads
// Attention workgroups of the general kernels (fp32, or D = 64): 8 waves (512
// threads), one per CU; all eight share each staged K/V chunk. Their backward
// uses 8-wave tiles too.
constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kRowsPerTile = kRowsPerWave * kAttnWaves;   // routed rows per 8-wave tile
// The attention kernels for 16-bit inputs with D = 128 (forward, and the
// backward's dQ) run 4-wave workgroups, two or three per CU: selected-block
// tiles of 128 routed rows, own-block tiles of 128 rows (heads x tokens).
constexpr int kSelWaves = 4;
constexpr int kSelRowsPerTile = kRowsPerWave * kSelWaves;
// Backward dK/dV tiles: 8 waves x 32 keys for 16-bit inputs with D = 128, else 4 waves.
constexpr int kDkvWaves = 8;
constexpr int kBkvWaves = 4;
constexpr int kMaxSelected = 16;           // topk - 1 limit (per-lane register lists)
constexpr int kMaxBlocksPerSeq = 16384;    // per-sequence block counters live in LDS

struct Plan {
  // problem
  int32_t nseq = 0;
  int64_t T = 0;
  int32_t hq = 0, hkv = 0, d = 0, dtype = 0;
  int32_t group = 1;        // Hq / Hkv
  int32_t hg = 1;           // heads of one group that share a gate workgroup: gcd(group, 8)
  int32_t block = 0, topk = 1, ks = 0;   // ks = topk - 1
  float scale = 0.f;
  // derived sizes
  int64_t nb = 0;           // total blocks over all sequences
  int32_t max_nb = 0;       // largest per-sequence block count
  int64_t max_len = 0;      // longest sequence
  int64_t span = 0;         // longest block: min(block, max_len); per-block tile grids use it
  int64_t tri = 0;          // sum_n Hkv * NB_n * (NB_n - 1) / 2 (route histograms)
  int64_t nlists = 0;       // nb * hkv
  int64_t nentries = 0;     // routed (row, slot) pairs
  int32_t sel_rows = 0;     // routed rows per selected-block tile (forward and dQ)
  // workspace offsets (bytes); -1 when not used
  size_t off_blk_base = 0, off_tri_base = 0, off_blk_seq = 0, off_blk_local = 0;
  size_t off_kbar = 0, off_kbar_split = 0, off_kbar_err = 0, off_gate_bound = 0;
  size_t off_gate_flags = 0, off_sel = 0;
  int64_t gate_tiles = 0;   // tiles of the gate grid (one screening flag each)
  size_t off_hist = 0, off_chunk_off = 0, off_list_count = 0, off_list_offsets = 0;
  size_t off_tile_offsets = 0, off_entries = 0;
  size_t off_o_sel = 0, off_lse_sel = 0;
  size_t total = 0;
};

// Launch bound on the tiles of the routed lists cut into tiles of `rows` rows: each list
// adds at most one partial tile. A grid sized by the bound of another tile size would
// leave workgroups idle and, under the XCD mapping, whole XCDs without work.
inline int64_t tile_bound(const Plan& p, int rows) { return p.nentries / rows + p.nlists + 1; }

// ---- launch grids, shared by the launchers and the plan's size check -------------
// Grids whose tile order is XCD-interleaved are padded to a multiple of the 8 XCDs.
inline int64_t pad8(int64_t n) { return (n + 7) / 8 * 8; }
// Tokens per tile of the 8-wave per-block tiles (gate, general attention kernels, dQ
// passes): 8 waves of 32 rows, hg heads side by side.
inline int tile_tokens8(const Plan& p) { return 32 * (8 / p.hg); }
// Heads side by side in an own-block tile of the 4-wave kernels: gcd(G, 4).
inline int attn4_heads(const Plan& p) {
  return (p.group % 4 == 0) ? 4 : (p.group % 2 == 0) ? 2 : 1;
}
inline int attn4_tokens(const Plan& p) { return 32 * (kSelWaves / attn4_heads(p)); }
// Tiles along the tokens of one block: no block is longer than `span`.
inline int tiles_per_block(const Plan& p, int tokens_per_tile) {
  return (int)((p.span + tokens_per_tile - 1) / tokens_per_tile);
}
inline int64_t gate_tile_count(const Plan& p) {
  return p.nb * tiles_per_block(p, tile_tokens8(p)) * (p.hq / p.hg);
}
inline int64_t self8_tile_count(const Plan& p) {
  return p.nb * tiles_per_block(p, tile_tokens8(p)) * (p.hq / p.hg);
}
inline int64_t self4_tile_count(const Plan& p) {
  return p.nb * tiles_per_block(p, attn4_tokens(p)) * (p.hq / attn4_heads(p));
}
inline int dense_tiles_per_seq(const Plan& p) {
  return (int)((p.max_len + tile_tokens8(p) - 1) / tile_tokens8(p));
}
inline int64_t dense_tile_count(const Plan& p) {
  return (int64_t)p.nseq * dense_tiles_per_seq(p) * (p.hq / p.hg);
}
// Work-items of the largest grid any launch of a forward (or, with `backward`, a
// backward) call on this plan makes; HIP takes fewer than 2^32 per grid dimension.
int64_t max_grid_items(const Plan& p, bool backward);
constexpr int64_t kMaxGridItems = (int64_t(1) << 32) - 1;

// Fills `plan` from validated arguments. Returns MOBA_OK or an error status and
// writes a message into `err` (size errlen).
moba_status_t make_plan(const int32_t* cu_host, int32_t nseq, const moba_shape_t* shape,
                        int32_t block, int32_t topk, bool need_block, Plan* plan, char* err,
                        size_t errlen);

// Device pointers into a carved workspace.
struct Work {
  int32_t* blk_base;     // [nseq + 1] first global block id of each sequence
  int32_t* tri_base;     // [nseq + 1] first route-histogram slot of each sequence
  int32_t* blk_seq;      // [nb] sequence of each global block
  int32_t* blk_local;    // [nb] index of each global block inside its sequence
  float* kbar;           // [nb, hkv, d] pooled keys
  bf16* kbar_split;      // [3, nb, hkv, d] pooled keys as hi + mid + lo bf16 (bf16 inputs)
  float* kbar_err;       // [nb, hkv] error bound of the hi term of each pooled key (bf16)
  float* gate_bound;     // [nseq, hkv] max of kbar_err over the sequence's blocks
  uint8_t* gate_flags;   // [gate_tiles] 1: a row of the tile needs the exact gate
  int32_t* sel;          // [T, hq, ks] selected blocks
  int32_t* hist;         // [tri] per (query block, kv-head) counts per past block
  int32_t* chunk_off;    // [tri] start of each (query block, kv-head) inside each list
  int32_t* list_count;   // [nlists]
  int32_t* list_offsets; // [nlists + 1]
  int32_t* tile_offsets; // [nlists + 1]
  int32_t* entries;      // [nentries] row * ks + slot, grouped by list
  void* o_sel;           // [T * hq * ks, d] selected-block partial outputs (fp16 for bf16
                         // inputs, else fp32)
  float* lse_sel;        // [T * hq * ks]
};

Work carve(const Plan& p, void* base);

// Kernel launchers (all asynchronous on `stream`).
hipError_t launch_setup(const Plan& p, const int32_t* cu_dev, const Work& w, hipStream_t s);
hipError_t launch_pool(const Plan& p, const void* k, const int32_t* cu_dev, const Work& w,
                       float* kbar, hipStream_t s);
hipError_t launch_gate(const Plan& p, const void* q, const int32_t* cu_dev, const Work& w,
                       int32_t* sel, hipStream_t s);
hipError_t launch_route(const Plan& p, const int32_t* sel, const int32_t* cu_dev, const Work& w,
                        int rows_per_tile,
                        int32_t* list_offsets, int32_t* entries, hipStream_t s);
hipError_t launch_attn_selected(const Plan& p, const void* q, const void* k, const void* v,
                                const int32_t* cu_dev, const Work& w, hipStream_t s);
// Self-block causal attention; writes the final output, merging the
// selected-block parts (ks > 0) in its epilogue.
hipError_t launch_attn_self(const Plan& p, const void* q, const void* k, const void* v,
                            const int32_t* cu_dev, const Work& w, void* out, float* lse_out,
                            hipStream_t s);
hipError_t launch_attn_dense(const Plan& p, const void* q, const void* k, const void* v,
                             const int32_t* cu_dev, void* out, float* lse_out, hipStream_t s);

// Copies `rows` rows of `width` bytes (a multiple of 4) between two strided layouts.
hipError_t launch_copy_rows(const void* src, int64_t sstride, void* dst, int64_t dstride,
                            int64_t rows, int64_t width, hipStream_t s);

// ---- backward (NEXT-1) --------------------------------------------------------
hipError_t launch_backward(const Plan& p, const void* q, const void* k, const void* v,
                           const void* out, const float* lse, const void* dout,
                           const int32_t* cu_dev, const Work& w, float* delta, float* lse2,
                           float* dq_sel, void* dq, void* dk, void* dv, hipStream_t s);

// ---- decoding against a KV cache (NEXT-2) ----------------------------------
struct DecodeArgs {
  const void* q;            // [Tq, hq, d] new rows
  const void* k;            // [Tk, hkv, d] cache (new tokens already appended)
  const void* v;
  const int32_t* cu_q;      // [nseq + 1] new rows per sequence (device)
  const int32_t* cu_k;      // [nseq + 1] cache lengths (device)
  const float* kbar;        // [nseq * max_blocks, hkv, d] pooled-key cache
  int max_blocks, nseq, hq, hkv, block, ks, nseg;
  int64_t rows;             // Tq * hq
  float scale_log2;
  int32_t* sel;             // [rows, ks] kept blocks
  float* part_o;            // [rows, ks + 1, nseg, d] per-segment outputs
  float* part_lse;          // [rows, ks + 1, nseg]
  void* out;                // [Tq, hq, d]
  float* lse_out;           // optional [Tq, hq]
};
int decode_segments(int block);
hipError_t launch_decode(const DecodeArgs& a, int d, int dtype, hipStream_t s);
hipError_t launch_kbar_append(const void* k, const int32_t* cu_dev, const int32_t* prev_dev,
                              int nseq, int hkv, int d, int dtype, int block, int max_blocks,
                              int new_max, float* kbar, hipStream_t s);

}  // namespace moba
