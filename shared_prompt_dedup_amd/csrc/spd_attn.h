// Internal declarations shared by the split-attention translation units.
//
// Work decomposition (How Prompt Deduplication Works, Phase 2 "Split
// Attention Optimization"): in the packed batch, group g owns the rows
// [po, po + pl) of its prompt followed by the rows of all its members'
// responses [ro, re), ro = po + pl.  A query row q sees
//   * keys k <= q of its own segment (k >= seg_start[q]), and
//   * when q is a response row, every key of its group's prompt.
// Query tiles never straddle a prompt/response boundary or a group; response
// query tiles may span several responses of one group (masking by seg_start
// keeps siblings apart).  Key tiles are cut the same way.
#pragma once

#include <algorithm>

#include "spd_internal.h"

namespace spd {

// A shared prefix (the prompts' common first columns, packed once ahead of
// every group) adds one level: its rows are keys of every later row.
//
// A query tile: rows [r0, r1); unmasked keys [v0, v1) (the shared prefix;
// empty without one or for the prefix's own tiles) and [u0, u1) (the group's
// prompt; empty for prompt tiles); own-segment keys start at s0 (masked by the
// rule above).
// A key tile: keys [r0, r1); masked query rows [u0, u1) (the rule above);
// unmasked query rows [s0, e0) (a prompt key tile's group responses; a prefix
// key tile's every later row).
//
// A key tile whose reader rows are many more than a CU's fair share is cut
// into chunks over its reader rows ([u0, u1) then [s0, e0); each chunk keeps
// its part of both ranges); a chunk writes fp32 partial dK / dV to its slot,
// and the last of the tile's chunks to finish (per kv head) adds the slots in
// chunk order, then scales and rounds once.
struct alignas(16) Tile {
  int r0, r1;
  int u0, u1;
  int s0, e0;
  int cost;
  int kind;   // 0 = prompt or prefix rows, 1 = response rows
  int v0, v1;
  int slot;   // key tiles: partial-sum slot of this chunk, -1 when the tile is not split
  int grp;    // key tiles: index of the split tile's SplitGroup, -1 when not split
};

// The chunks of one split key tile: keys [r0, r1), slots slot0 .. slot0 + n - 1.
struct SplitGroup {
  int r0, r1, slot0, n;
};

// Partial-sum slots of one backward call: each holds 256 keys x Hkv x D fp32
// for dK and for dV; at most 64, and at most 1024 / Hkv so that the slots stay
// within 256 MiB.  Chunks hold a multiple of 64 reader rows, at most 8 per tile.
constexpr int kMaxSplitSlots = 64;
constexpr int kSplitSlotHeads = 1024;
constexpr int kSplitRows = 64;
constexpr int kMaxChunks = 8;
inline int split_slots(int num_kv_heads) {
  const int n = std::min(kMaxSplitSlots, kSplitSlotHeads / num_kv_heads);
  return n >= 2 ? n : 0;
}

enum TileMode { kQueryTiles = 0, kKeyTiles = 1 };

// Upper bound on the tiles of one list (a partial tile per prompt, per
// response block and for the prefix).
inline int64_t tile_capacity(int64_t B, int64_t T, int rows_per_tile) {
  return (T + rows_per_tile - 1) / rows_per_tile + 2 * B + 2;
}

// One tile list to build on the device (one block), sorted by decreasing cost
// so that the heaviest tiles are dispatched first.  `tmp` and `out` hold
// `cap` tiles, `goff` B + 1 ints of scratch; *n_out receives the count.
// Key tiles may be split (see Tile) when `splits` is given: its groups are
// written there, and the arrival counters of each (group, kv head) in
// `arrivals` are cleared; `cap` then includes `max_slots` tiles of room for
// the extra chunks; `blocks_per_tile` (kv heads) and `n_cu` size a CU's fair
// share.
struct TileJob {
  int rows_per_tile = 0;
  int mode = kQueryTiles;
  int cap = 0;
  int *goff = nullptr;
  Tile *tmp = nullptr, *out = nullptr;
  int *n_out = nullptr;
  SplitGroup *splits = nullptr;
  int *arrivals = nullptr;
  int max_slots = 0, blocks_per_tile = 1, n_cu = 0;
};

// Builds `job`'s list, and `second`'s in the same launch when given (the two
// must not share scratch).
spd_status launch_build_tiles(const spd_plan &plan, int64_t T, const TileJob &job, hipStream_t st,
                              const TileJob *second = nullptr);

// fp32 correctness kernels (plain arithmetic, one row per thread).
spd_status attn_fwd_f32(const spd_attn_desc &d, const spd_plan &plan, int64_t T, const Tile *tiles,
                        const int *ntiles, int64_t cap, const float *q, const float *k, const float *v, float *o,
                        float *lse, hipStream_t st);
spd_status attn_bwd_f32(const spd_attn_desc &d, const spd_plan &plan, int64_t T, const Tile *qtiles,
                        const int *nq, int64_t capq, const Tile *ktiles, const int *nk, int64_t capk,
                        const float *q, const float *k, const float *v, const float *o, const float *lse,
                        const float *dout, float *dq, float *dk, float *dv, float *Dbuf, hipStream_t st);

// bf16 matrix-core kernels.
int fwd_bf16_rows_per_tile(const spd_attn_desc &d);
int dq_bf16_rows_per_tile(const spd_attn_desc &d);
int dkdv_bf16_rows_per_tile(const spd_attn_desc &d);
spd_status attn_fwd_bf16(const spd_attn_desc &d, const spd_plan &plan, int64_t T, const Tile *tiles,
                         const int *ntiles, int64_t cap, const void *q, const void *k, const void *v, void *o,
                         float *lse, hipStream_t st);
spd_status attn_bwd_bf16(const spd_attn_desc &d, const spd_plan &plan, int64_t T, const Tile *qtiles,
                         const int *nq, int64_t capq, const Tile *ktiles, const int *nk, int64_t capk,
                         const void *q, const void *k, const void *v, const void *o, const float *lse,
                         const void *dout, void *dq, void *dk, void *dv, float *Dbuf, float *L2buf, int *segp,
                         int64_t Tp, const SplitGroup *splits, int *arrivals, float *part_k, float *part_v,
                         hipStream_t st);

// Row stride of the backward's per-row scalar arrays: T rounded up to 64, plus
// one 64-row block, so that 64-row reads starting below T stay inside.
inline int64_t padded_rows(int64_t T) { return (T + 63) / 64 * 64 + 64; }

// Rows per tile of the fp32 kernels.
constexpr int kF32Rows = 64;

}  // namespace spd
