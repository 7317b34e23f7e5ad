// Work decomposition: which work item a workgroup takes, for the forward and
// backward grids.  Plain integer functions of the launch index and the sizes,
// compiled for the device (the kernels call them) and for the host (unit
// tests enumerate every workgroup and check that each item is visited
// exactly once).  The pages' decomposition is one workgroup per (query tile,
// head, batch) with the key loop serial inside it (TileLang tutorial, section
// 3.0; the forward blog's section 3); varlen grids locate their sequence
// through the prefix sums (tutorial section 5.3), and causal grids start with
// the heaviest tiles.  What is added here is the order: XCD-aware ranges, a
// persistent grid that pairs heavy and light causal tiles, and the varlen
// listing by tile index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Workgroups are handed to the 8 XCDs round robin; map the launch index so
// that each XCD receives one contiguous range of work items (the query tiles
// of a head share K/V through that XCD's L2).  Returns -1 for padding.  The
// grid is 8 * ceil(work_items / 8) workgroups.
__host__ __device__ inline int xcd_remap(int wg, int work_items) {
  const int per = ceil_div(work_items, 8);
  const int v = (wg % 8) * per + wg / 8;
  return v < work_items ? v : -1;
}

// Dense forward item v -> (b, h, query tile): (b, h) major; under a causal
// mask a head's tiles run from the last (heaviest) down.
__host__ __device__ inline void dense_item(int v, int tiles_per_head, int H, bool causal, int& b, int& h,
                                           int& tile) {
  const int bh = v / tiles_per_head;
  const int rank = v - bh * tiles_per_head;
  b = bh / H;
  h = bh - b * H;
  tile = causal ? tiles_per_head - 1 - rank : rank;
}

// Persistent dense grid of 8 * C workgroups (C per XCD; work_items a multiple
// of 8 C): workgroup blk sits on XCD blk % 8 and walks that XCD's contiguous
// share of the items in rounds of C, reversing direction every round, so a
// heavy causal tile is paired with a light one.  Item of round r, or -1 when
// the rounds are over.
__host__ __device__ inline int persist_dense_item(int blk, int r, int C, int work_items) {
  const int x = blk % 8, c = blk / 8;
  const int per = work_items / 8;
  if (r * C >= per) return -1;
  return x * per + r * C + ((r & 1) ? C - 1 - c : c);
}

// Persistent varlen grid: the same rounds over the v_items listed items of
// workgroup blk's XCD.  Index f of the XCD's list for round r, -1 when the
// rounds are over, -2 for the padding of the last round.
__host__ __device__ inline int64_t persist_listed_index(int blk, int r, int C, int64_t v_items) {
  const int c = blk / 8;
  if ((int64_t)r * C >= v_items) return -1;
  const int64_t f = (int64_t)r * C + ((r & 1) ? C - 1 - c : c);
  return f < v_items ? f : -2;
}

// Varlen persistent order of XCD x: its heads [x hpx, (x+1) hpx) (the query
// heads of one KV head stay on one L2); the items (sequence, tile, head) are
// listed by tile index, highest first (under a causal mask the cost of a tile
// grows with its index), then sequence, then head.  cum(t) must return the
// number of listed items with tile index >= t, hpx * sum_i max(0, tiles_i -
// t), and nth(t, k) the index of the k-th sequence (in index order) with more
// than t tiles; tmax is the largest tile count.  Item f (< cum(0)) is located
// by a binary search for its tile index.
template <class Cum, class Nth>
__host__ __device__ inline void listed_locate(int64_t f, int x, int hpx, int tmax, Cum&& cum, Nth&& nth, int& seq,
                                              int& tile, int& head) {
  // level t: cum(t+1) <= f < cum(t); cum falls as t grows
  int lo = 0, hi = tmax - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cum(mid) > f) {
      lo = mid;
    } else {
      hi = mid - 1;
    }
  }
  tile = lo;
  const int rr = (int)(f - cum(tile + 1));
  const int rank = rr / hpx;
  head = x * hpx + (rr - rank * hpx);
  seq = nth(tile, rank);
}

// Bounds [s0, s1) of varlen sequence bb from the prefix sums, clamped into
// [0, T] so that a malformed array cannot address outside the tensors.
__host__ __device__ inline void seq_bounds(const int32_t* cu, int T, int bb, int& s0, int& s1) {
  s0 = cu[bb];
  s1 = cu[bb + 1];
  s0 = s0 < 0 ? 0 : (s0 > T ? T : s0);
  s1 = s1 < s0 ? s0 : (s1 > T ? T : s1);
}

// Dispatched varlen forward item v -> (head, sequence, tile): h major, then
// the concatenated tiles (of `tile_rows` rows) of the sequences, last first
// under a causal mask.  False for items past the last tile.
__host__ __device__ inline bool varlen_item(const int32_t* cu, int B, int T, int tile_rows, int tiles_per_head,
                                            bool causal, int v, int& h, int& seq, int& tile) {
  h = v / tiles_per_head;
  int vt = v - h * tiles_per_head;
  if (causal) vt = tiles_per_head - 1 - vt;
  int acc = 0;
  for (int bb = 0; bb < B; ++bb) {
    int s0, s1;
    seq_bounds(cu, T, bb, s0, s1);
    const int nt = ceil_div(s1 - s0, tile_rows);
    if (vt < acc + nt) {
      seq = bb;
      tile = vt - acc;
      return true;
    }
    acc += nt;
  }
  return false;
}

// Backward, varlen: the per-head tile index vt of packed sequences with
// `tile`-row tiles (tiles of one sequence consecutive, sequences in order);
// sets the sequence's first row s0, its length and the tile within it.  False
// past the last tile.
__host__ __device__ inline bool varlen_tile(const int32_t* cu, int B, int T, int vt, int tile, int& s0, int& len,
                                            int& t_in) {
  int acc = 0;
  for (int bb = 0; bb < B; ++bb) {
    int a, e;
    seq_bounds(cu, T, bb, a, e);
    const int nt = ceil_div(e - a, tile);
    if (vt < acc + nt) {
      s0 = a;
      len = e - a;
      t_in = vt - acc;
      return true;
    }
    acc += nt;
  }
  return false;
}

// Backward, varlen, causal: the items listed by work, heaviest first.  An
// item of level r costs about r tile-pairs: key tile k of a sequence of n
// tiles has level n - k (it sees the query tiles k .. n-1), query tile t
// level t + 1.  Levels run from the largest n down to 1; within a level,
// sequences in order.  F(r) = sum_i max(0, n_i - r + 1) items have level >=
// r, so item f has the level r with F(r+1) <= f < F(r) (binary search), and
// is the (f - F(r+1))-th sequence with n_i >= r.  Sets s0, len and the level;
// false past the last item.  Costs a few scans of the prefix sums per
// workgroup, so it is used for short sequence lists only.
constexpr int kRankedSeqs = 64;
__host__ __device__ inline bool varlen_ranked(const int32_t* cu, int B, int T, int f, int tile, int& s0, int& len,
                                              int& level) {
  auto items_from = [&](int r) {  // F(r)
    int acc = 0;
    for (int bb = 0; bb < B; ++bb) {
      int a, e;
      seq_bounds(cu, T, bb, a, e);
      const int n = ceil_div(e - a, tile) - r + 1;
      acc += n > 0 ? n : 0;
    }
    return acc;
  };
  int nmax = 0;
  for (int bb = 0; bb < B; ++bb) {
    int a, e;
    seq_bounds(cu, T, bb, a, e);
    const int n = ceil_div(e - a, tile);
    nmax = n > nmax ? n : nmax;
  }
  if (nmax == 0 || f >= items_from(1)) return false;
  int lo = 1, hi = nmax;  // the largest r with F(r) > f
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (items_from(mid) > f) {
      lo = mid;
    } else {
      hi = mid - 1;
    }
  }
  level = lo;
  int j = f - items_from(lo + 1);
  for (int bb = 0; bb < B; ++bb) {
    int a, e;
    seq_bounds(cu, T, bb, a, e);
    if (ceil_div(e - a, tile) >= level && j-- == 0) {
      s0 = a;
      len = e - a;
      return true;
    }
  }
  return false;
}

// Backward dK/dV, dense: item -> (key tile kt, b * Hkv + kv head).  Causal:
// key tiles from the left (the heaviest: they see the most query tiles), all
// KV heads of a tile together; otherwise a KV head's tiles consecutive (the
// caller spreads them over the XCDs with xcd_remap).
__host__ __device__ inline void bwd_dkdv_item(int item, int nbk, int ktiles, bool causal, int& kt, int& bk) {
  kt = causal ? item / nbk : item % ktiles;
  bk = causal ? item - kt * nbk : item / ktiles;
}

// Backward dQ, dense: item -> (b * H + h, query tile).  Causal: query tiles
// from the bottom (the heaviest), all heads of a tile together; otherwise a
// head's tiles consecutive.
__host__ __device__ inline void bwd_dq_item(int item, int nbh, int qtiles, bool causal, int& bh, int& tile) {
  bh = causal ? item % nbh : item / qtiles;
  tile = causal ? qtiles - 1 - item / nbh : item - bh * qtiles;
}

}  // namespace attn
