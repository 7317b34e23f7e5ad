// Host-side entry points over the work-decomposition functions of
// attn_sched.h, the same code the kernels run, for the unit tests: a test
// enumerates every workgroup and round of a grid and checks that each work
// item is visited exactly once.  Built into its own small library
// (libattn09_sched.so), separate from the attention library; nothing here
// touches a GPU.
#include <stdint.h>

#include "attn_sched.h"

using namespace attn;

extern "C" {

int sched_xcd_remap(int wg, int work_items) { return xcd_remap(wg, work_items); }

void sched_dense_item(int v, int tiles_per_head, int H, int causal, int* b, int* h, int* tile) {
  dense_item(v, tiles_per_head, H, causal != 0, *b, *h, *tile);
}

int sched_persist_dense_item(int blk, int r, int C, int work_items) {
  return persist_dense_item(blk, r, C, work_items);
}

int64_t sched_persist_listed_index(int blk, int r, int C, int64_t v_items) {
  return persist_listed_index(blk, r, C, v_items);
}

// listed_locate with the counts computed by plain loops over the per-sequence
// tile counts (the kernel computes the same two quantities with wave
// reductions over tile counts staged in LDS)
void sched_listed_locate(const int32_t* seq_tiles, int B, int hpx, int64_t f, int x, int* seq, int* tile,
                         int* head) {
  int tmax = 0;
  for (int i = 0; i < B; ++i) tmax = seq_tiles[i] > tmax ? seq_tiles[i] : tmax;
  auto cum = [&](int t) {
    int64_t acc = 0;
    for (int i = 0; i < B; ++i) acc += seq_tiles[i] > t ? seq_tiles[i] - t : 0;
    return acc * hpx;
  };
  auto nth = [&](int t, int rank) {
    for (int i = 0; i < B; ++i)
      if (seq_tiles[i] > t && rank-- == 0) return i;
    return -1;
  };
  listed_locate(f, x, hpx, tmax, cum, nth, *seq, *tile, *head);
}

int sched_varlen_item(const int32_t* cu, int B, int T, int tile_rows, int tiles_per_head, int causal, int v,
                      int* h, int* seq, int* tile) {
  return varlen_item(cu, B, T, tile_rows, tiles_per_head, causal != 0, v, *h, *seq, *tile) ? 1 : 0;
}

int sched_varlen_tile(const int32_t* cu, int B, int T, int vt, int tile, int* s0, int* len, int* t_in) {
  return varlen_tile(cu, B, T, vt, tile, *s0, *len, *t_in) ? 1 : 0;
}

int sched_varlen_ranked(const int32_t* cu, int B, int T, int f, int tile, int* s0, int* len, int* level) {
  return varlen_ranked(cu, B, T, f, tile, *s0, *len, *level) ? 1 : 0;
}

void sched_bwd_dkdv_item(int item, int nbk, int ktiles, int causal, int* kt, int* bk) {
  bwd_dkdv_item(item, nbk, ktiles, causal != 0, *kt, *bk);
}

void sched_bwd_dq_item(int item, int nbh, int qtiles, int causal, int* bh, int* tile) {
  bwd_dq_item(item, nbh, qtiles, causal != 0, *bh, *tile);
}

int sched_ranked_max_seqs(void) { return kRankedSeqs; }

}  // extern "C"
