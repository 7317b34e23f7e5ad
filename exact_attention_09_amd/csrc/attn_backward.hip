// Backward pass of exact attention (dQ, dK, dV) for bf16 on gfx950.
//
// The gradients are those of the forward's definition (TileLang tutorial
// chapter 15, section 1.1), recomputed tile by tile from the saved log-sum-
// exp instead of a stored score matrix -- the pages' backward (the tutorial's
// section 5.4 reports its dQ error when partial dQ tiles are added with bf16
// atomics).  Per (batch, query head), with P = exp(s Q K^T - LSE):
//
//   Delta_i = rowsum(dO_i * O_i)
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - Delta),  dQ = s dS K,  dK = s dS^T Q
//
// Two tile kernels, no atomics, fixed summation orders (bitwise
// reproducible), in this order:
//   * dq_kernel: one workgroup per (batch, query head, 128 queries); each
//     wave keeps its 32 queries' Q and dO rows in registers and walks the key
//     tiles.  It also forms Delta (from the O rows) and the log2 LSE of its
//     rows and leaves them in the workspace.  dQ costs a second computation
//     of S and dP instead of atomic partial sums;
//   * dkdv_pair_kernel: one workgroup per (batch, KV head, 128 keys); a pair
//     of waves keeps 32 keys' K and V rows in registers (one each) and walks
//     the query tiles of every query head of the group, so the grouped-query
//     sum happens in registers.  It reads Delta and the log2 LSE.
// With sinks, dsink_kernel forms the sink gradients in between.
//
// Both tile kernels use v_mfma_f32_32x32x16_bf16 with the accumulator
// arranged so that the exponentiated scores are directly the B operand of the
// next product (as in the forward kernels): dK/dV computes S = Q K^T (one key
// per lane) and dV^T = dO^T P, dK^T = Q^T dS; dq computes S^T = K Q^T (one
// query per lane) and dQ^T = K^T dS^T.  Tiles sit row-major in LDS with the
// 16-byte chunk swizzle of attn_common.h; the transposed operands are read
// with ds_read_b64_tr_b16.  P and dS are rounded to bf16 (nearest even) for
// the products that consume them; every accumulation is fp32.
//
// Layouts: BHSD (rows d elements apart) or, in separate BSHD template
// variants, [B, S, H, d] tensors whose rows are H d (Hkv d) elements apart;
// the per-row Delta and log2 LSE stay in the LSE's [B, H, S] order either
// way, and the arithmetic and its order do not depend on the layout.
#include "attn_common.h"
#include "attn_internal.h"

namespace attn {

namespace {

constexpr float kLog2e = 1.44269504088896340736f;

#ifndef ATTN_BWD_AHEAD_DQ
#define ATTN_BWD_AHEAD_DQ 1
#endif

// ---------------------------------------------------------------- sinks

// dsink_h = -sum over the rows of head h of P_sink,i Delta_i, with
// P_sink,i = exp(sink_h - LSE_i) (the forward's LSE counts the sink; a row
// that saw no key has LSE = sink and Delta = 0).  One workgroup per head;
// each thread sums a fixed stride of rows, then a fixed tree: bitwise
// reproducible.
__global__ __launch_bounds__(256) void dsink_kernel(const float* __restrict__ sinks, const float* __restrict__ delta,
                                                    const float* __restrict__ lse2, float* __restrict__ dsinks, int nb,
                                                    int H, int S) {
  __shared__ float part[256];
  const int h = blockIdx.x;
  const float sk = sinks[h] * kLog2e;
  float acc = 0.0f;
  for (int b = 0; b < nb; ++b) {
    const int64_t row0 = ((int64_t)b * H + h) * S;
    for (int i = threadIdx.x; i < S; i += 256) acc += fast_exp2(sk - lse2[row0 + i]) * delta[row0 + i];
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int m = 128; m >= 1; m >>= 1) {
    if ((int)threadIdx.x < m) part[threadIdx.x] += part[threadIdx.x + m];
    __syncthreads();
  }
  if (threadIdx.x == 0) dsinks[h] = -part[0];
}

// ---------------------------------------------------------------- shared

// A row-major tile of `ROWS` rows of D bf16 in LDS, 16-byte chunks swizzled
// (lds_off), filled straight from HBM by buffer_load ... lds.  The tile is a
// run of 1 KB blocks; lane L of a block load writes bytes 16L .. 16L+15 of
// the block, which is row L / (2D/16) of the block at chunk position
// L % (2D/16), so the lane fetches the logical chunk that the swizzle puts
// there.  `voff(j, lane, rsb)` is that lane's byte offset in the HBM tile for
// block j, with rows rsb bytes apart there (2D in BHSD, 2 H D in BSHD).
template <int D, int ROWS>
struct SwizzledTile {
  static constexpr int ROWB = 2 * D;
  static constexpr int CPR = ROWB / 16;     // 16-byte chunks per row
  static constexpr int RPB = 1024 / ROWB;   // rows per 1 KB block
  static constexpr int NBLK = ROWS / RPB;   // blocks per tile
  static constexpr int BYTES = ROWS * ROWB;
  __device__ static int voff(int j, int lane, int rsb) {
    const int r = j * RPB + lane / CPR;
    return r * rsb + (((lane % CPR) ^ swz<D>(r)) << 4);
  }
};

// A operand (32 rows x 16 columns) of a row-major swizzled tile: rows
// row0 + l%32, columns 16c + 8(l/32) .. +8.
template <int D>
__device__ inline bf16x8 frag_rows(const unsigned char* tile, int row0, int c, int l32, int hh) {
  return *(const bf16x8*)(tile + lds_off<D>(row0 + l32, 2 * c + hh));
}

// A operand of the transposed tile: columns 32db + l%32 of the tile, over the
// 16 tile rows of chunk kc, in the row order the score accumulators use
// (see the forward kernels' P~ V product).
template <int D>
__device__ inline bf16x8 frag_cols(const unsigned char* tile, int kc, int db, int tr_row, int tr_col) {
  const int col = 32 * db + tr_col;
  const int row0 = 16 * kc + tr_row;
  const s16x4 lo = lds_read_tr16(tile + lds_off<D>(row0, col >> 3) + (col & 7) * 2);
  const s16x4 hi = lds_read_tr16(tile + lds_off<D>(row0 + 8, col >> 3) + (col & 7) * 2);
  return join_tr(lo, hi);
}

// bf16 x 8 of accumulator registers 8h .. 8h+7
__device__ inline bf16x8 half_bf16(const f32x16& a, int h) {
  const int rb = 8 * h;
  return to_bf16x8(a[rb + 0], a[rb + 1], a[rb + 2], a[rb + 3], a[rb + 4], a[rb + 5], a[rb + 6], a[rb + 7]);
}

// ---------------------------------------------------------------- dK, dV

// Keys stationary, two waves per 32 keys: workgroup (b, KV head, 128 keys)
// of 8 waves, waves w and w+4 (one SIMD) owning keys k0 + 32w .. +31.  Wave w
// (the S side) computes S = Q K^T, P and dV^T += dO^T P; wave w+4 (the dP
// side) computes dP = dO V^T and, with P handed over through LDS in fp32,
// dS = P (dP - Delta) and dK^T += Q^T dS.  Each wave holds one K or V row set
// and one of the two accumulators, so two waves fit a SIMD; the work and
// every rounding are fixed, so the results are bitwise reproducible.  Both
// sides run the same MFMA instructions on different operands; only their
// vector work differs.  (A one-wave-per-32-keys kernel holding both
// accumulators needs about 400 registers, so only one wave fits a SIMD; even
// written out as a software pipeline it ran 2-4 % slower than this pair.)
// BSHD: q, dO [B, Sq, H, d] and k, v, dK, dV [B, Skv, Hkv, d] (packed
// sequences: [T, H, d], [T, Hkv, d]); rows H d (Hkv d) elements apart, known
// at run time; off, every stride is the compile-time d.
template <int D, bool CAUSAL, bool VARLEN, bool LOCAL, bool BSHD>
__global__ __launch_bounds__(512, 1) void dkdv_pair_kernel(const Params p, const __bf16* __restrict__ dout,
                                                           const float* __restrict__ delta,
                                                           const float* __restrict__ lse2, __bf16* __restrict__ dk,
                                                           __bf16* __restrict__ dv) {
  constexpr int BK = 128;        // keys per workgroup
  constexpr int BQ = 64;         // queries per tile
  constexpr int NDC = D / 16;    // contraction chunks over d
  constexpr int NDB = D / 32;    // 32-column blocks of d
  constexpr int NQB = BQ / 32;   // 32-query halves of a tile
  using Tile = SwizzledTile<D, BQ>;
  constexpr int TILE = Tile::BYTES;
  constexpr int BPW = Tile::NBLK / 4;           // blocks per wave: waves 0-3 load Q, 4-7 dO
  constexpr int STAGE = 2 * TILE + 2 * BQ * 4;  // Q, dO, lse2, delta
  constexpr int PBUF = 64 * 16 * 4;             // one 32 x 32 fp32 P block, 4 KB
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE + 4 * NQB * PBUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const bool s_side = wu < 4;
  const int kb = wu & 3;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const float sl2 = p.scale_log2;

  // the item: (b, kv head, key tile); dense causal: key tiles in order of
  // decreasing work (a key tile's query range shrinks as the keys move
  // right), non-causal: XCD-aware (the key tiles of a KV head share its
  // Q/dO stream in one L2; the grid is padded to a multiple of 8); varlen:
  // (kv head, tile of the packed sequences), located through cu_seqlens.
  int kt, b, kvh, sq, skv;
  int64_t kv_row0, q_head_rows;  // row of this sequence's key 0; rows per query head (varlen: T)
  int64_t q_row_shift;           // varlen: the sequence's first row
  if constexpr (VARLEN) {
    const int ktu = p.tiles_per_head;
    int s0, len;
    if (CAUSAL && p.B <= kRankedSeqs) {
      // heaviest first over all KV heads: the heads interleaved
      kvh = (int)blockIdx.x % p.Hkv;
      int level;
      if (!varlen_ranked(p.cu, p.B, p.Sq, (int)blockIdx.x / p.Hkv, BK, s0, len, level)) return;
      kt = ceil_div(len, BK) - level;
    } else {
      kvh = (int)blockIdx.x / ktu;
      if (!varlen_tile(p.cu, p.B, p.Sq, (int)blockIdx.x - kvh * ktu, BK, s0, len, kt)) return;
    }
    b = 0;
    sq = skv = len;
    kv_row0 = (int64_t)kvh * p.Sq + s0;
    q_head_rows = p.Sq;
    q_row_shift = s0;
  } else {
    const int ktiles = ceil_div(p.Skv, BK);
    const int nbk = p.B * p.Hkv;
    const int item = CAUSAL ? (int)blockIdx.x : xcd_remap((int)blockIdx.x, nbk * ktiles);
    if (item < 0) return;
    int bk;  // b * Hkv + kvh
    bwd_dkdv_item(item, nbk, ktiles, CAUSAL, kt, bk);
    b = bk / p.Hkv;
    kvh = bk - b * p.Hkv;
    sq = p.Sq;
    skv = p.Skv;
    kv_row0 = (int64_t)bk * skv;
    q_head_rows = sq;
    q_row_shift = 0;
  }
  const int off = skv - sq;
  const int k0 = kt * BK;
  const int kw0 = k0 + 32 * kb;
  const int krow = kw0 + l32;
  // element offset of this sequence's key row 0 and the row strides
  const int q_rs = BSHD ? __builtin_amdgcn_readfirstlane(p.q_rs) : D;
  const int kv_rs = BSHD ? __builtin_amdgcn_readfirstlane(p.kv_rs) : D;
  const int64_t kv_el = BSHD ? (((int64_t)b * p.Skv + q_row_shift) * p.Hkv + kvh) * D : kv_row0 * D;

  // this lane's K row (S side) or V row (dP side): the B operand
  const __bf16* __restrict__ KV = (const __bf16*)(s_side ? p.k : p.v) + kv_el;
  bf16x8 kvf[NDC];
#pragma unroll
  for (int c = 0; c < NDC; ++c)
    kvf[c] = krow < skv ? *(const bf16x8*)(KV + (int64_t)krow * kv_rs + 16 * c + 8 * hh) : bf16x8{};

  f32x16 acc[NDB];  // dV^T (S side) or dK^T (dP side): rows d, column = this lane's key
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  // queries that see a key of this workgroup: i >= j - off (causal) and,
  // under a window W, i < j - off + W
  const int W = LOCAL ? p.window : 0;
  int qbeg = 0;
  if (CAUSAL) {
    qbeg = k0 - off;
    qbeg = qbeg < 0 ? 0 : qbeg;
  }
  int qend = sq;
  if (W > 0) {
    const long e = (long)k0 + BK - 1 - off + W;
    qend = e < 0 ? 0 : (e < sq ? (int)e : sq);
  }
  const int qt0 = qbeg / BQ;
  const int nqt = ceil_div(qend, BQ);
  const int per_head = nqt > qt0 ? nqt - qt0 : 0;
  const int nsteps = per_head * p.group;

  int voff[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) voff[i] = Tile::voff(kb * BPW + i, lane, 2 * q_rs);
  float lse_reg = 0.0f, del_reg = 0.0f;
  auto step_src = [&](int s, int& h, int& q0) {
    h = kvh * p.group + s / per_head;
    q0 = (qt0 + s % per_head) * BQ;
  };
  auto gload = [&](int s) {
    int h, q0;
    step_src(s, h, q0);
    const int64_t row0 = ((int64_t)b * p.H + h) * q_head_rows + q_row_shift + q0;
    if (wu == 0) {
      const int i = q0 + lane;
      lse_reg = i < sq ? lse2[row0 + lane] : INFINITY;
      del_reg = i < sq ? delta[row0 + lane] : 0.0f;
    }
    const int nrows = sq - q0 < BQ ? sq - q0 : BQ;
    // the tile's first row in q (dO); the descriptor ends right after row
    // nrows-1, so rows past it read as zeros
    const int64_t q_el = BSHD ? (((int64_t)b * p.Sq + q_row_shift + q0) * p.H + h) * D : row0 * D;
    const __bf16* src = s_side ? (const __bf16*)p.q + q_el : dout + q_el;
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(src, (nrows - 1) * 2 * q_rs + 2 * D);
    const unsigned dst = lds_u32(smem) + (s & 1) * STAGE + (s_side ? 0 : TILE) + kb * BPW * 1024;
#pragma unroll
    for (int i = 0; i < BPW; ++i) load_lds16(rs, voff[i], 0, dst + i * 1024);
  };
  auto lstore = [&](int stage) {
    if (wu == 0) {
      float* base = (float*)(smem + stage * STAGE + 2 * TILE);
      base[lane] = lse_reg;
      base[BQ + lane] = del_reg;
    }
  };

  const int g16 = lane >> 4;
  const int t16 = lane & 15;
  const int tr_row = 4 * (g16 >> 1) + (t16 >> 2);
  const int tr_col = 16 * (g16 & 1) + 4 * (t16 & 3);

  if (nsteps > 0) gload(0);
  __builtin_amdgcn_s_waitcnt(0);
  lstore(0);
  __syncthreads();

  // One 64-row tile per step, as two 32-row halves.  Both sides first run
  // the S (dP) products of both halves; the S side then forms P of half 0
  // and, after the first barrier, runs dV of half 0 while forming P of half
  // 1, so that its exponentials overlap MFMAs (its own and its partner's)
  // instead of leaving the SIMD's matrix unit idle.  Each side has its own
  // straight-line step (the compiler schedules within one block); both meet
  // the same three barriers per step.
  static_assert(NQB == 2, "a step is two 32-row halves");
  // S (S side) or dP (dP side) of half qb: rows of t_rows against this
  // lane's K or V row; query rows 32qb + 8(r/4) + 4hh + r%4 of this key
  auto rows_product = [&](const unsigned char* t_rows, const int qb) {
    f32x16 x = f32x16{};
#pragma unroll
    for (int c = 0; c < NDC; ++c) x = mfma32(frag_rows<D>(t_rows, 32 * qb, c, l32, hh), kvf[c], x);
    return x;
  };
  // dV^T += dO^T P (S side), dK^T += Q^T dS (dP side), 16 queries per product
  auto cols_product = [&](const unsigned char* t_cols, const f32x16& x, const int qb) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const bf16x8 xb = half_bf16(x, h2);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = mfma32(frag_cols<D>(t_cols, 2 * qb + h2, db, tr_row, tr_col), xb, acc[db]);
    }
  };
  auto pbuf_of = [&](const int qb) { return (float*)(smem + 2 * STAGE + (kb * NQB + qb) * PBUF); };
  if (s_side) {
    // P = exp2(S scale' - LSE') of half qb, masked, to this pair's LDS buffer
    // in fp32: the masks (only where this wave's 32 keys and the half's 32
    // rows cross the diagonal or the window's lower edge) ...
    auto mask_s = [&](f32x16& x, const int q0, const int qb) {
      const int qr_off = q0 + 32 * qb + off;
      const bool partial = (CAUSAL && kw0 + 31 > qr_off) || (LOCAL && W > 0 && kw0 <= qr_off + 31 - W);
      if (partial) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i_off = qr_off + 8 * (r >> 2) + 4 * hh + (r & 3);  // query row + off
          if (CAUSAL) x[r] = krow > i_off ? -INFINITY : x[r];
          if (LOCAL && W > 0) x[r] = krow <= i_off - W ? -INFINITY : x[r];
        }
      }
    };
    // ... then element r (the four of a group stored once the last is done)
    auto p_elem = [&](f32x16& x, const f32x4* lv, float* pbuf, const int r) {
      x[r] = fast_exp2(fmaf(x[r], sl2, -lv[r >> 2][r & 3]));
      if ((r & 3) == 3) {
        const int g = r >> 2;
        *(f32x4*)(pbuf + 256 * g + 4 * lane) = f32x4{x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
      }
    };
    constexpr int AH = 2, R = AH + 1;
    for (int s = 0; s < nsteps; ++s) {
      const int stage = s & 1;
      if (s + 1 < nsteps) gload(s + 1);
      int h, q0;
      step_src(s, h, q0);
      (void)h;
      const unsigned char* tq = smem + stage * STAGE;
      const unsigned char* tdo = tq + TILE;
      const float* tlse = (const float*)(tq + 2 * TILE);
      f32x4 lv0[4], lv1[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        lv0[g] = *(const f32x4*)(tlse + 8 * g + 4 * hh);
        lv1[g] = *(const f32x4*)(tlse + 32 + 8 * g + 4 * hh);
      }
      f32x16 x0 = rows_product(tq, 0);
      mask_s(x0, q0, 0);
      // S of half 1, with P of half 0 spread over its MFMAs (operands read
      // AH MFMAs ahead; sched_barrier keeps the order)
      f32x16 x1 = f32x16{};
      {
        bf16x8 fr[R];
        static_for<AH>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          fr[i] = frag_rows<D>(tq, 32, i, l32, hh);
        });
        constexpr int EPM = 16 / NDC;  // elements of P per MFMA
        static_for<NDC>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          x1 = mfma32(fr[i % R], kvf[i], x1);
          if constexpr (i + AH < NDC) fr[(i + AH) % R] = frag_rows<D>(tq, 32, i + AH, l32, hh);
          static_for<EPM>([&](auto ec) { p_elem(x0, lv0, pbuf_of(0), EPM * i + decltype(ec)::value); });
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      mask_s(x1, q0, 1);
      __syncthreads();
      // dV of half 0, with P of half 1 spread over its MFMAs
      {
        constexpr int NM = 2 * NDB;    // MFMAs of the product
        constexpr int EPM = 16 / NM;   // elements of P per MFMA
        bf16x8 fc[R];
        const bf16x8 xb[2] = {half_bf16(x0, 0), half_bf16(x0, 1)};
        static_for<AH>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          fc[i] = frag_cols<D>(tdo, i / NDB, i % NDB, tr_row, tr_col);
        });
        static_for<NM>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          acc[i % NDB] = mfma32(fc[i % R], xb[i / NDB], acc[i % NDB]);
          if constexpr (i + AH < NM) fc[(i + AH) % R] = frag_cols<D>(tdo, (i + AH) / NDB, (i + AH) % NDB, tr_row, tr_col);
          static_for<EPM>([&](auto ec) { p_elem(x1, lv1, pbuf_of(1), EPM * i + decltype(ec)::value); });
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      __syncthreads();
      cols_product(tdo, x1, 1);
      __builtin_amdgcn_s_waitcnt(0);
      if (s + 1 < nsteps) lstore(stage ^ 1);
      __syncthreads();
    }
  } else {
    // dS = P (dP - Delta), P from the partner's buffer
    auto make_ds = [&](f32x16& x, const float* tdel, const int qb) {
      const float* pbuf = pbuf_of(qb);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 pv = *(const f32x4*)(pbuf + 256 * g + 4 * lane);
        const f32x4 dl = *(const f32x4*)(tdel + 32 * qb + 8 * g + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * g + e] = pv[e] * (x[4 * g + e] - dl[e]);
      }
    };
    for (int s = 0; s < nsteps; ++s) {
      const int stage = s & 1;
      if (s + 1 < nsteps) gload(s + 1);
      const unsigned char* tq = smem + stage * STAGE;
      const unsigned char* tdo = tq + TILE;
      const float* tdel = (const float*)(tq + 2 * TILE) + BQ;
      f32x16 x0 = rows_product(tdo, 0);
      f32x16 x1 = rows_product(tdo, 1);
      __syncthreads();
      make_ds(x0, tdel, 0);
      cols_product(tq, x0, 0);
      __syncthreads();
      make_ds(x1, tdel, 1);
      cols_product(tq, x1, 1);
      __builtin_amdgcn_s_waitcnt(0);
      if (s + 1 < nsteps) lstore(stage ^ 1);
      __syncthreads();
    }
  }

  // dV = dV^T^T (S side), dK = s dK^T^T (dP side): this lane's key row
  if (krow < skv) {
    __bf16* row = (s_side ? dv : dk) + kv_el + (int64_t)krow * kv_rs;
    const float sc = s_side ? 1.0f : p.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[db][4 * rg + e] * sc);
        *(bf16x4*)(row + 32 * db + 8 * rg + 4 * hh) = w;
      }
  }
}

// ---------------------------------------------------------------- dQ

// Queries stationary: workgroup (b, query head, 128 queries), wave w owns
// queries q0 + 32w .. +31 (one per lane of a half-wave pair); key tiles of 64
// rows stream through LDS, double buffered, each worked in two 32-key
// halves.  Two workgroups share a CU.  BSHD as for the dK/dV kernel.
template <int D, bool CAUSAL, bool VARLEN, bool LOCAL, bool BSHD>
__global__ __launch_bounds__(256, 2) void dq_kernel(const Params p, const __bf16* __restrict__ dout,
                                                    float* __restrict__ delta, float* __restrict__ lse2,
                                                    __bf16* __restrict__ dq) {
  constexpr int BMQ = 128;
  constexpr int BN = 64;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NKB = BN / 32;
  using Tile = SwizzledTile<D, BN>;
  constexpr int TILE = Tile::BYTES;
  constexpr int BPW = Tile::NBLK / 2;  // blocks per wave: waves 0-1 load K, 2-3 V
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * 2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const float sl2 = p.scale_log2;

  // the item: (b, query head, query tile); dense causal: query tiles in
  // order of decreasing work (the last tiles see the most keys), non-causal:
  // XCD-aware as in the dK/dV kernel (the query tiles of a head share its
  // K/V stream in one L2); varlen: (query head, tile of the packed
  // sequences), located through cu_seqlens.
  int tile, sq, skv;
  int64_t row0, kv0;    // this head's (sequence's) query row 0 and key row 0, in rows of d
  int64_t q_el, kv_el;  // the element offsets of those rows in q (dO, dQ) and k (v)
  if constexpr (VARLEN) {
    const int qtu = p.tiles_per_head;
    int h, s0, len;
    if (CAUSAL && p.B <= kRankedSeqs) {
      // heaviest first over all query heads: the heads interleaved
      h = (int)blockIdx.x % p.H;
      int level;
      if (!varlen_ranked(p.cu, p.B, p.Sq, (int)blockIdx.x / p.H, BMQ, s0, len, level)) return;
      tile = level - 1;
    } else {
      h = (int)blockIdx.x / qtu;
      if (!varlen_tile(p.cu, p.B, p.Sq, (int)blockIdx.x - h * qtu, BMQ, s0, len, tile)) return;
    }
    sq = skv = len;
    row0 = (int64_t)h * p.Sq + s0;
    kv0 = (int64_t)(h / p.group) * p.Sq + s0;
    q_el = BSHD ? ((int64_t)s0 * p.H + h) * D : row0 * D;
    kv_el = BSHD ? ((int64_t)s0 * p.Hkv + h / p.group) * D : kv0 * D;
  } else {
    const int qtiles = ceil_div(p.Sq, BMQ);
    const int nbh = p.B * p.H;
    const int item = CAUSAL ? (int)blockIdx.x : xcd_remap((int)blockIdx.x, nbh * qtiles);
    if (item < 0) return;
    int bh;
    bwd_dq_item(item, nbh, qtiles, CAUSAL, bh, tile);
    const int b = bh / p.H;
    const int h = bh - b * p.H;
    sq = p.Sq;
    skv = p.Skv;
    row0 = (int64_t)bh * sq;
    kv0 = ((int64_t)b * p.Hkv + h / p.group) * skv;
    q_el = BSHD ? ((int64_t)b * sq * p.H + h) * D : row0 * D;
    kv_el = BSHD ? ((int64_t)b * skv * p.Hkv + h / p.group) * D : kv0 * D;
  }
  const int off = skv - sq;
  const int q0 = tile * BMQ;
  const int qw0 = q0 + 32 * wave;
  const int qrow = qw0 + l32;

  const int q_rs = BSHD ? __builtin_amdgcn_readfirstlane(p.q_rs) : D;
  const int kv_rs = BSHD ? __builtin_amdgcn_readfirstlane(p.kv_rs) : D;
  const __bf16* __restrict__ Q = (const __bf16*)p.q + q_el;
  const __bf16* __restrict__ dO = dout + q_el;
  const __bf16* __restrict__ K = (const __bf16*)p.k + kv_el;
  const __bf16* __restrict__ V = (const __bf16*)p.v + kv_el;

  bf16x8 qf[NDC], dof[NDC];
  float neg_lse = -INFINITY, del = 0.0f;  // -LSE log2(e) of this lane's row (-inf: P = 0)
  if (qrow < sq) {
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      qf[c] = *(const bf16x8*)(Q + (int64_t)qrow * q_rs + 16 * c + 8 * hh);
      dof[c] = *(const bf16x8*)(dO + (int64_t)qrow * q_rs + 16 * c + 8 * hh);
    }
    // Delta = rowsum(dO * O) of this lane's row and the LSE in log2 units
    // (+inf for a row that saw no key, so that its P is 0).  The sum runs in
    // a fixed order: 8 products per 16-byte chunk, the chunks of this half
    // of the row pairwise (a butterfly over the chunk index), then the other
    // half from lane l ^ 32.  Both go to the workspace for the dK/dV and
    // sink-gradient kernels, which run after this one.
    const __bf16* __restrict__ orow = (const __bf16*)p.o + q_el + (int64_t)qrow * q_rs;
    float part[NDC];
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      const bf16x8 a = *(const bf16x8*)(orow + 16 * c + 8 * hh);
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += (float)a[j] * (float)dof[c][j];
      part[c] = acc;
    }
#pragma unroll
    for (int m = NDC / 2; m >= 1; m >>= 1) {
      float nxt[NDC];
#pragma unroll
      for (int c = 0; c < NDC; ++c) nxt[c] = part[c] + part[c ^ m];
#pragma unroll
      for (int c = 0; c < NDC; ++c) part[c] = nxt[c];
    }
    del = part[0] + __shfl_xor(part[0], 32, 64);
    const float l = p.lse[row0 + qrow];
    const float l2 = l == -INFINITY ? INFINITY : l * kLog2e;
    neg_lse = -l2;
    if (hh == 0) {
      delta[row0 + qrow] = del;
      lse2[row0 + qrow] = l2;
    }
  } else {
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      qf[c] = bf16x8{};
      dof[c] = bf16x8{};
    }
  }

  const int q_hi = q0 + BMQ < sq ? q0 + BMQ : sq;
  const int kv_end = CAUSAL ? causal_kv_end(q_hi, off, skv) : skv;
  const int nt = ceil_div(kv_end, BN);
  // under a window W row i sees keys from i + off - W + 1: the workgroup
  // starts at the tile of its top row's first key, each wave skips the
  // tiles before its own
  const int W = LOCAL ? p.window : 0;
  auto win_lo = [&](const int i) {
    const long b = (long)i + off - W + 1;
    return b < 0 ? 0 : (b > skv ? skv : (int)b);
  };
  const int t_first = W > 0 ? (win_lo(q0) < kv_end ? win_lo(q0) : kv_end) / BN : 0;
  int w_end = 0, w_lo = 0;
  if (qw0 < sq) {
    const int w_hi = qw0 + 32 < sq ? qw0 + 32 : sq;
    w_end = CAUSAL ? causal_kv_end(w_hi, off, skv) : skv;
    if (W > 0) w_lo = win_lo(qw0);
  }

  const bool loads_v = wu >= 2;
  int voff[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) voff[i] = Tile::voff((wu & 1) * BPW + i, lane, 2 * kv_rs);
  auto gload = [&](int t) {
    const int kb0 = t * BN;
    const int nrows = skv - kb0 < BN ? skv - kb0 : BN;
    // the descriptor ends right after row nrows-1: rows past it read as zeros
    const __amdgpu_buffer_rsrc_t rs =
        uniform_rsrc((loads_v ? V : K) + (int64_t)kb0 * kv_rs, (nrows - 1) * 2 * kv_rs + 2 * D);
    const unsigned dst = lds_u32(smem) + (t & 1) * 2 * TILE + (loads_v ? TILE : 0) + (wu & 1) * BPW * 1024;
#pragma unroll
    for (int i = 0; i < BPW; ++i) load_lds16(rs, voff[i], 0, dst + i * 1024);
  };

  const int g16 = lane >> 4;
  const int t16 = lane & 15;
  const int tr_row = 4 * (g16 >> 1) + (t16 >> 2);
  const int tr_col = 16 * (g16 & 1) + 4 * (t16 & 3);

  f32x16 dqt[NDB];  // dQ^T: rows d, column = this lane's query
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqt[db] = f32x16{};

  if (t_first < nt) gload(t_first);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  int lim = skv;
  if (CAUSAL) {
    const int c_lim = qrow + off + 1;
    lim = c_lim < lim ? c_lim : lim;
  }
  // keys < lim (and >= lo under a window) are visible; compared as lim - 4hh
  // and lo - 4hh against a wave-uniform key
  const int lim_h = lim - 4 * hh;
  const int lo_h = (W > 0 ? qrow + off - W + 1 : -(1 << 30)) - 4 * hh;

  for (int t = t_first; t < nt; ++t) {
    const int stage = t & 1;
    const int k0 = t * BN;
    if (t + 1 < nt) gload(t + 1);
    const unsigned char* tk = smem + stage * 2 * TILE;
    const unsigned char* tv = tk + TILE;
    // skip the tiles no row of this wave sees (causal, window); a branch
    // around the whole step, so the accumulators stay where they are
    // the tile step, with the masks (causal, window) compiled in or out
    auto tile_step = [&](auto masked) {
      // Four MFMA phases written out as a software pipeline (sched_barrier
      // fences; left to itself the compiler read each operand one MFMA
      // ahead and ran the vector work between MFMA blocks):
      //   A: S^T and dP^T of keys 0-31    B: S^T and dP^T of keys 32-63
      //   C: dQ^T from keys 0-31          D: dQ^T from keys 32-63
      // with the vector work (mask, P, dS, bf16) of keys 0-31 spread over
      // the MFMAs of B and that of keys 32-63 over those of C, and every A
      // operand read AH MFMAs ahead into a register ring (one ahead: at two
      // waves per SIMD the other wave hides the rest of the latency, and a
      // deeper ring no longer fits the 256 registers).
      constexpr int NSD = 2 * NDC;  // S^T and dP^T MFMAs of a half
      constexpr int NG = 2 * NDB;   // dQ^T MFMAs of a half
      constexpr int NM = 2 * NSD + 2 * NG;
      constexpr int AH = ATTN_BWD_AHEAD_DQ;
      constexpr int R = AH + 1;
      constexpr int EPS_B = (16 + NSD - 1) / NSD;  // vector elements per MFMA slot of B
      constexpr int EPS_C = (16 + NG - 1) / NG;    // ... of C
      f32x16 st[NKB], dpt[NKB];  // S^T, dP^T: key rows, this lane's query
      bf16x8 sb[NKB][2];
      bf16x8 ring[R];
      auto fetch = [&](const int i) -> bf16x8 {
        if (i < 2 * NSD) {
          const int kbi = i / NSD, j = i % NSD;
          return frag_rows<D>((j & 1) ? tv : tk, 32 * kbi, j >> 1, l32, hh);
        }
        const int i2 = i - 2 * NSD, kbi = i2 / NG, j = i2 % NG;
        return frag_cols<D>(tk, 2 * kbi + j / NDB, j % NDB, tr_row, tr_col);
      };
      // key k0 + 32kbi + 8(r/4) + 4hh + r%4 of this lane's query
      auto vec_elem = [&](const int kbi, const int r) {
        float sv = st[kbi][r];
        const int kk = k0 + 32 * kbi + 8 * (r >> 2) + (r & 3);
        if (decltype(masked)::value && CAUSAL) sv = kk >= lim_h ? -INFINITY : sv;
        if (decltype(masked)::value && LOCAL) sv = kk < lo_h ? -INFINITY : sv;
        const float pv = fast_exp2(fmaf(sv, sl2, neg_lse));
        dpt[kbi][r] = pv * (dpt[kbi][r] - del);
        if (r == 7 || r == 15) sb[kbi][r >> 3] = half_bf16(dpt[kbi], r >> 3);
      };
      static_for<AH>([&](auto ic) { ring[decltype(ic)::value] = fetch(decltype(ic)::value); });
      st[0] = st[1] = dpt[0] = dpt[1] = f32x16{};
      static_for<NM>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if (i + AH < NM) ring[(i + AH) % R] = fetch(i + AH);
        const bf16x8 a = ring[i % R];
        if (i < 2 * NSD) {
          constexpr int kbi = i / NSD, j = i % NSD;
          if (j & 1) dpt[kbi] = mfma32(a, dof[j >> 1], dpt[kbi]);
          else st[kbi] = mfma32(a, qf[j >> 1], st[kbi]);
          if (kbi == 1) {
#pragma unroll
            for (int x = 0; x < EPS_B; ++x)
              if (j * EPS_B + x < 16) vec_elem(0, j * EPS_B + x);
          }
        } else {
          constexpr int i2 = i - 2 * NSD, kbi = i2 / NG, j = i2 % NG;
          dqt[j % NDB] = mfma32(a, sb[kbi][j / NDB], dqt[j % NDB]);
          if (kbi == 0) {
#pragma unroll
            for (int x = 0; x < EPS_C; ++x)
              if (j * EPS_C + x < 16) vec_elem(1, j * EPS_C + x);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    if (k0 < w_end && k0 + BN > w_lo) {
      // masks only on tiles that cross the diagonal or the window's lower
      // edge for some row of this wave; the packed-sequence kernels keep one
      // masked copy (two copies of the step spill there)
      const bool partial = (CAUSAL && k0 + BN - 1 > qw0 + off) || (LOCAL && W > 0 && k0 < qw0 + 31 + off - W + 1);
      if (VARLEN || partial) {
        tile_step(std::true_type{});
      } else {
        tile_step(std::false_type{});
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (qrow < sq) {
    __bf16* dqr = dq + q_el + (int64_t)qrow * q_rs;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(dqt[db][4 * rg + e] * sc);
        *(bf16x4*)(dqr + 32 * db + 8 * rg + 4 * hh) = w;
      }
  }
}

template <int D, bool VARLEN, bool LOCAL, bool BSHD>
hipError_t launch_tiles(const Params& p, const __bf16* dout, float* delta, float* lse2, __bf16* dq, __bf16* dk,
                        __bf16* dv, float* dsinks, hipStream_t st) {
  // dQ first: it also forms Delta and the log2 LSE of every row, which the
  // sink gradient and the dK/dV kernel read.  Dense non-causal grids are
  // padded to a multiple of 8 for the XCD mapping; varlen grids cover an
  // upper bound of the tiles per head (T / tile + sequences), the surplus
  // items exit at once.  LOCAL (a sliding window) is causal.
  auto pad8 = [](long n) { return (n + 7) / 8 * 8; };
  Params q = p;
  long g2;
  if (VARLEN) {
    q.tiles_per_head = p.Sq / 128 + p.B;
    g2 = (long)p.H * q.tiles_per_head;
  } else {
    g2 = (long)p.B * p.H * ceil_div(p.Sq, 128);
    if (!p.causal) g2 = pad8(g2);
  }
  if (LOCAL)
    hipLaunchKernelGGL((dq_kernel<D, true, VARLEN, true, BSHD>), dim3((unsigned)g2), dim3(256), 0, st, q, dout, delta,
                       lse2, dq);
  else if (p.causal)
    hipLaunchKernelGGL((dq_kernel<D, true, VARLEN, false, BSHD>), dim3((unsigned)g2), dim3(256), 0, st, q, dout, delta,
                       lse2, dq);
  else
    hipLaunchKernelGGL((dq_kernel<D, false, VARLEN, false, BSHD>), dim3((unsigned)g2), dim3(256), 0, st, q, dout, delta,
                       lse2, dq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.sinks != nullptr) {
    hipLaunchKernelGGL(dsink_kernel, dim3((unsigned)p.H), dim3(256), 0, st, p.sinks, (const float*)delta,
                       (const float*)lse2, dsinks, VARLEN ? 1 : p.B, p.H, p.Sq);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.Skv > 0) {
    long g1;
    if (VARLEN) {
      q.tiles_per_head = p.Sq / 128 + p.B;
      g1 = (long)p.Hkv * q.tiles_per_head;
    } else {
      g1 = (long)p.B * p.Hkv * ceil_div(p.Skv, 128);
      if (!p.causal) g1 = pad8(g1);
    }
    if (LOCAL)
      hipLaunchKernelGGL((dkdv_pair_kernel<D, true, VARLEN, true, BSHD>), dim3((unsigned)g1), dim3(512), 0, st, q,
                         dout, delta, lse2, dk, dv);
    else if (p.causal)
      hipLaunchKernelGGL((dkdv_pair_kernel<D, true, VARLEN, false, BSHD>), dim3((unsigned)g1), dim3(512), 0, st, q,
                         dout, delta, lse2, dk, dv);
    else
      hipLaunchKernelGGL((dkdv_pair_kernel<D, false, VARLEN, false, BSHD>), dim3((unsigned)g1), dim3(512), 0, st, q,
                         dout, delta, lse2, dk, dv);
    e = hipGetLastError();
  }
  return e;
}

template <int D>
hipError_t launch_bwd_d(const Params& p, const __bf16* dout, float* delta, float* lse2, __bf16* dq, __bf16* dk,
                        __bf16* dv, float* dsinks, hipStream_t st) {
  const bool var = p.cu != nullptr;
  const bool local = p.window > 0;
  if (p.bshd) {
    if (var)
      return local ? launch_tiles<D, true, true, true>(p, dout, delta, lse2, dq, dk, dv, dsinks, st)
                   : launch_tiles<D, true, false, true>(p, dout, delta, lse2, dq, dk, dv, dsinks, st);
    return local ? launch_tiles<D, false, true, true>(p, dout, delta, lse2, dq, dk, dv, dsinks, st)
                 : launch_tiles<D, false, false, true>(p, dout, delta, lse2, dq, dk, dv, dsinks, st);
  }
  if (var)
    return local ? launch_tiles<D, true, true, false>(p, dout, delta, lse2, dq, dk, dv, dsinks, st)
                 : launch_tiles<D, true, false, false>(p, dout, delta, lse2, dq, dk, dv, dsinks, st);
  return local ? launch_tiles<D, false, true, false>(p, dout, delta, lse2, dq, dk, dv, dsinks, st)
               : launch_tiles<D, false, false, false>(p, dout, delta, lse2, dq, dk, dv, dsinks, st);
}

}  // namespace

hipError_t launch_backward(const Params& p, const void* dout, float* delta, float* lse2, void* dq, void* dk,
                           void* dv, float* dsinks, hipStream_t st) {
  if ((long)p.B * p.H * p.Sq <= 0) return hipSuccess;
  if (p.d == 128)
    return launch_bwd_d<128>(p, (const __bf16*)dout, delta, lse2, (__bf16*)dq, (__bf16*)dk, (__bf16*)dv, dsinks, st);
  if (p.d == 64)
    return launch_bwd_d<64>(p, (const __bf16*)dout, delta, lse2, (__bf16*)dq, (__bf16*)dk, (__bf16*)dv, dsinks, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
