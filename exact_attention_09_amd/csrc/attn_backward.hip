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
// Three kernels, no atomics, fixed summation orders (bitwise reproducible):
//   * delta_kernel: Delta in fp32;
//   * dkdv_kernel: one workgroup per (batch, KV head, 128 keys); each wave
//     keeps its 32 keys' K and V rows in registers and walks the query tiles
//     of every query head of the group, so the grouped-query sum happens in
//     registers;
//   * dq_kernel: one workgroup per (batch, query head, 128 queries); each
//     wave keeps its 32 queries' Q and dO rows in registers and walks the key
//     tiles.  dQ costs a second computation of S and dP instead of atomic
//     partial sums.
//
// Both tile kernels use v_mfma_f32_32x32x16_bf16 with the accumulator
// arranged so that the exponentiated scores are directly the B operand of the
// next product (as in the forward kernels): dkdv computes S = Q K^T (one key
// per lane) and dV^T = dO^T P, dK^T = Q^T dS; dq computes S^T = K Q^T (one
// query per lane) and dQ^T = K^T dS^T.  Tiles sit row-major in LDS with the
// 16-byte chunk swizzle of attn_common.h; the transposed operands are read
// with ds_read_b64_tr_b16.  P and dS are rounded to bf16 (nearest even) for
// the products that consume them; every accumulation is fp32.
#include "attn_common.h"
#include "attn_internal.h"

namespace attn {

namespace {

constexpr float kLog2e = 1.44269504088896340736f;

// ---------------------------------------------------------------- Delta

// Delta = rowsum(dO * O) per row, fp32; D/8 lanes per row, 16 bytes each.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ dout,
                                                   float* __restrict__ delta, long rows) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int sub = threadIdx.x % TPR;
  const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
  float acc = 0.0f;
  if (row < rows) {
    const bf16x8 a = *(const bf16x8*)(o + row * D + 8 * sub);
    const bf16x8 b = *(const bf16x8*)(dout + row * D + 8 * sub);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += (float)a[j] * (float)b[j];
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && sub == 0) delta[row] = acc;
}

// ---------------------------------------------------------------- shared

// Row-major tile of `rows` rows of D bf16 in LDS (16-byte chunks swizzled),
// loaded through registers by 256 threads.
template <int D, int ROWS>
struct TileLoader {
  static constexpr int ROWB = D * 2;
  static constexpr int CH = D / 8;
  static constexpr int RPP = 256 / CH;
  static constexpr int PASSES = ROWS / RPP;
  static_assert(ROWS % RPP == 0, "tile rows must be a multiple of the load pass");
  u32x4 reg[PASSES];
  int c, r;
  __device__ void init(int tid) {
    c = tid % CH;
    r = tid / CH;
  }
  // rows [0, valid) of `base` (row stride D); the rest read as zero
  __device__ void load(const __bf16* base, int valid) {
    const int n = valid < ROWS ? (valid > 0 ? valid : 0) : ROWS;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, n * ROWB);
#pragma unroll
    for (int i = 0; i < PASSES; ++i) reg[i] = buffer_load16(rs, r * ROWB + c * 16, i * RPP * ROWB);
  }
  __device__ void store(unsigned char* lds) const {
#pragma unroll
    for (int i = 0; i < PASSES; ++i) *(u32x4*)(lds + lds_off<D>(r + RPP * i, c)) = reg[i];
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

// bf16 x 8 of accumulator registers 8(kc&1) .. +8 of block kc>>1
__device__ inline bf16x8 chunk_bf16(const f32x16* acc, int kc) {
  const f32x16& a = acc[kc >> 1];
  const int rb = 8 * (kc & 1);
  return to_bf16x8(a[rb + 0], a[rb + 1], a[rb + 2], a[rb + 3], a[rb + 4], a[rb + 5], a[rb + 6], a[rb + 7]);
}

// ---------------------------------------------------------------- dK, dV

// Keys stationary: workgroup (b, KV head, 128 keys), wave w owns keys
// k0 + 32w .. +31 (one per lane of a half-wave pair).  Query tiles of 64 rows
// of every query head of the group stream through LDS (Q, dO, log2-domain
// LSE and Delta), double buffered.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(const Params p, const __bf16* __restrict__ dout,
                                                      const float* __restrict__ delta, __bf16* __restrict__ dk,
                                                      __bf16* __restrict__ dv) {
  constexpr int BK = 128;        // keys per workgroup
  constexpr int BQ = 64;         // queries per tile
  constexpr int NDC = D / 16;    // contraction chunks over d
  constexpr int NDB = D / 32;    // 32-column blocks of d
  constexpr int NQB = BQ / 32;   // 32-query blocks of a tile
  constexpr int NQC = BQ / 16;   // 16-query chunks of a tile
  constexpr int TILE = BQ * D * 2;
  constexpr int STAGE = 2 * TILE + 2 * BQ * 4;  // Q, dO, lse, delta
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const float sl2 = p.scale_log2;

  // causal: key tiles in order of decreasing work (a key tile's query range
  // shrinks as the keys move right), so the light tiles fill the tail
  const int ktiles = ceil_div(p.Skv, BK);
  const int item = blockIdx.x;
  const int nbk = p.B * p.Hkv;
  const int kt = CAUSAL ? item / nbk : item % ktiles;
  const int bk = CAUSAL ? item - kt * nbk : item / ktiles;  // b * Hkv + kvh
  const int b = bk / p.Hkv;
  const int kvh = bk - b * p.Hkv;
  const int sq = p.Sq, skv = p.Skv, off = skv - sq;
  const int k0 = kt * BK;
  const int kw0 = k0 + 32 * wave;
  const int krow = kw0 + l32;

  const __bf16* __restrict__ K = (const __bf16*)p.k + (int64_t)bk * skv * D;
  const __bf16* __restrict__ V = (const __bf16*)p.v + (int64_t)bk * skv * D;

  // this lane's key row as the B operand of S = Q K^T and dP = dO V^T
  bf16x8 kf[NDC], vf[NDC];
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    if (krow < skv) {
      kf[c] = *(const bf16x8*)(K + (int64_t)krow * D + 16 * c + 8 * hh);
      vf[c] = *(const bf16x8*)(V + (int64_t)krow * D + 16 * c + 8 * hh);
    } else {
      kf[c] = bf16x8{};
      vf[c] = bf16x8{};
    }
  }

  f32x16 dkt[NDB], dvt[NDB];  // dK^T, dV^T: rows d, column = this lane's key
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dkt[db] = f32x16{};
    dvt[db] = f32x16{};
  }

  // queries that can see a key of this workgroup (bottom-right causal):
  // i >= j - off
  int qbeg = 0;
  if (CAUSAL) {
    qbeg = k0 - off;
    qbeg = qbeg < 0 ? 0 : qbeg;
  }
  const int qt0 = qbeg / BQ;
  const int nqt = ceil_div(sq, BQ);
  const int per_head = nqt > qt0 ? nqt - qt0 : 0;
  const int nsteps = per_head * p.group;

  TileLoader<D, BQ> lq, ldo;
  lq.init(tid);
  ldo.init(tid);
  float lse_reg = 0.0f, del_reg = 0.0f;
  auto step_src = [&](int s, int& h, int& q0) {
    h = kvh * p.group + s / per_head;
    q0 = (qt0 + s % per_head) * BQ;
  };
  auto gload = [&](int s) {
    int h, q0;
    step_src(s, h, q0);
    const int64_t row0 = ((int64_t)b * p.H + h) * sq + q0;
    lq.load((const __bf16*)p.q + row0 * D, sq - q0);
    ldo.load(dout + row0 * D, sq - q0);
    if (tid < BQ) {
      const int i = q0 + tid;
      // rows past the end and rows that saw no key take part with P = 0:
      // their log-sum-exp becomes +inf
      float l = i < sq ? p.lse[row0 + tid] : -INFINITY;
      lse_reg = l == -INFINITY ? INFINITY : l * kLog2e;
      del_reg = i < sq ? delta[row0 + tid] : 0.0f;
    }
  };
  auto lstore = [&](int stage) {
    unsigned char* base = smem + stage * STAGE;
    lq.store(base);
    ldo.store(base + TILE);
    if (tid < BQ) {
      ((float*)(base + 2 * TILE))[tid] = lse_reg;
      ((float*)(base + 2 * TILE + BQ * 4))[tid] = del_reg;
    }
  };

  const int g16 = lane >> 4;
  const int t16 = lane & 15;
  const int tr_row = 4 * (g16 >> 1) + (t16 >> 2);
  const int tr_col = 16 * (g16 & 1) + 4 * (t16 & 3);

  if (nsteps > 0) {
    gload(0);
    lstore(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const int stage = s & 1;
    if (s + 1 < nsteps) gload(s + 1);
    int h, q0;
    step_src(s, h, q0);
    (void)h;
    const unsigned char* tq = smem + stage * STAGE;
    const unsigned char* tdo = tq + TILE;
    const float* tlse = (const float*)(tq + 2 * TILE);
    const float* tdel = tlse + BQ;
    // this wave's keys see a query of the tile (causal) and exist
    const bool live = kw0 < skv && (!CAUSAL || kw0 <= q0 + BQ - 1 + off);
    if (live) {
      f32x16 sacc[NQB], dpacc[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        sacc[qb] = f32x16{};
        dpacc[qb] = f32x16{};
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
          sacc[qb] = mfma32(frag_rows<D>(tq, 32 * qb, c, l32, hh), kf[c], sacc[qb]);
          dpacc[qb] = mfma32(frag_rows<D>(tdo, 32 * qb, c, l32, hh), vf[c], dpacc[qb]);
        }
      }
      // P and dS, one key per lane, query rows 32qb + 8(r/4) + 4hh + r%4
      const bool partial = CAUSAL && (kw0 + 31 > q0 + off);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int rr = 32 * qb + 8 * g + 4 * hh;
          const f32x4 lv = *(const f32x4*)(tlse + rr);
          const f32x4 dl = *(const f32x4*)(tdel + rr);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float sv = sacc[qb][r];
            if (partial && krow > q0 + rr + e + off) sv = -INFINITY;
            const float pv = fast_exp2(fmaf(sv, sl2, -lv[e]));
            sacc[qb][r] = pv;
            dpacc[qb][r] = pv * (dpacc[qb][r] - dl[e]);
          }
        }
      }
      // dV^T += dO^T P, dK^T += Q^T dS (16 queries per step)
#pragma unroll
      for (int qc = 0; qc < NQC; ++qc) {
        const bf16x8 pb = chunk_bf16(sacc, qc);
        const bf16x8 sb = chunk_bf16(dpacc, qc);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dvt[db] = mfma32(frag_cols<D>(tdo, qc, db, tr_row, tr_col), pb, dvt[db]);
          dkt[db] = mfma32(frag_cols<D>(tq, qc, db, tr_row, tr_col), sb, dkt[db]);
        }
      }
    }
    if (s + 1 < nsteps) lstore(stage ^ 1);
    __syncthreads();
  }

  // dK = s dK^T^T, dV = dV^T^T: this lane's key row, d = 32db + 8rg + 4hh .. +4
  if (krow < skv) {
    __bf16* dkr = dk + ((int64_t)bk * skv + krow) * D;
    __bf16* dvr = dv + ((int64_t)bk * skv + krow) * D;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = (__bf16)(dkt[db][4 * rg + e] * sc);
          wv[e] = (__bf16)(dvt[db][4 * rg + e]);
        }
        *(bf16x4*)(dkr + 32 * db + 8 * rg + 4 * hh) = wk;
        *(bf16x4*)(dvr + 32 * db + 8 * rg + 4 * hh) = wv;
      }
  }
}

// ---------------------------------------------------------------- dQ

// Queries stationary: workgroup (b, query head, 128 queries), wave w owns
// queries q0 + 32w .. +31 (one per lane of a half-wave pair); key tiles of 64
// rows stream through LDS, double buffered.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void dq_kernel(const Params p, const __bf16* __restrict__ dout,
                                                    const float* __restrict__ delta, __bf16* __restrict__ dq) {
  constexpr int BMQ = 128;
  constexpr int BN = 64;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NKB = BN / 32;
  constexpr int NKC = BN / 16;
  constexpr int TILE = BN * D * 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * 2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const float sl2 = p.scale_log2;

  // causal: query tiles in order of decreasing work (the last tiles see the
  // most keys)
  const int qtiles = ceil_div(p.Sq, BMQ);
  const int item = blockIdx.x;
  const int nbh = p.B * p.H;
  const int bh = CAUSAL ? item % nbh : item / qtiles;
  const int tile = CAUSAL ? qtiles - 1 - item / nbh : item - bh * qtiles;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int sq = p.Sq, skv = p.Skv, off = skv - sq;
  const int q0 = tile * BMQ;
  const int qw0 = q0 + 32 * wave;
  const int qrow = qw0 + l32;
  const int64_t row0 = (int64_t)bh * sq;

  const __bf16* __restrict__ Q = (const __bf16*)p.q + row0 * D;
  const __bf16* __restrict__ dO = dout + row0 * D;
  const int64_t kv0 = ((int64_t)b * p.Hkv + h / p.group) * skv;
  const __bf16* __restrict__ K = (const __bf16*)p.k + kv0 * D;
  const __bf16* __restrict__ V = (const __bf16*)p.v + kv0 * D;

  bf16x8 qf[NDC], dof[NDC];
  float neg_lse = -INFINITY, del = 0.0f;  // -LSE log2(e) of this lane's row
  if (qrow < sq) {
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      qf[c] = *(const bf16x8*)(Q + (int64_t)qrow * D + 16 * c + 8 * hh);
      dof[c] = *(const bf16x8*)(dO + (int64_t)qrow * D + 16 * c + 8 * hh);
    }
    const float l = p.lse[row0 + qrow];
    neg_lse = l == -INFINITY ? -INFINITY : -l * kLog2e;  // no key seen: P = 0
    del = delta[row0 + qrow];
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
  int w_end = 0;
  if (qw0 < sq) {
    const int w_hi = qw0 + 32 < sq ? qw0 + 32 : sq;
    w_end = CAUSAL ? causal_kv_end(w_hi, off, skv) : skv;
  }

  TileLoader<D, BN> lk, lv;
  lk.init(tid);
  lv.init(tid);
  auto gload = [&](int t) {
    const int k0 = t * BN;
    lk.load(K + (int64_t)k0 * D, skv - k0);
    lv.load(V + (int64_t)k0 * D, skv - k0);
  };
  auto lstore = [&](int stage) {
    lk.store(smem + stage * 2 * TILE);
    lv.store(smem + stage * 2 * TILE + TILE);
  };

  const int g16 = lane >> 4;
  const int t16 = lane & 15;
  const int tr_row = 4 * (g16 >> 1) + (t16 >> 2);
  const int tr_col = 16 * (g16 & 1) + 4 * (t16 & 3);

  f32x16 dqt[NDB];  // dQ^T: rows d, column = this lane's query
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqt[db] = f32x16{};

  if (nt > 0) {
    gload(0);
    lstore(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  int lim = skv;
  if (CAUSAL) {
    const int c_lim = qrow + off + 1;
    lim = c_lim < lim ? c_lim : lim;
  }

  for (int t = 0; t < nt; ++t) {
    const int stage = t & 1;
    const int k0 = t * BN;
    if (t + 1 < nt) gload(t + 1);
    if (k0 < w_end) {
      const unsigned char* tk = smem + stage * 2 * TILE;
      const unsigned char* tv = tk + TILE;
      f32x16 st[NKB], dpt[NKB];  // S^T, dP^T: key rows, this lane's query
#pragma unroll
      for (int kbi = 0; kbi < NKB; ++kbi) {
        st[kbi] = f32x16{};
        dpt[kbi] = f32x16{};
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
          st[kbi] = mfma32(frag_rows<D>(tk, 32 * kbi, c, l32, hh), qf[c], st[kbi]);
          dpt[kbi] = mfma32(frag_rows<D>(tv, 32 * kbi, c, l32, hh), dof[c], dpt[kbi]);
        }
      }
      const bool partial = (k0 + BN > skv) || (CAUSAL && (k0 + BN - 1 > qw0 + off));
#pragma unroll
      for (int kbi = 0; kbi < NKB; ++kbi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sv = st[kbi][r];
          if (partial && k0 + 32 * kbi + 8 * (r >> 2) + 4 * hh + (r & 3) >= lim) sv = -INFINITY;
          const float pv = fast_exp2(fmaf(sv, sl2, neg_lse));
          dpt[kbi][r] = pv * (dpt[kbi][r] - del);
        }
      // dQ^T += K^T dS^T over 16-key steps
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const bf16x8 sb = chunk_bf16(dpt, kc);
#pragma unroll
        for (int db = 0; db < NDB; ++db) dqt[db] = mfma32(frag_cols<D>(tk, kc, db, tr_row, tr_col), sb, dqt[db]);
      }
    }
    if (t + 1 < nt) lstore(stage ^ 1);
    __syncthreads();
  }

  if (qrow < sq) {
    __bf16* dqr = dq + (row0 + qrow) * D;
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

template <int D>
hipError_t launch_bwd_d(const Params& p, const __bf16* dout, float* delta, __bf16* dq, __bf16* dk, __bf16* dv,
                        hipStream_t st) {
  const long rows = (long)p.B * p.H * p.Sq;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL(delta_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st,
                     (const __bf16*)p.o, dout, delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.Skv > 0) {
    const long g1 = (long)p.B * p.Hkv * ceil_div(p.Skv, 128);
    if (p.causal)
      hipLaunchKernelGGL((dkdv_kernel<D, true>), dim3((unsigned)g1), dim3(256), 0, st, p, dout, delta, dk, dv);
    else
      hipLaunchKernelGGL((dkdv_kernel<D, false>), dim3((unsigned)g1), dim3(256), 0, st, p, dout, delta, dk, dv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long g2 = (long)p.B * p.H * ceil_div(p.Sq, 128);
  if (p.causal)
    hipLaunchKernelGGL((dq_kernel<D, true>), dim3((unsigned)g2), dim3(256), 0, st, p, dout, delta, dq);
  else
    hipLaunchKernelGGL((dq_kernel<D, false>), dim3((unsigned)g2), dim3(256), 0, st, p, dout, delta, dq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const Params& p, const void* dout, float* delta, void* dq, void* dk, void* dv,
                           hipStream_t st) {
  if ((long)p.B * p.H * p.Sq <= 0) return hipSuccess;
  if (p.d == 128)
    return launch_bwd_d<128>(p, (const __bf16*)dout, delta, (__bf16*)dq, (__bf16*)dk, (__bf16*)dv, st);
  if (p.d == 64)
    return launch_bwd_d<64>(p, (const __bf16*)dout, delta, (__bf16*)dq, (__bf16*)dk, (__bf16*)dv, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
