// Tiled attention forward for bf16 inputs on gfx950 (prefill and varlen).
//
// The loop is the FlashAttention-2 order described in the TileLang tutorial
// chapter 15 ("15-operators-attention"), section 3.2: a workgroup owns a
// query tile, streams K/V tiles through LDS, keeps per row the running max m
// and denominator l, rescales the accumulator when m moves, accumulates
// P~ V and divides by l once at the end.  Causal loop trimming, the tail
// mask and the bottom-right diagonal follow its section 3.4; the guard for
// rows that have seen no key follows its section 5.1.
//
// gfx950 mapping:
//   * 256 threads = 4 waves; each wave owns 32 query rows (BM = 128), so
//     every row reduction stays inside one wave (the tutorial's "FullRow"
//     warp policy, its section 4.2).
//   * both products run on v_mfma_f32_32x32x16_bf16 in transposed form,
//     S^T = K Q^T and O^T = V^T P^T, so the accumulators of both put one
//     query row per lane (lane l: row l%32, lane halves split the keys / the
//     d columns).  The S^T accumulator registers are, after exp2 and the
//     bf16 conversion, directly the B operand of the second product.
//   * K and V tiles are staged row-major in LDS with a 16-byte chunk
//     swizzle; K is read as the A operand with ds_read_b128, V is read
//     transposed with ds_read_b64_tr_b16 (no register shuffles).
//   * K/V tiles are double buffered: the global loads of tile t+1 are issued
//     before the math of tile t and land in LDS after it (one barrier per
//     tile).
//   * the running max is updated lazily: the accumulator is rescaled only
//     when a row's max grows by more than 2^8 (in exp2 units).  The tutorial's
//     section 2.4 proof shows the result does not depend on which reference
//     max is used, only the range of the intermediates does; P~ stays
//     <= 256.
#include "attn_common.h"
#include "attn_internal.h"

namespace attn {

namespace {

constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units
constexpr float kLn2 = 0.69314718055994530942f;

template <int D, int BN, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(const Params p) {
  constexpr int BM = 128;
  constexpr int ROWB = D * 2;               // bytes per K/V row
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int TILE_B = BN * ROWB;         // bytes per K or V tile
  constexpr int RPP = 256 / CH;             // rows per load pass
  constexpr int PASSES = BN / RPP;          // 16-byte loads per thread per tile
  constexpr int NKB = BN / 32;              // 32-key blocks of S^T
  constexpr int NDB = D / 32;               // 32-column blocks of O^T
  constexpr int NDC = D / 16;               // contraction steps of QK^T
  constexpr int NKC = BN / 16;              // contraction steps of P~V
  static_assert(BN % RPP == 0, "tile rows must be a multiple of the load pass");

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * 2 * TILE_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const float sl2 = p.scale_log2;

  // ---- work item -> (b, h, query tile)
  const int v = xcd_remap(blockIdx.x, p.work_items);
  if (v < 0) return;
  int h, tile, sq, skv, off;
  int64_t q_row0, kv_row0;
  if constexpr (!VARLEN) {
    int b;
    dense_item(v, p.tiles_per_head, p.H, CAUSAL, b, h, tile);  // heavy tiles first
    sq = p.Sq;
    skv = p.Skv;
    off = skv - sq;
    q_row0 = ((int64_t)b * p.H + h) * sq;
    kv_row0 = ((int64_t)b * p.Hkv + h / p.group) * skv;
  } else {
    int bb;
    if (!varlen_item(p.cu, p.B, p.Sq, BM, p.tiles_per_head, CAUSAL, v, h, bb, tile)) return;
    int s0, s1;
    seq_bounds(p.cu, p.Sq, bb, s0, s1);
    sq = s1 - s0;
    skv = sq;
    off = 0;
    q_row0 = (int64_t)h * p.Sq + s0;
    kv_row0 = (int64_t)(h / p.group) * p.Sq + s0;
  }

  const __bf16* __restrict__ Q = (const __bf16*)p.q + q_row0 * D;
  const __bf16* __restrict__ K = (const __bf16*)p.k + kv_row0 * D;
  const __bf16* __restrict__ V = (const __bf16*)p.v + kv_row0 * D;
  __bf16* __restrict__ O = (__bf16*)p.o + q_row0 * D;

  const int q0 = tile * BM;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;

  // ---- Q fragments (B operand of S^T = K Q^T): row qrow, d = 16c + 8hh + j
  bf16x8 qf[NDC];
  if (qrow < sq) {
#pragma unroll
    for (int c = 0; c < NDC; ++c) qf[c] = *(const bf16x8*)(Q + (int64_t)qrow * D + 16 * c + 8 * hh);
  } else {
#pragma unroll
    for (int c = 0; c < NDC; ++c) qf[c] = bf16x8{};
  }

  // ---- key range: the workgroup loads up to kv_end; this wave needs w_end
  const int q_hi = q0 + BM < sq ? q0 + BM : sq;
  const int kv_end = CAUSAL ? causal_kv_end(q_hi, off, skv) : skv;
  const int nt = ceil_div(kv_end, BN);
  int w_end;
  if (qw0 >= sq) {
    w_end = 0;
  } else {
    const int w_hi = qw0 + 32 < sq ? qw0 + 32 : sq;
    w_end = CAUSAL ? causal_kv_end(w_hi, off, skv) : skv;
  }

  // ---- global -> register -> LDS tile loader.  Buffer loads over the
  // tile's valid rows: keys past skv read as zero (and are masked), the
  // per-lane offset is the same for every tile, only the base moves.
  const int ld_c = tid % CH;
  const int ld_r = tid / CH;
  const int ld_voff = ld_r * ROWB + ld_c * 16;
  u32x4 kreg[PASSES], vreg[PASSES];
  auto gload = [&](int k0) {
    const int rows = skv - k0 < BN ? skv - k0 : BN;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + (int64_t)k0 * D, rows * ROWB);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + (int64_t)k0 * D, rows * ROWB);
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      kreg[i] = buffer_load16(kr, ld_voff, i * RPP * ROWB);
      vreg[i] = buffer_load16(vr, ld_voff, i * RPP * ROWB);
    }
  };
  auto lstore = [&](int stage) {
    unsigned char* kb = smem + stage * (2 * TILE_B);
    unsigned char* vb = kb + TILE_B;
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int r = ld_r + RPP * i;
      *(u32x4*)(kb + lds_off<D>(r, ld_c)) = kreg[i];
      *(u32x4*)(vb + lds_off<D>(r, ld_c)) = vreg[i];
    }
  };

  // ---- per-lane constant parts of the transposed V read: lane (g, t) of
  // a 16-lane group addresses row 4*(g>>1) + (t>>2) (+16kc + 8e) and column
  // 16*(g&1) + 4*(t&3) (+32db); the result is V^T for d = 32db + l%32.
  const int g16 = lane >> 4;
  const int t16 = lane & 15;
  const int vtr_row = 4 * (g16 >> 1) + (t16 >> 2);
  const int vtr_col = 16 * (g16 & 1) + 4 * (t16 & 3);

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_used = -INFINITY;  // reference max (raw score units)
  float neg_ms = 0.0f;       // -m_used * scale_log2 (0 while no key seen)
  float l_part = 0.0f;       // this lane's share of the denominator

  if (nt > 0) {
    gload(0);
    lstore(0);
  }
  // Every global load issued so far (Q fragments, tile 0) completes here, so
  // the loop body only ever waits for its own prefetch.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int stage = t & 1;
    const int k0 = t * BN;
    if (t + 1 < nt) gload(k0 + BN);

    if (k0 < w_end) {
      const unsigned char* kb = smem + stage * (2 * TILE_B);
      const unsigned char* vb = kb + TILE_B;

      // S^T = K Q^T: lane holds S[qrow][k0 + 32kb + 8(r/4) + 4hh + r%4]
      f32x16 s[NKB];
#pragma unroll
      for (int kbi = 0; kbi < NKB; ++kbi) {
        s[kbi] = f32x16{};
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
          const bf16x8 a = *(const bf16x8*)(kb + lds_off<D>(kbi * 32 + l32, 2 * c + hh));
          s[kbi] = mfma32(a, qf[c], s[kbi]);
        }
      }

      // mask only tiles that cross the tail or the causal diagonal
      const bool partial = (k0 + BN > skv) || (CAUSAL && (k0 + BN - 1 > qw0 + off));
      if (partial) {
        int lim = skv;
        if (CAUSAL) {
          const int c_lim = qrow + off + 1;
          lim = c_lim < lim ? c_lim : lim;
        }
#pragma unroll
        for (int kbi = 0; kbi < NKB; ++kbi)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kbi + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= lim) s[kbi][r] = -INFINITY;
          }
      }

      // row max of the tile (in-lane, then across the two lane halves)
      float mx = -INFINITY;
#pragma unroll
      for (int kbi = 0; kbi < NKB; ++kbi)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kbi][r]);
      mx = pair32_max(mx);

      // lazy rescale: move the reference max only when P~ would exceed 2^tau
      const bool need = (mx > m_used) && ((mx - m_used) * sl2 > kTau);
      if (__any(need)) {
        const float m_new = need ? mx : m_used;
        const float alpha = need ? fast_exp2((m_used - m_new) * sl2) : 1.0f;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m_used = m_new;
        neg_ms = (m_used == -INFINITY) ? 0.0f : -m_used * sl2;
      }

      // P~ = exp2(S * s*log2e - m * s*log2e); denominator summed in fp32
      float rs = 0.0f;
#pragma unroll
      for (int kbi = 0; kbi < NKB; ++kbi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(fmaf(s[kbi][r], sl2, neg_ms));
          s[kbi][r] = e;
          rs += e;
        }
      l_part += rs;

      // O^T += V^T P~^T over 16-key steps
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const f32x16& sk = s[kc >> 1];
        const int rb = 8 * (kc & 1);
        const bf16x8 pb = to_bf16x8(sk[rb + 0], sk[rb + 1], sk[rb + 2], sk[rb + 3], sk[rb + 4],
                                    sk[rb + 5], sk[rb + 6], sk[rb + 7]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int col = 32 * db + vtr_col;
          const int row0 = 16 * kc + vtr_row;
          const s16x4 lo = lds_read_tr16(vb + lds_off<D>(row0, col >> 3) + (col & 7) * 2);
          const s16x4 hi = lds_read_tr16(vb + lds_off<D>(row0 + 8, col >> 3) + (col & 7) * 2);
          oacc[db] = mfma32(join_tr(lo, hi), pb, oacc[db]);
        }
      }
    }

    if (t + 1 < nt) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l (0 for rows that saw no key), LSE natural log
  const float l = pair32_sum(l_part);
  if (qrow < sq) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    __bf16* orow = O + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 w;
        w[0] = (__bf16)(oacc[db][4 * rg + 0] * inv);
        w[1] = (__bf16)(oacc[db][4 * rg + 1] * inv);
        w[2] = (__bf16)(oacc[db][4 * rg + 2] * inv);
        w[3] = (__bf16)(oacc[db][4 * rg + 3] * inv);
        *(bf16x4*)(orow + 32 * db + 8 * rg + 4 * hh) = w;
      }
    if (p.lse != nullptr && hh == 0)
      p.lse[q_row0 + qrow] = l > 0.0f ? (m_used * sl2 + fast_log2(l)) * kLn2 : -INFINITY;
  }
}

template <int D, int BN, bool CAUSAL, bool VARLEN>
hipError_t launch_one(const Params& p, hipStream_t st) {
  const int grid = 8 * ceil_div(p.work_items, 8);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, BN, CAUSAL, VARLEN>), dim3(grid), dim3(256), 0, st,
                     p);
  return hipGetLastError();
}

template <int D, int BN>
hipError_t launch_d(const Params& p, hipStream_t st) {
  const bool var = p.cu != nullptr;
  if (p.causal) return var ? launch_one<D, BN, true, true>(p, st) : launch_one<D, BN, true, false>(p, st);
  return var ? launch_one<D, BN, false, true>(p, st) : launch_one<D, BN, false, false>(p, st);
}

}  // namespace

int prefill_bf16_block_m() { return 128; }

hipError_t launch_prefill_bf16(const Params& p, hipStream_t st) {
  if (p.work_items <= 0) return hipSuccess;
  if (p.d == 128) return launch_d<128, 64>(p, st);
  return launch_d<64, 128>(p, st);
}

}  // namespace attn
