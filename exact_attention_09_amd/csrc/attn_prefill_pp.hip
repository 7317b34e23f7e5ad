// Tiled forward for bf16 (d = 64 or 128), with matrix and vector phases of two wave
// groups interleaved ("ping-pong"), gfx950.
//
// Same method as the basic tiled kernel (TileLang tutorial chapter 15,
// sections 3.2 and 3.4; guards from section 5.1): one workgroup per query
// tile, K/V tiles streamed through LDS, running max and denominator per row,
// one division at the end.  The difference is how the work is laid on the CU.
//
// Per K/V tile a wave has two kinds of work: a matrix phase (the P~V MFMAs of
// the previous tile and the QK^T MFMAs of this tile, d/4 MFMAs) and a vector
// phase (mask, exp2 against the reference max, row sum, bf16 conversion).  The
// tutorial's pipelining discussion (section 3.3) and the FA-3 / FA-4 notes of
// the CUDA course chapter 12 are about overlapping exactly these two.  Here
// the overlap comes from the other wave on the same SIMD:
//
//   * 8 waves (512 threads), 32 query rows each, BM = 256.  Waves 0-3 form
//     group A, waves 4-7 group B; wave w and wave w+4 share a SIMD.
//   * Time is cut into slots by workgroup barriers.  In every slot one group
//     runs its matrix phase while the other runs its vector phase; group B
//     runs one slot behind group A, so the roles alternate every slot.  Each
//     group runs its own copy of the slot sequence, so the role of every
//     slot is fixed in the code rather than tested at run time.
//   * Per-wave checks (is the tile computed, masked, the split tile) are
//     hoisted out of the loop: each wave's "steady" tiles, which it computes
//     whole with no key masked for any of its rows, form one range, and at
//     d = 128 (outside the window variant) the slot loop is split around it,
//     so a steady slot pair runs without any test.  Matrix phases inside an
//     item always run both products: a wave that does not compute a tile
//     holds P~ = 0 for it, so that tile's P~V adds nothing (K and V values
//     are assumed finite, as the masked keys of a partial tile already
//     require: 0 times a non-finite V would spread into the row).
//   * Each wave keeps a single S tile in registers (32 rows x 64 keys; at
//     d = 64, 128 keys), so the register footprint is that of the plain loop
//     (2 waves per SIMD).
//   * K/V tiles (64 keys; 128 at d = 64) live in a ring of PF + 2 LDS stages
//     of 32 KB.  A
//     tile is read during four consecutive slots (K by A then B, V by A then
//     B two slots later).  Tiles go from HBM straight to LDS (buffer_load ...
//     lds, no registers on the way), laid out in MFMA fragment order; tile u
//     is fetched in slots 2(u-PF) (V, by group B) and 2(u-PF)+1 (K, by group
//     A), each at the start of the loading group's vector phase, into the
//     stage of tile u-PF-2, after the barrier that ends that tile's last
//     read, and waited for at the end of slot 2u-1.
//   * S^T = K Q^T and O^T = V^T P~^T on v_mfma_f32_32x32x16_bf16 (one query
//     row per lane), K read with ds_read_b128, V with ds_read_b64_tr_b16.
//     Each fragment read covers one contiguous block (1 KB or 512 B), so it
//     is free of bank conflicts and its address is one register plus an
//     immediate.
//   * In steady state the P~V and QK^T MFMAs of a matrix phase (16 each) are
//     issued alternately, each with its operand read three MFMAs ahead:
//     pinned with sched_group_barrier in the BHSD d = 128 instantiations,
//     written out with a register ring and sched_barrier fences elsewhere
//     (where the scheduler drops the pins and every MFMA would wait for its
//     read).
//   * At d = 64 the 16-key chunks of a diagonal tile past every row of the
//     wave get no exponentials (P~ = 0), and a wave's first tile goes to the
//     exact reference update directly.
//   * Reference max without a per-tile max: P~ = exp2(S scale' - m scale')
//     against the current reference m, S kept in registers.  If some lane's
//     share of a row's tile sum exceeds 2^8 (so some P~ > 2^8), or a row has
//     no reference yet, the tile takes a rare path: exact row max, m <-
//     max(m, rowmax), O and l scaled by exp2((m_old - m_new) scale'), P~
//     again.  P~ stays <= 2^8 as with the lazy rescale of the basic kernel,
//     which instead compares the tile max with m every tile.
//   * Sliding window (causal only; TileLang tutorial section 5.2, the CUDA
//     course chapter 12, section 12.9.5): key j is visible to row i iff
//     i + off - W < j <= i + off.  The workgroup loads only the tiles from
//     the first key its top row sees, each wave computes only the tiles its
//     rows see, and tiles crossing the lower edge are masked like the
//     diagonal ones.  Rows whose first tiles are fully masked keep no
//     reference max until they see a key (the section 5.1 (1) check_inf).
//   * Attention sink (tutorial sections 4.6 and 4.7): in the epilogue the
//     sink's exp2(sink log2(e) - m*) joins the denominator, with
//     m* = max(m scale', sink log2(e)) so that a large sink cannot overflow.
//   * The epilogue writes the normalised O tile into the (then idle) LDS
//     ring and stores it as whole rows (tutorial section 3.4 (5): the MFMA
//     fragment layout needs a staging hop for coalesced stores).
//   * Work order: a persistent grid of one workgroup per CU where the items
//     allow it, XCD-aware, pairing heavy and light causal tiles; packed
//     sequences in a listed order located eight rounds at a time.
#include <type_traits>

#include "attn_common.h"
#include "attn_internal.h"

namespace attn {

namespace {

constexpr float kSumCap = 256.0f;  // 2^8: bound on a lane's share of a tile row sum
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
// sequences a varlen call may have for the persistent (listed) order
constexpr int kMaxListedSeqs = 1024;

// one varlen item of the persistent order, as passed between waves through
// LDS (state 0: an item, 1: padding, 2: the rounds are over)
struct ListedItem {
  int64_t q0, kv0, lse0;
  int tile, len, state;
  float sink;
};

#ifndef ATTN_PP_PRIO
#define ATTN_PP_PRIO 2
#endif
#ifndef ATTN_PP_PF
#define ATTN_PP_PF 2
#endif
#ifndef ATTN_PP_AHEAD
#define ATTN_PP_AHEAD 3
#endif

// LOCAL: the sliding-window / sink variant (causal only); off, the kernel is
// compiled without any of its code.  BSHD: [B, S, H, d] tensors (row
// strides H d and Hkv d, known at run time); off, rows are d apart and every
// stride is a compile-time constant, as the address arithmetic of the
// loaders is cheapest that way.
template <int D, bool CAUSAL, bool VARLEN, bool LOCAL, bool BSHD>
__global__ __launch_bounds__(512, 2) void prefill_pp_kernel(const Params p) {
  static_assert(CAUSAL || !LOCAL, "windows and sinks are causal");
  constexpr int BN = D == 128 ? 64 : 128;  // keys per tile: 16 + 16 MFMAs per matrix phase
  constexpr int NW = 8;
  constexpr int BM = 32 * NW;              // 256
  constexpr int NT = 64 * NW;              // 512 threads
  constexpr int ROWB = D * 2;              // bytes per K/V row
  constexpr int TILE_KV = BN * ROWB;       // one K or V tile, 16 KB
  constexpr int STAGE_B = 2 * TILE_KV;     // K then V
  constexpr int PF = ATTN_PP_PF;           // tiles fetched ahead
  constexpr int STAGES = PF + 2;
  constexpr int NKB = BN / 32;             // 32-key blocks of a tile
  constexpr int NDB = D / 32;              // 32-column blocks of d
  constexpr int NDC = D / 16;              // 16-column chunks of d
  constexpr int NKC = BN / 16;             // 16-key chunks of a tile
  constexpr int NPV = NKC * NDB;           // P~V MFMAs per tile
  constexpr int NQK = NDC * NKB;           // QK^T MFMAs per tile
  static_assert(NPV == NQK, "the fused matrix phase pairs one P~V and one QK^T MFMA");
  static_assert(NT == 512 && NDC * NKB == 16 && NKC * NDB == 16, "the loader gives each wave four 1 KB blocks");

  __shared__ __attribute__((aligned(16))) unsigned char smem[STAGES * STAGE_B];
  __shared__ int seq_tiles[kMaxListedSeqs];  // varlen persistent order: query tiles per sequence
  __shared__ ListedItem item_tab[NW];         // varlen persistent order: the items of NW rounds

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave >> 2;               // 0: group A, 1: group B (one slot behind)
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const float sl2 = p.scale_log2;

  // ---- one work item: query tile `tile` of a sequence of sq query rows
  // and skv keys (causal offset off).  Row 0 of its queries (and outputs)
  // is element q_el of q (o), row 0 of its keys and values element kv_el of
  // k and v; rows are p.q_rs and p.kv_rs elements apart.  Its LSE rows
  // start at lse_row.
  auto work = [&](const int tile_a, const int sq_a, const int skv_a, const int off_a, const int64_t q_el_a,
                  const int64_t kv_el_a, const int64_t lse_row_a, const float sink_l2) {
  // the arguments are wave-uniform; readfirstlane lets the compiler keep them
  // (and the load descriptors built from them) in scalar registers
  const int tile = __builtin_amdgcn_readfirstlane(tile_a);
  const int sq = __builtin_amdgcn_readfirstlane(sq_a);
  const int skv = __builtin_amdgcn_readfirstlane(skv_a);
  const int off = __builtin_amdgcn_readfirstlane(off_a);
  const int64_t q_el = uniform64(q_el_a);
  const int64_t kv_el = uniform64(kv_el_a);
  const int64_t lse_row = uniform64(lse_row_a);
  const int q_rs = BSHD ? __builtin_amdgcn_readfirstlane(p.q_rs) : D;
  const int kv_rs = BSHD ? __builtin_amdgcn_readfirstlane(p.kv_rs) : D;
  const int kv_rsb = 2 * kv_rs;  // bytes between key (value) rows
  const __bf16* __restrict__ Q = (const __bf16*)p.q + q_el;
  const __bf16* __restrict__ K = (const __bf16*)p.k + kv_el;
  const __bf16* __restrict__ V = (const __bf16*)p.v + kv_el;
  __bf16* __restrict__ O = (__bf16*)p.o + q_el;

  const int q0 = tile * BM;
  // the two waves on a SIMD take the two 32-row halves of one 64-row block,
  // so under a causal mask they end on the same key tile
  const int qw0 = q0 + 64 * (wave & 3) + 32 * grp;
  const int qrow = qw0 + l32;

  // ---- Q fragments (B operand of S^T = K Q^T): row qrow, d = 16c + 8hh + j
  bf16x8 qf[NDC];
  if (qrow < sq) {
#pragma unroll
    for (int c = 0; c < NDC; ++c) qf[c] = *(const bf16x8*)(Q + (int64_t)qrow * q_rs + 16 * c + 8 * hh);
  } else {
#pragma unroll
    for (int c = 0; c < NDC; ++c) qf[c] = bf16x8{};
  }

  // ---- key ranges.  Tiles are numbered from key 0; the workgroup loads
  // tiles t_first .. nt-1 (relative tile u is absolute tile t_first + u) and
  // this wave computes tiles w_first .. nw-1.
  const int W = LOCAL ? p.window : 0;
  const int q_hi = q0 + BM < sq ? q0 + BM : sq;
  const int kv_end = CAUSAL ? causal_kv_end(q_hi, off, skv) : skv;
  const int nt = ceil_div(kv_end, BN);
  // first key visible to row i under a window: i + off - W + 1
  auto win_lo = [&](const int i) {
    const long b = (long)i + off - W + 1;
    return b < 0 ? 0 : (b > skv ? skv : (int)b);
  };
  const int t_first = W > 0 ? (win_lo(q0) < kv_end ? win_lo(q0) : kv_end) / BN : 0;
  const int ntl = nt > t_first ? nt - t_first : 0;
  int w_end = 0, w_first = 0;
  if (qw0 < sq) {
    const int w_hi = qw0 + 32 < sq ? qw0 + 32 : sq;
    w_end = CAUSAL ? causal_kv_end(w_hi, off, skv) : skv;
    if (W > 0) w_first = win_lo(qw0) / BN;
  }
  const int nw = ceil_div(w_end, BN);
  // relative tile u is computed by this wave
  auto computes = [&](const int u) { return u >= 0 && t_first + u >= w_first && t_first + u < nw; };
  // Rows that see at most 64 keys in all (the first rows of a causal
  // sequence, short key sets) put their whole weight on a few P~ values, and
  // rounding those to bf16 for the P~V product can move O by a few
  // thousandths; with the output's own bf16 rounding that can pass 1e-2.
  // For the first key tile, which holds all of such rows' keys, the vector
  // phase runs the P~V product itself, split: P~ = hi + lo with hi =
  // bf16(P~) (the usual operand) and lo = bf16(P~ - hi), two MFMAs per step,
  // so the numerator carries P~ to about 2^-16; the next matrix phase then
  // skips that tile's product.  Only the first key tile of a sequence's
  // first query tile takes this path (the window variant keeps the plain
  // product).
  const bool few_keys = !LOCAL && (CAUSAL ? (qw0 + off + 1 <= 64) : (skv <= 64));
  auto precise = [&](const int u) { return few_keys && t_first + u == 0; };
  // keys < lim (and >= lo under a window) are visible to this lane's row;
  // kept as lim - 4hh and lo - 4hh so that the per-register key offset they
  // are compared with stays wave-uniform
  int lim = skv;
  if (CAUSAL) {
    const int c_lim = qrow + off + 1;
    lim = c_lim < lim ? c_lim : lim;
  }
  const int lim_h = lim - 4 * hh;
  const int lo_h = (W > 0 ? qrow + off - W + 1 : -(1 << 30)) - 4 * hh;

  // ---- HBM -> LDS in MFMA fragment order, no registers on the way (keys
  // past skv arrive as zeros).  K block j = (d/16) kbi + c (1 KB): lane L
  // holds K[32 kbi + L%32][16c + 8(L/32) ..+8].  V block j = (d/32) kc + db
  // (1 KB) = two transposed-read blocks e = L/32 of 512 B: lane L holds
  // V[16kc + 8e + 4(g>>1) + (L%8)/2][32db + 16(g&1) + 8(L%2) ..+8], g = (L%32)/8.
  // Waves 0-3 load the K blocks 4w .. 4w+3, waves 4-7 the V blocks
  // 4(w-4) .. +3: every wave reads whole 128-byte lines.
  const int k_lane_g = l32 * kv_rsb + hh * 16;
  const int vg = l32 >> 3;
  const int v_lane_g = (8 * hh + 4 * (vg >> 1) + ((lane & 7) >> 1)) * kv_rsb + (16 * (vg & 1) + 8 * (lane & 1)) * 2;
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  auto load_tile = [&](int u) {
    const int k0 = (t_first + u) * BN;
    const int nrows = skv - k0 < BN ? skv - k0 : BN;
    // the descriptor ends right after row nrows-1: rows past it (and their
    // neighbours' bytes in a strided layout) read as zeros
    const int span = (nrows - 1) * kv_rsb + ROWB;
    const unsigned st = lds_u32(smem) + (u % STAGES) * STAGE_B;
    if (wu < 4) {
      const __amdgpu_buffer_rsrc_t r = uniform_rsrc(K + (int64_t)k0 * kv_rs, span);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * wu + i, kbi = j / NDC, c = j % NDC;
        load_lds16(r, k_lane_g, kbi * 32 * kv_rsb + c * 32, st + j * 1024);
      }
    } else {
      const __amdgpu_buffer_rsrc_t r = uniform_rsrc(V + (int64_t)k0 * kv_rs, span);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * (wu - 4) + i, kc = j / NDB, db = j % NDB;
        load_lds16(r, v_lane_g, kc * 16 * kv_rsb + db * 64, st + TILE_KV + j * 1024);
      }
    }
  };

  // per-lane LDS read offsets: fragment blocks are read whole, lane L at 16L
  // (K, ds_read_b128) or 8L (V, two ds_read_b64_tr_b16 per fragment)
  const int k_lane = lane * 16;
  const int v_lane = TILE_KV + lane * 8;

  // ---- state
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_used = -INFINITY;  // reference max (raw score units)
  float neg_ms = 0.0f;       // -m_used * scale_log2 (0 while no key seen)
  float l_part = 0.0f;       // this lane's share of the denominator
  f32x16 s[NKB];             // S^T of the current tile
  bf16x8 pb[NKC];            // P~ of the tile waiting for its P~V product

  // ---- prologue: tiles 0 and 1
  for (int u = 0; u < PF; ++u)
    if (u < ntl) load_tile(u);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // The two phases of a slot for tile t (relative index): matrix = P~V of
  // tile t-1 and S^T of tile t, vector = mask, exponentials and row sums of
  // tile t.
  //
  // Matrix phase inside an item: both products, unconditionally (a wave
  // that did not compute tile t-1 holds P~ = 0, so its product adds nothing;
  // an S^T of a tile it does not compute is never read).
  auto matrix_steady = [&](const int t) {
    // the matrix phase issues first on this SIMD; the other group's
    // vector work fills the issue slots the MFMAs leave free
    __builtin_amdgcn_s_setprio(ATTN_PP_PRIO);
    const unsigned char* vb = smem + ((t + STAGES - 1) % STAGES) * STAGE_B + v_lane;
    const unsigned char* kb = smem + (t % STAGES) * STAGE_B + k_lane;
    // fragment (c, kbi) of K and (kc, db) of V, block offsets as immediates
    auto vfrag = [&](int kc, int db) {
      const unsigned char* a = vb + (NDB * kc + db) * 1024;
      return join_tr(lds_read_tr16(a), lds_read_tr16(a + 512));
    };
    auto kfrag = [&](int c, int kbi) { return *(const bf16x8*)(kb + (NDC * kbi + c) * 1024); };
    // the 16 P~V and 16 QK^T MFMAs are independent, so they are issued
    // alternately, each with its operand read a few MFMAs ahead
    {
      if constexpr (LOCAL || BSHD || D == 64) {
        // The same order written out MFMA pair by MFMA pair, each operand
        // read AHEAD pairs earlier into a register ring, and fenced with
        // sched_barrier.  In these instantiations the scheduler drops the
        // sched_group_barrier pins below in some or all matrix phases: every
        // MFMA then takes its operand from the same four registers and
        // waits for lgkmcnt(0) (window variant 23-29 % slower, BSHD 9-18 %).
        // In the BHSD d = 128 instantiations the pins hold, and there they
        // are about 1 % faster than this form.
        constexpr int AH = ATTN_PP_AHEAD;
        constexpr int R = AH + 1;
        bf16x8 vr[R], kr[R];
#pragma unroll
        for (int kbi = 0; kbi < NKB; ++kbi) s[kbi] = f32x16{};
        static_for<AH>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          vr[i] = vfrag(i / NDB, i % NDB);
          kr[i] = kfrag(i / NKB, i % NKB);
        });
        static_for<NPV>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          constexpr int kc = i / NDB, db = i % NDB;
          oacc[db] = mfma32(vr[i % R], pb[kc], oacc[db]);
          if constexpr (i + AH < NPV) vr[(i + AH) % R] = vfrag((i + AH) / NDB, (i + AH) % NDB);
          constexpr int c = i / NKB, kbi = i % NKB;
          s[kbi] = mfma32(kr[i % R], qf[c], s[kbi]);
          if constexpr (i + AH < NPV) kr[(i + AH) % R] = kfrag((i + AH) / NKB, (i + AH) % NKB);
          __builtin_amdgcn_sched_barrier(0);
        });
      } else {
        // (order pinned with sched_group_barrier: 0x100 LDS read, 0x008
        // MFMA)
#pragma unroll
        for (int kbi = 0; kbi < NKB; ++kbi) s[kbi] = f32x16{};
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
          const int kc = i / NDB, db = i % NDB;
          oacc[db] = mfma32(vfrag(kc, db), pb[kc], oacc[db]);
          const int c = i / NKB, kbi = i % NKB;
          s[kbi] = mfma32(kfrag(c, kbi), qf[c], s[kbi]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 3 * ATTN_PP_AHEAD, 0);
#pragma unroll
        for (int i = 0; i < NPV - ATTN_PP_AHEAD; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * ATTN_PP_AHEAD, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // First and last matrix phases of an item (S^T of tile 0 only, P~V of the
  // last tile only), each as the wave computes it; the operand reads of one
  // step are double buffered in registers, in flight during the MFMAs of the
  // step before.
  auto matrix_edge = [&](const int t, const bool do_pv, const bool do_qk) {
    // the matrix phase issues first on this SIMD; the other group's
    // vector work fills the issue slots the MFMAs leave free
    __builtin_amdgcn_s_setprio(ATTN_PP_PRIO);
    const unsigned char* vb = smem + ((t + STAGES - 1) % STAGES) * STAGE_B + v_lane;
    const unsigned char* kb = smem + (t % STAGES) * STAGE_B + k_lane;
    // fragment (c, kbi) of K and (kc, db) of V, block offsets as immediates
    auto vfrag = [&](int kc, int db) {
      const unsigned char* a = vb + (NDB * kc + db) * 1024;
      return join_tr(lds_read_tr16(a), lds_read_tr16(a + 512));
    };
    auto kfrag = [&](int c, int kbi) { return *(const bf16x8*)(kb + (NDC * kbi + c) * 1024); };
    {
    bf16x8 kf[2][NKB];
    if (do_pv) {
      bf16x8 vf[2][NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) vf[0][db] = vfrag(0, db);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        if (kc + 1 < NKC) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) vf[(kc + 1) & 1][db] = vfrag(kc + 1, db);
        } else if (do_qk) {
#pragma unroll
          for (int kbi = 0; kbi < NKB; ++kbi) kf[0][kbi] = kfrag(0, kbi);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(vf[kc & 1][db], pb[kc], oacc[db]);
      }
    } else if (do_qk) {
#pragma unroll
      for (int kbi = 0; kbi < NKB; ++kbi) kf[0][kbi] = kfrag(0, kbi);
    }
    if (do_qk) {
#pragma unroll
      for (int kbi = 0; kbi < NKB; ++kbi) s[kbi] = f32x16{};
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        if (c + 1 < NDC) {
#pragma unroll
          for (int kbi = 0; kbi < NKB; ++kbi) kf[(c + 1) & 1][kbi] = kfrag(c + 1, kbi);
        }
#pragma unroll
        for (int kbi = 0; kbi < NKB; ++kbi) s[kbi] = mfma32(kf[c & 1][kbi], qf[c], s[kbi]);
      }
    }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // Vector phase of tile t.  steady: a tile the wave computes whole (no key
  // masked for any of its rows) and that is not the split tile, so no
  // per-tile check is made; given as std::true_type / std::false_type or as
  // a run-time bool.
  auto vector_phase = [&](const int t, auto steady_c) {
    bool steady;
    if constexpr (std::is_same_v<decltype(steady_c), bool>) {
      steady = steady_c;
    } else {
      steady = decltype(steady_c)::value;
    }
    const int k0 = (t_first + t) * BN;
    bool partial = false;
    if (!steady)
      partial = __builtin_amdgcn_readfirstlane((int)((k0 + BN > skv) || (CAUSAL && (k0 + BN - 1 > qw0 + off)) ||
                                                     (W > 0 && k0 < qw0 + 31 + off - W + 1))) != 0;
    // 16-key chunk kc holds keys k0 + 16kc .. +15 (registers 8(kc%2) ..
    // +7 of S block kc/2).  At d = 64 (128-key tiles), chunks from `live` on
    // lie past the last key any row of this wave sees: they get no mask, no
    // exponentials and P~ = 0 (a wave-uniform bound, so the tests on it are
    // scalar branches; 8 % at d = 64, while at d = 128 the extra live
    // ranges cost registers and up to 2 %, so there every chunk is live)
    int live = NKC;
    if (partial) {
      if constexpr (D == 64) {
        int e = skv;
        if (CAUSAL) e = e < qw0 + 32 + off ? e : qw0 + 32 + off;
        const int n = (e - k0 + 15) >> 4;
        live = __builtin_amdgcn_readfirstlane(n < 0 ? 0 : (n > NKC ? NKC : n));
      }
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        if (kc >= live) continue;
        const int kbi = kc >> 1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {  // key = k0 + 32kbi + 8(r/4) + 4hh + r%4
          const int r = 8 * (kc & 1) + j;
          const int kk = k0 + 32 * kbi + 8 * (r >> 2) + (r & 3);
          if (kk >= lim_h || (LOCAL && kk < lo_h)) s[kbi][r] = -INFINITY;
        }
      }
    }
    // P~ against the current reference, S kept; this lane's share of the
    // row sum as four independent chains
    auto expo = [&]() {
      float rp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        if (kc >= live) {
          pb[kc] = bf16x8{};
          continue;
        }
        const f32x16& sk = s[kc >> 1];
        const int rb = 8 * (kc & 1);
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          e[j] = fast_exp2(fmaf(sk[rb + j], sl2, neg_ms));
          rp[j & 3] += e[j];
        }
        pb[kc] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      }
      return (rp[0] + rp[1]) + (rp[2] + rp[3]);
    };
    // A share above 2^8 means some P~ above 2^8, and a row without a
    // reference has no P~ yet: then the exact reference update, and P~
    // again.  At d = 64 a wave whose rows have no reference yet (its first
    // tile) goes to the update directly instead of discarding a first P~
    // (2 % there; at d = 128 the extra branch costs registers and 2-10 %).
    float ps = 0.0f;
    bool exact = __any(m_used == -INFINITY);
    if (D == 128 || !exact) {
      ps = expo();
      exact = __any(ps > kSumCap || m_used == -INFINITY);
    }
    if (exact) {
      float mp[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        if (kc >= live) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) mp[j & 3] = fmaxf(mp[j & 3], s[kc >> 1][8 * (kc & 1) + j]);
      }
      const float mx = pair32_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3])));
      const float m_new = fmaxf(m_used, mx);
      const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2((m_used - m_new) * sl2);
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_used = m_new;
      neg_ms = (m_used == -INFINITY) ? 0.0f : -m_used * sl2;
      ps = expo();
    }
    l_part += ps;
    bool split = false;
    if (!steady) split = __builtin_amdgcn_readfirstlane((int)precise(t)) != 0;
    if (split) {
      // the split P~V product of this tile (V of tile t is in stage
      // t % STAGES); the fp32 P~ is recomputed with expo()'s
      // instructions, so its bf16 part is pb exactly
      const unsigned char* vb = smem + (t % STAGES) * STAGE_B + v_lane;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        if (kc >= live) continue;
        const f32x16& sk = s[kc >> 1];
        const int rb = 8 * (kc & 1);
        float lo[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) lo[j] = fast_exp2(fmaf(sk[rb + j], sl2, neg_ms)) - (float)pb[kc][j];
        const bf16x8 pl = to_bf16x8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const unsigned char* a = vb + (NDB * kc + db) * 1024;
          const bf16x8 vf = join_tr(lds_read_tr16(a), lds_read_tr16(a + 512));
          oacc[db] = mfma32(vf, pb[kc], oacc[db]);
          oacc[db] = mfma32(vf, pl, oacc[db]);
        }
      }
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) pb[kc] = bf16x8{};
    }
  };
  // end of slot 2k+1: tile k+1 must have landed before slot 2k+2 reads it;
  // the four loads of each of tiles k+2 .. k+PF may still be in flight
  // (s_waitcnt immediate: expcnt and lgkmcnt at their maxima, vmcnt in the
  // low four bits)
  auto wait_tile = [&](const int k) {
    const int newer = (ntl - 1 < k + PF ? ntl - 1 : k + PF) - (k + 1);
    if (PF >= 3 && newer >= 2) {
      __builtin_amdgcn_s_waitcnt(0x0F78);
    } else if (newer >= 1) {
      __builtin_amdgcn_s_waitcnt(0x0F74);
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
  };

  // The tiles [st_lo, st_hi) (relative) are steady for this wave: computed,
  // with no key masked for any of its rows (before the causal diagonal of
  // its first row, after the window's lower edge for its last row, inside
  // the keys), and not the split tile.  Masks are monotone in the tile
  // index, so the steady tiles form one range.
  auto fdiv = [](const int a, const int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); };
  int st_lo = w_first - t_first;
  int st_hi = nw - t_first;
  st_hi = st_hi < skv / BN - t_first ? st_hi : skv / BN - t_first;                  // key tail
  if (CAUSAL) {
    const int d = fdiv(qw0 + off + 1, BN) - t_first;                                // diagonal
    st_hi = st_hi < d ? st_hi : d;
  }
  if (W > 0) {
    const int e = -fdiv(-(qw0 + off + 32 - W), BN) - t_first;                       // window edge
    st_lo = st_lo > e ? st_lo : e;
  }
  if (few_keys && t_first == 0) st_lo = st_lo > 1 ? st_lo : 1;                      // split tile
  st_lo = __builtin_amdgcn_readfirstlane(st_lo);
  st_hi = __builtin_amdgcn_readfirstlane(st_hi);
  // the vector phase of tile t, or P~ = 0 for a tile this wave does not
  // compute (the next matrix phase then adds nothing for it)
  auto vector_or_zero = [&](const int t) {
    if constexpr (D == 64 || LOCAL) {
      // one copy of the vector phase for both kinds of tile (two copies
      // spill in these instantiations)
      const bool steady = t >= st_lo && t < st_hi;
      bool comp = steady;
      if (!steady) comp = __builtin_amdgcn_readfirstlane((int)computes(t)) != 0;
      if (comp) {
        vector_phase(t, steady);
      } else {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) pb[kc] = bf16x8{};
      }
    } else {
      if (__builtin_amdgcn_readfirstlane((int)computes(t)) != 0) {
        vector_phase(t, std::false_type{});
      } else {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) pb[kc] = bf16x8{};
      }
    }
  };
  auto pv_last = [&](const int t) { return computes(t) && !precise(t); };
  // Slots 0 .. 2 ntl + 1, one barrier each.  Group A: matrix phase of tile t
  // in slot 2t, vector phase in slot 2t+1; group B one slot behind.  Tile
  // u = k + PF is fetched into the stage of tile k + PF - STAGES, whose last
  // read (its V, by group B) was in slot 2k-1: its V blocks by group B in
  // slot 2k, its K blocks by group A in slot 2k+1, in both cases at the
  // start of the loading group's vector phase.  (Loads issued by a wave that
  // is about to run its matrix phase delay that phase's MFMAs, and a burst
  // from all eight waves at once delays both phases: measured.)  Each group
  // runs its own copy of the slot sequence.
  //
  // one slot pair of each group; steady: a tile of [st_lo, st_hi), where the
  // vector phase makes no per-tile check
  auto pair_a = [&](const int t, auto steady_c) {
    if (t + PF < ntl) load_tile(t + PF);
    if constexpr (decltype(steady_c)::value) {
      vector_phase(t, std::true_type{});
    } else {
      vector_or_zero(t);
    }
    wait_tile(t);
    __syncthreads();
    // causal: outside the steady range, a wave with neither tile t nor t+1
    // to compute (past its rows' diagonal) skips the products (P~ = 0, S
    // unused): no time inside the slot, but less power, and the clock is
    // power-limited (the non-causal instantiations keep the unconditional
    // form, which measured 0.5 % faster there)
    if constexpr (decltype(steady_c)::value || !(VARLEN || CAUSAL)) {
      matrix_steady(t + 1);
    } else if (__builtin_amdgcn_readfirstlane((int)(computes(t) || computes(t + 1))) != 0) {
      matrix_steady(t + 1);
    }
    __syncthreads();
  };
  auto pair_b = [&](const int t, auto steady_c) {
    if constexpr (decltype(steady_c)::value || !(VARLEN || CAUSAL)) {
      matrix_steady(t);
    } else if (__builtin_amdgcn_readfirstlane((int)(computes(t - 1) || computes(t))) != 0) {
      matrix_steady(t);
    }
    wait_tile(t);
    __syncthreads();
    if (t + 1 + PF < ntl) load_tile(t + 1 + PF);
    if constexpr (decltype(steady_c)::value) {
      vector_phase(t, std::true_type{});
    } else {
      vector_or_zero(t);
    }
    __syncthreads();
  };
  if constexpr (D == 64 || LOCAL) {
    // one loop per group; the steady test is made per tile (split loops
    // spill registers in these instantiations)
    if (__builtin_amdgcn_readfirstlane(grp) == 0) {
      matrix_edge(0, false, computes(0));
      __syncthreads();
      for (int t = 0; t + 1 < ntl; ++t) {
        if (t + PF < ntl) load_tile(t + PF);
        vector_or_zero(t);
        wait_tile(t);
        __syncthreads();
        matrix_steady(t + 1);
        __syncthreads();
      }
      if (ntl > 0) {
        vector_or_zero(ntl - 1);
        wait_tile(ntl - 1);
        __syncthreads();
        matrix_edge(ntl, pv_last(ntl - 1), false);
        __syncthreads();
      }
      __syncthreads();
    } else {
      if (PF < ntl) load_tile(PF);
      __syncthreads();
      if (ntl > 0) {
        matrix_edge(0, false, computes(0));
        wait_tile(0);
        __syncthreads();
        if (1 + PF < ntl) load_tile(1 + PF);
        vector_or_zero(0);
        __syncthreads();
        for (int t = 1; t < ntl; ++t) {
          matrix_steady(t);
          wait_tile(t);
          __syncthreads();
          if (t + 1 + PF < ntl) load_tile(t + 1 + PF);
          vector_or_zero(t);
          __syncthreads();
        }
      }
      matrix_edge(ntl, ntl > 0 && pv_last(ntl - 1), false);
      __syncthreads();
    }
  } else {
    if (__builtin_amdgcn_readfirstlane(grp) == 0) {
      matrix_edge(0, false, computes(0));
      __syncthreads();
      // t in [0, ntl - 1): before, inside and after the steady range
      const int e = ntl - 1;
      const int a = st_lo < 0 ? 0 : (st_lo > e ? (e > 0 ? e : 0) : st_lo);
      const int b = st_hi < a ? a : (st_hi > e ? (e > a ? e : a) : st_hi);
      int t = 0;
      for (; t < a; ++t) pair_a(t, std::false_type{});
      for (; t < b; ++t) pair_a(t, std::true_type{});
      for (; t < e; ++t) pair_a(t, std::false_type{});
      if (ntl > 0) {
        vector_or_zero(ntl - 1);
        wait_tile(ntl - 1);
        __syncthreads();
        matrix_edge(ntl, pv_last(ntl - 1), false);
        __syncthreads();
      }
      __syncthreads();
    } else {
      if (PF < ntl) load_tile(PF);
      __syncthreads();
      if (ntl > 0) {
        matrix_edge(0, false, computes(0));
        wait_tile(0);
        __syncthreads();
        if (1 + PF < ntl) load_tile(1 + PF);
        vector_or_zero(0);
        __syncthreads();
        // t in [1, ntl)
        const int a = st_lo < 1 ? 1 : (st_lo > ntl ? ntl : st_lo);
        const int b = st_hi < a ? a : (st_hi > ntl ? ntl : st_hi);
        int t = 1;
        for (; t < a; ++t) pair_b(t, std::false_type{});
        for (; t < b; ++t) pair_b(t, std::true_type{});
        for (; t < ntl; ++t) pair_b(t, std::false_type{});
      }
      matrix_edge(ntl, ntl > 0 && pv_last(ntl - 1), false);
      __syncthreads();
    }
  }

  // ---- epilogue: O = acc / l (0 for rows that saw no key), LSE natural
  // log.  With a sink, acc and l are first brought to the reference
  // m* = max(m scale', sink) and the sink's term is added to l.
  float l = pair32_sum(l_part);
  float ref_l2 = m_used * sl2;  // log2 of the reference the sums are relative to
  float o_mul = 1.0f;
  if (LOCAL && sink_l2 > -INFINITY) {
    const float ms = fmaxf(m_used == -INFINITY ? -INFINITY : ref_l2, sink_l2);
    o_mul = m_used == -INFINITY ? 0.0f : fast_exp2(ref_l2 - ms);
    l = l * o_mul + fast_exp2(sink_l2 - ms);
    ref_l2 = ms;
  }
  // O goes through LDS (the ring is free once the last slot's barrier has
  // passed, and the next item's first loads come after the barrier that
  // ends this item) so that the stores to HBM are whole rows: a lane holds
  // 4-value pieces of one row, so a direct store instruction writes 16 bytes
  // in each of 32 rows; from LDS it writes 1 KB of consecutive rows.  Rows
  // are padded by 16 bytes, which spreads the 32 rows of a write over the
  // banks (two ways) and keeps every offset within a row an immediate.
  {
    constexpr int PROW = ROWB + 16;  // padded row
    static_assert(BM * PROW <= STAGES * STAGE_B, "the output tile fits the ring");
    const float inv = (qrow < sq && l > 0.0f) ? o_mul / l : 0.0f;
    unsigned char* wrow = smem + (qw0 - q0 + l32) * PROW + 8 * hh;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 w;
        w[0] = (__bf16)(oacc[db][4 * rg + 0] * inv);
        w[1] = (__bf16)(oacc[db][4 * rg + 1] * inv);
        w[2] = (__bf16)(oacc[db][4 * rg + 2] * inv);
        w[3] = (__bf16)(oacc[db][4 * rg + 3] * inv);
        *(bf16x4*)(wrow + 64 * db + 16 * rg) = w;
      }
    __syncthreads();
    constexpr int CH = D / 8;           // 16-byte chunks per row
    constexpr int RPI = 64 / CH;        // rows per store instruction
    constexpr int ROUNDS = BM / (NW * RPI);
#pragma unroll 2
    for (int i = 0; i < ROUNDS; ++i) {
      const int row = (wave * ROUNDS + i) * RPI + lane / CH;
      const int c = lane % CH;
      const u32x4 val = *(const u32x4*)(smem + row * PROW + 16 * c);
      if (q0 + row < sq) *(u32x4*)(O + (int64_t)(q0 + row) * q_rs + 8 * c) = val;
    }
  }
  if (qrow < sq && p.lse != nullptr && hh == 0)
    p.lse[lse_row + qrow] = l > 0.0f ? (ref_l2 + fast_log2(l)) * kLn2 : -INFINITY;
  };

  // ---- scheduling.  Round r of this workgroup names one item through
  // (tile, sq, skv, off, q_el, kv_el, lse_row); the rounds end when item()
  // returns false, and skip == true marks an empty item.
  int a_tile = 0, a_sq = 0, a_skv = 0, a_off = 0;
  int64_t a_q0 = 0, a_kv0 = 0, a_lse0 = 0;
  float a_sink = -INFINITY;  // sink of the item's query head, log2 units
  auto sink_of = [&](const int h) {
    return (LOCAL && p.sinks != nullptr) ? p.sinks[h] * kLog2e : -INFINITY;
  };
  // dense item v: (b, h) major, query tiles of a head heaviest first under
  // a causal mask
  auto dense_at = [&](const int v) {
    int b, h;
    dense_item(v, p.tiles_per_head, p.H, CAUSAL, b, h, a_tile);
    a_sq = p.Sq;
    a_skv = p.Skv;
    a_off = p.Skv - p.Sq;
    const int kvh = h / p.group;
    const int bh = b * p.H + h;
    if constexpr (BSHD) {  // [B, S, H, d]
      a_q0 = ((int64_t)b * p.Sq * p.H + h) * D;
      a_kv0 = ((int64_t)b * p.Skv * p.Hkv + kvh) * D;
    } else {       // [B, H, S, d]
      a_q0 = (int64_t)bh * p.Sq * D;
      a_kv0 = ((int64_t)b * p.Hkv + kvh) * p.Skv * D;
    }
    a_lse0 = (int64_t)bh * p.Sq;
    a_sink = sink_of(h);
  };
  // query tile `tile` of head h in varlen sequence bb
  auto seq_item = [&](const int h, const int bb, const int tile) {
    int s0, s1;
    seq_bounds(p.cu, p.Sq, bb, s0, s1);
    a_tile = tile;
    a_sq = a_skv = s1 - s0;
    a_off = 0;
    const int kvh = h / p.group;
    if constexpr (BSHD) {  // [T, H, d]
      a_q0 = ((int64_t)s0 * p.H + h) * D;
      a_kv0 = ((int64_t)s0 * p.Hkv + kvh) * D;
    } else {       // [1, H, T, d]
      a_q0 = ((int64_t)h * p.Sq + s0) * D;
      a_kv0 = ((int64_t)kvh * p.Sq + s0) * D;
    }
    a_lse0 = (int64_t)h * p.Sq + s0;
    a_sink = sink_of(h);
  };
  // dispatched varlen item v (h major, then the concatenated tiles of the
  // sequences, last first under a causal mask); false past the last tile
  auto varlen_at = [&](const int v) {
    int h, bb, tile;
    if (!varlen_item(p.cu, p.B, p.Sq, BM, p.tiles_per_head, CAUSAL, v, h, bb, tile)) return false;
    seq_item(h, bb, tile);
    return true;
  };
  // varlen persistent order: XCD x takes the heads [x H/8, (x+1) H/8) (the
  // query heads of one KV head stay on one L2); its items (sequence, tile,
  // head) are listed by tile index, highest first (under a causal mask the
  // cost of a tile grows with its index), then sequence, then head.  The
  // tiles per sequence are staged in LDS once; cum(t), the number of listed
  // items with tile index >= t, is (H/8) sum_i max(0, tiles_i - t).
  const int hpx = p.H / 8;
  int v_tmax = 0;
  int64_t v_items = 0;
  auto wave_sum = [&](int x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
  };
  auto wave_max = [&](int x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const int y = __shfl_xor(x, m, 64);
      x = y > x ? y : x;
    }
    return x;
  };
  auto tiles_at_or_above = [&](const int t) {  // sum_i max(0, tiles_i - t)
    int acc = 0;
    for (int i = lane; i < p.B; i += 64) {
      const int n = seq_tiles[i] - t;
      acc += n > 0 ? n : 0;
    }
    return wave_sum(acc);
  };
  if (VARLEN && p.persist_c > 0) {
    for (int i = tid; i < p.B; i += NT) {
      int s0, s1;
      seq_bounds(p.cu, p.Sq, i, s0, s1);
      seq_tiles[i] = ceil_div(s1 - s0, BM);
    }
    __syncthreads();
    int mx = 0;
    for (int i = lane; i < p.B; i += 64) mx = seq_tiles[i] > mx ? seq_tiles[i] : mx;
    v_tmax = wave_max(mx);
    v_items = (int64_t)tiles_at_or_above(0) * hpx;
  }
  // the items of XCD x's list (attn_sched.h, listed_locate): cum(t) from
  // the staged tile counts, the rank-th sequence with more than t tiles by a
  // ballot over 64 sequences at a time
  auto listed_at = [&](const int64_t f, const int x) {
    auto cum = [&](const int t) { return (int64_t)tiles_at_or_above(t) * hpx; };
    auto nth = [&](const int t, int rank) {
      for (int i0 = 0; i0 < p.B; i0 += 64) {
        const int i = i0 + lane;
        const int ti = seq_tiles[i < p.B ? i : 0];  // every lane reads inside the array
        uint64_t m = __ballot(i < p.B && ti > t);
        const int n = __popcll(m);
        if (rank < n) {
          for (int k = 0; k < rank; ++k) m &= m - 1;
          return i0 + __builtin_ctzll(m);
        }
        rank -= n;
      }
      return 0;  // not reached for f < cum(0)
    };
    int seq, tile, head;
    listed_locate(f, x, hpx, v_tmax, cum, nth, seq, tile, head);
    seq_item(head, seq, tile);
  };
  // one workgroup per item (persist_c == 0), or a persistent grid of one
  // workgroup per CU (8 XCDs x persist_c).  Persistent workgroups take items
  // in rounds of the grid size, reversing direction every round, so that a
  // heavy causal tile is paired with a light one.  Workgroup g sits on XCD
  // g % 8 and walks that XCD's share of the items.  Dense: the host makes the
  // item count a multiple of the grid.  Varlen: the listed order above; each
  // item is located by a search over the sequences' tile counts (the host
  // enables this only when that search is short and H is a multiple of 8),
  // NW rounds at a time.
  auto item = [&](const int r, bool& skip) {
    skip = false;
    if (p.persist_c == 0) {
      if (r > 0) return false;
      const int v = xcd_remap(blockIdx.x, p.work_items);
      if (v < 0) return false;
      if constexpr (VARLEN) {
        skip = !varlen_at(v);
      } else {
        dense_at(v);
      }
      return true;
    }
    if constexpr (!VARLEN) {
      const int v = persist_dense_item(blockIdx.x, r, p.persist_c, p.work_items);
      if (v < 0) return false;
      dense_at(v);
    } else {
      // NW rounds at a time: wave w locates round r + w (the search is a
      // chain of dependent LDS reads and cross-lane sums, so one wave per
      // round takes it off the critical path), and each round reads its
      // entry back
      if (r % NW == 0) {
        const int64_t f = persist_listed_index(blockIdx.x, r + wave, p.persist_c, v_items);
        ListedItem e;
        e.state = f == -1 ? 2 : (f < 0 ? 1 : 0);
        if (f >= 0) {
          listed_at(f, blockIdx.x % 8);
          e.tile = a_tile;
          e.len = a_sq;
          e.q0 = a_q0;
          e.kv0 = a_kv0;
          e.lse0 = a_lse0;
          e.sink = a_sink;
        }
        if (lane == 0) item_tab[wave] = e;
        __syncthreads();
      }
      const ListedItem e = item_tab[r % NW];
      if (e.state == 2) return false;
      if (e.state == 1) {
        skip = true;
      } else {
        a_tile = e.tile;
        a_sq = a_skv = e.len;
        a_off = 0;
        a_q0 = e.q0;
        a_kv0 = e.kv0;
        a_lse0 = e.lse0;
        a_sink = e.sink;
      }
    }
    return true;
  };
  for (int r = 0;; ++r) {
    bool skip;
    if (!item(r, skip)) break;
    if (!skip) work(a_tile, a_sq, a_skv, a_off, a_q0, a_kv0, a_lse0, a_sink);
    __syncthreads();
  }
}

template <int D, bool CAUSAL, bool VARLEN, bool LOCAL, bool BSHD>
hipError_t launch_one(const Params& p, hipStream_t st) {
  const int grid = p.persist_c > 0 ? 8 * p.persist_c : 8 * ceil_div(p.work_items, 8);
  hipLaunchKernelGGL((prefill_pp_kernel<D, CAUSAL, VARLEN, LOCAL, BSHD>), dim3(grid), dim3(512), 0, st, p);
  return hipGetLastError();
}

template <int D, bool BSHD>
hipError_t launch_dl(const Params& p, hipStream_t st) {
  const bool var = p.cu != nullptr;
  if (p.causal && (p.window > 0 || p.sinks != nullptr))
    return var ? launch_one<D, true, true, true, BSHD>(p, st) : launch_one<D, true, false, true, BSHD>(p, st);
  if (p.causal)
    return var ? launch_one<D, true, true, false, BSHD>(p, st) : launch_one<D, true, false, false, BSHD>(p, st);
  return var ? launch_one<D, false, true, false, BSHD>(p, st) : launch_one<D, false, false, false, BSHD>(p, st);
}

template <int D>
hipError_t launch_d(const Params& p, hipStream_t st) {
  return p.bshd ? launch_dl<D, true>(p, st) : launch_dl<D, false>(p, st);
}

}  // namespace

int prefill_pp_block_m() { return 256; }

hipError_t launch_prefill_pp(const Params& p, hipStream_t st) {
  if (p.work_items <= 0) return hipSuccess;
  if (p.d == 128) return launch_d<128>(p, st);
  if (p.d == 64) return launch_d<64>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
