// Split-KV decode (one query row per head, Sq == 1) for bf16 on gfx950.
//
// Flash-Decoding as the TileLang tutorial chapter 15 describes it (sections
// 4.8 (3) and 5.4): the keys of each (batch, KV head) are cut into
// num_splits contiguous chunks; each chunk yields an output normalised by
// its own denominator and its base-2 log-sum-exp (the page's glse); a second
// kernel combines the chunks with weights l_s / sum l.
//
// gfx950 mapping:
//   * one workgroup per (batch, KV head, split, group of up to 16 query
//     heads); the query heads that share the KV head (grouped-query
//     attention, tutorial section 4.8 (1)) form the 16 columns of
//     v_mfma_f32_16x16x32_bf16, so every K/V byte is read once per split and
//     used by every head of the group;
//   * the four waves stream interleaved 32-key chunks of the split on their
//     own (no workgroup barrier in the loop); K goes from HBM straight into
//     the MFMA A operand, V goes through a per-wave LDS buffer and comes back
//     transposed with ds_read_b64_tr_b16;
//   * the next chunk's loads are in flight while the current chunk is used;
//   * the four waves' (m, l, O) states are merged through LDS in fixed order
//     at the end, so the result is bitwise reproducible.
//
// Paged KV cache (PAGED): the keys of sequence b are read through its block
// table, key t from physical page block_table[b][t / page_size] at offset
// t % page_size (tutorial section 4.8 (2); the CUDA course chapter 12,
// section 12.9.4); the cache is [num_pages, Hkv, page_size, d], so the rows
// of one (page, KV head) are contiguous.  Sequence b has seqlens_k[b] keys and
// its splits are ceil(seqlens_k[b] / num_splits) keys long.  Table entries
// and lengths are clamped into range, so a malformed table gives wrong
// numbers, never an out-of-bounds access.  Nothing else changes: the
// indirection decides where the bytes come from, not what is computed.
//
// Sliding window (tutorial section 5.2): the single query row is the last
// position, so a window of W keys keeps keys Skv - W .. Skv - 1, and the
// splits cut that range.  An attention sink enters in the combine kernel.
#include "attn_common.h"
#include "attn_internal.h"

namespace attn {

namespace {

constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units

template <int D, bool PAGED>
__global__ __launch_bounds__(256, 2) void decode_split_bf16_kernel(const Params p) {
  constexpr int NW = 4;
  constexpr int NDC = D / 32;       // contraction steps of QK^T (32 d each)
  constexpr int NDB = D / 16;       // 16-column blocks of O^T
  constexpr int VB = 32 * D * 2;    // one wave's V staging buffer (32 keys)
  constexpr int SMEM = NW * 2 * VB;
  static_assert(SMEM >= NW * (16 * D + 32) * 4, "merge scratch must fit");
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int kg = lane >> 4;
  const float sl2 = p.scale_log2;

  // ---- work item -> (b, kvh, head group, split)
  const int S = p.num_splits;
  const int HG = ceil_div(p.group, 16);
  int w = blockIdx.x;
  const int s = w % S;
  w /= S;
  const int hgp = w % HG;
  w /= HG;
  const int kvh = w % p.Hkv;
  const int b = w / p.Hkv;

  int skv = p.Skv;
  if constexpr (PAGED) {
    const int cap = p.max_pages << p.page_shift;
    skv = p.seqlens_k[b];
    skv = skv < 0 ? 0 : (skv > cap ? cap : skv);
  }
  // a sliding window of W keys leaves the last W (the query is the last
  // position, so the band ends at the last key)
  const int kv_begin = (p.window > 0 && skv > p.window) ? skv - p.window : 0;
  const int split_len = ceil_div(skv - kv_begin, S);
  const int lo = kv_begin + s * split_len;
  int hi = lo + split_len;
  hi = hi < skv ? hi : skv;
  const int nchunks = hi > lo ? ceil_div(hi - lo, 32) : 0;

  const int hl = hgp * 16 + l16;         // this lane's query head within the group
  const bool qvalid = hl < p.group;
  const int h = kvh * p.group + (qvalid ? hl : 0);

  const __bf16* __restrict__ Q = (const __bf16*)p.q + ((int64_t)b * p.H + h) * D;
  // element offset of key 0 of this (b, KV head) and the row stride: BHSD
  // [B, Hkv, Skv, d] or BSHD [B, Skv, Hkv, d] (the query and output rows of
  // a decode step are laid out alike in both)
  int64_t kv0 = 0;
  if constexpr (!PAGED) {
    kv0 = p.bshd ? ((int64_t)b * p.Skv * p.Hkv + kvh) * D : ((int64_t)b * p.Hkv + kvh) * p.Skv * D;
  }
  const int kv_rs = PAGED ? D : p.kv_rs;
  const __bf16* __restrict__ K = (const __bf16*)p.k + kv0;
  const __bf16* __restrict__ V = (const __bf16*)p.v + kv0;
  const int32_t* __restrict__ table = PAGED ? p.block_table + (int64_t)b * p.max_pages : nullptr;
  // row of key `key` (< skv) relative to K and V
  auto key_row = [&](const int key) -> int64_t {
    if constexpr (PAGED) {
      int page = table[key >> p.page_shift];
      page = page < 0 ? 0 : (page >= p.num_pages ? p.num_pages - 1 : page);
      return (((int64_t)page * p.Hkv + kvh) << p.page_shift) + (key & ((1 << p.page_shift) - 1));
    } else {
      return key;
    }
  };

  // Q^T as the B operand: column l16 = head, d = 32c + 8kg + j
  bf16x8 qf[NDC];
#pragma unroll
  for (int c = 0; c < NDC; ++c)
    qf[c] = qvalid ? *(const bf16x8*)(Q + 32 * c + 8 * kg) : bf16x8{};

  // registers of one 32-key chunk: rows 16kb + l16, d = 32c + 8kg + j
  u32x4 kc_[2][NDC], vc_[2][NDC];
  u32x4 kn_[2][NDC], vn_[2][NDC];
  auto gload = [&](int ci, u32x4 (&kr)[2][NDC], u32x4 (&vr)[2][NDC]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      int key = lo + 32 * ci + 16 * kb + l16;
      key = key < hi ? key : hi - 1;
      const int64_t row = key_row(key);
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        kr[kb][c] = *(const u32x4*)(K + row * kv_rs + 32 * c + 8 * kg);
        vr[kb][c] = *(const u32x4*)(V + row * kv_rs + 32 * c + 8 * kg);
      }
    }
  };

  // transposed V read: lane (g, t) addresses row 4g + (t>>2) (+16e),
  // column 16db + 4(t&3); it receives V[4g + 16e + j][16db + t]
  const int vtr_row = 4 * kg + (l16 >> 2);
  const int vtr_col = 4 * (l16 & 3);

  f32x4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{};
  float m_used = -INFINITY, neg_ms = 0.0f, l_part = 0.0f;

  int ci = wave;
  if (ci < nchunks) gload(ci, kc_, vc_);
  int par = 0;
  for (; ci < nchunks; ci += NW) {
    if (ci + NW < nchunks) gload(ci + NW, kn_, vn_);

    // V chunk -> this wave's LDS buffer (row-major, swizzled)
    unsigned char* vb = smem + (wave * 2 + par) * VB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < NDC; ++c)
        *(u32x4*)(vb + lds_off<D>(16 * kb + l16, 4 * c + kg)) = vc_[kb][c];

    // S^T = K Q^T: lane holds S[head l16][key 16kb + 4kg + i]
    f32x4 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x4{};
#pragma unroll
      for (int c = 0; c < NDC; ++c)
        sc[kb] = mfma16(__builtin_bit_cast(bf16x8, kc_[kb][c]), qf[c], sc[kb]);
    }
    const int kbase = lo + 32 * ci;
    if (kbase + 32 > hi) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kbase + 16 * kb + 4 * kg + i >= hi) sc[kb][i] = -INFINITY;
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[kb][i]);
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));

    const bool need = (mx > m_used) && ((mx - m_used) * sl2 > kTau);
    if (__any(need)) {
      const float m_new = need ? mx : m_used;
      const float alpha = need ? fast_exp2((m_used - m_new) * sl2) : 1.0f;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[db][i] *= alpha;
      m_used = m_new;
      neg_ms = (m_used == -INFINITY) ? 0.0f : -m_used * sl2;
    }

    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(fmaf(sc[kb][i], sl2, neg_ms));
        sc[kb][i] = e;
        rs += e;
      }
    l_part += rs;
    const bf16x8 pb = to_bf16x8(sc[0][0], sc[0][1], sc[0][2], sc[0][3], sc[1][0], sc[1][1],
                                sc[1][2], sc[1][3]);

    // the wave's LDS writes above must land before its transposed reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int col = 16 * db + vtr_col;
      const s16x4 a0 = lds_read_tr16(vb + lds_off<D>(vtr_row, col >> 3) + (col & 7) * 2);
      const s16x4 a1 = lds_read_tr16(vb + lds_off<D>(vtr_row + 16, col >> 3) + (col & 7) * 2);
      oacc[db] = mfma16(join_tr(a0, a1), pb, oacc[db]);
    }

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        kc_[kb][c] = kn_[kb][c];
        vc_[kb][c] = vn_[kb][c];
      }
    par ^= 1;
  }

  // ---- merge the four waves (fixed order) and write the split partial
  float l = l_part + shfl_xor_f(l_part, 16);
  l += shfl_xor_f(l, 32);
  __syncthreads();  // every wave is done with its V buffers
  float* mo = (float*)smem;                // [NW][D][16] unnormalised O^T
  float* ml = mo + NW * D * 16;            // [NW][16] m
  float* ll = ml + NW * 16;                // [NW][16] l
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) mo[(wave * D + 16 * db + 4 * kg + i) * 16 + l16] = oacc[db][i];
  if (kg == 0) {
    ml[wave * 16 + l16] = m_used;
    ll[wave * 16 + l16] = l;
  }
  __syncthreads();

  // thread -> (head column hc, d range)
  const int hc = tid & 15;
  const int dpart = tid >> 4;                // 16 parts of D/16 columns
  const int hlc = hgp * 16 + hc;
  if (hlc >= p.group) return;
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, ml[ww * 16 + hc]);
  float f[NW];
  float L = 0.0f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    const float mw = ml[ww * 16 + hc];
    f[ww] = (mw == -INFINITY) ? 0.0f : fast_exp2((mw - M) * sl2);
    L += f[ww] * ll[ww * 16 + hc];
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const int hq = kvh * p.group + hlc;
  const int64_t slot = ((int64_t)b * p.H + hq) * S + s;
  float* wo = p.ws_o + slot * D;
  constexpr int DPT = D / 16;
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    const int d = dpart * DPT + j;
    float acc = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) acc += f[ww] * mo[(ww * D + d) * 16 + hc];
    wo[d] = acc * inv;
  }
  if (dpart == 0) p.ws_lse[slot] = L > 0.0f ? M * sl2 + fast_log2(L) : -INFINITY;
}

}  // namespace

hipError_t launch_decode_bf16(const Params& p, hipStream_t st) {
  const int HG = ceil_div(p.group, 16);
  const long grid = (long)p.B * p.Hkv * HG * p.num_splits;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const bool paged = p.block_table != nullptr;
  if (p.d == 128) {
    if (paged)
      hipLaunchKernelGGL((decode_split_bf16_kernel<128, true>), dim3((unsigned)grid), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((decode_split_bf16_kernel<128, false>), dim3((unsigned)grid), dim3(256), 0, st, p);
  } else {
    if (paged)
      hipLaunchKernelGGL((decode_split_bf16_kernel<64, true>), dim3((unsigned)grid), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((decode_split_bf16_kernel<64, false>), dim3((unsigned)grid), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace attn
