// fp32 attention forward on the vector ALUs (no low-precision step).
//
// Same tiled loop as the bf16 path (TileLang tutorial chapter 15, section
// 3.2; masks and guards from its sections 3.4 and 5.1) with the running max
// updated on every tile, as the section 2.3 recurrence is written.  One wave
// per workgroup owns 32 query rows; the two halves of the wave hold the two
// halves of the head dimension of the same row, so a score is one partial
// dot product per lane plus one cross-half add.  K/V tiles of 16 keys are
// staged in LDS and read as broadcasts.
//
// With `split` the kernel computes one key chunk of a decode row and writes
// the chunk's normalised output and base-2 log-sum-exp (the split-KV
// partials of the tutorial's section 5.4) instead of the final output.
#include "attn_common.h"
#include "attn_internal.h"

namespace attn {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;

template <int D, bool CAUSAL, bool VARLEN, bool SPLIT>
__global__ __launch_bounds__(64) void f32_kernel(const Params p) {
  constexpr int BM = 32;
  constexpr int BN = 16;
  constexpr int DH = D / 2;
  __shared__ __attribute__((aligned(16))) float ks[BN * D];
  __shared__ __attribute__((aligned(16))) float vs[BN * D];

  const int lane = threadIdx.x;
  const int r = lane & 31;
  const int half = lane >> 5;
  const float sl2 = p.scale_log2;

  int h, tile, sq, skv, off, split = 0;
  int64_t q_row0, kv_row0;
  if constexpr (!VARLEN) {
    int w = blockIdx.x;
    const int S = SPLIT ? p.num_splits : 1;
    split = w % S;
    w /= S;
    tile = w % p.tiles_per_head;
    const int bh = w / p.tiles_per_head;
    const int b = bh / p.H;
    h = bh - b * p.H;
    sq = p.Sq;
    skv = p.Skv;
    off = skv - sq;
    q_row0 = (int64_t)bh * sq;
    kv_row0 = ((int64_t)b * p.Hkv + h / p.group) * skv;
  } else {
    int bb;
    if (!varlen_item(p.cu, p.B, p.Sq, BM, p.tiles_per_head, false, blockIdx.x, h, bb, tile)) return;
    int s0, s1;
    seq_bounds(p.cu, p.Sq, bb, s0, s1);
    sq = s1 - s0;
    skv = sq;
    off = 0;
    q_row0 = (int64_t)h * p.Sq + s0;
    kv_row0 = (int64_t)(h / p.group) * p.Sq + s0;
  }

  const float* __restrict__ Q = (const float*)p.q + q_row0 * D;
  const float* __restrict__ K = (const float*)p.k + kv_row0 * D;
  const float* __restrict__ V = (const float*)p.v + kv_row0 * D;

  const int q0 = tile * BM;
  const int row = q0 + r;
  const bool rvalid = row < sq;

  float qv[DH];
#pragma unroll
  for (int t = 0; t < DH; ++t) qv[t] = rvalid ? Q[(int64_t)row * D + half * DH + t] : 0.0f;

  int klo = 0, khi = skv;
  if (SPLIT) {
    klo = split * p.split_len;
    klo = klo < skv ? klo : skv;
    khi = klo + p.split_len < skv ? klo + p.split_len : skv;
  } else if (CAUSAL) {
    const int q_hi = q0 + BM < sq ? q0 + BM : sq;
    khi = causal_kv_end(q_hi, off, skv);
  }
  int lim = khi;  // keys < lim are visible to this row
  if (CAUSAL) {
    const int c_lim = row + off + 1;
    lim = c_lim < lim ? c_lim : lim;
  }

  float m = -INFINITY, l = 0.0f;
  float o[DH];
#pragma unroll
  for (int t = 0; t < DH; ++t) o[t] = 0.0f;

  for (int k0 = klo; k0 < khi; k0 += BN) {
    __syncthreads();
    // BN x D floats, 4 per lane per pass
#pragma unroll
    for (int i = 0; i < BN * D / 256; ++i) {
      const int e = lane * 4 + 256 * i;
      int key = k0 + e / D;
      key = key < khi ? key : khi - 1;
      const int col = e % D;
      *(float4*)&ks[e] = *(const float4*)(K + (int64_t)key * D + col);
      *(float4*)&vs[e] = *(const float4*)(V + (int64_t)key * D + col);
    }
    __syncthreads();

    float sj[BN];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float dot = 0.0f;
#pragma unroll
      for (int t = 0; t < DH; ++t) dot = fmaf(qv[t], ks[j * D + half * DH + t], dot);
      dot += shfl_xor_f(dot, 32);
      sj[j] = (k0 + j < lim) ? dot : -INFINITY;
      mt = fmaxf(mt, sj[j]);
    }
    const float m_new = fmaxf(m, mt);
    const float offm = (m_new == -INFINITY) ? 0.0f : m_new * sl2;  // check_inf
    const float alpha = fast_exp2(fmaf(m, sl2, -offm));
    float rs = 0.0f;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      sj[j] = fast_exp2(fmaf(sj[j], sl2, -offm));
      rs += sj[j];
    }
    l = fmaf(alpha, l, rs);
#pragma unroll
    for (int t = 0; t < DH; ++t) {
      float a = alpha * o[t];
#pragma unroll
      for (int j = 0; j < BN; ++j) a = fmaf(sj[j], vs[j * D + half * DH + t], a);
      o[t] = a;
    }
    m = m_new;
  }

  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (!SPLIT) {
    if (rvalid) {
      float* orow = (float*)p.o + (q_row0 + row) * D + half * DH;
#pragma unroll
      for (int t = 0; t < DH; ++t) orow[t] = o[t] * inv;
      if (p.lse != nullptr && half == 0)
        p.lse[q_row0 + row] = l > 0.0f ? (m * sl2 + fast_log2(l)) * kLn2 : -INFINITY;
    }
  } else {
    if (row == 0) {
      const int64_t slot = q_row0 * p.num_splits + split;  // q_row0 = b*H + h when Sq == 1
      float* wo = p.ws_o + slot * D + half * DH;
#pragma unroll
      for (int t = 0; t < DH; ++t) wo[t] = o[t] * inv;
      if (half == 0) p.ws_lse[slot] = l > 0.0f ? m * sl2 + fast_log2(l) : -INFINITY;
    }
  }
}

template <int D, bool SPLIT>
hipError_t launch_d(const Params& p, hipStream_t st) {
  long grid;
  if (p.cu != nullptr)
    grid = (long)p.H * p.tiles_per_head;
  else
    grid = (long)p.B * p.H * p.tiles_per_head * (SPLIT ? p.num_splits : 1);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), blk(64);
  if (p.cu != nullptr) {
    if (p.causal)
      hipLaunchKernelGGL((f32_kernel<D, true, true, false>), g, blk, 0, st, p);
    else
      hipLaunchKernelGGL((f32_kernel<D, false, true, false>), g, blk, 0, st, p);
  } else if (SPLIT) {
    hipLaunchKernelGGL((f32_kernel<D, false, false, true>), g, blk, 0, st, p);
  } else if (p.causal) {
    hipLaunchKernelGGL((f32_kernel<D, true, false, false>), g, blk, 0, st, p);
  } else {
    hipLaunchKernelGGL((f32_kernel<D, false, false, false>), g, blk, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace

int f32_block_m() { return 32; }

hipError_t launch_f32(const Params& p, bool split, hipStream_t st) {
  if (p.d == 128) return split ? launch_d<128, true>(p, st) : launch_d<128, false>(p, st);
  return split ? launch_d<64, true>(p, st) : launch_d<64, false>(p, st);
}

}  // namespace attn
