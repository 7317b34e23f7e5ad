// Split-KV combine and the no-key fill.
//
// Combine (TileLang tutorial chapter 15, section 5.4): each split s of a
// decode row left O_s (normalised by its own l_s) and glse_s = log2 l_s +
// m_s * s * log2(e).  The output is sum_s w_s O_s with w_s = l_s / sum l,
// computed as 2^(glse_s - glse_tot), glse_tot = log2 sum 2^(glse_s - max) +
// max.  The splits are visited in index order by one lane each, so the
// result is bitwise reproducible.  Empty splits carry glse = -inf and weigh
// nothing; a row with no key at all gets O = 0 and LSE = -inf.
#include "attn_common.h"
#include "attn_internal.h"

namespace attn {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;

template <typename OutT>
__device__ inline OutT cast_out(float x);
template <>
__device__ inline float cast_out<float>(float x) { return x; }
template <>
__device__ inline __bf16 cast_out<__bf16>(float x) { return (__bf16)x; }

// one wave per (b, h) row; each lane owns D/64 columns
template <int D, typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(const Params p) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long)p.B * p.H) return;
  const int S = p.num_splits;
  const float* gl = p.ws_lse + row * S;
  const float* po = p.ws_o + row * S * D;

  float gmax = -INFINITY;
  for (int s = 0; s < S; ++s) gmax = fmaxf(gmax, gl[s]);
  OutT* orow = (OutT*)p.o + row * D;
  if (gmax == -INFINITY) {
#pragma unroll
    for (int j = 0; j < DPL; ++j) orow[lane * DPL + j] = cast_out<OutT>(0.0f);
    if (p.lse != nullptr && lane == 0) p.lse[row] = -INFINITY;
    return;
  }
  float tot = 0.0f;
  for (int s = 0; s < S; ++s) tot += fast_exp2(gl[s] - gmax);
  const float gtot = fast_log2(tot) + gmax;
  float acc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) acc[j] = 0.0f;
  for (int s = 0; s < S; ++s) {
    const float w = fast_exp2(gl[s] - gtot);
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[j] = fmaf(w, po[(long)s * D + lane * DPL + j], acc[j]);
  }
#pragma unroll
  for (int j = 0; j < DPL; ++j) orow[lane * DPL + j] = cast_out<OutT>(acc[j]);
  if (p.lse != nullptr && lane == 0) p.lse[row] = gtot * kLn2;
}

template <typename OutT>
__global__ __launch_bounds__(256) void fill_empty_kernel(OutT* o, float* lse, long rows, int d) {
  const long n = rows * d;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256)
    o[i] = cast_out<OutT>(0.0f);
  if (lse != nullptr)
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < rows; i += (long)gridDim.x * 256)
      lse[i] = -INFINITY;
}

}  // namespace

hipError_t launch_combine(const Params& p, bool out_bf16, hipStream_t st) {
  const long rows = (long)p.B * p.H;
  if (rows <= 0) return hipSuccess;
  const long grid = (rows + 3) / 4;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), blk(256);
  if (p.d == 128) {
    if (out_bf16)
      hipLaunchKernelGGL((combine_kernel<128, __bf16>), g, blk, 0, st, p);
    else
      hipLaunchKernelGGL((combine_kernel<128, float>), g, blk, 0, st, p);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((combine_kernel<64, __bf16>), g, blk, 0, st, p);
    else
      hipLaunchKernelGGL((combine_kernel<64, float>), g, blk, 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_fill_empty(const Params& p, bool out_bf16, hipStream_t st) {
  const long rows = p.cu != nullptr ? (long)p.H * p.Sq : (long)p.B * p.H * p.Sq;
  if (rows <= 0) return hipSuccess;
  long blocks = (rows * p.d + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (out_bf16)
    hipLaunchKernelGGL(fill_empty_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (__bf16*)p.o, p.lse, rows, p.d);
  else
    hipLaunchKernelGGL(fill_empty_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (float*)p.o, p.lse, rows, p.d);
  return hipGetLastError();
}

}  // namespace attn
