// Split-KV combine and the no-key fill.
//
// Combine (TileLang tutorial chapter 15, section 5.4): each split s of a
// decode row left O_s (normalised by its own l_s) and glse_s = log2 l_s +
// m_s * s * log2(e).  The output is sum_s w_s O_s with w_s = l_s / sum l,
// computed as 2^(glse_s - glse_tot), glse_tot = log2 sum 2^(glse_s - max) +
// max.  Every reduction has a fixed order, so the result is bitwise
// reproducible.  Empty splits carry glse = -inf and weigh
// nothing; a row with no key at all gets O = 0 and LSE = -inf.
#include "attn_common.h"
#include "attn_internal.h"

namespace attn {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

template <typename OutT>
__device__ inline OutT cast_out(float x);
template <>
__device__ inline float cast_out<float>(float x) { return x; }
template <>
__device__ inline __bf16 cast_out<__bf16>(float x) { return (__bf16)x; }

// one wave per (b, h) row.  The split LSEs are spread over the lanes (lane
// s % 64 holds split s) and reduced with a fixed butterfly; the partial rows
// are then read sixteen splits at a time, all loads in flight together, and
// added in split order.  Each lane owns D/64 adjacent columns.
template <int D, typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(const Params p) {
  constexpr int DPL = D / 64;
  constexpr int CHUNK = 16;
  typedef float vec_t __attribute__((ext_vector_type(DPL)));
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= (long)p.B * p.H) return;
  const int S = p.num_splits;
  const float* gl = p.ws_lse + row * S;
  const float* po = p.ws_o + row * S * D + lane * DPL;

  // an attention sink (tutorial sections 4.6 and 4.7) is one more term of
  // the denominator, with no value: it joins the max and the sum only
  const float sink = p.sinks != nullptr ? p.sinks[row % p.H] * kLog2e : -INFINITY;
  float gmax = -INFINITY;
  for (int s0 = 0; s0 < S; s0 += 64)
    if (s0 + lane < S) gmax = fmaxf(gmax, gl[s0 + lane]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) gmax = fmaxf(gmax, shfl_xor_f(gmax, m));
  gmax = fmaxf(gmax, sink);
  OutT* orow = (OutT*)p.o + row * D + lane * DPL;
  if (gmax == -INFINITY) {
#pragma unroll
    for (int j = 0; j < DPL; ++j) orow[j] = cast_out<OutT>(0.0f);
    if (p.lse != nullptr && lane == 0) p.lse[row] = -INFINITY;
    return;
  }
  float tot = 0.0f;
  for (int s0 = 0; s0 < S; s0 += 64)
    if (s0 + lane < S) tot += fast_exp2(gl[s0 + lane] - gmax);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) tot += shfl_xor_f(tot, m);
  if (sink > -INFINITY) tot += fast_exp2(sink - gmax);
  const float gtot = fast_log2(tot) + gmax;

  vec_t acc = {};
  for (int s0 = 0; s0 < S; s0 += 64) {
    // weight of split s0 + lane in this lane, handed out with readlane
    const float wl = s0 + lane < S ? fast_exp2(gl[s0 + lane] - gtot) : 0.0f;
    const int n = S - s0 < 64 ? S - s0 : 64;
    for (int c0 = 0; c0 < n; c0 += CHUNK) {
      vec_t part[CHUNK];
#pragma unroll
      for (int j = 0; j < CHUNK; ++j)
        part[j] = c0 + j < n ? *(const vec_t*)(po + (long)(s0 + c0 + j) * D) : vec_t{};
#pragma unroll
      for (int j = 0; j < CHUNK; ++j)
        acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), c0 + j)) * part[j];
    }
  }
#pragma unroll
  for (int j = 0; j < DPL; ++j) orow[j] = cast_out<OutT>(acc[j]);
  if (p.lse != nullptr && lane == 0) p.lse[row] = gtot * kLn2;
}

// Rows [head-major runs of `run` rows per head]: O = 0; LSE = -inf, or the
// head's sink when sinks are given (the sink is then the only term of the
// denominator).
template <typename OutT>
__global__ __launch_bounds__(256) void fill_empty_kernel(OutT* o, float* lse, long rows, int d, const float* sinks,
                                                         int H, int run) {
  const long n = rows * d;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256)
    o[i] = cast_out<OutT>(0.0f);
  if (lse != nullptr)
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < rows; i += (long)gridDim.x * 256)
      lse[i] = sinks != nullptr ? sinks[(i / run) % H] : -INFINITY;
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
  // lse is [B, H, Sq] (varlen [H, T]): runs of Sq rows per head
  const int run = p.Sq > 0 ? p.Sq : 1;
  if (out_bf16)
    hipLaunchKernelGGL(fill_empty_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (__bf16*)p.o, p.lse, rows, p.d, p.sinks, p.H, run);
  else
    hipLaunchKernelGGL(fill_empty_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (float*)p.o, p.lse, rows, p.d, p.sinks, p.H, run);
  return hipGetLastError();
}

}  // namespace attn
