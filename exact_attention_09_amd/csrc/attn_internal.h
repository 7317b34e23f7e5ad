// Launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include "attn_common.h"

namespace attn {

// bf16 tiled forward (dense or varlen); query tile height it was built with.
int prefill_bf16_block_m();
hipError_t launch_prefill_bf16(const Params& p, hipStream_t st);

// bf16 tiled forward, two wave groups in ping-pong (BM = 256), d = 64 or 128.
int prefill_pp_block_m();
hipError_t launch_prefill_pp(const Params& p, hipStream_t st);

// fp32 forward (VALU); with split set it writes decode partials instead.
int f32_block_m();
hipError_t launch_f32(const Params& p, bool split, hipStream_t st);

// bf16 split-KV decode partials (Sq == 1, dense).
hipError_t launch_decode_bf16(const Params& p, hipStream_t st);

// Fixed-order combine of the split partials into o and lse.
hipError_t launch_combine(const Params& p, bool out_bf16, hipStream_t st);

// Rows that can see no key at all (Skv == 0): O = 0, LSE = -inf.
hipError_t launch_fill_empty(const Params& p, bool out_bf16, hipStream_t st);

// Backward pass (bf16, BHSD, dense or varlen; p.window > 0: sliding window,
// p.sinks != null: sink gradients into dsinks [H]): Delta and the
// log2-domain LSE into `delta` and `lse2` (one float per query row each),
// then dK and dV, then dQ.
hipError_t launch_backward(const Params& p, const void* dout, float* delta, float* lse2, void* dq, void* dk,
                           void* dv, float* dsinks, hipStream_t st);

}  // namespace attn
