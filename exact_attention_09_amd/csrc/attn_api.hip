// C-ABI entry points: argument validation (before any HIP call), path
// selection (tiled forward, split-KV decode, no-key fill) and the split
// workspace.  See include/attn.h for the contract.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "attn.h"
#include "attn_common.h"
#include "attn_internal.h"

namespace {

thread_local char g_err[512] = "";

attn_status fail(attn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

attn_status hip_fail(hipError_t e, const char* what) {
  return fail(ATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr size_t kWsAlign = 256;

size_t ws_lse_offset(long rows, int d, int splits) {
  const size_t o_bytes = (size_t)rows * splits * d * sizeof(float);
  return (o_bytes + kWsAlign - 1) / kWsAlign * kWsAlign;
}

// Enough workgroups to cover the 256 CUs a few times over, chunks of at
// least 256 keys.
int heuristic_splits(int B, int Hkv, int Skv) {
  const long base = (long)B * Hkv;
  if (base <= 0 || Skv <= 0) return 1;
  long want = (1024 + base - 1) / base;
  long cap = Skv / 256;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want > ATTN_MAX_SPLITS) want = ATTN_MAX_SPLITS;
  return want < 1 ? 1 : (int)want;
}

}  // namespace

// compute units of the current device, looked up once per device
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// ---- the scratch memory of attn_fwd_noalloc: a static device array of
// ATTN_NOALLOC_SCRATCH_BYTES, one copy per GPU (loaded with the library's
// code object), holding the split-KV partials of the decode path.  Host code
// uses it only through the device address hipGetSymbolAddress returns for
// the current device (the array's name is a host-side stand-in).
constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The current device's address of the scratch array, looked up once per
// device (with that device current) and kept.
static attn_status scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_EUNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess || a == nullptr) return hip_fail(e, "hipGetSymbolAddress of the scratch array");
    addr[dev] = a;
  }
  *out = addr[dev];
  return ATTN_OK;
}

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported configuration";
    case ATTN_ENOMEM: return "out of memory";
    case ATTN_EHIP: return "HIP error";
  }
  return "unknown status";
}

const char* attn_last_error(void) { return g_err; }

size_t attn_workspace_bytes(int B, int H, int d, int num_splits) {
  if (B < 0 || H < 0 || d <= 0 || num_splits < 1 || num_splits > ATTN_MAX_SPLITS) return 0;
  const long rows = (long)B * H;
  return ws_lse_offset(rows, d, num_splits) + (size_t)rows * num_splits * sizeof(float);
}

int attn_decode_num_splits(int B, int Hkv, int Skv) { return heuristic_splits(B, Hkv, Skv); }

}  // extern "C"

namespace {

// The forward pass behind attn_fwd_ex and attn_fwd_window_sink: window > 0
// and sinks != NULL are the causal bf16 variants (validated by the caller).
attn_status forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                    int Sq, int Skv, int d, float scale, int causal, const int32_t* cu_seqlens, void* stream,
                    attn_dtype dtype, const attn_opts* opts, int window, const float* sinks,
                    attn_layout layout, bool use_scratch = false) {
  g_err[0] = '\0';
  // ---- validation: no HIP call until every check has passed
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return fail(ATTN_EINVAL, "unknown dtype %d", (int)dtype);
  if (layout != ATTN_BHSD && layout != ATTN_BSHD) return fail(ATTN_EINVAL, "unknown layout %d", (int)layout);
  if (layout == ATTN_BSHD && dtype != ATTN_BF16)
    return fail(ATTN_EUNSUPPORTED, "the BSHD layout is built for bf16 only");
  if (B < 0 || H < 0 || Hkv < 0 || Sq < 0 || Skv < 0 || d < 0)
    return fail(ATTN_EINVAL, "negative size (B=%d H=%d Hkv=%d Sq=%d Skv=%d d=%d)", B, H, Hkv, Sq, Skv, d);
  if (opts != nullptr && (opts->num_splits < 0 || opts->num_splits > ATTN_MAX_SPLITS))
    return fail(ATTN_EINVAL, "num_splits %d outside [0, %d]", opts->num_splits, ATTN_MAX_SPLITS);
  const unsigned flags = opts != nullptr ? opts->flags : 0u;
  if ((flags & ~(ATTN_FLAG_BASIC_PREFILL | ATTN_FLAG_NO_PERSIST)) != 0)
    return fail(ATTN_EINVAL, "unknown flag bits 0x%x", flags);
  if (B == 0 || H == 0 || Sq == 0) return ATTN_OK;  // nothing to compute
  if (q == nullptr || o == nullptr) return fail(ATTN_EINVAL, "q and o must not be NULL");
  if (Skv > 0 && (k == nullptr || v == nullptr))
    return fail(ATTN_EINVAL, "k and v must not be NULL when Skv > 0");
  if (Hkv < 1 || H % Hkv != 0) return fail(ATTN_EINVAL, "H=%d is not a multiple of Hkv=%d", H, Hkv);
  if (d != 64 && d != 128) return fail(ATTN_EUNSUPPORTED, "head dim %d (built: 64, 128)", d);
  if (!(std::isfinite(scale) && scale > 0.0f))
    return fail(ATTN_EINVAL, "scale must be finite and > 0 (got %g)", (double)scale);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(ATTN_EINVAL, "q, k, v, o must be 16-byte aligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(ATTN_EINVAL, "lse must be 4-byte aligned");
  const bool varlen = cu_seqlens != nullptr;
  if (varlen) {
    if (Sq != Skv) return fail(ATTN_EINVAL, "varlen needs Sq == Skv == total tokens (got %d, %d)", Sq, Skv);
    if (!aligned(cu_seqlens, 4)) return fail(ATTN_EINVAL, "cu_seqlens must be 4-byte aligned");
  }
  // element counts must fit the 64-bit offsets and the 32-bit row counters
  const long double q_elems = (long double)(varlen ? 1 : B) * H * Sq * d;
  const long double kv_elems = (long double)(varlen ? 1 : B) * Hkv * Skv * d;
  if (q_elems > 9.0e18L || kv_elems > 9.0e18L) return fail(ATTN_EINVAL, "tensor too large");
  // a K/V row (H * d elements apart in BSHD) times the rows of one tile (at
  // most 128) must stay inside the 32-bit byte range of a buffer descriptor
  if ((long)H * d >= (1L << 23)) return fail(ATTN_EINVAL, "H * d too large (must be below 2^23)");

  attn::Params p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.cu = cu_seqlens;
  p.B = B; p.H = H; p.Hkv = Hkv; p.Sq = Sq; p.Skv = Skv; p.d = d;
  p.group = H / Hkv;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  p.window = window;
  p.sinks = sinks;
  p.bshd = layout == ATTN_BSHD ? 1 : 0;
  p.q_rs = p.bshd ? H * d : d;
  p.kv_rs = p.bshd ? Hkv * d : d;
  hipStream_t st = (hipStream_t)stream;
  const bool bf16 = dtype == ATTN_BF16;
  const bool local = window > 0 || sinks != nullptr;

  if (!varlen && Skv == 0) {
    const hipError_t e = attn::launch_fill_empty(p, bf16, st);
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "fill kernel");
  }

  const bool decode = !varlen && Sq == 1;
  if (!decode) {
    // ATTN_FLAG_BASIC_PREFILL selects the basic tiled kernel instead (it has
    // no window, sink or BSHD layout)
    const bool pingpong = bf16 && (local || p.bshd || (flags & ATTN_FLAG_BASIC_PREFILL) == 0);
    const int bm = !bf16 ? attn::f32_block_m()
                         : (pingpong ? attn::prefill_pp_block_m() : attn::prefill_bf16_block_m());
    const long tiles = varlen ? (long)Sq / bm + B : attn::ceil_div(Sq, bm);
    const long work = (varlen ? (long)H : (long)B * H) * tiles;
    if (work > 0x7ffffff0L) return fail(ATTN_EINVAL, "too many query tiles");
    p.tiles_per_head = (int)tiles;
    p.work_items = (int)work;
    // a persistent grid of one workgroup per CU (the kernel pairs heavy and
    // light causal tiles): dense when the items divide evenly over the CUs,
    // varlen when locating an item (a scan over sequences and tile indices)
    // stays short; otherwise one workgroup per item and the hardware
    // dispatcher balances.  ATTN_FLAG_NO_PERSIST forces the latter.
    p.persist_c = 0;
    if (pingpong && (flags & ATTN_FLAG_NO_PERSIST) == 0) {
      const int cus = device_cus();
      const long c = cus / 8;
      const bool fits = varlen ? H % 8 == 0 && B <= 1024 && (long)B * attn::ceil_div(Sq, bm) <= 1L << 16
                               : work % (8 * c > 0 ? 8 * c : 1) == 0;
      if (c > 0 && cus % 8 == 0 && fits) p.persist_c = (int)c;
    }
    const hipError_t e = !bf16 ? attn::launch_f32(p, false, st)
                               : (pingpong ? attn::launch_prefill_pp(p, st) : attn::launch_prefill_bf16(p, st));
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "forward kernel");
  }

  // ---- split-KV decode
  const int keys = (window > 0 && window < Skv) ? window : Skv;  // keys the query sees
  int splits = (opts != nullptr && opts->num_splits > 0) ? opts->num_splits : attn_decode_num_splits(B, Hkv, keys);
  if (splits > keys) splits = keys;  // keep every split non-empty when possible
  if (splits < 1) splits = 1;
  p.num_splits = splits;
  p.split_len = attn::ceil_div(Skv, splits);
  p.tiles_per_head = 1;
  if ((long)B * H * splits > 0x7ffffff0L) return fail(ATTN_EINVAL, "too many decode rows");
  const size_t need = attn_workspace_bytes(B, H, d, splits);
  const long rows = (long)B * H;
  void* ws = nullptr;
  bool own = false;
  if (use_scratch) {
    // attn_fwd_noalloc: the static scratch array, never an allocation
    if (need > kScratchBytes)
      return fail(ATTN_EINVAL,
                  "the split partials need %zu bytes (B=%d H=%d d=%d splits=%d), more than the %zu bytes of "
                  "scratch attn_fwd_noalloc holds (ATTN_NOALLOC_SCRATCH_BYTES); use fewer splits or attn_fwd_ex",
                  need, B, H, d, splits, kScratchBytes);
    const attn_status sst = scratch_address(&ws);
    if (sst != ATTN_OK) return sst;
  } else if (opts != nullptr && opts->workspace != nullptr) {
    if (opts->workspace_bytes < need)
      return fail(ATTN_EINVAL, "workspace of %zu bytes, %zu needed", opts->workspace_bytes, need);
    if (!aligned(opts->workspace, kWsAlign)) return fail(ATTN_EINVAL, "workspace must be 256-byte aligned");
    ws = opts->workspace;
  } else {
    const hipError_t e = hipMallocAsync(&ws, need, st);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(ATTN_ENOMEM, "workspace of %zu bytes: %s", need, hipGetErrorString(e));
    }
    own = true;
  }
  p.ws_o = (float*)ws;
  p.ws_lse = (float*)((char*)ws + ws_lse_offset(rows, d, splits));

  hipError_t e = bf16 ? attn::launch_decode_bf16(p, st) : attn::launch_f32(p, true, st);
  attn_status status = ATTN_OK;
  if (e != hipSuccess) {
    status = hip_fail(e, "split kernel");
  } else {
    e = attn::launch_combine(p, bf16, st);
    if (e != hipSuccess) status = hip_fail(e, "combine kernel");
  }
  if (own) {
    const hipError_t ef = hipFreeAsync(ws, st);
    if (ef != hipSuccess && status == ATTN_OK) status = hip_fail(ef, "workspace release");
  }
  return status;
}

}  // namespace

extern "C" {

attn_status attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int Hkv, int Sq, int Skv, int d, float scale, int causal,
                        const int32_t* cu_seqlens, void* stream, attn_dtype dtype,
                        const attn_opts* opts) {
  return forward(q, k, v, o, lse, B, H, Hkv, Sq, Skv, d, scale, causal, cu_seqlens, stream, dtype, opts, 0,
                 nullptr, ATTN_BHSD);
}

attn_status attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                             int Hkv, int Sq, int Skv, int d, float scale, int causal, const int32_t* cu_seqlens,
                             void* stream, attn_dtype dtype, const attn_opts* opts) {
  g_err[0] = '\0';
  if (opts != nullptr && opts->workspace != nullptr)
    return fail(ATTN_EINVAL, "attn_fwd_noalloc takes no workspace (it uses its static scratch array)");
  return forward(q, k, v, o, lse, B, H, Hkv, Sq, Skv, d, scale, causal, cu_seqlens, stream, dtype, opts, 0,
                 nullptr, ATTN_BHSD, /*use_scratch=*/true);
}

attn_status attn_fwd_window_sink(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                 int Hkv, int Sq, int Skv, int d, float scale, const int32_t* cu_seqlens,
                                 int window, const float* sinks, void* stream, const attn_opts* opts) {
  g_err[0] = '\0';
  if (window < 0) return fail(ATTN_EINVAL, "window %d < 0", window);
  if (sinks != nullptr && !aligned(sinks, 4)) return fail(ATTN_EINVAL, "sinks must be 4-byte aligned");
  return forward(q, k, v, o, lse, B, H, Hkv, Sq, Skv, d, scale, 1, cu_seqlens, stream, ATTN_BF16, opts, window,
                 sinks, ATTN_BHSD);
}

attn_status attn_fwd_layout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                            int Sq, int Skv, int d, float scale, int causal, const int32_t* cu_seqlens,
                            attn_layout layout, int window, const float* sinks, void* stream,
                            const attn_opts* opts) {
  g_err[0] = '\0';
  if (window < 0) return fail(ATTN_EINVAL, "window %d < 0", window);
  if ((window > 0 || sinks != nullptr) && !causal)
    return fail(ATTN_EINVAL, "a window or sinks need causal attention");
  if (sinks != nullptr && !aligned(sinks, 4)) return fail(ATTN_EINVAL, "sinks must be 4-byte aligned");
  return forward(q, k, v, o, lse, B, H, Hkv, Sq, Skv, d, scale, causal, cu_seqlens, stream, ATTN_BF16, opts,
                 window, sinks, layout);
}

attn_status attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                           const int32_t* block_table, const int32_t* seqlens_k, int B, int H, int Hkv,
                           int d, int page_size, int max_pages, int num_pages, float scale, void* stream,
                           const attn_opts* opts) {
  g_err[0] = '\0';
  // ---- validation: no HIP call until every check has passed
  if (B < 0 || H < 0 || Hkv < 0 || d < 0 || max_pages < 0 || num_pages < 0)
    return fail(ATTN_EINVAL, "negative size (B=%d H=%d Hkv=%d d=%d max_pages=%d num_pages=%d)", B, H, Hkv, d,
                max_pages, num_pages);
  if (opts != nullptr && (opts->num_splits < 0 || opts->num_splits > ATTN_MAX_SPLITS))
    return fail(ATTN_EINVAL, "num_splits %d outside [0, %d]", opts->num_splits, ATTN_MAX_SPLITS);
  if (opts != nullptr && (opts->flags & ~(ATTN_FLAG_BASIC_PREFILL | ATTN_FLAG_NO_PERSIST)) != 0)
    return fail(ATTN_EINVAL, "unknown flag bits 0x%x", opts->flags);
  if (B == 0 || H == 0) return ATTN_OK;  // nothing to compute
  if (q == nullptr || o == nullptr || k_cache == nullptr || v_cache == nullptr || block_table == nullptr ||
      seqlens_k == nullptr)
    return fail(ATTN_EINVAL, "q, o, k_cache, v_cache, block_table and seqlens_k must not be NULL");
  if (Hkv < 1 || H % Hkv != 0) return fail(ATTN_EINVAL, "H=%d is not a multiple of Hkv=%d", H, Hkv);
  if (d != 64 && d != 128) return fail(ATTN_EUNSUPPORTED, "head dim %d (built: 64, 128)", d);
  if (page_size < 16 || page_size > (1 << 16) || (page_size & (page_size - 1)) != 0)
    return fail(ATTN_EUNSUPPORTED, "page size %d (built: powers of two from 16 to 65536)", page_size);
  if (max_pages < 1 || num_pages < 1) return fail(ATTN_EINVAL, "max_pages and num_pages must be >= 1");
  if ((long)max_pages * page_size > 0x7fffffffL)
    return fail(ATTN_EINVAL, "max_pages * page_size = %ld keys does not fit int32", (long)max_pages * page_size);
  if ((long double)num_pages * Hkv * page_size * d > 9.0e18L) return fail(ATTN_EINVAL, "cache too large");
  if (!(std::isfinite(scale) && scale > 0.0f))
    return fail(ATTN_EINVAL, "scale must be finite and > 0 (got %g)", (double)scale);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16))
    return fail(ATTN_EINVAL, "q, k_cache, v_cache, o must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seqlens_k, 4) || (lse != nullptr && !aligned(lse, 4)))
    return fail(ATTN_EINVAL, "block_table, seqlens_k and lse must be 4-byte aligned");

  attn::Params p{};
  p.q = q; p.k = k_cache; p.v = v_cache; p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.Hkv = Hkv; p.Sq = 1; p.Skv = max_pages * page_size; p.d = d;
  p.group = H / Hkv;
  p.scale = scale;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  p.block_table = block_table;
  p.seqlens_k = seqlens_k;
  p.q_rs = d;
  p.kv_rs = d;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  p.page_shift = shift;
  p.max_pages = max_pages;
  p.num_pages = num_pages;
  hipStream_t st = (hipStream_t)stream;

  int splits = (opts != nullptr && opts->num_splits > 0) ? opts->num_splits : attn_decode_num_splits(B, Hkv, p.Skv);
  if (splits > p.Skv) splits = p.Skv;
  if (splits < 1) splits = 1;
  p.num_splits = splits;
  p.tiles_per_head = 1;
  if ((long)B * H * splits > 0x7ffffff0L) return fail(ATTN_EINVAL, "too many decode rows");
  const size_t need = attn_workspace_bytes(B, H, d, splits);
  const long rows = (long)B * H;
  void* ws = nullptr;
  bool own = false;
  if (opts != nullptr && opts->workspace != nullptr) {
    if (opts->workspace_bytes < need)
      return fail(ATTN_EINVAL, "workspace of %zu bytes, %zu needed", opts->workspace_bytes, need);
    if (!aligned(opts->workspace, kWsAlign)) return fail(ATTN_EINVAL, "workspace must be 256-byte aligned");
    ws = opts->workspace;
  } else {
    const hipError_t e = hipMallocAsync(&ws, need, st);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(ATTN_ENOMEM, "workspace of %zu bytes: %s", need, hipGetErrorString(e));
    }
    own = true;
  }
  p.ws_o = (float*)ws;
  p.ws_lse = (float*)((char*)ws + ws_lse_offset(rows, d, splits));

  hipError_t e = attn::launch_decode_bf16(p, st);
  attn_status status = ATTN_OK;
  if (e != hipSuccess) {
    status = hip_fail(e, "paged split kernel");
  } else {
    e = attn::launch_combine(p, true, st);
    if (e != hipSuccess) status = hip_fail(e, "combine kernel");
  }
  if (own) {
    const hipError_t ef = hipFreeAsync(ws, st);
    if (ef != hipSuccess && status == ATTN_OK) status = hip_fail(ef, "workspace release");
  }
  return status;
}

size_t attn_bwd_workspace_bytes(int B, int H, int Sq) {
  if (B < 0 || H < 0 || Sq < 0) return 0;
  // Delta and the log2-domain LSE, each rounded up to the alignment
  return 2 * (((size_t)B * H * Sq * sizeof(float) + kWsAlign - 1) / kWsAlign * kWsAlign);
}

}  // extern "C"

namespace {

// The backward behind attn_bwd, attn_bwd_window_sink and attn_bwd_layout:
// window > 0 and sinks != NULL are causal (the callers validate that).
attn_status backward(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, int B, int H, int Hkv, int Sq, int Skv, int d, float scale,
                     int causal, const int32_t* cu_seqlens, int window, const float* sinks, float* dsinks,
                     void* stream, const attn_opts* opts, attn_layout layout) {
  g_err[0] = '\0';
  // ---- validation: no HIP call until every check has passed
  if (layout != ATTN_BHSD && layout != ATTN_BSHD) return fail(ATTN_EINVAL, "unknown layout %d", (int)layout);
  if (window < 0) return fail(ATTN_EINVAL, "window must be >= 0 (got %d)", window);
  if (sinks != nullptr && (!aligned(sinks, 4) || dsinks == nullptr || !aligned(dsinks, 4)))
    return fail(ATTN_EINVAL, "sinks need a 4-byte aligned dsinks output of H floats");
  if (B < 0 || H < 0 || Hkv < 0 || Sq < 0 || Skv < 0 || d < 0)
    return fail(ATTN_EINVAL, "negative size (B=%d H=%d Hkv=%d Sq=%d Skv=%d d=%d)", B, H, Hkv, Sq, Skv, d);
  if (B == 0 || H == 0 || (Sq == 0 && Skv == 0)) return ATTN_OK;
  if (Hkv < 1 || H % Hkv != 0) return fail(ATTN_EINVAL, "H=%d is not a multiple of Hkv=%d", H, Hkv);
  if (d != 64 && d != 128) return fail(ATTN_EUNSUPPORTED, "head dim %d (built: 64, 128)", d);
  if (!(std::isfinite(scale) && scale > 0.0f))
    return fail(ATTN_EINVAL, "scale must be finite and > 0 (got %g)", (double)scale);
  if (Sq > 0 && (q == nullptr || o == nullptr || dout == nullptr || lse == nullptr || dq == nullptr))
    return fail(ATTN_EINVAL, "q, o, dout, lse and dq must not be NULL");
  if (Skv > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
    return fail(ATTN_EINVAL, "k, v, dk and dv must not be NULL when Skv > 0");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(ATTN_EINVAL, "q, k, v, o, dout, dq, dk, dv must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(ATTN_EINVAL, "lse must be 4-byte aligned");
  const bool varlen = cu_seqlens != nullptr;
  if (varlen) {
    if (Sq != Skv) return fail(ATTN_EINVAL, "varlen needs Sq == Skv == total tokens (got %d, %d)", Sq, Skv);
    if (!aligned(cu_seqlens, 4)) return fail(ATTN_EINVAL, "cu_seqlens must be 4-byte aligned");
  }
  const long double q_elems = (long double)(varlen ? 1 : B) * H * Sq * d;
  const long double kv_elems = (long double)(varlen ? 1 : B) * Hkv * Skv * d;
  if (q_elems > 9.0e18L || kv_elems > 9.0e18L) return fail(ATTN_EINVAL, "tensor too large");
  // a row of q (H d elements apart in BSHD) times the rows of one tile (at
  // most 64) must stay inside the 32-bit byte range of a buffer descriptor
  if ((long)H * d >= (1L << 23)) return fail(ATTN_EINVAL, "H * d too large (must be below 2^23)");
  const long q_tiles = varlen ? (long)H * (Sq / 128 + B) : (long)B * H * attn::ceil_div(Sq, 128);
  const long k_tiles = varlen ? (long)Hkv * (Skv / 128 + B) : (long)B * Hkv * attn::ceil_div(Skv, 128);
  if (q_tiles > 0x7ffffff0L || k_tiles > 0x7ffffff0L) return fail(ATTN_EINVAL, "too many tiles");

  attn::Params p{};
  p.q = q; p.k = k; p.v = v; p.o = (void*)o; p.lse = (float*)lse; p.cu = cu_seqlens;
  p.B = B; p.H = H; p.Hkv = Hkv; p.Sq = Sq; p.Skv = Skv; p.d = d;
  p.group = H / Hkv;
  p.causal = causal ? 1 : 0;
  p.window = window;
  p.sinks = sinks;
  p.scale = scale;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  p.bshd = layout == ATTN_BSHD ? 1 : 0;
  p.q_rs = p.bshd ? H * d : d;
  p.kv_rs = p.bshd ? Hkv * d : d;
  hipStream_t st = (hipStream_t)stream;

  if (Sq == 0) {  // dense only: a varlen call with no token returned above
    // no query: dK = dV = 0
    // rows counted as B * Hkv * Skv in 64 bits by the fill kernel's launcher
    attn::Params z = p;
    z.B = B; z.H = Hkv; z.Sq = Skv; z.cu = nullptr; z.lse = nullptr; z.sinks = nullptr;
    z.o = dk;
    hipError_t e = attn::launch_fill_empty(z, true, st);
    if (e == hipSuccess) {
      z.o = dv;
      e = attn::launch_fill_empty(z, true, st);
    }
    if (e == hipSuccess && sinks != nullptr) {  // dsinks = 0: H fp32 zeros through the same fill kernel
      z.B = 1;
      z.H = 1;
      z.Sq = 1;
      z.d = H;
      z.o = dsinks;
      e = attn::launch_fill_empty(z, false, st);
    }
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "fill kernel");
  }
  const size_t need = attn_bwd_workspace_bytes(varlen ? 1 : B, H, Sq);
  void* ws = nullptr;
  bool own = false;
  if (opts != nullptr && opts->workspace != nullptr) {
    if (opts->workspace_bytes < need)
      return fail(ATTN_EINVAL, "workspace of %zu bytes, %zu needed", opts->workspace_bytes, need);
    if (!aligned(opts->workspace, kWsAlign)) return fail(ATTN_EINVAL, "workspace must be 256-byte aligned");
    ws = opts->workspace;
  } else {
    const hipError_t e = hipMallocAsync(&ws, need, st);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(ATTN_ENOMEM, "workspace of %zu bytes: %s", need, hipGetErrorString(e));
    }
    own = true;
  }
  attn_status status = ATTN_OK;
  float* delta = (float*)ws;
  float* lse2 = (float*)((char*)ws + need / 2);
  hipError_t e = attn::launch_backward(p, dout, delta, lse2, dq, dk, dv, dsinks, st);
  if (e != hipSuccess) status = hip_fail(e, "backward kernels");
  if (own) {
    const hipError_t ef = hipFreeAsync(ws, st);
    if (ef != hipSuccess && status == ATTN_OK) status = hip_fail(ef, "workspace release");
  }
  return status;
}

}  // namespace

extern "C" {

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, int B, int H, int Hkv, int Sq, int Skv, int d, float scale,
                     int causal, const int32_t* cu_seqlens, void* stream, const attn_opts* opts) {
  return backward(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, Sq, Skv, d, scale, causal, cu_seqlens, 0, nullptr,
                  nullptr, stream, opts, ATTN_BHSD);
}

attn_status attn_bwd_window_sink(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                 const float* lse, void* dq, void* dk, void* dv, float* dsinks, int B, int H, int Hkv,
                                 int Sq, int Skv, int d, float scale, const int32_t* cu_seqlens, int window,
                                 const float* sinks, void* stream, const attn_opts* opts) {
  return backward(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, Sq, Skv, d, scale, 1, cu_seqlens, window, sinks,
                  dsinks, stream, opts, ATTN_BHSD);
}

attn_status attn_bwd_layout(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, float* dsinks, int B, int H, int Hkv,
                            int Sq, int Skv, int d, float scale, int causal, const int32_t* cu_seqlens,
                            attn_layout layout, int window, const float* sinks, void* stream,
                            const attn_opts* opts) {
  g_err[0] = '\0';
  if ((window > 0 || sinks != nullptr) && !causal)
    return fail(ATTN_EINVAL, "a window or sinks need causal attention");
  return backward(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, Sq, Skv, d, scale, causal, cu_seqlens, window, sinks,
                  dsinks, stream, opts, layout);
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int Hkv, int Sq, int Skv, int d, float scale, int causal,
                     const int32_t* cu_seqlens, void* stream) {
  return attn_fwd_ex(q, k, v, o, lse, B, H, Hkv, Sq, Skv, d, scale, causal, cu_seqlens, stream,
                     ATTN_BF16, nullptr);
}

attn_status attn_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int H, int Hkv, int Sq, int Skv, int d, float scale, int causal,
                         const int32_t* cu_seqlens, void* stream) {
  return attn_fwd_ex(q, k, v, o, lse, B, H, Hkv, Sq, Skv, d, scale, causal, cu_seqlens, stream,
                     ATTN_F32, nullptr);
}

}  // extern "C"
