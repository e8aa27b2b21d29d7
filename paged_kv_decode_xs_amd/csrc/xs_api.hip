// C ABI of libxs.so: host-side argument checks, then one launch per call on the caller's stream.
// Every check here runs before any HIP call, so a rejected call touches no device state.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>
#include <vector>

#include "xs/xs.h"
#include "xs_internal.h"

#define XS_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return XS_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elt_bytes(int dtype) { return dtype == XS_BF16 ? 2 : 4; }

// Checks shared by the append and decode calls. `who` names the entry point in messages.
int check_pool_args(const char* who, int batch, int num_kv_heads, int head_dim, int block_size,
                    int max_blocks_per_seq, int num_blocks, int dtype) {
  if (batch < 0) return fail(XS_EINVAL, "%s: batch = %d < 0", who, batch);
  if (num_kv_heads < 1) return fail(XS_EINVAL, "%s: num_kv_heads = %d < 1", who, num_kv_heads);
  if (max_blocks_per_seq < 1) return fail(XS_EINVAL, "%s: max_blocks_per_seq = %d < 1", who, max_blocks_per_seq);
  if (num_blocks < 1) return fail(XS_EINVAL, "%s: num_blocks = %d < 1", who, num_blocks);
  if (dtype != XS_F32 && dtype != XS_BF16) return fail(XS_EUNSUPPORTED, "%s: dtype %d is not XS_F32 or XS_BF16", who, dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(XS_EUNSUPPORTED, "%s: head_dim = %d (supported: 64, 128)", who, head_dim);
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(XS_EUNSUPPORTED, "%s: block_size = %d (supported: 8, 16, 32)", who, block_size);
  if ((long long)max_blocks_per_seq * block_size > 0x7fffffffLL)
    return fail(XS_EINVAL, "%s: max_blocks_per_seq * block_size overflows int32", who);
  return XS_OK;
}

int launch_status(const char* who, hipError_t e) {
  if (e != hipSuccess) return fail(XS_ELAUNCH, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

}  // namespace

XS_API const char* xs_last_error(void) { return g_last_error.c_str(); }

XS_API int xs_version(void) { return 100; /* 0.1.0 */ }

XS_API int xs_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens, int batch, int num_kv_heads,
                        int head_dim, int block_size, int max_blocks_per_seq, int num_blocks, int dtype,
                        void* stream) {
  const char* who = "xs_kv_append";
  int st = check_pool_args(who, batch, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, dtype);
  if (st != XS_OK) return st;
  if (batch == 0) return ok();
  if (!k_new || !v_new || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(XS_EINVAL, "%s: a required pointer is NULL", who);
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(XS_EINVAL, "%s: k_new, v_new, k_cache and v_cache must be 16-byte aligned", who);
  if (2LL * batch * num_kv_heads * (head_dim * elt_bytes(dtype) / 16) > 0x7fffffffLL * 256LL)
    return fail(XS_EINVAL, "%s: batch * num_kv_heads too large", who);
  (void)hipGetLastError();  // clear a stale error so the status below is this launch's own
  return launch_status(who, xs::launch_kv_append(k_new, v_new, k_cache, v_cache, block_tables, context_lens, batch,
                                                 num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                                                 elt_bytes(dtype), static_cast<hipStream_t>(stream)));
}

namespace {

// Checks of a decode call (fused or not). Returns XS_OK, or the status of the first violation.
int check_decode(const char* who, const xs::DecodeArgs& a, int dtype) {
  int st = check_pool_args(who, a.batch, a.num_kv_heads, a.head_dim, a.block_size, a.max_blocks_per_seq,
                           a.num_blocks, dtype);
  if (st != XS_OK) return st;
  if (a.num_q_heads < 1) return fail(XS_EINVAL, "%s: num_q_heads = %d < 1", who, a.num_q_heads);
  if (a.num_q_heads % a.num_kv_heads != 0)
    return fail(XS_EINVAL, "%s: num_q_heads = %d is not a multiple of num_kv_heads = %d", who, a.num_q_heads,
                a.num_kv_heads);
  if (!isfinite(a.scale)) return fail(XS_EINVAL, "%s: scale is not finite", who);
  if (a.partition_size < 0) return fail(XS_EINVAL, "%s: partition_size = %d < 0", who, a.partition_size);
  const bool split = a.partition_size > 0;
  if (split) {
    if (a.partition_size % a.block_size != 0)
      return fail(XS_EINVAL, "%s: partition_size = %d is not a multiple of block_size = %d", who, a.partition_size,
                  a.block_size);
    if (a.max_partitions < 1)
      return fail(XS_EINVAL, "%s: max_partitions = %d < 1 with split-K", who, a.max_partitions);
  }
  const int group = a.num_q_heads / a.num_kv_heads;
  const int chunks = group / xs::heads_per_chunk(group);
  const long long grid = (long long)a.batch * a.num_kv_heads * chunks * (split ? a.max_partitions : 1);
  if (grid > 0x7fffffffLL) return fail(XS_EINVAL, "%s: %lld work items exceed the launch limit", who, grid);
  if (a.batch == 0) return XS_OK;
  if (!a.q || !a.k_cache || !a.v_cache || !a.block_tables || !a.context_lens)
    return fail(XS_EINVAL, "%s: a required pointer is NULL", who);
  if (split) {
    if (!a.part_o || !a.part_m || !a.part_l)
      return fail(XS_EINVAL, "%s: split-K (partition_size > 0) needs part_o, part_m and part_l", who);
    if (!aligned16(a.part_o)) return fail(XS_EINVAL, "%s: part_o must be 16-byte aligned", who);
  } else {
    if (!a.out) return fail(XS_EINVAL, "%s: out is NULL with partition_size == 0", who);
    if (a.part_o || a.part_m || a.part_l)
      return fail(XS_EINVAL, "%s: part_o/part_m/part_l must be NULL when partition_size == 0", who);
    if (!aligned16(a.out)) return fail(XS_EINVAL, "%s: out must be 16-byte aligned", who);
  }
  if (!aligned16(a.q) || !aligned16(a.k_cache) || !aligned16(a.v_cache))
    return fail(XS_EINVAL, "%s: q, k_cache and v_cache must be 16-byte aligned", who);
  return XS_OK;
}

xs::DecodeArgs decode_args(const void* q, const void* k_new, const void* v_new, const void* k_cache,
                           const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                           float scale, void* out, float* part_o, float* part_m, float* part_l, int batch,
                           int num_q_heads, int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                           int num_blocks, int partition_size, int max_partitions, int dtype) {
  xs::DecodeArgs a;
  a.q = q;
  a.k_cache = const_cast<void*>(k_cache);
  a.v_cache = const_cast<void*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.k_new = k_new;
  a.v_new = v_new;
  a.scale = scale;
  a.out = out;
  a.part_o = part_o;
  a.part_m = part_m;
  a.part_l = part_l;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.partition_size = partition_size;
  a.max_partitions = partition_size > 0 ? max_partitions : 1;
  a.bf16 = dtype == XS_BF16;
  return a;
}

}  // namespace

XS_API int xs_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                const int32_t* context_lens, float scale, void* out, float* part_o, float* part_m,
                                float* part_l, int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                int block_size, int max_blocks_per_seq, int num_blocks, int partition_size,
                                int max_partitions, int dtype, void* stream) {
  const char* who = "xs_paged_attn_decode";
  const xs::DecodeArgs a = decode_args(q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, scale, out,
                                       part_o, part_m, part_l, batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                       max_blocks_per_seq, num_blocks, partition_size, max_partitions, dtype);
  const int st = check_decode(who, a, dtype);
  if (st != XS_OK) return st;
  if (batch == 0) return ok();
  (void)hipGetLastError();
  return launch_status(who, xs::launch_paged_decode(a, static_cast<hipStream_t>(stream)));
}

XS_API int xs_paged_attn_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                       void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                       float scale, void* out, float* part_o, float* part_m, float* part_l, int batch,
                                       int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                       int max_blocks_per_seq, int num_blocks, int partition_size, int max_partitions,
                                       int dtype, void* stream) {
  const char* who = "xs_paged_attn_decode_append";
  const xs::DecodeArgs a = decode_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out,
                                       part_o, part_m, part_l, batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                       max_blocks_per_seq, num_blocks, partition_size, max_partitions, dtype);
  const int st = check_decode(who, a, dtype);
  if (st != XS_OK) return st;
  if (batch == 0) return ok();
  if (!k_new || !v_new) return fail(XS_EINVAL, "%s: k_new and v_new must not be NULL", who);
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(XS_EINVAL, "%s: k_new and v_new must be 16-byte aligned", who);
  (void)hipGetLastError();
  return launch_status(who, xs::launch_paged_decode(a, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------------------------------
// The decode step without a workspace argument: the split-K partials live in a file-scope
// device array. Each device holds its own copy of the array, at its own address; host code never
// passes the array's name to a kernel (on the host it is only a stand-in), only the device address
// that hipGetSymbolAddress gives for the current device, looked up once per device.

namespace {

static __device__ __align__(256) unsigned char scratch[XS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on that device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

XS_API int xs_paged_attn_decode_append_noalloc(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                               void* v_cache, const int32_t* block_tables,
                                               const int32_t* context_lens, float scale, void* out, int batch,
                                               int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                               int max_blocks_per_seq, int num_blocks, int partition_size,
                                               int max_partitions, int dtype, void* stream) {
  const char* who = "xs_paged_attn_decode_append_noalloc";
  // Checked as the split call with partials (stand-in pointers: the real ones come below).
  float* const stand_in = reinterpret_cast<float*>(static_cast<uintptr_t>(256));
  const bool split = partition_size > 0;
  xs::DecodeArgs a = decode_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                                 split ? nullptr : out, split ? stand_in : nullptr, split ? stand_in : nullptr,
                                 split ? stand_in : nullptr, batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                 max_blocks_per_seq, num_blocks, partition_size, max_partitions, dtype);
  const int st = check_decode(who, a, dtype);
  if (st != XS_OK) return st;
  if (batch == 0) return ok();
  if (!out || !aligned16(out)) return fail(XS_EINVAL, "%s: out must be a 16-byte aligned pointer", who);
  if (!k_new || !v_new) return fail(XS_EINVAL, "%s: k_new and v_new must not be NULL", who);
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(XS_EINVAL, "%s: k_new and v_new must be 16-byte aligned", who);
  a.out = out;
  size_t o_bytes = 0, ml_bytes = 0;
  if (split) {
    const size_t rows = (size_t)batch * num_q_heads * (size_t)max_partitions;
    o_bytes = align256(rows * head_dim * sizeof(float));
    ml_bytes = align256(rows * sizeof(float));
    const size_t need = o_bytes + 2 * ml_bytes;
    if (need > (size_t)XS_NOALLOC_SCRATCH_BYTES)
      return fail(XS_EINVAL,
                  "%s: the partials need %zu bytes (batch * num_q_heads * max_partitions * (head_dim + 2) * 4, "
                  "rounded); the scratch holds %zu: use xs_paged_attn_decode_append with caller buffers",
                  who, need, (size_t)XS_NOALLOC_SCRATCH_BYTES);
  }
  (void)hipGetLastError();
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!split) return launch_status(who, xs::launch_paged_decode(a, s));
  void* base = nullptr;
  const hipError_t e = scratch_address(&base);
  if (e != hipSuccess) return fail(XS_ELAUNCH, "%s: hipGetSymbolAddress: %s", who, hipGetErrorString(e));
  unsigned char* p = static_cast<unsigned char*>(base);
  a.part_o = reinterpret_cast<float*>(p);
  a.part_m = reinterpret_cast<float*>(p + o_bytes);
  a.part_l = reinterpret_cast<float*>(p + o_bytes + ml_bytes);
  hipError_t le = xs::launch_paged_decode(a, s);
  if (le == hipSuccess)
    le = xs::launch_paged_reduce(a.part_o, a.part_m, a.part_l, context_lens, out, batch, num_q_heads, head_dim,
                                 partition_size, a.max_partitions, a.bf16, s);
  return launch_status(who, le);
}

XS_API int xs_paged_attn_decode_sinks(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                      void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                      const void* sinks, int window_size, float scale, void* out, float* part_o,
                                      float* part_m, float* part_l, int batch, int num_q_heads, int num_kv_heads,
                                      int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                                      int partition_size, int max_partitions, int dtype, void* stream) {
  const char* who = "xs_paged_attn_decode_sinks";
  xs::DecodeArgs a = decode_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out, part_o,
                                 part_m, part_l, batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                 max_blocks_per_seq, num_blocks, partition_size, max_partitions, dtype);
  a.sinks = sinks;
  a.window = window_size;
  const int st = check_decode(who, a, dtype);
  if (st != XS_OK) return st;
  if (dtype != XS_BF16) return fail(XS_EUNSUPPORTED, "%s: sinks and windows need dtype XS_BF16", who);
  if (!xs::mfma_decode_supported(true, head_dim, block_size))
    return fail(XS_EUNSUPPORTED, "%s: block_size = %d (supported with sinks and windows: 16, 32)", who, block_size);
  if (window_size < 0) return fail(XS_EINVAL, "%s: window_size = %d < 0", who, window_size);
  if (batch == 0) return ok();
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(XS_EINVAL, "%s: k_new and v_new must both be given (fused append) or both be NULL", who);
  if (k_new && (!aligned16(k_new) || !aligned16(v_new)))
    return fail(XS_EINVAL, "%s: k_new and v_new must be 16-byte aligned", who);
  if (sinks && (reinterpret_cast<uintptr_t>(sinks) & 1u)) return fail(XS_EINVAL, "%s: sinks must be 2-byte aligned", who);
  (void)hipGetLastError();
  return launch_status(who, xs::launch_paged_decode(a, static_cast<hipStream_t>(stream)));
}

XS_API int xs_paged_attn_reduce_sinks(const float* part_o, const float* part_m, const float* part_l,
                                      const int32_t* context_lens, const void* sinks, int window_size, void* out,
                                      int batch, int num_q_heads, int head_dim, int partition_size,
                                      int max_partitions, int dtype, void* stream) {
  const char* who = "xs_paged_attn_reduce_sinks";
  if (batch < 0) return fail(XS_EINVAL, "%s: batch = %d < 0", who, batch);
  if (num_q_heads < 1) return fail(XS_EINVAL, "%s: num_q_heads = %d < 1", who, num_q_heads);
  if (dtype != XS_BF16) return fail(XS_EUNSUPPORTED, "%s: sinks and windows need dtype XS_BF16", who);
  if (head_dim != 64 && head_dim != 128)
    return fail(XS_EUNSUPPORTED, "%s: head_dim = %d (supported: 64, 128)", who, head_dim);
  if (partition_size < 1) return fail(XS_EINVAL, "%s: partition_size = %d < 1", who, partition_size);
  if (max_partitions < 1) return fail(XS_EINVAL, "%s: max_partitions = %d < 1", who, max_partitions);
  if (window_size < 0) return fail(XS_EINVAL, "%s: window_size = %d < 0", who, window_size);
  if ((long long)batch * num_q_heads > 0x7fffffffLL) return fail(XS_EINVAL, "%s: batch * num_q_heads too large", who);
  if (batch == 0) return ok();
  if (!part_o || !part_m || !part_l || !context_lens || !out)
    return fail(XS_EINVAL, "%s: a required pointer is NULL", who);
  if (!aligned16(part_o) || !aligned16(out)) return fail(XS_EINVAL, "%s: part_o and out must be 16-byte aligned", who);
  if (sinks && (reinterpret_cast<uintptr_t>(sinks) & 1u)) return fail(XS_EINVAL, "%s: sinks must be 2-byte aligned", who);
  (void)hipGetLastError();
  return launch_status(who, xs::launch_paged_reduce_sinks(part_o, part_m, part_l, context_lens, sinks, window_size, out,
                                                          batch, num_q_heads, head_dim, partition_size,
                                                          max_partitions, true, static_cast<hipStream_t>(stream)));
}

XS_API int xs_paged_attn_reduce(const float* part_o, const float* part_m, const float* part_l,
                                const int32_t* context_lens, void* out, int batch, int num_q_heads, int head_dim,
                                int partition_size, int max_partitions, int dtype, void* stream) {
  const char* who = "xs_paged_attn_reduce";
  if (batch < 0) return fail(XS_EINVAL, "%s: batch = %d < 0", who, batch);
  if (num_q_heads < 1) return fail(XS_EINVAL, "%s: num_q_heads = %d < 1", who, num_q_heads);
  if (dtype != XS_F32 && dtype != XS_BF16) return fail(XS_EUNSUPPORTED, "%s: dtype %d is not XS_F32 or XS_BF16", who, dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(XS_EUNSUPPORTED, "%s: head_dim = %d (supported: 64, 128)", who, head_dim);
  if (partition_size < 1) return fail(XS_EINVAL, "%s: partition_size = %d < 1", who, partition_size);
  if (max_partitions < 1) return fail(XS_EINVAL, "%s: max_partitions = %d < 1", who, max_partitions);
  if ((long long)batch * num_q_heads > 0x7fffffffLL) return fail(XS_EINVAL, "%s: batch * num_q_heads too large", who);
  if (batch == 0) return ok();
  if (!part_o || !part_m || !part_l || !context_lens || !out)
    return fail(XS_EINVAL, "%s: a required pointer is NULL", who);
  if (!aligned16(part_o) || !aligned16(out)) return fail(XS_EINVAL, "%s: part_o and out must be 16-byte aligned", who);
  (void)hipGetLastError();
  return launch_status(who, xs::launch_paged_reduce(part_o, part_m, part_l, context_lens, out, batch, num_q_heads,
                                                    head_dim, partition_size, max_partitions, dtype == XS_BF16,
                                                    static_cast<hipStream_t>(stream)));
}

XS_API int xs_stream_read_probe(const void* buf, size_t bytes, unsigned* sink, int nontemporal, int shape,
                                void* stream) {
  const char* who = "xs_stream_read_probe";
  if (!buf || !sink) return fail(XS_EINVAL, "%s: buf and sink must not be NULL", who);
  if (!aligned16(buf) || bytes % 16 != 0) return fail(XS_EINVAL, "%s: buf must be 16-byte aligned and bytes a multiple of 16", who);
  if (shape != 0 && shape != 1) return fail(XS_EINVAL, "%s: shape = %d (0 or 1)", who, shape);
  if (bytes == 0) return ok();
  (void)hipGetLastError();
  return launch_status(who, xs::launch_stream_read(buf, bytes, sink, nontemporal != 0, shape,
                                                   static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------------------------------
// Decode step as one HIP graph (captured once, replayed per step).

struct xs_step_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

namespace {

// Enqueues one decode step on `s`: the append (fused into the decode, or its own kernel), the
// decode, and the reduce when split. The arguments were checked by the caller.
hipError_t enqueue_step(const xs::DecodeArgs& a, const xs_step_desc* d, hipStream_t s) {
  hipError_t e;
  const bool sw = a.sinks != nullptr || a.window > 0;
  if (d->fused) {
    e = xs::launch_paged_decode(a, s);
  } else {
    e = xs::launch_kv_append(d->k_new, d->v_new, d->k_cache, d->v_cache, d->block_tables, d->context_lens, d->batch,
                             d->num_kv_heads, d->head_dim, d->block_size, d->max_blocks_per_seq, d->num_blocks,
                             elt_bytes(d->dtype), s);
    if (e != hipSuccess) return e;
    xs::DecodeArgs b = a;
    b.k_new = b.v_new = nullptr;
    e = xs::launch_paged_decode(b, s);
  }
  if (e != hipSuccess || a.partition_size == 0) return e;
  if (sw)
    return xs::launch_paged_reduce_sinks(a.part_o, a.part_m, a.part_l, a.context_lens, a.sinks, a.window, a.out,
                                         a.batch, a.num_q_heads, a.head_dim, a.partition_size, a.max_partitions,
                                         a.bf16, s);
  return xs::launch_paged_reduce(a.part_o, a.part_m, a.part_l, a.context_lens, a.out, a.batch, a.num_q_heads,
                                 a.head_dim, a.partition_size, a.max_partitions, a.bf16, s);
}

}  // namespace

namespace {

// Checks one step descriptor; builds its DecodeArgs.
int check_step(const char* who, int idx, const xs_step_desc* d, xs::DecodeArgs* out_args) {
  xs::DecodeArgs a = decode_args(d->q, d->k_new, d->v_new, d->k_cache, d->v_cache, d->block_tables,
                                 d->context_lens, d->scale, d->partition_size > 0 ? nullptr : d->out, d->part_o,
                                 d->part_m, d->part_l, d->batch, d->num_q_heads, d->num_kv_heads, d->head_dim,
                                 d->block_size, d->max_blocks_per_seq, d->num_blocks, d->partition_size,
                                 d->max_partitions, d->dtype);
  a.sinks = d->sinks;
  a.window = d->window_size;
  int st = check_decode(who, a, d->dtype);
  if (st != XS_OK) return st;
  a.out = d->out;  // the reduce's output when split
  if (d->batch < 1) return fail(XS_EINVAL, "%s: step %d: batch = %d < 1 (nothing to capture)", who, idx, d->batch);
  if (!d->k_new || !d->v_new)
    return fail(XS_EINVAL, "%s: step %d: the step appends: k_new and v_new are required", who, idx);
  if (!aligned16(d->k_new) || !aligned16(d->v_new))
    return fail(XS_EINVAL, "%s: step %d: k_new and v_new must be 16-byte aligned", who, idx);
  if (d->partition_size > 0 && (!d->out || !aligned16(d->out)))
    return fail(XS_EINVAL, "%s: step %d: out (the reduce's output) must be a 16-byte aligned pointer", who, idx);
  if (d->window_size < 0) return fail(XS_EINVAL, "%s: step %d: window_size = %d < 0", who, idx, d->window_size);
  if (d->sinks || d->window_size > 0) {
    if (d->dtype != XS_BF16)
      return fail(XS_EUNSUPPORTED, "%s: step %d: sinks and windows need dtype XS_BF16", who, idx);
    if (!xs::mfma_decode_supported(true, d->head_dim, d->block_size))
      return fail(XS_EUNSUPPORTED, "%s: step %d: block_size = %d (supported with sinks and windows: 16, 32)", who,
                  idx, d->block_size);
    if (d->sinks && (reinterpret_cast<uintptr_t>(d->sinks) & 1u))
      return fail(XS_EINVAL, "%s: step %d: sinks must be 2-byte aligned", who, idx);
  }
  *out_args = a;
  return XS_OK;
}

}  // namespace

XS_API int xs_step_graph_create(const xs_step_desc* descs, int num_steps, xs_step_graph** out_graph) {
  const char* who = "xs_step_graph_create";
  if (!out_graph) return fail(XS_EINVAL, "%s: out_graph is NULL", who);
  *out_graph = nullptr;
  if (!descs) return fail(XS_EINVAL, "%s: descs is NULL", who);
  if (num_steps < 1 || num_steps > 4096) return fail(XS_EINVAL, "%s: num_steps = %d (1..4096)", who, num_steps);
  std::vector<xs::DecodeArgs> args((size_t)num_steps);
  for (int i = 0; i < num_steps; ++i) {
    const int st = check_step(who, i, &descs[i], &args[(size_t)i]);
    if (st != XS_OK) return st;
  }
  (void)hipGetLastError();
  hipStream_t s = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (e != hipSuccess) return fail(XS_ELAUNCH, "%s: hipStreamCreateWithFlags: %s", who, hipGetErrorString(e));
  hipGraph_t graph = nullptr;
  e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    hipError_t le = hipSuccess;
    for (int i = 0; i < num_steps && le == hipSuccess; ++i) le = enqueue_step(args[(size_t)i], &descs[i], s);
    e = hipStreamEndCapture(s, &graph);  // always end the capture, even after a failed launch
    if (le != hipSuccess) e = le;
  }
  hipGraphExec_t exec = nullptr;
  if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipStreamDestroy(s);
  if (e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    return fail(XS_ELAUNCH, "%s: capture failed: %s", who, hipGetErrorString(e));
  }
  *out_graph = new xs_step_graph{graph, exec};
  return ok();
}

XS_API int xs_step_graph_launch(xs_step_graph* g, void* stream) {
  const char* who = "xs_step_graph_launch";
  if (!g) return fail(XS_EINVAL, "%s: graph is NULL", who);
  (void)hipGetLastError();
  return launch_status(who, hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)));
}

XS_API int xs_step_graph_destroy(xs_step_graph* g) {
  if (!g) return ok();
  const hipError_t e1 = hipGraphExecDestroy(g->exec);
  const hipError_t e2 = hipGraphDestroy(g->graph);
  delete g;
  if (e1 != hipSuccess || e2 != hipSuccess)
    return fail(XS_ELAUNCH, "xs_step_graph_destroy: %s", hipGetErrorString(e1 != hipSuccess ? e1 : e2));
  return ok();
}

// ------------------------------------------------------------------------------------------
// KV block swap between the pools and pinned host memory.

namespace {

// The device address of pinned host memory at `p` (NULL if `p` is not pinned host memory).
void* host_device_pointer(const void* p) {
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return d;
}

int swap_call(const char* who, bool out, const void* pool_k, const void* pool_v, const void* host_k,
              const void* host_v, const int32_t* src_idx, const int32_t* dst_idx, int num_pairs, int num_blocks,
              int num_slots, int num_kv_heads, int block_size, int head_dim, int dtype, void* stream) {
  if (num_pairs < 0) return fail(XS_EINVAL, "%s: num_pairs = %d < 0", who, num_pairs);
  if (num_blocks < 1 || num_slots < 1 || num_kv_heads < 1 || block_size < 1 || head_dim < 1)
    return fail(XS_EINVAL, "%s: num_blocks, num_slots, num_kv_heads, block_size and head_dim must be >= 1", who);
  if (dtype != XS_F32 && dtype != XS_BF16) return fail(XS_EUNSUPPORTED, "%s: dtype %d is not XS_F32 or XS_BF16", who, dtype);
  const size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * elt_bytes(dtype);
  if (block_bytes % 16 != 0) return fail(XS_EINVAL, "%s: a block (%zu bytes) is not a multiple of 16 bytes", who, block_bytes);
  if (block_bytes / 16 > 0x7fffffffULL) return fail(XS_EINVAL, "%s: blocks too large", who);
  if (num_pairs == 0) return ok();
  if (!pool_k || !pool_v || !host_k || !host_v || !src_idx || !dst_idx)
    return fail(XS_EINVAL, "%s: a required pointer is NULL", who);
  if (!aligned16(pool_k) || !aligned16(pool_v) || !aligned16(host_k) || !aligned16(host_v))
    return fail(XS_EINVAL, "%s: pools and host buffers must be 16-byte aligned", who);
  void* dk = host_device_pointer(host_k);
  void* dv = host_device_pointer(host_v);
  if (!dk || !dv) return fail(XS_EINVAL, "%s: k_host and v_host must be pinned host memory (hipHostMalloc)", who);
  (void)hipGetLastError();
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = out ? xs::launch_kv_swap(pool_k, pool_v, dk, dv, src_idx, dst_idx, num_pairs, num_blocks, num_slots,
                                          block_bytes, s)
                     : xs::launch_kv_swap(dk, dv, const_cast<void*>(pool_k), const_cast<void*>(pool_v), src_idx,
                                          dst_idx, num_pairs, num_slots, num_blocks, block_bytes, s);
  return launch_status(who, e);
}

}  // namespace

XS_API int xs_kv_swap_out(const void* k_cache, const void* v_cache, void* k_host, void* v_host,
                          const int32_t* src_blocks, const int32_t* dst_slots, int num_pairs, int num_blocks,
                          int num_slots, int num_kv_heads, int block_size, int head_dim, int dtype, void* stream) {
  return swap_call("xs_kv_swap_out", true, k_cache, v_cache, k_host, v_host, src_blocks, dst_slots, num_pairs,
                   num_blocks, num_slots, num_kv_heads, block_size, head_dim, dtype, stream);
}

XS_API int xs_kv_swap_in(const void* k_host, const void* v_host, void* k_cache, void* v_cache,
                         const int32_t* src_slots, const int32_t* dst_blocks, int num_pairs, int num_blocks,
                         int num_slots, int num_kv_heads, int block_size, int head_dim, int dtype, void* stream) {
  return swap_call("xs_kv_swap_in", false, k_cache, v_cache, k_host, v_host, src_slots, dst_blocks, num_pairs,
                   num_blocks, num_slots, num_kv_heads, block_size, head_dim, dtype, stream);
}

// ------------------------------------------------------------------------------------------
// Chunked prefill: multi-token append and causal attention of the chunk.

XS_API int xs_kv_append_chunk(const void* k_src, const void* v_src, void* k_cache, void* v_cache,
                              const int32_t* block_tables, const int32_t* start_pos, const int32_t* chunk_lens,
                              int batch, int num_kv_heads, int head_dim, int chunk_size, int block_size,
                              int max_blocks_per_seq, int num_blocks, int dtype, void* stream) {
  const char* who = "xs_kv_append_chunk";
  int st = check_pool_args(who, batch, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, dtype);
  if (st != XS_OK) return st;
  if (chunk_size < 0) return fail(XS_EINVAL, "%s: chunk_size = %d < 0", who, chunk_size);
  if (batch == 0 || chunk_size == 0) return ok();
  if (!k_src || !v_src || !k_cache || !v_cache || !block_tables || !start_pos || !chunk_lens)
    return fail(XS_EINVAL, "%s: a required pointer is NULL", who);
  if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(XS_EINVAL, "%s: k_src, v_src, k_cache and v_cache must be 16-byte aligned", who);
  if (2LL * batch * num_kv_heads * chunk_size * (head_dim * elt_bytes(dtype) / 16) > 0x7fffffffLL * 256LL)
    return fail(XS_EINVAL, "%s: batch * num_kv_heads * chunk_size too large", who);
  (void)hipGetLastError();
  return launch_status(who, xs::launch_kv_append_chunk(k_src, v_src, k_cache, v_cache, block_tables, start_pos,
                                                       chunk_lens, batch, num_kv_heads, head_dim, chunk_size,
                                                       block_size, max_blocks_per_seq, num_blocks, elt_bytes(dtype),
                                                       static_cast<hipStream_t>(stream)));
}

static int prefill_common(const char* who, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* start_pos, const int32_t* chunk_lens,
                          float scale, void* out, float* part_o, float* part_ml, int batch, int num_q_heads,
                          int num_kv_heads, int head_dim, int chunk_size, int block_size, int max_blocks_per_seq,
                          int num_blocks, int partition_size, int max_partitions, int dtype, void* stream,
                          const void* sinks = nullptr, int window = 0) {
  int st = check_pool_args(who, batch, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, dtype);
  if (st != XS_OK) return st;
  if (dtype != XS_BF16) return fail(XS_EUNSUPPORTED, "%s: only XS_BF16 is implemented", who);
  if (num_q_heads < 1) return fail(XS_EINVAL, "%s: num_q_heads = %d < 1", who, num_q_heads);
  if (num_q_heads % num_kv_heads != 0)
    return fail(XS_EINVAL, "%s: num_q_heads = %d is not a multiple of num_kv_heads = %d", who, num_q_heads,
                num_kv_heads);
  if (chunk_size < 0) return fail(XS_EINVAL, "%s: chunk_size = %d < 0", who, chunk_size);
  if (!isfinite(scale)) return fail(XS_EINVAL, "%s: scale is not finite", who);
  if (window < 0) return fail(XS_EINVAL, "%s: window_size = %d < 0", who, window);
  const int group = num_q_heads / num_kv_heads;
  if ((long long)chunk_size * group > 0x7fffffffLL - 64)
    return fail(XS_EINVAL, "%s: chunk_size * (num_q_heads / num_kv_heads) too large", who);
  const bool split = partition_size != 0;
  if (split) {
    if (partition_size < 0 || partition_size % 64 != 0)
      return fail(XS_EINVAL, "%s: partition_size = %d is not a positive multiple of 64", who, partition_size);
    const long long need = ((long long)max_blocks_per_seq * block_size + partition_size - 1) / partition_size;
    if (max_partitions < need)
      return fail(XS_EINVAL, "%s: max_partitions = %d < %lld (max_blocks_per_seq * block_size / partition_size)",
                  who, max_partitions, need);
  }
  if (batch == 0 || chunk_size == 0) return ok();
  const long long grid =
      (long long)batch * num_kv_heads * xs::prefill_row_blocks(chunk_size, group) * (split ? max_partitions : 1);
  if (grid > 0x7fffffffLL) return fail(XS_EINVAL, "%s: %lld workgroups exceed the launch limit", who, grid);
  if (split && ((long long)batch * num_q_heads * chunk_size + 3) / 2 > 0x7fffffffLL)
    return fail(XS_EINVAL, "%s: batch * num_q_heads * chunk_size too large", who);
  if (!q || !k_cache || !v_cache || !block_tables || !start_pos || !chunk_lens || !out)
    return fail(XS_EINVAL, "%s: a required pointer is NULL", who);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(XS_EINVAL, "%s: q, k_cache, v_cache and out must be 16-byte aligned", who);
  if (split && (!part_o || !part_ml)) return fail(XS_EINVAL, "%s: part_o and part_ml are required", who);
  if (split && (!aligned16(part_o) || reinterpret_cast<uintptr_t>(part_ml) % 8 != 0))
    return fail(XS_EINVAL, "%s: part_o must be 16-byte and part_ml 8-byte aligned", who);
  if (sinks && (reinterpret_cast<uintptr_t>(sinks) & 1u)) return fail(XS_EINVAL, "%s: sinks must be 2-byte aligned", who);
  xs::PrefillArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.start_pos = start_pos;
  a.chunk_lens = chunk_lens;
  a.scale = scale;
  a.out = out;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.chunk = chunk_size;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  if (split) {
    a.part_o = part_o;
    a.part_ml = part_ml;
    a.partition_size = partition_size;
    a.max_partitions = max_partitions;
  }
  a.sinks = sinks;
  a.window = window;
  (void)hipGetLastError();
  return launch_status(who, xs::launch_paged_prefill(a, static_cast<hipStream_t>(stream)));
}

XS_API int xs_paged_attn_prefill(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* start_pos, const int32_t* chunk_lens,
                                 float scale, void* out, int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                 int chunk_size, int block_size, int max_blocks_per_seq, int num_blocks, int dtype,
                                 void* stream) {
  return prefill_common("xs_paged_attn_prefill", q, k_cache, v_cache, block_tables, start_pos, chunk_lens, scale,
                        out, nullptr, nullptr, batch, num_q_heads, num_kv_heads, head_dim, chunk_size, block_size,
                        max_blocks_per_seq, num_blocks, 0, 0, dtype, stream);
}

XS_API int xs_paged_attn_prefill_split(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* start_pos,
                                       const int32_t* chunk_lens, float scale, void* out, float* part_o,
                                       float* part_ml, int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                       int chunk_size, int block_size, int max_blocks_per_seq, int num_blocks,
                                       int partition_size, int max_partitions, int dtype, void* stream) {
  const char* who = "xs_paged_attn_prefill_split";
  if (partition_size == 0) return fail(XS_EINVAL, "%s: partition_size = 0 (use xs_paged_attn_prefill)", who);
  return prefill_common(who, q, k_cache, v_cache, block_tables, start_pos, chunk_lens, scale, out, part_o, part_ml,
                        batch, num_q_heads, num_kv_heads, head_dim, chunk_size, block_size, max_blocks_per_seq,
                        num_blocks, partition_size, max_partitions, dtype, stream);
}

XS_API int xs_paged_attn_prefill_sinks(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* start_pos,
                                       const int32_t* chunk_lens, const void* sinks, int window_size, float scale,
                                       void* out, float* part_o, float* part_ml, int batch, int num_q_heads,
                                       int num_kv_heads, int head_dim, int chunk_size, int block_size,
                                       int max_blocks_per_seq, int num_blocks, int partition_size,
                                       int max_partitions, int dtype, void* stream) {
  return prefill_common("xs_paged_attn_prefill_sinks", q, k_cache, v_cache, block_tables, start_pos, chunk_lens,
                        scale, out, part_o, part_ml, batch, num_q_heads, num_kv_heads, head_dim, chunk_size,
                        block_size, max_blocks_per_seq, num_blocks, partition_size, max_partitions, dtype, stream,
                        sinks, window_size);
}
