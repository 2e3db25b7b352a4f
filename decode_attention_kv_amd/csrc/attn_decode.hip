// Entry points of libattn_decode: argument checks, parameter blocks, kernel
// choice and launches of the decode kernels (attn_general.hip,
// attn_narrow.hip, attn_wide.hip) and of the split merge defined here.
//
// Decode attention over a paged KV cache ("Hardware-Efficient Attention for
// Fast Decoding"): each work item of the host plan covers a sequence, a
// group (KV head or latent head) and a chunk of its tokens; sequences split
// into several chunks are merged through their softmax denominators
// (Hydragen's decomposition on the "Efficient Inference" tag page).
#include "attn_device.h"

#include <algorithm>
#include <atomic>
#include <mutex>

namespace attn_dev {
namespace {


// ----------------------------------------------------------------------------
// Merge the split partials of every sequence with n_splits > 1.
// grid (ceil(q_len*h_q / rows_per_block), batch); DV/4 threads per row.
template <typename T, int DV>
__global__ __launch_bounds__(256) void combine_kernel(Params p) {
  constexpr int TPR = DV / 4;
  constexpr int RPB = 256 / TPR;
  const float* __restrict__ o_part = p.o_part;
  const float* __restrict__ lse_part = p.lse_part;
  T* __restrict__ out = static_cast<T*>(p.out);
  float* __restrict__ lse = p.lse;
  const int rows_total = p.q_len * p.h_q;
  const int b = blockIdx.y;
  int n, base, L_unused, chunk_unused;
  seq_info(p, b, n, base, L_unused, chunk_unused);
  if (n <= 1) return;
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= rows_total) return;
  const int c4 = (threadIdx.x % TPR) * 4;
  // the first NB splits' partials are loaded at once (one memory round
  // trip); the arithmetic runs in split order as below
  constexpr int NB = 4;
  float ls[NB];
  f32x4 os[NB];
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    if (s < n) {
      const int64_t pr = (int64_t)(base + s) * rows_total + row;
      ls[s] = lse_part[pr];
      os[s] = *reinterpret_cast<const f32x4*>(o_part + pr * DV + c4);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < NB; ++s)
    if (s < n) M = fmaxf(M, ls[s]);
  for (int s = NB; s < n; ++s) M = fmaxf(M, lse_part[(int64_t)(base + s) * rows_total + row]);
  const float Ms = (M == -INFINITY) ? 0.f : M;
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    if (s < n) {
      const float w = __expf(ls[s] - Ms);
      W += w;
      a += w * os[s];
    }
  }
  for (int s = NB; s < n; ++s) {
    const int64_t pr = (int64_t)(base + s) * rows_total + row;
    const float w = __expf(lse_part[pr] - Ms);
    W += w;
    a += w * *reinterpret_cast<const f32x4*>(o_part + pr * DV + c4);
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  const int64_t orow = (int64_t)b * rows_total + row;
  if constexpr (sizeof(T) == 2) {
    __bf16 v4[4] = {(__bf16)(a[0] * inv), (__bf16)(a[1] * inv), (__bf16)(a[2] * inv),
                    (__bf16)(a[3] * inv)};
    *reinterpret_cast<uint2*>(out + orow * DV + c4) = __builtin_bit_cast(uint2, v4);
  } else {
    *reinterpret_cast<f32x4*>(out + orow * DV + c4) = a * inv;
  }
  if (lse && c4 == 0) lse[orow] = W > 0.f ? Ms + __logf(W) : -INFINITY;
}

// ----------------------------------------------------------------------------
// host side
bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// workgroups of `per_cu` per CU the current device keeps resident
int resident_slots(int per_cu) {
  // looked up once per device; calls from several host threads may race to
  // store the same value
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n * per_cu;
}

// the plan's device arrays, or a plan to pass in the launch arguments
bool plan_on_device(const attn_plan_t* plan) { return plan->items && plan->seqinfo; }
// The launch-argument form of a host plan: 0 (none), 1 (an int32 per
// chunk) or 2 (half an int32 per chunk).
int inline_form(const attn_plan_t* plan) {
  if (plan->items || plan->seqinfo || !plan->inline_ok || !plan->items_host ||
      !plan->seqinfo_host || plan->n_groups <= 0 || plan->batch >= 65536)
    return 0;
  // the packed fields: split count and chunk length in tiles, 16 bits each
  int max_splits = 1;
  for (int b = 0; b < plan->batch; ++b) {
    const int32_t* si = plan->seqinfo_host + 4 * (int64_t)b;
    if (si[0] < 1 || si[0] >= 65536 || si[3] <= 0 || si[3] % 64 || (si[3] >> 6) >= 65536)
      return 0;
    max_splits = std::max(max_splits, (int)si[0]);
  }
  const int64_t chunks = plan->n_items / plan->n_groups;
  const bool half = plan->batch <= 2048 && max_splits <= 32;
  if (3 * (int64_t)plan->batch + (half ? (chunks + 1) / 2 : chunks) > ATTN_PLAN_INLINE_MAX)
    return 0;
  return half ? 2 : 1;
}
bool plan_inline(const attn_plan_t* plan) { return inline_form(plan) != 0; }
// compact copy of a host plan into the launch arguments: per sequence
// n_splits | (chunk / 64) << 16, the partial slot base and L; per chunk
// b | split << 16 (form 1), or b | split << 11 in 16 bits, two per int32
// (form 2)
void pack_inline(Params& p, const attn_plan_t* plan) {
  const int form = inline_form(plan);
  p.plan_inline = form;
  p.inl_batch = plan->batch;
  for (int b = 0; b < plan->batch; ++b) {
    const int32_t* si = plan->seqinfo_host + 4 * (int64_t)b;
    p.inl[3 * b + 0] = (int32_t)((uint32_t)si[0] | ((uint32_t)(si[3] >> 6) << 16));
    p.inl[3 * b + 1] = si[1];
    p.inl[3 * b + 2] = si[2];
  }
  const int g = plan->n_groups;
  const int n_chunks = plan->n_items / g;
  int32_t* const ce = p.inl + 3 * plan->batch;
  if (form == 2) {
    for (int w = 0; w < (n_chunks + 1) / 2; ++w) ce[w] = 0;
    for (int c = 0; c < n_chunks; ++c) {
      const int32_t* it = plan->items_host + 4 * (int64_t)c * g;
      const uint32_t e = (uint32_t)it[0] | ((uint32_t)it[2] << 11);
      ce[c >> 1] = (int32_t)((uint32_t)ce[c >> 1] | (e << (16 * (c & 1))));
    }
  } else {
    for (int c = 0; c < n_chunks; ++c) {
      const int32_t* it = plan->items_host + 4 * (int64_t)c * g;
      ce[c] = (int32_t)((uint32_t)it[0] | ((uint32_t)it[2] << 16));
    }
  }
}

int ilog2_pow2(int v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

// The decode kernels take every sequence's length, split count and chunk
// from the plan (its device arrays are copies of the host arrays, or the
// host arrays travel in the launch arguments), not from kv->seqlens.  So the
// host arrays are checked before any launch: every length fits the page
// table's row (capacity = max_pages_per_seq * page_size) and, for causal
// calls, holds at least q_len keys; the chunks cover it; split partial
// slots stay inside the plan's count; every item names a real sequence,
// group and split with its chunk's first token.
int check_plan(const attn_plan_t* plan, int64_t capacity, int min_len) {
  if (!plan->seqinfo_host || !plan->items_host) return ATTN_ERR_INVALID_ARG;
  for (int b = 0; b < plan->batch; ++b) {
    const int32_t* si = plan->seqinfo_host + 4 * (int64_t)b;
    const int64_t n = si[0], base = si[1], L = si[2], chunk = si[3];
    if (n < 1 || L < 0 || L > capacity || L < min_len || chunk <= 0 || n * chunk < L)
      return ATTN_ERR_INVALID_ARG;
    if (n > 1 && (base < 0 || base + n > plan->n_partial_slots)) return ATTN_ERR_INVALID_ARG;
  }
  for (int64_t k = 0; k < plan->n_items; ++k) {
    const int32_t* it = plan->items_host + 4 * k;
    if (it[0] < 0 || it[0] >= plan->batch || it[1] != k % plan->n_groups) return ATTN_ERR_INVALID_ARG;
    const int32_t* si = plan->seqinfo_host + 4 * (int64_t)it[0];
    if (it[2] < 0 || it[2] >= si[0] || (int64_t)it[3] != (int64_t)it[2] * si[3])
      return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

int validate(const attn_paged_kv_t* kv, const void* q, const void* out, int q_len, int h_q,
             int groups, int flags, const attn_plan_t* plan, bool need_pool1, bool need_rope) {
  if (!kv || !q || !out || !plan) return ATTN_ERR_INVALID_ARG;
  if (!kv->pool0 || !kv->page_table || !kv->seqlens) return ATTN_ERR_INVALID_ARG;
  if (need_pool1 && !kv->pool1) return ATTN_ERR_INVALID_ARG;
  if (need_rope && !kv->rope_pool) return ATTN_ERR_INVALID_ARG;
  if (plan->n_items <= 0) return ATTN_ERR_INVALID_ARG;
  if (!plan_on_device(plan) && !plan_inline(plan)) return ATTN_ERR_INVALID_ARG;
  if (kv->batch <= 0 || kv->batch != plan->batch || plan->n_groups != groups ||
      plan->q_len != q_len)
    return ATTN_ERR_INVALID_ARG;
  if (q_len < 1 || q_len > 16 || h_q <= 0 || groups <= 0 || h_q % groups) return ATTN_ERR_INVALID_ARG;
  if (flags & ~(ATTN_CAUSAL | ATTN_DEFER_MERGE)) return ATTN_ERR_INVALID_ARG;
  if (kv->max_pages_per_seq <= 0 || kv->num_pages <= 0) return ATTN_ERR_INVALID_ARG;
  if (ilog2_pow2(kv->page_size) < 0) return ATTN_ERR_INVALID_ARG;
  if (kv->dtype != ATTN_BF16 && kv->dtype != ATTN_FP32) return ATTN_ERR_INVALID_ARG;
  const int es = kv->dtype == ATTN_BF16 ? 2 : 4;
  if (!aligned16(kv->pool0) || (kv->pool1 && !aligned16(kv->pool1)) ||
      (kv->rope_pool && !aligned16(kv->rope_pool)) || !aligned16(q) || !aligned16(out))
    return ATTN_ERR_INVALID_ARG;
  if ((kv->page_stride * es) % 16 || (kv->token_stride * es) % 16 || (kv->head_stride * es) % 16)
    return ATTN_ERR_INVALID_ARG;
  if (kv->token_stride < 0 || kv->page_stride < 0 || kv->head_stride < 0)
    return ATTN_ERR_INVALID_ARG;
  if (need_rope) {
    if ((kv->rope_page_stride * es) % 16 || (kv->rope_token_stride * es) % 16)
      return ATTN_ERR_INVALID_ARG;
    if (kv->rope_token_stride < 0 || kv->rope_page_stride < 0) return ATTN_ERR_INVALID_ARG;
  }
  return check_plan(plan, (int64_t)kv->max_pages_per_seq * kv->page_size,
                    (flags & ATTN_CAUSAL) && q_len > 1 ? q_len : 0);
}

// the caller's workspace: large enough for the plan and 256-byte aligned
int check_workspace(const attn_plan_t* plan, int h_q, int d_v, const void* ws, size_t ws_bytes) {
  const size_t need = attn_decode_workspace_size(plan, h_q, d_v);
  if (need > 0 && (!ws || ws_bytes < need || ((uintptr_t)ws & 255u))) return ATTN_ERR_WORKSPACE;
  return ATTN_OK;
}

void set_partials(Params& p, const attn_plan_t* plan, const void* ws, int q_len, int h_q,
                  int d_v) {
  char* w = static_cast<char*>(const_cast<void*>(ws));
  const size_t rows = (size_t)plan->n_partial_slots * q_len * h_q;
  if (rows > 0) {
    p.o_part = reinterpret_cast<float*>(w);
    p.lse_part = reinterpret_cast<float*>(w + (rows * d_v * 4 + 255) / 256 * 256);
  }
  p.flags = reinterpret_cast<int32_t*>(w + attn_internal::flags_offset(plan, h_q, d_v));
  p.counters = plan->counters;
}

void fill_common(Params& p, const attn_paged_kv_t* kv, const void* q, void* out, float* lse,
                 int q_len, int h_q, int groups, float scale, int flags, const attn_plan_t* plan,
                 void* ws, int d_v) {
  const int causal = flags & ATTN_CAUSAL;
  std::memset(&p, 0, sizeof(p));
  p.pool0 = static_cast<const char*>(kv->pool0);
  p.pool1 = static_cast<const char*>(kv->pool1);
  p.rope = static_cast<const char*>(kv->rope_pool);
  p.page_table = kv->page_table;
  p.page_stride = kv->page_stride;
  p.token_stride = kv->token_stride;
  p.head_stride = kv->head_stride;
  p.rpage_stride = kv->rope_page_stride;
  p.rtoken_stride = kv->rope_token_stride;
  p.rhead_stride = kv->rope_head_stride;
  p.max_pages = kv->max_pages_per_seq;
  p.page_shift = ilog2_pow2(kv->page_size);
  p.q = q;
  p.out = out;
  p.lse = lse;
  p.items = plan->items;
  p.seqinfo = plan->seqinfo;
  if (!plan_on_device(plan)) pack_inline(p, plan);
  p.q_len = q_len;
  p.h_q = h_q;
  p.g = h_q / groups;
  p.rows = p.g * q_len;
  p.causal = (causal && q_len > 1) ? 1 : 0;
  p.scale_log2 = scale * 1.4426950408889634f;
  set_partials(p, plan, ws, q_len, h_q, d_v);
}

template <typename T, int DV>
int launch_combine(const Params& p, const attn_plan_t* plan, hipStream_t stream) {
  if (plan->n_partial_slots <= 0) return ATTN_OK;
  constexpr int RPB = 256 / (DV / 4);
  const int rows_total = p.q_len * p.h_q;
  dim3 grid((rows_total + RPB - 1) / RPB, plan->batch);
  hipLaunchKernelGGL((combine_kernel<T, DV>), grid, dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_internal::KernelChoice choice_for(const attn_paged_kv_t* kv, attn_kind_t kind, int q_len,
                                       int h_q, int groups, int head_dim, int d_rope,
                                       int flags) {
  attn_shape_t sh;
  sh.kind = kind;
  sh.dtype = kv->dtype;
  sh.batch = kv->batch;
  sh.q_len = q_len;
  sh.h_q = h_q;
  sh.groups = groups;
  sh.head_dim = head_dim;
  sh.d_rope = d_rope;
  sh.page_size = kv->page_size;
  sh.flags = flags;
  return attn_internal::choose_kernel(sh);
}

// The GQA/GTA streaming kernel keeps each lane's byte offset within a
// 16-row slice of bf16 rows in 32 bits; larger token strides take the
// general kernel, which addresses in 64 bits.
bool slice_offsets_fit(int64_t token_stride) {
  return 16 * 2 * token_stride < (1LL << 32);
}

template <int KIND, typename T, int W0, int DR>
int run(const Params& p, const attn_plan_t* plan, int flags, hipStream_t stream) {
  int st = run_general(KIND, std::is_same<T, __bf16>::value, W0, p, plan->n_items, stream);
  if (st != ATTN_OK || (flags & ATTN_DEFER_MERGE)) return st;
  return launch_combine<T, W0>(p, plan, stream);
}

void rope_table(Params& p, int d_rope, float theta) {
  // revolutions per position for frequency k: theta^(-2k/d_r) / (2 pi),
  // computed in double and split into two floats
  for (int k = 0; k < d_rope / 2; ++k) {
    const double f = std::pow((double)theta, -2.0 * k / d_rope) / (2.0 * M_PI);
    const float hi = (float)f;
    p.rope_hi[k] = hi;
    p.rope_lo[k] = (float)(f - (double)hi);
  }
  p.rope_on = 1;
}

// GQA decode after validation, with workspace `ws` (the caller's, or the
// library's own device array for attn_decode_gqa_static).
int decode_gqa(const attn_paged_kv_t* kv, const void* q, void* out, float* lse, int q_len,
               int h_q, int h_kv, int d, float softmax_scale, int flags, const attn_plan_t* plan,
               void* ws, hipStream_t stream) {
  int st = ATTN_OK;
  Params p;
  fill_common(p, kv, q, out, lse, q_len, h_q, h_kv, softmax_scale, flags, plan, ws, d);
  const attn_internal::KernelChoice kc =
      choice_for(kv, ATTN_KIND_GQA, q_len, h_q, h_kv, d, 0, flags);
  if (kc.narrow && slice_offsets_fit(kv->token_stride)) {
    // the streaming kernel merges split rows itself when the plan carries
    // counters (and the merge is not deferred); otherwise a merge launch
    p.fuse_merge = (!(flags & ATTN_DEFER_MERGE) && plan->counters) ? 1 : 0;
    if (plan->queue) {
      p.queue = plan->queue;
      p.queue_base = resident_slots(kc.wgs_per_cu);
    }
    st = run_narrow(GQA, d, p, plan->n_items, h_kv, kc.stages, stream);
    if (st != ATTN_OK || (flags & ATTN_DEFER_MERGE) || p.fuse_merge) return st;
    return d == 128 ? launch_combine<__bf16, 128>(p, plan, stream)
                    : launch_combine<__bf16, 64>(p, plan, stream);
  }
  if (kv->dtype == ATTN_BF16)
    return d == 128 ? run<GQA, __bf16, 128, 0>(p, plan, flags, stream) : run<GQA, __bf16, 64, 0>(p, plan, flags, stream);
  return d == 128 ? run<GQA, float, 128, 0>(p, plan, flags, stream) : run<GQA, float, 64, 0>(p, plan, flags, stream);
}


}  // namespace
}  // namespace attn_dev

// Workspace of attn_decode_gqa_static: one array per GPU, in the library's
// code object, held until the process ends.  Host code never passes this name
// to a kernel or a copy (on the host it stands for a host-side shadow, not a
// device address); it uses the per-device address that static_scratch()
// looks up instead.
static __device__ __align__(256) char scratch[ATTN_STATIC_SCRATCH_BYTES];

namespace attn_dev {
namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
std::atomic<void*> scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  void* ptr = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    ptr = scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
        return ATTN_ERR_HIP;
      scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return ATTN_OK;
}

}  // namespace
}  // namespace attn_dev

using namespace attn_dev;

extern "C" {

int attn_decode_gqa(const attn_paged_kv_t* kv, const void* q, void* out, float* lse, int q_len,
                    int h_q, int h_kv, int d, float softmax_scale, int flags,
                    const attn_plan_t* plan, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = validate(kv, q, out, q_len, h_q, h_kv, flags, plan, true, false);
  if (st != ATTN_OK) return st;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  st = check_workspace(plan, h_q, d, ws, ws_bytes);
  if (st != ATTN_OK) return st;
  return decode_gqa(kv, q, out, lse, q_len, h_q, h_kv, d, softmax_scale, flags, plan, ws, stream);
}

int attn_decode_gqa_static(const attn_paged_kv_t* kv, const void* q, void* out, float* lse,
                           int q_len, int h_q, int h_kv, int d, float softmax_scale, int flags,
                           const attn_plan_t* plan, hipStream_t stream) {
  int st = validate(kv, q, out, q_len, h_q, h_kv, flags, plan, true, false);
  if (st != ATTN_OK) return st;
  if (flags & ATTN_DEFER_MERGE) return ATTN_ERR_INVALID_ARG;  // partials unreachable
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (attn_decode_workspace_size(plan, h_q, d) > ATTN_STATIC_SCRATCH_BYTES)
    return ATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st != ATTN_OK) return st;
  return decode_gqa(kv, q, out, lse, q_len, h_q, h_kv, d, softmax_scale, flags, plan, ws, stream);
}

int attn_decode_gta(const attn_paged_kv_t* kv, const void* q, void* out, float* lse, int q_len,
                    int h_q, int h_kv, int d, int d_rope, int n_rope_heads, float rope_theta,
                    float softmax_scale, int flags, const attn_plan_t* plan, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  int st = validate(kv, q, out, q_len, h_q, h_kv, flags, plan, false, true);
  if (st != ATTN_OK) return st;
  if (n_rope_heads != 1 || d_rope <= 0 || d_rope >= d) return ATTN_ERR_INVALID_ARG;
  if (kv->dtype != ATTN_BF16 || d != 128 || d_rope != 64) return ATTN_ERR_UNSUPPORTED;
  st = check_workspace(plan, h_q, d, ws, ws_bytes);
  if (st != ATTN_OK) return st;
  Params p;
  fill_common(p, kv, q, out, lse, q_len, h_q, h_kv, softmax_scale, flags, plan, ws, d);
  if (rope_theta > 0.f) rope_table(p, d_rope, rope_theta);
  const attn_internal::KernelChoice kc =
      choice_for(kv, ATTN_KIND_GTA, q_len, h_q, h_kv, d, d_rope, flags);
  if (kc.narrow && slice_offsets_fit(kv->token_stride) &&
      slice_offsets_fit(kv->rope_token_stride)) {
    p.fuse_merge = (!(flags & ATTN_DEFER_MERGE) && plan->counters) ? 1 : 0;
    st = run_narrow(kc.pair == 2 ? GTA2 : GTA, d, p, plan->n_items, h_kv, kc.stages, stream);
    if (st != ATTN_OK || (flags & ATTN_DEFER_MERGE) || p.fuse_merge) return st;
    return launch_combine<__bf16, 128>(p, plan, stream);
  }
  return run<GTA, __bf16, 128, 64>(p, plan, flags, stream);
}

int attn_decode_latent(const attn_paged_kv_t* kv, const void* q, void* out, float* lse,
                       int q_len, int h_q, int h_c, int d_c, int d_rope, float softmax_scale,
                       int flags, const attn_plan_t* plan, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  int st = validate(kv, q, out, q_len, h_q, h_c, flags, plan, false, true);
  if (st != ATTN_OK) return st;
  if (kv->dtype != ATTN_BF16 || d_rope != 64 || (d_c != 512 && d_c != 256))
    return ATTN_ERR_UNSUPPORTED;
  st = check_workspace(plan, h_q, d_c, ws, ws_bytes);
  if (st != ATTN_OK) return st;
  Params p;
  fill_common(p, kv, q, out, lse, q_len, h_q, h_c, softmax_scale, flags, plan, ws, d_c);
  const attn_internal::KernelChoice kc =
      choice_for(kv, ATTN_KIND_LATENT, q_len, h_q, h_c, d_c, d_rope, flags);
  // the streaming latent kernel addresses a 64-row tile with 32-bit offsets
  const bool offsets_fit = 64 * 2 * kv->token_stride < (1LL << 31) &&
                           64 * 2 * kv->rope_token_stride < (1LL << 31);
  if (kc.narrow && offsets_fit) {
    p.fuse_merge = (!(flags & ATTN_DEFER_MERGE) && plan->counters) ? 1 : 0;
    st = run_wide(d_c, p, plan->n_items, stream);
    if (st != ATTN_OK || (flags & ATTN_DEFER_MERGE) || p.fuse_merge) return st;
    return d_c == 512 ? launch_combine<__bf16, 512>(p, plan, stream)
                      : launch_combine<__bf16, 256>(p, plan, stream);
  }
  return d_c == 512 ? run<LAT, __bf16, 512, 64>(p, plan, flags, stream)
                    : run<LAT, __bf16, 256, 64>(p, plan, flags, stream);
}

int attn_decode_merge(const attn_plan_t* plan, int h_q, int d_v, attn_dtype_t dtype,
                      const void* ws, size_t ws_bytes, void* out, float* lse, hipStream_t stream) {
  if (!plan || !out || h_q <= 0 || plan->q_len <= 0 || plan->batch <= 0 || plan->n_groups <= 0)
    return ATTN_ERR_INVALID_ARG;
  if (!plan_on_device(plan) && !plan_inline(plan)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP32) return ATTN_ERR_INVALID_ARG;
  if (d_v != 64 && d_v != 128 && d_v != 256 && d_v != 512) return ATTN_ERR_UNSUPPORTED;
  if (h_q % plan->n_groups) return ATTN_ERR_INVALID_ARG;
  if (check_plan(plan, INT64_MAX, 0) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  if (plan->n_partial_slots <= 0) return ATTN_OK;
  const size_t need = attn_decode_workspace_size(plan, h_q, d_v);
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return ATTN_ERR_WORKSPACE;
  if (!aligned16(out)) return ATTN_ERR_INVALID_ARG;
  Params p;
  std::memset(&p, 0, sizeof(p));
  p.out = out;
  p.lse = lse;
  p.seqinfo = plan->seqinfo;
  if (!plan_on_device(plan)) pack_inline(p, plan);
  p.q_len = plan->q_len;
  p.h_q = h_q;
  set_partials(p, plan, ws, plan->q_len, h_q, d_v);
  const bool bf = dtype == ATTN_BF16;
  switch (d_v) {
    case 64: return bf ? launch_combine<__bf16, 64>(p, plan, stream) : launch_combine<float, 64>(p, plan, stream);
    case 128: return bf ? launch_combine<__bf16, 128>(p, plan, stream) : launch_combine<float, 128>(p, plan, stream);
    case 256: return bf ? launch_combine<__bf16, 256>(p, plan, stream) : launch_combine<float, 256>(p, plan, stream);
    default: return bf ? launch_combine<__bf16, 512>(p, plan, stream) : launch_combine<float, 512>(p, plan, stream);
  }
}

}  // extern "C"
