// Device-side definitions shared by the decode kernels: vector types, the
// launch parameter block, small wave-level helpers, and the launchers each
// kernel translation unit exports to the entry points.
#ifndef ATTN_DEVICE_H
#define ATTN_DEVICE_H

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "attn_decode.h"
#include "attn_kernels.h"

namespace attn_dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

constexpr int KT = 64;  // keys per tile
constexpr int kMaxRope = 64;

// GTA2: GTA with two groups per workgroup (their common RoPE rows shared)
enum Kind { GQA = 0, GTA = 1, LAT = 2, GTA2 = 3 };

struct Params {
  const char* pool0;
  const char* pool1;
  const char* rope;
  const int32_t* page_table;
  int64_t page_stride, token_stride, head_stride;     // elements
  int64_t rpage_stride, rtoken_stride, rhead_stride;  // elements
  int32_t max_pages;
  int32_t page_shift;
  const void* q;
  void* out;
  float* lse;
  float* o_part;
  float* lse_part;
  int32_t* flags;     // latent streaming kernel: per-workgroup fix-up flags
  uint32_t* counters; // merge arrival counters (streaming kernels)
  uint32_t* queue;    // work-queue counter (GQA streaming kernel) or null
  int32_t queue_base; // items handed out statically (= resident workgroups)
  int32_t fuse_merge; // streaming kernels: the last split workgroup merges
  const int32_t* items;
  const int32_t* seqinfo;
  int32_t q_len, h_q, g, rows;  // rows = g * q_len per group
  int32_t n_items, row_blocks;
  int32_t nrb;  // GQA/GTA streaming kernel: workgroups (blocks of 16 RT rows) per item
  int32_t causal;
  int32_t rope_on;  // GTA: rotate the key's and query's RoPE slices in-kernel
  float scale_log2;
  // RoPE: revolutions per position of frequency k as hi + lo floats
  float rope_hi[kMaxRope / 2];
  float rope_lo[kMaxRope / 2];
  // plan in the launch arguments (plan_inline = 1 or 2): inl[3 b .. 3 b + 2]
  // = n_splits | (chunk / 64) << 16, partial slot base, L of sequence b;
  // chunk c (whose groups are items c * groups + j) is inl[3 inl_batch + c]
  // = b | split << 16 (form 1), or the 16-bit b | split << 11 in half c % 2
  // of inl[3 inl_batch + c / 2] (form 2)
  int32_t plan_inline;
  int32_t inl_batch;
  int32_t inl[ATTN_PLAN_INLINE_MAX];
};

// One work item of the plan, from device arrays or the launch arguments;
// `item` is wave-uniform, and so are the fields.
struct PlanItem {
  int b, j, split, t0, n_splits, slot_base, L, chunk;
};
__device__ __forceinline__ void seq_info(const Params& p, int b, int& n_splits, int& slot_base,
                                         int& L, int& chunk) {
  if (p.plan_inline) {
    const int32_t* si = p.inl + 3 * b;
    const uint32_t w0 = (uint32_t)__builtin_amdgcn_readfirstlane(si[0]);
    n_splits = (int)(w0 & 0xffffu);
    chunk = (int)(w0 >> 16) << 6;
    slot_base = __builtin_amdgcn_readfirstlane(si[1]);
    L = __builtin_amdgcn_readfirstlane(si[2]);
  } else {
    const int32_t* si = p.seqinfo + 4 * b;
    n_splits = __builtin_amdgcn_readfirstlane(si[0]);
    slot_base = __builtin_amdgcn_readfirstlane(si[1]);
    L = __builtin_amdgcn_readfirstlane(si[2]);
    chunk = __builtin_amdgcn_readfirstlane(si[3]);
  }
}
__device__ __forceinline__ PlanItem load_item(const Params& p, int item) {
  PlanItem r;
  if (p.plan_inline) {
    const int n_groups = p.h_q / p.g;
    const int c = item / n_groups;
    if (p.plan_inline == 2) {
      const uint32_t w =
          (uint32_t)__builtin_amdgcn_readfirstlane(p.inl[3 * p.inl_batch + (c >> 1)]);
      const uint32_t e = (c & 1) ? (w >> 16) : (w & 0xffffu);
      r.b = (int)(e & 0x7ffu);
      r.split = (int)(e >> 11);
    } else {
      const uint32_t e = (uint32_t)__builtin_amdgcn_readfirstlane(p.inl[3 * p.inl_batch + c]);
      r.b = (int)(e & 0xffffu);
      r.split = (int)(e >> 16);
    }
    r.j = item - c * n_groups;
  } else {
    const int32_t* it = p.items + 4 * item;
    r.b = __builtin_amdgcn_readfirstlane(it[0]);
    r.j = __builtin_amdgcn_readfirstlane(it[1]);
    r.split = __builtin_amdgcn_readfirstlane(it[2]);
    r.t0 = __builtin_amdgcn_readfirstlane(it[3]);
  }
  seq_info(p, r.b, r.n_splits, r.slot_base, r.L, r.chunk);
  if (p.plan_inline) r.t0 = r.split * r.chunk;  // chunks of equal length
  return r;
}

template <typename T> struct DT;
template <> struct DT<__bf16> { static constexpr int EPC = 8; };   // elements per 16 B
template <> struct DT<float> { static constexpr int EPC = 4; };

__device__ __forceinline__ float wave_max4(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_sum4(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// sin/cos of 2*pi*(pos * f) with f = hi + lo, reducing the angle exactly
// enough for positions up to 2^24.
__device__ __forceinline__ void rope_sincos(float pos, float hi, float lo, float& s, float& c) {
  float p = pos * hi;
  float e = fmaf(pos, hi, -p);
  float r = p - floorf(p);
  r += fmaf(pos, lo, e);
  r -= floorf(r);
  s = __builtin_amdgcn_sinf(r);
  c = __builtin_amdgcn_cosf(r);
}


// Scalar (SMEM) load of one int32 from a wave-uniform address, waited for in
// the same asm block.  SMEM loads count on lgkmcnt, so looking up a page id
// does not drain the vmcnt-tracked direct-to-LDS loads in flight.
// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

// A wave-uniform 64-bit pointer, made explicit so it is allocated to SGPRs.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// Direct global->LDS loads for rows of small pages, issued from asm so that
// the compiler neither drains vmcnt before unrelated LDS reads nor waits on
// them itself (the kernels' own waits cover them).  dma16v: one 16-byte load
// per lane from a per-lane 64-bit address, nontemporal (cache rows are read
// once), lane l writing LDS bytes [lds + 16 l, lds + 16 l + 16).  dma4: one
// 4-byte load per active lane from base + voff (page ids), lane l writing
// LDS bytes [lds + 4 l, lds + 4 l + 4).
__device__ __forceinline__ void dma16v(uint64_t addr, uint32_t lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(addr), "s"(l)
               : "memory");
}
__device__ __forceinline__ void dma16v_cached(uint64_t addr, uint32_t lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(addr), "s"(l)
               : "memory");
}
__device__ __forceinline__ void dma4(const char* base, uint32_t voff, uint32_t lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" : : "v"(voff), "s"(base),
               "s"(l) : "memory");
}

__device__ __forceinline__ int sload_i32(const int32_t* ptr) {
  // the address is wave-uniform; readfirstlane makes that explicit so the
  // operand is allocated to SGPRs
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int32_t* up = reinterpret_cast<const int32_t*>(((uint64_t)hi << 32) | lo);
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(up));
  return v;
}

// Split partials that the streaming kernels merge themselves are stored and
// loaded with agent-scope relaxed atomics: on gfx950 these carry the sc1
// scope bit, so they are written through / read past the per-XCD L2s and
// need no cache-wide write-back or invalidate fence (the splits of one row
// block may run on different XCDs).
__device__ __forceinline__ void store_partial(float* dst, float v) {
  __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_partial4(float* dst, f32x4 v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) store_partial(dst + i, v[i]);
}
__device__ __forceinline__ float load_partial(const float* src) {
  return __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge of split partials (Hydragen's softmax-denominator decomposition on
// the "Efficient Inference" tag page) for rows [row0, row0 + nrows) of group
// j of sequence b: M = max_s lse_s, w_s = exp(lse_s - M),
// out = sum_s w_s O_s / sum_s w_s, lse = M + ln sum_s w_s.  Every thread of
// the workgroup takes (row, 4 columns) units.
template <int DV>
__device__ __forceinline__ void merge_split_rows(const Params& p, int b, int j, int row0, int nrows,
                                                 int n_splits, int slot_base) {
  constexpr int C4 = DV / 4;
  for (int w = threadIdx.x; w < nrows * C4; w += blockDim.x) {
    const int r = row0 + w / C4;
    const int c4 = (w % C4) * 4;
    const int tq = r / p.g;
    const int hq = j * p.g + (r - tq * p.g);
    float M = -INFINITY;
    for (int s = 0; s < n_splits; ++s)
      M = fmaxf(M, load_partial(p.lse_part + ((int64_t)(slot_base + s) * p.q_len + tq) * p.h_q + hq));
    const float Ms = (M == -INFINITY) ? 0.f : M;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    float W = 0.f;
    for (int s = 0; s < n_splits; ++s) {
      const int64_t pr = ((int64_t)(slot_base + s) * p.q_len + tq) * p.h_q + hq;
      const float wt = __expf(load_partial(p.lse_part + pr) - Ms);
      W += wt;
      const float* o = p.o_part + pr * DV + c4;
      a += wt * f32x4{load_partial(o), load_partial(o + 1), load_partial(o + 2), load_partial(o + 3)};
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    const int64_t orow = ((int64_t)b * p.q_len + tq) * p.h_q + hq;
    __bf16 v4[4] = {(__bf16)(a[0] * inv), (__bf16)(a[1] * inv), (__bf16)(a[2] * inv),
                    (__bf16)(a[3] * inv)};
    *reinterpret_cast<uint2*>(reinterpret_cast<__bf16*>(p.out) + orow * DV + c4) =
        __builtin_bit_cast(uint2, v4);
    if (p.lse && c4 == 0) p.lse[orow] = W > 0.f ? Ms + __logf(W) : -INFINITY;
  }
}

// After this workgroup stored its split's partials (store_partial): once
// every thread's stores completed, count the arrival on `counter`; the last
// of the n_splits arrivals (the counter wraps to zero) merges the rows.
// `is_last` is a workgroup-shared int.
template <int DV>
__device__ __forceinline__ void arrive_and_merge(const Params& p, uint32_t* counter, int* is_last,
                                                 int b, int j, int row0, int nrows, int n_splits,
                                                 int slot_base) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0)
    *is_last = __builtin_amdgcn_atomic_inc32(counter, (uint32_t)(n_splits - 1), __ATOMIC_RELAXED,
                                             "agent") == (uint32_t)(n_splits - 1);
  __syncthreads();
  if (*is_last) merge_split_rows<DV>(p, b, j, row0, nrows, n_splits, slot_base);
}

// Launchers, one per kernel family (each in its own translation unit).
// They set the grid-dependent fields of a copy of `p` and enqueue on `stream`.
// General kernel: every kind / dtype / width the entry points accept.
int run_general(int kind, bool bf16, int w0, const Params& p, int n_items, hipStream_t stream);
// Streaming GQA / GTA kernel (bf16, any power-of-two page size, <= 64 rows per group).
int run_narrow(int kind, int d, const Params& p, int n_items, int groups, int stages,
               hipStream_t stream);
// Streaming latent kernel (bf16, pages >= 64 tokens, d_c 256 or 512, d_r 64).
int run_wide(int d_c, const Params& p, int n_items, hipStream_t stream);

}  // namespace attn_dev

#endif  // ATTN_DEVICE_H
