// Measurement probes: the ceilings the decode kernels are compared with on
// the GPU they run on.  The decode path is bound by reading the KV cache
// from HBM ("Hardware-Efficient Attention for Fast Decoding", review page,
// Core claim) or, for latent heads at high intensity, by the matrix cores
// (the roofline of its Figure 3 caption); these kernels measure how fast
// this GPU streams a buffer from HBM and how fast its matrix cores run bf16
// products when nothing else limits them.
#include "attn_device.h"

namespace attn_dev {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlock = 64 * 1024;  // bytes one workgroup reads per step

// Streaming read into registers: each lane loads 16-byte units of 64 KB
// blocks (block i of the buffer goes to workgroup i mod grid) with the
// nontemporal hint, XORs them together and folds the result into `sink`.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(kProbeThreads) void probe_read_vgpr(const u32x4* buf, int64_t blocks,
                                                                 uint32_t* sink) {
  constexpr int U = kProbeBlock / 16 / kProbeThreads;  // 16-byte units per lane per block
  u32x4 x = {0u, 0u, 0u, 0u};
  for (int64_t blk = blockIdx.x; blk < blocks; blk += gridDim.x) {
    const u32x4* src = buf + blk * (kProbeBlock / 16) + threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u];
  }
  const uint32_t r = x[0] ^ x[1] ^ x[2] ^ x[3];
  if (r == 0x9e3779b9u) atomicXor(sink, r);  // keeps the loads; practically never taken
}

// Streaming read straight into LDS (global_load_lds_dwordx4 with the
// nontemporal hint), the path the decode kernels take: each wave keeps
// DEPTH 1 KB loads of its 16 KB quarter of a block in flight through a
// private LDS ring and never reads the ring back.
template <int DEPTH>
__global__ __launch_bounds__(kProbeThreads) void probe_read_lds(const char* buf, int64_t blocks,
                                                                uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) char ring[4][DEPTH * 1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t dst = lds_u32(ring[wave]);
  constexpr int LOADS = kProbeBlock / 4 / 1024;  // 1 KB loads per wave per block
  int issued = 0;
  for (int64_t blk = blockIdx.x; blk < blocks; blk += gridDim.x) {
    const char* base = uniform_ptr(buf + blk * kProbeBlock + wave * (kProbeBlock / 4));
    for (int k = 0; k < LOADS; ++k) {
      const uint32_t l = __builtin_amdgcn_readfirstlane(dst + (issued % DEPTH) * 1024);
      const uint32_t voff = (uint32_t)(k * 1024 + lane * 16);
      asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff),
                   "s"(base), "s"(l) : "memory");
      ++issued;
      // keep at most DEPTH - 1 loads in flight before reusing a ring slot
      if (issued >= DEPTH) __builtin_amdgcn_s_waitcnt((DEPTH - 2) | (0x7 << 4) | (0xf << 8));
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const uint32_t r = reinterpret_cast<const uint32_t*>(ring[wave])[lane];
  if (r == 0x9e3779b9u) atomicXor(sink, r);
}

// Matrix-core throughput: every wave runs `iters` rounds of kProbeAcc
// independent v_mfma_f32_16x16x32_bf16 products on register operands (no
// memory traffic), then folds its accumulators into `sink`.  The products
// are written as asm with each accumulator tied to its own AGPRs: from the
// builtin the compiler moved the accumulators between registers on every
// round, which measured those moves instead of the matrix cores.  The same
// accumulator is reused only kProbeAcc products later, past any dependency
// window.
constexpr int kProbeAcc = 8;
#define PROBE_MFMA(c) \
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b))
__global__ __launch_bounds__(kProbeThreads) void probe_mfma(int iters, float* sink) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + 0.0078125f * (float)((threadIdx.x + i) & 7));
    b[i] = (__bf16)(0.5f - 0.0078125f * (float)((threadIdx.x * 3 + i) & 7));
  }
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  for (int it = 0; it < iters; ++it) {
    PROBE_MFMA(c0);
    PROBE_MFMA(c1);
    PROBE_MFMA(c2);
    PROBE_MFMA(c3);
    PROBE_MFMA(c4);
    PROBE_MFMA(c5);
    PROBE_MFMA(c6);
    PROBE_MFMA(c7);
  }
  const f32x4 t = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  const float s = t[0] + t[1] + t[2] + t[3];
  if (s == 1234.5f) atomicAdd(sink, s);  // keeps the products; practically never taken
}
#undef PROBE_MFMA

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

}  // namespace
}  // namespace attn_dev

using namespace attn_dev;

extern "C" {

int attn_probe_stream_read(const void* buf, size_t bytes, int mode, uint32_t* sink,
                           hipStream_t stream) {
  if (!buf || !sink || bytes < (size_t)kProbeBlock || bytes % kProbeBlock ||
      ((uintptr_t)buf & 1023u) || (mode != 0 && mode != 1))
    return ATTN_ERR_INVALID_ARG;
  const int cus = cu_count();
  if (cus <= 0) return ATTN_ERR_HIP;
  const int64_t blocks = (int64_t)(bytes / kProbeBlock);
  // a few workgroups per CU keep enough bytes in flight to cover the latency
  const int64_t grid = std::min<int64_t>(blocks, (int64_t)cus * (mode == 0 ? 8 : 2));
  if (mode == 0)
    hipLaunchKernelGGL(probe_read_vgpr, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                       static_cast<const u32x4*>(buf), blocks, sink);
  else
    hipLaunchKernelGGL(probe_read_lds<16>, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                       static_cast<const char*>(buf), blocks, sink);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_probe_mfma(int iters, float* sink, double* flops_out, hipStream_t stream) {
  if (iters <= 0 || !sink || !flops_out) return ATTN_ERR_INVALID_ARG;
  const int cus = cu_count();
  if (cus <= 0) return ATTN_ERR_HIP;
  // two 4-wave workgroups per CU: two waves per SIMD
  const int grid = cus * 2;
  *flops_out = (double)grid * (kProbeThreads / 64) * iters * kProbeAcc * (2.0 * 16 * 16 * 32);
  hipLaunchKernelGGL(probe_mfma, dim3(grid), dim3(kProbeThreads), 0, stream, iters, sink);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
