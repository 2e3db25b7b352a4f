// Projections around the latent decode kernel.  MLA and GLA attend in the
// latent space: the cache holds latent rows c (one or h_c latent heads) and
// a shared RoPE key, and every query head scores [c || RoPE] and returns a
// latent output ("Hardware-Efficient Attention for Fast Decoding", review
// page: Core claim and What carries the argument).  The per-head key and
// value up-projections are folded into the query and the output instead of
// the cache: the query's non-RoPE part becomes q_lat = W_UK[h] q_nope (so
// that q_lat . c = q_nope . (W_UK[h]^T c)), and the latent output becomes
// o = W_UV[h] o_lat.  Both are per-head products with few rows (the step's
// tokens) against a weight matrix per head:
//   C[m][h][n] = sum_k A[m][h][k] * W[h][n][k]
// with the weights stored K-contiguous ([h][n][k]), so MFMA operands load as
// 16-byte rows and need no transposes.  Both forms below compute C^T = W A^T
// so that each lane ends with four consecutive output columns of one row
// (one 8-byte store), and keep all work of one head on one XCD, which reads
// the head's weights from HBM once.  K in {128, 256, 512}: the weights
// stream through LDS (proj_stream_kernel); other K: 64 x 64 output tiles with
// both operands straight from global memory (proj_kernel).
#include "attn_device.h"

namespace attn_dev {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

struct ProjParams {
  const __bf16* a;          // A[m][h][k] at a + m * a_tok + h * a_head + k
  const __bf16* w;          // W[h][n][k], contiguous
  __bf16* c;                // C[m][h][n] at c + m * c_tok + h * c_head + n
  const __bf16* r;          // RoPE part copied to C[m][h][N + j], or NULL
  int64_t a_tok, a_head, c_tok, c_head, r_tok, r_head;
  int32_t M, N, K, H, d_r, m_tiles, n_tiles;
};

constexpr int kTileM = 64, kTileN = 64;

// K in groups of KG 32-wide chunks; DB: the next group's loads are in flight
// while the current group's MFMAs run (one memory round trip per group, not
// per chunk).  K <= 32 KG takes a single group and no second buffer.
constexpr int KG = 4;

// Register-only form: a 4-wave workgroup computes a 64 x 64 output tile of
// one head (2 x 2 waves of 32 x 32, four 16 x 16 MFMA tiles each).
template <bool DB>
__global__ __launch_bounds__(256) void proj_kernel(ProjParams p) {
  // block -> (head, column tile, row tile): heads are dealt to the XCDs
  // (block i runs on XCD i mod 8) and all tiles of a head follow 8 blocks
  // apart on its XCD, which then reads the head's weights and inputs from
  // HBM once
  const int bid = blockIdx.x;
  const int slot = bid >> 3;
  const int per_head = p.n_tiles * p.m_tiles;
  const int hx = slot / per_head;
  const int rem = slot - hx * per_head;
  const int h = hx * 8 + (bid & 7);
  if (h >= p.H) return;
  const int nt = rem / p.m_tiles, mt = rem - nt * p.m_tiles;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, kg = lane >> 4;
  const int m0 = mt * kTileM + (wave >> 1) * 32;
  const int n0 = nt * kTileN + (wave & 1) * 32;

  // lane i of 16-row tile t: weight row n0 + 16 t + i and input row
  // m0 + 16 t + i, k elements 8 kg .. 8 kg + 7 of each 32-wide chunk
  const __bf16* wrow[2];
  const __bf16* arow[2];
  bool aok[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    wrow[t] = p.w + ((int64_t)h * p.N + n0 + 16 * t + i) * p.K + 8 * kg;
    const int m = m0 + 16 * t + i;
    aok[t] = m < p.M;
    arow[t] = p.a + (int64_t)(aok[t] ? m : 0) * p.a_tok + (int64_t)h * p.a_head + 8 * kg;
  }
  f32x4 acc[2][2];  // [column tile][row tile]
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bf16x8_t zero = {};
  bf16x8_t wv[DB ? 2 : 1][KG][2], av[DB ? 2 : 1][KG][2];  // [buffer][chunk][16-row tile]
  auto load_group = [&](int buf, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < KG; ++c) {
      const int k = k0 + 32 * c;
      const bool in = k < p.K;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        wv[buf][c][t] = in ? *reinterpret_cast<const bf16x8_t*>(wrow[t] + k) : zero;
        av[buf][c][t] = in && aok[t] ? *reinterpret_cast<const bf16x8_t*>(arow[t] + k) : zero;
      }
    }
  };
  auto mma_group = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < KG; ++c)
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[buf][c][x], av[buf][c][y],
                                                              acc[x][y], 0, 0, 0);
  };
  load_group(0, 0);
  if constexpr (DB) {
    for (int k0 = 0; k0 < p.K; k0 += 2 * 32 * KG) {
      if (k0 + 32 * KG < p.K) load_group(1, k0 + 32 * KG);
      mma_group(0);
      if (k0 + 32 * KG >= p.K) break;
      if (k0 + 64 * KG < p.K) load_group(0, k0 + 64 * KG);
      mma_group(1);
    }
  } else {
    mma_group(0);
  }

  // acc[x][y]: lane holds C[m0 + 16 y + i][n0 + 16 x + 4 kg + e], e < 4
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    const int m = m0 + 16 * y + i;
    if (m >= p.M) continue;
    __bf16* crow = p.c + (int64_t)m * p.c_tok + (int64_t)h * p.c_head + n0 + 4 * kg;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      __bf16 v4[4] = {(__bf16)acc[x][y][0], (__bf16)acc[x][y][1], (__bf16)acc[x][y][2],
                      (__bf16)acc[x][y][3]};
      *reinterpret_cast<uint2*>(crow + 16 * x) = __builtin_bit_cast(uint2, v4);
    }
  }

  // the first column tile of each (head, row tile) also copies its rows'
  // RoPE parts behind the product columns
  if (p.r && nt == 0) {
    const int units = p.d_r / 8;  // 16-byte units per row
    for (int x = threadIdx.x; x < kTileM * units; x += blockDim.x) {
      const int row = x / units, uu = x - row * units;
      const int m = mt * kTileM + row;
      if (m >= p.M) continue;
      *reinterpret_cast<uint4*>(p.c + (int64_t)m * p.c_tok + (int64_t)h * p.c_head + p.N + 8 * uu) =
          *reinterpret_cast<const uint4*>(p.r + (int64_t)m * p.r_tok + (int64_t)h * p.r_head +
                                          8 * uu);
    }
  }
}

// Streamed-weight form for K in {128, 256, 512}: a workgroup owns one head
// and 64 input rows; each wave keeps its 16 rows' K values in registers (the
// B operand) and the head's weights stream through LDS in blocks of 64
// output columns (double-buffered, filled by direct-to-LDS loads), so every
// weight byte reaches a workgroup once and the inputs are read once.  In
// LDS, the 16-byte chunk c of weight row r sits at position c ^ (r mod 16):
// the 16 lanes that read chunk c of rows r .. r + 15 then hit distinct banks.
// (Keeping all output columns in registers with a deeper ring measured no
// faster for 128 rows and slower for 1024: it costs occupancy.)
constexpr int kColsBlk = 64;

__device__ __forceinline__ void dma16w(uint64_t addr, uint32_t lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(addr), "s"(l)
               : "memory");
}

template <int K>
__global__ __launch_bounds__(256) void proj_stream_kernel(ProjParams p) {
  constexpr int NC = K / 32;                // 32-wide k chunks
  constexpr int RB = K * 2;                 // bytes per weight row
  constexpr int BLK = kColsBlk * RB;        // bytes per weight block
  constexpr int LPW = BLK / 1024 / 4;       // 1 KB loads per wave per block
  static_assert(RB / 16 >= 16 && BLK % 4096 == 0, "rows of at least 16 chunks");
  __shared__ __attribute__((aligned(1024))) char wbuf[2][BLK];

  // block -> (head, row block): a head's row blocks sit 8 blocks apart on one
  // XCD, which reads the head's weights from HBM once
  const int bid = blockIdx.x;
  const int slot = bid >> 3;
  const int hx = slot / p.m_tiles;
  const int mb = slot - hx * p.m_tiles;
  const int h = hx * 8 + (bid & 7);
  if (h >= p.H) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, kg = lane >> 4;

  // this wave's 16 input rows, k elements 8 kg .. 8 kg + 7 of every chunk
  const int m = mb * kTileM + wave * 16 + i;
  const bool mok = m < p.M;
  const __bf16* arow = p.a + (int64_t)(mok ? m : 0) * p.a_tok + (int64_t)h * p.a_head + 8 * kg;
  const bf16x8_t zero = {};
  bf16x8_t areg[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    areg[c] = mok ? *reinterpret_cast<const bf16x8_t*>(arow + 32 * c) : zero;

  // weight block nb (rows 64 nb .. 64 nb + 63) into buffer `buf`: this
  // wave's loads cover LDS bytes [1024 (LPW wave + q), + 1024) of the block
  const char* wbase = reinterpret_cast<const char*>(p.w + (int64_t)h * p.N * K);
  auto issue_block = [&](int nb, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int off = (wave * LPW + q) * 1024 + 16 * lane;
      const int row = off / RB, ch = (off % RB) / 16;
      const uint64_t src = reinterpret_cast<uint64_t>(wbase) +
                           (uint64_t)((int64_t)(nb * kColsBlk + row) * RB + (ch ^ (row & 15)) * 16);
      dma16w(src, lds_u32(&wbuf[buf][(wave * LPW + q) * 1024]));
    }
  };

  const int n_blocks = p.N / kColsBlk;
  issue_block(0, 0);
  for (int nb = 0; nb < n_blocks; ++nb) {
    const int buf = nb & 1;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of block nb (and older ones)
    __syncthreads();                // every wave's part landed; buffer buf ^ 1 is free
    if (nb + 1 < n_blocks) issue_block(nb + 1, buf ^ 1);
    // C^T tiles: A operand = weight rows 16 t + i of the block, chunk c
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const char* wb = wbuf[buf];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8_t wv = *reinterpret_cast<const bf16x8_t*>(
            wb + (16 * t + i) * RB + (((4 * c + kg) ^ i) * 16));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv, areg[c], acc[t], 0, 0, 0);
      }
    // acc[t]: lane holds C[m][64 nb + 16 t + 4 kg + e], e < 4
    if (mok) {
      __bf16* crow = p.c + (int64_t)m * p.c_tok + (int64_t)h * p.c_head + nb * kColsBlk + 4 * kg;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        __bf16 v4[4] = {(__bf16)acc[t][0], (__bf16)acc[t][1], (__bf16)acc[t][2], (__bf16)acc[t][3]};
        *reinterpret_cast<uint2*>(crow + 16 * t) = __builtin_bit_cast(uint2, v4);
      }
    }
  }

  // the RoPE parts of this workgroup's rows behind the product columns
  if (p.r) {
    const int units = p.d_r / 8;  // 16-byte units per row
    for (int x = threadIdx.x; x < kTileM * units; x += blockDim.x) {
      const int row = x / units, uu = x - row * units;
      const int mm = mb * kTileM + row;
      if (mm >= p.M) continue;
      *reinterpret_cast<uint4*>(p.c + (int64_t)mm * p.c_tok + (int64_t)h * p.c_head + p.N + 8 * uu) =
          *reinterpret_cast<const uint4*>(p.r + (int64_t)mm * p.r_tok + (int64_t)h * p.r_head +
                                          8 * uu);
    }
  }
}

bool aligned16(const void* q) { return ((uintptr_t)q & 15u) == 0; }

int launch_proj(const ProjParams& p, hipStream_t stream) {
  if (p.K == 128 || p.K == 256 || p.K == 512) {
    const int64_t sblocks = (int64_t)(p.H + 7) / 8 * 8 * p.m_tiles;
    if (sblocks > INT32_MAX) return ATTN_ERR_INVALID_ARG;
    const dim3 grid((unsigned)sblocks), block(256);
    if (p.K == 128)
      hipLaunchKernelGGL(proj_stream_kernel<128>, grid, block, 0, stream, p);
    else if (p.K == 256)
      hipLaunchKernelGGL(proj_stream_kernel<256>, grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL(proj_stream_kernel<512>, grid, block, 0, stream, p);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
  }
  const int64_t blocks = (int64_t)(p.H + 7) / 8 * 8 * p.n_tiles * p.m_tiles;
  if (blocks > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  if (p.K > 32 * KG)
    hipLaunchKernelGGL(proj_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(proj_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace
}  // namespace attn_dev

using namespace attn_dev;

extern "C" int attn_latent_absorb_query(const void* q_nope, const void* q_rope, const void* w_uk,
                                        void* q_out, int n_tok, int h_q, int d_nope, int d_c,
                                        int d_rope, hipStream_t stream) {
  if (n_tok < 0 || h_q < 1 || d_nope < 32 || d_nope % 32 || d_c < kTileN || d_c % kTileN)
    return ATTN_ERR_INVALID_ARG;
  if (d_rope < 0 || d_rope % 8) return ATTN_ERR_INVALID_ARG;
  if (n_tok == 0) return ATTN_OK;  // empty buffers may be NULL
  if ((d_rope > 0) != (q_rope != nullptr)) return ATTN_ERR_INVALID_ARG;
  if (!q_nope || !w_uk || !q_out) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_out) || (q_rope && !aligned16(q_rope)))
    return ATTN_ERR_INVALID_ARG;
  ProjParams p{};
  p.a = static_cast<const __bf16*>(q_nope);
  p.w = static_cast<const __bf16*>(w_uk);
  p.c = static_cast<__bf16*>(q_out);
  p.r = static_cast<const __bf16*>(q_rope);
  p.a_head = d_nope;
  p.a_tok = (int64_t)h_q * d_nope;
  p.c_head = d_c + d_rope;
  p.c_tok = (int64_t)h_q * (d_c + d_rope);
  p.r_head = d_rope;
  p.r_tok = (int64_t)h_q * d_rope;
  p.M = n_tok;
  p.N = d_c;
  p.K = d_nope;
  p.H = h_q;
  p.d_r = d_rope;
  p.m_tiles = (n_tok + kTileM - 1) / kTileM;
  p.n_tiles = d_c / kTileN;
  return launch_proj(p, stream);
}

extern "C" int attn_latent_project_output(const void* o_lat, const void* w_uv, void* out, int n_tok,
                                          int h_q, int d_c, int d_v, hipStream_t stream) {
  if (n_tok < 0 || h_q < 1 || d_c < 32 || d_c % 32 || d_v < kTileN || d_v % kTileN)
    return ATTN_ERR_INVALID_ARG;
  if (n_tok == 0) return ATTN_OK;  // empty buffers may be NULL
  if (!o_lat || !w_uv || !out) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out)) return ATTN_ERR_INVALID_ARG;
  ProjParams p{};
  p.a = static_cast<const __bf16*>(o_lat);
  p.w = static_cast<const __bf16*>(w_uv);
  p.c = static_cast<__bf16*>(out);
  p.r = nullptr;
  p.a_head = d_c;
  p.a_tok = (int64_t)h_q * d_c;
  p.c_head = d_v;
  p.c_tok = (int64_t)h_q * d_v;
  p.M = n_tok;
  p.N = d_v;
  p.K = d_c;
  p.H = h_q;
  p.m_tiles = (n_tok + kTileM - 1) / kTileM;
  p.n_tiles = d_v / kTileN;
  return launch_proj(p, stream);
}
