// Streaming decode kernel for latent heads (MLA, GLA) on gfx950.
#include "attn_device.h"

namespace attn_dev {
namespace {


// ----------------------------------------------------------------------------
// Streaming kernel for latent heads (MLA / GLA): wide rows, many query rows.
//
// One workgroup holds NW*RT*16 query rows of one latent group (the group's
// heads times the query tokens, or a block of them) and streams the group's
// [latent || RoPE key] rows of its chunk through a ring of STAGES 64-key LDS
// stages shared by all waves.  The ring is filled by direct-to-LDS loads
// issued from inline asm, so the compiler sees no pending vector loads and
// schedules the ordinary LDS operand reads with lgkmcnt waits only; one
// barrier per stage hands the stage from loads to readers.  Every K and V^T
// operand read from LDS feeds RT MFMAs (one per row tile of the wave).
// Scores are transposed (S^T = K Q^T, keys on M) so P^T is the B operand of
// O^T += V^T P^T straight from registers; V^T comes from
// ds_read_b64_tr_b16.
#ifndef WIDE_SB_K
#define WIDE_SB_K 0
#endif
#ifndef WIDE_SB_V
#define WIDE_SB_V 0
#endif
namespace wide {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// One direct global->LDS 16-byte load per lane: lane l writes LDS bytes
// [lds + 16 l, lds + 16 l + 16).  Issued from asm so that the compiler
// does not drain vmcnt before unrelated LDS reads; waits are explicit.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);  // wave-uniform LDS base
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(l)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

template <int DC, int DR> struct Geo {
  static constexpr int LROW = DC * 2;               // latent row bytes
  static constexpr int RROW = DR * 2;               // RoPE row bytes
  static constexpr int LCPR = LROW / 16;            // 16-byte chunks per latent row
  static constexpr int RCPR = RROW / 16;
  static constexpr int R_OFF = 64 * LROW;           // RoPE block after the latent block
  static constexpr int STAGE = 64 * (LROW + RROW);
  static constexpr int LLOADS = 64 * LROW / 1024;   // 1 KB loads per stage
  static constexpr int RLOADS = 64 * RROW / 1024;
  static constexpr int LOADS = LLOADS + RLOADS;
};

// Per-workgroup context of one work item.
struct Item {
  int b, j, split, t0, t_end, n_tiles, n_splits, slot_base, L, rblk;
};

// Stream the item's chunk through the LDS ring and write its output rows.
//
// RESCALE = false: each row keeps a FIXED reference max m_ref, the max of
// its first tile with a visible key (the visible keys of a chunk are a
// prefix of it, so that is the first tile, while O and l are still zero);
// O is never rescaled.  Probabilities exp2(s - m_ref) are exact in floating
// point; while no score exceeds m_ref by more than 2^64 (log2 units) every
// sum stays far below the fp32 range.  Returns true, without writing
// anything, if some row of the workgroup exceeded that bound.
// RESCALE = true: the classic online softmax (the running max is raised and
// O, l rescaled whenever a tile's max exceeds it); never fails.  It is only
// called for such rare workgroups, as a separate function so that its
// register needs do not burden the fixed-reference loop.
template <int DC, int DR, int NW, int RT, int STAGES, bool RESCALE>
__device__ __forceinline__ bool stream(const Params& p, const Item& itm, char* ring,
                                       int* restart_flag) {
  using G = Geo<DC, DR>;
  constexpr int DK = DC + DR;
  constexpr int NKC = DK / 32;     // 32-dim k-chunks
  constexpr int NDVT = DC / 16;    // 16-wide output tiles
  constexpr int ROWS = NW * RT * 16;
  constexpr int LPW = G::LOADS / NW;  // loads per wave per stage
  // k-chunks / V^T tiles per scheduling region (0: no fences)
  constexpr int SB_K = WIDE_SB_K;
  constexpr int SB_V = WIDE_SB_V;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int b = itm.b, j = itm.j, t0 = itm.t0, t_end = itm.t_end, n_tiles = itm.n_tiles;
  const int L = itm.L;
  const int t_last = t_end - 1;
  const int pmask = (1 << p.page_shift) - 1;
  const int32_t* pt_row = p.page_table + (int64_t)b * p.max_pages;

  int tq[RT], hq[RT], qlimit[RT];
  bool row_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = itm.rblk * ROWS + (wave * RT + rt) * 16 + col;
    row_ok[rt] = row < p.rows;
    tq[rt] = row_ok[rt] ? row / p.g : 0;
    hq[rt] = j * p.g + (row_ok[rt] ? row - tq[rt] * p.g : 0);
    qlimit[rt] = (p.causal && row_ok[rt]) ? L - p.q_len + tq[rt] : 0x7fffffff;
  }

  // ---- query B operands: Q^T[k = dims 32c + 8 grp ..][n = row]
  bf16x8 qreg[RT][NKC];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) +
                         ((int64_t)(b * p.q_len + tq[rt]) * p.h_q + hq[rt]) * DK;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      uint4 raw = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok[rt]) raw = *reinterpret_cast<const uint4*>(qrow + c * 32 + grp * 8);
      qreg[rt][c] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  // the query loads must be complete before the asm loads start counting
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)

  const uint32_t ring_base = lds_u32(ring);
  const int64_t head_off = (int64_t)j * p.head_stride;

  // this wave's share of the loads of tile t into stage u: load i covers
  // latent rows (i * 1024 / LROW ...) or RoPE rows, lane -> (row, chunk)
  auto issue = [&](int t, int u) {
    const int tt = min(t, n_tiles - 1);
    const int key0 = t0 + tt * 64;                  // 64-aligned, inside one page
    const int64_t page = sload_i32(pt_row + (key0 >> p.page_shift));
    const int slot0 = key0 & pmask;
    // rows of this tile that exist: keys key0 .. t_last; later rows re-read
    // row t_last (the trailing clamped issues re-read the last tile)
    const int valid = max(1, min(64, t_end - key0));
    const char* lbase =
        p.pool0 + (page * p.page_stride + (int64_t)slot0 * p.token_stride + head_off) * 2;
    const char* rbase = p.rope + (page * p.rpage_stride + (int64_t)slot0 * p.rtoken_stride) * 2;
    const uint32_t sbase = ring_base + u * G::STAGE;
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      const int i = wave + k * NW;   // load index within the stage (wave-uniform)
      if (i < G::LLOADS) {
        constexpr int RPL = 1024 / G::LROW;          // latent rows per load
        const int r = i * RPL + lane / G::LCPR;
        const int c = (lane % G::LCPR) ^ (r & (G::LCPR - 1));
        const int rr = min(r, valid - 1);
        dma16(lbase + (int64_t)rr * p.token_stride * 2 + c * 16, sbase + i * 1024);
      } else {
        constexpr int RPLR = 1024 / G::RROW;
        const int r = (i - G::LLOADS) * RPLR + lane / G::RCPR;
        const int c = (lane % G::RCPR) ^ (r & (G::RCPR - 1));
        const int rr = min(r, valid - 1);
        dma16(rbase + (int64_t)rr * p.rtoken_stride * 2 + c * 16,
              sbase + G::R_OFF + (i - G::LLOADS) * 1024);
      }
    }
  };

  f32x4 acc[RT][NDVT];
  float m_ref[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_ref[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int i = 0; i < NDVT; ++i) acc[rt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bool over = false;

  if (n_tiles > 0) {
#pragma unroll
    for (int u = 0; u < STAGES - 1; ++u) issue(u, u);
  }

  for (int t = 0; t < n_tiles; ++t) {
    const int u = t % STAGES;
    issue(t + STAGES - 1, (t + STAGES - 1) % STAGES);
    {
      constexpr int ahead = (STAGES - 1) * LPW;
      __builtin_amdgcn_s_waitcnt((ahead & 15) | ((ahead >> 4) << 14) | (0x7 << 4) | (0xf << 8));
    }
    __syncthreads();  // every wave's loads of stage u have landed
    const char* sb = ring + u * G::STAGE;
    const int key0 = t0 + t * 64;

    // scores S^T for the 64 keys: 4 M tiles of 16 keys, advanced together
    // over the k-chunks (4 x RT independent MFMA accumulation chains)
    f32x4 sa[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) sa[rt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      const int ch = 4 * c + grp;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int kr = mt * 16 + col;
        const char* src = (ch < G::LCPR)
            ? sb + kr * G::LROW + ((ch ^ (kr & (G::LCPR - 1))) * 16)
            : sb + G::R_OFF + kr * G::RROW + (((ch - G::LCPR) ^ (kr & (G::RCPR - 1))) * 16);
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(src);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          sa[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[rt][c], sa[rt][mt], 0, 0, 0);
      }
      if (SB_K > 0 && (c % SB_K) == SB_K - 1) __builtin_amdgcn_sched_barrier(0);
    }
    float s[RT][4][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[rt][mt][i] = sa[rt][mt][i] * p.scale_log2;

    // mask + softmax
    const bool full = (key0 + 64 <= t_end) && !p.causal;
    bf16x8 pb[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (!full) {
            const int key = key0 + mt * 16 + grp * 4 + i;
            if (!(key < t_end && key <= qlimit[rt])) s[rt][mt][i] = -INFINITY;
          }
          tmax = fmaxf(tmax, s[rt][mt][i]);
        }
      tmax = wave_max4(tmax);
      if constexpr (RESCALE) {
        // raise the running max and rescale O and l
        const float m_new = fmaxf(m_ref[rt], tmax);
        const float m_u = (m_new == -INFINITY) ? 0.f : m_new;
        const float a = __builtin_amdgcn_exp2f(m_ref[rt] - m_u);
        l_run[rt] *= a;
#pragma unroll
        for (int dt = 0; dt < NDVT; ++dt) acc[rt][dt] *= a;
        m_ref[rt] = m_new;
      } else {
        if (m_ref[rt] == -INFINITY) m_ref[rt] = tmax;
        over |= tmax > m_ref[rt] + 64.f;
      }
      const float m_use = (m_ref[rt] == -INFINITY) ? 0.f : m_ref[rt];
      float psum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(s[rt][mt][i] - m_use);
          psum += e;
          pb[rt][mt >> 1][(mt & 1) * 4 + i] = (__bf16)e;
        }
      l_run[rt] += psum;
    }

    // O^T += V^T P^T; per 32-key chunk kc the A operand holds keys
    // 32 kc + 4 grp + e (e < 4) and 32 kc + 16 + 4 grp + (e - 4)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int kl0 = kc * 32 + grp * 4 + (col >> 2);
      const int kl1 = kl0 + 16;
#pragma unroll
      for (int dt = 0; dt < NDVT; ++dt) {
        const int cidx = 2 * dt + ((col & 3) >> 1);
        const int half = (col & 1) * 8;
        const char* s0 = sb + kl0 * G::LROW + ((cidx ^ (kl0 & (G::LCPR - 1))) * 16) + half;
        const char* s1 = sb + kl1 * G::LROW + ((cidx ^ (kl1 & (G::LCPR - 1))) * 16) + half;
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(s0));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(s1));
        const bf16x8 va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rt][kc], acc[rt][dt], 0, 0, 0);
        if (SB_V > 0 && (dt % SB_V) == SB_V - 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // every wave is done reading stage u
  }
  __builtin_amdgcn_s_waitcnt(0);  // drain clamped trailing loads

  if constexpr (!RESCALE) {
    // workgroup-wide: did any row outgrow its reference?
    if (tid == 0) *restart_flag = 0;
    __syncthreads();
    if (__builtin_amdgcn_ballot_w64(over) != 0 && lane == 0) *restart_flag = 1;
    __syncthreads();
    const bool again = *restart_flag != 0;
    __syncthreads();
    if (again) return true;
  }

  // ---- epilogue: lane holds O^T[dv = 16 dt + 4 grp + i][row]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float l_row = wave_sum4(l_run[rt]);
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    const float lse_val =
        l_row > 0.f ? (m_ref[rt] + __log2f(l_row)) * 0.69314718055994531f : -INFINITY;
    if (!row_ok[rt]) continue;
    const int64_t orow = (int64_t)(b * p.q_len + tq[rt]) * p.h_q + hq[rt];
    if (itm.n_splits <= 1) {
      __bf16* o = reinterpret_cast<__bf16*>(p.out) + orow * DC;
#pragma unroll
      for (int dt = 0; dt < NDVT; ++dt) {
        __bf16 v4[4] = {(__bf16)(acc[rt][dt][0] * inv), (__bf16)(acc[rt][dt][1] * inv),
                        (__bf16)(acc[rt][dt][2] * inv), (__bf16)(acc[rt][dt][3] * inv)};
        *reinterpret_cast<uint2*>(o + dt * 16 + grp * 4) = __builtin_bit_cast(uint2, v4);
      }
      if (p.lse && grp == 0) p.lse[orow] = lse_val;
    } else {
      const int64_t prow =
          (int64_t)((itm.slot_base + itm.split) * p.q_len + tq[rt]) * p.h_q + hq[rt];
      float* o = p.o_part + prow * DC;
#pragma unroll
      for (int dt = 0; dt < NDVT; ++dt)
        *reinterpret_cast<f32x4*>(o + dt * 16 + grp * 4) = acc[rt][dt] * inv;
      if (grp == 0) p.lse_part[prow] = lse_val;
    }
  }
  return false;
}

// RESCALE = false: the fixed-reference pass; records per workgroup whether
// it had to give up (flags[block]).  RESCALE = true: the fix-up pass, a
// second launch over the same grid that only works where the flag is set.
template <int DC, int DR, int NW, int RT, int STAGES, bool RESCALE>
__global__ __launch_bounds__(NW * 64) void decode_wide(Params p) {
  using G = Geo<DC, DR>;
  static_assert(G::LOADS % NW == 0, "loads split evenly over the waves");
  static_assert(STAGES * G::STAGE <= 160 * 1024 - 1024, "LDS");
  static_assert((STAGES - 1) * (G::LOADS / NW) <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char ring[STAGES * G::STAGE];
  __shared__ int restart_flag;

  if constexpr (RESCALE) {
    if (p.flags[blockIdx.x] == 0) return;
  }
  // item and row block, with row blocks of one item 8 apart (same XCD)
  const int rb_count = p.row_blocks;
  const int bid = blockIdx.x;
  const int blk8 = bid / (8 * rb_count);
  const int rem = bid - blk8 * 8 * rb_count;
  Item itm;
  itm.rblk = rem >> 3;
  const int item = blk8 * 8 + (rem & 7);
  if (item >= p.n_items) return;
  const int32_t* it = p.items + 4 * item;
  itm.b = __builtin_amdgcn_readfirstlane(it[0]);
  itm.j = __builtin_amdgcn_readfirstlane(it[1]);
  itm.split = __builtin_amdgcn_readfirstlane(it[2]);
  itm.t0 = __builtin_amdgcn_readfirstlane(it[3]);
  const int32_t* si = p.seqinfo + 4 * itm.b;
  itm.n_splits = __builtin_amdgcn_readfirstlane(si[0]);
  itm.slot_base = __builtin_amdgcn_readfirstlane(si[1]);
  itm.L = __builtin_amdgcn_readfirstlane(si[2]);
  const int chunk = __builtin_amdgcn_readfirstlane(si[3]);
  itm.t_end = min(itm.t0 + chunk, itm.L);
  itm.n_tiles = (itm.t_end - itm.t0 + 63) / 64;

  const bool gave_up = stream<DC, DR, NW, RT, STAGES, RESCALE>(p, itm, ring, &restart_flag);
  if constexpr (!RESCALE) {
    if (threadIdx.x == 0) p.flags[blockIdx.x] = gave_up ? 1 : 0;
  }
}

}  // namespace wide

template <int DC, int DR, int NW, int RT, int S>
int launch_wide_one(Params p, int n_items, hipStream_t stream) {
  p.n_items = n_items;
  p.row_blocks = (p.rows + 16 * NW * RT - 1) / (16 * NW * RT);
  const int groups8 = (n_items + 7) / 8;
  const dim3 grid(groups8 * 8 * p.row_blocks);
  hipLaunchKernelGGL((wide::decode_wide<DC, DR, NW, RT, S, false>), grid, dim3(NW * 64), 0,
                     stream, p);
  // fix-up pass: exits at once unless the first pass flagged the workgroup
  hipLaunchKernelGGL((wide::decode_wide<DC, DR, NW, RT, S, true>), grid, dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// Latent heads: two row tiles per wave; two or four waves by the group's rows;
// as many 64-key stages as fit the LDS (2 for 512-wide, 3 for 256-wide).
template <int DC, int DR>
int launch_wide(const Params& p, int n_items, hipStream_t stream) {
  constexpr int S = (DC >= 512) ? 2 : 3;
  if constexpr (DC >= 512) {
    // 512-wide latents: one row tile per wave keeps O (128 regs) and Q in
    // the register file; 64 rows per workgroup
    return launch_wide_one<DC, DR, 4, 1, S>(p, n_items, stream);
  } else {
    // every SIMD gets a wave: one row tile per wave up to 64 rows
    if (p.rows <= 64) return launch_wide_one<DC, DR, 4, 1, S>(p, n_items, stream);
    return launch_wide_one<DC, DR, 4, 2, S>(p, n_items, stream);
  }
}

}  // namespace

int run_wide(int d_c, const Params& p, int n_items, hipStream_t stream) {
  return d_c == 512 ? launch_wide<512, 64>(p, n_items, stream)
                    : launch_wide<256, 64>(p, n_items, stream);
}

}  // namespace attn_dev
