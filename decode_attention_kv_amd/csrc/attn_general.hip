// Split-KV decode attention over a paged KV cache for gfx950 (MI355X).
//
// One workgroup handles one work item of the host plan: a sequence b, a
// group j (KV head or latent head) and a chunk [t0, t1) of its tokens, for
// up to 16*NW query rows (the group's heads times the query tokens).
// Per 64-key tile it
//   1. gathers the tile's cache rows through the page table into LDS with
//      16-byte loads (paged indirection; "Hardware-Efficient Attention for
//      Fast Decoding", "If this is right"),
//   2. assembles keys: GQA reads K; GTA reads the leading d - d_r entries of
//      the tied state and the shared RoPE key rotated at the key position
//      (Figure 2 caption); latent reads [latent_j || rope] (Core claim),
//   3. computes transposed scores S^T = K Q^T with MFMA 16x16x32 bf16
//      (keys on the M axis, query rows on N), so each lane owns one query
//      row and the softmax probabilities are already laid out as the B
//      operand of the P.V product,
//   4. runs an online softmax (running max, rescaled running sum) with
//      cross-lane max reductions over the four 16-lane groups,
//   5. accumulates O^T += V^T P^T with MFMA, V^T read from LDS,
// and writes either the final output (unsplit sequences) or an fp32
// partial output plus its log-sum-exp.  A second kernel merges partials
// through their softmax denominators (Hydragen's decomposition on the
#include "attn_device.h"

namespace attn_dev {
namespace {

// Row layout constants of the LDS tiles (elements), padded by 16 bytes so
// that 16 keys read at the same column fall in different bank groups.
template <typename T, int W> struct Row {
  static constexpr int PAD = DT<T>::EPC;
  static constexpr int STRIDE = W + PAD;
  static constexpr int CH = W / DT<T>::EPC;  // 16-byte chunks per row
};

// Cooperative gather of one tile of rows (width W elements) into LDS.
template <typename T, int W, int NT>
__device__ __forceinline__ void load_tile(T* lds, const char* pool, int64_t page_stride,
                                          int64_t token_stride, int64_t head_off,
                                          const int32_t* pt_row, int page_shift, int tile0,
                                          int t_end, int tid) {
  using R = Row<T, W>;
  constexpr int TOTAL = KT * R::CH;
  const int pmask = (1 << page_shift) - 1;
#pragma unroll 4
  for (int idx = tid; idx < TOTAL; idx += NT) {
    const int key = idx / R::CH;
    const int ch = idx - key * R::CH;
    const int tok = tile0 + key;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (tok < t_end) {
      const int64_t page = pt_row[tok >> page_shift];
      const int64_t off = page * page_stride + (int64_t)(tok & pmask) * token_stride + head_off +
                          (int64_t)ch * DT<T>::EPC;
      v = *reinterpret_cast<const uint4*>(pool + off * (int64_t)sizeof(T));
    }
    *reinterpret_cast<uint4*>(lds + key * R::STRIDE + ch * DT<T>::EPC) = v;
  }
}

// ----------------------------------------------------------------------------
// The decode kernel.
//   KIND: GQA (K = pool0, V = pool1), GTA (tied pool0 + rope), LAT (latent
//   pool0 + rope).  W0: width of pool0 rows; DR: RoPE width (0 for GQA);
//   NW: waves per workgroup; RT: 16-row tiles per wave (every K / V^T operand
//   read from LDS feeds RT MFMAs).
template <int KIND, typename T, int W0, int DR, int NW, int RT>
__global__ __launch_bounds__(NW * 64) void decode_kernel(Params p) {
  constexpr int NT = NW * 64;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int DK = (KIND == LAT) ? W0 + DR : W0;  // key width
  constexpr int DV = W0;                            // value width
  constexpr int DN = DK - DR;                       // key entries from pool0
  constexpr int QW = (KIND == LAT) ? W0 + DR : W0;  // query row width in memory
  // k-chunk of one MFMA step: 32 dims (bf16: 8 per lane) or 16 dims (fp32:
  // 4 per lane, spread over four 16x16x4 MFMAs)
  constexpr int KC = BF ? 32 : 16;
  constexpr int NKC = DK / KC;
  constexpr int NDVT = DV / 16;
  static_assert(DK % KC == 0 && DV % 16 == 0, "dims");
  static_assert(KIND != GTA || DR == 64, "GTA in-kernel RoPE pairs need d_r = 64");

  using RV = Row<T, W0>;
  using RR = Row<T, (DR > 0 ? DR : 8)>;
  __shared__ __attribute__((aligned(16))) T lds_v[KT * RV::STRIDE];
  __shared__ __attribute__((aligned(16))) T lds_k[KIND == GQA ? KT * RV::STRIDE : 8];
  __shared__ __attribute__((aligned(16))) T lds_r[DR > 0 ? KT * RR::STRIDE : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;   // query row within a 16-row tile / MFMA column
  const int grp = lane >> 4;   // 16-lane group

  // Workgroups are dealt round-robin to the 8 XCDs (block i -> XCD i % 8).
  // The row blocks of one item are placed 8 apart so that they run on the
  // same XCD at about the same time and share its L2 for the chunk's rows.
  const int rb_count = p.row_blocks;
  const int bid = blockIdx.x;
  const int grp8 = bid / (8 * rb_count);
  const int rem = bid - grp8 * 8 * rb_count;
  const int rblk = rem >> 3;
  const int item = grp8 * 8 + (rem & 7);
  if (item >= p.n_items) return;
  const PlanItem pi = load_item(p, item);
  const int b = pi.b, j = pi.j, split = pi.split, t0 = pi.t0;
  const int n_splits = pi.n_splits, slot_base = pi.slot_base, L = pi.L, chunk = pi.chunk;
  const int t_end = min(t0 + chunk, L);

  // query rows owned by this lane (one per row tile)
  int tq[RT], hq[RT], qlimit[RT];
  bool row_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rblk * (16 * NW * RT) + (wave * RT + rt) * 16 + col;
    row_ok[rt] = row < p.rows;
    tq[rt] = row_ok[rt] ? row / p.g : 0;
    hq[rt] = j * p.g + (row_ok[rt] ? row - tq[rt] * p.g : 0);
    qlimit[rt] = (p.causal && row_ok[rt]) ? L - p.q_len + tq[rt] : 0x7fffffff;
  }

  // ---- query B operands (Q^T[k = dims][n = row]) in registers
  typedef typename std::conditional<BF, bf16x8, f32x4>::type QV;
  QV qreg[RT][NKC];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const T* qrow = reinterpret_cast<const T*>(p.q) +
                    ((int64_t)(b * p.q_len + tq[rt]) * p.h_q + hq[rt]) * QW;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      uint4 raw = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok[rt]) raw = *reinterpret_cast<const uint4*>(qrow + c * KC + grp * DT<T>::EPC);
      qreg[rt][c] = __builtin_bit_cast(QV, raw);
    }
    if constexpr (KIND == GTA) {
      if (p.rope_on) {
        // chunks DN/32 and DN/32 + 1 hold RoPE entries u and u + 32 of this lane
        constexpr int c0 = DN / 32;
        const float qpos = (float)(L - p.q_len + tq[rt]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int k = grp * 8 + u;
          float sn, cs;
          rope_sincos(qpos, p.rope_hi[k], p.rope_lo[k], sn, cs);
          const float x = (float)qreg[rt][c0][u], y = (float)qreg[rt][c0 + 1][u];
          qreg[rt][c0][u] = (__bf16)(x * cs - y * sn);
          qreg[rt][c0 + 1][u] = (__bf16)(x * sn + y * cs);
        }
      }
    }
  }

  f32x4 acc[RT][NDVT];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int i = 0; i < NDVT; ++i) acc[rt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* pt_row = p.page_table + (int64_t)b * p.max_pages;
  const bool rotate = (KIND == GTA) && p.rope_on;

  for (int tile0 = t0; tile0 < t_end; tile0 += KT) {
    // ---- 1. gather the tile into LDS
    if constexpr (KIND == GQA) {
      load_tile<T, W0, NT>(lds_k, p.pool0, p.page_stride, p.token_stride,
                           (int64_t)j * p.head_stride, pt_row, p.page_shift, tile0, t_end, tid);
      load_tile<T, W0, NT>(lds_v, p.pool1, p.page_stride, p.token_stride,
                           (int64_t)j * p.head_stride, pt_row, p.page_shift, tile0, t_end, tid);
    } else {
      load_tile<T, W0, NT>(lds_v, p.pool0, p.page_stride, p.token_stride,
                           (int64_t)j * p.head_stride, pt_row, p.page_shift, tile0, t_end, tid);
      load_tile<T, DR, NT>(lds_r, p.rope, p.rpage_stride, p.rtoken_stride, 0, pt_row,
                           p.page_shift, tile0, t_end, tid);
    }
    __syncthreads();

    // ---- 2-3. scores S^T[key][row] for the 64 keys, four 16-key M tiles
    float s[RT][4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int kr = mt * 16 + col;  // key row this lane feeds into the A operand
      f32x4 sa[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sa[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (BF) {
        auto kload = [&](int c) {
          const int d0 = c * 32 + grp * 8;
          const T* src;
          if constexpr (KIND == GQA) src = lds_k + kr * RV::STRIDE + d0;
          else src = (d0 < DN) ? lds_v + kr * RV::STRIDE + d0 : lds_r + kr * RR::STRIDE + (d0 - DN);
          return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(src));
        };
        auto mma = [&](bf16x8 a, int c) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            sa[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[rt][c], sa[rt], 0, 0, 0);
        };
        if constexpr (KIND == GTA) {
          // chunks DN/32 and DN/32 + 1 hold RoPE entries u and u + 32 of this lane
          constexpr int c0 = DN / 32;
#pragma unroll
          for (int c = 0; c < c0; ++c) mma(kload(c), c);
          bf16x8 ka = kload(c0), kb = kload(c0 + 1);
          if (rotate) {
            const float kpos = (float)(tile0 + kr);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              float sn, cs;
              rope_sincos(kpos, p.rope_hi[grp * 8 + u], p.rope_lo[grp * 8 + u], sn, cs);
              const float x = (float)ka[u], y = (float)kb[u];
              ka[u] = (__bf16)(x * cs - y * sn);
              kb[u] = (__bf16)(x * sn + y * cs);
            }
          }
          mma(ka, c0);
          mma(kb, c0 + 1);
#pragma unroll
          for (int c = c0 + 2; c < NKC; ++c) mma(kload(c), c);
        } else {
#pragma unroll
          for (int c = 0; c < NKC; ++c) {
            mma(kload(c), c);
            if constexpr (NKC > 8) {
              if ((c & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
          const f32x4 kv = *reinterpret_cast<const f32x4*>(
              lds_k + kr * RV::STRIDE + c * 16 + grp * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              sa[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[e], qreg[rt][c][e], sa[rt], 0, 0, 0);
        }
      }
      // lane holds keys mt*16 + grp*4 + i for its query row
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = tile0 + mt * 16 + grp * 4 + i;
          const bool vis = key < t_end && key <= qlimit[rt];
          s[rt][mt][i] = vis ? sa[rt][i] * p.scale_log2 : -INFINITY;
        }
    }

    // ---- 4. online softmax (base 2, scale folded in)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s[rt][mt][i]);
      tmax = wave_max4(tmax);
      const float m_new = fmaxf(m_run[rt], tmax);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run[rt] - m_use);
      float psum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[rt][mt][i] = exp2f(s[rt][mt][i] - m_use);
          psum += s[rt][mt][i];
        }
      l_run[rt] = l_run[rt] * alpha + psum;
      m_run[rt] = m_new;
#pragma unroll
      for (int dt = 0; dt < NDVT; ++dt) acc[rt][dt] *= alpha;
    }

    // ---- 5. O^T += V^T P^T
    if constexpr (BF) {
      const u16* vb = reinterpret_cast<const u16*>(lds_v);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        bf16x8 pb[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pb[rt][i] = (__bf16)s[rt][2 * kc][i];
            pb[rt][4 + i] = (__bf16)s[rt][2 * kc + 1][i];
          }
        const int k0 = kc * 32 + grp * 4;  // keys k0..k0+3 and k0+16..k0+19
#pragma unroll
        for (int dt = 0; dt < NDVT; ++dt) {
          const int dv = dt * 16 + col;
          u16 e[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            e[i] = vb[(k0 + i) * RV::STRIDE + dv];
            e[4 + i] = vb[(k0 + 16 + i) * RV::STRIDE + dv];
          }
          const bf16x8 va = __builtin_bit_cast(bf16x8, e);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rt], acc[rt][dt], 0, 0, 0);
          // keep the scheduler from hoisting every V^T gather of the tile
          // (wide latent rows would not fit the register file)
          if constexpr (NDVT > 8) {
            if ((dt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = mt * 16 + grp * 4 + i;
#pragma unroll
          for (int dt = 0; dt < NDVT; ++dt) {
            const float v = lds_v[key * RV::STRIDE + dt * 16 + col];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, s[rt][mt][i], acc[rt][dt], 0, 0, 0);
          }
        }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds O^T[dv = 16*dt + 4*grp + i][row]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float l_row = wave_sum4(l_run[rt]);
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    const float lse_val =
        l_row > 0.f ? (m_run[rt] + __log2f(l_row)) * 0.69314718055994531f : -INFINITY;
    if (!row_ok[rt]) continue;
    const int64_t orow = (int64_t)(b * p.q_len + tq[rt]) * p.h_q + hq[rt];
    if (n_splits <= 1) {
      T* o = reinterpret_cast<T*>(p.out) + orow * DV;
#pragma unroll
      for (int dt = 0; dt < NDVT; ++dt) {
        const int dv = dt * 16 + grp * 4;
        if constexpr (BF) {
          __bf16 v4[4] = {(__bf16)(acc[rt][dt][0] * inv), (__bf16)(acc[rt][dt][1] * inv),
                          (__bf16)(acc[rt][dt][2] * inv), (__bf16)(acc[rt][dt][3] * inv)};
          *reinterpret_cast<uint2*>(o + dv) = __builtin_bit_cast(uint2, v4);
        } else {
          *reinterpret_cast<f32x4*>(o + dv) = acc[rt][dt] * inv;
        }
      }
      if (p.lse && grp == 0) p.lse[orow] = lse_val;
    } else {
      const int64_t prow = (int64_t)((slot_base + split) * p.q_len + tq[rt]) * p.h_q + hq[rt];
      float* o = p.o_part + prow * DV;
#pragma unroll
      for (int dt = 0; dt < NDVT; ++dt)
        *reinterpret_cast<f32x4*>(o + dt * 16 + grp * 4) = acc[rt][dt] * inv;
      if (grp == 0) p.lse_part[prow] = lse_val;
    }
  }
}
template <int KIND, typename T, int W0, int DR, int NW, int RT>
int launch_one(Params p, int n_items, hipStream_t stream) {
  p.n_items = n_items;
  p.row_blocks = (p.rows + 16 * NW * RT - 1) / (16 * NW * RT);
  const int groups8 = (n_items + 7) / 8;
  dim3 grid(groups8 * 8 * p.row_blocks);
  hipLaunchKernelGGL((decode_kernel<KIND, T, W0, DR, NW, RT>), grid, dim3(NW * 64), 0, stream, p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// Waves per workgroup follow the rows of a group (16 rows per row tile).
// Wide latent rows (d_c = 512) keep one row tile per wave and at most four
// waves so that Q and O stay in registers without spilling; 256-wide latent
// heads use two row tiles per wave, so every K / V^T operand read from LDS
// feeds two MFMAs.
template <int KIND, typename T, int W0, int DR>
int launch_decode(const Params& p, int n_items, hipStream_t stream) {
  const int tiles = (p.rows + 15) / 16;
  if constexpr (KIND == LAT && W0 == 512) {
    if (tiles >= 3) return launch_one<KIND, T, W0, DR, 4, 1>(p, n_items, stream);
    if (tiles == 2) return launch_one<KIND, T, W0, DR, 2, 1>(p, n_items, stream);
    return launch_one<KIND, T, W0, DR, 1, 1>(p, n_items, stream);
  } else if constexpr (KIND == LAT) {
    if (tiles >= 6) return launch_one<KIND, T, W0, DR, 4, 2>(p, n_items, stream);
    if (tiles >= 3) return launch_one<KIND, T, W0, DR, 2, 2>(p, n_items, stream);
    if (tiles == 2) return launch_one<KIND, T, W0, DR, 1, 2>(p, n_items, stream);
    return launch_one<KIND, T, W0, DR, 1, 1>(p, n_items, stream);
  } else {
    if (tiles >= 8) return launch_one<KIND, T, W0, DR, 8, 1>(p, n_items, stream);
    if (tiles >= 4) return launch_one<KIND, T, W0, DR, 4, 1>(p, n_items, stream);
    if (tiles >= 2) return launch_one<KIND, T, W0, DR, 2, 1>(p, n_items, stream);
    return launch_one<KIND, T, W0, DR, 1, 1>(p, n_items, stream);
  }
}

}  // namespace

int run_general(int kind, bool bf16, int w0, const Params& p, int n_items, hipStream_t stream) {
  if (kind == GQA) {
    if (bf16)
      return w0 == 128 ? launch_decode<GQA, __bf16, 128, 0>(p, n_items, stream)
                       : launch_decode<GQA, __bf16, 64, 0>(p, n_items, stream);
    return w0 == 128 ? launch_decode<GQA, float, 128, 0>(p, n_items, stream)
                     : launch_decode<GQA, float, 64, 0>(p, n_items, stream);
  }
  if (kind == GTA) return launch_decode<GTA, __bf16, 128, 64>(p, n_items, stream);
  return w0 == 512 ? launch_decode<LAT, __bf16, 512, 64>(p, n_items, stream)
                   : launch_decode<LAT, __bf16, 256, 64>(p, n_items, stream);
}

}  // namespace attn_dev
