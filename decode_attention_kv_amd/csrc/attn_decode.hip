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
// "Efficient Inference" tag page).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "attn_decode.h"
#include "attn_kernels.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

constexpr int KT = 64;  // keys per tile
constexpr int kMaxRope = 64;

enum Kind { GQA = 0, GTA = 1, LAT = 2 };

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
  const int32_t* items;
  const int32_t* seqinfo;
  int32_t q_len, h_q, g, rows;  // rows = g * q_len per group
  int32_t n_items, row_blocks;
  int32_t causal;
  int32_t rope_on;  // GTA: rotate the key's and query's RoPE slices in-kernel
  float scale_log2;
  // RoPE: revolutions per position of frequency k as hi + lo floats
  float rope_hi[kMaxRope / 2];
  float rope_lo[kMaxRope / 2];
};

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
  const int32_t* it = p.items + 4 * item;
  const int b = it[0], j = it[1], split = it[2], t0 = it[3];
  const int32_t* si = p.seqinfo + 4 * b;
  const int n_splits = si[0], slot_base = si[1], L = si[2], chunk = si[3];
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

// ----------------------------------------------------------------------------
// Streaming kernel for narrow groups (GQA, GTA; at most 16*RT query rows per
// group, bf16, pages of >= 64 tokens).
//
// Four waves share one work item and split every 64-key tile: wave w owns
// keys [16w, 16w + 16).  Each wave streams its slices through a private ring
// of STAGES LDS buffers filled by direct global->LDS 16-byte loads, so a wave
// waits only on its own loads (vmcnt) and the main loop has no barriers.
// Rows are stored with 16-byte chunks XOR-swizzled by the key index so the
// K-operand reads of 16 keys and the transposing V reads hit distinct banks.
// Per 16-key slice: S^T = K Q^T (MFMA 16x16x32), online softmax, and
// O^T += V^T P^T with MFMA 16x16x16 whose V^T operand comes from
// ds_read_b64_tr_b16.  The waves' (max, sum, O) states are merged through
// LDS at the end of the item.
namespace narrow {

constexpr int NW = 4;    // waves per workgroup
constexpr int KW = 16;   // keys per wave per tile
constexpr int KTILE = NW * KW;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// Scalar (SMEM) load of one int32 from a wave-uniform address, waited for in
// the same asm block.  SMEM loads count on lgkmcnt, so looking up a page id
// does not drain the vmcnt-tracked direct-to-LDS loads in flight.
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

// N transposing LDS reads (ds_read_b64_tr_b16) in one asm block that also
// waits for them.  The compiler cannot relate this instruction to the
// direct-to-LDS loads in flight and would otherwise drain vmcnt before it;
// here the caller's own vmcnt wait already covers the stage being read.
typedef unsigned long long u64_t;
template <int N>
__device__ __forceinline__ void tr_reads(const uint32_t (&addr)[N], u64_t (&out)[N]);
template <>
__device__ __forceinline__ void tr_reads<8>(const uint32_t (&a)[8], u64_t (&o)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
        "v"(a[7]));
}
template <>
__device__ __forceinline__ void tr_reads<4>(const uint32_t (&a)[4], u64_t (&o)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}

// N 16-byte LDS reads in one asm block that also waits for them (same
// reason as tr_reads: keep the compiler from draining the DMA pipeline).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <int N>
__device__ __forceinline__ void b128_reads(const uint32_t (&addr)[N], u32x4_t (&out)[N]);
template <>
__device__ __forceinline__ void b128_reads<4>(const uint32_t (&a)[4], u32x4_t (&o)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}
template <>
__device__ __forceinline__ void b128_reads<2>(const uint32_t (&a)[2], u32x4_t (&o)[2]) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1])
      : "v"(a[0]), "v"(a[1]));
}

// All LDS operand reads of one 16-key slice in a single asm block with one
// wait: NK 16-byte K-operand reads and NV transposing V reads.
template <int NK, int NV>
__device__ __forceinline__ void slice_reads(const uint32_t (&ka)[NK], const uint32_t (&va)[NV],
                                            u32x4_t (&ko)[NK], u64_t (&vo)[NV]);
template <>
__device__ __forceinline__ void slice_reads<4, 8>(const uint32_t (&ka)[4], const uint32_t (&va)[8],
                                                  u32x4_t (&ko)[4], u64_t (&vo)[8]) {
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %13\n\t"
      "ds_read_b128 %2, %14\n\t"
      "ds_read_b128 %3, %15\n\t"
      "ds_read_b64_tr_b16 %4, %16\n\t"
      "ds_read_b64_tr_b16 %5, %17\n\t"
      "ds_read_b64_tr_b16 %6, %18\n\t"
      "ds_read_b64_tr_b16 %7, %19\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %21\n\t"
      "ds_read_b64_tr_b16 %10, %22\n\t"
      "ds_read_b64_tr_b16 %11, %23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(ko[0]), "=&v"(ko[1]), "=&v"(ko[2]), "=&v"(ko[3]), "=&v"(vo[0]), "=&v"(vo[1]),
        "=&v"(vo[2]), "=&v"(vo[3]), "=&v"(vo[4]), "=&v"(vo[5]), "=&v"(vo[6]), "=&v"(vo[7])
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]),
        "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7]));
}
template <>
__device__ __forceinline__ void slice_reads<2, 4>(const uint32_t (&ka)[2], const uint32_t (&va)[4],
                                                  u32x4_t (&ko)[2], u64_t (&vo)[4]) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b64_tr_b16 %2, %8\n\t"
      "ds_read_b64_tr_b16 %3, %9\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(ko[0]), "=&v"(ko[1]), "=&v"(vo[0]), "=&v"(vo[1]), "=&v"(vo[2]), "=&v"(vo[3])
      : "v"(ka[0]), "v"(ka[1]), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

template <int KIND, int D, int DR> struct Geo {
  // per-wave bytes of one stage: K (or tied) rows, V rows (GQA), RoPE rows (GTA)
  static constexpr int ROW0 = D * 2;                 // K / tied row bytes
  static constexpr int ROWR = DR * 2;                // RoPE row bytes
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = KW * ROW0;            // GQA only
  static constexpr int R_OFF = KW * ROW0;            // GTA only
  static constexpr int WAVE_BYTES = (KIND == GQA) ? 2 * KW * ROW0 : KW * (ROW0 + ROWR);
  static constexpr int STAGE_BYTES = NW * WAVE_BYTES;
  static constexpr int LOADS = (KIND == GQA) ? 2 * KW * ROW0 / 1024 : KW * (ROW0 + ROWR) / 1024;
};

// Per-lane byte offsets of the direct-to-LDS loads of one 16-key slice of
// rows of ROWB bytes: lane l of load i covers row i*RPI + l/CPR at swizzled
// chunk position l%CPR, i.e. it fetches logical chunk (l%CPR) ^ (row % CPR).
template <int ROWB>
struct SliceDMA {
  static constexpr int CPR = ROWB / 16;  // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;   // rows per 1 KB load
  static constexpr int N = KW / RPI;     // loads per slice
  uint32_t off[N];                       // bytes from the slice's first row
  int row[N];
  __device__ __forceinline__ void init(int64_t token_stride, int lane) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      row[i] = i * RPI + lane / CPR;
      const int c = (lane % CPR) ^ (row[i] & (CPR - 1));
      off[i] = (uint32_t)(row[i] * token_stride * 2 + c * 16);
    }
  }
  // full slice: every row valid, contiguous within one page
  __device__ __forceinline__ void issue(char* dst, const char* base) const {
#pragma unroll
    for (int i = 0; i < N; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(base + off[i]), (lds_void_t*)(dst + i * 1024),
                                       16, 0, 0);
  }
  // partial slice: rows at or past `valid` re-read row valid-1 (same page)
  __device__ __forceinline__ void issue_clamped(char* dst, const char* base, int valid,
                                                int64_t token_stride) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = min(row[i], valid - 1);
      const char* src = base + off[i] + (int64_t)(r - row[i]) * token_stride * 2;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(dst + i * 1024), 16, 0, 0);
    }
  }
};

template <int KIND, int D, int DR, int RT, int STAGES>
__global__ __launch_bounds__(NW * 64) void decode_narrow(Params p) {
  using G = Geo<KIND, D, DR>;
  constexpr int DN = D - DR;          // key entries from the K / tied row
  constexpr int NKC = D / 32;         // 32-dim k-chunks of the score MFMA
  constexpr int NDVT = D / 16;        // 16-wide output tiles
  constexpr int CPR0 = G::ROW0 / 16;
  constexpr int CPRR = (DR > 0) ? G::ROWR / 16 : 1;
  static_assert(STAGES >= 2 && STAGES <= 6, "stages");
  static_assert(G::LOADS * 1024 == G::WAVE_BYTES, "whole 1 KB load instructions");

  __shared__ __attribute__((aligned(1024))) char st0[G::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st1[G::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st2[STAGES > 2 ? G::STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char st3[STAGES > 3 ? G::STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char st4[STAGES > 4 ? G::STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char st5[STAGES > 5 ? G::STAGE_BYTES : 16];
  __shared__ float merge_m[NW][16 * RT], merge_l[NW][16 * RT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;

  // Workgroups are dealt round-robin to the 8 XCDs (block i -> XCD i % 8).
  // The plan lists the groups of one (sequence, chunk) consecutively; they
  // are mapped to blocks 8 apart so they share one XCD's L2 (GTA's RoPE key
  // rows are read by every group).
  const int gsz = p.row_blocks;  // groups per (sequence, chunk)
  const int bid = blockIdx.x;
  const int blk = bid / (8 * gsz);
  const int rem = bid - blk * 8 * gsz;
  const int item = (blk * 8 + (rem & 7)) * gsz + (rem >> 3);
  if (item >= p.n_items) return;
  const int32_t* it = p.items + 4 * item;
  const int b = __builtin_amdgcn_readfirstlane(it[0]);
  const int j = __builtin_amdgcn_readfirstlane(it[1]);
  const int split = __builtin_amdgcn_readfirstlane(it[2]);
  const int t0 = __builtin_amdgcn_readfirstlane(it[3]);
  const int32_t* si = p.seqinfo + 4 * b;
  const int n_splits = __builtin_amdgcn_readfirstlane(si[0]);
  const int slot_base = __builtin_amdgcn_readfirstlane(si[1]);
  const int L = __builtin_amdgcn_readfirstlane(si[2]);
  const int chunk = __builtin_amdgcn_readfirstlane(si[3]);
  const int t_end = min(t0 + chunk, L);
  const int n_tiles = (t_end - t0 + KTILE - 1) / KTILE;
  const int t_last = t_end - 1;
  const int pmask = (1 << p.page_shift) - 1;
  const int32_t* pt_row = p.page_table + (int64_t)b * p.max_pages;

  // rows of this lane (every wave holds every row)
  int tq[RT], hq[RT], qlimit[RT];
  bool row_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + col;
    row_ok[rt] = row < p.rows;
    tq[rt] = row_ok[rt] ? row / p.g : 0;
    hq[rt] = j * p.g + (row_ok[rt] ? row - tq[rt] * p.g : 0);
    qlimit[rt] = (p.causal && row_ok[rt]) ? L - p.q_len + tq[rt] : 0x7fffffff;
  }

  auto stage = [&](int u) -> char* {
    switch (u) {
      case 0: return st0;
      case 1: return st1;
      case 2: return st2;
      case 3: return st3;
      case 4: return st4;
      default: return st5;
    }
  };

  // direct-to-LDS load offsets of this lane (loop invariant)
  SliceDMA<G::ROW0> dma0;
  SliceDMA<(DR > 0 ? G::ROWR : 16)> dmar;
  dma0.init(p.token_stride, lane);
  if constexpr (KIND == GTA) dmar.init(p.rtoken_stride, lane);

  // issue this wave's loads of tile `t` (clamped to the last tile) into stage u
  auto issue = [&](int t, int u) {
    const int tt = min(t, n_tiles - 1);
    const int key0 = t0 + tt * KTILE + wave * KW;   // 16-aligned, inside one page
    const int kc = min(key0, t_last);
    const int valid = t_last - kc + 1;              // rows of the slice that exist
    const int64_t page = sload_i32(pt_row + (kc >> p.page_shift));
    const int slot0 = kc & pmask & ~(KW - 1);       // first row of the slice in its page
    char* dst = stage(u) + wave * G::WAVE_BYTES;
    const int64_t row0 = page * p.page_stride + (int64_t)slot0 * p.token_stride +
                         (int64_t)j * p.head_stride;
    const char* b0 = p.pool0 + row0 * 2;
    // rows past the chunk's end re-read its last row (for a slice wholly
    // past the end, kc is that row and slot0 its 16-aligned block)
    const int v = min((key0 <= t_last) ? valid : ((kc & pmask) - slot0 + 1), KW);
    dma0.issue_clamped(dst + G::K_OFF, b0, v, p.token_stride);
    if constexpr (KIND == GQA) {
      dma0.issue_clamped(dst + G::V_OFF, p.pool1 + row0 * 2, v, p.token_stride);
    } else {
      dmar.issue_clamped(dst + G::R_OFF,
                         p.rope + (page * p.rpage_stride + (int64_t)slot0 * p.rtoken_stride) * 2,
                         v, p.rtoken_stride);
    }
  };

  // RoPE frequencies of this lane's 8 pairs (entries 8 grp + u), hoisted so
  // no per-lane kernel-argument loads sit inside the streaming loop
  float rh[8], rl[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    rh[u] = (KIND == GTA) ? p.rope_hi[grp * 8 + u] : 0.f;
    rl[u] = (KIND == GTA) ? p.rope_lo[grp * 8 + u] : 0.f;
  }

  // ---- query B operands in registers (rotated for GTA)
  bf16x8 qreg[RT][NKC];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) +
                         ((int64_t)(b * p.q_len + tq[rt]) * p.h_q + hq[rt]) * D;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      uint4 raw = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok[rt]) raw = *reinterpret_cast<const uint4*>(qrow + c * 32 + grp * 8);
      qreg[rt][c] = __builtin_bit_cast(bf16x8, raw);
    }
    if constexpr (KIND == GTA) {
      if (p.rope_on) {
        constexpr int c0 = DN / 32;
        const float qpos = (float)(L - p.q_len + tq[rt]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          float sn, cs;
          rope_sincos(qpos, rh[u], rl[u], sn, cs);
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

  // start the ring; then wait for the (older) query loads only, so no
  // query load is still pending when the streaming loop starts
  if (n_tiles > 0) {
#pragma unroll
    for (int u = 0; u < STAGES - 1; ++u) issue(u, u);
  }
  {
    constexpr int ahead = (STAGES - 1) * G::LOADS;
    __builtin_amdgcn_s_waitcnt((ahead & 15) | ((ahead >> 4) << 14) | (0x7 << 4) | (0xf << 8));
  }

  // byte offsets (within a wave's V rows) of this lane's transposing reads:
  // lane `col` of group `grp` addresses key row 4 grp + col/4 and the
  // 4-column group (col % 4) of each 16-wide output tile, whose 16-byte chunk
  // sits at its XOR-swizzled position
  uint32_t v_off[NDVT];
  {
    const int kl = grp * 4 + (col >> 2);
    const int sw = kl & (CPR0 - 1);
#pragma unroll
    for (int dt = 0; dt < NDVT; ++dt) {
      const int cidx = 2 * dt + ((col & 3) >> 1);
      v_off[dt] = kl * G::ROW0 + ((cidx ^ sw) * 16) + (col & 1) * 8;
    }
  }

  // byte offsets (within a wave's stage) of this lane's K-operand chunks
  uint32_t k_off[NKC];
#pragma unroll
  for (int c = 0; c < NKC; ++c) {
    const int ch = 4 * c + grp;
    k_off[c] = (KIND == GQA || ch < DN / 8)
                   ? G::K_OFF + col * G::ROW0 + ((ch ^ (col & (CPR0 - 1))) * 16)
                   : G::R_OFF + col * G::ROWR + (((ch - DN / 8) ^ (col & (CPRR - 1))) * 16);
  }

  // one 16-key slice of tile t, read from stage u
  auto compute = [&](int t, int u) {
    const char* sb = stage(u) + wave * G::WAVE_BYTES;
    const int key0 = t0 + t * KTILE + wave * KW;
    // scores
    f32x4 sa[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) sa[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // all operand reads of the slice: K chunks (8 dims 32c + 8 grp .. of
    // key `col`) and the V^T tiles, one LDS round trip
    u32x4_t kraw[NKC];
    u64_t vraw[NDVT];
    {
      const uint32_t sbase = lds_addr(sb);
      const uint32_t vbase = sbase + ((KIND == GQA) ? G::V_OFF : G::K_OFF);
      uint32_t ka_addr[NKC], va_addr[NDVT];
#pragma unroll
      for (int c = 0; c < NKC; ++c) ka_addr[c] = sbase + k_off[c];
#pragma unroll
      for (int dt = 0; dt < NDVT; ++dt) va_addr[dt] = vbase + v_off[dt];
      slice_reads<NKC, NDVT>(ka_addr, va_addr, kraw, vraw);
    }
    auto kread = [&](int c) { return __builtin_bit_cast(bf16x8, kraw[c]); };
    auto mma = [&](bf16x8 a, int c) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        sa[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[rt][c], sa[rt], 0, 0, 0);
    };
    if constexpr (KIND == GTA) {
      constexpr int c0 = DN / 32;
#pragma unroll
      for (int c = 0; c < c0; ++c) mma(kread(c), c);
      bf16x8 ka = kread(c0), kb = kread(c0 + 1);
      if (p.rope_on) {
        const float kpos = (float)(key0 + col);
#pragma unroll
        for (int u2 = 0; u2 < 8; ++u2) {
          float sn, cs;
          rope_sincos(kpos, rh[u2], rl[u2], sn, cs);
          const float x = (float)ka[u2], y = (float)kb[u2];
          ka[u2] = (__bf16)(x * cs - y * sn);
          kb[u2] = (__bf16)(x * sn + y * cs);
        }
      }
      mma(ka, c0);
      mma(kb, c0 + 1);
#pragma unroll
      for (int c = c0 + 2; c < NKC; ++c) mma(kread(c), c);
    } else {
#pragma unroll
      for (int c = 0; c < NKC; ++c) mma(kread(c), c);
    }
    // mask + online softmax; lane holds keys key0 + 4 grp + i of its rows.
    // The running max is only raised (and O, l rescaled) when a row's max
    // grows by more than 2^8: probabilities then stay below 256, harmless in
    // fp32 and bf16, and most slices skip the rescale of the accumulators.
    const bool full = (key0 + KW <= t_end) && !p.causal;
    float s[RT][4];
    bool any_raise = false;
    float m_upd[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sa[rt][i] * p.scale_log2;
        if (!full) {
          const int key = key0 + grp * 4 + i;
          v = (key < t_end && key <= qlimit[rt]) ? v : -INFINITY;
        }
        s[rt][i] = v;
        tmax = fmaxf(tmax, v);
      }
      tmax = wave_max4(tmax);
      const bool raise = tmax > m_run[rt] + 8.f;
      m_upd[rt] = raise ? tmax : m_run[rt];
      any_raise |= raise;
    }
    if (__builtin_amdgcn_ballot_w64(any_raise) != 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_upd[rt]);
        if (m_upd[rt] != m_run[rt]) {
          l_run[rt] *= alpha;
        }
        const float a = (m_upd[rt] != m_run[rt]) ? alpha : 1.f;
#pragma unroll
        for (int dt = 0; dt < NDVT; ++dt) acc[rt][dt] *= a;
        m_run[rt] = m_upd[rt];
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float m_use = (m_run[rt] == -INFINITY) ? 0.f : m_run[rt];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[rt][i] = __builtin_amdgcn_exp2f(s[rt][i] - m_use);
        psum += s[rt][i];
      }
      l_run[rt] += psum;
    }
    // O^T += V^T P^T (k = this wave's 16 keys; lane group g holds keys 4g..4g+3)
    bf16x4 pb[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[rt][i] = (__bf16)s[rt][i];
#pragma unroll
    for (int dt = 0; dt < NDVT; ++dt) {
      const bf16x4 va = __builtin_bit_cast(bf16x4, vraw[dt]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[rt], acc[rt][dt], 0, 0, 0);
    }
  };

  // ---- main loop, unrolled by STAGES so every stage is a distinct LDS object
  for (int t = 0; t < n_tiles; t += STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) {
      if (t + u < n_tiles) {
        // every wave has read stage (u-1) of the previous tile before reuse
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        issue(t + u + STAGES - 1, (u + STAGES - 1) % STAGES);
        // wait until this tile's loads (issued STAGES-1 tiles ago) landed
        constexpr int ahead = (STAGES - 1) * G::LOADS;
        __builtin_amdgcn_s_waitcnt((ahead & 15) | ((ahead >> 4) << 14) | (0x7 << 4) | (0xf << 8));
        compute(t + u, u);
      }
    }
  }

  // ---- merge the four waves' softmax states through LDS
  __builtin_amdgcn_s_waitcnt(0);   // drain this wave's clamped trailing loads
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float l_w = wave_sum4(l_run[rt]);
    if (grp == 0) {
      merge_m[wave][rt * 16 + col] = m_run[rt];
      merge_l[wave][rt * 16 + col] = l_w;
    }
  }
  __syncthreads();
  // columns merged per pass: the largest power of two whose four per-wave
  // 16-row slabs fit one stage buffer
  constexpr int DP0 = G::STAGE_BYTES / (NW * 16 * 4);
  constexpr int DP = DP0 >= D ? D : DP0 >= 128 ? 128 : DP0 >= 64 ? 64 : 32;
  static_assert(D % DP == 0 && DP % (NW * 4) == 0, "merge passes");
  float* obuf = reinterpret_cast<float*>(st0);  // [NW][16][DP] fp32
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + col;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, merge_m[w][r]);
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    float lt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) lt += merge_l[w][r] * exp2f(merge_m[w][r] - mu);
    const float sc = exp2f(m_run[rt] - mu);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_val = lt > 0.f ? (mu + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
    const int64_t orow = (int64_t)(b * p.q_len + tq[rt]) * p.h_q + hq[rt];
    const int64_t prow = (int64_t)((slot_base + split) * p.q_len + tq[rt]) * p.h_q + hq[rt];
#pragma unroll
    for (int pass = 0; pass < D / DP; ++pass) {
#pragma unroll
      for (int dt = pass * (DP / 16); dt < (pass + 1) * (DP / 16); ++dt)
        *reinterpret_cast<f32x4*>(obuf + ((wave * 16 + col) * DP + dt * 16 - pass * DP + grp * 4)) =
            acc[rt][dt] * sc;
      __syncthreads();
      // each wave finishes DP/NW columns of the 16 rows
      constexpr int COLS = DP / NW;
#pragma unroll
      for (int c4 = grp * 4; c4 < COLS; c4 += 16) {
        const int cl = wave * COLS + c4;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) o += *reinterpret_cast<const f32x4*>(obuf + ((w * 16 + col) * DP + cl));
        o *= inv;
        const int dv = pass * DP + cl;
        if (row_ok[rt]) {
          if (n_splits <= 1) {
            __bf16 v4[4] = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
            *reinterpret_cast<uint2*>(reinterpret_cast<__bf16*>(p.out) + orow * D + dv) =
                __builtin_bit_cast(uint2, v4);
          } else {
            *reinterpret_cast<f32x4*>(p.o_part + prow * D + dv) = o;
          }
        }
      }
      __syncthreads();
    }
    if (row_ok[rt] && wave == 0 && grp == 0) {
      if (n_splits <= 1) {
        if (p.lse) p.lse[orow] = lse_val;
      } else {
        p.lse_part[prow] = lse_val;
      }
    }
  }
}

}  // namespace narrow

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
    const int64_t page = narrow::sload_i32(pt_row + (key0 >> p.page_shift));
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

// ----------------------------------------------------------------------------
// Merge the split partials of every sequence with n_splits > 1.
// grid (ceil(q_len*h_q / rows_per_block), batch); DV/4 threads per row.
template <typename T, int DV>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_part,
                                                       const float* __restrict__ lse_part,
                                                       const int32_t* __restrict__ seqinfo,
                                                       T* __restrict__ out, float* __restrict__ lse,
                                                       int rows_total) {
  constexpr int TPR = DV / 4;
  constexpr int RPB = 256 / TPR;
  const int b = blockIdx.y;
  const int n = seqinfo[4 * b + 0];
  if (n <= 1) return;
  const int base = seqinfo[4 * b + 1];
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= rows_total) return;
  const int c4 = (threadIdx.x % TPR) * 4;
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, lse_part[(int64_t)(base + s) * rows_total + row]);
  const float Ms = (M == -INFINITY) ? 0.f : M;
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
  for (int s = 0; s < n; ++s) {
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

int ilog2_pow2(int v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

struct Common {
  int elem;
  int d_v;
};

int validate(const attn_paged_kv_t* kv, const void* q, const void* out, int q_len, int h_q,
             int groups, int flags, const attn_plan_t* plan, const void* ws, size_t ws_bytes, int d_v,
             int pool_width, bool need_pool1, bool need_rope, int rope_width) {
  if (!kv || !q || !out || !plan) return ATTN_ERR_INVALID_ARG;
  if (!kv->pool0 || !kv->page_table || !kv->seqlens) return ATTN_ERR_INVALID_ARG;
  if (need_pool1 && !kv->pool1) return ATTN_ERR_INVALID_ARG;
  if (need_rope && !kv->rope_pool) return ATTN_ERR_INVALID_ARG;
  if (!plan->items || !plan->seqinfo || plan->n_items <= 0) return ATTN_ERR_INVALID_ARG;
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
  (void)pool_width;
  (void)rope_width;
  const size_t need = attn_decode_workspace_size(plan, h_q, d_v);
  if (need > 0 && (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)))
    return ATTN_ERR_WORKSPACE;
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
  p.q_len = q_len;
  p.h_q = h_q;
  p.g = h_q / groups;
  p.rows = p.g * q_len;
  p.causal = (causal && q_len > 1) ? 1 : 0;
  p.scale_log2 = scale * 1.4426950408889634f;
  set_partials(p, plan, ws, q_len, h_q, d_v);
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

template <typename T, int DV>
int launch_combine(const Params& p, const attn_plan_t* plan, hipStream_t stream) {
  if (plan->n_partial_slots <= 0) return ATTN_OK;
  constexpr int RPB = 256 / (DV / 4);
  const int rows_total = p.q_len * p.h_q;
  dim3 grid((rows_total + RPB - 1) / RPB, plan->batch);
  hipLaunchKernelGGL((combine_kernel<T, DV>), grid, dim3(256), 0, stream, p.o_part, p.lse_part,
                     p.seqinfo, static_cast<T*>(p.out), p.lse, rows_total);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

template <int KIND, int D, int DR, int RT, int S>
int launch_narrow_s(Params p, int n_items, int groups, hipStream_t stream) {
  using G = narrow::Geo<KIND, D, DR>;
  if constexpr (S * G::STAGE_BYTES + 4096 > 163840) {
    return launch_narrow_s<KIND, D, DR, RT, S - 1>(p, n_items, groups, stream);
  } else {
    p.n_items = n_items;
    p.row_blocks = groups;
    const int blocks = (n_items + 8 * groups - 1) / (8 * groups) * 8 * groups;
    hipLaunchKernelGGL((narrow::decode_narrow<KIND, D, DR, RT, S>), dim3(blocks),
                       dim3(narrow::NW * 64), 0, stream, p);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
  }
}

template <int KIND, int D, int DR, int RT>
int launch_narrow_rt(const Params& p, int n_items, int groups, int stages, hipStream_t stream) {
  switch (stages) {
    case 2: return launch_narrow_s<KIND, D, DR, RT, 2>(p, n_items, groups, stream);
    case 3: return launch_narrow_s<KIND, D, DR, RT, 3>(p, n_items, groups, stream);
    case 4: return launch_narrow_s<KIND, D, DR, RT, 4>(p, n_items, groups, stream);
    case 5: return launch_narrow_s<KIND, D, DR, RT, 5>(p, n_items, groups, stream);
    default: return launch_narrow_s<KIND, D, DR, RT, 6>(p, n_items, groups, stream);
  }
}

template <int KIND, int D, int DR>
int launch_narrow(const Params& p, int n_items, int groups, int stages, hipStream_t stream) {
  const int rt = (p.rows + 15) / 16;
  if (rt <= 1) return launch_narrow_rt<KIND, D, DR, 1>(p, n_items, groups, stages, stream);
  if (rt <= 2) return launch_narrow_rt<KIND, D, DR, 2>(p, n_items, groups, stages, stream);
  return launch_narrow_rt<KIND, D, DR, 4>(p, n_items, groups, stages, stream);
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

template <int KIND, typename T, int W0, int DR>
int run(const Params& p, const attn_plan_t* plan, int flags, hipStream_t stream) {
  int st = launch_decode<KIND, T, W0, DR>(p, plan->n_items, stream);
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

}  // namespace

extern "C" {

int attn_decode_gqa(const attn_paged_kv_t* kv, const void* q, void* out, float* lse, int q_len,
                    int h_q, int h_kv, int d, float softmax_scale, int flags,
                    const attn_plan_t* plan, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = validate(kv, q, out, q_len, h_q, h_kv, flags, plan, ws, ws_bytes, d, d, true, false, 0);
  if (st != ATTN_OK) return st;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  Params p;
  fill_common(p, kv, q, out, lse, q_len, h_q, h_kv, softmax_scale, flags, plan, ws, d);
  const attn_internal::KernelChoice kc =
      choice_for(kv, ATTN_KIND_GQA, q_len, h_q, h_kv, d, 0, flags);
  if (kc.narrow) {
    st = d == 128 ? launch_narrow<GQA, 128, 0>(p, plan->n_items, h_kv, kc.stages, stream)
                  : launch_narrow<GQA, 64, 0>(p, plan->n_items, h_kv, kc.stages, stream);
    if (st != ATTN_OK || (flags & ATTN_DEFER_MERGE)) return st;
    return d == 128 ? launch_combine<__bf16, 128>(p, plan, stream)
                    : launch_combine<__bf16, 64>(p, plan, stream);
  }
  if (kv->dtype == ATTN_BF16)
    return d == 128 ? run<GQA, __bf16, 128, 0>(p, plan, flags, stream) : run<GQA, __bf16, 64, 0>(p, plan, flags, stream);
  return d == 128 ? run<GQA, float, 128, 0>(p, plan, flags, stream) : run<GQA, float, 64, 0>(p, plan, flags, stream);
}

int attn_decode_gta(const attn_paged_kv_t* kv, const void* q, void* out, float* lse, int q_len,
                    int h_q, int h_kv, int d, int d_rope, int n_rope_heads, float rope_theta,
                    float softmax_scale, int flags, const attn_plan_t* plan, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  int st = validate(kv, q, out, q_len, h_q, h_kv, flags, plan, ws, ws_bytes, d, d, false, true, d_rope);
  if (st != ATTN_OK) return st;
  if (n_rope_heads != 1 || d_rope <= 0 || d_rope >= d) return ATTN_ERR_INVALID_ARG;
  if (kv->dtype != ATTN_BF16 || d != 128 || d_rope != 64) return ATTN_ERR_UNSUPPORTED;
  Params p;
  fill_common(p, kv, q, out, lse, q_len, h_q, h_kv, softmax_scale, flags, plan, ws, d);
  if (rope_theta > 0.f) rope_table(p, d_rope, rope_theta);
  const attn_internal::KernelChoice kc =
      choice_for(kv, ATTN_KIND_GTA, q_len, h_q, h_kv, d, d_rope, flags);
  if (kc.narrow) {
    st = launch_narrow<GTA, 128, 64>(p, plan->n_items, h_kv, kc.stages, stream);
    if (st != ATTN_OK || (flags & ATTN_DEFER_MERGE)) return st;
    return launch_combine<__bf16, 128>(p, plan, stream);
  }
  return run<GTA, __bf16, 128, 64>(p, plan, flags, stream);
}

int attn_decode_latent(const attn_paged_kv_t* kv, const void* q, void* out, float* lse,
                       int q_len, int h_q, int h_c, int d_c, int d_rope, float softmax_scale,
                       int flags, const attn_plan_t* plan, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  int st = validate(kv, q, out, q_len, h_q, h_c, flags, plan, ws, ws_bytes, d_c, d_c, false, true, d_rope);
  if (st != ATTN_OK) return st;
  if (kv->dtype != ATTN_BF16 || d_rope != 64 || (d_c != 512 && d_c != 256))
    return ATTN_ERR_UNSUPPORTED;
  Params p;
  fill_common(p, kv, q, out, lse, q_len, h_q, h_c, softmax_scale, flags, plan, ws, d_c);
  const attn_internal::KernelChoice kc =
      choice_for(kv, ATTN_KIND_LATENT, q_len, h_q, h_c, d_c, d_rope, flags);
  if (kc.narrow) {  // the streaming latent kernel
    st = d_c == 512 ? launch_wide<512, 64>(p, plan->n_items, stream)
                    : launch_wide<256, 64>(p, plan->n_items, stream);
    if (st != ATTN_OK || (flags & ATTN_DEFER_MERGE)) return st;
    return d_c == 512 ? launch_combine<__bf16, 512>(p, plan, stream)
                      : launch_combine<__bf16, 256>(p, plan, stream);
  }
  return d_c == 512 ? run<LAT, __bf16, 512, 64>(p, plan, flags, stream)
                    : run<LAT, __bf16, 256, 64>(p, plan, flags, stream);
}

int attn_decode_merge(const attn_plan_t* plan, int h_q, int d_v, attn_dtype_t dtype,
                      const void* ws, size_t ws_bytes, void* out, float* lse, hipStream_t stream) {
  if (!plan || !out || !plan->seqinfo || h_q <= 0 || plan->q_len <= 0 || plan->batch <= 0)
    return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP32) return ATTN_ERR_INVALID_ARG;
  if (d_v != 64 && d_v != 128 && d_v != 256 && d_v != 512) return ATTN_ERR_UNSUPPORTED;
  if (plan->n_partial_slots <= 0) return ATTN_OK;
  const size_t need = attn_decode_workspace_size(plan, h_q, d_v);
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return ATTN_ERR_WORKSPACE;
  if (!aligned16(out)) return ATTN_ERR_INVALID_ARG;
  Params p;
  std::memset(&p, 0, sizeof(p));
  p.out = out;
  p.lse = lse;
  p.seqinfo = plan->seqinfo;
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
