// Streaming decode kernel for latent heads (MLA, GLA) on gfx950.
//
// A latent group's keys are [latent_j || RoPE] rows and its values are the
// latent rows themselves ("Hardware-Efficient Attention for Fast Decoding",
// Core claim; the MLA and GLA definitions).  One workgroup of 2 KQ waves
// holds 32*RT query rows of a group (the group's heads times the query
// tokens, or a block of them) and streams the rows of its chunk through a
// ring of STAGES 64-key LDS stages filled by direct global->LDS loads.
// Configurations (RT row tiles per wave, KQ key parts, RH row parts):
// 256-wide latents (2, 4, 2), eight waves two per SIMD, or (4, 2, 2) for
// groups of more than 64 rows, four waves of 64 rows each (one per SIMD),
// which halves the LDS operand bytes per row and doubles the MFMAs per
// operand read; 512-wide latents (2, 2, 2), one wave per SIMD, or on small
// pages (1, 2, 4), eight waves two per SIMD.
//
// Work split inside a workgroup of RH KQ waves: wave (kq, rh) owns the row
// part rh (16*RT rows) and
//   * scores S^T = K Q^T for key part kq of every tile (64 / KQ keys; its
//     rows' queries stay in registers as MFMA B operands),
//   * O^T += V^T P^T for the value-column part kq of its rows over all 64
//     keys of the tile; the probabilities of the other key parts come from
//     the partner waves (kq', rh) through a small LDS buffer.
// So every K element is read from LDS by RH waves (one per row part) and
// every V element by RH, against 2 KQ for a split over rows alone.
//
// Tile schedules.  Plain: per tile, wait for its stage, scores, softmax,
// exchange barrier, P V.  Pipelined (256-wide latents, groups of more than
// 64 rows): step i computes the scores of tile i, then P V of tile i - 1
// with tile i's softmax interleaved into those MFMAs, behind one barrier
// per step; probabilities alternate between two LDS buffers and one tile
// is in flight instead of two.
//
// LDS layout of a stage (the LDS serves 256 bytes per clock when a read's
// lanes hit distinct banks): latent blocks of 1 KB (one 512-wide row, or
// two 256-wide rows) sit 1056 bytes apart (a stride of 32 mod 64 bytes), set
// by the LDS base of each direct-to-LDS load (one 1 KB load per block);
// within a two-row block the second row's units are XOR-ed with 8.  With
// that stride the 16-byte K reads of 16 consecutive keys and the
// transposing V^T reads run at the full rate, measured for every operand
// pattern of this kernel; strides of 0, 16 or 48 mod 64 bytes halve it.
// RoPE rows are 128 bytes, unpadded, with units XOR-ed by (row / 2) mod 8.
// Every operand address is then one or two per-lane bases plus an
// immediate offset, and each load needs a single per-lane offset register.
//
// Softmax: every row keeps a fixed reference max m_ref, the pair-wide max
// of its first tile (the visible keys of a chunk are a prefix of it, so
// rows with any visible key have one there), and O is never rescaled;
// probabilities exp2(s - m_ref) stay far from fp32 and bf16 overflow while
// every score is within 64 (log2 units) of m_ref.  A workgroup in which
// some lane's running sum of probabilities passes 2^64 (as it does once a
// score exceeds m_ref by 64) writes nothing and sets its flag; a second
// launch redoes exactly those workgroups with the classic online rescaling
// (RESCALE = true).
//
// Pages of at least 64 tokens hold whole tiles: one page id per tile, from
// an LDS table filled once per item.  Smaller pages (SP = true, any power of
// two down to single-token pages) give every row its own page: each wave
// loads the rows of 64 / (2 KQ) consecutive keys of a tile, and a 4-byte
// direct-to-LDS load per lane brings those keys' page ids into a small
// per-wave LDS ring a stage ahead of the cache loads that need them (the
// offsets are spread over the lanes, and no scalar or vector wait sits
// between a page-table read and its use).
#include "attn_device.h"
#include "attn_kernels.h"

#ifndef WIDE_KD512
#define WIDE_KD512 6
#endif
#ifndef WIDE_VD512
#define WIDE_VD512 4
#endif

namespace attn_dev {
namespace {
namespace wide {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;



// One direct global->LDS 16-byte load per lane from base + voff (base in
// SGPRs, voff a per-lane 32-bit byte offset); lane l writes LDS bytes
// [lds + 16 l, lds + 16 l + 16).  Issued from asm so that the compiler does
// not drain vmcnt before unrelated LDS reads; waits are explicit.  The
// nontemporal hint (nt) suits data read once and raises streaming read
// bandwidth by about a tenth on gfx950.
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(base),
               "s"(l) : "memory");
}
// The same with the default cache policy, for the RoPE key rows: every
// latent group of a sequence reads them, on one XCD, so the groups after
// the first find them in its L2.
__device__ __forceinline__ void dma16_cached(const char* base, uint32_t voff, uint32_t lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base),
               "s"(l) : "memory");
}


template <int DC, int DR> struct Geo {
  static_assert((DC == 256 || DC == 512) && DR == 64, "latent widths");
  static constexpr bool PAIR = DC == 256;    // two latent rows per 1 KB block
  static constexpr int BSTR = 1056;          // latent block stride (32 mod 64 bytes)
  static constexpr int LLOADS = PAIR ? 32 : 64;   // latent blocks (1 KB loads) per stage
  static constexpr int R_OFF = (LLOADS * BSTR + 1023) / 1024 * 1024;  // 1 KB aligned
  static constexpr int RLOADS = 8;           // 64 RoPE rows x 128 bytes
  static constexpr int LOADS = LLOADS + RLOADS;
  static constexpr int STAGE = R_OFF + RLOADS * 1024;
  static constexpr int NKC = (DC + DR) / 32;  // 32-dim k-chunks of a score
  static constexpr int NKL = DC / 32;         // ... of which latent
  static_assert(R_OFF % 1024 == 0, "RoPE block alignment");
};

// Per-workgroup context of one work item.
struct Item {
  int b, j, split, t0, t_end, n_tiles, n_splits, slot_base, L, rblk;
};

constexpr int PT_MAX = 512;  // tiles whose page ids are kept in LDS

// LDS of a workgroup: the ring, one probability buffer (two for the
// pipelined schedule) and the page-id table
template <int DC, int RT, int STAGES, bool PIPE, int RH = 2> constexpr int wide_lds_bytes() {
  return STAGES * Geo<DC, 64>::STAGE + (PIPE ? 2 : 1) * RH * 2 * RT * 1024 + PT_MAX * 4;
}

// Stream the item's chunk and write its output rows; returns true, writing
// nothing, when (RESCALE = false) some row outgrew its fixed reference.
template <int DC, int DR, int RT, int STAGES, int KQ, bool RESCALE, bool SP, bool PIPE, int RH>
__device__ __forceinline__ bool stream(const Params& p, const Item& itm, char* ring) {
  using G = Geo<DC, DR>;
  constexpr int NW = RH * KQ;          // waves: key part kq = wave % KQ, row part wave / KQ
  constexpr int KPW = 64 / KQ;         // keys per wave per tile
  constexpr int MT = KPW / 16;         // 16-key M tiles per wave
  constexpr int NDVW = DC / 16 / KQ;   // 16-wide value tiles per wave
  static_assert(KQ == 2 || KQ == 4, "key split");
  static_assert(G::LLOADS % NW == 0 && G::RLOADS % NW == 0, "loads split evenly over the waves");
  constexpr int LPW = G::LOADS / NW;   // loads per wave per stage
  constexpr int R_WG = 16 * RT * RH;   // rows per workgroup
  constexpr int PBUF = STAGES * G::STAGE;
  constexpr int PTAB = PBUF + (PIPE ? 2 : 1) * RH * 2 * RT * 1024;   // page-id table
  // small pages: wave w loads the rows of keys [KR w, KR w + KR) of a tile;
  // their page ids sit in a ring of STAGES slots of NW x 64 bytes at PTAB
  constexpr int KR = 64 / NW;
  static_assert(!SP || (KR <= 16 && STAGES * NW * 64 <= PT_MAX * 4), "page-id ring");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = wave % KQ, rh = wave / KQ;
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
    const int row = itm.rblk * R_WG + (rh * RT + rt) * 16 + col;
    row_ok[rt] = row < p.rows;
    tq[rt] = row_ok[rt] ? row / p.g : 0;
    hq[rt] = j * p.g + (row_ok[rt] ? row - tq[rt] * p.g : 0);
    qlimit[rt] = (p.causal && row_ok[rt]) ? L - p.q_len + tq[rt] : 0x7fffffff;
  }

  // ---- query B operands: Q^T[k = dims 32c + 8 grp ..][n = row]
  bf16x8 qreg[RT][G::NKC];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) +
                         ((int64_t)(b * p.q_len + tq[rt]) * p.h_q + hq[rt]) * (DC + DR);
#pragma unroll
    for (int c = 0; c < G::NKC; ++c) {
      uint4 raw = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok[rt]) raw = *reinterpret_cast<const uint4*>(qrow + c * 32 + grp * 8);
      qreg[rt][c] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- per-lane source offsets of the direct-to-LDS loads.  Latent: a
  // 1 KB block is one 512-wide row (lane = 16-byte unit) or two 256-wide
  // rows (lanes 32..63 take the second row, units XOR-ed with 8).  RoPE:
  // load k covers rows 8k .. 8k + 7 (lane / 8), units XOR-ed with
  // (row / 2) mod 8, which for this wave's loads depends on wave parity only.
  const int64_t lts2 = p.token_stride * 2, rts2 = p.rtoken_stride * 2;
  const int lrow = G::PAIR ? (lane >> 5) : 0;                   // row within the block
  const int lunit = G::PAIR ? ((lane & 31) ^ (8 * lrow)) : lane;  // source unit
  const uint32_t vlat = (uint32_t)(lrow * lts2 + lunit * 16);
  const int rrow = lane >> 3;                                    // row within the load
  const int runit = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
  const uint32_t vrope = (uint32_t)(rrow * rts2 + runit * 16);
  const uint32_t ring_base = lds_u32(ring);
  const int64_t head_off = (int64_t)j * p.head_stride;

  // small pages: the page ids of this wave's KR keys of tile x (clamped to
  // the last tile, each key to the last row) into ring slot x % STAGES
  const char* const pt_base = uniform_ptr(reinterpret_cast<const char*>(pt_row));
  auto issue_ids = [&](int x) __attribute__((always_inline)) {
    const int kw = t0 + min(x, n_tiles - 1) * 64 + KR * wave;
    const uint32_t voff = (uint32_t)(min(kw + lane, t_last) >> p.page_shift) * 4u;
    const uint32_t dst = ring_base + PTAB + ((x % STAGES) * NW + wave) * 64;
    if (lane < KR) dma4(pt_base, voff, dst);
  };

  int* const ptab = reinterpret_cast<int*>(ring + PTAB);
  if constexpr (SP) {
    // the page ids of the first STAGES - 1 tiles; later tiles' ids travel
    // with the cache loads, STAGES - 1 tiles ahead of them
    if (n_tiles > 0) {
      for (int x = 0; x < STAGES - 1; ++x) issue_ids(x);
    }
  } else {
    // page ids of the item's first PT_MAX tiles in an LDS table (later
    // tiles look theirs up in the page table)
    for (int tt = tid; tt < min(n_tiles, PT_MAX); tt += NW * 64)
      ptab[tt] = pt_row[(t0 + tt * 64) >> p.page_shift];
  }
  // the query and page-id loads must be complete before the asm loads
  // start counting, and the page-id table visible to every wave
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  __syncthreads();

  // This wave's loads of tile t (clamped to the last tile) into stage u:
  // `prepare` looks up the page and forms the bases, `issue_load` issues
  // load k of a full tile, `issue_clamped` all loads of a partial tile.
  constexpr int LK = G::LLOADS / NW, RK = G::RLOADS / NW;
  constexpr int RPB = G::PAIR ? 2 : 1;   // rows per latent block
  struct Fetch {
    const char* lbase;
    const char* rbase;
    uint32_t sbase;
    int valid;  // rows of the tile that exist
  };
  auto prepare_page = [&](int t, int u, int64_t page) __attribute__((always_inline)) {
    const int tt = min(t, n_tiles - 1);
    const int key0 = t0 + tt * 64;                  // 64-aligned, inside one page
    const int slot0 = key0 & pmask;
    Fetch f;
    f.valid = min(64, t_end - key0);
    f.lbase = uniform_ptr(
        p.pool0 + (page * p.page_stride + (int64_t)slot0 * p.token_stride + head_off) * 2);
    f.rbase =
        uniform_ptr(p.rope + (page * p.rpage_stride + (int64_t)slot0 * p.rtoken_stride) * 2);
    f.sbase = ring_base + u * G::STAGE;
    return f;
  };
  auto prepare = [&](int t, int u) __attribute__((always_inline)) {
    const int tt = min(t, n_tiles - 1);
    const int64_t page = tt < PT_MAX ? __builtin_amdgcn_readfirstlane(ptab[tt])
                                     : sload_i32(pt_row + ((t0 + tt * 64) >> p.page_shift));
    return prepare_page(t, u, page);
  };
  auto issue_load = [&](const Fetch& f, int k) __attribute__((always_inline)) {
    const int blk = wave + NW * (k < LK ? k : k - LK);
    if (k < LK)
      dma16(f.lbase + (int64_t)blk * RPB * lts2, vlat, f.sbase + blk * G::BSTR);
    else
      dma16_cached(f.rbase + (int64_t)blk * 8 * rts2, vrope, f.sbase + G::R_OFF + blk * 1024);
  };
  // a partial last tile: rows past the end re-read the last row, so that
  // stale cache contents never reach the MFMAs
  auto issue_clamped = [&](const Fetch& f) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < LK; ++k) {
      const int blk = wave + NW * k;
      const int r = min(blk * RPB + lrow, f.valid - 1);
      dma16(f.lbase, (uint32_t)(r * lts2 + lunit * 16), f.sbase + blk * G::BSTR);
    }
#pragma unroll
    for (int k = 0; k < RK; ++k) {
      const int blk = wave + NW * k;
      const int r = min(blk * 8 + rrow, f.valid - 1);
      dma16_cached(f.rbase, (uint32_t)(r * rts2 + runit * 16), f.sbase + G::R_OFF + blk * 1024);
    }
  };
  // Small pages: every row's address from its own page id (rows past the
  // end re-read the last row).  512-wide rows: one row per load, a uniform
  // address formed at issue from the ids held by lanes 0..KR-1; 256-wide
  // row pairs and RoPE rows (8 per load): per-lane addresses formed here.
  struct FetchSP {
    int kw;          // first key of this wave's rows
    int idv;         // 512-wide: lane i < KR holds the page id of row i
    uint64_t al[G::PAIR ? LK : 1];
    uint64_t ar[RK];
    uint32_t sbase;
  };
  auto prepare_sp = [&](int t, int u) __attribute__((always_inline)) {
    FetchSP f;
    f.kw = t0 + min(t, n_tiles - 1) * 64 + KR * wave;
    f.sbase = ring_base + u * G::STAGE;
    const int* ids = reinterpret_cast<const int*>(ring + PTAB + ((t % STAGES) * NW + wave) * 64);
    if constexpr (G::PAIR) {
#pragma unroll
      for (int k = 0; k < LK; ++k) {
        const int r = 2 * k + lrow;
        const int key = min(f.kw + r, t_last);
        f.al[k] = reinterpret_cast<uint64_t>(p.pool0) +
                  (uint64_t)(((int64_t)ids[r] * p.page_stride +
                              (int64_t)(key & pmask) * p.token_stride + head_off) * 2) +
                  lunit * 16;
      }
      f.idv = 0;
    } else {
      f.idv = ids[lane & (KR - 1)];
      f.al[0] = 0;
    }
#pragma unroll
    for (int k = 0; k < RK; ++k) {
      const int r = 8 * k + rrow;
      const int key = min(f.kw + r, t_last);
      const int blk = wave * RK + k;
      const int ru = (lane & 7) ^ ((4 * (blk & 1) + (lane >> 4)) & 7);
      f.ar[k] = reinterpret_cast<uint64_t>(p.rope) +
                (uint64_t)(((int64_t)ids[r] * p.rpage_stride +
                            (int64_t)(key & pmask) * p.rtoken_stride) * 2) +
                ru * 16;
    }
    return f;
  };
  auto issue_load_sp = [&](const FetchSP& f, int k) __attribute__((always_inline)) {
    if (k < LK) {
      const uint32_t dst = f.sbase + (wave * LK + k) * G::BSTR;
      if constexpr (G::PAIR) {
        dma16v(f.al[k], dst);
      } else {
        const int key = min(f.kw + k, t_last);
        const int64_t id = __builtin_amdgcn_readlane(f.idv, k);
        const char* base = uniform_ptr(
            p.pool0 + (id * p.page_stride + (int64_t)(key & pmask) * p.token_stride + head_off) * 2);
        dma16(base, vlat, dst);
      }
    } else {
      const int kk = k - LK;
      dma16v_cached(f.ar[kk], f.sbase + G::R_OFF + (wave * RK + kk) * 1024);
    }
  };

  auto issue = [&](int t, int u) __attribute__((always_inline)) {
    if constexpr (SP) {
      const FetchSP f = prepare_sp(t, u);
      issue_ids(t + STAGES - 1);
#pragma unroll
      for (int k = 0; k < LPW; ++k) issue_load_sp(f, k);
    } else {
      const Fetch f = prepare(t, u);
      if (f.valid == 64) {
#pragma unroll
        for (int k = 0; k < LPW; ++k) issue_load(f, k);
      } else {
        issue_clamped(f);
      }
    }
  };

  // per-lane operand bases inside a stage (bytes).  K operand of key row
  // r = KPW kq + 16 mt + col, unit 4 c + grp: 512-wide rows sit at r * BSTR;
  // 256-wide row r in block r / 2, half r % 2, unit XOR-ed with 8 (r % 2),
  // which moves unit 4 c + grp by +-8 units as bit 1 of c is clear / set
  int s_lat_p, s_lat_m;
  if constexpr (G::PAIR) {
    const int bb = col & 1;
    const int base = (KPW / 2 * kq + (col >> 1)) * G::BSTR + bb * 512 + grp * 16;
    s_lat_p = base + 128 * bb;
    s_lat_m = base - 128 * bb;
  } else {
    s_lat_p = s_lat_m = (KPW * kq + col) * G::BSTR + grp * 16;
  }
  // RoPE operand: row r as above, unit (4 c + grp) XOR (r / 2) mod 8, for
  // the two RoPE k-chunks c = 0, 1
  const int rx = (col >> 1) & 7;
  const int s_rope0 = G::R_OFF + (KPW * kq + col) * 128 + ((grp) ^ rx) * 16;
  const int s_rope1 = G::R_OFF + (KPW * kq + col) * 128 + ((4 + grp) ^ rx) * 16;
  // V^T operand (transposing reads): rows 32 kc + 4 grp + col / 4 (+16),
  // value units 2 d + (col % 4) / 2 with d = kq NDVW + dt, byte half col % 2;
  // 256-wide rows move by +-8 units as bit 2 of d is clear / set, which is
  // bit 2 of dt when NDVW is a multiple of 8 and bit 0 of kq when NDVW = 4
  int v_tr_p, v_tr_m;
  if constexpr (G::PAIR) {
    const int bb = (col >> 2) & 1;
    const int base = (2 * grp + (col >> 3)) * G::BSTR + bb * 512 + ((col & 3) >> 1) * 16 +
                     (col & 1) * 8 + kq * NDVW * 32;
    v_tr_p = base + 128 * bb;
    v_tr_m = base - 128 * bb;
    if (NDVW % 8 != 0 && (kq & 1)) v_tr_p = v_tr_m;
  } else {
    v_tr_p = v_tr_m = (4 * grp + (col >> 2)) * G::BSTR + ((col & 3) >> 1) * 16 + (col & 1) * 8 +
                      kq * NDVW * 32;
  }
  // probability exchange: slot (rh, 16-key block, rt) of 512 bytes, 8 bytes
  // per lane; a 32-key chunk's B operand is blocks 2 kc and 2 kc + 1
  char* const pbuf = ring + PBUF;
  const int p_lane = rh * 4 * RT * 512 + lane * 8;   // + (block * RT + rt) * 512
  const int t_wr = ((rh * KQ + kq) * RT) * 16 + col;    // + rt * 16; partners kq'
  const int t_rh = (rh * KQ * RT) * 16 + col;           // + (kq' * RT + rt) * 16

  f32x4 acc[RT][NDVW];
  float m_ref[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_ref[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int i = 0; i < NDVW; ++i) acc[rt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  float neg_m[RT];  // -(reference max), fixed after the first tile
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) neg_m[rt] = 0.f;

  // ---- the phases of a tile
  // scores S^T of this wave's KPW keys of the tile at stage base sb: MT M
  // tiles x RT row tiles.  The K operand reads run KD steps ahead of the
  // MFMAs that consume them (scheduling fences keep that order); when
  // `spread` (a compile-time flag: a branch around each load cost a lone
  // wave per SIMD about 7 % at q_len 4), load k of the fetch nf is issued
  // after step 2 k + 1.
  auto score_phase_c = [&](const char* sb, const auto& nf, auto spread_c,
                           f32x4 (&sa)[RT][MT]) __attribute__((always_inline)) {
    constexpr bool spread = decltype(spread_c)::value;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) sa[rt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int NS = MT * G::NKC;  // step = (chunk c, M tile mt)
    static_assert(NS >= 2 * LPW, "every load finds a step");
    constexpr int KD = DC >= 512 && RT > 1 ? WIDE_KD512 : 6;
    auto kread = [&](int st) __attribute__((always_inline)) {
      const int c = st / MT, mt = st % MT;
      const char* src;
      if (c < G::NKL)
        src = sb + (((c >> 1) & 1) ? s_lat_m : s_lat_p) + mt * (G::PAIR ? 8 : 16) * G::BSTR +
              c * 64;
      else
        src = sb + (c == G::NKL ? s_rope0 : s_rope1) + mt * 16 * 128;
      return *reinterpret_cast<const bf16x8*>(src);
    };
    bf16x8 kb[KD];
#pragma unroll
    for (int st = 0; st < KD; ++st) kb[st] = kread(st);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int c = st / MT, mt = st % MT;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        sa[rt][mt] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[st % KD], qreg[rt][c], sa[rt][mt], 0, 0, 0);
      if (st + KD < NS) kb[st % KD] = kread(st + KD);
      if ((st & 1) && (st >> 1) < LPW && spread) {
        if constexpr (SP)
          issue_load_sp(nf, st >> 1);
        else
          issue_load(nf, st >> 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto score_phase = [&](const char* sb, const auto& nf, bool spread,
                         f32x4 (&sa)[RT][MT]) __attribute__((always_inline)) {
    if (spread)
      score_phase_c(sb, nf, std::true_type{}, sa);
    else
      score_phase_c(sb, nf, std::false_type{}, sa);
  };

  // x = scale * score + nm (log2 units); lane holds keys
  // key0 + KPW kq + 16 mt + 4 grp + i of row col.  Masked keys of a partial
  // or causal tile: key - (key0 + KPW kq + 4 grp) = 16 mt + i must stay
  // below the row's limit min(t_end, qlimit + 1) - (key0 + KPW kq + 4 grp).
  // Keys below L - q_len + 1 are visible to every row of a causal group, so
  // only tiles that reach past that (or past the chunk) mask.
  auto scale_mask = [&](int key0, const f32x4 (&sa)[RT][MT], bool first,
                        float (&x)[RT][MT][4]) __attribute__((always_inline)) {
    const bool full = key0 + 64 <= (p.causal ? min(t_end, L - p.q_len + 1) : t_end);
    const int kbase = key0 + KPW * kq + 4 * grp;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float nm = first ? 0.f : neg_m[rt];
      const int lim = min(t_end, qlimit[rt] == 0x7fffffff ? t_end : qlimit[rt] + 1) - kbase;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = fmaf(sa[rt][mt][i], p.scale_log2, nm);
          if (!full && !(16 * mt + i < lim)) v = -INFINITY;
          x[rt][mt][i] = v;
        }
    }
  };

  // reference max shared by the waves (kq = 0 .. KQ-1) of a row half through
  // the slots `tx` (taken on the first tile; on every tile when rescaling);
  // `realias`: the slots alias the probability buffer about to be written
  auto take_reference = [&](float (&x)[RT][MT][4], float* tx,
                            bool realias) __attribute__((always_inline)) {
    float tmax[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[rt][mt][i]);
      tmax[rt] = wave_max4(mx);
    }
    if (grp == 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) tx[t_wr + rt * 16] = tmax[rt];
    }
    __syncthreads();
    float other[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      other[rt] = -INFINITY;
#pragma unroll
      for (int k2 = 0; k2 < KQ; ++k2) other[rt] = fmaxf(other[rt], tx[t_rh + (k2 * RT + rt) * 16]);
    }
    if (realias) __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float pair_max = fmaxf(tmax[rt], other[rt]);
      if constexpr (RESCALE) {
        const float m_new = fmaxf(m_ref[rt], pair_max);
        const float a = __builtin_amdgcn_exp2f(m_ref[rt] - ((m_new == -INFINITY) ? 0.f : m_new));
        l_run[rt] *= a;
#pragma unroll
        for (int dt = 0; dt < NDVW; ++dt) acc[rt][dt] *= a;
        m_ref[rt] = m_new;
      } else {
        m_ref[rt] = pair_max;
      }
      neg_m[rt] = (m_ref[rt] == -INFINITY) ? 0.f : -m_ref[rt];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[rt][mt][i] += neg_m[rt];
    }
  };

  // probabilities exp2(x) into the running sums and, as bf16, into this
  // wave's slots of the probability buffer pb
  auto write_probs = [&](const float (&x)[RT][MT][4], char* pb) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        bf16x4 pv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(x[rt][mt][i]);
          l_run[rt] += e;
          pv[i] = (__bf16)e;
        }
        *reinterpret_cast<bf16x4*>(pb + p_lane + ((kq * MT + mt) * RT + rt) * 512) = pv;
      }
    }
  };

  // O^T += V^T P^T over all 64 keys of the tile at stage base sb for this
  // wave's value part, probabilities from buffer pb; for the 32-key chunk
  // kc the A operand holds keys 32 kc + 4 grp + e (e < 4) and
  // 32 kc + 16 + 4 grp + (e - 4), matching the B operand written by the
  // waves kq with keys in that chunk
  auto pv_phase = [&](const char* sb, const char* pb, auto hook) __attribute__((always_inline)) {
    bf16x8 pk[2][RT];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(pb + p_lane + ((2 * kc) * RT + rt) * 512);
        const bf16x4 hi =
            *reinterpret_cast<const bf16x4*>(pb + p_lane + ((2 * kc + 1) * RT + rt) * 512);
        pk[kc][rt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    // step = (kc, dt); the two V^T reads of a step run VD steps ahead
    constexpr int NP = 2 * NDVW;
    constexpr int VD = DC >= 512 && RT > 1 ? WIDE_VD512 : 4;
    auto vread = [&](int st) __attribute__((always_inline)) {
      const int kc = st / NDVW, dt = st % NDVW;
      constexpr int RS = G::PAIR ? 16 : 32;   // blocks per 32 keys
      const char* s0 = sb + ((NDVW % 8 == 0 && ((dt >> 2) & 1)) ? v_tr_m : v_tr_p) +
                       kc * RS * G::BSTR + dt * 32;
      const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(s0));
      const bf16x4 v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(s0 + RS / 2 * G::BSTR));
      return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 vb[VD];
#pragma unroll
    for (int st = 0; st < VD; ++st) vb[st] = vread(st);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NP; ++st) {
      const int kc = st / NDVW, dt = st % NDVW;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt][dt] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[st % VD], pk[kc][rt], acc[rt][dt], 0, 0, 0);
      if (st + VD < NP) vb[st % VD] = vread(st + VD);
      hook(st);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const auto no_hook = [](int) __attribute__((always_inline)) {};

  // page id of tile t (clamped to the last tile) from the LDS table, read
  // a tile (or step) before use, so that no LDS wait follows the barrier;
  // tiles past the table read the page table at use
  auto page_of = [&](int t) __attribute__((always_inline)) {
    return ptab[min(min(t, n_tiles - 1), PT_MAX - 1)];
  };
  auto page_at = [&](int t, int pid) __attribute__((always_inline)) {
    const int tn = min(t, n_tiles - 1);
    return tn < PT_MAX ? (int64_t)__builtin_amdgcn_readfirstlane(pid)
                       : (int64_t)sload_i32(pt_row + ((t0 + tn * 64) >> p.page_shift));
  };
  if constexpr (!PIPE) {
    int pid = 0;
    if (n_tiles > 0) {
#pragma unroll
      for (int u = 0; u < STAGES - 1; ++u) issue(u, u);
      if constexpr (!SP) pid = page_of(STAGES - 1);
    }

    // One tile in stage U; when U is a compile-time constant every LDS
    // operand address is a per-lane base plus an immediate.
    auto tile = [&](int t, auto ucst) __attribute__((always_inline)) {
      const int U = static_cast<int>(ucst);
      {
        // loads per tile and wave: LPW cache loads (+ one page-id load)
        constexpr int ahead = (STAGES - 2) * (LPW + (SP ? 1 : 0));
        __builtin_amdgcn_s_waitcnt((ahead & 15) | ((ahead >> 4) << 14) | (0x7 << 4) | (0xf << 8));
      }
      // every wave's loads of tile t have landed, and every wave is done
      // with tile t - 1 (its stage and the probability buffer are free again)
      __syncthreads();
      // refill the stage of tile t - 1 with tile t + STAGES - 1: a full
      // tile's loads are spread over the score MFMAs, a partial one's issued
      // now (small pages: always spread, after the page ids of tile
      // t + 2 STAGES - 2)
      const auto nf = [&]() __attribute__((always_inline)) {
        if constexpr (SP) {
          return prepare_sp(t + STAGES - 1, (U + STAGES - 1) % STAGES);
        } else {
          const Fetch f = prepare_page(t + STAGES - 1, (U + STAGES - 1) % STAGES,
                                       page_at(t + STAGES - 1, pid));
          pid = page_of(t + STAGES);
          return f;
        }
      }();
      bool spread = true;
      if constexpr (SP) {
        issue_ids(t + 2 * STAGES - 2);
      } else {
        spread = nf.valid == 64;
        if (!spread) issue_clamped(nf);
      }
      const char* sb = ring + U * G::STAGE;
      f32x4 sa[RT][MT];
      score_phase(sb, nf, spread, sa);
      float x[RT][MT][4];
      const bool first = RESCALE || t == 0;
      scale_mask(t0 + t * 64, sa, first, x);
      if (first) take_reference(x, reinterpret_cast<float*>(pbuf), true);
      write_probs(x, pbuf);
      __syncthreads();  // every key part's probabilities are in the buffer
      pv_phase(sb, pbuf, no_hook);
    };

    // the tile loop, unrolled by the ring depth (constant stage addresses)
    // except for 512-wide latents with two row tiles per wave, whose
    // register budget does not hold two copies of the loop body
    constexpr bool UNROLL = !(DC >= 512 && RT > 1);
    if constexpr (UNROLL) {
      for (int t = 0; t < n_tiles; t += STAGES) {
        tile(t, std::integral_constant<int, 0>{});
        if (t + 1 < n_tiles) tile(t + 1, std::integral_constant<int, 1>{});
        if constexpr (STAGES > 2) {
          if (t + 2 < n_tiles) tile(t + 2, std::integral_constant<int, 2>{});
        }
      }
    } else {
      for (int t = 0; t < n_tiles; ++t) tile(t, t % STAGES);
    }
  } else {
    // Pipelined schedule: step i computes the scores of tile i and P V of
    // tile i - 1, so each tile needs one barrier (instead of one for its
    // stage and one for the probability exchange), and one wave's softmax
    // overlaps the other waves' MFMAs.  A tile then lives in its stage for
    // two steps: stage i % 3 holds tile i (scores), stage (i - 1) % 3 tile
    // i - 1 (P V) and stage (i + 1) % 3 receives tile i + 1, issued over the
    // score MFMAs of step i.  Probabilities alternate between two buffers.
    static_assert(DC == 256 && STAGES == 3 && !SP && !RESCALE, "pipelined schedule");
    constexpr int PBS = RH * 2 * RT * 1024;
    int pid = 0;
    auto step = [&](int i, auto ucst) __attribute__((always_inline)) {
      const int U = static_cast<int>(ucst);
      // tile i has landed (no other loads are in flight), every wave is done
      // with step i - 1: tile i - 2's stage and probability buffer i % 2 are
      // free, tile i - 1's probabilities are complete
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      const bool more = i + 1 < n_tiles;
      const Fetch nf = prepare_page(i + 1, (U + 1) % 3, page_at(i + 1, pid));
      pid = page_of(i + 2);
      const bool spread = more && nf.valid == 64;
      if (more && !spread) issue_clamped(nf);
      f32x4 sa[RT][MT];
      score_phase(ring + U * G::STAGE, nf, spread, sa);
      if (i == 0) {
        float x[RT][MT][4];
        scale_mask(t0, sa, true, x);
        take_reference(x, reinterpret_cast<float*>(pbuf + PBS), false);
        write_probs(x, pbuf);
      } else {
        // this tile's softmax rides along the P V MFMAs of the previous one:
        // probability u (row tile, M tile, element) after P V step u
        const int key0 = t0 + i * 64;
        const bool full = key0 + 64 <= (p.causal ? min(t_end, L - p.q_len + 1) : t_end);
        if (!full) {
          float x[RT][MT][4];
          scale_mask(key0, sa, false, x);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (x[rt][mt][e] == -INFINITY) sa[rt][mt][e] = -INFINITY;
        }
        char* const pw = pbuf + (i & 1) * PBS;
        bf16x4 pv[RT][MT];
        constexpr int NU = RT * MT * 4;
        static_assert(NU % (2 * NDVW) == 0 || (2 * NDVW) % NU == 0, "units per step");
        auto hook = [&](int st) __attribute__((always_inline)) {
          constexpr int NP = 2 * NDVW;
          constexpr int PER = NU >= NP ? NU / NP : 1;
          if (NU < NP && st >= NU) return;
#pragma unroll
          for (int q = 0; q < PER; ++q) {
            const int u = st * PER + q;
            const int rt = u / (MT * 4), mt = (u / 4) % MT, e = u % 4;
            const float ex = __builtin_amdgcn_exp2f(fmaf(sa[rt][mt][e], p.scale_log2, neg_m[rt]));
            l_run[rt] += ex;
            pv[rt][mt][e] = (__bf16)ex;
            if (e == 3)
              *reinterpret_cast<bf16x4*>(pw + p_lane + ((kq * MT + mt) * RT + rt) * 512) = pv[rt][mt];
          }
        };
        pv_phase(ring + ((U + 2) % 3) * G::STAGE, pbuf + ((i - 1) & 1) * PBS, hook);
      }
    };
    if (n_tiles > 0) {
      issue(0, 0);
      pid = page_of(1);
      step(0, std::integral_constant<int, 0>{});
      for (int i = 1; i < n_tiles; i += 3) {
        step(i, std::integral_constant<int, 1>{});
        if (i + 1 < n_tiles) step(i + 1, std::integral_constant<int, 2>{});
        if (i + 2 < n_tiles) step(i + 2, std::integral_constant<int, 0>{});
      }
      __syncthreads();  // the last tile's probabilities are complete
      const int ul = (n_tiles - 1) % 3;
      pv_phase(ring + ul * G::STAGE, pbuf + ((n_tiles - 1) & 1) * PBS, no_hook);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // drain the clamped trailing loads
  __syncthreads();                // the ring is free

  // ---- workgroup-wide restart decision and the pair's row sums
  int* const flag = reinterpret_cast<int*>(ring);
  float* const lx = reinterpret_cast<float*>(ring + 256);
  // A probability above 2^64 (a score more than 64 above the reference,
  // log2 units) leaves a lane's running sum above 2^64 (or inf / NaN); so
  // does a sum that large of smaller ones, which the rescaling pass also
  // handles exactly.  The vote covers all lanes of the wave, taken before a
  // single lane stores it.
  bool over = false;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) over |= !(l_run[rt] <= 0x1p64f);
  const bool wave_over = __builtin_amdgcn_ballot_w64(over) != 0;
  if (!RESCALE && lane == 0) flag[wave] = wave_over ? 1 : 0;
  float lsum[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    lsum[rt] = wave_sum4(l_run[rt]);
    if (grp == 0) lx[t_wr + rt * 16] = lsum[rt];
  }
  __syncthreads();
  if constexpr (!RESCALE) {
    int any = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any |= flag[w];
    if (any) return true;
  }

  // ---- epilogue: lane holds O^T[dv = DC/KQ kq + 16 dt + 4 grp + i][row]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l_row = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < KQ; ++k2) l_row += lx[t_rh + (k2 * RT + rt) * 16];
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    const float lse_val =
        l_row > 0.f ? (m_ref[rt] + __log2f(l_row)) * 0.69314718055994531f : -INFINITY;
    if (!row_ok[rt]) continue;
    const int64_t orow = (int64_t)(b * p.q_len + tq[rt]) * p.h_q + hq[rt];
    const int dv0 = kq * (DC / KQ) + grp * 4;
    if (itm.n_splits <= 1) {
      __bf16* o = reinterpret_cast<__bf16*>(p.out) + orow * DC + dv0;
#pragma unroll
      for (int dt = 0; dt < NDVW; ++dt) {
        __bf16 v4[4] = {(__bf16)(acc[rt][dt][0] * inv), (__bf16)(acc[rt][dt][1] * inv),
                        (__bf16)(acc[rt][dt][2] * inv), (__bf16)(acc[rt][dt][3] * inv)};
        *reinterpret_cast<uint2*>(o + dt * 16) = __builtin_bit_cast(uint2, v4);
      }
      if (p.lse && kq == 0 && grp == 0) p.lse[orow] = lse_val;
    } else {
      const int64_t prow =
          (int64_t)((itm.slot_base + itm.split) * p.q_len + tq[rt]) * p.h_q + hq[rt];
      float* o = p.o_part + prow * DC + dv0;
      if (p.fuse_merge) {
#pragma unroll
        for (int dt = 0; dt < NDVW; ++dt) store_partial4(o + dt * 16, acc[rt][dt] * inv);
        if (kq == 0 && grp == 0) store_partial(p.lse_part + prow, lse_val);
      } else {
#pragma unroll
        for (int dt = 0; dt < NDVW; ++dt)
          *reinterpret_cast<f32x4*>(o + dt * 16) = acc[rt][dt] * inv;
        if (kq == 0 && grp == 0) p.lse_part[prow] = lse_val;
      }
    }
  }
  // the last split of this (sequence, group, row block) to finish merges
  // all splits of its rows
  if (itm.n_splits > 1 && p.fuse_merge) {
    const int row0 = itm.rblk * R_WG;
    arrive_and_merge<DC>(p, p.counters + ((int64_t)b * (p.h_q / p.g) + j) * p.row_blocks + itm.rblk,
                         reinterpret_cast<int*>(ring + 4096), b, j, row0, min(R_WG, p.rows - row0),
                         itm.n_splits, itm.slot_base);
  }
  return false;
}

// RESCALE = false: the fixed-reference pass; records per workgroup whether
// it had to give up (flags[block]).  RESCALE = true: the fix-up pass, a
// second launch over the same grid that only works where the flag is set.
// PIPE: the pipelined tile schedule (fixed-reference pass only).  RH row
// parts x KQ key parts = RH KQ waves, RH KQ / 4 per SIMD.
template <int DC, int DR, int RT, int STAGES, int KQ, bool RESCALE, bool SP, bool PIPE, int RH>
__global__ __launch_bounds__(RH * KQ * 64)
__attribute__((amdgpu_waves_per_eu(RH * KQ / 4, RH * KQ / 4)))
void decode_wide(Params p) {
  using G = Geo<DC, DR>;
  constexpr int LDS = wide_lds_bytes<DC, RT, STAGES, PIPE, RH>();
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert((STAGES - 2) * (G::LOADS / (RH * KQ) + 1) <= 63, "vmcnt range");
  static_assert(STAGES == 2 || STAGES == 3, "tile loop unrolled for 2 or 3 stages");
  __shared__ __attribute__((aligned(1024))) char ring[LDS];

  if constexpr (RESCALE) {
    if (p.flags[blockIdx.x] == 0) return;
  }
  // Item and row block.  The plan lists the groups of one (sequence, chunk)
  // consecutively; all their row blocks are mapped to blocks 8 apart, so
  // they run on one XCD and share its L2 (the groups read the same RoPE key
  // rows, the row blocks the same latent rows).
  const int rb_count = p.row_blocks;
  const int n_groups = p.h_q / p.g;
  const int per = n_groups * rb_count;   // workgroups of one (sequence, chunk)
  const int bid = blockIdx.x;
  const int blk8 = bid / (8 * per);
  const int rem = bid - blk8 * 8 * per;
  const int unit = blk8 * 8 + (rem & 7);
  const int sub = rem >> 3;
  const int jl = sub / rb_count;
  Item itm;
  itm.rblk = sub - jl * rb_count;
  const int item = unit * n_groups + jl;
  if (item >= p.n_items) return;
  const PlanItem pi = load_item(p, item);
  itm.b = pi.b;
  itm.j = pi.j;
  itm.split = pi.split;
  itm.t0 = pi.t0;
  itm.n_splits = pi.n_splits;
  itm.slot_base = pi.slot_base;
  itm.L = pi.L;
  const int chunk = pi.chunk;
  itm.t_end = min(itm.t0 + chunk, itm.L);
  itm.n_tiles = (itm.t_end - itm.t0 + 63) / 64;

  const bool gave_up = stream<DC, DR, RT, STAGES, KQ, RESCALE, SP, PIPE, RH>(p, itm, ring);
  if constexpr (!RESCALE) {
    if (threadIdx.x == 0) p.flags[blockIdx.x] = gave_up ? 1 : 0;
  }
}

}  // namespace wide

// RH row parts of RT row tiles (16 RT RH rows per workgroup), KQ key parts.
// The fix-up pass runs the same grid with two row halves of RH RT / 2 row
// tiles (the same rows per workgroup).
template <int DC, int DR, int RT, int S, int KQ, bool SP, int RH = 2>
int launch_wide_one(Params p, int n_items, hipStream_t stream) {
  static_assert(RH == 2 || (RH == 4 && RT == 1), "row parts");
  constexpr int RTF = RT * RH / 2;   // row tiles per wave of the fix-up pass
  p.n_items = n_items;
  p.row_blocks = (p.rows + 16 * RT * RH - 1) / (16 * RT * RH);
  const int n_groups = p.h_q / p.g;
  const int units = (n_items + n_groups - 1) / n_groups;   // (sequence, chunk) pairs
  const dim3 grid((units + 7) / 8 * 8 * n_groups * p.row_blocks);
  // 128-row workgroups run the pipelined schedule: it holds one tile in
  // flight instead of two but needs one barrier per tile instead of two,
  // and interleaves the softmax into the P V MFMAs, which a single wave per
  // SIMD needs (measured against the plain schedule with 64-row workgroups:
  // +31 % at q_len 4; with 64-row workgroups the pipelined form gained 12 %
  // at q_len 4 and lost 3-7 % at q_len 1, where one tile in flight is too
  // little to stream from HBM).
  if constexpr (RT == 4) {
    static_assert(DC == 256 && S == 3 && !SP, "128-row workgroups: 256-wide, whole tiles");
    hipLaunchKernelGGL((wide::decode_wide<DC, DR, RT, S, KQ, false, SP, true, RH>), grid,
                       dim3(RH * KQ * 64), 0, stream, p);
  } else {
    hipLaunchKernelGGL((wide::decode_wide<DC, DR, RT, S, KQ, false, SP, false, RH>), grid,
                       dim3(RH * KQ * 64), 0, stream, p);
  }
  // fix-up pass: exits at once unless the first pass flagged the workgroup
  hipLaunchKernelGGL((wide::decode_wide<DC, DR, RTF, S, KQ, true, SP, false, 2>), grid,
                     dim3(2 * KQ * 64), 0, stream, p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// Two row tiles per wave (64 rows per workgroup) unless the group has at
// most 32 rows; as many 64-key stages as fit the LDS beside the probability
// buffer (2 for 512-wide latents, 3 for 256-wide).  256-wide latents split
// each tile's keys four ways over eight waves (two per SIMD, so one wave's
// softmax and waits overlap another's MFMAs); 512-wide latents need the
// register budget of one wave per SIMD and split keys two ways.
template <int DC, int DR, bool SP>
int launch_wide_sp(const Params& p, int n_items, hipStream_t stream) {
  constexpr int S = (DC >= 512) ? 2 : 3;
  constexpr int KQ = attn_internal::wide_kq(DC);
  if constexpr (DC == 256 && !SP) {
    if (attn_internal::wide_rows128(DC, p.rows, 64))
      return launch_wide_one<DC, DR, 4, S, 2, SP>(p, n_items, stream);
  }
  if constexpr (attn_internal::wide_rt(DC, 64) == 1) {
    return launch_wide_one<DC, DR, 1, S, KQ, SP>(p, n_items, stream);
  } else {
    if (attn_internal::wide_rt(DC, p.rows) == 1)
      return launch_wide_one<DC, DR, 1, S, KQ, SP>(p, n_items, stream);
    // 512-wide latents with 33-128 rows on pages under 64 tokens: four row
    // parts of one row tile (eight waves, two per SIMD) instead of two of
    // two (four waves, one per SIMD), the same 64 rows per workgroup; more
    // waves issue the per-row loads (MLA at q_len 1, pages of 1 / 4 / 16
    // tokens: +4 to +7 %).  With whole-tile pages, or more rows (q_len 4:
    // -2.5 % at pages of 16), the eight waves' doubled K and V operand reads
    // cost more than their overlap gains (-2 % to -5 %).
    if constexpr (DC >= 512 && SP) {
      if (p.rows <= 128) return launch_wide_one<DC, DR, 1, S, KQ, SP, 4>(p, n_items, stream);
    }
    return launch_wide_one<DC, DR, 2, S, KQ, SP>(p, n_items, stream);
  }
}

// pages of fewer than 64 tokens: per-row page ids
template <int DC, int DR>
int launch_wide(const Params& p, int n_items, hipStream_t stream) {
  return p.page_shift < 6 ? launch_wide_sp<DC, DR, true>(p, n_items, stream)
                          : launch_wide_sp<DC, DR, false>(p, n_items, stream);
}

}  // namespace

int run_wide(int d_c, const Params& p, int n_items, hipStream_t stream) {
  return d_c == 512 ? launch_wide<512, 64>(p, n_items, stream)
                    : launch_wide<256, 64>(p, n_items, stream);
}

}  // namespace attn_dev
