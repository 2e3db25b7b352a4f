// Streaming decode kernel for narrow groups (GQA, GTA) on gfx950.
#include "attn_device.h"

namespace attn_dev {
namespace {

// ----------------------------------------------------------------------------
// Streaming kernel for narrow groups (GQA, GTA; at most 16*RT query rows per
// group, bf16, pages of >= 64 tokens).
//
// Four waves share one work item and split every 64-key tile: wave w owns
// keys [16w, 16w + 16).  Each wave streams its slices through a private ring
// of STAGES LDS buffers filled by direct global->LDS 16-byte loads, so a wave
// waits only on its own loads (vmcnt) and the main loop has no barriers.
// Rows are stored with 16-byte chunks XOR-swizzled by a function of the key
// index (chunk_swz) so the K-operand reads of 16 keys and the transposing V
// reads hit distinct banks.
// Per 16-key slice: S^T = K Q^T (MFMA 16x16x32), online softmax, and
// O^T += V^T P^T with MFMA 16x16x16 whose V^T operand comes from
// ds_read_b64_tr_b16.  The waves' (max, sum, O) states are merged through
// LDS at the end of the item.
// Groups of 33-64 rows on pages of at least 16 tokens (RH = 2): eight waves,
// two row halves of 32 rows over the same keys.  The two waves of a key
// slice each load half of it into one shared ring, so each tile waits on
// both (its own vmcnt, then one barrier per tile) and the ring, as deep as
// the LDS holds with one workgroup per CU, keeps more of the cache in flight
// than two 32-row workgroups that each read every tile.
namespace narrow {

constexpr int NW = 4;    // waves per workgroup
constexpr int KW = 16;   // keys per wave per tile
constexpr int KTILE = NW * KW;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

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
  // per-wave bytes of one stage: K (or tied) rows, V rows (GQA), the second
  // group's tied rows (GTA2), RoPE rows (GTA, GTA2)
  static constexpr int NT = KIND == GTA2 ? 2 : 1;   // tied groups per stage
  static constexpr int ROW0 = D * 2;                 // K / tied row bytes
  static constexpr int ROWR = DR * 2;                // RoPE row bytes
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = KW * ROW0;            // GQA only
  static constexpr int K2_OFF = KW * ROW0;           // GTA2 only
  static constexpr int R_OFF = NT * KW * ROW0;       // GTA, GTA2
  static constexpr int WAVE_BYTES = (KIND == GQA) ? 2 * KW * ROW0 : KW * (NT * ROW0 + ROWR);
  static constexpr int STAGE_BYTES = NW * WAVE_BYTES;
  static constexpr int LOADS = WAVE_BYTES / 1024;
};

// 16-byte chunk c of row r of a stage sits at chunk position
// c ^ chunk_swz(r, CPR).  Rows of 16 chunks (256 bytes, so every row starts
// at bank 0) swizzle by 2 r: the transposing V reads of a 32-lane group
// cover 8 rows x 2 chunks, which then hit 16 distinct 16-byte bank groups
// (swizzling by r puts chunks 2 d and 2 d + 1 of rows r and r ^ 1 on the
// same banks and halves their rate, measured); rows of 8 chunks (128 bytes,
// two rows per bank period) swizzle by r.  The K-operand reads of 16 keys
// run at the full rate with either.
__device__ __forceinline__ constexpr int chunk_swz(int r, int cpr) {
  return cpr >= 16 ? (2 * r) & (cpr - 1) : r & (cpr - 1);
}

// Per-lane byte offsets of the direct-to-LDS loads of one 16-key slice of
// rows of ROWB bytes: lane l of load i covers row i*RPI + l/CPR at swizzled
// chunk position l%CPR, i.e. it fetches logical chunk
// (l%CPR) ^ chunk_swz(row, CPR).
// Cache policy of the cache loads: nontemporal (streaming).  Every cache
// row is read once per call, and the hint raises streaming read bandwidth
// by about a tenth on gfx950.
constexpr int kStreamPolicy = 2;  // nt
// The GTA RoPE key rows are shared by every group of a sequence, whose
// workgroups run on one XCD: loaded with the default policy, so that the
// groups after the first find them in its L2.
constexpr int kSharedPolicy = 0;

template <int ROWB, int POLICY = kStreamPolicy>
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
      const int c = (lane % CPR) ^ chunk_swz(row[i], CPR);
      off[i] = (uint32_t)(row[i] * token_stride * 2 + c * 16);
    }
  }
  // pages smaller than a slice: byte offsets of this lane's rows from the
  // pool base, each row key min(kw + row, t_last) in its own page (ids[] =
  // page id per key of the slice, from LDS)
  __device__ __forceinline__ void offsets_sp(uint64_t* o, const int* ids, int kw, int t_last,
                                             int pmask, int64_t page_stride, int64_t token_stride,
                                             int64_t head_off) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int key = min(kw + row[i], t_last);
      o[i] = (uint64_t)(((int64_t)ids[row[i]] * page_stride + (int64_t)(key & pmask) * token_stride +
                         head_off) * 2) +
             (off[i] - (uint32_t)(row[i] * token_stride * 2));
    }
  }
  __device__ __forceinline__ void issue_sp(char* dst, const char* base, const uint64_t* o) const {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (POLICY == kStreamPolicy)
        dma16v(b + o[i], lds_u32(dst + i * 1024));
      else
        dma16v_cached(b + o[i], lds_u32(dst + i * 1024));
    }
  }
  // full slice: every row valid, contiguous within one page
  __device__ __forceinline__ void issue(char* dst, const char* base) const {
#pragma unroll
    for (int i = 0; i < N; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(base + off[i]), (lds_void_t*)(dst + i * 1024),
                                       16, 0, POLICY);
  }
  // partial slice: rows at or past `valid` re-read row valid-1 (same page)
  __device__ __forceinline__ void issue_clamped(char* dst, const char* base, int valid,
                                                int64_t token_stride) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = min(row[i], valid - 1);
      const char* src = base + off[i] + (int64_t)(r - row[i]) * token_stride * 2;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(dst + i * 1024), 16, 0,
                                       POLICY);
    }
  }
  // the same for a wave that shares the slice with another: loads
  // 2 k + h (h = 0, 1) only; the per-load values are selected, not indexed,
  // so they stay in registers
  __device__ __forceinline__ void issue_clamped_half(char* dst, const char* base, int valid,
                                                     int64_t token_stride, int h) const {
    static_assert(N % 2 == 0, "two equal parts");
#pragma unroll
    for (int k = 0; k < N / 2; ++k) {
      const int rw = h ? row[2 * k + 1] : row[2 * k];
      const uint32_t o = h ? off[2 * k + 1] : off[2 * k];
      const int r = min(rw, valid - 1);
      const char* src = base + o + (int64_t)(r - rw) * token_stride * 2;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(dst + (2 * k + h) * 1024),
                                       16, 0, POLICY);
    }
  }
};

template <int KIND, int D, int DR, int RT, int STAGES, bool SP, int RH>
// Two workgroups (two waves per SIMD) share a CU up to two row tiles per
// wave: with two, the register budget is held to that (one row tile fits
// without asking; four: one wave per SIMD).  RH = 2: one workgroup of
// eight waves, two row halves over the same keys (two waves per SIMD).
__global__ __launch_bounds__(NW * RH * 64) __attribute__((amdgpu_waves_per_eu(RT == 2 ? 2 : 1)))
void decode_narrow(Params p) {
  using G = Geo<KIND, D, DR>;
  constexpr bool TIED = KIND != GQA;   // tied state + one RoPE key head
  constexpr bool PAIR = KIND == GTA2;  // two groups per work item
  constexpr int DN = D - DR;          // key entries from the K / tied row
  constexpr int NKC = D / 32;         // 32-dim k-chunks of the score MFMA
  constexpr int NDVT = D / 16;        // 16-wide output tiles
  constexpr int CPR0 = G::ROW0 / 16;
  constexpr int CPRR = (DR > 0) ? G::ROWR / 16 : 1;
  static_assert(STAGES >= 2 && STAGES <= 6, "stages");
  static_assert(G::LOADS * 1024 == G::WAVE_BYTES, "whole 1 KB load instructions");
  static_assert(RH == 1 || (RH == 2 && !SP && !PAIR), "row halves: whole slices, one group");
  // cache loads per tile of one wave (+ the page-id load of small pages)
  constexpr int LW = G::LOADS / RH + (SP ? 1 : 0);

  __shared__ __attribute__((aligned(1024))) char st0[G::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st1[G::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st2[STAGES > 2 ? G::STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char st3[STAGES > 3 ? G::STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char st4[STAGES > 4 ? G::STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char st5[STAGES > 5 ? G::STAGE_BYTES : 16];
  __shared__ float merge_m[RH][NW][16 * RT], merge_l[RH][NW][16 * RT];
  __shared__ int merge_last;
  // pages smaller than a slice (SP): page ids of each wave's 16 keys of a
  // tile, in a ring of STAGES + 1 slots, loaded STAGES tiles ahead
  constexpr int PSLOTS = STAGES + 1;
  __shared__ int pid[SP ? PSLOTS * NW * KW : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // key wave (keys [16 wave, 16 wave + 16) of every tile) and row half
  const int wave = __builtin_amdgcn_readfirstlane(RH == 1 ? tid >> 6 : (tid >> 6) % NW);
  const int half = RH == 1 ? 0 : __builtin_amdgcn_readfirstlane((tid >> 6) / NW);
  const int col = lane & 15;
  const int grp = lane >> 4;

  // Workgroups are dealt round-robin to the 8 XCDs (block i -> XCD i % 8).
  // The plan lists the groups of one (sequence, chunk) consecutively; with
  // gsz > 1 they are mapped to blocks 8 apart so they share one XCD's L2
  // (GTA's RoPE key rows are read by every group); gsz = 1 keeps plan order.
  // With a work queue (GQA) the grid holds as many workgroups as the GPU
  // keeps resident: block i takes item i first, and later items go to the
  // workgroups that finish first, whatever their XCD.  Groups of more than
  // 32 rows without row halves split into nrb workgroups of 32 rows (row
  // block rblk), which run on the same XCD: the second reads the item's
  // cache rows from its L2.
  const int gsz = p.row_blocks;  // items per unit kept on one XCD
  const int nrb = p.nrb;         // workgroups per item
  const int bid = blockIdx.x;
  const int blk = bid / (8 * gsz * nrb);
  const int rem = bid - blk * 8 * gsz * nrb;
  const int rblk = (rem >> 3) % nrb;
  __shared__ int next_item;
  uint32_t ticket = 0;

  // GTA RoPE table per frequency k = 8 grp + u: revolutions per position as
  // hi + lo floats, and cos / sin of one tile (64 positions) of it
  __shared__ float rope_tab[TIED ? 32 * 4 : 1];
  if constexpr (TIED) {
    if (tid < 32) {
      const float hi = p.rope_hi[tid], lo = p.rope_lo[tid];
      float r = hi * (float)KTILE;  // exact (a power of two)
      r -= floorf(r);
      r += lo * (float)KTILE;
      r -= floorf(r);
      rope_tab[4 * tid + 0] = hi;
      rope_tab[4 * tid + 1] = lo;
      rope_tab[4 * tid + 2] = __builtin_amdgcn_cosf(r);
      rope_tab[4 * tid + 3] = __builtin_amdgcn_sinf(r);
    }
    __syncthreads();
  }
  // GTA2 works on pairs of plan items: items 2i and 2i + 1 are groups
  // j, j + 1 (j even) of one (sequence, chunk)
  const int n_units = PAIR ? p.n_items / 2 : p.n_items;
  for (int item = (blk * 8 + (rem & 7)) * gsz + (rem >> 3) / nrb; item < n_units;) {
  const PlanItem pi = load_item(p, PAIR ? 2 * item : item);
  const int b = pi.b, j = pi.j, split = pi.split, t0 = pi.t0;
  const int n_splits = pi.n_splits, slot_base = pi.slot_base, L = pi.L, chunk = pi.chunk;
  const int t_end = min(t0 + chunk, L);
  const int n_tiles = (t_end - t0 + KTILE - 1) / KTILE;
  const int t_last = t_end - 1;
  const int pmask = (1 << p.page_shift) - 1;
  const int32_t* pt_row = p.page_table + (int64_t)b * p.max_pages;

  // rows of this lane (every wave of a row half holds all of its rows); GTA2: rows
  // [0, p.rows) belong to group j, rows [p.rows, 2 p.rows) to group j + 1
  int tq[RT], hq[RT], qlimit[RT];
  bool row_ok[RT], row_b[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = ((rblk * RH + half) * RT + rt) * 16 + col;
    row_ok[rt] = row < (PAIR ? 2 : 1) * p.rows;
    row_b[rt] = PAIR && row >= p.rows;
    const int rr = row_b[rt] ? row - p.rows : row;
    tq[rt] = row_ok[rt] ? rr / p.g : 0;
    hq[rt] = (j + (row_b[rt] ? 1 : 0)) * p.g + (row_ok[rt] ? rr - tq[rt] * p.g : 0);
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
  SliceDMA<(DR > 0 ? G::ROWR : 16), kSharedPolicy> dmar;
  dma0.init(p.token_stride, lane);
  if constexpr (TIED) dmar.init(p.rtoken_stride, lane);

  // small pages: the page ids of this wave's 16 keys of tile x (clamped to
  // the last tile, each key to the last row), one 4-byte load per lane
  const char* const pt_base = uniform_ptr(reinterpret_cast<const char*>(pt_row));
  auto issue_ids = [&](int x) {
    const int kw = t0 + min(x, n_tiles - 1) * KTILE + wave * KW;
    const uint32_t voff = (uint32_t)(min(kw + lane, t_last) >> p.page_shift) * 4u;
    if (lane < KW) dma4(pt_base, voff, lds_u32(&pid[((x % PSLOTS) * NW + wave) * KW]));
  };

  // issue this wave's loads of tile `t` (clamped to the last tile) into stage u
  auto issue = [&](int t, int u) {
    if constexpr (SP) {
      // every row from its own page (rows past the end re-read the last
      // row); then the page ids of tile t + STAGES
      const int kw = t0 + min(t, n_tiles - 1) * KTILE + wave * KW;
      const int* ids = &pid[((t % PSLOTS) * NW + wave) * KW];
      char* dst = stage(u) + wave * G::WAVE_BYTES;
      uint64_t o[SliceDMA<G::ROW0>::N];
      dma0.offsets_sp(o, ids, kw, t_last, pmask, p.page_stride, p.token_stride,
                      (int64_t)j * p.head_stride);
      dma0.issue_sp(dst + G::K_OFF, p.pool0, o);
      // GTA2: the second group's rows sit one head further on
      if constexpr (PAIR) dma0.issue_sp(dst + G::K2_OFF, p.pool0 + p.head_stride * 2, o);
      if constexpr (KIND == GQA) {
        dma0.issue_sp(dst + G::V_OFF, p.pool1, o);
      } else {
        uint64_t orr[SliceDMA<(DR > 0 ? G::ROWR : 16), kSharedPolicy>::N];
        dmar.offsets_sp(orr, ids, kw, t_last, pmask, p.rpage_stride, p.rtoken_stride, 0);
        dmar.issue_sp(dst + G::R_OFF, p.rope, orr);
      }
      issue_ids(t + STAGES);
      return;
    }
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
    // row halves: the two waves of a slice issue alternate loads of it
    auto part = [&](const auto& dma, char* d, const char* base, int64_t ts) {
      if constexpr (RH == 1) {
        dma.issue_clamped(d, base, v, ts);
      } else {
        dma.issue_clamped_half(d, base, v, ts, half);
      }
    };
    part(dma0, dst + G::K_OFF, b0, p.token_stride);
    if constexpr (PAIR) dma0.issue_clamped(dst + G::K2_OFF, b0 + p.head_stride * 2, v, p.token_stride);
    if constexpr (KIND == GQA) {
      part(dma0, dst + G::V_OFF, p.pool1 + row0 * 2, p.token_stride);
    } else {
      part(dmar, dst + G::R_OFF,
           p.rope + (page * p.rpage_stride + (int64_t)slot0 * p.rtoken_stride) * 2,
           p.rtoken_stride);
    }
  };

  // this lane's RoPE frequencies are entries 8 grp + u of rope_tab; the
  // rotation of its key (key0 + col) is kept as sin / cos per frequency,
  // advanced by one tile per slice and recomputed exactly every 16 tiles
  const float* rtab = rope_tab + (TIED ? 32 * grp : 0);
  float rsn[8], rcs[8];

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
    if constexpr (TIED) {
      if (p.rope_on) {
        constexpr int c0 = DN / 32;
        const float qpos = (float)(L - p.q_len + tq[rt]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          float sn, cs;
          rope_sincos(qpos, rtab[4 * u], rtab[4 * u + 1], sn, cs);
          const float x = (float)qreg[rt][c0][u], y = (float)qreg[rt][c0 + 1][u];
          qreg[rt][c0][u] = (__bf16)(x * cs - y * sn);
          qreg[rt][c0 + 1][u] = (__bf16)(x * sn + y * cs);
        }
      }
    }
  }

  // The cache loads are asm the compiler cannot count, and its s_waitcnt
  // builtin orders no memory access, so a query load scheduled past the
  // waits below would be taken as pending at the loop head and drained
  // (vmcnt(0)) before every slice's first MFMA.  Redefining the query
  // registers here makes the compiler wait for them once, before the loop.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int c = 0; c < NKC; ++c) asm volatile("" : "+v"(qreg[rt][c]));

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
  if constexpr (SP) {
    // the page ids of the first STAGES tiles; later tiles' ids travel with
    // the cache loads, STAGES tiles ahead of them
    if (n_tiles > 0) {
      for (int x = 0; x < STAGES; ++x) issue_ids(x);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  }
  if (n_tiles > 0) {
#pragma unroll
    for (int u = 0; u < STAGES - 1; ++u) issue(u, u);
  }
  {
    constexpr int ahead = (STAGES - 1) * LW;
    __builtin_amdgcn_s_waitcnt((ahead & 15) | ((ahead >> 4) << 14) | (0x7 << 4) | (0xf << 8));
  }

  // byte offsets (within a wave's V rows) of this lane's transposing reads:
  // lane `col` of group `grp` addresses key row 4 grp + col/4 and the
  // 4-column group (col % 4) of each 16-wide output tile, whose 16-byte chunk
  // sits at its XOR-swizzled position
  uint32_t v_off[NDVT];
  {
    const int kl = grp * 4 + (col >> 2);
    const int sw = chunk_swz(kl, CPR0);
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
                   ? G::K_OFF + col * G::ROW0 + ((ch ^ chunk_swz(col, CPR0)) * 16)
                   : G::R_OFF + col * G::ROWR + (((ch - DN / 8) ^ chunk_swz(col, CPRR)) * 16);
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
      uint32_t sbase = lds_addr(sb);
      // row halves (eight waves, a deeper ring, 256 registers): operand
      // addresses are formed per slice rather than kept for every stage
      if constexpr (RH == 2) asm volatile("" : "+s"(sbase));
      const uint32_t vbase = sbase + ((KIND == GQA) ? G::V_OFF : G::K_OFF);
      uint32_t ka_addr[NKC], va_addr[NDVT];
#pragma unroll
      for (int c = 0; c < NKC; ++c) ka_addr[c] = sbase + k_off[c];
#pragma unroll
      for (int dt = 0; dt < NDVT; ++dt) va_addr[dt] = vbase + v_off[dt];
      slice_reads<NKC, NDVT>(ka_addr, va_addr, kraw, vraw);
    }
    // GTA2: the second group's non-RoPE K chunks and V^T tiles (the RoPE
    // chunks read above serve both groups)
    constexpr int NKB = PAIR ? DN / 32 : 1;
    u32x4_t kraw2[NKB];
    u64_t vraw2[PAIR ? NDVT : 1];
    if constexpr (PAIR) {
      const uint32_t sbase = lds_addr(sb);
      uint32_t ka_addr[NKB], va_addr[NDVT];
#pragma unroll
      for (int c = 0; c < NKB; ++c) ka_addr[c] = sbase + G::K2_OFF + k_off[c];
#pragma unroll
      for (int dt = 0; dt < NDVT; ++dt) va_addr[dt] = sbase + G::K2_OFF + v_off[dt];
      b128_reads<NKB>(ka_addr, kraw2);
      tr_reads<NDVT>(va_addr, vraw2);
    }
    auto kread = [&](int c) { return __builtin_bit_cast(bf16x8, kraw[c]); };
    auto mma = [&](bf16x8 a, int c) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        sa[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[rt][c], sa[rt], 0, 0, 0);
    };
    // the RoPE chunks (c0, c0 + 1) of this lane's key, rotated at its position
    auto rope_keys = [&](bf16x8& ka, bf16x8& kb) {
      if (p.rope_on) {
        if ((t & 15) == 0) {
          // exact angle of this lane's key (first tile of 16)
          const float kpos = (float)(key0 + col);
#pragma unroll
          for (int u2 = 0; u2 < 8; ++u2)
            rope_sincos(kpos, rtab[4 * u2], rtab[4 * u2 + 1], rsn[u2], rcs[u2]);
        } else {
          // one tile further: angle addition with the tile's cos / sin
#pragma unroll
          for (int u2 = 0; u2 < 8; ++u2) {
            const float c1 = rtab[4 * u2 + 2], s1 = rtab[4 * u2 + 3];
            const float sn = rsn[u2], cs = rcs[u2];
            rsn[u2] = fmaf(sn, c1, cs * s1);
            rcs[u2] = fmaf(cs, c1, -(sn * s1));
          }
        }
#pragma unroll
        for (int u2 = 0; u2 < 8; ++u2) {
          const float x = (float)ka[u2], y = (float)kb[u2];
          ka[u2] = (__bf16)(x * rcs[u2] - y * rsn[u2]);
          kb[u2] = (__bf16)(x * rsn[u2] + y * rcs[u2]);
        }
      }
    };
    if constexpr (KIND == GTA) {
      constexpr int c0 = DN / 32;
#pragma unroll
      for (int c = 0; c < c0; ++c) mma(kread(c), c);
      bf16x8 ka = kread(c0), kb = kread(c0 + 1);
      rope_keys(ka, kb);
      mma(ka, c0);
      mma(kb, c0 + 1);
#pragma unroll
      for (int c = c0 + 2; c < NKC; ++c) mma(kread(c), c);
    } else if constexpr (PAIR) {
      // rows of group j score its own non-RoPE chunks, rows of group j + 1
      // the second group's; both add the shared rotated RoPE chunks
      static_assert(DN / 32 + 2 == NKC, "tied non-RoPE chunks, then two RoPE chunks");
      constexpr int c0 = DN / 32;
      f32x4 sbn[RT], sr[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sbn[rt] = sr[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < c0; ++c) {
        mma(kread(c), c);
        const bf16x8 kbb = __builtin_bit_cast(bf16x8, kraw2[c]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          sbn[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbb, qreg[rt][c], sbn[rt], 0, 0, 0);
      }
      bf16x8 ka = kread(c0), kb = kread(c0 + 1);
      rope_keys(ka, kb);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        sr[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qreg[rt][c0], sr[rt], 0, 0, 0);
        sr[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qreg[rt][c0 + 1], sr[rt], 0, 0, 0);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[rt][i] = (row_b[rt] ? sbn[rt][i] : sa[rt][i]) + sr[rt][i];
    } else {
#pragma unroll
      for (int c = 0; c < NKC; ++c) mma(kread(c), c);
    }
    // mask + online softmax; lane holds keys key0 + 4 grp + i of its rows.
    // The running max is only raised (and O, l rescaled) when a row's max
    // grows by more than 2^8: probabilities then stay below 256, harmless in
    // fp32 and bf16, and most slices skip the rescale of the accumulators.
    // keys below L - q_len + 1 are visible to every row of a causal group,
    // so only the slices that reach past that (or past the chunk) mask
    const bool full = key0 + KW <= (p.causal ? min(t_end, L - p.q_len + 1) : t_end);
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
    if constexpr (PAIR) {
      // each row's probabilities meet its own group's values
      const bf16x4 zero4 = {};
      bf16x4 pa[RT], pbb[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        pa[rt] = row_b[rt] ? zero4 : pb[rt];
        pbb[rt] = row_b[rt] ? pb[rt] : zero4;
      }
#pragma unroll
      for (int dt = 0; dt < NDVT; ++dt) {
        const bf16x4 va = __builtin_bit_cast(bf16x4, vraw[dt]);
        const bf16x4 vb = __builtin_bit_cast(bf16x4, vraw2[dt]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pa[rt], acc[rt][dt], 0, 0, 0);
          acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vb, pbb[rt], acc[rt][dt], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < NDVT; ++dt) {
        const bf16x4 va = __builtin_bit_cast(bf16x4, vraw[dt]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[rt], acc[rt][dt], 0, 0, 0);
      }
    }
  };

  // ---- main loop, unrolled by STAGES so every stage is a distinct LDS object
  for (int t = 0; t < n_tiles; t += STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) {
      if (t + u < n_tiles) {
        if constexpr (RH == 1) {
          // every wave has read stage (u-1) of the previous tile before reuse
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
          issue(t + u + STAGES - 1, (u + STAGES - 1) % STAGES);
          // wait until this tile's loads (issued STAGES-1 tiles ago) landed
          constexpr int ahead = (STAGES - 1) * LW;
          __builtin_amdgcn_s_waitcnt((ahead & 15) | ((ahead >> 4) << 14) | (0x7 << 4) | (0xf << 8));
        } else {
          // row halves: this wave's part of tile t + u has landed; after the
          // barrier both parts have, and both halves are done with tile
          // t + u - 1, whose stage then takes tile t + u + STAGES - 1
          constexpr int ahead = (STAGES - 2) * LW;
          __builtin_amdgcn_s_waitcnt((ahead & 15) | ((ahead >> 4) << 14) | (0x7 << 4) | (0xf << 8));
          __syncthreads();
          issue(t + u + STAGES - 1, (u + STAGES - 1) % STAGES);
        }
        // the next item's ticket, drawn as the last tile starts so that the
        // atomic's round trip overlaps this tile's arithmetic
        if (p.queue && t + u == n_tiles - 1 && tid == 0)
          ticket = __hip_atomic_fetch_add(p.queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
      merge_m[half][wave][rt * 16 + col] = m_run[rt];
      merge_l[half][wave][rt * 16 + col] = l_w;
    }
  }
  __syncthreads();
  // columns merged per pass: the largest power of two whose four per-wave
  // 16-row slabs (of each row half) fit one stage buffer
  constexpr int DP0 = G::STAGE_BYTES / (RH * NW * 16 * 4);
  constexpr int DP = DP0 >= D ? D : DP0 >= 128 ? 128 : DP0 >= 64 ? 64 : 32;
  static_assert(D % DP == 0 && DP % (NW * 4) == 0, "merge passes");
  float* obuf = reinterpret_cast<float*>(st0) + half * (NW * 16 * DP);  // [NW][16][DP] fp32
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + col;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, merge_m[half][w][r]);
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    float lt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) lt += merge_l[half][w][r] * exp2f(merge_m[half][w][r] - mu);
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
          } else if (p.fuse_merge) {
            store_partial4(p.o_part + prow * D + dv, o);
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
      } else if (p.fuse_merge) {
        store_partial(p.lse_part + prow, lse_val);
      } else {
        p.lse_part[prow] = lse_val;
      }
    }
  }
  // the last split of this (sequence, group) to finish merges all splits
  if (n_splits > 1 && p.fuse_merge) {
#pragma unroll
    for (int jj = j; jj < j + (PAIR ? 2 : 1); ++jj)
      arrive_and_merge<D>(p, p.counters + ((int64_t)b * (p.h_q / p.g) + jj) * nrb + rblk,
                          &merge_last, b, jj, rblk * 16 * RT * RH,
                          min(16 * RT * RH, p.rows - rblk * 16 * RT * RH),
                          n_splits, slot_base);
  }

  // next item from the queue.  Every processed item draws one ticket, so
  // tickets 0 .. n_items - 1 are drawn in all; the draw of the last one
  // returns the counter to zero for the next call.
  if (!p.queue) break;
  if (tid == 0) {
    if (n_tiles == 0)
      ticket = __hip_atomic_fetch_add(p.queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (ticket == (uint32_t)(p.n_items - 1))
      __hip_atomic_store(p.queue, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    next_item = p.queue_base + (int)ticket;
  }
  __syncthreads();  // the ring and merge buffers are free, next_item is visible
  item = next_item;
  __syncthreads();  // every thread has read next_item before it changes
  }
}

}  // namespace narrow

template <int KIND, int D, int DR, int RT, int S, bool SP = false, int RH = 1>
int launch_narrow_s(Params p, int n_items, int groups, hipStream_t stream) {
  using G = narrow::Geo<KIND, D, DR>;
  if constexpr (S * G::STAGE_BYTES + 4096 > 163840) {
    return launch_narrow_s<KIND, D, DR, RT, S - 1, SP, RH>(p, n_items, groups, stream);
  } else {
    p.n_items = n_items;
    // GTA: the groups of one (sequence, chunk) share an XCD (its L2 serves
    // their common RoPE key rows); GQA groups share nothing and are dealt
    // round-robin like any item, which balances the XCDs
    // GTA2: a unit is a pair of plan items (two groups)
    const int gsz = KIND == GTA ? groups : KIND == GTA2 ? groups / 2 : 1;
    const int units = KIND == GTA2 ? n_items / 2 : n_items;
    const int nrb = (p.rows + 16 * RT * RH - 1) / (16 * RT * RH);  // workgroups per item
    p.row_blocks = gsz;
    p.nrb = nrb;
    int blocks = (units + 8 * gsz - 1) / (8 * gsz) * 8 * gsz * nrb;
    if (p.queue && KIND == GQA && nrb == 1 && p.queue_base > 0 && p.queue_base < n_items) {
      blocks = p.queue_base;  // resident workgroups; the rest come from the queue
    } else {
      p.queue = nullptr;
    }
    hipLaunchKernelGGL((narrow::decode_narrow<KIND, D, DR, RT, S, SP, RH>), dim3(blocks),
                       dim3(narrow::NW * RH * 64), 0, stream, p);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
  }
}

// pages of fewer than 16 tokens (or forced): per-row page ids
bool narrow_sp(const Params& p) {
  return p.page_shift < 4 || attn_internal::env_int("ATTN_FORCE_SP", 0);
}

template <int KIND, int D, int DR, int RT>
int launch_narrow_rt(const Params& p, int n_items, int groups, int stages, hipStream_t stream) {
  // small pages: rings of 2 to 4 stages
  if (narrow_sp(p)) {
    return stages >= 4   ? launch_narrow_s<KIND, D, DR, RT, 4, true>(p, n_items, groups, stream)
           : stages == 3 ? launch_narrow_s<KIND, D, DR, RT, 3, true>(p, n_items, groups, stream)
                         : launch_narrow_s<KIND, D, DR, RT, 2, true>(p, n_items, groups, stream);
  }
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
  // GTA2 is only chosen for groups of at most 8 rows: a pair fills one row tile
  if constexpr (KIND == GTA2) return launch_narrow_rt<KIND, D, DR, 1>(p, n_items, groups, stages, stream);
  const int rt = (p.rows + 15) / 16;
  if (rt <= 1) return launch_narrow_rt<KIND, D, DR, 1>(p, n_items, groups, stages, stream);
  // more than 32 rows on pages of 16 tokens or more: one workgroup of two
  // row halves of two row tiles each, over one ring; else two workgroups of
  // two row tiles (two waves per SIMD either way), unless ATTN_NARROW_RT4=1
  // keeps them in one of four row tiles
  if constexpr (KIND != GTA2) {
    if (rt > 2 && attn_internal::narrow_row_halves(p.page_shift >= 4) && !narrow_sp(p)) {
      switch (stages) {
        case 2: return launch_narrow_s<KIND, D, DR, 2, 2, false, 2>(p, n_items, groups, stream);
        case 3: return launch_narrow_s<KIND, D, DR, 2, 3, false, 2>(p, n_items, groups, stream);
        case 4: return launch_narrow_s<KIND, D, DR, 2, 4, false, 2>(p, n_items, groups, stream);
        case 5: return launch_narrow_s<KIND, D, DR, 2, 5, false, 2>(p, n_items, groups, stream);
        default: return launch_narrow_s<KIND, D, DR, 2, 6, false, 2>(p, n_items, groups, stream);
      }
    }
  }
  if (rt <= 2 || !attn_internal::env_narrow_rt4())
    return launch_narrow_rt<KIND, D, DR, 2>(p, n_items, groups, stages, stream);
  return launch_narrow_rt<KIND, D, DR, 4>(p, n_items, groups, stages, stream);
}

}  // namespace

int run_narrow(int kind, int d, const Params& p, int n_items, int groups, int stages,
               hipStream_t stream) {
  if (kind == GTA) return launch_narrow<GTA, 128, 64>(p, n_items, groups, stages, stream);
  if (kind == GTA2) return launch_narrow<GTA2, 128, 64>(p, n_items, groups, stages, stream);
  return d == 128 ? launch_narrow<GQA, 128, 0>(p, n_items, groups, stages, stream)
                  : launch_narrow<GQA, 64, 0>(p, n_items, groups, stages, stream);
}

}  // namespace attn_dev
