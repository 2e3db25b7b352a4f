// Internal: which decode kernel runs for a problem shape, and the facts the
// host planner needs about it.  Shared by the planner (attn_host.cpp) and the
// launchers (attn_decode.hip) so both always agree.
#ifndef ATTN_KERNELS_H
#define ATTN_KERNELS_H

#include <cstdint>
#include <cstdlib>

#include "attn_decode.h"

namespace attn_internal {

constexpr int kTile = 64;          // keys per tile; chunks are multiples of it

// Latent streaming kernel geometry: the waves of a workgroup split each
// tile's keys KQ ways (2 KQ waves, two row halves), and each wave holds RT
// tiles of 16 query rows, so a workgroup covers 32 RT rows of a group.
#ifndef WIDE_KQ512
#define WIDE_KQ512 2
#endif
#ifndef WIDE_KQ256
#define WIDE_KQ256 4
#endif
constexpr int wide_kq(int d_c) { return d_c >= 512 ? WIDE_KQ512 : WIDE_KQ256; }
constexpr int wide_rt(int d_c, int rows) {
  return (rows <= 32 || (d_c >= 512 && WIDE_KQ512 > 2)) ? 1 : 2;
}
inline int env_int(const char* name, int dflt);
// 256-wide latents on pages of at least 64 tokens with more than 64 rows
// per group (multi-token and speculative decode): four row tiles per wave
// and a two-way key split, 128 rows per workgroup of four waves (one per
// SIMD), which halves the LDS operand bytes per row against two row tiles;
// ATTN_WIDE_RT4=0 keeps 64-row workgroups
inline bool wide_rows128(int d_c, int rows, int page_size) {
  static const bool on = env_int("ATTN_WIDE_RT4", 1) != 0;
  return on && d_c == 256 && rows > 64 && page_size >= 64;
}
constexpr int kNarrowWaves = 4;    // waves per workgroup of the streaming kernel
constexpr int kNarrowStageTarget = 65536;  // LDS bytes of the streaming ring

struct KernelChoice {
  bool narrow;         // streaming kernel (GQA/GTA) vs general kernel
  int wgs_per_cu;      // workgroups one CU keeps resident
  int stages;          // streaming ring depth (narrow only)
  int64_t token_bytes; // cache bytes one work item reads per token
  int rows;            // query rows per group: (h_q / groups) * q_len
  int d_v;             // output width per head
  // Dispatch model used by the planner (fitted to measured chunk sweeps on
  // MI355X): workgroups are dealt to the 8 XCDs by block index; the groups
  // of one (sequence, chunk) go to one XCD when `same_xcd_groups`, and the
  // `row_blocks` workgroups of one item always do.  Active workgroups of an
  // XCD share its bandwidth; one alone runs at most `rmax` times its share
  // at full occupancy; every workgroup costs `fixed_tiles` extra tiles.
  bool same_xcd_groups;
  int row_blocks;
  int pair;            // plan items per workgroup: 2 when GTA groups go in pairs

  double rmax;
  double fixed_tiles;
};

// Bytes of one 64-key stage of the streaming kernel (four waves x 16 keys).
inline int narrow_stage_bytes(int kind, int head_dim, int d_rope) {
  const int per_key = (kind == ATTN_KIND_GQA) ? 2 * head_dim * 2 : (head_dim + d_rope) * 2;
  return kNarrowWaves * 16 * per_key;
}

// Environment overrides (read once): ATTN_NARROW_STAGES sets the ring depth,
// ATTN_FORCE_GENERAL=1 routes every call to the general kernel.
inline int env_int(const char* name, int dflt) {
  const char* e = std::getenv(name);
  return e ? std::atoi(e) : dflt;
}
inline int env_stages() {
  static const int v = env_int("ATTN_NARROW_STAGES", 0);
  return v;
}
// ATTN_GTA_PAIR=0 keeps every GTA group in a workgroup of its own
inline bool env_gta_pair() {
  static const bool v = env_int("ATTN_GTA_PAIR", 1) != 0;
  return v;
}
// ATTN_NARROW_RT4=1: groups of 33-64 rows in one workgroup of four row
// tiles per wave (one wave per SIMD) instead of two 32-row workgroups
inline bool env_narrow_rt4() {
  static const bool v = env_int("ATTN_NARROW_RT4", 0) != 0;
  return v;
}
// Groups of 33-64 rows on pages of 16 tokens or more: one workgroup of two
// row halves sharing one ring (ATTN_NARROW_HALVES=0: two 32-row workgroups)
inline bool narrow_row_halves(bool whole_slices) {
  static const bool v = env_int("ATTN_NARROW_HALVES", 1) != 0;
  return v && whole_slices && !env_narrow_rt4();
}
inline bool env_force_general() {
  static const bool v = env_int("ATTN_FORCE_GENERAL", 0) != 0;
  return v;
}

inline int narrow_stages(int kind, int head_dim, int d_rope) {
  int s = kNarrowStageTarget / narrow_stage_bytes(kind, head_dim, d_rope);
  if (env_stages() > 0) s = env_stages();
  return s < 2 ? 2 : s > 6 ? 6 : s;
}

inline KernelChoice choose_kernel(const attn_shape_t& sh) {
  KernelChoice k{};
  k.pair = 1;
  k.rows = (sh.groups > 0 ? sh.h_q / sh.groups : 0) * sh.q_len;
  k.d_v = sh.head_dim;
  const int elem = sh.dtype == ATTN_BF16 ? 2 : 4;
  k.token_bytes = (sh.kind == ATTN_KIND_GQA) ? 2LL * sh.head_dim * elem
                                             : (int64_t)(sh.head_dim + sh.d_rope) * elem;
  // any power-of-two page size: whole pages per 16-key slice (>= 16) or per
  // 64-key tile (>= 64) share one page id, smaller pages take one per row
  bool narrow = sh.dtype == ATTN_BF16 && k.rows <= 64 &&
                ((sh.kind == ATTN_KIND_GQA && (sh.head_dim == 64 || sh.head_dim == 128)) ||
                 (sh.kind == ATTN_KIND_GTA && sh.head_dim == 128 && sh.d_rope == 64));
  // latent heads: the wide streaming kernel (reported through `narrow` too:
  // "streaming" rather than the general kernel)
  const bool wide = sh.dtype == ATTN_BF16 && sh.kind == ATTN_KIND_LATENT && sh.d_rope == 64 &&
                    (sh.head_dim == 512 || sh.head_dim == 256);
  if (env_force_general()) narrow = false;
  k.narrow = narrow || (wide && !env_force_general());
  k.same_xcd_groups = false;
  k.row_blocks = 1;
  if (k.narrow && sh.kind == ATTN_KIND_LATENT) {
    k.stages = sh.head_dim >= 512 ? 2 : 3;
    k.wgs_per_cu = 1;
    const int wg_rows =
        wide_rows128(sh.head_dim, k.rows, sh.page_size) ? 128 : 32 * wide_rt(sh.head_dim, k.rows);
    k.row_blocks = (k.rows + wg_rows - 1) / wg_rows;
    k.same_xcd_groups = true;  // groups share RoPE rows, row blocks latent rows
    // a latent workgroup streams at its own pace: timelines show the same
    // per-workgroup rate with 182 or 256 of them active
    k.rmax = 1.0;
    k.fixed_tiles = 8.0;
    return k;
  }
  if (narrow) {
    k.stages = narrow_stages(sh.kind, sh.head_dim, sh.d_rope);
    if (sh.page_size < 16) k.stages = k.stages >= 4 ? 4 : 2;  // small-page rings
    const int lds = k.stages * narrow_stage_bytes(sh.kind, sh.head_dim, sh.d_rope) + 2048;
    int w = 163840 / lds;
    k.wgs_per_cu = w < 1 ? 1 : w > 2 ? 2 : w;
    // more than 32 rows on pages of 16 tokens or more: one workgroup of two
    // row halves that share one ring, as deep as the LDS holds; else two
    // workgroups of 32 rows on one XCD (the second reads the item's rows
    // from its L2), each as a group of 32 rows
    if (k.rows > 32 && narrow_row_halves(sh.page_size >= 16)) {
      k.wgs_per_cu = 1;
      if (env_stages() == 0) {
        const int s = (163840 - 4096) / narrow_stage_bytes(sh.kind, sh.head_dim, sh.d_rope);
        k.stages = s < 2 ? 2 : s > 6 ? 6 : s;
      }
    } else if (k.rows > 32 && !env_narrow_rt4()) {
      k.row_blocks = (k.rows + 31) / 32;
    }
    // with ATTN_NARROW_RT4=1, four row tiles per wave: one wave per SIMD,
    // and on pages of 16 tokens or more a shallower ring, which frees
    // registers for the row tiles (GTA: 2 stages, measured +6 % over 5 at
    // q_len 8; GQA with 128-wide heads: 3, +1.5 % over 4)
    if (k.rows > 32 && env_narrow_rt4()) {
      k.wgs_per_cu = 1;
      if (sh.page_size >= 16 && env_stages() == 0) {
        if (sh.kind == ATTN_KIND_GTA) k.stages = 2;
        else if (sh.head_dim == 128 && k.stages > 3) k.stages = 3;
      }
    }
    // GTA groups read the same RoPE key rows: keep them on one XCD's L2
    k.same_xcd_groups = sh.kind == ATTN_KIND_GTA;
    // GTA with an even number of groups of at most 8 rows: one workgroup
    // streams two groups, loading and rotating their common RoPE key rows
    // once (40 KB stages, a ring of 3, one workgroup per CU; measured on GTA
    // 8K against one group per workgroup: +11 % at page 1, +2.5-6 % at
    // pages 2-64)
    if (sh.kind == ATTN_KIND_GTA && sh.groups % 2 == 0 && k.rows <= 8 && env_gta_pair()) {
      k.pair = 2;
      k.stages = 3;
      k.wgs_per_cu = 1;
    }
    k.rmax = sh.kind == ATTN_KIND_GTA ? 1.5 : 3.0;
    k.fixed_tiles = sh.kind == ATTN_KIND_GTA ? 3.0 : 2.0;
  } else {
    k.stages = 1;
    k.wgs_per_cu = 1;
    // general kernel: 64 rows per workgroup for 512-wide latents, else 128
    const int rows_per_wg = (sh.kind == ATTN_KIND_LATENT && sh.head_dim >= 512) ? 64 : 128;
    k.row_blocks = (k.rows + rows_per_wg - 1) / rows_per_wg;
    k.rmax = 1.5;
    k.fixed_tiles = 2.0;
  }
  return k;
}

// Workspace layout: fp32 O_part [slots][q_len][h_q][d_v] (256-byte padded),
// fp32 LSE_part [slots][q_len][h_q] (256-byte padded), then one int32 flag
// per workgroup of the latent streaming kernel (its grid: the (sequence,
// chunk) units padded to a multiple of 8, times groups, times at most
// ceil(rows / 32) row blocks).
inline size_t flags_offset(const attn_plan_t* plan, int h_q, int d_v) {
  const size_t rows = (size_t)plan->n_partial_slots * plan->q_len * h_q;
  return (rows * d_v * 4 + 255) / 256 * 256 + (rows * 4 + 255) / 256 * 256;
}
// An upper bound of the row blocks of any streaming kernel: blocks of at
// least 32 rows (the plan does not record the latent width).
inline int64_t row_blocks_of(const attn_plan_t* plan, int h_q) {
  const int64_t rows = (int64_t)(plan->n_groups > 0 ? h_q / plan->n_groups : 0) * plan->q_len;
  return (rows + 31) / 32 > 0 ? (rows + 31) / 32 : 1;
}
inline size_t flags_bytes(const attn_plan_t* plan, int h_q) {
  // grid of the latent streaming kernel: (sequence, chunk) units padded to
  // a multiple of 8, times groups, times row blocks
  const int64_t g = plan->n_groups > 0 ? plan->n_groups : 1;
  const int64_t units = (plan->n_items + g - 1) / g;
  const int64_t blocks = (units + 7) / 8 * 8 * g * row_blocks_of(plan, h_q);
  return ((size_t)blocks * 4 + 255) / 256 * 256;
}
// Merge arrival counters (plan->counters): one per (sequence, group, block
// of 32 rows), of which the kernels use (b * groups + j) * row_blocks + block
// for their own row_blocks (blocks of 32 or 64 rows).
inline size_t counter_count(const attn_plan_t* plan, int h_q) {
  return (size_t)plan->batch * plan->n_groups * row_blocks_of(plan, h_q);
}

}  // namespace attn_internal

#endif  // ATTN_KERNELS_H
