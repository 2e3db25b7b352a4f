// Host-only part of libattn_decode: split planning, workspace sizing,
// descriptor checks and status strings.  Integer work only; no GPU calls,
// so these entry points also run on machines without a GPU.
#include "attn_decode.h"
#include "attn_kernels.h"

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

using attn_internal::kTile;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Estimated cost, in bytes-equivalent, of the whole decode for chunks of
// `ct` tiles: the larger of (total traffic spread over all CUs) and (the
// longest single work item, which streams at only 1/W of a CU's bandwidth
// when W workgroups share the CU), which bounds a greedy schedule's makespan.
struct CostModel {
  const std::vector<int64_t>* tiles;
  int64_t groups, token_bytes, split_bytes, item_bytes, cu, wgs_per_cu;
  double eval(int64_t ct) const {
    int64_t total = 0, longest = 0;
    bool any_split = false;
    for (int64_t t : *tiles) {
      int64_t n = std::max<int64_t>(1, ceil_div(t, ct));
      int64_t kv = t * kTile * token_bytes;
      total += groups * (kv + n * item_bytes + (n > 1 ? n * split_bytes : 0));
      int64_t chunk = std::min<int64_t>(t, ct) * kTile * token_bytes;
      longest = std::max(longest, chunk + item_bytes + (n > 1 ? split_bytes : 0));
      any_split |= n > 1;
    }
    // the merge kernel is a second launch: about 2 microseconds of the
    // whole GPU, i.e. what one CU streams in that time
    const double merge = any_split ? 64.0 * 1024.0 : 0.0;
    return std::max((double)total / (double)cu, (double)longest * (double)wgs_per_cu) + merge;
  }
};

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace or plan buffer too small";
    case ATTN_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int attn_decode_plan_max_items(int batch, int n_groups, int max_seqlen) {
  if (batch <= 0 || n_groups <= 0 || max_seqlen < 0) return ATTN_ERR_INVALID_ARG;
  int64_t per = std::max<int64_t>(1, ceil_div(max_seqlen, kTile));
  int64_t n = (int64_t)batch * n_groups * per;
  if (n > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  return (int)n;
}

int attn_decode_plan(const attn_shape_t* shape, const int32_t* seqlens_host, int cu_count,
                     int chunk_tokens, int32_t* items_host, int32_t* seqinfo_host,
                     int max_items, attn_plan_t* plan) {
  if (!shape || !seqlens_host || !items_host || !seqinfo_host || !plan) return ATTN_ERR_INVALID_ARG;
  const int batch = shape->batch, q_len = shape->q_len, h_q = shape->h_q;
  const int n_groups = shape->groups;
  const int causal = shape->flags & ATTN_CAUSAL;
  if (batch <= 0 || q_len <= 0 || h_q <= 0 || n_groups <= 0 || shape->head_dim <= 0 ||
      shape->d_rope < 0 || shape->page_size <= 0 || cu_count <= 0 || max_items <= 0)
    return ATTN_ERR_INVALID_ARG;
  if (shape->kind != ATTN_KIND_GQA && shape->kind != ATTN_KIND_GTA &&
      shape->kind != ATTN_KIND_LATENT)
    return ATTN_ERR_INVALID_ARG;
  if (h_q % n_groups) return ATTN_ERR_INVALID_ARG;
  if (chunk_tokens < 0 || chunk_tokens % kTile) return ATTN_ERR_INVALID_ARG;
  const attn_internal::KernelChoice kc = attn_internal::choose_kernel(*shape);
  const int64_t token_bytes = kc.token_bytes;
  const int d_v = kc.d_v;

  std::vector<int64_t> tiles(batch);
  int64_t max_tiles = 1;
  for (int b = 0; b < batch; ++b) {
    int64_t L = seqlens_host[b];
    if (L < 0) return ATTN_ERR_INVALID_ARG;
    if (causal && q_len > 1 && L < q_len) return ATTN_ERR_INVALID_ARG;
    tiles[b] = ceil_div(L, kTile);
    max_tiles = std::max(max_tiles, tiles[b]);
  }

  int64_t ct;  // chunk length in tiles
  if (chunk_tokens > 0) {
    ct = chunk_tokens / kTile;
  } else {
    const int64_t rows = (int64_t)(h_q / n_groups) * q_len;
    CostModel m;
    m.tiles = &tiles;
    m.groups = n_groups;
    m.token_bytes = token_bytes;
    // a split writes and the merge re-reads fp32 O and LSE for its rows
    m.split_bytes = 2 * rows * (d_v + 1) * 4;
    // fixed cost of an item: its query rows plus prologue/epilogue latency,
    // taken as the bytes one CU streams in about 1.5 microseconds
    m.item_bytes = rows * (d_v + 64) * 2 + 48 * 1024;
    m.cu = cu_count;
    m.wgs_per_cu = kc.wgs_per_cu;
    ct = max_tiles;
    double best = m.eval(ct);
    // candidate chunk lengths: the shortest chunk giving the longest sequence
    // n splits, for every n (about 2 sqrt(max_tiles) distinct values)
    int64_t prev = max_tiles;
    for (int64_t n = 2; n <= max_tiles; ++n) {
      const int64_t c = ceil_div(max_tiles, n);
      if (c == prev) continue;
      prev = c;
      const double v = m.eval(c);
      if (v < best * 0.999) { best = v; ct = c; }
    }
  }

  // items: full-length chunks first (longest-first), then the shorter tails
  int64_t n_items = 0, slot = 0;
  int max_splits = 1;
  for (int b = 0; b < batch; ++b) {
    int64_t n = std::max<int64_t>(1, ceil_div(tiles[b], ct));
    n_items += n * n_groups;
    max_splits = (int)std::max<int64_t>(max_splits, n);
  }
  if (n_items > max_items) return ATTN_ERR_WORKSPACE;

  const int32_t chunk = (int32_t)(ct * kTile);
  for (int b = 0; b < batch; ++b) {
    int64_t n = std::max<int64_t>(1, ceil_div(tiles[b], ct));
    seqinfo_host[4 * b + 0] = (int32_t)n;
    seqinfo_host[4 * b + 1] = (int32_t)(n > 1 ? slot : -1);
    seqinfo_host[4 * b + 2] = seqlens_host[b];
    seqinfo_host[4 * b + 3] = chunk;
    if (n > 1) slot += n;
  }
  int64_t k = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int b = 0; b < batch; ++b) {
      const int64_t L = seqlens_host[b];
      const int64_t n = seqinfo_host[4 * b + 0];
      for (int64_t s = 0; s < n; ++s) {
        const int64_t t0 = s * chunk;
        const bool full = (t0 + chunk) <= L;
        if ((pass == 0) != full) continue;
        for (int j = 0; j < n_groups; ++j) {
          items_host[4 * k + 0] = b;
          items_host[4 * k + 1] = j;
          items_host[4 * k + 2] = (int32_t)s;
          items_host[4 * k + 3] = (int32_t)t0;
          ++k;
        }
      }
    }
  }
  plan->n_items = (int32_t)n_items;
  plan->batch = batch;
  plan->n_groups = n_groups;
  plan->q_len = q_len;
  plan->max_splits = max_splits;
  plan->n_partial_slots = (int32_t)slot;
  plan->items = nullptr;
  plan->seqinfo = nullptr;
  return ATTN_OK;
}

size_t attn_decode_workspace_size(const attn_plan_t* plan, int h_q, int d_v) {
  if (!plan || h_q <= 0 || d_v <= 0 || plan->n_items <= 0) return 0;
  return attn_internal::flags_offset(plan, h_q, d_v) + attn_internal::flags_bytes(plan, h_q);
}

int attn_paged_kv_check(const attn_paged_kv_t* kv) {
  if (!kv || !kv->page_table || !kv->seqlens) return ATTN_ERR_INVALID_ARG;
  if (kv->batch <= 0 || kv->page_size <= 0 || kv->num_pages <= 0 || kv->max_pages_per_seq <= 0)
    return ATTN_ERR_INVALID_ARG;
  for (int b = 0; b < kv->batch; ++b) {
    const int64_t L = kv->seqlens[b];
    if (L < 0 || L > (int64_t)kv->max_pages_per_seq * kv->page_size) return ATTN_ERR_INVALID_ARG;
    const int64_t used = ceil_div(L, kv->page_size);
    for (int64_t p = 0; p < used; ++p) {
      const int32_t id = kv->page_table[(int64_t)b * kv->max_pages_per_seq + p];
      if (id < 0 || id >= kv->num_pages) return ATTN_ERR_INVALID_ARG;
    }
  }
  return ATTN_OK;
}

}  // extern "C"
