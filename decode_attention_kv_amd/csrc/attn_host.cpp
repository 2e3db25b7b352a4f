// Host-only part of libattn_decode: split planning, workspace sizing,
// descriptor checks and status strings.  Integer work only; no GPU calls,
// so these entry points also run on machines without a GPU.
#include "attn_decode.h"
#include "attn_kernels.h"

#include <algorithm>
#include <functional>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

using attn_internal::kTile;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Items of a plan with chunks of at most `ct` tiles, in launch order: full
// chunks first, then the shorter ones, longest first, so that the
// dispatcher's in-order list scheduling ends with the short ones.  With
// `balanced` a sequence split n = ceil(tiles / ct) ways gets n chunks of
// equal length (the last one shorter by the remainder).  Each entry is
// (sequence, split, tiles); groups are expanded by the caller.
struct Chunk {
  int32_t b, s, tiles;
};
// chunk length (tiles) of a sequence of `t` tiles under a plan of `ct`:
// ct itself, or with balanced splits the same number of chunks made equal
int64_t seq_chunk(int64_t t, int64_t ct, bool balanced) {
  if (!balanced) return ct;
  const int64_t n = std::max<int64_t>(1, ceil_div(t, ct));
  return std::max<int64_t>(1, ceil_div(t, n));
}
void chunks_in_order(const std::vector<int64_t>& tiles, int64_t ct, std::vector<Chunk>* out,
                     bool balanced) {
  out->clear();
  std::vector<Chunk> tails;
  const int batch = (int)tiles.size();
  for (int b = 0; b < batch; ++b) {
    const int64_t n = std::max<int64_t>(1, ceil_div(tiles[b], ct));
    const int64_t cb = seq_chunk(tiles[b], ct, balanced);
    for (int64_t s = 0; s < n; ++s) {
      const int64_t len = std::min<int64_t>(cb, tiles[b] - s * cb);
      if (len <= 0 && s > 0) break;  // (an empty sequence keeps its one item)
      (len == ct ? *out : tails).push_back({b, (int32_t)s, (int32_t)len});
    }
  }
  std::stable_sort(tails.begin(), tails.end(),
                   [](const Chunk& x, const Chunk& y) { return x.tiles > y.tiles; });
  out->insert(out->end(), tails.begin(), tails.end());
}

// Estimated decode time, in tiles at one workgroup's fair share, of the
// plan with chunks of `ct` tiles: every XCD runs its workgroups (block i
// goes to XCD i % 8) in launch order on `slots` slots; active workgroups
// share the XCD's bandwidth, each at most `rmax` times its share at full
// occupancy (processor sharing, simulated exactly with a virtual clock).
double simulate(const std::vector<Chunk>& chunks, int groups, const attn_internal::KernelChoice& kc,
                int slots) {
  // Launch order of the kernels: item units (the groups of one chunk when
  // `same_xcd_groups`, else single items with their row blocks) sit 8
  // blocks apart, so XCD x receives units x, x + 8, x + 16, ... in order,
  // each as `per_unit` consecutive workgroups.
  const int64_t n_items = (int64_t)chunks.size() * groups;
  const bool by_group = kc.same_xcd_groups;
  const int64_t units = by_group ? (int64_t)chunks.size() : n_items;
  const int per_unit = (by_group ? groups / std::max(1, kc.pair) : 1) * std::max(1, kc.row_blocks);
  double makespan = 0.0;
  std::vector<double> heap;
  heap.reserve(slots);
  for (int x = 0; x < 8; ++x) {
    heap.clear();
    double now = 0.0, vclock = 0.0;  // time, service each active workgroup got
    auto retire_one = [&]() {
      const double rate = std::min(kc.rmax, (double)slots / heap.size());
      std::pop_heap(heap.begin(), heap.end(), std::greater<double>());
      const double done = heap.back();
      heap.pop_back();
      now += (done - vclock) / rate;
      vclock = done;
    };
    for (int64_t u = x; u < units; u += 8) {
      const double work =
          chunks[by_group ? u : u / groups].tiles + kc.fixed_tiles;
      for (int k = 0; k < per_unit; ++k) {
        if ((int)heap.size() == slots) retire_one();
        heap.push_back(vclock + work);
        std::push_heap(heap.begin(), heap.end(), std::greater<double>());
      }
    }
    while (!heap.empty()) retire_one();
    makespan = std::max(makespan, now);
  }
  return makespan;
}

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
  std::vector<Chunk> chunks;
  // automatic plans split each sequence into chunks of equal length (one
  // long chunk beside a short tail would set the kernel's end); a forced
  // chunk length is used as given
  const bool balanced = chunk_tokens == 0;
  chunks.reserve(1024);
  if (chunk_tokens > 0) {
    ct = chunk_tokens / kTile;
  } else {
    // Pick the chunk length minimising simulated decode time plus the merge
    // of split partials.  Times in microseconds: a tile at a workgroup's
    // fair share of about 6 TB/s; the merge launch costs about 4 us, plus
    // about 0.55 us per split of the longest sequence, plus the partials'
    // write and re-read at about 5 TB/s.
    const int slots = std::max(1, cu_count / 8) * kc.wgs_per_cu;  // per XCD
    const double tile_us =
        (double)kTile * token_bytes / (6.0e6 / ((double)cu_count * kc.wgs_per_cu));
    const int64_t rows = (int64_t)(h_q / n_groups) * q_len;
    // cost of splitting the longest sequence n ways (microseconds)
    auto cost = [&](int n, int64_t* c_out) -> double {
      if (n < 1) return -1.0;
      const int64_t c = ceil_div(max_tiles, n);
      *c_out = c;
      if (c < std::min<int64_t>(4, max_tiles)) return -1.0;  // chunks of >= 256 keys
      chunks_in_order(tiles, c, &chunks, balanced);
      const int64_t wgs = (int64_t)chunks.size() * n_groups;
      if (wgs > max_items) return -1.0;
      if (n > 1 && wgs > 6 * 8 * (int64_t)slots) return -1.0;  // far finer than the GPU
      double t = simulate(chunks, n_groups, kc, slots) * tile_us;
      int64_t slots_used = 0, splits = 1;
      for (int b = 0; b < batch; ++b) {
        const int64_t nb = std::max<int64_t>(1, ceil_div(tiles[b], c));
        if (nb > 1) slots_used += nb;
        splits = std::max(splits, nb);
      }
      if (slots_used > 0)
        t += 4.0 + 0.55 * splits + 2.0 * slots_used * n_groups * rows * (d_v + 1) * 4 / 5.0e6;
      return t;
    };
    // coarse pass over powers of two, then the neighbours of the best
    double best = 0.0;
    int best_n = 1;
    ct = max_tiles;
    auto consider = [&](int n) {
      int64_t c;
      const double t = cost(n, &c);
      if (t >= 0.0 && (best_n == 0 || t < best * 0.995)) {
        best = t;
        best_n = n;
        ct = c;
      }
    };
    best_n = 0;
    for (int n = 1; n <= 64; n *= 2) {
      consider(n);
      if (best_n > 0 && n >= 4 * best_n) break;  // two steps past the best
    }
    const int n0 = best_n;
    if (n0 > 1) consider(n0 * 3 / 4);
    if (n0 > 0) consider(n0 * 3 / 2);
    if (best_n == 0) ct = max_tiles;
  }
  chunks_in_order(tiles, ct, &chunks, balanced);

  // items in launch order, groups of one chunk consecutive
  const int64_t n_items = (int64_t)chunks.size() * n_groups;
  int64_t slot = 0;
  int max_splits = 1;
  for (int b = 0; b < batch; ++b)
    max_splits = (int)std::max<int64_t>(max_splits, std::max<int64_t>(1, ceil_div(tiles[b], ct)));
  if (n_items > max_items) return ATTN_ERR_WORKSPACE;

  const int32_t chunk = (int32_t)(ct * kTile);
  for (int b = 0; b < batch; ++b) {
    int64_t n = std::max<int64_t>(1, ceil_div(tiles[b], ct));
    seqinfo_host[4 * b + 0] = (int32_t)n;
    seqinfo_host[4 * b + 1] = (int32_t)(n > 1 ? slot : -1);
    seqinfo_host[4 * b + 2] = seqlens_host[b];
    seqinfo_host[4 * b + 3] = (int32_t)(seq_chunk(tiles[b], ct, balanced) * kTile);
    if (n > 1) slot += n;
  }
  int64_t k = 0;
  for (const Chunk& c : chunks) {
    for (int j = 0; j < n_groups; ++j) {
      items_host[4 * k + 0] = c.b;
      items_host[4 * k + 1] = j;
      items_host[4 * k + 2] = c.s;
      items_host[4 * k + 3] = (int32_t)((int64_t)c.s * seq_chunk(tiles[c.b], ct, balanced) * kTile);
      ++k;
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
  plan->counters = nullptr;
  plan->queue = nullptr;
  plan->items_host = items_host;
  plan->seqinfo_host = seqinfo_host;
  // launch-argument form: three int32 per sequence (the split count and
  // the chunk length in tiles share one) and one per chunk, or half of one
  // (sequence in 11 bits, split in 5) for batches of at most 2048 sequences
  // split at most 32 ways
  const bool half = batch <= 2048 && max_splits <= 32;
  const int64_t chunk_words =
      half ? ((int64_t)chunks.size() + 1) / 2 : (int64_t)chunks.size();
  plan->inline_ok = (3 * (int64_t)batch + chunk_words <= ATTN_PLAN_INLINE_MAX &&
                     ct < 65536 &&
                     batch < 65536 && max_splits < 65536)
                        ? 1
                        : 0;
  return ATTN_OK;
}

size_t attn_decode_counter_count(const attn_plan_t* plan, int h_q) {
  if (!plan || h_q <= 0 || plan->batch <= 0 || plan->n_groups <= 0 || plan->q_len <= 0 ||
      h_q % plan->n_groups)
    return 0;
  return attn_internal::counter_count(plan, h_q);
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
