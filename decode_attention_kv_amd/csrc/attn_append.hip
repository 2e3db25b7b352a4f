// Paged KV append: the cache write that precedes each decode call.  The new
// tokens of a step (q_len per sequence) take positions L_b - q_len ..
// L_b - 1, L_b being the sequence length that already counts them, the
// same positions the decode kernels give the query rows; each row goes to
// physical page page_table[b][pos / P], slot pos % P, through the
// descriptor's strides.  GQA writes key and value rows, GTA the tied state
// and its raw RoPE key (the decode rotates it), MLA / GLA the latent rows and
// the RoPE key rotated here at its position ("Hardware-Efficient Attention
// for Fast Decoding", review page: Core claim, and the Circularity Check's
// free parameters on the separate partial-RoPE key head).
#include "attn_device.h"

namespace attn_dev {
namespace {

struct AppendParams {
  char* pool0;
  char* pool1;
  char* rope;
  const char* new0;
  const char* new1;
  const char* new_rope;
  const int32_t* page_table;
  const int32_t* seqlens;
  int64_t page_stride, token_stride, head_stride, rpage_stride, rtoken_stride;
  int32_t q_len, heads, width, d_rope, max_pages, num_pages, page_shift, rope_on;
  float rope_hi[kMaxRope / 2];
  float rope_lo[kMaxRope / 2];
};

// one workgroup per (sequence, new token); 16-byte copies of its rows
template <typename T>
__global__ __launch_bounds__(256) void append_kernel(AppendParams a) {
  const int bt = blockIdx.x;
  const int b = bt / a.q_len, t = bt - b * a.q_len;
  const int pos = a.seqlens[b] - a.q_len + t;
  // a position before the cache start, past the sequence's page-table row,
  // or on a page id outside the pools is skipped: nothing is written
  if (pos < 0 || (pos >> a.page_shift) >= a.max_pages) return;
  const int64_t page = a.page_table[(int64_t)b * a.max_pages + (pos >> a.page_shift)];
  if (page < 0 || page >= a.num_pages) return;
  const int64_t slot = pos & ((1 << a.page_shift) - 1);
  const int upr = a.width * (int)sizeof(T) / 16;  // 16-byte units per head row
  for (int u = threadIdx.x; u < a.heads * upr; u += blockDim.x) {
    const int h = u / upr, c = u - h * upr;
    const int64_t dst = (page * a.page_stride + slot * a.token_stride + h * a.head_stride) *
                            (int64_t)sizeof(T) + c * 16;
    const int64_t src = ((int64_t)bt * a.heads + h) * a.width * (int64_t)sizeof(T) + c * 16;
    *reinterpret_cast<uint4*>(a.pool0 + dst) = *reinterpret_cast<const uint4*>(a.new0 + src);
    if (a.new1)
      *reinterpret_cast<uint4*>(a.pool1 + dst) = *reinterpret_cast<const uint4*>(a.new1 + src);
  }
  if (a.new_rope) {
    const int half = a.d_rope / 2;
    T* dst = reinterpret_cast<T*>(a.rope + (page * a.rpage_stride + slot * a.rtoken_stride) *
                                               (int64_t)sizeof(T));
    const T* src = reinterpret_cast<const T*>(a.new_rope) + (int64_t)bt * a.d_rope;
    for (int k = threadIdx.x; k < half; k += blockDim.x) {
      float x = (float)src[k], y = (float)src[k + half];
      if (a.rope_on) {
        // rotate-half pair (k, k + d_r / 2) by pos * theta^(-2k / d_r)
        float s, c;
        rope_sincos((float)pos, a.rope_hi[k], a.rope_lo[k], s, c);
        const float xr = x * c - y * s, yr = x * s + y * c;
        x = xr;
        y = yr;
      }
      dst[k] = (T)x;
      dst[k + half] = (T)y;
    }
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace
}  // namespace attn_dev

using namespace attn_dev;

extern "C" int attn_kv_append(const attn_paged_kv_t* kv, int q_len, int heads, int width,
                              const void* new0, const void* new1, int d_rope, const void* new_rope,
                              float rope_theta, hipStream_t stream) {
  if (!kv || !kv->pool0 || !kv->page_table || !kv->seqlens || !new0) return ATTN_ERR_INVALID_ARG;
  if (kv->batch <= 0 || q_len < 1 || heads < 1 || width < 1 || kv->max_pages_per_seq <= 0 ||
      kv->num_pages <= 0)
    return ATTN_ERR_INVALID_ARG;
  if (kv->dtype != ATTN_BF16 && kv->dtype != ATTN_FP32) return ATTN_ERR_INVALID_ARG;
  const int P = kv->page_size;
  if (P <= 0 || (P & (P - 1))) return ATTN_ERR_INVALID_ARG;
  const int es = kv->dtype == ATTN_BF16 ? 2 : 4;
  if ((width * es) % 16 || !aligned16(kv->pool0) || !aligned16(new0)) return ATTN_ERR_INVALID_ARG;
  if (new1 && (!kv->pool1 || !aligned16(kv->pool1) || !aligned16(new1))) return ATTN_ERR_INVALID_ARG;
  if ((kv->page_stride * es) % 16 || (kv->token_stride * es) % 16 || (kv->head_stride * es) % 16 ||
      kv->page_stride < 0 || kv->token_stride < 0 || kv->head_stride < 0)
    return ATTN_ERR_INVALID_ARG;
  if (new_rope) {
    if (!kv->rope_pool || d_rope <= 0 || d_rope % 2 || d_rope > kMaxRope) return ATTN_ERR_INVALID_ARG;
    if (kv->rope_page_stride < 0 || kv->rope_token_stride < 0) return ATTN_ERR_INVALID_ARG;
  }
  if ((int64_t)kv->batch * q_len > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  AppendParams a;
  std::memset(&a, 0, sizeof(a));
  a.pool0 = static_cast<char*>(const_cast<void*>(kv->pool0));
  a.pool1 = static_cast<char*>(const_cast<void*>(kv->pool1));
  a.rope = static_cast<char*>(const_cast<void*>(kv->rope_pool));
  a.new0 = static_cast<const char*>(new0);
  a.new1 = static_cast<const char*>(new1);
  a.new_rope = static_cast<const char*>(new_rope);
  a.page_table = kv->page_table;
  a.seqlens = kv->seqlens;
  a.page_stride = kv->page_stride;
  a.token_stride = kv->token_stride;
  a.head_stride = kv->head_stride;
  a.rpage_stride = kv->rope_page_stride;
  a.rtoken_stride = kv->rope_token_stride;
  a.q_len = q_len;
  a.heads = heads;
  a.width = width;
  a.d_rope = new_rope ? d_rope : 0;
  a.max_pages = kv->max_pages_per_seq;
  a.num_pages = kv->num_pages;
  int shift = 0;
  while ((1 << shift) < P) ++shift;
  a.page_shift = shift;
  if (new_rope && rope_theta > 0.f) {
    // revolutions per position, split into two floats (as in the decode)
    for (int k = 0; k < d_rope / 2; ++k) {
      const double f = std::pow((double)rope_theta, -2.0 * k / d_rope) / (2.0 * M_PI);
      a.rope_hi[k] = (float)f;
      a.rope_lo[k] = (float)(f - (double)a.rope_hi[k]);
    }
    a.rope_on = 1;
  }
  const dim3 grid(kv->batch * q_len);
  if (kv->dtype == ATTN_BF16)
    hipLaunchKernelGGL(append_kernel<__bf16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<float>, grid, dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}
