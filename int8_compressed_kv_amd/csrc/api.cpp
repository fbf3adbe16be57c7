// C ABI of the attention library: host-side argument checks, then dispatch to the
// gfx950 kernels.  Nothing is enqueued when a check fails; the reason is kept in a
// thread-local string (fa_last_error).  No exception crosses the ABI.
#include "../../include/fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "kernel_args.hpp"

namespace {

thread_local std::string g_last_error;
thread_local const char* g_last_kernel = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_head_dim(int32_t d) {
  if (d <= 0) return fail(FA_ERR_INVALID, "head_dim must be positive (got %d)", d);
  if (d % 32 != 0 || d > FA_MAX_HEAD_DIM)
    return fail(FA_ERR_UNSUPPORTED, "head_dim must be a multiple of 32 in [32, %d] (got %d)",
                FA_MAX_HEAD_DIM, d);
  return FA_OK;
}

// Splits the op list by scope: output-tile ops into *out, K-tile (score) ops into *sops, or an
// error when sops is null (a call that forms no scores).
int fill_epilogue(const fa_epilogue_op* epi, int32_t n_epi, fa::EpiArgs* out, fa::EpiArgs* sops) {
  std::memset(out, 0, sizeof(*out));
  if (sops) std::memset(sops, 0, sizeof(*sops));
  if (n_epi < 0) return fail(FA_ERR_INVALID, "n_epi must be >= 0 (got %d)", n_epi);
  if (n_epi > FA_MAX_EPILOGUE)
    return fail(FA_ERR_UNSUPPORTED, "at most %d epilogue ops are supported (got %d)", FA_MAX_EPILOGUE, n_epi);
  if (n_epi > 0 && epi == nullptr) return fail(FA_ERR_INVALID, "epi is NULL but n_epi = %d", n_epi);
  for (int i = 0; i < n_epi; ++i) {
    const int k = epi[i].kind;
    if (k != FA_EPI_MUL && k != FA_EPI_ADD && k != FA_EPI_BIAS && k != FA_EPI_RELU)
      return fail(FA_ERR_INVALID, "epilogue op %d has unknown kind %d", i, k);
    if (k == FA_EPI_BIAS && (!epi[i].vec || (reinterpret_cast<uintptr_t>(epi[i].vec) & 3u)))
      return fail(FA_ERR_INVALID, "epilogue op %d (bias) needs a 4-byte aligned device vector", i);
    if (k != FA_EPI_BIAS && epi[i].vec)
      return fail(FA_ERR_INVALID, "epilogue op %d: vec must be NULL unless the kind is FA_EPI_BIAS", i);
    const int sc = epi[i].scope;
    if (sc != FA_SCOPE_OUTPUT_TILE && sc != FA_SCOPE_K_TILE && sc != FA_SCOPE_KERNEL)
      return fail(FA_ERR_INVALID, "epilogue op %d has unknown scope %d", i, sc);
    if (sc == FA_SCOPE_KERNEL)
      return fail(FA_ERR_UNSUPPORTED, "epilogue op %d: the kernel scope is not supported", i);
    if (sc == FA_SCOPE_K_TILE && !sops)
      return fail(FA_ERR_UNSUPPORTED, "epilogue op %d: K-tile ops need a call that forms scores", i);
    fa::EpiArgs* dst = sc == FA_SCOPE_K_TILE ? sops : out;
    dst->kind[dst->n] = k;
    dst->value[dst->n] = epi[i].value;
    dst->vec[dst->n] = epi[i].vec;
    ++dst->n;
  }
  return FA_OK;
}

float resolve_scale(float s, int32_t d) {
  return s > 0.f ? s : 1.0f / std::sqrt((float)d);
}

constexpr int32_t kMaxSplits = 4096;
constexpr int32_t kDecodeTile = 32;   // keys per decode tile
constexpr int32_t kTqAttnTile = 64;   // keys per TurboQuant attention tile

// The codebook c[0 .. 2^bits) as three signed 7-bit digits of c 2^-E (|c| 2^-E < 1/2):
// c ~ 2^E (d0 / 2^7 + d1 / 2^14 + d2 / 2^21), each digit the nearest integer to what remains;
// byte k of tab[t] holds digit t of entry k.  Returns E.
int codebook_digits(const float* cb, int32_t bits, uint32_t (*tab)[4]) {
  const int n = 1 << bits;
  double mx = 0.0;
  for (int k = 0; k < n; ++k) mx = std::fmax(mx, std::fabs((double)cb[k]));
  int E = 0;
  if (mx > 0.0) {
    (void)std::frexp(mx, &E);
    E += 1;
  }
  for (int t = 0; t < 3; ++t)
    for (int w = 0; w < 4; ++w) tab[t][w] = 0u;
  for (int k = 0; k < n; ++k) {
    double x = std::ldexp((double)cb[k], -E) * 128.0;
    for (int t = 0; t < 3; ++t) {
      const double dd = std::nearbyint(x);
      x = (x - dd) * 128.0;
      tab[t][k / 4] |= ((uint32_t)(int32_t)dd & 0xffu) << (8 * (k % 4));
    }
  }
  return E;
}

}  // namespace

extern "C" {

int32_t fa_version(void) { return 10100; }

const char* fa_last_error(void) { return g_last_error.c_str(); }

const char* fa_last_kernel(void) { return g_last_kernel; }

int fa_compress_kv(const void* x, int32_t x_dtype, int64_t n_tokens, int32_t head_dim, int8_t* q_out,
                   float* scale_out, void* stream) {
  g_last_error.clear();
  if (int r = check_head_dim(head_dim)) return r;
  if (x_dtype != FA_F32 && x_dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "compress_kv input must be FA_F32 or FA_BF16 (got %d)", x_dtype);
  if (n_tokens < 0) return fail(FA_ERR_INVALID, "n_tokens must be >= 0");
  if (n_tokens == 0) return FA_OK;
  if (!x || !q_out || !scale_out) return fail(FA_ERR_INVALID, "null pointer argument");
  if (!aligned16(x) || !aligned16(q_out) || (reinterpret_cast<uintptr_t>(scale_out) & 3u))
    return fail(FA_ERR_INVALID, "x and q_out must be 16-byte aligned, scale_out 4-byte aligned");
  const char* name = "";
  hipError_t e = fa::launch_compress(x, x_dtype, n_tokens, head_dim, q_out, scale_out,
                                     static_cast<hipStream_t>(stream), &name);
  if (e != hipSuccess) return hip_fail(e, "compress_kv launch");
  g_last_kernel = name;
  return FA_OK;
}

int fa_append_kv(const void* k_new, const void* v_new, int32_t x_dtype, int32_t bh_kv, int32_t n_new,
                 int32_t head_dim, const int32_t* pos, int32_t capacity, int8_t* k_cache, int8_t* v_cache,
                 float* k_scale, float* v_scale, void* stream) {
  return fa_append_kv_rope(k_new, v_new, x_dtype, bh_kv, n_new, head_dim, pos, capacity, nullptr, nullptr, k_cache,
                           v_cache, k_scale, v_scale, stream);
}

int fa_append_kv_rope(const void* k_new, const void* v_new, int32_t x_dtype, int32_t bh_kv, int32_t n_new,
                      int32_t head_dim, const int32_t* pos, int32_t capacity, const float* rope_cos,
                      const float* rope_sin, int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale,
                      void* stream) {
  g_last_error.clear();
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(FA_ERR_INVALID, "give both rope_cos and rope_sin, or neither");
  if (rope_cos && ((reinterpret_cast<uintptr_t>(rope_cos) & 15u) || (reinterpret_cast<uintptr_t>(rope_sin) & 15u)))
    return fail(FA_ERR_INVALID, "rope_cos and rope_sin must be 16-byte aligned");
  if (int r = check_head_dim(head_dim)) return r;
  if (x_dtype != FA_F32 && x_dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "append_kv input must be FA_F32 or FA_BF16 (got %d)", x_dtype);
  if (bh_kv <= 0) return fail(FA_ERR_INVALID, "bh_kv must be positive (got %d)", bh_kv);
  if (n_new < 0) return fail(FA_ERR_INVALID, "n_new must be >= 0 (got %d)", n_new);
  if (capacity <= 0) return fail(FA_ERR_INVALID, "capacity must be positive (got %d)", capacity);
  if (n_new == 0) return FA_OK;
  if (!k_new || !v_new || !pos || !k_cache || !v_cache || !k_scale || !v_scale)
    return fail(FA_ERR_INVALID, "null pointer argument");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(k_scale) & 3u) || (reinterpret_cast<uintptr_t>(v_scale) & 3u) ||
      (reinterpret_cast<uintptr_t>(pos) & 3u))
    return fail(FA_ERR_INVALID, "new tokens and caches must be 16-byte aligned, scales and pos 4-byte aligned");
  fa::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.pos = pos;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.bh_kv = bh_kv;
  a.n_new = n_new;
  a.capacity = capacity;
  const char* name = "";
  hipError_t e = fa::launch_append(a, head_dim, x_dtype, static_cast<hipStream_t>(stream), &name);
  if (e != hipSuccess) return hip_fail(e, "append_kv launch");
  g_last_kernel = name;
  return FA_OK;
}

int fa_forward(const void* q, int32_t q_dtype, const void* k, const void* v, int32_t kv_dtype,
               const float* k_scale, const float* v_scale, void* out, int32_t out_dtype, float* lse_out,
               int32_t bh_q, int32_t bh_kv, int32_t s_q, int32_t s_k, int32_t head_dim, float softmax_scale,
               int32_t causal, int32_t window, const fa_epilogue_op* epi, int32_t n_epi, void* stream) {
  g_last_error.clear();
  if (int r = check_head_dim(head_dim)) return r;
  if (bh_q <= 0 || bh_kv <= 0) return fail(FA_ERR_INVALID, "bh_q and bh_kv must be positive");
  if (bh_q % bh_kv != 0) return fail(FA_ERR_INVALID, "bh_q (%d) must be a multiple of bh_kv (%d)", bh_q, bh_kv);
  if (s_q < 0 || s_k < 0) return fail(FA_ERR_INVALID, "sequence lengths must be >= 0");
  if (window < 0) return fail(FA_ERR_INVALID, "window must be >= 0");
  if (window > 0 && !causal) return fail(FA_ERR_INVALID, "window > 0 requires causal");
  if (q_dtype != FA_F32 && q_dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "q dtype must be FA_F32 or FA_BF16");
  if (kv_dtype != FA_F32 && kv_dtype != FA_BF16 && kv_dtype != FA_I8)
    return fail(FA_ERR_UNSUPPORTED, "kv dtype must be FA_F32, FA_BF16 or FA_I8");
  if (out_dtype != FA_F32 && out_dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "out dtype must be FA_F32 or FA_BF16");
  const bool f32_path = q_dtype == FA_F32 && (kv_dtype == FA_F32 || kv_dtype == FA_I8);
  const bool bf16_path = q_dtype == FA_BF16 && (kv_dtype == FA_BF16 || kv_dtype == FA_I8);
  if (!f32_path && !bf16_path)
    return fail(FA_ERR_UNSUPPORTED, "unsupported (q, kv) dtype pair (%d, %d)", q_dtype, kv_dtype);
  if (kv_dtype == FA_I8) {
    if (!k_scale || !v_scale) return fail(FA_ERR_INVALID, "int8 K/V need k_scale and v_scale");
  } else if (k_scale || v_scale) {
    return fail(FA_ERR_INVALID, "k_scale/v_scale must be NULL unless kv dtype is FA_I8");
  }
  fa::EpiArgs ea, sa;
  if (int r = fill_epilogue(epi, n_epi, &ea, &sa)) return r;
  if (s_q == 0) return FA_OK;
  if (!q || !out) return fail(FA_ERR_INVALID, "null q or out");
  if (s_k > 0 && (!k || !v)) return fail(FA_ERR_INVALID, "null k or v");
  if (!aligned16(q) || !aligned16(out) || (s_k > 0 && (!aligned16(k) || !aligned16(v))))
    return fail(FA_ERR_INVALID, "q, k, v and out must be 16-byte aligned");
  if ((k_scale && (reinterpret_cast<uintptr_t>(k_scale) & 15u)) ||
      (v_scale && (reinterpret_cast<uintptr_t>(v_scale) & 15u)) ||
      (lse_out && (reinterpret_cast<uintptr_t>(lse_out) & 3u)))
    return fail(FA_ERR_INVALID, "scales must be 16-byte aligned and lse_out 4-byte aligned");

  fa::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.out = out;
  a.lse = lse_out;
  a.bh_q = bh_q;
  a.bh_kv = bh_kv;
  a.group = bh_q / bh_kv;
  a.s_q = s_q;
  a.s_k = s_k;
  a.causal = causal ? 1 : 0;
  a.window = (window > 0 && window < s_k) ? window : 0;   // W >= s_k is plain causal
  a.out_bf16 = out_dtype == FA_BF16;
  a.scale = resolve_scale(softmax_scale, head_dim);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.epi = ea;
  a.sops = sa;
  const char* name = "";
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = f32_path              ? fa::launch_prefill_f32(a, head_dim, kv_dtype, st, &name)
                 : kv_dtype == FA_I8   ? fa::launch_prefill_i8kv(a, head_dim, st, &name)
                                       : fa::launch_prefill_bf16(a, head_dim, st, &name);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  g_last_kernel = name;
  return FA_OK;
}

int fa_merge_lse(const float* o_parts, const float* lse_parts, int32_t n_parts, int64_t rows, int32_t head_dim,
                 void* out, int32_t out_dtype, float* lse_out, const fa_epilogue_op* epi, int32_t n_epi,
                 void* stream) {
  g_last_error.clear();
  if (int r = check_head_dim(head_dim)) return r;
  if (n_parts <= 0) return fail(FA_ERR_INVALID, "n_parts must be positive (got %d)", n_parts);
  if (rows < 0) return fail(FA_ERR_INVALID, "rows must be >= 0");
  if (out_dtype != FA_F32 && out_dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "out dtype must be FA_F32 or FA_BF16");
  fa::EpiArgs ea;
  if (int r = fill_epilogue(epi, n_epi, &ea, nullptr)) return r;
  if (rows == 0) return FA_OK;
  if (!o_parts || !lse_parts || !out) return fail(FA_ERR_INVALID, "null pointer argument");
  if (!aligned16(o_parts) || !aligned16(out) || (reinterpret_cast<uintptr_t>(lse_parts) & 3u) ||
      (lse_out && (reinterpret_cast<uintptr_t>(lse_out) & 3u)))
    return fail(FA_ERR_INVALID, "o_parts and out must be 16-byte aligned, lse arrays 4-byte aligned");
  fa::MergeArgs a;
  a.o_parts = o_parts;
  a.lse_parts = lse_parts;
  a.out = out;
  a.lse = lse_out;
  a.rows = rows;
  a.n_parts = n_parts;
  a.out_bf16 = out_dtype == FA_BF16;
  a.epi = ea;
  const char* name = "";
  hipError_t e = fa::launch_merge(a, head_dim, static_cast<hipStream_t>(stream), &name);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  g_last_kernel = name;
  return FA_OK;
}

namespace {
int check_tq(int32_t head_dim, int32_t bits) {
  if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(FA_ERR_UNSUPPORTED, "TurboQuant needs a power-of-two head_dim in [32, 256] (got %d)", head_dim);
  if (bits < 2 || bits > 4) return fail(FA_ERR_UNSUPPORTED, "TurboQuant bits must be 2, 3 or 4 (got %d)", bits);
  return FA_OK;
}
int check_codebook(const float* cb, int32_t bits) {
  if (!cb) return fail(FA_ERR_INVALID, "null codebook");
  for (int k = 1; k < (1 << bits); ++k)
    if (!(cb[k] > cb[k - 1])) return fail(FA_ERR_INVALID, "codebook must be strictly increasing");
  return FA_OK;
}
}  // namespace

int fa_tq_codebook(int32_t head_dim, int32_t bits, float* centroids) {
  g_last_error.clear();
  if (int r = check_tq(head_dim, bits)) return r;
  if (!centroids) return fail(FA_ERR_INVALID, "null centroids");
  fa::tq_codebook(head_dim, bits, centroids);
  return FA_OK;
}

int fa_tq_encode(const void* x, int32_t x_dtype, int64_t n_tokens, int32_t head_dim, int32_t bits,
                 const int8_t* signs, const float* codebook, uint8_t* codes_out, float* norms_out, void* stream) {
  g_last_error.clear();
  if (int r = check_tq(head_dim, bits)) return r;
  if (x_dtype != FA_F32 && x_dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "tq_encode input must be FA_F32 or FA_BF16 (got %d)", x_dtype);
  if (n_tokens < 0) return fail(FA_ERR_INVALID, "n_tokens must be >= 0");
  if (int r = check_codebook(codebook, bits)) return r;
  for (int k = 0; k < (1 << bits); ++k)
    if (codebook[k] != -codebook[(1 << bits) - 1 - k])
      return fail(FA_ERR_INVALID, "tq_encode codebook must be antisymmetric (c[k] == -c[2^bits - 1 - k])");
  if (n_tokens == 0) return FA_OK;
  if (!x || !signs || !codes_out || !norms_out) return fail(FA_ERR_INVALID, "null pointer argument");
  if (!aligned16(x) || !aligned16(codes_out) || (reinterpret_cast<uintptr_t>(norms_out) & 3u))
    return fail(FA_ERR_INVALID, "x and codes must be 16-byte aligned, norms 4-byte aligned");
  fa::TqArgs a{};
  a.x = x;
  a.signs = signs;
  a.codes = codes_out;
  a.norms = norms_out;
  a.n = n_tokens;
  a.inv_sqrt_d = 1.0f / std::sqrt((float)head_dim);
  for (int k = 0; k + 1 < (1 << bits); ++k) a.thr[k] = 0.5f * (codebook[k] + codebook[k + 1]);
  const char* name = "";
  hipError_t e = fa::launch_tq_encode(a, head_dim, bits, x_dtype, static_cast<hipStream_t>(stream), &name);
  if (e != hipSuccess) return hip_fail(e, "tq_encode launch");
  g_last_kernel = name;
  return FA_OK;
}

int fa_tq_decode(const uint8_t* codes, const float* norms, int64_t n_tokens, int32_t head_dim, int32_t bits,
                 const int8_t* signs, const float* codebook, void* out, int32_t out_dtype, void* stream) {
  g_last_error.clear();
  if (int r = check_tq(head_dim, bits)) return r;
  if (out_dtype != FA_F32 && out_dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "out dtype must be FA_F32 or FA_BF16");
  if (n_tokens < 0) return fail(FA_ERR_INVALID, "n_tokens must be >= 0");
  if (int r = check_codebook(codebook, bits)) return r;
  if (n_tokens == 0) return FA_OK;
  if (!codes || !norms || !signs || !out) return fail(FA_ERR_INVALID, "null pointer argument");
  if (!aligned16(codes) || !aligned16(out) || (reinterpret_cast<uintptr_t>(norms) & 3u))
    return fail(FA_ERR_INVALID, "codes and out must be 16-byte aligned, norms 4-byte aligned");
  fa::TqArgs a{};
  a.signs = signs;
  a.codes = const_cast<uint8_t*>(codes);
  a.norms = const_cast<float*>(norms);
  a.out = out;
  a.n = n_tokens;
  a.inv_sqrt_d = 1.0f / std::sqrt((float)head_dim);
  for (int k = 0; k < (1 << bits); ++k) a.cb[k] = codebook[k];
  const char* name = "";
  hipError_t e = fa::launch_tq_decode(a, head_dim, bits, out_dtype == FA_BF16, static_cast<hipStream_t>(stream), &name);
  if (e != hipSuccess) return hip_fail(e, "tq_decode launch");
  g_last_kernel = name;
  return FA_OK;
}

int32_t fa_decode_num_splits(int32_t bh_q, int32_t bh_kv, int32_t s_k, int32_t head_dim) {
  if (bh_kv <= 0 || bh_q <= 0 || s_k <= 0) return 1;
  const int32_t group = bh_q / bh_kv;
  const int32_t hpw = fa::decode_heads_per_workgroup(group, head_dim);
  const int32_t col_groups = (group + hpw - 1) / hpw;   // decode workgroups per (split, KV head)
  const int64_t units = (int64_t)bh_kv * col_groups;
  const int32_t tiles = (s_k + kDecodeTile - 1) / kDecodeTile;
  // one workgroup per CU (256), each split keeping at least 16 tiles (4 per wave)
  int64_t splits = (256 + units - 1) / units;
  const int64_t max_by_len = tiles / 16 > 0 ? tiles / 16 : 1;
  if (splits > max_by_len) splits = max_by_len;
  if (splits > kMaxSplits) splits = kMaxSplits;
  if (splits < 1) splits = 1;
  return (int32_t)splits;
}

size_t fa_decode_workspace_bytes(int32_t bh_q, int32_t bh_kv, int32_t s_k, int32_t head_dim, int32_t num_splits) {
  if (bh_q <= 0 || head_dim <= 0) return 0;
  if (num_splits <= 0) num_splits = fa_decode_num_splits(bh_q, bh_kv, s_k, head_dim);
  return (size_t)bh_q * (size_t)num_splits * (size_t)(head_dim + 2) * sizeof(float);
}

}  // extern "C"

namespace {

// fa_decode and fa_decode_noalloc: the same checks and kernels; `noalloc` selects the library's
// fixed scratch array instead of the caller's workspace.
int decode_impl(const void* q, int32_t q_dtype, const int8_t* k, const int8_t* v, const float* k_scale,
                const float* v_scale, void* out, int32_t out_dtype, float* lse_out, int32_t bh_q, int32_t bh_kv,
                int32_t s_k, int32_t head_dim, float softmax_scale, int32_t window, int32_t num_splits,
                const fa_epilogue_op* epi, int32_t n_epi, void* workspace, size_t workspace_bytes, bool noalloc,
                void* stream) {
  g_last_error.clear();
  if (int r = check_head_dim(head_dim)) return r;
  if (bh_q <= 0 || bh_kv <= 0) return fail(FA_ERR_INVALID, "bh_q and bh_kv must be positive");
  if (bh_q % bh_kv != 0) return fail(FA_ERR_INVALID, "bh_q (%d) must be a multiple of bh_kv (%d)", bh_q, bh_kv);
  if (s_k < 0) return fail(FA_ERR_INVALID, "s_k must be >= 0");
  if (window < 0) return fail(FA_ERR_INVALID, "window must be >= 0");
  if (q_dtype != FA_F32 && q_dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "decode q must be FA_F32 or FA_BF16");
  if (out_dtype != FA_F32 && out_dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "decode out must be FA_F32 or FA_BF16");
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(FA_ERR_INVALID, "num_splits must be in [0, %d] (got %d)", kMaxSplits, num_splits);
  fa::EpiArgs ea, sa;
  if (int r = fill_epilogue(epi, n_epi, &ea, &sa)) return r;
  if (!q || !out) return fail(FA_ERR_INVALID, "null q or out");
  if (s_k > 0 && (!k || !v || !k_scale || !v_scale)) return fail(FA_ERR_INVALID, "null k, v or scales");
  if (!aligned16(q) || !aligned16(out) || (s_k > 0 && (!aligned16(k) || !aligned16(v) || !aligned16(k_scale) ||
                                                        !aligned16(v_scale))))
    return fail(FA_ERR_INVALID, "q, k, v, scales and out must be 16-byte aligned");
  if (lse_out && (reinterpret_cast<uintptr_t>(lse_out) & 3u)) return fail(FA_ERR_INVALID, "lse_out must be 4-byte aligned");
  const int32_t splits = num_splits > 0 ? num_splits : fa_decode_num_splits(bh_q, bh_kv, s_k, head_dim);
  const size_t need = (size_t)bh_q * (size_t)splits * (size_t)(head_dim + 2) * sizeof(float);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (noalloc) {
    if (need > fa::kDecodeScratchBytes)
      return fail(FA_ERR_WORKSPACE, "decode partial states need %zu bytes, above the %zu-byte scratch of "
                  "fa_decode_noalloc (fewer splits or heads per call, or fa_decode with a workspace)",
                  need, fa::kDecodeScratchBytes);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    const int sdev = hipGetStreamDeviceId(st);
    if (sdev != dev)
      return fail(FA_ERR_INVALID, "the stream belongs to device %d but device %d is current", sdev, dev);
    e = fa::decode_scratch_address(dev, &workspace);
    if (e != hipSuccess) return hip_fail(e, "decode scratch address");
  } else {
    if (!workspace || workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "decode workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                  workspace ? "" : ", NULL");
    if (!aligned16(workspace)) return fail(FA_ERR_INVALID, "workspace must be 16-byte aligned");
  }

  fa::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.out = out;
  a.lse = lse_out;
  a.partial = static_cast<float*>(workspace);
  a.bh_q = bh_q;
  a.bh_kv = bh_kv;
  a.group = bh_q / bh_kv;
  a.s_k = s_k;
  a.key_lo = (window > 0 && window < s_k) ? s_k - window : 0;
  a.num_splits = splits;
  const int32_t tiles = (s_k - a.key_lo + kDecodeTile - 1) / kDecodeTile;
  a.tiles_per_split = (tiles + splits - 1) / splits;
  a.q_bf16 = q_dtype == FA_BF16;
  a.out_bf16 = out_dtype == FA_BF16;
  a.scale = resolve_scale(softmax_scale, head_dim);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.epi = ea;
  a.sops = sa;
  const char* name = "";
  hipError_t e = fa::launch_decode(a, head_dim, st, &name);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  g_last_kernel = name;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_decode(const void* q, int32_t q_dtype, const int8_t* k, const int8_t* v, const float* k_scale,
              const float* v_scale, void* out, int32_t out_dtype, float* lse_out, int32_t bh_q, int32_t bh_kv,
              int32_t s_k, int32_t head_dim, float softmax_scale, int32_t window, int32_t num_splits,
              const fa_epilogue_op* epi, int32_t n_epi, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, q_dtype, k, v, k_scale, v_scale, out, out_dtype, lse_out, bh_q, bh_kv, s_k, head_dim,
                     softmax_scale, window, num_splits, epi, n_epi, workspace, workspace_bytes, false, stream);
}

int fa_decode_noalloc(const void* q, int32_t q_dtype, const int8_t* k, const int8_t* v, const float* k_scale,
                      const float* v_scale, void* out, int32_t out_dtype, float* lse_out, int32_t bh_q,
                      int32_t bh_kv, int32_t s_k, int32_t head_dim, float softmax_scale, int32_t window,
                      int32_t num_splits, const fa_epilogue_op* epi, int32_t n_epi, void* stream) {
  return decode_impl(q, q_dtype, k, v, k_scale, v_scale, out, out_dtype, lse_out, bh_q, bh_kv, s_k, head_dim,
                     softmax_scale, window, num_splits, epi, n_epi, nullptr, 0, true, stream);
}

size_t fa_decode_noalloc_max_bytes(void) { return fa::kDecodeScratchBytes; }

int32_t fa_tq_attention_num_splits(int32_t bh_q, int32_t bh_kv, int32_t s_k, int32_t head_dim) {
  (void)head_dim;
  if (bh_kv <= 0 || bh_q <= 0 || s_k <= 0) return 1;
  const int32_t group = bh_q / bh_kv;
  const int64_t units = (int64_t)bh_kv * ((group + 3) / 4);
  const int32_t tiles = (s_k + kTqAttnTile - 1) / kTqAttnTile;
  // about 512 workgroups (two fit on a CU at once; more splits spread each workgroup's start, the
  // q rotation and digit split, over fewer tiles: 152 against 150 us at 8 and 4 splits per KV
  // head on the long-cache shape), each split keeping at least 8 tiles (2 per wave)
  int64_t splits = (512 + units - 1) / units;
  const int64_t max_by_len = tiles / 8 > 0 ? tiles / 8 : 1;
  if (splits > max_by_len) splits = max_by_len;
  if (splits > kMaxSplits) splits = kMaxSplits;
  if (splits < 1) splits = 1;
  return (int32_t)splits;
}

size_t fa_tq_attention_workspace_bytes(int32_t bh_q, int32_t bh_kv, int32_t s_k, int32_t head_dim,
                                       int32_t num_splits) {
  if (bh_q <= 0 || head_dim <= 0) return 0;
  if (num_splits <= 0) num_splits = fa_tq_attention_num_splits(bh_q, bh_kv, s_k, head_dim);
  return (size_t)bh_q * (size_t)num_splits * (size_t)(head_dim + 2) * sizeof(float);
}

int fa_tq_attention_decode(const void* q, int32_t q_dtype, const uint8_t* k_codes, const float* k_norms,
                           const int8_t* k_signs, int32_t k_bits, const float* k_codebook, const uint8_t* v_codes,
                           const float* v_norms, const int8_t* v_signs, int32_t v_bits, const float* v_codebook,
                           void* out, int32_t out_dtype, float* lse_out, int32_t bh_q, int32_t bh_kv, int32_t s_k,
                           int32_t head_dim, float softmax_scale, int32_t window, int32_t num_splits,
                           const fa_epilogue_op* epi, int32_t n_epi, void* workspace, size_t workspace_bytes,
                           void* stream) {
  g_last_error.clear();
  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "TurboQuant attention needs head_dim 64 or 128 (got %d)", head_dim);
  if (k_bits < 2 || k_bits > 4 || v_bits < 2 || v_bits > 4)
    return fail(FA_ERR_UNSUPPORTED, "TurboQuant attention reads 2-, 3- or 4-bit codes (got K %d, V %d)", k_bits, v_bits);
  if (bh_q <= 0 || bh_kv <= 0) return fail(FA_ERR_INVALID, "bh_q and bh_kv must be positive");
  if (bh_q % bh_kv != 0) return fail(FA_ERR_INVALID, "bh_q (%d) must be a multiple of bh_kv (%d)", bh_q, bh_kv);
  if (s_k < 0) return fail(FA_ERR_INVALID, "s_k must be >= 0");
  if (window < 0) return fail(FA_ERR_INVALID, "window must be >= 0");
  if (q_dtype != FA_F32 && q_dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "q must be FA_F32 or FA_BF16");
  if (out_dtype != FA_F32 && out_dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "out must be FA_F32 or FA_BF16");
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(FA_ERR_INVALID, "num_splits must be in [0, %d] (got %d)", kMaxSplits, num_splits);
  if (int r = check_codebook(k_codebook, k_bits)) return r;
  if (int r = check_codebook(v_codebook, v_bits)) return r;
  fa::EpiArgs ea, sa;
  if (int r = fill_epilogue(epi, n_epi, &ea, &sa)) return r;
  if (!q || !out || !k_signs || !v_signs) return fail(FA_ERR_INVALID, "null q, out or signs");
  if (s_k > 0 && (!k_codes || !v_codes || !k_norms || !v_norms)) return fail(FA_ERR_INVALID, "null codes or norms");
  if (!aligned16(q) || !aligned16(out) || (s_k > 0 && (!aligned16(k_codes) || !aligned16(v_codes))))
    return fail(FA_ERR_INVALID, "q, codes and out must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(k_norms) & 3u) || (reinterpret_cast<uintptr_t>(v_norms) & 3u) ||
      (lse_out && (reinterpret_cast<uintptr_t>(lse_out) & 3u)))
    return fail(FA_ERR_INVALID, "norms and lse_out must be 4-byte aligned");
  const int32_t splits = num_splits > 0 ? num_splits : fa_tq_attention_num_splits(bh_q, bh_kv, s_k, head_dim);
  const size_t need = (size_t)bh_q * (size_t)splits * (size_t)(head_dim + 2) * sizeof(float);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "TurboQuant attention workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return fail(FA_ERR_INVALID, "workspace must be 16-byte aligned");

  fa::TqAttnArgs a{};
  a.q = q;
  a.kc = k_codes;
  a.kn = k_norms;
  a.vc = v_codes;
  a.vn = v_norms;
  a.ks = k_signs;
  a.vs = v_signs;
  a.out = out;
  a.lse = lse_out;
  a.partial = static_cast<float*>(workspace);
  a.bh_q = bh_q;
  a.bh_kv = bh_kv;
  a.group = bh_q / bh_kv;
  a.s_k = s_k;
  a.key_lo = (window > 0 && window < s_k) ? s_k - window : 0;
  a.num_splits = splits;
  const int32_t tiles = (s_k - a.key_lo + kTqAttnTile - 1) / kTqAttnTile;
  a.tiles_per_split = (tiles + splits - 1) / splits;
  a.q_bf16 = q_dtype == FA_BF16;
  a.out_bf16 = out_dtype == FA_BF16;
  a.scale = resolve_scale(softmax_scale, head_dim);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.k_e = codebook_digits(k_codebook, k_bits, a.ktab);
  a.v_e = codebook_digits(v_codebook, v_bits, a.vtab);
  a.epi = ea;
  a.sops = sa;
  const char* name = "";
  hipError_t e = fa::launch_tq_attention(a, head_dim, k_bits, v_bits, static_cast<hipStream_t>(stream), &name);
  if (e != hipSuccess) return hip_fail(e, "TurboQuant attention launch");
  g_last_kernel = name;
  return FA_OK;
}

}  // extern "C"
