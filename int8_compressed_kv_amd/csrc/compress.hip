// Per-token int8 quantization of K/V rows (fkl.flash_attention PR, Summary: compress_kv(),
// int8 codes with one fp32 scale per token).
//
// Per token: a = max|x| (exact), s = a / 127 with one IEEE fp32 division, code =
// rint(x / s) with the IEEE fp32 quotient (ties to even), clamped to [-127, 127];
// an all-zero token gets s = 0 and codes 0.  The quotients are computed exactly as IEEE
// division would round them, from a correctly rounded reciprocal and one fma correction.
//
// HBM-bound streaming kernel: a token row is owned by a segment of lanes, each lane
// reading 16 contiguous bytes, so a wave's load covers whole rows with full coalescing.
// Traffic per token: d * sizeof(in) read, d + 4 bytes written.
#include "device_common.hpp"

namespace fa {
namespace {

constexpr int pow2_at_least(int r) { return r <= 1 ? 1 : 2 * pow2_at_least((r + 1) / 2); }

template <int N>
__device__ __forceinline__ float dpp_row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

// max over aligned groups of SEG lanes.  Groups of 16 or more use DPP rotations within each
// 16-lane row and the row / half-wave swaps (all VALU); smaller groups use lane shuffles.
template <int SEG>
__device__ __forceinline__ float segment_max(float a) {
  if constexpr (SEG >= 16) {
    a = fmaxf(a, dpp_row_ror<8>(a));
    a = fmaxf(a, dpp_row_ror<4>(a));
    a = fmaxf(a, dpp_row_ror<2>(a));
    a = fmaxf(a, dpp_row_ror<1>(a));
    if constexpr (SEG >= 32) a = max_xor16(a);
    if constexpr (SEG >= 64) a = max_xor32(a);
  } else {
#pragma unroll
    for (int off = SEG / 2; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  }
  return a;
}

// Codes and scale of one token row held by a segment of SEG lanes, ELEM values per lane (every
// lane of the segment holds valid values; idle lanes repeat a chunk).  Returns s; packed[] gets
// the lane's ELEM codes, four per word.
template <int ELEM, int SEG>
__device__ __forceinline__ float quantize_row(const float (&x)[ELEM], unsigned (&packed)[ELEM / 4]) {
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < ELEM; ++e) a = fmaxf(a, fabsf(x[e]));
  a = segment_max<SEG>(a);
  const float s = __fdiv_rn(a, 127.0f);
  // code = rint(RN(x / s)) clamped to [-127, 127].  The correctly rounded quotient comes from
  // the correctly rounded reciprocal y = RN(1 / s) and one correction step (Markstein):
  // q0 = RN(x y) is within an ulp of x / s, the residual e = x - s q0 is exact in one fma,
  // and RN(q0 + e y) = RN(x / s).  It needs no over- or underflow, which holds for
  // s >= 2^-64 (|x / s| <= 127 + 2^-16 here); smaller nonzero scales take the IEEE division.
  const float y = __fdiv_rn(1.0f, s);
  float c[ELEM];
#pragma unroll
  for (int e = 0; e < ELEM; ++e) {
    const float q0 = x[e] * y;
    const float r = __builtin_fmaf(-s, q0, x[e]);
    c[e] = __builtin_amdgcn_fmed3f(__builtin_rintf(__builtin_fmaf(r, y, q0)), -127.f, 127.f);
  }
  if (__builtin_expect(__any(s < 0x1p-64f && s > 0.f), 0)) {
#pragma unroll
    for (int e = 0; e < ELEM; ++e)
      if (s < 0x1p-64f) c[e] = __builtin_amdgcn_fmed3f(__builtin_rintf(__fdiv_rn(x[e], s)), -127.f, 127.f);
  }
#pragma unroll
  for (int e4 = 0; e4 < ELEM / 4; ++e4) {
    unsigned w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int ci = s > 0.f ? (int)c[4 * e4 + b] : 0;   // an all-zero token: s = 0, codes 0
      w |= ((unsigned)ci & 0xffu) << (8 * b);
    }
    packed[e4] = w;
  }
  return s;
}

// 16 bytes of a row: ELEM values (fp32 x4 or bf16 x8, bf16 widened exactly)
template <bool BF16_IN, int ELEM>
__device__ __forceinline__ void load_chunk(const void* p, float (&x)[ELEM]) {
  if constexpr (BF16_IN) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = w[e];
  }
}

// the lane's codes of a row at dst (ELEM bytes)
template <int ELEM>
__device__ __forceinline__ void store_codes(int8_t* dst, const unsigned (&packed)[ELEM / 4]) {
  if constexpr (ELEM == 8) {
    const u32x2 p2 = {packed[0], packed[ELEM / 4 - 1]};
    __builtin_nontemporal_store(p2, reinterpret_cast<u32x2*>(dst));
  } else {
    __builtin_nontemporal_store(packed[0], reinterpret_cast<unsigned*>(dst));
  }
}

template <int D, bool BF16_IN, int U>
__global__ __launch_bounds__(256) void compress_kernel(const void* __restrict__ xin, int64_t n,
                                                       int8_t* __restrict__ qout,
                                                       float* __restrict__ sout) {
  constexpr int ELEM = BF16_IN ? 8 : 4;      // elements per lane (16 bytes)
  constexpr int R = D / ELEM;                 // active lanes per row
  constexpr int SEG = pow2_at_least(R);       // lanes reserved per row
  constexpr int RPW = 64 / SEG;               // rows per wave
  static_assert(SEG <= 64 && D % ELEM == 0, "bad row split");

  const int lane = threadIdx.x & 63;
  const int seg_lane = lane % SEG;
  const int sub = lane / SEG;
  const bool lane_on = seg_lane < R;
  const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * 256) >> 6;

  // loads are issued unconditionally (rows past the end repeat the last row, idle lanes of a
  // segment repeat its last chunk) so the code stays straight-line; only the stores are guarded.
  // Loads and stores are nontemporal: every byte is touched once.
  const int chunk = lane_on ? seg_lane : R - 1;
  for (int64_t base = wave * (RPW * U); base < n; base += nwaves * (RPW * U)) {
    float x[U][ELEM];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = min(base + (int64_t)u * RPW + sub, n - 1);
      load_chunk<BF16_IN, ELEM>(static_cast<const char*>(xin) + (row * D + chunk * ELEM) * (BF16_IN ? 2 : 4), x[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      unsigned packed[ELEM / 4];
      const float s = quantize_row<ELEM, SEG>(x[u], packed);
      const int64_t row = base + (int64_t)u * RPW + sub;
      if (lane_on && row < n) {
        store_codes<ELEM>(qout + row * D + seg_lane * ELEM, packed);
        if (seg_lane == 0) __builtin_nontemporal_store(s, sout + row);
      }
    }
  }
}

// Decode-time append: the n_new new tokens of every KV head, of K and of V, quantized exactly as
// above into cache rows pos[b] + j (positions read on the device, so the call can be replayed
// at advancing positions; one position per head also covers sequences of different lengths).
// Global row r covers matrix r / (bh_kv n_new) (K, then V), head b and new token j; rows whose
// cache position falls outside [0, capacity) are not written.
// With ROPE, each K row is first rotated by rotate-half RoPE at its cache position p (FlashRT
// QKV Cache RoPE: the decode K write rotates K before writing the slot): channel i < d/2 pairs
// with i + d/2, out_i = x_i cos_i - x_{i+d/2} sin_i, out_{i+d/2} = x_{i+d/2} cos_i + x_i sin_i
// (cos, sin = row p of the tables), each product and the sum rounded on its own.  The partner half
// of a lane's chunk sits R/2 lanes away in the row's segment and is fetched by a lane shuffle.
template <int D, bool BF16_IN, bool ROPE>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int ELEM = BF16_IN ? 8 : 4;
  constexpr int R = D / ELEM;
  constexpr int SEG = pow2_at_least(R);
  constexpr int RPW = 64 / SEG;
  const int lane = threadIdx.x & 63;
  const int seg_lane = lane % SEG;
  const bool lane_on = seg_lane < R;
  const int64_t per_mat = (int64_t)a.bh_kv * a.n_new;
  const int64_t total = 2 * per_mat;
  const int64_t r = (((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6) * RPW + lane / SEG;
  // every lane takes part in the row reduction: rows past the end repeat the last row
  const int64_t re = min(r, total - 1);
  const bool is_v = re >= per_mat;
  const int64_t rem = is_v ? re - per_mat : re;
  const int b = (int)(rem / a.n_new), j = (int)(rem % a.n_new);
  const int chunk = lane_on ? seg_lane : R - 1;
  float x[ELEM];
  load_chunk<BF16_IN, ELEM>(static_cast<const char*>(is_v ? a.v_new : a.k_new) + (rem * D + chunk * ELEM) * (BF16_IN ? 2 : 4), x);
  const int p = a.pos[b] + j;
  if constexpr (ROPE) {
    constexpr int HALF = R / 2;                     // chunks per half row (D/2 is a multiple of ELEM)
    const bool lower = chunk < HALF;
    const int partner = (lane - seg_lane) + (lower ? chunk + HALF : chunk - HALF);
    float xp[ELEM];
#pragma unroll
    for (int e = 0; e < ELEM; ++e) xp[e] = __shfl(x[e], partner, 64);   // every lane takes part
    const int64_t prow = (int64_t)min(max(p, 0), a.capacity - 1) * (D / 2) + (lower ? chunk : chunk - HALF) * ELEM;
    float cs[ELEM], sn[ELEM];
#pragma unroll
    for (int e4 = 0; e4 < ELEM / 4; ++e4) {
      const f32x4 c4 = *reinterpret_cast<const f32x4*>(a.rope_cos + prow + 4 * e4);
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(a.rope_sin + prow + 4 * e4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cs[4 * e4 + e] = c4[e];
        sn[4 * e4 + e] = s4[e];
      }
    }
    if (!is_v) {
#pragma unroll
      for (int e = 0; e < ELEM; ++e) {
        const float t = mul_rn(xp[e], sn[e]);
        x[e] = add_rn(mul_rn(x[e], cs[e]), lower ? -t : t);
      }
    }
  }
  unsigned packed[ELEM / 4];
  const float s = quantize_row<ELEM, SEG>(x, packed);
  if (r < total && lane_on && p >= 0 && p < a.capacity) {
    const int64_t dst = (int64_t)b * a.capacity + p;
    store_codes<ELEM>((is_v ? a.v_cache : a.k_cache) + dst * D + seg_lane * ELEM, packed);
    if (seg_lane == 0) (is_v ? a.v_scale : a.k_scale)[dst] = s;
  }
}

template <int D>
hipError_t launch_append_d(const AppendArgs& a, bool bf16, hipStream_t st, const char** name) {
  const int elem = bf16 ? 8 : 4;
  const int64_t rows_per_block = 4 * (64 / pow2_at_least(D / elem));
  const int64_t total = 2 * (int64_t)a.bh_kv * a.n_new;
  const int64_t blocks = (total + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const bool rope = a.rope_cos != nullptr;
  if (bf16) {
    if (rope) hipLaunchKernelGGL((append_kernel<D, true, true>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((append_kernel<D, true, false>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    *name = rope ? "append_rope_bf16" : "append_bf16";
  } else {
    if (rope) hipLaunchKernelGGL((append_kernel<D, false, true>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((append_kernel<D, false, false>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    *name = rope ? "append_rope_f32" : "append_f32";
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const void* x, bool bf16, int64_t n, int8_t* q, float* s, hipStream_t st,
                    const char** name) {
  // two rows per lane segment, and a full grid: each wave takes one group of rows (a grid capped
  // at a few blocks per CU, striding over more rows per wave, reached 4.8 TB/s against 6.4 here)
  constexpr int U = 2;
  const int elem = bf16 ? 8 : 4;
  const int seg = pow2_at_least(D / elem);
  const int64_t rows_per_block = (int64_t)(256 / 64) * (64 / seg) * U;
  int64_t blocks = (n + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (blocks < 1) blocks = 1;
  if (bf16) {
    hipLaunchKernelGGL((compress_kernel<D, true, U>), dim3((unsigned)blocks), dim3(256), 0, st, x, n, q, s);
    *name = "compress_bf16";
  } else {
    hipLaunchKernelGGL((compress_kernel<D, false, U>), dim3((unsigned)blocks), dim3(256), 0, st, x, n, q, s);
    *name = "compress_f32";
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compress(const void* x, int32_t x_dtype, int64_t n_tokens, int32_t d, int8_t* q_out,
                           float* scale_out, hipStream_t stream, const char** name) {
  const bool bf16 = x_dtype == kBF16;
  switch (d) {
    case 32: return launch_d<32>(x, bf16, n_tokens, q_out, scale_out, stream, name);
    case 64: return launch_d<64>(x, bf16, n_tokens, q_out, scale_out, stream, name);
    case 96: return launch_d<96>(x, bf16, n_tokens, q_out, scale_out, stream, name);
    case 128: return launch_d<128>(x, bf16, n_tokens, q_out, scale_out, stream, name);
    case 160: return launch_d<160>(x, bf16, n_tokens, q_out, scale_out, stream, name);
    case 192: return launch_d<192>(x, bf16, n_tokens, q_out, scale_out, stream, name);
    case 224: return launch_d<224>(x, bf16, n_tokens, q_out, scale_out, stream, name);
    case 256: return launch_d<256>(x, bf16, n_tokens, q_out, scale_out, stream, name);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_append(const AppendArgs& a, int32_t d, int32_t x_dtype, hipStream_t stream, const char** name) {
  const bool bf16 = x_dtype == kBF16;
  switch (d) {
    case 32: return launch_append_d<32>(a, bf16, stream, name);
    case 64: return launch_append_d<64>(a, bf16, stream, name);
    case 96: return launch_append_d<96>(a, bf16, stream, name);
    case 128: return launch_append_d<128>(a, bf16, stream, name);
    case 160: return launch_append_d<160>(a, bf16, stream, name);
    case 192: return launch_append_d<192>(a, bf16, stream, name);
    case 224: return launch_append_d<224>(a, bf16, stream, name);
    case 256: return launch_append_d<256>(a, bf16, stream, name);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
