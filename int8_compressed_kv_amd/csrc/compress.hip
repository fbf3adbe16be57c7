// Per-token int8 quantization of K/V rows (fkl.flash_attention PR, Summary: compress_kv(),
// int8 codes with one fp32 scale per token).
//
// Per token: a = max|x| (exact), s = a / 127 with one IEEE fp32 division, code =
// rint(x / s) with the IEEE fp32 quotient (ties to even), clamped to [-127, 127];
// an all-zero token gets s = 0 and codes 0.
//
// HBM-bound streaming kernel: a token row is owned by a segment of lanes, each lane
// reading 16 contiguous bytes, so a wave's load covers whole rows with full coalescing.
// Traffic per token: d * sizeof(in) read, d + 4 bytes written.
#include "device_common.hpp"

namespace fa {
namespace {

constexpr int pow2_at_least(int r) { return r <= 1 ? 1 : 2 * pow2_at_least((r + 1) / 2); }

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

  for (int64_t base = wave * (RPW * U); base < n; base += nwaves * (RPW * U)) {
    float x[U][ELEM];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = base + (int64_t)u * RPW + sub;
      ok[u] = lane_on && row < n;
      if (BF16_IN) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (ok[u])
          w = *reinterpret_cast<const u32x4*>(static_cast<const unsigned short*>(xin) + row * D +
                                              seg_lane * ELEM);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[u][2 * e] = __uint_as_float(w[e] << 16);
          x[u][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
      } else {
        f32x4 w = {0.f, 0.f, 0.f, 0.f};
        if (ok[u])
          w = *reinterpret_cast<const f32x4*>(static_cast<const float*>(xin) + row * D + seg_lane * ELEM);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[u][e] = w[e];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < ELEM; ++e) a = fmaxf(a, fabsf(x[u][e]));
#pragma unroll
      for (int off = SEG / 2; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
      const float s = __fdiv_rn(a, 127.0f);
      unsigned packed[ELEM / 4];
#pragma unroll
      for (int e4 = 0; e4 < ELEM / 4; ++e4) {
        unsigned w = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float c = 0.f;
          if (s > 0.f) {
            c = __builtin_rintf(__fdiv_rn(x[u][4 * e4 + b], s));
            c = fminf(fmaxf(c, -127.f), 127.f);
          }
          w |= ((unsigned)((int)c) & 0xffu) << (8 * b);
        }
        packed[e4] = w;
      }
      const int64_t row = base + (int64_t)u * RPW + sub;
      if (ok[u]) {
        if (ELEM == 8) {
          u32x2 p2 = {packed[0], packed[ELEM / 4 - 1]};
          *reinterpret_cast<u32x2*>(qout + row * D + seg_lane * ELEM) = p2;
        } else {
          *reinterpret_cast<unsigned*>(qout + row * D + seg_lane * ELEM) = packed[0];
        }
        if (seg_lane == 0) sout[row] = s;
      }
    }
  }
}

template <int D>
hipError_t launch_d(const void* x, bool bf16, int64_t n, int8_t* q, float* s, hipStream_t st,
                    const char** name) {
  constexpr int U = 4;
  const int elem = bf16 ? 8 : 4;
  const int seg = pow2_at_least(D / elem);
  const int64_t rows_per_block = (int64_t)(256 / 64) * (64 / seg) * U;
  int64_t blocks = (n + rows_per_block - 1) / rows_per_block;
  const int64_t cap = 256 * 16;   // grid-stride beyond 16 blocks per CU
  if (blocks > cap) blocks = cap;
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

}  // namespace fa
