// TurboQuant KV codec: 2- or 4-bit codes per channel from a randomized Hadamard rotation, an
// L2 normalisation and a Lloyd-Max scalar codebook (Foundry attention/ README, section
// "TurboQuant KV Cache Compression": signs applied before the Hadamard transform, the L2 norm
// as normaliser, Lloyd-Max quantization against Beta(d/2, d/2) codebooks, bit-packing).
//
// Per vector x (head_dim d, a power of two) with random signs s:
//   y = H (s * x) (Sylvester Hadamard, unnormalised), n = ||x||, u = y / ||y||,
//   code_i = number of thresholds t_k <= u_i (thresholds = midpoints of the codebook),
//   packed little-endian, channel i at bit (i b) mod 8 of byte (i b) / 8; n stored as fp32.
// Decode: x_hat = s * H (n c[code]) / sqrt(d).
//
// A segment of d / ELEM lanes owns a vector, ELEM values per lane (16 bytes of input); the
// Hadamard butterflies run inside a lane for strides below ELEM and across lanes above it.
// The codebook itself is computed on the host (fa_tq_codebook): Lloyd-Max iterations with the
// cell masses and first moments of the Beta(d/2, d/2) law integrated by Gauss-Legendre
// quadrature.
#include <cmath>
#include <vector>

#include "device_common.hpp"

namespace fa {
namespace {

constexpr int pow2_at_least(int r) { return r <= 1 ? 1 : 2 * pow2_at_least((r + 1) / 2); }

// in-place Walsh-Hadamard (Sylvester order) of the ELEM values of each lane and across the SEG
// lanes of a segment: element index = ELEM * (lane % SEG) + e
template <int ELEM, int SEG>
__device__ __forceinline__ void hadamard_segment(float (&v)[ELEM], int lane) {
#pragma unroll
  for (int h = 1; h < ELEM; h <<= 1)
#pragma unroll
    for (int e = 0; e < ELEM; ++e)
      if ((e & h) == 0) {
        const float a = v[e], b = v[e + h];
        v[e] = a + b;
        v[e + h] = a - b;
      }
#pragma unroll
  for (int lh = 1; lh < SEG; lh <<= 1) {
    const bool upper = lane & lh;
#pragma unroll
    for (int e = 0; e < ELEM; ++e) {
      const float p = __shfl_xor(v[e], lh, 64);
      v[e] = upper ? p - v[e] : v[e] + p;
    }
  }
}

template <int SEG>
__device__ __forceinline__ float segment_sum(float a) {
#pragma unroll
  for (int o = SEG / 2; o >= 1; o >>= 1) a += __shfl_xor(a, o, 64);
  return a;
}

template <int D, bool BF16_IN, int BITS>
__global__ __launch_bounds__(256) void tq_encode_kernel(TqArgs a) {
  constexpr int ELEM = BF16_IN ? 8 : 4;
  constexpr int SEG = D / ELEM;                // lanes per vector (power of two)
  constexpr int RPW = 64 / SEG;
  constexpr int NT = (1 << BITS) - 1;          // thresholds
  const int lane = threadIdx.x & 63;
  const int sl = lane % SEG;
  const int64_t row = (((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6) * RPW + lane / SEG;
  // every lane takes part in the butterflies: rows past the end repeat the last row
  const int64_t r = min(row, a.n - 1);
  float v[ELEM];
  if constexpr (BF16_IN) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const unsigned short*>(a.x) + r * D + ELEM * sl);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
    const f32x4 w = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.x) + r * D + ELEM * sl);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = w[e];
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < ELEM; ++e) {
    ss = __builtin_fmaf(v[e], v[e], ss);
    v[e] = a.signs[ELEM * sl + e] < 0 ? -v[e] : v[e];
  }
  const float n = __fsqrt_rn(segment_sum<SEG>(ss));
  hadamard_segment<ELEM, SEG>(v, lane);
  float yy = 0.f;
#pragma unroll
  for (int e = 0; e < ELEM; ++e) yy = __builtin_fmaf(v[e], v[e], yy);
  const float ny = __fsqrt_rn(segment_sum<SEG>(yy));
  const float inv = ny > 0.f ? __fdiv_rn(1.0f, ny) : 0.f;
  unsigned packed = 0;
#pragma unroll
  for (int e = 0; e < ELEM; ++e) {
    const float u = v[e] * inv;
    int code = 0;
#pragma unroll
    for (int k = 0; k < NT; ++k) code += u >= a.thr[k] ? 1 : 0;
    packed |= (unsigned)code << (BITS * e);
  }
  if (row < a.n) {
    uint8_t* dst = a.codes + row * (D * BITS / 8) + sl * (ELEM * BITS / 8);
    if constexpr (ELEM * BITS == 32) *reinterpret_cast<unsigned*>(dst) = packed;
    else if constexpr (ELEM * BITS == 16) *reinterpret_cast<unsigned short*>(dst) = (unsigned short)packed;
    else *dst = (uint8_t)packed;
    if (sl == 0) a.norms[row] = n;
  }
}

template <int D, bool BF16_OUT, int BITS>
__global__ __launch_bounds__(256) void tq_decode_kernel(TqArgs a) {
  constexpr int ELEM = 4;                      // fp32 values per lane
  constexpr int SEG = D / ELEM;
  constexpr int RPW = 64 / SEG;
  const int lane = threadIdx.x & 63;
  const int sl = lane % SEG;
  const int64_t row = (((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6) * RPW + lane / SEG;
  const int64_t r = min(row, a.n - 1);
  const uint8_t* src = a.codes + r * (D * BITS / 8) + sl * (ELEM * BITS / 8);
  const unsigned packed = BITS == 4 ? *reinterpret_cast<const unsigned short*>(src) : *src;
  const float n = a.norms[r];
  float v[ELEM];
#pragma unroll
  for (int e = 0; e < ELEM; ++e) {
    const int code = (packed >> (BITS * e)) & ((1u << BITS) - 1);
    float c = a.cb[0];
#pragma unroll
    for (int k = 1; k < (1 << BITS); ++k) c = code == k ? a.cb[k] : c;
    v[e] = n * c;
  }
  hadamard_segment<ELEM, SEG>(v, lane);
  const float scale = a.inv_sqrt_d;
#pragma unroll
  for (int e = 0; e < ELEM; ++e) {
    const float x = v[e] * scale;
    v[e] = a.signs[ELEM * sl + e] < 0 ? -x : x;
  }
  if (row < a.n) {
    if constexpr (BF16_OUT) {
      const u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *reinterpret_cast<u32x2*>(static_cast<unsigned short*>(a.out) + row * D + ELEM * sl) = w;
    } else {
      const f32x4 w = {v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * D + ELEM * sl) = w;
    }
  }
}

template <int D, int BITS>
hipError_t launch_encode_d(const TqArgs& a, bool bf16, hipStream_t st, const char** name) {
  const int seg = D / (bf16 ? 8 : 4);
  const int64_t rows_per_block = 4 * (64 / seg);
  const int64_t blocks = (a.n + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (bf16) hipLaunchKernelGGL((tq_encode_kernel<D, true, BITS>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((tq_encode_kernel<D, false, BITS>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  *name = "tq_encode";
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t launch_decode_d(const TqArgs& a, bool bf16_out, hipStream_t st, const char** name) {
  const int64_t rows_per_block = 4 * (64 / (D / 4));
  const int64_t blocks = (a.n + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (bf16_out) hipLaunchKernelGGL((tq_decode_kernel<D, true, BITS>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((tq_decode_kernel<D, false, BITS>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  *name = "tq_decode";
  return hipGetLastError();
}

template <int BITS>
hipError_t encode_bits(const TqArgs& a, int32_t d, bool bf16, hipStream_t st, const char** name) {
  switch (d) {
    case 32: return launch_encode_d<32, BITS>(a, bf16, st, name);
    case 64: return launch_encode_d<64, BITS>(a, bf16, st, name);
    case 128: return launch_encode_d<128, BITS>(a, bf16, st, name);
    case 256: return launch_encode_d<256, BITS>(a, bf16, st, name);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS>
hipError_t decode_bits(const TqArgs& a, int32_t d, bool bf16_out, hipStream_t st, const char** name) {
  switch (d) {
    case 32: return launch_decode_d<32, BITS>(a, bf16_out, st, name);
    case 64: return launch_decode_d<64, BITS>(a, bf16_out, st, name);
    case 128: return launch_decode_d<128, BITS>(a, bf16_out, st, name);
    case 256: return launch_decode_d<256, BITS>(a, bf16_out, st, name);
    default: return hipErrorInvalidValue;
  }
}

// ---- host: Lloyd-Max codebook of u = 2B - 1, B ~ Beta(d/2, d/2), density prop. to (1 - u^2)^(d/2 - 1)

// Gauss-Legendre nodes and weights of order kGl on [-1, 1]: roots of P_n by Newton's method on
// the three-term recurrence, weights 2 / ((1 - x^2) P_n'(x)^2)
constexpr int kGl = 16;
struct GaussLegendre {
  double x[kGl], w[kGl];
  GaussLegendre() {
    for (int i = 0; i < kGl; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (kGl + 0.5)), dp = 1.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= kGl; ++k) {
          const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        dp = kGl * (z * p1 - p0) / (z * z - 1.0);
        const double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-16) break;
      }
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

// integrals of w(u) and u w(u) over [lo, hi], w(u) = (1 - u^2)^(a - 1), composite Gauss-Legendre
void moments(const GaussLegendre& gl, double a, double lo, double hi, double* m0, double* m1) {
  constexpr int kPieces = 24;
  double s0 = 0.0, s1 = 0.0;
  const double step = (hi - lo) / kPieces, half = 0.5 * step;
  for (int p = 0; p < kPieces; ++p) {
    const double mid = lo + (p + 0.5) * step;
    for (int i = 0; i < kGl; ++i) {
      const double u = mid + half * gl.x[i];
      const double w = std::exp((a - 1.0) * std::log1p(-u * u)) * gl.w[i] * half;
      s0 += w;
      s1 += w * u;
    }
  }
  *m0 = s0;
  *m1 = s1;
}

}  // namespace

int tq_codebook(int32_t d, int32_t bits, float* centroids) {
  const double a = d / 2.0;
  const int n = 1 << bits;
  // the law is concentrated within a few standard deviations (1 / sqrt(d + 1)) of 0; cells
  // beyond +-1 have no mass
  const double sd = 1.0 / std::sqrt(d + 1.0);
  std::vector<double> c(n), t(n + 1);
  for (int k = 0; k < n; ++k) c[k] = sd * (-2.5 + 5.0 * (k + 0.5) / n);
  static const GaussLegendre gl;
  for (int it = 0; it < 100000; ++it) {
    t[0] = -1.0;
    t[n] = 1.0;
    for (int k = 1; k < n; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    double change = 0.0;
    for (int k = 0; k < n; ++k) {
      double m0, m1;
      moments(gl, a, t[k], t[k + 1], &m0, &m1);
      const double ck = m1 / m0;
      change = std::fmax(change, std::fabs(ck - c[k]));
      c[k] = ck;
    }
    if (change < 1e-15) break;
  }
  for (int k = 0; k < n; ++k) centroids[k] = (float)c[k];
  return 0;
}

hipError_t launch_tq_encode(const TqArgs& a, int32_t d, int32_t bits, int32_t x_dtype, hipStream_t st,
                            const char** name) {
  const bool bf16 = x_dtype == kBF16;
  return bits == 4 ? encode_bits<4>(a, d, bf16, st, name) : encode_bits<2>(a, d, bf16, st, name);
}

hipError_t launch_tq_decode(const TqArgs& a, int32_t d, int32_t bits, bool bf16_out, hipStream_t st,
                            const char** name) {
  return bits == 4 ? decode_bits<4>(a, d, bf16_out, st, name) : decode_bits<2>(a, d, bf16_out, st, name);
}

}  // namespace fa
