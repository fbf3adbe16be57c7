// TurboQuant KV codec: 2-, 3- or 4-bit codes per channel from a randomized Hadamard rotation, an
// L2 normalisation and a Lloyd-Max scalar codebook (Foundry attention/ README, section
// "TurboQuant KV Cache Compression": signs applied before the Hadamard transform, the L2 norm
// as normaliser, Lloyd-Max quantization against Beta(d/2, d/2) codebooks, bit-packing).
//
// Per vector x (head_dim d, a power of two) with random signs s:
//   y = H (s * x) (Sylvester Hadamard, unnormalised), n = ||x||, u = y / ||y||,
//   code_i = number of thresholds t_k <= u_i (thresholds = midpoints of the codebook),
//   packed as one little-endian bit stream per vector, channel i at stream bits i b .. i b + b - 1
//   (a 3-bit code may straddle two bytes); n stored as fp32.
// Decode: x_hat = s * H (n c[code]) / sqrt(d).
//
// A segment of d / 16 lanes owns a vector, 16 values per lane; only the Hadamard stages over
// the lane bits of a channel index cross lanes (DPP quad permutes and ds_swizzle).  Decisions use
// the codebook's antisymmetry (a binary search over the positive thresholds: 2 steps at 3 bits,
// 3 at 4 bits, or a bucket table at 4 bits).
// The codebook itself is computed on the host (fa_tq_codebook): Lloyd-Max iterations with the
// cell masses and first moments of the Beta(d/2, d/2) law integrated by Gauss-Legendre
// quadrature.
#include <cmath>
#include <cstring>
#include <vector>

#include "device_common.hpp"

namespace fa {
namespace {

// A segment of SEG = d/16 lanes owns a vector, 16 values per lane: lane sl holds channels
// 16 sl .. 16 sl + 15 (NCH chunks of CE values, 16 bytes each), so its codes are 2 BITS contiguous
// bytes (one 8- or 4-byte word at 4 or 2 bits, three 2-byte words at 3 bits) and its loads and
// stores contiguous runs.  Channel c = 16 sl + CE j + e: the
// Hadamard stages over
// the bits of e and j stay inside the lane, the stages over the bits of sl cross lanes.
template <int CE>
struct Lay {
  static constexpr int NCH = 16 / CE;
};

// value of lane (lane ^ X) within aligned groups of X*2 lanes: DPP quad permutes for 1 and 2,
// ds_swizzle (xor mode over 32 lanes) for 4 and 8
template <int X>
__device__ __forceinline__ float lane_xor(float v) {
  const int b = __float_as_int(v);
  if constexpr (X == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, true));
  else if constexpr (X == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, true));
  else return __int_as_float(__builtin_amdgcn_ds_swizzle(b, (X << 10) | 0x1F));
}

// Butterfly across lanes l and l ^ X: with a on the lower lane and b on the upper, the lower takes
// a + b and the upper a - b, both partner + g * own with g = +1 (lower) or -1 (upper).
template <int X, int SEG>
__device__ __forceinline__ void cross_stage(float (&v)[16], int sl) {
  if constexpr (X < SEG) {
    const float g = (sl & X) ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __builtin_fmaf(g, v[i], lane_xor<X>(v[i]));
  }
}

// The same butterfly over quad lanes (X = 1, 2) as one DPP multiply-add per value: v = partner * g
// + own gives a + b on the lower lane and b - a = -(a - b) on the upper, so the upper lane's values
// come out negated.  After stages over the lane bits in `done`, a lane's values carry the sign
// (-1)^popcount(sl & done), the same for all 16 of them (partners of a later stage agree in the
// bits already done); the caller folds that sign into its per-lane scale.
template <int X, int SEG>
__device__ __forceinline__ void cross_stage_signed(float (&v)[16], int sl) {
  static_assert(X <= 2, "quad-lane stages only");
  if constexpr (X < SEG) {
    const float g = (sl & X) ? -1.f : 1.f;
    // v_fmac_f32 with its src0 read from the partner lane (DPP quad permute): the compiler does not
    // fold a DPP move into a multiply-accumulate, so the 16 are written out.  s_nop 1: the DPP read
    // of a VGPR must trail the VALU write of it by two wait states; inside the block no instruction
    // reads a register another one writes.
#define FA_DPP_FMAC(i) "v_fmac_f32_dpp %" #i ", %" #i ", %16 " QP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
#define FA_DPP_BLOCK                                                                                  \
  asm("s_nop 1\n" FA_DPP_FMAC(0) FA_DPP_FMAC(1) FA_DPP_FMAC(2) FA_DPP_FMAC(3) FA_DPP_FMAC(4) FA_DPP_FMAC(5)   \
      FA_DPP_FMAC(6) FA_DPP_FMAC(7) FA_DPP_FMAC(8) FA_DPP_FMAC(9) FA_DPP_FMAC(10) FA_DPP_FMAC(11)          \
      FA_DPP_FMAC(12) FA_DPP_FMAC(13) FA_DPP_FMAC(14) FA_DPP_FMAC(15)                                     \
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),   \
        "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]),         \
        "+v"(v[15])                                                                                    \
      : "v"(g))
    if constexpr (X == 1) {
#define QP "quad_perm:[1,0,3,2]"
      FA_DPP_BLOCK;
#undef QP
    } else {
#define QP "quad_perm:[2,3,0,1]"
      FA_DPP_BLOCK;
#undef QP
    }
#undef FA_DPP_BLOCK
#undef FA_DPP_FMAC
  }
}

// sign (+1 / -1) of a lane's values after hadamard16_signed
template <int SEG>
__device__ __forceinline__ float hadamard_lane_sign(int sl) {
  return (__builtin_popcount(sl & (SEG > 2 ? 3 : SEG - 1)) & 1) ? -1.f : 1.f;
}

template <int X, int SEG>
__device__ __forceinline__ float cross_sum(float a) {
  if constexpr (X < SEG) return a + lane_xor<X>(a);
  return a;
}

// in-place Walsh-Hadamard (Sylvester order) over the d = 16 SEG values of a segment;
// v[CE j + e] is channel 16 sl + CE j + e.  H0 = 2 when the caller has done the stage over
// channel bit 0 itself.  SIGNED: the quad-lane stages leave the lane's values multiplied by
// hadamard_lane_sign<SEG>(sl).
template <int CE, int SEG, int H0 = 1, bool SIGNED = false>
__device__ __forceinline__ void hadamard16(float (&v)[16], int sl) {
  constexpr int NCH = Lay<CE>::NCH;
#pragma unroll
  for (int h = H0; h < CE; h <<= 1)         // channel bits of e
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
  if constexpr (SIGNED) {                    // channel bits of sl
    cross_stage_signed<1, SEG>(v, sl);
    cross_stage_signed<2, SEG>(v, sl);
  } else {
    cross_stage<1, SEG>(v, sl);
    cross_stage<2, SEG>(v, sl);
  }
  cross_stage<4, SEG>(v, sl);
  cross_stage<8, SEG>(v, sl);
#pragma unroll
  for (int hj = 1; hj < NCH; hj <<= 1)      // channel bits of j
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (((i / CE) & hj) == 0) {
        const float a = v[i], b = v[i + CE * hj];
        v[i] = a + b;
        v[i + CE * hj] = a - b;
      }
}

template <int SEG>
__device__ __forceinline__ float segment_sum(float a) {
  a = cross_sum<1, SEG>(a);
  a = cross_sum<2, SEG>(a);
  a = cross_sum<4, SEG>(a);
  return cross_sum<8, SEG>(a);
}

// The per-lane channel factors f[i] = sign(channel of v[i]) * scale.
template <int CE, int SEG>
__device__ __forceinline__ void channel_factors(float (&f)[16], const int8_t* signs, int sl, float scale) {
#pragma unroll
  for (int i = 0; i < 16; ++i) f[i] = signs[16 * sl + i] < 0 ? -scale : scale;
}

// code = the number of thresholds <= u, for an antisymmetric codebook (thresholds t, with
// t[h - 1] = 0 and positive thresholds tp[m] = t[h + m], h = 2^(bits-1)): u >= 0 gives
// h + #{tp <= u}; u < 0 gives (h - 1) - #{tp < |u|}, and #{tp < |u|} is the <= count at the
// float just below |u|.  With m = -1 for u < 0 (0 otherwise) both are (count ^ m) + h.  u must
// not be -0.  The count over the h - 1 positive thresholds is a binary search: 2 steps over 3
// thresholds at 3 bits, 3 steps over 7 at 4 bits.
template <int BITS>
__device__ __forceinline__ unsigned tq_code(float u, const float (&tp)[7]) {
  constexpr int H = 1 << (BITS - 1);
  const int ub = __float_as_int(u);
  const int m = ub >> 31;
  const float x = __int_as_float((ub & 0x7fffffff) + m);
  int cnt;
  if constexpr (BITS == 2) {
    cnt = x >= tp[0] ? 1 : 0;
  } else if constexpr (BITS == 3) {
    const bool c0 = x >= tp[1];
    cnt = (c0 ? 2 : 0) + (x >= (c0 ? tp[2] : tp[0]) ? 1 : 0);
  } else {
    const bool c0 = x >= tp[3];
    const float t1 = c0 ? tp[5] : tp[1];
    const bool c1 = x >= t1;
    const float hi = c1 ? tp[6] : tp[4];
    const float lo = c1 ? tp[2] : tp[0];
    const float t2 = c0 ? hi : lo;
    cnt = (c0 ? 4 : 0) + (c1 ? 2 : 0) + (x >= t2 ? 1 : 0);
  }
  return (unsigned)((cnt ^ m) + H);
}

// The same 4-bit code by table: the sign of u and the float bits of |u| (clamped to [2^-7, 2))
// name one of 128 buckets, eight per binade and sign (index bit 6: the sign; bits 0..5: the
// exponent's low three bits and the top three mantissa bits).  Entry b holds the threshold inside
// bucket b (its float bits, or +inf if none) and the number of thresholds below the whole bucket,
// so the code, the number of thresholds <= u, is base + (u >= thr) with u compared unclamped.
// Valid when every nonzero threshold has 2^-7 <= |t| < 2 and no bucket holds two (checked on the
// host; the search above serves other codebooks).  u must not be -0.
constexpr unsigned kTabLo = 0x3C000000u;   // 2^-7
constexpr unsigned kTabHi = 0x3FFFFFFFu;   // the float below 2
__host__ __device__ inline unsigned tab_bucket_lo(unsigned b) { return ((120u + ((b & 63u) >> 3)) << 23) | ((b & 7u) << 20); }

__device__ __forceinline__ unsigned tq_code4_tab(float u, const u32x2* tab) {
  const unsigned ub = __float_as_uint(u);
  // |u| clamped as a float (one med3 with the absolute value as an input modifier)
  const unsigned cb = __float_as_uint(__builtin_amdgcn_fmed3f(fabsf(u), __uint_as_float(kTabLo), __uint_as_float(kTabHi)));
  const u32x2 e = tab[((ub >> 25) & 64u) | ((cb >> 20) & 63u)];
  return e[1] + (u >= __uint_as_float(e[0]) ? 1u : 0u);
}

// Row groups (RPW rows, one per segment) a wave takes in turn, the channel factors set up once
// per wave: one for encode, four for decode (interleaved timings at the C4 K cache: encode 0.50 ms
// with one group, 0.52-0.53 with 2, 4 or 8; decode 0.32 ms with four, 0.34 with 1, 2 or 8).
constexpr int kTqEncIter = 1;
constexpr int kTqDecIter = 4;

// The NCH 16-byte chunks of row r a lane holds (its 16 NCH contiguous bytes).  (Loading the row
// group as whole 1-KiB runs and handing each lane its chunks through LDS measured the same.)
template <int ROW_BYTES, int SEG, int NCH>
__device__ __forceinline__ void load_chunks(u32x4 (&w)[NCH], const void* x, int64_t r, int sl) {
  const char* p = static_cast<const char*>(x) + r * ROW_BYTES + 16 * NCH * sl;
#pragma unroll
  for (int j = 0; j < NCH; ++j) w[j] = *reinterpret_cast<const u32x4*>(p + 16 * j);
}

template <int D, bool BF16_IN, int BITS, bool TABLE>
__global__ __launch_bounds__(256) void tq_encode_kernel(TqArgs a) {
  constexpr int CE = BF16_IN ? 8 : 4;        // values per 16-byte chunk
  constexpr int NCH = 16 / CE;
  constexpr int SEG = D / 16;                // lanes per vector
  constexpr int RPW = 64 / SEG;
  constexpr int ROW_BYTES = D * (BF16_IN ? 2 : 4);
  const int lane = threadIdx.x & 63;
  const int sl = lane % SEG;
  float f[16];
  channel_factors<CE, SEG>(f, a.signs, sl, 1.0f);
  float tp[7];
#pragma unroll
  for (int k = 0; k < 7; ++k) tp[k] = a.thr[(1 << (BITS - 1)) + (k < (1 << (BITS - 1)) - 1 ? k : 0)];
  __shared__ u32x2 tab[TABLE ? 128 : 1];
  if constexpr (TABLE) {
    if (threadIdx.x < 128) tab[threadIdx.x] = u32x2{a.tab[threadIdx.x][0], a.tab[threadIdx.x][1]};
    __syncthreads();
  }
  const int64_t g0 = ((int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * kTqEncIter;
  // every lane takes part in the butterflies: rows past the end repeat the last row
  u32x4 cur[NCH], nxt[NCH];
  load_chunks<ROW_BYTES, SEG, NCH>(cur, a.x, min(g0 * RPW + lane / SEG, a.n - 1), sl);
#pragma unroll
  for (int it = 0; it < kTqEncIter; ++it) {
    if ((g0 + it) * RPW >= a.n) break;
    const int64_t row = (g0 + it) * RPW + lane / SEG;
    // the next row group's loads go out before this one's arithmetic
    if (it + 1 < kTqEncIter && (g0 + it + 1) * RPW < a.n)
      load_chunks<ROW_BYTES, SEG, NCH>(nxt, a.x, min(row + RPW, a.n - 1), sl);
    float v[16];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (BF16_IN) {
          v[CE * j + 2 * e] = __uint_as_float(cur[j][e] << 16);
          v[CE * j + 2 * e + 1] = __uint_as_float(cur[j][e] & 0xffff0000u);
        } else {
          v[CE * j + e] = __uint_as_float(cur[j][e]);
        }
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ss = __builtin_fmaf(v[i], v[i], ss);
    // the random signs (f = +-1, exact products) fused into the butterflies over channel bit 0:
    // fma(f1, x1, f0 x0) rounds exactly like f0 x0 + f1 x1
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float t = v[i] * f[i], b = v[i + 1];
      v[i] = __builtin_fmaf(f[i + 1], b, t);
      v[i + 1] = __builtin_fmaf(-f[i + 1], b, t);
    }
    const float n = __fsqrt_rn(segment_sum<SEG>(ss));
    hadamard16<CE, SEG, 2, true>(v, sl);
    float yy = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) yy = __builtin_fmaf(v[i], v[i], yy);
    const float ny = __fsqrt_rn(segment_sum<SEG>(yy));
    // 1 / ||y||, carrying the lane's Hadamard sign (exact: a sign flip of the rounded quotient)
    const float inv = (ny > 0.f ? __fdiv_rn(1.0f, ny) : 0.f) * hadamard_lane_sign<SEG>(sl);
    if (row < a.n) {
      // the lane's 16 codes, channel 16 sl + i at bit BITS i of a little-endian word of 16 BITS bits,
      // assembled as two 32-bit halves (codes 0..7 and 8..15 at 4 bits; at 2 and 3 bits the high half
      // holds what passes bit 31)
      unsigned w0 = 0, w1 = 0;
      // fma with +0 rounds like the product and turns a -0 product into +0
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const unsigned code = TABLE ? tq_code4_tab(__builtin_fmaf(v[i], inv, 0.0f), tab)
                                    : tq_code<BITS>(__builtin_fmaf(v[i], inv, 0.0f), tp);
        const int b = BITS * i;
        if (b + BITS <= 32) {
          w0 |= code << b;
        } else if (b >= 32) {
          w1 |= code << (b - 32);
        } else {   // a 3-bit code across bit 32
          w0 |= code << b;
          w1 |= code >> (32 - b);
        }
      }
      const uint64_t packed = (uint64_t)w0 | ((uint64_t)w1 << 32);
      uint8_t* dst = a.codes + row * (D * BITS / 8) + sl * (2 * BITS);
      if constexpr (BITS == 4) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{(unsigned)packed, (unsigned)(packed >> 32)};
      } else if constexpr (BITS == 3) {   // 6 bytes at an even offset
#pragma unroll
        for (int h = 0; h < 3; ++h) reinterpret_cast<unsigned short*>(dst)[h] = (unsigned short)(packed >> (16 * h));
      } else {
        *reinterpret_cast<unsigned*>(dst) = (unsigned)packed;
      }
      if (sl == 0) a.norms[row] = n;
    }
    if (it + 1 < kTqEncIter) {
#pragma unroll
      for (int j = 0; j < NCH; ++j) cur[j] = nxt[j];
    }
  }
}

template <int D, bool BF16_OUT, int BITS>
__global__ __launch_bounds__(256) void tq_decode_kernel(TqArgs a) {
  constexpr int CE = 4;                       // fp32 values per chunk of the layout
  constexpr int SEG = D / 16;
  constexpr int RPW = 64 / SEG;
  constexpr int NST = BF16_OUT ? 2 : 4;       // 16-byte output chunks per lane and row group
  __shared__ float cb[16];
  __shared__ u32x4 slot[4][64 * NST];         // per wave: one row group's output
  if (threadIdx.x < 16) cb[threadIdx.x] = a.cb[threadIdx.x];
  const int lane = threadIdx.x & 63;
  const int sl = lane % SEG;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g0 = ((int64_t)blockIdx.x * 4 + wv) * kTqDecIter;
  // all row groups' codes (the lane's contiguous 16) and norms are loaded up front (rows past the
  // end repeat the last row)
  uint64_t pk[kTqDecIter];   // the lane's 16 codes, channel 16 sl + i at bit BITS i
  float nn[kTqDecIter];
#pragma unroll
  for (int it = 0; it < kTqDecIter; ++it) {
    const int64_t r = min((g0 + it) * RPW + lane / SEG, a.n - 1);
    nn[it] = a.norms[r];
    const uint8_t* src = a.codes + r * (D * BITS / 8) + sl * (2 * BITS);
    if constexpr (BITS == 4) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(src);
      pk[it] = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
    } else if constexpr (BITS == 3) {
      const unsigned short* s16 = reinterpret_cast<const unsigned short*>(src);
      pk[it] = (uint64_t)s16[0] | ((uint64_t)s16[1] << 16) | ((uint64_t)s16[2] << 32);
    } else {
      pk[it] = *reinterpret_cast<const unsigned*>(src);
    }
  }
  float f[16];   // sign * 1/sqrt(d), times the lane's Hadamard sign
  channel_factors<CE, SEG>(f, a.signs, sl, a.inv_sqrt_d * hadamard_lane_sign<SEG>(sl));
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kTqDecIter; ++it) {
    if ((g0 + it) * RPW >= a.n) break;
    float v[16];
    // rounded on its own: an fma with the first butterfly's add would round differently
#pragma unroll
    for (int i = 0; i < 16; ++i)
      v[i] = mul_rn(nn[it], cb[(unsigned)(pk[it] >> (BITS * i)) & ((1u << BITS) - 1)]);
    hadamard16<CE, SEG, 1, true>(v, sl);
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = v[i] * f[i];
    // The group's RPW rows are one contiguous run of NST 16-byte chunks per lane (2 KiB of bf16,
    // 4 KiB of fp32).  A lane's own chunks sit NST apart, so storing them directly would make
    // every store instruction write every NST-th chunk of the run; they go through the wave's LDS
    // slot instead, and store k of lane l writes chunk 64 k + l: each store covers 1 KiB whole.
    u32x4 w[NST];
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      if constexpr (BF16_OUT)
        w[j] = u32x4{pack_bf16x2(y[8 * j], y[8 * j + 1]), pack_bf16x2(y[8 * j + 2], y[8 * j + 3]),
                     pack_bf16x2(y[8 * j + 4], y[8 * j + 5]), pack_bf16x2(y[8 * j + 6], y[8 * j + 7])};
      else
        w[j] = u32x4{__float_as_uint(y[4 * j]), __float_as_uint(y[4 * j + 1]), __float_as_uint(y[4 * j + 2]),
                     __float_as_uint(y[4 * j + 3])};
    }
    wave_lds_order();
#pragma unroll
    for (int j = 0; j < NST; ++j) slot[wv][NST * lane + j] = w[j];
    wave_lds_order();
#pragma unroll
    for (int k = 0; k < NST; ++k) w[k] = slot[wv][64 * k + lane];
    wave_lds_order();
    const int64_t row0 = (g0 + it) * RPW;
    char* dst = static_cast<char*>(a.out) + row0 * D * (BF16_OUT ? 2 : 4);
#pragma unroll
    for (int k = 0; k < NST; ++k) {
      const int chunk = 64 * k + lane;
      if (row0 + chunk / (NST * SEG) < a.n) *reinterpret_cast<u32x4*>(dst + 16 * chunk) = w[k];
    }
  }
}

// The 4-bit decision table (host): true and a.tab filled when every nonzero threshold has
// 2^-7 <= |t| < 2 and no (sign, bucket) holds two.
inline bool tq_table_build(TqArgs& a) {
  int seen[128] = {0};
  for (int k = 0; k < 15; ++k) {
    unsigned tb;
    std::memcpy(&tb, &a.thr[k], 4);
    const unsigned ab = tb & 0x7fffffffu;
    if (ab == 0u) continue;
    if (ab < kTabLo || ab > kTabHi) return false;
    if (seen[((tb >> 25) & 64u) | ((ab >> 20) & 63u)]++) return false;
  }
  for (unsigned t = 0; t < 128; ++t) {
    const bool neg = t >= 64u;
    const unsigned lo = tab_bucket_lo(t), hi = lo + (1u << 20);
    unsigned base = 0, tbits = 0x7f800000u;   // +inf: no threshold inside the bucket
    for (int k = 0; k < 15; ++k) {
      const float x = a.thr[k];
      unsigned xb;
      std::memcpy(&xb, &x, 4);
      const unsigned ab = xb & 0x7fffffffu;
      if (ab != 0u && (x < 0.f) == neg && ab >= lo && ab < hi) {
        tbits = xb;                            // compared against u
      } else if (neg ? (x < 0.f && ab >= hi) : (x <= 0.f || ab < lo)) {
        ++base;                                // at or below every u of the bucket
      }
    }
    a.tab[t][0] = tbits;
    a.tab[t][1] = base;
  }
  return true;
}

template <int D, int BITS>
hipError_t launch_encode_d(const TqArgs& a_in, bool bf16, hipStream_t st, const char** name) {
  TqArgs a = a_in;
  const int64_t rows_per_block = 4 * (64 / (D / 16)) * kTqEncIter;
  const int64_t blocks = (a.n + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(256);
  if (BITS == 4 && tq_table_build(a)) {
    if (bf16) hipLaunchKernelGGL((tq_encode_kernel<D, true, BITS, BITS == 4>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((tq_encode_kernel<D, false, BITS, BITS == 4>), grid, block, 0, st, a);
    *name = "tq_encode";
  } else {
    if (bf16) hipLaunchKernelGGL((tq_encode_kernel<D, true, BITS, false>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((tq_encode_kernel<D, false, BITS, false>), grid, block, 0, st, a);
    *name = BITS == 4 ? "tq_encode_search" : "tq_encode";
  }
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t launch_decode_d(const TqArgs& a, bool bf16_out, hipStream_t st, const char** name) {
  const int64_t rows_per_block = 4 * (64 / (D / 16)) * kTqDecIter;
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
  if (bits == 4) return encode_bits<4>(a, d, bf16, st, name);
  if (bits == 3) return encode_bits<3>(a, d, bf16, st, name);
  return encode_bits<2>(a, d, bf16, st, name);
}

hipError_t launch_tq_decode(const TqArgs& a, int32_t d, int32_t bits, bool bf16_out, hipStream_t st,
                            const char** name) {
  if (bits == 4) return decode_bits<4>(a, d, bf16_out, st, name);
  if (bits == 3) return decode_bits<3>(a, d, bf16_out, st, name);
  return decode_bits<2>(a, d, bf16_out, st, name);
}

}  // namespace fa
