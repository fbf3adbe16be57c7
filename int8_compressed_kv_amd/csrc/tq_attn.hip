// Split-KV decode attention read straight from a TurboQuant-coded KV cache: the codes are turned
// into MFMA operands in registers and the decoded cache never exists in global memory (Foundry
// attention/ README, section "TurboQuant KV Cache Compression": K and V stored as randomized
// Hadamard-rotated, L2-normalised Lloyd-Max codes; fkl.flash_attention PR, Summary: the
// compressed cache is dequantized inside q.k and p.v).
//
// With K^_j = s_K * H (n_j c_K[code_j]) / sqrt(d) (H the symmetric Sylvester Hadamard matrix,
// s_K the K signs), q . K^_j = n_j (H (s_K * q)) . c_K[code_j] / sqrt(d): q is rotated once per
// head (q' = H (s_K * q)) and every score is a dot product of q' with codebook entries.  With
// V^_j = s_V * H (n_j c_V[code_j]) / sqrt(d), sum_j p_j V^_j = s_V * H (sum_j p_j n_j c_V[code_j]) /
// sqrt(d): P.V is accumulated in the rotated domain and rotated back once per head, after the
// splits are merged.
//
// Both products run on the int8 MFMA (v_mfma_i32_16x16x64_i8) in the digit form of the int8
// decode:
//   * codebook entries as three signed 7-bit digits of c 2^-E, looked up per byte with v_perm_b32
//     from 16-byte digit tables (4 entries for 2-bit codes and 8 for 3-bit codes: one permute;
//     16 entries for 4-bit codes: two permutes and a byte select);
//   * 3-bit codes, which straddle bytes in the packed stream, are first widened in registers to
//     the 4-bit layout (each 24-bit run of 8 codes becomes one 32-bit word of nibbles), so both
//     products then read them exactly as 4-bit codes whose values stay below 8;
//   * q' as four signed 7-bit digits under a per-head power of two (B of S = K q'), and
//     P~_j = p_j n^V_j as four unsigned 7-bit digits of P~ / 2^F rounded at 28 bits (B of
//     O' += V^T P~), one MFMA column per (digit, head) for 4 heads;
//   * one accumulator per codebook digit; the digit columns are recombined in fp32.
// Sums of digit products are exact integers; what is rounded is the codebook (to 21 fractional
// bits of 2^E), q' and P~ (to 28 bits of their scale) and the fp32 recombination.
//
// Pass 1 (tq_attn_partial_kernel), one block per (split, bh_kv, group of 4 query heads), the
// ceil(G/4) head groups of one key range on one XCD: 4 waves stream 64-key tiles
// of one KV head (K codes straight into the MFMA operand layout, V codes through a wave-private
// LDS slot for the transposing byte reads) and leave (m, l, O') per (query head, split).
// Pass 2 (tq_attn_merge_kernel): per query head, the log-sum-exp merge of the splits, 1/l, the
// inverse rotation O = s_V * H O' / sqrt(d), the epilogue and the store.
#include "device_common.hpp"

namespace fa {
namespace {

constexpr float kTqLazyLog2 = 8.0f;
constexpr int kTqWaves = 4;
constexpr int kTqFlushTiles = 1024;   // P~V accumulators: 1024 tiles x 64 keys x 127 x 64 < 2^31
constexpr int kTqBufferFlags = 0x00020000;
constexpr int kTqNt = 2;   // nontemporal cache policy of a buffer access

template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

typedef int i32x2t __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) i32x2t lds_i32x2t;
typedef __attribute__((address_space(3))) unsigned char lds_u8t;

// In-place unnormalised Walsh-Hadamard transform of `rows` contiguous LDS vectors of length D
// (Sylvester order: y_r = sum_j (-1)^popcount(r & j) x_j), by threads t = 0 .. n-1 of the block:
// log2(D) butterfly stages (a, b) -> (a + b, a - b) over index bit h, one pair per thread and
// step, a barrier after each stage (the last one included, so x is ready on return).
template <int D>
__device__ __forceinline__ void lds_hadamard(float* x, int rows, int t, int n) {
  static_assert((D & (D - 1)) == 0, "Hadamard length is a power of two");
#pragma unroll
  for (int h = 1; h < D; h <<= 1) {
    for (int p = t; p < rows * (D / 2); p += n) {
      const int k = p % (D / 2);
      const int lo = (p / (D / 2)) * D + (k / h) * 2 * h + k % h;
      const float u = x[lo], w = x[lo + h];
      x[lo] = u + w;
      x[lo + h] = u - w;
    }
    __syncthreads();
  }
}

// Byte lookups of four code bytes (one code per byte, values below 2^BITS) in a digit table.
template <int BITS>
__device__ __forceinline__ unsigned lookup4(unsigned sel, const uint32_t (&tab)[4]) {
  if constexpr (BITS == 2) {
    return __builtin_amdgcn_perm(tab[0], tab[0], sel);                 // selectors 0..3: entries 0..3
  } else if constexpr (BITS == 3) {
    return __builtin_amdgcn_perm(tab[1], tab[0], sel);                 // selectors 0..7: entries 0..7
  } else {
    const unsigned s7 = sel & 0x07070707u;
    const unsigned lo = __builtin_amdgcn_perm(tab[1], tab[0], s7);     // entries 0..7
    const unsigned hi = __builtin_amdgcn_perm(tab[3], tab[2], s7);     // entries 8..15
    const unsigned pick = ((sel >> 1) & 0x04040404u) | 0x03020100u;    // byte i: i (lo) or 4 + i (hi)
    return __builtin_amdgcn_perm(hi, lo, pick);
  }
}

// The 8 three-bit fields in bits 0..23 of x (field k at bits 3k .. 3k + 2; bits 24..31 are
// ignored) as the 8 nibbles of a word (field k at bits 4k .. 4k + 2, bit 4k + 3 clear): three
// shift-and-merge steps, each moving half of the fields of every group by one more place.
__device__ __forceinline__ unsigned widen3to4(unsigned x) {
  const unsigned y = (x & 0x0000ffffu) | ((x << 4) & 0xffff0000u);     // fields 4..7 to bit 16
  const unsigned y2 = (y & 0x003f003fu) | ((y << 2) & 0xffc0ffc0u);    // fields 2, 3 (6, 7) up by 2
  const unsigned z = (y2 & 0x0f0f0f0fu) | ((y2 << 1) & 0xf0f0f0f0u);   // fields 1, 3, 5, 7 up by 1
  return z & 0x77777777u;
}

template <int D, int KBITS, int VBITS>
struct TqCfg {
  static constexpr int KT = 64;                       // keys per tile
  static constexpr int KG = 16;                       // keys per lane group
  static constexpr int NKB = KT / 16;                 // 16-key row blocks of S
  static constexpr int NKK = D / 64;                  // 64-deep k-steps of S
  static constexpr int LK = KBITS == 3 ? 4 : KBITS;   // code width of the register layout
  static constexpr int LV = VBITS == 3 ? 4 : VBITS;   // ... and of the LDS layout (3 bits widened)
  static constexpr int RKS = D * KBITS / 8;           // K code bytes per key in memory
  static constexpr int RVS = D * VBITS / 8;           // V code bytes per key in memory
  static constexpr int RK = D * LK / 8;               // K code bytes per key, register layout
  static constexpr int QBK = RK / 4;                  // ... per lane group and key
  static constexpr int KW = QBK / 4;                  // ... as 32-bit words
  static constexpr int QBK3 = 3 * D / 32;             // 3-bit K: bytes per lane group and key
  static constexpr int NW3 = D == 64 ? 2 : QBK3 / 4;  // 3-bit K: words loaded per row block
  static constexpr int NV3 = RVS / 4;                 // 3-bit V: words of one key row
  static constexpr int RV = D * LV / 8;               // V code bytes per key, LDS layout
  static constexpr int NC16V = RV / 16;               // 16-byte chunks per V row
  static constexpr int VCH = KT * NC16V / 64;         // 16-byte V loads per lane per tile
  static constexpr int FV = 8 / LV;                   // codes per V byte (LDS layout)
  static constexpr int NBLK = NC16V * FV;             // 16-channel blocks of O' (= D / 16)
  static constexpr int SP = NC16V >= 8 ? 8 : NC16V >= 4 ? 4 : NC16V >= 2 ? 2 : 1;   // LDS swizzle span
  static constexpr int SLOT = KT * RV + 8 * KT;       // wave-private LDS bytes (V tile, norms)
  static_assert(NBLK == D / 16, "block count");
  static_assert(QBK % 4 == 0 && NC16V >= 1, "layout");
  static_assert((D == 64 || D == 128) && (QBK3 % 4 == 0 || D == 64), "3-bit row pieces");
};

template <int SP>
__device__ __forceinline__ int tswz(int r) {
  return ((r >> 1) ^ (r >> 4)) & (SP - 1);
}

// Channel of k-slot s (0..15) of lane group hq in k-step kk: the lane's A bytes come from its
// code words in the order the lookups produce them (4-bit: low nibbles then high nibbles of each
// word; 2-bit: field 0 of the four bytes, then field 1, ...).
template <int D, int KBITS>
__device__ __forceinline__ int k_slot_channel(int kk, int hq, int s) {
  const int base = hq * (D / 4) + 16 * kk;
  const int w = s >> 2, e = s & 3;
  if constexpr (KBITS >= 3) return base + 8 * (w >> 1) + 2 * e + (w & 1);   // 3 bits: widened to 4
  else return base + 4 * e + w;
}

template <int D, int KBITS, int VBITS, bool SOPS>
__global__ __launch_bounds__(64 * kTqWaves, (D == 128 && KBITS == 4 && VBITS >= 3) ? 1 : 2)   // 4/4 needs > 256 VGPRs
void tq_attn_partial_kernel(TqAttnArgs a) {
  using C = TqCfg<D, KBITS, VBITS>;
  constexpr int KT = C::KT, KG = C::KG, NKB = C::NKB, NKK = C::NKK, RK = C::RK, QBK = C::QBK, KW = C::KW;
  constexpr int RV = C::RV, NC16V = C::NC16V, VCH = C::VCH, FV = C::FV, NBLK = C::NBLK, SP = C::SP;
  constexpr int RKS = C::RKS, RVS = C::RVS, QBK3 = C::QBK3, NW3 = C::NW3, NV3 = C::NV3;
  constexpr bool K3 = KBITS == 3, V3 = VBITS == 3;
  constexpr int HPW = 4;

  __shared__ __attribute__((aligned(16))) unsigned char lds_slot[kTqWaves][C::SLOT];
  __shared__ float lds_q[HPW][D];        // s_K * q, then q' = H (s_K * q)
  __shared__ float lds_m[kTqWaves][HPW];
  __shared__ float lds_l[kTqWaves][HPW];
  __shared__ float lds_o[kTqWaves][HPW][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int hq = lane >> 4;
  const int t_dig = n >> 2;
  const int gq = n & 3;

  // block -> (split, KV head, group of 4 query heads).  The Z = ceil(G/4) slices of one (split, KV
  // head) stream the same codes; they are dealt 8 blocks apart, so they land on one XCD (blocks go
  // to the 8 XCDs in turn) at about the same time and the repeated reads can hit its L2.
  const int Z = (a.group + HPW - 1) / HPW;
  const int64_t n_chunk = (int64_t)a.num_splits * a.bh_kv;
  const int64_t full = (n_chunk / 8) * 8 * Z;
  const int64_t bid = blockIdx.x;
  int64_t chunk;
  int zs;
  if (bid < full) {
    const int64_t j = bid / 8;
    chunk = 8 * (j / Z) + bid % 8;
    zs = (int)(j % Z);
  } else {
    chunk = (n_chunk / 8) * 8 + (bid - full) / Z;
    zs = (int)((bid - full) % Z);
  }
  const int split = (int)(chunk % a.num_splits);
  const int kvh = (int)(chunk / a.num_splits);
  const int zh = zs * HPW;
  const int nh = min(HPW, a.group - zh);
  const int64_t kv_base = (int64_t)kvh * a.s_k;
  const int head0 = kvh * a.group + zh;

  // ---- q' = H (s_K * q) for the workgroup's heads (absent heads are zero)
  for (int i = tid; i < HPW * D; i += 64 * kTqWaves) {
    const int g = i / D, j = i % D;
    float x = 0.f;
    if (g < nh) {
      const int64_t at = (int64_t)(head0 + g) * D + j;
      x = a.q_bf16 ? bf16_bits_to_f32(static_cast<const unsigned short*>(a.q)[at]) : static_cast<const float*>(a.q)[at];
      x = a.ks[j] < 0 ? -x : x;
    }
    lds_q[g][j] = x;
  }
  __syncthreads();
  lds_hadamard<D>(&lds_q[0][0], HPW, tid, 64 * kTqWaves);

  // ---- q' digit B operands (column n = (t_dig, gq), k-slots in the K lookup order)
  i32x4 qdig[NKK];
  float s_comb;   // 2^(E_q + E_k - 7 (t + 1) - 7) / sqrt(d) for this lane's digit column
  {
    float qv[NKK][16];
    float mx = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        qv[kk][s] = lds_q[gq][k_slot_channel<D, KBITS>(kk, hq, s)];
        mx = fmaxf(mx, fabsf(qv[kk][s]));
      }
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    int E = 0;
    if (mx > 0.f) {
      (void)frexpf(mx, &E);
      E += 1;
    }
    s_comb = ldexpf(1.0f / sqrtf((float)D), E + a.k_e - 7 * (t_dig + 1) - 7);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      unsigned w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        float x = ldexpf(qv[kk][s], -E) * 128.f;
        float dd[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          dd[t] = __builtin_rintf(x);
          x = (x - dd[t]) * 128.f;
        }
        const int dig = (int)(t_dig == 0 ? dd[0] : t_dig == 1 ? dd[1] : t_dig == 2 ? dd[2] : dd[3]);
        w[s / 4] |= ((unsigned)dig & 0xffu) << (8 * (s % 4));
      }
      qdig[kk] = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
  }

  uint32_t ktab[3][4], vtab[3][4];
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ktab[t][e] = a.ktab[t][e];
      vtab[t][e] = a.vtab[t][e];
    }

  // ---- tiles of this split; wave w takes tiles w, w + 4, ...
  const int n_tiles_total = (a.s_k - a.key_lo + KT - 1) / KT;
  const int ts = split * a.tiles_per_split;
  const int te = min(n_tiles_total, ts + a.tiles_per_split);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int n_w = te > ts + wave_u ? (te - ts - wave_u + kTqWaves - 1) / kTqWaves : 0;
  const int last_key = a.s_k - 1;

  // K: row block kb, lane n is key KG (n/4) + 4 kb + n%4 (so the score accumulator's lane group
  // hq owns keys KG hq .. KG hq + KG - 1, the keys the transposing V reads give it); the lane
  // loads its group's QBK bytes of that row.  V: 16-byte chunk F = 64 u + lane of the tile's
  // contiguous rows.  Norms: entry 64 e + lane of [K norms | V norms].
  // 3-bit codes: K rows as the lane group's packed words (widened in compute), V rows one key per
  // lane as packed words (widened into the LDS slot in compute).
  struct Tile {
    uint32_t k[NKB][K3 ? NW3 : KW];
    u32x4 v[V3 ? 1 : VCH];
    uint32_t v3[V3 ? NV3 : 1];
    float nrm[2];
  };
  int krow[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) krow[kb] = KG * (n >> 2) + 4 * kb + (n & 3);
  // Raw buffer loads: the resource is the wave-uniform tile base with the bytes left in the head
  // as its bound and the per-lane offsets are loop-invariant, so a load costs no vector
  // instruction; rows past the last key read zeros and are masked in compute.
  // 3-bit K: the lane group's QBK3 bytes start at byte hq QBK3 of the row, which is 4-byte aligned
  // except at head_dim 64 (6 bytes per group): there the load starts at the aligned word below and
  // the run is shifted down by sh3 bits (the last group's load still ends at the row's end).
  unsigned koff[NKB];
  const unsigned sh3 = K3 ? (unsigned)((hq * QBK3) & 3) * 8u : 0u;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
    koff[kb] = K3 ? (unsigned)(krow[kb] * RKS + ((hq * QBK3) & ~3)) : (unsigned)(krow[kb] * RK + hq * QBK);
  auto load = [&](int idx, Tile& T) {
    const int k0 = a.key_lo + (ts + wave_u + kTqWaves * idx) * KT;
    const int64_t left = a.s_k - k0;             // >= 1: loads never start past the last key
    const auto rsrc = [&](const void* base, int64_t bytes) {
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)min(bytes, (int64_t)0x7fffffff),
                                               kTqBufferFlags);
    };
    const __amdgpu_buffer_rsrc_t rk = rsrc(a.kc + (kv_base + k0) * RKS, left * RKS);
    const __amdgpu_buffer_rsrc_t rv = rsrc(a.vc + (kv_base + k0) * RVS, left * RVS);
    const __amdgpu_buffer_rsrc_t rkn = rsrc(a.kn + kv_base + k0, left * 4);
    const __amdgpu_buffer_rsrc_t rvn = rsrc(a.vn + kv_base + k0, left * 4);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if constexpr (K3 && NW3 == 3) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b96(rk, koff[kb], 0, kTqNt);
        T.k[kb][0] = (uint32_t)x[0];
        T.k[kb][1] = (uint32_t)x[1];
        T.k[kb][2] = (uint32_t)x[2];
      } else if constexpr (K3) {
        static_assert(NW3 == 2, "3-bit K run");
        const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk, koff[kb], 0, kTqNt));
        T.k[kb][0] = x[0];
        T.k[kb][1] = x[1];
      } else if constexpr (KW % 4 == 0) {
#pragma unroll
        for (int w4 = 0; w4 < KW / 4; ++w4) {
          const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff[kb] + 16 * w4, 0, kTqNt));
#pragma unroll
          for (int e = 0; e < 4; ++e) T.k[kb][4 * w4 + e] = x[e];
        }
      } else if constexpr (KW == 2) {
        const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk, koff[kb], 0, kTqNt));
        T.k[kb][0] = x[0];
        T.k[kb][1] = x[1];
      } else {
        T.k[kb][0] = __builtin_amdgcn_raw_buffer_load_b32(rk, koff[kb], 0, kTqNt);
      }
    }
    if constexpr (V3 && RVS % 16 == 0) {
#pragma unroll
      for (int u = 0; u < RVS / 16; ++u) {
        const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, RVS * lane + 16 * u, 0, kTqNt));
#pragma unroll
        for (int e = 0; e < 4; ++e) T.v3[4 * u + e] = x[e];
      }
    } else if constexpr (V3) {
#pragma unroll
      for (int u = 0; u < RVS / 8; ++u) {
        const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, RVS * lane + 8 * u, 0, kTqNt));
        T.v3[2 * u] = x[0];
        T.v3[2 * u + 1] = x[1];
      }
    } else {
#pragma unroll
      for (int u = 0; u < VCH; ++u)
        T.v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, 16u * (64 * u + lane), 0, kTqNt));
    }
    T.nrm[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rkn, 4u * lane, 0, kTqNt));
    T.nrm[1] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rvn, 4u * lane, 0, kTqNt));
  };
  unsigned char* slot = &lds_slot[wave][0];

  // O' = Of + sum_t Oi[t] 2^(F + E_v - 7 (t_q + 1) - 7 (t + 1)): Oi exact int32 sums since the last
  // flush (one per codebook digit t), Of the fp32 total before it.
  float Of[NBLK][4];
  i32x4 Oi[NBLK][3];
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
#pragma unroll
    for (int t = 0; t < 3; ++t) Oi[b][t] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int v = 0; v < 4; ++v) Of[b][v] = 0.f;
  }
  float m_run = neg_inf(), l_run = 0.f, mc = 0.f;
  int F = -1000;
  int since_flush = 0;
  const float c2 = a.scale_log2;
  const float lazy_thr = kTqLazyLog2 / c2;
  auto flush = [&]() {
    const int ex = F + a.v_e - 7 * (t_dig + 1) - 7;
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float y = __builtin_fmaf((float)Oi[b][2][v], 1.0f / 128.f, (float)Oi[b][1][v]);
        y = __builtin_fmaf(y, 1.0f / 128.f, (float)Oi[b][0][v]);
        Of[b][v] += ldexpf(y, ex);
      }
#pragma unroll
      for (int t = 0; t < 3; ++t) Oi[b][t] = i32x4{0, 0, 0, 0};
    }
    since_flush = 0;
  };

  auto compute = [&](int idx, bool valid, const Tile& T) {
    const int k0 = a.key_lo + (ts + wave_u + kTqWaves * idx) * KT;
    // V codes and the norms into the wave's LDS slot, after the previous tile's reads of it and
    // before this tile's
    wave_lds_order();
    if constexpr (V3) {
      // lane = key row: every 3 packed words hold 4 runs of 8 codes, each widened to a word of
      // nibbles, so the slot row is the row's 4-bit layout
#pragma unroll
      for (int j = 0; j < NC16V; ++j) {
        const unsigned a0 = T.v3[3 * j], a1 = T.v3[3 * j + 1], a2 = T.v3[3 * j + 2];
        const u32x4 w = {widen3to4(a0), widen3to4(__builtin_amdgcn_alignbit(a1, a0, 24)),
                         widen3to4(__builtin_amdgcn_alignbit(a2, a1, 16)), widen3to4(a2 >> 8)};
        *reinterpret_cast<u32x4*>(slot + lane * RV + 16 * (j ^ tswz<SP>(lane))) = w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < VCH; ++u) {
        const int Fc = 64 * u + lane;
        const int r = Fc / NC16V;
        *reinterpret_cast<u32x4*>(slot + r * RV + 16 * ((Fc % NC16V) ^ tswz<SP>(r))) = T.v[u];
      }
    }
    reinterpret_cast<float*>(slot + KT * RV)[lane] = T.nrm[0];
    reinterpret_cast<float*>(slot + KT * RV)[64 + lane] = T.nrm[1];
    wave_lds_order();
    const float* snk = reinterpret_cast<const float*>(slot + KT * RV);
    const float* snv = snk + KT;
    const bool tail = !valid || k0 + KT > a.s_k;
    const int key_lim = valid ? last_key - k0 - KG * hq : -1;

    // S: per row block, one accumulator per codebook digit, the k-steps accumulated in it
    float s[NKB][4];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      i32x4 acc[3] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
      // the row block's code words in the 4-bit register layout (3-bit runs widened)
      uint32_t kw[KW];
      if constexpr (K3 && NW3 == 3) {
        const unsigned a0 = T.k[kb][0], a1 = T.k[kb][1], a2 = T.k[kb][2];
        kw[0] = widen3to4(a0);
        kw[1] = widen3to4(__builtin_amdgcn_alignbit(a1, a0, 24));
        kw[2] = widen3to4(__builtin_amdgcn_alignbit(a2, a1, 16));
        kw[3] = widen3to4(a2 >> 8);
      } else if constexpr (K3) {
        const uint64_t x = ((((uint64_t)T.k[kb][1]) << 32) | T.k[kb][0]) >> sh3;
        kw[0] = widen3to4((unsigned)x);
        kw[1] = widen3to4((unsigned)(x >> 24));
      } else {
#pragma unroll
        for (int w = 0; w < KW; ++w) kw[w] = T.k[kb][w];
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        unsigned sel[4];
        if constexpr (KBITS >= 3) {
          const unsigned w0 = kw[2 * kk], w1 = kw[2 * kk + 1];
          sel[0] = w0 & 0x0f0f0f0fu;
          sel[1] = (w0 >> 4) & 0x0f0f0f0fu;
          sel[2] = w1 & 0x0f0f0f0fu;
          sel[3] = (w1 >> 4) & 0x0f0f0f0fu;
        } else {
          const unsigned w = kw[kk];
#pragma unroll
          for (int c = 0; c < 4; ++c) sel[c] = (w >> (2 * c)) & 0x03030303u;
        }
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          const i32x4 av = {(int)lookup4<KBITS>(sel[0], ktab[t]), (int)lookup4<KBITS>(sel[1], ktab[t]),
                            (int)lookup4<KBITS>(sel[2], ktab[t]), (int)lookup4<KBITS>(sel[3], ktab[t])};
          acc[t] = mfma16_i8(av, qdig[kk], acc[t]);
        }
      }
      const f32x4 kn = *reinterpret_cast<const f32x4*>(snk + KG * hq + 4 * kb);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
#pragma clang fp contract(off)
        // digits 1 and 2 joined exactly in int32 (|acc| < 2^20); the multiply stays apart from
        // the add, which then takes the DPP operand
        float y = __builtin_fmaf((float)(acc[1][v] * 128 + acc[2][v]), 1.0f / 16384.f, (float)acc[0][v]);
        y *= s_comb;
        y = y + row_ror<8>(y);
        y = y + row_ror<4>(y);
        s[kb][v] = y * kn[v];
      }
    }
    if constexpr (SOPS) {
      float x[NKB * 4];
#pragma unroll
      for (int j = 0; j < NKB * 4; ++j) x[j] = s[j / 4][j % 4];
      apply_score_ops(x, a.sops, [&](int j) { return min(k0 + KG * hq + j, last_key); });
#pragma unroll
      for (int j = 0; j < NKB * 4; ++j) s[j / 4][j % 4] = x[j];
    }
    if (tail) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (4 * kb + v > key_lim) s[kb][v] = neg_inf();
    }
    float mx = neg_inf();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[kb][v]);
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    const bool raised = __any(mx - m_run > lazy_thr);
    if (raised) {
      flush();
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < NBLK; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) Of[b][v] *= alpha;
      m_run = m_new;
      mc = m_use * c2;
    }
    float pt[NKB][4];
    float ps = 0.f, pmax = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const f32x4 vn = *reinterpret_cast<const f32x4*>(snv + KG * hq + 4 * kb);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][v], c2, -mc));
        ps += p;
        pt[kb][v] = p * vn[v];
        pmax = fmaxf(pmax, pt[kb][v]);
      }
    }
    l_run += ps;
    pmax = max_xor16(pmax);
    pmax = max_xor32(pmax);
    int Fp = -1000;
    if (pmax > 0.f) (void)frexpf(pmax, &Fp);
    const bool grow = __any(Fp > F) || since_flush >= kTqFlushTiles;
    if (grow && !raised) flush();
    if (raised || grow) F = Fp + 1;
    ++since_flush;
    // digit t_q of x = P~ / 2^F in [0, 1): bits 21 - 7 t_q .. 27 - 7 t_q of floor(x 2^28 + 1/2),
    // one fp32 multiply-add (exact while x 2^28 < 2^23; above, x 2^28 is an integer that the add
    // may raise by one); k-slot 4 kb + v of lane group hq is key KG hq + 4 kb + v
    const int sh = 21 - 7 * t_dig;
    const float sc = ldexpf(1.f, 28 - F);
    unsigned pw[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      unsigned w = 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const unsigned qx = (unsigned)__builtin_fmaf(pt[kb][v], sc, 0.5f);
        w |= __builtin_amdgcn_ubfe(qx, sh, 7) << (8 * v);
      }
      pw[kb] = w;
    }
    const i32x4 pdig = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]};

    // O'^T: byte column 16 b + n of the V rows holds codes FV (16 b + n) + c; the transposing
    // reads give lane n those bytes for keys KG hq .. KG hq + 15.
#pragma unroll
    for (int b = 0; b < NC16V; ++b) {
      int w4[4];
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int vrow = KG * hq + 8 * h8 + (n >> 1);
        const int off = vrow * RV + 16 * (b ^ tswz<SP>(vrow)) + 8 * (n & 1);
        const i32x2t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2t*)((lds_u8t*)slot + off));
        w4[2 * h8] = r[0];
        w4[2 * h8 + 1] = r[1];
      }
#pragma unroll
      for (int c = 0; c < FV; ++c) {
        unsigned sel[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) sel[e] = ((unsigned)w4[e] >> (C::LV * c)) & (C::LV == 4 ? 0x0f0f0f0fu : 0x03030303u);
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          const i32x4 av = {(int)lookup4<VBITS>(sel[0], vtab[t]), (int)lookup4<VBITS>(sel[1], vtab[t]),
                            (int)lookup4<VBITS>(sel[2], vtab[t]), (int)lookup4<VBITS>(sel[3], vtab[t])};
          Oi[b * FV + c][t] = mfma16_i8(av, pdig, Oi[b * FV + c][t]);
        }
      }
    }
  };

  // one tile in flight while the current one is computed; the loads past the end repeat the
  // last tile
  if (n_w > 0) {
    Tile cur, nxt;
    load(0, cur);
    for (int idx = 0; idx < n_w; ++idx) {
      load(min(idx + 1, n_w - 1), nxt);
      compute(idx, true, cur);
      cur = nxt;
    }
  }

  // ---- combine digit columns and lane groups, then the waves through LDS.  Block b * FV + c,
  // row 4 hq + v is channel FV (16 b + 4 hq + v) + c.
  flush();
  float lt = l_run;
  lt = add_xor16(lt);
  lt = add_xor32(lt);
  if (lane == gq) {
    lds_m[wave][gq] = m_run;
    lds_l[wave][gq] = lt;
  }
#pragma unroll
  for (int b = 0; b < NC16V; ++b)
#pragma unroll
    for (int c = 0; c < FV; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float y = Of[b * FV + c][v];
        y = y + row_ror<8>(y);
        y = y + row_ror<4>(y);
        if (t_dig == 0) lds_o[wave][gq][FV * (16 * b + 4 * hq + v) + c] = y;
      }
  __syncthreads();

  for (int idx = tid; idx < nh * (D + 2); idx += 64 * kTqWaves) {
    const int hz = idx / (D + 2), col = idx % (D + 2);
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < kTqWaves; ++w) M = fmaxf(M, lds_m[w][hz]);
    float acc = 0.f;
    if (col == 0) {
      acc = M;
    } else if (M != neg_inf()) {
#pragma unroll
      for (int w = 0; w < kTqWaves; ++w) {
        const float wt = __builtin_amdgcn_exp2f((lds_m[w][hz] - M) * c2);
        acc += wt * (col == 1 ? lds_l[w][hz] : lds_o[w][hz][col - 2]);
      }
    }
    const int64_t head = head0 + hz;
    a.partial[(head * a.num_splits + split) * (D + 2) + col] = acc;
  }
}

constexpr int kTqMergeBatch = 8;   // splits whose partial states are loaded together

// Pass 2: one workgroup of 64 lanes per query head.  The merged O' / L goes through LDS, where a
// Walsh-Hadamard transform forms H O'; the outputs are x_i = s_V[i] (H O')_i / sqrt(d).
template <int D>
__global__ __launch_bounds__(64) void tq_attn_merge_kernel(TqAttnArgs a) {
  constexpr int PER = D / 64;
  __shared__ float o_rot[D];
  const int lane = threadIdx.x;
  const int head = blockIdx.x;
  const float c2 = a.scale_log2;
  const int S = a.num_splits;
  const float* p = a.partial + (int64_t)head * S * (D + 2);
  // The partial states of up to kTqMergeBatch splits are loaded before any of them is used (one
  // memory round trip for the usual few splits); a later batch rescales what came before.
  float M = neg_inf(), L = 0.f;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int s0 = 0; s0 < S; s0 += kTqMergeBatch) {
    float ms[kTqMergeBatch], ls[kTqMergeBatch], os[kTqMergeBatch][PER];
#pragma unroll
    for (int j = 0; j < kTqMergeBatch; ++j) {
      const float* ps = p + (int64_t)min(s0 + j, S - 1) * (D + 2);
      ms[j] = s0 + j < S ? ps[0] : neg_inf();
      ls[j] = ps[1];
#pragma unroll
      for (int e = 0; e < PER; ++e) os[j][e] = ps[2 + min(lane + 64 * e, D - 1)];
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < kTqMergeBatch; ++j) Mb = fmaxf(Mb, ms[j]);
    if (Mb != neg_inf()) {
      const float r = __builtin_amdgcn_exp2f((M - Mb) * c2);   // 0 while M is -inf
      L *= r;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] *= r;
#pragma unroll
      for (int j = 0; j < kTqMergeBatch; ++j) {
        const float w = __builtin_amdgcn_exp2f((ms[j] - Mb) * c2);
        L += w * ls[j];
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] += w * os[j][e];
      }
      M = Mb;
    }
  }
  const float inv = L > 0.f ? __fdiv_rn(1.0f, L) : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) o_rot[lane + 64 * e] = o[e] * inv;
  __syncthreads();
  lds_hadamard<D>(o_rot, 1, lane, 64);
  const float rs = 1.0f / sqrtf((float)D);
  float y[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int i = lane + 64 * e;
    const float acc = o_rot[i] * rs;
    y[e] = a.vs[i] < 0 ? -acc : acc;
  }
  apply_epilogue_all(y, a.epi, [&](int e) { return lane + 64 * e; });
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int d = lane + 64 * e;
    if (a.out_bf16) static_cast<__bf16*>(a.out)[(int64_t)head * D + d] = (__bf16)y[e];
    else static_cast<float*>(a.out)[(int64_t)head * D + d] = y[e];
  }
  if (a.lse && lane == 0) a.lse[head] = L > 0.f ? M * a.scale + logf(L) : neg_inf();
}

template <int D, int KB, int VB>
hipError_t launch_tq_attn_d(const TqAttnArgs& a_in, hipStream_t st, const char** name) {
  TqAttnArgs a = a_in;
  constexpr int KT = TqCfg<D, KB, VB>::KT;
  const int tiles = (a.s_k - a.key_lo + KT - 1) / KT;
  a.tiles_per_split = (tiles + a.num_splits - 1) / a.num_splits;
  const dim3 grid((unsigned)((int64_t)a.num_splits * a.bh_kv * ((a.group + 3) / 4)));
  const bool so = a.sops.n > 0;
  if (so) hipLaunchKernelGGL((tq_attn_partial_kernel<D, KB, VB, true>), grid, dim3(64 * kTqWaves), 0, st, a);
  else hipLaunchKernelGGL((tq_attn_partial_kernel<D, KB, VB, false>), grid, dim3(64 * kTqWaves), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((tq_attn_merge_kernel<D>), dim3((unsigned)a.bh_q), dim3(64), 0, st, a);
  *name = so ? "tq_attention_decode_sops" : "tq_attention_decode";
  return hipGetLastError();
}

template <int D>
hipError_t launch_tq_attn_bits(const TqAttnArgs& a, int kb, int vb, hipStream_t st, const char** name) {
  if (kb == 4 && vb == 2) return launch_tq_attn_d<D, 4, 2>(a, st, name);
  if (kb == 4 && vb == 4) return launch_tq_attn_d<D, 4, 4>(a, st, name);
  if (kb == 2 && vb == 2) return launch_tq_attn_d<D, 2, 2>(a, st, name);
  if (kb == 2 && vb == 4) return launch_tq_attn_d<D, 2, 4>(a, st, name);
  if (kb == 3 && vb == 3) return launch_tq_attn_d<D, 3, 3>(a, st, name);
  if (kb == 3 && vb == 2) return launch_tq_attn_d<D, 3, 2>(a, st, name);
  if (kb == 3 && vb == 4) return launch_tq_attn_d<D, 3, 4>(a, st, name);
  if (kb == 4 && vb == 3) return launch_tq_attn_d<D, 4, 3>(a, st, name);
  if (kb == 2 && vb == 3) return launch_tq_attn_d<D, 2, 3>(a, st, name);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_tq_attention(const TqAttnArgs& a, int32_t d, int32_t kbits, int32_t vbits, hipStream_t st,
                               const char** name) {
  if ((int64_t)a.num_splits * a.bh_kv * ((a.group + 3) / 4) > 0x7fffffff) return hipErrorInvalidConfiguration;
  switch (d) {
    case 64: return launch_tq_attn_bits<64>(a, kbits, vbits, st, name);
    case 128: return launch_tq_attn_bits<128>(a, kbits, vbits, st, name);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
