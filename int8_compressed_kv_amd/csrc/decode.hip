// Split-KV decode over the int8 per-token KV cache (fkl.flash_attention PR, Verification: the
// decode check, one query row per head against the int8 cache; Summary: the cache is
// dequantized inside q.k and p.v and never expanded in global memory; kernbench2 ADR-0060
// commit: split decode whose partial running (m, l, O) states are reduced afterwards).
//
// Pass 1 (decode_partial_kernel), grid (splits, bh_kv, ceil(G/4)): a workgroup streams one
// contiguous range of keys of one KV head for up to 4 query heads of its GQA group and leaves
// one partial state (m, l, O unnormalised) per (query head, split) in the workspace.
// Pass 2 (decode_merge_kernel): per query head, M = max m_s, L = sum l_s e^(m_s - M),
// O = sum O_s e^(m_s - M) / L, then the epilogue and the store.
//
// HBM-bound.  Every K/V byte is read once for all query heads of its group.  Each wave streams
// its own tiles of 32 keys with plain 16-byte vector loads into two register tiles (the next
// tile is in flight while the current one is computed): on gfx950 this sustains a higher read
// rate than direct global -> LDS copies.  All cache reads, the per-key scales included, are
// nontemporal: ordinary cached loads of the small scale vectors interleaved with the streaming
// code loads measurably lower the achieved read bandwidth.  K is loaded
// straight into its MFMA operand layout; V passes through a small wave-private LDS slot so
// that the transposing read can hand each lane 16 keys of one head-dim column.  No barriers
// are needed until the final combine.
//
// Both products run exactly on the int8 MFMA (v_mfma_i32_16x16x64_i8), with no conversion of
// the cache:
//   * S = Q K^T.  A = K codes (16 keys x 64 head-dim), loaded from global memory.  B holds Q as four signed
//     7-bit digits, q = 2^E (d0/2^7 + d1/2^14 + d2/2^21 + d3/2^28), one MFMA column per
//     (digit, head): 4 digits x 4 heads fill the 16 columns that a single decode row would
//     otherwise leave empty.  The int32 products are exact; the digit columns are recombined
//     in fp32 with two DPP row rotations, so every lane ends up with the same S.
//   * O += P~ V with P~ = p * v_s.  B holds P~ as four unsigned 7-bit digits of P~ / 2^F
//     (2^F above the largest P~ so far), one column per (digit, head).  A = V^T codes, read
//     with transposing LDS reads (ds_read_b64_tr_b8) from the row-major tile.  The products
//     accumulate exactly in the int32 MFMA accumulators across tiles and are moved to fp32
//     only when the running max is raised or P~ outgrows 2^F (about 26 bits of P~ kept).
//   * Key order: MFMA row r of row-block kb holds key (KT/4)(r/4) + 4 kb + r%4, so lane group
//     g of the score accumulator owns keys (KT/4) g .. (KT/4) g + KT/4 - 1 -- exactly the keys
//     the transposing read gives that lane group for the P~ V product.
//   * The online softmax (running max raised lazily, as in the prefill kernel) runs in fp32.
#include "device_common.hpp"

namespace fa {
namespace {

constexpr float kLazyLog2 = 8.0f;
constexpr int kWaves = 4;
constexpr int kFlushTiles = 1024;   // int32 P~V accumulator bound: 1024 tiles x 64 keys x 127 x 127 < 2^31

template <int D>
struct DCfg {
  static constexpr int KT = 32;                           // keys per tile
  static constexpr int NC16 = D / 16;                     // 16-byte chunks per row
  static constexpr int SP = (NC16 % 8 == 0) ? 8 : (NC16 % 4 == 0) ? 4 : 2;   // swizzle span
  static constexpr int VCH = KT * NC16 / 64;              // 16-byte V loads per lane per tile
  static constexpr int NSC = 2 * KT / 64;                 // scale values per lane per tile
  static constexpr int SLOT = KT * D + 8 * KT;            // wave-private LDS bytes (V tile, scales)
  static constexpr int NT = 2;                            // register tile buffers per wave
};

template <int N>
__device__ __forceinline__ float dpp_row_ror(float x) {
  static_assert(N >= 1 && N <= 15, "row_ror amount");
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

typedef int i32x2v __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) i32x2v lds_i32x2;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

template <int SP>
__device__ __forceinline__ int dswz(int r) {
  return ((r >> 1) ^ (r >> 4)) & (SP - 1);
}

template <int D>
__global__ __launch_bounds__(64 * kWaves, 1) void decode_partial_kernel(DecodeArgs a) {
  using C = DCfg<D>;
  constexpr int KT = C::KT, NC16 = C::NC16, SP = C::SP, VCH = C::VCH;
  constexpr int KG = KT / 4;                    // keys per lane group
  constexpr int KB = KT / 16;                   // 16-row blocks of S per tile
  constexpr int NKK = (D + 63) / 64;            // 64-deep k-steps of Q.K
  constexpr int NB = D / 16;                    // 16-row blocks of O^T
  constexpr int HPW = 4;                        // query heads per workgroup

  __shared__ __attribute__((aligned(16))) unsigned char lds_slot[kWaves][C::SLOT];
  __shared__ float lds_m[kWaves][HPW];
  __shared__ float lds_l[kWaves][HPW];
  __shared__ float lds_o[kWaves][HPW][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;        // MFMA column: digit t = n / 4, head-in-tile gq = n % 4
  const int hq = lane >> 4;       // lane group (k-slot group of A/B, row group of C)
  const int t_dig = n >> 2;
  const int gq = n & 3;

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int zh = blockIdx.z * HPW;                      // first head of the group handled here
  const int nh = min(HPW, a.group - zh);                // heads handled here
  const int64_t kv_base = (int64_t)kvh * a.s_k;
  const int head0 = kvh * a.group + zh;

  // ---- Q digit B operands: column n = (t_dig, gq), k-slots 64 kk + 16 hq + i.  Each lane loads
  // its 16 contiguous head-dim values per k-step; E (max|q| * 2^-E < 1/2) comes from a max over
  // the lane's values and the other three lane groups (which hold the rest of the same head).
  i32x4 qdig[NKK];
  float s_comb;   // 2^(E - 7 (t + 1)) for this lane's digit column
  {
    const bool hv = gq < nh;
    const int64_t qrow = (int64_t)(head0 + (hv ? gq : 0)) * D;
    float qv[NKK][16];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int d0 = 64 * kk + 16 * hq;
      const bool ok = hv && d0 < D;
      const int64_t at = qrow + (ok ? d0 : 0);
      if (a.q_bf16) {
        const unsigned short* qp = static_cast<const unsigned short*>(a.q) + at;
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(qp);
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(qp + 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qv[kk][2 * e] = __uint_as_float(w0[e] << 16);
          qv[kk][2 * e + 1] = __uint_as_float(w0[e] & 0xffff0000u);
          qv[kk][8 + 2 * e] = __uint_as_float(w1[e] << 16);
          qv[kk][8 + 2 * e + 1] = __uint_as_float(w1[e] & 0xffff0000u);
        }
      } else {
        const float* qp = static_cast<const float*>(a.q) + at;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const f32x4 w = *reinterpret_cast<const f32x4*>(qp + 4 * e4);
#pragma unroll
          for (int e = 0; e < 4; ++e) qv[kk][4 * e4 + e] = w[e];
        }
      }
      if (!ok) {
#pragma unroll
        for (int i = 0; i < 16; ++i) qv[kk][i] = 0.f;
      }
    }
    float mx = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(qv[kk][i]));
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    int E = 0;
    if (mx > 0.f) {
      (void)frexpf(mx, &E);   // mx = f * 2^E, f in [0.5, 1)
      E += 1;
    }
    s_comb = ldexpf(1.f, E - 7 * (t_dig + 1));
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      unsigned w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = ldexpf(qv[kk][i], -E) * 128.f;
        float dd[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          dd[t] = __builtin_rintf(x);
          x = (x - dd[t]) * 128.f;
        }
        const int dig = (int)(t_dig == 0 ? dd[0] : t_dig == 1 ? dd[1] : t_dig == 2 ? dd[2] : dd[3]);
        w[i / 4] |= ((unsigned)dig & 0xffu) << (8 * (i % 4));
      }
      qdig[kk] = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
  }

  // ---- tiles of this split; wave w takes tiles w, w + 4, ... of the split
  const int n_tiles_total = (a.s_k - a.key_lo + KT - 1) / KT;
  const int ts = split * a.tiles_per_split;
  const int te = min(n_tiles_total, ts + a.tiles_per_split);
  const int n_w = te > ts + wave ? (te - ts - wave + kWaves - 1) / kWaves : 0;
  const int last_key = a.s_k - 1;

  // ---- register tiles: K in MFMA A layout (row n of block kb = key KG (n/4) + 4 kb + n%4,
  // 16 bytes at head-dim 64 kk + 16 hq); V rows as plain 16-byte chunks (chunk F = 64 u + lane:
  // row F / NC16, chunk F % NC16); scale value e of a lane is entry 64 e + lane of the tile's
  // [k scales | v scales] pair.
  constexpr int NSC = C::NSC;
  struct Tile {
    i32x4 k[KB][NKK];
    u32x4 v[VCH];
    float sc[NSC];
  };
  // Per-lane byte offsets inside a tile are loop-invariant; each load is a wave-uniform tile
  // base plus a 32-bit offset, with rows clamped to the last key (only the final tile of the
  // cache has rows past the end; they are masked in compute).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  int krow_off[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) krow_off[kb] = KG * (n >> 2) + 4 * kb + (n & 3);
  auto load = [&](int idx, Tile& T) {
    const int k0 = a.key_lo + (ts + wave_u + kWaves * idx) * KT;
    const int lim = last_key - k0;                 // last valid row inside this tile
    const int8_t* kt = a.k + (kv_base + k0) * D;
    const int8_t* vt = a.v + (kv_base + k0) * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int ro = min(krow_off[kb], lim) * D;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int cidx = 4 * kk + hq;
        T.k[kb][kk] = i32x4{0, 0, 0, 0};
        if (cidx < NC16) T.k[kb][kk] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(kt + ro + 16 * cidx));
      }
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int F = 64 * u + lane;
      const int o = min(F / NC16, lim) * D + 16 * (F % NC16);
      T.v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vt + o));
    }
    const float* kst = a.k_scale + kv_base + k0;
    const float* vst = a.v_scale + kv_base + k0;
#pragma unroll
    for (int e = 0; e < NSC; ++e) {
      const int slot_i = 64 * e + lane;            // < 2 KT
      const int r = min(slot_i % KT, lim);
      T.sc[e] = __builtin_nontemporal_load((slot_i < KT ? kst : vst) + r);
    }
  };
  unsigned char* slot = &lds_slot[wave][0];

  // O = Of + Oi * 2^(F - 7 (t + 1)): exact int32 MFMA sums since the last flush (Oi) and the
  // fp32 total before it (Of).  Oi is flushed when the running max is raised, when P~ outgrows
  // 2^F, and every kFlushTiles tiles.
  float Of[NB][4];
  i32x4 Oi[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    Oi[b] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int v = 0; v < 4; ++v) Of[b][v] = 0.f;
  }
  float m_run = neg_inf(), l_run = 0.f, mc = 0.f;
  int F = -1000;             // digit scale of Oi (per head column; equal on its 4 digit lanes)
  int since_flush = 0;
  const float c2 = a.scale_log2;
  const float lazy_thr = kLazyLog2 / c2;
  auto flush = [&]() {
    const float sc = ldexpf(1.f, F - 7 * (t_dig + 1));
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int v = 0; v < 4; ++v) Of[b][v] = __builtin_fmaf((float)Oi[b][v], sc, Of[b][v]);
      Oi[b] = i32x4{0, 0, 0, 0};
    }
    since_flush = 0;
  };

  auto compute = [&](int idx, bool valid, const Tile& T) {
    const int k0 = a.key_lo + (ts + wave_u + kWaves * idx) * KT;
    // V rows and the scales into the wave's LDS slot (row r, chunk c at chunk c ^ swz(r));
    // the previous tile's reads of the slot were consumed before this point.
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int F = 64 * u + lane;
      const int r = F / NC16;
      *reinterpret_cast<u32x4*>(slot + r * D + 16 * ((F % NC16) ^ dswz<SP>(r))) = T.v[u];
    }
#pragma unroll
    for (int e = 0; e < NSC; ++e) reinterpret_cast<float*>(slot + KT * D)[64 * e + lane] = T.sc[e];
    const unsigned char* vb_ = slot;
    const float* sk = reinterpret_cast<const float*>(slot + KT * D);
    const float* sv = sk + KT;
    // this lane's keys: KG hq + 4 kb + v
    float ks[KB][4], vs[KB][4];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(sk + KG * hq + 4 * kb);
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(sv + KG * hq + 4 * kb);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        ks[kb][v] = a4[v];
        vs[kb][v] = b4[v];
      }
    }
    const bool tail = !valid || k0 + KT > a.s_k;
    const int key_lim = valid ? last_key - k0 - KG * hq : -1;   // key KG hq + j is visible iff j <= key_lim

    // S^T: block kb, C-row 4 hq + v = key KG hq + 4 kb + v; A row n = key KG (n/4) + 4 kb + n%4
    float s[KB][4];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      i32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) acc = mfma16_i8(T.k[kb][kk], qdig[kk], acc);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float y = (float)acc[v] * s_comb;
        y = y + dpp_row_ror<8>(y);
        y = y + dpp_row_ror<4>(y);
        s[kb][v] = y * ks[kb][v];
      }
    }
    if (tail) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (4 * kb + v > key_lim) s[kb][v] = neg_inf();
    }
    float mx = neg_inf();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[kb][v]);
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    if (__any(mx - m_run > lazy_thr)) {
      flush();
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) Of[b][v] *= alpha;
      m_run = m_new;
      mc = m_use * c2;
    }
    float pt[KB][4];
    float ps = 0.f, pmax = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][v], c2, -mc));
        ps += p;
        pt[kb][v] = p * vs[kb][v];
        pmax = fmaxf(pmax, pt[kb][v]);
      }
    l_run += ps;
    pmax = max_xor16(pmax);
    pmax = max_xor32(pmax);
    int Fp = -1000;
    if (pmax > 0.f) (void)frexpf(pmax, &Fp);    // pmax < 2^Fp
    if (__any(Fp > F) || since_flush >= kFlushTiles) {
      flush();
      if (Fp > F) F = Fp + 1;                  // one octave of headroom for later tiles
    }
    ++since_flush;
    // digit t of x = P~ / 2^F in [0, 1) is bits 0..6 of floor(x 2^(7t+7)) (exact: the product
    // is a power-of-two scaling and x < 1 keeps it below 2^28); k-slot 4 kb + v of lane group
    // hq is key KG hq + 4 kb + v
    const float to_int = ldexpf(1.f, 7 * t_dig + 7 - F);
    unsigned pw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      unsigned w = 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) w |= (((unsigned)(pt[kb][v] * to_int)) & 0xffu) << (8 * v);
      pw[kb] = w & 0x7f7f7f7fu;
    }
    const i32x4 pdig = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]};

    // O^T block b (head-dim 16 b + row): A = V^T via transposing reads.  As a source lane, n
    // addresses key row KG hq + 8 h8 + n/2, bytes 16 b + 8 (n%2) .. + 8; lane n then receives
    // keys KG hq + 8 h8 + 0..7 of head-dim 16 b + n.
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      int w4[4] = {0, 0, 0, 0};
#pragma unroll
      for (int h8 = 0; h8 < KG / 8; ++h8) {
        const int vrow = KG * hq + 8 * h8 + (n >> 1);
        const int off = vrow * D + 16 * (b ^ dswz<SP>(vrow)) + 8 * (n & 1);
        const i32x2v r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)((lds_u8*)vb_ + off));
        w4[2 * h8] = r[0];
        w4[2 * h8 + 1] = r[1];
      }
      const i32x4 vt = {w4[0], w4[1], w4[2], w4[3]};
      Oi[b] = mfma16_i8(vt, pdig, Oi[b]);
    }
  };

  // ---- stream: a ring of NT register tiles keeps the loads of the next NT - 1 tiles in flight
  // while the current one is computed.  The loop is straight-line so that the compiler's
  // load-wait counts stay exact: loads are always issued (past the end they repeat the last
  // tile), the trip count is padded to a multiple of NT, and padded tiles compute fully masked.
  constexpr int NT = C::NT;
  Tile T[NT];
  if (n_w > 0) {
#pragma unroll
    for (int i = 0; i < NT - 1; ++i) load(min(i, n_w - 1), T[i]);
    for (int base = 0; base < n_w; base += NT) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int idx = base + j;
        load(min(idx + NT - 1, n_w - 1), T[(j + NT - 1) % NT]);
        compute(idx, idx < n_w, T[j]);
      }
    }
  }

  // ---- combine digit columns (O) and lane groups (l), then the waves through LDS
  flush();
  float O[NB][4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int v = 0; v < 4; ++v) O[b][v] = Of[b][v];
  float lt = l_run;
  lt = add_xor16(lt);
  lt = add_xor32(lt);
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float y = O[b][v];
      y = y + dpp_row_ror<8>(y);
      y = y + dpp_row_ror<4>(y);
      O[b][v] = y;
    }
  if (lane == gq) {  // t_dig == 0, hq == 0
    lds_m[wave][gq] = m_run;
    lds_l[wave][gq] = lt;
  }
  if (t_dig == 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) lds_o[wave][gq][16 * b + 4 * hq + v] = O[b][v];
  }
  __syncthreads();

  for (int idx = tid; idx < nh * (D + 2); idx += 64 * kWaves) {
    const int hz = idx / (D + 2), col = idx % (D + 2);
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds_m[w][hz]);
    float acc = 0.f;
    if (col == 0) {
      acc = M;
    } else if (M != neg_inf()) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = __builtin_amdgcn_exp2f((lds_m[w][hz] - M) * c2);
        acc += wt * (col == 1 ? lds_l[w][hz] : lds_o[w][hz][col - 2]);
      }
    }
    const int64_t head = head0 + hz;
    a.partial[(head * a.num_splits + split) * (D + 2) + col] = acc;
  }
}

// Pass 2: one single-wave workgroup per query head merges the splits' partial states; the
// split loop is unrolled so the partial-state loads of several splits are in flight together.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int PER = (D + 63) / 64;
  const int lane = threadIdx.x;
  const int head = blockIdx.x;
  const float c2 = a.scale_log2;
  const int S = a.num_splits;
  const float* p = a.partial + (int64_t)head * S * (D + 2);
  float M = neg_inf();
  for (int s = lane; s < S; s += 64) M = fmaxf(M, p[(int64_t)s * (D + 2)]);
#pragma unroll
  for (int o2 = 32; o2 >= 1; o2 >>= 1) M = fmaxf(M, __shfl_xor(M, o2, 64));
  float L = 0.f;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  if (M != neg_inf()) {
#pragma unroll 8
    for (int s = 0; s < S; ++s) {
      const float* ps = p + (int64_t)s * (D + 2);
      const float w = __builtin_amdgcn_exp2f((ps[0] - M) * c2);
      L += w * ps[1];
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int d = lane + 64 * e;
        if (d < D) o[e] += w * ps[2 + d];
      }
    }
  }
  const float inv = L > 0.f ? __fdiv_rn(1.0f, L) : 0.f;
  float y[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) y[e] = o[e] * inv;
  apply_epilogue_all(y, a.epi, [&](int e) { return min(lane + 64 * e, D - 1); });   // lanes past D discard
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int d = lane + 64 * e;
    if (d < D) {
      if (a.out_bf16) static_cast<__bf16*>(a.out)[(int64_t)head * D + d] = (__bf16)y[e];
      else static_cast<float*>(a.out)[(int64_t)head * D + d] = y[e];
    }
  }
  if (a.lse && lane == 0) a.lse[head] = L > 0.f ? M * a.scale + logf(L) : neg_inf();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a_in, hipStream_t st, const char** name) {
  DecodeArgs a = a_in;
  constexpr int KT = DCfg<D>::KT;
  const int tiles = (a.s_k - a.key_lo + KT - 1) / KT;
  a.tiles_per_split = (tiles + a.num_splits - 1) / a.num_splits;
  const dim3 grid((unsigned)a.num_splits, (unsigned)a.bh_kv, (unsigned)((a.group + 3) / 4));
  hipLaunchKernelGGL((decode_partial_kernel<D>), grid, dim3(64 * kWaves), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)a.bh_q), dim3(64), 0, st, a);
  *name = "decode_int8";
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int32_t d, hipStream_t stream, const char** name) {
  if (a.bh_kv > 65535 || (a.group + 3) / 4 > 65535) return hipErrorInvalidConfiguration;
  switch (d) {
    case 32: return launch_d<32>(a, stream, name);
    case 64: return launch_d<64>(a, stream, name);
    case 96: return launch_d<96>(a, stream, name);
    case 128: return launch_d<128>(a, stream, name);
    case 160: return launch_d<160>(a, stream, name);
    case 192: return launch_d<192>(a, stream, name);
    case 224: return launch_d<224>(a, stream, name);
    case 256: return launch_d<256>(a, stream, name);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
