// Split-KV decode over the int8 per-token KV cache (fkl.flash_attention PR, Verification: the
// decode check, one query row per head against the int8 cache; Summary: the cache is
// dequantized inside q.k and p.v and never expanded in global memory; kernbench2 ADR-0060
// commit: split decode whose partial running (m, l, O) states are reduced afterwards).
//
// Pass 1 (decode_partial_kernel), grid (splits, bh_kv, ceil(G/H)): a workgroup streams one
// contiguous range of keys of one KV head for up to H query heads of its GQA group (H = 4, or
// 8 as two MFMA column sets when G > 4 and head_dim <= 128) and leaves one partial state
// (m, l, O unnormalised) per (query head, split) in the workspace.
// Pass 2 (decode_merge_kernel): per query head, M = max m_s, L = sum l_s e^(m_s - M),
// O = sum O_s e^(m_s - M) / L, then the epilogue and the store.
//
// HBM-bound.  Every K/V byte is read once for all query heads of its group when G <= H (G <= 8
// at head_dim <= 128, G <= 4 above; a larger group reads the cache ceil(G/H) times).  Each wave
// streams its own tiles of 32 keys with 16-byte buffer loads into two register tiles (the next
// tile is in flight while the current one is computed): on gfx950 this sustains a higher read
// rate than direct global -> LDS copies.  All cache reads, the per-key scales included, are
// nontemporal: ordinary cached loads of the small scale vectors interleaved with the streaming
// code loads measurably lower the achieved read bandwidth.  K is loaded straight into its MFMA
// operand layout; V passes through a small wave-private LDS slot so that the transposing read
// can hand each lane 8 keys of one head-dim column.  No barriers are needed until the final
// combine.  With a group of 8 the wave issues twice the vector work per cache byte at one wave
// per SIMD, so the per-tile instruction count (loads with loop-invariant offsets, the V^T reads
// issued ahead of the softmax, DPP sums folded into the adds) sets its speed.
//
// Both products run exactly on the int8 MFMA (v_mfma_i32_16x16x64_i8 for Q.K, ..x32_i8 for
// P~.V), with no conversion of the cache:
//   * S = Q K^T.  A = K codes (16 keys x 64 head-dim), loaded from global memory.  B holds Q as four signed
//     7-bit digits, q = 2^E (d0/2^7 + d1/2^14 + d2/2^21 + d3/2^28), one MFMA column per
//     (digit, head): 4 digits x 4 heads fill the 16 columns that a single decode row would
//     otherwise leave empty.  The int32 products are exact; the digit columns are recombined
//     in fp32 with two DPP row rotations, so every lane ends up with the same S.
//   * O += P~ V with P~ = p * v_s.  x = P~ / 2^F (2^F above every P~ since the last flush) is
//     rounded (half up) at 28 fractional bits and split into four unsigned 7-bit digits, one
//     MFMA column per (digit, head).  A = V^T codes, read with transposing LDS reads
//     (ds_read_b64_tr_b8) from the row-major tile.  The products accumulate exactly in the
//     int32 MFMA accumulators across tiles and are moved to fp32 when the running max is raised,
//     when P~ outgrows 2^F, or after kFlushTiles tiles; F then restarts from the current tile.
//     Each P~ thus carries a rounding error of at most 2^(F - 29) (or 2^-23 of P~ where
//     P~ >= 2^(F - 5), below the fp32 rounding P~ already carries), F set by the largest P~ of
//     the tiles since the last flush under the same running max.
//   * Key order: MFMA row r of row-block kb holds key (KT/4)(r/4) + 4 kb + r%4, so lane group
//     g of the score accumulator owns keys (KT/4) g .. (KT/4) g + KT/4 - 1 -- exactly the keys
//     the transposing read gives that lane group for the P~ V product.
//   * The online softmax (running max raised lazily, as in the prefill kernel) runs in fp32.
#include <mutex>

#include "device_common.hpp"

namespace fa {

// Fixed scratch for the allocation-free decode entry point: the partial (m, l, O) states of
// every (query head, split), each written in full by the partial pass before the merge pass
// reads it, so nothing needs clearing between calls.  Host code never uses the array's name as
// an address (on the host it is only a stand-in); it uses the per-device address from
// hipGetSymbolAddress below.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch_address(int device, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *ptr = addr[device];
  return hipSuccess;
}
namespace {

constexpr float kLazyLog2 = 8.0f;
constexpr int kWaves = 4;
constexpr int kFlushTiles = 1024;   // int32 P~V accumulator bound: 1024 tiles x 64 keys x 127 x 127 < 2^31

template <int D>
struct DCfg {
  static constexpr int KT = 32;                           // keys per tile
  static constexpr int NC16 = D / 16;                     // 16-byte chunks per row
  static constexpr int VCH = KT * NC16 / 64;              // 16-byte V loads per lane per tile
  static constexpr int NSC = 2 * KT / 64;                 // scale values per lane per tile
  // LDS row stride of the V slot: 16 bytes of padding per row put the 8 rows that one quarter
  // of a transposing read touches on distinct banks, and keep every slot address a per-lane
  // base plus an immediate offset
  static constexpr int RS = D + 16;
  static constexpr int SLOT = KT * RS + 8 * KT;           // wave-private LDS bytes (V tile, scales)
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

constexpr int kBufferFlags = 0x00020000;
constexpr int kNt = 2;   // nontemporal cache policy of a buffer access

template <int D, int NS, bool SOPS>
__global__ __launch_bounds__(64 * kWaves, 1) void decode_partial_kernel(DecodeArgs a) {
  using C = DCfg<D>;
  constexpr int KT = C::KT, NC16 = C::NC16, VCH = C::VCH;
  constexpr int KG = KT / 4;                    // keys per lane group
  constexpr int KB = KT / 16;                   // 16-row blocks of S per tile
  constexpr int NKK = (D + 63) / 64;            // 64-deep k-steps of Q.K
  constexpr int NB = D / 16;                    // 16-row blocks of O^T
  constexpr int HPW = 4 * NS;                   // query heads per workgroup (NS column sets of 4)

  __shared__ __attribute__((aligned(16))) unsigned char lds_slot[kWaves][C::SLOT];
  __shared__ float lds_m[kWaves][HPW];
  __shared__ float lds_l[kWaves][HPW];
  __shared__ float lds_o[kWaves][HPW][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;        // MFMA column: digit t = n / 4, head-in-set gq = n % 4
  const int hq = lane >> 4;       // lane group (k-slot group of A/B, row group of C)
  const int t_dig = n >> 2;
  const int gq = n & 3;

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int zh = blockIdx.z * HPW;                      // first head of the group handled here
  const int nh = min(HPW, a.group - zh);                // heads handled here
  const int64_t kv_base = (int64_t)kvh * a.s_k;
  const int head0 = kvh * a.group + zh;

  // ---- Q digit B operands: column set c, column n = (t_dig, gq) is head 4 c + gq; k-slots
  // 64 kk + 16 hq + i.  Each lane loads its 16 contiguous head-dim values per k-step; E
  // (max|q| * 2^-E < 1/2) comes from a max over the lane's values and the other three lane
  // groups (which hold the rest of the same head).
  i32x4 qdig[NS][NKK];
  float s_comb[NS];   // 2^(E - 7 (t + 1)) for this lane's digit column
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    const bool hv = 4 * c + gq < nh;
    const int64_t qrow = (int64_t)(head0 + (hv ? 4 * c + gq : 0)) * D;
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
    s_comb[c] = ldexpf(1.f, E - 7 * (t_dig + 1));
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
      qdig[c][kk] = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
  }

  // ---- tiles of this split; wave w takes tiles w, w + 4, ... of the split
  const int n_tiles_total = (a.s_k - a.key_lo + KT - 1) / KT;
  const int ts = split * a.tiles_per_split;
  const int te = min(n_tiles_total, ts + a.tiles_per_split);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int n_w = te > ts + wave_u ? (te - ts - wave_u + kWaves - 1) / kWaves : 0;
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
  int krow_off[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) krow_off[kb] = KG * (n >> 2) + 4 * kb + (n & 3);
  // Tile loads are raw buffer loads: the resource is the wave-uniform tile base with the bytes
  // left in the head as its bound, and every per-lane offset is loop-invariant, so a load costs
  // no vector instruction.  Rows past the last key read zeros (offsets at or beyond the bound);
  // such keys are masked in compute.  K chunks past head_dim (head_dim not a multiple of 64)
  // read the next row's bytes, or zeros at the bound: their Q digits are zero.  The scale
  // lanes that belong to the other matrix get an offset beyond any bound and read zero.
  constexpr unsigned kOob = 0x80000000u;
  unsigned koff[KB][NKK], voff[VCH], skoff[NSC], svoff[NSC];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int cidx = 4 * kk + hq;
      koff[kb][kk] = (unsigned)(krow_off[kb] * D + 16 * cidx);
    }
#pragma unroll
  for (int u = 0; u < VCH; ++u) voff[u] = 16u * (64 * u + lane);
#pragma unroll
  for (int e = 0; e < NSC; ++e) {
    const int slot_i = 64 * e + lane;            // < 2 KT
    skoff[e] = slot_i < KT ? 4u * slot_i : kOob;
    svoff[e] = slot_i < KT ? kOob : 4u * (slot_i - KT);
  }
  auto load = [&](int idx, Tile& T) {
    const int k0 = a.key_lo + (ts + wave_u + kWaves * idx) * KT;
    const int64_t left = a.s_k - k0;             // >= 1: loads never start past the last key
    const int nrec = (int)min(left * D, (int64_t)0x7fffffff);
    const int nrec_s = (int)min(left * 4, (int64_t)0x7fffffff);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a.k + (kv_base + k0) * D), 0, nrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a.v + (kv_base + k0) * D), 0, nrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rks =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.k_scale + kv_base + k0), 0, nrec_s, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rvs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.v_scale + kv_base + k0), 0, nrec_s, kBufferFlags);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        T.k[kb][kk] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff[kb][kk], 0, kNt));
#pragma unroll
    for (int u = 0; u < VCH; ++u)
      T.v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff[u], 0, kNt));
#pragma unroll
    for (int e = 0; e < NSC; ++e)
      T.sc[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rks, skoff[e], 0, kNt) |
                                __builtin_amdgcn_raw_buffer_load_b32(rvs, svoff[e], 0, kNt));
  };
  unsigned char* slot = &lds_slot[wave][0];

  // Per column set: O = Of + Oi * 2^(F - 7 (t + 1)), Oi the exact int32 MFMA sums of P~ V since
  // the last flush and Of the fp32 total before it.  Oi is flushed when the running max is
  // raised, when P~ outgrows 2^F, and every kFlushTiles tiles; after a flush the digit scale F
  // restarts from the current tile's largest P~ (Oi is empty then), so it never stays high
  // after a raise of the running max.
  float Of[NS][NB][4];
  i32x4 Oi[NS][NB];
  float m_run[NS], l_run[NS], mc[NS];
  int F[NS];                 // digit scale of Oi (per head column; equal on its 4 digit lanes)
  int since_flush[NS];
#pragma unroll
  for (int c = 0; c < NS; ++c) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      Oi[c][b] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int v = 0; v < 4; ++v) Of[c][b][v] = 0.f;
    }
    m_run[c] = neg_inf();
    l_run[c] = 0.f;
    mc[c] = 0.f;
    F[c] = -1000;
    since_flush[c] = 0;
  }
  const float c2 = a.scale_log2;
  const float lazy_thr = kLazyLog2 / c2;
  // Oi -> Of.  ldexp keeps the scaling exact (no overflow of a separately formed 2^x) for any F.
  auto flush = [&](int c) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int v = 0; v < 4; ++v) Of[c][b][v] += ldexpf((float)Oi[c][b][v], F[c] - 7 * (t_dig + 1));
      Oi[c][b] = i32x4{0, 0, 0, 0};
    }
    since_flush[c] = 0;
  };

  auto compute = [&](int idx, bool valid, const Tile& T) {
    const int k0 = a.key_lo + (ts + wave_u + kWaves * idx) * KT;
    // V rows (row r at r RS) and the scales into the wave's LDS slot, after the previous tile's
    // reads of it and before this tile's
    wave_lds_order();
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int Fc = 64 * u + lane;
      const int r = Fc / NC16;
      *reinterpret_cast<u32x4*>(slot + r * C::RS + 16 * (Fc % NC16)) = T.v[u];
    }
#pragma unroll
    for (int e = 0; e < NSC; ++e) reinterpret_cast<float*>(slot + KT * C::RS)[64 * e + lane] = T.sc[e];
    wave_lds_order();
    const unsigned char* vb_ = slot;
    const float* sk = reinterpret_cast<const float*>(slot + KT * C::RS);
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
    // A = V^T of O^T block b (head-dim 16 b + row), read before the softmax so that the LDS
    // latency is hidden behind it.  As a source lane, n addresses key row KG hq + n/2, bytes
    // 16 b + 8 (n%2) .. + 8; lane n then receives keys KG hq + 0..7 of head-dim 16 b + n.
    static_assert(KG == 8, "P.V takes one 8-key k-group per lane group");
    long vt[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int vrow = KG * hq + (n >> 1);
      const int off = vrow * C::RS + 16 * b + 8 * (n & 1);
      vt[b] = __builtin_bit_cast(long, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)((lds_u8*)vb_ + off)));
    }
    const bool tail = !valid || k0 + KT > a.s_k;
    const int key_lim = valid ? last_key - k0 - KG * hq : -1;   // key KG hq + j is visible iff j <= key_lim

    // The column sets go through each phase of the tile together: the rare raise and flush
    // branches then split the code only between phases, and within a phase the sets' independent
    // instructions interleave (one wave per SIMD has no other wave to cover their latencies).
    // S^T: block kb, C-row 4 hq + v = key KG hq + 4 kb + v; A row n = key KG (n/4) + 4 kb + n%4
    float s[NS][KB][4];
#pragma unroll
    for (int c = 0; c < NS; ++c) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        i32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) acc = mfma16_i8(T.k[kb][kk], qdig[c][kk], acc);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
#pragma clang fp contract(off)
          float y = (float)acc[v] * s_comb[c];   // kept apart from the add, which then takes the DPP operand
          y = y + dpp_row_ror<8>(y);
          y = y + dpp_row_ror<4>(y);
          s[c][kb][v] = y * ks[kb][v];
        }
      }
      if constexpr (SOPS) {
        float x[KB * 4];
#pragma unroll
        for (int j = 0; j < KB * 4; ++j) x[j] = s[c][j / 4][j % 4];
        apply_score_ops(x, a.sops, [&](int j) { return min(k0 + KG * hq + j, last_key); });
#pragma unroll
        for (int j = 0; j < KB * 4; ++j) s[c][j / 4][j % 4] = x[j];
      }
    }
    if (tail) {
#pragma unroll
      for (int c = 0; c < NS; ++c)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (4 * kb + v > key_lim) s[c][kb][v] = neg_inf();
    }
    float mx[NS];
    bool raised[NS];   // wave-uniform
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      float m = neg_inf();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) m = fmaxf(m, s[c][kb][v]);
      m = max_xor16(m);
      mx[c] = max_xor32(m);
      raised[c] = __any(mx[c] - m_run[c] > lazy_thr);
    }
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      if (raised[c]) {
        flush(c);
        const float m_new = fmaxf(m_run[c], mx[c]);
        const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_run[c] - m_use) * c2);
        l_run[c] *= alpha;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 4; ++v) Of[c][b][v] *= alpha;
        m_run[c] = m_new;
        mc[c] = m_use * c2;
      }
    }
    float pt[NS][KB][4];
    int Fp[NS];
    bool grow[NS];     // wave-uniform
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      float ps = 0.f, pmax = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][kb][v], c2, -mc[c]));
          ps += p;
          pt[c][kb][v] = p * vs[kb][v];
          pmax = fmaxf(pmax, pt[c][kb][v]);
        }
      l_run[c] += ps;
      pmax = max_xor16(pmax);
      pmax = max_xor32(pmax);
      Fp[c] = -1000;
      if (pmax > 0.f) (void)frexpf(pmax, &Fp[c]);    // pmax < 2^Fp
      grow[c] = __any(Fp[c] > F[c]) || since_flush[c] >= kFlushTiles;
    }
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      if (grow[c] && !raised[c]) flush(c);
      if (raised[c] || grow[c]) F[c] = Fp[c] + 1;   // Oi is empty: restart the scale, one octave of headroom
      ++since_flush[c];
    }
    // x = P~ / 2^F lies in [0, 1): Q = floor(x 2^28 + 1/2) < 2^28 is x to 28 fractional bits
    // (one fp32 multiply-add: the scaling by a power of two is exact, and so is the added half
    // while x 2^28 < 2^23; above, x 2^28 is an integer and the add may round it up by one,
    // 2^-23 of x at most), and digit t of x is bits 21 - 7t .. 27 - 7t of Q.  k-slot
    // 4 kb + v of lane group hq is key KG hq + 4 kb + v.
    const int sh = 21 - 7 * t_dig;
    long pdig[NS];
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      unsigned pw[KB];
      const float sc = ldexpf(1.f, 28 - F[c]);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        unsigned w = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const unsigned qx = (unsigned)__builtin_fmaf(pt[c][kb][v], sc, 0.5f);
          w |= __builtin_amdgcn_ubfe(qx, sh, 7) << (8 * v);
        }
        pw[kb] = w;
      }
      pdig[c] = (long)(((unsigned long)pw[1] << 32) | pw[0]);
    }

    // O^T block b += V^T P~^T on the 32-deep int8 MFMA: the tile's 32 keys are its k-slots
    // (lane group hq holds keys KG hq .. KG hq + 7), V^T is shared by the column sets.
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int c = 0; c < NS; ++c) Oi[c][b] = __builtin_amdgcn_mfma_i32_16x16x32_i8(vt[b], pdig[c], Oi[c][b], 0, 0, 0);
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
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    flush(c);
    float lt = l_run[c];
    lt = add_xor16(lt);
    lt = add_xor32(lt);
    if (lane == gq) {  // t_dig == 0, hq == 0
      lds_m[wave][4 * c + gq] = m_run[c];
      lds_l[wave][4 * c + gq] = lt;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float y = Of[c][b][v];
        y = y + dpp_row_ror<8>(y);
        y = y + dpp_row_ror<4>(y);
        if (t_dig == 0) lds_o[wave][4 * c + gq][16 * b + 4 * hq + v] = y;
      }
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

// Pass 2: one single-wave workgroup per query head merges the splits' partial states.
constexpr int kMergeBatch = 8;
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int PER = (D + 63) / 64;
  const int lane = threadIdx.x;
  const int head = blockIdx.x;
  const float c2 = a.scale_log2;
  const int S = a.num_splits;
  const float* p = a.partial + (int64_t)head * S * (D + 2);
  // The partial states of up to kMergeBatch splits are loaded before any of them is used (one
  // memory round trip for the usual few splits); a later batch rescales what came before.
  float M = neg_inf(), L = 0.f;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int s0 = 0; s0 < S; s0 += kMergeBatch) {
    float ms[kMergeBatch], ls[kMergeBatch], os[kMergeBatch][PER];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const float* ps = p + (int64_t)min(s0 + j, S - 1) * (D + 2);
      ms[j] = s0 + j < S ? ps[0] : neg_inf();
      ls[j] = ps[1];
#pragma unroll
      for (int e = 0; e < PER; ++e) os[j][e] = ps[2 + min(lane + 64 * e, D - 1)];
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) Mb = fmaxf(Mb, ms[j]);
    if (Mb != neg_inf()) {
      const float r = __builtin_amdgcn_exp2f((M - Mb) * c2);   // 0 while M is -inf
      L *= r;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] *= r;
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        const float w = __builtin_amdgcn_exp2f((ms[j] - Mb) * c2);
        L += w * ls[j];
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] += w * os[j][e];
      }
      M = Mb;
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

template <int D, int NS>
hipError_t launch_d(const DecodeArgs& a_in, hipStream_t st, const char** name) {
  DecodeArgs a = a_in;
  constexpr int KT = DCfg<D>::KT;
  const int tiles = (a.s_k - a.key_lo + KT - 1) / KT;
  a.tiles_per_split = (tiles + a.num_splits - 1) / a.num_splits;
  const int hpw = 4 * NS;
  const dim3 grid((unsigned)a.num_splits, (unsigned)a.bh_kv, (unsigned)((a.group + hpw - 1) / hpw));
  const bool so = a.sops.n > 0;
  if (so) hipLaunchKernelGGL((decode_partial_kernel<D, NS, true>), grid, dim3(64 * kWaves), 0, st, a);
  else hipLaunchKernelGGL((decode_partial_kernel<D, NS, false>), grid, dim3(64 * kWaves), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)a.bh_q), dim3(64), 0, st, a);
  if (NS == 2) *name = so ? "decode_int8_h8_sops" : "decode_int8_h8";
  else *name = so ? "decode_int8_sops" : "decode_int8";
  return hipGetLastError();
}

template <int D>
hipError_t launch_hd(const DecodeArgs& a, hipStream_t st, const char** name) {
  if constexpr (D <= 128) {
    if (decode_heads_per_workgroup(a.group, D) == 8) return launch_d<D, 2>(a, st, name);
  }
  return launch_d<D, 1>(a, st, name);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int32_t d, hipStream_t stream, const char** name) {
  const int hpw = decode_heads_per_workgroup(a.group, d);
  if (a.bh_kv > 65535 || (a.group + hpw - 1) / hpw > 65535) return hipErrorInvalidConfiguration;
  switch (d) {
    case 32: return launch_hd<32>(a, stream, name);
    case 64: return launch_hd<64>(a, stream, name);
    case 96: return launch_hd<96>(a, stream, name);
    case 128: return launch_hd<128>(a, stream, name);
    case 160: return launch_hd<160>(a, stream, name);
    case 192: return launch_hd<192>(a, stream, name);
    case 224: return launch_hd<224>(a, stream, name);
    case 256: return launch_hd<256>(a, stream, name);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
