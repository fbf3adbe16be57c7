// bf16 attention forward on gfx950 MFMA, for bf16 Q, K and V (the int8-cache variant of the
// same kernel is prefill_i8kv.hip).
//
// Method: FlashAttention-2 style tiled forward with an online softmax (fkl.flash_attention
// PR, Summary: FA-2 forward, fp32 accumulation; Foundry attention/ README, References: the
// online-softmax recurrence).  For each key
// tile, with running row max m, running sum l and accumulator O:
//   S = sigma * Q K^T (masked) ; m' = max(m, rowmax S) ; P = exp(S - m') ;
//   l = exp(m - m') l + rowsum P ; O = exp(m - m') O + P V.
// Finally O / l, the epilogue ops in fp32, and the store.
//
// gfx950 mapping
//   * A workgroup is 8 waves = 256 query rows (4 waves for head_dim > 128, whose fragments
//     need the whole register file); each wave owns 32 rows and keeps their Q fragments in
//     registers.  Two waves per SIMD: while one runs the softmax on the vector ALU the other
//     keeps the matrix core busy.
//   * K and V tiles of 64 keys live in LDS row-major, 16-byte chunks XOR-swizzled by row so
//     that both operand reads below are free of bank conflicts.  Tiles are copied global -> LDS
//     directly (no staging registers): for head_dim <= 128 into four stages with one barrier per
//     two tiles, the tile loop unrolled so that the stage is a compile-time constant in every LDS
//     address; above 128 into two stages with one barrier per tile.
//   * S^T = K Q^T (keys = MFMA rows, queries = columns) on v_mfma_f32_32x32x16_bf16: each
//     query's scores sit in one lane pair, so the row max needs one exchange, and P^T in the
//     accumulator layout is already the B operand of O^T += V^T P^T.  The V^T operand (8 keys
//     of one head-dim column per lane) comes from two transposing LDS reads
//     (ds_read_b64_tr_b16) of the row-major tile.
//   * The running max is only raised when a row's tile max exceeds it by more than 2^8 in the
//     exp2 domain; otherwise the stale max is kept (O and l stay mutually consistent, the O
//     rescale is skipped) and P stays below 2^8.
//   * Tiles wholly outside a wave's causal / window band are skipped; element masks are
//     applied only on boundary tiles.  Blocks run longest-first under causal masks and are
//     dealt to the 8 XCDs so that the G query heads sharing a KV head stay on one XCD.
#include <type_traits>

#include "device_common.hpp"

namespace fa {
namespace {

typedef short s16x4v __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) s16x4v lds_s16x4;

template <int D>
struct Cfg {
  static constexpr int NW = D <= 128 ? 8 : 4;    // waves per workgroup (2 or 1 per SIMD)
  static constexpr int BM = 32 * NW;             // query rows per workgroup
  static constexpr int BN = 64;                  // keys per LDS tile
  static constexpr int NC = D / 8;               // 16-byte chunks per row
  static constexpr int TILE = BN * D;            // 16-bit elements per K or V tile
  static constexpr int SWZ = (NC % 16 == 0) ? 16 : (NC % 8 == 0) ? 8 : 4;   // swizzle span
  static constexpr float kLazyLog2 = 8.0f;       // stale-max headroom, exp2 domain
};

// chunk permutation of row r: rows r..r+3 land in disjoint 4-chunk groups, 16 rows in 16
// distinct chunks.
template <int SWZ>
__device__ __forceinline__ int swz(int r) {
  return (((r & 3) << 2) | ((r >> 2) & 3)) & (SWZ - 1);
}

// Direct global -> LDS copy of 16 bytes per lane: lane l writes the bytes at LDS byte address
// lds + 16 l.  Written as inline assembly (no output registers: the data goes to LDS) so that
// the compiler does not add a full wait before every later LDS read; the kernel waits for its
// own copies (wait_vmcnt0) before the barrier that publishes them.
__device__ __forceinline__ void copy16_to_lds(const void* src, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src)
               : "memory", "m0");
}
// The same copy addressed as a wave-uniform 64-bit base plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void copy16_to_lds(const void* sbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
// s_waitcnt vmcnt(0), the other counters unconstrained (gfx9 encoding)
__device__ __forceinline__ void wait_vmcnt0() {
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
}

template <int D, bool SOPS>
__global__ __launch_bounds__(64 * Cfg<D>::NW, 1) void prefill_bf16_kernel(PrefillArgs a) {
  using C = Cfg<D>;
  constexpr int NW = C::NW, BM = C::BM, BN = C::BN, NC = C::NC;
  // head_dim 64 and 128: tiles arrive by direct global -> LDS copies into four stages, one
  // barrier per two tiles; other head dims stage through registers into two stages.
  constexpr bool DMA = D <= 128;
  constexpr int NST = DMA ? 4 : 2;
  constexpr int SWZ = C::SWZ;
  constexpr int NKS = D / 16;   // 16-deep k-steps of Q.K
  constexpr int NDB = D / 32;   // 32-wide head-dim blocks of O

  __shared__ __attribute__((aligned(16))) unsigned short lds_k[NST][C::TILE];
  __shared__ __attribute__((aligned(16))) unsigned short lds_v[NST][C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
  const int h = lane >> 5;       // half of the wave (MFMA k-slot group)
  const int c = lane & 31;       // MFMA column (query) / row (key, head-dim)
  const int g16 = lane >> 4;     // 16-lane group of the transposing reads
  const int i16 = lane & 15;

  // ---- block -> (query block, head): longest-first, KV groups kept on one XCD
  const int G = a.group;
  const int n_qb = (a.s_q + BM - 1) / BM;
  const int64_t chunks = (int64_t)n_qb * a.bh_kv;
  const int64_t full = (chunks / 8) * 8 * G;
  const int64_t b = blockIdx.x;
  int64_t chunk;
  int g;
  if (b < full) {
    const int64_t x = b % 8, j = b / 8;
    chunk = 8 * (j / G) + x;
    g = (int)(j % G);
  } else {
    chunk = b / G;
    g = (int)(b % G);
  }
  const int rank = (int)(chunk / a.bh_kv);
  const int kvh = (int)(chunk % a.bh_kv);
  const int qblk = a.causal ? n_qb - 1 - rank : rank;
  const int head = kvh * G + g;
  const int q0 = qblk * BM;
  const int off = a.s_k - a.s_q;

  // ---- key range of the block
  const int r_last = min(q0 + BM, a.s_q) - 1;
  int lo = 0, hi = a.s_k;
  if (a.causal) hi = max(0, min(a.s_k, r_last + off + 1));
  if (a.window) lo = max(0, q0 + off - a.window + 1);
  const int t_lo = lo / BN;
  const int n_tiles = hi > lo ? (hi + BN - 1) / BN - t_lo : 0;
  const int64_t kv_base = (int64_t)kvh * a.s_k;

  // ---- Q fragments (B operand of S^T): Qf[ks] = Q[qw0 + c][16 ks + 8 h .. + 8]
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + c;
  const unsigned short* qp = static_cast<const unsigned short*>(a.q) + (int64_t)head * a.s_q * D;
  bf16x8 Qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qi < a.s_q) w = *reinterpret_cast<const u32x4*>(qp + (int64_t)qi * D + 16 * ks + 8 * h);
    Qf[ks] = __builtin_bit_cast(bf16x8, w);
  }

  const unsigned short* kp16 = static_cast<const unsigned short*>(a.k) + kv_base * D;
  const unsigned short* vp16 = static_cast<const unsigned short*>(a.v) + kv_base * D;

  // ---- per-wave state
  f32x16 O[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[db][i] = 0.f;
  float m_run = neg_inf(), l_run = 0.f, mc = 0.f;
  const float c2 = a.scale_log2;
  const float lazy_thr = C::kLazyLog2 / c2;   // raw-score headroom before the max is raised
  const int w_last = qw0 + 31;
  const bool wave_live = qw0 < a.s_q;

  // V^T fragments of 32-key half kb of a tile: vf[s2][db] holds keys kbase + 0..3 and
  // kbase + 8 + 0..3 (kbase = 32 kb + 16 s2 + 4 h) of head-dim 32 db + c, from two transposing
  // LDS reads of the row-major tile
  auto vread = [&](const unsigned short* Vt, int kb, u32x4 (&vf)[2][NDB]) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int krd = 32 * kb + 16 * s2 + 4 * (g16 >> 1) + (i16 >> 2);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + 16 * (g16 & 1) + 4 * (i16 & 3);
        const int e0 = krd * D + 8 * ((d >> 3) ^ swz<SWZ>(krd)) + (d & 7);
        const int e1 = (krd + 8) * D + 8 * ((d >> 3) ^ swz<SWZ>(krd + 8)) + (d & 7);
        const s16x4v r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)((__attribute__((address_space(3))) unsigned short*)Vt + e0));
        const s16x4v r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)((__attribute__((address_space(3))) unsigned short*)Vt + e1));
        const u32x2 w0 = __builtin_bit_cast(u32x2, r0), w1 = __builtin_bit_cast(u32x2, r1);
        vf[s2][db] = u32x4{w0[0], w0[1], w1[0], w1[1]};
      }
    }
  };
  // one V^T fragment (keys 32 kb + 16 s2 + ..., head-dim block db), read just before its MFMA
  // above head_dim 128, where a whole half tile of fragments would not fit the registers
  auto vread1 = [&](const unsigned short* Vt, int kb, int s2, int db) {
    const int krd = 32 * kb + 16 * s2 + 4 * (g16 >> 1) + (i16 >> 2);
    const int d = 32 * db + 16 * (g16 & 1) + 4 * (i16 & 3);
    const int e0 = krd * D + 8 * ((d >> 3) ^ swz<SWZ>(krd)) + (d & 7);
    const int e1 = (krd + 8) * D + 8 * ((d >> 3) ^ swz<SWZ>(krd + 8)) + (d & 7);
    const u32x2 w0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)((__attribute__((address_space(3))) unsigned short*)Vt + e0)));
    const u32x2 w1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)((__attribute__((address_space(3))) unsigned short*)Vt + e1)));
    return u32x4{w0[0], w0[1], w1[0], w1[1]};
  };

  // one tile from LDS stage `stage`; where the stage is a compile-time constant every LDS
  // address is a per-lane base plus an immediate offset
  auto compute = [&](const int t, auto stage) {
    const int st = static_cast<int>(stage);

    const int k0 = (t_lo + t) * BN;
    bool skip = !wave_live;
    if (a.causal && k0 > w_last + off) skip = true;
    if (a.window && k0 + BN - 1 <= qw0 + off - a.window) skip = true;
    if (!skip) {
      const bool need_mask = (k0 + BN > a.s_k) || (a.causal && k0 + BN - 1 > qw0 + off) ||
                             (a.window && k0 <= w_last + off - a.window);
      const unsigned short* Kt = lds_k[st];
      const unsigned short* Vt = lds_v[st];

      // scheduling hint: LLVM's small-GEMM interleave of MFMA with the surrounding instructions
      // (strategy 0; interleaved timings: C5 -2 to -3%, C3 -2.4%; strategies 1-3 and a second hint
      // before the softmax were no better)
      __builtin_amdgcn_iglp_opt(0);
      // S^T of both 32-key halves, two independent MFMA chains: S[kb] lane (c, h) element i holds
      // key 32 kb + 8 (i/4) + 4 h + i%4 (tile-relative) of query qi
      f32x16 S[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int krow = 32 * kb + c;
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Kt + krow * D + 8 * ((2 * ks + h) ^ swz<SWZ>(krow)));
          S[kb] = mfma32_bf16(kf, Qf[ks], S[kb]);
        }

      // V^T fragments of the first 32 keys, read while the softmax runs
      u32x4 vf0[2][NDB];
      if constexpr (D <= 128) vread(Vt, 0, vf0);

      if constexpr (SOPS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int kl0 = k0 + 32 * kb + 4 * h;
          float x[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = S[kb][i];
          apply_score_ops(x, a.sops, [&](int i) { return min(kl0 + 8 * (i / 4) + (i % 4), a.s_k - 1); });
#pragma unroll
          for (int i = 0; i < 16; ++i) S[kb][i] = x[i];
        }
      }

      if (need_mask) {
        // key offset of element i is 8 (i/4) + i%4 past kl0; visible iff lo_i <= it <= hi_i
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int kl0 = k0 + 32 * kb + 4 * h;
          int hi_i = a.s_k - 1 - kl0;
          if (a.causal) hi_i = min(hi_i, qi + off - kl0);
          const int lo_i = a.window ? qi + off - a.window + 1 - kl0 : -0x40000000;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ko = 8 * (i / 4) + (i % 4);
            if (ko > hi_i || ko < lo_i) S[kb][i] = neg_inf();
          }
        }
      }

      // online softmax over the tile's 64 keys with a lazily raised max
      float mx = neg_inf();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[kb][i]);
      mx = max_xor32(mx);
      if (__any(mx - m_run > lazy_thr)) {
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[db][i] *= alpha;
        m_run = m_new;
        mc = m_use * c2;
      }
      // P^T as B operands: k-step (kb, s2) takes the exponentials of S[kb][8 s2 .. 8 s2 + 7].  The
      // row sum adds the fp32 exponentials as a tree (plain adds: v_dot2 does not issue alongside
      // the matrix pipe), so l, and the LSE, are the exact sums of the exponentials.
      u32x4 Pw[2][2];
      float lpair[16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q2 = 0; q2 < 8; ++q2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][2 * q2], c2, -mc));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][2 * q2 + 1], c2, -mc));
          Pw[kb][q2 / 4][q2 % 4] = pack_bf16x2(p0, p1);
          lpair[kb * 8 + q2] = p0 + p1;
        }
#pragma unroll
      for (int st2 = 8; st2 >= 1; st2 >>= 1)
#pragma unroll
        for (int j = 0; j < st2; ++j) lpair[j] += lpair[j + st2];
      l_run += lpair[0];

      // O^T[db] += V^T P^T
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          if constexpr (D > 128) vf0[s2][db] = vread1(Vt, 0, s2, db);
          O[db] = mfma32_bf16(__builtin_bit_cast(bf16x8, vf0[s2][db]), __builtin_bit_cast(bf16x8, Pw[0][s2]), O[db]);
        }
      u32x4 vf1[2][NDB];
      if constexpr (D <= 128) vread(Vt, 1, vf1);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          if constexpr (D > 128) vf1[s2][db] = vread1(Vt, 1, s2, db);
          O[db] = mfma32_bf16(__builtin_bit_cast(bf16x8, vf1[s2][db]), __builtin_bit_cast(bf16x8, Pw[1][s2]), O[db]);
        }
    }

  };

  if constexpr (DMA) {
    // copies of tiles t and t + 1 are issued after a wave's compute of tile t - 2, so after the
    // barrier that ends the compute of tiles t - 4 and t - 3 (their stages), and are waited for
    // before the barrier ending the compute of tiles t - 2 and t - 1; between barriers the waves
    // run two tiles unsynchronised
    // 1-KiB segments per matrix and tile, and per wave: where they do not divide evenly (head_dim
    // 32 and 96) the first waves take SPW each and the rest take what is left, possibly none
    constexpr int SEGS = BN * NC / 64;
    constexpr int SPW = (SEGS + NW - 1) / NW;
    const unsigned short* kp = static_cast<const unsigned short*>(a.k) + kv_base * D;
    const unsigned short* vp = static_cast<const unsigned short*>(a.v) + kv_base * D;
    int crow[SPW], ccol[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int p = 64 * (SPW * wave + j) + lane;   // 16-byte position in the tile
      crow[j] = p / NC;
      ccol[j] = 8 * ((p % NC) ^ swz<SWZ>(p / NC));  // logical chunk stored at that position
    }
    const unsigned lds_k0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned short*)&lds_k[0][0];
    const unsigned lds_v0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned short*)&lds_v[0][0];
    const int last_key = a.s_k - 1;
    // whole tiles: a scalar tile base, a constant per-lane byte offset and scalar LDS segment
    // addresses, so a copy costs no vector instruction; the last, partial tile clamps its rows
    unsigned voff[SPW], seg_k[SPW], seg_v[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      voff[j] = 2u * (unsigned)(crow[j] * D + ccol[j]);
      seg_k[j] = __builtin_amdgcn_readfirstlane(lds_k0 + 1024u * (unsigned)(SPW * wave + j));
      seg_v[j] = __builtin_amdgcn_readfirstlane(lds_v0 + 1024u * (unsigned)(SPW * wave + j));
    }
    auto copy_tile = [&](int t) {
      const int k0 = (t_lo + t) * BN;
      const unsigned st_off = 2u * C::TILE * (unsigned)(t % NST);
      if (k0 + BN <= a.s_k) {
        const unsigned short* kt = kp + (int64_t)k0 * D;
        const unsigned short* vt = vp + (int64_t)k0 * D;
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
          if (SEGS % NW != 0 && SPW * wave + j >= SEGS) break;
          copy16_to_lds(kt, voff[j], seg_k[j] + st_off);
          copy16_to_lds(vt, voff[j], seg_v[j] + st_off);
        }
      } else {
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
          if (SEGS % NW != 0 && SPW * wave + j >= SEGS) break;
          const int64_t row = min(k0 + crow[j], last_key);   // rows past the end repeat the last key
          copy16_to_lds(kp + row * D + ccol[j], seg_k[j] + st_off);
          copy16_to_lds(vp + row * D + ccol[j], seg_v[j] + st_off);
        }
      }
    };
    auto pair = [&](int t, auto s0, auto s1) {
      if (t >= n_tiles) return;
      // The two waves of a SIMD take turns at issue priority, one tile each: left to the
      // oldest-first default, the first wave runs ahead and then idles at the barrier while its
      // partner finishes alone (interleaved timings of the long-context causal workload: -0.9%).
      if (wave >= NW / 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
      compute(t, s0);
      // issued between the two tiles so that they do not compete with tile t's first LDS reads
      if (t + 2 < n_tiles) copy_tile(t + 2);
      if (t + 3 < n_tiles) copy_tile(t + 3);
      if (wave >= NW / 2) __builtin_amdgcn_s_setprio(0);
      else __builtin_amdgcn_s_setprio(1);
      if (t + 1 < n_tiles) compute(t + 1, s1);
      wait_vmcnt0();
      __syncthreads();
    };
    if (n_tiles > 0) copy_tile(0);
    if (n_tiles > 1) copy_tile(1);
    wait_vmcnt0();
    __syncthreads();
    for (int t = 0; t < n_tiles; t += 4) {
      pair(t, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
      pair(t + 2, std::integral_constant<int, 2>{}, std::integral_constant<int, 3>{});
    }
  } else {
    static_assert((BN * NC / 64) % NW == 0, "whole 1-KiB copy segments per wave");
    // head_dim above 128 (4 waves): tile t + 1 is copied global -> LDS directly into the other of
    // two stages while tile t is computed (no staging registers: a 256-wide tile would need 128),
    // each wave waits for its own copies and one barrier per tile publishes them.  The copies
    // follow the layout of the copies above: lane l of segment g fills 16-byte position 64 g + l
    // with the logical chunk that belongs there; the last, partial tile clamps its rows.
    constexpr int SPW = (BN * NC / 64) / NW;      // 1-KiB segments per wave per matrix
    const unsigned lds_k0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned short*)&lds_k[0][0];
    const unsigned lds_v0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned short*)&lds_v[0][0];
    int crow[SPW], ccol[SPW];
    unsigned voff[SPW], seg_k[SPW], seg_v[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int p = 64 * (SPW * wave + j) + lane;
      crow[j] = p / NC;
      ccol[j] = 8 * ((p % NC) ^ swz<SWZ>(p / NC));
      voff[j] = 2u * (unsigned)(crow[j] * D + ccol[j]);
      seg_k[j] = __builtin_amdgcn_readfirstlane(lds_k0 + 1024u * (unsigned)(SPW * wave + j));
      seg_v[j] = __builtin_amdgcn_readfirstlane(lds_v0 + 1024u * (unsigned)(SPW * wave + j));
    }
    auto copy_tile = [&](int t, int st) {
      const int k0 = (t_lo + t) * BN;
      const unsigned st_off = 2u * C::TILE * (unsigned)st;
      if (k0 + BN <= a.s_k) {
        const unsigned short* kt = kp16 + (int64_t)k0 * D;
        const unsigned short* vt = vp16 + (int64_t)k0 * D;
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
          copy16_to_lds(kt, voff[j], seg_k[j] + st_off);
          copy16_to_lds(vt, voff[j], seg_v[j] + st_off);
        }
      } else {
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
          const int64_t row = min(k0 + crow[j], a.s_k - 1);   // rows past the end repeat the last key
          copy16_to_lds(kp16 + row * D + ccol[j], seg_k[j] + st_off);
          copy16_to_lds(vp16 + row * D + ccol[j], seg_v[j] + st_off);
        }
      }
    };
    if (n_tiles > 0) copy_tile(0, 0);
    wait_vmcnt0();
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
      const int st = t & 1;
      if (t + 1 < n_tiles) copy_tile(t + 1, st ^ 1);   // stage st^1 was last read before the previous barrier
      compute(t, st);
      wait_vmcnt0();
      __syncthreads();
    }
  }

  // ---- finalize: O / l (x 2^E for int8), epilogue, store; LSE = sigma m + ln l
  const float l_tot = add_xor32(l_run);
  float inv = l_tot > 0.f ? __fdiv_rn(1.0f, l_tot) : 0.f;
  if (qi < a.s_q) {
    float y[NDB * 16];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) y[16 * db + i] = O[db][i] * inv;
    // element 16 db + i sits at head-dim 32 db + 8 (i / 4) + 4 h + i % 4
    apply_epilogue_all(y, a.epi, [&](int j) { return 32 * (j / 16) + 8 * ((j % 16) / 4) + 4 * h + j % 4; });
    const int64_t row = (int64_t)head * a.s_q + qi;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * h;
        const float* yy = y + 16 * db + 4 * g4;
        if (a.out_bf16) {
          const u32x2 w = {pack_bf16x2(yy[0], yy[1]), pack_bf16x2(yy[2], yy[3])};
          *reinterpret_cast<u32x2*>(static_cast<unsigned short*>(a.out) + row * D + d0) = w;
        } else {
          const f32x4 w = {yy[0], yy[1], yy[2], yy[3]};
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * D + d0) = w;
        }
      }
    if (a.lse && h == 0) a.lse[row] = l_tot > 0.f ? m_run * a.scale + logf(l_tot) : neg_inf();
  }
}


template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t st, const char** name) {
  const int64_t n_qb = (a.s_q + Cfg<D>::BM - 1) / Cfg<D>::BM;
  const int64_t blocks = n_qb * a.bh_q;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.sops.n > 0) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true>), dim3((unsigned)blocks), dim3(64 * Cfg<D>::NW), 0, st, a);
    *name = "prefill_bf16_sops";
  } else {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, false>), dim3((unsigned)blocks), dim3(64 * Cfg<D>::NW), 0, st, a);
    *name = "prefill_bf16";
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, int32_t d, hipStream_t stream, const char** name) {
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
