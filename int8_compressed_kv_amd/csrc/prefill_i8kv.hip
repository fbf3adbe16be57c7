// Attention forward on gfx950 MFMA over the per-token int8 KV cache, for bf16 Q (the plain
// bf16 variant is prefill_bf16.hip, which shares this layout and schedule).
//
// Method: FlashAttention-2 style tiled forward with an online softmax (fkl.flash_attention
// PR, Summary: FA-2 forward, fp32 accumulation, compressed int8 KV dequantized inside q.k and
// p.v; Foundry attention/ README, References: the online-softmax recurrence).  For each key
// tile, with running row max m, running sum l and accumulator O:
//   S = sigma Q (k_s K8)^T (masked) ; m' = max(m, rowmax S) ; P = exp(S - m') ;
//   l = exp(m - m') l + rowsum P ; O = exp(m - m') O + P (v_s V8).
// Finally O / l, the epilogue ops in fp32, and the store.
//
// gfx950 mapping
//   * A workgroup is 8 waves = 256 query rows (4 waves for head_dim > 128, whose fragments
//     need the whole register file); each wave owns 32 rows and keeps their Q fragments in
//     registers.
//   * Dequantization happens once per workgroup and tile, on the way into the operand tiles in
//     LDS: K~ = fp16(k) * fp16(k_s 2^-Ek) and V~ = fp16(v) * fp16(v_s 2^-Ev) (codes are exact in
//     fp16; one packed fp16 multiply per pair), where 2^-Ek, 2^-Ev put the block's largest scale
//     in [128, 256).  Q is held in fp16 as Q 2^-Eq with the row's largest |q| in [2^14, 2^15)
//     (bf16 -> fp16 exact there); the row's exp2-domain factor absorbs 2^(Eq + Ek), and O is
//     multiplied by 2^Ev at the end.  The compressed cache is never expanded in global memory.
//   * head_dim 64 / 128: the codes and scales of a tile are copied global -> LDS directly into
//     four staging stages (tile t + 3 in flight while tile t is computed) and converted into two
//     operand stages; other head dims stage the codes through registers.  One barrier per tile.
//   * Operand tiles of 64 keys are row-major in LDS, 16-byte chunks XOR-swizzled by row so that
//     both operand reads below are free of bank conflicts.
//   * S^T = K~ Q~^T (keys = MFMA rows, queries = columns) on v_mfma_f32_32x32x16_f16: each
//     query's scores sit in one lane pair, so the row max needs one exchange, and P^T (fp16) in
//     the accumulator layout is already the B operand of O^T += V~^T P^T.  The V~^T operand
//     (8 keys of one head-dim column per lane) comes from two transposing LDS reads
//     (ds_read_b64_tr_b16) of the row-major tile.
//   * The running max is only raised when a row's tile max exceeds it by more than 2^8 in the
//     exp2 domain; otherwise the stale max is kept (O and l stay mutually consistent, the O
//     rescale is skipped) and P stays below 2^8, inside fp16.
//   * Tiles wholly outside a wave's causal / window band are skipped; element masks are
//     applied only on boundary tiles.  Blocks run longest-first under causal masks and are
//     dealt to the 8 XCDs so that the G query heads sharing a KV head stay on one XCD.
#include <type_traits>

#include "device_common.hpp"

namespace fa {
namespace {

typedef short s16x4v __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) s16x4v lds_s16x4;

// dword 3 of a raw buffer resource on gfx9-family parts (32-bit data format; no swizzle)
constexpr int kBufferFlags = 0x00020000;

template <int D>
struct Cfg {
  static constexpr int NW = D <= 128 ? 8 : 4;    // waves per workgroup (2 or 1 per SIMD)
  static constexpr int BM = 32 * NW;             // query rows per workgroup
  static constexpr int BN = 64;                  // keys per LDS tile
  static constexpr int NC = D / 8;               // 16-byte chunks per row
  static constexpr int TILE = BN * D;            // 16-bit elements per K or V tile
  static constexpr int SWZ = (NC % 16 == 0) ? 16 : (NC % 8 == 0) ? 8 : 4;   // swizzle span
  static constexpr int CH = (BN * NC + 64 * NW - 1) / (64 * NW);   // chunks per thread per matrix
  static constexpr float kLazyLog2 = 8.0f;       // stale-max headroom, exp2 domain
};

// chunk permutation of row r: rows r..r+3 land in disjoint 4-chunk groups, 16 rows in 16
// distinct chunks.
template <int SWZ>
__device__ __forceinline__ int swz(int r) {
  return (((r & 3) << 2) | ((r >> 2) & 3)) & (SWZ - 1);
}

// Direct global -> LDS copies (no output registers: the data goes to LDS, so the compiler adds
// no wait before later LDS reads; the kernel waits for its own copies before the barrier that
// publishes them).  16 bytes per lane land at LDS byte address lds + 16 l, 4 bytes at lds + 4 l.
__device__ __forceinline__ void copy16_to_lds(const void* src, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src)
               : "memory", "m0");
}
__device__ __forceinline__ void copy16_to_lds(const void* sbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
__device__ __forceinline__ void copy4_to_lds(const void* src, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(src)
               : "memory", "m0");
}
// s_waitcnt vmcnt(N) for N < 16, the other counters unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
}

template <int D, bool SOPS>
__global__ __launch_bounds__(64 * Cfg<D>::NW, 1) void prefill_i8kv_kernel(PrefillArgs a) {
  using C = Cfg<D>;
  constexpr int NW = C::NW, BM = C::BM, BN = C::BN, NC = C::NC, CH = C::CH;
  constexpr int SWZ = C::SWZ;
  constexpr int NKS = D / 16;   // 16-deep k-steps of Q.K
  constexpr int NDB = D / 32;   // 32-wide head-dim blocks of O
  // head_dim 64 and 128: int8 tiles arrive by direct global -> LDS copies into four staging
  // stages and are converted once per workgroup into the two operand stages; other head dims
  // stage the codes through registers.
  constexpr bool DMA = D == 64 || D == 128;
  constexpr int SEGS = BN * D / 1024;              // 1-KiB segments of one int8 tile
  constexpr int SPW = DMA ? 2 * SEGS / NW : 1;     // K and V segments copied per wave per tile
  constexpr int NS8 = DMA ? 4 : 1;
  constexpr int Q8 = DMA ? 2 * BN * D : 16;        // bytes per staging stage: K codes, then V codes

  __shared__ __attribute__((aligned(16))) unsigned short lds_k[2][C::TILE];
  __shared__ __attribute__((aligned(16))) unsigned short lds_v[2][C::TILE];
  __shared__ __attribute__((aligned(16))) int8_t lds_q8[NS8][Q8];
  __shared__ __attribute__((aligned(16))) float lds_s8[NS8][DMA ? 2 * BN : 4];
  __shared__ float lds_red[2][NW];

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

  const int8_t* kp8 = static_cast<const int8_t*>(a.k) + kv_base * D;
  const int8_t* vp8 = static_cast<const int8_t*>(a.v) + kv_base * D;
  const int last_key = a.s_k - 1;

  // Staging order of the 16-code chunks of a tile (head_dim 64 / 128): position pos holds chunk
  // staged_chunk(pos) of row staged_row(pos).  Within a block of 8 rows, consecutive positions run
  // over 4 chunks of row g, the same 4 chunks of row g + 4, (at head_dim 128) the next 4 chunks
  // of both rows, then the next g.  So any 8 threads converting consecutive positions cover two
  // rows whose swizzles differ in bit 0 (row bit 2) and 4 chunks of each: the 8 16-byte operand
  // writes of such a group land in 8 distinct chunk positions modulo 8, which keeps them in
  // distinct banks whether the LDS serves 8 or 16 lanes of a 16-byte write at a time, while
  // their reads of the staging stage stay contiguous.
  constexpr int NCR = D / 16;   // 16-code chunks per row
  auto staged_row = [&](int pos) __attribute__((always_inline)) {
    const int q = pos % (8 * NCR);
    return 8 * (pos / (8 * NCR)) + q / (2 * NCR) + 4 * ((q >> 2) & 1);
  };
  auto staged_chunk = [&](int pos) __attribute__((always_inline)) {
    const int q = pos % (8 * NCR);
    return 4 * ((q >> 3) % (NCR / 4)) + (q & 3);
  };

  // ---- direct global -> LDS staging (head_dim 64 / 128)
  // Per tile: wave w copies K/V segments SPW w .. SPW w + SPW - 1 (segment gs < SEGS is K
  // segment gs, else V segment gs - SEGS; lane l of a segment brings the 16 codes of staging
  // position 64 seg + l), wave 0 the 64 k scales and wave 1 the 64 v scales.
  // Tiles 0 .. 2 are copied in the prologue; tile t + 3's copies are issued in iteration t,
  // after the barrier that ended the conversion
  // of tile t - 1 (the last reader of that staging stage, in iteration t - 2); each wave waits
  // for its own copies of tile t + 3 at the end of iteration t + 1, before the barrier that
  // precedes their conversion in iteration t + 2.
  const unsigned q8_0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) int8_t*)&lds_q8[0][0];
  const unsigned s8_0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) float*)&lds_s8[0][0];
  int crow[SPW], ccol[SPW];
  unsigned voff[SPW], seg_lds[SPW];
  const int8_t* cbase[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int gs = SPW * wave + j;
    const int mat = gs / SEGS, seg = gs % SEGS;
    const int pos = 64 * seg + lane;            // 16-byte staging position within the matrix
    crow[j] = staged_row(pos);
    ccol[j] = 16 * staged_chunk(pos);
    voff[j] = (unsigned)(crow[j] * D + ccol[j]);
    cbase[j] = mat ? vp8 : kp8;
    seg_lds[j] = __builtin_amdgcn_readfirstlane(q8_0 + (unsigned)(mat * BN * D + 1024 * seg));
  }
  const float* sc_src = wave == 0 ? a.k_scale : a.v_scale;
  const unsigned sc_lds = s8_0 + (wave == 0 ? 0u : 4u * BN);
  auto copy_tile = [&](int t) __attribute__((always_inline)) {
    const int k0 = (t_lo + t) * BN;
    const unsigned st_off = (unsigned)(Q8 * (t % NS8));
    if (k0 + BN <= a.s_k) {
#pragma unroll
      for (int j = 0; j < SPW; ++j) copy16_to_lds(cbase[j] + (int64_t)k0 * D, voff[j], seg_lds[j] + st_off);
    } else {
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int64_t row = min(k0 + crow[j], last_key);   // rows past the end repeat the last key
        copy16_to_lds(cbase[j] + row * D + ccol[j], seg_lds[j] + st_off);
      }
    }
    if (wave < 2)
      copy4_to_lds(sc_src + kv_base + min(k0 + lane, last_key), sc_lds + (unsigned)(4 * 2 * BN * (t % NS8)));
  };
  // the copies of the latest tile may stay in flight; those of the one before must have landed
  auto wait_all_but_latest = [&]() __attribute__((always_inline)) {
    if (wave < 2) wait_vmcnt<SPW + 1>();
    else wait_vmcnt<SPW>();
  };

  // ---- prologue: the first three tiles' copies, the Q rows and the block's scales are all issued
  // before the first wait, so a block starts after one memory latency rather than one per step
  if constexpr (DMA) {
    if (n_tiles > 0) copy_tile(0);
    if (n_tiles > 1) copy_tile(1);
    if (n_tiles > 2) copy_tile(2);
  }
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + c;
  const unsigned short* qp = static_cast<const unsigned short*>(a.q) + (int64_t)head * a.s_q * D;
  u32x4 qraw[NKS];
  {
    const int64_t qrow = min(qi, a.s_q - 1);   // rows past the end load the last row, then read as 0
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qraw[ks] = *reinterpret_cast<const u32x4*>(qp + qrow * D + 16 * ks + 8 * h);
  }

  // ---- int8: power-of-two normalisers of the block's scales.  K~ = fp16(k) * fp16(k_s 2^-Ek) and
  // V~ = fp16(v) * fp16(v_s 2^-Ev), with 2^-Ek, 2^-Ev putting the largest scale over the keys of
  // the block's tiles in [128, 256), so that every |K~|, |V~| <= 127 * 256 stays inside fp16
  // (also on masked keys, whose P = 0 must not meet an infinite V~).  Eight scales of each matrix
  // per thread are loaded together (indices clamped to the range: repeats leave the max as is).
  float mk = 0.f, mv = 0.f;
  const int key_end = min(a.s_k, (t_lo + n_tiles) * BN);
  for (int j0 = t_lo * BN; j0 < key_end; j0 += 8 * 64 * NW) {
    float kk[8], vv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(j0 + tid + 64 * NW * u, key_end - 1);
      kk[u] = a.k_scale[kv_base + j];
      vv[u] = a.v_scale[kv_base + j];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      mk = fmaxf(mk, kk[u]);
      mv = fmaxf(mv, vv[u]);
    }
  }
#pragma unroll
  for (int o2 = 32; o2 >= 1; o2 >>= 1) {
    mk = fmaxf(mk, __shfl_xor(mk, o2, 64));
    mv = fmaxf(mv, __shfl_xor(mv, o2, 64));
  }
  if (lane == 0) {
    lds_red[0][wave] = mk;
    lds_red[1][wave] = mv;
  }
  if constexpr (DMA) wait_vmcnt<0>();   // the first tiles' copies, published by the barrier
  __syncthreads();
  mk = 0.f;
  mv = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mk = fmaxf(mk, lds_red[0][w]);
    mv = fmaxf(mv, lds_red[1][w]);
  }
  int ek = 0, ev = 0;
  if (mk > 0.f) (void)frexpf(mk, &ek);   // mk = f * 2^ek, f in [0.5, 1)
  if (mv > 0.f) (void)frexpf(mv, &ev);
  ek = max(ek, -60);
  ev = max(ev, -60);
  const float ks_norm = ldexpf(1.f, 8 - ek);
  const float vs_norm = ldexpf(1.f, 8 - ev);
  const float vs_unnorm = ldexpf(1.f, ev - 8);

  // ---- Q fragments (B operand of S^T) in fp16: Qf[ks] = Q~[qw0 + c][16 ks + 8 h .. + 8], Q~ = Q 2^-Eq
  // with 2^-Eq putting the row's largest |q| in [2^14, 2^15) (bf16 -> fp16 is then exact down to
  // 2^-28 of that largest value).  S~ = Q~ K~^T is S / (2^-Eq 2^-Ek): the row's exp2-domain factor
  // c2row absorbs both powers of two.
  float qmax = 0.f;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (qi >= a.s_q) qraw[ks] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      qmax = fmaxf(qmax, fmaxf(fabsf(__uint_as_float(qraw[ks][e2] << 16)), fabsf(__uint_as_float(qraw[ks][e2] & 0xffff0000u))));
  }
  qmax = max_xor32(qmax);
  int eq = 0;
  if (qmax > 0.f) (void)frexpf(qmax, &eq);
  eq = max(eq, -60);
  const float q_norm = ldexpf(1.f, 15 - eq);
  f16x8 Qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    u32x4 w;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      w[e2] = pack_f16x2(__uint_as_float(qraw[ks][e2] << 16) * q_norm, __uint_as_float(qraw[ks][e2] & 0xffff0000u) * q_norm);
    Qf[ks] = __builtin_bit_cast(f16x8, w);
  }
  // S = S~ 2^(eq - 15) 2^(ek - 8)
  const int es = (eq - 15) + (ek - 8);

  // ---- per-wave state
  f32x16 O[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[db][i] = 0.f;
  float m_run = neg_inf(), l_run = 0.f, mc = 0.f;   // m_run in units of S~
  const float c2 = ldexpf(a.scale_log2, es);       // exp2-domain factor of S~ for this row
  const float lazy_thr = C::kLazyLog2 / c2;        // S~ headroom before the max is raised
  const int w_last = qw0 + 31;
  const bool wave_live = qw0 < a.s_q;

  // V^T fragments of 32-key half kb of a tile: vf[s2][db] holds keys kbase + 0..3 and
  // kbase + 8 + 0..3 (kbase = 32 kb + 16 s2 + 4 h) of head-dim 32 db + c, from two transposing
  // LDS reads of the row-major tile
  auto vread = [&](const unsigned short* Vt, int kb, u32x4 (&vf)[2][NDB]) __attribute__((always_inline)) {
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
  auto vread1 = [&](const unsigned short* Vt, int kb, int s2, int db) __attribute__((always_inline)) {
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

  // one tile from operand stage `stage` (K~, V~ in fp16)
  auto compute = [&](const int t, auto stage) __attribute__((always_inline)) {
    const int st = static_cast<int>(stage);
    const int k0 = (t_lo + t) * BN;
    bool skip = !wave_live;
    if (a.causal && k0 > w_last + off) skip = true;
    if (a.window && k0 + BN - 1 <= qw0 + off - a.window) skip = true;
    if (skip) return;
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
        const f16x8 kf = *reinterpret_cast<const f16x8*>(Kt + krow * D + 8 * ((2 * ks + h) ^ swz<SWZ>(krow)));
        S[kb] = mfma32_f16(kf, Qf[ks], S[kb]);
      }

    // V^T fragments of the first 32 keys, read while the softmax runs
    u32x4 vf0[2][NDB];
    if constexpr (D <= 128) vread(Vt, 0, vf0);

    if constexpr (SOPS) {
      // the ops act on S = S~ 2^es (exact power-of-two rescalings either way)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kl0 = k0 + 32 * kb + 4 * h;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = ldexpf(S[kb][i], es);
        apply_score_ops(x, a.sops, [&](int i) { return min(kl0 + 8 * (i / 4) + (i % 4), last_key); });
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kb][i] = ldexpf(x[i], -es);
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
    float mx2 = neg_inf();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx2 = fmaxf(mx2, S[kb][i]);
    mx2 = max_xor32(mx2);
    if (__any(mx2 - m_run > lazy_thr)) {
      const float m_new = fmaxf(m_run, mx2);
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
    // P^T in fp16 as B operands: k-step (kb, s2) takes S[kb][8 s2 .. 8 s2 + 7].  The row sum adds
    // the fp32 exponentials as a tree, so l is their exact fp32 sum.
    u32x4 Pw[2][2];
    float lpair[16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q2 = 0; q2 < 8; ++q2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][2 * q2], c2, -mc));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][2 * q2 + 1], c2, -mc));
        Pw[kb][q2 / 4][q2 % 4] = pack_f16x2(p0, p1);
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
        O[db] = mfma32_f16(__builtin_bit_cast(f16x8, vf0[s2][db]), __builtin_bit_cast(f16x8, Pw[0][s2]), O[db]);
      }
    u32x4 vf1[2][NDB];
    if constexpr (D <= 128) vread(Vt, 1, vf1);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if constexpr (D > 128) vf1[s2][db] = vread1(Vt, 1, s2, db);
        O[db] = mfma32_f16(__builtin_bit_cast(f16x8, vf1[s2][db]), __builtin_bit_cast(f16x8, Pw[1][s2]), O[db]);
      }
  };

  // converted 16-byte chunk (8 values) of row r, logical chunk lc, into operand stage st
  auto put_chunks = [&](unsigned short* dst, int r, int lc, u32x4 w) __attribute__((always_inline)) {
    *reinterpret_cast<u32x4*>(dst + r * D + 8 * (lc ^ swz<SWZ>(r))) = w;
  };
  // 4 codes -> 4 fp16 values code * s (s: the row's scale times its normaliser, rounded to fp16).
  // The codes become exact fp16 as in i8x4_to_f16x4 (byte + 128 in the low mantissa bits of 1024,
  // minus 1152), written out here: routed through that helper's u32x2 result, the packed
  // multiply that follows lost its second half in hipcc (ROCm 7.2) -- both words came out equal.
  auto scaled4 = [&](unsigned codes, f16x2 s2v) __attribute__((always_inline)) {
    const unsigned u = codes ^ 0x80808080u;
    const f16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const f16x2 lo = (__builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u)) + bias) * s2v;
    const f16x2 hi = (__builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x05030402u)) + bias) * s2v;
    return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
  };
  auto half2_of = [&](float sv) __attribute__((always_inline)) {
    const _Float16 hv = (_Float16)sv;
    return f16x2{hv, hv};
  };

  if constexpr (DMA) {
    // staging stage s8 -> operand stage st: thread tid converts chunk tid + 64 NW u of the 2 BN D / 16
    // chunks (K chunks first), scaling each row by its scale times the block normaliser
    auto convert = [&](auto s8, auto stage) __attribute__((always_inline)) {
      constexpr int NCH8 = 2 * BN * D / 16;
      __builtin_amdgcn_iglp_opt(0);   // the same interleave hint (1-2% on C3, both orders timed)
#pragma unroll
      for (int u = 0; u < NCH8 / (64 * NW); ++u) {
        const int ci = tid + 64 * NW * u;
        const bool is_v = ci >= NCH8 / 2;
        const int cm = is_v ? ci - NCH8 / 2 : ci;
        const u32x4 w = *reinterpret_cast<const u32x4*>(&lds_q8[static_cast<int>(s8)][16 * ci]);
        const int r = staged_row(cm), lc = 2 * staged_chunk(cm);
        const f16x2 sr = half2_of(lds_s8[static_cast<int>(s8)][(is_v ? BN : 0) + r] * (is_v ? vs_norm : ks_norm));
        const u32x2 x0 = scaled4(w[0], sr), x1 = scaled4(w[1], sr);
        const u32x2 x2 = scaled4(w[2], sr), x3 = scaled4(w[3], sr);
        unsigned short* dst = is_v ? lds_v[static_cast<int>(stage)] : lds_k[static_cast<int>(stage)];
        put_chunks(dst, r, lc, u32x4{x0[0], x0[1], x1[0], x1[1]});
        put_chunks(dst, r, lc + 1, u32x4{x2[0], x2[1], x3[0], x3[1]});
      }
    };
    // iteration t: compute tile t, convert tile t + 1, copy tile t + 3, wait for tile t + 2, barrier
    auto iter = [&](int t, auto st, auto st1, auto s81) __attribute__((always_inline)) {
      if (t >= n_tiles) return;
      compute(t, st);
      // unconditional, so that it shares a basic block with the end of compute and the scheduler
      // can interleave its vector work with the last P.V products (C3: -0.9%); after the last tile
      // it converts a staging stage into an operand stage that nothing reads
      convert(s81, st1);
      if (t + 3 < n_tiles) {
        copy_tile(t + 3);
        wait_all_but_latest();
      } else {
        wait_vmcnt<0>();
      }
      __syncthreads();
    };
    // tiles 0 .. 2 landed before the prologue's barrier
    if (n_tiles > 0) {
      convert(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
      __syncthreads();
    }
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    for (int t = 0; t < n_tiles; t += 4) {
      iter(t, I0{}, I1{}, I1{});
      iter(t + 1, I1{}, I0{}, I2{});
      iter(t + 2, I0{}, I1{}, I3{});
      iter(t + 3, I1{}, I0{}, I0{});
    }
  } else {
    // ---- staging through registers: tile rows k0 .. k0 + 63 are read as 8-byte chunks of codes
    // with buffer loads (a scalar resource per tile, based at row k0 and ending at the head's last
    // key, plus a constant per-lane offset; rows past the end read as zero and are masked in the
    // softmax), double-buffered in registers with the scales of their rows, converted (K~, V~)
    // and written to LDS at row r, physical chunk lc ^ swz(r).
    u32x2 kreg[CH], vreg[CH];
    float ksr[CH], vsr[CH];
    int soff[CH], srow[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int idx = min(tid + 64 * NW * u, BN * NC - 1);
      soff[u] = (idx / NC) * D + 8 * (idx % NC);
      srow[u] = idx / NC;
    }
    auto load_tile = [&](int t) __attribute__((always_inline)) {
      const int k0 = (t_lo + t) * BN;
      const int64_t rem = (int64_t)(a.s_k - k0) * D;
      const int nrec = (int)(rem < 0x7fffffff ? rem : 0x7fffffff);
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(kp8 + (int64_t)k0 * D), 0, nrec, kBufferFlags);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(vp8 + (int64_t)k0 * D), 0, nrec, kBufferFlags);
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        kreg[u] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk, soff[u], 0, 0));
        vreg[u] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, soff[u], 0, 0));
        const int64_t key = kv_base + min(k0 + srow[u], last_key);
        ksr[u] = a.k_scale[key];
        vsr[u] = a.v_scale[key];
      }
    };
    auto store_tile = [&](int st) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int idx = tid + 64 * NW * u;
        if (BN * NC % (64 * NW) == 0 || idx < BN * NC) {
          const int r = idx / NC, lc = idx % NC;
          const f16x2 sk = half2_of(ksr[u] * ks_norm), sv = half2_of(vsr[u] * vs_norm);
          const u32x2 k0v = scaled4(kreg[u][0], sk), k1v = scaled4(kreg[u][1], sk);
          const u32x2 v0v = scaled4(vreg[u][0], sv), v1v = scaled4(vreg[u][1], sv);
          put_chunks(lds_k[st], r, lc, u32x4{k0v[0], k0v[1], k1v[0], k1v[1]});
          put_chunks(lds_v[st], r, lc, u32x4{v0v[0], v0v[1], v1v[0], v1v[1]});
        }
      }
    };
    // the global loads of tile t+1 are in flight while tile t is computed
    if (n_tiles > 0) {
      load_tile(0);
      store_tile(0);
    }
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
      const int st = t & 1;
      if (t + 1 < n_tiles) load_tile(t + 1);
      compute(t, st);
      if (t + 1 < n_tiles) store_tile(st ^ 1);   // stage st^1 was last read before the previous barrier
      __syncthreads();
    }
  }

  // ---- finalize: O / l x 2^Ev, epilogue, store; LSE = sigma m + ln l (m in units of S~)
  const float l_tot = add_xor32(l_run);
  float inv = l_tot > 0.f ? __fdiv_rn(1.0f, l_tot) : 0.f;
  inv *= vs_unnorm;
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
    if (a.lse && h == 0) a.lse[row] = l_tot > 0.f ? m_run * ldexpf(a.scale, es) + logf(l_tot) : neg_inf();
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t st, const char** name) {
  const int64_t n_qb = (a.s_q + Cfg<D>::BM - 1) / Cfg<D>::BM;
  const int64_t blocks = n_qb * a.bh_q;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.sops.n > 0)
    hipLaunchKernelGGL((prefill_i8kv_kernel<D, true>), dim3((unsigned)blocks), dim3(64 * Cfg<D>::NW), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_i8kv_kernel<D, false>), dim3((unsigned)blocks), dim3(64 * Cfg<D>::NW), 0, st, a);
  *name = a.sops.n > 0 ? "prefill_bf16_i8kv_sops" : "prefill_bf16_i8kv";
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_i8kv(const PrefillArgs& a, int32_t d, hipStream_t stream, const char** name) {
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
