// bf16 attention forward on gfx950 MFMA, for bf16 Q with bf16 K/V or with the int8
// per-token KV cache.
//
// Method: FlashAttention-2 style tiled forward with an online softmax (fkl.flash_attention
// PR, Summary: FA-2 forward, fp32 accumulation, compressed int8 KV dequantized inside q.k and
// p.v; Foundry attention/ README, References: the online-softmax recurrence).  For each key
// tile, with running row max m, running sum l and accumulator O:
//   S = sigma * Q K^T (masked) ; m' = max(m, rowmax S) ; P = exp(S - m') ;
//   l = exp(m - m') l + rowsum P ; O = exp(m - m') O + P V.
// Finally O / l, the epilogue ops in fp32, and the store.
//
// gfx950 mapping
//   * One workgroup = 4 waves; each wave owns 32*QB query rows (QB = 2 for head_dim <= 128)
//     and keeps its Q fragments in registers for the whole kernel.
//   * K and V tiles of 64 keys are staged through LDS with double buffering: the global loads
//     of tile t+1 are issued before the MFMAs of tile t and written to LDS after them, one
//     barrier per tile.  V is transposed on the way into LDS (keys contiguous per head-dim
//     row) so the P.V operand is two 8-byte LDS reads per lane.
//   * The transposed product S^T = K Q^T (keys = MFMA rows, queries = columns) puts each
//     query's scores in one lane pair; the row max needs one exchange between the pair, and
//     P^T in the MFMA accumulator layout is already the B operand of O^T += V^T P^T.
//   * The running max is only raised when a row's tile max exceeds it by more than 2^8 (in
//     the exp2 domain); otherwise the stale max is kept, which leaves O and l mutually
//     consistent and skips the O rescale.  P then stays below 2^8.
//   * int8 K/V: codes are converted exactly to bf16 (K) and fp16 (V) while staging into LDS
//     (the compressed cache is never expanded in global memory).  The per-token scale k_s is
//     applied to S in registers; v_s is folded into P, which is rounded to fp16 for the fp16
//     MFMA, after a power-of-two normalisation (2^-E, E from the largest v_s the block
//     visits) that keeps P * v_s inside fp16 range; O is multiplied back by 2^E at the end.
//   * Tiles wholly outside a wave's causal / window band are skipped; per-element masks are
//     applied only on boundary tiles.  Blocks are ordered longest-first for causal masks and
//     dealt to the 8 XCDs so that the G query heads sharing a KV head stay on one XCD.
#include "device_common.hpp"

namespace fa {
namespace {

template <int D>
struct Cfg {
  static constexpr int QB = D <= 128 ? 2 : 1;   // 32-row query blocks per wave
  static constexpr int NW = 4;                  // waves per workgroup
  static constexpr int BM = NW * 32 * QB;       // query rows per workgroup
  static constexpr int BN = 64;                 // keys per tile
  static constexpr int KST = D + 8;             // K row stride in LDS (16-bit elements)
  static constexpr int VST = BN + 4;            // V^T row stride in LDS (16-bit elements)
  static constexpr int K_ELEMS = BN * KST;
  static constexpr int V_ELEMS = D * VST;
  static constexpr int KCH = D / 32;            // K 8-element chunks per thread per tile
  static constexpr int VGRP = (2 * D + 255) / 256;  // V 4x8 groups per thread per tile
  static constexpr float kLazyLog2 = 8.0f;      // stale-max headroom, exp2 domain
};

__device__ __forceinline__ unsigned gather_byte(unsigned w0, unsigned w1, unsigned w2, unsigned w3, int b) {
  const unsigned s = 8u * b;
  return ((w0 >> s) & 0xffu) | (((w1 >> s) & 0xffu) << 8) | (((w2 >> s) & 0xffu) << 16) |
         (((w3 >> s) & 0xffu) << 24);
}

template <int D, bool KV_I8>
__global__ __launch_bounds__(256, 1) void prefill_bf16_kernel(PrefillArgs a) {
  using C = Cfg<D>;
  constexpr int QB = C::QB, BM = C::BM, BN = C::BN, KST = C::KST, VST = C::VST;
  constexpr int NKS = D / 16;   // 16-deep k-steps of Q.K
  constexpr int NDB = D / 32;   // 32-wide head-dim blocks of O

  __shared__ __attribute__((aligned(16))) unsigned short lds_k[2][C::K_ELEMS];
  __shared__ __attribute__((aligned(16))) unsigned short lds_v[2][C::V_ELEMS];
  __shared__ __attribute__((aligned(16))) float lds_ks[2][KV_I8 ? BN : 1];
  __shared__ __attribute__((aligned(16))) float lds_vs[2][KV_I8 ? BN : 1];
  __shared__ float lds_red[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int c = lane & 31;

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

  // ---- int8: power-of-two normalisation for P * v_s (largest v_s over [lo, hi))
  float vs_norm = 1.f, vs_unnorm = 1.f;
  if (KV_I8) {
    float mx = 0.f;
    for (int j = lo + tid; j < hi; j += 256) mx = fmaxf(mx, a.v_scale[kv_base + j]);
#pragma unroll
    for (int o2 = 32; o2 >= 1; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2, 64));
    if (lane == 0) lds_red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(lds_red[0], lds_red[1]), fmaxf(lds_red[2], lds_red[3]));
    int e = 0;
    if (mx > 0.f) (void)frexpf(mx, &e);   // mx = f * 2^e, f in [0.5, 1)
    vs_norm = ldexpf(1.f, -e);
    vs_unnorm = ldexpf(1.f, e);
  }

  // ---- Q fragments: Qf[qb][ks] = Q[row][16 ks + 8 h .. + 8], row = q0 + 32 QB wave + 32 qb + c
  const int qw0 = q0 + 32 * QB * wave;
  const unsigned short* qp = static_cast<const unsigned short*>(a.q) + (int64_t)head * a.s_q * D;
  bf16x8 Qf[QB][NKS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + 32 * qb + c;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row < a.s_q) w = *reinterpret_cast<const u32x4*>(qp + (int64_t)row * D + 16 * ks + 8 * h);
      Qf[qb][ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- staging registers and helpers
  const unsigned short* kp16 = static_cast<const unsigned short*>(a.k) + kv_base * D;
  const unsigned short* vp16 = static_cast<const unsigned short*>(a.v) + kv_base * D;
  const int8_t* kp8 = static_cast<const int8_t*>(a.k) + kv_base * D;
  const int8_t* vp8 = static_cast<const int8_t*>(a.v) + kv_base * D;

  u32x4 kreg[C::KCH];           // bf16: 8 elements; int8: 8 codes in [0..1]
  u32x4 vreg[C::VGRP][4];       // bf16: 4 keys x 8 elements; int8: 4 keys x 8 codes in [0..1]
  float sreg = 0.f;             // int8: one scale value per thread (threads < 128)

  auto load_tile = [&](int t) {
    const int k0 = (t_lo + t) * BN;
#pragma unroll
    for (int u = 0; u < C::KCH; ++u) {
      const int idx = tid + 256 * u;
      const int r = idx / (D / 8), c8 = idx % (D / 8);
      u32x4 w = {0u, 0u, 0u, 0u};
      if (k0 + r < a.s_k) {
        if (KV_I8) {
          const u32x2 w2 = *reinterpret_cast<const u32x2*>(kp8 + (int64_t)(k0 + r) * D + 8 * c8);
          w[0] = w2[0];
          w[1] = w2[1];
        } else {
          w = *reinterpret_cast<const u32x4*>(kp16 + (int64_t)(k0 + r) * D + 8 * c8);
        }
      }
      kreg[u] = w;
    }
#pragma unroll
    for (int u = 0; u < C::VGRP; ++u) {
      const int grp = tid + 256 * u;
      const int kq = grp / (D / 8), dc = grp % (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = k0 + 4 * kq + r;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (grp < 2 * D && j < a.s_k) {
          if (KV_I8) {
            const u32x2 w2 = *reinterpret_cast<const u32x2*>(vp8 + (int64_t)j * D + 8 * dc);
            w[0] = w2[0];
            w[1] = w2[1];
          } else {
            w = *reinterpret_cast<const u32x4*>(vp16 + (int64_t)j * D + 8 * dc);
          }
        }
        vreg[u][r] = w;
      }
    }
    if (KV_I8 && tid < 2 * BN) {
      const int j = k0 + (tid % BN);
      sreg = 0.f;
      if (j < a.s_k) sreg = tid < BN ? a.k_scale[kv_base + j] : a.v_scale[kv_base + j] * vs_norm;
    }
  };

  auto store_tile = [&](int stage) {
    unsigned short* ks_ = lds_k[stage];
    unsigned short* vs_ = lds_v[stage];
#pragma unroll
    for (int u = 0; u < C::KCH; ++u) {
      const int idx = tid + 256 * u;
      const int r = idx / (D / 8), c8 = idx % (D / 8);
      u32x4 w = kreg[u];
      if (KV_I8) {
        const u32x2 lo2 = i8x4_to_bf16x4(w[0]);
        const u32x2 hi2 = i8x4_to_bf16x4(w[1]);
        w[0] = lo2[0];
        w[1] = lo2[1];
        w[2] = hi2[0];
        w[3] = hi2[1];
      }
      *reinterpret_cast<u32x4*>(ks_ + r * KST + 8 * c8) = w;
    }
#pragma unroll
    for (int u = 0; u < C::VGRP; ++u) {
      const int grp = tid + 256 * u;
      if (grp < 2 * D) {
        const int kq = grp / (D / 8), dc = grp % (D / 8);
        if (KV_I8) {
          // 4 keys x 8 codes -> for each of the 8 head-dim rows, 4 keys as fp16
#pragma unroll
          for (int dd = 0; dd < 8; ++dd) {
            const int e = dd / 4, bb = dd % 4;
            const unsigned k4 = gather_byte(vreg[u][0][e], vreg[u][1][e], vreg[u][2][e], vreg[u][3][e], bb);
            const u32x2 f = i8x4_to_f16x4(k4);
            *reinterpret_cast<u32x2*>(vs_ + (8 * dc + dd) * VST + 4 * kq) = f;
          }
        } else {
          // 4 keys x 8 bf16 -> for each of the 8 head-dim rows, 4 keys (2 dwords)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned w0 = vreg[u][0][e], w1 = vreg[u][1][e], w2 = vreg[u][2][e], w3 = vreg[u][3][e];
            u32x2 lo_d, hi_d;
            lo_d[0] = __builtin_amdgcn_perm(w1, w0, 0x05040100u);
            lo_d[1] = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
            hi_d[0] = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
            hi_d[1] = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
            *reinterpret_cast<u32x2*>(vs_ + (8 * dc + 2 * e) * VST + 4 * kq) = lo_d;
            *reinterpret_cast<u32x2*>(vs_ + (8 * dc + 2 * e + 1) * VST + 4 * kq) = hi_d;
          }
        }
      }
    }
    if (KV_I8 && tid < 2 * BN) {
      if (tid < BN) lds_ks[stage][tid] = sreg;
      else lds_vs[stage][tid - BN] = sreg;
    }
  };

  // ---- per-wave state
  f32x16 O[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[qb][db][i] = 0.f;
  float m_run[QB], l_run[QB], mc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = neg_inf();
    l_run[qb] = 0.f;
    mc[qb] = 0.f;
  }
  const float c2 = a.scale_log2;
  const float lazy_thr = C::kLazyLog2 / c2;   // raw-score headroom before the max is raised
  const int w_last = qw0 + 32 * QB - 1;       // last query row of this wave (may be padding)
  const bool wave_live = qw0 < a.s_q;

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);

    const int k0 = (t_lo + t) * BN;
    bool skip = !wave_live;
    if (a.causal && k0 > w_last + off) skip = true;
    if (a.window && k0 + BN - 1 <= qw0 + off - a.window) skip = true;
    if (!skip) {
      const bool need_mask = (k0 + BN > a.s_k) || (a.causal && k0 + BN - 1 > qw0 + off) ||
                             (a.window && k0 <= w_last + off - a.window);
      const unsigned short* Kt = lds_k[stage];
      const unsigned short* Vt = lds_v[stage];

      // Two 32-key softmax steps per 64-key LDS tile (bounds the live score registers).
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // S^T[qb]: key 32 kb + 8 (i/4) + 4 h + i%4 (tile-relative), query 32 qb + c
        f32x16 S[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int i = 0; i < 16; ++i) S[qb][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Kt + (32 * kb + c) * KST + 16 * ks + 8 * h);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) S[qb] = mfma32_bf16(ka, Qf[qb][ks], S[qb]);
        }
        if (KV_I8) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 sc = *reinterpret_cast<const f32x4*>(&lds_ks[stage][32 * kb + 8 * g4 + 4 * h]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
              for (int e = 0; e < 4; ++e) S[qb][4 * g4 + e] *= sc[e];
          }
        }
        if (need_mask) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const int qi = qw0 + 32 * qb + c;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int j = k0 + 32 * kb + 8 * (i / 4) + 4 * h + (i % 4);
              bool vis = j < a.s_k;
              if (a.causal) vis = vis && (j <= qi + off);
              if (a.window) vis = vis && (j > qi + off - a.window);
              if (!vis) S[qb][i] = neg_inf();
            }
          }
        }

        // online softmax with a lazily raised max
        float tmax[QB];
        bool raise = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float mx = neg_inf();
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[qb][i]);
          mx = fmaxf(mx, xor32(mx));
          tmax[qb] = mx;
          raise = raise || (mx - m_run[qb] > lazy_thr);
        }
        if (__any(raise)) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const float m_new = fmaxf(m_run[qb], tmax[qb]);
            const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f((m_run[qb] - m_use) * c2);
            l_run[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
              for (int i = 0; i < 16; ++i) O[qb][db][i] *= alpha;
            m_run[qb] = m_new;
            mc[qb] = m_use * c2;
          }
        }

        // P^T as B operands: k-step s2 (0, 1) covers keys 32 kb + 16 s2 + 8 (i/4) + 4 h + i%4
        u32x4 Pw[QB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float p[16];
          float ps = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][i], c2, -mc[qb]));
            ps += p[i];
          }
          l_run[qb] += ps;
          if (KV_I8) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const f32x4 sc = *reinterpret_cast<const f32x4*>(&lds_vs[stage][32 * kb + 8 * g4 + 4 * h]);
#pragma unroll
              for (int e = 0; e < 4; ++e) p[4 * g4 + e] *= sc[e];
            }
#pragma unroll
            for (int q2 = 0; q2 < 8; ++q2) Pw[qb][q2 / 4][q2 % 4] = pack_f16x2(p[2 * q2], p[2 * q2 + 1]);
          } else {
#pragma unroll
            for (int q2 = 0; q2 < 8; ++q2) Pw[qb][q2 / 4][q2 % 4] = pack_bf16x2(p[2 * q2], p[2 * q2 + 1]);
          }
        }

        // O^T[qb][db] += V^T P^T
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int kbase = 32 * kb + 16 * s2 + 4 * h;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const unsigned short* vrow = Vt + (32 * db + c) * VST + kbase;
            const u32x2 v0 = *reinterpret_cast<const u32x2*>(vrow);
            const u32x2 v1 = *reinterpret_cast<const u32x2*>(vrow + 8);
            const u32x4 vw = {v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              if (KV_I8)
                O[qb][db] = mfma32_f16(__builtin_bit_cast(f16x8, vw), __builtin_bit_cast(f16x8, Pw[qb][s2]), O[qb][db]);
              else
                O[qb][db] = mfma32_bf16(__builtin_bit_cast(bf16x8, vw), __builtin_bit_cast(bf16x8, Pw[qb][s2]), O[qb][db]);
            }
          }
        }
      }
    }

    if (t + 1 < n_tiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- finalize: O / l (x 2^E for int8), epilogue, store; LSE = sigma m + ln l
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + xor32(l_run[qb]);
    float inv = l_tot > 0.f ? __fdiv_rn(1.0f, l_tot) : 0.f;
    if (KV_I8) inv *= vs_unnorm;
    const int qi = qw0 + 32 * qb + c;
    if (qi < a.s_q) {
      const int64_t row = (int64_t)head * a.s_q + qi;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = 32 * db + 8 * g4 + 4 * h;
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = apply_epilogue(O[qb][db][4 * g4 + e] * inv, a.epi);
          if (a.out_bf16) {
            u32x2 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            *reinterpret_cast<u32x2*>(static_cast<unsigned short*>(a.out) + row * D + d0) = w;
          } else {
            f32x4 w = {y[0], y[1], y[2], y[3]};
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * D + d0) = w;
          }
        }
      }
      if (a.lse && h == 0) a.lse[row] = l_tot > 0.f ? m_run[qb] * a.scale + logf(l_tot) : neg_inf();
    }
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, int32_t kv_dtype, hipStream_t st, const char** name) {
  const int64_t n_qb = (a.s_q + Cfg<D>::BM - 1) / Cfg<D>::BM;
  const int64_t blocks = n_qb * a.bh_q;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (kv_dtype == kI8) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    *name = "prefill_bf16_i8kv";
  } else {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, false>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    *name = "prefill_bf16";
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, int32_t d, int32_t kv_dtype, hipStream_t stream,
                               const char** name) {
  switch (d) {
    case 32: return launch_d<32>(a, kv_dtype, stream, name);
    case 64: return launch_d<64>(a, kv_dtype, stream, name);
    case 96: return launch_d<96>(a, kv_dtype, stream, name);
    case 128: return launch_d<128>(a, kv_dtype, stream, name);
    case 160: return launch_d<160>(a, kv_dtype, stream, name);
    case 192: return launch_d<192>(a, kv_dtype, stream, name);
    case 224: return launch_d<224>(a, kv_dtype, stream, name);
    case 256: return launch_d<256>(a, kv_dtype, stream, name);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
