// Split-KV decode over the int8 per-token KV cache (fkl.flash_attention PR, Verification: the
// decode check, one query row per head against the int8 cache; Summary: the cache is
// dequantized inside q.k and p.v and never expanded in global memory; kernbench2 ADR-0060
// commit: split decode whose partial running (m, l, O) states are reduced afterwards).
//
// Pass 1 (decode_partial_kernel), grid (splits, bh_kv, ceil(G/HPW)): a workgroup streams one
// contiguous range of keys of one KV head, for up to HPW = 4 query heads of its GQA group, and
// leaves one partial state (m, l, O unnormalised) per (query head, split) in the workspace.
// Pass 2 (decode_merge_kernel): per query head, M = max m_s, L = sum l_s e^(m_s - M),
// O = sum O_s e^(m_s - M) / L, then the epilogue and the store.
//
// HBM-bound: every K/V byte is read once for all query heads of its group.  Both products run
// on the int8 MFMA (v_mfma_i32_16x16x64_i8), exactly, with no conversion of the cache:
//   * S = Q K^T.  A = K codes (16 keys x 64 head-dim), straight from global memory.  B holds
//     Q as four signed 7-bit digits: q = 2^E (d0/2^7 + d1/2^14 + d2/2^21 + d3/2^28), one MFMA
//     column per (digit, head) -- 4 digits x 4 heads fill the 16 columns that a single decode
//     row would otherwise leave empty.  The int32 products are exact; the digit columns are
//     recombined in fp32 with two DPP row rotations, so every lane ends up with the same S.
//   * O += P~ V with P~ = p * v_s.  B holds P~ as four unsigned 7-bit digits of P~ / 2^F
//     (2^F above the tile's largest P~), again one column per (digit, head).  A = V^T codes,
//     obtained with in-register byte transposes of the loaded V rows.  The int32 tile sums are
//     exact and are accumulated in fp32 per digit, so the P.V product keeps about 28 bits.
//   * The online softmax (running max raised lazily, as in the prefill kernel) runs in fp32.
// Tiles are 64 keys; the four waves of a workgroup take interleaved tiles of the range and
// combine their states through LDS at the end.
#include "device_common.hpp"

namespace fa {
namespace {

constexpr float kLazyLog2 = 8.0f;

// keys per tile: 64, or 32 when head_dim > 128 (keeps the K/V registers of a tile bounded)
template <int D>
constexpr int tile_keys() { return D <= 128 ? 64 : 32; }

template <int N>
__device__ __forceinline__ float dpp_row_ror(float x) {
  static_assert(N >= 1 && N <= 15, "row_ror amount");
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

__device__ __forceinline__ unsigned gather_byte4(unsigned w0, unsigned w1, unsigned w2, unsigned w3, int b) {
  const unsigned s = 8u * b;
  return ((w0 >> s) & 0xffu) | (((w1 >> s) & 0xffu) << 8) | (((w2 >> s) & 0xffu) << 16) |
         (((w3 >> s) & 0xffu) << 24);
}

// D head dim; CT column tiles of 4 query heads (HPW = 4 * CT heads per workgroup; the
// launcher uses CT = 1).
template <int D, int CT>
__global__ __launch_bounds__(256, 2) void decode_partial_kernel(DecodeArgs a) {
  constexpr int NKK = (D + 63) / 64;          // 64-deep k-steps of Q.K
  constexpr int NDH = (D + 127) / 128;        // 128-wide head-dim segments for P.V
  constexpr int NB = 8 * NDH;                 // 16-row MFMA blocks of O^T
  constexpr int NW = 4;
  constexpr int HPW = 4 * CT;
  constexpr int kTile = tile_keys<D>();
  constexpr int KB = kTile / 16;              // 16-key row blocks per tile

  __shared__ float lds_sc[NW][2][kTile];       // per-wave k/v scales of the current tile
  __shared__ float lds_E[16];
  __shared__ float lds_m[NW][HPW];
  __shared__ float lds_l[NW][HPW];
  __shared__ float lds_o[NW][HPW][D];

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

  // ---- per-head exponent E: max|q| * 2^-E < 1/2
  {
    const int hz = tid >> 4, sub = tid & 15;
    float mx = 0.f;
    if (hz < nh) {
      for (int d = sub; d < D; d += 16) {
        const int64_t idx = (int64_t)(head0 + hz) * D + d;
        const float qv = a.q_bf16 ? bf16_bits_to_f32(static_cast<const unsigned short*>(a.q)[idx])
                                  : static_cast<const float*>(a.q)[idx];
        mx = fmaxf(mx, fabsf(qv));
      }
    }
#pragma unroll
    for (int o2 = 8; o2 >= 1; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2, 64));
    if (sub == 0) {
      int e = 0;
      if (mx > 0.f) (void)frexpf(mx, &e);
      lds_E[hz] = (float)(e + 1);
    }
  }
  __syncthreads();

  // ---- Q digit B operands: column n = (t_dig, gq) of tile ct, k-slots 64 kk + 16 hq + i
  i32x4 qdig[CT][NKK];
  float s_comb[CT];   // 2^(E - 7 (t + 1)) for this lane's digit column
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int hz = 4 * ct + gq;
    const bool hv = hz < nh;
    const int E = hv ? (int)lds_E[hz] : 0;
    s_comb[ct] = ldexpf(1.f, E - 7 * (t_dig + 1));
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      unsigned w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = 64 * kk + 16 * hq + i;
        int dig = 0;
        if (hv && d < D) {
          const int64_t idx = (int64_t)(head0 + hz) * D + d;
          const float qv = a.q_bf16 ? bf16_bits_to_f32(static_cast<const unsigned short*>(a.q)[idx])
                                    : static_cast<const float*>(a.q)[idx];
          float x = ldexpf(qv, -E) * 128.f;
          float dd[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            dd[t] = __builtin_rintf(x);
            x = (x - dd[t]) * 128.f;
          }
          dig = (int)(t_dig == 0 ? dd[0] : t_dig == 1 ? dd[1] : t_dig == 2 ? dd[2] : dd[3]);
        }
        w[i / 4] |= ((unsigned)dig & 0xffu) << (8 * (i % 4));
      }
      qdig[ct][kk] = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
  }

  // ---- tile range of this split; wave w takes tiles w, w + 4, ...
  const int n_tiles_total = (a.s_k - a.key_lo + kTile - 1) / kTile;
  const int ts = split * a.tiles_per_split;
  const int te = min(n_tiles_total, ts + a.tiles_per_split);

  float O[CT][NB][4];
  float m_run[CT], l_run[CT], mc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    m_run[ct] = neg_inf();
    l_run[ct] = 0.f;
    mc[ct] = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) O[ct][b][v] = 0.f;
  }
  const float c2 = a.scale_log2;
  const float lazy_thr = kLazyLog2 / c2;

  // K: kreg[kb][kk] = K[k0 + 16 kb + n][64 kk + 16 hq .. +16]
  // V: vreg[c4][r][dh] = V[k0 + 16 c4 + 4 hq + r][128 dh + 8 n .. +8]
  i32x4 kreg[KB][NKK];
  u32x2 vreg[KB][4][NDH];

  auto load_tile = [&](int tile) {
    const int k0 = a.key_lo + tile * kTile;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int j = k0 + 16 * kb + n;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int d = 64 * kk + 16 * hq;
        i32x4 w = {0, 0, 0, 0};
        if (j < a.s_k && d < D) w = *reinterpret_cast<const i32x4*>(a.k + (kv_base + j) * D + d);
        kreg[kb][kk] = w;
      }
    }
#pragma unroll
    for (int c4 = 0; c4 < KB; ++c4)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = k0 + 16 * c4 + 4 * hq + r;
#pragma unroll
        for (int dh = 0; dh < NDH; ++dh) {
          const int d = 128 * dh + 8 * n;
          u32x2 w = {0u, 0u};
          if (j < a.s_k && d < D) w = *reinterpret_cast<const u32x2*>(a.v + (kv_base + j) * D + d);
          vreg[c4][r][dh] = w;
        }
      }
    if (lane < kTile) {
      const int j = k0 + lane;
      float ks = 0.f, vs = 0.f;
      if (j < a.s_k) {
        ks = a.k_scale[kv_base + j];
        vs = a.v_scale[kv_base + j];
      }
      lds_sc[wave][0][lane] = ks;
      lds_sc[wave][1][lane] = vs;
    }
  };

  auto compute_tile = [&](int tile) {
    const int k0 = a.key_lo + tile * kTile;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // this lane's keys: k0 + 16 kb + 4 hq + v
    float ks[KB][4], vs[KB][4];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(&lds_sc[wave][0][16 * kb + 4 * hq]);
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(&lds_sc[wave][1][16 * kb + 4 * hq]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        ks[kb][v] = a4[v];
        vs[kb][v] = b4[v];
      }
    }
    const bool tail = k0 + kTile > a.s_k;

    // phase 1, per column tile: S, online softmax, digits of P~
    i32x4 pdig[CT];
    float o_scale[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      // S^T: rows = keys 16 kb + 4 hq + v, column n
      float s[KB][4];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        i32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) acc = mfma16_i8(kreg[kb][kk], qdig[ct][kk], acc);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float y = (float)acc[v] * s_comb[ct];
          y = y + dpp_row_ror<8>(y);
          y = y + dpp_row_ror<4>(y);
          float sv = y * ks[kb][v];
          if (tail && (k0 + 16 * kb + 4 * hq + v >= a.s_k)) sv = neg_inf();
          s[kb][v] = sv;
        }
      }
      float mx = neg_inf();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[kb][v]);
      mx = fmaxf(mx, xor16(mx));
      mx = fmaxf(mx, xor32(mx));
      const bool raise = mx - m_run[ct] > lazy_thr;
      if (__any(raise)) {
        const float m_new = fmaxf(m_run[ct], mx);
        const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_run[ct] - m_use) * c2);
        l_run[ct] *= alpha;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 4; ++v) O[ct][b][v] *= alpha;
        m_run[ct] = m_new;
        mc[ct] = m_use * c2;
      }
      float pt[KB][4];
      float ps = 0.f, pmax = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][v], c2, -mc[ct]));
          ps += p;
          pt[kb][v] = p * vs[kb][v];
          pmax = fmaxf(pmax, pt[kb][v]);
        }
      l_run[ct] += ps;
      pmax = fmaxf(pmax, xor16(pmax));
      pmax = fmaxf(pmax, xor32(pmax));
      int F = 0;
      if (pmax > 0.f) (void)frexpf(pmax, &F);     // pmax < 2^F
      const float to_x = ldexpf(1.f, 7 * t_dig - F);      // x * 2^(7 t)
      // digit t of x = P~ / 2^F in [0, 1): floor(x 2^(7t+7)) - 128 floor(x 2^(7t))
      unsigned pw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        unsigned w = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float hi = floorf(pt[kb][v] * to_x);
          const float lo = floorf(pt[kb][v] * (to_x * 128.f));
          const float dg = __builtin_fmaf(-128.f, hi, lo);
          w |= ((unsigned)(int)dg & 0xffu) << (8 * v);
        }
        pw[kb] = w;
      }
      pdig[ct] = i32x4{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]};
      o_scale[ct] = ldexpf(1.f, F - 7 * (t_dig + 1));
    }

    // phase 2: O^T += V^T P~^T.  A operand of block b (segment dh = b/8, row offset b8 = b%8):
    // dword c4 holds keys 16 c4 + 4 hq + 0..3 at head-dim 128 dh + 8 n + b8.
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int dh = b / 8, b8 = b % 8;
      const int e = b8 / 4, bb = b8 % 4;
      unsigned w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int c4 = 0; c4 < KB; ++c4)
        w[c4] = gather_byte4(vreg[c4][0][dh][e], vreg[c4][1][dh][e], vreg[c4][2][dh][e], vreg[c4][3][dh][e], bb);
      const i32x4 vt = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const i32x4 acc = mfma16_i8(vt, pdig[ct], i32x4{0, 0, 0, 0});
#pragma unroll
        for (int v = 0; v < 4; ++v) O[ct][b][v] = __builtin_fmaf((float)acc[v], o_scale[ct], O[ct][b][v]);
      }
    }
  };

  int tile = ts + wave;
  if (tile < te) load_tile(tile);
  while (tile < te) {
    compute_tile(tile);
    tile += NW;
    if (tile < te) load_tile(tile);
  }

  // ---- combine digit columns (O) and lane groups (l), then the 4 waves through LDS
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    float lt = l_run[ct];
    lt = lt + xor16(lt);
    lt = lt + xor32(lt);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float y = O[ct][b][v];
        y = y + dpp_row_ror<8>(y);
        y = y + dpp_row_ror<4>(y);
        O[ct][b][v] = y;
      }
    const int hz = 4 * ct + gq;
    {
      if (lane == gq) {  // t_dig == 0, hq == 0
        lds_m[wave][hz] = m_run[ct];
        lds_l[wave][hz] = lt;
      }
      if (t_dig == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int d = 128 * (b / 8) + 8 * (4 * hq + v) + (b % 8);
            if (d < D) lds_o[wave][hz][d] = O[ct][b][v];
          }
      }
    }
  }
  __syncthreads();

  for (int idx = tid; idx < nh * (D + 2); idx += 256) {
    const int hz = idx / (D + 2), col = idx % (D + 2);
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, lds_m[w][hz]);
    float acc = 0.f;
    if (col == 0) {
      acc = M;
    } else if (M != neg_inf()) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
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
  apply_epilogue_all(y, a.epi);
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

template <int D, int CT>
hipError_t launch_dct(const DecodeArgs& a_in, hipStream_t st) {
  DecodeArgs a = a_in;
  const int tiles = (a.s_k - a.key_lo + tile_keys<D>() - 1) / tile_keys<D>();
  a.tiles_per_split = (tiles + a.num_splits - 1) / a.num_splits;
  const dim3 grid((unsigned)a.num_splits, (unsigned)a.bh_kv, (unsigned)((a.group + 4 * CT - 1) / (4 * CT)));
  hipLaunchKernelGGL((decode_partial_kernel<D, CT>), grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)a.bh_q), dim3(64), 0, st, a);
  return hipGetLastError();
}

// One column tile (4 query heads) per workgroup: the per-tile registers of two or more column
// tiles exceed the budget of two waves per SIMD.  Groups larger than 4 run ceil(G/4)
// workgroups per (split, KV head).
template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t st, const char** name) {
  *name = "decode_int8";
  return launch_dct<D, 1>(a, st);
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
