// fp32 attention forward on fp32 MFMA (v_mfma_f32_32x32x2_f32), for fp32 Q with fp32 or
// int8 K/V.  This is the precision path: scores, probabilities and the P.V product stay
// in fp32, so the result is within fp32 rounding of exact attention on the same
// (dequantized) inputs.
//
// Method: FlashAttention-2 style tiled forward with an online softmax (fkl.flash_attention
// PR, Summary: FA-2 forward, fp32 accumulation; Foundry attention/ README, References:
// the online-softmax recurrence).  Per key tile: S = K Q^T on MFMA, masked by causal /
// window / sequence bounds, running max m and sum l updated, O rescaled by exp(m_old -
// m_new) and O += V^T P^T on MFMA.  int8 K/V are converted exactly to fp32 when staged
// into LDS; the per-token scales are applied to S (k) and to P (v) in registers.
//
// One wave per 32 query rows; all operands staged in LDS.  Working in the transposed
// orientation (keys as MFMA rows, queries as columns) keeps each query's scores and its
// output column in one lane pair, so the softmax needs one cross-lane exchange.
#include "device_common.hpp"

namespace fa {
namespace {

template <int D, bool KV_I8, bool SOPS>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int BM = 32;
  constexpr int BN = 32;
  constexpr int QST = D + 1;   // LDS row strides (floats), padded against bank conflicts
  constexpr int KST = D + 1;
  constexpr int VST = D + 8;
  constexpr int NDB = D / 32;  // 32-wide output column blocks
  __shared__ float Qs[BM * QST];
  __shared__ float Ks[BN * KST];
  __shared__ float Vs[BN * VST];
  __shared__ float kss[BN];
  __shared__ float vss[BN];

  const int lane = threadIdx.x;
  const int h = lane >> 5;
  const int c = lane & 31;
  const int n_qb = (a.s_q + BM - 1) / BM;
  const int head = blockIdx.x / n_qb;
  const int qblk = blockIdx.x % n_qb;
  const int kvh = head / a.group;
  const int q0 = qblk * BM;
  const int off = a.s_k - a.s_q;   // bottom-right causal alignment

  const float* qp = static_cast<const float*>(a.q) + (int64_t)head * a.s_q * D;
  for (int idx = lane; idx < BM * (D / 4); idx += 64) {
    const int r = idx / (D / 4), c4 = idx % (D / 4);
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
    if (q0 + r < a.s_q) w = *reinterpret_cast<const f32x4*>(qp + (int64_t)(q0 + r) * D + 4 * c4);
#pragma unroll
    for (int e = 0; e < 4; ++e) Qs[r * QST + 4 * c4 + e] = w[e];
  }

  // key range touched by any row of the block
  const int r_last = min(q0 + BM, a.s_q) - 1;
  int lo = 0, hi = a.s_k;
  if (a.causal) hi = max(0, min(a.s_k, r_last + off + 1));
  if (a.window) lo = max(0, q0 + off - a.window + 1);

  f32x16 O[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[b][i] = 0.f;
  float m_run = neg_inf();
  float l_run = 0.f;
  const float c2 = a.scale_log2;
  const int qi = q0 + c;

  for (int k0 = (lo / BN) * BN; k0 < hi; k0 += BN) {
    __syncthreads();
    if (KV_I8) {
      const int8_t* kp = static_cast<const int8_t*>(a.k) + ((int64_t)kvh * a.s_k) * D;
      const int8_t* vp = static_cast<const int8_t*>(a.v) + ((int64_t)kvh * a.s_k) * D;
      for (int idx = lane; idx < BN * (D / 4); idx += 64) {
        const int r = idx / (D / 4), c4 = idx % (D / 4);
        unsigned wk = 0, wv = 0;
        if (k0 + r < a.s_k) {
          wk = *reinterpret_cast<const unsigned*>(kp + (int64_t)(k0 + r) * D + 4 * c4);
          wv = *reinterpret_cast<const unsigned*>(vp + (int64_t)(k0 + r) * D + 4 * c4);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Ks[r * KST + 4 * c4 + e] = (float)(signed char)(wk >> (8 * e));
          Vs[r * VST + 4 * c4 + e] = (float)(signed char)(wv >> (8 * e));
        }
      }
      if (lane < BN) {
        const int j = k0 + lane;
        kss[lane] = j < a.s_k ? a.k_scale[(int64_t)kvh * a.s_k + j] : 0.f;
      } else {
        const int j = k0 + lane - BN;
        vss[lane - BN] = j < a.s_k ? a.v_scale[(int64_t)kvh * a.s_k + j] : 0.f;
      }
    } else {
      const float* kp = static_cast<const float*>(a.k) + ((int64_t)kvh * a.s_k) * D;
      const float* vp = static_cast<const float*>(a.v) + ((int64_t)kvh * a.s_k) * D;
      for (int idx = lane; idx < BN * (D / 4); idx += 64) {
        const int r = idx / (D / 4), c4 = idx % (D / 4);
        f32x4 wk = {0.f, 0.f, 0.f, 0.f}, wv = {0.f, 0.f, 0.f, 0.f};
        if (k0 + r < a.s_k) {
          wk = *reinterpret_cast<const f32x4*>(kp + (int64_t)(k0 + r) * D + 4 * c4);
          wv = *reinterpret_cast<const f32x4*>(vp + (int64_t)(k0 + r) * D + 4 * c4);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Ks[r * KST + 4 * c4 + e] = wk[e];
          Vs[r * VST + 4 * c4 + e] = wv[e];
        }
      }
    }
    __syncthreads();

    // S^T (keys x queries) = K Q^T
    f32x16 S;
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = 0.f;
#pragma unroll 8
    for (int ks = 0; ks < D / 2; ++ks) {
      const float ka = Ks[c * KST + 2 * ks + h];
      const float qb = Qs[c * QST + 2 * ks + h];
      S = mfma32_f32(ka, qb, S);
    }

    float tmax = neg_inf();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kl = 8 * (i / 4) + 4 * h + (i % 4);
      const int j = k0 + kl;
      float s = S[i];
      if (KV_I8) s *= kss[kl];
      if constexpr (SOPS) s = apply_epilogue(s, a.sops, min(j, a.s_k - 1));
      bool vis = j < a.s_k;
      if (a.causal) vis = vis && (j <= qi + off);
      if (a.window) vis = vis && (j > qi + off - a.window);
      s = vis ? s : neg_inf();
      S[i] = s;
      tmax = fmaxf(tmax, s);
    }
    tmax = max_xor32(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
    const float mc = m_use * c2;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[i], c2, -mc));
      psum += p;
      S[i] = p;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[b][i] *= alpha;

    // O^T (d x queries) += V^T P^T
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kl = 8 * (i / 4) + 4 * h + (i % 4);
      float p = S[i];
      if (KV_I8) p *= vss[kl];
#pragma unroll
      for (int b = 0; b < NDB; ++b) O[b] = mfma32_f32(Vs[kl * VST + 32 * b + c], p, O[b]);
    }
  }

  // finalize: O / l, epilogue, store; LSE = m * sigma + ln(l)
  const float l_tot = add_xor32(l_run);
  const float inv = l_tot > 0.f ? __fdiv_rn(1.0f, l_tot) : 0.f;
  if (qi < a.s_q) {
    const int64_t row = (int64_t)head * a.s_q + qi;
#pragma unroll
    for (int b = 0; b < NDB; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * b + 8 * g + 4 * h;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = apply_epilogue(O[b][4 * g + e] * inv, a.epi, d0 + e);
        if (a.out_bf16) {
          u32x2 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
          *reinterpret_cast<u32x2*>(static_cast<unsigned short*>(a.out) + row * D + d0) = w;
        } else {
          f32x4 w = {y[0], y[1], y[2], y[3]};
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * D + d0) = w;
        }
      }
    }
    if (a.lse && h == 0) a.lse[row] = l_tot > 0.f ? m_run * a.scale + logf(l_tot) : neg_inf();
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, int32_t kv_dtype, hipStream_t st, const char** name) {
  const int n_qb = (a.s_q + 31) / 32;
  const dim3 grid((unsigned)(n_qb * a.bh_q));
  const bool so = a.sops.n > 0;
  if (kv_dtype == kI8) {
    if (so) hipLaunchKernelGGL((prefill_f32_kernel<D, true, true>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((prefill_f32_kernel<D, true, false>), grid, dim3(64), 0, st, a);
    *name = so ? "prefill_f32_i8kv_sops" : "prefill_f32_i8kv";
  } else {
    if (so) hipLaunchKernelGGL((prefill_f32_kernel<D, false, true>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((prefill_f32_kernel<D, false, false>), grid, dim3(64), 0, st, a);
    *name = so ? "prefill_f32_sops" : "prefill_f32";
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, int32_t d, int32_t kv_dtype, hipStream_t stream,
                              const char** name) {
  if ((int64_t)((a.s_q + 31) / 32) * a.bh_q > 0x7fffffff) return hipErrorInvalidConfiguration;
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
