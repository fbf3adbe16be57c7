// Merge of attention outputs computed over disjoint sets of keys, by their log-sum-exp.
//
// A split or ring prefill computes, for the same query rows, one normalised output O_p and one
// log-sum-exp LSE_p per key chunk p (kernbench2 ADR-0060 commit: partial running (m, l, O)
// states reduced into one; Foundry attention/ README, References: the online-softmax
// recurrence, whose merge of two states is this one).  Exact attention over the union is
//   LSE = log sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p,
// evaluated against M = max_p LSE_p for range: w_p = exp(LSE_p - M), L = sum_p w_p,
// O = (sum_p w_p O_p) / L, LSE = M + log L.  Chunks with no visible key (LSE_p = -inf, O_p = 0)
// get weight 0; a row that no chunk covers returns 0 and LSE = -inf, like an empty row of the
// forward.  The Mul/Add epilogue runs on the merged row, before the cast.
//
// HBM-bound: a segment of D/4 lanes owns a row, each lane reading 16 contiguous bytes of every
// part (nontemporal loads and stores: each byte is read or written once).  Up to eight parts are
// handled per group with every load of the group -- their LSE values and their output rows --
// issued before the first use, so a wave waits for memory once per group rather than once per
// part; with more than eight parts a first pass finds M over the LSE values, eight loads in
// flight at a time.
#include "device_common.hpp"

namespace fa {
namespace {

constexpr int kPartGroup = 8;   // parts whose loads are in flight together
// Two waves per workgroup: at 8 chunks x 64 heads x 4096 rows, d = 128, workgroups of 128 threads
// ran 176.5 us against 181 (64), 194 (256), 198 (192), 179 (384) and 178 us (512) in interleaved
// timings, with the same outputs.
constexpr int kMergeThreads = 128;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  constexpr int SEG = D / 4;     // lanes per row
  constexpr int RPW = 64 / SEG;  // rows per wave (D <= 256, so SEG <= 64)
  constexpr int PG = kPartGroup;
  static_assert(D % 32 == 0 && SEG <= 64, "head_dim must be a multiple of 32, at most 256");
  const int lane = threadIdx.x & 63;
  const int sl = lane % SEG;
  const int64_t row = (((int64_t)blockIdx.x * kMergeThreads + threadIdx.x) >> 6) * RPW + lane / SEG;
  if (row >= a.rows) return;     // rows are independent: no lane exchange below
  const float* lse = a.lse_parts + row;
  const float* src = a.o_parts + row * D + 4 * sl;
  const int n = a.n_parts;

  float lp[PG];
  f32x4 x[PG];
  // loads of parts p .. p + 7 (those below n; a missing part reads as LSE -inf, weight 0)
  auto load_group = [&](int p) {
#pragma unroll
    for (int u = 0; u < PG; ++u) {
      if (p + u < n) {
        lp[u] = lse[(int64_t)(p + u) * a.rows];
        x[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + (int64_t)(p + u) * a.rows * D));
      } else {
        lp[u] = neg_inf();
        x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  float m = neg_inf();
  if (n <= PG) {
    load_group(0);
#pragma unroll
    for (int u = 0; u < PG; ++u) m = fmaxf(m, lp[u]);
  } else {
    for (int p = 0; p < n; p += PG) {
      float lq[PG];
#pragma unroll
      for (int u = 0; u < PG; ++u) lq[u] = p + u < n ? lse[(int64_t)(p + u) * a.rows] : neg_inf();
#pragma unroll
      for (int u = 0; u < PG; ++u) m = fmaxf(m, lq[u]);
    }
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  const float mm = m == neg_inf() ? 0.f : m;   // every weight is then 0 for an uncovered row
  // a part of weight 0 adds nothing even if its row holds garbage (select, not multiply)
  auto add_group = [&]() {
#pragma unroll
    for (int u = 0; u < PG; ++u) {
      const float w = __builtin_amdgcn_exp2f((lp[u] - mm) * 1.4426950408889634f);
      l += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = w > 0.f ? __builtin_fmaf(w, x[u][e], acc[e]) : acc[e];
    }
  };
  if (n <= PG) {
    add_group();
  } else {
    for (int p = 0; p < n; p += PG) {
      load_group(p);
      add_group();
    }
  }
  const float inv = l > 0.f ? __fdiv_rn(1.0f, l) : 0.f;
  float y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = acc[e] * inv;
  apply_epilogue_all(y, a.epi, [&](int e) { return 4 * sl + e; });
  if (a.out_bf16) {
    const u32x2 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(static_cast<unsigned short*>(a.out) + row * D + 4 * sl));
  } else {
    const f32x4 w = {y[0], y[1], y[2], y[3]};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * D + 4 * sl));
  }
  if (a.lse && sl == 0) a.lse[row] = l > 0.f ? m + logf(l) : neg_inf();
}

template <int D>
hipError_t launch_d(const MergeArgs& a, hipStream_t st, const char** name) {
  constexpr int rows_per_block = (kMergeThreads / 64) * (64 / (D / 4));
  const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((merge_kernel<D>), dim3((unsigned)blocks), dim3(kMergeThreads), 0, st, a);
  *name = "merge_lse";
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int32_t d, hipStream_t stream, const char** name) {
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
