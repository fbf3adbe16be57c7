// Plain argument blocks passed by value from the host dispatcher to the kernels,
// and the host-side launch functions each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr int kMaxEpilogue = 8;
constexpr int kEpiMul = 1;
constexpr int kEpiAdd = 2;
constexpr int kEpiBias = 3;   // + vec[channel]
constexpr int kEpiRelu = 4;   // max(x, +0)

// An op list of one scope.  Output scope (`epi`): ops on the normalised output row, a bias
// indexed by head-dim channel.  Score scope (`sops`): ops on every raw score q.k of a key tile
// before the mask and the softmax scale, a bias indexed by key position.
struct EpiArgs {
  int32_t n;
  int32_t kind[kMaxEpilogue];
  float value[kMaxEpilogue];
  const float* vec[kMaxEpilogue];   // vector of a bias op, else null
};

enum DType : int32_t { kF32 = 0, kBF16 = 1, kI8 = 2 };

struct PrefillArgs {
  const void* q;        // [bh_q, s_q, d]
  const void* k;        // [bh_kv, s_k, d]
  const void* v;        // [bh_kv, s_k, d]
  const float* k_scale; // [bh_kv, s_k] or null
  const float* v_scale; // [bh_kv, s_k] or null
  void* out;            // [bh_q, s_q, d]
  float* lse;           // [bh_q, s_q] or null
  int32_t bh_q, bh_kv, group;
  int32_t s_q, s_k;
  int32_t causal, window;
  int32_t out_bf16;
  float scale;          // softmax scale sigma
  float scale_log2;     // sigma * log2(e)
  EpiArgs epi;
  EpiArgs sops;         // score-scope ops (the kernel instantiation with them runs only when n > 0)
};

struct DecodeArgs {
  const void* q;        // [bh_q, d]
  const int8_t* k;      // [bh_kv, s_k, d]
  const int8_t* v;
  const float* k_scale; // [bh_kv, s_k]
  const float* v_scale;
  void* out;            // [bh_q, d]
  float* lse;           // [bh_q] or null
  float* partial;       // workspace [bh_q, num_splits, d + 2]
  int32_t bh_q, bh_kv, group;
  int32_t s_k;
  int32_t key_lo;       // first visible key (window), 0 otherwise
  int32_t num_splits;
  int32_t tiles_per_split;
  int32_t q_bf16, out_bf16;
  float scale, scale_log2;
  EpiArgs epi;
  EpiArgs sops;         // score-scope ops
};

struct AppendArgs {
  const void* k_new;    // [bh_kv, n_new, d]
  const void* v_new;
  const int32_t* pos;   // [bh_kv] cache row of each head's first new token
  int8_t* k_cache;      // [bh_kv, capacity, d]
  int8_t* v_cache;
  float* k_scale;       // [bh_kv, capacity]
  float* v_scale;
  const float* rope_cos; // [capacity, d/2] rotate-half RoPE table of K by cache position, or null
  const float* rope_sin;
  int32_t bh_kv, n_new, capacity;
};

struct MergeArgs {
  const float* o_parts;   // [n_parts, rows, d] normalised outputs
  const float* lse_parts; // [n_parts, rows]
  void* out;              // [rows, d]
  float* lse;             // [rows] or null
  int64_t rows;
  int32_t n_parts;
  int32_t out_bf16;
  EpiArgs epi;
};

struct TqArgs {
  const void* x;          // encode input [n, d] fp32 or bf16
  const int8_t* signs;    // [d], +-1
  uint8_t* codes;         // [n, d bits / 8] packed codes (written by encode, read by decode)
  float* norms;           // [n]
  void* out;              // decode output [n, d]
  int64_t n;
  float inv_sqrt_d;
  float thr[15];          // encode: the 2^bits - 1 thresholds, ascending
  float cb[16];           // decode: the 2^bits centroids, ascending
  uint32_t tab[128][2];   // 4-bit encode: decision table by (sign, bucket of |u|), filled by the launcher
};

struct TqAttnArgs {
  const void* q;          // [bh_q, d] bf16 or fp32
  const uint8_t* kc;      // K codes [bh_kv, s_k, d kbits / 8]
  const float* kn;        // K norms [bh_kv, s_k]
  const uint8_t* vc;      // V codes [bh_kv, s_k, d vbits / 8]
  const float* vn;        // V norms [bh_kv, s_k]
  const int8_t* ks;       // K rotation signs [d]
  const int8_t* vs;       // V rotation signs [d]
  void* out;              // [bh_q, d]
  float* lse;             // [bh_q] or null
  float* partial;         // workspace [bh_q, num_splits, d + 2]: m, l, rotated O
  int32_t bh_q, bh_kv, group;
  int32_t s_k, key_lo, num_splits, tiles_per_split;
  int32_t q_bf16, out_bf16;
  float scale, scale_log2;
  // codebooks as three signed 7-bit digits of c[k] 2^-E (c[k] ~ 2^E (d0/2^7 + d1/2^14 + d2/2^21)),
  // byte k of digit t's 16-byte table; E per codebook
  uint32_t ktab[3][4];
  uint32_t vtab[3][4];
  int32_t k_e, v_e;
  EpiArgs epi;
  EpiArgs sops;           // score-scope ops, on n_j (q'.c[code]) before the softmax scale
};

// Query heads one decode workgroup serves: 8 (two MFMA column sets) for groups of more than 4
// heads at head_dim <= 128, else 4.  The split count and the grid both follow it.
inline int decode_heads_per_workgroup(int group, int head_dim) { return (group > 4 && head_dim <= 128) ? 8 : 4; }

// Size of the fixed device scratch array fa_decode_noalloc keeps its partial states in.
constexpr size_t kDecodeScratchBytes = size_t(4) << 20;

// Launchers return hipSuccess or the launch error; *name receives the instantiation name.
hipError_t launch_compress(const void* x, int32_t x_dtype, int64_t n_tokens, int32_t d,
                           int8_t* q_out, float* scale_out, hipStream_t stream, const char** name);
hipError_t launch_append(const AppendArgs& a, int32_t d, int32_t x_dtype, hipStream_t stream, const char** name);
hipError_t launch_prefill_f32(const PrefillArgs& a, int32_t d, int32_t kv_dtype, hipStream_t stream,
                              const char** name);
hipError_t launch_prefill_bf16(const PrefillArgs& a, int32_t d, hipStream_t stream, const char** name);
hipError_t launch_prefill_i8kv(const PrefillArgs& a, int32_t d, hipStream_t stream, const char** name);
hipError_t launch_decode(const DecodeArgs& a, int32_t d, hipStream_t stream, const char** name);
// Device address of this device's copy of the decode scratch array (looked up once per device,
// then cached); `device` must be the current device.
hipError_t decode_scratch_address(int device, void** ptr);
hipError_t launch_merge(const MergeArgs& a, int32_t d, hipStream_t stream, const char** name);
hipError_t launch_tq_attention(const TqAttnArgs& a, int32_t d, int32_t kbits, int32_t vbits, hipStream_t stream,
                               const char** name);
hipError_t launch_tq_encode(const TqArgs& a, int32_t d, int32_t bits, int32_t x_dtype, hipStream_t stream,
                            const char** name);
hipError_t launch_tq_decode(const TqArgs& a, int32_t d, int32_t bits, bool bf16_out, hipStream_t stream,
                            const char** name);
int tq_codebook(int32_t d, int32_t bits, float* centroids);   // host

}  // namespace fa
