// Internal declarations shared by the HIP kernels and the C-ABI layer of the host-KV
// attention library (gfx950 / CDNA4 only: wave64, 32x32 MFMA, 160 KB LDS per CU).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dkv {

constexpr int kMaxBatch = 256;   // sequences per call (lengths travel in kernel arguments)
constexpr int kMaxD = 8192;      // model width held in LDS by the decode kernel
constexpr int kPageTokens = 16;  // token rows per page of a paged host cache
constexpr int kProjSmallRows = 256;   // projections of at most this many token rows take the small-tile kernel
constexpr int kMaxKeySplits = 32;     // key splits per pair at most, prefills of one query tile per pair
constexpr int kPagedDecodeChunk = 8192;  // keys per decode split at most, paged caches
constexpr int kPagedSuperchunk = 16384;  // keys per prefill launch at most, paged caches
constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

// ------------------------------------------------------------------ element traits
// Each element type is moved in 16-byte vectors (VEC elements) and computed in fp32.
template <typename T> struct Elem;

template <> struct Elem<__bf16> {
  static constexpr int VEC = 8;
  static constexpr int BYTES = 2;
  __device__ static inline void unpack(const uint4& r, float (&f)[8]) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static inline __bf16 from_float(float f) { return static_cast<__bf16>(f); }
  __device__ static inline float to_float(__bf16 x) { return static_cast<float>(x); }
  // acc + a + b in one dot2 instruction (fp32 accumulation)
  __device__ static inline float dot2_ones(__bf16 a, __bf16 b, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a, b}, one, acc, false);
  }
};

template <> struct Elem<_Float16> {
  static constexpr int VEC = 8;
  static constexpr int BYTES = 2;
  __device__ static inline void unpack(const uint4& r, float (&f)[8]) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      _Float16 lo, hi;
      uint16_t l16 = (uint16_t)(w[i] & 0xFFFFu), h16 = (uint16_t)(w[i] >> 16);
      __builtin_memcpy(&lo, &l16, 2);
      __builtin_memcpy(&hi, &h16, 2);
      f[2 * i] = (float)lo;
      f[2 * i + 1] = (float)hi;
    }
  }
  __device__ static inline _Float16 from_float(float f) { return static_cast<_Float16>(f); }
  __device__ static inline float to_float(_Float16 x) { return static_cast<float>(x); }
  __device__ static inline float dot2_ones(_Float16 a, _Float16 b, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(f16x2{a, b}, one, acc, false);
  }
};

template <> struct Elem<float> {
  static constexpr int VEC = 4;
  static constexpr int BYTES = 4;
  __device__ static inline void unpack(const uint4& r, float (&f)[4]) {
    f[0] = __uint_as_float(r.x);
    f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z);
    f[3] = __uint_as_float(r.w);
  }
  __device__ static inline float from_float(float f) { return f; }
  __device__ static inline float to_float(float x) { return x; }
};

// ------------------------------------------------------------------ MFMA traits
// 32x32 output block per wave instruction. Operand slot (lane l, element e) carries
// row/column l % 32 and reduction index (l / 32) * KPL + e; accumulator register v of
// lane l holds row 8*(v/4) + 4*(l/32) + v%4, column l % 32 (checked on gfx950).
template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
  static constexpr int KPL = 8;   // reduction elements per lane per instruction
  static constexpr int KSTEP = 16;
  typedef bf16x8 frag;
  __device__ static inline f32x16 mma(const frag& a, const frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<_Float16> {
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 16;
  typedef f16x8 frag;
  __device__ static inline f32x16 mma(const frag& a, const frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 2;
  typedef float frag;
  __device__ static inline f32x16 mma(const frag& a, const frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Row index (in rows of d elements) of token j of (sequence b, kv head g) in a host cache:
// contiguous [B][Hkv][cap][d], or paged, pool [n_pages][Hkv][kPageTokens][d] with the page of
// token j at table[b * max_pages + j / kPageTokens].
__device__ inline size_t host_row(const int32_t* table, int max_pages, int b, int g, int Hkv, int cap, int j) {
  if (table) {
    const int pg = table[(size_t)b * max_pages + j / kPageTokens];
    return ((size_t)pg * Hkv + g) * kPageTokens + j % kPageTokens;
  }
  return ((size_t)b * Hkv + g) * cap + j;
}

__device__ inline int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// Rotary angle of pair i (of d/2) at position pos: pos * theta^(-2i/d), in fp64, and its cosine and
// sine (fp64 library routines with their own argument reduction; a long position turns the first
// pairs through ~1e5 radians, which fp32 would carry with ~1e-2 radians of error).
__device__ inline void rope_angle_cs(int pos, int i, int d, double theta, double& c, double& s) {
  const double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)d);
  sincos(ang, &s, &c);
}

// Lanes l and l + 32 hold the same query row in the transposed score layout: combine their
// values with one lane-swap instruction (v_permlane32_swap: result[0] is x with its upper half
// replaced by the lower half, result[1] x with its lower half replaced by the upper half).
__device__ inline float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------------------ launch arguments
// Y = X·Wᵀ over up to three weight segments (Q, K, V) sharing one activation matrix.
struct ProjArgs {
  const void* x;            // [M = B*T, D]
  const void* w[3];         // segment weights [n_seg, D]; Q, K, V
  int32_t n_seg[3];         // output features per segment (0 = segment absent)
  int32_t tiles_seg[3];     // column tiles per segment (set by the launcher)
  int32_t M, D, T, B, d, Hkv, cap;
  void* q_out;              // [M, n_seg[0]] device (segment 0)
  void* kc;                 // host cache K (segment 1), rows [past_len[b] + t]
  void* vc;                 // host cache V (segment 2)
  void* k_dev;              // optional device copy of the new K rows [B, Hkv, T, d]
  void* v_dev;              // optional device copy of the new V rows
  int32_t host_out;         // 1: write the new K/V rows to the host cache (segments 1, 2)
  const int32_t* table;     // paged cache: device block table [B][max_pages]; null = contiguous
  int32_t max_pages;
  const float2* rope_cs;    // rotary embedding: (cos, sin) of row m = b*T + t, pair i at [m * d/2 + i]
                            // (rope_table_kernel); null = no rotation. Rotates Q and K (segments 0, 1)
  int32_t past_len[kMaxBatch];
};

struct DecodeArgs {
  const void* x;            // [B, D]
  const void* wq;           // [Hq*d, D]
  const void* wk;           // [Hkv*d, D]
  const void* wv;
  void* kc;                 // host cache
  void* vc;
  float* part;              // [n_splits_total][Hq][d + 2]: o (unnormalised), m, l
  void* out;                // [B, Hq*d]: written here directly when `direct`
  int32_t direct;           // 1: every sequence has one split, whose merged state is the output
                            // (no partials, no combine launch)
  float* qf;                // [B][Hq*d] queries projected once per step (fp32, unscaled), or
                            // null: each workgroup projects its own
  int32_t B, D, Hq, Hkv, cap, n_splits;
  const int32_t* table;     // paged cache: device block table [B][max_pages] (paged instances)
  int32_t max_pages;
  int32_t past_len[kMaxBatch];
  int32_t split_begin[kMaxBatch + 1];  // first global split of sequence b
  int32_t chunk;                       // keys per split
  double rope_theta;                   // rotary embedding base for q and the new k; 0 = none
};

struct CombineArgs {
  const float* part;
  void* out;                // [B, Hq*d]
  int32_t B, Hq, n_splits;
  int32_t split_begin[kMaxBatch + 1];
};

// Prefill attention over one super-chunk of keys [kc0, kc1) (absolute positions), updating a
// per-row running softmax state in device memory, plus a share of the work over this step's own
// keys (see attn_kernel).
struct AttnArgs {
  const void* q;            // [B, T, Hq, d] device
  const void* kc;           // host cache (rows < past_len[b] are read from here)
  const void* vc;
  const void* k_new;        // [B, Hkv, T, d] device copy of this step's rows
  const void* v_new;
  float* state;             // running o, m, l (log2 domain) per 32 query rows: see attn_state_bytes
  float* nstate;            // the same for this step's own keys (own-key items)
  void* out;                // [B, T, Hq*d]
  int32_t B, T, Hq, Hkv, cap;
  int32_t pair0, pairs;     // this launch serves (sequence, kv head) pairs [pair0, pair0 + pairs)
  int32_t kc0, kc1;         // super-chunk key range
  int32_t first, last;      // first super-chunk (no state to read) / last (finalise)
  int32_t q_tiles;          // row tiles per (b, g)
  int32_t xcd_group;        // 1: pair p is served only by XCD p % 8 (needs B*Hkv >= 8)
  int32_t new_from_host;    // 1: this step's rows are read back from the host cache too
  int32_t past_items;       // 1: the launch holds the q_tiles past-key items of every pair
  int32_t clip_past;        // 1: past-key items stop at past_len[b] (own keys are own-key items)
  int32_t fetchers;         // past-key items per pair dispatched before the own-key items
  int32_t dev_q0, dev_q1;   // own-key items of query tiles [dev_q0, dev_q1) per pair
  int32_t dev_final;        // 1: own-key items finalise the output (no past keys anywhere)
  int32_t merge_new;        // 1: finalising past-key items fold in nstate
  int32_t store_new;        // 1: own-key items write their tokens' new rows to the host cache
  int32_t n_splits;         // key-split mode (one query tile per pair): key splits per pair; 0 = off
  int32_t split_combine;    // key-split mode: 0 = the split items, 1 = the items merging their states
  int64_t split_stride;     // key-split mode: floats between two splits' state arrays (from `state`)
  int32_t split_storers;    // key-split mode: workgroups after the split items that copy this step's
                            // new K/V rows from their device copies to the host cache
  int32_t chunked;          // two-launch prefill: 1 = the chunk launch, 2 = the finish launch, 0 = off
                            // (n_splits = past super-chunks, split_stride = floats between their states)
  int32_t chunk_keys;       // two-launch prefill: keys per past super-chunk
  int32_t chunk_insert;     // two-launch prefill: chunk j's items dispatched before chunk j+1's fetchers
  int32_t n_own0;           // two-launch prefill: own-key items of query tiles [0, n_own0) in the chunk launch
  const int32_t* table;     // paged cache: device block table [B][max_pages] (paged instances)
  int32_t max_pages;
  int32_t past_len[kMaxBatch];
};

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error; argument checks happen in the ABI layer.
typedef hipError_t (*proj_fn)(const ProjArgs&, hipStream_t);
typedef hipError_t (*decode_fn)(const DecodeArgs&, hipStream_t);
typedef hipError_t (*combine_fn)(const CombineArgs&, hipStream_t);
typedef hipError_t (*attn_fn)(const AttnArgs&, hipStream_t);
typedef hipError_t (*qproj_fn)(const DecodeArgs&, hipStream_t);   // fills a.qf

proj_fn find_proj(int dtype, int d);
decode_fn find_decode(int dtype, int d, int G, bool paged);
combine_fn find_combine(int dtype, int d);
qproj_fn find_qproj(int dtype, int d);
attn_fn find_attn(int dtype, int d, int G, bool paged);

int decode_slots(int dtype, int d);  // key rows one decode WG consumes per step
int attn_rows_per_tile();            // query rows (token x head) per prefill WG
size_t attn_state_bytes(int d, int batch, int n_kv_heads, int T, int G);
int attn_key_tile(int dtype, int d);  // keys per LDS tile of the prefill attention

hipError_t launch_hostlink(void* p, size_t bytes, int mode, int n_wg, hipStream_t s);

// (cos, sin) of the rotary angle (past_len[b] + t) * theta^(-2i/d) for every row m = b*T + t of a
// call and pair i < d/2, into cs[m * d/2 + i] (proj.hip)
hipError_t launch_rope_table(const int32_t* past_len, int B, int T, int d, double theta, float2* cs,
                             hipStream_t s);

// decode-loop kernels around the layer (model.hip); dtype as dkv_dtype
hipError_t launch_rmsnorm(int dtype, const void* x, const void* w, void* y, int rows, int D, float eps,
                          hipStream_t s);
hipError_t launch_linear(int dtype, const void* x, const void* w, const void* res, void* y, int rows, int N, int K,
                         hipStream_t s);
hipError_t launch_swiglu(int dtype, const void* gu, void* y, int rows, int F, hipStream_t s);

}  // namespace dkv
