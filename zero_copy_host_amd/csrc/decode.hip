// Decode step: one new token per sequence attends to its whole host-resident KV cache.
//
// Follows "Paper Notes: DirectKV", System Architecture / Attention Fusion Engine, decode
// strategy: the single query sweeps every cached (K, V) row, and intermediate output is
// not re-read from device memory while it does. Each workgroup owns one (sequence b,
// kv head g, split s): it projects q for the G query heads of the group (and, in the
// split holding the new position, k and v of the new token, which it stores to the host
// cache row past_len[b]), then streams its share of host rows exactly once and writes one
// softmax partial (o, m, l). A small combine kernel merges the partials.
//
// On gfx950 the host rows are read by ordinary 16-byte vector loads from pinned mapped
// memory into registers: this path is a scan of the host link (about G flops per host
// byte), so latency is hidden by many resident waves with a full iteration of loads in
// flight each, and no LDS staging is needed for the key/value rows.
#include "dkv_internal.h"

namespace dkv {

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// dst[r] = scale * sum_k sx[k] * w[(row0 + r) * D + k] for r < nrows (w is [rows, D]).
// Waves take R rows at a time so that R weight loads per lane are in flight together.
template <typename T, int R>
__device__ void project_rows(const float* __restrict__ sx, const T* __restrict__ w, int D,
                             int row0, int nrows, float* __restrict__ dst, float scale) {
  constexpr int VEC = Elem<T>::VEC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  for (int r0 = wave * R; r0 < nrows; r0 += nwaves * R) {
    float acc[R];
#pragma unroll
    for (int i = 0; i < R; ++i) acc[i] = 0.f;
    for (int k = lane * VEC; k < D; k += 64 * VEC) {
      float xs[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) xs[e] = sx[k + e];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        if (r0 + i < nrows) {
          const uint4 raw = *reinterpret_cast<const uint4*>(w + (size_t)(row0 + r0 + i) * D + k);
          float f[VEC];
          Elem<T>::unpack(raw, f);
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[i] = fmaf(f[e], xs[e], acc[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) acc[i] = wave_sum(acc[i]);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < R; ++i)
        if (r0 + i < nrows) dst[r0 + i] = acc[i] * scale;
    }
  }
}

// log2(e)/sqrt(d). Scores, maxima and partial maxima stay raw dot products q.k; the scale is
// applied once, to the difference from the maximum, as exp2((s - m) * c): that difference is
// exact in fp32 for the keys that carry weight (they lie within a factor 2 of the maximum), so
// the weights keep full fp32 precision however large the scores are. (Scaling q first would
// round every product and partial sum at the scores' magnitude.)
__device__ inline float score_scale(int dh) { return 1.4426950408889634f * rsqrtf((float)dh); }

// The queries of a decode step, every (sequence, query head), projected once:
// qf[b][n] = sum_k x[b][k] * wq[n][k]. Each weight row streams from HBM once per
// BB sequences. The sum over k runs in project_rows' order (lane-strided vectors of VEC, fma in
// order, then the wave's xor tree), so these are bitwise the values a decode workgroup would
// compute for itself.
template <typename T, int DH, int R, int BB>
__global__ __launch_bounds__(256) void qproj_kernel(const DecodeArgs a) {
  constexpr int VEC = Elem<T>::VEC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nrows = a.Hq * DH;
  const int r0 = (blockIdx.x * 4 + wave) * R;
  const int b0 = blockIdx.y * BB;
  const int nb = min(BB, a.B - b0);
  if (r0 >= nrows) return;
  const T* __restrict__ w = reinterpret_cast<const T*>(a.wq);
  const T* __restrict__ x = reinterpret_cast<const T*>(a.x) + (size_t)b0 * a.D;
  float acc[R][BB];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < BB; ++j) acc[i][j] = 0.f;
  // several k steps of weight loads in flight per wave (the loop bound keeps every load in D)
#pragma unroll 4
  for (int k = lane * VEC; k < a.D; k += 64 * VEC) {
    float f[R][VEC];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      // a row past the end reads row 0 (in bounds); its sums are never stored
      const int row = r0 + i < nrows ? r0 + i : 0;
      Elem<T>::unpack(*reinterpret_cast<const uint4*>(w + (size_t)row * a.D + k), f[i]);
    }
#pragma unroll
    for (int j = 0; j < BB; ++j) {
      if (j < nb) {
        float xs[VEC];
        Elem<T>::unpack(*reinterpret_cast<const uint4*>(x + (size_t)j * a.D + k), xs);
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[i][j] = fmaf(f[i][e], xs[e], acc[i][j]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < BB; ++j) {
      const float v = wave_sum(acc[i][j]);
      if (lane == 0 && j < nb && r0 + i < nrows) a.qf[(size_t)(b0 + j) * nrows + r0 + i] = v;
    }
}

template <typename T, int DH, int G>
struct DecodeCfg {
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int LPR = DH / VEC;       // lanes holding one key row
  static constexpr int RPW = 64 / LPR;       // key rows per wave per step
  static constexpr int NSLOT = 4 * RPW;      // key rows per workgroup per step
  static constexpr int U = 4;                // steps per loop iteration (loads in flight)
  static constexpr int MERGE = NSLOT * G * DH + 2 * NSLOT * G;
  static constexpr int SMEM = MERGE > kMaxD ? MERGE : kMaxD;
};

// PAGED: the cache is a page pool addressed through the block table; the page ids of this
// split's rows are staged in LDS first, so row loads never wait on a table load.
template <typename T, int DH, int G, bool PAGED>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeArgs a) {
  using C = DecodeCfg<T, DH, G>;
  constexpr int VEC = C::VEC, LPR = C::LPR, RPW = C::RPW, NSLOT = C::NSLOT, U = C::U;
  __shared__ float s_buf[C::SMEM];   // activation row, then the per-slot merge area
  __shared__ float s_q[G * DH];
  __shared__ float s_kv[2 * DH];     // the new token's k and v (rounded to T)
  __shared__ int32_t s_pages[PAGED ? kPagedDecodeChunk / kPageTokens + 1 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.y;
  const int gs = blockIdx.x;
  int b = 0;
  while (b + 1 < a.B && a.split_begin[b + 1] <= gs) ++b;
  const int s = gs - a.split_begin[b];
  const int L = a.past_len[b];
  const int k0 = s * a.chunk;
  const int k1 = min(k0 + a.chunk, L + 1);
  const bool has_new = (k1 == L + 1);
  const int kp_end = min(k1, L);            // host rows [k0, kp_end) are read here
  const size_t bg = (size_t)b * a.Hkv + g;
  const T* __restrict__ kbase = reinterpret_cast<const T*>(a.kc) + (PAGED ? 0 : bg * a.cap * DH);
  const T* __restrict__ vbase = reinterpret_cast<const T*>(a.vc) + (PAGED ? 0 : bg * a.cap * DH);
  const int pg0 = k0 / kPageTokens;           // first page of this split
  if constexpr (PAGED) {
    const int npg = kp_end > k0 ? (kp_end - 1) / kPageTokens - pg0 + 1 : 0;
    for (int i = tid; i < npg; i += blockDim.x) s_pages[i] = a.table[(size_t)b * a.max_pages + pg0 + i];
  }

  // ---- projection of this token: q for heads g*G .. g*G+G-1 (and k, v if new). With several
  // splits per sequence the queries come projected once per step (a.qf, qproj_kernel), so the
  // Wq slice (G*d rows of D) is not read again by every split of the group.
  if (!a.qf || has_new) {
    const T* __restrict__ xrow = reinterpret_cast<const T*>(a.x) + (size_t)b * a.D;
    for (int k = tid; k < a.D; k += blockDim.x) s_buf[k] = Elem<T>::to_float(xrow[k]);
  }
  __syncthreads();
  if (a.qf) {
    const float* __restrict__ qsrc = a.qf + (size_t)b * a.Hq * DH + (size_t)g * G * DH;
    for (int i = tid; i < G * DH; i += blockDim.x) s_q[i] = qsrc[i];
  } else {
    project_rows<T, 8>(s_buf, reinterpret_cast<const T*>(a.wq), a.D, g * G * DH, G * DH, s_q, 1.f);
  }
  if (has_new) {
    project_rows<T, 8>(s_buf, reinterpret_cast<const T*>(a.wk), a.D, g * DH, DH, s_kv, 1.f);
    project_rows<T, 8>(s_buf, reinterpret_cast<const T*>(a.wv), a.D, g * DH, DH, s_kv + DH, 1.f);
  }
  __syncthreads();
  if (a.rope_theta > 0.0) {
    // rotary embedding at this token's position L: the G query heads and (if projected here) the
    // new key, pair (i, i + d/2) of each head, before the key is rounded and stored
    constexpr int HALF = DH / 2;
    const int nvec = G + (has_new ? 1 : 0);
    for (int idx = tid; idx < nvec * HALF; idx += blockDim.x) {
      const int h = idx / HALF, i = idx - h * HALF;
      float* v = h < G ? s_q + h * DH : s_kv;
      double c, sn;
      rope_angle_cs(L, i, DH, a.rope_theta, c, sn);
      const float lo = v[i], hi = v[i + HALF];
      v[i] = lo * (float)c - hi * (float)sn;
      v[i + HALF] = hi * (float)c + lo * (float)sn;
    }
    __syncthreads();
  }
  if (has_new) {
    // storer: round to the cache dtype and write host row L; attention below uses the
    // rounded values from LDS, never reading the row back over the link
    const size_t row = host_row(PAGED ? a.table : nullptr, a.max_pages, b, g, a.Hkv, a.cap, L);
    T* krow = reinterpret_cast<T*>(a.kc) + row * DH;
    T* vrow = reinterpret_cast<T*>(a.vc) + row * DH;
    for (int i = tid; i < 2 * DH; i += blockDim.x) {
      const T r = Elem<T>::from_float(s_kv[i]);
      if (i < DH) krow[i] = r; else vrow[i - DH] = r;
    }
    __syncthreads();
    for (int i = tid; i < 2 * DH; i += blockDim.x) s_kv[i] = Elem<T>::to_float(Elem<T>::from_float(s_kv[i]));
    __syncthreads();
  }

  // ---- stream the host rows
  const float c = score_scale(DH);
  const int slot = wave * RPW + lane / LPR;
  const int col = (lane % LPR) * VEC;
  float q[G][VEC], o[G][VEC], m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) { q[h][e] = s_q[h * DH + col + e]; o[h][e] = 0.f; }
  }

  auto fetch = [&](int base, uint4 (&kk)[U], uint4 (&vv)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u * NSLOT + slot;
      if (key < kp_end) {
        size_t row = key;
        if constexpr (PAGED)
          row = ((size_t)s_pages[key / kPageTokens - pg0] * a.Hkv + g) * kPageTokens + key % kPageTokens;
        kk[u] = *reinterpret_cast<const uint4*>(kbase + row * DH + col);
        vv[u] = *reinterpret_cast<const uint4*>(vbase + row * DH + col);
      } else {
        kk[u] = make_uint4(0, 0, 0, 0);
        vv[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  // one online-softmax update with U key rows per slot; invalid rows carry -inf scores
  auto consume = [&](int base, const uint4 (&kk)[U], const uint4 (&vv)[U]) {
    float sc[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VEC];
      Elem<T>::unpack(kk[u], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc = fmaf(q[h][e], kf[e], acc);
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
        sc[u][h] = acc;
      }
      const int key = base + u * NSLOT + slot;
      if (key >= kp_end) {
#pragma unroll
        for (int h = 0; h < G; ++h) sc[u][h] = -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = m[h];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][h]);
      if (mx == -INFINITY) continue;            // nothing valid seen yet
      const float alpha = exp2f((m[h] - mx) * c);   // exp2(-inf) = 0 on the first update
      m[h] = mx;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[h][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = exp2f((sc[u][h] - mx) * c);
        l[h] += p;
        sc[u][h] = p;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[VEC];
      Elem<T>::unpack(vv[u], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (m[h] == -INFINITY) continue;
        const float p = sc[u][h];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[h][e] = fmaf(p, vf[e], o[h][e]);
      }
    }
  };

  if (k0 < kp_end) {
    uint4 kc0[U], vc0[U], kc1[U], vc1[U];
    fetch(k0, kc0, vc0);
    int base = k0;
    constexpr int STEP = U * NSLOT;
    // two register sets: the next iteration's loads are issued before this one computes
    while (true) {
      const int nb = base + STEP;
      if (nb < kp_end) fetch(nb, kc1, vc1);
      consume(base, kc0, vc0);
      if (nb >= kp_end) break;
      base = nb;
      const int nb2 = base + STEP;
      if (nb2 < kp_end) fetch(nb2, kc0, vc0);
      consume(base, kc1, vc1);
      if (nb2 >= kp_end) break;
      base = nb2;
    }
  }

  // the new token's own key: folded in by slot 0 from LDS
  if (has_new && slot == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc = fmaf(q[h][e], s_kv[col + e], acc);
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
      const float mx = fmaxf(m[h], acc);
      const float alpha = exp2f((m[h] - mx) * c);
      const float p = exp2f((acc - mx) * c);
      m[h] = mx;
      l[h] = l[h] * alpha + p;
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[h][e] = fmaf(p, s_kv[DH + col + e], o[h][e] * alpha);
    }
  }

  // ---- merge the NSLOT slot states of this workgroup and write one partial per head
  __syncthreads();   // s_buf is reused
  float* s_o = s_buf;                        // [NSLOT][G][DH]
  float* s_m = s_buf + NSLOT * G * DH;       // [NSLOT][G]
  float* s_l = s_m + NSLOT * G;
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) s_o[(slot * G + h) * DH + col + e] = o[h][e];
    if (lane % LPR == 0) { s_m[slot * G + h] = m[h]; s_l[slot * G + h] = l[h]; }
  }
  __syncthreads();
  float* part = a.part + ((size_t)gs * a.Hq + (size_t)g * G) * (DH + 2);
  for (int idx = tid; idx < G * DH; idx += blockDim.x) {
    const int h = idx / DH, i = idx % DH;
    float M = -INFINITY;
    for (int sl = 0; sl < NSLOT; ++sl) M = fmaxf(M, s_m[sl * G + h]);
    float acc = 0.f, lsum = 0.f;
    for (int sl = 0; sl < NSLOT; ++sl) {
      const float ms = s_m[sl * G + h];
      if (ms == -INFINITY) continue;
      const float w = exp2f((ms - M) * c);
      acc = fmaf(s_o[(sl * G + h) * DH + i], w, acc);
      lsum = fmaf(s_l[sl * G + h], w, lsum);
    }
    if (a.direct) {
      // the only split of this sequence: its merged state is the output (what the combine
      // would compute from it, with weight 2^0 = 1)
      T* orow = reinterpret_cast<T*>(a.out) + ((size_t)b * a.Hq + (size_t)g * G + h) * DH;
      orow[i] = Elem<T>::from_float(acc / lsum);
    } else {
      float* ph = part + (size_t)h * (DH + 2);
      ph[i] = acc;
      if (i == 0) { ph[DH] = M; ph[DH + 1] = lsum; }
    }
  }
}

// Merge the splits of every (sequence, query head):
// O = sum_s o_s 2^((m_s - M) c) / sum_s l_s 2^((m_s - M) c), with raw maxima m_s and c = score_scale.
template <typename T, int DH>
__global__ __launch_bounds__(DH) void combine_kernel(const CombineArgs a) {
  const int b = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
  const float c = score_scale(DH);
  const int s0 = a.split_begin[b], s1 = a.split_begin[b + 1];
  float M = -INFINITY;
  for (int s = s0; s < s1; ++s) M = fmaxf(M, a.part[((size_t)s * a.Hq + h) * (DH + 2) + DH]);
  float acc = 0.f, lsum = 0.f;
  for (int s = s0; s < s1; ++s) {
    const float* p = a.part + ((size_t)s * a.Hq + h) * (DH + 2);
    const float w = exp2f((p[DH] - M) * c);
    acc = fmaf(p[i], w, acc);
    lsum = fmaf(p[DH + 1], w, lsum);
  }
  T* out = reinterpret_cast<T*>(a.out) + ((size_t)b * a.Hq + h) * DH;
  out[i] = Elem<T>::from_float(acc / lsum);
}

template <typename T, int DH, int G, bool PAGED>
static hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<T, DH, G, PAGED>), dim3(a.n_splits, a.Hkv), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int DH>
static hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((combine_kernel<T, DH>), dim3(a.B, a.Hq), dim3(DH), 0, s, a);
  return hipGetLastError();
}

constexpr int kQprojRows = 1;    // weight rows per wave: many waves per SIMD hide the HBM latency
constexpr int kQprojBatch = 8;   // sequences per workgroup (more go to further grid rows)

template <typename T, int DH>
static hipError_t launch_qproj(const DecodeArgs& a, hipStream_t s) {
  const int rows_per_wg = 4 * kQprojRows;
  const dim3 grid((a.Hq * DH + rows_per_wg - 1) / rows_per_wg, (a.B + kQprojBatch - 1) / kQprojBatch);
  hipLaunchKernelGGL((qproj_kernel<T, DH, kQprojRows, kQprojBatch>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---- pre-instantiated kernel table (dtype x head_dim x group size x cache layout)
template <typename T, int DH, bool PAGED>
static decode_fn pick_g(int G) {
  switch (G) {
    case 1: return launch_decode<T, DH, 1, PAGED>;
    case 2: return launch_decode<T, DH, 2, PAGED>;
    case 4: return launch_decode<T, DH, 4, PAGED>;
    case 8: return launch_decode<T, DH, 8, PAGED>;
    default: return nullptr;
  }
}

template <typename T>
static decode_fn pick_d(int d, int G, bool paged) {
  if (d == 64) return paged ? pick_g<T, 64, true>(G) : pick_g<T, 64, false>(G);
  if (d == 128) return paged ? pick_g<T, 128, true>(G) : pick_g<T, 128, false>(G);
  return nullptr;
}

decode_fn find_decode(int dtype, int d, int G, bool paged) {
  switch (dtype) {
    case 0: return pick_d<float>(d, G, paged);
    case 1: return pick_d<_Float16>(d, G, paged);
    case 2: return pick_d<__bf16>(d, G, paged);
    default: return nullptr;
  }
}

combine_fn find_combine(int dtype, int d) {
  if (d != 64 && d != 128) return nullptr;
  switch (dtype) {
    case 0: return d == 64 ? launch_combine<float, 64> : launch_combine<float, 128>;
    case 1: return d == 64 ? launch_combine<_Float16, 64> : launch_combine<_Float16, 128>;
    case 2: return d == 64 ? launch_combine<__bf16, 64> : launch_combine<__bf16, 128>;
    default: return nullptr;
  }
}

qproj_fn find_qproj(int dtype, int d) {
  if (d != 64 && d != 128) return nullptr;
  switch (dtype) {
    case 0: return d == 64 ? launch_qproj<float, 64> : launch_qproj<float, 128>;
    case 1: return d == 64 ? launch_qproj<_Float16, 64> : launch_qproj<_Float16, 128>;
    case 2: return d == 64 ? launch_qproj<__bf16, 64> : launch_qproj<__bf16, 128>;
    default: return nullptr;
  }
}

int decode_slots(int dtype, int d) {
  const int vec = dtype == 0 ? 4 : 8;
  const int lpr = d / vec;
  return 4 * (64 / lpr) * 4;  // NSLOT * U: key rows per loop iteration
}

}  // namespace dkv
