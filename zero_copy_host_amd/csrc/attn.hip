// Prefill attention over one super-chunk of keys, for T new tokens per sequence.
//
// Follows "Paper Notes: DirectKV", System Architecture / Attention Fusion Engine, prefill
// strategy, and Key Ideas (1), CPU-memory-aware tiling: a KV tile fetched from host memory
// is held on chip and reused by every query that needs it, while the cost of reloading is
// moved to device-resident tensors (the queries and a running softmax state).
//
// gfx950 mapping. The stationary buffer for host KV is an XCD's L2 (4 MB), shared by the
// 32 CUs of that XCD, rather than one CU's LDS: the host calls this kernel once per key
// super-chunk [kc0, kc1) sized to fit L2, and workgroup x runs on XCD x % 8 (round-robin
// dispatch), so all query tiles of one (sequence, kv head) pair sit on one XCD and read the
// super-chunk from L2 after its first fetch over the link. Each workgroup keeps its query
// tile in registers, streams the super-chunk through a double-buffered LDS tile, and
// carries the per-row softmax state (o, m, l) in device memory from one super-chunk launch
// to the next. Keys below past_len[b] come from the host cache; this step's new keys come
// from the device copy the projection left, so they never cross the link a second time.
//
// MFMA layout: scores are computed transposed, Sᵀ = K·Qᵀ (32 keys x 32 queries per block),
// so each lane owns one query column: row max / sum need one cross-half exchange, the
// accumulators are reused directly as the Pᵀ operand of Oᵀ += Vᵀ·Pᵀ, and Oᵀ rescaling is
// lane-local. V is transposed once into LDS when a tile is loaded.
#include "dkv_internal.h"

namespace dkv {

template <typename T, int DH>
struct AttnCfg {
  static constexpr int KT = 64;                  // keys per LDS tile
  static constexpr int ROWS = 128;               // query rows per workgroup (4 waves x 32)
  static constexpr int EB = sizeof(T);
  static constexpr int VEC = 16 / EB;
  static constexpr int LDK = DH + VEC;           // K tile row (elements), padded
  static constexpr int LDV = KT + 16 / EB;       // Vᵀ tile row (elements), padded
  static constexpr int KTILE = KT * LDK;
  static constexpr int VTILE = DH * LDV;
  static constexpr int CHUNKS = KT * DH / VEC;   // 16-byte chunks per K (or V) tile
  static constexpr int LOADS = CHUNKS / 256;     // per thread
  static constexpr int DB = DH / 32;             // 32-row blocks of Oᵀ
};

template <typename T, int DH, int G>
__global__ __launch_bounds__(256) void attn_kernel(const AttnArgs a) {
  using C = AttnCfg<T, DH>;
  using MF = Mfma<T>;
  constexpr int KT = C::KT, VEC = C::VEC, LDK = C::LDK, LDV = C::LDV, LOADS = C::LOADS, DB = C::DB;
  constexpr int KPL = MF::KPL, KSTEP = MF::KSTEP;
  __shared__ __attribute__((aligned(16))) T sK[2][C::KTILE];
  __shared__ __attribute__((aligned(16))) T sV[2][C::VTILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  // workgroup -> (query tile, sequence, kv head); kv head fastest so x % 8 picks the XCD
  const int g = blockIdx.x % a.Hkv;
  const int rest = blockIdx.x / a.Hkv;
  const int b = rest % a.B;
  const int qt = rest / a.B;
  const int L = a.past_len[b];
  const int nrows = a.T * G;                     // query rows of this (b, g): t*G + hh
  const int row0 = qt * C::ROWS;
  if (row0 >= nrows) return;
  const int rlast = min(row0 + C::ROWS, nrows) - 1;
  const int key_hi = min(a.kc1, L + rlast / G + 1);   // keys any row here may see, exclusive
  const int key_lo = a.kc0;
  const bool work = key_lo < key_hi;
  if (!work && !a.last) return;                  // nothing visible and nothing to finalise

  // this lane's query row
  const int r = row0 + wave * 32 + col;
  const bool rvalid = r < nrows;
  const int t = rvalid ? r / G : 0;
  const int hh = r - (r / G) * G;
  const int qpos = L + t;                        // absolute position of the query
  const size_t bg = (size_t)b * a.Hkv + g;
  float* st = a.state + (bg * nrows + (rvalid ? r : 0)) * (DH + 2);

  // running state: Oᵀ blocks (lane owns its query column), m and l in the log2 domain
  f32x16 o[DB];
  float m_run = -INFINITY, l_run = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  if (!a.first && rvalid) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[db][v] = st[db * 32 + acc_row(v, lane)];
    m_run = st[DH];
    l_run = st[DH + 1];
  }

  if (work) {
    // Qᵀ operand fragments for this lane's query, held for the whole sweep
    typename MF::frag qf[DH / KSTEP];
    {
      const T* qrow = reinterpret_cast<const T*>(a.q) + (((size_t)b * a.T + t) * a.Hq + g * G + hh) * DH;
#pragma unroll
      for (int ks = 0; ks < DH / KSTEP; ++ks) {
        if (rvalid) qf[ks] = *reinterpret_cast<const typename MF::frag*>(qrow + ks * KSTEP + half * KPL);
        else qf[ks] = typename MF::frag{};
      }
    }
    const float sl2 = 1.4426950408889634f * rsqrtf((float)DH);   // log2(e)/sqrt(d)

    const T* __restrict__ kh = reinterpret_cast<const T*>(a.kc) + bg * a.cap * DH;
    const T* __restrict__ vh = reinterpret_cast<const T*>(a.vc) + bg * a.cap * DH;
    const T* __restrict__ kn = reinterpret_cast<const T*>(a.k_new) + bg * a.T * DH;
    const T* __restrict__ vn = reinterpret_cast<const T*>(a.v_new) + bg * a.T * DH;

    uint4 rk[LOADS], rv[LOADS];
    auto gload = [&](int j0) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int c = tid + i * 256;
        const int kr = c / (DH / VEC), kc = (c % (DH / VEC)) * VEC;
        const int j = j0 + kr;
        if (j < key_hi) {
          const T* ks = j < L ? kh + (size_t)j * DH : kn + (size_t)(j - L) * DH;
          const T* vs = j < L ? vh + (size_t)j * DH : vn + (size_t)(j - L) * DH;
          rk[i] = *reinterpret_cast<const uint4*>(ks + kc);
          rv[i] = *reinterpret_cast<const uint4*>(vs + kc);
        } else {
          rk[i] = make_uint4(0, 0, 0, 0);
          rv[i] = make_uint4(0, 0, 0, 0);
        }
      }
    };
    auto sstore = [&](int buf) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int c = tid + i * 256;
        const int kr = c / (DH / VEC), kc = (c % (DH / VEC)) * VEC;
        *reinterpret_cast<uint4*>(&sK[buf][kr * LDK + kc]) = rk[i];
        const T* ve = reinterpret_cast<const T*>(&rv[i]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) sV[buf][(kc + e) * LDV + kr] = ve[e];
      }
    };

    gload(key_lo);
    sstore(0);
    __syncthreads();
    int buf = 0;
    for (int j0 = key_lo; j0 < key_hi; j0 += KT) {
      const bool more = j0 + KT < key_hi;
      if (more) gload(j0 + KT);
      const T* tK = sK[buf];
      const T* tV = sV[buf];
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb) {
        // Sᵀ block: 32 keys (rows) x 32 queries (columns)
        f32x16 s;
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < DH / KSTEP; ++ks) {
          const typename MF::frag ka =
              *reinterpret_cast<const typename MF::frag*>(tK + (kb * 32 + col) * LDK + ks * KSTEP + half * KPL);
          s = MF::mma(ka, qf[ks], s);
        }
        // scale, causal mask, and the column (query) maximum
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = j0 + kb * 32 + acc_row(v, lane);
          const bool ok = rvalid && j < key_hi && j <= qpos;
          s[v] = ok ? s[v] * sl2 : -INFINITY;
          mx = fmaxf(mx, s[v]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        if (m_new != -INFINITY) {
          const float alpha = exp2f(m_run - m_new);
          float ps = 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            s[v] = exp2f(s[v] - m_new);
            ps += s[v];
          }
          ps += __shfl_xor(ps, 32, 64);
          l_run = l_run * alpha + ps;
          m_run = m_new;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v) s[v] = 0.f;
        }
        // Oᵀ += Vᵀ · Pᵀ: reduction slot (half, e) of step st is the key held in
        // accumulator register st*KPL + e of that half
#pragma unroll
        for (int stp = 0; stp < 32 / KSTEP; ++stp) {
          typename MF::frag pb;
          if constexpr (KPL == 1) {
            pb = s[stp];
          } else {
#pragma unroll
            for (int e = 0; e < KPL; ++e) pb[e] = Elem<T>::from_float(s[stp * KPL + e]);
          }
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            typename MF::frag va;
            const T* vrow = tV + (db * 32 + col) * LDV + kb * 32;
            if constexpr (KPL == 1) {
              va = vrow[acc_row(stp, lane)];
            } else {
              // keys acc_row(stp*8 + e): two runs of four consecutive keys
#pragma unroll
              for (int e = 0; e < KPL; ++e) va[e] = vrow[acc_row(stp * KPL + e, lane)];
            }
            o[db] = MF::mma(va, pb, o[db]);
          }
        }
      }
      if (more) sstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  if (!rvalid) return;
  if (a.last) {
    const float inv = 1.f / l_run;
    T* orow = reinterpret_cast<T*>(a.out) + (((size_t)b * a.T + t) * a.Hq + g * G + hh) * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) orow[db * 32 + acc_row(v, lane)] = Elem<T>::from_float(o[db][v] * inv);
  } else {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) st[db * 32 + acc_row(v, lane)] = o[db][v];
    st[DH] = m_run;
    st[DH + 1] = l_run;
  }
}

template <typename T, int DH, int G>
static hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const int grid = a.q_tiles * a.B * a.Hkv;
  hipLaunchKernelGGL((attn_kernel<T, DH, G>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int DH>
static attn_fn pick_g(int G) {
  switch (G) {
    case 1: return launch_attn<T, DH, 1>;
    case 2: return launch_attn<T, DH, 2>;
    case 4: return launch_attn<T, DH, 4>;
    case 8: return launch_attn<T, DH, 8>;
    default: return nullptr;
  }
}

template <typename T>
static attn_fn pick_d(int d, int G) {
  if (d == 64) return pick_g<T, 64>(G);
  if (d == 128) return pick_g<T, 128>(G);
  return nullptr;
}

attn_fn find_attn(int dtype, int d, int G) {
  switch (dtype) {
    case 0: return pick_d<float>(d, G);
    case 1: return pick_d<_Float16>(d, G);
    case 2: return pick_d<__bf16>(d, G);
    default: return nullptr;
  }
}

int attn_rows_per_tile() { return 128; }

}  // namespace dkv
