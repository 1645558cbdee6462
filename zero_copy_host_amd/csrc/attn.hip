// Prefill attention over one super-chunk of keys, for T new tokens per sequence.
//
// Follows "Paper Notes: DirectKV", System Architecture / Attention Fusion Engine, prefill
// strategy, and Key Ideas (1), CPU-memory-aware tiling: a KV tile fetched from host memory
// is held on chip and reused by every query that needs it, while the cost of reloading is
// moved to device-resident tensors (the queries and a running softmax state).
//
// gfx950 mapping. The stationary buffer for host KV is an XCD's L2 (4 MB), shared by the
// 32 CUs of that XCD, rather than one CU's LDS: the host calls this kernel once per key
// super-chunk [kc0, kc1) sized to fit L2 (for each group of up to 8 (sequence, kv head)
// pairs), and workgroup i runs on XCD i % 8, so the query tiles of one pair are placed on
// one XCD and read the super-chunk from L2 after its first fetch over the link. Everything
// else a workgroup touches (queries, running state, output) is streamed with non-temporal
// loads and stores so that it does not push the super-chunk out of L2 between rounds of
// query tiles. Each workgroup keeps 256 query rows in registers (8 waves x 32), sweeps the
// super-chunk through double-buffered LDS tiles (loads issued two tiles ahead), and carries
// the per-row softmax state (o, m, l) in device memory from one super-chunk launch to the
// next (or, in the two-launch form, leaves one state per super-chunk for a finish launch to
// merge). Keys below past_len[b] come from the host cache; this step's new keys come from the
// device copy the projection left, so they never cross the link a second time. The launch
// (or launches) whose keys hold no host rows also writes this step's new rows to the host
// cache (the storer role), a share each.
//
// MFMA layout: scores are computed transposed, Sᵀ = K·Qᵀ (32 keys x 32 queries per block),
// so each lane owns one query column: row max / sum need one cross-half exchange, the
// accumulators are reused directly as the Pᵀ operand of Oᵀ += Vᵀ·Pᵀ, and Oᵀ rescaling is
// lane-local. V stays row-major in LDS and the Vᵀ operand is read with the gfx950 LDS
// transpose read (16-bit types); fp32 stores V transposed. The softmax reference maximum is
// raised lazily (only when a score exceeds it by more than 2^8), so the Oᵀ rescale is
// skipped by whole waves once the maximum has settled.
#include "dkv_internal.h"

namespace dkv {

// Build-time tunables (defaults are the tuned values).
#ifndef DKV_ATTN_KT
#define DKV_ATTN_KT 64
#endif
#ifndef DKV_ATTN_WAVES
#define DKV_ATTN_WAVES 8   // waves per workgroup, 32 query rows each
#endif
#ifndef DKV_ATTN_MINWAVES
#define DKV_ATTN_MINWAVES 2   // waves per SIMD the register allocation must allow (d = 128)
#endif
#ifndef DKV_ATTN_KPREF
#define DKV_ATTN_KPREF 4   // K fragments read from LDS ahead of the score products
#endif
#ifndef DKV_ATTN_KPAD
#define DKV_ATTN_KPAD 8    // elements of padding per K tile row (16-bit types)
#endif
#ifndef DKV_ATTN_VPAD
#define DKV_ATTN_VPAD 32   // elements of padding per row-major V tile row (16-bit types); 32 makes
                           // the transpose reads of the two 16-lane halves hit disjoint LDS banks
#endif

template <typename T, int DH>
struct AttnCfg {
  // keys per LDS tile; fp32 at d = 128 takes 32-key tiles, which keeps its scores, probabilities
  // and tile loads within the register budget of two waves per SIMD
  static constexpr int KT = sizeof(T) == 2 ? DKV_ATTN_KT : (DH == 128 ? 32 : 64);
  static constexpr int WAVES = DKV_ATTN_WAVES;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int ROWS = 32 * WAVES;        // query rows per workgroup
  static constexpr int EB = sizeof(T);
  static constexpr int VEC = 16 / EB;
  static constexpr int LDK = DH + (EB == 2 ? DKV_ATTN_KPAD : VEC);   // K tile row (elements), padded
  // 16-bit types keep V row-major ([key][d]) and read Vᵀ fragments with the gfx950 LDS
  // transpose read; fp32 stores Vᵀ ([d][key]) at load time instead.
  static constexpr bool VROW = EB == 2;
  static constexpr int LDV = VROW ? DH + DKV_ATTN_VPAD : KT + 16 / EB;
  static constexpr int KTILE = KT * LDK;
  static constexpr int VTILE = VROW ? KT * LDV : DH * LDV;
  static constexpr int CPR = DH / VEC;           // 16-byte chunks per key row
  static constexpr int LOADS = KT * CPR / THREADS;
  static constexpr int DB = DH / 32;             // 32-row blocks of Oᵀ
  static constexpr int SBLK = (DB * 16 + 2) * 64;  // floats of state per 32 query rows
  static_assert(LOADS >= 1 && KT * CPR % THREADS == 0, "tile load mapping");
  static_assert(2 * (KTILE + VTILE) * EB <= 160 * 1024, "LDS budget");
};

constexpr float kLazyRescale = 8.f;   // log2 units: raise the reference max past 2^8

// One unit of prefill attention work: the query tile qt of (sequence, kv head) pair p against
// the keys [kc0, kc1), carrying its running softmax state in `state`; `first` = no state to read
// yet, `last` = finalise the output after these keys, `merge` = at the finalisation, first merge
// the state the item kept for this step's own keys (AttnArgs::nstate).
struct AttnItem {
  int p, qt, kc0, kc1, first, last, merge;
  float* state;
  int split0 = 1;   // finalising with key splits: the first split state folded in (0: all of them)
};

// A 16-byte load of a key or value row piece; NT: non-temporal (the line is the first L2 evicts),
// for own-key items that share a launch with past-key items, whose super-chunk must stay in L2.
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
template <bool NT>
__device__ inline uint4 kv_load(const void* p) {
  if constexpr (NT) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

// Storer role: the new K and V rows of tokens [t0, t1) of pair p go from their device copy to the
// host cache rows [past_len[b] + t], 16 bytes per thread per step, with non-temporal stores.
template <typename T, int DH, bool PAGED>
__device__ inline void attn_store(const AttnArgs& a, const int p, const int t0, const int t1) {
  constexpr int VEC = 16 / (int)sizeof(T), CPR = DH / VEC;
  const int b = p / a.Hkv, g = p - b * a.Hkv;
  for (int c = t0 * CPR + (int)threadIdx.x; c < t1 * CPR; c += (int)blockDim.x) {
    const int t = c / CPR, col = (c - t * CPR) * VEC;
    const size_t src = ((size_t)p * a.T + t) * DH + col;
    const size_t dst = host_row(PAGED ? a.table : nullptr, a.max_pages, b, g, a.Hkv, a.cap, a.past_len[b] + t) * DH + col;
    const u32x4 kv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.k_new) + src);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.v_new) + src);
    __builtin_nontemporal_store(kv, reinterpret_cast<u32x4*>(reinterpret_cast<T*>(const_cast<void*>(a.kc)) + dst));
    __builtin_nontemporal_store(vv, reinterpret_cast<u32x4*>(reinterpret_cast<T*>(const_cast<void*>(a.vc)) + dst));
  }
}

// PAGED: the host cache is a page pool addressed through the block table; the page ids of
// the item's host keys are staged in LDS before the sweep. NTKV: key/value loads are
// non-temporal (own-key items beside past-key items in one launch).
// The workgroup's LDS: double-buffered key and value tiles and (paged caches) the page ids of a
// launch's keys. Declared once in the kernel, so that every kind of item in it (each an
// instantiation of attn_item) shares one allocation.
template <typename T, int DH, bool PAGED>
struct AttnLds {
  T k[2][AttnCfg<T, DH>::KTILE];
  T v[2][AttnCfg<T, DH>::VTILE];
  int32_t pages[PAGED ? kPagedSuperchunk / kPageTokens + 1 : 1];
};

template <typename T, int DH, int G, bool PAGED, bool NTKV = false>
__device__ __attribute__((always_inline)) inline void attn_item(const AttnArgs& a, const AttnItem it,
                                                                 AttnLds<T, DH, PAGED>& lds) {
  using C = AttnCfg<T, DH>;
  using MF = Mfma<T>;
  constexpr int KT = C::KT, VEC = C::VEC, LDK = C::LDK, LDV = C::LDV, LOADS = C::LOADS, DB = C::DB;
  constexpr int CPR = C::CPR, KPL = MF::KPL, KSTEP = MF::KSTEP;
  auto& sK = lds.k;
  auto& sV = lds.v;
  auto& s_pages = lds.pages;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int half = lane >> 5, col = lane & 31;
  const int p = it.p, qt = it.qt;
  const int b = p / a.Hkv, g = p - b * a.Hkv;
  const int L = a.past_len[b];
  const int nrows = a.T * G;                     // query rows of this pair: row = t*G + hh
  const int row0 = qt * C::ROWS;
  if (row0 >= nrows) return;
  const int rlast = min(row0 + C::ROWS, nrows) - 1;
  const int key_hi = min(it.kc1, L + rlast / G + 1);  // keys any row here may see, exclusive
  const int key_lo = it.kc0;
  const bool work = key_lo < key_hi;
  // nothing visible and nothing to finalise (a key split still leaves its empty state)
  if (!work && !it.last && !a.n_splits) return;
  const int key_all = L + row0 / G + 1;          // keys below this are visible to every row

  const int r = row0 + wave * 32 + col;          // this lane's query row
  const bool rvalid = r < nrows;
  const int t = rvalid ? r / G : 0;
  const int hh = r - (r / G) * G;
  const int qpos = L + t;
  const int nblk = (nrows + 31) >> 5;
  const bool wvalid = (row0 >> 5) + wave < nblk;   // this wave's 32-row block exists
  const size_t st_off = ((size_t)p * nblk + (wvalid ? (row0 >> 5) + wave : 0)) * C::SBLK;
  float* st = it.state + st_off;

  f32x16 o[DB];
  float m_run = -INFINITY, l_run = 0.f;          // log2 domain, scaled scores
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  if (!it.first && wvalid) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[db][v] = __builtin_nontemporal_load(st + (db * 16 + v) * 64 + lane);
    m_run = __builtin_nontemporal_load(st + DB * 16 * 64 + lane);
    l_run = __builtin_nontemporal_load(st + (DB * 16 + 1) * 64 + lane);
  }

  if (work) {
    typename MF::frag qf[DH / KSTEP];
    {
      const T* qrow = reinterpret_cast<const T*>(a.q) + (((size_t)b * a.T + t) * a.Hq + g * G + hh) * DH;
#pragma unroll
      for (int ks = 0; ks < DH / KSTEP; ++ks) {
        if (rvalid) qf[ks] = __builtin_nontemporal_load(reinterpret_cast<const typename MF::frag*>(qrow + ks * KSTEP + half * KPL));
        else qf[ks] = typename MF::frag{};
      }
    }
    const float sl2 = 1.4426950408889634f * rsqrtf((float)DH);   // log2(e)/sqrt(d)

    const size_t bg = (size_t)p;
    const T* __restrict__ kh = reinterpret_cast<const T*>(a.kc) + (PAGED ? 0 : bg * a.cap * DH);
    const T* __restrict__ vh = reinterpret_cast<const T*>(a.vc) + (PAGED ? 0 : bg * a.cap * DH);
    const T* __restrict__ kn = reinterpret_cast<const T*>(a.k_new) + bg * a.T * DH;
    const T* __restrict__ vn = reinterpret_cast<const T*>(a.v_new) + bg * a.T * DH;

    const int host_end = a.new_from_host ? key_hi : L;   // keys below this come from the host
    const int pg0 = key_lo / kPageTokens;                // first page of the launch's keys
    if constexpr (PAGED) {
      const int hend = min(key_hi, host_end);
      const int npg = hend > key_lo ? (hend - 1) / kPageTokens - pg0 + 1 : 0;
      for (int i = tid; i < npg; i += C::THREADS) s_pages[i] = a.table[(size_t)b * a.max_pages + pg0 + i];
      __syncthreads();
    }
    // element offset of host key j (row start) within the K or V pool
    auto hrow = [&](int j) __attribute__((always_inline)) -> size_t {
      if constexpr (PAGED)
        return (((size_t)s_pages[j / kPageTokens - pg0] * a.Hkv + g) * kPageTokens + j % kPageTokens) * DH;
      else
        return (size_t)j * DH;
    };
    // this thread's 16-byte chunks of a tile: chunk i is key row krow[i], element offset off[i]
    int krow[LOADS], off[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + i * C::THREADS;
      krow[i] = c / CPR;
      off[i] = krow[i] * DH + (c % CPR) * VEC;
    }
    // Global -> register loads (gk, gv) and register -> LDS stores (sk, sv) of one key tile.
    // Loads are unconditional (a row past the launch's keys reads the last key row instead,
    // always in bounds) and the zero fill for such rows happens at the LDS store, which waits
    // for the data anyway: a masked load into pre-zeroed registers would make the wave wait
    // for its loads right after issuing them.
    uint4 rk[2][LOADS], rv[2][LOADS];
    auto gk = [&](int set, int j0) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int j = min(j0 + krow[i], key_hi - 1);
        const int e = off[i] - krow[i] * DH;
        const T* ks = j < host_end ? kh + hrow(j) : kn + (size_t)(j - L) * DH;
        rk[set][i] = kv_load<NTKV>(ks + e);
      }
    };
    auto gv = [&](int set, int j0) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int j = min(j0 + krow[i], key_hi - 1);
        const int e = off[i] - krow[i] * DH;
        const T* vs = j < host_end ? vh + hrow(j) : vn + (size_t)(j - L) * DH;
        rv[set][i] = kv_load<NTKV>(vs + e);
      }
    };
    auto sk = [&](int buf, int set, int j0) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int kr = krow[i], kc = off[i] - kr * DH;
        *reinterpret_cast<uint4*>(&sK[buf][kr * LDK + kc]) = j0 + kr < key_hi ? rk[set][i] : make_uint4(0, 0, 0, 0);
      }
    };
    auto sv = [&](int buf, int set, int j0) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int kr = krow[i], kc = off[i] - kr * DH;
        const uint4 vz = j0 + kr < key_hi ? rv[set][i] : make_uint4(0, 0, 0, 0);
        if constexpr (C::VROW) {
          *reinterpret_cast<uint4*>(&sV[buf][kr * LDV + kc]) = vz;
        } else {
          const T* ve = reinterpret_cast<const T*>(&vz);
#pragma unroll
          for (int e = 0; e < VEC; ++e) sV[buf][(kc + e) * LDV + kr] = ve[e];
        }
      }
    };
    auto gload = [&](int set, int j0) __attribute__((always_inline)) { gk(set, j0); gv(set, j0); };
    auto sstore = [&](int buf, int set, int j0) __attribute__((always_inline)) { sk(buf, set, j0); sv(buf, set, j0); };

    // ---- the three parts of a key tile (KT keys) against this wave's 32 query rows
    typedef f32x16 Scores[KT / 32];                      // Sᵀ: KT/32 blocks of 32 keys x 32 queries
    typedef typename MF::frag Probs[KT / 32][32 / KSTEP];  // Pᵀ in MFMA operand form
    // The K fragments are read from LDS PD products ahead of their use, and the KT/32 key blocks'
    // product chains are interleaved (fragment f is key block f % NKB, reduction step f / NKB):
    // left to itself the compiler reads each fragment into the same registers right before its
    // product and waits for it, so every product paid the full LDS latency. Each chain still sums
    // its steps in ascending order, so the scores are unchanged bit for bit.
    auto qk = [&](const T* tK, Scores& sc) __attribute__((always_inline)) {
      constexpr int NKB = KT / 32, NF = NKB * (DH / KSTEP), PD = DKV_ATTN_KPREF < NF ? DKV_ATTN_KPREF : NF;
      auto kfrag = [&](const int f) __attribute__((always_inline)) {
        return *reinterpret_cast<const typename MF::frag*>(tK + ((f % NKB) * 32 + col) * LDK + (f / NKB) * KSTEP +
                                                           half * KPL);
      };
      typename MF::frag kf[PD];
#pragma unroll
      for (int f = 0; f < PD; ++f) kf[f] = kfrag(f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int kb = f % NKB, ks = f / NKB;
        sc[kb] = MF::mma(kf[f % PD], qf[ks], ks == 0 ? f32x16{} : sc[kb]);
        if (f + PD < NF) kf[f % PD] = kfrag(f + PD);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // mask, tile maximum and the lazy raise of the reference maximum (rescaling o and l);
    // MASK = false for tiles every row of the workgroup sees whole (the lean path)
    auto rebase = [&](const int j0, Scores& sc, auto mask_tag) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      // mask only where some row of this workgroup cannot see some key of the tile
      if (MASK && ((j0 + KT > key_hi) || (j0 + KT > key_all))) {
#pragma unroll
        for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int j = j0 + kb * 32 + acc_row(v, lane);
            if (j >= key_hi || j > qpos) sc[kb][v] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kb][v]);
      mx = half_max(mx) * sl2;
      // lazy reference maximum: raise it only when a score exceeds it by more than 2^8
      const bool raise = mx > m_run + kLazyRescale;
      if (__any(raise)) {
        const float m_new = raise ? mx : m_run;
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;   // 0 when m_run = -inf
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
      }
    };
    // Pᵀ = exp2(Sᵀ·scale - m) in operand form, and this lane's share of the row sums into l
    // (the two lanes of a row, l and l + 32, each sum their own keys; the halves are added when
    // the output is finalised). 16-bit types sum the rounded weights the PVᵀ product uses, two
    // per dot2 instruction, so numerator and denominator see the same weights.
    auto probs = [&](const Scores& sc, Probs& pb) __attribute__((always_inline)) {
      const float mref = (m_run == -INFINITY) ? 0.f : m_run;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
        for (int stp = 0; stp < 32 / KSTEP; ++stp) {
          if constexpr (KPL == 1) {
            const float w = __builtin_amdgcn_exp2f(fmaf(sc[kb][stp], sl2, -mref));
            ps += w;
            pb[kb][stp] = w;
          } else {
#pragma unroll
            for (int e = 0; e < KPL; ++e)
              pb[kb][stp][e] = Elem<T>::from_float(__builtin_amdgcn_exp2f(fmaf(sc[kb][stp * KPL + e], sl2, -mref)));
#pragma unroll
            for (int e = 0; e < KPL; e += 2) ps = Elem<T>::dot2_ones(pb[kb][stp][e], pb[kb][stp][e + 1], ps);
          }
        }
      l_run += ps;
    };
    // Oᵀ += Vᵀ · Pᵀ; reduction slot (half, e) of step stp is the key held in accumulator
    // register stp*KPL + e of that half, i.e. element e of pb[kb][stp]
    auto pv = [&](const T* tV, const Probs& pb) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb) {
#pragma unroll
        for (int stp = 0; stp < 32 / KSTEP; ++stp) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            typename MF::frag va;
            if constexpr (C::VROW) {
              // lane needs V[keys 16*stp + 4*half + {0..3}, +8 + ...][d = db*32 + col]. The
              // transpose read gives result lane i (of 16) value k from source lane 4k + i/4,
              // element i % 4; so source lane 4k + q of each 16-lane group points at
              // V[kbase + k][d0 + 4q], with d0 the group's first column.
              const int li = lane & 15, kk = li >> 2, qq = li & 3;
              const int d0 = db * 32 + (lane & 16);
              const int kbase = kb * 32 + 16 * stp + 4 * half;
              const T* src0 = tV + (kbase + kk) * LDV + d0 + 4 * qq;
              const T* src1 = src0 + 8 * LDV;
              typedef short v4s __attribute__((ext_vector_type(4)));
              const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(src0));
              const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(src1));
              __builtin_memcpy(&va, &lo, 8);
              __builtin_memcpy(reinterpret_cast<char*>(&va) + 8, &hi, 8);
            } else {
              const T* vrow = tV + (db * 32 + col) * LDV + kb * 32;
              va = vrow[acc_row(stp, lane)];
            }
            o[db] = MF::mma(va, pb[kb][stp], o[db]);
          }
        }
      }
    };

    const int n = (key_hi - key_lo + KT - 1) / KT;     // key tiles in this launch
    auto tj = [&](const int i) __attribute__((always_inline)) { return key_lo + i * KT; };   // tile i's first key
    Probs pb;
    // tile i computes from LDS buffer i % 2; register set 0 carries tiles 1, 3, 5, ... and set 1
    // tiles 2, 4, 6, ... (loaded two tiles ahead, stored to LDS one tile ahead)
    Scores sc;
    // A wave skips the products of a tile none of its rows can see: a 32-row block past the
    // pair's rows (the last query tile of a pair is often part-filled) or keys all later than its
    // last row. Such a tile would add exact zeros, so skipping it changes no bit.
    const int wave_keys = wvalid ? L + (min(row0 + wave * 32 + 31, nrows - 1)) / G + 1 : 0;   // exclusive
    auto tile = [&](const int j0, const int buf) __attribute__((always_inline)) {
      if (j0 >= wave_keys) return;
      qk(sK[buf], sc);
      rebase(j0, sc, std::true_type{});
      probs(sc, pb);
      pv(sV[buf], pb);
    };
    // Loads are issued unconditionally, also for tiles past the end (their rows are clamped
    // to the last key, which is already on chip): with a fixed issue order the wait before
    // each LDS store counts only the loads of its own register set, not the newer ones.
    gload(0, tj(0));
    sstore(0, 0, tj(0));
    gload(0, tj(1));
    gload(1, tj(2));
    __syncthreads();
    // Tile i: first tile i + 1 goes from its register set into the other LDS buffer (free since
    // the last barrier) and tile i + 3's loads are issued into that set, then tile i is computed.
    // Issuing the loads before the MFMA work lets a wave stalled on a full load queue give the
    // SIMD to its partner wave instead of stalling with it at the end of the tile (1-1.5%).
    // Whole pairs of tiles, then the odd tile: no exit mid-body, which keeps the load waits
    // exact (each LDS store waits for its own register set only).
    auto half = [&](const int i, const int buf, const int set) __attribute__((always_inline)) {
      if (i + 1 < n) sstore(1 - buf, set, tj(i + 1));
      gload(set, tj(i + 3));
      tile(tj(i), buf);
      __syncthreads();
    };
    int i = 0;
    // Lean steady state: leading tiles that lie whole inside the launch's keys, are seen whole by
    // every row of the workgroup (no causal mask), come from one source (the contiguous host cache
    // or this step's device rows) and whose loads three tiles ahead stay in range too. Their loads
    // need no clamp, their LDS stores no zero fill and their scores no mask, and the row address
    // is one uniform tile base plus a fixed per-thread offset.
    const int n_in = (key_hi - key_lo) / KT;                        // tiles whole inside the range
    const int n_vis = (max(min(key_hi, key_all), key_lo) - key_lo) / KT;   // and unmasked
    const bool one_src = !PAGED && (key_hi <= host_end || key_lo >= host_end);
    const int n_lean = one_src ? (max(0, min(n_vis, n_in - 3)) & ~1) : 0;
    if (n_lean > 0) {
      const T* __restrict__ ksrc = key_lo >= host_end ? kn - (size_t)L * DH : kh;   // row j at ksrc + j * DH
      const T* __restrict__ vsrc = key_lo >= host_end ? vn - (size_t)L * DH : vh;
      auto gload_lean = [&](int set, int j0) __attribute__((always_inline)) {
        const T* kt = ksrc + (size_t)j0 * DH;
        const T* vt = vsrc + (size_t)j0 * DH;
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
          rk[set][u] = kv_load<NTKV>(kt + off[u]);
          rv[set][u] = kv_load<NTKV>(vt + off[u]);
        }
      };
      auto sstore_lean = [&](int buf, int set) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
          const int kr = krow[u], kc = off[u] - kr * DH;
          *reinterpret_cast<uint4*>(&sK[buf][kr * LDK + kc]) = rk[set][u];
          if constexpr (C::VROW) {
            *reinterpret_cast<uint4*>(&sV[buf][kr * LDV + kc]) = rv[set][u];
          } else {
            const T* ve = reinterpret_cast<const T*>(&rv[set][u]);
#pragma unroll
            for (int e = 0; e < VEC; ++e) sV[buf][(kc + e) * LDV + kr] = ve[e];
          }
        }
      };
      auto half_lean = [&](const int i, const int buf, const int set) __attribute__((always_inline)) {
        sstore_lean(1 - buf, set);
        gload_lean(set, tj(i + 3));
        if (wvalid) {
          qk(sK[buf], sc);
          rebase(tj(i), sc, std::false_type{});
          probs(sc, pb);
          pv(sV[buf], pb);
        }
        __syncthreads();
      };
      for (; i < n_lean; i += 2) {
        half_lean(i, 0, 0);
        half_lean(i + 1, 1, 1);
      }
    }
    for (; i + 1 < n; i += 2) {
      half(i, 0, 0);
      half(i + 1, 1, 1);
    }
    if (i < n) half(i, 0, 0);
  }

  if (it.last) {
    if (a.n_splits && wvalid) {
      // key-split mode: fold in the states of splits split0 .. n_splits - 1 (an item with split0 = 1
      // read split 0's as its running state). A split whose keys this row cannot see left m = -inf
      // and is skipped; if the running state is still empty (split 0 without keys, or no keys
      // computed yet), the first split with keys is taken as it is.
      for (int j = it.split0; j < a.n_splits; ++j) {
        const float* ns = it.state + (size_t)j * a.split_stride + st_off;
        const float m2 = __builtin_nontemporal_load(ns + DB * 16 * 64 + lane);
        if (m2 == -INFINITY) continue;
        const float l2 = __builtin_nontemporal_load(ns + (DB * 16 + 1) * 64 + lane);
        const bool have = m_run != -INFINITY;
        const float M = have ? fmaxf(m_run, m2) : m2;
        const float a1 = have ? __builtin_amdgcn_exp2f(m_run - M) : 0.f;
        const float a2 = __builtin_amdgcn_exp2f(m2 - M);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float o2 = __builtin_nontemporal_load(ns + (db * 16 + v) * 64 + lane);
            o[db][v] = have ? fmaf(o[db][v], a1, o2 * a2) : o2;
          }
        l_run = have ? fmaf(l_run, a1, l2 * a2) : l2;
        m_run = M;
      }
    }
    if (it.merge && wvalid) {
      // fold in the state of this step's own keys: O = (o 2^(m - M) + o' 2^(m' - M)) / (l 2^(m - M) +
      // l' 2^(m' - M)), M = max(m, m'); a sequence with no past keys has only the latter
      const float* ns = a.nstate + st_off;
      const float m2 = __builtin_nontemporal_load(ns + DB * 16 * 64 + lane);
      const float l2 = __builtin_nontemporal_load(ns + (DB * 16 + 1) * 64 + lane);
      const bool have_past = L > 0;
      const float M = have_past ? fmaxf(m_run, m2) : m2;
      const float a1 = have_past ? __builtin_amdgcn_exp2f(m_run - M) : 0.f;
      const float a2 = __builtin_amdgcn_exp2f(m2 - M);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float o2 = __builtin_nontemporal_load(ns + (db * 16 + v) * 64 + lane);
          o[db][v] = have_past ? fmaf(o[db][v], a1, o2 * a2) : o2;
        }
      l_run = have_past ? fmaf(l_run, a1, l2 * a2) : l2;
    }
    const float l_row = half_sum(l_run);   // the two lanes of the row, each its own keys
    if (!rvalid) return;
    const float inv = 1.f / l_row;
    T* orow = reinterpret_cast<T*>(a.out) + (((size_t)b * a.T + t) * a.Hq + g * G + hh) * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        __builtin_nontemporal_store(Elem<T>::from_float(o[db][v] * inv), orow + db * 32 + acc_row(v, lane));
  } else if (wvalid) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) __builtin_nontemporal_store(o[db][v], st + (db * 16 + v) * 64 + lane);
    __builtin_nontemporal_store(m_run, st + DB * 16 * 64 + lane);
    __builtin_nontemporal_store(l_run, st + (DB * 16 + 1) * 64 + lane);
  }
}

// One launch per key super-chunk [a.kc0, a.kc1) of the pairs [a.pair0, a.pair0 + a.pairs), carrying
// a share of this step's own-key work: per pair, the items are taken in this order
//   - a.fetchers past-key items (the heaviest query tiles), which bring the super-chunk over the
//     host link into L2 while
//   - the own-key items of query tiles [a.dev_q0, a.dev_q1) (this step's keys, read from their
//     device copies: no host bytes, no L2 budget) keep the other CUs computing, then
//   - the remaining past-key items, which find the super-chunk in L2.
// No item waits for another: own-key items keep their own running state (a.nstate), which the
// past-key items of the last launch fold in when they finalise (a.merge_new). With
// a.past_items = 0 the launch holds own-key items only (a.dev_final: they finalise the output).
// With at least 8 pairs, pair p is served only by XCD p % 8 (workgroup i runs on XCD i % 8).
// The second bound is the minimum number of waves per SIMD: two, 256 VGPRs a lane. (Four waves
// per SIMD would leave 128, under what the three kinds of item need at d = 64.)
//
// Key-split mode (a.n_splits > 0; the pairs have one query tile each, so no key is shared between
// query tiles and nothing is gained by keeping a super-chunk in L2): workgroup i takes pair
// i % pairs and key split i / pairs, an equal share of the pair's key tiles (past and own keys),
// and leaves its running state in that split's state array; a.split_storers more workgroups
// write this step's new rows to the host cache meanwhile (the storer role). A second launch
// (a.split_combine) folds the splits' states together per pair and writes the output.
// This workgroup's pair and its position in that pair's sequence of items: with XCD placement
// pair p is served by XCD p % 8 (workgroup i runs on XCD i % 8); false for a padding workgroup.
__device__ inline bool attn_pair_slot(const AttnArgs& a, int& p, int& r) {
  const int P = a.pairs;
  if (a.xcd_group) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int ppx = (P + 7) >> 3;
    const int lp = (slot % ppx) * 8 + xcd;
    if (lp >= P) return false;
    p = a.pair0 + lp;
    r = slot / ppx;
  } else {
    p = a.pair0 + blockIdx.x % P;
    r = blockIdx.x / P;
  }
  return true;
}

template <typename T, int DH, int G, bool PAGED>
__global__ __launch_bounds__(64 * DKV_ATTN_WAVES, DKV_ATTN_MINWAVES)
void attn_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) AttnLds<T, DH, PAGED> lds;
  // Each mode below only picks this workgroup's item; one call at the end runs it, so the item's
  // code is compiled twice (with and without non-temporal K/V loads), not once per kind of item.
  AttnItem it;
  bool nt = false;      // non-temporal K/V loads: own-key items sharing a launch with past-key items
  int s0 = 0, s1 = 0;   // the storer role: tokens [s0, s1) of pair it.p whose new rows go to the host
  constexpr int TPT = AttnCfg<T, DH>::ROWS / G;   // tokens per query tile
  if (a.chunked) {
    // Two-launch prefill over past super-chunks. Per pair the chunk launch runs, in dispatch
    // order: F fetcher items of chunk 0, the own-key items of query tiles [0, n_own0), then per
    // chunk j its other items with chunk j+1's F fetchers inserted after the first chunk_insert of
    // them, so chunk j+1 crosses the link while chunk j's items compute from L2. Every past item
    // starts fresh and leaves its state in chunk j's array; no item waits for another. The finish
    // launch runs the own-key items of [n_own0, Q), which fold in every chunk's state as they
    // finalise, and for [0, n_own0) items that only merge the chunk states and the own-key state.
    int p, r;
    if (!attn_pair_slot(a, p, r)) return;
    const int Q = a.q_tiles, S = a.n_splits, F = min(a.fetchers, Q), Qa = a.n_own0;
    const int L = a.past_len[p / a.Hkv];
    if (a.chunked == 2) {
      const int qt = Q - 1 - r;
      if (r < Q - Qa) {
        it = AttnItem{p, qt, L, L + a.T, 1, 1, 0, a.state};
        it.split0 = 0;
        if (a.store_new) s0 = qt * TPT, s1 = min((qt + 1) * TPT, a.T);
      } else {
        it = AttnItem{p, qt, 0, 0, 0, 1, 1, a.state};
      }
    } else if (r >= F && r < F + Qa) {
      const int qt = Qa - 1 - (r - F);
      it = AttnItem{p, qt, L, L + a.T, 1, 0, 0, a.nstate};
      nt = true;
      if (a.store_new) s0 = qt * TPT, s1 = min((qt + 1) * TPT, a.T);
    } else {
      int j, idx;
      if (r < F) {
        j = 0;
        idx = r;
      } else {
        const int ins = min(a.chunk_insert, Q - F);
        const int o0 = r - F - Qa;
        j = min(o0 / Q, S - 1);                    // block j: Q - F of chunk j's items + F of chunk j+1's
        const int o = o0 - j * Q;
        const int fj = j + 1 < S ? F : 0;
        if (o < ins) {
          idx = F + o;
        } else if (o < ins + fj) {
          idx = o - ins;
          j += 1;
        } else {
          idx = F + o - fj;
        }
      }
      const int kc0 = min(j * a.chunk_keys, L), kc1 = min(kc0 + a.chunk_keys, L);
      it = AttnItem{p, Q - 1 - idx, kc0, kc1, 1, 0, 0, a.state + (size_t)j * a.split_stride};
    }
  } else if (a.n_splits) {
    if (!a.split_combine && (int)blockIdx.x >= a.pairs * a.n_splits) {
      // storer workgroup s: an equal share of the (pair, token) rows of this step, K and V, from
      // the device copies to the host cache, while the split items compute
      const int s = (int)blockIdx.x - a.pairs * a.n_splits;
      const int rows = a.pairs * a.T;
      const int r0 = (int)((long long)rows * s / a.split_storers);
      const int r1 = (int)((long long)rows * (s + 1) / a.split_storers);
      for (int row = r0; row < r1;) {   // runs of one pair's consecutive tokens
        const int pp = row / a.T, t0 = row - pp * a.T;
        const int t1 = min(a.T, t0 + (r1 - row));
        attn_store<T, DH, PAGED>(a, a.pair0 + pp, t0, t1);
        row += t1 - t0;
      }
      return;
    }
    const int p = a.pair0 + (int)blockIdx.x % a.pairs;
    if (a.split_combine) {
      it = AttnItem{p, 0, 0, 0, 0, 1, 0, a.state};
    } else {
      constexpr int KT = AttnCfg<T, DH>::KT;
      const int j = (int)blockIdx.x / a.pairs;
      const int nk = a.past_len[p / a.Hkv] + a.T;                 // the pair's keys, past and own
      const int tiles = (nk + KT - 1) / KT;
      const int t0 = (int)((long long)tiles * j / a.n_splits), t1 = (int)((long long)tiles * (j + 1) / a.n_splits);
      it = AttnItem{p, 0, t0 * KT, min(t1 * KT, nk), 1, 0, 0, a.state + (size_t)j * a.split_stride};
    }
  } else {
    int p, r;   // pair, and the item's position in that pair's sequence of items
    if (!attn_pair_slot(a, p, r)) return;
    const int Q = a.q_tiles;
    const int F = a.past_items ? min(a.fetchers, Q) : 0;
    const int ND = a.dev_q1 - a.dev_q0;
    const int L = a.past_len[p / a.Hkv];
    // query tiles go out last row first: under the causal mask later rows see more keys
    if (r >= F && r < F + ND) {
      const int qt = a.dev_q1 - 1 - (r - F);
      // the storer role: this item's query tile's tokens' new K/V rows go to the host cache (each
      // query tile has exactly one own-key item, so every new row is written once)
      if (a.store_new) s0 = qt * TPT, s1 = min((qt + 1) * TPT, a.T);
      it = AttnItem{p, qt, L, L + a.T, 1, a.dev_final, 0, a.nstate};
      nt = a.past_items != 0;
    } else {
      const int qt = Q - 1 - (r < F ? r : r - ND);
      const int kc1 = a.clip_past ? min(a.kc1, L) : a.kc1;
      it = AttnItem{p, qt, a.kc0, kc1, a.first, a.last, a.merge_new, a.state};
    }
  }
  if (s1 > s0) attn_store<T, DH, PAGED>(a, it.p, s0, s1);
  if (nt) attn_item<T, DH, G, PAGED, true>(a, it, lds);
  else attn_item<T, DH, G, PAGED, false>(a, it, lds);
}

template <typename T, int DH, int G, bool PAGED>
static hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const int P = a.pairs;
  const int items = a.chunked == 1 ? a.n_splits * a.q_tiles + a.n_own0
                    : a.chunked == 2 ? a.q_tiles
                    : a.n_splits   ? (a.split_combine ? 1 : a.n_splits)
                                   : (a.past_items ? a.q_tiles : 0) + a.dev_q1 - a.dev_q0;   // per pair
  const bool placed = a.xcd_group && (a.chunked || !a.n_splits);
  const int grid = placed ? 8 * ((P + 7) / 8) * items
                          : P * items + (a.n_splits && !a.chunked && !a.split_combine ? a.split_storers : 0);
  hipLaunchKernelGGL((attn_kernel<T, DH, G, PAGED>), dim3(grid), dim3(AttnCfg<T, DH>::THREADS), 0, s, a);
  return hipGetLastError();
}

template <typename T, int DH, bool PAGED>
static attn_fn pick_g(int G) {
  switch (G) {
    case 1: return launch_attn<T, DH, 1, PAGED>;
    case 2: return launch_attn<T, DH, 2, PAGED>;
    case 4: return launch_attn<T, DH, 4, PAGED>;
    case 8: return launch_attn<T, DH, 8, PAGED>;
    default: return nullptr;
  }
}

template <typename T>
static attn_fn pick_d(int d, int G, bool paged) {
  if (d == 64) return paged ? pick_g<T, 64, true>(G) : pick_g<T, 64, false>(G);
  if (d == 128) return paged ? pick_g<T, 128, true>(G) : pick_g<T, 128, false>(G);
  return nullptr;
}

attn_fn find_attn(int dtype, int d, int G, bool paged) {
  switch (dtype) {
    case 0: return pick_d<float>(d, G, paged);
    case 1: return pick_d<_Float16>(d, G, paged);
    case 2: return pick_d<__bf16>(d, G, paged);
    default: return nullptr;
  }
}

int attn_rows_per_tile() { return 32 * DKV_ATTN_WAVES; }

int attn_key_tile(int dtype, int d) {
  if (dtype == 0) return d == 128 ? AttnCfg<float, 128>::KT : AttnCfg<float, 64>::KT;
  return d == 128 ? AttnCfg<__bf16, 128>::KT : AttnCfg<__bf16, 64>::KT;
}

size_t attn_state_bytes(int d, int batch, int n_kv_heads, int T, int G) {
  const size_t nblk = ((size_t)T * G + 31) / 32;
  return (size_t)batch * n_kv_heads * nblk * (size_t)((d / 32) * 16 + 2) * 64 * sizeof(float);
}

}  // namespace dkv
