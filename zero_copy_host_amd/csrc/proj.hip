// Projection GEMM Y = X·Wᵀ for the new tokens of a layer step, over up to three weight
// segments (Q, K, V) that share the activation matrix X.
//
// Follows "Paper Notes: DirectKV", Fundamental Underlying Technologies / Kernel Fusion
// (K = X·Wk, V = X·Wv) and System Architecture / KV Cache Manager: the K and V rows go
// straight into the pinned host cache at rows [past_len[b], past_len[b] + T) (the storer
// role); Q goes to device memory, where the pages keep the queries. The new K/V rows can
// also (or only) be left in device memory, so that attention over them never reads them
// back across the host link; in a fused prefill the host copy is then written by the first
// attention launch, whose link traffic is otherwise all in the read direction.
//
// gfx950 mapping: for 16-bit types 4x2 waves (512 threads) per workgroup, one workgroup per CU;
// each wave owns 64 rows x 128 columns of Y (2x4 blocks of the 32x32x16 MFMA), a 256x256
// workgroup tile, with reduction steps of 32 through a double-buffered LDS tile (X and W both
// stored k-contiguous, padded by 16 bytes per row against bank conflicts). Per 16-deep
// reduction slice a wave reads 2 + 4 operand fragments for 8 MFMAs (0.75 KB of LDS per MFMA;
// a 64x64 wave tile needs 1 KB, which is the whole LDS bandwidth at the MFMA rate), and the CU
// pulls 32 KB of operands from L2 per step against 48 KB for two 128x256 workgroups. fp32
// keeps 2x2 waves of 64x64 tiles with steps of 64. The reduction depth needs D % 64 == 0, which the ABI
// checks. The epilogue is staged through LDS so every output row leaves as full 16-byte-per-
// lane contiguous writes (whole host cache lines for K and V).
#include <algorithm>

#include "dkv_internal.h"

namespace dkv {

#ifndef DKV_PROJ_BK
#define DKV_PROJ_BK 64   // reduction depth per LDS stage, 16-bit types (build-time tunable)
#endif
#ifndef DKV_PROJ_NB
#define DKV_PROJ_NB 4    // 32-column MFMA blocks per wave, 16-bit types (build-time tunable)
#endif
#ifndef DKV_PROJ_MB
#define DKV_PROJ_MB 2    // 32-row MFMA blocks per wave, 16-bit types (build-time tunable)
#endif
#ifndef DKV_PROJ_SETS
#define DKV_PROJ_SETS 1  // operand register sets, 16-bit types (2: loads two steps ahead instead of one)
#endif
#ifndef DKV_PROJ_WM
#define DKV_PROJ_WM 4    // waves along M per workgroup, 16-bit types (build-time tunable; 2 columns of waves)
#endif

template <typename T>
struct ProjCfg {
  static constexpr int EB = sizeof(T);
  static constexpr int MB = EB == 2 ? DKV_PROJ_MB : 2;       // 32-row MFMA blocks per wave
  static constexpr int NB = EB == 2 ? DKV_PROJ_NB : 2;       // 32-column MFMA blocks per wave
  static constexpr int BK = EB == 2 ? DKV_PROJ_BK : 64;
  static constexpr int WM = EB == 2 ? DKV_PROJ_WM : 2, WN = 2;   // waves along M and N
  static constexpr int THREADS = 64 * WM * WN;
  static constexpr int BM = WM * 32 * MB, BN = WN * 32 * NB;
  static constexpr int VEC = 16 / EB;            // elements per 16-byte chunk
  static constexpr int LDK = BK + VEC;           // padded row length in LDS (elements)
  static constexpr int CPR = BK / VEC;           // 16-byte chunks per tile row
  static constexpr int LOADS_X = BM * CPR / THREADS; // chunks per thread per X tile
  static constexpr int LOADS_W = BN * CPR / THREADS; // chunks per thread per W tile
  static constexpr int LDO = BN + VEC;           // padded output staging row
  static constexpr int TILE_X = BM * LDK, TILE_W = BN * LDK;   // elements of one buffer
  static constexpr int IN_BYTES = 2 * (TILE_X + TILE_W) * EB;  // X and W, double buffered
  static constexpr int OUT_BYTES = BM * LDO * EB;
  static constexpr int SMEM = IN_BYTES > OUT_BYTES ? IN_BYTES : OUT_BYTES;
  static_assert(BM * CPR % THREADS == 0 && BN * CPR % THREADS == 0 && 64 % BK == 0, "tile load mapping");
  // waves per SIMD the register allocation must allow (256 registers a lane at two)
  static constexpr int MIN_WAVES = (EB == 2 && DKV_PROJ_MB * DKV_PROJ_NB <= 8) ? 2 : 1;
};

// Write 16 bytes of output row m, columns [n, n + 16 bytes) of segment seg: Q to device memory,
// K and V to their host cache rows [past_len[b] + t] and/or the device copies of the new rows.
template <typename T>
__device__ inline void proj_store(const ProjArgs& a, const int seg, const int nseg, const int m, const int n,
                                  const uint4 val) {
  if (seg == 0) {
    *reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.q_out) + (size_t)m * nseg + n) = val;
    return;
  }
  const int b = m / a.T, t = m - b * a.T;
  const int gg = n / a.d, i = n - gg * a.d;
  const size_t bgk = (size_t)b * a.Hkv + gg;
  if (a.host_out) {
    T* cache = reinterpret_cast<T*>(seg == 1 ? a.kc : a.vc);
    const size_t row = host_row(a.table, a.max_pages, b, gg, a.Hkv, a.cap, a.past_len[b] + t);
    *reinterpret_cast<uint4*>(cache + row * a.d + i) = val;
  }
  void* dev = seg == 1 ? a.k_dev : a.v_dev;
  if (dev) *reinterpret_cast<uint4*>(reinterpret_cast<T*>(dev) + (bgk * a.T + t) * a.d + i) = val;
}

// The tile's epilogue: round to T into an LDS tile, then write whole rows (16 bytes a lane); with the
// rotary embedding, first rotate Q and K on the fp32 accumulators (staged in LDS a band at a time).
template <typename T, typename C>
__device__ __attribute__((always_inline)) inline void proj_epilogue(const ProjArgs& a, f32x16 (&acc)[C::MB][C::NB],
                                                                    unsigned char* smem, const int seg, const int nseg,
                                                                    const int m0, const int n0, const int wm, const int wn,
                                                                    const int lane, const int tid) {
  constexpr int BM = C::BM, BN = C::BN, VEC = C::VEC, MB = C::MB, NB = C::NB, THREADS = C::THREADS;
  constexpr int CH = BN / VEC;                   // 16-byte chunks per output row
  auto store_chunk = [&](const int m, const int n, const uint4 val) __attribute__((always_inline)) {
    proj_store<T>(a, seg, nseg, m, n, val);
  };

  if (a.rope_cs != nullptr && seg < 2) {
    // Rotary embedding of Q and K at positions past_len[b] + t, on the fp32 accumulators before the
    // rounding: the tile is staged in fp32, a band of wave rows at a time, and each 16-byte output
    // chunk is formed from its own columns and their partners d/2 away in the same head (a
    // workgroup's columns start at a multiple of 128 and hold whole heads).
    constexpr int LDF = BN + 4;                  // padded fp32 staging row
    constexpr int WROWS = 32 * MB;               // rows of one wave row
    constexpr int FIT = (C::SMEM / (LDF * 4)) / WROWS;   // wave rows whose fp32 tile fits the LDS
    constexpr int BAND = FIT >= C::WM ? C::WM : (FIT >= 2 ? 2 : 1);   // wave rows per band
    static_assert(C::WM % BAND == 0 && BAND * WROWS * LDF * 4 <= C::SMEM, "fp32 staging band");
    float* sF = reinterpret_cast<float*>(smem);
    const int half = a.d / 2;
    for (int band = 0; band < C::WM / BAND; ++band) {
      if (wm / BAND == band) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int r = (wm % BAND) * WROWS + i * 32 + acc_row(v, lane);
              sF[r * LDF + wn * 32 * NB + j * 32 + (lane & 31)] = acc[i][j][v];
            }
      }
      __syncthreads();
      for (int c = tid; c < BAND * WROWS * CH; c += THREADS) {
        const int rl = c / CH, cc = (c % CH) * VEC;
        const int m = m0 + band * BAND * WROWS + rl, n = n0 + cc;
        if (m >= a.M || n >= nseg) continue;
        const int hc = n % a.d;
        const bool low = hc < half;
        const int ip = low ? hc : hc - half;
        const float* own = sF + rl * LDF + cc;
        const float* oth = sF + rl * LDF + (low ? cc + half : cc - half);
        const float2* cs = a.rope_cs + (size_t)m * half + ip;
        T res[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float2 w = cs[e];
          const float y = low ? own[e] * w.x - oth[e] * w.y : own[e] * w.x + oth[e] * w.y;
          res[e] = Elem<T>::from_float(y);
        }
        uint4 val;
        __builtin_memcpy(&val, res, 16);
        store_chunk(m, n, val);
      }
      __syncthreads();
    }
    return;
  }

  T* sO = reinterpret_cast<T*>(smem);            // [BM][LDO]
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 32 * MB + i * 32 + acc_row(v, lane);
        const int cc = wn * 32 * NB + j * 32 + (lane & 31);
        sO[r * C::LDO + cc] = Elem<T>::from_float(acc[i][j][v]);
      }
  __syncthreads();
  for (int c = tid; c < BM * CH; c += THREADS) {
    const int r = c / CH, cc = (c % CH) * VEC;
    const int m = m0 + r, n = n0 + cc;
    if (m >= a.M || n >= nseg) continue;
    store_chunk(m, n, *reinterpret_cast<const uint4*>(sO + r * C::LDO + cc));
  }
}

// 16-bit types with the default tiles: one 256x256 workgroup of 8 waves per CU, two waves per
// SIMD (256 registers a lane). Against two 128x256 workgroups per CU it loads a third fewer
// operand bytes per MFMA into the CU.
template <typename T>
__global__ __launch_bounds__(ProjCfg<T>::THREADS, ProjCfg<T>::MIN_WAVES)
void proj_kernel(const ProjArgs a) {
  using C = ProjCfg<T>;
  using MF = Mfma<T>;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, VEC = C::VEC, LDK = C::LDK, CPR = C::CPR;
  constexpr int MB = C::MB, NB = C::NB, LOADS_X = C::LOADS_X, LOADS_W = C::LOADS_W;
  constexpr int KPL = MF::KPL, KSTEP = MF::KSTEP;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM];
  T* sX = reinterpret_cast<T*>(smem);            // [2][BM][LDK]
  T* sW = sX + 2 * C::TILE_X;                    // [2][BN][LDK]

  constexpr int THREADS = C::THREADS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;          // WM x 2 waves

  // which segment and column tile this workgroup owns. The K and V tiles, whose epilogue
  // writes go over the host link, are dispatched first so that those posted writes drain
  // while the Q tiles (device memory only) are still computing.
  constexpr int order[3] = {1, 2, 0};
  int oi = 0, ty = blockIdx.y;
  while (oi < 2 && ty >= a.tiles_seg[order[oi]]) { ty -= a.tiles_seg[order[oi]]; ++oi; }
  const int seg = order[oi];
  const int n0 = ty * BN;
  const int nseg = a.n_seg[seg];
  const int m0 = blockIdx.x * BM;
  const T* __restrict__ X = reinterpret_cast<const T*>(a.x);
  const T* __restrict__ W = reinterpret_cast<const T*>(a.w[seg]);
  const int D = a.D;

  // Operand loads of reduction step kt into register set `set`. Every load is issued: rows
  // past M or past the segment read the last valid row instead (their products land in
  // outputs the epilogue never stores) and steps past the last read the last step, so each
  // LDS store waits only for its own register set, SETS steps after the loads were issued.
  const int nk = D / BK;
  const int mlast = a.M - 1, nlast = nseg - 1;
  // (two named register sets chosen by a branch, never an array indexed by the set, which
  // the compiler would place in scratch memory once it merges the calls of both sets)
  uint4 rx0[LOADS_X], rw0[LOADS_W], rx1[LOADS_X], rw1[LOADS_W];
  auto gload = [&](const int set, const int kt) __attribute__((always_inline)) {
    const int k0 = min(kt, nk - 1) * BK;
#pragma unroll
    for (int j = 0; j < LOADS_X; ++j) {
      const int c = tid + j * THREADS;
      const int r = c / CPR, kc = (c % CPR) * VEC;
      const uint4 v = *reinterpret_cast<const uint4*>(X + (size_t)min(m0 + r, mlast) * D + k0 + kc);
      if (set == 0) rx0[j] = v;
      else rx1[j] = v;
    }
#pragma unroll
    for (int j = 0; j < LOADS_W; ++j) {
      const int c = tid + j * THREADS;
      const int r = c / CPR, kc = (c % CPR) * VEC;
      const uint4 v = *reinterpret_cast<const uint4*>(W + (size_t)min(n0 + r, nlast) * D + k0 + kc);
      if (set == 0) rw0[j] = v;
      else rw1[j] = v;
    }
  };
  auto sstore = [&](const int buf, const int set) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < LOADS_X; ++j) {
      const int c = tid + j * THREADS;
      const int r = c / CPR, kc = (c % CPR) * VEC;
      *reinterpret_cast<uint4*>(sX + buf * C::TILE_X + r * LDK + kc) = set == 0 ? rx0[j] : rx1[j];
    }
#pragma unroll
    for (int j = 0; j < LOADS_W; ++j) {
      const int c = tid + j * THREADS;
      const int r = c / CPR, kc = (c % CPR) * VEC;
      *reinterpret_cast<uint4*>(sW + buf * C::TILE_W + r * LDK + kc) = set == 0 ? rw0[j] : rw1[j];
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // step kt computes from LDS buffer kt % 2. 16-bit types: one register set (SETS = 1) carries
  // step kt + 1's operands, loaded during step kt - 1 and stored to LDS during step kt: at 64-deep
  // steps one step of products covers the load latency, and the second set would spill (70B-shaped
  // projection 5.59 -> 5.11-5.24 ms against 32-deep steps with two sets; 8B-shaped the same).
  // fp32 keeps two sets: set 0 carries steps 1, 3, 5, ... and set 1 steps 2, 4, 6, ... (loaded
  // two steps ahead, stored to LDS one step ahead).
  auto step = [&](const int kt, const int buf, const int set) __attribute__((always_inline)) {
    const T* tX = sX + buf * C::TILE_X;
    const T* tW = sW + buf * C::TILE_W;
#pragma unroll
    for (int ks = 0; ks < BK / KSTEP; ++ks) {
      typename MF::frag fa[MB], fb[NB];
      const int kk = ks * KSTEP + (lane >> 5) * KPL;
#pragma unroll
      for (int i = 0; i < MB; ++i)
        fa[i] = *reinterpret_cast<const typename MF::frag*>(tX + (wm * 32 * MB + i * 32 + (lane & 31)) * LDK + kk);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        fb[j] = *reinterpret_cast<const typename MF::frag*>(tW + (wn * 32 * NB + j * 32 + (lane & 31)) * LDK + kk);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = MF::mma(fa[i], fb[j], acc[i][j]);
    }
    constexpr int SETS = sizeof(T) == 2 ? DKV_PROJ_SETS : 2;
    if (kt + 1 < nk) sstore(buf ^ 1, SETS == 2 ? set : 0);
    gload(SETS == 2 ? set : 0, kt + 1 + SETS);
    __syncthreads();
  };
  gload(0, 0);
  sstore(0, 0);
  gload(0, 1);
  if (sizeof(T) != 2 || DKV_PROJ_SETS == 2) gload(1, 2);
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {   // whole pairs of steps, no exit mid-body
    step(kt, 0, 0);
    step(kt + 1, 1, 1);
  }
  if (kt < nk) step(kt, 0, 0);

  proj_epilogue<T, C>(a, acc, smem, seg, nseg, m0, n0, wm, wn, lane, tid);
}

// ---- few rows (M <= kProjSmallRows): the 256x256 tiles would leave most CUs idle (a 128-token step has
// one row of tiles), so each workgroup takes 32 rows x one head (d columns) of a segment and its
// 8 waves split the reduction: wave w takes reduction steps w, w + 8, ... and the partial tiles
// are summed in LDS in wave order. Operands come straight from L2 into MFMA fragments (no LDS
// staging: the matrices are small and every element is read by few workgroups). fp32 takes its
// fragments as 16-byte loads too: with the 32x32x2 instruction, lanes 0-31 supply reduction
// index 8j + s and lanes 32-63 index 8j + 4 + s for s = 0..3 (any order of the reduction index
// is the same sum, the same for both operands), so four instructions consume one load.
constexpr int kSmallWaves = 8;

template <typename T, int DH>
__global__ __launch_bounds__(64 * kSmallWaves) void proj_small_kernel(const ProjArgs a) {
  constexpr int EB = sizeof(T), VEC = 16 / EB;
  constexpr int NB = DH / 32;                         // 32-column blocks of the head
  constexpr int STEP = EB == 2 ? 16 : 8;              // reduction elements per step
  constexpr int LDR = DH + 4;                         // padded fp32 row of the partial tiles
  __shared__ __attribute__((aligned(16))) float sR[kSmallWaves * 32 * LDR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  constexpr int order[3] = {1, 2, 0};                 // K and V first (their rows go to the host)
  int oi = 0, ty = blockIdx.y;
  while (oi < 2 && ty >= a.tiles_seg[order[oi]]) { ty -= a.tiles_seg[order[oi]]; ++oi; }
  const int seg = order[oi];
  const int nseg = a.n_seg[seg];
  const int n0 = ty * DH, m0 = blockIdx.x * 32;
  const int D = a.D;
  const T* __restrict__ X = reinterpret_cast<const T*>(a.x) + (size_t)min(m0 + (lane & 31), a.M - 1) * D;
  const T* __restrict__ W = reinterpret_cast<const T*>(a.w[seg]) + (size_t)(n0 + (lane & 31)) * D;
  const int koff = (lane >> 5) * (STEP / 2);

  f32x16 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
  // a wave's steps go U at a time: all U steps' loads are issued before their products, so a
  // short reduction (a few steps per wave) waits for memory once, not once per step
  constexpr int U = 4;
  const int nsteps = D / STEP;
  for (int st0 = wave; st0 < nsteps; st0 += U * kSmallWaves) {
    uint4 xa[U], wb[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(st0 + u * kSmallWaves, nsteps - 1) * STEP + koff;   // past the end: reread the last step
      xa[u] = *reinterpret_cast<const uint4*>(X + k);
#pragma unroll
      for (int j = 0; j < NB; ++j) wb[u][j] = *reinterpret_cast<const uint4*>(W + (size_t)j * 32 * D + k);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // a step past the end adds the zero product (exact) instead of branching: a branch here
      // lets the compiler sink each step's loads down to their use
      if (st0 + u * kSmallWaves >= nsteps) xa[u] = make_uint4(0, 0, 0, 0);
      if constexpr (EB == 2) {
        typedef typename Mfma<T>::frag F;
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[j] = Mfma<T>::mma(__builtin_bit_cast(F, xa[u]), __builtin_bit_cast(F, wb[u][j]), acc[j]);
      } else {
        const float* fa = reinterpret_cast<const float*>(&xa[u]);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const float* fb = reinterpret_cast<const float*>(&wb[u][j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[j] = Mfma<float>::mma(fa[e], fb[e], acc[j]);
        }
      }
    }
  }
  // partial tiles to LDS, then the sum over waves in wave order
  float* mine = sR + wave * 32 * LDR;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) mine[acc_row(v, lane) * LDR + j * 32 + (lane & 31)] = acc[j][v];
  __syncthreads();
  for (int e = tid; e < 32 * DH; e += 64 * kSmallWaves) {
    const int r = e / DH, c = e - r * DH;
    float sum = sR[r * LDR + c];
#pragma unroll
    for (int w = 1; w < kSmallWaves; ++w) sum += sR[w * 32 * LDR + r * LDR + c];
    sR[r * LDR + c] = sum;
  }
  __syncthreads();
  // round (after the rotary embedding of Q and K, if any) and store 16-byte chunks
  const bool rope = a.rope_cs != nullptr && seg < 2;
  constexpr int HALF = DH / 2;
  for (int c = tid; c < 32 * (DH / VEC); c += 64 * kSmallWaves) {
    const int r = c / (DH / VEC), cc = (c % (DH / VEC)) * VEC;
    const int m = m0 + r;
    if (m >= a.M) continue;
    const float* own = sR + r * LDR + cc;
    T res[VEC];
    if (rope) {
      const bool low = cc < HALF;
      const float* oth = sR + r * LDR + (low ? cc + HALF : cc - HALF);
      const float2* cs = a.rope_cs + (size_t)m * HALF + (low ? cc : cc - HALF);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float2 w = cs[e];
        res[e] = Elem<T>::from_float(low ? own[e] * w.x - oth[e] * w.y : own[e] * w.x + oth[e] * w.y);
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) res[e] = Elem<T>::from_float(own[e]);
    }
    uint4 val;
    __builtin_memcpy(&val, res, 16);
    proj_store<T>(a, seg, nseg, m, n0 + cc, val);
  }
}

template <typename T>
static hipError_t launch_proj(const ProjArgs& args, hipStream_t s) {
  ProjArgs a = args;
  if (a.M <= kProjSmallRows) {
    for (int g = 0; g < 3; ++g) a.tiles_seg[g] = a.n_seg[g] / a.d;
    const dim3 grid((a.M + 31) / 32, a.tiles_seg[0] + a.tiles_seg[1] + a.tiles_seg[2]);
    if (a.d == 128) hipLaunchKernelGGL((proj_small_kernel<T, 128>), grid, dim3(64 * kSmallWaves), 0, s, a);
    else hipLaunchKernelGGL((proj_small_kernel<T, 64>), grid, dim3(64 * kSmallWaves), 0, s, a);
    return hipGetLastError();
  }
  constexpr int BM = ProjCfg<T>::BM, BN = ProjCfg<T>::BN;
  for (int g = 0; g < 3; ++g) a.tiles_seg[g] = (a.n_seg[g] + BN - 1) / BN;
  const int mt = (a.M + BM - 1) / BM;
  const int nt = a.tiles_seg[0] + a.tiles_seg[1] + a.tiles_seg[2];
  hipLaunchKernelGGL(proj_kernel<T>, dim3(mt, nt), dim3(ProjCfg<T>::THREADS), 0, s, a);
  return hipGetLastError();
}

// One thread per (row m = b*T + t, pair i): the rotary (cos, sin) at position past_len[b] + t.
struct RopeTableArgs {
  int32_t B, T, d;
  double theta;
  float2* cs;
  int32_t past_len[kMaxBatch];
};

__global__ __launch_bounds__(256) void rope_table_kernel(const RopeTableArgs a) {
  const int half = a.d / 2;
  const long long n = (long long)a.B * a.T * half;
  for (long long k = (long long)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (long long)gridDim.x * blockDim.x) {
    const int i = (int)(k % half);
    const long long m = k / half;
    const int b = (int)(m / a.T), t = (int)(m - (long long)b * a.T);
    double c, sn;
    rope_angle_cs(a.past_len[b] + t, i, a.d, a.theta, c, sn);
    a.cs[k] = make_float2((float)c, (float)sn);
  }
}

hipError_t launch_rope_table(const int32_t* past_len, int B, int T, int d, double theta, float2* cs,
                             hipStream_t s) {
  RopeTableArgs a;
  a.B = B;
  a.T = T;
  a.d = d;
  a.theta = theta;
  a.cs = cs;
  for (int b = 0; b < B && b < kMaxBatch; ++b) a.past_len[b] = past_len[b];
  const long long n = (long long)B * T * (d / 2);
  const int grid = (int)std::min<long long>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

proj_fn find_proj(int dtype, int d) {
  if (d != 64 && d != 128) return nullptr;
  switch (dtype) {
    case 0: return launch_proj<float>;
    case 1: return launch_proj<_Float16>;
    case 2: return launch_proj<__bf16>;
    default: return nullptr;
  }
}

}  // namespace dkv
