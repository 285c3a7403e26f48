// Triangular multiplicative update on gfx950.
//
// Edge (i, j) of the pair representation is updated from every third residue
// k as the sum over k of a_ik * b_jk, channel by channel ("Evoformer: the
// memory wall ZeRO cannot move", section "The three operations": O(N^3)
// time, O(N^2) memory).  a and b are projections of the layer-normalised
// pair representation; the update is projected back to c_z:
//   x = LN(z),  a = x . W_a^T,  b = x . W_b^T                 (c channels)
//   t[i,j,c] = sum_k keep[k] a[i,k,c] b[j,k,c]              (outgoing)
//   t[i,j,c] = sum_k keep[k] a[k,i,c] b[k,j,c]              (incoming)
//   out[i,j] = t[i,j] . W_o^T + b_o
// Steps:
//   1. the persistent row GEMM of the triangle-attention module (LayerNorm
//      fused, the normalised tensor never written) writes a and b
//      channel-major with padded rows, A_c[i][k] and B_c[j][k] (row = line,
//      column = place; incoming reads z transposed), zero where k is masked;
//      a small kernel zeroes the padding columns k >= N;
//   2. trimul_gemm: for every channel, T_c = A_c . B_c^T, a dense
//      contraction over k on the matrix cores (fp32 accumulation), 128 x 128
//      output tiles, K staged through double-buffered LDS (a single large
//      bf16 product, as in the outer product mean, uses pair_gemm_bf16:
//      256 x 128 tiles, A straight into registers, B through LDS);
//   3. trimul_out: out[p] = W_o . T[:, p] + b_o with T read channel-major,
//      staged through LDS and read with transposing LDS reads.
#include <algorithm>
#include <type_traits>

#include "evo_device.h"
#include "evo_kernels.h"

namespace evo {
namespace {

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
constexpr int kTile = 128;  // fp32 GEMM output tile (rows and columns)
constexpr int kRowPad = 256;  // operand rows are padded to a multiple of this

template <typename T> struct MulCfg;
// K columns per LDS stage; LDS row stride (elements)
template <> struct MulCfg<bf16_t> { static constexpr int BK = 64, RS = 72; };
template <> struct MulCfg<float> { static constexpr int BK = 32, RS = 36; };

// Columns [K, Kp) of rows [0, M) of the C matrices [Np][Kp] of a and of
// rows [0, M2) of the C matrices [Np2][Kp] of b: zero (a_frag: a in
// fragment order, frag_off).
template <typename T>
__global__ void __launch_bounds__(256) pad_cols_kernel(T* a, T* b, int C, int M, int M2, int K,
                                                       int Np, int Np2, int Kp, int a_frag) {
  const int padw = Kp - K, Mm = M > M2 ? M : M2;
  const int64_t total = (int64_t)C * Mm * padw;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int col = K + (int)(e % padw);
    const int64_t r = e / padw;  // matrix * Mm + row
    const int c = (int)(r / Mm), row = (int)(r - (int64_t)c * Mm);
    if (row < M)
      a[a_frag ? (int64_t)c * Np * Kp + frag_off(row, col, Kp)
               : ((int64_t)c * Np + row) * Kp + col] = T(0);
    if (row < M2) b[((int64_t)c * Np2 + row) * Kp + col] = T(0);
  }
}

// ----------------------------------------------------------------- GEMM
struct MulGemmParams {
  int C, N, Np, Kp;  // N: rows of each product (at most Np)
  int N2, Np2;       // columns of each product (rows of b, at most Np2)
  const void* a;  // [C][Np][Kp]
  const void* b;  // [C][Np2][Kp]
  void* t;        // [C][N][N2]
  int ntile, ntile2;  // Np / kTile, Np2 / kTile
  // pair_c > 0 (bf16 256 x 128 kernel, one product): T[(i, c)][(j, d)] is
  // written as pair rows t[(i * pair_n + j) * pair_c + c][d] times pair_scale
  // (rows and columns of T are residue * pair_c + channel)
  int pair_n, pair_c;
  float pair_scale;
};

// Row tiles per group of the work order.
constexpr int kGroup = 8;

template <typename T>
__device__ __forceinline__ void st4t(T* p, const f32x4& v);
template <>
__device__ __forceinline__ void st4t<bf16_t>(bf16_t* p, const f32x4& v) {
  uint2 u;
  u.x = uint32_t(Tr<bf16_t>::from_f(v[0])) | (uint32_t(Tr<bf16_t>::from_f(v[1])) << 16);
  u.y = uint32_t(Tr<bf16_t>::from_f(v[2])) | (uint32_t(Tr<bf16_t>::from_f(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}
template <>
__device__ __forceinline__ void st4t<float>(float* p, const f32x4& v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// One workgroup (4 waves, 2 x 2) per 128 x 128 tile of one channel; a wave
// owns 64 x 64 as 4 x 4 blocks of 16 x 16.  The product is formed as
// T^T = B . A^T so that a lane's accumulators hold 4 consecutive columns j
// of one row i (one 8- or 16-byte store).  Work order: channel slowest;
// within a channel, groups of kGroup row tiles, and in a group the row tile
// fastest, so that the tiles an XCD runs at one time (the XCD mapping gives
// it a contiguous range of the order) share a few row and column tiles of A
// and B in its L2.
template <typename T>
__global__ void __launch_bounds__(256) trimul_gemm_kernel(MulGemmParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int BK = MulCfg<T>::BK, RS = MulCfg<T>::RS;
  constexpr int E16 = 16 / sizeof(T);            // elements per 16-byte chunk
  constexpr int CPR = BK / E16;                  // chunks per tile row per stage
  constexpr int CPT = kTile * CPR / 256;         // chunks per thread per tile
  __shared__ __attribute__((aligned(16))) T sA[2][kTile * RS];
  __shared__ __attribute__((aligned(16))) T sB[2][kTile * RS];

  const int w = xcd_work_index(p.C * p.ntile * p.ntile2);
  if (w < 0) return;
  const int per_c = p.ntile * p.ntile2;
  const int c = w / per_c, r0 = w - c * per_c;
  const int first = r0 / (kGroup * p.ntile2) * kGroup;
  const int h = min(kGroup, p.ntile - first);
  const int r = r0 - first * p.ntile2;
  const int ti = first + r % h, tj = r / h;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t cs = (int64_t)p.Np * p.Kp, cs2 = (int64_t)p.Np2 * p.Kp;
  const T* A = static_cast<const T*>(p.a) + c * cs + (int64_t)ti * kTile * p.Kp;
  const T* B = static_cast<const T*>(p.b) + c * cs2 + (int64_t)tj * kTile * p.Kp;

  // staging: chunk e = tid + 256 u: tile row e / CPR, elements (e % CPR) * E16
  u32x4 ra[CPT], rb[CPT];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int e = tid + 256 * u, row = e / CPR, col = (e % CPR) * E16;
      ra[u] = *reinterpret_cast<const u32x4*>(A + (int64_t)row * p.Kp + k0 + col);
      rb[u] = *reinterpret_cast<const u32x4*>(B + (int64_t)row * p.Kp + k0 + col);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int e = tid + 256 * u, row = e / CPR, col = (e % CPR) * E16;
      *reinterpret_cast<u32x4*>(sA[buf] + row * RS + col) = ra[u];
      *reinterpret_cast<u32x4*>(sB[buf] + row * RS + col) = rb[u];
    }
  };

  f32x4 acc[4][4];  // [column block bj][row block bi]
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nstage = p.Kp / BK;
  fetch(0);
  for (int st = 0; st < nstage; ++st) {
    const int buf = st & 1;
    stage(buf);
    __syncthreads();
    if (st + 1 < nstage) fetch((st + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      Op af[4], bf[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        af[x] = *reinterpret_cast<const Op*>(sA[buf] + (wi * 64 + x * 16 + l16) * RS + ks * 32 + 8 * g);
        bf[x] = *reinterpret_cast<const Op*>(sB[buf] + (wj * 64 + x * 16 + l16) * RS + ks * 32 + 8 * g);
      }
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) acc[bj][bi] = mma32(bf[bj], af[bi], acc[bj][bi]);
    }
  }

  // lane (l16, g) holds T[i = .. + bi*16 + l16][j = .. + bj*16 + 4g + r]
  T* Tc = static_cast<T*>(p.t) + (int64_t)c * p.N * p.N2;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
    const int i = ti * kTile + wi * 64 + bi * 16 + l16;
    if (i >= p.N) continue;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int j0 = tj * kTile + wj * 64 + bj * 16 + 4 * g;
      T* dst = Tc + (int64_t)i * p.N2 + j0;
      if (j0 + 3 < p.N2 && (p.N2 & 3) == 0) {
        st4t<T>(dst, acc[bj][bi]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j0 + r < p.N2) dst[r] = Tr<T>::from_f(acc[bj][bi][r]);
      }
    }
  }
}

// bf16 products: a workgroup of 4*WJ waves owns a 256 x 128*WJ tile (rows i
// of A, rows j of B); wave (wi, wj) owns rows wi*64 .. +63 and columns
// wj*128 .. +127 as 4 x 8 accumulator blocks.  Each wave's A rows are its
// own, so its A operands come straight from global memory into registers,
// one 64-wide stage ahead: A is stored in fragment order (frag_off), so
// each operand is one contiguous 1 KB load (in row-major order the same
// load touches 16 rows x 64 bytes, four times slower through the load
// path: 2.02 vs 1.81 ms per outer product mean); only B goes through
// double-buffered LDS.  Per 32-wide K step a wave issues 32
// products against 8 LDS operand reads (a 64 x 64 wave tile with both
// operands in LDS needs 8 reads for 16), and per 64-wide stage the
// workgroup moves (256 + 128*WJ) x 128 bytes from L2.
constexpr int kBigI = 256, kBigJ = 128;

template <int WJ>
__global__ void __launch_bounds__(256 * WJ) pair_gemm_bf16_kernel(MulGemmParams p) {
  using T = bf16_t;
  using Op = bf16x8;
  constexpr int BK = 64, RS = 72;
  constexpr int NT = 256 * WJ;                 // threads
  constexpr int BROWS = kBigJ * WJ;            // B rows per tile
  constexpr int CPT = BROWS * (BK / 8) / NT;   // 16-byte B chunks per thread per stage
  __shared__ __attribute__((aligned(16))) T sB[2][BROWS * RS];

  const int nti = p.Np / kBigI, ntj = p.Np2 / BROWS;
  const int w = xcd_work_index(p.C * nti * ntj);
  if (w < 0) return;
  const int per_c = nti * ntj;
  const int c = w / per_c, r0 = w - c * per_c;
  constexpr int G = 4;  // row tiles per group of the work order
  const int first = r0 / (G * ntj) * G;
  const int h = min(G, nti - first);
  const int r = r0 - first * ntj;
  const int ti = first + r % h, tj = r / h;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int wi = wave & 3, wj = wave >> 2;
  const int64_t cs = (int64_t)p.Np * p.Kp, cs2 = (int64_t)p.Np2 * p.Kp;
  // this wave's first 16-row block of A (fragment order), this lane's slot
  const int kblk = p.Kp >> 5;  // 32-column blocks per row block
  const T* A = static_cast<const T*>(p.a) + c * cs +
               ((int64_t)(ti * kBigI + wi * 64) >> 4) * kblk * 512 + lane * 8;
  const T* B = static_cast<const T*>(p.b) + c * cs2 + (int64_t)tj * BROWS * p.Kp;

  u32x4 rb[CPT];
  auto fetch_b = [&](int k0) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int e = tid + NT * u, row = e >> 3, col = (e & 7) * 8;
      rb[u] = *reinterpret_cast<const u32x4*>(B + (int64_t)row * p.Kp + k0 + col);
    }
  };
  auto stage_b = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int e = tid + NT * u, row = e >> 3, col = (e & 7) * 8;
      *reinterpret_cast<u32x4*>(sB[buf] + row * RS + col) = rb[u];
    }
  };
  // A operands of one stage: [k step][row block]
  Op an[2][4], ac[2][4];
  auto fetch_a = [&](Op (&v)[2][4], int k0) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
        v[ks][bi] = *reinterpret_cast<const Op*>(A + ((int64_t)bi * kblk + (k0 >> 5) + ks) * 512);
  };

  f32x4 acc[8][4];  // [column block bj][row block bi]
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nstage = p.Kp / BK;
  fetch_b(0);
  fetch_a(an, 0);
  for (int st = 0; st < nstage; ++st) {
    const int buf = st & 1;
    stage_b(buf);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) ac[ks][bi] = an[ks][bi];
    // next stage (the last one again at the end: in bounds, exact waits)
    const int nk0 = min(st + 1, nstage - 1) * BK;
    fetch_b(nk0);
    fetch_a(an, nk0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        Op bf[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
          bf[x] = *reinterpret_cast<const Op*>(
              sB[buf] + (wj * kBigJ + (half * 4 + x) * 16 + l16) * RS + ks * 32 + 8 * g);
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int bi = 0; bi < 4; ++bi)
            acc[half * 4 + x][bi] = mma32(bf[x], ac[ks][bi], acc[half * 4 + x][bi]);
      }
    }
  }

  // lane (l16, g) holds T[i = .. + bi*16 + l16][j = .. + bj*16 + 4g + r]
  if (p.pair_c > 0) {
    // pair rows: the 4 consecutive j of a lane share one residue (pair_c is a
    // multiple of 32), so each stays one 8-byte store
    const int PC = p.pair_c;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      const int i = ti * kBigI + wi * 64 + bi * 16 + l16;
      if (i >= p.N) continue;
      const int ir = i / PC, ci = i - ir * PC;
#pragma unroll
      for (int bj = 0; bj < 8; ++bj) {
        const int j0 = tj * BROWS + wj * kBigJ + bj * 16 + 4 * g;
        if (j0 >= p.N2) continue;
        const int jr = j0 / PC, dj = j0 - jr * PC;
        st4t<T>(static_cast<T*>(p.t) + ((int64_t)(ir * p.pair_n + jr) * PC + ci) * PC + dj,
                acc[bj][bi] * p.pair_scale);
      }
    }
    return;
  }
  T* Tc = static_cast<T*>(p.t) + (int64_t)c * p.N * p.N2;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
    const int i = ti * kBigI + wi * 64 + bi * 16 + l16;
    if (i >= p.N) continue;
#pragma unroll
    for (int bj = 0; bj < 8; ++bj) {
      const int j0 = tj * BROWS + wj * kBigJ + bj * 16 + 4 * g;
      T* dst = Tc + (int64_t)i * p.N2 + j0;
      if (j0 + 3 < p.N2 && (p.N2 & 3) == 0) {
        st4t<T>(dst, acc[bj][bi]);
      } else {
#pragma unroll
        for (int r2 = 0; r2 < 4; ++r2)
          if (j0 + r2 < p.N2) dst[r2] = Tr<T>::from_f(acc[bj][bi][r2]);
      }
    }
  }
}

// ------------------------------------------------------ output projection
struct MulOutParams {
  int C, CZ, npos, ntiles;
  const void* t;     // [C][npos]
  const void* w_o;   // [CZ][C]
  const void* b_o;   // [CZ] or null
  void* out;         // [npos][CZ]
};

// Positions per workgroup tile (32 per wave).
constexpr int kOutP = 128;

template <typename T> struct OutLds;
// bf16: T tile [C][128 + 8] read with transposing reads; fp32: [128][C + 4]
// (stored transposed).
template <> struct OutLds<bf16_t> { static constexpr int TS = kOutP + 8; };
template <> struct OutLds<float> { static constexpr int TS = 128 + 4; };

// Persistent workgroups (4 waves) with W_o resident in LDS; per tile of 128
// positions: T[:, tile] staged in LDS, then out^T = W_o . T for each wave's
// 32 positions.
template <typename T, int CB, int KS>  // CB = CZ / 16, KS = C / 32
__global__ void __launch_bounds__(256) trimul_out_kernel(MulOutParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int TS = OutLds<T>::TS;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int C = 32 * KS, WS = C + 8;
  T* sW = reinterpret_cast<T*>(smem);        // [CZ][C + 8]
  T* sT = sW + CB * 16 * WS;                 // bf16 [C][TS]; fp32 [kOutP][TS]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int CZ = CB * 16;

  for (int e = tid; e < CZ * C; e += 256) {
    const int r = e / C, k = e - r * C;
    sW[r * WS + k] = static_cast<const T*>(p.w_o)[e];
  }
  float bo[CB / 2][8];
#pragma unroll
  for (int s = 0; s < CB / 2; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // column constant of output channel cb*16 + 4g + r, cb = 2s + j/4, r = j%4
      const int cz = (2 * s + (j >> 2)) * 16 + 4 * g + (j & 3);
      bo[s][j] = p.b_o ? Tr<T>::to_f(static_cast<const T*>(p.b_o)[cz]) : 0.f;
    }
  const T* Tg = static_cast<const T*>(p.t);
  const int ksteps = C / 32;
  // T[:, p0 .. p0+127] of a tile: chunk e = tid + 256 u: channel e / CPR,
  // positions 8*(e % CPR) (bf16; fp32 4).  The next tile's chunks are loaded
  // into registers while the current tile is computed.
  constexpr int E16 = 16 / sizeof(T);
  constexpr int CPR = kOutP / E16;
  constexpr int NU = C * CPR / 256;  // chunks per thread
  u32x4 tr[NU];
  auto fetch_t = [&](int tile) {
    const int p0 = tile * kOutP;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int e = tid + 256 * u;
      const int k = e / CPR, pc = (e % CPR) * E16;
      const int pos = p0 + pc;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (pos + E16 <= p.npos) {
        v = *reinterpret_cast<const u32x4*>(Tg + (int64_t)k * p.npos + pos);
      } else {
#pragma unroll
        for (int q = 0; q < E16; ++q)
          if (pos + q < p.npos) {
            const T x = Tg[(int64_t)k * p.npos + pos + q];
            if constexpr (sizeof(T) == 2)
              v[q >> 1] |= uint32_t(x) << (16 * (q & 1));
            else
              v[q] = __float_as_uint(x);
          }
      }
      tr[u] = v;
    }
  };
  fetch_t(min((int)blockIdx.x, p.ntiles - 1));
  for (int tile = blockIdx.x; tile < p.ntiles; tile += gridDim.x) {
    const int p0 = tile * kOutP;
    __syncthreads();  // previous tile's reads (and the weights) done
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int e = tid + 256 * u;
      const int k = e / CPR, pc = (e % CPR) * E16;
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<u32x4*>(sT + k * TS + pc) = tr[u];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) sT[(pc + q) * TS + k] = __uint_as_float(tr[u][q]);
      }
    }
    // the next tile (the last one again at the end: exact waits)
    fetch_t(min(tile + (int)gridDim.x, p.ntiles - 1));
    __syncthreads();
    f32x4 acc[CB][2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb][0] = acc[cb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < ksteps; ++ks) {
      Op tf[2];
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        const int pl = wave * 32 + pb * 16;  // tile-local position block
        if constexpr (sizeof(T) == 2) {
          // rows (channels) ks*32 + 8g .. +7 of column pl + l16
          const T* q0 = sT + (ks * 32 + 8 * g + (l16 >> 2)) * TS + pl + 4 * (l16 & 3);
          tf[pb] = lds_read_tr_op(q0, q0 + 4 * TS);
        } else {
          const float* q0 = sT + (pl + l16) * TS + ks * 32 + 8 * g;
          tf[pb] = f32x8{q0[0], q0[1], q0[2], q0[3], q0[4], q0[5], q0[6], q0[7]};
        }
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const Op wf = *reinterpret_cast<const Op*>(sW + (cb * 16 + l16) * WS + ks * 32 + 8 * g);
        acc[cb][0] = mma32(wf, tf[0], acc[cb][0]);
        acc[cb][1] = mma32(wf, tf[1], acc[cb][1]);
      }
    }
    // lane (l16, g) holds out[position .. + l16][cb*16 + 4g + r]
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      const int pos = p0 + wave * 32 + pb * 16 + l16;
      if (pos >= p.npos) continue;
      T* dst = static_cast<T*>(p.out) + (int64_t)pos * CZ + 4 * g;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        f32x4 v = acc[cb][pb];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += bo[cb >> 1][4 * (cb & 1) + r];
        st4t<T>(dst + cb * 16, v);
      }
    }
  }
}

template <typename T, int CB, int KS>
hipError_t launch_out_k(MulOutParams& o, hipStream_t s) {
  const size_t lds = (size_t)CB * 16 * (o.C + 8) * sizeof(T) +
                     (size_t)(sizeof(T) == 2 ? o.C : kOutP) * OutLds<T>::TS * sizeof(T);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&trimul_out_kernel<T, CB, KS>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int grid = std::min(o.ntiles, 512);
  hipLaunchKernelGGL((trimul_out_kernel<T, CB, KS>), dim3(grid), dim3(256), lds, s, o);
  return hipGetLastError();
}

template <typename T, int CB>
hipError_t launch_out(MulOutParams& o, hipStream_t s) {
  switch (o.C / 32) {
    case 1: return launch_out_k<T, CB, 1>(o, s);
    case 2: return launch_out_k<T, CB, 2>(o, s);
    case 3: return launch_out_k<T, CB, 3>(o, s);
    case 4: return launch_out_k<T, CB, 4>(o, s);
    default: return hipErrorInvalidValue;
  }
}

struct MulLayout {
  int64_t Np, Kp;
  size_t a, b, t, total;
};
MulLayout mul_layout(int dtype, int64_t N, int64_t C) {
  const size_t es = dtype == 1 ? 2 : 4;
  MulLayout L;
  L.Np = round_up(N, kRowPad);
  L.Kp = round_up(N, 64);
  const size_t ab = ((size_t)C * L.Np * L.Kp * es + 255) & ~size_t(255);
  L.a = 0;
  L.b = ab;
  L.t = 2 * ab;
  L.total = L.t + (((size_t)C * N * N * es + 255) & ~size_t(255));
  return L;
}

// T_c = A_c . B_c^T: A [C][Np][Kp] (M rows), B [C][Np2][Kp] (M2 rows), T
// [C][M][M2].
template <typename T>
hipError_t pair_gemm_t(int C, int M, int M2, int K, int Np, int Np2, int Kp, T* A, T* B, T* Tm,
                       bool a_frag, hipStream_t s, int pair_n = 0, int pair_c = 0,
                       float pair_scale = 1.f) {
  hipError_t e;
  if (Kp > K) {
    const int64_t total = (int64_t)C * std::max(M, M2) * (Kp - K);
    const int grid = (int)std::min<int64_t>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(pad_cols_kernel<T>, dim3(grid), dim3(256), 0, s, A, B, C, M, M2, K, Np,
                       Np2, Kp, (int)a_frag);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  MulGemmParams g{};
  g.C = C; g.N = M; g.Np = Np; g.Kp = Kp;
  g.N2 = M2; g.Np2 = Np2;
  g.a = A; g.b = B; g.t = Tm;
  g.ntile = Np / kTile;
  g.ntile2 = Np2 / kTile;
  g.pair_n = pair_n;
  g.pair_c = pair_c;
  g.pair_scale = pair_scale;
  // bf16: the 256 x 128 kernel for one large product (24576^2 by K = 1024:
  // 1.78 vs 1.93 ms), the 128 x 128 one for many small ones (128 products of
  // 768^2 by 768: 206 vs 218 us)
  if (sizeof(T) == 2 && C == 1 && a_frag) {
    constexpr int WJ = 1;  // 256 x 256 tiles with 8 waves (WJ = 2) measured slower
    const int total = C * (Np / kBigI) * (Np2 / (kBigJ * WJ));
    const int grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
    if constexpr (sizeof(T) == 2)
      hipLaunchKernelGGL(pair_gemm_bf16_kernel<WJ>, dim3(grid), dim3(256 * WJ), 0, s, g);
  } else {
    // the 128 x 128 kernel reads row-major A and writes T in plain rows
    if (a_frag || pair_c > 0) return hipErrorInvalidValue;
    const int total = C * g.ntile * g.ntile2;
    const int grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
    hipLaunchKernelGGL(trimul_gemm_kernel<T>, dim3(grid), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t trimul_t(const TriMulArgs& a, hipStream_t s) {
  const MulLayout L = mul_layout(a.dtype, a.N, a.C);
  char* ws = static_cast<char*>(a.workspace);
  T* A = reinterpret_cast<T*>(ws + L.a);
  T* B = reinterpret_cast<T*>(ws + L.b);
  T* Tm = reinterpret_cast<T*>(ws + L.t);
  const int N = (int)a.N, C = (int)a.C;
  // A_c[line][place], B_c likewise; incoming lines read z transposed
  ChannelProjectArgs pa{a.dtype, a.N, a.N, a.CZ, a.C, a.outgoing ? 0 : 1, a.z, a.mask,
                        a.ln_w, a.ln_b, a.eps, a.w_a, a.w_b, A, B,
                        L.Np * L.Kp, L.Kp, 1};
  hipError_t e = launch_channel_project(pa, s);
  if (e != hipSuccess) return e;
  if ((e = pair_gemm_t<T>(C, N, N, N, (int)L.Np, (int)L.Np, (int)L.Kp, A, B, Tm, false, s)) != hipSuccess)
    return e;
  MulOutParams o{};
  o.C = C; o.CZ = (int)a.CZ; o.npos = N * N;
  o.ntiles = (o.npos + kOutP - 1) / kOutP;
  o.t = Tm; o.w_o = a.w_o; o.b_o = a.b_o; o.out = a.out;
  switch (o.CZ / 16) {
    case 2: return launch_out<T, 2>(o, s);
    case 4: return launch_out<T, 4>(o, s);
    case 6: return launch_out<T, 6>(o, s);
    case 8: return launch_out<T, 8>(o, s);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------- backward
// Channel-major <-> position-major permutes for the backward, through LDS:
// a workgroup takes 64 columns q of one matrix row r for every channel, so
// it reads or writes C runs of 64 contiguous elements on the channel-major
// side and 64 rows of C contiguous elements on the position-major side.
constexpr int kPermQ = 64;
constexpr int kMaxC = 128;

template <typename T>
__device__ __forceinline__ void ld16e(const T* p, T (&v)[16 / sizeof(T)]) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(p);
  __builtin_memcpy(v, &u, 16);
}
template <typename T>
__device__ __forceinline__ void st16e(T* p, const T (&v)[16 / sizeof(T)]) {
  u32x4 u;
  __builtin_memcpy(&u, v, 16);
  *reinterpret_cast<u32x4*>(p) = u;
}

// Matrices [C] of (row r < rows, column q < ncols) at c*cs + r*ld + q to
// rows dst[pos][C], pos = r*N + q (q*N + r when trans); zero where keep is
// given and keep[q] == 0.  vec: cs and ld are multiples of 16 bytes.
// A thread loads the same 16-byte run of positions from 4 consecutive
// channels and writes each position's 4 channels as one LDS store; the
// 4-channel group g of position q sits in slot g ^ perm_swz(q) of its LDS
// row, which spreads the stores of a wave over all banks and keeps the two
// groups of an aligned 8-channel read adjacent and in order.
template <typename T>
__device__ __forceinline__ int perm_swz(int q) {
  return sizeof(T) == 2 ? 2 * ((q >> 3) & 7) : ((q >> 2) & 7);
}
template <typename T>
__global__ void __launch_bounds__(256) cm_to_pm_kernel(const T* src, T* dst, int C, int ncols,
                                                       int64_t ld, int64_t cs, int N, int trans,
                                                       const uint8_t* keep, int vec) {
  constexpr int E = 16 / sizeof(T), TS = kMaxC;
  using T4 = typename std::conditional<sizeof(T) == 2, uint2, u32x4>::type;
  __shared__ __attribute__((aligned(16))) T tile[kPermQ * TS];  // [q][c], swizzled groups
  const int r = blockIdx.y, q0 = blockIdx.x * kPermQ, tid = threadIdx.x;
  constexpr int CPS = kPermQ / E;  // 16-byte chunks per channel run
  for (int e = tid; e < C / 4 * CPS; e += 256) {
    const int cg = e / CPS, ql = (e % CPS) * E, q = q0 + ql;
    T v[4][E];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const T* sp = src + (int64_t)(4 * cg + u) * cs + (int64_t)r * ld + q;
      if (vec && q + E <= ncols) {
        ld16e(sp, v[u]);
      } else {
#pragma unroll
        for (int j = 0; j < E; ++j) v[u][j] = q + j < ncols ? sp[j] : T(0);
      }
    }
#pragma unroll
    for (int j = 0; j < E; ++j) {
      T w[4] = {v[0][j], v[1][j], v[2][j], v[3][j]};
      T4 x;
      __builtin_memcpy(&x, w, sizeof(x));
      const int slot = cg ^ perm_swz<T>(ql + j);
      *reinterpret_cast<T4*>(tile + (ql + j) * TS + 4 * slot) = x;
    }
  }
  __syncthreads();
  const int CPP = C / E;  // chunks per position
  for (int e = tid; e < kPermQ * CPP; e += 256) {
    const int ql = e / CPP, c0 = (e % CPP) * E, q = q0 + ql;
    if (q >= ncols) continue;
    const int64_t pos = trans ? (int64_t)q * N + r : (int64_t)r * N + q;
    const bool dead = keep && keep[q] == 0;
    const int slot = (c0 >> 2) ^ perm_swz<T>(ql);
    T v[E];
    ld16e(tile + ql * TS + 4 * slot, v);
#pragma unroll
    for (int j = 0; j < E; ++j) v[j] = dead ? T(0) : v[j];
    st16e(dst + pos * C + c0, v);
  }
}

// Rows src[pos][C] to matrices [C][Np][Kp] (row r, column q) at c*cs + r*Kp
// + q: src[pos][c] with pos = r*N + q (q*N + r when trans), zero for r >= N
// or q >= N.  Grid: (Kp / 64, Np).  A thread loads one 16-byte run of
// channels from 4 consecutive positions and writes each channel's 4
// positions as one LDS store, in slot pg ^ ((c / E) & 15) of the channel's
// row (pg: the group of 4 positions).
template <typename T>
__global__ void __launch_bounds__(256) pm_to_cm_kernel(const T* src, T* dst, int C, int N,
                                                       int64_t Kp, int64_t cs, int trans) {
  constexpr int E = 16 / sizeof(T), TS = kPermQ;
  using T4 = typename std::conditional<sizeof(T) == 2, uint2, u32x4>::type;
  __shared__ __attribute__((aligned(16))) T tile[kMaxC * TS];  // [c][q], swizzled groups
  const int r = blockIdx.y, q0 = blockIdx.x * kPermQ, tid = threadIdx.x;
  const int CPP = C / E;
  for (int e = tid; e < kPermQ / 4 * CPP; e += 256) {
    const int pg = e / CPP, cc = e % CPP, c0 = cc * E;
    T v[4][E];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + 4 * pg + u;
      if (r < N && q < N) {
        const int64_t pos = trans ? (int64_t)q * N + r : (int64_t)r * N + q;
        ld16e(src + pos * C + c0, v[u]);
      } else {
#pragma unroll
        for (int j = 0; j < E; ++j) v[u][j] = T(0);
      }
    }
    const int slot = pg ^ (cc & 15);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      T w[4] = {v[0][j], v[1][j], v[2][j], v[3][j]};
      T4 x;
      __builtin_memcpy(&x, w, sizeof(x));
      *reinterpret_cast<T4*>(tile + (c0 + j) * TS + 4 * slot) = x;
    }
  }
  __syncthreads();
  constexpr int CPS = kPermQ / E;
  for (int e = tid; e < C * CPS; e += 256) {
    const int c = e / CPS, ql = (e % CPS) * E;
    const int sw = (c / E) & 15;
    T v[E];
#pragma unroll
    for (int h = 0; h < E / 4; ++h) {
      const T4 x = *reinterpret_cast<const T4*>(tile + c * TS + 4 * ((ql / 4 + h) ^ sw));
      __builtin_memcpy(&v[4 * h], &x, sizeof(x));
    }
    st16e(dst + (int64_t)c * cs + (int64_t)r * Kp + q0 + ql, v);
  }
}

template <typename T>
hipError_t cm_to_pm(const T* src, T* dst, int C, int rows, int ncols, int64_t ld, int64_t cs,
                    int N, int trans, const uint8_t* keep, hipStream_t s) {
  constexpr int E = 16 / sizeof(T);
  const int vec = (ld % E == 0 && cs % E == 0) ? 1 : 0;
  hipLaunchKernelGGL(cm_to_pm_kernel<T>, dim3((ncols + kPermQ - 1) / kPermQ, rows), dim3(256), 0,
                     s, src, dst, C, ncols, ld, cs, N, trans, keep, vec);
  return hipGetLastError();
}
template <typename T>
hipError_t pm_to_cm(const T* src, T* dst, int C, int N, int64_t Np, int64_t Kp, int trans,
                    hipStream_t s) {
  hipLaunchKernelGGL(pm_to_cm_kernel<T>, dim3((unsigned)(Kp / kPermQ), (unsigned)Np), dim3(256),
                     0, s, src, dst, C, N, Kp, Np * Kp, trans);
  return hipGetLastError();
}

struct MulBwdLayout {
  int64_t Np, Kp;
  size_t s1, s2, a, b, at, bt, dtc, dtt, tm, tpm, dtpm, part, total;
};
MulBwdLayout mul_bwd_layout(int dtype, int64_t N, int64_t CZ, int64_t C) {
  const size_t es = dtype == 1 ? 2 : 4;
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  MulBwdLayout L;
  L.Np = round_up(N, kRowPad);
  L.Kp = round_up(N, 64);
  L.s1 = al((size_t)C * L.Np * L.Kp * es);
  L.s2 = al((size_t)C * N * N * es);
  L.a = 0;
  L.b = L.s1;
  L.at = 2 * L.s1;
  L.bt = 3 * L.s1;
  L.dtc = 4 * L.s1;
  L.dtt = 5 * L.s1;
  L.tm = 6 * L.s1;
  L.tpm = L.tm + L.s2;
  L.dtpm = L.tpm + L.s2;
  L.part = L.dtpm + L.s2;
  L.total = L.part + al(std::max(proj_bwd_workspace(N, CZ, C / kHeadDim),
                                 ln_proj_bwd_workspace(N * N, CZ, (int)C)));
  return L;
}

// Backward of the update: the chain rule of the forward, in matrix form per
// channel (A_c, B_c as in the forward, keep the residue mask):
//   dT = dout . W_o (position rows),  dW_o = sum dout^T t,  db_o = sum dout,
//   dA_c = dT_c . B_c * keep[k],  dB_c = dT_c^T . A_c * keep[k],
//   dz, dW_a, dW_b, dgamma, dbeta from the LayerNorm + projection backward.
// Steps: the forward's operands A_c, B_c (masked) and, from the same
// projection with the orientation flipped and no mask, their transposes
// A_c^T, B_c^T; T_c = A_c . B_c^T recomputed (for dW_o); the output
// projection's backward on T in position rows; dT_c and dT_c^T; the two
// products dA_c = dT_c . (B_c^T)^T and dB_c = dT_c^T . (A_c^T)^T (masked
// rows of A^T and B^T are not zero, so the mask is applied when dA and dB
// return to position rows); then the LayerNorm + projection backward.
template <typename T>
hipError_t trimul_bwd_t(const TriMulBwdArgs& a, hipStream_t s) {
  const MulBwdLayout L = mul_bwd_layout(a.dtype, a.N, a.CZ, a.C);
  char* ws = static_cast<char*>(a.workspace);
  auto at = [&](size_t off) { return reinterpret_cast<T*>(ws + off); };
  const int N = (int)a.N, C = (int)a.C;
  const int Np = (int)L.Np, Kp = (int)L.Kp;
  const int64_t cs = L.Np * L.Kp;
  ChannelProjectArgs pa{a.dtype, a.N, a.N, a.CZ, a.C, a.outgoing ? 0 : 1, a.z, a.mask,
                        a.ln_w, a.ln_b, a.eps, a.w_a, a.w_b, at(L.a), at(L.b),
                        cs, L.Kp, 1};
  hipError_t e = launch_channel_project(pa, s);
  if (e != hipSuccess) return e;
  ChannelProjectArgs pt = pa;
  pt.transposed = a.outgoing ? 1 : 0;
  pt.mask = nullptr;
  pt.a = at(L.at);
  pt.b = at(L.bt);
  if ((e = launch_channel_project(pt, s)) != hipSuccess) return e;
  // T_c (channel-major [C][N][N]) -> position rows
  if ((e = pair_gemm_t<T>(C, N, N, N, Np, Np, Kp, at(L.a), at(L.b), at(L.tm), false, s)) != hipSuccess)
    return e;
  if ((e = cm_to_pm<T>(at(L.tm), at(L.tpm), C, N, N, N, (int64_t)N * N, N, 0, nullptr, s)) !=
      hipSuccess)
    return e;
  // dT = dout . W_o, dW_o, db_o: the output projection's backward
  OutProjectBwdArgs ob{};
  ob.dtype = a.dtype; ob.N = a.N; ob.CZ = a.CZ; ob.H = a.C / kHeadDim; ob.ending = 0;
  ob.o = at(L.tpm); ob.w_o = a.w_o; ob.dout = a.dout; ob.d_o = at(L.dtpm);
  ob.dw_o = a.dw_o; ob.db_o = a.db_o; ob.workspace = ws + L.part;
  if ((e = launch_out_project_bwd(ob, s)) != hipSuccess) return e;
  if ((e = pm_to_cm<T>(at(L.dtpm), at(L.dtc), C, N, L.Np, L.Kp, 0, s)) != hipSuccess) return e;
  if ((e = pm_to_cm<T>(at(L.dtpm), at(L.dtt), C, N, L.Np, L.Kp, 1, s)) != hipSuccess) return e;
  // dA_c[i][k] = sum_j dT_c[i][j] B_c[j][k]; dB_c[j][k] = sum_i dT_c[i][j] A_c[i][k]
  T* dA = at(L.tm);
  T* dB = at(L.tpm);
  if ((e = pair_gemm_t<T>(C, N, N, N, Np, Np, Kp, at(L.dtc), at(L.bt), dA, false, s)) != hipSuccess)
    return e;
  if ((e = pair_gemm_t<T>(C, N, N, N, Np, Np, Kp, at(L.dtt), at(L.at), dB, false, s)) != hipSuccess)
    return e;
  // back to position rows (z order), masked third residues zeroed: A_c[i][k]
  // is the edge (i, k) outgoing, (k, i) incoming
  T* da = at(L.a);
  T* db = at(L.b);
  const int tr = a.outgoing ? 0 : 1;
  if ((e = cm_to_pm<T>(dA, da, C, N, N, N, (int64_t)N * N, N, tr, a.mask, s)) != hipSuccess)
    return e;
  if ((e = cm_to_pm<T>(dB, db, C, N, N, N, (int64_t)N * N, N, tr, a.mask, s)) != hipSuccess)
    return e;
  LnProjBwdArgs lb{};
  lb.dtype = a.dtype; lb.npos = a.N * a.N; lb.CZ = a.CZ; lb.nseg = 2; lb.seg_w = C;
  lb.dy[0] = da; lb.dy[1] = db; lb.w[0] = a.w_a; lb.w[1] = a.w_b;
  lb.z = a.z; lb.ln_w = a.ln_w; lb.ln_b = a.ln_b; lb.eps = a.eps;
  lb.dz = a.dz; lb.dw[0] = a.dw_a; lb.dw[1] = a.dw_b; lb.dln_w = a.dln_w; lb.dln_b = a.dln_b;
  lb.workspace = ws + L.part;
  return launch_ln_proj_bwd(lb, s);
}

}  // namespace

size_t trimul_workspace(int dtype, int64_t N, int64_t C) {
  return mul_layout(dtype, N, C).total;
}

hipError_t launch_trimul(const TriMulArgs& a, hipStream_t s) {
  return a.dtype == 1 ? trimul_t<bf16_t>(a, s) : trimul_t<float>(a, s);
}

size_t trimul_bwd_workspace(int dtype, int64_t N, int64_t CZ, int64_t C) {
  return mul_bwd_layout(dtype, N, CZ, C).total;
}

hipError_t launch_trimul_bwd(const TriMulBwdArgs& a, hipStream_t s) {
  return a.dtype == 1 ? trimul_bwd_t<bf16_t>(a, s) : trimul_bwd_t<float>(a, s);
}

int pair_gemm_row_tile() { return kRowPad; }

hipError_t launch_pair_gemm(int dtype, int C, int M, int K, int Np, int Kp, void* a, void* b,
                            void* t, bool a_frag, hipStream_t s) {
  return launch_pair_gemm_rect(dtype, C, M, M, K, Np, Np, Kp, a, b, t, a_frag, s);
}

hipError_t launch_pair_gemm_pairs(int M, int K, int Np, int Kp, void* a, void* b, void* pf,
                                  int N, int C, float scale, hipStream_t s) {
  if (Np % kRowPad != 0 || M > Np || K > Kp || Kp % MulCfg<bf16_t>::BK != 0 || C <= 0 ||
      C % 32 != 0 || (int64_t)N * C != M)
    return hipErrorInvalidValue;
  return pair_gemm_t<bf16_t>(1, M, M, K, Np, Np, Kp, static_cast<bf16_t*>(a),
                             static_cast<bf16_t*>(b), static_cast<bf16_t*>(pf), true, s, N, C,
                             scale);
}

hipError_t launch_pair_gemm_rect(int dtype, int C, int M, int M2, int K, int Np, int Np2, int Kp,
                                 void* a, void* b, void* t, bool a_frag, hipStream_t s) {
  if (Np % kRowPad != 0 || Np2 % kRowPad != 0 || M > Np || M2 > Np2 || K > Kp ||
      Kp % MulCfg<float>::BK != 0 || Kp % MulCfg<bf16_t>::BK != 0 ||
      (a_frag && (dtype != 1 || C != 1)))
    return hipErrorInvalidValue;
  return dtype == 1 ? pair_gemm_t<bf16_t>(C, M, M2, K, Np, Np2, Kp, static_cast<bf16_t*>(a),
                                          static_cast<bf16_t*>(b), static_cast<bf16_t*>(t),
                                          a_frag, s)
                    : pair_gemm_t<float>(C, M, M2, K, Np, Np2, Kp, static_cast<float*>(a),
                                         static_cast<float*>(b), static_cast<float*>(t), false,
                                         s);
}

hipError_t launch_cm_to_pm(int dtype, const void* src, void* dst, int C, int rows, int ncols,
                           int64_t ld, int64_t cs, int N, int trans, const uint8_t* keep,
                           hipStream_t s) {
  if (C % 32 != 0 || C > kMaxC) return hipErrorInvalidValue;
  return dtype == 1 ? cm_to_pm<bf16_t>(static_cast<const bf16_t*>(src), static_cast<bf16_t*>(dst),
                                       C, rows, ncols, ld, cs, N, trans, keep, s)
                    : cm_to_pm<float>(static_cast<const float*>(src), static_cast<float*>(dst),
                                      C, rows, ncols, ld, cs, N, trans, keep, s);
}

}  // namespace evo
