// Outer product mean on gfx950.
//
// The MSA representation m [S, N, CM] updates the pair representation
// through the mean over the S sequences of the outer product of MSA columns
// i and j ("Evoformer: the memory wall ZeRO cannot move", section "The three
// operations").  The pages give no formula; the reading taken, with two
// c-channel projections of the layer-normalised MSA and an output
// projection to c_z:
//   x = LN(m),  a = x . W_a^T,  b = x . W_b^T                  (c channels)
//   o[i,j,c,d] = (1/S) sum_s a[s,i,c] b[s,j,d]
//   out[i,j] = flatten(o[i,j]) . W_o^T + b_o                (d fastest)
// Steps:
//   1. the persistent row GEMM (LayerNorm fused) reads m transposed, one
//      residue's S rows after another, and writes A[(i, c)][s] and
//      B[(j, d)][s] with rows padded to the GEMM tile;
//   2. the per-channel product kernel of the multiplicative update, with one
//      channel: P = A . B^T, P[(i, c)][(j, d)] = sum_s a[s,i,c] b[s,j,d],
//      a dense contraction over s on the matrix cores (rows padded to its
//      256-row tile);
//   3. opm_out: out[i, j] = W_o . P[(i, :)][(j, :)] / S + b_o.  For a
//      residue i and 64 consecutive j a wave's B operand for c*C + d0 .. +31
//      is one contiguous 1 KiB run of row i*C + c of P, loaded straight into
//      registers one chunk ahead; W_o is streamed through double-buffered
//      LDS in chunks of K.
#include <algorithm>

#include "evo_device.h"
#include "evo_kernels.h"

namespace evo {
namespace {

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct OpmOutParams {
  int N, C, M, jtiles;  // M = N * C (row length of P)
  const void* p;        // [M][M]
  const void* w_o;      // [CZ][C * C]
  const void* b_o;      // [CZ] or null
  float scale;          // 1 / S
  void* out;            // [N][N][CZ]
};

constexpr int kPairs = 256;  // pairs (i, j0 .. j0 + 255) per workgroup

template <typename T>
__device__ __forceinline__ void st4o(T* p, const f32x4& v);
template <>
__device__ __forceinline__ void st4o<bf16_t>(bf16_t* p, const f32x4& v) {
  uint2 u;
  u.x = uint32_t(Tr<bf16_t>::from_f(v[0])) | (uint32_t(Tr<bf16_t>::from_f(v[1])) << 16);
  u.y = uint32_t(Tr<bf16_t>::from_f(v[2])) | (uint32_t(Tr<bf16_t>::from_f(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}
template <>
__device__ __forceinline__ void st4o<float>(float* p, const f32x4& v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// One workgroup (4 waves) per residue i and 256 consecutive j; a wave owns 64
// pairs (4 blocks of 16) and all CZ = 16 CB output channels, computing
// out^T[cz][pair] = sum_k W_o[cz][k] P_i[pair][k] with k = c*C + d.
// C is a multiple of 32, so a K step of 32 stays inside one c.
template <typename T, int CB>
__global__ void __launch_bounds__(256) opm_out_kernel(OpmOutParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int CZ = CB * 16;
  constexpr int KC = sizeof(T) == 2 ? 64 : 32;  // K per W_o chunk
  constexpr int KPC = KC / 32;                  // K steps per chunk
  constexpr int WS = KC + 16 / (int)sizeof(T);  // LDS row stride: 144 bytes
  constexpr int E16 = 16 / sizeof(T);
  constexpr int CPR = KC / E16;           // 16-byte chunks per W_o row per chunk
  constexpr int WPT = CZ * CPR / 256;     // per thread
  static_assert(CZ * CPR % 256 == 0, "W_o chunk must split evenly over 256 threads");
  __shared__ __attribute__((aligned(16))) T sW[2][CZ * WS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int i = blockIdx.x / p.jtiles, jt = blockIdx.x - i * p.jtiles;
  const int C = p.C, K = C * C, nchunk = K / KC;
  const T* P = static_cast<const T*>(p.p);
  const T* Wg = static_cast<const T*>(p.w_o);

  // B-operand base of each pair block: row i*C of P, column j*C + 8g
  const T* pbase[4];
  int jpair[4];
#pragma unroll
  for (int pb = 0; pb < 4; ++pb) {
    jpair[pb] = jt * kPairs + wave * 64 + pb * 16 + l16;
    const int jc = min(jpair[pb], p.N - 1);
    pbase[pb] = P + (int64_t)i * C * p.M + (int64_t)jc * C + 8 * g;
  }
  // operands of K step k0 (a multiple of 32): row i*C + k0/C, columns + k0%C
  auto load_p = [&](Op (&v)[4], int k0) {
    const int c = k0 / C, d0 = k0 - c * C;
    const int64_t off = (int64_t)c * p.M + d0;
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) v[pb] = *reinterpret_cast<const Op*>(pbase[pb] + off);
  };
  u32x4 wr[WPT];
  auto fetch_w = [&](int k0) {
#pragma unroll
    for (int u = 0; u < WPT; ++u) {
      const int e = tid + 256 * u, row = e / CPR, col = (e % CPR) * E16;
      wr[u] = *reinterpret_cast<const u32x4*>(Wg + (int64_t)row * K + k0 + col);
    }
  };
  auto stage_w = [&](int buf) {
#pragma unroll
    for (int u = 0; u < WPT; ++u) {
      const int e = tid + 256 * u, row = e / CPR, col = (e % CPR) * E16;
      *reinterpret_cast<u32x4*>(&sW[buf][row * WS + col]) = wr[u];
    }
  };

  f32x4 acc[CB][4];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) acc[cb][pb] = f32x4{0.f, 0.f, 0.f, 0.f};

  Op pc[KPC][4], pn[KPC][4];
  fetch_w(0);
#pragma unroll
  for (int ks = 0; ks < KPC; ++ks) load_p(pc[ks], 32 * ks);
  stage_w(0);
  __syncthreads();
  for (int ch = 0; ch < nchunk; ++ch) {
    const int buf = ch & 1;
    // next chunk (the last one again at the end: loads stay in bounds and the
    // waits stay exact)
    const int nk0 = min(ch + 1, nchunk - 1) * KC;
    fetch_w(nk0);
#pragma unroll
    for (int ks = 0; ks < KPC; ++ks) load_p(pn[ks], nk0 + 32 * ks);
#pragma unroll
    for (int ks = 0; ks < KPC; ++ks) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const Op a = *reinterpret_cast<const Op*>(&sW[buf][(cb * 16 + l16) * WS + ks * 32 + 8 * g]);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) acc[cb][pb] = mma32(a, pc[ks][pb], acc[cb][pb]);
      }
    }
    stage_w(buf ^ 1);  // read in the previous chunk, whose barrier has passed
#pragma unroll
    for (int ks = 0; ks < KPC; ++ks)
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) pc[ks][pb] = pn[ks][pb];
    __syncthreads();
  }

  // lane (l16, g) holds out[i][j = pair block + l16][cb*16 + 4g + r]
  float bo[CB][4];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      bo[cb][r] = p.b_o ? Tr<T>::to_f(static_cast<const T*>(p.b_o)[cb * 16 + 4 * g + r]) : 0.f;
#pragma unroll
  for (int pb = 0; pb < 4; ++pb) {
    if (jpair[pb] >= p.N) continue;
    T* dst = static_cast<T*>(p.out) + ((int64_t)i * p.N + jpair[pb]) * CZ + 4 * g;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      f32x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = __builtin_fmaf(acc[cb][pb][r], p.scale, bo[cb][r]);
      st4o<T>(dst + cb * 16, v);
    }
  }
}

template <typename T, int CB>
hipError_t launch_opm_out(const OpmOutParams& o, hipStream_t s) {
  hipLaunchKernelGGL((opm_out_kernel<T, CB>), dim3(o.N * o.jtiles), dim3(256), 0, s, o);
  return hipGetLastError();
}

struct OpmLayout {
  int64_t M, Np, Kp;
  size_t a, b, p, total;
};
OpmLayout opm_layout(int dtype, int64_t S, int64_t N, int64_t C) {
  const size_t es = dtype == 1 ? 2 : 4;
  OpmLayout L;
  L.M = N * C;
  L.Np = round_up(L.M, pair_gemm_row_tile());
  L.Kp = round_up(S, 64);
  const size_t ab = ((size_t)L.Np * L.Kp * es + 255) & ~size_t(255);
  L.a = 0;
  L.b = ab;
  L.p = 2 * ab;
  L.total = L.p + (((size_t)L.M * L.M * es + 255) & ~size_t(255));
  return L;
}

template <typename T>
hipError_t opm_t(const OpmArgs& a, hipStream_t s) {
  const OpmLayout L = opm_layout(a.dtype, a.S, a.N, a.C);
  char* ws = static_cast<char*>(a.workspace);
  T* A = reinterpret_cast<T*>(ws + L.a);
  T* B = reinterpret_cast<T*>(ws + L.b);
  T* Pm = reinterpret_cast<T*>(ws + L.p);
  // lines = residues, places = sequences: m row s*N + i is read for position
  // i*S + s, and a[s, i, c] lands at A[(i*C + c)][s]
  // bf16: A in fragment order for the product kernel (rows i*C + c, columns s)
  ChannelProjectArgs pa{a.dtype, a.N, a.S, a.CM, a.C, 1, a.m, nullptr, a.ln_w, a.ln_b,
                        a.eps, a.w_a, a.w_b, A, B, L.Kp, a.C * L.Kp, 1,
                        a.dtype == 1 ? L.Kp : 0};
  hipError_t e = launch_channel_project(pa, s);
  if (e != hipSuccess) return e;
  e = launch_pair_gemm(a.dtype, 1, (int)L.M, (int)a.S, (int)L.Np, (int)L.Kp, A, B, Pm,
                       a.dtype == 1, s);
  if (e != hipSuccess) return e;
  OpmOutParams o{};
  o.N = (int)a.N;
  o.C = (int)a.C;
  o.M = (int)L.M;
  o.jtiles = (int)((a.N + kPairs - 1) / kPairs);
  o.p = Pm;
  o.w_o = a.w_o;
  o.b_o = a.b_o;
  o.scale = 1.f / (float)a.S;
  o.out = a.out;
  switch (a.CZ / 16) {
    case 2: return launch_opm_out<T, 2>(o, s);
    case 4: return launch_opm_out<T, 4>(o, s);
    case 6: return launch_opm_out<T, 6>(o, s);
    case 8: return launch_opm_out<T, 8>(o, s);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------- backward
// dP[(i, c)][(j, d)] = (1/S) (dout[i, j] . W_o)[c*C + d], written twice as
// the first operand of a product: dP (rows (i, c), columns (j, d)) and its
// transpose (rows (j, d), columns (i, c)), bf16 in fragment order
// (frag_off, row length kp), fp32 row-major at row stride kp.  A workgroup
// owns a slice of CS values of c and 32 of d (ROWS = 32 CS rows of W_o^T,
// resident in LDS) and walks tiles of 64 consecutive pairs p = i*N + j: 4
// waves of ROWS/4 rows x 64 pairs on the matrix cores (K = CZ), the tile
// through LDS, then 16-byte stores: 8 (bf16) or 4 (fp32) consecutive d of
// one (pair, c) for dP, the slice's consecutive c of one (pair, d) for the
// transpose.
// An operand fragment of 8 consecutive elements (bf16: 16 bytes, fp32: 32).
template <typename T>
__device__ __forceinline__ typename Tr<T>::Op ld_op8(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const bf16x8*>(p);
  } else {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    return f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  }
}

template <typename T> struct DpCfg;
template <> struct DpCfg<bf16_t> { static constexpr int CS = 8; };
template <> struct DpCfg<float> { static constexpr int CS = 4; };
constexpr int kDpPairs = 64;

struct OpmDpParams {
  int N, C, CZ, npairs, ntiles;
  int64_t kp;         // row length of the dP matrices
  const void* dout;   // [N*N][CZ]
  const void* w_o;    // [CZ][C*C]
  float scale;        // 1 / S
  void* dp;
  void* dpt;
};

template <typename T>
__device__ __forceinline__ int64_t dp_off(int64_t r, int64_t k, int64_t kp) {
  if constexpr (sizeof(T) == 2) return frag_off(r, (int)k, (int)kp);
  else return r * kp + k;
}

template <typename T, int KS>  // KS = c_z / 32
__global__ void __launch_bounds__(256) opm_dp_kernel(OpmDpParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int CS = DpCfg<T>::CS, ROWS = 32 * CS, RPW = ROWS / 4, RB = RPW / 16;
  constexpr int E = 16 / sizeof(T);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int WS = p.CZ + 16 / (int)sizeof(T);
  constexpr int OS = ROWS + 16 / (int)sizeof(T);
  T* sW = reinterpret_cast<T*>(smem);                 // [ROWS][CZ + pad]: W_o^T slice
  T* sO = sW + ROWS * WS;                             // [64 pairs][ROWS + pad]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int C = p.C, nd = C / 32;
  const int slice = blockIdx.y;
  const int c0 = (slice / nd) * CS, d0 = (slice % nd) * 32;
  const T* Wg = static_cast<const T*>(p.w_o);
  // slice row q = cl*32 + dl  <->  W_o column (c0 + cl)*C + d0 + dl
  for (int e = tid; e < ROWS * p.CZ; e += 256) {
    const int q = e / p.CZ, o = e - q * p.CZ;
    sW[q * WS + o] = Wg[(int64_t)o * C * C + (int64_t)(c0 + q / 32) * C + d0 + (q & 31)];
  }
  __syncthreads();
  const T* D = static_cast<const T*>(p.dout);
  T* dP = static_cast<T*>(p.dp);
  T* dPt = static_cast<T*>(p.dpt);
  // A tile's dout operands: 4 blocks of 16 pairs, c_z in 32-wide steps.
  // The next tile's are loaded while the current one is computed, staged
  // and stored (after the last tile: the last tile again, in bounds).
  auto load_b = [&](Op (&b)[KS][4], int tile) {
    const int p0 = tile * kDpPairs;
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      const int pr = min(p0 + pb * 16 + l16, p.npairs - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) b[ks][pb] = ld_op8<T>(D + (int64_t)pr * (32 * KS) + 32 * ks + 8 * g);
    }
  };
  Op bn[KS][4];
  load_b(bn, min((int)blockIdx.x, p.ntiles - 1));
  for (int tile = blockIdx.x; tile < p.ntiles; tile += gridDim.x) {
    const int p0 = tile * kDpPairs;
    Op bc[KS][4];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) bc[ks][pb] = bn[ks][pb];
    load_b(bn, min(tile + (int)gridDim.x, p.ntiles - 1));
    f32x4 acc[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) acc[rb][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const Op a = ld_op8<T>(sW + (wave * RPW + rb * 16 + l16) * WS + 32 * ks + 8 * g);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) acc[rb][pb] = mma32(a, bc[ks][pb], acc[rb][pb]);
      }
    }
    __syncthreads();  // the previous tile's stores have read sO
    // lane (l16, g): rows wave*RPW + rb*16 + 4g + i of pair pb*16 + l16
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int pb = 0; pb < 4; ++pb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sO[(pb * 16 + l16) * OS + wave * RPW + rb * 16 + 4 * g + i] =
              Tr<T>::from_f(acc[rb][pb][i] * p.scale);
    __syncthreads();
    // dP: (pair, c, E consecutive d) per unit
    constexpr int UPC = 32 / E;  // units per (pair, c)
    for (int u = tid; u < kDpPairs * CS * UPC; u += 256) {
      const int pl = u / (CS * UPC), rem = u - pl * (CS * UPC);
      const int cl = rem / UPC, dl = (rem - cl * UPC) * E;
      const int pr = p0 + pl;
      if (pr >= p.npairs) continue;
      const int i = pr / p.N, j = pr - i * p.N;
      const int64_t r = (int64_t)i * C + c0 + cl, k = (int64_t)j * C + d0 + dl;
      *reinterpret_cast<u32x4*>(dP + dp_off<T>(r, k, p.kp)) =
          *reinterpret_cast<const u32x4*>(sO + pl * OS + cl * 32 + dl);
    }
    // transpose: (pair, d) per unit, the slice's CS consecutive c
    for (int u = tid; u < kDpPairs * 32; u += 256) {
      const int pl = u >> 5, dl = u & 31;
      const int pr = p0 + pl;
      if (pr >= p.npairs) continue;
      const int i = pr / p.N, j = pr - i * p.N;
      T v[E];
#pragma unroll
      for (int q = 0; q < E; ++q) v[q] = sO[pl * OS + q * 32 + dl];
      const int64_t r = (int64_t)j * C + d0 + dl, k = (int64_t)i * C + c0;
      u32x4 w;
      __builtin_memcpy(&w, v, 16);
      *reinterpret_cast<u32x4*>(dPt + dp_off<T>(r, k, p.kp)) = w;
    }
  }
}

// P[(i, c)][(j, d)] -> rows of pairs: Pf[(i*N + j)][c*C + d] = P * scale.
// One thread per 8 consecutive d (C is a multiple of 32, so they stay in one
// pair): one 16- (bf16) or 32-byte (fp32) read and write.
template <typename T>
__global__ void __launch_bounds__(256) opm_pair_rows_kernel(const T* P, T* Pf, int N, int C,
                                                            float scale) {
  const int64_t M = (int64_t)N * C;
  const int64_t total = M * M / 8;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / (M / 8), k = (e - r * (M / 8)) * 8;
    const int64_t i = r / C, c = r - i * C, j = k / C, d = k - j * C;
    T v[8];
    __builtin_memcpy(v, P + r * M + k, sizeof(v));
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = Tr<T>::from_f(Tr<T>::to_f(v[q]) * scale);
    __builtin_memcpy(Pf + ((i * N + j) * C + c) * C + d, v, sizeof(v));
  }
}

struct OpmBwdLayout {
  int64_t M, Np, Kp, Np2, Kp2;
  size_t a, b, ya, yb, p, pf, da, db, dapm, dbpm, part, total;
};
OpmBwdLayout opm_bwd_layout(int dtype, int64_t S, int64_t N, int64_t CM, int64_t C,
                            int64_t CZ) {
  const size_t es = dtype == 1 ? 2 : 4;
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  OpmBwdLayout L;
  L.M = N * C;
  L.Np = round_up(L.M, pair_gemm_row_tile());
  L.Kp = round_up(S, 64);
  L.Np2 = round_up(S, pair_gemm_row_tile());
  L.Kp2 = round_up(L.M, 64);
  const size_t ab = al((size_t)L.Np * L.Kp * es), yy = al((size_t)L.Np2 * L.Kp2 * es);
  const size_t pp = al(std::max((size_t)L.M * L.M, (size_t)L.Np * L.Kp2) * es);
  const size_t dd = al((size_t)L.M * S * es);
  L.a = 0;
  L.b = L.a + ab;
  L.ya = L.b + ab;
  L.yb = L.ya + yy;
  L.p = L.yb + yy;     // P, then dP
  L.pf = L.p + pp;     // pair rows of P, then dP^T
  L.da = L.pf + pp;
  L.db = L.da + dd;
  L.dapm = L.db + dd;
  L.dbpm = L.dapm + dd;
  L.part = L.dbpm + dd;
  L.total = L.part + al(std::max(col_wgrad_workspace(N * N, 256),
                                 ln_proj_bwd_workspace(S * N, CM, (int)C)));
  return L;
}

// Backward of the outer product mean: the chain rule of the forward,
//   dP = dout . W_o / S (per pair, the C x C block),  dW_o = sum dout^T P / S,
//   dA = dP . B  (rows (i, c), columns s),  dB = dP^T . A,
//   then the LayerNorm + projection backward of m from da, db.
// Steps: the forward's operands A, B and the product P recomputed as pair
// rows scaled by 1/S (bf16: written so by the product's epilogue; fp32: a
// separate pass) for dW_o, db_o (column weight-gradient reduction, 256
// columns of W_o at a time); the same projections written with sequences as
// rows (Y_a[s][(i, c)] = a[s, i, c], likewise Y_b) as the second operands;
// dP and dP^T (opm_dp_kernel); the two products dA = dP . Y_b^T and
// dB = dP^T . Y_a^T (rectangular: N*C rows by S columns); dA, dB to rows
// (s, i); the two-segment LayerNorm + projection backward.
template <typename T>
hipError_t opm_bwd_t(const OpmBwdArgs& a, hipStream_t s) {
  const OpmBwdLayout L = opm_bwd_layout(a.dtype, a.S, a.N, a.CM, a.C, a.CZ);
  char* ws = static_cast<char*>(a.workspace);
  auto at = [&](size_t off) { return reinterpret_cast<T*>(ws + off); };
  const int S = (int)a.S, N = (int)a.N, C = (int)a.C, CZ = (int)a.CZ;
  const int M = (int)L.M;
  const bool bf = a.dtype == 1;
  ChannelProjectArgs pa{a.dtype, a.N, a.S, a.CM, a.C, 1, a.m, nullptr, a.ln_w, a.ln_b,
                        a.eps, a.w_a, a.w_b, at(L.a), at(L.b), L.Kp, a.C * L.Kp, 1,
                        bf ? L.Kp : 0};
  hipError_t e = launch_channel_project(pa, s);
  if (e != hipSuccess) return e;
  if (bf) {
    // bf16: the product's epilogue writes the pair rows directly
    if ((e = launch_pair_gemm_pairs(M, S, (int)L.Np, (int)L.Kp, at(L.a), at(L.b), at(L.pf), N, C,
                                    1.f / (float)S, s)) != hipSuccess)
      return e;
  } else {
    if ((e = launch_pair_gemm(a.dtype, 1, M, S, (int)L.Np, (int)L.Kp, at(L.a), at(L.b), at(L.p),
                              false, s)) != hipSuccess)
      return e;
    const int64_t total = (int64_t)M * M / 8;
    const int grid = (int)std::min<int64_t>((total + 255) / 256, 16384);
    hipLaunchKernelGGL(opm_pair_rows_kernel<T>, dim3(grid), dim3(256), 0, s, at(L.p), at(L.pf),
                       N, C, 1.f / (float)S);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // dW_o[o][c*C + d] = sum over pairs of dout[pair][o] Pf[pair][c*C + d]
  for (int q = 0; q < C * C; q += 256) {
    ColWGradArgs cw{};
    cw.dtype = a.dtype; cw.npos = (int64_t)N * N;
    cw.a = a.dout; cw.a_w = CZ;
    cw.b = at(L.pf) + q; cw.b_w = 256; cw.b_ld = (int64_t)C * C;
    cw.dw = a.dw_o + q; cw.dw_ld = (int64_t)C * C;
    cw.dcol = q == 0 ? a.db_o : nullptr;
    cw.workspace = ws + L.part;
    if ((e = launch_col_wgrad(cw, s)) != hipSuccess) return e;
  }
  // Y_a[s][(i, c)] = a[s, i, c], Y_b likewise: lines = sequences
  ChannelProjectArgs py{a.dtype, a.S, a.N, a.CM, a.C, 0, a.m, nullptr, a.ln_w, a.ln_b,
                        a.eps, a.w_a, a.w_b, at(L.ya), at(L.yb), 1, L.Kp2, a.C, 0};
  if ((e = launch_channel_project(py, s)) != hipSuccess) return e;
  OpmDpParams d{};
  d.N = N; d.C = C; d.CZ = CZ; d.npairs = N * N;
  d.ntiles = (d.npairs + kDpPairs - 1) / kDpPairs;
  d.kp = L.Kp2; d.dout = a.dout; d.w_o = a.w_o; d.scale = 1.f / (float)S;
  d.dp = at(L.p); d.dpt = at(L.pf);
  {
    constexpr int ROWS = 32 * DpCfg<T>::CS;
    const size_t lds = ((size_t)ROWS * (CZ + 16 / sizeof(T)) +
                        (size_t)kDpPairs * (ROWS + 16 / sizeof(T))) * sizeof(T);
    const int slices = (C / DpCfg<T>::CS) * (C / 32);
    const int gx = std::max(1, std::min(d.ntiles, 1024 / slices));
    auto launch_dp = [&](auto kernel) {
      hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e2 != hipSuccess) return e2;
      hipLaunchKernelGGL(kernel, dim3(gx, slices), dim3(256), lds, s, d);
      return hipGetLastError();
    };
    switch (CZ / 32) {
      case 1: e = launch_dp(&opm_dp_kernel<T, 1>); break;
      case 2: e = launch_dp(&opm_dp_kernel<T, 2>); break;
      case 3: e = launch_dp(&opm_dp_kernel<T, 3>); break;
      case 4: e = launch_dp(&opm_dp_kernel<T, 4>); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  // dA[(i, c)][s] = sum_(j, d) dP[(i, c)][(j, d)] Y_b[s][(j, d)]; dB likewise
  if ((e = launch_pair_gemm_rect(a.dtype, 1, M, S, M, (int)L.Np, (int)L.Np2, (int)L.Kp2, at(L.p),
                                 at(L.yb), at(L.da), bf, s)) != hipSuccess)
    return e;
  if ((e = launch_pair_gemm_rect(a.dtype, 1, M, S, M, (int)L.Np, (int)L.Np2, (int)L.Kp2,
                                 at(L.pf), at(L.ya), at(L.db), bf, s)) != hipSuccess)
    return e;
  // rows (i*C + c), columns s -> position rows (s*N + i), C channels
  if ((e = launch_cm_to_pm(a.dtype, at(L.da), at(L.dapm), C, N, S, (int64_t)C * S, S, N, 1,
                           nullptr, s)) != hipSuccess)
    return e;
  if ((e = launch_cm_to_pm(a.dtype, at(L.db), at(L.dbpm), C, N, S, (int64_t)C * S, S, N, 1,
                           nullptr, s)) != hipSuccess)
    return e;
  LnProjBwdArgs lb{};
  lb.dtype = a.dtype; lb.npos = a.S * a.N; lb.CZ = a.CM; lb.nseg = 2; lb.seg_w = C;
  lb.dy[0] = at(L.dapm); lb.dy[1] = at(L.dbpm); lb.w[0] = a.w_a; lb.w[1] = a.w_b;
  lb.z = a.m; lb.ln_w = a.ln_w; lb.ln_b = a.ln_b; lb.eps = a.eps;
  lb.dz = a.dm; lb.dw[0] = a.dw_a; lb.dw[1] = a.dw_b; lb.dln_w = a.dln_w; lb.dln_b = a.dln_b;
  lb.workspace = ws + L.part;
  return launch_ln_proj_bwd(lb, s);
}

}  // namespace

size_t opm_workspace(int dtype, int64_t S, int64_t N, int64_t C) {
  return opm_layout(dtype, S, N, C).total;
}

hipError_t launch_opm(const OpmArgs& a, hipStream_t s) {
  return a.dtype == 1 ? opm_t<bf16_t>(a, s) : opm_t<float>(a, s);
}

size_t opm_bwd_workspace(int dtype, int64_t S, int64_t N, int64_t CM, int64_t C, int64_t CZ) {
  return opm_bwd_layout(dtype, S, N, CM, C, CZ).total;
}

hipError_t launch_opm_bwd(const OpmBwdArgs& a, hipStream_t s) {
  return a.dtype == 1 ? opm_bwd_t<bf16_t>(a, s) : opm_bwd_t<float>(a, s);
}

}  // namespace evo
