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

}  // namespace

size_t opm_workspace(int dtype, int64_t S, int64_t N, int64_t C) {
  return opm_layout(dtype, S, N, C).total;
}

hipError_t launch_opm(const OpmArgs& a, hipStream_t s) {
  return a.dtype == 1 ? opm_t<bf16_t>(a, s) : opm_t<float>(a, s);
}

}  // namespace evo
