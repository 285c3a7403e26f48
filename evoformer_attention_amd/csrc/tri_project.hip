// Triangle-attention module projections on gfx950.
//
// tri_attn_project: LayerNorm of each pair-representation row z[i,j,:]
// (fp32 statistics) fused with the Q/K/V/gate/pair-bias projections, so the
// normalised N x N x CZ tensor is never written to HBM (the fusion EvoFusion
// targets in "MegaFold: Efficient Training of Next-Generation 3D Attention
// Protein Models on Cross-Platform GPUs", section "Methodologie", item 3).
// tri_attn_out_project: the output projection back to CZ channels, written
// in z layout.
//
// Both are a row GEMM  Y[pos, :] = f(X[pos, :]) . W  over the N*N positions
// of a line-layout tile: a workgroup takes TP consecutive positions, builds
// f(X) for them in LDS once, then streams the weight matrix through LDS in
// chunks of 64 output columns (transposed on the way in, so both MFMA
// operands are contiguous 16-byte LDS reads).  Outputs are produced as
// Y^T = W^T . f(X)^T so each lane holds 4 consecutive output channels of one
// position, written as one 8- or 16-byte store.
//
// Orientation: position (line a, place n) of the line layout is z[a, n] for
// the starting node and z[n, a] for the ending node (line = a column of z).
// The pair bias of position (a, n) goes to bias[h][a*N + n] in both cases.
#include "evo_device.h"
#include "evo_kernels.h"

namespace evo {
namespace {

constexpr int COLS = 64;   // output columns per weight chunk
constexpr int PAD = 8;     // LDS row padding (elements)

template <typename T> struct GemmCfg;
template <> struct GemmCfg<bf16_t> { static constexpr int PB = 2; };  // 128 positions
template <> struct GemmCfg<float> { static constexpr int PB = 1; };   // 64 positions

struct GemmParams {
  int mode;        // 0 = project (LayerNorm + 5 outputs), 1 = out projection
  int N, K, HC, H, ending, ncols, total_tiles;
  int64_t npos;
  const void* x;   // z [N,N,K] (project) or O [N*N, K] (out projection)
  const void* ln_w;
  const void* ln_b;
  float eps;
  const void* w[5];     // project: w_q, w_k, w_v, w_g [K,HC], w_bias [K,H]
                        // out projection: w_o [K, ncols]
  const void* colbias;  // project: b_g [HC] (gate columns); out: b_o [ncols]
  void* y[5];           // project: q, k, v, g [npos, HC], bias [H, npos]
                        // out projection: out [npos, ncols] in z layout
};

// Source/destination row of z for line-layout position pidx.
__device__ __forceinline__ int64_t z_row(int64_t pidx, int N, int ending) {
  if (!ending) return pidx;
  const int64_t a = pidx / N, n = pidx - a * N;
  return n * N + a;
}

// Weight element W(k, col) of the concatenated column space.
template <typename T>
__device__ __forceinline__ T w_elem(const GemmParams& p, int k, int col) {
  if (col >= p.ncols) return T(0);
  if (p.mode == 1) return static_cast<const T*>(p.w[0])[(int64_t)k * p.ncols + col];
  const int m = col / p.HC;
  if (m < 4) return static_cast<const T*>(p.w[m])[(int64_t)k * p.HC + (col - m * p.HC)];
  return static_cast<const T*>(p.w[4])[(int64_t)k * p.H + (col - 4 * p.HC)];
}

template <typename T>
__global__ void __launch_bounds__(256)
rowgemm_kernel(GemmParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int PB = GemmCfg<T>::PB;
  constexpr int TP = 4 * 16 * PB;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int K = p.K, KS = K + PAD;
  T* sX = reinterpret_cast<T*>(smem);        // [TP][KS]
  T* sW = sX + TP * KS;                      // [COLS][KS]  (W^T chunk)

  const int tile = xcd_work_index(p.total_tiles);
  if (tile < 0) return;
  const int64_t pos0 = (int64_t)tile * TP;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const T* X = static_cast<const T*>(p.x);

  // ---- f(X) tile: 16 lanes per position, K/16 consecutive elements each.
  {
    const int span = K / 16;
    const int sub = lane >> 4;              // position within the quad
    for (int pp = wave * 4 + sub; pp < TP; pp += 16) {
      const int64_t pidx = pos0 + pp;
      float vals[16];
      const bool live = pidx < p.npos;
      const int64_t row = live ? (p.mode == 0 ? z_row(pidx, p.N, p.ending) : pidx) : 0;
      const T* src = X + row * K + l16 * span;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        vals[j] = (j < span && live) ? Tr<T>::to_f(src[j]) : 0.f;
      if (p.mode == 0) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) s += vals[j];
        s += __shfl_xor(s, 1, 64); s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 4, 64); s += __shfl_xor(s, 8, 64);
        const float mu = s / K;
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float d = (j < span) ? vals[j] - mu : 0.f;
          v += d * d;
        }
        v += __shfl_xor(v, 1, 64); v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 4, 64); v += __shfl_xor(v, 8, 64);
        const float rstd = rsqrtf(v / K + p.eps);
        const T* lw = static_cast<const T*>(p.ln_w) + l16 * span;
        const T* lb = static_cast<const T*>(p.ln_b) + l16 * span;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (j < span)
            vals[j] = live ? (vals[j] - mu) * rstd * Tr<T>::to_f(lw[j]) +
                                 Tr<T>::to_f(lb[j])
                           : 0.f;
      }
      T* dst = sX + pp * KS + l16 * span;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j < span) dst[j] = Tr<T>::from_f(vals[j]);
    }
  }

  for (int c0 = 0; c0 < p.ncols; c0 += COLS) {
    __syncthreads();  // sX ready / previous chunk consumed
    // ---- W^T chunk: sW[col][k] = W(k, c0 + col)
    for (int e = tid; e < COLS * K; e += 256) {
      const int col = e / K, k = e - col * K;
      sW[col * KS + k] = w_elem<T>(p, k, c0 + col);
    }
    __syncthreads();

    f32x4 acc[4][PB];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) acc[cb][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const T* xw = sX + (wave * 16 * PB) * KS;
    for (int k0 = 0; k0 < K; k0 += 32) {
      Op a[4], bx[PB];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        a[cb] = *reinterpret_cast<const Op*>(sW + (cb * 16 + l16) * KS + k0 + 8 * g);
#pragma unroll
      for (int pb = 0; pb < PB; ++pb)
        bx[pb] = *reinterpret_cast<const Op*>(xw + (pb * 16 + l16) * KS + k0 + 8 * g);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) acc[cb][pb] = mma32(a[cb], bx[pb], acc[cb][pb]);
    }

    // ---- epilogue: lane holds channels col..col+3 of position pidx
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      const int64_t pidx = pos0 + wave * 16 * PB + pb * 16 + l16;
      if (pidx >= p.npos) continue;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int col = c0 + cb * 16 + 4 * g;
        if (col >= p.ncols) continue;
        f32x4 val = acc[cb][pb];
        if (p.mode == 1) {
          if (p.colbias) {
            const T* cbp = static_cast<const T*>(p.colbias) + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) val[i] += Tr<T>::to_f(cbp[i]);
          }
          T* dst = static_cast<T*>(p.y[0]) + z_row(pidx, p.N, p.ending) * p.ncols + col;
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[i] = Tr<T>::from_f(val[i]);
        } else {
          const int m = col / p.HC;
          if (m < 4) {
            const int cc = col - m * p.HC;
            if (m == 3 && p.colbias) {
              const T* cbp = static_cast<const T*>(p.colbias) + cc;
#pragma unroll
              for (int i = 0; i < 4; ++i) val[i] += Tr<T>::to_f(cbp[i]);
            }
            T* dst = static_cast<T*>(p.y[m]) + pidx * p.HC + cc;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = Tr<T>::from_f(val[i]);
          } else {
            T* bias = static_cast<T*>(p.y[4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int hh = col - 4 * p.HC + i;
              if (hh < p.H) bias[(int64_t)hh * p.npos + pidx] = Tr<T>::from_f(val[i]);
            }
          }
        }
      }
    }
  }
}

template <typename T>
hipError_t launch_gemm(GemmParams& p, hipStream_t s) {
  constexpr int TP = 4 * 16 * GemmCfg<T>::PB;
  const int64_t tiles = (p.npos + TP - 1) / TP;
  if (tiles > (int64_t)INT32_MAX - 8) return hipErrorInvalidValue;
  p.total_tiles = (int)tiles;
  const int grid = ((p.total_tiles + kNumXcd - 1) / kNumXcd) * kNumXcd;
  const size_t lds = (size_t)(TP + COLS) * (p.K + PAD) * sizeof(T);
  hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&rowgemm_kernel<T>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rowgemm_kernel<T>, dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

hipError_t dispatch(int dtype, GemmParams& p, hipStream_t s) {
  return dtype == 1 ? launch_gemm<bf16_t>(p, s) : launch_gemm<float>(p, s);
}

}  // namespace

hipError_t launch_project(const ProjectArgs& a, hipStream_t s) {
  GemmParams p{};
  p.mode = 0;
  p.N = (int)a.N;
  p.K = (int)a.CZ;
  p.H = (int)a.H;
  p.HC = (int)(a.H * kHeadDim);
  p.ending = a.ending;
  p.ncols = 4 * p.HC + p.H;
  p.npos = a.N * a.N;
  p.x = a.z;
  p.ln_w = a.ln_w;
  p.ln_b = a.ln_b;
  p.eps = a.eps;
  p.w[0] = a.w_q; p.w[1] = a.w_k; p.w[2] = a.w_v; p.w[3] = a.w_g;
  p.w[4] = a.w_bias;
  p.colbias = a.b_g;
  p.y[0] = a.q; p.y[1] = a.k; p.y[2] = a.v; p.y[3] = a.g; p.y[4] = a.bias;
  return dispatch(a.dtype, p, s);
}

hipError_t launch_out_project(const OutProjectArgs& a, hipStream_t s) {
  GemmParams p{};
  p.mode = 1;
  p.N = (int)a.N;
  p.K = (int)(a.H * kHeadDim);
  p.H = (int)a.H;
  p.HC = p.K;
  p.ending = a.ending;
  p.ncols = (int)a.CZ;
  p.npos = a.N * a.N;
  p.x = a.o;
  p.w[0] = a.w_o;
  p.colbias = a.b_o;
  p.y[0] = a.out;
  return dispatch(a.dtype, p, s);
}

}  // namespace evo
