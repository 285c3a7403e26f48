// Backward of the triangle-attention module's projections on gfx950.
//
// The forward ("MegaFold: Efficient Training of Next-Generation 3D Attention
// Protein Models on Cross-Platform GPUs", section "Methodologie", item 3,
// EvoFusion: LayerNorm fused with the linear projections that follow it) is
//   x = LN(z) = xhat * gamma + beta,   y_m = x . W_m^T (+ b_m),
// and its backward is the chain rule of that definition:
//   dX[pos]    = sum_m dY_m[pos] . W_m                      (row GEMM)
//   dz[pos]    = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat)),
//                dxhat = dX * gamma                         (fused, per position)
//   dW_m       = sum_pos dY_m[pos]^T x[pos]                 (weight GEMM)
//   dgamma[c]  = sum_pos dX[pos, c] xhat[pos, c],  dbeta[c] = sum_pos dX[pos, c].
// The weight GEMM contracts over the N*N positions against xhat (not x):
// with M = sum_pos dY^T xhat and the column sums s = sum_pos dY,
//   dW[k, c]   = gamma[c] M[k, c] + beta[c] s[k]
//   dgamma[c]  = sum_k W[k, c] M[k, c],   dbeta[c] = sum_k W[k, c] s[k]
// (exact rearrangements of the sums above), so dgamma and dbeta need no
// reduction over positions of their own and dX never leaves the chip.
//
// Kernels.
//   rowgrad   dX = [dY_0 | dY_1 | ... | dBias] . W_ext^T for 32 positions per
//             wave: the extended weight (the W_m stacked along the
//             contraction, the pair-bias projection last) sits in LDS with its
//             output channels permuted so that the accumulators come out with
//             8 consecutive channels per lane; optionally the LayerNorm
//             backward follows in registers and dz is written, else dX is.
//             The pair-bias gradient (fp32) enters as a bf16 high part plus a
//             bf16 low part, each against its own copy of the weight row.
//   wgrad     per (row tile, chunk of positions): M += A^T B over 32-position
//             steps staged in LDS (bf16: row-major, read with transposing LDS
//             reads; fp32: stored transposed), B = xhat recomputed from z
//             (LayerNorm statistics per position) or a plain activation; the
//             column sums of A come from the staging registers.  Partials per
//             chunk, no atomics.
//   finish    sums the chunk partials in a fixed order and applies the
//             LayerNorm affine; lnparam reduces dgamma and dbeta.
// Everything is deterministic.
#include <algorithm>

#include "evo_device.h"
#include "evo_kernels.h"

namespace evo {
namespace {

constexpr int PW = 32;                 // positions per wave (rowgrad), per step (wgrad)
constexpr int PADE = 8;                // LDS row padding (elements)
constexpr size_t kLdsBudget = 150 * 1024;
constexpr int kMaxSeg = 4;

// z row of line-layout position pidx: z[a, n] (starting node) or z[n, a]
// (ending node) for line a, place n.  N*N < 2^31.
__device__ __forceinline__ uint32_t zrow_of(uint32_t pidx, uint32_t N, int ending) {
  if (!ending) return pidx;
  const uint32_t a = pidx / N, n = pidx - a * N;
  return n * N + a;
}

// Eight consecutive elements (16-byte aligned) as fp32.
__device__ __forceinline__ void ld8f(const bf16_t* p, float (&v)[8]) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void ld8f(const float* p, float (&v)[8]) {
  const u32x4 a = reinterpret_cast<const u32x4*>(p)[0];
  const u32x4 b = reinterpret_cast<const u32x4*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = __uint_as_float(a[i]);
    v[4 + i] = __uint_as_float(b[i]);
  }
}
__device__ __forceinline__ void st8f(bf16_t* p, const float (&v)[8]) {
  u32x4 u;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    u[i] = uint32_t(Tr<bf16_t>::from_f(v[2 * i])) |
           (uint32_t(Tr<bf16_t>::from_f(v[2 * i + 1])) << 16);
  *reinterpret_cast<u32x4*>(p) = u;
}
__device__ __forceinline__ void st8f(float* p, const float (&v)[8]) {
  reinterpret_cast<u32x4*>(p)[0] =
      u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
            __float_as_uint(v[3])};
  reinterpret_cast<u32x4*>(p)[1] =
      u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
            __float_as_uint(v[7])};
}
__device__ __forceinline__ bf16x8 to_op(const float (&v)[8], bf16x8*) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)v[j];
  return r;
}
__device__ __forceinline__ f32x8 to_op(const float (&v)[8], f32x8*) {
  f32x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = v[j];
  return r;
}
template <typename T>
__device__ __forceinline__ typename Tr<T>::Op ld_op(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const bf16x8*>(p);
  } else {
    float v[8];
    ld8f(p, v);
    return to_op(v, (f32x8*)nullptr);
  }
}

// ------------------------------------------------------------------ rowgrad
struct RowGradParams {
  int N, ending, npos, ntiles;
  int nseg, seg_w, in_zrow;     // input segments [npos][seg_w], addressed by
                                // z row (in_zrow) or line position
  const void* seg[kMaxSeg];
  const float* dbias;           // [H][npos] line layout, or null
  int H;
  int Kext;                     // nseg*seg_w (+32 with dbias)
  const void* wseg[kMaxSeg];    // [seg_w][cout]: W_ext[k][c] of segment s
  const void* wbias;            // [H][cout]
  int cout, kc, resident;       // output channels; LDS columns (all of W_ext
                                // when resident, else one segment at a time)
  int ln;                       // LayerNorm backward: write dz at z rows
  const void* z;                // [npos][cout] z layout (ln)
  const void* ln_w;
  float eps;
  void* y;                      // ln ? dz (z layout) : dX (line layout), [npos][cout]
};

// LDS row of output channel c: accumulator block cb = 2*(c/32) + (c%8)/4,
// row 4*((c%32)/8) + c%4 inside it, so that lane group g of block pair
// (2s, 2s+1) holds channels 32s + 8g .. +7.
__device__ __forceinline__ int wrow_of(int c) {
  const int s = c >> 5, rem = c & 31, gg = rem >> 3, j = rem & 7;
  return 16 * (2 * s + (j >> 2)) + 4 * gg + (j & 3);
}

template <typename T, int CB, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) rowgrad_kernel(RowGradParams p) {
  using Op = typename Tr<T>::Op;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sW = reinterpret_cast<T*>(smem);  // [cout][kc + PADE]
  const int KCS = p.kc + PADE;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int cout = p.cout;  // 16 * CB
  const int segK = p.nseg * p.seg_w;

  // W_ext columns [k0, k0 + kn) into LDS (channel-permuted rows).
  auto load_w = [&](int k0, int kn) {
    const int total = cout * kn;
    for (int e = tid; e < total; e += WAVES * 64) {
      const int kk = e / cout, c = e - kk * cout;
      const int k = k0 + kk;
      float w = 0.f;
      if (k < segK) {
        const int s = k / p.seg_w;
        w = Tr<T>::to_f(static_cast<const T*>(p.wseg[s])[(int64_t)(k - s * p.seg_w) * cout + c]);
      } else {
        const int slot = k - segK;  // slot h: high part of dBias[h]; H + h: low part
        if (slot < 2 * p.H)
          w = Tr<T>::to_f(static_cast<const T*>(p.wbias)[(int64_t)(slot % p.H) * cout + c]);
      }
      sW[wrow_of(c) * KCS + kk] = Tr<T>::from_f(w);  // exact: w is a T value
    }
  };
  if (p.resident) {
    load_w(0, p.Kext);
    __syncthreads();
  }

  const int seg_steps = p.seg_w / 32;  // 1..4
  for (int tile = blockIdx.x; tile < p.ntiles; tile += gridDim.x) {
    uint32_t pc[2], inrow[2];
    bool live[2];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      const uint32_t pidx = ((uint32_t)tile * WAVES + wave) * PW + pb * 16 + l16;
      live[pb] = pidx < (uint32_t)p.npos;
      pc[pb] = live[pb] ? pidx : 0u;  // past the end: position 0 (finite, not stored)
      inrow[pb] = p.in_zrow ? zrow_of(pc[pb], p.N, p.ending) : pc[pb];
    }
    f32x4 acc[CB][2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb][0] = acc[cb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K step ks of the LDS-resident columns starting at column kb: acc +=
    // W_ext[:, kb + 32ks ..] . x^T for both position blocks.
    auto mma_step = [&](int kb, const Op (&x)[2]) {
      const T* wr = sW + kb + 8 * g;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const Op a = ld_op<T>(wr + (cb * 16 + l16) * KCS);
        acc[cb][0] = mma32(a, x[0], acc[cb][0]);
        acc[cb][1] = mma32(a, x[1], acc[cb][1]);
      }
    };
    // One segment at a time (an LDS chunk when the weight is not resident):
    // the lane's 8 consecutive contraction values 32*ks + 8g .. +7 of its
    // position, all steps of the segment loaded before the first product.
    for (int s = 0; s < p.nseg; ++s) {
      if (!p.resident) {
        __syncthreads();  // every wave is done with the previous chunk
        load_w(s * p.seg_w, p.seg_w);
        __syncthreads();
      }
      const int kb = p.resident ? s * p.seg_w : 0;
      const T* src0 = static_cast<const T*>(p.seg[s]) + (int64_t)inrow[0] * p.seg_w + 8 * g;
      const T* src1 = static_cast<const T*>(p.seg[s]) + (int64_t)inrow[1] * p.seg_w + 8 * g;
      Op xf[4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (u < seg_steps) {
          xf[u][0] = ld_op<T>(src0 + 32 * u);
          xf[u][1] = ld_op<T>(src1 + 32 * u);
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (u < seg_steps) {
          mma_step(kb + 32 * u, xf[u]);
          // one step's weight fragments live at a time (register budget)
          __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (p.dbias) {
      // the pair-bias block: slot j' = 8g + j holds the high part of
      // dBias[j'] (j' < H) or the low part of dBias[j' - H] (j' < 2H)
      if (!p.resident) {
        __syncthreads();
        load_w(segK, 32);
        __syncthreads();
      }
      Op xb[2];
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int slot = 8 * g + j;
          float x = 0.f;
          if (slot < 2 * p.H) {
            const float d = p.dbias[(int64_t)(slot % p.H) * p.npos + pc[pb]];
            if constexpr (sizeof(T) == 2) {
              const float hi = (float)(__bf16)d;
              x = slot < p.H ? hi : d - hi;  // d - hi is exact in fp32
            } else {
              x = slot < p.H ? d : 0.f;
            }
          }
          v[j] = x;
        }
        xb[pb] = to_op(v, (Op*)nullptr);
      }
      mma_step(p.resident ? segK : 0, xb);
    }

    // Lane (l16, g) holds dX[position pb*16 + l16][32s + 8g + j] in
    // acc[2s + j/4][pb][j%4].
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      if (!p.ln) {
        if (live[pb]) {
          T* dst = static_cast<T*>(p.y) + (int64_t)pc[pb] * cout + 8 * g;
#pragma unroll
          for (int s = 0; s < CB / 2; ++s) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v[i] = acc[2 * s][pb][i];
              v[4 + i] = acc[2 * s + 1][pb][i];
            }
            st8f(dst + 32 * s, v);
          }
        }
        continue;
      }
      // LayerNorm backward of this position (statistics recomputed in fp32,
      // two-pass, population variance; sums over the 4 lane groups).
      const uint32_t zr = zrow_of(pc[pb], p.N, p.ending);
      const T* zsrc = static_cast<const T*>(p.z) + (int64_t)zr * cout + 8 * g;
      const T* gsrc = static_cast<const T*>(p.ln_w) + 8 * g;
      float xv[CB / 2][8];
      float sum = 0.f;
#pragma unroll
      for (int s = 0; s < CB / 2; ++s) {
        ld8f(zsrc + 32 * s, xv[s]);
#pragma unroll
        for (int j = 0; j < 8; ++j) sum += xv[s][j];
      }
      sum += shfl_xor(sum, 16);
      sum += shfl_xor(sum, 32);
      const float inv_n = 1.f / (float)cout;
      const float mu = sum * inv_n;
      float var = 0.f;
#pragma unroll
      for (int s = 0; s < CB / 2; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xv[s][j] -= mu;
          var = __builtin_fmaf(xv[s][j], xv[s][j], var);
        }
      var += shfl_xor(var, 16);
      var += shfl_xor(var, 32);
      const float rstd = rsqrtf(var * inv_n + p.eps);
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int s = 0; s < CB / 2; ++s) {
        float gm[8];
        ld8f(gsrc + 32 * s, gm);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xv[s][j] *= rstd;  // xhat
          const float d = acc[2 * s + (j >> 2)][pb][j & 3] * gm[j];
          acc[2 * s + (j >> 2)][pb][j & 3] = d;  // dxhat, in place
          a += d;
          b = __builtin_fmaf(d, xv[s][j], b);
        }
      }
      a += shfl_xor(a, 16);
      a += shfl_xor(a, 32);
      b += shfl_xor(b, 16);
      b += shfl_xor(b, 32);
      a *= inv_n;
      b *= inv_n;
      if (live[pb]) {
        T* dst = static_cast<T*>(p.y) + (int64_t)zr * cout + 8 * g;
#pragma unroll
        for (int s = 0; s < CB / 2; ++s) {
          float v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            v[j] = rstd * (acc[2 * s + (j >> 2)][pb][j & 3] - a - xv[s][j] * b);
          st8f(dst + 32 * s, v);
        }
      }
    }
  }
}

// -------------------------------------------------------------------- wgrad
struct WGradParams {
  int N, ending, npos;
  int nseg, a_w, a_zrow;        // A segments [npos][a_w] (row tile = segment)
  const void* aseg[kMaxSeg];
  const float* dbias;           // [H][npos]: one more row tile (16 rows), or null
  int H;
  int b_w, b_zrow, b_ln;        // B [npos][b_w]; LayerNorm-normalised (no affine)
  const void* b;
  float eps;
  int ntt, nchunks, chunk_pos;  // row tiles; positions per chunk (multiple of 32)
  float* part;                  // [nchunks][ntt*128][b_w]
  float* cpart;                 // [nchunks][ntt*128]
};

template <typename T> struct WLds;
// bf16: row-major [32 positions][128 + 16] (transposing reads); fp32:
// transposed [128][32 + 4].
template <> struct WLds<bf16_t> { static constexpr int ELEMS = 32 * 144, RS = 144; };
template <> struct WLds<float> { static constexpr int ELEMS = 128 * 36, PS = 36; };

template <typename T>
constexpr size_t wgrad_lds() {
  return 4 * WLds<T>::ELEMS * sizeof(T) + 4 * 128 * sizeof(float);
}

template <typename T>
__global__ void __launch_bounds__(256) wgrad_kernel(WGradParams p) {
  using Op = typename Tr<T>::Op;
  // A and B tiles, double-buffered, then the column-sum scratch (dynamic:
  // the fp32 tiles exceed the static limit)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T (*sA)[WLds<T>::ELEMS] = reinterpret_cast<T (*)[WLds<T>::ELEMS]>(smem);
  T (*sB)[WLds<T>::ELEMS] = sA + 2;
  float (*sred)[128] = reinterpret_cast<float (*)[128]>(smem + 4 * WLds<T>::ELEMS * sizeof(T));

  int w = xcd_work_index(p.ntt * p.nchunks);
  if (w < 0) return;
  const int tt = w % p.ntt, chunk = w / p.ntt;  // row tiles of one chunk side by side
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const bool btile = tt == p.nseg;  // the pair-bias row tile
  const int rows_t = btile ? 16 : p.a_w;
  const int RBn = rows_t / 16, CBn = p.b_w / 16;
  const int pbeg = chunk * p.chunk_pos;
  const int pend = min(p.npos, pbeg + p.chunk_pos);
  const int nst = (pend - pbeg + PW - 1) / PW;

  // Staging roles.  A (segment tile): chunks e = tid + 256u, position e/16,
  // channels 8*(e%16) .. +7 (the same 8 channels for u = 0, 1).  A (bias
  // tile): position tid/8, rows 2*(tid%8), +1.  B: position tid/8,
  // channels 16*(tid%8) .. +15.
  const T* A = btile ? nullptr : static_cast<const T*>(p.aseg[tt]);
  const T* Bsrc = static_cast<const T*>(p.b);
  float csum[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) csum[j] = 0.f;

  struct Raw {
    float a[2][8];   // A values (segment tile: two chunks; bias tile: a[0][0..1] raw dBias)
    float b[2][8];   // B values
  };
  auto fetch = [&](int st, Raw& r) {
    const int p0 = pbeg + st * PW;
    if (!btile) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = tid + 256 * u, pos = e >> 4, c8 = (e & 15) * 8;
        const int pidx = p0 + pos;
        if (pidx < pend && c8 < p.a_w) {
          const uint32_t row = p.a_zrow ? zrow_of(pidx, p.N, p.ending) : (uint32_t)pidx;
          ld8f(A + (int64_t)row * p.a_w + c8, r.a[u]);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) r.a[u][j] = 0.f;
        }
      }
    } else {
      const int pos = tid >> 3, r2 = (tid & 7) * 2;
      const int pidx = p0 + pos;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = r2 + j;
        r.a[0][j] = (pidx < pend && row < 2 * p.H)
                        ? p.dbias[(int64_t)(row % p.H) * p.npos + pidx] : 0.f;
      }
    }
    const int pos = tid >> 3, c16 = (tid & 7) * 16;
    const int pidx = p0 + pos;
    const bool ok = pidx < pend;
    const uint32_t row = ok ? (p.b_zrow ? zrow_of(pidx, p.N, p.ending) : (uint32_t)pidx) : 0u;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (ok && c16 + 8 * u < p.b_w) {
        ld8f(Bsrc + (int64_t)row * p.b_w + c16 + 8 * u, r.b[u]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) r.b[u][j] = 0.f;
      }
    }
  };
  // Column sums, LayerNorm of B, and the stores into LDS buffer `buf`.
  auto stage = [&](Raw& r, int buf) {
    T* a_ = sA[buf];
    T* b_ = sB[buf];
    if (!btile) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = tid + 256 * u, pos = e >> 4, c8 = (e & 15) * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) csum[j] += r.a[u][j];
        if (c8 < p.a_w) {
          if constexpr (sizeof(T) == 2) {
            st8f(a_ + pos * WLds<T>::RS + c8, r.a[u]);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) a_[(c8 + j) * WLds<T>::PS + pos] = r.a[u][j];
          }
        }
      }
    } else {
      const int pos = tid >> 3, r2 = (tid & 7) * 2;
      float v[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = r2 + j;
        const float d = r.a[0][j];
        if (row < p.H) csum[j] += d;
        if constexpr (sizeof(T) == 2) {
          const float hi = (float)(__bf16)d;
          v[j] = row < p.H ? hi : d - hi;
        } else {
          v[j] = row < p.H ? d : 0.f;
        }
      }
      if constexpr (sizeof(T) == 2) {
        const uint32_t u2 = uint32_t(Tr<bf16_t>::from_f(v[0])) |
                            (uint32_t(Tr<bf16_t>::from_f(v[1])) << 16);
        *reinterpret_cast<uint32_t*>(a_ + pos * WLds<T>::RS + r2) = u2;
      } else {
        a_[r2 * WLds<T>::PS + pos] = v[0];
        a_[(r2 + 1) * WLds<T>::PS + pos] = v[1];
      }
    }
    const int pos = tid >> 3, c16 = (tid & 7) * 16;
    if (p.b_ln) {
      // statistics over the 8 lanes of this position (lanes 8k .. 8k+7)
      const int nv = min(16, max(0, p.b_w - c16));
      float s = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) s += r.b[u][j];
      s += shfl_xor(s, 1);
      s += shfl_xor(s, 2);
      s += shfl_xor(s, 4);
      const float inv_n = 1.f / (float)p.b_w;
      const float mu = s * inv_n;
      float var = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float d = (8 * u + j < nv) ? r.b[u][j] - mu : 0.f;
          r.b[u][j] = d;
          var = __builtin_fmaf(d, d, var);
        }
      var += shfl_xor(var, 1);
      var += shfl_xor(var, 2);
      var += shfl_xor(var, 4);
      const float rstd = rsqrtf(var * inv_n + p.eps);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) r.b[u][j] *= rstd;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c8 = c16 + 8 * u;
      if (c8 < p.b_w) {
        if constexpr (sizeof(T) == 2) {
          st8f(b_ + pos * WLds<T>::RS + c8, r.b[u]);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) b_[(c8 + j) * WLds<T>::PS + pos] = r.b[u][j];
        }
      }
    }
  };
  // Operand fragment: column `col` of a [32 positions][cols] tile, positions
  // 8g .. 8g+7 (bf16: two transposing reads of the row-major tile).
  auto frag = [&](const T* t, int col0) -> Op {
    if constexpr (sizeof(T) == 2) {
      const T* p0 = t + (8 * g + (l16 >> 2)) * WLds<T>::RS + col0 + 4 * (l16 & 3);
      return lds_read_tr_op(p0, p0 + 4 * WLds<T>::RS);
    } else {
      return ld_op<T>(t + (col0 + l16) * WLds<T>::PS + 8 * g);
    }
  };

  f32x4 acc[8][2];  // [row block][column block of this wave]
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) acc[rb][0] = acc[rb][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  Raw raw;
  if (nst > 0) fetch(0, raw);
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    stage(raw, buf);
    __syncthreads();
    if (st + 1 < nst) fetch(st + 1, raw);
    Op bf[2];
#pragma unroll
    for (int ci = 0; ci < 2; ++ci)
      if (wave + 4 * ci < CBn) bf[ci] = frag(sB[buf], (wave + 4 * ci) * 16);
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
      if (rb >= RBn) break;
      const Op af = frag(sA[buf], rb * 16);
#pragma unroll
      for (int ci = 0; ci < 2; ++ci)
        if (wave + 4 * ci < CBn) acc[rb][ci] = mma32(af, bf[ci], acc[rb][ci]);
    }
  }

  // Partials: lane (l16, g) holds M[rb*16 + 4g + i][cb*16 + l16].
  const int rows_pad = p.ntt * 128;
  float* dst = p.part + ((int64_t)chunk * rows_pad + tt * 128) * p.b_w;
#pragma unroll
  for (int ci = 0; ci < 2; ++ci) {
    const int cb = wave + 4 * ci;
    if (cb >= CBn) continue;
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
      if (rb >= RBn) break;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[(int64_t)(rb * 16 + 4 * g + i) * p.b_w + cb * 16 + l16] = acc[rb][ci][i];
    }
  }
  // Column sums of A: reduce the lanes that staged the same rows, then the
  // four waves.
  if (!btile) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      csum[j] += shfl_xor(csum[j], 16);
      csum[j] += shfl_xor(csum[j], 32);
    }
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sred[wave][lane * 8 + j] = csum[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      csum[j] += shfl_xor(csum[j], 8);
      csum[j] += shfl_xor(csum[j], 16);
      csum[j] += shfl_xor(csum[j], 32);
    }
    if (lane < 8) {
      sred[wave][lane * 2] = csum[0];
      sred[wave][lane * 2 + 1] = csum[1];
    }
  }
  __syncthreads();
  if (tid < rows_t) {
    const float s = ((sred[0][tid] + sred[1][tid]) + sred[2][tid]) + sred[3][tid];
    p.cpart[(int64_t)chunk * rows_pad + tt * 128 + tid] = s;
  }
}

// ------------------------------------------------------------------- finish
struct FinishParams {
  int nchunks, rows_pad, ncols;
  int nseg, a_w, H, has_bias;
  const float* part;
  const float* cpart;
  int ln;                   // apply the LayerNorm affine, keep M and s for lnparam
  const void* ln_w;
  const void* ln_b;
  float* dw[kMaxSeg];       // [a_w][ncols] per segment
  float* dw_bias;           // [H][ncols]
  float* dcol[kMaxSeg];     // column sums of segment s ([a_w]) or null
  float* mred;              // [nseg*a_w + H][ncols] (ln)
  float* cred;              // [nseg*a_w + H] (ln)
};

template <typename T>
__global__ void __launch_bounds__(256) wgrad_finish_kernel(FinishParams p) {
  const int nrows = p.nseg * p.a_w + (p.has_bias ? p.H : 0);
  const int64_t total = (int64_t)nrows * p.ncols;
  const int64_t cstride = (int64_t)p.rows_pad * p.ncols;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int k = (int)(e / p.ncols), c = (int)(e - (int64_t)k * p.ncols);
    float m = 0.f, s = 0.f;
    int seg = -1, r = 0;
    if (k < p.nseg * p.a_w) {
      seg = k / p.a_w;
      r = k - seg * p.a_w;
      const int slot = seg * 128 + r;
      for (int ch = 0; ch < p.nchunks; ++ch) {
        m += p.part[ch * cstride + (int64_t)slot * p.ncols + c];
        s += p.cpart[(int64_t)ch * p.rows_pad + slot];
      }
    } else {
      r = k - p.nseg * p.a_w;  // head
      const int hi = p.nseg * 128 + r, lo = hi + p.H;
      float mh = 0.f, ml = 0.f;
      for (int ch = 0; ch < p.nchunks; ++ch) {
        mh += p.part[ch * cstride + (int64_t)hi * p.ncols + c];
        ml += p.part[ch * cstride + (int64_t)lo * p.ncols + c];
        s += p.cpart[(int64_t)ch * p.rows_pad + hi];
      }
      m = mh + ml;
    }
    float out = m;
    if (p.ln) {
      const float gm = Tr<T>::to_f(static_cast<const T*>(p.ln_w)[c]);
      const float bt = Tr<T>::to_f(static_cast<const T*>(p.ln_b)[c]);
      out = __builtin_fmaf(gm, m, bt * s);
      p.mred[e] = m;
      if (c == 0) p.cred[k] = s;
    }
    if (seg >= 0) {
      p.dw[seg][(int64_t)r * p.ncols + c] = out;
      if (c == 0 && p.dcol[seg]) p.dcol[seg][r] = s;
    } else {
      p.dw_bias[(int64_t)r * p.ncols + c] = out;
    }
  }
}

// dgamma[c] = sum_k W[k][c] M[k][c], dbeta[c] = sum_k W[k][c] s[k], over the
// rows of every segment weight and of the pair-bias weight.
struct LnParamParams {
  int nseg, a_w, H, ncols;
  const void* wseg[kMaxSeg];   // [a_w][ncols]
  const void* wbias;           // [H][ncols]
  const float* mred;
  const float* cred;
  float* dln_w;
  float* dln_b;
};

template <typename T>
__global__ void __launch_bounds__(256) lnparam_kernel(LnParamParams p) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= p.ncols) return;
  float dg = 0.f, db = 0.f;
  const int nrows = p.nseg * p.a_w + p.H;
  for (int k = 0; k < nrows; ++k) {
    const T* wr;
    if (k < p.nseg * p.a_w) {
      const int s = k / p.a_w;
      wr = static_cast<const T*>(p.wseg[s]) + (int64_t)(k - s * p.a_w) * p.ncols;
    } else {
      wr = static_cast<const T*>(p.wbias) + (int64_t)(k - p.nseg * p.a_w) * p.ncols;
    }
    const float wv = Tr<T>::to_f(wr[c]);
    dg = __builtin_fmaf(wv, p.mred[(int64_t)k * p.ncols + c], dg);
    db = __builtin_fmaf(wv, p.cred[k], db);
  }
  p.dln_w[c] = dg;
  p.dln_b[c] = db;
}

// ----------------------------------------------------------------- launches
template <typename T, int CB>
hipError_t launch_rowgrad_cb(RowGradParams& p, hipStream_t s) {
  // eight waves: the LayerNorm epilogue holds a position block's z row
  // next to both blocks' accumulators
  constexpr int WAVES = 8;
  const size_t wbytes = (size_t)p.cout * (p.Kext + PADE) * sizeof(T);
  p.resident = wbytes <= kLdsBudget;
  p.kc = p.resident ? p.Kext : std::max(p.seg_w, 32);
  const size_t lds = (size_t)p.cout * (p.kc + PADE) * sizeof(T);
  const int64_t tiles = ((int64_t)p.npos + PW * WAVES - 1) / (PW * WAVES);
  p.ntiles = (int)tiles;
  const int grid = (int)std::min<int64_t>(tiles, 256);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rowgrad_kernel<T, CB, WAVES>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((rowgrad_kernel<T, CB, WAVES>), dim3(grid), dim3(WAVES * 64), lds, s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rowgrad(RowGradParams& p, hipStream_t s) {
  switch (p.cout / 16) {
    case 2: return launch_rowgrad_cb<T, 2>(p, s);
    case 4: return launch_rowgrad_cb<T, 4>(p, s);
    case 6: return launch_rowgrad_cb<T, 6>(p, s);
    case 8: return launch_rowgrad_cb<T, 8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// Chunking of the positions for the weight GEMM: about `target` chunks of a
// multiple of 32 positions.
void chunking(int64_t npos, int target, int& nchunks, int& chunk_pos) {
  const int64_t steps = (npos + PW - 1) / PW;
  const int64_t per = std::max<int64_t>(1, (steps + target - 1) / target);
  chunk_pos = (int)(per * PW);
  nchunks = (int)((npos + chunk_pos - 1) / chunk_pos);
}
constexpr int kChunksModule = 128;   // 5 row tiles: ~640 workgroups
constexpr int kChunksOut = 512;      // 1 row tile

template <typename T>
hipError_t launch_wgrad(WGradParams& p, hipStream_t s) {
  const int total = p.ntt * p.nchunks;
  const int grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
  const size_t lds = wgrad_lds<T>();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&wgrad_kernel<T>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(wgrad_kernel<T>, dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_finish(FinishParams& f, hipStream_t s) {
  const int64_t total = (int64_t)(f.nseg * f.a_w + (f.has_bias ? f.H : 0)) * f.ncols;
  const int grid = (int)std::min<int64_t>((total + 255) / 256, 1024);
  hipLaunchKernelGGL(wgrad_finish_kernel<T>, dim3(grid), dim3(256), 0, s, f);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct PartLayout {
  size_t part, cpart, mred, cred, total;
};
PartLayout part_layout(int64_t N, int64_t CZ, int64_t H) {
  const int64_t npos = N * N, HC = H * kHeadDim;
  int nm, cm, no, co;
  chunking(npos, kChunksModule, nm, cm);
  chunking(npos, kChunksOut, no, co);
  const size_t part_m = (size_t)nm * 5 * 128 * CZ * 4, cpart_m = (size_t)nm * 5 * 128 * 4;
  const size_t part_o = (size_t)no * 128 * HC * 4, cpart_o = (size_t)no * 128 * 4;
  PartLayout L;
  L.part = 0;
  L.cpart = align256(std::max(part_m, part_o));
  L.mred = L.cpart + align256(std::max(cpart_m, cpart_o));
  L.cred = L.mred + align256((size_t)(4 * HC + H) * CZ * 4);
  L.total = L.cred + align256((size_t)(4 * HC + H) * 4);
  return L;
}

template <typename T>
hipError_t out_project_bwd_t(const OutProjectBwdArgs& a, hipStream_t s) {
  const int N = (int)a.N, CZ = (int)a.CZ, H = (int)a.H, HC = H * kHeadDim;
  const int npos = N * N;
  const PartLayout L = part_layout(a.N, a.CZ, a.H);
  char* ws = static_cast<char*>(a.workspace);
  // d_o[pos] = dout[z row of pos] . w_o   (w_o is [CZ][HC]: W_ext[k=cz][c=hc])
  RowGradParams r{};
  r.N = N; r.ending = a.ending; r.npos = npos;
  r.nseg = 1; r.seg_w = CZ; r.in_zrow = 1; r.seg[0] = a.dout;
  r.dbias = nullptr; r.H = H; r.Kext = CZ;
  r.wseg[0] = a.w_o; r.wbias = nullptr; r.cout = HC;
  r.ln = 0; r.y = a.d_o;
  hipError_t e = launch_rowgrad<T>(r, s);
  if (e != hipSuccess) return e;
  // dw_o = sum_pos dout[z row]^T o[pos], db_o = sum_pos dout
  WGradParams w{};
  w.N = N; w.ending = a.ending; w.npos = npos;
  w.nseg = 1; w.a_w = CZ; w.a_zrow = 1; w.aseg[0] = a.dout;
  w.dbias = nullptr; w.H = H;
  w.b_w = HC; w.b_zrow = 0; w.b_ln = 0; w.b = a.o; w.eps = 0.f;
  w.ntt = 1;
  chunking(npos, kChunksOut, w.nchunks, w.chunk_pos);
  w.part = reinterpret_cast<float*>(ws + L.part);
  w.cpart = reinterpret_cast<float*>(ws + L.cpart);
  if ((e = launch_wgrad<T>(w, s)) != hipSuccess) return e;
  FinishParams f{};
  f.nchunks = w.nchunks; f.rows_pad = 128; f.ncols = HC;
  f.nseg = 1; f.a_w = CZ; f.H = H; f.has_bias = 0;
  f.part = w.part; f.cpart = w.cpart;
  f.ln = 0;
  f.dw[0] = a.dw_o; f.dcol[0] = a.db_o;
  return launch_finish<T>(f, s);
}

template <typename T>
hipError_t project_bwd_t(const ProjectBwdArgs& a, hipStream_t s) {
  const int N = (int)a.N, CZ = (int)a.CZ, H = (int)a.H, HC = H * kHeadDim;
  const int npos = N * N;
  const PartLayout L = part_layout(a.N, a.CZ, a.H);
  char* ws = static_cast<char*>(a.workspace);
  const void* dys[4] = {a.dq, a.dk, a.dv, a.dg};
  const void* wts[4] = {a.w_q, a.w_k, a.w_v, a.w_g};
  // dz = LayerNorm backward of [dq | dk | dv | dg | dbias] . W_ext
  RowGradParams r{};
  r.N = N; r.ending = a.ending; r.npos = npos;
  r.nseg = 4; r.seg_w = HC; r.in_zrow = 0;
  for (int i = 0; i < 4; ++i) { r.seg[i] = dys[i]; r.wseg[i] = wts[i]; }
  r.dbias = a.dbias; r.H = H; r.Kext = 4 * HC + 32;
  r.wbias = a.w_bias; r.cout = CZ;
  r.ln = 1; r.z = a.z; r.ln_w = a.ln_w; r.eps = a.eps; r.y = a.dz;
  hipError_t e = launch_rowgrad<T>(r, s);
  if (e != hipSuccess) return e;
  // M = [dq | dk | dv | dg | dbias]^T xhat and the column sums
  WGradParams w{};
  w.N = N; w.ending = a.ending; w.npos = npos;
  w.nseg = 4; w.a_w = HC; w.a_zrow = 0;
  for (int i = 0; i < 4; ++i) w.aseg[i] = dys[i];
  w.dbias = a.dbias; w.H = H;
  w.b_w = CZ; w.b_zrow = 1; w.b_ln = 1; w.b = a.z; w.eps = a.eps;
  w.ntt = 5;
  chunking(npos, kChunksModule, w.nchunks, w.chunk_pos);
  w.part = reinterpret_cast<float*>(ws + L.part);
  w.cpart = reinterpret_cast<float*>(ws + L.cpart);
  if ((e = launch_wgrad<T>(w, s)) != hipSuccess) return e;
  FinishParams f{};
  f.nchunks = w.nchunks; f.rows_pad = 5 * 128; f.ncols = CZ;
  f.nseg = 4; f.a_w = HC; f.H = H; f.has_bias = 1;
  f.part = w.part; f.cpart = w.cpart;
  f.ln = 1; f.ln_w = a.ln_w; f.ln_b = a.ln_b;
  f.dw[0] = a.dw_q; f.dw[1] = a.dw_k; f.dw[2] = a.dw_v; f.dw[3] = a.dw_g;
  f.dw_bias = a.dw_bias;
  f.dcol[3] = a.db_g;
  f.mred = reinterpret_cast<float*>(ws + L.mred);
  f.cred = reinterpret_cast<float*>(ws + L.cred);
  if ((e = launch_finish<T>(f, s)) != hipSuccess) return e;
  LnParamParams l{};
  l.nseg = 4; l.a_w = HC; l.H = H; l.ncols = CZ;
  for (int i = 0; i < 4; ++i) l.wseg[i] = wts[i];
  l.wbias = a.w_bias; l.mred = f.mred; l.cred = f.cred;
  l.dln_w = a.dln_w; l.dln_b = a.dln_b;
  hipLaunchKernelGGL(lnparam_kernel<T>, dim3((CZ + 255) / 256), dim3(256), 0, s, l);
  return hipGetLastError();
}

}  // namespace

size_t proj_bwd_workspace(int64_t N, int64_t CZ, int64_t H) {
  return part_layout(N, CZ, H).total;
}

hipError_t launch_out_project_bwd(const OutProjectBwdArgs& a, hipStream_t s) {
  return a.dtype == 1 ? out_project_bwd_t<bf16_t>(a, s) : out_project_bwd_t<float>(a, s);
}

hipError_t launch_project_bwd(const ProjectBwdArgs& a, hipStream_t s) {
  return a.dtype == 1 ? project_bwd_t<bf16_t>(a, s) : project_bwd_t<float>(a, s);
}

}  // namespace evo
