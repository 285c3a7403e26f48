// Backward of the fused LayerNorm + linear + SwiGLU transition on gfx950.
//
// EvoFusion ("MegaFold: Efficient Training of Next-Generation 3D Attention
// Protein Models on Cross-Platform GPUs", section "Methodologie", item 3)
// targets the activation memory of these operators in training.  The
// backward is the chain rule of the forward
//   x = LN(z) = xhat * gamma + beta,  u = x . W_a^T,  v = x . W_b^T,
//   h = silu(u) * v,  out = h . W_o^T,
// with silu'(u) = sigmoid(u) * (1 + u * (1 - sigmoid(u))):
//   dh = dout . W_o,  du = dh * v * silu'(u),  dv = dh * silu(u),
//   dx = du . W_a + dv . W_b,  dz = LayerNorm backward of dx,
//   dW_a = sum_pos du^T x,  dW_b = sum_pos dv^T x,  dW_o = sum_pos dout^T h,
//   dgamma[c] = sum_k W_a[k,c] M_a[k,c] + W_b[k,c] M_b[k,c],
//   dbeta[c]  = sum_k W_a[k,c] s_a[k]   + W_b[k,c] s_b[k],
// where M = sum_pos d(.)^T xhat and s = sum_pos d(.) (the rearrangement the
// module backward uses: dW = gamma * M + beta * s).
//
// Kernels.
//   prep     once per call: per chunk of 32 hidden units, W_a, W_b (gamma
//            folded in) and W_o^T rows permuted so that the products come
//            out in the next product's operand layout, beta . W^T, and the
//            chunk's W_a, W_b columns transposed ([c_z][32]).
//   rows     persistent, 8 waves of 32 positions (the forward's structure):
//            xhat and dout rows held as operands; per chunk u, v and dh on
//            the matrix cores, du, dv, h in registers, written once (bf16 or
//            fp32) for the weight gradients, and dx^T += W_a^T du^T +
//            W_b^T dv^T accumulated in registers; then the LayerNorm backward
//            in registers and dz written.  No [N^2, c_z] intermediate.
//   weights  the module backward's fixed-order weight-gradient reduction over
//            positions (segments of 128 hidden units), then W_o^T -> W_o and
//            dgamma, dbeta from M and s.
#include <algorithm>

#include "evo_device.h"
#include "evo_kernels.h"

namespace evo {
namespace {

constexpr int PW = 32;     // positions per wave
constexpr int WAVES = 8;
constexpr int PADE = 8;
constexpr int HC = 32;     // hidden units per chunk
constexpr int SEG = 128;   // hidden units per weight-gradient segment

struct TransBwdParams {
  int npos, CZ, HID, ntiles;
  const void* z;
  const void* ln_w;
  const void* ln_b;
  float eps;
  const void* w_a;   // [HID][CZ]
  const void* w_b;   // [HID][CZ]
  const void* w_o;   // [CZ][HID]
  const void* dout;  // [npos][CZ]
  void* dz;          // [npos][CZ]
  void* wts;         // [nq][3*HC*CZ + 2*CZ*HC] prepared, per chunk
  float* cst;        // [nq][2][HC]
  void* du;          // [HID/SEG][npos][SEG] each
  void* dv;
  void* h;
};

__device__ __forceinline__ int hrow_of(int u) {  // u < 32
  const int gg = u >> 3, j = u & 7;
  return 16 * (j >> 2) + 4 * gg + (j & 3);
}

template <typename T>
__global__ void __launch_bounds__(256) transition_bwd_prep_kernel(TransBwdParams p) {
  const int CZ = p.CZ, HID = p.HID;
  const T* lnw = static_cast<const T*>(p.ln_w);
  const T* lnb = static_cast<const T*>(p.ln_b);
  const T* wa = static_cast<const T*>(p.w_a);
  const T* wb = static_cast<const T*>(p.w_b);
  const T* wo = static_cast<const T*>(p.w_o);
  T* out = static_cast<T*>(p.wts);
  const int64_t per_q = (int64_t)5 * HC * CZ;
  const int64_t total = (int64_t)(HID / HC) * per_q;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int q = (int)(e / per_q);
    const int64_t r = e - (int64_t)q * per_q;
    float v;
    if (r < (int64_t)3 * HC * CZ) {
      // [m][hrow(u)][k]: W_a * gamma, W_b * gamma, W_o^T
      const int m = (int)(r / (HC * CZ));
      const int rr = (int)(r - (int64_t)m * HC * CZ);
      const int row = rr / CZ, k = rr - row * CZ;
      int u = 0;
      for (int t = 0; t < HC; ++t)
        if (hrow_of(t) == row) u = t;
      const int hid = q * HC + u;
      if (m == 0) v = Tr<T>::to_f(wa[(int64_t)hid * CZ + k]) * Tr<T>::to_f(lnw[k]);
      else if (m == 1) v = Tr<T>::to_f(wb[(int64_t)hid * CZ + k]) * Tr<T>::to_f(lnw[k]);
      else v = Tr<T>::to_f(wo[(int64_t)k * HID + hid]);
    } else {
      // [m][c][u]: the chunk's W_a, W_b columns, transposed
      const int rr = (int)(r - (int64_t)3 * HC * CZ);
      const int m = rr / (CZ * HC);
      const int r2 = rr - m * CZ * HC;
      const int c = r2 / HC, u = r2 - c * HC;
      const int hid = q * HC + u;
      v = Tr<T>::to_f((m == 0 ? wa : wb)[(int64_t)hid * CZ + c]);
    }
    out[e] = Tr<T>::from_f(v);
  }
  // beta . W^T per (matrix, unit): one wave each, a fixed-order sum
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * 4;
  for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < 2 * HID; t += nwaves) {
    const int m = t / HID, hid = t - m * HID;
    const T* w = (m == 0 ? wa : wb) + (int64_t)hid * CZ;
    float acc = 0.f;
    for (int k = lane; k < CZ; k += 64) acc = __builtin_fmaf(Tr<T>::to_f(lnb[k]), Tr<T>::to_f(w[k]), acc);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) {
      const int q = hid / HC, u = hid - q * HC;
      p.cst[((int64_t)q * 2 + m) * HC + hrow_of(u)] = acc;
    }
  }
}

template <typename T>
__device__ __forceinline__ typename Tr<T>::Op to_op8(const float (&v)[8]) {
  typename Tr<T>::Op f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (sizeof(T) == 2) f[j] = (__bf16)v[j];
    else f[j] = v[j];
  }
  return f;
}

template <typename T, int KS>  // KS = CZ / 32
__global__ void __launch_bounds__(WAVES * 64) transition_bwd_kernel(TransBwdParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int CZ = KS * 32, CB = KS * 2;
  constexpr int WRS = CZ + PADE;           // unit rows (contraction over c_z)
  constexpr int TRS = HC + PADE;           // c_z rows (contraction over units)
  constexpr int BUF = 3 * HC * WRS + 2 * CZ * TRS;
  constexpr int NB = sizeof(T) == 2 ? 2 : 1;  // fp32: one buffer (LDS)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sbuf = reinterpret_cast<T*>(smem);                 // [NB][BUF]
  float* sC = reinterpret_cast<float*>(sbuf + NB * BUF);  // [NB][2][HC]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int nchunks = p.HID / HC;
  constexpr int E16 = 16 / sizeof(T);

  auto load_chunk = [&](int q, int buf) {
    T* sw = sbuf + buf * BUF;
    T* st = sw + 3 * HC * WRS;
    const T* gw = static_cast<const T*>(p.wts) + (int64_t)q * 5 * HC * CZ;
    const T* gt = gw + 3 * HC * CZ;
    for (int e = tid; e < 3 * HC * CZ / E16; e += WAVES * 64) {
      const int row = e / (CZ / E16), col = (e - row * (CZ / E16)) * E16;
      *reinterpret_cast<u32x4*>(sw + row * WRS + col) =
          *reinterpret_cast<const u32x4*>(gw + (int64_t)row * CZ + col);
    }
    for (int e = tid; e < 2 * CZ * HC / E16; e += WAVES * 64) {
      const int row = e / (HC / E16), col = (e - row * (HC / E16)) * E16;
      *reinterpret_cast<u32x4*>(st + row * TRS + col) =
          *reinterpret_cast<const u32x4*>(gt + (int64_t)row * HC + col);
    }
    for (int e = tid; e < 2 * HC; e += WAVES * 64) sC[buf * 2 * HC + e] = p.cst[(int64_t)q * 2 * HC + e];
  };

  // bf16 (two buffers): the next chunk's 16-byte blocks are loaded into
  // registers at the start of a chunk (buffer loads: uniform bases, each
  // lane's offset fixed) and copied into the other buffer at its end, so the
  // loads are in flight while the chunk is computed.
  constexpr int NW3 = 3 * HC * CZ / E16, NTT = 2 * CZ * HC / E16;
  constexpr int PER = (NW3 + NTT + WAVES * 64 - 1) / (WAVES * 64);
  u32x4 wreg[NB == 2 ? PER : 1];
  float creg = 0.f;
  const uint32_t wts_bytes = (uint32_t)((int64_t)nchunks * 5 * HC * CZ * sizeof(T));
  auto fetch_chunk = [&](int q) {
    const uint32_t qo = (uint32_t)(q * 5 * HC * CZ * sizeof(T));
    // the chunk's prepared blocks are contiguous: 16-byte block e sits at
    // byte 16 e of the chunk
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + u * WAVES * 64;
      if (e < NW3 + NTT) wreg[u] = buf_ld128(p.wts, wts_bytes, (uint32_t)e * 16u, qo);
    }
    if (tid < 2 * HC) creg = p.cst[(int64_t)q * 2 * HC + tid];
  };
  auto store_chunk = [&](int buf) {
    T* sw = sbuf + buf * BUF;
    T* st = sw + 3 * HC * WRS;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + u * WAVES * 64;
      if (e < NW3) {
        const int row = e / (CZ / E16), col = (e - row * (CZ / E16)) * E16;
        *reinterpret_cast<u32x4*>(sw + row * WRS + col) = wreg[u];
      } else if (e < NW3 + NTT) {
        const int e2 = e - NW3, row = e2 / (HC / E16), col = (e2 - row * (HC / E16)) * E16;
        *reinterpret_cast<u32x4*>(st + row * TRS + col) = wreg[u];
      }
    }
    if (tid < 2 * HC) sC[buf * 2 * HC + tid] = creg;
  };
  static_assert(2 * HC <= WAVES * 64, "one constant per thread");

  const T* Z = static_cast<const T*>(p.z);
  const T* D = static_cast<const T*>(p.dout);
  for (int tile = blockIdx.x; tile < p.ntiles; tile += gridDim.x) {
    uint32_t pidx[2];
    bool live[2];
    float mu[2], rstd[2];
    Op xf[2][KS], df[2][KS];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      pidx[pb] = ((uint32_t)tile * WAVES + wave) * PW + pb * 16 + l16;
      live[pb] = pidx[pb] < (uint32_t)p.npos;
      const int64_t row = (int64_t)(live[pb] ? pidx[pb] : 0) * CZ + 8 * g;
      float v[KS][8];
      float sum = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Raw8<T> r;
        ld_raw8(r, Z + row + 32 * s);
        f32x4 lo, hi;
        widen8(r, lo, hi);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[s][i] = lo[i];
          v[s][4 + i] = hi[i];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) sum += v[s][j];
        Raw8<T> rd;
        ld_raw8(rd, D + row + 32 * s);
        f32x4 dlo, dhi;
        widen8(rd, dlo, dhi);
        float dv8[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dv8[i] = dlo[i];
          dv8[4 + i] = dhi[i];
        }
        df[pb][s] = to_op8<T>(dv8);
      }
      sum += shfl_xor(sum, 16);
      sum += shfl_xor(sum, 32);
      mu[pb] = sum / CZ;
      float var = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          v[s][j] -= mu[pb];
          var = __builtin_fmaf(v[s][j], v[s][j], var);
        }
      var += shfl_xor(var, 16);
      var += shfl_xor(var, 32);
      rstd[pb] = rsqrtf(var / CZ + p.eps);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        float xv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = v[s][j] * rstd[pb];
        xf[pb][s] = to_op8<T>(xv);
      }
    }

    f32x4 dx[CB][2];  // dx^T blocks [c_z block][pb]
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) dx[cb][0] = dx[cb][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // the previous tile's last chunk is no longer read
    if constexpr (NB == 2) {
      fetch_chunk(0);
      store_chunk(0);
    } else {
      load_chunk(0, 0);
    }
    for (int q = 0; q < nchunks; ++q) {
      int buf = 0;
      if constexpr (NB == 2) {
        buf = q & 1;
        __syncthreads();  // chunk q is in LDS; chunk q-1's buffer is free
        if (q + 1 < nchunks) fetch_chunk(q + 1);
      } else {
        if (q > 0) {
          __syncthreads();  // chunk q-1 no longer read
          load_chunk(q, 0);
        }
        __syncthreads();
      }
      const T* sw = sbuf + buf * BUF;
      const T* st = sw + 3 * HC * WRS;
      const float* sc = sC + buf * 2 * HC;
      f32x4 ua[2][2], ub[2][2], dh[2][2];  // [unit block][pb]
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const f32x4 ca = *reinterpret_cast<const f32x4*>(sc + hb * 16 + 4 * g);
        const f32x4 cbv = *reinterpret_cast<const f32x4*>(sc + HC + hb * 16 + 4 * g);
        ua[hb][0] = ua[hb][1] = ca;
        ub[hb][0] = ub[hb][1] = cbv;
        dh[hb][0] = dh[hb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const Op fa = *reinterpret_cast<const Op*>(sw + (hb * 16 + l16) * WRS + 32 * s + 8 * g);
          const Op fb = *reinterpret_cast<const Op*>(sw + (HC + hb * 16 + l16) * WRS + 32 * s + 8 * g);
          const Op fo = *reinterpret_cast<const Op*>(sw + (2 * HC + hb * 16 + l16) * WRS + 32 * s + 8 * g);
#pragma unroll
          for (int pb = 0; pb < 2; ++pb) {
            ua[hb][pb] = mma32(fa, xf[pb][s], ua[hb][pb]);
            ub[hb][pb] = mma32(fb, xf[pb][s], ub[hb][pb]);
            dh[hb][pb] = mma32(fo, df[pb][s], dh[hb][pb]);
          }
        }
      }
      // lane (l16, g) of blocks (0, 1) holds units 8g .. 8g+7 of the chunk
      // for position pb*16 + l16: the operand of the dx product
      const int unit0 = q * HC + 8 * g;
      const int seg = unit0 / SEG, col = unit0 - seg * SEG;
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        float vu[8], vv[8], vh[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float u = ua[j >> 2][pb][j & 3];
          const float b = ub[j >> 2][pb][j & 3];
          const float d = dh[j >> 2][pb][j & 3];
          const float sg = rcp_fast(1.f + exp2_fast(-u * kLog2e));
          const float si = u * sg;
          vh[j] = si * b;
          vv[j] = d * si;
          vu[j] = d * b * sg * __builtin_fmaf(u, 1.f - sg, 1.f);
        }
        const Op fu = to_op8<T>(vu), fv = to_op8<T>(vv), fh = to_op8<T>(vh);
        if (live[pb]) {
          const int64_t off = ((int64_t)seg * p.npos + pidx[pb]) * SEG + col;
          *reinterpret_cast<Op*>(static_cast<T*>(p.du) + off) = fu;
          *reinterpret_cast<Op*>(static_cast<T*>(p.dv) + off) = fv;
          *reinterpret_cast<Op*>(static_cast<T*>(p.h) + off) = fh;
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const Op ta = *reinterpret_cast<const Op*>(st + (cb * 16 + l16) * TRS + 8 * g);
          const Op tb = *reinterpret_cast<const Op*>(st + (CZ + cb * 16 + l16) * TRS + 8 * g);
          dx[cb][pb] = mma32(ta, fu, dx[cb][pb]);
          dx[cb][pb] = mma32(tb, fv, dx[cb][pb]);
        }
      }
      if constexpr (NB == 2)
        if (q + 1 < nchunks) store_chunk(buf ^ 1);
    }

    // LayerNorm backward: lane (l16, g) holds dx[pos pb*16 + l16][cb*16 + 4g + i]
    const T* lnw = static_cast<const T*>(p.ln_w);
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      const int64_t row = (int64_t)(live[pb] ? pidx[pb] : 0) * CZ;
      float xh[CB][4], dxh[CB][4];
      float m1 = 0.f, m2 = 0.f;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int c0 = cb * 16 + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xh[cb][i] = (Tr<T>::to_f(Z[row + c0 + i]) - mu[pb]) * rstd[pb];
          dxh[cb][i] = dx[cb][pb][i] * Tr<T>::to_f(lnw[c0 + i]);
          m1 += dxh[cb][i];
          m2 = __builtin_fmaf(dxh[cb][i], xh[cb][i], m2);
        }
      }
      m1 += shfl_xor(m1, 16);
      m1 += shfl_xor(m1, 32);
      m2 += shfl_xor(m2, 16);
      m2 += shfl_xor(m2, 32);
      m1 /= CZ;
      m2 /= CZ;
      if (!live[pb]) continue;
      T* dst = static_cast<T*>(p.dz) + row;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int c0 = cb * 16 + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[c0 + i] = Tr<T>::from_f(rstd[pb] * (dxh[cb][i] - m1 - xh[cb][i] * m2));
      }
    }
  }
}

// dw_o[c][k] = the transposed reduction result dwoT[k][c].
__global__ void __launch_bounds__(256) transpose_kernel(const float* src, float* dst, int rows,
                                                        int cols) {
  const int64_t total = (int64_t)rows * cols;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int r = (int)(e / cols), c = (int)(e - (int64_t)r * cols);
    dst[(int64_t)c * rows + r] = src[e];
  }
}

// dgamma, dbeta from the reductions of both projections: one workgroup per
// channel, thread t over rows t, t+256, ..., then a fixed-order sum.
template <typename T>
__global__ void __launch_bounds__(256) transition_lnparam_kernel(
    const T* w_a, const T* w_b, const float* m_a, const float* m_b, const float* s_a,
    const float* s_b, int HID, int CZ, float* dln_w, float* dln_b) {
  __shared__ float red[2][256];
  const int c = blockIdx.x, tid = threadIdx.x;
  float dg = 0.f, db = 0.f;
  for (int k = tid; k < HID; k += 256) {
    const int64_t e = (int64_t)k * CZ + c;
    const float wa = Tr<T>::to_f(w_a[e]), wb = Tr<T>::to_f(w_b[e]);
    dg = __builtin_fmaf(wa, m_a[e], dg);
    dg = __builtin_fmaf(wb, m_b[e], dg);
    db = __builtin_fmaf(wa, s_a[k], db);
    db = __builtin_fmaf(wb, s_b[k], db);
  }
  red[0][tid] = dg;
  red[1][tid] = db;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      red[0][tid] += red[0][tid + w];
      red[1][tid] += red[1][tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    dln_w[c] = red[0][0];
    dln_b[c] = red[1][0];
  }
}

size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

struct BwdLayoutT {
  size_t wts, cst, du, dv, h, seg, mra, mrb, cra, crb, wot, total;
};
BwdLayoutT bwd_layout_t(int dtype, int64_t npos, int64_t CZ, int64_t HID) {
  const size_t es = dtype == 1 ? 2 : 4;
  BwdLayoutT L;
  size_t o = 0;
  L.wts = o; o += a256((size_t)HID * 5 * CZ * es);
  L.cst = o; o += a256((size_t)2 * HID * 4);
  const size_t act = a256((size_t)npos * HID * es);
  L.du = o; o += act;
  L.dv = o; o += act;
  L.h = o; o += act;
  L.seg = o; o += a256(seg_wgrad_workspace(npos, CZ));
  L.mra = o; o += a256((size_t)HID * CZ * 4);
  L.mrb = o; o += a256((size_t)HID * CZ * 4);
  L.cra = o; o += a256((size_t)HID * 4);
  L.crb = o; o += a256((size_t)HID * 4);
  L.wot = o; o += a256((size_t)HID * CZ * 4);
  L.total = o;
  return L;
}

template <typename T, int KS>
hipError_t launch_rows(TransBwdParams& p, hipStream_t s) {
  constexpr int CZ = KS * 32;
  constexpr int NB = sizeof(T) == 2 ? 2 : 1;
  const size_t lds = (size_t)NB * (3 * HC * (CZ + PADE) + 2 * CZ * (HC + PADE)) * sizeof(T) +
                     (size_t)NB * 2 * HC * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&transition_bwd_kernel<T, KS>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int grid = std::min(p.ntiles, 256);
  hipLaunchKernelGGL((transition_bwd_kernel<T, KS>), dim3(grid), dim3(WAVES * 64), lds, s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t transition_bwd_t(const TransitionBwdArgs& a, hipStream_t s) {
  const BwdLayoutT L = bwd_layout_t(a.dtype, a.npos, a.CZ, a.HID);
  char* ws = static_cast<char*>(a.workspace);
  TransBwdParams p{};
  p.npos = (int)a.npos; p.CZ = (int)a.CZ; p.HID = (int)a.HID;
  p.ntiles = (int)((a.npos + PW * WAVES - 1) / (PW * WAVES));
  p.z = a.z; p.ln_w = a.ln_w; p.ln_b = a.ln_b; p.eps = a.eps;
  p.w_a = a.w_a; p.w_b = a.w_b; p.w_o = a.w_o; p.dout = a.dout; p.dz = a.dz;
  p.wts = ws + L.wts;
  p.cst = reinterpret_cast<float*>(ws + L.cst);
  p.du = ws + L.du; p.dv = ws + L.dv; p.h = ws + L.h;
  hipLaunchKernelGGL(transition_bwd_prep_kernel<T>, dim3(256), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (p.CZ / 32) {
    case 1: e = launch_rows<T, 1>(p, s); break;
    case 2: e = launch_rows<T, 2>(p, s); break;
    case 3: e = launch_rows<T, 3>(p, s); break;
    case 4: e = launch_rows<T, 4>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  // weight gradients, segments of 128 hidden units (four at a time when
  // they divide evenly)
  const int nseg_all = (int)(a.HID / SEG);
  const int step = nseg_all % 4 == 0 ? 4 : 1;
  float* mra = reinterpret_cast<float*>(ws + L.mra);
  float* mrb = reinterpret_cast<float*>(ws + L.mrb);
  float* cra = reinterpret_cast<float*>(ws + L.cra);
  float* crb = reinterpret_cast<float*>(ws + L.crb);
  float* wot = reinterpret_cast<float*>(ws + L.wot);
  const size_t es = sizeof(T);
  const size_t seg_bytes = (size_t)a.npos * SEG * es;
  struct Job {
    char* act;
    const void* b;
    int ln;
    float* dw;
    float* mred;
    float* cred;
  } jobs[3] = {{ws + L.du, a.z, 1, a.dw_a, mra, cra},
               {ws + L.dv, a.z, 1, a.dw_b, mrb, crb},
               {ws + L.h, a.dout, 0, wot, nullptr, nullptr}};
  for (const Job& j : jobs) {
    for (int s0 = 0; s0 < nseg_all; s0 += step) {
      SegWGradArgs w{};
      w.dtype = a.dtype; w.npos = a.npos; w.nseg = step;
      for (int i = 0; i < step; ++i) {
        w.aseg[i] = j.act + (size_t)(s0 + i) * seg_bytes;
        w.dw[i] = j.dw + (size_t)(s0 + i) * SEG * a.CZ;
      }
      w.b = j.b; w.ncols = (int)a.CZ; w.b_ln = j.ln;
      w.ln_w = a.ln_w; w.ln_b = a.ln_b; w.eps = a.eps;
      w.mred = j.mred ? j.mred + (size_t)s0 * SEG * a.CZ : nullptr;
      w.cred = j.cred ? j.cred + (size_t)s0 * SEG : nullptr;
      w.workspace = ws + L.seg;
      if ((e = launch_seg_wgrad(w, s)) != hipSuccess) return e;
    }
  }
  const int64_t nw = a.HID * a.CZ;
  hipLaunchKernelGGL(transpose_kernel, dim3((int)std::min<int64_t>((nw + 255) / 256, 1024)),
                     dim3(256), 0, s, wot, a.dw_o, (int)a.HID, (int)a.CZ);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(transition_lnparam_kernel<T>, dim3((int)a.CZ), dim3(256), 0, s,
                     static_cast<const T*>(a.w_a), static_cast<const T*>(a.w_b), mra, mrb, cra,
                     crb, (int)a.HID, (int)a.CZ, a.dln_w, a.dln_b);
  return hipGetLastError();
}

}  // namespace

size_t transition_bwd_workspace(int dtype, int64_t npos, int64_t CZ, int64_t HID) {
  return bwd_layout_t(dtype, npos, CZ, HID).total;
}

hipError_t launch_transition_bwd(const TransitionBwdArgs& a, hipStream_t s) {
  if (a.HID % SEG != 0 || a.CZ % 32 != 0 || a.CZ > 128) return hipErrorInvalidValue;
  return a.dtype == 1 ? transition_bwd_t<bf16_t>(a, s) : transition_bwd_t<float>(a, s);
}

}  // namespace evo
