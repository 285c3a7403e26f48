// LayerNorm + linear + SwiGLU transition on gfx950, fused.
//
// EvoFusion ("MegaFold: Efficient Training of Next-Generation 3D Attention
// Protein Models on Cross-Platform GPUs", section "Methodologie", item 3)
// restructures the layer normalisation, the linear projections and the
// SwiGLU activation so that no N x N intermediate reaches HBM.  Per pair
// position:
//   x = LN(z),  h = silu(x . W_a^T) * (x . W_b^T),  out = h . W_o^T
// (hidden width HID, silu(u) = u * sigmoid(u), no bias vectors).
//
// One kernel.  Persistent workgroups of 8 waves, 32 positions per wave:
//   - the wave's z rows are loaded in the matrix-core operand layout and
//     normalised in registers (fp32 statistics); the normalised rows stay
//     there as bf16 operands for the whole hidden loop;
//   - the hidden units are processed in chunks of 64: the chunk's W_a and
//     W_b rows (LayerNorm weight folded in, rows permuted so that the
//     products come out in the operand layout of the next product), their
//     constant terms beta . W^T, and the matching 64 columns of W_o go
//     through LDS (double-buffered, the next chunk's weights loaded while
//     this one is computed); a small kernel prepares them once per call in
//     the caller's workspace, in the order the main kernel copies them;
//   - a, b = x . W^T for the chunk, h = silu(a) * b in registers, then
//     out^T += W_o[:, chunk] . h^T; the hidden activations never leave the
//     registers and the output accumulates across chunks.
#include <algorithm>

#include "evo_device.h"
#include "evo_kernels.h"

namespace evo {
namespace {

constexpr int PW = 32;       // positions per wave
constexpr int WAVES = 8;
constexpr int PADE = 8;
// hidden units per chunk: 64 (bf16); 32 (fp32, whose double-buffered
// weights would not fit the LDS at 64)
template <typename T> constexpr int chunk_units() { return sizeof(T) == 2 ? 64 : 32; }

struct TransParams {
  int npos, CZ, HID, ntiles;
  const void* z;
  const void* ln_w;
  const void* ln_b;
  float eps;
  const void* w_a;   // [HID][CZ]
  const void* w_b;   // [HID][CZ]
  const void* w_o;   // [CZ][HID]
  void* out;         // [npos][CZ]
  // prepared once per call (workspace), per chunk q of HC hidden units:
  void* wab;         // [nq][2][HC][CZ]: W_a, W_b rows * gamma, rows permuted
  void* wo;          // [nq][CZ][HC]: the chunk's columns of W_o
  float* cst;        // [nq][2][HC]: beta . W^T, permuted like the rows
};

// Byte layout of the prepared weights in the workspace.
struct PrepLayout {
  size_t wab, wo, cst, total;  // byte offsets
};
inline PrepLayout prep_layout(int64_t CZ, int64_t HID, size_t es) {
  PrepLayout L;
  L.wab = 0;
  L.wo = ((size_t)2 * HID * CZ * es + 255) & ~size_t(255);
  L.cst = L.wo + (((size_t)HID * CZ * es + 255) & ~size_t(255));
  L.total = L.cst + (((size_t)2 * HID * 4 + 255) & ~size_t(255));
  return L;
}

// LDS row of hidden unit u of a chunk (u < 64): accumulator block
// cb = 2*(u/32) + (u%8)/4, row 4*((u%32)/8) + u%4 inside it, so that lane
// group g of blocks (2s, 2s+1) holds units 32s + 8g .. +7: the operand
// layout of the second product.
__device__ __forceinline__ int hrow_of(int u) {
  const int s = u >> 5, rem = u & 31, gg = rem >> 3, j = rem & 7;
  return 16 * (2 * s + (j >> 2)) + 4 * gg + (j & 3);
}

// Once per call: the weights in the order the main kernel copies them.  The
// constants beta . W^T are one wave per (chunk, matrix, unit), the channels
// split over the lanes and summed in a fixed order.
template <typename T>
__global__ void __launch_bounds__(256) transition_prep_kernel(TransParams p) {
  constexpr int HC = chunk_units<T>();
  const int CZ = p.CZ, HID = p.HID;
  const T* lnw = static_cast<const T*>(p.ln_w);
  const T* lnb = static_cast<const T*>(p.ln_b);
  const int64_t nw = (int64_t)2 * HID * CZ, no = (int64_t)HID * CZ;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < nw + no;
       e += (int64_t)gridDim.x * 256) {
    if (e < nw) {
      // source element (matrix m, unit h, channel k)
      const int m = (int)(e / ((int64_t)HID * CZ));
      const int64_t r = e - (int64_t)m * HID * CZ;
      const int h = (int)(r / CZ), k = (int)(r - (int64_t)h * CZ);
      const int q = h / HC, u = h - q * HC;
      const T* w = static_cast<const T*>(m == 0 ? p.w_a : p.w_b);
      const float v = Tr<T>::to_f(w[r]) * Tr<T>::to_f(lnw[k]);
      static_cast<T*>(p.wab)[(((int64_t)q * 2 + m) * HC + hrow_of(u)) * CZ + k] = Tr<T>::from_f(v);
    } else {
      const int64_t r = e - nw;  // W_o element (c, h)
      const int c = (int)(r / HID), h = (int)(r - (int64_t)c * HID);
      const int q = h / HC, u = h - q * HC;
      static_cast<T*>(p.wo)[((int64_t)q * CZ + c) * HC + u] = static_cast<const T*>(p.w_o)[r];
    }
  }
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * 4;
  for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < 2 * HID; t += nwaves) {
    const int m = t / HID, h = t - m * HID;
    const T* w = static_cast<const T*>(m == 0 ? p.w_a : p.w_b) + (int64_t)h * CZ;
    float acc = 0.f;
    for (int k = lane; k < CZ; k += 64) acc = __builtin_fmaf(Tr<T>::to_f(lnb[k]), Tr<T>::to_f(w[k]), acc);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) {
      const int q = h / HC, u = h - q * HC;
      p.cst[((int64_t)q * 2 + m) * HC + hrow_of(u)] = acc;
    }
  }
}

template <typename T, int KS>  // KS = CZ / 32
__global__ void __launch_bounds__(WAVES * 64) transition_kernel(TransParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int HC = chunk_units<T>(), NHB = HC / 16, NS2 = HC / 32;
  constexpr int CZ = KS * 32, CB = KS * 2;      // output blocks of 16
  constexpr int WRS = CZ + PADE;                // W_a/W_b row stride
  constexpr int ORS = HC + PADE;                // W_o chunk row stride
  constexpr int BUF = 2 * HC * WRS + CZ * ORS;  // elements per buffer
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sbuf = reinterpret_cast<T*>(smem);                        // [2][BUF]
  float* sC = reinterpret_cast<float*>(sbuf + 2 * BUF);        // [2][2][HC]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int nchunks = p.HID / HC;

  // The chunk's prepared weights: 16-byte loads of the contiguous prepared
  // blocks into registers at the start of a chunk (fetch_chunk), copied into
  // the padded LDS rows of the other buffer at its end (store_chunk), so the
  // loads are in flight while the chunk is computed.
  constexpr int E16 = 16 / sizeof(T);
  constexpr int NWAB = 2 * HC * CZ / E16, NWO = CZ * HC / E16;
  constexpr int PER = (NWAB + NWO + WAVES * 64 - 1) / (WAVES * 64);
  u32x4 wreg[PER];
  float creg = 0.f;
  // buffer loads: the prepared arrays' bases and sizes uniform, each lane's
  // offset fixed, the chunk's offset added per chunk
  const uint32_t wab_bytes = (uint32_t)((int64_t)nchunks * 2 * HC * CZ * sizeof(T));
  const uint32_t wo_bytes = (uint32_t)((int64_t)nchunks * CZ * HC * sizeof(T));
  auto fetch_chunk = [&](int q) {
    const uint32_t qab = (uint32_t)(q * 2 * HC * CZ * sizeof(T));
    const uint32_t qo = (uint32_t)(q * CZ * HC * sizeof(T));
    // each prepared array is contiguous: its 16-byte block e sits at byte
    // 16 e of the chunk
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + u * WAVES * 64;
      if (e < NWAB)
        wreg[u] = buf_ld128(p.wab, wab_bytes, (uint32_t)e * 16u, qab);
      else if (e < NWAB + NWO)
        wreg[u] = buf_ld128(p.wo, wo_bytes, (uint32_t)(e - NWAB) * 16u, qo);
    }
    if (tid < 2 * HC) creg = p.cst[(int64_t)q * 2 * HC + tid];
  };
  auto store_chunk = [&](int buf) {
    T* sw = sbuf + buf * BUF;
    T* so = sw + 2 * HC * WRS;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + u * WAVES * 64;
      if (e < NWAB) {
        const int row = e / (CZ / E16), col = (e - row * (CZ / E16)) * E16;
        *reinterpret_cast<u32x4*>(sw + row * WRS + col) = wreg[u];
      } else if (e < NWAB + NWO) {
        const int e2 = e - NWAB, row = e2 / (HC / E16), col = (e2 - row * (HC / E16)) * E16;
        *reinterpret_cast<u32x4*>(so + row * ORS + col) = wreg[u];
      }
    }
    if (tid < 2 * HC) sC[buf * 2 * HC + tid] = creg;
  };
  static_assert(2 * HC <= WAVES * 64, "one constant per thread");

  const T* Z = static_cast<const T*>(p.z);
  for (int tile = blockIdx.x; tile < p.ntiles; tile += gridDim.x) {
    // ---- this wave's 32 rows, normalised, as operands: xf[pb][s] holds
    // channels 32s + 8g .. +7 of position pb*16 + l16
    uint32_t pidx[2];
    bool live[2];
    Op xf[2][KS];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      pidx[pb] = ((uint32_t)tile * WAVES + wave) * PW + pb * 16 + l16;
      live[pb] = pidx[pb] < (uint32_t)p.npos;
      const T* src = Z + (int64_t)(live[pb] ? pidx[pb] : 0) * CZ + 8 * g;
      float v[KS][8];
      float sum = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Raw8<T> r;
        ld_raw8(r, src + 32 * s);
        f32x4 lo, hi;
        widen8(r, lo, hi);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[s][i] = lo[i];
          v[s][4 + i] = hi[i];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) sum += v[s][j];
      }
      sum += shfl_xor(sum, 16);
      sum += shfl_xor(sum, 32);
      const float mu = sum / CZ;
      float var = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          v[s][j] -= mu;
          var = __builtin_fmaf(v[s][j], v[s][j], var);
        }
      var += shfl_xor(var, 16);
      var += shfl_xor(var, 32);
      const float rstd = rsqrtf(var / CZ + p.eps);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Op f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if constexpr (sizeof(T) == 2) f[j] = (__bf16)(v[s][j] * rstd);
          else f[j] = v[s][j] * rstd;
        }
        xf[pb][s] = f;
      }
    }

    f32x4 acc[CB][2];  // out^T blocks [cz block][pb]
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb][0] = acc[cb][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // the previous tile's last chunk is no longer read
    fetch_chunk(0);
    store_chunk(0);
    for (int q = 0; q < nchunks; ++q) {
      const int buf = q & 1;
      __syncthreads();  // chunk q is in LDS; chunk q-1's buffer is free
      if (q + 1 < nchunks) fetch_chunk(q + 1);
      const T* sw = sbuf + buf * BUF;
      const T* so = sw + 2 * HC * WRS;
      const float* sc = sC + buf * 2 * HC;
      // a, b for the chunk: 4 blocks of 16 units x 2 position blocks each
      f32x4 ua[NHB][2], ub[NHB][2];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const f32x4 ca = *reinterpret_cast<const f32x4*>(sc + hb * 16 + 4 * g);
        const f32x4 cbv = *reinterpret_cast<const f32x4*>(sc + HC + hb * 16 + 4 * g);
        ua[hb][0] = ua[hb][1] = ca;
        ub[hb][0] = ub[hb][1] = cbv;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const Op fa = *reinterpret_cast<const Op*>(sw + (hb * 16 + l16) * WRS + 32 * s + 8 * g);
          const Op fb = *reinterpret_cast<const Op*>(sw + (HC + hb * 16 + l16) * WRS + 32 * s + 8 * g);
          ua[hb][0] = mma32(fa, xf[0][s], ua[hb][0]);
          ua[hb][1] = mma32(fa, xf[1][s], ua[hb][1]);
          ub[hb][0] = mma32(fb, xf[0][s], ub[hb][0]);
          ub[hb][1] = mma32(fb, xf[1][s], ub[hb][1]);
        }
      }
      // h = silu(a) * b; lane (l16, g) of blocks (2s2, 2s2+1) holds units
      // 32 s2 + 8g .. +7 of position pb*16 + l16: the second product's
      // operand for contraction step s2
#pragma unroll
      for (int s2 = 0; s2 < NS2; ++s2) {
        Op hf[2];
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
          float h[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float u = ua[2 * s2 + (j >> 2)][pb][j & 3];
            const float b = ub[2 * s2 + (j >> 2)][pb][j & 3];
            h[j] = u * b * rcp_fast(1.f + exp2_fast(-u * kLog2e));
          }
          Op f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if constexpr (sizeof(T) == 2) f[j] = (__bf16)h[j];
            else f[j] = h[j];
          }
          hf[pb] = f;
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const Op wo = *reinterpret_cast<const Op*>(so + (cb * 16 + l16) * ORS + 32 * s2 + 8 * g);
          acc[cb][0] = mma32(wo, hf[0], acc[cb][0]);
          acc[cb][1] = mma32(wo, hf[1], acc[cb][1]);
        }
      }
      if (q + 1 < nchunks) store_chunk(buf ^ 1);
    }
    // lane (l16, g) holds out[position pb*16 + l16][cb*16 + 4g + i]
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      if (!live[pb]) continue;
      T* dst = static_cast<T*>(p.out) + (int64_t)pidx[pb] * CZ + 4 * g;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if constexpr (sizeof(T) == 2) {
          uint2 u;
          u.x = uint32_t(Tr<bf16_t>::from_f(acc[cb][pb][0])) |
                (uint32_t(Tr<bf16_t>::from_f(acc[cb][pb][1])) << 16);
          u.y = uint32_t(Tr<bf16_t>::from_f(acc[cb][pb][2])) |
                (uint32_t(Tr<bf16_t>::from_f(acc[cb][pb][3])) << 16);
          *reinterpret_cast<uint2*>(dst + cb * 16) = u;
        } else {
          *reinterpret_cast<float4*>(dst + cb * 16) =
              make_float4(acc[cb][pb][0], acc[cb][pb][1], acc[cb][pb][2], acc[cb][pb][3]);
        }
      }
    }
  }
}

template <typename T, int KS>
hipError_t launch_ks(TransParams& p, hipStream_t s) {
  constexpr int CZ = KS * 32, HC = chunk_units<T>();
  const size_t lds = 2 * (size_t)(2 * HC * (CZ + PADE) + CZ * (HC + PADE)) * sizeof(T) +
                     2 * 2 * HC * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&transition_kernel<T, KS>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int grid = std::min(p.ntiles, 256);
  hipLaunchKernelGGL((transition_kernel<T, KS>), dim3(grid), dim3(WAVES * 64), lds, s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t transition_t(const TransitionArgs& a, hipStream_t s) {
  TransParams p{};
  const PrepLayout L = prep_layout(a.CZ, a.HID, sizeof(T));
  char* ws = static_cast<char*>(a.workspace);
  p.wab = ws + L.wab;
  p.wo = ws + L.wo;
  p.cst = reinterpret_cast<float*>(ws + L.cst);
  p.npos = (int)a.npos;
  p.CZ = (int)a.CZ;
  p.HID = (int)a.HID;
  p.ntiles = (int)((a.npos + PW * WAVES - 1) / (PW * WAVES));
  p.z = a.z; p.ln_w = a.ln_w; p.ln_b = a.ln_b; p.eps = a.eps;
  p.w_a = a.w_a; p.w_b = a.w_b; p.w_o = a.w_o; p.out = a.out;
  hipLaunchKernelGGL(transition_prep_kernel<T>, dim3(256), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (p.CZ / 32) {
    case 1: return launch_ks<T, 1>(p, s);
    case 2: return launch_ks<T, 2>(p, s);
    case 3: return launch_ks<T, 3>(p, s);
    case 4: return launch_ks<T, 4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t transition_workspace(int dtype, int64_t CZ, int64_t HID) {
  return prep_layout(CZ, HID, dtype == 1 ? 2 : 4).total;
}

hipError_t launch_transition(const TransitionArgs& a, hipStream_t s) {
  return a.dtype == 1 ? transition_t<bf16_t>(a, s) : transition_t<float>(a, s);
}

}  // namespace evo
