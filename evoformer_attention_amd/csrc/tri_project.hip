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
// Both are a row GEMM  Y[pos, :] = f(X[pos, :]) . W^T  over the N*N positions
// (W in [out, in] layout).  Kernel structure:
//   - persistent workgroups, one per CU (16 waves up to 128 input channels,
//     else 8); each loads W^T (all output columns of one pass, padded rows)
//     into LDS once and then walks tiles of 32 positions per wave;
//   - a wave owns 32 positions: it loads their rows straight into the MFMA
//     B-operand layout (lane = position, 8 consecutive input channels per
//     contraction step), computes LayerNorm there (cross-lane sums over the
//     4 lane groups of a position) and keeps the normalised rows as bf16
//     fragments in registers - f(X) never touches LDS or HBM;
//   - for each block of 16 output columns: Y^T = W^T . f(X)^T on
//     v_mfma_f32_16x16x32 (A = W^T rows from LDS), so each lane ends up with
//     4 consecutive output channels of one position, stored as one 8- or
//     16-byte write.
//
// Orientation: position (line a, place n) of the line layout is z[a, n] for
// the starting node and z[n, a] for the ending node (line = a column of z).
// The pair bias of position (a, n) goes to bias[h][a*N + n] in both cases.
#include <algorithm>

#include "evo_device.h"
#include "evo_kernels.h"

namespace evo {
namespace {

constexpr int PW = 32;              // positions per wave
// Waves per workgroup: one workgroup per CU (W^T fills the LDS), so its wave
// count is the CU's occupancy.  16 waves (4 per SIMD) fit the register file
// up to K = 128 input channels; wider inputs use 8.
template <int KSTEPS> constexpr int waves_for() { return KSTEPS <= 4 ? 16 : 8; }
constexpr int PAD = 8;              // LDS row padding (elements)
constexpr size_t kLdsBudget = 150 * 1024;
constexpr int OS = 24;               // operand mode: staging row stride (elements)

struct GemmParams {
  int mode;        // 0 = project (LayerNorm + q,k,v,g,bias), 1 = out projection,
                   // 2 = multiplicative-update operands (LayerNorm + a, b)
  int N, K, HC, H, ending, ncols;   // ncols: all output columns
  int col0, pass_cols;              // this launch's column range (multiple of 16)
  int64_t npos;
  int ntiles;
  const void* x;   // z [N,N,K] (project) or O [N*N, K] (out projection)
  const void* ln_w;
  const void* ln_b;
  float eps;
  const void* w[5];     // [out, in]: project w_q, w_k, w_v, w_g [HC,K], w_bias [H,K];
                        // out projection: w_o [ncols, K]
  const void* colbias;  // project: b_g [HC] (gate columns); out: b_o [ncols]
  void* y[5];           // project: q, k, v, g [npos, HC], bias [H, npos]
                        // out projection: out [npos, ncols] in z layout
                        // operands: a, b, element (channel c, line, place) at
                        // c*s_ch + line*s_line + place*s_place (zero where
                        // the place is masked)
  const uint8_t* mask;  // operands: keep flags per place, or null
  int P, L;             // operands: places per line, lines (npos = P * L)
  int64_t s_ch, s_line, s_place;
  int64_t frag_kp;      // operands: > 0, a in fragment order (frag_off)
};

// z row (or output row) of line-layout position pidx (N*N < 2^31, so 32-bit
// index arithmetic).
__device__ __forceinline__ uint32_t z_row(uint32_t pidx, uint32_t N, int ending) {
  if (!ending) return pidx;
  const uint32_t a = pidx / N, n = pidx - a * N;
  return n * N + a;
}

// Line-layout position of element j (0..31) of wave `wave` in tile `tile`
// (WAVES*32 consecutive positions per tile); `live` is false past the end.
template <int WAVES, int PWV = PW>
__device__ __forceinline__ uint32_t tile_pos(const GemmParams& p, int tile, int wave, int j,
                                             bool& live) {
  const uint32_t pi = ((uint32_t)tile * WAVES + wave) * PWV + j;
  live = pi < (uint32_t)p.npos;
  return pi;
}

template <typename T>
__device__ __forceinline__ const T* w_row(const GemmParams& p, int c) {
  if (c >= p.ncols) return nullptr;
  if (p.mode == 1) return static_cast<const T*>(p.w[0]) + (int64_t)c * p.K;
  const int m = c / p.HC;
  if (m < 4) return static_cast<const T*>(p.w[m]) + (int64_t)(c - m * p.HC) * p.K;
  return static_cast<const T*>(p.w[4]) + (int64_t)(c - 4 * p.HC) * p.K;
}

template <typename T>
__device__ __forceinline__ void st4(T* p, const f32x4& v);
template <>
__device__ __forceinline__ void st4<bf16_t>(bf16_t* p, const f32x4& v) {
  uint2 u;
  u.x = uint32_t(Tr<bf16_t>::from_f(v[0])) | (uint32_t(Tr<bf16_t>::from_f(v[1])) << 16);
  u.y = uint32_t(Tr<bf16_t>::from_f(v[2])) | (uint32_t(Tr<bf16_t>::from_f(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}
template <>
__device__ __forceinline__ void st4<float>(float* p, const f32x4& v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// Store two adjacent 16-column blocks A (columns 0..15) and B (16..31) of
// one position row.  A lane of row group g (lanes 16g..16g+15) holds
// columns 4g..4g+3 of each.  v_permlane16_swap(x, y) exchanges the odd row
// groups of x with the even row groups of y (measured on gfx950: x becomes
// [x.r0, y.r0, x.r2, y.r2] and y [x.r1, y.r1, x.r3, y.r3]); with x = A and
// y = B, an even-g lane then holds columns 4g..4g+7 of A and an odd-g lane
// columns 4(g-1)..4g+3 of B, one contiguous 8-element chunk each, and a
// wave's store covers 16 positions x 64 contiguous bytes (bf16) instead of
// 16 x 32.  Every lane takes part in the swap; `live` only gates the store.
__device__ __forceinline__ void swap_rows16(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}
template <typename T>
__device__ __forceinline__ void store_pair(T* row, const f32x4& a, const f32x4& b, int g,
                                           bool live);
template <>
__device__ __forceinline__ void store_pair<bf16_t>(bf16_t* row, const f32x4& a, const f32x4& b,
                                                   int g, bool live) {
  auto pk = [](float x, float y) {
    return uint32_t(Tr<bf16_t>::from_f(x)) | (uint32_t(Tr<bf16_t>::from_f(y)) << 16);
  };
  uint32_t x0 = pk(a[0], a[1]), x1 = pk(a[2], a[3]);
  uint32_t y0 = pk(b[0], b[1]), y1 = pk(b[2], b[3]);
  swap_rows16(x0, y0);
  swap_rows16(x1, y1);
  if (live)
    *reinterpret_cast<u32x4*>(row + ((g & 1) ? 16 + 4 * (g - 1) : 4 * g)) = u32x4{x0, x1, y0, y1};
}
template <>
__device__ __forceinline__ void store_pair<float>(float* row, const f32x4& a, const f32x4& b,
                                                  int g, bool live) {
  u32x4 x, y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t xi = __float_as_uint(a[i]), yi = __float_as_uint(b[i]);
    swap_rows16(xi, yi);
    x[i] = xi;
    y[i] = yi;
  }
  if (live) {
    u32x4* dst = reinterpret_cast<u32x4*>(row + ((g & 1) ? 16 + 4 * (g - 1) : 4 * g));
    dst[0] = x;
    dst[1] = y;
  }
}

// MUL: the multiplicative-update operand mode (p.mode == 2), a separate
// instantiation so that the other modes' code is unchanged by it.
// SPLIT (bf16 projection, p.mode == 0): the LayerNorm output y = xhat * gamma
// + beta is formed in fp32 and handed to the matrix cores as two bf16
// operands, hi = bf16(y) and lo = bf16(y - hi) (16 significant bits), against
// the unmodified bf16 weights: the projection is then exact up to fp32
// accumulation before its one rounding to the output type, instead of
// rounding y (and W * gamma) to bf16 first.  Twice the products and the
// operand registers: up to 128 input channels, 16 positions per wave and
// 16 waves per workgroup (four per SIMD); up to 160, 32 positions and eight
// waves (wider inputs keep the single rounded operand).
template <typename T, int KSTEPS, int WAVES = waves_for<KSTEPS>(), bool MUL = false,
          bool SPLIT = false, int PB = 2>
__global__ void __launch_bounds__(WAVES * 64)
rowgemm_kernel(GemmParams p) {
  // PB: 16-position blocks per wave (1 only for the split operands)
  static_assert(PB == 2 || (SPLIT && PB == 1), "one block per wave only with split operands");
  constexpr int PWV = 16 * PB;        // positions per wave
  using Op = typename Tr<T>::Op;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int K = KSTEPS * 32;
  const int KS = K + PAD;
  T* sW = reinterpret_cast<T*>(smem);                           // [pass_cols][KS]
  float* sC = reinterpret_cast<float*>(sW + p.pass_cols * KS);  // [pass_cols]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  // operand mode (bf16): per wave, one 32-position x 16-channel block staged
  // row by position, read back channel by channel
  T* sO = reinterpret_cast<T*>(sC + p.pass_cols) + (MUL ? wave * 32 * OS : 0);
  // SPLIT: gamma and beta of the K input channels, after the column constants
  T* sG = reinterpret_cast<T*>(sC + p.pass_cols);

  const T* X = static_cast<const T*>(p.x);
  // Rows of position `pi` as loaded: channels 32s + 8g .. +7 in nx[s].
  // Positions past the end read row 0 (finite; never stored).
  auto load_rows = [&](Op (&nx)[PB][KSTEPS], int tile) {
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      bool live;
      const uint32_t pi = tile_pos<WAVES, PWV>(p, tile, wave, pb * 16 + l16, live);
      uint32_t row = 0;
      if (live) {
        if constexpr (MUL) {
          // operands: line-major positions; transposed rows are place * L + line
          const uint32_t ln = pi / (uint32_t)p.P, pl = pi - ln * (uint32_t)p.P;
          row = p.ending ? pl * (uint32_t)p.L + ln : pi;
        } else {
          row = p.mode != 1 ? z_row(pi, p.N, p.ending) : pi;
        }
      }
      const T* src = X + (int64_t)row * K + 8 * g;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) nx[pb][s] = *reinterpret_cast<const Op*>(src + 32 * s);
    }
  };
  // bf16: the next tile's rows are in flight during this tile, the first
  // tile's during the weight set-up (fp32 rows would not fit the register
  // budget and are loaded at the tile's start)
  constexpr bool PREFETCH = sizeof(T) == 2;
  Op nx[PB][KSTEPS];
  if (PREFETCH && blockIdx.x < p.ntiles) load_rows(nx, blockIdx.x);

  // ---- This pass's weights into LDS, with the LayerNorm affine folded in:
  // LN(x) . W^T = xhat . (W diag(gamma))^T + beta . W^T, xhat = (x - mu) *
  // rstd.  sW holds W diag(gamma) (rounded to the working dtype), sC the
  // per-column constant beta . W^T plus the column bias (gate or output).
  const T* lnw = static_cast<const T*>(p.ln_w);
  const T* lnb = static_cast<const T*>(p.ln_b);
  {
    // One chunk = 8 input channels of one column: a vector load of W and one
    // of gamma; four chunks per thread are in flight before any is used.
    const int chunks = K / 8;
    const int total = p.pass_cols * chunks;
    const int nthr = WAVES * 64;
    for (int e0 = tid; e0 < total; e0 += 4 * nthr) {
      Raw8<T> wr[4], gr[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * nthr;
        const int cl = e / chunks, k0 = (e - cl * chunks) * 8;
        const T* src = e < total ? w_row<T>(p, p.col0 + cl) : nullptr;
        if (src) {
          ld_raw8(wr[u], src + k0);
          if (p.mode != 1 && !SPLIT) ld_raw8(gr[u], lnw + k0);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * nthr;
        if (e >= total) break;
        const int cl = e / chunks, k0 = (e - cl * chunks) * 8;
        f32x4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = w0;
        if (w_row<T>(p, p.col0 + cl)) {
          widen8(wr[u], w0, w1);
          if (p.mode != 1 && !SPLIT) {
            f32x4 g0, g1;
            widen8(gr[u], g0, g1);
            w0 *= g0;
            w1 *= g1;
          }
        }
        T* dst = sW + cl * KS + k0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dst[j] = Tr<T>::from_f(w0[j]);
          dst[4 + j] = Tr<T>::from_f(w1[j]);
        }
      }
    }
    // Column constants, one thread per column: beta . W^T summed in channel
    // order (fixed order, deterministic), plus the column bias.
    for (int cl = tid; cl < p.pass_cols; cl += nthr) {
      const int c = p.col0 + cl;
      const T* src = w_row<T>(p, c);
      float acc = 0.f;
      if (src && p.mode != 1 && !SPLIT) {
#pragma unroll 4
        for (int k0 = 0; k0 < K; k0 += 8) {
          Raw8<T> wr, br;
          ld_raw8(wr, src + k0);
          ld_raw8(br, lnb + k0);
          f32x4 w0, w1, b0, b1;
          widen8(wr, w0, w1);
          widen8(br, b0, b1);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc = __builtin_fmaf(b0[j], w0[j], acc);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc = __builtin_fmaf(b1[j], w1[j], acc);
        }
      }
      if (src && p.colbias && p.mode != 2) {
        if (p.mode == 1) acc += Tr<T>::to_f(static_cast<const T*>(p.colbias)[c]);
        else if (c >= 3 * p.HC && c < 4 * p.HC)
          acc += Tr<T>::to_f(static_cast<const T*>(p.colbias)[c - 3 * p.HC]);
      }
      sC[cl] = acc;
    }
    if constexpr (SPLIT) {
      for (int c = tid; c < K; c += WAVES * 64) {
        sG[c] = lnw[c];
        sG[K + c] = lnb[c];
      }
    }
  }
  __syncthreads();

  // output matrix and column within it where this pass starts (passes start
  // at multiples of 32 columns, so never inside a block pair)
  const int m0 = p.mode == 0 ? min(p.col0 / p.HC, 4) : p.mode == 2 ? p.col0 / p.HC : 0;
  // operand mode: 8 consecutive positions from a multiple of 8 are 8
  // consecutive, 16-byte aligned places of one line
  const bool vec_ok = MUL && p.s_place == 1 && p.P % 8 == 0 && p.s_ch % 8 == 0 &&
                      p.s_line % 8 == 0;
  const int cbase0 = p.col0 - m0 * p.HC;
  for (int tile = blockIdx.x; tile < p.ntiles; tile += gridDim.x) {
    if (!PREFETCH) load_rows(nx, tile);
    // ---- this wave's 16 * PB rows, in B-operand layout: xf[pb][s] holds
    // channels 32s + 8g .. +7 of position base + pb*16 + l16 (SPLIT: the hi
    // part; xl the lo part).
    Op xf[PB][KSTEPS];
    Op xl[SPLIT ? PB : 1][SPLIT ? KSTEPS : 1];
    uint32_t pidx[PB];
    int64_t orow[PB];
    bool live[PB];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      pidx[pb] = tile_pos<WAVES, PWV>(p, tile, wave, pb * 16 + l16, live[pb]);
      // output row offset: line layout (project) or z layout (out projection)
      orow[pb] = p.mode == 0 ? (int64_t)pidx[pb] * p.HC
                             : (int64_t)(live[pb] ? z_row(pidx[pb], p.N, p.ending) : 0) * p.ncols;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) xf[pb][s] = nx[pb][s];  // raw rows
    }
    if (PREFETCH && tile + (int)gridDim.x < p.ntiles) load_rows(nx, tile + gridDim.x);
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      float v[1][KSTEPS][8];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[0][s][j] = (float)xf[pb][s][j];
      if (p.mode != 1) {
        // two-pass statistics in fp32 (population variance), centred in place
        float sum = 0.f;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j) sum += v[0][s][j];
        sum += shfl_xor(sum, 16);
        sum += shfl_xor(sum, 32);
        const float mu = sum / K;
        float var = 0.f;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            v[0][s][j] -= mu;
            var = __builtin_fmaf(v[0][s][j], v[0][s][j], var);
          }
        var += shfl_xor(var, 16);
        var += shfl_xor(var, 32);
        const float rstd = rsqrtf(var / K + p.eps);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j) v[0][s][j] *= rstd;
      }
      if constexpr (SPLIT) {
        // y = xhat * gamma + beta in fp32, as hi + lo bf16 operands
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          Raw8<T> gr, br;
          ld_raw8(gr, sG + 32 * s + 8 * g);
          ld_raw8(br, sG + K + 32 * s + 8 * g);
          f32x4 g0, g1, b0, b1;
          widen8(gr, g0, g1);
          widen8(br, b0, b1);
          Op hi, lo;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float y = __builtin_fmaf(v[0][s][j], j < 4 ? g0[j] : g1[j - 4], j < 4 ? b0[j] : b1[j - 4]);
            const __bf16 h = (__bf16)y;
            hi[j] = h;
            lo[j] = (__bf16)(y - (float)h);
          }
          xf[pb][s] = hi;
          xl[pb][s] = lo;
          // keep the next step's gamma/beta loads here (hoisting them all
          // ahead costs registers)
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          Op f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if constexpr (sizeof(T) == 2) f[j] = (__bf16)v[0][s][j];
            else f[j] = v[0][s][j];
          }
          xf[pb][s] = f;
        }
      }
    }

    // ---- Y^T in blocks of 16 output columns, output matrix by output
    // matrix (projection: q, k, v, g, then the pair bias; out projection:
    // one), two blocks at a time where both belong to one matrix (see
    // store_pair).  The accumulators start from the column constants.
    const int nblk = p.pass_cols / 16;
    for (int cb = 0, m = m0, cbase = cbase0; cb < nblk; ++m, cbase = 0) {
      const bool bias_out = p.mode == 0 && m == 4;
      const int width = p.mode == 1 ? p.ncols : (bias_out ? p.H : p.HC);
      T* out = static_cast<T*>(p.y[p.mode == 1 ? 0 : m]);  // mode 2: a, then b
      while (cb < nblk && cbase < width) {
        const bool pair = !MUL && !bias_out && cb + 1 < nblk && cbase + 32 <= width;
        f32x4 acc[2][PB];  // [block][pb]
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (j == 1 && !pair) break;
          const f32x4 cc4 = *reinterpret_cast<const f32x4*>(sC + (cb + j) * 16 + 4 * g);
#pragma unroll
          for (int pb = 0; pb < PB; ++pb) acc[j][pb] = cc4;
          const T* wr = sW + ((cb + j) * 16 + l16) * KS + 8 * g;
#pragma unroll
          for (int s = 0; s < KSTEPS; ++s) {
            const Op a = *reinterpret_cast<const Op*>(wr + 32 * s);
            if constexpr (SPLIT) {
#pragma unroll
              for (int pb = 0; pb < PB; ++pb) {
                acc[j][pb] = mma32(a, xl[pb][s], acc[j][pb]);
                acc[j][pb] = mma32(a, xf[pb][s], acc[j][pb]);
              }
            } else {
              acc[j][0] = mma32(a, xf[0][s], acc[j][0]);
              acc[j][1] = mma32(a, xf[1][s], acc[j][1]);
            }
          }
        }
        if (pair) {
#pragma unroll
          for (int pb = 0; pb < PB; ++pb)
            store_pair<T>(out + orow[pb] + cbase, acc[0][pb], acc[1][pb], g, live[pb]);
          cb += 2;
          cbase += 32;
          continue;
        }
        if constexpr (MUL && sizeof(T) == 2) {
          // Through the wave's staging tile: lane (l16, g) then holds channel
          // cbase + l16 of the 8 consecutive positions 8g .. 8g+7 of the
          // wave's 32, stored as one 16-byte run where they are consecutive
          // places of one line.
#pragma unroll
          for (int pb = 0; pb < 2; ++pb) {
            uint2 u;
            u.x = uint32_t(Tr<T>::from_f(acc[0][pb][0])) | (uint32_t(Tr<T>::from_f(acc[0][pb][1])) << 16);
            u.y = uint32_t(Tr<T>::from_f(acc[0][pb][2])) | (uint32_t(Tr<T>::from_f(acc[0][pb][3])) << 16);
            *reinterpret_cast<uint2*>(sO + (pb * 16 + l16) * OS + 4 * g) = u;
          }
          __builtin_amdgcn_wave_barrier();
          const T* q0 = sO + (8 * g + (l16 >> 2)) * OS + 4 * (l16 & 3);
          u32x4 v = __builtin_bit_cast(u32x4, lds_read_tr_op(q0, q0 + 4 * OS));
          const int c = cbase + l16;
          const uint32_t pi0 = ((uint32_t)tile * WAVES + wave) * PW + 8 * g;
          if (c < p.HC && pi0 < (uint32_t)p.npos) {
            uint32_t line = pi0 / (uint32_t)p.P, place = pi0 - line * (uint32_t)p.P;
            T* base = out + (int64_t)c * p.s_ch;
            // a in fragment order: row (c s_ch + line s_line) / frag_kp
            const bool frag = m == 0 && p.frag_kp > 0;
            if (vec_ok && pi0 + 8 <= (uint32_t)p.npos) {
              if (p.mask) {  // 8 keep flags, 8-byte aligned: zero the dead places
                const uint2 mb = *reinterpret_cast<const uint2*>(p.mask + place);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const uint32_t w = (i < 2 ? mb.x : mb.y) >> (16 * (i & 1));
                  v[i] &= ((w & 0xffu) ? 0xffffu : 0u) | ((w & 0xff00u) ? 0xffff0000u : 0u);
                }
              }
              if (frag)
                *reinterpret_cast<u32x4*>(
                    out + frag_off(((int64_t)c * p.s_ch + (int64_t)line * p.s_line) / p.frag_kp,
                                   (int)place, (int)p.frag_kp)) = v;
              else
                *reinterpret_cast<u32x4*>(base + (int64_t)line * p.s_line + place) = v;
            } else {
              // ragged: element by element, walking the places of the line
#pragma nounroll
              for (int j = 0; j < 8; ++j) {
                if (pi0 + j >= (uint32_t)p.npos) break;
                const bool dead = p.mask && p.mask[place] == 0;
                const uint32_t word = j < 2 ? v[0] : j < 4 ? v[1] : j < 6 ? v[2] : v[3];
                const uint32_t bits = (word >> (16 * (j & 1))) & 0xffffu;
                const T val = dead ? T(0) : __builtin_bit_cast(T, (uint16_t)bits);
                if (frag)
                  out[frag_off(((int64_t)c * p.s_ch + (int64_t)line * p.s_line) / p.frag_kp,
                               (int)place, (int)p.frag_kp)] = val;
                else
                  base[(int64_t)line * p.s_line + (int64_t)place * p.s_place] = val;
                if (++place == (uint32_t)p.P) { place = 0; ++line; }
              }
            }
          }
          __builtin_amdgcn_wave_barrier();
          cb += 1;
          cbase += 16;
          continue;
        }
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
          if (!live[pb]) continue;
          const int c = cbase + 4 * g;
          if constexpr (MUL && sizeof(T) != 2) {
            // element (line, place) of channel c+i
            const uint32_t line = pidx[pb] / (uint32_t)p.P, place = pidx[pb] - line * (uint32_t)p.P;
            const bool dead = p.mask && p.mask[place] == 0;
            T* dst = out + (int64_t)line * p.s_line + (int64_t)place * p.s_place;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (c + i < p.HC) dst[(c + i) * p.s_ch] = Tr<T>::from_f(dead ? 0.f : acc[0][pb][i]);
          } else if (!bias_out) {
            st4<T>(out + orow[pb] + c, acc[0][pb]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (c + i < p.H) out[(int64_t)(c + i) * p.npos + pidx[pb]] = Tr<T>::from_f(acc[0][pb][i]);
          }
        }
        cb += 1;
        cbase += 16;
      }
      if (p.mode == 1 || m == 4 || (MUL && m == 1)) break;
    }
  }
}

template <typename T, int KSTEPS, bool MUL, bool SPLIT = false>
hipError_t launch_pass_m(GemmParams& p, size_t lds, hipStream_t s) {
  // split operands: 16 positions per wave up to 128 input channels (16
  // waves), 32 positions and 8 waves above
  constexpr int PB = SPLIT && KSTEPS <= 4 ? 1 : 2;
  constexpr int WAVES = SPLIT ? (PB == 1 ? 16 : 8) : waves_for<KSTEPS>();
  constexpr int PWV = 16 * PB;
  const int64_t tiles = (p.npos + PWV * WAVES - 1) / (PWV * WAVES);
  if (tiles > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  p.ntiles = (int)tiles;
  const int grid = (int)std::min<int64_t>(tiles, 256);  // persistent: one per CU
  hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&rowgemm_kernel<T, KSTEPS, WAVES, MUL, SPLIT, PB>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((rowgemm_kernel<T, KSTEPS, WAVES, MUL, SPLIT, PB>), dim3(grid), dim3(WAVES * 64), lds,
                     s, p);
  return hipGetLastError();
}

template <typename T, int KSTEPS>
hipError_t launch_pass(GemmParams& p, size_t lds, hipStream_t s) {
  if (p.mode == 2) return launch_pass_m<T, KSTEPS, true>(p, lds, s);
  // split operands up to 160 input channels (beyond, their registers spill)
  if (p.mode == 0 && sizeof(T) == 2 && KSTEPS <= 5)
    return launch_pass_m<T, KSTEPS, false, true>(p, lds, s);
  return launch_pass_m<T, KSTEPS, false>(p, lds, s);
}

template <typename T>
hipError_t launch_gemm(GemmParams& p, hipStream_t s) {
  // LDS per output column: its weight row and its constant
  const size_t row_bytes = (size_t)(p.K + PAD) * sizeof(T) + sizeof(float);
  // operand mode: the per-wave staging tiles (at most 16 waves); bf16
  // projection: gamma and beta
  const size_t stage = p.mode == 2 ? (size_t)16 * 32 * OS * sizeof(T)
                       : (p.mode == 0 && sizeof(T) == 2 && p.K <= 160) ? (size_t)2 * p.K * sizeof(T)
                                                                      : 0;
  int per_pass = (int)((kLdsBudget - stage) / row_bytes) / 32 * 32;  // whole block pairs
  const int ncols_pad = (p.ncols + 15) / 16 * 16;
  per_pass = std::min(per_pass, ncols_pad);
  for (int c0 = 0; c0 < p.ncols; c0 += per_pass) {
    p.col0 = c0;
    p.pass_cols = std::min(per_pass, ncols_pad - c0);
    const size_t lds = (size_t)p.pass_cols * row_bytes + stage;
    hipError_t e;
    switch (p.K / 32) {
      case 1: e = launch_pass<T, 1>(p, lds, s); break;
      case 2: e = launch_pass<T, 2>(p, lds, s); break;
      case 3: e = launch_pass<T, 3>(p, lds, s); break;
      case 4: e = launch_pass<T, 4>(p, lds, s); break;
      case 5: e = launch_pass<T, 5>(p, lds, s); break;
      case 6: e = launch_pass<T, 6>(p, lds, s); break;
      case 7: e = launch_pass<T, 7>(p, lds, s); break;
      case 8: e = launch_pass<T, 8>(p, lds, s); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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

hipError_t launch_channel_project(const ChannelProjectArgs& a, hipStream_t s) {
  GemmParams p{};
  p.mode = 2;
  p.N = (int)a.L;
  p.K = (int)a.CZ;
  p.HC = (int)a.C;
  p.H = 1;
  p.ending = a.transposed;
  p.ncols = 2 * p.HC;
  p.npos = a.L * a.P;
  p.x = a.z;
  p.ln_w = a.ln_w;
  p.ln_b = a.ln_b;
  p.eps = a.eps;
  p.w[0] = a.w_a;
  p.w[1] = a.w_b;
  p.colbias = nullptr;
  p.y[0] = a.a;
  p.y[1] = a.b;
  p.mask = a.mask;
  p.P = (int)a.P;
  p.L = (int)a.L;
  p.s_ch = a.s_ch;
  p.s_line = a.s_line;
  p.s_place = a.s_place;
  p.frag_kp = a.a_frag_kp;
  if (p.frag_kp > 0 && (a.dtype != 1 || a.s_place != 1 || p.frag_kp % 32 != 0))
    return hipErrorInvalidValue;
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
