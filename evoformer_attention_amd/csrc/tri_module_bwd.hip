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

// NSEG = 4 (the module: q, k, v, gate segments, then the pair-bias block,
// LayerNorm backward), 2 (two segments and the LayerNorm backward, no
// pair-bias block: the multiplicative update's a and b) or 1 (the output
// projection: one z-layout segment, dX written).  Eight waves, 32 positions
// per wave per tile.
// FULL: segments 128 wide (four 32-wide steps, folded at compile time).
template <typename T, int CB, int NSEG, bool FULL = false>
__global__ void __launch_bounds__(512) rowgrad_kernel(RowGradParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int WAVES = 8;
  constexpr bool LN = NSEG != 1;  // LayerNorm backward (and with NSEG 4 the pair-bias block)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sW = reinterpret_cast<T*>(smem);  // [cout][kc + PADE]
  const int KCS = p.kc + PADE;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int cout = p.cout;  // 16 * CB
  const int segK = NSEG * p.seg_w;
  const int seg_steps = FULL ? 4 : p.seg_w / 32;  // 1..4

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

  // Positions of a tile (past the end: position 0, finite, never stored).
  struct Pos {
    uint32_t pc[2], inrow[2];
    bool live[2];
  };
  auto pos_of = [&](int tile) {
    Pos q;
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      const uint32_t pidx = ((uint32_t)tile * WAVES + wave) * PW + pb * 16 + l16;
      q.live[pb] = pidx < (uint32_t)p.npos;
      q.pc[pb] = q.live[pb] ? pidx : 0u;
      q.inrow[pb] = p.in_zrow ? zrow_of(q.pc[pb], p.N, p.ending) : q.pc[pb];
    }
    return q;
  };
  // Segment s of a tile: the lane's 8 consecutive contraction values
  // 32u + 8g .. +7 of its two positions, all steps of the segment.
  auto load_seg = [&](Op (&x)[4][2], int s, const Pos& q) {
    const T* src0 = static_cast<const T*>(p.seg[s]) + (int64_t)q.inrow[0] * p.seg_w + 8 * g;
    const T* src1 = static_cast<const T*>(p.seg[s]) + (int64_t)q.inrow[1] * p.seg_w + 8 * g;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < seg_steps) {
        x[u][0] = ld_op<T>(src0 + 32 * u);
        x[u][1] = ld_op<T>(src1 + 32 * u);
      }
  };

  f32x4 acc[CB][2];
  // acc += W_ext[:, kb .. kb+31] . x^T for both position blocks
  auto mma_step = [&](int kb, const Op (&x)[2]) {
    const T* wr = sW + kb + 8 * g;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const Op a = ld_op<T>(wr + (cb * 16 + l16) * KCS);
      acc[cb][0] = mma32(a, x[0], acc[cb][0]);
      acc[cb][1] = mma32(a, x[1], acc[cb][1]);
    }
  };
  auto comp_seg = [&](const Op (&x)[4][2], int s) {
    if (!p.resident) {
      __syncthreads();  // every wave is done with the previous chunk
      load_w(s * p.seg_w, p.seg_w);
      __syncthreads();
    }
    const int kb = p.resident ? s * p.seg_w : 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < seg_steps) {
        mma_step(kb + 32 * u, x[u]);
        // one step's weight fragments live at a time (register budget)
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  // The pair-bias block: slot j' = 8g + j holds the high part of dBias[j']
  // (j' < H) or the low part of dBias[j' - H] (j' < 2H); raw fp32 values.
  auto load_bias = [&](float (&b)[2][8], const Pos& q) {
#pragma unroll
    for (int pb = 0; pb < 2; ++pb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int slot = 8 * g + j;
        b[pb][j] = slot < 2 * p.H ? p.dbias[(int64_t)(slot % p.H) * p.npos + q.pc[pb]] : 0.f;
      }
  };
  auto comp_bias = [&](const float (&b)[2][8]) {
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
        const float d = b[pb][j];
        if constexpr (sizeof(T) == 2) {
          const float hi = (float)(__bf16)d;
          v[j] = slot < p.H ? hi : d - hi;  // d - hi is exact in fp32; 0 past 2H
        } else {
          v[j] = slot < p.H ? d : 0.f;
        }
      }
      xb[pb] = to_op(v, (Op*)nullptr);
    }
    mma_step(p.resident ? segK : 0, xb);
  };
  // The z rows of a tile's positions (LayerNorm backward), as loaded.
  using ZRaw = Raw8<T>;
  auto load_z = [&](ZRaw (&zr)[2][CB / 2], const Pos& q) {
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      const uint32_t row = zrow_of(q.pc[pb], p.N, p.ending);
      const T* src = static_cast<const T*>(p.z) + (int64_t)row * cout + 8 * g;
#pragma unroll
      for (int s = 0; s < CB / 2; ++s) ld_raw8(zr[pb][s], src + 32 * s);
    }
  };

  // Lane (l16, g) ends a tile with dX[position pb*16 + l16][32s + 8g + j] in
  // acc[2s + j/4][pb][j%4].
  auto epilogue = [&](const Pos& q, const ZRaw (&zr)[2][CB / 2]) {
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      if constexpr (!LN) {
        if (q.live[pb]) {
          T* dst = static_cast<T*>(p.y) + (int64_t)q.pc[pb] * cout + 8 * g;
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
      } else {
        // LayerNorm backward of this position: statistics recomputed in
        // fp32 (two-pass, population variance; sums over the 4 lane groups)
        float xv[CB / 2][8];
        float sum = 0.f;
#pragma unroll
        for (int s = 0; s < CB / 2; ++s) {
          f32x4 lo, hi;
          widen8(zr[pb][s], lo, hi);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            xv[s][i] = lo[i];
            xv[s][4 + i] = hi[i];
          }
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
        const T* gsrc = static_cast<const T*>(p.ln_w) + 8 * g;
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
        if (q.live[pb]) {
          const uint32_t zrow = zrow_of(q.pc[pb], p.N, p.ending);
          T* dst = static_cast<T*>(p.y) + (int64_t)zrow * cout + 8 * g;
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
  };

  // Software pipeline: the next segment's (or the next tile's first
  // segment's) loads are issued before the current segment's products.  Two
  // operand sets, xa and xb, used in turn; with four segments xa ends each
  // tile holding the next tile's first segment, so nothing is copied.
  // (fp32 operands are twice the registers: one set, no prefetch.)
  constexpr bool PIPE = sizeof(T) == 2;
  Op xa[4][2], xb[PIPE ? 4 : 1][2];
  int tile = blockIdx.x;
  if (tile >= p.ntiles) return;
  Pos cur = pos_of(tile);
  if constexpr (PIPE) load_seg(xa, 0, cur);
  for (; tile < p.ntiles; tile += gridDim.x) {
    const int nt = tile + (int)gridDim.x < p.ntiles ? tile + (int)gridDim.x : tile;
    const Pos nxt = pos_of(nt);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb][0] = acc[cb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    ZRaw zr[2][CB / 2];
    if constexpr (!PIPE) {
      for (int sg = 0; sg < NSEG; ++sg) {
        load_seg(xa, sg, cur);
        comp_seg(xa, sg);
      }
      if constexpr (NSEG == 4) {
        float bx[2][8];
        load_bias(bx, cur);
        comp_bias(bx);
      }
      if constexpr (LN) load_z(zr, cur);
    } else if constexpr (NSEG == 4) {
      float bx[2][8];
      load_seg(xb, 1, cur);
      load_z(zr, cur);
      comp_seg(xa, 0);
      load_seg(xa, 2, cur);
      comp_seg(xb, 1);
      load_seg(xb, 3, cur);
      comp_seg(xa, 2);
      load_bias(bx, cur);
      load_seg(xa, 0, nxt);  // the next tile's first segment
      comp_seg(xb, 3);
      comp_bias(bx);
    } else if constexpr (NSEG == 2) {
      load_seg(xb, 1, cur);
      load_z(zr, cur);
      comp_seg(xa, 0);
      load_seg(xa, 0, nxt);  // the next tile's first segment
      comp_seg(xb, 1);
    } else {
      load_seg(xb, 0, nxt);
      comp_seg(xa, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        xa[u][0] = xb[u < (PIPE ? 4 : 1) ? u : 0][0];
        xa[u][1] = xb[u < (PIPE ? 4 : 1) ? u : 0][1];
      }
    }
    epilogue(cur, zr);
    cur = nxt;
  }
}

// -------------------------------------------------------------------- wgrad
struct WGradParams {
  int N, ending, npos;
  int nseg, a_w, a_zrow;        // A segments [npos][a_w]
  const void* aseg[kMaxSeg];
  const float* dbias;           // [H][npos] (with nseg 4) or null
  int H;
  int b_w, b_zrow, b_ln;        // B [npos][b_w]; LayerNorm-normalised (no affine)
  const void* b;
  int64_t b_ld;                 // row stride of B (0: b_w)
  float eps;
  int rows_pad;                 // nseg*128 (+16 pair-bias rows): partial rows
  int nchunks, chunk_pos;       // one workgroup per chunk of positions
  float* part;                  // [nchunks][rows_pad][b_w]
  float* cpart;                 // [nchunks][rows_pad]
};

// LDS tiles of one 32-position step.  bf16: row-major [32 positions][cols]
// read with transposing reads (a 288-byte row stride spreads a read's four
// rows over distinct banks), double-buffered; fp32: transposed
// [cols][32 positions], single-buffered.
// A B tile of up to 256 columns (WIDE) is [32][272] (bf16) or [256][36]
// (fp32).
template <typename T> struct WL;
template <> struct WL<bf16_t> {
  static constexpr int RS = 144, BRS = 24;  // row strides: 128- and 16-column tiles
  static constexpr int TILE = 32 * RS, BTILE = 32 * BRS, NBUF = 2;
  static constexpr int RSW = 272, TILEW = 32 * RSW;
};
template <> struct WL<float> {
  static constexpr int PS = 36;             // position stride of a transposed tile
  static constexpr int TILE = 128 * PS, BTILE = 16 * PS, NBUF = 1;
  static constexpr int TILEW = 256 * PS;
};
template <typename T, int NSEG, bool WIDE = false>
constexpr size_t wgrad_lds() {
  return (size_t)WL<T>::NBUF *
             (NSEG * WL<T>::TILE + (WIDE ? WL<T>::TILEW : WL<T>::TILE) + WL<T>::BTILE) *
             sizeof(T) +
         8 * 144 * sizeof(float);
}

// One workgroup (eight waves) per chunk of positions computes every row of
// M = A^T B for that chunk, so each B row (and its LayerNorm) is formed once.
// NSEG = 4: the module (A = q, k, v, gate gradients + the pair-bias rows,
// B = xhat); NSEG = 2: the multiplicative update (A = its a and b
// gradients, B = xhat); NSEG = 1: the output projection (A = dout, B = o).  Wave w owns
// segment w / (8/NSEG) and the column blocks w % (8/NSEG) + (8/NSEG) i,
// i < NSEG (i < 2 NSEG when WIDE: B up to 256 columns); with NSEG = 4 also
// the pair-bias rows of column block w.
// FULL: every segment 128 wide and B 128 (WIDE: 256) columns, so the
// per-block guards fold away and the products are straight-line code.
template <typename T, int NSEG, bool BIAS = NSEG == 4, bool WIDE = false, bool FULL = false>
__global__ void __launch_bounds__(512) wgrad_kernel(WGradParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int WPS = 8 / NSEG;     // waves (and column groups) per segment
  constexpr int TPS = 512 / NSEG;   // staging threads per segment
  constexpr int NB = WL<T>::NBUF;
  constexpr int NCG = WIDE ? 2 * NSEG : NSEG;   // column blocks per wave
  constexpr int NBC = WIDE ? 2 : 1;             // 128-column B chunks per thread
  constexpr int BT = WIDE ? WL<T>::TILEW : WL<T>::TILE;
  static_assert(!(WIDE && BIAS), "the pair-bias rows go with 128-column B tiles");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sA = reinterpret_cast<T*>(smem);                   // [NB][NSEG][TILE]
  T* sB = sA + NB * NSEG * WL<T>::TILE;                  // [NB][BT]
  T* sBi = sB + NB * BT;                                 // [NB][BTILE]
  float (*sred)[144] = reinterpret_cast<float (*)[144]>(sBi + NB * WL<T>::BTILE);

  const int chunk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int pbeg = chunk * p.chunk_pos, pend = min(p.npos, pbeg + p.chunk_pos);
  const int nst = (pend - pbeg + PW - 1) / PW;
  const int RB = FULL ? 8 : p.a_w / 16, CBn = FULL ? (WIDE ? 16 : 8) : p.b_w / 16;
  const int wseg = wave / WPS, cw = wave % WPS;

  // Staging roles.  A: segment tid / TPS, channels 8*(tid%16) .. +7 of
  // positions (tid%TPS)/16 + (TPS/16) u, u < NSEG (the same channels every
  // step, so the column sums stay in 8 registers).  B: position tid/16,
  // channels 8*(tid%16) .. +7.  Pair-bias rows: position tid/16, row tid%16.
  const int a_seg = tid / TPS, a_c8 = (tid & 15) * 8, a_pos0 = (tid % TPS) >> 4;
  const T* Aseg = static_cast<const T*>(p.aseg[a_seg]);
  const T* Bsrc = static_cast<const T*>(p.b);
  const int64_t bld = p.b_ld ? p.b_ld : p.b_w;
  const int b_pos = tid >> 4, b_c8 = (tid & 15) * 8, bi_row = tid & 15;
  float csum[8], csum_b = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) csum[j] = 0.f;

  struct Raw {
    Raw8<T> a[NSEG];
    Raw8<T> b[NBC];
    float bi;
  };
  auto zero8 = [](Raw8<T>& r) {
    r.a = u32x4{0, 0, 0, 0};
    if constexpr (sizeof(T) == 4) r.b = u32x4{0, 0, 0, 0};
  };
  auto fetch = [&](int st, Raw& r) {
    const int p0 = pbeg + st * PW;
#pragma unroll
    for (int u = 0; u < NSEG; ++u) {
      const int pidx = p0 + a_pos0 + (TPS / 16) * u;
      if (pidx < pend && a_c8 < p.a_w) {
        const uint32_t row = p.a_zrow ? zrow_of(pidx, p.N, p.ending) : (uint32_t)pidx;
        ld_raw8(r.a[u], Aseg + (int64_t)row * p.a_w + a_c8);
      } else {
        zero8(r.a[u]);
      }
    }
#pragma unroll
    for (int q = 0; q < NBC; ++q) {
      const int pidx = p0 + b_pos, c8 = b_c8 + 128 * q;
      if (pidx < pend && c8 < p.b_w) {
        const uint32_t row = p.b_zrow ? zrow_of(pidx, p.N, p.ending) : (uint32_t)pidx;
        ld_raw8(r.b[q], Bsrc + (int64_t)row * bld + c8);
      } else {
        zero8(r.b[q]);
      }
    }
    if constexpr (BIAS) {
      const int pidx = p0 + b_pos;
      r.bi = (pidx < pend && bi_row < 2 * p.H)
                 ? p.dbias[(int64_t)(bi_row % p.H) * p.npos + pidx] : 0.f;
    }
  };
  // Store 8 values (channels c8 .. c8+7 of position pos) into a tile with
  // row stride rs (bf16).
  auto put8 = [&](T* tile, int pos, int c8, const float (&v)[8], int rs) {
    if constexpr (sizeof(T) == 2) {
      st8f(tile + pos * rs + c8, v);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) tile[(c8 + j) * WL<T>::PS + pos] = v[j];
    }
  };
  auto stage = [&](Raw& r, int buf) {
#pragma unroll
    for (int u = 0; u < NSEG; ++u) {
      float v[8];
      f32x4 lo, hi;
      widen8(r.a[u], lo, hi);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = lo[i];
        v[4 + i] = hi[i];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) csum[j] += v[j];
      if (a_c8 < p.a_w)
        put8(sA + (buf * NSEG + a_seg) * WL<T>::TILE, a_pos0 + (TPS / 16) * u, a_c8, v,
             sizeof(T) == 2 ? WL<bf16_t>::RS : 0);
    }
    {
      float v[NBC][8];
#pragma unroll
      for (int q = 0; q < NBC; ++q) {
        f32x4 lo, hi;
        widen8(r.b[q], lo, hi);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[q][i] = lo[i];
          v[q][4 + i] = hi[i];
        }
      }
      if (p.b_ln) {
        // statistics over the 16 lanes of this position (NBC chunks each)
        float sm = 0.f;
#pragma unroll
        for (int q = 0; q < NBC; ++q)
#pragma unroll
          for (int j = 0; j < 8; ++j) sm += v[q][j];
        sm += __shfl_xor(sm, 1, 64);
        sm += __shfl_xor(sm, 2, 64);
        sm += __shfl_xor(sm, 4, 64);
        sm += __shfl_xor(sm, 8, 64);
        const float inv_n = 1.f / (float)p.b_w;
        const float mu = sm * inv_n;
        float var = 0.f;
#pragma unroll
        for (int q = 0; q < NBC; ++q) {
          const bool in = b_c8 + 128 * q < p.b_w;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            v[q][j] = in ? v[q][j] - mu : 0.f;
            var = __builtin_fmaf(v[q][j], v[q][j], var);
          }
        }
        var += __shfl_xor(var, 1, 64);
        var += __shfl_xor(var, 2, 64);
        var += __shfl_xor(var, 4, 64);
        var += __shfl_xor(var, 8, 64);
        const float rstd = rsqrtf(var * inv_n + p.eps);
#pragma unroll
        for (int q = 0; q < NBC; ++q)
#pragma unroll
          for (int j = 0; j < 8; ++j) v[q][j] *= rstd;
      }
#pragma unroll
      for (int q = 0; q < NBC; ++q)
        if (b_c8 + 128 * q < p.b_w)
          put8(sB + buf * BT, b_pos, b_c8 + 128 * q, v[q],
               sizeof(T) == 2 ? (WIDE ? WL<bf16_t>::RSW : WL<bf16_t>::RS) : 0);
    }
    if constexpr (BIAS) {
      const float d = r.bi;
      if (bi_row < p.H) csum_b += d;
      T* t = sBi + buf * WL<T>::BTILE;
      if constexpr (sizeof(T) == 2) {
        const float hi = (float)(__bf16)d;
        t[b_pos * WL<T>::BRS + bi_row] = Tr<T>::from_f(bi_row < p.H ? hi : d - hi);
      } else {
        t[bi_row * WL<T>::PS + b_pos] = bi_row < p.H ? d : 0.f;
      }
    }
  };
  // Operand fragment: column col0 + l16 of a step's tile, positions 8g .. +7.
  auto frag = [&](const T* t, int col0, int rs) -> Op {
    if constexpr (sizeof(T) == 2) {
      const T* p0 = t + (8 * g + (l16 >> 2)) * rs + col0 + 4 * (l16 & 3);
      return lds_read_tr_op(p0, p0 + 4 * rs);
    } else {
      (void)rs;
      return ld_op<T>(t + (col0 + l16) * WL<T>::PS + 8 * g);
    }
  };

  f32x4 acc[8][NCG], accb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int rb = 0; rb < 8; ++rb)
#pragma unroll
    for (int i = 0; i < NCG; ++i) acc[rb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int rsA = sizeof(T) == 2 ? WL<bf16_t>::RS : 0;
  const int rsB = sizeof(T) == 2 ? (WIDE ? WL<bf16_t>::RSW : WL<bf16_t>::RS) : 0;
  const int rsBi = sizeof(T) == 2 ? WL<bf16_t>::BRS : 0;

  Raw raw;
  if (nst > 0) fetch(0, raw);
  for (int st = 0; st < nst; ++st) {
    const int buf = NB == 2 ? (st & 1) : 0;
    if (NB == 1 && st > 0) __syncthreads();  // the previous step's reads are done
    stage(raw, buf);
    __syncthreads();
    if (st + 1 < nst) fetch(st + 1, raw);
    const T* tA = sA + (buf * NSEG + wseg) * WL<T>::TILE;
    const T* tB = sB + buf * BT;
    if constexpr (sizeof(T) == 2) {
      Op bf[NCG];
#pragma unroll
      for (int i = 0; i < NCG; ++i)
        if (cw + WPS * i < CBn) bf[i] = frag(tB, (cw + WPS * i) * 16, rsB);
#pragma unroll
      for (int rb = 0; rb < 8; ++rb) {
        if (rb >= RB) break;
        const Op af = frag(tA, rb * 16, rsA);
#pragma unroll
        for (int i = 0; i < NCG; ++i)
          if (cw + WPS * i < CBn) acc[rb][i] = mma32(af, bf[i], acc[rb][i]);
      }
    } else {
      // fp32 fragments are twice the registers: one column block at a time
#pragma unroll
      for (int i = 0; i < NCG; ++i) {
        if (cw + WPS * i >= CBn) continue;
        const Op bfi = frag(tB, (cw + WPS * i) * 16, rsB);
#pragma unroll
        for (int rb = 0; rb < 8; ++rb) {
          if (rb >= RB) break;
          acc[rb][i] = mma32(frag(tA, rb * 16, rsA), bfi, acc[rb][i]);
        }
      }
    }
    if constexpr (BIAS) {
      if (wave < CBn) {
        const Op ab = frag(sBi + buf * WL<T>::BTILE, 0, rsBi);
        const Op bw = frag(tB, wave * 16, rsB);
        accb = mma32(ab, bw, accb);
      }
    }
  }

  // Partials: lane (l16, g) holds M[rb*16 + 4g + i][cb*16 + l16].
  float* dst = p.part + (int64_t)chunk * p.rows_pad * p.b_w;
#pragma unroll
  for (int i = 0; i < NCG; ++i) {
    const int cb = cw + WPS * i;
    if (cb >= CBn) continue;
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
      if (rb >= RB) break;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dst[(int64_t)(wseg * 128 + rb * 16 + 4 * g + r) * p.b_w + cb * 16 + l16] = acc[rb][i][r];
    }
  }
  if constexpr (BIAS) {
    if (wave < CBn) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dst[(int64_t)(NSEG * 128 + 4 * g + r) * p.b_w + wave * 16 + l16] = accb[r];
    }
  }
  // Column sums: lanes with equal tid % 16 of a wave staged the same
  // channels (and pair-bias row); then the waves of a segment.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    csum[j] += __shfl_xor(csum[j], 16, 64);
    csum[j] += __shfl_xor(csum[j], 32, 64);
  }
  csum_b += __shfl_xor(csum_b, 16, 64);
  csum_b += __shfl_xor(csum_b, 32, 64);
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sred[wave][lane * 8 + j] = csum[j];
    sred[wave][128 + lane] = csum_b;
  }
  __syncthreads();
  float* cdst = p.cpart + (int64_t)chunk * p.rows_pad;
  if (tid < NSEG * 128) {
    const int sg = tid >> 7, ch = tid & 127;
    if (ch < p.a_w) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < WPS; ++w) t += sred[sg * WPS + w][ch];
      cdst[sg * 128 + ch] = t;
    }
  }
  if constexpr (BIAS) {
    if (tid < 16) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) t += sred[w][128 + tid];
      cdst[NSEG * 128 + tid] = t;
    }
  }
}

// ------------------------------------------------------------------- finish
// First stage of the chunk reduction: group gi = blockIdx.y sums chunks
// 16 gi .. 16 gi + 15 in order (partials, then the column sums).
constexpr int kGroup = 16;
__global__ void __launch_bounds__(256) chunk_sum_kernel(const float* part, const float* cpart,
                                                        int nchunks, int rows_pad, int ncols,
                                                        float* part2, float* cpart2) {
  const int gi = blockIdx.y;
  const int c0 = gi * kGroup, c1 = min(nchunks, c0 + kGroup);
  const int64_t esize = (int64_t)rows_pad * ncols;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < esize + rows_pad;
       e += (int64_t)gridDim.x * 256) {
    float t = 0.f;
    if (e < esize) {
      for (int ch = c0; ch < c1; ++ch) t += part[ch * esize + e];
      part2[gi * esize + e] = t;
    } else {
      const int64_t r = e - esize;
      for (int ch = c0; ch < c1; ++ch) t += cpart[(int64_t)ch * rows_pad + r];
      cpart2[(int64_t)gi * rows_pad + r] = t;
    }
  }
}


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
  int64_t ldw;              // row stride of dw (0: ncols)
};

// Sum of 16 lanes' partials (lanes 16a .. 16a+15), complete in the first
// lane of the group (a fixed butterfly: the same order on every run).
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

// One output element per 16 lanes: lane j of the group sums chunks j, j+16,
// ..., then the group adds the 16 sums.
template <typename T>
__global__ void __launch_bounds__(256) wgrad_finish_kernel(FinishParams p) {
  const int nrows = p.nseg * p.a_w + (p.has_bias ? p.H : 0);
  const int64_t total = (int64_t)nrows * p.ncols;
  const int64_t cstride = (int64_t)p.rows_pad * p.ncols;
  const int j = threadIdx.x & 15;
  for (int64_t e0 = (int64_t)blockIdx.x * 16; e0 < total; e0 += (int64_t)gridDim.x * 16) {
    // elements e0 .. e0+15: lane group (threadIdx.x / 16) takes one
    const int64_t e = e0 + (threadIdx.x >> 4);
    const bool live = e < total;
    const int64_t ec = live ? e : total - 1;
    const int k = (int)(ec / p.ncols), c = (int)(ec - (int64_t)k * p.ncols);
    float m = 0.f, s = 0.f;
    int seg = -1, r = 0;
    if (k < p.nseg * p.a_w) {
      seg = k / p.a_w;
      r = k - seg * p.a_w;
      const int slot = seg * 128 + r;
      for (int ch = j; ch < p.nchunks; ch += 16) {
        m += p.part[ch * cstride + (int64_t)slot * p.ncols + c];
        s += p.cpart[(int64_t)ch * p.rows_pad + slot];
      }
    } else {
      r = k - p.nseg * p.a_w;  // head: high plus low part of dBias
      const int hi = p.nseg * 128 + r, lo = hi + p.H;
      for (int ch = j; ch < p.nchunks; ch += 16) {
        m += p.part[ch * cstride + (int64_t)hi * p.ncols + c] +
             p.part[ch * cstride + (int64_t)lo * p.ncols + c];
        s += p.cpart[(int64_t)ch * p.rows_pad + hi];
      }
    }
    m = sum16(m);
    s = sum16(s);
    if (!live || j != 0) continue;
    float out = m;
    if (p.ln) {
      const float gm = Tr<T>::to_f(static_cast<const T*>(p.ln_w)[c]);
      const float bt = Tr<T>::to_f(static_cast<const T*>(p.ln_b)[c]);
      out = __builtin_fmaf(gm, m, bt * s);
      p.mred[e] = m;
      if (c == 0) p.cred[k] = s;
    }
    if (seg >= 0) {
      p.dw[seg][(int64_t)r * (p.ldw ? p.ldw : p.ncols) + c] = out;
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

// One workgroup per column c: thread t takes rows t, t+256, ...; the
// workgroup then adds the 256 sums in a fixed order.
template <typename T>
__global__ void __launch_bounds__(256) lnparam_kernel(LnParamParams p) {
  __shared__ float red[2][4];
  const int c = blockIdx.x, tid = threadIdx.x;
  float dg = 0.f, db = 0.f;
  const int nrows = p.nseg * p.a_w + p.H;
  for (int k = tid; k < nrows; k += 256) {
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
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    dg += __shfl_xor(dg, m, 64);
    db += __shfl_xor(db, m, 64);
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = dg;
    red[1][tid >> 6] = db;
  }
  __syncthreads();
  if (tid == 0) {
    p.dln_w[c] = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
    p.dln_b[c] = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
  }
}

// ----------------------------------------------------------------- launches
template <typename T, int CB, int NSEG, bool FULL = false>
hipError_t launch_rowgrad_cb(RowGradParams& p, hipStream_t s) {
  constexpr int WAVES = 8;
  const size_t wbytes = (size_t)p.cout * (p.Kext + PADE) * sizeof(T);
  p.resident = wbytes <= kLdsBudget;
  p.kc = p.resident ? p.Kext : std::max(p.seg_w, 32);
  const size_t lds = (size_t)p.cout * (p.kc + PADE) * sizeof(T);
  const int64_t tiles = ((int64_t)p.npos + PW * WAVES - 1) / (PW * WAVES);
  p.ntiles = (int)tiles;
  const int grid = (int)std::min<int64_t>(tiles, 256);
  hipError_t e =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&rowgrad_kernel<T, CB, NSEG, FULL>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((rowgrad_kernel<T, CB, NSEG, FULL>), dim3(grid), dim3(WAVES * 64), lds, s,
                     p);
  return hipGetLastError();
}

// nseg 4 with the pair-bias block and the LayerNorm backward (the module),
// 2 with the LayerNorm backward only (the multiplicative update), or 1
// without either (the output projection).
template <typename T, int CB>
hipError_t launch_rowgrad_n(RowGradParams& p, hipStream_t s) {
  switch (p.nseg) {
    case 4:
      // the module at H*C = 128, c_z = 128
      if (CB == 8 && p.seg_w == 128) return launch_rowgrad_cb<T, CB, 4, true>(p, s);
      return launch_rowgrad_cb<T, CB, 4>(p, s);
    case 2: return launch_rowgrad_cb<T, CB, 2>(p, s);
    default: return launch_rowgrad_cb<T, CB, 1>(p, s);
  }
}
template <typename T>
hipError_t launch_rowgrad(RowGradParams& p, hipStream_t s) {
  if (p.nseg != 1 && p.nseg != 2 && p.nseg != 4) return hipErrorInvalidValue;
  if ((p.nseg == 4) != (p.dbias != nullptr) || (p.nseg != 1) != (p.ln != 0))
    return hipErrorInvalidValue;
  switch (p.cout / 16) {
    case 2: return launch_rowgrad_n<T, 2>(p, s);
    case 4: return launch_rowgrad_n<T, 4>(p, s);
    case 6: return launch_rowgrad_n<T, 6>(p, s);
    case 8: return launch_rowgrad_n<T, 8>(p, s);
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
// One workgroup of the weight-gradient kernel per CU (eight waves, about 100
// KB of LDS), each over one chunk of positions.
constexpr int kChunks = 256;

template <typename T, int NSEG, bool BIAS, bool WIDE = false, bool FULL = false>
hipError_t launch_wgrad_k(WGradParams& p, hipStream_t s) {
  const size_t lds = wgrad_lds<T, NSEG, WIDE>();
  hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&wgrad_kernel<T, NSEG, BIAS, WIDE, FULL>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((wgrad_kernel<T, NSEG, BIAS, WIDE, FULL>), dim3(p.nchunks), dim3(512), lds,
                     s, p);
  return hipGetLastError();
}
// four segments with or without the pair-bias rows; two or one without; B
// wider than 128 columns (up to 256) with two segments only
template <typename T>
hipError_t launch_wgrad(WGradParams& p, hipStream_t s) {
  const bool bias = p.dbias != nullptr;
  if (bias && p.nseg != 4) return hipErrorInvalidValue;
  if (p.b_w > 256 || (p.b_w > 128 && p.nseg != 2 && p.nseg != 1)) return hipErrorInvalidValue;
  if (p.b_w > 128)
    return p.nseg == 2 ? launch_wgrad_k<T, 2, false, true>(p, s)
                       : launch_wgrad_k<T, 1, false, true>(p, s);
  const bool full = p.a_w == 128 && p.b_w == 128;
  switch (p.nseg) {
    case 4:
      if (full)
        return bias ? launch_wgrad_k<T, 4, true, false, true>(p, s)
                    : launch_wgrad_k<T, 4, false, false, true>(p, s);
      return bias ? launch_wgrad_k<T, 4, true>(p, s) : launch_wgrad_k<T, 4, false>(p, s);
    case 2:
      return full ? launch_wgrad_k<T, 2, false, false, true>(p, s)
                  : launch_wgrad_k<T, 2, false>(p, s);
    case 1:
      return full ? launch_wgrad_k<T, 1, false, false, true>(p, s)
                  : launch_wgrad_k<T, 1, false>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// Sums the chunk partials in two fixed-order stages (groups of kGroup chunks
// into part2/cpart2, then the groups) and writes the gradients.
template <typename T>
hipError_t launch_finish(FinishParams& f, float* part2, float* cpart2, hipStream_t s) {
  const int ngroups = (f.nchunks + kGroup - 1) / kGroup;
  const int64_t esize = (int64_t)f.rows_pad * f.ncols + f.rows_pad;
  const int gx = (int)std::min<int64_t>((esize + 255) / 256, 1024);
  hipLaunchKernelGGL(chunk_sum_kernel, dim3(gx, ngroups), dim3(256), 0, s, f.part, f.cpart,
                     f.nchunks, f.rows_pad, f.ncols, part2, cpart2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  f.nchunks = ngroups;
  f.part = part2;
  f.cpart = cpart2;
  const int64_t total = (int64_t)(f.nseg * f.a_w + (f.has_bias ? f.H : 0)) * f.ncols;
  const int grid = (int)std::min<int64_t>((total + 15) / 16, 16384);
  hipLaunchKernelGGL(wgrad_finish_kernel<T>, dim3(grid), dim3(256), 0, s, f);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct PartLayout {
  size_t part, cpart, part2, cpart2, mred, cred, total;
};
PartLayout part_layout(int64_t N, int64_t CZ, int64_t H) {
  const int64_t npos = N * N, HC = H * kHeadDim;
  int nc, cp;
  chunking(npos, kChunks, nc, cp);
  const size_t part_m = (size_t)nc * (4 * 128 + 16) * CZ * 4, cpart_m = (size_t)nc * (4 * 128 + 16) * 4;
  const size_t part_o = (size_t)nc * 128 * HC * 4, cpart_o = (size_t)nc * 128 * 4;
  PartLayout L;
  L.part = 0;
  L.cpart = align256(std::max(part_m, part_o));
  const int ng = (nc + kGroup - 1) / kGroup;
  L.part2 = L.cpart + align256(std::max(cpart_m, cpart_o));
  L.cpart2 = L.part2 + align256((size_t)ng * (4 * 128 + 16) * std::max(CZ, HC) * 4);
  L.mred = L.cpart2 + align256((size_t)ng * (4 * 128 + 16) * 4);
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
  w.rows_pad = 128;
  chunking(npos, kChunks, w.nchunks, w.chunk_pos);
  w.part = reinterpret_cast<float*>(ws + L.part);
  w.cpart = reinterpret_cast<float*>(ws + L.cpart);
  if ((e = launch_wgrad<T>(w, s)) != hipSuccess) return e;
  FinishParams f{};
  f.nchunks = w.nchunks; f.rows_pad = w.rows_pad; f.ncols = HC;
  f.nseg = 1; f.a_w = CZ; f.H = H; f.has_bias = 0;
  f.part = w.part; f.cpart = w.cpart;
  f.ln = 0;
  f.dw[0] = a.dw_o; f.dcol[0] = a.db_o;
  return launch_finish<T>(f, reinterpret_cast<float*>(ws + L.part2),
                          reinterpret_cast<float*>(ws + L.cpart2), s);
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
  w.rows_pad = 4 * 128 + 16;
  chunking(npos, kChunks, w.nchunks, w.chunk_pos);
  w.part = reinterpret_cast<float*>(ws + L.part);
  w.cpart = reinterpret_cast<float*>(ws + L.cpart);
  if ((e = launch_wgrad<T>(w, s)) != hipSuccess) return e;
  FinishParams f{};
  f.nchunks = w.nchunks; f.rows_pad = w.rows_pad; f.ncols = CZ;
  f.nseg = 4; f.a_w = HC; f.H = H; f.has_bias = 1;
  f.part = w.part; f.cpart = w.cpart;
  f.ln = 1; f.ln_w = a.ln_w; f.ln_b = a.ln_b;
  f.dw[0] = a.dw_q; f.dw[1] = a.dw_k; f.dw[2] = a.dw_v; f.dw[3] = a.dw_g;
  f.dw_bias = a.dw_bias;
  f.dcol[3] = a.db_g;
  f.mred = reinterpret_cast<float*>(ws + L.mred);
  f.cred = reinterpret_cast<float*>(ws + L.cred);
  if ((e = launch_finish<T>(f, reinterpret_cast<float*>(ws + L.part2),
                           reinterpret_cast<float*>(ws + L.cpart2), s)) != hipSuccess)
    return e;
  LnParamParams l{};
  l.nseg = 4; l.a_w = HC; l.H = H; l.ncols = CZ;
  for (int i = 0; i < 4; ++i) l.wseg[i] = wts[i];
  l.wbias = a.w_bias; l.mred = f.mred; l.cred = f.cred;
  l.dln_w = a.dln_w; l.dln_b = a.dln_b;
  hipLaunchKernelGGL(lnparam_kernel<T>, dim3(CZ), dim3(256), 0, s, l);
  return hipGetLastError();
}

// ------------------------------------------- LayerNorm backward, 256 wide
// dz = LayerNorm backward of dX = sum_s dY_s . W_s for rows of 256 channels
// (too wide for rowgrad_kernel's registers).  Four waves, 16 positions per
// wave per tile: dX^T = W_ext^T . dY^T on the matrix cores with W_ext^T
// ([256][K], K = nseg * seg_w) in LDS (resident when it fits, else in
// column chunks of kc per tile), so lane (l16, g) ends with
// channels 16 cb + 4 g .. +3 of position l16 for cb < 16; then the
// LayerNorm backward in registers (statistics recomputed from z in fp32,
// two-pass, sums over the four lane groups).
struct LnWideParams {
  int npos, seg_w, K, kc, ntiles;
  const void* dy[2];
  const void* w[2];   // [seg_w][256]
  const void* z;      // [npos][256]
  const void* ln_w;
  float eps;
  void* dz;           // [npos][256]
};
constexpr int kWideC = 256;

template <typename T>
__device__ __forceinline__ void ld4f(const T* p, float (&v)[4]) {
  if constexpr (sizeof(T) == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(p);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  }
}
template <typename T>
__device__ __forceinline__ void st4f(T* p, const float (&v)[4]) {
  if constexpr (sizeof(T) == 2) {
    uint2 u;
    u.x = uint32_t(Tr<bf16_t>::from_f(v[0])) | (uint32_t(Tr<bf16_t>::from_f(v[1])) << 16);
    u.y = uint32_t(Tr<bf16_t>::from_f(v[2])) | (uint32_t(Tr<bf16_t>::from_f(v[3])) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <typename T>
__global__ void __launch_bounds__(256) ln_bwd_wide_kernel(LnWideParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int CB = kWideC / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int KS = p.kc + PADE;
  T* sW = reinterpret_cast<T*>(smem);                                  // [256][kc + PADE]
  float* sG = reinterpret_cast<float*>(smem + (size_t)kWideC * KS * sizeof(T));  // [256]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  // W_ext^T columns [k0, k0 + kc) into LDS
  auto load_w = [&](int k0) {
    for (int e = tid; e < kWideC * p.kc; e += 256) {
      const int o = e / p.kc, k = k0 + (e - o * p.kc);
      const int sg = k / p.seg_w;
      sW[o * KS + (k - k0)] =
          static_cast<const T*>(p.w[sg])[(int64_t)(k - sg * p.seg_w) * kWideC + o];
    }
  };
  const bool resident = p.kc == p.K;
  if (resident) load_w(0);
  for (int c = tid; c < kWideC; c += 256) sG[c] = Tr<T>::to_f(static_cast<const T*>(p.ln_w)[c]);
  __syncthreads();
  const int ksteps = p.kc / 32;
  const float inv_n = 1.f / (float)kWideC;
  for (int tile = blockIdx.x; tile < p.ntiles; tile += gridDim.x) {
    const int pos = (tile * 4 + wave) * 16 + l16;
    const bool live = pos < p.npos;
    const int pc = live ? pos : p.npos - 1;
    f32x4 acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < p.K; k0 += p.kc) {
      if (!resident) {
        __syncthreads();  // every wave is done with the previous chunk
        load_w(k0);
        __syncthreads();
      }
      for (int u = 0; u < ksteps; ++u) {
        const int k = k0 + 32 * u + 8 * g, sg = k / p.seg_w;
        const Op x = ld_op<T>(static_cast<const T*>(p.dy[sg]) + (int64_t)pc * p.seg_w +
                              (k - sg * p.seg_w));
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const Op a = ld_op<T>(sW + (cb * 16 + l16) * KS + 32 * u + 8 * g);
          acc[cb] = mma32(a, x, acc[cb]);
        }
      }
    }
    // lane (l16, g): dX[pos][16 cb + 4 g + i] in acc[cb][i]
    const T* zr = static_cast<const T*>(p.z) + (int64_t)pc * kWideC + 4 * g;
    float xv[CB][4];
    float sum = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      ld4f<T>(zr + 16 * cb, xv[cb]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sum += xv[cb][i];
    }
    sum += shfl_xor(sum, 16);
    sum += shfl_xor(sum, 32);
    const float mu = sum * inv_n;
    float var = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xv[cb][i] -= mu;
        var = __builtin_fmaf(xv[cb][i], xv[cb][i], var);
      }
    var += shfl_xor(var, 16);
    var += shfl_xor(var, 32);
    const float rstd = rsqrtf(var * inv_n + p.eps);
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xv[cb][i] *= rstd;  // xhat
        const float d = acc[cb][i] * sG[16 * cb + 4 * g + i];
        acc[cb][i] = d;     // dxhat
        a += d;
        b = __builtin_fmaf(d, xv[cb][i], b);
      }
    a += shfl_xor(a, 16);
    a += shfl_xor(a, 32);
    b += shfl_xor(b, 16);
    b += shfl_xor(b, 32);
    a *= inv_n;
    b *= inv_n;
    if (live) {
      T* dst = static_cast<T*>(p.dz) + (int64_t)pos * kWideC + 4 * g;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = rstd * (acc[cb][i] - a - xv[cb][i] * b);
        st4f<T>(dst + 16 * cb, v);
      }
    }
  }
}

template <typename T>
hipError_t launch_ln_bwd_wide(LnWideParams& p, hipStream_t s) {
  // all of W_ext^T when it fits the LDS budget, else 128-column chunks (fp32
  // with K = 256)
  p.kc = (size_t)kWideC * (p.K + PADE) * sizeof(T) <= kLdsBudget ? p.K : 128;
  const size_t lds = (size_t)kWideC * (p.kc + PADE) * sizeof(T) + kWideC * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ln_bwd_wide_kernel<T>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  p.ntiles = (p.npos + 63) / 64;
  const int grid = std::min(p.ntiles, 2048);
  hipLaunchKernelGGL(ln_bwd_wide_kernel<T>, dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

// Workspace of the two-segment LayerNorm + projection backward: chunk
// partials (256 rows: 128 per segment), their group sums, M and s.
struct LnProjLayout {
  size_t part, cpart, part2, cpart2, mred, cred, total;
};
LnProjLayout ln_proj_layout(int64_t npos, int64_t CZ, int seg_w) {
  int nc, cp;
  chunking(npos, kChunks, nc, cp);
  const int ng = (nc + kGroup - 1) / kGroup;
  LnProjLayout L;
  L.part = 0;
  L.cpart = align256((size_t)nc * 256 * CZ * 4);
  L.part2 = L.cpart + align256((size_t)nc * 256 * 4);
  L.cpart2 = L.part2 + align256((size_t)ng * 256 * CZ * 4);
  L.mred = L.cpart2 + align256((size_t)ng * 256 * 4);
  L.cred = L.mred + align256((size_t)2 * seg_w * CZ * 4);
  L.total = L.cred + align256((size_t)2 * seg_w * 4);
  return L;
}

// LayerNorm + nseg projections of z, backward from the projections'
// gradients (the multiplicative update's a and b, the outer product mean's
// a and b): dz, dW_s, dgamma, dbeta.
template <typename T>
hipError_t ln_proj_bwd_t(const LnProjBwdArgs& a, hipStream_t s) {
  const int CZ = (int)a.CZ, W = a.seg_w;
  const int npos = (int)a.npos;
  const LnProjLayout L = ln_proj_layout(a.npos, a.CZ, W);
  char* ws = static_cast<char*>(a.workspace);
  hipError_t e;
  if (CZ == kWideC) {
    LnWideParams q{};
    q.npos = npos; q.seg_w = W; q.K = a.nseg * W;
    for (int i = 0; i < a.nseg; ++i) { q.dy[i] = a.dy[i]; q.w[i] = a.w[i]; }
    q.z = a.z; q.ln_w = a.ln_w; q.eps = a.eps; q.dz = a.dz;
    e = launch_ln_bwd_wide<T>(q, s);
  } else {
    RowGradParams r{};
    r.N = 0; r.ending = 0; r.npos = npos;  // plain rows: no z-row mapping
    r.nseg = a.nseg; r.seg_w = W; r.in_zrow = 0;
    for (int i = 0; i < a.nseg; ++i) { r.seg[i] = a.dy[i]; r.wseg[i] = a.w[i]; }
    r.dbias = nullptr; r.H = 0; r.Kext = a.nseg * W;
    r.wbias = nullptr; r.cout = CZ;
    r.ln = 1; r.z = a.z; r.ln_w = a.ln_w; r.eps = a.eps; r.y = a.dz;
    e = launch_rowgrad<T>(r, s);
  }
  if (e != hipSuccess) return e;
  WGradParams w{};
  w.N = 0; w.ending = 0; w.npos = npos;
  w.nseg = a.nseg; w.a_w = W; w.a_zrow = 0;
  for (int i = 0; i < a.nseg; ++i) w.aseg[i] = a.dy[i];
  w.dbias = nullptr; w.H = 0;
  w.b_w = CZ; w.b_zrow = 0; w.b_ln = 1; w.b = a.z; w.eps = a.eps;
  w.rows_pad = a.nseg * 128;
  chunking(npos, kChunks, w.nchunks, w.chunk_pos);
  w.part = reinterpret_cast<float*>(ws + L.part);
  w.cpart = reinterpret_cast<float*>(ws + L.cpart);
  if ((e = launch_wgrad<T>(w, s)) != hipSuccess) return e;
  FinishParams f{};
  f.nchunks = w.nchunks; f.rows_pad = w.rows_pad; f.ncols = CZ;
  f.nseg = a.nseg; f.a_w = W; f.H = 0; f.has_bias = 0;
  f.part = w.part; f.cpart = w.cpart;
  f.ln = 1; f.ln_w = a.ln_w; f.ln_b = a.ln_b;
  for (int i = 0; i < a.nseg; ++i) f.dw[i] = a.dw[i];
  f.mred = reinterpret_cast<float*>(ws + L.mred);
  f.cred = reinterpret_cast<float*>(ws + L.cred);
  if ((e = launch_finish<T>(f, reinterpret_cast<float*>(ws + L.part2),
                           reinterpret_cast<float*>(ws + L.cpart2), s)) != hipSuccess)
    return e;
  LnParamParams l{};
  l.nseg = a.nseg; l.a_w = W; l.H = 0; l.ncols = CZ;
  for (int i = 0; i < a.nseg; ++i) l.wseg[i] = a.w[i];
  l.wbias = nullptr; l.mred = f.mred; l.cred = f.cred;
  l.dln_w = a.dln_w; l.dln_b = a.dln_b;
  hipLaunchKernelGGL(lnparam_kernel<T>, dim3(CZ), dim3(256), 0, s, l);
  return hipGetLastError();
}

struct SegLayout {
  size_t part, cpart, part2, cpart2, total;
};
SegLayout seg_layout(int64_t npos, int64_t ncols) {
  int nc, cp;
  chunking(npos, kChunks, nc, cp);
  const int ng = (nc + kGroup - 1) / kGroup;
  SegLayout L;
  L.part = 0;
  L.cpart = align256((size_t)nc * 512 * ncols * 4);
  L.part2 = L.cpart + align256((size_t)nc * 512 * 4);
  L.cpart2 = L.part2 + align256((size_t)ng * 512 * ncols * 4);
  L.total = L.cpart2 + align256((size_t)ng * 512 * 4);
  return L;
}

// M = A^T B over plain position rows, A [npos][a_w] (a_w <= 128), B
// [npos][b_w] at row stride b_ld (b_w <= 256): dw[r * dw_ld + c] = M[r][c],
// dcol[r] = the column sums of A (if given); fixed-order reduction.
template <typename T>
hipError_t col_wgrad_t(const ColWGradArgs& a, hipStream_t s) {
  const SegLayout L = seg_layout(a.npos, a.b_w);
  char* ws = static_cast<char*>(a.workspace);
  WGradParams w{};
  w.N = 0; w.ending = 0; w.npos = (int)a.npos;
  w.nseg = 1; w.a_w = a.a_w; w.a_zrow = 0; w.aseg[0] = a.a;
  w.dbias = nullptr; w.H = 0;
  w.b_w = a.b_w; w.b_zrow = 0; w.b_ln = 0; w.b = a.b; w.b_ld = a.b_ld; w.eps = 0.f;
  w.rows_pad = 128;
  chunking(a.npos, kChunks, w.nchunks, w.chunk_pos);
  w.part = reinterpret_cast<float*>(ws + L.part);
  w.cpart = reinterpret_cast<float*>(ws + L.cpart);
  hipError_t e = launch_wgrad<T>(w, s);
  if (e != hipSuccess) return e;
  FinishParams f{};
  f.nchunks = w.nchunks; f.rows_pad = w.rows_pad; f.ncols = a.b_w;
  f.nseg = 1; f.a_w = a.a_w; f.H = 0; f.has_bias = 0;
  f.part = w.part; f.cpart = w.cpart;
  f.ln = 0;
  f.dw[0] = a.dw; f.dcol[0] = a.dcol; f.ldw = a.dw_ld;
  return launch_finish<T>(f, reinterpret_cast<float*>(ws + L.part2),
                          reinterpret_cast<float*>(ws + L.cpart2), s);
}

template <typename T>
hipError_t seg_wgrad_t(const SegWGradArgs& a, hipStream_t s) {
  const SegLayout L = seg_layout(a.npos, a.ncols);
  char* ws = static_cast<char*>(a.workspace);
  WGradParams w{};
  w.N = 0; w.ending = 0; w.npos = (int)a.npos;  // plain rows: no z-row mapping
  w.nseg = a.nseg; w.a_w = 128; w.a_zrow = 0;
  for (int i = 0; i < a.nseg; ++i) w.aseg[i] = a.aseg[i];
  w.dbias = nullptr; w.H = 0;
  w.b_w = a.ncols; w.b_zrow = 0; w.b_ln = a.b_ln; w.b = a.b; w.eps = a.eps;
  w.rows_pad = a.nseg * 128;
  chunking(a.npos, kChunks, w.nchunks, w.chunk_pos);
  w.part = reinterpret_cast<float*>(ws + L.part);
  w.cpart = reinterpret_cast<float*>(ws + L.cpart);
  hipError_t e = launch_wgrad<T>(w, s);
  if (e != hipSuccess) return e;
  FinishParams f{};
  f.nchunks = w.nchunks; f.rows_pad = w.rows_pad; f.ncols = a.ncols;
  f.nseg = a.nseg; f.a_w = 128; f.H = 0; f.has_bias = 0;
  f.part = w.part; f.cpart = w.cpart;
  f.ln = a.b_ln; f.ln_w = a.ln_w; f.ln_b = a.ln_b;
  for (int i = 0; i < a.nseg; ++i) f.dw[i] = a.dw[i];
  f.mred = a.mred; f.cred = a.cred;
  return launch_finish<T>(f, reinterpret_cast<float*>(ws + L.part2),
                          reinterpret_cast<float*>(ws + L.cpart2), s);
}

}  // namespace

size_t seg_wgrad_workspace(int64_t npos, int64_t ncols) { return seg_layout(npos, ncols).total; }

hipError_t launch_seg_wgrad(const SegWGradArgs& a, hipStream_t s) {
  if ((a.nseg != 1 && a.nseg != 4) || a.ncols > 128 || a.ncols % 16 != 0)
    return hipErrorInvalidValue;
  return a.dtype == 1 ? seg_wgrad_t<bf16_t>(a, s) : seg_wgrad_t<float>(a, s);
}

size_t proj_bwd_workspace(int64_t N, int64_t CZ, int64_t H) {
  return part_layout(N, CZ, H).total;
}

hipError_t launch_out_project_bwd(const OutProjectBwdArgs& a, hipStream_t s) {
  return a.dtype == 1 ? out_project_bwd_t<bf16_t>(a, s) : out_project_bwd_t<float>(a, s);
}

hipError_t launch_project_bwd(const ProjectBwdArgs& a, hipStream_t s) {
  return a.dtype == 1 ? project_bwd_t<bf16_t>(a, s) : project_bwd_t<float>(a, s);
}

size_t ln_proj_bwd_workspace(int64_t npos, int64_t CZ, int seg_w) {
  return ln_proj_layout(npos, CZ, seg_w).total;
}

size_t col_wgrad_workspace(int64_t npos, int b_w) { return seg_layout(npos, b_w).total; }

hipError_t launch_col_wgrad(const ColWGradArgs& a, hipStream_t s) {
  if (a.a_w % 32 != 0 || a.a_w > 128 || a.b_w % 16 != 0 || a.b_w > 256 || a.npos <= 0 ||
      a.npos > INT32_MAX)
    return hipErrorInvalidValue;
  return a.dtype == 1 ? col_wgrad_t<bf16_t>(a, s) : col_wgrad_t<float>(a, s);
}

hipError_t launch_ln_proj_bwd(const LnProjBwdArgs& a, hipStream_t s) {
  if (a.nseg != 2 || a.seg_w % 32 != 0 || a.seg_w > 128 || a.CZ % 32 != 0 || a.CZ > 256 ||
      (a.CZ > 128 && a.CZ != 256) || a.npos <= 0 || a.npos > INT32_MAX)
    return hipErrorInvalidValue;
  return a.dtype == 1 ? ln_proj_bwd_t<bf16_t>(a, s) : ln_proj_bwd_t<float>(a, s);
}

}  // namespace evo
