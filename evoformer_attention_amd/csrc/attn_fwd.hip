// Forward of biased, gated attention on gfx950.
//
// Per attention line (b, r), head h:
//   Out[q] = sigmoid(G[q]) * sum_k softmax_k(<Q[q],K[k]>/sqrt(C) + bias[b,h,q,k]
//                                           + mask[k]) V[k]
// computed tile by tile with an online softmax, so the [N, N] logits of a
// line live only in registers (the memory wall of "Evoformer: the memory wall
// ZeRO cannot move", section "Where the memory goes"; the tiled online-softmax
// scheme of EvoFlash-3D in "MegaFold: Efficient Training of Next-Generation 3D
// Attention Protein Models on Cross-Platform GPUs", section "Methodologie",
// item 1).
//
// Work decomposition.  A workgroup (4 waves) owns 128 queries of one head
// and ROWS lines of one batch entry; each wave owns 32 queries.  Keys stream
// in tiles of 64.  The pair bias is the same for every line of a batch, so a
// bias tile is loaded once (converted to fp32, scaled to base 2, masked) and
// used for all ROWS lines of the workgroup.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, fp32 accumulate):
//   S^T = K . Q^T + bias^T   A = 16 keys x 32 dims (LDS), B = Q^T held in
//                            registers for the whole line, C = bias tile.
//   O^T += V^T . P^T         A = V^T from LDS, B = P^T taken straight from
//                            the S^T accumulators (no LDS round trip).
// In the accumulator layout a lane holds one query and 4 keys per 16-key
// block; the key order inside a tile is permuted so that each lane's 8
// keys of a 32-key half are consecutive, which makes the P^T operand
// exactly the registers the lane already holds, the bias/mask loads 16-byte
// vectors, and the V^T operand one 16-byte LDS read.
#include "evo_device.h"
#include "evo_kernels.h"

namespace evo {
namespace {

constexpr int C = kHeadDim;
constexpr int BK = 64;            // keys per tile
constexpr int BQW = 32;           // queries per wave
constexpr int WAVES = 4;
constexpr int BQ = BQW * WAVES;   // queries per workgroup
constexpr int kRowsShared = 2;    // lines per workgroup when masks are shared

template <typename T> struct FwdLds;
// Row strides (elements) of the LDS K tile [64 keys][32 dims] and V^T tile
// [32 dims][64 keys]; the padding spreads 16-byte reads over all banks.
template <> struct FwdLds<bf16_t> { static constexpr int KST = 40, VST = 72; };
template <> struct FwdLds<float> { static constexpr int KST = 36, VST = 68; };

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* gate;
  const uint8_t* mask;
  const void* bias;
  void* out;
  float* lse;
  int B, R, N, H, mask_rows;
  int n_qt, n_rg, total;
  float qscale;   // log2(e) / sqrt(C): logits are kept in base 2
  int vec_ok;     // N % 8 == 0: bias and mask rows allow 8-element vectors
};

// LDS row of physical key p (0..63) of a tile: A-operand lane m of block
// (half, kb) reads LDS row half*32 + kb*16 + m, which must hold physical key
// half*32 + 8*(m/4) + 4*kb + m%4.
__device__ __forceinline__ int k_lds_row(int p) {
  const int half = p >> 5, pp = p & 31;
  const int gg = pp >> 3, kb = (pp >> 2) & 1, i = pp & 3;
  return half * 32 + kb * 16 + gg * 4 + i;
}

// 16-byte-granular copies (fragments of 8 elements).
__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ f32x8 ld8(const float* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 4);
  f32x8 r;
  r[0] = __uint_as_float(a.x); r[1] = __uint_as_float(a.y);
  r[2] = __uint_as_float(a.z); r[3] = __uint_as_float(a.w);
  r[4] = __uint_as_float(b.x); r[5] = __uint_as_float(b.y);
  r[6] = __uint_as_float(b.z); r[7] = __uint_as_float(b.w);
  return r;
}
__device__ __forceinline__ void copy8(bf16_t* dst, const bf16_t* src) {
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}
__device__ __forceinline__ void copy8(float* dst, const float* src) {
  reinterpret_cast<uint4*>(dst)[0] = reinterpret_cast<const uint4*>(src)[0];
  reinterpret_cast<uint4*>(dst)[1] = reinterpret_cast<const uint4*>(src)[1];
}
__device__ __forceinline__ void zero8(bf16_t* dst) {
  *reinterpret_cast<uint4*>(dst) = make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ void zero8(float* dst) {
  reinterpret_cast<uint4*>(dst)[0] = make_uint4(0, 0, 0, 0);
  reinterpret_cast<uint4*>(dst)[1] = make_uint4(0, 0, 0, 0);
}

// Four consecutive elements -> fp32.
__device__ __forceinline__ f32x4 ld4f(const bf16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  f32x4 r;
  r[0] = __uint_as_float(u.x << 16);
  r[1] = __uint_as_float(u.x & 0xffff0000u);
  r[2] = __uint_as_float(u.y << 16);
  r[3] = __uint_as_float(u.y & 0xffff0000u);
  return r;
}
__device__ __forceinline__ f32x4 ld4f(const float* p) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  f32x4 r;
  r[0] = u.x; r[1] = u.y; r[2] = u.z; r[3] = u.w;
  return r;
}
__device__ __forceinline__ void st4f(bf16_t* p, const f32x4& v) {
  uint2 u;
  u.x = uint32_t(Tr<bf16_t>::from_f(v[0])) |
        (uint32_t(Tr<bf16_t>::from_f(v[1])) << 16);
  u.y = uint32_t(Tr<bf16_t>::from_f(v[2])) |
        (uint32_t(Tr<bf16_t>::from_f(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}
__device__ __forceinline__ void st4f(float* p, const f32x4& v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// Stage the K tile (key-permuted rows) and the V^T tile of one line.
template <typename T>
__device__ __forceinline__ void stage_kv(T* sK, T* sV, const T* kline,
                                         const T* vline, int k0, int N,
                                         int pos_stride) {
  constexpr int KST = FwdLds<T>::KST, VST = FwdLds<T>::VST;
  const int t = threadIdx.x;
  {  // K: thread -> (key, 8-dim chunk)
    const int kk = t >> 2, ch = t & 3;
    T* dst = sK + k_lds_row(kk) * KST + ch * 8;
    if (k0 + kk < N)
      copy8(dst, kline + (int64_t)(k0 + kk) * pos_stride + ch * 8);
    else
      zero8(dst);
  }
  {  // V: thread -> (key pair, 4-dim chunk), written transposed
    const int p = t & 31, ch = t >> 5;
    const int ka = k0 + 2 * p, kb = ka + 1;
    if constexpr (sizeof(T) == 2) {
      uint2 a = make_uint2(0, 0), b = make_uint2(0, 0);
      if (ka < N)
        a = *reinterpret_cast<const uint2*>(vline + (int64_t)ka * pos_stride + ch * 4);
      if (kb < N)
        b = *reinterpret_cast<const uint2*>(vline + (int64_t)kb * pos_stride + ch * 4);
      uint32_t* d = reinterpret_cast<uint32_t*>(sV);
      const int base = ((ch * 4) * VST + 2 * p) >> 1;
      const int rs = VST >> 1;
      d[base + 0 * rs] = (a.x & 0xffffu) | (b.x << 16);
      d[base + 1 * rs] = (a.x >> 16) | (b.x & 0xffff0000u);
      d[base + 2 * rs] = (a.y & 0xffffu) | (b.y << 16);
      d[base + 3 * rs] = (a.y >> 16) | (b.y & 0xffff0000u);
    } else {
      float4 a = make_float4(0, 0, 0, 0), b = make_float4(0, 0, 0, 0);
      if (ka < N)
        a = *reinterpret_cast<const float4*>(vline + (int64_t)ka * pos_stride + ch * 4);
      if (kb < N)
        b = *reinterpret_cast<const float4*>(vline + (int64_t)kb * pos_stride + ch * 4);
      float2* d0 = reinterpret_cast<float2*>(sV + (ch * 4 + 0) * VST + 2 * p);
      float2* d1 = reinterpret_cast<float2*>(sV + (ch * 4 + 1) * VST + 2 * p);
      float2* d2 = reinterpret_cast<float2*>(sV + (ch * 4 + 2) * VST + 2 * p);
      float2* d3 = reinterpret_cast<float2*>(sV + (ch * 4 + 3) * VST + 2 * p);
      *d0 = make_float2(a.x, b.x);
      *d1 = make_float2(a.y, b.y);
      *d2 = make_float2(a.z, b.z);
      *d3 = make_float2(a.w, b.w);
    }
  }
}

// Base-2, masked bias for 8 consecutive keys [kbase, kbase+8) of query q:
// returned as two accumulator quads (keys kbase..+3, kbase+4..+7).
template <typename T>
__device__ __forceinline__ void bias8(const FwdParams& p, const T* brow,
                                      const uint8_t* mrow, int kbase,
                                      f32x4& lo, f32x4& hi) {
  float x[8];
  const int N = p.N;
  if (p.vec_ok && kbase + 8 <= N) {
    if (brow) {
      const f32x4 a = ld4f(brow + kbase), b = ld4f(brow + kbase + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = a[j] * kLog2e;
        x[4 + j] = b[j] * kLog2e;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.f;
    }
    if (mrow) {
      const uint2 m = *reinterpret_cast<const uint2*>(mrow + kbase);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (((m.x >> (8 * j)) & 0xffu) == 0) x[j] = -INFINITY;
        if (((m.y >> (8 * j)) & 0xffu) == 0) x[4 + j] = -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kk = kbase + j;
      float b = -INFINITY;
      if (kk < N) {
        b = brow ? Tr<T>::to_f(brow[kk]) * kLog2e : 0.f;
        if (mrow && mrow[kk] == 0) b = -INFINITY;
      }
      x[j] = b;
    }
  }
  lo[0] = x[0]; lo[1] = x[1]; lo[2] = x[2]; lo[3] = x[3];
  hi[0] = x[4]; hi[1] = x[5]; hi[2] = x[6]; hi[3] = x[7];
}

template <typename T, int ROWS>
__global__ void __launch_bounds__(256)
attn_fwd_kernel(FwdParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int KST = FwdLds<T>::KST, VST = FwdLds<T>::VST;
  __shared__ __attribute__((aligned(16))) T sK[ROWS][BK * KST];
  __shared__ __attribute__((aligned(16))) T sV[ROWS][C * VST];

  const int w = xcd_work_index(p.total);
  if (w < 0) return;
  const int qt = w % p.n_qt;
  int t = w / p.n_qt;
  const int rg = t % p.n_rg;
  t /= p.n_rg;
  const int h = t % p.H;
  const int b = t / p.H;

  const int N = p.N, H = p.H, R = p.R;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int r0 = rg * ROWS;
  const int qw0 = qt * BQ + wave * BQW;
  const int pos_stride = H * C;                       // between positions n
  const int64_t line_stride = (int64_t)N * pos_stride;  // between lines r

  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);
  const T* Bias = static_cast<const T*>(p.bias);

  // Per-line state.
  Op qf[ROWS][2];
  f32x4 o[ROWS][2][2];
  float m[ROWS][2], l[ROWS][2];
#pragma unroll
  for (int rr = 0; rr < ROWS; ++rr) {
    const int r = r0 + rr;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int q = qw0 + qb * 16 + l16;
      if (r < R && q < N) {
        const T* src = Q + ((int64_t)b * R + r) * line_stride +
                       (int64_t)q * pos_stride + h * C + 8 * g;
        qf[rr][qb] = scale8(ld8(src), p.qscale);
      } else {
        qf[rr][qb] = Op{};
      }
      m[rr][qb] = -INFINITY;
      l[rr][qb] = 0.f;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) o[rr][qb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // Bias rows of this wave's queries (null when there is no bias); the
  // mask row is shared by all lines here (per-line masks use ROWS == 1).
  const T* brow[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q = qw0 + qb * 16 + l16;
    brow[qb] = (Bias && q < N) ? Bias + (((int64_t)b * H + h) * N + q) * N
                               : nullptr;
  }
  const uint8_t* mrow = nullptr;
  if (p.mask) {
    const int mr = (p.mask_rows == 1) ? 0 : r0;
    mrow = p.mask + ((int64_t)b * p.mask_rows + mr) * N;
  }

  for (int k0 = 0; k0 < N; k0 += BK) {
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr) {
      const int r = r0 + rr;
      if (r < R) {
        const int64_t lo = ((int64_t)b * R + r) * line_stride + h * C;
        stage_kv<T>(sK[rr], sV[rr], K + lo, V + lo, k0, N, pos_stride);
      }
    }
    // Bias tile in accumulator layout: bt[qb][half][kb].
    f32x4 bt[2][2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        bias8<T>(p, brow[qb], mrow, k0 + half * 32 + 8 * g, bt[qb][half][0],
                 bt[qb][half][1]);
    __syncthreads();

#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr) {
      if (r0 + rr >= R) continue;
      const T* kt = sK[rr];
      const T* vt = sV[rr];
      f32x4 s[2][2][2];  // [qb][half][kb]
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const Op kf = ld8(kt + (half * 32 + kb * 16 + l16) * KST + 8 * g);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            s[qb][half][kb] = mma32(kf, qf[rr][qb], bt[qb][half][kb]);
        }

#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[qb][half][kb][i]);
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float mnew = fmaxf(m[rr][qb], mx);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = exp2_fast(m[rr][qb] - muse);
        m[rr][qb] = mnew;
        float ls = 0.f;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float e = exp2_fast(s[qb][half][kb][i] - muse);
              s[qb][half][kb][i] = e;
              ls += e;
            }
        l[rr][qb] = l[rr][qb] * alpha + ls;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) o[rr][qb][cb] *= alpha;
      }

#pragma unroll
      for (int half = 0; half < 2; ++half) {
        Op vf[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          vf[cb] = ld8(vt + (cb * 16 + l16) * VST + half * 32 + 8 * g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const Op pf = pack8(s[qb][half][0], s[qb][half][1], (Op*)nullptr);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
            o[rr][qb][cb] = mma32(vf[cb], pf, o[rr][qb][cb]);
        }
      }
    }
  }

  // Epilogue: normalise, gate, store; LSE in natural log.
  const T* G = static_cast<const T*>(p.gate);
  T* Out = static_cast<T*>(p.out);
#pragma unroll
  for (int rr = 0; rr < ROWS; ++rr) {
    const int r = r0 + rr;
    if (r >= R) continue;
    const int64_t lo = ((int64_t)b * R + r) * line_stride + h * C;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float lt = l[rr][qb];
      lt += shfl_xor(lt, 16);
      lt += shfl_xor(lt, 32);
      const int q = qw0 + qb * 16 + l16;
      if (q >= N) continue;
      const float inv = lt > 0.f ? rcp_fast(lt) : 0.f;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int c = cb * 16 + 4 * g;
        const int64_t off = lo + (int64_t)q * pos_stride + c;
        f32x4 val = o[rr][qb][cb] * inv;
        if (G) {
          const f32x4 gv = ld4f(G + off);
#pragma unroll
          for (int i = 0; i < 4; ++i) val[i] *= sigmoid_f(gv[i]);
        }
        st4f(Out + off, val);
      }
      if (p.lse && g == 0) {
        p.lse[(((int64_t)b * R + r) * H + h) * N + q] =
            lt > 0.f ? (m[rr][qb] + log2_fast(lt)) * kLn2 : -INFINITY;
      }
    }
  }
}

template <typename T, int ROWS>
hipError_t launch_t(const FwdParams& p, hipStream_t s) {
  const int grid = ((p.total + kNumXcd - 1) / kNumXcd) * kNumXcd;
  hipLaunchKernelGGL((attn_fwd_kernel<T, ROWS>), dim3(grid), dim3(256), 0, s,
                     p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnFwdArgs& a, hipStream_t s) {
  FwdParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.gate = a.gate;
  p.mask = a.mask; p.bias = a.bias; p.out = a.out; p.lse = a.lse;
  p.B = (int)a.B; p.R = (int)a.R; p.N = (int)a.N; p.H = (int)a.H;
  p.mask_rows = a.mask ? (int)a.mask_rows : 1;
  p.qscale = kLog2e / sqrtf((float)C);
  p.vec_ok = (a.N % 8 == 0);
  // Lines share the bias tile; a per-line mask is folded into it, so then
  // each workgroup takes one line.
  const bool per_line_mask = a.mask && a.mask_rows > 1;
  const int rows = per_line_mask ? 1 : (a.dtype == 1 ? kRowsShared : 1);
  p.n_qt = (int)((a.N + BQ - 1) / BQ);
  p.n_rg = (int)((a.R + rows - 1) / rows);
  const int64_t total = a.B * a.H * (int64_t)p.n_rg * p.n_qt;
  if (total > (int64_t)INT32_MAX - 8) return hipErrorInvalidValue;
  p.total = (int)total;
  if (a.dtype == 1) {
    return rows == 1 ? launch_t<bf16_t, 1>(p, s)
                     : launch_t<bf16_t, kRowsShared>(p, s);
  }
  return launch_t<float, 1>(p, s);
}

}  // namespace evo
