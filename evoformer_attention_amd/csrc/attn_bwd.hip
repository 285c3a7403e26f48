// Backward of biased, gated attention on gfx950.
//
// Logits are recomputed tile by tile from the saved log-sum-exp; neither the
// logits nor their gradients are ever stored (the forward-and-backward
// recompute of EvoFlash-3D, "MegaFold: Efficient Training of Next-Generation
// 3D Attention Protein Models on Cross-Platform GPUs", section
// "Methodologie", item 1).  The pair bias is shared by every row of a batch,
// so its gradient is the sum over rows of dS; that sum is accumulated in
// registers across the rows of a row group and reduced over row groups in a
// deterministic pass, in O(H * N^2) memory.
//
// Chain rule (natural-log units):
//   dO = dOut * sigmoid(G),  dG = dOut * Out * (1 - sigmoid(G)),
//   D[q] = sum_c dOut * Out,  P = exp(s - LSE),  dP = dO . V^T,
//   dS = P * (dP - D),  dV = P^T dO,  dK = dS^T Q / sqrt(C),
//   dQ = dS K / sqrt(C),  dBias = sum over rows of dS.
//
// Kernels:
//   prep      dO, dG, D, base-2 LSE, and transposed copies Q^T, dO^T, K^T
//             (one [C, N] slab per line and head) so that every MFMA operand
//             below is a contiguous 16-byte load; the base-2, mask-folded
//             pair bias in both orientations.
//   dkdv      one line, one head, 128 keys per workgroup (32 per wave);
//             loops over queries.  Lane = key in the accumulator layout:
//             S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS.
//   dq_dbias  32 queries of one head for a group of rows; the 4 waves split
//             the keys (64-key tiles, interleaved) and hold their part of
//             dBias in registers across the rows.  Lane = query:
//             S^T = K Q^T + bias, dP^T = V dO^T, dQ^T += K^T dS^T, with a
//             cross-wave LDS sum of dQ per row.
//   reduce    dBias = sum of the row-group partials.
#include "evo_device.h"
#include "evo_kernels.h"

namespace evo {
namespace {

constexpr int C = kHeadDim;
constexpr int kMaxTilesPerWave = 4;         // dq_dbias: keys <= 4 * 4 * 64
constexpr int kMaxKeysBwd = 4 * kMaxTilesPerWave * 64;
constexpr int kTargetGroups = 1024;         // dq_dbias workgroups wanted

int64_t pad64(int64_t n) { return (n + 63) / 64 * 64; }

struct BwdLayout {
  int64_t Np, n_rg, rows_per_group;
  size_t off_dopre, off_qt, off_dot, off_kt, off_lse2, off_d, off_bp, off_bpt,
      off_dbpart, total;
};

size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

BwdLayout bwd_layout(int dtype, int64_t B, int64_t R, int64_t N, int64_t H) {
  BwdLayout L{};
  const size_t es = dtype == 1 ? 2 : 4;
  L.Np = pad64(N);
  const int64_t nq = L.Np / 32;
  int64_t want = (kTargetGroups + B * H * nq - 1) / (B * H * nq);
  if (want < 1) want = 1;
  if (want > R) want = R;
  L.rows_per_group = (R + want - 1) / want;
  L.n_rg = (R + L.rows_per_group - 1) / L.rows_per_group;
  const size_t lines = (size_t)B * R * H;
  size_t o = 0;
  L.off_dopre = o; o += a256((size_t)B * R * N * H * C * es);
  L.off_qt = o;    o += a256(lines * C * L.Np * es);
  L.off_dot = o;   o += a256(lines * C * L.Np * es);
  L.off_kt = o;    o += a256(lines * C * L.Np * es);
  L.off_lse2 = o;  o += a256(lines * L.Np * 4);
  L.off_d = o;     o += a256(lines * L.Np * 4);
  L.off_bp = o;    o += a256((size_t)B * H * L.Np * L.Np * 4);
  L.off_bpt = o;   o += a256((size_t)B * H * L.Np * L.Np * 4);
  L.off_dbpart = o;
  if (L.n_rg > 1) o += a256((size_t)L.n_rg * B * H * L.Np * L.Np * 4);
  L.total = o;
  return L;
}

// Query held at slot s (0..31) of a 32-query step in the dK/dV kernel: the
// accumulator layout gives lane group g the queries 4g..4g+3 of each of the
// two 16-query blocks, which become the 8 contraction slots 8g..8g+7.
__device__ __forceinline__ int slot_query(int s) {
  const int gg = s >> 3, j = s & 7;
  return j < 4 ? 4 * gg + j : 16 + 4 * gg + (j - 4);
}

template <typename T>
__device__ __forceinline__ typename Tr<T>::Op ldop(const T* p);
template <>
__device__ __forceinline__ bf16x8 ldop<bf16_t>(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
template <>
__device__ __forceinline__ f32x8 ldop<float>(const float* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f32x8 r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

__device__ __forceinline__ f32x4 ld4(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  return f32x4{a.x, a.y, a.z, a.w};
}

struct BwdParams {
  const void* q; const void* k; const void* v; const void* gate;
  const uint8_t* mask; const void* bias; const void* out; const float* lse;
  const void* dout;
  void* dq; void* dk; void* dv; void* dgate; float* dbias;
  void* dopre;   // dO (= dout when there is no gate)
  void* qt; void* dot; void* kt;
  float* lse2; float* dd; float* bp; float* bpt; float* dbpart;
  int B, R, N, H, Np, mask_rows, n_rg, rows_per_group, row_mask;
  float qscale;  // log2(e) / sqrt(C)
};

// ----------------------------------------------------------------- prep
// Workgroup: one line (b, r), one head, 32 positions.  Thread: position
// t/8, dims 4*(t%8)..+3.
template <typename T>
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdParams p) {
  __shared__ float sQ[32][33], sK[32][33], sO[32][33];
  const int nblk = p.Np / 32;
  int w = blockIdx.x;
  const int nb = w % nblk; w /= nblk;
  const int h = w % p.H;
  const int line = w / p.H;  // b * R + r
  const int t = threadIdx.x, n = t >> 3, c4 = (t & 7) * 4;
  const int N = p.N, H = p.H;
  const int pos = nb * 32 + n;
  const int64_t e0 = ((int64_t)line * N + pos) * H * C + h * C + c4;
  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* Out = static_cast<const T*>(p.out);
  const T* dOut = static_cast<const T*>(p.dout);
  const T* G = static_cast<const T*>(p.gate);
  float dsum = 0.f;
  float qv[4] = {0, 0, 0, 0}, kv[4] = {0, 0, 0, 0}, dov[4] = {0, 0, 0, 0};
  if (pos < N) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv[i] = Tr<T>::to_f(Q[e0 + i]);
      kv[i] = Tr<T>::to_f(K[e0 + i]);
      const float o = Tr<T>::to_f(Out[e0 + i]);
      const float d = Tr<T>::to_f(dOut[e0 + i]);
      dsum += d * o;
      if (G) {
        const float sg = sigmoid_f(Tr<T>::to_f(G[e0 + i]));
        dov[i] = d * sg;
        static_cast<T*>(p.dgate)[e0 + i] = Tr<T>::from_f(d * o * (1.f - sg));
        static_cast<T*>(p.dopre)[e0 + i] = Tr<T>::from_f(dov[i]);
      } else {
        dov[i] = d;
      }
    }
  }
  dsum += __shfl_xor(dsum, 1, 64);
  dsum += __shfl_xor(dsum, 2, 64);
  dsum += __shfl_xor(dsum, 4, 64);
  const int64_t lh = (int64_t)line * H + h;  // line-head index
  if ((t & 7) == 0) {
    float l2 = INFINITY;  // padded or fully masked: P = exp2(-inf) = 0
    if (pos < N) {
      const float lse = p.lse[lh * N + pos];
      if (lse != -INFINITY) l2 = lse * kLog2e;
    }
    p.lse2[lh * p.Np + pos] = l2;
    p.dd[lh * p.Np + pos] = pos < N ? dsum : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sQ[n][c4 + i] = qv[i];
    sK[n][c4 + i] = kv[i];
    sO[n][c4 + i] = dov[i];
  }
  __syncthreads();
  // Transposed slabs: thread -> dim c = t/8, slots 4*(t%8)..+3.
  const int c = t >> 3, s0 = (t & 7) * 4;
  T* Qt = static_cast<T*>(p.qt) + (lh * C + c) * p.Np + nb * 32 + s0;
  T* Dt = static_cast<T*>(p.dot) + (lh * C + c) * p.Np + nb * 32 + s0;
  T* Kt = static_cast<T*>(p.kt) + (lh * C + c) * p.Np + nb * 32 + s0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qq = slot_query(s0 + i);
    Qt[i] = Tr<T>::from_f(sQ[qq][c]);
    Dt[i] = Tr<T>::from_f(sO[qq][c]);
    Kt[i] = Tr<T>::from_f(sK[s0 + i][c]);
  }
}

// Base-2 pair bias with the shared key mask folded in, both orientations.
// bp[b,h,q,k] (q < Np, k < Np), bpt[b,h,k,q]; keys >= N are -inf.
template <typename T>
__global__ void __launch_bounds__(256) bwd_bias_kernel(BwdParams p) {
  __shared__ float tile[32][33];
  const int nblk = p.Np / 32;
  int w = blockIdx.x;
  const int kb = w % nblk; w /= nblk;
  const int qb = w % nblk; w /= nblk;
  const int bh = w;  // b * H + h
  const int b = bh / p.H;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const T* Bias = static_cast<const T*>(p.bias);
  const int N = p.N;
  for (int yy = ty; yy < 32; yy += 8) {
    const int q = qb * 32 + yy, k = kb * 32 + tx;
    float v = -INFINITY;
    if (k < N) {
      v = 0.f;
      if (Bias && q < N) v = Tr<T>::to_f(Bias[((int64_t)bh * N + q) * N + k]) * kLog2e;
      if (p.mask && !p.row_mask && p.mask[(int64_t)b * p.mask_rows * N + k] == 0)
        v = -INFINITY;
    }
    p.bp[((int64_t)bh * p.Np + q) * p.Np + k] = v;
    tile[yy][tx] = v;
  }
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8) {
    const int k = kb * 32 + yy, q = qb * 32 + tx;
    p.bpt[((int64_t)bh * p.Np + k) * p.Np + q] = tile[tx][yy];
  }
}

// ----------------------------------------------------------------- dK, dV
template <typename T>
__global__ void __launch_bounds__(256) bwd_dkdv_kernel(BwdParams p) {
  using Op = typename Tr<T>::Op;
  // LDS per 32-query step: Q rows, dO rows (row-major, +pad) and the
  // slot-ordered Q^T and dO^T slabs; base-2 LSE and D.
  constexpr int RS = 40;  // elements per row (32 + pad) keeps 16-byte reads spread
  __shared__ __attribute__((aligned(32))) T sQ[32 * RS], sDO[32 * RS],
      sQt[32 * RS], sDOt[32 * RS];
  __shared__ float sL[32], sD[32];

  const int nkt = (p.N + 127) / 128;
  int w = blockIdx.x;
  const int kt = w % nkt; w /= nkt;
  const int h = w % p.H;
  const int line = w / p.H;   // b * R + r
  const int b = line / p.R, r = line - b * p.R;
  const int N = p.N, H = p.H, Np = p.Np;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t lh = (int64_t)line * H + h;
  const int pos_stride = H * C;
  const int64_t lbase = (int64_t)line * N * pos_stride + h * C;

  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);
  const T* Q = static_cast<const T*>(p.q);
  const T* DO = static_cast<const T*>(p.dopre);
  const T* QT = static_cast<const T*>(p.qt) + lh * C * Np;
  const T* DT = static_cast<const T*>(p.dot) + lh * C * Np;
  const float* BPT = p.bpt + (int64_t)(b * H + h) * Np * Np;
  const uint8_t* mrow = (p.mask && p.row_mask)
                            ? p.mask + ((int64_t)b * p.mask_rows + r) * N
                            : nullptr;

  // This wave's keys: kbase + kb*16 + l16 (kb = 0, 1).
  const int kbase = kt * 128 + wave * 32;
  Op kf[2], vf[2];
  bool kdead[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kbase + kb * 16 + l16;
    if (key < N) {
      kf[kb] = scale8(ldop<T>(K + lbase + (int64_t)key * pos_stride + 8 * g), p.qscale);
      vf[kb] = ldop<T>(V + lbase + (int64_t)key * pos_stride + 8 * g);
    } else {
      kf[kb] = Op{};
      vf[kb] = Op{};
    }
    kdead[kb] = key >= N || (mrow && mrow[key] == 0);
  }
  f32x4 dk[2][2], dv[2][2];  // [cb][kb]
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      dk[cb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv[cb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  for (int q0 = 0; q0 < N; q0 += 32) {
    __syncthreads();
    {  // stage: thread -> (row, 8-element chunk) of each of the 4 tiles
      const int row = (tid >> 2) & 31, ch = tid & 3, which = tid >> 7;  // 2 tiles per half
      for (int rep = 0; rep < 2; ++rep) {
        const int tile = which * 2 + rep;  // 0 Q, 1 dO, 2 Q^T, 3 dO^T
        T* dst;
        const T* src = nullptr;
        if (tile == 0) {
          dst = sQ + row * RS + ch * 8;
          if (q0 + row < N) src = Q + lbase + (int64_t)(q0 + row) * pos_stride + ch * 8;
        } else if (tile == 1) {
          dst = sDO + row * RS + ch * 8;
          if (q0 + row < N) src = DO + lbase + (int64_t)(q0 + row) * pos_stride + ch * 8;
        } else if (tile == 2) {
          dst = sQt + row * RS + ch * 8;
          src = QT + (int64_t)row * Np + q0 + ch * 8;
        } else {
          dst = sDOt + row * RS + ch * 8;
          src = DT + (int64_t)row * Np + q0 + ch * 8;
        }
        if (src) {
          *reinterpret_cast<Op*>(dst) = ldop<T>(src);
        } else {
          *reinterpret_cast<Op*>(dst) = Op{};
        }
      }
      if (tid < 32) {
        sL[tid] = p.lse2[lh * Np + q0 + tid];
        sD[tid] = p.dd[lh * Np + q0 + tid];
      }
    }
    __syncthreads();

    // S[qb][kb]: lane holds queries qb*16 + 4g + i for key kbase + kb*16 + l16.
    f32x4 s[2][2], dp[2][2];
    Op qa[2], da[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      qa[qb] = *reinterpret_cast<const Op*>(sQ + (qb * 16 + l16) * RS + 8 * g);
      da[qb] = *reinterpret_cast<const Op*>(sDO + (qb * 16 + l16) * RS + 8 * g);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = kbase + kb * 16 + l16;
        const f32x4 cbias = ld4(BPT + (int64_t)min(key, Np - 1) * Np + q0 + qb * 16 + 4 * g);
        s[qb][kb] = mma32(qa[qb], kf[kb], cbias);
        dp[qb][kb] = mma32(da[qb], vf[kb], f32x4{0.f, 0.f, 0.f, 0.f});
      }
    // P and dS (natural-log units for dS).
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const f32x4 l2 = *reinterpret_cast<const f32x4*>(&sL[qb * 16 + 4 * g]);
      const f32x4 dd = *reinterpret_cast<const f32x4*>(&sD[qb * 16 + 4 * g]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = kdead[kb] ? 0.f : exp2_fast(s[qb][kb][i] - l2[i]);
          s[qb][kb][i] = pv;
          dp[qb][kb][i] = pv * (dp[qb][kb][i] - dd[i]);
        }
    }
    // dV^T += dO^T P,  dK^T += Q^T dS  (contraction over the 32 query slots)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const Op pf = pack8(s[0][kb], s[1][kb], (Op*)nullptr);
      const Op sf = pack8(dp[0][kb], dp[1][kb], (Op*)nullptr);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const Op dot = *reinterpret_cast<const Op*>(sDOt + (cb * 16 + l16) * RS + 8 * g);
        const Op qtf = *reinterpret_cast<const Op*>(sQt + (cb * 16 + l16) * RS + 8 * g);
        dv[cb][kb] = mma32(dot, pf, dv[cb][kb]);
        dk[cb][kb] = mma32(qtf, sf, dk[cb][kb]);
      }
    }
  }

  // Store: lane holds dims cb*16 + 4g + i of key kbase + kb*16 + l16.
  T* DK = static_cast<T*>(p.dk);
  T* DV = static_cast<T*>(p.dv);
  const float ks = 1.f / sqrtf((float)C);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kbase + kb * 16 + l16;
    if (key >= N) continue;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int64_t off = lbase + (int64_t)key * pos_stride + cb * 16 + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        DK[off + i] = Tr<T>::from_f(dk[cb][kb][i] * ks);
        DV[off + i] = Tr<T>::from_f(dv[cb][kb][i]);
      }
    }
  }
}

// ------------------------------------------------------------- dQ, dBias
// LDS row of physical key p within a 64-key tile (see attn_fwd.hip): the
// A-operand lane m of block (half, kb) holds key half*32 + 8*(m/4) + 4*kb + m%4.
__device__ __forceinline__ int perm_key(int half, int kb, int m) {
  return half * 32 + 8 * (m >> 2) + 4 * kb + (m & 3);
}

template <typename T, int TPW>
__global__ void __launch_bounds__(256) bwd_dq_dbias_kernel(BwdParams p) {
  using Op = typename Tr<T>::Op;
  __shared__ __attribute__((aligned(16))) float sRed[4][2][2][64][4];  // [wave][qb][cb][lane][i]

  const int nqt = p.Np / 32;
  int w = xcd_work_index(p.B * p.H * nqt * p.n_rg);
  if (w < 0) return;
  const int qt = w % nqt; w /= nqt;
  const int rg = w % p.n_rg; w /= p.n_rg;
  const int h = w % p.H;
  const int b = w / p.H;
  const int N = p.N, H = p.H, R = p.R, Np = p.Np;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int pos_stride = H * C;
  const int q0 = qt * 32;
  const int bh = b * H + h;
  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);
  const T* DO = static_cast<const T*>(p.dopre);
  const T* KT = static_cast<const T*>(p.kt);
  const float* BP = p.bp + (int64_t)bh * Np * Np;

  f32x4 db[TPW][2][2][2];  // [tile][qb][half][kb]
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) db[t][qb][half][kb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int r_begin = rg * p.rows_per_group;
  const int r_end = min(R, r_begin + p.rows_per_group);
  for (int r = r_begin; r < r_end; ++r) {
    const int64_t line = (int64_t)b * R + r;
    const int64_t lbase = line * N * pos_stride + h * C;
    const int64_t lh = line * H + h;
    const uint8_t* mrow = (p.mask && p.row_mask) ? p.mask + ((int64_t)b * p.mask_rows + r) * N
                                                 : nullptr;
    Op qf[2], df[2];
    float l2[2], dd[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int q = q0 + qb * 16 + l16;
      if (q < N) {
        qf[qb] = scale8(ldop<T>(Q + lbase + (int64_t)q * pos_stride + 8 * g), p.qscale);
        df[qb] = ldop<T>(DO + lbase + (int64_t)q * pos_stride + 8 * g);
      } else {
        qf[qb] = Op{};
        df[qb] = Op{};
      }
      l2[qb] = p.lse2[lh * Np + q];
      dd[qb] = p.dd[lh * Np + q];
    }
    f32x4 dq[2][2];  // [qb][cb]
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) dq[qb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int k0 = (wave + 4 * t) * 64;
      if (k0 >= N) continue;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x4 s[2][2], dp[2][2];  // [qb][kb]
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int key = k0 + perm_key(half, kb, l16);
          Op kf = Op{}, vf = Op{};
          if (key < N) {
            kf = ldop<T>(K + lbase + (int64_t)key * pos_stride + 8 * g);
            vf = ldop<T>(V + lbase + (int64_t)key * pos_stride + 8 * g);
          }
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const int q = q0 + qb * 16 + l16;
            const float* bsrc = BP + (int64_t)q * Np + k0 + half * 32 + 8 * g + 4 * kb;
            s[qb][kb] = mma32(kf, qf[qb], ld4(bsrc));
            dp[qb][kb] = mma32(vf, df[qb], f32x4{0.f, 0.f, 0.f, 0.f});
          }
        }
        // P and dS; keys of this lane: k0 + half*32 + 8g + 4kb + i.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          bool dead[4] = {false, false, false, false};
          if (mrow) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = k0 + half * 32 + 8 * g + 4 * kb + i;
              dead[i] = key < N && mrow[key] == 0;
            }
          }
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float pv = dead[i] ? 0.f : exp2_fast(s[qb][kb][i] - l2[qb]);
              const float ds = pv * (dp[qb][kb][i] - dd[qb]);
              dp[qb][kb][i] = ds;
              db[t][qb][half][kb][i] += ds;
            }
        }
        // dQ^T += K^T dS^T over this half's 32 keys.
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const T* ksrc = KT + (lh * C + cb * 16 + l16) * Np + k0 + half * 32 + 8 * g;
          const Op ktf = ldop<T>(ksrc);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const Op sf = pack8(dp[qb][0], dp[qb][1], (Op*)nullptr);
            dq[qb][cb] = mma32(ktf, sf, dq[qb][cb]);
          }
        }
      }
    }
    // Sum the four waves' partial dQ and store.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        *reinterpret_cast<f32x4*>(&sRed[wave][qb][cb][lane][0]) = dq[qb][cb];
    __syncthreads();
    {
      // thread -> (qb, cb, lane): 2*2*64 = 256 outputs of 4 values
      const int qb = tid >> 7, cb = (tid >> 6) & 1, ln = tid & 63;
      f32x4 acc = *reinterpret_cast<const f32x4*>(&sRed[0][qb][cb][ln][0]);
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) acc += *reinterpret_cast<const f32x4*>(&sRed[ww][qb][cb][ln][0]);
      const int q = q0 + qb * 16 + (ln & 15);
      if (q < N) {
        const float ks = 1.f / sqrtf((float)C);
        T* dst = static_cast<T*>(p.dq) + lbase + (int64_t)q * pos_stride + cb * 16 + 4 * (ln >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = Tr<T>::from_f(acc[i] * ks);
      }
    }
    __syncthreads();
  }

  // dBias partial of this row group (or the final value with one group).
  if (!p.dbias) return;
  float* dst = (p.n_rg == 1) ? nullptr : p.dbpart + ((int64_t)rg * p.B * H + bh) * Np * Np;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int k0 = (wave + 4 * t) * 64;
    if (k0 >= N) continue;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int q = q0 + qb * 16 + l16;
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int kk = k0 + half * 32 + 8 * g + 4 * kb;
          if (dst) {
            *reinterpret_cast<f32x4*>(dst + (int64_t)q * Np + kk) = db[t][qb][half][kb];
          } else if (q < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (kk + i < N) p.dbias[((int64_t)bh * N + q) * N + kk + i] = db[t][qb][half][kb][i];
          }
        }
    }
  }
}

// dBias[b,h,q,k] = sum over row groups of the partials.
__global__ void __launch_bounds__(256) bwd_dbias_reduce_kernel(BwdParams p) {
  const int64_t total = (int64_t)p.B * p.H * p.N * p.N;
  const int64_t stride = (int64_t)p.B * p.H * p.Np * p.Np;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int64_t k = e % p.N;
    int64_t t = e / p.N;
    const int64_t q = t % p.N;
    const int64_t bh = t / p.N;
    const int64_t src = (bh * p.Np + q) * p.Np + k;
    float acc = 0.f;
    for (int rg = 0; rg < p.n_rg; ++rg) acc += p.dbpart[rg * stride + src];
    p.dbias[e] = acc;
  }
}

template <typename T>
hipError_t launch_t(BwdParams& p, hipStream_t s) {
  const int64_t lines = (int64_t)p.B * p.R;
  const int nblk = p.Np / 32;
  hipLaunchKernelGGL(bwd_prep_kernel<T>, dim3((unsigned)(lines * p.H * nblk)), dim3(256), 0,
                     s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_bias_kernel<T>, dim3((unsigned)(p.B * p.H * nblk * nblk)), dim3(256),
                     0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nkt = (p.N + 127) / 128;
  hipLaunchKernelGGL(bwd_dkdv_kernel<T>, dim3((unsigned)(lines * p.H * nkt)), dim3(256), 0, s,
                     p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int total = p.B * p.H * (p.Np / 32) * p.n_rg;
  const int grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
  const int tiles = (int)((p.N + 63) / 64);
  const int tpw = (tiles + 3) / 4;
  switch (tpw) {
    case 1: hipLaunchKernelGGL((bwd_dq_dbias_kernel<T, 1>), dim3(grid), dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((bwd_dq_dbias_kernel<T, 2>), dim3(grid), dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL((bwd_dq_dbias_kernel<T, 3>), dim3(grid), dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((bwd_dq_dbias_kernel<T, 4>), dim3(grid), dim3(256), 0, s, p); break;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.n_rg > 1 && p.dbias) {
    hipLaunchKernelGGL(bwd_dbias_reduce_kernel, dim3(2048), dim3(256), 0, s, p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

size_t attn_bwd_workspace(int dtype, int64_t B, int64_t R, int64_t N,
                          int64_t H) {
  if (N > kMaxKeysBwd) return 0;
  return bwd_layout(dtype, B, R, N, H).total;
}

hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t s) {
  if (a.N > kMaxKeysBwd) return hipErrorInvalidValue;
  const BwdLayout L = bwd_layout(a.dtype, a.B, a.R, a.N, a.H);
  char* ws = static_cast<char*>(a.workspace);
  BwdParams p{};
  p.q = a.q; p.k = a.k; p.v = a.v; p.gate = a.gate; p.mask = a.mask;
  p.bias = a.bias; p.out = a.out; p.lse = a.lse; p.dout = a.dout;
  p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.dgate = a.dgate; p.dbias = a.dbias;
  p.dopre = a.gate ? (void*)(ws + L.off_dopre) : const_cast<void*>(a.dout);
  p.qt = ws + L.off_qt;
  p.dot = ws + L.off_dot;
  p.kt = ws + L.off_kt;
  p.lse2 = reinterpret_cast<float*>(ws + L.off_lse2);
  p.dd = reinterpret_cast<float*>(ws + L.off_d);
  p.bp = reinterpret_cast<float*>(ws + L.off_bp);
  p.bpt = reinterpret_cast<float*>(ws + L.off_bpt);
  p.dbpart = reinterpret_cast<float*>(ws + L.off_dbpart);
  p.B = (int)a.B; p.R = (int)a.R; p.N = (int)a.N; p.H = (int)a.H;
  p.Np = (int)L.Np;
  p.mask_rows = a.mask ? (int)a.mask_rows : 1;
  p.row_mask = a.mask && a.mask_rows > 1;
  p.n_rg = (int)L.n_rg;
  p.rows_per_group = (int)L.rows_per_group;
  p.qscale = kLog2e / sqrtf((float)C);
  return a.dtype == 1 ? launch_t<bf16_t>(p, s) : launch_t<float>(p, s);
}

}  // namespace evo
