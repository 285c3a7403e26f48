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
//   prep      an elementwise pass: dO, dG, -D and the base-2 LSE.
//   bias      the mask-folded pair bias, in the fragment orders of the dQ /
//             dBias kernels and (transposed) of the dK/dV kernel (fp16 for
//             bf16 inputs, as in the forward, fp32 for fp32).  The dK/dV and
//             dQ kernels prescale their resident Q or K operand by
//             log2(e)/sqrt(C) and start the logit product from -LSE (base 2),
//             so the exponent is the product plus bias*log2(e): one
//             mixed-precision FMA per logit straight from the fp16 bias.
//   dkdv      one line, one head, 128 keys per workgroup (32 per wave);
//             loops over 32-query steps staged through double-buffered LDS
//             (next step prefetched into registers).  Lane = key in the
//             accumulator layout: S = Q K^T + bias, dP = dO V^T,
//             dV^T += dO^T P, dK^T += Q^T dS; the transposed operands dO^T
//             and Q^T are read from the row-major tiles with transposing LDS
//             reads (bf16).
//   dq        one line, one head, 128 queries; loops over 64-key tiles in
//             double-buffered LDS.  Lane = query: S^T = K Q^T + bias,
//             dP^T = V dO^T, dQ^T += K^T dS^T (K^T likewise read transposed).
//   dbias     one head, a 128-query x 64-key tile, for a group of rows: the
//             bias tile and the dBias accumulator stay in registers while
//             the rows stream by (rows innermost), so the sum over rows
//             never leaves the chip until the group is done.
//   reduce    dBias = sum of the row-group partials (deterministic order).
#include <algorithm>

#include "evo_device.h"
#include "evo_kernels.h"

namespace evo {
namespace {

constexpr int C = kHeadDim;
constexpr float kSqrtC = 5.656854249492380f;  // sqrt(C)
static_assert(C == 32, "kSqrtC is sqrt(32)");
constexpr int kMaxKeysBwd = 1 << 16;
constexpr int kTargetGroups = 2048;         // dbias workgroups wanted

int64_t pad64(int64_t n) { return (n + 63) / 64 * 64; }
int64_t pad128(int64_t n) { return (n + 127) / 128 * 128; }

struct BwdLayout {
  int64_t Np, n_rg, rows_per_group;
  size_t off_dopre, off_lse2, off_d, off_bp, off_bpt,
      off_dbpart, total;
};

size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

BwdLayout bwd_layout(int dtype, int64_t B, int64_t R, int64_t N, int64_t H) {
  BwdLayout L{};
  const size_t es = dtype == 1 ? 2 : 4;
  L.Np = pad64(N);
  const int64_t tiles = B * H * ((N + 127) / 128) * (L.Np / 64);  // dbias tiles
  int64_t want = (kTargetGroups + tiles - 1) / tiles;
  if (want < 1) want = 1;
  if (want > R) want = R;
  L.rows_per_group = (R + want - 1) / want;
  L.n_rg = (R + L.rows_per_group - 1) / L.rows_per_group;
  const size_t lines = (size_t)B * R * H;
  size_t o = 0;
  L.off_dopre = o; o += a256((size_t)B * R * N * H * C * es);
  L.off_lse2 = o;  o += a256(lines * L.Np * 4);
  L.off_d = o;     o += a256(lines * L.Np * 4);
  L.off_bp = o;    o += a256((size_t)B * H * pad128(N) * L.Np * es);
  L.off_bpt = o;   o += a256((size_t)B * H * pad128(N) * L.Np * es);
  L.off_dbpart = o;
  if (L.n_rg > 1) o += a256((size_t)L.n_rg * B * H * L.Np * L.Np * 4);
  L.total = o;
  return L;
}

// Slot (0..31) of query q in a 32-query step of the dK/dV kernel: the
// accumulator layout gives lane group g the queries 4g..4g+3 of each of the
// two 16-query blocks, which become the 8 contraction slots 8g..8g+7, so
// query 4g + i sits at slot 8g + i and query 16 + 4g + i at slot 8g + 4 + i.
__device__ __forceinline__ int query_slot(int q) {
  return q < 16 ? 8 * (q >> 2) + (q & 3) : 8 * ((q - 16) >> 2) + 4 + (q & 3);
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

// Four consecutive elements <-> fp32.
__device__ __forceinline__ f32x4 ld4e(const bf16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
               __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ f32x4 ld4e(const float* p) { return ld4(p); }
__device__ __forceinline__ void st4e(bf16_t* p, const f32x4& v) {
  uint2 u;
  u.x = uint32_t(Tr<bf16_t>::from_f(v[0])) | (uint32_t(Tr<bf16_t>::from_f(v[1])) << 16);
  u.y = uint32_t(Tr<bf16_t>::from_f(v[2])) | (uint32_t(Tr<bf16_t>::from_f(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}
__device__ __forceinline__ void st4e(float* p, const f32x4& v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

struct BwdParams {
  const void* q; const void* k; const void* v; const void* gate;
  const uint8_t* mask; const void* bias; const void* out; const float* lse;
  const void* dout;
  void* dq; void* dk; void* dv; void* dgate; float* dbias;
  void* dopre;   // dO (= dout when there is no gate)
  float* lse2; float* dd; float* dbpart;
  void* bp; void* bpt;  // pair bias, natural units, masked, working dtype
  int B, R, N, H, Np, mask_rows, n_rg, rows_per_group, row_mask;
  float qscale;  // 1 / sqrt(C)
  float lscale;  // log2(e) / sqrt(C), the forward's scale of Q
};

// ----------------------------------------------------------------- prep
// Workgroup: one line (b, r), one head, 32 positions.  Thread: position
// t/8, dims 4*(t%8)..+3.
template <typename T>
__device__ __forceinline__ void ld_chunk(const T* p, float (&v)[16 / sizeof(T)]) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(p);
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(u[i]);
  }
}
template <typename T>
__device__ __forceinline__ void st_chunk(T* p, const float (&v)[16 / sizeof(T)]) {
  u32x4 u;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = uint32_t(Tr<bf16_t>::from_f(v[2 * i])) |
             (uint32_t(Tr<bf16_t>::from_f(v[2 * i + 1])) << 16);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = __float_as_uint(v[i]);
  }
  *reinterpret_cast<u32x4*>(p) = u;
}

// Elementwise pass over [B, R, N, H, C], one 16-byte chunk per thread (whole
// position rows per wave, so every access is contiguous): dO = dOut*sigmoid(G),
// dG = dOut*Out*(1 - sigmoid(G)), and per (line, head, position) the
// base-2 LSE and -D, D = sum_c dOut*Out (a butterfly over the head's lanes).
template <typename T>
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdParams p) {
  constexpr int E = 16 / sizeof(T);  // elements per chunk
  constexpr int CPH = C / E;         // chunks per head
  const int cpp = p.H * CPH;         // chunks per position
  const int64_t total = (int64_t)p.B * p.R * p.N * cpp;
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = gi < total;
  const int64_t pos = gi / cpp;      // (b*R + r)*N + n
  const int ci = (int)(gi - pos * cpp);
  const int64_t e0 = gi * E;         // chunks are contiguous in [.., H, C]
  float dsum = 0.f;
  if (live) {
    float o[E], d[E];
    ld_chunk<T>(static_cast<const T*>(p.out) + e0, o);
    ld_chunk<T>(static_cast<const T*>(p.dout) + e0, d);
#pragma unroll
    for (int i = 0; i < E; ++i) dsum += d[i] * o[i];
    if (p.gate) {
      float gv[E], dov[E], dg[E];
      ld_chunk<T>(static_cast<const T*>(p.gate) + e0, gv);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const float sg = sigmoid_f(gv[i]);
        dov[i] = d[i] * sg;
        dg[i] = d[i] * o[i] * (1.f - sg);
      }
      st_chunk<T>(static_cast<T*>(p.dgate) + e0, dg);
      st_chunk<T>(static_cast<T*>(p.dopre) + e0, dov);
    }
  }
#pragma unroll
  for (int m = 1; m < CPH; m <<= 1) dsum += __shfl_xor(dsum, m, 64);
  if (live && ci % CPH == 0) {
    const int h = ci / CPH;
    const int64_t line = pos / p.N;
    const int n = (int)(pos - line * p.N);
    const int64_t lh = line * p.H + h;  // line-head index
    const float lse = p.lse[lh * p.N + n];
    // fully masked query: P = exp2(-inf) = 0 everywhere
    p.lse2[lh * p.Np + n] = lse == -INFINITY ? INFINITY : lse * kLog2e;
    p.dd[lh * p.Np + n] = -dsum;  // -D: the dP accumulator's start
  }
  // padding queries n in [N, Np): P = 0, D = 0
  const int npad = p.Np - p.N;
  const int64_t pad_total = (int64_t)p.B * p.R * p.H * npad;
  for (int64_t e = gi; e < pad_total; e += (int64_t)gridDim.x * 256) {
    const int64_t lh = e / npad;
    const int n = p.N + (int)(e - lh * npad);
    p.lse2[lh * p.Np + n] = INFINITY;
    p.dd[lh * p.Np + n] = 0.f;
  }
}

// Pair bias (natural units) with the shared key mask and the padding folded
// in: -inf for masked keys and keys >= N, 0 without a bias, any finite value
// for queries >= N.  bf16 inputs store it in fp16, exactly as the forward
// prepares its own: every bf16 value of magnitude 2^-14 .. 65504 is exact,
// smaller ones are within 2^-25, finite values beyond +-65504 are clamped
// to it (so the backward recomputes the logits the forward normalised).  Two
// copies, each in the order one kernel reads it, so that every bias load is
// a contiguous block per wave:
//   bp  (dQ and dBias kernels; the forward's order): per (b, h) a grid of
//       [Nq128/128][Np/64] tiles, each [wave 4][qb 2][half 2][lane 64][8]:
//       lane (l16, g) of wave w holds query 128*qt + 32*w + 16*qb + l16,
//       keys 64*kt + 32*half + 8*g .. +7.
//   bpt (dK/dV kernel): per (b, h) a grid of [Nk128/128][Np/32] blocks (key
//       tile, 32-query step), each [wave 4][qb 2][lane 64][kb 2][i 4]: lane
//       (l16, g) of wave w holds key 128*kt + 32*w + 16*kb + l16 and
//       queries 32*st + 16*qb + 4*g + i (a wave reads each qb half as one
//       contiguous 1 KB load).
template <typename T>
__device__ __forceinline__ float bias_value(const BwdParams& p, int bh, int q, int k) {
  if (k >= p.N) return -INFINITY;
  const int b = bh / p.H;
  if (p.mask && !p.row_mask && p.mask[(int64_t)b * p.mask_rows * p.N + k] == 0) return -INFINITY;
  const T* Bias = static_cast<const T*>(p.bias);
  return (Bias && q < p.N) ? Tr<T>::to_f(Bias[((int64_t)bh * p.N + q) * p.N + k]) : 0.f;
}

// Four prepared-bias values: bf16 inputs store fp16 bits in the 16-bit
// slots (finite values clamped to +-65504, as in the forward), fp32 inputs
// fp32.
__device__ __forceinline__ void st4pb(bf16_t* p, const f32x4& v) {
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  f16x4 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = v[i];
    if (x == x && fabsf(x) != INFINITY) x = fminf(fmaxf(x, -65504.f), 65504.f);
    h[i] = (_Float16)x;
  }
  *reinterpret_cast<f16x4*>(p) = h;
}
__device__ __forceinline__ void st4pb(float* p, const f32x4& v) { st4e(p, v); }

// Element j (0..7) of a lane's raw 8-value prepared-bias chunk, in fp32
// (fp16 widens inside the consuming FMA: v_fma_mix_f32).
__device__ __forceinline__ float pb_elem(const Raw8<bf16_t>& r, int j) {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  return (float)__builtin_bit_cast(f16x8, r.a)[j];
}
__device__ __forceinline__ float pb_elem(const Raw8<float>& r, int j) {
  return __uint_as_float(j < 4 ? r.a[j] : r.b[j - 4]);
}

template <typename T>
__global__ void __launch_bounds__(256) bwd_bias_kernel(BwdParams p) {
  const int Np = p.Np, nq128 = (p.N + 127) / 128, nk64 = Np / 64, nst = Np / 32;
  const int64_t chunks = (int64_t)p.B * p.H * nq128 * 128 * Np / 8;  // per copy
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < 2 * chunks;
       e += (int64_t)gridDim.x * 256) {
    f32x4 v[2];
    if (e < chunks) {  // bp chunk e: 8 keys of one query
      const int lane = (int)(e & 63);
      int64_t t = e >> 6;
      const int half = (int)(t & 1); t >>= 1;
      const int qb = (int)(t & 1); t >>= 1;
      const int wv = (int)(t & 3); t >>= 2;
      const int kt = (int)(t % nk64); t /= nk64;
      const int qt = (int)(t % nq128);
      const int bh = (int)(t / nq128);
      const int q = qt * 128 + wv * 32 + qb * 16 + (lane & 15);
      const int k0 = kt * 64 + half * 32 + 8 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j >> 2][j & 3] = bias_value<T>(p, bh, q, k0 + j);
      T* dst = static_cast<T*>(p.bp) + e * 8;
      st4pb(dst, v[0]);
      st4pb(dst + 4, v[1]);
    } else {  // bpt chunk: the qb half of a lane's 16 values, 4 queries x 2 keys
      const int64_t f = e - chunks;
      const int lane = (int)(f & 63);
      const int qb = (int)((f >> 6) & 1);
      int64_t t = f >> 7;
      const int wv = (int)(t & 3); t >>= 2;
      const int st = (int)(t % nst); t /= nst;
      const int kt = (int)(t % nq128);
      const int bh = (int)(t / nq128);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int k = kt * 128 + wv * 32 + kb * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[kb][i] = bias_value<T>(p, bh, st * 32 + qb * 16 + 4 * (lane >> 4) + i, k);
      }
      T* dst = static_cast<T*>(p.bpt) + f * 8;
      st4pb(dst, v[0]);
      st4pb(dst + 4, v[1]);
    }
  }
}

// ----------------------------------------------------------------- dK, dV
// Staged per 32-query step: Q rows and dO rows (row-major; fp32 also the
// slot-ordered Q^T and dO^T slabs), each [32][32] (+pad); base-2 LSE and -D.
template <typename T> struct StageRaw;  // one 16-byte chunk (fp32: two)
template <> struct StageRaw<bf16_t> { u32x4 a; float l; };
template <> struct StageRaw<float> { u32x4 a, b; float l; };

template <typename T, bool ROW_MASK>
// Four waves per SIMD: the register cap costs a 12-byte spill of values
// used only after the query loop.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
bwd_dkdv_kernel(BwdParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int RS = 40;  // row stride (elements): 16-byte reads spread over banks
  constexpr int E16 = 16 / sizeof(T);
  // [buf][Q, dO, Q^T, dO^T]; bf16 reads the transposed operands straight
  // from the row-major tiles (lds_read_tr16), so only fp32 stores Q^T, dO^T
  __shared__ __attribute__((aligned(32))) T sT[2][sizeof(T) == 2 ? 2 : 4][32 * RS];
  __shared__ float sL[2][2][32];                                 // [buf][-lse2, -D]

  // Work order (fastest first): key tile, head within a head pair, line,
  // head pair.  The key tiles of one line read the same query-side data and
  // the two heads of a pair share every 128-byte line of it (heads are
  // interleaved at 64 bytes), so all of them run back to back on one XCD
  // and meet in its L2; a pair's bias^T (2 x N^2 elements) stays there too.
  const int nkt = (p.N + 127) / 128;
  const int HP = (p.H + 1) >> 1;
  int w = xcd_work_index(p.B * p.R * HP * 2 * nkt);
  if (w < 0) return;
  const int kt = w % nkt; w /= nkt;
  const int hi = w & 1; w >>= 1;
  const int line = w % (p.B * p.R);   // b * R + r
  const int h = 2 * (w / (p.B * p.R)) + hi;
  if (h >= p.H) return;  // odd H: the missing partner of the last pair
  const int b = line / p.R, r = line - b * p.R;
  const int N = p.N, H = p.H, Np = p.Np;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t lh = (int64_t)line * H + h;
  const int pos_stride = H * C;
  const int64_t lbase = (int64_t)line * N * pos_stride + h * C;

  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);
  const T* Q = static_cast<const T*>(p.q);
  const T* DO = static_cast<const T*>(p.dopre);
  // This lane's bias^T operands of step st: 8 values [kb][i] per qb at
  // BPT + st * 4096 + qb * 512 (prepared block order).
  const T* BPT = static_cast<const T*>(p.bpt) +
                 ((int64_t)(b * H + h) * nkt + kt) * (Np / 32) * 4096 + wave * 1024 + lane * 8;
  const uint8_t* mrow = ROW_MASK ? p.mask + ((int64_t)b * p.mask_rows + r) * N : nullptr;

  // This wave's keys: kbase + kb*16 + l16 (kb = 0, 1).  K is held scaled by
  // log2(e)/sqrt(C), so the logit product is already in base 2.
  const int kbase = kt * 128 + wave * 32;
  const float ksc = p.lscale;
  Op kf[2], vf[2];
  bool kdead[2];  // keys of a per-line mask (padding and shared masks are in the bias)
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kbase + kb * 16 + l16;
    if (key < N) {
      kf[kb] = scale8(ldop<T>(K + lbase + (int64_t)key * pos_stride + 8 * g), ksc);
      vf[kb] = ldop<T>(V + lbase + (int64_t)key * pos_stride + 8 * g);
    } else {
      kf[kb] = Op{};
      vf[kb] = Op{};
    }
    kdead[kb] = ROW_MASK && key < N && mrow[key] == 0;
  }
  f32x4 dk[2][2], dv[2][2];  // [cb][kb]
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      dk[cb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv[cb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // Staging: thread -> (tensor: Q or dO, query row, 8-dim chunk).  Each
  // 32-query step is stored in LDS row-major (the S and dP operands); bf16
  // reads the transposed dV and dK operands from there, fp32 also stores
  // them transposed with the queries in slot order.
  // Loads: bf16 uses buffer loads, with the wave's row base (waves 0-1 load
  // Q, 2-3 dO) and the step offset in scalar registers and the lane's offset
  // fixed, so no address register is rewritten while a prefetch is in
  // flight; query rows past N read zeros (their P and dS are 0).  fp32
  // clamps to query N-1.
  const int srow = (tid >> 2) & 31, sch = tid & 3, sten = wave >> 1;
  const T* sbase = (sten == 0 ? Q : DO) + lbase;
  const T* ssrc = sbase + sch * 8;
  const uint32_t s_nbytes = (uint32_t)((N - 1) * pos_stride + C) * (uint32_t)sizeof(T);
  const uint32_t s_voff = (uint32_t)(srow * pos_stride + sch * 8) * (uint32_t)sizeof(T);
  // LSE (lanes 0-31 of each wave) and -D (lanes 32-63).  Every wave loads
  // and stores them, so that no branch makes the waits for the other loads
  // conservative.
  const float* lsrc = ((lane & 32) ? p.dd : p.lse2) + lh * Np;
  const int sslot = query_slot(srow);
  auto fetch = [&](StageRaw<T>& raw, int q0) {
    if constexpr (sizeof(T) == 2) {
      raw.a = buf_ld128(sbase, s_nbytes, s_voff, (uint32_t)(q0 * pos_stride) * 2u);
    } else {
      const T* src = ssrc + (int64_t)min(q0 + srow, N - 1) * pos_stride;
      raw.a = reinterpret_cast<const u32x4*>(src)[0];
      raw.b = reinterpret_cast<const u32x4*>(src)[1];
    }
    raw.l = lsrc[min(q0 + (lane & 31), Np - 1)];
  };
  auto store = [&](const StageRaw<T>& raw, int buf) {
    T* drow = sT[buf][sten] + srow * RS + sch * 8;
    if constexpr (sizeof(T) == 2) {
      (void)sslot;
      *reinterpret_cast<u32x4*>(drow) = raw.a;
    } else {
      T* dcol = sT[buf][2 + sten] + (sch * 8) * RS + sslot;
      reinterpret_cast<u32x4*>(drow)[0] = raw.a;
      reinterpret_cast<u32x4*>(drow)[1] = raw.b;
      uint32_t* d32 = reinterpret_cast<uint32_t*>(dcol);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d32[j * RS] = raw.a[j];
        d32[(4 + j) * RS] = raw.b[j];
      }
    }
    // every wave writes the same values (no branch, see the LSE load);
    // -LSE starts the logit product, -D the dP product
    sL[buf][lane >> 5][lane & 31] = (lane & 32) ? raw.l : -raw.l;
  };
  (void)E16;
  // A step's bias^T operands (bf16: buffer loads; past this workgroup's
  // blocks they read zeros; fp32: the step index is clamped).
  const int nsteps = (N + 31) / 32;
  const T* bpt_w = static_cast<const T*>(p.bpt) +
                   ((int64_t)(b * H + h) * nkt + kt) * (Np / 32) * 4096 + wave * 1024;  // the wave's base
  const uint32_t b_nbytes = (uint32_t)((Np / 32) * 4096 - wave * 1024) * (uint32_t)sizeof(T);
  auto fetch_bias = [&](Raw8<T> (&bn)[2], int st) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t so = (uint32_t)st * 4096u * 2u;
      bn[0].a = buf_ld128(bpt_w, b_nbytes, (uint32_t)lane * 16u, so);
      bn[1].a = buf_ld128(bpt_w, b_nbytes, (uint32_t)lane * 16u + 1024u, so);
    } else {
      const T* src = BPT + (int64_t)min(st, nsteps - 1) * 4096;
      ld_raw8(bn[0], src);
      ld_raw8(bn[1], src + 512);
    }
  };

  // One 32-query step: stage `cur` (fetched a step earlier), then fetch the
  // next step into `nxt` while this one computes.  Two register sets used in
  // turn, so that no prefetch is copied; the fetches are unconditional, so
  // that every wait for them is exact.
  auto step = [&](int st, const StageRaw<T>& cur, StageRaw<T>& nxt, const Raw8<T> (&bc)[2],
                  Raw8<T> (&bx)[2]) {
    const int q0 = st * 32, buf = st & 1;
    // keep the scheduler from hoisting this store (and its wait for the
    // prefetch) into the previous step
    __builtin_amdgcn_sched_barrier(0);
    store(cur, buf);
    __syncthreads();
    fetch(nxt, q0 + 32);
    fetch_bias(bx, st + 1);
    __builtin_amdgcn_sched_barrier(0);  // issue the prefetch here, not later
    const T* sQ = sT[buf][0];
    const T* sDO = sT[buf][1];

    // S[qb][kb]: lane holds queries qb*16 + 4g + i for key kbase + kb*16 + l16,
    // base 2, starting from -LSE (the bias is added below).  dP starts from
    // -D, so the accumulator ends at dP - D.
    f32x4 s[2][2], dp[2][2];
    // products at raised wave priority (as in the forward): 677 -> 656 us
    // here and 680 -> 656 us in dBias at N = 768; dQ measured slower (its
    // registers spill), so it keeps the default
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const Op qa = *reinterpret_cast<const Op*>(sQ + (qb * 16 + l16) * RS + 8 * g);
      const Op da = *reinterpret_cast<const Op*>(sDO + (qb * 16 + l16) * RS + 8 * g);
      const f32x4 negl = *reinterpret_cast<const f32x4*>(&sL[buf][0][qb * 16 + 4 * g]);
      const f32x4 negd = *reinterpret_cast<const f32x4*>(&sL[buf][1][qb * 16 + 4 * g]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[qb][kb] = mma32(qa, kf[kb], negl);
        dp[qb][kb] = mma32(da, vf[kb], negd);
      }
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float pv = exp2_fast(__builtin_fmaf(pb_elem(bc[qb], kb * 4 + i), kLog2e, s[qb][kb][i]));
          if constexpr (ROW_MASK) pv = kdead[kb] ? 0.f : pv;
          s[qb][kb][i] = pv;
          dp[qb][kb][i] = pv * dp[qb][kb][i];
        }
    }
    // dV^T += dO^T P,  dK^T += Q^T dS  (contraction over the 32 query slots)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      Op dot, qtf;  // dO^T, Q^T: dims cb*16 + l16, query slots 8g .. +7
      if constexpr (sizeof(T) == 2) {
        // slots 8g + i and 8g + 4 + i hold queries 4g + i and 16 + 4g + i
        const int c0 = cb * 16 + 4 * (l16 & 3);
        const int r0 = (4 * g + (l16 >> 2)) * RS + c0, r1 = r0 + 16 * RS;
        dot = lds_read_tr_op(sDO + r0, sDO + r1);
        qtf = lds_read_tr_op(sQ + r0, sQ + r1);
      } else {
        dot = *reinterpret_cast<const Op*>(sT[buf][3] + (cb * 16 + l16) * RS + 8 * g);
        qtf = *reinterpret_cast<const Op*>(sT[buf][2] + (cb * 16 + l16) * RS + 8 * g);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const Op pf = pack8(s[0][kb], s[1][kb], (Op*)nullptr);
        const Op sf = pack8(dp[0][kb], dp[1][kb], (Op*)nullptr);
        dv[cb][kb] = mma32(dot, pf, dv[cb][kb]);
        dk[cb][kb] = mma32(qtf, sf, dk[cb][kb]);
      }
      __builtin_amdgcn_s_setprio(0);

    }
  };
  StageRaw<T> ra, rb;
  Raw8<T> ba[2], bb[2];
  fetch(ra, 0);
  fetch_bias(ba, 0);
  // An even number of steps, so that no tail copy of the step follows the
  // loop (its address registers would otherwise stay live across the loop
  // and spill).  An odd count gains one step of padded queries: the padding
  // is Np = pad64(N) >= 32 * (nsteps + 1), whose base-2 LSE is +inf, so its
  // P and dS are exactly 0.
  const int nsteps2 = (nsteps + 1) & ~1;
  for (int st = 0; st < nsteps2; st += 2) {
    step(st, ra, rb, ba, bb);
    step(st + 1, rb, ra, bb, ba);
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
      st4e(DK + off, dk[cb][kb] * ks);
      st4e(DV + off, dv[cb][kb]);
    }
  }
}

// ------------------------------------------------------------- dQ, dBias
// Key of A-operand lane m in block (half, kb) of a 64-key tile: the
// accumulator layout then gives lane group g the 8 consecutive keys
// half*32 + 8g .. +7 (the same permutation as the forward kernel).
__device__ __forceinline__ int k_lds_row(int p) {
  const int half = p >> 5, pp = p & 31;
  const int gg = pp >> 3, kb = (pp >> 2) & 1, i = pp & 3;
  return half * 32 + kb * 16 + gg * 4 + i;
}

// One thread's share of a 64-key tile, held in plain locals (16-byte
// chunks; fp32 needs two per tensor): key t/4, dims 8*(t%4)..+7 of K and V.
// Keys past N read key N-1 (finite; their dS is 0).
#define EVO_FETCH_K(T, K_, V_, k0_)                                               \
  do {                                                                        \
    const int t_ = threadIdx.x;                                               \
    const int kk_ = min((k0_) + (t_ >> 2), N - 1), ch_ = t_ & 3;              \
    const u32x4* ks_ = reinterpret_cast<const u32x4*>((K_) + (int64_t)kk_ * pos_stride + ch_ * 8); \
    const u32x4* vs_ = reinterpret_cast<const u32x4*>((V_) + (int64_t)kk_ * pos_stride + ch_ * 8); \
    rk0 = ks_[0]; rv0 = vs_[0];                                               \
    if constexpr (sizeof(T) == 4) { rk1 = ks_[1]; rv1 = vs_[1]; }             \
  } while (0)

// K and V rows key-permuted (the S and dP operands); fp32 also stores K
// transposed, keys in physical order (the dQ operand; bf16 reads it with a
// transposing LDS read instead).
#define EVO_STORE_K(T, sK_, sV_, sKt_, KS_, TS_)                                  \
  do {                                                                        \
    const int t_ = threadIdx.x, kk_ = t_ >> 2, ch_ = t_ & 3;                  \
    u32x4* dk_ = reinterpret_cast<u32x4*>((sK_) + k_lds_row(kk_) * (KS_) + ch_ * 8); \
    u32x4* dv_ = reinterpret_cast<u32x4*>((sV_) + k_lds_row(kk_) * (KS_) + ch_ * 8); \
    dk_[0] = rk0; dv_[0] = rv0;                                               \
    if constexpr (sizeof(T) == 4) {                                           \
      dk_[1] = rk1; dv_[1] = rv1;                                             \
      uint32_t* dt_ = reinterpret_cast<uint32_t*>(sKt_) + (ch_ * 8) * (TS_) + kk_; \
      for (int j_ = 0; j_ < 4; ++j_) {                                        \
        dt_[j_ * (TS_)] = rk0[j_];                                            \
        dt_[(4 + j_) * (TS_)] = rk1[j_];                                      \
      }                                                                       \
    }                                                                         \
  } while (0)

template <typename T> struct BLds;
template <> struct BLds<bf16_t> { static constexpr int KS = 40, TS = 72; };
template <> struct BLds<float> { static constexpr int KS = 36, TS = 68; };

// dQ: workgroup = one line, one head, 128 queries (32 per wave); loops over
// 64-key tiles (K, V rows key-permuted) through double-buffered LDS.  Lane = query: S^T = K Q^T + bias, P = exp2(S - LSE), dP^T = V dO^T,
// dS = P (dP - D), dQ^T += K^T dS^T.
template <typename T, bool ROW_MASK>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && !ROW_MASK ? 4 : 1)))
bwd_dq_kernel(BwdParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int KS = BLds<T>::KS, TS = BLds<T>::TS;
  // bf16 reads K^T straight from the key-permuted K tile (lds_read_tr16);
  // only fp32 stores a transposed copy
  __shared__ __attribute__((aligned(32))) T sK[2][64 * KS], sV[2][64 * KS],
      sKt[2][sizeof(T) == 2 ? 1 : 32 * TS];

  // Work order: query tile, head within a pair, line, head pair (as in the
  // dK/dV kernel): the pair's bias rows and shared K/V lines stay in L2.
  const int nqt = (p.N + 127) / 128;
  const int HP = (p.H + 1) >> 1;
  int w = xcd_work_index(p.B * p.R * HP * 2 * nqt);
  if (w < 0) return;
  const int qt = w % nqt; w /= nqt;
  const int hi = w & 1; w >>= 1;
  const int line = w % (p.B * p.R);
  const int h = 2 * (w / (p.B * p.R)) + hi;
  if (h >= p.H) return;
  const int b = line / p.R, r = line - b * p.R;
  const int N = p.N, H = p.H, Np = p.Np;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar
  const int l16 = lane & 15, g = lane >> 4;
  const int pos_stride = H * C;
  const int64_t lbase = (int64_t)line * N * pos_stride + h * C;
  const int64_t lh = (int64_t)line * H + h;
  const int qw0 = qt * 128 + wave * 32;
  const T* K = static_cast<const T*>(p.k) + lbase;
  const T* V = static_cast<const T*>(p.v) + lbase;
  const uint8_t* mrow = ROW_MASK ? p.mask + ((int64_t)b * p.mask_rows + r) * N : nullptr;

  // Q is held scaled by log2(e)/sqrt(C) and the logit product starts from
  // -LSE (base 2), so the exponent is the product plus bias*log2(e).
  Op qf[2], df[2];
  float l2[2], dd[2];  // dd = -D
  const float qsc = p.lscale;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q = qw0 + qb * 16 + l16;
    const int qc = min(q, N - 1);
    qf[qb] = scale8(ldop<T>(static_cast<const T*>(p.q) + lbase + (int64_t)qc * pos_stride + 8 * g),
                    qsc);
    df[qb] = ldop<T>(static_cast<const T*>(p.dopre) + lbase + (int64_t)qc * pos_stride + 8 * g);
    l2[qb] = q < N ? p.lse2[lh * Np + q] : INFINITY;
    dd[qb] = q < N ? p.dd[lh * Np + q] : 0.f;
  }
  // This lane's 8 bias values of (qb, half) in key tile `tile` sit at
  // BP + tile * 8192 + (qb*2 + half) * 512 (prepared tile order).
  const T* BP = static_cast<const T*>(p.bp) +
                (((int64_t)(b * H + h) * nqt + qt) * (Np / 64)) * 8192 + wave * 2048 + lane * 8;
  f32x4 dq[2][2];  // [qb][cb]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) dq[qb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 rk0, rk1, rv0, rv1;
  rk1 = rv1 = u32x4{0, 0, 0, 0};
  // bf16 tile loads are buffer loads: the workgroup's (wave's) base and the
  // tile offset in scalar registers, the lane's offset fixed for the loop,
  // so no address registers are rewritten while a prefetch is in flight;
  // keys past N and tiles past this workgroup's row read zeros.  fp32 uses
  // clamped addresses.
  const uint32_t kv_nbytes = (uint32_t)((N - 1) * pos_stride + C) * 2u;
  const uint32_t kv_voff = (uint32_t)((tid >> 2) * pos_stride + (tid & 3) * 8) * 2u;
  const T* BPw = static_cast<const T*>(p.bp) +
                 (((int64_t)(b * H + h) * nqt + qt) * (Np / 64)) * 8192 + wave * 2048;
  const uint32_t b_nbytes = (uint32_t)((Np / 64) * 8192 - wave * 2048) * 2u;
  // A tile's K and V into rk/rv, its bias operands [qb][half] (raw) into bn.
  auto fetch_tile = [&](int tile, Raw8<T> (&bn)[2][2]) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t so = (uint32_t)(tile * 64 * pos_stride) * 2u;
      rk0 = buf_ld128(K, kv_nbytes, kv_voff, so);
      rv0 = buf_ld128(V, kv_nbytes, kv_voff, so);
      const uint32_t bo = (uint32_t)tile * 8192u * 2u;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int half = 0; half < 2; ++half)
          bn[qb][half].a = buf_ld128(BPw, b_nbytes, (uint32_t)lane * 16u + (qb * 2 + half) * 1024u, bo);
    } else {
      const int nt = min(tile, (N + 63) / 64 - 1);
      EVO_FETCH_K(T, K, V, nt * 64);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int half = 0; half < 2; ++half)
          ld_raw8(bn[qb][half], BP + (int64_t)nt * 8192 + (qb * 2 + half) * 512);
    }
  };
  const f32x4 negl[2] = {f32x4{-l2[0], -l2[0], -l2[0], -l2[0]},
                         f32x4{-l2[1], -l2[1], -l2[1], -l2[1]}};
  Raw8<T> bn[2][2];  // the next tile's bias operands [qb][half], raw
  fetch_tile(0, bn);
  const int ntiles = (N + 63) / 64;
  for (int tile = 0; tile < ntiles; ++tile) {
    const int k0 = tile * 64, buf = tile & 1;
    EVO_STORE_K(T, sK[buf], sV[buf], sKt[buf], KS, TS);
    __syncthreads();
    Raw8<T> bc[2][2];  // this tile's
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int half = 0; half < 2; ++half) bc[qb][half] = bn[qb][half];
    // next tile (after the last: zeros for bf16, the last tile again for
    // fp32; unused)
    fetch_tile(tile + 1, bn);
    // issue that prefetch here: left to itself, the scheduler sinks it to
    // the end of the tile, next to the store that waits for it
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x4 s[2][2], dp[2][2];  // [qb][kb]; dP starts from -D
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const Op vf = *reinterpret_cast<const Op*>(sV[buf] + (half * 32 + kb * 16 + l16) * KS + 8 * g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          dp[qb][kb] = mma32(vf, df[qb], f32x4{dd[qb], dd[qb], dd[qb], dd[qb]});
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const Op kf = *reinterpret_cast<const Op*>(sK[buf] + (half * 32 + kb * 16 + l16) * KS + 8 * g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s[qb][kb] = mma32(kf, qf[qb], negl[qb]);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bool dead[4] = {false, false, false, false};
        if constexpr (ROW_MASK) {
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
            const float pv =
                dead[i] ? 0.f
                        : exp2_fast(__builtin_fmaf(pb_elem(bc[qb][half], kb * 4 + i), kLog2e,
                                                   s[qb][kb][i]));
            dp[qb][kb][i] = pv * dp[qb][kb][i];
          }
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        Op ktf;  // K^T: dims cb*16 + l16, keys half*32 + 8g .. +7
        if constexpr (sizeof(T) == 2) {
          // physical key half*32 + 8g + 4h + i sits in row half*32 + 16h + 4g + i
          const T* k0p = sK[buf] + (half * 32 + 4 * g + (l16 >> 2)) * KS + cb * 16 + 4 * (l16 & 3);
          ktf = lds_read_tr_op(k0p, k0p + 16 * KS);
        } else {
          ktf = *reinterpret_cast<const Op*>(sKt[buf] + (cb * 16 + l16) * TS + half * 32 + 8 * g);
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          dq[qb][cb] = mma32(ktf, pack8(dp[qb][0], dp[qb][1], (Op*)nullptr), dq[qb][cb]);
      }
    }
  }
  const float ks = 1.f / sqrtf((float)C);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q = qw0 + qb * 16 + l16;
    if (q >= N) continue;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      st4e(static_cast<T*>(p.dq) + lbase + (int64_t)q * pos_stride + cb * 16 + 4 * g,
           dq[qb][cb] * ks);
  }
}

#undef EVO_FETCH_K
#undef EVO_STORE_K

// dBias: workgroup = one head, 128 queries (32 per wave) x 64 keys, for a
// group of rows; the bias tile (MFMA accumulator operand) and the dBias
// accumulator stay in registers while the rows stream by, their K and V
// tiles shared by the 4 waves through double-buffered LDS.
template <typename T, bool ROW_MASK>
// bf16 without a per-line mask: three waves per SIMD (168 registers)
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && !ROW_MASK ? 3 : 1)))
bwd_dbias_kernel(BwdParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int KS = BLds<T>::KS;
  __shared__ __attribute__((aligned(32))) T sK[2][64 * KS], sV[2][64 * KS];

  // Work order: head within a pair, key tile, query tile, row group, head
  // pair, batch.  The two heads of a pair walk the same rows in lockstep and
  // share every 128-byte line of Q, dO, K and V.
  const int nqt = (p.N + 127) / 128, nkt = p.Np / 64;
  const int HP = (p.H + 1) >> 1;
  int w = xcd_work_index(p.B * HP * 2 * nqt * nkt * p.n_rg);
  if (w < 0) return;
  const int hi = w & 1; w >>= 1;
  const int kt = w % nkt; w /= nkt;
  const int qt = w % nqt; w /= nqt;
  const int rg = w % p.n_rg; w /= p.n_rg;
  const int h = 2 * (w % HP) + hi;
  const int b = w / HP;
  if (h >= p.H) return;
  const int N = p.N, H = p.H, R = p.R, Np = p.Np;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int pos_stride = H * C;
  const int bh = b * H + h;
  const int k0 = kt * 64;
  const int qw0 = qt * 128 + wave * 32;

  f32x4 cbias[2][2][2], db[2][2][2];  // [half][qb][kb]
  {
    // prepared tile order: this lane's 8 values of (qb, half) are contiguous
    const T* bt = static_cast<const T*>(p.bp) + (((int64_t)bh * nqt + qt) * nkt + kt) * 8192 +
                  wave * 2048 + lane * 8;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        Raw8<T> r;
        ld_raw8(r, bt + (qb * 2 + half) * 512);
        // the logit accumulators hold <Q,K> + bias*sqrt(C) (unscaled Q);
        // 1/sqrt(C) is applied in the exponent
#pragma unroll
        for (int j = 0; j < 8; ++j) cbias[half][qb][j >> 2][j & 3] = pb_elem(r, j) * kSqrtC;
        db[half][qb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        db[half][qb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
  }
  const float sc = p.qscale * kLog2e;
  const int r_begin = rg * p.rows_per_group;
  const int r_end = min(R, r_begin + p.rows_per_group);
  // thread t stages key t/4 (dims 8*(t%4)..+7) of K and V for one row;
  // the next row's tiles and query-side operands are prefetched into plain
  // locals (the last iteration re-fetches its own row, unused).
  const int kk = min(k0 + (tid >> 2), N - 1), ch = tid & 3;
  uint4 rk0, rk1, rv0, rv1;
  rk1 = rv1 = make_uint4(0, 0, 0, 0);
  Op qn0, qn1, dn0, dn1;
  float l2n0, l2n1, ddn0, ddn1;
  // Per-lane addresses in row r_begin; row r is `r - r_begin` line strides on.
  const int64_t lstride = (int64_t)N * pos_stride;       // one line of [.., N, H, C]
  const int64_t l0 = ((int64_t)b * R + r_begin) * lstride + h * C;
  const int qa = qw0 + l16, qbq = qw0 + 16 + l16;
  // LSE / -D reads clamped into the padded rows (queries >= N are never stored)
  const int qac = min(qa, Np - 1), qbc = min(qbq, Np - 1);
  const T* kp = static_cast<const T*>(p.k) + l0 + (int64_t)kk * pos_stride + ch * 8;
  const T* vp = static_cast<const T*>(p.v) + l0 + (int64_t)kk * pos_stride + ch * 8;
  // Q and dO rows.  bf16 loads them with four consecutive lanes covering one
  // position's 64 contiguous bytes (lane l: query qw0 + l/4 (+16), dims
  // 8*(l%4)..+7), which the vector memory path serves about four times
  // faster than the MFMA operand order (lane l: query l%16, dims 8*(l/16));
  // each wave then moves its rows into operand order through its own LDS
  // slots.  fp32 loads the operands directly.
  constexpr bool QD_LDS = sizeof(T) == 2;
  const int qr0 = QD_LDS ? qw0 + (lane >> 2) : qa, qr1 = QD_LDS ? qw0 + 16 + (lane >> 2) : qbq;
  const int qch = QD_LDS ? (lane & 3) * 8 : 8 * g;
  const T* qp0 = static_cast<const T*>(p.q) + l0 + (int64_t)min(qr0, N - 1) * pos_stride + qch;
  const T* qp1 = static_cast<const T*>(p.q) + l0 + (int64_t)min(qr1, N - 1) * pos_stride + qch;
  const T* op0 = static_cast<const T*>(p.dopre) + l0 + (int64_t)min(qr0, N - 1) * pos_stride + qch;
  const T* op1 = static_cast<const T*>(p.dopre) + l0 + (int64_t)min(qr1, N - 1) * pos_stride + qch;
  constexpr int QS = 40;  // LDS row stride (elements) of the per-wave Q / dO slots
  __shared__ __attribute__((aligned(16))) T sQD[QD_LDS ? 4 : 1][2][QD_LDS ? 32 * QS : 8];
  const int64_t lh0 = ((int64_t)b * R + r_begin) * H + h;
  const float* lp = p.lse2 + lh0 * Np;
  const float* dq_ = p.dd + lh0 * Np;
  const int64_t hstride = (int64_t)H * Np;                // one line of [.., H, Np]
#define EVO_FETCH_ROW(r_)                                                          \
  do {                                                                         \
    const int64_t ro_ = (int64_t)((r_) - r_begin);                             \
    const int64_t lo_ = ro_ * lstride, ho_ = ro_ * hstride;                     \
    const uint4* ks_ = reinterpret_cast<const uint4*>(kp + lo_);               \
    const uint4* vs_ = reinterpret_cast<const uint4*>(vp + lo_);               \
    rk0 = ks_[0]; rv0 = vs_[0];                                                \
    if constexpr (sizeof(T) == 4) { rk1 = ks_[1]; rv1 = vs_[1]; }              \
    qn0 = ldop<T>(qp0 + lo_);                                                  \
    qn1 = ldop<T>(qp1 + lo_);                                                  \
    dn0 = ldop<T>(op0 + lo_);                                                  \
    dn1 = ldop<T>(op1 + lo_);                                                  \
    l2n0 = lp[ho_ + qac];                                                      \
    l2n1 = lp[ho_ + qbc];                                                      \
    ddn0 = dq_[ho_ + qac];                                                     \
    ddn1 = dq_[ho_ + qbc];                                                     \
  } while (0)
  if (r_begin < r_end) EVO_FETCH_ROW(r_begin);
  for (int r = r_begin; r < r_end; ++r) {
    const int buf = (r - r_begin) & 1;
    {
      const int row = k_lds_row(tid >> 2);
      uint4* dk = reinterpret_cast<uint4*>(sK[buf] + row * KS + ch * 8);
      uint4* dv = reinterpret_cast<uint4*>(sV[buf] + row * KS + ch * 8);
      dk[0] = rk0;
      dv[0] = rv0;
      if constexpr (sizeof(T) == 4) {
        dk[1] = rk1;
        dv[1] = rv1;
      }
    }
    Op qf[2], df[2];
    if constexpr (QD_LDS) {
      // this wave's slots only: no barrier, LDS keeps a wave's accesses in order
      T* sq = sQD[wave][0];
      T* sd = sQD[wave][1];
      const int wr = (lane >> 2) * QS + (lane & 3) * 8;
      *reinterpret_cast<Op*>(sq + wr) = qn0;
      *reinterpret_cast<Op*>(sq + wr + 16 * QS) = qn1;
      *reinterpret_cast<Op*>(sd + wr) = dn0;
      *reinterpret_cast<Op*>(sd + wr + 16 * QS) = dn1;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        qf[qb] = *reinterpret_cast<const Op*>(sq + (qb * 16 + l16) * QS + 8 * g);
        df[qb] = *reinterpret_cast<const Op*>(sd + (qb * 16 + l16) * QS + 8 * g);
      }
    } else {
      qf[0] = qn0; qf[1] = qn1;
      df[0] = dn0; df[1] = dn1;
    }
    const float l2[2] = {l2n0, l2n1};
    const float dd[2] = {ddn0, ddn1};
    __syncthreads();
    EVO_FETCH_ROW(min(r + 1, r_end - 1));
    const uint8_t* mrow = ROW_MASK ? p.mask + ((int64_t)b * p.mask_rows + r) * N : nullptr;
    // one 16-key block at a time (short live ranges: this kernel's budget is
    // three waves per SIMD); dP starts from -D
    const f32x4 negd[2] = {f32x4{dd[0], dd[0], dd[0], dd[0]}, f32x4{dd[1], dd[1], dd[1], dd[1]}};
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const Op kf = *reinterpret_cast<const Op*>(sK[buf] + (half * 32 + kb * 16 + l16) * KS + 8 * g);
        const Op vf = *reinterpret_cast<const Op*>(sV[buf] + (half * 32 + kb * 16 + l16) * KS + 8 * g);
        f32x4 s[2], dp[2];
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          s[qb] = mma32(kf, qf[qb], cbias[half][qb][kb]);
          dp[qb] = mma32(vf, df[qb], negd[qb]);
        }
        __builtin_amdgcn_s_setprio(0);

        bool dead[4] = {false, false, false, false};
        if constexpr (ROW_MASK) {
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
            const float pv =
                dead[i] ? 0.f : exp2_fast(__builtin_fmaf(s[qb][i], sc, -l2[qb]));
            db[half][qb][kb][i] += pv * dp[qb][i];
          }
      }
  }

#undef EVO_FETCH_ROW
  if (!p.dbias) return;
  float* dst = (p.n_rg == 1) ? nullptr : p.dbpart + ((int64_t)rg * p.B * H + bh) * Np * Np;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q = qw0 + qb * 16 + l16;
    if (q >= N) continue;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kk2 = k0 + half * 32 + 8 * g + 4 * kb;
        if (dst) {
          *reinterpret_cast<f32x4*>(dst + (int64_t)q * Np + kk2) = db[half][qb][kb];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kk2 + i < N) p.dbias[((int64_t)bh * N + q) * N + kk2 + i] = db[half][qb][kb][i];
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
  {
    const int64_t chunks = lines * p.N * p.H * (C * (int64_t)sizeof(T) / 16);
    hipLaunchKernelGGL(bwd_prep_kernel<T>, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                       s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    const int64_t work = 2 * (int64_t)p.B * p.H * ((p.N + 127) / 128) * 128 * p.Np / 8;
    hipLaunchKernelGGL(bwd_bias_kernel<T>, dim3((unsigned)std::min<int64_t>((work + 255) / 256, 8192)),
                       dim3(256), 0, s, p);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int HP2 = (p.H + 1) / 2 * 2;  // heads rounded up to whole pairs
  {
    const int total = (int)(lines * HP2 * ((p.N + 127) / 128));
    const int grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (p.row_mask)
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, true>), dim3(grid), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, false>), dim3(grid), dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    const int total = (int)(lines * HP2 * ((p.N + 127) / 128));
    const int grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (p.row_mask)
      hipLaunchKernelGGL((bwd_dq_kernel<T, true>), dim3(grid), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<T, false>), dim3(grid), dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (p.dbias) {
    const int total = p.B * HP2 * ((p.N + 127) / 128) * (p.Np / 64) * p.n_rg;
    const int grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (p.row_mask)
      hipLaunchKernelGGL((bwd_dbias_kernel<T, true>), dim3(grid), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((bwd_dbias_kernel<T, false>), dim3(grid), dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
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
  p.lse2 = reinterpret_cast<float*>(ws + L.off_lse2);
  p.dd = reinterpret_cast<float*>(ws + L.off_d);
  p.bp = ws + L.off_bp;
  p.bpt = ws + L.off_bpt;
  p.dbpart = reinterpret_cast<float*>(ws + L.off_dbpart);
  p.B = (int)a.B; p.R = (int)a.R; p.N = (int)a.N; p.H = (int)a.H;
  p.Np = (int)L.Np;
  p.mask_rows = a.mask ? (int)a.mask_rows : 1;
  p.row_mask = a.mask && a.mask_rows > 1;
  p.n_rg = (int)L.n_rg;
  p.rows_per_group = (int)L.rows_per_group;
  p.qscale = 1.f / sqrtf((float)C);
  p.lscale = kLog2e / sqrtf((float)C);
  return a.dtype == 1 ? launch_t<bf16_t>(p, s) : launch_t<float>(p, s);
}

}  // namespace evo
