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
// Kernels.
//   bias_prep  writes the pair bias once per call (fp16 for bf16 inputs, fp32
//              for fp32), with the shared key mask and the padding keys
//              folded in as -inf, so the main loop needs no bounds or mask
//              logic.  It is stored in the main kernel's fragment order (see
//              the prep kernel): each wave's bias load is one contiguous 1 KB
//              block, 8 consecutive keys of one query per lane.
//   attn_fwd   a workgroup (4 waves) owns 128 queries of one head and one
//              line (ROWS = 1; the kernel is written for ROWS lines sharing
//              the bias tile); each wave owns 32 queries.  Keys stream in
//              tiles of 64 through double-buffered LDS, the next tile's K and
//              V being fetched into registers while the current one is
//              computed (one barrier per tile); each tile is processed as two
//              32-key halves (logits, softmax, PV), the bias one half ahead,
//              which keeps the kernel under 96 registers per lane: five
//              waves per SIMD.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, fp32 accumulate):
//   T^T = K . Q'^T - m       A = 16 keys x 32 dims (LDS), B = Q'^T = (Q
//                            log2(e)/sqrt(C))^T held in registers for the
//                            whole line, C = -m (the softmax reference of each
//                            query, splat); then + bias * log2(e), one
//                            v_fma_mix_f32 per logit straight from the fp16
//                            bias, so T is the base-2 exponent itself.
//   O^T += V^T . P^T         A = V^T from LDS, B = P^T taken straight from
//                            the S^T accumulators (no LDS round trip).
//   l += ones . P^T          (bf16) the row sums of P over each half, on the
//                            matrix core: every lane receives its query's
//                            whole sum, no cross-lane reduction.
// In the accumulator layout a lane holds one query and 4 keys per 16-key
// block; the key order inside a tile is permuted so that each lane's 8 keys
// of a 32-key half are consecutive: the P^T operand is then exactly the
// registers the lane holds, bias loads are 16-byte vectors and the V^T
// operand is one 16-byte LDS read.
//
// Softmax with a lazy reference.  p = exp2(T) uses a per-query reference m
// (base 2, subtracted inside the products) that is only raised when needed:
// the first half-tile (and any half while a query has seen no live key)
// computes the true maximum; a later half is recomputed with a raised
// reference only if a query's sum of p over it exceeds 2^10 (bf16, the
// matrix-core row sum; fp32: a lane's 8 values, 2^8).  So every p <= 2^10
// (no overflow in fp32 or bf16), m never exceeds the true maximum (no
// underflow of the result), and the common half costs one fma and one exp
// per logit plus half a pack and the row-sum product, with no cross-lane
// reduction and no conversion of the bias.  The result is exact up to
// rounding for any m, since O and l are scaled by the same exp2(-m).
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "evo_device.h"
#include "evo_kernels.h"

namespace evo {
namespace {

constexpr int C = kHeadDim;
constexpr int BK = 64;            // keys per tile
constexpr int BQW = 32;           // queries per wave
constexpr int WAVES = 4;
constexpr int BQ = BQW * WAVES;   // queries per workgroup
constexpr float kHeadroom = 256.f;  // 2^8: largest half-tile sum of p per lane (fp32)
constexpr float kHeadroomRow = 1024.f;  // 2^10: largest half-tile row sum

// Prepared-bias element: bf16 inputs are stored as fp16, which holds every
// bf16 value of magnitude 2^-14 .. 65504 exactly (8 significant bits fit in
// 11) and lets v_fma_mix_f32 add bias * log2(e) to an fp32 logit in one
// instruction; fp32 inputs stay fp32.
template <typename T> struct PB;
template <> struct PB<bf16_t> { using E = _Float16; };
template <> struct PB<float> { using E = float; };

template <typename T> struct FwdLds;
// Row strides (elements) of the LDS K tile [64 keys][32 dims] and V tile;
// the padding spreads the reads over all banks.
// bf16: V is stored row-major like K ([64 keys][VST]) and read transposed
// (lds_read_tr16); a row stride of 48 makes those reads conflict-free.
// fp32: V is stored transposed ([32 dims][VST]).
template <> struct FwdLds<bf16_t> { static constexpr int KST = 40, VST = 48, VROWS = BK; };
template <> struct FwdLds<float> { static constexpr int KST = 36, VST = 68, VROWS = C; };

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* gate;
  const uint8_t* mask;   // per-line masks only (shared masks are in biasp)
  const void* biasp;     // [B, H, Nq, Nk] fp16 (bf16 inputs) or fp32, or null (no bias, no mask)
  void* out;
  float* lse;
  int B, R, N, H, mask_rows;
  int Nq, Nk;            // padded bias dims
  int n_qt, n_rg, total;
  float qscale;          // log2(e) / sqrt(C): the products come out in base-2 units
};

// LDS row of physical key p (0..63) of a tile: A-operand lane m of block
// (half, kb) reads LDS row half*32 + kb*16 + m, which must hold physical key
// half*32 + 8*(m/4) + 4*kb + m%4.
__device__ __forceinline__ int k_lds_row(int p) {
  const int half = p >> 5, pp = p & 31;
  const int gg = pp >> 3, kb = (pp >> 2) & 1, i = pp & 3;
  return half * 32 + kb * 16 + gg * 4 + i;
}

// ---- raw tile data one thread fetches for one line: 8 K and 8 V elements
// of one key (fp32: 8 K elements of one key, 4 V elements of two keys).
// (native vector types: HIP's uint4 struct is copied as an aggregate, which
// can leave the tile in scratch memory)
template <typename T> struct KVRaw;
template <> struct KVRaw<bf16_t> { u32x4 k, v; };
template <> struct KVRaw<float> { u32x4 k0, k1, va, vb; };

// Keys at or beyond N have -inf logits on every path (the bias operand
// carries -inf for padding keys), so K and V there only need to be finite:
// bf16 loads zeros, fp32 reads key N-1 again (a clamped address instead of a
// guarded load, which the compiler would route through scratch memory).
template <typename T>
__device__ __forceinline__ void fetch_kv(KVRaw<T>& raw, const T* kline,
                                         const T* vline, int k0, int N,
                                         int pos_stride) {
  const int t = threadIdx.x;
  const int ch = t & 3;
  if constexpr (sizeof(T) == 2) {
    // K and V alike: one 16-byte chunk (8 dims of one key) per thread, so a
    // wave's load touches 16 keys x 64 bytes.  Buffer loads: the tile offset
    // is scalar, the lane's offset fixed, and keys at or past N (past the
    // range) read zeros.
    const uint32_t nbytes = (uint32_t)((N - 1) * pos_stride + C) * 2u;
    const uint32_t voff = (uint32_t)((t >> 2) * pos_stride + ch * 8) * 2u;
    const uint32_t soff = (uint32_t)(k0 * pos_stride) * 2u;
    raw.k = buf_ld128(kline, nbytes, voff, soff);
    raw.v = buf_ld128(vline, nbytes, voff, soff);
  } else {
    const int kk = min(k0 + (t >> 2), N - 1);
    const int p = t & 31, vc = t >> 5;               // V: key pair, 4-dim chunk
    const int ka = min(k0 + 2 * p, N - 1), kb = min(k0 + 2 * p + 1, N - 1);
    const u32x4* s = reinterpret_cast<const u32x4*>(kline + (int64_t)kk * pos_stride + ch * 8);
    raw.k0 = s[0];
    raw.k1 = s[1];
    raw.va = *reinterpret_cast<const u32x4*>(vline + (int64_t)ka * pos_stride + vc * 4);
    raw.vb = *reinterpret_cast<const u32x4*>(vline + (int64_t)kb * pos_stride + vc * 4);
  }
}

// Write one line's raw tile into LDS: K rows key-permuted, V transposed.
template <typename T>
__device__ __forceinline__ void store_kv(const KVRaw<T>& raw, T* sK, T* sV) {
  constexpr int KST = FwdLds<T>::KST, VST = FwdLds<T>::VST;
  const int t = threadIdx.x;
  const int kk = t >> 2, ch = t & 3;
  const int p = t & 31, vc = t >> 5;
  if constexpr (sizeof(T) == 2) {
    (void)p; (void)vc;
    *reinterpret_cast<u32x4*>(sK + k_lds_row(kk) * KST + ch * 8) = raw.k;
    // V row-major (physical key order), read transposed
    *reinterpret_cast<u32x4*>(sV + kk * VST + ch * 8) = raw.v;
  } else {
    u32x4* dk = reinterpret_cast<u32x4*>(sK + k_lds_row(kk) * KST + ch * 8);
    dk[0] = raw.k0;
    dk[1] = raw.k1;
    uint2* dv = reinterpret_cast<uint2*>(sV + (vc * 4) * VST + 2 * p);
    const int rs = VST / 2;  // row stride in uint2
    dv[0 * rs] = make_uint2(raw.va.x, raw.vb.x);
    dv[1 * rs] = make_uint2(raw.va.y, raw.vb.y);
    dv[2 * rs] = make_uint2(raw.va.z, raw.vb.z);
    dv[3 * rs] = make_uint2(raw.va.w, raw.vb.w);
  }
}

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
__device__ __forceinline__ f32x4 ldf4(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  return f32x4{a.x, a.y, a.z, a.w};
}

// Four consecutive elements <-> fp32.
__device__ __forceinline__ f32x4 ld4f(const bf16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
               __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ f32x4 ld4f(const float* p) { return ldf4(p); }
__device__ __forceinline__ void st4f(bf16_t* p, const f32x4& v) {
  uint2 u;
  u.x = uint32_t(Tr<bf16_t>::from_f(v[0])) | (uint32_t(Tr<bf16_t>::from_f(v[1])) << 16);
  u.y = uint32_t(Tr<bf16_t>::from_f(v[2])) | (uint32_t(Tr<bf16_t>::from_f(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}
__device__ __forceinline__ void st4f(float* p, const f32x4& v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// Bias prep.  The prepared bias holds, for every (b, h, query q < Nq, key
// k < Nk), the bias in natural units (0 without a bias), or -inf for keys
// masked by a shared mask or beyond N.  For bf16 inputs it is fp16: exact for
// every bf16 value of magnitude 2^-14 .. 65504, within 2^-25 below that, and
// finite values beyond +-65504 are clamped to it.  It is stored in the order the main
// kernel reads it, so that each wave's bias load is one contiguous 1 KB
// block: per (b, h) a grid of [Nq/128][Nk/64] tiles, each tile
// [wave 4][qb 2][half 2][lane 64][8 keys], where lane (l16, g) of wave w
// holds query 128*qt + 32*w + 16*qb + l16 and keys 64*kt + 32*half + 8*g
// .. +7 (the accumulator-operand layout of the logit tile).
template <typename T>
__global__ void __launch_bounds__(256) fwd_bias_prep_kernel(
    const T* bias, const uint8_t* mask, int shared_mask, typename PB<T>::E* biasp, int B,
    int H, int N, int Nq, int Nk) {
  using E = typename PB<T>::E;
  const int nqt = Nq / BQ, nkt = Nk / BK;
  const int64_t total = (int64_t)B * H * Nq * (Nk / 8);
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int lane = (int)(e & 63);
    int64_t t = e >> 6;
    const int half = (int)(t & 1); t >>= 1;
    const int qb = (int)(t & 1); t >>= 1;
    const int wv = (int)(t & 3); t >>= 2;
    const int kt = (int)(t % nkt); t /= nkt;
    const int qt = (int)(t % nqt);
    const int64_t bh = t / nqt;
    const int b = (int)(bh / H);
    const int q = qt * BQ + wv * BQW + qb * 16 + (lane & 15);
    const int k0 = kt * BK + half * 32 + 8 * (lane >> 4);
    E v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kk = k0 + j;
      float x = -INFINITY;
      if (kk < N) {
        x = (bias && q < N) ? Tr<T>::to_f(bias[(bh * N + q) * N + kk]) : 0.f;
        if (shared_mask && mask[(int64_t)b * N + kk] == 0) x = -INFINITY;
      }
      // fp16: finite values beyond its range are clamped to +-65504
      if (sizeof(E) == 2 && x == x && fabsf(x) != INFINITY) x = fminf(fmaxf(x, -65504.f), 65504.f);
      v[j] = (E)x;
    }
    if constexpr (sizeof(E) == 2) {
      *reinterpret_cast<u32x4*>(biasp + e * 8) = __builtin_bit_cast(u32x4, v);
    } else {
      *reinterpret_cast<u32x4*>(biasp + e * 8) = __builtin_bit_cast(u32x4, *reinterpret_cast<float(*)[4]>(v));
      *reinterpret_cast<u32x4*>(biasp + e * 8 + 4) = __builtin_bit_cast(u32x4, *reinterpret_cast<float(*)[4]>(v + 4));
    }
  }
}

// Exponents of one 32-key half `hf_` of the tile, base 2, all lines of the
// group: t = K . (Q log2(e)/sqrt(C))^T - ref + bias * log2(e), where the
// reference enters as the products' accumulator operand `ref_` ([qb] splats)
// and the prepared bias of the half (`braw`, 8 values per qb) is added by one
// fma per logit (v_fma_mix_f32 for the fp16 bias).  Dead keys: -inf.
#define EVO_FWD_T(hf_, ref_)                                                     \
  do {                                                                           \
    for (int rr = 0; rr < ROWS; ++rr)                                            \
      for (int kb = 0; kb < 2; ++kb) {                                           \
        const Op kf = ld8(sK[buf][rr] + ((hf_) * 32 + kb * 16 + l16) * KST + 8 * g); \
        for (int qb = 0; qb < 2; ++qb)                                           \
          t[rr][qb][kb] = mma32(kf, qf[rr][qb], ref_[rr][qb]);                   \
      }                                                                          \
    for (int rr = 0; rr < ROWS; ++rr)                                            \
      for (int qb = 0; qb < 2; ++qb) {                                           \
        if constexpr (HAS_BIAS) {                                                \
          add_bias8(t[rr][qb][0], t[rr][qb][1], braw[qb]);                        \
        } else {                                                                 \
          if (k0 + BK > N)                                                       \
            for (int kb = 0; kb < 2; ++kb)                                       \
              for (int i = 0; i < 4; ++i)                                        \
                if (k0 + (hf_) * 32 + 8 * g + 4 * kb + i >= N) t[rr][qb][kb][i] = -INFINITY; \
        }                                                                        \
      }                                                                          \
    if constexpr (ROW_MASK) {                                                    \
      for (int rr = 0; rr < ROWS; ++rr) {                                        \
        const int kbase = k0 + (hf_) * 32 + 8 * g;                               \
        for (int j = 0; j < 8; ++j) {                                            \
          const bool dead = kbase + j < N && mrow[rr][kbase + j] == 0;           \
          if (dead) {                                                            \
            t[rr][0][j >> 2][j & 3] = -INFINITY;                                 \
            t[rr][1][j >> 2][j & 3] = -INFINITY;                                 \
          }                                                                      \
        }                                                                        \
      }                                                                          \
    }                                                                            \
  } while (0)

// x += bias * log2(e) for the 8 prepared values of a lane (keys 0..3 -> x,
// 4..7 -> y): fp16 through v_fma_mix_f32 (no separate conversion), fp32
// through a plain fma.
__device__ __forceinline__ void add_bias8(f32x4& x, f32x4& y, const u32x4& raw) {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  const f16x8 h = __builtin_bit_cast(f16x8, raw);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = __builtin_fmaf((float)h[i], kLog2e, x[i]);
    y[i] = __builtin_fmaf((float)h[4 + i], kLog2e, y[i]);
  }
}
__device__ __forceinline__ void add_bias8(f32x4& x, f32x4& y, const Raw8<float>& raw) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = __builtin_fmaf(__uint_as_float(raw.a[i]), kLog2e, x[i]);
    y[i] = __builtin_fmaf(__uint_as_float(raw.b[i]), kLog2e, y[i]);
  }
}

template <typename T, int ROWS, bool ROW_MASK, bool HAS_BIAS>
__global__ void __launch_bounds__(256)
attn_fwd_kernel(FwdParams p) {
  using Op = typename Tr<T>::Op;
  constexpr int KST = FwdLds<T>::KST, VST = FwdLds<T>::VST;
  __shared__ __attribute__((aligned(16))) T sK[2][ROWS][BK * KST];
  __shared__ __attribute__((aligned(16))) T sV[2][ROWS][FwdLds<T>::VROWS * VST];

  // Work order (fastest first): query tile, head within a head pair, row
  // group, head pair, batch.  The heads of a position are interleaved at
  // 64-byte granularity, so heads 2j and 2j+1 share every 128-byte line of
  // Q, K, V and G: running them back to back on one XCD lets the second
  // find the lines in L2 instead of fetching them again from HBM.
  const int w = xcd_work_index(p.total);
  if (w < 0) return;
  const int qt = w % p.n_qt;
  int t = w / p.n_qt;
  const int h = 2 * ((t >> 1) / p.n_rg % ((p.H + 1) >> 1)) + (t & 1);
  const int rg = (t >> 1) % p.n_rg;
  const int b = (t >> 1) / p.n_rg / ((p.H + 1) >> 1);
  if (h >= p.H) return;  // odd H: the missing partner of the last pair

  const int N = p.N, H = p.H, R = p.R;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int r0 = rg * ROWS;
  const int qw0 = qt * BQ + wave * BQW;
  const int pos_stride = H * C;
  const int64_t line_stride = (int64_t)N * pos_stride;

  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);

  const T* kline[ROWS];
  const T* vline[ROWS];
  bool live[ROWS];
#pragma unroll
  for (int rr = 0; rr < ROWS; ++rr) {
    const int r = min(r0 + rr, R - 1);
    live[rr] = r0 + rr < R;
    const int64_t lo = ((int64_t)b * R + r) * line_stride + h * C;
    kline[rr] = K + lo;
    vline[rr] = V + lo;
  }

  // Per-line state.
  Op qf[ROWS][2];
  f32x4 o[ROWS][2][2];
  float m[ROWS][2], l[ROWS][2];
#pragma unroll
  for (int rr = 0; rr < ROWS; ++rr) {
    const int r = min(r0 + rr, R - 1);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int q = qw0 + qb * 16 + l16;
      if (q < N) {
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

  // This lane's 8 bias values of (qb, half) in key tile `tile` sit at
  // bbase + tile * BQ*BK + (qb*2 + half) * 512 (prepared tile order).
  using E = typename PB<T>::E;
  const E* btile = HAS_BIAS ? static_cast<const E*>(p.biasp) +
                                  (((int64_t)b * H + h) * (p.Nq / BQ) + qt) *
                                      (p.Nk / BK) * (BQ * BK)
                            : nullptr;  // this workgroup's row of tiles
  const E* bbase = HAS_BIAS ? btile + wave * 2048 + lane * 8 : nullptr;
  const uint8_t* mrow[ROWS];
  if constexpr (ROW_MASK) {
#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr)
      mrow[rr] = p.mask + ((int64_t)b * p.mask_rows + min(r0 + rr, R - 1)) * N;
  }

  KVRaw<T> raw[ROWS];
  // Bias values of the next half tile as loaded (raw), fetched into the
  // registers the current half has just used.  (bf16 inputs: 8 fp16 values
  // per (qb, half) in one buffer load from the workgroup's tile row with the
  // lane's offset fixed, like the K/V tiles.)
  using BRaw = std::conditional_t<sizeof(T) == 2, u32x4, Raw8<float>>;
  BRaw braw[2];  // [qb], one half tile ahead
  const uint32_t bvoff = (uint32_t)(wave * 2048 + lane * 8) * 2u;
  const uint32_t bbytes = (uint32_t)(p.Nk / BK) * (BQ * BK) * 2u;  // the row
#define EVO_FETCH_BIAS(k0_, half_)                                                 \
  do {                                                                         \
    if constexpr (HAS_BIAS) {                                                  \
      for (int qb = 0; qb < 2; ++qb) {                                         \
        if constexpr (sizeof(T) == 2)                                          \
          braw[qb] = buf_ld128(btile, bbytes, bvoff + (qb * 2 + (half_)) * 1024u, \
                               (uint32_t)((k0_) / BK) * (BQ * BK * 2u));       \
        else                                                                   \
          ld_raw8(braw[qb], bbase + (int64_t)((k0_) / BK) * (BQ * BK) + (qb * 2 + (half_)) * 512); \
      }                                                                        \
    }                                                                          \
  } while (0)
#pragma unroll
  for (int rr = 0; rr < ROWS; ++rr) fetch_kv<T>(raw[rr], kline[rr], vline[rr], 0, N, pos_stride);
  EVO_FETCH_BIAS(0, 0);

  // -m of each query as a splat accumulator operand of the logit products
  // (+inf while a query has seen no live key: its exponents are then inf or
  // NaN and force the exact path)
  f32x4 negm[ROWS][2];
#pragma unroll
  for (int rr = 0; rr < ROWS; ++rr)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) negm[rr][qb] = f32x4{INFINITY, INFINITY, INFINITY, INFINITY};
  f32x4 zero[ROWS][2];
#pragma unroll
  for (int rr = 0; rr < ROWS; ++rr)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) zero[rr][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Sum of p over a half tile for each query.  bf16: on the matrix core
  // (A = ones), so every lane holds its query's whole sum; fp32: the lane's
  // 8 values, summed across lanes in the epilogue.
  constexpr bool kRowSum = sizeof(T) == 2;
  auto half_sum = [&](const Op& pv) -> float {
    if constexpr (kRowSum) {
      Op ones;
#pragma unroll
      for (int j = 0; j < 8; ++j) ones[j] = (__bf16)1.0f;
      return mma32(ones, pv, f32x4{0.f, 0.f, 0.f, 0.f})[0];
    } else {
      return sum8(pv, 0.f);
    }
  };

  const int ntiles = (N + BK - 1) / BK;
  for (int tile = 0; tile < ntiles; ++tile) {
    const int k0 = tile * BK;
    const int buf = tile & 1;
#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr) store_kv<T>(raw[rr], sK[buf][rr], sV[buf][rr]);
    __syncthreads();
    // The next tile's K/V (after the last tile: keys past N, zeros for bf16,
    // key N-1 again for fp32; unused).  Unconditional, so that the waits for
    // these loads are exact.
#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr)
      fetch_kv<T>(raw[rr], kline[rr], vline[rr], k0 + BK, N, pos_stride);

    // The tile in two 32-key halves: logits, softmax and PV of one half
    // before the next (half the logit and P registers of a whole tile).  All
    // lines of the group go through each phase together, so the matrix-core
    // work of one line overlaps the softmax of the other.
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4 t[ROWS][2][2];  // [rr][qb][kb] exponents, base 2
      // The products run at raised wave priority, so that a wave reaching
      // them issues them ahead of the other waves' softmax arithmetic and
      // the matrix core is fed sooner.
      __builtin_amdgcn_s_setprio(1);
      EVO_FWD_T(hf, negm);
      __builtin_amdgcn_s_setprio(0);

      // p = exp2(t), rounded to the operand type at once: P^T is kept as
      // matrix-core operands and the row sums are taken over exactly the
      // rounded values the PV product uses.  Fast path: the current
      // reference; the first half of the first tile always takes the exact
      // maximum.
      Op pf[ROWS][2];  // [rr][qb]
      float psum[ROWS][2];
      bool slow = tile == 0 && hf == 0;
      if (!slow) {
        bool redo = false;
#pragma unroll
        for (int rr = 0; rr < ROWS; ++rr)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            f32x4 e[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i) e[kb][i] = exp2_fast(t[rr][qb][kb][i]);
            pf[rr][qb] = pack8(e[0], e[1], (Op*)nullptr);
            psum[rr][qb] = half_sum(pf[rr][qb]);
            // not yet anchored (inf or NaN), or too large
            redo |= !(psum[rr][qb] <= (kRowSum ? kHeadroomRow : kHeadroom));
          }
        slow = __builtin_amdgcn_ballot_w64(redo) != 0;
      }
      if (slow) {
        // The exponents again, relative to 0, and the reference raised to
        // the half's maximum where needed.
        EVO_FWD_T(hf, zero);
#pragma unroll
        for (int rr = 0; rr < ROWS; ++rr)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i) mx = fmaxf(mx, t[rr][qb][kb][i]);
            mx = fmaxf(mx, shfl_xor(mx, 16));
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const float mold = m[rr][qb];
            const float mnew = fmaxf(mold, mx);
            const float muse = (mnew == -INFINITY) ? 0.f : mnew;
            const float alpha = (mold == -INFINITY) ? 0.f : exp2_fast(mold - muse);
            m[rr][qb] = (mnew == -INFINITY) ? -INFINITY : muse;
            const float nm = -m[rr][qb];
            negm[rr][qb] = f32x4{nm, nm, nm, nm};
            l[rr][qb] *= alpha;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) o[rr][qb][cb] *= alpha;
            f32x4 e[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i) e[kb][i] = exp2_fast(t[rr][qb][kb][i] - muse);
            pf[rr][qb] = pack8(e[0], e[1], (Op*)nullptr);
            psum[rr][qb] = half_sum(pf[rr][qb]);
          }
      }
      // the bias of the next half (bf16 reads past the workgroup's row of
      // tiles as zeros, so it needs no test and its waits stay exact)
      if (hf == 0)
        EVO_FETCH_BIAS(k0, 1);
      else if (sizeof(T) == 2 || tile + 1 < ntiles)
        EVO_FETCH_BIAS(k0 + BK, 0);
#pragma unroll
      for (int rr = 0; rr < ROWS; ++rr)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) l[rr][qb] += psum[rr][qb];

#pragma unroll
      for (int rr = 0; rr < ROWS; ++rr) {
        Op vf[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          if constexpr (sizeof(T) == 2) {
            // V^T fragment: keys hf*32 + 8g .. +7 of dim cb*16 + l16
            const T* v0 = sV[buf][rr] + (hf * 32 + 8 * g + (l16 >> 2)) * VST + cb * 16 + 4 * (l16 & 3);
            vf[cb] = lds_read_tr_op(v0, v0 + 4 * VST);
          } else {
            vf[cb] = ld8(sV[buf][rr] + (cb * 16 + l16) * VST + hf * 32 + 8 * g);
          }
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
            o[rr][qb][cb] = mma32(vf[cb], pf[rr][qb], o[rr][qb][cb]);
        __builtin_amdgcn_s_setprio(0);
      }
    }
  }

  // Epilogue: normalise, gate, store; LSE in natural log.
  const T* G = static_cast<const T*>(p.gate);
  T* Out = static_cast<T*>(p.out);
#pragma unroll
  for (int rr = 0; rr < ROWS; ++rr) {
    if (!live[rr]) continue;
    const int r = r0 + rr;
    const int64_t lo = ((int64_t)b * R + r) * line_stride + h * C;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float lt = l[rr][qb];
      if constexpr (!kRowSum) {
        lt += shfl_xor(lt, 16);
        lt += shfl_xor(lt, 32);
      }
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

#undef EVO_FETCH_BIAS

template <typename T, int ROWS, bool ROW_MASK>
hipError_t launch_t(const FwdParams& p, hipStream_t s) {
  const int grid = ((p.total + kNumXcd - 1) / kNumXcd) * kNumXcd;
  if (p.biasp)
    hipLaunchKernelGGL((attn_fwd_kernel<T, ROWS, ROW_MASK, true>), dim3(grid), dim3(256), 0,
                       s, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<T, ROWS, ROW_MASK, false>), dim3(grid), dim3(256), 0,
                       s, p);
  return hipGetLastError();
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

size_t attn_fwd_workspace(int dtype, int64_t B, int64_t N, int64_t H) {
  return (size_t)(B * H * round_up(N, BQ) * round_up(N, BK) * (dtype == 1 ? 2 : 4));
}

// Scratch of the allocation-free forward entry point: a file-scope device
// array (every GPU the library runs on holds its own copy until the process
// ends).  In host code `scratch` names a host-side stand-in, not device
// memory, so its device address is looked up with hipGetSymbolAddress once
// per device, with that device current, and only that address is used.
namespace {
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t fwd_static_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

hipError_t launch_attn_fwd(const AttnFwdArgs& a, hipStream_t s) {
  FwdParams p{};
  p.q = a.q; p.k = a.k; p.v = a.v; p.gate = a.gate;
  p.out = a.out; p.lse = a.lse;
  p.B = (int)a.B; p.R = (int)a.R; p.N = (int)a.N; p.H = (int)a.H;
  p.mask_rows = a.mask ? (int)a.mask_rows : 1;
  p.qscale = kLog2e / sqrtf((float)C);
  p.Nq = (int)round_up(a.N, BQ);
  p.Nk = (int)round_up(a.N, BK);
  const bool row_mask = a.mask && a.mask_rows > 1;
  const bool shared_mask = a.mask && !row_mask;
  p.mask = row_mask ? a.mask : nullptr;
  p.biasp = nullptr;
  if (a.bias || shared_mask) {
    void* bp = a.workspace;
    const int64_t work = a.B * a.H * p.Nq * (p.Nk / 8);
    const int grid = (int)std::min<int64_t>((work + 255) / 256, 8192);
    if (a.dtype == 1)
      hipLaunchKernelGGL(fwd_bias_prep_kernel<bf16_t>, dim3(grid), dim3(256), 0, s,
                         static_cast<const bf16_t*>(a.bias), a.mask, (int)shared_mask,
                         static_cast<_Float16*>(bp), p.B, p.H, p.N, p.Nq, p.Nk);
    else
      hipLaunchKernelGGL(fwd_bias_prep_kernel<float>, dim3(grid), dim3(256), 0, s,
                         static_cast<const float*>(a.bias), a.mask, (int)shared_mask,
                         static_cast<float*>(bp), p.B, p.H, p.N, p.Nq, p.Nk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    p.biasp = bp;
  }
  // One line per workgroup.  (A two-line variant, sharing each bias tile
  // between two lines, needs ~210 registers per lane, hence two waves per
  // SIMD against four for one line; measured slower at N_res = 768.)
  const int rows = 1;
  p.n_qt = (int)((a.N + BQ - 1) / BQ);
  p.n_rg = (int)((a.R + rows - 1) / rows);
  const int64_t total = a.B * ((a.H + 1) / 2) * 2 * (int64_t)p.n_rg * p.n_qt;
  if (total > (int64_t)INT32_MAX - 8) return hipErrorInvalidValue;
  p.total = (int)total;
  if (a.dtype == 1)
    return row_mask ? launch_t<bf16_t, 1, true>(p, s) : launch_t<bf16_t, 1, false>(p, s);
  return row_mask ? launch_t<float, 1, true>(p, s) : launch_t<float, 1, false>(p, s);
}

}  // namespace evo
