// Device-side building blocks for the gfx950 (CDNA4) kernels: operand
// fragments, MFMA wrappers, conversions and the workgroup -> XCD mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace evo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bfloat16 storage in HBM

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

// Element traits.  An MFMA operand fragment holds, per lane, 8 values that
// are consecutive along the contraction index.
template <typename T> struct Tr;
template <> struct Tr<bf16_t> {
  using Op = bf16x8;
  static __device__ __forceinline__ float to_f(bf16_t x) {
    return __uint_as_float(uint32_t(x) << 16);
  }
  static __device__ __forceinline__ bf16_t from_f(float x) {
    __bf16 b = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(bf16_t, b);
  }
};
template <> struct Tr<float> {
  using Op = f32x8;
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
};

// 16x16 output tile, contraction depth 32.  Lane l holds A[l%16][8*(l/16)+j]
// and B[8*(l/16)+j][l%16] for j < 8, and C/D[4*(l/16)+i][l%16] for i < 4.
__device__ __forceinline__ f32x4 mma32(const bf16x8& a, const bf16x8& b,
                                       f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp32 version: eight 16x16x4 steps.  Step j contracts over the values each
// lane holds at position j, i.e. over the depth indices {8g + j : g < 4};
// the eight steps together cover the same 32 indices as the bf16 form, so
// both share one fragment layout.
__device__ __forceinline__ f32x4 mma32(const f32x8& a, const f32x8& b,
                                       f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float exp2_fast(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}
__device__ __forceinline__ float log2_fast(float x) {
  return __builtin_amdgcn_logf(x);  // v_log_f32 (base 2)
}
__device__ __forceinline__ float rcp_fast(float x) {
  return __builtin_amdgcn_rcpf(x);
}
__device__ __forceinline__ float sigmoid_f(float x) {
  return rcp_fast(1.0f + exp2_fast(-x * kLog2e));
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Pack 8 fp32 values into an operand fragment of type Op.
__device__ __forceinline__ bf16x8 pack8(const f32x4& a, const f32x4& b,
                                        bf16x8*) {
  bf16x8 r;
  r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2];
  r[3] = (__bf16)a[3]; r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1];
  r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
  return r;
}
__device__ __forceinline__ f32x8 pack8(const f32x4& a, const f32x4& b,
                                       f32x8*) {
  f32x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// acc + the sum of the 8 values of a fragment (bf16: v_dot2 with ones,
// fp32 accumulate; exact products, so only the additions round).
__device__ __forceinline__ float sum8(const bf16x8& v, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x2 pr = {v[2 * j], v[2 * j + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float sum8(const f32x8& v, float acc) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc += v[j];
  return acc;
}

// Scale every element of a fragment (in fp32, rounded back to the type).
__device__ __forceinline__ bf16x8 scale8(const bf16x8& v, float s) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)((float)v[j] * s);
  return r;
}
__device__ __forceinline__ f32x8 scale8(const f32x8& v, float s) {
  return v * s;
}

// Eight consecutive elements as loaded (16 bytes bf16, 32 bytes fp32), kept
// raw while a prefetch is in flight and widened to two fp32 accumulator
// operands (elements 0..3 and 4..7) only where they are used.  Native vector
// types, so the data never round-trips through scratch memory.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> { u32x4 a; };
template <> struct Raw8<float> { u32x4 a, b; };

__device__ __forceinline__ void ld_raw8(Raw8<bf16_t>& r, const bf16_t* p) {
  r.a = *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void ld_raw8(Raw8<float>& r, const float* p) {
  r.a = reinterpret_cast<const u32x4*>(p)[0];
  r.b = reinterpret_cast<const u32x4*>(p)[1];
}
__device__ __forceinline__ void widen8(const Raw8<bf16_t>& r, f32x4& x, f32x4& y) {
  x = f32x4{__uint_as_float(r.a.x << 16), __uint_as_float(r.a.x & 0xffff0000u),
            __uint_as_float(r.a.y << 16), __uint_as_float(r.a.y & 0xffff0000u)};
  y = f32x4{__uint_as_float(r.a.z << 16), __uint_as_float(r.a.z & 0xffff0000u),
            __uint_as_float(r.a.w << 16), __uint_as_float(r.a.w & 0xffff0000u)};
}
__device__ __forceinline__ void widen8(const Raw8<float>& r, f32x4& x, f32x4& y) {
  x = f32x4{__uint_as_float(r.a.x), __uint_as_float(r.a.y), __uint_as_float(r.a.z),
            __uint_as_float(r.a.w)};
  y = f32x4{__uint_as_float(r.b.x), __uint_as_float(r.b.y), __uint_as_float(r.b.z),
            __uint_as_float(r.b.w)};
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane r addresses a chunk of 4 consecutive 16-bit elements; lane i
// receives element i % 4 of the chunks addressed by lanes i / 4 + 4j,
// j = 0..3 (the mapping measured on gfx950).  So if lane r of group g points
// at row 8g + r/4 (+4 for a second read), columns c0 + 4(r % 4) .. +3, of a
// row-major tile, lane i gets column c0 + i of rows 8g .. 8g + 3 (+4): the
// 8 consecutive-row values of one column that an MFMA operand needs, read
// from a tile stored without transposition.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_ptr) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)lds_ptr);
#else
  (void)lds_ptr;
  return i16x4{};
#endif
}
// Two transposing reads (rows 8g..+3 at p0, 8g+4..+7 at p1) as one bf16
// operand fragment.
__device__ __forceinline__ bf16x8 lds_read_tr_op(const void* p0, const void* p1) {
  const i16x4 lo = lds_read_tr16(p0), hi = lds_read_tr16(p1);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// 16-byte buffer load from base + soff + voff.  `base` and `nbytes` must be
// the same across the wave (they form the buffer resource, in scalar
// registers), `soff` too; `voff` is the lane's byte offset.  Bytes at or
// past base + `nbytes` read as zero.  The whole offset goes into the lane
// offset operand (one add per load), which the buffer range check always
// covers; a scalar offset operand is documented as added after that check.
__device__ __forceinline__ u32x4 buf_ld128(const void* base, uint32_t nbytes, uint32_t voff,
                                           uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)(voff + soff), 0, 0);
#else
  (void)base; (void)nbytes; (void)voff; (void)soff;
  return u32x4{};
#endif
}

// Offset of element (row r, column k) of a row-major M x kp matrix stored
// in the order of MFMA A-operand fragments of 16 rows x 32 columns: per
// (16-row block, 32-column block) 64 lanes x 8 elements, lane l holding row
// l % 16 and columns 8 (l / 16) .. +7 of the block.  kp is a multiple of 32.
// A wave reads one block as one contiguous 1 KB load.
__device__ __forceinline__ int64_t frag_off(int64_t r, int k, int kp) {
  return ((r >> 4) * (kp >> 5) + (k >> 5)) * 512 + ((r & 15) + 16 * ((k >> 3) & 3)) * 8 + (k & 7);
}

// Workgroups are dispatched round-robin over the XCDs (workgroup i runs on
// XCD i % 8).  Remap so that XCD x receives the contiguous work range
// [x * per, (x + 1) * per): neighbouring work items, which share inputs,
// then run together on one XCD and meet in its L2.  `total` is the real
// number of work items; the grid has per * 8 workgroups and the function
// returns -1 for the padding ones.
__device__ __forceinline__ int xcd_work_index(int total) {
  const int per = (total + kNumXcd - 1) / kNumXcd;
  const int i = blockIdx.x;
  const int w = (i % kNumXcd) * per + i / kNumXcd;
  return w < total ? w : -1;
}

}  // namespace evo
