// Internal interface between the C-ABI layer (evo_api.cpp) and the kernel
// translation units.  Arguments reaching these functions are validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace evo {

struct AttnFwdArgs {
  int dtype;  // 0 fp32, 1 bf16
  int64_t B, R, N, H;
  const void* q;
  const void* k;
  const void* v;
  const void* gate;       // may be null
  const uint8_t* mask;    // may be null
  int64_t mask_rows;      // 1 or R
  const void* bias;       // may be null
  void* out;
  float* lse;             // may be null
  void* workspace;        // attn_fwd_workspace bytes when bias or mask given
};

struct AttnBwdArgs {
  int dtype;
  int64_t B, R, N, H;
  const void* q;
  const void* k;
  const void* v;
  const void* gate;
  const uint8_t* mask;
  int64_t mask_rows;
  const void* bias;
  const void* out;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  void* dgate;
  float* dbias;
  void* workspace;
};

struct ProjectArgs {
  int dtype;
  int64_t N, CZ, H;
  int ending;
  const void* z;
  const void* ln_w;
  const void* ln_b;
  float eps;
  const void* w_q;
  const void* w_k;
  const void* w_v;
  const void* w_g;
  const void* b_g;  // may be null
  const void* w_bias;
  void* q;
  void* k;
  void* v;
  void* g;
  void* bias;
};

struct OutProjectArgs {
  int dtype;
  int64_t N, CZ, H;
  int ending;
  const void* o;
  const void* w_o;
  const void* b_o;  // may be null
  void* out;
};

struct OutProjectBwdArgs {
  int dtype;
  int64_t N, CZ, H;
  int ending;
  const void* o;
  const void* w_o;
  const void* dout;
  void* d_o;
  float* dw_o;
  float* db_o;
  void* workspace;  // proj_bwd_workspace bytes
};

struct ProjectBwdArgs {
  int dtype;
  int64_t N, CZ, H;
  int ending;
  const void* z;
  const void* ln_w;
  const void* ln_b;
  float eps;
  const void* w_q;
  const void* w_k;
  const void* w_v;
  const void* w_g;
  const void* w_bias;
  const void* dq;
  const void* dk;
  const void* dv;
  const void* dg;
  const float* dbias;
  void* dz;
  float* dln_w;
  float* dln_b;
  float* dw_q;
  float* dw_k;
  float* dw_v;
  float* dw_g;
  float* db_g;
  float* dw_bias;
  void* workspace;  // proj_bwd_workspace bytes
};

// LayerNorm + two projections (a, b) of rows of a [lines x places x CZ]
// tensor, stored element (channel c, line, place) at c*s_ch + line*s_line +
// place*s_place, zero where the place is masked.  Row of (line, place):
// line*P + place, or place*L + line when transposed.
struct ChannelProjectArgs {
  int dtype;
  int64_t L, P, CZ, C;
  int transposed;
  const void* z;
  const uint8_t* mask;  // [P] keep flags or null
  const void* ln_w;
  const void* ln_b;
  float eps;
  const void* w_a;
  const void* w_b;
  void* a;
  void* b;
  int64_t s_ch, s_line, s_place;
  // > 0: a is written in MFMA fragment order (frag_off) as a matrix of rows
  // (c * s_ch + line * s_line) / a_frag_kp and columns `place` (s_place = 1);
  // 0: a and b both at the strides above
  int64_t a_frag_kp = 0;
};

struct TriMulArgs {
  int dtype;
  int64_t N, CZ, C;
  int outgoing;
  const void* z;
  const uint8_t* mask;
  const void* ln_w;
  const void* ln_b;
  float eps;
  const void* w_a;
  const void* w_b;
  const void* w_o;
  const void* b_o;
  void* out;
  void* workspace;  // trimul_workspace bytes
};

struct TransitionArgs {
  int dtype;
  int64_t npos, CZ, HID;
  const void* z;
  const void* ln_w;
  const void* ln_b;
  float eps;
  const void* w_a;
  const void* w_b;
  const void* w_o;
  void* out;
  void* workspace;  // transition_workspace bytes
};

constexpr int kHeadDim = 32;

size_t attn_fwd_workspace(int dtype, int64_t B, int64_t N, int64_t H);
hipError_t launch_attn_fwd(const AttnFwdArgs& a, hipStream_t s);
// The library's static forward scratch on the current device (its address,
// looked up once per device) and its size in bytes.
hipError_t fwd_static_scratch(void** ptr, size_t* bytes);
hipError_t launch_probe(int kind, int waves_per_simd, int iters, float* out, hipStream_t s);
size_t attn_bwd_workspace(int dtype, int64_t B, int64_t R, int64_t N,
                          int64_t H);
hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t s);
hipError_t launch_project(const ProjectArgs& a, hipStream_t s);
hipError_t launch_out_project(const OutProjectArgs& a, hipStream_t s);
size_t proj_bwd_workspace(int64_t N, int64_t CZ, int64_t H);
hipError_t launch_channel_project(const ChannelProjectArgs& a, hipStream_t s);
size_t trimul_workspace(int dtype, int64_t N, int64_t C);
hipError_t launch_trimul(const TriMulArgs& a, hipStream_t s);
// Backward of the multiplicative update: dz (dtype); dln_w, dln_b [CZ],
// dw_a, dw_b [C][CZ], dw_o [CZ][C], db_o [CZ] (fp32).
struct TriMulBwdArgs {
  int dtype;
  int64_t N, CZ, C;
  int outgoing;
  const void* z;
  const uint8_t* mask;
  const void* ln_w;
  const void* ln_b;
  float eps;
  const void* w_a;
  const void* w_b;
  const void* w_o;
  const void* dout;
  void* dz;
  float* dln_w;
  float* dln_b;
  float* dw_a;
  float* dw_b;
  float* dw_o;
  float* db_o;
  void* workspace;  // trimul_bwd_workspace bytes
};
size_t trimul_bwd_workspace(int dtype, int64_t N, int64_t CZ, int64_t C);
hipError_t launch_trimul_bwd(const TriMulBwdArgs& a, hipStream_t s);
// T_c = A_c . B_c^T for c < C: A, B [C][Np][Kp] (columns >= K zeroed here),
// T [C][M][M]; M <= Np, Np a multiple of pair_gemm_row_tile().
int pair_gemm_row_tile();
hipError_t launch_pair_gemm(int dtype, int C, int M, int K, int Np, int Kp, void* a, void* b,
                            void* t, bool a_frag, hipStream_t s);
// The same with M rows from a and M2 from b: A [C][Np][Kp], B [C][Np2][Kp],
// T [C][M][M2]; Np and Np2 multiples of pair_gemm_row_tile().
hipError_t launch_pair_gemm_rect(int dtype, int C, int M, int M2, int K, int Np, int Np2, int Kp,
                                 void* a, void* b, void* t, bool a_frag, hipStream_t s);
// bf16, one product with A in fragment order, M = N*C rows (i, c) and columns
// (j, d), C a multiple of 32: P written as pair rows pf[(i*N + j)*C + c][d] =
// scale * P[(i, c)][(j, d)], rounded once.
hipError_t launch_pair_gemm_pairs(int M, int K, int Np, int Kp, void* a, void* b, void* pf,
                                  int N, int C, float scale, hipStream_t s);
// Channel-major matrices [C] of (row r < rows, column q < ncols) at c*cs +
// r*ld + q to position rows dst[pos][C], pos = r*N + q (q*N + r when trans),
// zero where keep is given and keep[q] == 0.  C a multiple of 32, at most 128.
hipError_t launch_cm_to_pm(int dtype, const void* src, void* dst, int C, int rows, int ncols,
                           int64_t ld, int64_t cs, int N, int trans, const uint8_t* keep,
                           hipStream_t s);
// Outer product mean: m [S][N][CM] -> out [N][N][CZ].
struct OpmArgs {
  int dtype;
  int64_t S, N, CM, C, CZ;
  const void* m;
  const void* ln_w;
  const void* ln_b;
  float eps;
  const void* w_a;  // [C][CM]
  const void* w_b;  // [C][CM]
  const void* w_o;  // [CZ][C * C]
  const void* b_o;  // [CZ] or null
  void* out;
  void* workspace;  // opm_workspace bytes
};
size_t opm_workspace(int dtype, int64_t S, int64_t N, int64_t C);
hipError_t launch_opm(const OpmArgs& a, hipStream_t s);
// Backward of the outer product mean: dm (dtype); dln_w, dln_b [CM], dw_a,
// dw_b [C][CM], dw_o [CZ][C * C], db_o [CZ] (fp32).  CM at most 128, or 256.
struct OpmBwdArgs {
  int dtype;
  int64_t S, N, CM, C, CZ;
  const void* m;
  const void* ln_w;
  const void* ln_b;
  float eps;
  const void* w_a;
  const void* w_b;
  const void* w_o;
  const void* dout;
  void* dm;
  float* dln_w;
  float* dln_b;
  float* dw_a;
  float* dw_b;
  float* dw_o;
  float* db_o;
  void* workspace;  // opm_bwd_workspace bytes
};
size_t opm_bwd_workspace(int dtype, int64_t S, int64_t N, int64_t CM, int64_t C, int64_t CZ);
hipError_t launch_opm_bwd(const OpmBwdArgs& a, hipStream_t s);
// Weight gradients against plain position rows: for the nseg (1 or 4)
// segments A_s [npos][128] and B [npos][ncols] (LayerNorm-normalised from z
// when b_ln),  M_s = A_s^T B  and the column sums of A_s, reduced in a fixed
// order; dw_s [128][ncols] = M_s, or gamma * M_s + beta * colsum (b_ln), with
// M and the column sums also kept in mred [nseg*128][ncols], cred
// [nseg*128] (b_ln).
struct SegWGradArgs {
  int dtype;
  int64_t npos;
  int nseg;
  const void* aseg[4];
  const void* b;
  int ncols, b_ln;
  const void* ln_w;
  const void* ln_b;
  float eps;
  float* dw[4];
  float* mred;
  float* cred;
  void* workspace;  // seg_wgrad_workspace bytes
};
size_t seg_wgrad_workspace(int64_t npos, int64_t ncols);
hipError_t launch_seg_wgrad(const SegWGradArgs& a, hipStream_t s);
// Backward of the transition: dz [npos][CZ] (dtype); dln_w, dln_b [CZ],
// dw_a, dw_b [HID][CZ], dw_o [CZ][HID] (fp32).  HID a multiple of 128.
struct TransitionBwdArgs {
  int dtype;
  int64_t npos, CZ, HID;
  const void* z;
  const void* ln_w;
  const void* ln_b;
  float eps;
  const void* w_a;
  const void* w_b;
  const void* w_o;
  const void* dout;
  void* dz;
  float* dln_w;
  float* dln_b;
  float* dw_a;
  float* dw_b;
  float* dw_o;
  void* workspace;  // transition_bwd_workspace bytes
};
size_t transition_bwd_workspace(int dtype, int64_t npos, int64_t CZ, int64_t HID);
hipError_t launch_transition_bwd(const TransitionBwdArgs& a, hipStream_t s);
size_t transition_workspace(int dtype, int64_t CZ, int64_t HID);
hipError_t launch_transition(const TransitionArgs& a, hipStream_t s);
// Backward of a LayerNorm followed by nseg (2) bias-free projections of the
// rows z [npos][CZ]: with dY_s [npos][seg_w] the projections' gradients and
// W_s [seg_w][CZ] their weights,
//   dz = LayerNorm backward of sum_s dY_s . W_s       (dtype, [npos][CZ]),
//   dW_s = sum over positions of dY_s^T LN(z)         (fp32, [seg_w][CZ]),
//   dln_w, dln_b                                      (fp32, [CZ]),
// all reduced in a fixed order.  seg_w a multiple of 32, at most 128; CZ a
// multiple of 32, at most 128, or 256.
struct LnProjBwdArgs {
  int dtype;
  int64_t npos, CZ;
  int nseg, seg_w;
  const void* dy[2];
  const void* w[2];
  const void* z;
  const void* ln_w;
  const void* ln_b;
  float eps;
  void* dz;
  float* dw[2];
  float* dln_w;
  float* dln_b;
  void* workspace;  // ln_proj_bwd_workspace bytes
};
size_t ln_proj_bwd_workspace(int64_t npos, int64_t CZ, int seg_w);
// M = A^T B over npos plain rows: A [npos][a_w] (a_w a multiple of 32, at
// most 128), B [npos][b_w] at row stride b_ld (b_w a multiple of 16, at most
// 256); dw[r * dw_ld + c] = M[r][c] (fp32), dcol[r] = sum of A's column r
// (if dcol is given); fixed-order reduction.
struct ColWGradArgs {
  int dtype;
  int64_t npos;
  const void* a;
  int a_w;
  const void* b;
  int b_w;
  int64_t b_ld;
  float* dw;
  int64_t dw_ld;
  float* dcol;
  void* workspace;  // col_wgrad_workspace bytes
};
size_t col_wgrad_workspace(int64_t npos, int b_w);
hipError_t launch_col_wgrad(const ColWGradArgs& a, hipStream_t s);
hipError_t launch_ln_proj_bwd(const LnProjBwdArgs& a, hipStream_t s);
hipError_t launch_out_project_bwd(const OutProjectBwdArgs& a, hipStream_t s);
hipError_t launch_project_bwd(const ProjectBwdArgs& a, hipStream_t s);

}  // namespace evo
