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

// Triangular multiplicative update: LayerNorm + the a, b projections,
// stored channel-major with padded rows [C][Np][Kp] (row = line i, column =
// place k; zero where k is masked), for the per-channel products.
struct TriMulProjectArgs {
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
  void* a;
  void* b;
  int64_t Np, Kp;
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
size_t attn_bwd_workspace(int dtype, int64_t B, int64_t R, int64_t N,
                          int64_t H);
hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t s);
hipError_t launch_project(const ProjectArgs& a, hipStream_t s);
hipError_t launch_out_project(const OutProjectArgs& a, hipStream_t s);
size_t proj_bwd_workspace(int64_t N, int64_t CZ, int64_t H);
hipError_t launch_trimul_project(const TriMulProjectArgs& a, hipStream_t s);
size_t trimul_workspace(int dtype, int64_t N, int64_t C);
hipError_t launch_trimul(const TriMulArgs& a, hipStream_t s);
size_t transition_workspace(int dtype, int64_t CZ, int64_t HID);
hipError_t launch_transition(const TransitionArgs& a, hipStream_t s);
hipError_t launch_out_project_bwd(const OutProjectBwdArgs& a, hipStream_t s);
hipError_t launch_project_bwd(const ProjectBwdArgs& a, hipStream_t s);

}  // namespace evo
