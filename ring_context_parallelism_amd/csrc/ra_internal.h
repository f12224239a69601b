// Internal declarations shared by the host driver and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra.h"

namespace ra {

// Position map of one layout (see ra.h for the three layouts).  32-bit integers:
// S < 2^31 is validated on the host.
struct LayoutMap {
  int32_t layout;  // ra_layout_t
  int32_t S;       // total sequence
  int32_t p;       // ring size
  int32_t L;       // tokens per chunk
  int32_t h;       // zigzag sub-block, S / (2p)
};

// Global position of local token t of chunk c.
__host__ __device__ inline int32_t pos_of(const LayoutMap& m, int32_t c, int32_t t) {
  if (m.layout == RA_LAYOUT_CONTIGUOUS) return c * m.L + t;
  if (m.layout == RA_LAYOUT_STRIPED) return t * m.p + c;
  return t < m.h ? c * m.h + t : (2 * m.p - 1 - c) * m.h + (t - m.h);
}

__host__ __device__ inline int32_t clamp_i(int32_t x, int32_t lo, int32_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Number of local tokens u of chunk c with pos(c, u) <= X.  pos is increasing in
// u for every layout, so these tokens are exactly the prefix [0, count).  Under a
// causal mask this is the number of keys of chunk c a query at position X sees.
__host__ __device__ inline int32_t count_le(const LayoutMap& m, int32_t c, int32_t X) {
  if (m.layout == RA_LAYOUT_CONTIGUOUS) return clamp_i(X - c * m.L + 1, 0, m.L);
  if (m.layout == RA_LAYOUT_STRIPED) {
    if (X < c) return 0;
    int32_t n = (X - c) / m.p + 1;
    return n < m.L ? n : m.L;
  }
  return clamp_i(X - c * m.h + 1, 0, m.h) + clamp_i(X - (2 * m.p - 1 - c) * m.h + 1, 0, m.h);
}

// Arguments of one forward ring step.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_sb, q_sh, q_st;     // element strides of q
  int64_t kv_sb, kv_sh, kv_st;  // element strides of k and v
  int32_t B, Hq, Hkv, group;    // group = Hq / Hkv
  int32_t cq, ck;               // query chunk, KV chunk
  int32_t causal;
  int32_t n_qtiles;             // ceil(L / BM)
  LayoutMap map;
  float scale_log2;             // scale * log2(e)
  // merge input (nullable): fp32 contiguous [B, Hq, L, D] and [B, Hq, L]
  const float* acc_in;
  const float* lse_in;
  // output: fp32 contiguous when out_f32, else the problem dtype with o strides
  void* out;
  int32_t out_f32;
  int64_t o_sb, o_sh, o_st;
  float* lse_out;               // fp32 [B, Hq, L]
};

// Arguments of one backward ring step.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  int64_t q_sb, q_sh, q_st;
  int64_t kv_sb, kv_sh, kv_st;
  int64_t o_sb, o_sh, o_st;     // strides of dout
  int32_t B, Hq, Hkv, group;
  int32_t cq, ck, causal;
  int32_t n_ktiles;             // ceil(L / BN) key tiles
  LayoutMap map;
  float scale;                  // softmax scale
  float scale_log2;             // scale * log2(e)
  const float* lse;             // final merged LSE (natural log), [B, Hq, L]
  const float* delta;           // rowsum(dO * O), [B, Hq, L]
  float* dq;                    // [B, Hq, L, D]   (+=)
  float* dk;                    // [B, Hkv, L, D]  (+=)
  float* dv;                    // [B, Hkv, L, D]  (+=)
};

// Launchers (defined in the .hip files).  Return the hipError_t of the launch.
hipError_t launch_fwd(int dtype, int D, const FwdArgs& a, hipStream_t s);
// which: 1 = dK/dV kernel, 2 = dQ kernel, 3 = both.
hipError_t launch_bwd(int dtype, int D, const BwdArgs& a, int which, hipStream_t s);
int fwd_block_m(int dtype, int D);
int bwd_block_n(int dtype, int D);
hipError_t launch_lse_merge(int64_t rows, int32_t d, float* o_acc, float* lse_acc,
                            const float* o_part, const float* lse_part, hipStream_t s);
hipError_t launch_bwd_delta(int dtype, int32_t B, int32_t H, int32_t L, int32_t D,
                            const void* out, const void* dout, int64_t sb, int64_t sh,
                            int64_t st, float* delta, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t s);

}  // namespace ra
