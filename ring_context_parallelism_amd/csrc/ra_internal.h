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

// Document [lo, hi) of global position X in one batch element's boundary list
// e[0..n-1] (n >= 2, nondecreasing): e[j] <= X < e[j+1].  Returns false for right
// padding (X >= e[n-1]) and for X < e[0].  The search keeps e[a] <= X < e[b] and
// halves b - a, so it ends after at most log2(n) steps and reads only e[0..n-1]
// whatever the list holds.
__host__ __device__ inline bool doc_range(const int32_t* e, int32_t n, int32_t X, int32_t& lo,
                                          int32_t& hi) {
  if (X < e[0] || X >= e[n - 1]) return false;
  int32_t a = 0, b = n - 1;
  while (b - a > 1) {
    const int32_t m = (a + b) >> 1;
    if (e[m] <= X) a = m; else b = m;
  }
  lo = e[a];
  hi = e[b];
  return true;
}

// Keys of chunk ck visible to the query at global position P: the local interval
// [lo, hi) (pos is increasing in the local index, so the visible keys of one
// document are contiguous).  e == nullptr: dense sequence.  A query in the right
// padding sees nothing: lo = L, hi = 0.
__host__ __device__ inline void key_interval(const LayoutMap& m, int32_t ck, int32_t P,
                                             int32_t causal, const int32_t* e, int32_t n,
                                             int32_t& lo, int32_t& hi) {
  if (e == nullptr) {
    lo = 0;
    hi = causal ? count_le(m, ck, P) : m.L;
    return;
  }
  int32_t dlo, dhi;
  if (!doc_range(e, n, P, dlo, dhi)) {
    lo = m.L;
    hi = 0;
    return;
  }
  lo = count_le(m, ck, dlo - 1);
  hi = count_le(m, ck, causal ? P : dhi - 1);
}

// Queries of chunk cq that see the key at global position P: the local interval
// [lo, hi); a key in the right padding is seen by nobody: lo = L, hi = 0.
__host__ __device__ inline void query_interval(const LayoutMap& m, int32_t cq, int32_t P,
                                               int32_t causal, const int32_t* e, int32_t n,
                                               int32_t& lo, int32_t& hi) {
  if (e == nullptr) {
    lo = causal ? count_le(m, cq, P - 1) : 0;
    hi = m.L;
    return;
  }
  int32_t dlo, dhi;
  if (!doc_range(e, n, P, dlo, dhi)) {
    lo = m.L;
    hi = 0;
    return;
  }
  lo = count_le(m, cq, (causal ? P : dlo) - 1);
  hi = count_le(m, cq, dhi - 1);
}

#if defined(__HIPCC__)
// Vector types, constants and small helpers of the kernels.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMInit = -1.0e30f;  // finite start for the running max (no inf - inf)
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.4426950408889634f;
// Lazy rescale of the online softmax: a lane's partial row sum of one key tile may
// reach 2^8 before the reference max must move (so every p <= 2^8).
constexpr float kSumCap = 256.0f;

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Buffer resource over [base, base + bytes): a load past the end returns zeros.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Workgroup id -> logical work item.  Workgroups are dispatched round-robin over the
// 8 XCDs, so give every XCD one contiguous range of logical ids: the tiles that share
// a head (and so its K/V or Q reads) then share that XCD's L2.
__device__ inline int xcd_remap(int bid, int nblk) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = (nblk + 7) >> 3, rem = nblk & 7;
  if (rem == 0 || xcd < rem) return xcd * per + slot;
  return rem * per + (xcd - rem) * (per - 1) + slot;
}

// Max and sum over lanes l and l ^ 32 (the two halves of a wave).  permlane32_swap
// returns (own, partner) in lanes < 32 and (partner, own) in lanes >= 32, so a max or
// a sum of the pair needs no select.
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup-wide (min lo, max hi, max lo, min hi) of per-row intervals [lo, hi)
// (packed documents): tiles from min lo to max hi hold every visible pair, and
// [max lo, min hi) is visible to every row.  A lane holding several rows passes the
// min and max of its rows' bounds.  red: 4 ints of LDS.  Every thread of the
// workgroup must call it (two barriers).
__device__ inline void wg_interval_reduce(int* red, int lo_min, int hi_max, int lo_max,
                                          int hi_min, int n, int& min_lo, int& max_hi,
                                          int& max_lo, int& min_hi) {
  if (threadIdx.x == 0) {
    red[0] = n;
    red[1] = 0;
    red[2] = 0;
    red[3] = n;
  }
  __syncthreads();
  atomicMin(&red[0], lo_min);
  atomicMax(&red[1], hi_max);
  atomicMax(&red[2], lo_max);
  atomicMin(&red[3], hi_min);
  __syncthreads();
  min_lo = red[0];
  max_hi = red[1];
  max_lo = red[2];
  min_hi = red[3];
}
// One row per lane.
__device__ inline void wg_interval_reduce(int* red, int lo, int hi, int n, int& min_lo,
                                          int& max_hi, int& max_lo, int& min_hi) {
  wg_interval_reduce(red, lo, hi, lo, hi, n, min_lo, max_hi, max_lo, min_hi);
}
// Two rows per lane.
__device__ inline void wg_interval_reduce2(int* red, const int (&lo)[2], const int (&hi)[2],
                                           int n, int& min_lo, int& max_hi, int& max_lo,
                                           int& min_hi) {
  wg_interval_reduce(red, min(lo[0], lo[1]), max(hi[0], hi[1]), max(lo[0], lo[1]),
                     min(hi[0], hi[1]), n, min_lo, max_hi, max_lo, min_hi);
}
#endif

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
  const int32_t* seg;           // packed-document boundaries [B, seg_n], or nullptr
  int32_t seg_n;
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
  const int32_t* seg;           // packed-document boundaries [B, seg_n], or nullptr
  int32_t seg_n;
  int32_t write;                // 1: store the step's dq / dk, dv (every element, zeros
                                // included) instead of adding to them
};

// Launchers (defined in the .hip files).  Return the hipError_t of the launch.
// dk: the true head dim (the fp32 kernel skips the zero pad columns of QK^T).
hipError_t launch_fwd(int dtype, int D, int dk, const FwdArgs& a, hipStream_t s);
// The fp32 forward (ra_fwd_f32.hip), which launch_fwd calls for fp32 problems; its
// workgroups take kFwdF32BlockM query rows of one head.
constexpr int kFwdF32BlockM = 128;
hipError_t launch_fwd_f32(int D, int dk, bool packed, const FwdArgs& a, hipStream_t s);
// which: 1 = dK/dV kernel, 2 = dQ kernel, 3 = both.
hipError_t launch_bwd(int dtype, int D, const BwdArgs& a, int which, hipStream_t s);
int fwd_block_m(int dtype, int D, bool packed, int group);
int bwd_block_n(int dtype, int D);
hipError_t launch_lse_merge(int64_t rows, int32_t d, float* o_acc, float* lse_acc,
                            const float* o_part, const float* lse_part, hipStream_t s);
hipError_t launch_bwd_delta(int dtype, int32_t B, int32_t H, int32_t L, int32_t D,
                            const void* out, const void* dout, int64_t sb, int64_t sh,
                            int64_t st, float* delta, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t s);

// Static device scratch of ra_ring_bwd_noalloc (ra_noalloc.hip): its size, and the
// device address of the current device's copy (looked up once per device).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
hipError_t static_scratch(void** ptr);

}  // namespace ra
