// Memory-bound helper kernels: the standalone LSE merge, the backward's
// delta = rowsum(dO * O), and an fp32 fill (used instead of hipMemsetAsync so the
// drivers stay capturable in HIP graphs).
#include "ra_internal.h"

namespace ra {
namespace {

// One row of (o, lse) per group of G lanes; G divides 64 and the grid stride is a
// multiple of 256, so a row never spans two waves and every lane of a row reads
// lse_acc before the group leader rewrites it.  The grid is capped and strides over
// the rows, so any row count the entry point accepts fits one launch.
template <int G>
__global__ __launch_bounds__(256) void lse_merge_kernel(int64_t rows, int32_t d4, float* o_acc,
                                                        float* lse_acc, const float* o_part,
                                                        const float* lse_part) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < rows * G;
       gid += stride) {
    const int64_t row = gid / G;
    const int c0 = (int)(gid % G);
    const float la = lse_acc[row], lp = lse_part[row];
    if (lp == kNegInf) continue;  // empty partial: identity
    float wa, wp, lse;
    if (la == kNegInf) {
      wa = 0.0f;
      wp = 1.0f;
      lse = lp;
    } else {
      const float mx = fmaxf(la, lp);
      const float ea = __expf(la - mx), ep = __expf(lp - mx);
      const float den = ea + ep;
      wa = ea / den;
      wp = ep / den;
      lse = mx + __logf(den);
    }
    f32x4* oa = (f32x4*)(o_acc + row * (int64_t)d4 * 4);
    const f32x4* op = (const f32x4*)(o_part + row * (int64_t)d4 * 4);
    for (int c = c0; c < d4; c += G) {
      const f32x4 x = oa[c], y = op[c];
      f32x4 r;
      r[0] = x[0] * wa + y[0] * wp;
      r[1] = x[1] * wa + y[1] * wp;
      r[2] = x[2] * wa + y[2] * wp;
      r[3] = x[3] * wa + y[3] * wp;
      oa[c] = r;
    }
    if (c0 == 0) lse_acc[row] = lse;
  }
}

// delta[row] = sum_d dout[row, d] * out[row, d]; one row per group of G lanes, each
// lane reading 16 bytes of both tensors, then a butterfly reduction inside the group.
// Rows of one (batch, head) per workgroup block: G lanes share a row (16 bytes of
// each operand per lane), 256 / G rows per pass, kDeltaPasses passes whose loads are
// all issued before any is used.  Block -> (b*H + h, row block) is one scalar
// division per block; the grid is capped and strides over the blocks.
constexpr int kDeltaPasses = 4;

template <typename T, int D>
__device__ inline void bwd_delta_block(int32_t H, int32_t L, int64_t bh, int32_t blk,
                                       const T* out, const T* dout, int64_t sb, int64_t sh,
                                       int64_t st, float* delta) {
  constexpr int EPL = 16 / sizeof(T);  // elements per lane
  constexpr int G = D / EPL;           // lanes per row
  constexpr int RPP = 256 / G;         // rows per pass
  typedef T vec_t __attribute__((ext_vector_type(EPL)));
  const int64_t h = bh % H, b = bh / H;
  const int c = threadIdx.x % G, r = threadIdx.x / G;
  const T* ob = out + b * sb + h * sh + c * EPL;
  const T* db = dout + b * sb + h * sh + c * EPL;
  vec_t x[kDeltaPasses], y[kDeltaPasses];
#pragma unroll
  for (int p = 0; p < kDeltaPasses; ++p) {
    const int t = (blk * kDeltaPasses + p) * RPP + r;
    if (t < L) {
      x[p] = *(const vec_t*)(ob + (int64_t)t * st);
      y[p] = *(const vec_t*)(db + (int64_t)t * st);
    } else {
      x[p] = vec_t{};
      y[p] = vec_t{};
    }
  }
#pragma unroll
  for (int p = 0; p < kDeltaPasses; ++p) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc += (float)x[p][e] * (float)y[p][e];
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    const int t = (blk * kDeltaPasses + p) * RPP + r;
    if (t < L && c == 0) delta[bh * L + t] = acc;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(int32_t H, int32_t L, int32_t n_blk,
                                                        int64_t n_total, const T* out,
                                                        const T* dout, int64_t sb, int64_t sh,
                                                        int64_t st, float* delta) {
  for (int64_t id = blockIdx.x; id < n_total; id += gridDim.x)
    bwd_delta_block<T, D>(H, L, (int64_t)(id / n_blk), (int32_t)(id % n_blk), out, dout, sb, sh,
                          st, delta);
}

// Grid-stride fill: whole 16-byte chunks, then the n % 4 tail.
__global__ __launch_bounds__(256) void fill_kernel(float* p, int64_t n, float value) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n4 = n / 4;
  const f32x4 v = {value, value, value, value};
  for (int64_t i = i0; i < n4; i += stride) ((f32x4*)p)[i] = v;
  if (i0 < n - n4 * 4) p[n4 * 4 + i0] = value;
}

// Grids of the memory-bound helpers: enough workgroups to fill the chip many times
// over, capped so that a launch never exceeds the 2^32 work-item limit of one grid
// dimension; the kernels stride over whatever remains.
constexpr int64_t kMaxHelperBlocks = 1 << 20;

inline unsigned helper_grid(int64_t blocks) {
  return (unsigned)(blocks < kMaxHelperBlocks ? blocks : kMaxHelperBlocks);
}

template <typename T, int D>
hipError_t delta_launch(int32_t B, int32_t H, int32_t L, const void* out, const void* dout,
                        int64_t sb, int64_t sh, int64_t st, float* delta, hipStream_t s) {
  constexpr int RPB = 256 / (D / (16 / (int)sizeof(T))) * kDeltaPasses;  // rows per block
  const int32_t n_blk = (L + RPB - 1) / RPB;
  const int64_t blocks = (int64_t)B * H * n_blk;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3(helper_grid(blocks)), dim3(256), 0, s, H, L,
                     n_blk, blocks, (const T*)out, (const T*)dout, sb, sh, st, delta);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(int64_t rows, int32_t d, float* o_acc, float* lse_acc,
                            const float* o_part, const float* lse_part, hipStream_t s) {
  const int32_t d4 = d / 4;
  const int G = d4 <= 8 ? 8 : (d4 <= 16 ? 16 : (d4 <= 32 ? 32 : 64));
  const int64_t threads = rows * G;
  const int64_t blocks = (threads + 255) / 256;
  if (rows == 0) return hipSuccess;
  switch (G) {
    case 8:
      hipLaunchKernelGGL(lse_merge_kernel<8>, dim3(helper_grid(blocks)), dim3(256), 0, s, rows, d4,
                         o_acc, lse_acc, o_part, lse_part);
      break;
    case 16:
      hipLaunchKernelGGL(lse_merge_kernel<16>, dim3(helper_grid(blocks)), dim3(256), 0, s, rows, d4,
                         o_acc, lse_acc, o_part, lse_part);
      break;
    case 32:
      hipLaunchKernelGGL(lse_merge_kernel<32>, dim3(helper_grid(blocks)), dim3(256), 0, s, rows, d4,
                         o_acc, lse_acc, o_part, lse_part);
      break;
    default:
      hipLaunchKernelGGL(lse_merge_kernel<64>, dim3(helper_grid(blocks)), dim3(256), 0, s, rows, d4,
                         o_acc, lse_acc, o_part, lse_part);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_delta(int dtype, int32_t B, int32_t H, int32_t L, int32_t D,
                            const void* out, const void* dout, int64_t sb, int64_t sh,
                            int64_t st, float* delta, hipStream_t s) {
  if (dtype == RA_BF16) {
    if (D == 128) return delta_launch<__bf16, 128>(B, H, L, out, dout, sb, sh, st, delta, s);
    if (D == 64) return delta_launch<__bf16, 64>(B, H, L, out, dout, sb, sh, st, delta, s);
    if (D == 32) return delta_launch<__bf16, 32>(B, H, L, out, dout, sb, sh, st, delta, s);
  } else {
    if (D == 128) return delta_launch<float, 128>(B, H, L, out, dout, sb, sh, st, delta, s);
    if (D == 64) return delta_launch<float, 64>(B, H, L, out, dout, sb, sh, st, delta, s);
    if (D == 32) return delta_launch<float, 32>(B, H, L, out, dout, sb, sh, st, delta, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t n4 = (n + 3) / 4;
  const int64_t blocks = (n4 + 255) / 256;
  hipLaunchKernelGGL(fill_kernel, dim3(helper_grid(blocks)), dim3(256), 0, s, p, n, value);
  return hipGetLastError();
}

}  // namespace ra
