// Forward ring step for fp32 problems: one query chunk against one KV chunk, tiled
// online softmax with a fused LSE-merge epilogue.
//
// What it computes ("Ring Attention & Friends", "Flash Attention - Tiling with the
// Softmax Rescaling Trick"; Mosaic post, "How Ring Attention Works"): for every query
// row, the softmax-weighted sum of the visible values of this KV chunk, kept as a
// running max m, running sum l and unnormalised output O that are rescaled whenever
// m grows; at the end O/l and LSE = scale*m + ln l are the step's partial result,
// which the epilogue either writes or LSE-merges into an accumulator.
//
// Work decomposition (gfx950, wave64): one workgroup = 4 waves = 128 query rows of
// one (batch, query head), 32 rows per wave.  K and V tiles are staged row-major in
// LDS (rows padded by one float, so column reads are conflict-free) through registers
// (buffer loads, rows past the chunk end reading as zeros), double-buffered.  Scores are computed transposed, S^T = K Q^T, with the fp32
// 32x32x2 MFMA: every lane holds one query row (the two halves of a wave the same
// rows, different keys), and the QK^T contraction stops at the true head dim when
// that leaves a quarter of D as padding.  O^T += V^T P^T takes P^T straight from
// registers, two keys per MFMA.  As in the bf16 kernel, the reference max of the
// online softmax moves lazily: only a tile whose partial row sums exceed 2^8 pays for
// the exact row max and the rescale of O and l.
//
// This file is compiled apart from the bf16 forward because the two want different
// code generation: the default instruction scheduler and MFMA accumulators in VGPRs
// for this kernel, an ILP-oriented scheduler for the bf16 kernel.
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = kFwdF32BlockM;  // 32 rows per wave
static_assert(kBM == 32 * (kThreads / 64), "one 32-row MFMA tile per wave");


// Row state of the fp32 kernel, whose 32x32 accumulators give every lane one query
// row and the two halves of a wave the same rows.
struct RowState {
  float m;  // reference max of raw scores, at most the row max so far (shared by the
            // two halves of a row); it moves lazily, so exp2((s - m) * scale_log2) <= 2^8
  float l;  // running sum of exp2((s - m) * scale_log2) over this lane's keys
};

// Epilogue of the fp32 kernel: normalise, optionally LSE-merge, store.
// o_t[n] holds O^T[d][q] for d = dblk*32 + (i/4)*8 + hh*4 + i%4 with n = dblk*16 + i.
template <int D>
__device__ inline void fwd_epilogue(const FwdArgs& a, int b, int h, int tq, int hh,
                                    const RowState& st, f32x16 (&o_t)[D / 32]) {
  const int L = a.map.L;
  const float l_tot = pair_sum(st.l);
  const bool live = l_tot > 0.0f;
  const float lse_s = live ? (st.m * a.scale_log2 + __builtin_amdgcn_logf(l_tot)) * kLn2 : kNegInf;
  const float inv_l = live ? 1.0f / l_tot : 0.0f;
  if (tq >= L) return;
  const int64_t row = ((int64_t)b * a.Hq + h) * L + tq;
  float w_acc = 0.0f, w_s = inv_l, lse_new = lse_s;
  if (a.acc_in != nullptr) {
    const float lse_a = a.lse_in[row];
    if (!live) {
      w_acc = 1.0f;
      w_s = 0.0f;
      lse_new = lse_a;
    } else if (lse_a == kNegInf) {
      w_acc = 0.0f;
    } else {
      const float mx = fmaxf(lse_a, lse_s);
      const float ea = __expf(lse_a - mx), es = __expf(lse_s - mx);
      const float den = ea + es;
      lse_new = mx + __logf(den);
      w_acc = ea / den;
      w_s = es / den * inv_l;
    }
  }
  const float* acc = a.acc_in ? a.acc_in + row * D : nullptr;
  char* obase = (char*)a.out;
  const int64_t orow = (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)tq * a.o_st;
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = dblk * 32 + g * 8 + hh * 4;
      f32x4 v;
      v[0] = o_t[dblk][g * 4 + 0] * w_s;
      v[1] = o_t[dblk][g * 4 + 1] * w_s;
      v[2] = o_t[dblk][g * 4 + 2] * w_s;
      v[3] = o_t[dblk][g * 4 + 3] * w_s;
      if (acc != nullptr && w_acc != 0.0f) {
        const f32x4 av = *(const f32x4*)(acc + d0);
        v[0] += av[0] * w_acc;
        v[1] += av[1] * w_acc;
        v[2] += av[2] * w_acc;
        v[3] += av[3] * w_acc;
      }
      if (a.out_f32) {
        *(f32x4*)(obase + (orow + d0) * 4) = v;
      } else {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 w;
        w[0] = (__bf16)v[0];
        w[1] = (__bf16)v[1];
        w[2] = (__bf16)v[2];
        w[3] = (__bf16)v[3];
        *(bf16x4*)(obase + (orow + d0) * 2) = w;
      }
    }
  }
  if (hh == 0) a.lse_out[row] = lse_new;
}

// KP: column pairs of the QK^T contraction, D / 2, or 3 D / 8 when the true head dim
// is at most 3 D / 4 (the remaining columns are zero padding).
// Workgroups per CU the register allocation must allow: 4 at D = 32 (at most 128
// VGPRs; it measured 1% faster than at 3 per CU), else 2.
template <int D, int BN, bool PK, int KP>
__global__ __launch_bounds__(kThreads, D == 32 ? 4 : 2) void fwd_f32_kernel(FwdArgs a) {
  constexpr int DP = D + 1;            // padded LDS row (conflict-free column reads)
  constexpr int NB = BN / 32;
  constexpr int ND = D / 32;
  constexpr int NCH = BN * D / 4;      // float4 chunks per tile
  constexpr int NL = (NCH + kThreads - 1) / kThreads;
  __shared__ float kf[2][BN * DP];
  __shared__ float vf[2][BN * DP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int L = a.map.L;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qi = logical % a.n_qtiles;
  const int bh = logical / a.n_qtiles;
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int qt = a.n_qtiles - 1 - qi;
  const int t0 = qt * kBM;
  const int tq = t0 + wave * 32 + l32;
  const int g = h / a.group;

  const float* qb = (const float*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const float* kb = (const float*)a.k + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;
  const float* vb = (const float*)a.v + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;

  static_assert(KP == D / 2 || KP == 3 * D / 8, "full or three-quarter contraction");
  float qf[KP];
#pragma unroll
  for (int kk = 0; kk < KP; ++kk) qf[kk] = tq < L ? qb[(int64_t)tq * a.q_st + kk * 2 + hh] : 0.0f;

  // Visible keys [kv_lo, kv_lim) of this row; key tiles j0..n_tiles-1 hold those of
  // every row of the workgroup, and [full_lo, n_full) is visible to every row (no mask).
  int kv_lo = 0, kv_lim = L, j0 = 0, n_keys = L, full_lo = 0, n_full = L;
  if constexpr (PK) {
    __shared__ int red[4];
    if (tq < L) {
      key_interval(a.map, a.ck, pos_of(a.map, a.cq, tq), a.causal, a.seg + (int64_t)b * a.seg_n,
                   a.seg_n, kv_lo, kv_lim);
    } else {
      kv_lo = L;
      kv_lim = 0;
    }
    int min_lo;
    wg_interval_reduce(red, kv_lo, kv_lim, L, min_lo, n_keys, full_lo, n_full);
    j0 = min_lo / BN;
  } else if (a.causal) {
    const int t_last = min(t0 + kBM, L) - 1;
    kv_lim = count_le(a.map, a.ck, pos_of(a.map, a.cq, min(tq, L - 1)));
    n_keys = count_le(a.map, a.ck, pos_of(a.map, a.cq, t_last));
    n_full = count_le(a.map, a.ck, pos_of(a.map, a.cq, t0));
  }
  const int n_tiles = (n_keys + BN - 1) / BN;  // key tiles j0 .. n_tiles-1

  RowState st{kMInit, 0.0f};
  f32x16 o_t[ND];
#pragma unroll
  for (int n = 0; n < ND; ++n) o_t[n] = f32x16{};

  // K and V rows through buffer resources sized to the head's L rows: a row past the
  // chunk end reads as zeros (the host keeps L + 256 rows of bytes below 4 GiB, so the
  // 32-bit offsets of the last tile do not wrap).
  static_assert(NCH % kThreads == 0, "whole loads per thread");
  const uint32_t row_bytes = (uint32_t)(a.kv_st * 4);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(kb, (uint32_t)L * row_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vb, (uint32_t)L * row_bytes);
  // Thread tid moves 16-byte chunk tid % CPR of row tid / CPR of each RPI-row block: a
  // per-lane offset plus a wave-uniform one (the tile's and the block's first row).  The
  // whole offset goes in the VGPR operand, which the buffer bounds check always covers
  // (whether it also covers the SGPR offset is not something to rely on), so rows past
  // the chunk end read as zeros.
  constexpr int CPR = D / 4;            // float4 chunks per row
  constexpr int RPI = kThreads / CPR;   // rows per load instruction of the workgroup
  static_assert(kThreads % CPR == 0, "whole rows per load instruction");
  const uint32_t ld_lane = (uint32_t)(tid / CPR) * row_bytes + (uint32_t)(tid % CPR) * 16u;
  const int st_lane = (tid / CPR) * DP + (tid % CPR) * 4;
  f32x4 sk[NL], sv[NL];
  auto load = [&](int u0) {
#pragma unroll
    for (int it = 0; it < NL; ++it) {
      const uint32_t off = ld_lane + (uint32_t)(u0 + it * RPI) * row_bytes;
      sk[it] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
      sv[it] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0));
    }
  };
  auto store = [&](int buf) {
    float* kd = &kf[buf][st_lane];
    float* vd = &vf[buf][st_lane];
#pragma unroll
    for (int it = 0; it < NL; ++it)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kd[it * RPI * DP + e] = sk[it][e];
        vd[it * RPI * DP + e] = sv[it][e];
      }
  };
  if (n_tiles > j0) {
    load(j0 * BN);
    store(0);
  }

  for (int j = j0; j < n_tiles; ++j) {
    const int buf = (j - j0) & 1;
    __syncthreads();
    if (j + 1 < n_tiles) load((j + 1) * BN);

    // The contraction covers KP column pairs: the zero pad columns beyond the true
    // head dim add nothing (at d = 24 stored as 32: 12 MFMAs instead of 16).
    // Each lane's LDS reads are a per-lane base plus compile-time offsets: K row
    // blk * 32 + l32 at column kk * 2 + hh, V row blk * 32 + (i / 4) * 8 + hh * 4 + i % 4
    // at column n * 32 + l32.
    const float* krd = &kf[buf][l32 * DP + hh];
    const float* vrd = &vf[buf][hh * 4 * DP + l32];
    f32x16 s[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < KP; ++kk) {
        const float kop = krd[blk * 32 * DP + kk * 2];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kop, qf[kk], acc, 0, 0, 0);
      }
      s[blk] = acc;
    }
    const int u0 = j * BN;
    if (u0 < full_lo || u0 + BN > n_full) {
      // visible iff kv_lo <= u < kv_lim: one unsigned compare of u - kv_lo
      const uint32_t width = (uint32_t)max(kv_lim - kv_lo, 0);
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int u = u0 + blk * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
          if ((uint32_t)(u - kv_lo) >= width) s[blk][i] = kNegInf;
        }
    }
    f32x16 p[NB];
    auto expo = [&]() {
      const float mc = st.m * a.scale_log2;
      float ls[2] = {0.0f, 0.0f};
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = fast_exp2(__builtin_fmaf(s[blk][i], a.scale_log2, -mc));
          ls[i & 1] += pv;
          p[blk][i] = pv;
        }
      return ls[0] + ls[1];
    };
    // P against the current reference max first; every p is at most its lane's
    // partial row sum, so while the partials of a row stay <= 2^8 the reference may
    // stay.  Otherwise (the first visible tile, or a row whose max rose) the wave
    // finds the exact row max, rescales O and l, and takes P again.
    float part = expo();
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(part <= kSumCap)) != 0, 0)) {
      float v = kNegInf;
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) v = fmaxf(v, s[blk][i]);
      const float mx = pair_max(v);
      const bool reset = !(pair_max(part) <= kSumCap);
      const float m_new = reset ? fmaxf(mx, st.m) : st.m;
      const float alpha = fast_exp2((st.m - m_new) * a.scale_log2);
      st.m = m_new;
      st.l *= alpha;
#pragma unroll
      for (int n = 0; n < ND; ++n) o_t[n] *= alpha;
      part = expo();
    }
    st.l += part;

    // O^T += V^T P^T with K = 2 per MFMA: step i pairs the keys the two halves of
    // the wave hold in accumulator slot i.
#pragma unroll
    for (int n = 0; n < ND; ++n)
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float vop = vrd[(blk * 32 + (i >> 2) * 8 + (i & 3)) * DP + n * 32];
          o_t[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(vop, p[blk][i], o_t[n], 0, 0, 0);
        }

    if (j + 1 < n_tiles) store(buf ^ 1);
  }

  fwd_epilogue<D>(a, b, h, tq, hh, st, o_t);
}

template <int D, int BN, bool PK, int KP>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  const int64_t nblk = (int64_t)a.B * a.Hq * a.n_qtiles;
  hipLaunchKernelGGL((fwd_f32_kernel<D, BN, PK, KP>), dim3((unsigned)nblk), dim3(kThreads), 0,
                     s, a);
  return hipGetLastError();
}

template <bool PK>
hipError_t launch_t(int D, int dk, const FwdArgs& a, hipStream_t s) {
  const bool part = 4 * dk <= 3 * D;  // true head dim within the first 3/4 of the columns
  if (D == 128) return part ? launch<128, 32, PK, 48>(a, s) : launch<128, 32, PK, 64>(a, s);
  if (D == 64) return part ? launch<64, 64, PK, 24>(a, s) : launch<64, 64, PK, 32>(a, s);
  if (D == 32) return part ? launch<32, 64, PK, 12>(a, s) : launch<32, 64, PK, 16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_f32(int D, int dk, bool packed, const FwdArgs& a, hipStream_t s) {
  return packed ? launch_t<true>(D, dk, a, s) : launch_t<false>(D, dk, a, s);
}

}  // namespace ra
