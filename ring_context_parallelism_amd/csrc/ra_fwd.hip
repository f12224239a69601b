// Forward ring step: one query chunk against one KV chunk, tiled online softmax
// with an fused LSE-merge epilogue.
//
// What it computes ("Ring Attention & Friends", "Flash Attention - Tiling with the
// Softmax Rescaling Trick"; Mosaic post, "How Ring Attention Works"): for every query
// row, the softmax-weighted sum of the visible values of this KV chunk, kept as a
// running max m, running sum l and unnormalised output O that are rescaled whenever
// m grows; at the end O/l and LSE = scale*m + ln l are the step's partial result,
// which the epilogue either writes or LSE-merges into an accumulator.
//
// Work decomposition (gfx950, wave64):
//  * one workgroup = 4 waves = BM = 128 query rows of one (batch, query head);
//    each wave owns 32 query rows;
//  * the KV chunk is streamed in tiles of BN keys through double-buffered LDS;
//  * scores are computed transposed, S^T = K Q^T, with 32x32 MFMA tiles, so that in
//    the accumulator layout every lane holds one query row (column l % 32) and
//    half of that row's keys; the other half sits in lane l ^ 32.  The softmax
//    statistics are therefore per-lane scalars and a row max needs one exchange;
//  * P^T (rounded to bf16) is used directly from registers as the B operand of the
//    PV MFMA O^T += V^T P^T; V is written transposed into LDS with a key permutation
//    that matches the accumulator's key order, so each lane's 8 keys are one 16-byte
//    LDS read;
//  * fp32 problems use the fp32 32x32x2 MFMA with K and V row-major in LDS.
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMInit = -1.0e30f;  // finite start for the running max (no inf - inf)
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;

__device__ inline float partner(float x) { return __shfl_xor(x, 32, 64); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup id -> logical work item.  Workgroups are dispatched round-robin over the
// 8 XCDs, so give every XCD one contiguous range of logical ids: the query tiles of
// one head then share that XCD's L2 for their K/V reads.
__device__ inline int xcd_remap(int bid, int nblk) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = (nblk + 7) >> 3, rem = nblk & 7;
  if (rem == 0 || xcd < rem) return xcd * per + slot;
  return rem * per + (xcd - rem) * (per - 1) + slot;
}

struct RowState {
  float m;  // running max of raw scores (shared by the two halves of a row)
  float l;  // running sum of exp2((s - m) * scale_log2) over this lane's keys
};

// Epilogue shared by both dtypes: normalise, optionally LSE-merge, store.
// o_t[n] holds O^T[d][q] for d = dblk*32 + (i/4)*8 + hh*4 + i%4 with n = dblk*16 + i.
template <int D>
__device__ inline void fwd_epilogue(const FwdArgs& a, int b, int h, int tq, int hh,
                                    const RowState& st, f32x16 (&o_t)[D / 32]) {
  const int L = a.map.L;
  const float l_tot = st.l + partner(st.l);
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

// ------------------------------------------------------------------------- bf16 path

template <int D, int BN>
struct Bf16Tile {
  static constexpr int KCH = D / 8;                                     // 16B chunks per K row
  static constexpr int KSW = (KCH < 8 ? KCH : 8) - 1;                   // K swizzle mask
  static constexpr int VCH = BN / 8;                                    // 16B chunks per Vt row
  static constexpr int VSW = (VCH < 8 ? VCH : 8) - 1;                   // Vt swizzle mask
  static constexpr int NK = (BN * KCH + kThreads - 1) / kThreads;       // K chunks per thread
  static constexpr int NVG = (BN / 4) * KCH;                            // 4-key x 8-d V groups
  static constexpr int NV = (NVG + kThreads - 1) / kThreads;            // V groups per thread
};

// Offset (elements) of 16B chunk `c` of K row `r` in the swizzled K tile.
template <int D, int BN>
__device__ inline int k_off(int r, int c) {
  return r * D + ((c ^ (r & Bf16Tile<D, BN>::KSW)) << 3);
}
// Offset (elements) of chunk `c` of Vt row `d` (head-dim index) in the swizzled tile.
template <int D, int BN>
__device__ inline int vt_off(int d, int c) {
  return d * BN + ((c ^ ((d ^ (d >> 3)) & Bf16Tile<D, BN>::VSW)) << 3);
}
// Key permutation inside a Vt row: swap bits 2 and 3 of the key index.
__device__ inline int vt_col(int key) {
  return (key & ~0xC) | ((key >> 1) & 0x4) | ((key << 1) & 0x8);
}

template <int D, int BN>
struct Bf16Stage {
  uint4 k[Bf16Tile<D, BN>::NK];
  uint4 v[Bf16Tile<D, BN>::NV][4];
};

template <int D, int BN>
__device__ inline void bf16_load(Bf16Stage<D, BN>& st, const __bf16* kb, const __bf16* vb,
                                 int64_t kv_st, int u0, int L, int tid) {
  using T = Bf16Tile<D, BN>;
#pragma unroll
  for (int it = 0; it < T::NK; ++it) {
    const int ci = it * kThreads + tid;
    const int r = ci / T::KCH, c = ci % T::KCH;
    const int u = u0 + r;
    uint4 z = {0u, 0u, 0u, 0u};
    if (ci < BN * T::KCH && u < L) z = *(const uint4*)(kb + (int64_t)u * kv_st + c * 8);
    st.k[it] = z;
  }
#pragma unroll
  for (int it = 0; it < T::NV; ++it) {
    const int gi = it * kThreads + tid;
    const int kg = gi / T::KCH, dg = gi % T::KCH;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int u = u0 + kg * 4 + r;
      uint4 z = {0u, 0u, 0u, 0u};
      if (gi < T::NVG && u < L) z = *(const uint4*)(vb + (int64_t)u * kv_st + dg * 8);
      st.v[it][r] = z;
    }
  }
}

__device__ inline uint32_t half_of(const uint4& w, int e) {
  const uint32_t word = e < 2 ? w.x : (e < 4 ? w.y : (e < 6 ? w.z : w.w));
  return (e & 1) ? (word >> 16) : (word & 0xFFFFu);
}

template <int D, int BN>
__device__ inline void bf16_store(const Bf16Stage<D, BN>& st, __bf16* ks, __bf16* vts, int tid) {
  using T = Bf16Tile<D, BN>;
#pragma unroll
  for (int it = 0; it < T::NK; ++it) {
    const int ci = it * kThreads + tid;
    const int r = ci / T::KCH, c = ci % T::KCH;
    if (ci < BN * T::KCH) *(uint4*)(ks + k_off<D, BN>(r, c)) = st.k[it];
  }
#pragma unroll
  for (int it = 0; it < T::NV; ++it) {
    const int gi = it * kThreads + tid;
    if (gi < T::NVG) {
      const int kg = gi / T::KCH, dg = gi % T::KCH;
      const int col = vt_col(kg * 4);
      const int cchunk = col >> 3, within = col & 7;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = dg * 8 + e;
        uint2 w;
        w.x = half_of(st.v[it][0], e) | (half_of(st.v[it][1], e) << 16);
        w.y = half_of(st.v[it][2], e) | (half_of(st.v[it][3], e) << 16);
        *(uint2*)(vts + vt_off<D, BN>(d, cchunk) + within) = w;
      }
    }
  }
}

template <int D, int BN>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(FwdArgs a) {
  using T = Bf16Tile<D, BN>;
  constexpr int NKB = D / 16;  // 16-wide head-dim blocks of the QK^T contraction
  constexpr int ND = D / 32;   // 32-row head-dim blocks of O^T
  constexpr int NB = BN / 32;  // 32-key blocks per tile
  __shared__ __attribute__((aligned(16))) __bf16 ks[2][BN * D];
  __shared__ __attribute__((aligned(16))) __bf16 vts[2][D * BN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int L = a.map.L;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qi = logical % a.n_qtiles;
  const int bh = logical / a.n_qtiles;
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int qt = a.n_qtiles - 1 - qi;  // heaviest (latest) query tiles first
  const int t0 = qt * kBM;
  const int tq = t0 + wave * 32 + l32;
  const int g = h / a.group;

  const __bf16* qb = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const __bf16* kb = (const __bf16*)a.k + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;
  const __bf16* vb = (const __bf16*)a.v + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;

  // This lane's query row as the B operand of S^T = K Q^T.
  bf16x8 qr[NKB];
#pragma unroll
  for (int kk = 0; kk < NKB; ++kk) {
    bf16x8 z = {};
    if (tq < L) z = *(const bf16x8*)(qb + (int64_t)tq * a.q_st + kk * 16 + hh * 8);
    qr[kk] = z;
  }

  // Visible-key prefix of this row, and of the whole tile.
  const int t_last = min(t0 + kBM, L) - 1;
  int kv_lim = L, n_keys = L, n_full = L;
  if (a.causal) {
    kv_lim = count_le(a.map, a.ck, pos_of(a.map, a.cq, min(tq, L - 1)));
    n_keys = count_le(a.map, a.ck, pos_of(a.map, a.cq, t_last));
    n_full = count_le(a.map, a.ck, pos_of(a.map, a.cq, t0));
  }
  const int n_tiles = (n_keys + BN - 1) / BN;

  RowState st{kMInit, 0.0f};
  f32x16 o_t[ND];
#pragma unroll
  for (int n = 0; n < ND; ++n) o_t[n] = f32x16{};

  Bf16Stage<D, BN> stage;
  if (n_tiles > 0) {
    bf16_load<D, BN>(stage, kb, vb, a.kv_st, 0, L, tid);
    bf16_store<D, BN>(stage, ks[0], vts[0], tid);
  }

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    __syncthreads();
    if (j + 1 < n_tiles) bf16_load<D, BN>(stage, kb, vb, a.kv_st, (j + 1) * BN, L, tid);

    // S^T for this tile: NB blocks of 32 keys x 32 queries.
    f32x16 s[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
        const bf16x8 kop = *(const bf16x8*)(&ks[buf][k_off<D, BN>(blk * 32 + l32, kk * 2 + hh)]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qr[kk], acc, 0, 0, 0);
      }
      s[blk] = acc;
    }

    // Mask keys beyond this row's visible prefix (causal diagonal, ragged tail).
    const int u0 = j * BN;
    if (u0 + BN > n_full) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int u = u0 + blk * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
          if (u >= kv_lim) s[blk][i] = kNegInf;
        }
    }

    // Online softmax update.
    float mx = s[0][0];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[blk][i]);
    mx = fmaxf(mx, partner(mx));
    const float m_new = fmaxf(st.m, mx);
    const float alpha = fast_exp2((st.m - m_new) * a.scale_log2);
    st.m = m_new;
    const float mc = m_new * a.scale_log2;
    float lsum = 0.0f;
    bf16x8 pb[NB][2];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(__builtin_fmaf(s[blk][i], a.scale_log2, -mc));
        lsum += pv;
        pb[blk][i >> 3][i & 7] = (__bf16)pv;
      }
    st.l = st.l * alpha + lsum;
#pragma unroll
    for (int n = 0; n < ND; ++n) o_t[n] *= alpha;

    // O^T += V^T P^T.
#pragma unroll
    for (int n = 0; n < ND; ++n)
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const bf16x8 vop =
              *(const bf16x8*)(&vts[buf][vt_off<D, BN>(n * 32 + l32, blk * 4 + mm * 2 + hh)]);
          o_t[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[blk][mm], o_t[n], 0, 0, 0);
        }

    if (j + 1 < n_tiles) bf16_store<D, BN>(stage, ks[buf ^ 1], vts[buf ^ 1], tid);
  }

  fwd_epilogue<D>(a, b, h, tq, hh, st, o_t);
}

// ------------------------------------------------------------------------- fp32 path

template <int D, int BN>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdArgs a) {
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

  float qf[D / 2];
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) qf[kk] = tq < L ? qb[(int64_t)tq * a.q_st + kk * 2 + hh] : 0.0f;

  const int t_last = min(t0 + kBM, L) - 1;
  int kv_lim = L, n_keys = L, n_full = L;
  if (a.causal) {
    kv_lim = count_le(a.map, a.ck, pos_of(a.map, a.cq, min(tq, L - 1)));
    n_keys = count_le(a.map, a.ck, pos_of(a.map, a.cq, t_last));
    n_full = count_le(a.map, a.ck, pos_of(a.map, a.cq, t0));
  }
  const int n_tiles = (n_keys + BN - 1) / BN;

  RowState st{kMInit, 0.0f};
  f32x16 o_t[ND];
#pragma unroll
  for (int n = 0; n < ND; ++n) o_t[n] = f32x16{};

  f32x4 sk[NL], sv[NL];
  auto load = [&](int u0) {
#pragma unroll
    for (int it = 0; it < NL; ++it) {
      const int ci = it * kThreads + tid;
      const int r = ci / (D / 4), c = ci % (D / 4);
      const int u = u0 + r;
      f32x4 zk = {}, zv = {};
      if (ci < NCH && u < L) {
        zk = *(const f32x4*)(kb + (int64_t)u * a.kv_st + c * 4);
        zv = *(const f32x4*)(vb + (int64_t)u * a.kv_st + c * 4);
      }
      sk[it] = zk;
      sv[it] = zv;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int it = 0; it < NL; ++it) {
      const int ci = it * kThreads + tid;
      const int r = ci / (D / 4), c = ci % (D / 4);
      if (ci < NCH) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[buf][r * DP + c * 4 + e] = sk[it][e];
          vf[buf][r * DP + c * 4 + e] = sv[it][e];
        }
      }
    }
  };
  if (n_tiles > 0) {
    load(0);
    store(0);
  }

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    __syncthreads();
    if (j + 1 < n_tiles) load((j + 1) * BN);

    f32x16 s[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < D / 2; ++kk) {
        const float kop = kf[buf][(blk * 32 + l32) * DP + kk * 2 + hh];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kop, qf[kk], acc, 0, 0, 0);
      }
      s[blk] = acc;
    }
    const int u0 = j * BN;
    if (u0 + BN > n_full) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int u = u0 + blk * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
          if (u >= kv_lim) s[blk][i] = kNegInf;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[blk][i]);
    mx = fmaxf(mx, partner(mx));
    const float m_new = fmaxf(st.m, mx);
    const float alpha = fast_exp2((st.m - m_new) * a.scale_log2);
    st.m = m_new;
    const float mc = m_new * a.scale_log2;
    float lsum = 0.0f;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(__builtin_fmaf(s[blk][i], a.scale_log2, -mc));
        lsum += pv;
        s[blk][i] = pv;
      }
    st.l = st.l * alpha + lsum;
#pragma unroll
    for (int n = 0; n < ND; ++n) o_t[n] *= alpha;

    // O^T += V^T P^T with K = 2 per MFMA: step i pairs the keys the two halves of
    // the wave hold in accumulator slot i.
#pragma unroll
    for (int n = 0; n < ND; ++n)
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = blk * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
          const float vop = vf[buf][key * DP + n * 32 + l32];
          o_t[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(vop, s[blk][i], o_t[n], 0, 0, 0);
        }

    if (j + 1 < n_tiles) store(buf ^ 1);
  }

  fwd_epilogue<D>(a, b, h, tq, hh, st, o_t);
}

template <typename K>
hipError_t launch_grid(K kernel, const FwdArgs& a, hipStream_t s) {
  const int64_t nblk = (int64_t)a.B * a.Hq * a.n_qtiles;
  hipLaunchKernelGGL(kernel, dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int fwd_block_m(int /*dtype*/, int /*D*/) { return kBM; }

hipError_t launch_fwd(int dtype, int D, const FwdArgs& a, hipStream_t s) {
  if (dtype == RA_BF16) {
    if (D == 128) return launch_grid(fwd_bf16_kernel<128, 64>, a, s);
    if (D == 64) return launch_grid(fwd_bf16_kernel<64, 64>, a, s);
    if (D == 32) return launch_grid(fwd_bf16_kernel<32, 64>, a, s);
  } else {
    if (D == 128) return launch_grid(fwd_f32_kernel<128, 32>, a, s);
    if (D == 64) return launch_grid(fwd_f32_kernel<64, 64>, a, s);
    if (D == 32) return launch_grid(fwd_f32_kernel<32, 64>, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ra
