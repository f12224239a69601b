// Backward ring step: recompute P from the final LSE and produce dQ, dK, dV.
//
// What it computes (ringmaster page, "Status": flash-style reverse-ring backward):
// for the query rows of chunk cq and the keys of chunk ck,
//   P = exp(S*scale - LSE),  dV += P^T dO,  dP = dO V^T,  dS = P o (dP - delta),
//   dK += scale dS^T Q,      dQ += scale dS K,
// with dK, dV of a KV head summed over the query heads of its GQA group.
//
// Work decomposition (gfx950, wave64, 32x32x16 bf16 MFMA):
//  * one workgroup = 4 waves = 128 keys of one (batch, KV head); each wave owns 32
//    keys, keeps their K and V rows in registers and accumulates dK^T and dV^T for
//    them across every query head of the group and every visible query tile;
//  * query tiles of 32 rows stream through double-buffered LDS, each stored both
//    row-major (A operand of S = Q K^T and dP = dO V^T) and transposed with the
//    accumulator's row permutation (A operand of dK^T = Q^T dS and dV^T = dO^T P);
//  * scores are computed as S[q][key]: every lane holds one key and 16 query rows,
//    so P and dS feed the dK/dV MFMAs straight from registers;
//  * dS is exchanged through LDS (bf16, [q][key]) for dQ = dS K, which the four
//    waves split by head-dim block / key range and add to global dQ with fp32
//    atomics (several workgroups contribute to one query row);
//  * causal: only query tiles that see at least one of the workgroup's keys are
//    visited; the element mask runs only on tiles that straddle the diagonal.
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBN = 128;   // keys per workgroup
constexpr int kBMq = 32;   // query rows per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDsStride = kBN + 8;  // padded dS row (bank-conflict free)

__device__ inline int xcd_remap(int bid, int nblk) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = (nblk + 7) >> 3, rem = nblk & 7;
  if (rem == 0 || xcd < rem) return xcd * per + slot;
  return rem * per + (xcd - rem) * (per - 1) + slot;
}

// Swap bits 2 and 3 of a row index: the order in which the 32x32 accumulator holds
// rows, used as the column order of the transposed query tiles.
__device__ inline int perm_col(int r) { return (r & ~0xC) | ((r >> 1) & 0x4) | ((r << 1) & 0x8); }

template <int D>
struct BwdTile {
  static constexpr int KCH = D / 8;                     // 16B chunks per row-major row
  static constexpr int KSW = (KCH < 8 ? KCH : 8) - 1;   // row-major swizzle mask
  static constexpr int NG = (kBMq / 4) * KCH;           // 4-row x 8-col groups per tensor
  static constexpr int NKG = (kBN / 4) * KCH;           // groups of the K^T tile
};

// Row-major [rows][D] tile: offset of 16B chunk c of row r.
template <int D>
__device__ inline int rm_off(int r, int c) {
  return r * D + ((c ^ (r & BwdTile<D>::KSW)) << 3);
}
// Transposed query tile [D][32]: offset of chunk c (of 4) of row d.
__device__ inline int qt_off(int d, int c) { return d * kBMq + ((c ^ ((d >> 1) & 3)) << 3); }
// Transposed key tile [D][128]: offset of chunk c (of 16) of row d.
__device__ inline int kt_off(int d, int c) { return d * kBN + ((c ^ ((d ^ (d >> 3)) & 7)) << 3); }

__device__ inline uint32_t half_of(const uint4& w, int e) {
  const uint32_t word = e < 2 ? w.x : (e < 4 ? w.y : (e < 6 ? w.z : w.w));
  return (e & 1) ? (word >> 16) : (word & 0xFFFFu);
}

template <int D>
struct QStage {
  uint4 rows[4];  // 4 consecutive query rows x 8 head-dim columns (Q or dO)
  float lse2, delta;
};

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_bf16_kernel(BwdArgs a) {
  using T = BwdTile<D>;
  constexpr int NKB = D / 16;   // 16-wide head-dim blocks (S and dP contractions)
  constexpr int NDB = D / 32;   // 32-row head-dim blocks (dK^T, dV^T, dQ)
  constexpr int WPD = 4 / NDB;  // waves sharing one dQ head-dim block
  constexpr int KSTEPS = kBN / 16 / WPD;

  __shared__ __attribute__((aligned(16))) __bf16 s_q[2][kBMq * D];
  __shared__ __attribute__((aligned(16))) __bf16 s_do[2][kBMq * D];
  __shared__ __attribute__((aligned(16))) __bf16 s_qt[2][D * kBMq];
  __shared__ __attribute__((aligned(16))) __bf16 s_dot[2][D * kBMq];
  __shared__ __attribute__((aligned(16))) __bf16 s_kt[D * kBN];
  __shared__ __attribute__((aligned(16))) __bf16 s_ds[kBMq * kDsStride];
  __shared__ __attribute__((aligned(16))) float s_lse2[2][kBMq];
  __shared__ __attribute__((aligned(16))) float s_delta[2][kBMq];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int L = a.map.L;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = logical % a.n_ktiles;
  const int bg = logical / a.n_ktiles;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int u0 = kt * kBN;
  const int key = u0 + wave * 32 + l32;  // this lane's key
  const bool key_ok = key < L;

  const __bf16* kb = (const __bf16*)a.k + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;
  const __bf16* vb = (const __bf16*)a.v + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;

  // This lane's K and V rows as B operands (S = Q K^T, dP = dO V^T).
  bf16x8 kreg[NKB], vreg[NKB];
#pragma unroll
  for (int kk = 0; kk < NKB; ++kk) {
    bf16x8 zk = {}, zv = {};
    if (key_ok) {
      zk = *(const bf16x8*)(kb + (int64_t)key * a.kv_st + kk * 16 + hh * 8);
      zv = *(const bf16x8*)(vb + (int64_t)key * a.kv_st + kk * 16 + hh * 8);
    }
    kreg[kk] = zk;
    vreg[kk] = zv;
  }
  // K^T of the workgroup's keys for dQ = dS K (B operand, k = key).
  for (int gi = tid; gi < T::NKG; gi += kThreads) {
    const int kg = gi % (kBN / 4), dg = gi / (kBN / 4);
    uint4 r4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int u = u0 + kg * 4 + r;
      uint4 z = {0u, 0u, 0u, 0u};
      if (u < L) z = *(const uint4*)(kb + (int64_t)u * a.kv_st + dg * 8);
      r4[r] = z;
    }
    const int col = kg * 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint2 w;
      w.x = half_of(r4[0], e) | (half_of(r4[1], e) << 16);
      w.y = half_of(r4[2], e) | (half_of(r4[3], e) << 16);
      *(uint2*)(s_kt + kt_off(dg * 8 + e, col >> 3) + (col & 7)) = w;
    }
  }

  // Visible query range of this key tile.  Query t sees key u iff
  // pos(cq, t) >= pos(ck, u), i.e. t >= count_le(cq, pos(ck, u) - 1).
  int t_first = 0, t_mask_hi = 0, t_min_lane = 0;
  const int u_last = min(u0 + kBN, L) - 1;
  if (a.causal) {
    t_first = count_le(a.map, a.cq, pos_of(a.map, a.ck, u0) - 1);
    t_mask_hi = count_le(a.map, a.cq, pos_of(a.map, a.ck, u_last) - 1);
    t_min_lane = key_ok ? count_le(a.map, a.cq, pos_of(a.map, a.ck, key) - 1) : L;
  } else {
    t_min_lane = key_ok ? 0 : L;
  }
  if (u0 + kBN > L) t_mask_hi = L;  // ragged key tile: always mask
  const int qt_first = t_first / kBMq;
  const int n_qt = (L + kBMq - 1) / kBMq;
  const int per_head = n_qt - qt_first;
  const int n_iter = per_head > 0 ? per_head * a.group : 0;

  f32x16 dv_t[NDB], dk_t[NDB];
#pragma unroll
  for (int n = 0; n < NDB; ++n) {
    dv_t[n] = f32x16{};
    dk_t[n] = f32x16{};
  }

  // Staging of one query tile: threads [0, NG) load Q, [NG, 2 NG) load dO, and
  // threads [0, 32) also load the tile's LSE and delta rows.
  QStage<D> st;
  auto tile_of = [&](int it, int& h, int& t0) {
    h = g * a.group + it / per_head;
    t0 = (qt_first + it % per_head) * kBMq;
  };
  auto load = [&](int it) {
    int h, t0;
    tile_of(it, h, t0);
    if (tid < 2 * T::NG) {
      const bool is_do = tid >= T::NG;
      const int gi = is_do ? tid - T::NG : tid;
      const int qg = gi % (kBMq / 4), dg = gi / (kBMq / 4);
      const __bf16* base;
      int64_t st_t;
      if (is_do) {
        base = (const __bf16*)a.dout + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh;
        st_t = a.o_st;
      } else {
        base = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
        st_t = a.q_st;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + qg * 4 + r;
        uint4 z = {0u, 0u, 0u, 0u};
        if (t < L) z = *(const uint4*)(base + (int64_t)t * st_t + dg * 8);
        st.rows[r] = z;
      }
    }
    if (tid < kBMq) {
      const int r = tid;
      const int t = t0 + r;
      const int64_t row = ((int64_t)b * a.Hq + h) * L + t;
      // Rows past the chunk end get P = exp2(-inf) = 0 through an infinite LSE.
      st.lse2 = t < L ? a.lse[row] * kLog2e : __builtin_huge_valf();
      st.delta = t < L ? a.delta[row] : 0.0f;
    }
  };
  auto store = [&](int buf) {
    if (tid < 2 * T::NG) {
      const bool is_do = tid >= T::NG;
      const int gi = is_do ? tid - T::NG : tid;
      const int qg = gi % (kBMq / 4), dg = gi / (kBMq / 4);
      __bf16* rm = is_do ? s_do[buf] : s_q[buf];
      __bf16* tr = is_do ? s_dot[buf] : s_qt[buf];
#pragma unroll
      for (int r = 0; r < 4; ++r) *(uint4*)(rm + rm_off<D>(qg * 4 + r, dg)) = st.rows[r];
      const int col = perm_col(qg * 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 w;
        w.x = half_of(st.rows[0], e) | (half_of(st.rows[1], e) << 16);
        w.y = half_of(st.rows[2], e) | (half_of(st.rows[3], e) << 16);
        *(uint2*)(tr + qt_off(dg * 8 + e, col >> 3) + (col & 7)) = w;
      }
    }
    if (tid < kBMq) {
      const int r = tid;
      s_lse2[buf][r] = st.lse2;
      s_delta[buf][r] = st.delta;
    }
  };

  if (n_iter > 0) {
    load(0);
    store(0);
  }

  const int dq_blk = wave / WPD;
  const int dq_k0 = (wave % WPD) * KSTEPS;

  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    int h, t0;
    tile_of(it, h, t0);
    __syncthreads();  // tile `it` staged; every wave is done with s_ds of it-1
    if (it + 1 < n_iter) load(it + 1);

    // S[q][key] and dP[q][key] for this wave's 32 keys.
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      const bf16x8 qa = *(const bf16x8*)(&s_q[buf][rm_off<D>(l32, kk * 2 + hh)]);
      const bf16x8 da = *(const bf16x8*)(&s_do[buf][rm_off<D>(l32, kk * 2 + hh)]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kreg[kk], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vreg[kk], dp, 0, 0, 0);
    }

    // P = exp2(S * scale_log2 - LSE * log2 e); dS = P (dP - delta).
    const bool need_mask = t0 < t_mask_hi;
    bf16x8 pb[2], dsb[2];
    float dsv[16];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const f32x4 l4 = *(const f32x4*)(&s_lse2[buf][gq * 8 + hh * 4]);
      const f32x4 d4 = *(const f32x4*)(&s_delta[buf][gq * 8 + hh * 4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = gq * 4 + e;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], a.scale_log2, -l4[e]));
        if (need_mask && t0 + gq * 8 + hh * 4 + e < t_min_lane) p = 0.0f;
        const float ds = p * (dp[i] - d4[e]);
        pb[i >> 3][i & 7] = (__bf16)p;
        dsb[i >> 3][i & 7] = (__bf16)ds;
        dsv[i] = ds;
      }
    }

    // dV^T += dO^T P and dK^T += Q^T dS (k = query rows, in accumulator order).
#pragma unroll
    for (int n = 0; n < NDB; ++n)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const bf16x8 doa = *(const bf16x8*)(&s_dot[buf][qt_off(n * 32 + l32, mm * 2 + hh)]);
        const bf16x8 qta = *(const bf16x8*)(&s_qt[buf][qt_off(n * 32 + l32, mm * 2 + hh)]);
        dv_t[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(doa, pb[mm], dv_t[n], 0, 0, 0);
        dk_t[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qta, dsb[mm], dk_t[n], 0, 0, 0);
      }

    // dS to LDS as [q][key] for the dQ contraction.
    {
      __bf16* row = s_ds + wave * 32 + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = (i >> 2) * 8 + hh * 4 + (i & 3);
        row[q * kDsStride] = (__bf16)dsv[i];
      }
    }
    __syncthreads();

    // dQ[q][d] += scale * sum_key dS[q][key] K[key][d] over this wave's share.
    {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int k0 = (dq_k0 + ks) * 16;
        const bf16x8 dsa = *(const bf16x8*)(&s_ds[l32 * kDsStride + k0 + hh * 8]);
        const bf16x8 ktb = *(const bf16x8*)(&s_kt[kt_off(dq_blk * 32 + l32, (k0 >> 3) + hh)]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsa, ktb, acc, 0, 0, 0);
      }
      float* dqb = a.dq + (((int64_t)b * a.Hq + h) * L) * D + dq_blk * 32 + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = t0 + (i >> 2) * 8 + hh * 4 + (i & 3);
        if (t < L) atomicAdd(dqb + (int64_t)t * D, acc[i] * a.scale);
      }
    }

    if (it + 1 < n_iter) store(buf ^ 1);
  }

  // dK, dV of this lane's key: accumulator rows are head-dim indices
  // d = n*32 + (i/4)*8 + hh*4 + i%4.
  if (key_ok && n_iter > 0) {
    const int64_t row = (((int64_t)b * a.Hkv + g) * L + key) * D;
#pragma unroll
    for (int n = 0; n < NDB; ++n)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = n * 32 + gq * 8 + hh * 4;
        f32x4* pk = (f32x4*)(a.dk + row + d0);
        f32x4* pv = (f32x4*)(a.dv + row + d0);
        f32x4 ck = *pk, cv = *pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ck[e] += dk_t[n][gq * 4 + e] * a.scale;
          cv[e] += dv_t[n][gq * 4 + e];
        }
        *pk = ck;
        *pv = cv;
      }
  }
}

template <int D>
hipError_t launch(const BwdArgs& a, hipStream_t s) {
  const int64_t nblk = (int64_t)a.B * a.Hkv * a.n_ktiles;
  hipLaunchKernelGGL(bwd_bf16_kernel<D>, dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int bwd_block_n(int /*dtype*/, int /*D*/) { return kBN; }

hipError_t launch_bwd(int dtype, int D, const BwdArgs& a, hipStream_t s) {
  if (dtype != RA_BF16) return hipErrorNotSupported;
  if (D == 128) return launch<128>(a, s);
  if (D == 64) return launch<64>(a, s);
  if (D == 32) return launch<32>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace ra
