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
//    keys and accumulates dK^T and dV^T for them (in the accumulation registers)
//    across every query head of the group and every visible query tile; the
//    workgroup's K and V tiles stay in LDS for the whole launch;
//  * query tiles of 32 rows (Q, dO, LSE, delta) are fetched with direct-to-LDS
//    buffer loads into double-buffered LDS, stored once, row-major, with a swizzle
//    that is bank-conflict free both for 16-byte row reads (A operands of
//    S = Q K^T and dP = dO V^T) and for the LDS transpose reads that give Q^T and
//    dO^T (A operands of dK^T = Q^T dS and dV^T = dO^T P);
//  * scores are computed as S[q][key]: every lane holds one key and 16 query rows,
//    so P and dS feed the dK/dV MFMAs straight from registers;
//  * dS^T goes to LDS (bf16) and dQ = dS K is computed with transpose reads of dS^T
//    and of the workgroup's K tile; the four waves split dQ by head-dim block / key
//    range and add it to global dQ with fp32 atomics;
//  * rows past the chunk end read as zeros (Q = dO = delta = 0 gives dS = 0);
//    causal: only query tiles that see one of the workgroup's keys are visited and
//    the element mask runs only on tiles that straddle the diagonal.
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int kThreads = 256;
constexpr int kBN = 128;   // keys per workgroup
constexpr int kBMq = 32;   // query rows per tile
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline int xcd_remap(int bid, int nblk) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = (nblk + 7) >> 3, rem = nblk & 7;
  if (rem == 0 || xcd < rem) return xcd * per + slot;
  return rem * per + (xcd - rem) * (per - 1) + slot;
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Padded row-major tiles.  LDS serves 16 lanes x 16 bytes per clock from 64 banks;
// a row stride of 3 or 13 (mod 16) sixteen-byte chunks makes both access patterns
// of these tiles conflict free -- 16-byte reads of 16 consecutive rows at one
// column (MFMA row operands) and transpose reads of 4 consecutive rows x 32 bytes
// (MFMA transposed operands) -- and, unlike an XOR swizzle, keeps every address a
// per-lane base plus a compile-time offset.
template <int COLS>
struct Pad {
  static constexpr int CH = COLS / 8;  // data chunks per row
  static constexpr int SCH = CH <= 3 ? 3 : (CH <= 13 ? 13 : (CH <= 19 ? 19 : 29));
  static constexpr int PS = SCH * 8;   // row stride in elements
  // 16-byte slots of a ROWS-row tile, rounded up to whole wave loads
  static constexpr int slots(int rows) { return ((rows * SCH + 63) / 64) * 64; }
};

// Transpose read of a padded bf16 tile: lane j of each 16-lane group receives 4
// consecutive rows at one column; `p` is this lane's own source slot.
__device__ inline s16x4 tr_read(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
}

__device__ inline bf16x8 cat(s16x4 a, s16x4 b) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Direct-to-LDS loads of rows r0..r0+ROWS-1 (COLS bf16 each) into a padded tile.
// Pad slots, rows past ROWS and rows past the resource end are loaded as zeros.
template <int ROWS, int COLS>
__device__ inline void dma_rows(__amdgpu_buffer_rsrc_t rs, uint32_t row_bytes, int r0,
                                __bf16* tile, int wave, int lane) {
  using P = Pad<COLS>;
  constexpr int SLOTS = P::slots(ROWS);
#pragma unroll
  for (int it = 0; it < (SLOTS + kThreads - 1) / kThreads; ++it) {
    const int base = it * kThreads + wave * 64;
    if (SLOTS % kThreads != 0 && base >= SLOTS) break;  // wave-uniform
    const int slot = base + lane;
    const int r = slot / P::SCH, c = slot % P::SCH;
    const uint32_t off = (c < P::CH && r < ROWS) ? (uint32_t)(r0 + r) * row_bytes + (uint32_t)c * 16u
                                                 : 0xFFFFFFF0u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + base * 8), 16, off, 0, 0, 0);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_bf16_kernel(BwdArgs a) {
  constexpr int NKB = D / 16;   // 16-wide head-dim blocks (S and dP contractions)
  constexpr int NDB = D / 32;   // 32-row head-dim blocks (dK^T, dV^T, dQ)
  constexpr int WPD = 4 / NDB;  // waves sharing one dQ head-dim block
  constexpr int KSTEPS = kBN / 16 / WPD;

  using PD = Pad<D>;      // Q, dO, K, V tiles
  using PT = Pad<kBMq>;   // dS^T tile
  constexpr int PS = PD::PS, PST = PT::PS;
  constexpr int QEL = PD::slots(kBMq) * 8, KEL = PD::slots(kBN) * 8, TEL = PT::slots(kBN) * 8;

  // Distinct LDS objects for the two buffers of each tensor (see the forward).
  __shared__ __attribute__((aligned(16))) __bf16 q0[QEL];
  __shared__ __attribute__((aligned(16))) __bf16 q1[QEL];
  __shared__ __attribute__((aligned(16))) __bf16 do0[QEL];
  __shared__ __attribute__((aligned(16))) __bf16 do1[QEL];
  __shared__ __attribute__((aligned(16))) float ls0[64];  // LSE rows (upper half unused)
  __shared__ __attribute__((aligned(16))) float ls1[64];
  __shared__ __attribute__((aligned(16))) float dl0[64];  // delta rows
  __shared__ __attribute__((aligned(16))) float dl1[64];
  __shared__ __attribute__((aligned(16))) __bf16 s_k[KEL];    // K tile
  __shared__ __attribute__((aligned(16))) __bf16 s_v[KEL];    // V tile
  __shared__ __attribute__((aligned(16))) __bf16 s_dst[TEL];  // dS^T [key][q]

  // An (empty) statement that names an AGPR marks the kernel as using AGPRs, so the
  // MFMAs take their accumulator form: dK^T / dV^T then live in AGPRs and the VGPRs
  // stay free for operands instead of holding spilled copies.
  asm volatile("" ::: "a255");

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
  const uint32_t kv_row = (uint32_t)(a.kv_st * 2);
  const __amdgpu_buffer_rsrc_t kr_ = make_rsrc(kb, (uint32_t)L * kv_row);
  const __amdgpu_buffer_rsrc_t vr_ = make_rsrc(vb, (uint32_t)L * kv_row);

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

  // Query-tile order, rotated per key tile: workgroups of neighbouring key tiles
  // would otherwise walk the same query tiles in lockstep and contend for the same
  // dQ rows in their atomic adds.
  const int rot = per_head > 0 ? (kt * 5) % per_head : 0;
  auto tile_of = [&](int it, int& h, int& t0) {
    h = g * a.group + it / per_head;
    int qi = it % per_head + rot;
    if (qi >= per_head) qi -= per_head;
    t0 = (qt_first + qi) * kBMq;
  };
  // Direct-to-LDS loads of query tile `it`: Q and dO rows, LSE and delta.
  auto dma_q = [&](int it, __bf16* qn, __bf16* don, float* lsn, float* dln) {
    int h, t0;
    tile_of(it, h, t0);
    const __bf16* qb = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
    const __bf16* ob = (const __bf16*)a.dout + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh;
    const uint32_t q_row = (uint32_t)(a.q_st * 2), o_row = (uint32_t)(a.o_st * 2);
    dma_rows<kBMq, D>(make_rsrc(qb, (uint32_t)L * q_row), q_row, t0, qn, wave, lane);
    dma_rows<kBMq, D>(make_rsrc(ob, (uint32_t)L * o_row), o_row, t0, don, wave, lane);
    if (wave < 2) {
      const float* src = (wave == 0 ? a.lse : a.delta) + ((int64_t)b * a.Hq + h) * L;
      // lanes >= 32 (and rows >= L) fall outside the resource and write zeros
      const uint32_t off = lane < 32 ? (uint32_t)(t0 + lane) * 4u : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(src, (uint32_t)L * 4u),
                                               (lds_void_t*)(wave == 0 ? lsn : dln), 4, off,
                                               0, 0, 0);
    }
  };

  // Transpose-read source slot of this lane (see tr_read).
  const int src_row = (lane & 15) >> 2;
  const int src_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  const int dq_blk = wave / WPD;
  const int dq_k0 = (wave % WPD) * KSTEPS;

  auto step = [&](int it, const __bf16* qt, const __bf16* dot, const float* ls,
                  const float* dl, __bf16* qn, __bf16* don, float* lsn, float* dln) {
    int h, t0;
    tile_of(it, h, t0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile `it`
    __syncthreads();                     // every wave's loads; tile it-1 and dS^T free
    if (it + 1 < n_iter) dma_q(it + 1, qn, don, lsn, dln);

    // S[q][key] and dP[q][key] for this wave's 32 keys.
    f32x16 s = {}, dp = {};
    const int krow = wave * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      const int col = kk * 16 + hh * 8;
      const bf16x8 qa = *(const bf16x8*)(qt + l32 * PS + col);
      const bf16x8 da = *(const bf16x8*)(dot + l32 * PS + col);
      const bf16x8 kbv = *(const bf16x8*)(s_k + krow * PS + col);
      const bf16x8 vbv = *(const bf16x8*)(s_v + krow * PS + col);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kbv, s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vbv, dp, 0, 0, 0);
    }

    __builtin_amdgcn_sched_barrier(0);
    // P = exp2(S * scale_log2 - LSE * log2 e); dS = P (dP - delta).  Accumulator
    // slot i holds query row gq*8 + hh*4 + e with i = gq*4 + e.
    const bool need_mask = t0 < t_mask_hi;
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const f32x4 l4 = *(const f32x4*)(ls + gq * 8 + hh * 4);
      const f32x4 d4 = *(const f32x4*)(dl + gq * 8 + hh * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = gq * 4 + e;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], a.scale_log2, -l4[e] * kLog2e));
        if (need_mask && t0 + gq * 8 + hh * 4 + e < t_min_lane) p = 0.0f;
        const float ds = p * (dp[i] - d4[e]);
        pb[i >> 3][i & 7] = (__bf16)p;
        dsb[i >> 3][i & 7] = (__bf16)ds;
      }
    }

    __builtin_amdgcn_sched_barrier(0);
    // dV^T += dO^T P and dK^T += Q^T dS.  The A operands hold query rows
    // mm*16 + {0..3, 8..11} + 4 hh (the accumulator order), read transposed.
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int n = 0; n < NDB; ++n) {
        const int o = (mm * 16 + hh * 4 + src_row) * PS + n * 32 + src_col;
        const bf16x8 doa = cat(tr_read(dot + o), tr_read(dot + o + 8 * PS));
        const bf16x8 qta = cat(tr_read(qt + o), tr_read(qt + o + 8 * PS));
        dv_t[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(doa, pb[mm], dv_t[n], 0, 0, 0);
        dk_t[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qta, dsb[mm], dk_t[n], 0, 0, 0);
      }

    __builtin_amdgcn_sched_barrier(0);
    // dS^T[key][q] to LDS: this lane's 16 query rows are 4 runs of 4 consecutive
    // rows, i.e. 32-bit word pairs of the packed dS vectors (whole words are
    // stored, no 16-bit element shuffling).
    {
      const u32x4 w0 = __builtin_bit_cast(u32x4, dsb[0]);
      const u32x4 w1 = __builtin_bit_cast(u32x4, dsb[1]);
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      __bf16* row = s_dst + krow * PST + hh * 4;
      *(u32x2*)(row + 0) = u32x2{w0[0], w0[1]};
      *(u32x2*)(row + 8) = u32x2{w0[2], w0[3]};
      *(u32x2*)(row + 16) = u32x2{w1[0], w1[1]};
      *(u32x2*)(row + 24) = u32x2{w1[2], w1[3]};
    }
    __syncthreads();

    // dQ[q][d] += scale * sum_key dS[q][key] K[key][d] over this wave's share.
    {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int k0 = (dq_k0 + ks) * 16 + hh * 8 + src_row;
        const __bf16* pd = s_dst + k0 * PST + src_col;
        const __bf16* pk = s_k + k0 * PS + dq_blk * 32 + src_col;
        const bf16x8 dsa = cat(tr_read(pd), tr_read(pd + 4 * PST));
        const bf16x8 kbv = cat(tr_read(pk), tr_read(pk + 4 * PS));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsa, kbv, acc, 0, 0, 0);
      }
      // Rows past the chunk end fall outside the resource and are dropped.
      const __amdgpu_buffer_rsrc_t dqr =
          make_rsrc(a.dq + (((int64_t)b * a.Hq + h) * L) * D, (uint32_t)L * D * 4u);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = t0 + (i >> 2) * 8 + hh * 4 + (i & 3);
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
            acc[i] * a.scale, dqr, (uint32_t)(t * D + dq_blk * 32 + l32) * 4u, 0, 0);
      }
    }
  };

  // Pins the dK^T / dV^T accumulators to the accumulation registers at the step
  // boundaries, so both unrolled steps keep them in the same place.
  auto pin = [&]() {
#pragma unroll
    for (int n = 0; n < NDB; ++n) asm volatile("" : "+a"(dk_t[n]), "+a"(dv_t[n]));
  };

  if (n_iter > 0) {
    // The workgroup's K and V tiles: B operands of S = Q K^T, dP = dO V^T (row
    // reads) and of dQ = dS K (transpose reads).
    dma_rows<kBN, D>(kr_, kv_row, u0, s_k, wave, lane);
    dma_rows<kBN, D>(vr_, kv_row, u0, s_v, wave, lane);
    dma_q(0, q0, do0, ls0, dl0);
  }
  for (int it = 0; it < n_iter; it += 2) {
    pin();
    step(it, q0, do0, ls0, dl0, q1, do1, ls1, dl1);
    pin();
    if (it + 1 < n_iter) step(it + 1, q1, do1, ls1, dl1, q0, do0, ls0, dl0);
  }
  pin();

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
