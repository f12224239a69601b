// Forward ring step: one query chunk against one KV chunk, tiled online softmax
// with a fused LSE-merge epilogue.
//
// What it computes ("Ring Attention & Friends", "Flash Attention - Tiling with the
// Softmax Rescaling Trick"; Mosaic post, "How Ring Attention Works"): for every query
// row, the softmax-weighted sum of the visible values of this KV chunk, kept as a
// running max m, running sum l and unnormalised output O that are rescaled whenever
// m grows; at the end O/l and LSE = scale*m + ln l are the step's partial result,
// which the epilogue either writes or LSE-merges into an accumulator.
//
// Work decomposition (gfx950, wave64):
//  * one workgroup = 4 or 8 waves = BM = 128 or 256 query rows of one (batch,
//    query head) (8 at head dim 128); each wave owns 32 query rows;
//  * the KV chunk is streamed in tiles of BN keys through double-buffered LDS;
//  * bf16: scores are computed transposed, S^T = K Q^T, with 16x16x32 MFMA tiles;
//    every lane holds two query rows and a quarter of their keys, so the softmax
//    statistics are per-lane and row reductions take two lane exchanges.  P^T
//    (rounded to bf16) is the B operand of the PV MFMA O^T += V^T P^T straight
//    from registers, and V^T comes from LDS transpose loads;
//  * the reference max of the online softmax moves lazily: P is taken against the
//    current reference, and only when a lane's partial row sum of a tile exceeds
//    2^8 does the wave find the exact row max and rescale (so p <= 2^8 always);
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
constexpr int kThreads = 256;  // fp32 kernel and the bf16 kernel below D = 128
constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;

// Waves per bf16 workgroup (32 query rows each).  At D = 128 a workgroup of 8 waves
// (256 rows) shares each K/V tile between twice the rows, which measured 2-6% faster
// than 4 waves on dense sequences; with packed documents the 4-wave workgroup is
// faster (fewer workgroups straddle a document boundary, whose rows then see
// disjoint key ranges), and at D = 32 it is faster too.
template <int D, bool PK>
struct Bf16Cfg {
  static constexpr int NW = (D == 128 && !PK) ? 8 : 4;
  static constexpr int NT = 64 * NW;  // threads
  static constexpr int BM = 32 * NW;  // query rows
};

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

// Row state of the fp32 kernel, whose 32x32 accumulators give every lane one query
// row and the two halves of a wave the same rows.
struct RowState {
  float m;  // running max of raw scores (shared by the two halves of a row)
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

// ------------------------------------------------------------------------- bf16 path
//
// K and V tiles go global -> LDS with direct-to-LDS buffer loads (no staging
// registers): lane i of a load lands at tile + 16 i bytes, so each lane fetches
// the global 16-byte chunk that belongs at its LDS slot, which realises the XOR
// swizzles below.  Rows past the chunk end are outside the buffer resource and
// arrive as zeros.  V stays row-major; the PV operand V^T is read with the LDS
// transpose load (ds_read_b64_tr_b16).

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

template <int D>
struct Bf16Tile {
  static constexpr int KCH = D / 8;                 // 16-byte chunks per row
  static constexpr int RPW = 256 / (D * 2);         // rows per 256-byte bank window
};

// K tile: LDS serves 16 lanes x 16 bytes per clock from 64 four-byte banks, and the
// 16-byte K reads of one clock cover 16 consecutive rows at one chunk; XOR-ing the
// chunk with the row's window index spreads those rows over all 16 bank groups.
template <int D>
__device__ inline int k_swz(int r) { return (r / Bf16Tile<D>::RPW) & (Bf16Tile<D>::KCH - 1); }
// The bf16 kernel uses 16x16x32 MFMA tiles: on this chip a stream of them sustains
// about 15% more FLOP/s than 32x32x16 tiles under the board power limit.
// Accumulator layout of a 16x16 tile: lane l holds column l % 16 and rows
// 4 (l / 16) + r, r = 0..3; operands hold row (A) or column (B) l % 16 and the 8
// contraction indices 8 (l / 16) + j.
//  * S^T = K Q^T per 16-key x 16-query tile: each lane holds two query rows
//    (l % 16 and 16 + l % 16 of the wave's 32) and 4 keys of every 16-key tile; a
//    row's keys are spread over the four 16-lane groups.
//  * P^T feeds O^T += V^T P^T from registers: contraction slot 8 g + j of a 32-key
//    step holds key 4 g + j (j < 4) or 16 + 4 g + j - 4, which is what the
//    accumulators of the step's two key tiles give lane group g; V^T is read with
//    two transpose loads of 4 keys each.

// V tile swizzle for this access: one transpose read serves two 16-lane groups per
// clock, rows 4g..4g+7 at one 32-byte column pair; the chunk XOR puts those 8 rows x
// 2 chunks in 16 distinct bank groups.
template <int D>
__device__ inline int v_swz(int r) {
  if constexpr (Bf16Tile<D>::KCH >= 16) return ((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
  if constexpr (Bf16Tile<D>::KCH == 8) return ((r >> 1) & 3) << 1;
  return ((r >> 2) & 1) << 1;
}

template <int D, int BN, int NT>
__device__ inline void dma_tile(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                  uint32_t row_bytes, int u0, __bf16* ks, __bf16* vs, int wave,
                                  int lane) {
  constexpr int KCH = Bf16Tile<D>::KCH;
  constexpr int SLOTS = BN * KCH;
  constexpr int NI = SLOTS / NT;
  static_assert(SLOTS % NT == 0, "tile must be a whole number of workgroup loads");
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int base = it * NT + wave * 64;
    const int slot = base + lane;
    const int r = slot / KCH, pc = slot % KCH;
    const uint32_t roff = (uint32_t)(u0 + r) * row_bytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void_t*)(ks + base * 8), 16,
                                             roff + (uint32_t)((pc ^ k_swz<D>(r)) * 16), 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void_t*)(vs + base * 8), 16,
                                             roff + (uint32_t)((pc ^ v_swz<D>(r)) * 16), 0, 0, 0);
  }
}

// Max and sum over the four 16-lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48), which
// hold the same query rows.
__device__ inline float quad_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return pair_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ inline float quad_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return pair_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// Epilogue of one query row in the 16x16 layout: o[dt] holds O^T[d][q] for
// d = 16 dt + 4 grp + r.
template <int D>
__device__ inline void fwd_epilogue16(const FwdArgs& a, int b, int h, int tq, int grp, float m,
                                      float l, const f32x4 (&o)[D / 16]) {
  const int L = a.map.L;
  const float l_tot = quad_sum(l);
  const bool live = l_tot > 0.0f;
  const float lse_s = live ? (m * a.scale_log2 + __builtin_amdgcn_logf(l_tot)) * kLn2 : kNegInf;
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
  for (int dt = 0; dt < D / 16; ++dt) {
    const int d0 = dt * 16 + grp * 4;
    f32x4 v = o[dt] * w_s;
    if (acc != nullptr && w_acc != 0.0f) v += *(const f32x4*)(acc + d0) * w_acc;
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
  if (grp == 0) a.lse_out[row] = lse_new;
}

template <int D, int BN, bool PK>
__global__ __launch_bounds__((Bf16Cfg<D, PK>::NT), (Bf16Cfg<D, PK>::NW == 8 ? 1 : 2)) void fwd_bf16_kernel(
    FwdArgs a) {
  constexpr int kBM = Bf16Cfg<D, PK>::BM;
  constexpr int NT = Bf16Cfg<D, PK>::NT;
  constexpr int NKK = D / 32;   // 32-wide head-dim steps of the QK^T contraction
  constexpr int NDT = D / 16;   // 16-row head-dim tiles of O^T
  constexpr int NKT = BN / 16;  // 16-key tiles per KV tile
  constexpr int NC = BN / 32;   // 32-key steps of the PV contraction
  constexpr float kSumCap = 256.0f;  // lazy rescale bound on a lane's partial sum: p <= 2^8
  __shared__ __attribute__((aligned(16))) __bf16 ks0[BN * D];
  __shared__ __attribute__((aligned(16))) __bf16 ks1[BN * D];
  __shared__ __attribute__((aligned(16))) __bf16 vs0[BN * D];
  __shared__ __attribute__((aligned(16))) __bf16 vs1[BN * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, grp = lane >> 4;
  const int L = a.map.L;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qi = logical % a.n_qtiles;
  const int bh = logical / a.n_qtiles;
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int qt = a.n_qtiles - 1 - qi;  // heaviest (latest) query tiles first
  const int t0 = qt * kBM;
  const int tq[2] = {t0 + wave * 32 + l16, t0 + wave * 32 + 16 + l16};
  const int g = h / a.group;

  const __bf16* qb = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const __bf16* kb = (const __bf16*)a.k + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;
  const __bf16* vb = (const __bf16*)a.v + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;
  const uint32_t q_row = (uint32_t)(a.q_st * 2), kv_row = (uint32_t)(a.kv_st * 2);
  const __amdgpu_buffer_rsrc_t qr_ = make_rsrc(qb, (uint32_t)L * q_row);
  const __amdgpu_buffer_rsrc_t kr_ = make_rsrc(kb, (uint32_t)L * kv_row);
  const __amdgpu_buffer_rsrc_t vr_ = make_rsrc(vb, (uint32_t)L * kv_row);

  // The two query rows of this lane as B operands of S^T = K Q^T (rows >= L read 0).
  bf16x8 qr[2][NKK];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qr[x][kk] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                      qr_, (uint32_t)tq[x] * q_row + (uint32_t)(kk * 64 + grp * 16), 0, 0));

  // Visible keys [kv_lo, kv_lim) of each row; key tiles j0..n_tiles-1 hold those of
  // every row, and [full_lo, n_full) is visible to every row (no mask).
  int kv_lo[2] = {0, 0}, kv_lim[2] = {L, L};
  int j0 = 0, n_keys = L, full_lo = 0, n_full = L;
  if constexpr (PK) {
    __shared__ int red[4];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      if (tq[x] < L) {
        key_interval(a.map, a.ck, pos_of(a.map, a.cq, tq[x]), a.causal,
                     a.seg + (int64_t)b * a.seg_n, a.seg_n, kv_lo[x], kv_lim[x]);
      } else {
        kv_lo[x] = L;
        kv_lim[x] = 0;
      }
    }
    int min_lo;
    wg_interval_reduce2(red, kv_lo, kv_lim, L, min_lo, n_keys, full_lo, n_full);
    j0 = min_lo / BN;
  } else if (a.causal) {
    const int t_last = min(t0 + kBM, L) - 1;
#pragma unroll
    for (int x = 0; x < 2; ++x)
      kv_lim[x] = count_le(a.map, a.ck, pos_of(a.map, a.cq, min(tq[x], L - 1)));
    n_keys = count_le(a.map, a.ck, pos_of(a.map, a.cq, t_last));
    n_full = count_le(a.map, a.ck, pos_of(a.map, a.cq, t0));
  }
  const int n_tiles = (n_keys + BN - 1) / BN;

  float m[2] = {kMInit, kMInit}, l[2] = {0.0f, 0.0f};
  f32x4 o[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt][0] = o[dt][1] = f32x4{};

  if (n_tiles > j0) dma_tile<D, BN, NT>(kr_, vr_, kv_row, j0 * BN, ks0, vs0, wave, lane);

  // Transpose-read source of this lane: row l16 / 4 of its group's 4-row block,
  // columns 4 (l16 % 4) of the 16-column tile.
  const int src_row = l16 >> 2;
  const int src_col = (l16 & 3) * 4;

  auto tile = [&](int j, const __bf16* kt, const __bf16* vt, __bf16* kn, __bf16* vn) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile j landed
    __syncthreads();                     // ... and every other wave's; tile j-1 is free
    if (j + 1 < n_tiles) dma_tile<D, BN, NT>(kr_, vr_, kv_row, (j + 1) * BN, kn, vn, wave, lane);
    __builtin_amdgcn_iglp_opt(0);

    f32x4 s[NKT][2];
#pragma unroll
    for (int t = 0; t < NKT; ++t) s[t][0] = s[t][1] = f32x4{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int t = 0; t < NKT; ++t) {
        const int r = t * 16 + l16;
        const bf16x8 kop = *(const bf16x8*)(kt + r * D + (((kk * 4 + grp) ^ k_swz<D>(r)) << 3));
        s[t][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qr[0][kk], s[t][0], 0, 0, 0);
        s[t][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qr[1][kk], s[t][1], 0, 0, 0);
      }

    const int u0 = j * BN;
    if (__builtin_expect(u0 < full_lo || u0 + BN > n_full, 0)) {  // rare: keep it a branch
#pragma unroll
      for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int u = u0 + t * 16 + grp * 4 + r;
            if (u < kv_lo[x] || u >= kv_lim[x]) s[t][x][r] = kNegInf;
          }
    }

    bf16x8 pb[2][NC];
    auto expo = [&](int x) {
      const float mc = m[x] * a.scale_log2;
      float ls[2] = {0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = fast_exp2(__builtin_fmaf(s[t][x][r], a.scale_log2, -mc));
          ls[r & 1] += pv;
          pb[x][t >> 1][(t & 1) * 4 + r] = (__bf16)pv;
        }
      return ls[0] + ls[1];
    };
    // P against the current reference max first; every p is at most its lane's
    // partial row sum, so while the partials stay <= 2^8 the reference may stay.
    // Otherwise (the first visible tile, or a row whose max rose) the wave finds the
    // exact row max, rescales O and l, and takes P again.
    float part[2] = {expo(0), expo(1)};
    if (__builtin_expect(
            __builtin_amdgcn_ballot_w64(!(part[0] <= kSumCap && part[1] <= kSumCap)) != 0, 0)) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        float v = kNegInf;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) v = fmaxf(v, s[t][x][r]);
        const float mx = quad_max(v);
        const bool reset = !(quad_max(part[x]) <= kSumCap);
        const float m_new = reset ? fmaxf(mx, m[x]) : m[x];
        const float alpha = fast_exp2((m[x] - m_new) * a.scale_log2);
        m[x] = m_new;
        l[x] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt][x] *= alpha;
        part[x] = expo(x);
      }
    }
    l[0] += part[0];
    l[1] += part[1];

    // O^T += V^T P^T, one 32-key step at a time.
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 vop[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        s16x4 xv[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int r = c * 32 + half * 16 + grp * 4 + src_row;
          const int col = dt * 16 + src_col;
          const __bf16* ptr = vt + r * D + (((col >> 3) ^ v_swz<D>(r)) << 3) + (col & 7);
          xv[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)ptr);
        }
        vop[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(xv[0], xv[1], 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        o[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[dt], pb[0][c], o[dt][0], 0, 0, 0);
        o[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[dt], pb[1][c], o[dt][1], 0, 0, 0);
      }
    }
  };

  for (int j = j0; j < n_tiles; j += 2) {
    tile(j, ks0, vs0, ks1, vs1);
    if (j + 1 < n_tiles) tile(j + 1, ks1, vs1, ks0, vs0);
  }

#pragma unroll
  for (int x = 0; x < 2; ++x) {
    f32x4 ox[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) ox[dt] = o[dt][x];
    fwd_epilogue16<D>(a, b, h, tq[x], grp, m[x], l[x], ox);
  }
}

// ------------------------------------------------------------------------- fp32 path

template <int D, int BN, bool PK>
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

  // Visible keys of this row and of the workgroup, as in the bf16 kernel.
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
  if (n_tiles > j0) {
    load(j0 * BN);
    store(0);
  }

  for (int j = j0; j < n_tiles; ++j) {
    const int buf = (j - j0) & 1;
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
    if (u0 < full_lo || u0 + BN > n_full) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int u = u0 + blk * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
          if (u < kv_lo || u >= kv_lim) s[blk][i] = kNegInf;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[blk][i]);
    mx = pair_max(mx);
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
hipError_t launch_grid(K kernel, const FwdArgs& a, int threads, hipStream_t s) {
  const int64_t nblk = (int64_t)a.B * a.Hq * a.n_qtiles;
  hipLaunchKernelGGL(kernel, dim3((unsigned)nblk), dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int fwd_block_m(int dtype, int D, bool packed) {
  if (dtype != RA_BF16) return kBM;
  if (packed) return D == 128 ? Bf16Cfg<128, true>::BM : (D == 64 ? Bf16Cfg<64, true>::BM : Bf16Cfg<32, true>::BM);
  return D == 128 ? Bf16Cfg<128, false>::BM : (D == 64 ? Bf16Cfg<64, false>::BM : Bf16Cfg<32, false>::BM);
}

template <bool PK>
hipError_t launch_fwd_t(int dtype, int D, const FwdArgs& a, hipStream_t s) {
  if (dtype == RA_BF16) {
    if (D == 128) return launch_grid(fwd_bf16_kernel<128, 64, PK>, a, Bf16Cfg<128, PK>::NT, s);
    if (D == 64) return launch_grid(fwd_bf16_kernel<64, 64, PK>, a, Bf16Cfg<64, PK>::NT, s);
    if (D == 32) return launch_grid(fwd_bf16_kernel<32, 64, PK>, a, Bf16Cfg<32, PK>::NT, s);
  } else {
    if (D == 128) return launch_grid(fwd_f32_kernel<128, 32, PK>, a, kThreads, s);
    if (D == 64) return launch_grid(fwd_f32_kernel<64, 64, PK>, a, kThreads, s);
    if (D == 32) return launch_grid(fwd_f32_kernel<32, 64, PK>, a, kThreads, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(int dtype, int D, const FwdArgs& a, hipStream_t s) {
  return a.seg != nullptr ? launch_fwd_t<true>(dtype, D, a, s) : launch_fwd_t<false>(dtype, D, a, s);
}

}  // namespace ra
