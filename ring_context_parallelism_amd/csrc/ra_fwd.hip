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
//  * one workgroup = 4 or 8 waves = 128 or 256 query rows of one (batch, query
//    head) (8 at head dim 128), or, with GQA groups of 4 or more at head dim 128, 64
//    rows of each of 4 query heads that read one KV head; each wave owns 32 rows;
//  * the KV chunk is streamed in tiles of BN keys through double-buffered LDS;
//  * bf16: scores are computed transposed, S^T = K Q^T, with 16x16x32 MFMA tiles;
//    every lane holds two query rows and a quarter of their keys, so the softmax
//    statistics are per-lane and row reductions take two lane exchanges.  P^T
//    (rounded to bf16) is the B operand of the PV MFMA O^T += V^T P^T straight
//    from registers, and V^T comes from LDS transpose loads;
//  * the reference max of the online softmax moves lazily: P is taken against the
//    current reference, and only when a lane's partial row sum of a tile exceeds
//    2^8 does the wave find the exact row max and rescale (so p <= 2^8 always);
//  * fp32 problems go to ra_fwd_f32.hip (the fp32 32x32x2 MFMA), which is compiled
//    with the default instruction scheduler.
#include "ra_internal.h"

namespace ra {
namespace {

// Waves per bf16 workgroup (32 query rows each).  At D = 128 a workgroup of 8 waves
// (256 rows) shares each K/V tile between twice the rows, which measured 2-6% faster
// than 4 waves on dense sequences; with packed documents the 4-wave workgroup is
// faster (fewer workgroups straddle a document boundary, whose rows then see
// disjoint key ranges), and at D = 32 it is faster too.
//
// HG query heads of one GQA group share a workgroup (HG = 4 at D = 128 when the group
// allows it): 64 rows of each of 4 heads instead of 256 rows of one.  Each K/V tile
// still serves 256 query rows, but the workgroup's causal diagonal is 4x narrower, so
// fewer of its MFMAs fall above the diagonal and fewer of its tiles need a mask.
template <int D, bool PK, int HG = 1>
struct Bf16Cfg {
  static constexpr int NW = (D == 128 && !PK) ? 8 : 4;
  static constexpr int NT = 64 * NW;  // threads
  static constexpr int WPH = NW / HG;  // waves per query head
  static constexpr int BM = 32 * WPH;  // query rows per head
  static_assert(NW % HG == 0, "whole waves per head");
};


// ------------------------------------------------------------------------- bf16 path
//
// K and V tiles go global -> LDS with direct-to-LDS buffer loads (no staging
// registers): lane i of a load lands at tile + 16 i bytes, so each lane fetches
// the global 16-byte chunk that belongs at its LDS slot, which realises the XOR
// swizzles below.  Rows past the chunk end are outside the buffer resource and
// arrive as zeros.  V stays row-major; the PV operand V^T is read with the LDS
// transpose load (ds_read_b64_tr_b16).



template <int D>
struct Bf16Tile {
  static constexpr int KCH = D / 8;                 // 16-byte chunks per row
  static constexpr int RPW = 256 / (D * 2);         // rows per 256-byte bank window
};

// K tile (16-byte row reads only): a row-read pass serves the 16 lanes that agree in
// lane-id bits 0 and 5 (the LDS pass structure measured on this chip; the backward's
// pair tile describes it), here 8 keys of one parity at one chunk pair.  XOR-ing the chunk with the
// row's window index puts them in 16 distinct bank groups at D = 128; at D = 64 and 32,
// where a 256-byte window holds 2 or 4 rows, the rows of one parity share half of the
// groups and the reads take two passes.  A pair tile (one pass both ways at every D)
// measured 0.2-1.2% slower at D = 128 and 0.3% faster at D = 32, where the kernel is
// bound by its softmax VALU work, so the XOR tiles stay.
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

// Epilogue of the lane's two query rows in the 16x16 layout: o[dt][x] holds O^T[d][q]
// for d = 16 dt + 4 grp + r.  Every load (the accumulator rows and their LSE) is
// issued before the first store: the output may alias the accumulator, so a load
// behind a store would have to wait for it.
template <int D>
__device__ inline void fwd_epilogue16(const FwdArgs& a, int b, int h, const int (&tq)[2], int grp,
                                      const float (&m)[2], const float (&l)[2],
                                      const f32x4 (&o)[D / 16][2]) {
  constexpr int NDT = D / 16;
  const int L = a.map.L;
  float lse_s[2], inv_l[2];
  bool live[2], in[2];
  int64_t row[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const float l_tot = quad_sum(l[x]);
    live[x] = l_tot > 0.0f;
    lse_s[x] = live[x] ? (m[x] * a.scale_log2 + __builtin_amdgcn_logf(l_tot)) * kLn2 : kNegInf;
    inv_l[x] = live[x] ? 1.0f / l_tot : 0.0f;
    in[x] = tq[x] < L;
    row[x] = ((int64_t)b * a.Hq + h) * L + min(tq[x], L - 1);
  }
  float lse_a[2] = {kNegInf, kNegInf};
  f32x4 acc[2][NDT];
  if (a.acc_in != nullptr) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      if (!in[x]) continue;
      lse_a[x] = a.lse_in[row[x]];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        acc[x][dt] = *(const f32x4*)(a.acc_in + row[x] * D + dt * 16 + grp * 4);
    }
  }
  char* obase = (char*)a.out;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    if (!in[x]) continue;
    float w_acc = 0.0f, w_s = inv_l[x], lse_new = lse_s[x];
    if (a.acc_in != nullptr) {
      if (!live[x]) {
        w_acc = 1.0f;
        w_s = 0.0f;
        lse_new = lse_a[x];
      } else if (lse_a[x] != kNegInf) {
        const float mx = fmaxf(lse_a[x], lse_s[x]);
        const float ea = __expf(lse_a[x] - mx), es = __expf(lse_s[x] - mx);
        const float den = ea + es;
        lse_new = mx + __logf(den);
        w_acc = ea / den;
        w_s = es / den * inv_l[x];
      }
    }
    const int64_t orow = (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)tq[x] * a.o_st;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d0 = dt * 16 + grp * 4;
      f32x4 v = o[dt][x] * w_s;
      if (w_acc != 0.0f) v += acc[x][dt] * w_acc;
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
    if (grp == 0) a.lse_out[row[x]] = lse_new;
  }
}

template <int D, int BN, bool PK, int HG>
__global__ __launch_bounds__((Bf16Cfg<D, PK, HG>::NT), (Bf16Cfg<D, PK, HG>::NW == 8 ? 1 : 2)) void fwd_bf16_kernel(
    FwdArgs a) {
  constexpr int kBM = Bf16Cfg<D, PK, HG>::BM;
  constexpr int NT = Bf16Cfg<D, PK, HG>::NT;
  constexpr int WPH = Bf16Cfg<D, PK, HG>::WPH;
  constexpr int NKK = D / 32;   // 32-wide head-dim steps of the QK^T contraction
  constexpr int NDT = D / 16;   // 16-row head-dim tiles of O^T
  constexpr int NKT = BN / 16;  // 16-key tiles per KV tile
  constexpr int NC = BN / 32;   // 32-key steps of the PV contraction
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
  const int bh = logical / a.n_qtiles;  // (batch, group of HG query heads)
  const int hgn = a.Hq / HG;
  const int h0 = (bh % hgn) * HG, b = bh / hgn;
  const int h = h0 + wave / WPH;        // this wave's query head
  const int qt = a.n_qtiles - 1 - qi;  // heaviest (latest) query tiles first
  const int t0 = qt * kBM;
  const int wr = (wave % WPH) * 32;     // this wave's rows within the head's tile
  const int tq[2] = {t0 + wr + l16, t0 + wr + 16 + l16};
  const int g = h0 / a.group;           // HG divides the group: one KV head

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
      // Key u = u0 + 16 t + 4 grp + r is visible to row x iff kv_lo <= u < kv_lim: one
      // unsigned compare of u - kv_lo with the interval's width (u < kv_lo wraps to a
      // large value).  Two signed compares per key left 64 lane masks live at once,
      // which the compiler spilled to VGPR lanes.
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int base = u0 + grp * 4 - kv_lo[x];
        const uint32_t width = (uint32_t)max(kv_lim[x] - kv_lo[x], 0);
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if ((uint32_t)(base + t * 16 + r) >= width) s[t][x][r] = kNegInf;
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

  fwd_epilogue16<D>(a, b, h, tq, grp, m, l, o);
}

template <typename K>
hipError_t launch_grid(K kernel, const FwdArgs& a, int threads, hipStream_t s, int hg = 1) {
  const int64_t nblk = (int64_t)a.B * (a.Hq / hg) * a.n_qtiles;
  hipLaunchKernelGGL(kernel, dim3((unsigned)nblk), dim3(threads), 0, s, a);
  return hipGetLastError();
}

// Query heads per bf16 workgroup: 4 at D = 128 on dense sequences when the GQA group
// is a multiple of 4, else 1.
int fwd_heads_per_wg(int dtype, int D, bool packed, int group) {
  return (dtype == RA_BF16 && D == 128 && !packed && group % 4 == 0) ? 4 : 1;
}

}  // namespace

int fwd_block_m(int dtype, int D, bool packed, int group) {
  if (dtype != RA_BF16) return kFwdF32BlockM;
  if (packed) return D == 128 ? Bf16Cfg<128, true>::BM : (D == 64 ? Bf16Cfg<64, true>::BM : Bf16Cfg<32, true>::BM);
  if (fwd_heads_per_wg(dtype, D, packed, group) == 4) return Bf16Cfg<128, false, 4>::BM;
  return D == 128 ? Bf16Cfg<128, false>::BM : (D == 64 ? Bf16Cfg<64, false>::BM : Bf16Cfg<32, false>::BM);
}

template <bool PK>
hipError_t launch_fwd_t(int dtype, int D, int dk, const FwdArgs& a, hipStream_t s) {
  if (dtype == RA_BF16) {
    if (fwd_heads_per_wg(dtype, D, PK, a.group) == 4)
      return launch_grid(fwd_bf16_kernel<128, 64, false, 4>, a, Bf16Cfg<128, false, 4>::NT, s, 4);
    if (D == 128) return launch_grid(fwd_bf16_kernel<128, 64, PK, 1>, a, Bf16Cfg<128, PK>::NT, s);
    if (D == 64) return launch_grid(fwd_bf16_kernel<64, 64, PK, 1>, a, Bf16Cfg<64, PK>::NT, s);
    if (D == 32) return launch_grid(fwd_bf16_kernel<32, 64, PK, 1>, a, Bf16Cfg<32, PK>::NT, s);
  } else {
    return launch_fwd_f32(D, dk, PK, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(int dtype, int D, int dk, const FwdArgs& a, hipStream_t s) {
  return a.seg != nullptr ? launch_fwd_t<true>(dtype, D, dk, a, s)
                          : launch_fwd_t<false>(dtype, D, dk, a, s);
}

}  // namespace ra
