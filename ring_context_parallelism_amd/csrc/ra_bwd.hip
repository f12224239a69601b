// Backward ring step: recompute P from the final LSE and produce dQ, dK, dV.
//
// What it computes (ringmaster page, "Status": flash-style reverse-ring backward):
// for the query rows of chunk cq and the keys of chunk ck,
//   P = exp(S*scale - LSE),  dV += P^T dO,  dP = dO V^T,  dS = P o (dP - delta),
//   dK += scale dS^T Q,      dQ += scale dS K,
// with dK, dV of a KV head summed over the query heads of its GQA group.
//
// Two kernels, neither of which uses atomics (every output element has exactly
// one writer, so the result is deterministic):
//
//  * dK/dV kernel -- one workgroup = 4 waves = 128 keys of one (batch, KV head);
//    each wave owns 32 keys and walks every 32-row query tile that sees them.
//    Scores are computed as S[q][key] on 16x16x32 MFMA tiles (every lane holds two
//    keys and 8 query rows), so P and dS feed dV^T = dO^T P and dK^T = Q^T dS
//    straight from registers.  Each lane's K rows stay in registers and V in LDS;
//    query tiles (Q, dO) stream through double-buffered LDS, and LSE and delta reach
//    LDS through registers, pre-scaled.  Two workgroups per CU, so the two waves
//    sharing a SIMD belong to different workgroups and their barriers do not keep
//    them in step.
//
//  * dQ kernel -- the forward's shape: one workgroup = 8 waves = 256 query rows of
//    one (batch, query head) (4 waves = 128 rows with packed documents at D = 128),
//    KV tiles of 32 keys streamed through double-buffered LDS (each tile serves all
//    of the workgroup's rows).  Scores are computed transposed,
//    S^T = K Q^T, on 16x16x32 MFMA tiles, so every lane holds two query rows; the
//    dP^T accumulators start at -delta, and dS^T = P^T o (dP^T - delta) feeds
//    dQ^T += K^T dS^T from registers, with K^T read by LDS transpose loads.
//
// The dQ kernel recomputes S and dP (7 MFMA passes in all instead of 5); in
// exchange no dS exchange, no cross-workgroup reduction and no atomics remain.
#include "ra_internal.h"

namespace ra {
namespace {

__device__ inline bf16x8 load_row8(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}

__device__ inline s16x4 tr_read(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
}

__device__ inline bf16x8 cat(s16x4 a, s16x4 b) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ----------------------------------------------------------------------- LDS tiles
//
// Pair tile: the LDS layout of the tiles read both ways, by the 16-byte row reads and
// by the transpose reads of 16x16x32 MFMA operands.
//
// LDS passes on this chip (probe kernels under the bank-conflict counter; this pass
// structure is the one that fits every layout measured): a 16-byte read serves, per
// pass, the 16 lanes that agree in bits 0 and 5 of the lane id (the even or the odd
// lanes of one half-wave), and a transpose read serves one half-wave.  A pass takes
// one clock when its bytes fall in distinct banks.
//
// Each 256-byte line of the pair tile holds chunks 2j and 2j + 1 (16 bytes each) of
// the 8 rows of one octet o = m / 8, and row m's two chunks sit in bank groups
// 2 pi(m) and 2 pi(m) + 1 with pi(m) = (m mod 8) xor (o mod 2):
//   slot(m, c) = 16 (CH (m / 16) + (CH / 2) (o mod 2) + c / 2) + 2 pi(m) + c mod 2.
// A row-read pass (8 rows of one parity, one chunk pair) then has distinct pi over its
// rows, and a transpose pass (the rows of one octet, one chunk pair) covers the
// octet's 16 groups: both take one pass.  Four chunks further on, a row read is two
// lines further; two chunks further on, a transpose read is one line further, and 16
// rows further on a read is 16 COLS elements further, so every address is a per-lane base
// plus a compile-time offset.  Every 16 rows fill exactly CH lines (no padding): a
// 32-row tile at D = 128 is two 1 KB direct-to-LDS loads per wave of a 4-wave workgroup.
template <int COLS>
__host__ __device__ constexpr int pair_slot(int m, int c) {
  return 16 * ((COLS / 8) * (m >> 4) + (COLS / 16) * ((m >> 3) & 1) + (c >> 1)) +
         2 * ((m & 7) ^ ((m >> 3) & 1)) + (c & 1);
}
// The inverse: the row and chunk stored in a slot.
template <int COLS>
__host__ __device__ constexpr int pair_row(int slot) {
  constexpr int CH = COLS / 8;
  const int line = slot >> 4, o = (line % CH) / (CH / 2);
  return 16 * (line / CH) + 8 * o + (((slot & 15) >> 1) ^ o);
}
template <int COLS>
__host__ __device__ constexpr int pair_chunk(int slot) {
  constexpr int CH = COLS / 8;
  return 2 * ((slot >> 4) % CH % (CH / 2)) + (slot & 1);
}
// Element offsets in a pair tile: a row read 4 chunks on, a transpose read 2 chunks on.
template <int COLS>
constexpr int kPairRowStep = 8 * (pair_slot<COLS>(0, 4) - pair_slot<COLS>(0, 0));
template <int COLS>
constexpr int kPairTrStep = 8 * (pair_slot<COLS>(0, 2) - pair_slot<COLS>(0, 0));

// Compile-time check of the claims above: the slots are a bijection onto the tile, the
// inverse matches, each read steps by the compile-time offsets, and every row-read pass
// (8 rows of one parity in one 16-row half, one chunk pair) and every transpose pass
// (one octet, one chunk pair) covers 16 distinct bank groups.
template <int COLS>
constexpr bool pair_tile_ok() {
  constexpr int CH = COLS / 8;
  bool seen[32 * CH] = {};
  for (int m = 0; m < 32; ++m)
    for (int c = 0; c < CH; ++c) {
      const int s = pair_slot<COLS>(m, c);
      if (s < 0 || s >= 32 * CH || seen[s]) return false;
      if (pair_row<COLS>(s) != m || pair_chunk<COLS>(s) != c) return false;
      if (c >= 4 && 8 * pair_slot<COLS>(m, c) != 8 * pair_slot<COLS>(m, c - 4) + kPairRowStep<COLS>)
        return false;
      if (c >= 2 && 8 * pair_slot<COLS>(m, c) != 8 * pair_slot<COLS>(m, c - 2) + kPairTrStep<COLS>)
        return false;
      if (m >= 16 && pair_slot<COLS>(m, c) != pair_slot<COLS>(m - 16, c) + 16 * CH) return false;
      seen[s] = true;
    }
  for (int first = 0; first < 32; ++first) {  // row-read passes: rows first, first + 2, ...
    if ((first & 15) >= 2) continue;
    for (int c0 = 0; c0 < CH; c0 += 2) {
      bool g[16] = {};
      for (int i = 0; i < 8; ++i)
        for (int b = 0; b < 2; ++b) {
          const int grp = pair_slot<COLS>(first + 2 * i, c0 + b) & 15;
          if (g[grp]) return false;
          g[grp] = true;
        }
    }
  }
  for (int o = 0; o < 4; ++o)  // transpose passes
    for (int c0 = 0; c0 < CH; c0 += 2) {
      bool g[16] = {};
      for (int r = 0; r < 8; ++r)
        for (int b = 0; b < 2; ++b) {
          const int grp = pair_slot<COLS>(8 * o + r, c0 + b) & 15;
          if (g[grp]) return false;
          g[grp] = true;
        }
    }
  return true;
}
static_assert(pair_tile_ok<128>() && pair_tile_ok<64>() && pair_tile_ok<32>(),
              "pair tile: bijection, inverse, offsets and one pass per read");

// Swizzled tile (16-byte row reads only): XOR the chunk with the row's index among
// the rows that share one 256-byte bank window.  At D = 128 a row-read pass (8 rows of
// one parity, one chunk pair) then covers 16 distinct bank groups; at D = 64 and 32,
// where a window holds 2 or 4 rows, rows of one parity share half of the groups and
// the reads take two passes (the pair tile would avoid that).
template <int COLS>
__device__ inline int xsw(int r) {
  constexpr int CH = COLS / 8, RPW = 256 / (COLS * 2);
  return (r / RPW) & (CH - 1);
}
template <int COLS>
__device__ inline int xoff(int r, int col) {  // element offset of column col (multiple of 8)
  return r * COLS + ((((col >> 3) ^ xsw<COLS>(r))) << 3);
}

// Direct-to-LDS loads of rows r0..r0+31 into a pair tile: lane i of a load lands in
// slot base + i and fetches the global chunk that belongs there (the inverse of
// pair_slot).  Rows past the resource end arrive as zeros.
template <int COLS, int NT>
__device__ inline void dma_pairs(__amdgpu_buffer_rsrc_t rs, uint32_t row_bytes, int r0,
                                 __bf16* tile, int wave, int lane) {
  constexpr int CH = COLS / 8;
  constexpr int SLOTS = 32 * CH;
#pragma unroll
  for (int it = 0; it < (SLOTS + NT - 1) / NT; ++it) {
    const int base = it * NT + wave * 64;
    if (SLOTS % NT != 0 && base >= SLOTS) break;  // wave-uniform
    const int slot = base + lane;
    const int m = pair_row<COLS>(slot), c = pair_chunk<COLS>(slot);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + base * 8), 16,
                                             (uint32_t)(r0 + m) * row_bytes + (uint32_t)c * 16u,
                                             0, 0, 0);
  }
}

// Direct-to-LDS loads of rows r0..r0+ROWS-1 into a swizzled tile.
template <int ROWS, int COLS, int NT>
__device__ inline void dma_xor(__amdgpu_buffer_rsrc_t rs, uint32_t row_bytes, int r0,
                               __bf16* tile, int wave, int lane) {
  constexpr int CH = COLS / 8;
  constexpr int SLOTS = ROWS * CH;
  static_assert(SLOTS % 64 == 0, "tile must be whole wave loads");
#pragma unroll
  for (int it = 0; it < (SLOTS + NT - 1) / NT; ++it) {
    const int base = it * NT + wave * 64;
    if (SLOTS % NT != 0 && base >= SLOTS) break;  // wave-uniform
    const int slot = base + lane;
    const int r = slot / CH, pc = slot % CH;
    const uint32_t off = (uint32_t)(r0 + r) * row_bytes + (uint32_t)((pc ^ xsw<COLS>(r)) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + base * 8), 16, off, 0, 0, 0);
  }
}

// ------------------------------------------------------------------ dK/dV kernel

constexpr int kKvThreads = 256;  // 4 waves, each 32 keys
constexpr int kKvBN = 128;       // keys per workgroup
constexpr int kKvBQ = 32;        // query rows per iteration

// PACKED: packed documents (a.seg != nullptr), a separate instantiation.
//
// 16x16x32 MFMA tiles: a stream of them sustains about 15% more FLOP/s than 32x32x16
// tiles under the board power limit, which held this kernel back on 32x32x16 tiles.
// Accumulator layout of a 16x16 tile: lane l holds column l % 16 and rows
// 4 (l / 16) + r; operands hold row (A) or column (B) l % 16 and contraction
// indices 8 (l / 16) + j.  S and dP are computed as [query][key] tiles, so each lane
// holds two keys (l % 16 and 16 + l % 16 of the wave's 32) and 8 query rows, and P
// and dS feed dV^T += dO^T P and dK^T += Q^T dS from registers: contraction slot
// 8 g + j holds logical query row 4 g + j (j < 4) or 16 + 4 g + j - 4.
template <int D, bool PACKED>
__global__ __launch_bounds__(kKvThreads, 2) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NKK = D / 32;  // 32-wide head-dim steps of the S and dP contractions
  constexpr int NDT = D / 16;  // 16-row head-dim tiles of dK^T, dV^T
  constexpr int QEL = kKvBQ * D;  // pair tile of 32 rows

  // Two distinct LDS objects per streamed tensor: the compiler can then prove the
  // loads into one never alias the reads of the other.
  __shared__ __attribute__((aligned(16))) __bf16 q0[QEL];
  __shared__ __attribute__((aligned(16))) __bf16 q1[QEL];
  __shared__ __attribute__((aligned(16))) __bf16 do0[QEL];
  __shared__ __attribute__((aligned(16))) __bf16 do1[QEL];
  // LSE / delta slots: one 64-lane DMA fills 64; the first kKvBQ are the tile's
  __shared__ __attribute__((aligned(16))) float ls0[64];
  __shared__ __attribute__((aligned(16))) float ls1[64];
  __shared__ __attribute__((aligned(16))) float dl0[64];
  __shared__ __attribute__((aligned(16))) float dl1[64];
  __shared__ __attribute__((aligned(16))) __bf16 s_v[kKvBN * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l16 = lane & 15, grp = lane >> 4;
  const int kw = wave;  // 32-key block of this wave
  const int L = a.map.L;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = logical % a.n_ktiles;
  const int bg = logical / a.n_ktiles;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int u0 = kt * kKvBN;
  int krow[2], key[2];
  bool key_ok[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    krow[x] = kw * 32 + x * 16 + l16;  // this lane's keys within the tile
    key[x] = u0 + krow[x];
    key_ok[x] = key[x] < L;
  }

  const __bf16* kb = (const __bf16*)a.k + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;
  const __bf16* vb = (const __bf16*)a.v + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;
  const uint32_t kv_row = (uint32_t)(a.kv_st * 2);

  // Queries [q_lo, q_hi) of chunk cq that see each of this lane's keys; query tiles
  // from t_first to t_end hold those of every key, and rows in [full_lo, full_hi)
  // see every key of the workgroup (no mask).
  int q_lo[2] = {0, 0}, q_hi[2] = {L, L};
  int t_first = 0, t_end = L, full_lo = 0, full_hi = L;
  if constexpr (PACKED) {  // packed documents
    __shared__ int red[4];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      if (key_ok[x]) {
        query_interval(a.map, a.cq, pos_of(a.map, a.ck, key[x]), a.causal,
                       a.seg + (int64_t)b * a.seg_n, a.seg_n, q_lo[x], q_hi[x]);
      } else {
        q_lo[x] = L;
        q_hi[x] = 0;
      }
    }
    wg_interval_reduce2(red, q_lo, q_hi, L, t_first, t_end, full_lo, full_hi);
  } else {  // dense: query t sees key u iff t >= count_le(cq, pos(ck, u) - 1)
    const int u_last = min(u0 + kKvBN, L) - 1;
    if (a.causal) {
      t_first = count_le(a.map, a.cq, pos_of(a.map, a.ck, u0) - 1);
      full_lo = count_le(a.map, a.cq, pos_of(a.map, a.ck, u_last) - 1);
#pragma unroll
      for (int x = 0; x < 2; ++x)
        q_lo[x] = key_ok[x] ? count_le(a.map, a.cq, pos_of(a.map, a.ck, key[x]) - 1) : L;
    } else {
#pragma unroll
      for (int x = 0; x < 2; ++x) q_lo[x] = key_ok[x] ? 0 : L;
    }
    if (u0 + kKvBN > L) full_lo = L;  // ragged key tile: always mask
  }
  const int qt_first = t_first / kKvBQ;
  const int n_qt = (t_end + kKvBQ - 1) / kKvBQ;
  const int per_head = n_qt - qt_first;
  const int n_iter = per_head > 0 ? per_head * a.group : 0;
  if (n_iter == 0) {  // no query of this chunk sees these keys: zero gradient
    if (a.write) {
      const f32x4 z = {};
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (!key_ok[x]) continue;
        const int64_t grow = (((int64_t)b * a.Hkv + g) * L + key[x]) * D;
#pragma unroll
        for (int n = 0; n < NDT; ++n) {
          *(f32x4*)(a.dk + grow + n * 16 + grp * 4) = z;
          *(f32x4*)(a.dv + grow + n * 16 + grp * 4) = z;
        }
      }
    }
    return;
  }

  f32x4 dv_t[NDT][2], dk_t[NDT][2];  // [head-dim tile][key tile]
#pragma unroll
  for (int n = 0; n < NDT; ++n) {
    dv_t[n][0] = dv_t[n][1] = f32x4{};
    dk_t[n][0] = dk_t[n][1] = f32x4{};
  }

  // Iterations walk the query tiles [t_lo, t_hi) of one head, then the next head of
  // the GQA group.  The next DMA's tile (head base pointers and first row) advances
  // incrementally, without a division per iteration.
  const int t_lo = qt_first * kKvBQ, t_hi = n_qt * kKvBQ;
  const uint32_t q_row = (uint32_t)(a.q_st * 2), o_row = (uint32_t)(a.o_st * 2);
  const int h0 = g * a.group;
  const __bf16* nq = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)h0 * a.q_sh;
  const __bf16* no = (const __bf16*)a.dout + (int64_t)b * a.o_sb + (int64_t)h0 * a.o_sh;
  int nt = t_lo;   // first row of the next DMA's tile
  int ct = t_lo;   // first row of the current step's tile
  auto dma_q = [&](__bf16* qn, __bf16* don) {
    dma_pairs<D, kKvThreads>(make_rsrc(nq, (uint32_t)L * q_row), q_row, nt, qn, wave, lane);
    dma_pairs<D, kKvThreads>(make_rsrc(no, (uint32_t)L * o_row), o_row, nt, don, wave, lane);
    nt += kKvBQ;
    if (nt >= t_hi) {
      nt = t_lo;
      nq += a.q_sh;
      no += a.o_sh;
    }
  };
  // Row statistics pass through registers one tile ahead of their LDS slots, so they
  // are stored transformed: wave 0 keeps LSE * log2 e (the exponent is one FMA),
  // wave 1 keeps -delta (the dP accumulator starts from it).  Slot s holds query
  // row s of the tile (the first kKvBQ slots are used); rows past the chunk end read as 0,
  // where Q = dO = 0 gives dS = dV = 0.  The LDS write of tile j's statistic comes
  // before the step's DMA issue and the load of tile j + 1's after it.
  const float* sst = (wave == 0 ? a.lse : a.delta) + ((int64_t)b * a.Hq + h0) * L;
  int st_row = t_lo;
  const uint32_t st_lane = (uint32_t)lane;
  float stat_next = 0.0f;
  auto stat_write = [&](float* lsn, float* dln) {
    if (wave == 0) lsn[lane] = stat_next * kLog2e;
    if (wave == 1) dln[lane] = -stat_next;
  };
  auto stat_prefetch = [&](int it_next) {
    if (wave < 2 && it_next < n_iter) {
      stat_next = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(sst, (uint32_t)L * 4u),
                                                      ((uint32_t)st_row + st_lane) * 4u, 0, 0));
      st_row += kKvBQ;
      if (st_row >= t_hi) {
        st_row = t_lo;
        sst += L;
      }
    }
  };

  // This lane's two key rows of K as B operands of S = Q K^T, held in registers for
  // the whole kernel (rows past the chunk end read as 0).
  bf16x8 kreg[2][NKK];
  {
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kb, (uint32_t)L * kv_row);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        kreg[x][kk] = load_row8(kr, (uint32_t)key[x] * kv_row + (uint32_t)(kk * 64 + grp * 16));
  }
  // Element offsets in the pair tiles.  A-operand rows of S and dP: query rows
  // 16 h + l16 at chunk 4 kk + grp (+kk kPairRowStep); transpose-read sources: query
  // rows 16 h + 4 grp + l16 / 4, columns 16 n + 4 (l16 % 4) (+n kPairTrStep).
  int arow[2], trow[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    arow[hf] = 8 * pair_slot<D>(hf * 16 + l16, grp);
    trow[hf] = 8 * pair_slot<D>(hf * 16 + grp * 4 + (l16 >> 2), (l16 & 3) >> 1) + 4 * (l16 & 1);
  }
  // Query row of accumulator row r of half hf: 16 hf + r + goff.
  const int goff = 4 * grp;

  auto step = [&](int it, const __bf16* qt, const __bf16* dot, const float* ls,
                  const float* dl, __bf16* qn, __bf16* don, float* lsn, float* dln) {
    const int t0 = ct;
    ct = ct + kKvBQ >= t_hi ? t_lo : ct + kKvBQ;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile `it`
    __syncthreads();                     // every wave's; tile it-1 is free
    if (it + 1 < n_iter) {
      stat_write(lsn, dln);
      dma_q(qn, don);
      stat_prefetch(it + 2);
    }
    __builtin_amdgcn_iglp_opt(0);  // scheduling hint: interleave LDS reads with MFMAs

    // S[q][key] and dP[q][key] - delta[q] for the tile's two 16-row halves and this
    // lane's keys.
    f32x4 s[2][2], dp[2][2];  // [query half][key tile]
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 nd = *(const f32x4*)(dl + hf * 16 + grp * 4);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        s[hf][x] = f32x4{};
        dp[hf][x] = nd;
      }
    }
    // All S MFMAs first, then dP: the exponentials of S need only the former, and
    // the shorter live ranges of the operands keep the kernel free of spills.
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8 qa[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) qa[hf] = *(const bf16x8*)(qt + arow[hf] + kk * kPairRowStep<D>);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int x = 0; x < 2; ++x)
          s[hf][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[hf], kreg[x][kk], s[hf][x], 0, 0, 0);
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8 vbv[2], da[2];
#pragma unroll
      for (int x = 0; x < 2; ++x)
        vbv[x] = *(const bf16x8*)(s_v + xoff<D>(krow[x], kk * 32 + grp * 8));
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) da[hf] = *(const bf16x8*)(dot + arow[hf] + kk * kPairRowStep<D>);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int x = 0; x < 2; ++x)
          dp[hf][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da[hf], vbv[x], dp[hf][x], 0, 0, 0);
    }

    // P = exp2(S*scale_log2 - LSE*log2 e), dS = P (dP - delta).  Accumulator row r
    // of half hf is query row 16 hf + 4 grp + r = 16 hf + r + goff of the tile.
    const int tq0 = t0;
    // dense problems: every query at or after q_lo sees the key (q_hi = L)
    const bool need_mask = tq0 < full_lo || (PACKED && tq0 + 32 > full_hi);
    // Query row c + goff (c = 16 hf + r) is masked for key x when c < lo_c[x] or
    // c >= hi_c[x]; outside the masked tiles the limits admit every row.
    int lo_c[2], hi_c[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      lo_c[x] = need_mask ? q_lo[x] - tq0 - goff : -64;
      hi_c[x] = (PACKED && need_mask) ? q_hi[x] - tq0 - goff : 64;
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 l4 = *(const f32x4*)(ls + hf * 16 + grp * 4);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s[hf][x][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[hf][x][r], a.scale_log2, -l4[r]));
    }
    if (__builtin_expect(need_mask, 0)) {  // rare: keep it a branch
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        // packed: row c is kept iff lo_c <= c < hi_c, one unsigned compare of c - lo_c
        // with the interval's width (c < lo_c wraps to a large value)
        const uint32_t width = (uint32_t)max(hi_c[x] - lo_c[x], 0);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int c = 16 * hf + r;
            const bool drop = PACKED ? (uint32_t)(c - lo_c[x]) >= width : c < lo_c[x];
            if (drop) s[hf][x][r] = 0.0f;
          }
      }
    }
    bf16x8 pb[2], dsb[2];  // [key tile]; slot 4 hf + r
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pb[x][hf * 4 + r] = (__bf16)s[hf][x][r];
          dsb[x][hf * 4 + r] = (__bf16)(s[hf][x][r] * dp[hf][x][r]);
        }

    // dV^T += dO^T P, dK^T += Q^T dS per 16-row head-dim tile: the A operands hold
    // logical rows 4 grp + k and 16 + 4 grp + k, read transposed.
    __builtin_amdgcn_s_setprio(1);  // MFMA phase first when two waves compete for issue
#pragma unroll
    for (int n = 0; n < NDT; ++n) {
      const bf16x8 doa = cat(tr_read(dot + trow[0] + n * kPairTrStep<D>),
                               tr_read(dot + trow[1] + n * kPairTrStep<D>));
      const bf16x8 qta = cat(tr_read(qt + trow[0] + n * kPairTrStep<D>),
                               tr_read(qt + trow[1] + n * kPairTrStep<D>));
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        dv_t[n][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(doa, pb[x], dv_t[n][x], 0, 0, 0);
        dk_t[n][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qta, dsb[x], dk_t[n][x], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  dma_xor<kKvBN, D, kKvThreads>(make_rsrc(vb, (uint32_t)L * kv_row), kv_row, u0, s_v, wave, lane);
  stat_prefetch(0);
  stat_write(ls0, dl0);
  dma_q(q0, do0);
  stat_prefetch(1);
  for (int it = 0; it < n_iter; it += 2) {
    step(it, q0, do0, ls0, dl0, q1, do1, ls1, dl1);
    if (it + 1 < n_iter) step(it + 1, q1, do1, ls1, dl1, q0, do0, ls0, dl0);
  }

  // Store or add into dK and dV; accumulator row r of head-dim tile n is
  // d = 16 n + 4 grp + r of this lane's key.  When adding, a key's old values are all
  // loaded before its first store: dk and dv may alias for all the compiler knows,
  // so a load behind a store would wait for it.
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    if (!key_ok[x]) continue;
    const int64_t grow = (((int64_t)b * a.Hkv + g) * L + key[x]) * D;
    f32x4* pk = (f32x4*)(a.dk + grow + grp * 4);
    f32x4* pv = (f32x4*)(a.dv + grow + grp * 4);
    if (a.write) {
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        pk[4 * n] = dk_t[n][x] * a.scale;
        pv[4 * n] = dv_t[n][x];
      }
    } else {
      f32x4 ok[NDT], ov[NDT];
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        ok[n] = pk[4 * n];
        ov[n] = pv[4 * n];
      }
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        pk[4 * n] = ok[n] + dk_t[n][x] * a.scale;
        pv[4 * n] = ov[n] + dv_t[n][x];
      }
    }
  }
}

// ---------------------------------------------------------------------- dQ kernel

// Workgroup shape of the dQ kernel: 8 waves (256 query rows, each K/V tile serving
// all of them) on dense sequences; 4 waves (128 rows, two workgroups per CU) with
// packed documents at head dim 128, where fewer workgroups straddle a document
// boundary (7.7% faster there, 2% slower on dense sequences).  Other head dims keep
// the 8-wave shape, on which they were measured.
template <int D, bool PACKED>
struct QCfg {
  static constexpr int NW = (PACKED && D == 128) ? 4 : 8;
  static constexpr int NT = 64 * NW;  // threads
  static constexpr int BM = 32 * NW;  // query rows per workgroup
};
constexpr int kQBN = 32;        // keys per KV tile

template <int D, bool PACKED>
__global__ __launch_bounds__((QCfg<D, PACKED>::NT), (QCfg<D, PACKED>::NW == 4 ? 2 : 1)) void bwd_dq_kernel(
    BwdArgs a) {
  constexpr int kQThreads = QCfg<D, PACKED>::NT;
  constexpr int kQBM = QCfg<D, PACKED>::BM;
  constexpr int NKK = D / 32;  // 32-wide head-dim steps of the S^T and dP^T contractions
  constexpr int NDT = D / 16;  // 16-row head-dim tiles of dQ^T
  constexpr int KEL = kQBN * D;  // pair tile of 32 keys
  constexpr int VEL = kQBN * D;
  static_assert(kQBN == 32, "one 32-key contraction step per tile");

  __shared__ __attribute__((aligned(16))) __bf16 k0[KEL];
  __shared__ __attribute__((aligned(16))) __bf16 k1[KEL];
  __shared__ __attribute__((aligned(16))) __bf16 v0[VEL];
  __shared__ __attribute__((aligned(16))) __bf16 v1[VEL];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l16 = lane & 15, grp = lane >> 4;
  const int L = a.map.L;

  const int n_qtiles = (L + kQBM - 1) / kQBM;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qi = logical % n_qtiles;
  const int bh = logical / n_qtiles;
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int qt = n_qtiles - 1 - qi;  // heaviest (latest) query tiles first
  const int t0 = qt * kQBM;
  int tq[2];  // this lane's query rows
#pragma unroll
  for (int x = 0; x < 2; ++x) tq[x] = t0 + wave * 32 + x * 16 + l16;
  const int g = h / a.group;

  const __bf16* qb = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const __bf16* ob = (const __bf16*)a.dout + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh;
  const __bf16* kb = (const __bf16*)a.k + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;
  const __bf16* vb = (const __bf16*)a.v + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;
  const uint32_t q_row = (uint32_t)(a.q_st * 2), o_row = (uint32_t)(a.o_st * 2);
  const uint32_t kv_row = (uint32_t)(a.kv_st * 2);
  const __amdgpu_buffer_rsrc_t qr_ = make_rsrc(qb, (uint32_t)L * q_row);
  const __amdgpu_buffer_rsrc_t or_ = make_rsrc(ob, (uint32_t)L * o_row);
  const __amdgpu_buffer_rsrc_t kr_ = make_rsrc(kb, (uint32_t)L * kv_row);
  const __amdgpu_buffer_rsrc_t vr_ = make_rsrc(vb, (uint32_t)L * kv_row);

  // This lane's Q and dO rows: B operands of S^T = K Q^T and dP^T = V dO^T.
  bf16x8 qr[2][NKK], dr[2][NKK];
  float lse2[2], dlt[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qr[x][kk] = load_row8(qr_, (uint32_t)tq[x] * q_row + (uint32_t)(kk * 64 + grp * 16));
      dr[x][kk] = load_row8(or_, (uint32_t)tq[x] * o_row + (uint32_t)(kk * 64 + grp * 16));
    }
    const int64_t row = ((int64_t)b * a.Hq + h) * L + tq[x];
    lse2[x] = tq[x] < L ? a.lse[row] * kLog2e : 0.0f;
    dlt[x] = tq[x] < L ? a.delta[row] : 0.0f;
  }
  // -delta of each row, the start of the dP^T accumulators (they then hold dP^T - delta)
  f32x4 ndlt[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) ndlt[x] = f32x4{-dlt[x], -dlt[x], -dlt[x], -dlt[x]};

  // Visible keys of each row and of the workgroup (as in the forward): key tiles
  // j0..n_tiles-1, no mask inside [full_lo, n_full).
  int kv_lo[2] = {0, 0}, kv_lim[2] = {L, L};
  int j0 = 0, n_keys = L, full_lo = 0, n_full = L;
  if constexpr (PACKED) {  // packed documents
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
    j0 = min_lo / kQBN;
  } else if (a.causal) {
    const int t_last = min(t0 + kQBM, L) - 1;
#pragma unroll
    for (int x = 0; x < 2; ++x)
      kv_lim[x] = count_le(a.map, a.ck, pos_of(a.map, a.cq, min(tq[x], L - 1)));
    n_keys = count_le(a.map, a.ck, pos_of(a.map, a.cq, t_last));
    n_full = count_le(a.map, a.ck, pos_of(a.map, a.cq, t0));
  }
  const int n_tiles = (n_keys + kQBN - 1) / kQBN;

  f32x4 dq_t[NDT][2];  // [head-dim tile][query half]
#pragma unroll
  for (int n = 0; n < NDT; ++n) dq_t[n][0] = dq_t[n][1] = f32x4{};

  // The K tile, read both ways, is a pair tile; the V tile, read only by 16-byte row
  // reads, is XOR-swizzled.  Element offsets in the K tile: A-operand rows of S^T,
  // keys 16 t + l16 at chunk 4 kk + grp (+kk kPairRowStep); transpose-read sources of
  // K^T, keys 16 t + 4 grp + l16 / 4, columns 16 n + 4 (l16 % 4) (+n kPairTrStep).
  int krow[2], trow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    krow[t] = 8 * pair_slot<D>(t * 16 + l16, grp);
    trow[t] = 8 * pair_slot<D>(t * 16 + grp * 4 + (l16 >> 2), (l16 & 3) >> 1) + 4 * (l16 & 1);
  }
  // Key of accumulator row r of key tile t: u0 + 16 t + r + goff.
  const int goff = 4 * grp;

  auto dma_kv = [&](int j, __bf16* kn, __bf16* vn) {
    dma_pairs<D, kQThreads>(kr_, kv_row, j * kQBN, kn, wave, lane);
    dma_xor<kQBN, D, kQThreads>(vr_, kv_row, j * kQBN, vn, wave, lane);
  };

  auto tile = [&](int j, const __bf16* kt, const __bf16* vt, __bf16* kn, __bf16* vn) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile j
    __syncthreads();                     // every wave's; tile j-1 is free
    if (j + 1 < n_tiles) dma_kv(j + 1, kn, vn);

    // S^T and dP^T - delta for this tile: [key tile][query half] 16x16 blocks.
    f32x4 s[2][2], dp[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        s[t][x] = f32x4{};
        dp[t][x] = ndlt[x];
      }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 ka = *(const bf16x8*)(kt + krow[t] + kk * kPairRowStep<D>);
        const bf16x8 va = *(const bf16x8*)(vt + xoff<D>(t * 16 + l16, kk * 32 + grp * 8));
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          s[t][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qr[x][kk], s[t][x], 0, 0, 0);
          dp[t][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, dr[x][kk], dp[t][x], 0, 0, 0);
        }
      }

    // P^T = exp2(S^T*scale_log2 - LSE*log2 e) with keys outside the row's visible
    // interval masked; dS^T = P^T (dP^T - delta).
    const int u0 = j * kQBN;
    const bool need_mask = u0 < full_lo || u0 + kQBN > n_full;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s[t][x][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][x][r], a.scale_log2, -lse2[x]));
    if (__builtin_expect(need_mask, 0)) {  // rare: keep it a branch
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        // key u = u0 + 16 t + r + goff is kept iff kv_lo <= u < kv_lim: one unsigned
        // compare of u - kv_lo with the interval's width
        const int base = u0 + goff - kv_lo[x];
        const uint32_t width = (uint32_t)max(kv_lim[x] - kv_lo[x], 0);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if ((uint32_t)(base + 16 * t + r) >= width) s[t][x][r] = 0.0f;
      }
    }
    bf16x8 dsb[2];  // [query half]; slot 4 t + r holds logical key 16 t + 4 grp + r
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dsb[x][t * 4 + r] = (__bf16)(s[t][x][r] * dp[t][x][r]);

    // dQ^T += K^T dS^T per 16-row head-dim tile; K^T read transposed.
#pragma unroll
    for (int n = 0; n < NDT; ++n) {
      const bf16x8 kta = cat(tr_read(kt + trow[0] + n * kPairTrStep<D>),
                               tr_read(kt + trow[1] + n * kPairTrStep<D>));
#pragma unroll
      for (int x = 0; x < 2; ++x)
        dq_t[n][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kta, dsb[x], dq_t[n][x], 0, 0, 0);
    }
  };

  if (n_tiles > j0) dma_kv(j0, k0, v0);
  for (int j = j0; j < n_tiles; j += 2) {
    tile(j, k0, v0, k1, v1);
    if (j + 1 < n_tiles) tile(j + 1, k1, v1, k0, v0);
  }

  // dQ[q][d] (+)= scale * dQ^T[d][q]; accumulator row r of tile n is d = 16 n + 4 grp + r.
  // A row that sees no key of this chunk adds nothing, or stores zeros in write mode.
  // When adding, both rows' old values are loaded before the first store (a load
  // behind a store to a possibly aliasing row would wait for it).
  if (n_tiles > j0 || a.write) {
    f32x4* p[2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
      p[x] = (f32x4*)(a.dq + (((int64_t)b * a.Hq + h) * L + min(tq[x], L - 1)) * D + grp * 4);
    if (a.write) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (tq[x] >= L) continue;
#pragma unroll
        for (int n = 0; n < NDT; ++n) p[x][4 * n] = dq_t[n][x] * a.scale;
      }
    } else {
      f32x4 old[2][NDT];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (tq[x] >= L) continue;
#pragma unroll
        for (int n = 0; n < NDT; ++n) old[x][n] = p[x][4 * n];
      }
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (tq[x] >= L) continue;
#pragma unroll
        for (int n = 0; n < NDT; ++n) p[x][4 * n] = old[x][n] + dq_t[n][x] * a.scale;
      }
    }
  }
}

template <int D, bool PK>
hipError_t launch(const BwdArgs& a, int which, hipStream_t s) {
  if (which & 1) {
    const int64_t nkv = (int64_t)a.B * a.Hkv * a.n_ktiles;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, PK>), dim3((unsigned)nkv), dim3(kKvThreads), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (which & 2) {
    const int64_t nq = (int64_t)a.B * a.Hq * ((a.map.L + QCfg<D, PK>::BM - 1) / QCfg<D, PK>::BM);
    hipLaunchKernelGGL((bwd_dq_kernel<D, PK>), dim3((unsigned)nq), dim3(QCfg<D, PK>::NT), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

int bwd_block_n(int /*dtype*/, int /*D*/) { return kKvBN; }

hipError_t launch_bwd(int dtype, int D, const BwdArgs& a, int which, hipStream_t s) {
  if (dtype != RA_BF16) return hipErrorNotSupported;
  const bool pk = a.seg != nullptr;
  if (D == 128) return pk ? launch<128, true>(a, which, s) : launch<128, false>(a, which, s);
  if (D == 64) return pk ? launch<64, true>(a, which, s) : launch<64, false>(a, which, s);
  if (D == 32) return pk ? launch<32, true>(a, which, s) : launch<32, false>(a, which, s);
  return hipErrorInvalidValue;
}

}  // namespace ra
