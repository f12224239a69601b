// C ABI of the ring-attention step: argument validation, the ring drivers and the
// host-only helpers.  Everything is validated before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "ra_internal.h"

namespace {

thread_local char g_last_error[512] = "";

ra_status_t fail(ra_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

ra_status_t ok() {
  g_last_error[0] = '\0';
  return RA_OK;
}

ra_status_t hip_fail(hipError_t e, const char* where) {
  return fail(RA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t elem_size(int dtype) { return dtype == RA_BF16 ? 2 : 4; }

// Validates the problem description itself.
ra_status_t check_problem(const ra_problem_t* p) {
  if (p == nullptr) return fail(RA_ERR_NULL, "problem is NULL");
  if (p->batch < 1 || p->heads_q < 1 || p->heads_kv < 1)
    return fail(RA_ERR_SHAPE, "batch, heads_q and heads_kv must be >= 1");
  // The kernels take them as 32-bit integers; the bound also keeps batch * heads_q
  // below 2^62, so the size checks below cannot overflow.
  if (p->batch > INT32_MAX || p->heads_q > INT32_MAX || p->heads_kv > INT32_MAX)
    return fail(RA_ERR_SHAPE, "batch, heads_q and heads_kv must be < 2^31");
  if (p->heads_q % p->heads_kv != 0)
    return fail(RA_ERR_SHAPE, "heads_q (%lld) must be a multiple of heads_kv (%lld)",
                (long long)p->heads_q, (long long)p->heads_kv);
  if (p->head_dim_padded != 32 && p->head_dim_padded != 64 && p->head_dim_padded != 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim_padded must be 32, 64 or 128 (got %lld)",
                (long long)p->head_dim_padded);
  if (p->head_dim < 1 || p->head_dim > p->head_dim_padded)
    return fail(RA_ERR_SHAPE, "head_dim must be in [1, head_dim_padded]");
  if (p->world < 1) return fail(RA_ERR_SHAPE, "world must be >= 1");
  if (p->layout != RA_LAYOUT_CONTIGUOUS && p->layout != RA_LAYOUT_ZIGZAG &&
      p->layout != RA_LAYOUT_STRIPED)
    return fail(RA_ERR_UNSUPPORTED, "unknown layout %d", p->layout);
  if (p->causal != 0 && p->causal != 1) return fail(RA_ERR_SHAPE, "causal must be 0 or 1");
  if (p->dtype != RA_F32 && p->dtype != RA_BF16)
    return fail(RA_ERR_UNSUPPORTED, "unknown dtype %d", p->dtype);
  if (p->seg_count < 0 || p->seg_count == 1 || p->seg_count > (1 << 24))
    return fail(RA_ERR_SHAPE, "seg_count must be 0 (dense) or in [2, 2^24]");
  if ((p->seg_bounds == nullptr) != (p->seg_count == 0))
    return fail(RA_ERR_SHAPE, "seg_bounds and seg_count must be both set or both zero");
  if (((uintptr_t)p->seg_bounds & 3u) != 0)
    return fail(RA_ERR_SHAPE, "seg_bounds must be 4-byte aligned");
  if (!(p->scale >= 0.0f) || isinf(p->scale))
    return fail(RA_ERR_SHAPE, "scale must be finite and >= 0");
  if (p->seq_total < 1 || p->seq_total >= (int64_t(1) << 31))
    return fail(RA_ERR_SHAPE, "seq_total must be in [1, 2^31)");
  const int64_t div = p->layout == RA_LAYOUT_ZIGZAG ? 2 * (int64_t)p->world : p->world;
  if (p->seq_total % div != 0)
    return fail(RA_ERR_SHAPE, "seq_total (%lld) must be a multiple of %lld for this layout",
                (long long)p->seq_total, (long long)div);
  const int64_t es = elem_size(p->dtype);
  const int64_t* strides[3] = {p->q_stride, p->kv_stride, p->o_stride};
  const char* names[3] = {"q_stride", "kv_stride", "o_stride"};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) {
      if (strides[i][j] < 0) return fail(RA_ERR_SHAPE, "%s[%d] is negative", names[i], j);
      if (strides[i][j] >= (int64_t(1) << 48))  // keeps every product below in range
        return fail(RA_ERR_SHAPE, "%s[%d] must be < 2^48 elements", names[i], j);
      if ((strides[i][j] * es) % 16 != 0)
        return fail(RA_ERR_SHAPE, "%s[%d] * element size must be a multiple of 16 bytes",
                    names[i], j);
    }
  const int64_t L = p->seq_total / p->world;
  // The kernels address rows inside one head with 32-bit buffer offsets (a tile may
  // run up to 256 rows past the chunk end, where loads return zeros); the backward
  // reads dout that way too.
  // (L + 256) * row bytes >= 2^32, as a division: the product itself may not fit.
  for (int i = 0; i < 3; ++i)
    if (strides[i][2] * es > ((int64_t(1) << 32) - 1) / (L + 256))
      return fail(RA_ERR_UNSUPPORTED, "%s[2] too large: one head's rows must span < 4 GiB",
                  names[i]);
  if ((L + 256) * p->head_dim_padded * 4 >= (int64_t(1) << 32))
    return fail(RA_ERR_UNSUPPORTED, "chunk too long: one head's fp32 rows must span < 4 GiB");
  // Every attention kernel launches at most 2 work-items per query row (or key) of a
  // chunk rounded up to its tile, and one grid dimension holds fewer than 2^32.
  const int64_t rows = p->batch * p->heads_q;  // < 2^62
  if (rows > ((int64_t(1) << 31) - 1) / (L + 256))  // rows * (L + 256) >= 2^31
    return fail(RA_ERR_SHAPE,
                "problem too large for one launch: batch * heads_q * (L + 256) must be < 2^31");
  return RA_OK;
}

ra::LayoutMap make_map(const ra_problem_t* p) {
  ra::LayoutMap m;
  m.layout = p->layout;
  m.S = (int32_t)p->seq_total;
  m.p = p->world;
  m.L = (int32_t)(p->seq_total / p->world);
  m.h = (int32_t)(p->seq_total / (2 * (int64_t)p->world));
  return m;
}

float softmax_scale(const ra_problem_t* p) {
  return p->scale > 0.0f ? p->scale : (float)(1.0 / sqrt((double)p->head_dim));
}

ra_status_t check_chunk(const ra_problem_t* p, int32_t c, const char* what) {
  if (c < 0 || c >= p->world) return fail(RA_ERR_SHAPE, "%s %d outside [0, %d)", what, c, p->world);
  return RA_OK;
}

ra_status_t check_ptr(const void* ptr, const char* what) {
  if (ptr == nullptr) return fail(RA_ERR_NULL, "%s is NULL", what);
  if (!aligned16(ptr)) return fail(RA_ERR_SHAPE, "%s is not 16-byte aligned", what);
  return RA_OK;
}

#define RA_TRY(x)                  \
  do {                             \
    ra_status_t _st = (x);         \
    if (_st != RA_OK) return _st;  \
  } while (0)

// True when query chunk cq sees at least one key of KV chunk ck.
bool step_live(const ra_problem_t* p, const ra::LayoutMap& m, int cq, int ck) {
  if (!p->causal) return true;
  return ra::count_le(m, ck, ra::pos_of(m, cq, m.L - 1)) > 0;
}

ra::FwdArgs fwd_args(const ra_problem_t* p, const void* q, int cq, const void* k, const void* v,
                     int ck) {
  ra::FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_sb = p->q_stride[0];
  a.q_sh = p->q_stride[1];
  a.q_st = p->q_stride[2];
  a.kv_sb = p->kv_stride[0];
  a.kv_sh = p->kv_stride[1];
  a.kv_st = p->kv_stride[2];
  a.B = (int32_t)p->batch;
  a.Hq = (int32_t)p->heads_q;
  a.Hkv = (int32_t)p->heads_kv;
  a.group = (int32_t)(p->heads_q / p->heads_kv);
  a.cq = cq;
  a.ck = ck;
  a.causal = p->causal;
  a.map = make_map(p);
  const int bm = ra::fwd_block_m(p->dtype, (int)p->head_dim_padded, p->seg_bounds != nullptr,
                                 (int)(p->heads_q / p->heads_kv));
  a.n_qtiles = (a.map.L + bm - 1) / bm;
  a.scale_log2 = softmax_scale(p) * 1.4426950408889634f;
  a.seg = p->seg_bounds;
  a.seg_n = p->seg_count;
  return a;
}

// Output = fp32 contiguous [B, Hq, L, D].
void set_out_f32_contig(ra::FwdArgs& a, const ra_problem_t* p, float* o) {
  const int64_t D = p->head_dim_padded, L = a.map.L;
  a.out = o;
  a.out_f32 = 1;
  a.o_sb = p->heads_q * L * D;
  a.o_sh = L * D;
  a.o_st = D;
}

// Output = the user's out in the problem dtype with o strides.
void set_out_user(ra::FwdArgs& a, const ra_problem_t* p, void* out) {
  a.out = out;
  a.out_f32 = p->dtype == RA_F32;
  a.o_sb = p->o_stride[0];
  a.o_sh = p->o_stride[1];
  a.o_st = p->o_stride[2];
}

}  // namespace

extern "C" {

const char* ra_status_str(ra_status_t s) {
  switch (s) {
    case RA_OK: return "RA_OK";
    case RA_ERR_NULL: return "RA_ERR_NULL";
    case RA_ERR_SHAPE: return "RA_ERR_SHAPE";
    case RA_ERR_UNSUPPORTED: return "RA_ERR_UNSUPPORTED";
    case RA_ERR_WORKSPACE: return "RA_ERR_WORKSPACE";
    case RA_ERR_HIP: return "RA_ERR_HIP";
  }
  return "RA_ERR_UNKNOWN";
}

const char* ra_last_error(void) { return g_last_error; }

ra_status_t ra_positions(const ra_problem_t* prob, int32_t chunk, int64_t* host_out) {
  RA_TRY(check_problem(prob));
  RA_TRY(check_chunk(prob, chunk, "chunk"));
  if (host_out == nullptr) return fail(RA_ERR_NULL, "host_out is NULL");
  const ra::LayoutMap m = make_map(prob);
  for (int32_t t = 0; t < m.L; ++t) host_out[t] = ra::pos_of(m, chunk, t);
  return ok();
}

ra_status_t ra_visible_pairs(const ra_problem_t* prob, int32_t q_chunk, int32_t kv_chunk,
                             int64_t* pairs) {
  RA_TRY(check_problem(prob));
  RA_TRY(check_chunk(prob, q_chunk, "q_chunk"));
  RA_TRY(check_chunk(prob, kv_chunk, "kv_chunk"));
  if (pairs == nullptr) return fail(RA_ERR_NULL, "pairs is NULL");
  if (prob->seg_bounds != nullptr)
    return fail(RA_ERR_UNSUPPORTED, "packed problem: use ra_visible_pairs_packed");
  const ra::LayoutMap m = make_map(prob);
  int64_t n = 0;
  if (!prob->causal) {
    n = (int64_t)m.L * m.L;
  } else {
    for (int32_t t = 0; t < m.L; ++t) n += ra::count_le(m, kv_chunk, ra::pos_of(m, q_chunk, t));
  }
  *pairs = n;
  return ok();
}

ra_status_t ra_visible_pairs_packed(const ra_problem_t* prob, int32_t q_chunk,
                                    int32_t kv_chunk, const int32_t* host_bounds,
                                    int64_t* pairs) {
  RA_TRY(check_problem(prob));
  RA_TRY(check_chunk(prob, q_chunk, "q_chunk"));
  RA_TRY(check_chunk(prob, kv_chunk, "kv_chunk"));
  if (pairs == nullptr || host_bounds == nullptr)
    return fail(RA_ERR_NULL, "pairs or host_bounds is NULL");
  if (prob->seg_count < 2) return fail(RA_ERR_SHAPE, "not a packed problem (seg_count < 2)");
  const ra::LayoutMap m = make_map(prob);
  const int32_t n = prob->seg_count;
  int64_t total = 0;
  for (int64_t b = 0; b < prob->batch; ++b) {
    const int32_t* e = host_bounds + b * n;
    if (e[0] != 0 || e[n - 1] > m.S)
      return fail(RA_ERR_SHAPE, "batch %lld: bounds must start at 0 and end <= S", (long long)b);
    for (int32_t j = 1; j < n; ++j)
      if (e[j] < e[j - 1])
        return fail(RA_ERR_SHAPE, "batch %lld: bounds must be nondecreasing", (long long)b);
    for (int32_t t = 0; t < m.L; ++t) {
      int32_t lo, hi;
      ra::key_interval(m, kv_chunk, ra::pos_of(m, q_chunk, t), prob->causal, e, n, lo, hi);
      if (hi > lo) total += hi - lo;
    }
  }
  *pairs = total;
  return ok();
}

ra_status_t ra_block_attn_fwd(const ra_problem_t* prob, const void* q, int32_t q_chunk,
                              const void* k, const void* v, int32_t kv_chunk, float* o,
                              float* lse, int32_t mode, hipStream_t stream) {
  RA_TRY(check_problem(prob));
  RA_TRY(check_chunk(prob, q_chunk, "q_chunk"));
  RA_TRY(check_chunk(prob, kv_chunk, "kv_chunk"));
  RA_TRY(check_ptr(q, "q"));
  RA_TRY(check_ptr(k, "k"));
  RA_TRY(check_ptr(v, "v"));
  RA_TRY(check_ptr(o, "o"));
  if (lse == nullptr) return fail(RA_ERR_NULL, "lse is NULL");
  if (mode != RA_WRITE && mode != RA_MERGE) return fail(RA_ERR_UNSUPPORTED, "unknown mode %d", mode);
  ra::FwdArgs a = fwd_args(prob, q, q_chunk, k, v, kv_chunk);
  set_out_f32_contig(a, prob, o);
  a.lse_out = lse;
  if (mode == RA_MERGE) {
    a.acc_in = o;
    a.lse_in = lse;
  }
  hipError_t e = ra::launch_fwd(prob->dtype, (int)prob->head_dim_padded, (int)prob->head_dim, a, stream);
  if (e != hipSuccess) return hip_fail(e, "ra_block_attn_fwd launch");
  return ok();
}

ra_status_t ra_lse_merge(int64_t rows, int32_t d, float* o_acc, float* lse_acc,
                         const float* o_part, const float* lse_part, hipStream_t stream) {
  if (rows < 0 || rows >= (int64_t(1) << 34))
    return fail(RA_ERR_SHAPE, "rows must be in [0, 2^34) (one launch)");
  if (d < 4 || d > 1024 || d % 4 != 0) return fail(RA_ERR_SHAPE, "d must be in [4, 1024], d %% 4 == 0");
  if (rows == 0) return ok();
  RA_TRY(check_ptr(o_acc, "o_acc"));
  RA_TRY(check_ptr(o_part, "o_part"));
  if (lse_acc == nullptr || lse_part == nullptr) return fail(RA_ERR_NULL, "lse pointer is NULL");
  hipError_t e = ra::launch_lse_merge(rows, d, o_acc, lse_acc, o_part, lse_part, stream);
  if (e != hipSuccess) return hip_fail(e, "ra_lse_merge launch");
  return ok();
}

ra_status_t ra_ring_workspace_size(const ra_problem_t* prob, size_t* bytes) {
  RA_TRY(check_problem(prob));
  if (bytes == nullptr) return fail(RA_ERR_NULL, "bytes is NULL");
  const int64_t L = prob->seq_total / prob->world;
  *bytes = (size_t)(prob->batch * prob->heads_q * L * prob->head_dim_padded * 4);
  return ok();
}

ra_status_t ra_ring_fwd(const ra_problem_t* prob, int32_t rank, const void* q,
                        const void* const* k_chunks, const void* const* v_chunks, void* out,
                        float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  RA_TRY(check_problem(prob));
  RA_TRY(check_chunk(prob, rank, "rank"));
  RA_TRY(check_ptr(q, "q"));
  if (k_chunks == nullptr || v_chunks == nullptr) return fail(RA_ERR_NULL, "chunk array is NULL");
  for (int c = 0; c < prob->world; ++c) {
    RA_TRY(check_ptr(k_chunks[c], "k_chunks[c]"));
    RA_TRY(check_ptr(v_chunks[c], "v_chunks[c]"));
  }
  RA_TRY(check_ptr(out, "out"));
  if (lse == nullptr) return fail(RA_ERR_NULL, "lse is NULL");
  const ra::LayoutMap m = make_map(prob);
  int live[4096];
  if (prob->world > 4096) return fail(RA_ERR_UNSUPPORTED, "world > 4096");
  int n_live = 0;
  for (int s = 0; s < prob->world; ++s) {
    const int c = ((rank - s) % prob->world + prob->world) % prob->world;
    if (step_live(prob, m, rank, c)) live[n_live++] = c;
  }
  size_t need = 0;
  RA_TRY(ra_ring_workspace_size(prob, &need));
  if (n_live >= 2) {
    if (ws == nullptr || ws_bytes < need)
      return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
    if (((uintptr_t)ws & 255u) != 0) return fail(RA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  if (n_live == 0) live[n_live++] = rank;  // writes o = 0, lse = -inf
  for (int i = 0; i < n_live; ++i) {
    ra::FwdArgs a = fwd_args(prob, q, rank, k_chunks[live[i]], v_chunks[live[i]], live[i]);
    const bool first = i == 0, last = i == n_live - 1;
    if (last) {
      set_out_user(a, prob, out);
    } else {
      set_out_f32_contig(a, prob, (float*)ws);
    }
    if (!first) {
      a.acc_in = (const float*)ws;
      a.lse_in = lse;
    }
    a.lse_out = lse;
    hipError_t e = ra::launch_fwd(prob->dtype, (int)prob->head_dim_padded, (int)prob->head_dim, a, stream);
    if (e != hipSuccess) return hip_fail(e, "ra_ring_fwd launch");
  }
  return ok();
}

ra_status_t ra_bwd_delta(const ra_problem_t* prob, const void* out, const void* dout,
                         float* delta, hipStream_t stream) {
  RA_TRY(check_problem(prob));
  RA_TRY(check_ptr(out, "out"));
  RA_TRY(check_ptr(dout, "dout"));
  if (delta == nullptr) return fail(RA_ERR_NULL, "delta is NULL");
  const int32_t L = (int32_t)(prob->seq_total / prob->world);
  hipError_t e = ra::launch_bwd_delta(prob->dtype, (int32_t)prob->batch, (int32_t)prob->heads_q, L,
                                      (int32_t)prob->head_dim_padded, out, dout, prob->o_stride[0],
                                      prob->o_stride[1], prob->o_stride[2], delta, stream);
  if (e != hipSuccess) return hip_fail(e, "ra_bwd_delta launch");
  return ok();
}

ra_status_t ra_bwd_prepare(const ra_problem_t* prob, const void* out, const void* dout,
                           float* delta, float* dq, float* const* dk_chunks,
                           float* const* dv_chunks, hipStream_t stream) {
  RA_TRY(check_problem(prob));
  RA_TRY(check_ptr(dq, "dq"));
  if (dk_chunks == nullptr || dv_chunks == nullptr) return fail(RA_ERR_NULL, "chunk array is NULL");
  for (int c = 0; c < prob->world; ++c) {
    RA_TRY(check_ptr(dk_chunks[c], "dk_chunks[c]"));
    RA_TRY(check_ptr(dv_chunks[c], "dv_chunks[c]"));
  }
  RA_TRY(ra_bwd_delta(prob, out, dout, delta, stream));
  const int64_t L = prob->seq_total / prob->world;
  const int64_t D = prob->head_dim_padded;
  hipError_t e = ra::launch_fill_f32(dq, prob->batch * prob->heads_q * L * D, 0.0f, stream);
  if (e != hipSuccess) return hip_fail(e, "ra_bwd_prepare fill");
  const int64_t nkv = prob->batch * prob->heads_kv * L * D;
  for (int c = 0; c < prob->world; ++c) {
    e = ra::launch_fill_f32(dk_chunks[c], nkv, 0.0f, stream);
    if (e == hipSuccess) e = ra::launch_fill_f32(dv_chunks[c], nkv, 0.0f, stream);
    if (e != hipSuccess) return hip_fail(e, "ra_bwd_prepare fill");
  }
  return ok();
}

static ra_status_t bwd_supported(const ra_problem_t* prob) {
  if (prob->dtype != RA_BF16)
    return fail(RA_ERR_UNSUPPORTED, "the backward supports bf16 only");
  return RA_OK;
}

static ra::BwdArgs bwd_args(const ra_problem_t* prob, const void* q, int cq, const void* k,
                            const void* v, int ck, const void* dout, const float* lse,
                            const float* delta, float* dq, float* dk, float* dv) {
  ra::BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.q_sb = prob->q_stride[0];
  a.q_sh = prob->q_stride[1];
  a.q_st = prob->q_stride[2];
  a.kv_sb = prob->kv_stride[0];
  a.kv_sh = prob->kv_stride[1];
  a.kv_st = prob->kv_stride[2];
  a.o_sb = prob->o_stride[0];
  a.o_sh = prob->o_stride[1];
  a.o_st = prob->o_stride[2];
  a.B = (int32_t)prob->batch;
  a.Hq = (int32_t)prob->heads_q;
  a.Hkv = (int32_t)prob->heads_kv;
  a.group = (int32_t)(prob->heads_q / prob->heads_kv);
  a.cq = cq;
  a.ck = ck;
  a.causal = prob->causal;
  a.map = make_map(prob);
  const int bn = ra::bwd_block_n(prob->dtype, (int)prob->head_dim_padded);
  a.n_ktiles = (a.map.L + bn - 1) / bn;
  a.scale = softmax_scale(prob);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.seg = prob->seg_bounds;
  a.seg_n = prob->seg_count;
  return a;
}

static ra_status_t block_bwd(const ra_problem_t* prob, const void* q, int32_t q_chunk,
                             const void* k, const void* v, int32_t kv_chunk, const void* dout,
                             const float* lse, const float* delta, float* dq, float* dk,
                             float* dv, int which, int32_t mode, hipStream_t stream) {
  RA_TRY(check_problem(prob));
  RA_TRY(bwd_supported(prob));
  if (mode != RA_WRITE && mode != RA_MERGE) return fail(RA_ERR_UNSUPPORTED, "unknown mode %d", mode);
  RA_TRY(check_chunk(prob, q_chunk, "q_chunk"));
  RA_TRY(check_chunk(prob, kv_chunk, "kv_chunk"));
  RA_TRY(check_ptr(q, "q"));
  RA_TRY(check_ptr(k, "k"));
  RA_TRY(check_ptr(v, "v"));
  RA_TRY(check_ptr(dout, "dout"));
  if (which & 2) RA_TRY(check_ptr(dq, "dq"));
  if (which & 1) {
    RA_TRY(check_ptr(dk, "dk"));
    RA_TRY(check_ptr(dv, "dv"));
  }
  if (lse == nullptr || delta == nullptr) return fail(RA_ERR_NULL, "lse or delta is NULL");
  const ra::LayoutMap m = make_map(prob);
  ra::BwdArgs a = bwd_args(prob, q, q_chunk, k, v, kv_chunk, dout, lse, delta, dq, dk, dv);
  a.write = mode == RA_WRITE;
  hipError_t e = hipSuccess;
  if (step_live(prob, m, q_chunk, kv_chunk)) {
    e = ra::launch_bwd(prob->dtype, (int)prob->head_dim_padded, a, which, stream);
  } else if (a.write) {  // nothing visible: the step's gradients are zero
    const int64_t L = prob->seq_total / prob->world, D = prob->head_dim_padded;
    if (which & 2) e = ra::launch_fill_f32(dq, prob->batch * prob->heads_q * L * D, 0.0f, stream);
    if (e == hipSuccess && (which & 1)) {
      const int64_t n = prob->batch * prob->heads_kv * L * D;
      e = ra::launch_fill_f32(dk, n, 0.0f, stream);
      if (e == hipSuccess) e = ra::launch_fill_f32(dv, n, 0.0f, stream);
    }
  }
  if (e != hipSuccess) return hip_fail(e, "ra_block_attn_bwd launch");
  return ok();
}

ra_status_t ra_block_attn_bwd(const ra_problem_t* prob, const void* q, int32_t q_chunk,
                              const void* k, const void* v, int32_t kv_chunk, const void* dout,
                              const float* lse, const float* delta, float* dq, float* dk,
                              float* dv, hipStream_t stream) {
  return block_bwd(prob, q, q_chunk, k, v, kv_chunk, dout, lse, delta, dq, dk, dv, 3, RA_MERGE,
                   stream);
}

ra_status_t ra_block_attn_bwd_dkdv(const ra_problem_t* prob, const void* q, int32_t q_chunk,
                                   const void* k, const void* v, int32_t kv_chunk,
                                   const void* dout, const float* lse, const float* delta,
                                   float* dk, float* dv, int32_t mode, hipStream_t stream) {
  return block_bwd(prob, q, q_chunk, k, v, kv_chunk, dout, lse, delta, nullptr, dk, dv, 1, mode,
                   stream);
}

ra_status_t ra_block_attn_bwd_dq(const ra_problem_t* prob, const void* q, int32_t q_chunk,
                                 const void* k, const void* v, int32_t kv_chunk, const void* dout,
                                 const float* lse, const float* delta, float* dq, int32_t mode,
                                 hipStream_t stream) {
  return block_bwd(prob, q, q_chunk, k, v, kv_chunk, dout, lse, delta, dq, nullptr, nullptr, 2,
                   mode, stream);
}

ra_status_t ra_ring_bwd_workspace_size(const ra_problem_t* prob, size_t* bytes) {
  RA_TRY(check_problem(prob));
  if (bytes == nullptr) return fail(RA_ERR_NULL, "bytes is NULL");
  const int64_t L = prob->seq_total / prob->world;
  *bytes = (size_t)(prob->batch * prob->heads_q * L * 4);
  return ok();
}

ra_status_t ra_ring_bwd(const ra_problem_t* prob, int32_t rank, const void* q,
                        const void* const* k_chunks, const void* const* v_chunks,
                        const void* out, const void* dout, const float* lse, float* dq,
                        float* const* dk_chunks, float* const* dv_chunks, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  RA_TRY(check_problem(prob));
  RA_TRY(bwd_supported(prob));
  RA_TRY(check_chunk(prob, rank, "rank"));
  RA_TRY(check_ptr(q, "q"));
  RA_TRY(check_ptr(out, "out"));
  RA_TRY(check_ptr(dout, "dout"));
  RA_TRY(check_ptr(dq, "dq"));
  if (lse == nullptr) return fail(RA_ERR_NULL, "lse is NULL");
  if (k_chunks == nullptr || v_chunks == nullptr || dk_chunks == nullptr || dv_chunks == nullptr)
    return fail(RA_ERR_NULL, "chunk array is NULL");
  for (int c = 0; c < prob->world; ++c) {
    RA_TRY(check_ptr(k_chunks[c], "k_chunks[c]"));
    RA_TRY(check_ptr(v_chunks[c], "v_chunks[c]"));
    RA_TRY(check_ptr(dk_chunks[c], "dk_chunks[c]"));
    RA_TRY(check_ptr(dv_chunks[c], "dv_chunks[c]"));
  }
  size_t need = 0;
  RA_TRY(ra_ring_bwd_workspace_size(prob, &need));
  if (ws == nullptr || ws_bytes < need)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (((uintptr_t)ws & 255u) != 0) return fail(RA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const ra::LayoutMap m = make_map(prob);
  float* delta = (float*)ws;
  const int64_t L = prob->seq_total / prob->world, D = prob->head_dim_padded;
  RA_TRY(ra_bwd_delta(prob, out, dout, delta, stream));
  // Every chunk is visited once, so its dK, dV are stored (not added) by its step; dQ is
  // stored by the first live step and added by the others.  Buffers no step reaches are
  // zero-filled.
  bool dq_written = false;
  hipError_t e = hipSuccess;
  for (int s = 0; s < prob->world && e == hipSuccess; ++s) {
    const int c = ((rank - s) % prob->world + prob->world) % prob->world;
    if (!step_live(prob, m, rank, c)) {
      const int64_t n = prob->batch * prob->heads_kv * L * D;
      e = ra::launch_fill_f32(dk_chunks[c], n, 0.0f, stream);
      if (e == hipSuccess) e = ra::launch_fill_f32(dv_chunks[c], n, 0.0f, stream);
      continue;
    }
    ra::BwdArgs a = bwd_args(prob, q, rank, k_chunks[c], v_chunks[c], c, dout, lse, delta, dq,
                             dk_chunks[c], dv_chunks[c]);
    a.write = 1;
    e = ra::launch_bwd(prob->dtype, (int)D, a, 1, stream);
    if (e != hipSuccess) break;
    a.write = dq_written ? 0 : 1;
    e = ra::launch_bwd(prob->dtype, (int)D, a, 2, stream);
    dq_written = true;
  }
  if (e == hipSuccess && !dq_written)
    e = ra::launch_fill_f32(dq, prob->batch * prob->heads_q * L * D, 0.0f, stream);
  if (e != hipSuccess) return hip_fail(e, "ra_ring_bwd launch");
  return ok();
}

ra_status_t ra_ring_bwd_noalloc(const ra_problem_t* prob, int32_t rank, const void* q,
                                const void* const* k_chunks, const void* const* v_chunks,
                                const void* out, const void* dout, const float* lse, float* dq,
                                float* const* dk_chunks, float* const* dv_chunks,
                                hipStream_t stream) {
  RA_TRY(check_problem(prob));
  size_t need = 0;
  RA_TRY(ra_ring_bwd_workspace_size(prob, &need));
  if (need > ra::kStaticScratchBytes)
    return fail(RA_ERR_WORKSPACE,
                "needs %zu bytes of workspace; the static scratch holds %zu "
                "(batch * heads_q * L <= %zu)",
                need, ra::kStaticScratchBytes, ra::kStaticScratchBytes / sizeof(float));
  void* ws = nullptr;
  const hipError_t e = ra::static_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "ra_ring_bwd_noalloc: static scratch address");
  return ra_ring_bwd(prob, rank, q, k_chunks, v_chunks, out, dout, lse, dq, dk_chunks,
                     dv_chunks, ws, ra::kStaticScratchBytes, stream);
}

}  // extern "C"
