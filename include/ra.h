/*
 * ra.h -- C ABI of the blockwise ring-attention step for AMD MI355X (gfx950).
 *
 * One rank's query chunk is attended against the key/value chunks of a sequence
 * in ring order.  Each ring step is a tiled online softmax (running max and sum)
 * that emits a partial output and its log-sum-exp (LSE); partials are merged by
 * LSE, so the final result equals softmax(Q K^T * scale) V over the whole
 * sequence ("Ring Attention & Friends": "Flash Attention - Tiling with the
 * Softmax Rescaling Trick" and "Ring Attention"; Mosaic post, "How Ring Attention
 * Works"; ringmaster page, "Layout": ring/loop.py, ring/merge.py).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Shapes.  B = batch, Hq / Hkv = query / key-value heads (Hq % Hkv == 0, query
 *    head h reads KV head h / (Hq/Hkv)), S = total sequence, p = ring size,
 *    L = S / p tokens per chunk, D = head_dim_padded in {32, 64, 128}.
 *  * Tensors in the problem dtype (q, every k and v chunk, out, dout) are
 *    [B, H, L, D] with element strides (b, h, t) given in the problem and a unit
 *    stride along D; every row must start 16-byte aligned.  Columns
 *    head_dim..D-1 of q, k and v must be zero (storage padding).  Within one
 *    (b, h), (L + 256) rows at the t stride must span less than 4 GiB for q, the
 *    k/v chunks and out/dout (kernels address a head's rows with 32-bit offsets):
 *    RA_ERR_UNSUPPORTED otherwise.
 *  * fp32 buffers (partial/accumulated outputs o, dq, dk, dv) are contiguous
 *    [B, H, L, D]; lse and delta are contiguous [B, Hq, L].  LSE is the natural
 *    log of sum_j exp(scaled score); a row that sees no key has o = 0 and
 *    lse = -inf.
 *  * Positions.  Token t of chunk c has global position pos(c, t):
 *      RA_LAYOUT_CONTIGUOUS  c*L + t                    (dense shard)
 *      RA_LAYOUT_STRIPED     t*p + c                    (token i in chunk i mod p)
 *      RA_LAYOUT_ZIGZAG      with h = S/(2p): t < h -> c*h + t,
 *                            else (2p-1-c)*h + (t-h)    (head/tail balancing)
 *    (ringmaster page, "Layout": shard.py and balancers.py; "Ring Attention &
 *    Friends", "Striped Attention").  With causal != 0, key u of chunk k is
 *    visible to query t of chunk q iff pos(k, u) <= pos(q, t) (autoregressive,
 *    diagonal included).
 *  * Packed documents (optional; ringmaster page, "Native recurrent context
 *    parallelism": packed attention by global position boundaries, globally
 *    right-padded batches).  seg_bounds is a DEVICE array int32 [B, seg_count]
 *    of global positions 0 = e_0 <= e_1 <= ... <= e_{n-1} <= S per batch
 *    element (n = seg_count >= 2); document j is [e_j, e_{j+1}) (empty when
 *    equal; pad a shorter list by repeating its last entry).  A key is then
 *    visible only to queries of its own document (and causal as above).
 *    Positions >= e_{n-1} are right padding: no query sees them and they see no
 *    key (their output is 0, their lse -inf, they get no gradient).  The
 *    library cannot inspect device memory: a list that breaks these rules
 *    gives unspecified values but never an access outside the caller's
 *    buffers.  seg_bounds = NULL and seg_count = 0 mean one dense sequence.
 *  * Ownership.  The caller owns every buffer and the stream.  The library
 *    allocates nothing, keeps no pointer after returning, and holds no per-call
 *    state; calls on distinct streams are independent.  The one exception is
 *    ra_ring_bwd_noalloc: its calls on one GPU share a static device array (see
 *    its declaration).
 *  * Errors.  Every argument is validated before anything is enqueued; on
 *    failure nothing is written and the status plus ra_last_error() (a
 *    thread-local message) say why.  RA_OK means "enqueued": device faults
 *    surface at the next synchronisation of the stream.  Unsupported inputs are
 *    rejected up front, as the ringmaster page does for inputs it cannot handle
 *    ("Native recurrent context parallelism": left padding, holes and arbitrary
 *    masks are rejected).
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ra_status_t {
  RA_OK = 0,
  RA_ERR_NULL = 1,        /* a required pointer is NULL */
  RA_ERR_SHAPE = 2,       /* sizes, strides, alignment or chunk ids are inconsistent */
  RA_ERR_UNSUPPORTED = 3, /* valid but not implemented (dtype, head dim, mode) */
  RA_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  RA_ERR_HIP = 5          /* a HIP runtime call failed at enqueue time */
} ra_status_t;

typedef enum ra_layout_t {
  RA_LAYOUT_CONTIGUOUS = 0,
  RA_LAYOUT_ZIGZAG = 1,
  RA_LAYOUT_STRIPED = 2
} ra_layout_t;

typedef enum ra_dtype_t { RA_F32 = 0, RA_BF16 = 1 } ra_dtype_t;

typedef enum ra_mode_t {
  RA_WRITE = 0, /* write the step's normalised partial o and its lse */
  RA_MERGE = 1  /* LSE-merge the step's partial into (o, lse) in place */
} ra_mode_t;

/* The problem one rank solves.  Plain data, copied by value into every launch. */
typedef struct ra_problem_t {
  int64_t batch;           /* 1 <= B < 2^31 */
  int64_t heads_q;         /* 1 <= Hq < 2^31 */
  int64_t heads_kv;        /* 1 <= Hkv < 2^31, Hq % Hkv == 0 */
  int64_t head_dim;        /* true d (1..D); sets the default scale */
  int64_t head_dim_padded; /* D in {32, 64, 128} (storage) */
  int64_t seq_total;       /* S; S % p == 0 (S % 2p == 0 for zigzag); S < 2^31;
                              batch * heads_q * (S/p + 256) < 2^31 (one launch) */
  int32_t world;           /* p >= 1 */
  int32_t layout;          /* ra_layout_t */
  int32_t causal;          /* 0 or 1 */
  int32_t dtype;           /* ra_dtype_t of q, k, v, out, dout */
  float scale;             /* 0 -> 1/sqrt(head_dim) */
  int32_t seg_count;       /* boundaries per batch element (>= 2), or 0: dense */
  int64_t q_stride[3];     /* (b, h, t) element strides of q; every stride in
                              [0, 2^48), a multiple of 16 bytes (RA_ERR_SHAPE) */
  int64_t kv_stride[3];    /* (b, h, t) element strides of every k and v chunk */
  int64_t o_stride[3];     /* (b, h, t) element strides of out and dout */
  const int32_t* seg_bounds; /* device int32 [B, seg_count] document boundaries, or NULL */
} ra_problem_t;

/*
 * One ring step, forward ("Ring Attention & Friends", "Flash Attention - Tiling
 * with the Softmax Rescaling Trick"; Mosaic post, "How Ring Attention Works").
 * q: [B, Hq, L, D] query chunk q_chunk.  k, v: [B, Hkv, L, D] KV chunk kv_chunk.
 * o: fp32 [B, Hq, L, D], lse: fp32 [B, Hq, L] (contiguous, caller-owned).
 * mode RA_WRITE: o, lse := the step's normalised partial output and its LSE
 *   (rows that see no key of this chunk get 0 and -inf).
 * mode RA_MERGE: (o, lse) := LSE-merge of (o, lse) with the step's partial; the
 *   first step of a ring either uses RA_WRITE or starts from (0, -inf).
 * The step's visible (query, key) tiles are computed from global positions and
 * tiles with no visible pair are skipped.
 */
ra_status_t ra_block_attn_fwd(const ra_problem_t* prob, const void* q, int32_t q_chunk,
                              const void* k, const void* v, int32_t kv_chunk, float* o,
                              float* lse, int32_t mode, hipStream_t stream);

/*
 * In-place LSE merge of two partial results over disjoint key sets (ringmaster
 * page, "Layout": ring/merge.py; Mosaic post, "How Ring Attention Works").
 * o_acc, o_part: fp32 [rows, d]; lse_acc, lse_part: fp32 [rows] (contiguous).
 *   lse := log(exp(lse_acc) + exp(lse_part))
 *   o   := o_acc * exp(lse_acc - lse) + o_part * exp(lse_part - lse)
 * A part with lse = -inf is the identity (the accumulator is left unchanged when
 * lse_part = -inf).  d in 4..1024, d % 4 == 0; rows in [0, 2^34); pointers
 * 16-byte aligned.
 */
ra_status_t ra_lse_merge(int64_t rows, int32_t d, float* o_acc, float* lse_acc,
                         const float* o_part, const float* lse_part, hipStream_t stream);

/* Bytes of device workspace ra_ring_fwd needs (fp32 accumulator [B, Hq, L, D]). */
ra_status_t ra_ring_workspace_size(const ra_problem_t* prob, size_t* bytes);

/*
 * The ring driver, forward, for rank `rank` (Mosaic post, "How Ring Attention
 * Works": at step s the rank holds KV chunk (rank - s) mod p, having received it
 * from rank - 1).  k_chunks[c] / v_chunks[c] is a HOST array of p device pointers
 * indexed by chunk id.  Steps with no visible (query, key) pair are skipped.
 * out: [B, Hq, L, D] in the problem dtype with o_stride; lse: fp32 [B, Hq, L].
 * ws: device workspace of at least ra_ring_workspace_size() bytes, 256-byte
 * aligned.  Partials are accumulated in fp32; out is rounded once at the end.
 */
ra_status_t ra_ring_fwd(const ra_problem_t* prob, int32_t rank, const void* q,
                        const void* const* k_chunks, const void* const* v_chunks, void* out,
                        float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward preprocess: delta[b, h, t] = sum_d dout[b, h, t, d] * out[b, h, t, d]
 * (fp32), from the final forward output of this rank (ringmaster page, "Status":
 * flash-style backward).  out, dout: [B, Hq, L, D] in the problem dtype, o_stride.
 */
ra_status_t ra_bwd_delta(const ra_problem_t* prob, const void* out, const void* dout,
                         float* delta, hipStream_t stream);

/*
 * One ring step, backward: recompute P = exp(S * scale - lse) from the FINAL
 * merged lse, then (ringmaster page, "Status": reverse-ring backward)
 *   dv += P^T dO,  dP = dO V^T,  dS = P o (dP - delta),
 *   dq += scale dS K,  dk += scale dS^T Q,
 * with dk, dv of a KV head summed over the query heads of its group.
 * dq: fp32 [B, Hq, L, D]; dk, dv: fp32 [B, Hkv, L, D]; all ACCUMULATED (+=) into
 * caller-initialised buffers.  lse, delta: fp32 [B, Hq, L].
 * Supported: bf16, D in {32, 64, 128}.
 */
ra_status_t ra_block_attn_bwd(const ra_problem_t* prob, const void* q, int32_t q_chunk,
                              const void* k, const void* v, int32_t kv_chunk, const void* dout,
                              const float* lse, const float* delta, float* dq, float* dk,
                              float* dv, hipStream_t stream);

/*
 * The two halves of ra_block_attn_bwd, for callers that schedule them apart (in a
 * multi-device ring dQ stays with the query owner while dK and dV travel with the
 * KV chunk).  Same arguments and layouts as ra_block_attn_bwd;
 * ra_block_attn_bwd_dkdv produces dk and dv only, ra_block_attn_bwd_dq dq only.
 * mode RA_MERGE adds the step's gradients into the buffers (as ra_block_attn_bwd);
 * mode RA_WRITE stores them, every element included (zeros where no pair is
 * visible), so the buffers need no zero-fill when this step is the first to reach
 * them (in a ring, every KV chunk is visited once; dq by every step).  Neither uses
 * atomics: each output element has one writer, so results are deterministic.
 */
ra_status_t ra_block_attn_bwd_dkdv(const ra_problem_t* prob, const void* q, int32_t q_chunk,
                                   const void* k, const void* v, int32_t kv_chunk,
                                   const void* dout, const float* lse, const float* delta,
                                   float* dk, float* dv, int32_t mode, hipStream_t stream);
ra_status_t ra_block_attn_bwd_dq(const ra_problem_t* prob, const void* q, int32_t q_chunk,
                                 const void* k, const void* v, int32_t kv_chunk, const void* dout,
                                 const float* lse, const float* delta, float* dq, int32_t mode,
                                 hipStream_t stream);

/*
 * Backward prologue of one rank (ringmaster page, "Status": flash-style,
 * reverse-ring backward): delta as in ra_bwd_delta, then zero-fills dq (fp32
 * [B, Hq, L, D]) and, for every chunk c < p, dk_chunks[c] and dv_chunks[c] (fp32
 * [B, Hkv, L, D]; HOST arrays of p device pointers), so the step kernels can
 * accumulate into them.  The fills are kernels of this library, not memset nodes,
 * so a caller may capture the call into a graph.  Every pointer must be 16-byte
 * aligned.  Errors: the problem checks of the other entry points, RA_ERR_NULL for
 * a NULL pointer and RA_ERR_SHAPE for a misaligned one, all before anything is
 * launched; RA_ERR_HIP for a failed launch.
 */
ra_status_t ra_bwd_prepare(const ra_problem_t* prob, const void* out, const void* dout,
                           float* delta, float* dq, float* const* dk_chunks,
                           float* const* dv_chunks, hipStream_t stream);

/* Bytes of device workspace ra_ring_bwd needs (fp32 delta [B, Hq, L]). */
ra_status_t ra_ring_bwd_workspace_size(const ra_problem_t* prob, size_t* bytes);

/*
 * The ring driver, backward, for rank `rank`: delta (as ra_bwd_delta) into ws,
 * then every step with a visible pair, in ring order: each KV chunk's dk/dv is
 * stored by its step (RA_WRITE), dq is stored by the first live step and added by
 * the others; buffers no live step reaches are zero-filled.  No output needs to be
 * initialised by the caller.  out / lse are the forward's results for this rank.
 * dk_chunks and dv_chunks are HOST arrays of p device
 * pointers (fp32 [B, Hkv, L, D]); the result is this rank's share of the
 * gradients (its queries only).  ws: at least ra_ring_bwd_workspace_size()
 * bytes, 256-byte aligned.  Supported: bf16.
 */
ra_status_t ra_ring_bwd(const ra_problem_t* prob, int32_t rank, const void* q,
                        const void* const* k_chunks, const void* const* v_chunks,
                        const void* out, const void* dout, const float* lse, float* dq,
                        float* const* dk_chunks, float* const* dv_chunks, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/*
 * ra_ring_bwd without a workspace argument, for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the fp32 delta workspace lives in a static device array of 16 MiB, so
 * batch * heads_q * L <= 4,194,304 (RA_ERR_WORKSPACE otherwise, before anything is
 * enqueued).  The call allocates nothing; each GPU holds its own copy of the array
 * until the process ends, and its device address is looked up on the first call on
 * that device.  Every call on one GPU shares that GPU's array: two calls that
 * overlap on one GPU (on different streams, or from different threads) race and
 * give unspecified gradients.  Other arguments, results and errors as ra_ring_bwd.
 */
ra_status_t ra_ring_bwd_noalloc(const ra_problem_t* prob, int32_t rank, const void* q,
                                const void* const* k_chunks, const void* const* v_chunks,
                                const void* out, const void* dout, const float* lse, float* dq,
                                float* const* dk_chunks, float* const* dv_chunks,
                                hipStream_t stream);

/* Host only.  host_out[t] = pos(chunk, t) for t in [0, L).  No device access. */
ra_status_t ra_positions(const ra_problem_t* prob, int32_t chunk, int64_t* host_out);

/*
 * Host only.  Exact number of visible (query, key) pairs per (batch, query head)
 * between query chunk q_chunk and KV chunk kv_chunk (L*L when not causal).
 * Dense problems only (seg_bounds == NULL): use ra_visible_pairs_packed otherwise.
 */
ra_status_t ra_visible_pairs(const ra_problem_t* prob, int32_t q_chunk, int32_t kv_chunk,
                             int64_t* pairs);

/*
 * Host only.  Exact number of visible (query, key) pairs per query head, summed
 * over the batch, between query chunk q_chunk and KV chunk kv_chunk of a packed
 * problem.  host_bounds: a HOST copy of the int32 [B, prob->seg_count] boundary
 * lists (prob->seg_bounds itself is not read); each list is validated
 * (starts at 0, nondecreasing, ends <= S: RA_ERR_SHAPE otherwise).
 */
ra_status_t ra_visible_pairs_packed(const ra_problem_t* prob, int32_t q_chunk,
                                    int32_t kv_chunk, const int32_t* host_bounds,
                                    int64_t* pairs);

/* Static string naming a status. */
const char* ra_status_str(ra_status_t status);

/* Thread-local message describing the last failure on this thread ("" if none). */
const char* ra_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
