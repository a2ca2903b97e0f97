/*
 * libfa -- exact tiled attention (the FlashAttention forward pass) for AMD gfx950.
 *
 * The operation. For every batch entry b, query head h and query token i:
 *
 *     s_ij   = scale * dot(Q[b, h, i, :], K[b, hk, j, :])      for every key j visible to i
 *     O[b, h, i, :] = sum_j exp(s_ij - m_i) V[b, hk, j, :] / sum_j exp(s_ij - m_i)
 *     LSE[b, h, i]  = m_i + ln(sum_j exp(s_ij - m_i)),           m_i = max_j s_ij
 *
 * with hk = h / (heads_q / heads_kv); a query that sees no key at all gets O = 0 and
 * LSE = -inf. That is softmax(scale * Q K^T) V, the self-attention of the
 * "Flash Attention" notes (14cs17, sections "Prerequisites" and "Standard Attention Memory
 * Analysis"), computed tile by tile with the online softmax of that page's Theorem 2 and the
 * algorithm of its section "Flash Attention Algorithm": blocks of queries stay on chip while
 * blocks of keys and values stream past, and neither the N x N scores S nor the probabilities
 * P are ever written to device memory (same page, "Complexity Analysis", Theorem 3). Grouped
 * query heads and variable sequence lengths are the FlashAttention-2 features listed in the
 * section "Flash Attention 2 Improvements". The log-sum-exp output, the causal mask, the head
 * grouping and the packed-sequence layout are not spelled out on the pages; the readings are:
 *   - causal: key j is visible to query i iff j <= i (positions inside the sequence);
 *   - queries and keys of different lengths (a query chunk against a key/value cache: the notes
 *     list the KV cache as composable with the method, section "Connection to the Broader
 *     Curriculum"; the xspy page "FlashAttention and chunked prefill mechanics", section 1,
 *     pairs it with chunked prefill): the Nq queries are the last Nq of the Nk key positions,
 *     so causal visibility is j <= i + (Nk - Nq). With Nq == Nk this is the rule above;
 *   - grouped heads: query heads [g*r, (g+1)*r) share key/value head g, r = heads_q / heads_kv;
 *   - packed sequences: tokens of sequence s occupy [cu_seqlens[s], cu_seqlens[s+1]) and attend
 *     only inside that range;
 *   - LSE is the natural logarithm of the row's sum of exp(scaled score).
 *
 * Arithmetic: fp16 or bf16 inputs; products and sums in fp32 on the matrix cores; the
 * probabilities are rounded to the input type (round to nearest even) before the P V product;
 * O is rounded to the input type (round to nearest even); LSE is fp32.
 *
 * Threading and memory: libfa allocates nothing and keeps no state (apart from the static
 * scratch array of fa_fwd_splitkv_noalloc and its per-device address table); every call only
 * enqueues work on the given HIP stream and returns. The caller owns every buffer.
 */
#ifndef LIBFA_FA_H
#define LIBFA_FA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 8

/* Element type of Q, K, V and O. */
typedef enum fa_dtype {
  FA_F16 = 0,  /* IEEE binary16 */
  FA_BF16 = 1, /* bfloat16 */
  FA_E4M3 = 2  /* Q, K, V in OCP FP8 E4M3 with per-(batch, head) descales; O in bfloat16 (see
                  "FP8" below; fa_fwd only) */
} fa_dtype;

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* a size is out of range, or the grid would not fit */
  FA_ERR_UNSUPPORTED = 3, /* head_dim not 64 or 128, unknown dtype, non-finite scale, or
                             a feature the dtype does not support */
  FA_ERR_ALIGN = 4,       /* a base pointer is not 16-byte aligned, a stride is not a
                             non-negative multiple of 8 elements, or a token stride is below
                             head_dim (overlapping rows) or above 2^23 elements */
  FA_ERR_GQA = 5,         /* heads_q is not a multiple of heads_kv */
  FA_ERR_VARLEN = 6,      /* cu_seqlens given with batch != 1, num_seqs < 1 or a bad max_seqlen;
                             cu_seqlens_k without cu_seqlens; or packed queries whose keys
                             differ in length without cu_seqlens_k */
  FA_ERR_ABI = 7,         /* struct_size does not match this library's fa_fwd_params */
  FA_ERR_LAUNCH = 8,      /* the HIP launch failed (the HIP error text is kept per thread) */
  FA_ERR_SCRATCH = 9      /* fa_fwd_splitkv_noalloc: the split partials would exceed
                             FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

/*
 * Arguments of one forward call. All pointers are device pointers except the struct itself.
 *
 * Layout: q is [batch, heads_q, seqlen, head_dim]; k and v are [batch, heads_kv, seqlen_k,
 * head_dim]; o is [batch, heads_q, seqlen, head_dim]. The last (head_dim) dimension is
 * contiguous; the other three are given by the *_stride arrays, in elements, in the order
 * (batch, head, token). lse is a contiguous fp32 array [batch, heads_q, seqlen].
 * Self-attention sets seqlen_k = seqlen.
 *
 * Packed variable-length sequences: pass cu_seqlens (device, int32, num_seqs + 1 non-decreasing
 * prefix sums with cu_seqlens[0] == 0 and cu_seqlens[num_seqs] == seqlen), batch == 1, and
 * max_seqlen >= every sequence's query count (it sizes the grid). Zero-length sequences are
 * allowed. The keys of sequence s are [cu_seqlens_k[s], cu_seqlens_k[s + 1]) of the packed
 * K and V (cu_seqlens_k[num_seqs] == seqlen_k), or, with cu_seqlens_k NULL, the same ranges as
 * its queries (then seqlen_k must equal seqlen). libfa never reads device memory on the host,
 * so it cannot check the cu_seqlens contents: they are the caller's promise. Without
 * cu_seqlens, num_seqs, max_seqlen and cu_seqlens_k are ignored.
 */
typedef struct fa_fwd_params {
  uint32_t struct_size;   /* must equal sizeof(fa_fwd_params) (see fa_params_size) */
  int32_t dtype;          /* fa_dtype */
  const void* q;
  const void* k;
  const void* v;
  void* o;                /* written in full for every valid token */
  float* lse;             /* written in full for every valid token */
  int32_t batch;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t seqlen;         /* tokens per batch entry; total packed tokens with cu_seqlens */
  int32_t head_dim;       /* 64 or 128 */
  int32_t causal;         /* non-zero: key j visible to query i iff
                             j <= i + (keys - queries) of its sequence */
  float scale;            /* any finite value; 1/sqrt(head_dim) is the usual choice */
  int32_t num_seqs;
  int32_t max_seqlen;
  const int32_t* cu_seqlens; /* NULL for fixed-length batches */
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  /* since ABI version 2 */
  int32_t seqlen_k;            /* key/value tokens per batch entry (total packed keys with
                                  cu_seqlens_k); may be 0: then every query sees no key and
                                  k, v may be NULL */
  int32_t reserved0;           /* must be 0 */
  const int32_t* cu_seqlens_k; /* packed key ranges, or NULL (see above) */
  /* since ABI version 5: rotary position embedding (RoPE, see below) */
  const float* rope_cos;       /* NULL: no rotation; else fp32 [rope_rows, head_dim / 2] */
  const float* rope_sin;       /* fp32 [rope_rows, head_dim / 2]; both or neither */
  int32_t rope_rows;           /* positions the tables hold (rows are 16-byte aligned) */
  int32_t rope_interleaved;    /* non-zero: pairs (2i, 2i + 1); zero: pairs (i, i + head_dim/2) */
  void* k_rot;                 /* NULL: K holds keys that are already rotated; else the rotated
                                  keys are written here ([batch, heads_kv, seqlen_k, head_dim]
                                  with k_rot_stride; may be k itself with k's strides) and
                                  attention reads them */
  int64_t k_rot_stride[3];
  /* since ABI version 6: FP8 descales (FA_E4M3 only; NULL means 1 for every head) */
  const float* q_descale;      /* fp32 [batch, heads_q] */
  const float* k_descale;      /* fp32 [batch, heads_kv] */
  const float* v_descale;      /* fp32 [batch, heads_kv] */
} fa_fwd_params;

/*
 * RoPE. The "Flash Attention" notes list rotary position embedding among FlashAttention-2's
 * features ("Flash Attention 2 Improvements"). With rope_cos and rope_sin given, attention runs
 * on rotated Q and K: pair i of a row at position p becomes (a c - b s, a s + b c) with
 * c = rope_cos[p][i], s = rope_sin[p][i] (the standard tables hold cos and sin of
 * p * 10000^(-2i/head_dim); any tables are accepted). Positions count inside each sequence:
 * key j is at position j, and the queries are the last positions of the keys (query t of Nq
 * against Nk keys at Nk - Nq + t; below 0 taken as 0), so the causal alignment and the rotation
 * agree. Each rotated element is formed in fp32 as two rounded products and their rounded
 * difference or sum (no fused multiply-add), then rounded to the input type (round to nearest
 * even). Q is rotated as it is loaded; K is rotated once by a separate streaming kernel into
 * k_rot (each key tile is read by many query blocks, so rotating it there would repeat the
 * work), unless k_rot is NULL, in which case K is taken as already rotated (a cache of rotated
 * keys). Table rows must cover every key position: with cu_seqlens this is the caller's promise
 * (positions beyond the tables use the last row; nothing is read out of bounds), otherwise
 * rope_rows >= seqlen_k is checked. Errors: FA_ERR_NULL for one table without the other or
 * k_rot without tables; FA_ERR_ALIGN for a table not 16-byte aligned or a bad k_rot layout;
 * FA_ERR_SHAPE for too few table rows. The backward pass takes no RoPE arguments.
 */

/*
 * FP8 (dtype FA_E4M3). FP8 matrix cores are FlashAttention-3's second lever (xspy page
 * "FlashAttention and chunked prefill mechanics", section 1); the pages give no recipe, and
 * the one here is: Q, K, V hold E4M3 codes (OCP: bias 7, 3 mantissa bits, largest 448, no
 * infinities), and the tensor a code stands for is its value times the fp32 descale of its
 * (batch, head). The output is attention on those values: O in bfloat16 (o_stride in bf16
 * elements), LSE in fp32. S = Q K^T is formed on the E4M3 matrix instructions, whose own sum
 * of 64 products errs by up to about 2^-11 of the largest product (measured); the
 * probabilities are shifted by 2^8, scaled per block of 32 keys by a power of two (the
 * instruction's E8M0 block scale undoes it) and rounded to E4M3 before the P V product, so
 * |dO| <= max|v| (2^-4 + keys 2^-18 + 2^-12) per row beyond the score error and bf16
 * rounding; the log-sum-exp uses unrounded sums. Descales
 * must be finite (a negative product with scale flips the scores' sign, as a negative scale
 * does). Q, K, V strides are multiples of 16 elements (16 bytes). Not supported with FA_E4M3:
 * RoPE tables and fa_fwd_splitkv (FA_ERR_UNSUPPORTED).
 */

/*
 * Arguments of one backward call: the gradients dQ, dK, dV of the loss sum(O * dO) for the
 * forward pass above (self-attention: keys and queries of one length per sequence). The
 * backward recomputes S and P tile by tile from Q, K and the forward's LSE instead of storing
 * them ("Flash Attention" notes, Common Pitfalls, Pitfall 3; FromZero2AI page, "Core
 * Mechanisms", mechanism 3):
 *
 *     P = exp(scale Q K^T - LSE) on visible entries, D = rowsum(dO * O),
 *     dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,
 *
 * with the contributions of the query heads that share a key/value head summed.
 *
 * Layouts are those of fa_fwd_params: q, o, dout, dq are [batch, heads_q, seqlen, head_dim];
 * k, v, dk, dv are [batch, heads_kv, seqlen, head_dim]; head_dim contiguous, the other strides
 * in elements. lse is fa_fwd's output for the same q, k, v, scale and mask (contiguous fp32
 * [batch, heads_q, seqlen]). delta is a caller-owned contiguous fp32 workspace of two arrays of
 * that shape ([2, batch, heads_q, seqlen], 8 * batch * heads_q * seqlen bytes) that fa_bwd
 * overwrites: D in the first, -log2(e) * LSE in the second (the offset the dK/dV pass adds to
 * each scaled score); libfa allocates nothing. dq, dk, dv are written in full
 * for every valid token, rounded to the input type from fp32 accumulators. Calls that may run
 * at the same time need their own delta buffers.
 */
typedef struct fa_bwd_params {
  uint32_t struct_size;   /* must equal sizeof(fa_bwd_params) (see fa_bwd_params_size) */
  int32_t dtype;          /* fa_dtype */
  const void* q;
  const void* k;
  const void* v;
  const void* o;          /* fa_fwd's output */
  const void* dout;       /* dL/dO */
  const float* lse;       /* fa_fwd's log-sum-exp */
  float* delta;           /* workspace of 2 * batch * heads_q * seqlen floats, written */
  void* dq;
  void* dk;
  void* dv;
  int32_t batch;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t seqlen;
  int32_t head_dim;       /* 64 or 128 */
  int32_t causal;         /* non-zero: key j visible to query i iff j <= i */
  float scale;
  int32_t num_seqs;
  int32_t max_seqlen;
  int32_t reserved0;      /* must be 0 */
  const int32_t* cu_seqlens; /* NULL for fixed-length batches */
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  int64_t do_stride[3];
  int64_t dq_stride[3];
  int64_t dk_stride[3];
  int64_t dv_stride[3];
} fa_bwd_params;

/* FA_ABI_VERSION of the built library. */
int32_t fa_abi_version(void);

/* sizeof(fa_fwd_params) as compiled into the library. */
uint32_t fa_params_size(void);

/* Host-only argument validation (no device call): the checks fa_fwd performs first. */
fa_status fa_check_args(const fa_fwd_params* p);

/*
 * Enqueue the forward pass on `stream` (a hipStream_t; NULL means the default stream).
 * Returns FA_OK once the kernel is enqueued; argument errors are returned before any device
 * call. seqlen == 0 is a no-op returning FA_OK. Faults inside the kernel surface at the
 * caller's next synchronisation of the stream. NaN or Inf inputs are not checked and propagate.
 */
fa_status fa_fwd(const fa_fwd_params* p, void* stream);

/*
 * Split-KV forward: the outputs of fa_fwd (O and LSE, to rounding) for the same arguments,
 * organised for query chunks of a few tokens against a long key/value context (token-by-token
 * decode with a KV cache, the composition the "Flash Attention" notes name in "Connection to
 * the Broader Curriculum"). The query rows of every head that shares a kv head are packed into
 * one block, so each key/value tile is read once per head group, and the keys of every
 * (sequence, kv head) are divided into num_splits contiguous ranges that run as separate
 * workgroups. Each range keeps its own online-softmax state (Theorem 2 of the notes) and writes
 * a partial output normalised by its own sum, with its log-sum-exp, to `workspace`; a second
 * kernel merges the partials with the same rescaling rule. With one split the first kernel
 * writes O and LSE itself and no workspace is used. Any seqlen works, but for long query
 * chunks fa_fwd is the faster call.
 *
 * num_splits: 1 .. FA_MAX_SPLITS, or 0 for the library's choice from the shapes (the same
 * choice in both calls below). The choice is a function of the arguments only.
 */
#define FA_MAX_SPLITS 256

/*
 * Host only: resolves num_splits (into *splits, if not NULL) and the workspace bytes
 * fa_fwd_splitkv needs with it (into *workspace_bytes, if not NULL; 0 for one split).
 * Errors: those of fa_check_args; FA_ERR_SHAPE for num_splits outside [0, FA_MAX_SPLITS] or a
 * grid that would not fit.
 */
fa_status fa_splitkv_plan(const fa_fwd_params* p, int32_t num_splits, int32_t* splits,
                          uint64_t* workspace_bytes);

/*
 * Enqueue the split-KV forward on `stream`. workspace: caller-owned device memory, 16-byte
 * aligned, of at least the planned bytes (workspace_bytes gives its size); it may be NULL when
 * the plan needs none. Its contents on entry do not matter and on return are unspecified;
 * calls that may run at the same time need their own workspace. Errors: those of
 * fa_splitkv_plan; FA_ERR_NULL for a missing workspace, FA_ERR_ALIGN for a misaligned one,
 * FA_ERR_SHAPE for one that is too small; all before any device call.
 */
fa_status fa_fwd_splitkv(const fa_fwd_params* p, int32_t num_splits, void* workspace,
                         uint64_t workspace_bytes, void* stream);

/*
 * fa_fwd_splitkv for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments, kernels and results as
 * fa_fwd_splitkv, but the split partials go to a static device array that the library holds
 * (one per GPU, FA_NOALLOC_SCRATCH_BYTES, kept until the process ends) instead of a caller
 * workspace; the call itself allocates nothing. The caller still owns q, k, v, o, lse (and
 * k_rot). The array's device address is looked up on the first call on each device (with that
 * device current; the stream must belong to the current device).
 *
 * Every call on one GPU shares its array and overwrites it: calls that may overlap on one GPU
 * (different streams, or different host threads without ordering) race and can corrupt each
 * other's results; order them on one stream. Nothing in the array has to start at zero, and
 * no earlier contents reach an output.
 *
 * Errors: those of fa_splitkv_plan; FA_ERR_SCRATCH when the planned workspace exceeds
 * FA_NOALLOC_SCRATCH_BYTES (splits x batch x heads_q x seqlen x (head_dim + 1) x 4 bytes), all
 * before any device call; FA_ERR_LAUNCH if the address lookup or a launch fails.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)
fa_status fa_fwd_splitkv_noalloc(const fa_fwd_params* p, int32_t num_splits, void* stream);

/* sizeof(fa_bwd_params) as compiled into the library. */
uint32_t fa_bwd_params_size(void);

/* Host-only argument validation of a backward call (no device call). */
fa_status fa_bwd_check_args(const fa_bwd_params* p);

/*
 * Enqueue the backward pass on `stream`: writes delta, then dK and dV, then dQ. Argument
 * errors are returned before any device call; seqlen == 0 is a no-op returning FA_OK.
 */
fa_status fa_bwd(const fa_bwd_params* p, void* stream);

/* Static text for a status code; for FA_ERR_LAUNCH, the HIP error of this thread's last
 * failed launch. Never NULL. */
const char* fa_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* LIBFA_FA_H */
