/*
 * fa.h - C ABI of the exact attention forward for AMD MI355X (gfx950).
 *
 * Operation.  For every batch b, query head h and query row i:
 *
 *     O[b,h,i,:] = sum_j softmax_j(scale * Q[b,h,i,:] . K[b,g,j,:]) * V[b,g,j,:]
 *     lse[b,h,i] = ln( sum_j exp(scale * Q[b,h,i,:] . K[b,g,j,:]) )
 *
 * over the allowed keys j, with g = h / (Hq / Hkv).  This is the attention
 * formula of the course page "FlashAttention: IO-aware attention kernel"
 * (section 3.1), computed the way its section 3.2 describes: each query tile
 * keeps a running maximum, a running normaliser and an output accumulator
 * on chip, streams K/V tiles and rescales by exp(m_old - m_new), dividing by
 * the normaliser once at the end (section 2's two-loop picture).  No score
 * or probability matrix is written to memory.  lse carries the row maximum
 * and row sum that the kyonqi FlashAttention walkthrough ("Flash Attention
 * Backward") keeps for a backward pass, folded into one number per row.
 *
 * Masking.  causal = 0: every key 0 <= j < N_kv is allowed.  causal != 0:
 * key j is allowed for query i iff j <= i, with literal indices (top-left
 * alignment when N_q != N_kv; key 0 is always allowed, so no row is empty).
 *
 * Layout.  All tensors dense, row-major, head dimension fastest:
 *     q   [B, Hq,  N_q,  d]   dtype
 *     k,v [B, Hkv, N_kv, d]   dtype
 *     o   [B, Hq,  N_q,  d]   dtype (rounded to nearest even from fp32)
 *     lse [B, Hq,  N_q]       float32
 * q, k, v, o must be 16-byte aligned device pointers, lse 4-byte aligned.
 * o and lse must not overlap q, k or v (or each other).
 *
 * Arithmetic.  dtype FA_BF16 / FA_F16: products on the bf16/f16 matrix
 * cores with fp32 accumulation; probabilities are rounded to the input
 * dtype (round to nearest even) before the P*V product, and the normaliser
 * sums those rounded values in fp32 (O is an exact convex combination of V
 * rows with the rounded weights).  dtype FA_F32: fp32 matrix cores,
 * no intermediate rounding below fp32.
 *
 * Ownership.  The caller allocates and owns every buffer.  The library
 * allocates no device or host memory, keeps no pointer after a call returns
 * and holds no state besides per-kernel attributes set once.
 *
 * Errors.  Every entry point returns an fa_status.  All arguments are
 * validated on the host before any HIP call; an invalid call returns its
 * error code without touching the device.  FA_ERR_HIP reports a launch or
 * runtime error; fa_status_string(FA_ERR_HIP) then names the HIP error of
 * the calling thread's last failing call.  Launches are asynchronous: a
 * fault inside the kernel surfaces at the caller's next synchronisation.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL_PTR = 1,   /* a required pointer is NULL                        */
    FA_ERR_BAD_DIM = 2,    /* a dimension < 1, or too large (see fa_fwd)         */
    FA_ERR_HEAD_GROUP = 3, /* Hq is not a multiple of Hkv                        */
    FA_ERR_HEAD_DIM = 4,   /* d is not 64 or 128                                 */
    FA_ERR_DTYPE = 5,      /* dtype is not one of fa_dtype                       */
    FA_ERR_SCALE = 6,      /* scale is NaN or infinite                           */
    FA_ERR_ALIGN = 7,      /* a pointer is misaligned                            */
    FA_ERR_HIP = 8,        /* the HIP runtime reported an error                  */
    FA_ERR_ALIAS = 9,      /* o, lse or a workspace overlaps an input or another */
    FA_ERR_WORKSPACE = 10  /* workspace too small (or scratch too small: _noalloc) */
} fa_status;

typedef enum fa_dtype {
    FA_F32 = 0,
    FA_F16 = 1,
    FA_BF16 = 2
} fa_dtype;

/*
 * Exact attention forward, launched on the null (default) stream.
 * scale is applied as given (callers usually pass 1/sqrt(d)); any finite
 * value is accepted, including 0 and negative values.  Scores are formed in
 * fp32 as |scale| * log2(e) * (q . k), so every such product must stay
 * finite in fp32 (|scale * q . k| below about 2.3e38); beyond that the
 * outputs are undefined (the inputs decide it, so it is not checked).
 * Size limits (FA_ERR_BAD_DIM beyond them): one head of q or k/v, plus 256
 * rows, must stay below 2 GiB ((max(N_q, N_kv) + 256) * d * elem_size <
 * 2^31), B*Hq and B*Hkv below 2^31, and the grid below 2^31 workgroups.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int N_q, int N_kv, int d,
           float scale, int causal, int dtype);

/* Same as fa_fwd, launched on the given hipStream_t (NULL = null stream). */
int fa_fwd_stream(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int N_q, int N_kv, int d,
                  float scale, int causal, int dtype, void* stream);

/*
 * Host-only argument check used by both entry points: returns the status
 * fa_fwd would return for these arguments before launching (FA_OK when they
 * are valid).  Makes no HIP call.
 */
int fa_check_args(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, int B, int Hq, int Hkv, int N_q, int N_kv,
                  int d, float scale, int causal, int dtype);

/* Static description of a status code (FA_ERR_HIP adds the HIP error text). */
const char* fa_status_string(int status);

/*
 * Launch geometry the library uses for these arguments: query rows per
 * workgroup, keys per K/V tile, threads per workgroup, workgroups in the
 * grid and bytes of LDS per workgroup.  Returns an fa_status like
 * fa_check_args (pointers are not inspected).  Makes no HIP call.
 */
int fa_launch_info(int B, int Hq, int Hkv, int N_q, int N_kv, int d, int causal,
                   int dtype, int* rows_per_block, int* keys_per_tile,
                   int* threads_per_block, long long* blocks, int* lds_bytes);

/*
 * FP8 forward: the same operation, masking and layouts with 8-bit inputs,
 * the FlashAttention-3 direction named by the course page "FlashAttention:
 * IO-aware attention kernel" (section 3.3) and the omica exam notes (section
 * 4.5).  q, k and v hold codes of the OCP 8-bit floating point format, E4M3
 * variant (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest
 * finite 448, NaN codes 0x7F/0xFF, no infinities), one byte per element, in
 * the layouts of fa_fwd; the element value is code * descale_<tensor>:
 *
 *     O   = softmax(scale * (descale_q Q)(descale_k K)^T) (descale_v V)
 *     lse = its per-row logsumexp (natural log, fp32)
 *
 * o is written in bf16 [B, Hq, N_q, d], lse in fp32 [B, Hq, N_q].
 *
 * Arithmetic: Q K^T on the 8-bit matrix cores (exact products, fp32
 * accumulators; the instruction adds its 64 products with somewhat less than
 * fp32 precision); probabilities in fp32, rounded to E4M3 (round to nearest
 * even) for the P V product; the normaliser is the sum of those rounded
 * probabilities, so O is a convex combination of V rows.  The probabilities
 * of each 64-key tile are rounded relative to that tile's own power-of-two
 * reference (its largest probability lies in (1/2, 1]) and carried to the
 * row's common reference by an exact power-of-two block scale of the matrix
 * instruction.  The E4M3 rounding of P is the dominant error: relative 2^-4
 * per probability in E4M3's normal range, which also bounds the relative
 * error of the summed probabilities that lse is taken from.  Limits: a
 * probability below 2^-10 of the largest one of its tile is flushed to zero
 * (in the subnormal range, above that, the absolute error is at most 2^-10
 * of the tile's reference), so within one tile keys far below the tile's
 * strongest key lose their weight, while keys in other tiles keep theirs
 * however far below the row's maximum they lie; a tile whose weight is below
 * 2^-127 of the row's reference is dropped.  A long row with one dominant
 * key therefore keeps the summed mass of all its other tiles.
 *
 * scale: any finite value.  descale_q, descale_k, descale_v: finite and
 * > 0 (FA_ERR_SCALE otherwise).  d: 64 or 128.  Size limits as fa_fwd with
 * 2-byte elements.  q, k, v, o 16-byte aligned, lse 4-byte aligned
 * (FA_ERR_ALIGN); o and lse overlap no input or each other (FA_ERR_ALIAS).
 * One launch on `stream` (NULL = null stream); the library allocates nothing.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int N_q, int N_kv, int d,
               float scale, int causal,
               float descale_q, float descale_k, float descale_v, void* stream);

/*
 * Split-KV forward (FlashDecoding).  Same operation, arguments, layouts,
 * masking and rounding as fa_fwd, for shapes with few query rows per
 * key/value head, above all decoding (N_q = 1).  The course page
 * "FlashAttention: IO-aware attention kernel" (section 3, where the method
 * helps and where it does not; sections 8 and 9) names this decode variant,
 * FlashDecoding: it parallelises over the key/value length to fill the GPU.
 * Here the keys of every (batch, key/value head) are dealt into num_splits
 * chunks: with tiles of 32 keys, chunk s holds tiles s, s + num_splits,
 * s + 2*num_splits, ... (interleaved, so that concurrent chunks read
 * neighbouring memory); each chunk yields
 * the exact attention of its rows over that chunk alone (output O_s and
 * lse_s); a second launch merges them with the block merge rule of the
 * omica exam notes (section 2.3), written for normalised partials:
 *
 *     lse = ln sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) * O_s
 *
 * which equals attention over all keys.  For a decoding step pass causal = 0
 * (the new query sees every cached key; causal masking keeps the literal
 * j <= i convention of fa_fwd).  Chunks with no allowed key of a
 * row contribute nothing (lse_s = -inf).  The query heads that share a
 * key/value head are processed together: rows (h, i) of one group form one
 * sequence of Hq/Hkv * N_q "packed" rows, 32 per wave.
 *
 * dtype FA_BF16 or FA_F16 only (FA_ERR_DTYPE for FA_F32); d 64 or 128.
 * 1 <= num_splits <= min(ceil(N_kv / 32), FA_SPLITKV_MAX_SPLITS), else
 * FA_ERR_BAD_DIM.
 *
 * workspace: caller-owned device memory of at least
 * fa_splitkv_workspace_bytes(B, Hq, N_q, d, num_splits) bytes (FA_ERR_WORKSPACE
 * otherwise), 16-byte aligned (FA_ERR_ALIGN), not overlapping q, k, v, o or
 * lse (FA_ERR_ALIAS).  It holds the chunk results in fp32,
 *     O_s   [num_splits][B*Hq*N_q][d]   then
 *     lse_s [num_splits][B*Hq*N_q],
 * row index (b*Hq + h)*N_q + i, and is fully rewritten by every call; its
 * previous contents do not matter.  Both launches go to `stream` (NULL = null
 * stream); calls that share a workspace must be ordered on one stream.
 * The library itself still allocates nothing.
 */
#define FA_SPLITKV_MAX_SPLITS 256

size_t fa_splitkv_workspace_bytes(int B, int Hq, int N_q, int d, int num_splits);

/* A split count for these sizes that fills the GPU (about 2048 waves), with
 * at least 4 tiles per chunk; 0 when the sizes are invalid for fa_fwd_splitkv. */
int fa_splitkv_default_splits(int B, int Hq, int Hkv, int N_q, int N_kv, int d, int dtype);

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N_q, int N_kv, int d,
                   float scale, int causal, int dtype, int num_splits,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free form of fa_fwd_splitkv, for callers that cannot allocate
 * or hand over device memory at call time: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same operation,
 * arguments (minus the workspace), checks, kernels and result as
 * fa_fwd_splitkv: for the same inputs and num_splits the outputs are
 * bitwise identical.
 *
 * The chunk results go to a device array inside the library instead of a
 * caller workspace: FA_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, part of the
 * library's code object, held until the process ends.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a device looks up that device's copy of the array once.  Sizes
 * whose fa_splitkv_workspace_bytes(B, Hq, N_q, d, num_splits) exceeds
 * FA_NOALLOC_SCRATCH_BYTES return FA_ERR_WORKSPACE before any HIP call (e.g.
 * a decoding step of B = 8, Hq = 28, N_q = 1, d = 128 fits up to 145 splits).
 *
 * The array belongs to the GPU that `stream` runs on (NULL: the current
 * device); q, k, v, o and lse must be on that GPU.  Every call on one GPU
 * shares its array, which keeps the last call's contents; each call rewrites
 * every part it later reads, so nothing needs clearing.  Calls that overlap
 * in time on one GPU (different streams, or different host threads without
 * ordering) race on the array and give wrong results: order them on one
 * stream.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16 << 20)

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int N_q, int N_kv, int d,
                           float scale, int causal, int dtype, int num_splits, void* stream);

/*
 * Split-KV forward over paged K/V caches, for serving.  The course page
 * "FlashAttention: IO-aware attention kernel" (section 4, reading vLLM's
 * flash-attention backend) has the serving engine hand the kernel the query,
 * a paged K/V cache and its block tables.  Each sequence's keys live in
 * fixed-size blocks of a shared pool:
 *
 *     k_cache, v_cache  [num_blocks][block_size][Hkv][d]   dtype
 *     block_table       [B][max_blocks_per_seq]            int32
 *     seqlens_k         [B]                                int32
 *
 * key j of sequence b is slot j % block_size of block
 * block_table[b][j / block_size] (the cache layout vLLM's flash-attention
 * backend passes).  Only entries for j < seqlens_k[b] are read; keys, table
 * entries and lengths live in device memory and are read by the kernels, so
 * a caller can rewrite them between launches without any host work.
 *
 *     q [B][Hq][N_q][d], o [B][Hq][N_q][d] (dtype), lse [B][Hq][N_q] (fp32)
 *
 * The N_q queries of sequence b are its last N_q positions: with causal != 0
 * query i sees key j iff j <= seqlens_k[b] - N_q + i (decoding: N_q = 1 sees
 * every key either way).  A row that sees no key (seqlens_k[b] <= 0, or an
 * early query of a short sequence) gets O = 0 and lse = -inf.  Values of
 * seqlens_k above max_blocks_per_seq * block_size are taken as that maximum,
 * and block numbers outside [0, num_blocks) are clamped into it: a bad table
 * gives wrong values, never an access outside the caches.
 *
 * Work split, chunk results and merge: those of fa_fwd_splitkv, with N_kv =
 * max_blocks_per_seq * block_size for the split count and workspace size
 * (fa_splitkv_workspace_bytes, fa_splitkv_default_splits).  dtype FA_BF16 or
 * FA_F16; d 64 or 128; block_size a power of two in [16, 65536]; each cache
 * below 4 GiB (num_blocks * block_size * Hkv * d * elem_size < 2^32 - 4096)
 * and B * max_blocks_per_seq < 2^31, else FA_ERR_BAD_DIM.  q, the caches,
 * o and the workspace 16-byte aligned; lse, block_table and seqlens_k
 * 4-byte aligned (FA_ERR_ALIGN).  o, lse and the workspace overlap no input
 * and each other (FA_ERR_ALIAS).  Two launches on `stream`; the library
 * allocates nothing.
 */
int fa_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                 const int* block_table, const int* seqlens_k, void* o, float* lse,
                 int B, int Hq, int Hkv, int N_q, int d,
                 int num_blocks, int block_size, int max_blocks_per_seq,
                 float scale, int causal, int dtype, int num_splits,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass: gradients of the scalar sum(O * dO) with respect to q, k
 * and v, for the forward above (same arguments, layouts and masking), by
 * recomputation as the kyonqi walkthrough ("Flash Attention Backward") and
 * the omica exam notes (section 2.5) describe it: the forward's o and lse are
 * inputs, and S and P = exp(scale * q.k - lse) are formed again tile by tile,
 * never stored.  With D = rowsum(dO * O):
 *
 *     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
 *     dQ = scale * dS K,  dK = scale * dS^T Q,
 *
 * dK and dV of a key/value head summing over its Hq/Hkv query heads.
 *
 * Inputs q, k, v, o, dout (dtype) and lse (fp32) as the forward wrote them;
 * outputs dq [B,Hq,N_q,d], dk and dv [B,Hkv,N_kv,d] in the same dtype
 * (products on the matrix cores, fp32 accumulation, P and dS rounded to the
 * dtype before their products, one rounding of each output).  dtype FA_BF16
 * or FA_F16 (FA_ERR_DTYPE for FA_F32); d 64 or 128; any finite scale.
 *
 * workspace: caller-owned device memory of at least
 * fa_bwd_workspace_bytes(B, Hq, Hkv, N_q, N_kv, d) bytes, 16-byte aligned,
 * fully rewritten by every call: 8 bytes per query row (lse * log2(e) and D
 * in fp32) and, when the key/value pass deals the query heads of a group
 * over several workgroups (few key/value heads), their fp32 partial dK and
 * dV, which a fourth launch sums in a fixed order.
 * dq, dk, dv and the workspace must not overlap any input or each other
 * (FA_ERR_ALIAS); pointer alignment as for fa_fwd (FA_ERR_ALIGN).  Three or
 * four launches on `stream` (NULL = null stream): the row pass, the dK/dV
 * pass, its reduction when used, the dQ pass.  Every output element is written once, by one wave: the
 * result is deterministic.  The library allocates nothing.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int N_q, int N_kv, int d);

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv,
           int B, int Hq, int Hkv, int N_q, int N_kv, int d,
           float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
