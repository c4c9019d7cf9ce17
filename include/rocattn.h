/*
 * rocattn.h -- C ABI of the gfx950 (MI355X) causal attention library
 * (librocattn.so).
 *
 * The library computes, per batch b and query head hq,
 *
 *     O = softmax(scale * Q K^T + M) V                                   (1)
 *
 * with M the additive causal mask (0 where key j may be read by query row
 * i, -inf where it may not), on queries and keys that `rope_apply` has
 * rotated by position, and with several query heads sharing one K/V head.
 *
 * Sources (page title -- section):
 *   "Transformer" (ai-notes) -- Scaled dot-product attention:
 *       Attn(Q,K,V;M) = softmax(QK^T/sqrt(d_k) + M) V; What is the causal
 *       mask? (M[t,s] = 0 for s <= t, -inf otherwise); How to "kill" the
 *       sqrt(d_k) (an explicit temperature alpha may replace 1/sqrt(d_k));
 *       RoPE (theta_i(pos) = pos * 10000^(-2i/d_head)).
 *   "The Transformer architecture" -- Scaled dot-product attention
 *       (shapes, scale uses the per-head d_k); Now: RoPE (apply_rope with
 *       split-half pairing, cos/sin of shape (T, d/2)); What else the modern
 *       decoder-only model changed (GQA groups of n_rep query heads);
 *       Hands-on (with a cache, query row i sits at cache.pos + i and RoPE
 *       is sliced from cache.pos).
 *   "Transformer Math and Implementation Deep Dive" -- Attention Shapes
 *       (q: [B, n_q_heads, T, d_head], k/v: [B, n_kv_heads, T, d_head]).
 *   "Grasping Codes and Math 02" -- Flash Attention (one fused kernel that
 *       never materialises the T x T attention matrix).
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * Layout.  q and o are [B][Hq][Tq][d_head]; k and v are [B][Hkv][Tk][d_head];
 *   dense, row-major, d_head fastest.  o has q's element type.
 * Heads.  Query head hq reads K/V head hq / (Hq / Hkv) (contiguous groups,
 *   the grouping torch's repeat_interleave makes); Hq % Hkv must be 0.
 *   K/V are never replicated.
 * Causal rule.  With causal != 0, key j is visible to query row i iff
 *   j <= q_offset + i.  q_offset is the absolute position of the first
 *   query row: 0 for a plain prefill (Tq == Tk), Tk - Tq for a chunk of new
 *   rows appended to a cache, Tk - 1 for a one-token decode step.
 *   causal == 0 makes every key visible (q_offset is then ignored).
 * Pointers.  Device pointers (memory from hipMalloc or a torch CUDA tensor),
 *   each 16-byte aligned.  The caller owns every buffer; the library never
 *   frees or retains caller memory.  o must not overlap q, k or v.
 * Stream.  `stream` is a hipStream_t (NULL = the default stream).  Work is
 *   only enqueued: nothing synchronises, results are ready when the stream
 *   is, and a fault inside a kernel surfaces at the caller's next
 *   synchronisation, not in the returned status.
 * Errors.  Arguments are validated on the host before any launch; a
 *   rejected call launches nothing and writes nothing.  The status covers
 *   validation and launch errors only.
 * Threads.  Entry points are reentrant; the library keeps no state across
 *   calls apart from a per-device cache of the kernel properties it queries.
 */
#ifndef ROCATTN_H
#define ROCATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. */
typedef enum {
    ROCATTN_F32 = 0,   /* float32 in, float32 math, float32 out */
    ROCATTN_BF16 = 1   /* bfloat16 in, float32 accumulation, bfloat16 out (RNE) */
} rocattn_dtype;

/* Status codes (0 = success, negative = rejected or failed). */
typedef enum {
    ROCATTN_OK = 0,
    ROCATTN_ERR_NULL = -1,      /* a required pointer is NULL */
    ROCATTN_ERR_SHAPE = -2,     /* a size <= 0, Hq % Hkv != 0, overlap of o with an input,
                                   a tensor too large for 64-bit element offsets, or
                                   Tq + Tk > INT_MAX - 1024 (row/key limits are 32-bit) */
    ROCATTN_ERR_DTYPE = -3,     /* dtype not a rocattn_dtype */
    ROCATTN_ERR_HEADDIM = -4,   /* d_head not supported for this dtype / entry point */
    ROCATTN_ERR_OFFSET = -5,    /* causal with q_offset < 0: row 0 would see no key */
    ROCATTN_ERR_SCALE = -6,     /* scale (or RoPE base) not finite, or base <= 0 */
    ROCATTN_ERR_ALIGN = -7,     /* a pointer is not 16-byte aligned */
    ROCATTN_ERR_WORKSPACE = -8, /* workspace NULL or smaller than attn_workspace_bytes() */
    ROCATTN_ERR_HIP = -9        /* the HIP runtime reported an error while launching */
} rocattn_status;

/*
 * attn_fwd -- equation (1) for every (b, hq, query row).
 *
 *   q, k, v   inputs, layouts above; read only.
 *   o         output [B][Hq][Tq][d_head], fully overwritten.
 *   B, Hq, Hkv, Tq, Tk, d_head   sizes (all > 0, Hq % Hkv == 0).
 *   scale     multiplies q.k before the softmax; 1/sqrt(d_head) for standard
 *             attention, any finite value (a temperature; 0 gives the mean of
 *             the visible values).
 *   causal    non-zero: causal rule above; zero: no mask.
 *   q_offset  position of query row 0 (causal only; must be >= 0).  Any
 *             q_offset >= Tk - 1 makes every key visible to every row.
 *   dtype     rocattn_dtype of q, k, v and o.
 *   stream    hipStream_t.
 *
 * Supported head sizes: bf16 d_head in {64, 128}; f32 d_head <= 256 with
 * d_head % 4 == 0.  bf16 with Tq == 1 runs the split-K decode kernels, which
 * need a workspace, and a small bf16 prefill (fewer than 512 tiles of 128
 * query rows over all heads) is split over the keys when it has one:
 * attn_fwd takes attn_workspace_bytes() from the stream-ordered allocator
 * (hipMallocAsync / hipFreeAsync on `stream`); use attn_fwd_ws to pass one.
 * Returns a rocattn_status.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o,
             int B, int Hq, int Hkv, int Tq, int Tk, int d_head,
             float scale, int causal, int q_offset, int dtype, void* stream);

/*
 * attn_workspace_bytes -- bytes of device workspace attn_fwd_ws uses for
 * these sizes: required for a bf16 decode step (Tq == 1); for a small dense
 * bf16 prefill, optional (the partial results of its key splits, 4 (d + 2)
 * bytes per query row and split); 0 when the chosen kernels use none.  The
 * split count depends on the sizes only (not on q_offset or causal).
 * Returns 0 for arguments attn_fwd would reject.
 */
size_t attn_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int d_head, int dtype);

/*
 * attn_fwd_ws -- attn_fwd with a caller-owned workspace and an optional
 * log-sum-exp output.
 *
 *   workspace, ws_bytes  device buffer of at least attn_workspace_bytes()
 *             bytes (may be NULL when that is 0).  A bf16 decode step
 *             requires it (ERR_WORKSPACE); a small prefill uses it only when
 *             it is at least that large and otherwise runs unsplit (the two
 *             differ by float32 summation order, within the bf16 contract).
 *             Contents on entry are ignored and on return are unspecified.
 *             Calls that share a workspace must be ordered on one stream.
 *   lse       NULL, or float32 [B][Hq][Tq]: lse = log(sum_j exp(scale q_i.k_j))
 *             over the visible keys j (natural log), for a later backward
 *             pass or for merging partial attentions.
 * Other arguments and the result as attn_fwd.
 */
int attn_fwd_ws(const void* q, const void* k, const void* v, void* o,
                int B, int Hq, int Hkv, int Tq, int Tk, int d_head,
                float scale, int causal, int q_offset, int dtype, void* stream,
                void* workspace, size_t ws_bytes, float* lse);

/*
 * attn_fwd_noalloc -- attn_fwd_ws that allocates nothing, for callers that
 * cannot call hipMalloc: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Instead of a caller's workspace it
 * uses the library's fixed scratch buffer of the current device
 * (hipGetDevice; `stream` must belong to that device): 64 MiB of device
 * memory per GPU, a static array that each GPU the library runs on holds
 * until the process ends; its address is looked up once per device and no
 * allocating call (hipMalloc, hipMallocAsync, hipFree, torch) is made.
 *
 *   Arguments as attn_fwd_ws without workspace / ws_bytes; lse optional.
 *   A call whose required workspace (a bf16 decode step's partial results,
 *   attn_workspace_bytes()) exceeds 64 MiB is rejected with ERR_WORKSPACE
 *   before anything is launched; a small prefill uses the optional key
 *   splits when their partials fit, else runs unsplit.  Results are
 *   bit-identical to attn_fwd_ws with a workspace of attn_workspace_bytes()
 *   bytes whenever that is at most 64 MiB.
 *   Every call on one GPU shares its scratch buffer and leaves the last
 *   call's partial results in it: calls that overlap on one GPU (other
 *   streams, other host threads without ordering) race and must not be
 *   issued.  Returns a rocattn_status.
 */
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                     int B, int Hq, int Hkv, int Tq, int Tk, int d_head,
                     float scale, int causal, int q_offset, int dtype, void* stream, float* lse);

/*
 * attn_fwd_strided -- attn_fwd_ws on tensors laid out with arbitrary
 * batch / head / token strides, e.g. [B][T][H][d] ("BTHD") inputs sliced
 * from a fused projection and an output written straight in the
 * [B][T][H*d] order the heads are merged in ("Transformer Math and
 * Implementation Deep Dive" -- the transpose(1, 2).contiguous().view(B, T, C)
 * merge; "The Transformer architecture" -- Scaled dot-product attention,
 * y.transpose(1, 2)).
 *
 *   strides   host array of 12 element strides, in the order
 *             q(b, h, t), k(b, h, t), v(b, h, t), o(b, h, t); read during the
 *             call only.  The d_head elements of a row are contiguous.
 *             Element (b, h, t, c) of q is q[b*sq_b + h*sq_h + t*sq_t + c].
 *   other arguments as attn_fwd_ws; lse (if given) stays dense [B][Hq][Tq].
 *
 * Every stride is >= 0 and (stride * element size) % 16 == 0.  Inputs may
 * overlap each other (q, k and v may be views of one buffer, a zero stride
 * broadcasts); o's rows must not share elements (ordered by stride, each
 * level of size > 1 must step over the whole extent of the levels inside
 * it) and o's address range must not overlap the inputs' (ERR_SHAPE).
 * bf16 key and value token strides are at most 2^24 elements (ERR_SHAPE).
 * Results are bit-identical to attn_fwd_ws on the same values laid out
 * densely.  Returns a rocattn_status.
 */
int attn_fwd_strided(const void* q, const void* k, const void* v, void* o,
                     const long long* strides, int B, int Hq, int Hkv, int Tq, int Tk,
                     int d_head, float scale, int causal, int q_offset, int dtype,
                     void* stream, void* workspace, size_t ws_bytes, float* lse);

/*
 * rope_apply -- rotary position embedding, in place, on q and (optionally) k.
 *
 * Token t (0 <= t < T) sits at position pos0 + t (pos0 = cache.pos for a
 * cached step).  Channel pair p (0 <= p < d_head/2) is channels
 * (p, p + d_head/2) (split-half pairing) and turns by
 *     theta_p = (pos0 + t) * base^(-2p / d_head)
 * through [[cos, -sin], [sin, cos]]:
 *     x'[p]        = x[p] cos - x[p + d/2] sin
 *     x'[p + d/2]  = x[p] sin + x[p + d/2] cos.
 * The angle and its cosine and sine are formed in double precision and
 * rounded once to float32; the rotation runs in float32 and bf16 results are
 * rounded to nearest even.  Values are never rotated.
 *
 *   q         [B][Hq][T][d_head], rotated in place.
 *   k         [B][Hkv][T][d_head] rotated in place, or NULL (q only; Hkv is
 *             then ignored).  k may not overlap q (ERR_SHAPE); one launch
 *             turns both, sharing each (position, pair) angle.
 *   pos0      position of token 0 (>= 0).
 *   base      frequency base (10000 in the original schedule), finite, > 0.
 *   dtype     rocattn_dtype of q and k.
 * Supported: d_head even, 2 <= d_head <= 256.  Returns a rocattn_status.
 */
int rope_apply(void* q, void* k, int B, int Hq, int Hkv, int T, int d_head,
               int pos0, double base, int dtype, void* stream);

/* Channel pairing of rope_apply_ex. */
typedef enum {
    ROCATTN_ROPE_SPLIT_HALF = 0,   /* pair p = channels (p, p + d/2) */
    ROCATTN_ROPE_ADJACENT = 1      /* pair p = channels (2p, 2p + 1) */
} rocattn_rope_pairing;

/*
 * rope_apply_ex -- rope_apply with a choice of channel pairing: split-half
 * ("The Transformer architecture" -- Now: RoPE, apply_rope, the convention
 * rope_apply uses) or adjacent pairs (2p, 2p + 1) ("Transformer" (ai-notes)
 * -- RoPE, where each consecutive pair of channels is one plane).  The two
 * conventions differ by a fixed permutation of the channels, so a model must
 * use the one its weights were trained with.  Pair p turns by the same angle
 * theta_p in both:
 *     adjacent:  x'[2p] = x[2p] cos - x[2p+1] sin,  x'[2p+1] = x[2p] sin + x[2p+1] cos.
 * Other arguments, rounding and support as rope_apply; an unknown pairing
 * returns ROCATTN_ERR_SHAPE.
 */
int rope_apply_ex(void* q, void* k, int B, int Hq, int Hkv, int T, int d_head, int pos0,
                  double base, int dtype, void* stream, int pairing);

/*
 * rope_apply_pos -- rope_apply_ex with a position per token: token t of
 * sequence b sits at positions[b * T + t] (the pages take the angles from
 * the cache position onward, "The Transformer architecture" -- Hands-on;
 * here each sequence of a batch may sit at its own position, or a packed
 * row at any positions).  The angles and the rotation are rope_apply_ex's,
 * so positions[b][t] = pos0 + t gives rope_apply_ex's bits.
 *
 *   positions  device int32 [B][T], 4-byte aligned, read only; any values
 *              (the rotation is defined for every integer position).
 * Other arguments, rounding and support as rope_apply_ex; positions may not
 * overlap q or k (ERR_SHAPE).
 */
int rope_apply_pos(void* q, void* k, int B, int Hq, int Hkv, int T, int d_head,
                   const int* positions, double base, int dtype, void* stream, int pairing);

/*
 * attn_decode_step -- one cached generation step, Tn new tokens per
 * sequence ("The Transformer architecture" -- Hands-on: the new keys and
 * values are written into the cache along the token axis at cache.pos, RoPE
 * is sliced from cache.pos, and the new query rows sit at cache.pos + i;
 * "Transformer" (ai-notes) -- Notes on compute: with a KV cache each new
 * token costs one pass over the cached keys):
 *
 *   1. q (the new query rows) is rotated in place at positions pos + t;
 *   2. k_new is rotated at positions pos + t and written into k_cache at
 *      tokens pos .. pos + Tn - 1; v_new is copied into v_cache there;
 *   3. o = attention of the rotated q over cache tokens 0 .. pos + Tn - 1,
 *      causal, q_offset = pos (row i sees tokens <= pos + i).
 * bf16 with Tn == 1 (one new token per sequence, d_head 64 or 128, at
 * most 16 query heads per K/V head): the whole step is ONE launch -- the
 * split-K decode kernel rotates q as it loads it, the chunk of keys holding
 * pos rotates the new key, appends it and the new value and uses them, and
 * the last chunk of each (batch, K/V head) to finish merges the chunks'
 * partial results, writes o (and lse) and writes q back rotated.  Otherwise
 * steps 1-2 are one launch and step 3 is the attention of attn_fwd_ws (the
 * prefill kernel).
 *
 *   q         [B][Hq][Tn][d_head], rotated in place (read, then written).
 *   k_new, v_new  [B][Hkv][Tn][d_head], read only (k_new is not rotated in
 *             place: its rotated rows go to the cache).
 *   k_cache, v_cache  [B][Hkv][Tmax][d_head]; tokens pos .. pos + Tn - 1 are
 *             overwritten, tokens < pos are read, tokens >= pos + Tn are
 *             neither read nor written.
 *   o         [B][Hq][Tn][d_head], fully overwritten.
 *   pos       cache.pos: tokens already in the cache (0 <= pos, pos + Tn <= Tmax,
 *             else ERR_OFFSET).
 *   rope_base, pairing   as rope_apply_ex.
 *   scale, dtype, stream, lse   as attn_fwd_ws.
 *   workspace, ws_bytes  device buffer of at least
 *             attn_decode_step_workspace_bytes(B, Hq, Hkv, Tn, Tmax, d_head,
 *             dtype) bytes (enough for every pos; ERR_WORKSPACE when
 *             smaller).  For the one-launch step (bf16, Tn == 1) its last
 *             4 * B * Hkv bytes are arrival counters that MUST be zero before
 *             the first call with this workspace (clear them once after
 *             allocating, e.g. hipMemset); every call leaves them zero, so
 *             later steps need no clearing.  Calls that share a workspace
 *             must be ordered on one stream, and the buffer must not be
 *             handed to other entry points in between (they would overwrite
 *             the counters).  Other steps use it as attn_fwd_ws does.
 * No written buffer (q, the caches, o, lse, workspace) may overlap another
 * buffer (ERR_SHAPE).  Head sizes as attn_fwd; the rotation needs an even
 * d_head.  Returns a rocattn_status.
 */
/*
 * attn_decode_step_workspace_bytes -- bytes of workspace attn_decode_step
 * needs for these sizes and every pos with pos + Tn <= Tmax (see above);
 * 0 for arguments it would reject.
 */
size_t attn_decode_step_workspace_bytes(int B, int Hq, int Hkv, int Tn, int Tmax, int d_head, int dtype);

int attn_decode_step(void* q, const void* k_new, const void* v_new, void* k_cache,
                     void* v_cache, void* o, int B, int Hq, int Hkv, int Tn, int Tmax, int pos,
                     int d_head, float scale, double rope_base, int pairing, int dtype,
                     void* stream, void* workspace, size_t ws_bytes, float* lse);

/*
 * attn_fwd_dv -- attn_fwd with a value width d_v of its own: q and k rows
 * have d_k channels, v and o rows d_v ("The Transformer architecture" --
 * Scaled dot-product attention: only q and k must share a width; the
 * values need the keys' token count, not their width).  softmax(scale Q K^T
 * + M) V as attn_fwd; scale is typically 1/sqrt(d_k).
 *
 *   q   [B][Hq][Tq][d_k]     k   [B][Hkv][Tk][d_k]
 *   v   [B][Hkv][Tk][d_v]    o   [B][Hq][Tq][d_v], fully overwritten
 *   lse optional float32 [B][Hq][Tq] (as attn_fwd_ws)
 * Supported: bf16 with d_k, d_v in {64, 128} (every Tq on the prefill
 * kernel, no workspace); float32 with d_k, d_v <= 256, multiples of 4.
 * d_k == d_v gives the same result as attn_fwd.  Other arguments, checks
 * and status codes as attn_fwd.
 */
int attn_fwd_dv(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
                int Tq, int Tk, int d_k, int d_v, float scale, int causal, int q_offset,
                int dtype, void* stream, float* lse);

/*
 * attn_fwd_rope -- RoPE and attention of one prefill in two launches: k is
 * rotated in place at positions 0 .. Tk - 1 (the key rows a cache keeps,
 * "The Transformer architecture" -- Hands-on), and the attention of
 * attn_fwd_ws runs with each query row rotated as it is loaded, at position
 * q_offset + i, so q stays unrotated in memory and the rotation costs no
 * pass over q ("Transformer" (ai-notes) -- RoPE; "The Transformer
 * architecture" -- Now: RoPE: rotate q and k, not v, before the scores).
 * The result equals rope_apply_ex on q (at pos0 = q_offset) and k (at 0)
 * followed by attn_fwd_ws, bit for bit.
 *
 *   q          [B][Hq][Tq][d_head], read only (not rotated in memory).
 *   k          [B][Hkv][Tk][d_head], rotated in place (read, then written).
 *   v, o, lse, scale, causal, stream   as attn_fwd_ws.
 *   q_offset   position of query row 0 (and, with causal, the mask offset):
 *              0 <= q_offset and q_offset + Tq <= Tk, else ERR_OFFSET.
 *   rope_base, pairing   as rope_apply_ex.
 *   workspace  attn_fwd_rope_workspace_bytes(Tk, d_head) bytes of device
 *              memory, 16-byte aligned: the float32 (cos, sin) table
 *              [Tk][d_head / 2] the key pass writes and the query load reads;
 *              scratch afterwards.
 * Supported: bf16 (float32 returns ERR_DTYPE), d_head in {64, 128}; every Tq
 * runs on the prefill kernel (a one-token step is attn_decode_step's job).
 * k may not overlap q, v, o or lse; the workspace overlaps nothing (ERR_SHAPE).
 * Returns a rocattn_status.
 */
int attn_fwd_rope(const void* q, void* k, const void* v, void* o, int B, int Hq, int Hkv,
                  int Tq, int Tk, int d_head, float scale, int causal, int q_offset,
                  double rope_base, int pairing, int dtype, void* stream, void* workspace,
                  size_t ws_bytes, float* lse);

/* attn_fwd_rope_workspace_bytes -- bytes of the angle table attn_fwd_rope
 * needs: Tk * (d_head / 2) * 8 (0 for an unsupported head size). */
size_t attn_fwd_rope_workspace_bytes(int Tk, int d_head);

/*
 * attn_bwd -- gradients of attn_fwd: for an upstream gradient dO = dL/dO,
 * dq = dL/dq, dk = dL/dk, dv = dL/dv.  The pages train this operator
 * ("Transformer Math and Implementation Deep Dive" -- What To Implement:
 * tiny training loop) through the softmax, a differentiable allocation
 * ("The Transformer architecture" -- Softmax is a differentiable
 * allocation); the gradients are the chain rule of equation (1):
 *     P = exp(scale Q K^T + M - lse),  dV = P^T dO,  dP = dO V^T,
 *     D_i = sum_c dO_ic O_ic,  dS = P (dP - D),
 *     dQ = scale dS K,  dK = scale dS^T Q,
 * with a K/V head's dK and dV summed over the query heads of its group.
 *
 *   q, k, v, o   the forward's inputs and output (dense layouts as attn_fwd).
 *   dO           [B][Hq][Tq][d_head], the upstream gradient.
 *   lse          float32 [B][Hq][Tq], the forward's log-sum-exp rows (from
 *                attn_fwd_ws with a non-NULL lse on the same inputs).
 *   dq           [B][Hq][Tq][d_head], dk and dv [B][Hkv][Tk][d_head]; fully
 *                overwritten (keys no query sees get 0).
 *   workspace    attn_bwd_workspace_bytes(...) bytes of device memory.
 *   other arguments as attn_fwd.
 * Supported: bf16, d_head in {64, 128} (float32 returns ERR_DTYPE).
 * The workspace holds per-row statistics (256 bytes per 32 query rows of a
 * head); its contents need no initialisation and are scratch afterwards.
 * Outputs and workspace must not overlap each other or the inputs
 * (ERR_SHAPE).  Deterministic: a fixed summation order, no atomics.
 * Returns a rocattn_status.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
             const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Tq,
             int Tk, int d_head, float scale, int causal, int q_offset, int dtype, void* stream,
             void* workspace, size_t ws_bytes);

/* attn_bwd_workspace_bytes -- bytes of workspace attn_bwd needs (0 for a
 * shape or dtype it rejects). */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int d_head, int dtype);

/* attn_status_string -- static English text for a status code. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ROCATTN_H */
