/*
 * libmiattn - exact fused scaled-dot-product attention on AMD Instinct MI355X
 * (gfx950), behind a plain C ABI.
 *
 * What is computed (every entry point): for batch b, query head h, query row
 * i and key j,
 *
 *     s_ij   = scale * sum_c q[b,h,i,c] * k[b,kvh,j,c]     (visible pairs only)
 *     O[b,h,i,:] = sum_j softmax_j(s_i.) * v[b,kvh,j,:]
 *     LSE[b,h,i] = ln sum_j exp(s_ij)
 *
 * i.e. softmax(Q K^T / sqrt(d)) V as defined in "Chapter 3.1 - The Cost of
 * Attention" (section 2, "Why self-attention is quadratic, precisely"), with
 * `scale` standing in for 1/sqrt(d). The forward pass is one fused, tiled
 * kernel with an online softmax: the score matrix never reaches device memory
 * ("Quadratic Complexity Bottleneck", FlashAttention entry; grasp.study
 * efficient-attention lesson, "Tiling and Kernel Fusion" and "Online
 * Softmax"). The result equals the one-shot softmax up to rounding.
 *
 * Conventions shared by all entry points
 *   Layout    contiguous row-major. q, o: [B, H, Nq, d]; k, v: [B, Hkv, Nk, d];
 *             lse: [B, H, Nq]. Decode: q, o: [B, H, d]; caches [B, Hkv, Nk, d];
 *             lse [B, H].
 *   bf16      "bf16" tensors hold bfloat16 bit patterns (uint16). Outputs are
 *             rounded once, to nearest even, from fp32. Accumulation is fp32.
 *   GQA       query heads form Hkv contiguous groups of G = H / Hkv heads; head
 *             h reads K/V head h / G ("Quadratic Complexity Bottleneck", GQA
 *             and MQA entries). H % Hkv != 0 is MIATTN_EINVAL.
 *   causal    0 or 1. Query row i sits at absolute position p = i + Nk - Nq
 *             (bottom-right alignment), so a single query row sees the whole
 *             cache.
 *   window    0 = no window. W > 0: a query at position p sees keys
 *             j in [p - W, p] when causal (W keys to its left plus itself),
 *             |p - j| <= W otherwise ("Quadratic Complexity Bottleneck",
 *             sliding-window entry). Negative is MIATTN_EINVAL.
 *   scale     used exactly as passed; must be finite and > 0.
 *   empty     a query row that sees no key gets O = 0 and LSE = -inf. B, Nq
 *             or Nk may be 0 (Nk = 0 makes every row empty; B = 0 or Nq = 0
 *             does nothing). Pointers to tensors with no elements may be NULL.
 *   d         64 or 128, else MIATTN_EUNSUPPORTED.
 *   sizes     one head's K (or V) must stay under 4 GiB in fp32 terms
 *             (Nk * d * 4 < 2^32), else MIATTN_EUNSUPPORTED.
 *   lse       may be NULL: the LSE store is skipped.
 *   stream    a hipStream_t (NULL = the null stream). Work is enqueued
 *             asynchronously; no entry point synchronises.
 *
 * Ownership: the caller owns every buffer, including the decode and backward
 * workspaces, and keeps it alive until the stream work completes. The library allocates
 * and frees no device memory, keeps no pointer after returning, and holds no
 * per-call state. Calls are thread-safe.
 *
 * Errors: the return value is a status. Arguments are validated before any
 * HIP call, so argument errors return without touching the device. A failed
 * launch returns MIATTN_ELAUNCH. Faults inside a kernel surface at the
 * caller's next synchronisation, as with any asynchronous launch.
 */
#ifndef MIATTN_H
#define MIATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MIATTN_OK            0
#define MIATTN_EINVAL       -1 /* bad argument: null pointer, negative size, H % Hkv, ... */
#define MIATTN_EUNSUPPORTED -2 /* valid but not built: d not 64/128, sizes past 32-bit grids */
#define MIATTN_ELAUNCH      -3 /* the HIP runtime refused a launch */
#define MIATTN_EWORKSPACE   -4 /* workspace NULL or smaller than required */
#define MIATTN_ENODEVICE    -5 /* no HIP device is visible to this process */
#define MIATTN_ESCRATCH     -6 /* needs more than the library's own decode scratch */

/*
 * Prefill / training forward, bfloat16 in and out, fp32 LSE.
 * Steps: Q tile loaded once; K/V tiles streamed through LDS (skipping every
 * tile the causal / window mask hides entirely); S = Q K^T on bf16 matrix
 * cores with fp32 accumulation; the mask applied on boundary tiles only;
 * online-softmax update of the running row max and sum; O += P V; one
 * normalise-and-store at the end ("Chapter 3.1 - The Cost of Attention",
 * section 5; "Attention Research", section 2 for the sequence-parallel
 * partitioning of the query rows).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Hkv, int Nq, int Nk, int d,
             float scale, int causal, int window, void* stream);

/* Same contract with fp32 q, k, v, o: softmax(Q K^T / sqrt(d)) V exactly as
 * defined in "Chapter 3.1 - The Cost of Attention" (section 2), with the
 * running max / running sum of the online softmax ("Chapter 3.1", section 5;
 * grasp.study efficient-attention lesson, "Online Softmax"). The whole
 * computation is fp32 (vector ALU), with no bf16 rounding anywhere: inputs, P
 * and the output all stay fp32. */
int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                 int B, int H, int Hkv, int Nq, int Nk, int d,
                 float scale, int causal, int window, void* stream);

/*
 * FP8 forward: q and k in FP8 E4M3 (OCP e4m3fn: bias 7, max 448, no
 * infinities), each with one fp32 descale (the real value of a code is
 * code * descale); v and o bf16; lse fp32. The scores are
 * s_ij = scale * q_descale * k_descale * sum_c q8[b,h,i,c] * k8[b,kvh,j,c],
 * computed on the fp8 matrix cores with fp32 results; everything after the
 * scores (softmax, P V, output) is exactly as in attn_fwd. FP8 is used only
 * for the Q K^T product, where the pages place the low-precision gain
 * ("Chapter 3.1 - The Cost of Attention", section 6: FP8 where the accuracy
 * cost is negligible; "Attention Research", section 4: the softmax is what
 * makes low-precision attention harder than a GEMM).
 * Layout, masks, GQA and errors as for attn_fwd; q_descale and k_descale must
 * be finite and > 0 (MIATTN_EINVAL), and scale * q_descale * k_descale must
 * stay a finite, non-zero fp32 value (MIATTN_EUNSUPPORTED).
 */
int attn_fwd_fp8(const void* q8, const void* k8, const void* v, void* o, float* lse,
                 int B, int H, int Hkv, int Nq, int Nk, int d,
                 float scale, float q_descale, float k_descale,
                 int causal, int window, void* stream);

/*
 * Packed variable-length documents, bfloat16 in and out, fp32 LSE. Several
 * documents are packed along one token axis; the mask restarts at every
 * document boundary, so no row sees another document ("What Lost, and Why",
 * closing section: masking across packed documents is the silent bug to
 * avoid). Each document is attended exactly as attn_fwd attends one sequence:
 * bottom-right causal alignment and the window counted from the document's
 * own start, GQA as above.
 *
 * Layout: q, o [H, total_q, d]; k, v [Hkv, total_k, d]; lse [H, total_q] fp32
 * or NULL (the fixed-length layout with B = 1 and the documents end to end).
 * cu_seqlens_q, cu_seqlens_k: DEVICE int32 arrays of num_seqs + 1 offsets,
 * non-decreasing from 0 to total_q (resp. total_k); document e owns query
 * rows [cu_seqlens_q[e], cu_seqlens_q[e+1]) and key rows
 * [cu_seqlens_k[e], cu_seqlens_k[e+1]). Documents may be empty; one with
 * queries but no keys gets O = 0, LSE = -inf.
 * max_seqlen_q: a host-side bound, at least every document's query count; it
 * sizes the grid (num_seqs * H * ceil(max_seqlen_q / block_m) work-groups,
 * those past a document's end exit at once).
 *
 * Errors: host-visible arguments are validated as for attn_fwd (and the
 * offset arrays must be non-NULL when num_seqs > 0). The offsets live on the
 * device and are not read by the host: a document whose offsets are out of
 * order or out of range is skipped (its rows are not written), and query rows
 * past max_seqlen_q in a longer document are not written. Neither reads or
 * writes outside the buffers.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs,
                    int H, int Hkv, int total_q, int total_k, int max_seqlen_q, int d,
                    float scale, int causal, int window, void* stream);

/*
 * Backward pass of attn_fwd (bf16): the gradients dq, dk, dv of
 * L = sum(O * dout), recomputing the attention matrix from q, k and the
 * forward's LSE instead of storing it ("Quadratic Complexity Bottleneck",
 * FlashAttention entry; "Chapter 3.1 - The Cost of Attention", section 5).
 * With P = exp(scale q k^T - LSE) over visible pairs and D = rowsum(dout * o):
 *
 *     dv = P^T dout,  dS = P * (dout v^T - D),  dq = scale dS k,
 *     dk = scale dS^T q          (a K/V head sums over its G query heads).
 *
 * q, o, dout, dq: [B, H, Nq, d] bf16; k, v, dk, dv: [B, Hkv, Nk, d] bf16;
 * lse: [B, H, Nq] fp32 as written by attn_fwd for the same q, k, v, scale,
 * causal and window (rows that see no key have LSE = -inf and get dq = 0;
 * keys no row sees get dk = dv = 0). Outputs are rounded once to bf16 from
 * fp32. Every output element is written by exactly one work-item, so
 * results are deterministic.
 * workspace: device memory of at least attn_bwd_workspace_bytes(...) bytes
 * (else MIATTN_EWORKSPACE): D and the LSE in the exp2 domain (fp32 per query
 * row each), plus fp32 dk / dv partials per query head when H > Hkv. One
 * head's Q (or dO) rows must also stay under 4 GiB (Nq * d * 2 < 2^32; the
 * packed variant: total_q * d * 2), else MIATTN_EUNSUPPORTED. Other
 * conventions and errors as for attn_fwd.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d);
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv,
             int B, int H, int Hkv, int Nq, int Nk, int d,
             float scale, int causal, int window,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of attn_fwd_varlen (packed documents): dq, dk, dv of the packed
 * forward, each document's gradients depending only on its own rows.
 * Layout as attn_fwd_varlen: q, o, dout, dq [H, total_q, d] bf16; k, v, dk, dv
 * [Hkv, total_k, d] bf16; lse [H, total_q] fp32 as written by attn_fwd_varlen
 * for the same arguments; cu_seqlens_* device int32 [num_seqs + 1].
 * max_seqlen_q / max_seqlen_k: host-side bounds of every document's query /
 * key count (they size the grids). Key rows of a document with no queries get
 * dk = dv = 0. workspace: attn_bwd_workspace_bytes(1, H, Hkv, total_q,
 * total_k, d) bytes. A document with bad offsets is skipped, as in
 * attn_fwd_varlen: its dq rows are not written and, when H > Hkv, its dk / dv
 * rows are unspecified. Other conventions as for attn_bwd.
 */
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs,
                    int H, int Hkv, int total_q, int total_k,
                    int max_seqlen_q, int max_seqlen_k, int d,
                    float scale, int causal, int window,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Split-K decode: one query token per sequence against a KV cache
 * ("Quadratic Complexity Bottleneck", KV cache entry: past K and V are read
 * from the cache; "Attention Research", section 2: split-K over keys for
 * decode). The new token's K/V are already in the cache, so the query sits at
 * position Nk - 1 and sees every key (or the last window + 1 keys).
 *
 * The key range is cut into `num_splits` contiguous chunks of C = ceil(Nk/S)
 * keys (the last shorter, trailing ones possibly empty). A first kernel turns
 * each (sequence, KV head, chunk) into a normalised partial output O_s and its
 * log-sum-exp lse_s for all G query heads of the group, reading each K/V byte
 * once; a second kernel merges the partials: LSE = ln sum_s exp(lse_s),
 * O = sum_s exp(lse_s - LSE) O_s, a chunk with no visible key weighing 0.
 *
 * q, o: [B, H, d] bf16; k_cache, v_cache: [B, Hkv, Nk, d] bf16; lse [B, H]
 * fp32 or NULL. num_splits: 1..Nk, or 0 to let the library choose.
 * workspace: device memory of at least attn_decode_workspace_bytes(...) with
 * the same arguments (else MIATTN_EWORKSPACE). Any group size G = H / Hkv:
 * groups of more than 32 query heads are processed in blocks of 32 (each
 * block reads the group's keys).
 *
 * attn_decode_workspace_bytes returns B * H * (S + 1) * (d + 1) * 4 +
 * (B * (S + 1) + 2) * 4 bytes, where S is the split count the decode call
 * will use: room for the fp32 partial outputs O_s and their lse_s (B * H * S
 * of each here; up to B * H * (S + 1) for the per-sequence-length and paged
 * variants below), then the int32 work plan those variants build. The
 * contents are the library's own between calls. It takes Hkv and Nk (and not only
 * B, H, d and num_splits) because num_splits = 0 means "library's choice",
 * which depends on the number of (sequence, KV head) units B * Hkv and on the
 * key count Nk (attn_decode_num_splits); with the same arguments as the
 * decode call it always returns that call's requirement. It returns 0 for
 * arguments the decode call would reject.
 */
size_t attn_decode_workspace_bytes(int B, int H, int Hkv, int Nk, int d, int num_splits);
int attn_decode_splitk(const void* q, const void* k_cache, const void* v_cache,
                       void* o, float* lse,
                       int B, int H, int Hkv, int Nk, int d, float scale, int window,
                       int num_splits, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * attn_decode_splitk without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture into a HIP graph, tight
 * serving loops, harnesses that forbid allocation). The split partials go to
 * a scratch array that the library holds in device memory: a fixed
 * MIATTN_DECODE_SCRATCH_BYTES per GPU, allocated when the library's code is
 * loaded onto that GPU and kept until the process ends. This call allocates
 * and frees nothing.
 *
 * Arguments, results and errors are those of attn_decode_splitk with no
 * workspace. A call whose partials (attn_decode_workspace_bytes with the same
 * arguments) would exceed MIATTN_DECODE_SCRATCH_BYTES returns MIATTN_ESCRATCH
 * without touching the device. The work runs on the current device: a
 * non-NULL stream of another device is MIATTN_EINVAL.
 *
 * Every call on one GPU shares that GPU's scratch: calls whose work may
 * overlap on one GPU (other streams, other threads) race and must be ordered
 * by the caller, e.g. by issuing them on one stream. Each call writes every
 * partial it reads, so nothing needs clearing between calls.
 */
#define MIATTN_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
int attn_decode_splitk_noalloc(const void* q, const void* k_cache, const void* v_cache,
                               void* o, float* lse,
                               int B, int H, int Hkv, int Nk, int d, float scale, int window,
                               int num_splits, void* stream);

/*
 * Split-K decode over caches whose sequences hold different numbers of keys.
 * Sequence b uses the first kv_lens[b] rows of its [Hkv, Nk, d] cache slot;
 * its query sits at position kv_lens[b] - 1. The work follows the real
 * lengths and is balanced over the batch: the visible keys of all sequences
 * are laid end to end in tiles of 128 (each sequence's run starting at its
 * first visible key), and each of the work-groups per KV head (B *
 * num_splits of them at most, and no more than fit on the device at once,
 * so that each takes one long run) takes an equal run of whole tiles, cut at
 * sequence boundaries into pieces
 * that each yield one partial (O_s, lse_s) of one sequence; the merge then
 * combines a sequence's pieces as above. A small first kernel builds this
 * plan from kv_lens on the device, so the call needs no host copy of the
 * lengths. kv_lens: DEVICE int32 [B]; values are clamped to [0, Nk], and a
 * sequence of length 0 gets O = 0, LSE = -inf. Everything else (layout,
 * workspace size, split count, errors) is as for attn_decode_splitk; kv_lens
 * must be non-NULL when B > 0, and B * (num_splits + 1) and twice the batch's
 * tile count B * ceil(Nk / 128) must fit in an int (else MIATTN_EUNSUPPORTED).
 */
int attn_decode_splitk_varlen(const void* q, const void* k_cache, const void* v_cache,
                              const int* kv_lens, void* o, float* lse,
                              int B, int H, int Hkv, int Nk, int d, float scale, int window,
                              int num_splits, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Split-K decode over a paged KV cache ("Attention Research", section 2,
 * names paged variants among the attention kernel libraries): the keys and
 * values of all sequences live in fixed-size pages of one pool, and a block
 * table says which physical page holds each sequence's j-th run of
 * page_size keys. Only the address of a key row differs from
 * attn_decode_splitk_varlen; the result is the same as for a contiguous cache
 * holding the same keys.
 *
 * k_pages, v_pages: [num_pages, Hkv, page_size, d] bf16 (one page holds
 * page_size consecutive keys of every KV head). block_table: DEVICE int32
 * [B, max_pages]; key j of sequence b is row j % page_size of page
 * block_table[b * max_pages + j / page_size]. kv_lens: DEVICE int32 [B],
 * clamped to [0, max_pages * page_size]. Entries past a sequence's length
 * are never read; an entry inside it that is outside [0, num_pages) reads as
 * zero keys and values (a meaningless result, but nothing outside the pool
 * is touched). Pages may be shared between sequences.
 * page_size: a power of two in [1, 65536], else MIATTN_EINVAL.
 * workspace: attn_decode_workspace_bytes(B, H, Hkv, max_pages * page_size, d,
 * num_splits) bytes. q, o, lse, scale, window, num_splits as for
 * attn_decode_splitk.
 */
int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                      const int* block_table, const int* kv_lens, void* o, float* lse,
                      int B, int H, int Hkv, int d, int page_size, int num_pages,
                      int max_pages, float scale, int window, int num_splits,
                      void* workspace, size_t workspace_bytes, void* stream);

/* The split count attn_decode_splitk uses for these arguments (resolves 0),
 * or a negative status for invalid ones. */
int attn_decode_num_splits(int B, int Hkv, int Nk, int num_splits);

/* Query-tile (block_m) and key-tile (block_n) sizes of the forward kernels
 * for head dim d; is_f32 selects the fp32 kernel. Returns a status. */
int attn_fwd_tile_shape(int d, int is_f32, int* block_m, int* block_n);

/*
 * Instrumented attn_fwd (bf16): runs the same kernel and also writes, per
 * work-group, how many K/V tiles it loaded and how many of those it masked.
 * counts: device int32 [B, H, ceil(Nq / block_m), 2]. Used to show that tiles
 * the mask hides entirely are never loaded ("Attention Research", section 4:
 * a FLOP reduction only pays if the kernel skips whole blocks).
 */
int attn_fwd_tile_counts(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int Hkv, int Nq, int Nk, int d,
                         float scale, int causal, int window, int* counts, void* stream);

/* The same for attn_fwd_varlen: counts is device int32
 * [num_seqs, H, ceil(max_seqlen_q / block_m), 2]; work-groups past their
 * document's end write (0, 0). Shows that no tile of another document is
 * ever loaded. */
int attn_fwd_varlen_tile_counts(const void* q, const void* k, const void* v, void* o,
                                float* lse, const int* cu_seqlens_q, const int* cu_seqlens_k,
                                int num_seqs, int H, int Hkv, int total_q, int total_k,
                                int max_seqlen_q, int d, float scale, int causal, int window,
                                int* counts, void* stream);

/*
 * Ceiling probes (they compute no attention): the rates this device sustains,
 * reported next to the published peaks when pricing the kernels above.
 * attn_calib_mfma: `blocks` work-groups of 4 waves, each wave issuing
 *   iters x 8 independent bf16 32x32x16 matrix instructions;
 *   FLOPs = blocks * 4 * iters * 8 * 32768. sink: device float[blocks]
 *   (written only in a practically unreachable case).
 * attn_calib_read: streams `bytes` (a multiple of 16) from device buffer
 *   `buf` once with 16-byte loads over `blocks` work-groups of 256 threads.
 *   sink: device unsigned[1].
 */
int attn_calib_mfma(int blocks, int iters, float* sink, void* stream);
int attn_calib_read(const void* buf, size_t bytes, unsigned* sink, int blocks, void* stream);

/* Static string for a status code (never NULL; "unknown status" for a value
 * not listed above). The pages define no programming interface, so the status
 * codes and this call are the library's own error contract: every entry point
 * reports through its return value and nothing else. */
const char* attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* MIATTN_H */
