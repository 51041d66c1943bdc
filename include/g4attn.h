/*
 * g4attn.h -- C ABI of libg4attn: the attention block of Gemma 4 on AMD
 * Instinct MI355X (gfx950).
 *
 * The block interleaves two attention layer kinds:
 *   - local layers: causal sliding-window attention (window 512 or 1024 keys),
 *     2 query heads per KV head, head dim 256, rotary encoding on every pair;
 *   - global layers: causal attention over the whole preceding sequence,
 *     8 query heads per KV head, head dim 512, keys identical to values (one
 *     tensor serves both), and p-RoPE rotating only the first quarter of the
 *     rotary pairs.
 * Sources: "Guia visual do Gemma 4" (pt.news.hada.io), sections "Intercalacao
 * de camadas de atencao", "GQA (Grouped Query Attention)", "Tecnica K=V" and
 * "p-RoPE"; "Gemma 4: yak Google DeepMind pereosmyslyuye vidkryti modeli ..."
 * (techtoday.in.ua), section "Optymizovana uvaha: lokalni y hlobalni shary"
 * (local GQA ratio, 512 vs 256 head dims); "Visao geral do modelo Gemma 4"
 * (ai.google.dev), section "Principais Consideracoes para o planejamento de
 * memoria" (the KV cache grows with prompt and generated tokens).
 *
 * What every call computes, for query row (b, i, h) with G = Hq / Hkv:
 *     out[b,i,h] = sum_j softmax_j(s_j) * v[b,j,h/G]
 *     s_j = < R(pos_i) q[b,i,h], R(pos_j) k[b,j,h/G] > / sqrt(d)
 * over the keys j with 0 <= i - j < window (window 0: every j <= i).  R(P)
 * turns pair t = (dims 2t, 2t+1), for t < n_rot = floor(p * d / 2), by the
 * angle P * theta^(-2t/d), counter-clockwise; the other pairs are not turned.
 * Values are never rotated (for K=V the one tensor is rotated for the scores
 * and read raw as the values).  The mask uses the sequence index; positions
 * only set the rotation angles.
 *
 * Conventions shared by every call
 *   - All tensors are dense, row-major, in device memory (hipMalloc or any
 *     allocator of device memory).  The caller owns every buffer; the library
 *     allocates, frees and synchronises nothing, keeps no state between calls
 *     and is safe to call from several host threads.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *     the null stream).  A return of G4A_OK means the work was enqueued.
 *   - Argument errors are reported synchronously, before anything is
 *     launched, as a negative status.  Faults inside a kernel surface at the
 *     caller's next synchronisation of the stream.
 *   - Every tensor and workspace pointer must be 16-byte aligned.
 *   - dtype codes: G4A_F32 = 0 (float32), G4A_BF16 = 1 (bfloat16).
 *     Supported (in_dtype, out_dtype): (F32, F32), (BF16, F32), (BF16, BF16).
 *     Inside the kernels bf16 inputs are multiplied on the matrix cores with
 *     fp32 accumulation; f32 inputs are computed in fp32 throughout.
 *   - Supported shapes: d in {256, 512} for bf16 inputs, d in {64, 128, 256,
 *     512} for f32 inputs; G = Hq / Hkv in {1, 2, 4, 8}; other combinations
 *     return G4A_EUNSUPPORTED.  The bf16 prefill calls (causal and vision)
 *     also need Hkv * d * 2 < 2^24 (one token's keys of all KV heads under
 *     16 MiB: Hkv < 16384 at d = 512) and return G4A_EUNSUPPORTED otherwise.
 */
#ifndef G4ATTN_H
#define G4ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define G4A_OK 0
#define G4A_EINVAL (-1)      /* null pointer, bad size, Hq % Hkv != 0, p outside [0,1],
                                theta <= 0, window < 0, ring capacity != window */
#define G4A_EUNSUPPORTED (-2) /* head dim, group size or dtype pair not built */
#define G4A_EALIGN (-3)      /* a tensor or workspace pointer is not 16-byte aligned */
#define G4A_EWORKSPACE (-4)  /* workspace missing or smaller than the size query says */
#define G4A_EHIP (-5)        /* the HIP runtime refused a launch; see g4attn_last_hip_error */
#define G4A_ESCRATCH (-6)    /* g4attn_decode_noalloc: the partials exceed its fixed scratch */

/* dtype codes */
#define G4A_F32 0
#define G4A_BF16 1

/*
 * Prefill workspace: bf16 prefill first writes the rotated leading dims of
 * every key (all d dims, or the first 128 when d = 512 and at most 64 pairs
 * turn) into the workspace, once per key, and the attention kernel reads them
 * from there.  Returns the bytes a prefill call with these sizes needs:
 * B * S * Hkv * slab_dims * 2 for bf16 inputs, 0 for f32 inputs (0 also for
 * invalid sizes).  The contents need no initialisation and are garbage
 * afterwards; calls that share one workspace must be ordered on one stream.
 */
size_t g4attn_prefill_workspace_bytes(int B, int S, int Hkv, int d, float p, int in_dtype);

/*
 * Both causal prefill calls take the arguments the pages' statement of the
 * problem names (q, k/v or kv, positions, window, group size via Hq/Hkv, head
 * dim, theta, p) plus a workspace, sized by g4attn_prefill_workspace_bytes.
 * The workspace is an extension of that statement: keys are rotated once
 * each, by one pass into the workspace, instead of in every key tile load of
 * every query tile that reads them (about S/32 times per key for a global
 * layer), which measured faster and frees the attention kernel's registers.
 *
 * Sliding-window (local) causal prefill with separate keys and values.
 *   q    [B, S, Hq,  d]  in_dtype        k, v [B, S, Hkv, d]  in_dtype
 *   out  [B, S, Hq,  d]  out_dtype       pos  [B, S] int32 token positions
 *   window: keys per query including itself (0 = unbounded, i.e. global).
 *   theta: rotary base; p: rotated fraction of the pairs (1 = full RoPE).
 *   workspace: device memory of at least g4attn_prefill_workspace_bytes(...)
 *   bytes (may be NULL when that is 0).
 * Local layers: window 512/1024, G = 2, d = 256, theta 1e4, p = 1
 * ("Guia visual do Gemma 4", section "Intercalacao de camadas de atencao";
 * techtoday page, attention section, for G = 2 and d = 256).
 * Returns G4A_OK or a negative status; out is written in full.
 */
int g4attn_local_prefill(const void* q, const void* k, const void* v, void* out,
                         const int32_t* pos, int B, int S, int Hq, int Hkv, int d, int window,
                         float theta, float p, int in_dtype, int out_dtype, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Global causal prefill with keys identical to values (K=V): one tensor kv
 * is rotated for the scores and read raw as the values, so it is loaded once
 * for both products ("Guia visual do Gemma 4", sections "GQA", "Tecnica K=V",
 * "p-RoPE": G = 8, d = 512, p = 0.25).
 *   q   [B, S, Hq, d]   kv [B, S, Hkv, d]   out [B, S, Hq, d]   pos [B, S]
 *   window: 0 for global layers (a positive window also works).
 *   workspace: as for g4attn_local_prefill.
 * Returns G4A_OK or a negative status; out is written in full.
 */
int g4attn_global_prefill(const void* q, const void* kv, void* out, const int32_t* pos, int B,
                          int S, int Hq, int Hkv, int d, int window, float theta, float p,
                          int in_dtype, int out_dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Vision-encoder attention: every patch of an image attends to every patch
 * of the image (no causal mask), with 2D RoPE ("Guia visual do Gemma 4",
 * sections "Encoder de visao" and "Suporte a proporcao variavel").  Half c of
 * the head dims ([0, d/2) for c = 0, [d/2, d) for c = 1) is an ordinary RoPE
 * of a head of dim d/2, pair t = dims (2t, 2t+1) of the half turning by
 * pos2[..., c] * theta^(-2t/(d/2)); component 0 is the patch's column w,
 * component 1 its row h.
 *   q    [B, S, Hq, d]  bf16          k, v [B, S, Hkv, d]  bf16
 *   out  [B, S, Hq, d]  out_dtype     pos2 [B, S, 2] int32 (w, h) per patch
 *   lengths [B] int32, or NULL (every image has S patches): image b has
 *        lengths[b] valid patches (clamped to [0, S]); patches past them are
 *        not attended to and their output rows are zero.
 *   theta: rotary base of each half.
 *   d = 256, G in {1, 2, 4, 8}, in_dtype G4A_BF16 (others: G4A_EUNSUPPORTED).
 *   workspace: g4attn_prefill_workspace_bytes(B, S, Hkv, d, 1.0, G4A_BF16)
 *        bytes (the rotated keys).
 * Returns G4A_OK or a negative status; out is written in full.
 */
int g4attn_vision_prefill(const void* q, const void* k, const void* v, void* out,
                          const int32_t* pos2, const int32_t* lengths, int B, int S, int Hq,
                          int Hkv, int d, float theta, int in_dtype, int out_dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode: one query token per sequence against a KV cache.
 *   q        [B, Hq, d]              in_dtype
 *   k_cache  [B, Hkv, capacity, d]   in_dtype.  With a separate v_cache it
 *                                    holds every key already turned at its
 *                                    own position t (R(t) k, pairs
 *                                    t < floor(p*d/2), as g4attn_fill_cache
 *                                    writes it); for K=V it holds the raw
 *                                    tensor, whose keys are turned here.
 *   v_cache  [B, Hkv, capacity, d]   in_dtype, or NULL (or k_cache itself)
 *                                    for K=V (k_cache is read raw as the
 *                                    values)
 * Turning each key once when it enters the cache, not at every step, is this
 * library's reading of the cache the pages leave unspecified, and an
 * extension of the problem's statement: measured, it makes the batch-64
 * decode over 512-slot rings of separate keys and values about 12% faster
 * (25% over fp8 codes).  A K=V cache cannot hold turned keys, since its
 * values are the raw tensor.
 *   out      [B, Hq, d]              out_dtype
 *   pos      [B] int32: position P of each query token; its own key/value
 *            must already be in the cache.
 *   window > 0: ring cache, capacity == window; position t lives in slot
 *            t mod window and the query sees positions max(0, P-window+1)..P.
 *   window == 0: linear cache, row t holds position t; the query sees 0..P.
 *   Cache rows the query does not see are never read (they may hold NaN).
 *   A sequence with P < 0, or P >= capacity for a linear cache, gets an
 *   all-NaN output row.
 *   workspace: device memory of at least g4attn_decode_workspace_bytes(...)
 *   bytes for split partial results; its contents need no initialisation
 *   and are garbage afterwards.  Calls that share one workspace must be
 *   ordered on one stream.
 * The waves of a workgroup claim cache tiles at run time, so the order of
 * the partial sums, and the running max against which each P is rounded to
 * bf16, can vary from call to call: results are reproducible to that
 * rounding (about 1e-4 for unit-variance inputs), not bit for bit.
 * Returns G4A_OK or a negative status.
 */
int g4attn_decode(const void* q, const void* k_cache, const void* v_cache, void* out,
                  const int32_t* pos, int B, int Hq, int Hkv, int d, int capacity, int window,
                  float theta, float p, int in_dtype, int out_dtype, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Workspace bytes g4attn_decode needs for these sizes (0 on invalid sizes). */
size_t g4attn_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int capacity, int window);

/*
 * g4attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing.  The split partials
 * go to a fixed scratch array of 64 MiB that the library holds in device
 * memory on every GPU it runs on, until the process ends; its address on a
 * device is looked up on the first call with that device current.
 *   Arguments, layouts, results and errors are those of g4attn_decode, and it
 *   runs the same kernels.  A problem whose partials (the size
 *   g4attn_decode_workspace_bytes reports) exceed 64 MiB returns G4A_ESCRATCH
 *   before anything is launched: for example batch 64 of a ring cache of any
 *   size fits, as do 16 sequences over a 65536-row linear cache of head dim
 *   512 with 16 query heads (33.7 MB); 64 such sequences (135 MB) do not.
 *   f32 inputs need no partials and are never rejected for size.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap on
 *   one GPU (on different streams or from different host threads without
 *   ordering) race on it and give wrong results.  Calls ordered on one
 *   stream are safe; the scratch needs no clearing between calls.
 * Returns G4A_OK or a negative status.
 */
int g4attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out,
                          const int32_t* pos, int B, int Hq, int Hkv, int d, int capacity,
                          int window, float theta, float p, int in_dtype, int out_dtype,
                          void* stream);

/*
 * Cache fill: write the key (and value) rows of a prefill into the decode
 * cache layout, so decoding continues where the prefill ended (the KV cache
 * grows with the prompt and the generated tokens: "Visao geral do modelo
 * Gemma 4", section "Principais Consideracoes para o planejamento de
 * memoria").  New tokens are appended the same way, with S = their count.
 *   k        [B, S, Hkv, d]           dtype
 *   v        [B, S, Hkv, d]           dtype, or NULL for K=V (only k_cache
 *                                     is written)
 *   pos      [B, S] int32 positions of the tokens
 *   k_cache, v_cache [B, Hkv, capacity, d]  dtype (v_cache unused for K=V)
 *   window > 0: ring; the last min(S, capacity) tokens of each sequence go
 *            to slot pos mod capacity.
 *   window == 0: linear; a token with 0 <= pos < capacity goes to row pos.
 *   Tokens with negative positions are not written; cache rows not written
 *   keep their contents.  Positions written in one call must differ modulo
 *   capacity (consecutive positions do); otherwise which row lands in a
 *   shared slot is unspecified.
 *   theta, p: the layer's rotary base and rotated fraction (as for decode;
 *            validated also for K=V, where they are not used).
 *   dtype: G4A_F32 or G4A_BF16; d * element size must be a multiple of 16.
 * With separate values (v given), each key row is turned at its position
 * (pairs t < floor(p*d/2) by pos * theta^(-2t/d)) in fp32 and rounded to
 * dtype (bf16: round to nearest even) before it is written; value rows, and
 * the rows of a K=V cache, are copied unchanged.  A turning fill (v given,
 * p*d >= 2) needs d <= 512 (G4A_EUNSUPPORTED otherwise).
 * Returns G4A_OK or a negative status.
 */
int g4attn_fill_cache(const void* k, const void* v, const int32_t* pos, int B, int S, int Hkv,
                      int d, void* k_cache, void* v_cache, int capacity, int window, float theta,
                      float p, int dtype, void* stream);

/*
 * Decode of q_len query tokens per sequence at once: the verify step of
 * speculative decoding, where a draft model proposes tokens and the model
 * checks them in one pass (every Gemma 4 size ships a draft model: "Visao
 * geral do modelo Gemma 4", section "Recursos").  q_len = 1 is
 * g4attn_decode.
 *   q        [B, q_len, Hq, d]       in_dtype
 *   k_cache, v_cache                 as for g4attn_decode (NULL v: K=V)
 *   out      [B, q_len, Hq, d]       out_dtype
 *   pos      [B] int32: position P of the LAST query token; token j sits at
 *            P - q_len + 1 + j, and the keys/values of all q_len tokens must
 *            already be in the cache.  Token j sees positions
 *            max(0, Pj - window + 1) .. Pj (window 0: 0 .. Pj).
 *   window > 0: ring; position t lives in slot t mod capacity, and capacity
 *            must be at least window + q_len - 1 so that the ring still holds
 *            the whole window of the first token.
 *   window == 0: linear cache, row t holds position t.
 *   1 <= q_len <= 8.  Rows of a token with a negative position, and every row
 *   of a sequence with P >= capacity in a linear cache, are NaN.
 *   workspace: at least g4attn_decode_multi_workspace_bytes(...) bytes, as
 *   for g4attn_decode.
 * Returns G4A_OK or a negative status.
 */
int g4attn_decode_multi(const void* q, const void* k_cache, const void* v_cache, void* out,
                        const int32_t* pos, int B, int q_len, int Hq, int Hkv, int d,
                        int capacity, int window, float theta, float p, int in_dtype,
                        int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes g4attn_decode_multi needs for these sizes (0 on invalid
 * sizes). */
size_t g4attn_decode_multi_workspace_bytes(int B, int q_len, int Hq, int Hkv, int d, int capacity,
                                           int window);

/*
 * Low-precision KV cache: one byte per cached element, an OCP FP8 E4M3 code
 * (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals at
 * exponent 0, no infinities, 0x7F / 0xFF NaN), the cached value being
 * code value x scale of its KV head.  The pages count optimized KV caches
 * among the memory savings of the mobile checkpoints and note that the cache
 * grows with every token ("Visao geral do modelo Gemma 4", sections
 * "Treinamento com reconhecimento de quantizacao (QAT)" and "Principais
 * Consideracoes para o planejamento de memoria"); they give no format, and
 * E4M3 with a scale per KV head is the reading this library takes.  The cache
 * is half the bytes of a bf16 one, which halves decode's memory traffic.
 *
 * Cache fill into fp8 caches: as g4attn_fill_cache (same slots, same rules,
 * keys of a cache with separate values turned first, in fp32), each element
 * quantized on the way:
 *     code = E4M3(x / scale[h])
 * with the quotient rounded once to fp32 (IEEE division), then rounded to the
 * nearest E4M3 value, ties to the even mantissa; |quotient| >= 448 (infinity
 * included) saturates to +-448, NaN gives a NaN code.
 *   k, v        [B, S, Hkv, d]  in_dtype (G4A_F32 or G4A_BF16); v NULL: K=V
 *   k_scale, v_scale  [Hkv] fp32 device arrays, positive and finite (v_scale
 *               unused for K=V)
 *   k_cache, v_cache  [B, Hkv, capacity, d] uint8 codes
 *   d must be a multiple of 16.
 * Returns G4A_OK or a negative status.
 */
int g4attn_fill_cache_fp8(const void* k, const void* v, const float* k_scale,
                          const float* v_scale, const int32_t* pos, int B, int S, int Hkv, int d,
                          void* k_cache, void* v_cache, int capacity, int window, float theta,
                          float p, int in_dtype, void* stream);

/*
 * Decode of q_len query tokens per sequence (1 <= q_len <= 8; 1 is ordinary
 * decode) over fp8 caches: exactly g4attn_decode_multi over the dequantized
 * cache (code value x scale of the KV head).
 *   q        [B, q_len, Hq, d]  bfloat16
 *   k_cache, v_cache  [B, Hkv, capacity, d] uint8 E4M3 codes, the key codes
 *            of turned keys as g4attn_fill_cache_fp8 writes them; v_cache NULL
 *            (or equal to k_cache): K=V, raw codes, the values are k_cache
 *            with k_scale
 *   k_scale, v_scale  [Hkv] fp32 device arrays, positive and finite
 *   out      [B, q_len, Hq, d]  out_dtype (G4A_F32 or G4A_BF16)
 *   pos, window, capacity, theta, p: as for g4attn_decode_multi (a ring needs
 *   capacity >= window + q_len - 1).  d in {256, 512}; G in {1, 2, 4, 8}.
 *   workspace: at least g4attn_decode_fp8_workspace_bytes(...) bytes.
 * Inside, codes are widened exactly to bf16 and multiplied on the matrix
 * cores with fp32 accumulation; the scales multiply the scores and the
 * output.  Returns G4A_OK or a negative status.
 */
int g4attn_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                      const float* k_scale, const float* v_scale, void* out, const int32_t* pos,
                      int B, int q_len, int Hq, int Hkv, int d, int capacity, int window,
                      float theta, float p, int out_dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Workspace bytes g4attn_decode_fp8 needs for these sizes (0 on invalid sizes). */
size_t g4attn_decode_fp8_workspace_bytes(int B, int q_len, int Hq, int Hkv, int d, int capacity,
                                         int window);

/* Static text for a status code. */
const char* g4attn_strerror(int status);

/* hipError_t of the last failed launch on this host thread (0 if none). */
int g4attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* G4ATTN_H */
