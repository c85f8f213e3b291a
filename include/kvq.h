/*
 * kvq.h — C ABI of libkvq: KIVI-style asymmetric KV-cache quantization and
 * decode attention over the quantized cache, for AMD Instinct MI355X (gfx950).
 *
 * Sources the operations follow (web pages, cited by title and section):
 *   [KIVI-page]  "4.4 KV Cache 量化：KIVI 2-bit 与 FP8 KV Cache"
 *                (aiinfraguide.pages.dev), §2, §3.1–3.4, §5, §6.3
 *   [Tutorial]   "大模型量化从0到1（十三）：KV Cache 量化——长上下文为什么越跑越吃显存"
 *                (aiot.csdn.net), §二 (attention), §四 (byte formula),
 *                §五 (MHA/GQA), §八.4 (online critical path), §九 (KIVI),
 *                §十 (affine / FP8 formulas, granularity, residual window),
 *                §十八.4 (E4M3 vs E5M2), §十八.6 (per-attention-head scales)
 *   [Interview]  "KV Cache 量化是什么？它如何降低长上下文推理显存？"
 *                (offer.aigcbaba.com), §三 (byte formula), §四 (pipeline)
 *   [FP8-page]   "LLM推理加速KV Cache量化压缩实战方案" (yunthe.com),
 *                section "自定义KV Cache量化的实现路径" (per-tensor amax/448)
 *
 * The three operations of the pipeline (prefill → group statistics →
 * low-bit write; decode → append + dequantize inside attention) are stated in
 * [Tutorial] §八.4 and [Interview] §四; the grouped-plus-residual structure
 * and its flush rule in [KIVI-page] §3.2.
 *
 * ---------------------------------------------------------------------------
 * Conventions (apply to every entry point)
 * ---------------------------------------------------------------------------
 * - Memory. The caller allocates and frees every device buffer (sizes from
 *   kvq_layout_query / kvq_decode_workspace_bytes). The library never
 *   allocates device memory and never synchronizes the device; its only
 *   global state is the per-GPU partials array of kvq_decode_attention_static
 *   (KVQ_STATIC_WORKSPACE_BYTES, part of its loaded device code) and cached
 *   device properties. Pointers marked "device" must point to device memory of the
 *   current HIP device; "host" pointers to host memory. Every device pointer
 *   (cache buffers, inputs, outputs, workspace) must be 16-byte aligned
 *   (else KVQ_ERR_INVALID_ARG, or KVQ_ERR_WORKSPACE for the workspace).
 * - Streams. `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream). All device work is enqueued asynchronously on it, in call order.
 * - State. The fill levels (n_quant, n_resid) live in the host-side
 *   kvq_cache struct and are updated when the work is enqueued, so no call
 *   waits for the device. All `batch` sequences have the same length, unless
 *   the cache is ragged (KIVI only; see kvq_prefill_quantize_ragged): then
 *   each sequence b has its own fill levels seq_n_quant[b], seq_n_resid[b]
 *   in caller-owned host arrays, and the scalar n_quant, n_resid stay 0.
 * - Errors. Every argument and state check runs before anything is enqueued.
 *   A call that returns an error enqueued nothing and changed nothing.
 *   KVQ_ERR_DEVICE reports a failed HIP launch; then the cache state has
 *   still been advanced for the launched work only if the launch succeeded.
 *   No C++ exception or abort crosses this boundary. A fill state the state
 *   machine cannot reach (n_quant < 0, KIVI n_quant not a multiple of G,
 *   n_resid > Rcap, n_quant + n_resid > C, ...) is rejected with
 *   KVQ_ERR_STATE by every call that reads it.
 * - Inputs. K/V values must be finite fp16; non-finite input is undefined
 *   behaviour (not checked). Query values must be finite fp32.
 * - Supported (else KVQ_ERR_UNSUPPORTED): head_dim = 128; batch · num_kv_heads
 *   ≤ 65535; KIVI group_size ∈ {32, 64, 128} ([KIVI-page] §3.4 names 32
 *   and compares 64 and 128), bits ∈ {2, 4} and v_bits ∈ {0, 2, 4} (K and V
 *   bit widths), v_group_channels ∈ {0, 32}, residual_length a multiple of
 *   group_size (0 allowed);
 *   FP8 (E4M3 or E5M2) bits = 8, scale_per_head ∈ {0, 1} and fp8_attention
 *   ∈ {0, 1}; FP16 bits = 16; deterministic ∈ {0, 1}; num_q_heads a
 *   positive multiple of num_kv_heads.
 *
 * ---------------------------------------------------------------------------
 * Numerics (bit-exact contract for KIVI codes, scales and zero-points)
 * ---------------------------------------------------------------------------
 * The affine quantizer of [Tutorial] §十 (q = clamp(round(x/s)+z, qmin, qmax),
 * x̂ = (q−z)·s) is used in its min/max asymmetric form with the zero-point kept
 * as an fp32 offset (the form the pages leave open; see the design notes):
 *   mn, mx = min, max of the group in fp32 (exact from fp16)
 *   s      = (mx − mn) / (2^bits − 1)          fp32, each op correctly rounded
 *   z      = mn
 *   code   = min(max(rint((x − mn) / s), 0), 2^bits − 1)   (rint = round half
 *            to even; fp32 subtract and IEEE division), code = 0 when s == 0
 *   x̂      = (float)code · s + z               (reconstruction)
 * KIVI granularity ([KIVI-page] §2 and §3.2, [Tutorial] §九.1–九.3):
 *   K — per channel: one (s, z) per (group of G tokens, channel); groups are
 *       aligned to token index multiples of G from position 0.
 *   V — per token: one (s, z) per token over its head_dim channels; with
 *       v_group_channels = 32, one (s, z) per token and run of 32 channels
 *       [32m, 32m + 32) (the group granularity of [Tutorial] §十.1 along the
 *       channels of a token).
 *
 * FP8 path ([FP8-page], [Tutorial] §十 FP8 formula, [KIVI-page] §5 for the
 * 1-4-3 layout, [Tutorial] §十八.4 for E5M2), FMAX = 448 (E4M3) or 57344
 * (E5M2):
 *   s_K = amax(|K|) / FMAX over the whole prefill K tensor, s_V likewise
 *   (s = 0 when amax = 0: every code is then 0); with scale_per_head, one
 *   s_K and one s_V per KV head h, amax over all batch rows, tokens and
 *   channels of head h ([Tutorial] §十八.6, [KIVI-page] §6.3);
 *   code = fp8(min(max(x / s, −FMAX), FMAX)) with round-to-nearest-even,
 *   signed zero kept. E4M3 is OCP "fn" (no infinities; 0x7F/0xFF are NaN and
 *   never produced); E5M2 is OCP E5M2 (bias 15; infinities and NaN are never
 *   produced). x̂ = (float)fp8_value(code) · s.
 *   The scales are fixed at prefill; appended tokens reuse them and saturate.
 *
 * ---------------------------------------------------------------------------
 * Device layouts (all arrays contiguous, row-major, little-endian)
 * ---------------------------------------------------------------------------
 * Let B = batch, H = num_kv_heads, D = head_dim, G = group_size, b = bits
 * (K), b_V = v_bits if > 0 else bits (V),
 * C = capacity, NG = ceil(C / G) (group slots), CT = NG · G (token slots),
 * NT = CT / 32 (32-token tiles), Rcap = residual_length if > 0 else G.
 * KIVI:
 *   k_codes  uint32 [B][H][CT][D·b/32]   token t of (b,h): its D channel codes,
 *            code of channel d in word d/(32/b) at bits [b·(d%(32/b)), +b).
 *   v_codes  uint32 [B][H][NT][D][32·b_V/32] tile g (tokens 32g .. 32g + 31),
 *            channel d: the 32 token codes of that channel, 32/b_V tokens
 *            per word (token j of the tile in word j/(32/b_V)); with
 *            i = j % (32/b_V), the code sits at bits [b_V·(i/2), +b_V) when
 *            i is even and [16 + b_V·(i/2), +b_V) when i is odd (even tokens
 *            fill the low half-word, odd the high). V is quantized per token,
 *            so the tile size does not depend on G.
 *   k_scale, k_zero  fp32 [B][H][NG][D]   (per group, per channel)
 *   v_scale, v_zero  fp32 [B][H][CT]      (per token), or [B][H][CT][D/32]
 *            with v_group_channels = 32 (run m of token t at [t][m])
 *   k_resid, v_resid fp16 [B][H][Rcap][D] the FP16 residual window; slot i
 *            holds token n_quant + i.
 * Paged KIVI (page_tokens = P > 0, NP = num_pages): the grouped-region
 *   arrays are pools of pages, each page holding tokens of one sequence for
 *   every KV head in the layout above restricted to P tokens:
 *   k_codes uint32 [NP][H][P][D·b/32], v_codes uint32 [NP][H][P/32][D][32·b_V/32],
 *   k_scale, k_zero fp32 [NP][H][P/G][D], v_scale, v_zero fp32 [NP][H][P]
 *   (or [NP][H][P][D/32]); token t of sequence b is slot t mod P of page
 *   block_table[b][t / P]. The window stays [B][H][Rcap][D].
 * FP8 and FP16 (baseline, no quantization) use tiles of T = 32 tokens,
 * NT = ceil(C / T), CTT = NT · T:
 *   k_codes  [B][H][CTT][D]   token rows (uint8 FP8 codes, or fp16 values);
 *   v_codes  [B][H][NT][D][T] tile g, channel d: the values of tokens
 *            g·T .. g·T + T − 1 (element (t, d) at [t / T][d][t % T]);
 *            slots between the last prefilled token and the end of its tile
 *            are written as zero.
 *   tensor_scale (FP8 only) fp32 [NS][4], NS = H with scale_per_head else 1:
 *   row h = {s_K, s_V, amax_K, amax_V} of KV head h (or of the tensor); the
 *   amax slots are scratch of the prefill reduction.
 * Decode I/O: q, out fp32 [B][Hq][D]. Query head hq reads KV head
 *   hq / (Hq / H) (consecutive query heads share a KV head, [Tutorial] §五.3).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 11

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad enum     */
  KVQ_ERR_UNSUPPORTED = 2, /* valid but outside the supported set above     */
  KVQ_ERR_CAPACITY = 3,    /* would exceed the configured capacity          */
  KVQ_ERR_STATE = 4,       /* wrong fill state (prefill into a non-empty
                              cache, decode on an empty cache)              */
  KVQ_ERR_DEVICE = 5,      /* a HIP launch failed                           */
  KVQ_ERR_WORKSPACE = 6    /* decode workspace missing or too small         */
} kvq_status;

typedef enum {
  KVQ_FMT_FP16 = 0,     /* unquantized fp16 cache (baseline)                */
  KVQ_FMT_FP8_E4M3 = 1, /* FP8 E4M3, scale = amax / 448                     */
  KVQ_FMT_KIVI = 2,     /* K per-channel / V per-token groups + FP16 window */
  KVQ_FMT_FP8_E5M2 = 3  /* FP8 E5M2, scale = amax / 57344                   */
} kvq_format;

/* Cache configuration. The KIVI knobs mirror the pages' `nbits`,
 * `q_group_size`, `residual_length` ([KIVI-page] §3.4; [Tutorial] §十六). */
typedef struct {
  int32_t format;          /* kvq_format                                      */
  int32_t bits;            /* KIVI 2 or 4; FP8 8; FP16 16                     */
  int32_t group_size;      /* KIVI: G ∈ {32, 64, 128} (ignored otherwise)      */
  int32_t residual_length; /* KIVI: R, multiple of G, 0 allowed (ignored else) */
  int32_t batch;           /* B ≥ 1                                           */
  int32_t num_kv_heads;    /* H ≥ 1                                           */
  int32_t head_dim;        /* D = 128                                         */
  int32_t capacity;        /* C ≥ 1: max tokens per sequence                  */
  int32_t v_bits;          /* KIVI: V's bit width, 2 or 4; 0 = same as bits
                              (K 4-bit with V 2-bit and the reverse are the
                              mixed widths of [KIVI-page] §3.4); ignored else */
  int32_t scale_per_head;  /* FP8: 0 = one K and one V scale per tensor, 1 = one
                              pair per KV head ([Tutorial] §十八.6); ignored
                              else                                            */
  int32_t fp8_attention;   /* FP8: 1 = decode quantizes the query to E4M3 per
                              query head (kvq_quantize_query_fp8) and takes
                              the scores in the FP8 domain ([Tutorial]
                              §十八.7); 0 = the query stays fp32; ignored
                              else                                            */
  int32_t v_group_channels; /* KIVI: 0 = one V scale / zero-point per token;
                              32 = one per token and run of 32 channels
                              (D/32 per token); ignored else                  */
  int32_t deterministic;   /* 0 or 1. KIVI and FP8 decode: 0 = the
                              wavefronts of a split may take its 32-token
                              tiles from a shared counter as they go
                              (fastest; which wavefront sums which tile
                              varies, so outputs can differ from run to run
                              in the last bits, always within the accuracy
                              bound); 1 = a fixed tile order per wavefront
                              (bitwise identical runs). FP16 decodes are
                              always deterministic.                          */
  int32_t page_tokens;     /* KIVI: 0 = each sequence's grouped region is
                              contiguous; P > 0 = it lives in a pool of pages
                              of P tokens (a power of two ≥ 32 and a multiple
                              of group_size) of every KV head, reached through
                              the cache's block table ([Tutorial] §十三.1,
                              paged attention); the cache must be ragged.
                              Must be 0 for the other formats.                */
  int32_t num_pages;       /* KIVI with page_tokens > 0: pages in the pool
                              (≥ 1); ignored otherwise                        */
} kvq_config;

/* Bytes the caller must allocate for each device buffer (0 = unused). */
typedef struct {
  size_t k_codes, v_codes;
  size_t k_scale, k_zero, v_scale, v_zero;
  size_t k_resid, v_resid;
  size_t tensor_scale;
} kvq_layout;

/* A cache: its configuration, the caller-owned device buffers, and the
 * host-side fill state. Fill the pointers after kvq_cache_init; the library
 * only reads them. n_quant = tokens in the grouped (encoded) region,
 * n_resid = tokens in the FP16 residual window (always 0 for FP8/FP16). */
typedef struct {
  kvq_config cfg;
  void* k_codes;       /* device */
  void* v_codes;       /* device */
  float* k_scale;      /* device, KIVI */
  float* k_zero;       /* device, KIVI */
  float* v_scale;      /* device, KIVI */
  float* v_zero;       /* device, KIVI */
  void* k_resid;       /* device, KIVI */
  void* v_resid;       /* device, KIVI */
  float* tensor_scale; /* device, FP8: [NS][4] {s_K, s_V, amax_K, amax_V} */
  int64_t n_quant;
  int32_t n_resid;
  int32_t reserved;
  /* Ragged mode (KIVI): both non-NULL, host arrays of `batch` entries owned by
   * the caller, holding each sequence's fill levels (grouped tokens, window
   * tokens); the library reads and updates them like n_quant and n_resid.
   * NULL (both): every sequence has the scalar fill levels above. */
  int64_t* seq_n_quant;
  int32_t* seq_n_resid;
  /* Paged KIVI cache (cfg.page_tokens = P > 0): device int32
   * [batch][max_pages], max_pages = ceil(capacity / P), 4-byte aligned; entry
   * [b][j] is the pool page holding tokens [jP, jP + P) of sequence b. The
   * caller fills it before any call that writes or reads those tokens (a
   * prefill, an append whose flush reaches them, a decode over them); the
   * pages of different sequences must be distinct. Entries are read on the
   * device only; one outside [0, num_pages) is clamped into it (the results
   * are then undefined, but no access leaves the pool). NULL otherwise. */
  const int32_t* block_table;
} kvq_cache;

/* Largest batch of a ragged cache (the per-sequence fill levels travel to
 * the kernels as launch arguments). */
#define KVQ_MAX_RAGGED_BATCH 128

/* Sizes of every device buffer a cache with this configuration needs.
 * Errors: INVALID_ARG (null / non-positive fields / bad format),
 * UNSUPPORTED (outside the supported set). */
kvq_status kvq_layout_query(const kvq_config* cfg, kvq_layout* out);

/* Validates cfg (as kvq_layout_query), copies it into *cache, clears every
 * pointer and sets the state to empty (n_quant = n_resid = 0). */
kvq_status kvq_cache_init(kvq_cache* cache, const kvq_config* cfg);

/* Marks the cache empty again (host state only; enqueues nothing); a
 * ragged cache clears every sequence's fill levels. */
kvq_status kvq_cache_reset(kvq_cache* cache);

/* Prefill-time quantization ([Tutorial] §八.4, [Interview] §四; KIVI split
 * into groups and residual per [KIVI-page] §3.2).
 * k, v: device fp16 [B][H][seq_len][D]; read only; must not overlap the cache.
 * KIVI: the first n_quant = G·max(0, min(⌊S/G⌋, ⌈(S−R)/G⌉)) tokens are
 * quantized into groups, the remaining n_resid = S − n_quant (≤ Rcap) tokens
 * are copied into the FP16 window. FP8: amax → scale → encode all S tokens.
 * FP16: copy. Requires an empty cache (else STATE) and 1 ≤ seq_len ≤ C
 * (else INVALID_ARG / CAPACITY). All buffers of the format must be set. */
kvq_status kvq_prefill_quantize(kvq_cache* cache, const void* k, const void* v,
                                int64_t seq_len, void* stream);

/* Prefill of a ragged batch: sequences of different lengths, each
 * quantized as if it were alone in a batch of one (its groups start at its
 * own token 0, its window holds its own newest tokens; [KIVI-page] §3.2 per
 * sequence). The cache must be KIVI and ragged (seq_n_quant and seq_n_resid
 * set; else UNSUPPORTED / INVALID_ARG), with batch ≤ KVQ_MAX_RAGGED_BATCH
 * (else UNSUPPORTED), and every sequence empty (else STATE).
 * k, v: device fp16 [B][H][max_len][D], sequence b in its first seq_lens[b]
 * tokens (the rest is padding and is not read). seq_lens: host int64 [B],
 * 1 ≤ seq_lens[b] ≤ max_len (else INVALID_ARG) and ≤ capacity (else
 * CAPACITY). Sets seq_n_quant[b] = G·max(0, min(⌊S_b/G⌋, ⌈(S_b−R)/G⌉)) and
 * seq_n_resid[b] = S_b − seq_n_quant[b]. */
kvq_status kvq_prefill_quantize_ragged(kvq_cache* cache, const void* k, const void* v,
                                       int64_t max_len, const int64_t* seq_lens,
                                       void* stream);

/* Appends one token per (batch, KV head) ([KIVI-page] §3.1–3.2).
 * k_new, v_new: device fp16 [B][H][D].
 * KIVI: if the window is full (n_resid == Rcap) its Rcap tokens are first
 * quantized into new groups at n_quant (n_quant += Rcap, n_resid = 0); then
 * the token is stored in window slot n_resid. FP8: encoded with the frozen
 * prefill scales (saturating). FP16: copied. CAPACITY when n_quant + n_resid
 * == C. KIVI and FP16 may append to an empty cache; FP8 needs its prefill
 * scales first (else STATE). Ragged KIVI cache: every sequence appends one
 * token; each sequence whose window is full flushes it first, alone;
 * CAPACITY if any sequence is full. */
kvq_status kvq_append_token(kvq_cache* cache, const void* k_new,
                            const void* v_new, void* stream);

/* Workspace bytes kvq_decode_attention needs for any fill state of a cache
 * with this configuration and num_q_heads query heads (0 on invalid input).
 * The workspace holds split partials; its contents need no initialization. */
size_t kvq_decode_workspace_bytes(const kvq_config* cfg, int32_t num_q_heads);

/* One decode step of attention for a single query per head
 * ([Tutorial] §二: softmax(q·Kᵀ/√D)·V over all n_quant + n_resid cached
 * tokens; no mask; GQA mapping as stated above). K and V of the grouped
 * region are dequantized inside the kernel; the window is read as fp16.
 * FP8 caches with fp8_attention = 1 attend with q̂ = e4m3_value(code) · s_q,
 * the codes and scales kvq_quantize_query_fp8 gives for q (computed inside
 * the decode launch, not stored): attention in the FP8 domain.
 * q: device fp32 [B][Hq][D]; out: device fp32 [B][Hq][D] (written);
 * workspace: device, ≥ kvq_decode_workspace_bytes(&cache->cfg, Hq).
 * Ragged KIVI cache: each sequence attends over its own tokens.
 * Errors: STATE on an empty cache (ragged: any empty sequence), WORKSPACE if
 * too small, UNSUPPORTED if Hq is not a multiple of H. */
kvq_status kvq_decode_attention(const kvq_cache* cache, const float* q,
                                int32_t num_q_heads, float* out,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/* kvq_append_token, then kvq_decode_attention, on the same stream: one
 * streamed decode step ([Tutorial] §八.4: the new token's K/V enter the cache,
 * then attention reads it). Every check of both calls runs first (the decode's
 * on the fill state after the append), so on error nothing is enqueued and
 * the cache is unchanged. A KIVI cache with no flush due (ragged: no sequence
 * whose window is full) takes one launch: the decode stores the new token
 * into its window slot and reads it from k_new / v_new. A flush, and every
 * FP8 or FP16 cache, takes the append's launches, then the decode's. The
 * results equal the two calls' (bitwise with deterministic = 1).
 * Arguments as for the two calls; errors as theirs. */
kvq_status kvq_append_decode(kvq_cache* cache, const void* k_new, const void* v_new,
                             const float* q, int32_t num_q_heads, float* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* One decode over the attention layers of a model, layer by layer in index
 * order, for callers that hold every layer's query at once. Each layer keeps
 * its own cache ([Tutorial] §四.4: a layer has its own cache length and KV
 * head count, e.g. sliding-window layers that keep only their last tokens):
 * caches[l] may differ in format, capacity, fill state, num_kv_heads and
 * raggedness; a layer left unquantized ([KIVI-page] §7.1, sensitive layers
 * kept at full precision) is an FP16 cache. All layers share the batch size
 * and num_q_heads (a multiple of each layer's num_kv_heads).
 * q: device fp32 [n_layers][B][Hq][D]; out: same shape (written); workspace:
 * device, ≥ the largest kvq_decode_workspace_bytes of the layers (the
 * layers' launches run one after another on the stream and reuse it).
 * Every layer is checked as kvq_decode_attention checks it, and planned,
 * before anything is enqueued: on error nothing is enqueued and the status
 * is the first failing layer's (INVALID_ARG also for a null caches array,
 * n_layers < 1, a null layer or a batch size unlike layer 0's). */
kvq_status kvq_decode_attention_layers(const kvq_cache* const* caches, int32_t n_layers,
                                       const float* q, int32_t num_q_heads, float* out,
                                       void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Size in bytes of the device array kvq_decode_attention_static keeps its
 * split partials in (one array per GPU the library runs on, reserved when
 * the library's device code is loaded on that GPU and held until the
 * process ends). */
#define KVQ_STATIC_WORKSPACE_BYTES (32u << 20)

/* kvq_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid
 * allocation): the same decode with the same arguments, semantics and errors,
 * but no workspace argument. The split partials go to the library's own
 * device array of KVQ_STATIC_WORKSPACE_BYTES on the current GPU; the call
 * allocates nothing (no hipMalloc, no library allocation).
 * Limit: KVQ_ERR_WORKSPACE, with nothing enqueued, when the partials of the
 * decode as planned (B · Hq · splits · (D + 2) · 4 bytes) would not fit;
 * a configuration with kvq_decode_workspace_bytes(cfg, Hq) ≤
 * KVQ_STATIC_WORKSPACE_BYTES always fits. KVQ_ERR_DEVICE if the array's
 * address cannot be found on the current GPU.
 * Sharing: every call on one GPU uses that GPU's one array, and the array
 * keeps the last call's contents. Calls in stream order on one stream are
 * safe; calls that may run at the same time on one GPU (several streams,
 * several host threads without ordering) race on the array and must be
 * ordered by the caller. Nothing in the array needs clearing: each partial
 * is written before it is read. */
kvq_status kvq_decode_attention_static(const kvq_cache* cache, const float* q,
                                       int32_t num_q_heads, float* out, void* stream);

/* Per-query-head E4M3 quantization of decode queries, the first step of
 * attention in the FP8 domain ([Tutorial] §十八.7; [KIVI-page] §6): one scale
 * per (b, query head) as q_scale has one entry per head ([Tutorial] §十八.6),
 * taken from the current query row since no calibrated scale exists here:
 *   s[b][hq]        = amax_d |q[b][hq][d]| / 448 (fp32, IEEE division);
 *   codes[b][hq][d] = e4m3(min(max(q / s, −448), 448)), round to nearest
 *                     even, the cache's encoder; s = 0 gives codes 0.
 * q: device fp32 [batch][num_q_heads][head_dim], finite; codes: device uint8,
 * same shape; scales: device fp32 [batch][num_q_heads]. q and codes 16-byte
 * aligned, scales 4-byte aligned (else INVALID_ARG); batch, num_q_heads ≥ 1
 * (else INVALID_ARG), head_dim = 128 and batch·num_q_heads ≤ 2^31 − 1 (else
 * UNSUPPORTED). Caller-owned buffers; nothing is allocated. */
kvq_status kvq_quantize_query_fp8(const float* q, int32_t batch, int32_t num_q_heads,
                                  int32_t head_dim, uint8_t* codes, float* scales,
                                  void* stream);

/* Algorithmic bytes one decode step must read from the cache at its current
 * fill state: codes, scales and zero-points of the grouped region plus the
 * fp16 window (KIVI); codes plus the K and V scales, per tensor or per KV
 * head (FP8); fp16 K and V (FP16).
 * Query and output bytes are not included; a ragged cache sums its
 * sequences. −1 on invalid input. */
int64_t kvq_decode_bytes(const kvq_cache* cache, int32_t num_q_heads);

/* The pages' KV byte formula 2·L·B·S·H_kv·D·bytes_per_elem
 * ([KIVI-page] §1; [Tutorial] §四; [Interview] §三). */
double kvq_theoretical_bytes(int32_t num_layers, int32_t batch, int64_t seq_len,
                             int32_t num_kv_heads, int32_t head_dim,
                             double bytes_per_elem);

/* The pages' mixed-layer KV byte formula 2·B·bytes_per_elem·Σ_l S_l·H_kv,l·D_l
 * ([Tutorial] §四.4), for layers with their own cache length seq_len[l], KV
 * heads num_kv_heads[l] and head dim head_dim[l] (host arrays of n_layers).
 * −1 on invalid input (n_layers < 1, null arrays, negative sizes). */
double kvq_theoretical_bytes_layers(int32_t n_layers, int32_t batch, const int64_t* seq_len,
                                    const int32_t* num_kv_heads, const int32_t* head_dim,
                                    double bytes_per_elem);

/* Static description of a status code (never NULL). */
const char* kvq_status_str(kvq_status status);

/* KVQ_ABI_VERSION of the loaded library. */
int32_t kvq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
