/*
 * mla.h -- C ABI of the MI355X (gfx950) Multi-Head Latent Attention library.
 *
 * One attention layer in the weight-absorbed form over a latent KV cache:
 * each cached token is ONE row [c_kv (kv_lora) | k_rope (qk_rope)], the
 * RMS-normalised latent followed by the RoPE-rotated key shared by all heads
 * ("Multi-Head Latent Attention" post, sections 3.1 C cache and 3.6
 * Decoupled RoPE).  Decode folds W_UK into the query so scores are taken
 * against the latent rows directly and applies W_UV after the
 * probability-weighted latent sum (same post, section 3.3 Absorption,
 * eq. 3.3.3).  Prefill is causal and chunked (the "Transformer and KV Cache
 * Basics" page, KV Cache / mask design: query positions are offset by the
 * cached length).
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers.  Tensors (weights, hidden states, the cache, outputs, workspace)
 *   are DEVICE pointers.  The small ragged metadata arrays (pos, slot,
 *   seq_off, seq_len, cu_new, prior_len) are HOST arrays: the library
 *   validates them on the host before any launch and copies what the kernels
 *   need into the caller's workspace, asynchronously, through pinned staging
 *   memory it owns.
 * Element type.  Every tensor argument holds elements of the handle's dtype
 *   (bf16 for MLA_BF16, float for MLA_F32), row-major, densely packed.
 * Layouts.  Weight matrices are (out, in) row-major, like a linear layer's
 *   weight (y = x W^T).  Per head h, q_proj rows [h*(dn+dr), (h+1)*(dn+dr))
 *   are [q_nope_h | q_rope_h]; kv_b_proj rows [h*(dn+dv), (h+1)*(dn+dv)) are
 *   [K_nope_h ; V_h] ("Deepseek V2 Lite Inference Engine in C", MLA notes:
 *   the K and V values of each head are interleaved).  kv_a_proj rows are
 *   [latent (kv_lora) ; rope key (qk_rope)].  The cache is (cache_rows, R)
 *   with R = kv_lora + qk_rope, or cache_rows rows of mla_cache_row_bytes
 *   bytes when the config asks for FP8 rows (mla_kv_storage).
 * Ownership.  The caller owns every tensor, cache, output and workspace
 *   buffer.  The library owns only the handle, its repacked weight copies and
 *   its pinned staging memory.
 * Streams.  All calls are asynchronous on the handle's HIP stream (the one
 *   given to mla_create / mla_set_stream; NULL = the null stream).  Nothing
 *   synchronises implicitly except mla_absorb_weights and mla_destroy.
 * Graph capture.  mla_append_latent, mla_cache_write, mla_decode and
 *   mla_prefill may be captured into a HIP graph: while the stream is
 *   capturing, the metadata a call uploads are staged in pinned memory kept
 *   for the life of the handle (the graph's copy node reads it at every
 *   replay), so a replay re-runs the call with the metadata of capture time.
 * Errors.  Every call returns an mla_status.  Argument, shape and capacity
 *   errors are detected on the host before anything is launched and leave all
 *   device memory untouched.  MLA_ERR_HIP reports a failed HIP runtime call;
 *   mla_last_error(h) returns a description of the last failure on h.
 * Threads.  A handle may be used by one host thread at a time.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 9

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1, /* null pointer, count <= 0, pos != len-1, duplicate slot ... */
  MLA_ERR_SHAPE = -2,       /* unsupported dimensions (e.g. odd qk_rope) */
  MLA_ERR_CAPACITY = -3,    /* a slot or a sequence's rows fall outside the cache */
  MLA_ERR_STATE = -4,       /* call out of order (e.g. decode before absorb) */
  MLA_ERR_HIP = -5,         /* a HIP runtime call failed */
  MLA_ERR_WORKSPACE = -6    /* workspace missing, too small or misaligned */
} mla_status;

typedef enum mla_dtype { MLA_BF16 = 0, MLA_F32 = 1 } mla_dtype;

/* How the latent cache stores a row.  MLA_KV_DTYPE: R = kv_lora + qk_rope
 * values of the layer dtype.  MLA_KV_FP8_E4M3 ("Multi-Head Latent Attention"
 * post: low-precision storage, introduction; 1-byte FP8 cache elements,
 * section 3.1): fp8_row_bytes = 656 bytes per row for kv_lora 512 / qk_rope
 * 64, laid out as [kv_lora OCP FP8 E4M3 codes | qk_rope bf16 | fp32 scale s |
 * zero pad to a multiple of 16]; the latent values are c_i = s * value(code_i)
 * with s = max_i |c_i| / 448 (1 for an all-zero row) and code_i the E4M3
 * value nearest c_i / s (ties to even).  FP8 needs dtype MLA_BF16, kv_lora
 * 512, qk_rope 64 and n_heads a multiple of 16; it serves append, decode and
 * prefill (which decodes the key rows it reads to bf16, c_i rounded once). */
typedef enum mla_kv_storage { MLA_KV_DTYPE = 0, MLA_KV_FP8_E4M3 = 1 } mla_kv_storage;

/* How decode applies the absorbed weights ("Multi-Head Latent Attention"
 * post, section 3.5; "Deepseek V2 Lite Inference Engine in C", MLA notes,
 * variant 2 against variant 3).  MLA_ABSORB_FACTORED: the query path keeps
 * W_q (or W_qb) and W_UK apart (q_abs_h = W_UK_h^T (W_q x)_h) and the output
 * keeps W_UV and W_o apart (y = W_o [W_UV_h o_lat_h]_h).
 * MLA_ABSORB_MATERIALIZED: mla_absorb_weights also forms W^KQ_h = W_UK_h^T
 * W_q,nope_h (d_c x D, or d_c x q_lora) and W^OV_h = W_o,h W_UV_h (D x d_c)
 * once, so the decode step reads q_abs_h = W^KQ_h x straight from the
 * projection and y = sum_h W^OV_h o_lat_h from one product over the latent
 * sums: fewer launches, more weight bytes (V2-Lite: 71 MB against 21 MB per
 * step).  Materialised weights are used by the fused decode path (bf16
 * layers, kv_lora 512, up to 128 query rows); larger batches and prefill use
 * the factored weights, which the handle keeps as well. */
typedef enum mla_absorb { MLA_ABSORB_FACTORED = 0, MLA_ABSORB_MATERIALIZED = 1 } mla_absorb;

/* Layer dimensions (MLA post, section 3.2 constructor; section 3.6 widths).
 * qk_rope must be even (RoPE rotates pairs; MLA post section 3.7).  q_lora = 0
 * means the query is projected straight from the hidden state (w_q); > 0
 * means q = W_qb RMSNorm(W_qa x) (MLA post section 3.1, query compression). */
typedef struct mla_config {
  int32_t hidden;    /* D */
  int32_t n_heads;   /* H */
  int32_t qk_nope;   /* dn */
  int32_t qk_rope;   /* dr, even, <= 128; 0 allowed (no decoupled RoPE) */
  int32_t v_head;    /* dv */
  int32_t kv_lora;   /* dc */
  int32_t q_lora;    /* dq, 0 = none */
  float rope_base;   /* RoPE base, e.g. 10000 */
  float rms_eps;     /* RMSNorm epsilon, e.g. 1e-6 */
  float softmax_scale; /* 0 -> 1/sqrt(dn + dr) */
  int32_t dtype;     /* mla_dtype: storage type of every tensor (but see kv_storage) */
  int32_t kv_storage; /* mla_kv_storage: format of the latent cache rows */
  /* YaRN context extension of the RoPE frequencies (the C-engine notes,
   * "Deepseek V2 Lite Inference Engine in C", name YaRN without a formula;
   * read as YaRN's "NTK-by-parts" interpolation in the form DeepSeek layers
   * run it).  With rope_scale = s > 1: pair i of plain frequency theta_i =
   * base^(-2i/dr) turns rope_orig_max * theta_i / (2 pi) times over the
   * original context; let p(n) = dr * ln(rope_orig_max / (2 pi n)) /
   * (2 ln base) be the pair index that turns n times, lo = max(floor(
   * p(yarn_beta_fast)), 0), hi = min(ceil(p(yarn_beta_slow)), dr/2 - 1)
   * (hi = lo + 0.001 if hi <= lo) and w_i = clamp((i - lo) / (hi - lo), 0, 1);
   * the frequency used is (1 - w_i) theta_i + w_i theta_i / s.  When
   * softmax_scale is 0 the default scale is multiplied by YaRN's attention
   * factor (0.1 yarn_mscale ln s + 1)^2 (DeepSeek's per-model coefficient m;
   * 0 leaves the scale unchanged).  rope_scale <= 1 (0 included): plain RoPE,
   * the other four fields unused. */
  float rope_scale;
  int32_t rope_orig_max;  /* original context length, >= 1 when rope_scale > 1 */
  float yarn_beta_fast;   /* e.g. 32 */
  float yarn_beta_slow;   /* e.g. 1; 0 < slow < fast */
  float yarn_mscale;      /* e.g. 0.707 (V2-Lite) or 1 (V3); >= 0 */
  int32_t absorb;         /* mla_absorb: how the decode path applies the absorbed weights */
} mla_config;

typedef struct mla_ctx* mla_handle;

/* Host-only check of a configuration: MLA_OK, MLA_ERR_INVALID_ARG (cfg NULL,
 * a dimension <= 0 other than qk_rope/q_lora, a negative one, unknown dtype,
 * non-finite or non-positive base/eps, unknown kv_storage, rope_scale > 1 with
 * rope_orig_max < 1, not 0 < yarn_beta_slow < yarn_beta_fast or a negative or
 * non-finite yarn_mscale, unknown absorb) or MLA_ERR_SHAPE (odd qk_rope,
 * qk_rope > 128, kv_lora > 1024, v_head > 256, FP8 rows for a layer outside
 * the FP8 shapes, materialised absorption outside bf16 layers with kv_lora
 * 512).  Makes no HIP call; mla_create runs it
 * first. */
int mla_config_check(const mla_config* cfg);

/* Bytes of one cached latent row under cfg (R * element size, or the FP8 row
 * size); 0 if mla_config_check fails.  Host only.  A cache of cache_rows rows
 * is cache_rows * mla_cache_row_bytes(cfg) bytes. */
size_t mla_cache_row_bytes(const mla_config* cfg);

/* Host-only argument checks, run first by the corresponding calls and exported
 * so callers (and tests without a GPU) can validate before enqueuing.  They
 * make no HIP call and return the status the call itself would return for
 * these arguments (weights/workspace state aside). */
int mla_append_check(const mla_config* cfg, const int32_t* pos, const int64_t* slot, int32_t T,
                     int64_t cache_rows);
int mla_decode_check(const mla_config* cfg, const int32_t* pos, const int64_t* seq_off,
                     const int32_t* seq_len, int32_t B, int64_t cache_rows);
int mla_prefill_check(const mla_config* cfg, const int32_t* cu_new, const int32_t* prior_len,
                      const int64_t* seq_off, int32_t B, int64_t cache_rows);
/* The checks of mla_prefill_paged; see there. */
int mla_prefill_paged_check(const mla_config* cfg, const int32_t* cu_new,
                            const int32_t* prior_len, const int32_t* block_table,
                            int32_t max_pages, int32_t page_rows, int32_t B, int64_t cache_rows);
/* The checks of mla_decode_paged (writes = 0) and mla_decode_step_paged
 * (writes = 1); see there. */
int mla_decode_paged_check(const mla_config* cfg, const int32_t* pos, const int32_t* block_table,
                           int32_t max_pages, int32_t page_rows, const int32_t* seq_len, int32_t B,
                           int64_t cache_rows, int32_t writes);

/* Create a handle on the current HIP device.  stream: a hipStream_t or NULL.
 * *out receives the handle (NULL on failure).
 * With the environment variable MLA_LOG set (to anything but "0") when the
 * library first logs, mla_create and every decode and prefill call print one
 * line on stderr: the layer and its attention core, or the call's shape, work
 * plan (parts, segments, combine chunks, attention tiles) and workspace. */
int mla_create(const mla_config* cfg, void* stream, mla_handle* out);

/* Synchronise the handle's stream and free everything the library owns. */
int mla_destroy(mla_handle h);

/* Change the stream later calls are issued on. */
int mla_set_stream(mla_handle h, void* stream);

/* A1 -- copy and repack the layer weights (MLA post section 3.5: W_UK and W_UV
 * are split out of kv_b_proj per head and kept separate, NOT multiplied into
 * W^KQ / W^OV).  Pass w_q (H*(dn+dr), D) when q_lora == 0, else w_qa (dq, D),
 * q_norm_g (dq) and w_qb (H*(dn+dr), dq); the unused ones must be NULL.
 * w_kva (dc+dr, D); kv_norm_g (dc) or NULL for ones; w_kvb (H*(dn+dv), dc);
 * w_o (D, H*dv).  All device pointers; the caller may free them on return
 * (this call synchronises the stream).  May be called again to replace the
 * weights. */
int mla_absorb_weights(mla_handle h, const void* w_q, const void* w_qa,
                       const void* q_norm_g, const void* w_qb, const void* w_kva,
                       const void* kv_norm_g, const void* w_kvb, const void* w_o);

/* Workspace bytes mla_append_latent needs for T tokens (256-byte aligned
 * base required). */
size_t mla_append_workspace_bytes(mla_handle h, int32_t T);

/* A2 -- append T tokens to the latent cache: a = W_kva x;
 * cache[slot[t]] = [RMSNorm(a[:dc]) * kv_norm_g | RoPE(a[dc:], pos[t])],
 * rounded to the storage type, or for FP8 rows the latent part quantised
 * from its fp32 values as mla_kv_storage describes and the rope part rounded
 * to bf16 ("Deepseek V2 Lite Inference Engine in C", MLA notes: kv_a_proj
 * fuses the down-projection and the shared rope key; MLA post sections 3.5
 * and 3.7).  hidden: device (T, D).  pos, slot: HOST arrays of T
 * entries; pos >= 0; slots must be distinct and in [0, cache_rows)
 * (MLA_ERR_CAPACITY otherwise, the KV-cache page's overflow condition).
 * Rows not named in slot are not touched. */
int mla_append_latent(mla_handle h, const void* hidden, const int32_t* pos,
                      const int64_t* slot, int32_t T, void* cache, int64_t cache_rows,
                      void* ws, size_t ws_bytes);

/* Raw scatter of T ready-made rows into cache[slot[t]] -- the indexing half of
 * mla_append_latent on its own (bit-exact copy).  rows: device, T rows in the
 * cache's own format (T x R values, or T x mla_cache_row_bytes bytes for FP8
 * rows).  Same slot rules.  mla_cache_store takes the same arguments but rows
 * of R values in the layer dtype and stores them in the cache's format
 * (quantised as mla_kv_storage describes for FP8 rows, from the values as
 * given; a plain copy otherwise); its workspace is mla_cache_write's. */
size_t mla_cache_write_workspace_bytes(mla_handle h, int32_t T);
int mla_cache_write(mla_handle h, const void* rows, const int64_t* slot, int32_t T,
                    void* cache, int64_t cache_rows, void* ws, size_t ws_bytes);
int mla_cache_store(mla_handle h, const void* rows, const int64_t* slot, int32_t T,
                    void* cache, int64_t cache_rows, void* ws, size_t ws_bytes);

/* Workspace bytes mla_decode needs for B sequences holding total_rows cache
 * rows in all (sum of seq_len). */
size_t mla_decode_workspace_bytes(mla_handle h, int32_t B, int64_t total_rows);

/* A3..A8 -- decode one new token per sequence over a ragged batch, absorbed
 * form.  The caller has already appended each sequence's new row (write, then
 * read through the new position: MLA post section 3.2), so sequence b owns
 * cache rows [seq_off[b], seq_off[b] + seq_len[b]) holding positions
 * 0 .. seq_len[b]-1 and its query is at pos[b] == seq_len[b] - 1.
 *   hidden: device (B, D) -- the new tokens' hidden states.
 *   pos, seq_off, seq_len: HOST arrays of B entries.
 *   out: device (B, D) -- y = W_o [W_UV_h o_lat_h]_h.
 * Errors: B <= 0 or NULL -> INVALID_ARG; seq_len[b] < 1 or pos[b] !=
 * seq_len[b]-1 -> INVALID_ARG; seq_off[b] < 0 or seq_off[b]+seq_len[b] >
 * cache_rows -> CAPACITY; weights not absorbed -> STATE; workspace too small
 * -> WORKSPACE. */
int mla_decode(mla_handle h, const void* hidden, const int32_t* pos,
               const int64_t* seq_off, const int32_t* seq_len, int32_t B,
               const void* cache, int64_t cache_rows, void* out, void* ws,
               size_t ws_bytes);

/* Workspace bytes mla_decode_step needs (same arguments as for mla_decode). */
size_t mla_decode_step_workspace_bytes(mla_handle h, int32_t B, int64_t total_rows);

/* A2..A8 in one call -- append each sequence's new token, then decode it
 * (write, then read through the new position: MLA post section 3.2).  The
 * same arguments as mla_decode, but the caller has NOT appended the new rows:
 * this call writes row seq_off[b] + seq_len[b] - 1 of the cache (position
 * pos[b] = seq_len[b] - 1) from hidden[b] exactly as mla_append_latent would,
 * then decodes.  The latent down-projection and the query projection read the
 * same hidden states, so they run as one GEMM over [W_kva ; W_q] (or
 * [W_kva ; W_qa]).  Same errors as mla_decode, plus INVALID_ARG when two
 * sequences' new rows are the same cache row or a new row lies inside
 * another sequence's rows (it would be overwritten before it is read). */
int mla_decode_step(mla_handle h, const void* hidden, const int32_t* pos,
                    const int64_t* seq_off, const int32_t* seq_len, int32_t B, void* cache,
                    int64_t cache_rows, void* out, void* ws, size_t ws_bytes);

/* mla_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (tight serving loops, harnesses that forbid
 * hipMalloc).  The step's workspace is a static device array of
 * MLA_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held from
 * the library's load until the process ends; its address is taken at
 * mla_create, which also pins the host staging memory this call uses, so the
 * call itself allocates nothing.  Same arguments (minus ws / ws_bytes),
 * kernels, results and errors as mla_decode_step, plus: MLA_ERR_WORKSPACE when
 * mla_decode_step_workspace_bytes(h, B, sum of seq_len) exceeds
 * MLA_NOALLOC_SCRATCH_BYTES (32 MiB holds, e.g., a V2-Lite-shaped step of 64
 * sequences; 128-head layers need more) or the step's metadata exceed the
 * staged pinned memory; MLA_ERR_STATE while the handle's stream is being
 * captured into a graph.  All calls on one GPU share that GPU's array, which
 * keeps the last call's contents: calls that overlap on one GPU (other
 * streams, other handles, other threads) race and must be serialised by the
 * caller. */
#define MLA_NOALLOC_SCRATCH_BYTES (32u << 20)
int mla_decode_step_noalloc(mla_handle h, const void* hidden, const int32_t* pos,
                            const int64_t* seq_off, const int32_t* seq_len, int32_t B, void* cache,
                            int64_t cache_rows, void* out);

/* Paged latent cache -- mla_decode and mla_decode_step over a cache managed
 * as a pool of pages (the KV-cache page grows its cache as a memory pool; the
 * MLA post's reference code preallocates one contiguous buffer).  The cache
 * holds cache_rows rows in its usual row format; page k is rows
 * [k * page_rows, (k + 1) * page_rows), k < cache_rows / page_rows.  Position
 * t of sequence b is row block_table[b * max_pages + t / page_rows] *
 * page_rows + t % page_rows.  Pages may be shared between sequences (a
 * common prefix) and need not be in any order.
 *   block_table: HOST (B, max_pages) int32; only the first
 *     ceil(seq_len[b] / page_rows) entries of row b are read.
 *   page_rows: a power of two, 32 .. 2^30 (a 32-row tile of the decode cores
 *     never crosses a page).
 *   pos, seq_len: HOST, as for mla_decode (pos[b] == seq_len[b] - 1).
 * mla_decode_step_paged writes each new row at position seq_len[b] - 1,
 * through the block table; those rows must be distinct.  Results are those of
 * mla_decode / mla_decode_step on a contiguous cache holding the same rows
 * (bit for bit: the work split depends on seq_len only).  Workspace: the
 * contiguous call's (mla_decode_workspace_bytes,
 * mla_decode_step_workspace_bytes with the same B and total rows).
 * Errors: as mla_decode; page_rows not a power of two in range, max_pages < 1
 * or a NULL table -> INVALID_ARG; more pages needed than max_pages, or a page
 * index outside [0, cache_rows / page_rows) -> CAPACITY; two new rows of a
 * step on the same cache row, or a new row on a row that some sequence reads
 * as already cached (e.g. inside a shared prefix page) -> INVALID_ARG. */
int mla_decode_paged(mla_handle h, const void* hidden, const int32_t* pos,
                     const int32_t* block_table, int32_t max_pages, int32_t page_rows,
                     const int32_t* seq_len, int32_t B, const void* cache, int64_t cache_rows,
                     void* out, void* ws, size_t ws_bytes);
int mla_decode_step_paged(mla_handle h, const void* hidden, const int32_t* pos,
                          const int32_t* block_table, int32_t max_pages, int32_t page_rows,
                          const int32_t* seq_len, int32_t B, void* cache, int64_t cache_rows,
                          void* out, void* ws, size_t ws_bytes);

/* General decode call: q_len new tokens per sequence (multi-token decode: the
 * offset causal mask of "Transformer and KV Cache Basics", KV Cache section --
 * new token j of sequence b sits at position seq_len[b] - q_len + j and
 * attends to positions 0 .. that position; the MLA post's section 3.2 code
 * writes the new tokens' rows before reading), over a contiguous or a paged
 * cache, with or without the append of the new rows.  q_len = 1 is
 * mla_decode / mla_decode_step (or their paged forms), bit for bit. */
#define MLA_MAX_Q_LEN 16
typedef struct mla_decode_args {
  const void* hidden;         /* device (B * q_len, D): row b * q_len + j is token j of b */
  void* out;                  /* device (B * q_len, D), same order */
  int32_t B;                  /* sequences, >= 1 */
  int32_t q_len;              /* new tokens per sequence, 1 .. MLA_MAX_Q_LEN */
  const int32_t* seq_len;     /* HOST (B): rows of sequence b including its q_len new ones;
                                 >= q_len */
  const int64_t* seq_off;     /* HOST (B): contiguous cache, rows [seq_off[b], + seq_len[b]);
                                 NULL for a paged cache */
  const int32_t* block_table; /* HOST (B, max_pages): paged cache as for mla_decode_paged;
                                 NULL for a contiguous cache */
  int32_t max_pages;
  int32_t page_rows;
  void* cache;                /* device, cache_rows rows in the cache's row format */
  int64_t cache_rows;
  int32_t append;             /* 1: write the q_len new rows of every sequence from hidden
                                 first (as mla_append_latent would), then decode */
  void* ws;                   /* workspace of mla_decode_ex_workspace_bytes bytes */
  size_t ws_bytes;
} mla_decode_args;

/* Host-only checks of mla_decode_ex.  Errors: NULL args/seq_len, B < 1, q_len
 * outside 1 .. MLA_MAX_Q_LEN, seq_len[b] < q_len, both or neither of seq_off
 * and block_table -> INVALID_ARG; a contiguous sequence outside
 * [0, cache_rows) -> CAPACITY; paged: the errors of mla_decode_paged.  With
 * append, all B * q_len new rows must land on distinct cache rows, none of
 * them on a row some sequence reads as cached (INVALID_ARG otherwise). */
int mla_decode_ex_check(const mla_config* cfg, const mla_decode_args* a);
/* Workspace bytes for B sequences of total_rows rows in all (sum of seq_len),
 * q_len new tokens each, with (append = 1) or without the append. */
size_t mla_decode_ex_workspace_bytes(mla_handle h, int32_t B, int32_t q_len, int64_t total_rows,
                                     int32_t append);
/* Runs the decode described by a (A2 if append, then A3..A8 for all B * q_len
 * query rows).  Errors: those of mla_decode_ex_check, weights not absorbed ->
 * STATE, workspace too small -> WORKSPACE. */
int mla_decode_ex(mla_handle h, const mla_decode_args* a);

/* Where the staged intermediates of the last mla_decode with these (B,
 * total_rows) live inside its workspace, as byte offsets from ws:
 *   q_cat (B, H, R) storage type: [W_UK_h^T q_nope_h | RoPE(q_rope_h)] * scale
 *   o_lat (B, H, dc) storage type: the probability-weighted latent sum.
 * For staged parity tests; valid until the workspace is reused. */
int mla_decode_stage_offsets(mla_handle h, int32_t B, int64_t total_rows,
                             size_t* q_cat_off, size_t* o_lat_off);

/* Host-only view of the split-S work list mla_decode / mla_decode_step build
 * ("Multi-Head Latent Attention" post, section 3.6: every cached latent row is
 * read once per head group; here the rows of the whole batch are spread over
 * the compute units).  The concatenated rows of the B sequences are cut into
 * at most max_parts contiguous spans (one persistent workgroup each), each span
 * split at sequence boundaries into segments; spans are balanced on rows plus
 * a fixed per-segment cost, and cuts inside a sequence fall on multiples of 32
 * rows (one tile of the MFMA cores).  The library itself uses max_parts = the
 * device's compute units divided by the number of workgroups a part runs (one
 * per 16-head group; one per 128 heads for layers with a multiple of 128
 * heads, bf16 or FP8 rows).
 *   seq_len: HOST (B), each >= 1.
 *   part_begin: HOST out (max_parts + 1): segments of part p are
 *     [part_begin[p], part_begin[p+1]).
 *   seg_b, seg_r0, seg_r1: HOST out (B + max_parts - 1 each): segment i covers
 *     rows [seg_r0[i], seg_r1[i]) of sequence seg_b[i]; segments are in
 *     row order.
 *   n_parts, n_segs: HOST out.
 * No device work.  Errors: INVALID_ARG (null pointer, B or max_parts < 1, a
 * length < 1). */
int mla_decode_plan(int32_t B, const int32_t* seq_len, int32_t max_parts, int32_t* part_begin,
                    int32_t* seg_b, int32_t* seg_r0, int32_t* seg_r1, int32_t* n_parts,
                    int32_t* n_segs);

/* mla_decode_plan for q_len new tokens per sequence (mla_decode_ex): the
 * same work list, except that a sequence's last segment keeps at least q_len
 * rows, so every new token's causal limit (its own position) falls in that
 * segment and the segments before it are whole for every token.
 *   q_len: 1 .. MLA_MAX_Q_LEN; seq_len[b] >= q_len (cached rows + new rows).
 * Other arguments as mla_decode_plan; q_len = 1 gives its result.  Errors:
 * INVALID_ARG as there, or q_len out of range, or a length below q_len. */
int mla_decode_plan_tokens(int32_t B, const int32_t* seq_len, int32_t q_len, int32_t max_parts,
                           int32_t* part_begin, int32_t* seg_b, int32_t* seg_r0, int32_t* seg_r1,
                           int32_t* n_parts, int32_t* n_segs);

/* Workspace bytes mla_prefill (mla_prefill_paged) needs for T new tokens in
 * B sequences whose caches hold total_key_rows rows in all after the append.
 * An FP8 or paged cache adds room for the key rows gathered in the storage
 * type (total_key_rows * R elements). */
size_t mla_prefill_workspace_bytes(mla_handle h, int32_t T, int32_t B,
                                   int64_t total_key_rows);
size_t mla_prefill_paged_workspace_bytes(mla_handle h, int32_t T, int32_t B,
                                         int64_t total_key_rows);

/* P1 -- causal chunked prefill.  Sequence b has prior_len[b] cached rows and
 * new tokens hidden[cu_new[b] .. cu_new[b+1]) at positions prior_len[b],
 * prior_len[b]+1, ...; the caller has already appended the new rows, so the
 * sequence owns cache rows [seq_off[b], seq_off[b] + prior_len[b] + n_b).
 * Each new token attends to rows 0..its position (KV-cache page: the
 * position-offset causal mask).
 *   hidden: device (T, D), T = cu_new[B]; out: device (T, D).
 *   cu_new: HOST (B+1), cu_new[0] = 0, non-decreasing; prior_len, seq_off:
 *   HOST (B).
 * An FP8 cache's key rows are first decoded into the workspace (c_i = s *
 * value(code_i) rounded to bf16), then expanded and attended as bf16 rows.
 * Errors as for mla_decode (CAPACITY if a sequence's rows leave the cache;
 * INVALID_ARG if prior_len[b] + n_b exceeds INT32_MAX). */
int mla_prefill(mla_handle h, const void* hidden, const int32_t* cu_new,
                const int32_t* prior_len, const int64_t* seq_off, int32_t B,
                const void* cache, int64_t cache_rows, void* out, void* ws,
                size_t ws_bytes);

/* A2 + P1 -- the prefill step: appends the T new tokens' latent rows (as
 * mla_append_latent with pos = prior_len[b] + i at cache row seq_off[b] +
 * prior_len[b] + i) and then runs mla_prefill on them, in one call.  For a
 * layer with a query LoRA the append's product and the query's first
 * projection read the hidden states once (in the DeepSeek code the
 * "Multi-Head Latent Attention" post quotes in section 3.4, wkv_a and wq_a
 * both take the same hidden state): one product over [W_kva ; W_qa], or for
 * many tokens two products over one tiled copy of the hidden states.
 * Contiguous caches (bf16, fp32 or FP8 rows).
 *   Arguments as for mla_prefill; cache is written (the new rows) and read.
 *   Workspace: mla_prefill_step_workspace_bytes (>= mla_prefill's).
 * Errors: those of mla_prefill, and INVALID_ARG if two new rows share a cache
 * row or a new row is a row some sequence reads as cached
 * (mla_prefill_step_check). */
size_t mla_prefill_step_workspace_bytes(mla_handle h, int32_t T, int32_t B,
                                        int64_t total_key_rows);
int mla_prefill_step_check(const mla_config* cfg, const int32_t* cu_new,
                           const int32_t* prior_len, const int64_t* seq_off, int32_t B,
                           int64_t cache_rows);
int mla_prefill_step(mla_handle h, const void* hidden, const int32_t* cu_new,
                     const int32_t* prior_len, const int64_t* seq_off, int32_t B, void* cache,
                     int64_t cache_rows, void* out, void* ws, size_t ws_bytes);

/* mla_prefill over a paged cache (the page pool of mla_decode_paged; the
 * KV-cache page grows its cache as a memory pool): position t of sequence b
 * is row block_table[b * max_pages + t / page_rows] * page_rows + t %
 * page_rows, for t < prior_len[b] + n_b (the caller has appended the new rows
 * through the same table, e.g. with mla_append_latent).  The key rows are
 * gathered into the workspace (decoded from FP8 for an FP8 cache) and the
 * prefill runs on them; results equal mla_prefill's on a contiguous cache
 * holding the same rows in the same sequence order, bit for bit.
 *   block_table: HOST (B, max_pages) int32; page_rows: a power of two, 32 ..
 *   2^30.  Workspace: mla_prefill_paged_workspace_bytes.
 * Errors: those of mla_prefill; page_rows not a power of two in range,
 * max_pages < 1 or a NULL table -> INVALID_ARG; more pages needed than
 * max_pages, or a page index outside [0, cache_rows / page_rows) ->
 * CAPACITY. */
int mla_prefill_paged(mla_handle h, const void* hidden, const int32_t* cu_new,
                      const int32_t* prior_len, const int32_t* block_table, int32_t max_pages,
                      int32_t page_rows, int32_t B, const void* cache, int64_t cache_rows,
                      void* out, void* ws, size_t ws_bytes);

/* Measurement: with n_slots > 0, every later launch of the attention core
 * (the split-S kernel of mla_decode / mla_decode_step, the attention kernel of
 * mla_prefill) is bracketed by a pair of HIP events on the handle's stream,
 * kept in a ring of n_slots pairs.  The events are created without the
 * system-scope fence, so recording them neither writes back nor invalidates
 * caches.  Launches recorded while the stream is being captured into a graph
 * are not timed.  n_slots = 0 turns timing off.  Waits for the stream first.
 * Errors: INVALID_ARG (n_slots < 0), HIP. */
int mla_core_timing(mla_handle h, int32_t n_slots);

/* Durations in ms of the last min(n, timed launches, n_slots) timed core
 * launches, oldest first, into ms (HOST, n floats); *n_out = how many.  Waits
 * for those launches to finish. */
int mla_core_timing_read(mla_handle h, float* ms, int32_t n, int32_t* n_out);

/* Static text for a status code. */
const char* mla_status_string(int status);

/* Description of the last failure on h (empty string if none). */
const char* mla_last_error(mla_handle h);

/* ABI version the library was built with (MLA_ABI_VERSION). */
int mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
