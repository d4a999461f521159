/*
 * kvattn.h — C ABI of the MI355X (gfx950) grouped-query attention library.
 *
 * Four operators, each following one ONNX-Runtime contrib operator page:
 *
 *   gqa_attention     com.microsoft.GroupQueryAttention page
 *   decode_mha        com.microsoft.DecoderMaskedMultiHeadAttention page
 *   sparse_attention  com.microsoft.SparseAttention page
 *   packed_attention  com.microsoft.PackedAttention page
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors.  Every tensor argument is a kvattn_tensor: a DEVICE pointer to a
 * contiguous row-major buffer plus its element type and dims.  An optional
 * input that is absent has data == NULL and rank 0.  A present tensor with
 * no elements (a zero dim) may have data == NULL; calls over an empty batch
 * or an empty new sequence launch nothing that touches it.  The
 * input slots of each operator follow the order of that page's Inputs table;
 * the output slots follow its Outputs table.  The caller passes the slot
 * count it filled (n_inputs / n_outputs) and the library checks it.
 *
 * Host and device data.  Shapes, attributes and total_sequence_length are
 * host values; they fix grids, output shapes and broadcast strides.  Per-batch
 * lengths (seqlens_k, past_sequence_length, key_total_sequence_lengths), the
 * CSR layouts, token_offset and cumulative_sequence_length stay in device
 * memory and are read by the kernels, so a call never synchronises the
 * stream.  Device-data preconditions (lengths inside the cache capacity,
 * monotone CSR row pointers, a well-formed packed schedule) cannot be checked
 * without a copy; when they are violated the outputs are unspecified, but no
 * kernel reads or writes outside the buffers described by the dims.
 *
 * Ownership.  The caller allocates every input, output and the workspace.
 * The library never allocates, frees or synchronises; all work is enqueued
 * on `stream` (a hipStream_t; NULL = the default stream).  The workspace size
 * comes from the matching *_workspace_size call made with the same
 * arguments.  Every non-empty workspace begins with KVATTN_COUNTER_BYTES of
 * arrival counters: single-token decode calls (gqa_attention with a past and
 * S = 1, decode_mha, sparse_attention generating one token) keep one int32
 * there per (sample, kv head, query-head group) unit whose keys they split
 * over several pairs of waves; the pairs count themselves in and the last
 * one merges the unit (one launch, no merge dispatch).  Those bytes must be
 * zero when a call starts; every call leaves them zero and no call writes
 * anything else there.  So: allocate a workspace zero-filled once, then
 * reuse it for calls of any operator and shape.  The rest of the workspace
 * needs no initialisation and is not preserved.  Calls that may run at the
 * same time must not share a workspace.
 *
 * Errors.  Every call returns KVATTN_OK (0) or a negative kvattn_status.
 * All validation happens before the first launch, so a failed call writes
 * nothing.  kvattn_last_error() returns a thread-local message describing the
 * most recent failure on the calling thread.  Faults of enqueued kernels
 * surface at the caller's next stream synchronisation.  No C++ exception
 * crosses this interface.
 *
 * Storage types.  T is float32 or float16 for every operator (bfloat16 and
 * float8 are not implemented, as on the pages).  Kernels accumulate in
 * float32.  Head sizes must be multiples of 8 and at most 256.  The
 * GroupQueryAttention caches may instead hold int8 codes or packed uint8
 * nibbles (quantised caches, below).
 */
#ifndef KVATTN_H_
#define KVATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------------ */
/* Common types                                                             */
/* ------------------------------------------------------------------------ */

typedef enum kvattn_status {
  KVATTN_OK = 0,
  KVATTN_ERR_INVALID_ARG = -1,   /* shape, dtype, attribute or pairing violation */
  KVATTN_ERR_UNSUPPORTED = -2,   /* a feature the pages exclude or this library lacks */
  KVATTN_ERR_WORKSPACE = -3,     /* workspace too small (or NULL with a non-zero size) */
  KVATTN_ERR_HIP = -4            /* a HIP launch failed */
} kvattn_status;

typedef enum kvattn_dtype {
  KVATTN_DT_NONE = 0,
  KVATTN_DT_F32 = 1,
  KVATTN_DT_F16 = 2,
  KVATTN_DT_I32 = 3,
  KVATTN_DT_I8 = 4,    /* int8 cache codes */
  KVATTN_DT_U8 = 5     /* uint8: two packed 4-bit cache codes */
} kvattn_dtype;

/* Bytes of decode arrival counters at the start of every non-empty workspace. */
#define KVATTN_COUNTER_BYTES 32768

typedef struct kvattn_tensor {
  void* data;        /* device pointer, NULL = absent optional tensor */
  int32_t dtype;     /* kvattn_dtype */
  int32_t rank;      /* number of dims used, 0..4 */
  int64_t dims[4];   /* row-major sizes; the buffer is contiguous */
} kvattn_tensor;

/* Text of a status code (static storage). */
const char* kvattn_status_string(int32_t status);
/* Message of the last failure on the calling thread ("" if none). */
const char* kvattn_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int32_t kvattn_version(void);

/*
 * Measurement hook.  After kvattn_profile_events(start, stop, kind) on a
 * thread, in every later call on that thread the first kernel of the given
 * kind is launched so that it records its own dispatch start and stop times
 * on the caller-owned HIP events `start` and `stop` (hipEvent_t, created by
 * the caller), so hipEventElapsedTime(start, stop) is that kernel's duration.
 * kind selects:
 *   KVATTN_PROFILE_DECODE   split-key decode kernel (gqa_attention decode, decode_mha)
 *   KVATTN_PROFILE_FLASH    tiled attention kernel (prefill, sparse, packed)
 *   KVATTN_PROFILE_PREP     norm/rotary/append kernel
 *   KVATTN_PROFILE_GEMM     packed QKV projection GEMM
 *   KVATTN_PROFILE_SHIFT    sliding-window cache eviction (row shift)
 * Passing NULL events turns the hook off.  The library never creates or
 * destroys the events.
 */
enum {
  KVATTN_PROFILE_DECODE = 1,
  KVATTN_PROFILE_FLASH = 2,
  KVATTN_PROFILE_PREP = 3,
  KVATTN_PROFILE_GEMM = 4,
  KVATTN_PROFILE_SHIFT = 5
};
void kvattn_profile_events(void* start, void* stop, int32_t kind);

/*
 * Decode split control.  Single-token decode spreads every (sample, kv head,
 * query-head group) unit's live keys over pairs of waves so that the grid
 * fills the device; the split (GroupQueryAttention page, Implementation
 * variants: partitioning cached decode along the key axis and merging the
 * partial online-softmax results) aims at waves_per_cu waves per compute
 * unit (default 8).  kvattn_set_decode_split(w) sets that target for later
 * calls on the calling thread: 1..32, or 0 for the default.  Smaller targets
 * give fewer pairs per unit (1 gives one pair per unit at the decode
 * workload's shape); results agree up to float32 rounding order.  Returns the
 * previous setting (0 = default), or KVATTN_ERR_INVALID_ARG for values
 * outside 0..32 (the setting is then unchanged).
 */
int32_t kvattn_set_decode_split(int32_t waves_per_cu);

/* ------------------------------------------------------------------------ */
/* GroupQueryAttention                                                      */
/* (com.microsoft.GroupQueryAttention page: Description; Inputs, Outputs,   */
/*  Attributes tables; Implementation variants for the cache update and    */
/*  split-key decode)                                                       */
/* ------------------------------------------------------------------------ */

typedef enum gqa_input {
  GQA_IN_QUERY = 0,          /* T (B, S, N*H)                                   required */
  GQA_IN_KEY,                /* T (B, S, kvN*H)                                 required */
  GQA_IN_VALUE,              /* T (B, S, kvN*H)                                 required */
  GQA_IN_PAST_KEY,           /* T_CACHE (B, kvN, past_seq or capacity, Hc)      optional */
  GQA_IN_PAST_VALUE,         /* T_CACHE like past_key                           optional */
  GQA_IN_SEQLENS_K,          /* int32 (B): total length - 1 per sample (device) required */
  GQA_IN_COS_CACHE,          /* T (max_seq, H/2)                                optional */
  GQA_IN_SIN_CACHE,          /* T (max_seq, H/2)                                optional */
  GQA_IN_ATTENTION_BIAS,     /* T (B|1, N|1, S, total_sequence_length)          optional */
  GQA_IN_HEAD_SINK,          /* T (N)                                           optional */
  GQA_IN_K_SCALE,            /* float32 (1) PER_TENSOR or (kvN*H) PER_CHANNEL   quantised caches */
  GQA_IN_V_SCALE,            /* float32, like k_scale with v_quant_type         quantised caches */
  GQA_IN_Q_NORM_WEIGHT,      /* T (H), paired with k_norm_weight                optional */
  GQA_IN_K_NORM_WEIGHT,      /* T (H), paired with q_norm_weight                optional */
  GQA_NUM_INPUTS
} gqa_input;

typedef enum gqa_output {
  GQA_OUT_OUTPUT = 0,        /* T (B, S, N*H)                                   required */
  GQA_OUT_PRESENT_KEY,       /* T_CACHE (B, kvN, present_seq, Hc)               required */
  GQA_OUT_PRESENT_VALUE,     /* T_CACHE like present_key                        required */
  GQA_NUM_OUTPUTS
} gqa_output;

typedef struct gqa_attrs {
  int32_t num_heads;             /* N, required */
  int32_t kv_num_heads;          /* kvN, required, divides N */
  int32_t causal;                /* default 1; 0 = bidirectional (no past, window -1) */
  int32_t do_rotary;             /* default 0; 1 = NeoX rotary with cos/sin caches */
  int32_t local_window_size;     /* default -1 (off) */
  float qk_norm_epsilon;         /* default 1e-6 */
  float scale;                   /* default 0 = 1/sqrt(H) */
  int32_t sliding_window_cache;  /* default 0; 1 = window buffers evicting from the front (below) */
  int32_t smooth_softmax;        /* default -1; 1 adds exp(0) to the denominator */
  float softcap;                 /* default 0 = off */
  int32_t k_quant_type;          /* gqa_quant_type, default NONE */
  int32_t v_quant_type;          /* gqa_quant_type, default NONE */
  int32_t kv_cache_bit_width;    /* 0 (default, float caches), 8 or 4 */
} gqa_attrs;

typedef enum gqa_quant_type {
  GQA_QUANT_NONE = 0,
  GQA_QUANT_PER_TENSOR = 1,      /* one float32 scale */
  GQA_QUANT_PER_CHANNEL = 2      /* kv_num_heads * head_size scales, head-major */
} gqa_quant_type;

/* Fill the page defaults; num_heads and kv_num_heads are set to 0 (required). */
void gqa_attrs_default(gqa_attrs* attrs);

/*
 * gqa_attention — grouped-query attention with a BNSH key/value cache.
 *
 * Computes, per sample b, query s and head h (kv head h / (N/kvN)):
 *   total_b = seqlens_k[b] + 1; past_b = total_b - S with a past cache, else 0;
 *   q, k  <- per-head RMSNorm (both norm weights given), then NeoX rotary at
 *            position past_b + s (do_rotary);
 *   present rows [0, past_b) = past rows, rows [past_b, past_b + S) = new k, v
 *            (rounded to T, or quantised), other rows untouched;
 *   keys j < total_b visible with j <= past_b + s (causal) and
 *            j >= past_b + s - local_window_size (window >= 0); bidirectional
 *            (causal 0) sees all S new keys;
 *   score = scale * q.k -> softcap -> + attention_bias[b|0, h|0, s, j];
 *   softmax with exp(head_sink[h]) (or exp(0) for smooth_softmax = 1) added to
 *            the denominator; output = weights . values, BSH layout.
 *
 * Shared buffer: present_key.data == past_key.data (and likewise for values)
 * appends in place; the present must then have the past's dims.  Otherwise the
 * present's seq axis must hold past_b + S rows and rows [0, past_b) are copied.
 * Without a past cache the present's seq axis must be >= S, and a float
 * present cache may be float16 or float32 whatever T is (GroupQueryAttention
 * page, Description): the attention then reads the new keys and values in T
 * from the workspace (2 * B * kvN * S * H elements of T after the counter
 * bytes, which such a prompt leaves untouched), and the present
 * holds the same rows rounded once to its own type.  A past cache (and a
 * present with a past) has T's type.
 * total_sequence_length (host) must be >= every total_b and is the last dim
 * of attention_bias.  rotary needs cos/sin rows for every position used.
 *
 * sliding_window_cache = 1 (GroupQueryAttention page, Attributes table): the
 * buffers of capacity C (the present buffer's sequence axis) hold a sample's
 * most recent tokens, oldest first.  Before the call the past holds
 * F_b = min(total_b - S, C) rows; D_b = max(0, F_b + S - C) rows are evicted
 * from the front (past rows [D_b, F_b) go to present rows [0, F_b - D_b): a
 * shift when the buffers are shared, a copy when they are separate, in which
 * case the past's sequence axis must hold min(total_sequence_length - S, C)
 * rows and the present's rows from fill_b on keep what they held) and the S
 * new rows follow, so row i then holds absolute position total_b - fill_b + i,
 * fill_b = F_b - D_b + S.  Rotary and the causal/window bounds use absolute
 * positions.  Needs causal, local_window_size > 0, a past cache and
 * C >= local_window_size + S; no attention_bias.
 *
 * Quantised caches (GroupQueryAttention page, Attributes table: k_quant_type,
 * v_quant_type, kv_cache_bit_width; Inputs table: k_scale, v_scale and the
 * int4 packing).  With kv_cache_bit_width 8 or 4 both quant types must be
 * PER_TENSOR or PER_CHANNEL, both scales are given, and query, key, value,
 * output and the other T inputs are float32.  T_CACHE is int8 (KVATTN_DT_I8,
 * Hc = H) for 8 bits, uint8 (KVATTN_DT_U8, Hc = H/2) for 4 bits, where byte i
 * of a row holds dim 2i in its low nibble and dim 2i+1 in its high nibble,
 * each as code + 8.  A cache element stands for code * scale (the scale of
 * its kv head and dim); a new key (after norm and rotary) or value x is
 * stored as code = clamp(rint(x / scale), -2^(b-1), 2^(b-1) - 1), the
 * quotient in float32 and rounded half to even.  Scales must be positive and
 * finite (other values give unspecified codes).  Both widths serve prompts
 * (with or without a past: the new rows' codes are written, then the
 * attention reads every row's codes), decode (a past, S = 1) and the
 * sliding-window cache (the eviction moves code rows), over shared or
 * separate buffers; int4 decode (S = 1 with a past) needs H to be a multiple
 * of Hp / 8, where Hp is H rounded up to 64, 128 or 256.
 *
 * UNSUPPORTED: kv sequence length != S; sliding_window_cache with
 * attention_bias; int4 decode with other head sizes.
 */
int32_t gqa_attention(const gqa_attrs* attrs,
                      const kvattn_tensor* inputs, int32_t n_inputs,
                      int32_t total_sequence_length,
                      const kvattn_tensor* outputs, int32_t n_outputs,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_attention_noalloc — gqa_attention for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments and results as gqa_attention,
 * without the workspace: the library keeps KVATTN_NOALLOC_SCRATCH_BYTES of
 * device memory per GPU (a static array, held until the process ends) and
 * uses it as the workspace.  The first call on a device looks that array up
 * and clears its arrival counters on `stream`; no call allocates or frees.
 * Calls whose workspace would exceed the scratch (gqa_attention_workspace_size
 * tells) return KVATTN_ERR_WORKSPACE before any launch.  Every call on a GPU
 * shares that GPU's scratch: calls that may overlap in time on one GPU (other
 * streams, other threads) race and must be serialised by the caller.
 */
#define KVATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
int32_t gqa_attention_noalloc(const gqa_attrs* attrs,
                              const kvattn_tensor* inputs, int32_t n_inputs,
                              int32_t total_sequence_length,
                              const kvattn_tensor* outputs, int32_t n_outputs,
                              void* stream);

/* Workspace bytes gqa_attention needs for these arguments (validates them). */
int32_t gqa_attention_workspace_size(const gqa_attrs* attrs,
                                     const kvattn_tensor* inputs, int32_t n_inputs,
                                     int32_t total_sequence_length,
                                     const kvattn_tensor* outputs, int32_t n_outputs,
                                     size_t* workspace_bytes);

/* ------------------------------------------------------------------------ */
/* DecoderMaskedMultiHeadAttention                                          */
/* (com.microsoft.DecoderMaskedMultiHeadAttention page: Description;        */
/*  Inputs, Outputs, Attributes tables)                                     */
/* ------------------------------------------------------------------------ */

typedef enum dmmha_input {
  DMMHA_IN_QUERY = 0,             /* T (B, 1, N*H)                              required */
  DMMHA_IN_KEY,                   /* self: T (B, 1, N*H); cross: T (B, N, kv_S, H) required */
  DMMHA_IN_VALUE,                 /* shaped like key                            required */
  DMMHA_IN_MASK_INDEX,            /* int32 (B, total_S): 0 adds mask_filter_value optional */
  DMMHA_IN_ATTENTION_BIAS,        /* T (B|1, N|1, 1, total_S), self only         optional */
  DMMHA_IN_PAST_KEY,              /* T (B, N, capacity, H); selects self attention optional */
  DMMHA_IN_PAST_VALUE,            /* T like past_key                            optional */
  DMMHA_IN_PAST_SEQUENCE_LENGTH,  /* int32 (1): live length before this token (device) */
  DMMHA_NUM_INPUTS
} dmmha_input;

typedef enum dmmha_output {
  DMMHA_OUT_OUTPUT = 0,        /* T (B, 1, N*H)                                  required */
  DMMHA_OUT_PRESENT_KEY,       /* T, the past_key buffer itself (in place) or absent */
  DMMHA_OUT_PRESENT_VALUE,     /* T, the past_value buffer itself or absent          */
  DMMHA_OUT_QK,                /* QK (B, N, 1, kv_S): float32 or float16, either with any T; cross attention with output_qk = 1 */
  DMMHA_NUM_OUTPUTS
} dmmha_output;

typedef struct dmmha_attrs {
  int32_t num_heads;                  /* required */
  float mask_filter_value;            /* default -10000 */
  int32_t output_qk;                  /* default 0; must match the qk output's presence */
  int32_t past_present_share_buffer;  /* 1 for self attention, 0 for cross */
  float scale;                        /* default 0 = 1/sqrt(H) */
} dmmha_attrs;

void dmmha_attrs_default(dmmha_attrs* attrs);

/*
 * decode_mha — single-token decode attention.
 *
 * Self attention (past_key given, share buffer 1): P = past_sequence_length[0]
 * (device); the token's key/value rows are written at row P of every head,
 * other rows untouched; keys 0..P attended.  Cross attention: key/value are
 * whole encoder tensors, no cache.  score = scale*q.k + attention_bias[...]
 * (self only) + (mask_index[b, j] == 0 ? mask_filter_value : 0) — the mask
 * never removes a key; plain softmax; output = weights . values.  qk (cross
 * only) receives the scores after the mask, before the softmax.
 * P must be < capacity; mask_index and attention_bias must have >= P+1 columns
 * (self) or kv_S columns (cross).
 */
int32_t decode_mha(const dmmha_attrs* attrs,
                   const kvattn_tensor* inputs, int32_t n_inputs,
                   const kvattn_tensor* outputs, int32_t n_outputs,
                   void* workspace, size_t workspace_bytes, void* stream);

int32_t decode_mha_workspace_size(const dmmha_attrs* attrs,
                                  const kvattn_tensor* inputs, int32_t n_inputs,
                                  const kvattn_tensor* outputs, int32_t n_outputs,
                                  size_t* workspace_bytes);

/* ------------------------------------------------------------------------ */
/* SparseAttention                                                          */
/* (com.microsoft.SparseAttention page: Description; Inputs, Outputs,       */
/*  Attributes tables)                                                      */
/* ------------------------------------------------------------------------ */

typedef enum sparse_input {
  SPARSE_IN_QUERY = 0,                 /* T (B, S, N*H) or packed (B, S, (N+2kvN)*H) required */
  SPARSE_IN_KEY,                       /* T (B, S, kvN*H); absent for packed QKV        */
  SPARSE_IN_VALUE,                     /* T (B, S, kvN*H); absent for packed QKV        */
  SPARSE_IN_PAST_KEY,                  /* T (B, kvN, capacity, H), updated in place     */
  SPARSE_IN_PAST_VALUE,                /* T like past_key, updated in place             */
  SPARSE_IN_BLOCK_ROW_INDICES,         /* int32 (L, max_blocks + 1) CSR row pointers    */
  SPARSE_IN_BLOCK_COL_INDICES,         /* int32 (L, max_nnz) CSR columns, right-padded  */
  SPARSE_IN_KEY_TOTAL_SEQUENCE_LENGTHS,/* int32 (B), device                             */
  SPARSE_IN_COS_CACHE,                 /* T (max_rot_seq, rotary_dim/2)                 */
  SPARSE_IN_SIN_CACHE,                 /* T like cos_cache                              */
  SPARSE_NUM_INPUTS
} sparse_input;

typedef enum sparse_output {
  SPARSE_OUT_OUTPUT = 0,        /* T (B, S, N*H)                               required */
  SPARSE_OUT_PRESENT_KEY,       /* the past_key buffer itself, or absent                */
  SPARSE_OUT_PRESENT_VALUE,     /* the past_value buffer itself, or absent              */
  SPARSE_NUM_OUTPUTS
} sparse_output;

typedef struct sparse_attrs {
  int32_t num_heads;           /* required */
  int32_t kv_num_heads;        /* required, divides num_heads */
  int32_t sparse_block_size;   /* required: 16, 32, 64 or 128 */
  int32_t do_rotary;           /* default 0; only 1 enables rotary */
  int32_t rotary_interleaved;  /* default 0 (NeoX); only 1 selects interleaved */
  float scale;                 /* default 0 = 1/sqrt(H) */
} sparse_attrs;

void sparse_attrs_default(sparse_attrs* attrs);

/*
 * sparse_attention — block-sparse causal grouped-query attention.
 *
 * Prompt iff total_sequence_length == S (past_b = 0), else past_b =
 * key_total_sequence_lengths[b] - S.  Rotary (do_rotary 1) rotates the first
 * 2*cos_width dims of q and the new k at past_b + s; the new k, v are written
 * in place at rows [past_b, past_b + S).  Query head h uses layout h mod L and
 * kv head h / (N/kvN); key j is visible to position p iff j <= p,
 * j < key_total_sequence_lengths[b], and block j / block_size is among
 * cols[l][rp[l][p/bs] : rp[l][p/bs + 1]].  Plain softmax, weights . values.
 * total_sequence_length must fit the capacity, max_blocks * block_size and the
 * rotary rows.  rp must be monotone from 0 and its entries <= max_nnz; active
 * column entries must lie in [0, max_blocks).
 * Token generation (total_sequence_length != S) needs
 * key_total_sequence_lengths[b] >= S for every sample.
 */
int32_t sparse_attention(const sparse_attrs* attrs,
                         const kvattn_tensor* inputs, int32_t n_inputs,
                         int32_t total_sequence_length,
                         const kvattn_tensor* outputs, int32_t n_outputs,
                         void* workspace, size_t workspace_bytes, void* stream);

int32_t sparse_attention_workspace_size(const sparse_attrs* attrs,
                                        const kvattn_tensor* inputs, int32_t n_inputs,
                                        int32_t total_sequence_length,
                                        const kvattn_tensor* outputs, int32_t n_outputs,
                                        size_t* workspace_bytes);

/* ------------------------------------------------------------------------ */
/* PackedAttention                                                          */
/* (com.microsoft.PackedAttention page: Description; Inputs, Outputs,       */
/*  Attributes tables)                                                      */
/* ------------------------------------------------------------------------ */

typedef enum packed_input {
  PACKED_IN_INPUT = 0,                   /* T (token_count, D)                      required */
  PACKED_IN_WEIGHTS,                     /* T (D, q_hidden + k_hidden + v_hidden)  required */
  PACKED_IN_BIAS,                        /* T (q_hidden + k_hidden + v_hidden)     required */
  PACKED_IN_TOKEN_OFFSET,                /* int32 (B, S): padded flat index per token    */
  PACKED_IN_CUMULATIVE_SEQUENCE_LENGTH,  /* int32 (B + 1)                                */
  PACKED_IN_ATTENTION_BIAS,              /* T (B|1, N|1, S, S), padded coordinates optional */
  PACKED_NUM_INPUTS
} packed_input;

typedef enum packed_output {
  PACKED_OUT_OUTPUT = 0,   /* T (token_count, v_hidden), packed token order */
  PACKED_NUM_OUTPUTS
} packed_output;

typedef struct packed_attrs {
  int32_t num_heads;            /* required */
  int32_t qkv_hidden_sizes[3];  /* all 0 (default) = bias length / 3 each */
  float scale;                  /* default 0 = 1/sqrt(Hq) */
} packed_attrs;

void packed_attrs_default(packed_attrs* attrs);

/*
 * packed_attention — self-attention over a batch whose padding has been
 * removed (tokens of all sequences back to back), with the QKV projection
 * done in the same call.
 *
 * qkv = input . weights + bias (the weight columns hold Q for every head,
 * then K for every head, then V); the tokens cum[b] .. cum[b+1] - 1 belong
 * to sequence b and each token
 * attends every key of its own sequence (no mask); score = scale*q.k +
 * attention_bias[b|0, h|0, pad(t), pad(t')] with pad(t) = token_offset.flat[t]
 * - b*S; softmax; output (token_count, v_hidden) in packed order.
 * cum must start at 0, be non-decreasing with steps <= S and end at
 * token_count.
 *
 * UNSUPPORTED on the GPU: v_hidden != q_hidden; an input hidden size or a
 * weight column count that is not a multiple of 8; weights over 2 GiB.
 */
int32_t packed_attention(const packed_attrs* attrs,
                         const kvattn_tensor* inputs, int32_t n_inputs,
                         const kvattn_tensor* outputs, int32_t n_outputs,
                         void* workspace, size_t workspace_bytes, void* stream);

int32_t packed_attention_workspace_size(const packed_attrs* attrs,
                                        const kvattn_tensor* inputs, int32_t n_inputs,
                                        const kvattn_tensor* outputs, int32_t n_outputs,
                                        size_t* workspace_bytes);

/*
 * kvattn_packed_schedule — the device schedule packed_attention builds from
 * cumulative_sequence_length (PackedAttention page, Inputs table: the
 * tokens cum[i] .. cum[i+1] - 1 belong to sequence i), exposed so that it can be checked
 * on its own.  All pointers are device int32 buffers:
 *   cum             (batch + 1)    input
 *   bounds          (batch, 2)     per sequence [start, end): cum clamped to
 *                                  [0, token_count], end - start <= padded length
 *   work            (1 + 2*items)  work[0] = item count, then (sequence, tile)
 *                                  pairs, items = sum over sequences of
 *                                  ceil(len / tile_rows), longest sequences
 *                                  first (ties: lower index first)
 *   token_sequence  (token_count)  optional: owning sequence of each token
 *   token_position  (token_count)  optional (with token_sequence): position
 * work must hold 1 + 2 * batch * ceil(padded_sequence_length / tile_rows)
 * ints.  batch must be in 1..4096.  Enqueued on `stream`.
 */
int32_t kvattn_packed_schedule(const int32_t* cum, int32_t batch, int32_t token_count,
                               int32_t padded_sequence_length, int32_t tile_rows,
                               int32_t* bounds, int32_t* work, int32_t* token_sequence,
                               int32_t* token_position, void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* KVATTN_H_ */
