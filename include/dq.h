/*
 * dq.h -- C ABI of the D-Quant hot path on MI355X (gfx950).
 *
 * D-Quant ("D-Quant: Driftable Entropy Coding for KV Cache Quantization",
 * abstract; "D-Quant: Entropy Coding Meets KV Cache at 2.26 Bits", sections
 * "Why Fixed Width Is a Ceiling" and "Drift: Bending Variable Back to Fixed")
 * stores each token's K or V vector as an rANS-coded stream of quantised
 * symbols inside a fixed-size byte container, so attention can address the
 * compressed cache at a fixed stride and dequantise in parallel.
 *
 * Conventions for every call:
 *  - Return value: DQ_OK (0) or a negative DQ_ERR_* code.  Calls never abort
 *    and never print.  Argument errors are detected synchronously, before
 *    anything is launched.
 *  - "device" pointers are HIP device allocations owned by the caller; the
 *    library never allocates, frees or synchronises in dq_encode,
 *    dq_decode_symbols or dq_attn_decode.  Work is enqueued on `stream`
 *    (a hipStream_t; NULL means the default stream).  Faults inside a kernel
 *    surface at the caller's next synchronisation, as usual in HIP.
 *  - Codec objects are host-only, immutable after creation and safe to share
 *    between threads.  Creating one needs no GPU.
 *  - Layouts: head_dim is 128.  The compressed cache of one stream (K or V)
 *    is a pool of `num_slots` slots per kv head:
 *        cont[Hkv][num_slots][C]   uint8   (one C-byte container per vector)
 *        norm[Hkv][num_slots]      uint16  (fp16 bits of the vector norm)
 *    `cont` must be 16-byte aligned and num_slots * C a multiple of 16.
 */
#ifndef DQ_H_
#define DQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DQ_OK = 0,
  DQ_ERR_INVALID = -1,     /* bad argument (null, range, shape, alignment)  */
  DQ_ERR_UNSUPPORTED = -2, /* valid but not supported (head_dim != 128, ...) */
  DQ_ERR_BUDGET = -3,      /* the table cannot meet the container budget    */
  DQ_ERR_WORKSPACE = -4,   /* workspace too small                           */
  DQ_ERR_HIP = -5          /* a HIP runtime call failed                     */
};

typedef void *dq_stream_t; /* hipStream_t */

/* Human-readable text for a status code (static storage). */
const char *dq_status_string(int status);

/* ABI version: 100 * major + minor (101: dq_codec_desc.drift_order; 102: decode
 * with append; 103: dq_set_knob, dq_attn_decode_noalloc; 104:
 * DQ_KNOB_ENCODE_TWO_PASS; 105: DQ_KNOB_QK_VALU). */
int dq_version(void);

/* Path overrides, for tests and tuning.  Every value the library can pick by
 * itself gives the same results (the split length aside, which changes the
 * floating-point order of the attention sums); these force one choice so
 * that tests reach each code path.  Process-wide, thread-safe (atomic), read
 * once per call that plans a launch; -1 restores the library's own choice.
 *   DQ_KNOB_SPLIT_TOKENS     decode/prefill context chunk in tokens (a
 *                            multiple of 64, >= 64; other values: ignored)
 *   DQ_KNOB_LATENCY_MODE     1: decode in latency mode, 0: never
 *   DQ_KNOB_APPEND_FUSE      1: a decode step's encodes inside the split-K
 *                            launch, 0: in a launch of their own
 *   DQ_KNOB_ENCODE_WAVE_MAX  batch size (vectors) up to which dq_encode uses
 *                            the wave-per-vector kernel
 *   DQ_KNOB_ENCODE_KEY_SPAN  span of the encoder's in-group integer keys
 *                            (smaller spans take the float-scan fallback
 *                            sooner; same bytes)
 *   DQ_KNOB_SPLITK_WAVES     resident waves per CU of the decode split-K
 *                            kernel, 1..11 (fewer than the library's 12:
 *                            occupancy studies; same bytes)
 *   DQ_KNOB_WORK_QUEUE       1: split-K waves take their items from a device
 *                            work queue, 0: by the static deal (the library
 *                            uses the queue when the items take several
 *                            rounds of resident waves; same bytes)
 *   DQ_KNOB_SLOT_TABLE       0: decode steps read the slot's symbol, then its
 *                            entry (two LDS round trips); 1 (default where
 *                            the 64 KB fit): one per-slot entry (same bytes)
 *   DQ_KNOB_ENCODE_TWO_PASS  0: dq_encode's lane-per-vector path runs the
 *                            drift search inline, in one kernel; 1 (default):
 *                            a first kernel encodes the vectors that need no
 *                            drift and a second runs the search on the rest
 *                            (same bytes, norms and stats)
 *   DQ_KNOB_QK_VALU          1: decode attention's query-key products as fp32
 *                            fused multiply-adds on the vector ALU (the
 *                            rotated query read from global memory, four
 *                            dims at a time) instead of 4x4x4 MFMAs; a
 *                            measurement variant of the per-slot-table
 *                            kernel without appended encodes (other
 *                            launches ignore it).  Scores differ from the
 *                            MFMA path by fp32 rounding only.
 * dq_set_knob returns DQ_ERR_INVALID for an unknown knob or a value below
 * -1; dq_get_knob returns the value (or DQ_ERR_INVALID). */
enum {
  DQ_KNOB_SPLIT_TOKENS = 1,
  DQ_KNOB_LATENCY_MODE = 2,
  DQ_KNOB_APPEND_FUSE = 3,
  DQ_KNOB_ENCODE_WAVE_MAX = 4,
  DQ_KNOB_ENCODE_KEY_SPAN = 5,
  DQ_KNOB_SPLITK_WAVES = 6,
  DQ_KNOB_WORK_QUEUE = 7,
  DQ_KNOB_SLOT_TABLE = 8,
  DQ_KNOB_ENCODE_TWO_PASS = 9,
  DQ_KNOB_QK_VALU = 10,
  DQ_KNOB_COUNT = 11
};
int dq_set_knob(int knob, int64_t value);
int64_t dq_get_knob(int knob);

/* ------------------------------------------------------------------------ */
/* Codec: the parameters of one coded stream (K or V).
 *
 * The probability model is the analytic N(0,1) mass of each quantiser cell
 * (no calibration data), per "Drift: Bending Variable Back to Fixed"; keys use
 * 8 levels and values 6 there.  Cells are symmetric, uniform of width
 * step64/64 (in units of the per-coordinate standard deviation after
 * normalisation), the outermost cell open; masses are quantised to a 12-bit
 * rANS table with every frequency >= 16; the reconstruction level of a cell is
 * its centroid rounded to fp16.  The rotation is a randomized Walsh-Hadamard
 * transform whose signs for kv head g are the bits of SplitMix64 outputs
 * 2g and 2g+1 of the stream seeded with `seed`. */
typedef struct dq_codec *dq_codec_t;

typedef struct {
  int32_t head_dim;        /* must be 128, else DQ_ERR_UNSUPPORTED           */
  int32_t levels;          /* even, 2..16 (keys 8, values 6)                 */
  int32_t container_bytes; /* C in [5, 132]: 34 -> 2.25 bits/value with norm */
  int32_t num_kv_heads;    /* 1..1024; one sign vector per kv head           */
  uint64_t seed;           /* rotation seed                                  */
  int32_t step64;          /* cell width * 64, 1..1023; 0 = default for
                              (levels, C) where one exists, else DQ_ERR_INVALID */
  int32_t drift_order;     /* 0: magnitude order (default); 1: rate-distortion
                              order (below); else DQ_ERR_INVALID            */
} dq_codec_desc;

/* Drift order.  When a stream does not fit, candidates (symbols off the
 * innermost pair) move one level inward, the first k of a fixed order with
 * k minimal ("D-Quant: Entropy Coding Meets KV Cache at 2.26 Bits", Drift:
 * Bending Variable Back to Fixed).
 *   0  magnitude descending, then |y| ascending, then index ascending.
 *   1  rate-distortion (the page's So What points to that toolbox): the key
 *      (2|y| - n (l_m + l_{m-1})) * w_m ascending, then index ascending,
 *      where l are the fp16 levels of magnitudes m and m - 1, n the stored
 *      norm and w_m = (l_m - l_{m-1}) / log2(f_{m-1} / f_m) (double, rounded
 *      once to fp32); the key is the added squared error per bit saved up to
 *      the vector's common factor n, evaluated in fp32 with one rounding for
 *      the difference and one for the product.  Lower distortion at the same
 *      budget, more moves. */

/* Validates `desc`, builds the tables (host memory only) and returns a new
 * codec in *out.  DQ_ERR_BUDGET when a frequency would fall below 16, when
 * adjacent magnitude cells are not at least 1.15x apart in probability, or
 * when the all-innermost vector cannot fit C bytes. */
int dq_codec_create(const dq_codec_desc *desc, dq_codec_t *out);
int dq_codec_destroy(dq_codec_t codec); /* NULL is accepted */

/* The resolved parameters (step64 filled in). */
int dq_codec_info(dq_codec_t codec, dq_codec_desc *out);

/* Host copies of the tables, any pointer may be NULL:
 *   freq[levels], cum[levels + 1] (12-bit rANS table in symbol order, symbol
 *   0 = outermost negative cell), recon_f16[levels] (fp16 bits of the
 *   reconstruction levels), sign_words[2 * num_kv_heads] (bit i % 64 of word
 *   2g + i / 64 set means coordinate i of kv head g is negated). */
int dq_codec_tables(dq_codec_t codec, uint16_t *freq, uint16_t *cum,
                    uint16_t *recon_f16, uint64_t *sign_words);

/* ------------------------------------------------------------------------ */
/* Encode statistics, accumulated (atomically) by dq_encode into a
 * caller-zeroed device struct.  Drift rate = drifted_symbols / (128 *
 * vectors); the pages report 0.75% for keys and 5.00% for values
 * ("Drift: Bending Variable Back to Fixed"). */
#define DQ_MAX_CONTAINER 132
typedef struct {
  uint64_t vectors;           /* vectors encoded                          */
  uint64_t drifted_vectors;   /* vectors that needed at least one move    */
  uint64_t drifted_symbols;   /* one-level symbol moves                   */
  uint64_t multilevel_events; /* extra drift passes (expected 0)          */
  uint64_t bad_norms;         /* norm inf or NaN: coded as all-innermost  */
  uint64_t zero_norms;        /* norm rounds to 0: coded as all-innermost */
  uint64_t len_hist[DQ_MAX_CONTAINER + 1]; /* final stream length counts  */
} dq_stats;

/* dq_encode: rotate, normalise, quantise, rANS-code and drift T x Hkv
 * vectors into their containers ("Drift: Bending Variable Back to Fixed").
 *   x         device bf16, element (t, g, i) at x[t*stride_t + g*stride_h + i]
 *   slots     device int64[T]: pool slot of token t (0 <= slot < num_slots)
 *   cont      device uint8[Hkv][num_slots][C]   (written at the given slots)
 *   norm      device uint16[Hkv][num_slots]     (fp16 bits)
 *   stats     device dq_stats, may be NULL
 * Vectors with a zero, inf or NaN norm are coded as all innermost-positive
 * symbols (norm stored as 0, inf or 0x7E00).  A slot outside [0, num_slots)
 * writes nothing; the stats still count its vector.  Duplicate slots race:
 * which vector's container remains is unspecified, and the stats may count
 * only that one.  Until the call's work on `stream` completes, the norm of
 * a vector still in the drift search may read 0xFFFF (large batches run the
 * search's rare cases in a second kernel and mark them so).
 * T = 0 is a no-op; T * Hkv above 2^38 gives DQ_ERR_UNSUPPORTED. */
int dq_encode(dq_codec_t codec, const void *x, int64_t T, int64_t stride_t,
              int64_t stride_h, const int64_t *slots, int64_t num_slots,
              uint8_t *cont, uint16_t *norm, dq_stats *stats,
              dq_stream_t stream);

/* K and V of the same tokens in one call: the same bytes as dq_encode(ck,
 * k, ...) followed by dq_encode(cv, v, ...) with the shared slots, strides
 * and pools' slot count.  When both batches take the small-batch kernel
 * (a decode step's append) and the codecs share a drift order, it is one
 * launch instead of two.  k and v have the same shape and strides; the
 * codecs the same num_kv_heads (else DQ_ERR_INVALID); either stats may be
 * NULL. */
int dq_encode_kv(dq_codec_t ck, dq_codec_t cv, const void *k, const void *v,
                 int64_t T, int64_t stride_t, int64_t stride_h,
                 const int64_t *slots, int64_t num_slots, uint8_t *k_cont,
                 uint16_t *k_norm, uint8_t *v_cont, uint16_t *v_norm,
                 dq_stats *k_stats, dq_stats *v_stats, dq_stream_t stream);

/* dq_decode_symbols: container -> the 128 symbols, for kv head `head` at n
 * slots: the entropy decode alone, without dequantisation or attention, the
 * per-stream inverse of dq_encode ("D-Quant: Entropy Coding Meets KV Cache at
 * 2.26 Bits", intro: rANS coding of the quantised symbols; Drift: Bending
 * Variable Back to Fixed: one fixed-size container per vector), for
 * inspection and checking (attention decodes inside its own kernel).
 *   cont         device uint8[Hkv][num_slots][C], read-only
 *   slots        device int64[n]; a slot outside [0, num_slots) gives 128
 *                zero symbols, final state 0 and 0 bytes consumed
 *   head         kv head, 0 <= head < Hkv (else DQ_ERR_INVALID)
 *   sym_out      device uint8[n][128]
 *   final_state  device uint32[n] or NULL: decoder state after 128 symbols
 *                (2^23 for every container dq_encode wrote)
 *   consumed     device int32[n] or NULL: container bytes read
 * Bytes past the C-byte container read as 0 and are never fetched. */
int dq_decode_symbols(dq_codec_t codec, const uint8_t *cont, int64_t num_slots,
                      int32_t head, const int64_t *slots, int64_t n,
                      uint8_t *sym_out, uint32_t *final_state,
                      int32_t *consumed, dq_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Decode attention over the compressed cache ("D-Quant: Driftable Entropy
 * Coding for KV Cache Quantization", abstract: fixed-size streams give
 * regular memory access and parallel dequantisation inside attention; "D-Quant:
 * Entropy Coding Meets KV Cache at 2.26 Bits", So What: the entropy decoder
 * sits inside the attention kernel).
 *
 * One query token per sequence; GQA with query head h reading kv head
 * h / (Hq / Hkv); Hq / Hkv must be 1, 2 or 4.  Sequence b occupies pool
 * slots [seq_start[b], seq_start[b] + seq_len[b]).  Split-K: the context is
 * cut into chunks decoded in parallel and merged by a log-sum-exp combine.
 * The result is computed in the rotated basis and rotated back before the
 * store.
 *   q          device bf16 [B][Hq][128]
 *   seq_start  device int64[B]; seq_len device int32[B], 1 <= len <= max_len
 *              (lengths live on the device and are not checked: a length
 *              of 0 gives a zero output row, and tokens past max_len are
 *              not read)
 *   max_len    host: upper bound of seq_len, used to plan the split
 *   sm_scale   softmax scale (e.g. 1/sqrt(128))
 *   out_dtype  0: fp32, 1: bf16
 *   out        device [B][Hq][128]
 *   workspace  device scratch of at least the size reported by
 *              dq_attn_decode_workspace for the same (B, Hq, Hkv, max_len)
 * The two codecs must have the same num_kv_heads. */
int dq_attn_decode_workspace(int32_t B, int32_t Hq, int32_t Hkv,
                             int64_t max_len, size_t *bytes);

int dq_attn_decode(dq_codec_t ck, dq_codec_t cv, const void *q, int32_t B,
                   int32_t Hq, const uint8_t *k_cont, const uint16_t *k_norm,
                   const uint8_t *v_cont, const uint16_t *v_norm,
                   int64_t num_slots, const int64_t *seq_start,
                   const int32_t *seq_len, int64_t max_len, float sm_scale,
                   int32_t out_dtype, void *out, void *workspace,
                   size_t ws_bytes, dq_stream_t stream);

/* dq_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It calls no allocating routine.  The
 * workspace is a library-held device array of DQ_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, reserved with the library's code on each GPU it runs on
 * and held until the process ends; its address is looked up on the first
 * call on a device (that device current).  A call whose workspace need
 * (dq_attn_decode_workspace for the same B, Hq, Hkv, max_len) exceeds the
 * array returns DQ_ERR_WORKSPACE and launches nothing; batch 128 x 8K and
 * 32 sequences of up to 128K tokens (8 kv heads) fit.  Every call on one GPU
 * shares its array: calls that overlap on one GPU (concurrent streams,
 * threads) race and must be serialised by the caller.  Nothing in the array
 * needs to start at zero: every partial a call reads back it wrote earlier
 * in the same call.  `stream` must belong to the current device.  Every
 * other argument, the checks and the result (bit for bit) are those of
 * dq_attn_decode. */
#define DQ_NOALLOC_SCRATCH_BYTES (64u << 20)
int dq_attn_decode_noalloc(dq_codec_t ck, dq_codec_t cv, const void *q,
                           int32_t B, int32_t Hq, const uint8_t *k_cont,
                           const uint16_t *k_norm, const uint8_t *v_cont,
                           const uint16_t *v_norm, int64_t num_slots,
                           const int64_t *seq_start, const int32_t *seq_len,
                           int64_t max_len, float sm_scale, int32_t out_dtype,
                           void *out, dq_stream_t stream);

/* Chunked-prefill attention over the compressed cache.  A chunk of Tq new
 * tokens per sequence has been encoded with dq_encode at the end of the
 * sequence's slots, so seq_len[b] counts it; query j of sequence b sits at
 * position seq_len[b] - Tq + j and attends causally to tokens 0..that
 * position, all read from their containers ("D-Quant: Entropy Coding Meets
 * KV Cache at 2.26 Bits", The Numbers: served with an 8K prompt).
 *   q          bf16 [B][Tq][Hq][128], contiguous
 *   out        [B][Tq][Hq][128], fp32 (out_dtype 0) or bf16 (1)
 *   seq_len    device int32 [B], each >= Tq (a query with a negative
 *              position gets a zero output row) and <= max_len
 *   max_len    host value >= Tq; plans the context split
 *   workspace  >= dq_attn_prefill_workspace(B, Tq, Hq, Hkv, max_len) bytes,
 *              256-byte aligned
 * Pools, codecs, sm_scale and error codes as for dq_attn_decode. */
int dq_attn_prefill_workspace(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv,
                              int64_t max_len, size_t *bytes);
int dq_attn_prefill(dq_codec_t ck, dq_codec_t cv, const void *q, int32_t B,
                    int32_t Tq, int32_t Hq, const uint8_t *k_cont,
                    const uint16_t *k_norm, const uint8_t *v_cont,
                    const uint16_t *v_norm, int64_t num_slots,
                    const int64_t *seq_start, const int32_t *seq_len,
                    int64_t max_len, float sm_scale, int32_t out_dtype,
                    void *out, void *workspace, size_t ws_bytes,
                    dq_stream_t stream);

/* Paged pool: the same attention, with each sequence's cache split into
 * pages of DQ_PAGE_TOKENS consecutive slots anywhere in the pool (a block
 * table, so sequences can grow without contiguous reservations).  Token t
 * of sequence b is in slot pages[b * max_pages + t / 64] * 64 + t % 64 of
 * every kv head's plane; the fixed-stride container address the pages rely
 * on ("D-Quant: Driftable Entropy Coding for KV Cache Quantization",
 * abstract) is unchanged.
 *   pages      device int32 [B][max_pages]; entries past a sequence's last
 *              page are not read.  A page id outside [0, num_slots / 64)
 *              reads zero containers (a caller error, never a fault).
 *   max_pages  >= 1, and max_len <= max_pages * 64 (else DQ_ERR_INVALID);
 *              longer seq_len values are cut at max_pages * 64.
 * Every other argument, the workspace and the result are as for
 * dq_attn_decode; dq_encode writes a page by passing its slots. */
#define DQ_PAGE_TOKENS 64
int dq_attn_decode_paged(dq_codec_t ck, dq_codec_t cv, const void *q,
                         int32_t B, int32_t Hq, const uint8_t *k_cont,
                         const uint16_t *k_norm, const uint8_t *v_cont,
                         const uint16_t *v_norm, int64_t num_slots,
                         const int32_t *pages, int32_t max_pages,
                         const int32_t *seq_len, int64_t max_len,
                         float sm_scale, int32_t out_dtype, void *out,
                         void *workspace, size_t ws_bytes,
                         dq_stream_t stream);

/* dq_attn_decode plus a measurement hook: `split_begin` and `split_end`
 * (hipEvent_t, either may be NULL) are recorded on `stream` right before
 * and right after the split-K kernel, the one that reads the compressed
 * cache, so that its own duration can be taken with hipEventElapsedTime
 * without a profiler.  The events belong to the caller; results and
 * status codes are those of dq_attn_decode (an event record that fails
 * returns DQ_ERR_HIP). */
int dq_attn_decode_timed(dq_codec_t ck, dq_codec_t cv, const void *q,
                         int32_t B, int32_t Hq, const uint8_t *k_cont,
                         const uint16_t *k_norm, const uint8_t *v_cont,
                         const uint16_t *v_norm, int64_t num_slots,
                         const int64_t *seq_start, const int32_t *seq_len,
                         int64_t max_len, float sm_scale, int32_t out_dtype,
                         void *out, void *workspace, size_t ws_bytes,
                         dq_stream_t stream, void *split_begin,
                         void *split_end);

/* Decode step with append, in one call: the step's new token of every
 * sequence is encoded into the pools (as dq_encode would write it) and
 * attended to in the same call.  This is the fused append of the decode
 * step ("D-Quant: Entropy Coding Meets KV Cache at 2.26 Bits", The Numbers:
 * entropy coding costs the most at small batch, where a launch per step
 * matters).  The launch's first waves encode the new K and V vectors, one
 * wave per vector, while the others attend to the older tokens; each
 * encoding wave also writes the new token's own attention partial from the
 * symbols it chose, and the combine merges it with the older tokens'
 * partials.  When the attention items already fill every round of resident
 * waves (large batches), the same encodes run as a short launch of their
 * own before the attention instead, which then costs less; the results are
 * the same either way.
 *   k_new, v_new  device bf16: the new token of sequence b, kv head g, at
 *                 element b * new_stride_b + g * new_stride_h (128
 *                 contiguous values; 2-byte aligned)
 *   seq_len       includes the new token, which is at position
 *                 seq_len[b] - 1: slot seq_start[b] + seq_len[b] - 1 of
 *                 every kv head's plane (>= 1; the slot must be in the pool:
 *                 a slot outside it is not written)
 *   k_cont ...    the pools, written at the new slots and read elsewhere
 *   k_stats, v_stats  device dq_stats of the two encodes, may be NULL
 * The containers, norms and stats equal those of dq_encode_kv on the same
 * tokens.  The output is that of dq_attn_decode after that encode up to
 * floating-point order (the new token enters through the final merge).
 * Workspace: dq_attn_decode_workspace for the same shape. */
int dq_attn_decode_append(dq_codec_t ck, dq_codec_t cv, const void *q,
                          int32_t B, int32_t Hq, const void *k_new,
                          const void *v_new, int64_t new_stride_b,
                          int64_t new_stride_h, uint8_t *k_cont,
                          uint16_t *k_norm, uint8_t *v_cont, uint16_t *v_norm,
                          int64_t num_slots, const int64_t *seq_start,
                          const int32_t *seq_len, int64_t max_len,
                          float sm_scale, int32_t out_dtype, void *out,
                          void *workspace, size_t ws_bytes, dq_stats *k_stats,
                          dq_stats *v_stats, dq_stream_t stream);

/* dq_attn_decode_append plus the measurement hook of dq_attn_decode_timed:
 * `split_begin` and `split_end` (hipEvent_t, either may be NULL) are
 * recorded right before and after the split-K kernel, which here also runs
 * the append's encodes. */
int dq_attn_decode_append_timed(dq_codec_t ck, dq_codec_t cv, const void *q,
                                int32_t B, int32_t Hq, const void *k_new,
                                const void *v_new, int64_t new_stride_b,
                                int64_t new_stride_h, uint8_t *k_cont,
                                uint16_t *k_norm, uint8_t *v_cont,
                                uint16_t *v_norm, int64_t num_slots,
                                const int64_t *seq_start,
                                const int32_t *seq_len, int64_t max_len,
                                float sm_scale, int32_t out_dtype, void *out,
                                void *workspace, size_t ws_bytes,
                                dq_stats *k_stats, dq_stats *v_stats,
                                dq_stream_t stream, void *split_begin,
                                void *split_end);

/* dq_attn_decode_append over a paged pool (pages and max_pages as for
 * dq_attn_decode_paged): the new token of sequence b goes to slot
 * pages[b * max_pages + p / 64] * 64 + p % 64, p = seq_len[b] - 1. */
int dq_attn_decode_paged_append(dq_codec_t ck, dq_codec_t cv, const void *q,
                                int32_t B, int32_t Hq, const void *k_new,
                                const void *v_new, int64_t new_stride_b,
                                int64_t new_stride_h, uint8_t *k_cont,
                                uint16_t *k_norm, uint8_t *v_cont,
                                uint16_t *v_norm, int64_t num_slots,
                                const int32_t *pages, int32_t max_pages,
                                const int32_t *seq_len, int64_t max_len,
                                float sm_scale, int32_t out_dtype, void *out,
                                void *workspace, size_t ws_bytes,
                                dq_stats *k_stats, dq_stats *v_stats,
                                dq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DQ_H_ */
