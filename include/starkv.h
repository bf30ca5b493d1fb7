/*
 * libstarkv -- decode attention read directly from a low-rank, mixed-precision
 * quantised KV cache (STAR-KV), for AMD Instinct MI355X (gfx950).
 *
 * The method (STAR-KV summary page, "STAR-KV: Low-Rank KV Cache Compression via
 * Soft Thresholding for Adaptive Rank Control"):
 *   - Problem Statement: the cache stores hidden states projected into a
 *     low-rank latent instead of K and V; rebuilding K and V at inference costs
 *     compute, so attention should read the latent directly.
 *   - Methodology section 1: every head keeps the singular triplets of its
 *     projection whose singular value is above a per-head threshold; at
 *     inference the projection is truncated to them.
 *   - Methodology section 2: keys are factored head by head, values jointly over
 *     all heads; the reconstruction matrices are moved past the attention
 *     weights by reordering the operations.
 *   - Methodology section 3: the latent's leading (outlier) channels are
 *     quantised with more bits than the rest.
 *
 * Notation: H_q query heads, H_kv key/value heads (G = H_q / H_kv query heads
 * per KV head; query head h reads KV head h / G), d_h head dim, d hidden size,
 * r_g key rank of KV head g, n_key = sum_g r_g, r_v value rank, n_lat = n_key + r_v.
 *
 * Conventions for every call:
 *   - Device pointers are plain device addresses owned by the caller (for
 *     example PyTorch tensors); the library never frees them and keeps the ones
 *     passed to the bind/build/calibrate calls only as borrowed references:
 *     they must stay valid while the layer uses them.
 *   - "host" arrays are read before the call returns.
 *   - All GPU work is enqueued on the caller's stream; the three hot calls
 *     (compress_append, decode_attention, reconstruct) never allocate, never
 *     synchronise and never copy between host and device.
 *   - bf16 buffers hold raw bfloat16 bits (uint16), f16 buffers raw float16 bits.
 *   - Return value: STARKV_OK (0) or a negative status.  Arguments are checked
 *     before anything is enqueued; a failed check enqueues nothing.  A HIP
 *     launch failure is reported as STARKV_EHIP.  No C++ exception crosses the
 *     interface.
 *   - A layer handle may be used from several host threads only for the const
 *     calls (append, decode, reconstruct, queries); calibrate/build/bind are
 *     not thread-safe with respect to the same handle.
 */
#ifndef STARKV_H
#define STARKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STARKV_ABI_VERSION 2

/* status codes */
#define STARKV_OK 0
#define STARKV_EINVAL (-1)       /* bad argument: null pointer, bad size, bad enum, NaN threshold */
#define STARKV_ENOMEM (-2)       /* host or device allocation of the layer's own tables failed */
#define STARKV_ECAPACITY (-3)    /* append would write past T_max, or a length exceeds T_max */
#define STARKV_EUNSUPPORTED (-4) /* valid but unsupported combination (dtype/latent, sizes over limits) */
#define STARKV_EWORKSPACE (-5)   /* decode workspace smaller than starkv_decode_workspace_bytes() */
#define STARKV_EHIP (-6)         /* a HIP runtime call or kernel launch failed */
#define STARKV_ESTATE (-7)       /* factors or scales are not bound to the layer yet */

/* element types of X, q, factors and out */
#define STARKV_F32 0
#define STARKV_BF16 1

/* latent storage in the cache */
#define STARKV_LATENT_F32 0   /* fp32 latent, no quantisation (requires dtype F32) */
#define STARKV_LATENT_BF16 1  /* bf16 latent (round-to-nearest-even), no quantisation (dtype BF16) */
#define STARKV_LATENT_MIX84 2 /* int8 codes for the leading ceil(r/4) channels of every segment,
                                 int4 codes for the rest, per-channel fp16 scales (dtype BF16) */
#define STARKV_LATENT_HAD43 3 /* the block-rotated quantiser of the STAR-KV summary page,
                                 Methodology section 3: each segment's leading ceil(r/5)
                                 channels (outlier block) and the rest (inlier block) are
                                 rotated by independent Hadamard transforms folded into the
                                 factors (A' = A R, B' = R^T B / n per Sylvester piece of
                                 order n; blocks whose size is not a power of two are split
                                 into the power-of-two pieces of their binary decomposition,
                                 largest first), then quantised to 4-bit (|code| <= 7,
                                 outliers) and 3-bit (|code| <= 3, inliers) symmetric codes
                                 with per-channel fp16 scales.  Codes are stored in the
                                 mix84 byte format: outliers in the int8 region, inliers in
                                 the int4 region (dtype BF16). */
#define STARKV_LATENT_HAD43P 4 /* the same quantiser and codes as STARKV_LATENT_HAD43, stored at
                                 their own widths (the summary page's 3.2 bits per channel,
                                 Key Results): outlier codes as nibbles, inlier codes as 3-bit
                                 fields in bit planes.  Key row: K4/2 bytes of outlier nibbles
                                 (head after head, two's complement, low nibble first, K4 a
                                 multiple of 64), then the inlier channels of all heads in
                                 groups of 32: three little-endian 32-bit words P0, P1, P2, bit j
                                 of Pb = bit b of (code + 4) of the group's channel j (padding:
                                 0), K3 channels (a multiple of 64); row padded to 16 bytes.
                                 Value tile: V4/2 byte-rows of outlier channel pairs (nibbles,
                                 low = even channel), then the inlier channels as a byte stream
                                 over the following 32-byte rows: 12 bytes per channel, words
                                 P0, P1, P2 over the tile's 32 tokens with token t at bit
                                 8 (t >> 3) + 4 (t & 1) + ((t >> 1) & 3).  Decode with at most 32
                                 query rows per sequence (H_q * n_q <= 32); rotary layers
                                 attend over reconstructed K and V.  dtype BF16, d % 64 == 0. */

/* limits of the library */
#define STARKV_MAX_BATCH 128     /* sequences per call */
#define STARKV_MAX_QROWS 256     /* H_q * n_q per sequence */
#define STARKV_TILE_TOKENS 32    /* tokens per value tile */

typedef struct starkv_layer starkv_layer;

/* Description of one layer (one decoder block): shapes, storage, and the
 * spectra and thresholds that select the ranks (Methodology section 1). */
typedef struct starkv_layer_desc {
  int H_q, H_kv, d_h, d;
  int dtype;        /* STARKV_F32 or STARKV_BF16 */
  int latent;       /* STARKV_LATENT_* */
  int shrink;       /* 1: kept singular values become max(s - tau, 0) (soft threshold);
                       0: kept as they are (hard truncation) */
  int n_v;          /* number of value singular triplets provided (length of s_v) */
  const float* s_k; /* host [H_kv][d_h]: singular values of each key head, descending */
  const float* tau_k; /* host [H_kv]: threshold of each key head */
  const float* s_v; /* host [n_v]: singular values of the joint value projection, descending */
  float tau_v;      /* threshold of the value projection */
} starkv_layer_desc;

/* Sizes and layout of a created layer (all derived from the ranks). */
typedef struct starkv_layer_info {
  int H_q, H_kv, d_h, d, dtype, latent;
  int n_key, r_v, n_lat;
  int k_row_bytes;   /* bytes of one token's key row */
  int v_tile_rows;   /* rows of a value tile */
  int v_tile_bytes;  /* bytes of one value tile (STARKV_TILE_TOKENS tokens) */
  int K8, K4;        /* mix84 key row: int8 region channels (padded to 16), int4 region channels (padded to 32);
                        had43p: K8 = 0, K4 = outlier nibbles (padded to 64) */
  int V8, V4;        /* mix84 value tile: int8 rows (padded to 32), int4 channels (padded to 64);
                        had43p: V8 = 0, V4 = outlier channels (padded to 64) */
  int K3, V3;        /* had43p: inlier channels of the key row's and of the value tile's 3-bit
                        regions (each padded to 64); 0 otherwise */
  size_t a_bytes;    /* bytes of A^T  [n_lat][d] (dtype) */
  size_t bk_bytes;   /* bytes of B_k  [n_key][d_h] (dtype) */
  size_t bv_bytes;   /* bytes of B_v^T [H_kv*d_h][r_v] (dtype) */
  size_t scale_bytes;/* bytes of the fp16 scales [n_lat] (mix84, had43, had43p; 0 otherwise) */
} starkv_layer_info;

/*
 * The cache of one layer, caller-owned device memory:
 *
 * k_rows  [B][T_max][k_row_bytes]  one key row per token.
 *   mix84 (had43 alike, with the leading ceil(r_g/5) channels in the first region):
 *          bytes [0, K8): the leading ceil(r_g/4) channels of head 0, then of
 *          head 1, ... as int8 (two's complement), zero-padded; bytes
 *          [K8, K8 + K4/2): the remaining channels of head 0, head 1, ... as
 *          int4 two per byte (channel 2k in the low nibble, two's complement),
 *          zero-padded.
 *   bf16 / f32: the key latent in channel order (head 0's r_0 channels, head
 *          1's, ...), padded to a multiple of 16 bytes.
 * v_tiles [B][v_tile_rows/32][T_max/32][32][32 * elem]  value latent in tiles
 *          of 32 tokens, each tile row holding one channel (or channel pair)
 *          for the 32 tokens of the tile.  Rows are grouped in blocks of 32:
 *          block rb of tile t of sequence b is the contiguous 32 x 32 x elem
 *          bytes at [b][rb][t], so one row block's tiles follow each other.
 *   mix84: rows [0, V8): int8 value channels 0, 1, ... (zero-padded rows);
 *          rows [V8, V8 + V4/2): int4 value channels two per row byte (the
 *          even-numbered one of the pair in the low nibble); elem = 1.
 *   bf16 / f32: row c = value channel c (rows padded to a multiple of 32),
 *          elem = 2 or 4.
 * T_max must be a multiple of 32, and one sequence's key rows (T_max x row
 * bytes) must stay under 4 GiB (EUNSUPPORTED otherwise).  Token t of sequence b lives at k_rows row
 * [b][t] and, for value tile row v, at v_tiles [b][v/32][t/32][v%32][t%32].  Bytes of tokens at or beyond a
 * sequence's length are never read for the result.
 */
typedef struct starkv_cache {
  void* k_rows;
  void* v_tiles;
  int B;
  int T_max;
} starkv_cache;

/* ABI version of the library (STARKV_ABI_VERSION of the build). */
int starkv_abi_version(void);

/* Static description of a status code. */
const char* starkv_status_string(int status);

/*
 * Create a layer: rank selection (Methodology section 1, thresholds applied to
 * the singular values; at inference they are hard thresholds):
 *   r_g = #{ i : s_k[g][i] > tau_k[g] }  (fp32, strict), r_v likewise;
 * and the cache layout that follows from the ranks (see starkv_cache).
 * Host only: the layer's small device tables (channel maps, calibration
 * scratch) are allocated on the current device by the first
 * starkv_build_factors / starkv_bind_factors call.
 * Errors: EINVAL (null, non-positive sizes, H_q % H_kv != 0, n_v < 1 or above
 * min(d, H_kv*d_h), NaN or negative thresholds, non-finite or ascending singular
 * values: each spectrum must be non-increasing), EUNSUPPORTED (dtype/latent
 * combination, d not a multiple of 16, d_h not a multiple of 32 or above 256,
 * every key rank 0, r_v == 0, n_lat above 8192), ENOMEM.
 */
int starkv_layer_create(const starkv_layer_desc* desc, starkv_layer** out);

/* Free a layer handle and its device tables (the caller's buffers are untouched).
 * Waits for nothing: the caller must make sure no enqueued work still uses it. */
int starkv_layer_destroy(starkv_layer* layer);

int starkv_layer_get_info(const starkv_layer* layer, starkv_layer_info* info);

/* ranks_out (host, H_kv + 1 ints): r_0 .. r_{H_kv-1}, then r_v. */
int starkv_layer_ranks(const starkv_layer* layer, int32_t* ranks_out);

/*
 * Build the truncated factors on the GPU (Methodology sections 1 and 2; the
 * kept singular values live in the down-projection):
 *   key head g:  A_g = U_g[:, :r_g] diag(s'_g),  B_g = V_g[:, :r_g]^T
 *   values:      A_v = U_v[:, :r_v] diag(s'_v),  B_v = V_v[:, :r_v]^T
 * with s' = max(s - tau, 0) (shrink = 1) or s (shrink = 0); each element of A
 * is one fp32 multiply then a round-to-nearest-even to dtype, B is V^T rounded.
 * Inputs (device, fp32, row-major): U_k [H_kv][d][d_h], V_k [H_kv][d_h][d_h],
 * U_v [d][n_v], V_v [H_kv*d_h][n_v].
 * Outputs (device, dtype, caller-allocated with the sizes of starkv_layer_info):
 *   A_t  [n_lat][d]       row c = latent channel c (key channels of head 0, 1, ..., then value)
 *   B_k  [n_key][d_h]     row c = key channel c
 *   B_vt [H_kv*d_h][r_v]  B_v transposed: row g*d_h + e, column = value channel
 * The outputs are bound to the layer (as with starkv_bind_factors).
 */
int starkv_build_factors(starkv_layer* layer, const float* U_k, const float* V_k, const float* U_v,
                         const float* V_v, void* A_t, void* B_k, void* B_vt, hipStream_t stream);

/* Bind factor buffers already in the layout above (for example loaded from disk). */
int starkv_bind_factors(starkv_layer* layer, const void* A_t, const void* B_k, const void* B_vt);

/*
 * Per-channel fp16 scales from calibration statistics (Methodology section 3;
 * the abstract: the quantiser uses data statistics).  For every latent channel
 * c: scale_c = fp16_rne( fp32( max_t |(X_cal A)_{t,c}| ) / qmax_c ), with qmax_c
 * the channel's code limit: mix84 127 (int8 channels) and 7 (int4 channels); had43
 * 7 (4-bit outlier channels) and 3 (3-bit inlier channels), A being the rotated
 * down-projection.  X_cal: device [n_cal][d] (dtype).  scales_out: device fp16
 * [n_lat], bound to the layer.  Quantised layers only (mix84, had43; EUNSUPPORTED
 * otherwise); needs bound factors (ESTATE).  Uses the layer's own device scratch:
 * calls on the same layer must not overlap.
 */
int starkv_calibrate(starkv_layer* layer, const void* X_cal, int n_cal, uint16_t* scales_out,
                     hipStream_t stream);

/* Bind caller-provided fp16 scales [n_lat] (quantised layers: mix84, had43). */
int starkv_bind_scales(starkv_layer* layer, const uint16_t* scales);

/* Bytes of k_rows and v_tiles for B sequences of capacity T_max (a multiple of 32);
 * EUNSUPPORTED when one sequence's key rows would reach 4 GiB. */
int starkv_cache_bytes(const starkv_layer* layer, int B, int T_max, size_t* k_bytes, size_t* v_bytes);

/*
 * Project new tokens into the latent and store them (Problem Statement: the
 * cache holds the projected hidden states; Methodology section 3: mixed
 * precision).  For sequence b and new token i, x = X_new[b][i] A (fp32
 * accumulation) is stored at position lens_host[b] + i:
 *   f32 latent: x;  bf16 latent: bf16_rne(x);
 *   mix84 and had43: code_c = clamp(rne(x_c / scale_c), -qmax_c, qmax_c) with an
 *   IEEE fp32 division (code 0 where scale_c == 0) and the code limits of
 *   starkv_calibrate (mix84 127 / 7, had43 7 / 3; x from the rotated factors for
 *   had43), packed as starkv_cache documents (had43 codes in the same byte regions).
 * X_new: device [B][n_new][d] (dtype).  lens_host: host [B], the lengths before
 * the append (the caller updates its lengths itself).  lens_dev: null, or device
 * int32 [B] (4-byte aligned) read by the kernels when they run: the tokens then go
 * after position min(max(lens_dev[b], 0), lens_host[b]), lens_host being an upper
 * bound (see "Device lengths" below).  n_new == 0 is a no-op.
 * Errors: EINVAL, ECAPACITY (lens_host[b] + n_new > T_max), ESTATE, EHIP.
 */
int starkv_compress_append(const starkv_layer* layer, const starkv_cache* cache, const void* X_new, int B,
                           int n_new, const int32_t* lens_host, const int32_t* lens_dev, hipStream_t stream);

/*
 * Device lengths.  The decode calls below and starkv_compress_append take the
 * sequence lengths twice: lens_host (host memory, read during the call) and lens_dev
 * (null, or device int32 [B], read by the kernels when they run).  Without lens_dev
 * the lengths are lens_host.  With it, lens_host is an upper bound that sizes the
 * plan (the split table over 32-token chunks, the XCD placement, the workspace), and
 * sequence b has length T_b = min(max(lens_dev[b], n_q), lens_host[b]) (decode) at the
 * time the kernels run; chunks past T_b count as empty.  A launch sequence captured in
 * a HIP graph with lens_host at a capacity can so be replayed while the caller
 * advances lens_dev (the library never writes it).  The work of the kernels follows
 * lens_host: chunks past T_b are still visited (and masked).  Rotary layers that attend
 * over reconstructed keys (more than 32 query rows per KV head) return EUNSUPPORTED
 * with lens_dev.
 */

/* Workspace bytes that starkv_decode_attention needs for these lengths and n_q. */
int starkv_decode_workspace_bytes(const starkv_layer* layer, int B, int n_q, const int32_t* lens_host,
                                  size_t* bytes);

/*
 * Decode attention read directly from the latent cache (Methodology section 2:
 * the reconstruction matrices are moved past the attention weights).  For
 * sequence b of length T = lens_host[b] (including the n_q newest tokens),
 * query j (position T - n_q + j) and query head h with KV head g = h / G:
 *   q~   = q[b][j][h] B_g^T                       (query in the key latent space)
 *   s_t  = (q~ . x^_g[t]) / sqrt(d_h)  for t <= T - n_q + j   (x^ = code * scale, or the stored latent)
 *   p    = softmax(s)
 *   z    = sum_t p_t x^_v[t]                      (the joint value latent)
 *   out[b][j][h] = z B_v[:, g*d_h:(g+1)*d_h]
 * which equals dense attention over K_g = x^_g B_g and V = x^_v B_v.
 * q: device [B][n_q][H_q][d_h] (dtype); out: device, same shape and dtype.
 * lens_dev: null, or the device lengths (see "Device lengths").
 * ws: device workspace of at least starkv_decode_workspace_bytes() bytes (no
 * alignment beyond 256 bytes needed; contents need no initialisation).
 * Errors: EINVAL (n_q < 1, T < n_q, H_q*n_q > STARKV_MAX_QROWS, ...), ECAPACITY
 * (T > T_max), EWORKSPACE, ESTATE, EUNSUPPORTED, EHIP.  Deterministic: the same
 * inputs give bit-identical outputs.
 */
int starkv_decode_attention(const starkv_layer* layer, const starkv_cache* cache, const void* q, int B,
                            int n_q, const int32_t* lens_host, const int32_t* lens_dev, void* out, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * Weight absorption of the key factors into the query projection (Methodology
 * section 2: the reconstruction matrices are fused into the projections).  W_q:
 * device [d][H_q*d_h] (dtype), the layer's query projection (q = x W_q, head h in
 * columns [h*d_h, (h+1)*d_h)).  Builds, in device memory the layer owns (allocated
 * by the first call, freed by starkv_layer_destroy), for every query head h of KV
 * head g = h / G:  Wqk_h = W_q[:, h] B_g^T  (d x r_g, fp64 sums kept in fp32), so
 * that the query in the key latent space is x Wqk_h directly.  W_q is read during
 * the call only.  Binding or building new factors drops the absorbed factors.
 * Errors: EINVAL (null), ESTATE (no bound factors), ENOMEM, EHIP.
 */
int starkv_absorb_query(starkv_layer* layer, const void* W_q, hipStream_t stream);

/*
 * starkv_decode_attention with the query taken from hidden states: identical
 * except that q[b][j][h] = x[b][j] W_q[:, h] is formed as x[b][j] Wqk_h inside the
 * query projection (the absorbed factors of starkv_absorb_query).
 * x: device [B][n_q][d] (dtype); out: device [B][n_q][H_q][d_h] (dtype).  Same
 * workspace as starkv_decode_attention.  Errors: as starkv_decode_attention, plus
 * ESTATE when no absorbed factors are present.
 */
int starkv_decode_attention_hidden(const starkv_layer* layer, const starkv_cache* cache, const void* x, int B,
                                   int n_q, const int32_t* lens_host, const int32_t* lens_dev, void* out,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * One decode step of a layer (Problem Statement: the new tokens' hidden states are
 * projected into the cache, then attention reads it; Methodology section 2): append
 * the n_q new tokens X_new[b][0 .. n_q-1] at positions lens_host[b] - n_q ..
 * lens_host[b] - 1, then decode attention of q over lens_host[b] tokens.  The result
 * is that of starkv_compress_append (at lengths lens_host - n_q) followed by
 * starkv_decode_attention (at lengths lens_host), bit for bit; with B * n_q <= 16 new
 * rows the append and the query projection share one kernel launch.
 * X_new: device [B][n_q][d] (dtype); q, out: device [B][n_q][H_q][d_h] (dtype).
 * lens_host: host [B], the lengths after the append.  lens_dev: null, or the
 * device lengths after the append (see "Device lengths"; the new tokens go at
 * T_b - n_q ..).  ws: as for starkv_decode_attention (same B, n_q, lens).  Errors:
 * those of the two calls.
 */
int starkv_decode_step(const starkv_layer* layer, const starkv_cache* cache, const void* X_new, const void* q,
                       int B, int n_q, const int32_t* lens_host, const int32_t* lens_dev, void* out, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * Rotary position embedding of the keys and queries (the Llama-family layers the STAR-KV summary
 * page evaluates rotate both by position after the key projection; the latent cache holds the
 * keys before the rotation).  theta: the rotation base (10000 for Llama-2, 500000 for Llama-3);
 * rotary_dim: the rotated dimensions, which must equal d_h (0 turns the rotation off).  For
 * i < d_h / 2 the pair (x_i, x_{i + d_h/2}) of a key at cache position t, or of query j of a
 * chunk of n_q (position T - n_q + j), is rotated by the angle position * theta^(-2 i / d_h).
 * A position-dependent rotation does not commute with the key up-projection (Problem Statement:
 * the reconstruction cost; Methodology section 2: head-wise key factors keep it per head).  With
 * at most 32 query rows per KV head (G n_q <= 32) the decode calls rebuild each 32-token key tile
 * of a head from its latent inside the score kernel, rotate it and score it there; values stay
 * in the latent space.  With more rows starkv_decode_attention, starkv_decode_step and
 * starkv_decode_step_noalloc take the path of starkv_prefill_attention (their workspace query
 * returns its size).  starkv_decode_attention_hidden returns EUNSUPPORTED.
 * Errors: EINVAL (null, rotary_dim < 0 or > d_h, theta not finite and positive), EUNSUPPORTED
 * (rotary_dim != d_h, d_h not a multiple of 64, fp32 layers).  Setup call: not concurrent with
 * other calls on the layer.
 */
int starkv_layer_set_rope(starkv_layer* layer, float theta, int rotary_dim);

/* Workspace bytes of starkv_prefill_attention for these lengths (host math). */
int starkv_prefill_workspace_bytes(const starkv_layer* layer, int B, int n_q, const int32_t* lens_host,
                                   size_t* bytes);

/*
 * Attention of a chunk of n_q queries per sequence (prefill or chunked prefill; any n_q up to
 * the length) over keys and values reconstructed from the latent cache (Problem Statement:
 * reconstruction from the latent; Methodology section 2: K_g = L_g B_g head by head, V = C_v B_v
 * jointly).  Same result as starkv_decode_attention with that n_q (query j at position
 * lens_host[b] - n_q + j sees positions up to its own), with the rotation of
 * starkv_layer_set_rope when set.  For a long chunk rebuilding K and V once (2 T r_v d_h H_kv
 * flops) and attending densely is cheaper than the latent-space order (2 n_q T r_v per head).
 * Steps, all on the stream: the dequantised latent of every cached token (fp32), K^ and V^ per KV
 * head on MFMA (f16, rotated keys), then causal attention with an online softmax over 32-token
 * tiles.  q: device [B][n_q][H_q][d_h] (bf16); out: same shape.  ws: device workspace of
 * starkv_prefill_workspace_bytes (256-byte aligned, no initialisation): the latent and K^, V^ of
 * all sequences (each padded to a multiple of 32 tokens), and for int8/int4 layers an f16 copy of
 * B_v with the value scales folded in (the value reconstruction multiplies the codes by it).  bf16 layers only (EUNSUPPORTED for
 * fp32).  Reconstructed keys and values are held in f16: their magnitudes must stay within its
 * range.  Errors: EINVAL, ECAPACITY, EWORKSPACE, ESTATE, EUNSUPPORTED, EHIP.
 */
int starkv_prefill_attention(const starkv_layer* layer, const starkv_cache* cache, const void* q, int B, int n_q,
                             const int32_t* lens_host, void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * starkv_decode_step without a workspace argument and without any device allocation, for callers
 * that cannot allocate device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Identical results to starkv_decode_step (the
 * same kernels, bit for bit).  The workspace is a static device array of
 * STARKV_NOALLOC_SCRATCH_BYTES in the library, one copy per GPU, held until the process ends;
 * the call uses the copy of the current device (hipGetDevice), which must be the device of the
 * stream and buffers.  Its contents need no initialisation and persist between calls.  All calls
 * on one GPU share that array: calls that overlap in time on one GPU (concurrent streams, or
 * several host threads) race and corrupt each other's results; serialise them.  Errors: those of
 * starkv_decode_step, and EWORKSPACE when the step needs more workspace than the array holds
 * (starkv_decode_workspace_bytes > STARKV_NOALLOC_SCRATCH_BYTES).
 */
#define STARKV_NOALLOC_SCRATCH_BYTES (64u << 20)
int starkv_decode_step_noalloc(const starkv_layer* layer, const starkv_cache* cache, const void* X_new,
                               const void* q, int B, int n_q, const int32_t* lens_host, const int32_t* lens_dev,
                               void* out, hipStream_t stream);

/*
 * Rebuild dense keys and values of sequence b, tokens [t0, t1) (Problem
 * Statement: reconstruction from the latent): K_out[t][g] = x^_g[t] B_g and
 * V_out[t][g] = x^_v[t] B_v[:, g*d_h:(g+1)*d_h], fp32 accumulation, stored in
 * dtype.  K_out, V_out: device [t1 - t0][H_kv][d_h].  Errors: EINVAL (b out of
 * range, t0 > t1, t1 > T_max), ESTATE, EHIP.  t0 == t1 is a no-op.
 */
int starkv_reconstruct(const starkv_layer* layer, const starkv_cache* cache, int b, int t0, int t1,
                       void* K_out, void* V_out, hipStream_t stream);

/* Per-kernel timing of the library's own launches, for measurement (not part of the
 * method).  While enabled, each kernel launch is bracketed by two HIP events recorded on
 * the launch's stream.  starkv_profile_read waits for the recorded events, adds their
 * durations into per-kernel totals, and copies up to max_entries totals into out (host);
 * *n_entries receives the number of distinct kernels.  reset != 0 clears the totals
 * afterwards.  Process-wide; thread-safe.  Errors: EHIP if an event query fails. */
typedef struct starkv_kernel_time {
  char name[32];
  int launches;
  double total_ms;
} starkv_kernel_time;

int starkv_profile_enable(int on);
int starkv_profile_read(starkv_kernel_time* out, int max_entries, int* n_entries, int reset);

#ifdef __cplusplus
}
#endif

#endif /* STARKV_H */
