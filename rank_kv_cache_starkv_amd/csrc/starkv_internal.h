// Host-side state of a libstarkv layer and the launch descriptors of its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/starkv.h"

namespace skv {

constexpr int kTT = STARKV_TILE_TOKENS;  // tokens per value tile
constexpr int kTC = 32;                  // tokens per score chunk (= one value tile)
constexpr int kMaxB = STARKV_MAX_BATCH;
constexpr int kMaxCT = STARKV_MAX_QROWS / 16;  // 16-row column tiles of the key-score GEMM
constexpr int kMaxKT = 32;                     // K-tiles per column tile
constexpr int kMaxSplitsPerSeq = 64;
constexpr int kMaxVPos = 512;  // grid positions of an explicit value-split order

// Value cache [B][v_rows/32 row blocks][T_max/32 token tiles][32 rows][32 tokens x esz]: byte
// offset of row block rb of token tile `tile` of sequence b.  A block (32 rows x 32 tokens) is
// contiguous, and the tiles of one row block follow each other, so a reader that owns a few row
// blocks of a range of tiles streams contiguous memory.
__host__ __device__ __forceinline__ size_t vblock_off(int b, int rb, int tile, int v_rows, int T_max, int esz) {
  return (((size_t)b * (v_rows / 32) + rb) * (size_t)(T_max / kTT) + tile) * (size_t)(32 * kTT * esz);
}

#ifdef __HIPCC__
// Packed 3-bit layout (had43p): bit of token t (0..31) in a value plane word
__host__ __device__ __forceinline__ int token_bit3(int t) { return 8 * (t >> 3) + 4 * (t & 1) + ((t >> 1) & 3); }
// code of inlier channel u (head-major) of a key row: group u / 32 after the K4 / 2 nibble bytes,
// bit u % 32 of its three plane words
__device__ __forceinline__ int key_code3(const uint8_t* row, int K4, int u) {
  const uint32_t* w = (const uint32_t*)(row + K4 / 2 + 12 * (u >> 5));
  const int j = u & 31;
  return (int)(((w[0] >> j) & 1u) | (((w[1] >> j) & 1u) << 1) | (((w[2] >> j) & 1u) << 2)) - 4;
}
// code of inlier value channel w of token t of sequence b: plane words at stream bytes
// 12 w + 4 pb of the token's tile, stream byte x in row V4 / 2 + x / 32, column x % 32
__device__ __forceinline__ int val_code3(const uint8_t* v_tiles, int b, int t, int w, int V4, int v_rows, int T_max) {
  int f = 0;
  const int bit = token_bit3(t % kTT);
#pragma unroll
  for (int pb = 0; pb < 3; ++pb) {
    const int x = 12 * w + 4 * pb;
    const int row = V4 / 2 + (x >> 5);
    const uint32_t word =
        *(const uint32_t*)(v_tiles + vblock_off(b, row >> 5, t / kTT, v_rows, T_max, 1) + (row & 31) * kTT + (x & 31));
    f |= (int)((word >> bit) & 1u) << pb;
  }
  return f - 4;
}
#endif

// Per-KV-head tables on the device (int32 each, H_kv entries unless noted).
struct HeadTables {
  const int* koff;   // [H_kv + 1] first natural key channel of head g
  const int* n8;     // mix84: int8 channels of head g
  const int* off8;   // mix84: first int8 slot of head g
  const int* off4;   // mix84: first int4 slot of head g (relative to K8)
};

struct Layer {
  // description
  int H_q = 0, H_kv = 0, d_h = 0, d = 0, dtype = 0, latent = 0, shrink = 1, n_v = 0;
  int G = 1;
  std::vector<int> rk;      // key ranks
  int r_v = 0;
  std::vector<float> sp_k;  // [H_kv][d_h] kept singular values (s' or s)
  std::vector<float> sp_v;  // [n_v]
  // layout
  int n_key = 0, n_lat = 0;
  std::vector<int> koff, n8, n4, off8, off4;
  int K8 = 0, K4 = 0, V8 = 0, V4 = 0, n8v = 0, n4v = 0;
  int elem = 1;             // bytes per cache element (1 for mix84 codes)
  // block-rotated 4-bit/3-bit quantiser (STARKV_LATENT_HAD43): kept in the mix84 byte format,
  // so `latent` is MIX84 and this flag selects the outlier split, the code limits and the
  // rotated factors
  int had = 0;
  // had43p: the same codes packed to their widths -- outliers in the K4 / V4 nibble regions (no
  // int8 region: K8 = V8 = 0), inliers as 3-bit bit planes in K3 / V3 channels; n8 / n8v count
  // the outliers and n4 / n4v the inliers, off8 is a head's first outlier nibble and off4 its
  // first inlier channel
  int pack3 = 0;
  int K3 = 0, V3 = 0;
  int qmax_hi = 127, qmax_lo = 7;  // code limits of the int8 and int4 regions
  // rotary position embedding of the reconstructed keys and of the queries (0: none)
  float rope_theta = 0.f;
  int rotary_dim = 0;
  int k_row_bytes = 0, v_rows = 0, v_tile_bytes = 0;
  int key_slots = 0, val_slots = 0;  // columns of the append GEMM
  int key_kt = 0;           // K-positions per key-score K-tile (64 for int8 MFMA, 32 otherwise)
  int key_kpos = 0;         // key K-positions (slots) of the key row
  // device tables (owned)
  void* dev_tables = nullptr;
  int* d_slot_chan = nullptr;  // [key_slots + val_slots] natural channel of each GEMM column or -1
  double* d_rope_w = nullptr;  // rotary layers: [d_h / 2] theta^(-2 j / d_h)
  float* d_rope_tab = nullptr;  // rotary layers: [32][d_h / 2] (cos, sin) of r theta^(-2 j / d_h)
  int* d_koff = nullptr;
  int* d_n8 = nullptr;
  int* d_off8 = nullptr;
  int* d_off4 = nullptr;
  float* d_sp = nullptr;       // [n_lat] kept singular value of each natural channel
  int* d_src = nullptr;        // [n_lat] (head << 16) | local index; head = H_kv for values
  int* d_rot = nullptr;        // [n_lat] rotated factors: (first channel of the Hadamard piece << 5) | log2(order)
  uint32_t* d_absmax = nullptr;  // [n_lat] calibration scratch
  float* d_wqk = nullptr;        // [G * n_key][d] absorbed query factors W_q^h B_g^T, fp32 or bf16 hi + lo
                                 // (owned; null: none)
  // bound buffers (borrowed)
  const void* A_t = nullptr;
  const void* B_k = nullptr;
  const void* B_vt = nullptr;
  const uint16_t* scales = nullptr;

  HeadTables heads() const { return HeadTables{d_koff, d_n8, d_off8, d_off4}; }
  bool mix() const { return latent == STARKV_LATENT_MIX84; }
};

// ---------------------------------------------------------------------------
// decode plan (host-built per call, passed by value to the kernels)

struct DecodeGeom {
  int B, n_q, M_q, M_pad, nct, G, d_h, H_q, H_kv, d;
  int n_key, r_v, K8, K4, key_kt, key_kpos, k_row_bytes, v_rows, v_tile_bytes, T_max;
  int K3, pack3;  // packed 3-bit key region (channels) and the packed-layout flag
  int rv_ld;  // row stride (elements) of the value-latent workspace rows: r_v rounded up to 32
  int latent, dtype;
  float qscale;  // log2(e) / sqrt(d_h)
};

// K-tiles touched by each 16-row column tile of the key-score GEMM: at most two contiguous runs
// (bf16/fp32: one; int8/int4: one in each region), so K-tile jt of column tile ct is
// s0 + jt for jt < n0, else s1 + (jt - n0).
struct KtList {
  int n[kMaxCT];
  int s0[kMaxCT], n0[kMaxCT], s1[kMaxCT];
#ifdef __HIPCC__
  __host__ __device__ __forceinline__ int at(int ct, int jt) const { return jt < n0[ct] ? s0[ct] + jt : s1[ct] + (jt - n0[ct]); }
#endif
};

struct SeqTable {
  // every sequence the same length: positions follow by division (no table reads on the device)
  int uni, u_len, u_nch, u_nspl, u_nblk;
  // lengths read on the device at run time (null: the planned lengths are the lengths).  The
  // plan's lengths are then upper bounds: sequence b attends over min(max(lens_dev[b], len_lo),
  // planned length) tokens, so chunks and splits past that length are empty.
  const int32_t* lens_dev;
  int len_lo;
  int lens[kMaxB];
  int chunk_off[kMaxB + 1];  // prefix of 32-token chunks per sequence
  int split_off[kMaxB + 1];  // prefix of value splits per sequence
  int blk_off[kMaxB + 1];    // prefix of 128-token score blocks per sequence
};

// Explicit order of the value splits over the positions of the value grid (ragged batches): the
// workgroups of position p (p mod 8 = the XCD that runs them) take split sg[p]; 0xFFFF marks a
// position with no split.  n = 0: the kernels' own order.
struct ValueOrder {
  int n;  // positions, a multiple of 8 (at most kMaxVPos)
  uint16_t sg[kMaxVPos];
};

struct DecodeWs {
  // all device pointers into the caller's workspace
  void* qfrag;      // [B][nct][kMaxKT? -> nkt_max][2048 bytes]
  float* rowp;      // [B][M_pad][4]  (rho, bias_hi, bias_lo, 0)
  void* p;          // [total_chunks][M_pad][kTC] probabilities (f16 / bf16 / f32)
  float* cm;        // [total_chunks][M_pad] chunk max (log2 units)
  float* cl;        // [total_chunks][M_pad] chunk sum
  void* zp;         // [total_splits][M_pad][rv_ld] value-latent partials: fp32, weighted against
                    // sm (bf16/fp32 latents); f16, divided by the split's sum sl (int8/int4
                    // latents: a weighted mean of codes, within the code range)
  float* sl;        // [total_splits][M_pad] split sum of the probabilities, weighted against sm
  float* sm;        // [total_splits][M_pad] split maximum of the base-2 logits (the weights' reference)
  float* zt;        // [B][M_pad][rv_ld] merged value latent (scaled, normalised; zero padding)
  float* qraw;      // [qraw_parts][B n_q][G n_key] hidden-state query projection (absorbed path): K parts
  int qraw_parts;
  int nkt_max;
  int total_chunks, total_splits;
  int cps;          // score chunks per value split
  int blocks_per_wg;  // value blocks (waves) per value WG (several query-row tiles)
  int n_sl8, n_sl4;   // one-row-tile value kernel: slices of one-N-tile blocks / of int4 blocks
  int n_sl3;          // ... and (packed layout) slices of two 3-bit N-tiles
  int nbw8, nbw4;     // blocks per slice of each kind
  int n_grp;          // many-row value kernel: groups of four 32-channel N-tiles
};

struct DecodePlan {
  DecodeGeom g;
  DecodeWs ws;
  ValueOrder vo;
  size_t ws_bytes;
};

int plan_decode(const Layer& L, int B, int n_q, const int32_t* lens, int T_max, void* ws_base, DecodePlan* plan,
                KtList* kts, SeqTable* seq);

// q: [B][n_q][H_q][d_h] queries, or with wqk set [B][n_q][d] hidden states whose query
// projection is absorbed into wqk
// rotary layers: whether decode scores rebuilt key tiles in the latent-space path (else it attends
// over fully reconstructed keys and values)
bool rope_latent_scores(const Layer& L, int n_q);
hipError_t launch_decode(const Layer& L, const DecodePlan& plan, const KtList& kts, const SeqTable& seq,
                         const void* q, void* out, const void* k_rows, const void* v_tiles, hipStream_t s,
                         const float* wqk = nullptr);

// Absorbed query factors: wqk[G r_g-row block of head h][e] = sum_c W_q[e][h d_h + c] B_k[row][c]
// (fp32; bf16 layers: bf16 high part then bf16 low part, the same bytes).
hipError_t launch_absorb_query(const Layer& L, const void* W_q, float* wqk, hipStream_t s);

// out[m][c] = x[m] . wqk[c] for M hidden rows and the G n_key absorbed columns (fp32 out); the
// timing events start, stop (either may be null) bracket all of its launches.
hipError_t launch_hidden_query(const Layer& L, const void* x, int M, const void* wqk_hi, const void* wqk_lo,
                               float* out, hipStream_t s, hipEvent_t start, hipEvent_t stop);
// K parts of that projection for M hidden rows and NS absorbed columns: its output holds that many
// [M][NS] partial sums one after another (1 for the skinny form of at most 16 rows)
int hidden_query_parts(int M, int NS);

// A decode step: append n_q new tokens per sequence at lens_pre, then decode attention over
// plan's lengths (lens_pre + n_q); few new rows run the append and the query projection in one
// launch.
hipError_t launch_step(const Layer& L, const starkv_cache& c, const DecodePlan& plan, const KtList& kts,
                       const SeqTable& seq, const void* X_new, const int32_t* lens_pre, const void* q, void* out,
                       hipStream_t s);

hipError_t launch_build_factors(const Layer& L, const float* U_k, const float* V_k, const float* U_v,
                                const float* V_v, void* A_t, void* B_k, void* B_vt, hipStream_t s);

hipError_t launch_calibrate(const Layer& L, const void* X_cal, int n_cal, uint16_t* scales_out, hipStream_t s);

// lens_dev (optional): rows of sequence b go after max(lens_dev[b] - lens_sub, 0), at most lens[b]
hipError_t launch_append(const Layer& L, const starkv_cache& c, const void* X_new, int B, int n_new,
                         const int32_t* lens, hipStream_t s, const int32_t* lens_dev = nullptr, int lens_sub = 0);

hipError_t launch_reconstruct(const Layer& L, const starkv_cache& c, int b, int t0, int t1, void* K_out,
                              void* V_out, hipStream_t s);

// Attention over reconstructed keys and values (query chunks of any length; rotary layers):
// workspace bytes for these lengths, and the launch (q, out: [B][n_q][H_q][d_h], bf16 layers).
size_t prefill_workspace_bytes(const Layer& L, int B, const int32_t* lens);
hipError_t launch_prefill(const Layer& L, const starkv_cache& c, const void* q, int B, int n_q, const int32_t* lens,
                          void* out, void* ws, hipStream_t s);

}  // namespace skv
