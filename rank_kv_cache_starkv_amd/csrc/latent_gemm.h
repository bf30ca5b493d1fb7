// Latent projection of appended hidden states (x = X A, fp32 accumulation on MFMA) and the
// cache store of its result: argument block, epilogue, and the few-token body shared by the
// append kernel and the fused decode-step front kernel.
//
// STAR-KV summary page, Problem Statement: the cache holds the projected hidden states; Methodology
// section 3: the leading channels of each latent segment are stored as int8, the rest as int4
// (with the block-rotated quantiser: 4-bit outlier codes in the int8 region, 3-bit inlier codes
// in the int4 region).
#pragma once

#include "device_common.h"
#include "starkv_internal.h"

namespace skv {

struct GemmArgs {
  const void* X;        // [M][d]
  const void* A_t;      // [n_lat][d]
  const int* slot_chan; // [NS rounded up to 16]: natural channel of each column, -1 for padding
  int M, d, NS;
  int xmap_rt;          // k_latent_gemm: > 0: row tiles per column tile of an XCD-aware 1-D grid
  int key_slots, K8, V8;
  int pack3, K4, V4;     // had43p: 3-bit inlier planes from key slot K4 and value slot V4 on
  int qmax_hi, qmax_lo;  // code limits of the int8 and int4 regions
  int n_key, r_v;
  int latent;
  // append
  int n_new, T_max, k_row_bytes, v_rows;
  uint8_t* k_rows;
  uint8_t* v_tiles;
  const uint16_t* scales;
  int lens[kMaxB];
  // lengths read on the device (null: lens): rows go after max(lens_dev[b] - lens_sub, 0),
  // at most lens[b]
  const int32_t* lens_dev;
  int lens_sub;
  // calibrate
  uint32_t* absmax;
  // raw fp32 output [M][NS] (the hidden-state query projection): MODE 2 stores X A_t^T, MODE 4
  // stores X (A_t + A_t2)^T with the two parts loaded together
  float* out_f32;
  const void* A_t2;
  // raw output (MODE 2 / 4) of the tiled GEMM: K split over ksplit parts (grid z), part z storing
  // its partial sums at out_f32 + z * out_part (0 or 1: one part)
  int ksplit;
  size_t out_part;
};

// MODE 2 / 4 epilogue: out_f32[m][slot] = x for rows < M and slots < NS.
template <int MODE, int R>  // MODE only documents the caller
__device__ __forceinline__ void store_raw(const GemmArgs& a, int slot, const float* xs, const int* ms) {
#pragma unroll
  for (int v = 0; v < R; ++v) {
    if (ms[v] >= a.M || slot >= a.NS) continue;
    float* o = a.out_f32 + blockIdx.z * a.out_part + (size_t)ms[v] * a.NS + slot;
    *o = xs[v];
  }
}

template <int DT>
__device__ __forceinline__ void load_frag8(const void* base, size_t elem_off, bool ok, u32x4& lo, u32x4& hi) {
  // 8 consecutive elements: bf16 -> lo holds all 8; f32 -> lo elements 0..3, hi 4..7
  if (!ok) {
    lo = u32x4{0, 0, 0, 0};
    hi = lo;
    return;
  }
  if (DT == STARKV_BF16) {
    lo = ld16((const uint16_t*)base + elem_off);
    hi = u32x4{0, 0, 0, 0};
  } else {
    const float* p = (const float*)base + elem_off;
    lo = ld16(p);
    hi = ld16(p + 4);
  }
}

// Store R latent values of one cache slot (column) for R token rows: quantise/pack (mix84) or
// round (bf16) or store (f32).  For int4 slots the even-slot lane of each lane pair writes the
// byte holding both nibbles (the partner slot is in lane ^ 1, same rows); every lane of the wave
// must call this together.
// Cache position of token row m of the appended block (0 for rows past M); no branch, the length
// read at a clamped index.
__device__ __forceinline__ int row_pos(const GemmArgs& a, int m) {
  const int mc = min(m, a.M - 1);
  const int b = mc / a.n_new;
  const int l0 = a.lens_dev ? min(max(a.lens_dev[b] - a.lens_sub, 0), a.lens[b]) : a.lens[b];
  const int pos = l0 + (mc - b * a.n_new);
  return m < a.M ? pos : 0;
}

// Scale of latent channel `chan` for the int8/int4 store (read early by the callers, so that the
// store does not wait on it); 0 for a padding column.
__device__ __forceinline__ uint16_t scale_bits(const GemmArgs& a, int chan) { return a.scales[chan >= 0 ? chan : 0]; }

// Packed 3-bit inlier slots (had43p).  Fields are code + 4 (padding channels 0).  A key row's
// group is three words, one bit per channel, built with three ballots per row:
//   64 x 64 GEMM tiles (SK false): lane = slot, the 32 lanes of a half holding 32 consecutive
//     slots of one 32-channel group, rows d32_row(v, q); the first lane of each half stores the
//     three words.
//   skinny tiles (SK true): 16 consecutive slots (lane & 15) of half a group, rows 4 (lane >> 4)
//     + v; the first lane of each row group sets its 16 bits of the three words with atomic AND /
//     OR (the other half of each word belongs to another workgroup).
// A value channel's tile holds three words over the tile's 32 tokens: the lane merges its
// consecutive rows of one tile into a mask and sets those bits with atomic AND / OR (other tokens
// of the word may belong to earlier appends or to other lanes).
template <int R, bool SK = false>
__device__ __forceinline__ void store_planes3(const GemmArgs& a, int slot, int chan, uint16_t sc_bits, const float* xs,
                                              const int* ms, const int* ps) {
  const int lane = threadIdx.x & 63;
  const bool is_key = slot < a.key_slots;
  const float sc = chan >= 0 ? f16_to_f32(sc_bits) : 0.f;
  int fld[R];
#pragma unroll
  for (int v = 0; v < R; ++v) {
    int code = 0;
    if (sc != 0.f) {
      const float rq = fminf(fmaxf(__builtin_rintf(xs[v] / sc), -(float)a.qmax_lo), (float)a.qmax_lo);
      code = (int)rq;
    }
    fld[v] = chan >= 0 ? code + 4 : 0;
  }
  if (is_key && SK) {
    const int G = (slot - a.K4) >> 5;   // the tile's group (uniform)
    const int sh = (slot - a.K4) & 16;  // its half of the group's words
    const int n = lane & 15, rg = lane >> 4;
#pragma unroll
    for (int v = 0; v < R; ++v) {
      uint32_t w[3];
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        const uint64_t bal = __builtin_amdgcn_ballot_w64(((fld[v] >> b) & 1) != 0);
        w[b] = (uint32_t)(bal >> (16 * rg)) & 0xFFFFu;
      }
      const int m = ms[v];
      if (n != 0 || m >= a.M) continue;
      const int b = m / a.n_new;
      uint32_t* row = (uint32_t*)(a.k_rows + ((size_t)b * a.T_max + ps[v]) * a.k_row_bytes + a.K4 / 2 + 12 * G);
#pragma unroll
      for (int pb = 0; pb < 3; ++pb) {
        atomicAnd(row + pb, ~(0xFFFFu << sh));
        atomicOr(row + pb, w[pb] << sh);
      }
    }
    return;
  }
  if (is_key) {
    const int G = (slot - a.K4) >> 5;  // the wave's group (uniform)
#pragma unroll
    for (int v = 0; v < R; ++v) {
      uint32_t w[3];
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        const uint64_t bal = __builtin_amdgcn_ballot_w64(((fld[v] >> b) & 1) != 0);
        w[b] = (uint32_t)(bal >> (lane & 32));
      }
      const int m = ms[v];
      if ((lane & 31) != 0 || m >= a.M) continue;
      const int b = m / a.n_new;
      uint32_t* row = (uint32_t*)(a.k_rows + ((size_t)b * a.T_max + ps[v]) * a.k_row_bytes + a.K4 / 2 + 12 * G);
      row[0] = w[0];
      row[1] = w[1];
      row[2] = w[2];
    }
    return;
  }
  if (slot >= a.NS) return;
  const int k = slot - a.key_slots - a.V4;  // channel of the 3-bit stream
  const int r3 = a.V4 / 2;                  // first row of the stream
  int cur_b = -1, cur_tile = -1;
  uint32_t mask = 0, bits[3] = {0, 0, 0};
  auto flush = [&]() {
    if (cur_b < 0) return;
#pragma unroll
    for (int pb = 0; pb < 3; ++pb) {
      const int sb = 12 * k + 4 * pb;  // stream byte of the word
      const int row = r3 + (sb >> 5);
      uint32_t* wp = (uint32_t*)(a.v_tiles + vblock_off(cur_b, row >> 5, cur_tile, a.v_rows, a.T_max, 1) + (row & 31) * kTT +
                                 (sb & 31));
      atomicAnd(wp, ~mask);
      atomicOr(wp, bits[pb]);
    }
  };
#pragma unroll
  for (int v = 0; v < R; ++v) {
    const int m = ms[v];
    if (m >= a.M) continue;
    const int b = m / a.n_new;
    const int tile = ps[v] / kTT;
    if (b != cur_b || tile != cur_tile) {
      flush();
      cur_b = b;
      cur_tile = tile;
      mask = 0;
      bits[0] = bits[1] = bits[2] = 0;
    }
    const uint32_t bit = 1u << token_bit3(ps[v] % kTT);
    mask |= bit;
#pragma unroll
    for (int pb = 0; pb < 3; ++pb) bits[pb] |= ((fld[v] >> pb) & 1) ? bit : 0u;
  }
  flush();
}

template <int R, bool SK = false>
__device__ __forceinline__ void store_latent(const GemmArgs& a, int slot, int chan, uint16_t sc_bits, const float* xs,
                                             const int* ms, const int* ps) {
  const bool is_key = slot < a.key_slots;
  if (a.pack3 && (is_key ? slot >= a.K4 : slot - a.key_slots >= a.V4)) {
    store_planes3<R, SK>(a, slot, chan, sc_bits, xs, ms, ps);
    return;
  }
  if (a.latent == STARKV_LATENT_MIX84) {
    const bool nib = is_key ? slot >= a.K8 : (slot - a.key_slots) >= a.V8;
    // the nibbles hold the low block, or with the packed layout the outlier (high) block
    const int qmax = (nib && !a.pack3) ? a.qmax_lo : a.qmax_hi;
    const float sc = chan >= 0 ? f16_to_f32(sc_bits) : 0.f;
#pragma unroll
    for (int v = 0; v < R; ++v) {
      const int m = ms[v];
      int code = 0;
      if (sc != 0.f) {
        const float y = xs[v] / sc;  // IEEE fp32 division
        float rq = __builtin_rintf(y);
        rq = fminf(fmaxf(rq, -(float)qmax), (float)qmax);
        code = (int)rq;
      }
      const int partner = __shfl_xor(code, 1, 64);
      if (m >= a.M || slot >= a.NS) continue;
      const int b = m / a.n_new;
      const int pos = ps[v];
      if (is_key) {
        uint8_t* row = a.k_rows + ((size_t)b * a.T_max + pos) * a.k_row_bytes;
        if (!nib) row[slot] = (uint8_t)(code & 0xFF);
        else if ((slot & 1) == 0) row[a.K8 + (slot - a.K8) / 2] = (uint8_t)((code & 0xF) | ((partner & 0xF) << 4));
      } else {
        const int u = slot - a.key_slots;
        const int vr = nib ? a.V8 + (u - a.V8) / 2 : u;  // tile row: channel, or int4 channel pair
        uint8_t* cell = a.v_tiles + vblock_off(b, vr >> 5, pos / kTT, a.v_rows, a.T_max, 1) + (vr & 31) * kTT + pos % kTT;
        if (!nib) *cell = (uint8_t)(code & 0xFF);
        else if ((u & 1) == 0) *cell = (uint8_t)((code & 0xF) | ((partner & 0xF) << 4));
      }
    }
    return;
  }
  // unquantised latent: fp32 or bf16 elements
#pragma unroll
  for (int v = 0; v < R; ++v) {
    const int m = ms[v];
    if (m >= a.M || slot >= a.NS) continue;
    const int b = m / a.n_new;
    const int pos = ps[v];
    const float x = xs[v];
    if (is_key) {
      uint8_t* row = a.k_rows + ((size_t)b * a.T_max + pos) * a.k_row_bytes;
      if (a.latent == STARKV_LATENT_F32) ((float*)row)[slot] = x;
      else ((uint16_t*)row)[slot] = f32_to_bf16(x);
    } else {
      const int u = slot - a.key_slots;
      const int esz = a.latent == STARKV_LATENT_F32 ? 4 : 2;
      uint8_t* blk = a.v_tiles + vblock_off(b, u >> 5, pos / kTT, a.v_rows, a.T_max, esz);
      if (a.latent == STARKV_LATENT_F32) ((float*)blk)[(u & 31) * kTT + pos % kTT] = x;
      else ((uint16_t*)blk)[(u & 31) * kTT + pos % kTT] = f32_to_bf16(x);
    }
  }
}

// Natural latent channel of GEMM column `slot`, or -1 for a padding column.  Unquantised
// latents keep the natural order (key channels, padding to the row size, value channels), so
// the channel follows from the slot; the int8/int4 layout reorders channels (table lookup).
__device__ __forceinline__ int slot_channel(const GemmArgs& a, int slot) {
  if (slot >= a.NS) return -1;
  if (a.latent == STARKV_LATENT_MIX84) return a.slot_chan[slot];
  if (slot < a.n_key) return slot;
  if (slot < a.key_slots) return -1;
  const int u = slot - a.key_slots;
  return u < a.r_v ? a.n_key + u : -1;
}
// The same without branches (selects only, the table read at a clamped index), so that a
// kernel's prologue does not wait on argument loads one branch at a time.
template <bool MIX>
__device__ __forceinline__ int slot_channel_nb(const GemmArgs& a, int slot) {
  int ch;
  if (MIX) {
    ch = a.slot_chan[min(slot, a.NS - 1)];
  } else {
    const int u = slot - a.key_slots;
    ch = slot < a.n_key ? slot : ((slot >= a.key_slots && u < a.r_v) ? a.n_key + u : -1);
  }
  return slot < a.NS ? ch : -1;
}

// Few-token append (M <= 16 rows): the work is reading A once.  Workgroup = SW cache slots x all
// rows; its NWV waves split K = d and their 16x16 partial results are summed through LDS.
//   SW = 16 (M <= 16): MFMA row i = token i, column j = slot j.
//   SW = 8 (M <= 8): twice as many workgroups, so that every CU streams A.  Row i and column j
//     of the 16x16 tile take token i % 8 and slot j % 8 over K-half i / 8 (resp. j / 8); the tile
//     holds the two half-K partials of (token, slot) at (i, j) and (i + 8, j + 8), which are added
//     with a cross-lane read.
// A wave issues all its K-steps of loads before its MFMAs; every load is unconditional (rows
// past M read row 0 and are never stored; padding slots read channel 0 with the A_t operand
// zeroed).  The cache positions of the output rows are fetched at the start.
// 16x16x32 bf16 MFMA (16x16x4 f32 for the fp32 path).
template <int DT, int SW, bool MIX, int NWV = 8, int MODE = 0>
__device__ __forceinline__ void skinny_body(const GemmArgs& a, int blk, float (*red)[4][64]) {
  constexpr bool HALF = SW == 8;
  // K-steps per load batch: a wave's whole range with 8 waves; at most 32 16-byte loads per lane
  constexpr int KU0 = (DT == STARKV_BF16 ? (HALF ? 8 : 16) : (HALF ? 4 : 8)) * (8 / NWV);
  constexpr int KU = KU0 < (DT == STARKV_BF16 ? 16 : 8) ? KU0 : (DT == STARKV_BF16 ? 16 : 8);
  constexpr int NL = DT == STARKV_BF16 ? 1 : 2;  // 16-byte loads per operand per K-step
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int n = lane & 15, q = lane >> 4;
  const int s0 = blk * SW;
  const int jn = HALF ? (n & 7) : n;  // this lane's slot within the tile
  const int bslot = s0 + jn;
  int bchan;
  if (MIX) {
    // the tile's SW table entries (the table is padded to a multiple of 16) with uniform scalar
    // loads; each lane picks its own
    int t[SW];
#pragma unroll
    for (int i = 0; i < SW; ++i) t[i] = __builtin_amdgcn_readfirstlane(ld_uniform(a.slot_chan + s0 + i));
    bchan = t[0];
#pragma unroll
    for (int i = 1; i < SW; ++i) bchan = jn == i ? t[i] : bchan;
  } else {
    bchan = slot_channel_nb<false>(a, bslot);
  }
  const uint16_t sc_bits = MIX ? scale_bits(a, bchan) : (uint16_t)0;
  const bool b_ok = bchan >= 0;
  const int tok = HALF ? (n & 7) : n;
  const int khalf = HALF ? (n >> 3) : 0;
  const int kst_all = HALF ? a.d / 64 : a.d / 32;  // K-steps of this lane's K range
  const size_t koff = (size_t)khalf * (a.d / 2);
  const size_t a_base = (size_t)(tok < a.M ? tok : 0) * a.d + koff;
  const size_t b_base = (size_t)(b_ok ? bchan : 0) * a.d + koff;
  // output rows of this lane (wave 0 stores them): token 4q + v
  int ms[4], ps[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    ms[v] = (HALF && (q >= 2 || n >= 8)) ? a.M : 4 * q + v;
    ps[v] = row_pos(a, ms[v]);
  }
  const int per = (kst_all + NWV - 1) / NWV;
  const int k_beg = wave * per, k_end = min(kst_all, k_beg + per);
  f32x4 acc = {0, 0, 0, 0};
  for (int k0 = k_beg; k0 < k_end; k0 += KU) {
    u32x4 av[KU][NL], bv[KU][NL], bv2[KU][MODE == 4 ? NL : 1];
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const size_t ko = (size_t)min(k0 + j, k_end - 1) * 32 + 8 * q;
#pragma unroll
      for (int h = 0; h < NL; ++h) {
        if (DT == STARKV_BF16) {
          av[j][h] = ld16((const uint16_t*)a.X + a_base + ko);
          bv[j][h] = ld16((const uint16_t*)a.A_t + b_base + ko);
          if (MODE == 4) bv2[j][0] = ld16((const uint16_t*)a.A_t2 + b_base + ko);
        } else {
          av[j][h] = ld16((const float*)a.X + a_base + ko + 4 * h);
          bv[j][h] = ld16((const float*)a.A_t + b_base + ko + 4 * h);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load of the batch ahead of the MFMAs
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const bool live = b_ok && k0 + j < k_end;
#pragma unroll
      for (int h = 0; h < NL; ++h) bv[j][h] = live ? bv[j][h] : u32x4{0, 0, 0, 0};
      if (DT == STARKV_BF16) {
        acc = mfma16_bf16(as_bf16x8(av[j][0]), as_bf16x8(bv[j][0]), acc);
        if (MODE == 4) {
          const u32x4 b2 = live ? bv2[j][0] : u32x4{0, 0, 0, 0};
          acc = mfma16_bf16(as_bf16x8(av[j][0]), as_bf16x8(b2), acc);
        }
      } else {
#pragma unroll
        for (int h = 0; h < NL; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = mfma16_f32(__uint_as_float(av[j][h][e]), __uint_as_float(bv[j][h][e]), acc);
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave - 1][v][lane] = acc[v];
  }
  __syncthreads();
  if (wave != 0) return;
  float xs[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float x = acc[v];
#pragma unroll
    for (int w = 0; w < NWV - 1; ++w) x += red[w][v][lane];
    // second K-half of (token 4q + v, slot n): D element (4q + 8 + v, n + 8) in lane + 40
    if (HALF) x += __shfl(x, (lane + 40) & 63, 64);
    xs[v] = x;  // D row = token row; D column = n
  }
  if (MODE >= 2) store_raw<MODE, 4>(a, bslot, xs, ms);
  else store_latent<4, !HALF>(a, bslot, bchan, sc_bits, xs, ms, ps);  // (packed 3-bit keys: SW 16 only)
}

// Host side: argument blocks of the latent GEMM for a layer, and for an append into a cache.
void fill_gemm_args(const Layer& L, GemmArgs& a, const void* X, int M);
void fill_append_args(const Layer& L, const starkv_cache& c, GemmArgs& a, const void* X_new, int B, int n_new,
                      const int32_t* lens, const int32_t* lens_dev = nullptr, int lens_sub = 0);

}  // namespace skv
