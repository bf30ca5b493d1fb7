// Latent projection of hidden states (x = X A, fp32 accumulation on MFMA) with two epilogues:
//   append    -- quantise / round and store the new tokens into the cache
//                (STAR-KV summary page, Problem Statement: the cache holds the projected
//                hidden states; Methodology section 3: leading channels int8, the rest int4)
//   calibrate -- per-channel absmax of the calibration latent, then the fp16 scales
//                (abstract: the quantiser uses data statistics)
//
// GEMM shape: rows = tokens, columns = cache slots (the key-row slots then the value slots,
// in cache order, so that the two nibbles of an int4 byte are adjacent columns), K = d.
// Workgroup tile 64 x 64, four waves of 32 x 32 (v_mfma_f32_32x32x16_bf16, or 32x32x2_f32).
#include "device_common.h"
#include "profile.h"
#include "starkv_internal.h"

namespace skv {

struct GemmArgs {
  const void* X;        // [M][d]
  const void* A_t;      // [n_lat][d]
  const int* slot_chan; // [NS]
  int M, d, NS;
  int key_slots, K8, V8;
  int n_key, r_v;
  int latent;
  // append
  int n_new, T_max, k_row_bytes, v_rows;
  uint8_t* k_rows;
  uint8_t* v_tiles;
  const uint16_t* scales;
  int lens[kMaxB];
  // calibrate
  uint32_t* absmax;
};

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
  const int pos = a.lens[b] + (mc - b * a.n_new);
  return m < a.M ? pos : 0;
}

template <int R>
__device__ __forceinline__ void store_latent(const GemmArgs& a, int slot, int chan, const float* xs, const int* ms,
                                             const int* ps) {
  const bool is_key = slot < a.key_slots;
  if (a.latent == STARKV_LATENT_MIX84) {
    int qmax;
    if (is_key) qmax = slot < a.K8 ? 127 : 7;
    else qmax = (slot - a.key_slots) < a.V8 ? 127 : 7;
    const float sc = chan >= 0 ? f16_to_f32(a.scales[chan]) : 0.f;
    const bool nib = qmax == 7;
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
        uint8_t* tile = a.v_tiles + ((size_t)b * (a.T_max / kTT) + pos / kTT) * a.v_rows * kTT;
        if (!nib) tile[(size_t)u * kTT + pos % kTT] = (uint8_t)(code & 0xFF);
        else if ((u & 1) == 0)
          tile[(size_t)(a.V8 + (u - a.V8) / 2) * kTT + pos % kTT] = (uint8_t)((code & 0xF) | ((partner & 0xF) << 4));
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
      uint8_t* tile = a.v_tiles + ((size_t)b * (a.T_max / kTT) + pos / kTT) * a.v_rows * kTT * (a.latent == STARKV_LATENT_F32 ? 4 : 2);
      if (a.latent == STARKV_LATENT_F32) ((float*)tile)[(size_t)u * kTT + pos % kTT] = x;
      else ((uint16_t*)tile)[(size_t)u * kTT + pos % kTT] = f32_to_bf16(x);
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
// rows; the 8 waves split K = d and their 16x16 partial results are summed through LDS.
//   SW = 16 (M <= 16): MFMA row i = token i, column j = slot j.
//   SW = 8 (M <= 8): twice as many workgroups, so that every CU streams A.  Row i and column j
//     of the 16x16 tile take token i % 8 and slot j % 8 over K-half i / 8 (resp. j / 8); the tile
//     holds the two half-K partials of (token, slot) at (i, j) and (i + 8, j + 8), which are added
//     with a cross-lane read.
// A wave issues all its K-steps of loads before its MFMAs; every load is unconditional (rows
// past M read row 0 and are never stored; padding slots read channel 0 with the A_t operand
// zeroed).  The cache positions of the output rows are fetched at the start.
// 16x16x32 bf16 MFMA (16x16x4 f32 for the fp32 path).
template <int DT, int SW, bool MIX>
__global__ __launch_bounds__(512) void k_latent_gemm_skinny(GemmArgs a) {
  constexpr bool HALF = SW == 8;
  constexpr int KU = DT == STARKV_BF16 ? (HALF ? 8 : 16) : (HALF ? 4 : 8);
  constexpr int NL = DT == STARKV_BF16 ? 1 : 2;  // 16-byte loads per operand per K-step
  __shared__ float red[7][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int n = lane & 15, q = lane >> 4;
  const int s0 = blockIdx.x * SW;
  const int bslot = s0 + (HALF ? (n & 7) : n);
  const int bchan = slot_channel_nb<MIX>(a, bslot);
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
  const int per = (kst_all + 7) / 8;
  const int k_beg = wave * per, k_end = min(kst_all, k_beg + per);
  f32x4 acc = {0, 0, 0, 0};
  for (int k0 = k_beg; k0 < k_end; k0 += KU) {
    u32x4 av[KU][NL], bv[KU][NL];
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const size_t ko = (size_t)min(k0 + j, k_end - 1) * 32 + 8 * q;
#pragma unroll
      for (int h = 0; h < NL; ++h) {
        if (DT == STARKV_BF16) {
          av[j][h] = ld16((const uint16_t*)a.X + a_base + ko);
          bv[j][h] = ld16((const uint16_t*)a.A_t + b_base + ko);
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
    for (int w = 0; w < 7; ++w) x += red[w][v][lane];
    // second K-half of (token 4q + v, slot n): D element (4q + 8 + v, n + 8) in lane + 40
    if (HALF) x += __shfl(x, (lane + 40) & 63, 64);
    xs[v] = x;  // D row = token row; D column = n
  }
  store_latent<4>(a, bslot, bchan, xs, ms, ps);
}

template <int DT, int MODE>
__global__ __launch_bounds__(256) void k_latent_gemm(GemmArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave & 1, wn = wave >> 1;
  const int m0 = blockIdx.x * 64 + wm * 32;
  const int s0 = blockIdx.y * 64 + wn * 32;
  const int r = lane & 31, q = lane >> 5;

  const int arow = m0 + r;
  const bool a_ok = arow < a.M;
  const int bslot = s0 + r;
  const int bchan = slot_channel(a, bslot);
  const bool b_ok = bchan >= 0;
  const size_t a_base = (size_t)(a_ok ? arow : 0) * a.d;
  const size_t b_base = (size_t)(b_ok ? bchan : 0) * a.d;

  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;

  for (int k0 = 0; k0 < a.d; k0 += 16) {
    u32x4 alo, ahi, blo, bhi;
    load_frag8<DT>(a.X, a_base + k0 + 8 * q, a_ok, alo, ahi);
    load_frag8<DT>(a.A_t, b_base + k0 + 8 * q, b_ok, blo, bhi);
    if (DT == STARKV_BF16) {
      acc = mfma32_bf16(as_bf16x8(alo), as_bf16x8(blo), acc);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma32_f32(__uint_as_float(alo[e]), __uint_as_float(blo[e]), acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma32_f32(__uint_as_float(ahi[e]), __uint_as_float(bhi[e]), acc);
    }
  }

  // result: lane holds column n = r (slot s0 + r), rows d32_row(v, q)
  const int slot = s0 + r;
  const int chan = slot_channel(a, slot);

  if (MODE == 1) {
    // calibrate: absmax of this column over the 32 rows (rows >= M hold 0)
    float m = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) m = fmaxf(m, fabsf(acc[v]));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    if (q == 0 && chan >= 0) atomicMax(a.absmax + chan, __float_as_uint(m));
    return;
  }

  float xs[16];
  int ms[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    xs[v] = acc[v];
    ms[v] = m0 + d32_row(v, q);
  }
  int ps[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) ps[v] = row_pos(a, ms[v]);
  store_latent<16>(a, slot, chan, xs, ms, ps);
}

__global__ void k_fill_u32(uint32_t* p, int n, uint32_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(256) void k_finish_scales(const uint32_t* __restrict__ absmax, const int* __restrict__ src,
                                                       const int* __restrict__ n8, int n8v, int H_kv, int n_lat,
                                                       uint16_t* __restrict__ scales) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= n_lat) return;
  const int s = src[c];
  const int g = s >> 16, k = s & 0xFFFF;
  const bool is8 = (g < H_kv) ? (k < n8[g]) : (k < n8v);
  const float q = is8 ? 127.f : 7.f;
  scales[c] = f32_to_f16(__uint_as_float(absmax[c]) / q);
}

static void fill_common(const Layer& L, GemmArgs& a, const void* X, int M) {
  a.X = X;
  a.A_t = L.A_t;
  a.slot_chan = L.d_slot_chan;
  a.M = M;
  a.d = L.d;
  a.NS = L.key_slots + L.val_slots;
  a.key_slots = L.key_slots;
  a.K8 = L.K8;
  a.V8 = L.V8;
  a.n_key = L.n_key;
  a.r_v = L.r_v;
  a.latent = L.latent;
}

hipError_t launch_calibrate(const Layer& L, const void* X_cal, int n_cal, uint16_t* scales_out, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_u32, dim3((L.n_lat + 255) / 256), dim3(256), 0, s, L.d_absmax, L.n_lat, 0u);
  GemmArgs a = {};
  fill_common(L, a, X_cal, n_cal);
  a.absmax = L.d_absmax;
  dim3 grid((n_cal + 63) / 64, (a.NS + 63) / 64);
  if (L.dtype == STARKV_BF16) hipLaunchKernelGGL((k_latent_gemm<STARKV_BF16, 1>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_latent_gemm<STARKV_F32, 1>), grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_finish_scales, dim3((L.n_lat + 255) / 256), dim3(256), 0, s, (const uint32_t*)L.d_absmax,
                     (const int*)L.d_src, (const int*)L.d_n8, L.n8v, L.H_kv, L.n_lat, scales_out);
  return hipGetLastError();
}

hipError_t launch_append(const Layer& L, const starkv_cache& c, const void* X_new, int B, int n_new,
                         const int32_t* lens, hipStream_t s) {
  GemmArgs a = {};
  fill_common(L, a, X_new, B * n_new);
  a.n_new = n_new;
  a.T_max = c.T_max;
  a.k_row_bytes = L.k_row_bytes;
  a.v_rows = L.v_rows;
  a.k_rows = (uint8_t*)c.k_rows;
  a.v_tiles = (uint8_t*)c.v_tiles;
  a.scales = L.scales;
  for (int b = 0; b < B; ++b) a.lens[b] = lens[b];
  ProfScope ps("append");
  hipError_t e;
  const bool mix = L.mix();
  if (B * n_new <= 8 && L.d % 64 == 0) {
    const dim3 grid((a.NS + 7) / 8);
    if (L.dtype == STARKV_BF16)
      e = mix ? launch_k(ps, k_latent_gemm_skinny<STARKV_BF16, 8, true>, grid, dim3(512), s, a)
              : launch_k(ps, k_latent_gemm_skinny<STARKV_BF16, 8, false>, grid, dim3(512), s, a);
    else
      e = mix ? launch_k(ps, k_latent_gemm_skinny<STARKV_F32, 8, true>, grid, dim3(512), s, a)
              : launch_k(ps, k_latent_gemm_skinny<STARKV_F32, 8, false>, grid, dim3(512), s, a);
  } else if (B * n_new <= 16 && L.d % 32 == 0) {
    const dim3 grid((a.NS + 15) / 16);
    if (L.dtype == STARKV_BF16)
      e = mix ? launch_k(ps, k_latent_gemm_skinny<STARKV_BF16, 16, true>, grid, dim3(512), s, a)
              : launch_k(ps, k_latent_gemm_skinny<STARKV_BF16, 16, false>, grid, dim3(512), s, a);
    else
      e = mix ? launch_k(ps, k_latent_gemm_skinny<STARKV_F32, 16, true>, grid, dim3(512), s, a)
              : launch_k(ps, k_latent_gemm_skinny<STARKV_F32, 16, false>, grid, dim3(512), s, a);
  } else {
    const dim3 grid((B * n_new + 63) / 64, (a.NS + 63) / 64);
    if (L.dtype == STARKV_BF16) e = launch_k(ps, k_latent_gemm<STARKV_BF16, 0>, grid, dim3(256), s, a);
    else e = launch_k(ps, k_latent_gemm<STARKV_F32, 0>, grid, dim3(256), s, a);
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace skv
