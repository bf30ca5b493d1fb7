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
#include "latent_gemm.h"
#include "profile.h"
#include "starkv_internal.h"

namespace skv {

template <int DT, int SW, bool MIX>
__global__ __launch_bounds__(512) void k_latent_gemm_skinny(GemmArgs a) {
  __shared__ float red[7][4][64];
  skinny_body<DT, SW, MIX>(a, blockIdx.x, red);
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
  const uint16_t sc_bits = (MODE == 0 && a.latent == STARKV_LATENT_MIX84) ? scale_bits(a, bchan) : (uint16_t)0;
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
  store_latent<16>(a, slot, chan, sc_bits, xs, ms, ps);
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

void fill_gemm_args(const Layer& L, GemmArgs& a, const void* X, int M) {
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

void fill_append_args(const Layer& L, const starkv_cache& c, GemmArgs& a, const void* X_new, int B, int n_new,
                      const int32_t* lens) {
  fill_gemm_args(L, a, X_new, B * n_new);
  a.n_new = n_new;
  a.T_max = c.T_max;
  a.k_row_bytes = L.k_row_bytes;
  a.v_rows = L.v_rows;
  a.k_rows = (uint8_t*)c.k_rows;
  a.v_tiles = (uint8_t*)c.v_tiles;
  a.scales = L.scales;
  for (int b = 0; b < B; ++b) a.lens[b] = lens[b];
}

hipError_t launch_calibrate(const Layer& L, const void* X_cal, int n_cal, uint16_t* scales_out, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_u32, dim3((L.n_lat + 255) / 256), dim3(256), 0, s, L.d_absmax, L.n_lat, 0u);
  GemmArgs a = {};
  fill_gemm_args(L, a, X_cal, n_cal);
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
  fill_append_args(L, c, a, X_new, B, n_new, lens);
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
