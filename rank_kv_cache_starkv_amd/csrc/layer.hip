// Layer setup: rank selection, cache layout, device tables, and the factor-build kernels.
//
// STAR-KV summary page, Methodology section 1 (thresholds on the singular values,
// hard at inference, projections truncated) and section 2 (keys head by head,
// values jointly); section 3 for the leading-channel split of the latent and for the
// block-wise Hadamard rotation that is folded into the factors.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "device_common.h"
#include "starkv_internal.h"

namespace skv {

static int ceil_to(int x, int m) { return (x + m - 1) / m * m; }

int layer_init(const starkv_layer_desc& d, Layer* L) {
  L->H_q = d.H_q;
  L->H_kv = d.H_kv;
  L->d_h = d.d_h;
  L->d = d.d;
  L->dtype = d.dtype;
  // the block-rotated quantiser keeps the mix84 byte format (and kernels)
  L->had = d.latent == STARKV_LATENT_HAD43 || d.latent == STARKV_LATENT_HAD43P;
  L->pack3 = d.latent == STARKV_LATENT_HAD43P;
  L->latent = L->had ? STARKV_LATENT_MIX84 : d.latent;
  L->qmax_hi = L->had ? 7 : 127;  // 4-bit outlier codes, or int8
  L->qmax_lo = L->had ? 3 : 7;    // 3-bit inlier codes, or int4
  L->shrink = d.shrink;
  L->n_v = d.n_v;
  L->G = d.H_q / d.H_kv;
  // rank selection: strict comparison in fp32; kept values shrunk by tau (or not)
  L->rk.assign(d.H_kv, 0);
  L->sp_k.assign((size_t)d.H_kv * d.d_h, 0.f);
  for (int g = 0; g < d.H_kv; ++g) {
    const float tau = d.tau_k[g];
    int r = 0;
    for (int i = 0; i < d.d_h; ++i) {
      const float s = d.s_k[(size_t)g * d.d_h + i];
      if (s > tau) ++r;
      L->sp_k[(size_t)g * d.d_h + i] = d.shrink ? std::max(s - tau, 0.0f) : s;
    }
    L->rk[g] = r;
  }
  int rv = 0;
  L->sp_v.assign(d.n_v, 0.f);
  for (int i = 0; i < d.n_v; ++i) {
    if (d.s_v[i] > d.tau_v) ++rv;
    L->sp_v[i] = d.shrink ? std::max(d.s_v[i] - d.tau_v, 0.0f) : d.s_v[i];
  }
  L->r_v = rv;
  L->n_key = 0;
  L->koff.assign(d.H_kv + 1, 0);
  for (int g = 0; g < d.H_kv; ++g) {
    L->koff[g + 1] = L->koff[g] + L->rk[g];
  }
  L->n_key = L->koff[d.H_kv];
  L->n_lat = L->n_key + L->r_v;
  if (L->n_key == 0 || L->r_v == 0) return STARKV_EUNSUPPORTED;

  // cache layout
  L->n8.assign(d.H_kv, 0);
  L->n4.assign(d.H_kv, 0);
  L->off8.assign(d.H_kv + 1, 0);
  L->off4.assign(d.H_kv + 1, 0);
  if (L->mix()) {
    // high-precision block: the leading quarter (int8/int4), or the leading fifth (outliers)
    const int den = L->had ? 5 : 4;
    for (int g = 0; g < d.H_kv; ++g) {
      L->n8[g] = (L->rk[g] + den - 1) / den;
      L->n4[g] = L->rk[g] - L->n8[g];
      L->off8[g + 1] = L->off8[g] + L->n8[g];
      L->off4[g + 1] = L->off4[g] + L->n4[g];
    }
    L->n8v = (L->r_v + den - 1) / den;
    L->n4v = L->r_v - L->n8v;
    if (L->pack3) {
      // outlier nibbles, then inlier bit planes (groups of 32 channels, 12 bytes each)
      L->K8 = 0;
      L->K4 = ceil_to(L->off8[d.H_kv], 64);
      L->K3 = ceil_to(L->off4[d.H_kv], 64);
      L->k_row_bytes = ceil_to(L->K4 / 2 + 3 * L->K3 / 8, 16);
      L->V8 = 0;
      L->V4 = ceil_to(L->n8v, 64);
      L->V3 = ceil_to(L->n4v, 64);
      L->v_rows = ceil_to(L->V4 / 2 + 3 * L->V3 / 8, 32);
      L->key_slots = L->K4 + L->K3;
      L->val_slots = L->V4 + L->V3;
      L->key_kpos = L->K4 + L->K3;
    } else {
      L->K8 = ceil_to(L->off8[d.H_kv], 16);
      L->K4 = ceil_to(L->off4[d.H_kv], 32);
      L->k_row_bytes = L->K8 + L->K4 / 2;
      L->V8 = ceil_to(L->n8v, 32);
      L->V4 = ceil_to(L->n4v, 64);
      L->v_rows = L->V8 + L->V4 / 2;
      L->key_slots = L->K8 + L->K4;
      L->val_slots = L->V8 + L->V4;
      L->key_kpos = L->K8 + L->K4;
    }
    L->elem = 1;
    L->key_kt = 64;
  } else {
    L->elem = (L->latent == STARKV_LATENT_F32) ? 4 : 2;
    L->k_row_bytes = ceil_to(L->n_key * L->elem, 16);
    L->key_slots = L->k_row_bytes / L->elem;
    L->v_rows = ceil_to(L->r_v, 32);
    L->val_slots = L->v_rows;
    L->key_kt = 32;
    L->key_kpos = L->key_slots;
  }
  L->v_tile_bytes = L->v_rows * kTT * L->elem;
  return STARKV_OK;
}

int layer_write_rope(Layer* L);

int layer_upload_tables(Layer* L) {
  const int NS = L->key_slots + L->val_slots;
  // padded to a multiple of 16 entries (-1): a 16-slot GEMM tile reads its entries unclamped
  const int NSP = (NS + 15) / 16 * 16;
  std::vector<int> slot_chan(NSP, -1);
  if (L->pack3) {
    // key slots: outlier nibbles [0, K4), inlier planes [K4, K4 + K3); value slots likewise
    for (int g = 0; g < L->H_kv; ++g) {
      for (int k = 0; k < L->n8[g]; ++k) slot_chan[L->off8[g] + k] = L->koff[g] + k;
      for (int k = 0; k < L->n4[g]; ++k) slot_chan[L->K4 + L->off4[g] + k] = L->koff[g] + L->n8[g] + k;
    }
    for (int k = 0; k < L->n8v; ++k) slot_chan[L->key_slots + k] = L->n_key + k;
    for (int k = 0; k < L->n4v; ++k) slot_chan[L->key_slots + L->V4 + k] = L->n_key + L->n8v + k;
  } else if (L->mix()) {
    for (int g = 0; g < L->H_kv; ++g) {
      for (int k = 0; k < L->n8[g]; ++k) slot_chan[L->off8[g] + k] = L->koff[g] + k;
      for (int k = 0; k < L->n4[g]; ++k) slot_chan[L->K8 + L->off4[g] + k] = L->koff[g] + L->n8[g] + k;
    }
    for (int k = 0; k < L->n8v; ++k) slot_chan[L->key_slots + k] = L->n_key + k;
    for (int k = 0; k < L->n4v; ++k) slot_chan[L->key_slots + L->V8 + k] = L->n_key + L->n8v + k;
  } else {
    for (int c = 0; c < L->n_key; ++c) slot_chan[c] = c;
    for (int k = 0; k < L->r_v; ++k) slot_chan[L->key_slots + k] = L->n_key + k;
  }
  std::vector<float> sp(L->n_lat);
  std::vector<int> src(L->n_lat);
  for (int g = 0; g < L->H_kv; ++g)
    for (int k = 0; k < L->rk[g]; ++k) {
      sp[L->koff[g] + k] = L->sp_k[(size_t)g * L->d_h + k];
      src[L->koff[g] + k] = (g << 16) | k;
    }
  for (int k = 0; k < L->r_v; ++k) {
    sp[L->n_key + k] = L->sp_v[k];
    src[L->n_key + k] = (L->H_kv << 16) | k;
  }
  // Hadamard pieces of the rotated quantiser: each segment's outlier block, then its inlier
  // block, cut into the powers of two of their sizes (largest first); without rotation every
  // channel is a piece of order 1
  std::vector<int> rot(L->n_lat);
  auto pieces = [&](int c, int n) {
    for (int b = 30; b >= 0; --b)
      if ((n >> b) & 1) {
        for (int j = 0; j < (1 << b); ++j) rot[c + j] = (c << 5) | b;
        c += 1 << b;
      }
  };
  for (int g = 0; g < L->H_kv; ++g) {
    if (L->had) {
      pieces(L->koff[g], L->n8[g]);
      pieces(L->koff[g] + L->n8[g], L->n4[g]);
    } else {
      for (int k = 0; k < L->rk[g]; ++k) rot[L->koff[g] + k] = (L->koff[g] + k) << 5;
    }
  }
  if (L->had) {
    pieces(L->n_key, L->n8v);
    pieces(L->n_key + L->n8v, L->n4v);
  } else {
    for (int k = 0; k < L->r_v; ++k) rot[L->n_key + k] = (L->n_key + k) << 5;
  }
  const int H = L->H_kv;
  // one allocation: slot_chan | koff(H+1) | n8(H) | off8(H+1) | off4(H+1) | sp | src | rot | absmax
  // | (16-byte aligned) rotary frequencies [d_h / 2] (double) | rotary table [32][d_h / 2] (float2),
  // the last two written by starkv_layer_set_rope
  size_t n_int = (size_t)NSP + (H + 1) + H + (H + 1) + (H + 1);
  const size_t o_rope = (n_int * 4 + (size_t)L->n_lat * 4 * 4 + 15) & ~(size_t)15;
  size_t bytes = o_rope + (size_t)(L->d_h / 2) * 8 + 32 * (size_t)(L->d_h / 2) * 8;
  std::vector<uint8_t> host(bytes, 0);
  size_t o = 0;
  auto put = [&](const void* p, size_t nb) { memcpy(host.data() + o, p, nb); o += nb; };
  put(slot_chan.data(), NSP * 4);
  put(L->koff.data(), (H + 1) * 4);
  put(L->n8.data(), H * 4);
  put(L->off8.data(), (H + 1) * 4);
  put(L->off4.data(), (H + 1) * 4);
  put(sp.data(), L->n_lat * 4);
  put(src.data(), L->n_lat * 4);
  put(rot.data(), L->n_lat * 4);
  void* dev = nullptr;
  if (hipMalloc(&dev, bytes) != hipSuccess) return STARKV_ENOMEM;
  if (hipMemcpy(dev, host.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(dev);
    return STARKV_EHIP;
  }
  L->dev_tables = dev;
  uint8_t* b = (uint8_t*)dev;
  o = 0;
  L->d_slot_chan = (int*)(b + o); o += NSP * 4;
  L->d_koff = (int*)(b + o); o += (H + 1) * 4;
  L->d_n8 = (int*)(b + o); o += H * 4;
  L->d_off8 = (int*)(b + o); o += (H + 1) * 4;
  L->d_off4 = (int*)(b + o); o += (H + 1) * 4;
  L->d_sp = (float*)(b + o); o += L->n_lat * 4;
  L->d_src = (int*)(b + o); o += L->n_lat * 4;
  L->d_rot = (int*)(b + o); o += L->n_lat * 4;
  L->d_absmax = (uint32_t*)(b + o);
  L->d_rope_w = (double*)(b + o_rope);
  L->d_rope_tab = (float*)(b + o_rope + (size_t)(L->d_h / 2) * 8);
  return layer_write_rope(L);
}

// The rotation's frequencies theta^(-2 j / d_h) and the (cos, sin) of r times them for the 32
// token offsets of a tile, in fp64 (the table rounded to fp32), into the layer's device tables;
// nothing when the layer has no rotation or no device tables yet.
int layer_write_rope(Layer* L) {
  if (!L->dev_tables || !(L->rope_theta > 0.f)) return STARKV_OK;
  const int np = L->d_h / 2;
  std::vector<double> w(np);
  std::vector<float> tab(32 * (size_t)np * 2);
  const double lt = std::log2((double)L->rope_theta);
  for (int j = 0; j < np; ++j) w[j] = std::exp2(-2.0 * (double)j / (double)L->d_h * lt);
  for (int r = 0; r < 32; ++r)
    for (int j = 0; j < np; ++j) {
      const double ang = (double)r * w[j];
      tab[2 * ((size_t)r * np + j)] = (float)std::cos(ang);
      tab[2 * ((size_t)r * np + j) + 1] = (float)std::sin(ang);
    }
  if (hipMemcpy(L->d_rope_w, w.data(), np * sizeof(double), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(L->d_rope_tab, tab.data(), tab.size() * sizeof(float), hipMemcpyHostToDevice) != hipSuccess)
    return STARKV_EHIP;
  return STARKV_OK;
}

// ---------------------------------------------------------------------------
// factor build: A^T[c][i] = rne(U[i][k] * s'[c]), B_k[c][e] = rne(V_g[e][k]), B_v^T[j][k] = rne(V_v[j][k])

template <typename T>
__device__ __forceinline__ void store_dt(T* p, size_t i, float x);
template <>
__device__ __forceinline__ void store_dt<float>(float* p, size_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void store_dt<uint16_t>(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16(x); }

template <typename T>
__global__ __launch_bounds__(256) void k_build_a(const float* __restrict__ U_k, const float* __restrict__ U_v,
                                                 const float* __restrict__ sp, const int* __restrict__ src,
                                                 T* __restrict__ A_t, int d, int d_h, int n_v, int H_kv) {
  const int c = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= d) return;
  const int s = src[c];
  const int g = s >> 16, k = s & 0xFFFF;
  const float u = (g < H_kv) ? U_k[((size_t)g * d + i) * d_h + k] : U_v[(size_t)i * n_v + k];
  store_dt<T>(A_t, (size_t)c * d + i, __fmul_rn(u, sp[c]));
}

template <typename T>
__global__ __launch_bounds__(256) void k_build_bk(const float* __restrict__ V_k, const int* __restrict__ src,
                                                  T* __restrict__ B_k, int n_key, int d_h) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= n_key * d_h) return;
  const int c = idx / d_h, e = idx % d_h;
  const int s = src[c];
  const int g = s >> 16, k = s & 0xFFFF;
  store_dt<T>(B_k, idx, V_k[((size_t)g * d_h + e) * d_h + k]);
}

template <typename T>
__global__ __launch_bounds__(256) void k_build_bv(const float* __restrict__ V_v, T* __restrict__ B_vt, int rows,
                                                  int r_v, int n_v) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)rows * r_v) return;
  const size_t j = idx / r_v, k = idx % r_v;
  store_dt<T>(B_vt, idx, V_v[j * n_v + k]);
}

// Rotated factors (block-wise Hadamard folded into the factors, Methodology section 3): for
// the Sylvester piece of order n = 2^m starting at natural channel c0, with H[j][l] =
// (-1)^popcount(j & l),
//   A'[:, c0 + l] = sum_j H[j][l] fp32(U[:, c0 + j] s'[c0 + j])       (A' = A H)
//   B'[c0 + l, :] = (1/n) sum_j H[l][j] B[c0 + j, :]                   (B' = H^T B / n)
// so that A' B' = A B.  Sums in fp64, in piece order, then rounded to fp32 and to the
// factor type.
__device__ __forceinline__ double had_sign(int j, int l, double x) { return (__popc(j & l) & 1) ? -x : x; }
// fp64 -> fp32 (RNE); the empty register barrier keeps the compiler from merging this rounding
// and the later fp32 -> bf16 one into a single fp64 -> bf16 rounding, which differs at ties
__device__ __forceinline__ float to_f32_kept(double x) {
  float f = (float)x;
  asm volatile("" : "+v"(f));
  return f;
}

template <typename T>
__global__ __launch_bounds__(256) void k_build_a_rot(const float* __restrict__ U_k, const float* __restrict__ U_v,
                                                     const float* __restrict__ sp, const int* __restrict__ src,
                                                     const int* __restrict__ rot, T* __restrict__ A_t, int d, int d_h,
                                                     int n_v, int H_kv) {
  const int c = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= d) return;
  const int rt = rot[c];
  const int c0 = rt >> 5, n = 1 << (rt & 31), l = c - c0;
  double acc = 0.0;
  for (int j = 0; j < n; ++j) {
    const int s = src[c0 + j];
    const int g = s >> 16, k = s & 0xFFFF;
    const float u = (g < H_kv) ? U_k[((size_t)g * d + i) * d_h + k] : U_v[(size_t)i * n_v + k];
    acc += had_sign(j, l, (double)__fmul_rn(u, sp[c0 + j]));
  }
  store_dt<T>(A_t, (size_t)c * d + i, to_f32_kept(acc));
}

template <typename T>
__global__ __launch_bounds__(256) void k_build_bk_rot(const float* __restrict__ V_k, const int* __restrict__ src,
                                                      const int* __restrict__ rot, T* __restrict__ B_k, int n_key,
                                                      int d_h) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= n_key * d_h) return;
  const int c = idx / d_h, e = idx % d_h;
  const int rt = rot[c];
  const int c0 = rt >> 5, m = rt & 31, l = c - c0;
  double acc = 0.0;
  for (int j = 0; j < (1 << m); ++j) {
    const int s = src[c0 + j];
    const int g = s >> 16, k = s & 0xFFFF;
    acc += had_sign(l, j, (double)V_k[((size_t)g * d_h + e) * d_h + k]);
  }
  store_dt<T>(B_k, idx, to_f32_kept(acc / (double)(1 << m)));
}

template <typename T>
__global__ __launch_bounds__(256) void k_build_bv_rot(const float* __restrict__ V_v, const int* __restrict__ rot,
                                                      T* __restrict__ B_vt, int rows, int r_v, int n_v, int n_key) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)rows * r_v) return;
  const size_t jr = idx / r_v;
  const int k = (int)(idx % r_v);
  const int rt = rot[n_key + k];
  const int k0 = (rt >> 5) - n_key, m = rt & 31, l = k - k0;
  double acc = 0.0;
  for (int j = 0; j < (1 << m); ++j) acc += had_sign(l, j, (double)V_v[jr * n_v + k0 + j]);
  store_dt<T>(B_vt, idx, to_f32_kept(acc / (double)(1 << m)));
}

template <typename T>
static hipError_t build_factors_rot(const Layer& L, const float* U_k, const float* V_k, const float* U_v,
                                    const float* V_v, void* A_t, void* B_k, void* B_vt, hipStream_t s) {
  dim3 ga((L.d + 255) / 256, L.n_lat);
  hipLaunchKernelGGL(k_build_a_rot<T>, ga, dim3(256), 0, s, U_k, U_v, L.d_sp, L.d_src, L.d_rot, (T*)A_t, L.d, L.d_h,
                     L.n_v, L.H_kv);
  const int nbk = L.n_key * L.d_h;
  hipLaunchKernelGGL(k_build_bk_rot<T>, dim3((nbk + 255) / 256), dim3(256), 0, s, V_k, L.d_src, L.d_rot, (T*)B_k,
                     L.n_key, L.d_h);
  const size_t nbv = (size_t)L.H_kv * L.d_h * L.r_v;
  hipLaunchKernelGGL(k_build_bv_rot<T>, dim3((unsigned)((nbv + 255) / 256)), dim3(256), 0, s, V_v, L.d_rot,
                     (T*)B_vt, L.H_kv * L.d_h, L.r_v, L.n_v, L.n_key);
  return hipGetLastError();
}

template <typename T>
static hipError_t build_factors_t(const Layer& L, const float* U_k, const float* V_k, const float* U_v,
                                  const float* V_v, void* A_t, void* B_k, void* B_vt, hipStream_t s) {
  dim3 ga((L.d + 255) / 256, L.n_lat);
  hipLaunchKernelGGL(k_build_a<T>, ga, dim3(256), 0, s, U_k, U_v, L.d_sp, L.d_src, (T*)A_t, L.d, L.d_h, L.n_v,
                     L.H_kv);
  const int nbk = L.n_key * L.d_h;
  hipLaunchKernelGGL(k_build_bk<T>, dim3((nbk + 255) / 256), dim3(256), 0, s, V_k, L.d_src, (T*)B_k, L.n_key,
                     L.d_h);
  const size_t nbv = (size_t)L.H_kv * L.d_h * L.r_v;
  hipLaunchKernelGGL(k_build_bv<T>, dim3((unsigned)((nbv + 255) / 256)), dim3(256), 0, s, V_v, (T*)B_vt,
                     L.H_kv * L.d_h, L.r_v, L.n_v);
  return hipGetLastError();
}

hipError_t launch_build_factors(const Layer& L, const float* U_k, const float* V_k, const float* U_v,
                                const float* V_v, void* A_t, void* B_k, void* B_vt, hipStream_t s) {
  if (L.had) return build_factors_rot<uint16_t>(L, U_k, V_k, U_v, V_v, A_t, B_k, B_vt, s);
  if (L.dtype == STARKV_F32) return build_factors_t<float>(L, U_k, V_k, U_v, V_v, A_t, B_k, B_vt, s);
  return build_factors_t<uint16_t>(L, U_k, V_k, U_v, V_v, A_t, B_k, B_vt, s);
}

// Weight absorption of the key factors into the query projection (Methodology section 2: the
// reconstruction matrices move past the attention product, here into W_q): for query head h of
// KV head g = h / G (rank r_g, first key channel c0) and k < r_g,
//   wqk[G c0 + (h mod G) r_g + k][e] = sum_c W_q[e][h d_h + c] * B_k[c0 + k][c]
// summed in fp64 and kept in fp32 (no rounding to the layer dtype): as fp32 for fp32 layers, and
// for bf16 layers as a bf16 high part [rows][d] followed by a bf16 low part [rows][d] (the value
// minus the high part, rounded), the operands of the two bf16 MFMA passes of the projection.
// Grid (ceil(d / 256), H_q, largest rank); threads past d or the head's rank exit.
template <int DT>
__global__ __launch_bounds__(256) void k_absorb_query(const void* __restrict__ W_q, const void* __restrict__ B_k,
                                                      const int* __restrict__ koff, int G, int H_q, int d_h, int d,
                                                      int rows, float* __restrict__ wqk) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y, k = blockIdx.z;
  const int g = h / G, hh = h % G;
  const int c0 = koff[g], r = koff[g + 1] - c0;
  if (e >= d || k >= r) return;
  const size_t wrow = (size_t)e * H_q * d_h + (size_t)h * d_h;
  const size_t brow = (size_t)(c0 + k) * d_h;
  double acc = 0.0;
  for (int c = 0; c < d_h; ++c) {
    const float w = DT == STARKV_F32 ? ((const float*)W_q)[wrow + c] : bf16_to_f32(((const uint16_t*)W_q)[wrow + c]);
    const float bb = DT == STARKV_F32 ? ((const float*)B_k)[brow + c] : bf16_to_f32(((const uint16_t*)B_k)[brow + c]);
    acc += (double)w * (double)bb;
  }
  const size_t o = ((size_t)G * c0 + (size_t)hh * r + k) * d + e;
  const float v = (float)acc;
  if (DT == STARKV_F32) {
    wqk[o] = v;
  } else {
    const uint16_t hi = f32_to_bf16(v);
    uint16_t* w16 = (uint16_t*)wqk;
    w16[o] = hi;
    w16[(size_t)rows * d + o] = f32_to_bf16(v - bf16_to_f32(hi));
  }
}

hipError_t launch_absorb_query(const Layer& L, const void* W_q, float* wqk, hipStream_t s) {
  int rmax = 1;
  for (int g = 0; g < L.H_kv; ++g) rmax = std::max(rmax, L.rk[g]);
  const dim3 grid((L.d + 255) / 256, L.H_q, rmax);
  if (L.dtype == STARKV_F32)
    hipLaunchKernelGGL(k_absorb_query<STARKV_F32>, grid, dim3(256), 0, s, W_q, L.B_k, (const int*)L.d_koff, L.G,
                       L.H_q, L.d_h, L.d, L.G * L.n_key, wqk);
  else
    hipLaunchKernelGGL(k_absorb_query<STARKV_BF16>, grid, dim3(256), 0, s, W_q, L.B_k, (const int*)L.d_koff, L.G,
                       L.H_q, L.d_h, L.d, L.G * L.n_key, wqk);
  return hipGetLastError();
}

}  // namespace skv
