// Dense keys and values rebuilt from the latent cache (STAR-KV summary page, Problem
// Statement: reconstruction from the low-rank latent; Methodology section 2: keys per head
// K_g = x_g B_g, values jointly V = x_v B_v).  Off the decode path; one workgroup per token.
#include "device_common.h"
#include "starkv_internal.h"

namespace skv {

struct ReconArgs {
  const uint8_t* k_rows;
  const uint8_t* v_tiles;
  const void* B_k;   // [n_key][d_h]
  const void* B_vt;  // [H_kv*d_h][r_v]
  const uint16_t* scales;
  const int* koff;
  const int* n8;
  const int* off8;
  const int* off4;
  void* K_out;
  void* V_out;
  int b, t0, t1, T_max;
  int H_kv, d_h, n_key, r_v, n8v, K8, V8, k_row_bytes, v_rows, latent, dtype;
  int pack3, K4, V4;  // packed layout: outlier nibbles, then 3-bit planes from K4 / V4
};

template <int DT>
__device__ __forceinline__ float ld_dt(const void* p, size_t i) {
  if (DT == STARKV_F32) return ((const float*)p)[i];
  return bf16_to_f32(((const uint16_t*)p)[i]);
}

template <int DT>
__global__ __launch_bounds__(256) void k_reconstruct(ReconArgs a) {
  extern __shared__ float xs[];  // [n_key + r_v]
  const int t = a.t0 + blockIdx.x;
  const uint8_t* row = a.k_rows + ((size_t)a.b * a.T_max + t) * a.k_row_bytes;
  const int esz = a.latent == STARKV_LATENT_F32 ? 4 : (a.latent == STARKV_LATENT_BF16 ? 2 : 1);
  const int col = t % kTT;
  // this token's element of value-tile row vr
  auto vcell = [&](int vr) {
    return a.v_tiles + vblock_off(a.b, vr >> 5, t / kTT, a.v_rows, a.T_max, esz) + (size_t)((vr & 31) * kTT + col) * esz;
  };
  // dequantised latent of this token into LDS
  for (int c = threadIdx.x; c < a.n_key + a.r_v; c += blockDim.x) {
    float x;
    if (a.latent == STARKV_LATENT_MIX84) {
      int code;
      if (c < a.n_key) {
        const int g = find_segment(a.koff, a.H_kv, c);
        const int k = c - a.koff[g];
        if (a.pack3) {
          if (k < a.n8[g]) {
            const int u = a.off8[g] + k;
            code = snib(row[u / 2], u & 1);
          } else {
            code = key_code3(row, a.K4, a.off4[g] + (k - a.n8[g]));
          }
        } else if (k < a.n8[g]) {
          code = (int)(int8_t)row[a.off8[g] + k];
        } else {
          const int u = a.off4[g] + (k - a.n8[g]);
          code = snib(row[a.K8 + u / 2], u & 1);
        }
      } else {
        const int k = c - a.n_key;
        if (a.pack3) {
          code = k < a.n8v ? snib(*vcell(k / 2), k & 1) : val_code3(a.v_tiles, a.b, t, k - a.n8v, a.V4, a.v_rows, a.T_max);
        } else if (k < a.n8v) {
          code = (int)(int8_t)*vcell(k);
        } else {
          const int w = k - a.n8v;
          code = snib(*vcell(a.V8 + w / 2), w & 1);
        }
      }
      x = (float)code * f16_to_f32(a.scales[c]);
    } else if (a.latent == STARKV_LATENT_F32) {
      x = (c < a.n_key) ? ((const float*)row)[c] : *(const float*)vcell(c - a.n_key);
    } else {
      x = (c < a.n_key) ? bf16_to_f32(((const uint16_t*)row)[c])
                        : bf16_to_f32(*(const uint16_t*)vcell(c - a.n_key));
    }
    xs[c] = x;
  }
  __syncthreads();
  const int nout = a.H_kv * a.d_h;
  const size_t obase = (size_t)blockIdx.x * nout;
  for (int o = threadIdx.x; o < nout; o += blockDim.x) {
    const int g = o / a.d_h, e = o % a.d_h;
    float k = 0.f;
    for (int c = a.koff[g]; c < a.koff[g + 1]; ++c) k = fmaf(xs[c], ld_dt<DT>(a.B_k, (size_t)c * a.d_h + e), k);
    float v = 0.f;
    const size_t brow = (size_t)o * a.r_v;
    for (int c = 0; c < a.r_v; ++c) v = fmaf(xs[a.n_key + c], ld_dt<DT>(a.B_vt, brow + c), v);
    if (DT == STARKV_F32) {
      ((float*)a.K_out)[obase + o] = k;
      ((float*)a.V_out)[obase + o] = v;
    } else {
      ((uint16_t*)a.K_out)[obase + o] = f32_to_bf16(k);
      ((uint16_t*)a.V_out)[obase + o] = f32_to_bf16(v);
    }
  }
}

hipError_t launch_reconstruct(const Layer& L, const starkv_cache& c, int b, int t0, int t1, void* K_out,
                              void* V_out, hipStream_t s) {
  ReconArgs a = {};
  a.k_rows = (const uint8_t*)c.k_rows;
  a.v_tiles = (const uint8_t*)c.v_tiles;
  a.B_k = L.B_k;
  a.B_vt = L.B_vt;
  a.scales = L.scales;
  a.koff = L.d_koff;
  a.n8 = L.d_n8;
  a.off8 = L.d_off8;
  a.off4 = L.d_off4;
  a.K_out = K_out;
  a.V_out = V_out;
  a.b = b;
  a.t0 = t0;
  a.t1 = t1;
  a.T_max = c.T_max;
  a.H_kv = L.H_kv;
  a.d_h = L.d_h;
  a.n_key = L.n_key;
  a.r_v = L.r_v;
  a.n8v = L.n8v;
  a.K8 = L.K8;
  a.pack3 = L.pack3;
  a.K4 = L.K4;
  a.V4 = L.V4;
  a.V8 = L.V8;
  a.k_row_bytes = L.k_row_bytes;
  a.v_rows = L.v_rows;
  a.latent = L.latent;
  a.dtype = L.dtype;
  const size_t lds = (size_t)(L.n_lat) * sizeof(float);
  if (L.dtype == STARKV_F32)
    hipLaunchKernelGGL(k_reconstruct<STARKV_F32>, dim3(t1 - t0), dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL(k_reconstruct<STARKV_BF16>, dim3(t1 - t0), dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace skv
