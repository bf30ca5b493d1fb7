// Attention over keys and values reconstructed from the latent cache, for query chunks of any
// length (prefill, chunked prefill) and for layers whose keys carry a rotary position embedding.
//
// STAR-KV summary page, Problem Statement: the cache holds the projected hidden states, and
// rebuilding K and V from them costs compute; Methodology section 2: keys are factored head by
// head (K_g = L_g B_g), values jointly (V = C_v B_v).  The latent-space order used by decode moves
// B_g and B_v past the attention weights, which pays when a few queries meet many tokens; a chunk
// of n_q queries does 2 n_q T r_v value work in the latent space against 2 T r_v d_h H_kv to
// rebuild V once plus 2 n_q T d_h per head to attend, so long chunks rebuild K and V first.  A
// position-dependent rotation of the keys does not commute with B_g at all: a rotary layer always
// takes this path.
//
//   1. k_deq_latent  the dequantised latent of every cached token, token-major: key channels
//                    in fp32, xk[t][c] = code * scale_c (or the stored bf16 / fp32 latent); value
//                    channels as bf16 high and low parts of the same fp32 value, xv_hi[t][c] and
//                    xv_lo[t][c], rows padded with zeros to a multiple of 64 channels; int8/int4
//                    layers (r_v a multiple of 8) store the value codes themselves, exact in f16,
//                    in xv_hi, and k_scale_bv folds the scales into an f16 copy of B_v^T
//   2. k_recon       K^_g = xk_g B_g per KV head on MFMA (fp32 latent split into bf16 high and low
//                    parts), the rotation of the keys at their positions in the epilogue;
//      k_recon_v     V^ = (xv_hi + xv_lo) B_v for all heads at once (int8/int4: codes times the
//                    scaled B_v, one f16 MFMA instead of two bf16 ones), a GEMM whose operand tiles
//                    stream through LDS; stored as f16, K^ token-major and V^ transposed (dims x
//                    tokens)
//   3. k_flash       causal attention of the query chunk over K^, V^: 32-token key tiles with an
//                    online softmax (base 2), S^T = K^ Q^T and O^T = V^T P^T on f16 MFMA so that a
//                    row's softmax state lives in one lane
//
// Tokens of every sequence are laid out back to back, each sequence padded to a multiple of 32.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "device_common.h"
#include "profile.h"
#include "starkv_internal.h"

namespace skv {

namespace {

constexpr int kRT = 32;  // token tile of every prefill kernel

int ceil_div(int a, int b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// sequence whose padded token range holds token t (bases ascending, base[0] = 0)
__device__ __forceinline__ int seq_of_token(const int* base, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (base[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// sin and cos of a rotation angle given in fp64 (positions reach 2^15 and more, where an fp32
// angle would already be off by ~2^-9 rad): reduced to [-pi, pi] in fp64, then sincosf
__device__ __forceinline__ void rot_sincos(double ang, float* sn, float* cs) {
  constexpr double kTwoPi = 6.283185307179586476925287;
  const double red = ang - kTwoPi * rint(ang / kTwoPi);
  sincosf((float)red, sn, cs);
}

struct SeqBases {
  int B;
  int lens[kMaxB];
  int base[kMaxB + 1];  // first padded token of each sequence; base[B] = total
};

// ---------------------------------------------------------------------------------------------
// 1. dequantised latent, token-major

struct DeqArgs {
  const uint8_t* k_rows;
  const uint8_t* v_tiles;
  const uint16_t* scales;
  const int* src;  // [n_lat] (head << 16) | index within the head; head = H_kv for value channels
  HeadTables heads;
  float* xk;       // [total][n_key] (int8/int4 layers: f16 codes, [total][n_key] halves)
  uint16_t* xv_hi;  // [total][rvp]
  uint16_t* xv_lo;  // [total][rvp]
  int n_lat, n_key, r_v, rvp, H_kv, K8, V8, n8v, k_row_bytes, v_rows, T_max;
  int pack3, K4, V4;  // packed layout: outlier nibbles, then 3-bit planes from K4 / V4
  int codes;          // int8/int4 values: the codes, in f16, into xv_hi (xv_lo unused)
  SeqBases sb;
};

// Workgroup = one 32-token tile of one sequence; thread items walk (token, channel) with the
// channel fastest, so the stores are contiguous.  Tokens past the length get 0.
// CODE (int8/int4): the code alone, without its scale
template <int LAT, bool CODE = false>
__device__ __forceinline__ float deq_key(const DeqArgs& a, int b, int t, int c) {
  const uint8_t* row = a.k_rows + ((size_t)b * a.T_max + t) * a.k_row_bytes;
  if (LAT == STARKV_LATENT_MIX84) {
    const int s = a.src[c];
    const int g = s >> 16, k = s & 0xFFFF;
    const int n8 = a.heads.n8[g];
    int code;
    if (a.pack3) {
      if (k < n8) {
        const int u = a.heads.off8[g] + k;
        code = snib(row[u >> 1], u & 1);
      } else {
        code = key_code3(row, a.K4, a.heads.off4[g] + (k - n8));
      }
    } else if (k < n8) {
      code = (int)(int8_t)row[a.heads.off8[g] + k];
    } else {
      const int u = a.heads.off4[g] + (k - n8);
      const int byte = row[a.K8 + (u >> 1)];
      code = ((int)(((u & 1) ? byte >> 4 : byte) & 0xF) ^ 8) - 8;  // signed nibble
    }
    return CODE ? (float)code : (float)code * f16_to_f32(a.scales[c]);
  } else if (LAT == STARKV_LATENT_BF16) {
    return bf16_to_f32(((const uint16_t*)row)[c]);
  } else {
    return ((const float*)row)[c];
  }
}
// CODE (int8/int4): the code alone, without its scale
template <int LAT, bool CODE = false>
__device__ __forceinline__ float deq_value(const DeqArgs& a, int b, int t, int cv) {
  const int c = a.n_key + cv;
  if (LAT == STARKV_LATENT_MIX84 && a.pack3) {
    int code;
    if (cv < a.n8v) {
      const int byte = a.v_tiles[vblock_off(b, (cv >> 1) >> 5, t / kTT, a.v_rows, a.T_max, 1) +
                                 ((cv >> 1) & 31) * kTT + t % kTT];
      code = snib(byte, cv & 1);
    } else {
      code = val_code3(a.v_tiles, b, t, cv - a.n8v, a.V4, a.v_rows, a.T_max);
    }
    return CODE ? (float)code : (float)code * f16_to_f32(a.scales[c]);
  } else if (LAT == STARKV_LATENT_MIX84) {
    const bool i4 = cv >= a.n8v;
    const int w = cv - a.n8v;
    const int vr = i4 ? a.V8 + (w >> 1) : cv;
    const int byte = a.v_tiles[vblock_off(b, vr >> 5, t / kTT, a.v_rows, a.T_max, 1) + (vr & 31) * kTT + t % kTT];
    const int code = i4 ? ((int)(((w & 1) ? byte >> 4 : byte) & 0xF) ^ 8) - 8 : (int)(int8_t)byte;
    return CODE ? (float)code : (float)code * f16_to_f32(a.scales[c]);
  } else if (LAT == STARKV_LATENT_BF16) {
    const uint16_t* blk = (const uint16_t*)(a.v_tiles + vblock_off(b, cv >> 5, t / kTT, a.v_rows, a.T_max, 2));
    return bf16_to_f32(blk[(cv & 31) * kTT + t % kTT]);
  } else {
    const float* blk = (const float*)(a.v_tiles + vblock_off(b, cv >> 5, t / kTT, a.v_rows, a.T_max, 4));
    return blk[(cv & 31) * kTT + t % kTT];
  }
}
template <int LAT>
__global__ __launch_bounds__(256) void k_deq_latent(DeqArgs a) {
  const int tok0 = blockIdx.x * kRT;
  const int b = seq_of_token(a.sb.base, a.sb.B, tok0);
  const int t0 = tok0 - a.sb.base[b], len = a.sb.lens[b];
  // no branch around the loads (tokens of the tile past the length are still cache rows below
  // T_max; their values are replaced by 0 after the load), so unrolled iterations overlap
  if (LAT == STARKV_LATENT_MIX84) {
    // int8/int4 keys: the codes themselves, exact in f16 (k_recon folds the scales into B_g)
#pragma unroll 4
    for (int idx = threadIdx.x; idx < kRT * a.n_key; idx += 256) {
      const int tl = idx / a.n_key, c = idx % a.n_key;
      const int t = t0 + tl;
      const float x = deq_key<LAT, true>(a, b, t, c);
      ((uint16_t*)a.xk)[(size_t)(tok0 + tl) * a.n_key + c] = f32_to_f16(t < len ? x : 0.f);
    }
  } else {
#pragma unroll 4
    for (int idx = threadIdx.x; idx < kRT * a.n_key; idx += 256) {
      const int tl = idx / a.n_key, c = idx % a.n_key;
      const int t = t0 + tl;
      const float x = deq_key<LAT>(a, b, t, c);
      a.xk[(size_t)(tok0 + tl) * a.n_key + c] = t < len ? x : 0.f;
    }
  }
  // value channels in pairs: one 32-bit store of each part per pair
  const int np = a.rvp / 2;
  if (LAT == STARKV_LATENT_MIX84 && a.codes) {
#pragma unroll 4
    for (int idx = threadIdx.x; idx < kRT * np; idx += 256) {
      const int tl = idx / np, cv = 2 * (idx % np);
      const int t = t0 + tl;
      float x0 = deq_value<LAT, true>(a, b, t, min(cv, a.r_v - 1));
      float x1 = deq_value<LAT, true>(a, b, t, min(cv + 1, a.r_v - 1));
      x0 = t < len && cv < a.r_v ? x0 : 0.f;
      x1 = t < len && cv + 1 < a.r_v ? x1 : 0.f;
      *(uint32_t*)(a.xv_hi + (size_t)(tok0 + tl) * a.rvp + cv) =
          (uint32_t)f32_to_f16(x0) | ((uint32_t)f32_to_f16(x1) << 16);
    }
    return;
  }
#pragma unroll 4
  for (int idx = threadIdx.x; idx < kRT * np; idx += 256) {
    const int tl = idx / np, cv = 2 * (idx % np);
    const int t = t0 + tl;
    float x0 = deq_value<LAT>(a, b, t, min(cv, a.r_v - 1));
    float x1 = deq_value<LAT>(a, b, t, min(cv + 1, a.r_v - 1));
    x0 = t < len && cv < a.r_v ? x0 : 0.f;
    x1 = t < len && cv + 1 < a.r_v ? x1 : 0.f;
    const uint16_t h0 = f32_to_bf16(x0), h1 = f32_to_bf16(x1);
    const uint16_t l0 = f32_to_bf16(x0 - bf16_to_f32(h0)), l1 = f32_to_bf16(x1 - bf16_to_f32(h1));
    const size_t o = (size_t)(tok0 + tl) * a.rvp + cv;
    *(uint32_t*)(a.xv_hi + o) = (uint32_t)h0 | ((uint32_t)h1 << 16);
    *(uint32_t*)(a.xv_lo + o) = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
}

// ---------------------------------------------------------------------------------------------
// 2. reconstruction of K^ and V^ per KV head (bf16 factors)

struct ReconArgs {
  const float* xk;       // [total][n_key] (KC: f16 codes)
  const uint16_t* kscales;  // KC: the key channels' f16 scales
  const uint16_t* xv_hi;  // [total][rvp]
  const uint16_t* xv_lo;
  const uint16_t* B_k;   // [n_key][d_h]
  const uint16_t* B_vt;  // [H_kv d_h][r_v]
  const int* koff;       // [H_kv + 1]
  _Float16* kh;          // [total][H_kv][d_h]
  _Float16* vt;          // [H_kv d_h][total], tokens of each 16-group in swapped-middle order
  int n_lat, n_key, r_v, rvp, H_kv, d_h, total, rpad;
  float rope_theta;
  int rotary_dim;
  SeqBases sb;
};

// position of token t in the transposed value store: within each group of 16, tokens 4..7 and
// 8..11 trade places, so that lane half q of the attention's value operand reads 8 consecutive
// entries holding exactly the tokens its probability operand holds
__device__ __forceinline__ int vt_slot(int t) {
  const int u = t & 15;
  return (t & ~15) | (u & 3) | ((u & 4) << 1) | ((u & 8) >> 1);
}

// Workgroup = (128 tokens, KV head g, keys or values), four waves of 32 tokens x all d_h columns
// (NT = d_h / 32 column tiles of 32x32x16 bf16 MFMA).  The latent row of a token is split into
// bf16 high and low parts (two MFMAs), so the product is as accurate as fp32 x bf16.  KC
// (int8/int4 keys): the latent holds the codes in f16 and the staged B_g rows are scaled by their
// channel's scale and rounded to f16, one f16 MFMA per K-step.  Keys read
// B_g transposed from LDS (staged by the workgroup); values (only when r_v is not a multiple of 8:
// otherwise k_recon_v) read B_v^T rows directly and the latent's parts as stored.  Rotary keys
// (over the whole head dimension): the pair (e, e + d_h / 2) is rotated by
// position * theta^(-2 e / d_h), the angle formed and reduced in fp64.
template <int NT, bool VEC, int KIND, bool ROPE, bool KC = false>
__global__ __launch_bounds__(256) void k_recon(ReconArgs a) {
  extern __shared__ uint16_t bkt[];  // keys: B_g^T [d_h][rpad]
  __shared__ double inv_freq[128];    // rotary keys: theta^(-2 e / d_h), e < d_h / 2
  constexpr int kind = KIND;
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int r = lane & 31, q = lane >> 5;
  const int c_lo = kind == 0 ? a.koff[g] : a.n_key;
  const int rk = kind == 0 ? a.koff[g + 1] - c_lo : a.r_v;
  if (kind == 0) {
    // 16-byte pieces of B_g's rows (8 dims of channel k), four per thread in flight at once,
    // stored transposed; channels past the head's rank are zero
    constexpr int DH = 32 * NT;
    const int n16 = a.rpad * (DH / 8);
    for (int i0 = threadIdx.x; i0 < n16; i0 += 1024) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + 256 * u;
        const int k = i % a.rpad, e8 = i / a.rpad;
        v[u] = ld16(a.B_k + (size_t)min(c_lo + k, a.n_key - 1) * DH + 8 * min(e8, DH / 8 - 1));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + 256 * u;
        const int k = i % a.rpad, e8 = i / a.rpad;
        if (i < n16) {
          const float ks = KC && k < rk ? f16_to_f32(a.kscales[c_lo + k]) : 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint16_t bb = (uint16_t)(v[u][j >> 1] >> (16 * (j & 1)));
            bkt[(8 * e8 + j) * a.rpad + k] = k < rk ? (KC ? f32_to_f16(bf16_to_f32(bb) * ks) : bb) : (uint16_t)0;
          }
        }
      }
    }
    if (ROPE && (int)threadIdx.x < a.d_h / 2)
      inv_freq[threadIdx.x] = exp2(-2.0 * (double)threadIdx.x / (double)a.d_h * log2((double)a.rope_theta));
    __syncthreads();
  }
  const int tw = blockIdx.x * 128 + wave * 32;  // first token of this wave
  if (tw >= a.total) return;  // wave-uniform, after the only barrier
  const int tok = tw + r;     // this lane's A-operand token
  f32x16 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[nt][v] = 0.f;
  const float* xr = a.xk + (size_t)tok * a.n_key + c_lo;
  const uint16_t* xr16 = (const uint16_t*)a.xk + (size_t)tok * a.n_key + c_lo;
  for (int k0 = 0; k0 < rk; k0 += 16) {
    const int kb = k0 + 8 * q;
    bf16x8 ah, al;
    if (KC) {
      // f16 codes (channels past the head's rank: 0)
      uint32_t hw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t c0 = kb + 2 * i < rk ? xr16[kb + 2 * i] : 0u;
        const uint32_t c1 = kb + 2 * i + 1 < rk ? xr16[kb + 2 * i + 1] : 0u;
        hw[i] = c0 | (c1 << 16);
      }
      ah = as_bf16x8(u32x4{hw[0], hw[1], hw[2], hw[3]});  // (f16 bits; the MFMA reads them as f16)
      al = ah;
    } else if (kind == 0) {
      float xv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[i] = kb + i < rk ? xr[kb + i] : 0.f;
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t h0 = f32_to_bf16(xv[2 * i]), h1 = f32_to_bf16(xv[2 * i + 1]);
        const uint16_t l0 = f32_to_bf16(xv[2 * i] - bf16_to_f32(h0)), l1 = f32_to_bf16(xv[2 * i + 1] - bf16_to_f32(h1));
        hw[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lw[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
      ah = as_bf16x8(u32x4{hw[0], hw[1], hw[2], hw[3]});
      al = as_bf16x8(u32x4{lw[0], lw[1], lw[2], lw[3]});
    } else {
      // the stored parts (channels past r_v are zero up to rvp, a multiple of 64)
      ah = as_bf16x8(ld16(a.xv_hi + (size_t)tok * a.rvp + kb));
      al = as_bf16x8(ld16(a.xv_lo + (size_t)tok * a.rvp + kb));
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int e = nt * 32 + r;
      u32x4 bw;
      if (kind == 0) {
        bw = *(const u32x4*)(bkt + e * a.rpad + kb);
      } else if (VEC) {
        bw = kb < rk ? ld16(a.B_vt + (size_t)(g * a.d_h + e) * a.r_v + kb) : u32x4{0, 0, 0, 0};
      } else {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = kb + 2 * i;
          const uint32_t lo = k < rk ? a.B_vt[(size_t)(g * a.d_h + e) * a.r_v + k] : 0u;
          const uint32_t hi = k + 1 < rk ? a.B_vt[(size_t)(g * a.d_h + e) * a.r_v + k + 1] : 0u;
          w[i] = lo | (hi << 16);
        }
        bw = u32x4{w[0], w[1], w[2], w[3]};
      }
      if (kind == 0) {
        // keys: K^T tiles (rows = head dims, columns = tokens), so that a lane holds runs of 4
        // consecutive dims of one token for the token-major store
        if (KC) {
          acc[nt] = mfma32_f16(as_f16x8(bw), __builtin_bit_cast(f16x8, ah), acc[nt]);
        } else {
          acc[nt] = mfma32_bf16(as_bf16x8(bw), ah, acc[nt]);
          acc[nt] = mfma32_bf16(as_bf16x8(bw), al, acc[nt]);
        }
      } else {
        acc[nt] = mfma32_bf16(ah, as_bf16x8(bw), acc[nt]);
        acc[nt] = mfma32_bf16(al, as_bf16x8(bw), acc[nt]);
      }
    }
  }
  const int b = seq_of_token(a.sb.base, a.sb.B, tw);
  const int base = a.sb.base[b], len = a.sb.lens[b];
  // every token of the padded range is stored: padding tokens (past the length) hold zeros, so
  // the attention's masked products never meet uninitialised memory
  if (kind == 0) {
    // lane holds token tok, dims 32 nt + d32_row(v, q)
    const int t = tok - base;  // position in the sequence
    if (ROPE) {
      // rotary keys over the whole head dimension: pairs (e, e + d_h / 2) in tiles nt and
      // nt + NT / 2 of the same lane
#pragma unroll
      for (int nt = 0; nt < NT / 2; ++nt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float sn, cs;
          rot_sincos((double)t * inv_freq[nt * 32 + d32_row(v, q)], &sn, &cs);
          const float x0 = acc[nt][v], x1 = acc[nt + NT / 2][v];
          acc[nt][v] = x0 * cs - x1 * sn;
          acc[nt + NT / 2][v] = x0 * sn + x1 * cs;
        }
    }
    _Float16* kr = a.kh + ((size_t)tok * a.H_kv + g) * a.d_h;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        uint32_t w[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const _Float16 x0 = t < len ? (_Float16)acc[nt][4 * v4 + 2 * i] : (_Float16)0.f;
          const _Float16 x1 = t < len ? (_Float16)acc[nt][4 * v4 + 2 * i + 1] : (_Float16)0.f;
          w[i] = (uint32_t)__builtin_bit_cast(uint16_t, x0) | ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16);
        }
        st8(kr + nt * 32 + 8 * v4 + 4 * q, u32x2{w[0], w[1]});
      }
  } else {
    // lane holds column e = 32 nt + r of tokens tw + d32_row(v, q)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int e = nt * 32 + r;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tf = tw + d32_row(v, q);
        const _Float16 x = tf - base < len ? (_Float16)acc[nt][v] : (_Float16)0.f;
        a.vt[(size_t)(g * a.d_h + e) * a.total + vt_slot(tf)] = x;
      }
    }
  }
}

// V^ for all KV heads as one GEMM, C[m][n] = sum_k (xv_hi + xv_lo)[m][k] B_vt[n][k] (m = token of
// the padded token range, n = g d_h + e, k < r_v; r_v a multiple of 8), stored transposed in f16.
// Workgroup tile TM tokens x TN columns, four waves in 2 x 2 quadrants of (TM / 2) x (TN / 2) over
// the whole K, each quadrant in 32 x 32 MFMA tiles.  K advances in blocks of 64: the block's
// three operand tiles (latent high part, low part, B_vt rows; 128 bytes per row) arrive by
// 16-byte LDS DMA into a ring of NST stages, NST - 1 blocks ahead of the MFMAs; in a tile, row
// R's eight 16-byte K-chunks sit at chunk c ^ ((R >> 1) & 7), so the 16 lanes of a fragment read
// hit 16 different 4-bank groups.  A 128 x 128 tile reads each operand byte half as often as a
// 64 x 64 one: the kernel is bound by the bytes each CU pulls from L2.  B_vt is read through a
// buffer resource: its K-chunks past r_v read the next row (or zeros past the end), which meet
// zero latent parts (rows padded to rvp).  Tokens past total repeat the last token and are not
// stored.
struct ReconVArgs {
  const uint16_t* xv_hi;  // [total][rvp]
  const uint16_t* xv_lo;
  const uint16_t* B_vt;   // [N][r_v]
  _Float16* vt;           // [N][total]
  int rvp, r_v, N, total;
  SeqBases sb;
};

// CODES: xv_hi holds f16 value codes and B_vt the f16 scaled factors (k_scale_bv): one f16 MFMA
// per K-step and no low part.
template <int TM, int TN, int NST, bool CODES = false>
__global__ __launch_bounds__(256) void k_recon_v(ReconVArgs a) {
  constexpr int XB = TM * 128, WB = TN * 128;  // bytes of the operand tiles of a K block
  constexpr int SB = (CODES ? 1 : 2) * XB + WB;  // bytes of a stage
  constexpr int LX = TM / 32, LW = TN / 32;    // 16-byte loads per wave per X / W tile
  constexpr int MT = TM / 64, NTT = TN / 64;   // 32 x 32 tiles per wave, rows and columns
  extern __shared__ __align__(16) uint8_t ring_raw[];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int r = lane & 31, q = lane >> 5;
  const int mb = blockIdx.x * TM, nb = blockIdx.y * TN;
  const __amdgpu_buffer_rsrc_t wrs = buf_rsrc(a.B_vt, (uint32_t)a.N * (uint32_t)a.r_v * 2u);
  // this lane's DMA sources: load jj of the wave fills tile slot i = 64 (L wave + jj) + lane,
  // i.e. row i / 8 and stored chunk i % 8, which holds K-chunk (i % 8) ^ ((row >> 1) & 7)
  size_t xoff[LX];
  uint32_t woff[LW];
#pragma unroll
  for (int jj = 0; jj < LX; ++jj) {
    const int i = 64 * (LX * wave + jj) + lane;
    const int row = i >> 3;
    const int kc = (i & 7) ^ ((row >> 1) & 7);
    xoff[jj] = (size_t)min(mb + row, a.total - 1) * a.rvp + 8 * kc;
  }
#pragma unroll
  for (int jj = 0; jj < LW; ++jj) {
    const int i = 64 * (LW * wave + jj) + lane;
    const int row = i >> 3;
    const int kc = (i & 7) ^ ((row >> 1) & 7);
    woff[jj] = (uint32_t)(nb + row) * (uint32_t)a.r_v * 2u + 16u * (uint32_t)kc;
  }
  const int nkb = a.rvp / 64;
  const uint32_t ring0 = lds_addr(ring_raw);
  auto issue = [&](int kb, int st) {
    kb = min(kb, nkb - 1);  // past the end: reload the last block (never read)
    const uint32_t hb = ring0 + st * SB, lb = hb + XB, wb = CODES ? lb : lb + XB;
#pragma unroll
    for (int jj = 0; jj < LX; ++jj) {
      const uint32_t slot = 1024 * (LX * wave + jj);
      lds_dma16(a.xv_hi + xoff[jj] + 64 * kb, hb + slot);
      if (!CODES) lds_dma16(a.xv_lo + xoff[jj] + 64 * kb, lb + slot);
    }
#pragma unroll
    for (int jj = 0; jj < LW; ++jj)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wrs, (__attribute__((address_space(3))) void*)(uintptr_t)(wb + 1024 * (LW * wave + jj)), 16,
          (int)(woff[jj] + 128u * (uint32_t)kb), 0, 0, 0);
  };
  const int wm = wave & 1, wn = wave >> 1;
  int xo[MT], xsw[MT], wo[NTT], wsw[NTT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int row = (TM / 2) * wm + 32 * i + r;
    xo[i] = row * 128;
    xsw[i] = (row >> 1) & 7;
  }
#pragma unroll
  for (int j = 0; j < NTT; ++j) {
    const int row = (TN / 2) * wn + 32 * j + r;
    wo[j] = row * 128;
    wsw[j] = (row >> 1) & 7;
  }
  f32x16 acc[MT][NTT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
#pragma unroll
  for (int u = 0; u < NST - 1; ++u) issue(u, u);
  for (int kb = 0; kb < nkb; ++kb) {
    vm_wait<((CODES ? 1 : 2) * LX + LW) * (NST - 2)>();  // this wave's loads of block kb are in
    __builtin_amdgcn_s_barrier();            // ... and every wave's; block kb - 1's stage is free
    asm volatile("" ::: "memory");
    issue(kb + NST - 1, (kb + NST - 1) % NST);
    const uint8_t* ht = ring_raw + (kb % NST) * SB;
    const uint8_t* lt = ht + XB;
    const uint8_t* wt = CODES ? lt : lt + XB;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = 2 * ks + q;
      u32x4 xh[MT], xl[MT], wf[NTT];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        xh[i] = *(const u32x4*)(ht + xo[i] + 16 * (c ^ xsw[i]));
        if (!CODES) xl[i] = *(const u32x4*)(lt + xo[i] + 16 * (c ^ xsw[i]));
      }
#pragma unroll
      for (int j = 0; j < NTT; ++j) wf[j] = *(const u32x4*)(wt + wo[j] + 16 * (c ^ wsw[j]));
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTT; ++j) {
          if (CODES) {
            acc[i][j] = mfma32_f16(as_f16x8(xh[i]), as_f16x8(wf[j]), acc[i][j]);
          } else {
            acc[i][j] = mfma32_bf16(as_bf16x8(xh[i]), as_bf16x8(wf[j]), acc[i][j]);
            acc[i][j] = mfma32_bf16(as_bf16x8(xl[i]), as_bf16x8(wf[j]), acc[i][j]);
          }
        }
    }
  }
  vm_wait<0>();  // the trailing reloads land before the workgroup ends
  // lane holds column n of tokens m0 + d32_row(v, q); run h (v = 8 h .. 8 h + 7) covers tokens
  // 16 h + 4 q + {0..3} and 16 h + 8 + 4 q + {0..3}, which the transposed store keeps at the
  // 8 consecutive slots 16 h + 8 q .. + 7 (see vt_slot)
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m0 = mb + (TM / 2) * wm + 32 * i;
    if (m0 >= a.total) continue;
    const int b = seq_of_token(a.sb.base, a.sb.B, m0);  // a 32-token tile lies in one sequence
    const int tl = m0 - a.sb.base[b], len = a.sb.lens[b];
#pragma unroll
    for (int j = 0; j < NTT; ++j) {
      const int n = nb + (TN / 2) * wn + 32 * j + r;
      if (n >= a.N) continue;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int t0 = tl + d32_row(8 * h + e, q), t1 = tl + d32_row(8 * h + e + 1, q);
          const _Float16 x0 = t0 < len ? (_Float16)acc[i][j][8 * h + e] : (_Float16)0.f;
          const _Float16 x1 = t1 < len ? (_Float16)acc[i][j][8 * h + e + 1] : (_Float16)0.f;
          w[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, x0) | ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16);
        }
        st16(a.vt + (size_t)n * a.total + m0 + 16 * h + 8 * q, u32x4{w[0], w[1], w[2], w[3]});
      }
    }
  }
}

// B_v^T with the value scales folded in, for the code operand of k_recon_v:
// out[n][k] = f16(scale_(n_key + k) * B_vt[n][k]) for n < N, k < r_v (2 elements per thread).
__global__ __launch_bounds__(256) void k_scale_bv(const uint16_t* B_vt, const uint16_t* vscales, int N, int r_v,
                                                  uint16_t* out) {
  const size_t i = 2 * ((size_t)blockIdx.x * 256 + threadIdx.x);
  if (i >= (size_t)N * r_v) return;  // r_v is even (a multiple of 8): pairs stay in one row
  const int k = (int)(i % r_v);
  const uint32_t bv = *(const uint32_t*)(B_vt + i);
  const float x0 = bf16_to_f32((uint16_t)(bv & 0xFFFF)) * f16_to_f32(vscales[k]);
  const float x1 = bf16_to_f32((uint16_t)(bv >> 16)) * f16_to_f32(vscales[k + 1]);
  *(uint32_t*)(out + i) = (uint32_t)f32_to_f16(x0) | ((uint32_t)f32_to_f16(x1) << 16);
}

// ---------------------------------------------------------------------------------------------
// 3. causal attention over the reconstructed keys and values

struct FlashArgs {
  const void* q;  // [B][n_q][H_q][d_h] (dtype)
  void* out;      // same shape and dtype
  const _Float16* kh;
  const _Float16* vt;
  int n_q, H_q, H_kv, G, d_h, total;
  float qscale;  // log2(e) / sqrt(d_h)
  float rope_theta;
  int rotary_dim;
  SeqBases sb;
};

// Workgroup = (128 queries of one head, sequence), four waves of 32 queries.  Query j (position
// len - n_q + j) sees tokens <= its position.  Per 32-token key tile: S^T = K^ Q^T (lane = query
// row, 16 tokens), masked and scaled to base 2, an online softmax whose row maximum and sum stay
// in the lane (the two lane halves hold different tokens of the same rows and agree on the
// maximum through one exchange), then O^T += V^T P^T with the probabilities as the B operand
// straight from the S^T registers (the value store's token order matches them).
// STAGE (d_h = 64, 128, 256): the four waves share each key tile's K^ rows and V^T rows, which
// arrive by 16-byte LDS DMA in a ring of kFlashStages stages, two tiles ahead; every wave walks
// the workgroup's key tiles (tiles past a wave's own queries are fully masked).  In a stage, K^
// row t keeps its 16-byte dim chunk c at c ^ fk(t) and V^T row e its token chunk c at
// c ^ ((e >> 2) & 3), so the 16 lanes of a fragment read hit 16 different 4-bank groups.
// Otherwise each wave reads its tiles from memory itself, with no barrier.
constexpr int kFlashStages = 3;

template <int NT, int DT, bool STAGE>
__global__ __launch_bounds__(256) void k_flash(FlashArgs a) {
  constexpr int KS = NT * 2;  // 16-dim K-steps of the scores
  constexpr int DH = 32 * NT;
  constexpr int CPR = DH / 8;                                 // 16-byte chunks of a K^ row
  constexpr int FSH = CPR >= 16 ? 0 : (CPR == 8 ? 1 : 2);     // K^ chunk swizzle: row >> FSH ...
  constexpr int FMK = (CPR >= 16 ? 16 : CPR) - 1;             // ... masked
  constexpr int TBY = kRT * DH * 2;                           // bytes of a K^ tile and of a V^T tile
  constexpr int LPH = STAGE ? NT / 2 : 1;                     // DMA loads per wave per tile half
  extern __shared__ __align__(16) uint8_t fring[];
  const int h = blockIdx.y, b = blockIdx.z, g = h / a.G;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int r = lane & 31, q = lane >> 5;
  const int jw = blockIdx.x * 128 + wave * 32;  // first query of this wave
  if (!STAGE && jw >= a.n_q) return;            // wave-uniform (the staged kernel has barriers)
  const int len = a.sb.lens[b], base = a.sb.base[b];
  const int j = min(jw + r, a.n_q - 1);         // this lane's query (rows past n_q repeat the last, not stored)
  const int pos = len - a.n_q + j;
  const int pos_max = len - a.n_q + min(jw + 31, a.n_q - 1);
  // query fragments: K-step ks holds dims 16 ks + 8 q .. + 7; the rotation pairs dims e and
  // e + d_h / 2, which sit in K-steps ks and ks + KS / 2 of the same lane
  f16x8 qh[KS];
  const size_t qoff = (((size_t)b * a.n_q + j) * a.H_q + h) * a.d_h;
  auto ldq = [&](int ks, float x[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const size_t e = (size_t)ks * 16 + 8 * q + i;
      x[i] = DT == STARKV_F32 ? ((const float*)a.q)[qoff + e] : bf16_to_f32(((const uint16_t*)a.q)[qoff + e]);
    }
  };
#pragma unroll
  for (int ks = 0; ks < KS / 2; ++ks) {
    float x0[8], x1[8];
    ldq(ks, x0);
    ldq(ks + KS / 2, x1);
    if (a.rope_theta > 0.f) {
      const double lt = log2((double)a.rope_theta);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = ks * 16 + 8 * q + i;
        float sn, cs;
        rot_sincos((double)pos * exp2(-2.0 * (double)e / (double)a.d_h * lt), &sn, &cs);
        const float y0 = x0[i] * cs - x1[i] * sn;
        const float y1 = x0[i] * sn + x1[i] * cs;
        x0[i] = y0;
        x1[i] = y1;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qh[ks][i] = (_Float16)x0[i];
      qh[ks + KS / 2][i] = (_Float16)x1[i];
    }
  }

  f32x16 acc[NT];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[mt][v] = 0.f;
  float m_run = -INFINITY, l = 0.f;
  const _Float16* krow = a.kh + ((size_t)(base + r) * a.H_kv + g) * a.d_h + 8 * q;
  const size_t kstep = (size_t)kRT * a.H_kv * a.d_h;  // key-tile stride
  // key tiles: this wave's own (unstaged), or the workgroup's (staged: its last query's)
  const int n_kt = STAGE ? (len - a.n_q + min((int)blockIdx.x * 128 + 127, a.n_q - 1)) / kRT + 1 : pos_max / kRT + 1;
  // staged: DMA sources of this lane (piece u of the wave: slot 64 (LPH wave + u) + lane)
  const _Float16* ksrc[LPH];
  const _Float16* vsrc[LPH];
  if (STAGE) {
#pragma unroll
    for (int u = 0; u < LPH; ++u) {
      const int sl = 64 * (LPH * wave + u) + lane;
      const int kr = sl / CPR, kc = (sl % CPR) ^ ((kr >> FSH) & FMK);
      ksrc[u] = a.kh + ((size_t)(base + kr) * a.H_kv + g) * DH + 8 * kc;
      const int vr = sl >> 2, vc = (sl & 3) ^ ((vr >> 2) & 3);
      vsrc[u] = a.vt + (size_t)(g * DH + vr) * a.total + base + 8 * vc;
    }
  }
  const uint32_t ring0 = lds_addr(fring);
  auto issue = [&](int kt, int st) {
    kt = min(kt, n_kt - 1);  // past the end: reload the last tile (never read)
    const uint32_t kb = ring0 + st * 2 * TBY, vb = kb + TBY;
#pragma unroll
    for (int u = 0; u < LPH; ++u) {
      lds_dma16(ksrc[u] + (size_t)kt * kstep, kb + 1024 * (LPH * wave + u));
      lds_dma16(vsrc[u] + kt * kRT, vb + 1024 * (LPH * wave + u));
    }
  };
  if (STAGE) {
#pragma unroll
    for (int u = 0; u < kFlashStages - 1; ++u) issue(u, u);
  }
  for (int kt = 0; kt < n_kt; ++kt) {
    const uint8_t* kst = fring + (kt % kFlashStages) * 2 * TBY;
    const uint8_t* vst = kst + TBY;
    if (STAGE) {
      vm_wait<2 * LPH * (kFlashStages - 2)>();  // this wave's loads of tile kt are in
      __builtin_amdgcn_s_barrier();             // ... and every wave's; tile kt - 1's stage is free
      asm volatile("" ::: "memory");
      issue(kt + kFlashStages - 1, (kt + kFlashStages - 1) % kFlashStages);
    }
    // S^T: rows = tokens kt 32 + d32_row(v, q), columns = queries
    f32x16 s;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = 0.f;
    const _Float16* kp = krow + (size_t)kt * kstep;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 kf = STAGE ? *(const u32x4*)(kst + 16 * (CPR * r + ((2 * ks + q) ^ ((r >> FSH) & FMK))))
                             : ld16(kp + ks * 16);
      s = mfma32_f16(as_f16x8(kf), qh[ks], s);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int t = kt * kRT + d32_row(v, q);
      s[v] = t <= pos ? s[v] * a.qscale : -INFINITY;
      mt = fmaxf(mt, s[v]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);  // finite: token 0 is visible to every query
    const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    float ps = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s[v] = s[v] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s[v] - m_new);  // probability
      ps += s[v];
    }
    l = l * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int mt2 = 0; mt2 < NT; ++mt2)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt2][v] *= alpha;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f16x8 pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = (_Float16)s[8 * kk + i];
#pragma unroll
      for (int mt2 = 0; mt2 < NT; ++mt2) {
        u32x4 vf;
        if (STAGE) {
          const int vr = mt2 * 32 + r;
          vf = *(const u32x4*)(vst + 16 * (4 * vr + ((2 * kk + q) ^ ((vr >> 2) & 3))));
        } else {
          vf = ld16(a.vt + (size_t)(g * a.d_h + mt2 * 32 + r) * a.total + base + kt * kRT + 16 * kk + 8 * q);
        }
        acc[mt2] = mfma32_f16(as_f16x8(vf), pb, acc[mt2]);
      }
    }
  }
  if (STAGE) vm_wait<0>();  // the trailing reloads land before the workgroup ends
  l += __shfl_xor(l, 32, 64);
  if (jw + r >= a.n_q) return;
  const float il = 1.f / l;
  const size_t ooff = (((size_t)b * a.n_q + j) * a.H_q + h) * a.d_h;
  // O^T: lane holds query j, dims 32 mt + d32_row(v, q) (runs of 4)
#pragma unroll
  for (int mt2 = 0; mt2 < NT; ++mt2)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int e = mt2 * 32 + 8 * v4 + 4 * q;
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = acc[mt2][4 * v4 + i] * il;
      if (DT == STARKV_F32) {
        st16((float*)a.out + ooff + e, u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                                             __float_as_uint(o[3])});
      } else {
        st8((uint16_t*)a.out + ooff + e,
            u32x2{(uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16),
                  (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16)});
      }
    }
}

// ---------------------------------------------------------------------------------------------
// host side

void seq_bases(int B, const int32_t* lens, SeqBases* sb) {
  sb->B = B;
  sb->base[0] = 0;
  for (int b = 0; b < B; ++b) {
    sb->lens[b] = lens[b];
    sb->base[b + 1] = sb->base[b] + ceil_div(lens[b], kRT) * kRT;
  }
}

struct PrefillWs {
  size_t o_xk, o_xvh, o_xvl, o_kh, o_vt, bytes;
};

int value_rows_padded(const Layer& L) { return ceil_div(L.r_v, 64) * 64; }

// whether the value reconstruction takes the codes and the scaled B_v (int8/int4, r_v % 8 == 0)
bool value_codes(const Layer& L) { return L.latent == STARKV_LATENT_MIX84 && (L.r_v & 7) == 0; }

PrefillWs prefill_layout(const Layer& L, int total) {
  PrefillWs w;
  size_t o = 0;
  w.o_xk = o;
  o = align256(o + (size_t)total * L.n_key * 4);
  w.o_xvh = o;
  o = align256(o + (size_t)total * value_rows_padded(L) * 2);
  w.o_xvl = o;
  // int8/int4 layers with r_v a multiple of 8 keep the f16 scaled B_v^T here instead of a low part
  o = align256(o + std::max((size_t)total * value_rows_padded(L),
                            value_codes(L) ? (size_t)L.H_kv * L.d_h * L.r_v : (size_t)0) * 2);
  w.o_kh = o;
  o = align256(o + (size_t)total * L.H_kv * L.d_h * 2);
  w.o_vt = o;
  o = align256(o + (size_t)total * L.H_kv * L.d_h * 2);
  w.bytes = o;
  return w;
}

// launch with dynamic LDS, timed like launch_k
template <typename A>
hipError_t launch_lds(const ProfScope& ps, void (*kernel)(A), dim3 grid, dim3 block, size_t lds, hipStream_t s, A arg) {
  void* argv[] = {(void*)&arg};
  if (ps.start() && ps.stop())
    return hipExtLaunchKernel((const void*)kernel, grid, block, argv, lds, s, ps.start(), ps.stop(), 0);
  return hipLaunchKernel((const void*)kernel, grid, block, argv, lds, s);
}

constexpr int kReconVTile = 128, kReconVStages = 3;

template <int NT>
hipError_t launch_recon_flash(const Layer& L, const ReconArgs& ra, const ReconVArgs& va, const FlashArgs& fa, int B,
                              int n_q, hipStream_t s) {
  const int total = ra.total;
  const size_t lds = (size_t)L.d_h * ra.rpad * 2;
  const dim3 grid_r(ceil_div(total, 128), L.H_kv);
  {
    ProfScope ps("prefill_recon");
    const bool kc = L.latent == STARKV_LATENT_MIX84;
    const hipError_t e =
        ra.rope_theta > 0.f
            ? (kc ? launch_lds(ps, k_recon<NT, true, 0, true, true>, grid_r, dim3(256), lds, s, ra)
                  : launch_lds(ps, k_recon<NT, true, 0, true>, grid_r, dim3(256), lds, s, ra))
            : (kc ? launch_lds(ps, k_recon<NT, true, 0, false, true>, grid_r, dim3(256), lds, s, ra)
                  : launch_lds(ps, k_recon<NT, true, 0, false>, grid_r, dim3(256), lds, s, ra));
    if (e != hipSuccess) return e;
  }
  if (value_codes(L)) {
    ProfScope ps("prefill_recon_v");
    constexpr int T = kReconVTile;
    // the scaled factors into the low-part region, then codes x scaled factors
    ReconVArgs vc = va;
    const size_t n_el = (size_t)va.N * L.r_v;
    hipLaunchKernelGGL(k_scale_bv, dim3((unsigned)((n_el / 2 + 255) / 256)), dim3(256), 0, s, va.B_vt,
                       L.scales + L.n_key, va.N, L.r_v, (uint16_t*)va.xv_lo);
    vc.B_vt = va.xv_lo;
    const dim3 grid(ceil_div(total, T), ceil_div(va.N, T));
    const hipError_t e = launch_lds(ps, k_recon_v<T, T, kReconVStages, true>, grid, dim3(256),
                                    (size_t)kReconVStages * 2 * T * 128, s, vc);
    if (e != hipSuccess) return e;
  } else if ((L.r_v & 7) == 0) {
    ProfScope ps("prefill_recon_v");
    constexpr int T = kReconVTile;
    const dim3 grid(ceil_div(total, T), ceil_div(va.N, T));
    const hipError_t e = launch_lds(ps, k_recon_v<T, T, kReconVStages>, grid, dim3(256),
                                    (size_t)kReconVStages * 3 * T * 128, s, va);
    if (e != hipSuccess) return e;
  } else {
    ProfScope ps("prefill_recon_v");
    const hipError_t e = launch_lds(ps, k_recon<NT, false, 1, false>, grid_r, dim3(256), 0, s, ra);
    if (e != hipSuccess) return e;
  }
  ProfScope ps("prefill_attend");
  const dim3 grid(ceil_div(n_q, 128), L.H_q, B);
  constexpr bool stage = NT == 2 || NT == 4 || NT == 8;
  return launch_lds(ps, k_flash<NT, STARKV_BF16, stage>, grid, dim3(256),
                    stage ? (size_t)kFlashStages * 2 * kRT * 32 * NT * 2 : 0, s, fa);
}

}  // namespace

size_t prefill_workspace_bytes(const Layer& L, int B, const int32_t* lens) {
  size_t total = 0;
  for (int b = 0; b < B; ++b) total += (size_t)ceil_div(lens[b], kRT) * kRT;
  return prefill_layout(L, (int)total).bytes;
}

hipError_t launch_prefill(const Layer& L, const starkv_cache& c, const void* q, int B, int n_q, const int32_t* lens,
                          void* out, void* ws, hipStream_t s) {
  SeqBases sb;
  seq_bases(B, lens, &sb);
  const int total = sb.base[B];
  const PrefillWs w = prefill_layout(L, total);
  uint8_t* base = (uint8_t*)ws;
  float* xk = (float*)(base + w.o_xk);
  uint16_t* xvh = (uint16_t*)(base + w.o_xvh);
  uint16_t* xvl = (uint16_t*)(base + w.o_xvl);
  const int rvp = value_rows_padded(L);
  _Float16* kh = (_Float16*)(base + w.o_kh);
  _Float16* vt = (_Float16*)(base + w.o_vt);
  // 1. dequantised latent
  DeqArgs da;
  da.k_rows = (const uint8_t*)c.k_rows;
  da.v_tiles = (const uint8_t*)c.v_tiles;
  da.scales = L.scales;
  da.src = L.d_src;
  da.heads = L.heads();
  da.xk = xk;
  da.xv_hi = xvh;
  da.xv_lo = xvl;
  da.n_lat = L.n_lat;
  da.n_key = L.n_key;
  da.r_v = L.r_v;
  da.rvp = rvp;
  da.H_kv = L.H_kv;
  da.K8 = L.K8;
  da.pack3 = L.pack3;
  da.K4 = L.K4;
  da.V4 = L.V4;
  da.V8 = L.V8;
  da.n8v = L.n8v;
  da.k_row_bytes = L.k_row_bytes;
  da.v_rows = L.v_rows;
  da.T_max = c.T_max;
  da.codes = value_codes(L) ? 1 : 0;
  da.sb = sb;
  hipError_t e;
  {
    ProfScope ps("prefill_dequant");
    const dim3 grid(total / kRT);
    if (L.latent == STARKV_LATENT_MIX84) e = launch_k(ps, k_deq_latent<STARKV_LATENT_MIX84>, grid, dim3(256), s, da);
    else if (L.latent == STARKV_LATENT_BF16) e = launch_k(ps, k_deq_latent<STARKV_LATENT_BF16>, grid, dim3(256), s, da);
    else e = launch_k(ps, k_deq_latent<STARKV_LATENT_F32>, grid, dim3(256), s, da);
    if (e != hipSuccess) return e;
  }
  // 2 + 3. reconstruction, attention
  int rmax = 1;
  for (int g = 0; g < L.H_kv; ++g) rmax = std::max(rmax, L.rk[g]);
  ReconArgs ra;
  ra.xk = xk;
  ra.kscales = L.scales;
  ra.xv_hi = xvh;
  ra.xv_lo = xvl;
  ra.B_k = (const uint16_t*)L.B_k;
  ra.B_vt = (const uint16_t*)L.B_vt;
  ra.koff = L.d_koff;
  ra.kh = kh;
  ra.vt = vt;
  ra.n_lat = L.n_lat;
  ra.n_key = L.n_key;
  ra.r_v = L.r_v;
  ra.rvp = rvp;
  ra.H_kv = L.H_kv;
  ra.d_h = L.d_h;
  ra.total = total;
  ra.rpad = ceil_div(rmax, 16) * 16;
  ra.rope_theta = L.rope_theta;
  ra.rotary_dim = L.rotary_dim;
  ra.sb = sb;
  ReconVArgs va;
  va.xv_hi = xvh;
  va.xv_lo = xvl;
  va.B_vt = (const uint16_t*)L.B_vt;
  va.vt = vt;
  va.rvp = rvp;
  va.r_v = L.r_v;
  va.N = L.H_kv * L.d_h;
  va.total = total;
  va.sb = sb;
  FlashArgs fa;
  fa.q = q;
  fa.out = out;
  fa.kh = kh;
  fa.vt = vt;
  fa.n_q = n_q;
  fa.H_q = L.H_q;
  fa.H_kv = L.H_kv;
  fa.G = L.G;
  fa.d_h = L.d_h;
  fa.total = total;
  fa.qscale = (float)(1.4426950408889634 / sqrt((double)L.d_h));
  fa.rope_theta = L.rope_theta;
  fa.rotary_dim = L.rotary_dim;
  fa.sb = sb;
  switch (L.d_h / 32) {
    case 1: e = launch_recon_flash<1>(L, ra, va, fa, B, n_q, s); break;
    case 2: e = launch_recon_flash<2>(L, ra, va, fa, B, n_q, s); break;
    case 3: e = launch_recon_flash<3>(L, ra, va, fa, B, n_q, s); break;
    case 4: e = launch_recon_flash<4>(L, ra, va, fa, B, n_q, s); break;
    case 5: e = launch_recon_flash<5>(L, ra, va, fa, B, n_q, s); break;
    case 6: e = launch_recon_flash<6>(L, ra, va, fa, B, n_q, s); break;
    case 7: e = launch_recon_flash<7>(L, ra, va, fa, B, n_q, s); break;
    default: e = launch_recon_flash<8>(L, ra, va, fa, B, n_q, s); break;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace skv
