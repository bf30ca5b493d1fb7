// Decode attention read directly from the low-rank latent cache.
//
// STAR-KV summary page, Methodology section 2: keys are factored per head (HD), values
// jointly (JD), and the reconstruction matrices are moved past the attention weights by
// reordering the operations.  Per sequence b, query row i = (KV head g, query head in
// group, query j):
//   qproj   q^_i   = (q_i B_g^T) * scale_c * log2(e) / sqrt(d_h)      (query in latent space)
//   scores  s_i,t  = q^_i . code_g[t]  (base-2 logits), per 64-token chunk: max m, sum l,
//           p~ = 2^(s - m) stored (f16 / bf16 / f32)
//   values  z_i    = sum_t p~_i,t 2^(m_c - M_split) code_v[t]         (MFMA, split partials)
//   merge   out_i  = (sum_splits w z) * scale_v B_v^g / l             (log-sum-exp merge + up-projection)
// Key scores run on MFMA as a block-diagonal GEMM: rows = 16 tokens, columns = 16 query
// rows, K = key-row slots (the query fragments are zero outside their head's segment).
#include <math.h>

#include <algorithm>
#include <cstdlib>

#include "device_common.h"
#include "profile.h"
#include "starkv_internal.h"

namespace skv {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static int ceil_div(int a, int b) { return (a + b - 1) / b; }

static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

int plan_decode(const Layer& L, int B, int n_q, const int32_t* lens, int T_max, void* ws_base, DecodePlan* P,
                KtList* kts, SeqTable* seq) {
  DecodeGeom& g = P->g;
  g.B = B;
  g.n_q = n_q;
  g.M_q = L.H_q * n_q;
  g.M_pad = ceil_div(g.M_q, 32) * 32;
  g.nct = ceil_div(g.M_q, 16);
  g.G = L.G;
  g.d_h = L.d_h;
  g.H_q = L.H_q;
  g.H_kv = L.H_kv;
  g.n_key = L.n_key;
  g.r_v = L.r_v;
  g.K8 = L.K8;
  g.K4 = L.K4;
  g.key_kt = L.key_kt;
  g.key_kpos = L.key_kpos;
  g.k_row_bytes = L.k_row_bytes;
  g.v_rows = L.v_rows;
  g.v_tile_bytes = L.v_tile_bytes;
  g.T_max = T_max;
  g.latent = L.latent;
  g.dtype = L.dtype;
  g.qscale = (float)(1.4426950408889634 / sqrt((double)L.d_h));

  // K-tiles touched by every 16-row column tile (block-diagonal query fragments)
  const int rows_per_head = L.G * n_q;
  int nkt_max = 1;
  for (int ct = 0; ct < g.nct; ++ct) {
    const int i0 = ct * 16, i1 = std::min(i0 + 16, g.M_q);
    const int g_lo = i0 / rows_per_head, g_hi = (i1 - 1) / rows_per_head;
    bool used[256] = {false};
    auto mark = [&](int lo, int hi) {  // K positions [lo, hi)
      if (hi <= lo) return;
      for (int kt = lo / L.key_kt; kt <= (hi - 1) / L.key_kt; ++kt) used[kt] = true;
    };
    if (L.mix()) {
      mark(L.off8[g_lo], L.off8[g_hi + 1]);
      mark(L.K8 + L.off4[g_lo], L.K8 + L.off4[g_hi + 1]);
    } else {
      mark(L.koff[g_lo], L.koff[g_hi + 1]);
    }
    int n = 0;
    for (int kt = 0; kt < 256; ++kt)
      if (used[kt]) {
        if (n >= kMaxKT) return STARKV_EUNSUPPORTED;
        kts->kt[ct][n++] = (uint8_t)kt;
      }
    kts->n[ct] = (uint8_t)n;
    nkt_max = std::max(nkt_max, n);
  }

  // chunks and splits
  const int NB = L.v_rows / 32;
  int bpw = NB >= 16 ? 4 : (NB >= 8 ? 2 : 1);
  bpw = env_int("STARKV_BPW", bpw);
  if (bpw < 1 || bpw > 4) bpw = 4;
  const int n_slices = ceil_div(NB, bpw);
  int total_chunks = 0, max_chunks = 0;
  seq->chunk_off[0] = 0;
  for (int b = 0; b < B; ++b) {
    seq->lens[b] = lens[b];
    const int nc = ceil_div(lens[b], kTC);
    seq->chunk_off[b + 1] = seq->chunk_off[b] + nc;
    total_chunks += nc;
    max_chunks = std::max(max_chunks, nc);
  }
  int cps = std::max(1, (total_chunks * n_slices) / 512);
  cps = std::max(cps, ceil_div(max_chunks, kMaxSplitsPerSeq));
  const int cps_env = env_int("STARKV_CPS", 0);
  if (cps_env > 0) cps = std::max(cps_env, ceil_div(max_chunks, kMaxSplitsPerSeq));
  int total_splits = 0;
  seq->split_off[0] = 0;
  for (int b = 0; b < B; ++b) {
    const int nc = seq->chunk_off[b + 1] - seq->chunk_off[b];
    seq->split_off[b + 1] = seq->split_off[b] + ceil_div(nc, cps);
    total_splits += ceil_div(nc, cps);
  }

  // workspace
  DecodeWs& w = P->ws;
  const int esz_p = L.latent == STARKV_LATENT_F32 ? 4 : 2;
  size_t o = 0;
  const size_t o_qfrag = o; o = align256(o + (size_t)B * g.nct * nkt_max * 2048);
  const size_t o_rowp = o; o = align256(o + (size_t)B * g.M_pad * 16);
  const size_t o_p = o; o = align256(o + (size_t)total_chunks * g.M_pad * kTC * esz_p);
  const size_t o_cm = o; o = align256(o + (size_t)total_chunks * g.M_pad * 4);
  const size_t o_cl = o; o = align256(o + (size_t)total_chunks * g.M_pad * 4);
  const size_t o_zp = o; o = align256(o + (size_t)total_splits * g.M_pad * L.r_v * 4);
  const size_t o_sm = o; o = align256(o + (size_t)total_splits * g.M_pad * 4);
  const size_t o_sl = o; o = align256(o + (size_t)total_splits * g.M_pad * 4);
  P->ws_bytes = o;
  uint8_t* base = (uint8_t*)ws_base;
  w.qfrag = base + o_qfrag;
  w.rowp = (float*)(base + o_rowp);
  w.p = base + o_p;
  w.cm = (float*)(base + o_cm);
  w.cl = (float*)(base + o_cl);
  w.zp = (float*)(base + o_zp);
  w.sm = (float*)(base + o_sm);
  w.sl = (float*)(base + o_sl);
  w.nkt_max = nkt_max;
  w.total_chunks = total_chunks;
  w.total_splits = total_splits;
  w.cps = cps;
  w.blocks_per_wg = bpw;
  return STARKV_OK;
}

// ===========================================================================
// qproj: query fragments of the key-score GEMM

struct QprojArgs {
  const void* q;
  const void* B_k;
  const uint16_t* scales;
  HeadTables heads;
  uint8_t* qfrag;
  float* rowp;
  DecodeGeom g;
  int nkt_max;
  KtList kts;
};

template <int DT>
__device__ __forceinline__ float ldx(const void* p, size_t i) {
  if (DT == STARKV_F32) return ((const float*)p)[i];
  return bf16_to_f32(((const uint16_t*)p)[i]);
}

template <int DT, int LAT>
__global__ __launch_bounds__(256) void k_qproj(QprojArgs a) {
  constexpr int RMAX = 256;
  __shared__ float qh[16][RMAX];
  __shared__ float rho_s[16];
  __shared__ int seg_g[16];
  const int ct = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const DecodeGeom& g = a.g;
  const int rph = g.G * g.n_q;
  if (tid < 16) {
    const int i = ct * 16 + tid;
    seg_g[tid] = (i < g.M_q) ? i / rph : -1;
  }
  __syncthreads();
  // q^ = (q B_g^T) * scale * log2(e)/sqrt(d_h) over each row's segment
  for (int idx = tid; idx < 16 * RMAX; idx += 256) {
    const int n = idx / RMAX, k = idx % RMAX;
    const int gg = seg_g[n];
    float val = 0.f;
    if (gg >= 0) {
      const int c0 = a.heads.koff[gg];
      const int r = a.heads.koff[gg + 1] - c0;
      if (k < r) {
        const int i = ct * 16 + n;
        const int hh = (i % rph) / g.n_q, j = i % g.n_q;
        const int h = gg * g.G + hh;
        const size_t qoff = (((size_t)b * g.n_q + j) * g.H_q + h) * g.d_h;
        const size_t boff = (size_t)(c0 + k) * g.d_h;
        float acc = 0.f;
        for (int e = 0; e < g.d_h; ++e) acc = fmaf(ldx<DT>(a.q, qoff + e), ldx<DT>(a.B_k, boff + e), acc);
        float sc = 1.f;
        if (LAT == STARKV_LATENT_MIX84) sc = f16_to_f32(a.scales[c0 + k]);
        val = acc * sc * g.qscale;
      }
    }
    qh[n][k] = val;
  }
  __syncthreads();
  if (LAT == STARKV_LATENT_MIX84 && tid < 16) {
    const int gg = seg_g[tid];
    float amax = 0.f;
    if (gg >= 0) {
      const int r = a.heads.koff[gg + 1] - a.heads.koff[gg];
      for (int k = 0; k < r; ++k) amax = fmaxf(amax, fabsf(qh[tid][k]));
    }
    rho_s[tid] = amax > 0.f ? amax / 127.f : 1.f;
  }
  __syncthreads();
  // hi/lo split per element; int8 keeps rho * (hi + lo/254), bf16 keeps hi + lo
  __shared__ int8_t hi8[16][RMAX];
  __shared__ int8_t lo8[16][RMAX];
  for (int idx = tid; idx < 16 * RMAX; idx += 256) {
    const int n = idx / RMAX, k = idx % RMAX;
    const float x = qh[n][k];
    if (LAT == STARKV_LATENT_MIX84) {
      const float rho = rho_s[n];
      float hi = fminf(fmaxf(__builtin_rintf(x / rho), -127.f), 127.f);
      float lo = fminf(fmaxf(__builtin_rintf((x - hi * rho) * (254.f / rho)), -127.f), 127.f);
      hi8[n][k] = (int8_t)hi;
      lo8[n][k] = (int8_t)lo;
    }
  }
  __syncthreads();
  // row parameters
  if (tid < 16) {
    const int i = ct * 16 + tid;
    const int gg = seg_g[tid];
    if (gg >= 0) {
      float bh = 0.f, bl = 0.f;
      if (LAT == STARKV_LATENT_MIX84) {
        const int r = a.heads.koff[gg + 1] - a.heads.koff[gg];
        int sh = 0, sl = 0;
        for (int k = a.heads.n8[gg]; k < r; ++k) {
          sh += hi8[tid][k];
          sl += lo8[tid][k];
        }
        bh = (float)(8 * sh);
        bl = (float)(8 * sl);
      }
      float* rp = a.rowp + ((size_t)b * g.M_pad + i) * 4;
      rp[0] = LAT == STARKV_LATENT_MIX84 ? rho_s[tid] : 1.f;
      rp[1] = bh;
      rp[2] = bl;
      rp[3] = 0.f;
    }
  }
  // fragments
  const int wave = wave_id(), lane = tid & 63;
  const int n = lane & 15, qq = lane >> 4;
  const int gg = seg_g[n];
  const int nkt = a.kts.n[ct];
  for (int jt = wave; jt < nkt; jt += 4) {
    const int kt = a.kts.kt[ct][jt];
    uint8_t* frag = a.qfrag + (((size_t)b * g.nct + ct) * a.nkt_max + jt) * 2048;
    if (LAT == STARKV_LATENT_MIX84) {
      const int P0 = kt * 64 + 16 * qq;
      uint32_t wh[4] = {0, 0, 0, 0}, wl[4] = {0, 0, 0, 0};
      if (gg >= 0 && P0 < g.K8 + g.K4) {
        const int c0 = a.heads.koff[gg];
        const int n8g = a.heads.n8[gg];
        const int n4g = (a.heads.koff[gg + 1] - c0) - n8g;
        const int o8 = a.heads.off8[gg], o4 = a.heads.off4[gg];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          int k = -1;
          if (P0 < g.K8) {
            const int slot = P0 + e;
            if (slot >= o8 && slot < o8 + n8g) k = slot - o8;
          } else {
            const int u = P0 - g.K8 + int4_perm16(e);
            if (u >= o4 && u < o4 + n4g) k = n8g + (u - o4);
          }
          if (k >= 0) {
            wh[e >> 2] |= ((uint32_t)(uint8_t)hi8[n][k]) << (8 * (e & 3));
            wl[e >> 2] |= ((uint32_t)(uint8_t)lo8[n][k]) << (8 * (e & 3));
          }
        }
      }
      st16(frag + lane * 16, u32x4{wh[0], wh[1], wh[2], wh[3]});
      st16(frag + 1024 + lane * 16, u32x4{wl[0], wl[1], wl[2], wl[3]});
    } else {
      const int P0 = kt * 32 + 8 * qq;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = 0.f;
        if (gg >= 0) {
          const int k = P0 + e - a.heads.koff[gg];
          const int r = a.heads.koff[gg + 1] - a.heads.koff[gg];
          if (k >= 0 && k < r) v[e] = qh[n][k];
        }
      }
      if (LAT == STARKV_LATENT_F32) {
        st16(frag + lane * 32, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                     __float_as_uint(v[3])});
        st16(frag + lane * 32 + 16, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                                          __float_as_uint(v[7])});
      } else {
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const uint16_t h0 = f32_to_bf16(v[2 * e2]), h1 = f32_to_bf16(v[2 * e2 + 1]);
          const uint16_t l0 = f32_to_bf16(v[2 * e2] - bf16_to_f32(h0));
          const uint16_t l1 = f32_to_bf16(v[2 * e2 + 1] - bf16_to_f32(h1));
          wh[e2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          wl[e2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        st16(frag + lane * 16, u32x4{wh[0], wh[1], wh[2], wh[3]});
        st16(frag + 1024 + lane * 16, u32x4{wl[0], wl[1], wl[2], wl[3]});
      }
    }
  }
}

// ===========================================================================
// scores: per (sequence, 64-token chunk): p~ = 2^(s - m_chunk), chunk max and sum

struct ScoreArgs {
  const uint8_t* k_rows;
  const uint8_t* qfrag;
  const float* rowp;
  void* p;
  float* cm;
  float* cl;
  DecodeGeom g;
  int nkt_max;
  KtList kts;
  SeqTable seq;
};

template <int LAT>
__global__ __launch_bounds__(256) void k_scores(ScoreArgs a) {
  const DecodeGeom& g = a.g;
  const int cg = blockIdx.x;
  const int b = find_segment(a.seq.chunk_off, g.B, cg);
  const int c = cg - a.seq.chunk_off[b];
  const int t0 = c * kTC;
  const int len = a.seq.lens[b];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int W = blockDim.x >> 6;
  const int n = lane & 15, qq = lane >> 4;
  const uint8_t* kbase = a.k_rows + (size_t)b * g.T_max * g.k_row_bytes;

  for (int ct = wave; ct < g.nct; ct += W) {
    const int i = ct * 16 + n;  // query row of this lane's result column
    const bool rowvalid = i < g.M_q;
    const int pos = len - g.n_q + (i % g.n_q);
    float rho = 1.f, bh = 0.f, bl = 0.f;
    if (rowvalid) {
      const float* rp = a.rowp + ((size_t)b * g.M_pad + i) * 4;
      rho = rp[0];
      bh = rp[1];
      bl = rp[2];
    }
    const int nkt = a.kts.n[ct];
    const uint8_t* fbase = a.qfrag + ((size_t)b * g.nct + ct) * a.nkt_max * 2048;
    float s2[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int tok = t0 + tt * 16 + n;  // A-fragment row (token) of this lane
      const bool tok_ok = tok < len;
      const uint8_t* row = kbase + (size_t)(tok_ok ? tok : 0) * g.k_row_bytes;
      if (LAT == STARKV_LATENT_MIX84) {
        i32x4 ah = {0, 0, 0, 0}, al = {0, 0, 0, 0};
        for (int jt = 0; jt < nkt; ++jt) {
          const int kt = a.kts.kt[ct][jt];
          const i32x4 fh = __builtin_bit_cast(i32x4, ld16(fbase + jt * 2048 + lane * 16));
          const i32x4 fl = __builtin_bit_cast(i32x4, ld16(fbase + jt * 2048 + 1024 + lane * 16));
          const int P0 = kt * 64 + 16 * qq;
          i32x4 av = {0, 0, 0, 0};
          if (tok_ok) {
            if (P0 < g.K8) av = __builtin_bit_cast(i32x4, ld16(row + P0));
            else if (P0 < g.K8 + g.K4) av = unpack_int4_group(ld8(row + g.K8 + (P0 - g.K8) / 2));
          }
          ah = mfma16_i8(av, fh, ah);
          al = mfma16_i8(av, fl, al);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
          s2[tt][v] = rho * (float)(ah[v] - (int)bh) + (rho * (1.f / 254.f)) * (float)(al[v] - (int)bl);
      } else if (LAT == STARKV_LATENT_BF16) {
        f32x4 acc = {0, 0, 0, 0};
        for (int jt = 0; jt < nkt; ++jt) {
          const int kt = a.kts.kt[ct][jt];
          const u32x4 fh = ld16(fbase + jt * 2048 + lane * 16);
          const u32x4 fl = ld16(fbase + jt * 2048 + 1024 + lane * 16);
          const int P0 = kt * 32 + 8 * qq;
          u32x4 av = {0, 0, 0, 0};
          if (tok_ok && P0 < g.key_kpos) av = ld16(row + 2 * P0);
          acc = mfma16_bf16(as_bf16x8(av), as_bf16x8(fh), acc);
          acc = mfma16_bf16(as_bf16x8(av), as_bf16x8(fl), acc);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) s2[tt][v] = acc[v];
      } else {
        f32x4 acc = {0, 0, 0, 0};
        for (int jt = 0; jt < nkt; ++jt) {
          const int kt = a.kts.kt[ct][jt];
          const u32x4 f0 = ld16(fbase + jt * 2048 + lane * 32);
          const u32x4 f1 = ld16(fbase + jt * 2048 + lane * 32 + 16);
          const int P0 = kt * 32 + 8 * qq;
          u32x4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
          if (tok_ok && P0 < g.key_kpos) a0 = ld16(row + 4 * P0);
          if (tok_ok && P0 + 4 < g.key_kpos) a1 = ld16(row + 4 * P0 + 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = mfma16_f32(__uint_as_float(a0[e]), __uint_as_float(f0[e]), acc);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = mfma16_f32(__uint_as_float(a1[e]), __uint_as_float(f1[e]), acc);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) s2[tt][v] = acc[v];
      }
      // lane holds D[token 4*qq + v][column n]
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + tt * 16 + 4 * qq + v;
        const bool ok = rowvalid && t < len && t <= pos;
        s2[tt][v] = ok ? s2[tt][v] : -INFINITY;
      }
    }
    float m = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) m = fmaxf(m, s2[tt][v]);
    m = wave_max_xor(m, 16);
    m = wave_max_xor(m, 32);
    float l = 0.f;
    const size_t prow = ((size_t)cg * g.M_pad + i) * kTC;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      float e4[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        e4[v] = (s2[tt][v] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s2[tt][v] - m);
        l += e4[v];
      }
      const size_t off = prow + tt * 16 + 4 * qq;
      if (LAT == STARKV_LATENT_F32) {
        st16((float*)a.p + off, u32x4{__float_as_uint(e4[0]), __float_as_uint(e4[1]), __float_as_uint(e4[2]),
                                      __float_as_uint(e4[3])});
      } else if (LAT == STARKV_LATENT_BF16) {
        const uint32_t w0 = (uint32_t)f32_to_bf16(e4[0]) | ((uint32_t)f32_to_bf16(e4[1]) << 16);
        const uint32_t w1 = (uint32_t)f32_to_bf16(e4[2]) | ((uint32_t)f32_to_bf16(e4[3]) << 16);
        st8((uint16_t*)a.p + off, u32x2{w0, w1});
      } else {
        const uint32_t w0 = (uint32_t)f32_to_f16(e4[0]) | ((uint32_t)f32_to_f16(e4[1]) << 16);
        const uint32_t w1 = (uint32_t)f32_to_f16(e4[2]) | ((uint32_t)f32_to_f16(e4[3]) << 16);
        st8((uint16_t*)a.p + off, u32x2{w0, w1});
      }
    }
    l = wave_sum_xor(l, 16);
    l = wave_sum_xor(l, 32);
    if (qq == 0) {
      a.cm[(size_t)cg * g.M_pad + i] = m;
      a.cl[(size_t)cg * g.M_pad + i] = l;
    }
  }
}

// ===========================================================================
// values: z partial of one (sequence, split) for a slice of value blocks

struct ValueArgs {
  const uint8_t* v_tiles;
  const void* p;
  const float* cm;
  const float* cl;
  float* zp;
  float* sm;
  float* sl;
  DecodeGeom g;
  SeqTable seq;
  int cps, bpw, NB, V8, n8v, n4v;
};

// 8 tokens of one channel (int8 codes in 8 bytes) -> f16x8
__device__ __forceinline__ f16x8 deq_i8x8(uint32_t w0, uint32_t w1) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (_Float16)sbyte(w0, e);
    r[4 + e] = (_Float16)sbyte(w1, e);
  }
  return r;
}
// 8 tokens of a channel pair (8 bytes): low nibbles -> even channel, high -> odd channel
__device__ __forceinline__ void deq_i4x8(uint32_t w0, uint32_t w1, f16x8& ev, f16x8& od) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ev[e] = (_Float16)snib(w0, 2 * e);
    od[e] = (_Float16)snib(w0, 2 * e + 1);
    ev[4 + e] = (_Float16)snib(w1, 2 * e);
    od[4 + e] = (_Float16)snib(w1, 2 * e + 1);
  }
}

template <int LAT, int NMT>
__global__ __launch_bounds__(256) void k_values(ValueArgs a) {
  const DecodeGeom& g = a.g;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int nb = blockIdx.x * a.bpw + wave;  // value block of this wave (wave-uniform)
  if (nb >= a.NB) return;
  const int sg = blockIdx.y;
  const int b = find_segment(a.seq.split_off, g.B, sg);
  const int s = sg - a.seq.split_off[b];
  const int cbase = a.seq.chunk_off[b];
  const int nch = a.seq.chunk_off[b + 1] - cbase;
  const int c_lo = s * a.cps, c_hi = min(c_lo + a.cps, nch);
  const int len = a.seq.lens[b];
  const int r = lane & 31, q = lane >> 5;
  const bool is4 = (LAT == STARKV_LATENT_MIX84) && (nb >= a.V8 / 32);
  constexpr int esz = LAT == STARKV_LATENT_F32 ? 4 : (LAT == STARKV_LATENT_BF16 ? 2 : 1);

  // split max per row held by this lane (as an A-fragment row)
  float Ms[NMT], lsum[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int row = mt * 32 + r;
    float m = -INFINITY;
    if (row < g.M_q)
      for (int c = c_lo; c < c_hi; ++c) m = fmaxf(m, a.cm[(size_t)(cbase + c) * g.M_pad + row]);
    Ms[mt] = m;
    lsum[mt] = 0.f;
  }

  f32x16 acc[NMT][2];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][nt][v] = 0.f;

  const uint8_t* vb = a.v_tiles + (size_t)b * (g.T_max / kTT) * g.v_tile_bytes;
  for (int c = c_lo; c < c_hi; ++c) {
    const size_t cgl = (size_t)(cbase + c);
    float alpha[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int row = mt * 32 + r;
      float al = 0.f;
      if (row < g.M_q) {
        const float m = a.cm[cgl * g.M_pad + row];
        if (m != -INFINITY) al = __builtin_amdgcn_exp2f(m - Ms[mt]);
        lsum[mt] += al * a.cl[cgl * g.M_pad + row];
      }
      alpha[mt] = al;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int tt0 = c * kTC + half * 32;
      if (tt0 >= len) break;
      const uint8_t* trow = vb + (size_t)(tt0 / kTT) * g.v_tile_bytes + (size_t)(nb * 32 + r) * kTT * esz;
      // this lane's 16 tokens: tt0 + 16q .. +15
      u32x4 vraw[4];
      if (esz == 1) {
        vraw[0] = ld16(trow + 16 * q);
      } else if (esz == 2) {
        vraw[0] = ld16(trow + 32 * q);
        vraw[1] = ld16(trow + 32 * q + 16);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) vraw[k] = ld16(trow + 64 * q + 16 * k);
      }
      if (esz > 1 && tt0 + 32 > len) {
        // zero the elements of tokens at or past the length (their bits may be anything)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t = tt0 + 16 * q + e;
          if (t >= len) {
            if (esz == 2) {
              const uint32_t keep = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
              vraw[e >> 3][(e >> 1) & 3] = vraw[e >> 3][(e >> 1) & 3] & keep;
            } else {
              vraw[e >> 2][e & 3] = 0u;
            }
          }
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tk = 32 * half + 16 * q + 8 * h;  // token offset inside the chunk
        // value fragments of this K-step (8 tokens of one channel, or of a channel pair)
        f16x8 v_lo, v_hi;
        if (LAT == STARKV_LATENT_MIX84) {
          const uint32_t w0 = vraw[0][2 * h], w1 = vraw[0][2 * h + 1];
          if (is4) deq_i4x8(w0, w1, v_lo, v_hi);
          else v_lo = deq_i8x8(w0, w1);
        }
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          const int row = mt * 32 + r;
          const bool rok = row < g.M_q;
          if (LAT == STARKV_LATENT_F32) {
            const float* pp = (const float*)a.p + (cgl * g.M_pad + row) * kTC + tk;
            u32x4 p0 = {0, 0, 0, 0}, p1 = {0, 0, 0, 0};
            if (rok) {
              p0 = ld16(pp);
              p1 = ld16(pp + 4);
            }
            const u32x4 v0 = vraw[2 * h], v1 = vraw[2 * h + 1];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[mt][0] = mfma32_f32(__uint_as_float(p0[e]) * alpha[mt], __uint_as_float(v0[e]), acc[mt][0]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[mt][0] = mfma32_f32(__uint_as_float(p1[e]) * alpha[mt], __uint_as_float(v1[e]), acc[mt][0]);
          } else {
            const uint16_t* pp = (const uint16_t*)a.p + (cgl * g.M_pad + row) * kTC + tk;
            u32x4 praw = {0, 0, 0, 0};
            if (rok) praw = ld16(pp);
            if (LAT == STARKV_LATENT_BF16) {
              u32x4 ps;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float x0 = bf16_to_f32((uint16_t)(praw[e] & 0xFFFF)) * alpha[mt];
                const float x1 = bf16_to_f32((uint16_t)(praw[e] >> 16)) * alpha[mt];
                ps[e] = (uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16);
              }
              acc[mt][0] = mfma32_bf16(as_bf16x8(ps), as_bf16x8(vraw[h]), acc[mt][0]);
            } else {
              f16x8 ps;
              const f16x8 pin = as_f16x8(praw);
#pragma unroll
              for (int e = 0; e < 8; ++e) ps[e] = (_Float16)((float)pin[e] * alpha[mt]);
              acc[mt][0] = mfma32_f16(ps, v_lo, acc[mt][0]);
              if (is4) acc[mt][1] = mfma32_f16(ps, v_hi, acc[mt][1]);
            }
          }
        }
      }
    }
  }

  // z partial: lane holds column r of the block, rows d32_row(v, q) of each M-tile
  const int ntiles = is4 ? 2 : 1;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (nt >= ntiles) break;
    int vc;
    bool cok;
    if (LAT == STARKV_LATENT_MIX84) {
      if (!is4) {
        vc = nb * 32 + r;
        cok = vc < a.n8v;
      } else {
        const int w = 2 * ((nb - a.V8 / 32) * 32 + r) + nt;
        cok = w < a.n4v;
        vc = a.n8v + w;
      }
    } else {
      vc = nb * 32 + r;
      cok = vc < g.r_v;
    }
    if (!cok) continue;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = mt * 32 + d32_row(v, q);
        if (row < g.M_q) a.zp[((size_t)sg * g.M_pad + row) * g.r_v + vc] = acc[mt][nt][v];
      }
  }
  if (blockIdx.x == 0 && wave == 0 && q == 0) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int row = mt * 32 + r;
      if (row < g.M_q) {
        a.sm[(size_t)sg * g.M_pad + row] = Ms[mt];
        a.sl[(size_t)sg * g.M_pad + row] = lsum[mt];
      }
    }
  }
}

// ===========================================================================
// merge + up-projection: out = (sum_s w_s z_s) * scale_v B_v^g / l

struct MergeArgs {
  const float* zp;
  const float* sm;
  const float* sl;
  const void* B_vt;
  const uint16_t* vscales;  // value-channel scales (mix84) or null
  void* out;
  DecodeGeom g;
  SeqTable seq;
};

template <int DT>
__global__ __launch_bounds__(256) void k_merge(MergeArgs a) {
  const DecodeGeom& g = a.g;
  const int gk = blockIdx.x;  // KV head
  const int rph = g.G * g.n_q;
  const int Rg = g.B * rph;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  __shared__ float wts[16][kMaxSplitsPerSeq];
  __shared__ float invl[16];
  __shared__ int rb[16], ri[16];
  __shared__ float zf[16][33];
  __shared__ uint16_t zh[16][40], zl[16][40];
  if (tid < 16) {
    const int rr = blockIdx.y * 16 + tid;
    int bb = -1, ii = 0;
    if (rr < Rg) {
      bb = rr / rph;
      ii = gk * rph + rr % rph;
    }
    rb[tid] = bb;
    ri[tid] = ii;
    if (bb >= 0) {
      const int s0 = a.seq.split_off[bb], ns = a.seq.split_off[bb + 1] - s0;
      float M = -INFINITY;
      for (int s = 0; s < ns; ++s) M = fmaxf(M, a.sm[(size_t)(s0 + s) * g.M_pad + ii]);
      float l = 0.f;
      for (int s = 0; s < ns; ++s) {
        const float ms = a.sm[(size_t)(s0 + s) * g.M_pad + ii];
        const float w = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
        wts[tid][s] = w;
        l += w * a.sl[(size_t)(s0 + s) * g.M_pad + ii];
      }
      invl[tid] = 1.f / l;
    } else {
      invl[tid] = 0.f;
    }
  }
  __syncthreads();
  const int n_nt = g.d_h / 16;
  f32x4 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = f32x4{0, 0, 0, 0};
  const int n = lane & 15, qq = lane >> 4;
  for (int kc = 0; kc < g.r_v; kc += 32) {
    // merged, scaled, normalised value latent tile [16 rows][32 channels]
    for (int idx = tid; idx < 16 * 32; idx += 256) {
      const int rr = idx >> 5, cc = idx & 31;
      const int bb = rb[rr];
      float z = 0.f;
      if (bb >= 0 && kc + cc < g.r_v) {
        const int s0 = a.seq.split_off[bb], ns = a.seq.split_off[bb + 1] - s0;
        for (int s = 0; s < ns; ++s) z += wts[rr][s] * a.zp[((size_t)(s0 + s) * g.M_pad + ri[rr]) * g.r_v + kc + cc];
        if (a.vscales) z *= f16_to_f32(a.vscales[kc + cc]);
        z *= invl[rr];
      }
      if (DT == STARKV_F32) {
        zf[rr][cc] = z;
      } else {
        const uint16_t hb = f32_to_bf16(z);
        zh[rr][cc] = hb;
        zl[rr][cc] = f32_to_bf16(z - bf16_to_f32(hb));
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int nt = wave + 4 * k;
      if (nt >= n_nt) break;
      const size_t brow = (size_t)(gk * g.d_h + nt * 16 + n) * g.r_v;
      if (DT == STARKV_F32) {
        const float* bp = (const float*)a.B_vt + brow;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int cch = kc + 8 * qq + e;
          const float bv = (cch < g.r_v) ? bp[cch] : 0.f;
          acc[k] = mfma16_f32(zf[n][8 * qq + e], bv, acc[k]);
        }
      } else {
        const uint16_t* bp = (const uint16_t*)a.B_vt + brow;
        uint32_t bw[4], ah[4], al[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int c0 = kc + 8 * qq + 2 * e2;
          const uint32_t b0 = (c0 < g.r_v) ? bp[c0] : 0u;
          const uint32_t b1 = (c0 + 1 < g.r_v) ? bp[c0 + 1] : 0u;
          bw[e2] = b0 | (b1 << 16);
          ah[e2] = (uint32_t)zh[n][8 * qq + 2 * e2] | ((uint32_t)zh[n][8 * qq + 2 * e2 + 1] << 16);
          al[e2] = (uint32_t)zl[n][8 * qq + 2 * e2] | ((uint32_t)zl[n][8 * qq + 2 * e2 + 1] << 16);
        }
        const bf16x8 B8 = as_bf16x8(u32x4{bw[0], bw[1], bw[2], bw[3]});
        acc[k] = mfma16_bf16(as_bf16x8(u32x4{ah[0], ah[1], ah[2], ah[3]}), B8, acc[k]);
        acc[k] = mfma16_bf16(as_bf16x8(u32x4{al[0], al[1], al[2], al[3]}), B8, acc[k]);
      }
    }
    __syncthreads();
  }
  // lane holds D[row 4*qq + v][col n] of each N-tile
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int nt = wave + 4 * k;
    if (nt >= n_nt) break;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int rr = 4 * qq + v;
      const int bb = rb[rr];
      if (bb < 0) continue;
      const int ii = ri[rr] - gk * rph;
      const int hh = ii / g.n_q, j = ii % g.n_q;
      const int h = gk * g.G + hh;
      const size_t o = (((size_t)bb * g.n_q + j) * g.H_q + h) * g.d_h + nt * 16 + n;
      if (DT == STARKV_F32) ((float*)a.out)[o] = acc[k][v];
      else ((uint16_t*)a.out)[o] = f32_to_bf16(acc[k][v]);
    }
  }
}

// ===========================================================================

template <int LAT>
static void launch_values_nmt(int nmt, dim3 grid, dim3 block, hipStream_t s, const ValueArgs& va) {
  switch (nmt) {
    case 1: hipLaunchKernelGGL((k_values<LAT, 1>), grid, block, 0, s, va); break;
    case 2: hipLaunchKernelGGL((k_values<LAT, 2>), grid, block, 0, s, va); break;
    case 3: hipLaunchKernelGGL((k_values<LAT, 3>), grid, block, 0, s, va); break;
    case 4: hipLaunchKernelGGL((k_values<LAT, 4>), grid, block, 0, s, va); break;
    case 5: hipLaunchKernelGGL((k_values<LAT, 5>), grid, block, 0, s, va); break;
    case 6: hipLaunchKernelGGL((k_values<LAT, 6>), grid, block, 0, s, va); break;
    case 7: hipLaunchKernelGGL((k_values<LAT, 7>), grid, block, 0, s, va); break;
    default: hipLaunchKernelGGL((k_values<LAT, 8>), grid, block, 0, s, va); break;
  }
}

hipError_t launch_decode(const Layer& L, const DecodePlan& plan, const KtList& kts, const SeqTable& seq,
                         const void* q, void* out, const void* k_rows, const void* v_tiles, hipStream_t s) {
  const DecodeGeom& g = plan.g;
  const DecodeWs& w = plan.ws;
  // 1. query fragments
  QprojArgs qa;
  qa.q = q;
  qa.B_k = L.B_k;
  qa.scales = L.scales;
  qa.heads = L.heads();
  qa.qfrag = (uint8_t*)w.qfrag;
  qa.rowp = w.rowp;
  qa.g = g;
  qa.nkt_max = w.nkt_max;
  qa.kts = kts;
  dim3 gq(g.nct, g.B);
  {
  ProfScope ps("decode_qproj", s);
  if (L.dtype == STARKV_F32) {
    hipLaunchKernelGGL((k_qproj<STARKV_F32, STARKV_LATENT_F32>), gq, dim3(256), 0, s, qa);
  } else if (L.latent == STARKV_LATENT_BF16) {
    hipLaunchKernelGGL((k_qproj<STARKV_BF16, STARKV_LATENT_BF16>), gq, dim3(256), 0, s, qa);
  } else {
    hipLaunchKernelGGL((k_qproj<STARKV_BF16, STARKV_LATENT_MIX84>), gq, dim3(256), 0, s, qa);
  }
  }
  // 2. scores
  ScoreArgs sa;
  sa.k_rows = (const uint8_t*)k_rows;
  sa.qfrag = (const uint8_t*)w.qfrag;
  sa.rowp = w.rowp;
  sa.p = w.p;
  sa.cm = w.cm;
  sa.cl = w.cl;
  sa.g = g;
  sa.nkt_max = w.nkt_max;
  sa.kts = kts;
  sa.seq = seq;
  const int W = std::min(g.nct, 4);
  {
  ProfScope ps("decode_scores", s);
  if (L.latent == STARKV_LATENT_MIX84)
    hipLaunchKernelGGL(k_scores<STARKV_LATENT_MIX84>, dim3(w.total_chunks), dim3(64 * W), 0, s, sa);
  else if (L.latent == STARKV_LATENT_BF16)
    hipLaunchKernelGGL(k_scores<STARKV_LATENT_BF16>, dim3(w.total_chunks), dim3(64 * W), 0, s, sa);
  else
    hipLaunchKernelGGL(k_scores<STARKV_LATENT_F32>, dim3(w.total_chunks), dim3(64 * W), 0, s, sa);
  }
  // 3. values
  ValueArgs va;
  va.v_tiles = (const uint8_t*)v_tiles;
  va.p = w.p;
  va.cm = w.cm;
  va.cl = w.cl;
  va.zp = w.zp;
  va.sm = w.sm;
  va.sl = w.sl;
  va.g = g;
  va.seq = seq;
  va.cps = w.cps;
  va.bpw = w.blocks_per_wg;
  va.NB = L.v_rows / 32;
  va.V8 = L.V8;
  va.n8v = L.n8v;
  va.n4v = L.n4v;
  const int nmt = g.M_pad / 32;
  dim3 gv((va.NB + va.bpw - 1) / va.bpw, w.total_splits);
  dim3 bv(64 * va.bpw);
  {
  ProfScope ps("decode_values", s);
  if (L.latent == STARKV_LATENT_MIX84) launch_values_nmt<STARKV_LATENT_MIX84>(nmt, gv, bv, s, va);
  else if (L.latent == STARKV_LATENT_BF16) launch_values_nmt<STARKV_LATENT_BF16>(nmt, gv, bv, s, va);
  else launch_values_nmt<STARKV_LATENT_F32>(nmt, gv, bv, s, va);
  }
  // 4. merge + up-projection
  MergeArgs ma;
  ma.zp = w.zp;
  ma.sm = w.sm;
  ma.sl = w.sl;
  ma.B_vt = L.B_vt;
  ma.vscales = L.mix() ? L.scales + L.n_key : nullptr;
  ma.out = out;
  ma.g = g;
  ma.seq = seq;
  const int Rg = g.B * g.G * g.n_q;
  dim3 gm(g.H_kv, (Rg + 15) / 16);
  {
  ProfScope ps("decode_merge", s);
  if (L.dtype == STARKV_F32) hipLaunchKernelGGL(k_merge<STARKV_F32>, gm, dim3(256), 0, s, ma);
  else hipLaunchKernelGGL(k_merge<STARKV_BF16>, gm, dim3(256), 0, s, ma);
  }
  return hipGetLastError();
}

}  // namespace skv
