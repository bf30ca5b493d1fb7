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
// The K loop keeps two register batches of KU K-steps in flight: a batch's refill is issued right
// after its MFMAs, so each wave always has the next batch's loads outstanding.  Loads are
// unconditional and the loop has no branch but its own (rows past M and padding columns read
// row 0 / channel 0, K-steps past the end re-read the last one; their operands are zeroed after
// the load).
#include <algorithm>

#include "device_common.h"
#include "latent_gemm.h"
#include "profile.h"
#include "starkv_internal.h"

namespace skv {

template <int DT, int SW, bool MIX, int MODE = 0>
__global__ __launch_bounds__(512) void k_latent_gemm_skinny(GemmArgs a) {
  __shared__ float red[7][4][64];
  skinny_body<DT, SW, MIX, 8, MODE>(a, blockIdx.x, red);
}

// NW waves (4 or 8) split K; with 8, waves 4-7 hand their partial tiles to waves 0-3 first.
template <int DT, int MODE, int NW>
__global__ __launch_bounds__(64 * NW) void k_latent_gemm(GemmArgs a) {
  static_assert(NW == 4 || NW == 8, "waves per workgroup");
  __shared__ float part[4][4][16][64];  // [wave][32 x 32 quadrant][D element][lane]: 64 KiB
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int r = lane & 31, q = lane >> 5;
  int rt = blockIdx.x, ctl = blockIdx.y;
  if (a.xmap_rt > 0) {
    // 1-D grid, workgroups dealt to the eight XCDs in turn: the k-th workgroup of XCD x takes
    // row tile k mod xmap_rt of column tile x + 8 (k / xmap_rt), so the row tiles of a column
    // tile run one after another on one XCD and share its L2 copy of that slab of A
    const int k = blockIdx.x >> 3;
    rt = k % a.xmap_rt;
    ctl = (blockIdx.x & 7) + 8 * (k / a.xmap_rt);
    if (ctl * 64 >= a.NS) return;  // whole workgroup
  }
  const int mb = rt * 64, sb = ctl * 64;
  // operand rows of the tile's two 32-row halves (i) and two 32-slot halves (j)
  bool a_ok[2], b_ok[2];
  size_t a_base[2], b_base[2];
  uint16_t scb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int arow = mb + 32 * h + r;
    a_ok[h] = arow < a.M;
    a_base[h] = (size_t)(a_ok[h] ? arow : 0) * a.d;
    const int ch = slot_channel(a, sb + 32 * h + r);
    b_ok[h] = ch >= 0;
    b_base[h] = (size_t)(b_ok[h] ? ch : 0) * a.d;
    scb[h] = (MODE == 0 && a.latent == STARKV_LATENT_MIX84) ? scale_bits(a, ch) : (uint16_t)0;
  }
  // this wave's K-steps (16 each): an NW-th of the workgroup's part of K (one part, or with the
  // raw output ksplit parts, grid z)
  const int nk = a.d / 16;
  const int ksp = max(a.ksplit, 1);
  const int pk = (nk + ksp - 1) / ksp;
  const int k_lo = min(nk, (int)blockIdx.z * pk), k_hi = min(nk, k_lo + pk);
  const int per = (k_hi - k_lo + NW - 1) / NW;
  const int kb = k_lo + wave * per, ke = min(k_hi, kb + per);

  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.f;

  constexpr int NL = DT == STARKV_BF16 ? 1 : 2;  // 16-byte loads per operand fragment
  constexpr int KU = DT == STARKV_BF16 ? (MODE == 4 ? 2 : 4) : 2;  // K-steps per batch
  constexpr int NW2 = MODE == 4 ? 2 : 1;  // MODE 4 (bf16): second operand part (low) too
  struct Batch {
    u32x4 x[KU][2][NL], w[KU][2][NL], w2[KU][NW2][NL];
  };
  auto load = [&](Batch& f, int k0) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const size_t ko = (size_t)min(k0 + u, nk - 1) * 16 + 8 * q;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < NL; ++e) {
          if (DT == STARKV_BF16) {
            f.x[u][h][e] = ld16((const uint16_t*)a.X + a_base[h] + ko);
            f.w[u][h][e] = ld16((const uint16_t*)a.A_t + b_base[h] + ko);
            if (MODE == 4) f.w2[u][h % NW2][e] = ld16((const uint16_t*)a.A_t2 + b_base[h] + ko);
          } else {
            f.x[u][h][e] = ld16((const float*)a.X + a_base[h] + ko + 4 * e);
            f.w[u][h][e] = ld16((const float*)a.A_t + b_base[h] + ko + 4 * e);
          }
        }
    }
  };
  auto compute = [&](Batch& f, int k0) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const bool kin = k0 + u < ke;  // K-steps past the wave's range (clamped loads) add nothing
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < NL; ++e) {
          f.x[u][h][e] = a_ok[h] ? f.x[u][h][e] : u32x4{0, 0, 0, 0};
          f.w[u][h][e] = (b_ok[h] && kin) ? f.w[u][h][e] : u32x4{0, 0, 0, 0};
          if (MODE == 4) f.w2[u][h % NW2][e] = (b_ok[h] && kin) ? f.w2[u][h % NW2][e] : u32x4{0, 0, 0, 0};
        }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          if (DT == STARKV_BF16) {
            acc[x][y] = mfma32_bf16(as_bf16x8(f.x[u][x][0]), as_bf16x8(f.w[u][y][0]), acc[x][y]);
            if (MODE == 4) acc[x][y] = mfma32_bf16(as_bf16x8(f.x[u][x][0]), as_bf16x8(f.w2[u][y % NW2][0]), acc[x][y]);
          } else {
#pragma unroll
            for (int e = 0; e < NL; ++e)
#pragma unroll
              for (int c = 0; c < 4; ++c)
                acc[x][y] = mfma32_f32(__uint_as_float(f.x[u][x][e][c]), __uint_as_float(f.w[u][y][e][c]), acc[x][y]);
          }
        }
    }
  };
  if (kb < ke) {  // uniform
    Batch fa, fb;
    load(fa, kb);
    load(fb, kb + KU);
    for (int k0 = kb; k0 < ke; k0 += 2 * KU) {
      compute(fa, k0);
      load(fa, k0 + 2 * KU);
      compute(fb, k0 + KU);
      load(fb, k0 + 3 * KU);
    }
  }

  if (NW == 8) {
    // waves 4-7 hand their partial tiles to waves 0-3
    if (wave >= 4) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
          for (int v = 0; v < 16; ++v) part[wave - 4][2 * y + x][v][lane] = acc[x][y][v];
    }
    __syncthreads();
    if (wave < 4) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[x][y][v] += part[wave][2 * y + x][v][lane];
    }
    __syncthreads();
  }
  // add the four K-parts: with 4 waves wave w takes quadrant w (rows half w & 1, slots half
  // w >> 1); with 8, wave w takes half w >> 2 of the D elements of quadrant w & 3
  if (wave < 4) {
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int v = 0; v < 16; ++v) part[wave][2 * y + x][v][lane] = acc[x][y][v];
  }
  __syncthreads();
  constexpr int NVW = NW == 4 ? 16 : 8;  // D elements per lane in this wave's share
  const int qd = wave & 3;
  const int v0 = NW == 4 ? 0 : 8 * (wave >> 2);
  const int wm = qd & 1, wn = qd >> 1;
  float accq[NVW];
#pragma unroll
  for (int v = 0; v < NVW; ++v)
    accq[v] = part[0][qd][v0 + v][lane] + part[1][qd][v0 + v][lane] + part[2][qd][v0 + v][lane] +
              part[3][qd][v0 + v][lane];
  const int m0 = mb + 32 * wm;
  const int s0 = sb + 32 * wn;
  const uint16_t sc_bits = wn ? scb[1] : scb[0];

  // result: lane holds column n = r (slot s0 + r), rows d32_row(v, q)
  const int slot = s0 + r;
  const int chan = slot_channel(a, slot);

  if (MODE == 1) {
    // calibrate: absmax of this column over the 32 rows (rows >= M hold 0)
    float m = 0.f;
#pragma unroll
    for (int v = 0; v < NVW; ++v) m = fmaxf(m, fabsf(accq[v]));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    if (q == 0 && chan >= 0) atomicMax(a.absmax + chan, __float_as_uint(m));
    return;
  }

  float xs[NVW];
  int ms[NVW];
#pragma unroll
  for (int v = 0; v < NVW; ++v) {
    xs[v] = accq[v];
    ms[v] = m0 + d32_row(v0 + v, q);
  }
  if (MODE >= 2) {
    store_raw<MODE, NVW>(a, slot, xs, ms);
    return;
  }
  int ps[NVW];
#pragma unroll
  for (int v = 0; v < NVW; ++v) ps[v] = row_pos(a, ms[v]);
  store_latent<NVW>(a, slot, chan, sc_bits, xs, ms, ps);
}

// Epilogue of one wave's 32 x 32 quadrant of a 64 x 64 tile (rows mb + 32 wm .., slots
// sb + 32 wn ..): lane holds column n = r (slot), rows d32_row(v, q).  MODE 0 stores the cache
// rows (padding columns store zero), MODE 1 takes the per-channel absmax over the rows < M.
template <int MODE>
__device__ __forceinline__ void gemm_tile_epilogue(const GemmArgs& a, int mb, int sb, int wm, int wn, const f32x16& acc) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, q = lane >> 5;
  const int m0 = mb + 32 * wm;
  const int slot = sb + 32 * wn + r;
  const int chan = slot_channel(a, slot);
  if (MODE == 1) {
    float m = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) m = fmaxf(m, m0 + d32_row(v, q) < a.M ? fabsf(acc[v]) : 0.f);
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    if (q == 0 && chan >= 0) atomicMax(a.absmax + chan, __float_as_uint(m));
    return;
  }
  const uint16_t sc_bits = a.latent == STARKV_LATENT_MIX84 ? scale_bits(a, chan) : (uint16_t)0;
  float xs[16];
  int ms[16], ps[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    xs[v] = chan >= 0 ? acc[v] : 0.f;
    ms[v] = m0 + d32_row(v, q);
    ps[v] = row_pos(a, ms[v]);
  }
  store_latent<16>(a, slot, chan, sc_bits, xs, ms, ps);
}

// bf16 operands, d a multiple of 64: the X and A_t tiles stream through LDS.  Workgroup tile
// T token rows x T cache slots (T = 64 or 128), four waves in 2 x 2 quadrants of T/2 x T/2, each
// in 32 x 32 MFMA tiles over the whole K (no partial sums to add).  K advances in blocks of 64:
// a block's two operand tiles (T rows of 128 bytes each) arrive by 16-byte LDS DMA into a ring of
// NST stages, NST - 1 blocks ahead of the MFMAs, so the loads of a CU run deep without holding
// registers.  In a tile, row R's eight 16-byte K-chunks sit at chunk c ^ ((R >> 1) & 7): the 16
// lanes of a fragment read (rows R .. R + 15, one chunk) then hit 16 different 4-bank groups.
// Rows past M and padding columns load row 0 / channel 0 (valid addresses); such rows are never
// stored and padding columns store zero.  Grid as k_latent_gemm (MODE 0: store, MODE 1: absmax).
// On MI355X the kernel is bound by the operand bytes each CU pulls from L2 (about 40 GB/s per
// workgroup): a 128 x 128 tile pulls half the bytes per flop of a 64 x 64 one and serves the
// appends of many rows; short blocks of rows keep 64 x 64 tiles for their workgroup count.
template <int MODE, int NST, int T = 64>
__global__ __launch_bounds__(256) void k_latent_gemm_dma(GemmArgs a) {
  constexpr int TB = T * 128;      // bytes of one operand tile of a K block
  constexpr int LP = T / 32;       // 16-byte DMA loads per wave per tile
  constexpr int MQ = T / 64;       // 32 x 32 MFMA tiles per wave quadrant, each way (1 or 2)
  static_assert(T == 64 || T == 128, "tile");
  extern __shared__ __align__(16) uint8_t ring_raw[];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int r = lane & 31, q = lane >> 5;
  int rt = blockIdx.x, ctl = blockIdx.y;
  if (a.xmap_rt > 0) {
    const int k = blockIdx.x >> 3;
    rt = k % a.xmap_rt;
    ctl = (blockIdx.x & 7) + 8 * (k / a.xmap_rt);
    if (ctl * T >= a.NS) return;  // whole workgroup
  }
  const int mb = rt * T, sb = ctl * T;
  // this lane's DMA sources: load jj of the wave fills tile slot i = 64 (LP wave + jj) + lane,
  // i.e. row i / 8 and stored chunk i % 8, which holds K-chunk (i % 8) ^ ((row >> 1) & 7)
  const uint16_t* xsrc[LP];
  const uint16_t* wsrc[LP];
#pragma unroll
  for (int jj = 0; jj < LP; ++jj) {
    const int i = 64 * (LP * wave + jj) + lane;
    const int row = i >> 3;
    const int kc = (i & 7) ^ ((row >> 1) & 7);
    const int xr = mb + row < a.M ? mb + row : 0;
    const int ch = slot_channel(a, sb + row);
    xsrc[jj] = (const uint16_t*)a.X + (size_t)xr * a.d + 8 * kc;
    wsrc[jj] = (const uint16_t*)a.A_t + (size_t)(ch >= 0 ? ch : 0) * a.d + 8 * kc;
  }
  const int nkb = a.d / 64;
  const uint32_t ring0 = lds_addr(ring_raw);
  auto issue = [&](int kb, int st) {
    kb = min(kb, nkb - 1);  // past the end: reload the last block (never read)
    const uint32_t xb = ring0 + st * 2 * TB, wb = xb + TB;
#pragma unroll
    for (int jj = 0; jj < LP; ++jj) {
      lds_dma16(xsrc[jj] + 64 * kb, xb + 1024 * (LP * wave + jj));
      lds_dma16(wsrc[jj] + 64 * kb, wb + 1024 * (LP * wave + jj));
    }
  };
  const int wm = wave & 1, wn = wave >> 1;
  int xo[MQ], xsw[MQ], wo[MQ], wsw[MQ];
#pragma unroll
  for (int i = 0; i < MQ; ++i) {
    const int xrow = (T / 2) * wm + 32 * i + r, wrow = (T / 2) * wn + 32 * i + r;
    xo[i] = xrow * 128;
    wo[i] = wrow * 128;
    xsw[i] = (xrow >> 1) & 7;
    wsw[i] = (wrow >> 1) & 7;
  }
  f32x16 acc[MQ][MQ];
#pragma unroll
  for (int i = 0; i < MQ; ++i)
#pragma unroll
    for (int j = 0; j < MQ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
#pragma unroll
  for (int u = 0; u < NST - 1; ++u) issue(u, u);
  for (int kb = 0; kb < nkb; ++kb) {
    vm_wait<2 * LP * (NST - 2)>();  // this wave's loads of block kb are in
    __builtin_amdgcn_s_barrier();   // ... and every wave's; block kb - 1's stage is free
    asm volatile("" ::: "memory");
    issue(kb + NST - 1, (kb + NST - 1) % NST);
    const uint8_t* xt = ring_raw + (kb % NST) * 2 * TB;
    const uint8_t* wt = xt + TB;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = 2 * ks + q;
      u32x4 xf[MQ], wf[MQ];
#pragma unroll
      for (int i = 0; i < MQ; ++i) {
        xf[i] = *(const u32x4*)(xt + xo[i] + 16 * (c ^ xsw[i]));
        wf[i] = *(const u32x4*)(wt + wo[i] + 16 * (c ^ wsw[i]));
      }
#pragma unroll
      for (int i = 0; i < MQ; ++i)
#pragma unroll
        for (int j = 0; j < MQ; ++j) acc[i][j] = mfma32_bf16(as_bf16x8(xf[i]), as_bf16x8(wf[j]), acc[i][j]);
    }
  }
  vm_wait<0>();  // the trailing reloads land before the workgroup ends
  // (sub-tiles named with constant indexes: a loop the compiler leaves rolled would index the
  // accumulators dynamically, through scratch)
  const int m0 = mb + (T / 2) * wm, s0 = sb + (T / 2) * wn;
  gemm_tile_epilogue<MODE>(a, m0, s0, 0, 0, acc[0][0]);
  if (MQ > 1) {
    gemm_tile_epilogue<MODE>(a, m0, s0 + 32, 0, 0, acc[0][MQ - 1]);
    gemm_tile_epilogue<MODE>(a, m0 + 32, s0, 0, 0, acc[MQ - 1][0]);
    gemm_tile_epilogue<MODE>(a, m0 + 32, s0 + 32, 0, 0, acc[MQ - 1][MQ - 1]);
  }
}

__global__ void k_fill_u32(uint32_t* p, int n, uint32_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(256) void k_finish_scales(const uint32_t* __restrict__ absmax, const int* __restrict__ src,
                                                       const int* __restrict__ n8, int n8v, int H_kv, int n_lat,
                                                       float qmax_hi, float qmax_lo, uint16_t* __restrict__ scales) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= n_lat) return;
  const int s = src[c];
  const int g = s >> 16, k = s & 0xFFFF;
  const bool is8 = (g < H_kv) ? (k < n8[g]) : (k < n8v);
  const float q = is8 ? qmax_hi : qmax_lo;
  scales[c] = f32_to_f16(__uint_as_float(absmax[c]) / q);
}

void fill_gemm_args(const Layer& L, GemmArgs& a, const void* X, int M) {
  a.X = X;
  a.A_t = L.A_t;
  a.slot_chan = L.d_slot_chan;
  a.M = M;
  a.d = L.d;
  a.NS = L.key_slots + L.val_slots;
  a.xmap_rt = 0;
  a.key_slots = L.key_slots;
  a.K8 = L.K8;
  a.V8 = L.V8;
  a.pack3 = L.pack3;
  a.K4 = L.K4;
  a.V4 = L.V4;
  a.qmax_hi = L.qmax_hi;
  a.qmax_lo = L.qmax_lo;
  a.n_key = L.n_key;
  a.r_v = L.r_v;
  a.latent = L.latent;
}

void fill_append_args(const Layer& L, const starkv_cache& c, GemmArgs& a, const void* X_new, int B, int n_new,
                      const int32_t* lens, const int32_t* lens_dev, int lens_sub) {
  fill_gemm_args(L, a, X_new, B * n_new);
  a.n_new = n_new;
  a.T_max = c.T_max;
  a.k_row_bytes = L.k_row_bytes;
  a.v_rows = L.v_rows;
  a.k_rows = (uint8_t*)c.k_rows;
  a.v_tiles = (uint8_t*)c.v_tiles;
  a.scales = L.scales;
  for (int b = 0; b < B; ++b) a.lens[b] = lens[b];
  a.lens_dev = lens_dev;
  a.lens_sub = lens_sub;
}

hipError_t launch_calibrate(const Layer& L, const void* X_cal, int n_cal, uint16_t* scales_out, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_u32, dim3((L.n_lat + 255) / 256), dim3(256), 0, s, L.d_absmax, L.n_lat, 0u);
  GemmArgs a = {};
  fill_gemm_args(L, a, X_cal, n_cal);
  a.absmax = L.d_absmax;
  dim3 grid((n_cal + 63) / 64, (a.NS + 63) / 64);
  if (L.dtype == STARKV_BF16 && L.d % 64 == 0)
    hipLaunchKernelGGL((k_latent_gemm_dma<1, 4>), grid, dim3(256), 4 * 2 * 8192, s, a);
  else if (L.dtype == STARKV_BF16) hipLaunchKernelGGL((k_latent_gemm<STARKV_BF16, 1, 4>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_latent_gemm<STARKV_F32, 1, 4>), grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_finish_scales, dim3((L.n_lat + 255) / 256), dim3(256), 0, s, (const uint32_t*)L.d_absmax,
                     (const int*)L.d_src, (const int*)L.d_n8, L.n8v, L.H_kv, L.n_lat, (float)L.qmax_hi,
                     (float)L.qmax_lo, scales_out);
  return hipGetLastError();
}

// One launch with dynamic LDS, with the timing events attached when given.
template <typename A>
static hipError_t launch_lds(const ProfScope& ps, void (*kernel)(A), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                             A arg) {
  void* argv[] = {(void*)&arg};
  if (ps.start() && ps.stop())
    return hipExtLaunchKernel((const void*)kernel, grid, block, argv, lds, s, ps.start(), ps.stop(), 0);
  return hipLaunchKernel((const void*)kernel, grid, block, argv, lds, s);
}

// The DMA append GEMM (bf16, d a multiple of 64): 128 x 128 tiles when they still give every CU
// at least two workgroups; otherwise 64 x 64 tiles, with the XCD-aware grid for a short block of
// rows (the row tiles of a column tile run on one XCD and share its L2 copy of that slab of A).
static hipError_t launch_dma_append(const ProfScope& ps, GemmArgs& a, int M, hipStream_t s) {
  const int r128 = (M + 127) / 128, c128 = (a.NS + 127) / 128;
  if ((long)r128 * c128 >= 512)
    return launch_lds(ps, k_latent_gemm_dma<0, 3, 128>, dim3(r128, c128), dim3(256), 3 * 2 * 128 * 128, s, a);
  const int n_rt = (M + 63) / 64, n_ct = (a.NS + 63) / 64;
  if (n_rt <= 16) {
    a.xmap_rt = n_rt;
    return launch_lds(ps, k_latent_gemm_dma<0, 4>, dim3(8 * n_rt * ((n_ct + 7) / 8)), dim3(256), 4 * 2 * 8192, s, a);
  }
  return launch_lds(ps, k_latent_gemm_dma<0, 4>, dim3(n_rt, n_ct), dim3(256), 4 * 2 * 8192, s, a);
}

hipError_t launch_append(const Layer& L, const starkv_cache& c, const void* X_new, int B, int n_new,
                         const int32_t* lens, hipStream_t s, const int32_t* lens_dev, int lens_sub) {
  GemmArgs a = {};
  fill_append_args(L, c, a, X_new, B, n_new, lens, lens_dev, lens_sub);
  ProfScope ps("append");
  hipError_t e;
  const bool mix = L.mix();
  if (L.pack3 && B * n_new <= 16) {  // (packed layers: bf16, d a multiple of 64)
    // packed 3-bit planes from the 16-slot skinny tiles (the 8-slot form is not used: its key
    // plane words would take four writers)
    e = launch_k(ps, k_latent_gemm_skinny<STARKV_BF16, 16, true>, dim3((a.NS + 15) / 16), dim3(512), s, a);
  } else if (L.pack3) {
    // packed 3-bit planes from the GEMM tiles (32-slot groups in the lanes of a half-wave)
    e = launch_dma_append(ps, a, B * n_new, s);
  } else if (B * n_new <= 8 && L.d % 64 == 0) {
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
  } else if (L.dtype == STARKV_BF16 && L.d % 64 == 0) {
    // bf16: operands staged through LDS
    e = launch_dma_append(ps, a, B * n_new, s);
  } else {
    const int n_rt = (B * n_new + 63) / 64, n_ct = (a.NS + 63) / 64;
    if (n_rt <= 16) {
      // a short block of tokens: XCD-aware grid (each slab of A fetched into one L2) and eight
      // waves per workgroup (few workgroups: K split eight ways)
      a.xmap_rt = n_rt;
      const dim3 grid(8 * n_rt * ((n_ct + 7) / 8));
      if (L.dtype == STARKV_BF16) e = launch_k(ps, k_latent_gemm<STARKV_BF16, 0, 8>, grid, dim3(512), s, a);
      else e = launch_k(ps, k_latent_gemm<STARKV_F32, 0, 8>, grid, dim3(512), s, a);
    } else {
      const dim3 grid(n_rt, n_ct);
      if (L.dtype == STARKV_BF16) e = launch_k(ps, k_latent_gemm<STARKV_BF16, 0, 4>, grid, dim3(256), s, a);
      else e = launch_k(ps, k_latent_gemm<STARKV_F32, 0, 4>, grid, dim3(256), s, a);
    }
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

// Hidden-state query projection through the absorbed factors: out[m][c] = sum_e x[m][e] wqk[c][e]
// for the M = B n_q rows and the NS = G n_key absorbed columns, on the append GEMMs with a raw
// fp32 epilogue.  bf16 layers keep the factors as bf16 high and low parts (wqk_hi, wqk_lo), which
// both forms load together in one pass (MODE 4: one MFMA per part into the same accumulators).
// One launch, with the timing events attached when given.
template <typename A>
static hipError_t launch_ev(void (*kernel)(A), dim3 grid, dim3 block, hipStream_t s, A arg, hipEvent_t start,
                            hipEvent_t stop) {
  void* argv[] = {(void*)&arg};
  if (start || stop) return hipExtLaunchKernel((const void*)kernel, grid, block, argv, 0, s, start, stop, 0);
  return hipLaunchKernel((const void*)kernel, grid, block, argv, 0, s);
}

hipError_t launch_hidden_query(const Layer& L, const void* x, int M, const void* wqk_hi, const void* wqk_lo,
                               float* out, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  GemmArgs a = {};
  a.X = x;
  a.M = M;
  a.d = L.d;
  a.NS = L.G * L.n_key;
  a.n_key = a.NS;  // every column is a live channel (slot = channel)
  a.key_slots = a.NS;
  a.r_v = 0;
  a.latent = STARKV_LATENT_F32;  // not the int8/int4 table layout
  a.n_new = 1;
  a.xmap_rt = 0;
  a.out_f32 = out;
  const bool bf = L.dtype == STARKV_BF16;
  if (M <= 16 && L.d % 32 == 0) {
    // skinny form, one launch: bf16 loads the high and low parts together (MODE 4); twice the
    // workgroups (8 slots each) for at most 8 rows, as in the append
    a.A_t = wqk_hi;
    a.A_t2 = wqk_lo;
    if (M <= 8 && L.d % 64 == 0)
      return launch_ev(bf ? k_latent_gemm_skinny<STARKV_BF16, 8, false, 4> : k_latent_gemm_skinny<STARKV_F32, 8, false, 2>,
                       dim3((a.NS + 7) / 8), dim3(512), s, a, start, stop);
    return launch_ev(bf ? k_latent_gemm_skinny<STARKV_BF16, 16, false, 4> : k_latent_gemm_skinny<STARKV_F32, 16, false, 2>,
                     dim3((a.NS + 15) / 16), dim3(512), s, a, start, stop);
  }
  // tiled form, one launch: bf16 loads the high and low parts together (MODE 4); K split over
  // hidden_query_parts workgroups per tile, each storing its own partial sums
  const int n_rt = (M + 63) / 64, n_ct = (a.NS + 63) / 64;
  a.A_t = wqk_hi;
  a.A_t2 = wqk_lo;
  a.ksplit = hidden_query_parts(M, a.NS);
  a.out_part = (size_t)M * a.NS;
  a.xmap_rt = n_rt <= 16 ? n_rt : 0;
  if (a.xmap_rt > 0)
    return launch_ev(bf ? k_latent_gemm<STARKV_BF16, 4, 8> : k_latent_gemm<STARKV_F32, 2, 8>,
                     dim3(8 * n_rt * ((n_ct + 7) / 8), 1, a.ksplit), dim3(512), s, a, start, stop);
  hipError_t e = launch_ev(bf ? k_latent_gemm<STARKV_BF16, 4, 4> : k_latent_gemm<STARKV_F32, 2, 4>,
                           dim3(n_rt, n_ct, a.ksplit), dim3(256), s, a, start, stop);
  return e;
}

int hidden_query_parts(int M, int NS) {
  if (M <= 16) return 1;  // the skinny form
  const int tiles = ((M + 63) / 64) * ((NS + 63) / 64);
  // about two workgroups per CU, at most six parts (C4's 80 tiles: 1, 3, 6 parts measured 76, 66,
  // 55 us for the GEMM; the query projection then adds the parts)
  return std::max(1, std::min(6, 512 / tiles));
}

}  // namespace skv
