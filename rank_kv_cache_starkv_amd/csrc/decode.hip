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

#include <string.h>

#include <algorithm>
#include <numeric>
#include <cstdlib>

#include "device_common.h"
#include "latent_gemm.h"
#include "profile.h"
#include "starkv_internal.h"

namespace skv {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Value splits of a ragged batch in XCD order.  The value workgroups go to the eight XCDs in turn
// by grid position, and each XCD runs its share on its own 32 CUs, so an order that ignores the
// split lengths can leave one XCD with far more work than another.  Deal the splits (cps chunks
// each, the last of a sequence shorter) longest first, each to the XCD with the least work so far
// (the n_sl workgroups of a split stay on one XCD and share its L2), and estimate the time as the
// latest per-XCD finish when each XCD's workgroups, in that order, are list-scheduled onto its
// workgroup slots at a cost of (chunks + a fixed overhead).  Returns the estimate in chunk units,
// or -1 when the order needs more than kMaxVPos grid positions; fills *vo when given.  The
// estimate stops early (returning a value above `limit`) once it exceeds `limit`.
constexpr float kWgOvh = 2.f;  // fixed cost of a value workgroup, in chunks
static double order_splits(const SeqTable& seq, int B, int cps, int n_sl, ValueOrder* vo, float limit = 1e30f) {
  constexpr int kXcd = 8, kSlots = 64;  // 32 CUs per XCD, two value workgroups on each
  std::vector<std::pair<int, int>> sp;  // (-chunks, split)
  for (int b = 0, sg = 0; b < B; ++b) {
    const int nc = seq.chunk_off[b + 1] - seq.chunk_off[b];
    for (int c0 = 0; c0 < nc; c0 += cps) sp.emplace_back(-std::min(cps, nc - c0), sg++);
  }
  const int n = (int)sp.size();
  if (ceil_div(n, kXcd) * kXcd > kMaxVPos) return -1;
  std::sort(sp.begin(), sp.end());  // longest first, then by split
  float load[kXcd] = {};
  int cnt[kXcd] = {};
  std::vector<uint8_t> xcd_of(n);
  for (int i = 0; i < n; ++i) {
    int x = 0;
    for (int y = 1; y < kXcd; ++y)
      if (load[y] < load[x]) x = y;
    xcd_of[i] = (uint8_t)x;
    ++cnt[x];
    load[x] += (float)(-sp[i].first) + kWgOvh;
  }
  const int n_pos = kXcd * *std::max_element(cnt, cnt + kXcd);
  if (n_pos > kMaxVPos) return -1;
  // no XCD can finish before its work spread evenly over its slots
  const float lb = *std::max_element(load, load + kXcd) * n_sl / kSlots;
  if (!vo && lb > limit) return lb;
  float span = 0.f;
  for (int x = 0; x < kXcd; ++x) {
    float heap[kSlots] = {};  // slot free times, a binary min-heap
    for (int i = 0; i < n; ++i) {
      if (xcd_of[i] != x) continue;
      const float d = (float)(-sp[i].first) + kWgOvh;
      for (int k = 0; k < n_sl; ++k) {
        // the earliest free slot takes the workgroup: raise the root by d and sift it down
        const float v = heap[0] + d;
        int j = 0;
        for (;;) {
          int c = 2 * j + 1;
          if (c >= kSlots) break;
          if (c + 1 < kSlots && heap[c + 1] < heap[c]) ++c;
          if (heap[c] >= v) break;
          heap[j] = heap[c];
          j = c;
        }
        heap[j] = v;
        span = std::max(span, v);
      }
      if (!vo && span > limit) return span;
    }
  }
  if (vo) {
    vo->n = n_pos;
    for (int p = 0; p < n_pos; ++p) vo->sg[p] = 0xFFFF;
    int j[kXcd] = {};
    for (int i = 0; i < n; ++i) {
      const int x = xcd_of[i];
      vo->sg[kXcd * j[x]++ + x] = (uint16_t)sp[i].second;
    }
  }
  return span;
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
  g.d = L.d;
  g.H_q = L.H_q;
  g.H_kv = L.H_kv;
  g.n_key = L.n_key;
  g.r_v = L.r_v;
  g.K8 = L.K8;
  g.K4 = L.K4;
  g.K3 = L.K3;
  g.pack3 = L.pack3;
  // the packed layout's value kernel takes one tile of at most 32 query rows per sequence
  if (L.pack3 && g.M_pad > 32) return STARKV_EUNSUPPORTED;
  g.key_kt = L.key_kt;
  g.key_kpos = L.key_kpos;
  g.k_row_bytes = L.k_row_bytes;
  g.v_rows = L.v_rows;
  g.v_tile_bytes = L.v_tile_bytes;
  g.T_max = T_max;
  g.rv_ld = ceil_div(L.r_v, 32) * 32;
  g.latent = L.latent;
  g.dtype = L.dtype;
  g.qscale = (float)(1.4426950408889634 / sqrt((double)L.d_h));

  // K-tiles touched by every 16-row column tile (block-diagonal query fragments)
  memset(kts, 0, sizeof(*kts));
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
      // int8 (or packed: outlier nibble) positions, then int4 (or packed: 3-bit) positions
      const int base_lo = L.pack3 ? L.K4 : L.K8;
      mark(L.off8[g_lo], L.off8[g_hi + 1]);
      mark(base_lo + L.off4[g_lo], base_lo + L.off4[g_hi + 1]);
    } else {
      mark(L.koff[g_lo], L.koff[g_hi + 1]);
    }
    // the used K-tiles as (at most two) contiguous runs
    int n = 0, runs = 0;
    for (int kt = 0; kt < 256; ++kt) {
      if (!used[kt]) continue;
      if (kt == 0 || !used[kt - 1]) {
        if (runs == 0) kts->s0[ct] = kt;
        else if (runs == 1) kts->s1[ct] = kt;
        else return STARKV_EUNSUPPORTED;
        ++runs;
      }
      if (runs == 1) kts->n0[ct] = n + 1;
      ++n;
    }
    if (n > kMaxKT) return STARKV_EUNSUPPORTED;
    if (runs == 1) kts->s1[ct] = kts->s0[ct] + kts->n0[ct];
    kts->n[ct] = n;
    nkt_max = std::max(nkt_max, n);
  }

  // chunks and splits
  const int NB = L.v_rows / 32;
  const int bpw = NB >= 16 ? 4 : (NB >= 8 ? 2 : 1);
  int n_slices = ceil_div(NB, bpw);
  DecodeWs& w = P->ws;
  // one-M-tile value kernel: slices of up to nbw8 one-N-tile blocks and nbw4 int4 blocks
  {
    // int8 blocks are half the bytes of bf16 ones: bigger slices (measured on MI355X)
    w.nbw8 = L.mix() ? 4 : 2;
    w.nbw4 = 2;
  }
  const int nb8 = L.mix() ? L.V8 / 32 : NB;
  w.n_sl8 = ceil_div(nb8, w.nbw8);
  // int4 blocks: the rest, or with the packed layout the outlier blocks (V4 / 64) before the
  // 3-bit N-tiles (V3 / 32, two per slice)
  w.n_sl4 = L.mix() ? ceil_div((L.pack3 ? L.V4 / 64 : NB) - nb8, w.nbw4) : 0;
  w.n_sl3 = L.pack3 ? ceil_div(L.V3 / 32, 2) : 0;
  if (g.M_pad == 32) n_slices = w.n_sl8 + w.n_sl4 + w.n_sl3;
  // many query rows (bf16, int8/int4): groups of four 32-channel N-tiles
  const int n_nt = L.mix() ? nb8 + 2 * (NB - nb8) : NB;
  w.n_grp = ceil_div(n_nt, g.M_pad <= 160 ? 8 : 4);  // N-tiles per workgroup: 4 waves x (2, or 1 past 5 row tiles)
  if (g.M_pad > 32 && L.latent != STARKV_LATENT_F32) n_slices = w.n_grp;
  int total_chunks = 0, max_chunks = 0;
  seq->chunk_off[0] = 0;
  seq->blk_off[0] = 0;
  for (int b = 0; b < B; ++b) {
    seq->lens[b] = lens[b];
    const int nc = ceil_div(lens[b], kTC);
    seq->chunk_off[b + 1] = seq->chunk_off[b] + nc;
    seq->blk_off[b + 1] = seq->blk_off[b] + ceil_div(nc, 4);
    total_chunks += nc;
    max_chunks = std::max(max_chunks, nc);
  }
  // splits: aim at ~512 value workgroups (two per CU), at least 8 tiles (two per wave) per split
  const int target_wg = 512;
  int cps = std::max(8, ceil_div(total_chunks, std::max(1, target_wg / n_slices)));
  cps = std::max(cps, ceil_div(max_chunks, kMaxSplitsPerSeq));
  // at most 4 splits per sequence while that keeps >= 256 value workgroups: longer-lived
  // workgroups, and the split merge then folds into the up-projection
  if (B * 4 * n_slices >= 256) cps = std::max(cps, ceil_div(max_chunks, 4));
  // ragged lengths (value kernels that take an explicit order): the split length whose
  // longest-first XCD deal has the least estimated time, from the fewest splits the rules
  // above allow up to one split per sequence
  bool uniform = true;
  for (int b = 1; b < B; ++b)
    if (lens[b] != lens[0]) uniform = false;
  const bool ordered = !uniform && !(g.M_pad > 32 && L.latent == STARKV_LATENT_F32);
  int cps_lo = std::max(8, ceil_div(max_chunks, kMaxSplitsPerSeq));
  if (B * 4 * n_slices >= 256) cps_lo = std::max(cps_lo, ceil_div(max_chunks, 4));
  bool have_order = false;
  if (ordered) {
    double best_t = 0;
    for (int c = std::min(cps_lo, max_chunks);; c = std::min(max_chunks, c + std::max(1, c / 8))) {
      // a longer split takes at least its own length: no later one can win
      if (have_order && best_t < c + kWgOvh) break;
      const double t = order_splits(*seq, B, c, n_slices, nullptr, have_order ? (float)best_t : 1e30f);
      if (t >= 0 && (!have_order || t <= best_t)) {  // ties: the longer split (fewer partials)
        have_order = true;
        best_t = t;
        cps = c;
      }
      if (c >= max_chunks) break;
    }
  }
  P->vo.n = 0;
  if (ordered && order_splits(*seq, B, cps, n_slices, &P->vo) < 0) P->vo.n = 0;
  int total_splits = 0;
  seq->split_off[0] = 0;
  for (int b = 0; b < B; ++b) {
    const int nc = seq->chunk_off[b + 1] - seq->chunk_off[b];
    seq->split_off[b + 1] = seq->split_off[b] + ceil_div(nc, cps);
    total_splits += ceil_div(nc, cps);
  }
  seq->uni = uniform ? 1 : 0;
  seq->u_len = lens[0];
  seq->lens_dev = nullptr;
  seq->len_lo = n_q;
  seq->u_nch = seq->chunk_off[1];
  seq->u_nspl = seq->split_off[1];
  seq->u_nblk = seq->blk_off[1];

  // workspace
  const int esz_p = L.latent == STARKV_LATENT_F32 ? 4 : 2;
  size_t o = 0;
  const size_t o_qfrag = o; o = align256(o + (size_t)B * g.nct * nkt_max * 2048);
  const size_t o_rowp = o; o = align256(o + (size_t)B * g.M_pad * 16);
  const size_t o_p = o; o = align256(o + (size_t)total_chunks * g.M_pad * kTC * esz_p);
  const size_t o_cm = o; o = align256(o + (size_t)total_chunks * g.M_pad * 4);
  const size_t o_cl = o; o = align256(o + (size_t)total_chunks * g.M_pad * 4);
  const size_t o_zp = o; o = align256(o + (size_t)total_splits * g.M_pad * g.rv_ld * (L.mix() ? 2 : 4));
  const size_t o_sl = o; o = align256(o + (size_t)total_splits * g.M_pad * 4);
  const size_t o_sm = o; o = align256(o + (size_t)total_splits * g.M_pad * 4);
  const size_t o_zt = o; o = align256(o + (size_t)B * g.M_pad * g.rv_ld * 4);
  w.qraw_parts = hidden_query_parts(B * n_q, L.G * L.n_key);
  const size_t o_qraw = o; o = align256(o + (size_t)w.qraw_parts * B * n_q * L.G * L.n_key * 4);
  P->ws_bytes = o;
  uint8_t* base = (uint8_t*)ws_base;
  w.qfrag = base + o_qfrag;
  w.rowp = (float*)(base + o_rowp);
  w.p = base + o_p;
  w.cm = (float*)(base + o_cm);
  w.cl = (float*)(base + o_cl);
  w.zp = (void*)(base + o_zp);
  w.sl = (float*)(base + o_sl);
  w.sm = (float*)(base + o_sm);
  w.zt = (float*)(base + o_zt);
  w.qraw = (float*)(base + o_qraw);
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
  const void* q;        // queries [B][n_q][H_q][d_h], or hidden states [B][n_q][d] when wqk is set
  const void* B_k;
  const float* wqk;     // absorbed path: non-null (the projection x wqk^T is in qraw)
  const float* qraw;    // [qraw_parts][B n_q][G n_key] hidden-state query projection (K parts)
  int qraw_parts;
  const uint16_t* scales;
  HeadTables heads;
  uint8_t* qfrag;
  float* rowp;
  DecodeGeom g;
  int nkt_max;
  int qp_w;  // rows per workgroup of the query-projection launch
  KtList kts;
};

template <int DT>
__device__ __forceinline__ float ldx(const void* p, size_t i) {
  if (DT == STARKV_F32) return ((const float*)p)[i];
  return bf16_to_f32(((const uint16_t*)p)[i]);
}

// A workgroup takes rows of one KV head g: the rows of g in one sequence are its G query heads
// x n_q queries, and the workgroup's rows are a range of the flattened (sequence, row) index
// u = b * G n_q + row, so one workgroup may take the rows of several sequences.  A row's
// quantisation scale depends on that row alone.  Each row owns the 16-byte fragment chunks of its
// column in every K-tile of its column tile; the workgroup writes exactly those chunks (zeros
// outside g's segment), so no two workgroups write the same bytes.
constexpr int kQpRB = 8;      // query-projection rows per batch (fused step front)
constexpr int kQpRB16 = 16;   // ... (query-projection launch)
constexpr int kQpRMAX = 256;  // max rank (<= d_h <= 256)
template <int RB>
struct QprojSharedT {
  float qh[RB][kQpRMAX];
  uint32_t amax[RB];  // bits of each row's max |q^| (non-negative floats order as integers)
};

// Two-part int8 split of a latent query element x of a row with max |q^| = m:
// x ~ rho (hi + lo / 254), rho = m / 127 (1 for a zero row).
__device__ __forceinline__ float qrow_rho(uint32_t amax_bits) {
  const float m = __uint_as_float(amax_bits);
  return m > 0.f ? m / 127.f : 1.f;
}
__device__ __forceinline__ void qsplit(float x, float rho, int& hi, int& lo) {
  const float h = fminf(fmaxf(__builtin_rintf(x / rho), -127.f), 127.f);
  const float l = fminf(fmaxf(__builtin_rintf((x - h * rho) * (254.f / rho)), -127.f), 127.f);
  hi = (int)h;
  lo = (int)l;
}
using QprojShared = QprojSharedT<kQpRB>;

// Body of the query projection for the rows u in [u_lo, u_hi) of KV head gk (u = b G n_q + row of
// g in sequence b), RB rows per batch, with NT threads.
template <int DT, int LAT, int NT, bool HID = false, int RB = kQpRB>
__device__ __forceinline__ void qproj_body(const QprojArgs& a, int gk, int u_lo, int u_hi, QprojSharedT<RB>& sh) {
  constexpr int NWV = NT / 64;
  constexpr int SUB = 4;                            // lanes per dot product
  constexpr int EPL = DT == STARKV_F32 ? 4 : 8;    // elements per 16-byte load
  constexpr int NX = 4;                             // 16-byte loads per operand per lane per round
  constexpr int CH = SUB * NX * EPL;                // elements of d_h per load round
  auto& qh = sh.qh;
  auto& amax = sh.amax;
  const DecodeGeom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int rph = g.G * g.n_q;
  const int c0 = ld_uniform(a.heads.koff + gk);
  const int r = ld_uniform(a.heads.koff + gk + 1) - c0;
  const int n8g = (LAT == STARKV_LATENT_MIX84) ? ld_uniform(a.heads.n8 + gk) : 0;
  const int o8 = (LAT == STARKV_LATENT_MIX84) ? ld_uniform(a.heads.off8 + gk) : 0;
  const int o4 = (LAT == STARKV_LATENT_MIX84) ? ld_uniform(a.heads.off4 + gk) : 0;

  for (int ub0 = u_lo; ub0 < u_hi; ub0 += RB) {
    const int nrows = min(RB, u_hi - ub0);
    __syncthreads();  // the previous batch is done with qh and amax
    if (tid < RB) amax[tid] = 0u;
    __syncthreads();
    // q^[n][k] = (q_n . B_k[c0 + k]) * scale * log2(e)/sqrt(d_h): SUB adjacent lanes per dot
    // product, lane sub taking the 16-byte pieces sub, sub + SUB, ... of the q row and the B_k
    // row (loaded together, CH elements per round, unconditional loads at clamped offsets, masked
    // in the FMAs); the SUB lanes of a product are active together (NT and the item count are
    // multiples of SUB), so they add their parts with shuffles
    for (int ps = tid; ps < nrows * r * SUB; ps += NT) {
      const int p = ps / SUB, sub = ps % SUB;
      const int n = p / r, k = p % r;
      const int b = (ub0 + n) / rph, lr = (ub0 + n) - b * rph;  // sequence, row of g
      if (HID) {
        // hidden-state query: the projection x_(b, j) . wqk[row of (query head, k)] is in qraw
        const int hh = lr / g.n_q, j = lr % g.n_q;
        float sc = 1.f;
        if (LAT == STARKV_LATENT_MIX84) sc = f16_to_f32(a.scales[c0 + k]);
        // the projection's K parts, added in order
        const size_t part = (size_t)g.B * g.n_q * g.G * g.n_key;
        const size_t qi = ((size_t)b * g.n_q + j) * ((size_t)g.G * g.n_key) + (size_t)g.G * c0 + hh * r + k;
        float v = a.qraw[qi];
        for (int pp = 1; pp < a.qraw_parts; ++pp) v += a.qraw[qi + pp * part];
        if (sub == 0) {
          const float x = v * sc * g.qscale;
          qh[n][k] = x;
          if (LAT == STARKV_LATENT_MIX84) atomicMax(&amax[n], __float_as_uint(fabsf(x)));
        }
        continue;
      }
      const int hh = lr / g.n_q, j = lr % g.n_q;
      const size_t qoff = (((size_t)b * g.n_q + j) * g.H_q + gk * g.G + hh) * g.d_h;
      const size_t boff = (size_t)(c0 + k) * g.d_h;
      float acc = 0.f;
      for (int e0 = 0; e0 < g.d_h; e0 += CH) {
        u32x4 qv[NX], bv[NX];
#pragma unroll
        for (int x = 0; x < NX; ++x) {
          const int ee = min(e0 + (x * SUB + sub) * EPL, g.d_h - EPL);
          if (DT == STARKV_F32) {
            qv[x] = ld16((const float*)a.q + qoff + ee);
            bv[x] = ld16((const float*)a.B_k + boff + ee);
          } else {
            qv[x] = ld16((const uint16_t*)a.q + qoff + ee);
            bv[x] = ld16((const uint16_t*)a.B_k + boff + ee);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < NX; ++x) {
          const bool live = e0 + (x * SUB + sub) * EPL < g.d_h;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (DT == STARKV_F32) {
              acc = fmaf(live ? __uint_as_float(qv[x][e]) : 0.f, __uint_as_float(bv[x][e]), acc);
            } else {
              acc = fmaf(live ? bf16_to_f32((uint16_t)(qv[x][e] & 0xFFFF)) : 0.f,
                         bf16_to_f32((uint16_t)(bv[x][e] & 0xFFFF)), acc);
              acc = fmaf(live ? bf16_to_f32((uint16_t)(qv[x][e] >> 16)) : 0.f,
                         bf16_to_f32((uint16_t)(bv[x][e] >> 16)), acc);
            }
          }
        }
      }
#pragma unroll
      for (int o = 1; o < SUB; o <<= 1) acc += __shfl_xor(acc, o, 64);
      float sc = 1.f;
      if (LAT == STARKV_LATENT_MIX84) sc = f16_to_f32(a.scales[c0 + k]);
      if (sub == 0) {
        const float x = acc * sc * g.qscale;
        qh[n][k] = x;
        if (LAT == STARKV_LATENT_MIX84) atomicMax(&amax[n], __float_as_uint(fabsf(x)));
      }
    }
    __syncthreads();
    // row parameters: rho and the int4 offset-binary bias terms 8 * sum(int4 codes' weights)
    for (int n = wave; n < nrows; n += NWV) {
      // offset-binary codes: int4 nibbles read as code + 8; packed layout: outlier nibbles
      // code + 8, 3-bit inlier fields code + 4
      int sh = 0, sl = 0;
      const float rho = LAT == STARKV_LATENT_MIX84 ? qrow_rho(amax[n]) : 1.f;
      if (LAT == STARKV_LATENT_MIX84)
        for (int k = (g.pack3 ? 0 : n8g) + lane; k < r; k += 64) {
          const int wgt = (g.pack3 && k >= n8g) ? 4 : 8;
          int hi, lo;
          qsplit(qh[n][k], rho, hi, lo);
          sh += wgt * hi;
          sl += wgt * lo;
        }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        sh += __shfl_xor(sh, o, 64);
        sl += __shfl_xor(sl, o, 64);
      }
      if (lane == 0) {
        const int b = (ub0 + n) / rph, i = gk * rph + (ub0 + n) - b * rph;
        float* rp = a.rowp + ((size_t)b * g.M_pad + i) * 4;
        rp[0] = rho;
        rp[1] = (float)sh;
        rp[2] = (float)sl;
        rp[3] = 0.f;
      }
    }
    // fragment chunks of these rows: (row, K-tile, 16-position group qq), all rows in one pass
    int pre[RB + 1];  // first item of each row (rows past nrows have none)
    pre[0] = 0;
#pragma unroll
    for (int n = 0; n < RB; ++n) pre[n + 1] = pre[n] + (n < nrows ? 4 * a.kts.n[(gk * rph + (ub0 + n) % rph) >> 4] : 0);
    for (int it = tid; it < pre[RB]; it += NT) {
      int n = 0, item = it;
#pragma unroll
      for (int m = 1; m < RB; ++m)
        if (it >= pre[m]) {
          n = m;
          item = it - pre[m];
        }
      const int b = (ub0 + n) / rph, i = gk * rph + (ub0 + n) - b * rph;
      const int ct = i >> 4, col = i & 15;
      {
        const int jt = item >> 2, qq = item & 3;
        const int kt = a.kts.at(ct, jt);
        const int ln = col + 16 * qq;  // fragment lane holding this chunk
        uint8_t* frag = a.qfrag + (((size_t)b * g.nct + ct) * a.nkt_max + jt) * 2048;
        if (LAT == STARKV_LATENT_MIX84) {
          const int P0 = kt * 64 + 16 * qq;
          const float rho = qrow_rho(amax[n]);
          uint32_t wh[4] = {0, 0, 0, 0}, wl[4] = {0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            int k = -1;
            if (g.pack3) {
              if (P0 < g.K4) {  // outlier nibbles, unpacked as int4 groups
                const int u = P0 + int4_perm16(e);
                if (u >= o8 && u < o8 + n8g) k = u - o8;
              } else if (P0 < g.K4 + g.K3) {  // 3-bit planes: element e holds channel
                // 8 (e & 3) + (e >> 2) + 4 h of its 32-channel group (unpack_int3_group)
                const int rel = P0 - g.K4;
                const int u = (rel & ~31) + 8 * (e & 3) + (e >> 2) + 4 * ((rel >> 4) & 1);
                if (u >= o4 && u < o4 + (r - n8g)) k = n8g + (u - o4);
              }
            } else if (P0 < g.K8) {
              const int slot = P0 + e;
              if (slot >= o8 && slot < o8 + n8g) k = slot - o8;
            } else if (P0 < g.K8 + g.K4) {
              const int u = P0 - g.K8 + int4_perm16(e);
              if (u >= o4 && u < o4 + (r - n8g)) k = n8g + (u - o4);
            }
            if (k >= 0) {
              int hi, lo;
              qsplit(qh[n][k], rho, hi, lo);
              wh[e >> 2] |= ((uint32_t)(uint8_t)(int8_t)hi) << (8 * (e & 3));
              wl[e >> 2] |= ((uint32_t)(uint8_t)(int8_t)lo) << (8 * (e & 3));
            }
          }
          st16(frag + ln * 16, u32x4{wh[0], wh[1], wh[2], wh[3]});
          st16(frag + 1024 + ln * 16, u32x4{wl[0], wl[1], wl[2], wl[3]});
        } else {
          const int P0 = kt * 32 + 8 * qq;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int k = P0 + e - c0;
            v[e] = (k >= 0 && k < r) ? qh[n][k] : 0.f;
          }
          if (LAT == STARKV_LATENT_F32) {
            st16(frag + ln * 32, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                       __float_as_uint(v[3])});
            st16(frag + ln * 32 + 16, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
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
            st16(frag + ln * 16, u32x4{wh[0], wh[1], wh[2], wh[3]});
            st16(frag + 1024 + ln * 16, u32x4{wl[0], wl[1], wl[2], wl[3]});
          }
        }
      }
    }
  }
  // the last head also zeroes the chunks of the padding rows of the last column tile, in the
  // workgroup that holds the sequence's first row
  for (int b = (u_lo + rph - 1) / rph; gk == g.H_kv - 1 && b * rph < u_hi; ++b) {
    for (int i = g.M_q; i < g.nct * 16; ++i) {
      const int ct = i >> 4, col = i & 15;
      const int nkt = a.kts.n[ct];
      for (int item = tid; item < nkt * 4; item += NT) {
        const int jt = item >> 2, qq = item & 3, ln = col + 16 * qq;
        uint8_t* frag = a.qfrag + (((size_t)b * g.nct + ct) * a.nkt_max + jt) * 2048;
        if (LAT == STARKV_LATENT_F32) {
          st16(frag + ln * 32, u32x4{0, 0, 0, 0});
          st16(frag + ln * 32 + 16, u32x4{0, 0, 0, 0});
        } else {
          st16(frag + ln * 16, u32x4{0, 0, 0, 0});
          st16(frag + 1024 + ln * 16, u32x4{0, 0, 0, 0});
        }
      }
    }
  }
}

// HID: the query comes from hidden states; their projection through the absorbed factors is
// already in a.qraw.
// Grid (KV head, row group): group y takes the rows u in [y qp_w, (y + 1) qp_w) of the head.
template <int DT, int LAT, bool HID>
__global__ __launch_bounds__(256) void k_qproj(QprojArgs a) {
  __shared__ QprojSharedT<kQpRB16> sh;
  const int n_u = a.g.B * a.g.G * a.g.n_q;
  const int u_lo = blockIdx.y * a.qp_w;
  qproj_body<DT, LAT, 256, HID, kQpRB16>(a, blockIdx.x, u_lo, min(n_u, u_lo + a.qp_w), sh);
}

// ===========================================================================
// scores: per (sequence, 64-token chunk): p~ = 2^(s - m_chunk), chunk max and sum

// Sequence bookkeeping of the decode plan: with equal lengths every quantity is a product or a
// quotient; otherwise it is read from the prefix tables (segment search by the whole wave).
__device__ __forceinline__ int seq_len(const SeqTable& t, int b) {
  const int l = t.uni ? t.u_len : t.lens[b];
  return t.lens_dev ? min(max(t.lens_dev[b], t.len_lo), l) : l;
}
__device__ __forceinline__ int seq_chunk0(const SeqTable& t, int b) { return t.uni ? b * t.u_nch : t.chunk_off[b]; }
__device__ __forceinline__ int seq_nch(const SeqTable& t, int b) {
  return t.uni ? t.u_nch : t.chunk_off[b + 1] - t.chunk_off[b];
}
// chunks that hold tokens below the length the kernels see: the planned count, or with device
// lengths the chunks of that length (later chunks and the splits made of them are skipped)
__device__ __forceinline__ int seq_nch_live(const SeqTable& t, int b) {
  return t.lens_dev ? (seq_len(t, b) + kTC - 1) / kTC : seq_nch(t, b);
}
__device__ __forceinline__ int seq_split0(const SeqTable& t, int b) { return t.uni ? b * t.u_nspl : t.split_off[b]; }
__device__ __forceinline__ int seq_nsplit(const SeqTable& t, int b) {
  return t.uni ? t.u_nspl : t.split_off[b + 1] - t.split_off[b];
}
__device__ __forceinline__ int seq_blk0(const SeqTable& t, int b) { return t.uni ? b * t.u_nblk : t.blk_off[b]; }
// sequence of a global split / 128-token block / 32-token chunk (call with the whole wave active)
__device__ __forceinline__ int seq_of_split(const SeqTable& t, int B, int sg) {
  return t.uni ? sg / t.u_nspl : find_segment_wave(t.split_off, B, sg);
}
// Order in which the value workgroups take the splits: every split that is not the last of its
// sequence (all of full length) first, then the last split of each sequence (the only ones that
// may be short), so that with ragged lengths the short workgroups run at the end of the grid
// instead of full ones.  Every sequence has at least one split.  Returns the split of position
// idx and sets b to its sequence (call with the whole wave active).
__device__ __forceinline__ int value_split(const SeqTable& t, int B, int idx, int& b) {
  if (t.uni) {
    const int nn = t.u_nspl - 1;  // splits per sequence that are not its last
    const int n_nl = B * nn;
    if (idx < n_nl) {
      b = idx / nn;
      return b * t.u_nspl + idx % nn;
    }
    b = idx - n_nl;
    return b * t.u_nspl + nn;
  }
  const int n_nl = t.split_off[B] - B;
  if (idx < n_nl) {
    // non-last splits before sequence b': split_off[b'] - b' (non-decreasing in b'); b is the
    // largest b' < B with that count <= idx, and the split is idx + b
    const int lane = threadIdx.x & 63;
    const int i0 = min(lane + 1, B), i1 = min(lane + 65, B);
    const unsigned long long m0 = __ballot(lane + 1 < B && t.split_off[i0] - i0 <= idx);
    const unsigned long long m1 = __ballot(lane + 65 < B && t.split_off[i1] - i1 <= idx);
    b = __builtin_amdgcn_readfirstlane(__popcll(m0) + __popcll(m1));
    return idx + b;
  }
  b = idx - n_nl;
  return t.split_off[b + 1] - 1;
}
__device__ __forceinline__ int seq_of_blk(const SeqTable& t, int B, int k) {
  return t.uni ? k / t.u_nblk : find_segment_wave(t.blk_off, B, k);
}
__device__ __forceinline__ int seq_of_chunk(const SeqTable& t, int B, int c) {
  return t.uni ? c / t.u_nch : find_segment_wave(t.chunk_off, B, c);
}

struct ScoreArgs {
  const uint8_t* k_rows;
  const uint8_t* qfrag;
  const float* rowp;
  void* p;
  float* cm;
  float* cl;
  DecodeGeom g;
  int nkt_max;
  int nch_wg;        // 64-token chunks per workgroup
  int total_chunks;
  KtList kts;
  SeqTable seq;
};

// Workgroup = 4 waves over `nch_wg` consecutive 64-token chunks (global chunk numbering, so a
// workgroup may span sequences); work unit = (column tile ct, chunk).  Per unit the loop runs
// K-tile outer / 16-token tile inner, so each query fragment is loaded once per unit.
// Workgroup = (sequence, column tile ct, block of 128 tokens = four 32-token chunks).  The four
// waves split the K-tiles of ct (wave w takes K-tiles w, w+4, ...: waves read neighbouring K-tiles
// of the same key rows at the same time) and keep their query
// fragments in registers for the whole block; each wave computes partial scores of the 8
// 16-token tiles over its K-tiles (loads of 4 tiles x 2 K-tiles in flight: more per wave measured
// slower on MI355X), the partials are
// added through LDS, and wave w then finishes chunk w: mask, chunk max and sum, p~ = 2^(s - m).
template <int LAT>
__global__ __launch_bounds__(256) void k_scores(ScoreArgs a) {
  constexpr int KW = kMaxKT / 4;  // K-tiles per wave (max)
  constexpr int FR = LAT == STARKV_LATENT_F32 ? 2 : 2;  // 16-byte fragment loads per K-tile
  __shared__ float part[4][8][4][64];  // [wave][token tile][D element][lane]
  const DecodeGeom& g = a.g;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n = lane & 15, qq = lane >> 4;
  const int ct = blockIdx.x % g.nct;
  const int gblk = blockIdx.x / g.nct;
  const int b = seq_of_blk(a.seq, g.B, gblk);
  const int t_blk = (gblk - seq_blk0(a.seq, b)) * 128;
  const int len = seq_len(a.seq, b);
  if (t_blk >= len) return;  // past the device length: no value split reads it (whole workgroup)
  const uint8_t* kbase = a.k_rows + (size_t)b * g.T_max * g.k_row_bytes;
  const int nkt = a.kts.n[ct];
  const int nkw = nkt > wave ? (nkt - wave + 3) / 4 : 0;  // K-tiles of this wave (uniform)
  const uint8_t* fbase = a.qfrag + ((size_t)b * g.nct + ct) * a.nkt_max * 2048;

  // query fragments of this wave's K-tiles
  u32x4 fr[KW][FR];
  int p0[KW];
#pragma unroll
  for (int j = 0; j < KW; ++j) {
    const bool on = j < nkw;
    const int jt = wave + 4 * (on ? j : 0);
    const int kt = a.kts.at(ct, jt);
    p0[j] = (LAT == STARKV_LATENT_MIX84 ? kt * 64 + 16 * qq : kt * 32 + 8 * qq);
    const uint8_t* f = fbase + (size_t)jt * 2048;
#pragma unroll
    for (int k = 0; k < FR; ++k) {
      const int off = LAT == STARKV_LATENT_F32 ? lane * 32 + 16 * k : 1024 * k + lane * 16;
      fr[j][k] = on ? ld16(f + off) : u32x4{0, 0, 0, 0};
    }
  }
  float rho = 1.f;
  if (LAT == STARKV_LATENT_MIX84) {
    const int i = ct * 16 + n;
    if (i < g.M_q) rho = a.rowp[((size_t)b * g.M_pad + i) * 4];
  }

  // partial scores of the 8 token tiles over this wave's K-tiles, four tiles at a time
#pragma unroll
  for (int tg = 0; tg < 2; ++tg) {
    float sp[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) sp[t][v] = 0.f;
    const uint8_t* rowp[4];
    bool tok_ok[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tok = t_blk + (tg * 4 + t) * 16 + n;
      tok_ok[t] = tok < len;
      rowp[t] = kbase + (size_t)(tok_ok[t] ? tok : 0) * g.k_row_bytes;
    }
    for (int j0 = 0; j0 < nkw; j0 += 2) {
      if (LAT == STARKV_LATENT_MIX84) {
        i32x4 av[2][4];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int j = j0 + jj;
          const bool on = j < nkw;
          int P0 = 0;
#pragma unroll
          for (int x = 0; x < KW; ++x)
            if (x == j) P0 = p0[x];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            i32x4 v = {0, 0, 0, 0};
            if (on && tok_ok[t]) {
              if (P0 < g.K8) v = __builtin_bit_cast(i32x4, ld16(rowp[t] + P0));
              else if (P0 < g.K8 + g.K4) v = unpack_int4_group(ld8(rowp[t] + g.K8 + (P0 - g.K8) / 2));
            }
            av[jj][t] = v;
          }
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          i32x4 fh = {0, 0, 0, 0}, fl = {0, 0, 0, 0};
#pragma unroll
          for (int x = 0; x < KW; ++x)
            if (x == j0 + jj) {
              fh = __builtin_bit_cast(i32x4, fr[x][0]);
              fl = __builtin_bit_cast(i32x4, fr[x][1]);
            }
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const i32x4 h = mfma16_i8(av[jj][t], fh, i32x4{0, 0, 0, 0});
            const i32x4 l = mfma16_i8(av[jj][t], fl, i32x4{0, 0, 0, 0});
#pragma unroll
            for (int v = 0; v < 4; ++v) sp[t][v] += rho * (float)h[v] + (rho * (1.f / 254.f)) * (float)l[v];
          }
        }
      } else if (LAT == STARKV_LATENT_BF16) {
        u32x4 av[2][4];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int j = j0 + jj;
          const bool on = j < nkw;
          int P0 = 0;
#pragma unroll
          for (int x = 0; x < KW; ++x)
            if (x == j) P0 = p0[x];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            av[jj][t] = (on && tok_ok[t] && P0 < g.key_kpos) ? ld16(rowp[t] + 2 * P0) : u32x4{0, 0, 0, 0};
        }
        f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = f32x4{sp[t][0], sp[t][1], sp[t][2], sp[t][3]};
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          u32x4 fh = {0, 0, 0, 0}, fl = {0, 0, 0, 0};
#pragma unroll
          for (int x = 0; x < KW; ++x)
            if (x == j0 + jj) {
              fh = fr[x][0];
              fl = fr[x][1];
            }
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            acc[t] = mfma16_bf16(as_bf16x8(av[jj][t]), as_bf16x8(fh), acc[t]);
            acc[t] = mfma16_bf16(as_bf16x8(av[jj][t]), as_bf16x8(fl), acc[t]);
          }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) sp[t][v] = acc[t][v];
      } else {
        f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = f32x4{sp[t][0], sp[t][1], sp[t][2], sp[t][3]};
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int j = j0 + jj;
          if (j >= nkw) continue;
          int P0 = 0;
          u32x4 f0 = {0, 0, 0, 0}, f1 = {0, 0, 0, 0};
#pragma unroll
          for (int x = 0; x < KW; ++x)
            if (x == j) {
              P0 = p0[x];
              f0 = fr[x][0];
              f1 = fr[x][1];
            }
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const u32x4 a0 = (tok_ok[t] && P0 < g.key_kpos) ? ld16(rowp[t] + 4 * P0) : u32x4{0, 0, 0, 0};
            const u32x4 a1 = (tok_ok[t] && P0 + 4 < g.key_kpos) ? ld16(rowp[t] + 4 * P0 + 16) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[t] = mfma16_f32(__uint_as_float(a0[e]), __uint_as_float(f0[e]), acc[t]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[t] = mfma16_f32(__uint_as_float(a1[e]), __uint_as_float(f1[e]), acc[t]);
          }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) sp[t][v] = acc[t][v];
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) part[wave][tg * 4 + t][v][lane] = sp[t][v];
  }
  __syncthreads();

  // wave w finishes chunk w of the block (token tiles 2w, 2w + 1)
  const int t0 = t_blk + 32 * wave;
  const int nch_b = seq_nch(a.seq, b);
  const int cidx = t0 / kTC;
  if (cidx >= nch_b) return;
  const int cg = seq_chunk0(a.seq, b) + cidx;
  const int i = ct * 16 + n;
  const bool rowvalid = i < g.M_q;
  const int pos = len - g.n_q + (i % g.n_q);
  float bias = 0.f;
  if (LAT == STARKV_LATENT_MIX84 && rowvalid) {
    const float* rp = a.rowp + ((size_t)b * g.M_pad + i) * 4;
    bias = rp[0] * (rp[1] + rp[2] * (1.f / 254.f));
  }
  float s2[2][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int ti = 2 * wave + tt;
      float x = part[0][ti][v][lane] + part[1][ti][v][lane] + part[2][ti][v][lane] + part[3][ti][v][lane];
      x -= bias;
      const int t = t0 + tt * 16 + 4 * qq + v;
      const bool ok = rowvalid && t < len && t <= pos;
      s2[tt][v] = ok ? x : -INFINITY;
    }
  float m = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int v = 0; v < 4; ++v) m = fmaxf(m, s2[tt][v]);
  m = wave_max_xor(m, 16);
  m = wave_max_xor(m, 32);
  float l = 0.f;
  const size_t prow = ((size_t)cg * g.M_pad + i) * kTC;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
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

// Workgroup = 4 waves over `nch_wg` consecutive 32-token chunks (global chunk numbering, so a
// workgroup may span sequences); work unit = (column tile ct, chunk) = 2 MFMA row tiles of 16
// tokens.  Per unit the K-tiles are walked KU at a time: the loads of KU K-tiles (query
// fragments and key rows) are issued before their MFMAs.  KU = 4 when no column tile has more
// than six K-tiles (one or two batches per unit); with more K-tiles, KU = 2 (fewer registers,
// 6 instead of 4 waves per SIMD) was faster on MI355X.
// P3: the packed layout (outlier nibbles from position 0, 3-bit planes from K4); a 3-bit lane
// loads its 32-channel group's three plane words (12 bytes) and unpacks its half.
template <int LAT, int KU, bool P3 = false>
__global__ __launch_bounds__(256) void k_scores_chunk(ScoreArgs a) {
  const DecodeGeom& g = a.g;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n = lane & 15, qq = lane >> 4;
  const int units = g.nct * a.nch_wg;
  int b = -1;  // sequence of the current chunk: looked up once, then advanced (the chunks of a
               // wave's units never decrease)
  for (int u = wave; u < units; u += 4) {
    const int ct = u % g.nct;
    const int cg = blockIdx.x * a.nch_wg + u / g.nct;  // global chunk
    if (cg >= a.total_chunks) break;
    if (b < 0) b = seq_of_chunk(a.seq, g.B, cg);
    while (cg >= seq_chunk0(a.seq, b + 1)) ++b;
    const int t0 = (cg - seq_chunk0(a.seq, b)) * kTC;
    const int len = seq_len(a.seq, b);
    if (t0 >= len) continue;  // past the device length: no value split reads it
    const uint8_t* kbase = a.k_rows + (size_t)b * g.T_max * g.k_row_bytes;
    const int i = ct * 16 + n;  // query row of this lane's result column
    const bool rowvalid = i < g.M_q;
    const int pos = len - g.n_q + (i % g.n_q);
    float rho = 1.f, bh = 0.f, bl = 0.f;
    if (LAT == STARKV_LATENT_MIX84) {
      // row parameters at a clamped row (no branch around the load; padding rows are masked)
      const u32x4 rp = ld16(a.rowp + ((size_t)b * g.M_pad + min(i, g.M_q - 1)) * 4);
      rho = __uint_as_float(rp[0]);
      bh = __uint_as_float(rp[1]);
      bl = __uint_as_float(rp[2]);
    }
    const int nkt = a.kts.n[ct];
    // this column tile's K-tile list (two runs), read once per unit
    const int ks0 = a.kts.s0[ct], kn0 = a.kts.n0[ct], ks1 = a.kts.s1[ct];
    const uint8_t* fbase = a.qfrag + ((size_t)b * g.nct + ct) * a.nkt_max * 2048;
    const uint8_t* rowp[2];
    bool tok_ok[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = t0 + tt * 16 + n;
      tok_ok[tt] = tok < len;
      rowp[tt] = kbase + (size_t)(tok_ok[tt] ? tok : 0) * g.k_row_bytes;
    }
    float s2[2][4];
    if (LAT == STARKV_LATENT_MIX84) {
      // key rows of sequence b as a buffer: one 16-byte load per lane and K-tile, at the lane's
      // 16 int8 codes or at the aligned 16 bytes that hold its 16 int4 codes (key-row segments
      // are 16-byte aligned, so these never leave the row); a masked token or K-tile points past
      // the end, so no branch surrounds the loads
      const __amdgpu_buffer_rsrc_t krs = buf_rsrc(kbase, (uint32_t)g.T_max * (uint32_t)g.k_row_bytes);
      uint32_t trow[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) trow[tt] = (uint32_t)(t0 + tt * 16 + n) * (uint32_t)g.k_row_bytes;
      i32x4 ah[2], al[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) ah[tt] = al[tt] = i32x4{0, 0, 0, 0};
      for (int jt0 = 0; jt0 < nkt; jt0 += KU) {
        i32x4 fh[KU], fl[KU], av[KU][2];
        u32x4 rk[KU][2];
        u32x3 r3[P3 ? KU : 1][2];
        bool is8[KU], is4[KU], hi4[KU], is3[KU], h3[KU];
#pragma unroll
        for (int j = 0; j < KU; ++j) {
          const bool on = jt0 + j < nkt;
          const int jc = on ? jt0 + j : 0;
          const int kt = jc < kn0 ? ks0 + jc : ks1 + (jc - kn0);
          const int P0 = kt * 64 + 16 * qq;
          is8[j] = on && P0 < g.K8;
          is4[j] = on && P0 >= g.K8 && P0 < g.K8 + g.K4;
          fh[j] = __builtin_bit_cast(i32x4, ld16(fbase + jc * 2048 + lane * 16));
          fl[j] = __builtin_bit_cast(i32x4, ld16(fbase + jc * 2048 + 1024 + lane * 16));
          const uint32_t o4 = (uint32_t)(g.K8 + (P0 - g.K8) / 2);
          hi4[j] = (o4 & 8u) != 0;
          const uint32_t ok = is8[j] ? (uint32_t)P0 : (o4 & ~15u);
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) rk[j][tt] = bld16(krs, ((is8[j] || is4[j]) && tok_ok[tt]) ? trow[tt] + ok : kOOB);
          is3[j] = P3 && on && P0 >= g.K4 && P0 < g.K4 + g.K3;
          h3[j] = ((P0 - g.K4) >> 4) & 1;
          if (P3) {
            const uint32_t o3 = (uint32_t)(g.K4 / 2 + 12 * ((P0 - g.K4) >> 5));
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) r3[j % (P3 ? KU : 1)][tt] = bld12(krs, (is3[j] && tok_ok[tt]) ? trow[tt] + o3 : kOOB);
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // every load of the batch ahead of its use
#pragma unroll
        for (int j = 0; j < KU; ++j)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            // (a K-tile past nkt has neither flag: zero operand; masked tokens are masked below)
            av[j][tt] = is8[j] ? __builtin_bit_cast(i32x4, rk[j][tt])
                               : (is4[j] ? unpack_int4_group(hi4[j] ? u32x2{rk[j][tt][2], rk[j][tt][3]}
                                                                    : u32x2{rk[j][tt][0], rk[j][tt][1]})
                                         : ((P3 && is3[j]) ? unpack_int3_group(r3[j % (P3 ? KU : 1)][tt], h3[j])
                                                           : i32x4{0, 0, 0, 0}));
#pragma unroll
        for (int j = 0; j < KU; ++j)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            ah[tt] = mfma16_i8(av[j][tt], fh[j], ah[tt]);
            al[tt] = mfma16_i8(av[j][tt], fl[j], al[tt]);
          }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          s2[tt][v] = rho * (float)(ah[tt][v] - (int)bh) + (rho * (1.f / 254.f)) * (float)(al[tt][v] - (int)bl);
    } else if (LAT == STARKV_LATENT_BF16) {
      f32x4 acc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) acc[tt] = f32x4{0, 0, 0, 0};
      for (int jt0 = 0; jt0 < nkt; jt0 += KU) {
        u32x4 fh[KU], fl[KU], av[KU][2];
#pragma unroll
        for (int j = 0; j < KU; ++j) {
          const bool on = jt0 + j < nkt;
          const int kt = on ? a.kts.at(ct, jt0 + j) : 0;
          const int P0 = kt * 32 + 8 * qq;
          fh[j] = on ? ld16(fbase + (jt0 + j) * 2048 + lane * 16) : u32x4{0, 0, 0, 0};
          fl[j] = on ? ld16(fbase + (jt0 + j) * 2048 + 1024 + lane * 16) : u32x4{0, 0, 0, 0};
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            av[j][tt] = (on && tok_ok[tt] && P0 < g.key_kpos) ? ld16(rowp[tt] + 2 * P0) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < KU; ++j)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            acc[tt] = mfma16_bf16(as_bf16x8(av[j][tt]), as_bf16x8(fh[j]), acc[tt]);
            acc[tt] = mfma16_bf16(as_bf16x8(av[j][tt]), as_bf16x8(fl[j]), acc[tt]);
          }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) s2[tt][v] = acc[tt][v];
    } else {
      f32x4 acc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) acc[tt] = f32x4{0, 0, 0, 0};
      for (int jt = 0; jt < nkt; ++jt) {
        const int kt = a.kts.at(ct, jt);
        const u32x4 f0 = ld16(fbase + jt * 2048 + lane * 32);
        const u32x4 f1 = ld16(fbase + jt * 2048 + lane * 32 + 16);
        const int P0 = kt * 32 + 8 * qq;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const u32x4 a0 = (tok_ok[tt] && P0 < g.key_kpos) ? ld16(rowp[tt] + 4 * P0) : u32x4{0, 0, 0, 0};
          const u32x4 a1 = (tok_ok[tt] && P0 + 4 < g.key_kpos) ? ld16(rowp[tt] + 4 * P0 + 16) : u32x4{0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[tt] = mfma16_f32(__uint_as_float(a0[e]), __uint_as_float(f0[e]), acc[tt]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[tt] = mfma16_f32(__uint_as_float(a1[e]), __uint_as_float(f1[e]), acc[tt]);
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) s2[tt][v] = acc[tt][v];
    }
    // lane holds D[token 4*qq + v][column n] of each 16-token tile: mask, chunk max and sum
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + tt * 16 + 4 * qq + v;
        const bool ok = rowvalid && t < len && t <= pos;
        s2[tt][v] = ok ? s2[tt][v] : -INFINITY;
      }
    float m = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) m = fmaxf(m, s2[tt][v]);
    m = wave_max_xor(m, 16);
    m = wave_max_xor(m, 32);
    float l = 0.f;
    const size_t prow = ((size_t)cg * g.M_pad + i) * kTC;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
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

// Key scores of int8/int4 latents, walking chunks with the column tile's state in registers.
// Workgroup = (block of CPB = nch_wg consecutive 32-token chunks in the global numbering, possibly
// spanning sequences; pair of 16-row column tiles), four waves: wave w takes column tile
// 2 p + (w & 1) and chunks w >> 1, w >> 1 + 2, ... of the block.  The pairs of one block run on one
// XCD (grid position mod 8), so the key rows they share are fetched into one L2.  A wave keeps
// its column tile's query fragments, the per-lane key-row offsets of its K-tiles and its row's
// parameters in registers while it walks its chunks (the fragments and parameters are reloaded
// only when a chunk starts another sequence), with the key loads of its next NS chunks in flight.  Used when there are at least four column tiles to share the key rows
// (with two, the per-unit kernel above was faster on MI355X).  The two int8 query parts are combined in integers
// (254 hi + lo, minus the int4 offset bias) before one conversion.  Output as k_scores_chunk.
template <int KTM, int NS = (KTM <= 6 ? 3 : 2)>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_scores_mix(ScoreArgs a) {
  const int CPB = a.nch_wg;  // chunks per block
  const DecodeGeom& g = a.g;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n = lane & 15, qq = lane >> 4;
  const int n_pairs = (g.nct + 1) / 2;
  const int xcd = blockIdx.x & 7, kk = blockIdx.x >> 3;
  const int pr = kk % n_pairs, blk = 8 * (kk / n_pairs) + xcd;
  const int ct = 2 * pr + (wave & 1);
  const int c_first = blk * CPB + (wave >> 1);
  const int c_end = min(blk * CPB + CPB, a.total_chunks);
  if (ct >= g.nct || c_first >= c_end) return;  // wave-uniform; the kernel has no barrier

  // K-tiles of the column tile: per-lane byte offset in a key row of the lane's 16 int8 codes,
  // or of the 8 bytes that hold its 16 int4 codes (a 16-byte load from there: the lane uses the
  // first half), or 2^31 when the lane has no codes in the K-tile: past the end of the buffer
  // (zeros, no memory traffic) whenever a sequence's key rows span less than 2 GiB, and in any
  // case harmless (an unused K-tile is skipped; a padding lane meets a zero query fragment).
  const int nkt = a.kts.n[ct];
  const int ks0 = a.kts.s0[ct], kn0 = a.kts.n0[ct], ks1 = a.kts.s1[ct];
  uint32_t kofs[KTM];
  bool k8[KTM];
#pragma unroll
  for (int jt = 0; jt < KTM; ++jt) {
    const int kt = jt < kn0 ? ks0 + jt : ks1 + (jt - kn0);
    const int P0 = kt * 64 + 16 * qq;
    const bool on = jt < nkt;
    k8[jt] = on && P0 < g.K8;
    const bool i4 = on && P0 >= g.K8 && P0 < g.K8 + g.K4;
    const uint32_t o4 = (uint32_t)(g.K8 + (P0 - g.K8) / 2);
    kofs[jt] = k8[jt] ? (uint32_t)P0 : (i4 ? o4 : 0x80000000u);
  }
  const int i = ct * 16 + n;
  const bool rowvalid = i < g.M_q;
  // every row of the column tile is a query row: tokens need masking only near the end
  const bool tile_full = (ct + 1) * 16 <= g.M_q;
  const int jq = i % g.n_q;
  const uint32_t rb = (uint32_t)g.k_row_bytes;

  // Loads of the wave's chunks go out NS steps ahead of their use, into NS register sets that
  // take turns (no copies between them, so each wait covers only the set about to be used).
  // The issue side keeps its own chunk and sequence; past the wave's last chunk its buffer is
  // empty, so those loads return zeros without touching memory.  Tokens past the length (in the
  // last chunk of a sequence) load whatever the row holds and are masked in the scores.
  int ci = c_first;
  int bi = seq_of_chunk(a.seq, g.B, c_first);
  int bi_end = seq_chunk0(a.seq, bi + 1);
  int bi_len = seq_len(a.seq, bi);
  auto issue = [&](u32x4 kr[KTM][2]) {
    bool live = ci < c_end;  // wave-uniform
    if (live) {
      while (ci >= bi_end) {
        ++bi;
        bi_end = seq_chunk0(a.seq, bi + 1);
        bi_len = seq_len(a.seq, bi);
      }
      live = (ci - seq_chunk0(a.seq, bi)) * kTC < bi_len;  // (false only past a device length)
    }
    const __amdgpu_buffer_rsrc_t krs =
        buf_rsrc(a.k_rows + (size_t)bi * g.T_max * g.k_row_bytes, live ? (uint32_t)g.T_max * rb : 0u);
    const uint32_t t0 = (uint32_t)(ci - seq_chunk0(a.seq, bi)) * kTC;
    const uint32_t to0 = (t0 + n) * rb, to1 = to0 + 16 * rb;
#pragma unroll
    for (int jt = 0; jt < KTM; ++jt) {
      kr[jt][0] = bld16(krs, to0 + kofs[jt]);
      kr[jt][1] = bld16(krs, to1 + kofs[jt]);
    }
    ci += 2;
  };
  // query fragments and row parameters of sequence bb
  i32x4 fh[KTM], fl[KTM];
  float rs = 0.f;
  int ibias = 0;
  auto load_seq = [&](int bb) {
    const uint8_t* fbase = a.qfrag + ((size_t)bb * g.nct + ct) * a.nkt_max * 2048;
#pragma unroll
    for (int jt = 0; jt < KTM; ++jt) {
      const int jc = jt < nkt ? jt : 0;
      fh[jt] = __builtin_bit_cast(i32x4, ld16(fbase + jc * 2048 + lane * 16));
      fl[jt] = __builtin_bit_cast(i32x4, ld16(fbase + jc * 2048 + 1024 + lane * 16));
    }
    const u32x4 rp = ld16(a.rowp + ((size_t)bb * g.M_pad + min(i, g.M_q - 1)) * 4);
    rs = __uint_as_float(rp[0]) * (1.f / 254.f);
    ibias = 254 * (int)__uint_as_float(rp[1]) + (int)__uint_as_float(rp[2]);
  };
  // compute side: chunk cc of sequence bc (fragments of sequence bf loaded)
  int cc = c_first;
  int bc = bi, bf = -1;
  int bc0 = seq_chunk0(a.seq, bc), bc_end = bi_end, bc_len = seq_len(a.seq, bc);
  auto step = [&](const u32x4 kr[KTM][2]) {
    while (cc >= bc_end) {
      ++bc;
      bc0 = bc_end;
      bc_end = seq_chunk0(a.seq, bc + 1);
      bc_len = seq_len(a.seq, bc);
    }
    if ((cc - bc0) * kTC >= bc_len) {  // past a device length: no value split reads this chunk
      cc += 2;
      return;
    }
    if (bc != bf) {  // the block reaches another sequence (rare): its fragments first
      bf = bc;
      load_seq(bc);
      vm_wait<0>();  // so that no later wait counts the fragments as still in flight
    }
    // scores of chunk cc: lane holds tokens 16 tt + 4 qq + v of row i; the low part's
    // accumulator starts at minus the row's offset-binary bias
    i32x4 ah[2], al[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      ah[tt] = i32x4{0, 0, 0, 0};
      al[tt] = i32x4{-ibias, -ibias, -ibias, -ibias};
    }
#pragma unroll
    for (int jt = 0; jt < KTM; ++jt) {
      if (jt < nkt) {  // wave-uniform
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const i32x4 av = k8[jt] ? __builtin_bit_cast(i32x4, kr[jt][tt])
                                  : unpack_int4_group(u32x2{kr[jt][tt][0], kr[jt][tt][1]});
          ah[tt] = mfma16_i8(av, fh[jt], ah[tt]);
          al[tt] = mfma16_i8(av, fl[jt], al[tt]);
        }
      }
    }
    const int t0 = (cc - bc0) * kTC;
    float s2[2][4];
    float m = -INFINITY;
    if (tile_full && t0 + kTC - 1 <= bc_len - g.n_q) {  // wave-uniform: every row sees every token
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          s2[tt][v] = rs * (float)(254 * ah[tt][v] + al[tt][v]);
          m = fmaxf(m, s2[tt][v]);
        }
    } else {
      const int lim = rowvalid ? bc_len - g.n_q + jq : -1;  // last token this row sees
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = t0 + tt * 16 + 4 * qq + v;
          s2[tt][v] = t <= lim ? rs * (float)(254 * ah[tt][v] + al[tt][v]) : -INFINITY;
          m = fmaxf(m, s2[tt][v]);
        }
    }
    m = wave_max_xor(m, 16);
    m = wave_max_xor(m, 32);
    // exp2(-inf - m) is 0; a row with no visible token keeps m = -inf and takes 0 for reference
    const float mref = m == -INFINITY ? 0.f : m;
    float l = 0.f;
    const size_t prow = ((size_t)cc * g.M_pad + i) * kTC;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float e4[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        e4[v] = __builtin_amdgcn_exp2f(s2[tt][v] - mref);
        l += e4[v];
      }
      const uint32_t w0 = (uint32_t)f32_to_f16(e4[0]) | ((uint32_t)f32_to_f16(e4[1]) << 16);
      const uint32_t w1 = (uint32_t)f32_to_f16(e4[2]) | ((uint32_t)f32_to_f16(e4[3]) << 16);
      st8((uint16_t*)a.p + prow + tt * 16 + 4 * qq, u32x2{w0, w1});
    }
    l = wave_sum_xor(l, 16);
    l = wave_sum_xor(l, 32);
    // the four lanes of a row hold the same m and l: all store them (one store per wave, no branch)
    a.cm[(size_t)cc * g.M_pad + i] = m;
    a.cl[(size_t)cc * g.M_pad + i] = l;
    cc += 2;
  };

  const int n_mine = (c_end - c_first + 1) / 2;  // chunks c_first, c_first + 2, ... below c_end
  if (NS == 3) {
    u32x4 k0[KTM][2], k1[KTM][2], k2[KTM][2];
    issue(k0);
    issue(k1);
    issue(k2);
    int k = 0;
    for (; k + 3 <= n_mine; k += 3) {
      step(k0);
      issue(k0);
      step(k1);
      issue(k1);
      step(k2);
      issue(k2);
    }
    if (k < n_mine) step(k0);
    if (k + 1 < n_mine) step(k1);
  } else {
    u32x4 k0[KTM][2], k1[KTM][2];
    issue(k0);
    issue(k1);
    int k = 0;
    for (; k + 2 <= n_mine; k += 2) {
      step(k0);
      issue(k0);
      step(k1);
      issue(k1);
    }
    if (k < n_mine) step(k0);
  }
  vm_wait<0>();  // the trailing loads (at kOOB) have returned before the wave ends
}

// Key scores of int8/int4 latents with the chunk's key rows staged in LDS once per workgroup.
// Workgroup = block of nch_wg consecutive 32-token chunks (global numbering, possibly spanning
// sequences) x every column tile: wave w takes column tile w (nct waves).  The 32 key rows of a
// chunk are one contiguous span of the cache (32 k_row_bytes bytes); the waves copy it into a
// ring of NST LDS stages by 16-byte DMA (wave w issues the span's 1 KiB pieces w, w + nct, ...,
// DPW of them, the surplus repeating the last piece), NST - 1 chunks ahead of use, with one
// barrier per chunk.  Each wave then reads its K-tiles of the 32 rows from LDS (an int8 lane 16
// bytes, an int4 lane its exact 8 bytes) and runs the MFMAs, softmax statistics and stores of
// k_scores_mix.  Every key byte of a chunk crosses from L2 once per workgroup, where the
// per-column-tile kernel fetched each row's K-tiles once per column tile (whole 64-position
// K-tiles around each tile's few heads: about three times the key bytes on the 13B-class step).
constexpr int kScoresLdsStages = 4;
template <int KTM, int DPW>
__global__ __launch_bounds__(640) void k_scores_lds(ScoreArgs a) {
  constexpr int NST = kScoresLdsStages;
  constexpr int NSTORE = 4;  // vector memory stores per computed chunk (p~ twice, m, l)
  extern __shared__ __align__(16) uint8_t stg_raw[];
  const DecodeGeom& g = a.g;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int NW = g.nct;
  const int n = lane & 15, qq = lane >> 4;
  const int c_first = blockIdx.x * a.nch_wg;
  const int c_end = min(c_first + a.nch_wg, a.total_chunks);
  if (c_first >= c_end) return;  // whole workgroup
  const uint32_t rb = (uint32_t)g.k_row_bytes;
  const uint32_t span = 32u * rb;
  const int npc = (int)((span + 1023u) >> 10);  // 1 KiB pieces of a chunk's rows
  const uint32_t sbytes = (uint32_t)npc << 10;  // bytes of one stage
  const int ct = wave;

  // this lane's DMA: piece j of the wave is span piece min(wave + NW j, npc - 1); lane bytes past
  // the span reload its last 16 bytes (they land past the rows in the stage and are never read)
  uint32_t dsrc[DPW], ddst[DPW];
#pragma unroll
  for (int j = 0; j < DPW; ++j) {
    const int pc = min(wave + NW * j, npc - 1);
    dsrc[j] = min(((uint32_t)pc << 10) + 16u * lane, span - 16u);
    ddst[j] = (uint32_t)pc << 10;
  }

  // K-tiles of the column tile: per-lane byte offset in a key row of the lane's 16 int8 codes or
  // 8 bytes of 16 int4 codes (padding lanes: offset 0; they meet a zero query fragment)
  const int nkt = a.kts.n[ct];
  const int ks0 = a.kts.s0[ct], kn0 = a.kts.n0[ct], ks1 = a.kts.s1[ct];
  uint32_t kofs[KTM];
  bool k8[KTM];
#pragma unroll
  for (int jt = 0; jt < KTM; ++jt) {
    const int kt = jt < kn0 ? ks0 + jt : ks1 + (jt - kn0);
    const int P0 = kt * 64 + 16 * qq;
    const bool on = jt < nkt;
    k8[jt] = on && P0 < g.K8;
    const bool i4 = on && P0 >= g.K8 && P0 < g.K8 + g.K4;
    kofs[jt] = k8[jt] ? (uint32_t)P0 : (i4 ? (uint32_t)(g.K8 + (P0 - g.K8) / 2) : 0u);
  }
  const int i = ct * 16 + n;
  const bool rowvalid = i < g.M_q;
  const bool tile_full = (ct + 1) * 16 <= g.M_q;
  const int jq = i % g.n_q;

  // issue side: chunk ci of sequence bi (of length bi_len)
  int ci = c_first;
  int bi = seq_of_chunk(a.seq, g.B, c_first);
  int bi0 = seq_chunk0(a.seq, bi), bi_end = seq_chunk0(a.seq, bi + 1), bi_len = seq_len(a.seq, bi);
  const uint32_t ring0 = lds_addr(stg_raw);
  const uint8_t* last_base = a.k_rows + ((size_t)bi * g.T_max + (size_t)(ci - bi0) * kTC) * rb;
  auto issue = [&](int st) {
    if (ci < c_end) {  // wave-uniform
      while (ci >= bi_end) {
        ++bi;
        bi0 = bi_end;
        bi_end = seq_chunk0(a.seq, bi + 1);
        bi_len = seq_len(a.seq, bi);
      }
      if ((ci - bi0) * kTC < bi_len) last_base = a.k_rows + ((size_t)bi * g.T_max + (size_t)(ci - bi0) * kTC) * rb;
    }
    // (a chunk past a device length, or past the block's last chunk: the rows of the last live
    // chunk again, from L2, never read; the stage still takes DPW pieces, as the waits count)
#pragma unroll
    for (int j = 0; j < DPW; ++j) lds_dma16(last_base + dsrc[j], ring0 + (uint32_t)st * sbytes + ddst[j]);
    ++ci;
  };

  // query fragments and row parameters of sequence bb
  i32x4 fh[KTM], fl[KTM];
  float rs = 0.f;
  int ibias = 0;
  auto load_seq = [&](int bb) {
    const uint8_t* fbase = a.qfrag + ((size_t)bb * g.nct + ct) * a.nkt_max * 2048;
#pragma unroll
    for (int jt = 0; jt < KTM; ++jt) {
      const int jc = jt < nkt ? jt : 0;
      fh[jt] = __builtin_bit_cast(i32x4, ld16(fbase + jc * 2048 + lane * 16));
      fl[jt] = __builtin_bit_cast(i32x4, ld16(fbase + jc * 2048 + 1024 + lane * 16));
    }
    const u32x4 rp = ld16(a.rowp + ((size_t)bb * g.M_pad + min(i, g.M_q - 1)) * 4);
    rs = __uint_as_float(rp[0]) * (1.f / 254.f);
    ibias = 254 * (int)__uint_as_float(rp[1]) + (int)__uint_as_float(rp[2]);
  };

  int bc = seq_of_chunk(a.seq, g.B, c_first), bf = -1;
  int bc0 = seq_chunk0(a.seq, bc), bc_end = seq_chunk0(a.seq, bc + 1), bc_len = seq_len(a.seq, bc);

#pragma unroll
  for (int u = 0; u < NST - 1; ++u) issue(u);
  // The wait for chunk cc counts what this wave issued after chunk cc's pieces (the vector
  // memory counter drains in issue order, and the compiler barriers keep that order): the pieces
  // of the next NST - 2 chunks ((NST - 2) DPW, in the prologue too) and the stores of the last
  // NST - 1 iterations (NSTORE for each that computed its chunk, none for a skipped chunk or
  // before the first iteration; fragment loads at a sequence start come on top, which only makes
  // the wait stricter).
  uint32_t hist = 0;  // bit j: iteration k - 1 - j computed its chunk
  for (int cc = c_first; cc < c_end; ++cc) {
    const int k = cc - c_first;
    asm volatile("" ::: "memory");
    switch (__builtin_popcount(hist & ((1u << (NST - 1)) - 1u))) {  // wave-uniform
      case 0: vm_wait<(NST - 2) * DPW>(); break;
      case 1: vm_wait<(NST - 2) * DPW + NSTORE>(); break;
      case 2: vm_wait<(NST - 2) * DPW + 2 * NSTORE>(); break;
      case 3: vm_wait<(NST - 2) * DPW + 3 * NSTORE>(); break;
      case 4: vm_wait<(NST - 2) * DPW + 4 * NSTORE>(); break;
      default: vm_wait<(NST - 2) * DPW + 5 * NSTORE>(); break;
    }
    hist <<= 1;
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue((k + NST - 1) % NST);  // into the stage chunk cc - 1 used
    asm volatile("" ::: "memory");
    while (cc >= bc_end) {
      ++bc;
      bc0 = bc_end;
      bc_end = seq_chunk0(a.seq, bc + 1);
      bc_len = seq_len(a.seq, bc);
    }
    const int t0 = (cc - bc0) * kTC;
    if (ct >= NW || t0 >= bc_len) continue;  // past a device length: no value split reads this chunk
    hist |= 1u;
    if (bc != bf) {  // first chunk of a sequence in this block: its fragments
      bf = bc;
      load_seq(bc);
    }
    const uint8_t* st = stg_raw + (size_t)(k % NST) * sbytes;
    i32x4 ah[2], al[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      ah[tt] = i32x4{0, 0, 0, 0};
      al[tt] = i32x4{-ibias, -ibias, -ibias, -ibias};
    }
#pragma unroll
    for (int jt = 0; jt < KTM; ++jt) {
      if (jt < nkt) {  // wave-uniform
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          // 16 bytes at the lane's offset (an int4 lane uses the first 8; the stage has 16
          // bytes of slack past its last row)
          const uint8_t* src = st + (uint32_t)(16 * tt + n) * rb + kofs[jt];
          const u32x2 lo = *(const u32x2*)src;
          const u32x2 hi = *(const u32x2*)(src + 8);
          const i32x4 av = k8[jt] ? i32x4{(int)lo[0], (int)lo[1], (int)hi[0], (int)hi[1]} : unpack_int4_group(lo);
          ah[tt] = mfma16_i8(av, fh[jt], ah[tt]);
          al[tt] = mfma16_i8(av, fl[jt], al[tt]);
        }
      }
    }
    float s2[2][4];
    float m = -INFINITY;
    if (tile_full && t0 + kTC - 1 <= bc_len - g.n_q) {  // wave-uniform: every row sees every token
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          s2[tt][v] = rs * (float)(254 * ah[tt][v] + al[tt][v]);
          m = fmaxf(m, s2[tt][v]);
        }
    } else {
      const int lim = rowvalid ? bc_len - g.n_q + jq : -1;  // last token this row sees
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = t0 + tt * 16 + 4 * qq + v;
          s2[tt][v] = t <= lim ? rs * (float)(254 * ah[tt][v] + al[tt][v]) : -INFINITY;
          m = fmaxf(m, s2[tt][v]);
        }
    }
    m = wave_max_xor(m, 16);
    m = wave_max_xor(m, 32);
    const float mref = m == -INFINITY ? 0.f : m;
    float l = 0.f;
    const size_t prow = ((size_t)cc * g.M_pad + i) * kTC;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float e4[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        e4[v] = __builtin_amdgcn_exp2f(s2[tt][v] - mref);
        l += e4[v];
      }
      const uint32_t w0 = (uint32_t)f32_to_f16(e4[0]) | ((uint32_t)f32_to_f16(e4[1]) << 16);
      const uint32_t w1 = (uint32_t)f32_to_f16(e4[2]) | ((uint32_t)f32_to_f16(e4[3]) << 16);
      st8((uint16_t*)a.p + prow + tt * 16 + 4 * qq, u32x2{w0, w1});
    }
    l = wave_sum_xor(l, 16);
    l = wave_sum_xor(l, 32);
    a.cm[(size_t)cc * g.M_pad + i] = m;
    a.cl[(size_t)cc * g.M_pad + i] = l;
  }
  vm_wait<0>();  // the trailing DMA of the ring has landed before the workgroup ends
}

// Key scores of a rotary layer (keys rotated by position after the key projection): the rotation
// does not commute with B_g, so each key tile is rebuilt from the latent before the dot product
// (STAR-KV summary page, Problem Statement: the reconstruction cost; Methodology section 2: the
// head-wise key factors keep it per head, 2 r_g d_h flops per token and head).  Workgroup =
// (sequence b, KV head g, block of 4 cpw 32-token chunks), four waves of cpw chunks each.
// Staged in LDS once per workgroup: the MFMA A operand of the reconstruction (B_g^T in bf16 for
// bf16 latents; B_g^T with the channel scales folded in, in f16, for int8/int4 latents, whose
// codes are then exact f16), the head's query rows rotated to their positions (high and low f16
// parts, in the register order of the score MFMA's B operand) and the cos/sin of r w_e, r < 32.
// Each wave streams the head's latent bytes of its chunks into its own two LDS stages (4-byte
// LDS DMA, the next chunk in flight while the current one computes) and builds the cos/sin of
// 32 c w_e for each chunk; the rotation of token 32 c + r composes the two (angle sum).  Per chunk:
//   K^T tile  = A x^_g^T              (32x32x16 MFMA; lane = token, 16 of the d_h dims per tile)
//   rotation  of the pairs (e, e + d_h / 2), which sit in the same lane (tiles mt and mt + NT/2)
//   S^T       = K^ Q_rot^T            (32x32x16 f16 MFMA; the K^T registers are the A operand as
//                                      they are; lane = query row, 16 tokens)
// then the chunk statistics and p~ = 2^(s - m) in the format of the other score kernels, for the
// value, merge and up-projection kernels of the latent-space path.  At most 32 query rows per KV
// head (G n_q); d_h = 64 or 128.
struct RopeScoreArgs {
  const uint8_t* k_rows;
  const void* q;           // [B][n_q][H_q][d_h] bf16
  const uint16_t* B_k;     // [n_key][d_h] bf16
  const uint16_t* scales;  // int8/int4: [n_lat] f16
  HeadTables heads;
  void* p;
  float* cm;
  float* cl;
  DecodeGeom g;
  float rope_theta;
  const double* rope_w;    // [d_h / 2] theta^(-2 j / d_h)
  const float2* rope_tab;  // [32][d_h / 2] (cos, sin) of r theta^(-2 j / d_h)
  int rpad;                // staged B_g^T: rows of rpad + 8 halves (rpad = largest key rank rounded to 16)
  int cpw;                 // chunks per wave
  int npair_max;           // dword pairs of a latent stage (both segments), largest over the heads
  SeqTable seq;
};

// sin and cos of a rotation angle formed in fp64 (positions reach 2^15 and more): reduced to
// [-pi, pi] in fp64, then sincosf
__device__ __forceinline__ void rope_sincos(double ang, float* sn, float* cs) {
  constexpr double kTwoPi = 6.283185307179586476925287;
  const double red = ang - kTwoPi * rint(ang / kTwoPi);
  sincosf((float)red, sn, cs);
}

// The byte segments of KV head g in a key row that a latent stage holds, as dwords: bf16, the
// head's channels; int8/int4, its int8 codes (nd8 dwords) then its int4 codes (nd4).  A stage
// keeps each segment dword-pair-major: pair p is 256 bytes, lane l of its DMA holding dword
// 2 p + l / 32 of token l % 32 -- a load of one dword of 32 tokens touches 32 banks.
struct RopeSeg {
  int a8, nd8, a4, nd4;  // byte offsets of the segments' first dwords in the row; dword counts
  int np8, np4;          // dword pairs of each segment
  __host__ __device__ RopeSeg(bool mix, int c0, int rg, int o8, int n8, int o4, int K8) {
    if (mix) {
      a8 = o8 & ~3;
      nd8 = (o8 + n8 - a8 + 3) >> 2;
      const int b4lo = K8 + (o4 >> 1), b4hi = K8 + ((o4 + (rg - n8) + 1) >> 1);
      a4 = b4lo & ~3;
      nd4 = (b4hi - a4 + 3) >> 2;
    } else {
      a8 = (2 * c0) & ~3;
      nd8 = (2 * (c0 + rg) - a8 + 3) >> 2;
      a4 = 0;
      nd4 = 0;
    }
    np8 = (nd8 + 1) >> 1;
    np4 = (nd4 + 1) >> 1;
  }
};

// LDS layout of k_scores_rope (bytes), shared by the kernel and its launch
// qc (query-side chunk rotation): the shared query area holds the rows rotated to their
// positions in fp32, natural dim order ([rows][d_h]); each wave rotates them back by its chunk's
// base angle into its own fragment area (high then low parts) before the chunk's scores.
struct RopeLds {
  int tab_r, q_hi, q_lo, bkt, wave0, wstride, stage, total;
  int qst;   // bytes per staged query row (one part)
  int wst0;  // offset of a wave's stages in its region (its tab_c first, then with qc its fragments)
  __host__ __device__ RopeLds(int d_h, int rpad, int rows, int npair_max, bool qc) {
    const int np = d_h / 2, ks = d_h / 16;
    qst = ks * 32 + 16;
    tab_r = 0;                                    // [32][np + 1] float2
    q_hi = tab_r + 32 * (np + 1) * 8;             // [rows][qst], or with qc [rows][d_h] fp32
    q_lo = q_hi + (qc ? rows * d_h * 4 : rows * qst);
    bkt = q_lo + (qc ? 0 : rows * qst);           // [d_h][rpad + 8] halves
    wave0 = bkt + d_h * (rpad + 8) * 2;           // per wave: tab_c [np] float2, (fragments), two stages
    stage = (npair_max + 1) * 256;  // one pair of slack: windows that run past the segments
    wst0 = np * 8 + (qc ? 2 * rows * qst : 0);
    wstride = wst0 + 2 * stage;
    total = wave0 + 4 * wstride;
  }
};

template <int LAT, int NT, bool QC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_scores_rope(RopeScoreArgs a) {
  constexpr int DH = 32 * NT, NP = DH / 2, KS = 2 * NT;
  constexpr int LPP = 64 / NP;  // qc: lanes per rotation pair (lane l takes pair l % NP)
  constexpr bool MIX = LAT == STARKV_LATENT_MIX84;
  extern __shared__ __align__(16) uint8_t lds[];
  const DecodeGeom& g = a.g;
  const int b = blockIdx.z, gk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r = lane & 31, q = lane >> 5;
  const int nch = seq_nch_live(a.seq, b), len = seq_len(a.seq, b);
  const int cbase = blockIdx.x * 4 * a.cpw;
  if (cbase >= nch) return;  // whole workgroup, before any barrier
  const int rows = g.G * g.n_q;  // query rows of this KV head (at most 32)
  const RopeLds L(DH, a.rpad, rows, a.npair_max, QC);
  const int rst = a.rpad + 8;
  const int c0 = ld_uniform(a.heads.koff + gk);
  const int rg = ld_uniform(a.heads.koff + gk + 1) - c0;
  int n8 = 0, o8 = 0, o4 = 0;
  if (MIX) {
    n8 = ld_uniform(a.heads.n8 + gk);
    o8 = ld_uniform(a.heads.off8 + gk);
    o4 = ld_uniform(a.heads.off4 + gk);
  }
  const RopeSeg sg(MIX, c0, rg, o8, n8, o4, g.K8);
  const int c_first = cbase + wave * a.cpw;
  const int c_last = min(c_first + a.cpw, nch);  // this wave's chunks [c_first, c_last)
  const uint32_t wbase = lds_addr(lds) + L.wave0 + wave * L.wstride;
  float2* tab_c = (float2*)(lds + L.wave0 + wave * L.wstride);

  // latent bytes of chunk c into stage st: buffer loads straight into LDS through a resource that
  // ends at the sequence's last token, so tokens past it read as zero
  const __amdgpu_buffer_rsrc_t krs =
      buf_rsrc(a.k_rows + (size_t)b * g.T_max * g.k_row_bytes, (uint32_t)len * (uint32_t)g.k_row_bytes);
  auto issue = [&](int c, int st) {
    const uint32_t dst = wbase + L.wst0 + st * L.stage;
    const uint32_t vo = (uint32_t)(c * kTC + (lane & 31)) * (uint32_t)g.k_row_bytes + 4 * (lane >> 5);
    for (int pp = 0; pp < sg.np8; ++pp)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)(uintptr_t)(dst + 256 * pp),
                                               4, (int)(vo + sg.a8 + 8 * pp), 0, 0, 0);
    for (int pp = 0; pp < sg.np4; ++pp)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs,
                                               (__attribute__((address_space(3))) void*)(uintptr_t)(dst + 256 * (sg.np8 + pp)),
                                               4, (int)(vo + sg.a4 + 8 * pp), 0, 0, 0);
  };
  if (c_first < c_last) issue(c_first, 0);  // in flight during the set-up

  // inverse frequency of pair j: theta^(-2 j / d_h), from the layer's table
  auto omega = [&](int j) { return a.rope_w[j]; };

  // 1. the reconstruction's A operand: A[e][k] = B_g[k][e] (bf16), or B_g[k][e] s_k (f16); zero
  //    past the rank.  16-byte loads of B_g rows, all issued before the first LDS write.
  {
    constexpr int EV = DH / 8;              // 16-byte vectors per B_g row
    constexpr int MAXIT = 128 * EV / 256;   // rpad <= 128
    const int nv = a.rpad * EV;
    // buffer loads (zero past the head's rows): no branch, all in flight together
    const __amdgpu_buffer_rsrc_t brs = buf_rsrc(a.B_k + (size_t)c0 * DH, (uint32_t)(rg * DH * 2));
    u32x4 v[MAXIT];
    float sc[MAXIT];
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      const int i = tid + 256 * it;
      const int k = i % a.rpad, e0 = (i / a.rpad) * 8;
      const bool on = i < nv && k < rg;
      v[it] = bld16(brs, on ? (uint32_t)((k * DH + e0) * 2) : kOOB);
      if (MIX) sc[it] = f16_to_f32(a.scales[c0 + max(min(k, rg - 1), 0)]);
    }
    uint16_t* bkt = (uint16_t*)(lds + L.bkt);
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      const int i = tid + 256 * it;
      if (i < nv) {
        const int k = i % a.rpad, e0 = (i / a.rpad) * 8;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint16_t hb = (uint16_t)(v[it][u >> 1] >> (16 * (u & 1)));
          uint16_t o = hb;
          if (MIX) o = f32_to_f16(bf16_to_f32(hb) * sc[it]);
          bkt[(e0 + u) * rst + k] = o;
        }
      }
    }
  }
  // 2. cos/sin of r w_j, from the layer's table (rows padded by one pair in LDS)
  {
    float2 t[32 * NP / 256];
#pragma unroll
    for (int it = 0; it < 32 * NP / 256; ++it) t[it] = a.rope_tab[tid + 256 * it];
#pragma unroll
    for (int it = 0; it < 32 * NP / 256; ++it) {
      const int i = tid + 256 * it;
      ((float2*)(lds + L.tab_r))[(i / NP) * (NP + 1) + i % NP] = t[it];
    }
  }
  // 3. query rows rotated to their positions: dim e of row n goes to K-step 2 (e / 32) + (v / 8),
  //    half hq, element v % 8, where e % 32 = d32_row(v, hq) -- the order in which the K^T
  //    registers feed the score MFMA
  {
    constexpr int MAXIT = 32 * NP / 256;
    const int j = tid % NP;
    const double w = omega(j);
    float x0[MAXIT], x1[MAXIT];
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      const int n = min((tid + 256 * it) / NP, rows - 1);  // rows past the head's repeat its last
      const int hq = gk * g.G + n / g.n_q, jq = n % g.n_q;
      const uint16_t* qr = (const uint16_t*)a.q + (((size_t)b * g.n_q + jq) * g.H_q + hq) * DH;
      x0[it] = bf16_to_f32(qr[j]);
      x1[it] = bf16_to_f32(qr[j + NP]);
    }
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      const int n = (tid + 256 * it) / NP;
      if (n < rows) {
        const int pos = len - g.n_q + n % g.n_q;
        float sn, cs;
        rope_sincos((double)pos * w, &sn, &cs);
        const float y0 = x0[it] * cs - x1[it] * sn, y1 = x0[it] * sn + x1[it] * cs;
        if (QC) {
          ((float*)(lds + L.q_hi))[n * DH + j] = y0;
          ((float*)(lds + L.q_hi))[n * DH + j + NP] = y1;
          continue;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = j + h * NP;
          const float y = h ? y1 : y0;
          const int e32 = e & 31;
          const int vv = 4 * (e32 >> 3) + (e32 & 3), half = (e32 >> 2) & 1;
          const int ks = 2 * (e >> 5) + (vv >> 3);
          const int off = n * L.qst + (ks * 2 + half) * 16 + (vv & 7) * 2;
          const _Float16 yh = (_Float16)y;
          *(_Float16*)(lds + L.q_hi + off) = yh;
          *(_Float16*)(lds + L.q_lo + off) = (_Float16)(y - (float)yh);
        }
      }
    }
  }
  __syncthreads();

  // cos/sin of the chunk base angle 32 c w_j for pair j = lane % NP, advanced chunk by chunk by
  // the angle sum with 32 w_j (a few roundings of 2^-24 over at most eight steps)
  float ccs, csn, c32, s32;
  {
    const double wl = omega(lane % NP);
    rope_sincos((double)(c_first * kTC) * wl, &csn, &ccs);
    rope_sincos((double)kTC * wl, &s32, &c32);
  }
  const int lim = r < rows ? len - g.n_q + r % g.n_q : -1;  // last token row r sees
  const int ig = gk * rows + r;                             // the row among the sequence's rows
  const int qrow = min(r, rows - 1) * L.qst;
  const uint16_t* bkt = (const uint16_t*)(lds + L.bkt);
  for (int c = c_first; c < c_last; ++c) {
    const int st = (c - c_first) & 1;
    vm_wait<0>();  // this wave's latent bytes of chunk c are in its stage
    asm volatile("" ::: "memory");
    uint8_t* wq = lds + L.wave0 + wave * L.wstride + NP * 8;  // qc: this wave's query fragments
    if (QC) {
      // the query rows rotated back by the chunk's base angle 32 c w_j (the keys then turn by
      // their offset in the chunk only): lane l takes pair j = l % NP of rows l / NP + LPP i
      const int j = lane % NP;
      const float* qf = (const float*)(lds + L.q_hi);
      for (int n = lane / NP; n < rows; n += LPP) {
        const float x0 = qf[n * DH + j], x1 = qf[n * DH + j + NP];
        const float y0 = x0 * ccs + x1 * csn, y1 = x1 * ccs - x0 * csn;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = j + h * NP;
          const float y = h ? y1 : y0;
          const int e32 = e & 31;
          const int vv = 4 * (e32 >> 3) + (e32 & 3), half = (e32 >> 2) & 1;
          const int ks = 2 * (e >> 5) + (vv >> 3);
          const int off = n * L.qst + (ks * 2 + half) * 16 + (vv & 7) * 2;
          const _Float16 yh = (_Float16)y;
          *(_Float16*)(wq + off) = yh;
          *(_Float16*)(wq + rows * L.qst + off) = (_Float16)(y - (float)yh);
        }
      }
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0): the fragments are written
    } else if (lane < NP) {
      tab_c[lane] = float2{ccs, csn};
    }
    {
      const float nc = ccs * c32 - csn * s32, ns = csn * c32 + ccs * s32;
      ccs = nc;
      csn = ns;
    }
    __builtin_amdgcn_wave_barrier();
    if (c + 1 < c_last) issue(c + 1, st ^ 1);
    // 1. K^T tile: lane (token 32 c + r) holds dims 32 mt + d32_row(v, q)
    const uint8_t* seg8 = lds + L.wave0 + wave * L.wstride + L.wst0 + st * L.stage + 4 * r;
    const uint8_t* seg4 = seg8 + 256 * sg.np8;
    // dword dw of this lane's token in a segment (dw >= -1; -1 lands in the pair before)
    auto ldw = [&](const uint8_t* sb, int dw) { return *(const uint32_t*)(sb + 256 * (dw >> 1) + 128 * (dw & 1)); };
    const int dlim8 = 2 * sg.np8 - 1, dlim4 = 2 * sg.np4 - 1;  // last loaded dword of each segment
    f32x16 kt[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) kt[mt][v] = 0.f;
    for (int k0 = 0; k0 < rg; k0 += 16) {
      const int kb = k0 + 8 * q;
      const bool last = k0 + 16 > rg;  // the partial K-step: channels past the rank are masked
      uint32_t w[4];
      if (!MIX) {
        // channels kb .. kb + 7: dwords kb / 2 .. kb / 2 + 4 of the segment (one more when c0 is odd)
        const int d0 = kb / 2;
        uint32_t d[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) d[i] = ldw(seg8, last ? min(d0 + i, dlim8) : d0 + i);
        const uint32_t sh = (uint32_t)(c0 & 1) * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __builtin_amdgcn_alignbit(d[i + 1], d[i], sh);
        if (last) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t mlo = kb + 2 * i < rg ? 0xFFFFu : 0u;
            const uint32_t mhi = kb + 2 * i + 1 < rg ? 0xFFFF0000u : 0u;
            w[i] &= mlo | mhi;
          }
        }
      } else {
        // int8 codes of channels kb .. kb + 7 (bytes o8 - a8 + kb ..), and int4 codes of the
        // same channels (nibbles o4 + kb - n8 .. of the int4 segment); each channel takes one
        int code[8];
        {
          // past the int8 codes the window is clamped (same alignment; its bytes go unused)
          const int d0 = min(kb, n8 & ~7) / 4;
          const uint32_t sh = (uint32_t)(o8 - sg.a8) * 8;
          const uint32_t e0 = ldw(seg8, d0), e1 = ldw(seg8, min(d0 + 1, dlim8)), e2 = ldw(seg8, min(d0 + 2, dlim8));
          const uint32_t lo = __builtin_amdgcn_alignbit(e1, e0, sh), hi = __builtin_amdgcn_alignbit(e2, e1, sh);
#pragma unroll
          for (int i = 0; i < 8; ++i) code[i] = __builtin_amdgcn_sbfe((int)(i < 4 ? lo : hi), 8 * (i & 3), 8);
        }
        {
          // nibble offset from the int4 segment's first byte (>= -7: the window may start in the
          // dword before the segment when it begins with int8 channels)
          int nb = (o4 + kb - n8) - 2 * (sg.a4 - g.K8);
          if (nb < -7) nb &= 7;  // all eight channels are int8 ones: any window of the same phase
          const int f = (4 * nb) >> 5;  // dword of the first nibble (arithmetic shift: -1 for nb < 0)
          const uint32_t f0 = ldw(seg4, min(f, dlim4)), f1 = ldw(seg4, min(f + 1, dlim4));
          const uint32_t w4 = __builtin_amdgcn_alignbit(f1, f0, (uint32_t)((4 * nb) & 31));
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (kb + i >= n8) code[i] = __builtin_amdgcn_sbfe((int)w4, 4 * i, 4);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c_lo = (!last || kb + 2 * i < rg) ? code[2 * i] : 0;
          const int c_hi = (!last || kb + 2 * i + 1 < rg) ? code[2 * i + 1] : 0;
          const _Float16 h0 = (_Float16)(short)c_lo, h1 = (_Float16)(short)c_hi;
          w[i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        }
      }
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const u32x4 at = *(const u32x4*)(bkt + (mt * 32 + r) * rst + kb);
        if (MIX)
          kt[mt] = mfma32_f16(__builtin_bit_cast(f16x8, at), __builtin_bit_cast(f16x8, u32x4{w[0], w[1], w[2], w[3]}),
                              kt[mt]);
        else
          kt[mt] = mfma32_bf16(as_bf16x8(at), as_bf16x8(u32x4{w[0], w[1], w[2], w[3]}), kt[mt]);
      }
    }
    // 2. rotation of the key at position t = 32 c + r by the angle sum of the two tables
    const float2* tr = (const float2*)(lds + L.tab_r) + r * (NP + 1);
#pragma unroll
    for (int mt = 0; mt < NT / 2; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = mt * 32 + d32_row(v, q);
        const float2 tt = tr[j];
        float cs = tt.x, sn = tt.y;
        if (!QC) {
          const float2 tc = tab_c[j];
          cs = tc.x * tt.x - tc.y * tt.y;
          sn = tc.y * tt.x + tc.x * tt.y;
        }
        const float x0 = kt[mt][v], x1 = kt[mt + NT / 2][v];
        kt[mt][v] = x0 * cs - x1 * sn;
        kt[mt + NT / 2][v] = x0 * sn + x1 * cs;
      }
    // 3. S^T: lane (query row n = r, half q) holds tokens 32 c + d32_row(v, q)
    f32x16 s;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      f16x8 ak;
#pragma unroll
      for (int i = 0; i < 8; ++i) ak[i] = (_Float16)kt[ks >> 1][8 * (ks & 1) + i];
      const int off = qrow + (ks * 2 + q) * 16;
      const uint8_t* qh = QC ? wq : lds + L.q_hi;
      const uint8_t* ql = QC ? wq + rows * L.qst : lds + L.q_lo;
      s = mfma32_f16(ak, *(const f16x8*)(qh + off), s);
      s = mfma32_f16(ak, *(const f16x8*)(ql + off), s);
    }
    // 4. mask (only where a token of the chunk lies past some row's last; lanes past the head's
    //    rows hold finite values that are never stored), chunk statistics, p~
    float m = -INFINITY;
    if (c * kTC + kTC - 1 <= len - g.n_q) {  // wave-uniform: every row sees every token
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        s[v] *= g.qscale;
        m = fmaxf(m, s[v]);
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tt = c * kTC + d32_row(v, q);
        s[v] = tt <= lim ? s[v] * g.qscale : -INFINITY;
        m = fmaxf(m, s[v]);
      }
    }
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    // exp2(-inf - m) is 0; a row with no visible token keeps m = -inf and takes 0 for reference
    const float mref = m == -INFINITY ? 0.f : m;
    float l = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s[v] = __builtin_amdgcn_exp2f(s[v] - mref);
      l += s[v];
    }
    l += __shfl_xor(l, 32, 64);
    if (r < rows) {
      const size_t cgl = (size_t)seq_chunk0(a.seq, b) + c;
      const size_t prow = (cgl * g.M_pad + ig) * kTC;
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int tt = 8 * v4 + 4 * q;  // tokens tt .. tt + 3 of the chunk
        uint32_t w0, w1;
        if (MIX) {
          w0 = (uint32_t)f32_to_f16(s[4 * v4]) | ((uint32_t)f32_to_f16(s[4 * v4 + 1]) << 16);
          w1 = (uint32_t)f32_to_f16(s[4 * v4 + 2]) | ((uint32_t)f32_to_f16(s[4 * v4 + 3]) << 16);
        } else {
          w0 = (uint32_t)f32_to_bf16(s[4 * v4]) | ((uint32_t)f32_to_bf16(s[4 * v4 + 1]) << 16);
          w1 = (uint32_t)f32_to_bf16(s[4 * v4 + 2]) | ((uint32_t)f32_to_bf16(s[4 * v4 + 3]) << 16);
        }
        st8((uint16_t*)a.p + prow + tt, u32x2{w0, w1});
      }
      if (q == 0) {
        a.cm[cgl * g.M_pad + ig] = m;
        a.cl[cgl * g.M_pad + ig] = l;
      }
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
  void* zp;  // split partials (fp32, or f16 scaled by zsc: int8/int4 latents)
  float zsc;  // int8/int4 latents: power-of-two scale of the f16 partials
  float* sl;
  float* sm;
  DecodeGeom g;
  SeqTable seq;
  int cps, bpw, NB, V8, n8v, n4v;
  int n_sl8;  // one-M-tile kernel: slices of one-N-tile blocks (the rest hold int4 blocks)
  int n_sl4;  // one-M-tile kernel: slices of int4 blocks (packed layout: then 3-bit N-tiles)
  int NB4;    // end of the int4 blocks (packed layout: the outlier blocks, V4 / 64)
  int n3t;    // packed layout: 3-bit N-tiles (V3 / 32)
  int V4;     // packed layout: outlier channels (the 3-bit stream starts at row V4 / 2)
  int n_sl, n_splits;  // one-M-tile kernel: slices per split, splits in all
  ValueOrder vo;       // split of each grid position (vo.n = 0: the kernel's own order)
};
static_assert(sizeof(ValueArgs) <= 4096, "value kernel arguments");

// Largest of the chunk maxima cm[c][row] over chunks c = c0, c0 + step, ... (n >= 1 of them),
// NL loads at a time: the reference against which a value kernel weights its tiles.
template <int NL = 8>
__device__ __forceinline__ float chunks_max(const float* cm, int c0, int step, int n, int M_pad, size_t row) {
  float m = -INFINITY;
  for (int k0 = 0; k0 < n; k0 += NL) {
    float v[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) v[u] = cm[(size_t)(c0 + step * min(k0 + u, n - 1)) * M_pad + row];
#pragma unroll
    for (int u = 0; u < NL; ++u) m = fmaxf(m, v[u]);
  }
  return m;
}

// Weight 2^(m - ref) of a partial whose maximum is m, against the reference ref >= m (0 for an
// empty partial, m = -inf).
__device__ __forceinline__ float rel_weight(float m, float ref) {
  return m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - ref);
}

// 8 tokens of one channel (int8 codes in 8 bytes) -> f16x8
__device__ __forceinline__ f16x8 deq_i8x8(uint32_t w0, uint32_t w1) {
  // exact: a byte b in offset binary (b ^ 0x80) is the low mantissa of the half 0x6400 | u =
  // 1024 + u, and one packed subtraction of 1024 + 128 gives the code; bytes 2k, 2k + 1 of a word
  // go to the two halves of one dword by a byte permute (zeros between them)
  const u32x4 u = {__builtin_amdgcn_perm(0u, w0, 0x0C010C00u) ^ 0x64806480u,
                   __builtin_amdgcn_perm(0u, w0, 0x0C030C02u) ^ 0x64806480u,
                   __builtin_amdgcn_perm(0u, w1, 0x0C010C00u) ^ 0x64806480u,
                   __builtin_amdgcn_perm(0u, w1, 0x0C030C02u) ^ 0x64806480u};
  return __builtin_bit_cast(f16x8, u) - (_Float16)1152.0f;
}
// 8 tokens of one channel of an int4 pair (8 bytes; the even channel in the low nibbles, the odd
// one in the high nibbles; `odd` picks which), exactly: the nibble in offset binary (n ^ 8) is
// the low mantissa of the half 0x6400 | u, minus 1024 + 8
__device__ __forceinline__ f16x8 deq_i4x8_half(uint32_t w0, uint32_t w1, bool odd) {
  const int sh = odd ? 4 : 0;
  const uint32_t a = w0 >> sh, b = w1 >> sh;
  const u32x4 u = {(__builtin_amdgcn_perm(0u, a, 0x0C010C00u) & 0x000F000Fu) ^ 0x64086408u,
                   (__builtin_amdgcn_perm(0u, a, 0x0C030C02u) & 0x000F000Fu) ^ 0x64086408u,
                   (__builtin_amdgcn_perm(0u, b, 0x0C010C00u) & 0x000F000Fu) ^ 0x64086408u,
                   (__builtin_amdgcn_perm(0u, b, 0x0C030C02u) & 0x000F000Fu) ^ 0x64086408u};
  return __builtin_bit_cast(f16x8, u) - (_Float16)1032.0f;
}
// 8 tokens of one channel of an int4 pair (8 bytes): low nibbles -> even channel, high -> odd channel
__device__ __forceinline__ void deq_i4x8(uint32_t w0, uint32_t w1, f16x8& ev, f16x8& od) {
  ev = deq_i4x8_half(w0, w1, false);
  od = deq_i4x8_half(w0, w1, true);
}
// 8 tokens (byte `by` of the three token-plane words) of one packed 3-bit channel, exactly.
// The three plane bytes side by side (bits 0-7, 8-15, 16-23) hold tokens 2w and 2w + 1 of the
// byte at bits w and 4 + w; shifted by w and masked, the six bits multiplied by 0x4081
// (= 2^14 + 2^7 + 1) land without overlap at 14-16 (field of token 2w) and 18-20 (token
// 2w + 1).  Each field f = code + 4 becomes the half 0x6400 | f = 1024 + f, minus 1028.
__device__ __forceinline__ f16x8 deq_i3x8(uint32_t p0, uint32_t p1, uint32_t p2, int by) {
  const uint32_t sh = 8u * (uint32_t)by;
  const uint32_t B = ((p0 >> sh) & 0xFFu) | (((p1 >> sh) & 0xFFu) << 8) | (((p2 >> sh) & 0xFFu) << 16);
  u32x4 u;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t y = __umul24((B >> w) & 0x111111u, 0x4081u);
    u[w] = 0x64006400u | ((y >> 14) & 7u) | (((y >> 18) & 7u) << 16);
  }
  return __builtin_bit_cast(f16x8, u) - (_Float16)1028.0f;
}

// Workgroup = (slice of `bpw` value blocks, split of one sequence); wave = one value block
// (32 byte-rows of the value tiles).  The split's 32-token tiles are walked U at a time: the
// value rows, probabilities and chunk statistics of U tiles are loaded before their MFMAs.
template <int LAT, int NMT>
__global__ __launch_bounds__(256) void k_values(ValueArgs a) {
  constexpr int U = (LAT == STARKV_LATENT_F32) ? 1 : (NMT >= 3 ? 1 : (NMT == 2 ? 2 : 4));
  constexpr int esz = LAT == STARKV_LATENT_F32 ? 4 : (LAT == STARKV_LATENT_BF16 ? 2 : 1);
  constexpr int NV = esz == 1 ? 1 : (esz == 2 ? 2 : 4);  // 16-byte value loads per lane per tile
  constexpr int NP = LAT == STARKV_LATENT_F32 ? 2 : 1;   // 16-byte probability loads per lane per K-step
  const DecodeGeom& g = a.g;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int nb = blockIdx.x * a.bpw + wave;  // value block of this wave (wave-uniform)
  if (nb >= a.NB) return;
  const int sg = blockIdx.y;
  const int b = seq_of_split(a.seq, g.B, sg);
  const int s = sg - seq_split0(a.seq, b);
  const int cbase = seq_chunk0(a.seq, b);
  const int nch = seq_nch_live(a.seq, b);
  const int c_lo = s * a.cps, c_hi = min(c_lo + a.cps, nch);
  if (c_lo >= nch) return;  // a split past a device length (whole workgroup): the merges skip it
  const int len = seq_len(a.seq, b);
  const int r = lane & 31, q = lane >> 5;
  const bool is4 = (LAT == STARKV_LATENT_MIX84) && (nb >= a.V8 / 32);

  // maximum over the split's chunks of the rows this lane feeds as A-fragment rows: the
  // reference of this split's weights
  float Ms[NMT], lsum[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int row = min(mt * 32 + r, g.M_q - 1);
    Ms[mt] = chunks_max(a.cm, cbase + c_lo, 1, c_hi - c_lo, g.M_pad, row);
    lsum[mt] = 0.f;
  }

  f32x16 acc[NMT][2];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][nt][v] = 0.f;

  constexpr int blkb = 32 * kTT * esz;  // bytes of one 32-row block of a tile
  const uint8_t* vb = a.v_tiles + vblock_off(b, nb, 0, g.v_rows, g.T_max, esz) + (size_t)r * kTT * esz;
  for (int c0 = c_lo; c0 < c_hi; c0 += U) {
    u32x4 vr[U][NV];
    u32x4 pr[U][NMT][2][NP];
    float cmv[U][NMT], clv[U][NMT];
    // ---- loads of U tiles
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u;
      const bool on = c < c_hi;  // uniform
      const size_t cgl = (size_t)(cbase + (on ? c : c_lo));
      const uint8_t* trow = vb + (size_t)(on ? c : c_lo) * blkb;
#pragma unroll
      for (int k = 0; k < NV; ++k) vr[u][k] = on ? ld16(trow + 16 * NV * q + 16 * k) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int row = mt * 32 + r;
        const bool rok = on && row < g.M_q;
        cmv[u][mt] = rok ? a.cm[cgl * g.M_pad + row] : -INFINITY;
        clv[u][mt] = rok ? a.cl[cgl * g.M_pad + row] : 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int k = 0; k < NP; ++k) {
            const size_t pe = (cgl * g.M_pad + row) * kTC + 16 * q + 8 * h + 4 * k;
            pr[u][mt][h][k] = rok ? (LAT == STARKV_LATENT_F32 ? ld16((const float*)a.p + pe)
                                                              : ld16((const uint16_t*)a.p + pe))
                                  : u32x4{0, 0, 0, 0};
          }
      }
    }
    // ---- compute
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u;
      if (c >= c_hi) break;
      const int tt0 = c * kTC;
      float alpha[NMT];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const float m = cmv[u][mt];
        alpha[mt] = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - Ms[mt]);
        lsum[mt] += alpha[mt] * clv[u][mt];
      }
      if (esz > 1 && tt0 + kTT > len) {
        // zero the elements of tokens at or past the length (their bits may be anything)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t = tt0 + 16 * q + e;
          if (t >= len) {
            if (esz == 2) {
              const uint32_t keep = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
              vr[u][e >> 3][(e >> 1) & 3] = vr[u][e >> 3][(e >> 1) & 3] & keep;
            } else {
              vr[u][e >> 2][e & 3] = 0u;
            }
          }
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // value fragments of this K-step (8 tokens of one channel, or of a channel pair)
        f16x8 v_lo, v_hi;
        if (LAT == STARKV_LATENT_MIX84) {
          const uint32_t w0 = vr[u][0][2 * h], w1 = vr[u][0][2 * h + 1];
          if (is4) deq_i4x8(w0, w1, v_lo, v_hi);
          else v_lo = deq_i8x8(w0, w1);
        }
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          if (LAT == STARKV_LATENT_F32) {
            const u32x4 p0 = pr[u][mt][h][0], p1 = pr[u][mt][h][NP - 1];
            const u32x4 v0 = vr[u][2 * h], v1 = vr[u][2 * h + 1];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[mt][0] = mfma32_f32(__uint_as_float(p0[e]) * alpha[mt], __uint_as_float(v0[e]), acc[mt][0]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[mt][0] = mfma32_f32(__uint_as_float(p1[e]) * alpha[mt], __uint_as_float(v1[e]), acc[mt][0]);
          } else if (LAT == STARKV_LATENT_BF16) {
            const u32x4 praw = pr[u][mt][h][0];
            u32x4 ps;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x0 = bf16_to_f32((uint16_t)(praw[e] & 0xFFFF)) * alpha[mt];
              const float x1 = bf16_to_f32((uint16_t)(praw[e] >> 16)) * alpha[mt];
              ps[e] = (uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16);
            }
            acc[mt][0] = mfma32_bf16(as_bf16x8(ps), as_bf16x8(vr[u][h]), acc[mt][0]);
          } else {
            const f16x8 pin = as_f16x8(pr[u][mt][h][0]);
            f16x8 ps;
#pragma unroll
            for (int e = 0; e < 8; ++e) ps[e] = (_Float16)((float)pin[e] * alpha[mt]);
            acc[mt][0] = mfma32_f16(ps, v_lo, acc[mt][0]);
            if (is4) acc[mt][1] = mfma32_f16(ps, v_hi, acc[mt][1]);
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
        if (row < g.M_q) ((float*)a.zp)[((size_t)sg * g.M_pad + row) * g.rv_ld + vc] = acc[mt][nt][v];
      }
  }
  if (blockIdx.x == 0 && wave == 0 && q == 0) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int row = mt * 32 + r;
      if (row < g.M_q) {
        a.sl[(size_t)sg * g.M_pad + row] = lsum[mt];
        a.sm[(size_t)sg * g.M_pad + row] = Ms[mt];
      }
    }
  }
}

// One M-tile (at most 32 query rows per sequence): workgroup = (slice of value blocks of one
// kind, split of one sequence); the four waves take interleaved 32-token tiles of the split and
// each covers every block of the slice, so a probability fragment feeds up to four N-tiles.
// Slices [0, n_sl8) hold NBW8 blocks of one N-tile each (int8, bf16 or fp32 rows), slices
// [n_sl8, ...) NBW4 int4 blocks (two N-tiles each: even and odd channels of the byte pairs).
// Each wave double-buffers its tile loads in registers (the loads of the next U tiles go out
// before the MFMAs of the current U).  The waves' accumulators and probability sums are added
// through LDS at the end.
template <int LAT>
struct VLayout {
  static constexpr int esz = LAT == STARKV_LATENT_F32 ? 4 : (LAT == STARKV_LATENT_BF16 ? 2 : 1);
  static constexpr int NV = esz == 1 ? 1 : (esz == 2 ? 2 : 4);  // 16-byte value loads per lane per block
  static constexpr int NP = LAT == STARKV_LATENT_F32 ? 2 : 1;   // 16-byte probability loads per half
};

template <int LAT, int NBW>
struct VTile {
  u32x4 v[NBW][VLayout<LAT>::NV];
  u32x4 p[2][VLayout<LAT>::NP];
  float cm, cl;
};

// KIND 0: one-N-tile blocks (int8, bf16, fp32 rows); 1: int4 blocks (two N-tiles: even and odd
// channels); 2: packed 3-bit N-tiles (32 channels of the 3-bit stream; nb0 counts N-tiles).
template <int LAT, int NBW, int KIND>
__device__ __forceinline__ void values1_run(const ValueArgs& a, int slice, int sg, int nb0, int nblk,
                                            float* sred, float (*ssum)[32], float (*smx)[32]) {
  using VL = VLayout<LAT>;
  constexpr bool IS4 = KIND == 1;
  constexpr int NT = IS4 ? 2 * NBW : NBW;  // accumulator tiles
  constexpr int TU = NBW * VL::NV + 2 * VL::NP;  // 16-byte loads per lane per tile
  constexpr int U = TU <= 6 ? 2 : 1;       // tiles per pipeline stage
  const DecodeGeom& g = a.g;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int r = lane & 31, q = lane >> 5;
  const int b = seq_of_split(a.seq, g.B, sg);
  const int s = sg - seq_split0(a.seq, b);
  const int cbase = seq_chunk0(a.seq, b);
  const int nch = seq_nch_live(a.seq, b);
  const int c_lo = s * a.cps, c_hi = min(c_lo + a.cps, nch);
  if (c_lo >= nch) return;  // a split past a device length (whole workgroup): the merges skip it
  const int len = seq_len(a.seq, b);
  const bool rok = r < g.M_q;
  const size_t prow = (size_t)(rok ? r : 0);
  // tiles of this wave: chunks c_lo + wave + 4k, k < ntw (wave-uniform), walked from k = rot on
  // (cyclically): the slices of one split start on different tiles, so they do not all fetch the
  // same probability tile at the same moment
  const int ntw = c_lo + wave < c_hi ? (c_hi - c_lo - wave + 3) / 4 : 0;
  const int rot = ntw > 0 ? slice % ntw : 0;
  auto chunk_of = [&](int k) {
    const int kk = k + rot;
    return c_lo + wave + 4 * (kk >= ntw ? kk - ntw : kk);
  };
  constexpr int blkb = 32 * kTT * VL::esz;  // bytes of one 32-row block of a tile
  const uint8_t* vb = a.v_tiles + vblock_off(b, 0, 0, g.v_rows, g.T_max, VL::esz) + r * kTT * VL::esz + 16 * VL::NV * q;
  size_t boff[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) boff[j] = vblock_off(0, nb0 + (j < nblk ? j : 0), 0, g.v_rows, g.T_max, VL::esz);
  // packed 3-bit N-tiles: the lane's channel k = 32 (nb0 + j) + r has its three words at stream
  // bytes 12 k + 4 pb, stream byte x in row V4 / 2 + x / 32, column x % 32
  const uint8_t* vb3 = a.v_tiles + vblock_off(b, 0, 0, g.v_rows, g.T_max, 1);
  size_t off3[KIND == 2 ? NBW : 1][3];
  if (KIND == 2) {
#pragma unroll
    for (int j = 0; j < (KIND == 2 ? NBW : 1); ++j)
#pragma unroll
      for (int pb = 0; pb < 3; ++pb) {
        const int x = 12 * (32 * (nb0 + (j < nblk ? j : 0)) + r) + 4 * pb;
        const int row = a.V4 / 2 + (x >> 5);
        off3[j][pb] = vblock_off(0, row >> 5, 0, g.v_rows, g.T_max, 1) + (size_t)(row & 31) * kTT + (x & 31);
      }
  }

  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;
  float lsum = 0.f;
  float M = -INFINITY;  // this wave's reference: the largest chunk maximum of its tiles (its row)

  auto load = [&](VTile<LAT, NBW>& t, int k) {
    const int c = chunk_of(min(k, ntw - 1));
    const uint8_t* tb = vb + (size_t)c * blkb;
    if (KIND == 2) {
      const uint8_t* tb3 = vb3 + (size_t)c * blkb;
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        t.v[j][0] = u32x4{*(const uint32_t*)(tb3 + off3[j % (KIND == 2 ? NBW : 1)][0]),
                          *(const uint32_t*)(tb3 + off3[j % (KIND == 2 ? NBW : 1)][1]),
                          *(const uint32_t*)(tb3 + off3[j % (KIND == 2 ? NBW : 1)][2]), 0u};
    } else {
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int x = 0; x < VL::NV; ++x) t.v[j][x] = ld16(tb + boff[j] + 16 * x);
    }
    const size_t cr = (size_t)(cbase + c) * g.M_pad + prow;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int x = 0; x < VL::NP; ++x) {
        const size_t pe = cr * kTC + 16 * q + 8 * h + 4 * x;
        t.p[h][x] = LAT == STARKV_LATENT_F32 ? ld16((const float*)a.p + pe) : ld16((const uint16_t*)a.p + pe);
      }
    t.cm = a.cm[cr];
    t.cl = a.cl[cr];
  };

  auto compute = [&](VTile<LAT, NBW>& t, int k) {
    if (k >= ntw) return;  // uniform
    const int tt0 = chunk_of(k) * kTC;
    // rows past M_q read row 0's statistics; their results are never stored
    const float alpha = (t.cm == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(t.cm - M);
    lsum += alpha * t.cl;
    if (VL::esz > 1 && tt0 + kTT > len) {
      // zero the elements of tokens at or past the length (their bits may be anything)
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int tok = tt0 + 16 * q + e;
          if (tok >= len) {
            if (VL::esz == 2) {
              const uint32_t keep = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
              t.v[j][e >> 3][(e >> 1) & 3] &= keep;
            } else {
              t.v[j][e >> 2][e & 3] = 0u;
            }
          }
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (LAT == STARKV_LATENT_F32) {
        const u32x4 p0 = t.p[h][0], p1 = t.p[h][VL::NP - 1];
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          if (j >= nblk) continue;
          const u32x4 v0 = t.v[j][2 * h], v1 = t.v[j][(2 * h + 1) % VL::NV];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[j] = mfma32_f32(__uint_as_float(p0[e]) * alpha, __uint_as_float(v0[e]), acc[j]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[j] = mfma32_f32(__uint_as_float(p1[e]) * alpha, __uint_as_float(v1[e]), acc[j]);
        }
      } else if (LAT == STARKV_LATENT_BF16) {
        const u32x4 praw = t.p[h][0];
        u32x4 ps;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = bf16_to_f32((uint16_t)(praw[e] & 0xFFFF)) * alpha;
          const float x1 = bf16_to_f32((uint16_t)(praw[e] >> 16)) * alpha;
          ps[e] = (uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16);
        }
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          if (j >= nblk) continue;
          acc[j] = mfma32_bf16(as_bf16x8(ps), as_bf16x8(t.v[j][h % VL::NV]), acc[j]);
        }
      } else {
        const f16x8 pin = as_f16x8(t.p[h][0]);
        f16x8 ps;
#pragma unroll
        for (int e = 0; e < 8; ++e) ps[e] = (_Float16)((float)pin[e] * alpha);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          if (j >= nblk) continue;
          if (KIND == 2) {
            acc[j] = mfma32_f16(ps, deq_i3x8(t.v[j][0][0], t.v[j][0][1], t.v[j][0][2], 2 * q + h), acc[j]);
          } else if (!IS4) {
            acc[j] = mfma32_f16(ps, deq_i8x8(t.v[j][0][2 * h], t.v[j][0][2 * h + 1]), acc[j]);
          } else {
            f16x8 ev, od;
            deq_i4x8(t.v[j][0][2 * h], t.v[j][0][2 * h + 1], ev, od);
            acc[(2 * j) % NT] = mfma32_f16(ps, ev, acc[(2 * j) % NT]);
            acc[(2 * j + 1) % NT] = mfma32_f16(ps, od, acc[(2 * j + 1) % NT]);
          }
        }
      }
    }
  };

  if (ntw > 0) {
    // the chunk maxima of the wave's first 8 tiles go out first, then two register buffers of U
    // tiles each; a buffer's next loads go out before the other buffer's MFMAs.  Loads of tiles
    // past the wave's last are clamped to it (L2 hits), except for the refills, which are skipped
    // (uniform branches) when no tile is left.
    float cmx[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      cmx[u] = a.cm[(size_t)(cbase + c_lo + wave + 4 * min(u, ntw - 1)) * g.M_pad + prow];
    __builtin_amdgcn_sched_barrier(0);
    VTile<LAT, NBW> ta[U], tb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load(ta[u], u);
#pragma unroll
    for (int u = 0; u < U; ++u) load(tb[u], U + u);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 8; ++u) M = fmaxf(M, cmx[u]);
    if (ntw > 8) M = fmaxf(M, chunks_max(a.cm, cbase + c_lo + wave + 32, 4, ntw - 8, g.M_pad, prow));
    for (int k0 = 0; k0 < ntw; k0 += 2 * U) {
#pragma unroll
      for (int u = 0; u < U; ++u) compute(ta[u], k0 + u);
      if (k0 + U >= ntw) break;
      if (k0 + 2 * U < ntw) {
#pragma unroll
        for (int u = 0; u < U; ++u) load(ta[u], k0 + 2 * U + u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) compute(tb[u], k0 + U + u);
      if (k0 + 3 * U < ntw) {
#pragma unroll
        for (int u = 0; u < U; ++u) load(tb[u], k0 + 3 * U + u);
      }
    }
  }

  // add the four waves' accumulators and sums, each weighted against the split's maximum of the
  // row (the largest of the waves' references): every wave parks its accumulators in LDS, then
  // wave w adds and stores elements v = 4w .. 4w + 3 of every tile
  const int ntile = IS4 ? 2 * nblk : nblk;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t >= ntile) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) sred[((wave * NT + t) * 16 + v) * 64 + lane] = acc[t][v];
  }
  if (q == 0) {
    ssum[wave][r] = lsum;
    smx[wave][r] = M;
  }
  __syncthreads();
  // weights of the four waves for the rows of elements 4w .. 4w + 3
  float fw[4][4];
#pragma unroll
  for (int vv = 0; vv < 4; ++vv) {
    const int row = d32_row(4 * wave + vv, q);
    const float ms = fmaxf(fmaxf(smx[0][row], smx[1][row]), fmaxf(smx[2][row], smx[3][row]));
#pragma unroll
    for (int w = 0; w < 4; ++w) fw[vv][w] = rel_weight(smx[w][row], ms);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t >= ntile) continue;
    int vc;
    bool cok;
    if (KIND == 2) {
      const int w = (nb0 + t) * 32 + r;  // inlier channel
      cok = w < a.n4v;
      vc = a.n8v + w;
    } else if (!IS4) {
      vc = (nb0 + t) * 32 + r;
      cok = vc < (LAT == STARKV_LATENT_MIX84 ? a.n8v : g.r_v);
    } else {
      const int w = 2 * ((nb0 + t / 2 - a.V8 / 32) * 32 + r) + (t & 1);
      // the nibble pairs hold the int4 block, or with the packed layout the outliers
      cok = w < (g.pack3 ? a.n8v : a.n4v);
      vc = g.pack3 ? w : a.n8v + w;
    }
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) {
      const int v = 4 * wave + vv;
      float z = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) z += fw[vv][w] * sred[((w * NT + t) * 16 + v) * 64 + lane];
      const int row = d32_row(v, q);
      const size_t zi = ((size_t)sg * g.M_pad + row) * g.rv_ld + vc;
      if (LAT == STARKV_LATENT_MIX84) {
        if (cok && row < g.M_q) ((uint16_t*)a.zp)[zi] = f32_to_f16(z * a.zsc);
      } else if (cok && row < g.M_q) {
        ((float*)a.zp)[zi] = z;
      }
    }
  }
  if (slice == 0 && wave == 0 && q == 0 && rok) {
    const float ms = fmaxf(fmaxf(smx[0][r], smx[1][r]), fmaxf(smx[2][r], smx[3][r]));
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) l += rel_weight(smx[w][r], ms) * ssum[w][r];
    a.sl[(size_t)sg * g.M_pad + r] = l;
    a.sm[(size_t)sg * g.M_pad + r] = ms;
  }
}

// Grid: one dimension of n_sl x P workgroups, P grid positions (n_splits rounded up to 8, or
// a.vo.n).  Workgroups are handed to the eight XCDs in turn (id mod 8), so the k-th workgroup of
// XCD x takes slice k mod n_sl of the split at position 8 (k / n_sl) + x (the split itself, or
// a.vo.sg of it): all slices of a split run on one XCD and share its L2 copy of the split's
// probabilities.
template <int LAT, int NBW8, int NBW4>
__global__ __launch_bounds__(256) void k_values1(ValueArgs a) {
  // room for four accumulator tiles per wave whatever the instance needs: at 64 KiB of LDS at
  // most two workgroups share a CU, so the 2-per-CU grids spread evenly over the CUs
  __shared__ float sred[4 * 4 * 16 * 64];
  __shared__ float ssum[4][32];
  __shared__ float smx[4][32];
  const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
  const int slice = k % a.n_sl;
  const int pos = 8 * (k / a.n_sl) + xcd;
  if (pos >= (a.vo.n ? a.vo.n : a.n_splits)) return;
  const int sg = a.vo.n ? a.vo.sg[pos] : pos;
  if (sg == 0xFFFF) return;
  if (LAT == STARKV_LATENT_MIX84 && slice >= a.n_sl8 + a.n_sl4) {
    // packed layout: two 3-bit N-tiles per slice
    const int nt0 = (slice - a.n_sl8 - a.n_sl4) * 2;
    values1_run<LAT, 2, 2>(a, slice, sg, nt0, min(2, a.n3t - nt0), sred, ssum, smx);
  } else if (LAT == STARKV_LATENT_MIX84 && slice >= a.n_sl8) {
    const int nb0 = a.V8 / 32 + (slice - a.n_sl8) * NBW4;
    values1_run<LAT, NBW4, 1>(a, slice, sg, nb0, min(NBW4, a.NB4 - nb0), sred, ssum, smx);
  } else {
    const int nb0 = slice * NBW8;
    const int nbe = LAT == STARKV_LATENT_MIX84 ? a.V8 / 32 : a.NB;
    values1_run<LAT, NBW8, 0>(a, slice, sg, nb0, min(NBW8, nbe - nb0), sred, ssum, smx);
  }
}


// Many query rows per sequence (M_pad = 32 NMT > 32; bf16 or int8/int4 latents): workgroup =
// (split of one sequence, group of 4 NTW value N-tiles of 32 channels); wave w owns N-tiles
// NTW w .. NTW w + NTW - 1 of the group -- each a bf16 or int8 block of 32 channels, or the even
// or odd channels of an int4 block -- for all NMT row tiles, so the probability tile of a chunk is
// fetched once per 4 NTW N-tiles.  Each 32-token chunk's probability tile [M_pad][32] (as the
// key-score kernel stored it, relative to its chunk maximum), chunk maxima and sums, and the
// workgroup's value blocks are copied into a ring of D LDS stages by asynchronous LDS loads, D - 1
// chunks ahead, with no register cost.  Each wave scales its probability A-fragments by
// 2^(m_chunk - M_row) as it reads them (M_row: the row's largest chunk maximum over the split,
// read before the loop; fp16 fragments take one packed half multiply per pair), so one barrier
// per chunk suffices.  The probability rows of a stage are stored with their four 16-byte pieces
// rotated by (row / 4) mod 4, which makes the A-fragment reads of 16 consecutive rows hit distinct
// LDS banks.  Grid as k_values1 (one dimension; the groups of a split run on one XCD).
template <int LAT, int NMT, int NTW, int D>
__device__ __forceinline__ void values_mt_body(const ValueArgs& a) {
  static_assert(LAT != STARKV_LATENT_F32, "fp32 latents use k_values");
  constexpr int MP = 32 * NMT;
  constexpr int esz = LAT == STARKV_LATENT_BF16 ? 2 : 1;
  constexpr int NV = esz;                       // 16-byte B-fragment pieces per lane per chunk
  constexpr int BLKB = 32 * kTT * esz;          // bytes of one value block (32 rows x 32 tokens)
  constexpr int NPI = MP / 16;                  // 1 KiB probability loads per stage
  constexpr int NSI = NPI + 2;                  // + chunk maxima and sums
  constexpr int SPW = (NSI + 3) / 4;            // of those per wave (uniform count)
  constexpr int VPW = NTW * (BLKB / 1024);      // 1 KiB value loads per wave per stage
  constexpr int LPW = SPW + VPW;                // loads per wave per stage
  constexpr int P_OFF = 0, CM_OFF = MP * 64, CL_OFF = CM_OFF + 1024, V_OFF = CL_OFF + 1024;
  constexpr int STAGE = V_OFF + 4 * NTW * BLKB;
  static_assert(LPW * (D - 2) < 64, "vmcnt range");
  __shared__ __align__(16) uint8_t ring[D * STAGE];
  __shared__ float msplit[MP];
  const DecodeGeom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r = lane & 31, q = lane >> 5;
  const int xcd = blockIdx.x & 7, kk = blockIdx.x >> 3;
  const int grp = kk % a.n_sl;
  const int idx = 8 * (kk / a.n_sl) + xcd;
  if (idx >= (a.vo.n ? a.vo.n : a.n_splits)) return;
  if (a.vo.n && a.vo.sg[idx] == 0xFFFF) return;
  int b;
  const int sg = a.vo.n ? a.vo.sg[idx] : value_split(a.seq, g.B, idx, b);
  if (a.vo.n) b = seq_of_split(a.seq, g.B, sg);
  const int s = sg - seq_split0(a.seq, b);
  const int cbase = seq_chunk0(a.seq, b);
  const int nch = seq_nch_live(a.seq, b);
  const int c_lo = s * a.cps, c_hi = min(c_lo + a.cps, nch);
  if (c_lo >= nch) return;  // a split past a device length (whole workgroup): the merges skip it
  const int len = seq_len(a.seq, b);
  const uint32_t ring0 = lds_addr(ring);

  // this wave's N-tiles
  const int n_nt8 = LAT == STARKV_LATENT_MIX84 ? a.V8 / 32 : a.NB;
  const int n_nt = n_nt8 + (LAT == STARKV_LATENT_MIX84 ? 2 * (a.NB - a.V8 / 32) : 0);
  bool ntok[NTW], is4[NTW];
  int blk[NTW], par[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int nt = (grp * 4 + wave) * NTW + j;
    ntok[j] = nt < n_nt;  // wave-uniform
    blk[j] = 0;
    par[j] = 0;
    is4[j] = false;
    if (ntok[j]) {
      if (nt < n_nt8) {
        blk[j] = nt;
      } else {
        blk[j] = a.V8 / 32 + (nt - n_nt8) / 2;
        par[j] = (nt - n_nt8) & 1;
        is4[j] = true;
      }
    }
  }

  // Sources of this wave's asynchronous loads at the split's first chunk (a wave-uniform base and
  // a per-lane offset) and their strides per chunk.  Probability rows 16 i .. 16 i + 15: lane l
  // takes row 16 i + l / 4, rotated piece l % 4; i == NPI: the chunk maxima; past that, the sums
  // (indexes past NSI repeat them).  Value blocks: consecutive tiles of a row block are BLKB apart.
  const uint8_t* ubase[SPW];
  uint32_t uoff[SPW], ustr[SPW], udst[SPW];
  const size_t cg0 = (size_t)(cbase + c_lo);
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int i = wave * SPW + u;  // wave-uniform
    if (i < NPI) {
      const int row = 16 * i + (lane >> 2);
      const int piece = ((lane & 3) - (row >> 2)) & 3;
      ubase[u] = (const uint8_t*)a.p + cg0 * g.M_pad * (kTC * 2);
      uoff[u] = (uint32_t)(row * (kTC * 2) + 16 * piece);
      ustr[u] = (uint32_t)g.M_pad * (kTC * 2);
      udst[u] = P_OFF + i * 1024;
    } else {
      ubase[u] = (const uint8_t*)(i == NPI ? a.cm : a.cl) + cg0 * g.M_pad * 4;
      uoff[u] = (uint32_t)min(4 * lane, g.M_pad - 4) * 4;
      ustr[u] = (uint32_t)g.M_pad * 4;
      udst[u] = i == NPI ? CM_OFF : CL_OFF;
    }
  }
  const uint8_t* vbase[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) vbase[j] = a.v_tiles + vblock_off(b, blk[j], c_lo, g.v_rows, g.T_max, esz);
  // asynchronous loads of chunk c (clamped into the split) into stage st
  auto issue = [&](int c, int st) {
    const uint32_t dc = (uint32_t)(min(c, c_hi - 1) - c_lo);
    const uint32_t sb = ring0 + st * STAGE;
#pragma unroll
    for (int u = 0; u < SPW; ++u) lds_dma16(ubase[u] + dc * ustr[u] + uoff[u], sb + udst[u]);
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int x = 0; x < BLKB / 1024; ++x)
        lds_dma16(vbase[j] + dc * BLKB + 1024 * x + 16 * lane, sb + V_OFF + (wave * NTW + j) * BLKB + 1024 * x);
  };

  // the first D - 1 chunks go out, then each row's largest chunk maximum over the split
#pragma unroll
  for (int u = 0; u < D - 1; ++u) issue(c_lo + u, u);
  if (tid < MP) {
    const size_t row = (size_t)min(tid, g.M_q - 1);
    msplit[tid] = chunks_max<16>(a.cm, cbase + c_lo, 1, c_hi - c_lo, g.M_pad, row);
  }
  __syncthreads();
  float Ms[NMT], lsum[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    Ms[mt] = msplit[mt * 32 + r];
    lsum[mt] = 0.f;
  }

  f32x16 acc[NTW][NMT];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][mt][v] = 0.f;

  int st = 0, st_next = D - 1;  // stages of chunk c and of chunk c + D - 1
  for (int c = c_lo; c < c_hi; ++c) {
    vm_wait<LPW * (D - 2)>();  // this wave's loads of chunk c are in
    __builtin_amdgcn_s_barrier();  // ... and every wave's; chunk c - 1's stage is free
    asm volatile("" ::: "memory");
    issue(c + D - 1, st_next);
    st_next = st;
    const uint8_t* sp = ring + st * STAGE;
    st = st + 1 == D ? 0 : st + 1;
    // chunk weights of this lane's A-fragment rows (all reads first, no branch between them)
    float cmv[NMT], clv[NMT], alpha[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      cmv[mt] = ((const float*)(sp + CM_OFF))[mt * 32 + r];
      clv[mt] = ((const float*)(sp + CL_OFF))[mt * 32 + r];
    }
    const float lw = (wave == 0 && q == 0) ? 1.f : 0.f;  // one lane per row keeps the sum
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int row = mt * 32 + r;
      alpha[mt] = (row >= g.M_q || cmv[mt] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(cmv[mt] - Ms[mt]);
      lsum[mt] += lw * alpha[mt] * clv[mt];
    }
    // B fragments: 8 tokens of one channel (or channel pair) per K-step
    _Float16 alpha_h[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) alpha_h[mt] = (_Float16)alpha[mt];
    u32x4 vf[NTW][NV];
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int x = 0; x < NV; ++x)
        vf[j][x] = *(const u32x4*)(sp + V_OFF + (wave * NTW + j) * BLKB + r * kTT * esz + 16 * NV * q + 16 * x);
    if (LAT == STARKV_LATENT_BF16 && c * kTC + kTT > len) {
      // zero the elements of tokens at or past the length (their bits may be anything)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t = c * kTC + 16 * q + e;
          if (t >= len) {
            const uint32_t keep = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
            vf[j][e >> 3][(e >> 1) & 3] &= keep;
          }
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 af[NMT];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int row = mt * 32 + r;
        const int piece = ((2 * q + h) + (row >> 2)) & 3;
        const u32x4 raw = *(const u32x4*)(sp + P_OFF + row * 64 + 16 * piece);
        if (LAT == STARKV_LATENT_BF16) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = bf16_to_f32((uint16_t)(raw[e] & 0xFFFF)) * alpha[mt];
            const float x1 = bf16_to_f32((uint16_t)(raw[e] >> 16)) * alpha[mt];
            w[e] = (uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16);
          }
          af[mt] = w;
        } else {
          // fp16 probabilities: packed half multiplies by the weight rounded to half
          const f16x8 pv = as_f16x8(raw) * alpha_h[mt];
          af[mt] = __builtin_bit_cast(u32x4, pv);
        }
      }
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        u32x4 bfrag;
        if (LAT == STARKV_LATENT_BF16) {
          bfrag = vf[j][h % NV];
        } else {
          f16x8 ev;
          if (is4[j]) ev = deq_i4x8_half(vf[j][0][2 * h], vf[j][0][2 * h + 1], par[j]);
          else ev = deq_i8x8(vf[j][0][2 * h], vf[j][0][2 * h + 1]);
          bfrag = __builtin_bit_cast(u32x4, ev);
        }
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          if (LAT == STARKV_LATENT_BF16) acc[j][mt] = mfma32_bf16(as_bf16x8(af[mt]), as_bf16x8(bfrag), acc[j][mt]);
          else acc[j][mt] = mfma32_f16(as_f16x8(af[mt]), as_f16x8(bfrag), acc[j][mt]);
        }
      }
    }
  }
  vm_wait<0>();  // no asynchronous load may still be writing LDS when the workgroup ends

  // z partials: lane holds channel r of each N-tile, rows d32_row(v, q) of each row tile
  int vc[NTW];
  bool cok[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    if (!is4[j]) {
      vc[j] = blk[j] * 32 + r;
      cok[j] = ntok[j] && vc[j] < (LAT == STARKV_LATENT_MIX84 ? a.n8v : g.r_v);
    } else {
      const int w = 2 * ((blk[j] - a.V8 / 32) * 32 + r) + par[j];
      cok[j] = ntok[j] && w < a.n4v;
      vc[j] = a.n8v + w;
    }
  }
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = mt * 32 + d32_row(v, q);
      if (row >= g.M_q) continue;
      const size_t z0 = ((size_t)sg * g.M_pad + row) * g.rv_ld;
      if (LAT == STARKV_LATENT_MIX84) {
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          if (cok[j]) ((uint16_t*)a.zp)[z0 + vc[j]] = f32_to_f16(acc[j][mt][v] * a.zsc);
      } else {
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          if (cok[j]) ((float*)a.zp)[z0 + vc[j]] = acc[j][mt][v];
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // one row tile's conversions at a time (registers)
  }
  if (grp == 0 && wave == 0 && q == 0) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int row = mt * 32 + r;
      if (row < g.M_q) {
        a.sl[(size_t)sg * g.M_pad + row] = lsum[mt];
        a.sm[(size_t)sg * g.M_pad + row] = Ms[mt];
      }
    }
  }
}

// int8/int4 latents: two workgroups per CU (two waves per SIMD), with the accumulators in the
// unified register file; bf16 latents: their larger LDS stages allow one workgroup per CU.
template <int LAT, int NMT, int NTW, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_values_mt_w2(ValueArgs a) {
  values_mt_body<LAT, NMT, NTW, D>(a);
}
template <int LAT, int NMT, int NTW, int D>
__global__ __launch_bounds__(256) void k_values_mt_w1(ValueArgs a) {
  values_mt_body<LAT, NMT, NTW, D>(a);
}
template <int LAT, int NMT, int NTW, int D>
constexpr auto values_mt_kernel() {
  if constexpr (LAT == STARKV_LATENT_MIX84) return &k_values_mt_w2<LAT, NMT, NTW, D>;
  else return &k_values_mt_w1<LAT, NMT, NTW, D>;
}
template <int LAT, int NMT, int NTW, int D>
constexpr void (*k_values_mt)(ValueArgs) = values_mt_kernel<LAT, NMT, NTW, D>();

// ===========================================================================
// merge + up-projection: out = (sum_s z_s) * scale_v B_v^g / (sum_s l_s)

struct MergeArgs {
  const void* zp;  // split partials (fp32, or f16 scaled by zsc: int8/int4 latents)
  float zinv;      // int8/int4 latents: 1 / zsc
  const float* sl;
  const float* sm;
  float* zt;                // [B][M_pad][rv_ld] merged, scaled, normalised value latent
  const void* B_vt;         // [H_kv * d_h][r_v]
  const uint16_t* vscales;  // [r_v] f16 (mix84) or null
  void* out;
  DecodeGeom g;
  SeqTable seq;
  int nsp;  // split merge: lanes sharing 4 channels (1, or 4 for many splits)
  int cps;  // chunks per split
};

// Split merge.  Split s weighted its tiles against its own maximum m_s of the row, so with M the
// largest m_s: z~[c] = (sum_s 2^(m_s - M) z_s[c]) * scale_c / (sum_s 2^(m_s - M) l_s), and zero in
// the padding channels [r_v, rv_ld).  MIX (int8/int4 latents): the partials are f16, scaled by
// a power of two (zsc) that keeps them in range; zinv undoes it.  Workgroup = 4 rows x (256 / nsp) channels of one sequence;
// nsp adjacent lanes (1 or 4) share 4 channels and take every nsp-th split each, all their loads
// issued at once (NB splits per batch), keep a running maximum (rescaling their sums when it
// grows), and combine by lane exchange in a fixed order, so the result is deterministic.
template <bool MIX, int NB>
__global__ __launch_bounds__(256) void k_zmerge(MergeArgs a) {
  const DecodeGeom& g = a.g;
  const int nsp = a.nsp;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int sp = tid & (nsp - 1);
  const int i = blockIdx.y * 4 + (tid >> 6);
  const int c = blockIdx.x * (256 / nsp) + ((tid & 63) / nsp) * 4;
  const bool live = i < g.M_q && c < g.rv_ld;
  const int ic = min(i, g.M_q - 1), cc = min(c, g.rv_ld - 4);
  const int s0 = seq_split0(a.seq, b);
  const int ns = min(seq_nsplit(a.seq, b), (seq_nch_live(a.seq, b) + a.cps - 1) / a.cps);  // live splits
  const size_t zo = ((size_t)s0 * g.M_pad + ic) * g.rv_ld + cc;
  const float* zc = (const float*)a.zp + zo;
  const uint16_t* zh = (const uint16_t*)a.zp + zo;
  const float* lc = a.sl + (size_t)s0 * g.M_pad + ic;
  const float* mc = a.sm + (size_t)s0 * g.M_pad + ic;
  const size_t zs = (size_t)g.M_pad * g.rv_ld;
  // int8/int4 value scales of this lane's 4 channels, issued with the first partials
  uint16_t scv[4] = {0, 0, 0, 0};
  if (MIX) {
#pragma unroll
    for (int e = 0; e < 4; ++e) scv[e] = a.vscales[min(cc + e, g.r_v - 1)];
  }
  float z[4] = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  float M = -INFINITY;  // reference of z and l: the largest split maximum seen so far
  for (int s = sp; s < ns; s += NB * nsp) {
    u32x4 v[NB];
    float lv[NB], mv[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int ss = min(s + u * nsp, ns - 1);
      if (MIX) {
        const u32x2 h = ld8(zh + (size_t)ss * zs);
        v[u] = u32x4{h[0], h[1], 0, 0};
      } else {
        v[u] = ld16(zc + (size_t)ss * zs);
      }
      lv[u] = lc[(size_t)ss * g.M_pad];
      mv[u] = mc[(size_t)ss * g.M_pad];
    }
    __builtin_amdgcn_sched_barrier(0);  // all 3 NB loads go out before the first add
    float Mn = M;
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (s + u * nsp < ns) Mn = fmaxf(Mn, mv[u]);
    const float f0 = rel_weight(M, Mn);
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] *= f0;
    l *= f0;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (s + u * nsp < ns) {
        const float w = rel_weight(mv[u], Mn);
        if (MIX) {
          const float wz = w * a.zinv;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            z[e] += wz * f16_to_f32((uint16_t)(e & 1 ? v[u][e >> 1] >> 16 : v[u][e >> 1] & 0xFFFF));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] += w * __uint_as_float(v[u][e]);
        }
        l += w * lv[u];
      }
    }
    M = Mn;
  }
  for (int m = 1; m < nsp; m <<= 1) {
    const float Mo = __shfl_xor(M, m, 64);
    const float Mn = fmaxf(M, Mo);
    const float fs = rel_weight(M, Mn), fo = rel_weight(Mo, Mn);
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = fs * z[e] + fo * __shfl_xor(z[e], m, 64);
    l = fs * l + fo * __shfl_xor(l, m, 64);
    M = Mn;
  }
  if (!live || sp != 0) return;
  const float il = 1.f / l;
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int ce = c + e;
    float sc = il;
    if (MIX) sc *= f16_to_f32(scv[e]);
    o[e] = __float_as_uint(ce < g.r_v ? z[e] * sc : 0.f);
  }
  st16(a.zt + ((size_t)b * g.M_pad + i) * g.rv_ld + c, o);
}

// Up-projection for many rows per KV head (bf16, r_v % 8 == 0): workgroup = (g, 32-row tile of
// g's rows over all sequences), all d_h columns, four 32-column slices at a time.  Wave w takes a
// quarter of K = rv_ld (16-channel steps) for every column, so each element of z~ and of g's
// B_v^T slab is read and split into hi + lo bf16 parts once per workgroup; the four partial tiles
// are added through LDS, wave w finishing column slice w (32x32x16 bf16 MFMA).  Loads are
// unconditional and double-buffered: rows past the end read the last row (not stored); channels at
// or past r_v are zero in z~ and masked in B_v (their address clamped into the row).
template <int RT>
__global__ __launch_bounds__(256, 3 - RT) void k_upproj_tall(MergeArgs a) {
  constexpr int KB = 1;   // 16-channel K-steps per load batch
  constexpr int NCS = 4;  // 32-column slices per pass
  __shared__ float part[4][NCS][16][64];  // [wave][column slice][D element][lane]
  const DecodeGeom& g = a.g;
  const int gk = blockIdx.x;
  const int rph = g.G * g.n_q;
  const int Rg = g.B * rph;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int r = lane & 31, q = lane >> 5;
  const int row0 = blockIdx.y * 32 * RT;  // first row of this workgroup's RT row tiles
  const float* zr[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int rr = min(row0 + 32 * i + r, Rg - 1);
    zr[i] = a.zt + ((size_t)(rr / rph) * g.M_pad + gk * rph + rr % rph) * g.rv_ld + 8 * q;
  }
  const int nks = g.rv_ld / 16;
  const int kq = (nks + 3) / 4;
  const int k_beg = min(nks, wave * kq), k_end = min(nks, k_beg + kq);
  const int ncs = g.d_h / 32;
  for (int cs0 = 0; cs0 < ncs; cs0 += NCS) {
    const uint16_t* bp[NCS];
#pragma unroll
    for (int c = 0; c < NCS; ++c)
      bp[c] = (const uint16_t*)a.B_vt + (size_t)(gk * g.d_h + min(cs0 + c, ncs - 1) * 32 + r) * g.r_v;
    f32x16 acc[RT][NCS];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int c = 0; c < NCS; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][c][v] = 0.f;
    auto loadb = [&](u32x4 (&z)[KB][RT][2], u32x4 (&bw)[KB][NCS], int ks0) {
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int kc = 16 * min(ks0 + u, nks - 1);
#pragma unroll
        for (int i = 0; i < RT; ++i) {
          z[u][i][0] = ld16(zr[i] + kc);
          z[u][i][1] = ld16(zr[i] + kc + 4);
        }
#pragma unroll
        for (int c = 0; c < NCS; ++c) bw[u][c] = ld16(bp[c] + min(kc + 8 * q, g.r_v - 8));
      }
    };
    auto compb = [&](u32x4 (&z)[KB][RT][2], u32x4 (&bw)[KB][NCS], int ks0) {
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int kc = 16 * (ks0 + u);
        const bool live = ks0 + u < k_end && kc + 8 * q < g.r_v;
#pragma unroll
        for (int i = 0; i < RT; ++i) {
          u32x4 ah, al;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float z0 = __uint_as_float(z[u][i][e2 >> 1][2 * (e2 & 1)]);
            const float z1 = __uint_as_float(z[u][i][e2 >> 1][2 * (e2 & 1) + 1]);
            const uint16_t h0 = f32_to_bf16(z0), h1 = f32_to_bf16(z1);
            const uint16_t l0 = f32_to_bf16(z0 - bf16_to_f32(h0)), l1 = f32_to_bf16(z1 - bf16_to_f32(h1));
            ah[e2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            al[e2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
          }
#pragma unroll
          for (int c = 0; c < NCS; ++c) {
            const u32x4 bb = live ? bw[u][c] : u32x4{0, 0, 0, 0};
            acc[i][c] = mfma32_bf16(as_bf16x8(ah), as_bf16x8(bb), acc[i][c]);
            acc[i][c] = mfma32_bf16(as_bf16x8(al), as_bf16x8(bb), acc[i][c]);
          }
        }
      }
    };
    // three register sets take turns, two batches ahead of their use: every load is issued
    // unconditionally (clamped, masked in compb), so each wait covers only the set about to be
    // used (one batch in flight measured 38.5 us on C4, latency-bound)
    u32x4 zA[KB][RT][2], bA[KB][NCS], zB[KB][RT][2], bB[KB][NCS], zC[KB][RT][2], bC[KB][NCS];
    loadb(zA, bA, k_beg);
    loadb(zB, bB, k_beg + KB);
    loadb(zC, bC, k_beg + 2 * KB);
    int ks = k_beg;
    for (; ks + 3 * KB <= k_end; ks += 3 * KB) {
      compb(zA, bA, ks);
      loadb(zA, bA, ks + 3 * KB);
      compb(zB, bB, ks + KB);
      loadb(zB, bB, ks + 4 * KB);
      compb(zC, bC, ks + 2 * KB);
      loadb(zC, bC, ks + 5 * KB);
    }
    if (ks < k_end) compb(zA, bA, ks);
    if (ks + KB < k_end) compb(zB, bB, ks + KB);
    vm_wait<0>();  // the clamped loads past the end are not used
    // the four K-quarters of every column slice, added by the wave that finishes that slice;
    // one row tile at a time through the shared partial tiles
#pragma unroll
    for (int i = 0; i < RT; ++i) {
#pragma unroll
      for (int c = 0; c < NCS; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) part[wave][c][v][lane] = acc[i][c][v];
      __syncthreads();
      const int cs = cs0 + wave;
      if (cs < ncs) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float o = part[0][wave][v][lane] + part[1][wave][v][lane] + part[2][wave][v][lane] +
                          part[3][wave][v][lane];
          const int orow = row0 + 32 * i + d32_row(v, q);
          if (orow >= Rg) continue;
          const int ob = orow / rph, iw = orow % rph;
          const int hh = iw / g.n_q, j = iw % g.n_q;
          const int h = gk * g.G + hh;
          ((uint16_t*)a.out)[(((size_t)ob * g.n_q + j) * g.H_q + h) * g.d_h + cs * 32 + r] = f32_to_bf16(o);
        }
      }
      __syncthreads();  // the partial tiles are reused by the next row tile or pass
    }
  }
}

// Up-projection out_i = z~_i B_v^g for the rows of KV head g.  Workgroup = (g, 16-column slice of
// d_h, 16-row tile of g's rows over all sequences); the four waves split K = rv_ld in 32-channel
// chunks and add their partial outputs through LDS.  Every load is unconditional: rows past the
// tile's end read its last row (their outputs are not stored), chunks past a wave's range repeat
// its last chunk (not used), and channels at or past r_v are zero in z~ and masked in B_v.
// bf16: z~ split into hi + lo bf16 parts (two MFMAs).  VEC: r_v % 8 == 0, so 8 channels of a
// B_v^T row are one 16-byte load; otherwise they are loaded one by one.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void k_upproj(MergeArgs a) {
  const DecodeGeom& g = a.g;
  const int nsl_n = g.d_h / 16;
  const int gk = blockIdx.x / nsl_n, nsl = blockIdx.x % nsl_n;
  const int rph = g.G * g.n_q;
  const int Rg = g.B * rph;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n = lane & 15, qq = lane >> 4;
  __shared__ float red[3][4][64];
  const int rr = min((int)blockIdx.y * 16 + n, Rg - 1);  // A-fragment row of this lane
  const int bb = rr / rph;
  const int ii = gk * rph + rr % rph;
  const float* zr = a.zt + ((size_t)bb * g.M_pad + ii) * g.rv_ld + 8 * qq;
  const int col = gk * g.d_h + nsl * 16 + n;  // B_v^T row of this lane's output column
  const int nchk = g.rv_ld / 32;
  const int per = (nchk + 3) / 4;
  const int k_beg = wave * per, k_end = min(nchk, k_beg + per);
  f32x4 acc = {0, 0, 0, 0};
  constexpr int KU = 8;  // 32-channel chunks in flight
  for (int kc0 = k_beg; kc0 < k_end; kc0 += KU) {
    u32x4 z[KU][2];
    u32x4 bw[KU][DT == STARKV_F32 ? 2 : 1];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const bool live = kc0 + u < k_end;  // a repeated chunk contributes zero (B masked)
      const int c = 32 * min(kc0 + u, k_end - 1) + 8 * qq;  // first channel of this lane's 8
      z[u][0] = ld16(zr + 32 * min(kc0 + u, k_end - 1));
      z[u][1] = ld16(zr + 32 * min(kc0 + u, k_end - 1) + 4);
      if (DT == STARKV_F32) {
        const float* bp = (const float*)a.B_vt + (size_t)col * g.r_v;
        if (VEC) {
          const bool ok = live && c < g.r_v;
          const int cc = ok ? c : 0;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const u32x4 v = ld16(bp + cc + 4 * h);
            bw[u][h % 2] = ok ? v : u32x4{0, 0, 0, 0};
          }
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int ce = c + 4 * h + e;
              const float x = bp[min(ce, g.r_v - 1)];
              bw[u][h % 2][e] = (live && ce < g.r_v) ? __float_as_uint(x) : 0u;
            }
        }
      } else {
        const uint16_t* bp = (const uint16_t*)a.B_vt + (size_t)col * g.r_v;
        if (VEC) {
          const bool ok = live && c < g.r_v;
          const u32x4 v = ld16(bp + (ok ? c : 0));
          bw[u][0] = ok ? v : u32x4{0, 0, 0, 0};
        } else {
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const int ce = c + 2 * e2;
            const uint32_t b0 = bp[min(ce, g.r_v - 1)], b1 = bp[min(ce + 1, g.r_v - 1)];
            bw[u][0][e2] = (live && ce < g.r_v ? b0 : 0u) | ((live && ce + 1 < g.r_v ? b1 : 0u) << 16);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load of the batch ahead of the MFMAs
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      if (DT == STARKV_F32) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc = mfma16_f32(__uint_as_float(z[u][h][e]), __uint_as_float(bw[u][h % 2][e]), acc);
      } else {
        u32x4 ah, al;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float z0 = __uint_as_float(z[u][e2 >> 1][2 * (e2 & 1)]);
          const float z1 = __uint_as_float(z[u][e2 >> 1][2 * (e2 & 1) + 1]);
          const uint16_t h0 = f32_to_bf16(z0), h1 = f32_to_bf16(z1);
          const uint16_t l0 = f32_to_bf16(z0 - bf16_to_f32(h0));
          const uint16_t l1 = f32_to_bf16(z1 - bf16_to_f32(h1));
          ah[e2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          al[e2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        acc = mfma16_bf16(as_bf16x8(ah), as_bf16x8(bw[u][0]), acc);
        acc = mfma16_bf16(as_bf16x8(al), as_bf16x8(bw[u][0]), acc);
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave - 1][v][lane] = acc[v];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float o = acc[v] + red[0][v][lane] + red[1][v][lane] + red[2][v][lane];
    const int orow = blockIdx.y * 16 + 4 * qq + v;  // D row = row within the tile; D column = n
    if (orow >= Rg) continue;
    const int ob = orow / rph, iw = orow % rph;
    const int hh = iw / g.n_q, j = iw % g.n_q;
    const int h = gk * g.G + hh;
    const size_t off = (((size_t)ob * g.n_q + j) * g.H_q + h) * g.d_h + nsl * 16 + n;
    if (DT == STARKV_F32) ((float*)a.out)[off] = o;
    else ((uint16_t*)a.out)[off] = f32_to_bf16(o);
  }
}

// Split merge folded into the up-projection (sequences of at most 4 splits): workgroup = (g,
// 16-column slice of d_h, 16-row tile of g's rows over all sequences); its eight waves split K =
// rv_ld in 32-channel chunks.  A lane sums its row's split partials for its 8 channels (in split
// order, weighted 2^(m_s - M) as in k_zmerge; MIX: f16 partials, times zinv), scales them by
// scale_c / sum_s 2^(m_s - M) l_s,
// and feeds the MFMA as k_upproj does.  Padding channels (>= r_v) are zeroed; loads unconditional.
template <int DT, bool MIX>
__global__ __launch_bounds__(512) void k_upproj_merge(MergeArgs a) {
  constexpr int NSM = 4;  // splits per sequence, at most
  constexpr int KU = 4;   // 32-channel chunks per wave
  const DecodeGeom& g = a.g;
  const int nsl_n = g.d_h / 16;
  // workgroups go to the eight XCDs in turn (id mod 8): every column slice of KV head gk runs on
  // XCD gk mod 8, so the head's split partials are fetched into one L2 only
  const int k = blockIdx.x >> 3;
  const int nsl = k % nsl_n;
  const int gk = 8 * (k / nsl_n) + (blockIdx.x & 7);
  if (gk >= g.H_kv) return;
  const int rph = g.G * g.n_q;
  const int Rg = g.B * rph;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n = lane & 15, qq = lane >> 4;
  __shared__ float red[7][4][64];
  const int rr = min((int)blockIdx.y * 16 + n, Rg - 1);  // A-fragment row of this lane
  const int bb = rr / rph;
  const int ii = gk * rph + rr % rph;
  const int s0 = seq_split0(a.seq, bb);
  const int ns = min(seq_nsplit(a.seq, bb), (seq_nch_live(a.seq, bb) + a.cps - 1) / a.cps);  // live splits
  size_t zs[NSM];  // element offsets of this lane's partial rows
  float lv[NSM], mv[NSM];
#pragma unroll
  for (int sx = 0; sx < NSM; ++sx) {
    const size_t sp = (size_t)(s0 + min(sx, ns - 1));
    zs[sx] = (sp * g.M_pad + ii) * g.rv_ld + 8 * qq;
    lv[sx] = a.sl[sp * g.M_pad + ii];
    mv[sx] = a.sm[sp * g.M_pad + ii];
  }
  // split weights 2^(m_s - M) (zero for the padding splits past ns)
  float M = -INFINITY;
#pragma unroll
  for (int sx = 0; sx < NSM; ++sx)
    if (sx < ns) M = fmaxf(M, mv[sx]);
  float wsx[NSM];
  float l = 0.f;
#pragma unroll
  for (int sx = 0; sx < NSM; ++sx) {
    wsx[sx] = sx < ns ? rel_weight(mv[sx], M) : 0.f;
    l += wsx[sx] * lv[sx];
    if (MIX) wsx[sx] *= a.zinv;  // the f16 partials are scaled by zsc
  }
  const float il = 1.f / l;
  const int col = gk * g.d_h + nsl * 16 + n;  // B_v^T row of this lane's output column
  const int nchk = g.rv_ld / 32;
  const int k_beg = wave * KU;  // chunks [k_beg, k_beg + KU) of this wave (nchk <= 8 KU)
  u32x4 z[KU][NSM][2];
  u32x4 bw[KU][DT == STARKV_F32 ? 2 : 1];
  u32x4 sc[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int kc = min(k_beg + u, nchk - 1);
    const int c = 32 * kc + 8 * qq;  // first channel of this lane's 8
#pragma unroll
    for (int sx = 0; sx < NSM; ++sx) {
      if (MIX) {
        z[u][sx][0] = ld16((const uint16_t*)a.zp + zs[sx] + 32 * kc);  // 8 halves
      } else {
        z[u][sx][0] = ld16((const float*)a.zp + zs[sx] + 32 * kc);
        z[u][sx][1] = ld16((const float*)a.zp + zs[sx] + 32 * kc + 4);
      }
    }
    const int cc = c < g.r_v ? c : 0;
    if (DT == STARKV_F32) {
      const float* bp = (const float*)a.B_vt + (size_t)col * g.r_v;
      bw[u][0] = ld16(bp + cc);
      bw[u][DT == STARKV_F32 ? 1 : 0] = ld16(bp + cc + 4);
    } else {
      bw[u][0] = ld16((const uint16_t*)a.B_vt + (size_t)col * g.r_v + cc);
    }
    sc[u] = MIX ? ld16(a.vscales + cc) : u32x4{0, 0, 0, 0};
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the arithmetic
  f32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int c = 32 * (k_beg + u) + 8 * qq;
    const bool live = k_beg + u < nchk;
    float zz[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = 0.f;
#pragma unroll
      for (int sx = 0; sx < NSM; ++sx) {
        const uint32_t hw = z[u][sx][0][e >> 1];
        t += wsx[sx] * (MIX ? f16_to_f32((uint16_t)(e & 1 ? hw >> 16 : hw & 0xFFFF))
                            : __uint_as_float(z[u][sx][e >> 2][e & 3]));
      }
      float scl = il;
      if (MIX) scl *= f16_to_f32((uint16_t)(e & 1 ? sc[u][e >> 1] >> 16 : sc[u][e >> 1] & 0xFFFF));
      zz[e] = (live && c + e < g.r_v) ? t * scl : 0.f;
    }
    if (DT == STARKV_F32) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float bv = (live && c + 4 * h + e < g.r_v) ? __uint_as_float(bw[u][h % 2][e]) : 0.f;
          acc = mfma16_f32(zz[4 * h + e], bv, acc);
        }
    } else {
      u32x4 ah, al;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint16_t h0 = f32_to_bf16(zz[2 * e2]), h1 = f32_to_bf16(zz[2 * e2 + 1]);
        const uint16_t l0 = f32_to_bf16(zz[2 * e2] - bf16_to_f32(h0));
        const uint16_t l1 = f32_to_bf16(zz[2 * e2 + 1] - bf16_to_f32(h1));
        ah[e2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        al[e2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
      const u32x4 bv = (live && c < g.r_v) ? bw[u][0] : u32x4{0, 0, 0, 0};
      acc = mfma16_bf16(as_bf16x8(ah), as_bf16x8(bv), acc);
      acc = mfma16_bf16(as_bf16x8(al), as_bf16x8(bv), acc);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave - 1][v][lane] = acc[v];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float o = acc[v];
#pragma unroll
    for (int w = 0; w < 7; ++w) o += red[w][v][lane];
    const int orow = blockIdx.y * 16 + 4 * qq + v;  // D row = row within the tile; D column = n
    if (orow >= Rg) continue;
    const int ob = orow / rph, iw = orow % rph;
    const int hh = iw / g.n_q, j = iw % g.n_q;
    const int h = gk * g.G + hh;
    const size_t off = (((size_t)ob * g.n_q + j) * g.H_q + h) * g.d_h + nsl * 16 + n;
    if (DT == STARKV_F32) ((float*)a.out)[off] = o;
    else ((uint16_t*)a.out)[off] = f32_to_bf16(o);
  }
}

// ===========================================================================

// Scale of the f16 split partials of int8/int4 layers: a partial sums at most cps * 32 tokens'
// weights (each at most 1) times codes of at most 127 in magnitude; the largest power of two
// that keeps that bound within 32768 (half the f16 range).
static float partial_scale(int cps) {
  const double bound = (double)cps * kTC * 127.0;
  int k = 0;
  while (bound > 32768.0 * std::ldexp(1.0, k)) ++k;
  return (float)std::ldexp(1.0, -k);
}

template <int LAT>
static hipError_t launch_values_nmt(const ProfScope& ps, int nmt, dim3 grid, dim3 block, hipStream_t s,
                                    const ValueArgs& va) {
  switch (nmt) {
    case 1: return launch_k(ps, k_values<LAT, 1>, grid, block, s, va);
    case 2: return launch_k(ps, k_values<LAT, 2>, grid, block, s, va);
    case 3: return launch_k(ps, k_values<LAT, 3>, grid, block, s, va);
    case 4: return launch_k(ps, k_values<LAT, 4>, grid, block, s, va);
    case 5: return launch_k(ps, k_values<LAT, 5>, grid, block, s, va);
    case 6: return launch_k(ps, k_values<LAT, 6>, grid, block, s, va);
    case 7: return launch_k(ps, k_values<LAT, 7>, grid, block, s, va);
    default: return launch_k(ps, k_values<LAT, 8>, grid, block, s, va);
  }
}

template <int LAT>
static hipError_t launch_values_mt(const ProfScope& ps, int nmt, dim3 grid, hipStream_t s, const ValueArgs& va) {
  const dim3 blk(256);
  switch (nmt) {
    case 2: return launch_k(ps, k_values_mt<LAT, 2, 2, 3>, grid, blk, s, va);
    case 3: return launch_k(ps, k_values_mt<LAT, 3, 2, 3>, grid, blk, s, va);
    case 4: return launch_k(ps, k_values_mt<LAT, 4, 2, 3>, grid, blk, s, va);
    case 5: return launch_k(ps, k_values_mt<LAT, 5, 2, 3>, grid, blk, s, va);
    case 6: return launch_k(ps, k_values_mt<LAT, 6, 1, 3>, grid, blk, s, va);
    case 7: return launch_k(ps, k_values_mt<LAT, 7, 1, 3>, grid, blk, s, va);
    default: return launch_k(ps, k_values_mt<LAT, 8, 1, 3>, grid, blk, s, va);
  }
}

template <int LAT>
static hipError_t launch_values1(const ProfScope& ps, int nbw8, int nbw4, dim3 grid, hipStream_t s,
                                 const ValueArgs& va) {
  const dim3 blk(256);
  if (LAT != STARKV_LATENT_MIX84) nbw4 = 1;
  if (nbw4 == 1) {
    if (nbw8 == 1) return launch_k(ps, k_values1<LAT, 1, 1>, grid, blk, s, va);
    if (nbw8 == 2) return launch_k(ps, k_values1<LAT, 2, 1>, grid, blk, s, va);
    return launch_k(ps, k_values1<LAT, 4, 1>, grid, blk, s, va);
  }
  if (nbw8 == 1) return launch_k(ps, k_values1<LAT, 1, 2>, grid, blk, s, va);
  if (nbw8 == 2) return launch_k(ps, k_values1<LAT, 2, 2>, grid, blk, s, va);
  return launch_k(ps, k_values1<LAT, 4, 2>, grid, blk, s, va);
}

static QprojArgs qproj_args(const Layer& L, const DecodePlan& plan, const KtList& kts, const void* q) {
  QprojArgs qa;
  qa.q = q;
  qa.qp_w = 1;
  qa.B_k = L.B_k;
  qa.wqk = nullptr;
  qa.qraw = plan.ws.qraw;
  qa.qraw_parts = plan.ws.qraw_parts;
  qa.scales = L.scales;
  qa.heads = L.heads();
  qa.qfrag = (uint8_t*)plan.ws.qfrag;
  qa.rowp = plan.ws.rowp;
  qa.g = plan.g;
  qa.nkt_max = plan.ws.nkt_max;
  qa.kts = kts;
  return qa;
}

// query-projection row groups of the fused step front: few KV heads x sequences spread a head's
// rows over workgroups
static int qproj_row_groups(const DecodeGeom& g) {
  return std::min(g.G * g.n_q, std::max(1, ceil_div(256, g.H_kv * g.B)));
}

// rows per workgroup of the query-projection launch: the rows of one KV head in one sequence, split
// in row groups while there are few KV heads x sequences.  With 2048 or more (KV head, sequence)
// pairs a workgroup takes the rows of two sequences: half as many workgroups, each running the
// same chain of dependent steps over twice the dot products (13B-class ragged step: 25.5 ->
// 21.8 us on MI355X; the rows of four sequences per workgroup, 32.8 us).
static int qproj_rows_per_wg(const DecodeGeom& g) {
  if (qproj_row_groups(g) == 1 && g.H_kv * g.B >= 2048) return 2 * g.G * g.n_q;
  return ceil_div(g.G * g.n_q, qproj_row_groups(g));
}

// First launch of a fused decode step: the few-token append's workgroups and the query
// projection's workgroups in one grid.  The two parts touch disjoint memory (the append writes
// the new cache rows; the projection reads q and B_k and writes the workspace), and the key
// scores, the first reader of both, run in the next launch.
struct StepFrontArgs {
  GemmArgs ga;
  QprojArgs qa;
  int n_app;  // append workgroups; the rest are query-projection workgroups
  int nrg;    // query-projection row groups
};

// Grid: the query-projection workgroups first (their chain of dependent steps starts
// earliest), then the append workgroups; four waves each.
template <int DT, int LAT, int SW>
__global__ __launch_bounds__(256) void k_step_front(StepFrontArgs a) {
  __shared__ float red[3][4][64];
  __shared__ QprojShared sh;
  const int blk = blockIdx.x;
  const int H = a.qa.g.H_kv, B = a.qa.g.B;
  const int n_qp = H * B * a.nrg;
  if (blk < n_qp) {
    // workgroup (KV head, sequence b, row group rg of nrg): rows rg rpg .. of g in sequence b
    const int rph = a.qa.g.G * a.qa.g.n_q, rpg = (rph + a.nrg - 1) / a.nrg;
    const int b = (blk / H) % B, rg = blk / (H * B);
    const int r0 = min(rph, rg * rpg);
    qproj_body<DT, LAT, 256>(a.qa, blk % H, b * rph + r0, b * rph + min(rph, r0 + rpg), sh);
  } else {
    skinny_body<DT, SW, LAT == STARKV_LATENT_MIX84, 4>(a.ga, blk - n_qp, red);
  }
}

template <int SW>
static hipError_t launch_front(const Layer& L, const ProfScope& ps, dim3 grid, hipStream_t s, const StepFrontArgs& fa) {
  if (L.dtype == STARKV_F32) return launch_k(ps, k_step_front<STARKV_F32, STARKV_LATENT_F32, SW>, grid, dim3(256), s, fa);
  if (L.latent == STARKV_LATENT_BF16)
    return launch_k(ps, k_step_front<STARKV_BF16, STARKV_LATENT_BF16, SW>, grid, dim3(256), s, fa);
  return launch_k(ps, k_step_front<STARKV_BF16, STARKV_LATENT_MIX84, SW>, grid, dim3(256), s, fa);
}

static hipError_t launch_decode_tail(const Layer& L, const DecodePlan& plan, const KtList& kts, const SeqTable& seq,
                                     void* out, const void* k_rows, const void* v_tiles, hipStream_t s,
                                     bool scores = true);

// k_scores_lds: DMA pieces per wave per chunk (one of the instantiated counts, at least the
// chunk's 1 KiB pieces over the nct waves), or 0 when the kernel does not apply (three stages of
// a chunk's key rows must fit in LDS)
constexpr int kScoresLdsWgPerCu = 1;
static int scores_lds_dpw(const DecodeGeom& g) {
  const int npc = ceil_div(32 * g.k_row_bytes, 1024);
  if (kScoresLdsStages * (long)npc * 1024 + 16 > 160 * 1024) return 0;
  const int need = ceil_div(npc, g.nct);
  for (int d : {2, 3, 4, 6, 8})
    if (need <= d) return d;
  return 0;
}

template <int KTM>
static hipError_t launch_scores_lds(const ProfScope& ps, int dpw, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                                    const ScoreArgs& sa) {
  void* argv[] = {(void*)&sa};
  const void* k = dpw == 2 ? (const void*)k_scores_lds<KTM, 2>
                  : dpw == 3 ? (const void*)k_scores_lds<KTM, 3>
                  : dpw == 4 ? (const void*)k_scores_lds<KTM, 4>
                  : dpw == 6 ? (const void*)k_scores_lds<KTM, 6>
                             : (const void*)k_scores_lds<KTM, 8>;
  if (ps.start() && ps.stop()) return hipExtLaunchKernel(k, grid, block, argv, lds, s, ps.start(), ps.stop(), 0);
  return hipLaunchKernel(k, grid, block, argv, lds, s);
}

template <int NT>
static hipError_t launch_scores_rope(const Layer& L, const ProfScope& ps, dim3 grid, size_t lds, hipStream_t s,
                                     const RopeScoreArgs& ra, bool qc) {
  void* argv[] = {(void*)&ra};
  const void* k = L.latent == STARKV_LATENT_MIX84
                      ? (qc ? (const void*)k_scores_rope<STARKV_LATENT_MIX84, NT, true>
                            : (const void*)k_scores_rope<STARKV_LATENT_MIX84, NT, false>)
                      : (qc ? (const void*)k_scores_rope<STARKV_LATENT_BF16, NT, true>
                            : (const void*)k_scores_rope<STARKV_LATENT_BF16, NT, false>);
  if (ps.start() && ps.stop()) return hipExtLaunchKernel(k, grid, dim3(256), argv, lds, s, ps.start(), ps.stop(), 0);
  return hipLaunchKernel(k, grid, dim3(256), argv, lds, s);
}

bool rope_latent_scores(const Layer& L, int n_q) {
  return L.G * n_q <= 32 && (L.d_h == 64 || L.d_h == 128) && !L.pack3;
}

// Decode of a rotary layer: scores over rebuilt, rotated key tiles, then the latent-space value
// path (values are not rotated).
static hipError_t launch_decode_rope(const Layer& L, const DecodePlan& plan, const KtList& kts, const SeqTable& seq,
                                     const void* q, void* out, const void* k_rows, const void* v_tiles,
                                     hipStream_t s) {
  const DecodeGeom& g = plan.g;
  RopeScoreArgs ra;
  ra.k_rows = (const uint8_t*)k_rows;
  ra.q = q;
  ra.B_k = (const uint16_t*)L.B_k;
  ra.scales = L.scales;
  ra.heads = L.heads();
  ra.p = plan.ws.p;
  ra.cm = plan.ws.cm;
  ra.cl = plan.ws.cl;
  ra.g = g;
  ra.rope_theta = L.rope_theta;
  ra.rope_w = L.d_rope_w;
  ra.rope_tab = (const float2*)L.d_rope_tab;
  int rmax = 1, npair_max = 1;
  for (int gk = 0; gk < L.H_kv; ++gk) {
    rmax = std::max(rmax, L.rk[gk]);
    const RopeSeg sg(L.mix(), L.koff[gk], L.rk[gk], L.mix() ? L.off8[gk] : 0, L.mix() ? L.n8[gk] : 0,
                     L.mix() ? L.off4[gk] : 0, L.K8);
    npair_max = std::max(npair_max, sg.np8 + sg.np4);
  }
  ra.rpad = ceil_div(rmax, 16) * 16;
  ra.npair_max = npair_max;
  int max_nch = 1;
  for (int b = 0; b < g.B; ++b) max_nch = std::max(max_nch, seq.chunk_off[b + 1] - seq.chunk_off[b]);
  // chunks per wave: 8, fewer while that leaves under 1024 workgroups
  int cpw = 8;
  while (cpw > 1 && (long)g.B * g.H_kv * ceil_div(max_nch, 4 * cpw) < 1024) cpw /= 2;
  ra.cpw = cpw;
  ra.seq = seq;
  const dim3 grid(ceil_div(max_nch, 4 * cpw), g.H_kv, g.B);
  // a few query rows per KV head: each wave turns them by its chunk's base angle (cheaper than
  // composing the two angles for every key element), while two workgroups still fit on a CU
  const int rows = g.G * g.n_q;
  const size_t lds_plain = RopeLds(g.d_h, ra.rpad, rows, npair_max, false).total;
  const size_t lds_qc = RopeLds(g.d_h, ra.rpad, rows, npair_max, true).total;
  const bool qc = rows <= 8 && lds_qc <= std::max(lds_plain, (size_t)80 * 1024);
  const size_t lds = qc ? lds_qc : lds_plain;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  hipError_t e;
  {
    ProfScope ps("decode_scores");
    e = g.d_h == 64 ? launch_scores_rope<2>(L, ps, grid, lds, s, ra, qc) : launch_scores_rope<4>(L, ps, grid, lds, s, ra, qc);
    if (e != hipSuccess) return e;
  }
  return launch_decode_tail(L, plan, kts, seq, out, k_rows, v_tiles, s, false);
}

// The query fragments of a decode (and, with wqk, the hidden-state projection before them).
static hipError_t launch_query_frags(const Layer& L, const DecodePlan& plan, const KtList& kts, const void* q,
                                     hipStream_t s, const float* wqk) {
  const DecodeGeom& g = plan.g;
  hipError_t e = hipSuccess;
  QprojArgs qa = qproj_args(L, plan, kts, q);
  qa.wqk = wqk;
  if (wqk) {
    // hidden-state queries: x wqk^T for all heads (the absorbed factors) into qraw
    ProfScope ps("decode_hidden_q");
    const size_t half = (size_t)L.G * L.n_key * L.d;  // bf16 high part, then low part
    e = launch_hidden_query(L, q, g.B * g.n_q, wqk, (const uint16_t*)wqk + half, plan.ws.qraw, s, ps.start(),
                            ps.stop());
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("decode_qproj");
    qa.qp_w = qproj_rows_per_wg(g);
    const dim3 gq(g.H_kv, ceil_div(g.B * g.G * g.n_q, qa.qp_w));
    if (wqk) {
      if (L.dtype == STARKV_F32) e = launch_k(ps, k_qproj<STARKV_F32, STARKV_LATENT_F32, true>, gq, dim3(256), s, qa);
      else if (L.latent == STARKV_LATENT_BF16) e = launch_k(ps, k_qproj<STARKV_BF16, STARKV_LATENT_BF16, true>, gq, dim3(256), s, qa);
      else e = launch_k(ps, k_qproj<STARKV_BF16, STARKV_LATENT_MIX84, true>, gq, dim3(256), s, qa);
    } else {
      if (L.dtype == STARKV_F32) e = launch_k(ps, k_qproj<STARKV_F32, STARKV_LATENT_F32, false>, gq, dim3(256), s, qa);
      else if (L.latent == STARKV_LATENT_BF16) e = launch_k(ps, k_qproj<STARKV_BF16, STARKV_LATENT_BF16, false>, gq, dim3(256), s, qa);
      else e = launch_k(ps, k_qproj<STARKV_BF16, STARKV_LATENT_MIX84, false>, gq, dim3(256), s, qa);
    }
  }
  return e;
}

hipError_t launch_decode(const Layer& L, const DecodePlan& plan, const KtList& kts, const SeqTable& seq,
                         const void* q, void* out, const void* k_rows, const void* v_tiles, hipStream_t s,
                         const float* wqk) {
  if (L.rope_theta > 0.f) return launch_decode_rope(L, plan, kts, seq, q, out, k_rows, v_tiles, s);
  const hipError_t e = launch_query_frags(L, plan, kts, q, s, wqk);
  if (e != hipSuccess) return e;
  return launch_decode_tail(L, plan, kts, seq, out, k_rows, v_tiles, s);
}

hipError_t launch_step(const Layer& L, const starkv_cache& c, const DecodePlan& plan, const KtList& kts,
                       const SeqTable& seq, const void* X_new, const int32_t* lens_pre, const void* q, void* out,
                       hipStream_t s) {
  const DecodeGeom& g = plan.g;
  const int M = g.B * g.n_q;
  // packed 3-bit layers take the 16-slot front (see store_planes3)
  const int sw = (M <= 8 && L.d % 64 == 0 && !L.pack3) ? 8 : ((M <= 16 && L.d % 32 == 0) ? 16 : 0);
  if (sw == 0 || L.rope_theta > 0.f) {
    // many new rows: the tiled append, then the decode
    const hipError_t e = launch_append(L, c, X_new, g.B, g.n_q, lens_pre, s, seq.lens_dev, g.n_q);
    if (e != hipSuccess) return e;
    return launch_decode(L, plan, kts, seq, q, out, c.k_rows, c.v_tiles, s);
  }
  StepFrontArgs fa;
  fa.ga = GemmArgs{};
  fill_append_args(L, c, fa.ga, X_new, g.B, g.n_q, lens_pre, seq.lens_dev, g.n_q);
  fa.qa = qproj_args(L, plan, kts, q);
  fa.n_app = ceil_div(fa.ga.NS, sw);
  fa.nrg = qproj_row_groups(g);
  const dim3 grid(fa.n_app + g.H_kv * g.B * fa.nrg);
  hipError_t e;
  {
    ProfScope ps("step_front");
    e = sw == 8 ? launch_front<8>(L, ps, grid, s, fa) : launch_front<16>(L, ps, grid, s, fa);
  }
  if (e != hipSuccess) return e;
  return launch_decode_tail(L, plan, kts, seq, out, c.k_rows, c.v_tiles, s);
}

static hipError_t launch_decode_tail(const Layer& L, const DecodePlan& plan, const KtList& kts, const SeqTable& seq,
                                     void* out, const void* k_rows, const void* v_tiles, hipStream_t s, bool scores) {
  const DecodeGeom& g = plan.g;
  const DecodeWs& w = plan.ws;
  hipError_t e = hipSuccess;
  // 2. scores
  if (scores) {
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
  sa.total_chunks = w.total_chunks;
  {
    ProfScope ps("decode_scores");
    if (L.latent == STARKV_LATENT_MIX84) {
      // int8/int4 keys: work unit = (column tile, 32-token chunk), enough chunks per workgroup
      // that each of its four waves has a unit
      // chunks per workgroup: the smallest count that gives the four waves equal numbers of
      // (column tile, chunk) units
      if (L.pack3) {
        sa.nch_wg = 4 / std::gcd(g.nct, 4);
        const int n_wg = ceil_div(w.total_chunks, sa.nch_wg);
        if (w.nkt_max <= 6) e = launch_k(ps, k_scores_chunk<STARKV_LATENT_MIX84, 4, true>, dim3(n_wg), dim3(256), s, sa);
        else e = launch_k(ps, k_scores_chunk<STARKV_LATENT_MIX84, 2, true>, dim3(n_wg), dim3(256), s, sa);
      } else if (g.nct >= 4 && g.nct <= 10 && w.nkt_max <= 8 && scores_lds_dpw(g) > 0) {
        // many column tiles: each chunk's key rows staged in LDS once, one wave per column tile
        const int dpw = scores_lds_dpw(g);
        const int npc = ceil_div(32 * g.k_row_bytes, 1024);
        const size_t lds = kScoresLdsStages * (size_t)npc * 1024 + 16;
        sa.nch_wg = std::max(1, ceil_div(w.total_chunks, 256 * kScoresLdsWgPerCu));
        const dim3 grid(ceil_div(w.total_chunks, sa.nch_wg)), block(64 * g.nct);
        if (w.nkt_max <= 4) e = launch_scores_lds<4>(ps, dpw, grid, block, lds, s, sa);
        else if (w.nkt_max <= 6) e = launch_scores_lds<6>(ps, dpw, grid, block, lds, s, sa);
        else e = launch_scores_lds<8>(ps, dpw, grid, block, lds, s, sa);
      } else if (g.nct >= 4 && w.nkt_max <= 8) {
        // many column tiles: column-tile state in registers while walking blocks of chunks
        sa.nch_wg = 32;  // chunks per block (16 waves' worth of column tiles x 16 chunks each)
        const int n_pairs = (g.nct + 1) / 2;
        const int n_blk = ceil_div(w.total_chunks, sa.nch_wg);
        const dim3 grid(8 * n_pairs * ceil_div(n_blk, 8));
        if (w.nkt_max <= 4) e = launch_k(ps, k_scores_mix<4>, grid, dim3(256), s, sa);
        else if (w.nkt_max <= 6) e = launch_k(ps, k_scores_mix<6>, grid, dim3(256), s, sa);
        else e = launch_k(ps, k_scores_mix<8>, grid, dim3(256), s, sa);
      } else {
        sa.nch_wg = 4 / std::gcd(g.nct, 4);
        const int n_wg = (w.total_chunks + sa.nch_wg - 1) / sa.nch_wg;
        if (w.nkt_max <= 6) e = launch_k(ps, k_scores_chunk<STARKV_LATENT_MIX84, 4>, dim3(n_wg), dim3(256), s, sa);
        else e = launch_k(ps, k_scores_chunk<STARKV_LATENT_MIX84, 2>, dim3(n_wg), dim3(256), s, sa);
      }
    } else {
      // bf16/fp32 keys (many K-tiles per column tile): K split over the waves of a 128-token block
      sa.nch_wg = 4;
      const int n_wg = seq.blk_off[g.B] * g.nct;
      if (L.latent == STARKV_LATENT_BF16) e = launch_k(ps, k_scores<STARKV_LATENT_BF16>, dim3(n_wg), dim3(256), s, sa);
      else e = launch_k(ps, k_scores<STARKV_LATENT_F32>, dim3(n_wg), dim3(256), s, sa);
    }
    if (e != hipSuccess) return e;
  }
  }
  // 3. values
  ValueArgs va;
  va.v_tiles = (const uint8_t*)v_tiles;
  va.p = w.p;
  va.cm = w.cm;
  va.cl = w.cl;
  va.sm = w.sm;
  va.zp = w.zp;
  va.sl = w.sl;
  va.g = g;
  va.seq = seq;
  va.cps = w.cps;
  va.zsc = partial_scale(w.cps);
  va.bpw = w.blocks_per_wg;
  va.NB = L.v_rows / 32;
  va.V8 = L.V8;
  va.n8v = L.n8v;
  va.n4v = L.n4v;
  va.n_sl8 = w.n_sl8;
  va.n_sl4 = w.n_sl4;
  va.NB4 = L.pack3 ? L.V4 / 64 : va.NB;
  va.n3t = L.pack3 ? L.V3 / 32 : 0;
  va.V4 = L.V4;
  va.vo = plan.vo;
  const int n_pos = plan.vo.n ? plan.vo.n : (w.total_splits + 7) / 8 * 8;
  const int nmt = g.M_pad / 32;
  {
    ProfScope ps("decode_values");
    if (nmt == 1) {
      va.n_sl = w.n_sl8 + w.n_sl4 + w.n_sl3;
      va.n_splits = w.total_splits;
      const dim3 gv(va.n_sl * n_pos);
      if (L.latent == STARKV_LATENT_MIX84) e = launch_values1<STARKV_LATENT_MIX84>(ps, w.nbw8, w.nbw4, gv, s, va);
      else if (L.latent == STARKV_LATENT_BF16) e = launch_values1<STARKV_LATENT_BF16>(ps, w.nbw8, w.nbw4, gv, s, va);
      else e = launch_values1<STARKV_LATENT_F32>(ps, w.nbw8, w.nbw4, gv, s, va);
    } else if (L.latent != STARKV_LATENT_F32) {
      va.n_sl = w.n_grp;
      va.n_splits = w.total_splits;
      const dim3 gv(va.n_sl * n_pos);
      if (L.latent == STARKV_LATENT_MIX84) e = launch_values_mt<STARKV_LATENT_MIX84>(ps, nmt, gv, s, va);
      else e = launch_values_mt<STARKV_LATENT_BF16>(ps, nmt, gv, s, va);
    } else {
      const dim3 gv((va.NB + va.bpw - 1) / va.bpw, w.total_splits);
      const dim3 bv(64 * va.bpw);
      if (L.latent == STARKV_LATENT_MIX84) e = launch_values_nmt<STARKV_LATENT_MIX84>(ps, nmt, gv, bv, s, va);
      else if (L.latent == STARKV_LATENT_BF16) e = launch_values_nmt<STARKV_LATENT_BF16>(ps, nmt, gv, bv, s, va);
      else e = launch_values_nmt<STARKV_LATENT_F32>(ps, nmt, gv, bv, s, va);
    }
    if (e != hipSuccess) return e;
  }
  // 4. merge + up-projection
  MergeArgs ma;
  ma.zp = w.zp;
  ma.zinv = 1.f / partial_scale(w.cps);
  ma.cps = w.cps;
  ma.sl = w.sl;
  ma.sm = w.sm;
  ma.zt = w.zt;
  ma.B_vt = L.B_vt;
  ma.vscales = L.mix() ? L.scales + L.n_key : nullptr;
  ma.out = out;
  ma.g = g;
  ma.seq = seq;
  int max_ns = 1;
  for (int b = 0; b < g.B; ++b) max_ns = std::max(max_ns, seq.split_off[b + 1] - seq.split_off[b]);
  const int Rg = g.B * g.G * g.n_q;
  const bool vec = (g.r_v & 7) == 0;
  const bool tall = L.dtype == STARKV_BF16 && vec && Rg >= 64;
  if (max_ns <= 4 && vec && g.rv_ld <= 32 * 32 && !tall) {
    // one launch: the merge is folded into the up-projection
    ProfScope ps("decode_upproj");
    const dim3 gm((g.H_kv + 7) / 8 * 8 * (g.d_h / 16), (Rg + 15) / 16);
    if (L.dtype == STARKV_F32)
      e = L.mix() ? launch_k(ps, k_upproj_merge<STARKV_F32, true>, gm, dim3(512), s, ma)
                  : launch_k(ps, k_upproj_merge<STARKV_F32, false>, gm, dim3(512), s, ma);
    else
      e = L.mix() ? launch_k(ps, k_upproj_merge<STARKV_BF16, true>, gm, dim3(512), s, ma)
                  : launch_k(ps, k_upproj_merge<STARKV_BF16, false>, gm, dim3(512), s, ma);
    if (e != hipSuccess) return e;
    return hipGetLastError();
  }
  {
    ProfScope ps("decode_zmerge");
    ma.nsp = max_ns > 8 ? 4 : 1;
    const dim3 gz((g.rv_ld + 256 / ma.nsp - 1) / (256 / ma.nsp), (g.M_q + 3) / 4, g.B);
    // loads per batch: 4 when no sequence has more splits (one batch), else 16
    if (max_ns <= 4)
      e = L.mix() ? launch_k(ps, k_zmerge<true, 4>, gz, dim3(256), s, ma)
                  : launch_k(ps, k_zmerge<false, 4>, gz, dim3(256), s, ma);
    else
      e = L.mix() ? launch_k(ps, k_zmerge<true, 16>, gz, dim3(256), s, ma)
                  : launch_k(ps, k_zmerge<false, 16>, gz, dim3(256), s, ma);
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("decode_upproj");
    const dim3 gm(g.H_kv * (g.d_h / 16), (Rg + 15) / 16);
    if (tall)
      // two row tiles per workgroup while that leaves at least 128 workgroups: B_v^g is fetched
      // by half as many workgroups (the kernel is bound by the bytes each CU pulls from L2)
      if ((long)g.H_kv * ((Rg + 63) / 64) >= 128)
        e = launch_k(ps, k_upproj_tall<2>, dim3(g.H_kv, (Rg + 63) / 64), dim3(256), s, ma);
      else
        e = launch_k(ps, k_upproj_tall<1>, dim3(g.H_kv, (Rg + 31) / 32), dim3(256), s, ma);
    else if (L.dtype == STARKV_F32)
      e = vec ? launch_k(ps, k_upproj<STARKV_F32, true>, gm, dim3(256), s, ma)
              : launch_k(ps, k_upproj<STARKV_F32, false>, gm, dim3(256), s, ma);
    else
      e = vec ? launch_k(ps, k_upproj<STARKV_BF16, true>, gm, dim3(256), s, ma)
              : launch_k(ps, k_upproj<STARKV_BF16, false>, gm, dim3(256), s, ma);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace skv
